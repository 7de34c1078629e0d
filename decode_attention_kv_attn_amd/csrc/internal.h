// Launch-side interface between the host API and the kernel translation units.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace attn {

constexpr int kNumCUs = 256;  // MI355X: 8 XCDs x 32 CUs
constexpr int kNumXCDs = 8;

// Most sequences a balanced work list handles (4 per lane of a wave).
constexpr int kBalanceMaxB = 256;

// Arguments of one MHA/GQA/MQA decode launch.
struct GqaArgs {
  const void* q;
  const void* k;
  const void* v;
  float* out;        // final output when S == 1
  float* lse;        // final lse when S == 1 (nullable)
  float* o_part;     // [B, H_q, S, d] when S > 1
  float* lse_part;   // [B, H_q, S]    when S > 1
  const int32_t* seq_lens;   // nullable
  const int32_t* ring_head;  // nullable: linear addressing
  const int32_t* gpos;       // global positions (linear cache only), nullable
  int n_global;
  const int32_t* block_table;  // paged cache: [B, max_pages], else nullptr
  int max_pages, page_shift, num_pages;
  int B, H_q, H_kv, T_cap;  // paged: T_cap = max_pages << page_shift
  int window;       // visible-range window: w + L - 1 (0 = none)
  int L;            // query tokens per sequence (the last L positions)
  int wtok;         // each token's own window w (0 = none)
  int n;            // query heads per KV head
  int ncol;         // columns per KV head: n * L (head, token) pairs
  int head_chunks;  // work items per KV head along the query heads
  int S;            // splits of the visible range
  int chunk;        // positions per split
  int xcd_remap;    // 1: map consecutive work items onto one XCD
  float scale_log2; // softmax scale * log2(e)
  // Balanced work lists (balance.h).  1, both kernels: work item w is item w
  // of the per-sequence list by visible rows instead of a fixed split; pieces
  // of a sequence's units go to o_part / lse_part row w * heads_per_item +
  // column, and meta[2b], meta[2b+1] receive the sequence's first item and
  // its pieces per unit.  2, the matrix-core kernel: the even split; the
  // segment of unit ui in work group w goes to slot w + ui (rows slot *
  // heads_per_item + column), and meta[2ui], meta[2ui+1] receive the unit's
  // first slot and its pieces.  A unit in one piece is written to out / lse
  // directly.
  int balanced;
  int cap;          // items the list may hold (the grid)
  int even_lead;    // even split: lead tiles per unit (its start-up cost)
  int* meta;        // [B, 2] (list 1) or [B * units per sequence, 2] (list 2)
};

// Per-instantiation geometry of the VALU kernel, reported to the planner.
struct ValuGeometry {
  int heads_per_item;  // N: query heads one work item serves
  int tile_rows;       // positions per wave per tile
  int waves;           // waves per work group
};

// dtype: 0 = float32, 1 = bf16.  Returns false if no instantiation exists.
bool valu_geometry(int dtype, int d, int n, ValuGeometry* g);
// Picks the addressing mode from `a` (paged, global positions, or dense);
// each mode's instantiations live in a translation unit of their own.
hipError_t launch_gqa_valu(const GqaArgs& a, int dtype, int d, int grid,
                           hipStream_t stream);
hipError_t launch_gqa_valu_dense(const GqaArgs& a, int dtype, int d, int grid,
                                 hipStream_t stream);
hipError_t launch_gqa_valu_global(const GqaArgs& a, int dtype, int d, int grid,
                                  hipStream_t stream);
hipError_t launch_gqa_valu_paged(const GqaArgs& a, int dtype, int d, int grid,
                                 hipStream_t stream);

// Matrix-core path for bf16 groups of 3 or more columns, d in {64, 128, 256}.
int mfma_heads_per_item(int dtype, int d, int n);
int mfma_tile_rows();
int mfma_waves();
hipError_t launch_gqa_mfma(const GqaArgs& a, int d, int heads_per_item, int grid,
                           hipStream_t stream);

// Absorbed MLA on the matrix cores (bf16, d_rope = 64, d_c = 512 or 256).
int mla_heads_per_group(int d_c);  // (head, token) columns per work group
int mla_groups_per_cu(int d_c);    // work groups one CU holds at once (LDS)
int mla_tile_rows();
// true: the kernel writes its split partial values as fp16 (the o_part region
// keeps its float32 size; the fp16 rows fill its first half)
bool mla_half_parts(int d_c);
// L query tokens per sequence (q [B, L, H, DK], outputs [B, L, H, ...]) with
// DK = d_c + 64; block_table == nullptr: dense latent [B, T_cap, DK]; else a
// page pool [num_pages, 2^page_shift, DK] with T_cap = max_pages <<
// page_shift, and `chunk` a multiple of the tile rows.
// balanced: 0 fixed splits, 1 the per-sequence list, 2 the even split
// (only where mla_even_split(d_c); even_lead as GqaArgs::even_lead).
hipError_t launch_mla_mfma(const void* q, const void* latent, float* out,
                           float* lse, float* o_part, float* lse_part,
                           const int32_t* seq_lens, const int32_t* block_table,
                           int max_pages, int page_shift, int num_pages, int B,
                           int L, int H, int T_cap, int d_c, int S, int chunk,
                           int head_chunks, int balanced, int cap, int* meta,
                           int even_lead, float scale_log2, hipStream_t stream);

// The 512 + 64 latent with fixed splits: work groups of 64 (head, token)
// columns split into score and value waves (mla_pair.hip); o_part holds fp16
// partials [B * L * H, S, 512].
int mla_pair_columns();
hipError_t launch_mla_pair(const void* q, const void* latent, float* out, float* lse,
                           void* o_part, float* lse_part, const int32_t* seq_lens,
                           const int32_t* block_table, int max_pages, int page_shift,
                           int num_pages, int B, int L, int H, int T_cap, int S, int chunk,
                           int head_chunks, float scale_log2, hipStream_t stream);
// true where the geometry of latent width d_c runs the even split
bool mla_even_split(int d_c);

}  // namespace attn

// Page-geometry check shared by the paged entry points (api.hip); returns an
// ATTN_* status and log2(page_size) in *shift.
int attn_check_pages(int max_pages, int num_pages, int page_size, int rows_per_pos,
                     int* shift);

namespace attn {

hipError_t launch_combine(const float* o_part, const float* lse_part,
                          float* out, float* lse, int B, int H, int S, int d_v,
                          hipStream_t stream);

// Merge of a balanced work list's pieces (GqaArgs::balanced): output row
// (b * L + token) * H_q + head, for heads_per_item columns per item and
// head_chunks items per KV head; rows whose unit has one piece are left as
// the decode kernel wrote them.  per_unit: the even split's meta (one pair
// per unit), else the per-sequence list's.  o_part (float32, or fp16 when
// half_parts) and out 16-byte aligned, d_v in {64, 128, 256, 512}.
hipError_t launch_combine_balanced(const void* o_part, bool half_parts,
                                   const float* lse_part, const int* meta, float* out,
                                   float* lse, int B, int L, int H_q, int n,
                                   int head_chunks, int heads_per_item, int d_v,
                                   bool per_unit, hipStream_t stream);

// launch_combine with fp16 partial values (o_part [B, H, S, d_v] of _Float16,
// 16-byte aligned; d_v a multiple of 64 up to 512).
hipError_t launch_combine_half(const void* o_part, const float* lse_part, float* out,
                               float* lse, int B, int H, int S, int d_v,
                               hipStream_t stream);

}  // namespace attn
