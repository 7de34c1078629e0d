// Absorbed MLA decode: host entry points (checks, split planning, launches).
#include <math.h>
#include <stdlib.h>

#include "../../include/attn_decode.h"
#include "internal.h"

namespace {

inline bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

// Supported latent geometries: (512, 64) and (256, 64) (xuesongtap
// "attention-head" note, section 6: a 32-head model with latent width 256
// and RoPE width 64), both on the shared-tile MLA kernel.
int check_mla(int B, int H, int T_cap, int d_c, int d_rope) {
  if (B < 0 || H <= 0 || T_cap <= 0) return ATTN_ERR_SHAPE;
  if (!((d_c == 512 || d_c == 256) && d_rope == 64)) return ATTN_ERR_UNSUPPORTED;
  if ((long long)B * H > (1LL << 30)) return ATTN_ERR_SHAPE;
  return ATTN_OK;
}

struct MlaPlan {
  int head_chunks;  // column chunks of the balanced list (shared-latent kernel)
  int pair;         // 1: fixed splits run the role-split kernel (512 + 64)
  int fixed_chunks; // column chunks of the fixed splits
  int S, chunk;
  size_t ws_bytes;  // the larger of the two workspaces below
  size_t ws_fixed;  // fixed splits
  int cap;          // > 0: groups of the balanced list (calls with lengths)
  int even;         // 1: the list is the even split (one unit per head chunk)
};

inline size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// Fixed splits of the 512 + 64 latent run the role-split kernel (64 columns
// per group); ATTN_DECODE_MLA_KERNEL=shared keeps them on the shared-latent
// kernel (for comparisons; read at every plan, so a process can hold both).
bool mla_use_pair(int d_c) {
  const char* e = getenv("ATTN_DECODE_MLA_KERNEL");
  return d_c == 512 && !(e && e[0] == 's');
}

// Lead tiles per unit of the MLA even split: a segment's start (the query
// fragments of 128 heads, three tiles of loads before the first tile can be
// computed, the merge-ready partials at its end), and the cost of segments
// only a few tiles long.  Swept on B=64 with lengths 1k..8k (us per step):
// lead 0 138.0, 2 135.9, 4 132.2, 8 128.6, 12 128.0, 16 130.2, 24 133.1,
// against 131.4 for the per-sequence list (overridable for tuning sweeps
// through ATTN_DECODE_MLA_EVEN_LEAD).
int mla_even_lead() {
  static const int v = [] {
    const char* e = getenv("ATTN_DECODE_MLA_EVEN_LEAD");
    const int x = e ? atoi(e) : -1;
    return x >= 0 && x <= 256 ? x : 12;
  }();
  return v;
}

// Partial slots of the balanced list: one per group of the per-sequence
// list; one per (group, unit) segment of the even split, at most cap + B
// units.
size_t mla_slots(const MlaPlan& p, int B) {
  return p.even ? (size_t)p.cap + (size_t)B * p.head_chunks : (size_t)p.cap;
}

// Balanced list: o_part, lse_part (hg rows per slot) and the (first slot,
// pieces) pairs, per sequence or, for the even split, per unit.
size_t mla_balanced_bytes(const MlaPlan& p, int hg, int d_c, int B) {
  const size_t rows = mla_slots(p, B) * hg;
  const size_t pairs = p.even ? (size_t)B * p.head_chunks : (size_t)B;
  return round_up(rows * d_c * sizeof(float), 256) + round_up(rows * sizeof(float), 256) +
         round_up(pairs * 2 * sizeof(int), 256);
}

int plan_mla(int B, int H, int T_cap, int d_c, int d_rope, int num_splits,
             MlaPlan* p) {
  const int st = check_mla(B, H, T_cap, d_c, d_rope);
  if (st != ATTN_OK) return st;
  if (num_splits < 0 || num_splits > ATTN_MAX_SPLITS) return ATTN_ERR_ARG;
  const int hg = attn::mla_heads_per_group(d_c);
  p->head_chunks = (H + hg - 1) / hg;
  p->pair = mla_use_pair(d_c) ? 1 : 0;
  const int hf = p->pair ? attn::mla_pair_columns() : hg;
  p->fixed_chunks = (H + hf - 1) / hf;
  long long S;
  if (num_splits > 0) {
    S = num_splits;
  } else {
    // fill every CU with the groups it holds at once; keep at least two
    // tiles per group
    const long long units = (long long)(B > 0 ? B : 1) * p->fixed_chunks;
    const long long target =
        (long long)attn::kNumCUs * (p->pair ? 1 : attn::mla_groups_per_cu(d_c));
    S = (target + units - 1) / units;
    long long smax = T_cap / (2LL * attn::mla_tile_rows());
    if (smax < 1) smax = 1;
    if (S > smax) S = smax;
  }
  if (S < 1) S = 1;
  if (S > T_cap) S = T_cap;
  // splits start at multiples of the tile rows (a paged cache needs each
  // 16-row half of a tile inside one page)
  const int tr = attn::mla_tile_rows();
  p->chunk = (int)((T_cap + S - 1) / S);
  p->chunk = (p->chunk + tr - 1) / tr * tr;
  p->S = (T_cap + p->chunk - 1) / p->chunk;
  p->ws_fixed = attn_decode_workspace_bytes(B, H, d_c, p->S);
  p->ws_bytes = p->ws_fixed;
  // balanced list: when the fixed plan splits, a call with lengths cuts each
  // sequence by its own length into pieces of one common size (balance.h)
  p->cap = 0;
  // the even split (where the geometry runs it) numbers 32-row tiles plus
  // lead tiles of every unit with ints
  p->even = attn::mla_even_split(d_c) &&
            (long long)B * p->head_chunks * (T_cap / tr + 1 + mla_even_lead()) < (1LL << 31);
  const int cap = attn::kNumCUs * attn::mla_groups_per_cu(d_c);
  if (num_splits == 0 && p->S > 1 && B >= 1 && B <= attn::kBalanceMaxB &&
      (long long)B * p->head_chunks < cap && cap <= ATTN_MAX_SPLITS) {
    p->cap = cap;
    const size_t bb = mla_balanced_bytes(*p, hg, d_c, B);
    if (bb > p->ws_bytes) p->ws_bytes = bb;
  }
  return ATTN_OK;
}

}  // namespace

extern "C" {

int attn_decode_mla_splits(int B, int H, int T_cap, int d_c, int d_rope,
                           int num_splits) {
  MlaPlan p;
  const int st = plan_mla(B, H, T_cap, d_c, d_rope, num_splits, &p);
  return st == ATTN_OK ? p.S : st;
}

size_t attn_decode_mla_workspace_bytes(int B, int H, int T_cap, int d_c,
                                       int d_rope, int num_splits) {
  MlaPlan p;
  const int st = plan_mla(B, H, T_cap, d_c, d_rope, num_splits, &p);
  return st == ATTN_OK ? p.ws_bytes : (size_t)-1;
}

}  // extern "C"

namespace {

// L query tokens per sequence plan as H * L (head, token) columns.
int decode_mla(const void* q, const void* latent, float* out, float* lse_out,
               const int32_t* seq_lens, const int32_t* block_table,
               int max_pages, int page_shift, int num_pages, int B, int L, int H,
               int T_cap, int d_c, int d_rope, float scale, int num_splits,
               void* workspace, size_t workspace_bytes, void* stream) {
  if (L < 1 || L > ATTN_MAX_QLEN) return ATTN_ERR_ARG;
  if (H > 0 && (long long)H * L > (1 << 30)) return ATTN_ERR_SHAPE;
  MlaPlan p;
  int st = plan_mla(B, H * L, T_cap, d_c, d_rope, num_splits, &p);
  if (st != ATTN_OK) return st;
  if (!(scale > 0.f) || isinf(scale)) return ATTN_ERR_ARG;
  if (B == 0) return ATTN_OK;
  if (!q || !latent || !out) return ATTN_ERR_NULL;
  if (!aligned(q, 16) || !aligned(latent, 16) || !aligned(out, 16) ||
      (lse_out && !aligned(lse_out, 4)) || (seq_lens && !aligned(seq_lens, 4)))
    return ATTN_ERR_ALIGN;
  float* o_part = nullptr;
  float* lse_part = nullptr;
  int* meta = nullptr;
  const int hg = attn::mla_heads_per_group(d_c);
  // balanced list: lengths given and room for its parts; else fixed splits
  // the even split takes one query token per sequence; several tokens keep
  // the per-sequence list, whose parts fit in the same workspace
  if (L > 1) p.even = 0;
  const bool bal = p.cap > 0 && seq_lens && workspace && aligned(workspace, 16) &&
                   workspace_bytes >= mla_balanced_bytes(p, hg, d_c, B);
  if (bal) {
    const size_t rows = mla_slots(p, B) * hg;
    o_part = (float*)workspace;
    lse_part = (float*)((char*)workspace + round_up(rows * d_c * sizeof(float), 256));
    meta = (int*)((char*)lse_part + round_up(rows * sizeof(float), 256));
  } else if (p.S > 1) {
    if (!workspace || workspace_bytes < p.ws_fixed) return ATTN_ERR_WORKSPACE;
    if (!aligned(workspace, 16)) return ATTN_ERR_ALIGN;
    const size_t rows = (size_t)B * L * H * p.S;
    o_part = (float*)workspace;
    lse_part = (float*)((char*)workspace + round_up(rows * d_c * sizeof(float), 256));
  }
  if ((long long)B * p.S * p.fixed_chunks > 0x7fffffffLL) return ATTN_ERR_SHAPE;
  hipStream_t s = (hipStream_t)stream;
  if (!bal && p.pair) {
    if (attn::launch_mla_pair(q, latent, out, lse_out, o_part, lse_part, seq_lens,
                              block_table, max_pages, page_shift, num_pages, B, L, H, T_cap,
                              p.S, p.chunk, p.fixed_chunks, scale * 1.4426950408889634f,
                              s) != hipSuccess)
      return ATTN_ERR_HIP;
    if (p.S > 1 && attn::launch_combine_half(o_part, lse_part, out, lse_out, B, H * L, p.S,
                                             d_c, s) != hipSuccess)
      return ATTN_ERR_HIP;
    return ATTN_OK;
  }
  if (attn::launch_mla_mfma(q, latent, out, lse_out, o_part, lse_part, seq_lens,
                            block_table, max_pages, page_shift, num_pages, B, L, H,
                            T_cap, d_c, p.S, p.chunk, p.head_chunks,
                            bal ? (p.even ? 2 : 1) : 0, bal ? p.cap : 0, meta,
                            mla_even_lead(), scale * 1.4426950408889634f,
                            s) != hipSuccess)
    return ATTN_ERR_HIP;
  const bool half = attn::mla_half_parts(d_c);
  if (bal) {
    // columns are (head, token) pairs of one latent: n = H heads share it
    if (attn::launch_combine_balanced(o_part, half, lse_part, meta, out, lse_out, B, L,
                                      H, H, p.head_chunks, hg, d_c, p.even != 0,
                                      s) != hipSuccess)
      return ATTN_ERR_HIP;
  } else if (p.S > 1) {
    const hipError_t e =
        half ? attn::launch_combine_half(o_part, lse_part, out, lse_out, B, H * L, p.S,
                                         d_c, s)
             : attn::launch_combine(o_part, lse_part, out, lse_out, B, H * L, p.S, d_c, s);
    if (e != hipSuccess) return ATTN_ERR_HIP;
  }
  return ATTN_OK;
}

}  // namespace

extern "C" {

int attn_decode_mla(const void* q, const void* latent, float* out,
                    float* lse_out, const int32_t* seq_lens, int B, int H,
                    int T_cap, int d_c, int d_rope, float scale,
                    int num_splits, void* workspace, size_t workspace_bytes,
                    void* stream) {
  return decode_mla(q, latent, out, lse_out, seq_lens, nullptr, 0, 0, 0, B, 1, H,
                    T_cap, d_c, d_rope, scale, num_splits, workspace,
                    workspace_bytes, stream);
}

int attn_decode_mla_multi(const void* q, const void* latent, float* out,
                          float* lse_out, const int32_t* seq_lens, int B,
                          int q_len, int H, int T_cap, int d_c, int d_rope,
                          float scale, int num_splits, void* workspace,
                          size_t workspace_bytes, void* stream) {
  return decode_mla(q, latent, out, lse_out, seq_lens, nullptr, 0, 0, 0, B, q_len,
                    H, T_cap, d_c, d_rope, scale, num_splits, workspace,
                    workspace_bytes, stream);
}

int attn_decode_mla_paged(const void* q, const void* latent_pages, float* out,
                          float* lse_out, const int32_t* seq_lens,
                          const int32_t* block_table, int max_pages, int B,
                          int q_len, int H, int num_pages, int page_size,
                          int d_c, int d_rope, float scale, int num_splits,
                          void* workspace, size_t workspace_bytes,
                          void* stream) {
  int shift = 0;
  const int st = attn_check_pages(max_pages, num_pages, page_size, 1, &shift);
  if (st != ATTN_OK) return st;
  if (B > 0 && !block_table) return ATTN_ERR_NULL;
  if (block_table && !aligned(block_table, 4)) return ATTN_ERR_ALIGN;
  return decode_mla(q, latent_pages, out, lse_out, seq_lens, block_table,
                    max_pages, shift, num_pages, B, q_len, H, max_pages * page_size,
                    d_c, d_rope, scale, num_splits, workspace, workspace_bytes,
                    stream);
}

}  // extern "C"
