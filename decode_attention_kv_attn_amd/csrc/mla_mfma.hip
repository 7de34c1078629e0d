// Absorbed MLA decode on the matrix cores (kernel 4).
//
// Every query head of a sequence reads the same latent rows [c_j | k^R_j]
// (xuesongtap "attention-head" note, sections 5.2-5.3: keys absorbed into
// the query, the RoPE key shared by all heads, values projected after the
// weighted sum), so both products are dense and run on MFMA 16x16x32:
//
//   S^T[tokens, heads] = L[tokens, 0:576] . Q^T[576, heads]
//   Z^T[0:512, heads] += L[tokens, 0:512]^T . P^T[tokens, heads]
//
// One work group = one (sequence, split) and up to 128 heads: four waves,
// each owning 32 heads, share every latent tile, so the latent is read from
// HBM once.  Tiles of 32 rows (36 KiB) go straight from HBM into LDS with
// 16-byte direct-to-LDS buffer loads, three tiles ahead of the one being
// computed, through four stage buffers; every wait on those loads is
// explicit.  Score operands are read from the row-major tile; value
// operands come transposed through ds_read_b64_tr_b16.  Rows are swizzled
// in 16-byte chunks so both read patterns are free of bank conflicts.
//
// Precision, per geometry.  fp16 (the 512 + 64 latent, where the matrix
// cores bound the kernel): each tile is converted from bf16 to fp16 in place,
// once, by all waves together while the tile before it is computed (a bf16
// value converts exactly when 2^-14 <= |x| <= 65504, smaller ones with an
// absolute error below 2^-25; larger ones overflow), and the queries once at
// the start; the softmax weights enter the value product as fp16 (11
// significant bits, rounded to nearest), one MFMA per value block; a split's
// partial values (weighted means of latent values, so inside the same range)
// are stored as fp16 for the merge, halving that round trip.  bf16
// (the 256 + 64 latent, bound by memory): the data stays bf16 and the weights
// keep about 16 significant bits as a bf16 high part plus a bf16 remainder,
// two MFMAs per value block.
//
// Paged latent caches ([num_pages, P, 576], P a power of two >= 16; the
// paging the baidu article, section 四.3, names for MLA): splits and tiles
// start at multiples of 32 positions, so each 16-row half of a tile lies in
// one page and a tile needs two page ids, read with scalar loads a step
// ahead of the tile's loads.

#include <type_traits>

#include "balance.h"
#include "device_common.h"
#include "internal.h"
#include "mla_common.h"
#include "visible.h"

// Tuning knobs (compile-time; defaults are the measured best).
#ifndef ATTN_MLA_QK_AHEAD  // k-steps the score operand reads run ahead
#define ATTN_MLA_QK_AHEAD 2
#endif
#ifndef ATTN_MLA_V_AHEAD  // value blocks the transposed operand reads run ahead
#define ATTN_MLA_V_AHEAD 2
#endif

namespace attn {
namespace {

constexpr int kTT = 32;                   // rows per tile
constexpr int kLdsPerCU = 160 * 1024;

// Latent geometry and group shape: rows of DK = d_c + d_rope bf16, the first
// DV columns are the values; NW waves of HW (head, token) columns each;
// STAGES tiles in LDS (STAGES - 1 loading while one is computed).
template <int DK, int DV, int NW, int HW, int STAGES, bool F16>
struct MlaGeo {
  static constexpr int kDK = DK, kDV = DV, kNW = NW, kHW = HW, kStages = STAGES;
  static constexpr bool kF16 = F16;  // fp16 products (else bf16, split weights)
  static constexpr int kHB = HW / 16;                     // 16-column blocks per wave
  static constexpr int kHG = NW * HW;                     // columns per group
  static constexpr int kRowBytes = DK * 2;
  static constexpr int kCPR = kRowBytes / 16;             // 16-byte chunks per row
  static constexpr int kTileBytes = kTT * kRowBytes;
  static constexpr int kPieces = kTileBytes / 1024;       // 1 KiB loads per tile
  static constexpr int kDmaPerWave = (kPieces + NW - 1) / NW;
  static constexpr int kKS = DK / 32;                     // score k-steps
  static constexpr int kDB = DV / 16;                     // value blocks
  static_assert(DK % 32 == 0 && DV % 16 == 0 && DV <= DK, "latent widths");
  static_assert(kCPR % 8 == 0, "the swizzle permutes aligned groups of 8 chunks");
  // each 1 KiB load lies in one 16-row half of the tile (one page)
  static_assert((16 * kRowBytes) % 1024 == 0, "tile halves are whole loads");
  static_assert(16 * kRowBytes <= 65536, "per-lane offsets in a half fit 16 bits");
  static_assert(HW % 16 == 0 && (HW / 16 == 1 || HW / 16 == 2), "column blocks");
  static_assert(STAGES >= (F16 ? 3 : 2) && STAGES * kTileBytes <= kLdsPerCU, "stages");
  static constexpr int kGroupsPerCU = kLdsPerCU / (STAGES * kTileBytes);
};
// (512, 64): four waves of 32 heads, four stages (144 KiB, one group per
// CU); (256, 64): two waves of 16 heads, ATTN_MLA_NARROW_STAGES stages.
#ifndef ATTN_MLA_NARROW_STAGES
#define ATTN_MLA_NARROW_STAGES 4
#endif
#ifndef ATTN_MLA_WIDE_WAVES  // waves sharing the 128 heads of a group
#define ATTN_MLA_WIDE_WAVES 4
#endif
using GeoWide = MlaGeo<576, 512, ATTN_MLA_WIDE_WAVES, 128 / ATTN_MLA_WIDE_WAVES, 4, true>;
using GeoNarrow = MlaGeo<320, 256, 2, 16, ATTN_MLA_NARROW_STAGES, false>;


typedef __bf16 bf16x2_v __attribute__((ext_vector_type(2)));

// (a, b) -> packed bf16 high parts (round to nearest even, v_cvt_pk_bf16_f32)
// and packed bf16 remainders a - hi(a), b - hi(b): hi + lo carries about 16
// significant bits of each weight.
ATTN_DEV void split_bf16(float a, float b, uint32_t& hi, uint32_t& lo) {
  hi = __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_v{a, b}, bf16x2_v));
  const float ra = a - __uint_as_float(hi << 16);
  const float rb = b - __uint_as_float(hi & 0xffff0000u);
  lo = __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_v{ra, rb}, bf16x2_v));
}

// The MFMAs are written out (v_mfma_f32_16x16x32_f16 or _bf16, accumulating
// in place).  The compiler's own form keeps no accumulator in place once the
// 256 AGPRs are all taken by o: it routes each result through a scratch
// register and shuttles accumulators between the register files, and an
// MFMA that overwrites a register an earlier one still reads stalls the
// matrix pipe; in-place accumulation back to back runs at full rate.  The
// score accumulators are VGPRs, the value accumulators AGPRs.  Since the
// compiler does not see these as MFMAs, the hazards it would cover are
// covered here: VALU reads of an MFMA result wait out its latency
// (ATTN_MFMA_DRAIN), and operands written by VALU instructions get wait
// states before their first MFMA (the s_nop in the value product's prologue).
// Operands are 8 fp16 or 8 bf16 in four dwords.
template <bool F16>
ATTN_DEV void mfma_first_v(f32x4_t& acc, const u32x4& a, const u32x4& b) {
  if constexpr (F16)
    asm volatile("v_mfma_f32_16x16x32_f16 %0, %1, %2, 0" : "=&v"(acc) : "v"(a), "v"(b));
  else
    asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, 0" : "=&v"(acc) : "v"(a), "v"(b));
}
template <bool F16>
ATTN_DEV void mfma_v(f32x4_t& acc, const u32x4& a, const u32x4& b) {
  if constexpr (F16)
    asm volatile("v_mfma_f32_16x16x32_f16 %0, %1, %2, %0" : "+v"(acc) : "v"(a), "v"(b));
  else
    asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+v"(acc) : "v"(a), "v"(b));
}
template <bool F16>
ATTN_DEV void mfma_a(f32x4_t& acc, const u32x4& a, const u32x4& b) {
  if constexpr (F16)
    asm volatile("v_mfma_f32_16x16x32_f16 %0, %1, %2, %0" : "+a"(acc) : "v"(a), "v"(b));
  else
    asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+a"(acc) : "v"(a), "v"(b));
}
#define ATTN_MFMA_DRAIN "s_nop 15\n\ts_nop 15"


struct MlaArgs {
  const uint16_t* q;       // [B, H, DK]
  const uint16_t* latent;  // [B, T_cap, DK], or the page pool [num_pages, P, DK]
  const int32_t* block_table;  // [B, max_pages] (paged only)
  int max_pages, page_shift, num_pages;
  float* out;              // [B, H, DV] when S == 1
  float* lse;              // [B, H] (nullable) when S == 1
  float* o_part;           // [B, H, S, DV]; fp16 values when G::kF16
  float* lse_part;         // [B, H, S]
  const int32_t* seq_lens;
  int H, T_cap, S, chunk, head_chunks;
  int L;     // query tokens per sequence (the last L positions)
  int ncol;  // (head, token) columns: H * L
  float scale_log2;
  // Balanced work lists (balance.h).  1: group w is item w of the
  // per-sequence list by visible length; a sequence cut into several pieces
  // leaves partial rows w * kHG + column and meta[2b], meta[2b + 1] = (first
  // item, pieces).  2 (fp16 geometry): the even split; the segment of unit
  // ui = b * head_chunks + hc in group w leaves rows (w + ui) * kHG + column
  // and meta[2ui], meta[2ui + 1] = (first slot, pieces).
  int balanced, cap, B;
  int* meta;
  int even_lead;  // even split: lead tiles per unit
};

// MULTI: several query tokens per sequence (per-column causal limits); a
// separate instantiation so the single-token path carries none of it.  LIST:
// 0 fixed splits, 1 the per-sequence work list, 2 the even split (fp16
// geometry), likewise.
template <class G, int MODE, bool MULTI, int LIST>
__global__ __launch_bounds__(G::kNW * 64, G::kGroupsPerCU) void mla_decode_mfma(MlaArgs a) {
  constexpr int kDK = G::kDK, kDV = G::kDV, kNW = G::kNW, kHW = G::kHW, kHB = G::kHB;
  constexpr int kHG = G::kHG, kRowBytes = G::kRowBytes, kCPR = G::kCPR;
  constexpr int kTileBytes = G::kTileBytes, kPieces = G::kPieces;
  constexpr int kDmaPerWave = G::kDmaPerWave, kKS = G::kKS, kDB = G::kDB;
  constexpr int kStages = G::kStages;
  constexpr bool kF16 = G::kF16;
  __shared__ __attribute__((aligned(1024))) unsigned char stages[kStages * kTileBytes];
  // LDS of the stage that holds tile `it`
  auto stage_of = [&](int it) { return stages + (it % kStages) * kTileBytes; };

  const int lane = threadIdx.x & 63;
  // uniform across the wave: keep wave-derived offsets in scalar registers
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int li = lane & 15;
  const int lg = lane >> 4;

  const int item = blockIdx.x;
  // the even split's per-sequence plan (the registers are taken)
  __shared__ int plan_lds[LIST == 2 ? 3 * kBalanceMaxB : 1];

  // The (head, token) columns of head chunk hc of sequence b over the rows
  // [p0, p1) of vr.  Results go to out / lse when `direct`, else to partial
  // rows: row * S + slot (fixed splits, slot = split) or slot * kHG +
  // column (the lists).
  auto process = [&](int b, int hc, const VisibleRange& vr, int p0, int p1, bool direct,
                     int slot) {
    const int hw0 = hc * kHG + wave * kHW;  // first head of this wave
    const int span = p1 - p0;
    const int ntiles = span > 0 ? (span + kTT - 1) / kTT : 0;
    const unsigned char* lat_b =
        (const unsigned char*)(MODE == kAddrPaged ? a.latent
                                                  : a.latent + (size_t)b * a.T_cap * kDK);
    Pages pg{};
    if constexpr (MODE == kAddrPaged)
      pg = page_view(a.block_table, a.max_pages, b, vr.hi, a.page_shift, a.num_pages, 1);

    // Q^T fragments: column hw0 + 16*hb + li (a (head, token) pair),
    // elements 32*ks + 8*lg .. +7
    uint4 qf[kHB][kKS];
    int tl[kHB];  // causal limit of this lane's columns (several tokens)
#pragma unroll
    for (int hb = 0; hb < kHB; ++hb) {
      const int c = hw0 + 16 * hb + li;
      const uint16_t* qp =
          a.q + query_row(b, 0, min(c, a.ncol - 1), a.H, a.L, a.H) * kDK + 8 * lg;
#pragma unroll
      for (int ks = 0; ks < kKS; ++ks)
        qf[hb][ks] = c < a.ncol ? *(const uint4*)(qp + 32 * ks) : make_uint4(0, 0, 0, 0);
      tl[hb] = vr.hi - a.L + c % a.L;
    }
    constexpr bool multi = MULTI;

    f32x4_t o[kDB][kHB];
    float m[kHB], l[kHB];
#pragma unroll
    for (int hb = 0; hb < kHB; ++hb) {
      m[hb] = neg_inf();
      l[hb] = 0.f;
#pragma unroll
      for (int db = 0; db < kDB; ++db) o[db][hb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    }

    // Direct-to-LDS loads of a tile: LDS chunk p = blk*64 + lane holds row
    // p / 72, logical chunk (p % 72) ^ swz(row).  A 1 KiB block blk < 18 lies
    // in rows 0..15, the others in rows 16..31, so every load reads from one
    // 16-row half (one page of a paged cache).  This wave's loads are blocks
    // wave, wave + kNW, ... of the tile's kPieces; their per-lane byte offsets
    // from the start of their half are < 2^16, two per register.
    const int my_pieces =
        kPieces % kNW == 0 ? kDmaPerWave : (kPieces - wave + kNW - 1) / kNW;
    uint32_t dma_off[(kDmaPerWave + 1) / 2];
#pragma unroll
    for (int j = 0; j < kDmaPerWave; ++j) {
      const int p = min(wave + j * kNW, kPieces - 1) * 64 + lane;
      const int t = p / kCPR;
      const uint32_t off = (t & 15) * kRowBytes + 16 * ((p - t * kCPR) ^ swz(t));
      if (j & 1) dma_off[j >> 1] |= off << 16;
      else dma_off[j >> 1] = off;
    }

    // Pages of the two 16-row halves of the tile in each stage (paged caches
    // only), clamped to the pool.  Scalar buffer loads of the sequence's
    // table row (the scalar counter keeps them out of the vector-load waits
    // of the tile pipeline), a tile ahead of their use.
    int pid_cur[2] = {}, pid_next[2] = {};  // tile it + kStages - 1, tile it + kStages
    u32x4 table_rsrc = {};
    if constexpr (MODE == kAddrPaged) {
      const uint64_t t = (uint64_t)(uintptr_t)pg.table;
      table_rsrc = u32x4{(uint32_t)t, (uint32_t)(t >> 32) & 0xffffu,
                         (uint32_t)a.max_pages * 4u, (uint32_t)kBufferWord3};
    }
    auto fetch_pages = [&](int it, int (&pid)[2]) {
      if constexpr (MODE == kAddrPaged) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const int j = min((p0 + it * kTT + 16 * h) >> pg.shift, pg.last);
          const int v = scalar_buffer_load_i32(table_rsrc, 4 * j, 0);
          pid[h] = v < 0 ? 0 : (v >= pg.num_pages ? pg.num_pages - 1 : v);
        }
      }
    };
    // the page ids of the tile whose loads go out next (fetched a tile
    // earlier) become current; their wait lands right after the barrier,
    // where no LDS read is in flight
    auto pages_ready = [&]() {
      if constexpr (MODE == kAddrPaged) {
        pid_cur[0] = pid_next[0];
        pid_cur[1] = pid_next[1];
        const int lo = pid_cur[0], hi = pid_cur[1];
        asm volatile("" ::"s"(lo), "s"(hi));
      }
    };

    // Direct-to-LDS load j (of kDmaPerWave) of tile `it` into stage I: a
    // buffer load whose descriptor starts at the first row of the block's
    // half.
    // Load j of tile `src` into the stage of tile `dst` (dst = src, or a
    // tile past the end whose free stage receives a copy of the last tile).
    auto issue_piece = [&](const int (&pid)[2], int src, int dst, int j) {
      const int base = p0 + src * kTT;
      const int nvalid = p1 - base;  // rows of this tile inside the split (>= 1)
      const int blk = wave + j * kNW;
      uint32_t off = (dma_off[j >> 1] >> (16 * (j & 1))) & 0xffffu;
      // Rows past the split (the split's last tile may be partial) read chunk
      // lane % kCPR of the first row of the half instead, or of the tile when
      // the whole upper half is past the split: finite data that the softmax
      // masks.  A lane's row is past the split iff its offset from the half is
      // at least (nvalid - 16 * half) rows.
      int half = blk >= kPieces / 2 ? 1 : 0;  // uniform
      const int lim = (nvalid - 16 * half) * kRowBytes;
      if (nvalid <= 16) half = 0;
      off = (int)off < lim ? off : 16u * (lane % kCPR);
      long long row;  // first row of the half in the latent (or pool) rows
      if constexpr (MODE == kAddrPaged) {
        row = (long long)pid[half] * pg.stride + ((base + 16 * half) & ((1 << pg.shift) - 1));
      } else {
        row = base + 16 * half;
      }
      dma_16B(lat_b + row * kRowBytes, kTileBytes / 2, off,
              (uint32_t)(uintptr_t)(stage_of(dst) + blk * 1024));
    };
    auto issue_tile = [&](const int (&pid)[2], int src, int dst) {
#pragma unroll
      for (int j = 0; j < kDmaPerWave; ++j)
        if (j < my_pieces) issue_piece(pid, src, dst, j);
    };

    // fp16 conversion of this wave's own loads of a tile: its 1 KiB pieces
    // wave, wave + kNW, ... (chunk `lane` of each), converted in place once
    // they have landed -- no other wave's loads are involved, so no barrier
    // separates a wave's wait from its conversion.
    auto own_chunk = [&](int t, int j) -> uint4* {
      return (uint4*)(stage_of(t) + (wave + j * kNW) * 1024 + 16 * lane);
    };

    // Computes tile `it` from its stage.  The loads of tile it+3 (into the
    // stage of tile it-1, which every wave finished before the barrier) are
    // issued piece by piece between the score MFMAs, so their issue stalls
    // overlap matrix work; fp16: this wave's pieces of tile it+1, landed, are
    // read when the scores are done and written back converted between the
    // heads' softmax updates (the LDS serves no operand reads then; in the
    // score loop the same work competes with them).  Past the last tile the loads fetch a
    // copy of the last tile into that free stage (an L2 hit, never used, and
    // converted like any other): every step issues the same loads and
    // conversions, so the vmcnt waits are the same for all steps.
    auto compute_tile = [&](int it) {
      const unsigned char* tile = stage_of(it);
      const int base = p0 + it * kTT;
      const int next = min(it + kStages - 1, ntiles - 1);
      // page ids of tile it+4, a step ahead of its loads
      fetch_pages(min(it + kStages, ntiles - 1), pid_next);

      // scores.  Chunk (4*ks + lg) ^ swz(t) = 8*(ks/2) + ((4*(ks&1) + lg) ^ swz(t)):
      // two base addresses per row block, the rest is an immediate offset.
      const unsigned char* abase[2][2];  // [row block][chunk parity]
#pragma unroll
      for (int tb = 0; tb < 2; ++tb) {
        const int t = 16 * tb + li;
#pragma unroll
        for (int e = 0; e < 2; ++e)
          abase[tb][e] = tile + t * kRowBytes + 16 * ((4 * e + lg) ^ swz(t));
      }
      f32x4_t sc[2][kHB];
      // operand reads run kAhead k-steps ahead of the MFMAs that use them
      constexpr int kAhead = ATTN_MLA_QK_AHEAD;
      uint4 af[kAhead + 1][2];
#pragma unroll
      for (int k0 = 0; k0 < kAhead; ++k0)
#pragma unroll
        for (int tb = 0; tb < 2; ++tb)
          af[k0][tb] = *(const uint4*)(abase[tb][k0 & 1] + 128 * (k0 >> 1));
#pragma unroll
      for (int ks = 0; ks < kKS; ++ks) {
        // this wave's loads, spread evenly over the k-steps
#pragma unroll
        for (int j = 0; j < kDmaPerWave; ++j)
          if ((j * kKS) / kDmaPerWave == ks && j < my_pieces)
            issue_piece(pid_cur, next, it + kStages - 1, j);
        const int cur = ks % (kAhead + 1);
        const int kn = ks + kAhead;
        if (kn < kKS) {
#pragma unroll
          for (int tb = 0; tb < 2; ++tb)
            af[kn % (kAhead + 1)][tb] = *(const uint4*)(abase[tb][kn & 1] + 128 * (kn >> 1));
        }
#pragma unroll
        for (int tb = 0; tb < 2; ++tb)
#pragma unroll
          for (int hb = 0; hb < kHB; ++hb) {
            if (ks == 0) mfma_first_v<kF16>(sc[tb][hb], as_u32x4(af[cur][tb]), as_u32x4(qf[hb][ks]));
            else mfma_v<kF16>(sc[tb][hb], as_u32x4(af[cur][tb]), as_u32x4(qf[hb][ks]));
          }
      }
      // the softmax reads the scores with VALU instructions
      if constexpr (kHB == 2)
        asm volatile(ATTN_MFMA_DRAIN
                     : "+v"(sc[0][0]), "+v"(sc[0][kHB - 1]), "+v"(sc[1][0]), "+v"(sc[1][kHB - 1]));
      else
        asm volatile(ATTN_MFMA_DRAIN : "+v"(sc[0][0]), "+v"(sc[1][0]));

      // online softmax per head (lazy maximum); weights rounded to fp16, or
      // split into bf16 high parts and remainders
      const bool full = base + kTT <= p1;  // uniform: no masked row in the tile
      uint32_t ph[kHB][4], pl[kHB][4];
      // fp16: this wave's pieces of tile it+1 are read now and converted
      // between the heads' softmax updates, while the LDS is otherwise idle
      uint4 cw[kDmaPerWave];
      if constexpr (kF16) {
#pragma unroll
        for (int j = 0; j < kDmaPerWave; ++j)
          if (j < my_pieces) cw[j] = *own_chunk(it + 1, j);
        __builtin_amdgcn_sched_barrier(0);
      }
#pragma unroll
      for (int hb = 0; hb < kHB; ++hb) {
        // raw scores; the scale (> 0) is applied once to the maximum and fused
        // into the exponent below
        float x[8];
#pragma unroll
        for (int tb = 0; tb < 2; ++tb)
#pragma unroll
          for (int r = 0; r < 4; ++r) x[4 * tb + r] = sc[tb][hb][r];
        if (!full) {
#pragma unroll
          for (int j = 0; j < 8; ++j)
            if (base + 16 * (j >> 2) + 4 * lg + (j & 3) >= p1) x[j] = neg_inf();
        }
        if constexpr (MULTI) {  // each column's token sees positions <= tl
#pragma unroll
          for (int j = 0; j < 8; ++j)
            if (base + 16 * (j >> 2) + 4 * lg + (j & 3) > tl[hb]) x[j] = neg_inf();
        }
        float mt = x[0];
#pragma unroll
        for (int j = 1; j < 8; ++j) mt = fmaxf(mt, x[j]);
        mt = fmaxf(mt, xor16(mt));
        mt = fmaxf(mt, xor32(mt));
        mt *= a.scale_log2;
        if (mt > m[hb] + 8.f) {
          const float al = fast_exp2(m[hb] - mt);
          l[hb] *= al;
          asm volatile(ATTN_MFMA_DRAIN ::: "memory");
#pragma unroll
          for (int db = 0; db < kDB; ++db) {
            // keep the accumulators in AGPRs across this rare VALU update
            asm volatile("" : "+a"(o[db][hb]));
            o[db][hb] *= al;
            asm volatile("" : "+a"(o[db][hb]));
          }
          m[hb] = mt;
        }
        float p[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          // One token: every computed tile has a visible row (the split's
          // rows start at its first tile), so m is finite here and a masked
          // row's -inf gives exp2(-inf) = 0 without a test.  Several tokens:
          // a column may have seen no visible row yet (m = -inf), and
          // -inf - (-inf) would be NaN, so masked rows are set to 0.
          p[j] = (MULTI && x[j] == neg_inf())
                     ? 0.f
                     : fast_exp2(fmaf(x[j], a.scale_log2, -m[hb]));
          l[hb] += p[j];
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          if constexpr (kF16) ph[hb][j] = pack_f16(p[2 * j], p[2 * j + 1]);
          else split_bf16(p[2 * j], p[2 * j + 1], ph[hb][j], pl[hb][j]);
        }
        if constexpr (kF16) {
          // pieces [hb * D / kHB, (hb + 1) * D / kHB) after head block hb
          __builtin_amdgcn_sched_barrier(0);
#pragma unroll
          for (int j = 0; j < kDmaPerWave; ++j)
            if (j * kHB / kDmaPerWave == hb && j < my_pieces)
              *own_chunk(it + 1, j) = bf16x8_to_f16x8(cw[j]);
          __builtin_amdgcn_sched_barrier(0);
        }
      }

      // values: transposed 4x16 reads of rows 4*lg + li/4 (and +16), columns
      // 16*db + 4*(li&3).  Chunk 2*db + ((li&3)>>1) swizzled = 8*(db/4) +
      // ((2*(db&3) + ((li&3)>>1)) ^ swz(t)): four bases, the rest (including
      // the +16 rows, which share the swizzle) an immediate offset.  (One base
      // per read pair also keeps the alias information on every read, so the
      // compiler does not wait for the direct-to-LDS loads of other stages.)
      const int t0 = 4 * lg + (li >> 2);
      const int half = ((li & 3) & 1) * 8;
      const unsigned char* vbase[4];
#pragma unroll
      for (int e = 0; e < 4; ++e)
        vbase[e] = tile + t0 * kRowBytes + 16 * ((2 * e + ((li & 3) >> 1)) ^ swz(t0)) + half;
      typedef s16x4_t __attribute__((address_space(3))) * lds_s16x4;
      auto read_v = [&](int db) {
        const int imm = 128 * (db >> 2);
        const s16x4_t v0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_s16x4)(__attribute__((address_space(3))) unsigned char*)(vbase[db & 3] + imm));
        const s16x4_t v1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_s16x4)(__attribute__((address_space(3))) unsigned char*)(vbase[db & 3] +
                                                                        (16 * kRowBytes + imm)));
        return __builtin_shufflevector(v0, v1, 0, 1, 2, 3, 4, 5, 6, 7);
      };
      typedef short s16x8_t __attribute__((ext_vector_type(8)));
      u32x4 bh[kHB], bl[kHB];
#pragma unroll
      for (int hb = 0; hb < kHB; ++hb) {
        bh[hb] = u32x4{ph[hb][0], ph[hb][1], ph[hb][2], ph[hb][3]};
        if constexpr (!kF16) bl[hb] = u32x4{pl[hb][0], pl[hb][1], pl[hb][2], pl[hb][3]};
      }
      // wait states between the VALU writes of the weights and their MFMAs
      if constexpr (kF16)
        asm volatile("s_nop 4" ::"v"(bh[0]), "v"(bh[kHB - 1]));
      else
        asm volatile("s_nop 4" ::"v"(bh[0]), "v"(bl[0]), "v"(bh[kHB - 1]), "v"(bl[kHB - 1]));
      // transposed value reads run kVAhead blocks ahead of their MFMAs
      constexpr int kVAhead = ATTN_MLA_V_AHEAD < kDB ? ATTN_MLA_V_AHEAD : kDB - 1;
      s16x8_t vf[kVAhead + 1];
#pragma unroll
      for (int db = 0; db < kVAhead; ++db) vf[db] = read_v(db);
#pragma unroll
      for (int db = 0; db < kDB; ++db) {
        if (db + kVAhead < kDB) vf[(db + kVAhead) % (kVAhead + 1)] = read_v(db + kVAhead);
        const u32x4 av = __builtin_bit_cast(u32x4, vf[db % (kVAhead + 1)]);
#pragma unroll
        for (int hb = 0; hb < kHB; ++hb) {
          mfma_a<kF16>(o[db][hb], av, bh[hb]);
          if constexpr (!kF16) mfma_a<kF16>(o[db][hb], av, bl[hb]);
        }

      }
      // The compiler does not see these MFMAs, and where steps join it may
      // move an accumulator to other registers: their latency is waited out
      // before any such copy can read them.
      asm volatile(ATTN_MFMA_DRAIN ::: "memory");
#pragma unroll
      for (int db = 0; db < kDB; ++db)
#pragma unroll
        for (int hb = 0; hb < kHB; ++hb) asm volatile("" : "+a"(o[db][hb]));
    };

    // One pipeline step: tile `it` is computed (and, fp16, tile it+1 converted)
    // while the later tiles land and tile it+3 is issued.
    constexpr int kLanding = kF16 ? kStages - 3 : kStages - 2;  // tiles still landing
    auto step = [&](int it) {
      if (it >= ntiles) return;
      // fp16: this wave's loads of tile it+1 (converted during this step) must
      // have landed, those of later tiles may still be in flight, and the
      // barrier publishes tile it (converted by every wave during the step
      // before).  bf16: tile it must have landed.
      if (my_pieces == kDmaPerWave) wait_vmcnt<kLanding * kDmaPerWave>();
      else wait_vmcnt<kLanding * (kDmaPerWave - 1)>();
      lds_barrier();
      pages_ready();
      compute_tile(it);
    };

    if (ntiles > 0) {
#pragma unroll
      for (int t = 0; t + 1 < kStages; ++t) {
        int pid[2];
        fetch_pages(min(t, ntiles - 1), pid);
        issue_tile(pid, min(t, ntiles - 1), t);
      }
      fetch_pages(min(kStages - 1, ntiles - 1), pid_next);
      // the query fragments (and the first tiles) land here, once: the loop
      // then carries no wait on the query loads
      wait_vmcnt<0>();
      if constexpr (kF16) {
        // the queries and this wave's pieces of tile 0 go to fp16 here (step
        // 0's barrier publishes tile 0)
#pragma unroll
        for (int hb = 0; hb < kHB; ++hb)
#pragma unroll
          for (int ks = 0; ks < kKS; ++ks) qf[hb][ks] = bf16x8_to_f16x8(qf[hb][ks]);
#pragma unroll
        for (int j = 0; j < kDmaPerWave; ++j)
          if (j < my_pieces) *own_chunk(0, j) = bf16x8_to_f16x8(*own_chunk(0, j));
      }
      for (int it = 0; it < ntiles; ++it) step(it);
      // the last steps' loads (unused) must land before the group's LDS is
      // released
      wait_vmcnt<0>();
    }

    asm volatile(ATTN_MFMA_DRAIN ::: "memory");
#pragma unroll
    for (int db = 0; db < kDB; ++db)
#pragma unroll
      for (int hb = 0; hb < kHB; ++hb) asm volatile("" : "+a"(o[db][hb]));
    // per-head sums of the four lane groups, then write this wave's heads
#pragma unroll
    for (int hb = 0; hb < kHB; ++hb) {
      l[hb] += xor16(l[hb]);
      l[hb] += xor32(l[hb]);
    }
#pragma unroll
    for (int hb = 0; hb < kHB; ++hb) {
      const int c = hw0 + 16 * hb + li;
      if (c >= a.ncol) continue;
      const bool empty = !(l[hb] > 0.f);
      const float inv = empty ? 0.f : 1.f / l[hb];
      const float lse = empty ? neg_inf() : (m[hb] + fast_log2(l[hb])) * kLn2;
      const size_t row = query_row(b, 0, c, a.H, a.L, a.H);
      const size_t prow =
          LIST == 0 ? row * a.S + slot : (size_t)slot * kHG + (c - hc * kHG);
      if (kF16 && !direct) {
        // fp16 partials: a weighted mean of latent values, inside fp16's range
        // whenever the latent is
        uint16_t* dst = (uint16_t*)a.o_part + prow * kDV;
#pragma unroll
        for (int db = 0; db < kDB; ++db) {
          const f32x4_t v = o[db][hb] * inv;
          *(uint2*)(dst + 16 * db + 4 * lg) = make_uint2(pack_f16(v[0], v[1]),
                                                          pack_f16(v[2], v[3]));
        }
      } else {
        float* dst = direct ? a.out + row * kDV : a.o_part + prow * kDV;
#pragma unroll
        for (int db = 0; db < kDB; ++db)
          *(f32x4_t*)(dst + 16 * db + 4 * lg) = o[db][hb] * inv;
      }
      if (lg == 0) {
        if (direct) {
          if (a.lse) a.lse[row] = lse;
        } else {
          a.lse_part[prow] = lse;
        }
      }
    }
  };  // process

  if constexpr (LIST == 2) {
    // even split: this group's range of the line, one segment per unit
    const int U = a.head_chunks;
    const EvenPlanLds ep = even_plan_lds(a.seq_lens, a.B, a.T_cap, 0, nullptr, 0, U,
                                         a.cap, kTT, a.even_lead, 8, plan_lds);
    if (item >= ep.groups) return;  // uniform over the work group
    const int x1 = even_start(ep, item + 1);
    int x = even_start(ep, item);
    bool first = true;
    while (x < x1) {
      const EvenSeg sg = even_segment(ep, x, x1);
      x = sg.next;
      if (sg.t1 == sg.t0) continue;  // only lead tiles of this unit
      // every wave is done with the previous segment's stages before the
      // next segment's loads go out
      if (!first) __syncthreads();
      first = false;
      const int b = __builtin_amdgcn_readfirstlane(sg.b);
      const int ui = b * U + sg.u;
      if (sg.t0 == 0 && threadIdx.x == 0) {  // the group holding the unit's start
        a.meta[2 * ui] = sg.first + ui;
        a.meta[2 * ui + 1] = sg.last - sg.first + 1;
      }
      const VisibleRange vr = visible_range_of(sg.len, false, 0, a.T_cap, 0);
      const int p0 = min(sg.t0 * kTT, vr.n), p1 = min(sg.t1 * kTT, vr.n);
      process(b, sg.u, vr, p0, p1, sg.first == sg.last, item + ui);
    }
  } else {
    int hc, s, b, n_split = a.S, chunk = a.chunk, len_b = 0;
    if constexpr (LIST == 1) {
      // item r of sequence b: s * head_chunks + hc; pieces are whole tiles
      const WorkItem wi = balanced_item(a.seq_lens, nullptr, a.B, a.T_cap, 0, nullptr, 0,
                                        a.head_chunks, a.cap, kTT, 2 * kTT, item);
      if (!wi.valid) return;  // uniform over the work group
      // uniform values, kept in scalar registers (the tile loads' descriptors
      // are built from them)
      b = __builtin_amdgcn_readfirstlane(wi.b);
      len_b = __builtin_amdgcn_readfirstlane(wi.len);
      n_split = __builtin_amdgcn_readfirstlane(wi.k);
      chunk = __builtin_amdgcn_readfirstlane(wi.chunk);
      const int r = __builtin_amdgcn_readfirstlane(wi.r);
      hc = r % a.head_chunks;
      s = r / a.head_chunks;
      if (wi.r == 0 && threadIdx.x == 0) {
        a.meta[2 * b] = wi.first;
        a.meta[2 * b + 1] = wi.k;
      }
    } else {
      int bid = item;
      hc = bid % a.head_chunks;
      bid /= a.head_chunks;
      s = bid % a.S;
      b = bid / a.S;
    }

    const VisibleRange vr = LIST == 1 ? visible_range_of(len_b, false, 0, a.T_cap, 0)
                                : visible_range(a.seq_lens, nullptr, b, a.T_cap, 0);
    int p0, p1;
    split_range(vr, s, n_split, chunk, p0, p1);  // no window: rows = positions
    process(b, hc, vr, p0, p1, n_split == 1, LIST == 1 ? item : s);
  }
}

}  // namespace

int mla_heads_per_group(int d_c) { return d_c == 512 ? GeoWide::kHG : GeoNarrow::kHG; }
int mla_groups_per_cu(int d_c) {
  return d_c == 512 ? GeoWide::kGroupsPerCU : GeoNarrow::kGroupsPerCU;
}
int mla_tile_rows() { return kTT; }
bool mla_even_split(int d_c) { return d_c == 512 ? GeoWide::kF16 : GeoNarrow::kF16; }
bool mla_half_parts(int d_c) { return d_c == 512 ? GeoWide::kF16 : GeoNarrow::kF16; }

namespace {
template <class G, int LIST>
void launch_list(const MlaArgs& a, dim3 g, bool paged, hipStream_t stream) {
  const dim3 blk(G::kNW * 64);
  // several tokens: not with the even split (the planner keeps the
  // per-sequence list there; that instantiation would spill)
  if constexpr (LIST != 2) {
    if (a.L > 1) {
      if (paged)
        hipLaunchKernelGGL((mla_decode_mfma<G, kAddrPaged, true, LIST>), g, blk, 0, stream, a);
      else
        hipLaunchKernelGGL((mla_decode_mfma<G, kAddrDense, true, LIST>), g, blk, 0, stream, a);
      return;
    }
  }
  if (paged)
    hipLaunchKernelGGL((mla_decode_mfma<G, kAddrPaged, false, LIST>), g, blk, 0, stream, a);
  else
    hipLaunchKernelGGL((mla_decode_mfma<G, kAddrDense, false, LIST>), g, blk, 0, stream, a);
}
template <class G>
hipError_t launch_geo(const MlaArgs& a, dim3 g, bool paged, hipStream_t stream) {
  if (a.balanced == 2) {
    // the even split's plan takes 3 KiB of LDS: the fp16 geometry has it
    // free, the narrow one would lose its second group per CU; one token
    if constexpr (!G::kF16) return hipErrorInvalidValue;
    else if (a.L > 1) return hipErrorInvalidValue;
    else launch_list<G, 2>(a, g, paged, stream);
  } else if (a.balanced) {
    launch_list<G, 1>(a, g, paged, stream);
  } else {
    launch_list<G, 0>(a, g, paged, stream);
  }
  return hipGetLastError();
}
}  // namespace

hipError_t launch_mla_mfma(const void* q, const void* latent, float* out,
                           float* lse, float* o_part, float* lse_part,
                           const int32_t* seq_lens, const int32_t* block_table,
                           int max_pages, int page_shift, int num_pages, int B,
                           int L, int H, int T_cap, int d_c, int S, int chunk,
                           int head_chunks, int balanced, int cap, int* meta,
                           int even_lead, float scale_log2, hipStream_t stream) {
  MlaArgs a;
  a.q = (const uint16_t*)q;
  a.latent = (const uint16_t*)latent;
  a.block_table = block_table;
  a.max_pages = max_pages;
  a.page_shift = page_shift;
  a.num_pages = num_pages;
  a.out = out;
  a.lse = lse;
  a.o_part = o_part;
  a.lse_part = lse_part;
  a.seq_lens = seq_lens;
  a.H = H;
  a.L = L;
  a.ncol = H * L;
  a.T_cap = T_cap;
  a.S = S;
  a.chunk = chunk;
  a.head_chunks = head_chunks;
  a.scale_log2 = scale_log2;
  a.balanced = balanced;
  a.cap = cap;
  a.B = B;
  a.meta = meta;
  a.even_lead = even_lead;
  const dim3 g((unsigned)(balanced ? (long long)cap : (long long)B * S * head_chunks));
  if (d_c == 512) return launch_geo<GeoWide>(a, g, block_table != nullptr, stream);
  return launch_geo<GeoNarrow>(a, g, block_table != nullptr, stream);
}

}  // namespace attn
