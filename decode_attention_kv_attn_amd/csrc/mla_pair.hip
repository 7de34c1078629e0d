// Absorbed MLA decode of the 512 + 64 latent on the matrix cores, the work
// of every tile split by role (kernel 4, fixed splits).
//
// The products are those of the shared-latent kernel (xuesongtap
// "attention-head" note, sections 5.2-5.3: keys absorbed into the query, the
// RoPE key shared by all heads, values projected after the weighted sum):
//
//   S^T[tokens, heads] = L[tokens, 0:576] . Q^T[576, heads]
//   Z^T[0:512, heads] += L[tokens, 0:512]^T . P^T[tokens, heads]
//
// Here a work group holds 64 (head, token) columns, so the 128 heads of a
// sequence take two groups, and those two are placed on one XCD so the
// second read of each latent tile is served by that XCD's L2.  Halving the
// columns halves the outputs (64 x 512 fp32) and queries (64 x 576 bf16) a
// CU keeps in registers, which makes room for two waves per SIMD, and the
// eight waves split each tile's work by role:
//
//   * four score waves, 16 columns each: queries in registers (bf16), the
//     scores of all 32 rows on v_mfma_f32_16x16x32_bf16 (exact products),
//     the online softmax (lazy maximum), and the tile's weights written to
//     LDS as fp16 value-product operands, with each column's rescale factor;
//     they also issue the tile loads, between their score MFMAs;
//   * four value waves, 128 output columns each for all 64 columns: the
//     transposed latent values read through ds_read_b64_tr_b16, converted
//     bf16 -> fp16 in registers, and v_mfma_f32_16x16x32_f16 with the
//     weights.
//
// Each SIMD runs one wave of each role, so one wave's LDS reads and softmax
// overlap the other's matrix work.  The value waves trail the score waves by
// one tile: step i scores tile i while tile i-1's values are accumulated;
// one barrier per step.  Tiles of 32 rows go straight from HBM into four LDS
// stages with direct-to-LDS buffer loads two tiles ahead (a stage serves the
// scores of its tile in one step and the values in the next).
//
// Precision: as the shared-latent kernel's fp16 geometry -- a bf16 value
// converts exactly when 2^-14 <= |x| <= 65504 (smaller ones with an absolute
// error below 2^-25), weights enter the value product rounded to fp16, and
// a split's partial values (weighted means) are stored as fp16.

#include "device_common.h"
#include "internal.h"
#include "mla_common.h"
#include "visible.h"

namespace attn {
namespace {

constexpr int kRows = 32;                   // rows per tile
constexpr int kLat = 576, kVal = 512;       // latent row and value widths
constexpr int kRowB = kLat * 2;             // bytes per latent row
constexpr int kChunks = kRowB / 16;         // 16-byte chunks per row
constexpr int kTileB = kRows * kRowB;       // 36 KiB
constexpr int kLoads = kTileB / 1024;       // 1 KiB loads per tile
constexpr int kNStage = 4;
constexpr int kCols = 64;                   // (head, token) columns per group
constexpr int kKSteps = kLat / 32;          // score k-steps
constexpr int kLoadsPerW = kLoads / 4;      // tile loads issued by each score wave
constexpr int kVBlocks = kVal / 4 / 16;     // 16-column value blocks per value wave
static_assert(kLoads % 4 == 0 && (kLoads / 2) * 1024 == 16 * kRowB, "tile halves");
static_assert(kChunks % 8 == 0, "the swizzle permutes aligned groups of 8 chunks");

#ifndef ATTN_MLA_PAIR_AHEAD  // k-steps the score operand reads run ahead
#define ATTN_MLA_PAIR_AHEAD 6
#endif

typedef __bf16 bf16x8_v __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8_v __attribute__((ext_vector_type(8)));
typedef short s16x8_t __attribute__((ext_vector_type(8)));

ATTN_DEV f32x4_t mfma_bf16(const uint4& a, const uint4& b, const f32x4_t& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_v, a),
                                                 __builtin_bit_cast(bf16x8_v, b), c, 0, 0, 0);
}
ATTN_DEV f32x4_t mfma_f16(const uint4& a, const uint4& b, const f32x4_t& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8_v, a),
                                                __builtin_bit_cast(f16x8_v, b), c, 0, 0, 0);
}

struct PairArgs {
  const uint16_t* q;           // query rows of 576 bf16 (row query_row(b, 0, c, H, L, H))
  const uint16_t* latent;      // [B, T_cap, 576], or the page pool [num_pages, P, 576]
  const int32_t* block_table;  // [B, max_pages] (paged only)
  int max_pages, page_shift, num_pages;
  float* out;                  // [B, L, H, 512] when S == 1
  float* lse;                  // [B, L, H] (nullable) when S == 1
  uint16_t* o_part;            // fp16 [B * L * H, S, 512] when S > 1
  float* lse_part;             // [B * L * H, S]
  const int32_t* seq_lens;
  int H, L, ncol, T_cap, S, chunk, head_chunks;
  float scale_log2;
};

template <int MODE, bool MULTI>
__global__ __launch_bounds__(512) void mla_pair_decode(PairArgs a) {
  __shared__ __attribute__((aligned(1024))) unsigned char stages[kNStage * kTileB];
  // weights of tile t as the value product's operands: [t & 1][column block][lane]
  __shared__ __attribute__((aligned(16))) uint4 wbuf[2][4][64];
  __shared__ float alpha[2][kCols];                        // rescale factor per column
  __shared__ __attribute__((aligned(16))) int grew[2][4];  // any column of the block
  __shared__ float fin_l[kCols];                           // final sums per column

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int li = lane & 15;
  const int lg = lane >> 4;
  const int r4 = wave & 3;  // score wave: column block; value wave: value quarter

  // Work item: the head chunks of one (sequence, split) unit go to one XCD
  // (work groups are dealt to the XCDs in turn), so they share its L2.
  const int hcs = a.head_chunks;
  const int x = blockIdx.x;
  const int per = kNumXCDs * hcs;
  const int full = (int)gridDim.x / per * per;
  int hc, unit;
  if (x < full) {
    hc = (x / kNumXCDs) % hcs;
    unit = x / per * kNumXCDs + x % kNumXCDs;
  } else {
    const int r = x - full;
    hc = r % hcs;
    unit = full / hcs + r / hcs;
  }
  const int s = unit % a.S;
  const int b = unit / a.S;

  const VisibleRange vr = visible_range(a.seq_lens, nullptr, b, a.T_cap, 0);
  int p0, p1;
  split_range(vr, s, a.S, a.chunk, p0, p1);  // no window: rows = positions
  const int ntiles = p1 > p0 ? (p1 - p0 + kRows - 1) / kRows : 0;
  const bool direct = a.S == 1;
  auto stage = [&](int t) { return stages + (t % kNStage) * kTileB; };

  if (wave < 4) {
    // ------------------------------------------------------------ score wave
    const int col = hc * kCols + 16 * r4 + li;
    // Q^T fragments of column col: elements 32*ks + 8*lg .. +7
    uint4 qf[kKSteps];
    {
      const uint16_t* qp =
          a.q + query_row(b, 0, min(col, a.ncol - 1), a.H, a.L, a.H) * kLat + 8 * lg;
#pragma unroll
      for (int ks = 0; ks < kKSteps; ++ks)
        qf[ks] = col < a.ncol ? *(const uint4*)(qp + 32 * ks) : make_uint4(0, 0, 0, 0);
    }
    const int tl = vr.hi - a.L + col % a.L;  // several tokens: last visible position
    float m = neg_inf(), l = 0.f;

    const unsigned char* lat_b =
        (const unsigned char*)(MODE == kAddrPaged ? a.latent
                                                  : a.latent + (size_t)b * a.T_cap * kLat);
    Pages pg{};
    if constexpr (MODE == kAddrPaged)
      pg = page_view(a.block_table, a.max_pages, b, vr.hi, a.page_shift, a.num_pages, 1);

    // This wave's loads of a tile are the 1 KiB blocks r4, r4 + 4, ... : LDS
    // chunk p = blk*64 + lane holds row p / 72, logical chunk (p % 72) ^
    // swz(row).  Blocks below 18 lie in rows 0..15, the others in rows
    // 16..31 (one page each); byte offsets from the half are < 2^16.
    uint32_t dma_off[(kLoadsPerW + 1) / 2];
#pragma unroll
    for (int j = 0; j < kLoadsPerW; ++j) {
      const int p = (r4 + 4 * j) * 64 + lane;
      const int row = p / kChunks;
      const uint32_t off = (row & 15) * kRowB + 16 * ((p - row * kChunks) ^ swz(row));
      if (j & 1) dma_off[j >> 1] |= off << 16;
      else dma_off[j >> 1] = off;
    }

    // Page ids of the two 16-row halves of a tile (paged caches), clamped to
    // the pool, with scalar buffer loads a step ahead of the tile's loads.
    int pid_cur[2] = {}, pid_next[2] = {};
    u32x4 table_rsrc = {};
    if constexpr (MODE == kAddrPaged) {
      const uint64_t tp = (uint64_t)(uintptr_t)pg.table;
      table_rsrc = u32x4{(uint32_t)tp, (uint32_t)(tp >> 32) & 0xffffu,
                         (uint32_t)a.max_pages * 4u, (uint32_t)kBufferWord3};
    }
    auto fetch_pages = [&](int t, int (&pid)[2]) {
      if constexpr (MODE == kAddrPaged) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const int j = min((p0 + t * kRows + 16 * h) >> pg.shift, pg.last);
          const int pv = scalar_buffer_load_i32(table_rsrc, 4 * j, 0);
          pid[h] = pv < 0 ? 0 : (pv >= pg.num_pages ? pg.num_pages - 1 : pv);
        }
      }
    };
    auto pages_ready = [&]() {
      if constexpr (MODE == kAddrPaged) {
        pid_cur[0] = pid_next[0];
        pid_cur[1] = pid_next[1];
        const int lo = pid_cur[0], hi = pid_cur[1];
        asm volatile("" ::"s"(lo), "s"(hi));
      }
    };
    // Load j of tile `src` into the stage of tile `dst` (dst = src, or a
    // tile past the end whose free stage receives a copy of the last tile,
    // so that every step issues the same loads and waits alike).
    auto issue_piece = [&](const int (&pid)[2], int src, int dst, int j) {
      const int base = p0 + src * kRows;
      const int nvalid = p1 - base;  // rows of this tile inside the split (>= 1)
      const int blk = r4 + 4 * j;
      uint32_t off = (dma_off[j >> 1] >> (16 * (j & 1))) & 0xffffu;
      // Rows past the split read chunk lane % 72 of the first row of the half
      // (of the tile when the whole upper half is past it): finite data that
      // the weights (0 there) cancel.
      int half = blk >= kLoads / 2 ? 1 : 0;
      const int lim = (nvalid - 16 * half) * kRowB;
      if (nvalid <= 16) half = 0;
      off = (int)off < lim ? off : 16u * (lane % kChunks);
      long long row;
      if constexpr (MODE == kAddrPaged)
        row = (long long)pid[half] * pg.stride + ((base + 16 * half) & ((1 << pg.shift) - 1));
      else
        row = base + 16 * half;
      dma_16B(lat_b + row * kRowB, kTileB / 2, off,
              (uint32_t)(uintptr_t)(stage(dst) + blk * 1024));
    };

    // Scores of tile t; this wave's loads of tile t + 2 (into the stage tile
    // t - 2 has left; past the end a copy of the last tile, so that every
    // step issues the same loads and waits alike) go out between the MFMAs.
    auto score_tile = [&](int t) {
      const unsigned char* tile = stage(t);
      const int src = min(t + 2, ntiles - 1);
      // Chunk (4*ks + lg) ^ swz(row) = 8*(ks/2) + ((4*(ks&1) + lg) ^ swz(row)):
      // two base addresses per row block, the rest an immediate offset.
      const unsigned char* ab[2][2];
#pragma unroll
      for (int tb = 0; tb < 2; ++tb) {
        const int row = 16 * tb + li;
#pragma unroll
        for (int e = 0; e < 2; ++e)
          ab[tb][e] = tile + row * kRowB + 16 * ((4 * e + lg) ^ swz(row));
      }
      // Operand reads run kAh k-steps ahead of their MFMAs.  The scheduling
      // barriers keep that order: left alone, the scheduler moves each read
      // next to its MFMA, which then waits out a whole LDS latency.
      constexpr int kAh = ATTN_MLA_PAIR_AHEAD;
      uint4 af[kAh + 1][2];
#pragma unroll
      for (int k0 = 0; k0 < kAh; ++k0)
#pragma unroll
        for (int tb = 0; tb < 2; ++tb)
          af[k0][tb] = *(const uint4*)(ab[tb][k0 & 1] + 128 * (k0 >> 1));
      __builtin_amdgcn_sched_barrier(0);
      f32x4_t sc[2] = {f32x4_t{0.f, 0.f, 0.f, 0.f}, f32x4_t{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
      for (int ks = 0; ks < kKSteps; ++ks) {
#pragma unroll
        for (int j = 0; j < kLoadsPerW; ++j)
          if ((j * kKSteps) / kLoadsPerW == ks) issue_piece(pid_cur, src, t + 2, j);
        const int kn = ks + kAh;
        if (kn < kKSteps) {
#pragma unroll
          for (int tb = 0; tb < 2; ++tb)
            af[kn % (kAh + 1)][tb] = *(const uint4*)(ab[tb][kn & 1] + 128 * (kn >> 1));
        }
#pragma unroll
        for (int tb = 0; tb < 2; ++tb)
          sc[tb] = mfma_bf16(af[ks % (kAh + 1)][tb], qf[ks], sc[tb]);
        __builtin_amdgcn_sched_barrier(0);
      }

      // Online softmax of column col over the tile's rows: this lane holds
      // rows 16*tb + 4*lg + r (value-product k index 8*lg + 4*tb + r).
      const int base = p0 + t * kRows;
      float xv[8];
#pragma unroll
      for (int tb = 0; tb < 2; ++tb)
#pragma unroll
        for (int r = 0; r < 4; ++r) xv[4 * tb + r] = sc[tb][r];
      if (base + kRows > p1) {
#pragma unroll
        for (int j = 0; j < 8; ++j)
          if (base + 16 * (j >> 2) + 4 * lg + (j & 3) >= p1) xv[j] = neg_inf();
      }
      if constexpr (MULTI) {  // each column's token sees positions <= tl
#pragma unroll
        for (int j = 0; j < 8; ++j)
          if (base + 16 * (j >> 2) + 4 * lg + (j & 3) > tl) xv[j] = neg_inf();
      }
      float mt = xv[0];
#pragma unroll
      for (int j = 1; j < 8; ++j) mt = fmaxf(mt, xv[j]);
      mt = fmaxf(mt, xor16(mt));
      mt = fmaxf(mt, xor32(mt));
      mt *= a.scale_log2;  // raw scores; the scale (> 0) is fused below
      float al = 1.f;
      const bool grow = mt > m + 8.f;  // lazy: weights stay below 2^8
      if (grow) {
        al = fast_exp2(m - mt);
        l *= al;
        m = mt;
      }
      float pw[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        // One token: every tile has a visible row, so m is finite and a
        // masked row gives exp2(-inf) = 0.  Several tokens: a column may have
        // seen no visible row yet (m = -inf), so masked rows are set to 0.
        pw[j] = (MULTI && xv[j] == neg_inf()) ? 0.f
                                              : fast_exp2(fmaf(xv[j], a.scale_log2, -m));
        l += pw[j];
      }
      const int par = t & 1;
      wbuf[par][r4][lane] = make_uint4(pack_f16(pw[0], pw[1]), pack_f16(pw[2], pw[3]),
                                       pack_f16(pw[4], pw[5]), pack_f16(pw[6], pw[7]));
      if (lg == 0) alpha[par][16 * r4 + li] = al;
      const bool any = __ballot(grow) != 0ull;
      if (lane == 0) grew[par][r4] = any ? 1 : 0;
    };

    if (ntiles > 0) {
      {
        int pid[2];
        fetch_pages(0, pid);
#pragma unroll
        for (int j = 0; j < kLoadsPerW; ++j) issue_piece(pid, 0, 0, j);
        fetch_pages(min(1, ntiles - 1), pid);
#pragma unroll
        for (int j = 0; j < kLoadsPerW; ++j) issue_piece(pid, min(1, ntiles - 1), 1, j);
      }
      fetch_pages(min(2, ntiles - 1), pid_next);
      // the query fragments and the first two tiles land here, once: the
      // loop then carries no wait on the query loads
      wait_vmcnt<0>();
      for (int st = 0; st <= ntiles; ++st) {
        lds_barrier();
        pages_ready();
        if (st < ntiles) {
          score_tile(st);
        } else {
#pragma unroll
          for (int j = 0; j < kLoadsPerW; ++j) issue_piece(pid_cur, ntiles - 1, st + 2, j);
        }
        fetch_pages(min(st + 3, ntiles - 1), pid_next);
        wait_vmcnt<kLoadsPerW>();  // tile st + 1 has landed
      }
      // the last steps' loads (unused copies) land before the LDS is released
      wait_vmcnt<0>();
    }
    l += xor16(l);
    l += xor32(l);
    if (lg == 0) {
      fin_l[16 * r4 + li] = l;
      if (col < a.ncol) {
        const bool empty = !(l > 0.f);
        const float lse = empty ? neg_inf() : (m + fast_log2(l)) * kLn2;
        const size_t row = query_row(b, 0, col, a.H, a.L, a.H);
        if (direct) {
          if (a.lse) a.lse[row] = lse;
        } else {
          a.lse_part[row * a.S + s] = lse;
        }
      }
    }
    lds_barrier();
  } else {
    // ------------------------------------------------------------ value wave
    const int v = r4;  // output columns 128*v .. 128*v + 127
    f32x4_t o[kVBlocks][4];
#pragma unroll
    for (int db = 0; db < kVBlocks; ++db)
#pragma unroll
      for (int hb = 0; hb < 4; ++hb) o[db][hb] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    // Transposed value reads: rows 4*lg + li/4 (and +16), columns
    // 16*db + 4*(li&3) of this wave's quarter.  Chunk 2*db + ((li&3)>>1)
    // swizzled = 8*(db/4) + ((2*(db&3) + ((li&3)>>1)) ^ swz(row)): four bases,
    // the rest (the +16 rows share the swizzle) an immediate offset.
    const int t0 = 4 * lg + (li >> 2);
    const int hoff = (li & 1) * 8;
    int voff[4];
#pragma unroll
    for (int e = 0; e < 4; ++e)
      voff[e] = t0 * kRowB + 16 * ((2 * e + ((li & 3) >> 1)) ^ swz(t0)) + hoff;

    // Values of tile t.
    auto value_tile = [&](int t) {
      const unsigned char* tile = stage(t);
      const int par = t & 1;
      typedef s16x4_t __attribute__((address_space(3))) * lds_s16x4;
      auto read_v = [&](int db) {
        const unsigned char* p = tile + voff[db & 3] + 128 * (2 * v + (db >> 2));
        const s16x4_t v0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_s16x4)(__attribute__((address_space(3))) unsigned char*)p);
        const s16x4_t v1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_s16x4)(__attribute__((address_space(3))) unsigned char*)(p + 16 * kRowB));
        return __builtin_bit_cast(uint4, __builtin_shufflevector(v0, v1, 0, 1, 2, 3, 4, 5, 6, 7));
      };
      // The rescale flags are read first, then the weights and every value
      // block of the step at once: these reads queue behind the score waves'
      // operand reads, so the step waits out that latency once, not per
      // block (order held by scheduling barriers, as in the score loop).
      constexpr int kVAh = kVBlocks;
      const int4 gr = *(const int4*)&grew[par][0];
      uint4 pf[4];
#pragma unroll
      for (int hb = 0; hb < 4; ++hb) pf[hb] = wbuf[par][hb][lane];
      uint4 vr_[kVAh + 1];
#pragma unroll
      for (int db = 0; db < kVAh; ++db) vr_[db] = read_v(db);
      __builtin_amdgcn_sched_barrier(0);
      if (t > 0) {  // before tile 0 the outputs are zero
        const int g4[4] = {gr.x, gr.y, gr.z, gr.w};
#pragma unroll
        for (int hb = 0; hb < 4; ++hb) {
          if (g4[hb]) {
            const float al = alpha[par][16 * hb + li];
#pragma unroll
            for (int db = 0; db < kVBlocks; ++db) o[db][hb] *= al;
          }
        }
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int db = 0; db < kVBlocks; ++db) {
        if (db + kVAh < kVBlocks) vr_[(db + kVAh) % (kVAh + 1)] = read_v(db + kVAh);
        const uint4 vf = bf16x8_to_f16x8(vr_[db % (kVAh + 1)]);
#pragma unroll
        for (int hb = 0; hb < 4; ++hb) o[db][hb] = mfma_f16(vf, pf[hb], o[db][hb]);
        __builtin_amdgcn_sched_barrier(0);
      }
    };

    if (ntiles > 0) {
      for (int st = 0; st <= ntiles; ++st) {
        lds_barrier();
        if (st > 0) value_tile(st - 1);
      }
    }
    lds_barrier();  // the score waves' final sums

    // Outputs: column 16*hb + li of the group, values 128*v + 16*db + 4*lg .. +3.
#pragma unroll
    for (int hb = 0; hb < 4; ++hb) {
      const int c = hc * kCols + 16 * hb + li;
      if (c >= a.ncol) continue;
      const float lsum = fin_l[16 * hb + li];
      const float inv = lsum > 0.f ? 1.f / lsum : 0.f;
      const size_t row = query_row(b, 0, c, a.H, a.L, a.H);
      if (direct) {
        float* dst = a.out + row * kVal + 128 * v + 4 * lg;
#pragma unroll
        for (int db = 0; db < kVBlocks; ++db) *(f32x4_t*)(dst + 16 * db) = o[db][hb] * inv;
      } else {
        // fp16 partials: weighted means of latent values, inside fp16's range
        // whenever the latent is
        uint16_t* dst = a.o_part + (row * a.S + s) * kVal + 128 * v + 4 * lg;
#pragma unroll
        for (int db = 0; db < kVBlocks; ++db) {
          const f32x4_t w = o[db][hb] * inv;
          *(uint2*)(dst + 16 * db) = make_uint2(pack_f16(w[0], w[1]), pack_f16(w[2], w[3]));
        }
      }
    }
  }
}

}  // namespace

int mla_pair_columns() { return kCols; }

hipError_t launch_mla_pair(const void* q, const void* latent, float* out, float* lse,
                           void* o_part, float* lse_part, const int32_t* seq_lens,
                           const int32_t* block_table, int max_pages, int page_shift,
                           int num_pages, int B, int L, int H, int T_cap, int S, int chunk,
                           int head_chunks, float scale_log2, hipStream_t stream) {
  PairArgs a;
  a.q = (const uint16_t*)q;
  a.latent = (const uint16_t*)latent;
  a.block_table = block_table;
  a.max_pages = max_pages;
  a.page_shift = page_shift;
  a.num_pages = num_pages;
  a.out = out;
  a.lse = lse;
  a.o_part = (uint16_t*)o_part;
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
  const dim3 g((unsigned)((long long)B * S * head_chunks)), blk(512);
  const bool paged = block_table != nullptr;
  if (L > 1) {
    if (paged) hipLaunchKernelGGL((mla_pair_decode<kAddrPaged, true>), g, blk, 0, stream, a);
    else hipLaunchKernelGGL((mla_pair_decode<kAddrDense, true>), g, blk, 0, stream, a);
  } else {
    if (paged) hipLaunchKernelGGL((mla_pair_decode<kAddrPaged, false>), g, blk, 0, stream, a);
    else hipLaunchKernelGGL((mla_pair_decode<kAddrDense, false>), g, blk, 0, stream, a);
  }
  return hipGetLastError();
}

}  // namespace attn
