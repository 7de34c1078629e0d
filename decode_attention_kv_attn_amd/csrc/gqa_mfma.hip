// Decode attention on the matrix cores for head groups of 3 or more (GQA
// through MQA).
//
// When several query heads share one KV head (xuesongtap "attention-head"
// note, sections 2.1-2.2; MQA at 32 heads is the extreme), every K and V row
// serves all of them, and the scores of a tile are a dense product
// [tokens x d] . [d x heads].  The vector ALUs fall behind HBM from about
// six heads per row on (2n flop per K/V element), and even at four the
// matrix cores free the vector units for the softmax, so both products run
// on MFMA 16x16x32 (bf16 in, fp32 accumulate), with the head block padded
// to 16 or 32 columns:
//
//   S^T[tokens, heads] = K_tile[tokens, d] . Q^T[d, heads]
//       A = K rows straight from HBM (each lane's 8 elements are 16
//       contiguous bytes of one row), B = Q^T fragments kept in registers.
//   O^T[d, heads] += V_tile^T[d, tokens] . P^T[tokens, heads]
//       A = V^T fragments read from an LDS copy of the V tile with
//       ds_read_b64_tr_b16 (a 4x16 transpose per 16-lane group), B = the
//       softmax weights, which the S^T result already holds in the right
//       lanes (token order inside the 32-token k-block is permuted the same
//       way on both operands).
//
// The weights keep ~16 significant bits: P = P_hi + P_lo with both parts in
// bf16, so the second product costs two MFMAs per block; P in bf16 alone
// would carry a relative error of about 2^-9 per weight.
//
// Work item = (sequence, KV head, head chunk of NH query heads, split);
// four waves take the split's 32-token tiles in turn and are merged by the
// log-sum-exp rule through LDS.  Softmax state is per head and lives in the
// lanes that own that head (lane % 16), so rescaling O^T is lane-local.
// With lengths given and fewer (sequence, KV head, head chunk) units than the
// grid, the splits come from a list by visible rows instead (balance.h), so
// that short sequences take fewer work groups and the longest piece shrinks.
//
// The addressing mode (dense linear/ring, global positions, paged) is a
// template parameter; on a paged cache each wave fetches the page ids of
// its next tile with one vector load a tile ahead of the row loads.

#include <limits.h>
#include <stdlib.h>

#include "balance.h"
#include "device_common.h"
#include "internal.h"
#include "visible.h"

namespace attn {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

constexpr int kTT = 32;  // tokens per tile
constexpr int kNW = 4;   // waves per work group

ATTN_DEV uint4 nt_load16(const void* p) {
  const u32x4_t x = __builtin_nontemporal_load((const u32x4_t*)p);
  return make_uint4(x[0], x[1], x[2], x[3]);
}

ATTN_DEV bf16x8_t as_bf16x8(const uint4& u) { return __builtin_bit_cast(bf16x8_t, u); }

typedef __bf16 bf16x2_v __attribute__((ext_vector_type(2)));
typedef float f32x2_v __attribute__((ext_vector_type(2)));

// (a, b) -> packed bf16 high parts (round to nearest even, v_cvt_pk_bf16_f32)
// and packed bf16 remainders a - hi(a), b - hi(b): hi + lo carries about 16
// significant bits of each weight.
ATTN_DEV void split_bf16(float a, float b, uint32_t& hi, uint32_t& lo) {
  hi = __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_v{a, b}, bf16x2_v));
  const float ra = a - __uint_as_float(hi << 16);
  const float rb = b - __uint_as_float(hi & 0xffff0000u);
  lo = __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_v{ra, rb}, bf16x2_v));
}

// Chunk swizzle of the V tile in LDS: 16-byte chunk c of row t is stored at
// chunk c ^ swz(t), so the four rows a transposed read touches fall on
// distinct banks.
template <int D>
ATTN_DEV int vt_swz(int t) {
  if constexpr (D == 64) return 2 * ((t >> 1) & 1);
  else return 2 * (t & 3);
}

// DK: key row width (and row stride of the cache); DV: value width (equal
// for a K/V cache).
template <int DK, int DV, int NH>
struct MfmaCfg {
  static constexpr int KS = DK / 32;  // k-steps of the score product
  static constexpr int HB = NH / 16;  // head blocks
  static constexpr int DB = DV / 16;  // d blocks of the value product
  static constexpr int VT_BYTES = kTT * DV * 2;
  static constexpr int CPR = DV / 8;                      // 16-byte chunks per V row
  static constexpr int RPI = CPR >= 64 ? 1 : 64 / CPR;    // rows per load instruction
  static constexpr int VLD = kTT / RPI;                   // V loads per lane per tile
  // merge rows of DV + 4 floats: the 16 lanes of a group write 16 heads'
  // rows with one 16-byte store each, so an unpadded stride (a multiple of
  // the bank width) would put all of them on the same banks
  static constexpr int ORS = DV + 4;
  static constexpr int MERGE_BYTES = kNW * NH * (ORS + 3) * 4;
  static constexpr int LOOP_BYTES = kNW * VT_BYTES;
  static constexpr int SMEM = MERGE_BYTES > LOOP_BYTES ? MERGE_BYTES : LOOP_BYTES;
  static_assert(DV % 32 == 0 && DV == DK, "value columns");
};

// LIST: 0 fixed splits, 1 work items from the per-sequence list, 2 the even
// split (GqaArgs::balanced); a template parameter so that the fixed-split
// kernels carry none of the lists' setup.
template <int DK, int DV, int NH, int MODE, int LIST>
__global__ __launch_bounds__(kNW * 64) void gqa_decode_mfma(GqaArgs a) {
  using C = MfmaCfg<DK, DV, NH>;
  constexpr int KS = C::KS, HB = C::HB, DB = C::DB, CPR = C::CPR;
  constexpr int RPI = C::RPI, VLD = C::VLD;
  constexpr int D = DK;  // row stride of the cache and of q
  __shared__ __attribute__((aligned(16))) unsigned char smem[C::SMEM];

  const int lane = threadIdx.x & 63;
  // uniform across the wave: tile bases and page ids stay scalar
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int li = lane & 15;   // column inside a 16-wide block
  const int lg = lane >> 4;   // 16-lane group

  int bid = blockIdx.x;
  if (a.xcd_remap) {
    const int per = gridDim.x / kNumXCDs;
    bid = (bid % kNumXCDs) * per + bid / kNumXCDs;
  }
  const int item = bid;

  // The columns of head chunk hc of KV head g of sequence b over the virtual
  // rows [p0, p1) of vr.  Results go to out / lse when `direct`, else to
  // partial rows: row * S + slot (fixed splits, slot = split) or
  // slot * NH + column (the lists).
  auto process = [&](int b, int g, int hc, const VisibleRange& vr, int p0, int p1,
                     bool direct, int slot) {
    const bool ring = MODE == kAddrDense && a.ring_head != nullptr;
    const int c0 = hc * NH;                // first column (head, token) served
    const int nh = min(NH, a.ncol - c0);   // columns actually present

    Pages pg{};
    if constexpr (MODE == kAddrPaged)
      pg = page_view(a.block_table, a.max_pages, b, vr.hi, a.page_shift, a.num_pages,
                     a.H_kv);
    // K/V base: the (sequence, head) slab, or the head's rows in page 0
    const size_t kv_off = MODE == kAddrPaged
                              ? ((size_t)g << a.page_shift) * D
                              : (size_t)(b * a.H_kv + g) * (size_t)a.T_cap * D;
    const uint16_t* __restrict__ Kbg = (const uint16_t*)a.k + kv_off;
    const uint16_t* __restrict__ Vbg = (const uint16_t*)a.v + kv_off;

    // Q^T fragments: head li of block hb, elements 32*ks + 8*lg .. +7
    uint4 qf[HB][KS];
#pragma unroll
    for (int hb = 0; hb < HB; ++hb) {
      const int h = hb * 16 + li;
      const uint16_t* qh = (const uint16_t*)a.q +
                           query_row(b, g, min(c0 + h, a.ncol - 1), a.n, a.L, a.H_q) * D;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
        qf[hb][ks] =
            h < nh ? *(const uint4*)(qh + 32 * ks + 8 * lg) : make_uint4(0, 0, 0, 0);
    }
    auto q_frag = [&](int hb, int ks) -> uint4 { return qf[hb][ks]; };

    f32x4_t o[DB][HB];  // O^T blocks: d rows 16*db + 4*lg + r, head column li
    float m[HB], l[HB];
#pragma unroll
    for (int hb = 0; hb < HB; ++hb) {
      m[hb] = neg_inf();
      l[hb] = 0.f;
#pragma unroll
      for (int db = 0; db < DB; ++db) o[db][hb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    }

    unsigned char* vt = smem + wave * C::VT_BYTES;
    const int span = p1 - p0;
    const int ntiles = span > 0 ? (span + kTT - 1) / kTT : 0;

    // Several tokens: this lane's column of head block hb sees positions
    // tw[hb] .. tl[hb] only (unused when L == 1).
    const bool multi = a.L > 1;
    int tl[HB], tw[HB];
#pragma unroll
    for (int hb = 0; hb < HB; ++hb) {
      tl[hb] = vr.hi - a.L + (c0 + hb * 16 + li) % a.L;
      tw[hb] = a.wtok > 0 ? tl[hb] - a.wtok + 1 : INT_MIN;
    }

    // Cache row (from the K/V base) of row t of the tile at virtual row
    // `base`; rows past the split re-read the tile's first row.
    auto tile_row = [&](int base, int t, const int (&pid)[3]) -> int {
      int vi = base + t;
      vi = vi < p1 ? vi : base;
      if constexpr (MODE == kAddrDense) return slot_of(vr, ring, vr.lo + vi, a.T_cap);
      else if constexpr (MODE == kAddrGlobal)
        return row_slot(vr, false, base >= vr.n_extra, vi, a.T_cap);
      else return paged_row(pg, pid, vr.lo + base, vr.lo + vi);
    };
    // Page ids of tile `it` (paged caches only): one vector load, lane k
    // holding id k; read with readlane when the tile's loads are issued.
    auto fetch_pages = [&](int it) -> int {
      if constexpr (MODE == kAddrPaged)
        return tile_pages_lanes(pg, vr.lo + p0 + it * kTT, lane);
      else return 0;
    };
    auto page_ids = [&](int pv, int (&id)[3]) {
      if constexpr (MODE == kAddrPaged) page_ids_from_lanes(pg, pv, id);
    };

    // K fragments (token 16*tb + li, elements 32*ks + 8*lg..) and this lane's
    // share of the V tile (rows RPI*i + lane/CPR, chunk lane%CPR).
    // A tile index past the split (uniform) reads row 0 of the K/V base
    // instead: in bounds, shared by the work group's waves, never used.
    auto load_tile = [&](int it, int pv, uint4 (&kf)[2][KS],
                         uint4 (&vr_)[VLD > 0 ? VLD : 1]) {
      const int base = p0 + it * kTT;
      const bool dummy = it >= ntiles;
      int pid[3];
      page_ids(pv, pid);
#pragma unroll
      for (int tb = 0; tb < 2; ++tb) {
        const int row = dummy ? 0 : tile_row(base, 16 * tb + li, pid);
        const uint16_t* kp = Kbg + (size_t)row * D + 8 * lg;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) kf[tb][ks] = nt_load16(kp + 32 * ks);
      }
#pragma unroll
      for (int i = 0; i < VLD; ++i) {
        const int t = RPI * i + lane / CPR;
        const int row = dummy ? 0 : tile_row(base, t, pid);
        vr_[i] = nt_load16(Vbg + (size_t)row * D + 8 * (lane % CPR));
      }
      (void)vr_;
    };

    auto compute_tile = [&](int it, const uint4 (&kf)[2][KS],
                            const uint4 (&vr_)[VLD > 0 ? VLD : 1]) {
      const int base = p0 + it * kTT;
      // V tile -> LDS (row t, chunk c stored at chunk c ^ swz(t))
#pragma unroll
      for (int i = 0; i < VLD; ++i) {
        const int t = RPI * i + lane / CPR;
        const int c = lane % CPR;
        *(uint4*)(vt + t * (2 * DV) + 16 * (c ^ vt_swz<DV>(t))) = vr_[i];
      }

      // scores S^T: token rows 16*tb + 4*lg + r, head column li of block hb
      f32x4_t sc[2][HB];
#pragma unroll
      for (int hb = 0; hb < HB; ++hb) {
        f32x4_t acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          const bf16x8_t qv = as_bf16x8(q_frag(hb, ks));
          acc0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(kf[0][ks]), qv, acc0,
                                                          0, 0, 0);
          acc1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(kf[1][ks]), qv, acc1,
                                                          0, 0, 0);
        }
        sc[0][hb] = acc0;
        sc[1][hb] = acc1;
      }

      bool valid[2][4];
#pragma unroll
      for (int tb = 0; tb < 2; ++tb)
#pragma unroll
        for (int r = 0; r < 4; ++r) valid[tb][r] = base + 16 * tb + 4 * lg + r < p1;

      // online softmax per head (lazy maximum, as in the vector kernel)
      uint32_t phi[HB][4], plo[HB][4];  // packed bf16 pairs of P_hi / P_lo
#pragma unroll
      for (int hb = 0; hb < HB; ++hb) {
        float x[8];
#pragma unroll
        for (int tb = 0; tb < 2; ++tb)
#pragma unroll
          for (int r = 0; r < 4; ++r)
            x[4 * tb + r] = valid[tb][r] ? sc[tb][hb][r] * a.scale_log2 : neg_inf();
        if (multi) {  // uniform: each column's causal limit and window
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            const int pos = vr.lo + base + 16 * (j >> 2) + 4 * lg + (j & 3);
            if (pos > tl[hb] || pos < tw[hb]) x[j] = neg_inf();
          }
        }
        float mt = x[0];
#pragma unroll
        for (int j = 1; j < 8; ++j) mt = fmaxf(mt, x[j]);
        mt = fmaxf(mt, xor16(mt));
        mt = fmaxf(mt, xor32(mt));
        if (mt > m[hb] + 8.f) {
          const float al = fast_exp2(m[hb] - mt);
          l[hb] *= al;
#pragma unroll
          for (int db = 0; db < DB; ++db) o[db][hb] *= al;
          m[hb] = mt;
        }
        float p[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          p[j] = (x[j] == neg_inf()) ? 0.f : fast_exp2(x[j] - m[hb]);
          l[hb] += p[j];
        }
#pragma unroll
        for (int j = 0; j < 4; ++j)
          split_bf16(p[2 * j], p[2 * j + 1], phi[hb][j], plo[hb][j]);
      }

      // O^T += V^T . P^T over the 32 tokens of the tile
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        // lane j of group lg addresses row 4*lg + j/4 (+16), columns 16*db + 4*(j%4)
        const int t0 = 4 * lg + (li >> 2);
        const int col = 16 * db + 4 * (li & 3);
        const int c = col >> 3, half = (col & 7) * 2;
        const unsigned char* a0 = vt + t0 * (2 * DV) + 16 * (c ^ vt_swz<DV>(t0)) + half;
        const unsigned char* a1 =
            vt + (t0 + 16) * (2 * DV) + 16 * (c ^ vt_swz<DV>(t0 + 16)) + half;
        typedef s16x4_t __attribute__((address_space(3))) * lds_s16x4;
        const s16x4_t v0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_s16x4)(__attribute__((address_space(3))) unsigned char*)a0);
        const s16x4_t v1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_s16x4)(__attribute__((address_space(3))) unsigned char*)a1);
        const uint4 vtu = make_uint4(
            (uint32_t)(uint16_t)v0[0] | ((uint32_t)(uint16_t)v0[1] << 16),
            (uint32_t)(uint16_t)v0[2] | ((uint32_t)(uint16_t)v0[3] << 16),
            (uint32_t)(uint16_t)v1[0] | ((uint32_t)(uint16_t)v1[1] << 16),
            (uint32_t)(uint16_t)v1[2] | ((uint32_t)(uint16_t)v1[3] << 16));
        const bf16x8_t av = as_bf16x8(vtu);
#pragma unroll
        for (int hb = 0; hb < HB; ++hb) {
          const uint4 bh = make_uint4(phi[hb][0], phi[hb][1], phi[hb][2], phi[hb][3]);
          const uint4 bl = make_uint4(plo[hb][0], plo[hb][1], plo[hb][2], plo[hb][3]);
          o[db][hb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, as_bf16x8(bh),
                                                              o[db][hb], 0, 0, 0);
          o[db][hb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, as_bf16x8(bl),
                                                              o[db][hb], 0, 0, 0);
        }
      }
    };

    // two register stages; page ids run a tile ahead, loaded before the
    // current tile's rows so that waiting for them never waits for row data
    uint4 kA[2][KS], vA[VLD > 0 ? VLD : 1], kB[2][KS], vB[VLD > 0 ? VLD : 1];
    // The loop body is one pair of tiles with both loads unconditional (a
    // load behind a condition, or a break between the halves, makes the
    // compiler's wait for the current tile also cover the next tile's loads);
    // the tile after the wave's last re-reads row 0 of the K/V base instead
    // (never used).  Page ids (pA / pB, alternating like the stages) are loaded
    // a tile ahead of the rows.
    // this wave's tiles
    const int nt = wave < ntiles ? (ntiles - wave + kNW - 1) / kNW : 0;
    int pA = 0, pB = 0;
    if (nt > 0) {
      const int pcur = fetch_pages(wave);
      pA = fetch_pages(wave + kNW);
      load_tile(wave, pcur, kA, vA);
    }
    for (int j = 0; j + 1 < nt; j += 2) {
      const int it = wave + j * kNW;
      pB = fetch_pages(it + 2 * kNW);
      load_tile(it + kNW, pA, kB, vB);
      compute_tile(it, kA, vA);
      pA = fetch_pages(it + 3 * kNW);
      load_tile(it + 2 * kNW, pB, kA, vA);
      compute_tile(it + kNW, kB, vB);
    }
    if (nt & 1) compute_tile(wave + (nt - 1) * kNW, kA, vA);

    // per-head partial sums of the four lane groups
#pragma unroll
    for (int hb = 0; hb < HB; ++hb) {
      l[hb] += xor16(l[hb]);
      l[hb] += xor32(l[hb]);
    }

    __syncthreads();  // the V tiles are dead; reuse LDS for the merge
    constexpr int ORS = C::ORS;
    float* sm_o = (float*)smem;                       // [NW][NH][ORS]
    float* sm_m = sm_o + kNW * NH * ORS;              // [NW][NH]
    float* sm_l = sm_m + kNW * NH;                    // [NW][NH]
    float* sm_w = sm_l + kNW * NH;                    // [NW][NH] weight / L
#pragma unroll
    for (int hb = 0; hb < HB; ++hb) {
      const int h = hb * 16 + li;
#pragma unroll
      for (int db = 0; db < DB; ++db)
        *(f32x4_t*)(sm_o + ((size_t)wave * NH + h) * ORS + 16 * db + 4 * lg) = o[db][hb];
      if (lg == 0) {
        sm_m[wave * NH + h] = m[hb];
        sm_l[wave * NH + h] = l[hb];
      }
    }
    __syncthreads();

    // One lane per column merges the waves' (m, l) by the log-sum-exp rule
    // and leaves each wave's weight divided by the total, so the value pass
    // below is four multiply-adds per element with no exponentials.
    if (threadIdx.x < nh) {
      const int h = threadIdx.x;
      float M = neg_inf();
#pragma unroll
      for (int w = 0; w < kNW; ++w) M = fmaxf(M, sm_m[w * NH + h]);
      float wt[kNW], L = 0.f;
#pragma unroll
      for (int w = 0; w < kNW; ++w) {
        const float mw = sm_m[w * NH + h];
        wt[w] = (M == neg_inf() || mw == neg_inf()) ? 0.f : fast_exp2(mw - M);
        L = fmaf(wt[w], sm_l[w * NH + h], L);
      }
      const bool empty = !(L > 0.f);
      const float inv = empty ? 0.f : 1.f / L;
#pragma unroll
      for (int w = 0; w < kNW; ++w) sm_w[w * NH + h] = wt[w] * inv;
      const float lse = empty ? neg_inf() : (M + fast_log2(L)) * kLn2;
      const size_t row = query_row(b, g, c0 + h, a.n, a.L, a.H_q);
      if (direct) {
        if (a.lse) a.lse[row] = lse;
      } else {
        a.lse_part[LIST == 0 ? row * a.S + slot : (size_t)slot * NH + h] = lse;
      }
    }
    __syncthreads();

    // values: four adjacent columns per lane and step (16-byte LDS reads)
    constexpr int DV4 = DV / 4;
    for (int idx = threadIdx.x; idx < nh * DV4; idx += kNW * 64) {
      const int h = idx / DV4;
      const int e = 4 * (idx - h * DV4);
      f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int w = 0; w < kNW; ++w)
        acc += sm_w[w * NH + h] * *(const f32x4_t*)(sm_o + ((size_t)w * NH + h) * ORS + e);
      const size_t row = query_row(b, g, c0 + h, a.n, a.L, a.H_q);
      const size_t prow = LIST == 0 ? row * a.S + slot : (size_t)slot * NH + h;
      float* dst = direct ? a.out + row * DV + e : a.o_part + prow * DV + e;
#pragma unroll
      for (int i = 0; i < 4; ++i) dst[i] = acc[i];
    }
  };  // process

  if constexpr (LIST == 2) {
    // even split: this group's range of the line, one segment per unit
    const int U = a.H_kv * a.head_chunks;
    const EvenPlan ep = even_plan(a.seq_lens, a.B, a.T_cap, a.window,
                                  MODE == kAddrGlobal ? a.gpos : nullptr,
                                  MODE == kAddrGlobal ? a.n_global : 0, U, a.cap, kTT,
                                  a.even_lead, 2 * kNW);
    if (item >= ep.groups) return;  // uniform over the work group
    const int x1 = even_start(ep, item + 1);
    int x = even_start(ep, item);
    bool first = true;
    while (x < x1) {
      const EvenSeg sg = even_segment(ep, x, x1);
      x = sg.next;
      if (sg.t1 == sg.t0) continue;  // only lead tiles of this unit
      if (!first) __syncthreads();  // the last segment's merge reads are done
      first = false;
      const int ui = sg.b * U + sg.u;
      if (sg.t0 == 0 && threadIdx.x == 0) {  // the group holding the unit's start
        a.meta[2 * ui] = sg.first + ui;
        a.meta[2 * ui + 1] = sg.last - sg.first + 1;
      }
      const VisibleRange vr =
          visible_range_of(sg.len, false, 0, a.T_cap, a.window,
                           MODE == kAddrGlobal ? a.gpos : nullptr,
                           MODE == kAddrGlobal ? a.n_global : 0);
      const int p0 = min(sg.t0 * kTT, vr.n), p1 = min(sg.t1 * kTT, vr.n);
      process(sg.b, sg.u / a.head_chunks, sg.u % a.head_chunks, vr, p0, p1,
              sg.first == sg.last, item + ui);
    }
  } else {
    int hc, s, g, b, n_split = a.S, chunk = a.chunk;
    int len_b = 0, head_b = 0;  // balanced: the item's stored length and ring head
    if constexpr (LIST == 1) {
      // item r of sequence b: ((g * k + s) * head_chunks + hc), so the head
      // chunks of one piece, which read the same rows, are neighbours
      const WorkItem wi = balanced_item(
          a.seq_lens, MODE == kAddrDense ? a.ring_head : nullptr, a.B, a.T_cap,
          a.window, MODE == kAddrGlobal ? a.gpos : nullptr,
          MODE == kAddrGlobal ? a.n_global : 0, a.H_kv * a.head_chunks, a.cap,
          kNW * kTT, 2 * kNW * kTT, item);
      if (!wi.valid) return;  // uniform over the work group
      b = wi.b;
      len_b = wi.len;
      head_b = wi.head;
      n_split = wi.k;
      chunk = wi.chunk;
      int r = wi.r;
      hc = r % a.head_chunks;
      r /= a.head_chunks;
      s = r % wi.k;
      g = r / wi.k;
      if (wi.r == 0 && threadIdx.x == 0) {
        a.meta[2 * b] = wi.first;
        a.meta[2 * b + 1] = wi.k;
      }
    } else {
      hc = bid % a.head_chunks;
      bid /= a.head_chunks;
      s = bid % a.S;
      bid /= a.S;
      g = bid % a.H_kv;
      b = bid / a.H_kv;
    }
  
    const bool ring = MODE == kAddrDense && a.ring_head != nullptr;
    VisibleRange vr =
        LIST == 1 ? visible_range_of(len_b, ring, head_b, a.T_cap, a.window,
                               MODE == kAddrGlobal ? a.gpos : nullptr,
                               MODE == kAddrGlobal ? a.n_global : 0)
        : MODE == kAddrGlobal
            ? visible_range(a.seq_lens, nullptr, b, a.T_cap, a.window, a.gpos, a.n_global)
            : visible_range(a.seq_lens, MODE == kAddrDense ? a.ring_head : nullptr, b,
                            a.T_cap, a.window);
    ring_slot_order(vr, ring, a.L, a.T_cap);
    int p0, p1;  // this split's virtual rows
    split_range(vr, s, n_split, chunk, p0, p1);
    process(b, g, hc, vr, p0, p1, n_split == 1, LIST == 1 ? item : s);
  }
}

template <int DK, int DV, int NH, int MODE>
hipError_t launch_one(const GqaArgs& a, int grid, hipStream_t st) {
  if (a.balanced == 2) {
    // the even split runs at d <= 128 only (the planner's choice)
    if constexpr (DK > 128) return hipErrorInvalidValue;
    else
      hipLaunchKernelGGL((gqa_decode_mfma<DK, DV, NH, MODE, 2>), dim3(grid),
                         dim3(kNW * 64), 0, st, a);
  } else if (a.balanced)
    hipLaunchKernelGGL((gqa_decode_mfma<DK, DV, NH, MODE, 1>), dim3(grid),
                       dim3(kNW * 64), 0, st, a);
  else
    hipLaunchKernelGGL((gqa_decode_mfma<DK, DV, NH, MODE, 0>), dim3(grid),
                       dim3(kNW * 64), 0, st, a);
  return hipGetLastError();
}

template <int MODE>
hipError_t launch_mode(const GqaArgs& a, int dk, int dv, int heads_per_item, int grid,
                       hipStream_t st) {
  switch (dk * 1000000 + dv * 1000 + heads_per_item) {
    case 64064016: return launch_one<64, 64, 16, MODE>(a, grid, st);
    case 64064032: return launch_one<64, 64, 32, MODE>(a, grid, st);
    case 128128016: return launch_one<128, 128, 16, MODE>(a, grid, st);
    case 128128032: return launch_one<128, 128, 32, MODE>(a, grid, st);
    case 256256016: return launch_one<256, 256, 16, MODE>(a, grid, st);
  }
  return hipErrorInvalidValue;
}

}  // namespace

// Columns per work item on the matrix-core path (16 or 32; 16 at d = 256),
// or 0 if the path does not apply (float32 data, or groups small enough for
// the vector kernel).
int mfma_heads_per_item(int dtype, int d, int n) {
  // smallest group sent to the matrix cores (overridable for tuning sweeps
  // through ATTN_DECODE_MFMA_MIN_GROUP)
  static const int min_group = [] {
    const char* e = getenv("ATTN_DECODE_MFMA_MIN_GROUP");
    const int x = e ? atoi(e) : 0;
    return x > 0 ? x : 3;
  }();
  if (dtype != 1 || n < min_group) return 0;
  if (d == 256) return 16;  // 32 columns would not fit the registers
  if (d != 64 && d != 128) return 0;
  const int r = (n + 15) / 16 * 16;
  return r < 32 ? r : 32;
}

int mfma_tile_rows() { return kTT; }
int mfma_waves() { return kNW; }

hipError_t launch_gqa_mfma(const GqaArgs& a, int d, int heads_per_item, int grid,
                           hipStream_t st) {
  if (a.block_table) return launch_mode<kAddrPaged>(a, d, d, heads_per_item, grid, st);
  if (a.n_global > 0) return launch_mode<kAddrGlobal>(a, d, d, heads_per_item, grid, st);
  return launch_mode<kAddrDense>(a, d, d, heads_per_item, grid, st);
}

}  // namespace attn
