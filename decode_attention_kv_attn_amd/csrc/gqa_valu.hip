// Split-T decode attention on the vector ALUs (MHA / GQA, groups of <= 8).
//
// One work group owns (sequence b, KV head g, up to N query heads of g's
// group, split s of the visible range).  Its waves take the split's tiles in
// turn.  Each tile is TR consecutive visible positions; a wave reads the K
// and V rows of a tile once with 16-byte loads and serves all N query heads
// from them (the group's heads share one K/V head: xuesongtap
// "attention-head" note, section 2.2).
//
// Lane layout inside a wave: LPR lanes cover one cache row, each owning E
// elements (CPL 16-byte chunks; chunk c + k*LPR for k < CPL), so one load
// instruction covers RPI = 64/LPR whole rows -- LPR*16 contiguous bytes per
// row.  Dot products are finished with DPP sums inside the LPR-lane group.
// Every row group (the LPR lanes of one row) keeps its own running softmax
// state (max m in the log2 domain, sum l, value sums acc), so the main loop
// needs no wave-wide communication; the states are merged by the
// log-sum-exp rule at the end, first across row groups (DPP / swizzle), then
// across waves through LDS.
//
// Online softmax with a lazy maximum: a state keeps its reference max until a
// tile raises the max by more than 8 (log2 units), so weights stay <= 2^8 and
// the rescale of acc is rare.  The result is the same softmax: every weight
// and the normaliser use the same reference.
//
// Rows of a tile past the end of the split are not loaded from their own
// address: they re-read the tile's first row (always visible) and get weight
// 0, so no masked cache row is ever read (attention-head section 3).
//
// The addressing mode (dense linear/ring, global positions, paged) is a
// template parameter; this file is compiled once per mode (ATTN_VALU_MODE),
// so each translation unit holds one mode's instantiations.  On a paged
// cache the page ids of a wave's next tile are fetched with one vector load
// a tile ahead, so the row addresses never wait on the block table.

#include <limits.h>

#include "balance.h"
#include "device_common.h"
#include "internal.h"
#include "visible.h"

// Tuning knobs (compile-time; defaults are the measured best).
#ifndef ATTN_VALU_TILE_BYTES
#define ATTN_VALU_TILE_BYTES 8192
#endif
#ifndef ATTN_VALU_TILE_BYTES_WIDE  // per-wave tile bytes when N >= 7
#define ATTN_VALU_TILE_BYTES_WIDE 4096
#endif
#ifndef ATTN_VALU_E_SMALL  // elements per lane per row when N <= 4
#define ATTN_VALU_E_SMALL 16
#endif
#ifndef ATTN_VALU_WAVES  // waves per work group (upper bound)
#define ATTN_VALU_WAVES 4
#endif
#ifndef ATTN_VALU_NONTEMPORAL  // K/V are read once: stream past the caches
#define ATTN_VALU_NONTEMPORAL 1
#endif
#ifndef ATTN_VALU_MODE  // addressing mode of this translation unit
#define ATTN_VALU_MODE 0
#endif

namespace attn {
namespace {

template <typename T>
struct ElemTraits;

template <>
struct ElemTraits<float> {
  static constexpr int EPC = 4;  // elements per 16-byte chunk
  static ATTN_DEV float dot(const uint4& q, const uint4& k, float acc) {
    acc = fmaf(__uint_as_float(q.x), __uint_as_float(k.x), acc);
    acc = fmaf(__uint_as_float(q.y), __uint_as_float(k.y), acc);
    acc = fmaf(__uint_as_float(q.z), __uint_as_float(k.z), acc);
    acc = fmaf(__uint_as_float(q.w), __uint_as_float(k.w), acc);
    return acc;
  }
  static ATTN_DEV void unpack(const uint4& c, float (&f)[4]) {
    f[0] = __uint_as_float(c.x);
    f[1] = __uint_as_float(c.y);
    f[2] = __uint_as_float(c.z);
    f[3] = __uint_as_float(c.w);
  }
};

// bf16 stored as raw 16-bit patterns, two per dword (element 2j in the low
// half of dword j).
template <>
struct ElemTraits<uint16_t> {
  static constexpr int EPC = 8;
  static ATTN_DEV float dot(const uint4& q, const uint4& k, float acc) {
    acc = dot2_bf16(q.x, k.x, acc);
    acc = dot2_bf16(q.y, k.y, acc);
    acc = dot2_bf16(q.z, k.z, acc);
    acc = dot2_bf16(q.w, k.w, acc);
    return acc;
  }
  static ATTN_DEV void unpack(const uint4& c, float (&f)[8]) {
    f[0] = bf16_lo(c.x);
    f[1] = bf16_hi(c.x);
    f[2] = bf16_lo(c.y);
    f[3] = bf16_hi(c.y);
    f[4] = bf16_lo(c.z);
    f[5] = bf16_hi(c.z);
    f[6] = bf16_lo(c.w);
    f[7] = bf16_hi(c.w);
  }
};

// 16-byte global load of K/V data that is streamed once.
template <typename T>
ATTN_DEV uint4 load16(const T* p) {
#if ATTN_VALU_NONTEMPORAL
  typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
  const u32x4 x = __builtin_nontemporal_load((const u32x4*)p);
  return make_uint4(x[0], x[1], x[2], x[3]);
#else
  return *(const uint4*)p;
#endif
}

// Geometry of one instantiation.
template <typename T, int D, int N>
struct Cfg {
  static constexpr int EPC = ElemTraits<T>::EPC;
  static constexpr int E = (N <= 4) ? ATTN_VALU_E_SMALL : 8;  // per lane per row
  static constexpr int CPL = E / EPC;          // chunks per lane per row
  static constexpr int LPR = D / E;            // lanes per row
  static constexpr int RPI = 64 / LPR;         // rows per load instruction
  static constexpr int TR_BYTES =  // K+V per wave per tile
      N >= 7 ? ATTN_VALU_TILE_BYTES_WIDE : ATTN_VALU_TILE_BYTES;
  static constexpr int TR0 = TR_BYTES / (2 * D * (int)sizeof(T));
  static constexpr int TR = TR0 > RPI ? TR0 : RPI;  // rows per tile
  static constexpr int RPL = TR / RPI;              // rows per lane per tile
  static constexpr int NW0 = 15360 / (N * D);       // LDS cap for the merge
  static constexpr int NWL = NW0 >= 16 ? 16 : (NW0 >= 8 ? 8 : (NW0 >= 4 ? 4 : 2));
  static constexpr int NW = NWL < ATTN_VALU_WAVES ? NWL : ATTN_VALU_WAVES;
  static_assert(E % EPC == 0 && D % E == 0, "lane split");
  static_assert(LPR >= 1 && LPR <= 64 && 64 % LPR == 0, "lanes per row");
  static_assert(TR % RPI == 0, "tile rows");
  static_assert(TR <= 33, "a tile must fit in three pages of >= 16 rows");
};

// Fold the state held RPI_STEP row groups away into this lane's state.
template <int CTRL, int N, int E>
ATTN_DEV void merge_dpp(float (&m)[N], float (&l)[N], float (&acc)[N][E]) {
#pragma unroll
  for (int h = 0; h < N; ++h) {
    float a1, a2;
    lse_merge_scalars(m[h], l[h], dpp<CTRL>(m[h]), dpp<CTRL>(l[h]), a1, a2);
#pragma unroll
    for (int e = 0; e < E; ++e) acc[h][e] = a1 * acc[h][e] + a2 * dpp<CTRL>(acc[h][e]);
  }
}

template <int N, int E, typename F>
ATTN_DEV void merge_fn(float (&m)[N], float (&l)[N], float (&acc)[N][E], F mv) {
#pragma unroll
  for (int h = 0; h < N; ++h) {
    float a1, a2;
    lse_merge_scalars(m[h], l[h], mv(m[h]), mv(l[h]), a1, a2);
#pragma unroll
    for (int e = 0; e < E; ++e) acc[h][e] = a1 * acc[h][e] + a2 * mv(acc[h][e]);
  }
}

// BAL: work items from the balanced list (GqaArgs::balanced, balance.h); a
// template parameter so that the fixed-split kernels carry none of it.
template <typename T, int D, int N, int MODE, bool BAL>
__global__ __launch_bounds__((Cfg<T, D, N>::NW * 64)) void gqa_decode_valu(
    GqaArgs a) {
  using C = Cfg<T, D, N>;
  using ET = ElemTraits<T>;
  constexpr int EPC = C::EPC, E = C::E, CPL = C::CPL, LPR = C::LPR;
  constexpr int RPI = C::RPI, TR = C::TR, RPL = C::RPL, NW = C::NW;

  __shared__ float sm_acc[NW][N][D];
  __shared__ float sm_m[NW][N];
  __shared__ float sm_l[NW][N];
  __shared__ float sm_w[NW][N];  // each wave's merge weight divided by the total

  const int lane = threadIdx.x & 63;
  // uniform across the wave: tile bases and page ids stay scalar
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int rg = lane / LPR;  // row group
  const int cl = lane % LPR;  // lane inside the row

  // ---- work item: hc fastest, then split, KV head, sequence ---------------
  int bid = blockIdx.x;
  if (a.xcd_remap) {
    const int per = gridDim.x / kNumXCDs;
    bid = (bid % kNumXCDs) * per + bid / kNumXCDs;
  }
  const int item = bid;
  int hc, s, g, b, n_split = a.S, chunk = a.chunk;
  int len_b = 0;  // balanced: the item's stored length
  if constexpr (BAL) {
    // item r of sequence b: ((g * k + s) * head_chunks + hc)
    const WorkItem wi = balanced_item(
        a.seq_lens, nullptr, a.B, a.T_cap, a.window, MODE == kAddrGlobal ? a.gpos : nullptr,
        MODE == kAddrGlobal ? a.n_global : 0, a.H_kv * a.head_chunks, a.cap, NW * TR,
        2 * NW * TR, item);
    if (!wi.valid) return;  // uniform over the work group
    b = wi.b;
    len_b = wi.len;
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

  VisibleRange vr =
      BAL ? visible_range_of(len_b, false, 0, a.T_cap, a.window,
                             MODE == kAddrGlobal ? a.gpos : nullptr,
                             MODE == kAddrGlobal ? a.n_global : 0)
      : MODE == kAddrGlobal
          ? visible_range(a.seq_lens, nullptr, b, a.T_cap, a.window, a.gpos, a.n_global)
          : visible_range(a.seq_lens, MODE == kAddrDense ? a.ring_head : nullptr, b,
                          a.T_cap, a.window);
  const bool ring = MODE == kAddrDense && a.ring_head != nullptr;
  ring_slot_order(vr, ring, a.L, a.T_cap);
  int p0, p1;  // this split's virtual rows
  split_range(vr, s, n_split, chunk, p0, p1);
  const int c0 = hc * N;                   // first column (head, token) served
  const int nh = min(N, a.ncol - c0);      // columns actually present

  Pages pg{};
  if constexpr (MODE == kAddrPaged)
    pg = page_view(a.block_table, a.max_pages, b, vr.hi, a.page_shift, a.num_pages,
                   a.H_kv);
  // K/V base of this (sequence, KV head): a [T_cap, D] slab, or the head's
  // rows inside page 0 of the pool
  const size_t kv_off = MODE == kAddrPaged
                            ? ((size_t)g << a.page_shift) * D
                            : (size_t)(b * a.H_kv + g) * (size_t)a.T_cap * D;
  const T* __restrict__ Kbg = (const T*)a.k + kv_off;
  const T* __restrict__ Vbg = (const T*)a.v + kv_off;

  // ---- query chunks for this lane's elements ------------------------------
  uint4 qr[N][CPL];
  {
#pragma unroll
    for (int h = 0; h < N; ++h) {
      const T* qh = (const T*)a.q +
                    query_row(b, g, min(c0 + h, a.ncol - 1), a.n, a.L, a.H_q) * D;
#pragma unroll
      for (int k = 0; k < CPL; ++k)
        qr[h][k] = (h < nh) ? *(const uint4*)(qh + (cl + k * LPR) * EPC)
                            : make_uint4(0, 0, 0, 0);
    }
  }

  float m[N], l[N], acc[N][E];
#pragma unroll
  for (int h = 0; h < N; ++h) {
    m[h] = neg_inf();
    l[h] = 0.f;
#pragma unroll
    for (int e = 0; e < E; ++e) acc[h][e] = 0.f;
  }

  const int span = p1 - p0;
  const int ntiles = span > 0 ? (span + TR - 1) / TR : 0;

  // Several tokens: column h sees positions tl[h] - wtok + 1 .. tl[h] only
  // (uniform per column; unused when L == 1).
  const bool multi = a.L > 1;
  int tl[N], tw[N];
#pragma unroll
  for (int h = 0; h < N; ++h) {
    tl[h] = vr.hi - a.L + (c0 + h) % a.L;
    tw[h] = a.wtok > 0 ? tl[h] - a.wtok + 1 : INT_MIN;
  }

  // Cache row (from the K/V base) of virtual row vi of the tile at `base`;
  // `pid` holds that tile's page ids on a paged cache.
  auto row_of = [&](int base, int vi, const int (&pid)[3]) -> int {
    if constexpr (MODE == kAddrDense) return slot_of(vr, ring, vr.lo + vi, a.T_cap);
    else if constexpr (MODE == kAddrGlobal)
      return row_slot(vr, false, base >= vr.n_extra, vi, a.T_cap);
    else return paged_row(pg, pid, vr.lo + base, vr.lo + vi);
  };
  // Page ids of tile `it` (paged caches only): one vector load, lane k
  // holding id k; read with readlane when the tile's loads are issued.
  auto fetch_pages = [&](int it) -> int {
    if constexpr (MODE == kAddrPaged) return tile_pages_lanes(pg, vr.lo + p0 + it * TR, lane);
    else return 0;
  };
  auto page_ids = [&](int pv, int (&id)[3]) {
    if constexpr (MODE == kAddrPaged) page_ids_from_lanes(pg, pv, id);
  };

  // Issue the 16-byte K and V loads of tile `it` (rows past the split's end
  // re-read the tile's first row; they get weight 0 below).
  // A tile index past the split (uniform) reads row 0 of the K/V base
  // instead: in bounds, shared by the work group's waves, never used.
  auto load_tile = [&](int it, int pv, uint4 (&kr)[RPL][CPL],
                       uint4 (&vv)[RPL][CPL]) {
    const int base = p0 + it * TR;
    const bool dummy = it >= ntiles;
    int pid[3];
    page_ids(pv, pid);
#pragma unroll
    for (int i = 0; i < RPL; ++i) {
      const int vi = base + rg + i * RPI;
      const int slot = dummy ? 0 : row_of(base, vi < p1 ? vi : base, pid);
      const T* kp = Kbg + (size_t)slot * D + cl * EPC;
#pragma unroll
      for (int k = 0; k < CPL; ++k) kr[i][k] = load16(kp + k * LPR * EPC);
    }
#pragma unroll
    for (int i = 0; i < RPL; ++i) {
      const int vi = base + rg + i * RPI;
      const int slot = dummy ? 0 : row_of(base, vi < p1 ? vi : base, pid);
      const T* vp = Vbg + (size_t)slot * D + cl * EPC;
#pragma unroll
      for (int k = 0; k < CPL; ++k) vv[i][k] = load16(vp + k * LPR * EPC);
    }
  };

  // Scores, online softmax and value sums of tile `it`.
  auto compute_tile = [&](int it, const uint4 (&kr)[RPL][CPL],
                          const uint4 (&vv)[RPL][CPL]) {
    const int base = p0 + it * TR;
    bool valid[RPL];
#pragma unroll
    for (int i = 0; i < RPL; ++i) valid[i] = base + rg + i * RPI < p1;

    // scores (log2 domain)
    float sc[RPL][N];
#pragma unroll
    for (int i = 0; i < RPL; ++i)
#pragma unroll
      for (int h = 0; h < N; ++h) {
        float x = 0.f;
#pragma unroll
        for (int k = 0; k < CPL; ++k) x = ET::dot(qr[h][k], kr[i][k], x);
        sc[i][h] = x;
      }
#pragma unroll
    for (int i = 0; i < RPL; ++i)
#pragma unroll
      for (int h = 0; h < N; ++h) {
        const float x = group_sum<LPR>(sc[i][h]) * a.scale_log2;
        sc[i][h] = valid[i] ? x : neg_inf();
      }
    if (multi) {  // uniform: causal limit and window of each token's column
#pragma unroll
      for (int i = 0; i < RPL; ++i) {
        const int pos = vr.lo + base + rg + i * RPI;
#pragma unroll
        for (int h = 0; h < N; ++h)
          if (pos > tl[h] || pos < tw[h]) sc[i][h] = neg_inf();
      }
    }

    // lazy maximum
#pragma unroll
    for (int h = 0; h < N; ++h) {
      float mt = sc[0][h];
#pragma unroll
      for (int i = 1; i < RPL; ++i) mt = fmaxf(mt, sc[i][h]);
      if (mt > m[h] + 8.f) {
        const float al = fast_exp2(m[h] - mt);
        l[h] *= al;
#pragma unroll
        for (int e = 0; e < E; ++e) acc[h][e] *= al;
        m[h] = mt;
      }
    }

    // weights and value sums
#pragma unroll
    for (int i = 0; i < RPL; ++i) {
      float vf[CPL][EPC];
#pragma unroll
      for (int k = 0; k < CPL; ++k) ET::unpack(vv[i][k], vf[k]);
#pragma unroll
      for (int h = 0; h < N; ++h) {
        // masked entries (-inf) weigh 0, also while m is still -inf
        const float p = sc[i][h] == neg_inf() ? 0.f : fast_exp2(sc[i][h] - m[h]);
        l[h] += p;
#pragma unroll
        for (int k = 0; k < CPL; ++k)
#pragma unroll
          for (int e = 0; e < EPC; ++e)
            acc[h][k * EPC + e] = fmaf(p, vf[k][e], acc[h][k * EPC + e]);
      }
    }
  };

  // Two register stages: the loads of a wave's next tile are in flight
  // while it computes on the current one.  The loop body is one pair of
  // tiles with both loads unconditional (a load behind a condition, or a
  // break between the halves, makes the compiler's wait for the current
  // tile also cover the next tile's loads); the tile after the wave's last
  // re-reads row 0 of the K/V base instead (never used).  Page ids (pA /
  // pB, alternating like the stages) run a tile ahead of the rows.
  uint4 kA[RPL][CPL], vA[RPL][CPL], kB[RPL][CPL], vB[RPL][CPL];
  const int nt = wave < ntiles ? (ntiles - wave + NW - 1) / NW : 0;  // this wave's tiles
  int pA = 0, pB = 0;
  if (nt > 0) {
    const int pcur = fetch_pages(wave);
    pA = fetch_pages(wave + NW);
    load_tile(wave, pcur, kA, vA);
  }
  for (int j = 0; j + 1 < nt; j += 2) {
    const int it = wave + j * NW;
    pB = fetch_pages(it + 2 * NW);
    load_tile(it + NW, pA, kB, vB);
    compute_tile(it, kA, vA);
    pA = fetch_pages(it + 3 * NW);
    load_tile(it + 2 * NW, pB, kA, vA);
    compute_tile(it + NW, kB, vB);
  }
  if (nt & 1) compute_tile(wave + (nt - 1) * NW, kA, vA);

  // ---- merge the row groups of this wave ----------------------------------
  // Partners are RPI_k = LPR * 2^k lanes away; rotations inside a 16-lane row
  // reach every row group of the row, swizzles cross rows.
  if constexpr (LPR <= 1) merge_dpp<0x121, N, E>(m, l, acc);
  if constexpr (LPR <= 2) merge_dpp<0x122, N, E>(m, l, acc);
  if constexpr (LPR <= 4) merge_dpp<kDppRowRor4, N, E>(m, l, acc);
  if constexpr (LPR <= 8) merge_dpp<kDppRowRor8, N, E>(m, l, acc);
  if constexpr (LPR <= 16) merge_fn<N, E>(m, l, acc, [](float x) { return xor16(x); });
  if constexpr (LPR <= 32) merge_fn<N, E>(m, l, acc, [](float x) { return xor32(x); });

  if (rg == 0) {
#pragma unroll
    for (int h = 0; h < N; ++h)
#pragma unroll
      for (int k = 0; k < CPL; ++k)
#pragma unroll
        for (int e = 0; e < EPC; ++e)
          sm_acc[wave][h][(cl + k * LPR) * EPC + e] = acc[h][k * EPC + e];
    if (cl == 0) {
#pragma unroll
      for (int h = 0; h < N; ++h) {
        sm_m[wave][h] = m[h];
        sm_l[wave][h] = l[h];
      }
    }
  }
  __syncthreads();

  // ---- merge the waves and write ------------------------------------------
  // One lane per head merges the waves' (m, l) by the log-sum-exp rule and
  // leaves each wave's weight divided by the total; the value pass is then
  // NW multiply-adds per element with no exponentials.
  if (threadIdx.x < nh) {
    const int h = threadIdx.x;
    float M = neg_inf();
#pragma unroll
    for (int w = 0; w < NW; ++w) M = fmaxf(M, sm_m[w][h]);
    float wt[NW], L = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      const float mw = sm_m[w][h];
      wt[w] = (M == neg_inf() || mw == neg_inf()) ? 0.f : fast_exp2(mw - M);
      L = fmaf(wt[w], sm_l[w][h], L);
    }
    const bool empty = !(L > 0.f);
    const float inv = empty ? 0.f : 1.f / L;
#pragma unroll
    for (int w = 0; w < NW; ++w) sm_w[w][h] = wt[w] * inv;
    const float lse = empty ? neg_inf() : (M + fast_log2(L)) * kLn2;
    const size_t row = query_row(b, g, c0 + h, a.n, a.L, a.H_q);
    if (n_split == 1) {
      if (a.lse) a.lse[row] = lse;
    } else {
      a.lse_part[BAL ? (size_t)item * N + h : row * a.S + s] = lse;
    }
  }
  __syncthreads();
  for (int idx = threadIdx.x; idx < nh * D; idx += NW * 64) {
    const int h = idx / D;
    const int e = idx - h * D;
    float o = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w) o = fmaf(sm_w[w][h], sm_acc[w][h][e], o);
    const size_t row = query_row(b, g, c0 + h, a.n, a.L, a.H_q);
    if (n_split == 1) a.out[row * D + e] = o;
    else a.o_part[(BAL ? (size_t)item * N + h : row * a.S + s) * D + e] = o;
  }
}

template <typename T, int D, int N>
hipError_t launch_one(const GqaArgs& a, int grid, hipStream_t st) {
  if (a.balanced) {
    hipLaunchKernelGGL((gqa_decode_valu<T, D, N, ATTN_VALU_MODE, true>), dim3(grid),
                       dim3(Cfg<T, D, N>::NW * 64), 0, st, a);
    return hipGetLastError();
  }
  hipLaunchKernelGGL((gqa_decode_valu<T, D, N, ATTN_VALU_MODE, false>), dim3(grid),
                     dim3(Cfg<T, D, N>::NW * 64), 0, st, a);
  return hipGetLastError();
}

template <typename T, int D>
hipError_t launch_d(const GqaArgs& a, int N, int grid, hipStream_t st) {
  switch (N) {
    case 1: return launch_one<T, D, 1>(a, grid, st);
    case 2: return launch_one<T, D, 2>(a, grid, st);
    case 3: return launch_one<T, D, 3>(a, grid, st);
    case 4: return launch_one<T, D, 4>(a, grid, st);
    case 5: return launch_one<T, D, 5>(a, grid, st);
    case 6: return launch_one<T, D, 6>(a, grid, st);
    case 7: return launch_one<T, D, 7>(a, grid, st);
    case 8: return launch_one<T, D, 8>(a, grid, st);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_mode(const GqaArgs& a, int dtype, int d, int grid, hipStream_t st) {
  const int N = a.ncol <= 8 ? a.ncol : 8;
  if (dtype == 0) {
    if (d == 64) return launch_d<float, 64>(a, N, grid, st);
    if (d == 128) return launch_d<float, 128>(a, N, grid, st);
    if (d == 256) return launch_d<float, 256>(a, N, grid, st);
  } else if (dtype == 1) {
    if (d == 64) return launch_d<uint16_t, 64>(a, N, grid, st);
    if (d == 128) return launch_d<uint16_t, 128>(a, N, grid, st);
    if (d == 256) return launch_d<uint16_t, 256>(a, N, grid, st);
  }
  return hipErrorInvalidValue;
}

#if ATTN_VALU_MODE == 0
template <typename T, int D, int N>
void geometry_one(ValuGeometry* g) {
  g->heads_per_item = N;
  g->tile_rows = Cfg<T, D, N>::TR;
  g->waves = Cfg<T, D, N>::NW;
}

template <typename T, int D>
void geometry_d(int N, ValuGeometry* g) {
  switch (N) {
    case 1: geometry_one<T, D, 1>(g); break;
    case 2: geometry_one<T, D, 2>(g); break;
    case 3: geometry_one<T, D, 3>(g); break;
    case 4: geometry_one<T, D, 4>(g); break;
    case 5: geometry_one<T, D, 5>(g); break;
    case 6: geometry_one<T, D, 6>(g); break;
    case 7: geometry_one<T, D, 7>(g); break;
    default: geometry_one<T, D, 8>(g); break;
  }
}
#endif

}  // namespace

#if ATTN_VALU_MODE == 0
// Heads per work item: the whole group when it has <= 8 heads, else chunks
// of 8 (each chunk re-reads the group's K/V rows).
bool valu_geometry(int dtype, int d, int n, ValuGeometry* g) {
  const int N = n <= 8 ? n : 8;
  if (N < 1) return false;
  if (dtype == 0) {
    if (d == 64) geometry_d<float, 64>(N, g);
    else if (d == 128) geometry_d<float, 128>(N, g);
    else if (d == 256) geometry_d<float, 256>(N, g);
    else return false;
  } else if (dtype == 1) {
    if (d == 64) geometry_d<uint16_t, 64>(N, g);
    else if (d == 128) geometry_d<uint16_t, 128>(N, g);
    else if (d == 256) geometry_d<uint16_t, 256>(N, g);
    else return false;
  } else {
    return false;
  }
  return true;
}

hipError_t launch_gqa_valu(const GqaArgs& a, int dtype, int d, int grid,
                           hipStream_t st) {
  if (a.block_table) return launch_gqa_valu_paged(a, dtype, d, grid, st);
  if (a.n_global > 0) return launch_gqa_valu_global(a, dtype, d, grid, st);
  return launch_gqa_valu_dense(a, dtype, d, grid, st);
}

hipError_t launch_gqa_valu_dense(const GqaArgs& a, int dtype, int d, int grid,
                                 hipStream_t st) {
  return launch_mode(a, dtype, d, grid, st);
}
#elif ATTN_VALU_MODE == 1
hipError_t launch_gqa_valu_global(const GqaArgs& a, int dtype, int d, int grid,
                                  hipStream_t st) {
  return launch_mode(a, dtype, d, grid, st);
}
#elif ATTN_VALU_MODE == 2
hipError_t launch_gqa_valu_paged(const GqaArgs& a, int dtype, int d, int grid,
                                 hipStream_t st) {
  return launch_mode(a, dtype, d, grid, st);
}
#else
#error "ATTN_VALU_MODE must be 0 (dense), 1 (global positions) or 2 (paged)"
#endif

}  // namespace attn
