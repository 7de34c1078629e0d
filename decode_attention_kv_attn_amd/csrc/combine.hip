// Log-sum-exp merge of split results (kernel 2).
//
// For each (b, h): L = max_s lse_s, w_s = exp(lse_s - L),
//   out = sum_s w_s o_s / sum_s w_s,  lse = L + ln(sum_s w_s).
// Softmax over a union of disjoint key sets factors this way because each
// part's normaliser is exp(lse_s) (attention equation, xuesongtap
// "attention-head" note, section 1).  Parts with lse = -inf are empty and get
// weight 0; if every part is empty the output is 0 and lse is -inf.
//
// Partial values are float32, or fp16 where the producing kernel says so (the
// fp16 MLA geometry, whose values already lie in fp16's range); weights,
// sums and outputs are float32.
//
// Value widths that are a multiple of 64 up to 512 (every width the decode
// kernels produce): one wave per (b, h) -- two or four when rows are few and
// parts many -- each lane owning d_v / 64 adjacent columns, read as vectors;
// eight parts are in flight per wave, the first eight together with the
// log-sum-exps, and the weights come from the same wave, so a row of up to
// eight parts costs one memory round trip.  Other widths: one work group of
// 256 lanes per (b, h): lanes cover the columns (up to 256 at a time) and,
// when the value is narrower than 256, the remaining lanes split the parts
// between them and meet in LDS.

#include "device_common.h"
#include "internal.h"

namespace attn {
namespace {

constexpr int kMaxS = 1024;
constexpr int kThreads = 256;

// Empty parts (weight 0) contribute nothing, whatever their o_part holds.
ATTN_DEV float add_part(float acc, float w, float x) {
  return w > 0.f ? fmaf(w, x, acc) : acc;
}

// cl = lanes across columns (a multiple of 64 dividing 256); 256/cl lane
// groups split the parts.
__global__ __launch_bounds__(kThreads) void lse_combine(
    const float* __restrict__ o_part, const float* __restrict__ lse_part,
    float* __restrict__ out, float* __restrict__ lse_out, int S, int d_v, int cl) {
  __shared__ float wts[kMaxS];
  __shared__ float red[kThreads];
  __shared__ float tot_s;
  const size_t row = blockIdx.x;
  const float* lp = lse_part + row * S;
  const int tid = threadIdx.x;
  const int lane = tid & 63;

  if (tid < 64) {  // weights of the parts (natural-log input, log2 inside)
    float M = neg_inf();
    for (int s = lane; s < S; s += 64) M = fmaxf(M, lp[s] * kLog2e);
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) M = fmaxf(M, __shfl_xor(M, off));
    float tot = 0.f;
    for (int s = lane; s < S; s += 64) {
      const float x = lp[s];
      const float w = (x == neg_inf() || M == neg_inf()) ? 0.f : fast_exp2(x * kLog2e - M);
      wts[s] = w;
      tot += w;
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) tot += __shfl_xor(tot, off);
    if (lane == 0) {
      tot_s = tot;
      if (lse_out) lse_out[row] = (tot > 0.f) ? (M + fast_log2(tot)) * kLn2 : neg_inf();
    }
  }
  __syncthreads();
  const float tot = tot_s;
  const float inv = (tot > 0.f) ? 1.f / tot : 0.f;
  const int col = tid % cl;
  const int pg = tid / cl;
  const int npg = kThreads / cl;
  const float* op = o_part + row * (size_t)S * d_v;
  for (int e0 = 0; e0 < d_v; e0 += cl) {
    const int e = e0 + col;
    float acc = 0.f;
    if (e < d_v) {
      int s = pg;
      for (; s + 3 * npg < S; s += 4 * npg) {
        const float x0 = op[(size_t)s * d_v + e];
        const float x1 = op[(size_t)(s + npg) * d_v + e];
        const float x2 = op[(size_t)(s + 2 * npg) * d_v + e];
        const float x3 = op[(size_t)(s + 3 * npg) * d_v + e];
        acc = add_part(acc, wts[s], x0);
        acc = add_part(acc, wts[s + npg], x1);
        acc = add_part(acc, wts[s + 2 * npg], x2);
        acc = add_part(acc, wts[s + 3 * npg], x3);
      }
      for (; s < S; s += npg) acc = add_part(acc, wts[s], op[(size_t)s * d_v + e]);
    }
    if (npg == 1) {
      if (e < d_v) out[row * d_v + e] = acc * inv;
    } else {
      red[tid] = acc;
      __syncthreads();
      if (pg == 0 && e < d_v) {
        float sum = acc;
        for (int g = 1; g < npg; ++g) sum += red[g * cl + col];
        out[row * d_v + e] = sum * inv;
      }
      __syncthreads();
    }
  }
}

typedef _Float16 half2_v __attribute__((ext_vector_type(2)));
typedef _Float16 half4_v __attribute__((ext_vector_type(4)));

// N elements of P loaded as one vector
template <typename P, int N>
struct VecOf;
template <> struct VecOf<float, 1> { typedef float type; };
template <> struct VecOf<float, 2> { typedef float2 type; };
template <> struct VecOf<float, 4> { typedef float4 type; };
template <> struct VecOf<_Float16, 1> { typedef _Float16 type; };
template <> struct VecOf<_Float16, 2> { typedef half2_v type; };
template <> struct VecOf<_Float16, 4> { typedef half4_v type; };

template <typename P, int N>
ATTN_DEV void fma_vec(float (&acc)[N], float w, const typename VecOf<P, N>::type& x) {
  const P* xs = reinterpret_cast<const P*>(&x);
#pragma unroll
  for (int i = 0; i < N; ++i) acc[i] = add_part(acc[i], w, (float)xs[i]);
}

// Balanced work lists: output row (b * L + token) * H_q + head belongs to
// column c = (head % n) * L + token of KV head g = head / n, i.e. column
// c % nh of head chunk c / nh.  Per-sequence list (both GQA kernels, MLA):
// piece s of it is item meta[2b] + (g * k + s) * hc + c / nh with k =
// meta[2b + 1].  Even split (per_unit, the matrix-core GQA kernel): unit
// ui = (b * H_kv + g) * hc + c / nh has k = meta[2ui + 1] pieces in the
// consecutive slots from meta[2ui].  Each slot holds nh rows.
struct BalancedMap {
  const int* meta;
  int L, H_q, n, hc, nh;
  int per_unit;
};

// CPL = d_v / 64 columns per lane, read as CPL / VW vectors of VW elements of
// P (float32 or fp16 partial values).
// BAL: the parts come from a balanced work list (`bm`), else S parts per row
// stored next to each other.  WPR waves share a row (parts s = sub, sub +
// WPR, ...) and add their sums in LDS: few rows with many parts (one long
// sequence cut into many pieces) would otherwise leave most of the GPU idle
// while one wave per row walks every part.  Eight parts are in flight per
// wave.
template <typename P, int CPL, bool BAL, int WPR>
__global__ __launch_bounds__(kThreads) void lse_combine_rows(
    const P* __restrict__ o_part, const float* __restrict__ lse_part,
    float* __restrict__ out, float* __restrict__ lse_out, int rows, int S,
    BalancedMap bm) {
  constexpr int VW = CPL >= 4 ? 4 : CPL;
  constexpr int NV = CPL / VW;
  constexpr int d_v = 64 * CPL;
  constexpr int NWG = kThreads / 64;
  constexpr int RPB = NWG / WPR;  // rows per work group
  constexpr int DEPTH = 8;        // parts in flight per wave
  static_assert(NWG % WPR == 0 && (!BAL || WPR == 1), "waves per row");
  typedef typename VecOf<P, VW>::type vec;       // partial values
  typedef typename VecOf<float, VW>::type ovec;  // outputs
  __shared__ float wts[NWG][kMaxS];
  __shared__ float red[WPR > 1 ? NWG : 1][WPR > 1 ? d_v : 1];
  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int sub = wave % WPR;
  const size_t row = (size_t)blockIdx.x * RPB + wave / WPR;
  bool active = row < (size_t)rows;
  size_t base = row * S;  // part row of part 0
  int stride = 1;         // part rows between consecutive parts
  if constexpr (BAL) {
    if (!active) return;
    const int per_b = bm.L * bm.H_q;
    const int b = (int)(row / per_b);
    const int rem = (int)(row - (size_t)b * per_b);
    const int tok = rem / bm.H_q, head = rem - tok * bm.H_q;
    const int g = head / bm.n;
    const int c = (head - g * bm.n) * bm.L + tok;
    const int chunk = c / bm.nh;
    if (bm.per_unit) {
      const int ui = (b * (bm.H_q / bm.n) + g) * bm.hc + chunk;
      S = bm.meta[2 * ui + 1];
      if (S == 1) return;  // one piece: the decode kernel wrote this row
      base = (size_t)bm.meta[2 * ui] * bm.nh + (c - chunk * bm.nh);
      stride = bm.nh;
    } else {
      S = bm.meta[2 * b + 1];
      if (S == 1) return;
      base = (size_t)(bm.meta[2 * b] + g * S * bm.hc + chunk) * bm.nh + (c - chunk * bm.nh);
      stride = bm.hc * bm.nh;
    }
  }
  if constexpr (WPR == 1) {
    if (!active) return;
  }
  float acc[NV][VW] = {};
  float M = neg_inf(), tot = 0.f;
  if (active) {
    const float* lp = lse_part + base;
    float* w_s = wts[wave];
    // lane owns columns VW*(lane + 64 v) .. +VW-1 for v < NV
    const vec* op = reinterpret_cast<const vec*>(o_part + base * d_v) + lane;
    const size_t step = (size_t)stride * (d_v / VW);  // vectors between parts
    // The first DEPTH parts' values go out with the log-sum-exps (they do not
    // depend on the weights), so a row of up to DEPTH parts costs one memory
    // round trip instead of two.
    vec x0[DEPTH][NV];
#pragma unroll
    for (int k = 0; k < DEPTH; ++k)
      if (sub + k * WPR < S)
#pragma unroll
        for (int v = 0; v < NV; ++v) x0[k][v] = op[(size_t)(sub + k * WPR) * step + 64 * v];
    const float l_first = lane < S ? lp[(size_t)lane * stride] : neg_inf();

    // weights of every part (natural-log input, log2 inside), in this wave's
    // own LDS row, so no barrier is needed between writing and reading it
    M = l_first * kLog2e;
    for (int s = lane + 64; s < S; s += 64) M = fmaxf(M, lp[(size_t)s * stride] * kLog2e);
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) M = fmaxf(M, __shfl_xor(M, off));
    for (int s = lane; s < S; s += 64) {
      const float x = s == lane ? l_first : lp[(size_t)s * stride];
      const float w = (x == neg_inf() || M == neg_inf()) ? 0.f : fast_exp2(x * kLog2e - M);
      w_s[s] = w;
      tot += w;
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) tot += __shfl_xor(tot, off);
    if (sub == 0 && lane == 0 && lse_out)
      lse_out[row] = (tot > 0.f) ? (M + fast_log2(tot)) * kLn2 : neg_inf();

#pragma unroll
    for (int k = 0; k < DEPTH; ++k)
      if (sub + k * WPR < S)
#pragma unroll
        for (int v = 0; v < NV; ++v) fma_vec<P, VW>(acc[v], w_s[sub + k * WPR], x0[k][v]);
    int s = sub + DEPTH * WPR;
    for (; s + (DEPTH - 1) * WPR < S; s += DEPTH * WPR) {
      vec x[DEPTH][NV];
#pragma unroll
      for (int k = 0; k < DEPTH; ++k)
#pragma unroll
        for (int v = 0; v < NV; ++v) x[k][v] = op[(size_t)(s + k * WPR) * step + 64 * v];
#pragma unroll
      for (int k = 0; k < DEPTH; ++k)
#pragma unroll
        for (int v = 0; v < NV; ++v) fma_vec<P, VW>(acc[v], w_s[s + k * WPR], x[k][v]);
    }
    for (; s < S; s += WPR) {
#pragma unroll
      for (int v = 0; v < NV; ++v) fma_vec<P, VW>(acc[v], w_s[s], op[(size_t)s * step + 64 * v]);
    }
  }
  if constexpr (WPR > 1) {
    // the row's waves meet in LDS (element (v, i) of lane l at (v*VW+i)*64+l)
#pragma unroll
    for (int v = 0; v < NV; ++v)
#pragma unroll
      for (int i = 0; i < VW; ++i) red[wave][(v * VW + i) * 64 + lane] = acc[v][i];
    __syncthreads();
    if (!active || sub != 0) return;
#pragma unroll
    for (int j = 1; j < WPR; ++j)
#pragma unroll
      for (int v = 0; v < NV; ++v)
#pragma unroll
        for (int i = 0; i < VW; ++i) acc[v][i] += red[wave + j][(v * VW + i) * 64 + lane];
  }
  const float inv = (tot > 0.f) ? 1.f / tot : 0.f;
  ovec* dst = reinterpret_cast<ovec*>(out + row * d_v) + lane;
#pragma unroll
  for (int v = 0; v < NV; ++v) {
    ovec r;
    float* rs = reinterpret_cast<float*>(&r);
#pragma unroll
    for (int i = 0; i < VW; ++i) rs[i] = acc[v][i] * inv;
    dst[64 * v] = r;
  }
}

template <typename P, bool BAL, int WPR>
hipError_t launch_rows(int cpl, const P* o_part, const float* lse_part, float* out,
                       float* lse, int rows, int S, const BalancedMap& bm,
                       hipStream_t stream) {
  constexpr int RPB = kThreads / 64 / WPR;
  const dim3 g((unsigned)((rows + RPB - 1) / RPB)), blk(kThreads);
  switch (cpl) {
    case 1:
      hipLaunchKernelGGL((lse_combine_rows<P, 1, BAL, WPR>), g, blk, 0, stream, o_part,
                         lse_part, out, lse, rows, S, bm);
      break;
    case 2:
      hipLaunchKernelGGL((lse_combine_rows<P, 2, BAL, WPR>), g, blk, 0, stream, o_part,
                         lse_part, out, lse, rows, S, bm);
      break;
    case 4:
      hipLaunchKernelGGL((lse_combine_rows<P, 4, BAL, WPR>), g, blk, 0, stream, o_part,
                         lse_part, out, lse, rows, S, bm);
      break;
    case 8:
      hipLaunchKernelGGL((lse_combine_rows<P, 8, BAL, WPR>), g, blk, 0, stream, o_part,
                         lse_part, out, lse, rows, S, bm);
      break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_combine(const float* o_part, const float* lse_part,
                          float* out, float* lse, int B, int H, int S, int d_v,
                          hipStream_t stream) {
  if (S > kMaxS) return hipErrorInvalidValue;
  const int rows = B * H;
  const bool vec_ok = ((uintptr_t)o_part % 16 == 0) && ((uintptr_t)out % 16 == 0);
  const int cpl = d_v % 64 == 0 ? d_v / 64 : 0;  // columns per lane, one wave per row
  if (vec_ok && (cpl == 1 || cpl == 2 || cpl == 4 || cpl == 8)) {
    // waves per row: enough waves for the GPU when rows are few and parts
    // many (about four per CU), else one
    const BalancedMap none{};
    if (S >= 32 && rows <= 256)
      return launch_rows<float, false, 4>(cpl, o_part, lse_part, out, lse, rows, S, none, stream);
    if (S >= 16 && rows <= 512)
      return launch_rows<float, false, 2>(cpl, o_part, lse_part, out, lse, rows, S, none, stream);
    return launch_rows<float, false, 1>(cpl, o_part, lse_part, out, lse, rows, S, none, stream);
  }
  const int cl = d_v >= 256 ? 256 : (d_v > 128 ? 256 : (d_v > 64 ? 128 : 64));
  hipLaunchKernelGGL(lse_combine, dim3((unsigned)rows), dim3(kThreads), 0, stream,
                     o_part, lse_part, out, lse, S, d_v, cl);
  return hipGetLastError();
}

hipError_t launch_combine_half(const void* o_part, const float* lse_part, float* out,
                               float* lse, int B, int H, int S, int d_v,
                               hipStream_t stream) {
  if (S > kMaxS || (uintptr_t)o_part % 16 != 0 || (uintptr_t)out % 16 != 0 ||
      d_v % 64 != 0 || d_v > 512)
    return hipErrorInvalidValue;
  const BalancedMap none{};
  const int rows = B * H, cpl = d_v / 64;
  const _Float16* op = (const _Float16*)o_part;
  if (S >= 32 && rows <= 256)
    return launch_rows<_Float16, false, 4>(cpl, op, lse_part, out, lse, rows, S, none, stream);
  if (S >= 16 && rows <= 512)
    return launch_rows<_Float16, false, 2>(cpl, op, lse_part, out, lse, rows, S, none, stream);
  return launch_rows<_Float16, false, 1>(cpl, op, lse_part, out, lse, rows, S, none, stream);
}

hipError_t launch_combine_balanced(const void* o_part, bool half_parts,
                                   const float* lse_part, const int* meta, float* out,
                                   float* lse, int B, int L, int H_q, int n,
                                   int head_chunks, int heads_per_item, int d_v,
                                   bool per_unit, hipStream_t stream) {
  if ((uintptr_t)o_part % 16 != 0 || (uintptr_t)out % 16 != 0 || d_v % 64 != 0 ||
      d_v > 512)
    return hipErrorInvalidValue;
  const BalancedMap bm{meta, L, H_q, n, head_chunks, heads_per_item, per_unit ? 1 : 0};
  if (half_parts)
    return launch_rows<_Float16, true, 1>(d_v / 64, (const _Float16*)o_part, lse_part, out,
                                          lse, B * L * H_q, 0, bm, stream);
  return launch_rows<float, true, 1>(d_v / 64, (const float*)o_part, lse_part, out, lse,
                                     B * L * H_q, 0, bm, stream);
}

}  // namespace attn
