// Log-sum-exp merge of split results (kernel 2).
//
// For each (b, h): L = max_s lse_s, w_s = exp(lse_s - L),
//   out = sum_s w_s o_s / sum_s w_s,  lse = L + ln(sum_s w_s).
// Softmax over a union of disjoint key sets factors this way because each
// part's normaliser is exp(lse_s) (attention equation, xuesongtap
// "attention-head" note, section 1).  Parts with lse = -inf are empty and get
// weight 0; if every part is empty the output is 0 and lse is -inf.
//
// One work group of 256 lanes per (b, h): lanes cover the columns (up to
// 256 at a time) and, when the value is narrower than 256, the remaining
// lanes split the parts between them and meet in LDS.  Loads over the parts
// are independent and unrolled, so many are in flight per lane.

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

}  // namespace

hipError_t launch_combine(const float* o_part, const float* lse_part,
                          float* out, float* lse, int B, int H, int S, int d_v,
                          hipStream_t stream) {
  if (S > kMaxS) return hipErrorInvalidValue;
  const int cl = d_v >= 256 ? 256 : (d_v > 128 ? 256 : (d_v > 64 ? 128 : 64));
  hipLaunchKernelGGL(lse_combine, dim3((unsigned)B * H), dim3(kThreads), 0, stream,
                     o_part, lse_part, out, lse, S, d_v, cl);
  return hipGetLastError();
}

}  // namespace attn
