// Log-sum-exp merge of split results (kernel 2).
//
// For each (b, h): L = max_s lse_s, w_s = exp(lse_s - L),
//   out = sum_s w_s o_s / sum_s w_s,  lse = L + ln(sum_s w_s).
// Softmax over a union of disjoint key sets factors this way because each
// part's normaliser is exp(lse_s) (attention equation, xuesongtap
// "attention-head" note, section 1).  Parts with lse = -inf are empty and get
// weight 0; if every part is empty the output is 0 and lse is -inf.
//
// Grid: (b*h, 64-column slice).  Four waves per group: all compute the S
// weights into LDS, then wave w sums the parts s = w, w+4, ... for its lane's
// column with several loads in flight, and the four partial sums meet in LDS.
// Small batches with many splits (one long sequence) thus still spread over
// many waves instead of one wave walking every split.

#include "device_common.h"
#include "internal.h"

namespace attn {
namespace {

constexpr int kMaxS = 1024;
constexpr int kWaves = 4;

// Empty parts (weight 0) contribute nothing, whatever their o_part holds.
ATTN_DEV float add_part(float acc, float w, float x) {
  return w > 0.f ? fmaf(w, x, acc) : acc;
}

__global__ __launch_bounds__(kWaves * 64) void lse_combine(
    const float* __restrict__ o_part, const float* __restrict__ lse_part,
    float* __restrict__ out, float* __restrict__ lse_out, int S, int d_v) {
  __shared__ float wts[kMaxS];
  __shared__ float red[kWaves][64];
  __shared__ float tot_s;
  const size_t row = blockIdx.x;
  const float* lp = lse_part + row * S;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;

  // max over parts (natural-log input, log2 domain inside); wave 0 reduces
  if (wave == 0) {
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
      if (lse_out && blockIdx.y == 0)
        lse_out[row] = (tot > 0.f) ? (M + fast_log2(tot)) * kLn2 : neg_inf();
    }
  }
  __syncthreads();

  const int e = blockIdx.y * 64 + lane;
  float acc = 0.f;
  if (e < d_v) {
    const float* op = o_part + row * (size_t)S * d_v + e;
    int s = wave;
    for (; s + 3 * kWaves < S; s += 4 * kWaves) {
      const float x0 = op[(size_t)s * d_v];
      const float x1 = op[(size_t)(s + kWaves) * d_v];
      const float x2 = op[(size_t)(s + 2 * kWaves) * d_v];
      const float x3 = op[(size_t)(s + 3 * kWaves) * d_v];
      acc = add_part(acc, wts[s], x0);
      acc = add_part(acc, wts[s + kWaves], x1);
      acc = add_part(acc, wts[s + 2 * kWaves], x2);
      acc = add_part(acc, wts[s + 3 * kWaves], x3);
    }
    for (; s < S; s += kWaves) acc = add_part(acc, wts[s], op[(size_t)s * d_v]);
  }
  red[wave][lane] = acc;
  __syncthreads();
  if (wave == 0 && e < d_v) {
    float sum = red[0][lane];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) sum += red[w][lane];
    const float tot = tot_s;
    out[row * d_v + e] = (tot > 0.f) ? sum / tot : 0.f;
  }
}

}  // namespace

hipError_t launch_combine(const float* o_part, const float* lse_part,
                          float* out, float* lse, int B, int H, int S, int d_v,
                          hipStream_t stream) {
  if (S > kMaxS) return hipErrorInvalidValue;
  hipLaunchKernelGGL(lse_combine, dim3((unsigned)B * H, (d_v + 63) / 64),
                     dim3(kWaves * 64), 0, stream, o_part, lse_part, out, lse, S,
                     d_v);
  return hipGetLastError();
}

}  // namespace attn
