// Log-sum-exp merge of split results (kernel 2).
//
// For each (b, h): L = max_s lse_s, w_s = exp(lse_s - L),
//   out = sum_s w_s o_s / sum_s w_s,  lse = L + ln(sum_s w_s).
// Softmax over a union of disjoint key sets factors this way because each
// part's normaliser is exp(lse_s) (attention equation, xuesongtap
// "attention-head" note, section 1).  Parts with lse = -inf are empty and get
// weight 0; if every part is empty the output is 0 and lse is -inf.
//
// One work group of 64 lanes per (b, h).  The S weights are computed once per
// group into LDS (S <= 1024), then each lane streams d_v/64 output columns
// over the S partial rows; reads of one partial row are coalesced.

#include "device_common.h"
#include "internal.h"

namespace attn {
namespace {

constexpr int kMaxS = 1024;

__global__ __launch_bounds__(64) void lse_combine(const float* __restrict__ o_part,
                                                  const float* __restrict__ lse_part,
                                                  float* __restrict__ out,
                                                  float* __restrict__ lse_out,
                                                  int S, int d_v) {
  __shared__ float wts[kMaxS];
  const size_t row = blockIdx.x;
  const float* lp = lse_part + row * S;
  const int lane = threadIdx.x;

  // max over parts (natural-log domain -> log2 domain)
  float M = neg_inf();
  for (int s = lane; s < S; s += 64) M = fmaxf(M, lp[s] * kLog2e);
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1)
    M = fmaxf(M, __shfl_xor(M, off));

  float tot = 0.f;
  for (int s = lane; s < S; s += 64) {
    const float x = lp[s];
    const float w = (x == neg_inf() || M == neg_inf()) ? 0.f : fast_exp2(x * kLog2e - M);
    wts[s] = w;
    tot += w;
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) tot += __shfl_xor(tot, off);
  __syncthreads();

  const bool empty = !(tot > 0.f);
  const float inv = empty ? 0.f : 1.f / tot;
  const float* op = o_part + row * (size_t)S * d_v;
  for (int e = lane; e < d_v; e += 64) {
    float acc = 0.f;
    for (int s = 0; s < S; ++s) {
      const float w = wts[s];
      if (w != 0.f) acc = fmaf(w, op[(size_t)s * d_v + e], acc);
    }
    out[row * d_v + e] = acc * inv;
  }
  if (lse_out && lane == 0)
    lse_out[row] = empty ? neg_inf() : (M + fast_log2(tot)) * kLn2;
}

}  // namespace

hipError_t launch_combine(const float* o_part, const float* lse_part,
                          float* out, float* lse, int B, int H, int S, int d_v,
                          hipStream_t stream) {
  if (S > kMaxS) return hipErrorInvalidValue;
  hipLaunchKernelGGL(lse_combine, dim3((unsigned)B * H), dim3(64), 0, stream,
                     o_part, lse_part, out, lse, S, d_v);
  return hipGetLastError();
}

}  // namespace attn
