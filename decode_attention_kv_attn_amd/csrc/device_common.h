// Device helpers shared by the decode kernels (gfx950 / CDNA4, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#define ATTN_DEV __device__ __forceinline__

namespace attn {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

ATTN_DEV float neg_inf() { return -__builtin_inff(); }

// bf16 halves of a packed dword -> float32 (exact).
ATTN_DEV float bf16_lo(uint32_t u) { return __uint_as_float(u << 16); }
ATTN_DEV float bf16_hi(uint32_t u) { return __uint_as_float(u & 0xffff0000u); }

// a.x*b.x + a.y*b.y + c for packed bf16 pairs; the bf16 products are exact in
// float32 (v_dot2c_f32_bf16).
ATTN_DEV float dot2_bf16(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                         __builtin_bit_cast(bf16x2_t, b), c,
                                         false);
}

// 2^x on the transcendental unit; 2^-inf = 0.
ATTN_DEV float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
ATTN_DEV float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

// ---- cross-lane moves ------------------------------------------------------
// DPP controls (gfx9 encoding).
enum : int {
  kDppQuadXor1 = 0xB1,    // quad_perm [1,0,3,2]
  kDppQuadXor2 = 0x4E,    // quad_perm [2,3,0,1]
  kDppRowRor4 = 0x124,    // row_ror:4
  kDppRowRor8 = 0x128,    // row_ror:8  (== xor 8 inside a 16-lane row)
  kDppRowMirror = 0x140,  // lane i <- lane 15-i inside a row
  kDppHalfMirror = 0x141  // lane i <- lane 7-i inside each 8-lane half
};

template <int CTRL>
ATTN_DEV float dpp(float x) {
  return __int_as_float(
      __builtin_amdgcn_mov_dpp(__float_as_int(x), CTRL, 0xF, 0xF, true));
}

// Value of lane (i ^ 16).  v_permlane16_swap(x, x) returns, per 16-lane row
// r, the pair (x of row r&~1, x of row r|1) (checked on gfx950): the partner
// row is the second element on even rows and the first on odd rows.
ATTN_DEV float xor16(float x) {
  const unsigned u = __float_as_uint(x);
  const auto p = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  return __uint_as_float((__lane_id() & 16) ? p[0] : p[1]);
}
// Value of lane (i ^ 32): v_permlane32_swap(x, x) returns (x of the low half,
// x of the high half) in both halves.
ATTN_DEV float xor32(float x) {
  const unsigned u = __float_as_uint(x);
  const auto p = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return __uint_as_float((__lane_id() & 32) ? p[0] : p[1]);
}

// Sum over aligned groups of L consecutive lanes; every lane of the group
// receives the total.  The pairings need not be xor: each step adds a lane
// whose partial covers the other half of the current block.
template <int L>
ATTN_DEV float group_sum(float x) {
  static_assert(L == 1 || L == 2 || L == 4 || L == 8 || L == 16 || L == 32 ||
                    L == 64,
                "group size");
  if constexpr (L >= 2) x += dpp<kDppQuadXor1>(x);
  if constexpr (L >= 4) x += dpp<kDppQuadXor2>(x);
  if constexpr (L >= 8) x += dpp<kDppHalfMirror>(x);
  if constexpr (L >= 16) x += dpp<kDppRowMirror>(x);
  if constexpr (L >= 32) x += xor16(x);
  if constexpr (L >= 64) x += xor32(x);
  return x;
}

// Running softmax state of one row group: max m (log2 domain), sum l, and
// weighted value sums acc.  merge() folds another state over a disjoint key
// set into this one (the log-sum-exp rule).
ATTN_DEV void lse_merge_scalars(float& m, float& l, float mo, float lo,
                                float& a_self, float& a_other) {
  const float mn = fmaxf(m, mo);
  a_self = (m == neg_inf()) ? 0.f : fast_exp2(m - mn);
  a_other = (mo == neg_inf()) ? 0.f : fast_exp2(mo - mn);
  l = a_self * l + a_other * lo;
  m = mn;
}

}  // namespace attn
