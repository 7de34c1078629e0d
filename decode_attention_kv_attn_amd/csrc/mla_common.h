// Device helpers shared by the two MLA decode kernels: the latent tile's
// LDS layout (16-byte chunk swizzle), bf16 -> fp16 conversion, direct-to-LDS
// buffer loads and the waits and barriers that go with them.
#pragma once

#include <stdint.h>

#include "device_common.h"

namespace attn {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// s_buffer_load_dword (uniform offset, through the scalar cache).
__device__ int scalar_buffer_load_i32(u32x4 rsrc, int offset, int cachepolicy) __asm(
    "llvm.amdgcn.s.buffer.load.i32");

constexpr int kBufferWord3 = 0x00020000;  // raw buffer descriptor flags (gfx9)

// Chunk swizzle: logical 16-byte chunk c of row t sits at chunk c ^ swz(t);
// the xor stays inside an aligned group of 8 chunks.  Chosen by measured LDS
// read rate of the two read patterns (16 rows at one chunk for the score
// operand, 16 rows at two adjacent chunks for the transposed value operand).
// swz(t + 16) = swz(t): the two 16-row halves of a tile share their layout.
ATTN_DEV int swz(int t) { return t & 7; }

typedef _Float16 f16x2_v __attribute__((ext_vector_type(2)));
typedef float f32x2_v __attribute__((ext_vector_type(2)));

// (a, b) -> packed fp16, rounded to nearest even (v_cvt_pk_f16_f32).
ATTN_DEV uint32_t pack_f16(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_v{a, b}, f16x2_v));
}

// Two bf16 (one dword) -> two fp16 (exact in fp16's normal range).
ATTN_DEV uint32_t bf16x2_to_f16x2(uint32_t w) {
  return pack_f16(__uint_as_float(w << 16), __uint_as_float(w & 0xffff0000u));
}

ATTN_DEV uint4 bf16x8_to_f16x8(uint4 u) {
  return make_uint4(bf16x2_to_f16x2(u.x), bf16x2_to_f16x2(u.y), bf16x2_to_f16x2(u.z),
                    bf16x2_to_f16x2(u.w));
}

ATTN_DEV u32x4 as_u32x4(const uint4& u) { return __builtin_bit_cast(u32x4, u); }

// One direct-to-LDS buffer load: lane l copies the 16 bytes at `base` + voff
// (the descriptor covers `bytes`) to LDS address lds + 16 l.  Written out so
// the compiler does not track it: its own form makes every later LDS read
// it cannot tell apart from the destination wait for all such loads, which
// empties the prefetch pipeline.  Every wait on these loads is explicit
// (wait_vmcnt before the barrier that publishes a tile, and at the end).
ATTN_DEV void dma_16B(const void* base, uint32_t bytes, uint32_t voff, uint32_t lds) {
  const uint64_t b = (uint64_t)(uintptr_t)base;
  const u32x4 rsrc = {(uint32_t)b, (uint32_t)(b >> 32) & 0xffffu, bytes, (uint32_t)kBufferWord3};
  asm volatile(
      "s_mov_b32 m0, %1\n\t"
      "s_nop 0\n\t"
      "buffer_load_dwordx4 %0, %2, 0 offen lds"
      :
      : "v"(voff), "s"(lds), "s"(rsrc)
      : "m0");
}

// Work-group barrier that is also a compiler memory barrier, without the
// release fence of __syncthreads (which would wait for the direct-to-LDS
// loads still in flight for later tiles).  This wave's own LDS reads are
// drained first, so a stage is never refilled under a pending read.
ATTN_DEV void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// s_waitcnt vmcnt(n) (other counters unconstrained), gfx9 encoding.
template <int N>
ATTN_DEV void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

}  // namespace
}  // namespace attn
