// Cache append: write the new token's rows into the cache before a decode
// call (the pages' modules concatenate the current key and value onto the
// past ones along the sequence axis -- toolsku MHA / GQA / MLA modules; a
// sliding-window layer may instead reuse the oldest slot of a ring --
// xuesongtap "attention-head" note, section 3).
//
// One work group per (sequence, head): each lane moves 16-byte chunks of the
// row.  The work is a few KiB per call, so the kernel is launch-bound.  A
// paged pool is addressed through the block table (baidu article, section
// 四.3: KV-cache paging).

#include "../../include/attn_decode.h"
#include "device_common.h"
#include "internal.h"

namespace attn {
namespace {

// Linear: row positions[b] of every head (skipped unless 0 <= pos < T_cap).
// Ring: every head's row goes to the slot after ring_head[b] (mod T_cap);
// the head itself is advanced by a second kernel on the same stream, so no
// group reads a head that another group already moved.
__global__ __launch_bounds__(64) void append_rows(
    unsigned char* __restrict__ k_cache, unsigned char* __restrict__ v_cache,
    const unsigned char* __restrict__ k_new, const unsigned char* __restrict__ v_new,
    const int32_t* __restrict__ positions, const int32_t* __restrict__ ring_head,
    int H, int T_cap, int row_bytes) {
  const int b = blockIdx.x / H;
  int slot;
  if (ring_head) {
    int h = ring_head[b] % T_cap;
    h = h < 0 ? h + T_cap : h;
    slot = h + 1 == T_cap ? 0 : h + 1;
  } else {
    slot = positions[b];
    if (slot < 0 || slot >= T_cap) return;
  }
  const size_t src = (size_t)blockIdx.x * row_bytes;
  const size_t dst = ((size_t)blockIdx.x * T_cap + slot) * row_bytes;
  for (int c = threadIdx.x * 16; c < row_bytes; c += 64 * 16) {
    *(uint4*)(k_cache + dst + c) = *(const uint4*)(k_new + src + c);
    if (v_cache) *(uint4*)(v_cache + dst + c) = *(const uint4*)(v_new + src + c);
  }
}

// Paged: position positions[b] of sequence b goes to page
// table[b][pos >> shift], row pos & (P - 1), of every head (skipped unless
// 0 <= pos < max_pages * P; page ids are clamped to the pool).
__global__ __launch_bounds__(64) void append_rows_paged(
    unsigned char* __restrict__ k_pages, unsigned char* __restrict__ v_pages,
    const unsigned char* __restrict__ k_new, const unsigned char* __restrict__ v_new,
    const int32_t* __restrict__ positions, const int32_t* __restrict__ table,
    int max_pages, int shift, int num_pages, int H, int row_bytes) {
  const int b = blockIdx.x / H;
  const int h = blockIdx.x - b * H;
  const int pos = positions[b];
  if (pos < 0 || (pos >> shift) >= max_pages) return;
  int page = table[(size_t)b * max_pages + (pos >> shift)];
  page = page < 0 ? 0 : (page >= num_pages ? num_pages - 1 : page);
  const size_t src = (size_t)blockIdx.x * row_bytes;
  const size_t dst =
      ((((size_t)page * H + h) << shift) + (pos & ((1 << shift) - 1))) * row_bytes;
  for (int c = threadIdx.x * 16; c < row_bytes; c += 64 * 16) {
    *(uint4*)(k_pages + dst + c) = *(const uint4*)(k_new + src + c);
    if (v_pages) *(uint4*)(v_pages + dst + c) = *(const uint4*)(v_new + src + c);
  }
}

__global__ __launch_bounds__(64) void advance_ring(int32_t* ring_head, int B, int T_cap) {
  const int b = blockIdx.x * 64 + threadIdx.x;
  if (b >= B) return;
  int h = ring_head[b] % T_cap;
  h = h < 0 ? h + T_cap : h;
  ring_head[b] = h + 1 == T_cap ? 0 : h + 1;
}

int check(const void* k_cache, const void* k_new, int B, int H, int T_cap, int d,
          int dtype) {
  if (B < 0 || H <= 0 || T_cap <= 0 || d <= 0) return ATTN_ERR_SHAPE;
  if (dtype != ATTN_F32 && dtype != ATTN_BF16) return ATTN_ERR_DTYPE;
  const int s = dtype == ATTN_F32 ? 4 : 2;
  if ((d * s) % 16 != 0) return ATTN_ERR_ALIGN;
  if ((long long)B * H > 0x7fffffffLL) return ATTN_ERR_SHAPE;
  (void)k_cache;
  (void)k_new;
  return ATTN_OK;
}

}  // namespace
}  // namespace attn

using namespace attn;

extern "C" {

int attn_kv_append(void* k_cache, void* v_cache, const void* k_new,
                   const void* v_new, const int32_t* positions, int B, int H,
                   int T_cap, int d, int dtype, void* stream) {
  int st = check(k_cache, k_new, B, H, T_cap, d, dtype);
  if (st != ATTN_OK) return st;
  if (B == 0) return ATTN_OK;
  if (!k_cache || !k_new || !positions || (!v_cache != !v_new)) return ATTN_ERR_NULL;
  if (((uintptr_t)k_cache | (uintptr_t)k_new | (uintptr_t)v_cache | (uintptr_t)v_new) % 16)
    return ATTN_ERR_ALIGN;
  const int row_bytes = d * (dtype == ATTN_F32 ? 4 : 2);
  hipLaunchKernelGGL(append_rows, dim3((unsigned)(B * H)), dim3(64), 0,
                     (hipStream_t)stream, (unsigned char*)k_cache,
                     (unsigned char*)v_cache, (const unsigned char*)k_new,
                     (const unsigned char*)v_new, positions, nullptr, H, T_cap,
                     row_bytes);
  return hipGetLastError() == hipSuccess ? ATTN_OK : ATTN_ERR_HIP;
}

int attn_kv_append_ring(void* k_cache, void* v_cache, const void* k_new,
                        const void* v_new, int32_t* ring_head, int B, int H,
                        int T_cap, int d, int dtype, void* stream) {
  int st = check(k_cache, k_new, B, H, T_cap, d, dtype);
  if (st != ATTN_OK) return st;
  if (B == 0) return ATTN_OK;
  if (!k_cache || !k_new || !ring_head || (!v_cache != !v_new)) return ATTN_ERR_NULL;
  if (((uintptr_t)k_cache | (uintptr_t)k_new | (uintptr_t)v_cache | (uintptr_t)v_new) % 16)
    return ATTN_ERR_ALIGN;
  const int row_bytes = d * (dtype == ATTN_F32 ? 4 : 2);
  hipStream_t s = (hipStream_t)stream;
  hipLaunchKernelGGL(append_rows, dim3((unsigned)(B * H)), dim3(64), 0, s,
                     (unsigned char*)k_cache, (unsigned char*)v_cache,
                     (const unsigned char*)k_new, (const unsigned char*)v_new,
                     nullptr, (const int32_t*)ring_head, H, T_cap, row_bytes);
  if (hipGetLastError() != hipSuccess) return ATTN_ERR_HIP;
  hipLaunchKernelGGL(advance_ring, dim3((unsigned)((B + 63) / 64)), dim3(64), 0, s,
                     ring_head, B, T_cap);
  return hipGetLastError() == hipSuccess ? ATTN_OK : ATTN_ERR_HIP;
}

int attn_kv_append_paged(void* k_pages, void* v_pages, const void* k_new,
                         const void* v_new, const int32_t* positions,
                         const int32_t* block_table, int max_pages, int B, int H,
                         int num_pages, int page_size, int d, int dtype,
                         void* stream) {
  int shift = 0;
  int st = attn_check_pages(max_pages, num_pages, page_size, H, &shift);
  if (st != ATTN_OK) return st;
  st = check(k_pages, k_new, B, H, page_size, d, dtype);
  if (st != ATTN_OK) return st;
  if (B == 0) return ATTN_OK;
  if (!k_pages || !k_new || !positions || !block_table || (!v_pages != !v_new))
    return ATTN_ERR_NULL;
  if (((uintptr_t)k_pages | (uintptr_t)k_new | (uintptr_t)v_pages | (uintptr_t)v_new) % 16 ||
      (uintptr_t)positions % 4 || (uintptr_t)block_table % 4)
    return ATTN_ERR_ALIGN;
  const int row_bytes = d * (dtype == ATTN_F32 ? 4 : 2);
  hipLaunchKernelGGL(append_rows_paged, dim3((unsigned)(B * H)), dim3(64), 0,
                     (hipStream_t)stream, (unsigned char*)k_pages,
                     (unsigned char*)v_pages, (const unsigned char*)k_new,
                     (const unsigned char*)v_new, positions, block_table,
                     max_pages, shift, num_pages, H, row_bytes);
  return hipGetLastError() == hipSuccess ? ATTN_OK : ATTN_ERR_HIP;
}

}  // extern "C"
