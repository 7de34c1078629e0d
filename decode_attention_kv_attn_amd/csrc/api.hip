// Host side of the C ABI declared in include/attn_decode.h: argument checks
// (host values only, before any HIP call), split planning, launches.

#include <math.h>
#include <stdlib.h>

#include <atomic>
#include <mutex>

#include "../../include/attn_decode.h"
#include "internal.h"

namespace attn {
namespace {

inline bool aligned(const void* p, size_t a) {
  return ((uintptr_t)p % a) == 0;
}

inline size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// Work groups the planner aims for before it cuts the visible range into
// more splits: one per CU, each a full CU's worth of waves.  Overridable for
// tuning sweeps through ATTN_DECODE_TARGET_GROUPS.
// Lead tiles per unit of the even split: the start-up cost of a unit in a
// work group -- mostly one HBM round trip under load before its first tile
// can be computed, plus the waves' merge at its end -- in tiles of 32 rows.
// Measured at d = 128 (MQA, lengths 1k..32k) the best lead is 12 tiles,
// about 7 us; a tile of width d costs time in proportion to d, so the lead
// is 1536 / d tiles (overridable for tuning sweeps through
// ATTN_DECODE_EVEN_LEAD).
int even_lead(int d) {
  static const int v = [] {
    const char* e = getenv("ATTN_DECODE_EVEN_LEAD");
    const int x = e ? atoi(e) : -1;
    return x >= 0 && x <= 256 ? x : -1;
  }();
  return v >= 0 ? v : max(1, 1536 / d);
}

// Work groups a split plan (and a balanced list) aims for: one per CU for
// the matrix-core kernel, whose registers hold one group per CU; two per CU
// for the vector kernel, whose groups of four waves leave room for two
// (MHA B=1, 32768 rows: 85.0 us at one group per CU, 83.8 at two).
// Overridable for tuning sweeps through ATTN_DECODE_TARGET_GROUPS.
int target_groups(bool mfma) {
  static const int v = [] {
    const char* e = getenv("ATTN_DECODE_TARGET_GROUPS");
    const int x = e ? atoi(e) : 0;
    return x > 0 ? x : 0;
  }();
  return v > 0 ? v : (mfma ? kNumCUs : 2 * kNumCUs);
}

struct GqaPlan {
  int mfma;         // 1: matrix-core kernel, 0: vector kernel
  int N;            // heads per work item
  int head_chunks;  // work items per KV head along the heads
  int S;            // splits
  int chunk;        // positions per split
  int waves;        // waves per work group
  int tile_rows;    // positions per wave per tile
  size_t ws_bytes;  // workspace needed
  size_t ws_fixed;  // workspace of the fixed splits alone
  int cap;          // > 0: work groups of the balanced list (calls with lengths)
  int even;         // 1: the list is the even split (matrix-core kernel)
  int units;        // (KV head, head chunk) units per sequence
};

// Partial slots of a balanced list: one per item of the per-sequence list;
// the even split needs one per (group, unit) segment, at most groups plus
// the units of the batch.
size_t list_slots(const GqaPlan& p, int B) {
  return p.even ? (size_t)p.cap + (size_t)B * p.units : (size_t)p.cap;
}

// Workspace of a balanced list: o_part and lse_part (N rows per slot), then
// the (first slot, pieces) pairs, per sequence or, for the even split, per
// unit.
size_t balanced_bytes(const GqaPlan& p, int d, int B) {
  const size_t rows = list_slots(p, B) * p.N;
  const size_t pairs = p.even ? (size_t)B * p.units : (size_t)B;
  return round_up(rows * d * sizeof(float), 256) + round_up(rows * sizeof(float), 256) +
         round_up(pairs * 2 * sizeof(int), 256);
}

// Largest number of positions a non-global query can have visible (a query
// that is itself a global position sees more; the last split takes the rest).
int max_visible(int T_cap, int window, int ring, int n_global) {
  if (ring) return window > 0 ? window : T_cap;
  if (window <= 0) return T_cap;
  const long long v = (long long)window + n_global;
  return v < T_cap ? (int)v : T_cap;
}

int check_gqa_shape(int B, int H_q, int H_kv, int T_cap, int d, int dtype,
                    int window, int ring) {
  if (B < 0 || H_q <= 0 || H_kv <= 0 || T_cap <= 0) return ATTN_ERR_SHAPE;
  if (H_q % H_kv != 0) return ATTN_ERR_SHAPE;
  if (dtype != ATTN_F32 && dtype != ATTN_BF16) return ATTN_ERR_DTYPE;
  if (d != 64 && d != 128 && d != 256) return ATTN_ERR_UNSUPPORTED;
  if (window < 0) return ATTN_ERR_WINDOW;
  if (ring && window > T_cap) return ATTN_ERR_WINDOW;
  // 32-bit indices inside the kernels: positions and (row * H) products.
  if ((long long)B * H_q > (1LL << 30)) return ATTN_ERR_SHAPE;
  return ATTN_OK;
}

}  // namespace
}  // namespace attn

// Page geometry shared by the paged entry points: page_size a power of two
// in [16, 2^16], at least one page, every logical length and every row of
// the pool addressable with 32-bit indices.
int attn_check_pages(int max_pages, int num_pages, int page_size, int rows_per_pos,
                     int* shift) {
  if (max_pages <= 0 || num_pages <= 0 || rows_per_pos <= 0) return ATTN_ERR_SHAPE;
  if (page_size < 16 || page_size > (1 << 16) || (page_size & (page_size - 1)))
    return ATTN_ERR_UNSUPPORTED;
  if ((long long)max_pages * page_size > (1LL << 30)) return ATTN_ERR_SHAPE;
  if ((long long)num_pages * rows_per_pos * page_size > 0x7fffffffLL)
    return ATTN_ERR_SHAPE;
  int s = 0;
  while ((1 << s) < page_size) ++s;
  *shift = s;
  return ATTN_OK;
}

namespace attn {
namespace {

int plan_gqa(int B, int H_q, int H_kv, int T_cap, int d, int dtype, int window,
             int ring, int n_global, int num_splits, GqaPlan* p) {
  int st = check_gqa_shape(B, H_q, H_kv, T_cap, d, dtype, window, ring);
  if (st != ATTN_OK) return st;
  if (n_global < 0 || n_global > ATTN_MAX_GLOBAL || (ring && n_global > 0))
    return ATTN_ERR_ARG;
  if (num_splits < 0 || num_splits > ATTN_MAX_SPLITS) return ATTN_ERR_ARG;
  const int n = H_q / H_kv;
  ValuGeometry geo;
  const int nh_mfma = mfma_heads_per_item(dtype, d, n);
  if (nh_mfma > 0) {
    geo.heads_per_item = nh_mfma;
    geo.tile_rows = mfma_tile_rows();
    geo.waves = mfma_waves();
  } else if (!valu_geometry(dtype, d, n, &geo)) {
    return ATTN_ERR_UNSUPPORTED;
  }
  p->mfma = nh_mfma > 0;
  p->N = geo.heads_per_item;
  p->head_chunks = (n + geo.heads_per_item - 1) / geo.heads_per_item;
  p->waves = geo.waves;
  p->tile_rows = geo.tile_rows;
  const int mv = max_visible(T_cap, window, ring, n_global);
  long long S;
  if (num_splits > 0) {
    S = num_splits;
  } else {
    const long long units = (long long)(B > 0 ? B : 1) * H_kv * p->head_chunks;
    S = (target_groups(p->mfma) + units - 1) / units;
    // keep at least two tiles per wave
    long long smax = mv / ((long long)geo.waves * geo.tile_rows * 2);
    if (smax < 1) smax = 1;
    if (S > smax) S = smax;
  }
  if (S < 1) S = 1;
  if (S > ATTN_MAX_SPLITS) S = ATTN_MAX_SPLITS;
  if (S > mv) S = mv;
  p->chunk = (int)((mv + S - 1) / S);
  p->S = (mv + p->chunk - 1) / p->chunk;
  p->ws_fixed = attn_decode_workspace_bytes(B, H_q, d, p->S);
  p->ws_bytes = p->ws_fixed;
  // Balanced work list: when the fixed plan splits (fewer units than work
  // groups), a call with lengths cuts each sequence by its own visible rows.
  // Not for rings: once a sequence has wrapped its visible range is the
  // whole ring (or its window), the same for every sequence, and the list's
  // setup (about a microsecond per group) would buy nothing.
  p->cap = 0;
  p->units = H_kv * p->head_chunks;
  // the even split numbers tiles of 32 rows with ints: B * units * line
  // positions per unit (at most T_cap / 32 + 1 tiles plus the lead) must stay
  // below 2^31
  // (d = 256 keeps the per-sequence list: the segment loop would push that
  // instantiation, already at the register limit, into spills)
  p->even = p->mfma && d <= 128 && (long long)B * p->units *
                               (T_cap / mfma_tile_rows() + 1 + even_lead(d)) <
                           (1LL << 31);
  if (num_splits == 0 && p->S > 1 && !ring && B >= 1 && B <= kBalanceMaxB &&
      target_groups(p->mfma) <= ATTN_MAX_SPLITS) {
    p->cap = target_groups(p->mfma);
    const size_t bb = balanced_bytes(*p, d, B);
    if (bb > p->ws_bytes) p->ws_bytes = bb;
  }
  return ATTN_OK;
}

}  // namespace
}  // namespace attn

using namespace attn;

extern "C" {

size_t attn_decode_workspace_bytes(int B, int H, int d_v, int num_splits) {
  if (B <= 0 || H <= 0 || d_v <= 0 || num_splits <= 1) return 0;
  const size_t rows = (size_t)B * H * num_splits;
  return round_up(rows * d_v * sizeof(float), 256) +
         round_up(rows * sizeof(float), 256);
}

int attn_decode_gqa_splits(int B, int H_q, int H_kv, int T_cap, int d,
                           int dtype, int window, int ring, int num_splits) {
  GqaPlan p;
  const int st = plan_gqa(B, H_q, H_kv, T_cap, d, dtype, window, ring, 0,
                          num_splits, &p);
  return st == ATTN_OK ? p.S : st;
}

int attn_decode_gqa_plan(int B, int q_len, int H_q, int H_kv, int T_cap, int d,
                         int dtype, int window, int ring, int n_global,
                         int num_splits, attn_gqa_plan* plan) {
  if (!plan) return ATTN_ERR_NULL;
  if (q_len < 1 || q_len > ATTN_MAX_QLEN) return ATTN_ERR_ARG;
  if (q_len > 1 && n_global > 0) return ATTN_ERR_UNSUPPORTED;
  if (H_q > 0 && (long long)H_q * q_len > (1 << 30)) return ATTN_ERR_SHAPE;
  if (window < 0) return ATTN_ERR_WINDOW;
  GqaPlan p;
  const int st = plan_gqa(B, H_q * q_len, H_kv, T_cap, d, dtype,
                          window > 0 ? window + q_len - 1 : 0, ring ? 1 : 0,
                          n_global, num_splits, &p);
  if (st != ATTN_OK) return st;
  plan->kernel = p.mfma;
  plan->splits = p.S;
  plan->chunk = p.chunk;
  plan->heads_per_item = p.N;
  plan->tile_rows = p.tile_rows;
  plan->waves = p.waves;
  plan->groups = (long long)B * H_kv * p.head_chunks * p.S;
  plan->workspace_bytes = p.ws_bytes;
  plan->balanced_groups = p.cap;
  plan->even_split = p.cap > 0 && p.even;
  return ATTN_OK;
}

int attn_decode_gqa_global_splits(int B, int H_q, int H_kv, int T_cap, int d,
                                  int dtype, int window, int n_global,
                                  int num_splits) {
  GqaPlan p;
  const int st = plan_gqa(B, H_q, H_kv, T_cap, d, dtype, window, 0, n_global,
                          num_splits, &p);
  return st == ATTN_OK ? p.S : st;
}

size_t attn_decode_gqa_workspace_bytes(int B, int H_q, int H_kv, int T_cap,
                                       int d, int dtype, int window, int ring,
                                       int num_splits) {
  GqaPlan p;
  const int st = plan_gqa(B, H_q, H_kv, T_cap, d, dtype, window, ring, 0,
                          num_splits, &p);
  return st == ATTN_OK ? p.ws_bytes : (size_t)-1;
}

size_t attn_decode_gqa_global_workspace_bytes(int B, int H_q, int H_kv,
                                              int T_cap, int d, int dtype,
                                              int window, int n_global,
                                              int num_splits) {
  GqaPlan p;
  const int st = plan_gqa(B, H_q, H_kv, T_cap, d, dtype, window, 0, n_global,
                          num_splits, &p);
  return st == ATTN_OK ? p.ws_bytes : (size_t)-1;
}

}  // extern "C"

// ----------------------------------------------------------------------------
// attn_decode_gqa_noalloc: attn_decode_gqa with its split / balanced-list
// buffers in a file-scope device array instead of a caller's workspace.
// Each device holds its own copy of `scratch` until the process ends.  Host
// code never passes the array's name to a kernel or a copy (on the host it is
// only a stand-in for the symbol): the device address comes from
// hipGetSymbolAddress, looked up once per device with that device current,
// and is the only form of the buffer host code uses.
namespace attn {
namespace {

static __device__ __align__(256) unsigned char scratch[ATTN_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch_addr[kMaxDevices];
std::mutex g_scratch_mu;

// Device address of the current device's scratch (nullptr on failure).
void* scratch_addr(int* status) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    *status = ATTN_ERR_HIP;
    return nullptr;
  }
  void* p = g_scratch_addr[dev].load(std::memory_order_acquire);
  if (p) return p;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  p = g_scratch_addr[dev].load(std::memory_order_relaxed);
  if (!p) {
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) {
      *status = ATTN_ERR_HIP;
      return nullptr;
    }
    g_scratch_addr[dev].store(p, std::memory_order_release);
  }
  return p;
}

// Paged caches: (block_table, max_pages, page_shift, num_pages), with
// T_cap = max_pages << page_shift; block_table == nullptr otherwise.
struct PagedArgs {
  const int32_t* block_table;
  int max_pages, page_shift, num_pages;
};

// Shared body of the GQA entry points.
// L query tokens per sequence plan as H_q * L query heads (the (head,
// token) columns of a KV head) whose visible range is widened by L - 1
// positions for the earlier tokens' windows.
int decode_gqa(const void* q, const void* k, const void* v, float* out,
               float* lse_out, const int32_t* seq_lens, const int32_t* ring_head,
               const int32_t* gpos, int n_global, PagedArgs pg, int B, int L,
               int H_q, int H_kv, int T_cap, int d, int dtype, int window,
               float scale, int num_splits, void* workspace,
               size_t workspace_bytes, void* stream, bool use_scratch = false) {
  const int ring = ring_head != nullptr;
  if (L < 1 || L > ATTN_MAX_QLEN) return ATTN_ERR_ARG;
  if (L > 1 && n_global > 0) return ATTN_ERR_UNSUPPORTED;
  if (H_q > 0 && (long long)H_q * L > (1 << 30)) return ATTN_ERR_SHAPE;
  if (window < 0) return ATTN_ERR_WINDOW;
  const int wrange = window > 0 ? window + L - 1 : 0;
  GqaPlan p;
  int st = plan_gqa(B, H_q * L, H_kv, T_cap, d, dtype, wrange, ring, n_global,
                    num_splits, &p);
  if (st != ATTN_OK) return st;
  if (B == 0) return ATTN_OK;  // empty batch: nothing to read or write
  if (!q || !k || !v || !out) return ATTN_ERR_NULL;
  if (n_global > 0 && !gpos) return ATTN_ERR_NULL;
  if (gpos && !aligned(gpos, 4)) return ATTN_ERR_ALIGN;
  if (isinf(scale)) return ATTN_ERR_ARG;
  if (!(scale > 0.f)) scale = 1.0f / sqrtf((float)d);
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(out, 4) ||
      (lse_out && !aligned(lse_out, 4)) || (seq_lens && !aligned(seq_lens, 4)) ||
      (ring_head && !aligned(ring_head, 4)))
    return ATTN_ERR_ALIGN;
  if (use_scratch) {
    // the device array stands in for the workspace (after every host check,
    // since finding its address is a HIP call): the fixed splits must fit in
    // it, the balanced list is taken when it fits too
    if (p.S > 1 && p.ws_fixed > (size_t)ATTN_NOALLOC_SCRATCH_BYTES)
      return ATTN_ERR_WORKSPACE;
    workspace = nullptr;
    workspace_bytes = 0;
    if (p.S > 1) {
      workspace = scratch_addr(&st);
      if (!workspace) return st;
      workspace_bytes = ATTN_NOALLOC_SCRATCH_BYTES;
    }
  }
  // balanced work list: lengths given, out 16-byte aligned (the merge writes
  // whole vectors) and room for its parts; else the fixed splits
  const bool bal = p.cap > 0 && seq_lens && aligned(out, 16) && workspace &&
                   aligned(workspace, 16) &&
                   workspace_bytes >= balanced_bytes(p, d, B);
  if (p.S > 1 && !bal) {
    if (!workspace || workspace_bytes < p.ws_fixed) return ATTN_ERR_WORKSPACE;
    if (!aligned(workspace, 16)) return ATTN_ERR_ALIGN;
  }

  GqaArgs a;
  a.q = q;
  a.k = k;
  a.v = v;
  a.out = out;
  a.lse = lse_out;
  a.seq_lens = seq_lens;
  a.ring_head = ring_head;
  a.gpos = n_global > 0 ? gpos : nullptr;
  a.n_global = n_global;
  a.block_table = pg.block_table;
  a.max_pages = pg.max_pages;
  a.page_shift = pg.page_shift;
  a.num_pages = pg.num_pages;
  a.B = B;
  a.H_q = H_q;
  a.H_kv = H_kv;
  a.T_cap = T_cap;
  a.window = wrange;
  a.L = L;
  a.wtok = window;
  a.n = H_q / H_kv;
  a.ncol = a.n * L;
  a.head_chunks = p.head_chunks;
  a.S = p.S;
  a.chunk = p.chunk;
  a.scale_log2 = scale * 1.4426950408889634f;
  a.o_part = nullptr;
  a.lse_part = nullptr;
  a.balanced = bal ? (p.even ? 2 : 1) : 0;
  a.cap = bal ? p.cap : 0;
  a.even_lead = even_lead(d);
  a.meta = nullptr;
  if (bal) {
    const size_t rows = list_slots(p, B) * p.N;
    a.o_part = (float*)workspace;
    a.lse_part = (float*)((char*)workspace + round_up(rows * d * sizeof(float), 256));
    a.meta = (int*)((char*)a.lse_part + round_up(rows * sizeof(float), 256));
  } else if (p.S > 1) {
    const size_t rows = (size_t)B * L * H_q * p.S;
    a.o_part = (float*)workspace;
    a.lse_part = (float*)((char*)workspace + round_up(rows * d * sizeof(float), 256));
  }
  const long long grid = bal ? p.cap : (long long)B * H_kv * p.head_chunks * p.S;
  if (grid > 0x7fffffffLL) return ATTN_ERR_SHAPE;
  a.xcd_remap = (p.head_chunks > 1 && grid % kNumXCDs == 0) ? 1 : 0;
  hipStream_t s = (hipStream_t)stream;
  const hipError_t e = p.mfma ? launch_gqa_mfma(a, d, p.N, (int)grid, s)
                              : launch_gqa_valu(a, dtype, d, (int)grid, s);
  if (e != hipSuccess) return ATTN_ERR_HIP;
  if (bal) {
    if (launch_combine_balanced(a.o_part, false, a.lse_part, a.meta, out, lse_out, B, L,
                                H_q, a.n, p.head_chunks, p.N, d, p.even != 0,
                                s) != hipSuccess)
      return ATTN_ERR_HIP;
  } else if (p.S > 1) {
    if (launch_combine(a.o_part, a.lse_part, out, lse_out, B * L, H_q, p.S, d, s) !=
        hipSuccess)
      return ATTN_ERR_HIP;
  }
  return ATTN_OK;
}

}  // namespace
}  // namespace attn

extern "C" {

int attn_decode_gqa(const void* q, const void* k, const void* v, float* out,
                    float* lse_out, const int32_t* seq_lens,
                    const int32_t* ring_head, int B, int H_q, int H_kv,
                    int T_cap, int d, int dtype, int window, float scale,
                    int num_splits, void* workspace, size_t workspace_bytes,
                    void* stream) {
  return decode_gqa(q, k, v, out, lse_out, seq_lens, ring_head, nullptr, 0,
                    PagedArgs{nullptr, 0, 0, 0}, B, 1, H_q, H_kv, T_cap, d, dtype,
                    window, scale, num_splits, workspace, workspace_bytes, stream);
}

int attn_decode_gqa_noalloc(const void* q, const void* k, const void* v, float* out,
                            float* lse_out, const int32_t* seq_lens,
                            const int32_t* ring_head, int B, int H_q, int H_kv,
                            int T_cap, int d, int dtype, int window, float scale,
                            int num_splits, void* stream) {
  return decode_gqa(q, k, v, out, lse_out, seq_lens, ring_head, nullptr, 0,
                    PagedArgs{nullptr, 0, 0, 0}, B, 1, H_q, H_kv, T_cap, d, dtype,
                    window, scale, num_splits, nullptr, 0, stream, true);
}

int attn_decode_gqa_multi(const void* q, const void* k, const void* v,
                          float* out, float* lse_out, const int32_t* seq_lens,
                          const int32_t* ring_head, int B, int q_len, int H_q,
                          int H_kv, int T_cap, int d, int dtype, int window,
                          float scale, int num_splits, void* workspace,
                          size_t workspace_bytes, void* stream) {
  return decode_gqa(q, k, v, out, lse_out, seq_lens, ring_head, nullptr, 0,
                    PagedArgs{nullptr, 0, 0, 0}, B, q_len, H_q, H_kv, T_cap, d,
                    dtype, window, scale, num_splits, workspace, workspace_bytes,
                    stream);
}

int attn_decode_gqa_global(const void* q, const void* k, const void* v,
                           float* out, float* lse_out, const int32_t* seq_lens,
                           const int32_t* global_pos, int n_global, int B,
                           int H_q, int H_kv, int T_cap, int d, int dtype,
                           int window, float scale, int num_splits,
                           void* workspace, size_t workspace_bytes,
                           void* stream) {
  return decode_gqa(q, k, v, out, lse_out, seq_lens, nullptr, global_pos,
                    n_global, PagedArgs{nullptr, 0, 0, 0}, B, 1, H_q, H_kv, T_cap,
                    d, dtype, window, scale, num_splits, workspace, workspace_bytes,
                    stream);
}

int attn_decode_gqa_paged(const void* q, const void* k_pages,
                          const void* v_pages, float* out, float* lse_out,
                          const int32_t* seq_lens, const int32_t* block_table,
                          int max_pages, int B, int q_len, int H_q, int H_kv,
                          int num_pages, int page_size, int d, int dtype,
                          int window, float scale, int num_splits,
                          void* workspace, size_t workspace_bytes, void* stream) {
  int shift = 0;
  const int st = attn_check_pages(max_pages, num_pages, page_size, H_kv, &shift);
  if (st != ATTN_OK) return st;
  if (B > 0 && !block_table) return ATTN_ERR_NULL;
  if (block_table && !aligned(block_table, 4)) return ATTN_ERR_ALIGN;
  return decode_gqa(q, k_pages, v_pages, out, lse_out, seq_lens, nullptr, nullptr,
                    0, PagedArgs{block_table, max_pages, shift, num_pages}, B, q_len,
                    H_q, H_kv, max_pages * page_size, d, dtype, window, scale,
                    num_splits, workspace, workspace_bytes, stream);
}


int attn_combine(const float* o_part, const float* lse_part, float* out,
                 float* lse_out, int B, int H, int S, int d_v, void* stream) {
  if (B < 0 || H <= 0 || d_v <= 0 || d_v > 4096) return ATTN_ERR_SHAPE;
  if (S < 1 || S > ATTN_MAX_SPLITS) return ATTN_ERR_ARG;
  if ((long long)B * H > 0x7fffffffLL) return ATTN_ERR_SHAPE;
  if (B == 0) return ATTN_OK;
  if (!o_part || !lse_part || !out) return ATTN_ERR_NULL;
  if (!aligned(o_part, 4) || !aligned(lse_part, 4) || !aligned(out, 4) ||
      (lse_out && !aligned(lse_out, 4)))
    return ATTN_ERR_ALIGN;
  if (launch_combine(o_part, lse_part, out, lse_out, B, H, S, d_v,
                     (hipStream_t)stream) != hipSuccess)
    return ATTN_ERR_HIP;
  return ATTN_OK;
}

const char* attn_status_string(int status) {
  switch (status) {
    case ATTN_OK: return "ok";
    case ATTN_ERR_NULL: return "a required pointer is NULL";
    case ATTN_ERR_SHAPE: return "invalid shape";
    case ATTN_ERR_DTYPE: return "unknown dtype";
    case ATTN_ERR_UNSUPPORTED: return "unsupported head dimension or widths";
    case ATTN_ERR_WINDOW: return "invalid window";
    case ATTN_ERR_WORKSPACE: return "workspace missing or too small";
    case ATTN_ERR_ALIGN: return "misaligned pointer";
    case ATTN_ERR_HIP: return "HIP launch error";
    case ATTN_ERR_ARG: return "invalid scalar argument";
  }
  return "unknown status";
}

}  // extern "C"
