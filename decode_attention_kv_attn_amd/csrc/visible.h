// Visible set and row addressing of a decode query (the tile skipper).
//
// The query of sequence b sits at logical position t = T_b - 1 and sees
//   * the contiguous range [lo, T_b), where
//       lo = T_b - w          with a window of width w > 0 (positions
//                              t-w+1 .. t; xuesongtap "attention-head" note,
//                              section 3, worked example w=3: row 8 sees
//                              6, 7, 8),
//       lo >= T_b - S_cap     in ring mode, where only the newest S_cap
//                              positions are resident (same section: a pure
//                              sliding-window layer may reuse slots as a ring),
//       lo = 0                otherwise;
//   * plus, in a linear cache with global positions G (sorted, unique), every
//     g in G with g < lo; a query that is itself in G sees all of [0, T_b)
//     (same section, the window-plus-global pattern with G = {0, 5}).
//
// Kernels walk a dense virtual index vi in [0, n): vi < n_extra are the
// global positions before the window (G[vi]), the rest is lo + (vi - n_extra).
// A work item owns a sub-range of [0, n) and loads only rows inside it, so
// masked rows -- beyond a ragged end, outside the window, overwritten in the
// ring -- are never read.
//
// Ring addressing: position j lives in slot (head - (t - j)) mod S_cap, where
// head is the slot of the newest position.  For a resident j, 0 <= t-j <
// S_cap, so one conditional add replaces the modulo.
//
// Paged addressing (the KV-cache paging the baidu article, section 四.3,
// names as the system side of GQA and MLA): the cache is a pool of pages of
// P = 2^shift positions, [num_pages, H_kv, P, d] (one page holds every KV
// head's rows of its positions, each head's P rows contiguous); position j
// of sequence b lives in page table[b][j >> shift], row j & (P - 1).
#pragma once

#include "device_common.h"

namespace attn {

// Entries of the ascending list g[0..n) that are below x (binary search).
ATTN_DEV int count_below(const int32_t* g, int n, int x) {
  int a = 0, b = n;
  while (a < b) {
    const int mid = (a + b) >> 1;
    if (g[mid] < x) a = mid + 1; else b = mid;
  }
  return a;
}

struct VisibleRange {
  int lo;       // first windowed position
  int hi;       // one past the last visible position (== T_b)
  int t;        // query position
  int head;     // ring: slot of position t; linear: unused
  int n_extra;  // global positions before lo (virtual rows 0 .. n_extra-1)
  int n;        // visible rows
  const int32_t* gpos;  // global positions (valid when n_extra > 0)
};

// The range of a query whose cache holds T_b positions (as stored in
// seq_lens; clamped here) with ring write pointer head (ring mode only, any
// int: reduced mod T_cap).
ATTN_DEV VisibleRange visible_range_of(int T_b, bool ring, int head, int T_cap,
                                       int window, const int32_t* gpos = nullptr,
                                       int n_global = 0) {
  if (T_b < 0) T_b = 0;
  if (!ring && T_b > T_cap) T_b = T_cap;
  int lo = 0;
  if (window > 0) lo = max(lo, T_b - window);
  if (ring) lo = max(lo, T_b - T_cap);
  int n_extra = 0;
  if (n_global > 0 && T_b > 0 && lo > 0) {
    // G is sorted: n_extra = #{g < lo}; the query is global iff t is in G.
    n_extra = count_below(gpos, n_global, lo);
    const int k = count_below(gpos, n_global, T_b - 1);
    if (k < n_global && gpos[k] == T_b - 1) {
      lo = 0;
      n_extra = 0;
    }
  }
  VisibleRange r;
  r.lo = lo;
  r.hi = T_b;
  r.t = T_b - 1;
  r.head = 0;
  r.n_extra = n_extra;
  r.n = n_extra + (T_b - lo);
  r.gpos = gpos;
  if (ring) {
    const int h = head % T_cap;
    r.head = h < 0 ? h + T_cap : h;
  }
  return r;
}

ATTN_DEV VisibleRange visible_range(const int32_t* seq_lens,
                                    const int32_t* ring_head, int b, int T_cap,
                                    int window, const int32_t* gpos = nullptr,
                                    int n_global = 0) {
  return visible_range_of(seq_lens ? seq_lens[b] : T_cap, ring_head != nullptr,
                          ring_head ? ring_head[b] : 0, T_cap, window, gpos, n_global);
}

// A single query that sees the whole ring (every slot resident and inside
// its window) weighs all rows alike, so the visiting order is free: with the
// head taken as slot T_cap - 1, virtual row vi is slot vi, and the pieces of
// every sequence cover the same slot ranges whatever its write pointer
// (measured about 7% faster on a full 4096-slot ring than starting each
// sequence at its own oldest slot).  Only for one query token: several
// tokens derive positions from virtual rows.
ATTN_DEV void ring_slot_order(VisibleRange& r, bool ring, int L, int T_cap) {
  if (ring && L == 1 && r.n == T_cap) r.head = T_cap - 1;
}

// Logical position of virtual row vi (0 <= vi < n).  Global positions are
// clamped into the cache so a malformed list cannot address outside it.
ATTN_DEV int row_position(const VisibleRange& r, int vi, int T_cap) {
  if (vi < r.n_extra) {
    const int g = r.gpos[vi];
    return g < 0 ? 0 : (g >= T_cap ? T_cap - 1 : g);
  }
  return r.lo + (vi - r.n_extra);
}

// Cache row of a visible position.  `ring` is uniform across the work item.
ATTN_DEV int slot_of(const VisibleRange& r, bool ring, int pos, int T_cap) {
  if (!ring) return pos;
  const int s = r.head - (r.t - pos);
  return s < 0 ? s + T_cap : s;
}

// Cache row of virtual row vi.  When the whole tile [base, base + rows) lies
// past the global rows (the common case; `tile_fast`, uniform), the position
// is a plain offset.
ATTN_DEV int row_slot(const VisibleRange& r, bool ring, bool tile_fast, int vi,
                      int T_cap) {
  const int pos = tile_fast ? r.lo + (vi - r.n_extra) : row_position(r, vi, T_cap);
  return slot_of(r, ring, pos, T_cap);
}

// Virtual sub-range of split s when [0, n) is cut into pieces of `chunk`
// rows.  The last split also takes any rows past S*chunk (a query that is
// itself global sees more rows than the planner's bound).
ATTN_DEV void split_range(const VisibleRange& r, int s, int S, int chunk,
                          int& p0, int& p1) {
  const long long a = (long long)s * chunk;
  p0 = a < r.n ? (int)a : r.n;
  const long long e = (s == S - 1) ? (long long)r.n : a + chunk;
  p1 = e < r.n ? (int)e : r.n;
}

// Several query tokens per sequence (L >= 1, the last L positions of the
// cache): column c (0 <= c < n*L) of KV head g stands for query head
// g*n + c / L of token c % L, which sits at position T_b - L + c % L and is
// stored at row (b*L + token)*H_q + head of q and of the outputs.
ATTN_DEV size_t query_row(int b, int g, int c, int n, int L, int H_q) {
  const int hq = c / L;
  const int tok = c - hq * L;
  return ((size_t)b * L + tok) * H_q + g * n + hq;
}

// Addressing modes, fixed per kernel instantiation so that the common case
// carries no per-row branches: a dense [B, H_kv, T_cap, d] cache (linear or
// ring), a linear cache with global positions, or a paged cache.
enum AddrMode : int { kAddrDense = 0, kAddrGlobal = 1, kAddrPaged = 2 };

// One sequence's view of a paged cache.
struct Pages {
  const int32_t* table;  // this sequence's block-table row
  int shift;             // log2 of the page size
  int last;              // last table entry the sequence uses (>= 0)
  int num_pages;         // pool size: page ids are clamped to [0, num_pages)
  int stride;            // rows from one page to the next for one head
};

ATTN_DEV Pages page_view(const int32_t* block_table, int max_pages, int b,
                         int T_b, int shift, int num_pages, int H_kv) {
  Pages p;
  p.table = block_table + (size_t)b * max_pages;
  p.shift = shift;
  const int last = T_b > 0 ? (T_b - 1) >> shift : 0;
  p.last = last < max_pages ? last : max_pages - 1;
  p.num_pages = num_pages;
  p.stride = H_kv << shift;
  return p;
}

// Ids of the three pages starting with the one that holds position pos0:
// every tile of at most 2P + 1 rows starting at pos0 lies inside them.
// Entries past the sequence's last page repeat that page; ids outside the
// pool are clamped, so a corrupt table cannot address outside it.
ATTN_DEV void tile_pages(const Pages& p, int pos0, int (&id)[3]) {
  const int j0 = pos0 >> p.shift;
#pragma unroll
  for (int k = 0; k < 3; ++k) {
    const int j = min(j0 + k, p.last);
    const int v = p.table[j];
    id[k] = v < 0 ? 0 : (v >= p.num_pages ? p.num_pages - 1 : v);
  }
}

// The same three table entries with one vector load: lane k < 3 gets entry
// k (the others repeat entry 2), unclamped.  The caller reads them with
// page_ids_from_lanes only when it issues the tile's loads, so the wait for
// this load lands there and not next to the load.
ATTN_DEV int tile_pages_lanes(const Pages& p, int pos0, int lane) {
  const int j = min((pos0 >> p.shift) + min(lane, 2), p.last);
  return p.table[j];
}

// Ids (clamped to the pool) from the lanes filled by tile_pages_lanes.
ATTN_DEV void page_ids_from_lanes(const Pages& p, int pv, int (&id)[3]) {
#pragma unroll
  for (int k = 0; k < 3; ++k) {
    const int v = __builtin_amdgcn_readlane(pv, k);
    id[k] = v < 0 ? 0 : (v >= p.num_pages ? p.num_pages - 1 : v);
  }
}

// Row (in units of one head's rows, from the head's base) of position pos
// of a tile that starts at pos0 <= pos.
ATTN_DEV int paged_row(const Pages& p, const int (&id)[3], int pos0, int pos) {
  const int k = (pos >> p.shift) - (pos0 >> p.shift);
  const int page = k == 0 ? id[0] : (k == 1 ? id[1] : id[2]);
  return page * p.stride + (pos & ((1 << p.shift) - 1));
}

}  // namespace attn
