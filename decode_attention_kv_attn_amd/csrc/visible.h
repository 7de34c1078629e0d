// Visible range and slot addressing of a decode query (the tile skipper).
//
// The query of sequence b sits at logical position t = T_b - 1.  It sees a
// contiguous position range [lo, hi):
//   hi = T_b;
//   lo = T_b - w          when a window of width w > 0 is set (positions
//                          t-w+1 .. t; xuesongtap "attention-head" note,
//                          section 3, worked example w=3: row 8 sees 6, 7, 8);
//   lo = T_b - S_cap      at least, in ring mode, where only the newest S_cap
//                          positions are resident (same section: a pure
//                          sliding-window layer may reuse slots as a ring);
//   lo = 0                otherwise.
// A work item owns a sub-range of [lo, hi) and loads only rows inside it, so
// masked rows -- beyond a ragged end, outside the window, overwritten in the
// ring -- are never read.
//
// Ring addressing: position j lives in slot (head - (t - j)) mod S_cap, where
// head is the slot of the newest position.  For a resident j, 0 <= t-j <
// S_cap, so one conditional add replaces the modulo.
#pragma once

#include "device_common.h"

namespace attn {

struct VisibleRange {
  int lo;    // first visible position
  int hi;    // one past the last visible position (== T_b)
  int t;     // query position
  int head;  // ring: slot of position t; linear: unused
};

ATTN_DEV VisibleRange visible_range(const int32_t* seq_lens,
                                    const int32_t* ring_head, int b, int T_cap,
                                    int window) {
  int T_b = seq_lens ? seq_lens[b] : T_cap;
  const bool ring = ring_head != nullptr;
  if (T_b < 0) T_b = 0;
  if (!ring && T_b > T_cap) T_b = T_cap;
  int lo = 0;
  if (window > 0) lo = max(lo, T_b - window);
  if (ring) lo = max(lo, T_b - T_cap);
  VisibleRange r;
  r.lo = lo;
  r.hi = T_b;
  r.t = T_b - 1;
  r.head = 0;
  if (ring) {
    int h = ring_head[b] % T_cap;
    r.head = h < 0 ? h + T_cap : h;
  }
  return r;
}

// Cache row of visible position `pos` (lo <= pos < hi).  `ring` is uniform
// across the work item.
ATTN_DEV int slot_of(const VisibleRange& r, bool ring, int pos, int T_cap) {
  if (!ring) return pos;
  const int s = r.head - (r.t - pos);
  return s < 0 ? s + T_cap : s;
}

// Sub-range of split `s` when the visible range is cut into pieces of
// `chunk` positions starting at lo.  Empty when s*chunk >= hi-lo.
ATTN_DEV void split_range(const VisibleRange& r, int s, int chunk, int& p0,
                          int& p1) {
  const long long a = (long long)r.lo + (long long)s * chunk;
  p0 = a < r.hi ? (int)a : r.hi;
  const long long e = a + chunk;
  p1 = e < r.hi ? (int)e : r.hi;
}

}  // namespace attn
