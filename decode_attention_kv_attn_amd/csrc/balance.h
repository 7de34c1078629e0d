// Work assignment by visible rows, for batches whose sequences differ in
// length.
//
// A call's work is a list of items.  Each sequence has U units (its KV heads
// times the head chunks of each; they share the sequence's visible range),
// and each unit's n_b visible rows are cut into k_b = ceil(n_b / C) pieces of
// C rows (at least one piece, also for n_b = 0).  C is the smallest multiple
// of `tile` rows, at least c_min, for which the list fits in `cap` items, so
// one round of work groups covers it and its longest piece is as short as
// that round allows.  Sequence b owns items P_b*U .. (P_b + k_b)*U - 1, with
// P_b the sum of k over the sequences before it.  (Cutting a query's keys into
// disjoint pieces and merging the pieces' softmax results by their
// log-sum-exp is exact: softmax over a union of disjoint key sets,
// xuesongtap "attention-head" note, section 1.)
//
// The lengths live in device memory and the host never reads them, so the
// list is derived on the device: every wave of every work group computes it
// from seq_lens on its own (lane j holds sequences j, j + 64, ...), which
// needs neither LDS nor a barrier, then reads off the item it was given.

#pragma once

#include "device_common.h"
#include "internal.h"
#include "visible.h"

namespace attn {

struct WorkItem {
  int b;        // sequence
  int r;        // item of the sequence, 0 .. U*k - 1
  int k;        // pieces per unit of this sequence
  int chunk;    // rows per piece (C)
  int first;    // list number of the sequence's first item (P_b * U)
  bool valid;   // false: the list has fewer than w + 1 items
};

ATTN_DEV int wave_sum_i(int x) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) x += __shfl_xor(x, off);
  return x;
}

ATTN_DEV int wave_max_i(int x) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) x = max(x, __shfl_xor(x, off));
  return x;
}

// Inclusive prefix sum over the lanes of the wave.
ATTN_DEV int wave_incl_scan_i(int x) {
  const int lane = __lane_id();
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int y = __shfl_up(x, off);
    if (lane >= off) x += y;
  }
  return x;
}

// Item w of the list.  B <= kBalanceMaxB sequences, U units each, with
// U * B <= cap; `tile` and c_min in rows.  ring_head / gpos as for
// visible_range (nullptr when unused).  Uniform across the wave.
ATTN_DEV WorkItem balanced_item(const int32_t* seq_lens, const int32_t* ring_head,
                                int B, int T_cap, int window, const int32_t* gpos,
                                int n_global, int U, int cap, int tile, int c_min,
                                int w) {
  constexpr int kPer = kBalanceMaxB / 64;
  const int lane = __lane_id();
  const int rounds = (B + 63) >> 6;
  // visible rows of each held sequence, in tiles (-1: no sequence)
  int nt[kPer];
  int sum_t = 0, max_t = 0;
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const int b = 64 * i + lane;
    nt[i] = -1;
    if (i < rounds && b < B) {
      const int n =
          visible_range(seq_lens, ring_head, b, T_cap, window, gpos, n_global).n;
      nt[i] = (n + tile - 1) / tile;
      sum_t += nt[i];
      max_t = max(max_t, nt[i]);
    }
  }
  sum_t = wave_sum_i(sum_t);
  max_t = wave_max_i(max_t);
  const int slots = cap / U;  // pieces the list may hold per unit

  // pieces per unit of every sequence at C = m tiles; ceil(n / (m * tile))
  // equals ceil(ceil(n / tile) / m)
  auto count = [&](int m) {
    int c = 0;
#pragma unroll
    for (int i = 0; i < kPer; ++i)
      if (nt[i] >= 0) c += nt[i] <= m ? 1 : (nt[i] + m - 1) / m;
    return wave_sum_i(c);
  };
  // Bounds of the search: the list needs at least sum_t / m pieces, and
  // ceil(x / m) <= x / m + 1 bounds it by sum_t / m + B, so m =
  // ceil(sum_t / (slots - B)) fits whenever slots > B; one piece per
  // sequence (m = max_t) always fits.
  int lo = max((c_min + tile - 1) / tile,
               (int)(((long long)sum_t + slots - 1) / slots));
  lo = max(lo, 1);
  int hi = max(max_t, 1);
  if (slots > B) hi = min(hi, (sum_t + (slots - B) - 1) / (slots - B));
  hi = max(hi, lo);
  while (lo < hi) {  // smallest m in [lo, hi] whose list fits
    const int mid = (lo + hi) >> 1;
    if (count(mid) <= slots) hi = mid;
    else lo = mid + 1;
  }
  const int m = lo;

  // prefix of k over the sequences, round by round; the lane whose sequence
  // holds item w describes it
  WorkItem it;
  it.chunk = m * tile;
  it.valid = false;
  it.b = 0;
  it.first = 0;
  it.k = 1;
  int base = 0;
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    if (i < rounds) {
      const int k = nt[i] < 0 ? 0 : (nt[i] <= m ? 1 : (nt[i] + m - 1) / m);
      const int incl = wave_incl_scan_i(k);
      const long long p0 = (long long)(base + incl - k) * U;
      const bool mine = k > 0 && w >= p0 && w < p0 + (long long)k * U;
      const unsigned long long bal = __ballot(mine);
      if (bal) {
        const int src = __ffsll((long long)bal) - 1;
        it.valid = true;
        it.b = 64 * i + src;
        it.first = __shfl((int)p0, src);
        it.k = __shfl(k, src);
      }
      base += __shfl(incl, 63);
    }
  }
  it.r = it.valid ? w - it.first : 0;
  return it;
}

}  // namespace attn
