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
  int len;      // seq_lens[b] as stored
  int head;     // ring_head[b] as stored (ring mode), else 0
  int r;        // item of the sequence, 0 .. U*k - 1
  int k;        // pieces per unit of this sequence
  int chunk;    // rows per piece (C)
  int first;    // list number of the sequence's first item (P_b * U)
  bool valid;   // false: the list has fewer than w + 1 items
};

// Sum and maximum over the 64 lanes, every lane receiving the result: DPP
// moves inside rows of 16 lanes, then the permlane swaps across rows (the
// pattern of group_sum, on integers).
ATTN_DEV int lane_xor16_i(int x) {
  const unsigned u = (unsigned)x;
  const auto p = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  return (int)((__lane_id() & 16) ? p[0] : p[1]);
}
ATTN_DEV int lane_xor32_i(int x) {
  const unsigned u = (unsigned)x;
  const auto p = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return (int)((__lane_id() & 32) ? p[0] : p[1]);
}
template <int CTRL>
ATTN_DEV int dpp_i(int x) {
  return __builtin_amdgcn_mov_dpp(x, CTRL, 0xF, 0xF, true);
}
ATTN_DEV int wave_sum_i(int x) {
  x += dpp_i<kDppQuadXor1>(x);
  x += dpp_i<kDppQuadXor2>(x);
  x += dpp_i<kDppHalfMirror>(x);
  x += dpp_i<kDppRowMirror>(x);
  x += lane_xor16_i(x);
  return x + lane_xor32_i(x);
}
ATTN_DEV int wave_max_i(int x) {
  x = max(x, dpp_i<kDppQuadXor1>(x));
  x = max(x, dpp_i<kDppQuadXor2>(x));
  x = max(x, dpp_i<kDppHalfMirror>(x));
  x = max(x, dpp_i<kDppRowMirror>(x));
  x = max(x, lane_xor16_i(x));
  return max(x, lane_xor32_i(x));
}

// Inclusive prefix sum over the lanes of the wave: shifts inside each row of
// 16 lanes (out-of-row sources read 0), then the totals of the rows before.
template <int CTRL>
ATTN_DEV int dpp_shr_i(int x) {
  return __builtin_amdgcn_update_dpp(0, x, CTRL, 0xF, 0xF, true);
}
ATTN_DEV int wave_incl_scan_i(int x) {
  x += dpp_shr_i<0x111>(x);  // row_shr:1
  x += dpp_shr_i<0x112>(x);  // row_shr:2
  x += dpp_shr_i<0x114>(x);  // row_shr:4
  x += dpp_shr_i<0x118>(x);  // row_shr:8
  const int r0 = __builtin_amdgcn_readlane(x, 15);
  const int r1 = __builtin_amdgcn_readlane(x, 31);
  const int r2 = __builtin_amdgcn_readlane(x, 47);
  const int row = __lane_id() >> 4;
  return x + (row == 0 ? 0 : row == 1 ? r0 : row == 2 ? r0 + r1 : r0 + r1 + r2);
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
  // visible rows of each held sequence, in tiles (-1: no sequence); the
  // stored length and ring head stay in the lane, so the item's sequence
  // needs no second load
  int nt[kPer], len[kPer], head[kPer];
  int sum_t = 0, max_t = 0;
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const int b = 64 * i + lane;
    nt[i] = -1;
    len[i] = 0;
    head[i] = 0;
    if (i < rounds && b < B) {
      len[i] = seq_lens[b];
      head[i] = ring_head ? ring_head[b] : 0;
      const int n = visible_range_of(len[i], ring_head != nullptr, head[i], T_cap,
                                     window, gpos, n_global).n;
      nt[i] = (int)(((unsigned)n + tile - 1) / (unsigned)tile);
      sum_t += nt[i];
      max_t = max(max_t, nt[i]);
    }
  }
  // sums as unsigned: at most 256 sequences of 2^23 tiles (2^30 rows) each,
  // plus one piece per sequence, stay below 2^32
  const unsigned sum_all = (unsigned)wave_sum_i(sum_t);
  max_t = wave_max_i(max_t);
  const unsigned slots = (unsigned)(cap / U);  // pieces the list may hold per unit

  // pieces per unit of every sequence at C = m tiles; ceil(n / (m * tile))
  // equals ceil(ceil(n / tile) / m)
  auto count = [&](int m) {
    int c = 0;
#pragma unroll
    for (int i = 0; i < kPer; ++i)
      if (nt[i] >= 0) c += nt[i] <= m ? 1 : (nt[i] + m - 1) / m;
    return (unsigned)wave_sum_i(c);
  };
  // Bounds of the search: the list needs at least sum_all / m pieces, and
  // ceil(x / m) <= x / m + 1 bounds it by sum_all / m + B, so m =
  // ceil(sum_all / (slots - B)) fits whenever slots > B; one piece per
  // sequence (m = max_t) always fits.
  int lo = max((c_min + tile - 1) / tile, (int)((sum_all + slots - 1) / slots));
  lo = max(lo, 1);
  int hi = max(max_t, 1);
  if (slots > (unsigned)B) {
    const unsigned room = slots - (unsigned)B;
    hi = min(hi, (int)((sum_all + room - 1) / room));
  }
  hi = max(hi, lo);
  if (count(lo) <= slots) hi = lo;  // the common case: the lower bound fits
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
  it.len = 0;
  it.head = 0;
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
        it.first = __builtin_amdgcn_readlane((int)p0, src);
        it.k = __builtin_amdgcn_readlane(k, src);
        it.len = __builtin_amdgcn_readlane(len[i], src);
        it.head = __builtin_amdgcn_readlane(head[i], src);
      }
      base += __builtin_amdgcn_readlane(incl, 63);
    }
  }
  it.r = it.valid ? w - it.first : 0;
  return it;
}

// Even split (balanced == 2: the matrix-core GQA kernel at d <= 128, and the
// MLA kernel's 512 + 64 geometry for one query token).  The
// units' tiles are laid end to end -- sequence after sequence, the U units
// of a sequence one after another, each unit max(1, ceil(n_b / tile))
// tiles preceded by `lead` tiles that stand for the fixed cost of starting a
// unit (loading its queries, refilling the load pipeline, merging the
// waves) -- and that line is cut into `groups` ranges whose lengths differ
// by at most one tile, so every work group gets about the same time of work:
// a group that starts many short units gets fewer rows.  A range may end
// inside a unit and carry on into the next ones: its group computes one
// segment per unit whose rows it holds (a range that holds only part of a
// unit's lead tiles computes nothing for it).  Segment (unit ui, group w)
// keeps its partial result in slot w + ui.  Two segments never share a
// slot: w + ui = w' + ui' with w < w' needs ui > ui', but a later group
// never starts in an earlier unit.  A unit's slots are consecutive (its
// groups are), and the list needs at most groups + B*U of them.  Every wave
// derives the plan from seq_lens on its own, like balanced_item.
struct EvenPlan {
  int et[kBalanceMaxB / 64];   // tiles per unit of sequence 64 i + lane (-1: none)
  int pre[kBalanceMaxB / 64];  // line position of that sequence's first unit
  int len[kBalanceMaxB / 64];  // its stored length
  int rounds;                  // 64-sequence rounds held
  int lead;                    // lead tiles per unit
  int total;                   // line length (>= 1)
  int groups;                  // ranges, 1 .. cap
};

// Plan for B <= kBalanceMaxB sequences of U units; at least min_tiles line
// positions per range (fewer ranges than cap when the work is small).  The
// caller guarantees that B * U * (T_cap / tile + 1 + lead) fits an int.
ATTN_DEV EvenPlan even_plan(const int32_t* seq_lens, int B, int T_cap, int window,
                            const int32_t* gpos, int n_global, int U, int cap,
                            int tile, int lead, int min_tiles) {
  constexpr int kPer = kBalanceMaxB / 64;
  const int lane = __lane_id();
  EvenPlan p;
  p.rounds = (B + 63) >> 6;
  p.lead = lead;
  int base = 0;
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const int b = 64 * i + lane;
    p.et[i] = -1;
    p.len[i] = 0;
    p.pre[i] = 0;
    if (i < p.rounds) {  // uniform
      int e = 0;
      if (b < B) {
        p.len[i] = seq_lens[b];
        const int n = visible_range_of(p.len[i], false, 0, T_cap, window, gpos,
                                       n_global).n;
        e = max(1, (n + tile - 1) / tile);
        p.et[i] = e;
      }
      const int w = b < B ? (e + lead) * U : 0;
      const int incl = wave_incl_scan_i(w);
      p.pre[i] = base + incl - w;
      base += __builtin_amdgcn_readlane(incl, 63);
    }
  }
  p.total = base;
  p.groups = max(1, min(cap, base / max(1, min_tiles)));
  return p;
}

// Line position where range w starts (w = groups gives the end of the line).
ATTN_DEV int even_start(const EvenPlan& p, int w) {
  return (int)((long long)w * p.total / p.groups);
}

struct EvenSeg {
  int b, len;      // sequence and its stored length
  int u;           // unit of the sequence
  int t0, t1;      // the unit's tiles [t0, t1) in this range (t0 == t1: none)
  int next;        // line position after this segment
  int first, last; // the ranges holding the unit's first and last tiles
};

// The segment of sequence b (its first unit at line position pre, et tiles
// per unit) that starts at line position x, inside a range ending at x1.
ATTN_DEV EvenSeg even_cut(int groups, int total, int lead, int b, int len, int pre,
                          int et, int x, int x1);

// The segment that starts at line position x, inside a range ending at x1.
ATTN_DEV EvenSeg even_segment(const EvenPlan& p, int x, int x1) {
  constexpr int kPer = kBalanceMaxB / 64;
  int b = 0, len = 0, pre = 0, et = 1;
  // the starts grow with b, so the sequences starting at or before x are a
  // prefix: the last one holds x
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    if (i < p.rounds) {
      const unsigned long long bal = __ballot(p.et[i] >= 0 && p.pre[i] <= x);
      if (bal) {
        const int src = 63 - __clzll((long long)bal);
        b = 64 * i + src;
        pre = __builtin_amdgcn_readlane(p.pre[i], src);
        et = __builtin_amdgcn_readlane(p.et[i], src);
        len = __builtin_amdgcn_readlane(p.len[i], src);
      }
    }
  }
  return even_cut(p.groups, p.total, p.lead, b, len, pre, et, x, x1);
}

// The same plan with its per-sequence arrays in LDS, for kernels whose
// registers are taken: 3 * kBalanceMaxB ints (tiles per unit, first line
// position, stored length).  Every wave writes the same values and reads back
// only what it wrote itself, so no barrier is needed.
struct EvenPlanLds {
  const int* lds;
  int rounds, lead, total, groups;
};

ATTN_DEV EvenPlanLds even_plan_lds(const int32_t* seq_lens, int B, int T_cap, int window,
                                   const int32_t* gpos, int n_global, int U, int cap,
                                   int tile, int lead, int min_tiles, int* lds) {
  constexpr int kPer = kBalanceMaxB / 64;
  const EvenPlan p = even_plan(seq_lens, B, T_cap, window, gpos, n_global, U, cap, tile,
                               lead, min_tiles);
  const int lane = __lane_id();
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    if (i < p.rounds) {
      lds[64 * i + lane] = p.et[i];
      lds[kBalanceMaxB + 64 * i + lane] = p.pre[i];
      lds[2 * kBalanceMaxB + 64 * i + lane] = p.len[i];
    }
  }
  return EvenPlanLds{lds, p.rounds, p.lead, p.total, p.groups};
}

ATTN_DEV int even_start(const EvenPlanLds& p, int w) {
  return (int)((long long)w * p.total / p.groups);
}

ATTN_DEV EvenSeg even_segment(const EvenPlanLds& p, int x, int x1) {
  constexpr int kPer = kBalanceMaxB / 64;
  const int lane = __lane_id();
  int b = 0, len = 0, pre = 0, et = 1;
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    if (i < p.rounds) {
      const int e = p.lds[64 * i + lane];
      const int pr = p.lds[kBalanceMaxB + 64 * i + lane];
      const unsigned long long bal = __ballot(e >= 0 && pr <= x);
      if (bal) {
        const int src = 63 - __clzll((long long)bal);
        b = 64 * i + src;
        pre = __builtin_amdgcn_readlane(pr, src);
        et = __builtin_amdgcn_readlane(e, src);
        len = __builtin_amdgcn_readlane(p.lds[2 * kBalanceMaxB + 64 * i + lane], src);
      }
    }
  }
  return even_cut(p.groups, p.total, p.lead, b, len, pre, et, x, x1);
}

ATTN_DEV EvenSeg even_cut(int groups, int total, int lead, int b, int len, int pre,
                          int et, int x, int x1) {
  // the range holding line position y: the largest w with start(w) <= y
  auto group_of = [&](int y) { return (int)(((long long)(y + 1) * groups - 1) / total); };
  EvenSeg sg;
  sg.b = b;
  sg.len = len;
  const int span = et + lead;  // line positions per unit
  const int off = x - pre;
  sg.u = off / span;
  const int ustart = pre + sg.u * span;  // the unit's lead tiles start here
  const int rstart = ustart + lead;      // its tiles start here
  const int uend = ustart + span;
  sg.next = min(x1, uend);
  sg.t0 = max(x, rstart) - rstart;
  sg.t1 = max(sg.next, rstart) - rstart;
  sg.first = group_of(rstart);
  sg.last = group_of(uend - 1);
  return sg;
}

}  // namespace attn
