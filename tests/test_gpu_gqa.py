"""GPU parity of attn_decode_gqa / attn_combine against the float64 oracle.

Every case draws seeded inputs (synth), runs the HIP library through its C
ABI, and compares element by element with ``oracle.gqa_decode_ref`` on the
same values: max-abs <= 2e-3 and relative L2 <= 1e-3 for outputs, index logic
bit-exact through integer recovery.
"""

import math

import numpy as np
import pytest
import torch

import decode_attention_kv_attn_amd as L
import oracle
import synth
from oracle import bruteforce as BF
from helpers import (assert_lse, assert_lse_each, assert_parity,
                     assert_parity_each, map_units, to64)

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _case(B, H_q, H_kv, T_cap, d, dtype, seed, lens=None, heads=None,
          value_scale=1.0):
    q = synth.draw((B, H_q, d), seed, dtype, DEV, value_scale)
    k = synth.draw((B, H_kv, T_cap, d), seed + 1, dtype, DEV, value_scale)
    v = synth.draw((B, H_kv, T_cap, d), seed + 2, dtype, DEV, value_scale)
    sl = None if lens is None else torch.tensor(lens, dtype=torch.int32, device=DEV)
    rh = None if heads is None else torch.tensor(heads, dtype=torch.int32, device=DEV)
    return q, k, v, sl, rh


def _check(q, k, v, sl, rh, window=0, scale=None, num_splits=0, what=""):
    out, lse = L.attn_decode_gqa(q, k, v, sl, rh, window, scale, num_splits)
    torch.cuda.synchronize()
    ro, rl = oracle.gqa_decode_ref(q, k, v, sl, rh, window, scale)
    assert_parity(out, ro, what)
    assert_lse(lse, rl, what)
    return out, lse


def test_gqa_fp32_t512_workload():
    """B=1, 8 query heads over 2 KV heads, d=64, T=512, float32, no mask."""
    w = synth.workload("gqa_fp32_t512")
    inp = synth.gqa_inputs(w, DEV)
    _check(inp["q"], inp["k"], inp["v"], None, None, what="gqa_fp32_t512")


GRID = [(dt, d, n) for dt in ("bf16", "fp32") for d in (64, 128, 256)
        for n in (1, 2, 3, 4, 5, 6, 7, 8, 12, 32)]


@pytest.mark.parametrize("dtype,d,n", GRID,
                         ids=[f"{a}-d{b}-n{c}" for a, b, c in GRID])
def test_group_sizes(dtype, d, n):
    """Every head dim, element type and group size (1 = MHA, 32 = MQA-sized),
    two KV heads, ragged lengths with partial tiles."""
    T_cap = 300 if d < 256 else 200
    seed = 5000 + 37 * n + d + (0 if dtype == "bf16" else 1)
    q, k, v, sl, _ = _case(2, 2 * n, 2, T_cap, d, dtype, seed,
                           lens=[T_cap, 1 + (seed % (T_cap - 1))])
    _check(q, k, v, sl, None, what=f"{dtype} d={d} n={n}")


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_ragged_edges(dtype):
    """Lengths 0, 1, 2, a partial tile, T_cap-1 and T_cap in one batch."""
    T_cap = 257
    lens = [0, 1, 2, 33, T_cap - 1, T_cap]
    q, k, v, sl, _ = _case(len(lens), 8, 2, T_cap, 128, dtype, 6100, lens=lens)
    out, lse = _check(q, k, v, sl, None, what="ragged edges")
    assert torch.all(out[0] == 0) and torch.all(torch.isneginf(lse[0]))


@pytest.mark.parametrize("window", [1, 2, 31, 64, 257, 600, 10000])
def test_window_linear(window):
    T_cap = 600
    lens = [600, 599, 64, 1, 300]
    q, k, v, sl, _ = _case(len(lens), 12, 3, T_cap, 128, "bf16", 6200 + window,
                           lens=lens)
    _check(q, k, v, sl, None, window=window, what=f"window {window}")


@pytest.mark.parametrize("window", [0, 1, 64, 127, 128])
def test_ring(window):
    """Ring of 128 slots: lengths before, at and far past the wrap, heads at
    seeded offsets (lengths beyond the ring are logical)."""
    slots = 128
    lens = [0, 1, 50, 128, 129, 500, 1000, 77777]
    rng = np.random.default_rng(6300 + window)
    heads = rng.integers(0, slots, size=len(lens)).tolist()
    q, k, v, sl, rh = _case(len(lens), 8, 2, slots, 64, "bf16", 6300 + window,
                            lens=lens, heads=heads)
    _check(q, k, v, sl, rh, window=window, what=f"ring w={window}")


def test_ring_head_out_of_range_is_reduced():
    """ring_head values outside [0, T_cap) are reduced mod T_cap."""
    slots = 64
    lens = [200, 200]
    q, k, v, sl, rh = _case(2, 4, 1, slots, 64, "bf16", 6350, lens=lens,
                            heads=[64 + 5, -3])
    out, _ = L.attn_decode_gqa(q, k, v, sl, rh)
    rh2 = torch.tensor([5, slots - 3], dtype=torch.int32, device=DEV)
    ro, _ = oracle.gqa_decode_ref(q, k, v, sl, rh2)
    assert_parity(out, ro, "reduced heads")


def test_combine_many_splits_one_row():
    """One (b, h) row with the largest split count and a 512-wide value."""
    B, H, S, d_v = 1, 1, 1024, 512
    g = torch.Generator(device="cpu").manual_seed(6510)
    o = torch.randn(B, H, S, d_v, generator=g)
    l = torch.randn(B, H, S, generator=g) * 3
    out, lse = L.attn_combine(o.to(DEV), l.to(DEV))
    ro, rl = oracle.combine_ref(o.double().numpy(), l.double().numpy())
    assert_parity(out, ro, "combine S=1024")
    assert_lse(lse, rl, "combine S=1024")


@pytest.mark.parametrize("num_splits", [1, 2, 7, 64, 1024])
def test_split_invariance(num_splits):
    T_cap = 2000
    lens = [2000, 1500, 3, 0]
    q, k, v, sl, _ = _case(4, 16, 4, T_cap, 128, "bf16", 6400, lens=lens)
    S = L.attn_decode_gqa_splits(4, 16, 4, T_cap, 128, L.ATTN_BF16, 0, False,
                                 num_splits)
    assert 1 <= S <= min(num_splits, T_cap)
    _check(q, k, v, sl, None, num_splits=num_splits, what=f"S={num_splits}")


@pytest.mark.parametrize("d_v", [64, 128, 256, 512])
@pytest.mark.parametrize("S", [1, 3, 6, 9, 17, 40, 129])
def test_combine_widths(d_v, S):
    """The row merge at every width the decode kernels emit: 7 rows (not a
    multiple of the rows per group), part counts around the 8-part unroll and
    past the thresholds where two and four waves share a row (17, 40, 129),
    empty parts (their values poisoned: never read) and an all-empty row."""
    B, H = 1, 7
    g = torch.Generator(device="cpu").manual_seed(6520 + d_v + S)
    o = torch.randn(B, H, S, d_v, generator=g)
    l = torch.randn(B, H, S, generator=g) * 4
    l[0, 2, S - 1] = -math.inf
    l[0, 5, :] = -math.inf
    o_dev = o.clone()
    o_dev[0, 2, S - 1] = float("nan")
    out, lse = L.attn_combine(o_dev.to(DEV), l.to(DEV))
    ro, rl = oracle.combine_ref(o.double().numpy(), l.double().numpy())
    assert_parity(out, ro, f"combine d_v={d_v} S={S}")
    assert_lse(lse, rl, f"combine d_v={d_v} S={S}")
    assert torch.all(out[0, 5] == 0) and torch.isneginf(lse[0, 5])


def test_combine_entry():
    """attn_combine on its own, with empty parts and an all-empty row."""
    B, H, S, d_v = 3, 5, 9, 96
    g = torch.Generator(device="cpu").manual_seed(6500)
    o = torch.randn(B, H, S, d_v, generator=g)
    l = torch.randn(B, H, S, generator=g) * 4
    l[0, 1, 3] = -math.inf
    l[1, 2, :] = -math.inf
    o[1, 2, :] = 0
    o_dev = o.clone()
    o_dev[0, 1, 3] = float("nan")    # rows of empty parts are never read
    out, lse = L.attn_combine(o_dev.to(DEV), l.to(DEV))
    ro, rl = oracle.combine_ref(o.double().numpy(), l.double().numpy())
    assert_parity(out, ro, "combine")
    assert_lse(lse, rl, "combine")


def test_integer_recovery():
    """Bit-exact index logic: zero keys give every visible position weight
    exactly 1/n_vis; value column i holds bit i of the logical position in the
    slot (last column 1).  out*n_vis must round to the exact counts."""
    d = 64
    cases = [  # (T_cap, T_b, window, ring_head or None)
        (512, 512, 0, None), (512, 300, 0, None), (512, 511, 100, None),
        (512, 1, 0, None), (512, 0, 0, None), (256, 1000, 0, 17),
        (256, 1000, 37, 255), (256, 256, 256, 0), (256, 255, 1, 3),
        (256, 70000, 200, 128)]
    B = len(cases)
    T_cap = 512
    k = torch.zeros(B, 1, T_cap, d, dtype=torch.bfloat16)
    v = np.zeros((B, 1, T_cap, d), dtype=np.float32)
    for b, (cap, T_b, w, head) in enumerate(cases):
        for slot, pos in BF.visible_slots_brute(T_b, cap, 0, head):
            v[b, 0, slot, :d - 1] = [(pos >> i) & 1 for i in range(d - 1)]
            v[b, 0, slot, d - 1] = 1
    v = torch.from_numpy(v).to(torch.bfloat16)
    gen = torch.Generator(device="cpu").manual_seed(6900)
    q = torch.randn(B, 4, d, generator=gen).to(torch.bfloat16)
    # each batch entry has its own ring capacity: run them one by one
    for b, (cap, T_b, w, head) in enumerate(cases):
        kk = k[b:b + 1, :, :cap].contiguous().to(DEV)
        vv = v[b:b + 1, :, :cap].contiguous().to(DEV)
        sl = torch.tensor([T_b], dtype=torch.int32, device=DEV)
        rh = None if head is None else torch.tensor([head], dtype=torch.int32, device=DEV)
        out, lse = L.attn_decode_gqa(q[b:b + 1].to(DEV), kk, vv, sl, rh, w)
        torch.cuda.synchronize()
        vis = [p for _, p in BF.visible_slots_brute(T_b, cap, w, head)]
        n_vis = len(vis)
        o = to64(out)[0]
        if n_vis == 0:
            assert np.all(o == 0) and torch.isneginf(lse).all()
            continue
        want = [sum((p >> i) & 1 for p in vis) for i in range(d - 1)] + [n_vis]
        for h in range(4):
            got = np.rint(o[h] * n_vis).astype(np.int64).tolist()
            assert got == want, (cases[b], h)
            assert int(round(math.exp(float(lse[0, h])))) == n_vis


def test_poison_outside_visible_set():
    """Non-visible slots hold K = 1e4 (would dominate the softmax) and V = NaN
    (would poison any sum): the result must be finite and match the oracle,
    which never touches them."""
    slots, d = 256, 128
    lens = [256, 100, 1, 700, 300]
    heads = [None, None, None, 10, 200]
    for ring in (False, True):
        sel = [i for i, h in enumerate(heads) if (h is not None) == ring]
        ls = [lens[i] for i in sel]
        hs = [heads[i] for i in sel] if ring else None
        q, k, v, sl, rh = _case(len(ls), 8, 2, slots, d, "bf16", 6600 + ring,
                                lens=ls, heads=hs)
        window = 50 if ring else 0
        for b in range(len(ls)):
            vis = {s for s, _ in BF.visible_slots_brute(ls[b], slots, window,
                                                        hs[b] if ring else None)}
            mask = torch.tensor([s not in vis for s in range(slots)], device=DEV)
            k[b, :, mask] = 1e4
            v[b, :, mask] = float("nan")
        _check(q, k, v, sl, rh, window=window, what=f"poison ring={ring}")


def test_batch_zero_is_noop():
    q = torch.empty(0, 8, 64, dtype=torch.bfloat16, device=DEV)
    k = torch.empty(0, 2, 16, 64, dtype=torch.bfloat16, device=DEV)
    out, lse = L.attn_decode_gqa(q, k, k)
    assert out.shape == (0, 8, 64)


def test_default_scale_and_no_lse():
    q, k, v, sl, _ = _case(2, 8, 2, 100, 64, "bf16", 6700, lens=[100, 50])
    out, lse = L.attn_decode_gqa(q, k, v, sl, want_lse=False)
    assert lse is None
    ro, _ = oracle.gqa_decode_ref(q, k, v, sl, scale=1 / math.sqrt(64))
    assert_parity(out, ro, "default scale")


def test_large_scores_stay_finite():
    q, k, v, sl, _ = _case(2, 8, 2, 700, 128, "bf16", 6800, lens=[700, 333])
    _check(q, k, v, sl, None, scale=10.0, what="scale 10")


# ------------------------------------------- full-size workloads, every output
FULL = ["llama3_8b_gqa_t4096", "mha_t32k_b1", "mqa_t32k_b1",
        "swa_ring_w4096_t32k", "swa_linear_w4096_t32k", "wide_d256_t128k",
        "mqa_t32k_b64_ragged", "mha_t32k_b64_ragged", "mha_t32k_b64",
        "mqa_t32k_b64"]


def oracle_all_units(inp, w):
    """The float64 oracle for every (sequence, KV head) unit of a workload,
    one unit per host thread task.  Each task hands the oracle views of its
    own unit, so only that unit's K/V slab is copied from the device (the
    32 GiB cache of the B=64 MHA layer is never copied whole)."""
    B, H_q, H_kv, d = w["B"], w["H_q"], w["H_kv"], w["d"]
    n = H_q // H_kv
    q = inp["q"].cpu()
    sl = None if inp["seq_lens"] is None else inp["seq_lens"].cpu()
    rh = None if inp["ring_head"] is None else inp["ring_head"].cpu()

    def unit(u):
        b, g = u
        return oracle.gqa_decode_ref(
            q[b:b + 1, g * n:(g + 1) * n], inp["k"][b:b + 1, g:g + 1],
            inp["v"][b:b + 1, g:g + 1], None if sl is None else sl[b:b + 1],
            None if rh is None else rh[b:b + 1], inp["window"], inp["scale"])

    units = [(b, g) for b in range(B) for g in range(H_kv)]
    ro = np.zeros((B, H_q, d))
    rl = np.zeros((B, H_q))
    for (b, g), (o, l) in zip(units, map_units(unit, units)):
        ro[b, g * n:(g + 1) * n] = o[0]
        rl[b, g * n:(g + 1) * n] = l[0]
    return ro, rl


@pytest.mark.parametrize("name", FULL)
def test_full_size_every_output(name):
    """The workloads at their real sizes, in the launch configuration the
    bench uses (library-chosen splits; the balanced list where lengths are
    ragged): every output row and log-sum-exp against the oracle, over the
    whole tensor and sequence by sequence."""
    w = synth.workload(name)
    print(f"full size {name}: drawing inputs", flush=True)
    inp = synth.gqa_inputs(w, DEV)
    out, lse = L.attn_decode_gqa(inp["q"], inp["k"], inp["v"], inp["seq_lens"],
                                 inp["ring_head"], inp["window"], inp["scale"])
    torch.cuda.synchronize()
    print(f"full size {name}: oracle over {w['B'] * w['H_kv']} units", flush=True)
    ro, rl = oracle_all_units(inp, w)
    assert_parity_each(out, ro, name)
    assert_lse_each(lse, rl, name)
    del inp
    torch.cuda.empty_cache()
