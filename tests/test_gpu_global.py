"""GPU parity of attn_decode_gqa_global (sliding window plus global
positions, linear cache) against the float64 oracle.

The visible set of the query at t is its window t-w+1..t plus every global
position g < t-w+1; a query that is itself global sees 0..t (the
window-plus-global pattern of the attention-head note, section 3, example
G = {0, 5}).  Same bar as the other parity tests: max-abs <= 2e-3 and
relative L2 <= 1e-3, visible sets bit-exact through integer recovery.
"""

import math

import numpy as np
import pytest
import torch

import decode_attention_kv_attn_amd as L
import oracle
import synth
from oracle import bruteforce as BF
from helpers import assert_lse, assert_parity, to64

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _inputs(B, H_q, H_kv, T_cap, d, dtype, seed, value_scale=1.0):
    q = synth.draw((B, H_q, d), seed, dtype, DEV, value_scale)
    k = synth.draw((B, H_kv, T_cap, d), seed + 1, dtype, DEV, value_scale)
    v = synth.draw((B, H_kv, T_cap, d), seed + 2, dtype, DEV, value_scale)
    return q, k, v


def _gpos(g):
    return None if g is None else torch.tensor(sorted(g), dtype=torch.int32, device=DEV)


def _check(q, k, v, lens, window, G, num_splits=0, what=""):
    sl = None if lens is None else torch.tensor(lens, dtype=torch.int32, device=DEV)
    out, lse = L.attn_decode_gqa_global(q, k, v, _gpos(G), window, sl,
                                        num_splits=num_splits)
    torch.cuda.synchronize()
    ro, rl = oracle.gqa_decode_ref(q, k, v, sl, None, window,
                                   global_pos=None if G is None else sorted(G))
    assert_parity(out, ro, what)
    assert_lse(lse, rl, what)
    return out, lse


# (dtype, d, H_q, H_kv): vector kernel (group 4) and matrix-core kernel
# (bf16, group 16 and 32)
KERNELS = [("bf16", 128, 32, 8), ("fp32", 64, 8, 2), ("bf16", 64, 8, 8),
           ("bf16", 128, 32, 2), ("bf16", 64, 32, 1), ("bf16", 256, 8, 2)]


@pytest.mark.parametrize("dtype,d,H_q,H_kv", KERNELS,
                         ids=[f"{a}-d{b}-{c}x{e}" for a, b, c, e in KERNELS])
@pytest.mark.parametrize("num_splits", [0, 1, 3, 17])
def test_window_plus_globals(dtype, d, H_q, H_kv, num_splits):
    """Globals before, inside and after the window; queries that are global
    themselves (t = 5, t = 700); ragged lengths; forced split counts so that
    pieces start inside the global rows and straddle the window's start."""
    T_cap = 800
    G = [0, 5, 37, 38, 100, 333, 600, 700]
    lens = [800, 701, 6, 1, 0, 250, 799, 640]
    seed = 9100 + d + H_q + num_splits
    q, k, v = _inputs(len(lens), H_q, H_kv, T_cap, d, dtype, seed)
    _check(q, k, v, lens, 64, G, num_splits,
           what=f"{dtype} d={d} {H_q}/{H_kv} S={num_splits}")


@pytest.mark.parametrize("window", [1, 2, 33, 400, 5000])
def test_windows_and_dense_globals(window):
    """Every 7th position global, so tiles mix global rows and window rows
    for every window width (including one wider than the cache)."""
    T_cap = 1000
    G = list(range(0, T_cap, 7))
    lens = [1000, 999, 64, 3, 500, 701]
    q, k, v = _inputs(len(lens), 16, 4, T_cap, 128, "bf16", 9300 + window)
    _check(q, k, v, lens, window, G, what=f"w={window}")


def test_no_globals_matches_plain_entry_bitwise():
    """n_global = 0 is attn_decode_gqa without ring, to the bit."""
    q, k, v = _inputs(4, 32, 8, 2048, 128, "bf16", 9400)
    sl = torch.tensor([2048, 1500, 17, 0], dtype=torch.int32, device=DEV)
    a, la = L.attn_decode_gqa(q, k, v, sl, None, 300)
    b, lb = L.attn_decode_gqa_global(q, k, v, None, 300, sl)
    torch.cuda.synchronize()
    assert torch.equal(a, b) and torch.equal(la, lb)


def test_integer_recovery_globals():
    """Bit-exact visible sets: zero keys give each visible position weight
    exactly 1/n_vis; value column i holds bit i of the position (last column
    1), so out*n_vis rounds to the exact bit counts over the visible set."""
    d, T_cap = 64, 512
    G = [0, 1, 5, 64, 65, 200, 300, 511]
    cases = [(512, 64), (300, 64), (301, 1), (6, 2), (66, 10), (512, 0),
             (201, 100), (1, 1), (0, 8), (450, 33), (400, 16), (100, 20),
             (70, 3), (257, 50)]   # (T_b, window)
    k = torch.zeros(1, 1, T_cap, d, dtype=torch.bfloat16, device=DEV)
    pos = np.arange(T_cap)
    v = np.zeros((1, 1, T_cap, d), dtype=np.float32)
    for i in range(d - 1):
        v[0, 0, :, i] = (pos >> i) & 1
    v[0, 0, :, d - 1] = 1
    v = torch.from_numpy(v).to(torch.bfloat16).to(DEV)
    gen = torch.Generator(device="cpu").manual_seed(9500)
    q = torch.randn(1, 4, d, generator=gen).to(torch.bfloat16).to(DEV)
    for T_b, w in cases:
        sl = torch.tensor([T_b], dtype=torch.int32, device=DEV)
        out, lse = L.attn_decode_gqa_global(q, k, v, _gpos(G), w, sl)
        torch.cuda.synchronize()
        vis = [p for _, p in BF.visible_slots_brute(T_b, T_cap, w, None, G)]
        n_vis = len(vis)
        o = to64(out)[0]
        if n_vis == 0:
            assert np.all(o == 0) and torch.isneginf(lse).all()
            continue
        want = [sum((p >> i) & 1 for p in vis) for i in range(d - 1)] + [n_vis]
        for h in range(4):
            got = np.rint(o[h] * n_vis).astype(np.int64).tolist()
            assert got == want, (T_b, w, h)
            assert int(round(math.exp(float(lse[0, h])))) == n_vis


def test_poison_outside_visible_set():
    """NaN in every cache row outside the visible set leaves the result
    finite and equal to the oracle's on clean inputs: masked rows are never
    read."""
    T_cap, w = 700, 50
    G = [0, 3, 250, 251]
    lens = [700, 252, 400]
    q, k, v = _inputs(len(lens), 8, 2, T_cap, 128, "bf16", 9600)
    kp, vp = k.clone(), v.clone()
    for b, T_b in enumerate(lens):
        seen = {s for s, _ in BF.visible_slots_brute(T_b, T_cap, w, None, G)}
        for s in range(T_cap):
            if s not in seen:
                kp[b, :, s] = float("nan")
                vp[b, :, s] = float("nan")
    sl = torch.tensor(lens, dtype=torch.int32, device=DEV)
    out, lse = L.attn_decode_gqa_global(q, kp, vp, _gpos(G), w, sl, num_splits=5)
    torch.cuda.synchronize()
    ro, rl = oracle.gqa_decode_ref(q, k, v, sl, None, w, global_pos=G)
    assert_parity(out, ro, "poison")
    assert_lse(lse, rl, "poison")


def test_llama_shape_sink_tokens():
    """Llama-3-8B-shaped heads (32 query / 8 KV, d=128) at T=4096 with a
    1024-wide window, 64 leading sink positions and every 256th position
    global; the batch includes queries at global positions."""
    T_cap = 4096
    G = sorted(set(range(64)) | set(range(0, T_cap, 256)))
    lens = [4096, 3841, 2049, 1025, 65, 3000]
    q, k, v = _inputs(len(lens), 32, 8, T_cap, 128, "bf16", 9700)
    _check(q, k, v, lens, 1024, G, what="llama sink")
