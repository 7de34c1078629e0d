"""GPU parity of several query tokens per sequence (attn_decode_gqa_multi,
attn_decode_mla_multi and the q_len of the paged entry points) against the
float64 oracle.

Token l of an L-token chunk sits at T_b - L + l and sees what a single
decode query there sees (causal inside the chunk, its own window, the ring's
resident positions).  Bar: max-abs <= 2e-3 and relative L2 <= 1e-3; visible
sets bit-exact through integer recovery; L = 1 and paged forms bit-identical
to the single-token / dense kernels.
"""

import math

import numpy as np
import pytest
import torch

import decode_attention_kv_attn_amd as L
import oracle
import synth
from helpers import (assert_lse, assert_lse_each, assert_parity,
                     assert_parity_each, map_units, to64)

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _inputs(B, Lq, H_q, H_kv, T, d, dtype, seed):
    q = synth.draw((B, Lq, H_q, d), seed, dtype, DEV)
    k = synth.draw((B, H_kv, T, d), seed + 1, dtype, DEV)
    v = synth.draw((B, H_kv, T, d), seed + 2, dtype, DEV)
    return q, k, v


# (dtype, d, H_q, H_kv, L): vector kernel (fp32, d=256, one head and two
# tokens) and matrix-core kernel (bf16 columns n*L >= 3, up to three chunks)
CASES = [("fp32", 64, 8, 4, 2), ("bf16", 128, 32, 8, 4), ("bf16", 128, 8, 8, 2),
         ("bf16", 256, 8, 2, 3), ("bf16", 64, 32, 1, 3), ("bf16", 128, 16, 2, 7),
         ("fp32", 128, 4, 4, 8)]


@pytest.mark.parametrize("dtype,d,H_q,H_kv,Lq", CASES,
                         ids=[f"{a}-d{b}-{c}x{e}-L{f}" for a, b, c, e, f in CASES])
@pytest.mark.parametrize("window,S", [(0, 0), (50, 3), (7, 1)])
def test_gqa_multi_linear(dtype, d, H_q, H_kv, Lq, window, S):
    """Ragged lengths including sequences shorter than the chunk (tokens at
    negative positions see nothing)."""
    T = 320
    lens = [320, 300, Lq, 1, 0, 33]
    q, k, v = _inputs(len(lens), Lq, H_q, H_kv, T, d, dtype,
                      7000 + d + H_q + Lq + window)
    sl = torch.tensor(lens, dtype=torch.int32, device=DEV)
    out, lse = L.attn_decode_gqa_multi(q, k, v, sl, None, window, num_splits=S)
    torch.cuda.synchronize()
    ro, rl = oracle.gqa_decode_multi_ref(q, k, v, sl, None, window)
    assert_parity(out, ro, f"multi {dtype} d={d} {H_q}/{H_kv} L={Lq} w={window} S={S}")
    assert_lse(lse, rl, "multi")


@pytest.mark.parametrize("Lq,window", [(2, 0), (4, 64), (5, 252), (3, 1)])
def test_gqa_multi_ring(Lq, window):
    """Ring buffer of 256 slots, logical lengths past the capacity, the
    first token's window kept resident (window + L - 1 <= 256)."""
    T = 256
    lens = [256, 1000, 70000, 300, Lq + 1]
    heads = [255, 17, 3, 128, 0]
    q, k, v = _inputs(len(lens), Lq, 32, 8, T, 128, "bf16", 7100 + Lq + window)
    sl = torch.tensor(lens, dtype=torch.int32, device=DEV)
    rh = torch.tensor(heads, dtype=torch.int32, device=DEV)
    out, lse = L.attn_decode_gqa_multi(q, k, v, sl, rh, window, num_splits=3)
    torch.cuda.synchronize()
    ro, rl = oracle.gqa_decode_multi_ref(q, k, v, sl, rh, window)
    assert_parity(out, ro, f"ring L={Lq} w={window}")
    assert_lse(lse, rl, "ring")


@pytest.mark.parametrize("dtype,H_q,H_kv", [("bf16", 32, 8), ("fp32", 8, 2)])
def test_single_token_is_plain_decode_bitwise(dtype, H_q, H_kv):
    q, k, v = _inputs(4, 1, H_q, H_kv, 1024, 128, dtype, 7200)
    sl = torch.tensor([1024, 700, 3, 0], dtype=torch.int32, device=DEV)
    a, la = L.attn_decode_gqa_multi(q, k, v, sl, None, 100)
    b, lb = L.attn_decode_gqa(q[:, 0].contiguous(), k, v, sl, None, 100)
    torch.cuda.synchronize()
    assert torch.equal(a[:, 0], b) and torch.equal(la[:, 0], lb)


def test_multi_integer_recovery():
    """Bit-exact visible sets per token: zero keys give each visible
    position weight 1/n_vis; value column i holds bit i of the position."""
    d, T, Lq = 64, 256, 5
    cases = [(256, 0), (256, 9), (100, 3), (5, 0), (3, 2), (60, 1)]
    k = torch.zeros(1, 1, T, d, dtype=torch.bfloat16, device=DEV)
    pos = np.arange(T)
    v = np.zeros((1, 1, T, d), dtype=np.float32)
    for i in range(d - 1):
        v[0, 0, :, i] = (pos >> i) & 1
    v[0, 0, :, d - 1] = 1
    v = torch.from_numpy(v).to(torch.bfloat16).to(DEV)
    gen = torch.Generator(device="cpu").manual_seed(7300)
    q = torch.randn(1, Lq, 4, d, generator=gen).to(torch.bfloat16).to(DEV)
    for T_b, w in cases:
        sl = torch.tensor([T_b], dtype=torch.int32, device=DEV)
        out, lse = L.attn_decode_gqa_multi(q, k, v, sl, None, w)
        torch.cuda.synchronize()
        o = to64(out)[0]
        for tok in range(Lq):
            t = T_b - Lq + tok
            lo = max(0, t - w + 1) if w > 0 else 0
            vis = list(range(lo, t + 1)) if t >= 0 else []
            n_vis = len(vis)
            if n_vis == 0:
                assert np.all(o[tok] == 0) and torch.isneginf(lse[0, tok]).all()
                continue
            want = [sum((p >> i) & 1 for p in vis) for i in range(d - 1)] + [n_vis]
            for h in range(4):
                got = np.rint(o[tok, h] * n_vis).astype(np.int64).tolist()
                assert got == want, (T_b, w, tok, h)
                assert int(round(math.exp(float(lse[0, tok, h])))) == n_vis


def test_paged_multi_equals_dense_bitwise():
    """Several tokens over a shuffled page pool: bit-identical to the dense
    kernel on the same rows."""
    from test_gpu_paged import _pool_from_dense
    T, P, Lq = 512, 16, 4
    q, k, v = _inputs(3, Lq, 32, 8, T, 128, "bf16", 7400)
    kp, table = _pool_from_dense(k, P, 7401, poison=True)
    vp, _ = _pool_from_dense(v, P, 7401, poison=True)
    sl = torch.tensor([512, 260, 3], dtype=torch.int32, device=DEV)
    for window, S in [(0, 0), (40, 2)]:
        a, la = L.attn_decode_gqa_paged(q, kp, vp, table, sl, window, num_splits=S)
        b, lb = L.attn_decode_gqa_multi(q, k, v, sl, None, window, num_splits=S)
        torch.cuda.synchronize()
        assert torch.equal(a, b) and torch.equal(la, lb), (window, S)
        ro, rl = oracle.gqa_decode_multi_ref(q, k, v, sl, None, window)
        assert_parity(a, ro, "paged multi")


@pytest.mark.parametrize("Lq,H", [(2, 128), (4, 64), (3, 16)])
def test_mla_multi(Lq, H):
    """Absorbed MLA with several tokens: parity with the oracle; paged form
    bit-identical to the dense one."""
    from test_gpu_paged import _latent_pool
    B, T = 3, 768
    lens = [768, 400, 2]
    q = synth.draw((B, Lq, H, 576), 7500 + Lq, "bf16", DEV)
    lat = synth.draw((B, T, 576), 7501 + Lq, "bf16", DEV)
    sl = torch.tensor(lens, dtype=torch.int32, device=DEV)
    scale = 192 ** -0.5
    for S in (0, 2):
        z, lse = L.attn_decode_mla_multi(q, lat, 512, scale, sl, num_splits=S)
        torch.cuda.synchronize()
        rz, rl = oracle.mla_decode_multi_ref(q, lat, 512, scale, sl)
        assert_parity(z, rz, f"mla multi L={Lq} H={H} S={S}")
        assert_lse(lse, rl, "mla multi")
    pool, table = _latent_pool(lat, 32, 7502, poison=True)
    zp, lp = L.attn_decode_mla_paged(q, pool, table, 512, scale, sl)
    zd, ld = L.attn_decode_mla_multi(q, lat, 512, scale, sl)
    torch.cuda.synchronize()
    assert torch.equal(zp, zd) and torch.equal(lp, ld)


def test_mla_single_token_is_plain_decode_bitwise():
    q = synth.draw((2, 1, 128, 576), 7600, "bf16", DEV)
    lat = synth.draw((2, 1024, 576), 7601, "bf16", DEV)
    sl = torch.tensor([1024, 500], dtype=torch.int32, device=DEV)
    a, la = L.attn_decode_mla_multi(q, lat, 512, 0.07, sl)
    b, lb = L.attn_decode_mla(q[:, 0].contiguous(), lat, 512, 0.07, sl)
    torch.cuda.synchronize()
    assert torch.equal(a[:, 0], b) and torch.equal(la[:, 0], lb)


def test_llama_shape_speculative_verify_every_output():
    """Verifying 4 draft tokens on the Llama-3-8B-shaped layer (B=32, 32/8
    heads, d=128, T=4096), in its default launch configuration; every
    sequence against the oracle, one sequence per host thread task."""
    w = synth.workload("llama3_8b_gqa_t4096")
    inp = synth.gqa_inputs(w, DEV)
    q = synth.draw((32, 4, 32, 128), 7700, "bf16", DEV)
    out, lse = L.attn_decode_gqa_multi(q, inp["k"], inp["v"], inp["seq_lens"])
    torch.cuda.synchronize()
    qc = q.cpu()

    def seq(b):
        return oracle.gqa_decode_multi_ref(qc[b:b + 1], inp["k"][b:b + 1],
                                           inp["v"][b:b + 1])

    res = map_units(seq, list(range(32)))
    ro = np.concatenate([o for o, _ in res])
    rl = np.concatenate([l for _, l in res])
    assert_parity_each(out, ro, "speculative verify")
    assert_lse_each(lse, rl, "speculative verify")
