"""GPU parity of the paged entry points (attn_decode_gqa_paged,
attn_decode_mla_paged, attn_kv_append_paged) against the float64 oracle.

A paged cache is a shuffled pool of pages of P positions addressed through a
per-sequence block table (the KV-cache paging of the baidu article, section
四.3).  Besides the usual bar (max-abs <= 2e-3, relative L2 <= 1e-3) the
paged kernels must agree BIT FOR BIT with the dense kernels on the same rows
and the same split plan: paging changes where rows are read from, never the
arithmetic.  Appends are byte-exact.
"""

import numpy as np
import pytest
import torch

import decode_attention_kv_attn_amd as L
import oracle
import synth
from helpers import assert_lse, assert_parity, to64

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _pool_from_dense(k, P, seed, spare=5, poison=False):
    """Scatter a dense cache [B, H, T, d] into a shuffled pool
    [num_pages, H, P, d]; returns (pool, table).  Unused pages hold NaN when
    `poison` is set (they must never be read)."""
    B, H, T, d = k.shape
    npb = T // P
    n_pages = B * npb + spare
    g = torch.Generator(device="cpu").manual_seed(seed)
    perm = torch.randperm(n_pages, generator=g)
    table = perm[:B * npb].reshape(B, npb).to(torch.int32)
    fill = float("nan") if poison else 0.0
    pool = torch.full((n_pages, H, P, d), fill, dtype=k.dtype, device=k.device)
    src = k.reshape(B, H, npb, P, d).permute(0, 2, 1, 3, 4).reshape(B * npb, H, P, d)
    pool[table.reshape(-1).long().to(k.device)] = src
    return pool, table.to(k.device)


def _latent_pool(lat, P, seed, spare=5, poison=False):
    pool, table = _pool_from_dense(lat.unsqueeze(1), P, seed, spare, poison)
    return pool.squeeze(1).contiguous(), table


# (dtype, d, H_q, H_kv): vector kernel groups 1, 4, 8 and the matrix-core path
KERNELS = [("bf16", 128, 32, 8), ("fp32", 64, 8, 2), ("bf16", 64, 8, 8),
           ("bf16", 256, 16, 2), ("bf16", 128, 32, 1), ("bf16", 64, 32, 2)]


@pytest.mark.parametrize("dtype,d,H_q,H_kv", KERNELS,
                         ids=[f"{a}-d{b}-{c}x{e}" for a, b, c, e in KERNELS])
@pytest.mark.parametrize("P", [16, 32, 128])
def test_gqa_paged_parity_and_bitwise(dtype, d, H_q, H_kv, P):
    """Shuffled pools, ragged lengths (0, 1, partial pages, full), a window
    and forced splits; parity with the oracle and bit equality with the dense
    kernel on the same rows."""
    T = 768
    lens = [768, 700, 1, 0, 17, 385]
    seed = 9800 + d + H_q + P
    B = len(lens)
    q = synth.draw((B, H_q, d), seed, dtype, DEV)
    k = synth.draw((B, H_kv, T, d), seed + 1, dtype, DEV)
    v = synth.draw((B, H_kv, T, d), seed + 2, dtype, DEV)
    kp, table = _pool_from_dense(k, P, seed, poison=True)
    vp, _ = _pool_from_dense(v, P, seed, poison=True)
    sl = torch.tensor(lens, dtype=torch.int32, device=DEV)
    for window, S in [(0, 0), (200, 3), (0, 7)]:
        out, lse = L.attn_decode_gqa_paged(q, kp, vp, table, sl, window, num_splits=S)
        ref_o, ref_l = L.attn_decode_gqa(q, k, v, sl, None, window, num_splits=S)
        torch.cuda.synchronize()
        assert torch.equal(out, ref_o) and torch.equal(lse, ref_l), (window, S)
        ro, rl = oracle.gqa_decode_paged_ref(q, kp, vp, table, sl, window)
        assert_parity(out, ro, f"paged {dtype} d={d} P={P} w={window} S={S}")
        assert_lse(lse, rl, "paged")


def test_gqa_paged_unaligned_window_tiles():
    """Windows that start mid-page, so tiles straddle up to three pages of 16
    rows; lengths one past a page boundary."""
    T, P = 512, 16
    lens = [512, 497, 33, 17, 16, 15]
    q = synth.draw((6, 8, 128), 9900, "bf16", DEV)
    k = synth.draw((6, 2, T, 128), 9901, "bf16", DEV)
    v = synth.draw((6, 2, T, 128), 9902, "bf16", DEV)
    kp, table = _pool_from_dense(k, P, 9903, poison=True)
    vp, _ = _pool_from_dense(v, P, 9903, poison=True)
    sl = torch.tensor(lens, dtype=torch.int32, device=DEV)
    for window in (1, 7, 31, 33, 100):
        for S in (1, 5):
            out, lse = L.attn_decode_gqa_paged(q, kp, vp, table, sl, window,
                                               num_splits=S)
            torch.cuda.synchronize()
            ro, rl = oracle.gqa_decode_paged_ref(q, kp, vp, table, sl, window)
            assert_parity(out, ro, f"w={window} S={S}")
            assert_lse(lse, rl, f"w={window} S={S}")


def test_gqa_paged_out_of_range_ids_are_clamped():
    """Table ids outside the pool are clamped to it: the call completes and
    equals the oracle on the clamped table."""
    T, P = 64, 16
    q = synth.draw((2, 4, 64), 9950, "bf16", DEV)
    k = synth.draw((2, 1, T, 64), 9951, "bf16", DEV)
    v = synth.draw((2, 1, T, 64), 9952, "bf16", DEV)
    kp, table = _pool_from_dense(k, P, 9953, spare=0)
    vp, _ = _pool_from_dense(v, P, 9953, spare=0)
    n = kp.shape[0]
    bad = table.clone()
    bad[0, 1] = -5
    bad[1, 2] = n + 100
    out, lse = L.attn_decode_gqa_paged(q, kp, vp, bad, None)
    torch.cuda.synchronize()
    clamped = bad.clamp(0, n - 1)
    ro, rl = oracle.gqa_decode_paged_ref(q, kp, vp, clamped, [T, T])
    assert_parity(out, ro, "clamped ids")
    assert_lse(lse, rl, "clamped ids")


@pytest.mark.parametrize("P", [16, 32, 64, 256])
def test_mla_paged_parity_and_bitwise(P):
    """Absorbed MLA over a shuffled latent pool: bit equality with the dense
    MLA kernel on the same rows and parity with the oracle."""
    B, H, T = 4, 128, 1024
    lens = [1024, 1000, 33, 1]
    q = synth.draw((B, H, 576), 9960 + P, "bf16", DEV)
    lat = synth.draw((B, T, 576), 9961 + P, "bf16", DEV)
    pool, table = _latent_pool(lat, P, 9962 + P, poison=True)
    sl = torch.tensor(lens, dtype=torch.int32, device=DEV)
    scale = 192 ** -0.5
    for S in (0, 3):
        z, lse = L.attn_decode_mla_paged(q, pool, table, 512, scale, sl, num_splits=S)
        zd, ld = L.attn_decode_mla(q, lat, 512, scale, sl, num_splits=S)
        torch.cuda.synchronize()
        assert torch.equal(z, zd) and torch.equal(lse, ld), S
        rz, rl = oracle.mla_decode_paged_ref(q, pool, table, 512, scale, sl)
        assert_parity(z, rz, f"mla paged P={P} S={S}")
        assert_lse(lse, rl, "mla paged")


@pytest.mark.parametrize("dtype,H,d", [("bf16", 8, 128), ("fp32", 2, 64),
                                       ("bf16", 1, 576)])
def test_append_paged_is_byte_exact(dtype, H, d):
    """Each sequence's new row lands at page table[b][pos / P], row pos % P of
    every head; nothing else changes; positions past the table are skipped."""
    P, max_pages, n_pages, B = 16, 4, 12, 5
    g = torch.Generator(device="cpu").manual_seed(9970)
    table = torch.randperm(n_pages, generator=g)[:B * max_pages // 2]
    table = torch.cat([table, table]).reshape(B, max_pages).to(torch.int32)
    latent = H == 1 and d == 576
    shape = (n_pages, P, d) if latent else (n_pages, H, P, d)
    kp = synth.draw(shape, 9971, dtype, DEV)
    vp = None if latent else synth.draw(shape, 9972, dtype, DEV)
    kn = synth.draw((B, d) if latent else (B, H, d), 9973, dtype, DEV)
    vn = None if latent else synth.draw((B, H, d), 9974, dtype, DEV)
    pos = torch.tensor([0, 17, 63, 64, -1], dtype=torch.int32)
    want_k = oracle.kv_append_paged_ref(kp, kn, pos, table)
    want_v = None if latent else oracle.kv_append_paged_ref(vp, vn, pos, table)
    L.attn_kv_append_paged(kp, kn, pos.to(DEV), table.to(DEV), vp, vn)
    torch.cuda.synchronize()
    assert np.array_equal(to64(kp), want_k)
    if not latent:
        assert np.array_equal(to64(vp), want_v)


def test_paged_append_decode_loop():
    """Twenty decode steps: append the new token's rows into the pool, then
    decode over it; every step matches the oracle on the gathered history."""
    H_q, H_kv, d, P, max_pages, B = 8, 2, 128, 16, 4, 3
    n_pages = B * max_pages
    table = torch.arange(n_pages, dtype=torch.int32).reshape(B, max_pages).flip(1)
    kp = torch.zeros((n_pages, H_kv, P, d), dtype=torch.bfloat16, device=DEV)
    vp = torch.zeros_like(kp)
    lens = torch.tensor([0, 13, 30], dtype=torch.int32)
    pre_k = synth.draw((B, H_kv, 64, d), 9980, "bf16", DEV)
    pre_v = synth.draw((B, H_kv, 64, d), 9981, "bf16", DEV)
    tdev = table.to(DEV)
    for t in range(int(lens.max())):   # prefill the first lens[b] positions
        pos = torch.tensor([t if t < int(n) else 10**6 for n in lens], dtype=torch.int32)
        L.attn_kv_append_paged(kp, pre_k[:, :, t].contiguous(), pos.to(DEV), tdev, vp,
                               pre_v[:, :, t].contiguous())
    for step in range(20):
        kn = synth.draw((B, H_kv, d), 9990 + step, "bf16", DEV)
        vn = synth.draw((B, H_kv, d), 9890 + step, "bf16", DEV)
        q = synth.draw((B, H_q, d), 9790 + step, "bf16", DEV)
        L.attn_kv_append_paged(kp, kn, lens.to(DEV), tdev, vp, vn)
        lens = lens + 1
        out, lse = L.attn_decode_gqa_paged(q, kp, vp, tdev, lens.to(DEV))
        torch.cuda.synchronize()
        ro, rl = oracle.gqa_decode_paged_ref(q, kp, vp, table, lens)
        assert_parity(out, ro, f"step {step}")
        assert_lse(lse, rl, f"step {step}")


def test_llama_shape_paged_sampled():
    """The Llama-3-8B-shaped workload (B=32, 32/8 heads, d=128, T=4096) in a
    pool of 16-position pages, in the launch configuration of the dense path;
    bit equality with the dense kernel everywhere and oracle parity on a
    sample of sequences."""
    w = synth.workload("llama3_8b_gqa_t4096")
    inp = synth.gqa_inputs(w, DEV)
    kp, table = _pool_from_dense(inp["k"], 16, 9999)
    vp, _ = _pool_from_dense(inp["v"], 16, 9999)
    out, lse = L.attn_decode_gqa_paged(inp["q"], kp, vp, table, inp["seq_lens"])
    ref_o, ref_l = L.attn_decode_gqa(inp["q"], inp["k"], inp["v"], inp["seq_lens"])
    torch.cuda.synchronize()
    assert torch.equal(out, ref_o) and torch.equal(lse, ref_l)
    sample = [0, 13, 31]
    ro, rl = oracle.gqa_decode_ref(inp["q"], inp["k"], inp["v"], inp["seq_lens"],
                                   batches=sample)
    assert_parity(out[sample], ro[sample], "llama paged sample")
    assert_lse(lse[sample], rl[sample], "llama paged sample")
