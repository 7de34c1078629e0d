"""attn_decode_gqa_noalloc (through the C ABI) against attn_decode_gqa with a
caller workspace: two calls in a row on one GPU, the second on a smaller
input, each identical to the workspace form (same plan, same kernels) and
within the oracle's bar (max-abs 2e-3, relative L2 1e-3)."""

import numpy as np
import pytest
import torch

import decode_attention_kv_attn_amd as L
import oracle
import synth
from helpers import assert_lse, assert_parity

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _inputs(B, H_q, H_kv, T, d, seed, lens=None, heads=None):
    q = synth.draw((B, H_q, d), seed, "bf16", DEV)
    k = synth.draw((B, H_kv, T, d), seed + 1, "bf16", DEV)
    v = synth.draw((B, H_kv, T, d), seed + 2, "bf16", DEV)
    sl = None if lens is None else torch.tensor(lens, dtype=torch.int32, device=DEV)
    rh = None if heads is None else torch.tensor(heads, dtype=torch.int32, device=DEV)
    return q, k, v, sl, rh


def _both(q, k, v, sl, rh, window, what):
    B, H_q, d = q.shape
    print(f"noalloc: {what} B={B} H_q={H_q} H_kv={k.shape[1]} T={k.shape[2]} d={d}",
          flush=True)
    out = torch.full((B, H_q, d), float("nan"), device=DEV)
    lse = torch.full((B, H_q), float("nan"), device=DEV)
    L.attn_decode_gqa_noalloc(q, k, v, out, lse, sl, rh, window)
    ref_out, ref_lse = L.attn_decode_gqa(q, k, v, sl, rh, window)
    torch.cuda.synchronize()
    assert torch.equal(out, ref_out), what
    assert torch.equal(lse, ref_lse), what
    ro, rl = oracle.gqa_decode_ref(q, k, v, sl, rh, window)
    assert_parity(out, ro, what)
    assert_lse(lse, rl, what)


def test_noalloc_fixed_splits_then_smaller():
    """MHA, one long sequence (fixed splits through the array), then a
    shorter one with fewer splits."""
    _both(*_inputs(1, 32, 32, 16384, 128, 11000), 0, "fixed splits, large")
    _both(*_inputs(1, 32, 32, 2048, 128, 11010), 0, "fixed splits, smaller")


def test_noalloc_balanced_list_then_smaller():
    """Ragged MQA lengths (the balanced list's parts and per-sequence table in
    the array), then a smaller ragged batch that leaves most of the array as
    the first call wrote it."""
    rng = np.random.default_rng(11020)
    lens = rng.integers(1, 8193, size=8).tolist()
    _both(*_inputs(8, 32, 1, 8192, 128, 11020, lens=lens), 0, "balanced, large")
    _both(*_inputs(3, 32, 1, 2048, 128, 11030, lens=[2048, 5, 1000]), 0,
          "balanced, smaller")


def test_noalloc_ring_and_unsplit():
    """A ring with a window (fixed splits), then a batch large enough to need
    no split (nothing in the array)."""
    _both(*_inputs(4, 32, 8, 4096, 128, 11040, lens=[32768] * 4,
                   heads=[0, 17, 4095, 2000]), 4096, "ring")
    _both(*_inputs(32, 32, 8, 512, 128, 11050), 0, "no split")


def test_noalloc_too_large_is_rejected():
    """64 sequences x 32 heads x 16 splits x 128 floats exceed the 16 MiB
    array: an error before anything is enqueued."""
    q = torch.zeros(64, 32, 128, dtype=torch.bfloat16, device=DEV)
    k = torch.zeros(64, 32, 16, 128, dtype=torch.bfloat16, device=DEV)
    out = torch.empty(64, 32, 128, device=DEV)
    with pytest.raises(L.AttnError, match="workspace"):
        L.attn_decode_gqa_noalloc(q, k, k, out, num_splits=16)
