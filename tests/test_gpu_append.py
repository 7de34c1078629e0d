"""GPU checks of the cache append entry points (bit-exact copies) and of an
append -> decode loop against the oracle."""

import numpy as np
import pytest
import torch

import decode_attention_kv_attn_amd as L
import oracle
import synth
from helpers import assert_lse, assert_parity

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_linear_append_bit_exact(dtype):
    B, H, T_cap, d = 5, 3, 40, 128
    k = synth.draw((B, H, T_cap, d), 9000, dtype, DEV)
    v = synth.draw((B, H, T_cap, d), 9001, dtype, DEV)
    kn = synth.draw((B, H, d), 9002, dtype, DEV)
    vn = synth.draw((B, H, d), 9003, dtype, DEV)
    pos = torch.tensor([0, 39, 17, 40, -3], dtype=torch.int32, device=DEV)
    want_k = oracle.kv_append_ref(k, kn, pos)
    want_v = oracle.kv_append_ref(v, vn, pos)
    L.attn_kv_append(k, kn, pos, v, vn)
    torch.cuda.synchronize()
    assert np.array_equal(k.double().cpu().numpy(), want_k)
    assert np.array_equal(v.double().cpu().numpy(), want_v)


def test_ring_append_bit_exact_and_heads():
    B, H, T_cap, d = 4, 2, 16, 64
    k = synth.draw((B, H, T_cap, d), 9010, "bf16", DEV)
    kn = synth.draw((B, H, d), 9011, "bf16", DEV)
    heads = torch.tensor([15, 0, 7, -1], dtype=torch.int32, device=DEV)
    want_k, want_h = oracle.kv_append_ring_ref(k, kn, heads)
    L.attn_kv_append_ring(k, kn, heads)        # K only (v omitted)
    torch.cuda.synchronize()
    assert np.array_equal(k.double().cpu().numpy(), want_k)
    assert heads.cpu().numpy().tolist() == want_h.tolist()


def test_latent_append():
    B, T_cap, w = 3, 50, 576
    lat = synth.draw((B, T_cap, w), 9020, "bf16", DEV)
    row = synth.draw((B, 1, w), 9021, "bf16", DEV)[:, 0].contiguous()
    pos = torch.tensor([49, 0, 25], dtype=torch.int32, device=DEV)
    want = oracle.kv_append_ref(lat, row, pos)
    L.attn_kv_append(lat, row, pos)
    torch.cuda.synchronize()
    assert np.array_equal(lat.double().cpu().numpy(), want)


def test_ring_append_decode_loop():
    """20 decode steps of a windowed layer kept in an 8-slot ring: append the
    step's K/V, decode, compare with the oracle over the full linear history
    with the same window."""
    B, H_q, H_kv, cap, d, w, steps = 2, 8, 2, 8, 64, 6, 20
    hk = synth.draw((B, H_kv, steps, d), 9030, "bf16", DEV)
    hv = synth.draw((B, H_kv, steps, d), 9031, "bf16", DEV)
    qs = synth.draw((B, steps, H_q, d), 9032, "bf16", DEV)
    k = torch.zeros(B, H_kv, cap, d, dtype=torch.bfloat16, device=DEV)
    v = torch.zeros_like(k)
    head = torch.full((B,), cap - 1, dtype=torch.int32, device=DEV)
    for t in range(steps):
        L.attn_kv_append_ring(k, hk[:, :, t].contiguous(), head, v, hv[:, :, t].contiguous())
        lens = torch.full((B,), t + 1, dtype=torch.int32, device=DEV)
        q = qs[:, t].contiguous()
        out, lse = L.attn_decode_gqa(q, k, v, lens, head, w)
        torch.cuda.synchronize()
        ro, rl = oracle.gqa_decode_ref(q, hk[:, :, :t + 1], hv[:, :, :t + 1], lens,
                                       window=w)
        assert_parity(out, ro, f"step {t}")
        assert_lse(lse, rl, f"step {t}")
