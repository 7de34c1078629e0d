"""GPU parity of absorbed MLA on the second latent geometry -- 32 query
heads over latent rows of 256 + 64 (the 32-head, latent-256, RoPE-64 model
of the xuesongtap "attention-head" note, section 6) -- against the float64
oracle.  This geometry runs on the latent variant of the matrix-core
kernel: the value is the first 256 columns of each latent row, taken from
the key fragments already loaded."""

import math

import numpy as np
import pytest
import torch

import decode_attention_kv_attn_amd as L
import oracle
import synth
from helpers import (assert_lse, assert_lse_each, assert_parity,
                     assert_parity_each, mla_oracle_every_sequence, to64)

pytestmark = pytest.mark.gpu
DEV = "cuda"
D_C, D_R = 256, 64
SCALE = 1.0 / math.sqrt(128 + 64)


def _case(B, H, T_cap, seed, lens=None, value_scale=1.0 / math.sqrt(320), Lq=None):
    shape = (B, H, D_C + D_R) if Lq is None else (B, Lq, H, D_C + D_R)
    q = synth.draw(shape, seed, "bf16", DEV, value_scale)
    lat = synth.draw((B, T_cap, D_C + D_R), seed + 1, "bf16", DEV, value_scale)
    sl = None if lens is None else torch.tensor(lens, dtype=torch.int32, device=DEV)
    return q, lat, sl


def _check(q, lat, sl, scale=SCALE, num_splits=0, what=""):
    z, lse = L.attn_decode_mla(q, lat, D_C, scale, sl, num_splits)
    torch.cuda.synchronize()
    rz, rl = oracle.mla_decode_ref(q, lat, D_C, scale, sl)
    assert_parity(z, rz, what)
    assert_lse(lse, rl, what)
    return z, lse


@pytest.mark.parametrize("H", [8, 16, 32, 48])
@pytest.mark.parametrize("value_scale", [1.0 / math.sqrt(320), 1.0])
def test_head_counts(H, value_scale):
    q, lat, sl = _case(3, H, 600, 8800 + H, lens=[600, 333, 17], value_scale=value_scale)
    _check(q, lat, sl, what=f"H={H} vs={value_scale:.3f}")


def test_ragged_edges_and_splits():
    lens = [0, 1, 31, 32, 33, 64, 257]
    q, lat, sl = _case(len(lens), 32, 257, 8900, lens=lens, value_scale=1.0)
    for S in (0, 1, 3, 9):
        z, lse = _check(q, lat, sl, num_splits=S, what=f"ragged S={S}")
        assert torch.all(z[0] == 0) and torch.all(torch.isneginf(lse[0]))


def test_integer_recovery():
    """q = 0: every visible weight is exactly 1/T_b; value column i holds
    bit i of the position, column 255 is 1."""
    T_cap, B = 600, 3
    lens = [600, 257, 1]
    lat = np.zeros((B, T_cap, D_C + D_R), dtype=np.float32)
    pos = np.arange(T_cap)
    for i in range(10):
        lat[:, :, i] = ((pos >> i) & 1)[None, :]
    lat[:, :, D_C - 1] = 1.0
    lat[:, :, D_C:] = np.random.default_rng(8950).standard_normal((B, T_cap, D_R))
    latent = torch.from_numpy(lat).to(torch.bfloat16).to(DEV)
    q = torch.zeros(B, 32, D_C + D_R, dtype=torch.bfloat16, device=DEV)
    sl = torch.tensor(lens, dtype=torch.int32, device=DEV)
    z, lse = L.attn_decode_mla(q, latent, D_C, SCALE, sl, 3)
    torch.cuda.synchronize()
    zz = to64(z)
    for b, T_b in enumerate(lens):
        want = [sum((p >> i) & 1 for p in range(T_b)) for i in range(10)]
        got = np.rint(zz[b, :, :10] * T_b).astype(np.int64)
        assert (got == np.array(want)[None, :]).all(), b
        assert np.allclose(zz[b, :, 10:D_C - 1], 0)
        assert np.all(np.rint(zz[b, :, D_C - 1] * T_b) == T_b)
        assert np.all(np.rint(np.exp(to64(lse)[b])) == T_b)


def test_poison_past_length():
    lens = [300, 129, 2]
    q, lat, sl = _case(3, 32, 300, 9000, lens=lens, value_scale=1.0)
    ref = lat.clone()
    for b, T_b in enumerate(lens):
        lat[b, T_b:] = float("nan")
    z, lse = L.attn_decode_mla(q, lat, D_C, SCALE, sl)
    torch.cuda.synchronize()
    rz, rl = oracle.mla_decode_ref(q, ref, D_C, SCALE, sl)
    assert_parity(z, rz, "poison")
    assert_lse(lse, rl, "poison")


def test_paged_and_multi_token():
    """Paged latent pool (bit-identical to the dense call) and several query
    tokens per sequence (oracle parity)."""
    from test_gpu_paged import _latent_pool
    q, lat, sl = _case(3, 32, 512, 9100, lens=[512, 300, 3])
    pool, table = _latent_pool(lat, 16, 9101, poison=True)
    a, la = L.attn_decode_mla_paged(q, pool, table, D_C, SCALE, sl)
    b, lb = L.attn_decode_mla(q, lat, D_C, SCALE, sl)
    torch.cuda.synchronize()
    assert torch.equal(a, b) and torch.equal(la, lb)
    qm, _, _ = _case(3, 32, 512, 9102, Lq=3)
    z, lse = L.attn_decode_mla_multi(qm, lat, D_C, SCALE, sl)
    torch.cuda.synchronize()
    rz, rl = oracle.mla_decode_multi_ref(qm, lat, D_C, SCALE, sl)
    assert_parity(z, rz, "mla256 multi")
    assert_lse(lse, rl, "mla256 multi")


def test_full_size_every_output():
    """B=64, 32 heads, latent [64, 8192, 320], N(0,1)/sqrt(320), library
    splits; every sequence against the oracle."""
    w = synth.workload("mla256_b64_t8192")
    inp = synth.mla_inputs(w, DEV)
    z, lse = L.attn_decode_mla(inp["q"], inp["latent"], inp["d_c"], inp["scale"],
                               inp["seq_lens"])
    torch.cuda.synchronize()
    rz, rl = mla_oracle_every_sequence(inp, w)
    assert_parity_each(z, rz, "mla256_b64_t8192")
    assert_lse_each(lse, rl, "mla256_b64_t8192")
