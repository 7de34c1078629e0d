"""GPU parity of attn_decode_mla (absorbed MLA) against the float64 oracle."""

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
D_C, D_R = 512, 64
SCALE = 1.0 / math.sqrt(128 + 64)


def _case(B, H, T_cap, seed, lens=None, value_scale=1.0 / math.sqrt(576)):
    q = synth.draw((B, H, D_C + D_R), seed, "bf16", DEV, value_scale)
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


@pytest.mark.parametrize("H", [16, 32, 100, 128, 256])
def test_head_counts(H):
    """Head counts below, at and above one work group's 128 heads (100 leaves
    part of a wave empty; 256 needs two head chunks)."""
    q, lat, sl = _case(2, H, 300, 8000 + H, lens=[300, 77])
    _check(q, lat, sl, what=f"H={H}")


@pytest.mark.parametrize("value_scale", [1.0 / math.sqrt(576), 1.0])
def test_value_scales(value_scale):
    """The workload's N(0,1)/sqrt(576) draw and an unscaled N(0,1) draw, whose
    scores spread far wider (the scaled draw makes the softmax almost
    uniform)."""
    q, lat, sl = _case(2, 128, 500, 8100, lens=[500, 333], value_scale=value_scale)
    _check(q, lat, sl, what=f"value_scale={value_scale:.3f}")


def test_ragged_edges():
    lens = [0, 1, 31, 32, 33, 64, 257]
    q, lat, sl = _case(len(lens), 128, 257, 8200, lens=lens, value_scale=1.0)
    z, lse = _check(q, lat, sl, what="ragged edges")
    assert torch.all(z[0] == 0) and torch.all(torch.isneginf(lse[0]))


@pytest.mark.parametrize("num_splits", [1, 2, 7, 64])
def test_split_invariance(num_splits):
    q, lat, sl = _case(3, 128, 1000, 8300, lens=[1000, 500, 3], value_scale=1.0)
    _check(q, lat, sl, num_splits=num_splits, what=f"S={num_splits}")


def test_large_scale_stays_finite():
    q, lat, sl = _case(2, 64, 400, 8400, lens=[400, 100], value_scale=1.0)
    _check(q, lat, sl, scale=1.0, what="scale 1 on N(0,1)")


def test_fp16_range_edges():
    """Both products run in fp16, which holds every bf16 value with
    2^-14 <= |x| <= 65504 exactly (smaller ones with an absolute error below
    2^-25).  Latent rows carrying entries of +-6e4 next to many of +-1e-6,
    and queries with entries down to 1e-7: the relative L2 error stays within
    the bar and the largest error within 2e-3 of the largest output."""
    B, H, T = 2, 128, 700
    q, lat, sl = _case(B, H, T, 8450, lens=[700, 321], value_scale=1.0)
    g = torch.Generator(device="cpu").manual_seed(8451)
    big = torch.rand(lat.shape, generator=g) < 2e-4
    tiny = torch.rand(lat.shape, generator=g) < 0.1
    sign = torch.where(torch.rand(lat.shape, generator=g) < 0.5, -1.0, 1.0)
    lat32 = lat.float().cpu()
    lat32 = torch.where(big, sign * 6.0e4, torch.where(tiny, sign * 1.0e-6, lat32))
    lat = lat32.to(torch.bfloat16).to(DEV)
    q32 = q.float().cpu()
    q32 = torch.where(torch.rand(q.shape, generator=g) < 0.1, 1.0e-7, q32)
    q = q32.to(torch.bfloat16).to(DEV)
    assert float(lat.abs().max()) <= 65504 and int(big.sum()) > 10
    z, lse = L.attn_decode_mla(q, lat, D_C, 0.02, sl)
    torch.cuda.synchronize()
    rz, rl = oracle.mla_decode_ref(q, lat, D_C, 0.02, sl)
    assert_parity(z, rz, "fp16 range", atol=2e-3 * max(1.0, float(np.abs(rz).max())))
    assert_lse(lse, rl, "fp16 range", atol=2e-3 * max(1.0, float(np.abs(rl).max())))


def test_integer_recovery():
    """q = 0 makes every visible weight exactly 1/T_b; latent value column i
    holds bit i of the position (column 511 = 1), the RoPE part is random.
    z * T_b must round to the exact bit counts."""
    T_cap, B = 700, 4
    lens = [700, 513, 1, 64]
    lat = np.zeros((B, T_cap, D_C + D_R), dtype=np.float32)
    pos = np.arange(T_cap)
    for i in range(12):
        lat[:, :, i] = ((pos >> i) & 1)[None, :]
    lat[:, :, D_C - 1] = 1.0
    rng = np.random.default_rng(8500)
    lat[:, :, D_C:] = rng.standard_normal((B, T_cap, D_R))
    latent = torch.from_numpy(lat).to(torch.bfloat16).to(DEV)
    q = torch.zeros(B, 128, D_C + D_R, dtype=torch.bfloat16, device=DEV)
    sl = torch.tensor(lens, dtype=torch.int32, device=DEV)
    z, lse = L.attn_decode_mla(q, latent, D_C, SCALE, sl)
    torch.cuda.synchronize()
    zz = to64(z)
    for b, T_b in enumerate(lens):
        want = [sum((p >> i) & 1 for p in range(T_b)) for i in range(12)]
        got = np.rint(zz[b, :, :12] * T_b).astype(np.int64)
        assert (got == np.array(want)[None, :]).all(), b
        assert np.allclose(zz[b, :, 12:D_C - 1], 0)
        assert np.all(np.rint(zz[b, :, D_C - 1] * T_b) == T_b)
        assert np.all(np.rint(np.exp(to64(lse)[b])) == T_b)


def test_poison_past_length():
    """Rows at or past T_b hold NaN everywhere; they must never be read."""
    lens = [300, 129, 2]
    q, lat, sl = _case(3, 128, 300, 8600, lens=lens, value_scale=1.0)
    ref_lat = lat.clone()
    for b, T_b in enumerate(lens):
        lat[b, T_b:] = float("nan")
    z, lse = L.attn_decode_mla(q, lat, D_C, SCALE, sl)
    torch.cuda.synchronize()
    rz, rl = oracle.mla_decode_ref(q, ref_lat, D_C, SCALE, sl)
    assert_parity(z, rz, "poison")
    assert_lse(lse, rl, "poison")


@pytest.mark.parametrize("name", ["mla_b64_t8192", "mla_b64_t8192_ragged"])
def test_full_size_every_output(name):
    """B=64, 128 heads, latent [64, 8192, 576], N(0,1)/sqrt(576), scale
    1/sqrt(192), in its default launch configuration (uniform lengths: fixed
    splits; lengths on 1024..8192: the balanced list); every sequence against
    the oracle, one sequence per host thread task."""
    w = synth.workload(name)
    inp = synth.mla_inputs(w, DEV)
    z, lse = L.attn_decode_mla(inp["q"], inp["latent"], inp["d_c"], inp["scale"],
                               inp["seq_lens"])
    torch.cuda.synchronize()
    rz, rl = mla_oracle_every_sequence(inp, w)
    assert_parity_each(z, rz, name)
    assert_lse_each(lse, rl, name)
