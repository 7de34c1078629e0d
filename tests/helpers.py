"""Shared helpers of the GPU parity tests: tolerances and comparisons."""

import numpy as np
import torch

# Bar for floating-point results (fp32 accumulation, fp32 output): both must
# hold over the whole compared tensor.
MAX_ABS = 2e-3
REL_L2 = 1e-3


def to64(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


def parity_stats(got, want):
    got = to64(got) if isinstance(got, torch.Tensor) else np.asarray(got, np.float64)
    want = np.asarray(want, np.float64)
    assert got.shape == want.shape, (got.shape, want.shape)
    diff = got - want
    max_abs = float(np.max(np.abs(diff))) if diff.size else 0.0
    nrm = float(np.linalg.norm(want))
    rel = float(np.linalg.norm(diff)) / nrm if nrm > 0 else (0.0 if max_abs == 0 else np.inf)
    return max_abs, rel


def assert_parity(got, want, what="", atol=MAX_ABS, rtol_l2=REL_L2):
    got64 = to64(got) if isinstance(got, torch.Tensor) else np.asarray(got, np.float64)
    assert np.all(np.isfinite(got64)), f"{what}: non-finite output"
    max_abs, rel = parity_stats(got64, want)
    assert max_abs <= atol and rel <= rtol_l2, (
        f"{what}: max_abs={max_abs:.3e} (<= {atol}) rel_l2={rel:.3e} (<= {rtol_l2})")
    return max_abs, rel


def assert_lse(got, want, what="", atol=2e-3):
    g = to64(got)
    w = np.asarray(want, np.float64)
    assert np.array_equal(np.isneginf(g), np.isneginf(w)), f"{what}: empty-set pattern"
    fin = np.isfinite(w)
    if fin.any():
        err = float(np.max(np.abs(g[fin] - w[fin])))
        assert err <= atol, f"{what}: lse max_abs={err:.3e}"
