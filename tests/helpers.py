"""Shared helpers of the GPU parity tests: tolerances and comparisons."""

import os

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
    g = to64(got) if isinstance(got, torch.Tensor) else np.asarray(got, np.float64)
    w = np.asarray(want, np.float64)
    assert np.array_equal(np.isneginf(g), np.isneginf(w)), f"{what}: empty-set pattern"
    fin = np.isfinite(w)
    if fin.any():
        err = float(np.max(np.abs(g[fin] - w[fin])))
        assert err <= atol, f"{what}: lse max_abs={err:.3e}"


def host_workers():
    """Host threads for the per-unit oracle: the cores this process may use,
    at most 16."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def map_units(fn, units, workers=None):
    """fn(u) for every u of `units` on a pool of host threads, each numpy
    call on one BLAS thread (numpy releases the GIL inside its kernels, and
    one thread per small product is far faster than many); results in the
    order of `units`."""
    from concurrent.futures import ThreadPoolExecutor

    from threadpoolctl import threadpool_limits
    with threadpool_limits(limits=1):
        with ThreadPoolExecutor(max_workers=workers or host_workers()) as ex:
            return list(ex.map(fn, units))


def assert_parity_each(got, want, what="", atol=MAX_ABS, rtol_l2=REL_L2):
    """assert_parity over the whole tensor and over each leading index on its
    own (one sequence), so an error confined to one sequence cannot hide in
    the norm of the rest."""
    got64 = to64(got) if isinstance(got, torch.Tensor) else np.asarray(got, np.float64)
    want = np.asarray(want, np.float64)
    assert_parity(got64, want, what, atol, rtol_l2)
    for b in range(want.shape[0]):
        assert_parity(got64[b], want[b], f"{what} [{b}]", atol, rtol_l2)


def assert_lse_each(got, want, what="", atol=2e-3):
    g = to64(got)
    for b in range(g.shape[0]):
        assert_lse(g[b], np.asarray(want)[b], f"{what} [{b}]", atol)


def mla_oracle_every_sequence(inp, w):
    """The float64 MLA oracle for every sequence of a workload, one sequence
    per host thread task (each copies its own latent rows from the device)."""
    import oracle
    q = inp["q"].cpu()
    sl = None if inp["seq_lens"] is None else inp["seq_lens"].cpu()

    def seq(b):
        return oracle.mla_decode_ref(q[b:b + 1], inp["latent"][b:b + 1], inp["d_c"],
                                     inp["scale"], None if sl is None else sl[b:b + 1])

    res = map_units(seq, list(range(w["B"])))
    return (np.concatenate([z for z, _ in res]), np.concatenate([l for _, l in res]))


class GuardBands:
    """Allocator that surrounds every buffer with sentinel-filled margins.

    Each allocation is one larger device buffer: MARGIN bytes of FILL, the
    tensor itself, MARGIN bytes of FILL (MARGIN keeps the tensor's 256-byte
    alignment).  check() waits for the GPU and asserts that no margin byte
    changed, so a kernel that writes past either end of an output, a
    log-sum-exp or a workspace region fails the test that ran it."""

    MARGIN = 64 << 10
    FILL = 0x5A

    def __init__(self):
        self.buffers = []

    def empty(self, shape, dtype, device):
        n = 1
        for x in shape:
            n *= int(x)
        nbytes = n * torch.empty((), dtype=dtype).element_size()
        buf = torch.full((nbytes + 2 * self.MARGIN,), self.FILL, dtype=torch.uint8,
                         device=device)
        self.buffers.append((buf, nbytes, tuple(shape), dtype))
        return buf[self.MARGIN:self.MARGIN + nbytes].view(dtype).view(shape)

    def check(self):
        if not self.buffers:
            return
        if any(b.is_cuda for b, *_ in self.buffers):
            torch.cuda.synchronize()
        for buf, nbytes, shape, dtype in self.buffers:
            head = buf[:self.MARGIN]
            tail = buf[self.MARGIN + nbytes:]
            bad_head = int((head != self.FILL).sum())
            bad_tail = int((tail != self.FILL).sum())
            assert bad_head == 0 and bad_tail == 0, (
                f"guard band of a {dtype} {shape} buffer overwritten: "
                f"{bad_head} bytes before it, {bad_tail} after it")
