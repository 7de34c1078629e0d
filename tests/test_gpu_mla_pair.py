"""GPU parity of the role-split MLA kernel (fixed splits of the 512 + 64
latent) against the float64 oracle, and against the shared-latent kernel on
the same fixed splits.  Calls with lengths take the balanced work list (the
shared-latent kernel) whenever it applies, so these cases force a split count
to reach the fixed-split path."""

import math
import os

import numpy as np
import pytest
import torch

import decode_attention_kv_attn_amd as L
import oracle
import synth
from helpers import assert_lse, assert_parity, to64

pytestmark = pytest.mark.gpu
DEV = "cuda"
D_C, D_R = 512, 64
SCALE = 1.0 / math.sqrt(128 + 64)


def _case(B, H, T_cap, seed, lens, value_scale=1.0):
    q = synth.draw((B, H, D_C + D_R), seed, "bf16", DEV, value_scale)
    lat = synth.draw((B, T_cap, D_C + D_R), seed + 1, "bf16", DEV, value_scale)
    sl = torch.tensor(lens, dtype=torch.int32, device=DEV)
    return q, lat, sl


def _run(q, lat, sl, num_splits, kernel=None):
    """attn_decode_mla with ATTN_DECODE_MLA_KERNEL set for the call only."""
    old = os.environ.pop("ATTN_DECODE_MLA_KERNEL", None)
    try:
        if kernel is not None:
            os.environ["ATTN_DECODE_MLA_KERNEL"] = kernel
        z, lse = L.attn_decode_mla(q, lat, D_C, SCALE, sl, num_splits)
        torch.cuda.synchronize()
    finally:
        os.environ.pop("ATTN_DECODE_MLA_KERNEL", None)
        if old is not None:
            os.environ["ATTN_DECODE_MLA_KERNEL"] = old
    return z, lse


@pytest.mark.parametrize("num_splits", [1, 3])
def test_ragged_edges(num_splits):
    """Empty, one-row, tile-edge and ragged-tail sequences; an empty sequence
    gives z = 0 and lse = -inf."""
    lens = [0, 1, 31, 32, 33, 64, 257]
    q, lat, sl = _case(len(lens), 128, 257, 8500 + num_splits, lens)
    z, lse = _run(q, lat, sl, num_splits)
    rz, rl = oracle.mla_decode_ref(q, lat, D_C, SCALE, sl)
    assert_parity(z, rz, f"ragged edges S={num_splits}")
    assert_lse(lse, rl, "ragged edges")
    assert torch.all(z[0] == 0) and torch.all(torch.isneginf(lse[0]))


@pytest.mark.parametrize("H", [16, 100, 128, 192, 256])
def test_head_counts(H):
    """One head chunk of 64 columns (16), a partly empty second chunk (100),
    two, three and four chunks (the XCD placement of a unit's chunks)."""
    q, lat, sl = _case(3, H, 600, 8600 + H, [600, 255, 97])
    z, lse = _run(q, lat, sl, 2)
    rz, rl = oracle.mla_decode_ref(q, lat, D_C, SCALE, sl)
    assert_parity(z, rz, f"H={H}")
    assert_lse(lse, rl, f"H={H}")


@pytest.mark.parametrize("seed", range(4))
def test_random_batches(seed):
    """Seeded batches: 1..40 sequences, lengths from 0 to the capacity, split
    counts from 1 to 9 (pieces that end mid-tile or hold no row)."""
    rng = np.random.default_rng(8700 + seed)
    B = int(rng.integers(1, 41))
    T = int(rng.integers(40, 700))
    lens = rng.integers(0, T + 1, size=B)
    lens[rng.random(B) < 0.15] = 0
    S = int(rng.integers(1, 10))
    q, lat, sl = _case(B, 128, T, 8800 + seed, lens.tolist())
    z, lse = _run(q, lat, sl, S)
    rz, rl = oracle.mla_decode_ref(q, lat, D_C, SCALE, sl)
    assert_parity(z, rz, f"seed={seed} B={B} T={T} S={S}")
    assert_lse(lse, rl, f"seed={seed}")


def test_matches_shared_latent_kernel():
    """The same fixed splits on both kernels: both within the oracle's
    tolerance, and within that tolerance of each other."""
    q, lat, sl = _case(5, 128, 1500, 8900, [1500, 1024, 700, 33, 1])
    zp, lp = _run(q, lat, sl, 4)
    zs, ls = _run(q, lat, sl, 4, kernel="shared")
    rz, rl = oracle.mla_decode_ref(q, lat, D_C, SCALE, sl)
    assert_parity(zp, rz, "role-split kernel")
    assert_parity(zs, rz, "shared-latent kernel")
    assert_lse(lp, rl, "role-split kernel")
    assert_lse(ls, rl, "shared-latent kernel")
    assert_parity(zp, to64(zs), "role-split against shared-latent")


@pytest.mark.parametrize("num_splits", [2, 0], ids=["fixed", "balanced"])
def test_graph_replays(num_splits):
    """A captured MLA call (fixed splits on the role-split kernel, or the
    balanced list on the shared-latent kernel) replays correctly after the
    lengths and queries change: only kernels are captured, nothing is read
    on the host.  Eager work runs between the replays, and every replay is
    checked against the oracle."""
    B, H, T = 6, 128, 1024
    lens0 = [1024, 1, 0, 700, 33, 1000]
    q, lat, sl = _case(B, H, T, 9100 + num_splits, lens0)
    out = torch.empty(B, H, D_C, dtype=torch.float32, device=DEV)
    lse = torch.empty(B, H, dtype=torch.float32, device=DEV)
    ws = torch.empty(L.attn_decode_mla_workspace_bytes(B, H, T, D_C, D_R, num_splits),
                     dtype=torch.uint8, device=DEV)

    def call():
        L.attn_decode_mla(q, lat, D_C, SCALE, sl, num_splits, out=out, lse=lse, workspace=ws)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # warm up off the default stream, as capture requires
        call()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        call()
    torch.cuda.synchronize()
    for trial, lens in enumerate([lens0, [5, 1024, 1024, 0, 0, 17], [0] * B, [1024] * B]):
        sl.copy_(torch.tensor(lens, dtype=torch.int32))
        q.copy_(synth.draw((B, H, D_C + D_R), 9200 + trial, "bf16", DEV, 1.0))
        out.fill_(float("nan"))
        _ = (lat[:, :8].float().sum())  # eager work between the replays
        graph.replay()
        torch.cuda.synchronize()
        rz, rl = oracle.mla_decode_ref(q, lat, D_C, SCALE, sl)
        assert_parity(out, rz, f"replay {trial}")
        assert_lse(lse, rl, f"replay {trial}")


def test_many_sequences():
    """300 sequences (more than the balanced list takes, so ragged lengths
    run fixed splits too): 600 work groups over 256 CUs, several rounds, and
    a grid that is not a whole number of XCD rounds (the placement's tail)."""
    rng = np.random.default_rng(9300)
    B, T = 300, 96
    lens = rng.integers(0, T + 1, size=B)
    q, lat, sl = _case(B, 128, T, 9301, lens.tolist())
    assert L.attn_decode_mla_splits(B, 128, T, D_C, D_R, 0) == 1
    z, lse = _run(q, lat, sl, 0)
    rz, rl = oracle.mla_decode_ref(q, lat, D_C, SCALE, sl)
    assert_parity(z, rz, "B=300")
    assert_lse(lse, rl, "B=300")


def test_queries_beyond_fp16_range():
    """On fixed splits the scores are exact bf16 products summed in fp32, so
    query entries far outside fp16's range (here ~3e5) are accepted: the
    softmax is then nearly one-hot and the output is the winning row's
    values.  (Only the latent must lie in fp16's range.)"""
    B, H, T = 2, 128, 700
    q = synth.draw((B, H, D_C + D_R), 9400, "bf16", DEV, 3.0e5)
    lat = synth.draw((B, T, D_C + D_R), 9401, "bf16", DEV, 1.0 / math.sqrt(576))
    sl = torch.tensor([700, 333], dtype=torch.int32, device=DEV)
    assert float(q.float().abs().max()) > 65504.0
    z, lse = _run(q, lat, sl, 2)
    rz, rl = oracle.mla_decode_ref(q, lat, D_C, SCALE, sl)
    assert_parity(z, rz, "queries beyond fp16")
    # lse ~ 1e5 in magnitude: fp32 holds it to about 1e-2
    assert_lse(lse, rl, "queries beyond fp16", atol=5e-2)
