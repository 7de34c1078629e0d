"""GPU parity of the balanced work list against the float64 oracle.

When the library picks the splits and a batch has fewer (sequence, KV head)
units than work groups, a call that passes lengths cuts each sequence's
visible rows by its own length instead of cutting every sequence into the
same number of fixed pieces: the vector kernel takes pieces of one common
size (at least one per sequence); the matrix-core kernel lays the units'
32-row tiles end to end and gives every work group the same number of them
(the even split), so one group may finish a sequence and start the next
ones.  The lists are derived on the device from seq_lens, so these tests
cover its edges: empty and one-row sequences, a single long sequence among
empty ones, every sequence in one piece, the most sequences the list takes
(four per lane), two head chunks per KV head, several query tokens, global
positions and paged pools; rings keep the fixed splits.  Bar: max-abs <= 2e-3, relative L2 <=
1e-3; visited rows bit-exact through integer recovery.
"""

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


def _balanced(B, H_q, H_kv, T, d, window=0, ring=False, n_global=0, q_len=1):
    p = L.attn_decode_gqa_plan(B, H_q, H_kv, T, d, 1, window, ring, n_global, 0, q_len)
    return p["balanced_groups"] > 0


def _inputs(lens, H_q, H_kv, T, d, seed, Lq=None):
    B = len(lens)
    qs = (B, H_q, d) if Lq is None else (B, Lq, H_q, d)
    q = synth.draw(qs, seed, "bf16", DEV)
    k = synth.draw((B, H_kv, T, d), seed + 1, "bf16", DEV)
    v = synth.draw((B, H_kv, T, d), seed + 2, "bf16", DEV)
    sl = torch.tensor(lens, dtype=torch.int32, device=DEV)
    return q, k, v, sl


MIXES = {
    "extreme": [0, 1, 2048, 1500, 129, 128, 257, 2047, 1024, 3, 640, 2000],
    "one_long": [2048] + [0] * 15,
    "all_empty": [0] * 8,
    "uniform": [2048] * 8,
    "all_one_piece": [1, 2, 3, 100, 127, 255, 256, 200],
}
# (d, H_q, H_kv): matrix-core kernel -- MQA-sized groups, two KV heads of 16,
# d = 256, and 48 heads per KV head (two head chunks of 32 columns); vector
# kernel -- MHA at d = 64 and groups of 2 at d = 256
KERNELS = [(128, 32, 1), (64, 32, 2), (256, 16, 2), (128, 96, 2), (64, 8, 8),
           (256, 8, 4)]


@pytest.mark.parametrize("d,H_q,H_kv", KERNELS, ids=[f"d{a}-{b}x{c}" for a, b, c in KERNELS])
@pytest.mark.parametrize("mix", list(MIXES))
def test_length_mixes(d, H_q, H_kv, mix):
    lens = MIXES[mix]
    T = 2048
    assert _balanced(len(lens), H_q, H_kv, T, d)
    q, k, v, sl = _inputs(lens, H_q, H_kv, T, d, 12000 + d + H_q + len(mix))
    plan = L.attn_decode_gqa_plan(len(lens), H_q, H_kv, T, d, 1)
    assert plan["even_split"] == (plan["kernel"] == "mfma" and d <= 128)
    out, lse = L.attn_decode_gqa(q, k, v, sl)
    torch.cuda.synchronize()
    ro, rl = oracle.gqa_decode_ref(q, k, v, sl)
    assert_parity(out, ro, f"balanced {mix} d={d} {H_q}/{H_kv}")
    assert_lse(lse, rl, f"balanced {mix}")
    if mix == "all_empty":
        assert torch.all(out == 0) and torch.all(torch.isneginf(lse))
    # the fixed splits give the same result within the bar
    S = L.attn_decode_gqa_splits(len(lens), H_q, H_kv, T, d, 1)
    out2, _ = L.attn_decode_gqa(q, k, v, sl, num_splits=S)
    torch.cuda.synchronize()
    assert_parity(out2, ro, f"fixed {mix}")


EVEN_MIXES = {
    # groups that cross many short units, units that span many groups
    "short_and_long": [3000, 5, 0, 40, 2500, 31, 32, 33, 1, 4096, 64, 65] * 4,
    # every unit a single tile: each group covers several whole units
    "one_tile_each": [32] * 40 + [1] * 20 + [0] * 4,
    # one unit over every group but a few empty ones
    "one_over_all": [0, 0, 4096, 0, 0],
}


@pytest.mark.parametrize("mix", list(EVEN_MIXES))
@pytest.mark.parametrize("H_q,H_kv,d", [(32, 2, 128), (64, 1, 64)],
                         ids=["16x2-d128", "64x1-d64-two-chunks"])
def test_even_split_segments(mix, H_q, H_kv, d):
    """The even split's segments: one work group computes pieces of several
    (sequence, KV head, head chunk) units, each into its own slot, and a long
    unit's pieces come from consecutive groups; a second call on the same
    workspace with other lengths must not see the first call's slots or
    pairs."""
    lens = EVEN_MIXES[mix]
    B, T = len(lens), 4096
    plan = L.attn_decode_gqa_plan(B, H_q, H_kv, T, d, 1)
    assert plan["kernel"] == "mfma" and plan["even_split"] and plan["balanced_groups"] > 0
    q, k, v, sl = _inputs(lens, H_q, H_kv, T, d, 31000 + B + H_q + d)
    ws = torch.empty(plan["workspace_bytes"], dtype=torch.uint8, device=DEV)
    out, lse = L.attn_decode_gqa(q, k, v, sl, workspace=ws)
    torch.cuda.synchronize()
    ro, rl = oracle.gqa_decode_ref(q, k, v, sl)
    assert_parity(out, ro, f"even split {mix}")
    assert_lse(lse, rl, f"even split {mix}")
    # other lengths, same workspace
    sl2 = torch.flip(sl, [0]).contiguous()
    out2, lse2 = L.attn_decode_gqa(q, k, v, sl2, workspace=ws)
    torch.cuda.synchronize()
    ro2, rl2 = oracle.gqa_decode_ref(q, k, v, sl2)
    assert_parity(out2, ro2, f"even split {mix}, second call")
    assert_lse(lse2, rl2, f"even split {mix}, second call")


def _random_case(rng):
    """One random ragged batch that the planner sends to the matrix-core
    kernel's even split (shapes are drawn again until it does)."""
    while True:
        d = int(rng.choice([64, 128]))
        H_kv = int(rng.choice([1, 2, 4]))
        n = int(rng.choice([3, 4, 8, 16, 32, 48]))
        B = int(rng.choice([1, 2, 7, 33, 64, 130, 250]))
        T = int(rng.choice([1000, 2048, 4096]))
        plan = L.attn_decode_gqa_plan(B, H_kv * n, H_kv, T, d, 1)
        if plan["even_split"]:
            break
    kinds = rng.integers(0, 4, size=B)
    lens = np.where(kinds == 0, 0, np.where(kinds == 1, rng.integers(1, 40, size=B),
                                            rng.integers(1, T + 1, size=B)))
    return d, H_kv * n, H_kv, T, lens.astype(int).tolist()


@pytest.mark.parametrize("seed", range(12))
def test_even_split_random(seed):
    """Seeded random ragged batches (empty, one-row and long sequences mixed;
    1 to 250 sequences, group sizes 3..48 -- one or two head chunks, d = 64
    or 128) on the even split, against the oracle."""
    rng = np.random.default_rng(32000 + seed)
    d, H_q, H_kv, T, lens = _random_case(rng)
    B = len(lens)
    plan = L.attn_decode_gqa_plan(B, H_q, H_kv, T, d, 1)
    q, k, v, sl = _inputs(lens, H_q, H_kv, T, d, 32100 + 7 * seed)
    out, lse = L.attn_decode_gqa(q, k, v, sl)
    torch.cuda.synchronize()
    ro, rl = oracle.gqa_decode_ref(q, k, v, sl)
    what = f"seed {seed}: B={B} {H_q}/{H_kv} d={d} T={T} plan={plan}"
    print(what, flush=True)
    assert_parity(out, ro, what)
    assert_lse(lse, rl, what)


def test_fp32_vector_kernel():
    """float32 data always takes the vector kernel: the same list, MQA-sized
    group of 8 columns per item (four items per KV head)."""
    lens = [0, 1, 2048, 1500, 129, 2047]
    T, d = 2048, 64
    B = len(lens)
    p = L.attn_decode_gqa_plan(B, 32, 1, T, d, 0)
    assert p["kernel"] == "valu" and p["balanced_groups"] > 0
    q = synth.draw((B, 32, d), 12950, "fp32", DEV)
    k = synth.draw((B, 1, T, d), 12951, "fp32", DEV)
    v = synth.draw((B, 1, T, d), 12952, "fp32", DEV)
    sl = torch.tensor(lens, dtype=torch.int32, device=DEV)
    out, lse = L.attn_decode_gqa(q, k, v, sl)
    torch.cuda.synchronize()
    ro, rl = oracle.gqa_decode_ref(q, k, v, sl)
    assert_parity(out, ro, "balanced fp32")
    assert_lse(lse, rl, "balanced fp32")


def test_integer_recovery_balanced():
    """Zero keys give every visible position weight 1/n_vis; value column i
    holds bit i of the position (last column 1): out * n_vis must round to
    the exact counts, so every visible row is read exactly once whichever
    piece holds it."""
    d, T = 64, 2048
    lens = [0, 1, 2048, 1000, 129, 1500, 300, 2047, 4096, 640]
    B = len(lens)
    assert _balanced(B, 32, 1, T, d)
    k = torch.zeros(B, 1, T, d, dtype=torch.bfloat16, device=DEV)
    pos = np.arange(T)
    vv = np.zeros((T, d), np.float32)
    for i in range(d - 1):
        vv[:, i] = (pos >> i) & 1
    vv[:, d - 1] = 1
    v = torch.from_numpy(vv).to(torch.bfloat16).to(DEV).expand(B, 1, T, d).contiguous()
    gen = torch.Generator(device="cpu").manual_seed(12100)
    q = torch.randn(B, 32, d, generator=gen).to(torch.bfloat16).to(DEV)
    sl = torch.tensor(lens, dtype=torch.int32, device=DEV)
    out, lse = L.attn_decode_gqa(q, k, v, sl)
    torch.cuda.synchronize()
    o = to64(out)
    for b, T_b in enumerate(lens):
        n_vis = min(T_b, T)
        if n_vis == 0:
            assert np.all(o[b] == 0) and torch.isneginf(lse[b]).all()
            continue
        want = [int(((np.arange(n_vis) >> i) & 1).sum()) for i in range(d - 1)] + [n_vis]
        for h in (0, 13, 31):
            got = np.rint(o[b, h] * n_vis).astype(np.int64).tolist()
            assert got == want, (b, h)


def test_poison_past_lengths():
    """Rows past each length hold K = 1e4 and V = NaN: no piece may read them."""
    lens = [0, 1, 2048, 700, 129, 1999]
    q, k, v, sl = _inputs(lens, 32, 1, 2048, 128, 12200)
    for b, T_b in enumerate(lens):
        k[b, :, T_b:] = 1e4
        v[b, :, T_b:] = float("nan")
    out, lse = L.attn_decode_gqa(q, k, v, sl)
    torch.cuda.synchronize()
    ro, rl = oracle.gqa_decode_ref(q, k, v, sl)
    assert_parity(out, ro, "balanced poison")
    assert_lse(lse, rl, "balanced poison")


@pytest.mark.parametrize("B", [1, 200, 255])
def test_batch_sizes(B):
    """One sequence (its pieces follow its own length, not T_cap), 200 and 255
    sequences (four rounds of 64 lanes, the last partial); 256 units fill
    the grid and 257 sequences exceed the list: both keep the fixed splits."""
    T = 1024
    assert _balanced(B, 32, 1, T, 64)
    assert not _balanced(256, 32, 1, T, 64)
    assert not _balanced(257, 32, 1, T, 64)
    lens = [700] if B == 1 else synth.draw_ints(B, 0, T, 12300 + B).tolist()
    q, k, v, sl = _inputs(lens, 32, 1, T, 64, 12301)
    out, lse = L.attn_decode_gqa(q, k, v, sl)
    torch.cuda.synchronize()
    ro, rl = oracle.gqa_decode_ref(q, k, v, sl)
    assert_parity(out, ro, f"balanced B={B}")
    assert_lse(lse, rl, f"balanced B={B}")


@pytest.mark.parametrize("window", [0, 700, 1023])
def test_ring_keeps_fixed_splits(window):
    """Rings keep the fixed splits (visible ranges alike once wrapped): ring
    of 1024 slots, lengths before and far past the wrap, against the oracle."""
    slots = 1024
    lens = [0, 5, 1024, 1500, 100000, 700, 701, 3000]
    heads = np.random.default_rng(12400 + window).integers(0, slots, len(lens)).tolist()
    assert not _balanced(len(lens), 32, 1, slots, 128, window, True)
    q, k, v, sl = _inputs(lens, 32, 1, slots, 128, 12400 + window)
    rh = torch.tensor(heads, dtype=torch.int32, device=DEV)
    out, lse = L.attn_decode_gqa(q, k, v, sl, rh, window)
    torch.cuda.synchronize()
    ro, rl = oracle.gqa_decode_ref(q, k, v, sl, rh, window)
    assert_parity(out, ro, f"balanced ring w={window}")
    assert_lse(lse, rl, "balanced ring")


def test_global_positions():
    """Window plus global positions; sequence 3's query is itself global and
    sees every earlier position."""
    T, window = 2048, 512
    G = [0, 1, 2, 100, 1000]
    lens = [2048, 600, 0, 1001, 3, 1500, 513, 1999]
    assert _balanced(len(lens), 32, 1, T, 64, window, False, len(G))
    q, k, v, sl = _inputs(lens, 32, 1, T, 64, 12500)
    g = torch.tensor(G, dtype=torch.int32, device=DEV)
    out, lse = L.attn_decode_gqa_global(q, k, v, g, window, sl)
    torch.cuda.synchronize()
    ro, rl = oracle.gqa_decode_ref(q, k, v, sl, None, window, global_pos=G)
    assert_parity(out, ro, "balanced global")
    assert_lse(lse, rl, "balanced global")


@pytest.mark.parametrize("Lq,window", [(4, 0), (3, 600)])
def test_multi_token(Lq, window):
    """Several query tokens: 2 KV heads x 16 heads x Lq tokens = two head
    chunks of 32 columns at Lq = 4."""
    T = 2048
    lens = [2048, 3, 0, 1000, 1, 1777]
    assert _balanced(len(lens), 32, 2, T, 128, window, False, 0, Lq)
    q, k, v, sl = _inputs(lens, 32, 2, T, 128, 12600 + Lq, Lq=Lq)
    out, lse = L.attn_decode_gqa_multi(q, k, v, sl, None, window)
    torch.cuda.synchronize()
    ro, rl = oracle.gqa_decode_multi_ref(q, k, v, sl, None, window)
    assert_parity(out, ro, f"balanced multi L={Lq} w={window}")
    assert_lse(lse, rl, "balanced multi")


def test_paged_equals_dense_bitwise():
    """A shuffled pool of 16-position pages: the same list, the same bits as
    the dense cache."""
    T, P = 2048, 16
    lens = [2048, 1, 0, 1500, 17, 385, 2047, 640]
    q, k, v, sl = _inputs(lens, 32, 1, T, 128, 12700)
    B = len(lens)
    npb = T // P
    perm = torch.randperm(B * npb + 3, generator=torch.Generator().manual_seed(12701))
    table = perm[:B * npb].reshape(B, npb).to(torch.int32).to(DEV)

    def pool(x):
        p = torch.full((B * npb + 3, 1, P, 128), float("nan"), dtype=x.dtype, device=DEV)
        p[table.reshape(-1).long()] = x.reshape(B, 1, npb, P, 128).permute(
            0, 2, 1, 3, 4).reshape(B * npb, 1, P, 128)
        return p

    out, lse = L.attn_decode_gqa_paged(q, pool(k), pool(v), table, sl)
    ref_o, ref_l = L.attn_decode_gqa(q, k, v, sl)
    torch.cuda.synchronize()
    assert torch.equal(out, ref_o) and torch.equal(lse, ref_l)
    ro, rl = oracle.gqa_decode_ref(q, k, v, sl)
    assert_parity(out, ro, "balanced paged")


def test_fallbacks_to_fixed_splits():
    """A workspace that holds only the fixed splits' parts runs the fixed
    splits, bit for bit the call with the split count given; an output that
    is not 16-byte aligned runs them too."""
    lens = [2048, 1, 0, 1500, 129, 640]
    B, T, d = len(lens), 2048, 128
    q, k, v, sl = _inputs(lens, 32, 1, T, d, 12800)
    S = L.attn_decode_gqa_splits(B, 32, 1, T, d, 1)
    assert S > 1 and _balanced(B, 32, 1, T, d)
    fixed_o, fixed_l = L.attn_decode_gqa(q, k, v, sl, num_splits=S)
    buf = torch.empty(B * 32 * d + 1, dtype=torch.float32, device=DEV)
    out = buf[1:].view(B, 32, d)
    o1, l1 = L.attn_decode_gqa(q, k, v, sl, out=out)
    # through the C ABI: the binding would grow a small workspace itself
    nb = L.attn_decode_workspace_bytes(B, 32, d, S)
    assert nb < L.attn_decode_gqa_workspace_bytes(B, 32, 1, T, d, 1)
    ws = torch.empty(nb, dtype=torch.uint8, device=DEV)
    o2 = torch.empty_like(fixed_o)
    l2 = torch.empty_like(fixed_l)
    st = L.library().attn_decode_gqa(
        L._ptr(q), L._ptr(k), L._ptr(v), L._ptr(o2), L._ptr(l2), L._ptr(sl), None,
        B, 32, 1, T, d, 1, 0, 0.0, 0, L._ptr(ws), nb, L._stream(None, q.device))
    assert st == 0
    torch.cuda.synchronize()
    # the unaligned output also takes the merge's scalar form (another order
    # of the sums), so it is held to the oracle rather than to the bits
    ro, rl = oracle.gqa_decode_ref(q, k, v, sl)
    assert_parity(o1, ro, "unaligned out")
    assert_lse(l1, rl, "unaligned out")
    assert torch.equal(o2, fixed_o) and torch.equal(l2, fixed_l)


def test_graph_replays_follow_new_lengths():
    """The list is built on the device from seq_lens, so a captured call
    replays correctly after the lengths change (no host read of the lengths;
    only kernels are captured).  Eager work runs between the replays, and
    every replay is checked against the oracle."""
    T, d = 2048, 128
    lens0 = [2048, 1, 0, 1500, 129, 640, 2047, 300]
    B = len(lens0)
    q, k, v, sl = _inputs(lens0, 32, 1, T, d, 12900)
    assert _balanced(B, 32, 1, T, d)
    out = torch.empty(B, 32, d, dtype=torch.float32, device=DEV)
    lse = torch.empty(B, 32, dtype=torch.float32, device=DEV)
    ws = torch.empty(L.attn_decode_gqa_workspace_bytes(B, 32, 1, T, d, 1), dtype=torch.uint8,
                     device=DEV)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # warm up off the default stream, as capture requires
        L.attn_decode_gqa(q, k, v, sl, out=out, lse=lse, workspace=ws)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        L.attn_decode_gqa(q, k, v, sl, out=out, lse=lse, workspace=ws)
    torch.cuda.synchronize()
    for trial, lens in enumerate([lens0, [5, 2048, 2048, 0, 0, 17, 1000, 1],
                                  [0] * B, [2048] * B]):
        sl.copy_(torch.tensor(lens, dtype=torch.int32))
        out.fill_(float("nan"))
        graph.replay()
        torch.cuda.synchronize()
        ro, rl = oracle.gqa_decode_ref(q, k, v, sl)
        assert_parity(out, ro, f"replay {trial}")
        assert_lse(lse, rl, f"replay {trial}")


# ------------------------------------------------------------ absorbed MLA
MLA_GEOMS = [(512, 128), (256, 32)]  # (d_c, heads); d_rope = 64


@pytest.mark.parametrize("d_c,H", MLA_GEOMS, ids=[f"dc{a}-H{b}" for a, b in MLA_GEOMS])
@pytest.mark.parametrize("mix", ["extreme", "one_long", "all_empty", "all_one_piece"])
def test_mla_length_mixes(d_c, H, mix):
    """The MLA kernel takes the same list (pieces of whole 32-row tiles);
    against the oracle and against the fixed splits."""
    lens = MIXES[mix]
    B, T, dk = len(lens), 2048, d_c + 64
    q = synth.draw((B, H, dk), 13000 + d_c + len(mix), "bf16", DEV, dk ** -0.5)
    lat = synth.draw((B, T, dk), 13001 + d_c + len(mix), "bf16", DEV, dk ** -0.5)
    sl = torch.tensor(lens, dtype=torch.int32, device=DEV)
    scale = 192 ** -0.5
    z, lse = L.attn_decode_mla(q, lat, d_c, scale, sl)
    torch.cuda.synchronize()
    rz, rl = oracle.mla_decode_ref(q, lat, d_c, scale, sl)
    assert_parity(z, rz, f"mla balanced {mix} d_c={d_c}")
    assert_lse(lse, rl, f"mla balanced {mix}")
    S = L.attn_decode_mla_splits(B, H, T, d_c, 64)
    assert S > 1
    zf, _ = L.attn_decode_mla(q, lat, d_c, scale, sl, S)
    torch.cuda.synchronize()
    assert_parity(zf, rz, f"mla fixed {mix}")


@pytest.mark.parametrize("mix", list(EVEN_MIXES))
def test_mla_even_split_segments(mix):
    """The (512, 64) geometry runs the even split for one token per sequence:
    a group may compute pieces of several sequences, each restarting the
    group's tile pipeline; dense and paged pools give the same bits, and a
    second call on the same workspace with other lengths must not see the
    first call's slots or pairs."""
    from test_gpu_paged import _latent_pool
    lens = EVEN_MIXES[mix]
    B, T, H, dk = len(lens), 4096, 128, 576
    q = synth.draw((B, H, dk), 13200 + B, "bf16", DEV, dk ** -0.5)
    lat = synth.draw((B, T, dk), 13201 + B, "bf16", DEV, dk ** -0.5)
    sl = torch.tensor(lens, dtype=torch.int32, device=DEV)
    scale = 192 ** -0.5
    ws = torch.empty(L.attn_decode_mla_workspace_bytes(B, H, T, 512, 64),
                     dtype=torch.uint8, device=DEV)
    z, lse = L.attn_decode_mla(q, lat, 512, scale, sl, workspace=ws)
    torch.cuda.synchronize()
    rz, rl = oracle.mla_decode_ref(q, lat, 512, scale, sl)
    assert_parity(z, rz, f"mla even split {mix}")
    assert_lse(lse, rl, f"mla even split {mix}")
    pool, table = _latent_pool(lat, 64, 13202 + B, poison=True)
    zp, lp = L.attn_decode_mla_paged(q, pool, table, 512, scale, sl)
    torch.cuda.synchronize()
    assert torch.equal(zp, z) and torch.equal(lp, lse)
    sl2 = torch.flip(sl, [0]).contiguous()
    z2, l2 = L.attn_decode_mla(q, lat, 512, scale, sl2, workspace=ws)
    torch.cuda.synchronize()
    rz2, rl2 = oracle.mla_decode_ref(q, lat, 512, scale, sl2)
    assert_parity(z2, rz2, f"mla even split {mix}, second call")
    assert_lse(l2, rl2, f"mla even split {mix}, second call")


@pytest.mark.parametrize("seed", range(6))
def test_mla_even_split_random(seed):
    """Seeded random ragged batches on the (512, 64) geometry's even split
    (1 to 130 sequences, empty and one-row ones mixed, 32 or 128 heads)."""
    rng = np.random.default_rng(33000 + seed)
    B = int(rng.choice([1, 3, 17, 64, 130]))
    H = int(rng.choice([32, 128]))
    T, dk = 2048, 576
    kinds = rng.integers(0, 4, size=B)
    lens = np.where(kinds == 0, 0, np.where(kinds == 1, rng.integers(1, 40, size=B),
                                            rng.integers(1, T + 1, size=B))).astype(int)
    q = synth.draw((B, H, dk), 33100 + seed, "bf16", DEV, dk ** -0.5)
    lat = synth.draw((B, T, dk), 33200 + seed, "bf16", DEV, dk ** -0.5)
    sl = torch.tensor(lens.tolist(), dtype=torch.int32, device=DEV)
    scale = 192 ** -0.5
    z, lse = L.attn_decode_mla(q, lat, 512, scale, sl)
    torch.cuda.synchronize()
    rz, rl = oracle.mla_decode_ref(q, lat, 512, scale, sl)
    what = f"mla seed {seed}: B={B} H={H}"
    print(what, flush=True)
    assert_parity(z, rz, what)
    assert_lse(lse, rl, what)


def test_mla_paged_and_multi_token():
    """Paged latent pool (16-position pages): the same bits as the dense
    cache; three query tokens per sequence (three head chunks at 128 heads)
    against the oracle."""
    from test_gpu_paged import _latent_pool
    lens = [2048, 1, 0, 1500, 17, 385, 2047, 640]
    B, T, H = len(lens), 2048, 128
    q = synth.draw((B, 3, H, 576), 13100, "bf16", DEV, 576 ** -0.5)
    lat = synth.draw((B, T, 576), 13101, "bf16", DEV, 576 ** -0.5)
    sl = torch.tensor(lens, dtype=torch.int32, device=DEV)
    scale = 192 ** -0.5
    pool, table = _latent_pool(lat, 16, 13102, poison=True)
    zp, lp = L.attn_decode_mla_paged(q, pool, table, 512, scale, sl)
    zd, ld = L.attn_decode_mla_multi(q, lat, 512, scale, sl)
    torch.cuda.synchronize()
    assert torch.equal(zp, zd) and torch.equal(lp, ld)
    rz, rl = oracle.mla_decode_multi_ref(q, lat, 512, scale, sl)
    assert_parity(zd, rz, "mla balanced multi")
    assert_lse(ld, rl, "mla balanced multi")
