"""Pins of the CPU reference (``oracle/``) to things other than itself.

Each ``check_*`` function states one fact fixed by the pages or by the
mathematics and raises AssertionError if the reference disagrees.  The
``test_*`` functions run them; ``test_planted_*`` plants a plausible mistake
in the reference (on the CPU, through monkeypatch) and asserts that at least
one pin catches it.
"""

import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
from oracle import attention as A
from oracle import bruteforce as BF

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _rng(seed):
    return np.random.default_rng(seed)


# ---------------------------------------------------------------- byte sizes
def check_kv_bytes_golden():
    g = json.load(open(os.path.join(GOLD, "kv_bytes.json")))
    for e in g["kv"]:
        got = oracle.kv_cache_bytes(e["B"], e["T"], e["H_kv"], e["d"], e["s"],
                                    e["layers"])
        assert got == e["bytes"], (e["cite"], got)
    for e in g["mla"]:
        got = oracle.mla_cache_bytes(e["B"], e["T"], e["r"], e["d_rope"], e["s"])
        assert got == e["bytes"], (e["cite"], got)
    for e in g["mla_explicit"]:
        got = oracle.mla_explicit_cache_bytes(e["B"], e["T"], e["H"], e["d_c"],
                                              e["d_rope"], e["d_v"], e["s"])
        assert got == e["bytes"], (e["cite"], got)
    el = g["mla_elements_per_token"]
    lat = oracle.mla_cache_bytes(1, 1, 512, 64, 1)
    exp = oracle.mla_explicit_cache_bytes(1, 1, 128, 128, 64, 128, 1)
    assert lat == el[0]["value"] and exp == el[1]["value"]
    assert round(exp / lat, 1) == el[2]["value"]


def test_kv_bytes_golden():
    check_kv_bytes_golden()


def test_astro_blog_printed_sizes_are_half_its_formula():
    """The astro-blog helper multiplies T*H*d*2*dtype_bytes (K and V, bf16)
    but its printed results (32/8/1 MB for 4096 tokens, 32/8/1 heads, d=128)
    are half of that; the reference follows the formula, which agrees with
    attention-head section 1 and the llmdeepdive accounting."""
    printed_mb = {32: 32, 8: 8, 1: 1}
    for h, mb in printed_mb.items():
        got = oracle.kv_cache_bytes(1, 4096, h, 128, 2) / 2**20
        assert got == 2 * mb


# -------------------------------------------------------------- visibility
def check_window_golden():
    g = json.load(open(os.path.join(GOLD, "window_example.json")))
    for e in g["cases"]:
        got = oracle.visible_positions(e["T_b"], e["window"]).tolist()
        assert got == e["visible"], (e["cite"], got)
        bf = [p for _, p in BF.visible_slots_brute(e["T_b"], e["T_b"] + 4,
                                                    e["window"])]
        assert bf == e["visible"], (e["cite"], bf)


def test_window_golden():
    check_window_golden()


def check_ring_hand_enumerated():
    """Ring of 4 slots, newest position t=5 in slot 1.  Walking back from the
    head: slot 1 -> 5, slot 0 -> 4, slot 3 -> 3, slot 2 -> 2 (enumerated by
    hand); positions 0 and 1 were overwritten."""
    pos = oracle.visible_positions(6, 0, ring_capacity=4).tolist()
    assert pos == [2, 3, 4, 5], pos
    slots = oracle.ring_slot(np.array(pos), 5, 1, 4).tolist()
    assert slots == [2, 3, 0, 1], slots
    # window 2 inside the same ring: positions 4, 5 in slots 0, 1
    pos = oracle.visible_positions(6, 2, ring_capacity=4).tolist()
    assert pos == [4, 5]
    # not yet wrapped: T_b=3 with head at slot 3 -> positions 0,1,2 in slots 1,2,3
    pos = oracle.visible_positions(3, 0, ring_capacity=4).tolist()
    assert pos == [0, 1, 2]
    assert oracle.ring_slot(np.array(pos), 2, 3, 4).tolist() == [1, 2, 3]
    bf = BF.visible_slots_brute(6, 4, 0, ring_head=1)
    assert bf == [(2, 2), (3, 3), (0, 4), (1, 5)], bf


def test_ring_hand_enumerated():
    check_ring_hand_enumerated()


# ------------------------------------------------------------- brute force
def _tiny_case(rng, B, H_q, H_kv, T_cap, d, d_v=None, ring=False, ragged=True):
    d_v = d if d_v is None else d_v
    q = rng.standard_normal((B, H_q, d))
    k = rng.standard_normal((B, H_kv, T_cap, d))
    v = rng.standard_normal((B, H_kv, T_cap, d_v))
    if ring:
        lens = rng.integers(0, 3 * T_cap, size=B)
        heads = rng.integers(0, T_cap, size=B)
    else:
        lens = rng.integers(0, T_cap + 1, size=B) if ragged else np.full(B, T_cap)
        heads = None
    return q, k, v, lens, heads


def check_brute_force(seed=0, n_cases=60):
    rng = _rng(seed)
    combos = [(1, 1), (2, 1), (4, 2), (6, 3), (8, 2), (8, 8), (6, 1), (4, 4)]
    for c in range(n_cases):
        H_q, H_kv = combos[c % len(combos)]
        B = 1 + c % 2
        T_cap = int(rng.integers(1, 25))
        d = int(rng.choice([2, 4, 8]))
        ring = bool(c % 3 == 2)
        window = int(rng.choice([0, 1, 2, 3, 5, T_cap]))
        if ring:
            window = min(window, T_cap)
        q, k, v, lens, heads = _tiny_case(rng, B, H_q, H_kv, T_cap, d, ring=ring)
        scale = float(rng.choice([0.3, 1.0 / math.sqrt(d), 2.0]))
        o, l = oracle.gqa_decode_ref(q, k, v, lens, heads, window, scale)
        ob, lb = BF.gqa_decode_brute(q, k, v, lens, heads, window, scale)
        ob, lb = np.array(ob), np.array(lb)
        assert np.array_equal(np.isinf(l), np.isinf(lb)), c
        assert np.allclose(o, ob, rtol=0, atol=1e-12), c
        fin = np.isfinite(l)
        assert np.allclose(l[fin], lb[fin], rtol=0, atol=1e-12), c


def test_brute_force_agreement():
    check_brute_force()


def check_mla_brute_force(seed=1):
    rng = _rng(seed)
    for c in range(12):
        B, H, T = 1 + c % 2, int(rng.integers(1, 5)), int(rng.integers(1, 12))
        d_c, d_r = int(rng.choice([2, 4, 6])), int(rng.choice([1, 2, 3]))
        q = rng.standard_normal((B, H, d_c + d_r))
        lat = rng.standard_normal((B, T, d_c + d_r))
        lens = rng.integers(0, T + 1, size=B)
        z, l = oracle.mla_decode_ref(q, lat, d_c, 0.7, lens)
        zb, lb = BF.mla_decode_brute(q, lat, d_c, 0.7, lens)
        assert np.allclose(z, np.array(zb), atol=1e-12)
        lb = np.array(lb)
        assert np.array_equal(np.isinf(l), np.isinf(lb))
        fin = np.isfinite(l)
        assert np.allclose(l[fin], lb[fin], atol=1e-12)


def test_mla_brute_force_agreement():
    check_mla_brute_force()


# --------------------------------------------------------- closed forms
def check_identical_keys_give_mean(seed=2):
    """All keys equal -> every visible weight is 1/n_vis -> output is the mean
    of the visible values, lse = s + ln(n_vis) (from the attention equation)."""
    rng = _rng(seed)
    for ring in (False, True):
        for window in (0, 1, 3, 7):
            B, H_q, H_kv, T_cap, d = 2, 4, 2, 12, 4
            q = rng.standard_normal((B, H_q, d))
            krow = rng.standard_normal(d)
            k = np.broadcast_to(krow, (B, H_kv, T_cap, d)).copy()
            v = rng.standard_normal((B, H_kv, T_cap, d))
            lens = np.array([5, 30]) if ring else np.array([5, 12])
            heads = np.array([3, 7]) if ring else None
            o, l = oracle.gqa_decode_ref(q, k, v, lens, heads, window, 0.5)
            for b in range(B):
                sl = BF.visible_slots_brute(int(lens[b]), T_cap, window,
                                            None if heads is None else int(heads[b]))
                slots = [s for s, _ in sl]
                for h in range(H_q):
                    g = h // (H_q // H_kv)
                    mean = v[b, g, slots].mean(axis=0)
                    assert np.allclose(o[b, h], mean, atol=1e-13), (ring, window)
                    s = 0.5 * q[b, h] @ krow
                    assert abs(l[b, h] - (s + math.log(len(slots)))) < 1e-12


def test_identical_keys_give_mean():
    check_identical_keys_give_mean()


def check_single_visible_key(seed=3):
    """One visible key -> weight exactly 1 -> output equals that value row."""
    rng = _rng(seed)
    q = rng.standard_normal((1, 4, 8))
    k = rng.standard_normal((1, 2, 10, 8))
    v = rng.standard_normal((1, 2, 10, 8))
    o, _ = oracle.gqa_decode_ref(q, k, v, np.array([1]))          # T_b = 1
    assert np.array_equal(o[0, :2], np.repeat(v[0, 0, :1], 2, 0))
    assert np.array_equal(o[0, 2:], np.repeat(v[0, 1, :1], 2, 0))
    o, _ = oracle.gqa_decode_ref(q, k, v, np.array([7]), window=1)  # w = 1
    assert np.array_equal(o[0, 0], v[0, 0, 6]) and np.array_equal(o[0, 3], v[0, 1, 6])
    o, _ = oracle.gqa_decode_ref(q, k, v, np.array([25]), np.array([4]), window=1)
    assert np.array_equal(o[0, 1], v[0, 0, 4]) and np.array_equal(o[0, 2], v[0, 1, 4])


def test_single_visible_key():
    check_single_visible_key()


def check_two_key_closed_form(seed=4):
    """Two visible keys: weights are the logistic of the score difference,
    evaluated here in its overflow-free form for large score gaps."""
    rng = _rng(seed)
    for scale in (0.1, 1.0, 100.0, 1e4):
        q = rng.standard_normal((1, 1, 3))
        k = rng.standard_normal((1, 1, 2, 3))
        v = rng.standard_normal((1, 1, 2, 3))
        o, l = oracle.gqa_decode_ref(q, k, v, scale=scale)
        s0, s1 = scale * q[0, 0] @ k[0, 0, 0], scale * q[0, 0] @ k[0, 0, 1]
        x = s0 - s1
        w0 = 1 / (1 + math.exp(-x)) if x >= 0 else math.exp(x) / (1 + math.exp(x))
        want = w0 * v[0, 0, 0] + (1 - w0) * v[0, 0, 1]
        assert np.allclose(o[0, 0], want, rtol=1e-12, atol=1e-12), scale
        big = max(s0, s1)
        want_l = big + math.log1p(math.exp(-abs(x)))
        assert abs(l[0, 0] - want_l) <= 1e-12 * max(1.0, abs(want_l)), scale


def test_two_key_closed_form():
    check_two_key_closed_form()


def test_large_scores_stay_finite():
    """Scale 100 on N(0,1) data: scores reach the hundreds; the reference must
    not overflow and must agree with the scalar loops."""
    rng = _rng(5)
    q, k, v, lens, _ = _tiny_case(rng, 2, 4, 2, 20, 8, ragged=False)
    o, l = oracle.gqa_decode_ref(q, k, v, lens, scale=100.0)
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(l))
    ob, lb = BF.gqa_decode_brute(q, k, v, lens, scale=100.0)
    assert np.allclose(o, ob, atol=1e-12) and np.allclose(l, lb, rtol=1e-14)


def test_empty_visible_set():
    q = np.ones((2, 2, 4))
    k = np.ones((2, 1, 5, 4))
    v = np.ones((2, 1, 5, 4))
    o, l = oracle.gqa_decode_ref(q, k, v, np.array([0, 3]))
    assert np.all(o[0] == 0) and np.all(np.isneginf(l[0]))
    assert np.allclose(o[1], 1.0) and np.all(np.isfinite(l[1]))


# ---------------------------------------------------- reductions / invariants
def check_repeat_kv_equivalence(seed=6):
    """GQA equals MHA on K/V whose heads are repeated n times in a row (the
    toolsku ``_repeat_kv`` expansion)."""
    rng = _rng(seed)
    for H_q, H_kv in ((8, 2), (6, 3), (4, 1), (24, 4)):
        n = H_q // H_kv
        q, k, v, lens, _ = _tiny_case(rng, 2, H_q, H_kv, 16, 8)
        o, l = oracle.gqa_decode_ref(q, k, v, lens, window=5)
        kr = np.repeat(k, n, axis=1)
        vr = np.repeat(v, n, axis=1)
        o2, l2 = oracle.gqa_decode_ref(q, kr, vr, lens, window=5)
        assert np.allclose(o, o2, atol=1e-13) and np.allclose(l, l2, atol=1e-13)


def test_repeat_kv_equivalence():
    check_repeat_kv_equivalence()


def check_mqa_and_mha_degenerate(seed=7):
    """MQA (one KV head) equals MHA whose KV heads are all that head; GQA with
    as many KV heads as query heads is MHA, head by head."""
    rng = _rng(seed)
    q, k, v, lens, _ = _tiny_case(rng, 2, 6, 1, 10, 4)
    o, _ = oracle.gqa_decode_ref(q, k, v, lens)
    o2, _ = oracle.gqa_decode_ref(q, np.repeat(k, 6, 1), np.repeat(v, 6, 1), lens)
    assert np.allclose(o, o2, atol=1e-13)
    q, k, v, lens, _ = _tiny_case(rng, 1, 3, 3, 10, 4)
    o, _ = oracle.gqa_decode_ref(q, k, v, lens)
    for h in range(3):
        oh, _ = oracle.gqa_decode_ref(q[:, h:h + 1], k[:, h:h + 1], v[:, h:h + 1], lens)
        assert np.allclose(o[:, h], oh[:, 0], atol=1e-13)


def test_mqa_and_mha_degenerate():
    check_mqa_and_mha_degenerate()


def check_torch_sdpa(seed=8):
    """Compare with torch's own scaled_dot_product_attention (float64, CPU,
    grouped heads, boolean visibility mask): an independent library routine."""
    rng = _rng(seed)
    for H_q, H_kv, window in ((8, 2, 0), (6, 3, 4), (4, 4, 0), (4, 1, 2)):
        q, k, v, lens, _ = _tiny_case(rng, 2, H_q, H_kv, 18, 8, ragged=False)
        lens = np.array([18, 11])
        o, _ = oracle.gqa_decode_ref(q, k, v, lens, window=window, scale=0.4)
        mask = np.zeros((2, 1, 1, 18), dtype=bool)
        for b in range(2):
            t = lens[b] - 1
            for j in range(18):
                mask[b, 0, 0, j] = j <= t and (window == 0 or t - j < window)
        ref = torch.nn.functional.scaled_dot_product_attention(
            torch.from_numpy(q)[:, :, None, :], torch.from_numpy(k),
            torch.from_numpy(v), attn_mask=torch.from_numpy(mask),
            scale=0.4, enable_gqa=True)[:, :, 0, :].numpy()
        assert np.allclose(o, ref, atol=1e-12), (H_q, H_kv, window)


def test_torch_sdpa():
    check_torch_sdpa()


def check_split_invariance(seed=9):
    """Results over disjoint parts of the key set, merged by the log-sum-exp
    rule, equal the single pass -- for any partition, empty parts included."""
    rng = _rng(seed)
    for trial in range(20):
        n, m, d = 3, int(rng.integers(1, 40)), 5
        qr = rng.standard_normal((n, d))
        kr = rng.standard_normal((m, d))
        vr = rng.standard_normal((m, d))
        o, l = A.attend(qr, kr, vr, 0.6)
        S = int(rng.integers(1, 9))
        cuts = np.sort(rng.integers(0, m + 1, size=S - 1))
        bounds = [0, *cuts.tolist(), m]
        perm = rng.permutation(m) if trial % 2 else np.arange(m)
        op, lp = [], []
        for s in range(S):
            idx = perm[bounds[s]:bounds[s + 1]]
            a, b = oracle.partial_ref(qr, kr[idx], vr[idx], 0.6)
            op.append(a)
            lp.append(b)
        op = np.stack(op, axis=1)[None]      # [1, n, S, d]
        lp = np.stack(lp, axis=1)[None]      # [1, n, S]
        oc, lc = oracle.combine_ref(op, lp)
        assert np.allclose(oc[0], o, atol=1e-13) and np.allclose(lc[0], l, atol=1e-13)
        ob, lb = BF.combine_brute(op, lp)
        assert np.allclose(np.array(ob)[0], o, atol=1e-13)
        assert np.allclose(np.array(lb)[0], l, atol=1e-13)
    oc, lc = oracle.combine_ref(np.ones((1, 1, 3, 2)), np.full((1, 1, 3), -np.inf))
    assert np.all(oc == 0) and np.all(np.isneginf(lc))


def test_split_invariance():
    check_split_invariance()


def check_ring_equals_linear(seed=10):
    """A ring cache unrolled into a linear cache gives the same result; the
    unrolling here places position j at index j directly from the slot walk."""
    rng = _rng(seed)
    for trial in range(30):
        cap = int(rng.integers(1, 12))
        T_b = int(rng.integers(0, 3 * cap + 2))
        head = int(rng.integers(0, cap))
        window = int(rng.choice([0, 1, 2, cap]))
        window = min(window, cap)
        q = rng.standard_normal((1, 2, 4))
        k = rng.standard_normal((1, 1, cap, 4))
        v = rng.standard_normal((1, 1, cap, 4))
        o, l = oracle.gqa_decode_ref(q, k, v, np.array([T_b]), np.array([head]),
                                     window)
        L = max(T_b, 1)
        kl = np.full((1, 1, L, 4), 1e6)       # positions no longer resident
        vl = np.full((1, 1, L, 4), np.nan)
        for slot, pos in BF.visible_slots_brute(T_b, cap, 0, ring_head=head):
            kl[0, 0, pos] = k[0, 0, slot]
            vl[0, 0, pos] = v[0, 0, slot]
        o2, l2 = oracle.gqa_decode_ref(q, kl, vl, np.array([T_b]),
                                       window=window if window else cap)
        assert np.allclose(o, o2, atol=1e-13, equal_nan=False), trial
        assert np.allclose(l, l2, atol=1e-13), trial


def test_ring_equals_linear():
    check_ring_equals_linear()


def check_integer_recovery(seed=11):
    """Index logic to the bit: zero keys make every visible weight exactly
    1/n_vis, and V[slot, i] = bit i of the logical position in that slot (last
    column 1).  Then out[i] * n_vis rounds to the count of visible positions
    with bit i set and exp(lse) to n_vis -- integers fixed by counting."""
    rng = _rng(seed)
    d = 16
    for trial in range(40):
        ring = trial % 2 == 1
        cap = int(rng.integers(1, 200))
        T_b = int(rng.integers(0, 3 * cap + 1)) if ring else int(rng.integers(0, cap + 1))
        window = int(rng.choice([0, 1, 7, cap]))
        if ring:
            window = min(window, cap)
        head = int(rng.integers(0, cap)) if ring else None
        k = np.zeros((1, 1, cap, d))
        v = np.zeros((1, 1, cap, d))
        for slot in range(cap):
            pos = BF._slot_position(slot, T_b - 1, head, cap) if ring else slot
            for i in range(d - 1):
                v[0, 0, slot, i] = (pos >> i) & 1 if pos >= 0 else 0
            v[0, 0, slot, d - 1] = 1.0
        q = rng.standard_normal((1, 1, d))
        o, l = oracle.gqa_decode_ref(q, k, v, np.array([T_b]),
                                     None if head is None else np.array([head]), window)
        t = T_b - 1
        lo = 0 if not window else t - window + 1
        if ring:
            lo = max(lo, T_b - cap)
        want = list(range(max(lo, 0), t + 1))
        n_vis = len(want)
        if n_vis == 0:
            assert np.all(o == 0) and np.isneginf(l[0, 0])
            continue
        counts = [sum((p >> i) & 1 for p in want) for i in range(d - 1)] + [n_vis]
        got = np.rint(o[0, 0] * n_vis).astype(int).tolist()
        assert got == counts, (trial, got, counts)
        assert int(round(math.exp(l[0, 0]))) == n_vis


def test_integer_recovery():
    check_integer_recovery()


# ----------------------------------------------------------------- MLA pins
def check_mla_absorbed_equals_explicit(seed=12):
    """Absorbed MLA (query times U_K^T against the latent, values projected
    after the weighted sum) equals explicit per-head K/V attention
    [attention-head sections 5.2-5.3], with scale 1/sqrt(d_c_head + d_R)."""
    rng = _rng(seed)
    B, T, H, r, dch, dR, dv = 2, 9, 3, 16, 6, 4, 5
    C = rng.standard_normal((B, T, r))
    KR = rng.standard_normal((B, T, dR))
    qc = rng.standard_normal((B, H, dch))
    qr = rng.standard_normal((B, H, dR))
    UK = rng.standard_normal((H, r, dch))
    UV = rng.standard_normal((H, r, dv))
    scale = 1 / math.sqrt(dch + dR)
    explicit = oracle.mla_explicit_ref(C, KR, qc, qr, UK, UV, scale)
    qt = np.einsum("bhc,hrc->bhr", qc, UK)            # q~ = q^C U_K^T
    q = np.concatenate([qt, qr], axis=2)
    lat = np.concatenate([C, KR], axis=2)
    z, _ = oracle.mla_decode_ref(q, lat, r, scale)
    absorbed = np.einsum("bhr,hrv->bhv", z, UV)        # o = z U_V
    assert np.allclose(absorbed, explicit, atol=1e-12, rtol=1e-12)


def test_mla_absorbed_equals_explicit():
    check_mla_absorbed_equals_explicit()


def check_mla_is_shared_head_attention(seed=13):
    """MLA decode is the single-KV-head attention with K = the whole latent
    row and V = its first d_c columns."""
    rng = _rng(seed)
    q = rng.standard_normal((2, 4, 10))
    lat = rng.standard_normal((2, 7, 10))
    lens = np.array([7, 3])
    z, l = oracle.mla_decode_ref(q, lat, 8, 0.3, lens)
    o, l2 = oracle.gqa_decode_ref(q, lat[:, None], lat[:, None, :, :8], lens,
                                  scale=0.3)
    assert np.allclose(z, o, atol=1e-13) and np.allclose(l, l2, atol=1e-13)


def test_mla_is_shared_head_attention():
    check_mla_is_shared_head_attention()


# ------------------------------------------------------ planted mistakes
ALL_CHECKS = [
    check_kv_bytes_golden, check_window_golden, check_ring_hand_enumerated,
    check_brute_force, check_mla_brute_force, check_identical_keys_give_mean,
    check_single_visible_key, check_two_key_closed_form,
    check_repeat_kv_equivalence, check_mqa_and_mha_degenerate, check_torch_sdpa,
    check_split_invariance, check_ring_equals_linear, check_integer_recovery,
    check_mla_absorbed_equals_explicit, check_mla_is_shared_head_attention,
]


def _caught():
    for chk in ALL_CHECKS:
        try:
            chk()
        except (AssertionError, ValueError, IndexError):
            return True
    return False


MUTANTS = {
    "group_interleaved": ("_kv_head_for_query", lambda h, n: h % max(1, n)),
    "window_off_by_one": ("_window_low", lambda t, w: max(0, t - w) if w > 0 else 0),
    "window_too_narrow": ("_window_low", lambda t, w: max(0, t - w + 2) if w > 0 else 0),
    "ring_wrong_direction": ("ring_slot",
                             lambda p, t, h, c: (h + (t - np.asarray(p))) % c),
    "kv_bytes_no_factor_2": ("kv_cache_bytes",
                             lambda B, T, H, d, s, layers=1: B * T * H * d * s * layers),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_index_mistakes_are_caught(monkeypatch, name):
    attr, fn = MUTANTS[name]
    monkeypatch.setattr(A, attr, fn)
    if attr == "kv_cache_bytes":
        monkeypatch.setattr(oracle, attr, fn)
    if attr == "ring_slot":
        monkeypatch.setattr(oracle, attr, fn)
    assert _caught(), name


def _attend_no_max(q_rows, k_rows, v_rows, scale):
    q_rows, k_rows, v_rows = (np.asarray(x, float) for x in (q_rows, k_rows, v_rows))
    if k_rows.shape[0] == 0:
        return np.zeros((q_rows.shape[0], v_rows.shape[1])), np.full(q_rows.shape[0], -np.inf)
    with np.errstate(over="ignore", invalid="ignore"):
        p = np.exp(scale * q_rows @ k_rows.T)
        l = p.sum(1, keepdims=True)
        return (p @ v_rows) / l, np.log(l)[:, 0]


def _attend_wrong_sign(q_rows, k_rows, v_rows, scale):
    o, l = oracle.partial_ref(q_rows, -np.asarray(k_rows), v_rows, scale)
    return o, l


def _attend_no_scale(q_rows, k_rows, v_rows, scale):
    return oracle.partial_ref(q_rows, k_rows, v_rows, 1.0)


def _attend_transposed_value(q_rows, k_rows, v_rows, scale):
    v = np.asarray(v_rows, float)
    return oracle.partial_ref(q_rows, k_rows, v[::-1], scale)


@pytest.mark.parametrize("mutant", [_attend_no_max, _attend_wrong_sign,
                                    _attend_no_scale, _attend_transposed_value])
def test_planted_arithmetic_mistakes_are_caught(monkeypatch, mutant):
    # partial_ref keeps the true definition so that the mutant differs from it
    true_attend = A.attend
    monkeypatch.setattr(A, "partial_ref", true_attend)
    monkeypatch.setattr(oracle, "partial_ref", true_attend)
    monkeypatch.setattr(A, "attend", mutant)
    assert _caught(), mutant.__name__


def test_planted_mla_value_columns_are_caught(monkeypatch):
    orig = A.mla_decode_ref

    def wrong(q, latent, d_c, scale, seq_lens=None, batches=None):
        lat = np.asarray(latent, float)
        rolled = np.concatenate([lat[..., -d_c:], lat[..., :-d_c]], axis=-1)
        z, l = orig(q, lat, d_c, scale, seq_lens, batches)
        z2, _ = orig(q, rolled, d_c, scale, seq_lens, batches)
        return z2 if lat.shape[-1] > d_c else z, l

    monkeypatch.setattr(A, "mla_decode_ref", wrong)
    monkeypatch.setattr(oracle, "mla_decode_ref", wrong)
    assert _caught()


# ------------------------------------------------------------- cache append
def check_append_then_decode_equals_concat(seed=14):
    """Appending the new token's K/V and decoding equals decoding over the
    past cache concatenated with the new row (toolsku modules: torch.cat of
    past_kv and the new k, v along the sequence axis)."""
    rng = _rng(seed)
    B, H_q, H_kv, T_cap, d = 2, 4, 2, 12, 4
    past = np.array([5, 9])
    k = rng.standard_normal((B, H_kv, T_cap, d))
    v = rng.standard_normal((B, H_kv, T_cap, d))
    kn = rng.standard_normal((B, H_kv, d))
    vn = rng.standard_normal((B, H_kv, d))
    q = rng.standard_normal((B, H_q, d))
    k2 = oracle.kv_append_ref(k, kn, past)
    v2 = oracle.kv_append_ref(v, vn, past)
    o, l = oracle.gqa_decode_ref(q, k2, v2, past + 1)
    for b in range(B):
        kc = np.concatenate([k[b, :, :past[b]], kn[b][:, None]], axis=1)[None]
        vc = np.concatenate([v[b, :, :past[b]], vn[b][:, None]], axis=1)[None]
        ob, lb = oracle.gqa_decode_ref(q[b:b + 1], kc, vc)
        assert np.allclose(o[b], ob[0], atol=1e-13) and np.allclose(l[b], lb[0], atol=1e-13)
    # out-of-range positions are not written
    assert np.array_equal(oracle.kv_append_ref(k, kn, np.array([T_cap, -1])), k)


def test_append_then_decode_equals_concat():
    check_append_then_decode_equals_concat()


def check_ring_append_sequence(seed=15):
    """A long run of ring appends + windowed decode equals decoding the full
    linear history with the same window, at every step."""
    rng = _rng(seed)
    cap, d, steps, w = 5, 3, 13, 4
    hist_k = rng.standard_normal((steps, d))
    hist_v = rng.standard_normal((steps, d))
    q = rng.standard_normal((1, 2, d))
    ring_k = np.zeros((1, 1, cap, d))
    ring_v = np.zeros((1, 1, cap, d))
    head = np.array([cap - 1])        # empty ring: the first append lands in slot 0
    for t in range(steps):
        ring_k, _ = oracle.kv_append_ring_ref(ring_k, hist_k[t][None, None], head)
        ring_v, head = oracle.kv_append_ring_ref(ring_v, hist_v[t][None, None], head)
        o, l = oracle.gqa_decode_ref(q, ring_k, ring_v, np.array([t + 1]), head, w)
        lin_k = hist_k[None, None, :t + 1]
        lin_v = hist_v[None, None, :t + 1]
        o2, l2 = oracle.gqa_decode_ref(q, lin_k, lin_v, np.array([t + 1]), window=w)
        assert np.allclose(o, o2, atol=1e-13) and np.allclose(l, l2, atol=1e-13), t


def test_ring_append_sequence():
    check_ring_append_sequence()


ALL_CHECKS += [check_append_then_decode_equals_concat, check_ring_append_sequence]


def test_planted_append_off_by_one_is_caught(monkeypatch):
    orig = oracle.kv_append_ref

    def shifted(cache, new_rows, positions):
        return orig(cache, new_rows, np.asarray(positions) + 1)

    monkeypatch.setattr(oracle, "kv_append_ref", shifted)
    assert _caught()


# ------------------------------------------------------------ global tokens
def check_global_golden():
    g = json.load(open(os.path.join(GOLD, "window_example.json")))
    for e in g["global_cases"]:
        got = oracle.visible_positions(e["T_b"], e["window"],
                                       global_pos=e["globals"]).tolist()
        assert got == e["visible"], (e["cite"], got)
        bf = [p for _, p in BF.visible_slots_brute(e["T_b"], e["T_b"] + 3, e["window"],
                                                    global_pos=e["globals"])]
        assert bf == e["visible"], (e["cite"], bf)


def test_global_golden():
    check_global_golden()


def check_global_brute_force(seed=16):
    rng = _rng(seed)
    for c in range(30):
        T_cap = int(rng.integers(1, 30))
        G = sorted(set(rng.integers(0, T_cap + 3, size=int(rng.integers(0, 6))).tolist()))
        window = int(rng.choice([1, 2, 3, 5]))
        q, k, v, lens, _ = _tiny_case(rng, 2, 4, 2, T_cap, 4)
        o, l = oracle.gqa_decode_ref(q, k, v, lens, window=window, scale=0.7,
                                     global_pos=G)
        ob, lb = BF.gqa_decode_brute(q, k, v, lens, window=window, scale=0.7,
                                     global_pos=G)
        assert np.allclose(o, np.array(ob), atol=1e-12), c
        lb = np.array(lb)
        fin = np.isfinite(l)
        assert np.array_equal(fin, np.isfinite(lb)) and np.allclose(l[fin], lb[fin], atol=1e-12)


def test_global_brute_force():
    check_global_brute_force()


ALL_CHECKS += [check_global_golden, check_global_brute_force]


# -------------------------------------------------------------- paged caches
def _paged_pool(rng, lens, P, H, d, spare=3):
    """A shuffled pool holding each sequence's positions 0..len-1 in pages of
    P rows, plus a few unused pages; returns (pool, table)."""
    need = [max(1, -(-int(n) // P)) for n in lens]
    max_pages = max(need)
    n_pages = sum(need) + spare
    perm = rng.permutation(n_pages)
    pool = rng.standard_normal((n_pages, H, P, d))
    table = np.full((len(lens), max_pages), int(n_pages - 1), dtype=np.int64)
    k = 0
    for b, n in enumerate(need):
        table[b, :n] = perm[k:k + n]
        k += n
    return pool, table


def check_paged_brute_force(seed=17):
    """Vectorised paged reference == scalar page walk, over shuffled pools,
    page sizes 1..4, windows, ragged and empty sequences."""
    rng = _rng(seed)
    for c in range(25):
        P = int(rng.integers(1, 5))
        lens = rng.integers(0, 14, size=2)
        H_q, H_kv, d = 4, 2, 3
        kp, table = _paged_pool(rng, lens, P, H_kv, d)
        vp = rng.standard_normal(kp.shape)
        q = rng.standard_normal((2, H_q, d))
        w = int(rng.choice([0, 1, 2, 5]))
        o, l = oracle.gqa_decode_paged_ref(q, kp, vp, table, lens, w, 0.8)
        ob, lb = BF.gqa_decode_paged_brute(q, kp, vp, table, lens, w, 0.8)
        assert np.allclose(o, np.array(ob), atol=1e-12), c
        lb = np.array(lb)
        fin = np.isfinite(l)
        assert np.array_equal(fin, np.isfinite(lb)) and np.allclose(l[fin], lb[fin], atol=1e-12)


def test_paged_brute_force():
    check_paged_brute_force()


def check_paged_contiguous_reduction(seed=18):
    """A contiguous cache cut into pages with the identity block table is the
    linear cache: results equal the (pinned) linear reference exactly."""
    rng = _rng(seed)
    B, H_q, H_kv, T, d, P = 3, 6, 3, 24, 5, 4
    k = rng.standard_normal((B, H_kv, T, d))
    v = rng.standard_normal((B, H_kv, T, d))
    q = rng.standard_normal((B, H_q, d))
    lens = np.array([24, 13, 1])
    npb = T // P
    kp = k.reshape(B, H_kv, npb, P, d).transpose(0, 2, 1, 3, 4).reshape(B * npb, H_kv, P, d)
    vp = v.reshape(B, H_kv, npb, P, d).transpose(0, 2, 1, 3, 4).reshape(B * npb, H_kv, P, d)
    table = np.arange(B * npb).reshape(B, npb)
    for w in (0, 3):
        o, l = oracle.gqa_decode_paged_ref(q, kp, vp, table, lens, w)
        o2, l2 = oracle.gqa_decode_ref(q, k, v, lens, window=w)
        assert np.array_equal(o, o2) and np.array_equal(l, l2)


def test_paged_contiguous_reduction():
    check_paged_contiguous_reduction()


def check_paged_permutation_invariance(seed=19):
    """Moving pages inside the pool and rewriting the table to match changes
    nothing."""
    rng = _rng(seed)
    lens = np.array([11, 7])
    kp, table = _paged_pool(rng, lens, 2, 2, 3)
    vp = rng.standard_normal(kp.shape)
    q = rng.standard_normal((2, 4, 3))
    perm = rng.permutation(kp.shape[0])
    inv = np.argsort(perm)
    o, l = oracle.gqa_decode_paged_ref(q, kp, vp, table, lens)
    o2, l2 = oracle.gqa_decode_paged_ref(q, kp[perm], vp[perm], inv[table], lens)
    assert np.array_equal(o, o2) and np.array_equal(l, l2)


def test_paged_permutation_invariance():
    check_paged_permutation_invariance()


def check_mla_paged(seed=20):
    """Paged MLA == scalar page walk, and == the linear MLA reference on a
    contiguous cache cut into pages."""
    rng = _rng(seed)
    d_c, dk, P = 4, 6, 2
    lens = np.array([7, 0, 4])
    pool = rng.standard_normal((9, P, dk))
    table = np.array([[3, 0, 7, 5], [1, 1, 1, 1], [8, 2, 4, 4]])
    q = rng.standard_normal((3, 3, dk))
    z, l = oracle.mla_decode_paged_ref(q, pool, table, d_c, 0.5, lens)
    zb, lb = BF.mla_decode_paged_brute(q, pool, table, d_c, 0.5, lens)
    assert np.allclose(z, np.array(zb), atol=1e-12)
    fin = np.isfinite(l)
    assert np.array_equal(fin, np.isfinite(np.array(lb)))
    assert np.allclose(l[fin], np.array(lb)[fin], atol=1e-12)
    lat = rng.standard_normal((2, 8, dk))
    pages = lat.reshape(2 * 4, P, dk)
    t2 = np.arange(8).reshape(2, 4)
    z1, l1 = oracle.mla_decode_paged_ref(q[:2], pages, t2, d_c, 0.5, [8, 5])
    z2, l2 = oracle.mla_decode_ref(q[:2], lat, d_c, 0.5, [8, 5])
    assert np.array_equal(z1, z2) and np.array_equal(l1, l2)


def test_mla_paged():
    check_mla_paged()


def check_paged_append(seed=21):
    """Appending into a paged pool and decoding equals appending into the
    linear cache and decoding."""
    rng = _rng(seed)
    B, H_kv, T, d, P = 2, 2, 8, 3, 4
    k = rng.standard_normal((B, H_kv, T, d))
    kn = rng.standard_normal((B, H_kv, d))
    pos = np.array([5, 0])
    kp = k.reshape(B, H_kv, 2, P, d).transpose(0, 2, 1, 3, 4).reshape(B * 2, H_kv, P, d)
    kp = kp[[0, 2, 1, 3]]  # pool order: seq0 page0, seq1 page0, seq0 page1, seq1 page1
    table = np.array([[0, 2], [1, 3]])
    got = oracle.kv_append_paged_ref(kp, kn, pos, table)
    lin = oracle.kv_append_ref(k, kn, pos)
    q = rng.standard_normal((B, 4, d))
    o1, l1 = oracle.gqa_decode_paged_ref(q, got, got, table, pos + 1)
    o2, l2 = oracle.gqa_decode_ref(q, lin, lin, pos + 1)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)
    # positions past the table are not written
    assert np.array_equal(oracle.kv_append_paged_ref(kp, kn, [8, -1], table), kp)


def test_paged_append():
    check_paged_append()


ALL_CHECKS += [check_paged_brute_force, check_paged_contiguous_reduction,
               check_paged_permutation_invariance, check_mla_paged,
               check_paged_append]


@pytest.mark.parametrize("mutant", [
    lambda pos, row, P: (np.asarray(row)[np.asarray(pos) % P], np.asarray(pos) // P),
    lambda pos, row, P: (np.asarray(row)[np.asarray(pos) // P], (np.asarray(pos) + 1) % P),
    lambda pos, row, P: (np.asarray(row)[np.minimum(np.asarray(pos) // P + 1, len(row) - 1)],
                         np.asarray(pos) % P),
], ids=["page_row_swapped", "row_off_by_one", "next_page"])
def test_planted_paging_mistakes_are_caught(monkeypatch, mutant):
    monkeypatch.setattr(A, "paged_positions", mutant)
    assert _caught()


# ------------------------------------------------------ several query tokens
def check_multi_brute_force(seed=22):
    """L-token reference == scalar slot walk, linear and ring, windows,
    chunks longer than some sequences."""
    rng = _rng(seed)
    for c in range(30):
        L = int(rng.choice([1, 2, 3, 5]))
        ring = bool(rng.integers(0, 2))
        T_cap = int(rng.integers(max(2, L), 12))
        w = int(rng.choice([0, 1, 2, 4]))
        if ring and w + L - 1 > T_cap:
            w = 0 if L > T_cap else max(0, T_cap - L + 1)
            if w == 0 and ring:
                ring = False
        B, H_q, H_kv, d = 2, 4, 2, 3
        q = rng.standard_normal((B, L, H_q, d))
        k = rng.standard_normal((B, H_kv, T_cap, d))
        v = rng.standard_normal((B, H_kv, T_cap, d))
        if ring:
            lens = rng.integers(0, 3 * T_cap, size=B)
            heads = rng.integers(0, T_cap, size=B)
        else:
            lens = rng.integers(0, T_cap + 1, size=B)
            heads = None
        o, l = oracle.gqa_decode_multi_ref(q, k, v, lens, heads, w, 0.9)
        ob, lb = BF.gqa_decode_multi_brute(q, k, v, lens, heads, w, 0.9)
        assert np.allclose(o, np.array(ob), atol=1e-12), c
        lb = np.array(lb)
        fin = np.isfinite(l)
        assert np.array_equal(fin, np.isfinite(lb)) and np.allclose(l[fin], lb[fin], atol=1e-12)


def test_multi_brute_force():
    check_multi_brute_force()


def check_multi_token_reductions(seed=23):
    """One token is the decode reference; token l of a chunk is the decode
    reference on the cache cut after position T_b - L + l."""
    rng = _rng(seed)
    B, L, H_q, H_kv, T, d = 2, 4, 6, 2, 16, 5
    q = rng.standard_normal((B, L, H_q, d))
    k = rng.standard_normal((B, H_kv, T, d))
    v = rng.standard_normal((B, H_kv, T, d))
    lens = np.array([16, 9])
    for w in (0, 3):
        o, l = oracle.gqa_decode_multi_ref(q[:, :1], k, v, lens, window=w)
        o1, l1 = oracle.gqa_decode_ref(q[:, 0], k, v, lens, window=w)
        assert np.array_equal(o[:, 0], o1) and np.array_equal(l[:, 0], l1)
        o, l = oracle.gqa_decode_multi_ref(q, k, v, lens, window=w)
        for t in range(L):
            ot, lt = oracle.gqa_decode_ref(q[:, t], k, v, lens - L + t + 1, window=w)
            assert np.allclose(o[:, t], ot, atol=1e-13) and np.allclose(l[:, t], lt, atol=1e-13)


def test_multi_token_reductions():
    check_multi_token_reductions()


def check_multi_torch_causal_sdpa(seed=24):
    """A chunk over a linear cache without window is causal attention with
    the chunk aligned to the end of the keys (torch SDPA with an explicit
    mask, float64)."""
    rng = _rng(seed)
    B, L, H, T, d = 1, 5, 3, 11, 4
    q = rng.standard_normal((B, L, H, d))
    k = rng.standard_normal((B, H, T, d))
    v = rng.standard_normal((B, H, T, d))
    o, _ = oracle.gqa_decode_multi_ref(q, k, v, [T])
    mask = torch.tensor([[j <= T - L + i for j in range(T)] for i in range(L)])
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q).permute(0, 2, 1, 3), torch.from_numpy(k),
        torch.from_numpy(v), attn_mask=mask)
    assert np.allclose(o, ref.permute(0, 2, 1, 3).numpy(), atol=1e-12)


def test_multi_torch_causal_sdpa():
    check_multi_torch_causal_sdpa()


def check_mla_multi(seed=25):
    """L-token MLA == the decode MLA reference on the truncated cache, and
    == the scalar MLA loop."""
    rng = _rng(seed)
    B, L, H, T, d_c, dk = 2, 3, 2, 9, 4, 6
    q = rng.standard_normal((B, L, H, dk))
    lat = rng.standard_normal((B, T, dk))
    lens = np.array([9, 2])
    z, l = oracle.mla_decode_multi_ref(q, lat, d_c, 0.6, lens)
    for t in range(L):
        zt, lt = oracle.mla_decode_ref(q[:, t], lat, d_c, 0.6, np.maximum(lens - L + t + 1, 0))
        zb, lb = BF.mla_decode_brute(q[:, t], lat, d_c, 0.6, np.maximum(lens - L + t + 1, 0))
        assert np.allclose(z[:, t], zt, atol=1e-13)
        assert np.allclose(z[:, t], np.array(zb), atol=1e-12)
        fin = np.isfinite(lt)
        assert np.array_equal(np.isfinite(l[:, t]), fin)
        assert np.allclose(l[:, t][fin], lt[fin], atol=1e-13)


def test_mla_multi():
    check_mla_multi()


ALL_CHECKS += [check_multi_brute_force, check_multi_token_reductions,
               check_multi_torch_causal_sdpa, check_mla_multi]


@pytest.mark.parametrize("shift", [1, -1])
def test_planted_chunk_position_mistakes_are_caught(monkeypatch, shift):
    monkeypatch.setattr(A, "_chunk_position", lambda T_b, L, l: T_b - L + l + shift)
    assert _caught()
