"""The C ABI without a GPU: the library loads, exports every function the
header declares, and rejects bad arguments on the host before any HIP call."""

import ctypes
import os
import re

import pytest

import decode_attention_kv_attn_amd as L

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADERS = [os.path.join(ROOT, "include", h)
           for h in sorted(os.listdir(os.path.join(ROOT, "include"))) if h.endswith(".h")]


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(L.library_path):
        from decode_attention_kv_attn_amd import build
        build.build()
    return L.library()


def declared_functions():
    text = "".join(open(h).read() for h in HEADERS)
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\*?\s+\**(attn_\w+)\s*\(",
                                 text, flags=re.M)))


def test_header_declares_the_entry_points():
    names = declared_functions()
    for want in ("attn_decode_gqa", "attn_decode_mla", "attn_combine",
                 "attn_decode_workspace_bytes", "attn_status_string"):
        assert want in names, names


def test_every_declared_symbol_is_exported(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name
        assert name in L._SIGS, f"binding lacks {name}"


P16 = ctypes.c_void_p(4096)      # aligned, never dereferenced: calls fail first


def gqa(lib, q=P16, k=P16, v=P16, out=P16, lse=None, sl=None, rh=None, B=1,
        H_q=8, H_kv=2, T=512, d=64, dt=1, window=0, scale=0.0, S=0, ws=None,
        wsb=0):
    return lib.attn_decode_gqa(q, k, v, out, lse, sl, rh, B, H_q, H_kv, T, d,
                               dt, window, scale, S, ws, wsb, None)


def test_gqa_host_errors(lib):
    assert gqa(lib, q=None) == -1
    assert gqa(lib, out=None) == -1
    assert gqa(lib, H_kv=3) == -2            # 8 % 3 != 0
    assert gqa(lib, H_q=0) == -2
    assert gqa(lib, T=0) == -2
    assert gqa(lib, B=-1) == -2
    assert gqa(lib, dt=7) == -3
    assert gqa(lib, d=96) == -4
    assert gqa(lib, window=-1) == -5
    assert gqa(lib, rh=P16, window=513) == -5  # ring: window > slots
    assert gqa(lib, q=ctypes.c_void_p(4098)) == -7
    assert gqa(lib, out=ctypes.c_void_p(4098)) == -7
    assert gqa(lib, scale=float("inf")) == -9
    assert gqa(lib, S=-1) == -9
    assert gqa(lib, S=2000) == -9
    # two splits need a workspace of the reported size
    need = lib.attn_decode_gqa_workspace_bytes(1, 8, 2, 512, 64, 1, 0, 0, 4)
    assert need > 0
    assert gqa(lib, S=4) == -6
    assert gqa(lib, S=4, ws=P16, wsb=need - 1) == -6
    assert gqa(lib, S=4, ws=ctypes.c_void_p(4100), wsb=need) == -7
    # B == 0 is a no-op that succeeds without launching, NULL pointers allowed
    assert gqa(lib, B=0) == 0
    assert gqa(lib, B=0, q=None, k=None, v=None, out=None) == 0


def noalloc(lib, q=P16, k=P16, v=P16, out=P16, lse=None, sl=None, rh=None, B=1,
            H_q=8, H_kv=2, T=512, d=64, dt=1, window=0, scale=0.0, S=0):
    return lib.attn_decode_gqa_noalloc(q, k, v, out, lse, sl, rh, B, H_q, H_kv, T,
                                       d, dt, window, scale, S, None)


def test_gqa_noalloc_host_errors(lib):
    """The no-allocation form checks like attn_decode_gqa, and rejects a plan
    whose fixed splits exceed its device array before any HIP call."""
    assert noalloc(lib, q=None) == -1
    assert noalloc(lib, out=None) == -1
    assert noalloc(lib, H_kv=3) == -2
    assert noalloc(lib, dt=7) == -3
    assert noalloc(lib, d=96) == -4
    assert noalloc(lib, rh=P16, window=513) == -5
    assert noalloc(lib, out=ctypes.c_void_p(4098)) == -7
    assert noalloc(lib, scale=float("inf")) == -9
    assert noalloc(lib, S=2000) == -9
    assert noalloc(lib, B=0, q=None, k=None, v=None, out=None) == 0
    # 64 x 32 heads x 16 splits x 128 floats: 16 MiB of partials plus their
    # log-sum-exps -- past the array; 8 splits fit
    big = dict(B=64, H_q=32, H_kv=32, T=32768, d=128)
    assert lib.attn_decode_gqa_workspace_bytes(64, 32, 32, 32768, 128, 1, 0, 0, 16) \
        > L.ATTN_NOALLOC_SCRATCH_BYTES
    assert lib.attn_decode_gqa_workspace_bytes(64, 32, 32, 32768, 128, 1, 0, 0, 8) \
        <= L.ATTN_NOALLOC_SCRATCH_BYTES
    assert noalloc(lib, S=16, **big) == -6
    assert noalloc(lib, S=1000, B=1, H_q=32, H_kv=1, T=32768, d=256) == -6


def test_noalloc_binding_needs_out():
    import torch
    q = torch.zeros(1, 8, 64, dtype=torch.bfloat16)
    k = torch.zeros(1, 2, 16, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="out is required"):
        L.attn_decode_gqa_noalloc(q, k, k, None)


def test_combine_and_mla_host_errors(lib):
    assert lib.attn_combine(None, P16, P16, None, 1, 1, 2, 8, None) == -1
    assert lib.attn_combine(P16, P16, P16, None, 1, 1, 0, 8, None) == -9
    assert lib.attn_combine(P16, P16, P16, None, 1, 0, 2, 8, None) == -2
    assert lib.attn_combine(P16, P16, P16, None, 0, 1, 2, 8, None) == 0
    assert lib.attn_combine(None, None, None, None, 0, 1, 2, 8, None) == 0
    assert lib.attn_decode_mla(None, P16, P16, None, None, 1, 128, 64, 512, 64,
                               0.07, 0, None, 0, None) == -1
    assert lib.attn_decode_mla(P16, P16, P16, None, None, 1, 128, 64, 512, 64,
                               0.0, 0, None, 0, None) == -9
    assert lib.attn_decode_mla(P16, P16, P16, None, None, 1, 128, 64, 500, 64,
                               0.07, 0, None, 0, None) == -4


def test_status_strings(lib):
    for st in range(-9, 1):
        assert L.attn_status_string(st) != "unknown status"


def test_planner(lib):
    # splits never leave a structurally empty piece and fit the visible range
    for args in [(32, 32, 8, 4096, 128, 1, 0, 0), (1, 32, 32, 32768, 128, 1, 0, 0),
                 (4, 24, 4, 131072, 256, 1, 0, 0), (16, 32, 8, 4096, 128, 1, 4096, 1),
                 (1, 8, 2, 512, 64, 0, 0, 0), (64, 32, 1, 32768, 128, 1, 0, 0)]:
        S = lib.attn_decode_gqa_splits(*args, 0)
        assert 1 <= S <= 1024
        T, window = args[3], args[6]
        mv = window if window else T
        chunk = -(-mv // S)
        assert (S - 1) * chunk < mv
        ws = lib.attn_decode_gqa_workspace_bytes(*args, 0)
        fixed = 0 if S == 1 else lib.attn_decode_workspace_bytes(args[0], args[1], args[4], S)
        B, H_q, H_kv, _, d, dt, w, ring = args
        plan = L.attn_decode_gqa_plan(B, H_q, H_kv, T, d, dt, w, ring)
        cap = plan["balanced_groups"]
        # the balanced list is planned only where the fixed plan splits (no
        # rings), for either kernel, and keeps one round of work groups
        assert cap == 0 or (S > 1 and not ring and
                            B * H_kv * -(-H_q // H_kv // plan["heads_per_item"]) < cap)
        if S > 1 and not ring and B <= 256:
            assert cap > 0
        up = lambda x: -(-x // 256) * 256
        # the even split (matrix-core kernel) keeps a slot per (group, unit)
        # segment, at most cap + B * units, and a pair per unit; the
        # per-sequence list a slot per group and a pair per sequence
        units = H_kv * -(-H_q // H_kv // plan["heads_per_item"])
        assert plan["even_split"] == (cap > 0 and plan["kernel"] == "mfma" and d <= 128)
        slots = cap + B * units if plan["even_split"] else cap
        pairs = B * units if plan["even_split"] else B
        rows = slots * plan["heads_per_item"]
        bal = up(rows * d * 4) + up(rows * 4) + up(pairs * 8) if cap else 0
        assert ws == max(fixed, bal) == plan["workspace_bytes"]
    for S in (1, 2, 7, 64, 1024):
        got = lib.attn_decode_gqa_splits(4, 16, 4, 2000, 128, 1, 0, 0, S)
        assert 1 <= got <= S
    assert lib.attn_decode_workspace_bytes(2, 3, 64, 1) == 0
    assert lib.attn_decode_workspace_bytes(2, 3, 64, 5) % 256 == 0


def test_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    monkeypatch.setattr(L, "_LIB", None)
    monkeypatch.setattr(L, "library_path", str(tmp_path / "missing.so"))
    with pytest.raises(RuntimeError):
        L.library()


def test_append_host_errors(lib):
    ap = lib.attn_kv_append
    assert ap(None, None, P16, None, P16, 1, 2, 8, 64, 1, None) == -1
    assert ap(P16, P16, P16, None, P16, 1, 2, 8, 64, 1, None) == -1   # v pair mismatch
    assert ap(P16, None, P16, None, P16, 1, 0, 8, 64, 1, None) == -2
    assert ap(P16, None, P16, None, P16, 1, 2, 8, 64, 5, None) == -3
    assert ap(P16, None, P16, None, P16, 1, 2, 8, 3, 1, None) == -7    # 6-byte rows
    assert ap(ctypes.c_void_p(4100), None, P16, None, P16, 1, 2, 8, 64, 1, None) == -7
    assert ap(None, None, None, None, None, 0, 2, 8, 64, 1, None) == 0
    ar = lib.attn_kv_append_ring
    assert ar(P16, None, P16, None, None, 1, 2, 8, 64, 1, None) == -1
    assert ar(P16, None, P16, None, P16, 1, 2, 0, 64, 1, None) == -2


def test_global_host_errors(lib):
    def gg(gp=P16, n=2, q=P16, window=64, B=1, T=512, S=0, ws=None, wsb=0):
        return lib.attn_decode_gqa_global(q, P16, P16, P16, None, None, gp, n, B,
                                          8, 2, T, 64, 1, window, 0.0, S, ws,
                                          wsb, None)
    assert gg(gp=None) == -1                 # n_global > 0 needs the list
    assert gg(n=-1) == -9
    assert gg(n=65537) == -9
    assert gg(gp=ctypes.c_void_p(4098)) == -7
    assert gg(q=None) == -1
    assert gg(window=-1) == -5
    assert gg(B=0, gp=None, q=None) == 0
    # the planner's bound grows with the global count, and splits never exceed it
    for window, n in [(64, 0), (64, 2), (4096, 100), (0, 5)]:
        S = lib.attn_decode_gqa_global_splits(16, 32, 8, 32768, 128, 1, window, n, 0)
        mv = min(window + n, 32768) if window else 32768
        assert 1 <= S <= 1024
        chunk = -(-mv // S)
        assert (S - 1) * chunk < mv
        ws = lib.attn_decode_gqa_global_workspace_bytes(16, 32, 8, 32768, 128, 1,
                                                        window, n, 0)
        plan = L.attn_decode_gqa_plan(16, 32, 8, 32768, 128, 1, window, False, n)
        assert ws == plan["workspace_bytes"]
        assert ws >= (0 if S == 1 else lib.attn_decode_workspace_bytes(16, 32, 128, S))
    # without global positions the plan is attn_decode_gqa's
    assert (lib.attn_decode_gqa_global_splits(8, 32, 8, 4096, 128, 1, 512, 0, 0)
            == lib.attn_decode_gqa_splits(8, 32, 8, 4096, 128, 1, 512, 0, 0))


def test_paged_host_errors(lib):
    def gp(bt=P16, max_pages=8, num_pages=64, P=16, B=1, H_kv=2, q=P16):
        return lib.attn_decode_gqa_paged(q, P16, P16, P16, None, None, bt, max_pages,
                                         B, 1, 8, H_kv, num_pages, P, 64, 1, 0, 0.0, 0,
                                         None, 0, None)
    assert gp(bt=None) == -1
    assert gp(P=24) == -4            # not a power of two
    assert gp(P=8) == -4             # below the smallest page
    assert gp(max_pages=0) == -2
    assert gp(num_pages=0) == -2
    assert gp(num_pages=1 << 26, P=64) == -2   # pool rows overflow 32 bits
    assert gp(bt=ctypes.c_void_p(4098)) == -7
    assert gp(q=None) == -1
    assert gp(B=0, bt=None, q=None) == 0

    def mp(bt=P16, P=64, d_c=512):
        return lib.attn_decode_mla_paged(P16, P16, P16, None, None, bt, 4, 1, 1, 16, 8,
                                         P, d_c, 64, 0.07, 0, None, 0, None)
    assert mp(bt=None) == -1
    assert mp(P=48) == -4
    assert mp(d_c=384) == -4
    ap = lib.attn_kv_append_paged
    assert ap(P16, None, P16, None, P16, None, 4, 1, 2, 8, 16, 64, 1, None) == -1
    assert ap(P16, None, P16, None, P16, P16, 4, 1, 2, 8, 12, 64, 1, None) == -4
    assert ap(None, None, None, None, None, None, 4, 0, 2, 8, 16, 64, 1, None) == 0


def test_plan_info(lib):
    for (H_q, H_kv, d, dt, want) in [(32, 32, 128, 1, "valu"), (16, 8, 128, 1, "valu"),
                                     (24, 8, 128, 1, "mfma"), (32, 8, 128, 1, "mfma"),
                                     (32, 1, 64, 1, "mfma"), (32, 8, 128, 0, "valu"),
                                     (24, 4, 256, 1, "mfma"), (8, 4, 256, 1, "valu")]:
        p = L.attn_decode_gqa_plan(32, H_q, H_kv, 4096, d, dt)
        assert p["kernel"] == want, (H_q, H_kv, d, dt, p)
        assert p["splits"] == lib.attn_decode_gqa_splits(32, H_q, H_kv, 4096, d, dt, 0, 0, 0)
        assert p["groups"] % p["splits"] == 0 and p["groups"] >= 32 * H_kv
        n = H_q // H_kv
        if want == "mfma":
            assert p["heads_per_item"] in (16, 32)
            assert p["heads_per_item"] >= min(n, 32 if d < 256 else 16)
        else:
            assert p["heads_per_item"] == min(n, 8)
    assert lib.attn_decode_gqa_plan(1, 1, 8, 3, 64, 64, 1, 0, 0, 0, 0, None) == -1
    with pytest.raises(L.AttnError):
        L.attn_decode_gqa_plan(1, 8, 3, 64, 64, 1)



def test_multi_token_host_errors(lib):
    def gm(q_len=4, window=0, rh=None, T=512, q=P16, B=1):
        return lib.attn_decode_gqa_multi(q, P16, P16, P16, None, None, rh, B, q_len, 8,
                                         2, T, 64, 1, window, 0.0, 0, None, 0, None)
    assert gm(q_len=0) == -9
    assert gm(q_len=1025) == -9
    assert gm(window=-1) == -5
    assert gm(rh=P16, window=510) == -5      # ring: 510 + 4 - 1 > 512 slots
    assert gm(q=None) == -1
    assert gm(B=0, q=None) == 0
    # the plan of L tokens: (head, token) columns of a KV head
    p1 = L.attn_decode_gqa_plan(8, 32, 8, 4096, 128, 1)
    p4 = L.attn_decode_gqa_plan(8, 32, 8, 4096, 128, 1, q_len=4)
    assert p4["kernel"] == "mfma" and p4["heads_per_item"] == 16
    assert p1["heads_per_item"] == 16
    pv = L.attn_decode_gqa_plan(8, 8, 8, 4096, 128, 1, q_len=3)
    assert pv["kernel"] == "mfma"  # 3 columns per KV head
    assert L.attn_decode_gqa_plan(8, 8, 8, 4096, 128, 1)["kernel"] == "valu"
    for S in (2, 5):
        p = L.attn_decode_gqa_plan(8, 32, 8, 4096, 128, 1, num_splits=S, q_len=3)
        assert p["workspace_bytes"] == lib.attn_decode_workspace_bytes(8 * 3, 32, 128, p["splits"])
    assert lib.attn_decode_mla_multi(P16, P16, P16, None, None, 1, 0, 16, 64, 512, 64,
                                     0.07, 0, None, 0, None) == -9
