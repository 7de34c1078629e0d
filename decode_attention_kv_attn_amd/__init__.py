"""Python binding of the MI355X decode-attention library (``libattn_decode.so``).

Argument marshalling only: every function takes torch tensors that already
live on the GPU, passes their device pointers and the current HIP stream to
the C ABI declared in ``include/attn_decode.h``, and raises on a non-zero
status.  All arithmetic runs in the library's HIP kernels; there is no
fallback -- if the shared library is missing, every call raises.
"""

import ctypes
import math
import os

import torch

__all__ = [
    "ATTN_F32", "ATTN_BF16", "AttnError", "library", "library_path",
    "attn_decode_gqa", "attn_decode_mla", "attn_combine",
    "attn_decode_gqa_splits", "attn_decode_gqa_workspace_bytes",
    "attn_decode_mla_splits", "attn_decode_mla_workspace_bytes",
    "attn_decode_workspace_bytes", "attn_status_string",
    "attn_kv_append", "attn_kv_append_ring",
    "attn_decode_gqa_global", "attn_decode_gqa_global_splits",
    "attn_decode_gqa_global_workspace_bytes",
    "attn_decode_gqa_paged", "attn_decode_mla_paged", "attn_kv_append_paged",
    "attn_decode_gqa_plan", "attn_decode_gqa_multi", "attn_decode_mla_multi",
]

ATTN_F32 = 0
ATTN_BF16 = 1

_HERE = os.path.dirname(os.path.abspath(__file__))
library_path = os.path.join(_HERE, "libattn_decode.so")
_LIB = None

_vp, _i, _f, _sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
_SIGS = {
    "attn_decode_gqa": (_i, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i,
                             _i, _i, _i, _f, _i, _vp, _sz, _vp]),
    "attn_decode_gqa_global": (_i, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _i, _i,
                                    _i, _i, _i, _i, _i, _i, _f, _i, _vp, _sz,
                                    _vp]),
    "attn_decode_gqa_global_splits": (_i, [_i] * 9),
    "attn_decode_gqa_global_workspace_bytes": (_sz, [_i] * 9),
    "attn_decode_gqa_paged": (_i, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i,
                                   _i, _i, _i, _i, _i, _i, _i, _f, _i, _vp, _sz,
                                   _vp]),
    "attn_decode_mla_paged": (_i, [_vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i,
                                   _i, _i, _i, _i, _f, _i, _vp, _sz, _vp]),
    "attn_decode_gqa_multi": (_i, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i,
                                   _i, _i, _i, _i, _i, _f, _i, _vp, _sz, _vp]),
    "attn_decode_mla_multi": (_i, [_vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i,
                                   _i, _f, _i, _vp, _sz, _vp]),
    "attn_kv_append_paged": (_i, [_vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i,
                                  _i, _i, _i, _vp]),
    "attn_decode_gqa_plan": (_i, [_i] * 11 + [_vp]),
    "attn_decode_gqa_splits": (_i, [_i] * 9),
    "attn_decode_gqa_workspace_bytes": (_sz, [_i] * 9),
    "attn_decode_mla": (_i, [_vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _f,
                             _i, _vp, _sz, _vp]),
    "attn_decode_mla_splits": (_i, [_i] * 6),
    "attn_decode_mla_workspace_bytes": (_sz, [_i] * 6),
    "attn_combine": (_i, [_vp, _vp, _vp, _vp, _i, _i, _i, _i, _vp]),
    "attn_decode_workspace_bytes": (_sz, [_i] * 4),
    "attn_status_string": (ctypes.c_char_p, [_i]),
    "attn_kv_append": (_i, [_vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _vp]),
    "attn_kv_append_ring": (_i, [_vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _vp]),
    "attn_probe_read": (_i, [_vp, _sz, _vp, _i, _vp]),
    "attn_probe_copy": (_i, [_vp, _vp, _sz, _vp]),
}


class AttnError(RuntimeError):
    """A non-zero status from the library."""

    def __init__(self, fn, status):
        self.status = status
        super().__init__(f"{fn}: status {status} "
                         f"({library().attn_status_string(status).decode()})")


def library():
    """The loaded ``libattn_decode.so`` (ctypes handle); raises if absent."""
    global _LIB
    if _LIB is None:
        if not os.path.exists(library_path):
            raise RuntimeError(
                f"{library_path} is missing: build it with "
                "`python -m decode_attention_kv_attn_amd.build`")
        lib = ctypes.CDLL(library_path)
        for name, (res, args) in _SIGS.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _LIB = lib
    return _LIB


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream, device):
    if stream is None:
        stream = torch.cuda.current_stream(device)
    return ctypes.c_void_p(stream.cuda_stream)


def _check(fn, st):
    if st != 0:
        raise AttnError(fn, st)


def _dtype_code(t):
    if t.dtype == torch.float32:
        return ATTN_F32
    if t.dtype == torch.bfloat16:
        return ATTN_BF16
    raise TypeError(f"unsupported dtype {t.dtype}")


def _need_dev(*ts):
    for t in ts:
        if t is not None and not t.is_cuda:
            raise ValueError("tensors must be on the GPU")
        if t is not None and not t.is_contiguous():
            raise ValueError("tensors must be contiguous")


def attn_decode_gqa_splits(B, H_q, H_kv, T_cap, d, dtype, window=0, ring=False,
                           num_splits=0):
    return library().attn_decode_gqa_splits(B, H_q, H_kv, T_cap, d, dtype,
                                            window, int(bool(ring)), num_splits)


def attn_decode_gqa_workspace_bytes(B, H_q, H_kv, T_cap, d, dtype, window=0,
                                    ring=False, num_splits=0):
    return library().attn_decode_gqa_workspace_bytes(
        B, H_q, H_kv, T_cap, d, dtype, window, int(bool(ring)), num_splits)


class _GqaPlan(ctypes.Structure):
    _fields_ = [("kernel", ctypes.c_int), ("splits", ctypes.c_int),
                ("chunk", ctypes.c_int), ("heads_per_item", ctypes.c_int),
                ("tile_rows", ctypes.c_int), ("waves", ctypes.c_int),
                ("groups", ctypes.c_longlong), ("workspace_bytes", ctypes.c_size_t),
                ("balanced_groups", ctypes.c_int)]


def attn_decode_gqa_plan(B, H_q, H_kv, T_cap, d, dtype, window=0, ring=False,
                         n_global=0, num_splits=0, q_len=1):
    """How a GQA decode call would run: dict with kernel ("valu" / "mfma"),
    splits, chunk, heads_per_item, tile_rows, waves, groups, workspace_bytes,
    balanced_groups."""
    p = _GqaPlan()
    st = library().attn_decode_gqa_plan(B, q_len, H_q, H_kv, T_cap, d, dtype,
                                        window, int(bool(ring)), n_global,
                                        num_splits, ctypes.byref(p))
    _check("attn_decode_gqa_plan", st)
    return {"kernel": "mfma" if p.kernel else "valu", "splits": p.splits,
            "chunk": p.chunk, "heads_per_item": p.heads_per_item,
            "tile_rows": p.tile_rows, "waves": p.waves, "groups": p.groups,
            "workspace_bytes": p.workspace_bytes,
            "balanced_groups": p.balanced_groups}


def attn_decode_workspace_bytes(B, H, d_v, num_splits):
    return library().attn_decode_workspace_bytes(B, H, d_v, num_splits)


def attn_status_string(status):
    return library().attn_status_string(status).decode()


def _workspace(nbytes, device, workspace):
    if nbytes == 0:
        return workspace
    if workspace is None or workspace.numel() * workspace.element_size() < nbytes:
        workspace = torch.empty(nbytes, dtype=torch.uint8, device=device)
    return workspace


def attn_decode_gqa(q, k, v, seq_lens=None, ring_head=None, window=0,
                    scale=None, num_splits=0, out=None, lse=None,
                    workspace=None, want_lse=True, stream=None):
    """One decode step of MHA/GQA/MQA attention.

    q [B, H_q, d], k/v [B, H_kv, T_cap, d] (float32 or bfloat16, same dtype),
    seq_lens / ring_head int32 [B] or None.  Returns ``(out, lse)`` float32
    tensors ([B, H_q, d], [B, H_q] or None).  See include/attn_decode.h.
    """
    _need_dev(q, k, v, seq_lens, ring_head, out, lse)
    B, H_q, d = q.shape
    _, H_kv, T_cap, _ = k.shape
    dt = _dtype_code(q)
    if out is None:
        out = torch.empty((B, H_q, d), dtype=torch.float32, device=q.device)
    if lse is None and want_lse:
        lse = torch.empty((B, H_q), dtype=torch.float32, device=q.device)
    ring = ring_head is not None
    nbytes = attn_decode_gqa_workspace_bytes(B, H_q, H_kv, T_cap, d, dt,
                                             window, ring, num_splits)
    if nbytes == 2**64 - 1:
        nbytes = 0  # invalid arguments: the call below reports the status
    workspace = _workspace(nbytes, q.device, workspace)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = library().attn_decode_gqa(
        _ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), _ptr(seq_lens),
        _ptr(ring_head), B, H_q, H_kv, T_cap, d, dt, window,
        0.0 if scale is None else float(scale), num_splits, _ptr(workspace),
        ws_bytes, _stream(stream, q.device))
    _check("attn_decode_gqa", st)
    return out, lse


def attn_decode_gqa_global_splits(B, H_q, H_kv, T_cap, d, dtype, window,
                                  n_global, num_splits=0):
    return library().attn_decode_gqa_global_splits(
        B, H_q, H_kv, T_cap, d, dtype, window, n_global, num_splits)


def attn_decode_gqa_global_workspace_bytes(B, H_q, H_kv, T_cap, d, dtype,
                                           window, n_global, num_splits=0):
    return library().attn_decode_gqa_global_workspace_bytes(
        B, H_q, H_kv, T_cap, d, dtype, window, n_global, num_splits)


def attn_decode_gqa_global(q, k, v, global_pos, window, seq_lens=None,
                           scale=None, num_splits=0, out=None, lse=None,
                           workspace=None, want_lse=True, stream=None):
    """Sliding window plus global positions over a linear cache.

    ``global_pos``: sorted int32 [n_global] device tensor (or None for none);
    other arguments as for :func:`attn_decode_gqa` without ``ring_head``.
    """
    _need_dev(q, k, v, seq_lens, global_pos, out, lse)
    B, H_q, d = q.shape
    _, H_kv, T_cap, _ = k.shape
    dt = _dtype_code(q)
    n_global = 0 if global_pos is None else global_pos.numel()
    if out is None:
        out = torch.empty((B, H_q, d), dtype=torch.float32, device=q.device)
    if lse is None and want_lse:
        lse = torch.empty((B, H_q), dtype=torch.float32, device=q.device)
    nbytes = attn_decode_gqa_global_workspace_bytes(
        B, H_q, H_kv, T_cap, d, dt, window, n_global, num_splits)
    if nbytes == 2**64 - 1:
        nbytes = 0
    workspace = _workspace(nbytes, q.device, workspace)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = library().attn_decode_gqa_global(
        _ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), _ptr(seq_lens),
        _ptr(global_pos), n_global, B, H_q, H_kv, T_cap, d, dt, window,
        0.0 if scale is None else float(scale), num_splits, _ptr(workspace),
        ws_bytes, _stream(stream, q.device))
    _check("attn_decode_gqa_global", st)
    return out, lse


def attn_decode_mla_splits(B, H, T_cap, d_c, d_rope, num_splits=0):
    return library().attn_decode_mla_splits(B, H, T_cap, d_c, d_rope, num_splits)


def attn_decode_mla_workspace_bytes(B, H, T_cap, d_c, d_rope, num_splits=0):
    return library().attn_decode_mla_workspace_bytes(B, H, T_cap, d_c, d_rope,
                                                     num_splits)


def attn_decode_mla(q, latent, d_c, scale, seq_lens=None, num_splits=0,
                    out=None, lse=None, workspace=None, want_lse=True,
                    stream=None):
    """Absorbed MLA decode: q [B, H, d_c+d_rope], latent [B, T_cap, d_c+d_rope]
    (bfloat16).  Returns ``(z [B, H, d_c], lse [B, H])`` float32."""
    _need_dev(q, latent, seq_lens, out, lse)
    B, H, dk = q.shape
    _, T_cap, _ = latent.shape
    d_rope = dk - d_c
    if out is None:
        out = torch.empty((B, H, d_c), dtype=torch.float32, device=q.device)
    if lse is None and want_lse:
        lse = torch.empty((B, H), dtype=torch.float32, device=q.device)
    nbytes = attn_decode_mla_workspace_bytes(B, H, T_cap, d_c, d_rope, num_splits)
    if nbytes == 2**64 - 1:
        nbytes = 0
    workspace = _workspace(nbytes, q.device, workspace)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = library().attn_decode_mla(
        _ptr(q), _ptr(latent), _ptr(out), _ptr(lse), _ptr(seq_lens), B, H,
        T_cap, d_c, d_rope, float(scale), num_splits, _ptr(workspace), ws_bytes,
        _stream(stream, q.device))
    _check("attn_decode_mla", st)
    return out, lse


def attn_combine(o_part, lse_part, out=None, lse=None, want_lse=True,
                 stream=None):
    """Merge split results: o_part [B, H, S, d_v], lse_part [B, H, S]."""
    _need_dev(o_part, lse_part, out, lse)
    B, H, S, d_v = o_part.shape
    if out is None:
        out = torch.empty((B, H, d_v), dtype=torch.float32, device=o_part.device)
    if lse is None and want_lse:
        lse = torch.empty((B, H), dtype=torch.float32, device=o_part.device)
    st = library().attn_combine(_ptr(o_part), _ptr(lse_part), _ptr(out),
                                _ptr(lse), B, H, S, d_v,
                                _stream(stream, o_part.device))
    _check("attn_combine", st)
    return out, lse


def _cache_dims(cache):
    if cache.dim() == 4:
        B, H, T_cap, d = cache.shape
    elif cache.dim() == 3:  # latent cache [B, T_cap, width]
        (B, T_cap, d), H = cache.shape, 1
    else:
        raise ValueError("cache must be [B, H, T, d] or [B, T, d]")
    return B, H, T_cap, d


def attn_kv_append(k_cache, k_new, positions, v_cache=None, v_new=None,
                   stream=None):
    """Write k_new (and v_new) [B, H, d] at row positions[b] of the cache."""
    _need_dev(k_cache, k_new, positions, v_cache, v_new)
    B, H, T_cap, d = _cache_dims(k_cache)
    st = library().attn_kv_append(_ptr(k_cache), _ptr(v_cache), _ptr(k_new),
                                  _ptr(v_new), _ptr(positions), B, H, T_cap, d,
                                  _dtype_code(k_cache), _stream(stream, k_cache.device))
    _check("attn_kv_append", st)


def attn_kv_append_ring(k_cache, k_new, ring_head, v_cache=None, v_new=None,
                        stream=None):
    """Advance ring_head[b] (in place) and write the rows at the new slot."""
    _need_dev(k_cache, k_new, ring_head, v_cache, v_new)
    B, H, T_cap, d = _cache_dims(k_cache)
    st = library().attn_kv_append_ring(_ptr(k_cache), _ptr(v_cache), _ptr(k_new),
                                       _ptr(v_new), _ptr(ring_head), B, H, T_cap, d,
                                       _dtype_code(k_cache),
                                       _stream(stream, k_cache.device))
    _check("attn_kv_append_ring", st)


def _gqa_plan_bytes(B, L, H_q, H_kv, T_cap, d, dt, window, ring, num_splits):
    try:
        return attn_decode_gqa_plan(B, H_q, H_kv, T_cap, d, dt, window, ring, 0,
                                    num_splits, L)["workspace_bytes"]
    except AttnError:
        return 0  # invalid arguments: the call itself reports the status


def attn_decode_gqa_paged(q, k_pages, v_pages, block_table, seq_lens=None,
                          window=0, scale=None, num_splits=0, out=None, lse=None,
                          workspace=None, want_lse=True, stream=None):
    """Decode over a paged K/V pool: k_pages / v_pages [num_pages, H_kv, P,
    d], block_table int32 [B, max_pages]; q [B, H_q, d] (one token) or
    [B, L, H_q, d] (L tokens per sequence).  Returns ``(out, lse)`` shaped
    like q (float32) and q without its last dim."""
    _need_dev(q, k_pages, v_pages, block_table, seq_lens, out, lse)
    lead = q.shape[:-2]
    B, L = (q.shape[0], 1) if q.dim() == 3 else (q.shape[0], q.shape[1])
    H_q, d = q.shape[-2], q.shape[-1]
    num_pages, H_kv, P, _ = k_pages.shape
    max_pages = block_table.shape[1]
    dt = _dtype_code(q)
    if out is None:
        out = torch.empty((*lead, H_q, d), dtype=torch.float32, device=q.device)
    if lse is None and want_lse:
        lse = torch.empty((*lead, H_q), dtype=torch.float32, device=q.device)
    nbytes = _gqa_plan_bytes(B, L, H_q, H_kv, max_pages * P, d, dt, window, False,
                             num_splits)
    workspace = _workspace(nbytes, q.device, workspace)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = library().attn_decode_gqa_paged(
        _ptr(q), _ptr(k_pages), _ptr(v_pages), _ptr(out), _ptr(lse),
        _ptr(seq_lens), _ptr(block_table), max_pages, B, L, H_q, H_kv, num_pages,
        P, d, dt, window, 0.0 if scale is None else float(scale), num_splits,
        _ptr(workspace), ws_bytes, _stream(stream, q.device))
    _check("attn_decode_gqa_paged", st)
    return out, lse


def attn_decode_gqa_multi(q, k, v, seq_lens=None, ring_head=None, window=0,
                          scale=None, num_splits=0, out=None, lse=None,
                          workspace=None, want_lse=True, stream=None):
    """L query tokens per sequence: q [B, L, H_q, d] (the last L positions of
    each cache), k / v [B, H_kv, T_cap, d].  Returns ``(out [B, L, H_q, d],
    lse [B, L, H_q])`` float32."""
    _need_dev(q, k, v, seq_lens, ring_head, out, lse)
    B, L, H_q, d = q.shape
    _, H_kv, T_cap, _ = k.shape
    dt = _dtype_code(q)
    if out is None:
        out = torch.empty((B, L, H_q, d), dtype=torch.float32, device=q.device)
    if lse is None and want_lse:
        lse = torch.empty((B, L, H_q), dtype=torch.float32, device=q.device)
    nbytes = _gqa_plan_bytes(B, L, H_q, H_kv, T_cap, d, dt, window,
                             ring_head is not None, num_splits)
    workspace = _workspace(nbytes, q.device, workspace)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = library().attn_decode_gqa_multi(
        _ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), _ptr(seq_lens),
        _ptr(ring_head), B, L, H_q, H_kv, T_cap, d, dt, window,
        0.0 if scale is None else float(scale), num_splits, _ptr(workspace),
        ws_bytes, _stream(stream, q.device))
    _check("attn_decode_gqa_multi", st)
    return out, lse


def attn_decode_mla_paged(q, latent_pages, block_table, d_c, scale,
                          seq_lens=None, num_splits=0, out=None, lse=None,
                          workspace=None, want_lse=True, stream=None):
    """Absorbed MLA over a paged latent pool [num_pages, P, d_c+d_rope]
    (bfloat16) with block_table int32 [B, max_pages]; q [B, H, d_c+d_rope]
    or [B, L, H, d_c+d_rope] (L tokens per sequence)."""
    _need_dev(q, latent_pages, block_table, seq_lens, out, lse)
    lead = q.shape[:-2]
    B, L = (q.shape[0], 1) if q.dim() == 3 else (q.shape[0], q.shape[1])
    H, dk = q.shape[-2], q.shape[-1]
    num_pages, P, _ = latent_pages.shape
    max_pages = block_table.shape[1]
    d_rope = dk - d_c
    if out is None:
        out = torch.empty((*lead, H, d_c), dtype=torch.float32, device=q.device)
    if lse is None and want_lse:
        lse = torch.empty((*lead, H), dtype=torch.float32, device=q.device)
    nbytes = attn_decode_mla_workspace_bytes(B, H * L, max_pages * P, d_c, d_rope,
                                             num_splits)
    if nbytes == 2**64 - 1:
        nbytes = 0
    workspace = _workspace(nbytes, q.device, workspace)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = library().attn_decode_mla_paged(
        _ptr(q), _ptr(latent_pages), _ptr(out), _ptr(lse), _ptr(seq_lens),
        _ptr(block_table), max_pages, B, L, H, num_pages, P, d_c, d_rope,
        float(scale), num_splits, _ptr(workspace), ws_bytes,
        _stream(stream, q.device))
    _check("attn_decode_mla_paged", st)
    return out, lse


def attn_decode_mla_multi(q, latent, d_c, scale, seq_lens=None, num_splits=0,
                          out=None, lse=None, workspace=None, want_lse=True,
                          stream=None):
    """Absorbed MLA with L query tokens per sequence: q [B, L, H,
    d_c+d_rope], latent [B, T_cap, d_c+d_rope] (bfloat16).  Returns
    ``(z [B, L, H, d_c], lse [B, L, H])`` float32."""
    _need_dev(q, latent, seq_lens, out, lse)
    B, L, H, dk = q.shape
    _, T_cap, _ = latent.shape
    d_rope = dk - d_c
    if out is None:
        out = torch.empty((B, L, H, d_c), dtype=torch.float32, device=q.device)
    if lse is None and want_lse:
        lse = torch.empty((B, L, H), dtype=torch.float32, device=q.device)
    nbytes = attn_decode_mla_workspace_bytes(B, H * L, T_cap, d_c, d_rope, num_splits)
    if nbytes == 2**64 - 1:
        nbytes = 0
    workspace = _workspace(nbytes, q.device, workspace)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = library().attn_decode_mla_multi(
        _ptr(q), _ptr(latent), _ptr(out), _ptr(lse), _ptr(seq_lens), B, L, H,
        T_cap, d_c, d_rope, float(scale), num_splits, _ptr(workspace), ws_bytes,
        _stream(stream, q.device))
    _check("attn_decode_mla_multi", st)
    return out, lse


def attn_kv_append_paged(k_pages, k_new, positions, block_table, v_pages=None,
                         v_new=None, stream=None):
    """Write k_new (and v_new) [B, H, d] at position positions[b] of each
    sequence's pages ([num_pages, H, P, d]; a latent pool [num_pages, P, d]
    with [B, d] rows is taken as H = 1)."""
    _need_dev(k_pages, k_new, positions, block_table, v_pages, v_new)
    if k_pages.dim() == 3:
        num_pages, P, d = k_pages.shape
        H = 1
    else:
        num_pages, H, P, d = k_pages.shape
    B = positions.shape[0]
    st = library().attn_kv_append_paged(
        _ptr(k_pages), _ptr(v_pages), _ptr(k_new), _ptr(v_new), _ptr(positions),
        _ptr(block_table), block_table.shape[1], B, H, num_pages, P, d,
        _dtype_code(k_pages), _stream(stream, k_pages.device))
    _check("attn_kv_append_paged", st)


def attn_probe_read(src, sink, blocks=0, stream=None):
    """Stream-read every byte of ``src`` once (HBM read-rate probe)."""
    st = library().attn_probe_read(_ptr(src), src.numel() * src.element_size(),
                                   _ptr(sink), blocks, _stream(stream, src.device))
    _check("attn_probe_read", st)


def attn_probe_copy(dst, src, stream=None):
    """dst <- src byte for byte (a copy of known size)."""
    st = library().attn_probe_copy(_ptr(dst), _ptr(src),
                                   src.numel() * src.element_size(),
                                   _stream(stream, src.device))
    _check("attn_probe_copy", st)


def default_scale(d):
    """1/sqrt(d), the default softmax scale of the attention equation."""
    return 1.0 / math.sqrt(d)
