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
    "attn_decode_gqa_noalloc", "ATTN_NOALLOC_SCRATCH_BYTES",
]

ATTN_F32 = 0
ATTN_BF16 = 1
ATTN_NOALLOC_SCRATCH_BYTES = 16 << 20  # attn_decode_gqa_noalloc's device array

_HERE = os.path.dirname(os.path.abspath(__file__))
# ATTN_DECODE_LIBRARY names another build of the same library (the host-side
# sanitizer build of the tests); by default the in-tree one.
library_path = os.environ.get("ATTN_DECODE_LIBRARY") or os.path.join(_HERE, "libattn_decode.so")
_LIB = None

_vp, _i, _f, _sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
_SIGS = {
    "attn_decode_gqa": (_i, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i,
                             _i, _i, _i, _f, _i, _vp, _sz, _vp]),
    "attn_decode_gqa_noalloc": (_i, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i,
                                     _i, _i, _i, _i, _f, _i, _vp]),
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


def _dims(t, name, n):
    """t.shape, checked to have n dimensions (n an int or a tuple of ints)."""
    ok = (n,) if isinstance(n, int) else n
    if t.dim() not in ok:
        raise ValueError(f"{name} must have {' or '.join(map(str, ok))} dimensions, "
                         f"got shape {tuple(t.shape)}")
    return tuple(t.shape)


def _expect(t, name, shape=None, dtype=None, min_rows=None):
    """Shape / dtype check of an optional tensor argument (None passes)."""
    if t is None:
        return
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if min_rows is not None and (t.dim() != 2 or t.shape[0] < min_rows):
        raise ValueError(f"{name} must be 2-D with at least {min_rows} rows, "
                         f"got shape {tuple(t.shape)}")


def _same_dtype(ref, *named):
    for name, t in named:
        if t is not None and t.dtype != ref.dtype:
            raise ValueError(f"{name} must have the dtype of q ({ref.dtype}), got {t.dtype}")


def _on_device(ref, *ts):
    """Every tensor on the GPU, contiguous, on ref's device (checked after
    the shapes, so the shape checks run without a GPU)."""
    _need_dev(ref, *ts)
    for t in ts:
        if t is not None and t.device != ref.device:
            raise ValueError(f"tensors must share one device: {t.device} vs {ref.device}")


_I32 = torch.int32
_F32 = torch.float32


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
                ("balanced_groups", ctypes.c_int), ("even_split", ctypes.c_int)]


def attn_decode_gqa_plan(B, H_q, H_kv, T_cap, d, dtype, window=0, ring=False,
                         n_global=0, num_splits=0, q_len=1):
    """How a GQA decode call would run: dict with kernel ("valu" / "mfma"),
    splits, chunk, heads_per_item, tile_rows, waves, groups, workspace_bytes,
    balanced_groups, even_split."""
    p = _GqaPlan()
    st = library().attn_decode_gqa_plan(B, q_len, H_q, H_kv, T_cap, d, dtype,
                                        window, int(bool(ring)), n_global,
                                        num_splits, ctypes.byref(p))
    _check("attn_decode_gqa_plan", st)
    return {"kernel": "mfma" if p.kernel else "valu", "splits": p.splits,
            "chunk": p.chunk, "heads_per_item": p.heads_per_item,
            "tile_rows": p.tile_rows, "waves": p.waves, "groups": p.groups,
            "workspace_bytes": p.workspace_bytes,
            "balanced_groups": p.balanced_groups, "even_split": bool(p.even_split)}


def attn_decode_workspace_bytes(B, H, d_v, num_splits):
    return library().attn_decode_workspace_bytes(B, H, d_v, num_splits)


def attn_status_string(status):
    return library().attn_status_string(status).decode()


def _empty(shape, dtype, device):
    """Every output and workspace the binding allocates comes from here (one
    place a test can wrap, e.g. with guard bands around each buffer)."""
    return torch.empty(shape, dtype=dtype, device=device)


def _workspace(nbytes, device, workspace):
    if nbytes == 0:
        return workspace
    if workspace is None or workspace.numel() * workspace.element_size() < nbytes:
        workspace = _empty((nbytes,), torch.uint8, device)
    return workspace


def _gqa_shapes(q, k, v, out, lse, seq_lens, ring_head, q_dims=3):
    """B, L, H_q, d, H_kv, T_cap of a GQA call, after checking every tensor's
    shape and dtype against them: q [B, H_q, d] (or [B, L, H_q, d]), k and v
    [B, H_kv, T_cap, d] of q's dtype, out / lse float32 shaped like q,
    seq_lens / ring_head int32 [B]."""
    shp = _dims(q, "q", q_dims)
    B, H_q, d = shp[0], shp[-2], shp[-1]
    L = shp[1] if len(shp) == 4 else 1
    _dtype_code(q)
    _, H_kv, T_cap, dk = _dims(k, "k", 4)
    _expect(k, "k", (B, H_kv, T_cap, d))
    _expect(v, "v", tuple(k.shape))
    _same_dtype(q, ("k", k), ("v", v))
    _expect(out, "out", shp, _F32)
    _expect(lse, "lse", shp[:-1], _F32)
    _expect(seq_lens, "seq_lens", (B,), _I32)
    _expect(ring_head, "ring_head", (B,), _I32)
    return B, L, H_q, d, H_kv, T_cap


def attn_decode_gqa(q, k, v, seq_lens=None, ring_head=None, window=0,
                    scale=None, num_splits=0, out=None, lse=None,
                    workspace=None, want_lse=True, stream=None):
    """One decode step of MHA/GQA/MQA attention.

    q [B, H_q, d], k/v [B, H_kv, T_cap, d] (float32 or bfloat16, same dtype),
    seq_lens / ring_head int32 [B] or None.  Returns ``(out, lse)`` float32
    tensors ([B, H_q, d], [B, H_q] or None).  See include/attn_decode.h.
    """
    B, _, H_q, d, H_kv, T_cap = _gqa_shapes(q, k, v, out, lse, seq_lens, ring_head)
    _on_device(q, k, v, seq_lens, ring_head, out, lse, workspace)
    dt = _dtype_code(q)
    if out is None:
        out = _empty((B, H_q, d), torch.float32, q.device)
    if lse is None and want_lse:
        lse = _empty((B, H_q), torch.float32, q.device)
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


def attn_decode_gqa_noalloc(q, k, v, out, lse=None, seq_lens=None,
                            ring_head=None, window=0, scale=None, num_splits=0,
                            stream=None):
    """attn_decode_gqa with its split results in the library's per-GPU
    device array (no workspace, nothing allocated by the call): ``out``
    [B, H_q, d] float32 and the optional ``lse`` [B, H_q] float32 are
    supplied by the caller.  Calls that overlap on one GPU race (they share
    the array)."""
    if out is None:
        raise ValueError("out is required: the no-allocation form allocates nothing")
    B, _, H_q, d, H_kv, T_cap = _gqa_shapes(q, k, v, out, lse, seq_lens, ring_head)
    _on_device(q, k, v, seq_lens, ring_head, out, lse)
    st = library().attn_decode_gqa_noalloc(
        _ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), _ptr(seq_lens),
        _ptr(ring_head), B, H_q, H_kv, T_cap, d, _dtype_code(q), window,
        0.0 if scale is None else float(scale), num_splits,
        _stream(stream, q.device))
    _check("attn_decode_gqa_noalloc", st)
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
    B, _, H_q, d, H_kv, T_cap = _gqa_shapes(q, k, v, out, lse, seq_lens, None)
    if global_pos is not None:
        _dims(global_pos, "global_pos", 1)
        _expect(global_pos, "global_pos", dtype=_I32)
    _on_device(q, k, v, seq_lens, global_pos, out, lse, workspace)
    dt = _dtype_code(q)
    n_global = 0 if global_pos is None else global_pos.numel()
    if out is None:
        out = _empty((B, H_q, d), torch.float32, q.device)
    if lse is None and want_lse:
        lse = _empty((B, H_q), torch.float32, q.device)
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


def _mla_shapes(q, latent, d_c, out, lse, seq_lens, q_dims=3, paged=False):
    """B, L, H, dk of an MLA call after checking q [B, H, dk] (or [B, L, H,
    dk]) and the latent (or its page pool) bfloat16 with rows of dk, out /
    lse float32 shaped like q with d_c values, seq_lens int32 [B]."""
    shp = _dims(q, "q", q_dims)
    B, H, dk = shp[0], shp[-2], shp[-1]
    L = shp[1] if len(shp) == 4 else 1
    _expect(q, "q", dtype=torch.bfloat16)
    lshp = _dims(latent, "latent_pages" if paged else "latent", 3)
    if lshp[2] != dk or (not paged and lshp[0] != B):
        raise ValueError(f"latent rows must be [{'num_pages, P' if paged else f'{B}, T_cap'}, {dk}], "
                         f"got shape {lshp}")
    _expect(latent, "latent", dtype=torch.bfloat16)
    if not 0 < d_c < dk:
        raise ValueError(f"d_c must be in (0, {dk}), got {d_c}")
    _expect(out, "out", shp[:-1] + (d_c,), _F32)
    _expect(lse, "lse", shp[:-1], _F32)
    _expect(seq_lens, "seq_lens", (B,), _I32)
    return B, L, H, dk


def attn_decode_mla(q, latent, d_c, scale, seq_lens=None, num_splits=0,
                    out=None, lse=None, workspace=None, want_lse=True,
                    stream=None):
    """Absorbed MLA decode: q [B, H, d_c+d_rope], latent [B, T_cap, d_c+d_rope]
    (bfloat16).  Returns ``(z [B, H, d_c], lse [B, H])`` float32."""
    B, _, H, dk = _mla_shapes(q, latent, d_c, out, lse, seq_lens)
    _on_device(q, latent, seq_lens, out, lse, workspace)
    T_cap = latent.shape[1]
    d_rope = dk - d_c
    if out is None:
        out = _empty((B, H, d_c), torch.float32, q.device)
    if lse is None and want_lse:
        lse = _empty((B, H), torch.float32, q.device)
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
    B, H, S, d_v = _dims(o_part, "o_part", 4)
    _expect(o_part, "o_part", dtype=_F32)
    _expect(lse_part, "lse_part", (B, H, S), _F32)
    _expect(out, "out", (B, H, d_v), _F32)
    _expect(lse, "lse", (B, H), _F32)
    _on_device(o_part, lse_part, out, lse)
    if out is None:
        out = _empty((B, H, d_v), torch.float32, o_part.device)
    if lse is None and want_lse:
        lse = _empty((B, H), torch.float32, o_part.device)
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


def _append_shapes(k_cache, k_new, v_cache, v_new, B, H, d, index, index_name):
    """New rows [B, H, d] ([B, d] for a three-dimensional cache) of the
    cache's dtype, v given with both or neither of its tensors and shaped
    like k, the index tensor int32 [B]."""
    _dtype_code(k_cache)
    row = (B, H, d) if k_cache.dim() == 4 else (B, d)
    _expect(k_new, "k_new", row, k_cache.dtype)
    if (v_cache is None) != (v_new is None):
        raise ValueError("v_cache and v_new go together (both or neither)")
    _expect(v_cache, "v_cache", tuple(k_cache.shape), k_cache.dtype)
    _expect(v_new, "v_new", row, k_cache.dtype)
    _expect(index, index_name, (B,), _I32)


def attn_kv_append(k_cache, k_new, positions, v_cache=None, v_new=None,
                   stream=None):
    """Write k_new (and v_new) [B, H, d] at row positions[b] of the cache."""
    B, H, T_cap, d = _cache_dims(k_cache)
    _append_shapes(k_cache, k_new, v_cache, v_new, B, H, d, positions, "positions")
    _on_device(k_cache, k_new, positions, v_cache, v_new)
    st = library().attn_kv_append(_ptr(k_cache), _ptr(v_cache), _ptr(k_new),
                                  _ptr(v_new), _ptr(positions), B, H, T_cap, d,
                                  _dtype_code(k_cache), _stream(stream, k_cache.device))
    _check("attn_kv_append", st)


def attn_kv_append_ring(k_cache, k_new, ring_head, v_cache=None, v_new=None,
                        stream=None):
    """Advance ring_head[b] (in place) and write the rows at the new slot."""
    B, H, T_cap, d = _cache_dims(k_cache)
    _append_shapes(k_cache, k_new, v_cache, v_new, B, H, d, ring_head, "ring_head")
    _on_device(k_cache, k_new, ring_head, v_cache, v_new)
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
    shp = _dims(q, "q", (3, 4))
    B, H_q, d = shp[0], shp[-2], shp[-1]
    L = shp[1] if len(shp) == 4 else 1
    lead = shp[:-2]
    _dtype_code(q)
    num_pages, H_kv, P, _ = _dims(k_pages, "k_pages", 4)
    _expect(k_pages, "k_pages", (num_pages, H_kv, P, d))
    _expect(v_pages, "v_pages", tuple(k_pages.shape))
    _same_dtype(q, ("k_pages", k_pages), ("v_pages", v_pages))
    _expect(block_table, "block_table", dtype=_I32, min_rows=B)
    _expect(out, "out", shp, _F32)
    _expect(lse, "lse", shp[:-1], _F32)
    _expect(seq_lens, "seq_lens", (B,), _I32)
    _on_device(q, k_pages, v_pages, block_table, seq_lens, out, lse, workspace)
    max_pages = block_table.shape[1]
    dt = _dtype_code(q)
    if out is None:
        out = _empty((*lead, H_q, d), torch.float32, q.device)
    if lse is None and want_lse:
        lse = _empty((*lead, H_q), torch.float32, q.device)
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
    B, L, H_q, d, H_kv, T_cap = _gqa_shapes(q, k, v, out, lse, seq_lens, ring_head,
                                            q_dims=4)
    _on_device(q, k, v, seq_lens, ring_head, out, lse, workspace)
    dt = _dtype_code(q)
    if out is None:
        out = _empty((B, L, H_q, d), torch.float32, q.device)
    if lse is None and want_lse:
        lse = _empty((B, L, H_q), torch.float32, q.device)
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
    B, L, H, dk = _mla_shapes(q, latent_pages, d_c, out, lse, seq_lens, (3, 4),
                              paged=True)
    _expect(block_table, "block_table", dtype=_I32, min_rows=B)
    _on_device(q, latent_pages, block_table, seq_lens, out, lse, workspace)
    lead = tuple(q.shape[:-2])
    num_pages, P, _ = latent_pages.shape
    max_pages = block_table.shape[1]
    d_rope = dk - d_c
    if out is None:
        out = _empty((*lead, H, d_c), torch.float32, q.device)
    if lse is None and want_lse:
        lse = _empty((*lead, H), torch.float32, q.device)
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
    B, L, H, dk = _mla_shapes(q, latent, d_c, out, lse, seq_lens, 4)
    _on_device(q, latent, seq_lens, out, lse, workspace)
    T_cap = latent.shape[1]
    d_rope = dk - d_c
    if out is None:
        out = _empty((B, L, H, d_c), torch.float32, q.device)
    if lse is None and want_lse:
        lse = _empty((B, L, H), torch.float32, q.device)
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
    if k_pages.dim() == 3:
        num_pages, P, d = k_pages.shape
        H = 1
    elif k_pages.dim() == 4:
        num_pages, H, P, d = k_pages.shape
    else:
        raise ValueError("k_pages must be [num_pages, H, P, d] or [num_pages, P, d]")
    B = _dims(positions, "positions", 1)[0]
    _append_shapes(k_pages, k_new, v_pages, v_new, B, H, d, positions, "positions")
    _expect(block_table, "block_table", dtype=_I32, min_rows=B)
    _on_device(k_pages, k_new, positions, block_table, v_pages, v_new)
    st = library().attn_kv_append_paged(
        _ptr(k_pages), _ptr(v_pages), _ptr(k_new), _ptr(v_new), _ptr(positions),
        _ptr(block_table), block_table.shape[1], B, H, num_pages, P, d,
        _dtype_code(k_pages), _stream(stream, k_pages.device))
    _check("attn_kv_append_paged", st)


def attn_probe_read(src, sink, blocks=0, stream=None):
    """Stream-read every byte of ``src`` once (HBM read-rate probe)."""
    _expect(sink, "sink", dtype=_I32)
    if sink.numel() < 1:
        raise ValueError("sink must hold at least one int32")
    _on_device(src, sink)
    st = library().attn_probe_read(_ptr(src), src.numel() * src.element_size(),
                                   _ptr(sink), blocks, _stream(stream, src.device))
    _check("attn_probe_read", st)


def attn_probe_copy(dst, src, stream=None):
    """dst <- src byte for byte (a copy of known size)."""
    if dst.numel() * dst.element_size() < src.numel() * src.element_size():
        raise ValueError("dst is smaller than src")
    _on_device(src, dst)
    st = library().attn_probe_copy(_ptr(dst), _ptr(src),
                                   src.numel() * src.element_size(),
                                   _stream(stream, src.device))
    _check("attn_probe_copy", st)


def default_scale(d):
    """1/sqrt(d), the default softmax scale of the attention equation."""
    return 1.0 / math.sqrt(d)
