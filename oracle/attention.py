"""Vectorised float64 reference for decode attention (test infrastructure only).

This module is the plain definition of what one decode step computes; the
package docstring lists the pages cited here and who may import it.

Conventions (the readings of the pages this reference takes):

* One query token per sequence.  The cache of sequence ``b`` holds ``T_b``
  tokens including the current one, so the query sits at position
  ``t = T_b - 1`` and full causal attention sees positions ``0..t``
  [attention-head section 5.3: single-token causal decode, cache holds only the
  valid tokens up to the current position].
* Mask ``M``: a position is either visible (adds 0) or masked (adds -inf and
  drops out of the softmax); there is no other additive bias
  [attention-head section 1, attention equation; toolsku MHA module,
  masked_fill with -inf].
* Query head ``h`` reads KV head ``floor(h / n)`` with ``n = H_q / H_kv``:
  equal-size groups numbered contiguously [attention-head section 2;
  toolsku GQA module, ``_repeat_kv`` repeats each KV head n times in a row].
* Sliding window ``w > 0``: the query at ``t`` sees ``t-w+1 .. t`` (w keys
  including itself) [attention-head section 3, worked example w=3, row 8 sees
  6, 7, 8].
* Ring buffer (the pages say only that a pure sliding-window layer may recycle
  out-of-window slots in a ring buffer, attention-head section 3): the cache
  has ``S_cap = T_cap`` slots; ``ring_head[b]`` is the slot that holds the
  newest position ``t``; position ``j`` lives in slot
  ``(ring_head[b] - (t - j)) mod S_cap``; resident positions are
  ``max(0, T_b - S_cap) .. t``; visible = resident and inside the window,
  where ``window == 0`` means the whole resident set.
* Softmax scale defaults to ``1/sqrt(d)`` [attention-head section 1].
* An empty visible set yields ``out = 0`` and ``lse = -inf`` (the pages are
  silent; chosen so empty partial results merge uniformly).
* ``lse`` is the natural-log log-sum-exp of the scaled scores.
"""

import math

import numpy as np

__all__ = [
    "kv_cache_bytes",
    "mla_cache_bytes",
    "mla_explicit_cache_bytes",
    "visible_positions",
    "ring_slot",
    "attend",
    "gqa_decode_ref",
    "mla_decode_ref",
    "mla_explicit_ref",
    "combine_ref",
    "partial_ref",
    "kv_append_ref",
    "kv_append_ring_ref",
    "gqa_decode_multi_ref",
    "mla_decode_multi_ref",
    "paged_positions",
    "gqa_decode_paged_ref",
    "mla_decode_paged_ref",
    "kv_append_paged_ref",
]


# --------------------------------------------------------------------------
# Byte accounting
# --------------------------------------------------------------------------
def kv_cache_bytes(B, T, H_kv, d, s, layers=1):
    """Bytes of the K and V cache: ``2 * B * T * H_kv * d * s`` per layer.

    [attention-head section 1, the Bytes_KV equation: the factor 2 is K plus V;
    section 2 restates it for the [batch, head, sequence, head_dim] layout.]
    """
    return 2 * B * T * H_kv * d * s * layers


def mla_cache_bytes(B, T, r, d_rope, s, layers=1):
    """Bytes of an MLA latent cache: ``B * T * (r + d_R) * s`` per layer.

    No factor 2: the latent row carries both keys and values, the second term
    is the shared RoPE key [attention-head section 5.4, Bytes_MLA].
    """
    return B * T * (r + d_rope) * s * layers


def mla_explicit_cache_bytes(B, T, H, d_c, d_rope, d_v, s, layers=1):
    """Bytes of caching every head's expanded K and V: ``B*T*H*(d_c+d_R+d_v)*s``.

    [attention-head section 5.4, the element count of the explicit per-head
    cache used as the comparison point.]
    """
    return B * T * H * (d_c + d_rope + d_v) * s * layers


# --------------------------------------------------------------------------
# Index logic
# --------------------------------------------------------------------------
def _kv_head_for_query(h, n):
    """KV head read by query head ``h`` when ``n`` query heads share one.

    [attention-head section 2: equal-size, contiguously numbered groups;
    toolsku GQA module: ``_repeat_kv`` expands KV head g into query heads
    g*n .. g*n+n-1.]
    """
    return h // n


def _window_low(t, window):
    """First visible position of the query at ``t`` under window ``window``.

    [attention-head section 3: a window of width w keeps the current position
    and the w-1 before it.]  ``window == 0`` means no window.
    """
    if window > 0:
        return max(0, t - window + 1)
    return 0


def visible_positions(T_b, window=0, ring_capacity=None, global_pos=None):
    """Logical positions visible to the decode query of a length-``T_b`` sequence.

    With ``ring_capacity`` set, only the last ``ring_capacity`` positions are
    still resident in the ring buffer [attention-head section 3, ring-buffer
    reuse of out-of-window slots].

    ``global_pos`` (linear cache only) lists global token positions: every
    query also sees the global positions at or before it, and a query that is
    itself global sees its whole history [attention-head section 3, the
    window-plus-global pattern with G = {0, 5}: row 8 reaches 0 and 5 as well
    as 6, 7, 8; row 5 reaches 0..5].
    """
    if T_b <= 0:
        return np.zeros(0, dtype=np.int64)
    t = T_b - 1
    lo = _window_low(t, window)
    if ring_capacity is not None:
        lo = max(lo, T_b - ring_capacity)
    if global_pos is not None and len(global_pos):
        g = {int(x) for x in np.asarray(global_pos).reshape(-1)}
        if t in g:
            return np.arange(0, t + 1, dtype=np.int64)
        extra = sorted(x for x in g if 0 <= x < lo)
        return np.concatenate([np.array(extra, dtype=np.int64),
                               np.arange(lo, t + 1, dtype=np.int64)])
    return np.arange(lo, t + 1, dtype=np.int64)


def ring_slot(positions, t, ring_head, capacity):
    """Slot of logical position(s) ``positions`` in a ring whose newest
    position ``t`` sits in slot ``ring_head``."""
    return (ring_head - (t - np.asarray(positions, dtype=np.int64))) % capacity


# --------------------------------------------------------------------------
# The attention definition
# --------------------------------------------------------------------------
def attend(q_rows, k_rows, v_rows, scale):
    """softmax(scale * q K^T) V over an explicit key set, in float64.

    ``q_rows`` [n, d_k], ``k_rows`` [m, d_k], ``v_rows`` [m, d_v].  Returns
    ``(o [n, d_v], lse [n])``.  With ``m == 0``: ``o = 0``, ``lse = -inf``.

    [attention-head section 1, attention equation, with the mask already
    applied by passing only the visible keys; the softmax normalises along
    the key positions.]
    """
    q_rows = np.asarray(q_rows, dtype=np.float64)
    k_rows = np.asarray(k_rows, dtype=np.float64)
    v_rows = np.asarray(v_rows, dtype=np.float64)
    n = q_rows.shape[0]
    d_v = v_rows.shape[1]
    if k_rows.shape[0] == 0:
        return np.zeros((n, d_v)), np.full(n, -np.inf)
    s = scale * (q_rows @ k_rows.T)                      # [n, m]
    m = s.max(axis=1, keepdims=True)
    p = np.exp(s - m)
    l = p.sum(axis=1, keepdims=True)
    o = (p @ v_rows) / l
    lse = (m + np.log(l))[:, 0]
    return o, lse


def _as_f64(x):
    if hasattr(x, "detach"):  # a torch tensor: exact upcast through float32
        x = x.detach().cpu().float().numpy()
    return np.asarray(x, dtype=np.float64)


def _as_int(x, B, default):
    if x is None:
        return [default] * B
    if hasattr(x, "detach"):
        x = x.detach().cpu().numpy()
    return [int(v) for v in np.asarray(x).reshape(-1)]


def gqa_decode_ref(q, k, v, seq_lens=None, ring_head=None, window=0,
                   scale=None, batches=None, kv_heads=None, global_pos=None):
    """One decode step of MHA / GQA / MQA attention.

    q [B, H_q, d], k [B, H_kv, T_cap, d], v [B, H_kv, T_cap, d_v].
    ``seq_lens[b]`` is the logical length T_b (default T_cap); ``ring_head``
    switches the cache to ring-buffer addressing with T_cap slots;
    ``window`` is the sliding-window width (0 = full causal, and in ring mode
    0 = the whole resident set); ``global_pos`` adds global positions to a
    linear cache's window (see ``visible_positions``).
    Returns ``(out [B, H_q, d_v], lse [B, H_q])``
    in float64.  ``batches`` / ``kv_heads`` restrict the work to a subset
    (other entries stay 0 / -inf), for sampled checks on large inputs.

    H_kv = H_q is MHA, H_kv = 1 is MQA, anything between that divides H_q is
    GQA [attention-head sections 2.1 and 2.2].
    """
    q = _as_f64(q)
    B, H_q, d = q.shape
    k_shape = tuple(k.shape)
    _, H_kv, T_cap, d_k = k_shape
    d_v = tuple(v.shape)[3]
    if d_k != d:
        raise ValueError("q and k head dims differ")
    if H_q % H_kv != 0:
        raise ValueError("H_q must be divisible by H_kv")
    if window < 0:
        raise ValueError("window must be >= 0")
    if ring_head is not None and window > T_cap:
        raise ValueError("window larger than the ring")
    if ring_head is not None and global_pos is not None:
        raise ValueError("global positions need a linear cache")
    gp = None
    if global_pos is not None:
        if hasattr(global_pos, "detach"):
            global_pos = global_pos.detach().cpu().numpy()
        gp = [int(x) for x in np.asarray(global_pos).reshape(-1)]
    n = H_q // H_kv
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    lens = _as_int(seq_lens, B, T_cap)
    heads = _as_int(ring_head, B, 0) if ring_head is not None else None
    group_of = np.array([_kv_head_for_query(h, n) for h in range(H_q)])

    out = np.zeros((B, H_q, d_v))
    lse = np.full((B, H_q), -np.inf)
    for b in (range(B) if batches is None else batches):
        T_b = lens[b]
        if heads is None:
            if T_b > T_cap:
                raise ValueError("seq_len exceeds the cache capacity")
            pos = visible_positions(T_b, window, global_pos=gp)
            slots = pos
        else:
            pos = visible_positions(T_b, window, ring_capacity=T_cap)
            slots = ring_slot(pos, T_b - 1, heads[b], T_cap)
        for g in (range(H_kv) if kv_heads is None else kv_heads):
            hs = np.nonzero(group_of == g)[0]
            if hs.size == 0:
                continue
            k_rows = _as_f64(k[b, g])[slots]
            v_rows = _as_f64(v[b, g])[slots]
            o, l = attend(q[b, hs], k_rows, v_rows, scale)
            out[b, hs] = o
            lse[b, hs] = l
    return out, lse


def mla_decode_ref(q, latent, d_c, scale, seq_lens=None, batches=None):
    """Absorbed MLA decode over a latent cache [B, T_cap, d_c + d_rope].

    Each latent row is ``[c_j | k^R_j]`` and each query row is
    ``[q~ | q^R]`` (content part first).  The score of position j is
    ``scale * (q~ . c_j + q^R . k^R_j)`` -- one dot product over the full
    row -- with a single softmax over the summed scores, and the result is
    the latent ``z = sum_j p_j c_j`` (the per-head value up-projection is
    applied after this step) [attention-head section 5.2: keys absorbed into
    the query, values projected after the weighted sum; section 5.3: the RoPE
    part adds a second score term and contributes no value].

    ``scale`` has no default: it is ``1/sqrt(d_c_head + d_R)`` with the
    per-head content-key width, which the latent shape does not carry
    [attention-head section 5.3: the denominator is not r + d_R].
    Returns ``(z [B, H, d_c], lse [B, H])``.
    """
    q = _as_f64(q)
    B, H, dk = q.shape
    _, T_cap, dk2 = tuple(latent.shape)
    if dk != dk2:
        raise ValueError("q and latent widths differ")
    if not (0 < d_c <= dk):
        raise ValueError("bad d_c")
    lens = _as_int(seq_lens, B, T_cap)
    z = np.zeros((B, H, d_c))
    lse = np.full((B, H), -np.inf)
    for b in (range(B) if batches is None else batches):
        T_b = lens[b]
        if T_b > T_cap:
            raise ValueError("seq_len exceeds the cache capacity")
        pos = visible_positions(T_b)
        rows = _as_f64(latent[b])[pos]
        o, l = attend(q[b], rows, rows[:, :d_c], scale)
        z[b] = o
        lse[b] = l
    return z, lse


def mla_explicit_ref(C, K_rope, q_content, q_rope, U_K, U_V, scale):
    """Non-absorbed MLA: expand every head's keys and values, then attend.

    C [B, T, r] latents, K_rope [B, T, d_R] shared RoPE keys,
    q_content [B, H, d_c_head], q_rope [B, H, d_R], U_K [H, r, d_c_head],
    U_V [H, r, d_v].  Head h uses keys ``[C U_K[h] | K_rope]`` and values
    ``C U_V[h]`` [attention-head section 5.1, per-head content keys and values
    from one shared latent; section 5.3, the RoPE key concatenated to the
    content key].  Full causal over all T positions.  Returns o [B, H, d_v].
    """
    C = _as_f64(C)
    K_rope = _as_f64(K_rope)
    q_content = _as_f64(q_content)
    q_rope = _as_f64(q_rope)
    U_K = _as_f64(U_K)
    U_V = _as_f64(U_V)
    B, T, r = C.shape
    H = q_content.shape[1]
    d_v = U_V.shape[2]
    out = np.zeros((B, H, d_v))
    for b in range(B):
        for h in range(H):
            keys = np.concatenate([C[b] @ U_K[h], K_rope[b]], axis=1)
            vals = C[b] @ U_V[h]
            qh = np.concatenate([q_content[b, h], q_rope[b, h]])[None, :]
            o, _ = attend(qh, keys, vals, scale)
            out[b, h] = o[0]
    return out


# --------------------------------------------------------------------------
# Split results and their merge
# --------------------------------------------------------------------------
def partial_ref(q_rows, k_rows, v_rows, scale):
    """(o, lse) of attention restricted to one part of the key set; the same
    definition as ``attend``, named for its use on disjoint key subsets."""
    return attend(q_rows, k_rows, v_rows, scale)


def combine_ref(o_part, lse_part):
    """Merge results computed over disjoint key subsets.

    o_part [..., S, d_v], lse_part [..., S].  Softmax over a union of disjoint
    key sets: with ``L = max_s lse_s`` and ``w_s = exp(lse_s - L)``,
    ``out = sum_s w_s o_s / sum_s w_s`` and ``lse = L + log(sum_s w_s)``;
    all-empty gives out 0 and lse -inf.  This follows from the attention
    equation [attention-head section 1]: each part's normaliser is exp(lse_s).
    """
    o_part = _as_f64(o_part)
    lse_part = _as_f64(lse_part)
    L = lse_part.max(axis=-1, keepdims=True)
    empty = ~np.isfinite(L)
    Ls = np.where(empty, 0.0, L)
    w = np.where(np.isfinite(lse_part), np.exp(lse_part - Ls), 0.0)
    tot = w.sum(axis=-1, keepdims=True)
    safe = np.where(empty, 1.0, tot)
    out = (w[..., None] * o_part).sum(axis=-2) / safe
    out = np.where(empty, 0.0, out)
    lse = np.where(empty[..., 0], -np.inf, (Ls + np.log(safe))[..., 0])
    return out, lse


# --------------------------------------------------------------------------
# Cache append (the step before a decode call)
# --------------------------------------------------------------------------
def kv_append_ref(cache, new_rows, positions):
    """Linear cache: write each sequence's new row at its position.

    cache [B, H, T_cap, d] (or [B, T_cap, d] for a latent cache), new_rows
    [B, H, d] (or [B, d]), positions [B].  Returns a new array.  Appending
    the current token's key and value to the cached ones along the sequence
    axis is what the toolsku MHA / GQA / MLA modules do with ``past_kv``
    (``torch.cat`` on dim 2); here the cache is preallocated, so the append
    is a write at index T_b.  Positions outside [0, T_cap) are not written.
    """
    out = np.array(_as_f64(cache), copy=True)
    new_rows = _as_f64(new_rows)
    B = out.shape[0]
    T_cap = out.shape[-2]
    pos = _as_int(positions, B, 0)
    for b in range(B):
        if 0 <= pos[b] < T_cap:
            out[b, ..., pos[b], :] = new_rows[b]
    return out


def kv_append_ring_ref(cache, new_rows, ring_head):
    """Ring cache: advance each sequence's head one slot (mod T_cap) and write
    the new row there, overwriting the oldest position once the ring is full
    [attention-head section 3: a sliding-window layer may reuse the slots of
    positions that left the window].  Returns (new cache, new heads)."""
    out = np.array(_as_f64(cache), copy=True)
    new_rows = _as_f64(new_rows)
    B = out.shape[0]
    T_cap = out.shape[-2]
    heads = _as_int(ring_head, B, 0)
    new_heads = []
    for b in range(B):
        h = (heads[b] % T_cap + 1) % T_cap
        out[b, ..., h, :] = new_rows[b]
        new_heads.append(h)
    return out, np.array(new_heads, dtype=np.int64)


# --------------------------------------------------------------------------
# Paged caches
# --------------------------------------------------------------------------
# The baidu article (section 四.3) names KV-cache paging as the memory
# management a serving stack puts around GQA and MLA, without fixing a
# layout.  The reading taken here: a pool of pages of P consecutive
# positions; sequence b's position j lives in page block_table[b][j // P]
# at row j % P; a GQA page holds every KV head, [num_pages, H_kv, P, d], an
# MLA page the latent rows, [num_pages, P, d_c + d_rope].


def paged_positions(positions, block_table_row, page_size):
    """(page, row) of each logical position of one sequence."""
    positions = np.asarray(positions, dtype=np.int64)
    table = np.asarray(block_table_row, dtype=np.int64)
    return table[positions // page_size], positions % page_size


def gqa_decode_paged_ref(q, k_pages, v_pages, block_table, seq_lens=None,
                         window=0, scale=None):
    """Decode attention over a paged K/V pool: gather each sequence's rows
    through its block table into the linear layout, then apply the plain
    definition (``gqa_decode_ref``) to it.

    k_pages / v_pages [num_pages, H_kv, P, d]; block_table [B, max_pages];
    seq_lens [B] (default max_pages * P).
    """
    q64 = _as_f64(q)
    kp, vp = _as_f64(k_pages), _as_f64(v_pages)
    if hasattr(block_table, "detach"):
        block_table = block_table.detach().cpu().numpy()
    table = np.asarray(block_table, dtype=np.int64)
    B = q64.shape[0]
    _, H_kv, P, d = kp.shape
    T_cap = table.shape[1] * P
    lens = _as_int(seq_lens, B, T_cap)
    k_lin = np.zeros((B, H_kv, T_cap, d))
    v_lin = np.zeros((B, H_kv, T_cap, vp.shape[3]))
    for b in range(B):
        if lens[b] > T_cap:
            raise ValueError("seq_len exceeds the block table")
        pos = np.arange(lens[b])
        page, row = paged_positions(pos, table[b], P)
        k_lin[b][:, pos] = kp[page, :, row].transpose(1, 0, 2)
        v_lin[b][:, pos] = vp[page, :, row].transpose(1, 0, 2)
    return gqa_decode_ref(q64, k_lin, v_lin, lens, None, window, scale)


def mla_decode_paged_ref(q, latent_pages, block_table, d_c, scale,
                         seq_lens=None):
    """Absorbed MLA over a paged latent pool [num_pages, P, d_c + d_rope]:
    gather each sequence's rows through its block table, then apply
    ``mla_decode_ref``."""
    q64 = _as_f64(q)
    lp = _as_f64(latent_pages)
    if hasattr(block_table, "detach"):
        block_table = block_table.detach().cpu().numpy()
    table = np.asarray(block_table, dtype=np.int64)
    B = q64.shape[0]
    _, P, dk = lp.shape
    T_cap = table.shape[1] * P
    lens = _as_int(seq_lens, B, T_cap)
    lat = np.zeros((B, T_cap, dk))
    for b in range(B):
        if lens[b] > T_cap:
            raise ValueError("seq_len exceeds the block table")
        pos = np.arange(lens[b])
        page, row = paged_positions(pos, table[b], P)
        lat[b, pos] = lp[page, row]
    return mla_decode_ref(q64, lat, d_c, scale, lens)


def kv_append_paged_ref(pages, new_rows, positions, block_table):
    """Write each sequence's new row at its position of a paged pool.

    pages [num_pages, H, P, d] (or [num_pages, P, d] for a latent pool),
    new_rows [B, H, d] (or [B, d]), positions [B]; positions outside the
    block table are not written.  Returns a new array."""
    out = np.array(_as_f64(pages), copy=True)
    new_rows = _as_f64(new_rows)
    if hasattr(block_table, "detach"):
        block_table = block_table.detach().cpu().numpy()
    table = np.asarray(block_table, dtype=np.int64)
    latent = out.ndim == 3
    P = out.shape[1] if latent else out.shape[2]
    B = table.shape[0]
    pos = _as_int(positions, B, 0)
    for b in range(B):
        if 0 <= pos[b] < table.shape[1] * P:
            page, row = paged_positions([pos[b]], table[b], P)
            if latent:
                out[page[0], row[0]] = new_rows[b]
            else:
                out[page[0], :, row[0]] = new_rows[b]
    return out


# --------------------------------------------------------------------------
# Several query tokens per sequence
# --------------------------------------------------------------------------
# Speculative-decode verification and chunked prefill score L new tokens of a
# sequence in one call (the xuesongtap note, section 6, and the baidu
# article: longer contexts and more tokens per step are what the cache
# layouts are for).  The reading taken here: the L tokens are the last L
# positions of the cache, already written (positions T_b-L .. T_b-1); token
# l sits at t_l = T_b - L + l and sees what a single decode query at t_l
# sees -- positions 0..t_l (causal inside the chunk), cut to its own window
# t_l-w+1..t_l, and in a ring only positions still resident after all L
# tokens were written (the newest is T_b - 1).  A token with t_l < 0 sees
# nothing.  Layout: q [B, L, H_q, d] (token-major), outputs [B, L, H_q, d_v]
# and [B, L, H_q].


def _chunk_position(T_b, L, l):
    """Position of query token l of an L-token chunk that ends the cache."""
    return T_b - L + l


def gqa_decode_multi_ref(q, k, v, seq_lens=None, ring_head=None, window=0,
                         scale=None):
    """L query tokens per sequence against a head-shared K/V cache."""
    q = _as_f64(q)
    B, L, H_q, d = q.shape
    _, H_kv, T_cap, _ = tuple(k.shape)
    d_v = tuple(v.shape)[3]
    if H_q % H_kv != 0:
        raise ValueError("H_q must be divisible by H_kv")
    if ring_head is not None and window + L - 1 > T_cap:
        raise ValueError("the ring must hold the first token's window")
    n = H_q // H_kv
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    lens = _as_int(seq_lens, B, T_cap)
    heads = _as_int(ring_head, B, 0) if ring_head is not None else None
    out = np.zeros((B, L, H_q, d_v))
    lse = np.full((B, L, H_q), -np.inf)
    for b in range(B):
        T_b = lens[b]
        if heads is None and T_b > T_cap:
            raise ValueError("seq_len exceeds the cache capacity")
        newest = T_b - 1
        for l in range(L):
            t = _chunk_position(T_b, L, l)
            if t < 0:
                continue
            lo = _window_low(t, window)
            if heads is not None:
                lo = max(lo, T_b - T_cap)     # resident after the whole chunk
            pos = np.arange(lo, t + 1, dtype=np.int64)
            slots = pos if heads is None else ring_slot(pos, newest, heads[b], T_cap)
            for g in range(H_kv):
                hs = [h for h in range(H_q) if _kv_head_for_query(h, n) == g]
                k_rows = _as_f64(k[b, g])[slots]
                v_rows = _as_f64(v[b, g])[slots]
                o, m = attend(q[b, l, hs], k_rows, v_rows, scale)
                out[b, l, hs] = o
                lse[b, l, hs] = m
    return out, lse


def mla_decode_multi_ref(q, latent, d_c, scale, seq_lens=None):
    """Absorbed MLA with L query tokens per sequence (token l at
    T_b - L + l sees positions 0..T_b-L+l); q [B, L, H, d_c + d_rope]."""
    q = _as_f64(q)
    B, L, H, dk = q.shape
    _, T_cap, _ = tuple(latent.shape)
    lens = _as_int(seq_lens, B, T_cap)
    z = np.zeros((B, L, H, d_c))
    lse = np.full((B, L, H), -np.inf)
    for b in range(B):
        if lens[b] > T_cap:
            raise ValueError("seq_len exceeds the cache capacity")
        lat = _as_f64(latent[b])
        for l in range(L):
            t = _chunk_position(lens[b], L, l)
            if t < 0:
                continue
            rows = lat[:t + 1]
            o, m = attend(q[b, l], rows, rows[:, :d_c], scale)
            z[b, l] = o
            lse[b, l] = m
    return z, lse
