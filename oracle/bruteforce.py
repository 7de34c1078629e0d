"""Pure-Python scalar loops for tiny inputs (test infrastructure only).

A second, independently structured statement of the same method, used to pin
the vectorised reference in ``oracle.attention``.  It walks every cache slot
and decides visibility slot by slot (the inverse direction of the vectorised
reference, which maps positions to slots), uses ``h * H_kv // H_q`` for the
group of a query head, and accumulates with ``math.fsum``.  Sizes: a handful
of heads, tens of positions.  The pages cited are listed in ``oracle``'s
package docstring.
"""

import math


def _lst(x):
    if hasattr(x, "detach"):
        x = x.detach().cpu().double().numpy()
    if hasattr(x, "tolist"):
        return x.tolist()
    return x


def _slot_position(slot, t, ring_head, capacity):
    """Logical position held by ``slot`` of a ring whose newest position ``t``
    sits in ``ring_head``: walking back from the head, each slot is one
    position older [attention-head section 3, ring-buffer reuse]."""
    age = (ring_head - slot) % capacity
    return t - age


def visible_slots_brute(T_b, T_cap, window=0, ring_head=None, global_pos=None):
    """List of (slot, position) pairs the decode query reads, by testing each
    slot of the cache one at a time.  ``global_pos``: positions every query
    may also see; a global query sees everything before it (linear cache)."""
    if T_b <= 0:
        return []
    t = T_b - 1
    gset = set() if global_pos is None else {int(x) for x in global_pos}
    out = []
    for slot in range(T_cap):
        if ring_head is None:
            pos = slot
            if pos > t:          # not written yet (or beyond this sequence)
                continue
        else:
            pos = _slot_position(slot, t, ring_head, T_cap)
            if pos < 0:          # the ring has not wrapped this far yet
                continue
        if window > 0 and t - pos >= window:   # older than the window
            if pos not in gset and t not in gset:
                continue
        out.append((slot, pos))
    out.sort(key=lambda sp: sp[1])
    return out


def _softmax_weighted(scores, values):
    mx = max(scores)
    w = [math.exp(s - mx) for s in scores]
    tot = math.fsum(w)
    d_v = len(values[0])
    o = [math.fsum(w[j] * values[j][i] for j in range(len(w))) / tot
         for i in range(d_v)]
    return o, mx + math.log(tot)


def gqa_decode_brute(q, k, v, seq_lens=None, ring_head=None, window=0,
                     scale=None, global_pos=None):
    """Scalar-loop decode attention; same contract as
    ``oracle.attention.gqa_decode_ref``, returns nested lists."""
    q, k, v = _lst(q), _lst(k), _lst(v)
    B, H_q, d = len(q), len(q[0]), len(q[0][0])
    H_kv, T_cap = len(k[0]), len(k[0][0])
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    lens = [T_cap] * B if seq_lens is None else [int(x) for x in _lst(seq_lens)]
    heads = None if ring_head is None else [int(x) for x in _lst(ring_head)]
    out, lse = [], []
    for b in range(B):
        sl = visible_slots_brute(lens[b], T_cap, window,
                                 None if heads is None else heads[b], global_pos)
        ob, lb = [], []
        for h in range(H_q):
            g = h * H_kv // H_q
            if not sl:
                ob.append([0.0] * len(v[0][0][0]))
                lb.append(-math.inf)
                continue
            scores = [scale * math.fsum(q[b][h][i] * k[b][g][s][i]
                                        for i in range(d)) for s, _ in sl]
            vals = [v[b][g][s] for s, _ in sl]
            o, l = _softmax_weighted(scores, vals)
            ob.append(o)
            lb.append(l)
        out.append(ob)
        lse.append(lb)
    return out, lse


def mla_decode_brute(q, latent, d_c, scale, seq_lens=None):
    """Scalar-loop absorbed MLA: the content score and the RoPE score are
    computed as two separate sums and added before the softmax
    [attention-head section 5.3]; the value is the first ``d_c`` latent
    columns."""
    q, latent = _lst(q), _lst(latent)
    B, H, dk = len(q), len(q[0]), len(q[0][0])
    T_cap = len(latent[0])
    lens = [T_cap] * B if seq_lens is None else [int(x) for x in _lst(seq_lens)]
    out, lse = [], []
    for b in range(B):
        T_b = lens[b]
        ob, lb = [], []
        for h in range(H):
            if T_b <= 0:
                ob.append([0.0] * d_c)
                lb.append(-math.inf)
                continue
            scores = []
            for j in range(T_b):
                content = math.fsum(q[b][h][i] * latent[b][j][i] for i in range(d_c))
                rope = math.fsum(q[b][h][i] * latent[b][j][i] for i in range(d_c, dk))
                scores.append(scale * (content + rope))
            vals = [latent[b][j][:d_c] for j in range(T_b)]
            o, l = _softmax_weighted(scores, vals)
            ob.append(o)
            lb.append(l)
        out.append(ob)
        lse.append(lb)
    return out, lse


def combine_brute(o_part, lse_part):
    """Merge per-split results one output at a time with scalar loops."""
    o_part, lse_part = _lst(o_part), _lst(lse_part)
    res_o, res_l = [], []
    for ob, lb in zip(o_part, lse_part):
        ro, rl = [], []
        for oh, lh in zip(ob, lb):
            finite = [i for i, x in enumerate(lh) if x != -math.inf]
            d_v = len(oh[0])
            if not finite:
                ro.append([0.0] * d_v)
                rl.append(-math.inf)
                continue
            L = max(lh[i] for i in finite)
            w = {i: math.exp(lh[i] - L) for i in finite}
            tot = math.fsum(w.values())
            ro.append([math.fsum(w[i] * oh[i][e] for i in finite) / tot
                       for e in range(d_v)])
            rl.append(L + math.log(tot))
        res_o.append(ro)
        res_l.append(rl)
    return res_o, res_l


def gqa_decode_paged_brute(q, k_pages, v_pages, block_table, seq_lens,
                           window=0, scale=None):
    """Scalar-loop decode over a paged pool: walk every block-table entry and
    every row of its page, derive the row's logical position from where it
    sits (entry index * P + row), and keep it if it is visible."""
    q, kp, vp = _lst(q), _lst(k_pages), _lst(v_pages)
    table = [[int(x) for x in row] for row in _lst(block_table)]
    B, H_q, d = len(q), len(q[0]), len(q[0][0])
    H_kv, P = len(kp[0]), len(kp[0][0])
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    lens = [int(x) for x in _lst(seq_lens)]
    out, lse = [], []
    for b in range(B):
        t = lens[b] - 1
        rows = []  # (position, page, row)
        for j, page in enumerate(table[b]):
            for r in range(P):
                pos = j * P + r
                if pos > t:
                    continue
                if window > 0 and t - pos >= window:
                    continue
                rows.append((pos, page, r))
        ob, lb = [], []
        for h in range(H_q):
            g = h * H_kv // H_q
            if not rows:
                ob.append([0.0] * len(vp[0][0][0]))
                lb.append(-math.inf)
                continue
            scores = [scale * math.fsum(q[b][h][i] * kp[page][g][r][i]
                                        for i in range(d)) for _, page, r in rows]
            vals = [vp[page][g][r] for _, page, r in rows]
            o, l = _softmax_weighted(scores, vals)
            ob.append(o)
            lb.append(l)
        out.append(ob)
        lse.append(lb)
    return out, lse


def mla_decode_paged_brute(q, latent_pages, block_table, d_c, scale, seq_lens):
    """Scalar-loop absorbed MLA over a paged latent pool (same walk as
    ``gqa_decode_paged_brute``; content and RoPE sums kept apart)."""
    q, lp = _lst(q), _lst(latent_pages)
    table = [[int(x) for x in row] for row in _lst(block_table)]
    B, H, dk = len(q), len(q[0]), len(q[0][0])
    P = len(lp[0])
    lens = [int(x) for x in _lst(seq_lens)]
    out, lse = [], []
    for b in range(B):
        rows = [(j * P + r, page, r) for j, page in enumerate(table[b])
                for r in range(P) if j * P + r < lens[b]]
        ob, lb = [], []
        for h in range(H):
            if not rows:
                ob.append([0.0] * d_c)
                lb.append(-math.inf)
                continue
            scores = []
            for _, page, r in rows:
                row = lp[page][r]
                content = math.fsum(q[b][h][i] * row[i] for i in range(d_c))
                rope = math.fsum(q[b][h][i] * row[i] for i in range(d_c, dk))
                scores.append(scale * (content + rope))
            vals = [lp[page][r][:d_c] for _, page, r in rows]
            o, l = _softmax_weighted(scores, vals)
            ob.append(o)
            lb.append(l)
        out.append(ob)
        lse.append(lb)
    return out, lse


def gqa_decode_multi_brute(q, k, v, seq_lens, ring_head=None, window=0,
                           scale=None):
    """Scalar loops for L query tokens per sequence: every cache slot is
    tested against every token (its position from the ring walk of the
    newest token, then causal and window tests per token)."""
    q, k, v = _lst(q), _lst(k), _lst(v)
    B, L, H_q, d = len(q), len(q[0]), len(q[0][0]), len(q[0][0][0])
    H_kv, T_cap = len(k[0]), len(k[0][0])
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    lens = [int(x) for x in _lst(seq_lens)]
    heads = None if ring_head is None else [int(x) for x in _lst(ring_head)]
    out, lse = [], []
    for b in range(B):
        newest = lens[b] - 1
        ob, lb = [], []
        for l in range(L):
            t = lens[b] - L + l
            seen = []
            for slot in range(T_cap):
                pos = slot if heads is None else _slot_position(slot, newest, heads[b], T_cap)
                if pos < 0 or pos > t:
                    continue
                if window > 0 and t - pos >= window:
                    continue
                seen.append(slot)
            ol, ll = [], []
            for h in range(H_q):
                g = h * H_kv // H_q
                if not seen:
                    ol.append([0.0] * len(v[0][0][0]))
                    ll.append(-math.inf)
                    continue
                sc = [scale * math.fsum(q[b][l][h][i] * k[b][g][s][i] for i in range(d))
                      for s in seen]
                o, m = _softmax_weighted(sc, [v[b][g][s] for s in seen])
                ol.append(o)
                ll.append(m)
            ob.append(ol)
            lb.append(ll)
        out.append(ob)
        lse.append(lb)
    return out, lse
