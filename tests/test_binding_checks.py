"""The Python binding rejects mismatched tensors before it calls the library.

Every check on shapes and dtypes runs before the device check, so these
tests use host tensors and need no GPU: a mismatch raises ValueError naming
the argument, and a call whose shapes are all right still stops at the
device check, so nothing is ever launched from here.
"""

import pytest
import torch

import decode_attention_kv_attn_amd as L

bf, f32, i32 = torch.bfloat16, torch.float32, torch.int32


def gqa_args(B=2, H_q=8, H_kv=2, T=16, d=64, dt=bf):
    return dict(q=torch.zeros(B, H_q, d, dtype=dt),
                k=torch.zeros(B, H_kv, T, d, dtype=dt),
                v=torch.zeros(B, H_kv, T, d, dtype=dt))


def raises(match, fn, *a, **kw):
    with pytest.raises(ValueError, match=match):
        fn(*a, **kw)


GQA_BAD = [
    ("k", lambda a: a.update(k=a["k"].float(), v=a["v"].float()), "dtype of q"),
    ("v", lambda a: a.update(v=a["v"].float()), "v must have the dtype"),
    ("k_dim", lambda a: a.update(k=torch.zeros(2, 2, 16, 32, dtype=bf),
                                 v=torch.zeros(2, 2, 16, 32, dtype=bf)), "k must have shape"),
    ("k_batch", lambda a: a.update(k=torch.zeros(3, 2, 16, 64, dtype=bf),
                                   v=torch.zeros(3, 2, 16, 64, dtype=bf)), "k must have shape"),
    ("v_shape", lambda a: a.update(v=torch.zeros(2, 2, 15, 64, dtype=bf)), "v must have shape"),
    ("k_rank", lambda a: a.update(k=torch.zeros(2, 16, 64, dtype=bf)), "k must have 4"),
    ("q_rank", lambda a: a.update(q=torch.zeros(2, 8, 1, 64, dtype=bf)), "q must have 3"),
    ("out_dtype", lambda a: a.update(out=torch.zeros(2, 8, 64, dtype=bf)), "out must be"),
    ("out_shape", lambda a: a.update(out=torch.zeros(2, 8, 63, dtype=f32)), "out must have shape"),
    ("lse_shape", lambda a: a.update(lse=torch.zeros(2, 7, dtype=f32)), "lse must have shape"),
    ("lens_dtype", lambda a: a.update(seq_lens=torch.zeros(2, dtype=torch.int64)), "seq_lens must be"),
    ("lens_len", lambda a: a.update(seq_lens=torch.zeros(3, dtype=i32)), "seq_lens must have shape"),
    ("head_dtype", lambda a: a.update(ring_head=torch.zeros(2, dtype=f32)), "ring_head must be"),
    ("head_len", lambda a: a.update(ring_head=torch.zeros(1, dtype=i32)), "ring_head must have shape"),
]


@pytest.mark.parametrize("what,mutate,match", GQA_BAD, ids=[x[0] for x in GQA_BAD])
def test_gqa_mismatch_raises(what, mutate, match):
    a = gqa_args()
    mutate(a)
    raises(match, L.attn_decode_gqa, **a)


def test_gqa_unknown_dtype_raises():
    a = gqa_args(dt=torch.float16)
    with pytest.raises(TypeError):
        L.attn_decode_gqa(**a)


def test_gqa_right_shapes_stop_at_the_device_check():
    a = gqa_args()
    raises("on the GPU", L.attn_decode_gqa, **a,
           seq_lens=torch.zeros(2, dtype=i32), ring_head=torch.zeros(2, dtype=i32),
           out=torch.zeros(2, 8, 64), lse=torch.zeros(2, 8))


def test_multi_and_global_checks():
    a = gqa_args()
    q4 = torch.zeros(2, 3, 8, 64, dtype=bf)
    raises("q must have 4", L.attn_decode_gqa_multi, **a)
    raises("out must have shape", L.attn_decode_gqa_multi, q4, a["k"], a["v"],
           out=torch.zeros(2, 8, 64))
    raises("on the GPU", L.attn_decode_gqa_multi, q4, a["k"], a["v"])
    raises("global_pos must be", L.attn_decode_gqa_global, a["q"], a["k"], a["v"],
           torch.zeros(3, dtype=torch.int64), 4)
    raises("global_pos must have 1", L.attn_decode_gqa_global, a["q"], a["k"], a["v"],
           torch.zeros(1, 3, dtype=i32), 4)


def test_paged_checks():
    q = torch.zeros(2, 8, 64, dtype=bf)
    kp = torch.zeros(6, 2, 16, 64, dtype=bf)
    table = torch.zeros(2, 3, dtype=i32)
    raises("v_pages must have shape", L.attn_decode_gqa_paged, q, kp,
           torch.zeros(6, 2, 16, 32, dtype=bf), table)
    raises("block_table must have at least 2 rows|block_table must be 2-D",
           L.attn_decode_gqa_paged, q, kp, kp, table[:1])
    raises("block_table must be", L.attn_decode_gqa_paged, q, kp, kp,
           table.to(torch.int64))
    raises("k_pages must have shape", L.attn_decode_gqa_paged, q,
           torch.zeros(6, 2, 16, 128, dtype=bf), torch.zeros(6, 2, 16, 128, dtype=bf), table)
    raises("dtype of q", L.attn_decode_gqa_paged, q, kp.float(), kp.float(), table)
    raises("on the GPU", L.attn_decode_gqa_paged, q, kp, kp, table)


def mla_args(B=2, H=16, T=64, dk=576):
    return (torch.zeros(B, H, dk, dtype=bf), torch.zeros(B, T, dk, dtype=bf))


def test_mla_checks():
    q, lat = mla_args()
    raises("q must be", L.attn_decode_mla, q.float(), lat, 512, 0.1)
    raises("latent must be", L.attn_decode_mla, q, lat.float(), 512, 0.1)
    raises("latent rows", L.attn_decode_mla, q, torch.zeros(2, 64, 320, dtype=bf), 512, 0.1)
    raises("latent rows", L.attn_decode_mla, q, torch.zeros(3, 64, 576, dtype=bf), 512, 0.1)
    raises("d_c must be", L.attn_decode_mla, q, lat, 576, 0.1)
    raises("out must have shape", L.attn_decode_mla, q, lat, 512, 0.1,
           out=torch.zeros(2, 16, 576))
    raises("lse must be", L.attn_decode_mla, q, lat, 512, 0.1,
           lse=torch.zeros(2, 16, dtype=torch.float64))
    raises("seq_lens must have shape", L.attn_decode_mla, q, lat, 512, 0.1,
           torch.zeros(1, dtype=i32))
    raises("on the GPU", L.attn_decode_mla, q, lat, 512, 0.1)
    q4 = torch.zeros(2, 2, 16, 576, dtype=bf)
    raises("q must have 4", L.attn_decode_mla_multi, q, lat, 512, 0.1)
    raises("on the GPU", L.attn_decode_mla_multi, q4, lat, 512, 0.1)
    pool = torch.zeros(8, 16, 576, dtype=bf)
    raises("block_table must", L.attn_decode_mla_paged, q, pool,
           torch.zeros(1, 4, dtype=i32), 512, 0.1)
    raises("latent rows", L.attn_decode_mla_paged, q, torch.zeros(8, 16, 320, dtype=bf),
           torch.zeros(2, 4, dtype=i32), 512, 0.1)
    raises("on the GPU", L.attn_decode_mla_paged, q4, pool,
           torch.zeros(2, 4, dtype=i32), 512, 0.1)


def test_combine_checks():
    o = torch.zeros(2, 3, 4, 64)
    raises("o_part must be", L.attn_combine, o.double(), torch.zeros(2, 3, 4))
    raises("lse_part must have shape", L.attn_combine, o, torch.zeros(2, 3, 5))
    raises("out must have shape", L.attn_combine, o, torch.zeros(2, 3, 4),
           out=torch.zeros(2, 3, 32))
    raises("on the GPU", L.attn_combine, o, torch.zeros(2, 3, 4))


def test_append_checks():
    k = torch.zeros(2, 3, 10, 64, dtype=bf)
    kn = torch.zeros(2, 3, 64, dtype=bf)
    pos = torch.zeros(2, dtype=i32)
    raises("k_new must have shape", L.attn_kv_append, k, kn[:, :2].contiguous(), pos)
    raises("k_new must be", L.attn_kv_append, k, kn.float(), pos)
    raises("positions must have shape", L.attn_kv_append, k, kn, pos[:1])
    raises("positions must be", L.attn_kv_append, k, kn, pos.long())
    raises("both or neither", L.attn_kv_append, k, kn, pos, k)
    raises("v_new must have shape", L.attn_kv_append, k, kn, pos, k, kn[:1].contiguous())
    raises("v_cache must", L.attn_kv_append, k, kn, pos, k.float(), kn)
    raises("ring_head must have shape", L.attn_kv_append_ring, k, kn, pos[:1])
    raises("on the GPU", L.attn_kv_append, k, kn, pos, k.clone(), kn.clone())
    lat = torch.zeros(2, 10, 576, dtype=bf)
    raises("k_new must have shape", L.attn_kv_append, lat, torch.zeros(2, 1, 576, dtype=bf), pos)
    raises("on the GPU", L.attn_kv_append, lat, torch.zeros(2, 576, dtype=bf), pos)
    kp = torch.zeros(6, 3, 16, 64, dtype=bf)
    table = torch.zeros(2, 4, dtype=i32)
    raises("k_new must have shape", L.attn_kv_append_paged, kp, kn[:, :1].contiguous(), pos, table)
    raises("block_table must", L.attn_kv_append_paged, kp, kn, pos, table[:1])
    raises("on the GPU", L.attn_kv_append_paged, kp, kn, pos, table)


def test_probe_checks():
    raises("dst is smaller", L.attn_probe_copy, torch.zeros(10, dtype=torch.uint8),
           torch.zeros(11, dtype=torch.uint8))
    raises("sink must be", L.attn_probe_read, torch.zeros(16), torch.zeros(1))
