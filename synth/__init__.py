"""Seeded synthetic inputs shared by the tests, the smoke check and the bench.

This module only draws numbers: shapes, seeds and value distributions of the
workloads.  It holds none of the attention arithmetic and imports neither the
reference in ``oracle/`` nor the HIP library, so both sides can take their
inputs from it.

Recipe (the pages use no dataset; every input is synthetic):

* Base seed ``1234 + 100 * index`` per workload family; sub-seeds q = +0,
  K = +1, V = +2, lengths = +3, ring heads = +4, latent = +1.
* Tensors are drawn per batch entry from a generator seeded with
  ``sub_seed * 1_000_003 + b`` so one sequence can be regenerated alone.
* Floats are float32 N(0, 1) (times ``value_scale``) and, for bf16 workloads,
  rounded to bfloat16 by ``Tensor.to`` (round to nearest even).
* Ragged lengths are uniform integers in ``[lo, hi]`` inclusive; ring heads are
  uniform in ``[0, slots)``.
"""

import math

import torch

__all__ = ["WORKLOADS", "workload", "gqa_inputs", "mla_inputs", "draw",
           "draw_ints"]

_SEQ_MULT = 1_000_003

# name -> shape description.  "index" picks the base seed.
WORKLOADS = {
    # GQA, float32, tiny: B=1, 8 query heads over 2 KV heads, d=64, T=512.
    "gqa_fp32_t512": dict(kind="gqa", index=0, B=1, H_q=8, H_kv=2, d=64,
                          T_cap=512, dtype="fp32"),
    # Llama-3-8B-shaped GQA layer: 32 query heads over 8 KV heads, d=128.
    "llama3_8b_gqa_t4096": dict(kind="gqa", index=1, B=32, H_q=32, H_kv=8,
                                d=128, T_cap=4096, dtype="bf16",
                                scale=1.0 / math.sqrt(128)),
    # Long context, MHA (32 KV heads) and MQA (1 KV head), B = 1 and 64.
    "mha_t32k_b1": dict(kind="gqa", index=2, B=1, H_q=32, H_kv=32, d=128,
                        T_cap=32768, dtype="bf16"),
    "mha_t32k_b64": dict(kind="gqa", index=2, B=64, H_q=32, H_kv=32, d=128,
                         T_cap=32768, dtype="bf16"),
    "mqa_t32k_b1": dict(kind="gqa", index=2, B=1, H_q=32, H_kv=1, d=128,
                        T_cap=32768, dtype="bf16"),
    "mqa_t32k_b64": dict(kind="gqa", index=2, B=64, H_q=32, H_kv=1, d=128,
                         T_cap=32768, dtype="bf16"),
    # Ragged lengths drawn from [1024, 32768] in a 32768-slot cache.
    "mha_t32k_b64_ragged": dict(kind="gqa", index=2, B=64, H_q=32, H_kv=32,
                                d=128, T_cap=32768, dtype="bf16",
                                ragged=(1024, 32768)),
    "mqa_t32k_b64_ragged": dict(kind="gqa", index=2, B=64, H_q=32, H_kv=1,
                                d=128, T_cap=32768, dtype="bf16",
                                ragged=(1024, 32768)),
    # Sliding window w=4096 kept in a 4096-slot ring; logical length 32768.
    "swa_ring_w4096_t32k": dict(kind="gqa", index=3, B=16, H_q=32, H_kv=8,
                                d=128, T_cap=4096, dtype="bf16", window=4096,
                                ring=True, logical_len=32768),
    # The same window over a linear 32768-row cache: only the last 4096 rows
    # of each sequence are visible, so a kernel that skips masked rows reads
    # an eighth of the cache.
    "swa_linear_w4096_t32k": dict(kind="gqa", index=3, B=16, H_q=32, H_kv=8,
                                  d=128, T_cap=32768, dtype="bf16",
                                  window=4096),
    # Wide head (d=256), 24 query heads over 4 KV heads, T=131072.
    "wide_d256_t128k": dict(kind="gqa", index=3, B=4, H_q=24, H_kv=4, d=256,
                            T_cap=131072, dtype="bf16"),
    # Absorbed MLA: latent [64, 8192, 512+64], 128 heads, scale 1/sqrt(128+64).
    "mla_b64_t8192": dict(kind="mla", index=4, B=64, H=128, T_cap=8192,
                          d_c=512, d_rope=64, dtype="bf16",
                          scale=1.0 / math.sqrt(192),
                          value_scale=1.0 / math.sqrt(576)),
    # the same with lengths uniform on 1024..8192 (the ragged variant)
    "mla_b64_t8192_ragged": dict(kind="mla", index=4, B=64, H=128, T_cap=8192,
                                 d_c=512, d_rope=64, dtype="bf16",
                                 scale=1.0 / math.sqrt(192),
                                 value_scale=1.0 / math.sqrt(576),
                                 ragged=(1024, 8192)),
    # second latent geometry: 32 query heads, latent 256 + RoPE 64
    "mla256_b64_t8192": dict(kind="mla", index=5, B=64, H=32, T_cap=8192,
                             d_c=256, d_rope=64, dtype="bf16",
                             scale=1.0 / math.sqrt(192),
                             value_scale=1.0 / math.sqrt(320)),
}


def workload(name, **overrides):
    """A copy of a named workload description with fields overridden."""
    w = dict(WORKLOADS[name])
    w.update(overrides)
    w["name"] = name
    return w


def _torch_dtype(dtype):
    return {"fp32": torch.float32, "bf16": torch.bfloat16}[dtype]


def draw(shape, seed, dtype="bf16", device="cpu", value_scale=1.0):
    """[B, ...] float32 N(0,1)*value_scale drawn per leading index b with the
    generator seeded ``seed * 1_000_003 + b``, then cast to ``dtype``."""
    B = shape[0]
    out = torch.empty(shape, dtype=_torch_dtype(dtype), device=device)
    gen = torch.Generator(device=device)
    for b in range(B):
        gen.manual_seed(seed * _SEQ_MULT + b)
        x = torch.randn(shape[1:], generator=gen, device=device,
                        dtype=torch.float32)
        if value_scale != 1.0:
            x.mul_(value_scale)
        out[b].copy_(x.to(out.dtype))
        del x
    return out


def draw_ints(n, lo, hi, seed, device="cpu"):
    """``n`` int32 uniform on ``[lo, hi]`` inclusive, from a CPU generator."""
    gen = torch.Generator(device="cpu")
    gen.manual_seed(seed)
    x = torch.randint(lo, hi + 1, (n,), generator=gen, dtype=torch.int64)
    return x.to(torch.int32).to(device)


def gqa_inputs(w, device="cpu", seed=None):
    """Tensors for a "gqa" workload description: dict with q, k, v, seq_lens
    (or None), ring_head (or None), window, scale (or None)."""
    base = 1234 + 100 * w["index"] if seed is None else seed
    B, H_q, H_kv, d, T = w["B"], w["H_q"], w["H_kv"], w["d"], w["T_cap"]
    dt = w.get("dtype", "bf16")
    vs = w.get("value_scale", 1.0)
    q = draw((B, H_q, d), base + 0, dt, device, vs)
    k = draw((B, H_kv, T, d), base + 1, dt, device, vs)
    v = draw((B, H_kv, T, d), base + 2, dt, device, vs)
    seq_lens = None
    if w.get("ragged"):
        lo, hi = w["ragged"]
        seq_lens = draw_ints(B, lo, hi, base + 3, device)
    elif w.get("logical_len"):
        seq_lens = torch.full((B,), w["logical_len"], dtype=torch.int32,
                              device=device)
    ring_head = None
    if w.get("ring"):
        ring_head = draw_ints(B, 0, T - 1, base + 4, device)
    return dict(q=q, k=k, v=v, seq_lens=seq_lens, ring_head=ring_head,
                window=w.get("window", 0), scale=w.get("scale"))


def mla_inputs(w, device="cpu", seed=None):
    """Tensors for an "mla" workload: dict with q [B,H,d_c+d_rope],
    latent [B,T,d_c+d_rope], seq_lens (or None), d_c, scale."""
    base = 1234 + 100 * w["index"] if seed is None else seed
    B, H, T = w["B"], w["H"], w["T_cap"]
    dk = w["d_c"] + w["d_rope"]
    dt = w.get("dtype", "bf16")
    vs = w.get("value_scale", 1.0)
    q = draw((B, H, dk), base + 0, dt, device, vs)
    latent = draw((B, T, dk), base + 1, dt, device, vs)
    seq_lens = None
    if w.get("ragged"):
        lo, hi = w["ragged"]
        seq_lens = draw_ints(B, lo, hi, base + 3, device)
    return dict(q=q, latent=latent, seq_lens=seq_lens, d_c=w["d_c"],
                scale=w["scale"])
