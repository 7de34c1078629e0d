"""Plain CPU reference for one decode step of attention over a head-shared or
latent KV cache.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
link this package: only the test suite, the smoke check in
``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` use
it.  It shares no code with the HIP library and never imports it.

Everything is float64 numpy, written as the plain definition of the method
(no tiling, no splitting, no online softmax) so that a reader can check it
against the pages by eye.  Short names used for the pages in the citations:

* ``attention-head``  - the xuesongtap.github.io note on attention heads
  (2025-11-14): attention equation and ``Bytes_KV`` (section 1), cache layout
  and grouping (section 2, 2.1, 2.2 and its size table), sliding window and
  ring buffer (section 3), MLA absorption and decoupled RoPE (sections
  5.1-5.4).
* ``toolsku``  - "AI演算法注意力機制演進：從MHA到MLA與Flash Attention全解析"
  (toolsku.com): the MHA formula block, the GQA module and its
  ``_repeat_kv`` expansion, the MLA absorption box.
* ``llmdeepdive``  - "MQA, GQA e MLA" (llmdeepdive.com lesson 7.6),
  section "Conceito": per-token cache accounting.
* ``baidu``  - "大模型注意力机制对比：MLA与MQA该怎么选" (cloud.baidu.com),
  section 二: cache shapes of MHA, MQA and MLA; section 四.3: KV-cache
  paging as the serving side of both.
* ``astro-blog``  - "MHA vs MQA vs GQA vs MLA：四种 Attention 机制显存与性能全对比":
  the ``calc_kv_cache_memory`` helper.
"""

from .attention import (  # noqa: F401
    kv_cache_bytes,
    mla_cache_bytes,
    mla_explicit_cache_bytes,
    visible_positions,
    ring_slot,
    gqa_decode_ref,
    mla_decode_ref,
    mla_explicit_ref,
    combine_ref,
    partial_ref,
    kv_append_ref,
    kv_append_ring_ref,
    gqa_decode_multi_ref,
    mla_decode_multi_ref,
    paged_positions,
    gqa_decode_paged_ref,
    mla_decode_paged_ref,
    kv_append_paged_ref,
)
