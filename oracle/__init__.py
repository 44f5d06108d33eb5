"""Plain, slow, fp64 CPU oracle for the paged-KV-cache attention path.

TEST INFRASTRUCTURE ONLY. Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or call anything here. The HIP
library and its Python binding never import this package, and this package
imports nothing from them: the two share no code, tables or helpers.

Every function computes the plain definition of what the path computes, with
no blocking, fusion or reordering:

* the KV store copies each new token's K and V rows to the cache slot that the
  slot mapping names (page "nano-vLLM 最小化vLLM重新实现", section 5 "注意力机制",
  which describes the store kernel writing K/V into the paged cache through
  ``slot_mapping``);
* attention is ``softmax(q kᵀ / sqrt(head_dim)) v`` (page at
  bxzpzcl.cn/news/2159246, section 2.2.2 "两级注意力加速", the manual-attention
  fallback), with K and V gathered row by row through each sequence's block
  list (page "nano-vLLM 最小化vLLM重新实现", section 3 "块管理器" and section 4
  "模型运行器" for the ``[num_blocks, block_size, num_kv_heads, head_dim]``
  cache), in fp64.

* the step before the store (``qk_norm_rope``): RMSNorm of every query and
  key head, then the rotary embedding from a given cos/sin table (page
  "nano-vLLM 最小化vLLM重新实现", section 6 "模型" and "辅助层"); V passes
  through unchanged.

* the host block manager (``block_manager.BlockManager``): a pool of
  fixed-size blocks from a free list with reference counts, chained xxh64
  hashes of full token blocks for prefix reuse, and release on finish or
  preemption (page "nano-vLLM 最小化vLLM重新实现", section 3 "块管理器").

* the Gumbel-max sampler (``sampler.sample``): argmax of softmax(l / T) over
  exponential noise drawn with Philox4x32-10 (page "nano-vLLM
  最小化vLLM重新实现", "辅助层" and "关键设计选择").

Every function here is pinned by ``tests/test_oracle.py``,
``tests/test_oracle_rope.py``, ``tests/test_oracle_blocks.py`` and
``tests/test_oracle_sampler.py`` against closed forms,
invariants, a hand-worked golden example, a pure-Python brute force and
``torch.nn.functional.scaled_dot_product_attention``; none is "parity
unpinned".
"""

from .paged_attention import (  # noqa: F401
    bf16_to_f64,
    slot_of,
    store_kvcache,
    gather_rows,
    attention_rows,
    decode,
    prefill_varlen,
)
from .norm_rope import qk_norm_rope, rms_norm, rotate_half_pairs  # noqa: F401
