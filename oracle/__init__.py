"""CPU oracle for paged attention over a block-table KV cache.

TEST INFRASTRUCTURE. Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package. The product path
(``paged_kv_cache_221_amd``) never imports it, and this package imports
nothing from the product path: the two share no kernels, headers, helpers,
tables or constants.

Pages cited throughout (short tags used in every docstring):

* [P1] "从 token 调度到采样输出，追踪每一步张量维度的变化，搞懂 LLM 推理到底在算什么"
  (zizhi168.cn/news/2384056) -- sections 02 Paged Attention, 03 Embedding,
  04 Attention (with its Prefill/Decode table), 07 extensions.
* [P2] "别只当API调用侠了！一文带你深入大模型“体内”，看懂推理全流程"
  (su666666.com/news/35626) -- the "PagedAttention 机制深度解析" part: paging,
  the block table, copy-on-write, the two-request figure, where the block table
  lives.
* [P3] the LLM inference-optimisation survey at adg.csdn.net
  (695256bb5b9f5f31781b99f3) -- sections 1.4 KV缓存, 1.5 大模型内存需求,
  3.1-3.3 MHA/MQA/GQA, 3.4 FlashAttention, 3.5 PageAttention.

Every function is pinned by at least one ``-m "not gpu"`` test to something
other than itself (closed forms printed on the pages, a library attention,
brute force, invariants, special cases); see ``tests/test_oracle_*.py``.
Parity unpinned: none.
"""

from .paged_attention import (  # noqa: F401
    STORAGE_DTYPES,
    widen,
    write_kv,
    gather_blocks,
    attend,
    paged_decode,
    paged_varlen,
    splitk_partials,
    lse_merge,
)
from .sizes import (  # noqa: F401
    kv_bytes_per_token,
    total_kv_bytes,
    paged_cache_bytes,
)
