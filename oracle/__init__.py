"""Plain, slow CPU oracle for paged KV-cache attention (fp64) — TEST INFRASTRUCTURE.

This package is the checker, not the product.  Only the test suite, the smoke
check in ``__graft_entry__`` and the CPU-baseline leg of ``bench.py`` may import
it.  It shares no code, tables or constants with the HIP library: it reads the
same input bytes, decodes them exactly to float64 and evaluates the textbook
definitions the pages give.

Pages cited throughout (by title):

* "五十三：vLLM-PagedAttention" (book.bogosort.top LLM tutorial, lesson 53)
* "17. vLLM PagedAttention | 经典推理框架: 模拟 Continuous Batching 与
  PagedAttention" (datawhalechina llm-algo-leetcode)
* "vLLM 与 LLM 推理部署实战：从 PagedAttention 到生产级服务架构" (ybb.press)
* "vLLM与PagedAttention：大模型推理内存优化技术解析" (intelliparadigm.com)
* "推理引擎内部机制——PagedAttention、连续批处理、分块预填充"
  (ai-engineering.com.cn, Phase 17 · 04)

Every function here is pinned by a ``-m "not gpu"`` test against values the
pages print, closed forms, invariants or a library routine.  The only
conventions the pages leave open and that no pin can fix are the e4m3
saturation rule (``elements.e4m3_encode``) — "parity unpinned" for values
above 448 in magnitude — and the choice of split partition on the GPU side,
which the oracle does not model at all (it never splits).
"""

from .elements import (
    STORAGE_DTYPES,
    decode_elements,
    e4m3_value_table,
    e4m3_encode,
    int8_encode,
)
from .paged import (
    num_blocks,
    locate_token,
    gather_sequence,
    softmax_attention,
    decode_attention,
    prefill_chunk_attention,
    reshape_and_cache,
    copy_blocks,
    copy_block_rows,
    copy_blocks_layers,
    swap_blocks,
)

__all__ = [
    "STORAGE_DTYPES",
    "decode_elements",
    "e4m3_value_table",
    "e4m3_encode",
    "int8_encode",
    "num_blocks",
    "locate_token",
    "gather_sequence",
    "softmax_attention",
    "decode_attention",
    "prefill_chunk_attention",
    "reshape_and_cache",
    "copy_blocks",
    "copy_block_rows",
    "copy_blocks_layers",
    "swap_blocks",
]
