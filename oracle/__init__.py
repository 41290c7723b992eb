"""CPU oracle for paged-attention decode, the cache write and the block allocator.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
execute anything in this package: only ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code with the
HIP library (``paged_kv_cache_379_amd``) and imports nothing from it.

Page keys used in the citations of this package:

* [P1] "大模型KV Cache内存优化与PagedAttention显存管理机制详解" (yunthe.com):
  sections "PagedAttention分页内存管理原理" (paging principle),
  "PagedAttention注意力计算流程" (compute flow and its CUDA kernel sketch),
  "vLLM调度器与PagedAttention协同工作" (on-demand allocation, shared prefixes).
* [P2] "大模型部署中KV Cache优化策略与显存管理实践教程" (yunthe.com):
  section "量化压缩KV Cache的INT8与FP8方案" (INT8 KV cache).
* [P3] "vLLM推理框架源码初探：PagedAttention的显存管理设计" (trdm.cn):
  section 二 (core data structures: BlockTable, BlockManager, copy-on-write),
  section 三 (kernel points: gather through the table, block-major walk).

Every function is pinned by a ``-m "not gpu"`` test against something other
than itself (brute force, a library routine, closed forms, invariants, or the
pages' own printed tables); see the module docstrings for which pin covers what.
"""
from .paged_attention import (  # noqa: F401
    to_f64,
    paged_decode,
    reshape_and_cache,
    gather_context,
)
from .allocator_model import AllocatorModel, OutOfBlocks, DoubleFree  # noqa: F401
