"""CPU oracle for paged attention — TEST INFRASTRUCTURE ONLY.

Only the tests, `__graft_entry__.smoke()` and the benchmark's CPU-baseline leg may
import this package.  The product path (the HIP library and its binding) never
imports, links or calls it, and this package never imports the product path.

The oracle is the plain definition of what the paged-KV method computes,
written in NumPy float64 with no blocking, fusion or reordering beyond what
the definition states:

  * ``attention``  - gather a sequence's K/V through its block table into
    contiguous arrays, then textbook softmax attention (decode, chunked
    prefill, grouped heads, int8 storage with per-block scales);
  * ``allocator`` - the block manager: LIFO free list, reference counts,
    sequences, fork and copy-on-write on append;
  * ``cache_ops`` - writing new K/V rows into slots, and whole-block copies;
  * ``quantize``  - int8 storage of whole blocks with per-(block, KV head)
    scales.

Pages cited (each by its address; titles as published):
  [kongchang]  kongchang.com, "vLLM架构深度解析：PagedAttention如何实现高吞吐LLM推理"
  [cnnetsun]   cnnetsun.cn/a/1845762, "别再让GPU内存拖后腿了：vLLM的PagedAttention如何像操作系统一样管理KV Cache"
  [aisoosoo]   aisoosoo.com, "vLLM：大模型推理的加速引擎，PagedAttention 颠覆显存管理"
  [nxbn]       m.nxbn.cn/news/200425 (untitled VLLM walkthrough; numbered sections 一..六)

Every function is pinned by a CPU test against something other than itself
(library routines, closed forms, invariants, brute force, the pages' printed
allocator behaviour); no function here is "parity unpinned".
"""
from . import allocator, attention, cache_ops, quantize  # noqa: F401
