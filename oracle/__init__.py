"""CPU oracle for attention over a block-paged KV cache.

TEST INFRASTRUCTURE ONLY. This package is the slow, plain reference that the
HIP library is checked against. Only the test suite, the smoke check and the
CPU-baseline leg of the benchmark may import it; the library itself never does,
and the two share no code.

Sources (web pages, cited by title and section):
  [nano-vllm]  "nano vllm：轻量级大模型推理框架的KV Cache优化实践"
               (intelliparadigm.com)
  [mini-vllm]  "mini-vllm：基于 NanoGPT 的 PagedAttention 风格 KV 缓存管理实现"
               (zingnex.cn)

Modules:
  attention     store / gather / decode / split-decode / chunked prefill, fp64
  prefix_cache  rolling prefix hash and the hash-sharing block allocator
"""

from . import attention, prefix_cache  # noqa: F401
