"""CPU oracle for the TurboQuant KV-cache hot path -- TEST INFRASTRUCTURE ONLY.

This package is the plain, slow, float64 statement of what the GPU library must
compute.  Only the test suite, the smoke check and the benchmark's CPU-baseline
leg may import it; the product path (the HIP library and its Python binding)
never does, and this package imports nothing from the product.

Sources, cited by page title and section (the pages carry no formulas for most
steps; where they are silent the reading taken is named in the function):

  [TQ+ guide]   "TurboQuant+ 上游化实战指南：llama.cpp KV Cache 压缩分支的 4 阶段
                 PR 重构路线图" (bjdmk.com.cn developer community)
  [Orión plan]  "Plan de Integración: TurboQuant en Orión" (stig.sh)
  [TQ explainer] "Google TurboQuant 深度解析：KV Cache 压缩的技术革命" (lonae.com)

Layout of the package:
  tables.py  seeded rotation signs, Hadamard matrix, Gaussian JL matrix,
             Lloyd-Max Gaussian codebook and its thresholds
  encode.py  rotation -> norm -> scalar codebook -> bit packing -> QJL sketch
  decode.py  dequantisation, attention logits, softmax.V, top-k

Every function is pinned by tests under tests/ (test_oracle_*.py) against
closed forms, published quantiser tables, brute force and invariants.  One
item is "parity unpinned" by the pages: the exact byte layout of packed codes
(the pages fix only the sign-bit order); it is pinned by round trips and by
agreement with the GPU path only.
"""

from . import tables, encode, decode  # noqa: F401
