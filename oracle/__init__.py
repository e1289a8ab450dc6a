"""CPU oracle for the GEMM hot path -- test infrastructure, not product code.

Only the test suite, the package smoke check and the benchmark's CPU-baseline
leg may import this package.  The GPU library never calls it and shares no
code with it: every function here is written from the definitions on the
source pages and from the number formats' own specifications, in float64.
The contraction is the plain triple loop in C (contract.c, built with gcc by
native.py); decoding, dequantisation, epilogue and log-softmax are numpy.

Sources (cited by short name throughout):
  * "GEMM compute-cost page" -- kwkr.cn/news/191298, the article on why GEMM
    dominates LLM compute (FLOP count in its section 3.1, fusion in 5.1,
    LM head in 7.2).
  * "DeepGEMM page" -- zwxr.cn/news/240083, the article on a DeepGEMM-style
    kernel library (naive golden reference in its section 3.2, FP8 group
    scales in 2.4, self-check list in 4.4).
  * "tensor-core page" -- llmtrend.com, 大语言模型（LLM）推理加速的秘诀：
    矩阵乘法、tensor-core (data flow host -> DRAM -> shared -> registers).

Modules:
  formats  -- bf16 and OCP e4m3fn decode / round-to-nearest-even encode.
  gemm     -- the fp64 GEMM (decode, contraction, epilogue), FP8 / int8 /
              int4 dequantisation, the log-softmax head and its error
              bound, error metric and FLOP count.
  native   -- builds and calls contract.c, the k-ascending triple loop.
  quant    -- per-group FP8 quantiser (amax / 448 scales).

Parity status: every function is pinned by a CPU test against something other
than itself (exhaustive library decode, exact rational arithmetic, closed
forms, the pages' printed FLOP figures).  The bits the GPU returns for large
inputs are not unique (any summation order inside the tolerance is correct);
beyond the tolerance they are parity unpinned because the pages print no GEMM
output values.
"""

from . import formats, gemm, quant  # noqa: F401
