"""CPU oracle for the 6Bit-Diffusion per-linear hot path.

TEST INFRASTRUCTURE ONLY.  Nothing in the product library imports, calls or
links anything here; only the tests, the smoke check and the CPU-baseline leg
of the benchmark do.  The oracle shares no code, table or constant generator
with the GPU path.

It is a plain, slow, obviously-correct restatement of what the path computes:
numpy float32 where the method pins fp32 rounding, float64 / exact int64
elsewhere.  Pages cited (by title and section):

  [gist]  gist.science, "6Bit-Diffusion: Inference-Time Mixed-Precision
          Quantization for Video Diffusion Models" (technical summary of
          arXiv 2603.18742), sections 2.A DMPQ, 2.B TDC, 2.C PDR, 4.
  [yly]   youleyou.com, "清华大学6Bit-Diffusion技术实现视频生成AI模型3倍压缩与速度翻倍",
          sections 一 (DMPQ), 二 (TDC), 三 (PDR), 四, 七.

Number formats the pages name but do not define (NVFP4, E4M3, E2M1, INT8)
follow their public definitions: OCP 8-bit Floating Point Specification
(E4M3 "fn" variant), OCP Microscaling Formats v1.0 (FP4 E2M1 element), and
NVIDIA's NVFP4 layout (E2M1 elements, one E4M3 scale per 16 elements, one
fp32 per-tensor scale).

Every reading the pages leave open is stated at the function that adopts it.

Parity pinning: every function here is pinned by tests/test_oracle_*.py to
facts outside this package (closed forms, brute force, library casts,
hand-derived fixtures in tests/golden/).
"""
from . import formats, hadamard, quant, gemm, stats, dmpq  # noqa: F401
