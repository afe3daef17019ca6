"""CPU oracle for block-scaled FP8 / MXFP4 FlashAttention forward with optional
3D sliding-tile sparsity.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path (the HIP kernels, the
C-ABI library or its Python binding) imports, links or calls anything here.
Only the test suite, the smoke check and the CPU-baseline leg of the benchmark
use it.  It shares no code, tables or constants with the GPU path: every
format, quantizer and softmax step is written out again here, slowly and in
float64 where the method leaves the precision open, so that a reader can check
it against the pages by eye.

Modules
-------
formats    OCP FP8 E4M3 ("fn"), FP4 E2M1 and E8M0 encode/decode from the bit
           definitions.
quant      Q/K per-block FP8, V per-channel FP8, Q/K MXFP4 (E2M1 + E8M0 per 32).
attention  the staged-precision online-softmax recipe (KV tiles in ascending
           order, P requantised to FP8 with the fixed 1/448 tensor scale) and a
           float64 brute-force softmax(QK^T * scale) V.
sta        3D tile partition, token order and clipped window lists, by brute
           force.

Sources (web pages; cited by title and section):
  [FPS]  "FP8量化与稀疏性协同加速视频扩散模型" (FPSAttention) - §2.1, §2.2, §3.1, §3.3
  [FP4G] "Blackwell架构实战：如何用FP4量化让你的AI模型推理速度翻倍（附代码）" - §1
  [FA4]  "FA4极速LLM：10分钟搞定20倍内存直降！" - FlashAttention section, FA4 co-design list
  [FV]   FastVideo FP4 attention kernel article (wmrh.cn) - §2.1, §5.2

Parity status: every function here is pinned by a CPU test against closed
forms, code tables, invariants or brute force, except the end-to-end error of
the quantised recipe against the unquantised result, which the pages give no
number for ("parity unpinned"; the error is reported, not gated).
"""
