"""CPU oracle for fine-grained FP8 quantization and block-scaled FP8 GEMM.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or
execute this package; only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code, table or
helper with the HIP library under ``fp8_fine_grained_amd/``.

What it computes, and where the method is described:

* ``oracle.e4m3``   -- the 8-bit E4M3 format (1 sign, 4 exponent, 3 mantissa
  bits): DeepGEMM launch article (itstec.com.br), section "O que e FP8?", the
  figure comparing E4M3 / E5M2 / FP16 / BF16.  The article's own bullet list
  there gives the E5M2 split as "the" FP8 format; the figure text and the
  DeepSeek-V3 FP8 knowledge-base page (codingmall.com), section "Unified E4M3",
  settle on E4M3 for every tensor.  Reading: OCP E4M3FN (bias 7, max 448, no
  infinities, NaN = S.1111.111), round to nearest even, saturating at 448.
* ``oracle.quant``  -- online fine-grained quantization: activations per 1x128
  tile (one token, 128 channels), weights per 128x128 block, each scale taken
  from the current tile's max-abs.  "The Insider Secrets Of Deepseek
  Discovered", passage on Figure 7(a); knowledge-base page, sections on
  fine-grained and online quantization.
* ``oracle.gemm``   -- the GEMM the block-scaled kernels approximate,
  C = A . B^T, computed exactly on dequantized values in float64, plus the
  error bound the GPU result is judged by.  Dense and the two MoE grouped
  layouts (contiguous, masked): DeepGEMM article, "Principais
  caracteristicas" (dense and two MoE layouts).
* ``oracle.accum``  -- accumulation emulators (limited-width accumulation
  versus FP32 promotion every 128-wide K-block) for the K=4096 demonstration:
  "The Insider Secrets Of Deepseek Discovered", passages on limited
  accumulation precision and on promotion to CUDA cores (Figure 7(b)).

Every function is written for clarity, not speed, in float64 except where the
method fixes a float32 step (the scale and the scaled value are float32
results of IEEE division).
"""

from . import e4m3, quant, gemm, accum  # noqa: F401

__all__ = ["e4m3", "quant", "gemm", "accum"]
