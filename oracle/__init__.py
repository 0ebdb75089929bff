"""CPU oracle for the FP8 MoE quantization + grouped-GEMM path.

TEST INFRASTRUCTURE ONLY.  This package is a plain, slow, obviously correct
numpy implementation of what the GPU path computes.  Only ``tests/``,
``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` may
import it.  The product path (the HIP library and its Python binding) never
imports, calls or falls back to it, and it shares no code with that path:
no kernels, headers, helpers, tables or constant generators.

Precision: quantization decisions (scale division, scaling multiply, rounding
to FP8) are taken in IEEE fp32, the precision the kernels take them in, because
a floating-point result there decides an integer code.  GEMM references are
computed in fp64, where every FP8 x FP8 dot product is exact.

Sources (pages, cited by title and section throughout):
  [P1] AI Trends summary (aitrends.kr/articles/95981) of the PyTorch post
       "FP8 Training on AMD GPUs with TorchTitan and TorchAO".
  [P2] AI Trends summary (aitrends.kr/articles/16888) of the TorchAO MXFP8 MoE
       training post on Llama4 Scout.
  [P3] aihirek.info, "Az AMD GPU-kon is gyorsult az FP8-as PyTorch-tréning".
  [P4] aixai.ru blog, FP8 training on AMD with TorchTitan.

Readings the pages leave open are stated where they are used; the full list
with reasons is kept in the repository's design notes.

Parity status of each function: every function here is pinned by a CPU test
(``tests/test_oracle_*.py``) against something other than itself: an
independent library's FP8 dtypes, closed forms, hand-derived worked examples,
invariants and brute-force pure-Python loops.  None is "parity unpinned".
"""
from .codec import (E4M3FN, E4M3FNUZ, FMAX, decode_table, decode, encode,
                    encode_nearest, encode_arith, e8m0_decode, MX_FLOOR_OCP,
                    MX_CEIL, mx_shared_exponent)
from .quant import (EPS, bf16_to_f32, quantize_rowwise, quantize_colwise_grouped,
                    quantize_colwise_batched, quantize_mx_lastdim,
                    quantize_mx_rows_grouped, quantize_mx_rows_batched,
                    mx_rows_bound)
from . import blockwise, route, swiglu, tensorwise
from .gemm import (group_bounds, mm_grouped_m, mm_grouped_k, mm_grouped_m_mx,
                   mm_grouped_k_mx, mm_grouped_k_bf16, error_bounds_m,
                   error_bounds_k, ACC_FP32, ACC_FP8_MFMA)

__all__ = [n for n in dir() if not n.startswith("_")]
