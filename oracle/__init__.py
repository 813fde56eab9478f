"""Plain CPU oracle for the QLoRA NF4 hot path.

TEST INFRASTRUCTURE ONLY. Nothing in the product path (the HIP library and
its Python binding) imports, links or calls anything in this package; only
the tests, the smoke check and the CPU-baseline leg of the benchmark do.

It is written from the method as the QLoRA pages describe it:

* ``nf4``    -- the NF4 codebook (page "QLoRA 论文解读" / diycv.top, section
  方法总览 item 2, equation for q_i), blockwise absmax quantisation with block
  64 (same page, item 1), double quantisation of the block constants to an
  8-bit float in blocks of 256 after mean subtraction (item 3, equations
  0.5 / 0.127 / 0.373; neura.market analysis, "How It Works"), and the
  double dequantisation doubleDequant(c1, c2, W) (section 关键公式).
* ``linear`` -- the LoRA linear layer Y = X W + s X L1 L2 (section 问题背景,
  LoRA equation) and its backward pass that gives dX and the adapter
  gradients but no weight gradient (section 关键公式, text after the dtype
  table).

Everything is slow, vectorised NumPy with explicit IEEE rounding steps
(float32 where the method rounds to fp32, float64 for reductions and for
the reference matmuls). It shares no code, tables or helpers with the GPU
path.
"""

from . import nf4, linear  # noqa: F401
