"""CPU oracle for the block-scaled matmul -- TEST INFRASTRUCTURE ONLY.

A plain, slow, obviously correct numpy implementation of what the GPU path
computes.  Only the test suite, the package smoke check and the benchmark's
CPU-baseline leg may import it; the library and its Python binding never do,
and the oracle imports nothing from them (the two share no code, headers,
tables or helpers; the only shared module is ``synth``, which draws inputs and
holds none of the matmul's arithmetic).

Contents
--------
``formats``    OCP E4M3FN and E8M0 decode, IEEE round-to-nearest-even to fp32
               and bf16 (closed forms).
``scaled_mm``  the three scaled matmuls, an elementwise error bound and the
               comparison rule.

Sources (the pages this oracle is written from):

* PyTorch issue "torch._scaled_mm with blockwise scaling doesn't work with
  torch.compile": the scale-shape rules for tensorwise, rowwise and blockwise
  scaling, and the blockwise example shapes (16640, 64) / (64, 40).
* torchao PR "Remove int_scaled_mm's dependency on triton for cpu": the int8
  scaled matmul is an int32 matmul, a cast to the scale dtype, then a multiply.
* torchao issue "Unify scaled INT8 matmul": the scale step is
  ``acc_i32.to(f32) * scale.to(f32)``, with both activation and weight scales.
* Inductor ``torch/_inductor/kernel/mm.py``: ``apply_scaling`` (rowwise scales
  multiply the accumulator), ``check_supported_striding`` (A row-major, B
  column-major), ``decomposeK`` (split-K sums fp32 partials, then casts).
* ROCm aiter PR "Add opus fp8 mxscale BMM kernels for gfx950": the m-major
  layout x [M,G,K], w [G,N,K], x_scale [M,G,K/128], w_scale [G,N/128,K/128],
  e8m0 block scales, both m-major and batch-first layouts.

Every function is pinned by the CPU tests (``tests/test_oracle_*.py``) against
closed forms, brute force on tiny inputs, library routines and invariants.
The final floating-point output values have no printed example to pin to; the
pages print none (see the parity notes in the tests).
"""

from . import formats, scaled_mm  # noqa: F401
from .formats import (  # noqa: F401
    e4m3_value, e4m3_numerator, e8m0_value, round_f32, bf16_bits_from_f32,
    bf16_bits_from_f64, bf16_bits_to_f64,
)
from .scaled_mm import (  # noqa: F401
    int8_rowwise, fp8_blockwise, fp8_mx_bmm, compare, Result,
)
