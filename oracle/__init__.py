"""CPU oracle for the grouped block-scaled low-precision GEMM.

TEST INFRASTRUCTURE, NOT PART OF THE PRODUCT. Only ``tests/``,
``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` may
import, call or execute anything in this package. The library in
``mx_grouped_gemm_amd`` never routes through it, and this package never imports
that library: the two share no code, tables or helpers.

What it computes, and from which passages:

* ``formats``  - exact fp64 decoders for OCP e4m3fn, e2m1 (two per byte) and
  e8m0 codes, written from the bit-field definitions of the formats named on the
  Triton Gluon page "Overlapping Accumulator Block-Scaled Matrix
  Multiplication" (its ``random_quantized_tensor`` utility and the
  ``"e4m3"``/``"e2m1"`` operand formats of its ``async_mma_scaled_impl``).
* ``gemm.tile_map`` - the token-to-expert M-tile map (expert id of each
  128-row tile), from the ``expert_ids`` argument of the Modular MAX page
  "promote_accumulators" (grouped_matmul_sm100_blockwise_fp8), section Args.
* ``gemm.blockwise_grouped`` - the per-K-block partial product, scaled by
  ``a_scale * b_scale`` and promoted into a running accumulator, as the
  description paragraph of the same "promote_accumulators" page states, with
  ``b_scales`` shaped ``[num_experts, N // BN, K // BK]`` (section Args).
* ``gemm.blockwise_grouped_dequant`` - the same result by its plain definition:
  dequantise both operands, then one fp64 matmul per expert.
* ``gemm.mx_gemm`` - the MX (e8m0 per 32 K-elements) product, which the Gluon
  page's ``make_problem`` defines as ``A_ref @ B_ref.T`` on dequantised values.
* ``gemm.nv_gemm`` - the nvfp4 product of the same page (e2m1 elements, one
  ``float8_e4m3fn`` scale per 16 K-elements), again ``A_ref @ B_ref.T``.
* ``permute`` - the step before the GEMM: picks per expert, the row of each
  top-k pick in the padded expert-sorted A (the grouping ``expert_ids`` implies
  on the "promote_accumulators" page, section Args), and the 1 x 128 e4m3
  quantisation of token rows with an exact round-to-nearest-even encoder.

Every function works in fp64. Pins: ``tests/test_oracle_*.py`` (exact rational
brute force, power-of-two scale invariance, grouped == per-expert dense,
closed forms, library decoders). No function here is "parity unpinned".
"""

from . import formats, gemm  # noqa: F401
