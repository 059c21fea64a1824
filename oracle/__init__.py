"""CPU oracle for the quantized linear layer (W4A16 and W8A8_INT8).

TEST INFRASTRUCTURE ONLY. Nothing on the product path may import, call or run
this package: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it. It shares no code with the HIP
library under ``weight_activation_quantized_amd/`` and neither side imports
the other.

Every function is the plain definition of what the layer computes, written in
NumPy with float64 accumulation, so that a reader can check it against the
pages by eye:

* ``unpack_int4`` / ``dequant_w4`` / ``w4a16_ref`` -- the AWQ-style W4A16 path
  (LMDeploy overview, section 2.5 "Weight quantization (AWQ)": 4-bit weights,
  groups of 128; LMDeploy 4-bit deployment guide, section 2.2: scales are
  applied inside the same kernel as the weights).
* ``pack_int4`` / ``reorder_int4_ref`` / ``transpose_int4_ref`` -- bringing
  4-bit checkpoints packed in another field order or along the other axis
  into the library's layout (LMDeploy overview, sections 4.1 and 5.5: AWQ
  model format; pymllm Setup and Usage: compressed-tensors loading).
* ``quant_per_token_int8_ref`` / ``w8a8_acc_ref`` / ``w8a8_ref`` -- the
  W8A8_INT8 path (pymllm Setup and Usage, Overview: int8 weights and
  activations on INT8 tensor cores; section "W8A8 first-run JIT
  compilation": a per-token int8 activation quantizer and an int8 scaled
  matmul).

The pages fix names and schemes but print no formula, bit layout or worked
example. Where they are silent the readings are stated in each docstring
(nibble order, zero-point storage, divide-by-scale, ties-to-even, clamp to
[-127, 127], all-zero rows).

Pins: every function is checked in ``tests/test_oracle.py`` against values
that do not come from this package (independent loop packers, exact rational
arithmetic, closed forms, special cases that reduce to a textbook matmul).
"""

from .ref import (  # noqa: F401
    NIBBLES_PER_WORD,
    block_weights_ref,
    dequant_w4,
    kv_dequant_ref,
    kv_quant_ref,
    pack_int4,
    quant_per_token_int8_ref,
    reorder_int4_ref,
    transpose_int4_ref,
    unpack_int4,
    w4a16_ref,
    w8a8_acc_ref,
    w8a8_ref,
)
