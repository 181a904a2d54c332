"""CPU oracle for the FP8 flash-attention forward.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import, call or execute anything in this
package.  The HIP library never links it and the Python binding never imports
it; the two share no code.  The oracle is plain and slow on purpose:

* ``oracle.attention`` - float64 softmax(Q K^T * scale) V per segment and head,
  its LSE, and the FP8 recipe per row (E4M3 probabilities over dequantized
  E4M3 operands), used to show which rows no FP8 kernel can bring within the
  exact element-wise bar.
* ``oracle.quantize``  - per-head E4M3 quantization of Q/K/V (K centred by its
  segment's per-channel mean; optionally Q centred by its 128-row block mean,
  with the exact mean term in the Q operand).
* ``oracle.e4m3``      - bit-level OCP E4M3 encoder/decoder.
* ``oracle.compare``   - relative-RMS and max-abs comparators.
* ``oracle.mxfp4``     - the block-scaled FP4 variant: E2M1 codes with one
  power-of-two scale per 32 elements for Q (centred by its 128-row block
  mean, the mean term added back), K, V and the probabilities.

Every function is pinned by ``-m "not gpu"`` tests in ``tests/test_oracle_*.py``
against closed forms, brute force, a library routine or invariants.
"""
from . import attention, compare, e4m3, mxfp4, quantize  # noqa: F401
