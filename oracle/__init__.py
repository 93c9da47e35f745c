"""CPU oracle for block-causal GQA attention with QK-Norm and 3D RoPE.

TEST INFRASTRUCTURE ONLY.  This package is a plain, slow, float64 NumPy
restatement of what the attention path computes, written from the MAGI-1 pages
and kept independent of the HIP implementation: it shares no code, table or
helper with ``block_causal_attention_amd`` and never imports it.  Only the test
suite, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import it; the product path never calls it.

Functions (each cites the passage it follows in its docstring):

  qk_norm          RMS normalisation of each (token, head) vector, times a gain
  rope_inv_freq    per-pair rotation frequencies of the 3D RoPE
  rope_3d          rotary embedding over (t, h, w) coordinates
  video_mask       dense block-causal / KV-range / packed-video mask rows
  slices_mask      dense mask rows denoted by a list of AttnSlices
  window_mask      dense packed causal sliding-window mask rows
  attention        masked softmax attention with grouped K/V heads
  attention_backward  its gradients with respect to q, k and v
  forward          qk_norm -> rope_3d -> attention, end to end

Every function is pinned by ``tests/test_oracle_pins.py`` against library
routines, closed forms, brute force and invariants.  The one part no test can
pin is agreement with the released MAGI-1 model's own conventions (norm type,
RoPE axis split and pairing, causal alignment of non-square slices): the pages
do not state them, so those readings are "parity unpinned" with respect to the
model, while the oracle-vs-kernel parity is fully pinned.
"""
from .reference import (  # noqa: F401
    qk_norm, rope_inv_freq, rope_3d, video_mask, slices_mask, window_mask, attention, attention_backward,
    forward, MASK_FULL, MASK_CAUSAL, MASK_INVCAUSAL, MASK_BICAUSAL,
)
