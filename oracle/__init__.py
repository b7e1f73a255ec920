"""CPU oracle for the flash-attention forward path (test infrastructure only).

This package is the plain, slow, fp64 statement of what the GPU path must
compute. It is test infrastructure: only ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py`` may import it. The product path
(``tiled_attention_amd``) never imports it and shares no code with it; the
only code both sides use is the seeded input generator module
(``tiled_attention_amd.workloads``), which holds none of the method's
arithmetic.

Modules and the passages they follow (pages cited by title and section):

* ``attention``  -- materialised S = Q K^T * scale, mask as -inf, two-pass
  softmax, times V. "Flash MSA Attention Kernel Implementation Tutorial",
  sections "Why We Needed a New Attention Kernel" and "Understanding Flash MSA
  Core Mechanics"; scale 1/sqrt(head_dim) from that page's kernel listing.
  Causal and sliding-window visibility from "Optimizing Triton kernels for
  custom attention patterns on H100", Pattern B.
* ``recurrence`` -- the online-softmax recurrence over K/V tiles (running max
  m, running sum l, rescale by exp(m - m_new)) and the merge of partial
  results. "Flash MSA ...", "Understanding Flash MSA Core Mechanics" and the
  kernel listing in "Implementation Step-by-Step with Triton".
* ``paged``      -- block-table page gather, single-query decode, causal
  prefill of the last rows of a paged sequence, and block-sparse paged
  cross-attention (each query block over its own page list).
  "Optimizing Triton kernels ...", Pattern C (gather_pages and its uses).
* ``fp8``        -- OCP E4M3FN encode/decode and per-128-row-block
  quantisation with scale = block absmax / 448. "FlashAttention-3: Warp
  Specialization ...", section "FP8 Block Quantization".

Every function is pinned by tests in ``tests/test_oracle.py`` to closed forms,
invariants, brute force or independent library routines; none is marked
"parity unpinned".
"""

from .attention import visible, attention, probabilities, visible_pair_count
from .recurrence import tiled_attention, partial_state, merge_partials, split_attention
from .paged import gather, decode, prefill, cross, listed_keys
from .fp8 import (E4M3_MAX, e4m3_value, e4m3_table, e4m3_encode, quantize_blocks,
                  dequantize_blocks, pow2_scale)

__all__ = [
    "visible", "attention", "probabilities", "visible_pair_count",
    "tiled_attention", "partial_state", "merge_partials", "split_attention",
    "gather", "decode", "prefill", "cross", "listed_keys",
    "E4M3_MAX", "e4m3_value", "e4m3_table", "e4m3_encode", "quantize_blocks",
    "dequantize_blocks", "pow2_scale",
]
