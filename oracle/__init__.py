"""fp64 CPU oracle for exact (FlashAttention-style) attention — TEST INFRASTRUCTURE.

This package is the checker, not the product. Only the test suite, the smoke
check and the benchmark's CPU-baseline leg may import or call it; the HIP
library and its Python binding never do, and this package imports nothing
from them. It shares no code, tables or constants with the GPU path.

Contents
  softmax.py   safe (three-pass) softmax, the online-normaliser softmax
               recurrence, and log-sum-exp, in fp64.
  attention.py the definition of attention (scores, safe softmax, weighted sum
               of V) in fp64 per (batch, head), with causal masking, grouped
               query heads and the natural-log LSE; plus the two tiled
               online-softmax forms the pages describe (K/V-outer with the
               output renormalised each step, and Q-outer with the
               normalisation deferred), used only to check the definition.
  brute.py     the same definition in pure-Python loops (math.exp,
               math.fsum) for tiny shapes.
  backward.py  the gradients dQ, dK, dV of that definition (the chain rule
               written out in fp64, P recomputed from the saved LSE), summed
               over each K/V head's query-head group; the magnitude sums of
               their terms and the parity bar stated from them.
  attention.py and backward.py also hold the banded forms: a sliding window
               (left and right edges) with separate query and key lengths.
  precision.py the parity bars for fp32 and fp8 inputs (how far an evaluation
               in that precision may move each output, from the problem alone).
  dropout.py   dropout on the probabilities with a Philox4x32-10 keep mask,
               forward and backward with the mask fixed.
  additive.py  an additive (float) attention mask, forward and backward.
  pool.py      a process pool over (batch, head) units for big shapes.

Every function cites the passage of the pages it follows. Where the pages
are silent or garbled the reading taken is stated in the function's doc.
All functions are pinned by tests that do not re-type them (closed forms,
invariants, library routines, brute force); none is "parity unpinned".
"""
from .softmax import safe_softmax, online_softmax, logsumexp  # noqa: F401
from .attention import (attention_fp64, head_attention_fp64,  # noqa: F401
                        tiled_kv_outer_normalised, tiled_q_outer_deferred, kv_head_of,
                        band_visible, head_attention_band_fp64, attention_band_fp64)
from .brute import attention_brute  # noqa: F401
from .backward import (attention_bwd_fp64, head_attention_bwd_fp64,  # noqa: F401
                       attention_bwd_band_fp64, head_attention_bwd_band_fp64,
                       head_attention_bwd_magnitude_fp64, bwd_parity_bar)
from .additive import head_attention_additive_fp64, head_attention_bwd_additive_fp64  # noqa: F401
from .dropout import head_attention_dropout_fp64, head_attention_bwd_dropout_fp64, keep_mask  # noqa: F401
