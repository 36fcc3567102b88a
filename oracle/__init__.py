"""CPU oracle for fused attention forward.

TEST INFRASTRUCTURE ONLY.  Imported by ``tests/``, ``__graft_entry__.smoke()``
and the CPU-baseline leg of ``bench.py``; never by the product package.  It
shares no code with the HIP path.

* ``attention_ref`` -- float64 two-pass softmax attention (the definition).
* ``online_attention_ref`` -- float64 online-softmax recurrence over any key
  tiling, used to pin the recurrence against the definition.
* ``e4m3_decode`` / ``e4m3_encode`` / ``quantize_per_head`` -- OCP E4M3 codes
  and the per-head FP8 quantiser of the FP8-score forward.
* ``philox4x32`` / ``dropout_keep`` / ``attention_dropout_ref`` /
  ``attention_dropout_bwd_ref`` / ``attention_dropout_bwd_ref_rows`` -- the
  reproducible dropout mask and attention
  forward and backward with it.
* ``attention_bwd_ref`` / ``attention_bwd_ref_batched`` /
  ``attention_bwd_dq_rows_ref`` / ``attention_bwd_kv_rows_ref`` -- float64 gradients
  dQ, dK, dV by their definition; ``attention_bwd_tiled_ref`` -- the
  recomputing tiled backward, pinned against the definition.

Pins (all in ``tests/test_oracle.py``): the worked two-tile example of the
page "22. GPU Engineering: Correctness, Throughput, and Attention" (sec. 22.7),
closed forms (one key, zero scale, causal first row), invariants (rows of P sum
to one, constant V, score shift, key/query permutation), an independent
library routine (torch's float64 scaled-dot-product attention), a 50-digit
brute force on tiny inputs, and the recurrence under every tiling.
Backward pins (``tests/test_oracle_bwd.py``): central finite differences of
the forward definition, torch float64 autograd, closed forms (one key, zero
scale), invariants (key shift, value shift, query/key scale symmetry), and the
tiled method under many tilings.
"""
from .attention_ref import attention_ref, attention_ref_batched, bf16_bits_to_f64, f32_scale
from .attention_bwd_ref import (attention_bwd_dq_rows_ref, attention_bwd_kv_rows_ref,
                                attention_bwd_ref, attention_bwd_ref_batched,
                                attention_bwd_tiled_ref)
from .dropout_ref import (attention_dropout_bwd_ref, attention_dropout_bwd_ref_rows,
                          attention_dropout_ref, dropout_keep,
                          philox4x32)
from .fp8_ref import E4M3_MAX, e4m3_decode, e4m3_encode, quantize_per_head
from .online_ref import all_compositions, online_attention_ref, uniform_bounds

__all__ = ["attention_ref", "attention_ref_batched", "bf16_bits_to_f64", "f32_scale",
           "online_attention_ref", "all_compositions", "uniform_bounds",
           "attention_bwd_ref", "attention_bwd_ref_batched", "attention_bwd_tiled_ref",
           "attention_bwd_dq_rows_ref", "attention_bwd_kv_rows_ref",
           "E4M3_MAX", "e4m3_decode", "e4m3_encode", "quantize_per_head",
           "philox4x32", "dropout_keep", "attention_dropout_ref", "attention_dropout_bwd_ref",
           "attention_dropout_bwd_ref_rows"]
