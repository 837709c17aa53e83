"""CPU fp64 oracle for exact softmax attention.

TEST INFRASTRUCTURE. This package is the slow, obviously correct reference that
the HIP path is checked against. Only ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py`` may import or call it; the product
path (``io_aware_exact_attention_amd``) never does, and the oracle imports
nothing from the product path. Inputs reach it as plain tensors; it upcasts them
to float64 and evaluates the definition of attention directly.

Parity status of each function (what pins it, see ``tests/test_oracle_pins.py``):

* ``attention_probs`` / ``attention_forward``: pinned (row sums, uniform keys,
  one-hot query, shift and permutation invariance, causal row 0, torch-CPU
  fp64 ``scaled_dot_product_attention`` and ``torch.logsumexp``).
* ``attention_backward``: pinned (central finite differences, gradient
  invariants, torch fp64 autograd through ``scaled_dot_product_attention``).
* ``online_softmax_forward``: pinned (equals the one-shot definition for
  arbitrary key-block splits, and the pins above through that equality).
* ``attention_forward_varlen`` / ``attention_backward_varlen``: pinned
  (per-sequence agreement with torch fp64 SDPA on each sequence).
* ``decode_forward`` (grouped-query decoding): pinned (equals the dense
  functions above on key/value heads expanded per group, torch fp64 SDPA with
  an explicit bottom-right mask, one query token = no mask).
* ``decode_split_partials`` / ``merge_splits``: pinned (any key split merged
  equals the one-shot result; the merge is associative).
* ``oracle.fp8`` (FP8 forward with the Hadamard rotation: e4m3 codec,
  rotation, per-block quantisation, attention with P rounded per key block):
  pinned (format values, nearest-code search, scipy's Hadamard, score
  invariance, exact power-of-two cases against the dense oracle, a worked
  running-max example, the rounding bound, the rotation's benefit), see
  ``tests/pins_fp8.py``.
* ``oracle.schedule`` (greedy list scheduling and LPT): pinned to the page's
  worked example (``tests/golden/lpt_example.json``), brute-force optima and
  Graham's bounds, see ``tests/test_schedule.py``.
"""

from .attention import (  # noqa: F401
    attention_probs,
    attention_forward,
    attention_backward,
    online_softmax_forward,
    attention_forward_varlen,
    attention_backward_varlen,
)
from .decode import (  # noqa: F401
    decode_forward,
    decode_split_partials,
    merge_splits,
)
