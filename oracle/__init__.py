"""fp64 CPU oracle for fused causal scaled-dot-product attention.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path imports or calls this
package: only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline``
leg of ``bench.py`` use it.  It shares no code, header, table or helper with the
HIP kernels in ``causal_attention_fa_amd``; the only thing both sides share is
the seeded input generator in ``workloads`` (which holds no attention
arithmetic).

Two independently written forms:

* ``dense``  -- the plain definition, softmax(mask(scale * Q K^T)) V, and the
  textbook softmax-Jacobian backward.
* ``tiled``  -- the method itself: online softmax over KV tiles (Q-tile outer
  loop), logsumexp output, and the flash backward that recomputes P from L
  and uses D = rowsum(dO * O).

Every function is pinned by tests in ``tests/test_oracle.py`` against closed
forms, a hand-derived worked example (``tests/golden``), invariants, finite
differences and PyTorch's own fp64 CPU attention.  No function here is
"parity unpinned".
"""
from .dense import (  # noqa: F401
    sdpa_forward,
    sdpa_forward_rows,
    sdpa_backward,
    sdpa_dq_rows,
    sdpa_dkdv_keys,
    softmax_probs,
    visible,
    sdpa_forward_varlen,
    sdpa_backward_varlen,
)
from .tiled import online_forward, online_backward  # noqa: F401
