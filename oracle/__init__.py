"""CPU oracle for the redundant-expert MoE dispatch path -- TEST INFRASTRUCTURE ONLY.

Only the tests, the package's ``smoke()`` check and the benchmark's CPU
baseline leg may import this package.  It shares no code with the HIP
library or its binding and imports neither.

Parity pins (what checks the oracle against something other than itself)
are listed per function in the tests:

* ``maxvio``, ``plan``, ``layout``: hand-worked golden examples
  (tests/golden), invariants on random and adversarial routings, brute-force
  optimal replica counts on tiny inputs, and special cases that reduce to a
  stable argsort / bincount (one rank) or to plain expert parallelism
  (balanced routing).  The relay fallback inside ``plan``: hand-worked relay
  and switch chains, exhaustive search on tiny routings (it finds a plan
  within B slots whenever one exists there) and a mixed-integer feasibility
  check on medium ones.
* ``permute``, ``group_gemm``, ``combine``, ``replica_grad_fold``,
  ``unpermute_reduce``, ``combine_weight_grad``: a simulation of every rank
  that must reproduce the dense MoE definition, its per-expert weight
  gradients, its input gradient and its router-weight gradient exactly on
  small-integer inputs; ``unpermute_reduce`` is also checked as the adjoint
  of ``permute``.
* ``silu``, ``group_gemm_swiglu``, ``swiglu_backward`` (the gated variant):
  scipy's logistic function, closed forms (silu(x) - silu(-x) = x), central
  differences of the forward, and a dense gated MoE written copy by copy.
* ``bf16``: torch's CPU cast on sampled bit patterns.

Parity unpinned: any specific plan versus the original library's planner
(the pages print none).
"""
from .moe_ref import (  # noqa: F401
    STATUS_BAD_EXPERT_ID, STATUS_SLOT_OVERFLOW, HEADER_WORDS, Plan, Replica, maxvio, histogram,
    plan, plan_words, layout, layout_loops, permute, group_gemm, group_gemm_rows, wgrad_entries,
    combine, replica_grad_fold, prefetch, unpermute_reduce, combine_weight_grad, silu,
    group_gemm_swiglu, swiglu_backward,
)
from .bf16 import (  # noqa: F401
    bf16_bits_to_f32, bf16_bits_to_f64, f32_to_bf16_bits, f64_to_bf16_bits,
)
