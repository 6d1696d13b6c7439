"""CPU f64 oracle for the decode-time int4 MoE expert path.  TEST INFRASTRUCTURE.

This package is the plain, slow definition that the HIP library is checked
against.  Only the test suite, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import it.  It shares no code with the
library (``int4_grouped_expert_router_amd``) and imports nothing from it.

Sources (the web pages the method is described on), cited in each module as:

* [PR651]   "cuda: add experimental lossless compressed expert tier" (PR #651):
            per-row int4 experts, fused decode+matvec follow-up.
* [LOG-g4]  "Commit history of c/backend_cuda.cu", the commit opening "The grouped
            MoE kernels were per-row-only": group-wise int4 (fmt=4), group size
            gs, O*ceil(C/gs) scales, offset-binary nibbles, the tail group.
* [LOG-tc]  same page, the commit gating the TC_W4A16 branch: the 3-launch grouped
            path (dual gate/up, silu, down).
* [LOG-rt]  same page, the commit "First increment of the #431 plan": device router
            (E x D logits GEMV, sigmoid, bias-augmented top-K by choice with
            strict-> tie-breaking, weights from the raw logit, route-level top-p,
            norm_topk, routed_scale, packed result).
* [LOG-pipe] same page, the "GPU resident pipeline" commit: batched router over S
            rows, silu-mul, fixed-order row merge without atomics.
* [PR342]   "cuda: COLI_GROUP_ASYNC=1 - overlap the CPU expert rows with the GPU
            groups at decode", section "What": S<=4 small-batch grouped decode,
            issue/take split.
* [LOG-mla] same page, the "CUDA batch MLA attention, ..., W4A16 kernels" commit: the
            shared expert runs as a W4A16 MLP beside the expert groups.
* [PR434]   "cuda: COLI_CUDA_RESID=1 - expert-group results stay on device",
            section "What": per-expert weighting, fixed-order reduce into a
            per-issue slot, take reduces slots in issue order into the residual.

Readings of points the pages leave open are stated where they are used.  Every function here is pinned by ``tests/test_oracle_*``
against brute force, closed forms, invariants or library routines; none is
"parity unpinned".
"""

from . import block, brute, experts, int4, router  # noqa: F401
from .experts import (  # noqa: F401
    build_group,
    expert_forward,
    moe_layer,
    silu,
)
from .int4 import dequantize, dequantize_rows, matvec_rows, n_groups, unpack_nibbles  # noqa: F401
from .router import RouteResult, route, route_token, router_logits, select_topk, widen_activations  # noqa: F401
