"""CPU oracle for the placement-aware gradient-reduction + AdamW path.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the package's smoke check and
the benchmark's CPU-baseline leg may import this package.  The GPU product
path never imports, calls or links it, and it imports nothing from the
product package.

It is a plain, slow, step-by-step statement of what the path computes,
written from these pages:

* P1 -- NeMo Automodel issue #3857, "refactor(distributed): establish shared
  native TP replica ownership" (sections "Why this needs separate work",
  "Preserved prototype and evidence", "Proposed scope and acceptance
  criteria").
* P3 -- Cosmos 3 training framework, "distributed parallel" page (section 1,
  the dp_replicate axis whose replicas all-reduce gradients).
* P4 -- Mixle v0.8.1, "Distributed Transformer Training" (sections "Backend
  split" and "Optimizer and checkpoint semantics").

Precision: the pages fix the reduction and accumulation dtype as FP32 (P1,
"Preserved prototype and evidence": an FP32 reduction hook) and BF16
gradients; the master shard and Adam moments are FP32.  So every per-element
step is evaluated in FP32, one IEEE-rounded operation at a time, in the order
written in ``method.py``.  The global norm, whose precision the pages leave
open, is computed in FP64 as the correctly rounded sum of the exact squares.

Pins (tests marked ``not gpu``) tie each function to something other than
itself: closed forms, brute-force gradients of tiny sharded layers,
library special cases (torch.optim.AdamW, clip_grad_norm_, torch's bfloat16
cast, exact rational sums) and hand-enumerated ownership tables.
The whole path against the pages' own system is parity unpinned: the pages
print no values for it.
"""
from . import method  # noqa: F401
from .method import *  # noqa: F401,F403
