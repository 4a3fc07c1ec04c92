"""CPU oracle for the sequential MTP depth chain, the shared-head CE and verify.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path imports, links or runs
anything under ``oracle/``: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code with the HIP
library (no kernels, headers, helpers, tables or pre/post-processing); the
only thing both sides consume is the seeded input generator, which holds none
of the method's arithmetic.

Sources (web pages, cited by title and section):

* "M7.6 - DeepSeek MTP: Sequential Modules, Teacher Forcing, and Speculative
  Runtime" (here: M7.6) -- the depth contract (0x02), the module (0x03, 0x03C),
  tensor alignment (0x04), the row compiler (0x04C), the objective (0x05,
  0x05A), the gradient ledger (0x05A-0x05B) and the gradient through the
  whole chain (0x05A, 0x05B), the training loop (0x06A) and the
  one-proposal selector (0x09);
* the speculative-decoding explainer page (ailearn, "speculative-decoding") --
  the gamma-token accept / correct / bonus rule, the single-token invariant
  example and E[N_emit];
* "M7.4 - Multi-Token Prediction Foundations" (here: M7.4) -- the two-row
  packed fixture (0x01A, 0x02C), finite-difference reconciliation (0x04C).

Modules: ``rows`` (label/state compiler), ``chain`` (module forward),
``head`` (shared-head CE forward and its gradients), ``backward`` (the
gradient of L_MTP through every module to h^(0), the embedding and the
per-depth weights), ``verify`` (accept / resample), ``numerics`` (rounding
points).  All arithmetic is float64.

Parity status per function is stated in each module header; a function with
no independent pin says "parity unpinned".
"""
from . import numerics, rows, chain, head, backward, verify  # noqa: F401
