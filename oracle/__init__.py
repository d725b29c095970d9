"""fp64 CPU oracle for the DeltaLog decode step.  TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import anything from this package.  The product path (the HIP
library and its Python binding) never imports, calls or falls back to it, and
this package imports nothing from the product path.  The only code the two
sides share is the seeded input generator in ``workloads/``.

Sources (cited by title and equation / section; headings of the first paper
did not survive text extraction, so sections are named by their content):

[DL]   "DeltaLog: Deferred Materialization of Recurrent States for Linear
       Attention Decoding" -- Eq. 1 (causal linear attention), Eq. 3 (common
       decode step), Table 1 (operator instances), Algorithm 1 (append-merge
       cycle), the physical-state list and the logical-state equation of the
       design section, the operator-instantiation section (GDN, KDA, RWKV6).
[FPGA] "A Persistent-State Dataflow Accelerator for Memory-Bound Linear
       Attention Decode on FPGA" -- Table II (per-token profile).

Modules
  recurrence     E: the eager recurrence, Eq. 3, step by step (the parity target)
  deferred       F: base + cumulative log-decay + bounded log, Algorithm 1
  closed_forms   unrolled sums / products and an exact-rational brute force
  schedule       the append/merge bookkeeping in closed form
  pool           a tracked-slot driver of E for serving-pool workloads

Every function is pinned by ``tests/test_oracle_pins.py`` to something other
than itself (closed forms, invariants, exact rationals, the FPGA paper's
printed byte counts).  There is no worked numeric example of the decode step
on the pages, so no output value is pinned to a printed number.
"""

from .recurrence import eager_step, expand_heads, decay_factors  # noqa: F401
from .deferred import DeferredPool  # noqa: F401
from .pool import EagerPool, RelL2  # noqa: F401
from . import closed_forms, schedule  # noqa: F401
