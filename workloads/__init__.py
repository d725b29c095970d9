"""Seeded synthetic inputs for the DeltaLog decode-step workloads.

This package is the one thing the CPU oracle and the HIP path share: it draws
the per-step token inputs (q, k or a, v or b, log-decay, beta), the slot
schedule, and the initial / replacement base states, from fixed seeds.  It
contains none of the decode-step arithmetic (no decay, no outer product, no
replay): only the input distributions each workload prescribes.

Every returned floating-point array is float32 whose values are already exactly
representable in the workload's storage dtype (bf16 values are rounded to
nearest-even from float32 here), so both sides consume identical numbers.
"""

from .configs import (CONFIGS, SWEEP_OPERATORS, Config, at_batch, get_config, headline_gdn,  # noqa: F401
                      merge_sweep_config, small_variant)
from .gen import StepDesc, StepInputs, Workload, round_to_bf16  # noqa: F401
