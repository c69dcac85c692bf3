"""CPU oracle for the gated delta-rule recurrence.

TEST INFRASTRUCTURE: only tests/, __graft_entry__.smoke() and bench.py's
cpu_baseline leg import this package.  It shares no code with the HIP path.
"""
from .delta_oracle import (VARIANTS, delta_bwd, delta_decode, delta_fwd,  # noqa: F401
                           efla_step_size, group_heads, run_recurrence, ttt_pre_fwd)
