"""CPU oracle for the low-rank bottleneck block -- TEST INFRASTRUCTURE ONLY.

Only the tests, the smoke check's comparison and the benchmark's CPU-baseline
leg may import this package.  The product path (the HIP library and its Python
binding) never imports, calls or falls back to it, and the two share no code:
the oracle is a plain float64 NumPy restatement of what the block computes,
written from the BOOST pages:

  "BOOST: BOttleneck-Optimized Scalable Training Framework for Low-Rank Large
  Language Models" -- technical summary (gist.science, §1 Problem statement,
  §2.1 Bottleneck-aware tensor parallelism, §2.2 System-level optimisations,
  §4 results) and the arXiv abstract (2512.12131).

``block`` is the bottleneck block itself; ``mlp`` the per-projection low-rank
SwiGLU MLP (the other reading of the SwiGLU wiring).

Where the pages leave a step open (the block formula, the nonlinearity, the
RMSNorm formula, the checkpoint contents), the oracle takes the plain readings
listed in the design notes; each function names the reading it uses.

Pins: every function here is pinned by the ``-m "not gpu"`` tests in
``tests/test_oracle_*.py`` against brute-force loops, closed forms, invariants
and library routines (see each test's docstring).  No function is "parity
unpinned".
"""
from .block import (act_forward, act_backward, rms_stats, rmsnorm, block_fwd, block_bwd,
                    down_partial, up_finish, branch_slices, working_precision)
from .mlp import mlp_fwd, mlp_bwd

__all__ = ["act_forward", "act_backward", "rms_stats", "rmsnorm", "block_fwd", "block_bwd",
           "down_partial", "up_finish", "branch_slices", "working_precision", "mlp_fwd", "mlp_bwd"]
