"""Float64 CPU oracle for IBP, CROWN and alpha-CROWN bound propagation.

TEST INFRASTRUCTURE ONLY.  Only the tests, the package smoke check and the
benchmark's CPU-baseline leg may import or run anything in this package.  The
HIP library never calls it and shares no code with it; both sides read the
same seeded inputs from the ``workloads`` module and nothing else.

Source of the method: "Scaling Neural Network Verification with Tensor
Parallelism and Fully Sharded Data Parallelism" (Vorobyov, Ilyushin), which
names IBP, CROWN and alpha-CROWN as the bound-propagation algorithms
(Sec. 1, problem definition), the linear relaxation matrices A (Sec. 1,
Sec. 4.1), the relaxation slopes lambda_i obtained from intermediate bounds and
the IBP substitution for intermediate bounds (Sec. 2.1), and the per-neuron
alpha tensors (ReLU slopes, Sec. 3 and Sec. 4.3).  The page gives no formulas,
so the arithmetic is the standard published definition of each algorithm
(interval bound propagation; CROWN back-substitution with the adaptive
ReLU relaxation; alpha-CROWN projected gradient ascent on the lower slopes),
written out step by step in float64.

Every function is pinned by the CPU tests against brute force, closed forms,
hand-derived examples and an independent exact rational-arithmetic
implementation on tiny networks (every intermediate-bound mode).  Parity
unpinned: the absolute bound values of the large synthetic workloads (nothing
published to compare them to beyond soundness and structure) and the
architecture readings of the residual workload (its block layout is a reading,
not a value the pages fix).
"""
from .bounds import (Oracle, ibp, relaxation, backward, concretize, crown_bounds,
                     intermediate_bounds, spec_bounds_crown, spec_bounds_ibp)
from .alpha import alpha_crown, adam_ascent_step

__all__ = ["Oracle", "ibp", "relaxation", "backward", "concretize", "crown_bounds",
           "intermediate_bounds", "spec_bounds_crown", "spec_bounds_ibp", "alpha_crown",
           "adam_ascent_step"]
