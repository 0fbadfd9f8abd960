"""Plain, slow, fp64 CPU oracle for fused CSR graph attention and the degree-aware
neighbourhood reduction.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or link this
package: only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` use it.  It shares no code with the HIP library (no kernels, helpers,
tables or pre/post-processing); both sides read the same seeded inputs from
``graphgen`` and nothing else.

Source of what is computed: "On Efficient Scaling of GNNs via IO-Aware Layers
Implementations" (gist.science explainer of arXiv 2605.31500), Technical Summary >
Methodology, attention-based layers: per destination node, score every neighbour edge,
softmax-normalise the scores and aggregate the neighbour values; the backward reuses a
per-node log-sum-exp.  The fused kernels reach exactly (up to rounding order) plain
per-row masked softmax attention, so the oracle is that plain definition written out.

Modules
-------
attention   forward / backward definitions (fp64, per-row loops, two-pass softmax)
planner     reference degree-binning planner and CSC transpose (numpy, bit-exact target)
reduction   min / max neighbourhood pooling with its arg, and the routed gradient

Pins (what the oracle is checked against, in ``tests/test_oracle_*.py``):
dense masked attention brute force, torch's fp64 scaled_dot_product_attention with a
boolean mask, closed forms (hand-derived goldens in ``tests/golden/``), invariants
(weights sum to 1, single-neighbour rows, uniform scores give the mean, permutation
invariance, sum of dK is zero, sum of dV equals the sum of dOut), central finite
differences of the forward, fp64 torch autograd of dense masked attention, and for the
planner scipy's CSR->CSC conversion plus partition invariants; for the reduction a
hand-derived example with ties, signed zeros, a parallel edge and an empty row, torch's
scatter_reduce (amax / amin), a sequential brute-force scan, invariants, central finite
differences and torch autograd.  No function here is "parity unpinned".
"""
from . import attention, planner, reduction  # noqa: F401
