"""SGD with momentum on fp32 master weights, one rounding per operation.

TEST INFRASTRUCTURE ONLY (see the package docstring).

The pages: after the all-reduce every replica holds the same averaged
gradient and takes its local optimizer step, so replicas stay identical
(CS336 Lecture 8, "Data Parallelism (DDP)", step 4; "Distributed Training",
"Data parallelism and all-reduce", on momentum state needing identical
gradients); mixed precision keeps an FP32 master copy of the weights and
accumulates in FP32 ("Distributed Training", Related, "Mixed-Precision
Training").  No page writes the update formula.  Reading: the common
heavy-ball form with no dampening, no Nesterov term and no weight decay,

    v <- mu * v + g
    w <- w - lr * v

with lr and mu rounded to float32 and every multiply and add rounded to
float32 separately (no fused multiply-add).

Parity status: pinned by the tests against closed forms (v0 = 0, mu = 0,
power-of-two lr and mu with small-integer gradients, constant gradients over
k steps) and against torch.optim.SGD run in float64.
"""

import numpy as np


def sgd_momentum(g, w, v, lr, mu):
    """One momentum step.  g, w, v: float32 arrays of equal shape.
    Returns the new (w, v) as float32 arrays; the inputs are not modified."""
    g = np.asarray(g, dtype=np.float32)
    w = np.asarray(w, dtype=np.float32)
    v = np.asarray(v, dtype=np.float32)
    lr32 = np.float32(lr)
    mu32 = np.float32(mu)
    v_scaled = mu32 * v            # rounded to float32
    v_new = v_scaled + g           # rounded to float32
    step = lr32 * v_new            # rounded to float32
    w_new = w - step               # rounded to float32
    return w_new.astype(np.float32), v_new.astype(np.float32)
