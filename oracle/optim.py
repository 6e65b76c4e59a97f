"""Optimiser side of the training step: gradient accumulation over
microbatches, global gradient-norm clipping and AdamW.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Sources:

* "Megatron-LM walkthrough" (stanleyjacob.dev), Part IV:
  - Stage 4: a global batch is split into microbatches; with no pipeline
    parallelism the schedule is a plain loop over them, each a forward and a
    backward.
  - Stage 8: once the gradients are final, their norm over every
    model-parallel dimension is computed and the gradients are clipped, then
    AdamW updates the parameters; fp32 master parameters and the optimiser
    states are what the distributed optimiser shards.
  - Part II, the example launch: weight decay 0.1, gradient clip 1.0.
* "Megatron-Core Guide: 5D Distributed Training Architecture", section 1
  ("The Static Memory Wall"): Adam keeps a first moment m and a second moment
  v in fp32 and an fp32 master copy of each weight.

The pages do not write the update out.  The oracle follows the published
algorithm: Loshchilov & Hutter, "Decoupled Weight Decay Regularization"
(ICLR 2019), Algorithm 2 (AdamW), with the bias correction of Kingma & Ba,
"Adam" (ICLR 2015), Algorithm 1:

    m_t = b1 m_{t-1} + (1 - b1) g_t
    v_t = b2 v_{t-1} + (1 - b2) g_t^2
    theta_t = theta_{t-1} - lr * ( (m_t / (1 - b1^t)) / (sqrt(v_t / (1 - b2^t)) + eps)
                                   + wd * theta_{t-1} )

Readings where the pages are silent: b1 = 0.9,
b2 = 0.999, eps = 1e-8 unless a caller sets them; the decay acts on every
parameter tensor; clipping scales every gradient by
c = min(1, max_norm / (||g||_2 + 1e-6)), ||g||_2 the norm of all gradient
tensors together; the gradient of a global batch is the sum of its
microbatches' gradients (the loss is a sum over tokens), accumulated in fp32.
"""

from __future__ import annotations

import math
from typing import Dict, List, Sequence

import numpy as np

from .mlp import Params, dense_step

ADAM_BETA1 = 0.9
ADAM_BETA2 = 0.999
ADAM_EPS = 1e-8
CLIP_EPS = 1e-6


def microbatch_bounds(tokens: int, microbatches: int) -> List[tuple]:
    """Contiguous token slices [lo, hi) of a global batch: the first
    ``tokens % microbatches`` slices hold one token more than the rest."""
    if microbatches < 1:
        raise ValueError("microbatches must be >= 1")
    base, extra = divmod(tokens, microbatches)
    bounds, lo = [], 0
    for i in range(microbatches):
        hi = lo + base + (1 if i < extra else 0)
        bounds.append((lo, hi))
        lo = hi
    return bounds


def accumulated_grads(x, p: Params, act: str, eps: float, microbatches: int, dtype=np.float64,
                      storage: str = "exact") -> Dict[str, np.ndarray]:
    """Parameter gradients of the whole batch as the schedule forms them:
    one forward and backward per microbatch (a slice of the token rows), the
    per-microbatch gradients added in microbatch order."""
    x = np.asarray(x)
    total = None
    for lo, hi in microbatch_bounds(x.shape[0], microbatches):
        g = dense_step(x[lo:hi], p, act, eps, 0.0, dtype=dtype, storage=storage)["grads"]
        if total is None:
            total = {k: (None if v is None else np.array(v, dtype=dtype, copy=True)) for k, v in g.items()}
        else:
            for k, v in g.items():
                if v is not None:
                    total[k] = total[k] + v
    return total


def global_grad_norm(grads: Sequence[np.ndarray]) -> float:
    """Euclidean norm of all gradient tensors taken together, in fp64."""
    s = 0.0
    for g in grads:
        if g is not None:
            a = np.asarray(g, dtype=np.float64)
            s += float(np.sum(a * a))
    return math.sqrt(s)


def clip_coefficient(norm: float, max_norm: float) -> float:
    """Factor every gradient is multiplied by before the update; 1 when the
    norm is within max_norm or when clipping is off (max_norm <= 0)."""
    if max_norm <= 0:
        return 1.0
    return min(1.0, max_norm / (norm + CLIP_EPS))


def adamw_update(theta, grad, m, v, step: int, lr: float, weight_decay: float, beta1: float = ADAM_BETA1,
                 beta2: float = ADAM_BETA2, eps: float = ADAM_EPS, grad_scale: float = 1.0):
    """One AdamW update of one tensor (step counts from 1).  Returns the new
    (theta, m, v) in fp64; the inputs are left unchanged."""
    if step < 1:
        raise ValueError("step counts from 1")
    theta = np.asarray(theta, dtype=np.float64)
    g = np.asarray(grad, dtype=np.float64) * grad_scale
    m_new = beta1 * np.asarray(m, dtype=np.float64) + (1.0 - beta1) * g
    v_new = beta2 * np.asarray(v, dtype=np.float64) + (1.0 - beta2) * g * g
    m_hat = m_new / (1.0 - beta1 ** step)
    v_hat = v_new / (1.0 - beta2 ** step)
    theta_new = theta - lr * (m_hat / (np.sqrt(v_hat) + eps) + weight_decay * theta)
    return theta_new, m_new, v_new


def adamw_step(params: Dict[str, np.ndarray], grads: Dict[str, np.ndarray], m: Dict[str, np.ndarray],
               v: Dict[str, np.ndarray], step: int, lr: float, weight_decay: float, max_norm: float = 0.0,
               beta1: float = ADAM_BETA1, beta2: float = ADAM_BETA2, eps: float = ADAM_EPS) -> dict:
    """The optimiser step over a set of tensors: the global gradient norm,
    the clip coefficient, then AdamW on every tensor.  ``params`` are the
    fp32 master values (or the parameters themselves when there are no
    masters)."""
    names = [k for k in params if params[k] is not None]
    norm = global_grad_norm([grads[k] for k in names])
    coef = clip_coefficient(norm, max_norm)
    new_p, new_m, new_v = {}, {}, {}
    for k in names:
        new_p[k], new_m[k], new_v[k] = adamw_update(params[k], grads[k], m[k], v[k], step, lr, weight_decay,
                                                    beta1, beta2, eps, coef)
    return dict(norm=norm, coef=coef, params=new_p, m=new_m, v=new_v)
