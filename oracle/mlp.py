"""Plain CPU definition of the MLP sublayer, dense and tensor-parallel sharded.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Sources (the pages' formulas were lost in extraction; the math below is the
plain reading of the code that survives on them):

* "Megatron tensor-parallel MLP" (synapticradio.com):
  - "Start with the dense block": the block is residual + down(SiLU(gate(N)) * up(N)) + b_down
    with N = rms_norm(x, norm_weight); gate/up stacked as w_gate_up[2, F, H]
    (plane 0 gate, plane 1 up), w_down [H, F], b_down [H].
  - the shard-slicing listing after the shape trace: shard r owns the FFN
    interval [r F/P, (r+1) F/P) of both gate/up planes and of the down columns;
    F % P == 0 is asserted.
  - "Split the expansion": each shard computes its own gate/up/SwiGLU channels
    from the replicated N, with no communication.
  - "Split the contraction": each shard produces a full-width partial of the
    down projection; the partials are summed (all-reduce), then residual and
    bias are added once.  Backward of that sum is the identity.
  - "Put the other collective in backward": each shard's contribution to the
    gradient of the replicated N must be summed before RMSNorm's backward.
  - "Remove each collective": the two ablations and the record fields.
* "Megatron-LM walkthrough" (Stanley Jacob), Part II ParallelMLP listing and
  Part V "Deep dive: tensor parallelism and the f and g operators": the GeLU
  variant (fc1 column-parallel with bias, gelu, fc2 row-parallel with bias,
  skip_bias_add so biases are added after the reduction) and the f/g pair.

Readings where the pages are silent:
  rms_norm(x, w) = x / sqrt(mean_H(x^2) + eps) * w, no mean subtraction, no bias;
  SiLU(v) = v * sigmoid(v); GeLU is the exact erf form;
  loss = sum(out^2) / 2, so d loss / d out = out;
  the optimiser is plain SGD, p <- p - lr * grad on every parameter.

Storage precision.  The bf16 workloads state "bf16 weights and activations
with fp32 accumulate".  With ``storage="bf16"`` every activation tensor the
block stores is a bf16 tensor: N, the gate/up (or fc1) pre-activations, the
activation A, the block output, the pre-activation gradients, and dx are
each rounded once (to nearest, ties to even) where they are produced, and
later steps consume the rounded values; contractions, partial sums, row
statistics and parameter gradients stay exact (the accumulation type).
Updated bf16 parameters are rounded; fp32 master copies are not.
``storage="exact"`` (the default) rounds nothing.
"""

from __future__ import annotations

import dataclasses
import math
from typing import List, Optional

import numpy as np
from scipy.special import erf as _erf

MODES = ("equivalence", "missing_forward_reduce", "missing_backward_reduce")


def bf16_round(v):
    """Round to the nearest bfloat16 value, ties to even (8 significant bits,
    the fp32 exponent range).  Returns the rounded values in v's dtype
    (float32 stays float32, anything else becomes float64).

    float32 input: on the bit pattern, add 0x7fff plus the lowest kept bit
    and clear the 16 dropped bits (round-half-even of the dropped part;
    finite values only, overflow carries into the exponent and gives inf).
    float64 input: v = m 2^e with 1/2 <= |m| < 1; m 2^8 is rounded to an
    integer half-to-even and scaled back (no double rounding through fp32)."""
    v = np.asarray(v)
    if v.dtype == np.float32:
        u = v.view(np.uint32).astype(np.uint32, copy=True)
        u += np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
        u &= np.uint32(0xFFFF0000)
        return u.view(np.float32)
    v = v.astype(np.float64, copy=False)
    m, e = np.frexp(v)
    r = np.ldexp(np.rint(np.ldexp(m, 8)), e - 8)
    return np.where(np.abs(r) > 3.3895313892515355e38, np.copysign(np.inf, v), r)


def _identity(v):
    return v


def storage_rounding(storage: str):
    """The rounding applied where the block stores an activation."""
    if storage == "exact":
        return _identity
    if storage == "bf16":
        return bf16_round
    raise ValueError(storage)


@dataclasses.dataclass
class Params:
    """Parameters of the block (dense, or one shard's local slice).

    norm_w [H]; w_in [2, F, H] (SwiGLU: plane 0 gate, plane 1 up) or [F, H]
    (GeLU fc1); b_in [F] (GeLU fc1 bias) or None; w_down [H, F]; b_down [H].
    """

    norm_w: np.ndarray
    w_in: np.ndarray
    w_down: np.ndarray
    b_down: np.ndarray
    b_in: Optional[np.ndarray] = None

    def astype(self, dtype) -> "Params":
        cv = lambda a: None if a is None else np.asarray(a, dtype=dtype).copy()
        return Params(cv(self.norm_w), cv(self.w_in), cv(self.w_down), cv(self.b_down), cv(self.b_in))

    def names(self):
        return [k for k in ("norm_w", "w_in", "b_in", "w_down", "b_down") if getattr(self, k) is not None]


# ---------------------------------------------------------------- elementwise

def sigmoid(v):
    return 1.0 / (1.0 + np.exp(-v))


def silu(v):
    """SiLU(v) = v * sigmoid(v) (F.silu of the dense block listing)."""
    return v * sigmoid(v)


def silu_grad(v):
    """d SiLU / dv = sigmoid(v) * (1 + v * (1 - sigmoid(v)))."""
    s = sigmoid(v)
    return s * (1.0 + v * (1.0 - s))


def gelu(v):
    """Exact GeLU: v * Phi(v) = v/2 * (1 + erf(v / sqrt 2))."""
    return 0.5 * v * (1.0 + _erf(v / math.sqrt(2.0)))


def gelu_grad(v):
    """d GeLU / dv = Phi(v) + v * phi(v), phi the standard normal density."""
    cdf = 0.5 * (1.0 + _erf(v / math.sqrt(2.0)))
    pdf = np.exp(-0.5 * v * v) / math.sqrt(2.0 * math.pi)
    return cdf + v * pdf


# -------------------------------------------------------------------- RMSNorm

def rms_norm_fwd(x, w, eps):
    """Pre-norm of the dense block: r_t = 1/sqrt(mean_i x_ti^2 + eps),
    n_ti = x_ti * r_t * w_i.  Returns (n [T,H], r [T])."""
    H = x.shape[1]
    ms = np.sum(x * x, axis=1) / H
    r = 1.0 / np.sqrt(ms + eps)
    n = x * r[:, None] * w[None, :]
    return n, r


def rms_norm_bwd(dN, x, r, w):
    """Backward of rms_norm_fwd for an incoming gradient dN of the normed
    activation.  With c_t = (1/H) sum_i dN_ti w_i x_ti:
        d x_ti = r_t dN_ti w_i - x_ti r_t^3 c_t
        d w_i  = sum_t dN_ti x_ti r_t
    Returns (dx_norm [T,H], dw [H]).  The residual's gradient is added by
    the caller."""
    H = x.shape[1]
    c = np.sum(dN * w[None, :] * x, axis=1) / H
    dx = r[:, None] * dN * w[None, :] - x * (r ** 3)[:, None] * c[:, None]
    dw = np.sum(dN * x * r[:, None], axis=0)
    return dx, dw


# ------------------------------------------------------ expansion / contraction

def activation_fwd(pre, act: str, R=_identity):
    """The activation applied locally to a shard's pre-activations ("Split the
    expansion": no communication).  SwiGLU: pre = (g, u), a = SiLU(g) * u;
    GeLU: pre = (h,), a = gelu(h).  ``R`` is the storage rounding of a."""
    if act == "swiglu":
        g, u = pre
        return R(silu(g) * u)
    if act == "gelu":
        (h,) = pre
        return R(gelu(h))
    raise ValueError(act)


def activation_bwd(da, pre, act: str, R=_identity):
    """Backward of activation_fwd for incoming da = dL/da.  SwiGLU:
    dg = da * u * SiLU'(g), du = da * SiLU(g); GeLU: dh = da * gelu'(h).
    Returns the tuple of pre-activation gradients, each rounded by ``R``
    (they are stored tensors: the pre-activation gradients)."""
    if act == "swiglu":
        g, u = pre
        return R(da * u * silu_grad(g)), R(da * silu(g))
    if act == "gelu":
        (h,) = pre
        return (R(da * gelu_grad(h)),)
    raise ValueError(act)


def expansion_fwd(n, p: Params, act: str, R=_identity):
    """Column-parallel expansion on whatever channels ``p`` holds.
    SwiGLU: g = n Wg^T, u = n Wu^T, a = SiLU(g) * u; returns (pre=(g, u), a).
    GeLU:   h = n W1^T + b1, a = gelu(h);             returns (pre=(h,), a).
    ``R`` is the storage rounding of the pre-activations and of a."""
    if act == "swiglu":
        pre = (R(n @ p.w_in[0].T), R(n @ p.w_in[1].T))
    elif act == "gelu":
        pre = (R(n @ p.w_in.T + p.b_in[None, :]),)
    else:
        raise ValueError(act)
    return pre, activation_fwd(pre, act, R)


def expansion_bwd(da, n, pre, p: Params, act: str, R=_identity, with_d_pre: bool = False):
    """Backward of expansion_fwd for incoming da.  Returns
    (d_w_in, d_b_in or None, dN contribution of these channels), and with
    ``with_d_pre`` also the pre-activation gradients (dg, du) or (dh,).
    ``R`` is the storage rounding of the pre-activation gradients."""
    d_pre = activation_bwd(da, pre, act, R)
    if act == "swiglu":
        dg, du = d_pre
        res = (np.stack([dg.T @ n, du.T @ n]), None, dg @ p.w_in[0] + du @ p.w_in[1])
    else:
        (dh,) = d_pre
        res = (dh.T @ n, np.sum(dh, axis=0), dh @ p.w_in)
    return res + (d_pre,) if with_d_pre else res


def _sgd(p: Params, grads: dict, lr, R=_identity) -> Params:
    """Plain SGD, p <- p - lr * grad, on every parameter tensor; ``R`` is
    the storage rounding of the updated parameters."""
    new = {}
    for k in ("norm_w", "w_in", "b_in", "w_down", "b_down"):
        v = getattr(p, k)
        new[k] = None if v is None else R(v - lr * grads[k])
    return Params(new["norm_w"], new["w_in"], new["w_down"], new["b_down"], new["b_in"])


# ------------------------------------------------------------------ dense step

def dense_step(x, p: Params, act: str, eps: float, lr: float, dtype=np.float64, storage: str = "exact") -> dict:
    """One dense training step of the block: forward, loss = sum(out^2)/2,
    backward with d out = out, SGD.  All arithmetic in ``dtype``; stored
    activations rounded per ``storage`` (see the module docstring).
    ``new_params`` are the updated parameters in storage precision,
    ``new_masters`` the unrounded updates (fp32 master copies)."""
    R = storage_rounding(storage)
    x = np.asarray(x, dtype=dtype)
    p = p.astype(dtype)
    n, r = rms_norm_fwd(x, p.norm_w, eps)
    n = R(n)
    pre, a = expansion_fwd(n, p, act, R)
    z = a @ p.w_down.T
    out = R(x + z + p.b_down[None, :])
    loss = 0.5 * np.sum(out * out)
    dY = out
    g = {}
    g["b_down"] = np.sum(dY, axis=0)
    g["w_down"] = dY.T @ a
    da = dY @ p.w_down
    g["w_in"], g["b_in"], dN, d_pre = expansion_bwd(da, n, pre, p, act, R, with_d_pre=True)
    dxn, g["norm_w"] = rms_norm_bwd(dN, x, r, p.norm_w)
    dx = R(dY + dxn)
    return dict(x=x, n=n, rstd=r, pre=pre, a=a, z=z, out=out, loss=loss, dY=dY, da=da,
                d_pre=d_pre, dN=dN, dx=dx, grads=g, params=p, new_params=_sgd(p, g, lr, R), new_masters=_sgd(p, g, lr))


# ---------------------------------------------------------------- sharded step

def _shard_params(p: Params, s: int, shards: int, act: str) -> Params:
    F = p.w_down.shape[1]
    if F % shards != 0:
        raise ValueError(f"ffn width {F} is not divisible by {shards} shards")
    fl = F // shards
    lo, hi = s * fl, (s + 1) * fl
    w_in = p.w_in[:, lo:hi, :] if act == "swiglu" else p.w_in[lo:hi, :]
    b_in = None if p.b_in is None else p.b_in[lo:hi].copy()
    # The replicated tensors (norm weight, down bias) are the same on every shard.
    return Params(p.norm_w.copy(), np.ascontiguousarray(w_in), np.ascontiguousarray(p.w_down[:, lo:hi]),
                  p.b_down.copy(), b_in)


def _ordered_sum(parts: List[np.ndarray]) -> np.ndarray:
    """Fixed-order sum ((p0 + p1) + p2) + ... standing in for the all-reduce."""
    acc = parts[0].copy()
    for q in parts[1:]:
        acc = acc + q
    return acc


def sharded_step(x, p: Params, act: str, eps: float, lr: float, shards: int,
                 mode: str = "equivalence", dtype=np.float64, storage: str = "exact") -> dict:
    """The tensor-parallel decomposition of dense_step over ``shards`` ranks,
    run one rank after the other.  Coded separately from dense_step.

    mode "equivalence": the partial down outputs are summed before residual and
    bias (forward boundary), and the ranks' contributions to d N are summed
    before RMSNorm's backward (backward boundary).
    mode "missing_forward_reduce": each rank takes its own partial as the whole
    MLP output (out_r = x + z_r + b) and back-propagates from its own loss; the
    backward sum of d N is still performed.
    mode "missing_backward_reduce": the forward sum is kept; each rank feeds
    only its own d N_r into RMSNorm's backward.

    Returns per-rank lists (index r) of every local tensor, plus ``partials``."""
    if mode not in MODES:
        raise ValueError(mode)
    R = storage_rounding(storage)
    x = np.asarray(x, dtype=dtype)
    p = p.astype(dtype)
    ranks = []
    for s in range(shards):
        lp = _shard_params(p, s, shards, act)
        n, r = rms_norm_fwd(x, lp.norm_w, eps)          # replicated input, computed per rank
        n = R(n)
        pre, a = expansion_fwd(n, lp, act, R)            # local channels, no communication
        z = a @ lp.w_down.T                              # full-width partial output
        ranks.append(dict(params=lp, n=n, rstd=r, pre=pre, a=a, z=z))

    # Forward boundary (g): all-reduce of the partials, then residual + bias once.
    if mode == "missing_forward_reduce":
        for rk in ranks:
            rk["out"] = R(x + rk["z"] + rk["params"].b_down[None, :])
    else:
        zsum = _ordered_sum([rk["z"] for rk in ranks])
        for rk in ranks:
            rk["out"] = R(x + zsum + rk["params"].b_down[None, :])

    # Backward up to the replicated normed input.  g's backward is the identity,
    # so every rank starts from the same d out (= out, from loss sum(out^2)/2).
    for rk in ranks:
        lp, dY = rk["params"], rk["out"]
        rk["loss"] = 0.5 * np.sum(dY * dY)
        g = {"b_down": np.sum(dY, axis=0), "w_down": dY.T @ rk["a"]}
        da = dY @ lp.w_down
        g["w_in"], g["b_in"], rk["dN_partial"], rk["d_pre"] = expansion_bwd(da, rk["n"], rk["pre"], lp, act, R,
                                                                          with_d_pre=True)
        rk["da"] = da
        rk["grads"] = g

    # Backward boundary (f): all-reduce of the d N contributions.
    if mode == "missing_backward_reduce":
        for rk in ranks:
            rk["dN"] = rk["dN_partial"]
    else:
        dNsum = _ordered_sum([rk["dN_partial"] for rk in ranks])
        for rk in ranks:
            rk["dN"] = dNsum

    for rk in ranks:
        lp = rk["params"]
        dxn, rk["grads"]["norm_w"] = rms_norm_bwd(rk["dN"], x, rk["rstd"], lp.norm_w)
        rk["dx"] = R(rk["out"] + dxn)
        rk["new_params"] = _sgd(lp, rk["grads"], lr, R)
    return dict(ranks=ranks, mode=mode, shards=shards, act=act)


def assemble(sh: dict, key: str, which: str = "grads") -> np.ndarray:
    """Re-assemble a sharded parameter tensor (from rank 0..S-1 slices) into
    its dense shape.  ``which`` is "grads", "params" or "new_params"."""
    ranks, act = sh["ranks"], sh["act"]
    get = (lambda rk: rk[which][key]) if which == "grads" else (lambda rk: getattr(rk[which], key))
    parts = [get(rk) for rk in ranks]
    if key == "w_in":
        return np.concatenate(parts, axis=1 if act == "swiglu" else 0)
    if key == "w_down":
        return np.concatenate(parts, axis=1)
    if key == "b_in":
        return np.concatenate(parts, axis=0)
    raise KeyError(key)


def fixture_record(dense: dict, sh: dict) -> dict:
    """The comparison record of the page's fixture ("Reproduce one dense
    training step" / "Remove each collective"): max-abs differences of the
    sharded step against the dense step, maximised over ranks."""
    ranks, act = sh["ranks"], sh["act"]
    mx = lambda arrs: float(max(np.max(np.abs(a)) if a.size else 0.0 for a in arrs))
    dg = dense["grads"]
    rec = {"mode": sh["mode"], "world_size": sh["shards"]}
    rec["forward_max_abs_diff"] = mx([rk["out"] - dense["out"] for rk in ranks])
    rec["loss_abs_diff"] = float(max(abs(float(rk["loss"]) - float(dense["loss"])) for rk in ranks))
    rec["input_grad_max_abs_diff"] = mx([rk["dx"] - dense["dx"] for rk in ranks])
    rec["norm_grad_max_abs_diff"] = mx([rk["grads"]["norm_w"] - dg["norm_w"] for rk in ranks])
    fl = dense["params"].w_down.shape[1] // sh["shards"]
    sl = lambda s: slice(s * fl, (s + 1) * fl)
    if act == "swiglu":
        gu = [rk["grads"]["w_in"] - dg["w_in"][:, sl(s), :] for s, rk in enumerate(ranks)]
    else:
        gu = [rk["grads"]["w_in"] - dg["w_in"][sl(s), :] for s, rk in enumerate(ranks)]
    rec["gate_up_grad_max_abs_diff"] = mx(gu)
    rec["down_grad_max_abs_diff"] = mx([rk["grads"]["w_down"] - dg["w_down"][:, sl(s)]
                                        for s, rk in enumerate(ranks)])
    rec["down_bias_grad_max_abs_diff"] = mx([rk["grads"]["b_down"] - dg["b_down"] for rk in ranks])
    post = []
    dn = dense["new_params"]
    for s, rk in enumerate(ranks):
        npar = rk["new_params"]
        post.append(npar.norm_w - dn.norm_w)
        post.append(npar.b_down - dn.b_down)
        post.append(npar.w_down - dn.w_down[:, sl(s)])
        post.append(npar.w_in - (dn.w_in[:, sl(s), :] if act == "swiglu" else dn.w_in[sl(s), :]))
        if npar.b_in is not None:
            post.append(npar.b_in - dn.b_in[sl(s)])
    rec["post_step_weight_max_abs_diff"] = mx(post)
    return rec


def inspect_record(seq: int, batch: int, hidden: int, ffn: int, world: int, rank: int = 0) -> dict:
    """Shape record of the page's ``inspect`` mode ("Reproduce one dense
    training step"), produced by running the dense block and one rank's shard
    on a [seq, batch, hidden] input and reading the shapes of what they made."""
    T = seq * batch
    rng = np.random.default_rng(0)
    x = rng.standard_normal((T, hidden))
    p = Params(np.ones(hidden), rng.standard_normal((2, ffn, hidden)) * 0.1,
               rng.standard_normal((hidden, ffn)) * 0.1, np.zeros(hidden))
    d = dense_step(x, p, "swiglu", 1e-6, 0.1)
    sh = sharded_step(x, p, "swiglu", 1e-6, 0.1, world)
    rk = sh["ranks"][rank]
    tok = lambda a: [seq, batch] + list(a.shape[1:])
    return {
        "world_size": world,
        "block_path": "pre-RMSNorm -> fused gate/up -> SwiGLU -> down projection -> residual add",
        "dense_shapes": {
            "x": tok(d["x"]),
            "norm_weight": list(d["params"].norm_w.shape),
            "w_gate_up": list(d["params"].w_in.shape),
            "w_down": list(d["params"].w_down.shape),
            "output": tok(d["out"]),
        },
        "rank_local_shapes": {
            "gate_up_weight": list(rk["params"].w_in.shape),
            "gate": tok(rk["pre"][0]),
            "up": tok(rk["pre"][1]),
            "swiglu": tok(rk["a"]),
            "down_weight": list(rk["params"].w_down.shape),
            "partial_output": tok(rk["z"]),
        },
    }


# ------------------------------------------------------------ row-sampled step

def row_forward_backward(x_rows, p: Params, act: str, eps: float, dtype=np.float64, storage: str = "exact") -> dict:
    """Forward and the activation-gradient part of the backward for a subset of
    token rows.  Every one of these quantities depends only on its own row
    (the block is row-independent and d out = out), so a sample of rows of a
    full-size workload can be checked exactly without the other rows."""
    R = storage_rounding(storage)
    x = np.asarray(x_rows, dtype=dtype)
    p = p.astype(dtype)
    n, r = rms_norm_fwd(x, p.norm_w, eps)
    n = R(n)
    pre, a = expansion_fwd(n, p, act, R)
    out = R(x + a @ p.w_down.T + p.b_down[None, :])
    da = out @ p.w_down
    _, _, dN = expansion_bwd(da, n, pre, p, act, R)
    dxn, _ = rms_norm_bwd(dN, x, r, p.norm_w)
    return dict(n=n, rstd=r, pre=pre, a=a, out=out, da=da, dN=dN, dx=R(out + dxn))
