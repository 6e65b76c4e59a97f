"""Sequence-parallel form of the tensor-parallel MLP sublayer.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Sources:

* "Megatron-LM walkthrough" (stanleyjacob.dev):
  - Part V, "Deep dive: sequence parallelism, memory for free": the regions
    between the parallel linears (norm, residual add) run on a slice of the
    sequence per tensor-parallel rank; the tensor-parallel all-reduce is split
    into its two halves, an all-gather entering the tensor-parallel region and
    a reduce-scatter leaving it, with the same bytes moved.
  - Part IV, Stage 5: with sequence parallelism each all-reduce of a block
    becomes an all-gather entering the tensor-parallel region and a
    reduce-scatter leaving it.
  - Part IV, Stage 7: with sequence parallelism the norm parameters are
    replicated across the tensor-parallel group but each rank computes their
    gradient from its own sequence slice, so those gradients must be summed
    over the group; leaving this out trains, wrongly, without any error.
* "Megatron-Core Guide: 5D Distributed Training Architecture", section on
  sequence parallelism: rank i holds X_i, a 1/N slice of the sequence; the
  row-parallel output is reduce-scattered, the norm runs on the slice, and an
  all-gather rebuilds the full sequence before the next column-parallel linear.

Layout and readings: x is [T, H] with the sequence axis
outermost, so a sequence slice is a contiguous block of token rows; rank r
holds rows [lo_r, hi_r), the first T % S ranks one row more than the rest
(the pages assume T divisible by S; the ragged split is a harmless
generalisation).  The bias b_down is added after the reduce-scatter, once per
row, and like norm_w it is replicated, so its gradient is summed over the
ranks as well.  Sums over ranks run in rank order.
"""

from __future__ import annotations

from typing import List

import numpy as np

from .mlp import (Params, _shard_params, _sgd, expansion_bwd, expansion_fwd, rms_norm_bwd, rms_norm_fwd,
                  storage_rounding)

SP_MODES = ("equivalence", "missing_norm_grad_reduce")


def sequence_slices(tokens: int, ranks: int) -> List[tuple]:
    """Rows [lo, hi) of each rank's sequence slice."""
    base, extra = divmod(tokens, ranks)
    out, lo = [], 0
    for r in range(ranks):
        hi = lo + base + (1 if r < extra else 0)
        out.append((lo, hi))
        lo = hi
    return out


def _rank_order_sum(parts):
    acc = parts[0].copy()
    for p in parts[1:]:
        acc = acc + p
    return acc


def sequence_parallel_step(x, p: Params, act: str, eps: float, lr: float, shards: int, mode: str = "equivalence",
                           dtype=np.float64, storage: str = "exact") -> dict:
    """One training step with S tensor-parallel ranks in the sequence-parallel
    layout.  Rank r owns FFN channels [r F/S, (r+1) F/S) (as in the plain
    tensor-parallel split) and token rows sequence_slices(T, S)[r] of the
    regions outside the tensor-parallel linears."""
    if mode not in SP_MODES:
        raise ValueError(mode)
    R = storage_rounding(storage)
    x = np.asarray(x, dtype=dtype)
    p = p.astype(dtype)
    T = x.shape[0]
    sl = sequence_slices(T, shards)
    ranks = [dict(lo=lo, hi=hi) for lo, hi in sl]
    locs = [_shard_params(p, r, shards, act) for r in range(shards)]

    # forward: the norm on each rank's slice, then the all-gather of N
    for rk in ranks:
        n_r, rstd_r = rms_norm_fwd(x[rk["lo"]:rk["hi"]], p.norm_w, eps)
        rk["n"], rk["rstd"] = R(n_r), rstd_r
    n_full = np.concatenate([rk["n"] for rk in ranks], axis=0)
    # tensor-parallel region: every rank on the full sequence, its own channels
    for rk, lp in zip(ranks, locs):
        rk["pre"], rk["a"] = expansion_fwd(n_full, lp, act, R)
        rk["z"] = rk["a"] @ lp.w_down.T
    # reduce-scatter leaving the region, then residual and bias on the slice
    for rk in ranks:
        lo, hi = rk["lo"], rk["hi"]
        zsum = _rank_order_sum([q["z"][lo:hi] for q in ranks])
        rk["out"] = R(x[lo:hi] + zsum + p.b_down[None, :])
    out = np.concatenate([rk["out"] for rk in ranks], axis=0)
    loss = 0.5 * float(np.sum(out * out))

    # backward: the gradient of the reduce-scatter is the all-gather of dY
    dY = out
    for rk, lp in zip(ranks, locs):
        g = {}
        g["w_down"] = dY.T @ rk["a"]
        da = dY @ lp.w_down
        g["w_in"], g["b_in"], rk["dN_part"] = expansion_bwd(da, n_full, rk["pre"], lp, act, R)
        rk["grads"] = g
    # gradient of the all-gather: reduce-scatter of the dN partials, then the
    # norm backward and the residual on the slice
    for rk in ranks:
        lo, hi = rk["lo"], rk["hi"]
        dN_r = _rank_order_sum([q["dN_part"][lo:hi] for q in ranks])
        dxn, rk["d_norm_w_local"] = rms_norm_bwd(dN_r, x[lo:hi], rk["rstd"], p.norm_w)
        rk["dN"] = dN_r
        rk["dx"] = R(dY[lo:hi] + dxn)
        rk["d_b_down_local"] = np.sum(dY[lo:hi], axis=0)
    dx = np.concatenate([rk["dx"] for rk in ranks], axis=0)
    # the replicated norm weight and bias: gradients summed over the group
    if mode == "equivalence":
        d_norm_w = _rank_order_sum([rk["d_norm_w_local"] for rk in ranks])
        d_b_down = _rank_order_sum([rk["d_b_down_local"] for rk in ranks])
        for rk in ranks:
            rk["d_norm_w"], rk["d_b_down"] = d_norm_w, d_b_down
    else:
        for rk in ranks:
            rk["d_norm_w"], rk["d_b_down"] = rk["d_norm_w_local"], rk["d_b_down_local"]
    # update: each rank's channel slices; the replicated tensors with the rank's gradient
    for rk, lp in zip(ranks, locs):
        g = dict(rk["grads"])
        g["norm_w"], g["b_down"] = rk["d_norm_w"], rk["d_b_down"]
        rk["new_params"] = _sgd(lp, g, lr, R)
        rk["params"] = lp
    return dict(ranks=ranks, out=out, loss=loss, dx=dx, n=n_full, slices=sl)
