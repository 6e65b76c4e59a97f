"""Selected entries of the dense step at full workload size.

TEST INFRASTRUCTURE ONLY (see the package docstring).

``dense_step`` at the largest workloads needs 18 T H F flops and many
[T, F] temporaries.  The entries checked at full size need less: the whole
forward and the gradient of the activation (8 T H F) are computed, and then
only sampled token rows (row-local quantities: dN, dx), sampled FFN channels
(weight-gradient rows/columns of those channels) and sampled hidden columns
(the norm-weight gradient, which needs a column of dN over all tokens).  The
arithmetic is the same definition as ``dense_step``; ``tests`` pin this
function to ``dense_step`` entry by entry on small shapes.
"""

from __future__ import annotations

import numpy as np

from .mlp import Params, expansion_fwd, gelu_grad, rms_norm_bwd, rms_norm_fwd, silu, silu_grad, storage_rounding


def sampled_step(x, p: Params, act: str, eps: float, lr: float, rows, chans, cols, dtype=np.float32,
                 storage: str = "exact") -> dict:
    """Returns out [T,H] (full), loss, d_b_down [H], d_b_in [F] (GeLU),
    and at the samples: dN[rows], dx[rows], d_w_down[:, chans],
    d_w_in[(planes,) chans, :], d_norm_w[cols], act[:, chans], plus the
    post-SGD values of those parameter entries (new_*)."""
    R = storage_rounding(storage)
    rows, chans, cols = (np.asarray(v, dtype=np.int64) for v in (rows, chans, cols))
    x = np.asarray(x, dtype=dtype)
    p = p.astype(dtype)
    n, r = rms_norm_fwd(x, p.norm_w, eps)
    n = R(n.astype(dtype))
    pre, a = expansion_fwd(n, p, act, lambda v: R(np.asarray(v, dtype=dtype)))
    out = R((x + a @ p.w_down.T + p.b_down[None, :]).astype(dtype))
    res = {"out": out, "loss": 0.5 * np.sum(out.astype(np.float64) ** 2)}
    dY = out
    res["d_b_down"] = np.sum(dY, axis=0)
    da = dY @ p.w_down
    if act == "swiglu":
        g, u = pre
        dpre = (R((da * u * silu_grad(g)).astype(dtype)), R((da * silu(g)).astype(dtype)))
        wins = (p.w_in[0], p.w_in[1])
        del g, u
    else:
        (h,) = pre
        dpre = (R((da * gelu_grad(h)).astype(dtype)),)
        wins = (p.w_in,)
        res["d_b_in"] = np.sum(dpre[0], axis=0)
        del h
    del da, pre
    # row-local quantities
    dN_rows = sum(dp[rows] @ wi for dp, wi in zip(dpre, wins))
    dxn, _ = rms_norm_bwd(dN_rows, x[rows], r[rows], p.norm_w)
    res["dN_rows"] = dN_rows
    res["dx_rows"] = R(dY[rows] + dxn)
    # channel-sampled weight gradients
    res["act_chans"] = a[:, chans]
    res["d_w_down_chans"] = dY.T @ a[:, chans]                      # [H, C]
    dwin = [dp[:, chans].T @ n for dp in dpre]                       # each [C, H]
    res["d_w_in_chans"] = np.stack(dwin) if act == "swiglu" else dwin[0]
    # column-sampled norm-weight gradient: needs dN[:, cols] over all tokens
    dN_cols = sum(dp @ wi[:, cols] for dp, wi in zip(dpre, wins))   # [T, Ccols]
    res["d_norm_w_cols"] = np.sum(dN_cols * x[:, cols] * r[:, None], axis=0)
    # SGD on the sampled entries (updated parameters in storage precision)
    res["new_norm_w_cols"] = R(p.norm_w[cols] - lr * res["d_norm_w_cols"])
    res["new_b_down"] = R(p.b_down - lr * res["d_b_down"])
    res["new_w_down_chans"] = R(p.w_down[:, chans] - lr * res["d_w_down_chans"])
    if act == "swiglu":
        res["new_w_in_chans"] = R(p.w_in[:, chans, :] - lr * res["d_w_in_chans"])
    else:
        res["new_w_in_chans"] = R(p.w_in[chans, :] - lr * res["d_w_in_chans"])
        res["new_b_in"] = R(p.b_in - lr * res["d_b_in"])
    return res
