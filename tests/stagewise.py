"""Stage-wise parity: each kernel of the step against the oracle's stage fed
the GPU's own stored inputs.

An end-to-end comparison of a bf16 step mixes two effects: the error of the
kernel that produced a tensor, and rounding flips upstream (a stored bf16
value whose exact form lies next to a rounding midpoint is rounded one way by
the GPU's fp32 accumulation and the other by the fp64 oracle; the flip then
travels, amplified by SiLU's slope, through every later stage).  At the full
workload sizes a correct fp32-accumulating implementation is up to 1.9e-2 from
the fp64 oracle end to end on the activation, dN and dx (measured with the
oracle itself run in fp32 arithmetic), which leaves no margin under the bf16
bound.  Here every stage's oracle reference is computed in fp64 from exactly
the tensors the GPU stored before it, so each check measures one kernel's own
error (a few fp32 roundings plus at most one bf16 rounding of its output)
against the same 2e-2 floored bound, element by element over whole tensors.

Stages (the steps of one training step of "Megatron tensor-parallel MLP",
synapticradio.com, split at the two tensor-parallel boundaries):
  F1  RMSNorm forward                 x                      -> normed, rstd
  F2  gate/up GEMM + activation       normed                 -> pre, act      (per shard)
  F3  down GEMM                       act                    -> z partial     (per shard; S = 1: out)
  F4  forward boundary sum            z partials, x, b_down  -> out           (S > 1)
  B1  d_act GEMM + activation bwd     out (= dY), pre        -> d_pre         (per shard)
  B2  down weight gradient            out, act               -> d_w_down      (per shard)
  B3  gate/up input gradient          d_pre                  -> dN partial    (per shard)
  B5  backward boundary sum           dN partials            -> dN            (S > 1)
  B4  gate/up weight gradient         d_pre, normed          -> d_w_in (d_b_in)
  B6  RMSNorm backward + residual     dN, x, out, rstd       -> dx, d_norm_w, d_b_down
  U1  SGD                             every gradient         -> new parameters (masters)
Large tensors are processed in blocks of token rows; each element's
reference is the same dot product or elementwise formula either way, and the
floored error's floor for [T, .] tensors is the row's own RMS.
"""

from __future__ import annotations

import numpy as np
import torch

import oracle
from tolerance import BF16_RTOL, FP32_ATOL

STAGES = ("F1", "F2", "F3", "F4", "B1", "B2", "B3", "B5", "B4", "B6", "U1")
ROWS = 4096  # token rows per block


def collect(st) -> dict:
    """Host copies of every tensor a ShardedStep stored (bf16 stays bf16)."""
    st.materialize_dN()
    c = lambda t: None if t is None else t.detach().cpu()
    h = {"normed": c(st.normed), "rstd": c(st.rstd), "out": c(st.out), "dN": c(st.dN), "dx": c(st.dx),
         "d_norm_w": c(st.d_norm_w), "d_b_down": c(st.d_b_down), "shards": [],
         "new": {k: c(v) for k, v in st.new.items()},
         "new_masters": {k: c(v) for k, v in st.new_masters.items()},
         "masters": {k: c(v) for k, v in (st.masters or {}).items()}}
    for sh in st.shards:
        h["shards"].append({k: c(sh[k]) for k in ("pre", "act", "z", "d_pre", "d_w_in", "d_b_in", "d_w_down",
                                                 "dN_part", "w_in", "w_down", "b_in")})
    return h


def _f64(t):
    return None if t is None else t.detach().double().numpy()


def _blocks(T):
    return [(lo, min(T, lo + ROWS)) for lo in range(0, T, ROWS)] or [(0, 0)]


class Checker:
    """Accumulates the worst error of each named tensor over blocks and
    asserts the bound of the workload's dtype once a tensor is complete."""

    def __init__(self, w, report: dict):
        self.bf16 = w.dtype == "bf16"
        self.report = report

    def rows(self, name, got, ref):
        """Part of a [T, .] tensor: the floor is each row's RMS."""
        g, r = np.asarray(got, dtype=np.float64), np.asarray(ref, dtype=np.float64)
        assert g.shape == r.shape, (name, g.shape, r.shape)
        if g.size == 0:
            e = 0.0
        elif self.bf16:
            rho = np.sqrt(np.mean(r * r, axis=-1, keepdims=True))
            den = np.maximum(np.abs(r), rho)
            e = float(np.max(np.abs(g - r) / np.where(den > 0, den, 1.0)))
        else:
            e = float(np.max(np.abs(g - r)) / max(1.0, float(np.sqrt(np.mean(r * r)))))
        self.report[name] = max(self.report.get(name, 0.0), e)

    def whole(self, name, got, ref):
        """A parameter-shaped tensor: the floor is the tensor's RMS."""
        g, r = np.asarray(got, dtype=np.float64), np.asarray(ref, dtype=np.float64)
        assert g.shape == r.shape, (name, g.shape, r.shape)
        if g.size == 0:
            e = 0.0
        else:
            rho = float(np.sqrt(np.mean(r * r)))
            if self.bf16:
                den = np.maximum(np.abs(r), rho)
                e = float(np.max(np.abs(g - r) / np.where(den > 0, den, 1.0)))
            else:
                e = float(np.max(np.abs(g - r))) / max(1.0, rho)
        self.report[name] = max(self.report.get(name, 0.0), e)

    def verify(self):
        bound = BF16_RTOL if self.bf16 else FP32_ATOL
        bad = {k: v for k, v in self.report.items() if not v <= bound}
        assert not bad, f"above {bound}: " + ", ".join(f"{k} {v:.3e}" for k, v in sorted(bad.items()))


def _shard_weights(w, t, s):
    """fp64 copies of shard s's expansion weight as [P, H] (SwiGLU rows gate then up),
    its fc1 bias (GeLU) and its down columns [H, F]."""
    F = w.ffn_local
    lo, hi = s * F, (s + 1) * F
    if w.act == "swiglu":
        win = np.concatenate([_f64(t["w_in"][0, lo:hi, :]), _f64(t["w_in"][1, lo:hi, :])], axis=0)
        bin_ = None
    else:
        win = _f64(t["w_in"][lo:hi, :])
        bin_ = _f64(t["b_in"][lo:hi])
    return win, bin_, _f64(t["w_down"][:, lo:hi])


def _split(w, pre):
    """[rows, P] pre-activation (or its gradient) -> the oracle's tuple (g, u) or (h,)."""
    if w.act == "swiglu":
        F = pre.shape[1] // 2
        return pre[:, :F], pre[:, F:]
    return (pre,)


def run_stage(stage: str, w, t, h: dict, report: dict) -> None:
    """Check one stage (see the module docstring) of a step whose host
    tensors are ``h`` (collect) on inputs ``t`` (synth.draw)."""
    ck = Checker(w, report)
    R = oracle.storage_rounding("bf16" if w.dtype == "bf16" else "exact")
    T, S = w.tokens, w.n_run
    fused = w.shards == 1
    norm_w, b_down = _f64(t["norm_w"]), _f64(t["b_down"])
    blocks = _blocks(T)
    x = lambda lo, hi: _f64(t["x"][lo:hi])
    if stage == "F1":
        for lo, hi in blocks:
            n, r = oracle.rms_norm_fwd(x(lo, hi), norm_w, w.eps)
            ck.rows("normed", _f64(h["normed"][lo:hi]), R(n))
        _, r = oracle.rms_norm_fwd(_f64(t["x"]), norm_w, w.eps)
        ck.whole("rstd", _f64(h["rstd"]), r)
    elif stage == "F2":
        for s in range(S):
            win, bin_, _ = _shard_weights(w, t, s)
            sh = h["shards"][s]
            for lo, hi in blocks:
                pre = _f64(h["normed"][lo:hi]) @ win.T
                if bin_ is not None:
                    pre = pre + bin_[None, :]
                ck.rows(f"pre[{s}]", _f64(sh["pre"][lo:hi]), R(pre))
                ck.rows(f"act[{s}]", _f64(sh["act"][lo:hi]),
                        oracle.activation_fwd(_split(w, _f64(sh["pre"][lo:hi])), w.act, R))
    elif stage == "F3":
        for s in range(S):
            _, _, wd = _shard_weights(w, t, s)
            sh = h["shards"][s]
            for lo, hi in blocks:
                z = _f64(sh["act"][lo:hi]) @ wd.T
                if fused:
                    ck.rows("out (fused F3+F4)", _f64(h["out"][lo:hi]), R(x(lo, hi) + z + b_down[None, :]))
                else:
                    ck.rows(f"z[{s}]", _f64(sh["z"][lo:hi]), z)
    elif stage == "F4":
        if fused:
            return  # S = 1: the down GEMM's epilogue wrote out (checked in F3)
        for lo, hi in blocks:
            zsum = sum(_f64(h["shards"][s]["z"][lo:hi]) for s in range(S))
            ck.rows("out", _f64(h["out"][lo:hi]), R(x(lo, hi) + zsum + b_down[None, :]))
    elif stage == "B1":
        for s in range(S):
            _, _, wd = _shard_weights(w, t, s)
            sh = h["shards"][s]
            for lo, hi in blocks:
                da = _f64(h["out"][lo:hi]) @ wd
                ref = oracle.activation_bwd(da, _split(w, _f64(sh["pre"][lo:hi])), w.act, R)
                ck.rows(f"d_pre[{s}]", _f64(sh["d_pre"][lo:hi]), np.concatenate(ref, axis=1))
    elif stage == "B2":
        for s in range(S):
            sh = h["shards"][s]
            ref = sum(_f64(h["out"][lo:hi]).T @ _f64(sh["act"][lo:hi]) for lo, hi in blocks)
            ck.whole(f"d_w_down[{s}]", _f64(sh["d_w_down"]), ref)
    elif stage == "B3":
        for s in range(S):
            win, _, _ = _shard_weights(w, t, s)
            sh = h["shards"][s]
            for lo, hi in blocks:
                ck.rows(f"dN_part[{s}]", _f64(sh["dN_part"][lo:hi]), _f64(sh["d_pre"][lo:hi]) @ win)
    elif stage == "B5":
        if fused:
            return  # S = 1: dN is the single partial (checked in B3)
        for lo, hi in blocks:
            ck.rows("dN", _f64(h["dN"][lo:hi]), sum(_f64(h["shards"][s]["dN_part"][lo:hi]) for s in range(S)))
    elif stage == "B4":
        for s in range(S):
            sh = h["shards"][s]
            ref = sum(_f64(sh["d_pre"][lo:hi]).T @ _f64(h["normed"][lo:hi]) for lo, hi in blocks)
            ck.whole(f"d_w_in[{s}]", _f64(sh["d_w_in"]).reshape(ref.shape), ref)
            if w.act == "gelu":
                db = sum(np.sum(_f64(sh["d_pre"][lo:hi]), axis=0) for lo, hi in blocks)
                ck.whole(f"d_b_in[{s}]", _f64(sh["d_b_in"]), db)
    elif stage == "B6":
        rstd = _f64(h["rstd"])
        dw = np.zeros(w.hidden)
        db = np.zeros(w.hidden)
        for lo, hi in blocks:
            dY = _f64(h["out"][lo:hi])
            dxn, dwb = oracle.rms_norm_bwd(_f64(h["dN"][lo:hi]), x(lo, hi), rstd[lo:hi], norm_w)
            ck.rows("dx", _f64(h["dx"][lo:hi]), R(dY + dxn))
            dw += dwb
            db += np.sum(dY, axis=0)
        ck.whole("d_norm_w", _f64(h["d_norm_w"]), dw)
        ck.whole("d_b_down", _f64(h["d_b_down"]), db)
    elif stage == "U1":
        lr = w.lr
        grads = {"norm_w": h["d_norm_w"], "b_down": h["d_b_down"]}
        params = {"norm_w": t["norm_w"], "b_down": t["b_down"]}
        F = w.ffn_local
        for s in range(S):
            sh = h["shards"][s]
            lo, hi = s * F, (s + 1) * F
            grads[f"w_in.{s}"] = sh["d_w_in"]
            params[f"w_in.{s}"] = t["w_in"][:, lo:hi, :] if w.act == "swiglu" else t["w_in"][lo:hi, :]
            grads[f"w_down.{s}"] = sh["d_w_down"]
            params[f"w_down.{s}"] = t["w_down"][:, lo:hi]
            if w.act == "gelu":
                grads[f"b_in.{s}"] = sh["d_b_in"]
                params[f"b_in.{s}"] = t["b_in"][lo:hi]
        for k, g in grads.items():
            g = _f64(g)
            p = _f64(params[k]).reshape(g.shape)
            if w.master:
                m = _f64(h["masters"][k]).reshape(g.shape)
                np.testing.assert_array_equal(m, p)  # masters start as the exact upcasts
                ck.whole(f"master.{k}", _f64(h["new_masters"][k]).reshape(g.shape), m - lr * g)
                # the stored parameter is the rounding of the GPU's own new master
                ck.whole(f"new.{k}", _f64(h["new"][k]).reshape(g.shape), R(_f64(h["new_masters"][k]).reshape(g.shape)))
            else:
                ck.whole(f"new.{k}", _f64(h["new"][k]).reshape(g.shape), R(p - lr * g))
    else:
        raise ValueError(stage)
    ck.verify()
