"""FP8 GEMMs with per-tensor delayed scaling for the MLP sublayer's step.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Sources:

* "Megatron-Core Guide: 5D Distributed Training Architecture": Transformer
  Engine runs the matrix products in FP8 with delayed scaling (its feature list,
  item 6) and this is where the doubled matrix throughput comes from (the
  "Memory Engine" layer of its architecture figure).
* "Megatron-LM walkthrough" (stanleyjacob.dev), Part III: Transformer Engine
  kernels and FP8 supply the last few percent of utilisation.

The pages name the method and nothing more: neither the formats, nor the
scaling rule, nor which tensors are cast.  The readings taken here are those
of Transformer Engine's default recipe, the plainest reading of "FP8 with
delayed scaling through Transformer Engine":

* Formats (OCP FP8): forward tensors (the normed input N, the weights, the
  activation A) in E4M3 -- 4 exponent bits with bias 7, 3 mantissa bits,
  subnormals, no infinities, largest finite value 448; backward gradients (the
  output gradient dY and the pre-activation gradient dP) in E5M2 -- 5 exponent
  bits with bias 15, 2 mantissa bits, subnormals, largest finite 57344.
* Encoding: round to nearest, ties to even, after clamping to +-max.  The
  encoded value is round(clamp(fp32(x) * fp32(s))): the product is formed in
  fp32, so both sides take each rounding decision on the same number.
* Per-tensor delayed scaling: a tensor's meta holds its scale s (initially 1),
  the running amax of this step and a history of the last L amaxes (newest
  first).  Every cast during a step uses the current s and folds max|x| into
  the running amax (NaN elements have no magnitude and are ignored).  At the end of the step the running amax enters the
  history (the oldest entry drops out), the running amax returns to 0, and
  s becomes fmt_max / max(history) in fp32 when that maximum is positive and
  finite; otherwise s keeps its value (so an all-zero history keeps s = 1).
* A product of two cast tensors is dequantised by the fp32 product of their
  fp32 inverse scales, 1/s_a * 1/s_b.
* Every GEMM of the step runs in FP8: the forward F2 (N W_in^T) and F3
  (A W_down^T); the backward d_act = dY W_down, dW_down = dY^T A,
  dN = dP W_in and dW_in = dP^T N, each on the codes of its operands (a
  transposed operand is the transpose of the same codes, with the same scale).
  Everything between the GEMMs -- the norm, the activation and its backward,
  the residual and bias, the sums over shards, the update -- is the bf16 step
  of oracle.mlp on the tensors this step produces.
* Tensor-parallel shards share one meta per tensor role, so the amax is the
  maximum over the group (the amax reduction over the tensor-parallel group):
  every shard casts with the same scale, and the sharded step equals the
  dense step up to the order of the sums.
"""

from __future__ import annotations

import dataclasses
from typing import Dict, List

import numpy as np

from .mlp import (Params, _ordered_sum, _sgd, _shard_params, gelu, gelu_grad, rms_norm_bwd, rms_norm_fwd, silu,
                  silu_grad, storage_rounding)


@dataclasses.dataclass(frozen=True)
class Fp8Format:
    name: str
    exp_bits: int
    mant_bits: int
    bias: int
    max: float

    @property
    def min_normal_exp(self) -> int:
        return 1 - self.bias

    @property
    def sub_step(self) -> float:
        """Spacing of the subnormal values, 2^(1 - bias - mant_bits)."""
        return 2.0 ** (1 - self.bias - self.mant_bits)


E4M3 = Fp8Format("e4m3", 4, 3, 7, 448.0)
E5M2 = Fp8Format("e5m2", 5, 2, 15, 57344.0)
FORMATS = {"e4m3": E4M3, "e5m2": E5M2}


def encode(y, fmt: Fp8Format) -> np.ndarray:
    """Codes (uint8) of finite values y with |y| <= fmt.max: the nearest
    representable value, ties to the even mantissa."""
    y = np.asarray(y, dtype=np.float64)
    if not np.all(np.isfinite(y)) or np.any(np.abs(y) > fmt.max):
        raise ValueError(f"encode takes finite values within +-{fmt.max}")
    a = np.abs(y)
    _, e2 = np.frexp(a)
    e = e2.astype(np.int64) - 1                        # floor(log2 a) for a > 0
    normal = (a > 0) & (e >= fmt.min_normal_exp)
    # subnormal range: a whole number of sub_steps (a round-up to 2^mant_bits steps is the smallest normal's code)
    sub = np.rint(a / fmt.sub_step).astype(np.int64)
    # normal range: the mantissa fraction in units of 2^-mant_bits, a carry moves to the next binade
    ee = np.where(normal, e, 0)
    m = np.rint((a / np.ldexp(1.0, ee) - 1.0) * (1 << fmt.mant_bits)).astype(np.int64)
    carry = normal & (m == (1 << fmt.mant_bits))
    ee = np.where(carry, ee + 1, ee)
    m = np.where(carry, 0, m)
    norm_code = ((ee + fmt.bias) << fmt.mant_bits) | m
    mag = np.where(normal, norm_code, sub)
    return (mag | (np.signbit(y).astype(np.int64) << 7)).astype(np.uint8)


def decode(codes, fmt: Fp8Format) -> np.ndarray:
    """Values (float64) of codes; NaN and infinity codes decode to NaN / inf."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    emask = (1 << fmt.exp_bits) - 1
    ex = (c >> fmt.mant_bits) & emask
    mant = c & ((1 << fmt.mant_bits) - 1)
    val = np.where(ex == 0, mant * fmt.sub_step,
                   (1.0 + mant / float(1 << fmt.mant_bits)) * np.ldexp(1.0, ex - fmt.bias))
    if fmt.name == "e4m3":
        val = np.where((ex == emask) & (mant == 7), np.nan, val)       # no infinities; S.1111.111 is NaN
    else:
        val = np.where(ex == emask, np.where(mant == 0, np.inf, np.nan), val)
    return sign * val


def quantize(x, scale, fmt: Fp8Format) -> np.ndarray:
    """Codes of x under `scale`: encode(clamp(fp32(x) * fp32(scale)))."""
    y = np.asarray(x, dtype=np.float32) * np.float32(scale)
    return encode(np.clip(y.astype(np.float64), -fmt.max, fmt.max), fmt)


@dataclasses.dataclass
class Fp8Meta:
    """Delayed-scaling state of one tensor role."""

    fmt: Fp8Format
    history: np.ndarray                    # [L] float32, newest first
    scale: np.float32 = np.float32(1.0)
    amax: np.float32 = np.float32(0.0)     # running max|x| of the casts of this step

    @staticmethod
    def new(fmt: Fp8Format, history_len: int) -> "Fp8Meta":
        if history_len < 1:
            raise ValueError("history_len must be >= 1")
        return Fp8Meta(fmt, np.zeros(history_len, dtype=np.float32))

    def copy(self) -> "Fp8Meta":
        return Fp8Meta(self.fmt, self.history.copy(), np.float32(self.scale), np.float32(self.amax))

    def scale_inv(self) -> np.float32:
        return np.float32(1.0 / float(self.scale))

    def record(self, x) -> None:
        """Fold max|x| into the running amax; NaN elements are ignored (an
        amax is a maximum of magnitudes, and a NaN has none)."""
        a = np.abs(np.asarray(x, dtype=np.float32))
        a = a[~np.isnan(a)]
        if a.size:
            self.amax = np.float32(max(float(self.amax), float(np.max(a))))

    def update(self) -> None:
        """End of step: the running amax enters the history; a new scale."""
        self.history = np.concatenate([[self.amax], self.history[:-1]]).astype(np.float32)
        self.amax = np.float32(0.0)
        m = float(np.max(self.history))
        if 0.0 < m < np.inf:
            self.scale = np.float32(self.fmt.max / m)


def cast(x, meta: Fp8Meta) -> np.ndarray:
    """Codes of x with the meta's current scale; x's amax is recorded."""
    codes = quantize(x, meta.scale, meta.fmt)
    meta.record(x)
    return codes


def fp8_gemm_nt(a_codes, a_meta: Fp8Meta, b_codes, b_meta: Fp8Meta) -> np.ndarray:
    """C[m, n] = (sum_k dec(A)[m, k] dec(B)[n, k]) * fp32(1/s_a * 1/s_b):
    exact products and fp64 sums of the decoded codes, then the dequantisation."""
    deq = float(np.float32(a_meta.scale_inv()) * np.float32(b_meta.scale_inv()))
    return (decode(a_codes, a_meta.fmt) @ decode(b_codes, b_meta.fmt).T) * deq


# tensor roles and their formats (E4M3 forward, E5M2 gradients)
ROLES = {"normed": E4M3, "w_in": E4M3, "act": E4M3, "w_down": E4M3, "d_out": E5M2, "d_pre": E5M2}


def new_metas(history_len: int = 16) -> Dict[str, Fp8Meta]:
    return {k: Fp8Meta.new(f, history_len) for k, f in ROLES.items()}


def copy_metas(metas: Dict[str, Fp8Meta]) -> Dict[str, Fp8Meta]:
    return {k: m.copy() for k, m in metas.items()}


def _w_in_rows(w_in, act):
    """The expansion weight as the rows of one [P, H] matrix (SwiGLU: the
    gate channels, then the up channels)."""
    return w_in.reshape(-1, w_in.shape[-1]) if act == "swiglu" else w_in


def _expansion_fwd_fp8(nq, p: Params, act, metas, R):
    """F2 on the codes of N and of W_in, then the activation on the stored
    pre-activations; returns (pre, a, w_in codes)."""
    F = p.w_down.shape[1]
    wq = cast(_w_in_rows(p.w_in, act), metas["w_in"])
    h = fp8_gemm_nt(nq, metas["normed"], wq, metas["w_in"])
    if act == "swiglu":
        g, u = R(h[:, :F]), R(h[:, F:])
        return (g, u), R(silu(g) * u), wq
    pre = R(h + p.b_in[None, :])
    return (pre,), R(gelu(pre)), wq


def _act_bwd(da, pre, act, R):
    """Activation backward on the stored pre-activations: dP = [dg | du] or dh."""
    if act == "swiglu":
        g, u = pre
        return np.concatenate([R(da * u * silu_grad(g)), R(da * silu(g))], axis=1)
    (h,) = pre
    return R(da * gelu_grad(h))


def fp8_dense_step(x, p: Params, act: str, eps: float, lr: float, metas: Dict[str, Fp8Meta],
                   storage: str = "bf16") -> dict:
    """One training step of the dense block with every GEMM in FP8 (metas
    updated in place at the end).  Stored tensors are rounded per `storage`
    as in oracle.dense_step; SGD as there."""
    R = storage_rounding(storage)
    x = np.asarray(x, dtype=np.float64)
    p = p.astype(np.float64)
    n, r = rms_norm_fwd(x, p.norm_w, eps)
    n = R(n)
    nq = cast(n, metas["normed"])
    pre, a, wq = _expansion_fwd_fp8(nq, p, act, metas, R)
    aq = cast(a, metas["act"])
    wdq = cast(p.w_down, metas["w_down"])
    z = fp8_gemm_nt(aq, metas["act"], wdq, metas["w_down"])
    out = R(x + z + p.b_down[None, :])
    loss = 0.5 * float(np.sum(out * out))

    dY = out
    dyq = cast(dY, metas["d_out"])
    g = {"b_down": np.sum(dY, axis=0)}
    da = fp8_gemm_nt(dyq, metas["d_out"], wdq.T, metas["w_down"])                 # dY W_down
    g["w_down"] = fp8_gemm_nt(dyq.T, metas["d_out"], aq.T, metas["act"])          # dY^T A
    dP = _act_bwd(da, pre, act, R)
    dpq = cast(dP, metas["d_pre"])
    dN = fp8_gemm_nt(dpq, metas["d_pre"], wq.T, metas["w_in"])                    # dP W_in
    d_w_in = fp8_gemm_nt(dpq.T, metas["d_pre"], nq.T, metas["normed"])            # dP^T N
    g["w_in"] = d_w_in.reshape(p.w_in.shape)
    g["b_in"] = np.sum(dP, axis=0) if act == "gelu" else None
    dxn, g["norm_w"] = rms_norm_bwd(dN, x, r, p.norm_w)
    dx = R(dY + dxn)
    scale_inv = {k: m.scale_inv() for k, m in metas.items()}
    codes = dict(normed=nq, w_in=wq, act=aq, w_down=wdq, d_out=dyq, d_pre=dpq)
    for m in metas.values():
        m.update()
    return dict(x=x, n=n, rstd=r, pre=pre, a=a, z=z, out=out, loss=loss, dY=dY, da=da, dP=dP, dN=dN, dx=dx,
                grads=g, params=p, new_params=_sgd(p, g, lr, R), codes=codes, scale_inv=scale_inv)


def fp8_sharded_step(x, p: Params, act: str, eps: float, lr: float, shards: int, metas: Dict[str, Fp8Meta],
                     storage: str = "bf16") -> dict:
    """The same step as S tensor-parallel shards (FFN channels split as in
    oracle.sharded_step), the metas shared by the shards; the forward and
    backward partials are summed in shard order."""
    R = storage_rounding(storage)
    x = np.asarray(x, dtype=np.float64)
    p = p.astype(np.float64)
    locs = [_shard_params(p, s, shards, act) for s in range(shards)]
    n, r = rms_norm_fwd(x, p.norm_w, eps)
    n = R(n)
    ranks: List[dict] = [dict() for _ in range(shards)]
    for rk, lp in zip(ranks, locs):
        rk["nq"] = cast(n, metas["normed"])   # every rank casts its copy of N
        rk["pre"], rk["a"], rk["wq"] = _expansion_fwd_fp8(rk["nq"], lp, act, metas, R)
        rk["aq"] = cast(rk["a"], metas["act"])
        rk["wdq"] = cast(lp.w_down, metas["w_down"])
        rk["z"] = fp8_gemm_nt(rk["aq"], metas["act"], rk["wdq"], metas["w_down"])
    out = R(x + _ordered_sum([rk["z"] for rk in ranks]) + p.b_down[None, :])
    dY = out
    for rk, lp in zip(ranks, locs):
        dyq = cast(dY, metas["d_out"])
        da = fp8_gemm_nt(dyq, metas["d_out"], rk["wdq"].T, metas["w_down"])
        gr = {"w_down": fp8_gemm_nt(dyq.T, metas["d_out"], rk["aq"].T, metas["act"])}
        dP = _act_bwd(da, rk["pre"], act, R)
        dpq = cast(dP, metas["d_pre"])
        rk["dN_part"] = fp8_gemm_nt(dpq, metas["d_pre"], rk["wq"].T, metas["w_in"])
        gr["w_in"] = fp8_gemm_nt(dpq.T, metas["d_pre"], rk["nq"].T, metas["normed"]).reshape(lp.w_in.shape)
        gr["b_in"] = np.sum(dP, axis=0) if act == "gelu" else None
        rk["grads"], rk["dP"] = gr, dP
    dN = _ordered_sum([rk["dN_part"] for rk in ranks])
    dxn, d_norm_w = rms_norm_bwd(dN, x, r, p.norm_w)
    dx = R(dY + dxn)
    d_b_down = np.sum(dY, axis=0)
    for rk, lp in zip(ranks, locs):
        gr = dict(rk["grads"], norm_w=d_norm_w, b_down=d_b_down)
        rk["new_params"] = _sgd(lp, gr, lr, R)
    for m in metas.values():
        m.update()
    return dict(out=out, dx=dx, dN=dN, n=n, rstd=r, d_norm_w=d_norm_w, d_b_down=d_b_down, ranks=ranks)


def product_error_bound(a, b, sa, sb, fa: Fp8Format, fb: Fp8Format) -> np.ndarray:
    """Bound on |C_fp8 - A B^T| elementwise for A, B cast with scales sa, sb:
    a cast value differs from x by at most (2^-(mant_bits+1) + 2^-23) |x|
    (the fp8 rounding of the fp32 product x s, itself rounded) in the normal
    range, sub_step / 2 / s in the subnormal range, plus |x| - max / s where
    the cast saturates, so each product term is off by at most e_a (|b| + e_b) + |a| e_b,
    summed over k; the fp32 inverse scales and their product add a relative
    2^-21 of the perturbed terms on top."""
    ea = (np.abs(a) * (2.0 ** -(fa.mant_bits + 1) + 2.0 ** -23) + fa.sub_step / 2 / float(sa)
          + np.maximum(0.0, np.abs(a) - fa.max / float(sa)))
    eb = (np.abs(b) * (2.0 ** -(fb.mant_bits + 1) + 2.0 ** -23) + fb.sub_step / 2 / float(sb)
          + np.maximum(0.0, np.abs(b) - fb.max / float(sb)))
    bound = ea @ (np.abs(b) + eb).T + np.abs(a) @ eb.T
    return bound + 2.0 ** -21 * ((np.abs(a) + ea) @ (np.abs(b) + eb).T)


def _cast_rows(x, meta: Fp8Meta, chunk: int = 1024) -> np.ndarray:
    """cast() of a large [rows, cols] matrix, a block of rows at a time (the
    same codes and amax; bounded temporaries)."""
    x = np.asarray(x)
    codes = np.empty(x.shape, dtype=np.uint8)
    for lo in range(0, x.shape[0], chunk):
        codes[lo:lo + chunk] = cast(x[lo:lo + chunk], meta)
    return codes


def fp8_sampled_step(x, p: Params, act: str, eps: float, lr: float, metas: Dict[str, Fp8Meta], rows, chans, cols,
                     dtype=np.float32, storage: str = "bf16") -> dict:
    """Selected entries of fp8_dense_step at full workload size (metas updated
    in place).  The whole forward, the output gradient and the pre-activation
    gradient are computed on the codes; then only sampled token rows (dN, dx),
    FFN channels (the weight-gradient slices of those channels, the
    activation) and hidden columns (the norm-weight gradient, which needs a
    column of dN over all tokens), as oracle.sampled_step does for the bf16
    step.  Products of decoded codes are summed in `dtype`; tests pin this
    function to fp8_dense_step entry by entry on small shapes (in float64)."""
    R = storage_rounding(storage)
    rows, chans, cols = (np.asarray(v, dtype=np.int64) for v in (rows, chans, cols))
    x = np.asarray(x, dtype=dtype)
    p = p.astype(dtype)
    dec = lambda c, m: decode(c, m.fmt).astype(dtype)
    deq = lambda ma, mb: dtype(np.float32(ma.scale_inv()) * np.float32(mb.scale_inv()))
    F = p.w_down.shape[1]
    n, r = rms_norm_fwd(x, p.norm_w, eps)
    n = R(n.astype(dtype)).astype(dtype)
    nq = _cast_rows(n, metas["normed"])
    wrows = _w_in_rows(p.w_in, act)
    wq = _cast_rows(wrows, metas["w_in"])
    Wq = dec(wq, metas["w_in"])                                   # [P, H]
    h = (dec(nq, metas["normed"]) @ Wq.T) * deq(metas["normed"], metas["w_in"])
    if act == "swiglu":
        g, u = R(h[:, :F]).astype(dtype), R(h[:, F:]).astype(dtype)
        a = R(silu(g) * u).astype(dtype)
        pre = (g, u)
    else:
        hh = R(h + p.b_in[None, :]).astype(dtype)
        a = R(gelu(hh)).astype(dtype)
        pre = (hh,)
    del h
    aq = _cast_rows(a, metas["act"])
    wdq = _cast_rows(p.w_down, metas["w_down"])
    Wd = dec(wdq, metas["w_down"])                                # [H, F]
    Aq = dec(aq, metas["act"])
    out = R(x + (Aq @ Wd.T) * deq(metas["act"], metas["w_down"]) + p.b_down[None, :]).astype(dtype)
    res = {"out": out, "act_chans": a[:, chans]}
    dY = out
    res["d_b_down"] = np.sum(dY, axis=0, dtype=np.float64)
    dyq = _cast_rows(dY, metas["d_out"])
    DY = dec(dyq, metas["d_out"])
    da = (DY @ Wd) * deq(metas["d_out"], metas["w_down"])
    dP = _act_bwd(da, pre, act, lambda v: R(np.asarray(v, dtype=dtype)).astype(dtype))
    del da, pre
    if act == "gelu":
        res["d_b_in"] = np.sum(dP, axis=0, dtype=np.float64)
    dpq = _cast_rows(dP, metas["d_pre"])
    DP = dec(dpq, metas["d_pre"])
    k_in = deq(metas["d_pre"], metas["w_in"])
    # row-local quantities
    res["dN_rows"] = (DP[rows] @ Wq) * k_in
    dxn, _ = rms_norm_bwd(res["dN_rows"], x[rows], r[rows], p.norm_w)
    res["dx_rows"] = R(dY[rows] + dxn)
    # channel-sampled weight gradients (SwiGLU: the gate and the up row of each channel)
    res["d_w_down_chans"] = (DY.T @ Aq[:, chans]) * deq(metas["d_out"], metas["act"])
    sel = np.concatenate([chans, F + chans]) if act == "swiglu" else chans
    dwin = (DP[:, sel].T @ dec(nq, metas["normed"])) * deq(metas["d_pre"], metas["normed"])
    res["d_w_in_chans"] = dwin.reshape(2, len(chans), -1) if act == "swiglu" else dwin
    # column-sampled norm-weight gradient: dN[:, cols] over all tokens
    dN_cols = (DP @ Wq[:, cols]) * k_in
    res["d_norm_w_cols"] = np.sum(dN_cols * x[:, cols] * r[:, None], axis=0)
    # SGD on the sampled entries
    res["new_norm_w_cols"] = R(p.norm_w[cols] - lr * res["d_norm_w_cols"])
    res["new_b_down"] = R(p.b_down - lr * res["d_b_down"])
    res["new_w_down_chans"] = R(p.w_down[:, chans] - lr * res["d_w_down_chans"])
    if act == "swiglu":
        res["new_w_in_chans"] = R(p.w_in[:, chans, :] - lr * res["d_w_in_chans"])
    else:
        res["new_w_in_chans"] = R(p.w_in[chans, :] - lr * res["d_w_in_chans"])
        res["new_b_in"] = R(p.b_in - lr * res["d_b_in"])
    for m in metas.values():
        m.update()
    return res
