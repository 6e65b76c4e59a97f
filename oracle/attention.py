"""The tensor-parallel attention sublayer (pre-RMSNorm, grouped-query causal
self-attention, row-parallel output projection).

TEST INFRASTRUCTURE ONLY (see the package docstring).

Sources:

* "Megatron-LM walkthrough" (stanleyjacob.dev):
  - Part IV, Stage 5: the QKV projection is column-parallel, so each
    tensor-parallel rank computes Q, K and V of its own heads with no
    communication; attention runs locally per head; the output projection is
    row-parallel and its partial sum is all-reduced (the g operator).
  - Part IV, Stage 6 and Part V, "Deep dive: tensor parallelism and the f and
    g operators": in backward the f operator all-reduces the gradient of the
    QKV projection's input; the table there gives the attention block one
    all-reduce in each direction, exactly as the MLP block.
* "Megatron tensor-parallel MLP" (synapticradio.com), closing section: the next
  reconstruction is tensor-parallel grouped-query attention that keeps
  complete query/KV head groups together.

Readings (the pages give no formula for attention itself):

* x is [b, s, H] flattened batch-major to [T, H] (T = b s): the token rows of
  one sequence are contiguous.
* N = rms_norm(x, norm_w) as for the MLP block.
* Heads: n_q query heads and n_kv key/value heads of width d, n_q a multiple
  of n_kv; query head h uses key/value head h // (n_q / n_kv).  The fused
  projection weight w_qkv has rows [Q heads | K heads | V heads], each head d
  rows: q_h = N Wq_h^T, k_g = N Wk_g^T, v_g = N Wv_g^T; no projection biases.
* Causal softmax attention with the standard 1/sqrt(d) scale and no
  positional rotation (the pages mention none):
      S_h = q_h k_g^T / sqrt(d) over the positions of one sequence,
      P_h = softmax over keys j <= i,   o_h = P_h v_g.
  O = [o_0 | ... | o_{n_q-1}]  [T, n_q d].
* out = x + O W_o^T + b_o, W_o [H, n_q d], b_o [H] added once after the
  partial sums (as b_down in the MLP block).
* Tensor-parallel split over S shards: shard r owns key/value heads
  [r n_kv/S, (r+1) n_kv/S) and the query heads of those groups, i.e. complete
  GQA groups; its W_qkv rows are those heads' rows and its W_o columns those
  query heads' columns.
* Loss 1/2 sum out^2 (dY = out) and plain SGD, as for the MLP block; stored
  tensors rounded per `storage` (N, Q, K, V, O, out, dQKV, dO, dx).
"""

from __future__ import annotations

import dataclasses
import math
from typing import List, Optional

import numpy as np

from .mlp import _ordered_sum, rms_norm_bwd, rms_norm_fwd, storage_rounding

ATTN_MODES = ("equivalence", "missing_forward_reduce", "missing_backward_reduce")


@dataclasses.dataclass(frozen=True)
class AttnShape:
    batch: int
    seq: int
    n_q: int
    n_kv: int
    d: int

    @property
    def tokens(self) -> int:
        return self.batch * self.seq

    @property
    def group(self) -> int:
        return self.n_q // self.n_kv

    @property
    def qkv_width(self) -> int:
        return (self.n_q + 2 * self.n_kv) * self.d


@dataclasses.dataclass
class AttnParams:
    """norm_w [H]; w_qkv [(n_q + 2 n_kv) d, H] (rows: Q heads, K heads, V heads);
    w_o [H, n_q d]; b_o [H]."""

    norm_w: np.ndarray
    w_qkv: np.ndarray
    w_o: np.ndarray
    b_o: np.ndarray

    def astype(self, dtype) -> "AttnParams":
        return AttnParams(*(np.asarray(v, dtype=dtype).copy() for v in (self.norm_w, self.w_qkv, self.w_o, self.b_o)))


def split_qkv(qkv, sh: AttnShape):
    """[T, (n_q + 2 n_kv) d] -> q [b, n_q, s, d], k, v [b, n_kv, s, d]."""
    b, s, d = sh.batch, sh.seq, sh.d
    q = qkv[:, :sh.n_q * d].reshape(b, s, sh.n_q, d).transpose(0, 2, 1, 3)
    k = qkv[:, sh.n_q * d:(sh.n_q + sh.n_kv) * d].reshape(b, s, sh.n_kv, d).transpose(0, 2, 1, 3)
    v = qkv[:, (sh.n_q + sh.n_kv) * d:].reshape(b, s, sh.n_kv, d).transpose(0, 2, 1, 3)
    return q, k, v


def merge_heads(o, sh: AttnShape):
    """[b, n, s, d] -> [T, n d]."""
    b, n, s, d = o.shape
    return o.transpose(0, 2, 1, 3).reshape(b * s, n * d)


def split_heads(t, n: int, sh: AttnShape):
    """[T, n d] -> [b, n, s, d]."""
    return t.reshape(sh.batch, sh.seq, n, sh.d).transpose(0, 2, 1, 3)


def causal_attention_fwd(q, k, v, group: int):
    """o_h = softmax(q_h k_g^T / sqrt(d), keys j <= i) v_g for every batch and
    query head h (g = h // group).  Returns (o, lse) with lse the log of each
    row's softmax denominator after the row maximum is added back:
    lse_i = log sum_{j<=i} exp(s_ij)."""
    b, nq, s, d = q.shape
    scale = 1.0 / math.sqrt(d)
    mask = np.tril(np.ones((s, s), dtype=bool))
    o = np.zeros_like(q)
    lse = np.zeros((b, nq, s), dtype=q.dtype)
    for h in range(nq):
        g = h // group
        sc = (q[:, h] @ k[:, g].transpose(0, 2, 1)) * scale          # [b, s, s]: s_ij = q_i . k_j / sqrt(d)
        sc = np.where(mask[None], sc, -np.inf)
        m = np.max(sc, axis=-1, keepdims=True)
        e = np.exp(sc - m)
        den = np.sum(e, axis=-1, keepdims=True)
        p = e / den
        o[:, h] = p @ v[:, g]
        lse[:, h] = (m + np.log(den))[..., 0]
    return o, lse


def causal_attention_bwd(q, k, v, o, do, group: int):
    """Gradients of causal_attention_fwd for an incoming do:
       dv_g = sum_{h in g} P_h^T do_h;  dP_h = do_h v_g^T;
       dS_h = P_h * (dP_h - rowsum(do_h * o_h));  dq_h = dS_h k_g / sqrt(d);
       dk_g = sum_{h in g} dS_h^T q_h / sqrt(d)."""
    b, nq, s, d = q.shape
    scale = 1.0 / math.sqrt(d)
    mask = np.tril(np.ones((s, s), dtype=bool))
    dq, dk, dv = np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)
    for h in range(nq):
        g = h // group
        sc = (q[:, h] @ k[:, g].transpose(0, 2, 1)) * scale
        sc = np.where(mask[None], sc, -np.inf)
        p = np.exp(sc - np.max(sc, axis=-1, keepdims=True))
        p = p / np.sum(p, axis=-1, keepdims=True)
        dv[:, g] += p.transpose(0, 2, 1) @ do[:, h]
        dp = do[:, h] @ v[:, g].transpose(0, 2, 1)
        delta = np.sum(do[:, h] * o[:, h], axis=-1, keepdims=True)
        ds = p * (dp - delta)
        dq[:, h] = (ds @ k[:, g]) * scale
        dk[:, g] += (ds.transpose(0, 2, 1) @ q[:, h]) * scale
    return dq, dk, dv


def _sgd(p: AttnParams, g: dict, lr, R) -> AttnParams:
    return AttnParams(R(p.norm_w - lr * g["norm_w"]), R(p.w_qkv - lr * g["w_qkv"]), R(p.w_o - lr * g["w_o"]),
                      R(p.b_o - lr * g["b_o"]))


def attn_dense_step(x, p: AttnParams, sh: AttnShape, eps: float, lr: float, dtype=np.float64,
                    storage: str = "exact") -> dict:
    """One dense training step of the attention sublayer (forward, backward
    with dY = out, SGD)."""
    R = storage_rounding(storage)
    x = np.asarray(x, dtype=dtype)
    p = p.astype(dtype)
    n, r = rms_norm_fwd(x, p.norm_w, eps)
    n = R(n)
    qkv = R(n @ p.w_qkv.T)
    q, k, v = split_qkv(qkv, sh)
    o4, lse = causal_attention_fwd(q, k, v, sh.group)
    O = R(merge_heads(o4, sh))
    z = O @ p.w_o.T
    out = R(x + z + p.b_o[None, :])
    dY = out
    g = {"b_o": np.sum(dY, axis=0), "w_o": dY.T @ O}
    dO = R(dY @ p.w_o)
    dq, dk, dv = causal_attention_bwd(q, k, v, split_heads(O, sh.n_q, sh), split_heads(dO, sh.n_q, sh), sh.group)
    dqkv = R(np.concatenate([merge_heads(dq, sh), merge_heads(dk, sh), merge_heads(dv, sh)], axis=1))
    g["w_qkv"] = dqkv.T @ n
    dN = dqkv @ p.w_qkv
    dxn, g["norm_w"] = rms_norm_bwd(dN, x, r, p.norm_w)
    dx = R(dY + dxn)
    return dict(x=x, n=n, rstd=r, qkv=qkv, O=O, lse=lse, z=z, out=out, loss=0.5 * float(np.sum(out * out)), dY=dY,
                dO=dO, dqkv=dqkv, dN=dN, dx=dx, grads=g, params=p, new_params=_sgd(p, g, lr, R), lr=lr)


def shard_heads(sh: AttnShape, r: int, shards: int):
    """Query heads, key/value heads of shard r (complete GQA groups)."""
    if sh.n_kv % shards:
        raise ValueError(f"{sh.n_kv} key/value heads are not divisible by {shards} shards")
    kv_per = sh.n_kv // shards
    kv = list(range(r * kv_per, (r + 1) * kv_per))
    q = [h for g in kv for h in range(g * sh.group, (g + 1) * sh.group)]
    return q, kv


def shard_rows(sh: AttnShape, r: int, shards: int):
    """Rows of w_qkv (its Q, K and V heads, in that order) and columns of w_o
    owned by shard r."""
    q, kv = shard_heads(sh, r, shards)
    d = sh.d
    rows = lambda heads, base: [base + h * d + i for h in heads for i in range(d)]
    qkv_rows = rows(q, 0) + rows(kv, sh.n_q * d) + rows(kv, (sh.n_q + sh.n_kv) * d)
    return qkv_rows, rows(q, 0)


def shard_params(p: AttnParams, sh: AttnShape, r: int, shards: int):
    """The shard's parameter slices and its local shape."""
    q, kv = shard_heads(sh, r, shards)
    qkv_rows, o_cols = shard_rows(sh, r, shards)
    local = AttnShape(sh.batch, sh.seq, len(q), len(kv), sh.d)
    return AttnParams(p.norm_w.copy(), np.ascontiguousarray(p.w_qkv[qkv_rows]), np.ascontiguousarray(p.w_o[:, o_cols]),
                      p.b_o.copy()), local


def attn_sharded_step(x, p: AttnParams, sh: AttnShape, eps: float, lr: float, shards: int,
                      mode: str = "equivalence", dtype=np.float64, storage: str = "exact") -> dict:
    """The same step as S tensor-parallel shards of complete GQA groups, coded
    per rank: each rank computes N, its heads' Q/K/V, attention and its
    output-projection partial; the partials are summed in rank order (the
    forward all-reduce, then residual and bias once); in backward each rank's
    partial of dN is summed (the backward all-reduce) before RMSNorm's
    backward.  The ablations drop one of the two sums as in oracle.sharded_step."""
    if mode not in ATTN_MODES:
        raise ValueError(mode)
    R = storage_rounding(storage)
    x = np.asarray(x, dtype=dtype)
    p = p.astype(dtype)
    n, r = rms_norm_fwd(x, p.norm_w, eps)
    n = R(n)
    ranks: List[dict] = []
    for s in range(shards):
        lp, lsh = shard_params(p, sh, s, shards)
        qkv = R(n @ lp.w_qkv.T)
        q, k, v = split_qkv(qkv, lsh)
        o4, _ = causal_attention_fwd(q, k, v, lsh.group)
        O = R(merge_heads(o4, lsh))
        ranks.append(dict(lp=lp, lsh=lsh, qkv=qkv, O=O, z=O @ lp.w_o.T))
    if mode == "missing_forward_reduce":
        outs = [R(x + rk["z"] + p.b_o[None, :]) for rk in ranks]
    else:
        out = R(x + _ordered_sum([rk["z"] for rk in ranks]) + p.b_o[None, :])
        outs = [out] * shards
    for rk, o_s in zip(ranks, outs):
        lp, lsh = rk["lp"], rk["lsh"]
        dY = o_s
        g = {"w_o": dY.T @ rk["O"]}
        dO = R(dY @ lp.w_o)
        q, k, v = split_qkv(rk["qkv"], lsh)
        dq, dk, dv = causal_attention_bwd(q, k, v, split_heads(rk["O"], lsh.n_q, lsh), split_heads(dO, lsh.n_q, lsh),
                                          lsh.group)
        dqkv = R(np.concatenate([merge_heads(dq, lsh), merge_heads(dk, lsh), merge_heads(dv, lsh)], axis=1))
        g["w_qkv"] = dqkv.T @ n
        rk.update(grads=g, dN_partial=dqkv @ lp.w_qkv, out=o_s, dO=dO, dqkv=dqkv)
    if mode == "missing_backward_reduce":
        dNs = [rk["dN_partial"] for rk in ranks]
    else:
        dNs = [_ordered_sum([rk["dN_partial"] for rk in ranks])] * shards
    for rk, dN in zip(ranks, dNs):
        dY = rk["out"]
        dxn, d_norm_w = rms_norm_bwd(dN, x, r, p.norm_w)
        rk["dx"] = R(dY + dxn)
        rk["grads"].update(norm_w=d_norm_w, b_o=np.sum(dY, axis=0))
        rk["dN"] = dN
        rk["new_params"] = _sgd(rk["lp"], rk["grads"], lr, R)
    return dict(ranks=ranks, n=n, rstd=r)


def assemble_attn(ranks, sh: AttnShape, shards: int, key: str, which: str = "grads") -> np.ndarray:
    """A dense tensor from the shards' slices (w_qkv rows or w_o columns) of
    each rank's `which` ("grads": dict entries; "new_params": AttnParams)."""
    get = (lambda rk: rk[which][key]) if which == "grads" else (lambda rk: getattr(rk[which], key))
    first = get(ranks[0])
    if key == "w_qkv":
        full = np.zeros((sh.qkv_width, first.shape[1]))
        for s, rk in enumerate(ranks):
            full[shard_rows(sh, s, shards)[0]] = get(rk)
        return full
    if key == "w_o":
        full = np.zeros((first.shape[0], sh.n_q * sh.d))
        for s, rk in enumerate(ranks):
            full[:, shard_rows(sh, s, shards)[1]] = get(rk)
        return full
    raise KeyError(key)
