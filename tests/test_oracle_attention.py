"""Pins of the attention-sublayer oracle (oracle/attention.py) against what
fixes it from outside: PyTorch autograd of the block typed with library
routines (F.rms_norm, F.linear, F.scaled_dot_product_attention with causal
masking and grouped-query heads), central finite differences of every
parameter and input of a tiny block, brute-force per-row attention, closed
forms (zero output projection, zero queries give the causal running mean of
V, one position gives V itself), the sharded step equal to the dense step,
and the two ablations' signatures."""

import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

from oracle import attention as A
from oracle.mlp import bf16_round


def _block(seed, sh: A.AttnShape, H, std=0.3):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((sh.tokens, H))
    p = A.AttnParams(1.0 + 0.2 * rng.standard_normal(H), rng.standard_normal((sh.qkv_width, H)) * std,
                     rng.standard_normal((H, sh.n_q * sh.d)) * std, 0.2 * rng.standard_normal(H))
    return x, p


def _torch_block(x, p: A.AttnParams, sh: A.AttnShape, eps):
    """The sublayer in PyTorch float64 from library routines; returns out, loss and leaf tensors."""
    t = lambda a: torch.tensor(a, dtype=torch.float64, requires_grad=True)
    X, nw, wqkv, wo, bo = t(x), t(p.norm_w), t(p.w_qkv), t(p.w_o), t(p.b_o)
    H = x.shape[1]
    n = F.rms_norm(X, (H,), weight=nw, eps=eps)
    qkv = F.linear(n, wqkv)
    d, b, s = sh.d, sh.batch, sh.seq
    q = qkv[:, :sh.n_q * d].reshape(b, s, sh.n_q, d).transpose(1, 2)
    k = qkv[:, sh.n_q * d:(sh.n_q + sh.n_kv) * d].reshape(b, s, sh.n_kv, d).transpose(1, 2)
    v = qkv[:, (sh.n_q + sh.n_kv) * d:].reshape(b, s, sh.n_kv, d).transpose(1, 2)
    o = F.scaled_dot_product_attention(q, k, v, is_causal=True, enable_gqa=True)
    O = o.transpose(1, 2).reshape(b * s, sh.n_q * d)
    out = X + F.linear(O, wo) + bo
    loss = 0.5 * (out * out).sum()
    loss.backward()
    return out, loss, dict(x=X, norm_w=nw, w_qkv=wqkv, w_o=wo, b_o=bo)


SHAPES = [A.AttnShape(2, 5, 4, 2, 3), A.AttnShape(1, 7, 3, 3, 4), A.AttnShape(3, 4, 4, 1, 2)]


@pytest.mark.parametrize("sh", SHAPES, ids=lambda s: f"b{s.batch}s{s.seq}q{s.n_q}kv{s.n_kv}d{s.d}")
def test_dense_step_matches_torch_autograd(sh):
    H = 6
    x, p = _block(1, sh, H)
    r = A.attn_dense_step(x, p, sh, 1e-6, 0.1)
    out, loss, leaves = _torch_block(x, p, sh, 1e-6)
    close = lambda a, b: np.testing.assert_allclose(a, b, rtol=1e-10, atol=1e-12)
    close(r["out"], out.detach().numpy())
    close(r["loss"], float(loss.detach()))
    close(r["dx"], leaves["x"].grad.numpy())
    for k in ("norm_w", "w_qkv", "w_o", "b_o"):
        close(r["grads"][k], leaves[k].grad.numpy())
    np.testing.assert_allclose(r["new_params"].w_qkv, p.w_qkv - 0.1 * leaves["w_qkv"].grad.numpy(), rtol=1e-12)


def test_finite_differences_of_every_scalar():
    sh = A.AttnShape(1, 3, 2, 1, 2)
    H = 4
    x, p = _block(2, sh, H, std=0.5)
    r = A.attn_dense_step(x, p, sh, 1e-6, 0.1)

    def loss(xx, pp):
        return A.attn_dense_step(xx, pp, sh, 1e-6, 0.1)["loss"]

    checked = 0
    for name in ("x", "norm_w", "w_qkv", "w_o", "b_o"):
        base = x if name == "x" else getattr(p, name)
        grad = r["dx"] if name == "x" else r["grads"][name]
        # dL/dx: the residual gives dY directly and dx also carries the norm's term -- r["dx"] is the full gradient
        for idx in np.ndindex(base.shape):
            h = 1e-6 * max(1.0, abs(base[idx]))
            plus, minus = base.copy(), base.copy()
            plus[idx] += h
            minus[idx] -= h
            if name == "x":
                fd = (loss(plus, p) - loss(minus, p)) / (2 * h)
            else:
                pp = A.AttnParams(**{k: (plus if k == name else getattr(p, k)) for k in ("norm_w", "w_qkv", "w_o", "b_o")})
                pm = A.AttnParams(**{k: (minus if k == name else getattr(p, k)) for k in ("norm_w", "w_qkv", "w_o", "b_o")})
                fd = (loss(x, pp) - loss(x, pm)) / (2 * h)
            assert abs(fd - grad[idx]) <= 1e-6 * max(1.0, abs(fd)), (name, idx, fd, grad[idx])
            checked += 1
    assert checked == 12 + 4 + 32 + 16 + 4  # x, norm_w, w_qkv, w_o, b_o


def test_attention_against_brute_force_rows():
    rng = np.random.default_rng(3)
    b, nq, nkv, s, d = 2, 4, 2, 6, 3
    q, k, v = rng.standard_normal((b, nq, s, d)), rng.standard_normal((b, nkv, s, d)), rng.standard_normal((b, nkv, s, d))
    o, lse = A.causal_attention_fwd(q, k, v, nq // nkv)
    for bb in range(b):
        for h in range(nq):
            g = h // (nq // nkv)
            for i in range(s):
                sc = [sum(q[bb, h, i, e] * k[bb, g, j, e] for e in range(d)) / math.sqrt(d) for j in range(i + 1)]
                m = max(sc)
                w = [math.exp(c - m) for c in sc]
                z = sum(w)
                for e in range(d):
                    assert abs(o[bb, h, i, e] - sum(w[j] * v[bb, g, j, e] for j in range(i + 1)) / z) < 1e-12
                assert abs(lse[bb, h, i] - (m + math.log(z))) < 1e-12


def test_closed_forms():
    sh = A.AttnShape(2, 6, 4, 2, 3)
    H = 5
    x, p = _block(4, sh, H)
    # zero output projection: out = x + b_o and dx = out (nothing flows back through attention)
    p0 = A.AttnParams(p.norm_w, p.w_qkv, np.zeros_like(p.w_o), p.b_o)
    r = A.attn_dense_step(x, p0, sh, 1e-6, 0.1)
    np.testing.assert_allclose(r["out"], x + p.b_o[None, :], rtol=1e-14, atol=1e-14)
    np.testing.assert_allclose(r["dx"], r["out"], rtol=1e-14, atol=1e-14)
    assert np.abs(r["grads"]["w_qkv"]).max() == 0 and np.abs(r["grads"]["norm_w"]).max() == 0
    # zero query rows: uniform weights over j <= i, each head's output is the running mean of its V
    wq = p.w_qkv.copy()
    wq[:sh.n_q * sh.d] = 0
    r = A.attn_dense_step(x, A.AttnParams(p.norm_w, wq, p.w_o, p.b_o), sh, 1e-6, 0.1)
    _, _, v = A.split_qkv(r["qkv"], sh)
    O = A.split_heads(r["O"], sh.n_q, sh)
    for h in range(sh.n_q):
        run = np.cumsum(v[:, h // sh.group], axis=1) / np.arange(1, sh.seq + 1)[None, :, None]
        np.testing.assert_allclose(O[:, h], run, rtol=1e-12, atol=1e-14)
    # one position per sequence: attention returns V
    sh1 = A.AttnShape(5, 1, 4, 2, 3)
    x1, p1 = _block(5, sh1, H)
    r = A.attn_dense_step(x1, p1, sh1, 1e-6, 0.1)
    _, _, v = A.split_qkv(r["qkv"], sh1)
    O = A.split_heads(r["O"], sh1.n_q, sh1)
    for h in range(sh1.n_q):
        np.testing.assert_allclose(O[:, h], v[:, h // sh1.group], rtol=1e-14)


def test_shards_keep_whole_groups():
    sh = A.AttnShape(1, 4, 8, 4, 2)
    seen_q, seen_kv = [], []
    for r in range(2):
        q, kv = A.shard_heads(sh, r, 2)
        assert all(h // sh.group in kv for h in q)          # every query head with its own KV head
        assert len(q) == sh.group * len(kv)
        seen_q += q
        seen_kv += kv
    assert sorted(seen_q) == list(range(8)) and sorted(seen_kv) == list(range(4))
    with pytest.raises(ValueError):
        A.shard_heads(sh, 0, 3)


@pytest.mark.parametrize("S", [1, 2, 4])
def test_sharded_step_is_the_dense_step(S):
    sh = A.AttnShape(2, 5, 8, 4, 3)
    H = 6
    x, p = _block(6, sh, H)
    d = A.attn_dense_step(x, p, sh, 1e-6, 0.1)
    r = A.attn_sharded_step(x, p, sh, 1e-6, 0.1, S)
    close = lambda a, b: np.testing.assert_allclose(a, b, rtol=1e-11, atol=1e-12)
    for rk in r["ranks"]:
        close(rk["out"], d["out"])
        close(rk["dx"], d["dx"])
        close(rk["grads"]["norm_w"], d["grads"]["norm_w"])
        close(rk["grads"]["b_o"], d["grads"]["b_o"])
    close(A.assemble_attn(r["ranks"], sh, S, "w_qkv"), d["grads"]["w_qkv"])
    close(A.assemble_attn(r["ranks"], sh, S, "w_o"), d["grads"]["w_o"])
    close(A.assemble_attn(r["ranks"], sh, S, "w_qkv", "new_params"), d["new_params"].w_qkv)
    # each rank's partial is its own heads' contribution: the partials add up to the dense projection
    close(sum(rk["z"] for rk in r["ranks"]), d["z"])


def test_ablation_signatures():
    sh = A.AttnShape(2, 5, 4, 2, 3)
    H = 6
    x, p = _block(7, sh, H, std=0.5)
    d = A.attn_dense_step(x, p, sh, 1e-6, 0.1)
    fwd = A.attn_sharded_step(x, p, sh, 1e-6, 0.1, 2, mode="missing_forward_reduce")
    bwd = A.attn_sharded_step(x, p, sh, 1e-6, 0.1, 2, mode="missing_backward_reduce")
    scale = np.abs(d["out"]).max()
    # without the forward sum each rank's output misses the other rank's heads
    for rk in fwd["ranks"]:
        assert np.abs(rk["out"] - d["out"]).max() > 1e-2 * scale
    # without the backward sum: output and the weight gradients are intact, dx and the norm gradient are not
    for rk in bwd["ranks"]:
        np.testing.assert_allclose(rk["out"], d["out"], rtol=1e-12, atol=1e-12)
        assert np.abs(rk["dx"] - d["dx"]).max() > 1e-3 * np.abs(d["dx"]).max()
        assert np.abs(rk["grads"]["norm_w"] - d["grads"]["norm_w"]).max() > 1e-3 * np.abs(d["grads"]["norm_w"]).max()
    np.testing.assert_allclose(A.assemble_attn(bwd["ranks"], sh, 2, "w_qkv"), d["grads"]["w_qkv"], rtol=1e-11,
                               atol=1e-12)
    # the per-rank dN partials add up to the dense dN
    np.testing.assert_allclose(sum(rk["dN"] for rk in bwd["ranks"]), d["dN"], rtol=1e-11, atol=1e-12)


def test_bf16_storage_rounds_the_stored_tensors():
    sh = A.AttnShape(1, 4, 2, 1, 4)
    x, p = _block(8, sh, 8)
    x, p = bf16_round(x), A.AttnParams(*(bf16_round(v) for v in (p.norm_w, p.w_qkv, p.w_o, p.b_o)))
    r = A.attn_dense_step(x, p, sh, 1e-6, 0.1, storage="bf16")
    for k in ("n", "qkv", "O", "out", "dO", "dqkv", "dx"):
        np.testing.assert_array_equal(r[k], bf16_round(r[k]))
    e = A.attn_dense_step(x, p, sh, 1e-6, 0.1)
    assert 0 < np.abs(r["out"] - e["out"]).max() < 3e-2
