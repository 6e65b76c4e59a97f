"""Pins of the CPU oracle against things other than itself.

Each test ties an oracle function to something it does not compute itself:
finite differences, PyTorch library routines and autograd, closed forms,
brute force, or the numbers the page prints.  A plausible slip anywhere in
the oracle (a dropped term, a wrong sign or index, a transposed operand, a
bias added per shard) fails at least one of them.
"""

import json
import math
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
from oracle.mlp import Params, assemble
import synth

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _params(rng, T, H, Fw, act, std, perturb=True):
    x = rng.standard_normal((T, H))
    norm_w = 1.0 + (0.3 * rng.standard_normal(H) if perturb else 0.0)
    if act == "swiglu":
        w_in = rng.standard_normal((2, Fw, H)) * std
        b_in = None
    else:
        w_in = rng.standard_normal((Fw, H)) * std
        b_in = 0.3 * rng.standard_normal(Fw)
    w_down = rng.standard_normal((H, Fw)) * std
    b_down = 0.3 * rng.standard_normal(H) if perturb else np.zeros(H)
    return x, Params(np.asarray(norm_w, float) * np.ones(H), w_in, w_down, b_down, b_in)


# ------------------------------------------------------------ library routines

def test_rms_norm_matches_torch_rms_norm():
    rng = np.random.default_rng(1)
    x = rng.standard_normal((7, 24)) * 3.0
    w = rng.standard_normal(24)
    n, r = oracle.rms_norm_fwd(x, w, 1e-6)
    ref = F.rms_norm(torch.from_numpy(x), (24,), torch.from_numpy(w), eps=1e-6).numpy()
    np.testing.assert_allclose(n, ref, rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(r, 1.0 / np.sqrt((x ** 2).mean(1) + 1e-6), rtol=1e-14)


def test_elementwise_match_torch_routines():
    v = np.linspace(-12, 12, 2001)
    tv = torch.from_numpy(v).requires_grad_(True)
    np.testing.assert_allclose(oracle.silu(v), F.silu(tv).detach().numpy(), rtol=1e-14, atol=1e-300)
    np.testing.assert_allclose(oracle.gelu(v), F.gelu(tv).detach().numpy(), rtol=1e-13, atol=1e-300)
    (gs,) = torch.autograd.grad(F.silu(tv).sum(), tv)
    (gg,) = torch.autograd.grad(F.gelu(tv).sum(), tv)
    np.testing.assert_allclose(oracle.silu_grad(v), gs.numpy(), rtol=1e-12, atol=1e-15)
    np.testing.assert_allclose(oracle.gelu_grad(v), gg.numpy(), rtol=1e-12, atol=1e-15)


def test_elementwise_special_values():
    assert oracle.silu(np.array(0.0)) == 0.0
    assert oracle.silu_grad(np.array(0.0)) == 0.5
    assert oracle.gelu(np.array(0.0)) == 0.0
    assert oracle.gelu_grad(np.array(0.0)) == 0.5
    for v in (-3.0, -0.5, 0.7, 2.5):
        assert math.isclose(float(oracle.sigmoid(np.array(v))), 1.0 / (1.0 + math.exp(-v)), rel_tol=1e-15)
        assert math.isclose(float(oracle.gelu(np.array(v))), 0.5 * v * (1 + math.erf(v / math.sqrt(2))),
                            rel_tol=1e-14)
    # large |v| limits: silu -> v (v >> 0) and -> 0 (v << 0)
    assert abs(float(oracle.silu(np.array(40.0))) - 40.0) < 1e-12
    assert abs(float(oracle.silu(np.array(-40.0)))) < 1e-15


# ------------------------------------------------------------- finite differences

def _loss(x, p, act, eps):
    return oracle.dense_step(x, p, act, eps, 0.1)["loss"]


@pytest.mark.parametrize("act", ["swiglu", "gelu"])
@pytest.mark.parametrize("scale", ["unit", "page"])
def test_backward_matches_central_differences(act, scale):
    """Brute force: every one of the 432 scalars of the tiny block (T=4, H=8,
    F=16: x 32 + norm 8 + gate/up 256 + down 128 + bias 8; GeLU: fc1 128 +
    fc1 bias 16 instead of gate/up) is perturbed and the fp64 central
    difference of the loss compared with the analytic gradient."""
    rng = np.random.default_rng(7)
    T, H, Fw = 4, 8, 16
    std = 0.02 if scale == "page" else 1.0 / math.sqrt(H)
    x, p = _params(rng, T, H, Fw, act, std)
    eps = 1e-6
    d = oracle.dense_step(x, p, act, eps, 0.1)
    analytic = {"x": d["dx"], **{k: d["grads"][k] for k in p.names()}}

    def fd(get_arr, idx):
        arr = get_arr()
        v0 = arr[idx]
        h = 1e-6 * max(1.0, abs(v0))
        arr[idx] = v0 + h
        lp = _loss(x, p, act, eps)
        arr[idx] = v0 - h
        lm = _loss(x, p, act, eps)
        arr[idx] = v0
        return (lp - lm) / (2 * h)

    checked = 0
    for name in ["x"] + p.names():
        get = (lambda: x) if name == "x" else (lambda name=name: getattr(p, name))
        arr = get()
        num = np.zeros_like(arr)
        for idx in np.ndindex(arr.shape):
            num[idx] = fd(get, idx)
            checked += 1
        np.testing.assert_allclose(analytic[name], num, rtol=1e-6, atol=2e-8, err_msg=name)
    assert checked == (432 if act == "swiglu" else 32 + 8 + 128 + 16 + 128 + 8)


# ------------------------------------------------------- autograd of the block

def _torch_block(x, p, act, eps):
    """The dense block of the page's listing, typed with PyTorch library
    routines; its backward comes from autograd."""
    t = lambda a: torch.from_numpy(np.array(a)).requires_grad_(True)
    xt, nw, wi, wd, bd = t(x), t(p.norm_w), t(p.w_in), t(p.w_down), t(p.b_down)
    bi = t(p.b_in) if p.b_in is not None else None
    n = F.rms_norm(xt, (x.shape[1],), nw, eps=eps)
    if act == "swiglu":
        hidden = F.silu(F.linear(n, wi[0])) * F.linear(n, wi[1])
    else:
        hidden = F.gelu(F.linear(n, wi, bi))
    out = xt + F.linear(hidden, wd, bd)
    loss = 0.5 * (out * out).sum()
    loss.backward()
    leaves = dict(x=xt, norm_w=nw, w_in=wi, w_down=wd, b_down=bd)
    if bi is not None:
        leaves["b_in"] = bi
    return out.detach().numpy(), float(loss), {k: v.grad.numpy() for k, v in leaves.items()}


@pytest.mark.parametrize("act", ["swiglu", "gelu"])
def test_dense_step_matches_torch_autograd(act):
    rng = np.random.default_rng(11)
    x, p = _params(rng, 13, 24, 40, act, 0.2)
    d = oracle.dense_step(x, p, act, 1e-6, 0.1)
    out, loss, grads = _torch_block(x, p, act, 1e-6)
    np.testing.assert_allclose(d["out"], out, rtol=1e-12, atol=1e-12)
    assert math.isclose(d["loss"], loss, rel_tol=1e-12)
    np.testing.assert_allclose(d["dx"], grads["x"], rtol=1e-10, atol=1e-11)
    for k in p.names():
        np.testing.assert_allclose(d["grads"][k], grads[k], rtol=1e-10, atol=1e-11, err_msg=k)


# ---------------------------------------------------------------- closed forms

def test_zero_down_weight_gives_residual_plus_bias():
    rng = np.random.default_rng(3)
    x, p = _params(rng, 5, 8, 12, "swiglu", 0.5)
    p.w_down[:] = 0.0
    d = oracle.dense_step(x, p, "swiglu", 1e-6, 0.1)
    assert np.array_equal(d["out"], x + p.b_down[None, :])
    assert np.all(d["dN"] == 0.0)


def test_zero_gate_gives_identity_block():
    """silu(0) = 0, so a zero gate plane kills the MLP branch in forward and
    every gradient through it: out = x + b, dN = 0, dx = d out = out."""
    rng = np.random.default_rng(4)
    x, p = _params(rng, 5, 8, 12, "swiglu", 0.5)
    p.w_in[0] = 0.0
    d = oracle.dense_step(x, p, "swiglu", 1e-6, 0.1)
    assert np.array_equal(d["out"], x + p.b_down[None, :])
    assert np.all(d["dN"] == 0.0)
    assert np.array_equal(d["dx"], d["out"])
    assert np.all(d["grads"]["norm_w"] == 0.0)
    np.testing.assert_array_equal(d["grads"]["b_down"], d["out"].sum(0))


def test_constant_row_and_scale_invariance():
    w = np.linspace(0.5, 1.5, 16)
    for c in (-3.0, 0.25, 7.0):
        n, r = oracle.rms_norm_fwd(np.full((1, 16), c), w, 1e-6)
        np.testing.assert_allclose(n[0], c / math.sqrt(c * c + 1e-6) * w, rtol=1e-15)
    rng = np.random.default_rng(5)
    x = rng.standard_normal((3, 16))
    n1, _ = oracle.rms_norm_fwd(x, w, 0.0)
    n2, _ = oracle.rms_norm_fwd(50.0 * x, w, 0.0)
    np.testing.assert_allclose(n1, n2, rtol=1e-14)


def test_one_by_one_hand_case():
    """H = F = 1, x = 2, w = 1, eps = 0: n = 1, so g = Wg, u = Wu and
    out = 2 + silu(Wg) Wu Wd + b."""
    wg, wu, wd, b = 0.7, -1.3, 0.4, 0.25
    p = Params(np.array([1.0]), np.array([[[wg]], [[wu]]]), np.array([[wd]]), np.array([b]))
    d = oracle.dense_step(np.array([[2.0]]), p, "swiglu", 0.0, 0.1)
    silu = wg / (1.0 + math.exp(-wg))
    assert d["n"][0, 0] == 1.0
    assert math.isclose(d["out"][0, 0], 2.0 + silu * wu * wd + b, rel_tol=1e-15)
    # H = 1 RMSNorm is x / |x|: its derivative is zero, so dx = d out exactly.
    assert math.isclose(d["dx"][0, 0], d["out"][0, 0], rel_tol=0, abs_tol=1e-15)


def test_loss_gradient_is_output():
    rng = np.random.default_rng(6)
    x, p = _params(rng, 4, 8, 8, "swiglu", 0.3)
    d = oracle.dense_step(x, p, "swiglu", 1e-6, 0.1)
    assert d["loss"] == pytest.approx(0.5 * float((d["out"] ** 2).sum()), rel=1e-15)
    assert d["dY"] is d["out"]


def test_sgd_closed_form():
    rng = np.random.default_rng(8)
    x, p = _params(rng, 6, 8, 16, "gelu", 0.3)
    lr = 0.1
    d = oracle.dense_step(x, p, "gelu", 1e-6, lr)
    for k in p.names():
        np.testing.assert_allclose((getattr(p, k) - getattr(d["new_params"], k)) / lr, d["grads"][k],
                                   rtol=1e-12, atol=1e-13)


# ------------------------------------------------------------ sharding identity

@pytest.mark.parametrize("act", ["swiglu", "gelu"])
@pytest.mark.parametrize("S", [1, 2, 4, 8])
def test_sharded_equals_dense_fp64(act, S):
    rng = np.random.default_rng(20 + S)
    x, p = _params(rng, 6, 16, 32, act, 0.3)
    d = oracle.dense_step(x, p, act, 1e-6, 0.1)
    sh = oracle.sharded_step(x, p, act, 1e-6, 0.1, S)
    for rk in sh["ranks"]:
        np.testing.assert_allclose(rk["out"], d["out"], rtol=0, atol=1e-13)
        np.testing.assert_allclose(rk["dx"], d["dx"], rtol=0, atol=1e-13)
        np.testing.assert_allclose(rk["grads"]["norm_w"], d["grads"]["norm_w"], rtol=0, atol=1e-12)
        np.testing.assert_allclose(rk["grads"]["b_down"], d["grads"]["b_down"], rtol=0, atol=1e-13)
    for k in ["w_in", "w_down"] + (["b_in"] if act == "gelu" else []):
        np.testing.assert_allclose(assemble(sh, k), d["grads"][k], rtol=0, atol=1e-13, err_msg=k)
        np.testing.assert_allclose(assemble(sh, k, "new_params"), getattr(d["new_params"], k),
                                   rtol=0, atol=1e-13, err_msg=k)
    if S == 1:
        rk = sh["ranks"][0]
        assert np.array_equal(rk["out"], d["out"])
        assert np.array_equal(rk["dx"], d["dx"])
        assert np.array_equal(rk["grads"]["w_in"], d["grads"]["w_in"])


def test_shard_width_must_divide():
    rng = np.random.default_rng(9)
    x, p = _params(rng, 2, 8, 12, "swiglu", 0.3)
    with pytest.raises(ValueError):
        oracle.sharded_step(x, p, "swiglu", 1e-6, 0.1, 5)


def test_sharded_partials_are_the_channel_blocks():
    """Each rank's partial is exactly the dense contraction restricted to its
    channel interval (brute-force sum over its channels)."""
    rng = np.random.default_rng(10)
    x, p = _params(rng, 3, 8, 12, "swiglu", 0.4)
    sh = oracle.sharded_step(x, p, "swiglu", 1e-6, 0.1, 2)
    d = oracle.dense_step(x, p, "swiglu", 1e-6, 0.1)
    for s, rk in enumerate(sh["ranks"]):
        ref = np.zeros((3, 8))
        for t in range(3):
            for k in range(8):
                ref[t, k] = sum(d["a"][t, j] * p.w_down[k, j] for j in range(6 * s, 6 * s + 6))
        np.testing.assert_allclose(rk["z"], ref, rtol=1e-13, atol=1e-15)


# ------------------------------------------------------------------ ablations

def test_ablation_closed_forms():
    """Dropping the forward sum leaves each rank short by exactly the other
    ranks' partials; dropping the backward sum leaves each rank's dN short by
    exactly the other ranks' contributions."""
    rng = np.random.default_rng(12)
    x, p = _params(rng, 5, 8, 16, "swiglu", 0.4)
    S = 4
    eq = oracle.sharded_step(x, p, "swiglu", 1e-6, 0.1, S)
    af = oracle.sharded_step(x, p, "swiglu", 1e-6, 0.1, S, mode="missing_forward_reduce")
    ab = oracle.sharded_step(x, p, "swiglu", 1e-6, 0.1, S, mode="missing_backward_reduce")
    zs = [rk["z"] for rk in eq["ranks"]]
    dns = [rk["dN_partial"] for rk in eq["ranks"]]
    for s in range(S):
        others = sum(zs[q] for q in range(S) if q != s)
        np.testing.assert_allclose(af["ranks"][s]["out"] - eq["ranks"][s]["out"], -others, atol=1e-13)
        others_dn = sum(dns[q] for q in range(S) if q != s)
        np.testing.assert_allclose(ab["ranks"][s]["dN"] - eq["ranks"][s]["dN"], -others_dn, atol=1e-13)
        # forward and local weight grads are untouched by the backward ablation
        assert np.array_equal(ab["ranks"][s]["out"], eq["ranks"][s]["out"])
        assert np.array_equal(ab["ranks"][s]["grads"]["w_in"], eq["ranks"][s]["grads"]["w_in"])
        assert np.array_equal(ab["ranks"][s]["grads"]["w_down"], eq["ranks"][s]["grads"]["w_down"])


_FIELDS = ["forward_max_abs_diff", "loss_abs_diff", "input_grad_max_abs_diff", "norm_grad_max_abs_diff",
           "gate_up_grad_max_abs_diff", "down_grad_max_abs_diff", "post_step_weight_max_abs_diff"]


def _signature(rec, scale=None, small=1e-6, large=1e-3):
    """Classify each field of a record as 'small' (rounding level) or 'large'
    (broken).  ``scale`` gives the magnitude of the compared quantity per
    field; the page's own values are classified in absolute terms."""
    sig = {}
    for k in _FIELDS:
        v = rec[k] / (scale[k] if scale else 1.0)
        sig[k] = "small" if v <= small else ("large" if v >= large else "mid")
    return sig


def _scales(d):
    g, p = d["grads"], d["new_params"]
    m = lambda a: float(np.max(np.abs(a)))
    return {"forward_max_abs_diff": m(d["out"]), "loss_abs_diff": abs(float(d["loss"])),
            "input_grad_max_abs_diff": m(d["dx"]), "norm_grad_max_abs_diff": m(g["norm_w"]),
            "gate_up_grad_max_abs_diff": m(g["w_in"]), "down_grad_max_abs_diff": m(g["w_down"]),
            "post_step_weight_max_abs_diff": max(m(getattr(p, k)) for k in p.names())}


def _page_sized(rng, std):
    """Fixture-sized tensors: seq 3 x batch 2 tokens, hidden 8, ffn 12, two
    ranks, a small nonzero bias (the page's shapes; values are ours)."""
    x = rng.standard_normal((6, 8)).astype(np.float32)
    p = Params(np.ones(8), rng.standard_normal((2, 12, 8)) * std, rng.standard_normal((8, 12)) * std,
               0.05 * rng.standard_normal(8))
    return x, p


def test_fixture_records_match_page_signatures():
    """Fp32 dense vs fp32 two-rank step on the page's shapes: the equivalence
    record shows rounding-level differences of the page's order (forward ~1e-7,
    post-step ~1e-8), and each ablation breaks exactly the fields the page's
    records break."""
    with open(os.path.join(GOLD, "fixture_records.json")) as f:
        page = json.load(f)
    rng = np.random.default_rng(2024)
    x, p = _page_sized(rng, 1.0 / math.sqrt(8))
    lr = 0.05
    recs = {}
    d32 = oracle.dense_step(x, p, "swiglu", 1e-6, lr, dtype=np.float32)
    for mode in oracle.MODES:
        sh = oracle.sharded_step(x, p, "swiglu", 1e-6, lr, 2, mode=mode, dtype=np.float32)
        recs[mode] = oracle.fixture_record(d32, sh)
    eq = recs["equivalence"]
    sc = _scales(d32)
    # the page: 1.27e-7 forward, 1.49e-8 post-step, i.e. a few fp32 ulps of the
    # compared values; ours must be the same few ulps of our magnitudes
    ulp = float(np.finfo(np.float32).eps)
    for k in _FIELDS:
        assert eq[k] <= 16 * ulp * sc[k], (k, eq[k], sc[k])
    assert eq["down_bias_grad_max_abs_diff"] <= 16 * ulp * float(np.abs(d32["grads"]["b_down"]).max())
    for mode in ("missing_forward_reduce", "missing_backward_reduce"):
        ours, theirs = _signature(recs[mode], sc, small=1e-5), _signature(page[mode])
        assert ours == theirs, (mode, ours, theirs)


def test_backward_ablation_post_step_is_lr_times_norm_grad_gap():
    """Only the norm weight's gradient is wrong in the backward ablation, so
    the post-step gap is lr times the norm-grad gap.  The page's record obeys
    the same relation with lr = 0.05 (0.20240137 * 0.05 = 0.01012007 against
    0.01012015, one fp32 ulp of a unit-size weight)."""
    with open(os.path.join(GOLD, "fixture_records.json")) as f:
        pg = json.load(f)["missing_backward_reduce"]
    assert abs(pg["post_step_weight_max_abs_diff"] - 0.05 * pg["norm_grad_max_abs_diff"]) < 1.2e-7
    rng = np.random.default_rng(99)
    x, p = _page_sized(rng, 0.4)
    x = x.astype(np.float64)
    lr = 0.05
    d = oracle.dense_step(x, p, "swiglu", 1e-6, lr)
    rec = oracle.fixture_record(d, oracle.sharded_step(x, p, "swiglu", 1e-6, lr, 2,
                                                       mode="missing_backward_reduce"))
    assert rec["post_step_weight_max_abs_diff"] == pytest.approx(lr * rec["norm_grad_max_abs_diff"], rel=1e-10)
    assert rec["gate_up_grad_max_abs_diff"] < 1e-14 and rec["down_grad_max_abs_diff"] < 1e-14


def test_ablations_detectable_on_tiny_workload():
    """On the tiny fp32 workload (weights N(0, 0.02)) the MLP branch is small,
    but each ablation still moves its fields by far more than both the
    equivalence gaps and the 1e-5 fp32 tolerance."""
    w = synth.workload("tiny_fp32_tp2")
    t = synth.draw(w)
    x = synth.to_numpy64(t["x"])
    p = Params(*(synth.to_numpy64(t[k]) for k in ("norm_w", "w_in", "w_down", "b_down")))
    d = oracle.dense_step(x, p, "swiglu", w.eps, w.lr)
    rec = {m: oracle.fixture_record(d, oracle.sharded_step(x, p, "swiglu", w.eps, w.lr, 2, mode=m))
           for m in oracle.MODES}
    eq_max = max(v for k, v in rec["equivalence"].items() if k.endswith("_diff"))
    assert eq_max < 1e-13
    af, ab = rec["missing_forward_reduce"], rec["missing_backward_reduce"]
    assert af["forward_max_abs_diff"] > max(1e-5, 100 * eq_max)
    assert ab["forward_max_abs_diff"] < 1e-13 and ab["loss_abs_diff"] < 1e-12
    assert ab["input_grad_max_abs_diff"] > max(1e-5, 100 * eq_max)
    assert ab["norm_grad_max_abs_diff"] > max(1e-5, 100 * eq_max)
    assert ab["post_step_weight_max_abs_diff"] > 1e-6


# ---------------------------------------------------------------- page record

def test_inspect_record_matches_page():
    with open(os.path.join(GOLD, "inspect_record.json")) as f:
        page = json.load(f)
    rec = oracle.inspect_record(seq=3, batch=2, hidden=8, ffn=12, world=2)
    for k in ("world_size", "block_path", "dense_shapes", "rank_local_shapes"):
        assert rec[k] == page[k], k
    # rank 1 holds the same local shapes
    assert oracle.inspect_record(3, 2, 8, 12, 2, rank=1)["rank_local_shapes"] == page["rank_local_shapes"]


# --------------------------------------------------------------- row sampling

@pytest.mark.parametrize("act", ["swiglu", "gelu"])
def test_row_sampled_step_equals_full_step(act):
    rng = np.random.default_rng(30)
    x, p = _params(rng, 9, 16, 24, act, 0.3)
    d = oracle.dense_step(x, p, act, 1e-6, 0.1)
    rows = np.array([0, 4, 8])
    r = oracle.row_forward_backward(x[rows], p, act, 1e-6)
    for k in ("out", "dx", "dN", "a"):
        np.testing.assert_allclose(r[k], d[k][rows], rtol=1e-13, atol=1e-14, err_msg=k)


# ---------------------------------------------------------- full-size sampling

@pytest.mark.parametrize("act", ["swiglu", "gelu"])
def test_sampled_step_equals_dense_step(act):
    rng = np.random.default_rng(31)
    x, p = _params(rng, 11, 16, 24, act, 0.3)
    d = oracle.dense_step(x, p, act, 1e-6, 0.1)
    rows, chans, cols = [1, 5, 10], [0, 7, 23], [2, 15]
    s = oracle.sampled_step(x, p, act, 1e-6, 0.1, rows, chans, cols, dtype=np.float64)
    g, npar = d["grads"], d["new_params"]
    close = lambda a, b: np.testing.assert_allclose(a, b, rtol=1e-12, atol=1e-13)
    close(s["out"], d["out"])
    close(s["dN_rows"], d["dN"][rows])
    close(s["dx_rows"], d["dx"][rows])
    close(s["act_chans"], d["a"][:, chans])
    close(s["d_b_down"], g["b_down"])
    close(s["d_w_down_chans"], g["w_down"][:, chans])
    close(s["d_norm_w_cols"], g["norm_w"][cols])
    close(s["new_norm_w_cols"], npar.norm_w[cols])
    close(s["new_b_down"], npar.b_down)
    close(s["new_w_down_chans"], npar.w_down[:, chans])
    if act == "swiglu":
        close(s["d_w_in_chans"], g["w_in"][:, chans, :])
        close(s["new_w_in_chans"], npar.w_in[:, chans, :])
    else:
        close(s["d_w_in_chans"], g["w_in"][chans, :])
        close(s["d_b_in"], g["b_in"])
        close(s["new_w_in_chans"], npar.w_in[chans, :])
        close(s["new_b_in"], npar.b_in)


# ------------------------------------------------------------ bf16 storage model

def _torch_bf16(v):
    return torch.from_numpy(np.asarray(v, dtype=np.float32)).to(torch.bfloat16).double().numpy()


def test_bf16_round_matches_torch_conversion():
    rng = np.random.default_rng(40)
    v = (rng.standard_normal(200000) * np.exp(rng.uniform(-20, 20, 200000))).astype(np.float32)
    # exact ties: a bf16 value plus half of its last place, for both parities of that place
    base = _torch_bf16(rng.standard_normal(1000)).astype(np.float32)
    ulp = np.ldexp(1.0, np.frexp(base)[1] - 8)
    ties = (base + 0.5 * ulp).astype(np.float32)
    for arr in (v, ties, np.array([0.0, -0.0, 1.0, -3.5, 65504.0, 3.3e38], dtype=np.float32)):
        ref = _torch_bf16(arr)
        np.testing.assert_array_equal(oracle.bf16_round(arr).astype(np.float64), ref)
        np.testing.assert_array_equal(oracle.bf16_round(arr.astype(np.float64)), ref)
    assert oracle.bf16_round(np.float32(1.0) + np.float32(2.0 ** -8)) == 1.0          # tie, even stays
    assert oracle.bf16_round(np.float32(1.0) + np.float32(3 * 2.0 ** -8)) == 1.0 + 2.0 ** -6  # tie, odd rounds up


def _is_bf16(a):
    a = np.asarray(a, dtype=np.float64)
    return np.array_equal(oracle.bf16_round(a), a)


@pytest.mark.parametrize("act", ["swiglu", "gelu"])
def test_bf16_storage_tensors_are_bf16(act):
    rng = np.random.default_rng(41)
    x, p = _params(rng, 9, 16, 24, act, 0.3)
    x, p = _torch_bf16(x), p.astype(np.float64)
    for k in p.names():
        setattr(p, k, _torch_bf16(getattr(p, k)))
    d = oracle.dense_step(x, p, act, 1e-6, 0.1, storage="bf16")
    for name in ("n", "a", "out", "dx"):
        assert _is_bf16(d[name]), name
    for t in d["pre"]:
        assert _is_bf16(t)
    # the pre-activation gradients (dg, du | dh) are stored tensors too
    assert len(d["d_pre"]) == (2 if act == "swiglu" else 1)
    for t in d["d_pre"]:
        assert _is_bf16(t)
    # ... and are the rounding of the exact product of the stored inputs
    ref = oracle.activation_bwd(d["da"], d["pre"], act)
    for t, r in zip(d["d_pre"], ref):
        np.testing.assert_array_equal(t, oracle.bf16_round(r))
    for k in p.names():
        assert _is_bf16(getattr(d["new_params"], k)), k
    # masters are not rounded, and round to the stored parameters
    np.testing.assert_array_equal(oracle.bf16_round(d["new_masters"].w_in), d["new_params"].w_in)
    e = oracle.dense_step(x, p, act, 1e-6, 0.1)
    assert not np.array_equal(d["out"], e["out"])


def test_bf16_forward_matches_torch_bf16_forward():
    """The bf16 storage forward against PyTorch's CPU bf16 forward of the
    page's block (bf16 tensors, fp32 accumulation inside each op)."""
    rng = np.random.default_rng(42)
    T, H, Fw = 64, 96, 160
    x = _torch_bf16(rng.standard_normal((T, H)))
    p = Params(_torch_bf16(1 + 0.2 * rng.standard_normal(H)), _torch_bf16(rng.standard_normal((2, Fw, H)) * 0.1),
               _torch_bf16(rng.standard_normal((H, Fw)) * 0.1), _torch_bf16(0.1 * rng.standard_normal(H)))
    d = oracle.dense_step(x, p, "swiglu", 1e-6, 0.1, storage="bf16")
    b = lambda a: torch.from_numpy(np.asarray(a, dtype=np.float32)).to(torch.bfloat16)
    with torch.no_grad():
        n = F.rms_norm(b(x), (H,), b(p.norm_w), eps=1e-6)
        g, u = F.linear(n, b(p.w_in[0])), F.linear(n, b(p.w_in[1]))
        hidden = F.silu(g) * u
        out = b(x) + F.linear(hidden, b(p.w_down), b(p.b_down))
    one_ulp = lambda a: np.ldexp(1.0, np.frexp(np.abs(a))[1] - 8)
    # single rounded ops agree to one bf16 place
    assert np.all(np.abs(n.double().numpy() - d["n"]) <= one_ulp(d["n"]))
    # with the oracle's N, each projection is one fp32-accumulated dot product rounded once
    with torch.no_grad():
        g1 = F.linear(b(d["n"]), b(p.w_in[0])).double().numpy()
    assert np.all(np.abs(g1 - d["pre"][0]) <= one_ulp(d["pre"][0]))
    # the whole output: PyTorch rounds more often (SiLU, product, projection,
    # bias and residual adds each round to bf16); the gap stays inside the
    # bf16 tolerance
    rho = np.sqrt(np.mean(d["out"] ** 2))
    err = np.max(np.abs(out.double().numpy() - d["out"]) / np.maximum(np.abs(d["out"]), rho))
    assert err < 2e-2


def _floored(got, ref, rowwise):
    ref = np.asarray(ref, dtype=np.float64)
    rho = np.sqrt(np.mean(ref * ref, axis=-1, keepdims=True)) if rowwise else np.sqrt(np.mean(ref * ref))
    return float(np.max(np.abs(np.asarray(got, dtype=np.float64) - ref) / np.maximum(np.abs(ref), rho)))


def _bf16_block_case(act):
    rng = np.random.default_rng(43)
    T, H, Fw = 48, 64, 96
    x = _torch_bf16(rng.standard_normal((T, H)))
    if act == "swiglu":
        w_in, b_in = _torch_bf16(rng.standard_normal((2, Fw, H)) * 0.15), None
    else:
        w_in, b_in = _torch_bf16(rng.standard_normal((Fw, H)) * 0.15), _torch_bf16(0.2 * rng.standard_normal(Fw))
    p = Params(_torch_bf16(1 + 0.2 * rng.standard_normal(H)), w_in, _torch_bf16(rng.standard_normal((H, Fw)) * 0.1),
               _torch_bf16(0.1 * rng.standard_normal(H)), b_in)
    return x, p


@pytest.mark.parametrize("act", ["swiglu", "gelu"])
def test_bf16_backward_matches_torch_bf16_autograd(act):
    """Where the bf16 storage model's backward rounds, against PyTorch's CPU
    bf16 autograd of the page's block (bf16 tensors, fp32 accumulation inside
    each op, d out = out).

    Per op: each backward op of PyTorch is fed the storage model's own stored
    inputs (its out, N, pre-activations, pre-activation gradients, dN) and its
    result agrees with the model's within the floored bf16 bound 2e-2:
    activation backward (dg, du | dh), the expansion's input and weight
    gradients, the down projection's input, weight and bias gradients, and
    RMSNorm's backward plus the residual.  PyTorch's activation backward is
    three roundings, R(R(R(da) u) SiLU'(g)) (R(R(da) gelu'(h)) for GeLU),
    to within one bf16 place, where the model rounds the stored gradient once.
    End to end, PyTorch rounds more often (SiLU, the product, da, every op's
    output), so its whole step is not within 2e-2 of either model at these
    magnitudes; it is closer to the storage model than to the exact oracle on
    every stored backward tensor."""
    x, p = _bf16_block_case(act)
    H = x.shape[1]
    R = oracle.bf16_round
    d = oracle.dense_step(x, p, act, 1e-6, 0.1, storage="bf16")
    e = oracle.dense_step(x, p, act, 1e-6, 0.1)
    bt = lambda a: torch.from_numpy(np.asarray(a, dtype=np.float32)).to(torch.bfloat16)
    leaf = lambda a: bt(a).requires_grad_(True)
    c = lambda t: t.detach().double().numpy()
    gr = d["grads"]
    # down projection: out = x + A Wd^T + b, upstream d out = out
    at, wd, bd = leaf(d["a"]), leaf(p.w_down), leaf(p.b_down)
    F.linear(at, wd, bd).backward(bt(d["out"]))
    assert _floored(c(at.grad), d["da"], True) < 2e-2
    assert _floored(c(wd.grad), gr["w_down"], False) < 2e-2
    assert _floored(c(bd.grad), gr["b_down"], False) < 2e-2
    # activation backward on the model's stored pre-activations and PyTorch's da
    pre_t = [leaf(v) for v in d["pre"]]
    a_t = F.silu(pre_t[0]) * pre_t[1] if act == "swiglu" else F.gelu(pre_t[0])
    da_t = at.grad
    a_t.backward(da_t)
    da_r = c(da_t)
    if act == "swiglu":
        g, u = d["pre"]
        model = R(R(da_r * u) * oracle.silu_grad(g))
    else:
        (h,) = d["pre"]
        model = R(da_r * oracle.gelu_grad(h))
    # PyTorch forms SiLU'/gelu' in fp32, the model here in fp64: a value that
    # lies within fp32 rounding of a bf16 midpoint may land one place away
    got = c(pre_t[0].grad)
    one_ulp = np.ldexp(1.0, np.frexp(np.abs(model))[1] - 8)
    assert np.all(np.abs(got - model) <= one_ulp)
    assert np.mean(got == model) > 0.99
    for t, ref in zip(pre_t, d["d_pre"]):
        assert _floored(c(t.grad), ref, True) < 2e-2
    # expansion backward on the model's stored N and pre-activation gradients
    nt = leaf(d["n"])
    if act == "swiglu":
        wg, wu = leaf(p.w_in[0]), leaf(p.w_in[1])
        torch.autograd.backward([F.linear(nt, wg), F.linear(nt, wu)], [bt(v) for v in d["d_pre"]])
        assert _floored(c(wg.grad), gr["w_in"][0], False) < 2e-2
        assert _floored(c(wu.grad), gr["w_in"][1], False) < 2e-2
    else:
        w1, b1 = leaf(p.w_in), leaf(p.b_in)
        F.linear(nt, w1, b1).backward(bt(d["d_pre"][0]))
        assert _floored(c(w1.grad), gr["w_in"], False) < 2e-2
        assert _floored(c(b1.grad), gr["b_in"], False) < 2e-2
    assert _floored(c(nt.grad), d["dN"], True) < 2e-2
    # RMSNorm backward on the model's dN, then the residual branch (d out = out)
    xt, wt = leaf(x), leaf(p.norm_w)
    F.rms_norm(xt, (H,), wt, eps=1e-6).backward(bt(d["dN"]))
    assert _floored(c(bt(c(xt.grad) + d["out"])), d["dx"], True) < 2e-2
    assert _floored(c(wt.grad), gr["norm_w"], False) < 2e-2
    # the whole step in PyTorch bf16: closer to the storage model than to the exact oracle
    xt, wt, wd, bd = leaf(x), leaf(p.norm_w), leaf(p.w_down), leaf(p.b_down)
    n = F.rms_norm(xt, (H,), wt, eps=1e-6)
    n.retain_grad()
    if act == "swiglu":
        wg, wu = leaf(p.w_in[0]), leaf(p.w_in[1])
        pre = (F.linear(n, wg), F.linear(n, wu))
        a = F.silu(pre[0]) * pre[1]
    else:
        pre = (F.linear(n, leaf(p.w_in), leaf(p.b_in)),)
        a = F.gelu(pre[0])
    for t in pre:
        t.retain_grad()
    out = xt + F.linear(a, wd, bd)
    out.backward(out.detach())
    l1 = lambda got, ref: float(np.sum(np.abs(c(got) - ref)))
    for t, rs, rx in zip(pre, d["d_pre"], e["d_pre"]):
        assert l1(t.grad, rs) < l1(t.grad, rx)
    assert l1(n.grad, d["dN"]) < l1(n.grad, e["dN"])
    assert l1(xt.grad, d["dx"]) < l1(xt.grad, e["dx"])
    assert l1(out, d["out"]) < l1(out, e["out"])


@pytest.mark.parametrize("act", ["swiglu", "gelu"])
def test_activation_stages_match_autograd(act):
    """activation_fwd / activation_bwd (the stages the stage-wise GPU checks
    call on their own) against PyTorch's routines and autograd in float64."""
    rng = np.random.default_rng(44)
    pre = tuple(rng.standard_normal((7, 11)) * 3 for _ in range(2 if act == "swiglu" else 1))
    da = rng.standard_normal((7, 11))
    tp = [torch.tensor(v, requires_grad=True) for v in pre]
    a = F.silu(tp[0]) * tp[1] if act == "swiglu" else F.gelu(tp[0])
    a.backward(torch.tensor(da))
    np.testing.assert_allclose(oracle.activation_fwd(pre, act), a.detach().numpy(), rtol=1e-13, atol=1e-15)
    for got, t in zip(oracle.activation_bwd(da, pre, act), tp):
        np.testing.assert_allclose(got, t.grad.numpy(), rtol=1e-12, atol=1e-14)
