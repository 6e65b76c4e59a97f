"""Parity of the optimiser path (through the C ABI) with the CPU oracle:
gradient accumulation over microbatches (TP_MLP_ACCUMULATE_GRADS), the
global gradient norm and clip coefficient (tp_mlp_clip_grad_norm) and AdamW
(tp_mlp_adamw_step_multi).

AdamW is checked one step at a time from the GPU's own state (the oracle
takes the GPU's parameters, moments and gradients of that step in fp64), so
each step is compared to the exact update of the same inputs: fp32 state to
a few fp32 ulps, bf16 parameters to one bf16 rounding.  Tolerances of the
accumulated gradients: tests/tolerance.py.
"""

import sys

import numpy as np
import pytest
import torch

import oracle
import synth
from oracle.mlp import Params
from tolerance import check

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from tensor_transformer_mlp_rmsnorm_amd import _lib
    _lib.lib()  # must load: there is no fallback
    yield
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def f64(t):
    return t.detach().double().cpu().numpy()


SIZES = [1, 7, 8, 2049, 5003]


def _grads(gen, sizes, scale):
    return [(torch.randn(n, generator=gen) * scale).cuda() for n in sizes]


@pytest.mark.parametrize("kind", ["fp32", "bf16_master", "bf16"])
def test_adamw_matches_oracle_step_by_step(kind):
    from tensor_transformer_mlp_rmsnorm_amd import _lib as L
    say(f"[gpu] adamw {kind} sizes={SIZES}")
    gen = torch.Generator().manual_seed(11)
    pdt = torch.float32 if kind == "fp32" else torch.bfloat16
    params = [torch.randn(n, generator=gen).to(pdt).cuda() for n in SIZES]
    masters = [p.float().clone() for p in params] if kind == "bf16_master" else None
    ms = [torch.zeros(n, device="cuda") for n in SIZES]
    vs = [torch.zeros(n, device="cuda") for n in SIZES]
    norm, coef = torch.zeros(1, device="cuda"), torch.zeros(1, device="cuda")
    ws = torch.empty(max(16, L.tp_mlp_clip_grad_norm_workspace_bytes(SIZES)), dtype=torch.uint8, device="cuda")
    lr, wd, b1, b2, eps, max_norm = 1e-2, 0.1, 0.9, 0.95, 1e-8, 2.0
    for step in range(1, 4):
        grads = _grads(gen, SIZES, 0.3 * step)
        theta0 = [f64(m) for m in masters] if masters else [f64(p) for p in params]
        m0, v0 = [f64(m) for m in ms], [f64(v) for v in vs]
        L.tp_mlp_clip_grad_norm(grads, SIZES, max_norm, norm, coef, ws)
        hp = L.make_adamw_hparams(lr, step, wd, b1, b2, eps)
        if masters:
            rows = [(None, p, g, mm, mm, m, v, p.numel()) for p, g, mm, m, v in zip(params, grads, masters, ms, vs)]
        else:
            rows = [(p, p, g, None, None, m, v, p.numel()) for p, g, m, v in zip(params, grads, ms, vs)]
        L.tp_mlp_adamw_step_multi(rows, L.F32 if kind == "fp32" else L.BF16, hp, grad_scale=coef)
        torch.cuda.synchronize()
        ref = oracle.adamw_step(dict(enumerate(theta0)), dict(enumerate(f64(g) for g in grads)),
                                dict(enumerate(m0)), dict(enumerate(v0)), step, lr, wd, max_norm, b1, b2, eps)
        assert float(norm) == pytest.approx(ref["norm"], rel=1e-6)
        assert ref["coef"] < 1 and float(coef) == pytest.approx(ref["coef"], rel=1e-6)
        for i in range(len(SIZES)):
            np.testing.assert_allclose(f64(ms[i]), ref["m"][i], rtol=1e-5, atol=1e-9)
            np.testing.assert_allclose(f64(vs[i]), ref["v"][i], rtol=1e-5, atol=1e-12)
            r = ref["params"][i]
            if kind == "fp32":
                np.testing.assert_allclose(f64(params[i]), r, rtol=0, atol=2e-6 * max(1.0, np.abs(r).max()))
            elif kind == "bf16_master":
                np.testing.assert_allclose(f64(masters[i]), r, rtol=0, atol=2e-6 * max(1.0, np.abs(r).max()))
                # the bf16 parameter is the rounding of its master
                assert torch.equal(params[i], masters[i].to(torch.bfloat16))
            else:
                # one bf16 rounding of the fp32 result: at most one bf16 ulp from the exact value
                got, rr = f64(params[i]), oracle.bf16_round(r)
                ulp = np.abs(rr) * 2.0 ** -7 + 1e-30
                assert np.all(np.abs(got - rr) <= ulp), f"tensor {i}: bf16 update off by more than one ulp"


def test_clip_grad_norm_matches_oracle_and_is_deterministic():
    from tensor_transformer_mlp_rmsnorm_amd import _lib as L
    gen = torch.Generator().manual_seed(12)
    sizes = [0, 1, 5, 2048, 2049, 70001] + [(97 * k) % 3001 for k in range(34)]  # 40 tensors: two launches
    grads = [(torch.randn(n, generator=gen) * (1 + k % 5)).cuda() for k, n in enumerate(sizes)]
    say(f"[gpu] clip_grad_norm {len(sizes)} tensors, {sum(sizes)} elements")
    ws = torch.empty(max(16, L.tp_mlp_clip_grad_norm_workspace_bytes(sizes)), dtype=torch.uint8, device="cuda")
    ref_norm = oracle.global_grad_norm([f64(g) for g in grads])
    outs = []
    for max_norm in (1.0, 1.0, 0.0, 1e9):
        norm, coef = torch.zeros(1, device="cuda"), torch.zeros(1, device="cuda")
        L.tp_mlp_clip_grad_norm(grads, sizes, max_norm, norm, coef, ws)
        torch.cuda.synchronize()
        assert float(norm) == pytest.approx(ref_norm, rel=1e-6)
        assert float(coef) == pytest.approx(oracle.clip_coefficient(ref_norm, max_norm), rel=1e-6)
        outs.append((norm.clone(), coef.clone()))
    assert torch.equal(outs[0][0], outs[1][0]) and torch.equal(outs[0][1], outs[1][1])
    assert float(outs[2][1]) == 1.0 and float(outs[3][1]) == 1.0


ACCUM = [
    # name,                 T,   H,   F_full, S, act,      dtype,  M, master
    ("fp32_tiny_S2_M2", 4, 8, 16, 2, "swiglu", "fp32", 2, False),
    ("fp32_gelu_S1_M2", 131, 72, 200, 1, "gelu", "fp32", 2, False),
    ("bf16_swiglu_S2_M3", 300, 136, 144, 2, "swiglu", "bf16", 3, False),
    ("bf16_gelu_S2_M4", 129, 264, 272, 2, "gelu", "bf16", 4, False),
    ("bf16_swiglu_S1_M4_master", 257, 64, 128, 1, "swiglu", "bf16", 4, True),
]


@pytest.mark.parametrize("case", ACCUM, ids=[c[0] for c in ACCUM])
def test_microbatch_accumulation_matches_oracle(case):
    """M microbatches, gradients accumulated in fp32 on the device, against
    the oracle's per-microbatch gradients summed in order; the outputs of
    every row against the whole-batch step (rows are independent)."""
    from tensor_transformer_mlp_rmsnorm_amd.step import ShardedStep
    name, T, H, Ff, S, act, dt, M, master = case
    w = synth.Workload(name, tokens=T, hidden=H, ffn_full=Ff, shards=S, act=act, dtype=dt, w_std=0.05,
                       seed=200 + T, master=master)
    say(f"[gpu] accumulate {name}: T={T} H={H} F_full={Ff} S={S} {act} {dt} M={M}")
    t = synth.draw(w, perturb=True)
    st = ShardedStep(w, t, out_of_place_sgd=True)
    for sh in st.shards:  # stale values must not leak into the first microbatch
        for k in ("d_w_in", "d_w_down", "d_b_in"):
            if sh[k] is not None:
                sh[k].fill_(7.0)
    st.d_norm_w.fill_(7.0)
    st.d_b_down.fill_(7.0)
    st.step(microbatches=M, update=False)
    torch.cuda.synchronize()
    res = st.results()
    x = synth.to_numpy64(t["x"])
    p = Params(*(synth.to_numpy64(t[k]) for k in ("norm_w", "w_in", "w_down", "b_down", "b_in")))
    storage = "bf16" if dt == "bf16" else "exact"
    acc = oracle.accumulated_grads(x, p, act, w.eps, M, storage=storage)
    tol = dt if (dt == "bf16" or name.startswith("fp32_tiny")) else "fp32-scaled"
    report = {}
    check("d_w_in", res["d_w_in"], acc["w_in"], tol, report=report)
    check("d_w_down", res["d_w_down"], acc["w_down"], tol, report=report)
    check("d_norm_w", res["d_norm_w"], acc["norm_w"], tol, report=report)
    check("d_b_down", res["d_b_down"], acc["b_down"], tol, report=report)
    if act == "gelu":
        check("d_b_in", res["d_b_in"], acc["b_in"], tol, report=report)
    whole = oracle.dense_step(x, p, act, w.eps, 0.0, storage=storage)
    check("out", res["out"], whole["out"], tol, rowwise=True, report=report)
    check("dx", res["dx"], whole["dx"], tol, rowwise=True, report=report)
    say(f"  worst: {max(report.items(), key=lambda kv: kv[1])}")


def test_microbatches_then_adamw_step():
    """The whole optimiser path of one global batch: 3 microbatches, the clip
    coefficient, AdamW with fp32 masters.  The accumulated gradients are
    checked against the oracle's; the update against the oracle's AdamW on
    the GPU's own gradients (the first step moves each weight by about
    lr * sign(g), so gradients within rounding noise of zero are compared
    where they are produced, not through the sign)."""
    from tensor_transformer_mlp_rmsnorm_amd.step import ShardedStep
    w = synth.Workload("adamw_path", tokens=192, hidden=128, ffn_full=256, shards=2, act="swiglu", dtype="bf16",
                       w_std=0.05, seed=31, master=True)
    say("[gpu] microbatches + clip + adamw: T=192 H=128 F_full=256 S=2 bf16 masters M=3")
    t = synth.draw(w, perturb=True)
    st = ShardedStep(w, t, out_of_place_sgd=True)
    st.step(microbatches=3, update=False)
    lr, wd, max_norm = 1e-3, 0.1, 1.0
    st.adamw(lr, weight_decay=wd, max_norm=max_norm)
    torch.cuda.synchronize()
    res = st.results()
    x = synth.to_numpy64(t["x"])
    p = Params(*(synth.to_numpy64(t[k]) for k in ("norm_w", "w_in", "w_down", "b_down", "b_in")))
    acc = oracle.accumulated_grads(x, p, w.act, w.eps, 3, storage="bf16")
    names = ["norm_w", "w_in", "w_down", "b_down"]
    for k in names:
        check(f"d_{k}", res[f"d_{k}"], acc[k], "bf16")
    gpu_g = {k: f64(res[f"d_{k}"]) for k in names}
    zeros = {k: np.zeros_like(getattr(p, k)) for k in names}
    ref = oracle.adamw_step({k: getattr(p, k) for k in names}, gpu_g, zeros, zeros, 1, lr, wd, max_norm)
    assert ref["coef"] < 1
    assert float(st.grad_norm) == pytest.approx(ref["norm"], rel=1e-6)
    assert float(st.clip_coef) == pytest.approx(ref["coef"], rel=1e-6)
    for k in names:
        r = ref["params"][k]
        np.testing.assert_allclose(f64(res[f"master_{k}"]), r, rtol=0, atol=2e-6 * max(1.0, np.abs(r).max()))
        assert torch.equal(res[f"new_{k}"], res[f"master_{k}"].to(torch.bfloat16).float())
