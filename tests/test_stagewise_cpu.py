"""The stage-wise checker (tests/stagewise.py) on the CPU: fed the oracle's
own sharded step laid out as the GPU stores it, every stage passes; with
one planted wrong element in any stage's output, that stage fails."""

import numpy as np
import pytest
import torch

import oracle
import synth
from oracle.mlp import Params
from stagewise import STAGES, run_stage


def _host_from_oracle(w, t):
    """The tensors ShardedStep would store, taken from oracle.sharded_step
    (fp64 arithmetic, the workload's storage model), in the GPU's dtypes."""
    c = synth.to_numpy64
    p = Params(c(t["norm_w"]), c(t["w_in"]), c(t["w_down"]), c(t["b_down"]), c(t["b_in"]))
    storage = "bf16" if w.dtype == "bf16" else "exact"
    sh = oracle.sharded_step(c(t["x"]), p, w.act, w.eps, w.lr, w.shards, storage=storage)
    act_t = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    A = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(act_t)      # a stored activation
    G = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(torch.float32)  # fp32 buffers
    r0 = sh["ranks"][0]
    h = {"normed": A(r0["n"]), "rstd": G(r0["rstd"]), "out": A(r0["out"]), "dx": A(r0["dx"]),
         "d_norm_w": G(r0["grads"]["norm_w"]), "d_b_down": G(r0["grads"]["b_down"]), "shards": [],
         "new": {"norm_w": A(r0["new_params"].norm_w), "b_down": A(r0["new_params"].b_down)},
         "new_masters": {}, "masters": {}}
    h["dN"] = G(r0["dN"])
    for s, rk in enumerate(sh["ranks"]):
        lp = rk["params"]
        h["shards"].append({
            "pre": A(np.concatenate(rk["pre"], axis=1)), "act": A(rk["a"]),
            "z": None if w.shards == 1 else G(rk["z"]), "d_pre": A(np.concatenate(rk["d_pre"], axis=1)),
            "d_w_in": G(rk["grads"]["w_in"]), "d_b_in": None if lp.b_in is None else G(rk["grads"]["b_in"]),
            "d_w_down": G(rk["grads"]["w_down"]), "dN_part": G(rk["dN_partial"]), "w_in": None, "w_down": None,
            "b_in": None})
        h["new"][f"w_in.{s}"] = A(rk["new_params"].w_in)
        h["new"][f"w_down.{s}"] = A(rk["new_params"].w_down)
        if lp.b_in is not None:
            h["new"][f"b_in.{s}"] = A(rk["new_params"].b_in)
    if w.master:
        dense_new = {}
        # masters: exact upcasts of the bf16 parameters, updated in fp32 and rounded for the copy
        for k in list(h["new"]):
            base, _, s = k.partition(".")
            if base == "norm_w":
                pm, g = p.norm_w, r0["grads"]["norm_w"]
            elif base == "b_down":
                pm, g = p.b_down, r0["grads"]["b_down"]
            else:
                rk = sh["ranks"][int(s)]
                pm, g = getattr(rk["params"], base), rk["grads"][base]
            h["masters"][k] = G(pm)
            h["new_masters"][k] = G(pm - w.lr * g)
            dense_new[k] = A(oracle.bf16_round(h["new_masters"][k].double().numpy()))
        h["new"] = dense_new
    return h


CASES = [
    synth.Workload("cpu_swiglu_S2", tokens=300, hidden=136, ffn_full=272, shards=2, act="swiglu", dtype="bf16",
                   w_std=0.05, seed=7),
    synth.Workload("cpu_gelu_S1", tokens=130, hidden=72, ffn_full=96, shards=1, act="gelu", dtype="bf16",
                   w_std=0.05, seed=8),
    synth.Workload("cpu_master_S1", tokens=96, hidden=64, ffn_full=72, shards=1, act="swiglu", dtype="bf16",
                   w_std=0.05, seed=5, master=True, outlier_frac=0.05),
    synth.Workload("cpu_fp32_S2", tokens=40, hidden=24, ffn_full=32, shards=2, act="swiglu", dtype="fp32",
                   w_std=0.1, seed=9),
]


@pytest.mark.parametrize("w", CASES, ids=[c.name for c in CASES])
def test_every_stage_passes_on_the_oracle(w):
    t = synth.draw(w, perturb=True)
    h = _host_from_oracle(w, t)
    for stage in STAGES:
        report = {}
        run_stage(stage, w, t, h, report)
        assert all(v < 5e-3 for v in report.values()), (stage, report)


# (stage, how to reach the tensor in h, index of the element to break)
PLANTS = [
    ("F1", lambda h: h["normed"], (17, 5)),
    ("F2", lambda h: h["shards"][1]["pre"], (250, 3)),
    ("F2", lambda h: h["shards"][0]["act"], (0, 135)),
    ("F3", lambda h: h["shards"][1]["z"], (299, 0)),
    ("F4", lambda h: h["out"], (123, 77)),
    ("B1", lambda h: h["shards"][0]["d_pre"], (299, 271)),
    ("B2", lambda h: h["shards"][1]["d_w_down"], (135, 0)),
    ("B3", lambda h: h["shards"][0]["dN_part"], (64, 64)),
    ("B5", lambda h: h["dN"], (1, 2)),
    ("B4", lambda h: h["shards"][1]["d_w_in"], (1, 67, 100)),
    ("B6", lambda h: h["dx"], (299, 135)),
    ("B6", lambda h: h["d_norm_w"], (3,)),
    ("U1", lambda h: h["new"]["w_in.1"], (0, 3, 3)),
]


@pytest.mark.parametrize("stage,get,idx", PLANTS, ids=[f"{p[0]}-{i}" for i, p in enumerate(PLANTS)])
def test_a_planted_wrong_element_fails_its_stage(stage, get, idx):
    w = CASES[0]
    t = synth.draw(w, perturb=True)
    h = _host_from_oracle(w, t)
    tensor = get(h)
    ref = tensor.double()
    rms = float(torch.sqrt(torch.mean(ref * ref)))
    tensor[idx] = tensor[idx] + 0.1 * rms  # 10% of the tensor's RMS on one element
    with pytest.raises(AssertionError):
        run_stage(stage, w, t, h, {})
