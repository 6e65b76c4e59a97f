"""The page's equivalence harness, on the GPU path.

    python -m tensor_transformer_mlp_rmsnorm_amd.fixture --mode MODE [--weights workload|unit]

"Megatron tensor-parallel MLP" (synapticradio.com), sections "Reproduce one
dense training step" and "Remove each collective": one training step of the
dense block and of its tensor-parallel form, compared field by field.  Here
both run on the GPU through the library: the dense reference is the
unsharded step (S = 1), the tensor-parallel form is S = 2 shards run one after
the other with the two boundary sums (tp_partial_sum), in one of three modes:

  equivalence              both sums performed
  missing_forward_reduce   each shard takes its own partial as the whole
                           output (out_s = x + z_s + b_down), its own loss
                           and backward; the backward sum is kept
  missing_backward_reduce  the forward sum is kept; each shard feeds its own
                           dN_s into RMSNorm's backward

Each shard then takes one SGD step with its own gradients.  The record has
the page's keys: the max-abs difference of every compared quantity, the
maximum over the shards, and ``passed`` (every difference within the fp32
tolerance 1e-5).  The workload is the tiny fp32 block (4 tokens, hidden 8,
FFN 16, two shards of 8 channels); ``--weights unit`` redraws the weights at
unit scale (N(0, 1/fan_in)-like std 0.3, with a perturbed norm weight and
bias) so that the ablations move the record by O(0.1 - 1), as on the page.

The differences are measurement of the harness, computed on the host from
the GPU's outputs; every step of the method itself runs in libtpmlp.
"""

from __future__ import annotations

import argparse
import dataclasses
import json
import sys

import torch

from . import _lib as L
from .step import MODES, ShardedStep

FP32_TOL = 1e-5
RECORD_KEYS = ("forward_max_abs_diff", "loss_abs_diff", "input_grad_max_abs_diff", "norm_grad_max_abs_diff",
               "gate_up_grad_max_abs_diff", "down_grad_max_abs_diff", "down_bias_grad_max_abs_diff",
               "post_step_weight_max_abs_diff")


def _loss(out: torch.Tensor) -> float:
    """The page's scalar loss for d out = out: sum(out^2) / 2 (fp64 on the host)."""
    o = out.detach().double().cpu()
    return float(0.5 * torch.sum(o * o))


def _max_abs(pairs) -> float:
    return float(max((torch.max(torch.abs(a.detach().double().cpu() - b.detach().double().cpu())).item()
                      if a.numel() else 0.0) for a, b in pairs))


def _sharded_updates(st: ShardedStep, mode: str):
    """Per shard: its own SGD step (tp_mlp_sgd_step_multi) on the replicated
    parameters with its own replicated-parameter gradients and on its local
    slices; returns a list over shards of dicts of the updated tensors."""
    fp = st.w.dtype == "fp32"
    assert fp, "the page's harness is fp32"
    res = []
    for s, sh in enumerate(st.shards):
        if mode == "equivalence":
            d_nw, d_bd = st.d_norm_w, st.d_b_down
        else:
            d_nw, d_bd = st._abl["d_norm_w"][s], st._abl["d_b_down"][s]
        new = {"norm_w": torch.empty_like(st.norm_w), "b_down": torch.empty_like(st.b_down),
               "w_in": torch.empty_like(sh["w_in"]), "w_down": torch.empty_like(sh["w_down"])}
        lst = [(st.norm_w, new["norm_w"], d_nw, None, None, st.norm_w.numel()),
               (st.b_down, new["b_down"], d_bd, None, None, st.b_down.numel()),
               (sh["w_in"], new["w_in"], sh["d_w_in"], None, None, sh["w_in"].numel()),
               (sh["w_down"], new["w_down"], sh["d_w_down"], None, None, sh["w_down"].numel())]
        L.tp_mlp_sgd_step_multi(lst, L.F32, st.w.lr, stream=st.stream)
        res.append(new)
    return res


def run_record(w, tensors: dict, mode: str, device: str = "cuda") -> dict:
    """The page's comparison record for workload ``w`` (SwiGLU, fp32, S
    shards) on ``tensors`` (synth.draw), GPU S-shard step in ``mode`` against
    the GPU unsharded step."""
    if mode not in MODES:
        raise ValueError(mode)
    if w.dtype != "fp32" or w.act != "swiglu":
        raise ValueError("the page's harness runs the fp32 SwiGLU block")
    dense_w = dataclasses.replace(w, shards=1, shards_run=None)
    dense = ShardedStep(dense_w, tensors, device=device, out_of_place_sgd=True)
    dense.step()
    sh = ShardedStep(w, tensors, device=device, out_of_place_sgd=True)
    sh.step(mode, update=False)
    news = _sharded_updates(sh, mode)
    torch.cuda.synchronize()

    S, F = len(sh.shards), w.ffn_local
    fwd_abl = mode == "missing_forward_reduce"
    per_out = sh._abl["out"] if fwd_abl else [sh.out] * S
    if mode == "equivalence":
        dxs, dws, dbs = [sh.dx] * S, [sh.d_norm_w] * S, [sh.d_b_down] * S
    else:
        dxs, dws, dbs = sh._abl["dx"], sh._abl["d_norm_w"], sh._abl["d_b_down"]
    dsh = dense.shards[0]
    sl = lambda s: slice(s * F, (s + 1) * F)
    rec = {"mode": mode, "world_size": S}
    rec["forward_max_abs_diff"] = _max_abs([(o, dense.out) for o in per_out])
    rec["loss_abs_diff"] = max(abs(_loss(o) - _loss(dense.out)) for o in per_out)
    rec["input_grad_max_abs_diff"] = _max_abs([(d, dense.dx) for d in dxs])
    rec["norm_grad_max_abs_diff"] = _max_abs([(d, dense.d_norm_w) for d in dws])
    rec["gate_up_grad_max_abs_diff"] = _max_abs([(sh.shards[s]["d_w_in"], dsh["d_w_in"][:, sl(s), :])
                                                 for s in range(S)])
    rec["down_grad_max_abs_diff"] = _max_abs([(sh.shards[s]["d_w_down"], dsh["d_w_down"][:, sl(s)])
                                              for s in range(S)])
    rec["down_bias_grad_max_abs_diff"] = _max_abs([(d, dense.d_b_down) for d in dbs])
    post = []
    for s, nw in enumerate(news):
        post += [(nw["norm_w"], dense.new["norm_w"]), (nw["b_down"], dense.new["b_down"]),
                 (nw["w_in"], dense.new["w_in.0"][:, sl(s), :]), (nw["w_down"], dense.new["w_down.0"][:, sl(s)])]
    rec["post_step_weight_max_abs_diff"] = _max_abs(post)
    rec["passed"] = all(rec[k] <= FP32_TOL for k in RECORD_KEYS)
    return rec


def tiny_inputs(weights: str = "workload"):
    """The tiny fp32 workload and its tensors; ``weights="unit"`` redraws the
    weights at unit scale (std 0.3) with a perturbed norm weight and bias."""
    import synth

    w = synth.workload("tiny_fp32_tp2")
    if weights == "unit":
        w = dataclasses.replace(w, name="tiny_fp32_tp2_unit", w_std=0.3, seed=7)
        return w, synth.draw(w, perturb=True)
    if weights != "workload":
        raise ValueError(weights)
    return w, synth.draw(w)


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--mode", choices=MODES, default="equivalence")
    ap.add_argument("--weights", choices=("workload", "unit"), default="workload")
    args = ap.parse_args(argv)
    if not torch.cuda.is_available():
        print(json.dumps({"error": "no GPU visible"}), flush=True)
        return 1
    w, t = tiny_inputs(args.weights)
    print(json.dumps(run_record(w, t, args.mode, device="cuda:0")), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
