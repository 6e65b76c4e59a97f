"""Benchmark: one training step of a Llama-3-8B-shaped TP=8 MLP layer on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

A step is the whole path for one batch: RMSNorm, for each of the 8 shards the
gate/up GEMM with SwiGLU and the down GEMM to an fp32 partial, the forward
partial sum with residual and bias, for each shard the four backward GEMMs,
the backward partial sum, RMSNorm's backward, and SGD on every parameter.
Inputs are resident in HBM before the timed region; SGD writes new parameter
buffers so every timed step does identical work.

Prints one JSON line.  `value` is the algorithmic GEMM TFLOP/s of the whole
step (18 T H F_full flops per step for SwiGLU); per-kernel times come from
HIP events the library records on its launch stream during the timed steps.
The CPU oracle is timed on a bounded token slice of the same workload.

After the timed step, `other_workloads` times the other bf16 workloads the
same way (GPT-2-small GeLU tp=1, one Llama-3-70B TP=8 rank, Llama-3-8B full
width with fp32 masters), each with its dominant kernel's roofline, and
`optimizer_path` reports the optimiser side on the same
workload (unless --no-extras): the global-norm clip plus AdamW over every
shard's parameters (each kernel against HBM bandwidth), and the step run as 2
microbatches whose weight gradients accumulate in fp32.  `sequence_parallel`
times the same step in the sequence-parallel layout (norm, residual and bias
on each rank's token rows; reduce-scatter and all-gather at the boundaries).
`fp8_path` times the step with every GEMM on FP8 codes (delayed scaling),
its GEMMs against the fp8 MFMA peak and its casts against HBM bandwidth.
`attention_path` times the tensor-parallel attention sublayer's step on the
Llama-3-8B TP=8 attention shape (32 query / 8 KV heads of 128, 2 causal
sequences of 4096), each kernel against the bf16 peak.
"""

from __future__ import annotations

import argparse
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "fwd+bwd TFLOP/s per TP-shard SwiGLU MLP, % of bf16 MFMA peak; tokens/s"
PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_FP32_TFLOPS = 157.3    # MI355X fp32 matrix
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
PEAK_FP8_TFLOPS = 5000.0    # MI355X dense fp8 MFMA
# the bf16 workloads timed besides the main one (the tiny fp32 one is correctness only)
OTHER_WORKLOADS = ("gpt2s_gelu_tp1", "llama3_70b_tp8_rank", "llama3_8b_tp1_master")


def gemm_flops(w) -> dict:
    """Algorithmic flops of one launch of each GEMM, by kernel name (a
    weight-gradient GEMM that applies the SGD update as it forms the gradient
    is named with the suffix _sgd)."""
    T, H, F = w.tokens, w.hidden, w.ffn_local
    if w.act == "swiglu":
        fl = {"gemm_gate_up_swiglu": 2 * T * 2 * F * H, "gemm_down_partial": 2 * T * H * F,
              "gemm_down_residual": 2 * T * H * F, "gemm_dact_swiglu_bwd": 2 * T * F * H,
              "gemm_wgrad_down": 2 * H * F * T, "gemm_dgrad_normed": 2 * T * H * 2 * F,
              "gemm_wgrad_gate_up": 2 * 2 * F * H * T}
    else:
        fl = {"gemm_fc1_gelu": 2 * T * F * H, "gemm_down_partial": 2 * T * H * F,
              "gemm_down_residual": 2 * T * H * F, "gemm_dact_gelu_bwd": 2 * T * F * H,
              "gemm_wgrad_down": 2 * H * F * T, "gemm_dgrad_normed": 2 * T * H * F, "gemm_wgrad_fc1": 2 * F * H * T}
    for k in ("gemm_wgrad_down", "gemm_wgrad_gate_up", "gemm_wgrad_fc1"):
        if k in fl:
            fl[k + "_sgd"] = fl[k]
    return fl


def gemm_ksplit(M: int, N: int, K: int) -> int:
    """The library's k-slice count of a bf16 fp32-output GEMM (a function of
    the shape: fewer than 192 tiles of 256 x 256 take the most slices, at most
    8, that keep one round of 256 CUs and 1024 of k per slice)."""
    tiles = -(-M // 256) * -(-N // 256)
    if tiles >= 192:
        return 1
    ks = 1
    while ks < 8 and tiles * (ks + 1) <= 256 and K // (ks + 1) >= 1024:
        ks += 1
    return ks


def fused_update(w) -> bool:
    """Whether the step takes the weight matrices' SGD update inside their
    weight-gradient GEMMs (tp_mlp_fused_sgd; the bf16 steps here do)."""
    return w.dtype == "bf16"


def hbm_bytes_per_step(w) -> dict:
    """Algorithmic HBM bytes per step of each bandwidth-bound kernel
    (compulsory reads + writes of its operands), by kernel name."""
    T, H, F, S = w.tokens, w.hidden, w.ffn_local, w.n_run
    es = 2 if w.dtype == "bf16" else 4
    P = 2 * F if w.act == "swiglu" else F
    n_w = S * (P * H + H * F)  # the weight matrices' elements
    n_params = H + H + n_w + S * (F if w.act == "gelu" else 0)
    per_param = (4 + 4 + 4 + es) if w.master else (es + 4 + es)
    n_t = n_w if w.dtype == "bf16" else 0  # the weights' transposed copies, written with the update
    fused = fused_update(w)
    # with the update fused, the separate SGD takes the vectors only; a weight-gradient GEMM with k
    # slices leaves them to sgd_ksplit, which reads the slices and the weight (or master) and writes the
    # weight, its transposed copy (and the master)
    sgd_bytes = (n_params - n_w) * per_param if fused else n_params * per_param + n_t * es
    upd = (4 + 4 + es) if w.master else (es + es)
    ksplit_bytes = 0
    if fused:
        for M, N in ((H, F), (P, H)):
            ks = gemm_ksplit(M, N, T)
            if ks > 1:
                ksplit_bytes += S * M * N * (ks * 4 + upd + es)
    # with the update fused and the w_in gradient GEMM on K-contiguous operands (no masters, T a multiple
    # of 8, k not split), N is transposed once per step
    nt = fused and not w.master and T % 8 == 0 and gemm_ksplit(P, H, T) == 1
    return {
        "transpose_bf16": 2 * T * H * es if nt else 0,
        "sgd_ksplit": ksplit_bytes,
        "rmsnorm_fwd": T * H * 2 * es + 4 * T + H * es,                 # x in, N out, rstd out, w in
        "partial_sum_residual": S * 4 * T * H + 2 * es * T * H + H * es,  # S fp32 partials + x in, out
        "partial_sum": S * 4 * T * H + 4 * T * H,                        # S fp32 partials in, dN out
        # the S fp32 partials of dN (summed as they are read), x, dY in, dx out
        "rmsnorm_bwd": T * H * (4 * S + 3 * es) + 4 * T + H * es,
        "sgd": sgd_bytes,                                                # p (or master), g in; p (+master), W^T out
        # optimiser path: AdamW reads g, m, v and p (or master) and writes m, v, p (+ master)
        "adamw": n_params * ((4 + 4 + 4 + 8 + 8 + es) if w.master else (2 * es + 4 + 8 + 8)),
        "grad_norm": n_params * 4,                                         # every fp32 gradient read once
    }


def roofline_entry(name, launches, total_ms, w, steps):
    secs = total_ms / 1e3
    fl = gemm_flops(w)
    if name in fl:
        peak = PEAK_BF16_TFLOPS if w.dtype == "bf16" else PEAK_FP32_TFLOPS
        ach = fl[name] * launches / secs / 1e12
        return {"bound": "mfma", "achieved": ach, "peak": peak, "unit": "TFLOP/s", "frac": ach / peak,
                "per_launch": fl[name], "avg_ms": total_ms / launches, "launches": launches}
    by = hbm_bytes_per_step(w)
    if name in by:
        ach = by[name] * steps / secs / 1e9
        return {"bound": "hbm", "achieved": ach, "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": ach / PEAK_HBM_GBS,
                "per_launch": by[name] * steps // launches, "avg_ms": total_ms / launches, "launches": launches}
    return {"bound": None, "avg_ms": total_ms / launches, "launches": launches}


KERNEL_SOURCES = ("tensor_transformer_mlp_rmsnorm_amd/csrc/gemm_bf16.hip", "tensor_transformer_mlp_rmsnorm_amd/csrc/common.h",
                  "tensor_transformer_mlp_rmsnorm_amd/csrc/kernels.h")


def kernel_sources_fingerprint() -> str:
    """sha256 of the GEMM sources' code: every line with its // comment and
    trailing blanks removed, empty lines skipped (the sources hold no // inside
    string literals).  A traffic record stays valid across comment edits and
    not across code edits."""
    import hashlib
    import re

    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel)) as f:
            for line in f:
                code = re.sub(r"//.*$", "", line).rstrip()
                if code:
                    h.update(code.encode() + b"\n")
    return h.hexdigest()


def measured_traffic(kernel: str, workload: str):
    """HBM bytes per launch of `kernel` from the committed counter record
    (profiles/traffic_<kernel>_<workload>.json: FETCH_SIZE and WRITE_SIZE
    scaled by a plain-copy calibration), or None when there is no record or
    the kernel code changed since the counters were taken."""
    path = os.path.join(ROOT, "profiles", f"traffic_{kernel}_{workload}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("kernel_sources_sha256") != kernel_sources_fingerprint():
        return None
    return float(rec["traffic_bytes_per_launch"])


def cpu_baseline(w, t, budget_s: float = 15.0) -> dict:
    """The oracle as it stands (fp64 numpy, sharded step) on a token slice of
    the workload, sized to roughly ``budget_s`` of CPU time."""
    import numpy as np

    import oracle
    import synth
    from oracle.mlp import Params

    c = synth.to_numpy64
    p = Params(c(t["norm_w"]), c(t["w_in"]), c(t["w_down"]), c(t["b_down"]), c(t["b_in"]))
    x = c(t["x"])

    def run(tp):
        t0 = time.perf_counter()
        oracle.sharded_step(x[:tp], p, w.act, w.eps, w.lr, w.n_run)
        return time.perf_counter() - t0

    # grow the slice until one run takes at least half the budget (or is the whole batch)
    tp = min(64, w.tokens)
    secs = run(tp)
    while secs < 0.5 * budget_s and tp < w.tokens:
        grow = max(2.0, min(8.0, budget_s / max(secs, 1e-3)))
        tp = min(w.tokens, max(tp + 64, int(tp * grow) // 64 * 64))
        secs = run(tp)
    mult = 18 if w.act == "swiglu" else 12
    flops = mult * tp * w.hidden * w.ffn_local * w.n_run
    try:
        from threadpoolctl import threadpool_info

        cores = max((i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"), default=1)
    except Exception:  # pragma: no cover
        cores = 1
    return {"value": flops / secs / 1e12, "unit": "TFLOP/s", "cores": int(cores), "kind": "oracle",
            "sample": f"oracle.sharded_step (fp64 numpy) on the first {tp} of {w.tokens} tokens, all "
                      f"{w.n_run} shards, full H and F; {secs:.2f} s; tokens/s {tp / secs:.1f}",
            "host_cpus": os.cpu_count(), "cpu_model": cpu_model()}


def optimizer_path(st, w, steps: int, warmup: int) -> dict:
    """The clip + AdamW update (its kernels against HBM bandwidth) and the
    step run as 2 accumulating microbatches, on the benchmark's step object."""
    import torch
    from tensor_transformer_mlp_rmsnorm_amd import _lib as L

    hp = dict(lr=1e-4, weight_decay=0.1, max_norm=1.0)
    st.step(update=False)  # the gradients AdamW reads (a step with the update fused does not write them)
    for _ in range(max(1, warmup)):
        st.adamw(**hp)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        st.adamw(**hp)
    torch.cuda.synchronize()
    upd_ms = (time.perf_counter() - t0) / steps * 1e3
    L.tp_mlp_profile_enable(True)  # per-kernel durations from a second run
    for _ in range(steps):
        st.adamw(**hp)
    torch.cuda.synchronize()
    L.tp_mlp_profile_enable(False)
    prof = L.tp_mlp_profile_entries()
    res = {"update": "global-norm clip (max_norm 1.0) + AdamW (lr 1e-4, wd 0.1), every shard's parameters",
           "update_ms": upd_ms,
           "kernels": {k: roofline_entry(k, n, tot, w, steps) for k, (n, tot) in prof.items()}}
    for _ in range(max(1, warmup)):
        st.step(microbatches=2)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        st.step(microbatches=2)
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) / steps * 1e3
    res["microbatch_step"] = {"microbatches": 2, "tokens_each": w.tokens // 2, "ms_per_step": ms,
                              "tflops": w.flops_per_step / (ms / 1e3) / 1e12,
                              "note": "forward + backward per microbatch, fp32 gradient accumulation, one SGD update"}
    return res


def fp8_cast_bytes(w) -> dict:
    """Algorithmic HBM bytes of one launch of each FP8 cast kernel (bf16 in,
    row codes + transposed codes out), by kernel name.  Per shard the
    weights cast launches twice (w_in, then w_down); their mean is listed."""
    T, H, F = w.tokens, w.hidden, w.ffn_local
    P = 2 * F if w.act == "swiglu" else F
    Tp = (T + 15) // 16 * 16
    both = lambda r, c, rows_t: r * c * 2 + r * c + c * rows_t
    return {"fp8_cast_normed": both(T, H, Tp), "fp8_cast_d_out": both(T, H, Tp), "fp8_cast_act": both(T, F, Tp),
            "fp8_cast_d_pre": both(T, P, Tp), "fp8_cast_weights": (both(P, H, P) + both(H, F, H)) // 2}


def fp8_path(w, t, steps: int, warmup: int) -> dict:
    """The same step with every GEMM on FP8 codes (E4M3 forward, E5M2
    gradients, per-tensor delayed scaling): its time, and each FP8 GEMM
    against the fp8 MFMA peak and each cast against HBM bandwidth."""
    import torch
    from tensor_transformer_mlp_rmsnorm_amd import _lib as L
    from tensor_transformer_mlp_rmsnorm_amd.step import Fp8Step

    st = Fp8Step(w, t, device="cuda:0", out_of_place_sgd=True, fused_sgd=True)
    for _ in range(max(1, warmup)):
        st.step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        st.step()
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) / steps * 1e3
    # the per-kernel durations from a second run with the library's event timing on
    L.tp_mlp_profile_enable(True)
    for _ in range(steps):
        st.step()
    torch.cuda.synchronize()
    L.tp_mlp_profile_enable(False)
    prof = L.tp_mlp_profile_entries()
    del st
    torch.cuda.empty_cache()
    fl = {k + "_fp8": v for k, v in gemm_flops(w).items()}
    by = fp8_cast_bytes(w)
    kernels = {}
    for k, (n, tot) in prof.items():
        secs = tot / 1e3
        if k in fl:
            ach = fl[k] * n / secs / 1e12
            kernels[k] = {"bound": "mfma", "achieved": ach, "peak": PEAK_FP8_TFLOPS, "unit": "TFLOP/s",
                          "frac": ach / PEAK_FP8_TFLOPS, "per_launch": fl[k], "avg_ms": tot / n, "launches": n}
        elif k in by:
            ach = by[k] * n / secs / 1e9
            kernels[k] = {"bound": "hbm", "achieved": ach, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                          "frac": ach / PEAK_HBM_GBS, "per_launch": by[k], "avg_ms": tot / n, "launches": n}
        else:
            kernels[k] = roofline_entry(k, n, tot, w, steps)
    gemm_ms = sum(tot for k, (n, tot) in prof.items() if k in fl) / steps
    return {"recipe": "E4M3 N/weights/activation, E5M2 gradients; delayed scaling, amax history 16, amax shared by "
                      "the shards", "ms_per_step": ms, "tflops": w.flops_per_step / (ms / 1e3) / 1e12,
            "gemm_ms_per_step": gemm_ms,
            "gemm_tflops": w.flops_per_step / (gemm_ms / 1e3) / 1e12 if gemm_ms > 0 else None,
            "gemm_pct_of_fp8_peak": 100.0 * w.flops_per_step / (gemm_ms / 1e3) / 1e12 / PEAK_FP8_TFLOPS
            if gemm_ms > 0 else None, "kernels": kernels}


def attention_flops(aw) -> dict:
    """Algorithmic flops of one launch of each attention-sublayer kernel of
    one shard, by kernel name.  Causal attention touches the
    s (s + 1) / 2 query-key pairs of each sequence: forward 2 products
    (S, PV), backward 4 (dP, dS -> dQ, dK, dV); the dK/dV kernel is charged
    dP, dK and dV, the dQ kernel dQ."""
    T, H, D, S = aw.tokens, aw.hidden, aw.d, aw.shards
    nq, nkv = aw.n_q // S, aw.n_kv // S
    W, Wo = (nq + 2 * nkv) * D, nq * D
    pd = 2 * (aw.batch * aw.seq * (aw.seq + 1) // 2) * D * nq  # one product over the causal pairs
    return {"gemm_qkv": 2 * T * H * W, "gemm_out_proj_partial": 2 * T * H * Wo, "gemm_out_proj_residual": 2 * T * H * Wo,
            "gemm_attn_dgrad_out": 2 * T * H * Wo, "gemm_attn_wgrad_out": 2 * H * Wo * T,
            "gemm_attn_dgrad_normed": 2 * T * W * H, "gemm_attn_wgrad_qkv": 2 * W * H * T,
            "attention_fwd": 2 * pd, "attention_bwd_dkdv": 3 * pd, "attention_bwd_dq": pd}


def attention_hbm_bytes(aw) -> dict:
    """Algorithmic HBM bytes per step of the attention step's bandwidth-bound
    kernels (bf16 storage): the RMSNorm forward, the forward boundary sum, the
    RMSNorm backward with the backward boundary streamed into it (a separate
    dN sum only in the ablation modes) and the SGD over every shard's
    parameters, by kernel name."""
    T, H, S = aw.tokens, aw.hidden, aw.shards
    w_qkv = (aw.n_q + 2 * aw.n_kv) * aw.d * H  # all shards' rows of the fused projection
    w_o = H * aw.n_q * aw.d
    n_params = 2 * H + w_qkv + w_o
    return {"rmsnorm_fwd": T * H * 2 * 2 + 4 * T + 2 * H,
            "partial_sum_residual": S * 4 * T * H + 2 * 2 * T * H + 2 * H,
            "partial_sum": S * 4 * T * H + 4 * T * H,
            # the S fp32 partials of dN (summed as they are read), x, dY in, dx out
            "rmsnorm_bwd": T * H * (4 * S + 3 * 2) + 4 * T + 2 * H,
            "sgd": n_params * (2 + 4 + 2)}


def attention_path(steps: int, warmup: int, name: str = "attn_llama3_8b_tp8") -> dict:
    """The tensor-parallel attention sublayer's step (forward, backward, SGD
    over all shards in sequence) on the Llama-3-8B TP=8 attention shape: its
    time and each kernel against its roofline."""
    import torch
    import synth
    from tensor_transformer_mlp_rmsnorm_amd import _lib as L
    from tensor_transformer_mlp_rmsnorm_amd.step import AttnStep

    aw = synth.attn_workload(name)
    st = AttnStep(aw, synth.draw_attn(aw), device="cuda:0", out_of_place_sgd=True)
    for _ in range(max(1, warmup)):
        st.step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        st.step()
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) / steps * 1e3
    # the per-kernel durations from a second run with the library's event timing on
    L.tp_mlp_profile_enable(True)
    for _ in range(steps):
        st.step()
    torch.cuda.synchronize()
    L.tp_mlp_profile_enable(False)
    prof = L.tp_mlp_profile_entries()
    del st
    torch.cuda.empty_cache()
    fl, by = attention_flops(aw), attention_hbm_bytes(aw)
    kernels = {}
    for k, (n, tot) in prof.items():
        if k in fl:
            ach = fl[k] * n / (tot / 1e3) / 1e12
            kernels[k] = {"bound": "mfma", "achieved": ach, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                          "frac": ach / PEAK_BF16_TFLOPS, "per_launch": fl[k], "avg_ms": tot / n, "launches": n}
        elif k in by:  # one launch per step
            ach = by[k] * n / (tot / 1e3) / 1e9
            kernels[k] = {"bound": "hbm", "achieved": ach, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                          "frac": ach / PEAK_HBM_GBS, "per_launch": by[k], "avg_ms": tot / n, "launches": n}
        else:
            kernels[k] = {"bound": None, "avg_ms": tot / n, "launches": n}
    return {"workload": name, "batch": aw.batch, "seq": aw.seq, "hidden": aw.hidden, "n_q": aw.n_q, "n_kv": aw.n_kv,
            "head_dim": aw.d, "shards": aw.shards, "causal": True, "ms_per_step": ms,
            "tflops": aw.flops_per_step / (ms / 1e3) / 1e12, "tokens_per_s": aw.tokens / (ms / 1e3),
            "kernels": kernels}


def sequence_parallel_timing(w, t, steps: int, warmup: int) -> dict:
    """The step in the sequence-parallel layout, same inputs and flop count."""
    import torch
    from tensor_transformer_mlp_rmsnorm_amd.step import SequenceParallelStep

    sp = SequenceParallelStep(w, t, device="cuda:0", out_of_place_sgd=True, fused_sgd=fused_update(w))
    for _ in range(max(1, warmup)):
        sp.step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        sp.step()
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) / steps * 1e3
    del sp
    torch.cuda.empty_cache()
    return {"ranks": w.shards, "tokens_per_rank_slice": w.tokens // w.shards, "ms_per_step": ms,
            "tflops": w.flops_per_step / (ms / 1e3) / 1e12}


def workload_timing(name: str, steps: int, warmup: int) -> dict:
    """One more workload's step, timed as the main one is (inputs resident,
    SGD out of place, no events in the timed steps), with every kernel's
    duration from a second run and the dominant kernel against its roofline."""
    import torch

    import synth
    from tensor_transformer_mlp_rmsnorm_amd import _lib as L
    from tensor_transformer_mlp_rmsnorm_amd.step import ShardedStep

    w = synth.workload(name)
    st = ShardedStep(w, synth.draw(w), device="cuda:0", out_of_place_sgd=True, fused_sgd=fused_update(w))
    for _ in range(max(1, warmup)):
        st.step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        st.step()
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) / steps * 1e3
    L.tp_mlp_profile_enable(True)
    for _ in range(steps):
        st.step()
    torch.cuda.synchronize()
    L.tp_mlp_profile_enable(False)
    prof = L.tp_mlp_profile_entries()
    del st
    torch.cuda.empty_cache()
    kernels = {k: roofline_entry(k, n, tot, w, steps) for k, (n, tot) in prof.items()}
    dom = max(prof.items(), key=lambda kv: kv[1][1])[0]
    gemm_ms = sum(tot for k, (n, tot) in prof.items() if k in gemm_flops(w)) / steps
    peak = PEAK_BF16_TFLOPS if w.dtype == "bf16" else PEAK_FP32_TFLOPS
    tflops = w.flops_per_step / (ms / 1e3) / 1e12
    d = kernels[dom]
    return {"workload": name, "tokens": w.tokens, "hidden": w.hidden, "ffn_full": w.ffn_full, "shards": w.shards,
            "shards_run": w.n_run, "act": w.act, "master": w.master, "ms_per_step": ms, "tflops": tflops,
            "pct_of_bf16_peak": 100.0 * tflops / peak, "tokens_per_s": w.tokens / (ms / 1e3),
            "gemm_ms_per_step": gemm_ms,
            "gemm_tflops": w.flops_per_step / (gemm_ms / 1e3) / 1e12 if gemm_ms > 0 else None,
            "roofline": {"kernel": dom, "bound": d.get("bound"), "achieved": d.get("achieved"), "peak": d.get("peak"),
                         "unit": d.get("unit"), "frac": d.get("frac"), "per_launch": d.get("per_launch"),
                         "avg_ms": d.get("avg_ms")},
            "kernels": kernels}


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="llama3_8b_tp8")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=15.0)
    ap.add_argument("--no-extras", action="store_true", help="skip the measurements after the timed step")
    ap.add_argument("--extras", default="configs,optimizer,sp,fp8,attention",
                    help="comma-separated measurements after the timed step: configs (the other bf16 workloads: "
                         "GPT-2-small GeLU, one Llama-3-70B TP=8 rank, Llama-3-8B full width with fp32 masters), "
                         "optimizer, sp, fp8, attention")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="only run a plain device copy of MIB MiB (3 times), to calibrate HBM byte counters")
    args = ap.parse_args()
    if args.gpus != 1:
        print(json.dumps({"error": "this benchmark runs on exactly one GPU: the tensor-parallel shards are "
                                   "processed in sequence on one device and there is no multi-GPU path",
                          "n_gpus": args.gpus}), flush=True)
        return 2

    import torch

    import synth
    from tensor_transformer_mlp_rmsnorm_amd import _lib as L
    from tensor_transformer_mlp_rmsnorm_amd.step import ShardedStep

    if not torch.cuda.is_available():
        print(json.dumps({"error": "no GPU visible"}), flush=True)
        return 1
    torch.cuda.set_device(0)
    if args.calibrate_copy:
        n = args.calibrate_copy * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device="cuda:0")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"calibrate_copy_bytes_each_way": n * 4, "launches": 3}), flush=True)
        return 0
    w = synth.workload(args.workload)
    t = synth.draw(w)
    st = ShardedStep(w, t, device="cuda:0", out_of_place_sgd=True, fused_sgd=fused_update(w))
    for _ in range(args.warmup):
        st.step()
    torch.cuda.synchronize()

    # Every kernel's duration, from steps run before the timed region with
    # the library's event timing on; the dominant kernel is the one with the
    # largest total time there.
    L.tp_mlp_profile_enable(True)
    for _ in range(args.steps):
        st.step()
    torch.cuda.synchronize()
    L.tp_mlp_profile_enable(False)
    prof = L.tp_mlp_profile_entries()
    dom = max(prof.items(), key=lambda kv: kv[1][1])[0]

    # The timed region: events bracket the dominant kernel's launches only.
    L.tp_mlp_profile_only(dom)
    L.tp_mlp_profile_enable(True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        st.step()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    L.tp_mlp_profile_enable(False)
    L.tp_mlp_profile_only(None)
    prof_dom = L.tp_mlp_profile_entries()

    ms = elapsed / args.steps * 1e3
    # Per-step times from a separate pass with an event pair around each step: their median and
    # minimum, beside the mean over the K steps timed as one block above (which is `ms_per_step`).
    pairs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    for a, b in pairs:
        a.record()
        st.step()
        b.record()
    torch.cuda.synchronize()
    per_step = [a.elapsed_time(b) for a, b in pairs]
    flops = w.flops_per_step
    tflops = flops / (ms / 1e3) / 1e12
    peak = PEAK_BF16_TFLOPS if w.dtype == "bf16" else PEAK_FP32_TFLOPS
    kernels = {k: roofline_entry(k, n, tot, w, args.steps) for k, (n, tot) in prof.items()}
    gemm_ms = sum(tot for k, (n, tot) in prof.items() if k in gemm_flops(w)) / args.steps
    n_dom, tot_dom = prof_dom[dom]
    d = roofline_entry(dom, n_dom, tot_dom, w, args.steps)
    roof = {"kernel": dom, "bound": d.get("bound"), "achieved": d.get("achieved"), "peak": d.get("peak"),
            "unit": d.get("unit"), "frac": d.get("frac"), "traffic": measured_traffic(dom, w.name),
            "traffic_unit": "HBM bytes per launch (rocprofv3 FETCH_SIZE + WRITE_SIZE, copy-calibrated)",
            "per_launch": d.get("per_launch"), "avg_ms": d.get("avg_ms")}
    out = {
        "metric": METRIC, "value": tflops, "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": w.dtype, "data": "synthetic",
        "config": {"workload": w.name, "tokens": w.tokens, "batch": w.batch, "seq": w.seq, "hidden": w.hidden,
                   "ffn_full": w.ffn_full, "ffn_local": w.ffn_local, "shards": w.shards, "shards_run": w.n_run,
                   "act": w.act, "parallelism": f"tp{w.shards} emulated: shards in sequence on one GPU"},
        "pct_of_bf16_peak": 100.0 * tflops / peak,
        "step_ms_median": statistics.median(per_step), "step_ms_min": min(per_step),
        "tokens_per_s": w.tokens / (ms / 1e3),
        "shard_tokens_per_s": w.tokens / (ms / 1e3 / w.n_run),
        "flops_per_step": flops,
        "gemm_ms_per_step": gemm_ms,
        "gemm_tflops": flops / (gemm_ms / 1e3) / 1e12 if gemm_ms > 0 else None,
        "roofline": roof,
        "kernels": kernels,
    }
    extras = set() if args.no_extras else {e.strip() for e in args.extras.split(",") if e.strip()}
    if "configs" in extras:
        out["other_workloads"] = {}
        for name in OTHER_WORKLOADS:
            if name != w.name:
                out["other_workloads"][name] = workload_timing(name, args.steps, args.warmup)
    if "optimizer" in extras:
        out["optimizer_path"] = optimizer_path(st, w, args.steps, args.warmup)
    if "sp" in extras and w.n_run == w.shards and w.shards > 1:
        out["sequence_parallel"] = sequence_parallel_timing(w, t, args.steps, args.warmup)
    if "fp8" in extras and w.dtype == "bf16" and w.hidden % 16 == 0 and w.ffn_local % 16 == 0:
        del st
        torch.cuda.empty_cache()
        st = None
        out["fp8_path"] = fp8_path(w, t, args.steps, args.warmup)
    if "attention" in extras:
        if st is not None:
            del st
            torch.cuda.empty_cache()
            st = None
        out["attention_path"] = attention_path(args.steps, args.warmup)
    if not args.no_cpu_baseline:
        st = None
        torch.cuda.empty_cache()
        out["cpu_baseline"] = cpu_baseline(w, t, args.cpu_budget)
    else:
        out["cpu_baseline"] = None
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
