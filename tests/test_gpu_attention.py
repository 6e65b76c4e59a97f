"""Parity of the attention sublayer's HIP path (through the C ABI) with the
attention oracle (oracle/attention.py, pinned in tests/test_oracle_attention.py).

* The attention kernels alone: tp_attention_forward against the oracle's
  causal GQA attention of the same bf16 Q, K, V; tp_attention_backward fed
  the oracle's O and log-sum-exp (so it does not depend on the GPU forward)
  against the oracle's gradients; head widths 64 and 128, group sizes 1, 2
  and 4, ragged sequence lengths.
* The sublayer step (AttnStep: QKV projection, attention, row-parallel output
  projection, the two sums, RMSNorm, SGD) against oracle.attn_dense_step, and
  its two ablations against oracle.attn_sharded_step.
* The Llama-3-8B TP=8 attention layer at full size against the fp32 oracle.
Tolerances: tests/tolerance.py (bf16 storage, fp32 accumulation).
"""

import sys
import time

import numpy as np
import pytest
import torch

import synth
from oracle import attention as A
from oracle.mlp import bf16_round
from tolerance import check, check_sum_of_stored

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


def _bf(a):
    return torch.from_numpy(np.asarray(a, np.float32)).to(torch.bfloat16)


KERNEL_CASES = [
    # batch, seq, n_q, n_kv, D, extra ld columns
    (1, 1, 1, 1, 64, 0),
    (2, 5, 4, 2, 64, 0),
    (1, 64, 2, 2, 128, 0),
    (2, 65, 4, 1, 64, 8),
    (1, 200, 4, 4, 128, 0),
    (3, 130, 8, 2, 128, 16),
    (2, 300, 2, 1, 64, 0),
]


@pytest.mark.parametrize("case", KERNEL_CASES, ids=[f"b{c[0]}s{c[1]}q{c[2]}kv{c[3]}d{c[4]}" for c in KERNEL_CASES])
def test_attention_kernels_match_oracle(case):
    from tensor_transformer_mlp_rmsnorm_amd import _lib as L
    b, s, nq, nkv, D, pad = case
    sh = A.AttnShape(b, s, nq, nkv, D)
    T, W = b * s, sh.qkv_width
    ld = W + pad
    say(f"[gpu] attention kernels b={b} s={s} n_q={nq} n_kv={nkv} D={D} ld={ld}")
    rng = np.random.default_rng(b * 1000 + s * 10 + D)
    qkv = bf16_round(rng.standard_normal((T, ld)) * 1.5)
    q, k, v = A.split_qkv(qkv[:, :W], sh)
    o_ref, lse_ref = A.causal_attention_fwd(q, k, v, sh.group)
    O_ref = A.merge_heads(o_ref, sh)
    qkv_d = _bf(qkv).cuda()
    O = torch.full((T, nq * D), float("nan"), dtype=torch.bfloat16, device="cuda")
    lse = torch.full((nq, T), float("nan"), dtype=torch.float32, device="cuda")
    L.tp_attention_forward(b, s, nq, nkv, D, qkv_d, ld, O, lse)
    torch.cuda.synchronize()
    report = {}
    check("O", O.cpu(), O_ref, "bf16", rowwise=True, report=report)
    lse_flat = np.stack([lse_ref[:, h].reshape(-1) for h in range(nq)])  # [n_q, T]
    err = float(np.max(np.abs(lse.cpu().double().numpy() - lse_flat)))
    assert err <= 1e-3 * max(1.0, float(np.abs(lse_flat).max())), ("lse", err)
    # backward from the oracle's stored O (bf16) and lse
    O_st = bf16_round(O_ref)
    dO = bf16_round(rng.standard_normal((T, nq * D)))
    dq, dk, dv = A.causal_attention_bwd(q, k, v, A.split_heads(O_st, nq, sh), A.split_heads(dO, nq, sh), sh.group)
    dqkv_ref = np.concatenate([A.merge_heads(dq, sh), A.merge_heads(dk, sh), A.merge_heads(dv, sh)], axis=1)
    dqkv = torch.full((T, ld), 7.0, dtype=torch.bfloat16, device="cuda")
    wsb = L.tp_attention_backward_workspace_bytes(b, s, nq, nkv, D)
    ws = torch.full((wsb,), 0x7f, dtype=torch.uint8, device="cuda")  # garbage: every byte read is written first
    L.tp_attention_backward(b, s, nq, nkv, D, qkv_d, ld, _bf(O_st).cuda(), _bf(dO).cuda(),
                            torch.from_numpy(lse_flat.astype(np.float32)).cuda(), ws, wsb, dqkv)
    torch.cuda.synchronize()
    got = dqkv.cpu()
    check("dQ", got[:, :nq * D], dqkv_ref[:, :nq * D], "bf16", rowwise=True, report=report)
    check("dK", got[:, nq * D:(nq + nkv) * D], dqkv_ref[:, nq * D:(nq + nkv) * D], "bf16", rowwise=True, report=report)
    check("dV", got[:, (nq + nkv) * D:W], dqkv_ref[:, (nq + nkv) * D:], "bf16", rowwise=True, report=report)
    if pad:
        assert torch.all(got[:, W:] == 7.0)  # the padding columns are not written
    say(f"  worst: {max(report.items(), key=lambda kv: kv[1])}")


def _params(t) -> A.AttnParams:
    c = synth.to_numpy64
    return A.AttnParams(c(t["norm_w"]), c(t["w_qkv"]), c(t["w_o"]), c(t["b_o"]))


def _compare_step(res, d, report, prefix=""):
    g, npar = d["grads"], d["new_params"]
    check(prefix + "out", res["out"], d["out"], "bf16", rowwise=True, report=report)
    check(prefix + "normed", res["normed"], d["n"], "bf16", rowwise=True, report=report)
    check(prefix + "attn_out", res["attn_out"], d["O"], "bf16", rowwise=True, report=report)
    check(prefix + "dN", res["dN"], d["dN"], "bf16", rowwise=True, report=report)
    check(prefix + "dx", res["dx"], d["dx"], "bf16", rowwise=True, report=report)
    check(prefix + "d_norm_w", res["d_norm_w"], g["norm_w"], "bf16", report=report)
    check(prefix + "d_b_o", res["d_b_o"], g["b_o"], "bf16", report=report)
    # the weight gradients are sums over tokens of stored bf16 tensors (dQKV, dO... with N, O): see
    # tolerance.check_sum_of_stored -- the keys of the first positions of every sequence are attended by all
    # later queries, so their gradient rows dominate sums over tokens
    check_sum_of_stored(prefix + "d_w_qkv", res["d_w_qkv"], g["w_qkv"], d["dqkv"], d["n"], report=report)
    check_sum_of_stored(prefix + "d_w_o", res["d_w_o"], g["w_o"], d["dY"], d["O"], report=report)
    lr = d["lr"]
    new_qkv_ref, new_o_ref = npar.w_qkv, npar.w_o
    check_sum_of_stored(prefix + "new_w_qkv", res["new_w_qkv"], new_qkv_ref, d["dqkv"], d["n"], scale=lr,
                        report=report)
    check_sum_of_stored(prefix + "new_w_o", res["new_w_o"], new_o_ref, d["dY"], d["O"], scale=lr, report=report)
    check(prefix + "new_norm_w", res["new_norm_w"], npar.norm_w, "bf16", report=report)
    check(prefix + "new_b_o", res["new_b_o"], npar.b_o, "bf16", report=report)


STEPS = [
    # name,          batch, seq, H,   n_q, n_kv, D,   S
    ("gqa_S2", 2, 100, 256, 8, 4, 64, 2),
    ("mha_S1_fused", 1, 130, 192, 2, 2, 128, 1),
    ("gqa4_S2_d128", 2, 70, 512, 8, 2, 128, 2),
    ("tiny_S2", 1, 5, 64, 4, 2, 64, 2),
]


@pytest.mark.parametrize("case", STEPS, ids=[c[0] for c in STEPS])
def test_attention_step_matches_oracle(case):
    from tensor_transformer_mlp_rmsnorm_amd.step import AttnStep
    name, b, s, H, nq, nkv, D, S = case
    w = synth.AttnWorkload("attn_" + name, batch=b, seq=s, hidden=H, n_q=nq, n_kv=nkv, d=D, shards=S, w_std=0.05,
                           seed=700 + s)
    t = synth.draw_attn(w, perturb=True)
    say(f"[gpu] attention step {name} b={b} s={s} H={H} n_q={nq} n_kv={nkv} D={D} S={S}")
    st = AttnStep(w, t, out_of_place_sgd=True)
    st.step()
    torch.cuda.synchronize()
    res = st.results()
    sh = A.AttnShape(b, s, nq, nkv, D)
    d = A.attn_dense_step(synth.to_numpy64(t["x"]), _params(t), sh, w.eps, w.lr, storage="bf16")
    report = {}
    _compare_step(res, d, report)
    say(f"  worst: {max(report.items(), key=lambda kv: kv[1])}")


@pytest.mark.parametrize("shards", [2, 4])
def test_attention_norm_parts_equal_summed_dN(shards):
    """The NORM phase on the shards' dN partials (summed as the RMSNorm
    backward reads them) gives bit for bit what it gives on the dN that
    tp_partial_sum forms from the same partials."""
    from tensor_transformer_mlp_rmsnorm_amd import _lib as L
    from tensor_transformer_mlp_rmsnorm_amd.step import AttnStep
    w = synth.AttnWorkload("attn_parts", batch=2, seq=72, hidden=264, n_q=8, n_kv=4, d=64, shards=shards, w_std=0.05,
                           seed=91)
    t = synth.draw_attn(w, perturb=True)
    say(f"[gpu] attention NORM on {shards} partials vs their sum")
    st = AttnStep(w, t, out_of_place_sgd=True)
    st.step()
    st.materialize_dN()  # dN = tp_partial_sum of the same partials
    dx, dw, db = torch.empty_like(st.dx), torch.empty_like(st.d_norm_w), torch.empty_like(st.d_b_o)
    L.tp_attn_backward(st._desc(), L.BWD_NORM, x=st.x, rstd=st.rstd, norm_w=st.norm_w, d_out=st.out,
                       d_normed=st.dN, d_x=dx, d_norm_w=dw, d_b_o=db, workspace=st.workspace)
    torch.cuda.synchronize()
    assert torch.equal(dx, st.dx) and torch.equal(dw, st.d_norm_w) and torch.equal(db, st.d_b_o)


@pytest.mark.parametrize("mode", ["missing_forward_reduce", "missing_backward_reduce"])
def test_attention_ablations_match_oracle(mode):
    from tensor_transformer_mlp_rmsnorm_amd.step import AttnStep
    w = synth.AttnWorkload("attn_ablation", batch=2, seq=40, hidden=128, n_q=4, n_kv=2, d=64, shards=2, w_std=0.2,
                           seed=77)
    t = synth.draw_attn(w, perturb=True)
    say(f"[gpu] attention ablation {mode}")
    st = AttnStep(w, t, out_of_place_sgd=True)
    st.step(mode)
    torch.cuda.synchronize()
    res = st.results(mode)
    sh = A.AttnShape(w.batch, w.seq, w.n_q, w.n_kv, w.d)
    x, p = synth.to_numpy64(t["x"]), _params(t)
    ab = A.attn_sharded_step(x, p, sh, w.eps, w.lr, w.shards, mode=mode, storage="bf16")
    dense = A.attn_dense_step(x, p, sh, w.eps, w.lr, storage="bf16")
    for s, rk in enumerate(ab["ranks"]):
        out_s = res["out"][s] if mode == "missing_forward_reduce" else res["out"]
        check(f"out[{s}]", out_s, rk["out"], "bf16", rowwise=True)
        check(f"dx[{s}]", res["dx"][s], rk["dx"], "bf16", rowwise=True)
        check(f"d_norm_w[{s}]", res["d_norm_w"][s], rk["grads"]["norm_w"], "bf16")
        # and each differs from the dense step where the ablation says it does
        gap = float(np.max(np.abs(res["dx"][s].double().numpy() - dense["dx"])))
        assert gap > 5e-2 * float(np.abs(dense["dx"]).max()), (s, gap)


@pytest.mark.parametrize("name", ["attn_llama3_8b_tp8", "attn_gpt2s_tp1"])
def test_attention_full_size(name):
    """The Llama-3-8B TP=8 attention layer (32 query heads, 8 KV heads of 128,
    2 sequences of 4096) in the benchmark's configuration, and the GPT-2-small
    layer (12 heads of 64, 4 sequences of 1024, one shard: the fused output
    epilogue), every output against the oracle's dense step in fp32."""
    from tensor_transformer_mlp_rmsnorm_amd.step import AttnStep
    w = synth.attn_workload(name)
    t = synth.draw_attn(w)
    say(f"[gpu] attention full size {w.name}")
    st = AttnStep(w, t, out_of_place_sgd=True)
    st.step()
    torch.cuda.synchronize()
    res = st.results()
    del st
    torch.cuda.empty_cache()
    sh = A.AttnShape(w.batch, w.seq, w.n_q, w.n_kv, w.d)
    t0 = time.time()
    d = A.attn_dense_step(synth.to_numpy64(t["x"]).astype(np.float32), _params(t), sh, w.eps, w.lr,
                          dtype=np.float32, storage="bf16")
    say(f"  oracle dense step (fp32): {time.time() - t0:.1f} s")
    report = {}
    _compare_step(res, d, report)
    say(f"  worst: {max(report.items(), key=lambda kv: kv[1])}")
