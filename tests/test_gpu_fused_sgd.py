"""The SGD update taken inside the weight-gradient GEMMs (tp_mlp_fused_sgd).

A step with the update fused must give exactly the parameters (and their
transposed copies and fp32 masters) of the step that writes the gradients
and then runs tp_mlp_sgd_step_multi: the same fp32 gradient (the GEMM's own
accumulators, or its k-slices summed in the same order) goes through the
same update arithmetic and the same rounding.  So the fused step is compared
with the unfused one bit for bit, on every tensor both write, for shapes
that cover one and several output tiles with ragged edges in both weight
dimensions, no k split and k splits of 2 and 4 slices (few tiles, long T),
SwiGLU and GeLU, fp32 masters, in-place and out-of-place updates, and the
path that forms the w_in update from N and d_pre transposed (dW_in^T, both
operands K-contiguous); cases also go through the C ABI directly.  The unfused step is
held to the oracle in test_gpu_parity.py; here one case is also compared
with the fp64 oracle directly.
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


def bits(t: torch.Tensor) -> torch.Tensor:
    return t.detach().contiguous().view(torch.int16 if t.element_size() == 2 else torch.int32)


def assert_same_bits(name, got, ref):
    assert got.shape == ref.shape, name
    diff = int((bits(got) != bits(ref)).sum())
    assert diff == 0, f"{name}: {diff} of {ref.numel()} elements differ"


CASES = [
    # name, T, H, F_full, S, act, master, oop
    ("swiglu_S2_ragged", 300, 136, 240, 2, "swiglu", False, True),
    ("swiglu_S3_tiles", 600, 520, 3 * 264, 3, "swiglu", False, True),
    ("swiglu_S2_ksplit2", 2500, 264, 272, 2, "swiglu", False, True),
    ("swiglu_S1_ksplit4_master", 4100, 264, 136, 1, "swiglu", True, True),
    ("gelu_S1_master_inplace", 1000, 520, 600, 1, "gelu", True, False),
    ("gelu_S2_ksplit", 3000, 136, 2 * 264, 2, "gelu", False, False),
    ("swiglu_S2_inplace", 700, 264, 2 * 232, 2, "swiglu", False, False),
    # T a multiple of 8, no masters, no k split: the w_in gradient GEMM on N^T and d_pre^T (dW_in^T)
    ("swiglu_S2_nt_inplace", 704, 264, 2 * 232, 2, "swiglu", False, False),
    ("gelu_S2_nt", 1000, 264, 2 * 264, 2, "gelu", False, True),
]


def _run(w, t, oop, fused):
    from tensor_transformer_mlp_rmsnorm_amd.step import ShardedStep
    st = ShardedStep(w, t, out_of_place_sgd=oop, fused_sgd=fused)
    st.step()
    torch.cuda.synchronize()
    return st


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_fused_update_equals_unfused_bitwise(case):
    name, T, H, Ff, S, act, master, oop = case
    w = synth.Workload(name, tokens=T, hidden=H, ffn_full=Ff, shards=S, act=act, dtype="bf16", w_std=0.05,
                       seed=11, master=master)
    say(f"[gpu] fused sgd {name}: T={T} H={H} F_full={Ff} S={S} {act} master={master} oop={oop}")
    t = synth.draw(w, perturb=True)
    ref = _run(w, t, oop, fused=False)
    got = _run(w, t, oop, fused=True)
    for pname, _ in ref._param_list():
        assert_same_bits("new " + pname, got.new[pname], ref.new[pname])
        if master:
            assert_same_bits("master " + pname, got.new_masters[pname], ref.new_masters[pname])
    for key, (tt, _, _) in ref.new_t.items():
        assert_same_bits("transposed " + key, got.new_t[key][0], tt)
    # everything else the step writes is unchanged by the fusion
    for attr in ("out", "dx", "d_norm_w", "d_b_down", "normed"):
        assert_same_bits(attr, getattr(got, attr), getattr(ref, attr))
    for s, (a, b) in enumerate(zip(got.shards, ref.shards)):
        assert_same_bits(f"d_pre.{s}", a["d_pre"], b["d_pre"])
        assert_same_bits(f"dN_part.{s}", a["dN_part"], b["dN_part"])
        if act == "gelu":
            assert_same_bits(f"d_b_in.{s}", a["d_b_in"], b["d_b_in"])
    res = got.results()
    assert res["d_w_in"] is None and res["d_w_down"] is None  # applied, never written
    nt = T % 8 == 0 and not master and name not in ("swiglu_S2_ksplit2", "gelu_S2_ksplit")
    assert (got.d_pre_t is not None) == nt, name
    if nt:  # the last shard's d_pre, transposed by the d_act GEMM's epilogue
        assert_same_bits("d_pre_t", got.d_pre_t, got.shards[-1]["d_pre"].t().contiguous())


def test_fused_update_against_oracle():
    """A fused step's new parameters against the fp64 oracle's dense step (bf16 storage model)."""
    w = synth.Workload("fused_oracle", tokens=900, hidden=264, ffn_full=2 * 232, shards=2, act="swiglu",
                       dtype="bf16", w_std=0.05, seed=5, master=True)
    t = synth.draw(w, perturb=True)
    st = _run(w, t, True, fused=True)
    res = st.results()
    c = synth.to_numpy64
    p = Params(c(t["norm_w"]), c(t["w_in"]), c(t["w_down"]), c(t["b_down"]), c(t["b_in"]))
    d = oracle.dense_step(c(t["x"]), p, w.act, w.eps, w.lr, storage="bf16")
    report = {}
    for key, ref in (("new_w_in", d["new_params"].w_in), ("new_w_down", d["new_params"].w_down),
                     ("master_w_in", d["new_masters"].w_in), ("master_w_down", d["new_masters"].w_down),
                     ("new_norm_w", d["new_params"].norm_w), ("new_b_down", d["new_params"].b_down)):
        check(key, res[key], ref, "bf16", rowwise=False, report=report)
    say(f"  worst: {max(report.items(), key=lambda kv: kv[1])}")


@pytest.mark.parametrize("ksplit", [False, True], ids=["one_pass", "ksplit"])
def test_fused_update_without_transposed_copies_abi(ksplit):
    """Through the C ABI: the SHARD phase with the update fused and no
    transposed targets, out of place, against the unfused phase followed by
    tp_mlp_sgd_step_multi (same bits)."""
    from tensor_transformer_mlp_rmsnorm_amd import _lib as L
    T, H, F = (3000, 264, 136) if ksplit else (520, 264, 136)
    dev = "cuda:0"
    g = torch.Generator().manual_seed(3)
    r = lambda *s, std=1.0: (torch.randn(*s, generator=g) * std).to(torch.bfloat16).to(dev)
    normed, d_out = r(T, H), r(T, H)
    pre, act = r(T, 2 * F), r(T, F)
    w_in, w_down = r(2, F, H, std=0.05), r(H, F, std=0.05)
    desc = L.make_desc(T, H, F, L.ACT_SWIGLU, L.BF16, 1e-6, 0)
    ws = torch.empty(L.tp_mlp_workspace_bytes(desc, L.BWD_SHARD), dtype=torch.uint8, device=dev)
    f32 = lambda *s: torch.empty(*s, dtype=torch.float32, device=dev)
    bf = lambda *s: torch.empty(*s, dtype=torch.bfloat16, device=dev)
    common = dict(normed=normed, pre_act=pre, act=act, w_in=w_in, w_down=w_down, d_out=d_out, workspace=ws)
    # unfused: gradients, then the SGD step
    d_pre0, dn0, gi, gd = bf(T, 2 * F), f32(T, H), f32(2, F, H), f32(H, F)
    L.tp_mlp_backward(desc, L.BWD_SHARD, d_pre=d_pre0, d_normed_part=dn0, d_w_in=gi, d_w_down=gd, **common)
    wi0, wd0 = bf(2, F, H), bf(H, F)
    L.tp_mlp_sgd_step_multi([(w_in, wi0, gi, None, None, w_in.numel()), (w_down, wd0, gd, None, None, w_down.numel())],
                            L.BF16, 0.1)
    # fused, no transposed copies
    d_pre1, dn1, wi1, wd1 = bf(T, 2 * F), f32(T, H), bf(2, F, H), bf(H, F)
    L.tp_mlp_backward(desc, L.BWD_SHARD, d_pre=d_pre1, d_normed_part=dn1,
                      fused_sgd=dict(lr=0.1, w_in_out=wi1, w_down_out=wd1), **common)
    torch.cuda.synchronize()
    assert_same_bits("w_in", wi1, wi0)
    assert_same_bits("w_down", wd1, wd0)
    assert_same_bits("d_pre", d_pre1, d_pre0)
    assert_same_bits("d_normed_part", dn1, dn0)


@pytest.mark.parametrize("act", ["swiglu", "gelu"])
def test_transposed_activation_path_abi(act):
    """Through the C ABI: d_pre_t is the exact transpose of d_pre, and the
    w_in update formed from normed_t and d_pre_t (dW_in^T, both operands
    K-contiguous) writes the bits of the unfused phase + tp_mlp_sgd_step_multi,
    with the transposed target or without it."""
    from tensor_transformer_mlp_rmsnorm_amd import _lib as L
    T, H, F = 520, 264, 136  # ragged tiles in both weight dimensions, one k range
    sw = act == "swiglu"
    P = 2 * F if sw else F
    dev = "cuda:0"
    g = torch.Generator().manual_seed(4)
    r = lambda *s, std=1.0: (torch.randn(*s, generator=g) * std).to(torch.bfloat16).to(dev)
    normed, d_out = r(T, H), r(T, H)
    pre, act_t = r(T, P), r(T, F)
    w_in, w_down = r(P, H, std=0.05), r(H, F, std=0.05)
    b_in = None if sw else r(F, std=0.05)
    w_in_t, w_down_t = w_in.t().contiguous(), w_down.t().contiguous()
    normed_t = normed.t().contiguous()
    desc = L.make_desc(T, H, F, L.ACT_SWIGLU if sw else L.ACT_GELU, L.BF16, 1e-6, 0)
    ws = torch.empty(L.tp_mlp_workspace_bytes(desc, L.BWD_SHARD), dtype=torch.uint8, device=dev)
    f32 = lambda *s: torch.empty(*s, dtype=torch.float32, device=dev)
    bf = lambda *s: torch.empty(*s, dtype=torch.bfloat16, device=dev)
    common = dict(normed=normed, pre_act=pre, act=act_t, w_in=w_in, w_down=w_down, d_out=d_out, workspace=ws,
                  w_in_t=w_in_t, w_down_t=w_down_t)
    d_pre0, dn0, gi, gd = bf(T, P), f32(T, H), f32(P, H), f32(H, F)
    dbi = None if sw else f32(F)
    L.tp_mlp_backward(desc, L.BWD_SHARD, d_pre=d_pre0, d_normed_part=dn0, d_w_in=gi, d_w_down=gd, d_b_in=dbi,
                      **common)
    wi0, wit0 = bf(P, H), bf(H, P)
    L.tp_mlp_sgd_step_multi([(w_in, wi0, gi, None, None, w_in.numel(), wit0, P, H)], L.BF16, 0.1)
    for targets in ("both", "plain_only"):
        d_pre1, dn1, wi1, wit1, wd1, dpt = bf(T, P), f32(T, H), bf(P, H), bf(H, P), bf(H, F), bf(P, T)
        fu = dict(lr=0.1, w_down_out=wd1, w_in_out=wi1)
        if targets == "both":
            fu["w_in_t_out"] = wit1
        L.tp_mlp_backward(desc, L.BWD_SHARD, d_pre=d_pre1, d_normed_part=dn1, d_b_in=None if sw else f32(F),
                          normed_t=normed_t, d_pre_t=dpt, fused_sgd=fu, **common)
        torch.cuda.synchronize()
        assert_same_bits("d_pre", d_pre1, d_pre0)
        assert_same_bits("d_pre_t", dpt, d_pre0.t().contiguous())
        assert_same_bits("d_normed_part", dn1, dn0)
        assert_same_bits("w_in " + targets, wi1, wi0)
        if targets != "plain_only":
            assert_same_bits("w_in_t " + targets, wit1, wit0)


@pytest.mark.parametrize("shape", [(8, 8), (72, 136), (520, 264), (4096, 1792), (8192, 4096)],
                         ids=lambda s: f"{s[0]}x{s[1]}")
def test_transpose_bf16_exact(shape):
    """tp_mlp_transpose_bf16 (the step's N^T, the weights' first transposed copies): every element moved bit for
    bit, ragged 64 x 64 tiles included."""
    from tensor_transformer_mlp_rmsnorm_amd import _lib as L
    R, C = shape
    g = torch.Generator().manual_seed(R + C)
    x = torch.randn(R, C, generator=g).to(torch.bfloat16).to("cuda:0")
    out = torch.full((C, R), float("nan"), dtype=torch.bfloat16, device="cuda:0")
    L.tp_mlp_transpose_bf16(x, out, R, C)
    torch.cuda.synchronize()
    assert_same_bits("transpose", out, x.t().contiguous())


@pytest.mark.parametrize("master", [False, True], ids=["plain", "masters"])
def test_fused_update_empty_tokens(master):
    """T = 0 with the update fused: every weight gradient is an empty sum, so the fused update (a GEMM with
    no k) writes back the parameters, their transposed copies and masters unchanged."""
    w = synth.Workload("fused_empty", tokens=0, hidden=64, ffn_full=128, shards=2, act="swiglu", dtype="bf16",
                       w_std=0.05, seed=3, master=master)
    t = synth.draw(w, perturb=True)
    st = _run(w, t, True, fused=True)
    for s, sh in enumerate(st.shards):
        for key in ("w_in", "w_down"):
            name = f"{key}.{s}"
            assert_same_bits("new " + name, st.new[name], sh[key])
            assert_same_bits("transposed " + name, st.new_t[name][0], sh[key + "_t"])
            if master:
                assert_same_bits("master " + name, st.new_masters[name], st.masters[name])
