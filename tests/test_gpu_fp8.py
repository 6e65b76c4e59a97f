"""Parity of the FP8 path (through the C ABI) with the FP8 oracle
(oracle/fp8.py, pinned in tests/test_oracle_fp8.py).

* Casts: the codes are integers decided in fp32 on both sides, so they are
  compared bit for bit, row copy and transposed copy with its zero padding,
  and the running amax exactly.
* Scale update: bit for bit (the scale is one IEEE division, its inverse one
  more).
* The FP8 GEMM on codes both sides share: every output within the block-sum
  bound of the matrix unit (tests/tolerance.py, FP8_GEMM_REL), for both format
  pairs, ragged and padded shapes, a k split and accumulation.
* F2 with its activation epilogue and the backward's d_act GEMM with the
  activation backward, on codes of given tensors: the bf16 tolerance
  elementwise, as for the bf16 path.
* The whole FP8 step: its casts take computed tensors whose codes can differ
  by one FP8 step where the bf16 input differs by an ulp, so each output is
  compared by its relative Frobenius error (FP8_STEP_FROB); the weight
  gradients must also sit much closer to the FP8 oracle than to the bf16 one,
  so the comparison could not pass on a path that skipped the quantisation.
"""

import sys

import numpy as np
import pytest
import torch

import oracle
import synth
from oracle import fp8
from tolerance import check, check_fp8_gemm, check_fp8_step, frob_rel
from test_gpu_parity import compare_full, np_params

pytestmark = pytest.mark.gpu

FMTS = {0: fp8.E4M3, 1: fp8.E5M2}


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


def meta_tensor(fmt: int, L: int, scale=1.0, amax=0.0, hist=None) -> torch.Tensor:
    s = np.float32(scale)
    h = np.zeros(L, np.float32) if hist is None else np.asarray(hist, np.float32)
    vals = np.concatenate([[s, np.float32(1.0 / float(s)), np.float32(amax), np.float32(FMTS[fmt].max)], h])
    return torch.from_numpy(vals.astype(np.float32)).cuda()


def bf16_inputs(rng, R, C, fmt, scale):
    """bf16 values over the whole range of the format under `scale`:
    normal and subnormal magnitudes, exact ties, values that saturate, zeros."""
    f = FMTS[fmt]
    v = rng.standard_normal((R, C)) * 2.0 ** rng.integers(-14, 9, (R, C)) * (f.max / 448.0)
    flat = v.reshape(-1)
    grid = np.sort(np.unique(np.abs(fp8.decode(np.arange(256, dtype=np.uint8), f))))
    grid = grid[np.isfinite(grid)]
    mids = (grid[:-1] + grid[1:]) / 2 / float(np.float32(scale))
    k = min(len(mids), flat.size // 4)
    flat[:k] = mids[:k] * np.where(rng.random(k) < 0.5, -1, 1)
    flat[k:k + 8] = [0.0, -0.0, 3 * f.max / float(scale), -5 * f.max / float(scale), 1e-30, -1e-30,
                     f.max / float(scale), f.sub_step / float(scale)]
    return torch.from_numpy(v.astype(np.float32)).to(torch.bfloat16)


@pytest.mark.parametrize("fmt", [0, 1], ids=["e4m3", "e5m2"])
@pytest.mark.parametrize("pow2", [True, False], ids=["pow2_scale", "scale"])
@pytest.mark.parametrize("R,C", [(200, 136), (1000, 4096), (16, 8)])
def test_cast_codes_are_the_oracles(fmt, pow2, R, C):
    from tensor_transformer_mlp_rmsnorm_amd import _lib as L
    rng = np.random.default_rng(R * 7 + C + fmt)
    scale = np.float32(8.0 if pow2 else FMTS[fmt].max / 3.7)
    x = bf16_inputs(rng, R, C, fmt, scale)
    ldt = (R + 15) // 16 * 16 + (16 if R == 200 else 0)
    say(f"[gpu] fp8 cast fmt={fmt} R={R} C={C} ldt={ldt} scale={scale}")
    meta = meta_tensor(fmt, 4, scale=scale)
    xd = x.cuda()
    out = torch.full((R, C), 0xAA, dtype=torch.uint8, device="cuda")
    out_t = torch.full((C, ldt), 0xAA, dtype=torch.uint8, device="cuda")
    L.tp_mlp_fp8_cast(R, C, xd, fmt, meta, out, out_t, ldt)
    torch.cuda.synchronize()
    xn = x.double().numpy()
    ref = fp8.quantize(xn, scale, FMTS[fmt])
    got, got_t = out.cpu().numpy(), out_t.cpu().numpy()
    bad = np.nonzero(got != ref)
    assert bad[0].size == 0, (bad[0][:5], bad[1][:5], got[bad][:5], ref[bad][:5], xn[bad][:5])
    np.testing.assert_array_equal(got_t[:, :R], ref.T)
    assert np.all(got_t[:, R:] == 0)
    m = meta.cpu().numpy()
    assert m[2] == np.float32(np.abs(xn).max())
    assert m[0] == scale and m[3] == np.float32(FMTS[fmt].max)
    # a second cast folds its amax into the running one; the row copy alone
    x2 = (x.float() * 0.25).to(torch.bfloat16)
    L.tp_mlp_fp8_cast(R, C, x2.cuda(), fmt, meta, out, None, 0)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(out.cpu().numpy(), fp8.quantize(x2.double().numpy(), scale, FMTS[fmt]))
    assert meta.cpu().numpy()[2] == np.float32(np.abs(xn).max())


def test_cast_transposed_only_and_padding_only():
    from tensor_transformer_mlp_rmsnorm_amd import _lib as L
    meta = meta_tensor(0, 2, scale=2.0)
    x = torch.randn(37, 24).to(torch.bfloat16)
    out_t = torch.full((24, 64), 0x55, dtype=torch.uint8, device="cuda")
    L.tp_mlp_fp8_cast(37, 24, x.cuda(), 0, meta, None, out_t, 64)
    torch.cuda.synchronize()
    ref = fp8.quantize(x.double().numpy(), 2.0, fp8.E4M3)
    got = out_t.cpu().numpy()
    np.testing.assert_array_equal(got[:, :37], ref.T)
    assert np.all(got[:, 37:] == 0)
    # no rows: the padding is still written, [24, 32] here, and nothing past it
    buf = torch.full((24 * 32 + 256,), 0x55, dtype=torch.uint8, device="cuda")
    L.tp_mlp_fp8_cast(0, 24, None, 0, meta, None, buf, 32)
    torch.cuda.synchronize()
    got = buf.cpu().numpy()
    assert np.all(got[:24 * 32] == 0) and np.all(got[24 * 32:] == 0x55)


def test_update_scales_match_oracle():
    from tensor_transformer_mlp_rmsnorm_amd import _lib as L
    rng = np.random.default_rng(11)
    Ls = 5
    cases = [  # fmt, prior scale, amax, history
        (0, 3.0, 0.0, np.zeros(Ls)),                               # all zero: scale kept
        (0, 1.0, 2.5, rng.uniform(0, 4, Ls)),
        (1, 7.0, 1e-3, rng.uniform(0, 1e-3, Ls)),
        (0, 2.0, np.inf, rng.uniform(0, 4, Ls)),                   # non-finite amax: scale kept
        (1, 5.0, np.nan, rng.uniform(0, 4, Ls)),
        (0, 1.0, 0.0, np.r_[0.0, 0.0, 0.0, 0.0, 9.0]),            # the oldest entry drops out: scale kept
        (1, 1.0, 3.3e4, rng.uniform(0, 10, Ls)),
    ]
    metas, refs = [], []
    for fmt, sc, am, hist in cases:
        metas.append(meta_tensor(fmt, Ls, scale=sc, amax=am, hist=hist))
        o = fp8.Fp8Meta(FMTS[fmt], np.asarray(hist, np.float32), np.float32(sc), np.float32(am))
        o.update()
        refs.append(o)
    L.tp_mlp_fp8_update_scales(metas, Ls)
    torch.cuda.synchronize()
    for i, (m, o) in enumerate(zip(metas, refs)):
        g = m.cpu().numpy()
        assert g[0] == o.scale, (i, g[0], o.scale)
        assert g[1] == o.scale_inv(), (i, g[1], o.scale_inv())
        assert g[2] == 0.0
        h = g[4:]
        same = (h == o.history) | (np.isnan(h) & np.isnan(o.history))
        assert same.all(), (i, h, o.history)
    # a longer history: every entry shifts by one
    L2 = 1024
    hist = rng.uniform(0, 1, L2).astype(np.float32)
    m = meta_tensor(0, L2, amax=0.5, hist=hist)
    L.tp_mlp_fp8_update_scales([m], L2)
    torch.cuda.synchronize()
    g = m.cpu().numpy()
    np.testing.assert_array_equal(g[4:], np.r_[np.float32(0.5), hist[:-1]].astype(np.float32))
    assert g[0] == np.float32(448.0 / float(max(0.5, hist[:-1].max())))


def _state_of(metas: dict) -> dict:
    """An oracle meta state in the form Fp8Step.load_meta_state takes."""
    return {k: (float(m.scale), float(m.scale_inv()), float(m.amax), m.history.copy()) for k, m in metas.items()}


def _meta_scales(rng, roles):
    """Seeded scales of the shape a warm step has (fmt_max / an amax)."""
    amax = dict(normed=4.0, w_in=0.2, act=1.5, w_down=0.2, d_out=5.0, d_pre=0.1)
    return {k: np.float32(FMTS[0 if fp8.ROLES[k] is fp8.E4M3 else 1].max / (amax[k] * rng.uniform(0.8, 1.25)))
            for k in roles}


def _fmt_code(role):
    return 0 if fp8.ROLES[role] is fp8.E4M3 else 1


GEMMS = [
    # M,   N,    K,    lda,  ldb, ldc,  fmt_a, accumulate
    (300, 200, 272, 272, 272, 200, 0, False),
    (257, 520, 1040, 1056, 1040, 528, 1, True),
    (64, 4096, 8192, 8192, 8192, 4100, 1, False),   # k split over 8 workgroups
    (1, 16, 16, 16, 16, 16, 0, False),
    (129, 260, 304, 304, 320, 260, 1, True),        # k extent of a padded transpose
    (520, 264, 8192, 8192, 8192, 264, 0, True),     # k split, accumulating
]


@pytest.mark.parametrize("case", GEMMS, ids=[f"{c[0]}x{c[1]}x{c[2]}_f{c[6]}{'_acc' if c[7] else ''}" for c in GEMMS])
def test_fp8_gemm_matches_oracle(case):
    """The FP8 GEMM on codes that both sides share: within the block-sum bound of every output."""
    from tensor_transformer_mlp_rmsnorm_amd import _lib as L
    M, N, K, lda, ldb, ldc, fa, acc = case
    say(f"[gpu] fp8 gemm M={M} N={N} K={K} lda={lda} ldb={ldb} ldc={ldc} fmt_a={fa} accumulate={acc}")
    rng = np.random.default_rng(M + 3 * N + 7 * K)
    sa, sb = np.float32(FMTS[fa].max / 3.0), np.float32(448.0 / 0.15)
    a = rng.standard_normal((M, lda)) * np.where(rng.random((M, lda)) < 0.02, 8.0, 1.0)
    b = rng.standard_normal((N, ldb)) * 0.05
    ca = fp8.quantize(a, sa, FMTS[fa])
    cb = fp8.quantize(b, sb, fp8.E4M3)
    ma, mb = fp8.Fp8Meta.new(FMTS[fa], 1), fp8.Fp8Meta.new(fp8.E4M3, 1)
    ma.scale, mb.scale = sa, sb
    ref = fp8.fp8_gemm_nt(ca[:, :K], ma, cb[:, :K], mb)
    absprod = np.abs(fp8.decode(ca[:, :K], FMTS[fa])) @ np.abs(fp8.decode(cb[:, :K], fp8.E4M3)).T
    deq = float(np.float32(ma.scale_inv()) * np.float32(mb.scale_inv()))
    c0 = rng.standard_normal((M, N)).astype(np.float32)
    if acc:
        ref = ref + c0
    C = torch.full((M, ldc), 7.0, dtype=torch.float32, device="cuda")
    C[:, :N] = torch.from_numpy(c0).cuda()
    sinv = torch.tensor([ma.scale_inv(), mb.scale_inv()], dtype=torch.float32, device="cuda")
    ws_bytes = L.tp_mlp_fp8_gemm_workspace_bytes(M, N, K, ldc)
    ws = torch.empty(max(ws_bytes, 16), dtype=torch.uint8, device="cuda")
    L.tp_mlp_fp8_gemm(M, N, K, torch.from_numpy(ca).cuda(), lda, fa, sinv[0:1], torch.from_numpy(cb).cuda(), ldb,
                      0, sinv[1:2], C, ldc, accumulate=acc, workspace=ws)
    torch.cuda.synchronize()
    got = C[:, :N].cpu()
    e = check_fp8_gemm("C", got, ref, absprod, deq)
    say(f"  error / bound {e:.3e}; k split workspace {ws_bytes} bytes")
    assert torch.all(C[:, N:] == 7.0)  # the columns past N are not touched


@pytest.mark.parametrize("act", ["swiglu", "gelu"])
def test_fp8_forward_expansion_strict(act):
    """F2 with its activation epilogue on codes of given tensors (N with
    NORMED_READY, the weights): pre-activations and activation within the
    bf16 tolerance; the weight codes bit for bit."""
    from tensor_transformer_mlp_rmsnorm_amd import _lib as L
    T, H, F = 200, 272, 144
    P = 2 * F if act == "swiglu" else F
    Tp = (T + 15) // 16 * 16
    rng = np.random.default_rng(17 + (act == "gelu"))
    bf = lambda v: torch.from_numpy(np.asarray(v, np.float32)).to(torch.bfloat16)
    normed = bf(rng.standard_normal((T, H)) * (1 + (rng.random((T, 1)) < 0.05) * 3))
    w_in = bf(rng.standard_normal((2, F, H) if act == "swiglu" else (F, H)) * 0.05)
    b_in = None if act == "swiglu" else bf(0.1 * rng.standard_normal(F))
    w_down = bf(rng.standard_normal((H, F)) * 0.05)
    sc = _meta_scales(rng, fp8.ROLES)
    Lh = 4
    metas = {k: meta_tensor(_fmt_code(k), Lh, scale=sc[k]) for k in fp8.ROLES}
    say(f"[gpu] fp8 forward strict {act} T={T} H={H} F={F}")
    u8 = lambda *shape: torch.zeros(shape, dtype=torch.uint8, device="cuda")
    codes = dict(normed_q=u8(T, H), normed_t=u8(H, Tp), w_in_q=u8(P, H), w_in_t=u8(H, P), act_q=u8(T, F),
                 act_t=u8(F, Tp), w_down_q=u8(H, F), w_down_t=u8(F, H), d_out_q=None, d_out_t=None, d_pre_q=None,
                 d_pre_t=None)
    nd = normed.cuda()
    L.tp_mlp_fp8_cast(T, H, nd, 0, metas["normed"], codes["normed_q"], codes["normed_t"], Tp)
    f8 = L.make_fp8_args(Lh, **{"meta_" + k: m for k, m in metas.items()}, **codes)
    pre = torch.empty((T, P), dtype=torch.bfloat16, device="cuda")
    actd = torch.empty((T, F), dtype=torch.bfloat16, device="cuda")
    z = torch.empty((T, H), dtype=torch.float32, device="cuda")
    rstd = torch.ones(T, dtype=torch.float32, device="cuda")
    desc = L.make_desc(T, H, F, L.ACT_SWIGLU if act == "swiglu" else L.ACT_GELU, L.BF16, 1e-6, L.NORMED_READY)
    L.tp_mlp_forward_fp8(desc, nd, torch.ones(H, dtype=torch.bfloat16, device="cuda"), w_in.cuda(),
                         None if b_in is None else b_in.cuda(), w_down.cuda(), nd, rstd, pre, actd, z, None, f8)
    torch.cuda.synchronize()
    # oracle: the expansion on the codes of N and W_in, the activation on the stored pre-activations
    R = oracle.bf16_round
    om = {k: fp8.Fp8Meta(fp8.ROLES[k], np.zeros(Lh, np.float32), sc[k]) for k in fp8.ROLES}
    n64 = normed.double().numpy()
    wrows = w_in.double().numpy().reshape(P, H)
    nq = fp8.quantize(n64, sc["normed"], fp8.E4M3)
    wq = fp8.quantize(wrows, sc["w_in"], fp8.E4M3)
    np.testing.assert_array_equal(codes["w_in_q"].cpu().numpy(), wq)
    np.testing.assert_array_equal(codes["w_in_t"].cpu().numpy(), wq.T)
    np.testing.assert_array_equal(codes["w_down_q"].cpu().numpy(), fp8.quantize(w_down.double().numpy(),
                                                                                sc["w_down"], fp8.E4M3))
    h = fp8.fp8_gemm_nt(nq, om["normed"], wq, om["w_in"])
    if act == "swiglu":
        g, u = R(h[:, :F]), R(h[:, F:])
        pre_ref, act_ref = np.concatenate([g, u], 1), R(oracle.silu(g) * u)
    else:
        pre_ref = R(h + b_in.double().numpy()[None, :])
        act_ref = R(oracle.gelu(pre_ref))
    report = {}
    check("pre_act", pre.cpu(), pre_ref, "bf16", rowwise=True, report=report)
    check("act", actd.cpu(), act_ref, "bf16", rowwise=True, report=report)
    # the amax of every cast of this forward
    for k, ref_amax in (("normed", np.abs(n64).max()), ("w_in", np.abs(wrows).max()),
                        ("w_down", np.abs(w_down.double().numpy()).max())):
        assert metas[k].cpu().numpy()[2] == np.float32(ref_amax), k
    say(f"  worst: {max(report.items(), key=lambda kv: kv[1])}")


@pytest.mark.parametrize("act", ["swiglu", "gelu"])
def test_fp8_backward_strict(act):
    """The backward's d_act GEMM with the activation backward fused, and the
    down-weight gradient, on codes of given tensors (d_out, act, the weights):
    d_pre within the bf16 tolerance, d_w_down within the FP8 GEMM bound, the
    d_out codes and d_pre's codes (formed in the d_act epilogue) bit for bit.  The two GEMMs on the codes of d_pre follow the
    step criterion (d_pre is computed, its codes can flip)."""
    from tensor_transformer_mlp_rmsnorm_amd import _lib as L
    T, H, F = 136, 256, 144
    P = 2 * F if act == "swiglu" else F
    Tp = (T + 15) // 16 * 16
    rng = np.random.default_rng(23 + (act == "gelu"))
    bf = lambda v: torch.from_numpy(np.asarray(v, np.float32)).to(torch.bfloat16)
    d_out = bf(rng.standard_normal((T, H)))
    normed = bf(rng.standard_normal((T, H)))
    pre_act = bf(rng.standard_normal((T, P)))
    actv = bf(rng.standard_normal((T, F)) * 0.5)
    w_in = bf(rng.standard_normal((2, F, H) if act == "swiglu" else (F, H)) * 0.05)
    w_down = bf(rng.standard_normal((H, F)) * 0.05)
    sc = _meta_scales(rng, fp8.ROLES)
    Lh = 4
    metas = {k: meta_tensor(_fmt_code(k), Lh, scale=sc[k]) for k in fp8.ROLES}
    say(f"[gpu] fp8 backward strict {act} T={T} H={H} F={F}")
    u8 = lambda *shape: torch.zeros(shape, dtype=torch.uint8, device="cuda")
    codes = dict(normed_q=None, normed_t=u8(H, Tp), w_in_q=None, w_in_t=u8(H, P), act_q=None, act_t=u8(F, Tp),
                 w_down_q=None, w_down_t=u8(F, H), d_out_q=u8(T, H), d_out_t=u8(H, Tp), d_pre_q=u8(T, P),
                 d_pre_t=u8(P, Tp))
    cu = {k: v.cuda() for k, v in dict(d_out=d_out, normed=normed, pre_act=pre_act, act=actv, w_in=w_in,
                                       w_down=w_down).items()}
    # the forward's transposed codes, cast from the given tensors
    L.tp_mlp_fp8_cast(T, H, cu["normed"], 0, metas["normed"], None, codes["normed_t"], Tp)
    L.tp_mlp_fp8_cast(T, F, cu["act"], 0, metas["act"], None, codes["act_t"], Tp)
    L.tp_mlp_fp8_cast(P, H, cu["w_in"], 0, metas["w_in"], None, codes["w_in_t"], P)
    L.tp_mlp_fp8_cast(H, F, cu["w_down"], 0, metas["w_down"], None, codes["w_down_t"], H)
    f8 = L.make_fp8_args(Lh, **{"meta_" + k: m for k, m in metas.items()}, **codes)
    f32 = lambda *shape: torch.zeros(shape, dtype=torch.float32, device="cuda")
    outs = dict(d_pre=torch.empty((T, P), dtype=torch.bfloat16, device="cuda"), d_w_in=f32(*w_in.shape),
                d_b_in=None if act == "swiglu" else f32(F), d_w_down=f32(H, F), d_normed_part=f32(T, H))
    desc = L.make_desc(T, H, F, L.ACT_SWIGLU if act == "swiglu" else L.ACT_GELU, L.BF16, 1e-6, 0)
    ws = torch.empty(max(L.tp_mlp_workspace_bytes(desc, L.BWD_SHARD), 16), dtype=torch.uint8, device="cuda")
    L.tp_mlp_backward_fp8(desc, L.BWD_SHARD, f8, normed=cu["normed"], pre_act=cu["pre_act"], act=cu["act"],
                          w_in=cu["w_in"], w_down=cu["w_down"], d_out=cu["d_out"], workspace=ws, **outs)
    torch.cuda.synchronize()
    R = oracle.bf16_round
    om = {k: fp8.Fp8Meta(fp8.ROLES[k], np.zeros(Lh, np.float32), sc[k]) for k in fp8.ROLES}
    dy = d_out.double().numpy()
    dyq = fp8.quantize(dy, sc["d_out"], fp8.E5M2)
    np.testing.assert_array_equal(codes["d_out_q"].cpu().numpy(), dyq)
    np.testing.assert_array_equal(codes["d_out_t"].cpu().numpy()[:, :T], dyq.T)
    assert np.all(codes["d_out_t"].cpu().numpy()[:, T:] == 0)
    wdq = fp8.quantize(w_down.double().numpy(), sc["w_down"], fp8.E4M3)
    aq = fp8.quantize(actv.double().numpy(), sc["act"], fp8.E4M3)
    da = fp8.fp8_gemm_nt(dyq, om["d_out"], wdq.T, om["w_down"])
    pre64 = pre_act.double().numpy()
    pre = (pre64[:, :F], pre64[:, F:]) if act == "swiglu" else (pre64,)
    dP = fp8._act_bwd(da, pre, act, R)
    report = {}
    check("d_pre", outs["d_pre"].cpu(), dP, "bf16", rowwise=True, report=report)
    dwd = fp8.fp8_gemm_nt(dyq.T, om["d_out"], aq.T, om["act"])
    deq = float(np.float32(om["d_out"].scale_inv()) * np.float32(om["act"].scale_inv()))
    absprod = np.abs(fp8.decode(dyq, fp8.E5M2)).T @ np.abs(fp8.decode(aq, fp8.E4M3))
    check_fp8_gemm("d_w_down", outs["d_w_down"].cpu(), dwd, absprod, deq, report=report)
    # the GEMMs on d_pre's codes
    dpq = fp8.quantize(dP, sc["d_pre"], fp8.E5M2)
    wq = fp8.quantize(w_in.double().numpy().reshape(P, H), sc["w_in"], fp8.E4M3)
    nq = fp8.quantize(normed.double().numpy(), sc["normed"], fp8.E4M3)
    check_fp8_step("d_normed_part", outs["d_normed_part"].cpu(), fp8.fp8_gemm_nt(dpq, om["d_pre"], wq.T, om["w_in"]),
                   report=report)
    check_fp8_step("d_w_in", outs["d_w_in"].cpu().reshape(P, H), fp8.fp8_gemm_nt(dpq.T, om["d_pre"], nq.T,
                                                                                om["normed"]), report=report)
    if act == "gelu":
        check("d_b_in", outs["d_b_in"].cpu(), np.sum(dP, axis=0), "bf16", report=report)
    assert metas["d_out"].cpu().numpy()[2] == np.float32(np.abs(dy).max())
    # d_pre's codes, formed in the d_act GEMM's epilogue: the oracle's quantisation of the stored d_pre, bit for
    # bit (row copy, transposed copy, zero padding columns T .. Tp-1), and its amax in the meta
    dp_gpu = outs["d_pre"].cpu().double().numpy()
    dpq_gpu = fp8.quantize(dp_gpu, sc["d_pre"], fp8.E5M2)
    np.testing.assert_array_equal(codes["d_pre_q"].cpu().numpy(), dpq_gpu)
    np.testing.assert_array_equal(codes["d_pre_t"].cpu().numpy()[:, :T], dpq_gpu.T)
    assert np.all(codes["d_pre_t"].cpu().numpy()[:, T:] == 0)
    assert metas["d_pre"].cpu().numpy()[2] == np.float32(np.abs(dp_gpu).max())
    say(f"  worst: {report}")


SMALL = [
    # name,                  T,   H,   F_full, S, act
    ("swiglu_S2", 300, 256, 384, 2, "swiglu"),
    ("gelu_ragged_S2", 129, 272, 288, 2, "gelu"),
    ("swiglu_S1_fused", 200, 128, 144, 1, "swiglu"),
    ("swiglu_S4_T40", 40, 512, 1024, 4, "swiglu"),
]


def _step_outputs(w, res, d):
    g, npar = d["grads"], d["new_params"]
    items = [("out", res["out"], d["out"]), ("normed", res["normed"], d["n"]), ("act", res["act"], d["a"]),
             ("dN", res["dN"], d["dN"]), ("dx", res["dx"], d["dx"]), ("d_norm_w", res["d_norm_w"], g["norm_w"]),
             ("d_b_down", res["d_b_down"], g["b_down"]), ("d_w_in", res["d_w_in"], g["w_in"]),
             ("d_w_down", res["d_w_down"], g["w_down"]), ("new_w_in", res["new_w_in"], npar.w_in),
             ("new_w_down", res["new_w_down"], npar.w_down), ("new_norm_w", res["new_norm_w"], npar.norm_w),
             ("new_b_down", res["new_b_down"], npar.b_down)]
    if w.act == "gelu":
        items += [("d_b_in", res["d_b_in"], g["b_in"]), ("new_b_in", res["new_b_in"], npar.b_in)]
    return items


@pytest.mark.parametrize("case", SMALL, ids=[c[0] for c in SMALL])
def test_fp8_step_small_parity(case):
    """The whole FP8 step (shards in sequence, shared metas) against
    oracle.fp8_dense_step, a cold step and then a warm one from the oracle's
    metas: every output within the step criterion, the weight gradients at
    most a third as far from the FP8 oracle as from the bf16 one, and the
    metas afterwards those of this step's amaxes."""
    from tensor_transformer_mlp_rmsnorm_amd.step import Fp8Step
    name, T, H, Ff, S, act = case
    w = synth.Workload("fp8_" + name, tokens=T, hidden=H, ffn_full=Ff, shards=S, act=act, dtype="bf16",
                       w_std=0.05, seed=500 + T)
    t = synth.draw(w, perturb=True)
    x, p = synth.to_numpy64(t["x"]), np_params(t)
    Lh = 8
    say(f"[gpu] fp8 step {name} T={T} H={H} F_full={Ff} S={S} {act}")
    st = Fp8Step(w, t, out_of_place_sgd=True, history_len=Lh)
    om = fp8.new_metas(Lh)
    bf = oracle.dense_step(x, p, act, w.eps, w.lr, storage="bf16")
    for phase in ("cold", "warm"):
        if phase == "warm":
            # both sides start the second step from the oracle's metas after the first
            st.load_meta_state(_state_of(om))
        st.step()
        torch.cuda.synchronize()
        res = st.results()
        d = fp8.fp8_dense_step(x, p, act, w.eps, w.lr, om, storage="bf16")
        report = {}
        for k, got, ref in _step_outputs(w, res, d):
            check_fp8_step(k, got, ref, report=report)
        say(f"  {phase} worst: {max(report.items(), key=lambda kv: kv[1])}")
        for key, ref8, ref16 in (("d_w_in", d["grads"]["w_in"], bf["grads"]["w_in"]),
                                 ("d_w_down", d["grads"]["w_down"], bf["grads"]["w_down"])):
            e8, e16 = frob_rel(res[key], ref8), frob_rel(res[key], ref16)
            assert e8 < e16 / 3, (phase, key, e8, e16)
        gs = st.meta_state()
        for k, m in om.items():
            sc, si, am, hist = gs[k]
            assert am == 0.0, k
            h = hist.numpy()
            np.testing.assert_array_equal(h[1:], m.history[1:])
            assert abs(h[0] - m.history[0]) <= 2e-2 * abs(m.history[0]), (k, h[0], m.history[0])
            assert sc == np.float32(m.fmt.max / float(h.max())), k
            assert si == np.float32(1.0 / sc), k


def test_fp8_full_size_sampled():
    """The Llama-3-8B TP=8 workload in the configuration bench.py times
    (Fp8Step, out-of-place SGD): a cold step, then a warm step from the
    oracle's metas after the first, each against oracle.fp8_sampled_step on
    the whole output and sampled rows / FFN channels / hidden columns, by the
    step criterion."""
    import time
    from tensor_transformer_mlp_rmsnorm_amd.step import Fp8Step
    from test_gpu_parity import _gather, _sample
    w = synth.workload("llama3_8b_tp8")
    t = synth.draw(w)
    Lh = 16
    say(f"[gpu] fp8 full size {w.name} T={w.tokens} H={w.hidden} F_full={w.ffn_full} S={w.shards}")
    st = Fp8Step(w, t, out_of_place_sgd=True, history_len=Lh)
    rng = np.random.default_rng(w.seed + 7)
    rows = _sample(rng, w.tokens, 32, must=[0, w.tokens - 1])
    chans = _sample(rng, w.ffn_full, 32, must=[0, w.ffn_full - 1, w.ffn_local - 1, w.ffn_local])
    cols = _sample(rng, w.hidden, 32, must=[0, w.hidden - 1])
    om = fp8.new_metas(Lh)
    x32, p = synth.to_numpy64(t["x"]).astype(np.float32), np_params(t)
    for phase in ("cold", "warm"):
        if phase == "warm":
            st.load_meta_state(_state_of(om))
        st.step()
        torch.cuda.synchronize()
        got = _gather(st, rows, chans, cols)
        t0 = time.time()
        ref = fp8.fp8_sampled_step(x32, p, w.act, w.eps, w.lr, om, rows, chans, cols, dtype=np.float32)
        say(f"  {phase}: oracle sampled FP8 step {time.time() - t0:.1f} s")
        report = {}
        for k in ("out", "dx_rows", "dN_rows", "act_chans", "d_b_down", "d_norm_w_cols", "d_w_down_chans",
                  "d_w_in_chans", "new_norm_w_cols", "new_b_down", "new_w_down_chans", "new_w_in_chans"):
            check_fp8_step(k, got[k], ref[k], report=report)
        say(f"  {phase} worst: {max(report.items(), key=lambda kv: kv[1])}")
        gs = st.meta_state()
        for k, m in om.items():
            h = gs[k][3].numpy()
            assert abs(h[0] - m.history[0]) <= 2e-2 * abs(m.history[0]), (k, h[0], m.history[0])
    del st
    torch.cuda.empty_cache()


FUSED = [
    ("swiglu_S2_ragged", 200, 144, 2 * 144, 2, "swiglu"),
    ("gelu_S1_ksplit", 2500, 272, 272, 1, "gelu"),
    ("llama3_8b_tp8", None, None, None, None, None),
]


@pytest.mark.parametrize("case", FUSED, ids=[c[0] for c in FUSED])
def test_fp8_fused_update_equals_unfused_bitwise(case):
    """The FP8 step with the weight matrices' update taken in their FP8
    weight-gradient GEMMs (as bench.py times it) against the FP8 step that
    writes the gradients and runs the SGD kernels: the same fp32 gradients,
    the same update, so the new parameters and every other output are the same
    bits, over two steps (cold, then warm metas)."""
    from tensor_transformer_mlp_rmsnorm_amd.step import Fp8Step
    name, T, H, Ff, S, act = case
    if T is None:
        w = synth.workload(name)
    else:
        w = synth.Workload("fp8_fused_" + name, tokens=T, hidden=H, ffn_full=Ff, shards=S, act=act, dtype="bf16",
                           w_std=0.05, seed=700 + T)
    t = synth.draw(w, perturb=T is not None)
    say(f"[gpu] fp8 fused update {name} T={w.tokens} H={w.hidden} F_full={w.ffn_full} S={w.shards} {w.act}")
    ref = Fp8Step(w, t, out_of_place_sgd=False, history_len=8)
    got = Fp8Step(w, t, out_of_place_sgd=False, history_len=8, fused_sgd=True)
    bits = lambda x: x.view(torch.int16 if x.element_size() == 2 else torch.int32)
    for step in range(2):
        ref.step()
        got.step()
        torch.cuda.synchronize()
        for pname, _ in ref._param_list():
            diff = int((bits(got.new[pname]) != bits(ref.new[pname])).sum())
            assert diff == 0, (step, pname, diff)
        for attr in ("out", "dx", "d_norm_w", "d_b_down"):
            assert torch.equal(bits(getattr(got, attr)), bits(getattr(ref, attr))), (step, attr)
        for k in ("meta_w_in", "meta_d_pre", "meta_act"):
            assert torch.equal(got.metas[k], ref.metas[k]), (step, k)
    say(f"  two steps, {len(ref._param_list())} parameters: same bits")
    del ref, got
    torch.cuda.empty_cache()
