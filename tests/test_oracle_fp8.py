"""Pins of the FP8 oracle (oracle/fp8.py) against what fixes it from outside:
PyTorch's float8_e4m3fn / float8_e5m2 conversions (a library routine) for the
codec, the formats' closed-form extremes, the round-to-nearest-even rule at
every tie, the delayed-scaling rule on a hand-worked amax sequence, exactness
when the operands lie on the FP8 grid, the elementwise error bound of a
product of quantised operands for every GEMM of the step, and the sharded step
equal to the dense step when the shards share their metas."""

import numpy as np
import pytest
import torch

import oracle
from oracle import fp8
from oracle.fp8 import E4M3, E5M2
from oracle.mlp import Params

TORCH = {"e4m3": torch.float8_e4m3fn, "e5m2": torch.float8_e5m2}


def torch_codes(y, fmt):
    t = torch.from_numpy(np.asarray(y, dtype=np.float32))
    return t.to(TORCH[fmt.name]).view(torch.uint8).numpy()


def finite_codes(fmt):
    c = np.arange(256, dtype=np.uint8)
    return c[np.isfinite(fp8.decode(c, fmt))]


@pytest.mark.parametrize("fmt", [E4M3, E5M2], ids=["e4m3", "e5m2"])
def test_decode_matches_torch_for_every_code(fmt):
    c = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(c).view(TORCH[fmt.name]).float().double().numpy()
    got = fp8.decode(c, fmt)
    same = (got == ref) | (np.isnan(got) & np.isnan(ref))
    assert same.all(), c[~same]


def test_closed_form_extremes():
    d4 = lambda c: float(fp8.decode(np.uint8(c), E4M3))
    d5 = lambda c: float(fp8.decode(np.uint8(c), E5M2))
    assert d4(0x7E) == 448.0 and np.isnan(d4(0x7F)) and d4(0x01) == 2.0 ** -9 and d4(0x08) == 2.0 ** -6
    assert d4(0x38) == 1.0 and d4(0xB8) == -1.0
    assert d5(0x7B) == 57344.0 and d5(0x7C) == np.inf and d5(0x01) == 2.0 ** -16 and d5(0x04) == 2.0 ** -14
    assert d5(0x3C) == 1.0
    assert len(finite_codes(E4M3)) == 254 and len(finite_codes(E5M2)) == 248


@pytest.mark.parametrize("fmt", [E4M3, E5M2], ids=["e4m3", "e5m2"])
def test_round_trip_and_monotone(fmt):
    c = finite_codes(fmt)
    c = c[c != 0x80]  # -0 encodes back to 0x80 only through its sign bit; checked separately
    np.testing.assert_array_equal(fp8.encode(fp8.decode(c, fmt), fmt), c)
    assert fp8.encode(np.array([-0.0]), fmt)[0] == 0x80
    pos = np.sort(fp8.decode(c[c < 0x80], fmt))
    assert np.all(np.diff(pos) > 0)


@pytest.mark.parametrize("fmt", [E4M3, E5M2], ids=["e4m3", "e5m2"])
def test_encode_matches_torch_at_ties_and_random_values(fmt):
    v = np.sort(np.unique(np.abs(fp8.decode(finite_codes(fmt), fmt))))
    mids = (v[:-1] + v[1:]) / 2                        # every tie of round-to-nearest
    rng = np.random.default_rng(7)
    rand = np.concatenate([rng.uniform(-fmt.max, fmt.max, 20000),
                           rng.standard_normal(20000) * 2.0 ** rng.integers(-18, 12, 20000)])
    rand = np.clip(rand, -fmt.max, fmt.max).astype(np.float32).astype(np.float64)
    near = np.concatenate([mids * (1 + 2.0 ** -20), mids * (1 - 2.0 ** -20)])
    y = np.concatenate([mids, -mids, rand, near[np.abs(near) <= fmt.max], v, -v])
    np.testing.assert_array_equal(fp8.encode(y, fmt), torch_codes(y, fmt))


def test_ties_go_to_even_mantissa():
    # 1.0625 lies between 1.0 (mantissa 0) and 1.125 (mantissa 1); 1.1875 between 1.125 and 1.25 (mantissa 2)
    assert fp8.encode(np.array([1.0625]), E4M3)[0] == 0x38
    assert fp8.encode(np.array([1.1875]), E4M3)[0] == 0x3A
    # the subnormal / normal boundary: 15/16 of the smallest normal rounds to it (even code 0x08)
    assert fp8.encode(np.array([2.0 ** -6 * 15 / 16]), E4M3)[0] == 0x08


def test_quantize_clamps_and_uses_the_fp32_product():
    q = fp8.quantize(np.array([1e4, -1e4, 500.0]), 1.0, E4M3)
    np.testing.assert_array_equal(q, [0x7E, 0xFE, 0x7E])
    assert fp8.quantize(np.array([1e9]), 1.0, E5M2)[0] == 0x7B
    # a case where the exact x*s lies just above a tie but its fp32 rounding is the tie itself:
    # the fp32 product decides (ties to the even code, below), the exact one would round up
    found = None
    for x in (3.0, 5.0, 7.0, 9.0, 11.0, 13.0):
        s = np.nextafter(np.float32(3.125 / x), np.float32(np.inf))
        exact = float(x) * float(s)
        if exact > 3.125 and np.float32(x) * s == np.float32(3.125):
            found = (x, s, exact)
            break
    assert found is not None
    x, s, exact = found
    assert fp8.quantize(np.array([x]), s, E4M3)[0] == fp8.encode(np.array([3.0]), E4M3)[0]
    assert fp8.encode(np.array([exact]), E4M3)[0] == fp8.encode(np.array([3.25]), E4M3)[0]


def test_delayed_scaling_rule_worked_sequence():
    m = fp8.Fp8Meta.new(E4M3, 3)
    assert m.scale == 1.0 and m.scale_inv() == 1.0
    expect = []
    hist = []
    for amax in (2.0, 8.0, 1.0, 0.5, 0.25):
        m.record(np.array([amax, -amax / 2]))
        m.record(np.array([amax / 4]))
        m.update()
        hist = ([amax] + hist)[:3]
        expect.append(448.0 / max(hist))
        assert m.amax == 0.0
        np.testing.assert_array_equal(m.history[:len(hist)], np.float32(hist))
        assert m.scale == np.float32(expect[-1])
    assert expect == [224.0, 56.0, 56.0, 56.0, 448.0]
    # an all-zero history keeps the scale; so does a non-finite amax
    z = fp8.Fp8Meta.new(E5M2, 2)
    z.update()
    assert z.scale == 1.0
    z.record(np.array([4.0]))
    z.update()
    assert z.scale == np.float32(57344.0 / 4.0)
    z.amax = np.float32(np.inf)
    z.update()
    assert z.scale == np.float32(57344.0 / 4.0)
    # the amax is that of the values, not of the scaled values; NaN elements do not count, inf does
    w = fp8.Fp8Meta.new(E4M3, 1)
    w.scale = np.float32(64.0)
    fp8.cast(np.array([-3.0, 2.0]), w)
    assert w.amax == 3.0
    w.record(np.array([np.nan, -5.0]))
    assert w.amax == 5.0
    w.record(np.array([np.nan]))
    assert w.amax == 5.0
    w.record(np.array([-np.inf]))
    assert w.amax == np.inf


@pytest.mark.parametrize("fa,fb", [(E4M3, E4M3), (E5M2, E4M3)], ids=["e4m3xe4m3", "e5m2xe4m3"])
def test_gemm_is_exact_on_the_grid(fa, fb):
    rng = np.random.default_rng(3)
    ca = rng.choice(finite_codes(fa), size=(9, 40))
    cb = rng.choice(finite_codes(fb), size=(7, 40))
    sa, sb = np.float32(2.0 ** 5), np.float32(2.0 ** -3)   # powers of two: x * s is exact
    a = fp8.decode(ca, fa) / float(sa)
    b = fp8.decode(cb, fb) / float(sb)
    ma, mb = fp8.Fp8Meta.new(fa, 1), fp8.Fp8Meta.new(fb, 1)
    ma.scale, mb.scale = sa, sb
    qa, qb = fp8.cast(a, ma), fp8.cast(b, mb)
    np.testing.assert_array_equal(fp8.decode(qa, fa), fp8.decode(ca, fa))
    np.testing.assert_array_equal(fp8.decode(qb, fb), fp8.decode(cb, fb))
    np.testing.assert_allclose(fp8.fp8_gemm_nt(qa, ma, qb, mb), a @ b.T, rtol=1e-13, atol=1e-300)


def _block(seed, T, H, F, act, std=0.05):
    rng = np.random.default_rng(seed)
    bf = oracle.bf16_round
    x = bf(rng.standard_normal((T, H)))
    w_in = bf(rng.standard_normal((2, F, H) if act == "swiglu" else (F, H)) * std)
    b_in = bf(0.1 * rng.standard_normal(F)) if act == "gelu" else None
    p = Params(bf(1.0 + 0.1 * rng.standard_normal(H)), w_in, bf(rng.standard_normal((H, F)) * std),
               bf(0.1 * rng.standard_normal(H)), b_in)
    return x, p


def _warm_metas(x, p, act, L=4):
    """The metas as one earlier step on the same block leaves them."""
    metas = fp8.new_metas(L)
    fp8.fp8_dense_step(x, p, act, 1e-6, 0.1, metas)
    return metas


@pytest.mark.parametrize("act", ["swiglu", "gelu"])
@pytest.mark.parametrize("warm", [False, True], ids=["cold", "warm"])
def test_every_gemm_within_the_quantisation_bound(act, warm):
    x, p = _block(5, 24, 48, 40, act)
    metas = _warm_metas(x, p, act) if warm else fp8.new_metas(4)
    sc = {k: m.scale for k, m in metas.items()}
    r = fp8.fp8_dense_step(x, p, act, 1e-6, 0.1, metas)
    R = oracle.bf16_round
    wrows = fp8._w_in_rows(p.w_in, act)
    F = p.w_down.shape[1]
    checks = []
    # F2: the stored pre-activations against the exact product of the same N and W_in
    h = r["n"] @ wrows.T
    b2 = fp8.product_error_bound(r["n"], wrows, sc["normed"], sc["w_in"], E4M3, E4M3)
    pre = np.concatenate(r["pre"], axis=1) if act == "swiglu" else r["pre"][0] - p.b_in[None, :]
    checks.append(("F2", pre, h, b2 + 2.0 ** -8 * np.abs(pre) + 1e-12))
    # F3, d_act, dW_down, dN, dW_in: the exact products of the step's own operands
    checks.append(("F3", r["z"], r["a"] @ p.w_down.T,
                   fp8.product_error_bound(r["a"], p.w_down, sc["act"], sc["w_down"], E4M3, E4M3)))
    checks.append(("d_act", r["da"], r["dY"] @ p.w_down,
                   fp8.product_error_bound(r["dY"], p.w_down.T, sc["d_out"], sc["w_down"], E5M2, E4M3)))
    checks.append(("dW_down", r["grads"]["w_down"], r["dY"].T @ r["a"],
                   fp8.product_error_bound(r["dY"].T, r["a"].T, sc["d_out"], sc["act"], E5M2, E4M3)))
    checks.append(("dN", r["dN"], r["dP"] @ wrows,
                   fp8.product_error_bound(r["dP"], wrows.T, sc["d_pre"], sc["w_in"], E5M2, E4M3)))
    checks.append(("dW_in", r["grads"]["w_in"].reshape(wrows.shape), r["dP"].T @ r["n"],
                   fp8.product_error_bound(r["dP"].T, r["n"].T, sc["d_pre"], sc["normed"], E5M2, E4M3)))
    for name, got, exact, bound in checks:
        err = np.abs(got - exact)
        assert np.all(err <= bound), (name, float((err / bound).max()))
        # and the FP8 rounding is really there: the error is not negligible against the bound
        assert err.max() > 1e-3 * bound.max(), name
    # the bf16 steps between the GEMMs are those of the dense step, on this step's tensors
    if act == "swiglu":
        g, u = r["pre"]
        np.testing.assert_array_equal(r["a"], R(oracle.silu(g) * u))
    assert r["scale_inv"]["normed"] == np.float32(1.0 / float(sc["normed"]))


def test_fp8_step_is_close_to_the_exact_step():
    # with warm scales the FP8 step tracks the full-precision step to a few percent of each tensor's scale
    x, p = _block(6, 32, 64, 48, "swiglu")
    r = fp8.fp8_dense_step(x, p, "swiglu", 1e-6, 0.1, _warm_metas(x, p, "swiglu"))
    d = oracle.dense_step(x, p, "swiglu", 1e-6, 0.1, storage="bf16")
    for k, a, b in (("out", r["out"], d["out"]), ("dx", r["dx"], d["dx"]),
                    ("w_in", r["grads"]["w_in"], d["grads"]["w_in"]),
                    ("w_down", r["grads"]["w_down"], d["grads"]["w_down"])):
        rel = np.abs(a - b).max() / np.abs(b).max()
        assert 1e-4 < rel < 0.1, (k, rel)


@pytest.mark.parametrize("act", ["swiglu", "gelu"])
@pytest.mark.parametrize("S", [1, 2, 4])
def test_sharded_step_equals_dense_step(act, S):
    x, p = _block(8, 16, 32, 48, act)
    md, ms = _warm_metas(x, p, act), _warm_metas(x, p, act)
    d = fp8.fp8_dense_step(x, p, act, 1e-6, 0.1, md)
    s = fp8.fp8_sharded_step(x, p, act, 1e-6, 0.1, S, ms)
    close = lambda a, b: np.testing.assert_allclose(a, b, rtol=1e-12, atol=1e-12)
    close(s["out"], d["out"])
    close(s["dx"], d["dx"])
    close(s["d_norm_w"], d["grads"]["norm_w"])
    F = p.w_down.shape[1] // S
    for i, rk in enumerate(s["ranks"]):
        close(rk["grads"]["w_down"], d["grads"]["w_down"][:, i * F:(i + 1) * F])
        wi = d["grads"]["w_in"]
        close(rk["grads"]["w_in"], wi[:, i * F:(i + 1) * F] if act == "swiglu" else wi[i * F:(i + 1) * F])
    # the shared metas saw the group's amax: the same state after both steps
    for k in md:
        assert md[k].scale == ms[k].scale, k
        np.testing.assert_array_equal(md[k].history, ms[k].history)


def test_metas_follow_the_step_amaxes_over_steps():
    x, p = _block(9, 16, 32, 24, "swiglu")
    metas = fp8.new_metas(2)
    seen = []
    for step in range(3):
        before = {k: m.scale for k, m in metas.items()}
        r = fp8.fp8_dense_step(x, p, "swiglu", 1e-6, 0.01, metas)
        amax = {"normed": np.abs(r["n"]).max(), "act": np.abs(r["a"]).max(), "d_out": np.abs(r["dY"]).max(),
                "d_pre": np.abs(r["dP"]).max(), "w_down": np.abs(p.w_down).max(), "w_in": np.abs(p.w_in).max()}
        seen.append(amax)
        for k, m in metas.items():
            assert m.history[0] == np.float32(amax[k]), k
            assert m.scale == np.float32(m.fmt.max / max(float(s[k]) for s in seen[-2:])), k
            if step == 0:
                assert before[k] == 1.0
        p = r["new_params"]


@pytest.mark.parametrize("act", ["swiglu", "gelu"])
def test_sampled_step_is_the_dense_step(act):
    x, p = _block(12, 40, 32, 24, act)
    rows, chans, cols = [0, 7, 39], [0, 5, 23], [0, 9, 31]
    for warm in (False, True):
        md = _warm_metas(x, p, act) if warm else fp8.new_metas(4)
        ms = fp8.copy_metas(md)
        d = fp8.fp8_dense_step(x, p, act, 1e-6, 0.1, md)
        s = fp8.fp8_sampled_step(x, p, act, 1e-6, 0.1, ms, rows, chans, cols, dtype=np.float64)
        close = lambda a, b: np.testing.assert_allclose(a, b, rtol=1e-11, atol=1e-12)
        close(s["out"], d["out"])
        close(s["act_chans"], d["a"][:, chans])
        close(s["d_b_down"], d["grads"]["b_down"])
        close(s["dN_rows"], d["dN"][rows])
        close(s["dx_rows"], d["dx"][rows])
        close(s["d_w_down_chans"], d["grads"]["w_down"][:, chans])
        wi = d["grads"]["w_in"]
        close(s["d_w_in_chans"], wi[:, chans] if act == "swiglu" else wi[chans])
        close(s["d_norm_w_cols"], d["grads"]["norm_w"][cols])
        close(s["new_w_down_chans"], d["new_params"].w_down[:, chans])
        close(s["new_norm_w_cols"], d["new_params"].norm_w[cols])
        if act == "gelu":
            close(s["d_b_in"], d["grads"]["b_in"])
        for k in md:
            assert md[k].scale == ms[k].scale
            np.testing.assert_array_equal(md[k].history, ms[k].history)
