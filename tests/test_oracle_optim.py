"""Pins of the optimiser oracle (gradient accumulation, global-norm clipping,
AdamW) against things other than itself: PyTorch's own AdamW and
clip_grad_norm_ (library routines), closed forms of the update, and the
identity that the summed gradients of a batch's microbatches are the
gradients of the batch."""

import numpy as np
import pytest
import torch

import oracle


def _tensors(seed, shapes):
    rng = np.random.default_rng(seed)
    return [rng.standard_normal(s) for s in shapes]


SHAPES = [(5,), (3, 4), (2, 3, 2)]


def test_adamw_matches_torch_adamw_over_steps():
    params = _tensors(1, SHAPES)
    lr, wd, b1, b2, eps = 3e-3, 0.1, 0.9, 0.95, 1e-6
    tp = [torch.tensor(p, dtype=torch.float64, requires_grad=True) for p in params]
    opt = torch.optim.AdamW(tp, lr=lr, betas=(b1, b2), eps=eps, weight_decay=wd)
    ours = [p.copy() for p in params]
    m = [np.zeros_like(p) for p in params]
    v = [np.zeros_like(p) for p in params]
    for step in range(1, 7):
        grads = _tensors(100 + step, SHAPES)
        for t, g in zip(tp, grads):
            t.grad = torch.tensor(g, dtype=torch.float64)
        opt.step()
        for i, g in enumerate(grads):
            ours[i], m[i], v[i] = oracle.adamw_update(ours[i], g, m[i], v[i], step, lr, wd, b1, b2, eps)
        for t, o in zip(tp, ours):
            np.testing.assert_allclose(o, t.detach().numpy(), rtol=1e-13, atol=1e-15)


def test_adamw_first_step_closed_form():
    # step 1, no decay: m_hat = g and sqrt(v_hat) = |g|, so the move is lr * g / (|g| + eps)
    theta, g = _tensors(2, [(7,), (7,)])
    lr, eps = 1e-2, 1e-8
    new, m, v = oracle.adamw_update(theta, g, np.zeros(7), np.zeros(7), 1, lr, 0.0, eps=eps)
    np.testing.assert_allclose(new, theta - lr * g / (np.abs(g) + eps), rtol=1e-14, atol=1e-16)
    np.testing.assert_allclose(m, (1 - oracle.ADAM_BETA1) * g, rtol=1e-15)
    np.testing.assert_allclose(v, (1 - oracle.ADAM_BETA2) * g * g, rtol=1e-15)


def test_adamw_constant_gradient_closed_form():
    # with the same g every step the bias-corrected moments are exactly g and g^2
    theta, g = _tensors(3, [(6,), (6,)])
    lr, eps = 5e-3, 1e-8
    m = v = np.zeros(6)
    cur = theta
    for step in range(1, 11):
        cur, m, v = oracle.adamw_update(cur, g, m, v, step, lr, 0.0, eps=eps)
    np.testing.assert_allclose(cur, theta - 10 * lr * g / (np.abs(g) + eps), rtol=1e-12, atol=1e-14)


def test_adamw_pure_decay_closed_form():
    # zero gradient: only the decoupled decay acts, theta_t = theta_0 (1 - lr wd)^t
    theta = _tensors(4, [(5,)])[0]
    lr, wd = 1e-2, 0.1
    m = v = np.zeros(5)
    cur = theta
    for step in range(1, 6):
        cur, m, v = oracle.adamw_update(cur, np.zeros(5), m, v, step, lr, wd)
    np.testing.assert_allclose(cur, theta * (1 - lr * wd) ** 5, rtol=1e-14)


def test_adamw_grad_scale_is_a_gradient_multiplier():
    theta, g = _tensors(5, [(4,), (4,)])
    a = oracle.adamw_update(theta, g, np.zeros(4), np.zeros(4), 1, 1e-3, 0.1, grad_scale=0.25)
    b = oracle.adamw_update(theta, 0.25 * g, np.zeros(4), np.zeros(4), 1, 1e-3, 0.1)
    for x, y in zip(a, b):
        np.testing.assert_allclose(x, y, rtol=1e-15)


def test_clip_matches_torch_clip_grad_norm():
    grads = _tensors(6, SHAPES)
    for max_norm in (0.5, 1.0, 100.0):
        tg = [torch.tensor(g, dtype=torch.float64, requires_grad=True) for g in grads]
        for t, g in zip(tg, grads):
            t.grad = torch.tensor(g, dtype=torch.float64)
        total = torch.nn.utils.clip_grad_norm_(tg, max_norm)
        norm = oracle.global_grad_norm(grads)
        assert norm == pytest.approx(float(total), rel=1e-14)
        c = oracle.clip_coefficient(norm, max_norm)
        for t, g in zip(tg, grads):
            np.testing.assert_allclose(c * g, t.grad.numpy(), rtol=1e-14)


def test_clip_closed_form_and_off():
    assert oracle.global_grad_norm([np.array([3.0]), np.array([[4.0]])]) == 5.0
    assert oracle.clip_coefficient(5.0, 1.0) == pytest.approx(1.0 / (5.0 + 1e-6), rel=1e-15)
    assert oracle.clip_coefficient(5.0, 10.0) == 1.0
    assert oracle.clip_coefficient(5.0, 0.0) == 1.0


def test_adamw_step_clips_then_updates():
    params = dict(zip("abc", _tensors(7, SHAPES)))
    grads = dict(zip("abc", _tensors(8, SHAPES)))
    zeros = {k: np.zeros_like(p) for k, p in params.items()}
    out = oracle.adamw_step(params, grads, zeros, zeros, 1, 1e-3, 0.1, max_norm=0.5)
    assert out["norm"] == pytest.approx(oracle.global_grad_norm(list(grads.values())), rel=1e-15)
    assert out["coef"] < 1
    for k in params:
        ref = oracle.adamw_update(params[k], grads[k], zeros[k], zeros[k], 1, 1e-3, 0.1, grad_scale=out["coef"])
        np.testing.assert_allclose(out["params"][k], ref[0], rtol=1e-15)


def test_microbatch_bounds_partition():
    for T in (1, 7, 8, 100):
        for M in (1, 2, 3, 7):
            b = oracle.microbatch_bounds(T, M)
            assert len(b) == M and b[0][0] == 0 and b[-1][1] == T
            assert all(b[i][1] == b[i + 1][0] for i in range(M - 1))
            sizes = [hi - lo for lo, hi in b]
            assert max(sizes) - min(sizes) <= 1 and sizes == sorted(sizes, reverse=True)


def _block(seed, T, H, F, act):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((T, H))
    w_in = rng.standard_normal((2, F, H) if act == "swiglu" else (F, H)) * 0.3
    b_in = 0.3 * rng.standard_normal(F) if act == "gelu" else None
    p = oracle.Params(1.0 + 0.3 * rng.standard_normal(H), w_in, rng.standard_normal((H, F)) * 0.3,
                      0.3 * rng.standard_normal(H), b_in)
    return x, p


@pytest.mark.parametrize("act", ["swiglu", "gelu"])
@pytest.mark.parametrize("M", [1, 2, 3, 7])
def test_accumulated_grads_equal_whole_batch_grads(act, M):
    # the loss is a sum over token rows, so per-microbatch gradients add up to the batch gradient
    x, p = _block(9, 7, 8, 12, act)  # 7 rows: ragged slices for M = 2, 3
    whole = oracle.dense_step(x, p, act, 1e-6, 0.0)["grads"]
    acc = oracle.accumulated_grads(x, p, act, 1e-6, M)
    for k, g in whole.items():
        if g is None:
            continue
        np.testing.assert_allclose(acc[k], g, rtol=1e-12, atol=1e-14)
