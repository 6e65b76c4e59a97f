"""Pins of the sequence-parallel oracle.  Sequence parallelism only moves
where the two boundary sums happen (an all-gather and a reduce-scatter
instead of an all-reduce) and which rows each rank's norm sees, so its step
must reproduce the dense step exactly; its one extra reduction (the norm
weight and bias gradients summed over the ranks) is pinned by its ablation:
the per-rank gradients add up to the dense gradient and each alone differs."""

import numpy as np
import pytest

import oracle
from oracle.mlp import Params
from oracle.sequence import sequence_parallel_step, sequence_slices


def _block(seed, T, H, F, act, std=0.3):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((T, H))
    w_in = rng.standard_normal((2, F, H) if act == "swiglu" else (F, H)) * std
    b_in = 0.3 * rng.standard_normal(F) if act == "gelu" else None
    p = Params(1.0 + 0.3 * rng.standard_normal(H), w_in, rng.standard_normal((H, F)) * std,
               0.3 * rng.standard_normal(H), b_in)
    return x, p


def test_sequence_slices_partition():
    for T in (0, 1, 7, 8, 9):
        for S in (1, 2, 3, 4):
            sl = sequence_slices(T, S)
            assert len(sl) == S and sl[0][0] == 0 and sl[-1][1] == T
            assert all(sl[i][1] == sl[i + 1][0] for i in range(S - 1))
            sizes = [hi - lo for lo, hi in sl]
            assert max(sizes) - min(sizes) <= 1


def _assembled(sp, key, act):
    r = sp["ranks"]
    if key == "w_in":
        return np.concatenate([q["grads"]["w_in"] for q in r], axis=1 if act == "swiglu" else 0)
    if key == "w_down":
        return np.concatenate([q["grads"]["w_down"] for q in r], axis=1)
    if key == "b_in":
        return np.concatenate([q["grads"]["b_in"] for q in r])
    raise KeyError(key)


@pytest.mark.parametrize("act", ["swiglu", "gelu"])
@pytest.mark.parametrize("S,T", [(1, 7), (2, 8), (2, 7), (3, 7), (4, 9)])
def test_sequence_parallel_step_is_the_dense_step(act, S, T):
    x, p = _block(21, T, 8, 12, act)
    sp = sequence_parallel_step(x, p, act, 1e-6, 0.1, S)
    d = oracle.dense_step(x, p, act, 1e-6, 0.1)
    close = lambda a, b: np.testing.assert_allclose(a, b, rtol=1e-12, atol=1e-12)
    close(sp["out"], d["out"])
    close(sp["loss"], d["loss"])
    close(sp["dx"], d["dx"])
    close(sp["n"], d["n"])
    for k in ("w_in", "w_down") + (("b_in",) if act == "gelu" else ()):
        close(_assembled(sp, k, act), d["grads"][k])
    for rk in sp["ranks"]:
        close(rk["d_norm_w"], d["grads"]["norm_w"])
        close(rk["d_b_down"], d["grads"]["b_down"])
        close(rk["new_params"].norm_w, d["new_params"].norm_w)
        close(rk["new_params"].b_down, d["new_params"].b_down)
    # each rank's slice of the reduce-scattered dN is the dense dN on those rows
    for rk in sp["ranks"]:
        close(rk["dN"], d["dN"][rk["lo"]:rk["hi"]])


def test_sequence_parallel_partials_match_tensor_parallel_ranks():
    # inside the tensor-parallel region nothing changes: rank r's partial is the TP rank's partial
    x, p = _block(22, 8, 8, 12, "swiglu")
    sp = sequence_parallel_step(x, p, "swiglu", 1e-6, 0.1, 2)
    tp = oracle.sharded_step(x, p, "swiglu", 1e-6, 0.1, 2)
    for a, b in zip(sp["ranks"], tp["ranks"]):
        np.testing.assert_allclose(a["z"], b["z"], rtol=1e-13, atol=1e-14)
        np.testing.assert_allclose(a["dN_part"], b["dN_partial"], rtol=1e-13, atol=1e-14)


@pytest.mark.parametrize("act", ["swiglu", "gelu"])
def test_missing_norm_grad_reduce_signature(act):
    x, p = _block(23, 9, 8, 12, act, std=0.5)
    S = 3
    ab = sequence_parallel_step(x, p, act, 1e-6, 0.1, S, mode="missing_norm_grad_reduce")
    d = oracle.dense_step(x, p, act, 1e-6, 0.1)
    local_w = [rk["d_norm_w"] for rk in ab["ranks"]]
    local_b = [rk["d_b_down"] for rk in ab["ranks"]]
    # the per-rank gradients are slices of one sum
    np.testing.assert_allclose(sum(local_w), d["grads"]["norm_w"], rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(sum(local_b), d["grads"]["b_down"], rtol=1e-12, atol=1e-12)
    scale = np.abs(d["grads"]["norm_w"]).max()
    for lw in local_w:
        assert np.abs(lw - d["grads"]["norm_w"]).max() > 1e-2 * scale
    # nothing else moves: forward, dx and the tensor-parallel weight gradients are exact
    np.testing.assert_allclose(ab["out"], d["out"], rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(ab["dx"], d["dx"], rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(_assembled(ab, "w_in", act), d["grads"]["w_in"], rtol=1e-12, atol=1e-12)
    # the replicated weights drift apart across ranks after the update
    nw = [rk["new_params"].norm_w for rk in ab["ranks"]]
    assert max(np.abs(a - b).max() for a in nw for b in nw) > 0
