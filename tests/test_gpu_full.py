"""Full-size parity of the step in the benchmark's configuration.

Each full workload (GPT-2-small GeLU tp=1, Llama-3-8B TP=8 with all 8
shards, one Llama-3-70B TP=8 rank, Llama-3-8B full width with fp32 masters)
runs once on the GPU as bench.py times it (ShardedStep, new parameters
written out of place) but with the weight gradients written; every tensor it
stores is copied to the host, and then:

* test_fused_update_bitwise: the step exactly as bench.py times it, with the
  weight matrices' SGD update taken inside their weight-gradient GEMMs
  (gradients never written), gives the same bits in every parameter,
  transposed copy, master, out, dx and norm/bias gradient.

* test_stage: every kernel's output, element by element over the whole
  tensor, against the fp64 oracle stage fed the GPU's own stored inputs
  (tests/stagewise.py), within the bf16 bound 2e-2 (floored relative).
* test_end_to_end: every tensor of the step against the fp64 oracle's whole
  dense step (storage model: each stored activation rounded to bf16 once),
  element by element within 2e-2, except the activation, the pre-activation
  gradients, dN and dx.  For those, any correct fp32-accumulating
  implementation sits up to 1.9e-2 (act, dN, dx) and 5.5e-2 (pre-activation
  gradients) from the fp64 oracle end to end at these sizes, measured with
  the oracle itself run in fp32 arithmetic: a stored bf16 pre-activation g or
  u whose exact value lies next to a rounding midpoint is rounded one way in
  fp32 and the other in fp64; the flip moves a by up to 2^-8 |g u|, that
  channel's column of W_d spreads it over the row of z and of out (flipping
  many of the row's stored outputs), and since d out = out it returns through
  W_d^T into the same channel's d_act with gain |W_d[:, j]|^2 (about 1.6 at
  these shapes).  Those four are held to 2e-2 stage by stage, and their
  end-to-end error is printed.  The full-width workload (34.6 TFLOP and
  ~470 M-element activation tensors per dense oracle step) is compared end to
  end on sampled rows, channels and columns that the oracle computes exactly
  (oracle.sampled_step), in fp32 accumulation.
* test_against_exact_storage: every tensor of the dense workloads against
  the fp64 oracle with no storage rounding at all (storage="exact").  The
  bound 2e-2 is asserted for each tensor on which the bf16 storage model
  itself stays within 1.5e-2 of exact; on the others bf16 storage alone
  (one rounding of each stored activation, every contraction exact) already
  moves the result past or near 2e-2 -- at Llama-3-8B TP=8: out 2.1e-2,
  act 5.1e-2, dN 2.4e-2, dx 3.7e-2, the weight gradients 2.9-3.9e-2,
  the pre-activation gradients 0.11 -- so there the GPU is held to at most
  twice the storage model's own distance from exact, and both are printed.
"""

import sys
import time

import numpy as np
import pytest
import torch

import oracle
import synth
from oracle.mlp import Params
from stagewise import STAGES, collect, run_stage
from tolerance import check, floored_rel

pytestmark = pytest.mark.gpu

FULL = ["gpt2s_gelu_tp1", "llama3_8b_tp8", "llama3_70b_tp8_rank", "llama3_8b_tp1_master"]
DENSE_END_TO_END = {"gpt2s_gelu_tp1", "llama3_8b_tp8", "llama3_70b_tp8_rank"}


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", params=FULL)
def full(request):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from tensor_transformer_mlp_rmsnorm_amd import _lib
    from tensor_transformer_mlp_rmsnorm_amd.step import ShardedStep

    _lib.lib()  # must load: there is no fallback
    w = synth.workload(request.param)
    t = synth.draw(w)
    say(f"[gpu] full {w.name} T={w.tokens} H={w.hidden} F_full={w.ffn_full} S={w.shards} {w.act} {w.dtype}")
    st = ShardedStep(w, t, device="cuda:0", out_of_place_sgd=True)
    st.step()
    torch.cuda.synchronize()
    h = collect(st)
    # the benchmark's step takes the weight matrices' update inside their weight-gradient GEMMs: its
    # new parameters (transposed copies, masters) must be the bits of the step above
    fu = ShardedStep(w, t, device="cuda:0", out_of_place_sgd=True, fused_sgd=True)
    fu.step()
    torch.cuda.synchronize()
    bits = lambda x: x.view(torch.int16 if x.element_size() == 2 else torch.int32)
    diff = lambda a, b: int((bits(a) != bits(b)).sum())
    mism = {}
    for name, _ in st._param_list():
        mism["new " + name] = diff(fu.new[name], st.new[name])
        if w.master:
            mism["master " + name] = diff(fu.new_masters[name], st.new_masters[name])
    for key, (tt, _, _) in st.new_t.items():
        mism["transposed " + key] = diff(fu.new_t[key][0], tt)
    for attr in ("out", "dx", "d_norm_w", "d_b_down"):
        mism[attr] = diff(getattr(fu, attr), getattr(st, attr))
    h["fused_mismatch"] = mism
    del st, fu
    torch.cuda.empty_cache()
    yield w, t, h


def test_fused_update_bitwise(full):
    """The step as the benchmark times it (update fused into the weight-gradient
    GEMMs) writes the same bits as the step whose every tensor is checked here."""
    w, _, h = full
    bad = {k: v for k, v in h["fused_mismatch"].items() if v}
    say(f"  {w.name}: fused vs unfused, {len(h['fused_mismatch'])} tensors compared, differing: {bad}")
    assert not bad


@pytest.mark.parametrize("stage", STAGES)
def test_stage(full, stage):
    w, t, h = full
    report = {}
    t0 = time.time()
    try:
        run_stage(stage, w, t, h, report)
    finally:
        say(f"  {w.name} {stage}: " + ", ".join(f"{k} {v:.2e}" for k, v in report.items())
            + f"  ({time.time() - t0:.1f} s)")


def _np_params(t) -> Params:
    c = synth.to_numpy64
    return Params(c(t["norm_w"]), c(t["w_in"]), c(t["w_down"]), c(t["b_down"]), c(t["b_in"]))


def _cat_shards(h, key, axis):
    return torch.cat([sh[key].float() for sh in h["shards"]], dim=axis)


def _pre_of_shards(w, pre_tuple, s):
    """The oracle's dense pre-activations (or their gradients) sliced to shard s's [T, P] layout."""
    lo, hi = s * w.ffn_local, (s + 1) * w.ffn_local
    return np.concatenate([p[:, lo:hi] for p in pre_tuple], axis=1)


_DENSE = {}


def _dense(w, t, storage):
    """The fp64 oracle's dense step of workload w, kept for the tests of the
    same workload (one workload's steps at a time)."""
    key = (w.name, storage)
    if key not in _DENSE:
        for k in [k for k in _DENSE if k[0] != w.name]:
            del _DENSE[k]
        t0 = time.time()
        _DENSE[key] = oracle.dense_step(synth.to_numpy64(t["x"]), _np_params(t), w.act, w.eps, w.lr,
                                        storage=storage)
        say(f"  oracle dense step (fp64, {storage} storage): {time.time() - t0:.1f} s")
    return _DENSE[key]


def test_end_to_end(full):
    w, t, h = full
    report, printed = {}, {}
    t0 = time.time()
    if w.name not in DENSE_END_TO_END:
        _sampled_end_to_end(w, t, h, report)
        say(f"  {w.name} end-to-end (sampled): " + ", ".join(f"{k} {v:.2e}" for k, v in report.items())
            + f"  ({time.time() - t0:.1f} s)")
        return
    d = _dense(w, t, "bf16")
    g, npar = d["grads"], d["new_params"]
    swiglu = w.act == "swiglu"
    fails = []

    def cmp(name, got, ref, rowwise):
        try:
            check(name, got, ref, w.dtype, rowwise=rowwise, report=report)
        except AssertionError as e:
            fails.append(str(e))

    cmp("normed", h["normed"], d["n"], True)
    cmp("out", h["out"], d["out"], True)
    for s, sh in enumerate(h["shards"]):
        cmp(f"pre[{s}]", sh["pre"], _pre_of_shards(w, d["pre"], s), True)
    cmp("d_w_in", _cat_shards(h, "d_w_in", 1 if swiglu else 0), g["w_in"], False)
    cmp("d_w_down", _cat_shards(h, "d_w_down", 1), g["w_down"], False)
    cmp("d_norm_w", h["d_norm_w"], g["norm_w"], False)
    cmp("d_b_down", h["d_b_down"], g["b_down"], False)
    new = h["new"]
    n = len(h["shards"])
    cmp("new_norm_w", new["norm_w"], npar.norm_w, False)
    cmp("new_b_down", new["b_down"], npar.b_down, False)
    cmp("new_w_in", torch.cat([new[f"w_in.{s}"].float() for s in range(n)], dim=1 if swiglu else 0), npar.w_in, False)
    cmp("new_w_down", torch.cat([new[f"w_down.{s}"].float() for s in range(n)], dim=1), npar.w_down, False)
    if not swiglu:
        cmp("d_b_in", _cat_shards(h, "d_b_in", 0), g["b_in"], False)
        cmp("new_b_in", torch.cat([new[f"b_in.{s}"].float() for s in range(n)]), npar.b_in, False)
    # held stage-wise (test_stage); printed here
    printed["act"] = floored_rel(_cat_shards(h, "act", 1), d["a"], True)
    printed["d_pre"] = max(floored_rel(sh["d_pre"], _pre_of_shards(w, d["d_pre"], s), True)
                           for s, sh in enumerate(h["shards"]))
    printed["dN"] = floored_rel(h["dN"], d["dN"], True)
    printed["dx"] = floored_rel(h["dx"], d["dx"], True)
    say(f"  {w.name} end-to-end: " + ", ".join(f"{k} {v:.2e}" for k, v in report.items())
        + "; stage-wise only: " + ", ".join(f"{k} {v:.2e}" for k, v in printed.items())
        + f"  ({time.time() - t0:.1f} s)")
    assert not fails, "; ".join(fails)


def _step_tensors(w, h):
    """(name, GPU tensor, field of an oracle dense step, rowwise) for every
    tensor the step stores or updates; per-shard pre-activations and their
    gradients are listed per shard."""
    swiglu = w.act == "swiglu"
    n = len(h["shards"])
    new = h["new"]
    items = [("normed", h["normed"], lambda d: d["n"], True),
             ("out", h["out"], lambda d: d["out"], True),
             ("act", _cat_shards(h, "act", 1), lambda d: d["a"], True),
             ("dN", h["dN"], lambda d: d["dN"], True),
             ("dx", h["dx"], lambda d: d["dx"], True),
             ("d_w_in", _cat_shards(h, "d_w_in", 1 if swiglu else 0), lambda d: d["grads"]["w_in"], False),
             ("d_w_down", _cat_shards(h, "d_w_down", 1), lambda d: d["grads"]["w_down"], False),
             ("d_norm_w", h["d_norm_w"], lambda d: d["grads"]["norm_w"], False),
             ("d_b_down", h["d_b_down"], lambda d: d["grads"]["b_down"], False),
             ("new_norm_w", new["norm_w"], lambda d: d["new_params"].norm_w, False),
             ("new_b_down", new["b_down"], lambda d: d["new_params"].b_down, False),
             ("new_w_in", torch.cat([new[f"w_in.{s}"].float() for s in range(n)], dim=1 if swiglu else 0),
              lambda d: d["new_params"].w_in, False),
             ("new_w_down", torch.cat([new[f"w_down.{s}"].float() for s in range(n)], dim=1),
              lambda d: d["new_params"].w_down, False)]
    if not swiglu:
        items += [("d_b_in", _cat_shards(h, "d_b_in", 0), lambda d: d["grads"]["b_in"], False),
                  ("new_b_in", torch.cat([new[f"b_in.{s}"].float() for s in range(n)]),
                   lambda d: d["new_params"].b_in, False)]
    for s, sh in enumerate(h["shards"]):
        items.append((f"pre[{s}]", sh["pre"], lambda d, s=s: _pre_of_shards(w, d["pre"], s), True))
        items.append((f"d_pre[{s}]", sh["d_pre"], lambda d, s=s: _pre_of_shards(w, d["d_pre"], s), True))
    return items


EXACT_ASSERTED_BELOW = 1.5e-2  # storage model's own distance from exact under which 2e-2 is asserted


def test_against_exact_storage(full):
    """The GPU step against the fp64 oracle with no bf16 storage rounding."""
    w, t, h = full
    if w.name not in DENSE_END_TO_END:
        pytest.skip("the full-width workload's dense oracle step does not fit the test's time")
    t0 = time.time()
    dm, de = _dense(w, t, "bf16"), _dense(w, t, "exact")
    held, storage_bound = [], []
    fails = []
    for name, got, field, rowwise in _step_tensors(w, h):
        ref = field(de)
        e_gpu = floored_rel(got, ref, rowwise)
        e_model = floored_rel(field(dm), ref, rowwise)
        if e_model <= EXACT_ASSERTED_BELOW:
            held.append((name, e_gpu, e_model))
            if not e_gpu <= 2e-2:
                fails.append(f"{name}: {e_gpu:.3e} from exact > 2e-2 (storage model {e_model:.3e})")
        else:
            storage_bound.append((name, e_gpu, e_model))
            if not e_gpu <= 2.0 * e_model:
                fails.append(f"{name}: {e_gpu:.3e} from exact > twice the storage model's {e_model:.3e}")
    fmt = lambda lst: ", ".join(f"{k} {a:.2e} (model {b:.2e})" for k, a, b in lst)
    say(f"  {w.name} against exact storage, held to 2e-2: {fmt(held)}")
    say(f"  {w.name} against exact storage, bf16 storage alone {EXACT_ASSERTED_BELOW:.1e}+: {fmt(storage_bound)}"
        f"  ({time.time() - t0:.1f} s)")
    assert not fails, "; ".join(fails)


def _sample(rng, n, k, must=()):
    k = min(k, n)
    s = set(int(v) for v in must if 0 <= v < n)
    s.update(int(v) for v in rng.choice(n, size=k, replace=False))
    return np.array(sorted(s), dtype=np.int64)


def _sampled_end_to_end(w, t, h, report):
    """The whole output plus sampled token rows (dx, dN), FFN channels (act,
    weight gradients and updated weights of those channels) and hidden
    columns (norm-weight gradient and update) against oracle.sampled_step,
    which computes those entries exactly (fp32 accumulation)."""
    rng = np.random.default_rng(w.seed)
    rows = _sample(rng, w.tokens, 64, must=[0, w.tokens - 1] + t["outlier_rows"][:16].tolist())
    chans = _sample(rng, w.ffn_full, 64, must=[0, w.ffn_full - 1, w.ffn_local - 1, w.ffn_local])
    cols = _sample(rng, w.hidden, 64, must=[0, w.hidden - 1])
    ri, ci = torch.as_tensor(rows), torch.as_tensor(cols)
    F = w.ffn_local
    got = {"out": h["out"].float(), "dx_rows": h["dx"][ri].float(), "dN_rows": h["dN"][ri].float(),
           "d_norm_w_cols": h["d_norm_w"][ci], "d_b_down": h["d_b_down"],
           "new_norm_w_cols": h["new"]["norm_w"][ci].float(), "new_b_down": h["new"]["b_down"].float()}
    act, dwd, dwi, nwd, nwi = [], [], [], [], []
    for j in chans:
        s, jl = int(j) // F, int(j) % F
        sh = h["shards"][s]
        act.append(sh["act"][:, jl].float())
        dwd.append(sh["d_w_down"][:, jl])
        nwd.append(h["new"][f"w_down.{s}"][:, jl].float())
        if w.act == "swiglu":
            dwi.append(sh["d_w_in"][:, jl, :])
            nwi.append(h["new"][f"w_in.{s}"][:, jl, :].float())
        else:
            dwi.append(sh["d_w_in"][jl, :])
            nwi.append(h["new"][f"w_in.{s}"][jl, :].float())
    ax = 1 if w.act == "swiglu" else 0
    got.update(act_chans=torch.stack(act, dim=1), d_w_down_chans=torch.stack(dwd, dim=1),
               new_w_down_chans=torch.stack(nwd, dim=1), d_w_in_chans=torch.stack(dwi, dim=ax),
               new_w_in_chans=torch.stack(nwi, dim=ax))
    t0 = time.time()
    ref = oracle.sampled_step(synth.to_numpy64(t["x"]).astype(np.float32), _np_params(t), w.act, w.eps, w.lr,
                              rows, chans, cols, dtype=np.float32, storage="bf16")
    say(f"  oracle sampled step: {time.time() - t0:.1f} s")
    fails = []
    for k, rowwise in (("out", True), ("d_b_down", False), ("d_norm_w_cols", False), ("d_w_down_chans", False),
                       ("d_w_in_chans", False), ("new_norm_w_cols", False), ("new_b_down", False),
                       ("new_w_down_chans", False), ("new_w_in_chans", False)):
        try:
            check(k, got[k], ref[k], w.dtype, rowwise=rowwise, report=report)
        except AssertionError as e:
            fails.append(str(e))
    # the activation, dN and dx are held stage-wise (test_stage); printed here
    for k, rowwise in (("dx_rows", True), ("dN_rows", True), ("act_chans", False)):
        report[k + " (stage-wise only)"] = floored_rel(got[k], ref[k], rowwise)
    assert not fails, "; ".join(fails)
