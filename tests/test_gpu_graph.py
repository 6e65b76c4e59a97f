"""The training step captured in a HIP graph (torch.cuda.CUDAGraph) and replayed.

The library allocates no device memory and records no memset, copy or
synchronisation inside a step, so a whole step (forward, backward, update)
can be captured.  Each replay here is followed by eager work on the device
(an eager step of a second instance on the same inputs) and a
synchronisation, and every replay's outputs must equal that eager step's
element for element, bit for bit.
"""

import sys

import pytest
import torch

import synth

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


CASES = [
    # shards in sequence with both transposed weight copies (bf16), ragged in every dimension
    ("graph_swiglu_bf16_s2", dict(tokens=300, hidden=264, ffn_full=560, shards=2, act="swiglu", dtype="bf16")),
    # one shard: the fused residual epilogue, the GeLU path and its bias gradient
    ("graph_gelu_bf16_s1", dict(tokens=260, hidden=192, ffn_full=320, shards=1, act="gelu", dtype="bf16")),
    ("graph_swiglu_fp32_s2", dict(tokens=64, hidden=64, ffn_full=128, shards=2, act="swiglu", dtype="fp32")),
    # the benchmark's form of the step: the weight matrices' update fused into their gradient GEMMs, the gate/up
    # weight gradient on N^T and d_pre^T (T a multiple of 8, one k range), and with k split (the slices' update)
    ("graph_swiglu_bf16_s2_fused", dict(tokens=304, hidden=264, ffn_full=560, shards=2, act="swiglu", dtype="bf16",
                                        fused=True)),
    ("graph_swiglu_bf16_s2_fused_ksplit", dict(tokens=2504, hidden=264, ffn_full=560, shards=2, act="swiglu",
                                               dtype="bf16", fused=True)),
]


def _equal(a, b) -> bool:
    if a is None or b is None:
        return a is None and b is None
    if isinstance(a, list):
        return len(a) == len(b) and all(_equal(x, y) for x, y in zip(a, b))
    return torch.equal(a, b)


@pytest.mark.parametrize("name,kw", CASES, ids=[c[0] for c in CASES])
def test_graph_replays_equal_eager_steps(name, kw):
    from tensor_transformer_mlp_rmsnorm_amd.step import ShardedStep

    kw = dict(kw)
    fused = kw.pop("fused", False)
    w = synth.Workload(name, w_std=0.05, seed=31, **kw)
    t = synth.draw(w)
    say(f"[gpu] {name}: T={w.tokens} H={w.hidden} F_full={w.ffn_full} S={w.shards} {w.act} {w.dtype} fused={fused}")
    st = ShardedStep(w, t, out_of_place_sgd=True, fused_sgd=fused)
    ref = ShardedStep(w, t, out_of_place_sgd=True, fused_sgd=fused)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        st.step()  # first launches outside the capture
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        st.step()
    torch.cuda.synchronize()
    for rep in range(3):
        g.replay()
        ref.step()  # eager work between the replays
        torch.cuda.synchronize()
        got, want = st.results(), ref.results()
        assert sorted(got) == sorted(want)
        bad = [k for k in want if not _equal(got[k], want[k])]
        say(f"  replay {rep}: {len(want)} tensors, {len(bad)} differ")
        assert not bad, f"replay {rep}: {bad} differ from the eager step"
