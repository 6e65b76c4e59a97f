"""tp_mlp_backward_noalloc (the backward with the library's own scratch, for
callers that cannot allocate) against tp_mlp_backward with a caller
workspace: identical results, bit for bit, on two calls in a row whose second
has fewer tokens (a different k split of the weight-gradient GEMMs), in both
phases, for SwiGLU and GeLU; a call needing more scratch than the library
holds is rejected before any work."""

import dataclasses

import pytest
import torch

import synth

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from tensor_transformer_mlp_rmsnorm_amd import _lib
    _lib.lib()
    yield


def _run_both(w, t):
    """Forward once, then each backward phase through both entry points
    into separate outputs; returns the pairs of outputs."""
    from tensor_transformer_mlp_rmsnorm_amd import _lib as L
    from tensor_transformer_mlp_rmsnorm_amd.step import ShardedStep

    st = ShardedStep(w, t, device="cuda:0")
    st.forward()
    sh = st.shards[0]
    desc = st._desc()
    print(f"[gpu] noalloc {w.name} T={w.tokens} H={w.hidden} F={w.ffn_local} {w.act}: "
          f"SHARD scratch {L.tp_mlp_workspace_bytes(desc, L.BWD_SHARD)} B, "
          f"NORM scratch {L.tp_mlp_workspace_bytes(desc, L.BWD_NORM)} B", flush=True)
    outs = []
    for noalloc in (False, True):
        o = {k: torch.full_like(sh[k], float("nan")) for k in ("d_pre", "d_w_in", "d_w_down", "dN_part")}
        o["d_b_in"] = None if sh["d_b_in"] is None else torch.full_like(sh["d_b_in"], float("nan"))
        kw = dict(normed=st.normed, pre_act=sh["pre"], act=sh["act"], w_in=sh["w_in"], w_down=sh["w_down"],
                  d_out=st.out, d_pre=o["d_pre"], d_w_in=o["d_w_in"], d_b_in=o["d_b_in"],
                  d_w_down=o["d_w_down"], d_normed_part=o["dN_part"])
        if noalloc:
            L.tp_mlp_backward_noalloc(desc, L.BWD_SHARD, **kw)
        else:
            L.tp_mlp_backward(desc, L.BWD_SHARD, workspace=st.workspace, **kw)
        o["dx"] = torch.full_like(st.dx, float("nan"))
        o["d_norm_w"] = torch.full_like(st.d_norm_w, float("nan"))
        o["d_b_down"] = torch.full_like(st.d_b_down, float("nan"))
        kw = dict(x=st.x, rstd=st.rstd, norm_w=st.norm_w, d_out=st.out, d_normed=o["dN_part"], d_x=o["dx"],
                  d_norm_w=o["d_norm_w"], d_b_down=o["d_b_down"])
        if noalloc:
            L.tp_mlp_backward_noalloc(desc, L.BWD_NORM, **kw)
        else:
            L.tp_mlp_backward(desc, L.BWD_NORM, workspace=st.workspace, **kw)
        outs.append(o)
    torch.cuda.synchronize()
    return outs


@pytest.mark.parametrize("act", ["swiglu", "gelu"])
def test_noalloc_backward_equals_workspace_backward(act):
    # the first call k-splits the down weight gradient 4 ways (K = 4096 tokens), the second 2 ways
    base = synth.Workload(f"noalloc_{act}", tokens=4096, hidden=768, ffn_full=1024, shards=1, act=act,
                          dtype="bf16", w_std=0.04, seed=21)
    for w in (base, dataclasses.replace(base, name=base.name + "_smaller", tokens=2500, seed=22)):
        ref, got = _run_both(w, synth.draw(w, perturb=True))
        for k in ref:
            if ref[k] is None:
                continue
            assert not torch.isnan(got[k]).any(), k
            assert torch.equal(got[k], ref[k]), k


def test_noalloc_rejects_scratch_beyond_its_size():
    from tensor_transformer_mlp_rmsnorm_amd import _lib as L

    # the bf16 d_act GEMM reads W_d transposed from the scratch: 2 F H bytes > 128 MiB
    desc = L.make_desc(1, 16384, 8192, L.ACT_SWIGLU, L.BF16, 1e-6, 0)
    need = L.tp_mlp_workspace_bytes(desc, L.BWD_SHARD)
    assert need > L.NOALLOC_SCRATCH_BYTES
    dummy = torch.empty(16, dtype=torch.bfloat16, device="cuda:0")
    with pytest.raises(L.TPMLPError) as e:
        L.tp_mlp_backward_noalloc(desc, L.BWD_SHARD, normed=dummy, pre_act=dummy, act=dummy, w_in=dummy,
                                  w_down=dummy, d_out=dummy, d_pre=dummy, d_w_in=dummy, d_w_down=dummy,
                                  d_normed_part=dummy)
    assert "scratch" in str(e.value)
