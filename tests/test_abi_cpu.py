"""Host-side checks of the C ABI (no GPU needed).

The shared library loads, exports every function include/tp_mlp.h declares,
and rejects bad arguments with the documented codes.  Every call here fails
argument validation (or is a documented no-op) before any HIP call, so the
dummy pointer values below are never dereferenced or passed to a kernel.
"""

import ctypes
import os
import re

import pytest

from tensor_transformer_mlp_rmsnorm_amd import _lib as L

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "tp_mlp.h")

A = 0x10000  # an aligned dummy address, never dereferenced
MIS = 0x10008  # misaligned


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\*?\s+\*?(tp_[a-z_0-9]+)\s*\(", src, flags=re.M)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(L.LIB_PATH):
        pytest.fail(f"{L.LIB_PATH} not built; run python -m tensor_transformer_mlp_rmsnorm_amd.build")
    return L.lib()


def test_every_declared_symbol_is_exported(lib):
    names = declared_functions()
    assert set(names) == set(L.EXPORTED), names
    raw = ctypes.CDLL(L.LIB_PATH)
    for n in names:
        assert hasattr(raw, n), n


def test_no_other_c_symbols_are_exported(lib):
    """Every exported symbol with C linkage (an unmangled name) is one the
    header declares: internal helpers stay internal."""
    import shutil
    import subprocess

    nm = shutil.which("nm")
    if nm is None:
        pytest.skip("nm not available")
    out = subprocess.run([nm, "-D", "--defined-only", L.LIB_PATH], capture_output=True, text=True, check=True).stdout
    c_names = {f[2] for f in (line.split() for line in out.splitlines())
               if len(f) == 3 and f[1] == "T" and not f[2].startswith("_Z")}
    assert c_names == set(declared_functions()), sorted(c_names ^ set(declared_functions()))


def test_version(lib):
    assert "gfx950" in L.tp_mlp_version()


def _desc(T=16, H=64, F=32, act=L.ACT_SWIGLU, dt=L.BF16, eps=1e-6, flags=0):
    return L.make_desc(T, H, F, act, dt, eps, flags)


def _fwd(desc, **kw):
    args = dict(x=A, norm_w=A, w_in=A, b_in=None, w_down=A, normed=A, rstd=A, pre_act=A, act=A, out=A, b_down=A)
    args.update(kw)
    return lib_call("tp_mlp_forward", ctypes.byref(desc), *[args[k] for k in
                    ("x", "norm_w", "w_in", "b_in", "w_down", "normed", "rstd", "pre_act", "act", "out", "b_down")],
                    None)


def lib_call(name, *args):
    return getattr(L.lib(), name)(*args)


@pytest.mark.parametrize("kw,code", [
    (dict(H=60), L.ESHAPE),
    (dict(H=0), L.ESHAPE),
    (dict(H=16392), L.ESHAPE),
    (dict(F=12), L.ESHAPE),
    (dict(T=-1), L.EINVAL),
    (dict(dt=7), L.EDTYPE),
    (dict(act=3), L.EINVAL),
    (dict(flags=8), L.EINVAL),
    (dict(eps=-1.0), L.EINVAL),
    (dict(T=1 << 20, H=4096), L.ESHAPE),  # 2^32 elements in [T, H]
    (dict(T=1 << 17, H=8192), L.ESHAPE),  # 2^30 bf16 elements: past the 2 GiB operand limit
])
def test_forward_rejects_bad_descriptor(lib, kw, code):
    assert _fwd(_desc(**kw)) == code
    assert L.tp_mlp_last_error() != ""


def test_forward_workspace_bytes(lib):
    """The down projection splits k through the forward's workspace only when
    it has few tiles (bf16): the GPT-2-small shape does, the Llama shapes and
    fp32 do not; fused, z and the further slices; partial, the further slices."""
    kb = lambda **kw: L.tp_mlp_forward_workspace_bytes(_desc(**kw))
    T, H, F = 4096, 768, 3072  # 48 tiles of 256 x 256, k 3072: 3 slices
    assert kb(T=T, H=H, F=F, act=L.ACT_GELU, flags=L.FUSE_EPILOGUE) == 3 * T * H * 4
    assert kb(T=T, H=H, F=F, act=L.ACT_GELU) == 2 * T * H * 4
    assert kb(T=T, H=H, F=F, act=L.ACT_GELU, dt=L.F32) == 0
    assert kb(T=8192, H=4096, F=1792) == 0
    assert kb(T=0, H=H, F=F) == 0


def test_forward_ws_rejects_small_workspace(lib):
    d = _desc(T=4096, H=768, F=3072, act=L.ACT_GELU, flags=L.FUSE_EPILOGUE)
    need = L.tp_mlp_forward_workspace_bytes(d)
    args = (A, A, A, A, A, A, A, A, A, A, A)  # x .. b_down (b_in given: GeLU)
    assert lib.tp_mlp_forward_ws(ctypes.byref(d), *args, A, need - 16, None) == L.EWORKSPACE
    assert "workspace" in L.tp_mlp_last_error()
    assert lib.tp_mlp_forward_ws(ctypes.byref(d), *args, None, 0, None) == L.EWORKSPACE


def test_forward_pointer_checks(lib):
    assert lib.tp_mlp_forward(None, *([A] * 11), None) == L.EINVAL
    assert _fwd(_desc(), x=None) == L.EINVAL
    assert _fwd(_desc(), w_in=MIS) == L.EALIGN
    assert _fwd(_desc(), b_in=A) == L.EINVAL          # SwiGLU takes no fc1 bias
    assert _fwd(_desc(act=L.ACT_GELU), b_in=None) == L.EINVAL
    assert _fwd(_desc(flags=L.FUSE_EPILOGUE), b_down=None) == L.EINVAL
    # T = 0 is a documented no-op: succeeds without touching any buffer
    assert _fwd(_desc(T=0), x=None, normed=None, out=None) == L.OK


def _parts(ptrs):
    return (ctypes.c_void_p * max(1, len(ptrs)))(*ptrs)


def test_partial_sum_checks(lib):
    f = lib.tp_partial_sum
    assert f(None, 1, 4, 8, None, None, L.F32, A, L.F32, None) == L.EINVAL
    assert f(_parts([A]), 0, 4, 8, None, None, L.F32, A, L.F32, None) == L.EINVAL
    assert f(_parts([A] * 65), 65, 4, 8, None, None, L.F32, A, L.F32, None) == L.EINVAL
    assert f(_parts([A]), 1, 4, 6, None, None, L.F32, A + 4096, L.F32, None) == L.ESHAPE
    assert f(_parts([A]), 1, 4, 8, None, None, 5, A + 4096, L.F32, None) == L.EDTYPE
    assert f(_parts([A]), 1, 4, 8, None, None, L.F32, A, L.F32, None) == L.EINVAL    # out aliases a part
    assert f(_parts([MIS]), 1, 4, 8, None, None, L.F32, A, L.F32, None) == L.EALIGN
    assert f(_parts([None]), 1, 4, 8, None, None, L.F32, A, L.F32, None) == L.EINVAL
    assert f(_parts([A]), 1, 4, 8, MIS, None, L.F32, A + 4096, L.F32, None) == L.EALIGN
    assert f(_parts([A]), 1, 0, 8, None, None, L.F32, A + 4096, L.F32, None) == L.OK  # empty: no-op


def test_backward_checks(lib):
    d = _desc(T=128, act=L.ACT_GELU)
    need = L.tp_mlp_workspace_bytes(d, L.BWD_SHARD)
    assert need > 0
    assert L.tp_mlp_workspace_bytes(d, L.BWD_NORM) > 0
    assert L.tp_mlp_workspace_bytes(_desc(T=128, dt=L.F32), L.BWD_SHARD) == 0
    # bf16: the transposed down weight [F, H] for the d_act GEMM
    assert L.tp_mlp_workspace_bytes(_desc(T=128), L.BWD_SHARD) >= 32 * 64 * 2
    assert L.tp_mlp_workspace_bytes(_desc(T=0), L.BWD_SHARD) == 0
    a = L.tp_mlp_bwd_args()
    for name, _ in L.tp_mlp_bwd_args._fields_:
        if name not in ("workspace_bytes", "d_normed_parts", "n_d_normed_parts", "w_down_t", "w_in_t", "fused_sgd",
                        "normed_t", "d_pre_t"):
            setattr(a, name, A)
    a.workspace_bytes = need - 16
    assert lib.tp_mlp_backward(ctypes.byref(d), L.BWD_SHARD, ctypes.byref(a), None) == L.EWORKSPACE
    a.workspace_bytes = need
    assert lib.tp_mlp_backward(ctypes.byref(d), 5, ctypes.byref(a), None) == L.EINVAL
    assert lib.tp_mlp_backward(ctypes.byref(d), L.BWD_SHARD, None, None) == L.EINVAL
    a.d_w_in = MIS
    assert lib.tp_mlp_backward(ctypes.byref(d), L.BWD_SHARD, ctypes.byref(a), None) == L.EALIGN
    a.d_w_in = A
    a.d_b_in = None
    assert lib.tp_mlp_backward(ctypes.byref(d), L.BWD_SHARD, ctypes.byref(a), None) == L.EINVAL
    # NORM phase without a workspace
    a.workspace = None
    assert lib.tp_mlp_backward(ctypes.byref(d), L.BWD_NORM, ctypes.byref(a), None) == L.EWORKSPACE
    assert "workspace" in L.tp_mlp_last_error()


def test_sgd_checks(lib):
    f = lib.tp_mlp_sgd_step
    assert f(A, A, A, None, None, -1, L.BF16, 0.1, None) == L.EINVAL
    assert f(A, A, A, None, None, 8, 9, 0.1, None) == L.EDTYPE
    assert f(A, A, A, A, A, 8, L.F32, 0.1, None) == L.EDTYPE      # masters only with bf16
    assert f(A, A, A, A, None, 8, L.BF16, 0.1, None) == L.EINVAL  # master_in without master_out
    assert f(MIS, A, A, None, None, 8, L.BF16, 0.1, None) == L.EALIGN
    assert f(None, None, None, None, None, 0, L.BF16, 0.1, None) == L.OK  # n = 0: no-op


def test_sgd_multi_checks(lib):
    T = L.tp_mlp_sgd_tensor
    arr = lambda *ts: (T * max(1, len(ts)))(*ts)
    f = lib.tp_mlp_sgd_step_multi
    assert f(None, 0, L.BF16, 0.1, None) == L.OK                              # nothing to do
    assert f(None, 1, L.BF16, 0.1, None) == L.EINVAL
    assert f(arr(T(A, A, A, None, None, 8)), -1, L.BF16, 0.1, None) == L.EINVAL
    assert f(arr(T(A, A, A, None, None, 8), T(A, A, A, A, A, 8)), 2, L.BF16, 0.1, None) == L.EINVAL  # mixed masters
    assert f(arr(T(A, A, A, None, None, 8), T(A, MIS, A, None, None, 8)), 2, L.BF16, 0.1, None) == L.EALIGN
    assert f(arr(T(A, A, A, None, None, -3)), 1, L.BF16, 0.1, None) == L.EINVAL
    assert f(arr(T(None, None, None, None, None, 0)), 1, L.BF16, 0.1, None) == L.OK  # n = 0: no-op


def test_adamw_checks(lib):
    T = L.tp_mlp_adamw_tensor
    arr = lambda *ts: (T * max(1, len(ts)))(*ts)
    hp = L.make_adamw_hparams(1e-3, 1, weight_decay=0.1)
    f = lambda a, n, dt=L.BF16, h=hp, scale=None: lib.tp_mlp_adamw_step_multi(a, n, dt, ctypes.byref(h) if h else None,
                                                                                scale, None)
    plain = T(A, A, A, None, None, A, A, 8)
    withm = T(None, A, A, A, A, A, A, 8)
    assert f(None, 0) == L.OK                                     # nothing to do
    assert f(None, 1) == L.EINVAL                                 # list missing
    assert f(arr(plain), -1) == L.EINVAL
    assert f(arr(plain), 1, h=None) == L.EINVAL                   # hparams missing
    assert f(arr(plain), 1, dt=7) == L.EDTYPE
    assert f(arr(withm), 1, dt=L.F32) == L.EDTYPE                 # masters only with bf16
    assert f(arr(plain, withm), 2) == L.EINVAL                    # mixed masters
    assert f(arr(T(A, A, None, None, None, A, A, 8)), 1) == L.EINVAL   # no grad
    assert f(arr(T(A, A, A, None, None, None, A, 8)), 1) == L.EINVAL   # no m
    assert f(arr(T(None, A, A, A, None, A, A, 8)), 1) == L.EINVAL      # master_out missing
    assert f(arr(T(A, A, A, None, None, A, MIS, 8)), 1) == L.EALIGN
    assert f(arr(T(A, A, A, None, None, A, A, -1)), 1) == L.EINVAL
    assert f(arr(T(None, None, None, None, None, None, None, 0)), 1) == L.OK  # n = 0: no-op
    assert f(arr(plain), 1, scale=A + 2) == L.EALIGN                   # grad_scale must be 4-byte aligned
    for bad in (L.make_adamw_hparams(1e-3, 0), L.make_adamw_hparams(1e-3, 1, beta1=1.0),
                L.make_adamw_hparams(1e-3, 1, beta2=-0.1), L.make_adamw_hparams(1e-3, 1, eps=0.0),
                L.make_adamw_hparams(1e-3, 1, weight_decay=-1.0), L.make_adamw_hparams(float("inf"), 1)):
        assert f(arr(plain), 1, h=bad) == L.EINVAL


def test_clip_grad_norm_checks(lib):
    P = ctypes.c_void_p
    ptrs = lambda *p: (P * max(1, len(p)))(*p)
    cnts = lambda *c: (ctypes.c_int64 * max(1, len(c)))(*c)
    ws_bytes = lib.tp_mlp_clip_grad_norm_workspace_bytes
    # one fp64 partial per started 16384-element block of each tensor
    assert ws_bytes(cnts(1, 16384, 16385, 0), 4) == 8 * (1 + 1 + 2 + 0)
    assert ws_bytes(None, 0) == 0 and ws_bytes(cnts(-1), 1) == 0
    f = lib.tp_mlp_clip_grad_norm
    assert f(ptrs(A), cnts(8), -1, 1.0, A, A, A, 4096, None) == L.EINVAL
    assert f(None, None, 1, 1.0, A, A, A, 4096, None) == L.EINVAL
    assert f(ptrs(A), cnts(8), 1, 1.0, A, None, A, 4096, None) == L.EINVAL       # coef_out missing
    assert f(ptrs(A), cnts(-8), 1, 1.0, A, A, A, 4096, None) == L.EINVAL
    assert f(ptrs(None), cnts(8), 1, 1.0, A, A, A, 4096, None) == L.EINVAL
    assert f(ptrs(MIS), cnts(8), 1, 1.0, A, A, A, 4096, None) == L.EALIGN
    assert f(ptrs(A), cnts(8), 1, 1.0, A, A, None, 0, None) == L.EWORKSPACE
    assert f(ptrs(A), cnts(20000), 1, 1.0, A, A, A, 8, None) == L.EWORKSPACE      # needs 16 bytes
    assert f(ptrs(A), cnts(8), 1, 1.0, A, A, MIS, 4096, None) == L.EALIGN
    assert f(ptrs(A), cnts(8), 1, float("nan"), A, A, A, 4096, None) == L.EINVAL


def test_rmsnorm_forward_checks(lib):
    f = lib.tp_rmsnorm_forward
    assert f(-1, 64, L.BF16, 1e-6, A, A, A, A, None) == L.EINVAL
    assert f(4, 60, L.BF16, 1e-6, A, A, A, A, None) == L.ESHAPE
    assert f(4, 16392, L.BF16, 1e-6, A, A, A, A, None) == L.ESHAPE
    assert f(4, 64, 5, 1e-6, A, A, A, A, None) == L.EDTYPE
    assert f(4, 64, L.BF16, float("nan"), A, A, A, A, None) == L.EINVAL
    assert f(4, 64, L.BF16, 1e-6, None, A, A, A, None) == L.EINVAL
    assert f(4, 64, L.BF16, 1e-6, A, A, MIS, A, None) == L.EALIGN
    assert f(4, 64, L.BF16, 1e-6, A, A, A, A + 2, None) == L.EALIGN   # rstd: 4-byte alignment
    assert f(0, 64, L.BF16, 1e-6, None, None, None, None, None) == L.OK  # no rows: no-op


def test_backward_rejects_unknown_flags(lib):
    d = L.make_desc(4, 8, 8, L.ACT_SWIGLU, L.F32, 1e-6, flags=8)
    a = L.tp_mlp_bwd_args()
    assert lib.tp_mlp_backward(ctypes.byref(d), L.BWD_NORM, ctypes.byref(a), None) == L.EINVAL


def test_binding_raises_with_message(lib):
    with pytest.raises(L.TPMLPError) as ei:
        L.tp_partial_sum([A], 4, 6, None, None, L.F32, A + 4096, L.F32, stream=0)
    assert ei.value.code == L.ESHAPE and "multiple of 4" in str(ei.value)


def test_step_driver_api():
    """The step driver (the path bench.py and the GPU tests run) exposes its phases."""
    from tensor_transformer_mlp_rmsnorm_amd import step
    for m in ("forward", "backward", "backward_rows", "sgd", "adamw", "step", "results"):
        assert callable(getattr(step.ShardedStep, m, None)), m
    assert step.microbatch_bounds(7, 3) == [(0, 3), (3, 5), (5, 7)]


def _fp8_args(**kw):
    f = L.tp_mlp_fp8_args()
    f.history_len = kw.pop("history_len", 4)
    for n in L.FP8_META_FIELDS + L.FP8_CODE_FIELDS:
        setattr(f, n, kw.pop(n, A))
    assert not kw
    return f


def test_fp8_checks(lib):
    fwd = lambda d, f: lib.tp_mlp_forward_fp8(ctypes.byref(d), A, A, A, None, A, A, A, A, A, A, A,
                                              ctypes.byref(f) if f is not None else None, None)
    assert fwd(_desc(dt=L.F32), _fp8_args()) == L.EDTYPE                # bf16 only
    assert fwd(_desc(H=72), _fp8_args()) == L.ESHAPE                    # H multiple of 16
    assert fwd(_desc(F=40), _fp8_args()) == L.ESHAPE                    # F multiple of 16
    assert fwd(_desc(), None) == L.EINVAL
    assert fwd(_desc(), _fp8_args(history_len=0)) == L.EINVAL
    assert fwd(_desc(), _fp8_args(history_len=1025)) == L.EINVAL
    assert fwd(_desc(), _fp8_args(meta_act=None)) == L.EINVAL
    assert fwd(_desc(), _fp8_args(meta_act=A + 2)) == L.EALIGN
    assert fwd(_desc(), _fp8_args(act_t=MIS)) == L.EALIGN
    assert fwd(_desc(flags=8), _fp8_args()) == L.EINVAL                 # SHARED_READY is a backward flag
    # T = 0 forward: a no-op that needs no activation buffers
    assert lib.tp_mlp_forward_fp8(ctypes.byref(_desc(T=0)), None, A, A, None, A, None, None, None, None, None, A,
                                  ctypes.byref(_fp8_args(normed_q=None, normed_t=None, act_q=None, act_t=None)),
                                  None) == L.OK
    a = L.tp_mlp_bwd_args()
    for name, _ in L.tp_mlp_bwd_args._fields_:
        if name not in ("workspace_bytes", "d_normed_parts", "n_d_normed_parts", "w_down_t", "w_in_t", "fused_sgd",
                        "normed_t", "d_pre_t"):
            setattr(a, name, A)
    a.d_b_in = None
    a.workspace_bytes = 1 << 30
    bwd = lambda d, f, phase=L.BWD_SHARD: lib.tp_mlp_backward_fp8(ctypes.byref(d), phase, ctypes.byref(a),
                                                                  ctypes.byref(f), None)
    assert bwd(_desc(dt=L.F32), _fp8_args()) == L.EDTYPE
    assert bwd(_desc(), _fp8_args(), phase=3) == L.EINVAL
    assert bwd(_desc(flags=16), _fp8_args()) == L.EINVAL
    assert bwd(_desc(), _fp8_args(d_pre_t=None)) == L.EINVAL
    assert bwd(_desc(), _fp8_args(meta_d_pre=None)) == L.EINVAL
    # meta init, cast and update validate before launching
    assert lib.tp_mlp_fp8_meta_init(A, 2, 4, None) == L.EINVAL
    assert lib.tp_mlp_fp8_meta_init(A, 0, 0, None) == L.EINVAL
    assert lib.tp_mlp_fp8_meta_init(None, 0, 4, None) == L.EINVAL
    cast = lib.tp_mlp_fp8_cast
    assert cast(4, 12, A, 0, A, A, None, 0, None) == L.ESHAPE           # cols multiple of 8
    assert cast(4, 16, A, 0, A, None, None, 0, None) == L.EINVAL        # nothing to write
    assert cast(20, 16, A, 0, A, None, A, 16, None) == L.ESHAPE         # ldt < rows
    assert cast(4, 16, A, 0, A, None, A, 24, None) == L.ESHAPE          # ldt not a multiple of 16
    assert cast(4, 16, A, 5, A, A, None, 0, None) == L.EINVAL           # format
    assert cast(4, 16, A, 0, None, A, None, 0, None) == L.EINVAL        # meta
    assert cast(4, 16, MIS, 0, A, A, None, 0, None) == L.EALIGN
    assert cast(0, 16, None, 0, A, A, None, 0, None) == L.OK            # no rows, no padding: no-op
    P = ctypes.c_void_p
    upd = lib.tp_mlp_fp8_update_scales
    assert upd((P * 17)(*([A] * 17)), 17, 4, None) == L.EINVAL          # at most 16 metas
    assert upd((P * 1)(None), 1, 4, None) == L.EINVAL
    assert upd((P * 1)(A), 1, 2000, None) == L.EINVAL
    assert upd(None, 0, 4, None) == L.OK
    g = lib.tp_mlp_fp8_gemm
    sinv = A
    call = lambda M=64, N=64, K=64, lda=64, ldb=64, fa=0, fb=0, ldc=64, ws=None, wsb=0, Ap=A, C=A + 65536: \
        g(M, N, K, Ap, lda, fa, sinv, A, ldb, fb, sinv, C, ldc, 0, ws, wsb, None)
    assert call(fa=1, fb=1) == L.EINVAL                                 # (E5M2, E5M2) is not a pair
    assert call(fa=0, fb=1) == L.EINVAL
    assert call(K=40, lda=48, ldb=48) == L.ESHAPE                       # K multiple of 16
    assert call(lda=32) == L.ESHAPE                                     # lda >= K
    assert call(N=62, ldc=64) == L.ESHAPE                               # N multiple of 4
    assert call(ldc=60) == L.ESHAPE
    assert call(M=-1) == L.EINVAL
    assert call(Ap=MIS) == L.EALIGN
    assert call(C=None) == L.EINVAL
    assert call(M=0) == L.OK                                            # empty: no-op
    need = lib.tp_mlp_fp8_gemm_workspace_bytes(64, 4096, 8192, 4096)
    assert need == 7 * 64 * 4096 * 4        # 16 tiles of 256 x 256, K = 8192: 8 k-slices, 7 in the workspace
    assert call(N=4096, K=8192, lda=8192, ldb=8192, ldc=4096) == L.EWORKSPACE
    assert call(N=4096, K=8192, lda=8192, ldb=8192, ldc=4096, ws=MIS, wsb=need) == L.EALIGN



def test_attention_checks(lib):
    def desc(**kw):
        a = dict(batch=2, seq=64, hidden=128, n_q=4, n_kv=2, head_dim=64, eps=1e-6, flags=0, dtype=L.BF16)
        a.update(kw)
        return L.make_attn_desc(a["batch"], a["seq"], a["hidden"], a["n_q"], a["n_kv"], a["head_dim"], a["eps"],
                                a["flags"], a["dtype"])

    fwd = lambda d, **p: lib.tp_attn_forward(ctypes.byref(d), *[p.get(k, A) for k in (
        "x", "norm_w", "w_qkv", "w_o", "normed", "rstd", "qkv", "attn_out", "lse", "out", "b_o")],
        p.get("ws", None), p.get("ws_bytes", 0), None)
    assert fwd(desc(head_dim=96)) == L.ESHAPE                 # 64 or 128
    assert fwd(desc(n_q=3, n_kv=2)) == L.ESHAPE               # n_q a multiple of n_kv
    assert fwd(desc(dtype=L.F32)) == L.EDTYPE                 # bf16 only
    assert fwd(desc(hidden=100)) == L.ESHAPE
    assert fwd(desc(seq=1 << 22)) == L.ESHAPE                 # one sequence's QKV of 2^30 elements
    assert fwd(desc(flags=8)) == L.EINVAL
    assert fwd(desc(batch=-1)) == L.EINVAL
    assert fwd(desc(), w_qkv=None) == L.EINVAL
    assert fwd(desc(), qkv=MIS) == L.EALIGN
    assert fwd(desc(), lse=A + 2) == L.EALIGN                 # lse: 4-byte alignment
    assert fwd(desc(flags=L.FUSE_EPILOGUE), b_o=None) == L.EINVAL
    assert fwd(desc(seq=0), x=None, qkv=None, out=None) == L.OK   # no tokens: a no-op
    assert lib.tp_attn_forward(None, *([A] * 11), None, 0, None) == L.EINVAL
    fneed = lib.tp_attn_forward_workspace_bytes(ctypes.byref(desc(batch=1, seq=8192, hidden=4096, n_q=4, n_kv=1,
                                                                  head_dim=128)))
    assert fneed >= 2 * 8192 * 768 * 4                         # the QKV product's k slices (fp32)
    big = desc(batch=1, seq=8192, hidden=4096, n_q=4, n_kv=1, head_dim=128)
    assert fwd(big, ws=A, ws_bytes=fneed - 16) == L.EWORKSPACE
    assert fwd(big, ws=MIS, ws_bytes=fneed) == L.EALIGN
    assert lib.tp_attn_forward_workspace_bytes(ctypes.byref(desc())) == 0   # K = 128: no split
    d = desc()
    need = lib.tp_attn_workspace_bytes(ctypes.byref(d), L.BWD_SHARD)
    assert need >= 4 * 2 * 64 * 4                              # delta [n_q, T] at least
    a = L.tp_attn_bwd_args()
    for name, _ in L.tp_attn_bwd_args._fields_:
        if name not in ("workspace_bytes", "d_normed_parts", "n_d_normed_parts", "w_down_t", "w_in_t", "fused_sgd",
                        "normed_t", "d_pre_t"):
            setattr(a, name, A)
    a.workspace_bytes = need - 16
    assert lib.tp_attn_backward(ctypes.byref(d), L.BWD_SHARD, ctypes.byref(a), None) == L.EWORKSPACE
    a.workspace_bytes = need
    assert lib.tp_attn_backward(ctypes.byref(d), 7, ctypes.byref(a), None) == L.EINVAL
    a.d_qkv = MIS
    assert lib.tp_attn_backward(ctypes.byref(d), L.BWD_SHARD, ctypes.byref(a), None) == L.EALIGN
    bare = lib.tp_attention_forward
    assert bare(1, 8, 2, 1, 64, A, 200, A, A, None) == L.ESHAPE          # ld < (n_q + 2 n_kv) D
    assert bare(1, 8, 2, 1, 64, A, 260, A, A, None) == L.ESHAPE          # ld not a multiple of 8
    assert bare(1, 8, 2, 1, 32, A, 256, A, A, None) == L.ESHAPE          # head_dim
    assert bare(1, 1 << 22, 2, 1, 64, A, 256, A, A, None) == L.ESHAPE    # one sequence of 2^30 elements
    assert bare(0, 8, 2, 1, 64, None, 256, None, None, None) == L.OK     # empty
    bb = lib.tp_attention_backward
    wsb = lib.tp_attention_backward_workspace_bytes
    assert wsb(1, 8, 2, 2, 64) >= 2 * 8 * 4                    # delta [n_q, T]
    assert wsb(1, 8, 2, 1, 64) >= wsb(1, 8, 2, 2, 64) + 2 * 8 * 2 * 64 * 4   # + per-head dK/dV shares
    assert wsb(1, 8, 0, 1, 64) == 0
    need_b = wsb(1, 8, 2, 1, 64)
    assert bb(1, 8, 2, 1, 64, A, 256, A, A, A, None, need_b, A, None) == L.EWORKSPACE   # workspace missing
    assert bb(1, 8, 2, 1, 64, A, 256, A, A, A, A, need_b - 4, A, None) == L.EWORKSPACE  # too small
    assert bb(1, 8, 2, 1, 64, A, 256, A, A, A, MIS, need_b, A, None) == L.EALIGN
    assert bb(0, 8, 2, 1, 64, None, 256, None, None, None, None, 0, None, None) == L.OK  # empty


def test_backward_fused_sgd_checks(lib):
    """The SHARD phase with the update fused (tp_mlp_fused_sgd): bf16 only,
    not with accumulated gradients, targets present and aligned, a master's
    output given with it, and the gradients then optional; the same checks in
    the FP8 backward.  All checked before any launch."""
    d = _desc(T=128)
    a = L.tp_mlp_bwd_args()
    for name, _ in L.tp_mlp_bwd_args._fields_:
        if name not in ("workspace_bytes", "d_normed_parts", "n_d_normed_parts", "w_down_t", "w_in_t", "fused_sgd",
                        "d_b_in", "normed_t", "d_pre_t"):
            setattr(a, name, A)
    a.workspace_bytes = L.tp_mlp_workspace_bytes(d, L.BWD_SHARD)
    f = L.tp_mlp_fused_sgd(lr=0.1, w_in_out=A, w_down_out=A)
    a.fused_sgd = ctypes.pointer(f)
    call = lambda desc=d: lib.tp_mlp_backward(ctypes.byref(desc), L.BWD_SHARD, ctypes.byref(a), None)
    assert call(_desc(T=128, dt=L.F32)) == L.EDTYPE
    assert call(_desc(T=128, flags=L.ACCUMULATE_GRADS)) == L.EINVAL
    f.lr = float("nan")
    assert call() == L.EINVAL
    f.lr = 0.1
    f.w_in_out = None
    assert call() == L.EINVAL
    f.w_in_out = MIS
    assert call() == L.EALIGN
    f.w_in_out = A
    f.w_down_t_out = MIS
    assert call() == L.EALIGN
    f.w_down_t_out = A
    f.w_in_master = A
    assert call() == L.EINVAL  # no w_in_master_out
    assert "w_in_master_out" in L.tp_mlp_last_error()
    f.w_in_master = None
    # the gradients are not written: NULL is accepted (checked up to the missing d_pre)
    a.d_w_in = a.d_w_down = None
    a.d_pre = None
    assert call() == L.EINVAL
    assert "d_pre" in L.tp_mlp_last_error()
    a.d_pre = A
    # the transposed activations: bf16, T a multiple of 8, aligned, d_pre_t only with w_down_t
    a.d_pre_t = A
    assert call() == L.EINVAL and "w_down_t" in L.tp_mlp_last_error()
    a.w_down_t = A
    a.d_pre_t = MIS
    assert call() == L.EALIGN
    a.d_pre_t = A
    a.normed_t = MIS
    assert call() == L.EALIGN
    a.normed_t = A
    assert call(_desc(T=124)) == L.ESHAPE
    a.d_pre_t = a.normed_t = a.w_down_t = None
    a.workspace_bytes = 1 << 30
    fp8 = L.make_fp8_args(1, **{n: A for n in L.FP8_META_FIELDS + L.FP8_CODE_FIELDS})
    # the FP8 backward takes the fused update too: with no master it reads the old w_in, which must be given
    a.w_in = None
    assert lib.tp_mlp_backward_fp8(ctypes.byref(d), L.BWD_SHARD, ctypes.byref(a), ctypes.byref(fp8), None) == L.EINVAL
    assert "w_in" in L.tp_mlp_last_error()
    a.w_in = A
    d_acc = _desc(T=128, flags=L.ACCUMULATE_GRADS)
    assert lib.tp_mlp_backward_fp8(ctypes.byref(d_acc), L.BWD_SHARD, ctypes.byref(a), ctypes.byref(fp8),
                                   None) == L.EINVAL


def test_backward_norm_parts_checks(lib):
    """The NORM phase's streamed partials: count in [0, 64], a non-NULL
    array when the count is positive, every part non-NULL and aligned; all
    checked before any launch."""
    d = _desc(T=128)
    a = L.tp_mlp_bwd_args()
    for name, _ in L.tp_mlp_bwd_args._fields_:
        if name not in ("workspace_bytes", "d_normed_parts", "n_d_normed_parts", "w_down_t", "w_in_t", "fused_sgd",
                        "normed_t", "d_pre_t"):
            setattr(a, name, A)
    a.workspace_bytes = L.tp_mlp_workspace_bytes(d, L.BWD_NORM)
    a.n_d_normed_parts = 65
    assert lib.tp_mlp_backward(ctypes.byref(d), L.BWD_NORM, ctypes.byref(a), None) == L.EINVAL
    a.n_d_normed_parts = -1
    assert lib.tp_mlp_backward(ctypes.byref(d), L.BWD_NORM, ctypes.byref(a), None) == L.EINVAL
    a.n_d_normed_parts = 2
    assert lib.tp_mlp_backward(ctypes.byref(d), L.BWD_NORM, ctypes.byref(a), None) == L.EINVAL  # NULL array
    arr = (ctypes.c_void_p * 2)(A, None)
    a.d_normed_parts = ctypes.cast(arr, ctypes.POINTER(ctypes.c_void_p))
    assert lib.tp_mlp_backward(ctypes.byref(d), L.BWD_NORM, ctypes.byref(a), None) == L.EINVAL
    assert b"part" in lib.tp_mlp_last_error()
    arr2 = (ctypes.c_void_p * 2)(A, MIS)
    a.d_normed_parts = ctypes.cast(arr2, ctypes.POINTER(ctypes.c_void_p))
    assert lib.tp_mlp_backward(ctypes.byref(d), L.BWD_NORM, ctypes.byref(a), None) == L.EALIGN


def test_attn_backward_norm_parts_checks(lib):
    """The attention NORM phase's streamed partials are checked as the MLP's:
    count in [0, 64], a non-NULL array when the count is positive, every part
    non-NULL and aligned; all before any launch."""
    d = L.make_attn_desc(2, 64, 256, 4, 2, 64, 1e-6)
    a = L.tp_attn_bwd_args()
    for name, _ in L.tp_attn_bwd_args._fields_:
        if name not in ("workspace_bytes", "d_normed_parts", "n_d_normed_parts"):
            setattr(a, name, A)
    a.workspace_bytes = lib.tp_attn_workspace_bytes(ctypes.byref(d), L.BWD_NORM)
    a.n_d_normed_parts = 65
    assert lib.tp_attn_backward(ctypes.byref(d), L.BWD_NORM, ctypes.byref(a), None) == L.EINVAL
    a.n_d_normed_parts = -1
    assert lib.tp_attn_backward(ctypes.byref(d), L.BWD_NORM, ctypes.byref(a), None) == L.EINVAL
    a.n_d_normed_parts = 2
    assert lib.tp_attn_backward(ctypes.byref(d), L.BWD_NORM, ctypes.byref(a), None) == L.EINVAL  # NULL array
    arr = (ctypes.c_void_p * 2)(A, None)
    a.d_normed_parts = ctypes.cast(arr, ctypes.POINTER(ctypes.c_void_p))
    assert lib.tp_attn_backward(ctypes.byref(d), L.BWD_NORM, ctypes.byref(a), None) == L.EINVAL
    assert b"part" in lib.tp_mlp_last_error()
    arr2 = (ctypes.c_void_p * 2)(A, MIS)
    a.d_normed_parts = ctypes.cast(arr2, ctypes.POINTER(ctypes.c_void_p))
    assert lib.tp_attn_backward(ctypes.byref(d), L.BWD_NORM, ctypes.byref(a), None) == L.EALIGN


def test_sgd_transposed_copy_checks(lib):
    """The SGD tensor's transposed copy: bf16 only, t_rows x t_cols == n with
    both multiples of 8, an aligned pointer; and tp_mlp_transpose_bf16's
    shape checks; all before any launch."""
    t = L.tp_mlp_sgd_tensor(A, A, A, None, None, 64 * 32, A, 64, 32)
    assert lib.tp_mlp_sgd_step_multi(ctypes.byref(t), 1, L.F32, ctypes.c_float(0.1), None) == L.EDTYPE
    t.t_rows = 60
    t.t_cols = 32
    assert lib.tp_mlp_sgd_step_multi(ctypes.byref(t), 1, L.BF16, ctypes.c_float(0.1), None) == L.ESHAPE
    t.t_rows, t.t_cols = 64, 16  # product != n
    assert lib.tp_mlp_sgd_step_multi(ctypes.byref(t), 1, L.BF16, ctypes.c_float(0.1), None) == L.ESHAPE
    t.t_cols, t.param_out_t = 32, MIS
    assert lib.tp_mlp_sgd_step_multi(ctypes.byref(t), 1, L.BF16, ctypes.c_float(0.1), None) == L.EALIGN
    assert lib.tp_mlp_transpose_bf16(A, A, 12, 16, None) == L.ESHAPE
    assert lib.tp_mlp_transpose_bf16(A, MIS, 16, 16, None) == L.EALIGN
    assert lib.tp_mlp_transpose_bf16(None, None, 0, 16, None) == L.OK
