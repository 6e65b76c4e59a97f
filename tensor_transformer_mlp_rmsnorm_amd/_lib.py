"""ctypes binding of libtpmlp (include/tp_mlp.h): argument marshalling only.

Each function takes torch tensors (device memory) or ints and calls the C
entry point of the same name on the current HIP stream.  A non-zero return
code raises TPMLPError with the library's message.  There is no fallback:
if the shared library is missing, loading raises.
"""

from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

import torch

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libtpmlp.so")

OK, EINVAL, ESHAPE, EDTYPE, EALIGN, EWORKSPACE, EHIP = 0, -1, -2, -3, -4, -5, -6
ACT_SWIGLU, ACT_GELU = 0, 1
F32, BF16 = 0, 1
FUSE_EPILOGUE, NORMED_READY, ACCUMULATE_GRADS = 1, 2, 4
BWD_SHARD, BWD_NORM = 0, 1
FP8_E4M3, FP8_E5M2 = 0, 1
FP8_SHARED_READY = 8
FP8_MAX_HISTORY = 1024


def fp8_meta_floats(history_len: int) -> int:
    return 4 + history_len

# every symbol include/tp_mlp.h declares
EXPORTED = ("tp_mlp_forward", "tp_partial_sum", "tp_mlp_backward", "tp_mlp_workspace_bytes",
            "tp_mlp_sgd_step", "tp_mlp_last_error", "tp_mlp_version", "tp_mlp_profile_enable",
            "tp_mlp_profile_count", "tp_mlp_profile_entry", "tp_mlp_sgd_step_multi", "tp_mlp_adamw_step_multi",
            "tp_mlp_clip_grad_norm", "tp_mlp_clip_grad_norm_workspace_bytes", "tp_rmsnorm_forward",
            "tp_mlp_fp8_meta_init", "tp_mlp_fp8_cast", "tp_mlp_fp8_update_scales", "tp_mlp_forward_fp8",
            "tp_mlp_backward_fp8", "tp_mlp_fp8_gemm", "tp_mlp_fp8_gemm_workspace_bytes", "tp_attn_forward",
            "tp_attn_backward", "tp_attn_workspace_bytes", "tp_attention_forward", "tp_attention_backward",
            "tp_attention_backward_workspace_bytes", "tp_mlp_profile_only", "tp_attn_forward_workspace_bytes",
            "tp_mlp_backward_noalloc", "tp_mlp_transpose_bf16", "tp_mlp_forward_ws", "tp_mlp_forward_workspace_bytes")


class TPMLPError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"libtpmlp error {code}: {msg}")
        self.code = code


class tp_mlp_desc(ctypes.Structure):
    _fields_ = [("tokens", ctypes.c_int64), ("hidden", ctypes.c_int64), ("ffn_local", ctypes.c_int64),
                ("act", ctypes.c_int32), ("dtype", ctypes.c_int32), ("eps", ctypes.c_float),
                ("flags", ctypes.c_int32)]


_vp = ctypes.c_void_p


class tp_mlp_sgd_tensor(ctypes.Structure):
    _fields_ = [("param_in", ctypes.c_void_p), ("param_out", ctypes.c_void_p), ("grad", ctypes.c_void_p),
                ("master_in", ctypes.c_void_p), ("master_out", ctypes.c_void_p), ("n", ctypes.c_int64),
                ("param_out_t", ctypes.c_void_p), ("t_rows", ctypes.c_int64), ("t_cols", ctypes.c_int64)]


class tp_mlp_adamw_hparams(ctypes.Structure):
    _fields_ = [("lr", ctypes.c_float), ("beta1", ctypes.c_float), ("beta2", ctypes.c_float), ("eps", ctypes.c_float),
                ("weight_decay", ctypes.c_float), ("step", ctypes.c_int32)]


class tp_mlp_adamw_tensor(ctypes.Structure):
    _fields_ = [("param_in", ctypes.c_void_p), ("param_out", ctypes.c_void_p), ("grad", ctypes.c_void_p),
                ("master_in", ctypes.c_void_p), ("master_out", ctypes.c_void_p), ("m", ctypes.c_void_p),
                ("v", ctypes.c_void_p), ("n", ctypes.c_int64)]


class tp_mlp_fused_sgd(ctypes.Structure):
    _fields_ = [("lr", ctypes.c_float)] + [(n, _vp) for n in (
        "w_in_out", "w_in_t_out", "w_in_master", "w_in_master_out",
        "w_down_out", "w_down_t_out", "w_down_master", "w_down_master_out")]


class tp_mlp_bwd_args(ctypes.Structure):
    _fields_ = [(n, _vp) for n in ("x", "normed", "rstd", "pre_act", "act", "norm_w", "w_in", "w_down", "d_out",
                                   "d_pre", "d_w_in", "d_b_in", "d_w_down", "d_normed_part", "d_normed", "d_x",
                                   "d_norm_w", "d_b_down", "workspace")] + [("workspace_bytes", ctypes.c_size_t)] + \
        [("d_normed_parts", ctypes.POINTER(_vp)), ("n_d_normed_parts", ctypes.c_int32), ("w_down_t", _vp),
         ("w_in_t", _vp), ("fused_sgd", ctypes.POINTER(tp_mlp_fused_sgd)), ("normed_t", _vp), ("d_pre_t", _vp)]


FP8_META_FIELDS = ("meta_normed", "meta_w_in", "meta_act", "meta_w_down", "meta_d_out", "meta_d_pre")
FP8_CODE_FIELDS = ("normed_q", "normed_t", "w_in_q", "w_in_t", "act_q", "act_t", "w_down_q", "w_down_t",
                   "d_out_q", "d_out_t", "d_pre_q", "d_pre_t")


class tp_mlp_fp8_args(ctypes.Structure):
    _fields_ = [("history_len", ctypes.c_int32)] + [(n, _vp) for n in FP8_META_FIELDS + FP8_CODE_FIELDS]


class tp_attn_desc(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int64), ("seq", ctypes.c_int64), ("hidden", ctypes.c_int64),
                ("n_q", ctypes.c_int32), ("n_kv", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("dtype", ctypes.c_int32), ("eps", ctypes.c_float), ("flags", ctypes.c_int32)]


class tp_attn_bwd_args(ctypes.Structure):
    _fields_ = [(n, _vp) for n in ("x", "normed", "rstd", "qkv", "attn_out", "lse", "norm_w", "w_qkv", "w_o", "d_out",
                                   "d_attn_out", "d_qkv", "d_w_qkv", "d_w_o", "d_normed_part", "d_normed", "d_x",
                                   "d_norm_w", "d_b_o", "workspace")] + [("workspace_bytes", ctypes.c_size_t)] + \
        [("d_normed_parts", ctypes.POINTER(_vp)), ("n_d_normed_parts", ctypes.c_int32)]


_LIB: Optional[ctypes.CDLL] = None


def lib() -> ctypes.CDLL:
    """Load libtpmlp.so (once).  Raises if it has not been built."""
    global _LIB
    if _LIB is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m tensor_transformer_mlp_rmsnorm_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        L.tp_mlp_forward.argtypes = [ctypes.POINTER(tp_mlp_desc)] + [_vp] * 12
        L.tp_mlp_forward_ws.argtypes = [ctypes.POINTER(tp_mlp_desc)] + [_vp] * 12 + [ctypes.c_size_t, _vp]
        L.tp_mlp_forward_workspace_bytes.argtypes = [ctypes.POINTER(tp_mlp_desc)]
        L.tp_mlp_forward_workspace_bytes.restype = ctypes.c_size_t
        L.tp_mlp_forward.restype = ctypes.c_int
        L.tp_partial_sum.argtypes = [ctypes.POINTER(_vp), ctypes.c_int32, ctypes.c_int64, ctypes.c_int64, _vp, _vp,
                                     ctypes.c_int32, _vp, ctypes.c_int32, _vp]
        L.tp_partial_sum.restype = ctypes.c_int
        L.tp_mlp_backward.argtypes = [ctypes.POINTER(tp_mlp_desc), ctypes.c_int32, ctypes.POINTER(tp_mlp_bwd_args),
                                      _vp]
        L.tp_mlp_backward.restype = ctypes.c_int
        L.tp_mlp_backward_noalloc.argtypes = [ctypes.POINTER(tp_mlp_desc), ctypes.c_int32,
                                              ctypes.POINTER(tp_mlp_bwd_args), _vp]
        L.tp_mlp_backward_noalloc.restype = ctypes.c_int
        L.tp_mlp_workspace_bytes.argtypes = [ctypes.POINTER(tp_mlp_desc), ctypes.c_int32]
        L.tp_mlp_workspace_bytes.restype = ctypes.c_size_t
        L.tp_mlp_transpose_bf16.argtypes = [_vp, _vp, ctypes.c_int64, ctypes.c_int64, _vp]
        L.tp_mlp_transpose_bf16.restype = ctypes.c_int
        L.tp_mlp_sgd_step.argtypes = [_vp, _vp, _vp, _vp, _vp, ctypes.c_int64, ctypes.c_int32, ctypes.c_float, _vp]
        L.tp_mlp_sgd_step.restype = ctypes.c_int
        L.tp_mlp_sgd_step_multi.argtypes = [ctypes.POINTER(tp_mlp_sgd_tensor), ctypes.c_int32, ctypes.c_int32,
                                            ctypes.c_float, _vp]
        L.tp_mlp_sgd_step_multi.restype = ctypes.c_int
        L.tp_mlp_adamw_step_multi.argtypes = [ctypes.POINTER(tp_mlp_adamw_tensor), ctypes.c_int32, ctypes.c_int32,
                                              ctypes.POINTER(tp_mlp_adamw_hparams), _vp, _vp]
        L.tp_mlp_adamw_step_multi.restype = ctypes.c_int
        L.tp_mlp_clip_grad_norm.argtypes = [ctypes.POINTER(_vp), ctypes.POINTER(ctypes.c_int64), ctypes.c_int32,
                                            ctypes.c_float, _vp, _vp, _vp, ctypes.c_size_t, _vp]
        L.tp_mlp_clip_grad_norm.restype = ctypes.c_int
        L.tp_mlp_clip_grad_norm_workspace_bytes.argtypes = [ctypes.POINTER(ctypes.c_int64), ctypes.c_int32]
        L.tp_mlp_clip_grad_norm_workspace_bytes.restype = ctypes.c_size_t
        L.tp_rmsnorm_forward.argtypes = [ctypes.c_int64, ctypes.c_int64, ctypes.c_int32, ctypes.c_float, _vp, _vp,
                                         _vp, _vp, _vp]
        L.tp_rmsnorm_forward.restype = ctypes.c_int
        L.tp_mlp_fp8_meta_init.argtypes = [_vp, ctypes.c_int32, ctypes.c_int32, _vp]
        L.tp_mlp_fp8_meta_init.restype = ctypes.c_int
        L.tp_mlp_fp8_cast.argtypes = [ctypes.c_int64, ctypes.c_int64, _vp, ctypes.c_int32, _vp, _vp, _vp,
                                      ctypes.c_int64, _vp]
        L.tp_mlp_fp8_cast.restype = ctypes.c_int
        L.tp_mlp_fp8_update_scales.argtypes = [ctypes.POINTER(_vp), ctypes.c_int32, ctypes.c_int32, _vp]
        L.tp_mlp_fp8_update_scales.restype = ctypes.c_int
        L.tp_mlp_forward_fp8.argtypes = [ctypes.POINTER(tp_mlp_desc)] + [_vp] * 11 + \
            [ctypes.POINTER(tp_mlp_fp8_args), _vp]
        L.tp_mlp_forward_fp8.restype = ctypes.c_int
        L.tp_mlp_backward_fp8.argtypes = [ctypes.POINTER(tp_mlp_desc), ctypes.c_int32,
                                          ctypes.POINTER(tp_mlp_bwd_args), ctypes.POINTER(tp_mlp_fp8_args), _vp]
        L.tp_mlp_backward_fp8.restype = ctypes.c_int
        L.tp_mlp_fp8_gemm.argtypes = [ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, _vp, ctypes.c_int64,
                                      ctypes.c_int32, _vp, _vp, ctypes.c_int64, ctypes.c_int32, _vp, _vp,
                                      ctypes.c_int64, ctypes.c_int32, _vp, ctypes.c_size_t, _vp]
        L.tp_mlp_fp8_gemm.restype = ctypes.c_int
        L.tp_mlp_fp8_gemm_workspace_bytes.argtypes = [ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64]
        L.tp_mlp_fp8_gemm_workspace_bytes.restype = ctypes.c_size_t
        L.tp_attn_forward.argtypes = [ctypes.POINTER(tp_attn_desc)] + [_vp] * 12 + [ctypes.c_size_t, _vp]
        L.tp_attn_forward_workspace_bytes.argtypes = [ctypes.POINTER(tp_attn_desc)]
        L.tp_attn_forward_workspace_bytes.restype = ctypes.c_size_t
        L.tp_attn_forward.restype = ctypes.c_int
        L.tp_attn_backward.argtypes = [ctypes.POINTER(tp_attn_desc), ctypes.c_int32, ctypes.POINTER(tp_attn_bwd_args),
                                       _vp]
        L.tp_attn_backward.restype = ctypes.c_int
        L.tp_attn_workspace_bytes.argtypes = [ctypes.POINTER(tp_attn_desc), ctypes.c_int32]
        L.tp_attn_workspace_bytes.restype = ctypes.c_size_t
        L.tp_attention_forward.argtypes = [ctypes.c_int64, ctypes.c_int64, ctypes.c_int32, ctypes.c_int32,
                                           ctypes.c_int32, _vp, ctypes.c_int64, _vp, _vp, _vp]
        L.tp_attention_forward.restype = ctypes.c_int
        L.tp_attention_backward.argtypes = [ctypes.c_int64, ctypes.c_int64, ctypes.c_int32, ctypes.c_int32,
                                            ctypes.c_int32, _vp, ctypes.c_int64, _vp, _vp, _vp, _vp,
                                            ctypes.c_size_t, _vp, _vp]
        L.tp_attention_backward.restype = ctypes.c_int
        L.tp_attention_backward_workspace_bytes.argtypes = [ctypes.c_int64, ctypes.c_int64, ctypes.c_int32,
                                                            ctypes.c_int32, ctypes.c_int32]
        L.tp_attention_backward_workspace_bytes.restype = ctypes.c_size_t
        L.tp_mlp_last_error.argtypes = []
        L.tp_mlp_last_error.restype = ctypes.c_char_p
        L.tp_mlp_version.argtypes = []
        L.tp_mlp_version.restype = ctypes.c_char_p
        L.tp_mlp_profile_enable.argtypes = [ctypes.c_int32]
        L.tp_mlp_profile_enable.restype = ctypes.c_int
        L.tp_mlp_profile_only.argtypes = [ctypes.c_char_p]
        L.tp_mlp_profile_only.restype = ctypes.c_int
        L.tp_mlp_profile_count.argtypes = []
        L.tp_mlp_profile_count.restype = ctypes.c_int32
        L.tp_mlp_profile_entry.argtypes = [ctypes.c_int32, ctypes.POINTER(ctypes.c_char_p),
                                           ctypes.POINTER(ctypes.c_int64), ctypes.POINTER(ctypes.c_double)]
        L.tp_mlp_profile_entry.restype = ctypes.c_int
        _LIB = L
    return _LIB


def _ptr(t) -> Optional[int]:
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    return stream if isinstance(stream, int) else stream.cuda_stream


def _check(rc: int) -> None:
    if rc != OK:
        raise TPMLPError(rc, lib().tp_mlp_last_error().decode())


def make_desc(tokens: int, hidden: int, ffn_local: int, act: int, dtype: int, eps: float,
              flags: int = 0) -> tp_mlp_desc:
    return tp_mlp_desc(tokens, hidden, ffn_local, act, dtype, eps, flags)


def tp_mlp_forward(desc: tp_mlp_desc, x, norm_w, w_in, b_in, w_down, normed, rstd, pre_act, act, out,
                   b_down=None, stream=None) -> None:
    _check(lib().tp_mlp_forward(ctypes.byref(desc), _ptr(x), _ptr(norm_w), _ptr(w_in), _ptr(b_in), _ptr(w_down),
                                _ptr(normed), _ptr(rstd), _ptr(pre_act), _ptr(act), _ptr(out), _ptr(b_down),
                                _stream(stream)))


def tp_mlp_forward_ws(desc: tp_mlp_desc, x, norm_w, w_in, b_in, w_down, normed, rstd, pre_act, act, out,
                      b_down=None, workspace=None, workspace_bytes=None, stream=None) -> None:
    if workspace_bytes is None:
        workspace_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().tp_mlp_forward_ws(ctypes.byref(desc), _ptr(x), _ptr(norm_w), _ptr(w_in), _ptr(b_in), _ptr(w_down),
                                   _ptr(normed), _ptr(rstd), _ptr(pre_act), _ptr(act), _ptr(out), _ptr(b_down),
                                   _ptr(workspace), workspace_bytes, _stream(stream)))


def tp_mlp_forward_workspace_bytes(desc: tp_mlp_desc) -> int:
    return int(lib().tp_mlp_forward_workspace_bytes(ctypes.byref(desc)))


def tp_rmsnorm_forward(rows: int, hidden: int, dtype: int, eps: float, x, w, normed, rstd, stream=None) -> None:
    _check(lib().tp_rmsnorm_forward(rows, hidden, dtype, eps, _ptr(x), _ptr(w), _ptr(normed), _ptr(rstd),
                                    _stream(stream)))


def tp_partial_sum(parts: Sequence, rows: int, cols: int, residual, bias, in_dtype: int, out, out_dtype: int,
                   stream=None) -> None:
    arr = (_vp * max(1, len(parts)))(*[_ptr(p) for p in parts])
    _check(lib().tp_partial_sum(arr, len(parts), rows, cols, _ptr(residual), _ptr(bias), in_dtype, _ptr(out),
                                out_dtype, _stream(stream)))


def tp_mlp_workspace_bytes(desc: tp_mlp_desc, phase: int) -> int:
    return int(lib().tp_mlp_workspace_bytes(ctypes.byref(desc), phase))


def tp_mlp_backward(desc: tp_mlp_desc, phase: int, stream=None, **tensors) -> None:
    """``tensors`` are the fields of tp_mlp_bwd_args (torch tensors or None);
    ``workspace`` may be given, ``workspace_bytes`` defaults to its size."""
    a = _bwd_args(tensors)
    _check(lib().tp_mlp_backward(ctypes.byref(desc), phase, ctypes.byref(a), _stream(stream)))


def tp_mlp_backward_noalloc(desc: tp_mlp_desc, phase: int, stream=None, **tensors) -> None:
    """tp_mlp_backward with the library's own scratch: ``workspace`` is not
    taken (the C call ignores it)."""
    if "workspace" in tensors or "workspace_bytes" in tensors:
        raise TypeError("tp_mlp_backward_noalloc takes no workspace")
    a = _bwd_args(tensors)
    _check(lib().tp_mlp_backward_noalloc(ctypes.byref(desc), phase, ctypes.byref(a), _stream(stream)))


NOALLOC_SCRATCH_BYTES = 128 << 20


def _bwd_args(tensors: dict) -> tp_mlp_bwd_args:
    """``d_normed_parts`` may be a sequence of tensors (the NORM phase then
    sums them); the pointer array stays alive with the returned struct."""
    a = tp_mlp_bwd_args()
    fused = tensors.pop("fused_sgd", None)
    if fused:
        f = tp_mlp_fused_sgd()
        for name, _ in tp_mlp_fused_sgd._fields_:
            if name == "lr":
                f.lr = float(fused["lr"])
            else:
                setattr(f, name, _ptr(fused.get(name)))
        unknown = set(fused) - {n for n, _ in tp_mlp_fused_sgd._fields_}
        if unknown:
            raise TypeError(f"unknown fused_sgd fields: {sorted(unknown)}")
        a._fused_keepalive = f
        a.fused_sgd = ctypes.pointer(f)
    parts = tensors.pop("d_normed_parts", None)
    if parts:
        arr = (_vp * len(parts))(*[_ptr(p) for p in parts])
        a._parts_keepalive = arr
        a.d_normed_parts = ctypes.cast(arr, ctypes.POINTER(_vp))
        a.n_d_normed_parts = len(parts)
    for name, _ in tp_mlp_bwd_args._fields_:
        if name in ("workspace_bytes", "d_normed_parts", "n_d_normed_parts", "fused_sgd"):
            continue
        v = tensors.pop(name, None)
        setattr(a, name, _ptr(v))
        if name == "workspace" and v is not None and not isinstance(v, int):
            a.workspace_bytes = v.numel() * v.element_size()
    if "workspace_bytes" in tensors:
        a.workspace_bytes = tensors.pop("workspace_bytes")
    if tensors:
        raise TypeError(f"unknown backward arguments: {sorted(tensors)}")
    return a


def make_fp8_args(history_len: int, **buffers) -> tp_mlp_fp8_args:
    """``buffers``: the meta_* and code fields of tp_mlp_fp8_args (tensors or None)."""
    f = tp_mlp_fp8_args()
    f.history_len = history_len
    for name in FP8_META_FIELDS + FP8_CODE_FIELDS:
        setattr(f, name, _ptr(buffers.pop(name, None)))
    if buffers:
        raise TypeError(f"unknown fp8 arguments: {sorted(buffers)}")
    return f


def tp_mlp_fp8_meta_init(meta, fmt: int, history_len: int, stream=None) -> None:
    _check(lib().tp_mlp_fp8_meta_init(_ptr(meta), fmt, history_len, _stream(stream)))


def tp_mlp_fp8_cast(rows: int, cols: int, x, fmt: int, meta, out, out_t=None, ldt: int = 0, stream=None) -> None:
    _check(lib().tp_mlp_fp8_cast(rows, cols, _ptr(x), fmt, _ptr(meta), _ptr(out), _ptr(out_t), ldt,
                                 _stream(stream)))


def tp_mlp_fp8_update_scales(metas: Sequence, history_len: int, stream=None) -> None:
    arr = (_vp * max(1, len(metas)))(*[_ptr(m) for m in metas])
    _check(lib().tp_mlp_fp8_update_scales(arr, len(metas), history_len, _stream(stream)))


def tp_mlp_forward_fp8(desc: tp_mlp_desc, x, norm_w, w_in, b_in, w_down, normed, rstd, pre_act, act, out,
                       b_down, f8: tp_mlp_fp8_args, stream=None) -> None:
    _check(lib().tp_mlp_forward_fp8(ctypes.byref(desc), _ptr(x), _ptr(norm_w), _ptr(w_in), _ptr(b_in),
                                    _ptr(w_down), _ptr(normed), _ptr(rstd), _ptr(pre_act), _ptr(act), _ptr(out),
                                    _ptr(b_down), ctypes.byref(f8), _stream(stream)))


def tp_mlp_backward_fp8(desc: tp_mlp_desc, phase: int, f8: tp_mlp_fp8_args, stream=None, **tensors) -> None:
    """``tensors`` as for tp_mlp_backward."""
    a = _bwd_args(tensors)
    _check(lib().tp_mlp_backward_fp8(ctypes.byref(desc), phase, ctypes.byref(a), ctypes.byref(f8),
                                     _stream(stream)))


def tp_mlp_fp8_gemm_workspace_bytes(M: int, N: int, K: int, ldc: int) -> int:
    return int(lib().tp_mlp_fp8_gemm_workspace_bytes(M, N, K, ldc))


def tp_mlp_fp8_gemm(M: int, N: int, K: int, A, lda: int, fmt_a: int, scale_inv_a, B, ldb: int, fmt_b: int,
                    scale_inv_b, C, ldc: int, accumulate: bool = False, workspace=None, stream=None) -> None:
    """``scale_inv_a`` / ``scale_inv_b``: one-element fp32 device tensors (or a meta viewed at [1:])."""
    nbytes = 0 if workspace is None or isinstance(workspace, int) else workspace.numel() * workspace.element_size()
    _check(lib().tp_mlp_fp8_gemm(M, N, K, _ptr(A), lda, fmt_a, _ptr(scale_inv_a), _ptr(B), ldb, fmt_b,
                                 _ptr(scale_inv_b), _ptr(C), ldc, 1 if accumulate else 0, _ptr(workspace), nbytes,
                                 _stream(stream)))


def make_attn_desc(batch: int, seq: int, hidden: int, n_q: int, n_kv: int, head_dim: int, eps: float,
                   flags: int = 0, dtype: int = BF16) -> tp_attn_desc:
    return tp_attn_desc(batch, seq, hidden, n_q, n_kv, head_dim, dtype, eps, flags)


def tp_attn_forward(desc: tp_attn_desc, x, norm_w, w_qkv, w_o, normed, rstd, qkv, attn_out, lse, out, b_o=None,
                    workspace=None, workspace_bytes: int = 0, stream=None) -> None:
    _check(lib().tp_attn_forward(ctypes.byref(desc), _ptr(x), _ptr(norm_w), _ptr(w_qkv), _ptr(w_o), _ptr(normed),
                                 _ptr(rstd), _ptr(qkv), _ptr(attn_out), _ptr(lse), _ptr(out), _ptr(b_o),
                                 _ptr(workspace), workspace_bytes, _stream(stream)))


def tp_attn_forward_workspace_bytes(desc: tp_attn_desc) -> int:
    return int(lib().tp_attn_forward_workspace_bytes(ctypes.byref(desc)))


def tp_attn_workspace_bytes(desc: tp_attn_desc, phase: int) -> int:
    return int(lib().tp_attn_workspace_bytes(ctypes.byref(desc), phase))


def tp_attn_backward(desc: tp_attn_desc, phase: int, stream=None, **tensors) -> None:
    """``tensors``: the fields of tp_attn_bwd_args (torch tensors or None);
    ``d_normed_parts`` may be a sequence of tensors (the NORM phase then sums them)."""
    a = tp_attn_bwd_args()
    parts = tensors.pop("d_normed_parts", None)
    if parts:
        arr = (_vp * len(parts))(*[_ptr(p) for p in parts])
        a._parts_keepalive = arr
        a.d_normed_parts = ctypes.cast(arr, ctypes.POINTER(_vp))
        a.n_d_normed_parts = len(parts)
    for name, _ in tp_attn_bwd_args._fields_:
        if name in ("workspace_bytes", "d_normed_parts", "n_d_normed_parts", "fused_sgd"):
            continue
        v = tensors.pop(name, None)
        setattr(a, name, _ptr(v))
        if name == "workspace" and v is not None and not isinstance(v, int):
            a.workspace_bytes = v.numel() * v.element_size()
    if tensors:
        raise TypeError(f"unknown attention backward arguments: {sorted(tensors)}")
    _check(lib().tp_attn_backward(ctypes.byref(desc), phase, ctypes.byref(a), _stream(stream)))


def tp_attention_forward(batch: int, seq: int, n_q: int, n_kv: int, head_dim: int, qkv, ld: int, o, lse,
                         stream=None) -> None:
    _check(lib().tp_attention_forward(batch, seq, n_q, n_kv, head_dim, _ptr(qkv), ld, _ptr(o), _ptr(lse),
                                      _stream(stream)))


def tp_attention_backward(batch: int, seq: int, n_q: int, n_kv: int, head_dim: int, qkv, ld: int, o, d_o, lse,
                          workspace, workspace_bytes: int, d_qkv, stream=None) -> None:
    _check(lib().tp_attention_backward(batch, seq, n_q, n_kv, head_dim, _ptr(qkv), ld, _ptr(o), _ptr(d_o), _ptr(lse),
                                       _ptr(workspace), workspace_bytes, _ptr(d_qkv), _stream(stream)))


def tp_attention_backward_workspace_bytes(batch: int, seq: int, n_q: int, n_kv: int, head_dim: int) -> int:
    return int(lib().tp_attention_backward_workspace_bytes(batch, seq, n_q, n_kv, head_dim))


def tp_mlp_sgd_step(param_in, param_out, grad, master_in, master_out, n: int, param_dtype: int, lr: float,
                    stream=None) -> None:
    _check(lib().tp_mlp_sgd_step(_ptr(param_in), _ptr(param_out), _ptr(grad), _ptr(master_in), _ptr(master_out),
                                 n, param_dtype, lr, _stream(stream)))


def tp_mlp_sgd_step_multi(tensors: Sequence, param_dtype: int, lr: float, stream=None) -> None:
    """``tensors``: sequence of (param_in, param_out, grad, master_in, master_out, n), or of
    (..., n, param_out_t, t_rows, t_cols) for a tensor that also gets its transposed copy."""
    def one(t):
        a, b, c, d, e, n = t[:6]
        pt, rows, cols = t[6:] if len(t) > 6 else (None, 0, 0)
        return tp_mlp_sgd_tensor(_ptr(a), _ptr(b), _ptr(c), _ptr(d), _ptr(e), n, _ptr(pt), rows, cols)
    arr = (tp_mlp_sgd_tensor * max(1, len(tensors)))(*[one(t) for t in tensors])
    _check(lib().tp_mlp_sgd_step_multi(arr, len(tensors), param_dtype, lr, _stream(stream)))


def tp_mlp_transpose_bf16(x, out, rows: int, cols: int, stream=None) -> None:
    _check(lib().tp_mlp_transpose_bf16(_ptr(x), _ptr(out), rows, cols, _stream(stream)))


def make_adamw_hparams(lr: float, step: int, weight_decay: float = 0.0, beta1: float = 0.9, beta2: float = 0.999,
                       eps: float = 1e-8) -> tp_mlp_adamw_hparams:
    return tp_mlp_adamw_hparams(lr, beta1, beta2, eps, weight_decay, step)


def tp_mlp_adamw_step_multi(tensors: Sequence, param_dtype: int, hp: tp_mlp_adamw_hparams, grad_scale=None,
                            stream=None) -> None:
    """``tensors``: sequence of (param_in, param_out, grad, master_in, master_out, m, v, n);
    ``grad_scale``: a one-element fp32 device tensor (e.g. the clip coefficient) or None."""
    arr = (tp_mlp_adamw_tensor * max(1, len(tensors)))(
        *[tp_mlp_adamw_tensor(*[_ptr(t) for t in row[:7]], row[7]) for row in tensors])
    _check(lib().tp_mlp_adamw_step_multi(arr, len(tensors), param_dtype, ctypes.byref(hp), _ptr(grad_scale),
                                         _stream(stream)))


def tp_mlp_clip_grad_norm_workspace_bytes(counts: Sequence[int]) -> int:
    arr = (ctypes.c_int64 * max(1, len(counts)))(*counts)
    return int(lib().tp_mlp_clip_grad_norm_workspace_bytes(arr, len(counts)))


def tp_mlp_clip_grad_norm(grads: Sequence, counts: Sequence[int], max_norm: float, norm_out, coef_out, workspace,
                          workspace_bytes: Optional[int] = None, stream=None) -> None:
    garr = (_vp * max(1, len(grads)))(*[_ptr(g) for g in grads])
    carr = (ctypes.c_int64 * max(1, len(counts)))(*counts)
    if workspace_bytes is None:
        workspace_bytes = 0 if workspace is None or isinstance(workspace, int) else \
            workspace.numel() * workspace.element_size()
    _check(lib().tp_mlp_clip_grad_norm(garr, carr, len(grads), max_norm, _ptr(norm_out), _ptr(coef_out),
                                       _ptr(workspace), workspace_bytes, _stream(stream)))


def tp_mlp_last_error() -> str:
    return lib().tp_mlp_last_error().decode()


def tp_mlp_version() -> str:
    return lib().tp_mlp_version().decode()


def tp_mlp_profile_enable(on: bool) -> None:
    _check(lib().tp_mlp_profile_enable(1 if on else 0))


def tp_mlp_profile_only(name) -> None:
    """Record only the kernels named ``name`` (None: every kernel)."""
    _check(lib().tp_mlp_profile_only(name.encode() if name is not None else None))


def tp_mlp_profile_entries() -> dict:
    """{kernel name: (launches, total_ms)} of the recorded launches."""
    n = lib().tp_mlp_profile_count()
    if n < 0:
        _check(n)
    out = {}
    for i in range(n):
        name, cnt, ms = ctypes.c_char_p(), ctypes.c_int64(), ctypes.c_double()
        _check(lib().tp_mlp_profile_entry(i, ctypes.byref(name), ctypes.byref(cnt), ctypes.byref(ms)))
        out[name.value.decode()] = (int(cnt.value), float(ms.value))
    return out
