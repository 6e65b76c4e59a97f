// C ABI of libtpmlp (declared in include/tp_mlp.h): argument checking and the
// sequence of kernel launches for each call.
#include <stdarg.h>
#include <cmath>
#include <mutex>
#include <stdio.h>

#include "../../include/tp_mlp.h"
#include "kernels.h"

using namespace tpmlp;

namespace {

thread_local char g_err[512] = "";

int fail(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return code;
}

int hip_fail(hipError_t e, const char* where) {
  return fail(TP_MLP_EHIP, "%s: %s", where, hipGetErrorString(e));
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

#define REQUIRE_PTR(p)                                                              \
  do {                                                                              \
    if (!(p)) return fail(TP_MLP_EINVAL, "%s: argument '%s' is NULL", fn, #p);      \
    if (!aligned16(p)) return fail(TP_MLP_EALIGN, "%s: '%s' is not 16-byte aligned", fn, #p); \
  } while (0)

// rstd is read and written one float at a time: 4-byte alignment suffices
// (so a row slice of it, a microbatch, is a valid argument).
#define REQUIRE_PTR4(p)                                                             \
  do {                                                                              \
    if (!(p)) return fail(TP_MLP_EINVAL, "%s: argument '%s' is NULL", fn, #p);      \
    if (reinterpret_cast<uintptr_t>(p) & 3u) return fail(TP_MLP_EALIGN, "%s: '%s' is not 4-byte aligned", fn, #p); \
  } while (0)

#define CHECK_HIP(expr, where)                  \
  do {                                          \
    const hipError_t e_ = (expr);               \
    if (e_ != hipSuccess) return hip_fail(e_, where); \
  } while (0)

int check_desc(const tp_mlp_desc* d, const char* fn, int32_t extra_flags = 0) {
  if (!d) return fail(TP_MLP_EINVAL, "%s: descriptor is NULL", fn);
  if (d->tokens < 0) return fail(TP_MLP_EINVAL, "%s: tokens < 0", fn);
  if (d->hidden <= 0 || d->hidden % 8) return fail(TP_MLP_ESHAPE, "%s: hidden must be a positive multiple of 8", fn);
  if (d->hidden > 16384) return fail(TP_MLP_ESHAPE, "%s: hidden > 16384 is not supported", fn);
  if (d->ffn_local <= 0 || d->ffn_local % 8)
    return fail(TP_MLP_ESHAPE, "%s: ffn_local must be a positive multiple of 8", fn);
  if (d->act != TP_MLP_ACT_SWIGLU && d->act != TP_MLP_ACT_GELU) return fail(TP_MLP_EINVAL, "%s: unknown act", fn);
  if (d->dtype != TP_MLP_F32 && d->dtype != TP_MLP_BF16) return fail(TP_MLP_EDTYPE, "%s: unknown dtype", fn);
  if (d->flags & ~(TP_MLP_FUSE_EPILOGUE | TP_MLP_NORMED_READY | TP_MLP_ACCUMULATE_GRADS | extra_flags))
    return fail(TP_MLP_EINVAL, "%s: unknown flags", fn);
  if (!(d->eps >= 0.0f)) return fail(TP_MLP_EINVAL, "%s: eps must be >= 0", fn);
  // Element counts stay below 2^31 so per-tensor int arithmetic in the
  // launchers is safe; byte offsets are 64-bit throughout.
  // The bf16 GEMM addresses each operand through a buffer descriptor whose
  // range check needs the operand below 2 GiB.
  const int64_t lim = d->dtype == TP_MLP_BF16 ? (int64_t)1 << 30 : (int64_t)1 << 31;
  const int64_t T = d->tokens, H = d->hidden, F = d->ffn_local;
  if (T * H >= lim || T * 2 * F >= lim || 2 * F * H >= lim)
    return fail(TP_MLP_ESHAPE, "%s: a tensor would hold %lld or more elements", fn, (long long)lim);
  return TP_MLP_OK;
}

DType dt_of(int32_t d) { return d == TP_MLP_BF16 ? kBF16 : kF32; }

}  // namespace

extern "C" {

const char* tp_mlp_last_error(void) { return g_err; }

const char* tp_mlp_version(void) { return "libtpmlp 0.1 gfx950"; }

}  // extern "C"

namespace {

// k slices of the down projection (bf16, through the forward's workspace)
int forward_ksplit(const tp_mlp_desc* d) {
  if (d->dtype != TP_MLP_BF16 || d->tokens <= 0) return 1;
  return gemm_ksplit(d->tokens, d->hidden, d->ffn_local);
}

size_t forward_ws_bytes(const tp_mlp_desc* d) {
  const int ks = forward_ksplit(d);
  if (ks <= 1) return 0;
  const size_t th = (size_t)d->tokens * (size_t)d->hidden * sizeof(float);
  // fused: z then the ks - 1 further slices; partial: the further slices (slice 0 writes out)
  return (d->flags & TP_MLP_FUSE_EPILOGUE) ? (size_t)ks * th : (size_t)(ks - 1) * th;
}

// with_ws: tp_mlp_forward_ws (the down projection may split k through the workspace); otherwise
// tp_mlp_forward, which never splits
int forward_checked(const tp_mlp_desc* d, const void* x, const void* norm_w, const void* w_in, const void* b_in,
                    const void* w_down, void* normed, float* rstd, void* pre_act, void* act, void* out,
                    const void* b_down, bool with_ws, void* workspace, size_t workspace_bytes, void* stream,
                    const char* fn) {
  g_err[0] = 0;
  int rc = check_desc(d, fn);
  if (rc) return rc;
  const int64_t T = d->tokens, H = d->hidden, F = d->ffn_local;
  const bool swiglu = d->act == TP_MLP_ACT_SWIGLU;
  const bool fuse = d->flags & TP_MLP_FUSE_EPILOGUE;
  REQUIRE_PTR(norm_w);
  REQUIRE_PTR(w_in);
  REQUIRE_PTR(w_down);
  if (swiglu && b_in) return fail(TP_MLP_EINVAL, "%s: b_in must be NULL for SwiGLU", fn);
  if (!swiglu) REQUIRE_PTR(b_in);
  if (fuse) REQUIRE_PTR(b_down);
  if (T == 0) return TP_MLP_OK;
  REQUIRE_PTR(x);
  REQUIRE_PTR(normed);
  REQUIRE_PTR4(rstd);
  REQUIRE_PTR(pre_act);
  REQUIRE_PTR(act);
  REQUIRE_PTR(out);
  const DType dt = dt_of(d->dtype);
  hipStream_t s = static_cast<hipStream_t>(stream);
  // the down projection's k split (tp_mlp_forward_ws only)
  const int ks = with_ws ? forward_ksplit(d) : 1;
  if (ks > 1) {
    if (!workspace || workspace_bytes < forward_ws_bytes(d))
      return fail(TP_MLP_EWORKSPACE, "%s: workspace of %zu bytes, %zu needed", fn, workspace ? workspace_bytes : 0,
                  forward_ws_bytes(d));
    REQUIRE_PTR(workspace);
  }

  if (!(d->flags & TP_MLP_NORMED_READY))
    CHECK_HIP(launch_rmsnorm_fwd(dt, x, norm_w, normed, rstd, T, H, d->eps, s), "rmsnorm forward");

  // Expansion: [T, H] x [2F | F, H]^T with the activation fused.
  GemmArgs g{};
  g.M = T;
  g.N = swiglu ? 2 * F : F;
  g.K = H;
  g.A = normed;
  g.lda = H;
  g.B = w_in;
  g.ldb = H;
  g.pre = pre_act;
  g.act = act;
  g.bias = b_in;
  g.ffn = F;
  g.tag = swiglu ? "gemm_gate_up_swiglu" : "gemm_fc1_gelu";
  CHECK_HIP(launch_gemm(dt, true, true, swiglu ? kEpiSwigluFwd : kEpiGeluFwd, g, s), "expansion GEMM");

  // Contraction: [T, F] x [H, F]^T -> fp32 partial, or x + z + b_down.
  GemmArgs c{};
  c.M = T;
  c.N = H;
  c.K = F;
  c.A = act;
  c.lda = F;
  c.B = w_down;
  c.ldb = F;
  c.C = out;
  c.ldc = H;
  c.aux = x;
  c.bias = b_down;
  c.ffn = F;
  c.tag = fuse ? "gemm_down_residual" : "gemm_down_partial";
  // short k (F <= 2048): tiles grouped by 2 tile rows instead of 4 (measured 116.8 -> 108.5 us at T 8192,
  // H 4096, F 1792; at F 3584 no change, at F 14336 slower)
  c.tile_group = F <= 2048 ? 2 : 0;
  if (ks > 1) {
    // k split: the slices go to the workspace and are added in index order
    c.ksplit = ks;
    if (fuse) {
      float* z = static_cast<float*>(workspace);
      c.C = z;
      c.ws = z + T * H;
      CHECK_HIP(launch_gemm(dt, true, true, kEpiStoreF32, c, s), "down GEMM");
      const float* parts[1] = {z};
      CHECK_HIP(launch_partial_sum(parts, 1, T, H, x, b_down, dt, out, dt, s), "residual and bias");
    } else {
      c.ws = static_cast<float*>(workspace);
      CHECK_HIP(launch_gemm(dt, true, true, kEpiStoreF32, c, s), "down GEMM");
    }
    return TP_MLP_OK;
  }
  CHECK_HIP(launch_gemm(dt, true, true, fuse ? kEpiResidual : kEpiStoreF32, c, s), "down GEMM");
  return TP_MLP_OK;
}

}  // namespace

extern "C" {

int tp_mlp_forward(const tp_mlp_desc* d, const void* x, const void* norm_w, const void* w_in, const void* b_in,
                   const void* w_down, void* normed, float* rstd, void* pre_act, void* act, void* out,
                   const void* b_down, void* stream) {
  return forward_checked(d, x, norm_w, w_in, b_in, w_down, normed, rstd, pre_act, act, out, b_down, false, nullptr, 0,
                         stream, "tp_mlp_forward");
}

size_t tp_mlp_forward_workspace_bytes(const tp_mlp_desc* d) {
  if (!d || d->tokens < 0 || d->hidden <= 0 || d->ffn_local <= 0) return 0;
  return forward_ws_bytes(d);
}

int tp_mlp_forward_ws(const tp_mlp_desc* d, const void* x, const void* norm_w, const void* w_in, const void* b_in,
                      const void* w_down, void* normed, float* rstd, void* pre_act, void* act, void* out,
                      const void* b_down, void* workspace, size_t workspace_bytes, void* stream) {
  return forward_checked(d, x, norm_w, w_in, b_in, w_down, normed, rstd, pre_act, act, out, b_down, true, workspace,
                         workspace_bytes, stream, "tp_mlp_forward_ws");
}

int tp_partial_sum(const float* const* parts, int32_t n_parts, int64_t rows, int64_t cols, const void* residual,
                   const void* bias, int32_t in_dtype, void* out, int32_t out_dtype, void* stream) {
  const char* fn = "tp_partial_sum";
  g_err[0] = 0;
  if (!parts) return fail(TP_MLP_EINVAL, "%s: parts is NULL", fn);
  if (n_parts < 1 || n_parts > 64) return fail(TP_MLP_EINVAL, "%s: n_parts must be in [1, 64]", fn);
  if (rows < 0 || cols < 0) return fail(TP_MLP_EINVAL, "%s: negative size", fn);
  if (cols % 4) return fail(TP_MLP_ESHAPE, "%s: cols must be a multiple of 4", fn);
  if ((in_dtype != TP_MLP_F32 && in_dtype != TP_MLP_BF16) || (out_dtype != TP_MLP_F32 && out_dtype != TP_MLP_BF16))
    return fail(TP_MLP_EDTYPE, "%s: unknown dtype", fn);
  if (rows == 0 || cols == 0) return TP_MLP_OK;
  REQUIRE_PTR(out);
  for (int i = 0; i < n_parts; ++i) {
    if (!parts[i]) return fail(TP_MLP_EINVAL, "%s: parts[%d] is NULL", fn, i);
    if (!aligned16(parts[i])) return fail(TP_MLP_EALIGN, "%s: parts[%d] is not 16-byte aligned", fn, i);
    if ((const void*)parts[i] == out) return fail(TP_MLP_EINVAL, "%s: out aliases parts[%d]", fn, i);
  }
  if (residual && !aligned16(residual)) return fail(TP_MLP_EALIGN, "%s: residual is not 16-byte aligned", fn);
  if (bias && !aligned16(bias)) return fail(TP_MLP_EALIGN, "%s: bias is not 16-byte aligned", fn);
  CHECK_HIP(launch_partial_sum(parts, n_parts, rows, cols, residual, bias, dt_of(in_dtype), out, dt_of(out_dtype),
                               static_cast<hipStream_t>(stream)),
            "partial sum");
  return TP_MLP_OK;
}

int tp_rmsnorm_forward(int64_t rows, int64_t hidden, int32_t dtype, float eps, const void* x, const void* w,
                       void* normed, float* rstd, void* stream) {
  const char* fn = "tp_rmsnorm_forward";
  g_err[0] = 0;
  if (rows < 0) return fail(TP_MLP_EINVAL, "%s: rows < 0", fn);
  if (hidden <= 0 || hidden % 8 != 0 || hidden > 16384)
    return fail(TP_MLP_ESHAPE, "%s: hidden must be a positive multiple of 8, at most 16384", fn);
  if (dtype != TP_MLP_F32 && dtype != TP_MLP_BF16) return fail(TP_MLP_EDTYPE, "%s: unknown dtype", fn);
  if (!(eps >= 0.0f) || !std::isfinite(eps)) return fail(TP_MLP_EINVAL, "%s: eps must be finite and >= 0", fn);
  if (rows == 0) return TP_MLP_OK;
  REQUIRE_PTR(x);
  REQUIRE_PTR(w);
  REQUIRE_PTR(normed);
  REQUIRE_PTR4(rstd);
  CHECK_HIP(launch_rmsnorm_fwd(dt_of(dtype), x, w, normed, rstd, rows, hidden, eps, static_cast<hipStream_t>(stream)),
            "rmsnorm forward");
  return TP_MLP_OK;
}

size_t tp_mlp_workspace_bytes(const tp_mlp_desc* d, int32_t phase) {
  if (!d || d->tokens < 0 || d->hidden <= 0 || d->ffn_local <= 0) return 0;
  const int64_t T = d->tokens, H = d->hidden, F = d->ffn_local;
  if (phase == TP_MLP_BWD_NORM) return rmsnorm_bwd_workspace(T, H);
  if (phase != TP_MLP_BWD_SHARD) return 0;
  size_t need = d->act == TP_MLP_ACT_GELU ? colsum_workspace(T, F) : 0;
  if (d->dtype == TP_MLP_BF16) {
    // k-split slices of the two weight-gradient GEMMs (K = T); they run one
    // after the other and share the workspace
    // (the FP8 backward's k extent is T rounded up to 16)
    // The bf16 d_act GEMM reads Wd transposed ([F, H]) from the workspace
    // before either of them runs.
    const int64_t P = d->act == TP_MLP_ACT_SWIGLU ? 2 * F : F;
    if (T > 0) need = need > (size_t)(F * H * 2) ? need : (size_t)(F * H * 2);
    // (with the update fused, tp_mlp_fused_sgd, every slice goes to the workspace)
    for (const int64_t K : {T, (T + 15) / 16 * 16}) {
      const size_t w2 = gemm_ksplit_workspace_sgd(H, F, K), w4 = gemm_ksplit_workspace_sgd(P, H, K);
      need = need > w2 ? need : w2;
      need = need > w4 ? need : w4;
    }
    // and of the input-gradient GEMM (K = P) when it has few tiles
    const size_t w3 = gemm_ksplit_workspace(T, H, P);
    need = need > w3 ? need : w3;
  }
  return need;
}

}  // extern "C"

namespace {

// The backward of both phases after the descriptor, the phase and the args
// pointer have been checked; a->workspace is the scratch its kernels use.
int backward_checked(const tp_mlp_desc* d, int32_t phase, const tp_mlp_bwd_args* a, void* stream, const char* fn) {
  const int64_t T = d->tokens, H = d->hidden, F = d->ffn_local;
  const bool swiglu = d->act == TP_MLP_ACT_SWIGLU;
  const DType dt = dt_of(d->dtype);
  const bool accum = (d->flags & TP_MLP_ACCUMULATE_GRADS) != 0;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const size_t need = tp_mlp_workspace_bytes(d, phase);
  if (need > 0) {
    if (!a->workspace || a->workspace_bytes < need)
      return fail(TP_MLP_EWORKSPACE, "%s: workspace of %zu bytes required, %zu given", fn, need,
                  a->workspace ? a->workspace_bytes : (size_t)0);
    if (!aligned16(a->workspace)) return fail(TP_MLP_EALIGN, "%s: workspace is not 16-byte aligned", fn);
  }

  if (phase == TP_MLP_BWD_NORM) {
    REQUIRE_PTR(a->norm_w);
    REQUIRE_PTR(a->d_norm_w);
    REQUIRE_PTR(a->d_b_down);
    const int np = a->n_d_normed_parts;
    if (np < 0 || np > kMaxNormParts)
      return fail(TP_MLP_EINVAL, "%s: n_d_normed_parts must be in [0, %d]", fn, kMaxNormParts);
    if (np > 0 && !a->d_normed_parts) return fail(TP_MLP_EINVAL, "%s: d_normed_parts is NULL", fn);
    const float* dn_one[1] = {a->d_normed};
    const float* const* parts = np > 0 ? a->d_normed_parts : dn_one;
    if (T > 0) {
      if (np > 0) {
        for (int k = 0; k < np; ++k) {
          const float* part = parts[k];
          REQUIRE_PTR(part);
        }
      } else {
        REQUIRE_PTR(a->d_normed);
      }
      REQUIRE_PTR(a->x);
      REQUIRE_PTR(a->d_out);
      REQUIRE_PTR4(a->rstd);
      REQUIRE_PTR(a->d_x);
    }
    CHECK_HIP(launch_rmsnorm_bwd(dt, parts, np > 0 ? np : 1, a->x, a->d_out, a->rstd, a->norm_w, a->d_x, a->d_norm_w,
                                 a->d_b_down, a->workspace, T, H, accum, s),
              "rmsnorm backward");
    return TP_MLP_OK;
  }

  // SHARD phase
  REQUIRE_PTR(a->w_in);
  REQUIRE_PTR(a->w_down);
  if (a->w_down_t) {
    if (!aligned16(a->w_down_t)) return fail(TP_MLP_EALIGN, "%s: 'w_down_t' is not 16-byte aligned", fn);
    if (dt != kBF16) return fail(TP_MLP_EDTYPE, "%s: w_down_t is taken for bf16 only", fn);
  }
  if (a->w_in_t) {
    if (!aligned16(a->w_in_t)) return fail(TP_MLP_EALIGN, "%s: 'w_in_t' is not 16-byte aligned", fn);
    if (dt != kBF16) return fail(TP_MLP_EDTYPE, "%s: w_in_t is taken for bf16 only", fn);
  }
  const tp_mlp_fused_sgd* fu = a->fused_sgd;
  if (fu) {
    if (dt != kBF16) return fail(TP_MLP_EDTYPE, "%s: fused_sgd is taken for bf16 only", fn);
    if (accum) return fail(TP_MLP_EINVAL, "%s: fused_sgd with TP_MLP_ACCUMULATE_GRADS", fn);
    if (!std::isfinite(fu->lr)) return fail(TP_MLP_EINVAL, "%s: fused_sgd->lr is not finite", fn);
    REQUIRE_PTR(fu->w_in_out);
    REQUIRE_PTR(fu->w_down_out);
    if (fu->w_in_t_out && !aligned16(fu->w_in_t_out))
      return fail(TP_MLP_EALIGN, "%s: 'fused_sgd->w_in_t_out' is not 16-byte aligned", fn);
    if (fu->w_down_t_out && !aligned16(fu->w_down_t_out))
      return fail(TP_MLP_EALIGN, "%s: 'fused_sgd->w_down_t_out' is not 16-byte aligned", fn);
    if (fu->w_in_master) {
      REQUIRE_PTR(fu->w_in_master);
      REQUIRE_PTR(fu->w_in_master_out);
    }
    if (fu->w_down_master) {
      REQUIRE_PTR(fu->w_down_master);
      REQUIRE_PTR(fu->w_down_master_out);
    }
  } else {
    REQUIRE_PTR(a->d_w_in);
    REQUIRE_PTR(a->d_w_down);
  }
  if (!swiglu) REQUIRE_PTR(a->d_b_in);
  if (swiglu && a->d_b_in) return fail(TP_MLP_EINVAL, "%s: d_b_in must be NULL for SwiGLU", fn);
  if (T > 0) {
    REQUIRE_PTR(a->d_out);
    REQUIRE_PTR(a->normed);
    REQUIRE_PTR(a->pre_act);
    REQUIRE_PTR(a->act);
    REQUIRE_PTR(a->d_pre);
    REQUIRE_PTR(a->d_normed_part);
  }
  const int64_t P = swiglu ? 2 * F : F;  // width of pre-activations
  if (a->d_pre_t || a->normed_t) {
    if (dt != kBF16) return fail(TP_MLP_EDTYPE, "%s: d_pre_t / normed_t are taken for bf16 only", fn);
    if (T % 8 != 0) return fail(TP_MLP_ESHAPE, "%s: d_pre_t / normed_t need T a multiple of 8", fn);
    if (a->d_pre_t && !aligned16(a->d_pre_t)) return fail(TP_MLP_EALIGN, "%s: 'd_pre_t' is not 16-byte aligned", fn);
    if (a->normed_t && !aligned16(a->normed_t))
      return fail(TP_MLP_EALIGN, "%s: 'normed_t' is not 16-byte aligned", fn);
    if (a->d_pre_t && !a->w_down_t) return fail(TP_MLP_EINVAL, "%s: d_pre_t needs w_down_t", fn);
  }
  // The w_in weight-gradient GEMM on K-contiguous operands (dW_in^T = normed_t d_pre_t^T): with the
  // update fused, no w_in masters (they are laid out as w_in), the old values read from w_in_t, and k
  // not split.
  const bool b4_nt = fu && !fu->w_in_master && a->w_in_t && a->normed_t && a->d_pre_t && T > 0 &&
                     gemm_ksplit(P, H, T) == 1;

  // d_act = d_out Wd ([T,H] x [H,F]), with the activation backward fused.  In
  // bf16 both operands are made K-contiguous (Wd^T [F, H] in the workspace) for
  // the ping-pong GEMM: the transpose moves 4 F H bytes, the GEMM gains more.
  GemmArgs b1{};
  b1.M = T;
  b1.N = F;
  b1.K = H;
  b1.A = a->d_out;
  b1.lda = H;
  b1.B = a->w_down;
  b1.ldb = F;
  b1.pre = a->d_pre;
  b1.aux = a->pre_act;
  b1.ffn = F;
  b1.tag = swiglu ? "gemm_dact_swiglu_bwd" : "gemm_dact_gelu_bwd";
  const Epi act_bwd = swiglu ? kEpiSwigluBwd : kEpiGeluBwd;
  if (dt == kBF16 && T > 0) {
    if (a->w_down_t) {
      b1.B = a->w_down_t;  // the caller's transposed copy
    } else {
      CHECK_HIP(launch_transpose_bf16(a->w_down, a->workspace, H, F, s), "Wd transpose");
      b1.B = a->workspace;
    }
    b1.ldb = H;
    b1.pre_t = a->d_pre_t;  // the transposed copy of d_pre as well, when asked for
    b1.ld_t = T;
    const Epi e1 = a->d_pre_t ? (swiglu ? kEpiSwigluBwdT : kEpiGeluBwdT) : act_bwd;
    CHECK_HIP(launch_gemm(dt, true, true, e1, b1, s), "d_act GEMM");
  } else {
    CHECK_HIP(launch_gemm(dt, true, false, act_bwd, b1, s), "d_act GEMM");
  }

  // d_w_down = d_out^T act ([H,T] x [T,F]); with the update fused, applied to
  // w_down as it is formed (d_act above has already read w_down / w_down_t).
  GemmArgs b2{};
  b2.M = H;
  b2.N = F;
  b2.K = T;
  b2.A = a->d_out;
  b2.lda = H;
  b2.B = a->act;
  b2.ldb = F;
  b2.C = a->d_w_down;
  b2.ldc = F;
  b2.tag = fu ? "gemm_wgrad_down_sgd" : "gemm_wgrad_down";
  b2.ksplit = gemm_ksplit(b2.M, b2.N, b2.K);
  b2.ws = static_cast<float*>(a->workspace);
  b2.accum = accum;
  if (fu) {
    b2.sgd = SgdEpi{a->w_down, a->w_down_t, fu->w_down_out, fu->w_down_t_out, fu->w_down_master,
                    fu->w_down_master_out, fu->lr};
    CHECK_HIP(launch_gemm(dt, false, false, kEpiSgd, b2, s), "d_w_down GEMM + SGD");
  } else {
    CHECK_HIP(launch_gemm(dt, false, false, kEpiStoreF32, b2, s), "d_w_down GEMM");
  }

  // d_w_in = d_pre^T normed ([P,T] x [T,H]), or with the update fused, w_in's update.
  GemmArgs b4{};
  b4.M = P;
  b4.N = H;
  b4.K = T;
  b4.A = a->d_pre;
  b4.lda = P;
  b4.B = a->normed;
  b4.ldb = H;
  b4.C = a->d_w_in;
  b4.ldc = H;
  b4.tag = fu ? (swiglu ? "gemm_wgrad_gate_up_sgd" : "gemm_wgrad_fc1_sgd")
              : (swiglu ? "gemm_wgrad_gate_up" : "gemm_wgrad_fc1");
  b4.ksplit = gemm_ksplit(b4.M, b4.N, b4.K);
  b4.ws = static_cast<float*>(a->workspace);
  b4.accum = accum;
  if (fu)
    b4.sgd = SgdEpi{a->w_in, a->w_in_t, fu->w_in_out, fu->w_in_t_out, fu->w_in_master, fu->w_in_master_out, fu->lr};
  if (b4_nt) {  // dW_in^T [H, P] = normed_t [H, T] x d_pre_t [P, T]^T
    b4.M = H;
    b4.N = P;
    b4.A = a->normed_t;
    b4.lda = T;
    b4.B = a->d_pre_t;
    b4.ldb = T;
    b4.ksplit = 1;
  }
  auto run_b4 = [&]() -> int {
    if (b4_nt) {
      CHECK_HIP(launch_gemm(dt, true, true, kEpiSgdT, b4, s), "d_w_in^T GEMM + SGD");
    } else if (fu) {
      CHECK_HIP(launch_gemm(dt, false, false, kEpiSgd, b4, s), "d_w_in GEMM + SGD");
    } else {
      CHECK_HIP(launch_gemm(dt, false, false, kEpiStoreF32, b4, s), "d_w_in GEMM");
    }
    return TP_MLP_OK;
  };
  // An in-place update of w_in must wait for the d_normed GEMM below, which reads it.
  const bool b4_after_b3 = fu && (fu->w_in_out == a->w_in || (a->w_in_t && fu->w_in_t_out == a->w_in_t));
  if (!b4_after_b3) {
    const int rc = run_b4();
    if (rc) return rc;
  }

  if (!swiglu)
    CHECK_HIP(launch_colsum(dt, a->d_pre, a->d_b_in, a->workspace, T, F, accum, s), "d_b_in column sum");

  // d_normed partial = d_pre w_in ([T,P] x [P,H]), last: the norm backward
  // that follows the last shard reads this partial while it is still in the
  // memory-side cache, instead of evicting a weight gradient written after it.
  GemmArgs b3{};
  b3.M = T;
  b3.N = H;
  b3.K = P;
  b3.A = a->d_pre;
  b3.lda = P;
  b3.B = a->w_in;
  b3.ldb = H;
  b3.C = a->d_normed_part;
  b3.ldc = H;
  b3.tag = "gemm_dgrad_normed";
  b3.ksplit = gemm_ksplit(b3.M, b3.N, b3.K);
  b3.ws = static_cast<float*>(a->workspace);
  if (dt == kBF16 && a->w_in_t) {
    b3.B = a->w_in_t;  // the caller's transposed copy: both operands K-contiguous
    b3.ldb = P;
    CHECK_HIP(launch_gemm(dt, true, true, kEpiStoreF32, b3, s), "d_normed GEMM");
  } else {
    CHECK_HIP(launch_gemm(dt, true, false, kEpiStoreF32, b3, s), "d_normed GEMM");
  }
  if (b4_after_b3) return run_b4();
  return TP_MLP_OK;
}

int check_bwd_call(const tp_mlp_desc* d, int32_t phase, const tp_mlp_bwd_args* a, const char* fn) {
  const int rc = check_desc(d, fn);
  if (rc) return rc;
  if (!a) return fail(TP_MLP_EINVAL, "%s: args is NULL", fn);
  if (phase != TP_MLP_BWD_SHARD && phase != TP_MLP_BWD_NORM) return fail(TP_MLP_EINVAL, "%s: unknown phase", fn);
  return TP_MLP_OK;
}

// Scratch of tp_mlp_backward_noalloc: a device array of the library's own,
// one per GPU (each device's copy lives at its own address for as long as
// the process runs).  Host code never passes the array's name to a kernel:
// the name is a host-side stand-in; the device address is taken once per
// device with hipGetSymbolAddress, with that device current, and kept.
static __device__ __align__(256) unsigned char scratch[TP_MLP_NOALLOC_SCRATCH_BYTES];
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

int scratch_of_current_device(const char* fn, void** out) {
  int dev = -1;
  CHECK_HIP(hipGetDevice(&dev), "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices) return fail(TP_MLP_EINVAL, "%s: device index %d out of range", fn, dev);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    CHECK_HIP(hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)), "hipGetSymbolAddress(scratch)");
    if (!ptr) return fail(TP_MLP_EHIP, "%s: no device address for the scratch array", fn);
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return TP_MLP_OK;
}

}  // namespace

extern "C" {

int tp_mlp_backward(const tp_mlp_desc* d, int32_t phase, const tp_mlp_bwd_args* a, void* stream) {
  const char* fn = "tp_mlp_backward";
  g_err[0] = 0;
  const int rc = check_bwd_call(d, phase, a, fn);
  if (rc) return rc;
  return backward_checked(d, phase, a, stream, fn);
}

int tp_mlp_backward_noalloc(const tp_mlp_desc* d, int32_t phase, const tp_mlp_bwd_args* a, void* stream) {
  const char* fn = "tp_mlp_backward_noalloc";
  g_err[0] = 0;
  int rc = check_bwd_call(d, phase, a, fn);
  if (rc) return rc;
  const size_t need = tp_mlp_workspace_bytes(d, phase);
  if (need > (size_t)TP_MLP_NOALLOC_SCRATCH_BYTES)
    return fail(TP_MLP_EWORKSPACE, "%s: this call needs %zu bytes of scratch, more than the %zu the library holds",
                fn, need, (size_t)TP_MLP_NOALLOC_SCRATCH_BYTES);
  void* ptr = nullptr;
  rc = scratch_of_current_device(fn, &ptr);
  if (rc) return rc;
  tp_mlp_bwd_args b = *a;  // the caller's tensors with the library's scratch
  b.workspace = ptr;
  b.workspace_bytes = (size_t)TP_MLP_NOALLOC_SCRATCH_BYTES;
  return backward_checked(d, phase, &b, stream, fn);
}

}  // extern "C"

namespace {

int check_sgd_tensor(const tp_mlp_sgd_tensor& t, int32_t param_dtype, bool master, const char* fn) {
  if (t.n < 0) return fail(TP_MLP_EINVAL, "%s: n < 0", fn);
  if ((t.master_in != nullptr) != master)
    return fail(TP_MLP_EINVAL, "%s: either every tensor has a master copy or none does", fn);
  if (t.master_in && param_dtype != TP_MLP_BF16)
    return fail(TP_MLP_EDTYPE, "%s: a master copy is only used with bf16 parameters", fn);
  if (t.n == 0) return TP_MLP_OK;
  const void* param_in = t.param_in;
  void* param_out = t.param_out;
  const float* grad = t.grad;
  REQUIRE_PTR(param_in);
  REQUIRE_PTR(param_out);
  REQUIRE_PTR(grad);
  if (t.master_in) {
    const float* master_in = t.master_in;
    float* master_out = t.master_out;
    REQUIRE_PTR(master_in);
    REQUIRE_PTR(master_out);
  }
  if (t.param_out_t) {
    void* param_out_t = t.param_out_t;
    REQUIRE_PTR(param_out_t);
    if (param_dtype != TP_MLP_BF16) return fail(TP_MLP_EDTYPE, "%s: a transposed copy is written for bf16 only", fn);
    if (t.t_rows <= 0 || t.t_cols <= 0 || t.t_rows % 8 || t.t_cols % 8 || t.t_rows * t.t_cols != t.n)
      return fail(TP_MLP_ESHAPE, "%s: t_rows x t_cols must equal n, both positive multiples of 8", fn);
  }
  return TP_MLP_OK;
}

int sgd_list(const tp_mlp_sgd_tensor* list, int32_t count, int32_t param_dtype, float lr, void* stream,
             const char* fn) {
  if (count < 0) return fail(TP_MLP_EINVAL, "%s: count < 0", fn);
  if (count > 0 && !list) return fail(TP_MLP_EINVAL, "%s: list is NULL", fn);
  if (param_dtype != TP_MLP_F32 && param_dtype != TP_MLP_BF16) return fail(TP_MLP_EDTYPE, "%s: unknown dtype", fn);
  const bool master = count > 0 && list[0].master_in != nullptr;
  for (int i = 0; i < count; ++i) {
    const int rc = check_sgd_tensor(list[i], param_dtype, master, fn);
    if (rc) return rc;
  }
  if (count == 0) return TP_MLP_OK;
  static_assert(sizeof(tp_mlp_sgd_tensor) == sizeof(SgdTensor), "SGD tensor layouts match");
  CHECK_HIP(launch_sgd(dt_of(param_dtype), reinterpret_cast<const SgdTensor*>(list), count, master, lr,
                       static_cast<hipStream_t>(stream)),
            "sgd");
  return TP_MLP_OK;
}

}  // namespace

extern "C" {

int tp_mlp_transpose_bf16(const void* in, void* out, int64_t rows, int64_t cols, void* stream) {
  const char* fn = "tp_mlp_transpose_bf16";
  g_err[0] = 0;
  if (rows < 0 || cols < 0 || rows % 8 || cols % 8)
    return fail(TP_MLP_ESHAPE, "%s: rows and cols must be non-negative multiples of 8", fn);
  if (rows == 0 || cols == 0) return TP_MLP_OK;
  REQUIRE_PTR(in);
  REQUIRE_PTR(out);
  if (rows * cols >= ((int64_t)1 << 31)) return fail(TP_MLP_ESHAPE, "%s: 2^31 or more elements", fn);
  CHECK_HIP(launch_transpose_bf16(in, out, rows, cols, static_cast<hipStream_t>(stream)), "transpose");
  return TP_MLP_OK;
}

int tp_mlp_sgd_step(const void* param_in, void* param_out, const float* grad, const float* master_in,
                    float* master_out, int64_t n, int32_t param_dtype, float lr, void* stream) {
  g_err[0] = 0;
  const tp_mlp_sgd_tensor t{param_in, param_out, grad, master_in, master_out, n, nullptr, 0, 0};
  return sgd_list(&t, 1, param_dtype, lr, stream, "tp_mlp_sgd_step");
}

int tp_mlp_sgd_step_multi(const tp_mlp_sgd_tensor* list, int32_t count, int32_t param_dtype, float lr,
                          void* stream) {
  g_err[0] = 0;
  return sgd_list(list, count, param_dtype, lr, stream, "tp_mlp_sgd_step_multi");
}

int tp_mlp_adamw_step_multi(const tp_mlp_adamw_tensor* list, int32_t count, int32_t param_dtype,
                            const tp_mlp_adamw_hparams* hp, const float* grad_scale, void* stream) {
  const char* fn = "tp_mlp_adamw_step_multi";
  g_err[0] = 0;
  if (count < 0) return fail(TP_MLP_EINVAL, "%s: count < 0", fn);
  if (count > 0 && !list) return fail(TP_MLP_EINVAL, "%s: list is NULL", fn);
  if (!hp) return fail(TP_MLP_EINVAL, "%s: hparams is NULL", fn);
  if (param_dtype != TP_MLP_F32 && param_dtype != TP_MLP_BF16) return fail(TP_MLP_EDTYPE, "%s: unknown dtype", fn);
  if (hp->step < 1) return fail(TP_MLP_EINVAL, "%s: step must be >= 1", fn);
  if (!(hp->beta1 >= 0.0f && hp->beta1 < 1.0f) || !(hp->beta2 >= 0.0f && hp->beta2 < 1.0f))
    return fail(TP_MLP_EINVAL, "%s: betas must lie in [0, 1)", fn);
  if (!(hp->eps > 0.0f) || !(hp->weight_decay >= 0.0f) || !std::isfinite(hp->lr))
    return fail(TP_MLP_EINVAL, "%s: eps must be > 0, weight_decay >= 0, lr finite", fn);
  if (grad_scale && (reinterpret_cast<uintptr_t>(grad_scale) & 3))
    return fail(TP_MLP_EALIGN, "%s: grad_scale is not 4-byte aligned", fn);
  const bool master = count > 0 && list[0].master_in != nullptr;
  for (int i = 0; i < count; ++i) {
    const tp_mlp_adamw_tensor& t = list[i];
    if (t.n < 0) return fail(TP_MLP_EINVAL, "%s: n < 0", fn);
    if ((t.master_in != nullptr) != master)
      return fail(TP_MLP_EINVAL, "%s: either every tensor has a master copy or none does", fn);
    if (t.master_in && param_dtype != TP_MLP_BF16)
      return fail(TP_MLP_EDTYPE, "%s: a master copy is only used with bf16 parameters", fn);
    if (t.n == 0) continue;
    void* param_out = t.param_out;
    const float* grad = t.grad;
    float* m = t.m;
    float* v = t.v;
    REQUIRE_PTR(param_out);
    REQUIRE_PTR(grad);
    REQUIRE_PTR(m);
    REQUIRE_PTR(v);
    if (master) {
      float* master_out = t.master_out;
      REQUIRE_PTR(master_out);
      if (!aligned16(t.master_in) || !aligned16(master_out))
        return fail(TP_MLP_EALIGN, "%s: tensor %d master is not 16-byte aligned", fn, i);
    } else {
      const void* param_in = t.param_in;
      REQUIRE_PTR(param_in);
      if (!aligned16(param_in)) return fail(TP_MLP_EALIGN, "%s: tensor %d param_in is not 16-byte aligned", fn, i);
    }
    if (!aligned16(param_out) || !aligned16(grad) || !aligned16(m) || !aligned16(v))
      return fail(TP_MLP_EALIGN, "%s: tensor %d has a pointer that is not 16-byte aligned", fn, i);
  }
  if (count == 0) return TP_MLP_OK;
  static_assert(sizeof(tp_mlp_adamw_tensor) == sizeof(AdamwTensor), "AdamW tensor layouts match");
  AdamwConst c;
  c.lr = hp->lr;
  c.beta1 = hp->beta1;
  c.beta2 = hp->beta2;
  c.eps = hp->eps;
  c.weight_decay = hp->weight_decay;
  c.bc1 = (float)(1.0 - std::pow((double)hp->beta1, (double)hp->step));
  c.bc2 = (float)(1.0 - std::pow((double)hp->beta2, (double)hp->step));
  CHECK_HIP(launch_adamw(dt_of(param_dtype), reinterpret_cast<const AdamwTensor*>(list), count, master, c, grad_scale,
                         static_cast<hipStream_t>(stream)),
            "adamw");
  return TP_MLP_OK;
}

size_t tp_mlp_clip_grad_norm_workspace_bytes(const int64_t* counts, int32_t count) {
  if (count <= 0 || !counts) return 0;
  for (int i = 0; i < count; ++i)
    if (counts[i] < 0) return 0;
  return sumsq_blocks(counts, count) * sizeof(double);
}

int tp_mlp_clip_grad_norm(const float* const* grads, const int64_t* counts, int32_t count, float max_norm,
                          float* norm_out, float* coef_out, void* workspace, size_t workspace_bytes,
                          void* stream) {
  const char* fn = "tp_mlp_clip_grad_norm";
  g_err[0] = 0;
  if (count < 0) return fail(TP_MLP_EINVAL, "%s: count < 0", fn);
  if (count > 0 && (!grads || !counts)) return fail(TP_MLP_EINVAL, "%s: grads or counts is NULL", fn);
  REQUIRE_PTR(coef_out);
  if (!std::isfinite(max_norm)) return fail(TP_MLP_EINVAL, "%s: max_norm is not finite", fn);
  for (int i = 0; i < count; ++i) {
    if (counts[i] < 0) return fail(TP_MLP_EINVAL, "%s: counts[%d] < 0", fn, i);
    if (counts[i] == 0) continue;
    if (!grads[i]) return fail(TP_MLP_EINVAL, "%s: grads[%d] is NULL", fn, i);
    if (!aligned16(grads[i])) return fail(TP_MLP_EALIGN, "%s: grads[%d] is not 16-byte aligned", fn, i);
  }
  const size_t need = tp_mlp_clip_grad_norm_workspace_bytes(counts, count);
  if (need > 0) {
    if (!workspace || workspace_bytes < need)
      return fail(TP_MLP_EWORKSPACE, "%s: workspace of %zu bytes required, %zu given", fn, need,
                  workspace ? workspace_bytes : (size_t)0);
    if (!aligned16(workspace)) return fail(TP_MLP_EALIGN, "%s: workspace is not 16-byte aligned", fn);
  }
  CHECK_HIP(launch_clip_grad_norm(grads, counts, count, max_norm, norm_out, coef_out, static_cast<double*>(workspace),
                                  static_cast<hipStream_t>(stream)),
            "gradient norm");
  return TP_MLP_OK;
}

// ------------------------------------------------------------------ FP8

}  // extern "C"

namespace {

int check_meta_args(int32_t history_len, const char* fn) {
  if (history_len < 1 || history_len > TP_MLP_FP8_MAX_HISTORY)
    return fail(TP_MLP_EINVAL, "%s: history_len must be in [1, %d]", fn, TP_MLP_FP8_MAX_HISTORY);
  return TP_MLP_OK;
}

#define REQUIRE_META(p)                                                            \
  do {                                                                             \
    if (!(p)) return fail(TP_MLP_EINVAL, "%s: meta '%s' is NULL", fn, #p);         \
    if (reinterpret_cast<uintptr_t>(p) & 3u) return fail(TP_MLP_EALIGN, "%s: meta '%s' is not 4-byte aligned", fn, #p); \
  } while (0)

int check_fp8_desc(const tp_mlp_desc* d, const tp_mlp_fp8_args* f8, const char* fn) {
  if (d->dtype != TP_MLP_BF16) return fail(TP_MLP_EDTYPE, "%s: the FP8 path takes bf16 tensors", fn);
  if (d->hidden % 16 || d->ffn_local % 16)
    return fail(TP_MLP_ESHAPE, "%s: hidden and ffn_local must be multiples of 16 for FP8", fn);
  if (!f8) return fail(TP_MLP_EINVAL, "%s: fp8 args are NULL", fn);
  return check_meta_args(f8->history_len, fn);
}

GemmArgs fp8_gemm(int64_t M, int64_t N, int64_t K, const void* A, int64_t lda, const float* meta_a, const void* B,
                  int64_t ldb, const float* meta_b, const char* tag) {
  GemmArgs g{};
  g.M = M;
  g.N = N;
  g.K = K;
  g.A = A;
  g.lda = lda;
  g.B = B;
  g.ldb = ldb;
  g.scale_inv_a = meta_a + 1;
  g.scale_inv_b = meta_b + 1;
  g.tag = tag;
  return g;
}

}  // namespace

extern "C" {

int tp_mlp_fp8_meta_init(float* meta, int32_t fmt, int32_t history_len, void* stream) {
  const char* fn = "tp_mlp_fp8_meta_init";
  g_err[0] = 0;
  if (fmt != TP_MLP_FP8_E4M3 && fmt != TP_MLP_FP8_E5M2) return fail(TP_MLP_EINVAL, "%s: unknown format", fn);
  int rc = check_meta_args(history_len, fn);
  if (rc) return rc;
  REQUIRE_META(meta);
  CHECK_HIP(launch_fp8_meta_init(meta, fmt, history_len, static_cast<hipStream_t>(stream)), "fp8 meta init");
  return TP_MLP_OK;
}

int tp_mlp_fp8_cast(int64_t rows, int64_t cols, const void* x, int32_t fmt, float* meta, uint8_t* out,
                    uint8_t* out_t, int64_t ldt, void* stream) {
  const char* fn = "tp_mlp_fp8_cast";
  g_err[0] = 0;
  if (fmt != TP_MLP_FP8_E4M3 && fmt != TP_MLP_FP8_E5M2) return fail(TP_MLP_EINVAL, "%s: unknown format", fn);
  if (rows < 0 || cols < 0) return fail(TP_MLP_EINVAL, "%s: negative size", fn);
  if (cols % 8) return fail(TP_MLP_ESHAPE, "%s: cols must be a multiple of 8", fn);
  if (rows * cols >= ((int64_t)1 << 31)) return fail(TP_MLP_ESHAPE, "%s: 2^31 or more elements", fn);
  if (!out && !out_t) return fail(TP_MLP_EINVAL, "%s: out and out_t are both NULL", fn);
  if (out_t && (ldt < rows || ldt % 16)) return fail(TP_MLP_ESHAPE, "%s: ldt must be >= rows and a multiple of 16", fn);
  if (out_t && cols * ldt >= ((int64_t)1 << 31)) return fail(TP_MLP_ESHAPE, "%s: out_t too large", fn);
  REQUIRE_META(meta);
  if (cols == 0 || (rows == 0 && (!out_t || ldt == 0))) return TP_MLP_OK;
  if (rows > 0) REQUIRE_PTR(x);  // rows = 0: only the zero padding of out_t is written
  if (out) REQUIRE_PTR(out);
  if (out_t) REQUIRE_PTR(out_t);
  CHECK_HIP(launch_fp8_cast(fmt, x, rows, cols, out, out_t, ldt, meta, "fp8_cast", static_cast<hipStream_t>(stream)),
            "fp8 cast");
  return TP_MLP_OK;
}

int tp_mlp_fp8_update_scales(float* const* metas, int32_t count, int32_t history_len, void* stream) {
  const char* fn = "tp_mlp_fp8_update_scales";
  g_err[0] = 0;
  if (count < 0 || count > kFp8MaxMetas) return fail(TP_MLP_EINVAL, "%s: count must be in [0, %d]", fn, kFp8MaxMetas);
  if (count > 0 && !metas) return fail(TP_MLP_EINVAL, "%s: metas is NULL", fn);
  int rc = check_meta_args(history_len, fn);
  if (rc) return rc;
  for (int i = 0; i < count; ++i) {
    float* m = metas[i];
    REQUIRE_META(m);
  }
  CHECK_HIP(launch_fp8_update(metas, count, history_len, static_cast<hipStream_t>(stream)), "fp8 scale update");
  return TP_MLP_OK;
}

size_t tp_mlp_fp8_gemm_workspace_bytes(int64_t M, int64_t N, int64_t K, int64_t ldc) {
  if (M <= 0 || N <= 0 || K <= 0 || ldc < N) return 0;
  return (size_t)(gemm_ksplit(M, N, K) - 1) * (size_t)M * (size_t)ldc * sizeof(float);
}

int tp_mlp_fp8_gemm(int64_t M, int64_t N, int64_t K, const uint8_t* A, int64_t lda, int32_t fmt_a,
                    const float* scale_inv_a, const uint8_t* B, int64_t ldb, int32_t fmt_b, const float* scale_inv_b,
                    float* C, int64_t ldc, int32_t accumulate, void* workspace, size_t workspace_bytes, void* stream) {
  const char* fn = "tp_mlp_fp8_gemm";
  g_err[0] = 0;
  if (M < 0 || N < 0 || K < 0) return fail(TP_MLP_EINVAL, "%s: negative size", fn);
  if (!((fmt_a == TP_MLP_FP8_E4M3 && fmt_b == TP_MLP_FP8_E4M3) || (fmt_a == TP_MLP_FP8_E5M2 && fmt_b == TP_MLP_FP8_E4M3)))
    return fail(TP_MLP_EINVAL, "%s: formats must be (E4M3, E4M3) or (E5M2, E4M3)", fn);
  if (K % 16 || lda % 16 || ldb % 16 || lda < K || ldb < K)
    return fail(TP_MLP_ESHAPE, "%s: K, lda, ldb must be multiples of 16 with K <= lda, ldb", fn);
  if (N % 4 || ldc < N || ldc % 4) return fail(TP_MLP_ESHAPE, "%s: N and ldc must be multiples of 4, ldc >= N", fn);
  if (M * lda >= ((int64_t)1 << 31) || N * ldb >= ((int64_t)1 << 31) || M * ldc >= ((int64_t)1 << 31))
    return fail(TP_MLP_ESHAPE, "%s: an operand holds 2^31 or more elements", fn);
  if (M == 0 || N == 0) return TP_MLP_OK;
  REQUIRE_PTR(C);
  REQUIRE_META(scale_inv_a);
  REQUIRE_META(scale_inv_b);
  if (K > 0) {
    REQUIRE_PTR(A);
    REQUIRE_PTR(B);
  }
  const size_t need = tp_mlp_fp8_gemm_workspace_bytes(M, N, K, ldc);
  if (need > 0) {
    if (!workspace || workspace_bytes < need)
      return fail(TP_MLP_EWORKSPACE, "%s: workspace of %zu bytes required, %zu given", fn, need,
                  workspace ? workspace_bytes : (size_t)0);
    if (!aligned16(workspace)) return fail(TP_MLP_EALIGN, "%s: workspace is not 16-byte aligned", fn);
  }
  GemmArgs g{};
  g.M = M;
  g.N = N;
  g.K = K;
  g.A = A;
  g.lda = lda;
  g.B = B;
  g.ldb = ldb;
  g.C = C;
  g.ldc = ldc;
  g.scale_inv_a = scale_inv_a;
  g.scale_inv_b = scale_inv_b;
  g.accum = accumulate != 0;
  g.ksplit = gemm_ksplit(M, N, K);
  g.ws = static_cast<float*>(workspace);
  g.tag = "gemm_fp8";
  CHECK_HIP(launch_gemm_fp8(fmt_a, fmt_b, kEpiStoreF32, g, static_cast<hipStream_t>(stream)), "fp8 GEMM");
  return TP_MLP_OK;
}

int tp_mlp_forward_fp8(const tp_mlp_desc* d, const void* x, const void* norm_w, const void* w_in, const void* b_in,
                       const void* w_down, void* normed, float* rstd, void* pre_act, void* act, void* out,
                       const void* b_down, const tp_mlp_fp8_args* f8, void* stream) {
  const char* fn = "tp_mlp_forward_fp8";
  g_err[0] = 0;
  int rc = check_desc(d, fn);
  if (rc) return rc;
  rc = check_fp8_desc(d, f8, fn);
  if (rc) return rc;
  const int64_t T = d->tokens, H = d->hidden, F = d->ffn_local;
  const bool swiglu = d->act == TP_MLP_ACT_SWIGLU;
  const bool fuse = d->flags & TP_MLP_FUSE_EPILOGUE;
  const bool ready = d->flags & TP_MLP_NORMED_READY;
  const int64_t P = swiglu ? 2 * F : F, Tp = (T + 15) / 16 * 16;
  REQUIRE_PTR(norm_w);
  REQUIRE_PTR(w_in);
  REQUIRE_PTR(w_down);
  if (swiglu && b_in) return fail(TP_MLP_EINVAL, "%s: b_in must be NULL for SwiGLU", fn);
  if (!swiglu) REQUIRE_PTR(b_in);
  if (fuse) REQUIRE_PTR(b_down);
  REQUIRE_META(f8->meta_normed);
  REQUIRE_META(f8->meta_w_in);
  REQUIRE_META(f8->meta_act);
  REQUIRE_META(f8->meta_w_down);
  REQUIRE_PTR(f8->w_in_q);
  REQUIRE_PTR(f8->w_in_t);
  REQUIRE_PTR(f8->w_down_q);
  REQUIRE_PTR(f8->w_down_t);
  if (T == 0) return TP_MLP_OK;
  REQUIRE_PTR(x);
  REQUIRE_PTR(normed);
  REQUIRE_PTR4(rstd);
  REQUIRE_PTR(pre_act);
  REQUIRE_PTR(act);
  REQUIRE_PTR(out);
  REQUIRE_PTR(f8->normed_q);
  REQUIRE_PTR(f8->normed_t);
  REQUIRE_PTR(f8->act_q);
  REQUIRE_PTR(f8->act_t);
  if (T * H >= ((int64_t)1 << 30) || H * Tp >= ((int64_t)1 << 30) || F * Tp >= ((int64_t)1 << 30))
    return fail(TP_MLP_ESHAPE, "%s: a transposed code tensor would hold 2^30 or more elements", fn);
  hipStream_t s = static_cast<hipStream_t>(stream);

  if (!ready) {
    CHECK_HIP(launch_rmsnorm_fwd(kBF16, x, norm_w, normed, rstd, T, H, d->eps, s), "rmsnorm forward");
    CHECK_HIP(launch_fp8_cast(kFp8E4M3, normed, T, H, f8->normed_q, f8->normed_t, Tp, f8->meta_normed,
                              "fp8_cast_normed", s),
              "normed cast");
  }
  CHECK_HIP(launch_fp8_cast(kFp8E4M3, w_in, P, H, f8->w_in_q, f8->w_in_t, P, f8->meta_w_in, "fp8_cast_weights", s),
            "w_in cast");

  GemmArgs g = fp8_gemm(T, P, H, f8->normed_q, H, f8->meta_normed, f8->w_in_q, H, f8->meta_w_in,
                        swiglu ? "gemm_gate_up_swiglu_fp8" : "gemm_fc1_gelu_fp8");
  g.pre = pre_act;
  g.act = act;
  g.bias = b_in;
  g.ffn = F;
  CHECK_HIP(launch_gemm_fp8(kFp8E4M3, kFp8E4M3, swiglu ? kEpiSwigluFwd : kEpiGeluFwd, g, s), "expansion GEMM");

  CHECK_HIP(launch_fp8_cast(kFp8E4M3, act, T, F, f8->act_q, f8->act_t, Tp, f8->meta_act, "fp8_cast_act", s),
            "act cast");
  CHECK_HIP(launch_fp8_cast(kFp8E4M3, w_down, H, F, f8->w_down_q, f8->w_down_t, H, f8->meta_w_down,
                            "fp8_cast_weights", s),
            "w_down cast");
  GemmArgs c = fp8_gemm(T, H, F, f8->act_q, F, f8->meta_act, f8->w_down_q, F, f8->meta_w_down,
                        fuse ? "gemm_down_residual_fp8" : "gemm_down_partial_fp8");
  c.C = out;
  c.ldc = H;
  c.aux = x;
  c.bias = b_down;
  c.ffn = F;
  CHECK_HIP(launch_gemm_fp8(kFp8E4M3, kFp8E4M3, fuse ? kEpiResidual : kEpiStoreF32, c, s), "down GEMM");
  return TP_MLP_OK;
}

int tp_mlp_backward_fp8(const tp_mlp_desc* d, int32_t phase, const tp_mlp_bwd_args* a, const tp_mlp_fp8_args* f8,
                        void* stream) {
  const char* fn = "tp_mlp_backward_fp8";
  g_err[0] = 0;
  int rc = check_desc(d, fn, TP_MLP_FP8_SHARED_READY);
  if (rc) return rc;
  rc = check_fp8_desc(d, f8, fn);
  if (rc) return rc;
  if (phase == TP_MLP_BWD_NORM) {
    tp_mlp_desc dn = *d;
    dn.flags &= ~TP_MLP_FP8_SHARED_READY;
    return tp_mlp_backward(&dn, phase, a, stream);
  }
  if (phase != TP_MLP_BWD_SHARD) return fail(TP_MLP_EINVAL, "%s: unknown phase", fn);
  if (!a) return fail(TP_MLP_EINVAL, "%s: args is NULL", fn);
  const int64_t T = d->tokens, H = d->hidden, F = d->ffn_local;
  const bool swiglu = d->act == TP_MLP_ACT_SWIGLU;
  const bool accum = (d->flags & TP_MLP_ACCUMULATE_GRADS) != 0;
  const bool shared_ready = (d->flags & TP_MLP_FP8_SHARED_READY) != 0;
  const int64_t P = swiglu ? 2 * F : F, Tp = (T + 15) / 16 * 16;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const size_t need = tp_mlp_workspace_bytes(d, phase);
  if (need > 0) {
    if (!a->workspace || a->workspace_bytes < need)
      return fail(TP_MLP_EWORKSPACE, "%s: workspace of %zu bytes required, %zu given", fn, need,
                  a->workspace ? a->workspace_bytes : (size_t)0);
    if (!aligned16(a->workspace)) return fail(TP_MLP_EALIGN, "%s: workspace is not 16-byte aligned", fn);
  }
  const tp_mlp_fused_sgd* fu = a->fused_sgd;
  if (fu) {
    if (accum) return fail(TP_MLP_EINVAL, "%s: fused_sgd with TP_MLP_ACCUMULATE_GRADS", fn);
    if (!std::isfinite(fu->lr)) return fail(TP_MLP_EINVAL, "%s: fused_sgd->lr is not finite", fn);
    REQUIRE_PTR(fu->w_in_out);
    REQUIRE_PTR(fu->w_down_out);
    if (fu->w_in_t_out && !aligned16(fu->w_in_t_out))
      return fail(TP_MLP_EALIGN, "%s: 'fused_sgd->w_in_t_out' is not 16-byte aligned", fn);
    if (fu->w_down_t_out && !aligned16(fu->w_down_t_out))
      return fail(TP_MLP_EALIGN, "%s: 'fused_sgd->w_down_t_out' is not 16-byte aligned", fn);
    if (fu->w_in_master) {
      REQUIRE_PTR(fu->w_in_master);
      REQUIRE_PTR(fu->w_in_master_out);
    } else {
      REQUIRE_PTR(a->w_in);  // the old values
    }
    if (fu->w_down_master) {
      REQUIRE_PTR(fu->w_down_master);
      REQUIRE_PTR(fu->w_down_master_out);
    } else {
      REQUIRE_PTR(a->w_down);
    }
  } else {
    REQUIRE_PTR(a->d_w_in);
    REQUIRE_PTR(a->d_w_down);
  }
  if (!swiglu) REQUIRE_PTR(a->d_b_in);
  if (swiglu && a->d_b_in) return fail(TP_MLP_EINVAL, "%s: d_b_in must be NULL for SwiGLU", fn);
  REQUIRE_META(f8->meta_normed);
  REQUIRE_META(f8->meta_w_in);
  REQUIRE_META(f8->meta_act);
  REQUIRE_META(f8->meta_w_down);
  REQUIRE_META(f8->meta_d_out);
  REQUIRE_META(f8->meta_d_pre);
  REQUIRE_PTR(f8->w_in_t);
  REQUIRE_PTR(f8->w_down_t);
  if (T > 0) {
    REQUIRE_PTR(a->d_out);
    REQUIRE_PTR(a->pre_act);
    REQUIRE_PTR(a->d_pre);
    REQUIRE_PTR(a->d_normed_part);
    REQUIRE_PTR(f8->normed_t);
    REQUIRE_PTR(f8->act_t);
    REQUIRE_PTR(f8->d_out_q);
    REQUIRE_PTR(f8->d_out_t);
    REQUIRE_PTR(f8->d_pre_q);
    REQUIRE_PTR(f8->d_pre_t);
    if (T * H >= ((int64_t)1 << 30) || H * Tp >= ((int64_t)1 << 30) || P * Tp >= ((int64_t)1 << 30))
      return fail(TP_MLP_ESHAPE, "%s: a transposed code tensor would hold 2^30 or more elements", fn);
  }
  // T = 0: the casts and the GEMMs with M = T do nothing; the weight-gradient GEMMs (k extent 0)
  // write zeros, or leave the buffers as they are when accumulating.
  if (!shared_ready)
    CHECK_HIP(launch_fp8_cast(kFp8E5M2, a->d_out, T, H, f8->d_out_q, f8->d_out_t, Tp, f8->meta_d_out,
                              "fp8_cast_d_out", s),
              "d_out cast");

  // d_act = d_out Wd on d_out_q [T, H] and w_down_t [F, H], the activation backward fused.
  GemmArgs b1 = fp8_gemm(T, F, H, f8->d_out_q, H, f8->meta_d_out, f8->w_down_t, H, f8->meta_w_down,
                         swiglu ? "gemm_dact_swiglu_bwd_fp8" : "gemm_dact_gelu_bwd_fp8");
  b1.pre = a->d_pre;
  b1.aux = a->pre_act;
  b1.ffn = F;
  CHECK_HIP(launch_gemm_fp8(kFp8E5M2, kFp8E4M3, swiglu ? kEpiSwigluBwd : kEpiGeluBwd, b1, s), "d_act GEMM");

  // d_w_down = d_out^T act on d_out_t [H, Tp] and act_t [F, Tp].
  GemmArgs b2 = fp8_gemm(H, F, Tp, f8->d_out_t, Tp, f8->meta_d_out, f8->act_t, Tp, f8->meta_act, "gemm_wgrad_down_fp8");
  b2.C = a->d_w_down;
  b2.ldc = F;
  b2.ksplit = gemm_ksplit(b2.M, b2.N, b2.K);
  b2.ws = static_cast<float*>(a->workspace);
  b2.accum = accum;
  // With the update fused it is applied here (the FP8 GEMMs read the weights' codes, cast before the
  // step, so an in-place update of the bf16 weights needs no ordering).
  if (fu) {
    b2.tag = "gemm_wgrad_down_sgd_fp8";
    b2.sgd = SgdEpi{a->w_down, nullptr, fu->w_down_out, fu->w_down_t_out, fu->w_down_master, fu->w_down_master_out,
                    fu->lr};
  }
  CHECK_HIP(launch_gemm_fp8(kFp8E5M2, kFp8E4M3, fu ? kEpiSgd : kEpiStoreF32, b2, s), "d_w_down GEMM");

  CHECK_HIP(launch_fp8_cast(kFp8E5M2, a->d_pre, T, P, f8->d_pre_q, f8->d_pre_t, Tp, f8->meta_d_pre,
                            "fp8_cast_d_pre", s),
            "d_pre cast");

  // d_w_in = d_pre^T normed on d_pre_t [P, Tp] and normed_t [H, Tp].
  GemmArgs b4 = fp8_gemm(P, H, Tp, f8->d_pre_t, Tp, f8->meta_d_pre, f8->normed_t, Tp, f8->meta_normed,
                         swiglu ? "gemm_wgrad_gate_up_fp8" : "gemm_wgrad_fc1_fp8");
  b4.C = a->d_w_in;
  b4.ldc = H;
  b4.ksplit = gemm_ksplit(b4.M, b4.N, b4.K);
  b4.ws = static_cast<float*>(a->workspace);
  b4.accum = accum;
  if (fu) {
    b4.tag = swiglu ? "gemm_wgrad_gate_up_sgd_fp8" : "gemm_wgrad_fc1_sgd_fp8";
    b4.sgd = SgdEpi{a->w_in, nullptr, fu->w_in_out, fu->w_in_t_out, fu->w_in_master, fu->w_in_master_out, fu->lr};
  }
  CHECK_HIP(launch_gemm_fp8(kFp8E5M2, kFp8E4M3, fu ? kEpiSgd : kEpiStoreF32, b4, s), "d_w_in GEMM");

  if (!swiglu)
    CHECK_HIP(launch_colsum(kBF16, a->d_pre, a->d_b_in, a->workspace, T, F, accum, s), "d_b_in column sum");

  // d_normed partial = d_pre w_in on d_pre_q [T, P] and w_in_t [H, P]; last, as in
  // the bf16 backward (the norm backward then reads it from the memory-side cache).
  GemmArgs b3 = fp8_gemm(T, H, P, f8->d_pre_q, P, f8->meta_d_pre, f8->w_in_t, P, f8->meta_w_in,
                         "gemm_dgrad_normed_fp8");
  b3.C = a->d_normed_part;
  b3.ldc = H;
  b3.ksplit = gemm_ksplit(b3.M, b3.N, b3.K);
  b3.ws = static_cast<float*>(a->workspace);
  CHECK_HIP(launch_gemm_fp8(kFp8E5M2, kFp8E4M3, kEpiStoreF32, b3, s), "d_normed GEMM");
  return TP_MLP_OK;
}

// ------------------------------------------------------------- attention

}  // extern "C"

namespace {

int check_attn_shape(int64_t batch, int64_t seq, int32_t n_q, int32_t n_kv, int32_t head_dim, const char* fn) {
  if (batch < 0 || seq < 0) return fail(TP_MLP_EINVAL, "%s: batch and seq must be >= 0", fn);
  if (head_dim != 64 && head_dim != 128) return fail(TP_MLP_ESHAPE, "%s: head_dim must be 64 or 128", fn);
  if (n_q <= 0 || n_kv <= 0 || n_q % n_kv) return fail(TP_MLP_ESHAPE, "%s: n_q must be a positive multiple of n_kv", fn);
  if (seq > (1 << 24) || batch > (1 << 24)) return fail(TP_MLP_ESHAPE, "%s: batch or seq too large", fn);
  return TP_MLP_OK;
}

int check_attn_desc(const tp_attn_desc* d, const char* fn) {
  if (!d) return fail(TP_MLP_EINVAL, "%s: descriptor is NULL", fn);
  int rc = check_attn_shape(d->batch, d->seq, d->n_q, d->n_kv, d->head_dim, fn);
  if (rc) return rc;
  if (d->hidden <= 0 || d->hidden % 8 || d->hidden > 16384)
    return fail(TP_MLP_ESHAPE, "%s: hidden must be a positive multiple of 8, <= 16384", fn);
  if (d->seq * (int64_t)(d->n_q + 2 * d->n_kv) * d->head_dim >= ((int64_t)1 << 30))
    return fail(TP_MLP_ESHAPE, "%s: one sequence's QKV rows hold 2^30 or more elements", fn);
  if (d->dtype != TP_MLP_BF16) return fail(TP_MLP_EDTYPE, "%s: the attention sublayer takes bf16 tensors", fn);
  if (d->flags & ~(TP_MLP_FUSE_EPILOGUE | TP_MLP_NORMED_READY | TP_MLP_ACCUMULATE_GRADS))
    return fail(TP_MLP_EINVAL, "%s: unknown flags", fn);
  if (!(d->eps >= 0.0f)) return fail(TP_MLP_EINVAL, "%s: eps must be >= 0", fn);
  const int64_t T = d->batch * d->seq, H = d->hidden;
  const int64_t W = (int64_t)(d->n_q + 2 * d->n_kv) * d->head_dim, Wo = (int64_t)d->n_q * d->head_dim;
  const int64_t lim = (int64_t)1 << 30;
  if (T * H >= lim || T * W >= lim || W * H >= lim || T * Wo >= lim || (int64_t)d->n_q * T >= lim)
    return fail(TP_MLP_ESHAPE, "%s: a tensor would hold 2^30 or more elements", fn);
  return TP_MLP_OK;
}

AttnShapeArgs attn_args(const tp_attn_desc* d) {
  AttnShapeArgs a;
  a.batch = d->batch;
  a.seq = d->seq;
  a.ld = (int64_t)(d->n_q + 2 * d->n_kv) * d->head_dim;
  a.n_q = d->n_q;
  a.n_kv = d->n_kv;
  a.head_dim = d->head_dim;
  return a;
}

// Workspace of the SHARD phase: the k-split slices of the dO GEMM and of the
// two weight-gradient GEMMs (they run one after the other and share them),
// then the attention backward's own (delta [n_q, T] and the per-head dK/dV
// shares).
size_t attn_ksplit_bytes(const tp_attn_desc* d) {
  const int64_t T = d->batch * d->seq, H = d->hidden;
  const int64_t W = (int64_t)(d->n_q + 2 * d->n_kv) * d->head_dim, Wo = (int64_t)d->n_q * d->head_dim;
  size_t m = gemm_ksplit_workspace(H, Wo, T);
  const size_t b = gemm_ksplit_workspace(W, H, T), c = gemm_ksplit_workspace_bf16(T, Wo, H);  // dW_qkv, dO
  if (b > m) m = b;
  if (c > m) m = c;
  return (m + 255) / 256 * 256;
}

}  // namespace

extern "C" {

size_t tp_attn_workspace_bytes(const tp_attn_desc* d, int32_t phase) {
  if (!d || d->batch < 0 || d->seq < 0 || d->hidden <= 0 || d->n_q <= 0) return 0;
  const int64_t T = d->batch * d->seq;
  if (phase == TP_MLP_BWD_NORM) return rmsnorm_bwd_workspace(T, d->hidden);
  if (phase != TP_MLP_BWD_SHARD) return 0;
  (void)T;
  return attn_ksplit_bytes(d) + attention_bwd_workspace(attn_args(d));
}

size_t tp_attention_backward_workspace_bytes(int64_t batch, int64_t seq, int32_t n_q, int32_t n_kv,
                                             int32_t head_dim) {
  if (batch < 0 || seq < 0 || n_q <= 0 || n_kv <= 0 || head_dim <= 0) return 0;
  AttnShapeArgs a{batch, seq, (int64_t)(n_q + 2 * n_kv) * head_dim, n_q, n_kv, head_dim};
  return attention_bwd_workspace(a);
}

size_t tp_attn_forward_workspace_bytes(const tp_attn_desc* d) {
  if (!d || d->batch < 0 || d->seq < 0 || d->hidden <= 0 || d->n_q <= 0 || d->n_kv <= 0 || d->head_dim <= 0) return 0;
  const int64_t T = d->batch * d->seq, W = (int64_t)(d->n_q + 2 * d->n_kv) * d->head_dim;
  return gemm_ksplit_workspace_bf16(T, W, d->hidden);
}

int tp_attn_forward(const tp_attn_desc* d, const void* x, const void* norm_w, const void* w_qkv, const void* w_o,
                    void* normed, float* rstd, void* qkv, void* attn_out, float* lse, void* out, const void* b_o,
                    void* workspace, size_t workspace_bytes, void* stream) {
  const char* fn = "tp_attn_forward";
  g_err[0] = 0;
  int rc = check_attn_desc(d, fn);
  if (rc) return rc;
  const int64_t T = d->batch * d->seq, H = d->hidden;
  const int64_t W = (int64_t)(d->n_q + 2 * d->n_kv) * d->head_dim, Wo = (int64_t)d->n_q * d->head_dim;
  const bool fuse = d->flags & TP_MLP_FUSE_EPILOGUE;
  REQUIRE_PTR(norm_w);
  REQUIRE_PTR(w_qkv);
  REQUIRE_PTR(w_o);
  if (fuse) REQUIRE_PTR(b_o);
  const size_t need = tp_attn_forward_workspace_bytes(d);
  if (workspace) {
    if (workspace_bytes < need)
      return fail(TP_MLP_EWORKSPACE, "%s: workspace of %zu bytes required, %zu given", fn, need, workspace_bytes);
    if (!aligned16(workspace)) return fail(TP_MLP_EALIGN, "%s: workspace is not 16-byte aligned", fn);
  }
  if (T == 0) return TP_MLP_OK;
  REQUIRE_PTR(x);
  REQUIRE_PTR(normed);
  REQUIRE_PTR4(rstd);
  REQUIRE_PTR(qkv);
  REQUIRE_PTR(attn_out);
  REQUIRE_PTR4(lse);
  REQUIRE_PTR(out);
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (!(d->flags & TP_MLP_NORMED_READY))
    CHECK_HIP(launch_rmsnorm_fwd(kBF16, x, norm_w, normed, rstd, T, H, d->eps, s), "rmsnorm forward");
  GemmArgs g{};
  g.M = T;
  g.N = W;
  g.K = H;
  g.A = normed;
  g.lda = H;
  g.B = w_qkv;
  g.ldb = H;
  g.C = qkv;
  g.ldc = W;
  if (workspace && need > 0) {  // k split over workgroups: the QKV product alone has few output tiles
    g.ksplit = gemm_ksplit(T, W, H);
    g.ws = static_cast<float*>(workspace);
  }
  g.tag = "gemm_qkv";
  CHECK_HIP(launch_gemm_bf16(true, true, kEpiStoreBf16, g, s), "QKV GEMM");
  const AttnShapeArgs a = attn_args(d);
  CHECK_HIP(launch_attention_fwd(a, qkv, attn_out, lse, s), "attention");
  GemmArgs c{};
  c.M = T;
  c.N = H;
  c.K = Wo;
  c.A = attn_out;
  c.lda = Wo;
  c.B = w_o;
  c.ldb = Wo;
  c.C = out;
  c.ldc = H;
  c.aux = x;
  c.bias = b_o;
  c.tag = fuse ? "gemm_out_proj_residual" : "gemm_out_proj_partial";
  CHECK_HIP(launch_gemm_bf16(true, true, fuse ? kEpiResidual : kEpiStoreF32, c, s), "output projection");
  return TP_MLP_OK;
}

int tp_attn_backward(const tp_attn_desc* d, int32_t phase, const tp_attn_bwd_args* a, void* stream) {
  const char* fn = "tp_attn_backward";
  g_err[0] = 0;
  int rc = check_attn_desc(d, fn);
  if (rc) return rc;
  if (!a) return fail(TP_MLP_EINVAL, "%s: args is NULL", fn);
  if (phase != TP_MLP_BWD_SHARD && phase != TP_MLP_BWD_NORM) return fail(TP_MLP_EINVAL, "%s: unknown phase", fn);
  const int64_t T = d->batch * d->seq, H = d->hidden;
  const int64_t W = (int64_t)(d->n_q + 2 * d->n_kv) * d->head_dim, Wo = (int64_t)d->n_q * d->head_dim;
  const bool accum = (d->flags & TP_MLP_ACCUMULATE_GRADS) != 0;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const size_t need = tp_attn_workspace_bytes(d, phase);
  if (need > 0) {
    if (!a->workspace || a->workspace_bytes < need)
      return fail(TP_MLP_EWORKSPACE, "%s: workspace of %zu bytes required, %zu given", fn, need,
                  a->workspace ? a->workspace_bytes : (size_t)0);
    if (!aligned16(a->workspace)) return fail(TP_MLP_EALIGN, "%s: workspace is not 16-byte aligned", fn);
  }
  if (phase == TP_MLP_BWD_NORM) {
    REQUIRE_PTR(a->norm_w);
    REQUIRE_PTR(a->d_norm_w);
    REQUIRE_PTR(a->d_b_o);
    const int np = a->n_d_normed_parts;
    if (np < 0 || np > kMaxNormParts)
      return fail(TP_MLP_EINVAL, "%s: n_d_normed_parts must be in [0, %d]", fn, kMaxNormParts);
    if (np > 0 && !a->d_normed_parts) return fail(TP_MLP_EINVAL, "%s: d_normed_parts is NULL", fn);
    const float* dn_one[1] = {a->d_normed};
    const float* const* parts = np > 0 ? a->d_normed_parts : dn_one;
    if (T > 0) {
      if (np > 0) {
        for (int k = 0; k < np; ++k) {
          const float* part = parts[k];
          REQUIRE_PTR(part);
        }
      } else {
        REQUIRE_PTR(a->d_normed);
      }
      REQUIRE_PTR(a->x);
      REQUIRE_PTR(a->d_out);
      REQUIRE_PTR4(a->rstd);
      REQUIRE_PTR(a->d_x);
    }
    CHECK_HIP(launch_rmsnorm_bwd(kBF16, parts, np > 0 ? np : 1, a->x, a->d_out, a->rstd, a->norm_w, a->d_x,
                                 a->d_norm_w, a->d_b_o, a->workspace, T, H, accum, s),
              "rmsnorm backward");
    return TP_MLP_OK;
  }
  REQUIRE_PTR(a->w_qkv);
  REQUIRE_PTR(a->w_o);
  REQUIRE_PTR(a->d_w_qkv);
  REQUIRE_PTR(a->d_w_o);
  if (T > 0) {
    REQUIRE_PTR(a->normed);
    REQUIRE_PTR(a->qkv);
    REQUIRE_PTR(a->attn_out);
    REQUIRE_PTR4(a->lse);
    REQUIRE_PTR(a->d_out);
    REQUIRE_PTR(a->d_attn_out);
    REQUIRE_PTR(a->d_qkv);
    REQUIRE_PTR(a->d_normed_part);
  }
  float* ksws = static_cast<float*>(a->workspace);
  void* attn_ws = static_cast<char*>(a->workspace) + attn_ksplit_bytes(d);

  // dO = d_out W_o ([T, H] x [H, n_q D])
  GemmArgs b1{};
  b1.M = T;
  b1.N = Wo;
  b1.K = H;
  b1.A = a->d_out;
  b1.lda = H;
  b1.B = a->w_o;
  b1.ldb = Wo;
  b1.C = a->d_attn_out;
  b1.ldc = Wo;
  b1.ksplit = gemm_ksplit(b1.M, b1.N, b1.K);
  b1.ws = ksws;
  b1.tag = "gemm_attn_dgrad_out";
  CHECK_HIP(launch_gemm_bf16(true, false, kEpiStoreBf16, b1, s), "dO GEMM");
  // d_w_o = d_out^T O ([H, T] x [T, n_q D])
  GemmArgs b2{};
  b2.M = H;
  b2.N = Wo;
  b2.K = T;
  b2.A = a->d_out;
  b2.lda = H;
  b2.B = a->attn_out;
  b2.ldb = Wo;
  b2.C = a->d_w_o;
  b2.ldc = Wo;
  b2.ksplit = gemm_ksplit(b2.M, b2.N, b2.K);
  b2.ws = ksws;
  b2.accum = accum;
  b2.tag = "gemm_attn_wgrad_out";
  CHECK_HIP(launch_gemm_bf16(false, false, kEpiStoreF32, b2, s), "d_w_o GEMM");
  CHECK_HIP(launch_attention_bwd(attn_args(d), a->qkv, a->attn_out, a->d_attn_out, a->lse, attn_ws, a->d_qkv, s),
            "attention backward");
  // d_w_qkv = d_qkv^T N ([W, T] x [T, H])
  GemmArgs b4{};
  b4.M = W;
  b4.N = H;
  b4.K = T;
  b4.A = a->d_qkv;
  b4.lda = W;
  b4.B = a->normed;
  b4.ldb = H;
  b4.C = a->d_w_qkv;
  b4.ldc = H;
  b4.ksplit = gemm_ksplit(b4.M, b4.N, b4.K);
  b4.ws = ksws;
  b4.accum = accum;
  b4.tag = "gemm_attn_wgrad_qkv";
  CHECK_HIP(launch_gemm_bf16(false, false, kEpiStoreF32, b4, s), "d_w_qkv GEMM");
  // d_normed partial = d_qkv W_qkv ([T, W] x [W, H]); last, as in the MLP backward
  GemmArgs b3{};
  b3.M = T;
  b3.N = H;
  b3.K = W;
  b3.A = a->d_qkv;
  b3.lda = W;
  b3.B = a->w_qkv;
  b3.ldb = H;
  b3.C = a->d_normed_part;
  b3.ldc = H;
  b3.tag = "gemm_attn_dgrad_normed";
  CHECK_HIP(launch_gemm_bf16(true, false, kEpiStoreF32, b3, s), "d_normed GEMM");
  return TP_MLP_OK;
}

int tp_attention_forward(int64_t batch, int64_t seq, int32_t n_q, int32_t n_kv, int32_t head_dim, const void* qkv,
                         int64_t ld, void* o, float* lse, void* stream) {
  const char* fn = "tp_attention_forward";
  g_err[0] = 0;
  int rc = check_attn_shape(batch, seq, n_q, n_kv, head_dim, fn);
  if (rc) return rc;
  if (ld < (int64_t)(n_q + 2 * n_kv) * head_dim || ld % 8) return fail(TP_MLP_ESHAPE, "%s: bad ld", fn);
  if (seq * ld >= ((int64_t)1 << 30)) return fail(TP_MLP_ESHAPE, "%s: one sequence holds 2^30 or more elements", fn);
  const int64_t T = batch * seq;
  if (T * ld >= ((int64_t)1 << 31) || T * n_q * head_dim >= ((int64_t)1 << 31))
    return fail(TP_MLP_ESHAPE, "%s: 2^31 or more elements", fn);
  if (T == 0) return TP_MLP_OK;
  REQUIRE_PTR(qkv);
  REQUIRE_PTR(o);
  REQUIRE_PTR4(lse);
  AttnShapeArgs a{batch, seq, ld, n_q, n_kv, head_dim};
  CHECK_HIP(launch_attention_fwd(a, qkv, o, lse, static_cast<hipStream_t>(stream)), "attention");
  return TP_MLP_OK;
}

int tp_attention_backward(int64_t batch, int64_t seq, int32_t n_q, int32_t n_kv, int32_t head_dim, const void* qkv,
                          int64_t ld, const void* o, const void* d_o, const float* lse, void* workspace,
                          size_t workspace_bytes, void* d_qkv, void* stream) {
  const char* fn = "tp_attention_backward";
  g_err[0] = 0;
  int rc = check_attn_shape(batch, seq, n_q, n_kv, head_dim, fn);
  if (rc) return rc;
  if (ld < (int64_t)(n_q + 2 * n_kv) * head_dim || ld % 8) return fail(TP_MLP_ESHAPE, "%s: bad ld", fn);
  if (seq * ld >= ((int64_t)1 << 30)) return fail(TP_MLP_ESHAPE, "%s: one sequence holds 2^30 or more elements", fn);
  const int64_t T = batch * seq;
  if (T * ld >= ((int64_t)1 << 31) || T * n_q * head_dim >= ((int64_t)1 << 31))
    return fail(TP_MLP_ESHAPE, "%s: 2^31 or more elements", fn);
  if (T == 0) return TP_MLP_OK;
  REQUIRE_PTR(qkv);
  REQUIRE_PTR(o);
  REQUIRE_PTR(d_o);
  REQUIRE_PTR4(lse);
  REQUIRE_PTR(d_qkv);
  AttnShapeArgs a{batch, seq, ld, n_q, n_kv, head_dim};
  const size_t need = attention_bwd_workspace(a);
  if (!workspace || workspace_bytes < need)
    return fail(TP_MLP_EWORKSPACE, "%s: workspace of %zu bytes required, %zu given", fn, need,
                workspace ? workspace_bytes : (size_t)0);
  if (!aligned16(workspace)) return fail(TP_MLP_EALIGN, "%s: workspace is not 16-byte aligned", fn);
  CHECK_HIP(launch_attention_bwd(a, qkv, o, d_o, lse, workspace, d_qkv, static_cast<hipStream_t>(stream)),
            "attention backward");
  return TP_MLP_OK;
}

}  // extern "C"
