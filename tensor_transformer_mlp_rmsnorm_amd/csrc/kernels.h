// Host-side launchers of the libtpmlp kernels.  Argument checking happens in
// api.hip before any of these is called; the launchers assume valid shapes.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace tpmlp {

enum DType { kF32 = 0, kBF16 = 1 };

// Brackets one kernel launch with HIP events on its stream while kernel
// timing is switched on (tp_mlp_profile_enable); a no-op otherwise.
class KernelTimer {
 public:
  KernelTimer(const char* name, hipStream_t s);
  ~KernelTimer();
  KernelTimer(const KernelTimer&) = delete;
  KernelTimer& operator=(const KernelTimer&) = delete;

 private:
  const char* name_;
  hipStream_t stream_;
  hipEvent_t start_ = nullptr, stop_ = nullptr;
  bool active_ = false;
};

// Epilogues of the MFMA GEMM.
enum Epi {
  kEpiStoreF32 = 0,   // C fp32
  kEpiSwigluFwd = 1,  // pre = [g | u] (T), act = SiLU(g) * u (T); B tile pairs gate/up channels
  kEpiGeluFwd = 2,    // h = acc + b_in (T), act = gelu(h) (T)
  kEpiResidual = 3,   // out = acc + x + b_down (T)
  kEpiSwigluBwd = 4,  // d_pre = [dg | du] from d_act = acc and saved [g | u]
  kEpiGeluBwd = 5,    // dh = d_act * gelu'(h)
  kEpiStoreBf16 = 6,  // C bf16 [M, ldc]
  kEpiSgd = 7,        // the product is the gradient of a bf16 weight [M, N]: SGD update applied (GemmArgs.sgd)
  kEpiSgdT = 8,       // the product is the gradient of W^T for a bf16 weight W [N, M]: the same update
  kEpiSwigluBwdT = 9, // kEpiSwigluBwd, and d_pre also written transposed to pre_t
  kEpiGeluBwdT = 10,  // kEpiGeluBwd, and d_pre also written transposed to pre_t
};

// kEpiSgd: where the update of a weight W [M, N] (bf16, row-major) goes.  The
// product C = dW is never stored; W_out = round(W_in - lr C), or with fp32
// masters M_out = M_in - lr C and W_out = round(M_out); W_out_t (optional)
// receives the same values transposed, [N, M].  Outputs may equal inputs.
// kEpiSgdT: the product is dW^T [M, N] of a weight W [N, M]; the old values
// are read from w_in_t (W^T), W^T goes to w_out_t and W to w_out (either may
// be null); no masters.
struct SgdEpi {
  const void* w_in;
  const void* w_in_t;
  void* w_out;
  void* w_out_t;
  const float* m_in;
  float* m_out;
  float lr;
};

// Operand layouts: A is [M, K] when a_kcontig, else [K, M]; B is [N, K] when
// b_kcontig, else [K, N].  Leading dimensions are in elements.
struct GemmArgs {
  int64_t M, N, K;
  const void* A;
  int64_t lda;
  const void* B;
  int64_t ldb;
  // epilogue operands (meaning per Epi)
  void* C;        // kEpiStoreF32: fp32 C [M, ldc]; kEpiResidual: out [M, ldc]
  int64_t ldc;
  void* pre;      // SwiGLU/GeLU fwd: pre-activations out; bwd: d_pre out
  void* act;      // fwd: activation out
  const void* aux;   // SwiGLU/GeLU bwd: saved pre-activations; residual: x
  const void* bias;  // GeLU fwd: b_in [N]; residual: b_down [N]
  int64_t ffn;       // F (column offset of the up half in [T, 2F] tensors)
  const char* tag;   // kernel name for timing
  // kEpiStoreF32: split the k range over `ksplit` workgroups per tile;
  // slice 0 writes C, slice s > 0 writes ws + (s - 1) * M * ldc, and a second
  // kernel adds the slices to C in index order.  kEpiStoreBf16: every slice s
  // writes fp32 to ws + s * M * N (row length N) and the second kernel writes
  // their sum, in index order, to C as bf16.  ksplit = 1 ignores ws.
  int ksplit;
  float* ws;
  // kEpiStoreF32 only: add C's current values to the product (slice 0 reads
  // and adds them; with a k split the other slices are then added as usual).
  int accum;
  // FP8 operands: device pointers to the inverse scales of A and B; the
  // product is multiplied by scale_inv_a[0] * scale_inv_b[0] before the epilogue.
  const float* scale_inv_a;
  const float* scale_inv_b;
  // kEpiSgd only (with a k split, every slice goes to ws and a second kernel
  // sums them in index order and applies the update)
  SgdEpi sgd;
  // kEpiSwigluBwdT / kEpiGeluBwdT: d_pre transposed, [2F | F rows][ld_t] (M a
  // multiple of 8); the up half's rows follow the gate half's
  void* pre_t;
  int64_t ld_t;
  // bf16 GEMMs: tile rows per group in the order workgroups take tiles (0: 4).
  // Each XCD takes a contiguous run of tiles, row by row inside groups of
  // this many tile rows, which sets how many operand strips one round of an
  // XCD's workgroups shares; the best value depends on the shape (measured).
  int tile_group;
};

// Number of k-slices for a bf16 fp32-output GEMM: a function of the shape only
// (so results are bitwise reproducible).  Shapes with fewer than 192 tiles of
// 256 x 256 take the most slices (at most 8) that keep all workgroups in one
// round of 256 CUs and every slice at least 1024 of k.
inline int gemm_ksplit(int64_t M, int64_t N, int64_t K) {
  const int64_t tiles = ((M + 255) / 256) * ((N + 255) / 256);
  if (tiles >= 192) return 1;
  int ks = 1;
  while (ks < 8 && tiles * (ks + 1) <= 256 && K / (ks + 1) >= 1024) ++ks;
  return ks;
}
inline size_t gemm_ksplit_workspace(int64_t M, int64_t N, int64_t K) {
  return (size_t)(gemm_ksplit(M, N, K) - 1) * (size_t)(M * N) * sizeof(float);
}
// The same for a weight-gradient GEMM with the SGD update applied (kEpiSgd:
// every slice in the workspace).
inline size_t gemm_ksplit_workspace_sgd(int64_t M, int64_t N, int64_t K) {
  const int ks = gemm_ksplit(M, N, K);
  return ks > 1 ? (size_t)ks * (size_t)(M * N) * sizeof(float) : 0;
}
// The same for a bf16-output GEMM (every slice in the workspace).
inline size_t gemm_ksplit_workspace_bf16(int64_t M, int64_t N, int64_t K) {
  const int ks = gemm_ksplit(M, N, K);
  return ks > 1 ? (size_t)ks * (size_t)(M * N) * sizeof(float) : 0;
}

hipError_t launch_gemm(DType dt, bool a_kcontig, bool b_kcontig, Epi epi, const GemmArgs& g,
                       hipStream_t s);
// The bf16 kernel (256 x 256 tiles); launch_gemm routes bf16 here.
hipError_t launch_gemm_bf16(bool a_kcontig, bool b_kcontig, Epi epi, const GemmArgs& g, hipStream_t s);

// FP8 formats (the MFMA's numbering).
enum Fp8Fmt { kFp8E4M3 = 0, kFp8E5M2 = 1 };

// FP8 GEMM, both operands K-contiguous codes ([M, K] and [N, K], K a multiple
// of 16): (fmt_a, fmt_b) = (E4M3, E4M3) with the forward epilogues or
// kEpiStoreF32, (E5M2, E4M3) with the activation-backward epilogues or
// kEpiStoreF32.  Needs g.scale_inv_a / g.scale_inv_b.
hipError_t launch_gemm_fp8(int fmt_a, int fmt_b, Epi epi, const GemmArgs& g, hipStream_t s);

// FP8 casts with delayed scaling (meta layout in fp8.hip).  x is bf16
// [R, C] (C a multiple of 8); out [R, C] and/or out_t [C, ldt] (ldt >= R, a
// multiple of 16; columns R .. ldt-1 written as zero); either may be null.
constexpr int kFp8MaxMetas = 16;
constexpr int kFp8MaxHistory = 1024;
hipError_t launch_fp8_cast(int fmt, const void* x, int64_t R, int64_t C, uint8_t* out, uint8_t* out_t, int64_t ldt,
                           float* meta, const char* tag, hipStream_t s);
hipError_t launch_fp8_update(float* const* metas, int count, int history_len, hipStream_t s);
hipError_t launch_fp8_meta_init(float* meta, int fmt, int history_len, hipStream_t s);

// Causal grouped-query attention on a [T, ld] QKV tensor (attention.hip).
struct AttnShapeArgs {
  int64_t batch, seq;  // T = batch * seq rows, a sequence's rows contiguous
  int64_t ld;          // row length of qkv and dqkv (elements)
  int n_q, n_kv, head_dim;
};
// O [T, n_q D] bf16, lse [n_q, T] fp32.
hipError_t launch_attention_fwd(const AttnShapeArgs& a, const void* qkv, void* O, float* lse, hipStream_t s);
// dqkv [T, ld] bf16 (every Q, K and V column written).  workspace (16-byte
// aligned, attention_bwd_workspace bytes): delta [n_q, T] fp32, padded to 256
// bytes, then (n_q > n_kv only) the per-head dK/dV shares [group][T][n_kv][2 D] fp32.
size_t attention_delta_bytes(const AttnShapeArgs& a);
size_t attention_bwd_workspace(const AttnShapeArgs& a);
hipError_t launch_attention_bwd(const AttnShapeArgs& a, const void* qkv, const void* O, const void* dO,
                                const float* lse, void* workspace, void* dqkv, hipStream_t s);

hipError_t launch_rmsnorm_fwd(DType dt, const void* x, const void* w, void* n, float* rstd,
                              int64_t T, int64_t H, float eps, hipStream_t s);

// RMSNorm backward + residual: dx, and per-block column partials of
// d_norm_w and d_b_down in `ws` followed by the fixed-order reduction.  The
// gradient of N is the sum, in index order, of the n_parts (1 .. 64) [T, H]
// fp32 arrays dN_parts (a host array of device pointers).
constexpr int kMaxNormParts = 64;
size_t rmsnorm_bwd_workspace(int64_t T, int64_t H);
// With `accum`, dw and db receive their current values plus the column sums.
hipError_t launch_rmsnorm_bwd(DType dt, const float* const* dN_parts, int n_parts, const void* x, const void* dY,
                              const float* rstd, const void* w, void* dx, float* dw, float* db,
                              void* ws, int64_t T, int64_t H, bool accum, hipStream_t s);

// Column sums of a [rows, cols] matrix in dtype dt into fp32 out[cols], in a
// fixed order (two stages through `ws`); with `accum` added to out's values.
size_t colsum_workspace(int64_t rows, int64_t cols);
hipError_t launch_colsum(DType dt, const void* in, float* out, void* ws, int64_t rows, int64_t cols, bool accum,
                         hipStream_t s);
// out[c] = (accum ? out[c] : 0) + sum_{b=0}^{nparts-1} ws[b][c], in a fixed order.
hipError_t launch_reduce_partial_rows(const float* ws, float* out, int64_t nparts, int64_t cols, bool accum,
                                      hipStream_t s);

hipError_t launch_partial_sum(const float* const* parts, int n_parts, int64_t rows, int64_t cols,
                              const void* residual, const void* bias, DType in_dt, void* out,
                              DType out_dt, hipStream_t s);

// C[m, n] = ((C[m, n] + ws[0][m, n]) + ws[1][m, n]) + ... over `nslices`
// [M, ldc] fp32 slices (the k-slices of a split GEMM, added in index order).
hipError_t launch_ksplit_reduce_bf16(void* C, const float* ws, int nslices, int64_t M, int64_t N, int64_t ldc,
                                     hipStream_t s);
hipError_t launch_ksplit_reduce(float* C, const float* ws, int nslices, int64_t M, int64_t N, int64_t ldc,
                                hipStream_t s);

// out [C, R] = in [R, C]^T, bf16, row-major; R and C multiples of 8.
hipError_t launch_transpose_bf16(const void* in, void* out, int64_t R, int64_t C, hipStream_t s);

struct SgdTensor {
  const void* param_in;
  void* param_out;
  const float* grad;
  const float* master_in;
  float* master_out;
  int64_t n;
  // optional (bf16): the updated values of the [t_rows, t_cols] parameter
  // also written transposed, [t_cols, t_rows], to param_out_t
  void* param_out_t;
  int64_t t_rows, t_cols;
};
// One SGD update of every tensor in `list` (all in dtype dt; all with fp32
// masters when `master`).
hipError_t launch_sgd(DType dt, const SgdTensor* list, int count, bool master, float lr, hipStream_t s);
// The SGD update of one bf16 weight [M, N] whose gradient is the sum, in
// index order, of `nslices` [M, N] fp32 slices at ws (a split GEMM's
// k-slices), with the optional transposed copy: the arithmetic of launch_sgd.
hipError_t launch_sgd_ksplit(const SgdEpi& u, const float* ws, int nslices, int64_t M, int64_t N, hipStream_t s);

struct AdamwTensor {
  const void* param_in;
  void* param_out;
  const float* grad;
  const float* master_in;
  float* master_out;
  float* m;
  float* v;
  int64_t n;
};
struct AdamwConst {
  float lr, beta1, beta2, eps, weight_decay;
  float bc1, bc2;  // 1 - beta1^step, 1 - beta2^step (formed in double on the host)
};
// One AdamW update of every tensor in `list` (dtype dt; fp32 masters when
// `master`); `scale` is a device pointer to the gradient factor, or null.
hipError_t launch_adamw(DType dt, const AdamwTensor* list, int count, bool master, const AdamwConst& c,
                        const float* scale, hipStream_t s);

// Global gradient norm: per-2048-element-block fp64 sums of squares into ws,
// then one workgroup adds them in order and writes norm and the clip factor.
size_t sumsq_blocks(const int64_t* counts, int count);
hipError_t launch_clip_grad_norm(const float* const* grads, const int64_t* counts, int count, float max_norm,
                                 float* norm_out, float* coef_out, double* ws, hipStream_t s);

}  // namespace tpmlp
