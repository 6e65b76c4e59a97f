/*
 * tp_mlp.h - C ABI of one tensor-parallel rank's share of the pre-RMSNorm
 * MLP sublayer (forward, backward, SGD or AdamW) on an AMD Instinct MI355X (gfx950).
 *
 * The block is the one rebuilt in "Megatron tensor-parallel MLP"
 * (synapticradio.com), section "Start with the dense block":
 *     N   = rms_norm(x, norm_w)
 *     A   = SiLU(N Wg^T) * (N Wu^T)          (gate/up stacked as w_in[2, F, H])
 *     out = x + A Wd^T + b_down              (Wd = w_down[H, F])
 * and its GeLU variant from "Megatron-LM walkthrough", Part II:
 *     A   = gelu(N W1^T + b1)                (w_in[F, H], b_in[F])
 * A rank owns F = F_full / S channels of the FFN axis ("Split the expansion",
 * "Split the contraction").  Its down projection yields a full-width
 * partial; the partials are summed (the forward all-reduce), then residual
 * and bias are added once.  In backward each rank's gradient of the
 * replicated N is a partial that is summed (the backward all-reduce) before
 * RMSNorm's backward ("Put the other collective in backward").  In this
 * library both sums are tp_partial_sum, an on-device reduction over shard
 * partials computed one after the other on the same GPU, never a collective.
 *
 * Conventions for every call
 *   - All tensor arguments are DEVICE pointers, row-major and contiguous,
 *     16-byte aligned (rstd: 4-byte aligned), owned by the caller.  The library allocates no device
 *     memory and keeps no device state between calls.
 *   - `stream` is a hipStream_t (NULL = the null stream).  Calls only
 *     enqueue work on it and return; synchronisation is the caller's.
 *   - Shapes: T = tokens (any value >= 0), H = hidden, F = ffn_local.  H and
 *     F must be positive multiples of 8; H <= 16384.  T = 0 is a no-op.
 *     Every [T,H], [T,2F] and [2F,H] tensor must hold fewer than 2^30
 *     elements for bf16 (each GEMM operand is addressed through a buffer
 *     descriptor limited to 2 GiB) and fewer than 2^31 for fp32.
 *   - dtype TP_MLP_F32: every tensor fp32.  dtype TP_MLP_BF16: parameters and
 *     activations bf16 (round to nearest even), accumulation fp32; partial
 *     sums, rstd and every parameter gradient are fp32 in both cases.
 *   - Return 0 on success or a negative TP_MLP_E* code; tp_mlp_last_error()
 *     then describes the failure.  Argument errors are detected before any
 *     work is enqueued.  No exception crosses the ABI.
 */
#ifndef TP_MLP_H
#define TP_MLP_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
  TP_MLP_OK = 0,
  TP_MLP_EINVAL = -1,     /* null pointer, negative size, bad enum */
  TP_MLP_ESHAPE = -2,     /* H or F not a positive multiple of 8, H too large,
                             F_full not divisible by the shard count */
  TP_MLP_EDTYPE = -3,     /* unknown dtype / dtype combination */
  TP_MLP_EALIGN = -4,     /* a pointer is not 16-byte aligned */
  TP_MLP_EWORKSPACE = -5, /* workspace missing or smaller than required */
  TP_MLP_EHIP = -6        /* the HIP runtime reported an error on launch */
};

enum { TP_MLP_ACT_SWIGLU = 0, TP_MLP_ACT_GELU = 1 };
enum { TP_MLP_F32 = 0, TP_MLP_BF16 = 1 };

/* tp_mlp_desc.flags */
enum {
  /* Forward: write out = x + z + b_down (act dtype) directly from the down
   * projection instead of the fp32 partial z.  Only valid for an unsharded
   * block (S = 1), where the partial sum has a single term. */
  TP_MLP_FUSE_EPILOGUE = 1,
  /* Forward: `normed` and `rstd` already hold rms_norm(x) from an earlier call
   * with the same x and norm_w (the replicated input of another shard), so
   * the norm is not recomputed. */
  TP_MLP_NORMED_READY = 2,
  /* Backward (both phases): add this call's parameter gradients (d_w_in,
   * d_b_in, d_w_down, d_norm_w, d_b_down) to what those buffers hold instead
   * of overwriting them: gradient accumulation over the microbatches of a
   * global batch ("Megatron-LM walkthrough", Part IV, Stage 4: a global batch
   * is split into microbatches, each run forward and backward, before the
   * optimiser step).  Activation gradients are always overwritten. */
  TP_MLP_ACCUMULATE_GRADS = 4
};

typedef struct {
  int64_t tokens;    /* T */
  int64_t hidden;    /* H */
  int64_t ffn_local; /* F: channels of the FFN axis owned by this shard */
  int32_t act;       /* TP_MLP_ACT_* */
  int32_t dtype;     /* TP_MLP_F32 | TP_MLP_BF16 */
  float eps;         /* RMSNorm epsilon, added to mean(x^2) under the root */
  int32_t flags;     /* TP_MLP_FUSE_EPILOGUE | TP_MLP_NORMED_READY | TP_MLP_ACCUMULATE_GRADS
                        (| TP_MLP_FP8_SHARED_READY for tp_mlp_backward_fp8) */
} tp_mlp_desc;

/*
 * tp_mlp_forward - one shard's forward: RMSNorm, column-parallel expansion
 * with its activation, row-parallel down projection.
 *   ("Start with the dense block"; "Split the expansion"; "Split the
 *    contraction", synapticradio.com)
 *
 *   x        [T, H]    dtype   block input; also the residual
 *   norm_w   [H]       dtype   RMSNorm weight (replicated)
 *   w_in     SwiGLU [2, F, H] (plane 0 gate, plane 1 up) | GeLU [F, H], dtype
 *   b_in     GeLU: [F] dtype fc1 bias; SwiGLU: must be NULL
 *   w_down   [H, F]    dtype   this shard's columns of the down weight
 *   normed   [T, H]    dtype   out: N = x * rstd * norm_w (in, with NORMED_READY)
 *   rstd     [T]       fp32    out: 1 / sqrt(mean_H(x^2) + eps) (in, with NORMED_READY)
 *   pre_act  SwiGLU [T, 2F] (cols [0,F) gate, [F,2F) up) | GeLU [T, F], dtype
 *                              out: pre-activations, saved for backward
 *   act      [T, F]    dtype   out: SiLU(g) * u  |  gelu(h), saved for backward
 *   out      without FUSE_EPILOGUE: [T, H] fp32, this shard's partial z = A Wd^T
 *            with FUSE_EPILOGUE:    [T, H] dtype, x + z + b_down
 *   b_down   [H] dtype; read only with FUSE_EPILOGUE (else may be NULL)
 */
int tp_mlp_forward(const tp_mlp_desc* d, const void* x, const void* norm_w, const void* w_in,
                   const void* b_in, const void* w_down, void* normed, float* rstd,
                   void* pre_act, void* act, void* out, const void* b_down, void* stream);

/*
 * tp_mlp_forward_ws - tp_mlp_forward with a caller-owned workspace, which
 * lets the down projection split its k range (F) over several workgroups per
 * output tile when the GEMM has few tiles (bf16; a function of the shape
 * only, so results are run-to-run identical): the slices are summed in index
 * order in fp32, and with TP_MLP_FUSE_EPILOGUE the residual and bias are then
 * added by tp_partial_sum's kernel (out = x + z + b_down).  The results equal
 * tp_mlp_forward's up to the order of the fp32 additions.
 *   workspace        device, 16-byte aligned, >= tp_mlp_forward_workspace_bytes(d)
 *                    bytes (NULL allowed when that is 0)
 * Errors: as tp_mlp_forward, and TP_MLP_EWORKSPACE when the workspace is
 * smaller than needed (checked before any launch).
 */
size_t tp_mlp_forward_workspace_bytes(const tp_mlp_desc* d);
int tp_mlp_forward_ws(const tp_mlp_desc* d, const void* x, const void* norm_w, const void* w_in,
                      const void* b_in, const void* w_down, void* normed, float* rstd,
                      void* pre_act, void* act, void* out, const void* b_down,
                      void* workspace, size_t workspace_bytes, void* stream);

/*
 * tp_rmsnorm_forward - the RMSNorm of tp_mlp_forward on its own, for a
 * sequence-parallel rank's slice of the token rows ("Megatron-LM
 * walkthrough", Part V, "Deep dive: sequence parallelism": the norm runs on
 * each rank's slice of the sequence; the slices are then gathered into the
 * full normed input of the tensor-parallel region, which tp_mlp_forward takes
 * with TP_MLP_NORMED_READY).
 *   rstd_t = 1 / sqrt(mean_i x[t,i]^2 + eps),   normed[t,i] = x[t,i] rstd_t w[i]
 *   x [rows, hidden] dtype; w [hidden] dtype; normed [rows, hidden] dtype;
 *   rstd [rows] fp32.  hidden: positive multiple of 8, <= 16384; rows >= 0
 *   (0 is a no-op).  dtype TP_MLP_F32 | TP_MLP_BF16.
 */
int tp_rmsnorm_forward(int64_t rows, int64_t hidden, int32_t dtype, float eps, const void* x, const void* w,
                       void* normed, float* rstd, void* stream);

/*
 * tp_partial_sum - the sum that stands in for the all-reduce at the two
 * tensor-parallel boundaries ("Split the contraction": partial outputs summed,
 * then residual and bias added once; "Put the other collective in backward":
 * the shards' gradients of N summed before RMSNorm's backward).
 *
 *   out[r, c] = ((parts[0][r,c] + parts[1][r,c]) + ...) + residual[r,c] + bias[c]
 *
 *   parts     HOST array of n_parts DEVICE pointers, each [rows, cols] fp32;
 *             summed in index order with fp32 accumulation (deterministic).
 *             1 <= n_parts <= 64.  No part is written.
 *   residual  [rows, cols] in `in_dtype`, or NULL
 *   bias      [cols] in `in_dtype`, or NULL
 *   out       [rows, cols] in `out_dtype` (TP_MLP_F32 or TP_MLP_BF16); may
 *             not alias a part.
 *   cols must be a multiple of 4.
 */
int tp_partial_sum(const float* const* parts, int32_t n_parts, int64_t rows, int64_t cols,
                   const void* residual, const void* bias, int32_t in_dtype, void* out,
                   int32_t out_dtype, void* stream);

/* Backward phases (see tp_mlp_backward). */
enum { TP_MLP_BWD_SHARD = 0, TP_MLP_BWD_NORM = 1 };

/*
 * The SGD update of a shard's two weight matrices taken inside the SHARD
 * phase ("Reproduce one dense training step": one SGD update of every
 * parameter; in a tensor-parallel rank the sharded weights' gradients need no
 * reduction, so the update can follow their weight-gradient GEMMs at once).
 * bf16 only.  Each GEMM's fp32 product dW is applied where it is formed and
 * never written:
 *   master == NULL:  W_out = round_bf16(W - lr dW)           (fp32 arithmetic)
 *   master != NULL:  M_out = M - lr dW (fp32),  W_out = round_bf16(M_out)
 * the bits tp_mlp_sgd_step_multi gives from the gradient the unfused phase
 * would have written.  W_t_out (optional) receives the same values transposed
 * (w_in: [H, 2F] | [H, F]; w_down: [F, H]), the copies tp_mlp_backward takes
 * as w_in_t / w_down_t.
 *   w_in_out       [2,F,H] | [F,H] bf16; may equal w_in (in place)
 *   w_in_t_out     NULL or [H, 2F] | [H, F] bf16; may equal w_in_t
 *   w_in_master    NULL or [2F|F, H] fp32, read; w_in_master_out then
 *                  required, may equal it
 *   w_down_*       the same for w_down [H, F] (transposed copy [F, H])
 * Outputs must not partially overlap any tensor the phase reads.  When
 * w_in_out equals w_in or w_in_t_out equals w_in_t, the phase forms its
 * d_normed partial (which reads w_in) before it updates w_in.
 */
typedef struct {
  float lr;
  void* w_in_out;
  void* w_in_t_out;
  const float* w_in_master;
  float* w_in_master_out;
  void* w_down_out;
  void* w_down_t_out;
  const float* w_down_master;
  float* w_down_master_out;
} tp_mlp_fused_sgd;

typedef struct {
  /* saved from tp_mlp_forward */
  const void* x;          /* [T, H]  dtype */
  const void* normed;     /* [T, H]  dtype */
  const float* rstd;      /* [T]     fp32  */
  const void* pre_act;    /* [T, 2F] | [T, F] dtype */
  const void* act;        /* [T, F]  dtype */
  /* parameters */
  const void* norm_w;     /* [H] dtype */
  const void* w_in;       /* [2, F, H] | [F, H] dtype */
  const void* w_down;     /* [H, F] dtype */
  /* upstream gradient of the block output, [T, H] dtype (with the page's
     loss sum(out^2)/2 this is out itself) */
  const void* d_out;
  /* SHARD phase outputs */
  void* d_pre;            /* [T, 2F] | [T, F] dtype: gradient of the pre-activations */
  float* d_w_in;          /* [2, F, H] | [F, H] fp32 */
  float* d_b_in;          /* GeLU: [F] fp32; SwiGLU: NULL */
  float* d_w_down;        /* [H, F] fp32 */
  float* d_normed_part;   /* [T, H] fp32: this shard's partial of dL/dN */
  /* NORM phase input and outputs */
  const float* d_normed;  /* [T, H] fp32: dL/dN summed over shards */
  void* d_x;              /* [T, H] dtype */
  float* d_norm_w;        /* [H] fp32 */
  float* d_b_down;        /* [H] fp32 */
  /* scratch, caller-owned: k-split slices and column partials of the
     deterministic reductions; in bf16 also Wd transposed ([F, H]) for the
     d_act GEMM */
  void* workspace;
  size_t workspace_bytes;
  /* NORM phase, instead of d_normed: the shards' partials of dL/dN
     (d_normed_part of each SHARD call), summed by the RMSNorm backward as it
     reads them -- in index order with fp32 additions, the sum tp_partial_sum
     forms, so the results are the same bits -- rather than summed into
     d_normed first and read back.  A HOST array of n_d_normed_parts DEVICE
     pointers, each [T, H] fp32, 1 <= n_d_normed_parts <= 64.
     n_d_normed_parts = 0 (as in zero-initialised args): d_normed is read. */
  const float* const* d_normed_parts;
  int32_t n_d_normed_parts;
  /* SHARD phase, optional (bf16): w_down transposed, [F, H], as
     tp_mlp_transpose_bf16 or the SGD's transposed copy write it.  Given, the
     d_act GEMM reads it; NULL, the phase transposes w_down into the
     workspace first.  It must hold the transpose of this w_down. */
  const void* w_down_t;
  /* SHARD phase, optional (bf16): w_in transposed, [H, 2F] | [H, F] (w_in read
     as a [2F, H] | [F, H] matrix), as tp_mlp_transpose_bf16 or the SGD's
     transposed copy write it.  Given, the d_normed GEMM reads both operands
     K-contiguous; NULL, it reads w_in as it lies.  It must hold the transpose
     of this w_in. */
  const void* w_in_t;
  /* SHARD phase, optional (bf16): the SGD update of w_in and w_down taken in
     their weight-gradient GEMMs (see tp_mlp_fused_sgd).  Given, d_w_in and
     d_w_down are not written (they may be NULL) and TP_MLP_ACCUMULATE_GRADS
     is an error; GeLU's d_b_in is still written.  NULL: the gradients are
     written and the update is the caller's (tp_mlp_sgd_step_multi). */
  const tp_mlp_fused_sgd* fused_sgd;
  /* SHARD phase, optional (bf16, T a multiple of 8): the activations of the
     w_in weight-gradient GEMM in the layout that makes its k (the tokens)
     contiguous in both operands.
       d_pre_t   [2F | F, T] written: the transpose of d_pre (written with it;
                 needs w_down_t).
       normed_t  [H, T] read: the transpose of normed (tp_mlp_transpose_bf16).
     When both are given with fused_sgd (no w_in masters), w_in_t and a
     w_in weight-gradient GEMM whose k is not split, that GEMM forms dW_in^T
     = normed_t d_pre_t^T and the update writes w_in_t_out from it directly
     and w_in_out transposed: the same values.  Otherwise they change nothing
     but the extra write of d_pre_t. */
  const void* normed_t;
  void* d_pre_t;
} tp_mlp_bwd_args;

/*
 * tp_mlp_backward - the backward of tp_mlp_forward, in two phases split at
 * the backward all-reduce ("Put the other collective in backward": the sum of
 * the shards' dN must happen before RMSNorm's backward).
 *
 * phase TP_MLP_BWD_SHARD (per shard, before the sum):
 *   d_act        = d_out Wd                         (the forward sum's backward is the identity)
 *   d_pre        = SwiGLU: dg = d_act * u * s(g) (1 + g (1 - s(g))), du = d_act * SiLU(g)
 *                  GeLU:   dh = d_act * gelu'(h)
 *   d_w_down     = d_out^T act
 *   d_w_in       = d_pre^T normed          (fp32, [2F, H] rows gate then up | [F, H])
 *   d_b_in       = sum_t dh                (GeLU only)
 *   d_normed_part= d_pre w_in              (fp32 partial, summed by tp_partial_sum)
 *   This phase reads normed, pre_act, act, w_in, w_down and d_out.  With
 *   a->fused_sgd, d_w_down and d_w_in are applied to the weights as they are
 *   formed instead of being written.
 * phase TP_MLP_BWD_NORM (once, after the sum, or with the sum streamed in
 * through d_normed_parts):
 *   c_t      = (1/H) sum_i d_normed[t,i] norm_w[i] x[t,i]
 *   d_x      = d_out + rstd d_normed norm_w - x rstd^3 c        (residual + RMSNorm)
 *   d_norm_w = sum_t d_normed x rstd,   d_b_down = sum_t d_out
 * Column sums are reduced in a fixed order (run-to-run deterministic).
 * With TP_MLP_ACCUMULATE_GRADS in d->flags, d_w_in, d_b_in, d_w_down,
 * d_norm_w and d_b_down receive buffer + gradient instead of the gradient.
 * Workspace: at least tp_mlp_workspace_bytes(d, phase) bytes.
 */
int tp_mlp_backward(const tp_mlp_desc* d, int32_t phase, const tp_mlp_bwd_args* a, void* stream);

/* Bytes of workspace tp_mlp_backward needs for this descriptor and phase. */
size_t tp_mlp_workspace_bytes(const tp_mlp_desc* d, int32_t phase);

/*
 * tp_mlp_backward_noalloc - tp_mlp_backward for callers that cannot allocate
 * device memory (code being captured into a HIP graph, tight serving loops,
 * harnesses that forbid allocation): the same phases, arguments, checks,
 * kernels and results, but a->workspace and a->workspace_bytes are ignored.
 * The scratch is instead a device array of TP_MLP_NOALLOC_SCRATCH_BYTES that
 * the library itself holds, one per GPU it runs on, for the life of the
 * process; the first call on a device looks up that device's copy (the
 * device current at the call).  The call allocates nothing.
 *   Returns TP_MLP_EWORKSPACE, before any work is enqueued, when
 *   tp_mlp_workspace_bytes(d, phase) exceeds TP_MLP_NOALLOC_SCRATCH_BYTES.
 *   Every call on one GPU shares that GPU's scratch: calls whose work may
 *   overlap on one device (other streams, other threads) race; order them
 *   on one stream or synchronise them.  The scratch holds no state from one
 *   call to the next that a later call relies on (every element a call reads
 *   was written by that call).
 */
#define TP_MLP_NOALLOC_SCRATCH_BYTES (128u << 20)
int tp_mlp_backward_noalloc(const tp_mlp_desc* d, int32_t phase, const tp_mlp_bwd_args* a, void* stream);

/*
 * tp_mlp_sgd_step - one plain SGD update, p <- p - lr * g (the page's one SGD
 * update of every parameter, "Reproduce one dense training step").
 *   param_in  [n] in param_dtype, param_out [n] in param_dtype (may equal
 *             param_in: in-place); grad [n] fp32.
 *   master_in == NULL: param_out = round(param_in - lr * grad), in fp32.
 *   master_in != NULL: fp32 master copies, master_out = master_in - lr * grad
 *             and param_out = round_bf16(master_out); param_dtype must be BF16
 *             and master_out non-NULL (may equal master_in).
 *   n >= 0 (n = 0 is a no-op).  Partially overlapping in/out ranges are an
 *   error only in the sense that results are then undefined.
 */
int tp_mlp_sgd_step(const void* param_in, void* param_out, const float* grad, const float* master_in,
                    float* master_out, int64_t n, int32_t param_dtype, float lr, void* stream);

/* One tensor of tp_mlp_sgd_step_multi (fields as in tp_mlp_sgd_step).
 * Optionally (bf16 parameters only) the updated values are also written
 * transposed: param_out_t != NULL receives the parameter seen as [t_rows,
 * t_cols] row-major (t_rows * t_cols == n, both multiples of 8) transposed,
 * [t_cols, t_rows], in the same bits as param_out.  This keeps the
 * transposed down weight that tp_mlp_backward can take (w_down_t) in step
 * with w_down [H, F]: t_rows = H, t_cols = F.  Zero-initialised: no copy. */
typedef struct {
  const void* param_in;
  void* param_out;
  const float* grad;
  const float* master_in;
  float* master_out;
  int64_t n;
  void* param_out_t;
  int64_t t_rows;
  int64_t t_cols;
} tp_mlp_sgd_tensor;

/*
 * tp_mlp_transpose_bf16 - out [cols, rows] = in [rows, cols] transposed, bf16,
 * row-major (a layout helper: the transposed down weight w_down_t of
 * tp_mlp_backward).  rows, cols >= 0 and multiples of 8; in and out DEVICE
 * pointers, 16-byte aligned, not overlapping.
 */
int tp_mlp_transpose_bf16(const void* in, void* out, int64_t rows, int64_t cols, void* stream);

/*
 * tp_mlp_sgd_step_multi - tp_mlp_sgd_step on `count` tensors with one kernel
 * launch (and one more for the tensors with a transposed copy).  `list` is a HOST array (read before the call returns).  All
 * tensors share param_dtype; either every tensor has fp32 masters or none
 * does.  Each tensor's rules are those of tp_mlp_sgd_step.  count >= 0.
 */
int tp_mlp_sgd_step_multi(const tp_mlp_sgd_tensor* list, int32_t count, int32_t param_dtype, float lr,
                          void* stream);

/*
 * AdamW ("Megatron-LM walkthrough", Part IV, Stage 8: after the gradient norm
 * is computed and the gradients clipped, AdamW updates the parameters; the
 * optimiser keeps fp32 moments and fp32 master weights, "Megatron-Core Guide:
 * 5D Distributed Training Architecture", section 1).  The update is the
 * published algorithm (Loshchilov & Hutter, decoupled weight decay, with
 * Adam's bias correction), per element, in fp32:
 *   g     = grad * s                  (s = *grad_scale, or 1 if grad_scale is NULL)
 *   m     = beta1 m + (1 - beta1) g
 *   v     = beta2 v + (1 - beta2) g^2
 *   theta = theta - lr * ( (m / (1 - beta1^step)) / (sqrt(v / (1 - beta2^step)) + eps)
 *                          + weight_decay * theta )
 * theta is the fp32 master when the tensor has one (then param_out =
 * round_bf16(theta)), else the parameter itself.
 */
typedef struct {
  float lr;
  float beta1;         /* in [0, 1) */
  float beta2;         /* in [0, 1) */
  float eps;           /* > 0 */
  float weight_decay;  /* >= 0 */
  int32_t step;        /* 1 for the first update; the bias corrections use it */
} tp_mlp_adamw_hparams;

/* One tensor of tp_mlp_adamw_step_multi. */
typedef struct {
  const void* param_in;    /* [n] param dtype; read only when there is no master */
  void* param_out;         /* [n] param dtype (may equal param_in) */
  const float* grad;       /* [n] fp32 */
  const float* master_in;  /* [n] fp32 master, or NULL (no master) */
  float* master_out;       /* [n] fp32 (may equal master_in); NULL iff master_in is */
  float* m;                /* [n] fp32 first moment, updated in place */
  float* v;                /* [n] fp32 second moment, updated in place */
  int64_t n;               /* >= 0 */
} tp_mlp_adamw_tensor;

/*
 * tp_mlp_adamw_step_multi - one AdamW update of `count` tensors (one kernel
 * launch per 32 tensors).  `list` and `hp` are HOST pointers, read before the
 * call returns.  All tensors share param_dtype; either every tensor has an
 * fp32 master or none does (masters require param_dtype BF16).  grad_scale is
 * a DEVICE pointer to one fp32 factor applied to every gradient (for example
 * the coefficient written by tp_mlp_clip_grad_norm), or NULL.  count >= 0.
 */
int tp_mlp_adamw_step_multi(const tp_mlp_adamw_tensor* list, int32_t count, int32_t param_dtype,
                            const tp_mlp_adamw_hparams* hp, const float* grad_scale, void* stream);

/*
 * tp_mlp_clip_grad_norm - the global gradient norm and clip coefficient of
 * Stage 8 ("the gradient norm is computed ... and clipped"):
 *   norm = sqrt( sum over all tensors and elements of grad^2 )
 *   coef = min(1, max_norm / (norm + 1e-6))   (coef = 1 when max_norm <= 0)
 * Squares are summed in fp64 in a fixed order (per 16384-element block, then
 * the block sums in tensor and block order): run-to-run deterministic.
 *   grads     HOST array of `count` DEVICE pointers to fp32 gradients
 *   counts    HOST array of their element counts (each >= 0)
 *   norm_out  DEVICE fp32 [1] receiving norm, or NULL
 *   coef_out  DEVICE fp32 [1] receiving coef (pass it as grad_scale to
 *             tp_mlp_adamw_step_multi; the gradients themselves are unchanged)
 *   workspace caller-owned DEVICE scratch of at least
 *             tp_mlp_clip_grad_norm_workspace_bytes(counts, count) bytes
 */
int tp_mlp_clip_grad_norm(const float* const* grads, const int64_t* counts, int32_t count, float max_norm,
                          float* norm_out, float* coef_out, void* workspace, size_t workspace_bytes,
                          void* stream);

/* Bytes of workspace tp_mlp_clip_grad_norm needs (counts: HOST array). */
size_t tp_mlp_clip_grad_norm_workspace_bytes(const int64_t* counts, int32_t count);

/*
 * FP8 GEMMs with per-tensor delayed scaling ("Megatron-Core Guide: 5D
 * Distributed Training Architecture": Transformer Engine runs the matrix
 * products in FP8 with delayed scaling, feature list item 6).  The pages give
 * no recipe; this is Transformer Engine's default one:
 *   - formats (OCP FP8): E4M3 (largest finite 448) for the normed input N,
 *     the weights and the activation A; E5M2 (largest 57344) for the output
 *     gradient and the pre-activation gradient;
 *   - code(x) = round-to-nearest-even(clamp(fp32(x) * s, +-max)), s the
 *     tensor role's current scale;
 *   - a GEMM of codes is dequantised by (1/s_a)(1/s_b) in fp32;
 *   - every cast folds max|x| into its role's running amax; at the end of the
 *     step tp_mlp_fp8_update_scales pushes it into an amax history of length
 *     L and sets s = max / max(history) when that is positive and finite
 *     (else s is kept).  Shards that share a meta share the amax: the amax
 *     reduction over the tensor-parallel group.
 * Every GEMM of the step runs on FP8 codes: the forward F2 and F3 on
 * E4M3 x E4M3, the backward d_act, d_w_down, d_normed and d_w_in on
 * E5M2 x E4M3; everything between them (norm, activation and its backward,
 * residual, sums, update) is the bf16 path's.
 *
 * Meta: a DEVICE fp32 array of TP_MLP_FP8_META_FLOATS(L) elements:
 *   [0] scale s   [1] 1/s   [2] running amax   [3] format max   [4..4+L) history, newest first.
 * Initialise it with tp_mlp_fp8_meta_init; the library updates it from then
 * on.  A caller may restore a saved meta (a checkpoint) by writing all of
 * its floats, [1] being the fp32 reciprocal of [0].  1 <= L <= 1024.
 */
enum { TP_MLP_FP8_E4M3 = 0, TP_MLP_FP8_E5M2 = 1 };
#define TP_MLP_FP8_META_FLOATS(L) (4 + (L))
#define TP_MLP_FP8_MAX_HISTORY 1024

/* s = 1, 1/s = 1, amax = 0, format max, zero history (a kernel on `stream`). */
int tp_mlp_fp8_meta_init(float* meta, int32_t fmt, int32_t history_len, void* stream);

/*
 * tp_mlp_fp8_cast - codes of a bf16 matrix x [rows, cols] with meta's scale:
 * out [rows, cols] and/or out_t [cols, ldt] = the codes transposed (either may
 * be NULL, not both); max|x| folds into meta's running amax.  cols: a
 * multiple of 8.  out_t: ldt >= rows and a multiple of 16; its columns rows ..
 * ldt-1 are written as 0 (the zero padding that lets a transposed operand
 * have a k extent of ldt).  fmt must be the format meta was initialised with.
 */
int tp_mlp_fp8_cast(int64_t rows, int64_t cols, const void* x, int32_t fmt, float* meta, uint8_t* out,
                    uint8_t* out_t, int64_t ldt, void* stream);

/* End of step: every meta's running amax enters its history (then is zeroed)
 * and its scale is renewed.  metas: HOST array of count DEVICE pointers
 * (count <= 16), all with history length history_len. */
int tp_mlp_fp8_update_scales(float* const* metas, int32_t count, int32_t history_len, void* stream);

/* Metas and code buffers of one shard's FP8 step.  Tp = T rounded up to a
 * multiple of 16; P = 2F (SwiGLU) or F (GeLU).  Every buffer is DEVICE
 * memory, 16-byte aligned, owned by the caller; shapes are row-major. */
typedef struct {
  int32_t history_len;  /* L of every meta */
  float* meta_normed;   /* E4M3 */
  float* meta_w_in;     /* E4M3 */
  float* meta_act;      /* E4M3 */
  float* meta_w_down;   /* E4M3 */
  float* meta_d_out;    /* E5M2 */
  float* meta_d_pre;    /* E5M2 */
  /* written by tp_mlp_forward_fp8 (normed_q / normed_t: unless NORMED_READY,
     then read), read by tp_mlp_backward_fp8 */
  uint8_t* normed_q;    /* [T, H]  */
  uint8_t* normed_t;    /* [H, Tp] */
  uint8_t* w_in_q;      /* [P, H]  */
  uint8_t* w_in_t;      /* [H, P]  */
  uint8_t* act_q;       /* [T, F]  */
  uint8_t* act_t;       /* [F, Tp] */
  uint8_t* w_down_q;    /* [H, F]  */
  uint8_t* w_down_t;    /* [F, H]  */
  /* written by tp_mlp_backward_fp8 (d_out_q / d_out_t: unless
     TP_MLP_FP8_SHARED_READY, then read) */
  uint8_t* d_out_q;     /* [T, H]  */
  uint8_t* d_out_t;     /* [H, Tp] */
  uint8_t* d_pre_q;     /* [T, P]  */
  uint8_t* d_pre_t;     /* [P, Tp] */
} tp_mlp_fp8_args;

/*
 * tp_mlp_fp8_gemm - the FP8 GEMM on its own:
 *   C[m, n] (+)= (sum_k dec(A[m, k]) dec(B[n, k])) * scale_inv_a[0] * scale_inv_b[0]
 *   A [M, lda] codes in fmt_a, B [N, ldb] codes in fmt_b (both K-contiguous;
 *   K <= lda, K <= ldb, K a multiple of 16, lda and ldb multiples of 16);
 *   (fmt_a, fmt_b) = (E4M3, E4M3) or (E5M2, E4M3).  scale_inv_a/b: DEVICE
 *   pointers to one fp32 each (a meta + 1).  C [M, ldc] fp32 (N and ldc
 *   multiples of 4, ldc >= N); with accumulate != 0 the product is added to
 *   C.  The k range may be split over workgroups (a function of M, N and K
 *   only, so the result is run-to-run deterministic); the split needs a
 *   workspace of tp_mlp_fp8_gemm_workspace_bytes(M, N, K, ldc) bytes (may be 0).
 * The hardware sums each 128-long block of k with about 12 bits of precision
 * relative to the block's largest product, then adds the block sums in fp32.
 */
int tp_mlp_fp8_gemm(int64_t M, int64_t N, int64_t K, const uint8_t* A, int64_t lda, int32_t fmt_a,
                    const float* scale_inv_a, const uint8_t* B, int64_t ldb, int32_t fmt_b, const float* scale_inv_b,
                    float* C, int64_t ldc, int32_t accumulate, void* workspace, size_t workspace_bytes, void* stream);
size_t tp_mlp_fp8_gemm_workspace_bytes(int64_t M, int64_t N, int64_t K, int64_t ldc);

/* tp_mlp_desc.flags for tp_mlp_backward_fp8: d_out_q and d_out_t already
 * hold this step's codes of d_out (an earlier shard's call wrote them). */
enum { TP_MLP_FP8_SHARED_READY = 8 };

/*
 * tp_mlp_forward_fp8 - tp_mlp_forward with F2 and F3 on FP8 codes.  Same
 * arguments and outputs (dtype must be TP_MLP_BF16; H and F multiples of 16),
 * plus f8: casts N (normed_q, normed_t; skipped with NORMED_READY), w_in
 * (w_in_q, w_in_t), A (act_q, act_t) and w_down (w_down_q, w_down_t), each
 * row copy for the forward GEMM and transposed copy for the backward.
 */
int tp_mlp_forward_fp8(const tp_mlp_desc* d, const void* x, const void* norm_w, const void* w_in,
                       const void* b_in, const void* w_down, void* normed, float* rstd, void* pre_act,
                       void* act, void* out, const void* b_down, const tp_mlp_fp8_args* f8, void* stream);

/*
 * tp_mlp_backward_fp8 - tp_mlp_backward (phase TP_MLP_BWD_SHARD) with its
 * four GEMMs on FP8 codes: d_act = d_out Wd on d_out_q and w_down_t;
 * d_w_down = d_out^T act on d_out_t and act_t; d_normed_part = d_pre w_in on
 * d_pre_q and w_in_t; d_w_in = d_pre^T normed on d_pre_t and normed_t.  It
 * casts d_out (unless TP_MLP_FP8_SHARED_READY) and d_pre; the codes of the
 * forward must be those of the same step.  The other tp_mlp_bwd_args fields,
 * the workspace (tp_mlp_workspace_bytes) and ACCUMULATE_GRADS are as for
 * tp_mlp_backward; phase TP_MLP_BWD_NORM is tp_mlp_backward's.
 */
int tp_mlp_backward_fp8(const tp_mlp_desc* d, int32_t phase, const tp_mlp_bwd_args* a,
                        const tp_mlp_fp8_args* f8, void* stream);

/*
 * The attention sublayer of one tensor-parallel rank, the same pattern as the
 * MLP block ("Megatron-LM walkthrough", Part IV, Stages 5-6 and Part V, "Deep
 * dive: tensor parallelism and the f and g operators": the QKV projection is
 * column-parallel, so each rank computes Q, K and V of its own heads; attention
 * runs locally per head; the output projection is row-parallel and its partial
 * is summed across the ranks; in backward the gradient of the QKV input is
 * summed).  Ranks own complete grouped-query head groups ("Megatron
 * tensor-parallel MLP", closing section).  With the pages silent on the
 * attention itself, it is:
 *     N   = rms_norm(x, norm_w)                   (as in tp_mlp_forward)
 *     QKV = N W_qkv^T                             (no bias), columns [Q heads | K heads | V heads]
 *     o_h = softmax_causal(q_h k_g^T / sqrt(D)) v_g,   g = h / (n_q / n_kv)
 *     out = x + O W_o^T + b_o                     (b_o once, after the partial sum)
 * x is [batch, seq, H] flattened to T = batch * seq rows (a sequence's rows
 * contiguous); causal means key position <= query position within a sequence.
 * bf16 only (fp32 accumulation).  D (head_dim) is 64 or 128; seq * W < 2^30
 * (W defined below; TP_MLP_ESHAPE otherwise).
 */
typedef struct {
  int64_t batch;     /* sequences */
  int64_t seq;       /* positions per sequence (T = batch * seq) */
  int64_t hidden;    /* H: positive multiple of 8, <= 16384 */
  int32_t n_q;       /* query heads of this rank */
  int32_t n_kv;      /* key/value heads of this rank; n_q a multiple of it */
  int32_t head_dim;  /* D: 64 or 128 */
  int32_t dtype;     /* TP_MLP_BF16 */
  float eps;         /* RMSNorm epsilon */
  int32_t flags;     /* TP_MLP_FUSE_EPILOGUE | TP_MLP_NORMED_READY | TP_MLP_ACCUMULATE_GRADS */
} tp_attn_desc;

/*
 * tp_attn_forward - one rank's attention forward.  W = (n_q + 2 n_kv) D.
 *   x [T, H], norm_w [H], w_qkv [W, H] (rows: this rank's Q heads, then K heads,
 *   then V heads, D rows each), w_o [H, n_q D] (this rank's columns), bf16;
 *   normed [T, H] bf16 and rstd [T] fp32 out (in, with NORMED_READY);
 *   qkv [T, W] bf16 out; attn_out [T, n_q D] bf16 out (O); lse [n_q, T] fp32
 *   out (log of each row's softmax denominator, for the backward);
 *   out: without FUSE_EPILOGUE [T, H] fp32, this rank's partial O W_o^T; with
 *   it [T, H] bf16 x + O W_o^T + b_o (b_o [H] bf16, read only then).
 *   workspace: NULL, or DEVICE scratch (16-byte aligned) of at least
 *   tp_attn_forward_workspace_bytes(d) bytes (TP_MLP_EWORKSPACE if smaller):
 *   with it the QKV product, whose W columns give few output tiles, splits
 *   its k range over more workgroups (fp32 slices added in a fixed order);
 *   without it the product runs unsplit.  The result bits do not depend on
 *   workspace's address, only on whether one is given.
 */
int tp_attn_forward(const tp_attn_desc* d, const void* x, const void* norm_w, const void* w_qkv, const void* w_o,
                    void* normed, float* rstd, void* qkv, void* attn_out, float* lse, void* out, const void* b_o,
                    void* workspace, size_t workspace_bytes, void* stream);
size_t tp_attn_forward_workspace_bytes(const tp_attn_desc* d);

typedef struct {
  /* saved from tp_attn_forward */
  const void* x;           /* [T, H] */
  const void* normed;      /* [T, H] */
  const float* rstd;       /* [T] */
  const void* qkv;         /* [T, W] */
  const void* attn_out;    /* [T, n_q D] */
  const float* lse;        /* [n_q, T] */
  /* parameters */
  const void* norm_w;      /* [H] */
  const void* w_qkv;       /* [W, H] */
  const void* w_o;         /* [H, n_q D] */
  const void* d_out;       /* [T, H] bf16: gradient of the sublayer output (= out for the loss sum(out^2)/2) */
  /* SHARD phase outputs */
  void* d_attn_out;        /* [T, n_q D] bf16: dO = d_out W_o */
  void* d_qkv;             /* [T, W] bf16 */
  float* d_w_qkv;          /* [W, H] fp32 */
  float* d_w_o;            /* [H, n_q D] fp32 */
  float* d_normed_part;    /* [T, H] fp32: this rank's partial of dL/dN */
  /* NORM phase */
  const float* d_normed;   /* [T, H] fp32: summed over ranks */
  void* d_x;               /* [T, H] bf16 */
  float* d_norm_w;         /* [H] fp32 */
  float* d_b_o;            /* [H] fp32 */
  void* workspace;
  size_t workspace_bytes;
  /* NORM phase, instead of d_normed: the shards' partials of dL/dN
     (d_normed_part of each SHARD call), summed by the RMSNorm backward as it
     reads them -- in index order with fp32 additions, the sum tp_partial_sum
     forms, so the results are the same bits.  A HOST array of
     n_d_normed_parts DEVICE pointers, each [T, H] fp32,
     1 <= n_d_normed_parts <= 64.  n_d_normed_parts = 0 (as in
     zero-initialised args): d_normed is read. */
  const float* const* d_normed_parts;
  int32_t n_d_normed_parts;
} tp_attn_bwd_args;

/*
 * tp_attn_backward - the backward of tp_attn_forward in the two phases of
 * tp_mlp_backward.  SHARD: dO = d_out W_o; d_w_o = d_out^T O; the attention
 * backward (dS = P (dP - rowsum(dO o O)), P recomputed from lse) gives
 * d_qkv; d_w_qkv = d_qkv^T N; d_normed_part = d_qkv W_qkv.  NORM: RMSNorm's
 * backward with the residual, d_norm_w and d_b_o = sum_t d_out, on dN given
 * summed (d_normed) or as the shards' partials (d_normed_parts).
 * Workspace: tp_attn_workspace_bytes(d, phase).  Deterministic.
 */
int tp_attn_backward(const tp_attn_desc* d, int32_t phase, const tp_attn_bwd_args* a, void* stream);
size_t tp_attn_workspace_bytes(const tp_attn_desc* d, int32_t phase);

/*
 * tp_attention_forward / tp_attention_backward - the causal grouped-query
 * attention on its own (the kernels tp_attn_* run between the projections).
 *   qkv [batch seq, ld] bf16 with the Q, K, V head columns at 0, n_q D and
 *   (n_q + n_kv) D (ld >= (n_q + 2 n_kv) D, a multiple of 8); o and d_o
 *   [batch seq, n_q D] bf16; lse [n_q, batch seq] fp32; d_qkv [batch seq, ld]
 *   bf16 (its first (n_q + 2 n_kv) D columns written).  head_dim 64 or 128;
 *   seq * ld < 2^30 (TP_MLP_ESHAPE otherwise: the kernels address one
 *   sequence's rows with 32-bit byte offsets).
 *   workspace: DEVICE scratch, 16-byte aligned, of at least
 *   tp_attention_backward_workspace_bytes(...) bytes (the softmax row terms
 *   rowsum(dO o O) and, when n_q > n_kv, each query head's fp32 share of dK
 *   and dV, added in a fixed order); TP_MLP_EWORKSPACE if smaller.
 *   Deterministic.
 */
int tp_attention_forward(int64_t batch, int64_t seq, int32_t n_q, int32_t n_kv, int32_t head_dim, const void* qkv,
                         int64_t ld, void* o, float* lse, void* stream);
int tp_attention_backward(int64_t batch, int64_t seq, int32_t n_q, int32_t n_kv, int32_t head_dim, const void* qkv,
                          int64_t ld, const void* o, const void* d_o, const float* lse, void* workspace,
                          size_t workspace_bytes, void* d_qkv, void* stream);
size_t tp_attention_backward_workspace_bytes(int64_t batch, int64_t seq, int32_t n_q, int32_t n_kv,
                                             int32_t head_dim);

/*
 * Kernel timing, a measurement aid (off by default).  While enabled, every
 * kernel the library launches is bracketed by two hipEvents recorded on the
 * launch's own stream; durations are aggregated per kernel name.
 *   tp_mlp_profile_enable(1) clears earlier records and starts recording;
 *   tp_mlp_profile_enable(0) stops recording (records are kept).
 *   tp_mlp_profile_count() waits for the recorded events and returns the
 *   number of distinct kernel names (or a negative error code);
 *   tp_mlp_profile_entry(i, ...) returns entry i: name (valid until the next
 *   enable(1) or count call), number of launches and total milliseconds.
 *   tp_mlp_profile_only(name) restricts recording to the kernels of that
 *   name (the names tp_mlp_profile_entry reports); NULL records every kernel
 *   again.  The name is copied.
 * Event recording adds a few microseconds per launch; leave it off outside
 * measurements, or restrict it to the kernel being measured.
 */
int tp_mlp_profile_enable(int32_t on);
int tp_mlp_profile_only(const char* name);
int32_t tp_mlp_profile_count(void);
int tp_mlp_profile_entry(int32_t i, const char** name, int64_t* launches, double* total_ms);

/* Message describing the last failure on the calling thread ("" if none). */
const char* tp_mlp_last_error(void);

/* Library version string. */
const char* tp_mlp_version(void);

#ifdef __cplusplus
}
#endif

#endif /* TP_MLP_H */
