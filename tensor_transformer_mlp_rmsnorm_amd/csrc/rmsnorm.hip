// RMSNorm forward and backward (+ residual) of the pre-norm MLP sublayer.
//
// Forward  ("Start with the dense block", synapticradio.com: N = rms_norm(x, norm_weight)):
//   rstd_t = 1 / sqrt(mean_i x_ti^2 + eps),   N_ti = x_ti rstd_t w_i
// Backward ("Put the other collective in backward": the summed dN goes
// through RMSNorm's backward and into the residual input):
//   c_t   = (1/H) sum_i dN_ti w_i x_ti
//   dx_ti = dY_ti + rstd_t dN_ti w_i - x_ti rstd_t^3 c_t
//   dw_i  = sum_t dN_ti x_ti rstd_t,   db_i = sum_t dY_ti
// Both are HBM-bound.  The forward reads each row once (one wavefront per
// row, the row held in registers) and writes N and rstd.  The backward
// streams dN (fp32), x and dY once, writes dx, and reduces the two column
// sums deterministically: each workgroup owns a fixed range of rows and
// fixed columns per thread, writes one partial row, and a second kernel sums
// the partial rows in index order.
#include "common.h"
#include "kernels.h"

namespace tpmlp {
namespace {

constexpr int kFwdRowsPerBlock = 4;  // one wave per row

template <typename T, int NC>
__global__ __launch_bounds__(256) void rmsnorm_fwd_kernel(const T* __restrict__ x, const T* __restrict__ w,
                                                          T* __restrict__ n, float* __restrict__ rstd,
                                                          int64_t rows, int H, float eps) {
  constexpr int E = Elem<T>::kPerChunk;
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * kFwdRowsPerBlock + (threadIdx.x >> 6);
  if (row >= rows) return;
  const int nch = H / E;
  const T* xr = x + row * H;
  uint4 v[NC];
  float ss = 0.f;
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    const int idx = lane + 64 * c;
    v[c] = make_uint4(0, 0, 0, 0);
    if (idx < nch) v[c] = *reinterpret_cast<const uint4*>(xr + (int64_t)idx * E);
    float f[E];
    Chunk<T>::unpack(v[c], f);
#pragma unroll
    for (int e = 0; e < E; ++e) ss += f[e] * f[e];
  }
  ss = wave_sum(ss);
  const float r = 1.0f / sqrtf(ss / (float)H + eps);
  if (lane == 0) rstd[row] = r;
  T* nr = n + row * H;
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    const int idx = lane + 64 * c;
    if (idx >= nch) continue;
    float f[E], wf[E];
    Chunk<T>::unpack(v[c], f);
    Chunk<T>::unpack(*reinterpret_cast<const uint4*>(w + (int64_t)idx * E), wf);
#pragma unroll
    for (int e = 0; e < E; ++e) f[e] = f[e] * r * wf[e];
    *reinterpret_cast<uint4*>(nr + (int64_t)idx * E) = Chunk<T>::pack(f);
  }
}

template <typename T>
hipError_t fwd_t(const void* x, const void* w, void* n, float* rstd, int64_t T_, int64_t H, float eps,
                 hipStream_t s) {
  constexpr int E = Elem<T>::kPerChunk;
  const int64_t nch = H / E;
  const int64_t per_lane = (nch + 63) / 64;
  const dim3 grid((unsigned)((T_ + kFwdRowsPerBlock - 1) / kFwdRowsPerBlock));
  const T* xp = static_cast<const T*>(x);
  const T* wp = static_cast<const T*>(w);
  T* np_ = static_cast<T*>(n);
  KernelTimer timer("rmsnorm_fwd", s);
#define TPMLP_FWD(NC) \
  hipLaunchKernelGGL((rmsnorm_fwd_kernel<T, NC>), grid, dim3(256), 0, s, xp, wp, np_, rstd, T_, (int)H, eps)
  if (per_lane <= 1) TPMLP_FWD(1);
  else if (per_lane <= 2) TPMLP_FWD(2);
  else if (per_lane <= 4) TPMLP_FWD(4);
  else if (per_lane <= 8) TPMLP_FWD(8);
  else if (per_lane <= 16) TPMLP_FWD(16);
  else TPMLP_FWD(32);
#undef TPMLP_FWD
  return hipGetLastError();
}

// ------------------------------------------------------------------ backward

constexpr int kBwdThreads = 256;

// Rows per workgroup of the backward: a function of (T, H) only, so the
// reduction order (and the result bits) never depend on the device.
__host__ __device__ inline int64_t bwd_rows_per_block(int64_t T_) {
  const int64_t kMaxBlocks = 512;
  int64_t r = (T_ + kMaxBlocks - 1) / kMaxBlocks;
  return r < 8 ? 8 : r;
}

template <typename T, int UPT>
__global__ __launch_bounds__(kBwdThreads) void rmsnorm_bwd_kernel(
    const float* __restrict__ dN, const T* __restrict__ x, const T* __restrict__ dY,
    const float* __restrict__ rstd, const T* __restrict__ w, T* __restrict__ dx, float* __restrict__ ws_dw,
    float* __restrict__ ws_db, int64_t rows, int H, int64_t rows_per_block) {
  __shared__ float red[2][kBwdThreads / 64];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int nunits = H / 4;  // 4 columns per unit
  const int64_t r0 = (int64_t)blockIdx.x * rows_per_block;
  const int64_t r1 = min(rows, r0 + rows_per_block);
  floatx4 wv[UPT], dwa[UPT], dba[UPT];
#pragma unroll
  for (int u = 0; u < UPT; ++u) {
    const int q = tid + kBwdThreads * u;
    wv[u] = (q < nunits) ? load4<T>(w + 4 * q) : floatx4{0.f, 0.f, 0.f, 0.f};
    dwa[u] = floatx4{0.f, 0.f, 0.f, 0.f};
    dba[u] = floatx4{0.f, 0.f, 0.f, 0.f};
  }
  const float invH = 1.0f / (float)H;
  for (int64_t t = r0; t < r1; ++t) {
    const float r = rstd[t];
    floatx4 dn[UPT], xv[UPT], dy[UPT];
    float part = 0.f;
#pragma unroll
    for (int u = 0; u < UPT; ++u) {
      const int q = tid + kBwdThreads * u;
      if (q < nunits) {
        const int64_t off = t * H + 4 * q;
        dn[u] = load4<float>(dN + off);
        xv[u] = load4<T>(x + off);
        dy[u] = load4<T>(dY + off);
      } else {
        dn[u] = xv[u] = dy[u] = floatx4{0.f, 0.f, 0.f, 0.f};
      }
      const floatx4 p = dn[u] * wv[u] * xv[u];
      part += (p[0] + p[1]) + (p[2] + p[3]);
    }
    part = wave_sum(part);
    const int slot = (int)(t & 1);
    if (lane == 0) red[slot][wave] = part;
    __syncthreads();
    float c = 0.f;
#pragma unroll
    for (int i = 0; i < kBwdThreads / 64; ++i) c += red[slot][i];
    c *= invH;
    const float r3c = r * r * r * c;
#pragma unroll
    for (int u = 0; u < UPT; ++u) {
      const int q = tid + kBwdThreads * u;
      if (q >= nunits) continue;
      const floatx4 d = dy[u] + r * dn[u] * wv[u] - xv[u] * r3c;
      store4<T>(dx + t * H + 4 * q, d);
      dwa[u] += dn[u] * xv[u] * r;
      dba[u] += dy[u];
    }
  }
#pragma unroll
  for (int u = 0; u < UPT; ++u) {
    const int q = tid + kBwdThreads * u;
    if (q >= nunits) continue;
    store4<float>(ws_dw + (int64_t)blockIdx.x * H + 4 * q, dwa[u]);
    store4<float>(ws_db + (int64_t)blockIdx.x * H + 4 * q, dba[u]);
  }
}

}  // namespace

// Fixed-order sum over `nparts` partial rows: out[c] = sum_{b=0}^{nparts-1} ws[b][c]
// (added to out's current value when `accum`).
// A workgroup owns 32 columns; its 8 waves-quarters each sum a contiguous
// eighth of the rows (in row order) for one column, and the 8 group sums are
// added in group order.  The order depends only on nparts: deterministic.
constexpr int kRedCols = 32, kRedGroups = 8;

__global__ __launch_bounds__(256) void reduce_partial_rows_kernel(const float* __restrict__ ws, float* __restrict__ out,
                                                                  int64_t nparts, int64_t cols, int accum) {
  __shared__ float part[kRedGroups][kRedCols];
  const int tc = threadIdx.x % kRedCols, grp = threadIdx.x / kRedCols;
  const int64_t c = (int64_t)blockIdx.x * kRedCols + tc;
  const int64_t per = (nparts + kRedGroups - 1) / kRedGroups;
  const int64_t b0 = grp * per, b1 = min(nparts, b0 + per);
  float acc = 0.f;
  if (c < cols)
    for (int64_t b = b0; b < b1; ++b) acc += ws[b * cols + c];
  part[grp][tc] = acc;
  __syncthreads();
  if (grp == 0 && c < cols) {
    float s = part[0][tc];
#pragma unroll
    for (int g = 1; g < kRedGroups; ++g) s += part[g][tc];
    out[c] = accum ? out[c] + s : s;
  }
}

hipError_t launch_reduce_partial_rows(const float* ws, float* out, int64_t nparts, int64_t cols, bool accum,
                                      hipStream_t s) {
  if (cols == 0) return hipSuccess;
  KernelTimer timer("column_reduce", s);
  hipLaunchKernelGGL(reduce_partial_rows_kernel, dim3((unsigned)((cols + kRedCols - 1) / kRedCols)), dim3(256), 0, s,
                     ws, out, nparts, cols, accum ? 1 : 0);
  return hipGetLastError();
}

hipError_t launch_rmsnorm_fwd(DType dt, const void* x, const void* w, void* n, float* rstd, int64_t T_, int64_t H,
                              float eps, hipStream_t s) {
  if (T_ == 0) return hipSuccess;
  if (dt == kBF16) return fwd_t<bf16_t>(x, w, n, rstd, T_, H, eps, s);
  return fwd_t<float>(x, w, n, rstd, T_, H, eps, s);
}

size_t rmsnorm_bwd_workspace(int64_t T_, int64_t H) {
  if (T_ <= 0) return 0;
  const int64_t nblk = (T_ + bwd_rows_per_block(T_) - 1) / bwd_rows_per_block(T_);
  return (size_t)(2 * nblk * H) * sizeof(float);
}

template <typename T>
static hipError_t bwd_t(const float* dN, const void* x, const void* dY, const float* rstd, const void* w, void* dx,
                        float* dw, float* db, void* ws, int64_t T_, int64_t H, bool accum, hipStream_t s) {
  const int64_t rpb = bwd_rows_per_block(T_);
  const int64_t nblk = (T_ + rpb - 1) / rpb;
  float* ws_dw = static_cast<float*>(ws);
  float* ws_db = ws_dw + nblk * H;
  const int64_t units = H / 4;
  const int64_t upt = (units + kBwdThreads - 1) / kBwdThreads;
  const T* xp = static_cast<const T*>(x);
  const T* dyp = static_cast<const T*>(dY);
  const T* wp = static_cast<const T*>(w);
  T* dxp = static_cast<T*>(dx);
  if (nblk > 0) {
    KernelTimer timer("rmsnorm_bwd", s);
#define TPMLP_BWD(U)                                                                                           \
  hipLaunchKernelGGL((rmsnorm_bwd_kernel<T, U>), dim3((unsigned)nblk), dim3(kBwdThreads), 0, s, dN, xp, dyp, rstd, \
                     wp, dxp, ws_dw, ws_db, T_, (int)H, rpb)
  if (upt <= 1) TPMLP_BWD(1);
  else if (upt <= 2) TPMLP_BWD(2);
  else if (upt <= 4) TPMLP_BWD(4);
  else if (upt <= 8) TPMLP_BWD(8);
  else TPMLP_BWD(16);
#undef TPMLP_BWD
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  hipError_t e;
  e = launch_reduce_partial_rows(ws_dw, dw, nblk, H, accum, s);
  if (e != hipSuccess) return e;
  return launch_reduce_partial_rows(ws_db, db, nblk, H, accum, s);
}

hipError_t launch_rmsnorm_bwd(DType dt, const float* dN, const void* x, const void* dY, const float* rstd,
                              const void* w, void* dx, float* dw, float* db, void* ws, int64_t T_, int64_t H,
                              bool accum, hipStream_t s) {
  // T = 0 still writes the (empty, zero) column sums (or leaves accumulated ones as they are).
  if (dt == kBF16) return bwd_t<bf16_t>(dN, x, dY, rstd, w, dx, dw, db, ws, T_, H, accum, s);
  return bwd_t<float>(dN, x, dY, rstd, w, dx, dw, db, ws, T_, H, accum, s);
}

}  // namespace tpmlp
