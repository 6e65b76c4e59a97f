// HBM-bound kernels around the contractions: the shard partial sum, a
// deterministic column sum, and the SGD update.
#include "common.h"
#include "kernels.h"

namespace tpmlp {

hipError_t launch_reduce_partial_rows(const float* ws, float* out, int64_t nparts, int64_t cols, hipStream_t s);

namespace {

constexpr int kMaxParts = 64;

struct PartList {
  const float* p[kMaxParts];
};

// out = ((p0 + p1) + ...) + residual + bias, 4 columns per thread-step.
// "Split the contraction" (synapticradio.com): the partial down outputs are
// summed, then the replicated residual and bias are added once.
template <typename TI, typename TO, bool RES, bool BIAS>
__global__ __launch_bounds__(256) void partial_sum_kernel(PartList parts, int n_parts, int64_t n4, int64_t cols4,
                                                          const TI* __restrict__ residual, const TI* __restrict__ bias,
                                                          TO* __restrict__ out) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; e < n4; e += stride) {
    floatx4 acc = load4<float>(parts.p[0] + 4 * e);
    for (int k = 1; k < n_parts; ++k) acc += load4<float>(parts.p[k] + 4 * e);
    if constexpr (RES) acc += load4<TI>(residual + 4 * e);
    if constexpr (BIAS) acc += load4<TI>(bias + 4 * (e % cols4));
    store4<TO>(out + 4 * e, acc);
  }
}

inline unsigned grid_for(int64_t n, int64_t per_block) {
  int64_t b = (n + per_block - 1) / per_block;
  const int64_t cap = 256 * 32;  // 32 workgroups per CU, grid-stride beyond that
  if (b > cap) b = cap;
  return (unsigned)(b < 1 ? 1 : b);
}

template <typename TI, typename TO>
hipError_t psum_t(const PartList& pl, int n, int64_t rows, int64_t cols, const void* res, const void* bias, void* out,
                  hipStream_t s) {
  const int64_t n4 = rows * cols / 4, cols4 = cols / 4;
  const TI* r = static_cast<const TI*>(res);
  const TI* b = static_cast<const TI*>(bias);
  TO* o = static_cast<TO*>(out);
  const dim3 grid(grid_for(n4, 256)), block(256);
  KernelTimer timer((r || b) ? "partial_sum_residual" : "partial_sum", s);
  if (r && b) hipLaunchKernelGGL((partial_sum_kernel<TI, TO, true, true>), grid, block, 0, s, pl, n, n4, cols4, r, b, o);
  else if (r) hipLaunchKernelGGL((partial_sum_kernel<TI, TO, true, false>), grid, block, 0, s, pl, n, n4, cols4, r, b, o);
  else if (b) hipLaunchKernelGGL((partial_sum_kernel<TI, TO, false, true>), grid, block, 0, s, pl, n, n4, cols4, r, b, o);
  else hipLaunchKernelGGL((partial_sum_kernel<TI, TO, false, false>), grid, block, 0, s, pl, n, n4, cols4, r, b, o);
  return hipGetLastError();
}

// Column sums, stage 1: workgroup b sums rows [b R, (b+1) R) of its column
// units in row order and writes partial row b.
constexpr int kColThreads = 256;
constexpr int kColRows = 64;

template <typename T>
__global__ __launch_bounds__(kColThreads) void colsum_partial_kernel(const T* __restrict__ in, float* __restrict__ ws,
                                                                      int64_t rows, int64_t cols) {
  const int64_t q = (int64_t)blockIdx.y * kColThreads + threadIdx.x;  // column unit (4 columns)
  if (4 * q >= cols) return;
  const int64_t r0 = (int64_t)blockIdx.x * kColRows;
  const int64_t r1 = min(rows, r0 + kColRows);
  floatx4 acc = {0.f, 0.f, 0.f, 0.f};
  for (int64_t t = r0; t < r1; ++t) acc += load4<T>(in + t * cols + 4 * q);
  store4<float>(ws + (int64_t)blockIdx.x * cols + 4 * q, acc);
}

// SGD: p <- p - lr g ("Reproduce one dense training step": one SGD update).
// Out of place when pout != pin (the input is then left unchanged).
template <typename T, bool MASTER>
__global__ __launch_bounds__(256) void sgd_kernel(const T* pin, T* pout, const float* __restrict__ g,
                                                  const float* min_, float* mout, int64_t n, float lr) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  const int64_t n4 = n / 4;
  for (int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; e < n4; e += stride) {
    const floatx4 gv = load4<float>(g + 4 * e);
    floatx4 v;
    if constexpr (MASTER) {
      v = load4<float>(min_ + 4 * e) - lr * gv;
      store4<float>(mout + 4 * e, v);
    } else {
      v = load4<T>(pin + 4 * e) - lr * gv;
    }
    store4<T>(pout + 4 * e, v);
  }
  // tail (n % 4 elements), handled by the first threads of the grid
  const int64_t t = 4 * n4 + (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (t < n) {
    float v;
    if constexpr (MASTER) {
      v = min_[t] - lr * g[t];
      mout[t] = v;
    } else {
      v = Elem<T>::to_f32(pin[t]) - lr * g[t];
    }
    pout[t] = Elem<T>::from_f32(v);
  }
}

__global__ __launch_bounds__(256) void ksplit_reduce_kernel(float* __restrict__ C, const float* __restrict__ ws,
                                                             int nslices, int64_t M, int64_t N4, int64_t ldc) {
  const int64_t total = M * N4, stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; e < total; e += stride) {
    const int64_t m = e / N4, n = 4 * (e - m * N4);
    const int64_t off = m * ldc + n;
    floatx4 acc = load4<float>(C + off);
    for (int s = 0; s < nslices; ++s) acc += load4<float>(ws + (int64_t)s * M * ldc + off);
    store4<float>(C + off, acc);
  }
}

}  // namespace

hipError_t launch_ksplit_reduce(float* C, const float* ws, int nslices, int64_t M, int64_t N, int64_t ldc,
                                hipStream_t s) {
  if (M == 0 || N == 0 || nslices == 0) return hipSuccess;
  KernelTimer timer("ksplit_reduce", s);
  hipLaunchKernelGGL(ksplit_reduce_kernel, dim3(grid_for(M * N / 4, 256)), dim3(256), 0, s, C, ws, nslices, M, N / 4,
                     ldc);
  return hipGetLastError();
}

hipError_t launch_partial_sum(const float* const* parts, int n_parts, int64_t rows, int64_t cols, const void* residual,
                              const void* bias, DType in_dt, void* out, DType out_dt, hipStream_t s) {
  if (rows == 0 || cols == 0) return hipSuccess;
  PartList pl{};
  for (int i = 0; i < n_parts; ++i) pl.p[i] = parts[i];
  if (in_dt == kBF16) {
    if (out_dt == kBF16) return psum_t<bf16_t, bf16_t>(pl, n_parts, rows, cols, residual, bias, out, s);
    return psum_t<bf16_t, float>(pl, n_parts, rows, cols, residual, bias, out, s);
  }
  if (out_dt == kBF16) return psum_t<float, bf16_t>(pl, n_parts, rows, cols, residual, bias, out, s);
  return psum_t<float, float>(pl, n_parts, rows, cols, residual, bias, out, s);
}

size_t colsum_workspace(int64_t rows, int64_t cols) {
  const int64_t nb = (rows + kColRows - 1) / kColRows;
  return (size_t)(nb * cols) * sizeof(float);
}

hipError_t launch_colsum(DType dt, const void* in, float* out, void* ws, int64_t rows, int64_t cols, hipStream_t s) {
  const int64_t nb = (rows + kColRows - 1) / kColRows;
  float* w = static_cast<float*>(ws);
  if (nb > 0) {
    const dim3 grid((unsigned)nb, (unsigned)((cols / 4 + kColThreads - 1) / kColThreads));
    KernelTimer timer("column_sum", s);
    if (dt == kBF16)
      hipLaunchKernelGGL(colsum_partial_kernel<bf16_t>, grid, dim3(kColThreads), 0, s,
                         static_cast<const bf16_t*>(in), w, rows, cols);
    else
      hipLaunchKernelGGL(colsum_partial_kernel<float>, grid, dim3(kColThreads), 0, s, static_cast<const float*>(in),
                         w, rows, cols);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return launch_reduce_partial_rows(w, out, nb, cols, s);
}

hipError_t launch_sgd(DType dt, const void* param_in, void* param_out, const float* grad, const float* master_in,
                      float* master_out, int64_t n, float lr, hipStream_t s) {
  if (n == 0) return hipSuccess;
  const dim3 grid(grid_for(n / 4 + 1, 256)), block(256);
  KernelTimer timer("sgd", s);
  if (dt == kBF16) {
    const bf16_t* pi = static_cast<const bf16_t*>(param_in);
    bf16_t* po = static_cast<bf16_t*>(param_out);
    if (master_in)
      hipLaunchKernelGGL((sgd_kernel<bf16_t, true>), grid, block, 0, s, pi, po, grad, master_in, master_out, n, lr);
    else
      hipLaunchKernelGGL((sgd_kernel<bf16_t, false>), grid, block, 0, s, pi, po, grad, master_in, master_out, n, lr);
  } else {
    hipLaunchKernelGGL((sgd_kernel<float, false>), grid, block, 0, s, static_cast<const float*>(param_in),
                       static_cast<float*>(param_out), grad, master_in, master_out, n, lr);
  }
  return hipGetLastError();
}

}  // namespace tpmlp
