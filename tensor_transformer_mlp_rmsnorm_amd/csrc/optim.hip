// Optimiser kernels: AdamW over a list of tensors, and the global gradient
// norm with its clip coefficient ("Megatron-LM walkthrough", Part IV, Stage 8:
// the gradient norm is computed and the gradients clipped, then AdamW updates
// the parameters).  Both are HBM-bound streams over every parameter.
//
// AdamW is the published algorithm (Loshchilov & Hutter, decoupled weight
// decay, with Adam's bias correction); per element, in fp32:
//   g = grad * s;  m = b1 m + (1 - b1) g;  v = b2 v + (1 - b2) g^2
//   theta -= lr * ((m / bc1) / (sqrt(v / bc2) + eps) + wd * theta)
// with bc1 = 1 - b1^step, bc2 = 1 - b2^step.
#include "common.h"
#include "kernels.h"

namespace tpmlp {
namespace {

// AdamW: 4 elements (one 16-byte vector of each fp32 stream) per thread, the
// fastest of 4, 8 and 16 on this memory system.  Sum of squares: 64 elements
// per thread (16 coalesced vectors, each under its bounds check), so the
// per-workgroup reduction is amortised over 16384 elements; with 8 waves per
// SIMD the loads in flight suffice (issuing a thread's 16 loads together
// measured no faster).
constexpr int kPerThread = 4, kBlock = 256, kPerBlock = kPerThread * kBlock;
constexpr int kSumPerThread = 64, kSumPerBlock = kSumPerThread * kBlock;
constexpr int kMaxTensors = 32;

struct AdamwSeg {
  const void* pin;
  void* pout;
  const float* g;
  const float* min;
  float* mout;
  float* m;
  float* v;
  int64_t n;
  int64_t block0;  // first workgroup of this tensor
};
struct AdamwList {
  AdamwSeg seg[kMaxTensors];
  int count;
};

template <typename T, bool MASTER>
__global__ __launch_bounds__(kBlock) void adamw_kernel(AdamwList L, AdamwConst c, const float* __restrict__ scale) {
  int t = 0;
  while (t + 1 < L.count && (int64_t)blockIdx.x >= L.seg[t + 1].block0) ++t;
  const AdamwSeg& sg = L.seg[t];
  const float s = scale ? *scale : 1.0f;
  const T* pin = static_cast<const T*>(sg.pin);
  T* pout = static_cast<T*>(sg.pout);
  const float omb1 = 1.0f - c.beta1, omb2 = 1.0f - c.beta2;
  auto update = [&](float theta, float g, float& m, float& v) {
    g *= s;
    m = c.beta1 * m + omb1 * g;
    v = c.beta2 * v + omb2 * g * g;
    const float mhat = m / c.bc1;
    const float denom = sqrtf(v / c.bc2) + c.eps;
    return theta - c.lr * (mhat / denom + c.weight_decay * theta);
  };
  const int64_t e0 = ((int64_t)blockIdx.x - sg.block0) * kPerBlock + (int64_t)threadIdx.x * kPerThread;
  if (e0 + kPerThread <= sg.n) {
#pragma unroll
    for (int h = 0; h < kPerThread / 4; ++h) {
      const int64_t e = e0 + 4 * h;
      const floatx4 gv = load4<float>(sg.g + e);
      floatx4 mv = load4<float>(sg.m + e), vv = load4<float>(sg.v + e);
      const floatx4 th = MASTER ? load4<float>(sg.min + e) : load4<T>(pin + e);
      floatx4 out;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        float mr = mv[r], vr = vv[r];
        out[r] = update(th[r], gv[r], mr, vr);
        mv[r] = mr;
        vv[r] = vr;
      }
      store4<float>(sg.m + e, mv);
      store4<float>(sg.v + e, vv);
      if constexpr (MASTER) store4<float>(sg.mout + e, out);
      store4<T>(pout + e, out);
    }
  } else {
    for (int64_t e = e0; e < sg.n; ++e) {
      float mr = sg.m[e], vr = sg.v[e];
      const float th = MASTER ? sg.min[e] : Elem<T>::to_f32(pin[e]);
      const float out = update(th, sg.g[e], mr, vr);
      sg.m[e] = mr;
      sg.v[e] = vr;
      if constexpr (MASTER) sg.mout[e] = out;
      pout[e] = Elem<T>::from_f32(out);
    }
  }
}

// ---------------------------------------------------------- gradient norm

struct SumsqSeg {
  const float* g;
  int64_t n;
  int64_t block0;
};
struct SumsqList {
  SumsqSeg seg[kMaxTensors];
  int count;
  int64_t out0;  // index of this launch's first partial
};

// Fixed-order workgroup sum of one double per thread: a butterfly inside each
// wave (the same exchange pattern every time), then the 4 wave sums in order.
__device__ __forceinline__ double block_sum(double x, double* sh) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o, 64);
  if ((threadIdx.x & 63) == 0) sh[threadIdx.x >> 6] = x;
  __syncthreads();
  return ((sh[0] + sh[1]) + sh[2]) + sh[3];
}

// Partial b: sum of g^2 over the workgroup's 16384 elements; thread i takes
// the vectors i, i + 256, ... of the block (coalesced), in that order.
__global__ __launch_bounds__(kBlock) void sumsq_kernel(SumsqList L, double* __restrict__ partials) {
  __shared__ double sh[kBlock / 64];
  int t = 0;
  while (t + 1 < L.count && (int64_t)blockIdx.x >= L.seg[t + 1].block0) ++t;
  const SumsqSeg& sg = L.seg[t];
  const int64_t e0 = ((int64_t)blockIdx.x - sg.block0) * kSumPerBlock + (int64_t)threadIdx.x * 4;
  double acc = 0.0;
#pragma unroll
  for (int h = 0; h < kSumPerThread / 4; ++h) {
    const int64_t e = e0 + (int64_t)h * 4 * kBlock;
    if (e + 4 <= sg.n) {
      const floatx4 gv = load4<float>(sg.g + e);
#pragma unroll
      for (int r = 0; r < 4; ++r) acc += (double)gv[r] * (double)gv[r];
    } else {
      for (int64_t q = e; q < sg.n; ++q) acc += (double)sg.g[q] * (double)sg.g[q];
    }
  }
  const double tot = block_sum(acc, sh);
  if (threadIdx.x == 0) partials[L.out0 + blockIdx.x] = tot;
}

// One workgroup: thread i adds partials i, i + 256, ... in order; then the
// fixed tree; then norm and the clip coefficient.
__global__ __launch_bounds__(kBlock) void clip_finalize_kernel(const double* __restrict__ partials, int64_t nparts,
                                                               float max_norm, float* __restrict__ norm_out,
                                                               float* __restrict__ coef_out) {
  __shared__ double sh[kBlock / 64];
  double acc = 0.0;
  for (int64_t i = threadIdx.x; i < nparts; i += kBlock) acc += partials[i];
  const double tot = block_sum(acc, sh);
  if (threadIdx.x == 0) {
    const double norm = sqrt(tot);
    double coef = 1.0;
    if (max_norm > 0.0f) {
      coef = (double)max_norm / (norm + 1e-6);
      if (coef > 1.0) coef = 1.0;
    }
    if (norm_out) *norm_out = (float)norm;
    *coef_out = (float)coef;
  }
}

inline int64_t blocks_of(int64_t n) { return (n + kPerBlock - 1) / kPerBlock; }
inline int64_t sum_blocks_of(int64_t n) { return (n + kSumPerBlock - 1) / kSumPerBlock; }

}  // namespace

hipError_t launch_adamw(DType dt, const AdamwTensor* list, int count, bool master, const AdamwConst& c,
                        const float* scale, hipStream_t s) {
  KernelTimer timer("adamw", s);
  for (int first = 0; first < count; first += kMaxTensors) {
    AdamwList L{};
    int64_t blocks = 0;
    for (int i = first; i < count && i < first + kMaxTensors; ++i) {
      if (list[i].n == 0) continue;
      AdamwSeg& sg = L.seg[L.count++];
      sg.pin = list[i].param_in;
      sg.pout = list[i].param_out;
      sg.g = list[i].grad;
      sg.min = list[i].master_in;
      sg.mout = list[i].master_out;
      sg.m = list[i].m;
      sg.v = list[i].v;
      sg.n = list[i].n;
      sg.block0 = blocks;
      blocks += blocks_of(sg.n);
    }
    if (L.count == 0) continue;
    const dim3 grid((unsigned)blocks), block(kBlock);
    if (dt == kBF16) {
      if (master) hipLaunchKernelGGL((adamw_kernel<bf16_t, true>), grid, block, 0, s, L, c, scale);
      else hipLaunchKernelGGL((adamw_kernel<bf16_t, false>), grid, block, 0, s, L, c, scale);
    } else {
      hipLaunchKernelGGL((adamw_kernel<float, false>), grid, block, 0, s, L, c, scale);
    }
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

size_t sumsq_blocks(const int64_t* counts, int count) {
  int64_t b = 0;
  for (int i = 0; i < count; ++i) b += sum_blocks_of(counts[i]);
  return (size_t)b;
}

hipError_t launch_clip_grad_norm(const float* const* grads, const int64_t* counts, int count, float max_norm,
                                 float* norm_out, float* coef_out, double* ws, hipStream_t s) {
  KernelTimer timer("grad_norm", s);
  int64_t done = 0;
  for (int first = 0; first < count; first += kMaxTensors) {
    SumsqList L{};
    L.out0 = done;
    int64_t blocks = 0;
    for (int i = first; i < count && i < first + kMaxTensors; ++i) {
      if (counts[i] == 0) continue;
      SumsqSeg& sg = L.seg[L.count++];
      sg.g = grads[i];
      sg.n = counts[i];
      sg.block0 = blocks;
      blocks += sum_blocks_of(sg.n);
    }
    if (L.count == 0) continue;
    hipLaunchKernelGGL(sumsq_kernel, dim3((unsigned)blocks), dim3(kBlock), 0, s, L, ws);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    done += blocks;
  }
  hipLaunchKernelGGL(clip_finalize_kernel, dim3(1), dim3(kBlock), 0, s, ws, done, max_norm, norm_out, coef_out);
  return hipGetLastError();
}

}  // namespace tpmlp
