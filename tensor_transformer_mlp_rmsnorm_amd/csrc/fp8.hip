// FP8 casts and delayed-scaling metadata (gfx950 / CDNA4).
//
// FP8 training with per-tensor delayed scaling ("Megatron-Core Guide: 5D
// Distributed Training Architecture", Transformer Engine FP8 in its feature
// list): every tensor role has a meta in device memory,
//
//   meta[0] scale s         the factor a cast multiplies by (initially 1)
//   meta[1] scale_inv       1 / s, rounded to fp32 (the GEMMs' dequantisation)
//   meta[2] amax            running max|x| of this step's casts
//   meta[3] fmt_max         448 (E4M3) or 57344 (E5M2)
//   meta[4 .. 4 + L)        amax history, newest first
//
// A cast reads s, writes the codes round(clamp(fp32(x) * s, +-fmt_max)) and
// folds max|x| into meta[2] (atomic maximum on the bit pattern, which orders
// non-negative floats); the update at the end of a step pushes meta[2] into
// the history, clears it, and sets s = fmt_max / max(history) when that is
// positive and finite (otherwise s is kept).  Nothing here reads a scale on
// the host: the whole step is asynchronous.
#include "common.h"
#include "kernels.h"

namespace tpmlp {
namespace {

constexpr int kCastRows = 128, kCastCols = 64, kCastThreads = 256;
constexpr int kPadT = 16;  // LDS row padding of the transposed tile (bytes)

template <int FMT>
__device__ __forceinline__ uint32_t cvt_pair(float a, float b) {
  if constexpr (FMT == kFp8E4M3) return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false) & 0xffffu;
  else return (uint32_t)__builtin_amdgcn_cvt_pk_bf8_f32(a, b, 0, false) & 0xffffu;
}

// Codes of 8 bf16 values (one 16-byte chunk) as 8 bytes.
template <int FMT>
__device__ __forceinline__ uint2 cast8(const uint4& u, float s, float lim, float& amax) {
  float f[8];
  Chunk<bf16_t>::unpack(u, f);
  uint32_t w[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    amax = fmaxf(amax, fmaxf(fabsf(f[2 * i]), fabsf(f[2 * i + 1])));
    const float a = fminf(fmaxf(f[2 * i] * s, -lim), lim);
    const float b = fminf(fmaxf(f[2 * i + 1] * s, -lim), lim);
    w[i] = cvt_pair<FMT>(a, b);
  }
  return make_uint2(w[0] | (w[1] << 16), w[2] | (w[3] << 16));
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, kWave));
  return v;
}

// One 128 x 64 tile of a bf16 [R, C] matrix: codes to out [R, C] (if ROW) and
// to out_t [C, ldt] (if TRANS; columns R .. ldt-1 of out_t are written as 0
// by the tiles of the last tile-row).  Thread t loads rows t/8 + 32 i, chunk t%8.
template <int FMT, bool ROW, bool TRANS>
__global__ __launch_bounds__(kCastThreads) void cast_kernel(const bf16_t* __restrict__ x, int64_t R, int64_t C,
                                                            uint8_t* __restrict__ out, uint8_t* __restrict__ out_t,
                                                            int64_t ldt, float* __restrict__ meta) {
  __shared__ __align__(16) uint8_t tile_t[kCastCols][kCastRows + kPadT];  // codes, column-major
  const int t = threadIdx.x;
  const int64_t r0 = (int64_t)blockIdx.y * kCastRows, c0 = (int64_t)blockIdx.x * kCastCols;
  const float s = meta[0], lim = meta[3];
  const int cc = (t & 7) * 8;
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int rr = (t >> 3) + 32 * i;
    const int64_t r = r0 + rr, c = c0 + cc;
    uint2 q = make_uint2(0u, 0u);  // rows past R give zero codes (the transposed padding)
    if (r < R && c < C) {
      const uint4 u = *reinterpret_cast<const uint4*>(x + r * C + c);
      q = cast8<FMT>(u, s, lim, amax);
      if constexpr (ROW) *reinterpret_cast<uint2*>(out + r * C + c) = q;
    }
    if constexpr (TRANS) {
      const uint32_t w[2] = {q.x, q.y};
#pragma unroll
      for (int e = 0; e < 8; ++e) tile_t[cc + e][rr] = (uint8_t)(w[e >> 2] >> (8 * (e & 3)));
    }
  }
  if constexpr (TRANS) {
    __syncthreads();
    // thread t: column t/4, rows (t%4)*32 .. +31 of the tile -> out_t row c0 + t/4
    const int col = t >> 2, seg = (t & 3) * 32;
    const int64_t c = c0 + col, r = r0 + seg;
    if (c < C && r < ldt) {
      const uint4* src = reinterpret_cast<const uint4*>(&tile_t[col][seg]);
      uint4* dst = reinterpret_cast<uint4*>(out_t + c * ldt + r);
      dst[0] = src[0];
      if (r + 16 < ldt) dst[1] = src[1];
    }
  }
  amax = wave_max(amax);
  if ((t & 63) == 0 && amax > 0.0f) atomicMax(reinterpret_cast<unsigned int*>(meta + 2), __float_as_uint(amax));
}

// End of step for each meta: history push, amax cleared, new scale.
struct MetaList {
  float* meta[kFp8MaxMetas];
};

__global__ __launch_bounds__(256) void update_kernel(MetaList list, int L) {
  float* m = list.meta[blockIdx.x];
  float* hist = m + 4;
  const float amax = m[2];
  constexpr int kPer = kFp8MaxHistory / 256;
  float v[kPer];
  float mx = 0.0f;
  bool nonfinite = false;
#pragma unroll
  for (int j = 0; j < kPer; ++j) {
    const int i = threadIdx.x + 256 * j;
    v[j] = i < L ? (i == 0 ? amax : hist[i - 1]) : 0.0f;
    if (i < L) {
      nonfinite |= !(v[j] <= 3.402823466e38f);  // NaN or inf
      mx = fmaxf(mx, v[j]);
    }
  }
  __syncthreads();  // every old entry is read before any is overwritten
#pragma unroll
  for (int j = 0; j < kPer; ++j) {
    const int i = threadIdx.x + 256 * j;
    if (i < L) hist[i] = v[j];
  }
  __shared__ float red[4];
  __shared__ int bad[4];
  mx = wave_max(mx);
  const int anybad = __any(nonfinite) ? 1 : 0;
  if ((threadIdx.x & 63) == 0) {
    red[threadIdx.x >> 6] = mx;
    bad[threadIdx.x >> 6] = anybad;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    const float hmax = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
    const bool finite = !(bad[0] | bad[1] | bad[2] | bad[3]);
    if (finite && hmax > 0.0f) {
      const float s = m[3] / hmax;  // IEEE division (correctly rounded in HIP's default mode)
      m[0] = s;
      m[1] = 1.0f / s;
    }
    m[2] = 0.0f;
  }
}

__global__ __launch_bounds__(256) void init_kernel(float* meta, int L, float fmt_max) {
  for (int i = threadIdx.x; i < L + 4; i += 256) {
    float v = 0.0f;
    if (i == 0 || i == 1) v = 1.0f;
    else if (i == 3) v = fmt_max;
    meta[i] = v;
  }
}

template <int FMT, bool ROW, bool TRANS>
hipError_t launch_cast_t(const bf16_t* x, int64_t R, int64_t C, uint8_t* out, uint8_t* out_t, int64_t ldt,
                         float* meta, hipStream_t s) {
  const int64_t rows = TRANS ? (R > ldt ? R : ldt) : R;  // the transposed padding needs its tile-rows too
  const dim3 grid((unsigned)((C + kCastCols - 1) / kCastCols), (unsigned)((rows + kCastRows - 1) / kCastRows));
  hipLaunchKernelGGL((cast_kernel<FMT, ROW, TRANS>), grid, dim3(kCastThreads), 0, s, x, R, C, out, out_t, ldt, meta);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_fp8_cast(int fmt, const void* x, int64_t R, int64_t C, uint8_t* out, uint8_t* out_t, int64_t ldt,
                           float* meta, const char* tag, hipStream_t s) {
  if (C == 0 || (R == 0 && (out_t == nullptr || ldt == 0))) return hipSuccess;
  KernelTimer timer(tag ? tag : "fp8_cast", s);
  const bf16_t* xb = static_cast<const bf16_t*>(x);
  const bool row = out != nullptr, tr = out_t != nullptr;
  if (fmt == kFp8E4M3) {
    if (row && tr) return launch_cast_t<kFp8E4M3, true, true>(xb, R, C, out, out_t, ldt, meta, s);
    if (row) return launch_cast_t<kFp8E4M3, true, false>(xb, R, C, out, out_t, ldt, meta, s);
    if (tr) return launch_cast_t<kFp8E4M3, false, true>(xb, R, C, out, out_t, ldt, meta, s);
  } else {
    if (row && tr) return launch_cast_t<kFp8E5M2, true, true>(xb, R, C, out, out_t, ldt, meta, s);
    if (row) return launch_cast_t<kFp8E5M2, true, false>(xb, R, C, out, out_t, ldt, meta, s);
    if (tr) return launch_cast_t<kFp8E5M2, false, true>(xb, R, C, out, out_t, ldt, meta, s);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_fp8_update(float* const* metas, int count, int history_len, hipStream_t s) {
  if (count == 0) return hipSuccess;
  MetaList list{};
  for (int i = 0; i < count; ++i) list.meta[i] = metas[i];
  KernelTimer timer("fp8_scale_update", s);
  hipLaunchKernelGGL(update_kernel, dim3(count), dim3(256), 0, s, list, history_len);
  return hipGetLastError();
}

hipError_t launch_fp8_meta_init(float* meta, int fmt, int history_len, hipStream_t s) {
  hipLaunchKernelGGL(init_kernel, dim3(1), dim3(256), 0, s, meta, history_len,
                     fmt == kFp8E4M3 ? 448.0f : 57344.0f);
  return hipGetLastError();
}

}  // namespace tpmlp
