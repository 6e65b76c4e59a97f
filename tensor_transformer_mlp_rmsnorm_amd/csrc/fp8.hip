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

constexpr int kCastTile = 128, kCastThreads = 256;
constexpr int kCastBlocks = 512;  // workgroups a cast aims for (two per CU)

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

// LDS code tile [128 rows][32 dwords]; dword d of row r is stored at d ^ 8 (r >> 6 & 1), so
// that the column reads below (rows r and r + 64 in one instruction) fall in distinct banks.
__device__ __forceinline__ int tile_dword(int r, int d) { return r * 32 + (d ^ (((r >> 6) & 1) << 3)); }

// The 4 x 4 byte transpose of the dwords a, b, c, e (byte k of each): out[k]
// holds byte k of a, b, c, e in that order.
__device__ __forceinline__ void transpose4x4(uint32_t a, uint32_t b, uint32_t c, uint32_t e, uint32_t (&out)[4]) {
  const uint32_t ab01 = __builtin_amdgcn_perm(b, a, 0x05010400u), ab23 = __builtin_amdgcn_perm(b, a, 0x07030602u);
  const uint32_t ce01 = __builtin_amdgcn_perm(e, c, 0x05010400u), ce23 = __builtin_amdgcn_perm(e, c, 0x07030602u);
  out[0] = __builtin_amdgcn_perm(ce01, ab01, 0x05040100u);
  out[1] = __builtin_amdgcn_perm(ce01, ab01, 0x07060302u);
  out[2] = __builtin_amdgcn_perm(ce23, ab23, 0x05040100u);
  out[3] = __builtin_amdgcn_perm(ce23, ab23, 0x07060302u);
}

// Codes of a bf16 [R, C] matrix, 128 x 128 tiles over a grid-stride loop:
// out [R, C] (if ROW) and out_t [C, ldt] (if TRANS; the rows R .. ldt-1 of
// the tiles give zero codes, so out_t's padding columns are written as 0).
// Load: thread t takes rows t/8 + 32 i (i < 4) and the 16 columns 16 (t%8) ..;
// a tile wholly inside the matrix is loaded one iteration ahead, its 8 loads
// in flight while the previous tile's codes are stored, so that each
// workgroup's reads and writes overlap (edge tiles load under guards, when
// they are cast).  Transposed store: thread t reads the code dwords
// of columns 4 (t%32) .. + 3 in rows 16 (t/32) .. + 15 from LDS, transposes
// them in registers (byte permutes) and writes 16 bytes to each of the four
// columns.  One atomic maximum per workgroup folds the amax into meta[2].
template <int FMT, bool ROW, bool TRANS>
__global__ __launch_bounds__(kCastThreads) void cast_kernel(const bf16_t* __restrict__ x, int64_t R, int64_t C,
                                                            uint8_t* __restrict__ out, uint8_t* __restrict__ out_t,
                                                            int64_t ldt, int tiles_c, int tiles, float* __restrict__ meta) {
  __shared__ uint32_t tile[kCastTile * 32];
  __shared__ float red[kCastThreads / kWave];
  const int t = threadIdx.x;
  const float s = meta[0], lim = meta[3];
  const int cq = (t & 7) * 16;  // first of this thread's 16 columns
  float amax = 0.0f;
  // whether tile id lies wholly inside the matrix (the same for the whole workgroup)
  auto full_tile = [&](int id) {
    return (int64_t)(id / tiles_c + 1) * kCastTile <= R && (int64_t)(id % tiles_c + 1) * kCastTile <= C;
  };
  uint4 v[4][2];  // the raw chunks of the next full tile
  auto load_tile = [&](int id) {
    const int64_t r0 = (int64_t)(id / tiles_c) * kCastTile, c0 = (int64_t)(id % tiles_c) * kCastTile;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const bf16_t* src = x + (r0 + (t >> 3) + 32 * i) * C + c0 + cq;
      v[i][0] = *reinterpret_cast<const uint4*>(src);
      v[i][1] = *reinterpret_cast<const uint4*>(src + 8);
    }
  };
  if ((int)blockIdx.x < tiles && full_tile(blockIdx.x)) load_tile(blockIdx.x);
  for (int tid = blockIdx.x; tid < tiles; tid += gridDim.x) {
    const int64_t r0 = (int64_t)(tid / tiles_c) * kCastTile, c0 = (int64_t)(tid % tiles_c) * kCastTile;
    const bool full = full_tile(tid);
    uint2 q[4][2];
    if (full) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        q[i][0] = cast8<FMT>(v[i][0], s, lim, amax);
        q[i][1] = cast8<FMT>(v[i][1], s, lim, amax);
      }
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int64_t r = r0 + (t >> 3) + 32 * i, c = c0 + cq;
        q[i][0] = q[i][1] = make_uint2(0u, 0u);  // past R or C: zero codes
        if (r < R) {
          const bf16_t* src = x + r * C + c;
          if (c < C) q[i][0] = cast8<FMT>(*reinterpret_cast<const uint4*>(src), s, lim, amax);
          if (c + 8 < C) q[i][1] = cast8<FMT>(*reinterpret_cast<const uint4*>(src + 8), s, lim, amax);
        }
      }
    }
    const int next = tid + (int)gridDim.x;
    if (next < tiles && full_tile(next)) load_tile(next);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int rr = (t >> 3) + 32 * i;
      const int64_t r = r0 + rr, c = c0 + cq;
      if constexpr (ROW) {
        uint8_t* dst = out + r * C + c;  // 8-byte aligned (C is a multiple of 8); 16 when C is of 16
        if (full && (C & 15) == 0) {
          *reinterpret_cast<uint4*>(dst) = make_uint4(q[i][0].x, q[i][0].y, q[i][1].x, q[i][1].y);
        } else if (r < R) {
          if (c < C) *reinterpret_cast<uint2*>(dst) = q[i][0];
          if (c + 8 < C) *reinterpret_cast<uint2*>(dst + 8) = q[i][1];
        }
      }
      if constexpr (TRANS)
        *reinterpret_cast<uint4*>(&tile[tile_dword(rr, cq >> 2)]) =
            make_uint4(q[i][0].x, q[i][0].y, q[i][1].x, q[i][1].y);
    }
    if constexpr (TRANS) {
      __syncthreads();
      const int dw = t & 31, rb = t >> 5;
      uint32_t d[16];
#pragma unroll
      for (int j = 0; j < 16; ++j) d[j] = tile[tile_dword(16 * rb + j, dw)];
      uint32_t o[4][4];  // [row quad m][column k]
#pragma unroll
      for (int m = 0; m < 4; ++m) transpose4x4(d[4 * m], d[4 * m + 1], d[4 * m + 2], d[4 * m + 3], o[m]);
      const int64_t r = r0 + 16 * rb;
      if (r < ldt) {  // ldt and r are multiples of 16: the whole 16 bytes lie inside the row
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const int64_t c = c0 + 4 * dw + k;
          if (c < C) *reinterpret_cast<uint4*>(out_t + c * ldt + r) = make_uint4(o[0][k], o[1][k], o[2][k], o[3][k]);
        }
      }
      __syncthreads();  // the tile is rewritten by the next iteration
    }
  }
  amax = wave_max(amax);
  if ((t & 63) == 0) red[t >> 6] = amax;
  __syncthreads();
  if (t == 0) {
    float m = red[0];
#pragma unroll
    for (int w = 1; w < kCastThreads / kWave; ++w) m = fmaxf(m, red[w]);
    if (m > 0.0f) atomicMax(reinterpret_cast<unsigned int*>(meta + 2), __float_as_uint(m));
  }
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
  const int64_t tc = (C + kCastTile - 1) / kCastTile, tr = (rows + kCastTile - 1) / kCastTile;
  const int64_t tiles = tc * tr;
  const int64_t per_block = (tiles + kCastBlocks - 1) / kCastBlocks;  // tiles per workgroup, evened out
  const int blocks = (int)((tiles + per_block - 1) / per_block);
  hipLaunchKernelGGL((cast_kernel<FMT, ROW, TRANS>), dim3(blocks), dim3(kCastThreads), 0, s, x, R, C, out, out_t, ldt,
                     (int)tc, (int)tiles, meta);
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
