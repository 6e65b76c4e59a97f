// HBM-bound kernels around the contractions: the shard partial sum, a
// deterministic column sum, and the SGD update.
#include "common.h"
#include "kernels.h"

namespace tpmlp {

namespace {

constexpr int kMaxParts = 64;

struct PartList {
  const float* p[kMaxParts];
};

constexpr int kSgdMaxTensors = 48;
struct SgdSeg {
  const void* pin;
  void* pout;
  const float* g;
  const float* min;
  float* mout;
  int64_t n;
  int64_t block0;  // first workgroup of this tensor
};
struct SgdList {
  SgdSeg seg[kSgdMaxTensors];
  int count;
};

// out = ((p0 + p1) + ...) + residual + bias, 4 columns per thread.
// "Split the contraction" (synapticradio.com): the partial down outputs are
// summed, then the replicated residual and bias are added once.  Each partial
// is read exactly once, so its loads are non-temporal (they do not displace
// reusable lines from the caches); one 4-column group per thread, no grid-stride
// loop (the faster form on this memory system).
template <typename TI, typename TO, bool RES, bool BIAS>
__global__ __launch_bounds__(256) void partial_sum_kernel(PartList parts, int n_parts, int64_t n4, int64_t cols4,
                                                          const TI* __restrict__ residual, const TI* __restrict__ bias,
                                                          TO* __restrict__ out) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; e < n4; e += stride) {
    floatx4 acc = __builtin_nontemporal_load(reinterpret_cast<const floatx4*>(parts.p[0] + 4 * e));
    for (int k = 1; k < n_parts; ++k)
      acc += __builtin_nontemporal_load(reinterpret_cast<const floatx4*>(parts.p[k] + 4 * e));
    if constexpr (RES) acc += load4<TI>(residual + 4 * e);
    if constexpr (BIAS) acc += load4<TI>(bias + 4 * (e % cols4));
    store4<TO>(out + 4 * e, acc);
  }
}

// One work item per thread up to 2^31 - 1 workgroups; the kernels still loop
// (grid-stride) so any size is covered.
inline unsigned grid_for(int64_t n, int64_t per_block) {
  int64_t b = (n + per_block - 1) / per_block;
  const int64_t cap = 0x7fffffff;
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
  KernelTimer timer((r || b) ? "partial_sum_residual" : "partial_sum", s);
  const dim3 grid(grid_for(n4, 256)), block(256);
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
  int64_t t = r0;
  for (; t + 8 <= r1; t += 8) {  // eight loads in flight; the additions stay in row order
    floatx4 v[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) v[k] = load4<T>(in + (t + k) * cols + 4 * q);
#pragma unroll
    for (int k = 0; k < 8; ++k) acc += v[k];
  }
  for (; t < r1; ++t) acc += load4<T>(in + t * cols + 4 * q);
  store4<float>(ws + (int64_t)blockIdx.x * cols + 4 * q, acc);
}

// SGD: p <- p - lr g ("Reproduce one dense training step": one SGD update),
// over a list of parameter tensors in one launch.  Workgroup b belongs to the
// tensor whose [block0, block0 + blocks) contains b; each thread updates 8
// consecutive elements (a 16-byte bf16 or 2 x 16-byte fp32 parameter chunk).
// Out of place when pout != pin (the input is then left unchanged).
constexpr int kSgdPerThread = 8, kSgdBlock = 256, kSgdPerBlock = kSgdPerThread * kSgdBlock;

// The update of 8 consecutive elements from e (16-byte accesses throughout:
// every pointer is 16-byte aligned; the gradient is read once, with the
// non-temporal hint): v = p - lr g, or with masters m' = m - lr g (written)
// and v = m'.  Shared by the flat and the transposing kernels, so both give
// the same bits.
// The old values of the 8 elements from e: the fp32 masters, or the parameter.
template <typename T, bool MASTER>
__device__ __forceinline__ void sgd8_old(const T* pin, const float* min, int64_t e, floatx4& p0, floatx4& p1) {
  if constexpr (MASTER) {
    p0 = load4<float>(min + e);
    p1 = load4<float>(min + e + 4);
  } else if constexpr (sizeof(T) == 2) {
    float f[8];
    Chunk<bf16_t>::unpack(*reinterpret_cast<const uint4*>(pin + e), f);
    p0 = floatx4{f[0], f[1], f[2], f[3]};
    p1 = floatx4{f[4], f[5], f[6], f[7]};
  } else {
    p0 = load4<T>(pin + e);
    p1 = load4<T>(pin + e + 4);
  }
}

// The updated values v = p - lr g (with masters also stored as the new masters).
template <bool MASTER>
__device__ __forceinline__ void sgd8_new(floatx4 p0, floatx4 p1, floatx4 g0, floatx4 g1, float* mout, int64_t e,
                                         float lr, floatx4& v0, floatx4& v1) {
  v0 = sgd_value4(p0, g0, lr);
  v1 = sgd_value4(p1, g1, lr);
  if constexpr (MASTER) {
    store4<float>(mout + e, v0);
    store4<float>(mout + e + 4, v1);
  }
}

template <typename T, bool MASTER>
__device__ __forceinline__ void sgd8_apply(const T* pin, floatx4 g0, floatx4 g1, const float* min, float* mout,
                                           int64_t e, float lr, floatx4& v0, floatx4& v1) {
  floatx4 p0, p1;
  sgd8_old<T, MASTER>(pin, min, e, p0, p1);
  sgd8_new<MASTER>(p0, p1, g0, g1, mout, e, lr, v0, v1);
}

template <typename T, bool MASTER>
__device__ __forceinline__ void sgd8(const T* pin, const float* g, const float* min, float* mout, int64_t e, float lr,
                                     floatx4& v0, floatx4& v1) {
  const floatx4 g0 = __builtin_nontemporal_load(reinterpret_cast<const floatx4*>(g + e));
  const floatx4 g1 = __builtin_nontemporal_load(reinterpret_cast<const floatx4*>(g + e + 4));
  sgd8_apply<T, MASTER>(pin, g0, g1, min, mout, e, lr, v0, v1);
}

template <typename T, bool MASTER>
__global__ __launch_bounds__(kSgdBlock) void sgd_kernel(SgdList L, float lr) {
  int t = 0;
  while (t + 1 < L.count && (int64_t)blockIdx.x >= L.seg[t + 1].block0) ++t;
  const SgdSeg& sg = L.seg[t];
  const T* pin = static_cast<const T*>(sg.pin);
  T* pout = static_cast<T*>(sg.pout);
  const int64_t e0 = ((int64_t)blockIdx.x - sg.block0) * kSgdPerBlock + (int64_t)threadIdx.x * kSgdPerThread;
  if (e0 + kSgdPerThread <= sg.n) {
    floatx4 v0, v1;
    sgd8<T, MASTER>(pin, sg.g, sg.min, sg.mout, e0, lr, v0, v1);
    if constexpr (sizeof(T) == 2) {
      const float f[8] = {v0[0], v0[1], v0[2], v0[3], v1[0], v1[1], v1[2], v1[3]};
      *reinterpret_cast<uint4*>(pout + e0) = Chunk<bf16_t>::pack(f);
    } else {
      store4<T>(pout + e0, v0);
      store4<T>(pout + e0 + 4, v1);
    }
  } else {
    for (int64_t e = e0; e < sg.n; ++e) {
      float v;
      if constexpr (MASTER) {
        v = sgd_value(sg.min[e], sg.g[e], lr);
        sg.mout[e] = v;
      } else {
        v = sgd_value(Elem<T>::to_f32(pin[e]), sg.g[e], lr);
      }
      pout[e] = Elem<T>::from_f32(v);
    }
  }
}

// SGD of bf16 tensors that also receive their updated values transposed:
// the parameter seen as [rows, cols] (row-major) is updated in 64 x 64 tiles;
// each tile's new values are written row-major to pout and, through an LDS
// tile, as [cols, rows] to pout_t (the layout another contraction reads with
// its k contiguous).  The update itself is sgd8, as in sgd_kernel.
constexpr int kSgdTMaxTensors = 16, kSgdTTile = 64;
struct SgdTSeg {
  const void* pin;
  void* pout;
  void* pout_t;
  const float* g;
  const float* min;
  float* mout;
  int64_t rows, cols, tiles_c;
  int64_t block0;
};
struct SgdTList {
  SgdTSeg seg[kSgdTMaxTensors];
  int count;
};

// One 64 x 64 tile of the transposing update: each thread updates two chunks
// of 8 consecutive elements of a row (16-byte accesses, the flat kernel's
// arithmetic), stores them row-major and, as one 16-byte write, into an LDS
// tile whose rows are padded to 144 bytes; then each thread reads 8 rows x 2
// adjacent columns back with 4-byte reads and stores the two 8-element column
// chunks of the transposed copy.  Eight consecutive lanes take the 8 row
// groups of one column pair, so each wave writes whole 128-byte column
// segments.  grad8(e, g0, g1) yields the gradient of elements e .. e + 7; pt
// may be null (no transposed copy).
template <bool MASTER, class G>
__device__ __forceinline__ void sgd_t_tile(const bf16_t* pin, bf16_t* pout, bf16_t* pt, const float* min, float* mout,
                                           int64_t rows, int64_t cols, int64_t r0, int64_t c0, float lr,
                                           const G& grad8) {
  __shared__ __align__(16) bf16_t tile[kSgdTTile][kSgdTTile + 8];
  // 64 rows x 8 chunks of 8 columns, two chunks per thread (rows and cols are multiples of 8).  Both
  // chunks' loads are issued before any store (a store could alias a later load as far as the
  // compiler knows, so interleaving them would leave one chunk's loads in flight at a time).
  floatx4 g[2][2], p[2][2];
  bool ok[2];
  int64_t e[2];
#pragma unroll
  for (int pass = 0; pass < 2; ++pass) {
    const int ch = threadIdx.x + 256 * pass, row = ch >> 3, col8 = (ch & 7) * 8;
    const int64_t gr = r0 + row, gc = c0 + col8;
    ok[pass] = gr < rows && gc < cols;
    e[pass] = gr * cols + gc;
    if (ok[pass]) {
      grad8(e[pass], g[pass][0], g[pass][1]);
      sgd8_old<bf16_t, MASTER>(pin, min, e[pass], p[pass][0], p[pass][1]);
    }
  }
#pragma unroll
  for (int pass = 0; pass < 2; ++pass) {
    const int ch = threadIdx.x + 256 * pass, row = ch >> 3, col8 = (ch & 7) * 8;
    if (ok[pass]) {
      floatx4 v0, v1;
      sgd8_new<MASTER>(p[pass][0], p[pass][1], g[pass][0], g[pass][1], mout, e[pass], lr, v0, v1);
      const float f[8] = {v0[0], v0[1], v0[2], v0[3], v1[0], v1[1], v1[2], v1[3]};
      const uint4 u = Chunk<bf16_t>::pack(f);
      *reinterpret_cast<uint4*>(pout + e[pass]) = u;
      *reinterpret_cast<uint4*>(&tile[row][col8]) = u;
    }
  }
  if (!pt) return;  // (uniform over the workgroup)
  __syncthreads();
  const int c = 2 * (threadIdx.x >> 3), rr = 8 * (threadIdx.x & 7);
  const int64_t gc = c0 + c, gr = r0 + rr;
  if (gc < cols && gr < rows) {  // (cols and rows are multiples of 8: the pair and the 8 rows are whole)
    uint32_t w[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) w[i] = *reinterpret_cast<const uint32_t*>(&tile[rr + i][c]);
    uint32_t lo[4], hi[4];  // column c (low halves) and column c + 1 (high halves), rows rr .. rr + 7
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      lo[i] = (w[2 * i] & 0xffffu) | (w[2 * i + 1] << 16);
      hi[i] = (w[2 * i] >> 16) | (w[2 * i + 1] & 0xffff0000u);
    }
    *reinterpret_cast<uint4*>(pt + gc * rows + gr) = make_uint4(lo[0], lo[1], lo[2], lo[3]);
    *reinterpret_cast<uint4*>(pt + (gc + 1) * rows + gr) = make_uint4(hi[0], hi[1], hi[2], hi[3]);
  }
}

template <bool MASTER>
__global__ __launch_bounds__(256) void sgd_t_kernel(SgdTList L, float lr) {
  int t = 0;
  while (t + 1 < L.count && (int64_t)blockIdx.x >= L.seg[t + 1].block0) ++t;
  const SgdTSeg& sg = L.seg[t];
  const int64_t b = (int64_t)blockIdx.x - sg.block0;
  const int64_t r0 = (b / sg.tiles_c) * kSgdTTile, c0 = (b % sg.tiles_c) * kSgdTTile;
  const float* grad = sg.g;
  sgd_t_tile<MASTER>(static_cast<const bf16_t*>(sg.pin), static_cast<bf16_t*>(sg.pout),
                     static_cast<bf16_t*>(sg.pout_t), sg.min, sg.mout, sg.rows, sg.cols, r0, c0, lr,
                     [grad](int64_t e, floatx4& g0, floatx4& g1) {
                       g0 = __builtin_nontemporal_load(reinterpret_cast<const floatx4*>(grad + e));
                       g1 = __builtin_nontemporal_load(reinterpret_cast<const floatx4*>(grad + e + 4));
                     });
}

// The update of one weight whose gradient is the sum of a split GEMM's
// k-slices, ((s0 + s1) + s2) + ..., the order of ksplit_reduce_kernel, so the
// gradient has the bits the unfused path stores (and then reads back).
template <bool MASTER>
__global__ __launch_bounds__(256) void sgd_ksplit_kernel(SgdEpi u, const float* __restrict__ ws, int nslices,
                                                         int64_t rows, int64_t cols, int64_t tiles_c) {
  const int64_t b = blockIdx.x;
  const int64_t r0 = (b / tiles_c) * kSgdTTile, c0 = (b % tiles_c) * kSgdTTile;
  const int64_t slice = rows * cols;
  sgd_t_tile<MASTER>(static_cast<const bf16_t*>(u.w_in), static_cast<bf16_t*>(u.w_out),
                     static_cast<bf16_t*>(u.w_out_t), u.m_in, u.m_out, rows, cols, r0, c0, u.lr,
                     [ws, nslices, slice](int64_t e, floatx4& g0, floatx4& g1) {
                       g0 = __builtin_nontemporal_load(reinterpret_cast<const floatx4*>(ws + e));
                       g1 = __builtin_nontemporal_load(reinterpret_cast<const floatx4*>(ws + e + 4));
                       for (int k = 1; k < nslices; ++k) {
                         const float* p = ws + (int64_t)k * slice + e;
                         g0 += __builtin_nontemporal_load(reinterpret_cast<const floatx4*>(p));
                         g1 += __builtin_nontemporal_load(reinterpret_cast<const floatx4*>(p + 4));
                       }
                     });
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

// C (bf16) = the sum of nslices fp32 slices [M, N] (row length N) in index order.
__global__ __launch_bounds__(256) void ksplit_reduce_bf16_kernel(bf16_t* __restrict__ C, const float* __restrict__ ws,
                                                                  int nslices, int64_t M, int64_t N4, int64_t ldc) {
  const int64_t total = M * N4, stride = (int64_t)gridDim.x * blockDim.x, slice = M * N4 * 4;
  for (int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; e < total; e += stride) {
    const int64_t m = e / N4, n = 4 * (e - m * N4);
    const float* src = ws + m * N4 * 4 + n;
    floatx4 acc = load4<float>(src);
    for (int s = 1; s < nslices; ++s) acc += load4<float>(src + (int64_t)s * slice);
    store4<bf16_t>(C + m * ldc + n, acc);
  }
}

// out[c, r] = in[r, c] for a row-major [R, C] bf16 matrix (R, C multiples of
// 8) through 64 x 64 LDS tiles, 16-byte loads along C and 16-byte stores
// along R.  With a row pitch of 33 dwords the 8 rows that one store gathers
// (of one column) sit on distinct banks across a wave.
constexpr int kTrTile = 64;
// out [C, R] = in [R, C]^T in 64 x 64 tiles: each thread loads two 16-byte row
// chunks into an LDS tile whose rows are padded to 144 bytes, then reads 8
// rows x 2 adjacent columns back with 4-byte reads and stores the two
// 8-element column chunks (eight consecutive lanes cover one column pair, so
// each wave writes whole 128-byte segments): the transposed store of
// sgd_t_tile.  R and C are multiples of 8.
__global__ __launch_bounds__(256) void transpose_bf16_kernel(const bf16_t* __restrict__ in, bf16_t* __restrict__ out,
                                                              int64_t R, int64_t C, int tiles_c) {
  __shared__ __align__(16) bf16_t tile[kTrTile][kTrTile + 8];
  const int64_t r0 = (int64_t)(blockIdx.x / tiles_c) * kTrTile, c0 = (int64_t)(blockIdx.x % tiles_c) * kTrTile;
  uint4 v[2];
#pragma unroll
  for (int pass = 0; pass < 2; ++pass) {  // both loads issued before either LDS store
    const int ch = threadIdx.x + 256 * pass, row = ch >> 3, col8 = (ch & 7) * 8;
    v[pass] = (r0 + row < R && c0 + col8 < C) ? *reinterpret_cast<const uint4*>(in + (r0 + row) * C + c0 + col8)
                                              : make_uint4(0, 0, 0, 0);
  }
#pragma unroll
  for (int pass = 0; pass < 2; ++pass) {
    const int ch = threadIdx.x + 256 * pass, row = ch >> 3, col8 = (ch & 7) * 8;
    *reinterpret_cast<uint4*>(&tile[row][col8]) = v[pass];
  }
  __syncthreads();
  const int c = 2 * (threadIdx.x >> 3), rr = 8 * (threadIdx.x & 7);
  const int64_t gc = c0 + c, gr = r0 + rr;
  if (gc < C && gr < R) {
    uint32_t w[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) w[i] = *reinterpret_cast<const uint32_t*>(&tile[rr + i][c]);
    uint32_t lo[4], hi[4];  // column c (low halves) and column c + 1 (high halves), rows rr .. rr + 7
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      lo[i] = (w[2 * i] & 0xffffu) | (w[2 * i + 1] << 16);
      hi[i] = (w[2 * i] >> 16) | (w[2 * i + 1] & 0xffff0000u);
    }
    *reinterpret_cast<uint4*>(out + gc * R + gr) = make_uint4(lo[0], lo[1], lo[2], lo[3]);
    *reinterpret_cast<uint4*>(out + (gc + 1) * R + gr) = make_uint4(hi[0], hi[1], hi[2], hi[3]);
  }
}

}  // namespace

hipError_t launch_ksplit_reduce_bf16(void* C, const float* ws, int nslices, int64_t M, int64_t N, int64_t ldc,
                                     hipStream_t s) {
  if (M == 0 || N == 0) return hipSuccess;
  KernelTimer timer("ksplit_reduce_bf16", s);
  hipLaunchKernelGGL(ksplit_reduce_bf16_kernel, dim3(grid_for(M * N / 4, 256)), dim3(256), 0, s,
                     static_cast<bf16_t*>(C), ws, nslices, M, N / 4, ldc);
  return hipGetLastError();
}

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

hipError_t launch_colsum(DType dt, const void* in, float* out, void* ws, int64_t rows, int64_t cols, bool accum,
                         hipStream_t s) {
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
  return launch_reduce_partial_rows(w, out, nb, cols, accum, s);
}

hipError_t launch_sgd(DType dt, const SgdTensor* list, int count, bool master, float lr, hipStream_t s) {
  KernelTimer timer("sgd", s);
  // Each launch takes the next (up to) kSgdMaxTensors non-empty tensors of the
  // list that have no transposed copy, so every tensor is updated exactly once.
  for (int i = 0; i < count;) {
    SgdList L{};
    int64_t blocks = 0;
    for (; i < count && L.count < kSgdMaxTensors; ++i) {
      if (list[i].n == 0 || list[i].param_out_t) continue;
      SgdSeg& sg = L.seg[L.count++];
      sg.pin = list[i].param_in;
      sg.pout = list[i].param_out;
      sg.g = list[i].grad;
      sg.min = list[i].master_in;
      sg.mout = list[i].master_out;
      sg.n = list[i].n;
      sg.block0 = blocks;
      blocks += (sg.n + kSgdPerBlock - 1) / kSgdPerBlock;
    }
    if (L.count == 0) break;
    if (dt == kBF16) {
      if (master) hipLaunchKernelGGL((sgd_kernel<bf16_t, true>), dim3((unsigned)blocks), dim3(kSgdBlock), 0, s, L, lr);
      else hipLaunchKernelGGL((sgd_kernel<bf16_t, false>), dim3((unsigned)blocks), dim3(kSgdBlock), 0, s, L, lr);
    } else {
      hipLaunchKernelGGL((sgd_kernel<float, false>), dim3((unsigned)blocks), dim3(kSgdBlock), 0, s, L, lr);
    }
    const hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
  }
  // Then the tensors with a transposed copy (bf16), up to kSgdTMaxTensors per launch.
  for (int i = 0; i < count;) {
    SgdTList L{};
    int64_t blocks = 0;
    for (; i < count && L.count < kSgdTMaxTensors; ++i) {
      if (list[i].n == 0 || !list[i].param_out_t) continue;
      if (dt != kBF16) return hipErrorInvalidValue;
      SgdTSeg& sg = L.seg[L.count++];
      sg.pin = list[i].param_in;
      sg.pout = list[i].param_out;
      sg.pout_t = list[i].param_out_t;
      sg.g = list[i].grad;
      sg.min = list[i].master_in;
      sg.mout = list[i].master_out;
      sg.rows = list[i].t_rows;
      sg.cols = list[i].t_cols;
      sg.tiles_c = (sg.cols + kSgdTTile - 1) / kSgdTTile;
      sg.block0 = blocks;
      blocks += ((sg.rows + kSgdTTile - 1) / kSgdTTile) * sg.tiles_c;
    }
    if (L.count == 0) break;
    if (master) hipLaunchKernelGGL((sgd_t_kernel<true>), dim3((unsigned)blocks), dim3(256), 0, s, L, lr);
    else hipLaunchKernelGGL((sgd_t_kernel<false>), dim3((unsigned)blocks), dim3(256), 0, s, L, lr);
    const hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
  }
  return hipSuccess;
}

hipError_t launch_sgd_ksplit(const SgdEpi& u, const float* ws, int nslices, int64_t M, int64_t N, hipStream_t s) {
  if (M == 0 || N == 0) return hipSuccess;
  if (M % 8 || N % 8 || nslices < 1) return hipErrorInvalidValue;
  KernelTimer timer("sgd_ksplit", s);
  const int64_t tr = (M + kSgdTTile - 1) / kSgdTTile, tc = (N + kSgdTTile - 1) / kSgdTTile;
  if (u.m_in)
    hipLaunchKernelGGL(sgd_ksplit_kernel<true>, dim3((unsigned)(tr * tc)), dim3(256), 0, s, u, ws, nslices, M, N, tc);
  else
    hipLaunchKernelGGL(sgd_ksplit_kernel<false>, dim3((unsigned)(tr * tc)), dim3(256), 0, s, u, ws, nslices, M, N, tc);
  return hipGetLastError();
}

hipError_t launch_transpose_bf16(const void* in, void* out, int64_t R, int64_t C, hipStream_t s) {
  if (R == 0 || C == 0) return hipSuccess;
  if (R % 8 || C % 8) return hipErrorInvalidValue;
  KernelTimer timer("transpose_bf16", s);
  const int64_t tr = (R + kTrTile - 1) / kTrTile, tc = (C + kTrTile - 1) / kTrTile;
  hipLaunchKernelGGL(transpose_bf16_kernel, dim3((unsigned)(tr * tc)), dim3(256), 0, s,
                     static_cast<const bf16_t*>(in), static_cast<bf16_t*>(out), R, C, (int)tc);
  return hipGetLastError();
}

}  // namespace tpmlp
