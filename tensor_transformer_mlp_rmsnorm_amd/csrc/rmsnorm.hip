// RMSNorm forward and backward (+ residual) of the pre-norm MLP sublayer.
//
// Forward  ("Start with the dense block", synapticradio.com: N = rms_norm(x, norm_weight)):
//   rstd_t = 1 / sqrt(mean_i x_ti^2 + eps),   N_ti = x_ti rstd_t w_i
// Backward ("Put the other collective in backward": the summed dN goes
// through RMSNorm's backward and into the residual input; the sum of the
// shards' partials can be formed here, as the rows are read):
//   c_t   = (1/H) sum_i dN_ti w_i x_ti
//   dx_ti = dY_ti + rstd_t dN_ti w_i - x_ti rstd_t^3 c_t
//   dw_i  = sum_t dN_ti x_ti rstd_t,   db_i = sum_t dY_ti
// Both are HBM-bound.  The forward reads each row once (one wavefront per
// row, the row held in registers, the next row loading meanwhile) and writes
// N and rstd.  The backward
// streams dN (fp32), x and dY once, writes dx, and reduces the two column
// sums deterministically: each workgroup owns a fixed set of rows (every
// G-th row, G workgroups) and fixed columns per thread, writes one partial
// row, and a second kernel sums the partial rows in index order.
#include "common.h"
#include "kernels.h"

namespace tpmlp {
namespace {

// 16 bytes read with the non-temporal hint (data read once: it need not stay
// in the caches).
typedef unsigned u32x4_nt __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 load_nt16(const void* p) {
  const u32x4_nt v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_nt*>(p));
  return make_uint4(v[0], v[1], v[2], v[3]);
}
// Loads are issued unconditionally from a clamped index and the values of
// lanes past the row end zeroed afterwards, so no load sits in a branch (the
// compiler would wait for each one before leaving it).
__device__ __forceinline__ int clampi(int i, int n) { return i < n ? i : n - 1; }
__device__ __forceinline__ uint4 masked16(uint4 v, bool ok) { return ok ? v : make_uint4(0, 0, 0, 0); }
__device__ __forceinline__ floatx4 masked4(floatx4 v, bool ok) { return ok ? v : floatx4{0.f, 0.f, 0.f, 0.f}; }

// Four consecutive elements as they come from memory, and their fp32 values.
template <typename T>
struct RawVec;
template <>
struct RawVec<float> {
  using type = floatx4;
  static __device__ __forceinline__ type load(const float* p) { return *reinterpret_cast<const floatx4*>(p); }
  static __device__ __forceinline__ floatx4 value(type v) { return v; }
};
template <>
struct RawVec<bf16_t> {
  using type = uint2;
  static __device__ __forceinline__ type load(const bf16_t* p) { return *reinterpret_cast<const uint2*>(p); }
  static __device__ __forceinline__ floatx4 value(type u) {
    return floatx4{__uint_as_float(u.x << 16), __uint_as_float(u.x & 0xffff0000u), __uint_as_float(u.y << 16),
                   __uint_as_float(u.y & 0xffff0000u)};
  }
};

// Forward: one wave per row, 4 waves per workgroup, each wave taking rows
// w, w + 4, w + 8, w + 12 of the workgroup's 16; the norm weight is read once
// per wave and the next row is loaded while the current one is reduced.
constexpr int kFwdWaves = 4, kFwdRowsPerWave = 1, kFwdRowsPerBlock = kFwdWaves * kFwdRowsPerWave;

// FULL: the row is exactly NC chunks per lane (no lane past its end), so no
// access needs a guard.
template <typename T, int NC, bool FULL>
__global__ __launch_bounds__(256) void rmsnorm_fwd_kernel(const T* __restrict__ x, const T* __restrict__ w,
                                                          T* __restrict__ n, float* __restrict__ rstd,
                                                          int64_t rows, int H, float eps) {
  constexpr int E = Elem<T>::kPerChunk;
  // Rows of up to 4096 bf16 (2048 fp32) keep the weight and the next row in
  // registers too (two row buffers used in turn, so no register copy waits
  // for a load); wider rows reload the weight and load one row at a time.
  constexpr bool kPf = NC <= 8;
  constexpr int NB = kPf ? 2 : 1;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t row0 = (int64_t)blockIdx.x * kFwdRowsPerBlock + wave;
  if (row0 >= rows) return;
  const int nch = H / E;
  uint4 wv[kPf ? NC : 1], v[NB][NC];
  auto load_row = [&](int64_t row, uint4* dst) {
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      const int idx = lane + 64 * c;
      dst[c] = FULL ? load_nt16(x + row * H + (int64_t)idx * E)
                    : masked16(load_nt16(x + row * H + (int64_t)clampi(idx, nch) * E), idx < nch);
    }
  };
  load_row(row0, v[0]);
  if constexpr (kPf) {
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      const int idx = lane + 64 * c;
      wv[c] = FULL ? *reinterpret_cast<const uint4*>(w + (int64_t)idx * E)
                   : masked16(*reinterpret_cast<const uint4*>(w + (int64_t)clampi(idx, nch) * E), idx < nch);
    }
  }
#pragma unroll
  for (int i = 0; i < kFwdRowsPerWave; ++i) {
    const int64_t row = row0 + (int64_t)kFwdWaves * i;
    if (row >= rows) break;
    const int64_t next = row + kFwdWaves;
    uint4* cur = v[kPf ? (i & 1) : 0];
    if (kPf && i + 1 < kFwdRowsPerWave && next < rows) load_row(next, v[(i + 1) & (NB - 1)]);
    float ss = 0.f;
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      float f[E];
      Chunk<T>::unpack(cur[c], f);
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
      if (!FULL && idx >= nch) continue;
      float f[E], wf[E];
      Chunk<T>::unpack(cur[c], f);
      if constexpr (kPf) Chunk<T>::unpack(wv[c], wf);
      else Chunk<T>::unpack(*reinterpret_cast<const uint4*>(w + (int64_t)idx * E), wf);
#pragma unroll
      for (int e = 0; e < E; ++e) f[e] = f[e] * r * wf[e];
      *reinterpret_cast<uint4*>(nr + (int64_t)idx * E) = Chunk<T>::pack(f);
    }
    if (!kPf && i + 1 < kFwdRowsPerWave && next < rows) load_row(next, v[0]);
  }
}

// Rows wider than 16 chunks per lane (bf16 rows over 8192 columns, fp32 over
// 4096; held in registers they would spill): one wave per row in two passes
// over the row (sum of squares, then the scaled store), re-reading x.
template <typename T>
__global__ __launch_bounds__(256) void rmsnorm_fwd_loop_kernel(const T* __restrict__ x, const T* __restrict__ w,
                                                               T* __restrict__ n, float* __restrict__ rstd,
                                                               int64_t rows, int H, float eps) {
  constexpr int E = Elem<T>::kPerChunk;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t row = (int64_t)blockIdx.x * 4 + wave;
  if (row >= rows) return;
  const int nch = H / E;
  const T* xr = x + row * H;
  float ss = 0.f;
  for (int c = lane; c < nch; c += 64) {
    float f[E];
    Chunk<T>::unpack(*reinterpret_cast<const uint4*>(xr + (int64_t)c * E), f);
#pragma unroll
    for (int e = 0; e < E; ++e) ss += f[e] * f[e];
  }
  ss = wave_sum(ss);
  const float r = 1.0f / sqrtf(ss / (float)H + eps);
  if (lane == 0) rstd[row] = r;
  T* nr = n + row * H;
  for (int c = lane; c < nch; c += 64) {
    float f[E], wf[E];
    Chunk<T>::unpack(*reinterpret_cast<const uint4*>(xr + (int64_t)c * E), f);
    Chunk<T>::unpack(*reinterpret_cast<const uint4*>(w + (int64_t)c * E), wf);
#pragma unroll
    for (int e = 0; e < E; ++e) f[e] = f[e] * r * wf[e];
    *reinterpret_cast<uint4*>(nr + (int64_t)c * E) = Chunk<T>::pack(f);
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
#define TPMLP_FWD(NC)                                                                                      \
  if (nch == 64 * (NC))                                                                                      \
    hipLaunchKernelGGL((rmsnorm_fwd_kernel<T, NC, true>), grid, dim3(256), 0, s, xp, wp, np_, rstd, T_, (int)H, \
                       eps);                                                                                 \
  else                                                                                                       \
    hipLaunchKernelGGL((rmsnorm_fwd_kernel<T, NC, false>), grid, dim3(256), 0, s, xp, wp, np_, rstd, T_,      \
                       (int)H, eps)
  if (per_lane <= 1) {
    TPMLP_FWD(1);
  } else if (per_lane <= 2) {
    TPMLP_FWD(2);
  } else if (per_lane <= 4) {
    TPMLP_FWD(4);
  } else if (per_lane <= 8) {
    TPMLP_FWD(8);
  } else if (per_lane <= 16) {
    TPMLP_FWD(16);
  } else {
    hipLaunchKernelGGL(rmsnorm_fwd_loop_kernel<T>, dim3((unsigned)((T_ + 3) / 4)), dim3(256), 0, s, xp, wp, np_, rstd,
                       T_, (int)H, eps);
  }
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

// The gradient of N as shard partials summed inside the backward ("Put the
// other collective in backward": the shards' partials are summed before
// RMSNorm's backward; here the sum is streamed into it instead of written out
// and read back): dN = ((p[0] + p[1]) + p[2]) + ..., fp32, in index order --
// the order of the partial-sum kernel, so both forms give the same bits.
struct NormParts {
  const float* p[kMaxNormParts];
  int n;
};

// The dN units of one row: NP > 0 parts known at compile time (every part's
// loads issued before the first addition), NP = 0 any count (one part's loads
// at a time).
template <int NP, int UPT, bool FULL>
__device__ __forceinline__ void load_dn(const NormParts& parts, int64_t row, int H, int tid, int nunits,
                                        floatx4 (&dn)[UPT]) {
  if constexpr (NP > 0) {
    floatx4 v[NP][UPT];
#pragma unroll
    for (int k = 0; k < NP; ++k)
#pragma unroll
      for (int u = 0; u < UPT; ++u) {
        const int q = tid + kBwdThreads * u;
        const int64_t off = row * H + 4 * (FULL ? q : clampi(q, nunits));
        v[k][u] = masked4(__builtin_nontemporal_load(reinterpret_cast<const floatx4*>(parts.p[k] + off)),
                          FULL || q < nunits);
      }
#pragma unroll
    for (int u = 0; u < UPT; ++u) {
      floatx4 acc = v[0][u];
#pragma unroll
      for (int k = 1; k < NP; ++k) acc += v[k][u];
      dn[u] = acc;
    }
  } else {
#pragma unroll
    for (int u = 0; u < UPT; ++u) {
      const int q = tid + kBwdThreads * u;
      const int64_t off = row * H + 4 * (FULL ? q : clampi(q, nunits));
      dn[u] = masked4(__builtin_nontemporal_load(reinterpret_cast<const floatx4*>(parts.p[0] + off)), FULL || q < nunits);
    }
    for (int k = 1; k < parts.n; ++k) {
      floatx4 v[UPT];
#pragma unroll
      for (int u = 0; u < UPT; ++u) {
        const int q = tid + kBwdThreads * u;
        const int64_t off = row * H + 4 * (FULL ? q : clampi(q, nunits));
        v[u] = masked4(__builtin_nontemporal_load(reinterpret_cast<const floatx4*>(parts.p[k] + off)), FULL || q < nunits);
      }
#pragma unroll
      for (int u = 0; u < UPT; ++u) dn[u] += v[u];
    }
  }
}

// FULL: every thread's UPT units lie inside the row (no guards needed).
template <typename T, int UPT, bool FULL, int NP>
__global__ __launch_bounds__(kBwdThreads) void rmsnorm_bwd_kernel(
    const NormParts parts, const T* __restrict__ x, const T* __restrict__ dY,
    const float* __restrict__ rstd, const T* __restrict__ w, T* __restrict__ dx, float* __restrict__ ws_dw,
    float* __restrict__ ws_db, int64_t rows, int H, int64_t rows_per_block) {
  __shared__ float red[2][2][kBwdThreads / 64];  // [slot][row of the pair][wave]
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int nunits = H / 4;  // 4 columns per unit
  // Workgroup b takes rows b, b + G, b + 2G, ... (G workgroups): at any time
  // the workgroups work on neighbouring rows, so the GPU sweeps each tensor
  // front to back (a fixed assignment, so the column sums' order is fixed).
  const int64_t G = gridDim.x;
  floatx4 wv[UPT], dwa[UPT], dba[UPT];
#pragma unroll
  for (int u = 0; u < UPT; ++u) {
    const int q = tid + kBwdThreads * u;
    wv[u] = FULL ? load4<T>(w + 4 * q) : masked4(load4<T>(w + 4 * clampi(q, nunits)), q < nunits);
    dwa[u] = floatx4{0.f, 0.f, 0.f, 0.f};
    dba[u] = floatx4{0.f, 0.f, 0.f, 0.f};
  }
  const float invH = 1.0f / (float)H;
  // Rows go two at a time (one at a time for wide rows and for summed
  // partials): both rows' loads are issued together, the two row sums share
  // one barrier (which waits only for LDS), then both dx rows are written.
  constexpr int NR = (UPT <= 4 && NP == 1) ? 2 : 1;
  int64_t it = 0;
  for (int64_t t = blockIdx.x; t < rows; t += NR * G, ++it) {
    floatx4 dn[NR][UPT], xv[NR][UPT], dy[NR][UPT];
    float r[NR], part[NR];
#pragma unroll
    for (int k = 0; k < NR; ++k) {
      const int64_t tk = t + k * G < rows ? t + k * G : t;  // a missing second row repeats the first (not written)
      r[k] = rstd[tk];
#pragma unroll
      for (int u = 0; u < UPT; ++u) {
        const int q = tid + kBwdThreads * u;
        const bool ok = FULL || q < nunits;
        const int64_t off = tk * H + 4 * (FULL ? q : clampi(q, nunits));
        xv[k][u] = masked4(load4<T>(x + off), ok);
        dy[k][u] = masked4(load4<T>(dY + off), ok);
      }
      load_dn<NP, UPT, FULL>(parts, tk, H, tid, nunits, dn[k]);
    }
    __builtin_amdgcn_sched_barrier(0);  // every load of the pair is issued before any use
#pragma unroll
    for (int k = 0; k < NR; ++k) {
      float pk = 0.f;
#pragma unroll
      for (int u = 0; u < UPT; ++u) {
        const floatx4 p = dn[k][u] * wv[u] * xv[k][u];
        pk += (p[0] + p[1]) + (p[2] + p[3]);
      }
      part[k] = wave_sum(pk);
    }
    const int slot = (int)(it & 1);
    if (lane == 0) {
#pragma unroll
      for (int k = 0; k < NR; ++k) red[slot][k][wave] = part[k];
    }
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
#pragma unroll
    for (int k = 0; k < NR; ++k) {
      if (t + k * G >= rows) break;
      float c = 0.f;
#pragma unroll
      for (int i = 0; i < kBwdThreads / 64; ++i) c += red[slot][k][i];
      c *= invH;
      const float r3c = r[k] * r[k] * r[k] * c;
#pragma unroll
      for (int u = 0; u < UPT; ++u) {
        const int q = tid + kBwdThreads * u;
        if (!FULL && q >= nunits) continue;
        const floatx4 d = dy[k][u] + r[k] * dn[k][u] * wv[u] - xv[k][u] * r3c;
        store4<T>(dx + (t + k * G) * H + 4 * q, d);
        dwa[u] += dn[k][u] * xv[k][u] * r[k];
        dba[u] += dy[k][u];
      }
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

// The backward with NP > 1 shard partials, software-pipelined over its rows:
// the loads of row t + G (NP partials, x, dY) are issued before row t's
// reduction, barrier, dx stores and column accumulation, so the next row's
// reads are in flight while the current one is finished.  The issue sits in
// the loop body with no branch around it (the last row is finished after the
// loop): the compiler waits for every load issued inside a branch before
// leaving it, which would take the overlap away.  Partials are summed in index
// order as soon as they land.  The running column sums of dw and db live in
// LDS; each thread reads and writes only its own slots, in row order.
template <typename T, int UPT, bool FULL, int NP>
__global__ __launch_bounds__(kBwdThreads) void rmsnorm_bwd_parts_kernel(
    const NormParts parts, const T* __restrict__ x, const T* __restrict__ dY, const float* __restrict__ rstd,
    const T* __restrict__ w, T* __restrict__ dx, float* __restrict__ ws_dw, float* __restrict__ ws_db, int64_t rows,
    int H, int64_t rows_per_block) {
  static_assert(NP > 1, "the single-partial backward is rmsnorm_bwd_kernel");
  __shared__ float red[2][kBwdThreads / 64];
  __shared__ floatx4 col_dw[UPT][kBwdThreads], col_db[UPT][kBwdThreads];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int nunits = H / 4;
  const int64_t G = gridDim.x;  // rows b, b + G, ... as in rmsnorm_bwd_kernel
  floatx4 wv[UPT];
#pragma unroll
  for (int u = 0; u < UPT; ++u) {
    const int q = tid + kBwdThreads * u;
    wv[u] = FULL ? load4<T>(w + 4 * q) : masked4(load4<T>(w + 4 * clampi(q, nunits)), q < nunits);
    col_dw[u][tid] = floatx4{0.f, 0.f, 0.f, 0.f};
    col_db[u][tid] = floatx4{0.f, 0.f, 0.f, 0.f};
  }
  const float invH = 1.0f / (float)H;
  // The row in flight, as loaded: the loop carries these registers unchanged
  // until the row is taken (a conversion or mask at the load would make the
  // compiler wait for the load where it sits).
  using Raw = typename RawVec<T>::type;
  floatx4 pv[NP][UPT];
  Raw xn[UPT], dyn[UPT];
  // Row t's loads.  The row's base is uniform over the workgroup and a lane's
  // column offset is one 32-bit value shared by every tensor it reads.
  auto issue = [&](int64_t t) {
    const int64_t ro = t * H;
#pragma unroll
    for (int u = 0; u < UPT; ++u) {
      const int q = tid + kBwdThreads * u;
      const uint32_t c = 4u * (uint32_t)(FULL ? q : clampi(q, nunits));
#pragma unroll
      for (int k = 0; k < NP; ++k)
        pv[k][u] = __builtin_nontemporal_load(reinterpret_cast<const floatx4*>((parts.p[k] + ro) + c));
      xn[u] = RawVec<T>::load((x + ro) + c);
      dyn[u] = RawVec<T>::load((dY + ro) + c);
    }
  };
  // dN of the row in flight, in index order, with its x and dY (units past the
  // row's end read a clamped address and are zeroed here).
  auto take = [&](floatx4 (&dn)[UPT], floatx4 (&xv)[UPT], floatx4 (&dy)[UPT]) {
#pragma unroll
    for (int u = 0; u < UPT; ++u) {
      const bool ok = FULL || tid + kBwdThreads * u < nunits;
      floatx4 acc = pv[0][u];
#pragma unroll
      for (int k = 1; k < NP; ++k) acc += pv[k][u];
      dn[u] = masked4(acc, ok);
      xv[u] = masked4(RawVec<T>::value(xn[u]), ok);
      dy[u] = masked4(RawVec<T>::value(dyn[u]), ok);
      // the converted values exist here, so the loaded registers are free for the next row
      // (otherwise the conversion sinks to its use and the loop carries copies of the loads)
      asm volatile("" : "+v"(dn[u]), "+v"(xv[u]), "+v"(dy[u]));
    }
  };
  // Row t's reduction, dx and column sums.
  auto finish = [&](int64_t t, int slot, float r, const floatx4 (&dn)[UPT], const floatx4 (&xv)[UPT],
                    const floatx4 (&dy)[UPT]) {
    float pk = 0.f;
#pragma unroll
    for (int u = 0; u < UPT; ++u) {
      const floatx4 p = dn[u] * wv[u] * xv[u];
      pk += (p[0] + p[1]) + (p[2] + p[3]);
    }
    pk = wave_sum(pk);
    if (lane == 0) red[slot][wave] = pk;
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    float c = 0.f;
#pragma unroll
    for (int i = 0; i < kBwdThreads / 64; ++i) c += red[slot][i];
    c *= invH;
    const float r3c = r * r * r * c;
#pragma unroll
    for (int u = 0; u < UPT; ++u) {
      const int q = tid + kBwdThreads * u;
      if (!FULL && q >= nunits) continue;
      const floatx4 d = dy[u] + r * dn[u] * wv[u] - xv[u] * r3c;
      store4<T>((dx + t * H) + 4u * (uint32_t)q, d);
      col_dw[u][tid] += dn[u] * xv[u] * r;
      col_db[u][tid] += dy[u];
    }
  };
  int64_t t = blockIdx.x, it = 0;
  if (t < rows) {  // (no rows: the partial column sums are zero)
    issue(t);
    for (; t + G < rows; t += G, ++it) {
      floatx4 dn[UPT], xv[UPT], dy[UPT];
      take(dn, xv, dy);
      const float r = rstd[t];
      __builtin_amdgcn_sched_barrier(0);  // this row's partials are summed before their registers take the next row
      issue(t + G);
      __builtin_amdgcn_sched_barrier(0);  // the next row's loads are issued before this row's work
      finish(t, (int)(it & 1), r, dn, xv, dy);
    }
    floatx4 dn[UPT], xv[UPT], dy[UPT];
    take(dn, xv, dy);
    finish(t, (int)(it & 1), rstd[t], dn, xv, dy);
  }
#pragma unroll
  for (int u = 0; u < UPT; ++u) {
    const int q = tid + kBwdThreads * u;
    if (q >= nunits) continue;
    store4<float>(ws_dw + (int64_t)blockIdx.x * H + 4 * q, col_dw[u][tid]);
    store4<float>(ws_db + (int64_t)blockIdx.x * H + 4 * q, col_db[u][tid]);
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
  if (c < cols) {
    // eight loads in flight at a time; the additions stay in row order
    int64_t b = b0;
    for (; b + 8 <= b1; b += 8) {
      float v[8];
#pragma unroll
      for (int k = 0; k < 8; ++k) v[k] = ws[(b + k) * cols + c];
#pragma unroll
      for (int k = 0; k < 8; ++k) acc += v[k];
    }
    for (; b < b1; ++b) acc += ws[b * cols + c];
  }
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

template <typename T, int UPT, bool FULL>
static void launch_bwd_np(const NormParts& parts, dim3 grid, hipStream_t s, const T* xp, const T* dyp, const float* rstd,
                          const T* wp, T* dxp, float* ws_dw, float* ws_db, int64_t T_, int H, int64_t rpb) {
  // every part's loads in flight together for the usual shard counts while they fit in registers
  if (parts.n == 1)
    hipLaunchKernelGGL((rmsnorm_bwd_kernel<T, UPT, FULL, 1>), grid, dim3(kBwdThreads), 0, s, parts, xp, dyp, rstd, wp,
                       dxp, ws_dw, ws_db, T_, H, rpb);
  else if (parts.n == 2 && UPT <= 8)
    hipLaunchKernelGGL((rmsnorm_bwd_parts_kernel<T, (UPT <= 8 ? UPT : 1), FULL, 2>), grid, dim3(kBwdThreads), 0, s,
                       parts, xp, dyp, rstd, wp, dxp, ws_dw, ws_db, T_, H, rpb);
  else if (parts.n == 4 && UPT <= 4)
    hipLaunchKernelGGL((rmsnorm_bwd_parts_kernel<T, (UPT <= 4 ? UPT : 1), FULL, 4>), grid, dim3(kBwdThreads), 0, s,
                       parts, xp, dyp, rstd, wp, dxp, ws_dw, ws_db, T_, H, rpb);
  else if (parts.n == 8 && UPT <= 4)
    hipLaunchKernelGGL((rmsnorm_bwd_parts_kernel<T, (UPT <= 4 ? UPT : 1), FULL, 8>), grid, dim3(kBwdThreads), 0, s,
                       parts, xp, dyp, rstd, wp, dxp, ws_dw, ws_db, T_, H, rpb);
  else
    hipLaunchKernelGGL((rmsnorm_bwd_kernel<T, UPT, FULL, 0>), grid, dim3(kBwdThreads), 0, s, parts, xp, dyp, rstd, wp,
                       dxp, ws_dw, ws_db, T_, H, rpb);
}

template <typename T>
static hipError_t bwd_t(const NormParts& parts, const void* x, const void* dY, const float* rstd, const void* w,
                        void* dx, float* dw, float* db, void* ws, int64_t T_, int64_t H, bool accum, hipStream_t s) {
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
#define TPMLP_BWD(U)                                                                                          \
  if (units == (int64_t)kBwdThreads * (U))                                                                      \
    launch_bwd_np<T, U, true>(parts, dim3((unsigned)nblk), s, xp, dyp, rstd, wp, dxp, ws_dw, ws_db, T_, (int)H, rpb); \
  else                                                                                                          \
    launch_bwd_np<T, U, false>(parts, dim3((unsigned)nblk), s, xp, dyp, rstd, wp, dxp, ws_dw, ws_db, T_, (int)H, rpb)
    if (upt <= 1) {
      TPMLP_BWD(1);
    } else if (upt <= 2) {
      TPMLP_BWD(2);
    } else if (upt <= 4) {
      TPMLP_BWD(4);
    } else if (upt <= 8) {
      TPMLP_BWD(8);
    } else {
      TPMLP_BWD(16);
    }
#undef TPMLP_BWD
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  hipError_t e;
  e = launch_reduce_partial_rows(ws_dw, dw, nblk, H, accum, s);
  if (e != hipSuccess) return e;
  return launch_reduce_partial_rows(ws_db, db, nblk, H, accum, s);
}

hipError_t launch_rmsnorm_bwd(DType dt, const float* const* dN_parts, int n_parts, const void* x, const void* dY,
                              const float* rstd, const void* w, void* dx, float* dw, float* db, void* ws, int64_t T_,
                              int64_t H, bool accum, hipStream_t s) {
  if (n_parts < 1 || n_parts > kMaxNormParts) return hipErrorInvalidValue;
  NormParts parts{};
  for (int k = 0; k < n_parts; ++k) parts.p[k] = dN_parts[k];
  parts.n = n_parts;
  // T = 0 still writes the (empty, zero) column sums (or leaves accumulated ones as they are).
  if (dt == kBF16) return bwd_t<bf16_t>(parts, x, dY, rstd, w, dx, dw, db, ws, T_, H, accum, s);
  return bwd_t<float>(parts, x, dY, rstd, w, dx, dw, db, ws, T_, H, accum, s);
}

}  // namespace tpmlp
