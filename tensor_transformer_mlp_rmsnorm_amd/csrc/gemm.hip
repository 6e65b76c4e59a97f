// MFMA GEMM for the six contractions of the MLP sublayer (gfx950 / CDNA4):
// the fp32 path (the bf16 path is gemm_bf16.hip).
//
//   C[m, n] = sum_k A(m, k) B(k, n)
//   A(m, k) = A[m * lda + k]  (a_kcontig)  or  A[k * lda + m]
//   B(k, n) = B[n * ldb + k]  (b_kcontig)  or  B[k * ldb + n]
//
// Forward expansion and down projection have both operands K-contiguous
// ("NT"); the activation gradients have B N-contiguous ("NN"); the weight
// gradients contract over tokens with both operands MN-contiguous ("TN").
//
// Design (one 256-thread workgroup per 128 x 128 output tile):
//  * Four waves in a 2 x 2 grid, each owning a 64 x 64 sub-tile as 4 x 4
//    MFMA 16x16 blocks: v_mfma_f32_16x16x32_bf16 for bf16 (one 16-byte
//    fragment of 8 k-values per lane), v_mfma_f32_16x16x4_f32 x 4 for fp32.
//  * LDS always holds both tiles as [row][128 bytes of k], 16-byte chunks
//    XOR-swizzled by (row & 7), so the inner loop is the same for every
//    layout.  MN-contiguous operands are transposed in registers (8 x 8 bf16
//    or 4 x 4 fp32 blocks) on their way from HBM to LDS.
//  * Two LDS stages; the next k-tile's global loads are in flight while the
//    current one is multiplied; one barrier per k-tile.
//  * The B operand is passed to the MFMA as its first source, so each lane's
//    accumulator holds four consecutive columns of one output row; every
//    epilogue then works on 4-wide vectors.
//  * Tiles are ordered per XCD (each of the 8 XCDs gets a contiguous range of
//    tile ids, since workgroups are dealt round-robin over XCDs) and grouped
//    by 8 tile-rows inside that range for L2 reuse of the B panel.
//  * SwiGLU forward: a tile covers 64 FFN channels; each wave's 64 B rows are
//    32 gate rows followed by the same 32 channels' up rows, so a lane holds
//    g and u of the same (token, channel) and SiLU(g) * u is formed in
//    registers ("Split the expansion": gate and up channels stay paired).
//    g and u are stored (bf16) for the backward, and the activation is
//    formed from those stored values.
#include "common.h"
#include "kernels.h"

namespace tpmlp {
namespace {

constexpr int kBM = 128;
constexpr int kBN = 128;
constexpr int kRowBytes = 128;          // bytes of k per LDS row
constexpr int kChunks = kRowBytes / 16;  // 16-byte chunks per LDS row
constexpr int kThreads = 256;
constexpr int kSwigluChannels = 64;  // FFN channels per tile in the SwiGLU forward

__device__ __forceinline__ int swz(int row, int chunk) { return row * kChunks + (chunk ^ (row & 7)); }

// 8 x 8 transpose of bf16: in[e] holds 8 consecutive mn values at k = e;
// out[j] receives 8 consecutive k values at mn = j.
__device__ __forceinline__ void transpose_chunks(const uint4 (&in)[8], uint4 (&out)[8]) {
  const uint32_t* w = reinterpret_cast<const uint32_t*>(in);
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    uint32_t o[4];
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const uint32_t lo = w[(2 * p) * 4 + (j >> 1)];
      const uint32_t hi = w[(2 * p + 1) * 4 + (j >> 1)];
      o[p] = (j & 1) ? ((lo >> 16) | (hi & 0xffff0000u)) : ((lo & 0xffffu) | (hi << 16));
    }
    out[j] = make_uint4(o[0], o[1], o[2], o[3]);
  }
}

// 4 x 4 transpose of fp32.
__device__ __forceinline__ void transpose_chunks(const uint4 (&in)[4], uint4 (&out)[4]) {
  out[0] = make_uint4(in[0].x, in[1].x, in[2].x, in[3].x);
  out[1] = make_uint4(in[0].y, in[1].y, in[2].y, in[3].y);
  out[2] = make_uint4(in[0].z, in[1].z, in[2].z, in[3].z);
  out[3] = make_uint4(in[0].w, in[1].w, in[2].w, in[3].w);
}

template <typename T>
__device__ __forceinline__ void mfma_chunk(floatx4& acc, const uint4& bfrag, const uint4& afrag);

template <>
__device__ __forceinline__ void mfma_chunk<bf16_t>(floatx4& acc, const uint4& bfrag, const uint4& afrag) {
  acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, bfrag),
                                                __builtin_bit_cast(bf16x8, afrag), acc, 0, 0, 0);
}

template <>
__device__ __forceinline__ void mfma_chunk<float>(floatx4& acc, const uint4& bfrag, const uint4& afrag) {
  acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(bfrag.x), __uint_as_float(afrag.x), acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(bfrag.y), __uint_as_float(afrag.y), acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(bfrag.z), __uint_as_float(afrag.z), acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(bfrag.w), __uint_as_float(afrag.w), acc, 0, 0, 0);
}

// Loader of one operand tile (kBM or kBN rows of the LDS tile).
//   KCONTIG: the operand is stored [rows][k]; a thread moves whole 16-byte
//            chunks (kRows * kChunks / kThreads of them).
//   else:    stored [k][rows]; a thread moves one E x E block (E k-rows of E
//            row-values each), transposes it, and writes E chunks.
//   `unit_offset` rotates which threads carry the transposed blocks, so two
//   transposed operands use disjoint threads.
template <typename T, bool KCONTIG, int ROWS>
struct TileLoader {
  static constexpr int E = Elem<T>::kPerChunk;
  static constexpr int kKElems = kRowBytes / (int)sizeof(T);
  static constexpr int kRegs = KCONTIG ? (ROWS * kChunks / kThreads) : E;
  static constexpr int kUnits = (kKElems / E) * (ROWS / E);  // transposed blocks per tile
  static_assert(KCONTIG || kUnits <= kThreads, "one transposed block per thread at most");
  uint4 reg[kRegs];
};

// Physical row of logical tile row r, or -1 when outside the operand.
struct RowMap {
  int64_t base;    // first logical row of the tile
  int64_t limit;   // number of valid rows
  bool swiglu;     // B of the SwiGLU forward: channel-paired gate/up rows
  int64_t ffn;     // F, with swiglu

  __device__ __forceinline__ int64_t operator()(int r) const {
    if (!swiglu) {
      const int64_t g = base + r;
      return g < limit ? g : -1;
    }
    const int wave_n = r >> 6, w = r & 63;
    const int64_t ch = base + wave_n * 32 + (w & 31);
    if (ch >= ffn) return -1;
    return (w >> 5) * ffn + ch;
  }
};

template <typename T, bool KCONTIG, int ROWS>
__device__ __forceinline__ void load_tile(TileLoader<T, KCONTIG, ROWS>& L, const T* __restrict__ p,
                                          int64_t ld, const RowMap& rm, int64_t k0, int64_t K, int tid,
                                          int unit_offset) {
  using TL = TileLoader<T, KCONTIG, ROWS>;
  constexpr int E = TL::E;
  if constexpr (KCONTIG) {
#pragma unroll
    for (int i = 0; i < TL::kRegs; ++i) {
      const int q = tid + kThreads * i;
      const int r = q / kChunks, c = q % kChunks;
      const int64_t grow = rm(r);
      const int64_t gk = k0 + (int64_t)c * E;
      uint4 v = make_uint4(0, 0, 0, 0);
      if (grow >= 0 && gk < K) v = *reinterpret_cast<const uint4*>(p + grow * ld + gk);
      L.reg[i] = v;
    }
  } else {
    const int u = (tid + unit_offset) % kThreads;
    constexpr int kMnBlocks = ROWS / E;
    const int mb = u % kMnBlocks, kc = u / kMnBlocks;
    const int64_t mn = rm.base + (int64_t)mb * E;
    const bool mn_ok = (u < TL::kUnits) && (mn < rm.limit);
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const int64_t kr = k0 + (int64_t)kc * E + e;
      uint4 v = make_uint4(0, 0, 0, 0);
      if (mn_ok && kr < K) v = *reinterpret_cast<const uint4*>(p + kr * ld + mn);
      L.reg[e] = v;
    }
  }
}

template <typename T, bool KCONTIG, int ROWS>
__device__ __forceinline__ void store_tile(const TileLoader<T, KCONTIG, ROWS>& L, uint4* __restrict__ lds,
                                           int tid, int unit_offset) {
  using TL = TileLoader<T, KCONTIG, ROWS>;
  constexpr int E = TL::E;
  if constexpr (KCONTIG) {
#pragma unroll
    for (int i = 0; i < TL::kRegs; ++i) {
      const int q = tid + kThreads * i;
      lds[swz(q / kChunks, q % kChunks)] = L.reg[i];
    }
  } else {
    const int u = (tid + unit_offset) % kThreads;
    if (u < TL::kUnits) {
      constexpr int kMnBlocks = ROWS / E;
      const int mb = u % kMnBlocks, kc = u / kMnBlocks;
      uint4 t[E];
      transpose_chunks(L.reg, t);
#pragma unroll
      for (int j = 0; j < E; ++j) lds[swz(mb * E + j, kc)] = t[j];
    }
  }
}

// blockIdx -> (tile_m, tile_n): per-XCD contiguous ranges, then groups of 8
// tile-rows.
__device__ __forceinline__ void tile_coords(int pid, int ntm, int ntn, int& tm, int& tn) {
  const int ntiles = ntm * ntn;
  const int xcd = pid & 7, local = pid >> 3;
  const int per = ntiles >> 3, rem = ntiles & 7;
  const int tile = (xcd < rem) ? xcd * (per + 1) + local : rem * (per + 1) + (xcd - rem) * per + local;
  constexpr int kGroup = 8;
  const int in_group = kGroup * ntn;
  const int group = tile / in_group;
  const int first_m = group * kGroup;
  const int gsize = min(ntm - first_m, kGroup);
  const int t = tile - group * in_group;
  tm = first_m + t % gsize;
  tn = t / gsize;
}

template <typename T, bool AK, bool BKC, int EPI>
__global__ __launch_bounds__(kThreads, 2) void gemm_kernel(GemmArgs g, int ntm, int ntn) {
  using LA = TileLoader<T, AK, kBM>;
  using LB = TileLoader<T, BKC, kBN>;
  constexpr int kKElems = kRowBytes / (int)sizeof(T);
  constexpr int kStage = (kBM + kBN) * kChunks;  // uint4 per LDS stage
  __shared__ uint4 smem[2 * kStage];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;

  int tm, tn;
  tile_coords(blockIdx.x, ntm, ntn, tm, tn);

  const T* __restrict__ A = static_cast<const T*>(g.A);
  const T* __restrict__ B = static_cast<const T*>(g.B);
  const int64_t K = g.K;

  RowMap ra{(int64_t)tm * kBM, g.M, false, 0};
  RowMap rb = (EPI == kEpiSwigluFwd) ? RowMap{(int64_t)tn * kSwigluChannels, g.N, true, g.ffn}
                                     : RowMap{(int64_t)tn * kBN, g.N, false, 0};
  // Transposed operands: A's blocks on threads [0, 128), B's on [128, 256).
  constexpr int kOffA = 0, kOffB = kThreads / 2;

  LA la;
  LB lb;
  floatx4 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = floatx4{0.f, 0.f, 0.f, 0.f};

  const int nk = (int)((K + kKElems - 1) / kKElems);
  load_tile(la, A, g.lda, ra, 0, K, tid, kOffA);
  load_tile(lb, B, g.ldb, rb, 0, K, tid, kOffB);
  store_tile(la, smem, tid, kOffA);
  store_tile(lb, smem + kBM * kChunks, tid, kOffB);
  __syncthreads();

  const int frow = lane & 15, fchunk = lane >> 4;
  for (int kt = 0; kt < nk; ++kt) {
    const bool more = kt + 1 < nk;
    if (more) {
      const int64_t k0 = (int64_t)(kt + 1) * kKElems;
      load_tile(la, A, g.lda, ra, k0, K, tid, kOffA);
      load_tile(lb, B, g.ldb, rb, k0, K, tid, kOffB);
    }
    const uint4* sa = smem + (kt & 1) * kStage;
    const uint4* sb = sa + kBM * kChunks;
#pragma unroll
    for (int s = 0; s < kChunks / 4; ++s) {
      uint4 af[4], bfr[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) af[i] = sa[swz(wm * 64 + i * 16 + frow, s * 4 + fchunk)];
#pragma unroll
      for (int j = 0; j < 4; ++j) bfr[j] = sb[swz(wn * 64 + j * 16 + frow, s * 4 + fchunk)];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) mfma_chunk<T>(acc[i][j], bfr[j], af[i]);
    }
    if (more) {
      uint4* dst = smem + ((kt + 1) & 1) * kStage;
      store_tile(la, dst, tid, kOffA);
      store_tile(lb, dst + kBM * kChunks, tid, kOffB);
    }
    __syncthreads();
  }

  // ------------------------------------------------------------- epilogue
  const int64_t M = g.M, N = g.N, F = g.ffn;
  const int col4 = 4 * (lane >> 4);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int64_t m = (int64_t)tm * kBM + wm * 64 + i * 16 + frow;
    if (m >= M) continue;
    if constexpr (EPI == kEpiSwigluFwd) {
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int64_t ch = (int64_t)tn * kSwigluChannels + wn * 32 + j * 16 + col4;
        if (ch >= F) continue;
        // g and u are stored tensors: the activation is formed from their stored values
        const floatx4 gv = stored<T>(acc[i][j]), uv = stored<T>(acc[i][j + 2]);
        floatx4 av;
#pragma unroll
        for (int r = 0; r < 4; ++r) av[r] = gv[r] * sigmoid_f(gv[r]) * uv[r];
        T* pre = static_cast<T*>(g.pre) + m * 2 * F;
        store4<T>(pre + ch, gv);
        store4<T>(pre + F + ch, uv);
        store4<T>(static_cast<T*>(g.act) + m * F + ch, av);
      }
    } else {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int64_t n = (int64_t)tn * kBN + wn * 64 + j * 16 + col4;
        if (n >= N) continue;
        const floatx4 v = acc[i][j];
        if constexpr (EPI == kEpiStoreF32) {
          float* c = static_cast<float*>(g.C) + m * g.ldc + n;
          store4<float>(c, g.accum ? v + load4<float>(c) : v);
        } else if constexpr (EPI == kEpiResidual) {
          const floatx4 xr = load4<T>(static_cast<const T*>(g.aux) + m * g.ldc + n);
          const floatx4 bb = load4<T>(static_cast<const T*>(g.bias) + n);
          store4<T>(static_cast<T*>(g.C) + m * g.ldc + n, v + xr + bb);
        } else if constexpr (EPI == kEpiGeluFwd) {
          const floatx4 bb = load4<T>(static_cast<const T*>(g.bias) + n);
          const floatx4 h = stored<T>(v + bb);
          floatx4 a;
#pragma unroll
          for (int r = 0; r < 4; ++r) a[r] = gelu_f(h[r]);
          store4<T>(static_cast<T*>(g.pre) + m * N + n, h);
          store4<T>(static_cast<T*>(g.act) + m * N + n, a);
        } else if constexpr (EPI == kEpiSwigluBwd) {
          const T* sv = static_cast<const T*>(g.aux) + m * 2 * F;
          const floatx4 gv = load4<T>(sv + n), uv = load4<T>(sv + F + n);
          floatx4 dg, du;
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const float sg = sigmoid_f(gv[r]);
            dg[r] = v[r] * uv[r] * sg * (1.0f + gv[r] * (1.0f - sg));
            du[r] = v[r] * gv[r] * sg;
          }
          T* dp = static_cast<T*>(g.pre) + m * 2 * F;
          store4<T>(dp + n, dg);
          store4<T>(dp + F + n, du);
        } else if constexpr (EPI == kEpiGeluBwd) {
          const floatx4 h = load4<T>(static_cast<const T*>(g.aux) + m * N + n);
          floatx4 dh;
#pragma unroll
          for (int r = 0; r < 4; ++r) dh[r] = v[r] * gelu_grad_f(h[r]);
          store4<T>(static_cast<T*>(g.pre) + m * N + n, dh);
        }
      }
    }
  }
}

template <typename T, bool AK, bool BKC, int EPI>
hipError_t launch_t(const GemmArgs& g, hipStream_t s) {
  const int ntm = (int)((g.M + kBM - 1) / kBM);
  const int ntn = (EPI == kEpiSwigluFwd) ? (int)((g.ffn + kSwigluChannels - 1) / kSwigluChannels)
                                         : (int)((g.N + kBN - 1) / kBN);
  if (ntm == 0 || ntn == 0) return hipSuccess;
  KernelTimer timer(g.tag ? g.tag : "gemm", s);
  hipLaunchKernelGGL((gemm_kernel<T, AK, BKC, EPI>), dim3(ntm * ntn), dim3(kThreads), 0, s, g, ntm, ntn);
  return hipGetLastError();
}

template <typename T>
hipError_t dispatch(bool ak, bool bk, Epi epi, const GemmArgs& g, hipStream_t s) {
  if (ak && bk) {
    switch (epi) {
      case kEpiStoreF32: return launch_t<T, true, true, kEpiStoreF32>(g, s);
      case kEpiSwigluFwd: return launch_t<T, true, true, kEpiSwigluFwd>(g, s);
      case kEpiGeluFwd: return launch_t<T, true, true, kEpiGeluFwd>(g, s);
      case kEpiResidual: return launch_t<T, true, true, kEpiResidual>(g, s);
      default: break;
    }
  } else if (ak && !bk) {
    switch (epi) {
      case kEpiStoreF32: return launch_t<T, true, false, kEpiStoreF32>(g, s);
      case kEpiSwigluBwd: return launch_t<T, true, false, kEpiSwigluBwd>(g, s);
      case kEpiGeluBwd: return launch_t<T, true, false, kEpiGeluBwd>(g, s);
      default: break;
    }
  } else if (!ak && !bk) {
    if (epi == kEpiStoreF32) return launch_t<T, false, false, kEpiStoreF32>(g, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_gemm(DType dt, bool a_kcontig, bool b_kcontig, Epi epi, const GemmArgs& g, hipStream_t s) {
  if (dt == kBF16) return launch_gemm_bf16(a_kcontig, b_kcontig, epi, g, s);
  return dispatch<float>(a_kcontig, b_kcontig, epi, g, s);
}

}  // namespace tpmlp
