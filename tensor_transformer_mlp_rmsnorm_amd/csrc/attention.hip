// Causal grouped-query attention, forward and backward (gfx950 / CDNA4).
//
// The attention each tensor-parallel rank runs on its own heads ("Megatron-LM
// walkthrough", Part IV, Stage 5: the column-parallel QKV projection gives each
// rank the Q, K and V of its heads, and attention runs locally per head):
//
//   S_h = q_h k_g^T / sqrt(D) on the positions of one sequence, g = h / group,
//   P_h = softmax of S_h over keys j <= i,   o_h = P_h v_g.
//
// Layout: qkv [T, ld] bf16 with T = batch x seq rows (a sequence's rows are
// contiguous) and columns [Q heads | K heads | V heads], D columns per head;
// O [T, n_q D] bf16; lse [n_q, T] fp32 (natural log of each row's softmax
// denominator, the row maximum included).
//
// All products are v_mfma_f32_16x16x32_bf16 (D[x][y] += sum_k X[x][k] Y[y][k];
// lane l supplies row l % 16 of X and of Y with the 8 k of its lane group
// l / 16 and holds D[4 (l / 16) + r][l % 16], r < 4).  The scores are formed
// transposed, S^T = K Q^T, so a lane holds 4 keys of one query: the softmax
// statistics of a query stay in one lane column, and the lane's exp'd scores
// are directly the Y operand of O^T = V^T P^T once the 32 keys of an MFMA step
// are assigned to the lanes' k slots as key = 16 (slot / 4) + 4 (l / 16) +
// slot % 4 -- the same order in which the lane holds them.  The X operand V^T
// then needs V's column e = l % 16 at those keys, which the LDS transpose read
// (ds_read_b64_tr_b16) delivers: in each 16-lane group, result lane i element
// j is the (i mod 4)-th 16-bit value at the address of lane 4 j + i / 4.  The
// backward kernels use the same device for Q^T, dO^T and K^T.
//
// Forward: one workgroup of 8 waves per (query block of 64, head, batch),
// two 64-key tiles per step, each wave 32 queries x 32 keys of a tile; online
// softmax in exp2 with the 1/sqrt(D) scale folded in, the key parts of a
// query merged at the end.  The score gradients dS (and the forward's P)
// enter their products as a bf16 pair (hi + lo, see pack_slots).  Backward
// (no atomics): dK and dV per (key block of 64, query head, batch) over the
// query blocks at or after the key block, the shares of a group's query heads
// then added in a fixed order by a small kernel; dQ per (query block, head,
// batch) over the key blocks up to it; both recompute P from lse and use
// delta = rowsum(dO o O) from a small kernel.  Tiles reach LDS by DMA into
// two buffers used in turn.
#include "common.h"
#include "kernels.h"

namespace tpmlp {
namespace {

constexpr int kAttnBlock = 64;
constexpr float kLog2e = 1.4426950408889634f, kLn2 = 0.6931471805599453f;
// The forward's running maximum is raised (and the partial output rescaled)
// only when a score exceeds it by more than this many powers of two, so the
// probabilities formed against it stay below 2^8.
constexpr float kLazyRescale = 8.0f;

typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float float2v __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;

__device__ __forceinline__ floatx4 mma(const uint4& x, const uint4& y, floatx4 acc) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, x), __builtin_bit_cast(bf16x8, y), acc,
                                                 0, 0, 0);
}

// 2^x with the hardware instruction: the arguments here are <= 8 (or -inf),
// and results below 2^-126 are negligible next to the row's largest term.
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Two fp32 values as bf16 (round to nearest even), the first in the low half.
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(float2v{a, b}, bf16x2));
}

template <typename T>
struct Flag {
  static constexpr bool value = T::value;
};
struct Masked {
  static constexpr bool value = true;
};
struct Unmasked {
  static constexpr bool value = false;
};

// A [64][D] bf16 tile in LDS, 16-byte chunks XOR-swizzled by row.  The LDS
// serves a 16-byte read (ds_read_b128) in four passes of the lanes
// p, p + 4, ..., p + 60, and a transpose read (ds_read_b64_tr_b16) in two
// passes of 32 lanes; a pass is conflict-free when its lanes hit distinct
// bank groups (16 bytes, or 8 bytes for the transpose read) of the 256-byte
// bank row (measured with rocprofv3's SQ_LDS_BANK_CONFLICT on isolated reads).
// The row reads here take 16 rows x chunks 4 ks .. 4 ks + 3 (lane: row l % 16,
// chunk l / 16), the transpose reads 8 rows x 2 adjacent chunks per pass.
//  * swz(r) = 2 (r mod K/2) + (r / (K/2) mod 2), K = D / 8 chunks per row:
//    conflict-free transpose reads, 2-way conflicts in the row reads of D = 128.
//  * CF (D = 128 only): swz(r) = 4 ((r mod 4) ^ (r / 4 mod 4)) + 2 (r / 4 mod 2)
//    gives rows r, r + 4, r + 8, r + 12 distinct chunk quads and any 8 rows
//    from a multiple of 8 distinct chunk pairs: both reads conflict-free, for
//    about 12 more address instructions per step, which pays only in the dK/dV
//    kernel (the most LDS reads per MFMA).
// For D = 64 (128-byte rows, two to a bank row) the row reads of a pass share
// one half of the bank row whatever the swizzle.
template <int D, bool CF = false>
struct Tile {
  static_assert(!CF || D == 128, "the conflict-free layout is for 16 chunks per row");
  static constexpr int kChunks = D / 8;  // 16-byte chunks per row
  __device__ __forceinline__ static int swz(int row) {
    if constexpr (CF) return (((row & 3) ^ ((row >> 2) & 3)) << 2) | (((row >> 2) & 1) << 1);
    else return 2 * (row & (kChunks / 2 - 1)) | ((row / (kChunks / 2)) & 1);
  }
  __device__ __forceinline__ static int chunk_off(int row, int chunk) {
    return (row * kChunks + (chunk ^ swz(row))) * 16;
  }
  // Row `row`, elements 8 c .. 8 c + 7.
  __device__ __forceinline__ static uint4 row8(const char* __restrict__ base, int row, int c) {
    return *reinterpret_cast<const uint4*>(base + chunk_off(row, c));
  }
  // Column fragment for this lane (X or Y operand row e0 + l % 16) at the 8
  // rows 32 m + 16 h + 4 (l / 16) + j, h < 2, j < 4: two transpose reads.
  __device__ __forceinline__ static uint4 col8(const char* __restrict__ base, int m, int e0, int lane) {
    const int g = lane >> 4, a = lane & 15;
    uint2 out[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int row = 32 * m + 16 * h + 4 * g + (a >> 2);
      const int e = e0 + 4 * (a & 3);
      const int off = chunk_off(row, e >> 3) + (e & 7) * 2;
      bf16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(base + off));
      out[h] = __builtin_bit_cast(uint2, v);
    }
    return make_uint4(out[0].x, out[0].y, out[1].x, out[1].y);
  }
};

// Four floats from LDS.  Like the tile reads above, the pointer is restrict:
// the reads of a step touch only the buffer the previous step's DMA filled,
// never the one the current step's DMA is writing (the barrier that ends a
// step waits for that DMA), and saying so keeps the compiler from waiting for
// the in-flight DMA before every read.
__device__ __forceinline__ floatx4 lds_load4(const float* __restrict__ p) {
  return *reinterpret_cast<const floatx4*>(p);
}

// LDS DMA of [64][D] bf16 tiles from the rows of one sequence (a [seq, ld]
// matrix): buffer_load_dwordx4 ... lds writes a wave's 64 x 16 bytes to 1 KiB
// of LDS at a wave-uniform address, lane j at byte 16 j, with no registers in
// between; each lane fetches the global chunk that belongs at its slot under
// the tile's swizzle.  A 1 KiB block holds kRows = 512 / D rows; wave w of NW
// fills blocks w, w + NW, ... of a tile, whose rows share one swizzle pattern
// (NW is a multiple of 4), so a lane's offset inside its blocks is one
// register.  Lanes whose row is past the sequence get an offset beyond the
// buffer (the buffer unit returns zeros) and blocks wholly past it a zero SGPR
// offset, so no offset wraps; the host keeps a sequence below 2^30 elements.
template <int D, int NW, bool CF = false>
struct TileDma {
  static constexpr int kChunks = D / 8, kRows = 512 / D, kBlocks = kAttnBlock / kRows, kPerWave = kBlocks / NW;
  static_assert(kPerWave >= 1 && kBlocks % NW == 0 && NW % 4 == 0, "block split");
  static constexpr unsigned kOut = 0x80000000u;
  __amdgpu_buffer_rsrc_t rsrc;
  int64_t ld, rows;
  unsigned vlane;  // this lane's byte offset inside one of its blocks
  int lrow, w;
  __device__ __forceinline__ TileDma(const bf16_t* seq_base, int64_t ld_, int64_t rows_, int wave, int lane)
      : ld(ld_), rows(rows_), w(wave) {
    rsrc = __builtin_amdgcn_make_buffer_rsrc(const_cast<bf16_t*>(seq_base), (short)0, (int)(rows_ * ld_ * 2),
                                             0x00020000);
    lrow = lane / kChunks;
    const int row = kRows * w + lrow;  // a representative row: every block of this wave has the same pattern
    vlane = (unsigned)((lrow * ld_ + 8 * ((lane % kChunks) ^ Tile<D, CF>::swz(row))) * 2);
  }
  // Tile `blk` of the columns col0 .. col0 + D - 1 into the LDS tile at `dst`.
  __device__ __forceinline__ void issue(char* dst, int blk, int64_t col0) const {
#pragma unroll
    for (int i = 0; i < kPerWave; ++i) {
      const int bb = w + NW * i;
      const int64_t r0 = (int64_t)blk * kAttnBlock + kRows * bb;
      const bool in = r0 < rows;
      const unsigned soff = in ? (unsigned)((r0 * ld + col0) * 2) : 0u;
      const unsigned voff = r0 + lrow < rows ? vlane : kOut;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (__attribute__((address_space(3))) void*)(dst + bb * 1024), 16,
                                               voff, (int)soff, 0, 0);
    }
  }
};

// The lane's 8 k-slot values of one 32-row step m from its two 16-row blocks
// (block 2m: slots 0-3, block 2m + 1: slots 4-7) as one bf16 operand.
__device__ __forceinline__ uint4 pack_slots1(const floatx4& b0, const floatx4& b1) {
  return make_uint4(pack_bf16x2(b0[0], b0[1]), pack_bf16x2(b0[2], b0[3]), pack_bf16x2(b1[0], b1[1]),
                    pack_bf16x2(b1[2], b1[3]));
}

// The same as two bf16 operands whose sum carries the fp32 value to 2^-17:
// hi = bf16(v), lo = bf16(v - hi).  The score gradients dS are multiplied this
// way: their sum over keys cancels (it is zero up to rounding for every
// query), so a single bf16 rounding of each term would dominate dQ and dK.
struct SlotPair {
  uint4 hi, lo;
};
__device__ __forceinline__ float lo_half(uint32_t u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float hi_half(uint32_t u) { return __uint_as_float(u & 0xffff0000u); }
__device__ __forceinline__ SlotPair pack_slots(const floatx4& b0, const floatx4& b1) {
  const uint4 hi = pack_slots1(b0, b1);
  const floatx4 r0 = {b0[0] - lo_half(hi.x), b0[1] - hi_half(hi.x), b0[2] - lo_half(hi.y), b0[3] - hi_half(hi.y)};
  const floatx4 r1 = {b1[0] - lo_half(hi.z), b1[1] - hi_half(hi.z), b1[2] - lo_half(hi.w), b1[3] - hi_half(hi.w)};
  return SlotPair{hi, pack_slots1(r0, r1)};
}

__device__ __forceinline__ floatx4 mma2(const uint4& x, const SlotPair& y, floatx4 acc) {
  return mma(x, y.lo, mma(x, y.hi, acc));
}

// max / sum of the four lanes l, l ^ 16, l ^ 32, l ^ 48 (gfx950 lane swaps:
// each returns the value and its partner's, one of them the lane's own).
__device__ __forceinline__ float max_xor16(float v) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float max_xor32(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_xor16(float v) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float sum_xor32(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

struct AttnDims {
  int64_t batch, seq, ld, ldo;  // ld: row length of qkv / dqkv; ldo: of O / dO (n_q D)
  int n_q, n_kv, group;
  float scale_log2;             // log2(e) / sqrt(D)
  float scale;                  // 1 / sqrt(D)
};

// blockIdx -> (block index, head, batch), the block index descending: the
// workgroups with the most work start first, and those the chip cannot hold
// at once fill the units that finish first.
__device__ __forceinline__ void block_coords(int nblocks, int heads, int batch, int& blk, int& head, int& b) {
  const int per = heads * batch, r = (int)blockIdx.x;
  blk = nblocks - 1 - r / per;
  head = (r % per) / batch;
  b = r % batch;
}

constexpr int kSplitWaves = 8, kSplitThreads = kSplitWaves * 64;

// Forward: 64 queries of one head per workgroup of 8 waves, which takes two
// 64-key tiles per step (tiles 0 .. qb, the last one -- the diagonal, which
// also holds any keys past the sequence end -- with the causal mask): wave w
// takes queries 32 (w % 2) .. + 31 and, of tile 2 step + (w / 4), keys
// 32 (w / 2 % 2) .. + 31.  Each K fragment read from LDS feeds two query
// blocks and each V fragment four products, and the longest workgroup takes
// half as many steps as there are tiles.  Each wave keeps its own online
// softmax over its keys; the four key parts of a query are merged at the end
// through LDS in a fixed order.  The tiles are double-buffered in LDS and
// filled by DMA: a step starts the next step's tiles into the other buffer
// and ends with the one barrier, which also waits for them.
template <int D>
__global__ __launch_bounds__(kSplitThreads, 1) void attn_fwd_kernel(const bf16_t* __restrict__ qkv,
                                                                    bf16_t* __restrict__ O, float* __restrict__ lse,
                                                                    AttnDims dm) {
  constexpr int kTile = kAttnBlock * D * 2, KS = D / 32, EB = D / 16;
  __shared__ __align__(16) char smem[2][2][2][kTile];  // [buffer][tile of the step][K, V]
  const int tid = threadIdx.x, lane = tid & 63, g = lane >> 4, c = lane & 15;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6), qh = w & 1, kp = w >> 1, kh = kp & 1, tp = kp >> 1;
  const int nqb = (int)((dm.seq + kAttnBlock - 1) / kAttnBlock);
  int qb, h, b;
  block_coords(nqb, dm.n_q, (int)dm.batch, qb, h, b);
  const int kvh = h / dm.group;
  const int64_t t0 = (int64_t)b * dm.seq;
  const int q0 = qb * kAttnBlock + 32 * qh;  // this wave's first query; lane queries q0 + 16 jq + c
  uint4 qf[2][KS];
#pragma unroll
  for (int jq = 0; jq < 2; ++jq) {
    const int q = q0 + 16 * jq + c;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      qf[jq][ks] = q < dm.seq
                       ? *reinterpret_cast<const uint4*>(qkv + (t0 + q) * dm.ld + (int64_t)h * D + 32 * ks + 8 * g)
                       : make_uint4(0u, 0u, 0u, 0u);
  }
  floatx4 acc[2][EB];
#pragma unroll
  for (int jq = 0; jq < 2; ++jq)
#pragma unroll
    for (int i = 0; i < EB; ++i) acc[jq][i] = floatx4{0.f, 0.f, 0.f, 0.f};
  float m[2] = {-INFINITY, -INFINITY}, lsum[2] = {0.0f, 0.0f};
  const int64_t kcol = (int64_t)(dm.n_q + kvh) * D, vcol = (int64_t)(dm.n_q + dm.n_kv + kvh) * D;
  const TileDma<D, kSplitWaves> dma(qkv + t0 * dm.ld, dm.ld, dm.seq, w, lane);
  const int nsteps = (qb + 2) / 2;
  auto issue_step = [&](int st, int buf) {
#pragma unroll
    for (int t = 0; t < 2; ++t)
      if (2 * st + t <= qb) {
        dma.issue(smem[buf][t][0], 2 * st + t, kcol);
        dma.issue(smem[buf][t][1], 2 * st + t, vcol);
      }
  };
  issue_step(0, 0);
  __syncthreads();
  auto tile = [&](int kb, const char* kt, const char* vt, auto mask) {
    constexpr bool MASK = Flag<decltype(mask)>::value;
    // S^T[key][q]; lane: key = 32 kh + 16 kk + 4 g + r (in the tile), q = q0 + 16 jq + c
    floatx4 s[2][2];  // [kk][jq]
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      s[kk][0] = s[kk][1] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const uint4 kf = Tile<D>::row8(kt, 32 * kh + 16 * kk + c, 4 * ks + g);
        s[kk][0] = mma(kf, qf[0][ks], s[kk][0]);
        s[kk][1] = mma(kf, qf[1][ks], s[kk][1]);
      }
    }
    if constexpr (MASK) {
#pragma unroll
      for (int kk = 0; kk < 2; ++kk)
#pragma unroll
        for (int jq = 0; jq < 2; ++jq)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int key = kb * kAttnBlock + 32 * kh + 16 * kk + 4 * g + r, q = q0 + 16 * jq + c;
            if (!(key <= q && key < dm.seq)) s[kk][jq][r] = -INFINITY;
          }
    }
    float bmax[2];
#pragma unroll
    for (int jq = 0; jq < 2; ++jq) {
      const float v = fmaxf(fmaxf(fmaxf(s[0][jq][0], s[0][jq][1]), fmaxf(s[0][jq][2], s[0][jq][3])),
                            fmaxf(fmaxf(s[1][jq][0], s[1][jq][1]), fmaxf(s[1][jq][2], s[1][jq][3])));
      bmax[jq] = max_xor32(max_xor16(v)) * dm.scale_log2;
    }
    if (__builtin_amdgcn_ballot_w64(bmax[0] > m[0] + kLazyRescale || bmax[1] > m[1] + kLazyRescale)) {
#pragma unroll
      for (int jq = 0; jq < 2; ++jq) {  // m = -inf until a key is seen (a masked tile can leave it so)
        const float mnew = fmaxf(m[jq], bmax[jq]);
        const float alpha = m[jq] == -INFINITY ? 0.0f : fast_exp2(m[jq] - mnew);
        m[jq] = mnew;
        lsum[jq] *= alpha;
#pragma unroll
        for (int i = 0; i < EB; ++i) acc[jq][i] *= alpha;
      }
    }
#pragma unroll
    for (int jq = 0; jq < 2; ++jq) {
      const float mref = m[jq] == -INFINITY ? 0.0f : m[jq];  // with m = -inf every score here is -inf
#pragma unroll
      for (int kk = 0; kk < 2; ++kk)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          s[kk][jq][r] = fast_exp2(__builtin_fmaf(s[kk][jq][r], dm.scale_log2, -mref));
          lsum[jq] += s[kk][jq][r];
        }
    }
    const SlotPair pf0 = pack_slots(s[0][0], s[1][0]);
    const SlotPair pf1 = pack_slots(s[0][1], s[1][1]);
#pragma unroll
    for (int eb = 0; eb < EB; ++eb) {
      const uint4 vf = Tile<D>::col8(vt, kh, 16 * eb, lane);
      acc[0][eb] = mma2(vf, pf0, acc[0][eb]);
      acc[1][eb] = mma2(vf, pf1, acc[1][eb]);
    }
  };
  // Every step but the last holds only tiles before the diagonal.
  for (int st = 0; st + 1 < nsteps; ++st) {
    const int buf = st & 1;
    issue_step(st + 1, buf ^ 1);  // the other buffer's last readers were step st - 1
    tile(2 * st + tp, smem[buf][tp][0], smem[buf][tp][1], Unmasked{});
    __syncthreads();  // this step's tiles are read; the next step's have landed
  }
  {
    const int st = nsteps - 1, buf = st & 1, kb = 2 * st + tp;
    if (kb < qb) tile(kb, smem[buf][tp][0], smem[buf][tp][1], Unmasked{});
    else if (kb == qb) tile(kb, smem[buf][tp][0], smem[buf][tp][1], Masked{});
    __syncthreads();
  }
  // Merge the four key parts of each query: waves with kp > 0 hand (O, m, l)
  // to the wave with kp = 0 and the same queries, which adds them in kp order.
  lsum[0] = sum_xor32(sum_xor16(lsum[0]));
  lsum[1] = sum_xor32(sum_xor16(lsum[1]));
  constexpr int kX = (2 * EB * 4 + 4) * 64;  // floats per handed-over state
  float* xbase = reinterpret_cast<float*>(&smem[0][0][0][0]);
  if (kp > 0) {
    float* x = xbase + ((kp - 1) * 2 + qh) * kX;
#pragma unroll
    for (int jq = 0; jq < 2; ++jq) {
#pragma unroll
      for (int eb = 0; eb < EB; ++eb) *reinterpret_cast<floatx4*>(x + ((jq * EB + eb) * 64 + lane) * 4) = acc[jq][eb];
      x[(2 * EB * 4 + 2 * jq) * 64 + lane] = m[jq];
      x[(2 * EB * 4 + 2 * jq + 1) * 64 + lane] = lsum[jq];
    }
  }
  __syncthreads();
  if (kp == 0) {
#pragma unroll
    for (int jq = 0; jq < 2; ++jq) {
      float mp[3], lp[3];
      float mm = m[jq];
#pragma unroll
      for (int p2 = 0; p2 < 3; ++p2) {
        const float* x = xbase + (p2 * 2 + qh) * kX;
        mp[p2] = x[(2 * EB * 4 + 2 * jq) * 64 + lane];
        lp[p2] = x[(2 * EB * 4 + 2 * jq + 1) * 64 + lane];
        mm = fmaxf(mm, mp[p2]);
      }
      const float a0 = m[jq] == -INFINITY ? 0.0f : fast_exp2(m[jq] - mm);
      float ap[3];
      float l = lsum[jq] * a0;
#pragma unroll
      for (int p2 = 0; p2 < 3; ++p2) {
        ap[p2] = mp[p2] == -INFINITY ? 0.0f : fast_exp2(mp[p2] - mm);
        l += lp[p2] * ap[p2];
      }
      const int q = q0 + 16 * jq + c;
      if (q < dm.seq) {
        const float inv = 1.0f / l;
        bf16_t* dst = O + (t0 + q) * dm.ldo + (int64_t)h * D;
#pragma unroll
        for (int eb = 0; eb < EB; ++eb) {
          floatx4 o = acc[jq][eb] * a0;
#pragma unroll
          for (int p2 = 0; p2 < 3; ++p2)
            o += *reinterpret_cast<const floatx4*>(xbase + (p2 * 2 + qh) * kX + ((jq * EB + eb) * 64 + lane) * 4) *
                 ap[p2];
          store4<bf16_t>(dst + 16 * eb + 4 * g, o * inv);
        }
        if (g == 0) lse[(int64_t)h * dm.batch * dm.seq + t0 + q] = (mm + log2f(l)) * kLn2;
      }
    }
  }
}

// delta[h][t] = sum_e dO[t][h D + e] O[t][h D + e].  D / 8 consecutive lanes
// share a row (16 bytes of O and of dO each, so a row is read as one
// contiguous segment) and add their partial sums with lane shuffles in a
// fixed order.
template <int D>
__global__ __launch_bounds__(256) void attn_delta_kernel(const bf16_t* __restrict__ O, const bf16_t* __restrict__ dO,
                                                          float* __restrict__ delta, int64_t T, int n_q, int64_t ldo) {
  constexpr int L = D / 8;  // lanes per row; divides the wave, so a row's lanes sit in one wave
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t i = gid / L;  // (head, token) pair, token fastest
  const int c = (int)(gid % L);
  const bool ok = i < T * n_q;
  const int h = ok ? (int)(i / T) : 0;
  const int64_t t = ok ? i % T : 0;
  float acc = 0.0f;
  if (ok) {
    const int64_t off = t * ldo + (int64_t)h * D + 8 * c;
    float a[8], e[8];
    Chunk<bf16_t>::unpack(*reinterpret_cast<const uint4*>(O + off), a);
    Chunk<bf16_t>::unpack(*reinterpret_cast<const uint4*>(dO + off), e);
#pragma unroll
    for (int k = 0; k < 8; ++k) acc += a[k] * e[k];
  }
#pragma unroll
  for (int m = L / 2; m > 0; m >>= 1) acc += __shfl_xor(acc, m, kWave);
  if (ok && c == 0) delta[(int64_t)h * T + t] = acc;
}

// dK and dV of 64 keys from one query head: one workgroup of 8 waves per key
// block, query head and sequence (grid order: the key blocks with the most
// query tiles after them first), over the query tiles kb .. nqb - 1 two per
// step.  Wave w owns keys 16 (w % 4) .. + 15 and takes the step's tile
// w / 4; the first and last steps (the diagonal tile and the one that may end
// past the sequence) apply the masks.  Q and dO tiles, and the tiles' lse and
// delta, come in by DMA into double-buffered LDS.  At the end the two tile
// parities' dK and dV are added through LDS.  With one query head per KV head
// the result goes to dqkv; otherwise each head's share goes to
// part[h % group][t][kv head][2 D] (fp32, dK then dV) and attn_reduce_kernel
// adds the group's shares in order.
template <int D>
__global__ __launch_bounds__(kSplitThreads, 1) void attn_dkdv_kernel(const bf16_t* __restrict__ qkv,
                                                                     const bf16_t* __restrict__ dO,
                                                                     const float* __restrict__ lse,
                                                                     const float* __restrict__ delta,
                                                                     bf16_t* __restrict__ dqkv,
                                                                     float* __restrict__ part, AttnDims dm) {
  constexpr int kTile = kAttnBlock * D * 2, KS = D / 32, EB = D / 16;
  constexpr bool kCF = D == 128;  // conflict-free tile layout (see Tile)
  using TL = Tile<D, kCF>;
  // One LDS object for the tiles and the statistics: with the reads' restrict
  // pointers the compiler can then tell that a step's reads do not touch what
  // the DMA in flight writes (with two objects it waits for that DMA first).
  struct Lds {
    char tiles[2][2][2][kTile];        // [buffer][tile of the step][Q, dO]
    float stat[2][2][2][kAttnBlock];   // [buffer][tile][lse, delta]
  };
  __shared__ __align__(16) Lds lds;
  auto& smem = lds.tiles;
  auto& stat = lds.stat;
  const int tid = threadIdx.x, lane = tid & 63, g = lane >> 4, c = lane & 15;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6), kw = w & 3, tp = w >> 2;
  const int nqb = (int)((dm.seq + kAttnBlock - 1) / kAttnBlock);
  const int per = dm.n_q * (int)dm.batch;
  const int rank = blockIdx.x;  // key block ascending: the heaviest first
  const int kb = rank / per, hq = (rank % per) / (int)dm.batch, b = rank % (int)dm.batch;
  const int kvh = hq / dm.group;
  const int64_t t0 = (int64_t)b * dm.seq, T = dm.batch * dm.seq;
  const int key = kb * kAttnBlock + 16 * kw + c;  // this lane's key (Y-operand row)
  const int64_t kcol = (int64_t)(dm.n_q + kvh) * D, vcol = (int64_t)(dm.n_q + dm.n_kv + kvh) * D;
  uint4 kf[KS], vf[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    const bool ok = key < dm.seq;
    kf[ks] = ok ? *reinterpret_cast<const uint4*>(qkv + (t0 + key) * dm.ld + kcol + 32 * ks + 8 * g)
                : make_uint4(0u, 0u, 0u, 0u);
    vf[ks] = ok ? *reinterpret_cast<const uint4*>(qkv + (t0 + key) * dm.ld + vcol + 32 * ks + 8 * g)
                : make_uint4(0u, 0u, 0u, 0u);
  }
  floatx4 dk[EB], dv[EB];
#pragma unroll
  for (int i = 0; i < EB; ++i) dk[i] = dv[i] = floatx4{0.f, 0.f, 0.f, 0.f};
  const TileDma<D, kSplitWaves, kCF> q_dma(qkv + t0 * dm.ld, dm.ld, dm.seq, w, lane);
  const TileDma<D, kSplitWaves, kCF> d_dma(dO + t0 * dm.ldo, dm.ldo, dm.seq, w, lane);
  // lse and delta of a tile: 64 floats each, one 4-byte DMA per tile and kind
  // (waves 0-3: tile w / 2 of the step, lse for even w, delta for odd).
  const float* stat_src = (w & 1) ? delta + (int64_t)hq * T + t0 : lse + (int64_t)hq * T + t0;
  const __amdgpu_buffer_rsrc_t stat_rsrc =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(stat_src), (short)0, (int)(dm.seq * 4), 0x00020000);
  const int ntiles = nqb - kb, nsteps = (ntiles + 1) / 2;
  auto issue_step = [&](int st, int buf) {
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const int qt = kb + 2 * st + t;
      if (qt < nqb) {
        q_dma.issue(smem[buf][t][0], qt, (int64_t)hq * D);
        d_dma.issue(smem[buf][t][1], qt, (int64_t)hq * D);
        if (w < 4 && (w >> 1) == t) {
          const int qq = qt * kAttnBlock + lane;
          __builtin_amdgcn_raw_ptr_buffer_load_lds(
              stat_rsrc, (__attribute__((address_space(3))) void*)&stat[buf][t][w & 1][0], 4,
              qq < dm.seq ? (unsigned)(lane * 4) : 0x80000000u, qt * kAttnBlock * 4, 0, 0);
        }
      }
    }
  };
  auto tile = [&](int qt, int buf, auto mask) {
    constexpr bool MASK = Flag<decltype(mask)>::value;
    const char* qtl = smem[buf][tp][0];
    const char* dtl = smem[buf][tp][1];
    const float* lse_t = stat[buf][tp][0];
    const float* del_t = stat[buf][tp][1];
    // S[q][key] and dP[q][key] for the tile's 4 x 16 queries; lane: q = 16 qq + 4 g + r, key = c
    floatx4 p[4], ds[4];
#pragma unroll
    for (int qq = 0; qq < 4; ++qq) {
      floatx4 sv = floatx4{0.f, 0.f, 0.f, 0.f}, dp = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        sv = mma(TL::row8(qtl, 16 * qq + c, 4 * ks + g), kf[ks], sv);
        dp = mma(TL::row8(dtl, 16 * qq + c, 4 * ks + g), vf[ks], dp);
      }
      const floatx4 l4 = lds_load4(lse_t + 16 * qq + 4 * g);
      const floatx4 d4 = lds_load4(del_t + 16 * qq + 4 * g);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        float pv = fast_exp2(__builtin_fmaf(sv[r], dm.scale_log2, -l4[r] * kLog2e));
        if constexpr (MASK) {
          const int qpos = qt * kAttnBlock + 16 * qq + 4 * g + r;
          if (!(key <= qpos && qpos < dm.seq && key < dm.seq)) pv = 0.0f;
        }
        p[qq][r] = pv;
        ds[qq][r] = pv * (dp[r] - d4[r]);
      }
    }
    // dV^T[e][key] += dO^T P, dK^T[e][key] += Q^T dS (the 1/sqrt(D) is applied at the end)
#pragma unroll
    for (int mm = 0; mm < 2; ++mm) {
      const uint4 pf = pack_slots1(p[2 * mm], p[2 * mm + 1]);
      const SlotPair sf = pack_slots(ds[2 * mm], ds[2 * mm + 1]);
#pragma unroll
      for (int eb = 0; eb < EB; ++eb) {
        dv[eb] = mma(TL::col8(dtl, mm, 16 * eb, lane), pf, dv[eb]);
        dk[eb] = mma2(TL::col8(qtl, mm, 16 * eb, lane), sf, dk[eb]);
      }
    }
  };
  issue_step(0, 0);
  __syncthreads();
  // The first step holds the diagonal tile, the last the sequence's last
  // tile; the steps in between hold neither.
  {
    if (nsteps > 1) issue_step(1, 1);
    const int qt = kb + tp;
    if (qt < nqb) tile(qt, 0, Masked{});
    __syncthreads();
  }
  for (int st = 1; st + 1 < nsteps; ++st) {
    const int buf = st & 1;
    issue_step(st + 1, buf ^ 1);
    tile(kb + 2 * st + tp, buf, Unmasked{});
    __syncthreads();
  }
  if (nsteps > 1) {
    const int st = nsteps - 1, qt = kb + 2 * st + tp;
    if (qt < nqb) tile(qt, st & 1, Masked{});
    __syncthreads();
  }
  // dK, dV = (even tiles) + (odd tiles), through LDS.
  constexpr int kX = 2 * EB * 4 * 64;
  float* xbase = reinterpret_cast<float*>(&smem[0][0][0][0]) + kw * kX;
  if (tp == 1) {
#pragma unroll
    for (int eb = 0; eb < EB; ++eb) {
      *reinterpret_cast<floatx4*>(xbase + (eb * 64 + lane) * 4) = dk[eb];
      *reinterpret_cast<floatx4*>(xbase + ((EB + eb) * 64 + lane) * 4) = dv[eb];
    }
  }
  __syncthreads();
  if (tp == 0 && key < dm.seq) {
#pragma unroll
    for (int eb = 0; eb < EB; ++eb) {
      dk[eb] += *reinterpret_cast<const floatx4*>(xbase + (eb * 64 + lane) * 4);
      dv[eb] += *reinterpret_cast<const floatx4*>(xbase + ((EB + eb) * 64 + lane) * 4);
    }
    if (dm.group == 1) {
      bf16_t* krow = dqkv + (t0 + key) * dm.ld + kcol;
      bf16_t* vrow = dqkv + (t0 + key) * dm.ld + vcol;
#pragma unroll
      for (int eb = 0; eb < EB; ++eb) {
        store4<bf16_t>(krow + 16 * eb + 4 * g, dk[eb] * dm.scale);
        store4<bf16_t>(vrow + 16 * eb + 4 * g, dv[eb]);
      }
    } else {
      float* row = part + (((int64_t)(hq % dm.group) * T + t0 + key) * dm.n_kv + kvh) * (2 * D);
#pragma unroll
      for (int eb = 0; eb < EB; ++eb) {
        store4<float>(row + 16 * eb + 4 * g, dk[eb] * dm.scale);
        store4<float>(row + D + 16 * eb + 4 * g, dv[eb]);
      }
    }
  }
}

// dqkv's K and V columns = the group's shares of part added in order.
template <int D>
__global__ __launch_bounds__(256) void attn_reduce_kernel(const float* __restrict__ part, bf16_t* __restrict__ dqkv,
                                                          AttnDims dm) {
  const int64_t T = dm.batch * dm.seq;
  const int64_t n4 = T * dm.n_kv * (2 * D) / 4;
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n4) return;
  const int64_t e4 = i * 4;  // element of a [T][n_kv][2 D] share
  const int64_t t = e4 / (dm.n_kv * 2 * D);
  const int rem = (int)(e4 % (dm.n_kv * 2 * D));
  const int kvh = rem / (2 * D), e = rem % (2 * D);
  floatx4 acc = load4<float>(part + e4);
  for (int j = 1; j < dm.group; ++j) acc += load4<float>(part + (int64_t)j * T * dm.n_kv * 2 * D + e4);
  const int64_t col = e < D ? (int64_t)(dm.n_q + kvh) * D + e : (int64_t)(dm.n_q + dm.n_kv + kvh) * D + (e - D);
  store4<bf16_t>(dqkv + t * dm.ld + col, acc);
}

// dQ of 64 queries of one head, split over 8 waves and two key tiles per
// step as in the forward; the four key parts' dQ are added through LDS at the
// end, in a fixed order.  Key tiles 0 .. qb, the last (the diagonal) with the
// masks.
template <int D>
__global__ __launch_bounds__(kSplitThreads, 1) void attn_dq_kernel(const bf16_t* __restrict__ qkv,
                                                                   const bf16_t* __restrict__ dO,
                                                                   const float* __restrict__ lse,
                                                                   const float* __restrict__ delta,
                                                                   bf16_t* __restrict__ dqkv, AttnDims dm) {
  constexpr int kTile = kAttnBlock * D * 2, KS = D / 32, EB = D / 16;
  __shared__ __align__(16) char smem[2][2][2][kTile];  // [buffer][tile of the step][K, V]
  const int tid = threadIdx.x, lane = tid & 63, g = lane >> 4, c = lane & 15;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6), qh = w & 1, kp = w >> 1, kh = kp & 1, tp = kp >> 1;
  const int nqb = (int)((dm.seq + kAttnBlock - 1) / kAttnBlock);
  int qb, h, b;
  block_coords(nqb, dm.n_q, (int)dm.batch, qb, h, b);
  const int kvh = h / dm.group;
  const int64_t t0 = (int64_t)b * dm.seq, T = dm.batch * dm.seq;
  const int q0 = qb * kAttnBlock + 32 * qh;
  uint4 qf[2][KS], df[2][KS];
  float lse2[2], dl[2];
#pragma unroll
  for (int jq = 0; jq < 2; ++jq) {
    const int q = q0 + 16 * jq + c;
    const bool ok = q < dm.seq;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      qf[jq][ks] = ok ? *reinterpret_cast<const uint4*>(qkv + (t0 + q) * dm.ld + (int64_t)h * D + 32 * ks + 8 * g)
                      : make_uint4(0u, 0u, 0u, 0u);
      df[jq][ks] = ok ? *reinterpret_cast<const uint4*>(dO + (t0 + q) * dm.ldo + (int64_t)h * D + 32 * ks + 8 * g)
                      : make_uint4(0u, 0u, 0u, 0u);
    }
    lse2[jq] = ok ? lse[(int64_t)h * T + t0 + q] * kLog2e : 0.0f;
    dl[jq] = ok ? delta[(int64_t)h * T + t0 + q] : 0.0f;
  }
  floatx4 dq[2][EB];
#pragma unroll
  for (int jq = 0; jq < 2; ++jq)
#pragma unroll
    for (int i = 0; i < EB; ++i) dq[jq][i] = floatx4{0.f, 0.f, 0.f, 0.f};
  const int64_t kcol = (int64_t)(dm.n_q + kvh) * D, vcol = (int64_t)(dm.n_q + dm.n_kv + kvh) * D;
  const TileDma<D, kSplitWaves> dma(qkv + t0 * dm.ld, dm.ld, dm.seq, w, lane);
  const int nsteps = (qb + 2) / 2;
  auto issue_step = [&](int st, int buf) {
#pragma unroll
    for (int t = 0; t < 2; ++t)
      if (2 * st + t <= qb) {
        dma.issue(smem[buf][t][0], 2 * st + t, kcol);
        dma.issue(smem[buf][t][1], 2 * st + t, vcol);
      }
  };
  issue_step(0, 0);
  __syncthreads();
  auto tile = [&](int kb, const char* kt, const char* vt, auto mask) {
    constexpr bool MASK = Flag<decltype(mask)>::value;
    // S^T[key][q], dP^T[key][q]; lane: key = 32 kh + 16 kk + 4 g + r (in the tile), q = q0 + 16 jq + c
    floatx4 ds[2][2];  // [kk][jq]
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      floatx4 sv[2], dp[2];
      sv[0] = sv[1] = dp[0] = dp[1] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const uint4 kf = Tile<D>::row8(kt, 32 * kh + 16 * kk + c, 4 * ks + g);
        const uint4 vf = Tile<D>::row8(vt, 32 * kh + 16 * kk + c, 4 * ks + g);
        sv[0] = mma(kf, qf[0][ks], sv[0]);
        sv[1] = mma(kf, qf[1][ks], sv[1]);
        dp[0] = mma(vf, df[0][ks], dp[0]);
        dp[1] = mma(vf, df[1][ks], dp[1]);
      }
#pragma unroll
      for (int jq = 0; jq < 2; ++jq)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          float pv = fast_exp2(__builtin_fmaf(sv[jq][r], dm.scale_log2, -lse2[jq]));
          if constexpr (MASK) {
            const int key = kb * kAttnBlock + 32 * kh + 16 * kk + 4 * g + r, q = q0 + 16 * jq + c;
            if (!(key <= q && key < dm.seq && q < dm.seq)) pv = 0.0f;
          }
          ds[kk][jq][r] = pv * (dp[jq][r] - dl[jq]);
        }
    }
    // dQ^T[e][q] += K^T dS^T over this wave's 32 keys
    const SlotPair sf0 = pack_slots(ds[0][0], ds[1][0]);
    const SlotPair sf1 = pack_slots(ds[0][1], ds[1][1]);
#pragma unroll
    for (int eb = 0; eb < EB; ++eb) {
      const uint4 kf = Tile<D>::col8(kt, kh, 16 * eb, lane);
      dq[0][eb] = mma2(kf, sf0, dq[0][eb]);
      dq[1][eb] = mma2(kf, sf1, dq[1][eb]);
    }
  };
  for (int st = 0; st + 1 < nsteps; ++st) {
    const int buf = st & 1;
    issue_step(st + 1, buf ^ 1);
    tile(2 * st + tp, smem[buf][tp][0], smem[buf][tp][1], Unmasked{});
    __syncthreads();
  }
  {
    const int st = nsteps - 1, buf = st & 1, kb = 2 * st + tp;
    if (kb < qb) tile(kb, smem[buf][tp][0], smem[buf][tp][1], Unmasked{});
    else if (kb == qb) tile(kb, smem[buf][tp][0], smem[buf][tp][1], Masked{});
    __syncthreads();
  }
  // dQ = the key parts added in kp order, through LDS.
  constexpr int kX = 2 * EB * 4 * 64;
  float* xbase = reinterpret_cast<float*>(&smem[0][0][0][0]);
  if (kp > 0) {
    float* x = xbase + ((kp - 1) * 2 + qh) * kX;
#pragma unroll
    for (int jq = 0; jq < 2; ++jq)
#pragma unroll
      for (int eb = 0; eb < EB; ++eb) *reinterpret_cast<floatx4*>(x + ((jq * EB + eb) * 64 + lane) * 4) = dq[jq][eb];
  }
  __syncthreads();
  if (kp == 0) {
#pragma unroll
    for (int jq = 0; jq < 2; ++jq) {
      const int q = q0 + 16 * jq + c;
      if (q < dm.seq) {
        bf16_t* dst = dqkv + (t0 + q) * dm.ld + (int64_t)h * D;
#pragma unroll
        for (int eb = 0; eb < EB; ++eb) {
          floatx4 v = dq[jq][eb];
#pragma unroll
          for (int p2 = 0; p2 < 3; ++p2)
            v += *reinterpret_cast<const floatx4*>(xbase + (p2 * 2 + qh) * kX + ((jq * EB + eb) * 64 + lane) * 4);
          store4<bf16_t>(dst + 16 * eb + 4 * g, v * dm.scale);
        }
      }
    }
  }
}

AttnDims make_dims(const AttnShapeArgs& a) {
  AttnDims d;
  d.batch = a.batch;
  d.seq = a.seq;
  d.ld = a.ld;
  d.ldo = (int64_t)a.n_q * a.head_dim;
  d.n_q = a.n_q;
  d.n_kv = a.n_kv;
  d.group = a.n_q / a.n_kv;
  d.scale = 1.0f / sqrtf((float)a.head_dim);
  d.scale_log2 = kLog2e * d.scale;
  return d;
}

template <int D>
hipError_t fwd_t(const AttnShapeArgs& a, const void* qkv, void* O, float* lse, hipStream_t s) {
  const AttnDims dm = make_dims(a);
  const int nqb = (int)((a.seq + kAttnBlock - 1) / kAttnBlock);
  KernelTimer timer("attention_fwd", s);
  hipLaunchKernelGGL(attn_fwd_kernel<D>, dim3(nqb * a.n_q * (int)a.batch), dim3(kSplitThreads), 0, s,
                     static_cast<const bf16_t*>(qkv), static_cast<bf16_t*>(O), lse, dm);
  return hipGetLastError();
}

template <int D>
hipError_t bwd_t(const AttnShapeArgs& a, const void* qkv, const void* O, const void* dO, const float* lse,
                 void* workspace, void* dqkv, hipStream_t s) {
  const AttnDims dm = make_dims(a);
  const int64_t T = a.batch * a.seq;
  const int nb = (int)((a.seq + kAttnBlock - 1) / kAttnBlock);
  float* delta = static_cast<float*>(workspace);
  float* part = reinterpret_cast<float*>(static_cast<char*>(workspace) + attention_delta_bytes(a));
  {
    KernelTimer timer("attention_delta", s);
    const int64_t n = T * a.n_q * (D / 8);  // threads: D / 8 per (head, token)
    hipLaunchKernelGGL(attn_delta_kernel<D>, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s,
                       static_cast<const bf16_t*>(O), static_cast<const bf16_t*>(dO), delta, T, a.n_q, dm.ldo);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  {
    KernelTimer timer("attention_bwd_dkdv", s);
    hipLaunchKernelGGL(attn_dkdv_kernel<D>, dim3(nb * a.n_q * (int)a.batch), dim3(kSplitThreads), 0, s,
                       static_cast<const bf16_t*>(qkv), static_cast<const bf16_t*>(dO), lse, delta,
                       static_cast<bf16_t*>(dqkv), part, dm);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (dm.group > 1) {
    KernelTimer timer("attention_bwd_reduce", s);
    const int64_t n4 = T * a.n_kv * 2 * D / 4;
    hipLaunchKernelGGL(attn_reduce_kernel<D>, dim3((unsigned)((n4 + 255) / 256)), dim3(256), 0, s, part,
                       static_cast<bf16_t*>(dqkv), dm);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  KernelTimer timer("attention_bwd_dq", s);
  hipLaunchKernelGGL(attn_dq_kernel<D>, dim3(nb * a.n_q * (int)a.batch), dim3(kSplitThreads), 0, s,
                     static_cast<const bf16_t*>(qkv), static_cast<const bf16_t*>(dO), lse, delta,
                     static_cast<bf16_t*>(dqkv), dm);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attention_fwd(const AttnShapeArgs& a, const void* qkv, void* O, float* lse, hipStream_t s) {
  if (a.batch == 0 || a.seq == 0) return hipSuccess;
  if (a.head_dim == 64) return fwd_t<64>(a, qkv, O, lse, s);
  if (a.head_dim == 128) return fwd_t<128>(a, qkv, O, lse, s);
  return hipErrorInvalidValue;
}

size_t attention_delta_bytes(const AttnShapeArgs& a) {
  return ((size_t)a.n_q * (size_t)(a.batch * a.seq) * sizeof(float) + 255) / 256 * 256;
}

size_t attention_bwd_workspace(const AttnShapeArgs& a) {
  const size_t part = a.n_q == a.n_kv ? 0 : (size_t)a.n_q * (size_t)(a.batch * a.seq) * 2 * a.head_dim * sizeof(float);
  return attention_delta_bytes(a) + part;
}

hipError_t launch_attention_bwd(const AttnShapeArgs& a, const void* qkv, const void* O, const void* dO,
                                const float* lse, void* workspace, void* dqkv, hipStream_t s) {
  if (a.batch == 0 || a.seq == 0) return hipSuccess;
  if (a.head_dim == 64) return bwd_t<64>(a, qkv, O, dO, lse, workspace, dqkv, s);
  if (a.head_dim == 128) return bwd_t<128>(a, qkv, O, dO, lse, workspace, dqkv, s);
  return hipErrorInvalidValue;
}

}  // namespace tpmlp
