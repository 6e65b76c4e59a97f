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
// Forward: one workgroup per (query block of 64, head, batch), 4 waves of 16
// queries; K and V tiles of 64 keys in LDS; online softmax in exp2 with the
// 1/sqrt(D) scale folded in.  The probabilities P and the score gradients dS
// enter their products as a bf16 pair (hi + lo, see pack_slots).  Backward
// (no atomics): dK and dV per (key block of 64, query head, batch) over the
// query blocks at or after the key block, the shares of a group's query heads
// then added in a fixed order by a small kernel; dQ per (query block, head,
// batch) over the key blocks up to it; both recompute P from lse and use
// delta = rowsum(dO o O) from a small kernel.  Every loop issues the global
// loads of its next tile before the products of the current one.
#include "common.h"
#include "kernels.h"

namespace tpmlp {
namespace {

constexpr int kAttnBlock = 64, kAttnThreads = 256;
constexpr float kLog2e = 1.4426950408889634f, kLn2 = 0.6931471805599453f;

typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;

__device__ __forceinline__ floatx4 mma(const uint4& x, const uint4& y, floatx4 acc) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, x), __builtin_bit_cast(bf16x8, y), acc,
                                                 0, 0, 0);
}

// A [64][D] bf16 tile in LDS, 16-byte chunks XOR-swizzled by row.
template <int D>
struct Tile {
  static constexpr int kChunks = D / 8;  // 16-byte chunks per row
  __device__ __forceinline__ static int chunk_off(int row, int chunk) {
    return (row * kChunks + (chunk ^ (row & (kChunks - 1)))) * 16;
  }
  // Row `row`, elements 8 c .. 8 c + 7.
  __device__ __forceinline__ static uint4 row8(const char* base, int row, int c) {
    return *reinterpret_cast<const uint4*>(base + chunk_off(row, c));
  }
  // Column fragment for this lane (X or Y operand row e0 + l % 16) at the 8
  // rows 32 m + 16 h + 4 (l / 16) + j, h < 2, j < 4: two transpose reads.
  __device__ __forceinline__ static uint4 col8(const char* base, int m, int e0, int lane) {
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
  // A tile's worth of this thread's chunks, staged in registers so the next
  // tile's global loads overlap the current tile's products.
  static constexpr int kPer = kAttnBlock * kChunks / kAttnThreads;
  struct Regs {
    uint4 v[kPer];
  };
  // Global rows r0 .. r0 + 63 (ld elements apart), columns col0 .. col0 + D - 1;
  // rows at or past `rows` are zero.
  __device__ __forceinline__ static void fetch(Regs& r, const bf16_t* src, int64_t ld, int64_t r0, int64_t rows,
                                               int64_t col0, int tid) {
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int idx = tid + kAttnThreads * i;
      const int row = idx / kChunks, c = idx % kChunks;
      r.v[i] = make_uint4(0u, 0u, 0u, 0u);
      if (r0 + row < rows) r.v[i] = *reinterpret_cast<const uint4*>(src + (r0 + row) * ld + col0 + 8 * c);
    }
  }
  __device__ __forceinline__ static void store(char* base, const Regs& r, int tid) {
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int idx = tid + kAttnThreads * i;
      *reinterpret_cast<uint4*>(base + chunk_off(idx / kChunks, idx % kChunks)) = r.v[i];
    }
  }
};

// The lane's 8 k-slot values of one 32-row step m from its two 16-row blocks
// (block 2m: slots 0-3, block 2m + 1: slots 4-7) as two bf16 operands whose
// sum carries the fp32 value to 2^-17: hi = bf16(v), lo = bf16(v - hi).  P and
// dS are the only product operands formed inside the kernels (Q, K, V and dO
// are bf16 tensors already); two MFMAs on the same other operand keep their
// products at fp32-like precision, as the oracle's exact probabilities.
struct SlotPair {
  uint4 hi, lo;
};
__device__ __forceinline__ SlotPair pack_slots(const floatx4& b0, const floatx4& b1) {
  float v[8] = {b0[0], b0[1], b0[2], b0[3], b1[0], b1[1], b1[2], b1[3]};
  uint32_t h[4], l[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const bf16_t h0 = f32_to_bf16(v[2 * i]), h1 = f32_to_bf16(v[2 * i + 1]);
    const bf16_t l0 = f32_to_bf16(v[2 * i] - bf16_to_f32(h0)), l1 = f32_to_bf16(v[2 * i + 1] - bf16_to_f32(h1));
    h[i] = (uint32_t)h0 | ((uint32_t)h1 << 16);
    l[i] = (uint32_t)l0 | ((uint32_t)l1 << 16);
  }
  return SlotPair{make_uint4(h[0], h[1], h[2], h[3]), make_uint4(l[0], l[1], l[2], l[3])};
}

__device__ __forceinline__ floatx4 mma2(const uint4& x, const SlotPair& y, floatx4 acc) {
  return mma(x, y.lo, mma(x, y.hi, acc));
}

struct AttnDims {
  int64_t batch, seq, ld, ldo;  // ld: row length of qkv / dqkv; ldo: of O / dO (n_q D)
  int n_q, n_kv, group;
  float scale_log2;             // log2(e) / sqrt(D)
  float scale;                  // 1 / sqrt(D)
};

// blockIdx -> (block index, head, batch), the block index descending so that
// the longest causal rows start first.
__device__ __forceinline__ void block_coords(int nblocks, int heads, int batch, int& blk, int& head, int& b) {
  const int x = blockIdx.x, per = heads * batch;
  blk = nblocks - 1 - x / per;
  head = (x % per) / batch;
  b = x % batch;
}

template <int D>
__global__ __launch_bounds__(kAttnThreads) void attn_fwd_kernel(const bf16_t* __restrict__ qkv, bf16_t* __restrict__ O,
                                                                float* __restrict__ lse, AttnDims dm) {
  __shared__ __align__(16) char ktile[kAttnBlock * D * 2];
  __shared__ __align__(16) char vtile[kAttnBlock * D * 2];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, g = lane >> 4, c = lane & 15;
  const int nqb = (int)((dm.seq + kAttnBlock - 1) / kAttnBlock);
  int qb, h, b;
  block_coords(nqb, dm.n_q, (int)dm.batch, qb, h, b);
  const int kvh = h / dm.group;
  const int64_t t0 = (int64_t)b * dm.seq;
  const int q = qb * kAttnBlock + 16 * w + c;  // this lane's query position
  constexpr int KS = D / 32, EB = D / 16;
  uint4 qf[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks)
    qf[ks] = q < dm.seq ? *reinterpret_cast<const uint4*>(qkv + (t0 + q) * dm.ld + (int64_t)h * D + 32 * ks + 8 * g)
                        : make_uint4(0u, 0u, 0u, 0u);
  floatx4 acc[EB];
#pragma unroll
  for (int i = 0; i < EB; ++i) acc[i] = floatx4{0.f, 0.f, 0.f, 0.f};
  float m = -INFINITY, lsum = 0.0f;
  const int64_t kcol = (int64_t)(dm.n_q + kvh) * D, vcol = (int64_t)(dm.n_q + dm.n_kv + kvh) * D;
  const int nkb = qb + 1;  // key blocks 0 .. qb hold every key <= a query of this block
  const bf16_t* src = qkv + t0 * dm.ld;
  typename Tile<D>::Regs kr, vr;
  Tile<D>::fetch(kr, src, dm.ld, 0, dm.seq, kcol, tid);
  Tile<D>::fetch(vr, src, dm.ld, 0, dm.seq, vcol, tid);
  for (int kb = 0; kb < nkb; ++kb) {
    __syncthreads();  // the previous tiles are no longer read
    Tile<D>::store(ktile, kr, tid);
    Tile<D>::store(vtile, vr, tid);
    __syncthreads();
    if (kb + 1 < nkb) {  // the next tiles load while these are multiplied
      Tile<D>::fetch(kr, src, dm.ld, (int64_t)(kb + 1) * kAttnBlock, dm.seq, kcol, tid);
      Tile<D>::fetch(vr, src, dm.ld, (int64_t)(kb + 1) * kAttnBlock, dm.seq, vcol, tid);
    }
    floatx4 s[4];
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      s[kk] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) s[kk] = mma(Tile<D>::row8(ktile, 16 * kk + c, 4 * ks + g), qf[ks], s[kk]);
    }
    float bmax = -INFINITY;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int key = kb * kAttnBlock + 16 * kk + 4 * g + r;
        s[kk][r] = (key <= q && key < dm.seq) ? s[kk][r] * dm.scale_log2 : -INFINITY;
        bmax = fmaxf(bmax, s[kk][r]);
      }
    bmax = fmaxf(bmax, __shfl_xor(bmax, 16, kWave));
    bmax = fmaxf(bmax, __shfl_xor(bmax, 32, kWave));
    const float mnew = fmaxf(m, bmax);
    const float alpha = exp2f(m - mnew);  // m = -inf on the first block: alpha = 0
    m = mnew;
    lsum *= alpha;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        s[kk][r] = exp2f(s[kk][r] - mnew);
        lsum += s[kk][r];
      }
#pragma unroll
    for (int i = 0; i < EB; ++i) acc[i] *= alpha;
#pragma unroll
    for (int mm = 0; mm < 2; ++mm) {
      const SlotPair pf = pack_slots(s[2 * mm], s[2 * mm + 1]);
#pragma unroll
      for (int eb = 0; eb < EB; ++eb) acc[eb] = mma2(Tile<D>::col8(vtile, mm, 16 * eb, lane), pf, acc[eb]);
    }
  }
  lsum += __shfl_xor(lsum, 16, kWave);
  lsum += __shfl_xor(lsum, 32, kWave);
  if (q < dm.seq) {
    const float inv = 1.0f / lsum;
    bf16_t* dst = O + (t0 + q) * dm.ldo + (int64_t)h * D;
#pragma unroll
    for (int eb = 0; eb < EB; ++eb) store4<bf16_t>(dst + 16 * eb + 4 * g, acc[eb] * inv);
    if (g == 0) lse[(int64_t)h * dm.batch * dm.seq + t0 + q] = (m + log2f(lsum)) * kLn2;
  }
}

// delta[h][t] = sum_e dO[t][h D + e] O[t][h D + e]
template <int D>
__global__ __launch_bounds__(256) void attn_delta_kernel(const bf16_t* __restrict__ O, const bf16_t* __restrict__ dO,
                                                          float* __restrict__ delta, int64_t T, int n_q, int64_t ldo) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= T * n_q) return;
  const int h = (int)(i / T);
  const int64_t t = i % T;
  const bf16_t* o = O + t * ldo + (int64_t)h * D;
  const bf16_t* d = dO + t * ldo + (int64_t)h * D;
  float acc = 0.0f;
#pragma unroll
  for (int c = 0; c < D / 8; ++c) {
    float a[8], e[8];
    Chunk<bf16_t>::unpack(*reinterpret_cast<const uint4*>(o + 8 * c), a);
    Chunk<bf16_t>::unpack(*reinterpret_cast<const uint4*>(d + 8 * c), e);
#pragma unroll
    for (int k = 0; k < 8; ++k) acc += a[k] * e[k];
  }
  delta[(int64_t)h * T + t] = acc;
}

// dK and dV of 64 keys from one query head (one workgroup per key block,
// query head and sequence; the key blocks with the most query blocks after
// them are dispatched first): every query block at or after the key block.
// Wave w owns keys 16 w .. 16 w + 15.  With one query head per KV head the
// result goes to dqkv; otherwise each head's share goes to
// part[h % group][t][kv head][2 D] (fp32, dK then dV) and attn_reduce_kernel
// adds the group's shares in order.
template <int D>
__global__ __launch_bounds__(kAttnThreads) void attn_dkdv_kernel(const bf16_t* __restrict__ qkv,
                                                                 const bf16_t* __restrict__ dO,
                                                                 const float* __restrict__ lse,
                                                                 const float* __restrict__ delta,
                                                                 bf16_t* __restrict__ dqkv, float* __restrict__ part,
                                                                 AttnDims dm) {
  __shared__ __align__(16) char qtile[kAttnBlock * D * 2];
  __shared__ __align__(16) char dotile[kAttnBlock * D * 2];
  __shared__ float lse2_s[kAttnBlock], delta_s[kAttnBlock];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, g = lane >> 4, c = lane & 15;
  const int nkb = (int)((dm.seq + kAttnBlock - 1) / kAttnBlock);
  const int per = dm.n_q * (int)dm.batch;
  const int kb = blockIdx.x / per, hq = (blockIdx.x % per) / (int)dm.batch, b = blockIdx.x % (int)dm.batch;
  const int kvh = hq / dm.group;
  const int64_t t0 = (int64_t)b * dm.seq, T = dm.batch * dm.seq;
  const int key = kb * kAttnBlock + 16 * w + c;  // this lane's key (Y-operand row)
  constexpr int KS = D / 32, EB = D / 16;
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
  const int nqb = nkb;
  const bf16_t* qsrc = qkv + t0 * dm.ld;
  const bf16_t* dsrc = dO + t0 * dm.ldo;
  typename Tile<D>::Regs qr, dr;
  float lr = 0.0f, dl = 0.0f;
  auto fetch = [&](int qb) {
    Tile<D>::fetch(qr, qsrc, dm.ld, (int64_t)qb * kAttnBlock, dm.seq, (int64_t)hq * D, tid);
    Tile<D>::fetch(dr, dsrc, dm.ldo, (int64_t)qb * kAttnBlock, dm.seq, (int64_t)hq * D, tid);
    if (tid < kAttnBlock) {
      const int qq = qb * kAttnBlock + tid;
      const bool ok = qq < dm.seq;
      lr = ok ? lse[(int64_t)hq * T + t0 + qq] * kLog2e : 0.0f;
      dl = ok ? delta[(int64_t)hq * T + t0 + qq] : 0.0f;
    }
  };
  fetch(kb);
  for (int qb = kb; qb < nqb; ++qb) {
    __syncthreads();
    Tile<D>::store(qtile, qr, tid);
    Tile<D>::store(dotile, dr, tid);
    if (tid < kAttnBlock) {
      lse2_s[tid] = lr;
      delta_s[tid] = dl;
    }
    __syncthreads();
    if (qb + 1 < nqb) fetch(qb + 1);
    // S[q][key] and dP[q][key] for the block's 4 x 16 queries; lane: q = 16 qq + 4 g + r, key = c
    floatx4 p[4], ds[4];
#pragma unroll
    for (int qq = 0; qq < 4; ++qq) {
      floatx4 sv = floatx4{0.f, 0.f, 0.f, 0.f}, dp = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        sv = mma(Tile<D>::row8(qtile, 16 * qq + c, 4 * ks + g), kf[ks], sv);
        dp = mma(Tile<D>::row8(dotile, 16 * qq + c, 4 * ks + g), vf[ks], dp);
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int ql = 16 * qq + 4 * g + r, qpos = qb * kAttnBlock + ql;
        const bool ok = key <= qpos && qpos < dm.seq && key < dm.seq;
        const float pv = ok ? exp2f(sv[r] * dm.scale_log2 - lse2_s[ql]) : 0.0f;
        p[qq][r] = pv;
        ds[qq][r] = pv * (dp[r] - delta_s[ql]);
      }
    }
    // dV^T[e][key] += dO^T P, dK^T[e][key] += Q^T dS (the 1/sqrt(D) is applied at the end)
#pragma unroll
    for (int mm = 0; mm < 2; ++mm) {
      const SlotPair pf = pack_slots(p[2 * mm], p[2 * mm + 1]);
      const SlotPair sf = pack_slots(ds[2 * mm], ds[2 * mm + 1]);
#pragma unroll
      for (int eb = 0; eb < EB; ++eb) {
        dv[eb] = mma2(Tile<D>::col8(dotile, mm, 16 * eb, lane), pf, dv[eb]);
        dk[eb] = mma2(Tile<D>::col8(qtile, mm, 16 * eb, lane), sf, dk[eb]);
      }
    }
  }
  if (key < dm.seq) {
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

// dQ of 64 queries of one head: every key block up to the query block.
template <int D>
__global__ __launch_bounds__(kAttnThreads) void attn_dq_kernel(const bf16_t* __restrict__ qkv,
                                                               const bf16_t* __restrict__ dO,
                                                               const float* __restrict__ lse,
                                                               const float* __restrict__ delta,
                                                               bf16_t* __restrict__ dqkv, AttnDims dm) {
  __shared__ __align__(16) char ktile[kAttnBlock * D * 2];
  __shared__ __align__(16) char vtile[kAttnBlock * D * 2];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, g = lane >> 4, c = lane & 15;
  const int nqb = (int)((dm.seq + kAttnBlock - 1) / kAttnBlock);
  int qb, h, b;
  block_coords(nqb, dm.n_q, (int)dm.batch, qb, h, b);
  const int kvh = h / dm.group;
  const int64_t t0 = (int64_t)b * dm.seq, T = dm.batch * dm.seq;
  const int q = qb * kAttnBlock + 16 * w + c;
  constexpr int KS = D / 32, EB = D / 16;
  uint4 qf[KS], df[KS];
  const bool qok = q < dm.seq;
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    qf[ks] = qok ? *reinterpret_cast<const uint4*>(qkv + (t0 + q) * dm.ld + (int64_t)h * D + 32 * ks + 8 * g)
                 : make_uint4(0u, 0u, 0u, 0u);
    df[ks] = qok ? *reinterpret_cast<const uint4*>(dO + (t0 + q) * dm.ldo + (int64_t)h * D + 32 * ks + 8 * g)
                 : make_uint4(0u, 0u, 0u, 0u);
  }
  const float lse2 = qok ? lse[(int64_t)h * T + t0 + q] * kLog2e : 0.0f;
  const float dl = qok ? delta[(int64_t)h * T + t0 + q] : 0.0f;
  floatx4 dq[EB];
#pragma unroll
  for (int i = 0; i < EB; ++i) dq[i] = floatx4{0.f, 0.f, 0.f, 0.f};
  const int64_t kcol = (int64_t)(dm.n_q + kvh) * D, vcol = (int64_t)(dm.n_q + dm.n_kv + kvh) * D;
  const bf16_t* src = qkv + t0 * dm.ld;
  typename Tile<D>::Regs kr, vr;
  Tile<D>::fetch(kr, src, dm.ld, 0, dm.seq, kcol, tid);
  Tile<D>::fetch(vr, src, dm.ld, 0, dm.seq, vcol, tid);
  for (int kb = 0; kb <= qb; ++kb) {
    __syncthreads();
    Tile<D>::store(ktile, kr, tid);
    Tile<D>::store(vtile, vr, tid);
    __syncthreads();
    if (kb + 1 <= qb) {
      Tile<D>::fetch(kr, src, dm.ld, (int64_t)(kb + 1) * kAttnBlock, dm.seq, kcol, tid);
      Tile<D>::fetch(vr, src, dm.ld, (int64_t)(kb + 1) * kAttnBlock, dm.seq, vcol, tid);
    }
    // S^T[key][q], dP^T[key][q]; lane: key = 16 kk + 4 g + r, q = c
    floatx4 ds[4];
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      floatx4 s = floatx4{0.f, 0.f, 0.f, 0.f}, dp = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        s = mma(Tile<D>::row8(ktile, 16 * kk + c, 4 * ks + g), qf[ks], s);
        dp = mma(Tile<D>::row8(vtile, 16 * kk + c, 4 * ks + g), df[ks], dp);
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int key = kb * kAttnBlock + 16 * kk + 4 * g + r;
        const bool ok = key <= q && key < dm.seq && qok;
        const float pv = ok ? exp2f(s[r] * dm.scale_log2 - lse2) : 0.0f;
        ds[kk][r] = pv * (dp[r] - dl);
      }
    }
    // dQ^T[e][q] += K^T dS^T
#pragma unroll
    for (int mm = 0; mm < 2; ++mm) {
      const SlotPair sf = pack_slots(ds[2 * mm], ds[2 * mm + 1]);
#pragma unroll
      for (int eb = 0; eb < EB; ++eb) dq[eb] = mma2(Tile<D>::col8(ktile, mm, 16 * eb, lane), sf, dq[eb]);
    }
  }
  if (qok) {
    bf16_t* dst = dqkv + (t0 + q) * dm.ld + (int64_t)h * D;
#pragma unroll
    for (int eb = 0; eb < EB; ++eb) store4<bf16_t>(dst + 16 * eb + 4 * g, dq[eb] * dm.scale);
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
  hipLaunchKernelGGL(attn_fwd_kernel<D>, dim3(nqb * a.n_q * (int)a.batch), dim3(kAttnThreads), 0, s,
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
    const int64_t n = T * a.n_q;
    hipLaunchKernelGGL(attn_delta_kernel<D>, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s,
                       static_cast<const bf16_t*>(O), static_cast<const bf16_t*>(dO), delta, T, a.n_q, dm.ldo);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  {
    KernelTimer timer("attention_bwd_dkdv", s);
    hipLaunchKernelGGL(attn_dkdv_kernel<D>, dim3(nb * a.n_q * (int)a.batch), dim3(kAttnThreads), 0, s,
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
  hipLaunchKernelGGL(attn_dq_kernel<D>, dim3(nb * a.n_q * (int)a.batch), dim3(kAttnThreads), 0, s,
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
