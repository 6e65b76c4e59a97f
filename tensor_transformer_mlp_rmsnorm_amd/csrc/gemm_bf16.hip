// bf16 MFMA GEMM for the six contractions of the MLP sublayer (gfx950 / CDNA4).
//
//   C[m, n] = sum_k A(m, k) B(k, n),  A(m,k) = A[m*lda + k] (a_kcontig) or A[k*lda + m],
//                                     B(k,n) = B[n*ldb + k] (b_kcontig) or B[k*ldb + n].
//
// One 512-thread workgroup computes a 256 x 256 output tile (variant: 224-wide
// tiles where they fill the CUs better, below):
//  * 8 waves in a 2 (M) x 4 (N) grid; each wave owns 128 x 64 outputs as 8 x 4
//    blocks of v_mfma_f32_16x16x32_bf16 (128 fp32 accumulators per lane).  The
//    LDS bytes read per flop are a quarter of what a 64 x 64 wave tile needs.
//  * k is staged 64 at a time.  A K-contiguous operand is stored [row][64 k]
//    (128-byte rows, 16-byte chunks XOR-swizzled by row); an MN-contiguous
//    operand is stored as it lies in memory, [k][256 rows] (512-byte rows,
//    chunks XOR-swizzled by k), and its MFMA fragments are read with the gfx950
//    LDS transpose read (ds_read_b64_tr_b16): in each 16-lane group, result lane
//    i element j is the (i mod 4)-th 16-bit value at the address of lane
//    4j + i/4, so lanes that point at 4 consecutive k-rows x 4 column quads
//    receive 4 consecutive k of one column.  Two such reads give the 8 k-values
//    of an MFMA operand.
//  * Global -> LDS with buffer_load_dwordx4 ... lds (no staging registers).
//  * Two schedules:
//    - both operands K-contiguous (the forward GEMMs): ping-pong.  The wave
//      groups 0-3 (tile rows 0-127) and 4-7 (rows 128-255), one wave of each on
//      every SIMD, run one phase apart: while one group reads a k-tile's
//      fragments from LDS and issues tile loads, the other multiplies the tile
//      it read before, so the matrix unit of each SIMD has a wave feeding it in
//      every phase and the multiplying wave never stalls on a memory
//      instruction.  LDS is a ring of 5 operand slots of 32 KiB: operand tile x
//      (A of k-tile j is x = 2j, B is 2j+1) sits in slot x mod 5, so a slot is
//      refilled only after both groups have read it.  A 256 x 224 tile (2 x 2
//      waves of 64 x 112 per group) serves N that 224 divides into fewer rounds
//      of the CUs, except for the SwiGLU forward.
//    - otherwise (a transposed operand): two LDS stages of 64 KiB; all waves
//      read and multiply each k-tile in step, with the next k-tile's loads issued
//      first and one barrier per k-tile.  The transpose reads are slower, and
//      with the phases of a ping-pong the read phase would outlast the multiply
//      phase; here both share every phase.  On the 224 x 256 tile and on the
//      256 x 256 tile with A K-contiguous and B MN-contiguous the loop is
//      pipelined by half a k-tile: a wave reads the fragments of the next
//      k-half before it multiplies the current one, so its LDS reads are in
//      flight under its own MFMAs.
//  * B is the MFMA's first operand, so a lane's accumulator holds 4 consecutive
//    output columns of one row and the epilogues work on 4-wide vectors.
//  * Tile order: each of the 8 XCDs gets a contiguous range of tile ids
//    (workgroups are dealt round-robin over XCDs), grouped by 4 tile-rows.
//  * SwiGLU forward ("Split the expansion", synapticradio.com: gate and up
//    channels stay paired): a tile covers 128 FFN channels; each wave's 64 B
//    rows are 32 gate channels followed by the same 32 up channels, so one lane
//    holds g and u of the same (token, channel).
#include "common.h"
#include "kernels.h"

namespace tpmlp {
namespace {

constexpr int kBM = 256, kBN = 256, kBK = 64, kThreads = 512;
constexpr int kSwigluChannels = 128;               // FFN channels per tile in the SwiGLU forward
constexpr int kTileU4 = 256 * kBK * 2 / 16;        // uint4 per operand tile (32 KiB)
constexpr int kStageU4 = 2 * kTileU4;              // A + B (two-stage schedule)
constexpr int kSlots = 5;                          // operand slots (ping-pong schedule)

// Output tile shapes of the two-stage kernel: the tile (TM x TN), its wave grid
// (NW waves, GN of them along N) and each wave's 16 x 16 MFMA blocks (WMB x
// WNB).  Loads always fill 256-row operand tiles; a 224-wide tile just leaves 32
// of them unused.  224 = 7 x 32 makes 1792- and 3584-wide GEMMs exactly 8 and 16
// tiles.
struct Tile256x256 {
  static constexpr int TM = 256, TN = 256, NW = 8, GN = 4, WMB = 8, WNB = 4;
};
struct Tile256x224 {
  static constexpr int TM = 256, TN = 224, NW = 8, GN = 2, WMB = 4, WNB = 7;
};
struct Tile224x256 {
  static constexpr int TM = 224, TN = 256, NW = 8, GN = 4, WMB = 7, WNB = 4;
};

typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));

// 4 values rounded to bf16 as store4<bf16_t> stores them.
__device__ __forceinline__ uint2 pack_bf16x4(floatx4 v) {
  return make_uint2((uint32_t)f32_to_bf16(v[0]) | ((uint32_t)f32_to_bf16(v[1]) << 16),
                    (uint32_t)f32_to_bf16(v[2]) | ((uint32_t)f32_to_bf16(v[3]) << 16));
}
typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;
typedef __attribute__((address_space(3))) char lds_char;

// K-contiguous tile [256 rows][8 chunks of 8 k]: chunk index XOR (row & 7).
__device__ __forceinline__ int kc_index(int row, int chunk) { return row * 8 + (chunk ^ (row & 7)); }
// MN-contiguous tile [64 k][32 chunks of 8 rows]: chunk index XOR f(k), f in
// {0,2,..,14}: the 4 k-rows of one transpose-read group land in distinct bank
// quads, and so do the k-rows 8 apart read by the next lane group.
__device__ __forceinline__ int mn_swz(int k) { return ((k & 3) << 1) ^ (((k >> 3) & 1) << 3); }
__device__ __forceinline__ int mn_index(int k, int chunk) { return k * 32 + (chunk ^ mn_swz(k)); }

// Physical row of logical tile row r (or -1 outside the operand).  SwiGLU B
// tiles: each wave's 2 x chans rows are chans gate channels followed by the
// same chans up channels (32 per wave in 256-row tiles, 56 in 224-row ones;
// rows past the tile's `rows` are not loaded).
struct RowMap {
  int64_t base, limit;
  bool swiglu;
  int64_t ffn;
  int chans = 32, rows = 256;
  __device__ __forceinline__ int64_t operator()(int r) const {
    if (!swiglu) {
      const int64_t g = base + r;
      return g < limit ? g : -1;
    }
    if (r >= rows) return -1;
    const int wave_n = r / (2 * chans), w = r - wave_n * 2 * chans;
    const int64_t ch = base + wave_n * chans + (w < chans ? w : w - chans);
    return ch < ffn ? (w < chans ? 0 : ffn) + ch : -1;
  }
};

// Global -> LDS without registers: buffer_load_dwordx4 ... lds writes a
// wave's 64 x 16 bytes to 1 KiB of LDS at the wave-uniform address in M0, lane
// j at byte 16 j.  Each of NW waves fills 32 / NW such blocks of each operand tile, and each
// lane fetches the global chunk that belongs at its LDS slot, so the swizzle is
// applied on the global side.  Lanes outside the operand (rows past M or N, k
// past K) use an offset beyond the buffer's size, for which the buffer unit's
// range check returns zeros: ragged tiles are zero-padded without branches.
constexpr unsigned kOutOfRange = 0x80000000u;  // every operand is < 2 GiB (checked on the host)

struct Operand {
  __amdgpu_buffer_rsrc_t rsrc;
  int64_t ld;
};

__device__ __forceinline__ Operand make_operand(const void* p, int64_t rows, int64_t ld, int elem_bytes = 2) {
  const int64_t bytes = rows * ld * (int64_t)elem_bytes;
  return Operand{__builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)bytes, 0x00020000), ld};
}

template <bool KC, int EB = 2, int NW = 8>
__device__ __forceinline__ void issue_tile(const Operand& op, uint4* __restrict__ lds_tile, const RowMap& rm,
                                           int64_t k0, int64_t K, int wave, int lane) {
  static_assert(KC || EB == 2, "MN-contiguous tiles hold bf16");
  static_assert(NW == 8 || NW == 16, "32 blocks per operand tile");
  constexpr int kChunkElems = 16 / EB;
  constexpr int kPerWave = 32 / NW;
#pragma unroll
  for (int i = 0; i < kPerWave; ++i) {
    const int b = wave * kPerWave + i;  // 1 KiB block of the tile
    unsigned off = kOutOfRange;
    if constexpr (KC) {
      const int r = 8 * b + (lane >> 3);
      const int c = (lane & 7) ^ (r & 7);  // kc_index(r, c) == r * 8 + (lane & 7)
      const int64_t grow = rm(r), gk = k0 + kChunkElems * c;
      if (grow >= 0 && gk < K) off = (unsigned)((grow * op.ld + gk) * EB);
    } else {
      const int kr = 2 * b + (lane >> 5);
      const int c = (lane & 31) ^ mn_swz(kr);  // mn_index(kr, c) == kr * 32 + (lane & 31)
      const int64_t gk = k0 + kr, mn = rm.base + 8 * c;
      if (gk < K && mn < rm.limit) off = (unsigned)((gk * op.ld + mn) * 2);
    }
    __builtin_amdgcn_raw_ptr_buffer_load_lds(op.rsrc, (__attribute__((address_space(3))) void*)(lds_tile + b * 64),
                                             16, off, 0, 0, 0);
  }
}

// Ping-pong loads: a wave's quarter of a K-contiguous operand tile, blocks
// 8 q .. 8 q + 7 (rows 64 q .. 64 q + 63).  The lane-dependent part of each
// block's offset is formed once per kernel; the block-dependent part, the same
// for all lanes, goes in the instruction's SGPR offset.  A block that lies
// wholly past the operand gets SGPR offset 0, so the sum stays below 2^31 and a
// lane marked out of range (VGPR offset 0x80000000) stays out of range.
// SwiGLU B tiles (CH channels per wave, RowMap's layout): every 8-row block is
// 8 consecutive channels of one plane.
template <bool SWIGLU, int EB = 2, int CH = 32>
struct QuarterLoads {
  static_assert(CH == 32 || CH == 56, "SwiGLU tiles of 4 x 32 or 2 x 56 channels");
  unsigned vbase;     // byte offset of this lane's chunk in block 0
  int left;           // rows (SwiGLU: channels) from this lane's block-0 row to the operand's end, clamped
  int k8;             // this lane's k offset inside the tile
  int64_t first_row;  // block 0's first row (SwiGLU: channel), the same for all lanes
  int64_t lim;        // rows (SwiGLU: channels) of the operand

  __device__ __forceinline__ QuarterLoads(const Operand& op, const RowMap& rm, int q, int lane) {
    const int lr = lane >> 3;       // row inside an 8-row block
    const int c = (lane & 7) ^ lr;  // stored chunk: block rows start at multiples of 8
    // SwiGLU, 32 channels per wave: logical row 64 q + 8 i + lr is channel base + 32 q + 8 (i & 3) + lr
    // of plane i >> 2; 56 per wave: channels are counted from the tile's base (see issue)
    first_row = SWIGLU ? (CH == 32 ? rm.base + 32 * q : rm.base) : rm.base + 64 * q;
    lim = SWIGLU ? rm.ffn : rm.limit;
    const int64_t d = lim - (first_row + lr);
    left = d > (1 << 20) ? (1 << 20) : (d < -1 ? -1 : (int)d);
    vbase = (unsigned)(((first_row + lr) * op.ld + (16 / EB) * c) * EB);
    k8 = (16 / EB) * c;
  }

  __device__ __forceinline__ void issue(const Operand& op, uint4* __restrict__ lds_tile, int q, int64_t k0, int64_t K) {
    asm volatile("" : "+v"(vbase), "+v"(left), "+v"(k8));  // keep the 8 block offsets from being precomputed
    uint4* dst = lds_tile + 8 * q * 64;
    const bool kok = k0 + k8 < K;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      int dr;             // row (SwiGLU: channel) step of block i within its plane
      int64_t plane = 0;  // SwiGLU: the plane's first row
      bool used = true;   // 224-row tiles: blocks 28-31 are loaded as zeros (the load count stays fixed)
      if constexpr (SWIGLU && CH == 56) {
        const int b = 8 * q + i, wb = b % 14;  // block b: wave b / 14, plane wb / 7
        dr = 56 * (b / 14) + 8 * (wb % 7);
        plane = (wb / 7) * lim;
        used = b < 28;
      } else {
        dr = SWIGLU ? 8 * (i & 3) : 8 * i;
        plane = SWIGLU ? (i >> 2) * lim : 0;
      }
      const bool block_in = used && first_row + dr < lim;  // the same for all lanes
      const unsigned soff = block_in ? (unsigned)(((plane + dr) * op.ld + k0) * EB) : 0u;
      const unsigned voff = (kok && used && dr < left) ? vbase : kOutOfRange;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(op.rsrc, (__attribute__((address_space(3))) void*)(dst + i * 64), 16,
                                               voff, (int)soff, 0, 0);
    }
  }
};

// MFMA operand fragment: 16 rows starting at `row0`, k = 32*s + 8*(lane/16) .. +7.
template <bool KC>
__device__ __forceinline__ uint4 read_frag(const uint4* __restrict__ lds, int row0, int s, int lane) {
  if constexpr (KC) {
    return lds[kc_index(row0 + (lane & 15), 4 * s + (lane >> 4))];
  } else {
    const int g = lane >> 4, sl = lane & 15;
    const int mn = row0 + 4 * (sl & 3);
    const int c = mn >> 3, half = (mn >> 2) & 1;
    lds_char* base = (lds_char*)(lds);
    uint2 out[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int k = 32 * s + 8 * g + 4 * h + (sl >> 2);
      const int off = mn_index(k, c) * 16 + half * 8;
      bf16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(base + off));
      out[h] = __builtin_bit_cast(uint2, v);
    }
    return make_uint4(out[0].x, out[0].y, out[1].x, out[1].y);
  }
}

// blockIdx -> (tile_m, tile_n, k slice): each of the 8 XCDs gets a contiguous
// range of ids (workgroups are dealt round-robin over XCDs); k slices are the
// slowest index, tiles inside a slice are grouped by `group` tile-rows (0: 4).
__device__ __forceinline__ void tile_coords(int pid, int ntm, int ntn, int nks, int group, int& tm, int& tn,
                                            int& ks) {
  const int ntiles = ntm * ntn, total = ntiles * nks;
  const int xcd = pid & 7, local = pid >> 3;
  const int per = total >> 3, rem = total & 7;
  const int lin = (xcd < rem) ? xcd * (per + 1) + local : rem * (per + 1) + (xcd - rem) * per + local;
  ks = lin / ntiles;
  const int tile = lin - ks * ntiles;
  const int kg = group > 0 ? group : 4;
  const int in_group = kg * ntn;
  const int gi = tile / in_group;
  const int first_m = gi * kg;
  const int gsize = min(ntm - first_m, kg);
  const int t = tile - gi * in_group;
  tm = first_m + t % gsize;
  tn = t / gsize;
}

template <int WMB, int WNB>
__device__ __forceinline__ void mma_half(floatx4 (&acc)[WMB][WNB], const uint4 (&af)[WMB], const uint4 (&bf)[WNB]) {
#pragma unroll
  for (int i = 0; i < WMB; ++i)
#pragma unroll
    for (int j = 0; j < WNB; ++j)
      acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, bf[j]),
                                                          __builtin_bit_cast(bf16x8, af[i]), acc[i][j], 0, 0, 0);
}

template <bool AK, bool BKC, int WMB, int WNB>
__device__ __forceinline__ void read_half(uint4 (&af)[WMB], uint4 (&bf)[WNB], const uint4* stage, int s, int wm,
                                          int wn, int lane) {
#pragma unroll
  for (int i = 0; i < WMB; ++i) af[i] = read_frag<AK>(stage, wm * WMB * 16 + i * 16, s, lane);
#pragma unroll
  for (int j = 0; j < WNB; ++j) bf[j] = read_frag<BKC>(stage + kTileU4, wn * WNB * 16 + j * 16, s, lane);
}

// Epilogue of the activation backward GEMMs:
// d_act = acc meets the saved pre-activation ([g | u] rows of 2F for SwiGLU,
// h rows of N for GeLU), and d_pre is stored in the same layout.  The saved
// values of one 16-row block are loaded a block ahead, all at once and
// unconditionally (addresses clamped into the tensor; lanes outside it discard
// what they read), so a wave waits for memory about once per block instead of
// once per load; only the stores are guarded.
// With STASH, the stored bf16 bits of each block's dg and du (or dh) are also
// left in stash[i][j][0 | 1] for the transposed copy.
template <int EPI, int WMB, int WNB, bool STASH = false>
__device__ __forceinline__ void epilogue_act_bwd(const GemmArgs& g, const floatx4 (&acc)[WMB][WNB], int64_t m0,
                                                 int64_t n0, int lane, uint2 (*stash)[WNB][2] = nullptr) {
  static_assert(EPI == kEpiSwigluBwd || EPI == kEpiGeluBwd, "activation backward epilogues only");
  constexpr bool kSwiglu = EPI == kEpiSwigluBwd;
  constexpr int NL = kSwiglu ? 2 : 1;  // saved tensors per output: g and u, or h
  const int64_t M = g.M, N = g.N;
  const int64_t ld = kSwiglu ? 2 * g.ffn : N;  // row length of the saved and the stored tensor
  const int64_t second = kSwiglu ? g.ffn : 0;  // offset of u after g
  asm volatile("" : "+v"(lane));
  const int col4 = 4 * (lane >> 4), frow = lane & 15;
  const bf16_t* __restrict__ aux = static_cast<const bf16_t*>(g.aux);
  bf16_t* __restrict__ out = static_cast<bf16_t*>(g.pre);
  uint2 buf[2][WNB][NL];
  auto load_block = [&](int i, uint2 (&dst)[WNB][NL]) {
    const int64_t m = min(m0 + i * 16 + frow, M - 1);
#pragma unroll
    for (int j = 0; j < WNB; ++j) {
      const int64_t n = min(n0 + j * 16 + col4, N - 4);  // N is a multiple of 4
#pragma unroll
      for (int l = 0; l < NL; ++l) dst[j][l] = *reinterpret_cast<const uint2*>(aux + m * ld + l * second + n);
    }
  };
  auto unpack = [](uint2 u) {
    floatx4 r;
    r[0] = __uint_as_float(u.x << 16);
    r[1] = __uint_as_float(u.x & 0xffff0000u);
    r[2] = __uint_as_float(u.y << 16);
    r[3] = __uint_as_float(u.y & 0xffff0000u);
    return r;
  };
  // When the wave's whole tile of saved values fits in the registers the main
  // loop has freed (56 loads of 8 bytes: the 64 x 112 wave tile with g and u),
  // every load is issued before the first is used, so the tile's reads are in
  // flight together; otherwise one 16-row block ahead.
  constexpr bool kAllAhead = WMB * WNB * NL <= 56;
  uint2 all[kAllAhead ? WMB : 1][WNB][NL];
  if constexpr (kAllAhead) {
#pragma unroll
    for (int i = 0; i < WMB; ++i) load_block(i, all[i]);
  } else {
    load_block(0, buf[0]);
  }
#pragma unroll
  for (int i = 0; i < WMB; ++i) {
    if (!kAllAhead && i + 1 < WMB) load_block(i + 1, buf[(i + 1) & 1]);
    const uint2 (&cur)[WNB][NL] = kAllAhead ? all[kAllAhead ? i : 0] : buf[i & 1];
    const int64_t m = m0 + i * 16 + frow;
#pragma unroll
    for (int j = 0; j < WNB; ++j) {
      const int64_t n = n0 + j * 16 + col4;
      const floatx4 v = acc[i][j];
      if constexpr (kSwiglu) {
        const floatx4 gv = unpack(cur[j][0]), uv = unpack(cur[j][NL - 1]);
        floatx4 dg, du;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float sg = sigmoid_f(gv[r]);
          dg[r] = v[r] * uv[r] * sg * (1.0f + gv[r] * (1.0f - sg));
          du[r] = v[r] * gv[r] * sg;
        }
        if (m < M && n < N) {
          store4<bf16_t>(out + m * ld + n, dg);
          store4<bf16_t>(out + m * ld + second + n, du);
        }
        if constexpr (STASH) {
          stash[i][j][0] = pack_bf16x4(dg);
          stash[i][j][1] = pack_bf16x4(du);
        }
      } else {
        const floatx4 h = unpack(cur[j][0]);
        floatx4 dh;
#pragma unroll
        for (int r = 0; r < 4; ++r) dh[r] = v[r] * gelu_grad_f(h[r]);
        if (m < M && n < N) store4<bf16_t>(out + m * ld + n, dh);
        if constexpr (STASH) stash[i][j][0] = pack_bf16x4(dh);
      }
    }
  }
}

// Epilogue: acc holds this wave's (16 WMB) x (16 WNB) outputs from row m0 and
// column n0 (SwiGLU forward: 32 channels from ch0, gate blocks then up blocks);
// see the Epi enum.
// SwiGLU forward on a 224-row B tile: a wave's 7 blocks of 16 B rows are 56
// gate channels (blocks 0-2 and lane groups 0-1 of block 3) followed by the
// same 56 up channels (lane groups 2-3 of block 3 and blocks 4-6).  Lane group
// G of gate block j holds channels 16 j + 4 G .. + 3; their up values sit in
// lane group G + 2 of block j + 3 (G < 2) or G - 2 of block j + 4 (G >= 2), 32
// lanes away in the same row.  v_permlane32_swap of blocks j + 3 and j + 4
// (the first operand's lanes 32-63 take the second's lanes 0-31 and the second's
// lanes 0-31 take the first's lanes 32-63) brings both halves beside the gate
// values.  Every lane runs the exchanges; only the stores are guarded.
template <int WMB>
__device__ __forceinline__ void epilogue_swiglu224(const GemmArgs& g, const floatx4 (&acc)[WMB][7], int64_t m0,
                                                   int64_t ch0, int lane) {
  const int64_t M = g.M, F = g.ffn;
  const int G = lane >> 4, frow = lane & 15;
  const bool lo = lane < 32;
  auto swap = [](float a, float b) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(a), __float_as_uint(b), false, false);
    return make_float2(__uint_as_float(r[0]), __uint_as_float(r[1]));
  };
#pragma unroll
  for (int i = 0; i < WMB; ++i) {
    const int64_t m = m0 + i * 16 + frow;
    const bool mok = m < M;
    // g and u are stored tensors: the activation is formed from their stored values
    floatx4 sv[7];
#pragma unroll
    for (int j = 0; j < 7; ++j) sv[j] = stored<bf16_t>(acc[i][j]);
    bf16_t* pre = static_cast<bf16_t*>(g.pre) + m * 2 * F;
    bf16_t* act = static_cast<bf16_t*>(g.act) + m * F;
#pragma unroll
    for (int j = 0; j < 7; ++j) {
      const int r = 16 * j + 4 * G;  // the wave's B row of this lane's first value
      const int64_t ch = ch0 + (r < 56 ? r : r - 56);
      if (mok && ch < F) store4<bf16_t>(pre + (r < 56 ? 0 : F) + ch, sv[j]);
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      floatx4 uv;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        // block 3's gate half (lanes 0-31) takes block 6's upper half
        const float2 t = j < 3 ? swap(sv[j + 3][e], sv[j + 4][e]) : swap(sv[6][e], sv[6][e]);
        uv[e] = lo ? t.y : t.x;
      }
      floatx4 av;
#pragma unroll
      for (int e = 0; e < 4; ++e) av[e] = sv[j][e] * sigmoid_f(sv[j][e]) * uv[e];
      const int64_t ch = ch0 + 16 * j + 4 * G;
      if (mok && ch < F && (j < 3 || lo)) store4<bf16_t>(act + ch, av);
    }
  }
}

template <int EPI, int WMB, int WNB>
__device__ __forceinline__ void epilogue(const GemmArgs& g, const floatx4 (&acc)[WMB][WNB], int64_t m0, int64_t n0,
                                         int64_t ch0, int ks, int lane) {
  if constexpr (EPI == kEpiSwigluBwd || EPI == kEpiGeluBwd) {
    epilogue_act_bwd<EPI, WMB, WNB>(g, acc, m0, n0, lane);
    return;
  }
  if constexpr (EPI == kEpiSwigluFwd && WNB == 7) {
    epilogue_swiglu224<WMB>(g, acc, m0, ch0, lane);
  } else {
  const int64_t M = g.M, N = g.N, F = g.ffn;
  asm volatile("" : "+v"(lane));  // addresses are formed here, not kept live through the main loop
  const int col4 = 4 * (lane >> 4), frow = lane & 15;
#pragma unroll
  for (int i = 0; i < WMB; ++i) {
    const int64_t m = m0 + i * 16 + frow;
    if (m >= M) continue;
    if constexpr (EPI == kEpiSwigluFwd) {
      static_assert(WNB == 4, "SwiGLU pairing: 2 gate blocks then 2 up blocks per wave");
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int64_t ch = ch0 + j * 16 + col4;
        if (ch >= F) continue;
        // g and u are stored tensors: the activation is formed from their stored values
        const floatx4 gv = stored<bf16_t>(acc[i][j]), uv = stored<bf16_t>(acc[i][j + 2]);
        floatx4 av;
#pragma unroll
        for (int r = 0; r < 4; ++r) av[r] = gv[r] * sigmoid_f(gv[r]) * uv[r];
        bf16_t* pre = static_cast<bf16_t*>(g.pre) + m * 2 * F;
        store4<bf16_t>(pre + ch, gv);
        store4<bf16_t>(pre + F + ch, uv);
        store4<bf16_t>(static_cast<bf16_t*>(g.act) + m * F + ch, av);
      }
    } else {
#pragma unroll
      for (int j = 0; j < WNB; ++j) {
        const int64_t n = n0 + j * 16 + col4;
        if (n >= N) continue;
        const floatx4 v = acc[i][j];
        if constexpr (EPI == kEpiStoreF32) {
          float* c = ks == 0 ? static_cast<float*>(g.C) : g.ws + (int64_t)(ks - 1) * M * g.ldc;
          store4<float>(c + m * g.ldc + n, (g.accum && ks == 0) ? v + load4<float>(c + m * g.ldc + n) : v);
        } else if constexpr (EPI == kEpiStoreBf16) {
          store4<bf16_t>(static_cast<bf16_t*>(g.C) + m * g.ldc + n, v);
        } else if constexpr (EPI == kEpiResidual) {
          const floatx4 xr = load4<bf16_t>(static_cast<const bf16_t*>(g.aux) + m * g.ldc + n);
          const floatx4 bb = load4<bf16_t>(static_cast<const bf16_t*>(g.bias) + n);
          store4<bf16_t>(static_cast<bf16_t*>(g.C) + m * g.ldc + n, v + xr + bb);
        } else if constexpr (EPI == kEpiGeluFwd) {
          const floatx4 bb = load4<bf16_t>(static_cast<const bf16_t*>(g.bias) + n);
          const floatx4 h = stored<bf16_t>(v + bb);
          floatx4 a;
#pragma unroll
          for (int r = 0; r < 4; ++r) a[r] = gelu_f(h[r]);
          store4<bf16_t>(static_cast<bf16_t*>(g.pre) + m * N + n, h);
          store4<bf16_t>(static_cast<bf16_t*>(g.act) + m * N + n, a);
        }
      }
    }
  }
  }
}


// Transposed stores of an output tile through LDS (the main loop's LDS is
// free by then).  A lane holds 4 consecutive columns ln .. ln + 3 of one tile
// row lm; the tile is staged as [columns][TM + 8] bf16 (a column of the tile
// becomes a row): lanes of neighbouring rows (lane ^ 1) swap halves so that
// each writes whole dwords holding two rows of one column, and the 16-byte row
// pad puts the 8 rows one dword store touches in distinct banks.  Then every
// thread writes 16-byte chunks of the staged rows.
template <int kPitch>
__device__ __forceinline__ void stage_t4(bf16_t* lds, int lm, int ln, uint2 bits, bool odd) {
  const uint32_t b0 = bits.x & 0xffffu, b1 = bits.x >> 16, b2 = bits.y & 0xffffu, b3 = bits.y >> 16;
  // even lanes (row lm) keep columns 0, 1 and take the odd neighbour's (row lm + 1); odd lanes keep
  // columns 2, 3 and take the even neighbour's (row lm - 1)
  const uint32_t send = odd ? (b0 | (b1 << 16)) : (b2 | (b3 << 16));
  const uint32_t recv = (uint32_t)__shfl_xor((int)send, 1, kWave);
  const int c0 = odd ? 2 : 0, r0 = odd ? lm - 1 : lm;
  const uint32_t lo = odd ? (recv & 0xffffu) | (b2 << 16) : b0 | (recv << 16);
  const uint32_t hi = odd ? (recv >> 16) | (b3 << 16) : b1 | (recv & 0xffff0000u);
  *reinterpret_cast<uint32_t*>(lds + (ln + c0) * kPitch + r0) = lo;
  *reinterpret_cast<uint32_t*>(lds + (ln + c0 + 1) * kPitch + r0) = hi;
}

// The staged tile's rows c < TN (tile columns n0 + c < N) to dst[(n0 + c) * ld + m0 + r], r < TM
// (m0 + r < M; M a multiple of 8, so a 16-byte chunk is wholly inside or outside).
template <int TM, int TN, int NTHREADS>
__device__ __forceinline__ void store_t_tile(const bf16_t* lds, bf16_t* dst, int64_t ld, int64_t m0, int64_t n0,
                                             int64_t M, int64_t N) {
  constexpr int kPitch = TM + 8, kChunks = TM / 8;
  for (int c = threadIdx.x; c < TN * kChunks; c += NTHREADS) {
    const int ln = c / kChunks, lc = (c - ln * kChunks) * 8;
    const int64_t n = n0 + ln, m = m0 + lc;
    if (n < N && m < M)
      *reinterpret_cast<uint4*>(dst + n * ld + m) = *reinterpret_cast<const uint4*>(lds + ln * kPitch + lc);
  }
}

template <int TM, int TN>
constexpr size_t t_stage_bytes() {
  return (size_t)TN * (TM + 8) * sizeof(bf16_t);
}

// kEpiSgd / kEpiSgdT: the product is the gradient of a bf16 weight and the SGD
// step is taken here, so the gradient never goes to memory.  Each lane updates
// its 4 consecutive columns of a row exactly as the SGD kernels do (sgd_value:
// one fma, then the round to bf16) and stores them in the product's layout;
// the transposed layout goes through LDS (stage_t4, store_t_tile).
//   kEpiSgd:  the product is dW, W [M, N]: old values from w_in (or the
//             masters m_in), W to w_out directly, W^T [N, M] to w_out_t.
//   kEpiSgdT: the product is dW^T, W [N, M]: old values from w_in_t (W^T, in
//             the product's layout), W^T to w_out_t directly, W to w_out.
// The tile is TM x TN from (tile_m0, tile_n0), the wave's blocks from (wr0,
// wc0) within it; NTHREADS threads per workgroup.
template <int TM, int TN, int WMB, int WNB, int NTHREADS, bool MASTER, bool ROLE_T>
__device__ __forceinline__ void epilogue_sgd(const GemmArgs& g, const floatx4 (&acc)[WMB][WNB], int64_t tile_m0,
                                             int64_t tile_n0, int wr0, int wc0, int lane, uint4* smem) {
  static_assert(!(MASTER && ROLE_T), "the transposed-role update keeps no masters");
  constexpr int kPitch = TM + 8;  // bf16 per LDS row (one column of the tile)
  const int64_t M = g.M, N = g.N;
  const SgdEpi& u = g.sgd;
  const float lr = u.lr;
  const bf16_t* __restrict__ src = static_cast<const bf16_t*>(ROLE_T ? u.w_in_t : u.w_in);
  bf16_t* const direct = static_cast<bf16_t*>(ROLE_T ? u.w_out_t : u.w_out);
  bf16_t* const trans = static_cast<bf16_t*>(ROLE_T ? u.w_out : u.w_out_t);
  bf16_t* const lds = reinterpret_cast<bf16_t*>(smem);
  const int frow = lane & 15, col4 = 4 * (lane >> 4);
  const bool odd = lane & 1;
  __syncthreads();  // every wave is past its last read of the main loop's LDS
#pragma unroll
  for (int i = 0; i < WMB; ++i) {
    const int lm = wr0 + i * 16 + frow;  // row of the product within the tile
    const int64_t m = tile_m0 + lm;
    floatx4 p[WNB];
#pragma unroll
    for (int j = 0; j < WNB; ++j) {  // the old values of the row's blocks, loaded together
      const int64_t n = tile_n0 + wc0 + j * 16 + col4;
      const bool ok = m < M && n < N;  // (N is a multiple of 4: the lane's 4 columns are whole)
      if constexpr (MASTER) p[j] = ok ? load4<float>(u.m_in + m * N + n) : floatx4{0.f, 0.f, 0.f, 0.f};
      else p[j] = ok ? load4<bf16_t>(src + m * N + n) : floatx4{0.f, 0.f, 0.f, 0.f};
    }
#pragma unroll
    for (int j = 0; j < WNB; ++j) {
      const int ln = wc0 + j * 16 + col4;  // column of the product within the tile
      const int64_t n = tile_n0 + ln;
      const floatx4 v = sgd_value4(p[j], acc[i][j], lr);
      if (m < M && n < N) {
        if constexpr (MASTER) store4<float>(u.m_out + m * N + n, v);
        if (direct) store4<bf16_t>(direct + m * N + n, v);
      }
      if (trans) stage_t4<kPitch>(lds, lm, ln, pack_bf16x4(v), odd);
    }
  }
  if (!trans) return;  // (uniform)
  __syncthreads();
  store_t_tile<TM, TN, NTHREADS>(lds, trans, M, tile_m0, tile_n0, M, N);
}

// Ping-pong fragment reads: the 24 ds_read_b128 of one k-tile (A: 8 row blocks,
// B: 4, each for k 0-31 and 32-63) in one block that also waits for them.  No
// LDS read is left in flight past it, and the compiler does not add its own
// wait on the tile loads still in flight (it cannot tell they write other
// slots).  abase/bbase: this lane's byte address in the first A / B fragment;
// row block r is 2048 bytes further, and the k 32-63 chunk is at address ^ 64.
template <int WMB, int WNB>
struct Frags {
  uint4 a[2][WMB], b[2][WNB];
};

__device__ __forceinline__ void read_frags_kc(Frags<8, 4>& f, unsigned abase, unsigned bbase) {
  asm volatile(
      "ds_read_b128 %0, %24 offset:0\n"
      "ds_read_b128 %1, %24 offset:2048\n"
      "ds_read_b128 %2, %24 offset:4096\n"
      "ds_read_b128 %3, %24 offset:6144\n"
      "ds_read_b128 %4, %24 offset:8192\n"
      "ds_read_b128 %5, %24 offset:10240\n"
      "ds_read_b128 %6, %24 offset:12288\n"
      "ds_read_b128 %7, %24 offset:14336\n"
      "ds_read_b128 %8, %25 offset:0\n"
      "ds_read_b128 %9, %25 offset:2048\n"
      "ds_read_b128 %10, %25 offset:4096\n"
      "ds_read_b128 %11, %25 offset:6144\n"
      "ds_read_b128 %12, %26 offset:0\n"
      "ds_read_b128 %13, %26 offset:2048\n"
      "ds_read_b128 %14, %26 offset:4096\n"
      "ds_read_b128 %15, %26 offset:6144\n"
      "ds_read_b128 %16, %26 offset:8192\n"
      "ds_read_b128 %17, %26 offset:10240\n"
      "ds_read_b128 %18, %26 offset:12288\n"
      "ds_read_b128 %19, %26 offset:14336\n"
      "ds_read_b128 %20, %27 offset:0\n"
      "ds_read_b128 %21, %27 offset:2048\n"
      "ds_read_b128 %22, %27 offset:4096\n"
      "ds_read_b128 %23, %27 offset:6144\n"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(f.a[0][0]), "=&v"(f.a[0][1]), "=&v"(f.a[0][2]), "=&v"(f.a[0][3]), "=&v"(f.a[0][4]), "=&v"(f.a[0][5]),
        "=&v"(f.a[0][6]), "=&v"(f.a[0][7]), "=&v"(f.b[0][0]), "=&v"(f.b[0][1]), "=&v"(f.b[0][2]), "=&v"(f.b[0][3]),
        "=&v"(f.a[1][0]), "=&v"(f.a[1][1]), "=&v"(f.a[1][2]), "=&v"(f.a[1][3]), "=&v"(f.a[1][4]), "=&v"(f.a[1][5]),
        "=&v"(f.a[1][6]), "=&v"(f.a[1][7]), "=&v"(f.b[1][0]), "=&v"(f.b[1][1]), "=&v"(f.b[1][2]), "=&v"(f.b[1][3])
      : "v"(abase), "v"(bbase), "v"(abase ^ 64u), "v"(bbase ^ 64u)
      : "memory");
}

// The same for a 64 x 112 wave tile (A: 4 row blocks, B: 7): 22 reads.
__device__ __forceinline__ void read_frags_kc(Frags<4, 7>& f, unsigned abase, unsigned bbase) {
  asm volatile(
      "ds_read_b128 %0, %22 offset:0\n"
      "ds_read_b128 %1, %22 offset:2048\n"
      "ds_read_b128 %2, %22 offset:4096\n"
      "ds_read_b128 %3, %22 offset:6144\n"
      "ds_read_b128 %4, %23 offset:0\n"
      "ds_read_b128 %5, %23 offset:2048\n"
      "ds_read_b128 %6, %23 offset:4096\n"
      "ds_read_b128 %7, %23 offset:6144\n"
      "ds_read_b128 %8, %23 offset:8192\n"
      "ds_read_b128 %9, %23 offset:10240\n"
      "ds_read_b128 %10, %23 offset:12288\n"
      "ds_read_b128 %11, %24 offset:0\n"
      "ds_read_b128 %12, %24 offset:2048\n"
      "ds_read_b128 %13, %24 offset:4096\n"
      "ds_read_b128 %14, %24 offset:6144\n"
      "ds_read_b128 %15, %25 offset:0\n"
      "ds_read_b128 %16, %25 offset:2048\n"
      "ds_read_b128 %17, %25 offset:4096\n"
      "ds_read_b128 %18, %25 offset:6144\n"
      "ds_read_b128 %19, %25 offset:8192\n"
      "ds_read_b128 %20, %25 offset:10240\n"
      "ds_read_b128 %21, %25 offset:12288\n"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(f.a[0][0]), "=&v"(f.a[0][1]), "=&v"(f.a[0][2]), "=&v"(f.a[0][3]), "=&v"(f.b[0][0]), "=&v"(f.b[0][1]),
        "=&v"(f.b[0][2]), "=&v"(f.b[0][3]), "=&v"(f.b[0][4]), "=&v"(f.b[0][5]), "=&v"(f.b[0][6]), "=&v"(f.a[1][0]),
        "=&v"(f.a[1][1]), "=&v"(f.a[1][2]), "=&v"(f.a[1][3]), "=&v"(f.b[1][0]), "=&v"(f.b[1][1]), "=&v"(f.b[1][2]),
        "=&v"(f.b[1][3]), "=&v"(f.b[1][4]), "=&v"(f.b[1][5]), "=&v"(f.b[1][6])
      : "v"(abase), "v"(bbase), "v"(abase ^ 64u), "v"(bbase ^ 64u)
      : "memory");
}

// Wave tiles of the ping-pong kernel: the two groups (waves 0-3 and 4-7) own
// tile rows 0-127 and 128-255; inside a group a wave owns 128 x 64 (PpTile256,
// 256-wide tiles) or 64 x 112 (PpTile224: 2 x 2 waves over 128 x 224, for N
// that 224 divides into fewer rounds of the CUs).
struct PpTile256 {
  static constexpr int TN = 256, WMB = 8, WNB = 4;
  __device__ __forceinline__ static int row0(int wave) { return (wave >> 2) * 128; }
  __device__ __forceinline__ static int col0(int wave) { return (wave & 3) * 64; }
};
struct PpTile224 {
  static constexpr int TN = 224, WMB = 4, WNB = 7;
  __device__ __forceinline__ static int row0(int wave) { return (wave >> 2) * 128 + ((wave >> 1) & 1) * 64; }
  __device__ __forceinline__ static int col0(int wave) { return (wave & 1) * 112; }
};

// Operand element types of the ping-pong kernel: bf16, or FP8 codes in the
// OCP formats FA (of A) and FB (of B), with the MFMA's format numbering
// (0 = E4M3, 1 = E5M2).  A k-tile is 128 bytes of every row in both cases:
// 64 bf16 or 128 FP8 values.
struct PpBf16 {
  static constexpr int kBytes = 2;
  static constexpr bool kFp8 = false;
};
template <int FA, int FB>
struct PpFp8 {
  static constexpr int kBytes = 1;
  static constexpr bool kFp8 = true;
};

template <int WMB, int WNB>
__device__ __forceinline__ void mma_tile(floatx4 (&acc)[WMB][WNB], const Frags<WMB, WNB>& f, PpBf16) {
#pragma unroll
  for (int s = 0; s < kBK / 32; ++s)
#pragma unroll
    for (int i = 0; i < WMB; ++i)
#pragma unroll
      for (int j = 0; j < WNB; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, f.b[s][j]),
                                                            __builtin_bit_cast(bf16x8, f.a[s][i]), acc[i][j], 0, 0, 0);
}

typedef int intx4 __attribute__((ext_vector_type(4)));
typedef int intx8 __attribute__((ext_vector_type(8)));
constexpr int kUnitScales = 0x7f7f7f7f;  // E8M0 block scales of 2^0: the scaled MFMA without scaling

// FP8: one 16 x 16 x 128 MFMA per block and k-tile.  A lane's 32-byte operand
// is its row's k chunks (lane / 16) and 4 + lane / 16 -- the two 16-byte
// fragments the bf16 schedule reads for its two k halves.  Any assignment of
// the 128 k to lane bytes gives the same sums as long as A and B use the same
// one, and they do.
template <int FA, int FB, int WMB, int WNB>
__device__ __forceinline__ void mma_tile(floatx4 (&acc)[WMB][WNB], const Frags<WMB, WNB>& f, PpFp8<FA, FB>) {
  intx8 bv[WNB];
#pragma unroll
  for (int j = 0; j < WNB; ++j)
    bv[j] = __builtin_shufflevector(__builtin_bit_cast(intx4, f.b[0][j]), __builtin_bit_cast(intx4, f.b[1][j]), 0, 1,
                                    2, 3, 4, 5, 6, 7);
#pragma unroll
  for (int i = 0; i < WMB; ++i) {
    const intx8 av = __builtin_shufflevector(__builtin_bit_cast(intx4, f.a[0][i]), __builtin_bit_cast(intx4, f.a[1][i]),
                                             0, 1, 2, 3, 4, 5, 6, 7);
#pragma unroll
    for (int j = 0; j < WNB; ++j)
      acc[i][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(bv[j], av, acc[i][j], FB, FA, 0, kUnitScales, 0,
                                                                   kUnitScales);
  }
}

// Phase boundary: wait until at most VM of this wave's tile loads are in flight
// (kNoVm: no wait on them) and its LDS reads are done, then the workgroup
// barrier.  The scheduling barriers keep the compiler from moving work across.
constexpr int kNoVm = 63;
template <int VM>
__device__ __forceinline__ void phase_end() {
  static_assert(VM >= 0 && VM < 64, "vmcnt range");
  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_s_waitcnt((VM & 15) | ((VM >> 4) << 14) | 0x0070);  // vmcnt(VM) expcnt(7) lgkmcnt(0)
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_sched_barrier(0);
}

__device__ __forceinline__ int slot_u4(int x) { return (x % kSlots) * kTileU4; }

template <int EPI, class OP, class PT = PpTile256>
__global__ __launch_bounds__(kThreads, 1) void gemm_nt_pingpong_kernel(GemmArgs g, int ntm, int ntn) {
  extern __shared__ uint4 smem[];  // 5 operand slots = 160 KiB
  constexpr bool kSwiglu = EPI == kEpiSwigluFwd;
  // SwiGLU: channels per wave and per tile (256-row B tiles: 4 waves of 32; 224-row: 2 waves of 56)
  constexpr int kWaveChans = PT::TN == 256 ? 32 : 56, kTileChans = PT::TN == 256 ? 128 : 112;
  constexpr int WMB = PT::WMB, WNB = PT::WNB;
  constexpr int EB = OP::kBytes;
  constexpr int kK = 128 / EB;  // k per tile

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 2, q = wave & 3;

  int tm, tn, ks;
  tile_coords(blockIdx.x, ntm, ntn, g.ksplit, g.tile_group, tm, tn, ks);
  const int64_t K = g.K;
  const int64_t kper = ((K + (int64_t)g.ksplit * kK - 1) / ((int64_t)g.ksplit * kK)) * kK;
  const int64_t kbeg = (int64_t)ks * kper;
  const int64_t kend = K < kbeg + kper ? K : kbeg + kper;
  const RowMap ra{(int64_t)tm * kBM, g.M, false, 0};
  const RowMap rb = kSwiglu ? RowMap{(int64_t)tn * kTileChans, g.N, true, g.ffn, kWaveChans, PT::TN}
                            : RowMap{(int64_t)tn * PT::TN, g.N, false, 0};

  floatx4 acc[WMB][WNB];
#pragma unroll
  for (int i = 0; i < WMB; ++i)
#pragma unroll
    for (int j = 0; j < WNB; ++j) acc[i][j] = floatx4{0.f, 0.f, 0.f, 0.f};

  const Operand opa = make_operand(g.A, g.M, g.lda, EB);
  const Operand opb = make_operand(g.B, kSwiglu ? 2 * g.ffn : g.N, g.ldb, EB);
  const int nk = kend > kbeg ? (int)((kend - kbeg + kK - 1) / kK) : 0;
  // prologue: every wave loads 4 blocks of each of A_0, B_0, A_1
  issue_tile<true, EB>(opa, smem + slot_u4(0), ra, kbeg, kend, wave, lane);
  issue_tile<true, EB>(opb, smem + slot_u4(1), rb, kbeg, kend, wave, lane);
  if (nk > 1) issue_tile<true, EB>(opa, smem + slot_u4(2), ra, kbeg + kK, kend, wave, lane);
  phase_end<0>();

  const unsigned lane_part = (unsigned)((lane & 15) * 128 + (((lane >> 4) ^ (lane & 7)) * 16));
  const unsigned smem_addr = (unsigned)(uintptr_t)(__attribute__((address_space(3))) void*)smem;
  // kc_index(row0 + (lane & 15), lane >> 4) * 16: rows are 128 bytes
  const unsigned a_lane = smem_addr + lane_part + PT::row0(wave) * 128;
  const unsigned b_lane = smem_addr + lane_part + PT::col0(wave) * 128;
  auto slot_bytes = [](int x) { return (unsigned)(slot_u4(x) * 16); };
  Frags<WMB, WNB> f;
  // group A loads B tiles, group B loads A tiles
  QuarterLoads<kSwiglu, EB, kWaveChans> lb(opb, rb, q, lane);
  QuarterLoads<false, EB> la(opa, ra, q, lane);
  if (wm == 0) {
    // phase 2j: read k-tile j, load B of k-tile j+1; phase 2j+1: multiply k-tile j
    for (int j = 0; j < nk; ++j) {
      read_frags_kc(f, a_lane + slot_bytes(2 * j), b_lane + slot_bytes(2 * j + 1));
      if (j + 1 < nk) lb.issue(opb, smem + slot_u4(2 * j + 3), q, kbeg + (int64_t)(j + 1) * kK, kend);
      phase_end<kNoVm>();
      mma_tile(acc, f, OP{});
      phase_end<0>();  // B of k-tile j+1 has landed
    }
    if (nk > 0) phase_end<kNoVm>();  // idle in the last phase
  } else {
    // phase 2j+1: read k-tile j, load A of k-tile j+2; phase 2j+2: multiply k-tile j
    if (nk > 0) phase_end<kNoVm>();  // idle in phase 0
    for (int j = 0; j < nk; ++j) {
      read_frags_kc(f, a_lane + slot_bytes(2 * j), b_lane + slot_bytes(2 * j + 1));
      if (j + 2 < nk) {
        la.issue(opa, smem + slot_u4(2 * j + 4), q, kbeg + (int64_t)(j + 2) * kK, kend);
        phase_end<8>();  // A of k-tile j+1 has landed; k-tile j+2's may be in flight
      } else {
        phase_end<0>();
      }
      mma_tile(acc, f, OP{});
      phase_end<kNoVm>();
    }
  }
  if constexpr (OP::kFp8) {
    // dequantisation: the product of the operands' inverse scales, read after the main loop
    const float deq = g.scale_inv_a[0] * g.scale_inv_b[0];
#pragma unroll
    for (int i = 0; i < WMB; ++i)
#pragma unroll
      for (int j = 0; j < WNB; ++j) acc[i][j] *= deq;
  }
  const int64_t tile_m0 = (int64_t)tm * kBM, tile_n0 = (int64_t)tn * PT::TN;
  if constexpr (EPI == kEpiSgdT) {
    epilogue_sgd<kBM, PT::TN, WMB, WNB, kThreads, false, true>(g, acc, tile_m0, tile_n0, PT::row0(wave),
                                                               PT::col0(wave), lane, smem);
  } else if constexpr (EPI == kEpiSgd) {  // (the FP8 weight gradients)
    if (g.sgd.m_in)
      epilogue_sgd<kBM, PT::TN, WMB, WNB, kThreads, true, false>(g, acc, tile_m0, tile_n0, PT::row0(wave),
                                                                 PT::col0(wave), lane, smem);
    else
      epilogue_sgd<kBM, PT::TN, WMB, WNB, kThreads, false, false>(g, acc, tile_m0, tile_n0, PT::row0(wave),
                                                                  PT::col0(wave), lane, smem);
  } else if constexpr (EPI == kEpiSwigluBwdT || EPI == kEpiGeluBwdT) {
    // the activation backward, then d_pre transposed (gate rows, then up rows) through LDS
    constexpr int kBase = EPI == kEpiSwigluBwdT ? kEpiSwigluBwd : kEpiGeluBwd;
    constexpr int NL = EPI == kEpiSwigluBwdT ? 2 : 1;
    uint2 stash[WMB][WNB][2];
    epilogue_act_bwd<kBase, WMB, WNB, true>(g, acc, tile_m0 + PT::row0(wave), tile_n0 + PT::col0(wave), lane, stash);
    constexpr int kPitch = kBM + 8;
    bf16_t* const lds = reinterpret_cast<bf16_t*>(smem);
    const int frow = lane & 15, col4 = 4 * (lane >> 4);
#pragma unroll
    for (int l = 0; l < NL; ++l) {
      __syncthreads();  // the LDS is free: the main loop (l = 0) or the previous half's stores are done
#pragma unroll
      for (int i = 0; i < WMB; ++i)
#pragma unroll
        for (int j = 0; j < WNB; ++j)
          stage_t4<kPitch>(lds, PT::row0(wave) + i * 16 + frow, PT::col0(wave) + j * 16 + col4, stash[i][j][l],
                           lane & 1);
      __syncthreads();
      store_t_tile<kBM, PT::TN, kThreads>(lds, static_cast<bf16_t*>(g.pre_t) + (int64_t)l * g.ffn * g.ld_t, g.ld_t,
                                          tile_m0, tile_n0, g.M, g.N);
    }
  } else {
    epilogue<EPI, WMB, WNB>(g, acc, tile_m0 + PT::row0(wave), tile_n0 + PT::col0(wave),
                            (int64_t)tn * kTileChans + (PT::col0(wave) / (2 * kWaveChans)) * kWaveChans, ks, lane);
  }
}

template <bool AK, bool BKC, int EPI, class SH>
__global__ __launch_bounds__(SH::NW * 64, 1) void gemm_bf16_kernel(GemmArgs g, int ntm, int ntn) {
  extern __shared__ uint4 smem[];  // 2 stages x (A tile + B tile) = 128 KiB
  static_assert(!(AK && BKC), "both operands K-contiguous: the ping-pong kernel");

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / SH::GN, wn = wave % SH::GN;
  static_assert(SH::NW / SH::GN * SH::WMB * 16 == SH::TM && SH::GN * SH::WNB * 16 == SH::TN, "waves cover the tile");

  int tm, tn, ks;
  tile_coords(blockIdx.x, ntm, ntn, g.ksplit, g.tile_group, tm, tn, ks);

  const bf16_t* __restrict__ A = static_cast<const bf16_t*>(g.A);
  const bf16_t* __restrict__ B = static_cast<const bf16_t*>(g.B);
  const int64_t K = g.K;
  // this workgroup's k range [kbeg, kend); the slice length is a multiple of kBK
  const int64_t kper = ((K + (int64_t)g.ksplit * kBK - 1) / ((int64_t)g.ksplit * kBK)) * kBK;
  const int64_t kbeg = (int64_t)ks * kper;
  const int64_t kend = min(K, kbeg + kper);
  static_assert(EPI != kEpiSwigluFwd, "the SwiGLU forward is a K-contiguous (ping-pong) GEMM");
  const RowMap ra{(int64_t)tm * SH::TM, g.M, false, 0};
  const RowMap rb{(int64_t)tn * SH::TN, g.N, false, 0};

  floatx4 acc[SH::WMB][SH::WNB];
#pragma unroll
  for (int i = 0; i < SH::WMB; ++i)
#pragma unroll
    for (int j = 0; j < SH::WNB; ++j) acc[i][j] = floatx4{0.f, 0.f, 0.f, 0.f};

  const Operand opa = make_operand(A, AK ? g.M : K, g.lda);
  const Operand opb = make_operand(B, BKC ? g.N : K, g.ldb);
  const int nk = kend > kbeg ? (int)((kend - kbeg + kBK - 1) / kBK) : 0;
  issue_tile<AK, 2, SH::NW>(opa, smem, ra, kbeg, kend, wave, lane);
  issue_tile<BKC, 2, SH::NW>(opb, smem + kTileU4, rb, kbeg, kend, wave, lane);
  __syncthreads();  // waits for the loads (vmcnt) before the barrier

  for (int kt = 0; kt < nk; ++kt) {
    if (kt + 1 < nk) {
      // the other stage was last read in iteration kt - 1, before the barrier that ended it
      uint4* dst = smem + ((kt + 1) & 1) * kStageU4;
      const int64_t k0 = kbeg + (int64_t)(kt + 1) * kBK;
      issue_tile<AK, 2, SH::NW>(opa, dst, ra, k0, kend, wave, lane);
      issue_tile<BKC, 2, SH::NW>(opb, dst + kTileU4, rb, k0, kend, wave, lane);
    }
    const uint4* st = smem + (kt & 1) * kStageU4;
#pragma unroll
    for (int s = 0; s < kBK / 32; ++s) {
      uint4 af[SH::WMB], bfr[SH::WNB];
      read_half<AK, BKC>(af, bfr, st, s, wm, wn, lane);
      mma_half(acc, af, bfr);
    }
    __syncthreads();  // next stage landed; this stage free
  }

  if constexpr (EPI == kEpiSgd) {
    constexpr int NT = SH::NW * 64;
    const int wr0 = wm * SH::WMB * 16, wc0 = wn * SH::WNB * 16;
    if (g.sgd.m_in)
      epilogue_sgd<SH::TM, SH::TN, SH::WMB, SH::WNB, NT, true, false>(g, acc, (int64_t)tm * SH::TM,
                                                                      (int64_t)tn * SH::TN, wr0, wc0, lane, smem);
    else
      epilogue_sgd<SH::TM, SH::TN, SH::WMB, SH::WNB, NT, false, false>(g, acc, (int64_t)tm * SH::TM,
                                                                       (int64_t)tn * SH::TN, wr0, wc0, lane, smem);
  } else {
    epilogue<EPI, SH::WMB, SH::WNB>(g, acc, (int64_t)tm * SH::TM + wm * SH::WMB * 16,
                                    (int64_t)tn * SH::TN + wn * SH::WNB * 16, 0, ks, lane);
  }
}

// The two-stage schedule with the fragment reads one k-half ahead: each wave
// holds two fragment sets; the reads of k-half h + 1 are issued before the
// MFMAs of k-half h, so their LDS latency runs under those MFMAs instead of
// stalling both waves of a SIMD at the start of every k-tile.  Per k-tile:
//   reads  set1 <- (tile j, k 32-63)          MFMAs on set0 (tile j, k 0-31)
//   wait for this wave's reads and its loads of tile j+1; barrier (tile j+1
//   published, every wave done with tile j's stage)
//   loads of tile j+2 into tile j's stage
//   reads  set0 <- (tile j+1, k 0-31)         MFMAs on set1 (tile j, k 32-63)
// Every fragment read of a k-half is issued before the first MFMA that
// follows it (left to itself the compiler sinks the reads below most of the
// MFMAs, and they are then still in flight at the barrier).
__device__ __forceinline__ void pipe_order() { __builtin_amdgcn_sched_barrier(0); }

template <bool AK, bool BKC, int EPI, class SH>
__global__ __launch_bounds__(SH::NW * 64, 1) void gemm_bf16_pipe_kernel(GemmArgs g, int ntm, int ntn) {
  extern __shared__ uint4 smem[];  // 2 stages x (A tile + B tile) = 128 KiB
  static_assert(!(AK && BKC), "both operands K-contiguous: the ping-pong kernel");
  static_assert(EPI != kEpiSwigluFwd, "the SwiGLU forward is a K-contiguous (ping-pong) GEMM");
  static_assert(SH::NW / SH::GN * SH::WMB * 16 == SH::TM && SH::GN * SH::WNB * 16 == SH::TN, "waves cover the tile");

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / SH::GN, wn = wave % SH::GN;

  int tm, tn, ks;
  tile_coords(blockIdx.x, ntm, ntn, g.ksplit, g.tile_group, tm, tn, ks);
  const bf16_t* __restrict__ A = static_cast<const bf16_t*>(g.A);
  const bf16_t* __restrict__ B = static_cast<const bf16_t*>(g.B);
  const int64_t K = g.K;
  const int64_t kper = ((K + (int64_t)g.ksplit * kBK - 1) / ((int64_t)g.ksplit * kBK)) * kBK;
  const int64_t kbeg = (int64_t)ks * kper;
  const int64_t kend = min(K, kbeg + kper);
  const RowMap ra{(int64_t)tm * SH::TM, g.M, false, 0};
  const RowMap rb{(int64_t)tn * SH::TN, g.N, false, 0};

  floatx4 acc[SH::WMB][SH::WNB];
#pragma unroll
  for (int i = 0; i < SH::WMB; ++i)
#pragma unroll
    for (int j = 0; j < SH::WNB; ++j) acc[i][j] = floatx4{0.f, 0.f, 0.f, 0.f};

  const Operand opa = make_operand(A, AK ? g.M : K, g.lda);
  const Operand opb = make_operand(B, BKC ? g.N : K, g.ldb);
  const int nk = kend > kbeg ? (int)((kend - kbeg + kBK - 1) / kBK) : 0;
  issue_tile<AK, 2, SH::NW>(opa, smem, ra, kbeg, kend, wave, lane);
  issue_tile<BKC, 2, SH::NW>(opb, smem + kTileU4, rb, kbeg, kend, wave, lane);
  __syncthreads();  // tile 0 landed
  if (nk > 1) {
    issue_tile<AK, 2, SH::NW>(opa, smem + kStageU4, ra, kbeg + kBK, kend, wave, lane);
    issue_tile<BKC, 2, SH::NW>(opb, smem + kStageU4 + kTileU4, rb, kbeg + kBK, kend, wave, lane);
  }
  uint4 a0[SH::WMB], b0[SH::WNB], a1[SH::WMB], b1[SH::WNB];
  read_half<AK, BKC>(a0, b0, smem, 0, wm, wn, lane);
  for (int kt = 0; kt < nk; ++kt) {
    const uint4* st = smem + (kt & 1) * kStageU4;
    read_half<AK, BKC>(a1, b1, st, 1, wm, wn, lane);
    pipe_order();
    mma_half(acc, a0, b0);
    __syncthreads();  // this wave's reads and its loads of tile kt+1 done; every wave past tile kt's stage
    if (kt + 2 < nk) {
      uint4* dst = smem + (kt & 1) * kStageU4;
      const int64_t k0 = kbeg + (int64_t)(kt + 2) * kBK;
      issue_tile<AK, 2, SH::NW>(opa, dst, ra, k0, kend, wave, lane);
      issue_tile<BKC, 2, SH::NW>(opb, dst + kTileU4, rb, k0, kend, wave, lane);
    }
    // the next tile's first half (the stage after the last tile holds whatever it held; unused)
    read_half<AK, BKC>(a0, b0, smem + ((kt + 1) & 1) * kStageU4, 0, wm, wn, lane);
    pipe_order();
    mma_half(acc, a1, b1);
  }

  if constexpr (EPI == kEpiSgd) {
    constexpr int NT = SH::NW * 64;
    const int wr0 = wm * SH::WMB * 16, wc0 = wn * SH::WNB * 16;
    if (g.sgd.m_in)
      epilogue_sgd<SH::TM, SH::TN, SH::WMB, SH::WNB, NT, true, false>(g, acc, (int64_t)tm * SH::TM,
                                                                      (int64_t)tn * SH::TN, wr0, wc0, lane, smem);
    else
      epilogue_sgd<SH::TM, SH::TN, SH::WMB, SH::WNB, NT, false, false>(g, acc, (int64_t)tm * SH::TM,
                                                                       (int64_t)tn * SH::TN, wr0, wc0, lane, smem);
  } else {
    epilogue<EPI, SH::WMB, SH::WNB>(g, acc, (int64_t)tm * SH::TM + wm * SH::WMB * 16,
                                    (int64_t)tn * SH::TN + wn * SH::WNB * 16, 0, ks, lane);
  }
}

constexpr size_t kSmemBytes = 2 * kStageU4 * sizeof(uint4);
constexpr size_t kSmemBytesPingPong = kSlots * kTileU4 * sizeof(uint4);

// Compute units of the current device (queried once).
inline int device_cus() {
  static int cus = 0;
  if (cus == 0) {
    int dev = 0, n = 0;
    if (hipGetDevice(&dev) == hipSuccess && hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) ==
                                                 hipSuccess && n > 0)
      cus = n;
    else
      cus = 256;
  }
  return cus;
}

template <class SH>
inline int64_t tile_cost(const GemmArgs& g, int ksplit, int cus) {
  const int64_t tiles = ((g.M + SH::TM - 1) / SH::TM) * ((g.N + SH::TN - 1) / SH::TN) * ksplit;
  return ((tiles + cus - 1) / cus) * SH::TM * SH::TN;  // rounds of one workgroup per CU x work per tile
}

// Which two-stage main loop a tile shape runs: the pipelined one where it was
// measured faster -- the 224 x 256 tile (the gate/up weight gradient: 240 ->
// 224 us) and the NN 256 x 256 tile (the input gradient: 237 -> 214 us) --
// and the plain one for the 256 x 224 and the TN 256 x 256
// tiles, where reading a whole k-half ahead measured slower.
template <bool AK, bool BKC, class SH>
constexpr bool pipelined_loop() {
  if constexpr (SH::NW != 8) return false;
  else if constexpr (SH::TM == 224 && SH::TN == 256) return true;
  else return SH::TM == 256 && SH::TN == 256 && AK && !BKC;
}

template <bool AK, bool BKC, int EPI, class SH>
hipError_t launch_two_stage(const GemmArgs& ga, hipStream_t s) {
  const int ntm = (int)((ga.M + SH::TM - 1) / SH::TM), ntn = (int)((ga.N + SH::TN - 1) / SH::TN);
  void (*kernel)(GemmArgs, int, int);
  if constexpr (pipelined_loop<AK, BKC, SH>()) kernel = gemm_bf16_pipe_kernel<AK, BKC, EPI, SH>;
  else kernel = gemm_bf16_kernel<AK, BKC, EPI, SH>;
  // the SGD epilogue stages the transposed tile in LDS: [TN][TM + 8] bf16 (132 KiB for 256 x 256)
  constexpr size_t stage = t_stage_bytes<SH::TM, SH::TN>();
  constexpr size_t smem = EPI == kEpiSgd && stage > kSmemBytes ? stage : kSmemBytes;
  static_assert(smem <= 160 * 1024, "LDS of one CU");
  static bool configured = false;  // raise the dynamic LDS limit once per instantiation
  if (!configured) {
    const hipError_t e =
        hipFuncSetAttribute(reinterpret_cast<const void*>(kernel), hipFuncAttributeMaxDynamicSharedMemorySize,
                            (int)smem);
    if (e != hipSuccess) return e;
    configured = true;
  }
  hipLaunchKernelGGL(kernel, dim3(ntm * ntn * ga.ksplit), dim3(SH::NW * 64), smem, s, ga, ntm, ntn);
  return hipGetLastError();
}

template <int EPI, class OP, class PT = PpTile256>
hipError_t launch_pingpong(const GemmArgs& ga, int ntm, int ntn, hipStream_t s) {
  auto kernel = gemm_nt_pingpong_kernel<EPI, OP, PT>;
  static bool configured = false;  // raise the dynamic LDS limit once per instantiation
  if (!configured) {
    const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kernel),
                                             hipFuncAttributeMaxDynamicSharedMemorySize, (int)kSmemBytesPingPong);
    if (e != hipSuccess) return e;
    configured = true;
  }
  hipLaunchKernelGGL(kernel, dim3(ntm * ntn * ga.ksplit), dim3(kThreads), kSmemBytesPingPong, s, ga, ntm, ntn);
  return hipGetLastError();
}

// The GEMM's workgroups alone (no k-split reduction).  OP: PpBf16, or
// PpFp8<FA, FB> (both operands K-contiguous).
template <bool AK, bool BKC, int EPI, class OP = PpBf16>
hipError_t launch_tiles(const GemmArgs& ga, int ntm, int ntn, hipStream_t s) {
  static_assert(!OP::kFp8 || (AK && BKC), "FP8 operands are K-contiguous");
  KernelTimer timer(ga.tag ? ga.tag : "gemm", s);
  if constexpr (AK && BKC) {
    // 224-wide tiles when (rounds of one workgroup per CU) x (tile width) is smaller, as for the
    // two-stage kernel's tile choice (SwiGLU: 112 channels per tile instead of 128)
    const int64_t cus = device_cus();
    const int64_t ntn224 = EPI == kEpiSwigluFwd ? (ga.ffn + 111) / 112 : (ga.N + 223) / 224;
    const int64_t r256 = ((int64_t)ntm * ntn * ga.ksplit + cus - 1) / cus;
    const int64_t r224 = ((int64_t)ntm * ntn224 * ga.ksplit + cus - 1) / cus;
    if (r224 * 224 < r256 * 256) return launch_pingpong<EPI, OP, PpTile224>(ga, ntm, (int)ntn224, s);
    return launch_pingpong<EPI, OP>(ga, ntm, ntn, s);
  } else {
    // the tile shape with the least (rounds of one workgroup per CU) x (tile area); a function of the
    // shape and the CU count only, so results are reproducible on a given device
    const int cus = device_cus();
    const int64_t c0 = tile_cost<Tile256x256>(ga, ga.ksplit, cus);
    const int64_t cn = tile_cost<Tile256x224>(ga, ga.ksplit, cus);
    const int64_t cm = tile_cost<Tile224x256>(ga, ga.ksplit, cus);
    if (cn < c0 && cn <= cm) return launch_two_stage<AK, BKC, EPI, Tile256x224>(ga, s);
    if (cm < c0) return launch_two_stage<AK, BKC, EPI, Tile224x256>(ga, s);
    return launch_two_stage<AK, BKC, EPI, Tile256x256>(ga, s);
  }
}

template <bool AK, bool BKC, int EPI, class OP = PpBf16>
hipError_t launch_t(const GemmArgs& g, hipStream_t s) {
  const int ntm = (int)((g.M + kBM - 1) / kBM);
  const int ntn = (EPI == kEpiSwigluFwd) ? (int)((g.ffn + kSwigluChannels - 1) / kSwigluChannels)
                                         : (int)((g.N + kBN - 1) / kBN);
  if (ntm == 0 || ntn == 0) return hipSuccess;
  GemmArgs ga = g;
  if constexpr (EPI == kEpiStoreBf16 && !OP::kFp8) {
    if (ga.ws && ga.ksplit > 1 && ga.N % 4 == 0) {
      // every slice in fp32 in the workspace, then their sum as bf16
      GemmArgs gf = ga;
      gf.C = ga.ws;
      gf.ldc = ga.N;
      gf.ws = ga.ws + ga.M * ga.N;
      gf.accum = 0;
      const hipError_t e = launch_tiles<AK, BKC, kEpiStoreF32, OP>(gf, ntm, ntn, s);
      if (e != hipSuccess) return e;
      return launch_ksplit_reduce_bf16(ga.C, ga.ws, ga.ksplit, ga.M, ga.N, ga.ldc, s);
    }
  }
  if constexpr (EPI == kEpiSgd) {
    if (ga.ws && ga.ksplit > 1) {
      // every slice in fp32 in the workspace, then their sum in index order and the update
      GemmArgs gf = ga;
      gf.C = ga.ws;
      gf.ldc = ga.N;
      gf.ws = ga.ws + ga.M * ga.N;
      gf.accum = 0;
      const hipError_t e = launch_tiles<AK, BKC, kEpiStoreF32, OP>(gf, ntm, ntn, s);
      if (e != hipSuccess) return e;
      return launch_sgd_ksplit(ga.sgd, ga.ws, ga.ksplit, ga.M, ga.N, s);
    }
  }
  if ((EPI != kEpiStoreF32 && EPI != kEpiSgd) || !ga.ws) ga.ksplit = 1;
  if (EPI == kEpiSgd) ga.ksplit = 1;
  if (ga.ksplit < 1) ga.ksplit = 1;
  const hipError_t e = launch_tiles<AK, BKC, EPI, OP>(ga, ntm, ntn, s);
  if (e != hipSuccess || ga.ksplit == 1) return e;
  return launch_ksplit_reduce(static_cast<float*>(ga.C), ga.ws, ga.ksplit - 1, ga.M, ga.N, ga.ldc, s);
}

}  // namespace

hipError_t launch_gemm_bf16(bool ak, bool bk, Epi epi, const GemmArgs& g, hipStream_t s) {
  if (ak && bk) {
    switch (epi) {
      case kEpiStoreF32: return launch_t<true, true, kEpiStoreF32>(g, s);
      case kEpiSwigluFwd: return launch_t<true, true, kEpiSwigluFwd>(g, s);
      case kEpiGeluFwd: return launch_t<true, true, kEpiGeluFwd>(g, s);
      case kEpiResidual: return launch_t<true, true, kEpiResidual>(g, s);
      case kEpiStoreBf16: return launch_t<true, true, kEpiStoreBf16>(g, s);
      case kEpiSwigluBwd: return launch_t<true, true, kEpiSwigluBwd>(g, s);
      case kEpiGeluBwd: return launch_t<true, true, kEpiGeluBwd>(g, s);
      case kEpiSwigluBwdT: return launch_t<true, true, kEpiSwigluBwdT>(g, s);
      case kEpiGeluBwdT: return launch_t<true, true, kEpiGeluBwdT>(g, s);
      case kEpiSgdT: return launch_t<true, true, kEpiSgdT>(g, s);
      default: break;
    }
  } else if (ak && !bk) {
    switch (epi) {
      case kEpiStoreF32: return launch_t<true, false, kEpiStoreF32>(g, s);
      case kEpiStoreBf16: return launch_t<true, false, kEpiStoreBf16>(g, s);
      case kEpiSwigluBwd: return launch_t<true, false, kEpiSwigluBwd>(g, s);
      case kEpiGeluBwd: return launch_t<true, false, kEpiGeluBwd>(g, s);
      default: break;
    }
  } else if (!ak && !bk) {
    if (epi == kEpiStoreF32) return launch_t<false, false, kEpiStoreF32>(g, s);
    if (epi == kEpiSgd) return launch_t<false, false, kEpiSgd>(g, s);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_gemm_fp8(int fmt_a, int fmt_b, Epi epi, const GemmArgs& g, hipStream_t s) {
  if (fmt_a == kFp8E4M3 && fmt_b == kFp8E4M3) {
    using OP = PpFp8<kFp8E4M3, kFp8E4M3>;
    switch (epi) {
      case kEpiStoreF32: return launch_t<true, true, kEpiStoreF32, OP>(g, s);
      case kEpiSwigluFwd: return launch_t<true, true, kEpiSwigluFwd, OP>(g, s);
      case kEpiGeluFwd: return launch_t<true, true, kEpiGeluFwd, OP>(g, s);
      case kEpiResidual: return launch_t<true, true, kEpiResidual, OP>(g, s);
      default: break;
    }
  } else if (fmt_a == kFp8E5M2 && fmt_b == kFp8E4M3) {
    using OP = PpFp8<kFp8E5M2, kFp8E4M3>;
    switch (epi) {
      case kEpiStoreF32: return launch_t<true, true, kEpiStoreF32, OP>(g, s);
      case kEpiSgd: return launch_t<true, true, kEpiSgd, OP>(g, s);
      case kEpiSwigluBwd: return launch_t<true, true, kEpiSwigluBwd, OP>(g, s);
      case kEpiGeluBwd: return launch_t<true, true, kEpiGeluBwd, OP>(g, s);
      default: break;
    }
  }
  return hipErrorInvalidValue;
}

}  // namespace tpmlp
