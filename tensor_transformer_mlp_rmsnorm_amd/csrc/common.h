// Device-side helpers shared by the kernels of libtpmlp (gfx950 / CDNA4).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tpmlp {

typedef uint16_t bf16_t;  // storage of a bfloat16 value
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

constexpr int kWave = 64;  // CDNA wavefront width

// ---------------------------------------------------------------- conversions

__device__ __forceinline__ float bf16_to_f32(bf16_t h) { return __uint_as_float((uint32_t)h << 16); }

// Round to nearest even (the hardware v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ bf16_t f32_to_bf16(float f) {
  __bf16 b = (__bf16)f;
  return __builtin_bit_cast(bf16_t, b);
}

// Element traits: storage type T in {float, bf16_t}.
template <typename T>
struct Elem;

template <>
struct Elem<float> {
  static constexpr int kPerChunk = 4;  // elements per 16-byte chunk
  __device__ __forceinline__ static float to_f32(float v) { return v; }
  __device__ __forceinline__ static float from_f32(float v) { return v; }
};

template <>
struct Elem<bf16_t> {
  static constexpr int kPerChunk = 8;
  __device__ __forceinline__ static float to_f32(bf16_t v) { return bf16_to_f32(v); }
  __device__ __forceinline__ static bf16_t from_f32(float v) { return f32_to_bf16(v); }
};

// The value a stored element of type T holds (round to T and back).
template <typename T>
__device__ __forceinline__ floatx4 stored(floatx4 v) {
  if constexpr (sizeof(T) == 2) {
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] = bf16_to_f32(f32_to_bf16(v[i]));
  }
  return v;
}

// Load / store 4 consecutive elements as fp32.
template <typename T>
__device__ __forceinline__ floatx4 load4(const T* p);

template <>
__device__ __forceinline__ floatx4 load4<float>(const float* p) {
  return *reinterpret_cast<const floatx4*>(p);
}

template <>
__device__ __forceinline__ floatx4 load4<bf16_t>(const bf16_t* p) {
  uint2 u = *reinterpret_cast<const uint2*>(p);
  floatx4 r;
  r[0] = __uint_as_float(u.x << 16);
  r[1] = __uint_as_float(u.x & 0xffff0000u);
  r[2] = __uint_as_float(u.y << 16);
  r[3] = __uint_as_float(u.y & 0xffff0000u);
  return r;
}

template <typename T>
__device__ __forceinline__ void store4(T* p, floatx4 v);

template <>
__device__ __forceinline__ void store4<float>(float* p, floatx4 v) {
  *reinterpret_cast<floatx4*>(p) = v;
}

template <>
__device__ __forceinline__ void store4<bf16_t>(bf16_t* p, floatx4 v) {
  uint2 u;
  u.x = (uint32_t)f32_to_bf16(v[0]) | ((uint32_t)f32_to_bf16(v[1]) << 16);
  u.y = (uint32_t)f32_to_bf16(v[2]) | ((uint32_t)f32_to_bf16(v[3]) << 16);
  *reinterpret_cast<uint2*>(p) = u;
}

// A 16-byte chunk as fp32 values (4 for fp32, 8 for bf16) and back.
template <typename T>
struct Chunk {
  static constexpr int N = Elem<T>::kPerChunk;
  __device__ __forceinline__ static void unpack(const uint4& u, float (&f)[N]);
  __device__ __forceinline__ static uint4 pack(const float (&f)[N]);
};

template <>
__device__ __forceinline__ void Chunk<float>::unpack(const uint4& u, float (&f)[4]) {
  f[0] = __uint_as_float(u.x);
  f[1] = __uint_as_float(u.y);
  f[2] = __uint_as_float(u.z);
  f[3] = __uint_as_float(u.w);
}

template <>
__device__ __forceinline__ uint4 Chunk<float>::pack(const float (&f)[4]) {
  return make_uint4(__float_as_uint(f[0]), __float_as_uint(f[1]), __float_as_uint(f[2]), __float_as_uint(f[3]));
}

template <>
__device__ __forceinline__ void Chunk<bf16_t>::unpack(const uint4& u, float (&f)[8]) {
  const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f[2 * i] = __uint_as_float(w[i] << 16);
    f[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
  }
}

template <>
__device__ __forceinline__ uint4 Chunk<bf16_t>::pack(const float (&f)[8]) {
  uint32_t w[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) w[i] = (uint32_t)f32_to_bf16(f[2 * i]) | ((uint32_t)f32_to_bf16(f[2 * i + 1]) << 16);
  return make_uint4(w[0], w[1], w[2], w[3]);
}

// ------------------------------------------------------------------- SGD

// One SGD update, p - lr g, as a single fused multiply-add (every kernel that
// applies the update goes through these, so all give the same bits).
__device__ __forceinline__ float sgd_value(float p, float g, float lr) { return __builtin_fmaf(-lr, g, p); }
__device__ __forceinline__ floatx4 sgd_value4(floatx4 p, floatx4 g, float lr) {
  floatx4 r;
#pragma unroll
  for (int i = 0; i < 4; ++i) r[i] = sgd_value(p[i], g[i], lr);
  return r;
}

// ------------------------------------------------------------ wave reductions

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, kWave);
  return v;
}

// ------------------------------------------------------------- activations

// The reciprocal by v_rcp_f32 (about 1 ulp) instead of an IEEE division, which
// takes nine instructions; the results are rounded to bf16 or compared at 1e-5.
__device__ __forceinline__ float sigmoid_f(float v) { return __builtin_amdgcn_rcpf(1.0f + __expf(-v)); }

__device__ __forceinline__ float gelu_f(float v) { return 0.5f * v * (1.0f + erff(v * 0.70710678118654752f)); }

__device__ __forceinline__ float gelu_grad_f(float v) {
  const float cdf = 0.5f * (1.0f + erff(v * 0.70710678118654752f));
  const float pdf = 0.39894228040143268f * __expf(-0.5f * v * v);
  return cdf + v * pdf;
}

}  // namespace tpmlp
