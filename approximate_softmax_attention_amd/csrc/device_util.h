// Device-side helpers shared by the kernels: element loads/stores for the two
// input types, wave-level reductions and scans, and the counter-based draws.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace ha {

typedef uint16_t bf16_t;   // bfloat16 bit pattern in memory

__device__ __forceinline__ float bf16_to_f32(bf16_t x) {
  return __uint_as_float(uint32_t(x) << 16);
}

// Round to nearest even (inputs are finite here).
__device__ __forceinline__ bf16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return bf16_t(u >> 16);
}

template <typename T> __device__ __forceinline__ float to_f32(T x);
template <> __device__ __forceinline__ float to_f32<float>(float x) { return x; }
template <> __device__ __forceinline__ float to_f32<bf16_t>(bf16_t x) { return bf16_to_f32(x); }

template <typename T> __device__ __forceinline__ T from_f32(float x);
template <> __device__ __forceinline__ float from_f32<float>(float x) { return x; }
template <> __device__ __forceinline__ bf16_t from_f32<bf16_t>(float x) { return f32_to_bf16(x); }

// Load 8 consecutive elements as floats (p must be 16-byte aligned for bf16,
// 32-byte for float).
template <typename T> __device__ __forceinline__ void load8(const T* p, float* out);
template <> __device__ __forceinline__ void load8<bf16_t>(const bf16_t* p, float* out) {
  const uint4 v = *reinterpret_cast<const uint4*>(p);
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    out[2 * i] = __uint_as_float(w[i] << 16);
    out[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
  }
}
template <> __device__ __forceinline__ void load8<float>(const float* p, float* out) {
  const float4 a = reinterpret_cast<const float4*>(p)[0];
  const float4 b = reinterpret_cast<const float4*>(p)[1];
  out[0] = a.x; out[1] = a.y; out[2] = a.z; out[3] = a.w;
  out[4] = b.x; out[5] = b.y; out[6] = b.z; out[7] = b.w;
}

__device__ __forceinline__ int lane_id() { return threadIdx.x & 63; }

template <typename V>
__device__ __forceinline__ V wave_max(V x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    V y = __shfl_xor(x, o, 64);
    x = y > x ? y : x;
  }
  return x;
}

template <typename V>
__device__ __forceinline__ V wave_sum(V x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o, 64);
  return x;
}

// Inclusive prefix sum across the 64 lanes of a wave.
__device__ __forceinline__ uint64_t wave_incl_scan(uint64_t x) {
  const int lane = lane_id();
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    uint64_t y = __shfl_up(x, o, 64);
    if (lane >= o) x += y;
  }
  return x;
}

// SplitMix64 output for the state x (Steele, Lea and Flood, OOPSLA 2014) and
// the counter-based draw: mix64(mix64(seed) ^ (purpose<<60 | head<<44 |
// node<<24 | counter)).
__host__ __device__ inline uint64_t mix64(uint64_t x) {
  uint64_t z = x + 0x9E3779B97F4A7C15ull;
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

__host__ __device__ inline uint64_t draw(uint64_t key, uint64_t purpose, uint64_t head,
                                          uint64_t node, uint64_t counter) {
  return mix64(key ^ ((purpose << 60) | (head << 44) | (node << 24) | counter));
}

}  // namespace ha
