// sv_device.hpp -- device building blocks for the verify kernels (gfx950,
// wave64): element loads, order-preserving keys, wave and block reductions.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sv {

constexpr int kWave = 64;
constexpr float kLog2e = 1.4426950408889634f;

// ---------------------------------------------------------------------------
// Element types.  fp32 logits are `float`; bf16 logits are raw 16-bit
// patterns (`uint16_t`), widened exactly to fp32 by a 16-bit shift.
template <typename T>
struct Elem;
template <>
struct Elem<float> {
  static constexpr int kPerVec = 4;  // elements per 16-byte load
  __device__ static __forceinline__ float load1(const float* p) { return *p; }
  __device__ static __forceinline__ void unpack(const uint4& v, float* out) {
    out[0] = __uint_as_float(v.x);
    out[1] = __uint_as_float(v.y);
    out[2] = __uint_as_float(v.z);
    out[3] = __uint_as_float(v.w);
  }
};
template <>
struct Elem<uint16_t> {
  static constexpr int kPerVec = 8;
  __device__ static __forceinline__ float load1(const uint16_t* p) {
    return __uint_as_float(((uint32_t)*p) << 16);
  }
  __device__ static __forceinline__ void unpack(const uint4& v, float* out) {
    out[0] = __uint_as_float(v.x << 16);
    out[1] = __uint_as_float(v.x & 0xFFFF0000u);
    out[2] = __uint_as_float(v.y << 16);
    out[3] = __uint_as_float(v.y & 0xFFFF0000u);
    out[4] = __uint_as_float(v.z << 16);
    out[5] = __uint_as_float(v.z & 0xFFFF0000u);
    out[6] = __uint_as_float(v.w << 16);
    out[7] = __uint_as_float(v.w & 0xFFFF0000u);
  }
};

__device__ __forceinline__ uint4 load16(const void* p) {
  return *reinterpret_cast<const uint4*>(p);
}

// Loads the n (<= 8) consecutive elements starting at element e of `row`
// into out[0..7] (missing ones become -inf, i.e. zero probability).  The
// vector path needs a 16-byte aligned row and e a multiple of 8.
template <typename T, bool VEC>
__device__ __forceinline__ void load8(const T* row, int64_t e, int64_t V, float* out) {
  constexpr int P = Elem<T>::kPerVec;
  if (VEC && e + 8 <= V) {
#pragma unroll
    for (int h = 0; h < 8 / P; ++h) Elem<T>::unpack(load16(row + e + h * P), out + h * P);
  } else {
#pragma unroll
    for (int i = 0; i < 8; ++i)
      out[i] = (e + i < V) ? Elem<T>::load1(row + e + i) : -__builtin_inff();
  }
}

// ---------------------------------------------------------------------------
// Order-preserving keys: key(a) < key(b) iff a < b for non-NaN floats, with
// -0 mapped to +0 so that equal values share one key.
__device__ __forceinline__ uint32_t key_of(float f) {
  uint32_t b = __float_as_uint(f);
  b = (b == 0x80000000u) ? 0u : b;
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}
__device__ __forceinline__ float value_of(uint32_t k) {
  uint32_t b = (k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k;
  return __uint_as_float(b);
}
constexpr uint32_t kKeyNegInf = 0x007FFFFFu;  // key_of(-inf)
constexpr uint32_t kKeyPosInf = 0xFF800000u;  // key_of(+inf)
// A logit is usable (finite or -inf) iff kKeyNegInf <= key < kKeyPosInf.
__device__ __forceinline__ bool bad_logit(float f) {
  return __builtin_isnan(f) || f == __builtin_inff();
}

// 16-bit keys of bf16 patterns (the upper half of key_of for the widened
// value, except that -0 keeps its own key 0x7FFF).
__device__ __forceinline__ uint32_t key16_of_bits(uint32_t h) {
  return (h & 0x8000u) ? (~h & 0xFFFFu) : (h | 0x8000u);
}
__device__ __forceinline__ float value_of_key16(uint32_t k) {
  uint32_t h = (k & 0x8000u) ? (k & 0x7FFFu) : (~k & 0xFFFFu);
  return __uint_as_float(h << 16);
}

// ---------------------------------------------------------------------------
// Wave-level reductions and scans (wave64).
template <typename F>
__device__ __forceinline__ F wave_sum(F x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o, kWave);
  return x;
}
__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x = fmaxf(x, __shfl_xor(x, o, kWave));
  return x;
}
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x = max(x, (uint32_t)__shfl_xor((int)x, o, kWave));
  return x;
}
__device__ __forceinline__ uint32_t wave_min_u32(uint32_t x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x = min(x, (uint32_t)__shfl_xor((int)x, o, kWave));
  return x;
}
__device__ __forceinline__ uint32_t wave_or(uint32_t x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x |= (uint32_t)__shfl_xor((int)x, o, kWave);
  return x;
}
// Inclusive prefix scan (lane i gets x_0 + ... + x_i).
template <typename F>
__device__ __forceinline__ F wave_incl_scan(F x) {
  const int lane = threadIdx.x & (kWave - 1);
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    F y = __shfl_up(x, o, kWave);
    if (lane >= o) x += y;
  }
  return x;
}
// Inclusive suffix scan (lane i gets x_i + ... + x_63).
template <typename F>
__device__ __forceinline__ F wave_incl_suffix(F x) {
  const int lane = threadIdx.x & (kWave - 1);
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    F y = __shfl_down(x, o, kWave);
    if (lane + o < kWave) x += y;
  }
  return x;
}

// ---------------------------------------------------------------------------
// Block-level reductions through a small LDS array of one slot per wave.
// Every thread of the block must call them; all threads get the result.
template <int NT, typename F>
__device__ __forceinline__ F block_sum(F x, F* slots) {
  constexpr int NW = NT / kWave;
  x = wave_sum(x);
  __syncthreads();
  if ((threadIdx.x & (kWave - 1)) == 0) slots[threadIdx.x / kWave] = x;
  __syncthreads();
  F r = slots[0];
#pragma unroll
  for (int w = 1; w < NW; ++w) r += slots[w];
  return r;
}
template <int NT>
__device__ __forceinline__ float block_max(float x, float* slots) {
  constexpr int NW = NT / kWave;
  x = wave_max(x);
  __syncthreads();
  if ((threadIdx.x & (kWave - 1)) == 0) slots[threadIdx.x / kWave] = x;
  __syncthreads();
  float r = slots[0];
#pragma unroll
  for (int w = 1; w < NW; ++w) r = fmaxf(r, slots[w]);
  return r;
}
template <int NT>
__device__ __forceinline__ uint32_t block_max_u32(uint32_t x, uint32_t* slots) {
  constexpr int NW = NT / kWave;
  x = wave_max_u32(x);
  __syncthreads();
  if ((threadIdx.x & (kWave - 1)) == 0) slots[threadIdx.x / kWave] = x;
  __syncthreads();
  uint32_t r = slots[0];
#pragma unroll
  for (int w = 1; w < NW; ++w) r = max(r, slots[w]);
  return r;
}
template <int NT>
__device__ __forceinline__ uint32_t block_min_u32(uint32_t x, uint32_t* slots) {
  constexpr int NW = NT / kWave;
  x = wave_min_u32(x);
  __syncthreads();
  if ((threadIdx.x & (kWave - 1)) == 0) slots[threadIdx.x / kWave] = x;
  __syncthreads();
  uint32_t r = slots[0];
#pragma unroll
  for (int w = 1; w < NW; ++w) r = min(r, slots[w]);
  return r;
}
template <int NT>
__device__ __forceinline__ uint32_t block_or(uint32_t x, uint32_t* slots) {
  constexpr int NW = NT / kWave;
  x = wave_or(x);
  __syncthreads();
  if ((threadIdx.x & (kWave - 1)) == 0) slots[threadIdx.x / kWave] = x;
  __syncthreads();
  uint32_t r = slots[0];
#pragma unroll
  for (int w = 1; w < NW; ++w) r |= slots[w];
  return r;
}

// Block-wide inclusive suffix scan over one value per thread, in thread order
// (thread t gets x_t + ... + x_{NT-1}); also returns the block total.
template <int NT, typename F>
__device__ __forceinline__ F block_incl_suffix(F x, F* slots, F* total) {
  constexpr int NW = NT / kWave;
  const int w = threadIdx.x / kWave;
  F s = wave_incl_suffix(x);
  __syncthreads();
  if ((threadIdx.x & (kWave - 1)) == 0) slots[w] = s;  // wave total
  __syncthreads();
  F above = F(0);
  F all = F(0);
#pragma unroll
  for (int v = NW - 1; v >= 0; --v) {
    if (v > w) above += slots[v];
  }
#pragma unroll
  for (int v = NW - 1; v >= 0; --v) all += slots[v];
  *total = all;
  return s + above;
}

}  // namespace sv
