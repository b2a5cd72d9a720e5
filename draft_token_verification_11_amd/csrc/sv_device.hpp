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

// 2^x for a double x <= 0 (or moderately positive), to about 1e-7 relative:
// the integer part exactly through ldexp, the fraction in [0, 1) through the
// hardware single-precision exp2.  Needs no double-precision polynomial
// constants (which a long-lived kernel would otherwise keep in registers).
__device__ __forceinline__ double exp2_d(double x) {
  if (!(x > -1100.0)) return 0.0;
  const double n = __builtin_floor(x);
  return __builtin_ldexp((double)__builtin_amdgcn_exp2f((float)(x - n)), (int)n);
}

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

// Raw form of load8: the 8 elements as 16-byte words (1 for bf16, 2 for
// fp32), missing elements filled with -inf bits, unpacked later by unpack8.
template <typename T>
struct Raw8 {
  uint4 v[8 / Elem<T>::kPerVec];
};
template <typename T, bool VEC>
__device__ __forceinline__ void load8_raw(const T* row, int64_t e, int64_t V, Raw8<T>& out) {
  constexpr int P = Elem<T>::kPerVec;
  if (VEC && e + 8 <= V) {
#pragma unroll
    for (int h = 0; h < 8 / P; ++h) out.v[h] = load16(row + e + h * P);
  } else if constexpr (sizeof(T) == 2) {
    uint32_t w[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t lo = (e + 2 * i < V) ? (uint32_t)row[e + 2 * i] : 0xFF80u;
      const uint32_t hi = (e + 2 * i + 1 < V) ? (uint32_t)row[e + 2 * i + 1] : 0xFF80u;
      w[i] = lo | (hi << 16);
    }
    out.v[0] = make_uint4(w[0], w[1], w[2], w[3]);
  } else {
    uint32_t w[8];
#pragma unroll
    for (int i = 0; i < 8; ++i)
      w[i] = (e + i < V) ? __float_as_uint(((const float*)row)[e + i]) : 0xFF800000u;
    out.v[0] = make_uint4(w[0], w[1], w[2], w[3]);
    out.v[1] = make_uint4(w[4], w[5], w[6], w[7]);
  }
}
template <typename T>
__device__ __forceinline__ void unpack8(const Raw8<T>& r, float* out) {
  constexpr int P = Elem<T>::kPerVec;
#pragma unroll
  for (int h = 0; h < 8 / P; ++h) Elem<T>::unpack(r.v[h], out + h * P);
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

// 16-bit order keys of bf16 patterns: negative patterns h map to 0xFFFF - h,
// non-negative ones to 0x8000 + h, so key order is value order (-0 at key
// 0x7FFF sits next to +0 at 0x8000; callers fold the two).  -inf is key
// 0x007F, +inf 0xFF80; keys below 0x007F or from 0xFF80 up are NaN/+inf.
__device__ __forceinline__ uint32_t raw_of_key16(uint32_t k) {
  return k >= 0x8000u ? k - 0x8000u : 0xFFFFu - k;
}
__device__ __forceinline__ float value_of_key16(uint32_t k) {
  return __uint_as_float(raw_of_key16(k) << 16);
}
constexpr uint32_t kKey16NegInf = 0x007Fu;
constexpr uint32_t kKey16NegZero = 0x7FFFu;
constexpr uint32_t kKey16PosZero = 0x8000u;

// ---------------------------------------------------------------------------
// Wave-level scans and reductions (wave64) built from DPP row shifts inside
// each 16-lane row and v_readlane fix-ups across the four rows: no LDS
// round-trips, so serial chains of them stay cheap.
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t x, uint32_t fill) {
  // lanes whose source lies outside their row receive `fill`
  return (uint32_t)__builtin_amdgcn_update_dpp((int)fill, (int)x, CTRL, 0xF, 0xF, false);
}
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float x, float fill) {
  return __uint_as_float(dpp_u32<CTRL>(__float_as_uint(x), __float_as_uint(fill)));
}
template <int CTRL>
__device__ __forceinline__ double dpp_f64(double x, double fill) {
  const uint64_t b = (uint64_t)__double_as_longlong(x), f = (uint64_t)__double_as_longlong(fill);
  const uint32_t lo = dpp_u32<CTRL>((uint32_t)b, (uint32_t)f);
  const uint32_t hi = dpp_u32<CTRL>((uint32_t)(b >> 32), (uint32_t)(f >> 32));
  return __longlong_as_double((long long)(((uint64_t)hi << 32) | lo));
}
template <int CTRL>
struct Dpp {
  __device__ static __forceinline__ uint32_t mov(uint32_t x, uint32_t f) { return dpp_u32<CTRL>(x, f); }
  __device__ static __forceinline__ float mov(float x, float f) { return dpp_f32<CTRL>(x, f); }
  __device__ static __forceinline__ double mov(double x, double f) { return dpp_f64<CTRL>(x, f); }
};

// Uniform-lane broadcast (the lane index must be wave-uniform).
__device__ __forceinline__ uint32_t bcast(uint32_t x, int l) {
  return (uint32_t)__builtin_amdgcn_readlane((int)x, l);
}
__device__ __forceinline__ float bcast(float x, int l) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), l));
}
__device__ __forceinline__ double bcast(double x, int l) {
  const uint64_t b = (uint64_t)__double_as_longlong(x);
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)b, l);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(b >> 32), l);
  return __longlong_as_double((long long)(((uint64_t)hi << 32) | lo));
}

struct OpAdd {
  template <typename F>
  __device__ __forceinline__ F operator()(F a, F b) const { return a + b; }
};
struct OpMax {
  __device__ __forceinline__ float operator()(float a, float b) const { return fmaxf(a, b); }
  __device__ __forceinline__ uint32_t operator()(uint32_t a, uint32_t b) const { return max(a, b); }
};
struct OpMin {
  __device__ __forceinline__ uint32_t operator()(uint32_t a, uint32_t b) const { return min(a, b); }
};
struct OpOr {
  __device__ __forceinline__ uint32_t operator()(uint32_t a, uint32_t b) const { return a | b; }
};

// threadIdx.x passed through an empty asm statement: what a helper derives
// from it is recomputed where it is used instead of being hoisted out of a
// caller's loop and held in a register for the whole kernel.
__device__ __forceinline__ int opaque_tid() {
  int t = threadIdx.x;
  asm volatile("" : "+v"(t));
  return t;
}

// Inclusive prefix scan: lane i gets op(x_0, ..., x_i).
template <typename F, typename Op>
__device__ __forceinline__ F wave_prefix(F x, F id, Op op) {
  x = op(x, Dpp<0x111>::mov(x, id));  // row_shr:1
  x = op(x, Dpp<0x112>::mov(x, id));  // row_shr:2
  x = op(x, Dpp<0x114>::mov(x, id));  // row_shr:4
  x = op(x, Dpp<0x118>::mov(x, id));  // row_shr:8
  const F t0 = bcast(x, 15), t1 = bcast(x, 31), t2 = bcast(x, 47);
  const int row = (opaque_tid() & (kWave - 1)) >> 4;
  const F t01 = op(t0, t1);
  const F t012 = op(t01, t2);
  const F add = row == 0 ? id : (row == 1 ? t0 : (row == 2 ? t01 : t012));
  return row == 0 ? x : op(add, x);
}
// Inclusive suffix scan: lane i gets op(x_i, ..., x_63).
template <typename F, typename Op>
__device__ __forceinline__ F wave_suffix(F x, F id, Op op) {
  x = op(x, Dpp<0x101>::mov(x, id));  // row_shl:1
  x = op(x, Dpp<0x102>::mov(x, id));  // row_shl:2
  x = op(x, Dpp<0x104>::mov(x, id));  // row_shl:4
  x = op(x, Dpp<0x108>::mov(x, id));  // row_shl:8
  const F t1 = bcast(x, 16), t2 = bcast(x, 32), t3 = bcast(x, 48);
  const int row = (opaque_tid() & (kWave - 1)) >> 4;
  const F t23 = op(t2, t3);
  const F t123 = op(t1, t23);
  const F add = row == 3 ? id : (row == 2 ? t3 : (row == 1 ? t23 : t123));
  return row == 3 ? x : op(x, add);
}

template <typename F>
__device__ __forceinline__ F wave_incl_scan(F x) { return wave_prefix(x, F(0), OpAdd()); }
template <typename F>
__device__ __forceinline__ F wave_incl_suffix(F x) { return wave_suffix(x, F(0), OpAdd()); }
template <typename F>
__device__ __forceinline__ F wave_sum(F x) { return bcast(wave_prefix(x, F(0), OpAdd()), kWave - 1); }
__device__ __forceinline__ float wave_max(float x) {
  return bcast(wave_prefix(x, -__builtin_inff(), OpMax()), kWave - 1);
}
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t x) {
  return bcast(wave_prefix(x, 0u, OpMax()), kWave - 1);
}
__device__ __forceinline__ uint32_t wave_min_u32(uint32_t x) {
  return bcast(wave_prefix(x, 0xFFFFFFFFu, OpMin()), kWave - 1);
}
__device__ __forceinline__ uint32_t wave_or(uint32_t x) {
  return bcast(wave_prefix(x, 0u, OpOr()), kWave - 1);
}

// ---------------------------------------------------------------------------
// Workgroup barrier that orders LDS only: unlike __syncthreads() it does not
// wait for outstanding global loads, so a prefetch issued before it stays in
// flight across it.
__device__ __forceinline__ void block_sync_lds() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// ---------------------------------------------------------------------------
// Block-level reductions through a small LDS array of one slot per wave.
// Every thread of the block must call them; all threads get the result.
template <int NT, typename F>
__device__ __forceinline__ F block_sum(F x, F* slots) {
  constexpr int NW = NT / kWave;
  x = wave_sum(x);
  block_sync_lds();
  if (const int t = opaque_tid(); (t & (kWave - 1)) == 0) slots[t / kWave] = x;
  block_sync_lds();
  F r = slots[0];
#pragma unroll
  for (int w = 1; w < NW; ++w) r += slots[w];
  return r;
}
template <int NT>
__device__ __forceinline__ float block_max(float x, float* slots) {
  constexpr int NW = NT / kWave;
  x = wave_max(x);
  block_sync_lds();
  if (const int t = opaque_tid(); (t & (kWave - 1)) == 0) slots[t / kWave] = x;
  block_sync_lds();
  float r = slots[0];
#pragma unroll
  for (int w = 1; w < NW; ++w) r = fmaxf(r, slots[w]);
  return r;
}
template <int NT>
__device__ __forceinline__ uint32_t block_max_u32(uint32_t x, uint32_t* slots) {
  constexpr int NW = NT / kWave;
  x = wave_max_u32(x);
  block_sync_lds();
  if (const int t = opaque_tid(); (t & (kWave - 1)) == 0) slots[t / kWave] = x;
  block_sync_lds();
  uint32_t r = slots[0];
#pragma unroll
  for (int w = 1; w < NW; ++w) r = max(r, slots[w]);
  return r;
}
template <int NT>
__device__ __forceinline__ uint32_t block_min_u32(uint32_t x, uint32_t* slots) {
  constexpr int NW = NT / kWave;
  x = wave_min_u32(x);
  block_sync_lds();
  if (const int t = opaque_tid(); (t & (kWave - 1)) == 0) slots[t / kWave] = x;
  block_sync_lds();
  uint32_t r = slots[0];
#pragma unroll
  for (int w = 1; w < NW; ++w) r = min(r, slots[w]);
  return r;
}
template <int NT>
__device__ __forceinline__ uint32_t block_or(uint32_t x, uint32_t* slots) {
  constexpr int NW = NT / kWave;
  x = wave_or(x);
  block_sync_lds();
  if (const int t = opaque_tid(); (t & (kWave - 1)) == 0) slots[t / kWave] = x;
  block_sync_lds();
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
  const int t = opaque_tid();
  const int w = t / kWave;
  F s = wave_incl_suffix(x);
  block_sync_lds();
  if ((t & (kWave - 1)) == 0) slots[w] = s;  // wave total
  block_sync_lds();
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
