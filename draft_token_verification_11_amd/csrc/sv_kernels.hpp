// sv_kernels.hpp -- HIP kernels (gfx950) of the speculative-decoding verify
// step: row statistics (max, normaliser, top-k/top-p threshold), greedy
// argmax, the per-sequence ratio test / first-rejection stop / residual
// inverse-CDF draw, and dense probabilities.
//
// The rule implemented is the one in the encyclopedia entry "Speculative
// decoding" (glopedia, 推测解码), section "Basic steps of proposal and
// verification" (提议与核验的基本步骤); see include/specverify.h for the
// readings taken where the entry is silent.
//
// Probability of token x in a row:  p(x) = [l_x >= thr] * 2^((l_x - m) a) / z
// with m the row's largest finite logit, a = log2(e) / T, thr the filter
// threshold (-inf without filters) and z the sum of 2^((l - m) a) over the
// kept set.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "specverify.h"
#include "sv_device.hpp"

namespace sv {

// ---------------------------------------------------------------------------
// Workspace records.
struct RowStat {  // 32 bytes
  float m;        // largest finite logit
  float thr;      // kept set is {l >= thr}
  double z;       // sum over the kept set of 2^((l - m) a)
  int32_t valid;  // 0: NaN/+inf present or no finite logit
  int32_t pad[3];
};
struct Partial {   // 16 bytes: one V-chunk of one row
  float m;         // chunk max (-inf if the chunk holds no finite logit)
  uint32_t flags;  // bit 0: NaN or +inf seen
  double s;        // sum of 2^((l - m) a) over the chunk
};
struct GPartial {  // 16 bytes: greedy partial of one V-chunk
  uint32_t key;    // order key of the chunk's largest finite logit (0 = none)
  int32_t idx;     // its lowest index
  uint32_t flags;  // bit 0: NaN or +inf seen
  uint32_t pad;
};
constexpr uint32_t kFlagBad = 1u;
constexpr int kDrawChunks = 8;  // chunk sums kept per wave by the residual draw

// Rows of a call.  Dense layout (nt == 0): a sequence holds `per_seq` flat
// rows, the first `k1` its target rows 0..k1-1 at (t_seq, t_pos), the rest
// its draft rows at (d_seq, d_pos); flat row r = b per_seq + w.
//
// Pooled layout (nt > 0): rows shared by several sequences (the branches of
// one request, the prefix nodes of a candidate tree) live once in a target
// pool of nt rows and a draft pool of nd rows, each at its row stride
// (t_pos, d_pos).  Target row j of sequence b is pool row tmap[b k1 + j]
// (b k1 + j without a map), draft row j pool row dmap[b k + j] (b k + j
// without a map).  The row passes number the target pool 0..nt-1 and the
// draft pool nt..nt+nd-1; a map entry outside its pool names no row (sidx
// -1) and makes that row ill-formed.
struct RowMap {
  const void* tgt;
  int64_t t_seq, t_pos;
  const void* drf;
  int64_t d_seq, d_pos;
  int32_t per_seq;
  int32_t k1;
  int32_t nt = 0, nd = 0;
  const int32_t* tmap = nullptr;
  const int32_t* dmap = nullptr;

  // flat row r of a row pass
  template <typename T>
  __device__ __forceinline__ const T* row(int64_t r) const {
    if (nt > 0) {
      if (r < nt) return reinterpret_cast<const T*>(tgt) + r * t_pos;
      return reinterpret_cast<const T*>(drf) + (r - nt) * d_pos;
    }
    const int64_t b = r / per_seq;
    const int64_t w = r - b * per_seq;
    if (w < k1) return reinterpret_cast<const T*>(tgt) + b * t_seq + w * t_pos;
    return reinterpret_cast<const T*>(drf) + b * d_seq + (w - k1) * d_pos;
  }
  // flat row (index of the row's statistics) of slot w of sequence b (w < k1:
  // target row w, else draft row w - k1); -1 for a map entry outside its pool
  __device__ __forceinline__ int64_t sidx(int64_t b, int w) const {
    if (nt == 0) return b * per_seq + w;
    if (w < k1) {
      const int64_t i = tmap ? (int64_t)tmap[b * k1 + w] : b * k1 + w;
      return (i >= 0 && i < nt) ? i : -1;
    }
    const int k = k1 - 1;
    const int64_t i = dmap ? (int64_t)dmap[b * k + (w - k1)] : b * k + (w - k1);
    return (i >= 0 && i < nd) ? nt + i : -1;
  }
  // the row of slot w of sequence b (flat row 0 when its map entry is bad:
  // readable, and never used for a decision)
  template <typename T>
  __device__ __forceinline__ const T* at(int64_t b, int w) const {
    const int64_t r = sidx(b, w);
    return row<T>(r < 0 ? 0 : r);
  }
};

// ---------------------------------------------------------------------------
// Unfiltered rows: per (row, chunk) max and sum of 2^((l - m_c) a).  Each of
// the 256 threads holds VPT groups of 8 consecutive elements in registers;
// group g of the chunk starts at element chunk_lo + 8 g (coalesced 16-byte
// loads: 1 load per group for bf16, 2 for fp32).
template <typename T, bool VEC, int VPT>
__global__ __launch_bounds__(256) void k_row_partials(RowMap map, int64_t V, int nchunks,
                                                      float a, Partial* __restrict__ part) {
  constexpr int NT = 256;
  __shared__ float fslot[NT / kWave];
  __shared__ double dslot[NT / kWave];
  __shared__ uint32_t uslot[NT / kWave];
  const int64_t bid = blockIdx.x;
  const int64_t r = bid / nchunks;
  const int c = (int)(bid - r * nchunks);
  const T* row = map.row<T>(r);
  const int64_t lo = (int64_t)c * (NT * VPT * 8);
  const int64_t hi = min(V, lo + (int64_t)NT * VPT * 8);

  float x[VPT][8];
#pragma unroll
  for (int v = 0; v < VPT; ++v) {
    const int64_t e = lo + ((int64_t)v * NT + threadIdx.x) * 8;
    if (e < hi) {
      load8<T, VEC>(row, e, hi, x[v]);
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) x[v][i] = -__builtin_inff();
    }
  }
  float m = -__builtin_inff();
  uint32_t bad = 0;
#pragma unroll
  for (int v = 0; v < VPT; ++v)
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      bad |= bad_logit(x[v][i]) ? 1u : 0u;
      m = fmaxf(m, x[v][i]);
    }
  m = block_max<NT>(m, fslot);
  bad = block_or<NT>(bad, uslot);
  double s = 0.0;
  if (!bad && m > -__builtin_inff()) {
#pragma unroll
    for (int v = 0; v < VPT; ++v) {
      float e[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) e[i] = __builtin_amdgcn_exp2f((x[v][i] - m) * a);
      s += (double)(((e[0] + e[1]) + (e[2] + e[3])) + ((e[4] + e[5]) + (e[6] + e[7])));
    }
  }
  s = block_sum<NT>(s, dslot);
  if (threadIdx.x == 0) {
    Partial p;
    p.m = m;
    p.flags = bad ? kFlagBad : 0u;
    p.s = s;
    part[bid] = p;
  }
}

// Merges the chunk partials of one row into a RowStat (unfiltered row).
__device__ __forceinline__ RowStat merge_partials(const Partial* p, int nchunks, float a) {
  RowStat st;
  float m = -__builtin_inff();
  uint32_t flags = 0;
  for (int c = 0; c < nchunks; ++c) {
    m = fmaxf(m, p[c].m);
    flags |= p[c].flags;
  }
  double z = 0.0;
  if (m > -__builtin_inff()) {
    for (int c = 0; c < nchunks; ++c)
      if (p[c].m > -__builtin_inff()) z += p[c].s * exp2_d(((double)p[c].m - (double)m) * (double)a);
  }
  st.m = m;
  st.thr = -__builtin_inff();
  st.z = z;
  st.valid = (!(flags & kFlagBad) && m > -__builtin_inff()) ? 1 : 0;
  st.pad[0] = st.pad[1] = st.pad[2] = 0;
  return st;
}

// The same merge by all 64 lanes of a wave (rows split into many chunks, e.g.
// a single sequence's rows spread over the chip); every lane gets the result.
__device__ __forceinline__ RowStat merge_partials_wave(const Partial* p, int nchunks, float a,
                                                       int lane) {
  float m = -__builtin_inff();
  uint32_t flags = 0;
  for (int c = lane; c < nchunks; c += kWave) {
    m = fmaxf(m, p[c].m);
    flags |= p[c].flags;
  }
  m = wave_max(m);
  flags = wave_or(flags);
  double z = 0.0;
  if (m > -__builtin_inff()) {
    for (int c = lane; c < nchunks; c += kWave)
      if (p[c].m > -__builtin_inff()) z += p[c].s * exp2_d(((double)p[c].m - (double)m) * (double)a);
  }
  z = wave_sum(z);
  RowStat st;
  st.m = m;
  st.thr = -__builtin_inff();
  st.z = z;
  st.valid = (!(flags & kFlagBad) && m > -__builtin_inff()) ? 1 : 0;
  st.pad[0] = st.pad[1] = st.pad[2] = 0;
  return st;
}

// ---------------------------------------------------------------------------
// Greedy: per (row, chunk) largest finite logit (as an order key) and its
// lowest index.
__device__ __forceinline__ uint64_t pack_best(uint32_t key, int32_t idx) {
  return ((uint64_t)key << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)idx);
}
__device__ __forceinline__ uint64_t wave_max_u64(uint64_t x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    uint32_t lo = (uint32_t)__shfl_xor((int)(uint32_t)x, o, kWave);
    uint32_t hi = (uint32_t)__shfl_xor((int)(uint32_t)(x >> 32), o, kWave);
    uint64_t y = ((uint64_t)hi << 32) | lo;
    x = y > x ? y : x;
  }
  return x;
}

template <typename T, bool VEC, int VPT>
__global__ __launch_bounds__(256) void k_greedy_partials(RowMap map, int64_t V, int nchunks,
                                                         GPartial* __restrict__ part) {
  constexpr int NT = 256;
  __shared__ uint64_t bslot[NT / kWave];
  __shared__ uint32_t uslot[NT / kWave];
  const int64_t bid = blockIdx.x;
  const int64_t r = bid / nchunks;
  const int c = (int)(bid - r * nchunks);
  const T* row = map.row<T>(r);
  const int64_t lo = (int64_t)c * (NT * VPT * 8);
  const int64_t hi = min(V, lo + (int64_t)NT * VPT * 8);
  uint64_t best = 0;
  uint32_t bad = 0;
#pragma unroll
  for (int v = 0; v < VPT; ++v) {
    const int64_t e = lo + ((int64_t)v * NT + threadIdx.x) * 8;
    if (e < hi) {
      float x[8];
      load8<T, VEC>(row, e, hi, x);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const bool b = bad_logit(x[i]);
        bad |= b ? 1u : 0u;
        const uint32_t k = key_of(x[i]);
        if (!b && k > kKeyNegInf && e + i < hi) {
          const uint64_t cand = pack_best(k, (int32_t)(e + i));
          best = cand > best ? cand : best;
        }
      }
    }
  }
  best = wave_max_u64(best);
  bad = wave_or(bad);
  const int w = threadIdx.x / kWave;
  if ((threadIdx.x & (kWave - 1)) == 0) {
    bslot[w] = best;
    uslot[w] = bad;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    uint64_t bb = bslot[0];
    uint32_t fl = uslot[0];
    for (int i = 1; i < NT / kWave; ++i) {
      bb = bslot[i] > bb ? bslot[i] : bb;
      fl |= uslot[i];
    }
    GPartial g;
    g.key = (uint32_t)(bb >> 32);
    g.idx = (int32_t)(0xFFFFFFFFu - (uint32_t)bb);
    g.flags = fl ? kFlagBad : 0u;
    g.pad = 0;
    part[bid] = g;
  }
}

// One wave per sequence: merge each target row's greedy partials, compare
// with the drafts, stop at the first mismatch, emit.  Dense partials are
// cleared here; pooled ones (shared by sequences) by a pass after the tail.
__global__ __launch_bounds__(64) void k_greedy_tail(RowMap map, int64_t V, int k, int nchunks,
                                                    const int32_t* __restrict__ tokens,
                                                    GPartial* __restrict__ part,
                                                    uint64_t* __restrict__ pbest,
                                                    uint32_t* __restrict__ pbad,
                                                    int32_t* __restrict__ accepted_len,
                                                    int32_t* __restrict__ out_tokens) {
  const int64_t b = blockIdx.x;
  const int lane = threadIdx.x;
  const int k1 = k + 1;
  const bool pooled = map.nt > 0;
  __shared__ int32_t best_idx[SPEC_MAX_K + 1];  // -1 for an invalid row
  if (pbest) {
    // one merged record per row (pack_best order; bad flags or-ed), cleared here
    for (int j = lane; j < k1; j += kWave) {
      const int64_t r = map.sidx(b, j);
      const uint64_t bb = pbest[r];
      const uint32_t fl = pbad[r];
      pbest[r] = 0ull;
      pbad[r] = 0u;
      const uint32_t key = (uint32_t)(bb >> 32);
      best_idx[j] = (fl == 0 && key != 0) ? (int32_t)(0xFFFFFFFFu - (uint32_t)bb) : -1;
    }
  } else if (nchunks > 16) {
    // many chunks per row (e.g. the fused LM head's vocabulary tiles): the
    // whole wave merges one row's records at a time
    for (int j = 0; j < k1; ++j) {
      const int64_t r = map.sidx(b, j);
      if (r < 0) {
        if (lane == 0) best_idx[j] = -1;
        continue;
      }
      GPartial* p = part + r * (int64_t)nchunks;
      uint64_t bb = 0;
      uint32_t fl = 0;
      for (int c = lane; c < nchunks; c += kWave) {
        const GPartial g = p[c];
        const uint64_t cand = pack_best(g.key, g.idx);
        if (g.key != 0 && cand > bb) bb = cand;
        fl |= g.flags;
        if (!pooled) {
          GPartial zero = {0u, 0, 0u, 0u};
          p[c] = zero;
        }
      }
      bb = wave_max_u64(bb);
      fl = wave_or(fl);
      const uint32_t key = (uint32_t)(bb >> 32);
      if (lane == 0) best_idx[j] = (fl == 0 && key != 0) ? (int32_t)(0xFFFFFFFFu - (uint32_t)bb) : -1;
    }
  } else {
    for (int j = lane; j < k1; j += kWave) {
      const int64_t r = map.sidx(b, j);
      if (r < 0) {
        best_idx[j] = -1;
        continue;
      }
      GPartial* p = part + r * (int64_t)nchunks;
      uint64_t bb = 0;
      uint32_t fl = 0;
      for (int c = 0; c < nchunks; ++c) {
        const uint64_t cand = pack_best(p[c].key, p[c].idx);
        if (p[c].key != 0 && cand > bb) bb = cand;
        fl |= p[c].flags;
      }
      if (!pooled) {
        for (int c = 0; c < nchunks; ++c) {
          GPartial zero = {0u, 0, 0u, 0u};
          p[c] = zero;
        }
      }
      const uint32_t key = (uint32_t)(bb >> 32);
      best_idx[j] = (fl == 0 && key != 0) ? (int32_t)(0xFFFFFFFFu - (uint32_t)bb) : -1;
    }
  }
  __syncthreads();
  // Positions in order up to the first mismatch; only what the walk consults
  // can make the sequence invalid.
  bool formed = false, match = false;
  if (lane < k) {
    const int32_t tok = tokens[b * k + lane];
    formed = best_idx[lane] >= 0 && tok >= 0 && (int64_t)tok < V;
    match = formed && tok == best_idx[lane];
  }
  const uint64_t stop = __ballot(lane < k && !match);
  const uint64_t ill = __ballot(lane < k && !formed);
  const int n = stop ? (__ffsll((unsigned long long)stop) - 1) : k;
  const bool valid = n < k ? !((ill >> n) & 1ull) : best_idx[k] >= 0;
  int32_t* out = out_tokens + b * k1;
  if (!valid) {
    for (int j = lane; j < k1; j += kWave) out[j] = -1;
    if (lane == 0) accepted_len[b] = -1;
    return;
  }
  for (int j = lane; j < k1; j += kWave) {
    int32_t v = -1;
    if (j < n) v = tokens[b * k + j];
    else if (j == n) v = best_idx[n];
    out[j] = v;
  }
  if (lane == 0) accepted_len[b] = n;
}

// ---------------------------------------------------------------------------
// Filtered rows, generic path: the top-k and top-p thresholds found by
// bisection over the 32-bit order keys, each probe a pass over the row
// (count of keys >= c for top-k, sum of 2^((l - m) a) over keys >= c for
// top-p).  Used for fp32 rows and as the fallback of the bf16 histogram.
template <typename T, bool VEC, int NT>
__device__ void filter_row_bisect(const T* row, int64_t V, float a, int top_k, float top_p,
                                  RowStat* out, double* dslot, uint32_t* uslot) {
  const int64_t ngroups = (V + 7) / 8;
  uint32_t bad = 0, mk = 0;
  for (int64_t g = threadIdx.x; g < ngroups; g += NT) {
    float x[8];
    load8<T, VEC>(row, g * 8, V, x);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const bool b = bad_logit(x[i]);
      bad |= b ? 1u : 0u;
      const uint32_t k = key_of(x[i]);
      if (!b && k > kKeyNegInf) mk = max(mk, k);
    }
  }
  bad = block_or<NT>(bad, uslot);
  mk = block_max_u32<NT>(mk, uslot);
  if (bad || mk == 0) {
    if (threadIdx.x == 0) {
      RowStat st = {__builtin_nanf(""), __builtin_nanf(""), 0.0, 0, {0, 0, 0}};
      *out = st;
    }
    return;
  }
  const float m = value_of(mk);
  auto count_ge = [&](uint32_t c) -> uint32_t {
    uint32_t n = 0;
    for (int64_t g = threadIdx.x; g < ngroups; g += NT) {
      float x[8];
      load8<T, VEC>(row, g * 8, V, x);
#pragma unroll
      for (int i = 0; i < 8; ++i) n += (g * 8 + i < V && key_of(x[i]) >= c) ? 1u : 0u;
    }
    return block_sum<NT>(n, uslot);
  };
  auto mass_ge = [&](uint32_t c) -> double {
    double s = 0.0;
    for (int64_t g = threadIdx.x; g < ngroups; g += NT) {
      float x[8];
      load8<T, VEC>(row, g * 8, V, x);
      float e[8];
#pragma unroll
      for (int i = 0; i < 8; ++i)
        e[i] = key_of(x[i]) >= c ? __builtin_amdgcn_exp2f((x[i] - m) * a) : 0.0f;
      s += (double)(((e[0] + e[1]) + (e[2] + e[3])) + ((e[4] + e[5]) + (e[6] + e[7])));
    }
    return block_sum<NT>(s, dslot);
  };
  const bool use_k = top_k > 0 && (int64_t)top_k < V;
  const bool use_p = top_p < 1.0f;
  uint32_t tk = 0;
  if (use_k) {
    uint32_t c = 0;
    for (int bit = 31; bit >= 0; --bit) {
      const uint32_t cand = c | (1u << bit);
      if (count_ge(cand) >= (uint32_t)top_k) c = cand;
    }
    tk = c;
  }
  const double zk = mass_ge(tk);
  uint32_t thr_key = tk;
  double z = zk;
  if (use_p) {
    const double target = (double)top_p * zk;
    uint32_t c = 0;
    for (int bit = 31; bit >= 0; --bit) {
      const uint32_t cand = c | (1u << bit);
      if (mass_ge(max(cand, tk)) >= target) c = cand;
    }
    thr_key = max(c, tk);
    z = mass_ge(thr_key);
  }
  if (threadIdx.x == 0) {
    RowStat st;
    st.m = m;
    st.thr = (use_k || use_p) ? value_of(thr_key) : -__builtin_inff();
    st.z = z;
    st.valid = 1;
    st.pad[0] = st.pad[1] = st.pad[2] = 0;
    *out = st;
  }
}

template <typename T, bool VEC>
__global__ __launch_bounds__(1024) void k_filter_bisect(RowMap map, int64_t V, float a, int top_k,
                                                        float top_p, RowStat* __restrict__ stats) {
  __shared__ double dslot[16];
  __shared__ uint32_t uslot[16];
  const int64_t r = blockIdx.x;
  filter_row_bisect<T, VEC, 1024>(map.row<T>(r), V, a, top_k, top_p, stats + r, dslot, uslot);
}

// ---------------------------------------------------------------------------
// Filtered bf16 rows: an exact 65536-bin count histogram of the 16-bit order
// keys in LDS (two 16-bit counters per 32-bit word).  Equal bf16 values have
// equal probabilities, so the counts give the row's sorted value distribution
// exactly: the max, the top-k threshold (by counts), the per-value masses
// count * 2^((v - m) a), the top-p cut (by masses) and the normaliser all come
// from the histogram after one streaming pass, with no per-element exp.
// Overflow (>= 65536 equal values) is detected by the count total and falls
// back to the bisection path.
struct HistScratch {
  uint16_t list[1024];   // non-empty 64-key groups, descending key order
  uint32_t lcnt[1024];   // count of list entry i
  float gmass[1024];     // mass of list entry i relative to the reference value
  uint32_t wcount[16], wtot[16], wbad[16];
  double dslot[16];
  uint32_t uslot[16];
  uint32_t tk, tk_entry;
  RowStat res;  // the row's statistics, as also written to the caller's record
};

__device__ __forceinline__ void hist_clear(uint32_t* hist) {
  uint4* h4 = reinterpret_cast<uint4*>(hist);
  for (int i = opaque_tid(); i < 8192; i += 1024) h4[i] = make_uint4(0u, 0u, 0u, 0u);
}

// The histogram counts raw bf16 patterns (code c: 16-bit half c & 1 of word
// c >> 1); the scan reads it in key order through raw_of_key16.
__device__ __forceinline__ void hist_add1(uint32_t* hist, uint32_t code) {
  atomicAdd(&hist[code >> 1], 1u + (code & 1u) * 0xFFFFu);
}

__device__ __forceinline__ void hist_add8(uint32_t* hist, uint4 v) {
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    atomicAdd(&hist[(w[i] & 0xFFFFu) >> 1], 1u + (w[i] & 1u) * 0xFFFFu);
    atomicAdd(&hist[w[i] >> 17], 1u + ((w[i] >> 16) & 1u) * 0xFFFFu);
  }
}

// Streams one bf16 row into the (cleared) histogram.
template <bool VEC>
__device__ __forceinline__ void hist_count_row(uint32_t* hist, const uint16_t* row, int64_t V) {
  constexpr int NT = 1024;
  const int64_t ngroups = (V + 7) / 8;
  int64_t g = threadIdx.x;
  if (VEC) {
    for (; (g + 3 * NT + 1) * 8 <= V; g += 4 * NT) {
      const uint4 v0 = load16(row + g * 8);
      const uint4 v1 = load16(row + (g + NT) * 8);
      const uint4 v2 = load16(row + (g + 2 * NT) * 8);
      const uint4 v3 = load16(row + (g + 3 * NT) * 8);
      hist_add8(hist, v0);
      hist_add8(hist, v1);
      hist_add8(hist, v2);
      hist_add8(hist, v3);
    }
  }
  for (; g < ngroups; g += NT) {
    const int64_t e = g * 8;
    if (VEC && e + 8 <= V) {
      hist_add8(hist, load16(row + e));
    } else {
      for (int i = 0; i < 8 && e + i < V; ++i) hist_add1(hist, row[e + i]);
    }
  }
}

// Mass of `key` (count c) relative to the max logit m.
__device__ __forceinline__ float key_mass(uint32_t key, uint32_t c, float m, float a) {
  return c ? (float)c * __builtin_amdgcn_exp2f((value_of_key16(key) - m) * a) : 0.0f;
}

// A list entry's mass, entry-major: an octet of lanes (eight consecutive
// lanes, sub = lane % 8) holds the 64 keys of one entry, eight each in
// ascending key order; x[i] are the masses of keys 8 sub + i.  Each lane sums
// its eight by a fixed tree, the octet's sums meet by quads and then by the
// octet (DPP inside the lanes' 16-lane row); lane 8 o + 4 returns the entry's
// mass.  The 16-bit histogram's scan and the exponent-window scans form their
// entries' masses by these same additions, so a row's statistics agree bit
// for bit between the two histograms.
__device__ __forceinline__ float octet_mass(const float (&x)[8]) {
  float s = ((x[0] + x[1]) + (x[2] + x[3])) + ((x[4] + x[5]) + (x[6] + x[7]));
  s += Dpp<0xB1>::mov(s, 0.0f);   // quad_perm 1,0,3,2: pairs
  s += Dpp<0x4E>::mov(s, 0.0f);   // quad_perm 2,3,0,1: quads
  s += Dpp<0x114>::mov(s, 0.0f);  // row_shr:4: lane 8o + 4 takes quad 8o..8o+3
  return s;
}

// Masses of eight keys of one sign whose bf16 codes are rb .. rb + 7 (so
// ascending magnitude) with counts c[j]: c 2^((v - m) a), the exponent
// clamped at 0 (every key with a count lies at or below the max m, and the
// empty keys above it stay finite); with top-k, keys whose value lies below
// vtk get 0.
__device__ __forceinline__ void x_masses8(float (&x)[8], const uint32_t (&c)[8], uint32_t rb,
                                          float m, float a, bool use_k, float vtk) {
  const uint32_t vb = rb << 16;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const float v = __uint_as_float(vb + ((uint32_t)j << 16));
    x[j] = (float)c[j] * __builtin_amdgcn_exp2f(fminf((v - m) * a, 0.0f));
  }
  if (use_k) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float v = __uint_as_float(vb + ((uint32_t)j << 16));
      x[j] = v >= vtk ? x[j] : 0.0f;
    }
  }
}

// Row statistics from a filled histogram (all 1024 threads).  Returns 0 on
// success (RowStat written to S.res and, if given, *out), 1 for an invalid
// row (written), 2 on counter overflow (nothing written: the caller takes the
// bisection path).  Leaves the histogram all zero when it returns 0 or 1;
// S.res can be read by every thread on return.
__device__ __forceinline__ int hist_row_stats(uint32_t* hist, HistScratch& S, int64_t V, float a, int top_k,
                              float top_p, RowStat* out) {
  constexpr int NT = 1024;
  // The thread index is made opaque here so that the addresses derived from
  // it are recomputed for each row instead of being kept live (in registers
  // the streaming loop needs) across a persistent kernel's row loop.
  int tid = threadIdx.x;
  asm volatile("" : "+v"(tid));
  const int lane = tid & (kWave - 1);
  const int wv = tid / kWave;
  uint16_t* c16 = reinterpret_cast<uint16_t*>(hist);
  const bool use_k = top_k > 0 && (int64_t)top_k < V;
  const bool use_p = top_p < 1.0f;

  // Counts of key group g = 1023 - tid (keys 64 g .. 64 g + 63; 8 rotated
  // 16-byte reads of its raw group), validity, total, and the compacted list
  // of non-empty groups in descending order.  -0 (key 0x7FFF, last of group
  // 511) is counted with +0 (key 0x8000, first of group 512).
  const int g = 1023 - tid;
  const uint32_t rg = g >= 512 ? (uint32_t)g - 512u : 1023u - (uint32_t)g;
  uint32_t cnt = 0;
  {
    const uint4* h4 = reinterpret_cast<const uint4*>(hist);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const uint4 w = h4[rg * 8 + ((j + rg) & 7)];
      cnt += (w.x & 0xFFFFu) + (w.x >> 16) + (w.y & 0xFFFFu) + (w.y >> 16) + (w.z & 0xFFFFu) +
             (w.z >> 16) + (w.w & 0xFFFFu) + (w.w >> 16);
    }
    const uint32_t neg0 = c16[0x8000];
    if (g == 511) cnt -= neg0;
    if (g == 512) cnt += neg0;
  }
  // keys below 0x7F (groups 0 and 1 but for its last key, -inf) are negative
  // NaNs; groups 1022 and 1023 hold +inf and positive NaNs
  const bool bad = (cnt != 0 && (g == 0 || g >= 1022)) ||
                   (g == 1 && cnt != c16[raw_of_key16(kKey16NegInf)]);
  const uint64_t ne = __ballot(cnt != 0);
  const uint32_t wsum = wave_sum(cnt);
  const uint64_t wbad = __ballot(bad);
  if (lane == 0) {
    S.wcount[wv] = (uint32_t)__popcll(ne);
    S.wtot[wv] = wsum;
    S.wbad[wv] = wbad ? 1u : 0u;
  }
  block_sync_lds();
  // lane v < 16 takes wave v's figures: total, validity, list offsets
  const uint32_t vcount = lane < 16 ? S.wcount[lane] : 0u;
  const uint32_t vtot = lane < 16 ? S.wtot[lane] : 0u;
  const bool anybad = __ballot(lane < 16 && S.wbad[lane] != 0) != 0;
  const uint32_t vincl = wave_incl_scan(vcount);
  const uint32_t total = wave_sum(vtot);
  const uint32_t nl = bcast(vincl, 15);
  const uint32_t off = wv > 0 ? bcast(vincl, wv - 1) : 0u;
  if (cnt != 0) {
    const uint32_t pos = off + (uint32_t)__popcll(ne & ((1ull << lane) - 1ull));
    S.list[pos] = (uint16_t)g;
    S.lcnt[pos] = cnt;
  }
  block_sync_lds();

  // count of key `key` (with -0 folded into +0)
  auto kcount = [&](uint32_t key) -> uint32_t {
    if (key == kKey16NegZero) return 0u;
    const uint32_t c = c16[raw_of_key16(key)];
    return key == kKey16PosZero ? c + c16[0x8000] : c;
  };
  auto clear_listed = [&]() {  // zero the groups that hold counts
    uint4* h4 = reinterpret_cast<uint4*>(hist);
    for (uint32_t i = tid >> 3; i < nl; i += NT / 8) {
      const uint32_t gl = S.list[i];
      const uint32_t rgl = gl >= 512 ? gl - 512u : 1023u - gl;
      h4[rgl * 8 + (tid & 7)] = make_uint4(0u, 0u, 0u, 0u);
    }
    if (tid == 0) c16[0x8000] = 0;  // -0 (its group may not be listed)
  };
  if (anybad) {
    if (tid == 0) {
      RowStat st = {__builtin_nanf(""), __builtin_nanf(""), 0.0, 0, {0, 0, 0}};
      S.res = st;
      if (out) *out = st;
    }
    block_sync_lds();
    clear_listed();
    return 1;
  }
  if ((int64_t)total != V) return 2;  // a 16-bit counter overflowed

  // Every wave finds the max finite key in the highest non-empty group.
  const uint32_t g0 = S.list[0];
  const uint64_t nzmax = __ballot(kcount(g0 * 64 + lane) != 0 && g0 * 64 + lane > kKey16NegInf);
  if (!nzmax) {  // no finite logit (only -inf)
    if (tid == 0) {
      RowStat st = {__builtin_nanf(""), __builtin_nanf(""), 0.0, 0, {0, 0, 0}};
      S.res = st;
      if (out) *out = st;
    }
    block_sync_lds();
    clear_listed();
    return 1;
  }
  const uint32_t max_key = g0 * 64 + (63 - __clzll((long long)nzmax));
  const float m = value_of_key16(max_key);
  // Wave 0, with top-k: the top-k key by exact counts.
  if (use_k && wv == 0) {
    if (lane == 0) {
      S.tk = 0;
      S.tk_entry = nl - 1;
    }
    uint32_t carry = 0;
    for (uint32_t base = 0; base < nl; base += kWave) {
      const uint32_t x = (base + lane < nl) ? S.lcnt[base + lane] : 0u;
      const uint32_t inc = wave_incl_scan(x) + carry;
      const uint64_t hit = __ballot(base + lane < nl && inc >= (uint32_t)top_k);
      if (hit) {
        const int L = __ffsll((unsigned long long)hit) - 1;
        const uint32_t before = bcast(inc - x, L);
        const uint32_t gk = S.list[base + L];
        const uint32_t c = kcount(gk * 64 + lane);
        const uint32_t suf = wave_incl_suffix(c) + before;
        const uint64_t ok = __ballot(suf >= (uint32_t)top_k);
        if (lane == 0) {
          S.tk = gk * 64 + (63 - __clzll((long long)ok));
          S.tk_entry = base + L;
        }
        break;
      }
      carry = bcast(inc, kWave - 1);
    }
  }
  if (use_k) block_sync_lds();
  const uint32_t tk = use_k ? S.tk : 0u;
  const uint32_t last = use_k ? S.tk_entry : nl - 1;  // entries after it lie below tk

  // Masses over keys >= tk, entry-major (octet_mass): the entries' masses
  // into S.gmass.
  {
    const uint32_t sub = (uint32_t)tid & 7u;
    const float vtk = value_of_key16(tk);
    const uint4* h4 = reinterpret_cast<const uint4*>(hist);
    for (uint32_t base = 0; base <= last; base += NT / 8) {
      const uint32_t e = base + (uint32_t)tid / 8u;
      float x[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
      if (e <= last) {
        const uint32_t gl = S.list[e];
        const bool posg = gl >= 512u;
        // the lane's keys 64 gl + 8 sub .. + 7 in raw-code order (magnitude
        // order for both signs): 16-byte word q holds the codes rb .. rb + 7
        const uint32_t q = (posg ? gl - 512u : 1023u - gl) * 8u + (posg ? sub : 7u - sub);
        const uint32_t rb = 8u * q;
        const uint4 w = h4[q];
        uint32_t c[8] = {w.x & 0xFFFFu, w.x >> 16, w.y & 0xFFFFu, w.y >> 16,
                         w.z & 0xFFFFu, w.z >> 16, w.w & 0xFFFFu, w.w >> 16};
        if (rb == 0u) c[0] += c16[0x8000];  // +0 takes the count of -0
        if (rb == 0x8000u) c[0] = 0u;       // -0
        x_masses8(x, c, rb, m, a, use_k, vtk);
      }
      const float gm = octet_mass(x);
      if (e <= last && sub == 4u) S.gmass[e] = gm;
    }
  }
  block_sync_lds();  // entry masses visible to wave 0

  // Wave 0: the fp64 prefix over the entries in list order, 64 at a time:
  // its total is the normaliser; then the top-p cut by cumulative mass from
  // the top.
  if (wv == 0) {
    double zk = 0.0;
    for (uint32_t base = 0; base <= last; base += kWave) {
      const uint32_t i = base + lane;
      zk = bcast(wave_incl_scan(i <= last ? (double)S.gmass[i] : 0.0) + zk, kWave - 1);
    }
    uint32_t thr_key = tk;
    double z = zk;
    if (use_p) {
      float tp = top_p;
      asm volatile("" : "+v"(tp));  // converted here, not held in registers across the scan
      const double target = (double)tp * zk;
      // the first entry whose running sum reaches the target (the last one
      // if rounding leaves none), then inside it the lowest key from which
      // the keys above still reach it
      double run = 0.0;
      for (uint32_t base = 0; base <= last; base += kWave) {
        const bool in = base + lane <= last;
        const double x = in ? (double)S.gmass[base + lane] : 0.0;
        const double inc = wave_incl_scan(x) + run;
        const uint64_t hit = __ballot(in && inc >= target);
        if (hit || base + kWave > last) {
          const int L = hit ? __ffsll((unsigned long long)hit) - 1 : (int)(last - base);
          const double before = bcast(inc - x, L);
          const uint32_t gc = S.list[base + L];
          const uint32_t key = gc * 64 + lane;
          const double e = key >= tk ? (double)key_mass(key, kcount(key), m, a) : 0.0;
          const double suf = wave_incl_suffix(e) + before;
          const uint64_t ok = __ballot(suf >= target);
          int pick;
          if (ok) {
            pick = 63 - __clzll((long long)ok);
          } else {  // rounding corner: the lowest key with mass in the group
            const uint64_t nzm = __ballot(e > 0.0);
            pick = nzm ? __ffsll((unsigned long long)nzm) - 1 : 0;
          }
          thr_key = max(tk, gc * 64 + (uint32_t)pick);
          z = bcast(suf, pick);
          break;
        }
        run = bcast(inc, kWave - 1);
      }
    }
    if (lane == 0) {
      RowStat st;
      st.m = m;
      st.thr = (use_k || use_p) ? value_of_key16(thr_key) : -__builtin_inff();
      st.z = z;
      st.valid = 1;
      st.pad[0] = st.pad[1] = st.pad[2] = 0;
      S.res = st;
      if (out) *out = st;
    }
  }
  block_sync_lds();
  clear_listed();
  return 0;
}

template <bool VEC>
__global__ __launch_bounds__(1024) void k_filter_bf16_hist(RowMap map, int64_t V, float a,
                                                           int top_k, float top_p,
                                                           RowStat* __restrict__ stats) {
  __shared__ uint32_t hist[32768];
  __shared__ HistScratch S;
  const int64_t r = blockIdx.x;
  const uint16_t* row = map.row<uint16_t>(r);
  hist_clear(hist);
  __syncthreads();
  hist_count_row<VEC>(hist, row, V);
  __syncthreads();
  if (hist_row_stats(hist, S, V, a, top_k, top_p, stats + r) == 2) {
    __syncthreads();
    filter_row_bisect<uint16_t, VEC, 1024>(row, V, a, top_k, top_p, stats + r, S.dslot, S.uslot);
  }
}

// ---------------------------------------------------------------------------
// Per-sequence tail of the stochastic verify, run by one workgroup of NT
// threads: row statistics, ratio test at every drafted position, first
// rejection, then the residual max(0, p - q) at the rejected position (or the
// bonus row's p) drawn by inverse CDF in ascending vocabulary order:
// wave-contiguous segments of the row, 8 elements per lane per step, fp64
// running sums (wave totals -> crossing wave -> crossing step -> crossing
// lane -> crossing element, all from the same additions).
struct DrawJob;

struct TailArgs {
  RowMap map;
  int64_t V;
  int32_t k;
  float a;
  const int32_t* tokens;
  const float* u;
  RowStat* rowstat;  // filtered rows (one per row), or nullptr
  Partial* part;     // unfiltered rows (nchunks per row), or nullptr
  int32_t nchunks;
  int32_t* accepted_len;
  int32_t* out_tokens;
  float* accept_prob;
  // non-null: the correction draw is left to k_draw_split; the tail writes
  // each valid sequence's job and every output but the drawn token and the
  // accepted length
  DrawJob* jobs = nullptr;
};

struct TailScratch {
  RowStat st[2 * SPEC_MAX_K + 1];
  double csum[8 * kDrawChunks];  // residual-draw chunk sums (512 threads)
  int32_t n, valid, emit;
};

__device__ __forceinline__ double prob_at(float l, const RowStat& s, float a) {
  if (!(l >= s.thr)) return 0.0;
  return exp2_d(((double)l - (double)s.m) * (double)a) / s.z;
}

// Buffer descriptor of one aligned bf16 row's full 16-byte groups: the
// streaming loads then take one 32-bit VGPR offset and a scalar offset per
// load in flight, which keeps the address registers out of the way (a load
// past the row's whole groups returns zeros).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t row_rsrc(const uint16_t* row, int64_t V) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(row), (short)0,
                                           (int)((V / 8) * 16), 0x00020000);
}

__device__ __forceinline__ uint4 rsrc_load16(__amdgpu_buffer_rsrc_t rs, uint32_t voff,
                                             uint32_t soff) {
  const auto v = __builtin_amdgcn_raw_buffer_load_b128(rs, (int)voff, (int)soff, 0);
  return make_uint4(v[0], v[1], v[2], v[3]);
}

// Inverse-CDF draw in ascending vocabulary order from the normalised residual
// max(0, p - q) of two processed rows, or from p alone (has_q false, or a
// residual without mass).  All NT threads take part; every thread returns the
// drawn index.  csum ([NT / 64][kDrawChunks] doubles) and emit_slot are LDS
// scratch.
struct DrawStats {  // what the draw needs of a processed row
  float m, thr;
  double z;
};

__device__ __forceinline__ DrawStats draw_stats(const RowStat& s) { return {s.m, s.thr, s.z}; }

// log2(z) of a row's normaliser, so that p = 2^((l - m) a - log2 z): the
// exponent plus log2 of the mantissa (hardware single-precision log2 on
// [1, 2)).  l - m is exact for the logits of one row, so even huge logits
// keep their probabilities.
__device__ __forceinline__ float log2_norm(double z) {
  int e = 0;
  const double f = __builtin_frexp(z, &e);  // z = f 2^e, f in [0.5, 1)
  return (float)((double)(e - 1) + (double)__builtin_amdgcn_logf((float)(2.0 * f)));
}

template <typename T, bool VEC, int NT, int U, int PD = 0>
__device__ __forceinline__ int32_t residual_draw(const T* prow, const T* qrow, bool has_q, const DrawStats sp,
                                 const DrawStats sq, float a, int64_t V, float u, double* csum,
                                 int32_t* emit_slot) {
  constexpr int NW = NT / kWave;
  constexpr int E = NW * kDrawChunks / kWave;  // chunk entries per lane in the prefix
  static_assert(E * kWave == NW * kDrawChunks, "chunk table must fill whole lanes");
  int tid = threadIdx.x;
  asm volatile("" : "+v"(tid));
  const int lane = tid & (kWave - 1);
  const int w = tid / kWave;
  const float lzp = log2_norm(sp.z), lzq = log2_norm(sq.z);
  bool resid = has_q;
  const int64_t nsteps = (V + 511) / 512;
  const int64_t spw = (nsteps + NW - 1) / NW;
  const int64_t s0 = (int64_t)w * spw;
  const int64_t s1 = min(nsteps, s0 + spw);
  // Each wave's span is cut into at most kDrawChunks chunks of cs steps whose
  // sums are kept (csum[w][c], zero past the wave's last chunk), so the
  // crossing is located from the table and one chunk is read again.  A
  // chunk's sum is each lane's fp64 share over the chunk's steps, reduced
  // once across the wave; the second pass walks the same per-step values in
  // step order (the two differ only in the order of fp64 additions).
  const int64_t cs = (spw + kDrawChunks - 1) / kDrawChunks;

  // Residual (or p) of the 8 elements of lane `lane` in step s; returns their
  // sum (fp32 in element order -- the same additions the crossing search
  // repeats -- widened to fp64).
  auto residual8 = [&](const float* lp, const float* lq, float* r8) -> double {
    float acc = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float p = lp[i] >= sp.thr
                          ? __builtin_amdgcn_exp2f(__builtin_fmaf(lp[i] - sp.m, a, -lzp))
                          : 0.0f;
      float r = p;
      if (resid) {
        const float q = lq[i] >= sq.thr
                            ? __builtin_amdgcn_exp2f(__builtin_fmaf(lq[i] - sq.m, a, -lzq))
                            : 0.0f;
        r = fmaxf(p - q, 0.0f);
      }
      r8[i] = r;
      acc += r;
    }
    return (double)acc;
  };
  // U steps per batch: all their loads are issued before any is used.
  auto load_batch = [&](int64_t s, Raw8<T>* rp, Raw8<T>* rq) {
#pragma unroll
    for (int v = 0; v < U; ++v) {
      const int64_t e = (s + v) * 512 + lane * 8;
      load8_raw<T, VEC>(prow, e, V, rp[v]);
      if (resid) load8_raw<T, VEC>(qrow, e, V, rq[v]);
    }
  };
  auto step_values = [&](const Raw8<T>& rp, const Raw8<T>& rq, float* r8) -> double {
    float lp[8], lq[8];
    unpack8<T>(rp, lp);
    if (resid) unpack8<T>(rq, lq);
    return residual8(lp, lq, r8);
  };

  // Pass 1: chunk sums; then every wave forms the same prefix over the
  // table (chunk order = vocabulary order) and locates the crossing.
  double S = 0.0, inc = 0.0, lsum = 0.0;
  double ent[E];
  for (int attempt = 0; attempt < 2; ++attempt) {
    if (lane < kDrawChunks) csum[w * kDrawChunks + lane] = 0.0;
    double cacc = 0.0;
    int ci = 0;
    int64_t cend = s0 + cs;
    // this lane's values of step st (wave-uniform st) into the chunk sums
    auto account = [&](int64_t st, double ls) {
      cacc += ls;
      if (st + 1 == cend || st + 1 == s1) {
        const double tot = wave_sum(cacc);
        if (lane == 0) csum[w * kDrawChunks + ci] = tot;
        ++ci;
        cacc = 0.0;
        cend += cs;
      }
    };
    int64_t s = s0;
    if constexpr (PD > 0 && VEC && sizeof(T) == 2) {
      // Aligned bf16 rows: a rolling window of PD steps in flight per wave
      // (one 16-byte vector per lane and row each), refilled as each step
      // is used, over the steps that lie wholly inside the row.
      const int64_t sf = min(s1, V / 512);
      const __amdgpu_buffer_rsrc_t rsp = row_rsrc(prow, V);
      const __amdgpu_buffer_rsrc_t rsq = row_rsrc(qrow, V);
      const uint32_t lo = (uint32_t)lane * 16u;
      uint4 bp[PD], bq[PD];
#pragma unroll
      for (int d = 0; d < PD; ++d) {
        if (s0 + d < sf) {
          const uint32_t off = (uint32_t)(s0 + d) * 1024u + lo;
          bp[d] = rsrc_load16(rsp, off, 0u);
          if (resid) bq[d] = rsrc_load16(rsq, off, 0u);
        }
      }
      for (; s < sf; s += PD) {
#pragma unroll
        for (int d = 0; d < PD; ++d) {
          const int64_t st = s + d;
          if (st < sf) {
            Raw8<T> rp, rq;
            rp.v[0] = bp[d];
            rq.v[0] = resid ? bq[d] : bp[d];
            if (st + PD < sf) {
              const uint32_t off = (uint32_t)(st + PD) * 1024u + lo;
              bp[d] = rsrc_load16(rsp, off, 0u);
              if (resid) bq[d] = rsrc_load16(rsq, off, 0u);
            }
            float r8[8];
            account(st, step_values(rp, rq, r8));
          }
        }
      }
      s = max(s0, sf);
    }
    // the remaining steps (all of them for other rows), U at a time
    for (; s < s1; s += U) {
      Raw8<T> rp[U], rq[U];
      load_batch(s, rp, rq);
#pragma unroll
      for (int v = 0; v < U; ++v) {
        float r8[8];
        const double ls = step_values(rp[v], rq[v], r8);
        if (s + v < s1) account(s + v, ls);  // this lane's share of the chunk
      }
    }
    block_sync_lds();
    lsum = 0.0;
#pragma unroll
    for (int e = 0; e < E; ++e) {
      ent[e] = csum[lane * E + e];
      lsum += ent[e];
    }
    inc = wave_incl_scan(lsum);
    S = bcast(inc, kWave - 1);
    if (S > 0.0 || !resid) break;
    resid = false;  // a residual without mass falls back to p at that position
    block_sync_lds();
  }
  const double target = (double)u * S;
  // the first table entry whose running sum exceeds the target; if rounding
  // leaves none, the last entry with mass
  int gstar = -1;
  double cum = 0.0;
  {
    const uint64_t hit = __ballot(inc > target);
    int L;
    bool crossed = hit != 0;
    if (crossed) {
      L = __ffsll((unsigned long long)hit) - 1;
    } else {
      const uint64_t pos = __ballot(lsum > 0.0);
      L = pos ? 63 - __clzll((long long)pos) : 0;
    }
    double base = bcast(inc - lsum, L);
    int epick = -1, elast = 0;
    double run = base, before = base, before_last = base;
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const double x = bcast(ent[e], L);
      if (x > 0.0) {
        elast = e;
        before_last = run;
      }
      if (epick < 0 && crossed && run + x > target) {
        epick = e;
        before = run;
      }
      run += x;
    }
    if (epick < 0) {
      epick = elast;
      before = before_last;
    }
    gstar = L * E + epick;
    cum = before;
  }
  const int wstar = gstar / kDrawChunks, cstar = gstar % kDrawChunks;
  if (w == wstar) {
    const int64_t c0 = s0 + (int64_t)cstar * cs, c1 = min(s1, c0 + cs);
    double wt = 0.0;
    bool done = false;
    for (int64_t s = c0; s < c1 && !done; s += U) {
      Raw8<T> rp[U], rq[U];
      load_batch(s, rp, rq);
#pragma unroll
      for (int v = 0; v < U; ++v) {
        if (done || s + v >= c1) continue;
        float r8[8];
        const double ls = step_values(rp[v], rq[v], r8);
        const double sinc = wave_incl_scan(ls);
        const double stot = bcast(sinc, kWave - 1);
        if (cum + (wt + stot) > target || s + v == c1 - 1) {
          const uint64_t hit = __ballot(cum + (wt + sinc) > target);
          const uint64_t pos = __ballot(ls > 0.0);
          int L;
          if (hit) {
            L = __ffsll((unsigned long long)hit) - 1;
            if (!((pos >> L) & 1ull)) {  // rounding corner: nearest lane with mass
              const uint64_t below = pos & ((2ull << L) - 1ull);
              L = below ? 63 - __clzll((long long)below)
                        : (pos ? __ffsll((unsigned long long)pos) - 1 : L);
            }
          } else {
            L = pos ? 63 - __clzll((long long)pos) : 0;
          }
          const double excl = L > 0 ? bcast(sinc, L - 1) : 0.0;
          if (lane == L) {
            const double base = cum + (wt + excl);
            float run = 0.0f;
            int pick = -1, lastpos = -1;
            for (int i = 0; i < 8; ++i) {
              if (r8[i] > 0.0f) lastpos = i;
              run += r8[i];
              if (pick < 0 && base + (double)run > target) pick = i;
            }
            if (pick < 0 || !(r8[pick] > 0.0f)) pick = lastpos >= 0 ? lastpos : 0;
            *emit_slot = (int32_t)((s + v) * 512 + lane * 8 + pick);
          }
          done = true;
          continue;
        }
        wt += stot;
      }
    }
  }
  block_sync_lds();
  return *emit_slot;
}

// ---------------------------------------------------------------------------
// Correction draw spread over the chip, for small batches on the row-pass
// path (one tail workgroup per sequence would read the two rows at the stop
// alone while the other CUs sit idle).  The tail writes each sequence's
// DrawJob; k_draw_split computes the residual's sum over every chunk of
// kDrawChunk elements of the two rows at the stop (one workgroup per
// chunk), and the workgroup that writes a sequence's last chunk sum finds
// the chunk where the running sum in ascending vocabulary order passes u S,
// and the element inside it.  A chunk's sum is formed by the same additions
// both times (per-thread fp64 sums of fp32 group sums, then one block
// scan), so the chunk picked from the table always holds the crossing.
struct DrawJob {  // 48 bytes
  DrawStats sp, sq;  // processed target row at the stop, and draft row (unused for the bonus)
  int32_t n;         // the stop (k: the bonus draw from p_k)
  int32_t active;    // 0: nothing to draw (invalid sequence, outputs already written)
  uint32_t done;     // chunk sums written so far (the last writer draws)
  int32_t pad;
};
constexpr int kDrawThreads = 256;
constexpr int kDrawGroups = 2;  // groups of 8 elements per thread
constexpr int64_t kDrawChunk = (int64_t)kDrawThreads * kDrawGroups * 8;  // 4,096 elements

// This thread's share of chunk c: the fp32 sums of its groups (in element
// order) and their fp64 total (in group order); with r32, also every
// element's value (the picking workgroup walks them without reading again).
template <typename T, bool VEC>
__device__ __forceinline__ double draw_thread_sum(const T* prow, const T* qrow, bool resid,
                                                  const DrawJob& J, float lzp, float lzq, float a,
                                                  int64_t V, int64_t c, int tid, float* gs,
                                                  float* r32 = nullptr) {
  const int64_t e0 = c * kDrawChunk + (int64_t)tid * (kDrawGroups * 8);
  Raw8<T> rp[kDrawGroups], rq[kDrawGroups];
#pragma unroll
  for (int g = 0; g < kDrawGroups; ++g) {  // every load issued before any is used
    load8_raw<T, VEC>(prow, e0 + 8 * g, V, rp[g]);
    if (resid) load8_raw<T, VEC>(qrow, e0 + 8 * g, V, rq[g]);
  }
  double tot = 0.0;
#pragma unroll
  for (int g = 0; g < kDrawGroups; ++g) {
    float lp[8], lq[8];
    unpack8<T>(rp[g], lp);
    if (resid) unpack8<T>(rq[g], lq);
    float acc = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float p = lp[i] >= J.sp.thr
                          ? __builtin_amdgcn_exp2f(__builtin_fmaf(lp[i] - J.sp.m, a, -lzp))
                          : 0.0f;
      float r = p;
      if (resid) {
        const float q = lq[i] >= J.sq.thr
                            ? __builtin_amdgcn_exp2f(__builtin_fmaf(lq[i] - J.sq.m, a, -lzq))
                            : 0.0f;
        r = fmaxf(p - q, 0.0f);
      }
      if (r32) r32[8 * g + i] = r;
      acc += r;
    }
    gs[g] = acc;
    tot += (double)acc;
  }
  return tot;
}

// Inclusive scan of one double per thread over the 256 threads (wave scans,
// then the four wave totals added in wave order); *total is the last
// thread's value, formed by the same additions.
__device__ __forceinline__ double block_incl_scan256(double x, double* slots, double* total) {
  const int tid = threadIdx.x, lane = tid & (kWave - 1), w = tid / kWave;
  const double inc = wave_incl_scan(x);
  if (lane == kWave - 1) slots[w] = inc;
  block_sync_lds();
  double base = 0.0;
  for (int v = 0; v < w; ++v) base += slots[v];
  *total = ((slots[0] + slots[1]) + slots[2]) + slots[3];
  return base + inc;
}

// Chunk sums pass between the workgroups of a sequence (on any XCD; the
// XCDs' L2 caches are not coherent with one another) through atomic
// read-modify-writes and atomic loads at device scope, without cache
// flushes.
__device__ __forceinline__ void sum_publish(double* p, double v) {
  (void)__hip_atomic_exchange(reinterpret_cast<uint64_t*>(p), __builtin_bit_cast(uint64_t, v),
                              __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ double sum_read(const double* p) {
  return __builtin_bit_cast(double, __hip_atomic_load(reinterpret_cast<const uint64_t*>(p),
                                                      __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
}

// The draw of sequence b from its chunk sums (one workgroup, after every
// chunk sum is written); writes the emitted token and the accepted length,
// then leaves the sequence's job and chunk sums zero for the next call.
template <typename T, bool VEC>
__device__ void draw_pick(RowMap map, int64_t V, int k, float a, DrawJob* __restrict__ jobs,
                          int64_t nch, double* __restrict__ sums, const float* __restrict__ u,
                          int32_t* __restrict__ accepted_len, int32_t* __restrict__ out_tokens,
                          int64_t b, const DrawJob& J, double* slots) {
  __shared__ int32_t emit;
  __shared__ int64_t sh_chunk;
  __shared__ double sh_target, sh_S;
  __shared__ int32_t sh_last, sh_pick;
  __shared__ uint64_t sh_hits[kDrawThreads / kWave], sh_pos[kDrawThreads / kWave];
  const int tid = threadIdx.x, lane = tid & (kWave - 1), w = tid / kWave;
  const int n = J.n;
  bool resid = n < k;
  const T* prow = map.template at<T>(b, n);
  const T* qrow = resid ? map.template at<T>(b, k + 1 + n) : prow;
  const float uu = u[b * (k + 1) + k];
  double* sb = sums + b * nch;
  const float lzp = log2_norm(J.sp.z), lzq = resid ? log2_norm(J.sq.z) : 0.0f;

  // A residual without mass falls back to p at the stop: this workgroup
  // forms p's chunk sums (the rows are read once more; rounding makes this
  // case all but unreachable).
  if (w == 0) {
    double carry = 0.0;
    for (int64_t base = 0; base < nch; base += kWave)
      carry += wave_sum(base + lane < nch ? sum_read(sb + base + lane) : 0.0);
    if (lane == 0) sh_S = carry;
  }
  block_sync_lds();
  if (resid && !(sh_S > 0.0)) {
    resid = false;
    for (int64_t c = 0; c < nch; ++c) {
      float gs[kDrawGroups];
      const double x = draw_thread_sum<T, VEC>(prow, qrow, false, J, lzp, lzq, a, V, c, tid, gs);
      double total;
      (void)block_incl_scan256(x, slots, &total);
      if (tid == 0) sum_publish(sb + c, total);
      block_sync_lds();  // slots are rewritten by the next chunk's scan
    }
    __syncthreads();
  }

  // Wave 0: S, the target u S, and the first chunk whose running sum
  // exceeds it (if rounding leaves none, the last chunk with mass).
  if (w == 0) {
    double carry = 0.0;
    for (int64_t base = 0; base < nch; base += kWave)
      carry += wave_sum(base + lane < nch ? sum_read(sb + base + lane) : 0.0);
    const double S = carry, target = (double)uu * S;
    int64_t pick = -1, lastpos = -1;
    double before = 0.0, before_last = 0.0, run = 0.0;
    for (int64_t base = 0; base < nch && pick < 0; base += kWave) {
      const double x = base + lane < nch ? sum_read(sb + base + lane) : 0.0;
      const double inc = wave_incl_scan(x) + run;
      const uint64_t hit = __ballot(base + lane < nch && inc > target);
      const uint64_t pos = __ballot(base + lane < nch && x > 0.0);
      if (pos) {
        const int L = 63 - __clzll((long long)pos);
        lastpos = base + L;
        before_last = bcast(inc - x, L);
      }
      if (hit) {
        const int L = __ffsll((unsigned long long)hit) - 1;
        pick = base + L;
        before = bcast(inc - x, L);
      }
      run = bcast(inc, kWave - 1);
    }
    if (lane == 0) {
      sh_S = S;
      sh_last = pick < 0 ? 1 : 0;
      sh_chunk = pick >= 0 ? pick : (lastpos >= 0 ? lastpos : 0);
      sh_target = target - (pick >= 0 ? before : before_last);
    }
  }
  block_sync_lds();
  int32_t emitted;
  {
    const int64_t c = sh_chunk;
    const bool last = sh_last != 0;
    const double tc = sh_target;  // the target within chunk c
    float gs[kDrawGroups], r32[kDrawGroups * 8];
    const double x = draw_thread_sum<T, VEC>(prow, qrow, resid, J, lzp, lzq, a, V, c, tid, gs, r32);
    double total;
    const double inc = block_incl_scan256(x, slots, &total);
    // the first thread whose running sum exceeds the target, else the last
    // thread with mass
    const uint64_t hit = __ballot(!last && inc > tc);
    const uint64_t pos = __ballot(x > 0.0);
    if (lane == 0) {
      sh_hits[w] = hit;
      sh_pos[w] = pos;
    }
    block_sync_lds();
    if (tid == 0) {
      int t = -1;
      for (int v = 0; v < kDrawThreads / kWave && t < 0; ++v)
        if (sh_hits[v]) t = v * kWave + __ffsll((unsigned long long)sh_hits[v]) - 1;
      if (t < 0)
        for (int v = kDrawThreads / kWave - 1; v >= 0 && t < 0; --v)
          if (sh_pos[v]) t = v * kWave + 63 - __clzll((long long)sh_pos[v]);
      sh_pick = t < 0 ? 0 : t;
      emit = -1;
    }
    block_sync_lds();
    if (tid == sh_pick) {
      // walk this thread's groups, then the elements of the crossing group
      const bool crossing = !last && inc > tc;
      double run = inc - x;
      const int64_t e0 = c * kDrawChunk + (int64_t)tid * (kDrawGroups * 8);
      int64_t found = -1, lastpos = -1;
      for (int g = 0; g < kDrawGroups && found < 0; ++g) {
        if (crossing && !(run + (double)gs[g] > tc)) {
          run += (double)gs[g];
          continue;
        }
        const float* r8 = r32 + 8 * g;  // the values summed above, the same arithmetic
        for (int i = 0; i < 8; ++i) {
          if (r8[i] > 0.0f) lastpos = e0 + 8 * g + i;
          if (crossing && found < 0 && run + (double)r8[i] > tc) found = e0 + 8 * g + i;
          run += (double)r8[i];
        }
        if (crossing) break;  // the crossing group: rounding inside it ends the walk here
      }
      emit = (int32_t)(found >= 0 ? found : (lastpos >= 0 ? lastpos : c * kDrawChunk));
    }
    block_sync_lds();
    emitted = emit;
  }
  if (tid == 0) {
    out_tokens[b * (k + 1) + n] = emitted;
    accepted_len[b] = n;
  }
  // leave this sequence's job and chunk sums zero for the next call
  block_sync_lds();
  for (int64_t i = tid; i < nch; i += kDrawThreads) sums[b * nch + i] = 0.0;
  if (tid < (int)(sizeof(DrawJob) / 4)) reinterpret_cast<int32_t*>(jobs + b)[tid] = 0;
}

// One workgroup per (chunk, sequence): the chunk's sum; the last of a
// sequence's workgroups to write its sum then draws the token.
template <typename T, bool VEC>
__global__ __launch_bounds__(kDrawThreads) void k_draw_split(RowMap map, int64_t V, int k, float a,
                                                            DrawJob* __restrict__ jobs, int64_t nch,
                                                            double* __restrict__ sums,
                                                            const float* __restrict__ u,
                                                            int32_t* __restrict__ accepted_len,
                                                            int32_t* __restrict__ out_tokens) {
  __shared__ double slots[kDrawThreads / kWave];
  __shared__ int32_t sh_is_last;
  const int64_t b = blockIdx.y, c = blockIdx.x;
  const DrawJob J = jobs[b];
  if (!J.active) return;  // outputs already written; job and sums stay zero
  const bool resid = J.n < k;
  const T* prow = map.template at<T>(b, J.n);
  const T* qrow = resid ? map.template at<T>(b, k + 1 + J.n) : prow;
  const float lzp = log2_norm(J.sp.z), lzq = resid ? log2_norm(J.sq.z) : 0.0f;
  float gs[kDrawGroups];
  const double x = draw_thread_sum<T, VEC>(prow, qrow, resid, J, lzp, lzq, a, V, c,
                                           (int)threadIdx.x, gs);
  double total;
  (void)block_incl_scan256(x, slots, &total);
  if (threadIdx.x == 0) {
    sum_publish(sums + b * nch + c, total);
    // the exchange has completed before the count goes up: a workgroup that
    // sees the count at nch - 1 finds every chunk's sum in place
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    const uint32_t prev = __hip_atomic_fetch_add(&jobs[b].done, 1u, __ATOMIC_RELAXED,
                                                 __HIP_MEMORY_SCOPE_AGENT);
    sh_is_last = prev + 1u == (uint32_t)nch ? 1 : 0;
  }
  block_sync_lds();
  if (!sh_is_last) return;
  draw_pick<T, VEC>(map, V, k, a, jobs, nch, sums, u, accepted_len, out_tokens, b, J, slots);
}

__device__ __forceinline__ void write_draw_job(DrawJob* job, const DrawStats& sp, const DrawStats& sq,
                                               int n) {
  DrawJob J;
  J.sp = sp;
  J.sq = sq;
  J.n = n;
  J.active = 1;
  J.done = 0u;
  J.pad = 0;
  *job = J;
}

template <typename T, bool VEC, int NT>
__device__ void seq_tail(const TailArgs& A, int64_t b, TailScratch& TS) {
  const int k = A.k;
  const int nr = 2 * k + 1;
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int w = tid / kWave;
  const int64_t V = A.V;
  const float a = A.a;

  // Wave 0, lane j < k: position j's drafted token, its draw and the two
  // logits at the token (a bad map entry reads flat row 0, which is readable
  // and decides nothing).  With row records to read they are loaded first,
  // so that their round trips overlap the records'; when wave 0 merges
  // partials or reads rows itself, after the statistics.
  int32_t x_j = -1;
  float u_j = 0.0f, lt_j = 0.0f, ld_j = 0.0f;
  auto load_position = [&]() {
    if (w == 0 && lane < k) {
      x_j = A.tokens[b * k + lane];
      u_j = A.u[b * (k + 1) + lane];
      if (x_j >= 0 && (int64_t)x_j < V) {
        lt_j = Elem<T>::load1(A.map.at<T>(b, lane) + x_j);
        ld_j = Elem<T>::load1(A.map.at<T>(b, k + 1 + lane) + x_j);
      }
    }
  };
  const bool early = A.rowstat != nullptr;
  if (early) load_position();

  // Row statistics of this sequence.  Dense rows belong to this sequence
  // alone and their workspace records are cleared here; pooled records are
  // shared and cleared by a pass of their own after every sequence is done.
  const bool pooled = A.map.nt > 0;
  if (!A.rowstat && !A.part) {
    // small unfiltered rows (no row pass): each wave computes the max and
    // the sum of 2^((l - m) a) of its rows, reading each row twice (the
    // second read from cache)
    constexpr int NW = NT / kWave;
    for (int t = w; t < nr; t += NW) {
      const int64_t rr = A.map.sidx(b, t);
      RowStat s = {0.f, 0.f, 0.0, 0, {0, 0, 0}};
      if (rr >= 0) {
        const T* row = A.map.template row<T>(rr);
        float m = -__builtin_inff();
        bool bad = false;
        for (int64_t e = (int64_t)lane * 8; e < V; e += kWave * 8) {
          float x[8];
          load8<T, VEC>(row, e, V, x);
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            bad = bad || bad_logit(x[i]);
            m = fmaxf(m, x[i]);
          }
        }
        m = wave_max(m);
        bad = __ballot(bad) != 0;
        double z = 0.0;
        if (!bad && m > -__builtin_inff()) {
          for (int64_t e = (int64_t)lane * 8; e < V; e += kWave * 8) {
            float x[8], ex[8];
            load8<T, VEC>(row, e, V, x);
#pragma unroll
            for (int i = 0; i < 8; ++i) ex[i] = __builtin_amdgcn_exp2f((x[i] - m) * a);
            z += (double)(((ex[0] + ex[1]) + (ex[2] + ex[3])) + ((ex[4] + ex[5]) + (ex[6] + ex[7])));
          }
          z = wave_sum(z);
        }
        s.m = m;
        s.thr = -__builtin_inff();
        s.z = z;
        s.valid = (!bad && m > -__builtin_inff()) ? 1 : 0;
      }
      if (lane == 0) TS.st[t] = s;
    }
  } else if (!A.rowstat && A.nchunks > 16) {
    // many chunks per row (a small batch spread over the chip): one wave
    // merges each row's partials
    constexpr int NW = NT / kWave;
    for (int t = w; t < nr; t += NW) {
      const int64_t rr = A.map.sidx(b, t);
      RowStat s = {0.f, 0.f, 0.0, 0, {0, 0, 0}};
      if (rr >= 0) {
        Partial* p = A.part + rr * A.nchunks;
        s = merge_partials_wave(p, A.nchunks, a, lane);
        if (!pooled) {
          for (int c = lane; c < A.nchunks; c += kWave) {
            Partial zero = {0.f, 0u, 0.0};
            p[c] = zero;
          }
        }
      }
      if (lane == 0) TS.st[t] = s;
    }
  } else {
    for (int t = tid; t < nr; t += NT) {
      const int64_t rr = A.map.sidx(b, t);
      RowStat s = {0.f, 0.f, 0.0, 0, {0, 0, 0}};
      if (rr >= 0) {
        if (A.rowstat) {
          s = A.rowstat[rr];
          if (!pooled) {
            RowStat zero = {0.f, 0.f, 0.0, 0, {0, 0, 0}};
            A.rowstat[rr] = zero;
          }
        } else {
          Partial* p = A.part + rr * A.nchunks;
          s = merge_partials(p, A.nchunks, a);
          if (!pooled) {
            for (int c = 0; c < A.nchunks; ++c) {
              Partial zero = {0.f, 0u, 0.0};
              p[c] = zero;
            }
          }
        }
      }
      TS.st[t] = s;
    }
  }
  block_sync_lds();
  if (!early) load_position();

  // Ratio test (wave 0, lane j = position j).  Positions are walked in
  // order and the first rejection stops the walk: the sequence is invalid
  // only if an ill-formed position (invalid row or token out of range) comes
  // before it, or every position passes and the bonus row is invalid.
  if (w == 0) {
    bool formed = false, acc = false;
    if (lane < k) {
      const int32_t x = x_j;
      formed = TS.st[lane].valid != 0 && TS.st[k + 1 + lane].valid != 0 && x >= 0 &&
               (int64_t)x < V;
      float alpha_out = __builtin_nanf("");
      if (formed) {
        const double p = prob_at(lt_j, TS.st[lane], a);
        const double q = prob_at(ld_j, TS.st[k + 1 + lane], a);
        const double alpha = q > 0.0 ? fmin(1.0, p / q) : (p > 0.0 ? 1.0 : 0.0);
        acc = (double)u_j < alpha;
        alpha_out = (float)alpha;
      }
      if (A.accept_prob) A.accept_prob[b * k + lane] = alpha_out;
    }
    const uint64_t stop = __ballot(lane < k && !acc);
    const uint64_t ill = __ballot(lane < k && !formed);
    if (lane == 0) {
      const int n = stop ? (__ffsll((unsigned long long)stop) - 1) : k;
      TS.n = n;
      TS.valid = (n < k ? !((ill >> n) & 1ull) : TS.st[k].valid != 0) ? 1 : 0;
    }
  }
  block_sync_lds();
  int32_t* out = A.out_tokens + b * (k + 1);
  if (!TS.valid) {
    for (int j = tid; j <= k; j += NT) out[j] = -1;
    if (tid == 0) A.accepted_len[b] = -1;
    return;
  }
  const int n = TS.n;

  // Residual max(0, p_n - q_n) (n < k) or the bonus row's p_k (n = k).
  const bool has_q = n < k;
  if (A.jobs) {
    for (int j = tid; j <= k; j += NT)
      if (j != n) out[j] = j < n ? A.tokens[b * k + j] : -1;
    if (tid == 0) write_draw_job(A.jobs + b, draw_stats(TS.st[n]),
                                 draw_stats(has_q ? TS.st[k + 1 + n] : TS.st[n]), n);
    return;
  }
  const T* prow = A.map.at<T>(b, n);
  const T* qrow = has_q ? A.map.at<T>(b, k + 1 + n) : prow;
  const int32_t emitted =
      residual_draw<T, VEC, NT, sizeof(T) == 2 ? 4 : 2, 4>(prow, qrow, has_q, draw_stats(TS.st[n]),
                                draw_stats(has_q ? TS.st[k + 1 + n] : TS.st[n]), a, V,
                                A.u[b * (k + 1) + k], TS.csum, &TS.emit);
  for (int j = tid; j <= k; j += NT) {
    int32_t v = -1;
    if (j < n) v = A.tokens[b * k + j];
    else if (j == n) v = emitted;
    out[j] = v;
  }
  if (tid == 0) A.accepted_len[b] = n;
}

// Out-of-line entry point of the bisection fallback, so that its registers do
// not burden the persistent kernel's streaming loop.
template <typename T, bool VEC, int NT>
__device__ __noinline__ void filter_row_bisect_call(const T* row, int64_t V, float a, int top_k,
                                                   float top_p, RowStat* out, double* dslot,
                                                   uint32_t* uslot) {
  filter_row_bisect<T, VEC, NT>(row, V, a, top_k, top_p, out, dslot, uslot);
}

template <typename T, bool VEC>
__global__ __launch_bounds__(512) void k_tail(TailArgs A) {
  __shared__ TailScratch TS;
  seq_tail<T, VEC, 512>(A, blockIdx.x, TS);
}

// ---------------------------------------------------------------------------
// Arguments of the persistent bf16 filter (sv_window.hpp), and the row
// streaming of the kernels that keep a row's histogram in LDS: while a row's
// histogram is scanned, the first PF vectors per thread of the next row are
// already loading (the scan's barriers order LDS only, so they do not wait
// for those loads).
struct FilterArgs {
  RowMap map;
  int64_t V;
  int64_t R;
  float a;
  int32_t top_k;
  float top_p;
  RowStat* stats;
};

// Streams one aligned bf16 row into the (cleared) histogram, D 16-byte loads
// in flight per thread; the first PF vectors of each thread come from `pf`
// when pf_ok (prefetched by prefetch_row during the previous row's scan).
template <int PF, int D>
__device__ __forceinline__ void hist_count_stream(uint32_t* hist, const uint16_t* row, int64_t V,
                                                  const uint4 (&pf)[PF], bool pf_ok) {
  constexpr uint32_t NT = 1024;
  uint32_t tid = threadIdx.x;
  asm volatile("" : "+v"(tid));  // recomputed per row, not held across the caller's loop
  const uint32_t nfull = (uint32_t)(V / 8);  // full 16-byte groups
  const uint32_t ngroups = (uint32_t)((V + 7) / 8);
  const __amdgpu_buffer_rsrc_t rs = row_rsrc(row, V);
  uint32_t g = tid;
  if (pf_ok) {
#pragma unroll
    for (int j = 0; j < PF; ++j) {
      const uint32_t gj = tid + (uint32_t)j * NT;
      if (gj < nfull) {
        hist_add8(hist, pf[j]);
      } else {
        for (uint32_t i = 0; i < 8 && (int64_t)gj * 8 + i < V; ++i) hist_add1(hist, row[gj * 8 + i]);
      }
    }
    g = tid + (uint32_t)PF * NT;
  }
  for (; g + (D - 1) * NT < nfull; g += D * NT) {
    uint4 v[D];
#pragma unroll
    for (int d = 0; d < D; ++d) v[d] = rsrc_load16(rs, g * 16u, (uint32_t)d * NT * 16u);
#pragma unroll
    for (int d = 0; d < D; ++d) hist_add8(hist, v[d]);
  }
  // Fewer than D full vectors per thread remain.  Two or more are loaded
  // together (one at a time, each would wait a full memory latency: at
  // V = 128,256 five or six per thread); a single one, and the partial
  // group, one at a time.
  if (g + NT < nfull) {
    uint4 v[D - 1];
#pragma unroll
    for (int d = 0; d < D - 1; ++d) {
      const uint32_t gd = g + (uint32_t)d * NT;
      v[d] = gd < nfull ? rsrc_load16(rs, gd * 16u, 0u) : make_uint4(0u, 0u, 0u, 0u);
    }
#pragma unroll
    for (int d = 0; d < D - 1; ++d)
      if (g + (uint32_t)d * NT < nfull) hist_add8(hist, v[d]);
    g += (nfull - g + NT - 1) / NT * NT;  // the first of this thread's groups past the full ones
  }
  for (; g < ngroups; g += NT) {
    if (g < nfull) {
      hist_add8(hist, rsrc_load16(rs, g * 16u, 0u));
    } else {
      for (uint32_t i = 0; i < 8 && (int64_t)g * 8 + i < V; ++i) hist_add1(hist, row[g * 8 + i]);
    }
  }
}

template <int PF>
__device__ __forceinline__ void prefetch_row(uint4 (&pf)[PF], const uint16_t* row, int64_t V) {
  const uint32_t nfull = (uint32_t)(V / 8);
  const __amdgpu_buffer_rsrc_t rs = row_rsrc(row, V);
  uint32_t tid = threadIdx.x;
  asm volatile("" : "+v"(tid));
#pragma unroll
  for (int j = 0; j < PF; ++j) {
    const uint32_t g = tid + (uint32_t)j * 1024u;
    if (g < nfull) pf[j] = rsrc_load16(rs, tid * 16u, (uint32_t)j * 16384u);
  }
}

// ---------------------------------------------------------------------------
// Whole-sequence stochastic verify for large batches of aligned bf16 rows.
// One persistent workgroup per CU takes sequences from a queue and walks each
// one's positions in order -- target row j, draft row j, ratio test at j --
// until the first rejection (or ill-formed position), then draws the
// correction from the residual of the two rows just read, or, when every
// position passes, reads the bonus row and draws from it.  Rows past the stop
// are never read.  When accept_prob is requested every position is processed
// (alpha is reported past the stop); the decisions are the same.
struct SeqArgs {
  RowMap map;
  int64_t V;
  int32_t k, B;
  float a;
  int32_t top_k;
  float top_p;
  const int32_t* tokens;
  const float* u;
  int32_t* accepted_len;
  int32_t* out_tokens;
  float* accept_prob;
  // [4] sequences taken, workgroups out, sequences done, help records
  // allocated: zero on entry; the last workgroup out zeroes them again
  uint32_t* queue;
  const RowStat* tstats;  // pooled rows: statistics of the target pool (flat rows 0..nt-1)
  // Help with the rows of other workgroups' walks once the queue is empty,
  // in the region at `help` (HelpView): per-workgroup progress, help entries
  // and help records.
  uint64_t* help;
};

// Most workgroups the whole-sequence walk launches (one per CU).
constexpr int kMaxWalkGrid = 1024;

// The help region of the whole-sequence walk, for kMaxWalkGrid workgroups
// and walks of up to nr = 2k+1 steps:
//   hwg[g]     (1 + sequence) << 32 | (1 + step) of the walk of workgroup g,
//              or 0 when it walks none;
//   hent[g][w] step w of the walk of workgroup g: (tag << 32) | (state << 30)
//              | record, tag = 1 + the sequence; state 0: its walker counts
//              the row, 1: a helper counts it, 2: the helper's figures are in
//              hpool[record].  A walker's sequences grow, so an entry with a
//              smaller tag is stale;
//   hpool      help records: enough for every step of two sequences per
//              workgroup (beyond that a helper publishes without figures).
struct HelpView {
  uint64_t* hwg;
  uint64_t* hent;
  RowStat* hpool;
  uint32_t hcap;
  __host__ __device__ static int64_t records(int64_t nr) { return 2 * kMaxWalkGrid * nr; }
  __host__ __device__ static int64_t bytes(int64_t nr) {
    return 8 * kMaxWalkGrid + 8 * kMaxWalkGrid * nr + 32 * records(nr);
  }
  __device__ HelpView(uint64_t* base, int nr)
      : hwg(base),
        hent(base + kMaxWalkGrid),
        hpool(reinterpret_cast<RowStat*>(base + kMaxWalkGrid + (int64_t)kMaxWalkGrid * nr)),
        hcap((uint32_t)records(nr)) {}
};

struct SeqScratch {
  RowStat st[2 * SPEC_MAX_K + 1];  // statistics of the rows read, by row
  int32_t tok[SPEC_MAX_K];         // draft tokens of the sequence
  float uu[SPEC_MAX_K];            // accept draws of the sequence
  double csum[16 * kDrawChunks];   // residual-draw chunk sums
  int32_t emit;
  uint32_t next;      // the sequence taken next
  int32_t formed, accepted;  // decision at the current position
  RowStat hst;        // figures of the current row published by a helper
  int32_t hmode;      // 1: hst holds the current row's figures
  uint64_t hprev;     // the next step's entry before this walker claimed it
  int32_t hjob_g, hjob_s, hjob_slot, hjob_state;  // a helper's claimed row
  uint32_t hjob_tag;
};

constexpr uint32_t kHelpClaimed = 1u, kHelpPublished = 2u;
constexpr uint32_t kHelpNoRecord = 0x3FFFFFFFu;  // published without figures (records used up)
constexpr int kHelpWaitIters = 20000;  // bound of a walker's wait for a helper (~2 ms)

__device__ __forceinline__ uint64_t ld_agent(const uint64_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_agent(uint64_t* p, uint64_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Walk step w -> row slot of the sequence (target rows 0..k, draft rows k+1..).
// Whole rows: t_j is step 2j, d_j step 2j+1, the bonus row t_k step 2k.
// Pooled rows (target figures from the pre-pass): d_j is step j.
template <bool POOL>
__device__ __forceinline__ int step_slot(int w, int k) {
  if (POOL) return k + 1 + w;
  return (w & 1) ? k + 1 + (w >> 1) : (w >> 1);
}

// A walker's view of a step it claimed one row earlier: 1 with the figures
// in *out when a helper has published them (waiting, within a bound, for a
// helper that is counting the row), 0 when the walker counts it itself.
__device__ __noinline__ int help_resolve(uint64_t* ent, uint64_t prev, uint32_t tag,
                                         const RowStat* pool, RowStat* out) {
  if ((uint32_t)(prev >> 32) != tag) return 0;  // stale: the walker holds the step
  uint64_t e = prev;
  for (int it = 0; ((uint32_t)e >> 30) == kHelpClaimed; ++it) {
    if (it == kHelpWaitIters) return 0;
    __builtin_amdgcn_s_sleep(4);
    e = ld_agent(ent);
  }
  if ((uint32_t)(e >> 32) != tag || ((uint32_t)e >> 30) != kHelpPublished) return 0;
  const uint32_t rec = (uint32_t)e & 0x3FFFFFFFu;
  if (rec == kHelpNoRecord) return 0;
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
  const uint64_t* src = reinterpret_cast<const uint64_t*>(pool + rec);
  uint64_t* dst = reinterpret_cast<uint64_t*>(out);
  for (int i = 0; i < 4; ++i) dst[i] = ld_agent(src + i);
  return 1;
}

// The bf16 draw of a 1024-thread workgroup with scalar arguments: U steps
// per batch in the loop over the remaining steps, and PD steps in flight per
// wave in the rolling window over a row's whole steps (0: no window).
template <int U = 2, int PD = 0>
__device__ __forceinline__ int32_t residual_draw_call(const uint16_t* prow, const uint16_t* qrow,
                                                   bool has_q, float pm, float pthr, double pz,
                                                   float qm, float qthr, double qz, float a,
                                                   int64_t V, float u, double* csum,
                                                   int32_t* emit_slot) {
  return residual_draw<uint16_t, true, 1024, U, PD>(prow, qrow, has_q, DrawStats{pm, pthr, pz},
                                             DrawStats{qm, qthr, qz}, a, V, u, csum, emit_slot);
}

template <int PF, int D, bool POOL>
__global__ __launch_bounds__(1024) void k_verify_seq_bf16(SeqArgs A) {
  constexpr int NT = 1024;
  __shared__ uint32_t hist[32768];
  __shared__ HistScratch S;
  __shared__ SeqScratch Q;
  // thread index, opaque so that what derives from it is not held in
  // registers across the walk
  auto TID = []() {
    int t = threadIdx.x;
    asm volatile("" : "+v"(t));
    return t;
  };
  const int64_t V = A.V;
  const int k = A.k, k1 = k + 1, nr = 2 * k + 1;
  const int nsteps = POOL ? k : nr;
  const bool all_pos = A.accept_prob != nullptr;
  const int g = blockIdx.x;

  uint4 pf[PF];
  const uint16_t* pf_row = nullptr;  // the row whose first vectors pf holds
  hist_clear(hist);
  if (TID() == 0) Q.next = atomicAdd(&A.queue[0], 1u);
  block_sync_lds();
  uint32_t cur = Q.next;
  if (cur < (uint32_t)A.B) {
    pf_row = POOL ? A.map.template at<uint16_t>(cur, k1) : A.map.template row<uint16_t>((int64_t)cur * nr);
    prefetch_row(pf, pf_row, V);
  }

  while (cur < (uint32_t)A.B) {
    const int64_t b = cur;
    const uint32_t tag = cur + 1u;
    // the next sequence is taken from the queue late -- before the bonus row
    // or the correction -- so a workgroup never holds one it cannot start
    uint32_t grabbed = 0;
    bool have_next = false;
    // tokens and uniforms of the positions, published to LDS after the first
    // row's stream (their loads are back by then)
    int32_t tok_in = 0;
    float u_in = 0.0f, lt = 0.0f, ld = 0.0f;
    if (TID() < k) {
      tok_in = A.tokens[b * k + TID()];
      u_in = A.u[b * k1 + TID()];
    }
    // pooled rows: the target rows' statistics come from the pre-pass over
    // the target pool; only draft rows are streamed here
    RowStat tst_in = {0.f, 0.f, 0.0, 0, {0, 0, 0}};
    if constexpr (POOL) {
      if (TID() <= k) {
        const int64_t r = A.map.sidx(b, TID());
        if (r >= 0) tst_in = A.tstats[r];
      }
    }
    uint32_t nxt = (uint32_t)A.B;
    int j = 0, n = -1;
    bool draft = POOL, valid = true;
    for (;;) {
      const int ridx = draft ? k1 + j : j;
      const int w = POOL ? j : 2 * j + (draft ? 1 : 0);  // walk step
      // pooled: a map entry outside the pool names no row (flat row 0 is
      // read, and the row counts as invalid)
      bool no_row = false;
      const uint16_t* row;
      if constexpr (POOL) {
        const int64_t pr = A.map.sidx(b, ridx);
        no_row = pr < 0;
        row = A.map.template row<uint16_t>(no_row ? 0 : pr);
      } else {
        row = A.map.template row<uint16_t>(b * nr + ridx);
      }
      const bool bonus = !draft && j == k;
      if (TID() == 0) {
        if (bonus) grabbed = atomicAdd(&A.queue[0], 1u);
        const HelpView H(A.help, nr);
        st_agent(H.hwg + g, ((uint64_t)tag << 32) | (uint32_t)(w + 1));
        // steps after the first were claimed one row earlier
        Q.hmode = w > 0 ? help_resolve(H.hent + (int64_t)g * nr + w, Q.hprev, tag, H.hpool, &Q.hst)
                        : 0;
      }
      block_sync_lds();
      const bool helped = Q.hmode != 0;
      // count (the prefetched vectors first, when they belong to this row)
      if (!helped) hist_count_stream<PF, D>(hist, row, V, pf, row == pf_row);
      if (bonus && TID() == 0) Q.next = grabbed;
      if (POOL ? j == 0 : ridx == 0) {
        if (TID() < k) {
          Q.tok[TID()] = tok_in;
          Q.uu[TID()] = u_in;
        }
        if (POOL && TID() <= k) Q.st[TID()] = tst_in;
      }
      if (draft && TID() == j) {
        // the two logits of the ratio test, back before the scan ends
        const int32_t x = Q.tok[j];
        if (x >= 0 && (int64_t)x < V) {
          const uint16_t* trow = POOL ? A.map.template at<uint16_t>(b, j)
                                      : A.map.template row<uint16_t>(b * nr + j);
          lt = __builtin_bit_cast(float, (uint32_t)trow[x] << 16);
          ld = __builtin_bit_cast(float, (uint32_t)row[x] << 16);
        }
      }
      block_sync_lds();
      if (bonus) {
        nxt = Q.next;
        have_next = true;
      }
      // prefetch the row most likely next: d_j after t_j, t_{j+1} after d_j
      // (acceptance), the next sequence's t_0 after the bonus row; the
      // walker claims a step of its own sequence before helpers can
      const uint16_t* next_row = nullptr;
      if (POOL) {  // d_{j+1} after d_j
        if (j + 1 < k) next_row = A.map.template at<uint16_t>(b, k1 + j + 1);
      } else if (!draft && j < k) next_row = A.map.template row<uint16_t>(b * nr + k1 + j);
      else if (draft) next_row = A.map.template row<uint16_t>(b * nr + j + 1);
      else if (nxt < (uint32_t)A.B) next_row = A.map.template row<uint16_t>((int64_t)nxt * nr);
      uint64_t claim = 0;
      const bool claim_next = w + 1 < nsteps && !bonus;
      if (claim_next && TID() == 0)
        claim = __hip_atomic_fetch_max(HelpView(A.help, nr).hent + (int64_t)g * nr + w + 1,
                                       (uint64_t)tag << 32, __ATOMIC_RELAXED,
                                       __HIP_MEMORY_SCOPE_AGENT);
      pf_row = next_row;
      if (next_row) prefetch_row(pf, next_row, V);
      RowStat st;
      if (helped) {
        st = Q.hst;
      } else if (hist_row_stats(hist, S, V, A.a, A.top_k, A.top_p, nullptr) == 2) {
        block_sync_lds();
        filter_row_bisect_call<uint16_t, true, NT>(row, V, A.a, A.top_k, A.top_p, &S.res, S.dslot,
                                                    S.uslot);
        __syncthreads();
        st = S.res;
        hist_clear(hist);
      } else {
        st = S.res;
      }
      if (claim_next && TID() == 0) Q.hprev = claim;
      if (no_row) st.valid = 0;
      if (TID() == 0) Q.st[ridx] = st;
      if (!draft) {
        if (j == k) {  // bonus row: every position passed
          valid = st.valid != 0;
          n = k;
          break;
        }
        if (!st.valid && !all_pos) {  // ill-formed position before any stop
          valid = false;
          n = j;
          break;
        }
        draft = true;
        continue;
      }
      // ratio test at position j (thread j holds its token, uniform, logits)
      if (TID() == j) {
        const RowStat st_t = Q.st[j];  // written by thread 0 before a barrier
        const int32_t my_tok = Q.tok[j];
        const float my_u = Q.uu[j];
        const bool formed = st_t.valid && st.valid && my_tok >= 0 && (int64_t)my_tok < V;
        float alpha_out = __builtin_nanf("");
        bool acc = false;
        if (formed) {
          const double p = prob_at(lt, st_t, A.a);
          const double q = prob_at(ld, st, A.a);
          const double alpha = q > 0.0 ? fmin(1.0, p / q) : (p > 0.0 ? 1.0 : 0.0);
          acc = (double)my_u < alpha;
          alpha_out = (float)alpha;
        }
        if (all_pos) A.accept_prob[b * k + j] = alpha_out;
        Q.formed = formed ? 1 : 0;
        Q.accepted = acc ? 1 : 0;
      }
      block_sync_lds();
      const bool formed = Q.formed != 0, acc = Q.accepted != 0;
      if (n < 0 && !(formed && acc)) {
        n = j;
        valid = formed;
      }
      draft = POOL;
      ++j;
      if (POOL && n < 0 && j == k) {  // every position passed: the bonus row's pre-pass figures
        valid = Q.st[k].valid != 0;
        n = k;
        break;
      }
      if (n >= 0 && (!all_pos || j == k)) break;
    }

    if (TID() == 0) {
      st_agent(HelpView(A.help, nr).hwg + g, 0ull);  // no more rows of this sequence to help with
      if (!have_next) grabbed = atomicAdd(&A.queue[0], 1u);
    }
    // correction from the residual of the rows at n, or the bonus draw
    int32_t emitted = -1;
    if (valid) {
      const bool has_q = n < k;
      const uint16_t* prow = POOL ? A.map.template at<uint16_t>(b, n)
                                  : A.map.template row<uint16_t>(b * nr + n);
      const uint16_t* qrow = !has_q ? prow
                             : POOL ? A.map.template at<uint16_t>(b, k1 + n)
                                    : A.map.template row<uint16_t>(b * nr + k1 + n);
      block_sync_lds();  // Q.st written by thread 0
      const RowStat& sp = Q.st[n];
      const RowStat& sq = Q.st[has_q ? k1 + n : n];
      emitted = residual_draw_call(prow, qrow, has_q, sp.m, sp.thr, sp.z, sq.m, sq.thr, sq.z, A.a,
                                   V, A.u[b * k1 + k], Q.csum, &Q.emit);
    }
    int32_t* out = A.out_tokens + b * k1;
    for (int t = TID(); t <= k; t += NT) {
      int32_t v = -1;
      if (valid) {
        if (t < n) v = A.tokens[b * k + t];
        else if (t == n) v = emitted;
      }
      out[t] = v;
    }
    if (TID() == 0) {
      A.accepted_len[b] = valid ? n : -1;
      atomicAdd(&A.queue[2], 1u);  // sequences done
    }
    if (!have_next) {
      if (TID() == 0) Q.next = grabbed;
      block_sync_lds();
      nxt = Q.next;
    }
    cur = nxt;
    block_sync_lds();  // everyone has read Q before the next sequence writes it
  }

  const HelpView H(A.help, nr);
  // The queue is empty: count rows ahead of the other workgroups' walks (the
  // step after the one each walker has claimed, and the one after that) and
  // publish their figures, until every sequence is done.  A helper never
  // waits for anything but the walks' progress, and a walker waits only for
  // a row a helper is already counting, so every wave exits.
  for (;;) {
    if (TID() < kWave) {
      const int lane = TID();
      int found = 0;
      uint32_t c_tag = 0;
      int c_g = 0, c_s = 0;
      uint64_t c_e = 0;
      const uint32_t done = __hip_atomic_load(&A.queue[2], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if (done < (uint32_t)A.B) {
        for (int i = lane; i < (int)gridDim.x && !found; i += kWave) {
          const int gg = (g + 1 + i) % (int)gridDim.x;
          const uint64_t hw = ld_agent(H.hwg + gg);
          const uint32_t t = (uint32_t)(hw >> 32), p = (uint32_t)hw;
          if (t == 0 || p == 0) continue;
          for (int s = (int)p + 1; s <= (int)p + 2 && s < nsteps && !found; ++s) {
            const uint64_t e = ld_agent(H.hent + (int64_t)gg * nr + s);
            if ((uint32_t)(e >> 32) < t) {
              found = 1;
              c_tag = t;
              c_g = gg;
              c_s = s;
              c_e = e;
            }
          }
        }
      }
      const uint64_t any = __ballot(found);
      int state = done >= (uint32_t)A.B ? -1 : 0;  // -1 exit, 0 idle, 1 job
      if (any) {
        const int first = __ffsll((unsigned long long)any) - 1;
        if (lane == first) {
          uint64_t expect = c_e;
          const uint64_t mine = ((uint64_t)c_tag << 32) | (kHelpClaimed << 30);
          if (__hip_atomic_compare_exchange_strong(H.hent + (int64_t)c_g * nr + c_s, &expect, mine,
                                                   __ATOMIC_RELAXED, __ATOMIC_RELAXED,
                                                   __HIP_MEMORY_SCOPE_AGENT)) {
            // a record for the figures, taken once the row is this helper's
            const uint32_t slot = atomicAdd(&A.queue[3], 1u);
            state = 1;
            Q.hjob_g = c_g;
            Q.hjob_s = c_s;
            Q.hjob_slot = (int32_t)(slot < H.hcap ? slot : kHelpNoRecord);
            Q.hjob_tag = c_tag;
          }
          Q.hjob_state = state;
        }
      } else if (lane == 0) {
        Q.hjob_state = state;
      }
      if (!any && state == 0) __builtin_amdgcn_s_sleep(32);
    }
    block_sync_lds();
    const int state = Q.hjob_state;
    if (state < 0) break;
    if (state == 0) {
      block_sync_lds();  // Q.hjob_state is rewritten only after every wave has read it
      continue;
    }
    const int64_t hb = (int64_t)Q.hjob_tag - 1;
    const int ridx = step_slot<POOL>(Q.hjob_s, k);
    bool no_row = false;
    const uint16_t* row;
    if constexpr (POOL) {
      const int64_t pr = A.map.sidx(hb, ridx);
      no_row = pr < 0;
      row = A.map.template row<uint16_t>(no_row ? 0 : pr);
    } else {
      row = A.map.template row<uint16_t>(hb * nr + ridx);
    }
    hist_count_stream<PF, D>(hist, row, V, pf, false);
    block_sync_lds();
    if (hist_row_stats(hist, S, V, A.a, A.top_k, A.top_p, nullptr) == 2) {
      block_sync_lds();
      filter_row_bisect_call<uint16_t, true, NT>(row, V, A.a, A.top_k, A.top_p, &S.res, S.dslot,
                                                  S.uslot);
      __syncthreads();
      hist_clear(hist);
    }
    if (TID() == 0) {
      RowStat st = S.res;
      if (no_row) st.valid = 0;
      const uint32_t slot = (uint32_t)Q.hjob_slot;
      if (slot != kHelpNoRecord) {
        const uint64_t* src = reinterpret_cast<const uint64_t*>(&st);
        uint64_t* dst = reinterpret_cast<uint64_t*>(H.hpool + slot);
        for (int i = 0; i < 4; ++i) st_agent(dst + i, src[i]);
      }
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
      __hip_atomic_fetch_max(H.hent + (int64_t)Q.hjob_g * nr + Q.hjob_s,
                             ((uint64_t)Q.hjob_tag << 32) | (kHelpPublished << 30) | slot,
                             __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    block_sync_lds();  // S and Q.hjob read before the next round rewrites them
  }

  // The last workgroup out leaves the queue, the help entries and the used
  // help records zero for the next call.
  block_sync_lds();  // every wave has left the helping loop
  if (TID() == 0) {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
    const uint32_t out = atomicAdd(&A.queue[1], 1u);
    Q.hmode = out == gridDim.x - 1 ? 1 : 0;
  }
  block_sync_lds();
  if (Q.hmode) {
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
    const uint32_t used = min(__hip_atomic_load(&A.queue[3], __ATOMIC_RELAXED,
                                                __HIP_MEMORY_SCOPE_AGENT), H.hcap);
    const int64_t nent = (int64_t)gridDim.x * nr;
    for (int64_t i = TID(); i < nent; i += NT) H.hent[i] = 0ull;
    for (int i = TID(); i < (int)gridDim.x; i += NT) H.hwg[i] = 0ull;
    uint4* pool4 = reinterpret_cast<uint4*>(H.hpool);
    for (int64_t i = TID(); i < 2 * (int64_t)used; i += NT) pool4[i] = make_uint4(0u, 0u, 0u, 0u);
    block_sync_lds();
    if (TID() < 4) A.queue[TID()] = 0u;
  }
}

// ---------------------------------------------------------------------------
// Stochastic verify for large batches of aligned bf16 rows, scheduled as a
// queue of position tasks.  Task (s, j), j < k, counts target row j and draft
// row j of sequence s and makes the ratio test at j; a rejection ends the
// sequence with the correction drawn from the residual of those two rows, an
// ill-formed position ends it invalid, an acceptance appends task (s, j + 1)
// to the queue.  Task (s, k) counts the bonus row and draws from it.  Tasks
// are taken in queue order (the B position-0 tasks first), so the sequences
// advance position by position across the whole batch and the call does not
// end with a few workgroups walking long sequences alone.  The kernel is
// k_verify_pair_bf16 (sv_window.hpp); the queue's words and helpers are here.
//
// Once workgroups wait for work (the end of a call), a task appends its
// successor (s, j + 1) as soon as its rows are counted, before its own ratio
// test: the successor's rows are then counted while position j is still
// being decided.
// A task commits its outcome only after every earlier position of its
// sequence has passed (the per-sequence word `seqstate`); it is dropped when
// the sequence stopped before it.  So the outputs depend on the rows up to
// the first rejection only, as the rule says, while an idle workgroup may
// read rows past it.
struct TaskArgs {
  RowMap map;
  int64_t V;
  int32_t k, B;
  float a;
  int32_t top_k;
  float top_p;
  const int32_t* tokens;
  const float* u;
  int32_t* accepted_len;
  int32_t* out_tokens;
  // [4]: queue positions taken, workgroups out, then one 64-bit word
  // (tasks appended << 32 | tasks finished); zero on entry, zeroed again by
  // the last workgroup out
  uint32_t* queue;
  // appended tasks in queue order, 1 + s (k + 1) + j each, with kTaskSpec
  // set when appended before position j - 1 was decided (0: not written
  // yet; kTaskExit: no task left): B k + gridDim.x entries.  The B words at
  // seqstate: kSeqStop | the position of the stop once a sequence has
  // stopped, else the number of positions that passed, written by a task
  // that appended its successor early.  Zero on entry and zeroed again by
  // the last workgroup out.
  uint32_t* slots;
  uint32_t* seqstate;
};

constexpr uint32_t kTaskExit = 0xFFFFFFFFu;
constexpr uint32_t kTaskSpec = 0x80000000u;  // task ids stay below 2^31 (B (k + 1) < 2^31)
constexpr uint32_t kSeqStop = 0x80000000u;

__device__ __forceinline__ uint32_t ld_agent32(const uint32_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Slots and sequence words are written with atomic read-modify-writes, like
// the queue counters, so that readers on every XCD observe them where they
// observe the counters (the L2 caches of the XCDs are not coherent with one
// another).
__device__ __forceinline__ void task_publish(uint32_t* p, uint32_t v) {
  (void)__hip_atomic_exchange(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Appends and finishes share one 64-bit counter, so that they are ordered
// with respect to each other: the finish that makes the finished count equal
// to B plus the appends is the last task of the call, since only unfinished
// tasks append.
__device__ __forceinline__ uint64_t* task_af(uint32_t* queue) {
  return reinterpret_cast<uint64_t*>(queue + 2);
}
__device__ __forceinline__ uint32_t task_appended(uint32_t* queue) {
  return (uint32_t)(__hip_atomic_load(task_af(queue), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) >> 32);
}
__device__ __forceinline__ void task_append(uint32_t* queue, uint32_t* slots, uint32_t task) {
  const uint64_t old = __hip_atomic_fetch_add(task_af(queue), 1ull << 32, __ATOMIC_RELAXED,
                                              __HIP_MEMORY_SCOPE_AGENT);
  task_publish(slots + (uint32_t)(old >> 32), task);
}

// The task in queue position i, or 0 while its slot is unwritten: the first
// B positions are the sequences' position-0 tasks; a later one is written
// by the workgroup that took that position among the appends.
__device__ __forceinline__ uint32_t task_peek(uint32_t i, const uint32_t* slots, uint32_t B,
                                              uint32_t k1) {
  return i < B ? 1u + i * k1 : ld_agent32(slots + (i - B));
}

// The task in queue position i, waiting until its slot is written.  Called
// only by a workgroup that holds no unfinished task: every position is then
// filled by an unfinished task's append or, once every task is finished, by
// the exit fill, so the wait ends.
__device__ __forceinline__ uint32_t task_wait(uint32_t i, const uint32_t* slots, uint32_t B,
                                              uint32_t k1) {
  uint32_t v;
  while ((v = task_peek(i, slots, B, k1)) == 0u) __builtin_amdgcn_s_sleep(1);
  return v;
}

// Queue positions are taken with one atomic add each, never by
// compare-and-swap: workgroups that reach this point together (all of them
// at the start of a call) would otherwise retry one round trip each per
// winner.  A position is resolved with task_wait once the taker's own task
// is finished.
constexpr uint32_t kNoClaim = 0xFFFFFFFFu;

// A workgroup takes its next position early (so that the next task's first
// row can be prefetched) only when more than kClaimMargin tasks are queued:
// a position taken before its task is appended would hold that task back for
// the rest of the taker's current task (up to a correction draw) while other
// workgroups sit idle.  Measured at 512 sequences of four positions on 256
// workgroups: 224 queued tasks 4.8 % faster than 64, 192 3.0-4.4 %, 160 and
// 256 1.1-1.5 %, 32 5 % slower.
constexpr uint32_t kClaimMargin = 224;

// ---------------------------------------------------------------------------
// Logits processing: merge (unfiltered) partials or copy (filtered) stats into
// the caller's per-row records; keep a RowStat per row for the dense pass.
__device__ __forceinline__ void write_row_stats(const RowStat& s, spec_row_stats_t* out) {
  spec_row_stats_t o;
  if (s.valid) {
    o.max_logit = s.m;
    o.threshold = s.thr;
    o.log_norm = (float)log(s.z);
    o.valid = 1;
  } else {
    o.max_logit = o.threshold = o.log_norm = __builtin_nanf("");
    o.valid = 0;
  }
  *out = o;
}

// Rows split into many chunks: one wave merges each row's partials.
__global__ __launch_bounds__(256) void k_process_stats_wide(int64_t R, int nchunks, float a,
                                                            Partial* __restrict__ part,
                                                            RowStat* __restrict__ rowstat,
                                                            spec_row_stats_t* __restrict__ out) {
  const int64_t r = (int64_t)blockIdx.x * 4 + threadIdx.x / kWave;
  const int lane = threadIdx.x & (kWave - 1);
  if (r >= R) return;  // whole waves
  const RowStat s = merge_partials_wave(part + r * nchunks, nchunks, a, lane);
  if (lane == 0) {
    rowstat[r] = s;
    if (out) write_row_stats(s, out + r);
  }
}

__global__ __launch_bounds__(256) void k_process_stats(int64_t R, int nchunks, float a,
                                                       Partial* __restrict__ part,
                                                       RowStat* __restrict__ rowstat,
                                                       spec_row_stats_t* __restrict__ out) {
  const int64_t r = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (r >= R) return;
  RowStat s;
  if (part) {
    s = merge_partials(part + r * nchunks, nchunks, a);
    rowstat[r] = s;
  } else {
    s = rowstat[r];
  }
  if (out) write_row_stats(s, out + r);
}

template <typename T, bool VEC, int VPT>
__global__ __launch_bounds__(256) void k_probs(RowMap map, int64_t V, int nchunks, float a,
                                               const RowStat* __restrict__ rowstat,
                                               float* __restrict__ probs) {
  constexpr int NT = 256;
  const int64_t bid = blockIdx.x;
  const int64_t r = bid / nchunks;
  const int c = (int)(bid - r * nchunks);
  const T* row = map.row<T>(r);
  const RowStat s = rowstat[r];
  const float iz = s.valid ? (float)(1.0 / s.z) : __builtin_nanf("");
  const int64_t lo = (int64_t)c * (NT * VPT * 8);
  const int64_t hi = min(V, lo + (int64_t)NT * VPT * 8);
  float* dst = probs + r * V;
#pragma unroll
  for (int v = 0; v < VPT; ++v) {
    const int64_t e = lo + ((int64_t)v * NT + threadIdx.x) * 8;
    if (e < hi) {
      float x[8];
      load8<T, VEC>(row, e, hi, x);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        if (e + i < hi) {
          float p = x[i] >= s.thr ? __builtin_amdgcn_exp2f((x[i] - s.m) * a) * iz : 0.0f;
          if (!s.valid) p = __builtin_nanf("");
          dst[e + i] = p;
        }
      }
    }
  }
}

// Clears `n` 16-byte words of workspace (used where a call's records are not
// consumed by a per-sequence tail that clears them itself).
__global__ __launch_bounds__(256) void k_clear(uint4* __restrict__ p, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = make_uint4(0u, 0u, 0u, 0u);
}

// ---------------------------------------------------------------------------
// Predicted-outcome lookup: one wave per sequence compares its outcome (n,
// emitted token) with its predicted set, 64 entries at a time, and keeps the
// first match; a second pass counts the hits.
__global__ __launch_bounds__(256) void k_outcome_lookup(const int32_t* __restrict__ acc,
                                                        const int32_t* __restrict__ out, int64_t B,
                                                        int k, const int32_t* __restrict__ plen,
                                                        const int32_t* __restrict__ ptok, int P,
                                                        int32_t* __restrict__ hit) {
  const int64_t b = (int64_t)blockIdx.x * 4 + threadIdx.x / kWave;
  const int lane = threadIdx.x & (kWave - 1);
  if (b >= B) return;  // whole waves
  const int32_t n = acc[b];
  int32_t idx = -1;
  if (n >= 0 && n <= k) {
    const int32_t t = out[b * (k + 1) + n];
    const int32_t* pl = plen + b * P;
    const int32_t* pt = ptok + b * P;
    for (int base = 0; base < P; base += kWave) {
      const int i = base + lane;
      const bool m = i < P && pl[i] == n && pt[i] == t;  // empty entries (< 0) never equal n
      const uint64_t hits = __ballot(m);
      if (hits) {
        idx = base + __ffsll((unsigned long long)hits) - 1;
        break;
      }
    }
  }
  if (lane == 0) hit[b] = idx;
}

__global__ __launch_bounds__(1024) void k_count_hits(const int32_t* __restrict__ hit, int64_t B,
                                                     int32_t* __restrict__ count) {
  __shared__ uint32_t slots[1024 / kWave];
  uint32_t c = 0;
  for (int64_t i = threadIdx.x; i < B; i += 1024) c += hit[i] >= 0 ? 1u : 0u;
  const uint32_t total = block_sum<1024>(c, slots);
  if (threadIdx.x == 0) *count = (int32_t)total;
}

// ---------------------------------------------------------------------------
// Logits processors: allow mask (-inf outside it) and repetition penalty (l /
// theta for l > 0, l * theta otherwise, on the penalised tokens), 8 elements
// per thread, 2048 per workgroup; bf16 output rounded to nearest even.
struct ApplyArgs {
  const void* in;
  int64_t in_seq, in_pos;
  void* out;
  int64_t out_seq, out_pos;
  int32_t rows;
  int64_t V;
  int nchunks;
  const uint32_t* allow;
  int64_t a_seq, a_pos;
  const uint32_t* pen;
  int64_t p_seq, p_pos;
  float theta;
};

__device__ __forceinline__ uint32_t bf16_rne(float f) {
  const uint32_t b = __float_as_uint(f);
  if (__builtin_isnan(f)) return 0x7FC0u;
  return (b + 0x7FFFu + ((b >> 16) & 1u)) >> 16;
}

// Four groups of 8 elements per thread, 2,048 elements apart (each load
// instruction of a wave covers 1,024 consecutive elements), all loads in
// flight together.
constexpr int kApplyGroups = 4;
constexpr int64_t kApplyChunk = 256 * kApplyGroups * 8;  // elements per workgroup

template <typename TI, typename TO, bool VEC>
__global__ __launch_bounds__(256) void k_logits_apply(ApplyArgs A) {
  const int64_t blk = blockIdx.x;
  const int64_t r = blk / A.nchunks;
  const int64_t c = blk - r * A.nchunks;
  const int64_t s = r / A.rows, j = r - s * A.rows;
  const int64_t e0 = c * kApplyChunk + (int64_t)threadIdx.x * 8;
  if (e0 >= A.V) return;
  const TI* row = reinterpret_cast<const TI*>(A.in) + s * A.in_seq + j * A.in_pos;
  const uint32_t* am = A.allow ? A.allow + s * A.a_seq + j * A.a_pos : nullptr;
  const uint32_t* pm = A.pen ? A.pen + s * A.p_seq + j * A.p_pos : nullptr;
  Raw8<TI> raw[kApplyGroups];
  uint32_t aw[kApplyGroups], pw[kApplyGroups];
#pragma unroll
  for (int q = 0; q < kApplyGroups; ++q) {
    const int64_t eq = e0 + 2048 * q;
    if (eq < A.V) {
      load8_raw<TI, VEC>(row, eq, A.V, raw[q]);
      // eq is a multiple of 8: its 8 bits lie in one word
      aw[q] = am ? am[eq >> 5] >> (uint32_t)(eq & 31) : 0xFFu;
      pw[q] = pm ? pm[eq >> 5] >> (uint32_t)(eq & 31) : 0u;
    }
  }
#pragma unroll
  for (int q = 0; q < kApplyGroups; ++q) {
    const int64_t eq = e0 + 2048 * q;
    if (eq >= A.V) break;
    float l[8];
    unpack8<TI>(raw[q], l);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      float v = l[i];
      if (!((aw[q] >> i) & 1u)) v = -__builtin_inff();
      else if ((pw[q] >> i) & 1u) v = v > 0.0f ? v / A.theta : v * A.theta;
      l[i] = v;
    }
    const int64_t n = A.V - eq < 8 ? A.V - eq : 8;
    if constexpr (sizeof(TO) == 4) {
      float* o = reinterpret_cast<float*>(A.out) + s * A.out_seq + j * A.out_pos + eq;
      if (VEC && n == 8) {
        *reinterpret_cast<float4*>(o) = make_float4(l[0], l[1], l[2], l[3]);
        *reinterpret_cast<float4*>(o + 4) = make_float4(l[4], l[5], l[6], l[7]);
      } else {
        for (int i = 0; i < n; ++i) o[i] = l[i];
      }
    } else {
      uint16_t* o = reinterpret_cast<uint16_t*>(A.out) + s * A.out_seq + j * A.out_pos + eq;
      uint32_t h[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) h[i] = bf16_rne(l[i]);
      if (VEC && n == 8) {
        *reinterpret_cast<uint4*>(o) = make_uint4(h[0] | (h[1] << 16), h[2] | (h[3] << 16),
                                                  h[4] | (h[5] << 16), h[6] | (h[7] << 16));
      } else {
        for (int i = 0; i < n; ++i) o[i] = (uint16_t)h[i];
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Fused LM head + greedy verify: logits[m][v] = sum_c hidden[m][c] W[v][c]
// (bf16 inputs, fp32 MFMA accumulation) reduced on the fly to each row's
// (largest logit, lowest index) per 256-wide vocabulary tile; the logits
// never reach memory.  Each row's tiles are merged with one 64-bit atomic max
// per (row, tile) into a per-row record that k_greedy_tail reads.
//
// v_mfma_f32_16x16x32_bf16 lane layout (checked on gfx950): lane l holds
// A[l % 16][8 (l / 16) .. +8] and Bt[l % 16][8 (l / 16) .. +8] (B as its
// transpose, here W rows), and C[4 (l / 16) + r][l % 16] for r = 0..3.
typedef __bf16 sv_bf16x8 __attribute__((ext_vector_type(8)));
typedef float sv_f32x4 __attribute__((ext_vector_type(4)));

struct LmHeadArgs {
  const uint16_t* hidden;  // row (b, j) at hidden + b * h_seq + j * h_pos, d elements
  int64_t h_seq, h_pos;
  int32_t k1;              // rows per sequence
  const uint16_t* weight;  // W[v] at weight + v * w_stride, d elements
  int64_t w_stride;
  int64_t M, V;
  int32_t d;
  int32_t n_tiles, m_chunks;
  uint64_t* best;          // [M]: merged (order key, lowest index) of each row, pack_best order
  uint32_t* bad;           // [M]: NaN / +inf seen
};

__device__ __forceinline__ sv_bf16x8 ld_bf16x8(const uint16_t* p) {
  const uint4 v = *reinterpret_cast<const uint4*>(p);
  return __builtin_bit_cast(sv_bf16x8, v);
}

template <int MB, int KU, int NB>
__global__ __launch_bounds__(256) void k_lmhead_argmax(LmHeadArgs A) {
  constexpr int TW = 4 * 16 * NB;  // vocabulary tile: 4 waves x NB column blocks of 16
  constexpr int MR = 16 * MB;  // rows per chunk
  __shared__ uint64_t best_s[4][MR];
  __shared__ uint32_t bad_s[4][MR];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  // XCD-aware order: the workgroups of one XCD take a contiguous range of
  // (tile, chunk) pairs, chunks fastest, so one tile's W is reused from L2
  const int64_t nblk = (int64_t)A.n_tiles * A.m_chunks;
  const int64_t per_xcd = (nblk + 7) / 8;
  const int64_t pidx = (int64_t)(blockIdx.x & 7) * per_xcd + (blockIdx.x >> 3);
  if (pidx >= nblk) return;
  const int64_t tile = pidx / A.m_chunks, chunk = pidx - tile * A.m_chunks;
  const int64_t n0 = tile * TW + (int64_t)w * 16 * NB;  // this wave's columns
  const int64_t m0 = chunk * MR;
  const int r16 = lane & 15, kq = (lane >> 4) * 8;

  // row pointers of this lane's A fragments (rows past M read row 0: their
  // results are discarded) and W fragments (columns past V read row 0)
  const uint16_t* ap[MB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
    int64_t m = m0 + 16 * mb + r16;
    if (m >= A.M) m = 0;
    const int64_t b = m / A.k1, j = m - b * A.k1;
    ap[mb] = A.hidden + b * A.h_seq + j * A.h_pos + kq;
  }
  const uint16_t* bp[NB];
#pragma unroll
  for (int cb = 0; cb < NB; ++cb) {
    int64_t v = n0 + 16 * cb + r16;
    if (v >= A.V) v = 0;
    bp[cb] = A.weight + v * A.w_stride + kq;
  }
  sv_f32x4 acc[MB][NB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int cb = 0; cb < NB; ++cb) acc[mb][cb] = sv_f32x4{0.f, 0.f, 0.f, 0.f};

  // KU steps of 32 per batch: every fragment of a batch is loaded before the
  // first MFMA uses one (steps past d, when d is not a multiple of 32 KU,
  // are zero and add nothing)
  const sv_bf16x8 zero8 = __builtin_bit_cast(sv_bf16x8, make_uint4(0u, 0u, 0u, 0u));
  for (int c = 0; c < A.d; c += 32 * KU) {
    sv_bf16x8 af[KU][MB], bfr[KU][NB];
#pragma unroll
    for (int u = 0; u < KU; ++u) {
      const bool in = c + 32 * u < A.d;
#pragma unroll
      for (int cb = 0; cb < NB; ++cb) bfr[u][cb] = in ? ld_bf16x8(bp[cb] + c + 32 * u) : zero8;
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) af[u][mb] = in ? ld_bf16x8(ap[mb] + c + 32 * u) : zero8;
    }
#pragma unroll
    for (int u = 0; u < KU; ++u)
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int cb = 0; cb < NB; ++cb)
          acc[mb][cb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[u][mb], bfr[u][cb], acc[mb][cb],
                                                                0, 0, 0);
  }

  // epilogue: per row, the best (order key, lowest index) of this lane's
  // columns, then over the 16 lanes that hold the same rows, then the waves
  const int rq = (lane >> 4) * 4;
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      uint64_t best = 0;
      uint32_t bad = 0;
#pragma unroll
      for (int cb = 0; cb < NB; ++cb) {
        const int64_t v = n0 + 16 * cb + r16;
        const float x = acc[mb][cb][r];
        if (v < A.V) {
          if (bad_logit(x)) {
            bad = 1u;
          } else if (x > -__builtin_inff()) {
            const uint64_t cand = pack_best(key_of(x), (int32_t)v);
            best = cand > best ? cand : best;
          }
        }
      }
#pragma unroll
      for (int off = 8; off >= 1; off >>= 1) {  // the 16 lanes holding these rows
        const uint32_t lo = (uint32_t)__shfl_xor((int)(uint32_t)best, off, 16);
        const uint32_t hi = (uint32_t)__shfl_xor((int)(uint32_t)(best >> 32), off, 16);
        const uint64_t o = ((uint64_t)hi << 32) | lo;
        best = o > best ? o : best;
        bad |= (uint32_t)__shfl_xor((int)bad, off, 16);
      }
      if (r16 == 0) {
        best_s[w][16 * mb + rq + r] = best;
        bad_s[w][16 * mb + rq + r] = bad;
      }
    }
  }
  __syncthreads();
  for (int i = threadIdx.x; i < MR; i += 256) {
    const int64_t m = m0 + i;
    if (m >= A.M) continue;
    uint64_t best = 0;
    uint32_t bad = 0;
#pragma unroll
    for (int ww = 0; ww < 4; ++ww) {
      best = best_s[ww][i] > best ? best_s[ww][i] : best;
      bad |= bad_s[ww][i];
    }
    // merged across tiles on the fly: the largest packed word is the largest
    // logit with the lowest index
    if (best) __hip_atomic_fetch_max(A.best + m, best, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (bad) atomicOr(A.bad + m, 1u);
  }
}

// The fused LM head for larger batches, tiled as a matrix product: a
// 256-thread workgroup computes a BM-row x BN-entry tile, the four waves as
// 2 x 2 blocks of (BM / 2) x (BN / 2), each made of 16 x 16 MFMA blocks.
// The hidden and head tiles pass through LDS in stages of BK along d, double
// buffered: the next stage's 16-byte global loads are in flight while the
// current stage's fragments are read from LDS and multiplied, so every
// fragment is loaded from memory once per workgroup instead of once per
// wave.  LDS rows are stored with their 16-byte chunks permuted by row
// (an XOR swizzle), so that the rows a fragment read touches fall on
// different banks.  With one stage in flight per workgroup the kernel is
// bound by memory latency, so it is built for two workgroups per CU (at
// most 80 KiB of LDS and 256 registers per lane each), whose stages overlap.
template <int BM, int BN, int BK, int WGM = 2>
__global__ __launch_bounds__(256, 2) void k_lmhead_gemm_argmax(LmHeadArgs A) {
  constexpr int WGN = 4 / WGM;                  // the four waves as WGM x WGN blocks
  constexpr int WM = BM / WGM, WN = BN / WGN;   // this wave's block
  constexpr int MBk = WM / 16, NBk = WN / 16;   // its MFMA blocks
  static_assert(MBk * 16 * WGM == BM && NBk * 16 * WGN == BN, "whole MFMA blocks per wave");
  // LDS rows of BK bf16, unpadded; the 16-byte chunk c of row r is stored at
  // chunk c ^ f(r), so that the 16-byte accesses of any eight consecutive
  // lanes -- a fragment read's eight rows at one chunk, a stage store's rows
  // and chunks -- fall on the 32 banks without conflict (measured against
  // rows padded by 16 bytes: 5 % faster at 144 and 432 rows)
  constexpr int kRow = BK;
  constexpr int kChunks = BK / 8, kSh = kChunks == 4 ? 1 : 0;
  static_assert(kChunks == 4 || kChunks == 8, "stages of 32 or 64 along d");
  auto swz = [](int r, int c) { return c ^ ((r >> kSh) & (kChunks - 1)); };
  constexpr int TPR = BK / 8;                   // threads per row in the global -> LDS copy
  constexpr int RPP = 256 / TPR;                // rows per pass
  constexpr int NPA = (BM + RPP - 1) / RPP, NPB = BN / RPP;  // passes (the last of A's may be partial)
  static_assert(NPB * RPP == BN, "head tile rows must fill whole passes");
  __shared__ __attribute__((aligned(16))) uint16_t As[2][BM * kRow];
  __shared__ __attribute__((aligned(16))) uint16_t Bs[2][BN * kRow];
  __shared__ uint64_t best_s[WGN][BM];
  __shared__ uint32_t bad_s[WGN][BM];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int wm = w / WGN, wn = w % WGN;
  // XCD-aware order: the workgroups of one XCD take a contiguous range of
  // (tile, chunk) pairs, chunks fastest, so a head tile is reused from L2
  const int64_t nblk = (int64_t)A.n_tiles * A.m_chunks;
  const int64_t per_xcd = (nblk + 7) / 8;
  const int64_t pidx = (int64_t)(blockIdx.x & 7) * per_xcd + (blockIdx.x >> 3);
  if (pidx >= nblk) return;
  const int64_t tile = pidx / A.m_chunks, chunk = pidx - tile * A.m_chunks;
  const int64_t n0 = tile * BN, m0 = chunk * BM;

  // global -> LDS copy: thread t moves 16-byte column (t % TPR) of rows
  // (t / TPR) + RPP i of both tiles (rows past M or V read row 0: their
  // results are discarded)
  const int cc = tid % TPR, r0 = tid / TPR;
  const uint16_t* ag[NPA];
  const uint16_t* bg[NPB];
#pragma unroll
  for (int i = 0; i < NPA; ++i) {
    int64_t m = m0 + r0 + RPP * i;
    if (m >= A.M) m = 0;
    const int64_t b = m / A.k1, j = m - b * A.k1;
    ag[i] = A.hidden + b * A.h_seq + j * A.h_pos + 8 * cc;
  }
#pragma unroll
  for (int i = 0; i < NPB; ++i) {
    int64_t v = n0 + r0 + RPP * i;
    if (v >= A.V) v = 0;
    bg[i] = A.weight + v * A.w_stride + 8 * cc;
  }
  auto load_stage = [&](int c, uint4 (&ra)[NPA], uint4 (&rb)[NPB]) {
    const bool in = c + 8 * cc < A.d;  // d is a multiple of 32: whole 16-byte columns
#pragma unroll
    for (int i = 0; i < NPA; ++i)
      ra[i] = in && r0 + RPP * i < BM ? *reinterpret_cast<const uint4*>(ag[i] + c)
                                      : make_uint4(0u, 0u, 0u, 0u);
#pragma unroll
    for (int i = 0; i < NPB; ++i)
      rb[i] = in ? *reinterpret_cast<const uint4*>(bg[i] + c) : make_uint4(0u, 0u, 0u, 0u);
  };
  auto store_stage = [&](int buf, const uint4 (&ra)[NPA], const uint4 (&rb)[NPB]) {
#pragma unroll
    for (int i = 0; i < NPA; ++i) {
      const int r = r0 + RPP * i;
      if (r < BM) *reinterpret_cast<uint4*>(&As[buf][r * kRow + 8 * swz(r, cc)]) = ra[i];
    }
#pragma unroll
    for (int i = 0; i < NPB; ++i) {
      const int r = r0 + RPP * i;
      *reinterpret_cast<uint4*>(&Bs[buf][r * kRow + 8 * swz(r, cc)]) = rb[i];
    }
  };

  sv_f32x4 acc[MBk][NBk];
#pragma unroll
  for (int mb = 0; mb < MBk; ++mb)
#pragma unroll
    for (int nb = 0; nb < NBk; ++nb) acc[mb][nb] = sv_f32x4{0.f, 0.f, 0.f, 0.f};

  const int r16 = lane & 15, kq = (lane >> 4) * 8;
  uint4 ra[NPA], rb[NPB];
  load_stage(0, ra, rb);
  store_stage(0, ra, rb);
  __syncthreads();
  int buf = 0;
  for (int c = 0; c < A.d; c += BK) {
    const bool more = c + BK < A.d;
    if (more) load_stage(c + BK, ra, rb);  // in flight during this stage's MFMAs
#pragma unroll
    for (int ks = 0; ks < BK; ks += 32) {
      sv_bf16x8 af[MBk], bfr[NBk];
#pragma unroll
      for (int mb = 0; mb < MBk; ++mb) {
        const int r = wm * WM + 16 * mb + r16;
        af[mb] = __builtin_bit_cast(sv_bf16x8, *reinterpret_cast<const uint4*>(
                     &As[buf][r * kRow + 8 * swz(r, (ks + kq) / 8)]));
      }
#pragma unroll
      for (int nb = 0; nb < NBk; ++nb) {
        const int r = wn * WN + 16 * nb + r16;
        bfr[nb] = __builtin_bit_cast(sv_bf16x8, *reinterpret_cast<const uint4*>(
                      &Bs[buf][r * kRow + 8 * swz(r, (ks + kq) / 8)]));
      }
#pragma unroll
      for (int mb = 0; mb < MBk; ++mb)
#pragma unroll
        for (int nb = 0; nb < NBk; ++nb)
          acc[mb][nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[mb], bfr[nb], acc[mb][nb], 0, 0, 0);
    }
    if (more) {
      store_stage(buf ^ 1, ra, rb);  // the other buffer: last read before the previous barrier
      __syncthreads();
      buf ^= 1;
    }
  }

  // epilogue: per row, the best (order key, lowest index) of this lane's
  // columns, over the 16 lanes holding the same rows, then over the WGN
  // waves sharing those rows; one atomic per (row, tile)
  const int rq = (lane >> 4) * 4;
#pragma unroll
  for (int mb = 0; mb < MBk; ++mb) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      uint64_t best = 0;
      uint32_t bad = 0;
#pragma unroll
      for (int nb = 0; nb < NBk; ++nb) {
        const int64_t v = n0 + wn * WN + 16 * nb + r16;
        const float x = acc[mb][nb][r];
        if (v < A.V) {
          if (bad_logit(x)) {
            bad = 1u;
          } else if (x > -__builtin_inff()) {
            const uint64_t cand = pack_best(key_of(x), (int32_t)v);
            best = cand > best ? cand : best;
          }
        }
      }
#pragma unroll
      for (int off = 8; off >= 1; off >>= 1) {
        const uint32_t lo = (uint32_t)__shfl_xor((int)(uint32_t)best, off, 16);
        const uint32_t hi = (uint32_t)__shfl_xor((int)(uint32_t)(best >> 32), off, 16);
        const uint64_t o = ((uint64_t)hi << 32) | lo;
        best = o > best ? o : best;
        bad |= (uint32_t)__shfl_xor((int)bad, off, 16);
      }
      if (r16 == 0) {
        best_s[wn][wm * WM + 16 * mb + rq + r] = best;
        bad_s[wn][wm * WM + 16 * mb + rq + r] = bad;
      }
    }
  }
  __syncthreads();
  for (int i = tid; i < BM; i += 256) {
    const int64_t m = m0 + i;
    if (m < A.M) {
      uint64_t best = best_s[0][i];
      uint32_t bad = bad_s[0][i];
#pragma unroll
      for (int g = 1; g < WGN; ++g) {
        best = best_s[g][i] > best ? best_s[g][i] : best;
        bad |= bad_s[g][i];
      }
      if (best) __hip_atomic_fetch_max(A.best + m, best, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if (bad) atomicOr(A.bad + m, 1u);
    }
  }
}

}  // namespace sv
