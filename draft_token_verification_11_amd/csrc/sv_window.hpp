// sv_window.hpp -- the persistent bf16 row filter at two workgroups per CU,
// each with a 64 KiB histogram of the bf16 codes in an exponent window.
//
// One workgroup per CU with a histogram of every bf16 code (128 KiB of the
// CU's 160 KiB of LDS) leaves HBM idle while a row's histogram is scanned:
// the workgroup streams a row only between scans.  Two 512-thread workgroups
// per CU, each with half that LDS, overlap one workgroup's scan with the
// other's row stream.
//
// The window: bf16 codes whose exponent field lies in [96, 159], i.e.
// |x| in [2^-31, 2^33), both signs -- 16,384 codes, one 32-bit counter each
// (64 KiB, increments of 1, no overflow).  For a code c, y = c + 0x1000
// (mod 2^16) has bits 14..13 equal to 10 exactly for the window's codes, and
// its counter is (y & 0x1FFF) | (sign << 13).  Every other code is counted on
// the side: +-0, -inf, NaN or +inf (the row is invalid), finite values of
// magnitude below 2^-31 (tiny) or at least 2^33 (huge).  Zeros and tiny values
// sit between the window's negative and positive codes in value order and are
// scanned as one entry of value 0; a decision (the max, the top-k threshold,
// the top-p cut) that lands on that entry while tiny values exist, huge values
// anywhere, or tiny values at a temperature so low that their exponentials
// would differ from 2^(-m a) send the row to the exact bisection path.
#pragma once

#include "sv_kernels.hpp"

namespace sv {

constexpr int kWinThreads = 512;
constexpr int kWinWords = 16384;   // counters (64 KiB)
constexpr int kWinGroups = 256;    // 64 counters (keys) each
constexpr uint32_t kWinAdd = 0x10001000u;  // added to both codes of a 32-bit word

enum : int { kSideZero = 0, kSideNegInf, kSideBad, kSideTinyNeg, kSideTinyPos, kSideHuge, kSides };

// List entries of the scan: key-ordered window groups 0..255 (group kg holds
// the 64 keys from win_key(kg, 0)), the zero entry and the -inf entry.
constexpr uint16_t kEntZero = 0x100, kEntNegInf = 0x101;
constexpr int kWinListMax = kWinGroups + 2;

struct WinScratch {
  uint16_t list[kWinListMax];  // non-empty entries in descending key order
  uint32_t lcnt[kWinListMax];  // count of entry i
  float gmass[kWinListMax];    // mass of entry i (first kTop entries)
  uint32_t side[8];            // side counters (kSides used)
  uint32_t wcount[16];
  double dslot[16];
  uint32_t uslot[16];
  uint32_t tk, tk_entry, fallback, nl;
  float m;      // the row's max logit, between the two parts of the scan
  float top_p;  // the call's top_p, set once by the kernel: read from LDS at the cut
  RowStat res;
};

// Order key (16-bit, ascending with the value) of key-ordered group kg, lane j.
__device__ __forceinline__ uint32_t win_key(uint32_t kg, uint32_t j) {
  return (kg < 128u ? 0x3000u + 64u * kg : 0xB000u + 64u * (kg - 128u)) + j;
}
// Counter of a window key.
__device__ __forceinline__ uint32_t win_idx(uint32_t key) {
  return key >= 0x8000u ? key - 0xB000u : 0x2000u + (0x4FFFu - key);
}
// Key of list entry `ent`, lane j (the zero and -inf entries use lane 0 only).
__device__ __forceinline__ uint32_t win_ent_key(uint32_t ent, uint32_t j) {
  if (ent < (uint32_t)kWinGroups) return win_key(ent, j);
  return ent == kEntZero ? kKey16PosZero : kKey16NegInf;
}

template <int NT>
__device__ __forceinline__ void win_clear(uint32_t* hist, uint32_t* side) {
  uint4* h4 = reinterpret_cast<uint4*>(hist);
  for (int i = opaque_tid(); i < kWinWords / 4; i += NT) h4[i] = make_uint4(0u, 0u, 0u, 0u);
  if (opaque_tid() < 8) side[opaque_tid()] = 0u;
}

// Zeroes the groups on S's list and the side counters (threads 0..NT-1 of
// those calling, index t).
template <int NT>
__device__ __forceinline__ void win_clear_listed(uint32_t* hist, WinScratch& S, int t);

__device__ __forceinline__ void win_inc(uint32_t* hist, uint32_t byte_off) {
  atomicAdd(reinterpret_cast<uint32_t*>(reinterpret_cast<char*>(hist) + byte_off), 1u);
}

// One code of any kind.
__device__ __forceinline__ void win_add1(uint32_t* hist, uint32_t* side, uint32_t c) {
  const uint32_t y = (c + 0x1000u) & 0xFFFFu;
  if ((y & 0x6000u) == 0x4000u) {
    win_inc(hist, ((y & 0x1FFFu) << 2) | (y & 0x8000u));
    return;
  }
  const uint32_t mag = c & 0x7FFFu;
  int cls;
  if (mag == 0u) cls = kSideZero;
  else if (c == 0xFF80u) cls = kSideNegInf;
  else if (mag >= 0x7F80u) cls = kSideBad;  // +inf, NaN
  else if (mag < 0x3000u) cls = (c & 0x8000u) ? kSideTinyNeg : kSideTinyPos;
  else cls = kSideHuge;
  atomicAdd(&side[cls], 1u);
}

// Eight codes of a 16-byte vector: when all lie in the window (the common
// case) one add per word gives both counters' offsets; otherwise each code
// goes through win_add1.  A carry out of a word's low half happens only for a
// low code outside the window, which sends the vector the general way.
__device__ __forceinline__ void win_add8(uint32_t* hist, uint32_t* side, uint4 v) {
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
  uint32_t y[4], bad = 0u;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    y[i] = w[i] + kWinAdd;
    bad |= (y[i] & 0x60006000u) ^ 0x40004000u;
  }
  if (bad == 0u) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      win_inc(hist, ((y[i] & 0x1FFFu) << 2) | (y[i] & 0x8000u));
      win_inc(hist, ((y[i] >> 14) & 0x7FFCu) | ((y[i] >> 16) & 0x8000u));
    }
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      win_add1(hist, side, w[i] & 0xFFFFu);
      win_add1(hist, side, w[i] >> 16);
    }
  }
}

// Streams one aligned bf16 row into the (cleared) window histogram, D 16-byte
// loads in flight per thread; the first PF vectors of each thread come from
// `pf` when pf_ok (prefetched during the previous row's scan).
template <int PF, int D, int NTH>
__device__ __forceinline__ void win_count_stream(uint32_t* hist, uint32_t* side, const uint16_t* row,
                                                 int64_t V, const uint4 (&pf)[PF], bool pf_ok) {
  constexpr uint32_t NT = NTH;
  uint32_t tid = threadIdx.x;
  asm volatile("" : "+v"(tid));
  const uint32_t nfull = (uint32_t)(V / 8);
  const uint32_t ngroups = (uint32_t)((V + 7) / 8);
  const __amdgpu_buffer_rsrc_t rs = row_rsrc(row, V);
  uint32_t g = tid;
  if (pf_ok) {
#pragma unroll
    for (int j = 0; j < PF; ++j) {
      const uint32_t gj = tid + (uint32_t)j * NT;
      if (gj < nfull) {
        win_add8(hist, side, pf[j]);
      } else {
        for (uint32_t i = 0; i < 8 && (int64_t)gj * 8 + i < V; ++i) win_add1(hist, side, row[gj * 8 + i]);
      }
    }
    g = tid + (uint32_t)PF * NT;
  }
  for (; g + (D - 1) * NT < nfull; g += D * NT) {
    uint4 v[D];
#pragma unroll
    for (int d = 0; d < D; ++d) v[d] = rsrc_load16(rs, g * 16u, (uint32_t)d * NT * 16u);
#pragma unroll
    for (int d = 0; d < D; ++d) win_add8(hist, side, v[d]);
  }
  // fewer than D full vectors per thread remain: two or more are loaded
  // together, a single one and the partial group one at a time
  if (g + NT < nfull) {
    uint4 v[D - 1];
#pragma unroll
    for (int d = 0; d < D - 1; ++d) {
      const uint32_t gd = g + (uint32_t)d * NT;
      v[d] = gd < nfull ? rsrc_load16(rs, gd * 16u, 0u) : make_uint4(0u, 0u, 0u, 0u);
    }
#pragma unroll
    for (int d = 0; d < D - 1; ++d)
      if (g + (uint32_t)d * NT < nfull) win_add8(hist, side, v[d]);
    g += (nfull - g + NT - 1) / NT * NT;
  }
  for (; g < ngroups; g += NT) {
    if (g < nfull) {
      win_add8(hist, side, rsrc_load16(rs, g * 16u, 0u));
    } else {
      for (uint32_t i = 0; i < 8 && (int64_t)g * 8 + i < V; ++i) win_add1(hist, side, row[g * 8 + i]);
    }
  }
}

template <int PF, int NT>
__device__ __forceinline__ void win_prefetch_row(uint4 (&pf)[PF], const uint16_t* row, int64_t V) {
  const uint32_t nfull = (uint32_t)(V / 8);
  const __amdgpu_buffer_rsrc_t rs = row_rsrc(row, V);
  uint32_t tid = threadIdx.x;
  asm volatile("" : "+v"(tid));
#pragma unroll
  for (int j = 0; j < PF; ++j) {
    const uint32_t g = tid + (uint32_t)j * NT;
    if (g < nfull) pf[j] = rsrc_load16(rs, tid * 16u, (uint32_t)j * NT * 16u);
  }
}

template <int NT>
__device__ __forceinline__ void win_clear_listed(uint32_t* hist, WinScratch& S, int t) {
  uint4* h4 = reinterpret_cast<uint4*>(hist);
  const uint32_t nl = S.nl;
  for (uint32_t i = (uint32_t)t >> 4; i < nl; i += NT / 16) {
    const uint32_t e = S.list[i];
    if (e < (uint32_t)kWinGroups) {
      const uint32_t sg = e >= 128u ? e - 128u : 255u - e;
      h4[sg * 16u + ((uint32_t)t & 15u)] = make_uint4(0u, 0u, 0u, 0u);
    }
  }
  if (t < 8) S.side[t] = 0u;
}

// Row statistics from a filled window histogram (S.top_p must hold top_p),
// every thread of the NT-thread workgroup, in two parts.  win_stats_list
// builds the list of non-empty entries and finds the max and the top-k key;
// win_stats_mass then computes the masses, the normaliser and the top-p
// cut.  Between the two, the row's figures live in S.  Results: 0 success
// (RowStat in S.res and, if given, *out), 1 invalid row (written), 2 the row
// needs the exact bisection path (nothing written; the histogram is left as
// it is for the caller to clear).  The histogram and side counters are left
// zero after 0 or 1.
template <int NT>
__device__ __forceinline__ int win_stats_list(uint32_t* hist, WinScratch& S, int64_t V, float a,
                                              int top_k, RowStat* out) {
  static_assert(NT == 512 || NT == 1024, "two or four threads per key group");
  constexpr int NW = NT / kWave;
  int tid = threadIdx.x;
  asm volatile("" : "+v"(tid));
  const int lane = tid & (kWave - 1);
  const int wv = tid / kWave;
  const bool use_k = top_k > 0 && (int64_t)top_k < V;
  const uint32_t s_zero = S.side[kSideZero], s_ninf = S.side[kSideNegInf];
  const uint32_t s_bad = S.side[kSideBad], s_huge = S.side[kSideHuge];
  const uint32_t s_tneg = S.side[kSideTinyNeg], s_tpos = S.side[kSideTinyPos];
  const uint32_t tiny = s_tneg + s_tpos;
  const uint32_t zcnt = s_zero + tiny;  // the zero entry: zeros and tiny values
  const uint32_t nz = zcnt != 0u ? 1u : 0u;
  auto gsum = [&](uint32_t kg, uint32_t first, uint32_t R, uint32_t rot) -> uint32_t {
    // R of the 16 16-byte words of key-ordered group kg, from `first`, rotated
    const uint32_t sg = kg >= 128u ? kg - 128u : 255u - kg;
    const uint4* h4 = reinterpret_cast<const uint4*>(hist) + sg * 16u + first;
    uint32_t c = 0;
#pragma unroll
    for (uint32_t j = 0; j < R; ++j) {
      const uint4 w = h4[(j + rot) % R];
      c += w.x + w.y + w.z + w.w;
    }
    return c;
  };

  // The list of non-empty entries in descending key order: positive window
  // groups (kg 255..128), the zero entry, negative groups (127..0), -inf.
  uint32_t npos = 0, nwin = 0;
  {
    // the TPG threads of key-ordered group kg = 255 - tid/TPG take a share
    // each, met by lane swaps; the first half of the waves holds the positive
    // groups (descending), the second half the negative ones
    constexpr uint32_t TPG = NT / kWinGroups;
    const uint32_t gi = (uint32_t)tid / TPG;
    uint32_t cnt = gsum(255u - gi, ((uint32_t)tid % TPG) * (16u / TPG), 16u / TPG, gi);
    cnt += (uint32_t)__builtin_amdgcn_mov_dpp((int)cnt, 0xB1, 0xF, 0xF, false);  // quad_perm 1,0,3,2
    if (TPG == 4)
      cnt += (uint32_t)__builtin_amdgcn_mov_dpp((int)cnt, 0x4E, 0xF, 0xF, false);  // quad_perm 2,3,0,1
    const bool own = (uint32_t)tid % TPG == 0u && cnt != 0;
    const uint64_t ball = __ballot(own);
    if (lane == 0) S.wcount[wv] = (uint32_t)__popcll(ball);
    block_sync_lds();
    uint32_t off = 0;
#pragma unroll
    for (int v = 0; v < NW; ++v) {
      const uint32_t c = S.wcount[v];
      if (v < wv) off += c;
      if (v < NW / 2) npos += c;
      nwin += c;
    }
    if (own) {
      const uint32_t pos =
          off + (wv >= NW / 2 ? nz : 0u) + (uint32_t)__popcll(ball & ((1ull << lane) - 1ull));
      S.list[pos] = (uint16_t)(255u - gi);
      S.lcnt[pos] = cnt;
    }
  }
  const uint32_t nl = nwin + nz + (s_ninf ? 1u : 0u);
  if (tid == 0) {
    if (nz) {
      S.list[npos] = kEntZero;
      S.lcnt[npos] = zcnt;
    }
    if (s_ninf) {
      S.list[nwin + nz] = kEntNegInf;
      S.lcnt[nwin + nz] = s_ninf;
    }
    S.nl = nl;
    S.fallback = 0u;
  }
  block_sync_lds();

  auto kcount = [&](uint32_t ent, uint32_t j) -> uint32_t {
    if (ent < (uint32_t)kWinGroups) return hist[win_idx(win_key(ent, j))];
    if (j != 0u) return 0u;
    return ent == kEntZero ? zcnt : s_ninf;
  };
  // NaN/+inf, or no finite logit (finite values outside the window count)
  if (s_bad || ((nl == 0u || S.list[0] == kEntNegInf) && s_huge == 0u)) {
    if (tid == 0) {
      RowStat st = {__builtin_nanf(""), __builtin_nanf(""), 0.0, 0, {0, 0, 0}};
      S.res = st;
      if (out) *out = st;
    }
    block_sync_lds();
    win_clear_listed<NT>(hist, S, tid);
    return 1;
  }
  // huge finite values, or tiny ones whose exponentials at this temperature
  // would not all equal 2^(-m a): the exact path
  if (s_huge || (tiny && a > 16.0f)) return 2;
  const uint32_t e0 = S.list[0];
  uint32_t max_key;
  if (e0 == kEntZero) {
    if (s_tpos || !s_zero) return 2;  // the max is a tiny value
    max_key = kKey16PosZero;
  } else {
    const uint64_t nzm = __ballot(kcount(e0, (uint32_t)lane) != 0u);
    max_key = win_key(e0, 63u - (uint32_t)__clzll((long long)nzm));
  }

  // Wave 0 (or the one wave): the max, and with top-k the top-k key by exact counts.
  if (wv == 0 && lane == 0) {
    S.m = value_of_key16(max_key);
    S.tk = 0;
    S.tk_entry = nl - 1;
  }
  if (use_k && wv == 0) {
    uint32_t carry = 0;
    for (uint32_t base = 0; base < nl; base += kWave) {
      const uint32_t x = (base + lane < nl) ? S.lcnt[base + lane] : 0u;
      const uint32_t inc = wave_incl_scan(x) + carry;
      const uint64_t hit = __ballot(base + lane < nl && inc >= (uint32_t)top_k);
      if (hit) {
        const int L = __ffsll((unsigned long long)hit) - 1;
        const uint32_t before = bcast(inc - x, L);
        const uint32_t ek = S.list[base + L];
        const uint32_t c = kcount(ek, (uint32_t)lane);
        const uint32_t suf = wave_incl_suffix(c) + before;
        const uint64_t ok = __ballot(suf >= (uint32_t)top_k);
        if (lane == 0) {
          S.tk = win_ent_key(ek, 63u - (uint32_t)__clzll((long long)ok));
          S.tk_entry = base + L;
          if (ek == kEntZero && tiny) S.fallback = 1u;
        }
        break;
      }
      carry = bcast(inc, kWave - 1);
    }
  }
  block_sync_lds();
  return S.fallback ? 2 : 0;
}

// The second part (every thread of the NT-thread workgroup), after
// win_stats_list returned 0 for this histogram and S.
template <int NT>
__device__ __forceinline__ int win_stats_mass(uint32_t* hist, WinScratch& S, int64_t V, float a,
                                              int top_k, float top_p, RowStat* out) {
  constexpr int NW = NT / kWave;
  int tid = threadIdx.x;
  asm volatile("" : "+v"(tid));
  const int lane = tid & (kWave - 1);
  const int wv = tid / kWave;
  const bool use_k = top_k > 0 && (int64_t)top_k < V;
  const bool use_p = top_p < 1.0f;
  const uint32_t zcnt = S.side[kSideZero] + S.side[kSideTinyNeg] + S.side[kSideTinyPos];
  const uint32_t tiny = S.side[kSideTinyNeg] + S.side[kSideTinyPos];
  const uint32_t s_ninf = S.side[kSideNegInf];
  const float m = S.m;
  const uint32_t tk = S.tk;
  const uint32_t last = S.tk_entry;
  auto kcount = [&](uint32_t ent, uint32_t j) -> uint32_t {
    if (ent < (uint32_t)kWinGroups) return hist[win_idx(win_key(ent, j))];
    if (j != 0u) return 0u;
    return ent == kEntZero ? zcnt : s_ninf;
  };

  // Masses over keys >= tk, one wave per entry; the first kTop entries keep
  // their totals for the cut.
  constexpr uint32_t kTop = 32;
  auto emass = [&](uint32_t ent, uint32_t j) -> float {
    const uint32_t key = win_ent_key(ent, j);
    return key >= tk ? key_mass(key, kcount(ent, j), m, a) : 0.0f;
  };
  float acc = 0.0f;
  for (uint32_t i = (uint32_t)wv; i <= last; i += NW) {
    const float e = emass(S.list[i], (uint32_t)lane);
    acc += e;
    if (i < kTop) {
      const float gs = wave_sum(e);
      if (lane == 0) S.gmass[i] = gs;
    }
  }
  {
    const double ws = wave_sum((double)acc);
    if (lane == 0) S.dslot[wv] = ws;
  }
  block_sync_lds();

  // Wave 0: the normaliser, then the top-p cut by cumulative mass from the top.
  if (wv == 0) {
    double zk = 0.0;
#pragma unroll
    for (int v = 0; v < NW; ++v) zk += S.dslot[v];
    uint32_t thr_key = tk;
    double z = zk;
    bool fb = false;
    if (use_p) {
      // top_p comes from LDS here: a register copy held across the scan
      // would be spilled, and its reload would wait for the loads in flight
      const double target = (double)S.top_p * zk;
      double carry = 0.0;
      for (uint32_t base = 0; base <= last; base += kWave) {
        const bool in = base + lane <= last;
        double x = 0.0;
        if (base < kTop) x = (in && base + lane < kTop) ? (double)S.gmass[base + lane] : 0.0;
        const double inc = wave_incl_scan(x) + carry;
        uint64_t hit = __ballot(in && base + lane < kTop && inc >= target);
        int L = hit ? __ffsll((unsigned long long)hit) - 1 : -1;
        double before = L >= 0 ? bcast(inc - x, L) : 0.0;
        if (L < 0 && base + kWave >= kTop) {
          double run = bcast(inc, kWave - 1);
          for (uint32_t i = max(base, kTop); i <= last; ++i) {
            const double gm = wave_sum((double)emass(S.list[i], (uint32_t)lane));
            if (run + gm >= target || i == last) {
              L = (int)(i - base);
              before = run;
              break;
            }
            run += gm;
          }
        }
        if (L >= 0 || base + kWave > last) {
          if (L < 0) {  // rounding corner: the last entry
            L = (int)(last - base);
            before = bcast(inc - x, L);
          }
          const uint32_t ec = S.list[base + L];
          const double e = (double)emass(ec, (uint32_t)lane);
          const double suf = wave_incl_suffix(e) + before;
          const uint64_t ok = __ballot(suf >= target);
          int pick;
          if (ok) {
            pick = 63 - __clzll((long long)ok);
          } else {  // rounding corner: the lowest key with mass in the entry
            const uint64_t nzm = __ballot(e > 0.0);
            pick = nzm ? __ffsll((unsigned long long)nzm) - 1 : 0;
          }
          thr_key = max(tk, win_ent_key(ec, (uint32_t)pick));
          z = bcast(suf, pick);
          fb = ec == kEntZero && tiny != 0u;
          break;
        }
        carry = bcast(inc, kWave - 1);
      }
    }
    if (lane == 0) {
      RowStat st;
      st.m = m;
      st.thr = (use_k || use_p) ? value_of_key16(thr_key) : -__builtin_inff();
      st.z = z;
      st.valid = 1;
      st.pad[0] = st.pad[1] = st.pad[2] = 0;
      S.fallback = fb ? 1u : 0u;
      if (!fb) {
        S.res = st;
        if (out) *out = st;
      }
    }
  }
  block_sync_lds();
  if (S.fallback) return 2;
  win_clear_listed<NT>(hist, S, tid);
  return 0;
}

// Both parts, every thread of the NT-thread workgroup.
template <int NT>
__device__ __forceinline__ int win_row_stats(uint32_t* hist, WinScratch& S, int64_t V, float a,
                                             int top_k, float top_p, RowStat* out) {
  const int r = win_stats_list<NT>(hist, S, V, a, top_k, out);
  return r != 0 ? r : win_stats_mass<NT>(hist, S, V, a, top_k, top_p, out);
}

// ---------------------------------------------------------------------------
// Persistent bf16 filter at two 512-thread workgroups per CU: each workgroup
// walks its rows (XCD-aware: the workgroups of XCD x take the rows of one
// contiguous range) and prefetches the next row's first vectors while it
// scans; the other workgroup on the CU streams its own row meanwhile, so the
// CU's HBM stream does not stop for a scan.
template <int PF, int D>
__global__ __launch_bounds__(kWinThreads) __attribute__((amdgpu_waves_per_eu(4, 4)))
void k_filter_win_persistent(FilterArgs F) {
  __shared__ uint32_t hist[kWinWords];
  __shared__ WinScratch S;
  const int nwg = gridDim.x;
  const int xcd = blockIdx.x & 7, slot = blockIdx.x >> 3;
  const int per_xcd = nwg >> 3;  // nwg is a multiple of 8
  const int64_t rx = (F.R + 7) / 8;
  const int64_t r_lo = (int64_t)xcd * rx, r_hi = min(F.R, r_lo + rx);
  const int64_t V = F.V;

  uint4 pf[PF];
  int64_t r = r_lo + slot;
  if (threadIdx.x == 0) S.top_p = F.top_p;
  if (r < r_hi) win_prefetch_row<PF, kWinThreads>(pf, F.map.template row<uint16_t>(r), V);
  win_clear<kWinThreads>(hist, S.side);  // afterwards each row's scan leaves the histogram zero
  for (; r < r_hi; r += per_xcd) {
    const uint16_t* row = F.map.template row<uint16_t>(r);
    block_sync_lds();
    win_count_stream<PF, D, kWinThreads>(hist, S.side, row, V, pf, true);
    block_sync_lds();
    if (r + per_xcd < r_hi) win_prefetch_row<PF, kWinThreads>(pf, F.map.template row<uint16_t>(r + per_xcd), V);
    if (win_row_stats<kWinThreads>(hist, S, V, F.a, F.top_k, F.top_p, F.stats + r) == 2) {
      block_sync_lds();
      filter_row_bisect_call<uint16_t, true, kWinThreads>(row, V, F.a, F.top_k, F.top_p,
                                                           F.stats + r, S.dslot, S.uslot);
      __syncthreads();
      win_clear<kWinThreads>(hist, S.side);
    }
  }
}

}  // namespace sv
