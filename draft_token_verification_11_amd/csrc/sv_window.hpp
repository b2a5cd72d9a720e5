// sv_window.hpp -- exact bf16 row statistics from 64 KiB histograms of the
// bf16 codes in an exponent window: the persistent row filter at two
// workgroups per CU, and the position-task verify that counts a position's
// target and draft rows at once into two such histograms.
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
  float gmass[kWinListMax];    // mass of entry i
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

// Mass of key `lane` of list entry `ent` relative to the max m:
// count * 2^((v - m) a) for keys >= tk, else 0 (the zero entry's count is
// zcnt, the -inf entry's mass 0).  The entry is the same in the whole wave,
// so it is moved to a scalar register and its kind is a scalar branch; the
// mass needs no branch (every key with a count lies at or below m, so
// clamping the exponent at 0 changes none of them and keeps the empty keys
// above m finite).
__device__ __forceinline__ float win_entry_mass(const uint32_t* hist, uint32_t ent, uint32_t lane,
                                                float m, float a, uint32_t tk, uint32_t zcnt) {
  ent = (uint32_t)__builtin_amdgcn_readfirstlane((int)ent);
  uint32_t key, c;
  if (ent < (uint32_t)kWinGroups) {
    key = win_key(ent, lane);
    c = hist[win_idx(key)];
  } else if (ent == kEntZero) {
    key = kKey16PosZero;
    c = lane == 0u ? zcnt : 0u;
  } else {  // -inf
    return 0.0f;
  }
  const float x = fminf((value_of_key16(key) - m) * a, 0.0f);
  const float e = (float)c * __builtin_amdgcn_exp2f(x);
  return key >= tk ? e : 0.0f;
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
// Thread `tid` of the NTH counting threads.
template <int PF, int D, int NTH>
__device__ __forceinline__ void win_count_stream(uint32_t* hist, uint32_t* side, const uint16_t* row,
                                                 int64_t V, const uint4 (&pf)[PF], bool pf_ok,
                                                 uint32_t tid) {
  constexpr uint32_t NT = NTH;
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
__device__ __forceinline__ void win_prefetch_row(uint4 (&pf)[PF], const uint16_t* row, int64_t V,
                                                 uint32_t tid) {
  const uint32_t nfull = (uint32_t)(V / 8);
  const __amdgpu_buffer_rsrc_t rs = row_rsrc(row, V);
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

// Masses, normaliser and top-p cut of a window histogram whose list is set,
// given the row's max m, top-k key tk and last entry at or above it; NT
// threads, index t; does
// its work only when `active` (the same value in all NT threads) but passes
// its two barriers either way.  The entries' masses are formed entry-major
// (an octet of lanes per entry, eight keys per lane, octet_mass); one wave
// then runs the fp64 prefix over the entries in list order, 64 at a time
// with every chunk's scan issued together: its total is the normaliser, and
// the top-p cut lies in the first entry where it reaches top_p times that.  Wave `lead` does that
// part.  Sets S.res, or S.fallback when the cut lands on the zero entry while
// tiny values exist.
template <int NT>
__device__ __forceinline__ void win_mass_cut(const uint32_t* hist, WinScratch& S, int t, float a,
                                             bool use_k, bool use_p, uint32_t zcnt, uint32_t tiny,
                                             bool active, float m, uint32_t tk, uint32_t last,
                                             int lead = 0) {
  const int lane = t & (kWave - 1), wv = t / kWave;
  if (active) {
    const uint32_t sub = (uint32_t)t & 7u;
    const float vtk = value_of_key16(tk);
    for (uint32_t base = 0; base <= last; base += NT / 8) {
      const uint32_t e = base + (uint32_t)t / 8u;
      float x[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
      if (e <= last) {
        const uint32_t ent = S.list[e];
        // the lane's eight keys in counter order, which is magnitude order
        // for both signs: counter i0 + j holds the bf16 code rb + j
        uint4 lo = make_uint4(0u, 0u, 0u, 0u), hi = lo;
        uint32_t rb = 0;
        if (ent < (uint32_t)kWinGroups) {
          const uint32_t k0 = win_key(ent, 8u * sub);  // keys k0 .. k0 + 7
          const bool pos = k0 >= 0x8000u;
          const uint32_t i0 = win_idx(pos ? k0 : k0 + 7u);
          rb = pos ? k0 - 0x8000u : 0xFFFFu - (k0 + 7u);
          const uint4* h4 = reinterpret_cast<const uint4*>(hist + i0);
          lo = h4[0];
          hi = h4[1];
        } else if (ent == kEntZero && sub == 0u) {
          lo.x = zcnt;  // +0 (code 0) stands for the zeros and tiny values
        }
        const uint32_t c[8] = {lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
        x_masses8(x, c, rb, m, a, use_k, vtk);
      }
      const float gm = octet_mass(x);
      if (e <= last && sub == 4u) S.gmass[e] = gm;
    }
  }
  block_sync_lds();

  if (active && wv == lead) {
    auto emass = [&](uint32_t ent, uint32_t j) -> float {
      return win_entry_mass(hist, ent, j, m, a, tk, zcnt);
    };
    // the prefix over the entries, all its chunks at once
    constexpr int kC = (kWinListMax + kWave - 1) / kWave;
    double inc[kC];
    double run = 0.0;
#pragma unroll
    for (int c = 0; c < kC; ++c) {
      inc[c] = 0.0;
      if ((uint32_t)(c * kWave) <= last) {
        const uint32_t i = (uint32_t)(c * kWave + lane);
        inc[c] = wave_incl_scan(i <= last ? (double)S.gmass[i] : 0.0);
      }
    }
#pragma unroll
    for (int c = 0; c < kC; ++c) {
      if ((uint32_t)(c * kWave) <= last) {
        inc[c] += run;
        run = bcast(inc[c], kWave - 1);
      }
    }
    const double zk = run;
    uint32_t thr_key = tk;
    double z = zk;
    bool fb = false;
    if (use_p) {
      // the first entry whose running sum reaches top_p times the
      // normaliser (the last entry if rounding leaves none), then inside it
      // the lowest key from which the keys above still reach it
      const double target = (double)S.top_p * zk;
      int cc = -1, L = 0;
#pragma unroll
      for (int c = 0; c < kC; ++c) {
        if (cc < 0 && (uint32_t)(c * kWave) <= last) {
          const uint64_t hit = __ballot((uint32_t)(c * kWave + lane) <= last && inc[c] >= target);
          if (hit) {
            cc = c;
            L = __ffsll((unsigned long long)hit) - 1;
          }
        }
      }
      if (cc < 0) {
        cc = (int)(last / kWave);
        L = (int)(last % kWave);
      }
      double incc = inc[0];
#pragma unroll
      for (int c = 1; c < kC; ++c)
        if (c == cc) incc = inc[c];
      const uint32_t eL = (uint32_t)(cc * kWave + L);
      const double before = bcast(incc, L) - (double)S.gmass[eL];
      const uint32_t ec = S.list[eL];
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
    }
    if (lane == 0) {
      S.fallback = fb ? 1u : 0u;
      if (!fb)
        S.res = RowStat{m, (use_k || use_p) ? value_of_key16(thr_key) : -__builtin_inff(), z, 1,
                        {0, 0, 0}};
    }
  }
  block_sync_lds();
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
  int tid = threadIdx.x;
  asm volatile("" : "+v"(tid));
  const bool use_k = top_k > 0 && (int64_t)top_k < V;
  const bool use_p = top_p < 1.0f;
  const uint32_t zcnt = S.side[kSideZero] + S.side[kSideTinyNeg] + S.side[kSideTinyPos];
  const uint32_t tiny = S.side[kSideTinyNeg] + S.side[kSideTinyPos];
  win_mass_cut<NT>(hist, S, tid, a, use_k, use_p, zcnt, tiny, true, S.m, S.tk, S.tk_entry);
  if (S.fallback) return 2;
  if (out && tid == 0) *out = S.res;
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

// Two rows at once: threads 0..511 of a 1024-thread workgroup scan one
// histogram (with its own S), threads 512..1023 the other, t = the thread's
// index within its half.  Wave `lead` of the half makes its one-wave steps
// (the max, the top-k key, the prefix and the cut): with lead 0 for one half
// and 1 for the other they fall on different SIMDs of the CU, where the
// halves' first waves share one.  The same statistics as win_row_stats<512> for each
// row, but with no early return: every thread passes the same barriers (five, four without top-k)
// whatever either row holds, so the halves never wait at different ones.
// Returns this half's status: 0 success (S.res), 1 invalid row (S.res
// written invalid), 2 the row needs the exact bisection path (the histogram
// is left for the caller to clear).  After 0 or 1 the histogram and side
// counters are zero.
__device__ __forceinline__ int win_pair_stats(uint32_t* hist, WinScratch& S, int t, int lead,
                                              int64_t V, float a, int top_k, float top_p) {
  constexpr int NT = 512, NW = NT / kWave;
  const int lane = t & (kWave - 1);
  const int wv = t / kWave;
  const bool use_k = top_k > 0 && (int64_t)top_k < V;
  const bool use_p = top_p < 1.0f;
  const uint32_t s_zero = S.side[kSideZero], s_ninf = S.side[kSideNegInf];
  const uint32_t s_bad = S.side[kSideBad], s_huge = S.side[kSideHuge];
  const uint32_t s_tneg = S.side[kSideTinyNeg], s_tpos = S.side[kSideTinyPos];
  const uint32_t tiny = s_tneg + s_tpos;
  const uint32_t zcnt = s_zero + tiny;  // the zero entry: zeros and tiny values
  const uint32_t nz = zcnt != 0u ? 1u : 0u;

  // The list of non-empty entries in descending key order (as win_stats_list):
  // two threads per key-ordered group kg = 255 - t/2, met by a lane swap.
  uint32_t npos = 0, nwin = 0;
  {
    const uint32_t gi = (uint32_t)t / 2u;
    const uint32_t kg = 255u - gi;
    const uint32_t sg = kg >= 128u ? kg - 128u : 255u - kg;
    const uint4* h4 = reinterpret_cast<const uint4*>(hist) + sg * 16u + ((uint32_t)t % 2u) * 8u;
    uint32_t cnt = 0;
#pragma unroll
    for (uint32_t j = 0; j < 8u; ++j) {
      const uint4 w = h4[(j + gi) % 8u];
      cnt += w.x + w.y + w.z + w.w;
    }
    cnt += (uint32_t)__builtin_amdgcn_mov_dpp((int)cnt, 0xB1, 0xF, 0xF, false);  // quad_perm 1,0,3,2
    const bool own = (uint32_t)t % 2u == 0u && cnt != 0;
    const uint64_t ball = __ballot(own);
    if (lane == 0) S.wcount[wv] = (uint32_t)__popcll(ball);
    block_sync_lds();  // 1
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
      S.list[pos] = (uint16_t)kg;
      S.lcnt[pos] = cnt;
    }
  }
  const uint32_t nl = nwin + nz + (s_ninf ? 1u : 0u);
  if (t == 0) {
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
  block_sync_lds();  // 2

  auto kcount = [&](uint32_t ent, uint32_t j) -> uint32_t {
    if (ent < (uint32_t)kWinGroups) return hist[win_idx(win_key(ent, j))];
    if (j != 0u) return 0u;
    return ent == kEntZero ? zcnt : s_ninf;
  };
  // status, the same in every thread of the half (it depends on LDS only)
  int st = 0;
  uint32_t max_key = 0u;
  const uint32_t e0 = nl != 0u ? (uint32_t)S.list[0] : (uint32_t)kEntNegInf;
  if (s_bad || (e0 == kEntNegInf && s_huge == 0u)) {
    st = 1;  // NaN/+inf, or no finite logit
    if (t == 0) S.res = RowStat{__builtin_nanf(""), __builtin_nanf(""), 0.0, 0, {0, 0, 0}};
  } else if (s_huge || (tiny && a > 16.0f) || (e0 == kEntZero && (s_tpos || !s_zero))) {
    st = 2;  // huge values, tiny ones at a low temperature, or a tiny max
  } else {
    if (e0 == kEntZero) {
      max_key = kKey16PosZero;
    } else {
      const uint64_t nzm = __ballot(kcount(e0, (uint32_t)lane) != 0u);
      max_key = win_key(e0, 63u - (uint32_t)__clzll((long long)nzm));
    }
    if (wv == lead && lane == 0) {
      S.m = value_of_key16(max_key);
      S.tk = 0;
      S.tk_entry = nl - 1;
    }
    if (use_k && wv == lead) {  // the top-k key by exact counts
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
  }
  // 3: the top-k key; without top-k every thread has the max and the
  // figures already (the halves agree on use_k, so both skip this barrier)
  if (use_k) block_sync_lds();
  if (st == 0 && S.fallback) st = 2;

  // Masses, normaliser and top-p cut: barriers 4 and 5.
  win_mass_cut<NT>(hist, S, t, a, use_k, use_p, zcnt, tiny, st == 0,
                   use_k ? S.m : value_of_key16(max_key), use_k ? S.tk : 0u,
                   use_k ? S.tk_entry : nl - 1u, lead);
  if (st == 0 && S.fallback) st = 2;
  if (st != 2) win_clear_listed<NT>(hist, S, t);
  return st;
}

// ---------------------------------------------------------------------------
// Stochastic verify for large batches of aligned bf16 rows: the position-task
// queue (protocol, words and helpers with TaskArgs in sv_kernels.hpp), one
// 1024-thread workgroup per CU.  A task (s, j) counts target row j with
// threads 0..511 into one exponent-window histogram and draft row j with
// threads 512..1023 into another, and scans both at once (win_pair_stats):
// one scan per position instead of two one after the other, while the count
// keeps every thread's loads in flight over the two rows.  The bonus task
// counts and scans its one row with every thread.  Thread kQ makes the
// queue's round trips: it reads the queue figures, the drafted token, its
// draw and the two logits of the ratio test as a task starts, appends
// the successor early and claims the next position (when plenty are queued)
// once the rows are counted, and reads the claimed slot after the scan; the
// next task's first vectors are then prefetched during the commit, or after
// the correction draw when there is one (whose loads take the registers).
struct PairScratch {
  double csum[16 * kDrawChunks];  // residual-draw chunk sums
  int32_t emit;
  int32_t pst[2];  // the halves' scan statuses
  uint32_t nidx;   // queue position taken for the next task (kNoClaim: none)
  uint32_t next;   // its task once known (0: slot not written yet)
  uint32_t fill;   // the exit fill's first slot when this workgroup finished the last task, else kNoClaim
  int32_t formed, accepted, keep, last;
};

template <int PF, int D>
__global__ __launch_bounds__(1024) void k_verify_pair_bf16(TaskArgs A) {
  constexpr int NT = 1024;
  constexpr int kQ = 512;
  __shared__ uint32_t hist[2 * kWinWords];
  __shared__ WinScratch S[2];
  __shared__ PairScratch Q;
  const int64_t V = A.V;
  const int k = A.k, k1 = k + 1, nr = 2 * k + 1;
  const uint32_t B = (uint32_t)A.B;

  uint4 pf[PF];
  uint32_t pf_task = 0u;  // the task whose rows' first vectors pf holds (0: none)
  bool starved = false;   // thread kQ: the last task found workgroups waiting for work
  win_clear<NT>(hist, S[0].side);
  win_clear<NT>(hist + kWinWords, S[1].side);
  if (opaque_tid() == kQ) {
    S[0].top_p = A.top_p;
    S[1].top_p = A.top_p;
    Q.next = task_wait(atomicAdd(&A.queue[0], 1u), A.slots, B, (uint32_t)k1);
  }
  block_sync_lds();
  uint32_t task = Q.next;

  while (task != kTaskExit) {
    const bool early = (task & kTaskSpec) != 0u;  // appended before j - 1 was decided
    task &= ~kTaskSpec;
    const int64_t b = (int64_t)((task - 1u) / (uint32_t)k1);
    const int j = (int)((task - 1u) - (uint32_t)b * (uint32_t)k1);
    const bool bonus = j == k;
    const uint16_t* trow = A.map.template row<uint16_t>(b * nr + j);
    const uint16_t* drow = bonus ? trow : A.map.template row<uint16_t>(b * nr + k1 + j);
    // Thread kQ reads the queue figures, the drafted token, its draw and the
    // two logits of the ratio test as the task starts; a wave's loads
    // complete in order, so they arrive with its count's first vectors.
    // While workgroups wait for work (as the previous task found), the
    // successor is appended at once, which waits for those loads; otherwise
    // after the count.
    int32_t tok = 0;
    float uj = 0.0f;
    uint16_t lt16 = 0, ld16 = 0;
    bool claim = false, spec = false;
    uint32_t q_head = 0, q_app = 0, q_seq = 0, nidx = kNoClaim;
    if (opaque_tid() == kQ) {
      q_head = ld_agent32(&A.queue[0]);
      q_app = task_appended(A.queue);
      if (!bonus) {
        tok = A.tokens[b * k + j];
        uj = A.u[b * k1 + j];
        if (early) q_seq = ld_agent32(A.seqstate + b);
        if (tok >= 0 && (int64_t)tok < V) {  // the two logits of the ratio test
          lt16 = trow[tok];
          ld16 = drow[tok];
        }
        if (starved && q_head > B + q_app && (q_seq & kSeqStop) == 0u) {
          task_append(A.queue, A.slots, (task + 1u) | kTaskSpec);
          spec = true;
        }
      }
      starved = q_head > B + q_app;
    }
    const bool pf_ok = pf_task == task;
    if (bonus) {
      win_count_stream<PF, D, NT>(hist, S[0].side, trow, V, pf, pf_ok, (uint32_t)opaque_tid());
    } else {
      const uint32_t t = (uint32_t)opaque_tid(), h = t >> 9;
      win_count_stream<PF, D, NT / 2>(hist + h * kWinWords, S[h].side, h ? drow : trow, V, pf,
                                       pf_ok, t & (NT / 2 - 1));
    }
    if (opaque_tid() == kQ) {
      if (!bonus && !spec && q_head > B + q_app && (q_seq & kSeqStop) == 0u) {
        task_append(A.queue, A.slots, (task + 1u) | kTaskSpec);
        spec = true;
      }
      claim = B + q_app > q_head + kClaimMargin;
      if (claim) nidx = atomicAdd(&A.queue[0], 1u);
    }
    block_sync_lds();
    if (bonus) {
      if (win_row_stats<NT>(hist, S[0], V, A.a, A.top_k, A.top_p, nullptr) == 2) {
        block_sync_lds();
        filter_row_bisect_call<uint16_t, true, NT>(trow, V, A.a, A.top_k, A.top_p, &S[0].res,
                                                    S[0].dslot, S[0].uslot);
        __syncthreads();
        win_clear<NT>(hist, S[0].side);
      }
    } else {
      const uint32_t t = (uint32_t)opaque_tid(), h = t >> 9;
      const int st = win_pair_stats(hist + h * kWinWords, S[h], (int)(t & (NT / 2 - 1)), h, V, A.a,
                                    A.top_k, A.top_p);
      if ((t & (NT / 2 - 1)) == 0u) Q.pst[h] = st;
      block_sync_lds();
      if (Q.pst[0] == 2 || Q.pst[1] == 2) {
#pragma unroll 1
        for (int hh = 0; hh < 2; ++hh) {
          if (Q.pst[hh] != 2) continue;
          filter_row_bisect_call<uint16_t, true, NT>(hh ? drow : trow, V, A.a, A.top_k, A.top_p,
                                                      &S[hh].res, S[hh].dslot, S[hh].uslot);
          __syncthreads();
          win_clear<NT>(hist + hh * kWinWords, S[hh].side);
        }
        block_sync_lds();
      }
    }
    // The successor appended early when workgroups wait for work; the ratio
    // test at j; the claimed position's slot read (its task is resolved at
    // the finish).
    uint32_t nx0 = 0u;
    if (opaque_tid() == kQ) {
      if (claim) nx0 = task_peek(nidx, A.slots, B, (uint32_t)k1);
      Q.nidx = nidx;
      const RowStat st_t = S[0].res;
      bool formed = st_t.valid != 0;
      bool acc = false;
      if (!bonus) {
        const RowStat st_d = S[1].res;
        formed = formed && st_d.valid && tok >= 0 && (int64_t)tok < V;
        if (formed) {
          const float lt = __builtin_bit_cast(float, (uint32_t)lt16 << 16);
          const float ld = __builtin_bit_cast(float, (uint32_t)ld16 << 16);
          const double p = prob_at(lt, st_t, A.a);
          const double q = prob_at(ld, st_d, A.a);
          const double alpha = q > 0.0 ? fmin(1.0, p / q) : (p > 0.0 ? 1.0 : 0.0);
          acc = (double)uj < alpha;
        }
      }
      Q.formed = formed ? 1 : 0;
      Q.accepted = acc ? 1 : 0;
    }
    block_sync_lds();
    const bool valid = Q.formed != 0;
    const bool stop = bonus || !(valid && Q.accepted != 0);
    const int n = j;
    // Commit once every earlier position has passed.  A task appended early
    // waits for the task of position j - 1, which was taken from the queue
    // before this one was appended and commits without waiting on anything
    // later; any other task was appended by that commit.
    if (opaque_tid() == kQ) {
      int keep = 1;
      if (early) {
        uint32_t d;
        while (((d = ld_agent32(A.seqstate + b)) & kSeqStop) == 0u && d < (uint32_t)j)
          __builtin_amdgcn_s_sleep(1);
        keep = (d & kSeqStop) == 0u;
      }
      if (keep) {
        if (spec) task_publish(A.seqstate + b, stop ? (kSeqStop | (uint32_t)j) : (uint32_t)(j + 1));
        else if (!stop) task_append(A.queue, A.slots, task + 1u);
      }
      Q.keep = keep;
      Q.next = claim ? nx0 : 0u;
    }
    block_sync_lds();
    // The next task's first vectors: now, unless a correction is drawn first
    // (its loads take the registers, and the draw leaves time for nothing
    // else), then after the draw.
    auto prefetch_task = [&](uint32_t nx) {
      if (nx == 0u || nx == kTaskExit) return;
      pf_task = nx & ~kTaskSpec;
      const uint32_t nt = pf_task - 1u;
      const int64_t nb = (int64_t)(nt / (uint32_t)k1);
      const int nj = (int)(nt - (uint32_t)nb * (uint32_t)k1);
      const uint32_t t = (uint32_t)opaque_tid(), h = t >> 9;
      if (nj == k)
        win_prefetch_row<PF, NT>(pf, A.map.template row<uint16_t>(nb * nr + nj), V, t);
      else
        win_prefetch_row<PF, NT / 2>(pf, A.map.template row<uint16_t>(nb * nr + nj + h * k1), V,
                                     t & (NT / 2 - 1));
    };
    const bool draws = Q.keep && stop;
    pf_task = 0u;
    if (!draws) prefetch_task(Q.next);
    if (draws) {
      // correction from the residual of the two rows at n, or the bonus draw
      int32_t emitted = -1;
      if (valid) {
        const RowStat& sp = S[0].res;
        const RowStat& sq = S[bonus ? 0 : 1].res;
        // one step per batch and a window of two steps in flight per wave:
        // what the kernel's register budget holds without spilling in the loop
        emitted = residual_draw_call<1, 2>(trow, drow, !bonus, sp.m, sp.thr, sp.z, sq.m, sq.thr,
                                           sq.z, A.a, V, A.u[b * k1 + k], Q.csum, &Q.emit);
      }
      int32_t* out = A.out_tokens + b * k1;
      for (int t = opaque_tid(); t <= k; t += NT) {
        int32_t v = -1;
        if (valid) {
          if (t < n) v = A.tokens[b * k + t];
          else if (t == n) v = emitted;
        }
        out[t] = v;
      }
      if (opaque_tid() == 0) A.accepted_len[b] = valid ? n : -1;
    }
    // Every task, kept or dropped, counts as finished after its appends: the
    // count reaching every task ever appended means none is left, so none can
    // be appended any more, and the queue positions past the last task tell
    // each workgroup to leave.  A workgroup that already holds its next task
    // cannot have finished the last one, so it does not wait for the count;
    // otherwise the position for the next task is taken in the same round
    // trip.  The workgroup that finishes the last task writes the exit slots
    // with all its threads (one slot each), then waits on its own position.
    if (opaque_tid() == kQ) {
      Q.fill = kNoClaim;
      if (Q.next != 0u) {
        (void)__hip_atomic_fetch_add(task_af(A.queue), 1ull, __ATOMIC_RELAXED,
                                     __HIP_MEMORY_SCOPE_AGENT);
      } else {
        const uint64_t af = __hip_atomic_fetch_add(task_af(A.queue), 1ull, __ATOMIC_RELAXED,
                                                   __HIP_MEMORY_SCOPE_AGENT) + 1ull;
        const uint32_t i = Q.nidx != kNoClaim ? Q.nidx : atomicAdd(&A.queue[0], 1u);
        const uint32_t P = (uint32_t)(af >> 32);
        Q.nidx = i;
        if ((uint32_t)af == B + P) Q.fill = P;
        else Q.next = task_wait(i, A.slots, B, (uint32_t)k1);
      }
    }
    block_sync_lds();
    if (Q.fill != kNoClaim) {
      for (uint32_t e = (uint32_t)opaque_tid(); e < gridDim.x; e += NT)
        task_publish(A.slots + Q.fill + e, kTaskExit);
      if (opaque_tid() == kQ) Q.next = task_wait(Q.nidx, A.slots, B, (uint32_t)k1);
      block_sync_lds();
    }
    task = Q.next;
    if (pf_task == 0u) prefetch_task(task);
    block_sync_lds();  // everyone has read Q before the next task writes it
  }

  // The last workgroup out leaves the queue words, the used slots and the
  // sequence words zero.
  if (opaque_tid() == kQ) {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
    Q.last = atomicAdd(&A.queue[1], 1u) == gridDim.x - 1 ? 1 : 0;
  }
  block_sync_lds();
  if (Q.last) {
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
    const uint32_t used = task_appended(A.queue) + gridDim.x;
    for (uint32_t i = (uint32_t)opaque_tid(); i < used; i += NT) A.slots[i] = 0u;
    for (uint32_t i = (uint32_t)opaque_tid(); i < B; i += NT) A.seqstate[i] = 0u;
    block_sync_lds();
    if (opaque_tid() < 4) A.queue[opaque_tid()] = 0u;
  }
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
  if (r < r_hi) win_prefetch_row<PF, kWinThreads>(pf, F.map.template row<uint16_t>(r), V, opaque_tid());
  win_clear<kWinThreads>(hist, S.side);  // afterwards each row's scan leaves the histogram zero
  for (; r < r_hi; r += per_xcd) {
    const uint16_t* row = F.map.template row<uint16_t>(r);
    block_sync_lds();
    win_count_stream<PF, D, kWinThreads>(hist, S.side, row, V, pf, true, opaque_tid());
    block_sync_lds();
    if (r + per_xcd < r_hi)
      win_prefetch_row<PF, kWinThreads>(pf, F.map.template row<uint16_t>(r + per_xcd), V, opaque_tid());
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
