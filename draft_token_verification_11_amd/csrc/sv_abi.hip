// sv_abi.hip -- the C ABI of libspecverify: argument validation, workspace
// layout and kernel launches for gfx950.  See include/specverify.h for the
// contract of every entry point.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <mutex>

#include "specverify.h"
#include "sv_kernels.hpp"
#include "sv_window.hpp"

namespace {

constexpr int kRowThreads = 256;     // split-V chunk kernels
constexpr int kFilterThreads = 1024;  // one workgroup per filtered row
constexpr int kTailThreads = 512;     // one workgroup per sequence
constexpr int64_t kMinBlocks = 2048;  // split-V target occupancy (8 per CU)
constexpr int64_t kMaxWorkItems = (int64_t(1) << 32) - 1;

struct Layout {
  bool filtered = false;
  int vpt = 1;       // 8-element groups per thread in split-V kernels
  int nchunks = 1;   // V-chunks per row
  int64_t rows = 0;  // rows processed
  size_t rowstat_off = 0, part_off = 0, queue_off = 0, total = 0;
  size_t help_off = 0;  // whole-sequence walk: the help region (sv::HelpView)
  size_t slots_off = 0;  // position-task queue: the appended tasks (sv::TaskArgs::slots)
  // correction draw spread over the chip (small batches on the row-pass path)
  bool split_draw = false;
  int64_t draw_chunks = 0;
  size_t jobs_off = 0, dsums_off = 0;
};

using sv::kMaxWalkGrid;

// The whole-sequence walk's queue words and help region, and (B > 0) the
// position-task queue's slots (at most B k appended tasks plus one exit
// entry per workgroup) followed by one state word per sequence.
size_t walk_regions(Layout& L, size_t off, int64_t k, int64_t B) {
  L.queue_off = off;
  off = (off + 4 * sizeof(uint32_t) + 255) & ~size_t(255);
  L.help_off = off;
  off = (off + size_t(sv::HelpView::bytes(2 * k + 1)) + 255) & ~size_t(255);
  if (B > 0) {
    L.slots_off = off;
    off = (off + size_t(B * k + kMaxWalkGrid + B) * sizeof(uint32_t) + 255) & ~size_t(255);
  }
  return off;
}

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

// Batches of at most this many sequences may spread their correction draws
// over the chip (when they leave most CUs idle and the rows span chunks).
constexpr int64_t kSplitDrawMaxB = 128;

// Unfiltered rows of at most this many elements get their statistics in the
// tail (one launch fewer; a wave reads such a row in a few steps).
constexpr int64_t kDirectMaxV = 4096;

int64_t chunk_elems(int vpt) { return int64_t(kRowThreads) * vpt * 8; }

int pick_vpt(int64_t rows, int64_t V) {
  // Largest register tile that still gives the chip enough workgroups.
  for (int vpt : {8, 4, 2}) {
    const int64_t nch = (V + chunk_elems(vpt) - 1) / chunk_elems(vpt);
    if (rows * nch >= kMinBlocks) return vpt;
  }
  return 1;
}

bool is_filtered(const spec_sampling_t& s, int64_t V) {
  return (s.top_k > 0 && int64_t(s.top_k) < V) || s.top_p < 1.0f;
}

Layout make_layout(int op, int64_t B, int64_t k, int64_t V, const spec_sampling_t* s) {
  Layout L;
  if (op == SPEC_OP_STOCHASTIC) L.rows = B * (2 * k + 1);
  else if (op == SPEC_OP_GREEDY) L.rows = B * (k + 1);
  else L.rows = B;
  L.filtered = (op != SPEC_OP_GREEDY) && is_filtered(*s, V);
  L.vpt = pick_vpt(L.rows, V);
  L.nchunks = int((V + chunk_elems(L.vpt) - 1) / chunk_elems(L.vpt));
  size_t off = 0;
  const bool need_rowstat = L.filtered || op == SPEC_OP_PROCESS;
  const bool need_part = !L.filtered;
  if (need_rowstat) {
    L.rowstat_off = off;
    off = align256(off + size_t(L.rows) * sizeof(sv::RowStat));
  }
  if (need_part) {
    L.part_off = off;
    off = align256(off + size_t(L.rows) * size_t(L.nchunks) * 16);
  }
  if (op == SPEC_OP_STOCHASTIC) off = walk_regions(L, off, k, B);  // whole-sequence kernels
  if (op == SPEC_OP_STOCHASTIC && B <= kSplitDrawMaxB) {
    // per sequence a draw job and the residual's sum over each chunk
    L.split_draw = true;
    L.draw_chunks = (V + sv::kDrawChunk - 1) / sv::kDrawChunk;
    L.jobs_off = off;
    off = align256(off + size_t(B) * sizeof(sv::DrawJob));
    L.dsums_off = off;
    off = align256(off + size_t(B) * size_t(L.draw_chunks) * sizeof(double));
  }
  L.total = off < 256 ? 256 : off;
  return L;
}

// Pooled rows: the row passes run over the pools (nt target rows, then nd
// draft rows; greedy: the nt target rows).  The row-statistics region always
// exists: the whole-sequence walk keeps the target pool's statistics there.
Layout make_pooled_layout(int op, int64_t nt, int64_t nd, int64_t k, int64_t V,
                          const spec_sampling_t* s) {
  Layout L;
  const bool greedy = op == SPEC_OP_GREEDY;
  L.rows = greedy ? nt : nt + nd;
  L.filtered = !greedy && is_filtered(*s, V);
  L.vpt = pick_vpt(L.rows, V);
  L.nchunks = int((V + chunk_elems(L.vpt) - 1) / chunk_elems(L.vpt));
  size_t off = 0;
  if (!greedy) {
    L.rowstat_off = off;
    off = align256(off + size_t(L.rows) * sizeof(sv::RowStat));
  }
  if (!L.filtered) {
    L.part_off = off;
    off = align256(off + size_t(L.rows) * size_t(L.nchunks) * 16);
  }
  if (!greedy) off = walk_regions(L, off, k, 0);
  L.total = off < 256 ? 256 : off;
  return L;
}

int check_pools(int64_t nt, int64_t nd, const int32_t* tmap, const int32_t* dmap, int64_t B,
                int64_t k, bool need_draft) {
  if (nt < 1 || (need_draft && nd < 1)) return SPEC_ERR_INVALID_ARG;
  if (!tmap && nt < B * (k + 1)) return SPEC_ERR_INVALID_ARG;
  if (need_draft && !dmap && nd < B * k) return SPEC_ERR_INVALID_ARG;
  return SPEC_OK;
}

size_t elem_size(int dtype) { return dtype == SPEC_DTYPE_BF16 ? 2 : 4; }

int check_logits(const spec_logits_t& t, int64_t V) {
  if (t.dtype != SPEC_DTYPE_F32 && t.dtype != SPEC_DTYPE_BF16) return SPEC_ERR_UNSUPPORTED;
  if (!t.data) return SPEC_ERR_INVALID_ARG;
  if (reinterpret_cast<uintptr_t>(t.data) % elem_size(t.dtype)) return SPEC_ERR_INVALID_ARG;
  if (t.pos_stride < V || t.seq_stride < 0) return SPEC_ERR_INVALID_ARG;
  return SPEC_OK;
}

bool vec_ok(const spec_logits_t& t) {
  const size_t es = elem_size(t.dtype);
  return reinterpret_cast<uintptr_t>(t.data) % 16 == 0 && (size_t(t.pos_stride) * es) % 16 == 0 &&
         (size_t(t.seq_stride) * es) % 16 == 0;
}

int check_sampling(const spec_sampling_t* s) {
  if (!s) return SPEC_ERR_INVALID_ARG;
  if (!std::isfinite(s->temperature) || !(s->temperature > 0.0f)) return SPEC_ERR_INVALID_ARG;
  if (s->top_k < 0) return SPEC_ERR_INVALID_ARG;
  if (!(s->top_p > 0.0f && s->top_p <= 1.0f)) return SPEC_ERR_INVALID_ARG;
  return SPEC_OK;
}

int check_sizes(int64_t B, int64_t k, int64_t V, bool need_k) {
  if (B < 1 || V < 1) return SPEC_ERR_INVALID_ARG;
  if (need_k && k < 1) return SPEC_ERR_INVALID_ARG;
  if (B > (int64_t(1) << 24) || V > SPEC_MAX_V || (need_k && k > SPEC_MAX_K))
    return SPEC_ERR_UNSUPPORTED;
  return SPEC_OK;
}

int check_workspace(void* ws, size_t bytes, const Layout& L) {
  if (!ws || bytes < L.total || reinterpret_cast<uintptr_t>(ws) % 256) return SPEC_ERR_WORKSPACE;
  return SPEC_OK;
}

bool grid_fits(int64_t blocks, int threads) { return blocks >= 1 && blocks * threads <= kMaxWorkItems; }

bool row_pass_fits(const Layout& L, int dtype, bool vec) {
  if (!L.filtered) return grid_fits(L.rows * L.nchunks, kRowThreads);
  if (dtype == SPEC_DTYPE_BF16 && vec) return true;  // persistent: one workgroup per CU
  return grid_fits(L.rows, kFilterThreads);
}

float log2e_over(float T) { return float(1.4426950408889634 / double(T)); }

// The compute-unit count of each device, queried once per device (the first
// call on a device, with a thread-safe once) and kept until the process ends.
// Grids are sized by the device of the stream a call is enqueued on.
constexpr int kMaxDevices = 64;
constexpr int kDefaultCus = 256;  // used when the device cannot be queried
std::once_flag g_cus_once[kMaxDevices];
int g_cus[kMaxDevices];

int query_cus(int dev) {
  int cus = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      cus <= 0)
    cus = kDefaultCus;
  return cus;
}

int stream_device(hipStream_t st) {
  int dev = -1;
  if (st != nullptr) {
    hipDevice_t d = -1;
    if (hipStreamGetDevice(st, &d) == hipSuccess) dev = d;
  } else if (hipGetDevice(&dev) != hipSuccess) {
    dev = -1;
  }
  return dev;
}

int device_cus(hipStream_t st) {
  const int dev = stream_device(st);
  if (dev < 0) return kDefaultCus;
  if (dev >= kMaxDevices) return query_cus(dev);
  std::call_once(g_cus_once[dev], [dev] { g_cus[dev] = query_cus(dev); });
  return g_cus[dev];
}

int walk_grid_for(int cus) { return cus < kMaxWalkGrid ? cus : kMaxWalkGrid; }

// Workgroups of the persistent filter: `per_cu` per CU, a multiple of 8 (one
// range of rows per XCD), no more than needed.
int persistent_grid(int64_t rows, int cus, int per_cu = 1) {
  int64_t g = int64_t(cus) * per_cu;
  if (rows < g) g = rows;
  g = (g + 7) / 8 * 8;
  return int(g);
}

// The whole-sequence kernel (rows read in walk order, nothing past the stop)
// pays off once every CU has several sequences to take from the queue;
// smaller batches spread their rows over the chip instead.
constexpr int kSeqPerCu = 2;

// Which kernels a stochastic call runs (spec_path_t): aligned bf16 rows with
// at least kSeqPerCu sequences per CU read rows in walk order in one kernel
// -- the position-task queue, or the whole-sequence walk when alpha is asked
// for (it is reported past the stop, so every row is read); anything else a
// row pass over every row followed by the per-sequence tail.
int stochastic_path(int dtype, bool vec, int64_t B, int cus, bool want_alpha) {
  if (dtype != SPEC_DTYPE_BF16 || !vec || B < int64_t(kSeqPerCu) * cus) return SPEC_PATH_ROW_PASS;
  return want_alpha ? SPEC_PATH_SEQUENCE_WALK : SPEC_PATH_TASK_QUEUE;
}

constexpr int kPrefetch = 2;  // 16-byte vectors per thread prefetched for the next row
constexpr int kLoadDepth = 8;  // 16-byte loads in flight per thread in the row stream

template <typename T, bool VEC>
void launch_partials(const Layout& L, const sv::RowMap& map, int64_t V, float a, sv::Partial* part,
                     hipStream_t st) {
  const dim3 grid(unsigned(L.rows * L.nchunks)), block(kRowThreads);
  switch (L.vpt) {
    case 8: hipLaunchKernelGGL((sv::k_row_partials<T, VEC, 8>), grid, block, 0, st, map, V, L.nchunks, a, part); break;
    case 4: hipLaunchKernelGGL((sv::k_row_partials<T, VEC, 4>), grid, block, 0, st, map, V, L.nchunks, a, part); break;
    case 2: hipLaunchKernelGGL((sv::k_row_partials<T, VEC, 2>), grid, block, 0, st, map, V, L.nchunks, a, part); break;
    default: hipLaunchKernelGGL((sv::k_row_partials<T, VEC, 1>), grid, block, 0, st, map, V, L.nchunks, a, part); break;
  }
}

template <typename T, bool VEC>
void launch_greedy_partials(const Layout& L, const sv::RowMap& map, int64_t V, sv::GPartial* part,
                            hipStream_t st) {
  const dim3 grid(unsigned(L.rows * L.nchunks)), block(kRowThreads);
  switch (L.vpt) {
    case 8: hipLaunchKernelGGL((sv::k_greedy_partials<T, VEC, 8>), grid, block, 0, st, map, V, L.nchunks, part); break;
    case 4: hipLaunchKernelGGL((sv::k_greedy_partials<T, VEC, 4>), grid, block, 0, st, map, V, L.nchunks, part); break;
    case 2: hipLaunchKernelGGL((sv::k_greedy_partials<T, VEC, 2>), grid, block, 0, st, map, V, L.nchunks, part); break;
    default: hipLaunchKernelGGL((sv::k_greedy_partials<T, VEC, 1>), grid, block, 0, st, map, V, L.nchunks, part); break;
  }
}

template <typename T, bool VEC>
void launch_probs(const Layout& L, const sv::RowMap& map, int64_t V, float a, const sv::RowStat* rs,
                  float* probs, hipStream_t st) {
  const dim3 grid(unsigned(L.rows * L.nchunks)), block(kRowThreads);
  switch (L.vpt) {
    case 8: hipLaunchKernelGGL((sv::k_probs<T, VEC, 8>), grid, block, 0, st, map, V, L.nchunks, a, rs, probs); break;
    case 4: hipLaunchKernelGGL((sv::k_probs<T, VEC, 4>), grid, block, 0, st, map, V, L.nchunks, a, rs, probs); break;
    case 2: hipLaunchKernelGGL((sv::k_probs<T, VEC, 2>), grid, block, 0, st, map, V, L.nchunks, a, rs, probs); break;
    default: hipLaunchKernelGGL((sv::k_probs<T, VEC, 1>), grid, block, 0, st, map, V, L.nchunks, a, rs, probs); break;
  }
}

template <typename T, bool VEC>
void launch_filter(const Layout& L, const sv::RowMap& map, int64_t V, float a,
                   const spec_sampling_t& s, sv::RowStat* rs, hipStream_t st, int cus) {
  const dim3 grid(unsigned(L.rows)), block(kFilterThreads);
  if constexpr (sizeof(T) == 2) {
    if (VEC) {
      // two 512-thread workgroups per CU, each with a 64 KiB window histogram
      sv::FilterArgs F{map, V, L.rows, a, s.top_k, s.top_p, rs};
      hipLaunchKernelGGL((sv::k_filter_win_persistent<kPrefetch, kLoadDepth>),
                         dim3(persistent_grid(L.rows, cus, 2)), dim3(sv::kWinThreads), 0, st, F);
    } else {
      hipLaunchKernelGGL((sv::k_filter_bf16_hist<VEC>), grid, block, 0, st, map, V, a, s.top_k,
                         s.top_p, rs);
    }
  } else {
    hipLaunchKernelGGL((sv::k_filter_bisect<T, VEC>), grid, block, 0, st, map, V, a, s.top_k,
                       s.top_p, rs);
  }
}

template <typename T, bool VEC>
void launch_tail(int64_t B, const sv::TailArgs& args, hipStream_t st) {
  hipLaunchKernelGGL((sv::k_tail<T, VEC>), dim3(unsigned(B)), dim3(kTailThreads), 0, st, args);
}

// Runs f<T, VEC>() for the dtype / alignment at hand.
template <template <typename, bool> class F, typename... Args>
void dispatch(int dtype, bool vec, Args&&... args) {
  if (dtype == SPEC_DTYPE_BF16) {
    if (vec) F<uint16_t, true>::run(args...);
    else F<uint16_t, false>::run(args...);
  } else {
    if (vec) F<float, true>::run(args...);
    else F<float, false>::run(args...);
  }
}

template <typename T, bool VEC>
struct StochasticRun {
  static void run(const Layout& L, const sv::RowMap& map, int64_t B, int64_t V, float a,
                  const spec_sampling_t& s, sv::TailArgs& args, char* ws, hipStream_t st,
                  int walk_grid, int cus) {
    if constexpr (sizeof(T) == 2 && VEC) {
      if (walk_grid > 0 && !args.accept_prob) {
        sv::TaskArgs A{map, V, args.k, int32_t(B), a, s.top_k, s.top_p, args.tokens, args.u,
                       args.accepted_len, args.out_tokens,
                       reinterpret_cast<uint32_t*>(ws + L.queue_off),
                       reinterpret_cast<uint32_t*>(ws + L.slots_off),
                       reinterpret_cast<uint32_t*>(ws + L.slots_off) + (B * args.k + kMaxWalkGrid)};
        hipLaunchKernelGGL((sv::k_verify_pair_bf16<kPrefetch, kLoadDepth>),
                           dim3(unsigned(walk_grid)), dim3(kFilterThreads), 0, st, A);
        return;
      }
      if (walk_grid > 0) {
        sv::SeqArgs A{map, V, args.k, int32_t(B), a, s.top_k, s.top_p, args.tokens, args.u,
                      args.accepted_len, args.out_tokens, args.accept_prob,
                      reinterpret_cast<uint32_t*>(ws + L.queue_off), nullptr,
                      reinterpret_cast<uint64_t*>(ws + L.help_off)};
        hipLaunchKernelGGL((sv::k_verify_seq_bf16<kPrefetch, kLoadDepth, false>),
                           dim3(unsigned(walk_grid)), dim3(kFilterThreads), 0, st, A);
        return;
      }
    }
    if (L.filtered) {
      auto* rs = reinterpret_cast<sv::RowStat*>(ws + L.rowstat_off);
      launch_filter<T, VEC>(L, map, V, a, s, rs, st, cus);
      args.rowstat = rs;
      args.part = nullptr;
    } else if (V <= kDirectMaxV) {
      // small unfiltered rows: the tail computes their statistics itself
      args.rowstat = nullptr;
      args.part = nullptr;
    } else {
      auto* part = reinterpret_cast<sv::Partial*>(ws + L.part_off);
      launch_partials<T, VEC>(L, map, V, a, part, st);
      args.rowstat = nullptr;
      args.part = part;
    }
    args.nchunks = L.nchunks;
    // small batches: the draws spread over the chip instead of one tail
    // workgroup per sequence reading its two rows alone
    const bool split = VEC && L.split_draw && L.draw_chunks >= 2 && 2 * B <= cus;
    auto* jobs = reinterpret_cast<sv::DrawJob*>(ws + L.jobs_off);
    auto* dsums = reinterpret_cast<double*>(ws + L.dsums_off);
    args.jobs = split ? jobs : nullptr;
    launch_tail<T, VEC>(B, args, st);
    if (split) {
      hipLaunchKernelGGL((sv::k_draw_split<T, VEC>), dim3(unsigned(L.draw_chunks), unsigned(B)),
                         dim3(sv::kDrawThreads), 0, st, map, V, args.k, a, jobs, L.draw_chunks,
                         dsums, args.u, args.accepted_len, args.out_tokens);
    }
  }
};

template <typename T, bool VEC>
struct GreedyRun {
  static void run(const Layout& L, const sv::RowMap& map, int64_t V, sv::GPartial* part, hipStream_t st) {
    launch_greedy_partials<T, VEC>(L, map, V, part, st);
  }
};

template <typename T, bool VEC>
struct ProcessRun {
  static void run(const Layout& L, const sv::RowMap& map, int64_t V, float a, const spec_sampling_t& s,
                  spec_row_stats_t* row_stats, float* probs, char* ws, hipStream_t st, int cus) {
    auto* rs = reinterpret_cast<sv::RowStat*>(ws + L.rowstat_off);
    sv::Partial* part = nullptr;
    if (L.filtered) {
      launch_filter<T, VEC>(L, map, V, a, s, rs, st, cus);
    } else {
      part = reinterpret_cast<sv::Partial*>(ws + L.part_off);
      launch_partials<T, VEC>(L, map, V, a, part, st);
    }
    if (part && L.nchunks > 16)  // many chunks per row: one wave per row merges them
      hipLaunchKernelGGL(sv::k_process_stats_wide, dim3(unsigned((L.rows + 3) / 4)), dim3(256), 0,
                         st, L.rows, L.nchunks, a, part, rs, row_stats);
    else
      hipLaunchKernelGGL(sv::k_process_stats, dim3(unsigned((L.rows + 255) / 256)), dim3(256), 0,
                         st, L.rows, L.nchunks, a, part, rs, row_stats);
    if (probs) launch_probs<T, VEC>(L, map, V, a, rs, probs, st);
  }
};

template <typename T, bool VEC>
struct PooledStochasticRun {
  static void run(const Layout& L, const sv::RowMap& map, int64_t B, int64_t V, float a,
                  const spec_sampling_t& s, sv::TailArgs& args, char* ws, hipStream_t st,
                  int walk_grid, int cus) {
    auto* rs = reinterpret_cast<sv::RowStat*>(ws + L.rowstat_off);
    int64_t clear_bytes = 0;
    if constexpr (sizeof(T) == 2 && VEC) {
      if (walk_grid > 0) {
        // target pool statistics first, then the walk over the draft rows
        const int64_t nt = map.nt;
        sv::FilterArgs F{map, V, nt, a, s.top_k, s.top_p, rs};
        hipLaunchKernelGGL((sv::k_filter_win_persistent<kPrefetch, kLoadDepth>),
                           dim3(persistent_grid(nt, cus, 2)), dim3(sv::kWinThreads), 0, st, F);
        sv::SeqArgs A{map, V, args.k, int32_t(B), a, s.top_k, s.top_p, args.tokens, args.u,
                      args.accepted_len, args.out_tokens, args.accept_prob,
                      reinterpret_cast<uint32_t*>(ws + L.queue_off), rs,
                      reinterpret_cast<uint64_t*>(ws + L.help_off)};
        hipLaunchKernelGGL((sv::k_verify_seq_bf16<kPrefetch, kLoadDepth, true>),
                           dim3(unsigned(walk_grid)), dim3(kFilterThreads), 0, st, A);
        clear_bytes = nt * int64_t(sizeof(sv::RowStat));
      }
    }
    if (clear_bytes == 0) {
      if (L.filtered) {
        launch_filter<T, VEC>(L, map, V, a, s, rs, st, cus);
        args.rowstat = rs;
        args.part = nullptr;
        clear_bytes = L.rows * int64_t(sizeof(sv::RowStat));
      } else {
        auto* part = reinterpret_cast<sv::Partial*>(ws + L.part_off);
        launch_partials<T, VEC>(L, map, V, a, part, st);
        args.rowstat = nullptr;
        args.part = part;
        clear_bytes = L.rows * L.nchunks * 16;
      }
      args.nchunks = L.nchunks;
      launch_tail<T, VEC>(B, args, st);
    }
    // shared records are cleared once every sequence has read them
    char* base = args.part ? ws + L.part_off : ws + L.rowstat_off;
    const int64_t words = (clear_bytes + 15) / 16;
    hipLaunchKernelGGL(sv::k_clear, dim3(unsigned((words + 255) / 256)), dim3(256), 0, st,
                       reinterpret_cast<uint4*>(base), words);
  }
};

template <typename TI, typename TO>
void launch_apply(bool vec, unsigned nblk, const sv::ApplyArgs& A, hipStream_t st) {
  if (vec) hipLaunchKernelGGL((sv::k_logits_apply<TI, TO, true>), dim3(nblk), dim3(256), 0, st, A);
  else hipLaunchKernelGGL((sv::k_logits_apply<TI, TO, false>), dim3(nblk), dim3(256), 0, st, A);
}

// Fused LM head: 256-wide vocabulary tiles (4 waves x 4 column blocks of 16;
// narrower tiles measured slower); per row one merged 8-byte record and a
// 4-byte flag word.
constexpr int64_t kLmTile = 256;
size_t lmhead_bad_off(int64_t M) { return align256(size_t(M) * 8); }
size_t lmhead_workspace(int64_t B, int64_t k, int64_t V) {
  (void)V;
  const int64_t M = B * (k + 1);
  return lmhead_bad_off(M) + align256(size_t(M) * 4);
}

int finish_launch() {
  return hipGetLastError() == hipSuccess ? SPEC_OK : SPEC_ERR_HIP;
}

int check_stochastic_args(const spec_logits_t& target, const spec_logits_t& draft,
                          const int32_t* draft_tokens, const float* uniforms, int64_t B,
                          int64_t k, int64_t V, const spec_sampling_t* sampling,
                          const int32_t* accepted_len, const int32_t* out_tokens) {
  int rc;
  if ((rc = check_sizes(B, k, V, true)) != SPEC_OK) return rc;
  if ((rc = check_sampling(sampling)) != SPEC_OK) return rc;
  if ((rc = check_logits(target, V)) != SPEC_OK) return rc;
  if ((rc = check_logits(draft, V)) != SPEC_OK) return rc;
  if (target.dtype != draft.dtype) return SPEC_ERR_INVALID_ARG;
  if (!draft_tokens || !uniforms || !accepted_len || !out_tokens) return SPEC_ERR_INVALID_ARG;
  return SPEC_OK;
}

// ---------------------------------------------------------------------------
// Workspace of spec_verify_stochastic_noalloc: one array per GPU in the
// library's code object, kept until the process ends.  In host code the
// array's name is only a stand-in for the device symbol: its device address
// is taken once per device (with that device current) by
// hipGetSymbolAddress and only that address is handed to kernels.
constexpr size_t kScratchBytes = size_t(16) << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

std::once_flag g_scratch_once[kMaxDevices];
void* g_scratch_ptr[kMaxDevices];
hipError_t g_scratch_rc[kMaxDevices];

// The scratch array's address on device `dev` (nullptr if it cannot be had).
void* scratch_on(int dev) {
  if (dev < 0 || dev >= kMaxDevices) return nullptr;
  std::call_once(g_scratch_once[dev], [dev] {
    int cur = -1;
    hipError_t rc = hipGetDevice(&cur);
    if (rc == hipSuccess && cur != dev) rc = hipSetDevice(dev);
    void* ptr = nullptr;
    if (rc == hipSuccess) rc = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (cur >= 0 && cur != dev) (void)hipSetDevice(cur);
    g_scratch_rc[dev] = rc;
    g_scratch_ptr[dev] = rc == hipSuccess ? ptr : nullptr;
  });
  return g_scratch_ptr[dev];
}

}  // namespace

extern "C" {

size_t spec_workspace_size(int32_t op, int32_t B, int32_t k, int32_t V,
                           const spec_sampling_t* sampling) {
  if (op == SPEC_OP_GREEDY_LMHEAD) {
    if (check_sizes(B, k, V, true) != SPEC_OK) return 0;
    return lmhead_workspace(B, k, V);
  }
  if (op != SPEC_OP_STOCHASTIC && op != SPEC_OP_GREEDY && op != SPEC_OP_PROCESS) return 0;
  if (check_sizes(B, k, V, op != SPEC_OP_PROCESS) != SPEC_OK) return 0;
  spec_sampling_t plain = {1.0f, 0, 1.0f};
  if (op != SPEC_OP_GREEDY) {
    if (check_sampling(sampling) != SPEC_OK) return 0;
  } else {
    sampling = &plain;
  }
  return make_layout(op, B, k, V, sampling).total;
}

int spec_verify_stochastic(spec_logits_t target, spec_logits_t draft, const int32_t* draft_tokens,
                           const float* uniforms, int32_t B, int32_t k, int32_t V,
                           const spec_sampling_t* sampling, int32_t* accepted_len,
                           int32_t* out_tokens, float* accept_prob, void* workspace,
                           size_t workspace_bytes, void* stream) {
  int rc;
  if ((rc = check_stochastic_args(target, draft, draft_tokens, uniforms, B, k, V, sampling,
                                  accepted_len, out_tokens)) != SPEC_OK)
    return rc;
  const Layout L = make_layout(SPEC_OP_STOCHASTIC, B, k, V, sampling);
  if ((rc = check_workspace(workspace, workspace_bytes, L)) != SPEC_OK) return rc;
  const bool vec = vec_ok(target) && vec_ok(draft);
  const int cus = device_cus(static_cast<hipStream_t>(stream));
  const int path = stochastic_path(target.dtype, vec, B, cus, accept_prob != nullptr);
  const int walk_grid = path != SPEC_PATH_ROW_PASS ? walk_grid_for(cus) : 0;
  if (!walk_grid && (!row_pass_fits(L, target.dtype, vec) || !grid_fits(B, kTailThreads)))
    return SPEC_ERR_UNSUPPORTED;

  sv::RowMap map{target.data, target.seq_stride, target.pos_stride, draft.data, draft.seq_stride,
                 draft.pos_stride, 2 * k + 1, k + 1};
  const float a = log2e_over(sampling->temperature);
  sv::TailArgs args{};
  args.map = map;
  args.V = V;
  args.k = k;
  args.a = a;
  args.tokens = draft_tokens;
  args.u = uniforms;
  args.accepted_len = accepted_len;
  args.out_tokens = out_tokens;
  args.accept_prob = accept_prob;
  (void)hipGetLastError();
  dispatch<StochasticRun>(target.dtype, vec, L, map, int64_t(B), int64_t(V), a, *sampling, args,
                          static_cast<char*>(workspace), static_cast<hipStream_t>(stream),
                          walk_grid, cus);
  return finish_launch();
}

int spec_verify_stochastic_noalloc(spec_logits_t target, spec_logits_t draft,
                                   const int32_t* draft_tokens, const float* uniforms, int32_t B,
                                   int32_t k, int32_t V, const spec_sampling_t* sampling,
                                   int32_t* accepted_len, int32_t* out_tokens, float* accept_prob,
                                   void* stream) {
  int rc;
  if ((rc = check_stochastic_args(target, draft, draft_tokens, uniforms, B, k, V, sampling,
                                  accepted_len, out_tokens)) != SPEC_OK)
    return rc;
  const Layout L = make_layout(SPEC_OP_STOCHASTIC, B, k, V, sampling);
  if (L.total > kScratchBytes) return SPEC_ERR_UNSUPPORTED;
  auto st = static_cast<hipStream_t>(stream);
  void* ws = scratch_on(stream_device(st));
  if (!ws) return SPEC_ERR_HIP;
  // The array keeps whatever the last call on this GPU left: the region the
  // call uses is zeroed first, by a kernel (no memset node, so the call can
  // be captured into a graph).
  const int64_t words = int64_t(L.total / 16);
  (void)hipGetLastError();
  hipLaunchKernelGGL(sv::k_clear, dim3(unsigned((words + 255) / 256)), dim3(256), 0, st,
                     static_cast<uint4*>(ws), words);
  if ((rc = finish_launch()) != SPEC_OK) return rc;
  return spec_verify_stochastic(target, draft, draft_tokens, uniforms, B, k, V, sampling,
                                accepted_len, out_tokens, accept_prob, ws, kScratchBytes, stream);
}

int spec_verify_greedy(spec_logits_t target, const int32_t* draft_tokens, int32_t B, int32_t k,
                       int32_t V, int32_t* accepted_len, int32_t* out_tokens, void* workspace,
                       size_t workspace_bytes, void* stream) {
  int rc;
  if ((rc = check_sizes(B, k, V, true)) != SPEC_OK) return rc;
  if ((rc = check_logits(target, V)) != SPEC_OK) return rc;
  if (!draft_tokens || !accepted_len || !out_tokens) return SPEC_ERR_INVALID_ARG;
  const spec_sampling_t plain = {1.0f, 0, 1.0f};
  const Layout L = make_layout(SPEC_OP_GREEDY, B, k, V, &plain);
  if ((rc = check_workspace(workspace, workspace_bytes, L)) != SPEC_OK) return rc;
  if (!grid_fits(L.rows * L.nchunks, kRowThreads) || !grid_fits(B, 64)) return SPEC_ERR_UNSUPPORTED;
  sv::RowMap map{target.data, target.seq_stride, target.pos_stride, target.data, target.seq_stride,
                 target.pos_stride, k + 1, k + 1};
  auto* part = reinterpret_cast<sv::GPartial*>(static_cast<char*>(workspace) + L.part_off);
  auto st = static_cast<hipStream_t>(stream);
  (void)hipGetLastError();
  dispatch<GreedyRun>(target.dtype, vec_ok(target), L, map, int64_t(V), part, st);
  hipLaunchKernelGGL(sv::k_greedy_tail, dim3(unsigned(B)), dim3(64), 0, st, map, int64_t(V), k,
                     L.nchunks, draft_tokens, part, nullptr, nullptr, accepted_len, out_tokens);
  return finish_launch();
}

int spec_logits_process(spec_logits_t logits, int32_t R, int32_t V, const spec_sampling_t* sampling,
                        spec_row_stats_t* row_stats, float* probs, void* workspace,
                        size_t workspace_bytes, void* stream) {
  int rc;
  if ((rc = check_sizes(R, 1, V, false)) != SPEC_OK) return rc;
  if ((rc = check_sampling(sampling)) != SPEC_OK) return rc;
  logits.seq_stride = logits.pos_stride;  // row r lives at data + r * pos_stride
  if ((rc = check_logits(logits, V)) != SPEC_OK) return rc;
  const Layout L = make_layout(SPEC_OP_PROCESS, R, 1, V, sampling);
  if ((rc = check_workspace(workspace, workspace_bytes, L)) != SPEC_OK) return rc;
  if (!row_pass_fits(L, logits.dtype, vec_ok(logits)) || !grid_fits(L.rows * L.nchunks, kRowThreads))
    return SPEC_ERR_UNSUPPORTED;
  sv::RowMap map{logits.data, logits.pos_stride, 0, logits.data, logits.pos_stride, 0, 1, 1};
  const float a = log2e_over(sampling->temperature);
  auto st = static_cast<hipStream_t>(stream);
  (void)hipGetLastError();
  dispatch<ProcessRun>(logits.dtype, vec_ok(logits), L, map, int64_t(V), a, *sampling, row_stats,
                       probs, static_cast<char*>(workspace), st, device_cus(st));
  // Leave the workspace zero-filled, as the contract promises.
  const int64_t words = int64_t(L.total / 16);
  hipLaunchKernelGGL(sv::k_clear, dim3(unsigned((words + 255) / 256)), dim3(256), 0, st,
                     reinterpret_cast<uint4*>(workspace), words);
  return finish_launch();
}

size_t spec_workspace_size_pooled(int32_t op, int32_t n_target_rows, int32_t n_draft_rows,
                                  int32_t B, int32_t k, int32_t V,
                                  const spec_sampling_t* sampling) {
  if (op != SPEC_OP_STOCHASTIC && op != SPEC_OP_GREEDY) return 0;
  if (check_sizes(B, k, V, true) != SPEC_OK) return 0;
  const bool greedy = op == SPEC_OP_GREEDY;
  if (n_target_rows < 1 || (!greedy && n_draft_rows < 1)) return 0;
  spec_sampling_t plain = {1.0f, 0, 1.0f};
  if (!greedy) {
    if (check_sampling(sampling) != SPEC_OK) return 0;
  } else {
    sampling = &plain;
  }
  return make_pooled_layout(op, n_target_rows, greedy ? 0 : n_draft_rows, k, V, sampling).total;
}

int spec_verify_stochastic_pooled(spec_logits_t target_pool, int32_t n_target_rows,
                                  const int32_t* target_map, spec_logits_t draft_pool,
                                  int32_t n_draft_rows, const int32_t* draft_map,
                                  const int32_t* draft_tokens, const float* uniforms,
                                  int32_t B, int32_t k, int32_t V,
                                  const spec_sampling_t* sampling, int32_t* accepted_len,
                                  int32_t* out_tokens, float* accept_prob, void* workspace,
                                  size_t workspace_bytes, void* stream) {
  int rc;
  if ((rc = check_sizes(B, k, V, true)) != SPEC_OK) return rc;
  if ((rc = check_sampling(sampling)) != SPEC_OK) return rc;
  if ((rc = check_pools(n_target_rows, n_draft_rows, target_map, draft_map, B, k, true)) != SPEC_OK)
    return rc;
  target_pool.seq_stride = target_pool.pos_stride;  // pool row r at data + r * pos_stride
  draft_pool.seq_stride = draft_pool.pos_stride;
  if ((rc = check_logits(target_pool, V)) != SPEC_OK) return rc;
  if ((rc = check_logits(draft_pool, V)) != SPEC_OK) return rc;
  if (target_pool.dtype != draft_pool.dtype) return SPEC_ERR_INVALID_ARG;
  if (!draft_tokens || !uniforms || !accepted_len || !out_tokens) return SPEC_ERR_INVALID_ARG;
  const Layout L = make_pooled_layout(SPEC_OP_STOCHASTIC, n_target_rows, n_draft_rows, k, V, sampling);
  if ((rc = check_workspace(workspace, workspace_bytes, L)) != SPEC_OK) return rc;
  const bool vec = vec_ok(target_pool) && vec_ok(draft_pool);
  const int cus = device_cus(static_cast<hipStream_t>(stream));
  const int walk_grid =
      (target_pool.dtype == SPEC_DTYPE_BF16 && vec && int64_t(B) >= int64_t(kSeqPerCu) * cus)
          ? walk_grid_for(cus) : 0;
  if (!walk_grid && (!row_pass_fits(L, target_pool.dtype, vec) || !grid_fits(B, kTailThreads)))
    return SPEC_ERR_UNSUPPORTED;

  sv::RowMap map{target_pool.data, 0, target_pool.pos_stride, draft_pool.data, 0,
                 draft_pool.pos_stride, 2 * k + 1, k + 1, n_target_rows, n_draft_rows,
                 target_map, draft_map};
  sv::TailArgs args{};
  args.map = map;
  args.V = V;
  args.k = k;
  args.a = log2e_over(sampling->temperature);
  args.tokens = draft_tokens;
  args.u = uniforms;
  args.accepted_len = accepted_len;
  args.out_tokens = out_tokens;
  args.accept_prob = accept_prob;
  (void)hipGetLastError();
  dispatch<PooledStochasticRun>(target_pool.dtype, vec, L, map, int64_t(B), int64_t(V), args.a,
                                *sampling, args, static_cast<char*>(workspace),
                                static_cast<hipStream_t>(stream), walk_grid, cus);
  return finish_launch();
}

int spec_verify_greedy_pooled(spec_logits_t target_pool, int32_t n_target_rows,
                              const int32_t* target_map, const int32_t* draft_tokens,
                              int32_t B, int32_t k, int32_t V, int32_t* accepted_len,
                              int32_t* out_tokens, void* workspace, size_t workspace_bytes,
                              void* stream) {
  int rc;
  if ((rc = check_sizes(B, k, V, true)) != SPEC_OK) return rc;
  if ((rc = check_pools(n_target_rows, 0, target_map, nullptr, B, k, false)) != SPEC_OK) return rc;
  target_pool.seq_stride = target_pool.pos_stride;
  if ((rc = check_logits(target_pool, V)) != SPEC_OK) return rc;
  if (!draft_tokens || !accepted_len || !out_tokens) return SPEC_ERR_INVALID_ARG;
  const spec_sampling_t plain = {1.0f, 0, 1.0f};
  const Layout L = make_pooled_layout(SPEC_OP_GREEDY, n_target_rows, 0, k, V, &plain);
  if ((rc = check_workspace(workspace, workspace_bytes, L)) != SPEC_OK) return rc;
  if (!grid_fits(L.rows * L.nchunks, kRowThreads) || !grid_fits(B, 64)) return SPEC_ERR_UNSUPPORTED;
  sv::RowMap map{target_pool.data, 0, target_pool.pos_stride, target_pool.data, 0,
                 target_pool.pos_stride, k + 1, k + 1, n_target_rows, 0, target_map, nullptr};
  auto* part = reinterpret_cast<sv::GPartial*>(static_cast<char*>(workspace) + L.part_off);
  auto st = static_cast<hipStream_t>(stream);
  (void)hipGetLastError();
  dispatch<GreedyRun>(target_pool.dtype, vec_ok(target_pool), L, map, int64_t(V), part, st);
  hipLaunchKernelGGL(sv::k_greedy_tail, dim3(unsigned(B)), dim3(64), 0, st, map, int64_t(V), k,
                     L.nchunks, draft_tokens, part, nullptr, nullptr, accepted_len, out_tokens);
  // the pooled partials are shared by sequences: cleared after the tail
  const int64_t words = L.rows * L.nchunks;  // 16 bytes each
  hipLaunchKernelGGL(sv::k_clear, dim3(unsigned((words + 255) / 256)), dim3(256), 0, st,
                     reinterpret_cast<uint4*>(part), words);
  return finish_launch();
}

int spec_verify_greedy_lmhead(const void* hidden, int64_t hidden_seq_stride,
                              int64_t hidden_pos_stride, const void* weight,
                              int64_t weight_stride, int32_t d, const int32_t* draft_tokens,
                              int32_t B, int32_t k, int32_t V, int32_t* accepted_len,
                              int32_t* out_tokens, void* workspace, size_t workspace_bytes,
                              void* stream) {
  int rc;
  if ((rc = check_sizes(B, k, V, true)) != SPEC_OK) return rc;
  if (!hidden || !weight || !draft_tokens || !accepted_len || !out_tokens)
    return SPEC_ERR_INVALID_ARG;
  if (d < 32 || d % 32 != 0) return SPEC_ERR_INVALID_ARG;
  if (d > 65536) return SPEC_ERR_UNSUPPORTED;
  if (reinterpret_cast<uintptr_t>(hidden) % 16 || reinterpret_cast<uintptr_t>(weight) % 16)
    return SPEC_ERR_INVALID_ARG;
  if (hidden_seq_stride < 0 || hidden_pos_stride < 0 || hidden_seq_stride % 8 ||
      hidden_pos_stride % 8 || weight_stride < d || weight_stride % 8)
    return SPEC_ERR_INVALID_ARG;
  const size_t need = lmhead_workspace(B, k, V);
  if (!workspace || workspace_bytes < need || reinterpret_cast<uintptr_t>(workspace) % 256)
    return SPEC_ERR_WORKSPACE;
  const int64_t M = int64_t(B) * (k + 1);
  // Up to 64 rows: 256-entry tiles, fragments loaded straight from memory,
  // 16, 32 or 64 rows per chunk.  More rows: the LDS-staged tiling, two
  // workgroups per CU, 128 x 128 tiles in 64-wide stages up to 128 rows,
  // 128 x 256 tiles in 32-wide stages beyond (fewer LDS reads per product;
  // measured best of 128 x 128, 256 x 128 and 128 x 256 at 72 to 864 rows).
  const bool gemm = M > 64, wide = M > 128;
  // wide: 144-row tiles (the four waves side by side along the vocabulary)
  // where they leave fewer padded rows than 128-row tiles
  const bool rows144 = wide && (M + 143) / 144 * 144 < (M + 127) / 128 * 128;
  // 144-row tiles 192 or 256 entries wide: the chip runs two workgroups per
  // CU, so a call takes ceil(tiles / slots) rounds of workgroups; the narrower
  // tile does 3/4 of the work per round at ~7 % lower efficiency per entry
  // (measured 0.36 vs 0.46 ms at 144 rows, 0.77 vs 0.69 at 432, 1.40 vs 1.22
  // at 864), so it is taken when r192 * 0.75 * 1.07 < r256
  bool n192 = false;
  if (rows144) {
    const int64_t slots = 2 * int64_t(device_cus(static_cast<hipStream_t>(stream)));
    const int64_t ch = (M + 143) / 144;
    const int64_t r256 = ((int64_t(V) + 255) / 256 * ch + slots - 1) / slots;
    const int64_t r192 = ((int64_t(V) + 191) / 192 * ch + slots - 1) / slots;
    n192 = r192 * 321 < r256 * 400;
  }
  const int mb = M <= 16 ? 1 : (M <= 32 ? 2 : 4);
  const int64_t tw = gemm ? (n192 ? 192 : wide ? 256 : 128) : kLmTile,
                mr = gemm ? (rows144 ? 144 : 128) : 16 * mb;
  const int64_t tiles = (int64_t(V) + tw - 1) / tw;
  const int64_t chunks = (M + mr - 1) / mr;
  const int64_t nblk = tiles * chunks;
  const int64_t grid = (nblk + 7) / 8 * 8;
  if (!grid_fits(grid, 256) || !grid_fits(B, 64)) return SPEC_ERR_UNSUPPORTED;
  auto* best = static_cast<uint64_t*>(workspace);
  auto* bad = reinterpret_cast<uint32_t*>(static_cast<char*>(workspace) + lmhead_bad_off(M));
  sv::LmHeadArgs A{static_cast<const uint16_t*>(hidden), hidden_seq_stride, hidden_pos_stride,
                   k + 1, static_cast<const uint16_t*>(weight), weight_stride, M, int64_t(V), d,
                   int32_t(tiles), int32_t(chunks), best, bad};
  auto st = static_cast<hipStream_t>(stream);
  (void)hipGetLastError();
  if (gemm) {
    if (n192)
      hipLaunchKernelGGL((sv::k_lmhead_gemm_argmax<144, 192, 32, 1>), dim3(unsigned(grid)), dim3(256), 0, st, A);
    else if (rows144)
      hipLaunchKernelGGL((sv::k_lmhead_gemm_argmax<144, 256, 32, 1>), dim3(unsigned(grid)), dim3(256), 0, st, A);
    else if (wide)
      hipLaunchKernelGGL((sv::k_lmhead_gemm_argmax<128, 256, 32>), dim3(unsigned(grid)), dim3(256), 0, st, A);
    else
      hipLaunchKernelGGL((sv::k_lmhead_gemm_argmax<128, 128, 64>), dim3(unsigned(grid)), dim3(256), 0, st, A);
  } else switch (mb) {
    case 1: hipLaunchKernelGGL((sv::k_lmhead_argmax<1, 2, 4>), dim3(unsigned(grid)), dim3(256), 0, st, A); break;
    case 2: hipLaunchKernelGGL((sv::k_lmhead_argmax<2, 2, 4>), dim3(unsigned(grid)), dim3(256), 0, st, A); break;
    default: hipLaunchKernelGGL((sv::k_lmhead_argmax<4, 2, 4>), dim3(unsigned(grid)), dim3(256), 0, st, A); break;
  }
  // the greedy rule over the per-tile records (dense rows: b (k+1) + j)
  sv::RowMap map{nullptr, 0, 0, nullptr, 0, 0, k + 1, k + 1};
  hipLaunchKernelGGL(sv::k_greedy_tail, dim3(unsigned(B)), dim3(64), 0, st, map, int64_t(V), k, 1,
                     draft_tokens, nullptr, best, bad, accepted_len, out_tokens);
  return finish_launch();
}

int spec_logits_apply(spec_logits_t in, int32_t S, int32_t rows, int32_t V,
                      const spec_processors_t* proc, spec_logits_t out, void* stream) {
  int rc;
  if ((rc = check_sizes(S, 1, V, false)) != SPEC_OK) return rc;
  if (rows < 1) return SPEC_ERR_INVALID_ARG;
  if (rows > 2 * SPEC_MAX_K + 1) return SPEC_ERR_UNSUPPORTED;
  if (!proc) return SPEC_ERR_INVALID_ARG;
  if (!std::isfinite(proc->theta) || !(proc->theta > 0.0f)) return SPEC_ERR_INVALID_ARG;
  if ((rc = check_logits(in, V)) != SPEC_OK) return rc;
  if ((rc = check_logits(out, V)) != SPEC_OK) return rc;
  if (proc->allow_seq_stride < 0 || proc->allow_pos_stride < 0 || proc->pen_seq_stride < 0 ||
      proc->pen_pos_stride < 0)
    return SPEC_ERR_INVALID_ARG;
  const int64_t nch = (int64_t(V) + sv::kApplyChunk - 1) / sv::kApplyChunk;
  const int64_t blocks = int64_t(S) * rows * nch;
  if (!grid_fits(blocks, 256)) return SPEC_ERR_UNSUPPORTED;
  sv::ApplyArgs A{in.data, in.seq_stride, in.pos_stride, const_cast<void*>(out.data),
                  out.seq_stride, out.pos_stride, rows, int64_t(V), int(nch), proc->allow,
                  proc->allow_seq_stride, proc->allow_pos_stride, proc->penalize,
                  proc->pen_seq_stride, proc->pen_pos_stride, proc->theta};
  const bool vec = vec_ok(in) && vec_ok(out);
  auto st = static_cast<hipStream_t>(stream);
  const unsigned nblk = unsigned(blocks);
  (void)hipGetLastError();
  const bool ib = in.dtype == SPEC_DTYPE_BF16, ob = out.dtype == SPEC_DTYPE_BF16;
  if (ib && ob) launch_apply<uint16_t, uint16_t>(vec, nblk, A, st);
  else if (ib) launch_apply<uint16_t, float>(vec, nblk, A, st);
  else if (ob) launch_apply<float, uint16_t>(vec, nblk, A, st);
  else launch_apply<float, float>(vec, nblk, A, st);
  return finish_launch();
}

int spec_outcome_lookup(const int32_t* accepted_len, const int32_t* out_tokens, int32_t B,
                        int32_t k, const int32_t* pred_len, const int32_t* pred_token,
                        int32_t P, int32_t* hit_index, int32_t* hit_count, void* stream) {
  int rc;
  if ((rc = check_sizes(B, k, 1, true)) != SPEC_OK) return rc;
  if (P < 1) return SPEC_ERR_INVALID_ARG;
  if (P > 4096) return SPEC_ERR_UNSUPPORTED;
  if (!accepted_len || !out_tokens || !pred_len || !pred_token || !hit_index)
    return SPEC_ERR_INVALID_ARG;
  auto st = static_cast<hipStream_t>(stream);
  (void)hipGetLastError();
  hipLaunchKernelGGL(sv::k_outcome_lookup, dim3(unsigned((int64_t(B) + 3) / 4)), dim3(256), 0, st,
                     accepted_len, out_tokens, int64_t(B), k, pred_len, pred_token, P, hit_index);
  if (hit_count)
    hipLaunchKernelGGL(sv::k_count_hits, dim3(1), dim3(1024), 0, st, hit_index, int64_t(B),
                       hit_count);
  return finish_launch();
}

int spec_verify_stochastic_path(spec_logits_t target, spec_logits_t draft, int32_t B, int32_t k,
                                int32_t V, const spec_sampling_t* sampling, int32_t with_accept_prob,
                                void* stream) {
  int rc;
  if ((rc = check_sizes(B, k, V, true)) != SPEC_OK) return -rc;
  if ((rc = check_sampling(sampling)) != SPEC_OK) return -rc;
  if ((rc = check_logits(target, V)) != SPEC_OK) return -rc;
  if ((rc = check_logits(draft, V)) != SPEC_OK) return -rc;
  if (target.dtype != draft.dtype) return -SPEC_ERR_INVALID_ARG;
  const bool vec = vec_ok(target) && vec_ok(draft);
  return stochastic_path(target.dtype, vec, B, device_cus(static_cast<hipStream_t>(stream)),
                         with_accept_prob != 0);
}

int spec_device_cu_count(void* stream) { return device_cus(static_cast<hipStream_t>(stream)); }

const char* spec_status_string(int status) {
  switch (status) {
    case SPEC_OK: return "SPEC_OK";
    case SPEC_ERR_INVALID_ARG: return "SPEC_ERR_INVALID_ARG: invalid argument";
    case SPEC_ERR_UNSUPPORTED: return "SPEC_ERR_UNSUPPORTED: dtype or size outside the supported limits";
    case SPEC_ERR_WORKSPACE: return "SPEC_ERR_WORKSPACE: workspace missing, too small or misaligned";
    case SPEC_ERR_HIP: return "SPEC_ERR_HIP: a HIP launch or runtime call failed";
    default: return "unknown status";
  }
}

}  // extern "C"
