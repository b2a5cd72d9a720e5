/*
 * specverify.h -- C ABI of libspecverify, the speculative-decoding verify step
 * on one AMD Instinct MI355X (gfx950).
 *
 * The operation is the one stated in the encyclopedia entry "Speculative
 * decoding" (glopedia, 推测解码), section "Basic steps of proposal and
 * verification" (提议与核验的基本步骤):
 *   - a drafted token x at position j is accepted with probability
 *     min(1, p(x)/q(x)), where p (target) and q (proposer) are the
 *     conditional probabilities under the sampling settings in force;
 *   - acceptance stops at the first rejected position, which is redrawn from
 *     the normalised positive residual max(0, p - q);
 *   - when all k candidates pass, one extra (bonus) token is drawn from the
 *     target's next distribution;
 *   - greedy decoding compares each draft with the target's most probable
 *     token and replaces the first mismatch with it;
 *   - temperature, top-k and nucleus (top-p) settings are applied in the same
 *     way to p and q.
 *
 * Conventions (readings where the entry is silent):
 *   - target logits hold k+1 rows per sequence; row k is the bonus row;
 *   - uniforms are [B][k+1] floats in [0,1): column j < k is position j's
 *     accept draw (accept iff u < alpha), column k the one draw for the
 *     corrected or bonus token;
 *   - sampling is an inverse CDF in ascending vocabulary order (the first
 *     index whose running sum exceeds u * S);
 *   - alpha = 1 when q(x) = 0 < p(x) and 0 when both are 0;
 *   - a residual without mass falls back to p at that position;
 *   - processing order: z = (l - max l) / T, then top-k (keep every logit >=
 *     the top_k-th largest, duplicates counted), then top-p over the top-k
 *     probabilities (keep the shortest descending prefix whose mass reaches
 *     top_p; ties at the cut kept); a row's kept set is {l >= threshold};
 *   - greedy ties go to the lowest index; greedy ignores temperature/filters.
 *
 * Memory: every array argument is a DEVICE pointer unless marked "host".  The
 * caller owns all buffers; the library allocates nothing on these paths and
 * keeps no pointer after a call returns.  A call only enqueues work on
 * `stream` (a hipStream_t, NULL = the default stream) and never synchronises;
 * outputs are valid once the stream reaches that point.
 *
 * Errors: the return value reports argument validation and launch failures
 * (spec_status_t).  Data faults are reported per sequence with
 * accepted_len[b] = -1 and out_tokens[b][*] = -1.  A position is ill-formed
 * when its target row or draft row holds a NaN or +inf logit or no finite
 * logit, or its draft token lies outside [0, V).  Positions are walked in
 * order and the first rejection (greedy: mismatch) ends the walk; the
 * sequence is invalid when an ill-formed position comes before that end, or
 * when every position passes and the bonus row is invalid.  Rows past the
 * end are not consulted and cannot invalidate the sequence.  -inf logits are
 * allowed (vocabulary masking).
 */
#ifndef SPECVERIFY_H
#define SPECVERIFY_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  SPEC_OK = 0,
  SPEC_ERR_INVALID_ARG = 1, /* null pointer, bad size, bad setting, misaligned data */
  SPEC_ERR_UNSUPPORTED = 2, /* dtype or size outside the supported limits */
  SPEC_ERR_WORKSPACE = 3,   /* workspace missing, too small or misaligned */
  SPEC_ERR_HIP = 4          /* a HIP launch or runtime call failed */
} spec_status_t;

typedef enum { SPEC_DTYPE_F32 = 0, SPEC_DTYPE_BF16 = 1 } spec_dtype_t;

/* Limits: 1 <= k <= SPEC_MAX_K, 1 <= V <= SPEC_MAX_V, 1 <= B <= 2^24. */
#define SPEC_MAX_K 64
#define SPEC_MAX_V (1 << 24)

/* A logits tensor in device memory.  Element (b, j, x) lives at
 *   data[b * seq_stride + j * pos_stride + x]   (strides in elements).
 * seq_stride 0 broadcasts one sequence to all B; pos_stride >= V.  data must
 * be aligned to its element size; 16-byte aligned rows take the vector path. */
typedef struct {
  const void* data;
  int32_t dtype; /* spec_dtype_t */
  int32_t reserved;
  int64_t seq_stride;
  int64_t pos_stride;
} spec_logits_t;

/* Sampling settings (host struct), applied identically to target and draft. */
typedef struct {
  float temperature; /* finite, > 0 (greedy ignores it) */
  int32_t top_k;     /* 0 = off, else keep the top_k largest (>= V is off) */
  float top_p;       /* 1.0 = off, else in (0, 1) */
} spec_sampling_t;

/* Per-row result of spec_logits_process:
 *   p(x) = (l_x >= threshold) ? exp((l_x - max_logit) / T - log_norm) : 0.
 * valid = 0 marks a row with NaN/+inf or no finite logit (other fields NaN). */
typedef struct {
  float max_logit;
  float threshold; /* -inf when no filter is active */
  float log_norm;
  int32_t valid;
} spec_row_stats_t;

typedef enum {
  SPEC_OP_STOCHASTIC = 0,
  SPEC_OP_GREEDY = 1,
  SPEC_OP_PROCESS = 2,
  SPEC_OP_GREEDY_LMHEAD = 3
} spec_op_t;

/* Bytes of device workspace the given call needs (0 for invalid arguments).
 * For SPEC_OP_PROCESS, B is the row count R and k is ignored.  The
 * workspace must be zero-filled before its first use with this library and
 * left untouched by the caller between calls; every call leaves it
 * zero-filled when it completes.  Calls that share one workspace must be
 * ordered on one stream. */
size_t spec_workspace_size(int32_t op, int32_t B, int32_t k, int32_t V,
                           const spec_sampling_t* sampling /* host */);

/* Stochastic verify of B sequences with k drafted positions each.
 *   target        [B][k+1][V] logits (row k = bonus row)
 *   draft         [B][k][V] logits, same dtype as target
 *   draft_tokens  [B][k] int32, drawn by the proposer from the processed q
 *   uniforms      [B][k+1] float in [0,1)
 *   sampling      host struct, applied to both target and draft
 *   accepted_len  [B] int32 out: n = accepted draft count, or -1
 *   out_tokens    [B][k+1] int32 out: drafts 0..n-1, then the corrected (n<k)
 *                 or bonus (n=k) token, then -1 padding
 *   accept_prob   [B][k] float out or NULL: alpha_j for every j < k (also past
 *                 the first rejection); NaN at an ill-formed position
 *   workspace     device scratch of spec_workspace_size(SPEC_OP_STOCHASTIC...)
 *                 bytes, 256-byte aligned (see spec_workspace_size). */
int spec_verify_stochastic(spec_logits_t target, spec_logits_t draft,
                           const int32_t* draft_tokens, const float* uniforms,
                           int32_t B, int32_t k, int32_t V,
                           const spec_sampling_t* sampling,
                           int32_t* accepted_len, int32_t* out_tokens,
                           float* accept_prob, void* workspace,
                           size_t workspace_bytes, void* stream);

/* spec_verify_stochastic without a workspace argument, for callers that
 * cannot allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid allocation).  The call allocates nothing: its
 * kernels use a scratch array of SPEC_NOALLOC_SCRATCH_BYTES in the library's
 * own code object, one per GPU, held until the process ends.  The caller
 * still passes every input and output (device pointers, as in
 * spec_verify_stochastic, with the same results).
 * Limits: calls whose spec_workspace_size(SPEC_OP_STOCHASTIC, ...) exceeds
 * SPEC_NOALLOC_SCRATCH_BYTES return SPEC_ERR_UNSUPPORTED before anything is
 * enqueued.  The region a call uses is zeroed by a kernel at its start.
 * All calls on one GPU share that GPU's array: calls that may overlap on one
 * GPU (other streams, other host threads) race and must be ordered by the
 * caller.  SPEC_ERR_HIP if the array's device address cannot be obtained. */
#define SPEC_NOALLOC_SCRATCH_BYTES (16u << 20)
int spec_verify_stochastic_noalloc(spec_logits_t target, spec_logits_t draft,
                                   const int32_t* draft_tokens, const float* uniforms,
                                   int32_t B, int32_t k, int32_t V,
                                   const spec_sampling_t* sampling, int32_t* accepted_len,
                                   int32_t* out_tokens, float* accept_prob, void* stream);

/* Greedy verify: a*_j = argmax_x target[b][j][x] (lowest index on ties);
 * n = first j < k with draft_tokens[b][j] != a*_j, else k; out_tokens gets
 * the n matching drafts, then a*_n, then -1 padding. */
int spec_verify_greedy(spec_logits_t target, const int32_t* draft_tokens,
                       int32_t B, int32_t k, int32_t V, int32_t* accepted_len,
                       int32_t* out_tokens, void* workspace,
                       size_t workspace_bytes, void* stream);

/* Logits processing of R rows (row r at data + r * pos_stride; seq_stride is
 * ignored): per-row statistics and, if probs != NULL, the dense fp32
 * probabilities [R][V] (row-major, stride V).  Either output may be NULL. */
int spec_logits_process(spec_logits_t logits, int32_t R, int32_t V,
                        const spec_sampling_t* sampling,
                        spec_row_stats_t* row_stats, float* probs,
                        void* workspace, size_t workspace_bytes, void* stream);

/* Pooled rows: verify with rows shared by several sequences.
 *
 * The encyclopedia entry "Speculative decoding" (glopedia, 推测解码), section
 * "Proposal methods and implementation forms" (提议方式与实现形态), names
 * candidate trees beside chains; the predicted-outcome sets of "Speculative
 * Speculative Decoding" (ai-stack.site summary, section 1 on its novelty,
 * 研究创新性) hold several candidate outcomes per request.  Sequences (branches, or the
 * root-to-leaf paths of a candidate tree) then share rows: the branches of
 * one request share its target rows, and the paths through a tree node share
 * that node's rows.  Each shared row is stored and processed once.
 *
 * Reading (the pages give no rule for combining branches): every sequence is
 * verified on its own by the chain rule above, on the rows its maps name; an
 * out-of-range map entry makes that row ill-formed (a data fault at a
 * consulted position, as above).
 *
 *   target_pool   n_target_rows rows of V logits, row r at
 *                 data + r * pos_stride (seq_stride is ignored)
 *   target_map    [B][k+1] int32: pool row of target row j of sequence b;
 *                 NULL = row b * (k+1) + j (needs n_target_rows >= B (k+1))
 *   draft_pool    n_draft_rows rows, as target_pool, same dtype
 *   draft_map     [B][k] int32: pool row of draft row j of sequence b;
 *                 NULL = row b * k + j (needs n_draft_rows >= B k)
 * The other arguments are those of spec_verify_stochastic, with a workspace
 * of spec_workspace_size_pooled(SPEC_OP_STOCHASTIC, ...) bytes.  Pool sizes:
 * 1 <= n_target_rows, n_draft_rows <= 2^31 - 1. */
size_t spec_workspace_size_pooled(int32_t op, int32_t n_target_rows, int32_t n_draft_rows,
                                  int32_t B, int32_t k, int32_t V,
                                  const spec_sampling_t* sampling /* host */);

int spec_verify_stochastic_pooled(spec_logits_t target_pool, int32_t n_target_rows,
                                  const int32_t* target_map, spec_logits_t draft_pool,
                                  int32_t n_draft_rows, const int32_t* draft_map,
                                  const int32_t* draft_tokens, const float* uniforms,
                                  int32_t B, int32_t k, int32_t V,
                                  const spec_sampling_t* sampling, int32_t* accepted_len,
                                  int32_t* out_tokens, float* accept_prob, void* workspace,
                                  size_t workspace_bytes, void* stream);

/* Greedy verify over pooled target rows (target_pool and target_map as in
 * spec_verify_stochastic_pooled); the workspace is
 * spec_workspace_size_pooled(SPEC_OP_GREEDY, n_target_rows, 0, B, k, V, NULL). */
int spec_verify_greedy_pooled(spec_logits_t target_pool, int32_t n_target_rows,
                              const int32_t* target_map, const int32_t* draft_tokens,
                              int32_t B, int32_t k, int32_t V, int32_t* accepted_len,
                              int32_t* out_tokens, void* workspace, size_t workspace_bytes,
                              void* stream);

/* Fused LM head + greedy verify.  The target processes the prefix extended
 * by the candidates once and gets its distribution at every drafted position
 * (the entry's section "Basic steps of proposal and verification"): its
 * logits are the
 * hidden states times the LM head, logits[b][j][v] = sum_c hidden[b][j][c] *
 * weight[v][c].  This call computes them tile by tile on the matrix cores
 * (bf16 inputs, fp32 accumulation) and reduces each row to its argmax
 * (lowest index on ties) without writing the logits to memory, then runs the
 * greedy rule of spec_verify_greedy.
 *   hidden        [B][k+1][d] bf16, row (b, j) at hidden + b * hidden_seq_stride
 *                 + j * hidden_pos_stride (elements; multiples of 8; 16-byte aligned)
 *   weight        [V][d] bf16, row v at weight + v * weight_stride (>= d, a
 *                 multiple of 8; 16-byte aligned) -- the LM head as stored
 *   d             hidden size, a multiple of 32, 32 <= d <= 65536
 * Workspace: spec_workspace_size(SPEC_OP_GREEDY_LMHEAD, B, k, V, NULL).
 * Reading: the argmax is taken on fp32 logits; where two logits lie within
 * the fp32 rounding of their sums, either may be reported. */
int spec_verify_greedy_lmhead(const void* hidden, int64_t hidden_seq_stride,
                              int64_t hidden_pos_stride, const void* weight,
                              int64_t weight_stride, int32_t d, const int32_t* draft_tokens,
                              int32_t B, int32_t k, int32_t V, int32_t* accepted_len,
                              int32_t* out_tokens, void* workspace, size_t workspace_bytes,
                              void* stream);

/* Logits processors applied before verification.  The encyclopedia entry's
 * section "Basic steps of proposal and verification" requires the target and
 * proposal distributions to be computed under every processing rule in force
 * -- naming repetition penalty, vocabulary masking and structured-output
 * constraints beside temperature, top-k and nucleus -- and consistently in
 * the correction step.  spec_logits_apply applies the first three to rows of
 * logits; applying the same processor rows to the target and draft logits of
 * a position, then calling a verify entry point, meets that requirement.
 *
 * Bitmask rows: bit (x % 32) of word (x / 32) refers to token x; the row of
 * (s, j) starts at words + s * seq_stride + j * pos_stride (strides in
 * 32-bit words; 0 broadcasts).  A structured-output constraint is a
 * per-position allow mask.
 *
 * Readings: a token whose allow bit is 0 gets logit -inf; a token whose
 * penalise bit is 1 (one already in the sequence's history) gets l / theta
 * if l > 0, else l * theta (the repetition penalty of Keskar et al., 2019),
 * computed in fp32; masking comes first; NaN and +inf pass unchanged (the
 * verify marks such rows invalid).  A bf16 output rounds to nearest even. */
typedef struct {
  const uint32_t* allow;     /* allow-mask rows, or NULL (every token allowed) */
  int64_t allow_seq_stride;  /* words */
  int64_t allow_pos_stride;  /* words */
  const uint32_t* penalize;  /* penalise-mask rows, or NULL (no penalty) */
  int64_t pen_seq_stride;    /* words */
  int64_t pen_pos_stride;    /* words */
  float theta;               /* repetition penalty, finite and > 0 (1 = none) */
} spec_processors_t;

/* Applies the processors to S x rows logits rows: row (s, j) of `in`
 * (spec_logits_t addressing) is processed with bitmask row (s, j) and written
 * to row (s, j) of `out` (F32 or BF16; out may be in itself, same strides).
 * 1 <= S <= 2^24, 1 <= rows <= 2 * SPEC_MAX_K + 1, 1 <= V <= SPEC_MAX_V. */
int spec_logits_apply(spec_logits_t in, int32_t S, int32_t rows, int32_t V,
                      const spec_processors_t* proc /* host */, spec_logits_t out,
                      void* stream);

/* Predicted-outcome lookup, the step after verify in speculative
 * speculative decoding ("Speculative Speculative Decoding", ai-stack.site
 * summary, section 1 on its novelty, 研究创新性, and section 2 on its
 * theory, 理论贡献与关键假设): while the target verifies, the proposer
 * prepares drafts for a set of likely verification outcomes; when the actual
 * outcome is in the set the prepared draft is used at once (a hit), and the
 * share of hits is the speculation cache hit rate.
 *
 * Reading: the outcome of sequence b is the pair (n, t) with n =
 * accepted_len[b] and t = out_tokens[b][n] (the corrected or bonus token);
 * with the drafts fixed it determines the emitted string.
 *   accepted_len  [B] int32, out_tokens [B][k+1] int32: a verify call's outputs
 *   pred_len      [B][P] int32: predicted accepted lengths; an entry < 0 is empty
 *   pred_token    [B][P] int32: predicted emitted tokens
 *   hit_index     [B] int32 out: the first i with pred_len[b][i] == n and
 *                 pred_token[b][i] == t, or -1 (also -1 for an invalid
 *                 sequence, n < 0, and for n > k)
 *   hit_count     [1] int32 out or NULL: the number of sequences with a hit
 * 1 <= B <= 2^24, 1 <= k <= SPEC_MAX_K, 1 <= P <= 4096.  No workspace. */
int spec_outcome_lookup(const int32_t* accepted_len, const int32_t* out_tokens, int32_t B,
                        int32_t k, const int32_t* pred_len, const int32_t* pred_token,
                        int32_t P, int32_t* hit_index, int32_t* hit_count, void* stream);

/* Kernel paths of a stochastic verify call (spec_verify_stochastic_path). */
typedef enum {
  SPEC_PATH_ROW_PASS = 0,      /* a pass over every row, then one tail per sequence */
  SPEC_PATH_TASK_QUEUE = 1,    /* one kernel of position tasks, rows read in walk order */
  SPEC_PATH_SEQUENCE_WALK = 2  /* one kernel walking whole sequences (accept_prob asked for) */
} spec_path_t;

/* The path spec_verify_stochastic takes for these arguments on the device of
 * `stream` (nothing is launched; the logits' data is not read): aligned bf16
 * rows (16-byte aligned base and strides) in batches of at least two
 * sequences per compute unit are read in walk order by one kernel, the
 * task queue or, when accept_prob is requested (with_accept_prob != 0), the
 * whole-sequence walk; other calls take the row pass.  Returns a
 * spec_path_t, or minus a spec_status_t for arguments the call would
 * reject (sizes, settings, logits descriptors). */
int spec_verify_stochastic_path(spec_logits_t target, spec_logits_t draft, int32_t B, int32_t k,
                                int32_t V, const spec_sampling_t* sampling /* host */,
                                int32_t with_accept_prob, void* stream);

/* The compute-unit count the library sizes its grids by on the device of
 * `stream` (NULL: the current device): queried once per device and kept
 * until the process ends; 256 when no device can be queried. */
int spec_device_cu_count(void* stream);

/* Static description of a status code. */
const char* spec_status_string(int status);

#ifdef __cplusplus
}
#endif
#endif /* SPECVERIFY_H */
