/*
 * oracle.h -- interface of the CPU oracle for the speculative-decoding verify
 * step.  TEST INFRASTRUCTURE: only the test suite, the package smoke check and
 * the benchmark's CPU-baseline leg may load this code.  It shares no source,
 * header or constant with the GPU library (its structs, decoding and
 * arithmetic are its own).
 *
 * All logits are HOST pointers.  A logits tensor is addressed as
 *   element(b, j, x) = base[b * seq_stride + j * pos_stride + x]
 * with strides counted in elements (seq_stride may be 0 to broadcast one
 * sequence to every b).  dtype ORC_F32 means IEEE binary32, ORC_BF16 means the
 * upper 16 bits of a binary32 (bfloat16), both decoded exactly to double.
 */
#ifndef SPECVERIFY_ORACLE_H
#define SPECVERIFY_ORACLE_H

#ifdef __cplusplus
extern "C" {
#endif

#define ORC_F32 0
#define ORC_BF16 1

/* Boundary-detector bits (per sequence), judged on the oracle's fp64 values. */
#define ORC_NEAR_ACCEPT 1 /* some accept draw u_j lies within 1e-6 of alpha_j   */
#define ORC_NEAR_SAMPLE 2 /* the sample draw lies within 1e-6 of a CDF breakpoint */
#define ORC_NEAR_TOPP 4   /* a top-p cumulative mass at the cut is within 1e-6 of top_p */

/* Process one row of V logits (temperature -> top-k -> top-p -> normalise).
 * prob (V doubles, may be NULL) receives p; stats (5 doubles, may be NULL)
 * receives {max logit, threshold logit, log normaliser, top-p mass strictly
 * above the cut value, top-p mass at or above the cut value} (the last two are
 * NaN when top-p is off).  Returns 1 for a valid row, 0 for an invalid one
 * (NaN, +inf, or no finite logit). */
int orc_process_row(const void* row, int dtype, int V, double temperature,
                    int top_k, double top_p, double* prob, double* stats);

/* Inverse-CDF draw from the processed distribution of one row with uniform u:
 * the smallest index whose running sum (ascending vocabulary order) exceeds
 * u * total.  Returns -1 for an invalid row. */
int orc_sample_row(const void* row, int dtype, int V, double temperature,
                   int top_k, double top_p, double u);

/* Index of the first maximum of a row (-1 for an invalid row). */
int orc_argmax_row(const void* row, int dtype, int V);

/* Stochastic verify of B sequences with k drafted positions each.
 * target: [B][k+1][V], draft: [B][k][V] (same dtype), tokens: [B][k],
 * u: [B][k+1] (columns 0..k-1 accept draws, column k the sample draw).
 * Outputs: accepted_len [B] (-1 for an invalid sequence), out_tokens [B][k+1]
 * (accepted drafts, then the emitted token, then -1 padding), accept_prob
 * [B][k] (alpha_j for every j; may be NULL), flags [B] (boundary bits; may be
 * NULL).  Returns 0, or -1 on an allocation failure. */
int orc_verify_stochastic(const void* target, long long t_seq, long long t_pos,
                          const void* draft, long long d_seq, long long d_pos,
                          int dtype, const int* tokens, const float* u, int B,
                          int k, int V, double temperature, int top_k,
                          double top_p, int* accepted_len, int* out_tokens,
                          double* accept_prob, int* flags);

/* Greedy verify: argmax compare, first mismatch replaced by the target's
 * argmax; if all k match, the argmax of target row k is appended. */
int orc_verify_greedy(const void* target, long long t_seq, long long t_pos,
                      int dtype, const int* tokens, int B, int k, int V,
                      int* accepted_len, int* out_tokens);

#ifdef __cplusplus
}
#endif
#endif
