/*
 * moe_oracle.h -- CPU oracle for the local MoE expert layer (TEST INFRASTRUCTURE ONLY).
 *
 * This is a plain, slow, fp64 reference of what the GPU path computes. Only the
 * test suite, the smoke check and the CPU-baseline leg of the benchmark may load
 * it. The product library never links, loads or calls it, and it shares no code,
 * header, table or constant with the HIP path.
 *
 * Sources (web pages this follows):
 *  - GitHub issue "End-to-end DeepEP v2 non-expand + SonicMoE integration"
 *    (Dao-AILab/sonic-moe #68): the non-expand inputs x [N,H], topk_idx [N,K]
 *    (-1 = invalid slot), topk_weights [N,K]; the seven metadata arrays
 *    (expert_frequency, expert_frequency_offset, x_gather_idx, s_scatter_idx,
 *    s_reverse_scatter_idx, num_activated_expert_per_token_offset, compact
 *    router_scores [P]); the token-major compact pair list with ascending
 *    token_indices; the local output [N_recv,H]; question 4 on router-score
 *    gradients in [N_recv,K] layout.
 *  - Hysen Labs page on Dao-AILab/sonic-moe, sections "The MoE class takes a
 *    routing count and a kernel backend" (SwiGLU, no bias) and "Interleaved by
 *    default, concatenated if your model is HuggingFace" (gate0, up0, gate1, up1).
 *  - Qwen3.6 serving-script commit notes, "Optimization (CCCL segmented-sort
 *    pattern)" steps 1-5: flatten pairs, sort by expert, contiguous per-expert
 *    inputs, silu x up, one scatter-add back.
 *  - AWS NKI unpermute_a2av reference: scatter-add of expert rows back to token
 *    positions, accumulating over top-k contributions.
 *
 * Readings where the pages are silent (pair order, sort stability, direction of
 * the scatter indices, dtypes) are listed with the function that uses them.
 *
 * Parity pins: every function here is checked in tests/ against a construction
 * that does not reuse its code (brute force, textbook stable sort, exhaustive
 * enumeration, dense-MLP special case, central finite differences). No function
 * is "parity unpinned".
 *
 * Conventions: all index arrays int32; all sizes int64_t; tensors row-major.
 * Floating-point inputs of the sampled entry points are passed as (pointer,
 * dtype code): ORACLE_BF16 = raw bf16 bit patterns (uint16), ORACLE_F32,
 * ORACLE_F64. Results are always fp64 and never rounded.
 */
#ifndef MOE_ORACLE_H
#define MOE_ORACLE_H
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum { ORACLE_BF16 = 0, ORACLE_F32 = 1, ORACLE_F64 = 2 };
enum { ORACLE_FLAG_BAD_EXPERT = 1u };

/* Metadata (routing) from the non-expand [N,K] layout. Returns P.
 * Output arrays sized: freq [E], foff [E+1], x_gather/s_scatter/s_rev/
 * router_scores/pair_token/pair_slot/pair_expert [N*K] (only [0,P) written),
 * tok_off [N+1]. Any of pair_token/pair_slot/pair_expert may be NULL. */
int64_t oracle_build_metadata(int64_t N, int64_t K, int64_t E,
                              const int32_t *topk_idx, const float *topk_weights,
                              int32_t *expert_frequency, int32_t *expert_frequency_offset,
                              int32_t *x_gather_idx, int32_t *s_scatter_idx,
                              int32_t *s_reverse_scatter_idx,
                              int32_t *num_activated_expert_per_token_offset,
                              float *router_scores,
                              int32_t *pair_token, int32_t *pair_slot, int32_t *pair_expert,
                              uint32_t *flags);

/* Full forward on fp64 tensors (small sizes). x [N,H], w_up [E,H,2I]
 * (interleaved gate/up columns), w_down [E,I,H]. Metadata as produced by
 * oracle_build_metadata. Writes h [P,2I], a [P,I], y [P,H], out [N,H]. */
void oracle_forward(int64_t N, int64_t H, int64_t I, int64_t E,
                    const double *x, const double *w_up, const double *w_down,
                    const int32_t *expert_frequency_offset, const int32_t *x_gather_idx,
                    const int32_t *s_reverse_scatter_idx,
                    const int32_t *num_activated_expert_per_token_offset,
                    const float *router_scores,
                    double *h, double *a, double *y, double *out);

/* Full backward on fp64 tensors (small sizes). Consumes the forward's h, a, y.
 * Writes dx [N,H], dw_up [E,H,2I], dw_down [E,I,H], d_topk_weights [N,K]. */
void oracle_backward(int64_t N, int64_t K, int64_t H, int64_t I, int64_t E,
                     const double *x, const double *w_up, const double *w_down,
                     const double *dout,
                     const int32_t *expert_frequency_offset, const int32_t *x_gather_idx,
                     const int32_t *s_scatter_idx, const int32_t *s_reverse_scatter_idx,
                     const int32_t *num_activated_expert_per_token_offset,
                     const float *router_scores,
                     const int32_t *pair_token, const int32_t *pair_slot,
                     const double *h, const double *a, const double *y,
                     double *dx, double *dw_up, double *dw_down, double *d_topk_weights);

/* Brute force forward, independent of the metadata: for every token and every
 * valid slot, out[t] += w[t,k] * down_e(SwiGLU(up_e(x[t]))). fp64 tensors. */
void oracle_bruteforce_forward(int64_t N, int64_t K, int64_t H, int64_t I, int64_t E,
                               const double *x, const int32_t *topk_idx,
                               const float *topk_weights,
                               const double *w_up, const double *w_down, double *out);

/* ---- Sampled entry points (any size; typed inputs) ---------------------- */

/* For each token in tokens[0..n_tok): out row [H] (forward combine), and if
 * dout != NULL also dx row [H] and d_topk_weights row [K]. Outputs are packed
 * per listed token: out_rows [n_tok,H], dx_rows [n_tok,H], dtw_rows [n_tok,K]. */
void oracle_sample_tokens(int64_t N, int64_t K, int64_t H, int64_t I, int64_t E,
                          const void *x, int x_dt, const void *w_up, int w_dt,
                          const void *w_down, const void *dout, int dout_dt,
                          const int32_t *topk_idx, const float *topk_weights,
                          int64_t n_tok, const int64_t *tokens,
                          double *out_rows, double *dx_rows, double *dtw_rows);

/* Saved activation rows h[s,:] [2I] for listed sorted positions s. */
void oracle_sample_h_rows(int64_t H, int64_t I, int64_t E,
                          const void *x, int x_dt, const void *w_up, int w_dt,
                          const int32_t *expert_frequency_offset, const int32_t *x_gather_idx,
                          int64_t n_rows, const int64_t *rows, double *h_rows);

/* Rows dw_down[e, j, :] [H] for listed (e, j). */
void oracle_sample_dw_down_rows(int64_t H, int64_t I, int64_t E,
                                const void *x, int x_dt, const void *w_up, int w_dt,
                                const void *dout, int dout_dt,
                                const int32_t *expert_frequency_offset,
                                const int32_t *x_gather_idx, const int32_t *s_scatter_idx,
                                const float *router_scores,
                                int64_t n, const int64_t *e_list, const int64_t *j_list,
                                double *rows);

/* Column pairs dw_up[e, :, 2jj] and dw_up[e, :, 2jj+1] for listed (e, jj);
 * written as cols [n, 2, H]. */
void oracle_sample_dw_up_cols(int64_t H, int64_t I, int64_t E,
                              const void *x, int x_dt, const void *w_up, int w_dt,
                              const void *w_down, const void *dout, int dout_dt,
                              const int32_t *expert_frequency_offset,
                              const int32_t *x_gather_idx, const int32_t *s_scatter_idx,
                              const float *router_scores,
                              int64_t n, const int64_t *e_list, const int64_t *jj_list,
                              double *cols);

/* Router ahead of the metadata (Hysen Labs page on Dao-AILab/sonic-moe, section
 * "Three routing strategies, selected on the command line"). Per token t, the K
 * experts with the largest logits, listed largest first (reading: equal logits go
 * to the lower expert id), with weights
 *   mode 0, softmax over the top-K logits:  w_k = exp(l_k) / sum over the K of exp(l);
 *   mode 1, top-K of the softmax over all E: w_k = exp(l_k) / sum over all E of exp(l),
 *           divided by the sum of the K selected values when renormalize != 0.
 * Selecting by logits equals selecting by softmax probabilities (softmax is
 * increasing); the choice is made exactly on the given values.
 * aux (reading: the page names the auxiliary load-balancing loss the layer returns,
 * without a formula; this is the usual load-balancing product form):
 *   aux = E * sum_e f_e * P_e,  f_e = (slots routed to e) / (N*K),
 *   P_e = (1/N) * sum_t softmax over all E of logits[t,:], at e.
 * logits [N,E] typed (ORACLE_BF16 / F32 / F64). Outputs topk_idx [N,K],
 * topk_weights [N,K] (fp64), *aux (0 when N = 0). Requires 1 <= K <= E. */
void oracle_route(int64_t N, int64_t E, int64_t K, const void *logits, int logits_dt, int mode,
                  int renormalize, int32_t *topk_idx, double *topk_weights, double *aux);

/* Threads the OpenMP loops use (for the benchmark's CPU-baseline report). */
int oracle_num_threads(void);

#ifdef __cplusplus
}
#endif
#endif
