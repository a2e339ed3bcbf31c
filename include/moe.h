/*
 * moe.h -- C ABI of the MI355X (gfx950) local MoE expert layer.
 *
 * One expert-parallel rank's local expert compute, taken from the DeepEP-style
 * non-expand layout that GitHub issue #68 on Dao-AILab/sonic-moe ("End-to-end
 * DeepEP v2 non-expand + SonicMoE integration") describes:
 *   x [N,H], topk_idx [N,K] (local expert id, -1 = invalid slot),
 *   topk_weights [N,K]  ->  local_out [N,H],
 * with the routing metadata built directly from [N,K] on the device (no host
 * sync, no materialised [P] pair list), a gathered grouped up-projection GEMM
 * with fused SwiGLU, a grouped down-projection GEMM, a deterministic
 * router-weighted combine, and the backward pass including the router-weight
 * gradient in [N,K] layout (question 4 of that issue).
 *
 * Memory and ownership
 *  - Every tensor pointer is a DEVICE pointer; the caller allocates and owns all
 *    memory (inputs, outputs, metadata arrays, workspace). No call allocates,
 *    frees, synchronises, or reads device memory on the host.
 *  - Every call only enqueues kernels on `stream` (a hipStream_t; NULL is the
 *    null stream) and returns; results are ready when the stream reaches them.
 *  - Tensors are dense and row-major. Index arrays are int32.
 *
 * Errors
 *  - Argument errors (null required pointer, bad sizes, short workspace,
 *    unsupported shape or dtype) are returned synchronously, before anything is
 *    enqueued. A launch failure returns MOE_EHIP.
 *  - Data errors never abort: they set bits in meta->status on the device
 *    (MOE_DEV_*), which the caller reads whenever it next synchronises.
 *    An expert id outside [-1,E) is treated as -1. If the pair count P exceeds
 *    meta->capacity, metadata entries at positions >= capacity are dropped and
 *    forward/backward write zeros to out, dx, dw_up, dw_down, d_topk_weights.
 *
 * Concurrency: calls that share a workspace or metadata object must be ordered
 * on one stream.
 */
#ifndef MOE_H
#define MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MOE_OK = 0,
  MOE_EINVAL = 1,       /* bad argument */
  MOE_ENOSPC = 2,       /* workspace smaller than the matching *_workspace() query */
  MOE_EUNSUPPORTED = 3, /* shape/dtype/layout this library does not implement */
  MOE_EHIP = 4          /* a HIP launch failed */
} moe_status;

/* Element type of x, weights, saved activations, outputs and gradients.
 * topk_weights, router_scores and d_topk_weights are always fp32. */
typedef enum {
  MOE_BF16 = 0, /* bf16 storage, fp32 accumulation (matrix cores) */
  MOE_FP32 = 1  /* fp32 storage and arithmetic: the checking mode */
} moe_dtype;

/* Column order of W_up [E,H,2I] (and of dW_up):
 *  INTERLEAVED: column 2j = gate_j, 2j+1 = up_j (the Hysen Labs page on SonicMoE: the
 *               interleaved format is the default);
 *  CONCAT:      columns [0,I) = gates, [I,2I) = ups (the concatenated gate/up format of
 *               HF-style checkpoints that page contrasts it with).
 * The saved activation h_save is always stored interleaved: it is written by the
 * forward and read only by the backward of this library. */
typedef enum { MOE_GATEUP_INTERLEAVED = 0, MOE_GATEUP_CONCAT = 1 } moe_gateup_layout;

/* Device status bits, OR-ed into *meta->status (zeroed by moe_build_metadata). */
enum { MOE_DEV_BAD_EXPERT = 1u, MOE_DEV_OVER_CAPACITY = 2u };

/* Limits of this library (checked synchronously). */
enum { MOE_MAX_EXPERTS = 1024, MOE_MAX_TOPK = 64 };

/* Routing metadata (GitHub issue #68, the list of arrays SonicMoE's grouped GEMM
 * needs). A host struct holding device pointers, all caller-owned.
 * Pairs are the valid slots of topk_idx taken token-major, ascending slot k
 * within a token; q in [0,P) is that pair index. Sorted position s in [0,P)
 * orders pairs by expert, stably (ascending q within an expert). */
typedef struct {
  int32_t N, K, E;  /* rows, slots per row, local experts */
  int32_t capacity; /* length of the [capacity] arrays (pointers may be NULL when
                       0); P <= capacity <= N*K (pass DeepEP's total_pairs) */
  int32_t *expert_frequency;        /* [E]   pairs per expert */
  int32_t *expert_frequency_offset; /* [E+1] exclusive scan; [E] = P */
  int32_t *x_gather_idx;            /* [capacity] s -> token row of x */
  int32_t *s_scatter_idx;           /* [capacity] s -> pair q */
  int32_t *s_reverse_scatter_idx;   /* [capacity] q -> s */
  int32_t *num_activated_expert_per_token_offset; /* [N+1] exclusive scan of
                                                     valid slots per row; [N] = P */
  float *router_scores;             /* [capacity] q -> topk_weights[t,k] */
  uint32_t *status;                 /* [1] MOE_DEV_* bits */
} moe_metadata;

/* Workspace byte counts. Zero means no workspace is needed. */
size_t moe_build_metadata_workspace(int32_t N, int32_t K, int32_t E);
size_t moe_route_workspace(int32_t N, int32_t K, int32_t E);
size_t moe_expert_forward_workspace(const moe_metadata *meta, int32_t H, int32_t I,
                                    moe_dtype dt);
size_t moe_expert_backward_workspace(const moe_metadata *meta, int32_t H, int32_t I,
                                     moe_dtype dt);

/* Builds every array of *meta from topk_idx [N,K] (int32) and topk_weights [N,K]
 * (fp32), and zeroes-then-sets meta->status. The pair count P stays on the
 * device (expert_frequency_offset[E] and num_activated_expert_per_token_offset[N]).
 * Steps: per-block expert histograms (LDS counters), a cross-block scan, then a
 * stable counting-sort scatter ranked inside wavefronts (Qwen3.6 serving-script notes,
 * "Optimization (CCCL segmented-sort pattern)", steps 1-3).
 * Requires 1 <= K <= MOE_MAX_TOPK, 1 <= E <= MOE_MAX_EXPERTS, N >= 0,
 * N*K < 2^31, 0 <= capacity. */
moe_status moe_build_metadata(const int32_t *topk_idx, const float *topk_weights,
                              const moe_metadata *meta, void *workspace,
                              size_t workspace_bytes, void *stream);

/* Allocation-free variant of moe_build_metadata, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc). Same arguments without the workspace, same kernels and the same
 * results: the workspace is a library-owned static device array of
 * MOE_NOALLOC_SCRATCH_BYTES on each GPU (held until the process ends), on the GPU
 * current for the calling thread (the stream must belong to it). A build whose
 * workspace would exceed that (moe_build_metadata_workspace(N, K, E) >
 * MOE_NOALLOC_SCRATCH_BYTES) returns MOE_ENOSPC before anything is enqueued; argument
 * errors as for moe_build_metadata; MOE_EHIP if the array's address cannot be found.
 * Allocates and frees nothing. Every call on one GPU shares that GPU's array, which
 * keeps the last call's contents (no part of it needs to start zeroed): calls that
 * overlap on one GPU (other streams, or unordered host threads) race on it and must
 * not be issued; calls ordered on one stream are safe. */
enum { MOE_NOALLOC_SCRATCH_BYTES = 4 << 20 };
moe_status moe_build_metadata_noalloc(const int32_t *topk_idx, const float *topk_weights,
                                      const moe_metadata *meta, void *stream);

/* Router top-K from logits, fused with the metadata build (the Hysen Labs page on
 * Dao-AILab/sonic-moe, section "Three routing strategies, selected on the command
 * line": softmax over the top-K logits, or top-K over the softmax of all experts with
 * optional renormalisation; the layer also returns an auxiliary load-balancing loss).
 *  logits        [N,E] bf16 or fp32 (logits_dtype), N, K, E taken from *meta; K <= E.
 *  topk_idx      [N,K] int32 out: per token the K experts with the largest logits,
 *                largest first; equal logits go to the lower expert id.
 *  topk_weights  [N,K] fp32 out: MOE_ROUTE_SOFTMAX_TOPK: exp(l_k) / sum over the K;
 *                MOE_ROUTE_TOPK_SOFTMAX: exp(l_k) / sum over all E, divided by the
 *                sum of the K when renormalize != 0.
 *  aux_loss      [1] fp32 out or NULL: E * sum_e f_e * P_e, f_e = share of the N*K
 *                slots routed to e, P_e = mean over tokens of the softmax over all E
 *                at e (0 when N = 0).
 *  meta          filled exactly as moe_build_metadata(topk_idx, topk_weights) would.
 * Device pointers, caller-owned; workspace >= moe_route_workspace(N, K, E). Errors as
 * for moe_build_metadata (MOE_EINVAL also when K > E); only enqueues on stream. */
typedef enum { MOE_ROUTE_SOFTMAX_TOPK = 0, MOE_ROUTE_TOPK_SOFTMAX = 1 } moe_route_mode;
moe_status moe_route(const void *logits, moe_dtype logits_dtype, moe_route_mode mode,
                     int32_t renormalize, int32_t *topk_idx, float *topk_weights,
                     float *aux_loss, const moe_metadata *meta, void *workspace,
                     size_t workspace_bytes, void *stream);

/* Forward (issue #68 dataflow: native non-expand metadata + local expert
 * compute -> local_out [N_recv,H]). For sorted position s of expert e, token t:
 *   h[s,:]  = x[t,:] W_up[e]                     (W_up [E,H,2I], interleaved)
 *   a[s,j]  = silu(h[s,2j]) * h[s,2j+1]          (SwiGLU, no bias)
 *   y[s,:]  = a[s,:] W_down[e]                   (W_down [E,I,H])
 *   out[t,:] = sum over the token's pairs q, ascending, of
 *              router_scores[q] * y[s_reverse_scatter_idx[q],:]   (fp32 sum)
 * Rows with no valid slot are 0. h_save [capacity,2I] (same dtype) receives h
 * for the backward; pass NULL for inference. out is [N,H].
 * H and I must be positive multiples of 8 (whole 16-byte bf16 chunks), at most
 * 2^20; other sizes return MOE_EUNSUPPORTED. Sizes that are not multiples of the
 * 128-wide tiles run with partial edge tiles. */
moe_status moe_expert_forward(const moe_metadata *meta, const void *x, const void *w_up,
                              const void *w_down, int32_t H, int32_t I, moe_dtype dt,
                              moe_gateup_layout layout, void *h_save, void *out,
                              void *workspace, size_t workspace_bytes, void *stream);

/* Backward of moe_expert_forward for upstream gradient dout [N,H]:
 *   dx [N,H], dw_up [E,H,2I], dw_down [E,I,H] (same dtype as x; fully
 *   overwritten, exact zeros for experts with no rows), and
 *   d_topk_weights [N,K] fp32 = <dout[t], y[s]> at every valid slot, 0 at
 *   invalid slots (issue #68, question 4: gradients for routing scores returned
 *   in [N_recv,K] layout).
 * h_saved is the h_save written by the forward with the same metadata.
 * topk_idx is the [N,K] array the metadata was built from. H and I as for the
 * forward. */
moe_status moe_expert_backward(const moe_metadata *meta, const int32_t *topk_idx,
                               const void *x, const void *w_up, const void *w_down,
                               const void *h_saved, const void *dout, int32_t H, int32_t I,
                               moe_dtype dt, moe_gateup_layout layout, void *dx, void *dw_up,
                               void *dw_down, float *d_topk_weights, void *workspace,
                               size_t workspace_bytes, void *stream);

const char *moe_status_string(moe_status s);

/* ---- Diagnostics: per-kernel timing with caller-created events ---------------
 * The kernels the three calls enqueue, in launch order. */
typedef enum {
  MOE_KERNEL_META_HIST = 0,    /* moe_build_metadata: per-chunk expert histograms
                                  (above 2048 slots) */
  MOE_KERNEL_META_SCAN = 1,    /* moe_build_metadata: prefixes over chunks, totals
                                  (above 256 chunks of 512 slots or 34 experts) */
  MOE_KERNEL_META_SCATTER = 2, /* moe_build_metadata: offsets + stable scatter (up to
                                  2048 slots: the whole build, counts included) */
  MOE_KERNEL_UP_SWIGLU = 3,    /* forward: gathered up-projection + SwiGLU */
  MOE_KERNEL_DOWN = 4,         /* forward: down projection */
  MOE_KERNEL_COMBINE = 5,      /* forward: weighted combine to [N,H] */
  MOE_KERNEL_DOWN_BWD = 6,     /* backward: dout_g W_down^T + dSwiGLU + dscore partials */
  MOE_KERNEL_WGRAD_DOWN = 7,   /* backward: dW_down */
  MOE_KERNEL_UP_BWD = 8,       /* backward: dh W_up^T */
  MOE_KERNEL_WGRAD_UP = 9,     /* backward: dW_up */
  MOE_KERNEL_COMBINE_DX = 10,  /* backward: dx = sum over the token's rows, and
                                  d_topk_weights in [N,K] */
  MOE_KERNEL_ROUTE = 11,       /* moe_route: top-K, weights, histograms, P sums
                                  (then META_SCAN and META_SCATTER, which also form the
                                  load-balancing loss) */
  MOE_KERNEL_COUNT = 12
} moe_kernel_id;

/* After this call, the i-th launch of `kernel` (i < n_launches, counted from this
 * call) made by the calling host thread is bracketed by hipEventRecord(events[2i])
 * just before it and hipEventRecord(events[2i+1]) just after it, on the launch's
 * stream. events holds 2*n_launches hipEvent_t created by the caller (none NULL,
 * else MOE_EINVAL); events == NULL stops recording. The hook is per host thread:
 * launches made by other threads are never bracketed and never touch it. For
 * benchmarks only. Returns the number of launches bracketed since the previous call
 * (from this thread) through *n_recorded (may be NULL). */
moe_status moe_time_kernel(moe_kernel_id kernel, void *const *events, int32_t n_launches,
                           int32_t *n_recorded);
const char *moe_kernel_name(moe_kernel_id kernel);

#ifdef __cplusplus
}
#endif
#endif
