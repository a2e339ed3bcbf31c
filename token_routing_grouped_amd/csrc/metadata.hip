// Routing metadata from the non-expand [N,K] layout, without a host sync.
//
// GitHub issue #68 on Dao-AILab/sonic-moe (metadata list) names the arrays; the
// Qwen3.6 serving-script notes ("Optimization (CCCL segmented-sort pattern)",
// steps 1-3) give the method: flatten the (token, expert) pairs, sort them by
// expert so each expert's rows are contiguous. Pairs are the valid slots taken
// token-major with ascending slot; the sort is a stable counting sort, so the
// result is unique.
//
// Two kernels:
//  1. meta_hist: each workgroup counts its chunk of slots per expert (LDS
//     integer atomics) and flags ids outside [-1,E).
//  2. meta_scatter: each workgroup sums the histograms of all chunks (column
//     totals give expert_frequency and its scan; the chunks before it give its
//     base per expert), then ranks its own slots stably: inside a wavefront the
//     lanes holding the same expert are found with one ballot per expert-id bit
//     and ranked with mbcnt; per-wave running counts in LDS order the rounds and
//     the four waves. Every output index is written exactly once.
#include "common.h"
#include "kernels.h"
#include "../../include/moe.h"

namespace moe {

__global__ __launch_bounds__(kMetaThreads) void meta_hist_kernel(const int32_t *__restrict__ idx,
                                                                 int64_t NK, int E,
                                                                 int32_t *__restrict__ hist) {
  extern __shared__ int32_t sh[];  // [E+1]: counts, then the bad-id flag
  for (int e = threadIdx.x; e <= E; e += kMetaThreads) sh[e] = 0;
  __syncthreads();
  const int64_t base = (int64_t)blockIdx.x * kMetaChunk + threadIdx.x;
  int v[kMetaItems];
#pragma unroll
  for (int i = 0; i < kMetaItems; i++) {
    const int64_t j = base + (int64_t)i * kMetaThreads;
    v[i] = j < NK ? idx[j] : -1;
  }
  int bad = 0;
#pragma unroll
  for (int i = 0; i < kMetaItems; i++) {
    if ((unsigned)v[i] < (unsigned)E)
      atomicAdd(&sh[v[i]], 1);
    else if (v[i] != -1)
      bad = 1;
  }
  if (bad) atomicOr(&sh[E], 1);
  __syncthreads();
  int32_t *row = hist + (int64_t)blockIdx.x * (E + 1);
  for (int e = threadIdx.x; e <= E; e += kMetaThreads) row[e] = sh[e];
}

__global__ __launch_bounds__(kMetaThreads) void meta_scatter_kernel(
    const int32_t *__restrict__ idx, const float *__restrict__ wts, int N, int K, int E,
    int nbits, int nblk, int cap, const int32_t *__restrict__ hist, MetaOut out) {
  extern __shared__ int32_t sh[];
  int32_t *s_total = sh;                // [E+2]: column totals, then flag; scanned in place
  int32_t *s_before = s_total + E + 2;  // [E+1]: counts in earlier chunks -> bases
  int32_t *s_run = s_before + E + 1;    // [4][E] per-wave running counts
  int32_t *s_misc = s_run + 4 * E;      // [8]: per-wave valid counts, valid-before, flag
  const int tid = threadIdx.x;
  const int64_t NK = (int64_t)N * K;

  for (int i = tid; i < 2 * E + 3 + 4 * E + 8; i += kMetaThreads) sh[i] = 0;
  __syncthreads();

  // column sums over all chunks' histograms
  const int W = E + 1;
  const int tot = nblk * W;  // < 2^31, checked by the host
  const int me = blockIdx.x;
  for (int i = tid; i < tot; i += kMetaThreads) {
    const int b = i / W;
    const int e = i - b * W;
    const int v = hist[i];
    if (v == 0) continue;
    if (e < E) {
      atomicAdd(&s_total[e], v);
      if (b < me) atomicAdd(&s_before[e], v);
    } else {
      atomicOr(&s_misc[5], v);
    }
  }
  __syncthreads();
  for (int e = tid; e < E; e += kMetaThreads)
    if (s_before[e]) atomicAdd(&s_misc[4], s_before[e]);  // valid pairs before this chunk
  if (me == 0)
    for (int e = tid; e < E; e += kMetaThreads) out.expert_frequency[e] = s_total[e];
  __syncthreads();
  wave0_exclusive_scan(s_total, E);  // s_total[e] = expert_frequency_offset[e], [E] = P
  __syncthreads();
  const int P = s_total[E];
  if (me == 0) {
    for (int e = tid; e <= E; e += kMetaThreads) out.expert_frequency_offset[e] = s_total[e];
    if (tid == 0) {
      out.tok_off[N] = P;
      uint32_t st = 0;
      if (s_misc[5]) st |= MOE_DEV_BAD_EXPERT;
      if (P > cap) st |= MOE_DEV_OVER_CAPACITY;
      *out.status = st;
    }
  }
  for (int e = tid; e < E; e += kMetaThreads) s_before[e] += s_total[e];  // base of this chunk
  const int valid_before = s_misc[4];

  // ---- stable in-chunk ranks: wave w owns the w-th quarter of the chunk, in rounds of 64
  const int w = tid / kWave;
  const int lane = tid % kWave;
  const int64_t wbase = (int64_t)me * kMetaChunk + (int64_t)w * (kMetaChunk / 4);
  int r_e[kMetaItems], r_rank[kMetaItems], r_vrank[kMetaItems];
  float r_w[kMetaItems];
  int vrun = 0;
  int32_t *run = s_run + w * E;
#pragma unroll
  for (int it = 0; it < kMetaItems; it++) {
    const int64_t j = wbase + it * kWave + lane;
    int e = j < NK ? idx[j] : -1;
    r_w[it] = j < NK ? wts[j] : 0.0f;
    const bool v = (unsigned)e < (unsigned)E;
    const uint64_t vm = ballot64(v);
    uint64_t m = vm;
    for (int b = 0; b < nbits; b++) {
      const bool bit = v && ((e >> b) & 1);
      const uint64_t bm = ballot64(bit);
      m &= bit ? bm : ~bm;
    }
    int prev = 0;
    if (v) prev = run[e];
    const bool leader = v && (__builtin_ctzll(m) == lane);
    if (leader) run[e] = prev + __builtin_popcountll(m);
    r_e[it] = v ? e : -1;
    r_rank[it] = prev + popc_below(m);
    r_vrank[it] = vrun + popc_below(vm);
    vrun += __builtin_popcountll(vm);
  }
  if (lane == 0) s_misc[w] = vrun;
  __syncthreads();

  int vbase = valid_before;
  for (int w2 = 0; w2 < w; w2++) vbase += s_misc[w2];
#pragma unroll
  for (int it = 0; it < kMetaItems; it++) {
    const int64_t j = wbase + it * kWave + lane;
    if (j >= NK) break;
    const int q = vbase + r_vrank[it];  // valid slots before slot j
    const int t = (int)(j / K);
    if (j - (int64_t)t * K == 0) out.tok_off[t] = q;
    const int e = r_e[it];
    if (e < 0) continue;
    int s = s_before[e] + r_rank[it];
    for (int w2 = 0; w2 < w; w2++) s += s_run[w2 * E + e];
    if (s < cap) {
      out.x_gather_idx[s] = t;
      out.s_scatter_idx[s] = q;
    }
    if (q < cap) {
      out.s_reverse_scatter_idx[q] = s;
      out.router_scores[q] = r_w[it];
    }
  }
}

hipError_t launch_meta_hist(const int32_t *topk_idx, int N, int K, int E, int32_t *hist_ws,
                            hipStream_t stream) {
  const int64_t NK = (int64_t)N * K;
  hipLaunchKernelGGL(meta_hist_kernel, dim3(meta_blocks(NK)), dim3(kMetaThreads),
                     (size_t)(E + 1) * sizeof(int32_t), stream, topk_idx, NK, E, hist_ws);
  return hipGetLastError();
}

hipError_t launch_meta_scatter(const int32_t *topk_idx, const float *topk_weights, int N, int K,
                               int E, int capacity, const int32_t *hist_ws, const MetaOut &out,
                               hipStream_t stream) {
  const int nblk = meta_blocks((int64_t)N * K);
  int nbits = 0;
  while ((1 << nbits) < E) nbits++;
  const size_t sh = (size_t)(2 * E + 3 + 4 * E + 8) * sizeof(int32_t);
  hipLaunchKernelGGL(meta_scatter_kernel, dim3(nblk), dim3(kMetaThreads), sh, stream, topk_idx,
                     topk_weights, N, K, E, nbits, nblk, capacity, hist_ws, out);
  return hipGetLastError();
}

}  // namespace moe
