// Routing metadata from the non-expand [N,K] layout, without a host sync.
//
// GitHub issue #68 on Dao-AILab/sonic-moe (metadata list) names the arrays; the
// Qwen3.6 serving-script notes ("Optimization (CCCL segmented-sort pattern)",
// steps 1-3) give the method: flatten the (token, expert) pairs, sort them by
// expert so each expert's rows are contiguous. Pairs are the valid slots taken
// token-major with ascending slot; the sort is a stable counting sort, so the
// result is unique.
//
// The slots are cut into chunks of kMetaThreads * ITEMS (ITEMS from the slot count);
// three kernels:
//  1. meta_hist: each workgroup counts its chunk per expert (LDS integer atomics),
//     flags ids outside [-1,E) and counts its valid slots. Columns: E experts,
//     the flag, the valid count; stored column-major [E+2][nblk].
//  2. meta_scan: one workgroup per column segment of up to 2048 chunks (4096 for longer
//     columns): exclusive prefix over chunks (each thread sums 8, or 16, consecutive
//     chunks, then DPP scans inside wavefronts), stored row-major [nblk][E+2], and the
//     column total; columns of more than 4096 chunks take a first pass of segment sums.
//  3. meta_scatter: each workgroup reads its row of prefixes and the totals (one
//     memory round trip; with at most 256 chunks and 34 experts it instead sums the
//     count columns itself and the scan launch is skipped, a two-launch build), scans
//     the totals into expert_frequency_offset, then
//     ranks its own slots stably: inside a wavefront the lanes holding the same
//     expert are found through a per-wave LDS mask per expert (up to 256 experts and
//     below 2^21 slots; else one ballot per expert-id bit) and ranked with mbcnt;
//     per-wave running counts in LDS order the rounds and the waves. Every output
//     index is written exactly once.
// Up to 2048 slots (decode-sized batches) one workgroup holds every slot: it counts
// them itself and the build is the scatter kernel alone, one launch.
#include <atomic>

#include "common.h"
#include "kernels.h"
#include "../../include/moe.h"

namespace moe {
namespace {
// Lets `fn` use up to 160 KB of dynamic LDS (a launch gets 64 KB by default), once per
// device: `done` holds one bit per device where it has been set.
hipError_t allow_large_lds(const void *fn, std::atomic<uint64_t> &done) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return hipErrorInvalidDevice;
  const uint64_t bit = 1ull << dev;
  if (done.load(std::memory_order_acquire) & bit) return hipSuccess;
  const hipError_t e =
      hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
  if (e == hipSuccess) done.fetch_or(bit, std::memory_order_release);
  return e;
}
}  // namespace

template <int ITEMS>
__global__ __launch_bounds__(kMetaThreads) void meta_hist_kernel(const int32_t *__restrict__ idx,
                                                                 int64_t NK, int E,
                                                                 int32_t *__restrict__ hist) {
  constexpr int CHUNK = kMetaThreads * ITEMS;
  extern __shared__ int32_t sh[];  // [E+2]: counts, bad-id flag, valid count
  for (int e = threadIdx.x; e < E + 2; e += kMetaThreads) sh[e] = 0;
  __syncthreads();
  const int64_t base = (int64_t)blockIdx.x * CHUNK + threadIdx.x;
  int v[ITEMS];
#pragma unroll
  for (int i = 0; i < ITEMS; i++) {
    const int64_t j = base + (int64_t)i * kMetaThreads;
    v[i] = j < NK ? idx[j] : -1;
  }
  int bad = 0, nvalid = 0;
#pragma unroll
  for (int i = 0; i < ITEMS; i++) {
    const bool ok = (unsigned)v[i] < (unsigned)E;
    if (ok)
      atomicAdd(&sh[v[i]], 1);
    else if (v[i] != -1)
      bad = 1;
    nvalid += __builtin_popcountll(ballot64(ok));
  }
  if (bad) atomicOr(&sh[E], 1);
  if (lane_id() == 0) atomicAdd(&sh[E + 1], nvalid);
  __syncthreads();
  for (int e = threadIdx.x; e < E + 2; e += kMetaThreads)
    hist[(int64_t)e * gridDim.x + blockIdx.x] = sh[e];
}

// Column scans. Column c of hist (c < W) gives pre[b][c] = sum of hist[c][b'] over
// b' < b and tot[c] = the column's sum; the router's probability columns (c >= W,
// fcol) only need their sums. A column is cut into segments of PER * 256 chunks, one
// workgroup each; thread i of a segment covers PER consecutive chunks, the thread sums
// are scanned with DPP inside each wavefront and the four wavefront totals in LDS.
// Columns of more than one segment take two passes: pass 0 writes each segment's
// sum, pass 1 adds the sums of the earlier segments (in order) as the base.
template <typename T, int PER>
__device__ __forceinline__ T segment_sum_scan(const T *__restrict__ col, int c0, int n, T *v,
                                              T *run_out, T *s_wave) {
  const int tid = threadIdx.x, w = tid / kWave, lane = tid % kWave;
  const int b0 = c0 + tid * PER;
  T s = 0;
#pragma unroll
  for (int r = 0; r < PER; r++) {
    v[r] = (tid * PER + r < n) ? col[b0 + r] : (T)0;
    s += v[r];
  }
  T incl;
  if constexpr (std::is_integral<T>::value) {
    incl = wave_inclusive_scan_dpp(s);
  } else {
    incl = wave_sum_dpp_f32(s);  // floats: only the total is used
  }
  if (lane == kWave - 1) s_wave[w] = incl;
  __syncthreads();
  T run = incl - s, total = 0;
#pragma unroll
  for (int i = 0; i < kMetaThreads / kWave; i++) {
    const T t = s_wave[i];
    run += i < w ? t : (T)0;
    total += t;
  }
  *run_out = run;
  return total;
}

template <int PER>
__global__ __launch_bounds__(kMetaThreads) void meta_scan_kernel(
    const int32_t *__restrict__ hist, int W, int nblk, int nseg, int pass,
    int32_t *__restrict__ pre, int32_t *__restrict__ tot, int32_t *__restrict__ segsum,
    const float *__restrict__ fcol, float *__restrict__ fsum, float *__restrict__ fsegsum,
    int Wf) {
  __shared__ int32_t s_wave[kMetaThreads / kWave];
  __shared__ int32_t s_base;
  const int ncol = W + Wf;
  const int c = blockIdx.x % ncol, seg = blockIdx.x / ncol;
  const int tid = threadIdx.x;
  constexpr int SEG = kMetaThreads * PER;
  const int c0 = seg * SEG;
  const int n = min(SEG, nblk - c0);  // chunks in this segment
  if (c >= W) {  // router probability column: fixed-order sums
    const int cf = c - W;
    if (pass == 1 && nseg > 1) {
      if (seg == 0 && tid == 0) {
        float t = 0.0f;
        for (int q = 0; q < nseg; q++) t += fsegsum[(int64_t)cf * nseg + q];
        fsum[cf] = t;
      }
      return;
    }
    float v[PER], run;
    const float t = segment_sum_scan<float, PER>(fcol + (int64_t)cf * nblk, c0, n, v, &run,
                                            (float *)s_wave);
    if (tid == 0) {
      if (nseg > 1) fsegsum[(int64_t)cf * nseg + seg] = t;
      else fsum[cf] = t;
    }
    return;
  }
  int v[PER], run;
  const int32_t *col = hist + (int64_t)c * nblk;
  const int t = segment_sum_scan<int32_t, PER>(col, c0, n, v, &run, s_wave);
  if (pass == 0) {  // segment sums of a long column
    if (tid == 0) segsum[(int64_t)c * nseg + seg] = t;
    return;
  }
  if (tid == 0) {
    int base = 0;
    for (int q = 0; q < seg; q++) base += segsum[(int64_t)c * nseg + q];
    s_base = base;
  }
  __syncthreads();
  run += s_base;
#pragma unroll
  for (int r = 0; r < PER; r++) {
    if (tid * PER + r < n) pre[(int64_t)(c0 + tid * PER + r) * W + c] = run;
    run += v[r];
  }
  if (tid == 0 && seg == nseg - 1) tot[c] = s_base + t;
}

// Limits of the scatter pass that scans the chunk counts itself (kMetaFused): at most
// kFusedCols columns per wavefront of a four-wavefront workgroup (E + 2 <= 36) and
// kFusedChunks chunks, so every count a workgroup needs is loaded at once.
constexpr int kFusedCols = 9, kFusedChunks = 256;

// NW wavefronts per workgroup; each ranks ITEMS rounds of 64 slots of its share of the
// chunk (the 2048-slot chunks take 8 wavefronts, so a wavefront's rounds stay at 4).
// MODE kMetaScanned: `pre` is the chunk's exclusive prefix row, `tot` the column totals.
// kMetaFused: `pre` is the per-chunk count columns [E+2][nblk] (nblk = the grid) and `tot`
// is unused; each workgroup sums the counts of the chunks before its own and of all
// chunks itself, so the build needs no separate scan launch. kMetaSolo: one workgroup
// holds every slot and counts them itself (LDS integer atomics, as the histogram pass),
// so the build is this one launch and reads no workspace.
template <int ITEMS, int NW, int MODE>
__global__ __launch_bounds__(64 * NW) void meta_scatter_kernel(
    const int32_t *__restrict__ idx, const float *__restrict__ wts, int N, int K, int E,
    int nbits, int cap, const int32_t *__restrict__ pre, const int32_t *__restrict__ tot,
    MetaOut out) {
  constexpr int NT = 64 * NW;
  constexpr int CHUNK = NT * ITEMS;
  static_assert(NW <= 8, "per-wave valid counts");
  extern __shared__ int32_t sh[];
  // [NW][E] 64-bit masks of a round's lanes per expert (see meta_use_mask)
  const bool use_mask = meta_use_mask((int64_t)N * K, E);
  uint64_t *s_mask = reinterpret_cast<uint64_t *>(sh);
  // [E+2]: totals, scanned in place -> offsets, [E] = P, [E+1] = bad-id flags
  int32_t *s_off = sh + (use_mask ? 2 * NW * E : 0);
  int32_t *s_base = s_off + E + 2;  // [E+2]: this chunk's prefix row -> bases
  int32_t *s_run = s_base + E + 2;  // [NW][E] per-wave running counts
  int32_t *s_misc = s_run + NW * E;  // [8]: per-wave valid counts
  int32_t *s_loc = s_misc + 8;      // [E+1]: this chunk's slots of experts < e (in-chunk)
  int32_t *s_ps = s_loc + E + 1;    // [CHUNK] sorted position of the k-th sorted slot
  int32_t *s_pt = s_ps + CHUNK;     // [CHUNK] its token
  int32_t *s_pq = s_pt + CHUNK;     // [CHUNK] its pair index
  const int tid = threadIdx.x;
  const int w = tid / kWave;
  const int lane = tid % kWave;
  const int64_t NK = (int64_t)N * K;
  // chunk of this workgroup: each XCD (workgroup id modulo 8) takes a contiguous run
  // of chunks, so the sorted-position writes of consecutive chunks into an expert's
  // segment meet in one L2 and leave it as whole lines
  int me;
  {
    const int b = blockIdx.x, G = gridDim.x, x = b % kNumXcd, i = b / kNumXcd;
    const int q = G / kNumXcd, r = G % kNumXcd;
    me = x * q + (x < r ? x : r) + i;
  }
  const int W = E + 2;

  // this wave's slots (the w-th quarter of the chunk, rounds of 64), the chunk's
  // prefix row and the totals: all loads issued together
  const int64_t wbase = (int64_t)me * CHUNK + (int64_t)w * (CHUNK / NW);
  int r_e[ITEMS];
  float r_w[ITEMS];
#pragma unroll
  for (int it = 0; it < ITEMS; it++) {
    const int64_t j = wbase + it * kWave + lane;
    r_e[it] = j < NK ? idx[j] : -1;
    r_w[it] = j < NK ? wts[j] : 0.0f;
  }
  const bool aux = me == 0 && out.aux;  // router: the load-balancing loss
  float *s_prod = (float *)(s_pq + CHUNK);  // [E] (router only)
  if constexpr (MODE == kMetaSolo) {
    for (int c = tid; c < W; c += NT) {
      s_base[c] = 0;  // no chunk before this one
      s_off[c] = 0;
    }
    __syncthreads();
    int bad = 0;
#pragma unroll
    for (int it = 0; it < ITEMS; it++) {
      const int e = r_e[it];
      if ((unsigned)e < (unsigned)E)
        atomicAdd(&s_off[e], 1);
      else if (e != -1)
        bad = 1;
    }
    if (bad) atomicOr(&s_off[E + 1], 1);
    __syncthreads();
    for (int e = tid; e < E; e += NT) out.expert_frequency[e] = s_off[e];
  } else if constexpr (MODE == kMetaFused) {
    // wavefront w sums columns w, w + NW, ...: all of its counts are loaded first (one
    // memory round trip), then per column the chunks before this one and all chunks,
    // each by a DPP wavefront scan
    static_assert(NW == 4, "fused scan layout");
    const int nblk = gridDim.x;
    int v[kFusedCols][kFusedChunks / kWave];
#pragma unroll
    for (int ci = 0; ci < kFusedCols; ci++)
#pragma unroll
      for (int bi = 0; bi < kFusedChunks / kWave; bi++) {
        const int c = w + ci * NW, b = lane + bi * kWave;
        v[ci][bi] = (c < W && b < nblk) ? pre[(int64_t)c * nblk + b] : 0;
      }
#pragma unroll
    for (int ci = 0; ci < kFusedCols; ci++) {
      const int c = w + ci * NW;
      if (c >= W) break;  // wave-uniform
      int sb = 0, sa = 0;
#pragma unroll
      for (int bi = 0; bi < kFusedChunks / kWave; bi++) {
        sa += v[ci][bi];
        sb += lane + bi * kWave < me ? v[ci][bi] : 0;
      }
      sb = __builtin_amdgcn_readlane(wave_inclusive_scan_dpp(sb), kWave - 1);
      sa = __builtin_amdgcn_readlane(wave_inclusive_scan_dpp(sa), kWave - 1);
      if (lane == 0) {
        s_base[c] = sb;
        if (c <= E) {
          s_off[c < E ? c : E + 1] = sa;
          if (me == 0 && c < E) out.expert_frequency[c] = sa;
        }
      }
    }
  } else {
    const int32_t *prow = pre + (int64_t)me * W;
    for (int c = tid; c < W; c += NT) {
      s_base[c] = prow[c];
      if (c <= E) {
        const int t = tot[c];
        s_off[c < E ? c : E + 1] = t;
        if (me == 0 && c < E) out.expert_frequency[c] = t;
        if (aux && c < E) s_prod[c] = out.psum ? (float)t * out.psum[c] : 0.0f;
      }
    }
  }
  for (int i = tid; i < NW * E + 8; i += NT) s_run[i] = 0;
  if (use_mask)
    for (int i = tid; i < NW * E; i += NT) s_mask[i] = 0;
  __syncthreads();
  if (aux && tid < kWave) {  // lane-strided partials, then the wave sum: fixed order
    float a = 0.0f;
    for (int e = tid; e < E; e += kWave) a += s_prod[e];
    a = wave_sum_dpp_f32(a);
    if (tid == 0) *out.aux = a * out.aux_scale;
  }
  wave0_exclusive_scan(s_off, E);  // s_off[e] = expert_frequency_offset[e], [E] = P
  __syncthreads();
  const int P = s_off[E];
  if (me == 0) {
    for (int e = tid; e <= E; e += NT) out.expert_frequency_offset[e] = s_off[e];
    if (tid == 0) {
      out.tok_off[N] = P;
      uint32_t st = 0;
      if (s_off[E + 1]) st |= MOE_DEV_BAD_EXPERT;
      if (P > cap) st |= MOE_DEV_OVER_CAPACITY;
      *out.status = st;
    }
  }
  const int valid_before = s_base[E + 1];
  for (int e = tid; e < E; e += NT) s_base[e] += s_off[e];  // base of this chunk

  // ---- stable in-chunk ranks
  int r_rank[ITEMS], r_vrank[ITEMS];
  int vrun = 0;
  int32_t *run = s_run + w * E;
#pragma unroll
  for (int it = 0; it < ITEMS; it++) {
    const int e = r_e[it];
    const bool v = (unsigned)e < (unsigned)E;
    const uint64_t vm = ballot64(v);
    // m: the valid lanes among the current 64 slots holding the same expert as this lane
    uint64_t m = vm;
    if (use_mask) {
      // each valid lane ORs its bit into its expert's mask of this wave, reads the mask
      // back and clears it. A wavefront's LDS instructions execute in issue order, so the
      // read sees every lane's OR for these 64 slots and the clear precedes the next 64's
      // ORs; the OR commutes, so no order among lanes is assumed.
      uint64_t *mk = s_mask + w * E;
      if (v) atomicOr(reinterpret_cast<unsigned long long *>(&mk[e]), 1ull << lane);
      m = v ? mk[e] : 0;
      if (v) mk[e] = 0;
    } else {
      // agree with e on every id bit. Invalid lanes (e = -1) enter the ballots too but
      // are not in vm, so never in m. Per bit: m &= bit ? bm : ~bm, as bm ^ (bit - 1) on
      // each 32-bit half (bit - 1 is 0 or all ones)
      for (int b = 0; b < nbits; b++) {
        const uint32_t bit = ((uint32_t)e >> b) & 1u;
        const uint64_t bm = ballot64(bit != 0u);
        const uint32_t t = bit - 1u;
        const uint32_t lo = (uint32_t)m & ((uint32_t)bm ^ t);
        const uint32_t hi = (uint32_t)(m >> 32) & ((uint32_t)(bm >> 32) ^ t);
        m = ((uint64_t)hi << 32) | lo;
      }
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
  // From 2^18 slots the chunk's slots are staged in LDS in sorted order and leave as runs
  // of consecutive sorted positions (coalesced writes; measured 20 % faster at 2^23
  // slots); below, each lane writes its own slot's entries (0.5 us less at 2^17).
  const bool staged = NK >= ((int64_t)1 << 18);
  if (staged) {
    for (int e = tid; e < E; e += NT) {
      int c = 0;
#pragma unroll
      for (int q = 0; q < NW; q++) c += s_run[q * E + e];
      s_loc[e] = c;
    }
    __syncthreads();
    wave0_exclusive_scan(s_loc, E);  // s_loc[e] = in-chunk slots of experts < e, [E] = total
    __syncthreads();
  }

  int vbase = valid_before;
  for (int w2 = 0; w2 < w; w2++) vbase += s_misc[w2];
  const bool small = NK <= 0x7fffffff;
#pragma unroll
  for (int it = 0; it < ITEMS; it++) {
    const int64_t j = wbase + it * kWave + lane;
    if (j >= NK) break;
    const int q = vbase + r_vrank[it];  // valid slots before slot j
    const int t = small ? (int)((uint32_t)j / (uint32_t)K) : (int)(j / K);
    if (j - (int64_t)t * K == 0) out.tok_off[t] = q;
    const int e = r_e[it];
    if (e < 0) continue;
    int rk = r_rank[it];  // rank among this chunk's slots of expert e
    for (int w2 = 0; w2 < w; w2++) rk += s_run[w2 * E + e];
    const int s = s_base[e] + rk;
    if (staged) {
      const int pl = s_loc[e] + rk;  // in-chunk sorted position
      s_ps[pl] = s;
      s_pt[pl] = t;
      s_pq[pl] = q;
    } else if ((unsigned)s < (unsigned)cap) {
      out.x_gather_idx[s] = t;
      out.s_scatter_idx[s] = q;
    }
    if ((unsigned)q < (unsigned)cap) {
      out.s_reverse_scatter_idx[q] = s;
      out.router_scores[q] = r_w[it];
    }
  }
  if (!staged) return;
  __syncthreads();
  const int nloc = s_loc[E];
  for (int pl = tid; pl < nloc; pl += NT) {
    const int s = s_ps[pl];
    if ((unsigned)s < (unsigned)cap) {
      out.x_gather_idx[s] = s_pt[pl];
      out.s_scatter_idx[s] = s_pq[pl];
    }
  }
}

hipError_t launch_meta_hist(const int32_t *topk_idx, int N, int K, int E, int32_t *ws,
                            hipStream_t stream) {
  const int64_t NK = (int64_t)N * K;
  const MetaWs L = meta_ws_layout(NK, E);
  const size_t sh = (size_t)(E + 2) * sizeof(int32_t);
  if (meta_items(NK) == 8)
    hipLaunchKernelGGL(meta_hist_kernel<8>, dim3(L.nblk), dim3(kMetaThreads), sh, stream, topk_idx,
                       NK, E, ws + L.hist);
  else if (meta_items(NK) == 4)
    hipLaunchKernelGGL(meta_hist_kernel<4>, dim3(L.nblk), dim3(kMetaThreads), sh, stream, topk_idx,
                       NK, E, ws + L.hist);
  else
    hipLaunchKernelGGL(meta_hist_kernel<2>, dim3(L.nblk), dim3(kMetaThreads), sh, stream, topk_idx,
                       NK, E, ws + L.hist);
  return hipGetLastError();
}

hipError_t launch_meta_scan(int N, int K, int E, int32_t *ws, hipStream_t stream,
                            const float *fcol, float *fsum) {
  const MetaWs L = meta_ws_layout((int64_t)N * K, E);
  const int W = E + 2, Wf = fcol ? E : 0;
  int32_t *segsum = ws + L.seg;
  float *fsegsum = (float *)(segsum + (size_t)W * L.nseg);
  const dim3 grid((unsigned)((W + Wf) * L.nseg));
  auto kern = scan_per(L.nblk) == 16 ? meta_scan_kernel<16> : meta_scan_kernel<8>;
  if (L.nseg > 1) {
    hipLaunchKernelGGL(kern, grid, dim3(kMetaThreads), 0, stream, ws + L.hist, W, L.nblk,
                       L.nseg, 0, ws + L.pre, ws + L.tot, segsum, fcol, fsum, fsegsum, Wf);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(kern, grid, dim3(kMetaThreads), 0, stream, ws + L.hist, W, L.nblk, L.nseg,
                     1, ws + L.pre, ws + L.tot, segsum, fcol, fsum, fsegsum, Wf);
  return hipGetLastError();
}

bool meta_fused_scan(int64_t NK, int E) {
  return meta_items(NK) == 2 && E + 2 <= 4 * kFusedCols && meta_blocks(NK) <= kFusedChunks;
}

bool meta_solo(int64_t NK) { return NK <= kMetaSoloSlots; }

hipError_t launch_meta_scatter(const int32_t *topk_idx, const float *topk_weights, int N, int K,
                               int E, int capacity, const int32_t *ws, const MetaOut &out,
                               hipStream_t stream, int mode) {
  const int64_t NK = (int64_t)N * K;
  const MetaWs L = meta_ws_layout(NK, E);
  int nbits = 0;
  while ((1 << nbits) < E) nbits++;
  if (mode == kMetaSolo) {
    if (!meta_solo(NK) || out.aux) return hipErrorInvalidValue;
    // one workgroup: four wavefronts of two rounds of 64 slots up to 512 slots, eight
    // wavefronts of two rounds up to 1024, of four rounds up to 2048
#define MOE_SOLO(ITEMS_, NW_)                                                                \
  {                                                                                        \
    constexpr int chunk = 64 * (NW_) * (ITEMS_);                                           \
    const size_t sh = (size_t)(2 * (E + 2) + (NW_) * E + 8 + (E + 1) + 3 * chunk +          \
                               meta_mask_ints(NK, E, NW_)) * sizeof(int32_t);               \
    static std::atomic<uint64_t> done{0};                                                  \
    const hipError_t attr = allow_large_lds(                                               \
        reinterpret_cast<const void *>(&meta_scatter_kernel<ITEMS_, NW_, kMetaSolo>), done); \
    if (attr != hipSuccess) return attr;                                                   \
    hipLaunchKernelGGL((meta_scatter_kernel<ITEMS_, NW_, kMetaSolo>), dim3(1),             \
                       dim3(64 * (NW_)), sh, stream, topk_idx, topk_weights, N, K, E, nbits, \
                       capacity, nullptr, nullptr, out);                                   \
  }
    if (NK <= 512)
      MOE_SOLO(2, 4)
    else if (NK <= 1024)
      MOE_SOLO(2, 8)
    else
      MOE_SOLO(4, 8)
#undef MOE_SOLO
    return hipGetLastError();
  }
  const int items = meta_items(NK);
  const int nw = items == 8 ? 8 : 4;  // wavefronts of the scatter workgroup
  const size_t sh = (size_t)(2 * (E + 2) + nw * E + 8 + (E + 1) + 3 * meta_chunk(NK) +
                             (out.aux ? E : 0) + meta_mask_ints(NK, E, nw)) * sizeof(int32_t);
  if (mode == kMetaFused) {
    if (!meta_fused_scan(NK, E) || out.aux) return hipErrorInvalidValue;
    hipLaunchKernelGGL((meta_scatter_kernel<2, 4, kMetaFused>), dim3(L.nblk), dim3(64 * 4), sh, stream,
                       topk_idx, topk_weights, N, K, E, nbits, capacity, ws + L.hist, nullptr,
                       out);
  } else if (items == 8) {
    // with 1024 experts the eight waves' running counts take the stage past the 64 KB of
    // dynamic LDS a launch gets by default (a workgroup may use up to 160 KB)
    static std::atomic<uint64_t> done{0};
    const hipError_t attr = allow_large_lds(
        reinterpret_cast<const void *>(&meta_scatter_kernel<4, 8, kMetaScanned>), done);
    if (attr != hipSuccess) return attr;
    hipLaunchKernelGGL((meta_scatter_kernel<4, 8, kMetaScanned>), dim3(L.nblk), dim3(64 * 8), sh,
                       stream, topk_idx, topk_weights, N, K, E, nbits, capacity, ws + L.pre,
                       ws + L.tot, out);
  } else if (items == 4)
    hipLaunchKernelGGL((meta_scatter_kernel<4, 4, kMetaScanned>), dim3(L.nblk), dim3(64 * 4), sh,
                       stream, topk_idx, topk_weights, N, K, E, nbits, capacity, ws + L.pre,
                       ws + L.tot, out);
  else
    hipLaunchKernelGGL((meta_scatter_kernel<2, 4, kMetaScanned>), dim3(L.nblk), dim3(64 * 4), sh,
                       stream, topk_idx, topk_weights, N, K, E, nbits, capacity, ws + L.pre,
                       ws + L.tot, out);
  return hipGetLastError();
}

}  // namespace moe
