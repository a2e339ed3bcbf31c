// Router top-K fused with the first pass of the metadata build.
//
// The Hysen Labs page on Dao-AILab/sonic-moe ("Three routing strategies, selected on
// the command line") names two orders of softmax and top-K selection and says the
// layer also returns an auxiliary load-balancing loss:
//  - softmax over the top-K logits: w_k = exp(l_k) / sum over the K selected exp(l);
//  - top-K of the softmax over all E experts, optionally renormalised over the K.
// Both select the K largest logits (softmax is increasing); equal logits go to the
// lower expert id, and the slots list the experts largest first. The loss is
// E * sum_e f_e * P_e with f_e the share of the N*K slots routed to e and P_e the mean
// over tokens of the full softmax at e (the usual load-balancing product form; the page
// gives no formula).
//
// route_hist: 16 lanes per token (E <= 256, K <= 16; four tokens per wavefront), else
// a whole wavefront per token. The K experts come from K rounds of a group maximum
// over 64-bit keys (order-preserving logit bits, then the inverted expert id) taken
// with DPP lane moves, so the choice is exact and deterministic. Each workgroup owns one chunk of kMetaChunk slots of the flattened
// [N,K] layout, exactly like the metadata histogram pass: it writes the slots of its
// chunk (tokens straddling a chunk edge are evaluated by both workgroups, each writing
// its own slots), counts them per expert into its histogram column, and sums the full
// softmax of the tokens whose first slot it owns into a per-chunk column of P sums.
// The metadata scan pass also sums each expert's P column in a fixed order, and the
// scatter pass's first workgroup forms the loss.
#include "common.h"
#include "kernels.h"
#include "../../include/moe.h"

namespace moe {
namespace {

constexpr int kMaxPerLane = 16;  // experts per lane: E <= 16 * lanes per token
constexpr int kRouteThreads = 1024;  // 16 wavefronts share one chunk of kMetaChunk slots

__device__ __forceinline__ float to_f32(float v) { return v; }
__device__ __forceinline__ float to_f32(uint16_t v) { return bf16_to_f32(v); }

// float -> unsigned key with the same order (negative values reversed)
__device__ __forceinline__ uint32_t ordered(float f) {
  const uint32_t b = __float_as_uint(f);
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}
__device__ __forceinline__ float unordered(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7fffffffu) : ~k);
}

// Reductions over the LPT lanes that share a token, with DPP lane moves (no LDS).
// LPT = 16: one DPP row per token; rotations by 1, 2, 4, 8 give every lane of the
// row the row's result. LPT = 64: Hillis-Steele shifts inside rows, then rows
// combined with row_bcast:15 / row_bcast:31; lane 63 holds the result, read back to
// every lane. Max results are exact; a sum is taken from one lane, so every lane of a
// token uses the same value.
template <int CTRL, int ROWS, bool BC>
__device__ __forceinline__ uint32_t dpp(uint32_t old, uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp((int)old, (int)v, CTRL, ROWS, 0xf, BC);
}
__device__ __forceinline__ uint64_t max64(uint64_t a, uint64_t b) { return a > b ? a : b; }

template <int LPT>
__device__ __forceinline__ uint64_t group_max_u64(uint64_t v) {
  uint32_t lo = (uint32_t)v, hi = (uint32_t)(v >> 32);
#define MOE_STEP(C, R, B)                                                       \
  {                                                                             \
    const uint32_t l2 = dpp<C, R, B>(0u, lo), h2 = dpp<C, R, B>(0u, hi);        \
    const uint64_t m = max64(((uint64_t)hi << 32) | lo, ((uint64_t)h2 << 32) | l2); \
    lo = (uint32_t)m;                                                           \
    hi = (uint32_t)(m >> 32);                                                   \
  }
  if constexpr (LPT == 16) {
    MOE_STEP(0x121, 0xf, false)  // row_ror:1
    MOE_STEP(0x122, 0xf, false)  // row_ror:2
    MOE_STEP(0x124, 0xf, false)  // row_ror:4
    MOE_STEP(0x128, 0xf, false)  // row_ror:8
    return ((uint64_t)hi << 32) | lo;
  } else {
    MOE_STEP(0x111, 0xf, true)   // row_shr:1
    MOE_STEP(0x112, 0xf, true)   // row_shr:2
    MOE_STEP(0x114, 0xf, true)   // row_shr:4
    MOE_STEP(0x118, 0xf, true)   // row_shr:8
    MOE_STEP(0x142, 0xa, false)  // row_bcast:15 -> rows 1, 3
    MOE_STEP(0x143, 0xc, false)  // row_bcast:31 -> rows 2, 3
    const uint32_t l = __builtin_amdgcn_readlane(lo, kWave - 1);
    const uint32_t h = __builtin_amdgcn_readlane(hi, kWave - 1);
    return ((uint64_t)h << 32) | l;
  }
#undef MOE_STEP
}

template <int LPT>
__device__ __forceinline__ float group_max_f32(float v) {
  const uint32_t NEG_INF = 0xff800000u;
#define MOE_STEP(C, R, B) v = fmaxf(v, __uint_as_float(dpp<C, R, B>(NEG_INF, __float_as_uint(v))));
  if constexpr (LPT == 16) {
    MOE_STEP(0x121, 0xf, false)
    MOE_STEP(0x122, 0xf, false)
    MOE_STEP(0x124, 0xf, false)
    MOE_STEP(0x128, 0xf, false)
    return v;
  } else {
    MOE_STEP(0x111, 0xf, false)
    MOE_STEP(0x112, 0xf, false)
    MOE_STEP(0x114, 0xf, false)
    MOE_STEP(0x118, 0xf, false)
    MOE_STEP(0x142, 0xa, false)
    MOE_STEP(0x143, 0xc, false)
    return __uint_as_float(__builtin_amdgcn_readlane(__float_as_uint(v), kWave - 1));  // bits
  }
#undef MOE_STEP
}

template <int LPT>
__device__ __forceinline__ float group_sum_f32(float v) {
#define MOE_STEP(C, R, B) v += __uint_as_float(dpp<C, R, B>(0u, __float_as_uint(v)));
  if constexpr (LPT == 16) {
    MOE_STEP(0x121, 0xf, false)
    MOE_STEP(0x122, 0xf, false)
    MOE_STEP(0x124, 0xf, false)
    MOE_STEP(0x128, 0xf, false)
    return __shfl(v, lane_id() & ~15, kWave);  // the row's first lane
  } else {
    MOE_STEP(0x111, 0xf, true)
    MOE_STEP(0x112, 0xf, true)
    MOE_STEP(0x114, 0xf, true)
    MOE_STEP(0x118, 0xf, true)
    MOE_STEP(0x142, 0xa, false)
    MOE_STEP(0x143, 0xc, false)
    return __uint_as_float(__builtin_amdgcn_readlane(__float_as_uint(v), kWave - 1));  // bits
  }
#undef MOE_STEP
}

// sum over the whole wave, the same value in every lane
__device__ __forceinline__ float wave_sum_f32(float v) { return group_sum_f32<64>(v); }

// LPT lanes per token (16: E <= 256 and K <= 16, four tokens per wave; else 64).
// Lane s of a token's group holds experts s, s+LPT, ...; after the selection, lane k
// of the group holds the k-th expert.
template <typename T, int LPT>
__global__ __launch_bounds__(kRouteThreads) void route_hist_kernel(
    const T *__restrict__ logits, int N, int E, int K, int mode, int renorm, int want_p,
    int32_t *__restrict__ topk_idx, float *__restrict__ topk_w, int32_t *__restrict__ hist,
    float *__restrict__ ppart) {
  constexpr int TPW = kWave / LPT;                     // tokens per wave
  constexpr int NW = kRouteThreads / kWave;            // wavefronts per workgroup
  constexpr int TPB = TPW * NW;                        // tokens per workgroup round
  extern __shared__ int32_t sh[];
  int32_t *s_cnt = sh;                     // [E+2]: counts, bad-id flag (0), valid count
  float *s_p = (float *)(s_cnt + E + 2);   // [NW][E] per-wave P sums
  const int tid = threadIdx.x, w = tid / kWave, lane = tid % kWave;
  const int sub = lane / LPT, sl = lane % LPT;
  const int b = blockIdx.x, nblk = gridDim.x;
  for (int i = tid; i < E + 2; i += kRouteThreads) s_cnt[i] = 0;
  for (int i = tid; i < NW * E; i += kRouteThreads) s_p[i] = 0.0f;
  __syncthreads();

  const int64_t NK = (int64_t)N * K;
  const int64_t j0 = (int64_t)b * kMetaChunk;
  const int64_t j1 = min(j0 + kMetaChunk, NK);  // this workgroup's slots [j0, j1)
  const int t0 = (int)(j0 / K), t1 = j1 > j0 ? (int)((j1 - 1) / K) : t0 - 1;
  const int nv = (E + LPT - 1) / LPT;
  float pacc[kMaxPerLane];
#pragma unroll
  for (int i = 0; i < kMaxPerLane; i++) pacc[i] = 0.0f;
  int nslots = 0;

  // uniform trip count for the whole wave; lanes of a token past t1 compute on a
  // clamped token and write nothing
  for (int base = t0 + w * TPW; base <= t1; base += TPB) {
    const bool live = base + sub <= t1;
    const int t = live ? base + sub : t1;
    float v[kMaxPerLane];
#pragma unroll
    for (int i = 0; i < kMaxPerLane; i++) {
      const int e = sl + LPT * i;
      v[i] = (i < nv && e < E) ? to_f32(logits[(int64_t)t * E + e]) : -INFINITY;
    }
    float lmax = -INFINITY;
#pragma unroll
    for (int i = 0; i < kMaxPerLane; i++) lmax = fmaxf(lmax, v[i]);
    const float mx = group_max_f32<LPT>(lmax);
    float ex[kMaxPerLane];
    float zl = 0.0f;
#pragma unroll
    for (int i = 0; i < kMaxPerLane; i++) {
      const int e = sl + LPT * i;
      ex[i] = (i < nv && e < E) ? expf(v[i] - mx) : 0.0f;
      zl += ex[i];
    }
    const float z_all = group_sum_f32<LPT>(zl);

    // K rounds of a group maximum over (logit, inverted id) keys
    uint32_t taken = 0;
    int my_e = 0;
    float my_v = 0.0f;
    for (int k = 0; k < K; k++) {
      uint64_t best = 0;
#pragma unroll
      for (int i = 0; i < kMaxPerLane; i++) {
        const int e = sl + LPT * i;
        if (i < nv && e < E && !((taken >> i) & 1u)) {
          const uint64_t key = ((uint64_t)ordered(v[i]) << 32) | (uint32_t)(0xffffffffu - e);
          best = key > best ? key : best;
        }
      }
      best = group_max_u64<LPT>(best);
      const int e = (int)(0xffffffffu - (uint32_t)best);
      if (sl == (e % LPT)) taken |= 1u << (e / LPT);
      if (sl == k) {
        my_e = e;
        my_v = unordered((uint32_t)(best >> 32));
      }
    }
    const float ek = sl < K ? expf(my_v - mx) : 0.0f;
    float wk;
    if (mode == MOE_ROUTE_SOFTMAX_TOPK) {
      wk = ek / group_sum_f32<LPT>(ek);
    } else {
      const float pk = ek / z_all;
      wk = renorm ? pk / group_sum_f32<LPT>(pk) : pk;
    }
    const int64_t j = (int64_t)t * K + sl;
    if (live && sl < K && j >= j0 && j < j1) {
      topk_idx[j] = my_e;
      topk_w[j] = wk;
      atomicAdd(&s_cnt[my_e], 1);
      nslots++;
    }
    if (want_p && live && (int64_t)t * K >= j0) {  // this workgroup owns token t
#pragma unroll
      for (int i = 0; i < kMaxPerLane; i++) pacc[i] += ex[i] / z_all;
    }
  }
  nslots = (int)wave_sum_f32((float)nslots);
  if (lane == 0) atomicAdd(&s_cnt[E + 1], nslots);
  if (want_p) {
    // the wave's token groups, in group order, into the wave's LDS row (one wave's
    // LDS operations complete in issue order)
    for (int q = 0; q < TPW; q++) {
      if (sub == q) {
#pragma unroll
        for (int i = 0; i < kMaxPerLane; i++) {
          const int e = sl + LPT * i;
          if (i < nv && e < E) s_p[w * E + e] += pacc[i];
        }
      }
    }
  }
  __syncthreads();
  for (int e = tid; e < E + 2; e += kRouteThreads) hist[(int64_t)e * nblk + b] = s_cnt[e];
  if (want_p)
    for (int e = tid; e < E; e += kRouteThreads) {
      float s = 0.0f;
      for (int q = 0; q < NW; q++) s += s_p[q * E + e];  // wave order
      ppart[(int64_t)e * nblk + b] = s;
    }
}

}  // namespace

size_t route_ws_floats(int64_t NK, int E) { return (size_t)(meta_blocks(NK) + 1) * (size_t)E; }

hipError_t launch_route_hist(const void *logits, bool bf16, int N, int E, int K, int mode,
                             int renorm, bool want_p, int32_t *topk_idx, float *topk_w,
                             int32_t *meta_ws, float *ppart, hipStream_t stream) {
  const MetaWs L = meta_ws_layout((int64_t)N * K, E);
  const size_t sh = (size_t)(E + 2) * sizeof(int32_t) +
                    (size_t)(kRouteThreads / kWave) * E * sizeof(float);
  const bool narrow = E <= 16 * kMaxPerLane && K <= 16;  // 16 lanes per token
#define MOE_ROUTE(T, LPT)                                                                  \
  hipLaunchKernelGGL((route_hist_kernel<T, LPT>), dim3(L.nblk), dim3(kRouteThreads), sh, stream, \
                     (const T *)logits, N, E, K, mode, renorm, (int)want_p, topk_idx, topk_w, \
                     meta_ws + L.hist, ppart)
  if (bf16) {
    if (narrow) MOE_ROUTE(uint16_t, 16); else MOE_ROUTE(uint16_t, 64);
  } else {
    if (narrow) MOE_ROUTE(float, 16); else MOE_ROUTE(float, 64);
  }
#undef MOE_ROUTE
  return hipGetLastError();
}

}  // namespace moe
