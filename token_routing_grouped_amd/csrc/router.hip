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
// route_hist: 8 lanes per token (E <= 128, K <= 8; eight tokens per wavefront), 16
// (E <= 256, K <= 16; four tokens per wavefront), else a whole wavefront per token; each lane holds NV (a power of two, from E) logits. The
// K experts come from K rounds of two group reductions taken with DPP lane moves: the
// maximum of the order-preserving logit bits, then the lowest expert id holding it, so
// the choice is exact and deterministic. Each workgroup owns one metadata chunk of the flattened
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
#ifndef MOE_ROUTE_THREADS
#define MOE_ROUTE_THREADS 512
#endif
constexpr int kRouteThreads = MOE_ROUTE_THREADS;  // wavefronts sharing one chunk of slots

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
// LPT = 8: half a DPP row per token; pairwise exchanges (xor 1, xor 2, mirrored
// halves) give every lane the group's result. LPT = 16: one DPP row per token;
// rotations by 1, 2, 4, 8 give every lane of the row the row's result. LPT = 64: Hillis-Steele shifts inside rows, then rows
// combined with row_bcast:15 / row_bcast:31; lane 63 holds the result, read back to
// every lane. Max results are exact; a sum is taken from one lane, so every lane of a
// token uses the same value.
template <int CTRL, int ROWS, bool BC>
__device__ __forceinline__ uint32_t dpp(uint32_t old, uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp((int)old, (int)v, CTRL, ROWS, 0xf, BC);
}
template <int LPT>
__device__ __forceinline__ float group_max_f32(float v) {
  const uint32_t NEG_INF = 0xff800000u;
#define MOE_STEP(C, R, B) v = fmaxf(v, __uint_as_float(dpp<C, R, B>(NEG_INF, __float_as_uint(v))));
  if constexpr (LPT == 8) {
    MOE_STEP(0xB1, 0xf, false)   // quad_perm [1,0,3,2]
    MOE_STEP(0x4E, 0xf, false)   // quad_perm [2,3,0,1]
    MOE_STEP(0x141, 0xf, false)  // row_half_mirror
    return v;
  } else if constexpr (LPT == 16) {
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

// unsigned max / min over the token's lanes (ID: the identity, fed to lanes a shift
// leaves without a source)
template <int LPT, bool MAX>
__device__ __forceinline__ uint32_t group_ext_u32(uint32_t v) {
  constexpr uint32_t ID = MAX ? 0u : 0xffffffffu;
#define MOE_STEP(C, R, B)                                                       \
  {                                                                             \
    const uint32_t o_ = dpp<C, R, B>(ID, v);                                    \
    v = MAX ? (o_ > v ? o_ : v) : (o_ < v ? o_ : v);                            \
  }
  if constexpr (LPT == 8) {
    MOE_STEP(0xB1, 0xf, false)
    MOE_STEP(0x4E, 0xf, false)
    MOE_STEP(0x141, 0xf, false)
    return v;
  } else if constexpr (LPT == 16) {
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
    return __builtin_amdgcn_readlane(v, kWave - 1);
  }
#undef MOE_STEP
}

template <int LPT>
__device__ __forceinline__ float group_sum_f32(float v) {
#define MOE_STEP(C, R, B) v += __uint_as_float(dpp<C, R, B>(0u, __float_as_uint(v)));
  if constexpr (LPT == 8) {
    // lanes exchange pairwise (xor 1, xor 2, then mirrored halves), so every lane adds
    // the same two operands at every step: the eight results are bit-identical
    MOE_STEP(0xB1, 0xf, false)
    MOE_STEP(0x4E, 0xf, false)
    MOE_STEP(0x141, 0xf, false)
    return v;
  } else if constexpr (LPT == 16) {
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

// LPT lanes per token (8: E <= 128 and K <= 8; 16: E <= 256 and K <= 16; else 64), NV
// logits per lane. Lane s of a token's group holds experts s, s+LPT, ...; after the
// selection, lane k of the group holds the k-th expert. FULL: E == LPT * NV, so every
// lane's NV experts exist and no per-logit bound is tested.
template <typename T, int LPT, int NV, bool FULL>
__global__ __launch_bounds__(kRouteThreads) void route_hist_kernel(
    const T *__restrict__ logits, int N, int E, int K, int mode, int renorm, int want_p,
    int32_t *__restrict__ topk_idx, float *__restrict__ topk_w, int32_t *__restrict__ hist,
    float *__restrict__ ppart, int chunk) {
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
  __syncthreads();

  const int64_t NK = (int64_t)N * K;
  const int64_t j0 = (int64_t)b * chunk;
  const int64_t j1 = min(j0 + chunk, NK);  // this workgroup's slots [j0, j1)
  const int t0 = (int)(j0 / K), t1 = j1 > j0 ? (int)((j1 - 1) / K) : t0 - 1;
  float pacc[NV];
#pragma unroll
  for (int i = 0; i < NV; i++) pacc[i] = 0.0f;
  int nslots = 0;

  // uniform trip count for the whole wave; lanes of a token past t1 compute on a
  // clamped token and write nothing
  for (int base = t0 + w * TPW; base <= t1; base += TPB) {
    const bool live = base + sub <= t1;
    const int t = live ? base + sub : t1;
    float v[NV];
#pragma unroll
    for (int i = 0; i < NV; i++) {
      const int e = sl + LPT * i;
      v[i] = (FULL || e < E) ? to_f32(logits[(int64_t)t * E + e]) : -INFINITY;
    }
    float lmax = -INFINITY;
#pragma unroll
    for (int i = 0; i < NV; i++) lmax = fmaxf(lmax, v[i]);
    const float mx = group_max_f32<LPT>(lmax);
    float ex[NV];
    float zl = 0.0f;
#pragma unroll
    for (int i = 0; i < NV; i++) {
      ex[i] = (FULL || sl + LPT * i < E) ? expf(v[i] - mx) : 0.0f;
      zl += ex[i];
    }
    const float z_all = group_sum_f32<LPT>(zl);

    // K rounds: the group maximum of the order-preserving logit bits, then the lowest
    // expert id holding that value (equal logits go to the lower id). A key of 0 marks a
    // taken or absent expert; valid keys are at least 1 (only the all-ones NaN pattern
    // is moved, from 0 to 1).
    uint32_t key[NV];
#pragma unroll
    for (int i = 0; i < NV; i++) {
      const uint32_t o = ordered(v[i]);
      key[i] = (FULL || sl + LPT * i < E) ? (o > 1u ? o : 1u) : 0u;
    }
    int my_e = 0;
    float my_v = 0.0f;
    for (int k = 0; k < K; k++) {
      uint32_t m = 0;
#pragma unroll
      for (int i = 0; i < NV; i++) m = key[i] > m ? key[i] : m;
      m = group_ext_u32<LPT, true>(m);
      uint32_t cand = 0xffffffffu;  // this lane's lowest id holding m
#pragma unroll
      for (int i = NV - 1; i >= 0; i--) cand = key[i] == m ? (uint32_t)(sl + LPT * i) : cand;
      const int e = (int)group_ext_u32<LPT, false>(cand);
      if (sl == (e % LPT)) {
#pragma unroll
        for (int i = 0; i < NV; i++)
          if (i == e / LPT) key[i] = 0;
      }
      if (sl == k) {
        my_e = e;
        my_v = unordered(m);
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
      const float rz = 1.0f / z_all;
#pragma unroll
      for (int i = 0; i < NV; i++) pacc[i] += ex[i] * rz;
    }
  }
  nslots = (int)wave_sum_f32((float)nslots);
  if (lane == 0) atomicAdd(&s_cnt[E + 1], nslots);
  if (want_p) {
    // the wave's token groups summed over a fixed tree (lanes sl of every group hold
    // the same experts), then the first group's lanes write the wave's row
#pragma unroll
    for (int o = LPT; o < kWave; o <<= 1)
#pragma unroll
      for (int i = 0; i < NV; i++) pacc[i] += __shfl_xor(pacc[i], o, kWave);
    if (sub == 0) {
#pragma unroll
      for (int i = 0; i < NV; i++) {
        const int e = sl + LPT * i;
        if (FULL || e < E) s_p[w * E + e] = pacc[i];
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


hipError_t launch_route_hist(const void *logits, bool bf16, int N, int E, int K, int mode,
                             int renorm, bool want_p, int32_t *topk_idx, float *topk_w,
                             int32_t *meta_ws, float *ppart, hipStream_t stream) {
  const MetaWs L = meta_ws_layout((int64_t)N * K, E);
  const size_t sh = (size_t)(E + 2) * sizeof(int32_t) +
                    (size_t)(kRouteThreads / kWave) * E * sizeof(float);
  // 8 lanes per token when E <= 128 and K <= 8 (the K selected experts end on lanes
  // 0..K-1); 16 when E <= 256 and K <= 16; else a whole wavefront
  const bool eighth = E <= 8 * kMaxPerLane && K <= 8;
  const bool narrow = E <= 16 * kMaxPerLane && K <= 16;
  const int lpt = eighth ? 8 : narrow ? 16 : kWave;
  const int need = (E + lpt - 1) / lpt;  // logits per lane, rounded up to a power of two
  const int nv = need <= 1 ? 1 : need <= 2 ? 2 : need <= 4 ? 4 : need <= 8 ? 8 : 16;
#define MOE_ROUTE(T, LPT, NV)                                                              \
  if (E == (LPT) * (NV))                                                                   \
    hipLaunchKernelGGL((route_hist_kernel<T, LPT, NV, true>), dim3(L.nblk), dim3(kRouteThreads), \
                       sh, stream, (const T *)logits, N, E, K, mode, renorm, (int)want_p,   \
                       topk_idx, topk_w, meta_ws + L.hist, ppart, meta_chunk((int64_t)N * K)); \
  else                                                                                     \
    hipLaunchKernelGGL((route_hist_kernel<T, LPT, NV, false>), dim3(L.nblk), dim3(kRouteThreads), \
                       sh, stream, (const T *)logits, N, E, K, mode, renorm, (int)want_p,   \
                       topk_idx, topk_w, meta_ws + L.hist, ppart, meta_chunk((int64_t)N * K))
#define MOE_ROUTE_NV(T, LPT)                                                               \
  switch (nv) {                                                                            \
    case 1: MOE_ROUTE(T, LPT, 1); break;                                                   \
    case 2: MOE_ROUTE(T, LPT, 2); break;                                                   \
    case 4: MOE_ROUTE(T, LPT, 4); break;                                                   \
    case 8: MOE_ROUTE(T, LPT, 8); break;                                                   \
    default: MOE_ROUTE(T, LPT, 16); break;                                                 \
  }
  if (bf16) {
    if (eighth) { MOE_ROUTE_NV(uint16_t, 8) }
    else if (narrow) { MOE_ROUTE_NV(uint16_t, 16) }
    else { MOE_ROUTE_NV(uint16_t, 64) }
  } else {
    if (eighth) { MOE_ROUTE_NV(float, 8) }
    else if (narrow) { MOE_ROUTE_NV(float, 16) }
    else { MOE_ROUTE_NV(float, 64) }
  }
#undef MOE_ROUTE_NV
#undef MOE_ROUTE
  return hipGetLastError();
}

}  // namespace moe
