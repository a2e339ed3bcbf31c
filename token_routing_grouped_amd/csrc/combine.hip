// Weighted combine back to token order, and the router-weight gradient.
//
// The serving-script notes (Qwen3.6 commit, step 5) scatter expert rows back with
// one index_add_, and the AWS NKI unpermute_a2av reference scatter-adds received
// rows to their token positions, accumulating over top-k. Both orders of summation
// depend on atomics. Here each token's row is produced by one wavefront that
// walks the token's pairs in ascending pair order (the CSR row pointer
// num_activated_expert_per_token_offset) and sums in fp32 with one final
// rounding: deterministic, no atomics, every output row written once.
//
// The wavefront first loads the token's pair metadata lane-parallel (lane j holds
// pair q0+j: its sorted position and weight), then streams the expert rows with
// several pairs' loads in flight. The backward variant also writes the token's
// row of d_topk_weights (issue #68, question 4: router gradients in [N,K]): slot k
// of a valid expert id is the token's (number of valid slots before k)-th pair,
// and its gradient is the sum, in tile order, of the per-column-tile partials the
// down-projection backward wrote for that pair.
#include "common.h"
#include "kernels.h"

namespace moe {
namespace {

constexpr int CT = 256;  // 4 tokens per workgroup, one wave each
// Row split: with few tokens (decode) one wave per token would stream its rows with only a
// few loads in flight, so the row is cut into column blocks of 64 chunks, one wave each
// (grid.y), and all of a block's pairs are loaded together.
constexpr int kSplitTokens = 4096;  // fewer tokens than this take the column blocks

template <typename T>
struct Vec;
template <>
struct Vec<uint16_t> {  // bf16: 8 elements per 16 bytes
  static constexpr int n = 8;
  __device__ static void add(const u32x4 &v, float w, float *f) {
#pragma unroll
    for (int i = 0; i < 4; i++) {
      f[2 * i] += w * bf16_to_f32((uint16_t)(v[i] & 0xffffu));
      f[2 * i + 1] += w * bf16_to_f32((uint16_t)(v[i] >> 16));
    }
  }
  __device__ static u32x4 pack(const float *f) {
    return u32x4{pack_bf16x2(f[0], f[1]), pack_bf16x2(f[2], f[3]), pack_bf16x2(f[4], f[5]),
                 pack_bf16x2(f[6], f[7])};
  }
};
template <>
struct Vec<float> {  // fp32: 4 elements per 16 bytes
  static constexpr int n = 4;
  __device__ static void add(const u32x4 &v, float w, float *f) {
#pragma unroll
    for (int i = 0; i < 4; i++) f[i] += w * __uint_as_float(v[i]);
  }
  __device__ static u32x4 pack(const float *f) {
    return u32x4{__float_as_uint(f[0]), __float_as_uint(f[1]), __float_as_uint(f[2]),
                 __float_as_uint(f[3])};
  }
};

struct DscoreArgs {
  const int32_t *topk_idx;
  int K, E;
  const float *partial;
  int nnt;
  float *dtw;
};

// CHUNKS: 16-byte chunks per lane per pass over the row; PAIRS: pairs whose rows are
// loaded together; grid.y: column blocks of 64*CHUNKS chunks (1 = whole rows)
template <typename T, bool DSCORE, int CHUNKS, int PAIRS>
__global__ __launch_bounds__(CT) void combine_kernel(const T *__restrict__ y,
                                                    const int32_t *__restrict__ tok_off,
                                                    const int32_t *__restrict__ s_rev,
                                                    const float *__restrict__ scores, int N,
                                                    int H, int cap, T *__restrict__ out,
                                                    DscoreArgs ds) {
  constexpr int V = Vec<T>::n;
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * (CT / 64) + (threadIdx.x >> 6);
  if (t >= N) return;
  const bool over = tok_off[N] > cap;
  const int q0 = tok_off[t];
  const int n = over ? 0 : tok_off[t + 1] - q0;  // pairs of this token (<= K <= 64)
  // lane j: the j-th pair's sorted position and weight
  const int my_s = lane < n ? s_rev[q0 + lane] : 0;
  const float my_w = lane < n ? (scores ? scores[q0 + lane] : 1.0f) : 0.0f;

  const int nchunk = H / V;
  u32x4 *orow = (u32x4 *)(out + (int64_t)t * H);
  for (int c0 = blockIdx.y * 64 * CHUNKS; c0 < nchunk; c0 += gridDim.y * 64 * CHUNKS) {
    float acc[CHUNKS][V];
#pragma unroll
    for (int i = 0; i < CHUNKS; i++)
#pragma unroll
      for (int v = 0; v < V; v++) acc[i][v] = 0.0f;
    for (int j0 = 0; j0 < n; j0 += PAIRS) {
      u32x4 raw[PAIRS][CHUNKS];
      float w[PAIRS];
#pragma unroll
      for (int p = 0; p < PAIRS; p++) {
        const int j = j0 + p < n ? j0 + p : j0;  // a missing second pair re-reads the first
        const int s = __shfl(my_s, j, kWave);
        w[p] = __shfl(my_w, j, kWave);
        const u32x4 *yrow = (const u32x4 *)(y + (int64_t)s * H);
#pragma unroll
        for (int i = 0; i < CHUNKS; i++) {
          const int c = c0 + i * 64 + lane;
          raw[p][i] = c < nchunk ? yrow[c] : u32x4{0, 0, 0, 0};
        }
      }
      // ascending pair order within and across groups
#pragma unroll
      for (int p = 0; p < PAIRS; p++) {
        if (j0 + p >= n) break;  // wave-uniform
#pragma unroll
        for (int i = 0; i < CHUNKS; i++) Vec<T>::add(raw[p][i], w[p], acc[i]);
      }
    }
#pragma unroll
    for (int i = 0; i < CHUNKS; i++) {
      const int c = c0 + i * 64 + lane;
      if (c < nchunk) __builtin_nontemporal_store(Vec<T>::pack(acc[i]), orow + c);  // final output
    }
  }

  if (DSCORE && blockIdx.y == 0) {
    const int K = ds.K;
    const int e = lane < K ? ds.topk_idx[(int64_t)t * K + lane] : -1;
    const bool valid = (unsigned)e < (unsigned)ds.E;
    const uint64_t vm = ballot64(valid);
    float v = 0.0f;
    if (valid && !over) {
      const int s = s_rev[q0 + popc_below(vm)];
      const float *p = ds.partial + (int64_t)s * ds.nnt;
      for (int i = 0; i < ds.nnt; i++) v += p[i];
    }
    if (lane < K) ds.dtw[(int64_t)t * K + lane] = v;
  }
}

template <typename T, bool DSCORE>
hipError_t launch_t(const void *y, const int32_t *tok_off, const int32_t *s_rev,
                    const float *scores, int N, int H, int cap, void *out, const DscoreArgs &ds,
                    hipStream_t stream) {
  const int grid = (N + 3) / 4;
  if (N < kSplitTokens) {
    constexpr int CH = 1;  // one chunk per lane: a column block is 64 chunks
    const int nblk = (H / Vec<T>::n + 64 * CH - 1) / (64 * CH);
    hipLaunchKernelGGL((combine_kernel<T, DSCORE, CH, 8>), dim3(grid, nblk), dim3(CT), 0, stream,
                       (const T *)y, tok_off, s_rev, scores, N, H, cap, (T *)out, ds);
  } else {
    hipLaunchKernelGGL((combine_kernel<T, DSCORE, 4, 2>), dim3(grid), dim3(CT), 0, stream,
                       (const T *)y, tok_off, s_rev, scores, N, H, cap, (T *)out, ds);
  }
  return hipGetLastError();
}

template <bool DSCORE>
hipError_t launch(bool bf16, const void *y, const int32_t *tok_off, const int32_t *s_rev,
                  const float *scores, int N, int H, int cap, void *out, const DscoreArgs &ds,
                  hipStream_t stream) {
  if (bf16)
    return launch_t<uint16_t, DSCORE>(y, tok_off, s_rev, scores, N, H, cap, out, ds, stream);
  return launch_t<float, DSCORE>(y, tok_off, s_rev, scores, N, H, cap, out, ds, stream);
}

}  // namespace

hipError_t launch_combine(bool bf16, const void *y, const int32_t *tok_off, const int32_t *s_rev,
                          const float *scores, int N, int H, int cap, void *out,
                          hipStream_t stream) {
  if (N == 0) return hipSuccess;
  DscoreArgs ds = {};
  return launch<false>(bf16, y, tok_off, s_rev, scores, N, H, cap, out, ds, stream);
}

hipError_t launch_combine_dscore(bool bf16, const void *dxg, const int32_t *tok_off,
                                 const int32_t *s_rev, int N, int H, int cap, void *dx,
                                 const int32_t *topk_idx, int K, int E, const float *partial,
                                 int n_ntiles, float *d_topk_weights, hipStream_t stream) {
  if (N == 0) return hipSuccess;
  DscoreArgs ds = {topk_idx, K, E, partial, n_ntiles, d_topk_weights};
  return launch<true>(bf16, dxg, tok_off, s_rev, nullptr, N, H, cap, dx, ds, stream);
}

}  // namespace moe
