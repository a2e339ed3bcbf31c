// Weighted combine back to token order, and the router-weight gradient.
//
// The serving-script notes (Qwen3.6 commit, step 5) scatter expert rows back with
// one index_add_, and the AWS NKI unpermute_a2av reference scatter-adds received
// rows to their token positions, accumulating over top-k. Both orders of summation
// depend on atomics. Here each token's row is produced by one wavefront that
// walks the token's pairs in ascending pair order (the CSR row pointer
// num_activated_expert_per_token_offset) and sums in fp32 with one final
// rounding: deterministic, no atomics, every output row written once.
#include "common.h"
#include "kernels.h"

namespace moe {
namespace {

constexpr int CT = 256;  // 4 tokens per workgroup, one wave each
constexpr int CHUNKS = 4;  // 16-byte chunks per lane kept in flight

template <typename T>
struct Vec;
template <>
struct Vec<uint16_t> {  // bf16: 8 elements per 16 bytes
  static constexpr int n = 8;
  __device__ static void to_f32(const uint4 &v, float *f) {
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; i++) {
      f[2 * i] = bf16_to_f32((uint16_t)(w[i] & 0xffffu));
      f[2 * i + 1] = bf16_to_f32((uint16_t)(w[i] >> 16));
    }
  }
  __device__ static uint4 from_f32(const float *f) {
    return make_uint4(pack_bf16x2(f[0], f[1]), pack_bf16x2(f[2], f[3]), pack_bf16x2(f[4], f[5]),
                      pack_bf16x2(f[6], f[7]));
  }
};
template <>
struct Vec<float> {  // fp32: 4 elements per 16 bytes
  static constexpr int n = 4;
  __device__ static void to_f32(const uint4 &v, float *f) {
    f[0] = __uint_as_float(v.x);
    f[1] = __uint_as_float(v.y);
    f[2] = __uint_as_float(v.z);
    f[3] = __uint_as_float(v.w);
  }
  __device__ static uint4 from_f32(const float *f) {
    return make_uint4(__float_as_uint(f[0]), __float_as_uint(f[1]), __float_as_uint(f[2]),
                      __float_as_uint(f[3]));
  }
};

template <typename T>
__global__ __launch_bounds__(CT) void combine_kernel(const T *__restrict__ y,
                                                    const int32_t *__restrict__ tok_off,
                                                    const int32_t *__restrict__ s_rev,
                                                    const float *__restrict__ scores, int N,
                                                    int H, int cap, T *__restrict__ out) {
  constexpr int V = Vec<T>::n;
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * (CT / 64) + (threadIdx.x >> 6);
  if (t >= N) return;
  const bool over = tok_off[N] > cap;
  const int q0 = tok_off[t];
  const int q1 = over ? q0 : tok_off[t + 1];
  const int nchunk = H / V;
  uint4 *orow = (uint4 *)(out + (int64_t)t * H);
  for (int c0 = 0; c0 < nchunk; c0 += 64 * CHUNKS) {
    float acc[CHUNKS][V];
#pragma unroll
    for (int i = 0; i < CHUNKS; i++)
#pragma unroll
      for (int v = 0; v < V; v++) acc[i][v] = 0.0f;
    for (int q = q0; q < q1; q++) {
      const int s = s_rev[q];
      const float w = scores ? scores[q] : 1.0f;
      const uint4 *yrow = (const uint4 *)(y + (int64_t)s * H);
      uint4 raw[CHUNKS];
#pragma unroll
      for (int i = 0; i < CHUNKS; i++) {
        const int c = c0 + i * 64 + lane;
        raw[i] = c < nchunk ? yrow[c] : make_uint4(0, 0, 0, 0);
      }
#pragma unroll
      for (int i = 0; i < CHUNKS; i++) {
        float f[V];
        Vec<T>::to_f32(raw[i], f);
#pragma unroll
        for (int v = 0; v < V; v++) acc[i][v] += w * f[v];
      }
    }
#pragma unroll
    for (int i = 0; i < CHUNKS; i++) {
      const int c = c0 + i * 64 + lane;
      if (c < nchunk) orow[c] = Vec<T>::from_f32(acc[i]);
    }
  }
}

__global__ __launch_bounds__(256) void dscore_kernel(const int32_t *__restrict__ idx, int N,
                                                     int K, int E,
                                                     const int32_t *__restrict__ tok_off,
                                                     const int32_t *__restrict__ s_rev,
                                                     const float *__restrict__ partial, int nnt,
                                                     int cap, float *__restrict__ dtw) {
  const int t = blockIdx.x * 256 + threadIdx.x;
  if (t >= N) return;
  const bool over = tok_off[N] > cap;
  int q = tok_off[t];
  for (int k = 0; k < K; k++) {
    const int e = idx[(int64_t)t * K + k];
    float v = 0.0f;
    if ((unsigned)e < (unsigned)E) {
      if (!over) {
        const float *p = partial + (int64_t)s_rev[q] * nnt;
        for (int i = 0; i < nnt; i++) v += p[i];
      }
      q++;
    }
    dtw[(int64_t)t * K + k] = v;
  }
}

}  // namespace

hipError_t launch_combine(bool bf16, const void *y, const int32_t *tok_off, const int32_t *s_rev,
                          const float *scores, int N, int H, int cap, void *out,
                          hipStream_t stream) {
  if (N == 0) return hipSuccess;
  const int grid = (N + 3) / 4;
  if (bf16)
    hipLaunchKernelGGL(combine_kernel<uint16_t>, dim3(grid), dim3(CT), 0, stream,
                       (const uint16_t *)y, tok_off, s_rev, scores, N, H, cap, (uint16_t *)out);
  else
    hipLaunchKernelGGL(combine_kernel<float>, dim3(grid), dim3(CT), 0, stream, (const float *)y,
                       tok_off, s_rev, scores, N, H, cap, (float *)out);
  return hipGetLastError();
}

hipError_t launch_dscore(const int32_t *topk_idx, int N, int K, int E, const int32_t *tok_off,
                         const int32_t *s_rev, const float *partial, int n_ntiles, int cap,
                         float *d_topk_weights, hipStream_t stream) {
  if (N == 0) return hipSuccess;
  hipLaunchKernelGGL(dscore_kernel, dim3((N + 255) / 256), dim3(256), 0, stream, topk_idx, N, K,
                     E, tok_off, s_rev, partial, n_ntiles, cap, d_topk_weights);
  return hipGetLastError();
}

}  // namespace moe
