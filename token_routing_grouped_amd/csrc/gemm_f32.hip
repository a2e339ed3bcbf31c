// fp32 checking mode of the grouped GEMMs: fp32 storage and fp32 FMA arithmetic, so
// the method's indexing and epilogue arithmetic can be checked at fp32 tolerance
// instead of under bf16 rounding. Shared with the bf16 matrix-core kernels: the row
// maps (x_gather_idx, sorted positions, the expert segments of
// expert_frequency_offset), the per-expert row tiles found from the offsets on the
// device, and the epilogue formulas (SwiGLU; dSwiGLU with the router weight and the
// per-column-tile dscore partials; exact zeros for experts with no rows). Not shared:
// the tile schedules (one non-persistent 128x128 workgroup per tile, weight-gradient
// tiles dealt out flat rather than per XCD) and the store paths (direct per-lane
// stores, no LDS staging or lane exchanges), so a pass here says nothing about those
// parts of the bf16 kernels. Not tuned for speed.
#include "common.h"
#include "kernels.h"
#include "../../include/moe.h"

namespace moe {
namespace {

constexpr int BM = kGemmBM, BN = kGemmBN, BK = 16, NT = 256;
enum { GROUPED_M = 0, VARLEN_K = 1 };
enum { EPI_STORE = 0, EPI_SWIGLU = 1, EPI_DSWIGLU = 2 };

template <int MODE, bool A_KC, bool B_KC, int EPI>
__global__ __launch_bounds__(NT) void gemm_f32_kernel(GemmArgs g) {
  __shared__ float As[BK][BM + 4];
  __shared__ float Bs[BK][BN + 4];
  __shared__ int s_pref[MOE_MAX_EXPERTS + 2];
  const int tid = threadIdx.x, tx = tid & 15, ty = tid >> 4;
  const int P = g.foff[g.E];
  const float *A = (const float *)g.A;
  const float *B = (const float *)g.B;

  int e, mt = 0, nt, row0 = 0, rows = 0, seg0 = 0, seglen = 0, kend;
  if constexpr (MODE == GROUPED_M) {
    if (P > g.cap) return;
    for (int i = tid; i < g.E; i += NT) s_pref[i] = (g.foff[i + 1] - g.foff[i] + BM - 1) / BM;
    __syncthreads();
    wave0_exclusive_scan(s_pref, g.E);
    __syncthreads();
    const int ntn = (g.N + BN - 1) / BN;  // partial edge tiles: every access is bounded
    const int G = s_pref[g.E] * ntn;
    if ((int)blockIdx.x >= G) return;
    const int mtile = blockIdx.x / ntn;
    nt = blockIdx.x - mtile * ntn;
    int lo = 0, hi = g.E - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (s_pref[mid] <= mtile) lo = mid; else hi = mid - 1;
    }
    e = lo;
    row0 = g.foff[e] + (mtile - s_pref[e]) * BM;
    rows = min(BM, g.foff[e + 1] - row0);
    kend = g.K;
  } else {
    const int mtn = (g.M + BM - 1) / BM, ntn = (g.N + BN - 1) / BN;
    e = blockIdx.x / (mtn * ntn);
    const int r = blockIdx.x - e * (mtn * ntn);
    mt = r / ntn;
    nt = r - mt * ntn;
    seg0 = g.foff[e];
    seglen = P > g.cap ? 0 : g.foff[e + 1] - seg0;
    kend = seglen;
  }

  float acc[8][8];
#pragma unroll
  for (int i = 0; i < 8; i++)
#pragma unroll
    for (int j = 0; j < 8; j++) acc[i][j] = 0.0f;

  for (int k0 = 0; k0 < kend; k0 += BK) {
    // A tile -> As[k][m]
    if constexpr (MODE == GROUPED_M) {  // rows of A are k-contiguous
      const int r = tid >> 1, kk = (tid & 1) * 8;
      const bool ok = r < rows;
      const int s = row0 + r;
      const int64_t gr = ok ? (g.a_rows ? g.a_rows[s] : s) : 0;
#pragma unroll
      for (int i = 0; i < 8; i++)
        As[kk + i][r] = ok && k0 + kk + i < g.K ? A[gr * g.lda + k0 + kk + i] : 0.0f;
    } else {  // k-rows of A are m-contiguous
      const int kr = tid >> 4, m = (tid & 15) * 8;
      const int kk = k0 + kr;
      const bool ok = kk < seglen;
      const int64_t gr = ok ? (g.a_rows ? g.a_rows[seg0 + kk] : seg0 + kk) : 0;
#pragma unroll
      for (int i = 0; i < 8; i++) {
        const int mm = mt * BM + m + i;
        As[kr][m + i] = ok && mm < g.M ? A[gr * g.lda + mm] : 0.0f;
      }
    }
    // B tile -> Bs[k][n]
    if constexpr (MODE == GROUPED_M && B_KC) {  // weights [N][K]
      const int n = tid >> 1, kk = (tid & 1) * 8;
      const bool ok = nt * BN + n < g.N;
      const float *src = B + (int64_t)e * g.b_es + ((int64_t)nt * BN + n) * g.ldb + k0 + kk;
#pragma unroll
      for (int i = 0; i < 8; i++) Bs[kk + i][n] = ok && k0 + kk + i < g.K ? src[i] : 0.0f;
    } else if constexpr (MODE == GROUPED_M) {  // weights [K][N]
      const int kr = tid >> 4, n = (tid & 15) * 8;
      const bool ok = k0 + kr < g.K;
      const float *row = B + (int64_t)e * g.b_es + (int64_t)(k0 + kr) * g.ldb;
      if (EPI == EPI_SWIGLU && g.gu_concat) {  // tile column c holds gate/up of pair c/2
#pragma unroll
        for (int i = 0; i < 8; i++) {
          const int c = nt * BN + n + i;
          Bs[kr][n + i] = ok && c < g.N ? row[(c & 1) ? g.N / 2 + (c >> 1) : (c >> 1)] : 0.0f;
        }
      } else {
#pragma unroll
        for (int i = 0; i < 8; i++) {
          const int c = nt * BN + n + i;
          Bs[kr][n + i] = ok && c < g.N ? row[c] : 0.0f;
        }
      }
    } else {
      const int kr = tid >> 4, n = (tid & 15) * 8;
      const int kk = k0 + kr;
      const bool ok = kk < seglen;
      const int64_t gr = ok ? (g.b_rows ? g.b_rows[seg0 + kk] : seg0 + kk) : 0;
#pragma unroll
      for (int i = 0; i < 8; i++) {
        const int c = nt * BN + n + i;
        Bs[kr][n + i] = ok && c < g.N ? B[gr * g.ldb + c] : 0.0f;
      }
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < BK; kk++) {
      float a[8], b[8];
#pragma unroll
      for (int i = 0; i < 8; i++) a[i] = As[kk][ty * 8 + i];
#pragma unroll
      for (int j = 0; j < 8; j++) b[j] = Bs[kk][tx * 8 + j];
#pragma unroll
      for (int i = 0; i < 8; i++)
#pragma unroll
        for (int j = 0; j < 8; j++) acc[i][j] = fmaf(a[i], b[j], acc[i][j]);
    }
    __syncthreads();
  }

  // thread owns tile rows ty*8 + i, columns tx*8 + j
  if constexpr (EPI == EPI_STORE) {
    float *C = (float *)g.C;
#pragma unroll
    for (int i = 0; i < 8; i++) {
      const int row = ty * 8 + i;
      int64_t off;
      if constexpr (MODE == GROUPED_M) {
        if (row >= rows) continue;
        off = (int64_t)(row0 + row) * g.ldc;
      } else {
        if (mt * BM + row >= g.M) continue;
        off = (int64_t)e * g.c_es + (int64_t)(mt * BM + row) * g.ldc;
      }
#pragma unroll
      for (int j = 0; j < 8; j++) {
        const int c = nt * BN + tx * 8 + j;
        if (c < g.N) C[off + c] = acc[i][j];
      }
    }
  } else if constexpr (EPI == EPI_SWIGLU) {
    float *Hs = (float *)g.C;
    float *Aout = (float *)g.C2;
#pragma unroll
    for (int i = 0; i < 8; i++) {
      const int row = ty * 8 + i;
      if (row >= rows) continue;
      const int64_t s = row0 + row;
#pragma unroll
      for (int p = 0; p < 4; p++) {
        const int col = nt * BN + tx * 8 + 2 * p;
        if (col >= g.N) continue;
        const float gt = acc[i][2 * p], up = acc[i][2 * p + 1];
        if (Hs) {
          Hs[s * g.ldc + col] = gt;
          Hs[s * g.ldc + col + 1] = up;
        }
        Aout[s * g.ldc2 + col / 2] = silu_f(gt) * up;
      }
    }
  } else {  // EPI_DSWIGLU
    float *dH = (float *)g.C;
    float *AW = (float *)g.C2;
    const float *Hs = (const float *)g.Hs;
#pragma unroll
    for (int i = 0; i < 8; i++) {
      const int row = ty * 8 + i;
      float part = 0.0f;
      if (row < rows) {
        const int64_t s = row0 + row;
        const float wq = g.scores[g.s_scatter[s]];
#pragma unroll
        for (int jj = 0; jj < 8; jj++) {
          const int j = nt * BN + tx * 8 + jj;
          if (j >= g.N) continue;
          const float gt = Hs[s * g.ldh + 2 * j], up = Hs[s * g.ldh + 2 * j + 1];
          const float dau = acc[i][jj];
          const float sg = sigmoid_f(gt);
          const float a = gt * sg * up;
          part += dau * a;
          const float da = wq * dau;
          const int64_t cg = g.gu_concat ? j : 2 * j, cu = g.gu_concat ? g.N + j : 2 * j + 1;
          dH[s * g.ldc + cg] = da * up * sg * (1.0f + gt * (1.0f - sg));
          dH[s * g.ldc + cu] = da * gt * sg;
          AW[s * g.ldc2 + j] = wq * a;
        }
      }
#pragma unroll
      for (int o = 8; o >= 1; o >>= 1) part += __shfl_xor(part, o, kWave);
      if (tx == 0 && row < rows) g.partial[(int64_t)(row0 + row) * g.n_ntiles + nt] = part;
    }
  }
}

}  // namespace

hipError_t launch_gemm_f32(GemmKind kind, const GemmArgs &g, hipStream_t st) {
  const int grid = gemm_grid_f32(kind, g);
  if (grid < 0) return hipErrorInvalidValue;
  if (grid == 0) return hipSuccess;
  switch (kind) {
    case kUpSwiGLU:
      hipLaunchKernelGGL((gemm_f32_kernel<GROUPED_M, true, false, EPI_SWIGLU>), dim3(grid),
                         dim3(NT), 0, st, g);
      break;
    case kDown:
      hipLaunchKernelGGL((gemm_f32_kernel<GROUPED_M, true, false, EPI_STORE>), dim3(grid),
                         dim3(NT), 0, st, g);
      break;
    case kDownBwd:
      hipLaunchKernelGGL((gemm_f32_kernel<GROUPED_M, true, true, EPI_DSWIGLU>), dim3(grid),
                         dim3(NT), 0, st, g);
      break;
    case kUpBwd:
      hipLaunchKernelGGL((gemm_f32_kernel<GROUPED_M, true, true, EPI_STORE>), dim3(grid),
                         dim3(NT), 0, st, g);
      break;
    case kWeightGrad:
      hipLaunchKernelGGL((gemm_f32_kernel<VARLEN_K, false, false, EPI_STORE>), dim3(grid),
                         dim3(NT), 0, st, g);
      break;
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace moe
