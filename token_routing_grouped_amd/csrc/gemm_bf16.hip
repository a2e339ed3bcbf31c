// Grouped GEMMs of the expert layer on gfx950 bf16 matrix cores (fp32 accumulation).
//
// The serving-script notes (Qwen3.6 commit, "Optimization (CCCL segmented-sort
// pattern)") sort pairs by expert so each expert's rows are contiguous, but keep
// one F.linear per expert because variable-size GEMMs cannot be batched there;
// GitHub issue #68 keeps SonicMoE's grouped GEMM for the expert compute. Here one
// launch covers every expert:
//  - grouped-M: a workgroup owns a 128x128 output tile of one expert segment.
//    It reads the segment offsets (expert_frequency_offset), counts
//    ceil(freq_e/128) row tiles per expert, and finds its (expert, first row,
//    column tile) itself, so the grid is sized from the capacity alone and no
//    host sync is needed; surplus workgroups exit. Partial row tiles are padded
//    with zeros in LDS, never in memory. The A rows are gathered through a row
//    map (x_gather_idx) directly in the tile load.
//  - varlen-K (weight gradients): a workgroup owns a 128x128 tile of one
//    expert's gradient and reduces over that expert's rows; empty experts write
//    exact zeros.
// Workgroup ids are regrouped so that each of the 8 XCDs runs a contiguous run
// of tiles (tiles of one expert share weights, consecutive column tiles share
// the gathered rows), which keeps the reuse inside one L2.
//
// Tile: 128x128x64, 256 threads = 2x2 waves of 64x64, each wave 2x2
// v_mfma_f32_32x32x16_bf16. LDS holds two stages of an A and a B tile. Operands
// whose reduction index is contiguous in memory are stored [rows][64+8] and read
// with 16-byte LDS loads; operands contiguous along M or N are stored as loaded,
// [64][128+16], and read with ds_read_b64_tr_b16 (transposing LDS reads), so no
// operand is transposed in registers.
#include "common.h"
#include "kernels.h"
#include "../../include/moe.h"

namespace moe {
namespace {

constexpr int BM = kGemmBM, BN = kGemmBN, BK = kGemmBK, NT = 256;
constexpr int LDK = BK + 8;    // row stride of a reduction-contiguous tile [128][BK]
constexpr int LDC = 128 + 16;  // row stride of an M/N-contiguous tile [BK][128]
constexpr int TILE = 128 * LDK;
static_assert(BK * LDC == TILE, "both tile kinds take the same LDS");

enum { GROUPED_M = 0, VARLEN_K = 1 };
enum { EPI_STORE = 0, EPI_SWIGLU = 1, EPI_DSWIGLU = 2 };

typedef short i16x8 __attribute__((ext_vector_type(8)));

__device__ __forceinline__ bf16x8 frag_kc(const uint16_t *tile, int r, int kk) {
  return __builtin_bit_cast(bf16x8, *(const uint4 *)(tile + r * LDK + kk));
}

// B (or A) operand of v_mfma_f32_32x32x16_bf16 from a [k][col] tile: lane l needs
// rows kbase + (l/32)*8 + 0..7 of column cbase + l%32. One ds_read_b64_tr_b16 gives
// each lane of a 16-lane group 4 consecutive rows of one column when lane j of the
// group points at row k0 + j/4, columns c0 + (j%4)*4 .. +3.
__device__ __forceinline__ bf16x8 frag_mn(const uint16_t *tile, int kbase, int cbase, int lane) {
  const int g = lane >> 4, j = lane & 15;
  const int c = cbase + (g & 1) * 16 + (j & 3) * 4;
  const int k = kbase + (g >> 1) * 8 + (j >> 2);
  i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)(tile + k * LDC + c));
  i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)(tile + (k + 4) * LDC + c));
  i16x8 v = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  return __builtin_bit_cast(bf16x8, v);
}

template <int MODE, bool A_KC, bool B_KC, int EPI>
__global__ __launch_bounds__(NT, 2) void gemm_bf16_kernel(GemmArgs g) {
  __shared__ __attribute__((aligned(16))) uint16_t smem[4 * TILE];  // [stage][A | B]
  __shared__ int s_pref[MOE_MAX_EXPERTS + 2];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int P = g.foff[g.E];
  const uint16_t *A = (const uint16_t *)g.A;
  const uint16_t *B = (const uint16_t *)g.B;

  int e, mt = 0, nt, row0 = 0, rows = 0, seg0 = 0, seglen = 0, nk;
  if constexpr (MODE == GROUPED_M) {
    if (P > g.cap) return;
    for (int i = tid; i < g.E; i += NT) s_pref[i] = (g.foff[i + 1] - g.foff[i] + BM - 1) / BM;
    __syncthreads();
    wave0_exclusive_scan(s_pref, g.E);
    __syncthreads();
    const int ntn = g.N / BN;
    const int G = s_pref[g.E] * ntn;
    if ((int)blockIdx.x >= G) return;
    const int L = xcd_chunked(blockIdx.x, G);
    const int mtile = L / ntn;
    nt = L - mtile * ntn;
    int lo = 0, hi = g.E - 1;  // largest e with s_pref[e] <= mtile
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (s_pref[mid] <= mtile) lo = mid; else hi = mid - 1;
    }
    e = lo;
    row0 = g.foff[e] + (mtile - s_pref[e]) * BM;
    rows = min(BM, g.foff[e + 1] - row0);
    nk = g.K / BK;
  } else {
    const int mtn = g.M / BM, ntn = g.N / BN;
    const int L = xcd_chunked(blockIdx.x, g.E * mtn * ntn);
    e = L / (mtn * ntn);
    const int r = L - e * (mtn * ntn);
    mt = r / ntn;
    nt = r - mt * ntn;
    seg0 = g.foff[e];
    seglen = P > g.cap ? 0 : g.foff[e + 1] - seg0;
    nk = (seglen + BK - 1) / BK;
  }

  // ---- per-thread load state
  // k-contiguous tiles: rows (tid>>3) + 32*i, 16-byte chunk (tid&7)
  // mn-contiguous tiles: k-rows (tid>>4) + 16*i, 16-byte chunk (tid&15)
  const uint16_t *a_row[4];
  bool a_ok[4];
  const uint16_t *b_row[4];
  if constexpr (MODE == GROUPED_M) {
#pragma unroll
    for (int i = 0; i < 4; i++) {
      const int r = (tid >> 3) + 32 * i;
      a_ok[i] = r < rows;
      const int s = row0 + r;
      const int64_t gr = a_ok[i] ? (g.a_rows ? g.a_rows[s] : s) : 0;
      a_row[i] = A + gr * g.lda + (tid & 7) * 8;
      if constexpr (B_KC) {
        const int64_t n = (int64_t)nt * BN + (tid >> 3) + 32 * i;
        b_row[i] = B + (int64_t)e * g.b_es + n * g.ldb + (tid & 7) * 8;
      } else {
        b_row[i] = B + (int64_t)e * g.b_es + (int64_t)((tid >> 4) + 16 * i) * g.ldb +
                   (int64_t)nt * BN + (tid & 15) * 8;
      }
    }
  }

  uint4 ra[4], rb[4];
  auto load = [&](int k0) {
    if constexpr (MODE == GROUPED_M) {
#pragma unroll
      for (int i = 0; i < 4; i++) {
        ra[i] = a_ok[i] ? *(const uint4 *)(a_row[i] + k0) : make_uint4(0, 0, 0, 0);
        if constexpr (B_KC)
          rb[i] = *(const uint4 *)(b_row[i] + k0);
        else
          rb[i] = *(const uint4 *)(b_row[i] + (int64_t)k0 * g.ldb);
      }
    } else {
#pragma unroll
      for (int i = 0; i < 4; i++) {
        const int kk = k0 + (tid >> 4) + 16 * i;
        if (kk < seglen) {
          const int s = seg0 + kk;
          const int64_t ga = g.a_rows ? g.a_rows[s] : s;
          const int64_t gb = g.b_rows ? g.b_rows[s] : s;
          ra[i] = *(const uint4 *)(A + ga * g.lda + (int64_t)mt * BM + (tid & 15) * 8);
          rb[i] = *(const uint4 *)(B + gb * g.ldb + (int64_t)nt * BN + (tid & 15) * 8);
        } else {
          ra[i] = make_uint4(0, 0, 0, 0);
          rb[i] = make_uint4(0, 0, 0, 0);
        }
      }
    }
  };
  auto store = [&](int stage) {
    uint16_t *As = smem + stage * 2 * TILE;
    uint16_t *Bs = As + TILE;
#pragma unroll
    for (int i = 0; i < 4; i++) {
      if constexpr (A_KC)
        *(uint4 *)(As + ((tid >> 3) + 32 * i) * LDK + (tid & 7) * 8) = ra[i];
      else
        *(uint4 *)(As + ((tid >> 4) + 16 * i) * LDC + (tid & 15) * 8) = ra[i];
      if constexpr (B_KC) {
        *(uint4 *)(Bs + ((tid >> 3) + 32 * i) * LDK + (tid & 7) * 8) = rb[i];
      } else if constexpr (EPI == EPI_SWIGLU) {
        // interleaved (gate_j, up_j) columns -> gates of the wave's 32 pairs, then ups
        const int nc = tid & 15;
        const int base = ((tid >> 4) + 16 * i) * LDC + (nc >> 3) * 64 + 4 * (nc & 7);
        const uint4 v = rb[i];
        uint2 gate, up;
        gate.x = (v.x & 0xffffu) | (v.y << 16);
        gate.y = (v.z & 0xffffu) | (v.w << 16);
        up.x = (v.x >> 16) | (v.y & 0xffff0000u);
        up.y = (v.z >> 16) | (v.w & 0xffff0000u);
        *(uint2 *)(Bs + base) = gate;
        *(uint2 *)(Bs + base + 32) = up;
      } else {
        *(uint4 *)(Bs + ((tid >> 4) + 16 * i) * LDC + (tid & 15) * 8) = rb[i];
      }
    }
  };

  f32x16 acc[2][2];
#pragma unroll
  for (int mi = 0; mi < 2; mi++)
#pragma unroll
    for (int ni = 0; ni < 2; ni++)
#pragma unroll
      for (int r = 0; r < 16; r++) acc[mi][ni][r] = 0.0f;

  if (nk > 0) {
    load(0);
    store(0);
  }
  __syncthreads();
  for (int kt = 0; kt < nk; kt++) {
    const int cur = kt & 1;
    if (kt + 1 < nk) load((kt + 1) * BK);
    const uint16_t *As = smem + cur * 2 * TILE;
    const uint16_t *Bs = As + TILE;
#pragma unroll
    for (int ks = 0; ks < BK / 16; ks++) {
      bf16x8 af[2], bfr[2];
#pragma unroll
      for (int mi = 0; mi < 2; mi++) {
        if constexpr (A_KC)
          af[mi] = frag_kc(As, wm * 64 + mi * 32 + (lane & 31), ks * 16 + (lane >> 5) * 8);
        else
          af[mi] = frag_mn(As, ks * 16, wm * 64 + mi * 32, lane);
      }
#pragma unroll
      for (int ni = 0; ni < 2; ni++) {
        if constexpr (B_KC)
          bfr[ni] = frag_kc(Bs, wn * 64 + ni * 32 + (lane & 31), ks * 16 + (lane >> 5) * 8);
        else
          bfr[ni] = frag_mn(Bs, ks * 16, wn * 64 + ni * 32, lane);
      }
#pragma unroll
      for (int mi = 0; mi < 2; mi++)
#pragma unroll
        for (int ni = 0; ni < 2; ni++)
          acc[mi][ni] =
              __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[mi], bfr[ni], acc[mi][ni], 0, 0, 0);
    }
    if (kt + 1 < nk) store(cur ^ 1);
    __syncthreads();
  }

  // ---- epilogues. Accumulator (mi, ni, r) of lane l holds tile row
  // wm*64 + mi*32 + (r/4)*8 + (l/32)*4 + r%4 and column wn*64 + ni*32 + l%32.
  const int col_l = lane & 31;
  if constexpr (EPI == EPI_STORE) {
    uint16_t *C = (uint16_t *)g.C;
#pragma unroll
    for (int mi = 0; mi < 2; mi++)
#pragma unroll
      for (int r = 0; r < 16; r++) {
        const int row = wm * 64 + mi * 32 + (r >> 2) * 8 + (lane >> 5) * 4 + (r & 3);
        int64_t off;
        if constexpr (MODE == GROUPED_M) {
          if (row >= rows) continue;
          off = (int64_t)(row0 + row) * g.ldc;
        } else {
          off = (int64_t)e * g.c_es + (int64_t)(mt * BM + row) * g.ldc;
        }
#pragma unroll
        for (int ni = 0; ni < 2; ni++)
          C[off + (int64_t)nt * BN + wn * 64 + ni * 32 + col_l] = f32_to_bf16(acc[mi][ni][r]);
      }
  } else if constexpr (EPI == EPI_SWIGLU) {
    uint16_t *Hs = (uint16_t *)g.C;  // may be null (inference)
    uint16_t *Aout = (uint16_t *)g.C2;
    const int pair = nt * (BN / 2) + wn * 32 + col_l;
#pragma unroll
    for (int mi = 0; mi < 2; mi++)
#pragma unroll
      for (int r = 0; r < 16; r++) {
        const int row = wm * 64 + mi * 32 + (r >> 2) * 8 + (lane >> 5) * 4 + (r & 3);
        if (row >= rows) continue;
        const int64_t s = row0 + row;
        const float gt = acc[mi][0][r], up = acc[mi][1][r];
        if (Hs) *(uint32_t *)(Hs + s * g.ldc + 2 * pair) = pack_bf16x2(gt, up);
        Aout[s * g.ldc2 + pair] = f32_to_bf16(silu_f(gt) * up);
      }
  } else {  // EPI_DSWIGLU: acc = da_u = dout_g W_down^T for pair columns j
    uint16_t *dH = (uint16_t *)g.C;
    uint16_t *AW = (uint16_t *)g.C2;
    const uint16_t *Hs = (const uint16_t *)g.Hs;
    float *red = (float *)smem;  // [2][128] row partials of the two column waves
#pragma unroll
    for (int mi = 0; mi < 2; mi++)
#pragma unroll
      for (int r = 0; r < 16; r++) {
        const int row = wm * 64 + mi * 32 + (r >> 2) * 8 + (lane >> 5) * 4 + (r & 3);
        float part = 0.0f;
        if (row < rows) {
          const int64_t s = row0 + row;
          const float wq = g.scores[g.s_scatter[s]];
#pragma unroll
          for (int ni = 0; ni < 2; ni++) {
            const int j = nt * BN + wn * 64 + ni * 32 + col_l;
            const uint32_t hv = *(const uint32_t *)(Hs + s * g.ldh + 2 * j);
            const float gt = bf16_to_f32((uint16_t)(hv & 0xffffu));
            const float up = bf16_to_f32((uint16_t)(hv >> 16));
            const float dau = acc[mi][ni][r];
            const float sg = sigmoid_f(gt);
            const float a = gt * sg * up;
            part += dau * a;
            const float da = wq * dau;
            const float dg = da * up * sg * (1.0f + gt * (1.0f - sg));
            const float du = da * gt * sg;
            *(uint32_t *)(dH + s * g.ldc + 2 * j) = pack_bf16x2(dg, du);
            AW[s * g.ldc2 + j] = f32_to_bf16(wq * a);
          }
        }
#pragma unroll
        for (int o = 16; o >= 1; o >>= 1) part += __shfl_xor(part, o, kWave);
        if (col_l == 0) red[wn * 128 + row] = part;
      }
    __syncthreads();
    if (tid < BM && tid < rows)
      g.partial[(int64_t)(row0 + tid) * g.n_ntiles + nt] = red[tid] + red[128 + tid];
  }
}

}  // namespace

int gemm_grid(GemmKind kind, const GemmArgs &g) {
  if (kind == kWeightGrad) return g.E * (g.M / BM) * (g.N / BN);
  const int64_t mt = ((int64_t)g.cap + (int64_t)g.E * (BM - 1)) / BM;
  const int64_t grid = mt * (g.N / BN);
  return grid > 0x7fffffff ? -1 : (int)grid;
}

hipError_t launch_gemm_bf16(GemmKind kind, const GemmArgs &g, hipStream_t st) {
  const int grid = gemm_grid(kind, g);
  if (grid < 0) return hipErrorInvalidValue;
  if (grid == 0) return hipSuccess;
  switch (kind) {
    case kUpSwiGLU:
      hipLaunchKernelGGL((gemm_bf16_kernel<GROUPED_M, true, false, EPI_SWIGLU>), dim3(grid),
                         dim3(NT), 0, st, g);
      break;
    case kDown:
      hipLaunchKernelGGL((gemm_bf16_kernel<GROUPED_M, true, false, EPI_STORE>), dim3(grid),
                         dim3(NT), 0, st, g);
      break;
    case kDownBwd:
      hipLaunchKernelGGL((gemm_bf16_kernel<GROUPED_M, true, true, EPI_DSWIGLU>), dim3(grid),
                         dim3(NT), 0, st, g);
      break;
    case kUpBwd:
      hipLaunchKernelGGL((gemm_bf16_kernel<GROUPED_M, true, true, EPI_STORE>), dim3(grid),
                         dim3(NT), 0, st, g);
      break;
    case kWeightGrad:
      hipLaunchKernelGGL((gemm_bf16_kernel<VARLEN_K, false, false, EPI_STORE>), dim3(grid),
                         dim3(NT), 0, st, g);
      break;
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace moe
