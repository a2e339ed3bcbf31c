// Host-side launchers of the gfx950 kernels (internal to libmoe).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

// ---- routing metadata -------------------------------------------------------
constexpr int kMetaThreads = 256;
// Slots per thread of the metadata kernels: 2 (chunks of 512 slots, enough workgroups
// to fill the chip) below 2^20 slots, 4 (chunks of 1024) below 2^22, else 8: longer runs
// per expert in the sorted writes and fewer, shorter prefix columns as the slots grow
// (512 -> 1024 measured 84 -> 70 us at 2^23 slots).
inline int meta_items(int64_t NK) {
  return NK >= ((int64_t)1 << 22) ? 8 : NK >= ((int64_t)1 << 20) ? 4 : 2;
}
inline int meta_chunk(int64_t NK) { return kMetaThreads * meta_items(NK); }
// The scatter pass ranks a round's lanes per expert through per-wave LDS masks (64-bit
// words, [waves][E] ahead of its other LDS arrays) up to 256 experts and below 2^21
// slots; otherwise with one ballot per expert-id bit. Above 2^21 slots the pass is bound
// by its LDS traffic (the sorted staging), and the masks' three LDS instructions per
// round cost more than the ballots (measured 2-4 % slower there, 2-4 % faster below).
constexpr int kMetaMaskExperts = 256;
constexpr int64_t kMetaMaskSlots = (int64_t)1 << 21;
constexpr bool meta_use_mask(int64_t NK, int E) {
  return E <= kMetaMaskExperts && NK < kMetaMaskSlots;
}
inline int meta_mask_ints(int64_t NK, int E, int waves) {
  return meta_use_mask(NK, E) ? 2 * waves * E : 0;
}

struct MetaOut {
  int32_t *expert_frequency, *expert_frequency_offset, *x_gather_idx, *s_scatter_idx,
      *s_reverse_scatter_idx, *tok_off;
  float *router_scores;
  uint32_t *status;
  // router only: aux = aux_scale * sum_e count_e * psum[e] (written by workgroup 0)
  float *aux = nullptr;
  const float *psum = nullptr;
  float aux_scale = 0.0f;
};

inline int meta_blocks(int64_t NK) {
  const int c = meta_chunk(NK);
  int64_t b = (NK + c - 1) / c;
  return b < 1 ? 1 : (int)b;
}
// metadata workspace, in int32 elements: per-chunk histogram columns [E+2][nblk],
// per-chunk exclusive prefixes [nblk][E+2], column totals [E+2], and the segment sums
// of the two-pass scan for long columns ([2E+2][nseg]: the E+2 count columns, then the
// router's E probability columns)
// chunks per scan thread: 8 up to 2048 chunks, else 16 (one pass up to 4096 chunks)
inline int scan_per(int nblk) { return nblk > kMetaThreads * 8 ? 16 : 8; }
inline int scan_seg(int nblk) { return kMetaThreads * scan_per(nblk); }  // chunks per segment
struct MetaWs {
  int nblk, nseg;
  size_t hist, pre, tot, seg, total;
};
inline MetaWs meta_ws_layout(int64_t NK, int E) {
  MetaWs L;
  L.nblk = meta_blocks(NK);
  L.nseg = (L.nblk + scan_seg(L.nblk) - 1) / scan_seg(L.nblk);
  const size_t cells = (size_t)L.nblk * (size_t)(E + 2);
  L.hist = 0;
  L.pre = cells;
  L.tot = 2 * cells;
  L.seg = L.tot + (size_t)(E + 2);
  L.total = L.seg + (size_t)(2 * E + 2) * (size_t)L.nseg;
  return L;
}
inline size_t meta_workspace_bytes(int64_t NK, int E) {
  return meta_ws_layout(NK, E).total * sizeof(int32_t);
}
hipError_t launch_meta_hist(const int32_t *topk_idx, int N, int K, int E, int32_t *ws,
                            hipStream_t stream);
// fcol (router only, else null): E float columns [E][nblk] whose fixed-order sums go
// to fsum [E]
hipError_t launch_meta_scan(int N, int K, int E, int32_t *ws, hipStream_t stream,
                            const float *fcol = nullptr, float *fsum = nullptr);
// Scatter pass modes. kMetaScanned: after the histogram and scan launches. kMetaFused:
// after the histogram launch only, summing the per-chunk counts itself; where
// meta_fused_scan(N*K, E) holds (few chunks and experts). kMetaSolo: the whole build in
// one workgroup (counts included) and no workspace; where meta_solo(N*K) holds. The
// router's build is always kMetaScanned.
enum { kMetaScanned = 0, kMetaFused = 1, kMetaSolo = 2 };
constexpr int64_t kMetaSoloSlots = 2048;  // one workgroup of 512 threads, 4 slots each
hipError_t launch_meta_scatter(const int32_t *topk_idx, const float *topk_weights, int N, int K,
                               int E, int capacity, const int32_t *ws, const MetaOut &out,
                               hipStream_t stream, int mode = kMetaScanned);
bool meta_fused_scan(int64_t NK, int E);
bool meta_solo(int64_t NK);

// ---- router (top-K + the metadata histogram pass, and the aux loss) ---------
size_t route_ws_floats(int64_t NK, int E);  // per-chunk P sums [E][nblk], then their totals [E]
hipError_t launch_route_hist(const void *logits, bool bf16, int N, int E, int K, int mode,
                             int renorm, bool want_p, int32_t *topk_idx, float *topk_w,
                             int32_t *meta_ws, float *ppart, hipStream_t stream);

// ---- grouped GEMMs (bf16 MFMA) ----------------------------------------------
// Two schedules:
//  grouped-M: C[s,:] = A[row(s),:] B_e for the rows s of each expert segment
//             (M varies per expert, N and K fixed);
//  varlen-K:  C_e = sum over the segment's rows s of A[row(s),:]^T B[row(s),:]
//             (M and N fixed, the reduction length varies per expert).
enum GemmKind {
  kUpSwiGLU = 0,   // h = x_g W_up (B [K][N]); epilogue writes h and a = silu(g)*u
  kDown = 1,       // y = a W_down (B [K][N])
  kDownBwd = 2,    // da_u = dout_g W_down^T (B [N][K]); epilogue: dSwiGLU, dscore partials
  kUpBwd = 3,      // dxg = dh W_up^T (B [N][K])
  kWeightGrad = 4  // varlen-K: dW_e = A_g^T B_g (both row-major over the segment)
};

struct GemmArgs {
  const int32_t *foff;  // [E+1] segment offsets of the sorted positions
  int E, cap;
  int M, N, K;  // grouped-M uses N, K; varlen-K uses M, N
  const void *A;
  int64_t lda, a_es;
  const int32_t *a_rows;  // row map (gather) or null = identity
  const void *B;
  int64_t ldb, b_es;
  const int32_t *b_rows;
  void *C;
  int64_t ldc, c_es;
  void *C2;  // kUpSwiGLU: a [cap,I]; kDownBwd: w*a [cap,I]
  int64_t ldc2;
  const void *Hs;  // kDownBwd: saved h [cap,2I]
  int64_t ldh;
  const float *scores;       // router_scores [cap] (pair order)
  const int32_t *s_scatter;  // s -> q
  float *partial;            // kDownBwd: [cap, n_ntiles] per-tile partial dscore
  int n_ntiles;
  int gu_concat;  // kUpSwiGLU / kDownBwd: W_up (and dh) columns are [gates | ups]
};

constexpr int kGemmBM = 128, kGemmBN = 128, kGemmBK = 64;  // smallest tile; fp32 mode tile
constexpr int64_t kGemmFewTiles = 256;  // grouped-M: below this many 256x256 tiles, 128x128
constexpr int64_t kWgradFewRows = 128;  // varlen-K: below this many rows per expert, 128x128
// bf16 tile shape chosen for a GEMM (BM x BN x BK), whether its edges are partial
// tiles, and its grid size (-1: too large)
bool gemm_ragged(GemmKind kind, const GemmArgs &g);
void gemm_tile(GemmKind kind, const GemmArgs &g, int *bm, int *bn, int *bk);
int gemm_grid(GemmKind kind, const GemmArgs &g);
int gemm_grid_f32(GemmKind kind, const GemmArgs &g);
hipError_t launch_gemm_bf16(GemmKind kind, const GemmArgs &g, hipStream_t stream);
hipError_t launch_gemm_f32(GemmKind kind, const GemmArgs &g, hipStream_t stream);

// ---- combine and router-weight gradient --------------------------------------
// out[t,:] = sum over the token's pairs q (ascending) of w_q * y[s_rev[q],:]
// (w_q = 1 when scores is null); fp32 accumulation, one rounding.
hipError_t launch_combine(bool bf16, const void *y, const int32_t *tok_off,
                          const int32_t *s_rev, const float *scores, int N, int H, int cap,
                          void *out, hipStream_t stream);
// The same for dx with unit weights, also writing d_topk_weights[t,k] = the sum over
// column tiles of partial[s_rev[q],tile] for the slot's pair q (0 at invalid slots).
hipError_t launch_combine_dscore(bool bf16, const void *dxg, const int32_t *tok_off,
                                 const int32_t *s_rev, int N, int H, int cap, void *dx,
                                 const int32_t *topk_idx, int K, int E, const float *partial,
                                 int n_ntiles, float *d_topk_weights, hipStream_t stream);

}  // namespace moe
