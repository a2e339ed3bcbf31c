// Grouped GEMMs of the expert layer on gfx950 bf16 matrix cores (fp32 accumulation).
//
// The serving-script notes (Qwen3.6 commit, "Optimization (CCCL segmented-sort
// pattern)") sort pairs by expert so each expert's rows are contiguous, but keep
// one F.linear per expert because variable-size GEMMs cannot be batched there;
// GitHub issue #68 keeps SonicMoE's grouped GEMM for the expert compute. Here one
// launch covers every expert:
//  - grouped-M: a tile is a BMxBN output block of one expert segment. Each
//    workgroup reads the segment offsets (expert_frequency_offset), counts
//    ceil(freq_e/BM) row tiles per expert and finds the (expert, first row, column
//    tile) of every tile it takes itself, so the launch needs no host sync. The
//    workgroups are persistent (as many as the chip holds at once) and walk the
//    tiles of their XCD. Partial row tiles are padded in LDS (the padding rows read a
//    row of zeros), never in memory. A rows are gathered through a row map
//    (x_gather_idx) directly in the tile load.
//  - varlen-K (weight gradients): a workgroup owns a BMxBN tile of one expert's
//    gradient and reduces over that expert's rows; empty experts write zeros.
// Each of the 8 XCDs runs a contiguous run of tiles (tiles of one expert share
// weights, consecutive column tiles share the gathered rows), which keeps the reuse
// inside one L2; the weight gradients give each XCD whole experts where the experts'
// row counts are even enough, else a rectangle of every expert's tiles.
//
// Tiles (BM x BN x BK): 256x256x32 with 8 waves (2x4, wave tile 128x64), 128x128 with
// 4 waves, 32x128x64 with 2 waves; each wave's tile is built from
// v_mfma_f32_32x32x16_bf16. LDS holds two stages of an A and a B tile, filled from two
// register sets loaded two tiles ahead; the eight-wave grouped-M kernels run the two
// wave groups of each SIMD half a k-step apart (ping-pong), one multiplying while the
// other reads fragments and stages the next tile. Operands whose reduction index is
// contiguous in memory are stored [rows][BK] with 16-byte chunks swizzled per row and
// read with 16-byte LDS loads; operands contiguous along M or N are stored as loaded,
// [BK][cols+pad], and read with ds_read_b64_tr_b16 (transposing LDS reads), so no
// operand is transposed in registers (the padding: padc below). Outputs are staged
// through LDS so every row leaves as whole 128-byte lines.
//
// H and I need only be multiples of 8 (one 16-byte chunk). Shapes that leave partial
// tiles at the column (and reduction, or varlen-K row) edges take 128x128x32 tiles
// built with RAG, which bound every load and store at those edges without a
// condition around any memory access.
#include "common.h"
#include "kernels.h"
#include "../../include/moe.h"

namespace moe {
namespace {
// A row of zeros that padding rows of grouped-M tiles read (static storage starts zeroed
// and nothing writes it)
constexpr int kZeroRowElems = 1 << 16;
__device__ uint16_t g_zero_row[kZeroRowElems];

#ifndef MOE_KC_SWIZZLE
#define MOE_KC_SWIZZLE 1
#endif
// extra elements per row of a reduction-contiguous tile [rows][BK] (0: chunk swizzle)
constexpr int PADK = MOE_KC_SWIZZLE ? 0 : 8;
// extra columns of an M/N-contiguous tile [BK][cols]: 32 for 256-wide tiles (rows then
// start 64 bytes apart modulo the 256-byte bank span, and the transposing fragment reads
// of a wave run at 158-164 B/clk per CU against 128 with 16; measured on this part), 16
// for narrower tiles, where 32 would cost the second workgroup per CU its LDS
template <int R>
constexpr int padc() { return R >= 256 ? 32 : 16; }

enum { GROUPED_M = 0, VARLEN_K = 1 };
// EPI_SWIGLU: W_up interleaved (gate_j, up_j at 2j, 2j+1); EPI_SWIGLU_CAT: [gates | ups]
enum { EPI_STORE = 0, EPI_SWIGLU = 1, EPI_DSWIGLU = 2, EPI_SWIGLU_CAT = 3 };

typedef short i16x8 __attribute__((ext_vector_type(8)));

template <bool KC, int R, int BK>
struct TileShape {  // one LDS stage of an operand with R rows (M or N) and BK reduction
  static constexpr int ld = KC ? BK + PADK : R + padc<R>();
  static constexpr int elems = KC ? R * (BK + PADK) : BK * (R + padc<R>());
};

// Reduction-contiguous tile [rows][BK], unpadded: 16-byte chunk c of row r is stored at
// chunk c ^ kc_swz(r). Sixteen consecutive rows at one chunk (a fragment read) and one
// contiguous 256-byte run (a 16-lane group of the stage store) then cover all 64 banks:
// measured 196 B/clk per CU for the fragment reads, and the stage stores go from a
// 2.5x-conflicted pattern (padded rows) to conflict-free.
template <int BK>
__device__ __forceinline__ int kc_swz(int r) {
  constexpr int CPK = BK / 8, RPB = 16 / CPK;  // chunks per row, rows per 256 bytes
  return MOE_KC_SWIZZLE ? (r / RPB) % CPK : 0;
}
template <int LD, int BK>
__device__ __forceinline__ bf16x8 frag_kc(const uint16_t *tile, int r, int kk) {
  return __builtin_bit_cast(bf16x8,
                            *(const u32x4 *)(tile + r * LD + (((kk >> 3) ^ kc_swz<BK>(r)) << 3)));
}

// Operand of v_mfma_f32_32x32x16_bf16 from a [k][col] tile with row stride ld:
// lane l needs rows kbase + (l/32)*8 + 0..7 of column cbase + l%32. One
// ds_read_b64_tr_b16 gives each lane of a 16-lane group 4 consecutive rows of one
// column when lane j of the group points at row k0 + j/4, columns c0 + (j%4)*4 ..+3.
template <int LD>
__device__ __forceinline__ bf16x8 frag_mn(const uint16_t *tile, int kbase, int cbase, int lane) {
  const int g = lane >> 4, j = lane & 15;
  const int c = cbase + (g & 1) * 16 + (j & 3) * 4;
  const int k = kbase + (g >> 1) * 8 + (j >> 2);
  i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)(tile + k * LD + c));
  i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)(tile + (k + 4) * LD + c));
  i16x8 v = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  return __builtin_bit_cast(bf16x8, v);
}

// WGM x WGN waves per workgroup; NT threads. GA (varlen-K): bit 0 = the A rows are
// gathered through a_rows, bit 1 = the B rows through b_rows (else rows are positions).
template <int MODE, bool A_KC, bool B_KC, int EPI, int BM, int BN, int BK, int WGM, int WGN,
          int GA, bool RAG>
__global__ __launch_bounds__(64 * WGM * WGN,
                             (BM * BN > 128 * 128) ? (WGM * WGN == 8 ? 2 : 1) : (BK == 32 ? 3 : 2))
void gemm_bf16_kernel(GemmArgs g) {
  constexpr int NT = 64 * WGM * WGN;
  constexpr int WM = BM / WGM, WN = BN / WGN;  // wave tile
  constexpr int TM = WM / 32, TN = WN / 32;    // 32x32 sub-tiles per wave
  constexpr bool SWI = EPI == EPI_SWIGLU || EPI == EPI_SWIGLU_CAT;
  static_assert(TM >= 1 && TN >= 1 && (EPI != EPI_SWIGLU_CAT || TN % 2 == 0), "wave tile");
  // RAG: the output columns (and, grouped-M, the reduction; varlen-K, the output rows)
  // need not fill whole tiles, only whole 8-element chunks. Chunks past an edge are
  // loaded from a clamped in-range address (every load stays unconditional), reduction
  // chunks past the edge are zeroed when staged, and stores past an edge rewrite the
  // last in-range chunk with its own bytes.
  static_assert(!RAG || MODE == VARLEN_K || A_KC, "grouped-M A is reduction-contiguous");
  using AS = TileShape<A_KC, BM, BK>;
  using BS = TileShape<B_KC, BN, BK>;
  constexpr int CPK = BK / 8;  // 16-byte chunks per row of a reduction-contiguous tile
  constexpr int STAGE = AS::elems + BS::elems;
  constexpr int CLD = BN + 8;  // C staging row stride (elements)
  // one buffer holds the two stages, then the bf16 C tile for the plain store
  constexpr int SMEM = (2 * STAGE > BM * CLD) ? 2 * STAGE : BM * CLD;
  static_assert(SMEM * 2 >= (2 * MOE_MAX_EXPERTS + 2) * 4, "tile tables fit");
  constexpr int A_LD = BM * BK / (8 * NT);  // 16-byte chunks per thread per stage
  constexpr int B_LD = BN * BK / (8 * NT);
  __shared__ __attribute__((aligned(16))) uint16_t smem[SMEM];
  // EPI_DSWIGLU: router weight of every tile row, fetched while the main loop starts
  __shared__ __attribute__((aligned(16))) float s_wq[EPI == EPI_DSWIGLU ? BM : 4];
  // grouped-M: row tiles before each expert (prefix) and the expert offsets, built once
  __shared__ int s_tab[MODE == GROUPED_M ? 2 * (MOE_MAX_EXPERTS + 1) : 1];
  int *s_pref = s_tab, *s_off = s_tab + (MODE == GROUPED_M ? MOE_MAX_EXPERTS + 1 : 0);

  int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;  // re-derived per tile below
  int wm = wave / WGN, wn = wave % WGN;
  const int P = g.foff[g.E];
  const uint16_t *A = (const uint16_t *)g.A;
  const uint16_t *B = (const uint16_t *)g.B;

  int e = 0, mt = 0, nt = 0, row0 = 0, rows = 0, seg0 = 0, seglen = 0, nk = 0;
  // Grouped-M workgroups are persistent: XCD x (= blockIdx % 8, the hardware's
  // round-robin) owns one contiguous run of the tiles, which its workgroups take in
  // turn, so the tiles in flight on an XCD are neighbours (shared weights and rows in
  // its L2). The grid is a multiple of 8 workgroups.
  int tl = 0, tcnt = 0, tstart = 0, tstep = 1, ntn = 1;
  auto decode = [&](int L, int &e_, int &nt_, int &row0_, int &rows_) {
    const int mtile = L / ntn;
    nt_ = L - mtile * ntn;
    int lo = 0, hi = g.E - 1;  // largest e with s_pref[e] <= mtile
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (s_pref[mid] <= mtile) lo = mid; else hi = mid - 1;
    }
    // wave-uniform values, kept in scalar registers
    e_ = __builtin_amdgcn_readfirstlane(lo);
    nt_ = __builtin_amdgcn_readfirstlane(nt_);
    row0_ = __builtin_amdgcn_readfirstlane(s_off[lo] + (mtile - s_pref[lo]) * BM);
    rows_ = __builtin_amdgcn_readfirstlane(min(BM, s_off[lo + 1] - row0_));
  };
  if constexpr (MODE == GROUPED_M) {
    if (P > g.cap) return;
    for (int i = tid; i <= g.E; i += NT) {
      const int o = g.foff[i];
      s_off[i] = o;
      if (i < g.E) s_pref[i] = (g.foff[i + 1] - o + BM - 1) / BM;
    }
    __syncthreads();
    wave0_exclusive_scan(s_pref, g.E);
    __syncthreads();
    ntn = RAG ? (g.N + BN - 1) / BN : g.N / BN;
    const int G = s_pref[g.E] * ntn;
    const int x = blockIdx.x % kNumXcd, q = G / kNumXcd, rq = G % kNumXcd;
    tstart = x * q + min(x, rq);
    tcnt = q + (x < rq ? 1 : 0);
    tl = blockIdx.x / kNumXcd;
    tstep = gridDim.x / kNumXcd;
    if (tl >= tcnt) return;
    decode(tstart + tl, e, nt, row0, rows);
    nk = RAG ? (g.K + BK - 1) / BK : g.K / BK;
  } else {
    // Work per tile is the expert's row count, which can be very skewed. Experts are
    // taken largest first, and every XCD gets one contiguous eighth of each expert's
    // tiles: balanced across XCDs, and an XCD's tiles of one expert share rows in L2.
    int *s_freq = (int *)smem;
    int *s_order = s_freq + g.E;
    for (int i = tid; i < g.E; i += NT) s_freq[i] = g.foff[i + 1] - g.foff[i];
    __syncthreads();
    for (int i = tid; i < g.E; i += NT) {
      const int f = s_freq[i];
      int rank = 0;
      for (int j = 0; j < g.E; j++) {
        const int fj = s_freq[j];
        rank += (fj > f) || (fj == f && j < i);
      }
      s_order[rank] = i;
    }
    __syncthreads();
    // An expert's tile grid (mtn x ntn) is cut into xa row bands x xb column bands, one
    // rectangle per XCD: an XCD then reads the A columns of its row band and the B
    // columns of its column band, so the bytes all XCDs fetch per reduction row are
    // xb * M + xa * N; the cut with the fewest is taken (ties: more row bands). Grids
    // that no cut divides are dealt out flat.
    const int mtn = RAG ? (g.M + BM - 1) / BM : g.M / BM;
    const int ntn = RAG ? (g.N + BN - 1) / BN : g.N / BN, tpe = mtn * ntn;
    int xa = 0, xb = 0;
    for (int a = kNumXcd; a >= 1; a >>= 1) {
      const int b = kNumXcd / a;
      if (mtn % a || ntn % b) continue;
      if (!xa || (int64_t)b * g.M + (int64_t)a * g.N < (int64_t)xb * g.M + (int64_t)xa * g.N) {
        xa = a;
        xb = b;
      }
    }
    // Where the experts' row counts are even enough, each XCD takes whole experts instead:
    // the expert ranks are dealt to the XCDs in a snake (0..7, 7..0, ...), and if no
    // XCD's rows exceed the mean by more than 1/32 (and the XCDs get equal tile counts),
    // XCD x runs its experts one after the other, each expert's tiles in groups of up to
    // four row tiles (column tiles outer within a group). Its 32 tiles in flight then
    // share the A columns of at most four row tiles and B columns of eight column tiles,
    // where one rectangle per XCD of a small tile grid reads a band of each operand for
    // every few tiles.
    int *s_xrows = s_order + g.E;  // [kNumXcd]
    if (tid < kNumXcd) {
      int t = 0;
      for (int r = 0; r < g.E / kNumXcd; r++)
        t += s_freq[s_order[r * kNumXcd + ((r & 1) ? kNumXcd - 1 - tid : tid)]];
      s_xrows[tid] = t;
    }
    __syncthreads();
    bool whole = g.E % kNumXcd == 0;
    {
      int64_t mx = 0, sum = 0;
      for (int x = 0; x < kNumXcd; x++) {
        mx = max(mx, (int64_t)s_xrows[x]);
        sum += s_xrows[x];
      }
      whole = whole && mx * kNumXcd * 32 <= sum * 33;
    }
    int rank;
    if (whole) {
      const int x = blockIdx.x % kNumXcd, i = blockIdx.x / kNumXcd;
      const int r = i / tpe, l = i - r * tpe;
      rank = r * kNumXcd + ((r & 1) ? kNumXcd - 1 - x : x);
      constexpr int GM = 4;
      const int gi = l / (GM * ntn), rem = l - gi * GM * ntn;
      const int gm = min(GM, mtn - gi * GM);
      nt = rem / gm;
      mt = gi * GM + (rem - nt * gm);
    } else if (xa) {
      const int c = tpe / kNumXcd, x = blockIdx.x % kNumXcd, i = blockIdx.x / kNumXcd;
      rank = i / c;
      const int l = i - rank * c, bn = ntn / xb;  // tile l of this XCD's rectangle
      mt = (x / xb) * (mtn / xa) + l / bn;
      nt = (x % xb) * bn + l % bn;
    } else {
      rank = blockIdx.x / tpe;
      const int tile = blockIdx.x - rank * tpe;
      mt = tile / ntn;
      nt = tile - mt * ntn;
    }
    e = s_order[rank];
    seg0 = g.foff[e];
    seglen = P > g.cap ? 0 : g.foff[e + 1] - seg0;
    nk = (seglen + BK - 1) / BK;
    __syncthreads();  // the order table's LDS is reused by the stages below
  }

  // ---- per-thread load state (grouped-M): fixed row pointers
  //  k-contiguous tile of R rows: rows tid/CPK + (NT/CPK)*i, 16-byte chunk tid%CPK
  //  mn-contiguous tile of C cols: k-rows (tid / (C/8)) + (256/(C/8))*i, chunk tid % (C/8)
  const uint16_t *a_row[A_LD];
  const uint16_t *b_ptr[B_LD];
  // pair position of A chunk row i of a tile (rows past the segment: the tile's first)
  auto a_pos = [&](int i, int row0_, int rows_) {
    const int r = tid / CPK + (NT / CPK) * i;
    return row0_ + (r < rows_ ? r : 0);
  };
  // memory row m of A chunk row i, stored as -(m + 1) past the segment (where m is the
  // tile's first row); the row map is read at the clamped position either way (an
  // unconditional load)
  auto a_mem = [&](int i, int row0_, int rows_) {
    const int s_ = a_pos(i, row0_, rows_);
    const int m_ = (GA & 1) ? g.a_rows[s_] : s_;
    return tid / CPK + (NT / CPK) * i < rows_ ? m_ : -m_ - 1;
  };
  // Rows past the segment read a row of zeros where the reduction fits it (their
  // accumulator rows are never stored; zeros only spare the matrix cores' power), else
  // the tile's first row again.
  const bool zrows = MODE == GROUPED_M && g.K <= kZeroRowElems;
  // row pointers of a tile, from the memory rows of its A chunks
  auto set_ptrs = [&](const int *arow, int e_, int nt_) {
#pragma unroll
    for (int i = 0; i < A_LD; i++) {
      const bool pad = arow[i] < 0;
      const int m_ = pad ? -arow[i] - 1 : arow[i];
      a_row[i] = (pad && zrows ? g_zero_row : A + (int64_t)m_ * g.lda) + (tid % CPK) * 8;
    }
#pragma unroll
    for (int i = 0; i < B_LD; i++) {
      if constexpr (B_KC) {
        int64_t n = (int64_t)nt_ * BN + tid / CPK + (NT / CPK) * i;
        if constexpr (RAG) n = min(n, (int64_t)g.N - 1);
        b_ptr[i] = B + (int64_t)e_ * g.b_es + n * g.ldb + (tid % CPK) * 8;
      } else {
        constexpr int CPR = BN / 8;  // chunks per k-row
        const int kr = tid / CPR + (NT / CPR) * i;
        int64_t col = (int64_t)nt_ * BN + (tid % CPR) * 8;
        if constexpr (EPI == EPI_SWIGLU_CAT) {
          // LDS chunk -> the gate or up columns it holds in the per-wave [gates | ups]
          // order the concatenated-layout SwiGLU epilogue reads
          static_assert((WN / 2) % 8 == 0, "gate/up halves in whole chunks");
          const int c = (tid % CPR) * 8, w = c / WN, cw = c % WN;
          const int jb = nt_ * (BN / 2) + w * (WN / 2);
          if constexpr (RAG) {  // pairs past I read the last in-range chunk
            const int j = min(cw < WN / 2 ? jb + cw : jb + (cw - WN / 2), g.N / 2 - 8);
            col = cw < WN / 2 ? j : g.N / 2 + j;
          } else {
            col = cw < WN / 2 ? jb + cw : g.N / 2 + jb + (cw - WN / 2);
          }
        } else if constexpr (RAG) {
          col = min(col, (int64_t)g.N - 8);
        }
        b_ptr[i] = B + (int64_t)e_ * g.b_es + (int64_t)kr * g.ldb + col;
      }
    }
  };
  int arow[A_LD];  // grouped-M: memory rows of the A chunks of the next tile
  if constexpr (MODE == GROUPED_M) {
#pragma unroll
    for (int i = 0; i < A_LD; i++) arow[i] = a_mem(i, row0, rows);
    set_ptrs(arow, e, nt);
  }

  // Register sets and LDS stages are handled by macros so every array index is a
  // compile-time constant in this scope (the arrays then live in VGPRs).
  //  LOAD(ra, rb, ia, ib, k0): global -> registers for the tile at reduction offset k0
  //  STORE(ra, rb, st): registers -> LDS stage st
  //  COMPUTE(st): the MFMAs over LDS stage st
  //  ROWS(ia, ib, k0): (varlen-K) memory rows of the tile at reduction offset k0
#define MOE_ROWS(ia, ib, k0_)                                                              \
  do {                                                                                     \
    /* unconditional loads at a clamped position (a per-lane condition around them would  \
       make the compiler wait for every load in flight, data included, at the join);      \
       rows past the segment are zeroed where the data is used */                         \
    constexpr int CPA = BM / 8, CPB = BN / 8;                                              \
    _Pragma("unroll") for (int i = 0; i < A_LD; i++) {                                     \
      const int kc = seg0 + min((k0_) + tid / CPA + (NT / CPA) * i, seglen - 1);           \
      ia[i] = (GA & 1) ? g.a_rows[kc] : kc;                                                \
    }                                                                                      \
    _Pragma("unroll") for (int i = 0; i < B_LD; i++) {                                     \
      const int kc = seg0 + min((k0_) + tid / CPB + (NT / CPB) * i, seglen - 1);           \
      ib[i] = (GA & 2) ? g.b_rows[kc] : kc;                                                \
    }                                                                                      \
  } while (0)

#define MOE_LOAD(ra, rb, ia, ib, k0_)                                                      \
  do {                                                                                     \
    const int k0 = (k0_);                                                                  \
    if constexpr (MODE == GROUPED_M) {                                                     \
      /* RAG: a reduction chunk past K reads the row's last chunk (zeroed when staged) */ \
      const int kc_ = RAG ? min(k0, g.K - 8 - (tid % CPK) * 8) : k0;                       \
      _Pragma("unroll") for (int i = 0; i < A_LD; i++) ra[i] =                             \
          *(const u32x4 *)(a_row[i] + kc_);                                                \
      _Pragma("unroll") for (int i = 0; i < B_LD; i++) {                                   \
        if constexpr (B_KC) {                                                              \
          rb[i] = *(const u32x4 *)(b_ptr[i] + kc_);                                        \
        } else {                                                                           \
          constexpr int CPR_ = BN / 8;                                                     \
          const int kr_ = RAG ? min(k0, g.K - 1 - (tid / CPR_ + (NT / CPR_) * i)) : k0;    \
          rb[i] = *(const u32x4 *)(b_ptr[i] + (int64_t)kr_ * g.ldb);                       \
        }                                                                                  \
      }                                                                                    \
    } else {                                                                               \
      /* rows were looked up two tiles earlier (ia/ib); rows past the segment are zeroed  \
         when the set is stored (a select here would wait for these loads at once) */     \
      constexpr int CPA = BM / 8, CPB = BN / 8;                                            \
      if constexpr (RAG) { /* columns past an edge read the last in-range chunk */      \
        const int ca_ = min(mt * BM + (tid % CPA) * 8, g.M - 8);                           \
        const int cb_ = min(nt * BN + (tid % CPB) * 8, g.N - 8);                           \
        _Pragma("unroll") for (int i = 0; i < A_LD; i++)                                   \
          ra[i] = *(const u32x4 *)(A + (int64_t)ia[i] * g.lda + ca_);                      \
        _Pragma("unroll") for (int i = 0; i < B_LD; i++)                                   \
          rb[i] = *(const u32x4 *)(B + (int64_t)ib[i] * g.ldb + cb_);                      \
      } else {                                                                             \
        _Pragma("unroll") for (int i = 0; i < A_LD; i++)                                   \
          ra[i] = *(const u32x4 *)(A + (int64_t)ia[i] * g.lda + (int64_t)mt * BM + (tid % CPA) * 8); \
        _Pragma("unroll") for (int i = 0; i < B_LD; i++)                                   \
          rb[i] = *(const u32x4 *)(B + (int64_t)ib[i] * g.ldb + (int64_t)nt * BN + (tid % CPB) * 8); \
      }                                                                                    \
      MOE_ROWS(ia, ib, k0 + 2 * BK);                                                       \
    }                                                                                      \
  } while (0)

#define MOE_STORE(ra, rb, st, tile_)                                                       \
  do {                                                                                     \
    uint16_t *As_ = smem + (st) * STAGE;                                                   \
    uint16_t *Bs_ = As_ + AS::elems;                                                       \
    if constexpr (MODE == VARLEN_K) { /* rows past the segment -> 0 */                     \
      constexpr int CPA = BM / 8, CPB = BN / 8;                                            \
      const int kt_ = (tile_) * BK;                                                        \
      _Pragma("unroll") for (int i = 0; i < A_LD; i++)                                     \
        if (kt_ + tid / CPA + (NT / CPA) * i >= seglen) ra[i] = u32x4{0, 0, 0, 0};         \
      _Pragma("unroll") for (int i = 0; i < B_LD; i++)                                     \
        if (kt_ + tid / CPB + (NT / CPB) * i >= seglen) rb[i] = u32x4{0, 0, 0, 0};         \
    } else if constexpr (RAG) { /* reduction chunks past K -> 0 */                         \
      const int kt_ = (tile_) * BK;                                                        \
      _Pragma("unroll") for (int i = 0; i < A_LD; i++)                                     \
        if (kt_ + (tid % CPK) * 8 >= g.K) ra[i] = u32x4{0, 0, 0, 0};                       \
      _Pragma("unroll") for (int i = 0; i < B_LD; i++) {                                   \
        constexpr int CPB = BN / 8;                                                        \
        if (B_KC ? kt_ + (tid % CPK) * 8 >= g.K : kt_ + tid / CPB + (NT / CPB) * i >= g.K) \
          rb[i] = u32x4{0, 0, 0, 0};                                                       \
      }                                                                                    \
    }                                                                                      \
    _Pragma("unroll") for (int i = 0; i < A_LD; i++) {                                     \
      if constexpr (A_KC) {                                                                \
        const int r_ = tid / CPK + (NT / CPK) * i;                                         \
        *(u32x4 *)(As_ + r_ * AS::ld + (((tid % CPK) ^ kc_swz<BK>(r_)) << 3)) = ra[i];     \
      } else {                                                                             \
        constexpr int CPA = BM / 8;                                                        \
        *(u32x4 *)(As_ + (tid / CPA + (NT / CPA) * i) * AS::ld + (tid % CPA) * 8) = ra[i]; \
      }                                                                                    \
    }                                                                                      \
    _Pragma("unroll") for (int i = 0; i < B_LD; i++) {                                     \
      if constexpr (B_KC) {                                                                \
        const int r_ = tid / CPK + (NT / CPK) * i;                                         \
        *(u32x4 *)(Bs_ + r_ * BS::ld + (((tid % CPK) ^ kc_swz<BK>(r_)) << 3)) = rb[i];     \
      } else {                                                                             \
        constexpr int CPB = BN / 8;                                                        \
        const int kr = tid / CPB + (NT / CPB) * i;                                         \
        const int nc = tid % CPB;                                                          \
        *(u32x4 *)(Bs_ + kr * BS::ld + nc * 8) = rb[i];                                    \
      }                                                                                    \
    }                                                                                      \
  } while (0)

#define MOE_COMPUTE(st)                                                                    \
  do {                                                                                     \
    const uint16_t *As_ = smem + (st) * STAGE;                                             \
    const uint16_t *Bs_ = As_ + AS::elems;                                                 \
    _Pragma("unroll") for (int ks = 0; ks < BK / 16; ks++) {                               \
      bf16x8 af[TM], bfr[TN];                                                              \
      _Pragma("unroll") for (int mi = 0; mi < TM; mi++) {                                  \
        if constexpr (A_KC)                                                                \
          af[mi] = frag_kc<AS::ld, BK>(As_, wm * WM + mi * 32 + (lane & 31), ks * 16 + (lane >> 5) * 8); \
        else                                                                               \
          af[mi] = frag_mn<AS::ld>(As_, ks * 16, wm * WM + mi * 32, lane);                 \
      }                                                                                    \
      _Pragma("unroll") for (int ni = 0; ni < TN; ni++) {                                  \
        if constexpr (B_KC)                                                                \
          bfr[ni] = frag_kc<BS::ld, BK>(Bs_, wn * WN + ni * 32 + (lane & 31), ks * 16 + (lane >> 5) * 8); \
        else                                                                               \
          bfr[ni] = frag_mn<BS::ld>(Bs_, ks * 16, wn * WN + ni * 32, lane);                \
      }                                                                                    \
      _Pragma("unroll") for (int mi = 0; mi < TM; mi++)                                    \
        _Pragma("unroll") for (int ni = 0; ni < TN; ni++) acc[mi][ni] =                    \
            __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[mi], bfr[ni], acc[mi][ni], 0, 0, 0); \
    }                                                                                      \
  } while (0)

  // Ping-pong schedule: the fragments of a whole tile are read in one phase and
  // multiplied in the next, so one wave group's LDS and memory work runs beside the
  // other group's MFMAs. The scheduling barriers around each workgroup barrier keep
  // the compiler from moving MFMAs (register-only work) across a phase boundary.
#define MOE_FRAGS(st)                                                                      \
  do {                                                                                     \
    const uint16_t *As_ = smem + (st) * STAGE;                                             \
    const uint16_t *Bs_ = As_ + AS::elems;                                                 \
    _Pragma("unroll") for (int ks = 0; ks < BK / 16; ks++) {                               \
      _Pragma("unroll") for (int mi = 0; mi < TM; mi++) {                                  \
        if constexpr (A_KC)                                                                \
          paf[ks][mi] = frag_kc<AS::ld, BK>(As_, wm * WM + mi * 32 + (lane & 31), ks * 16 + (lane >> 5) * 8); \
        else                                                                               \
          paf[ks][mi] = frag_mn<AS::ld>(As_, ks * 16, wm * WM + mi * 32, lane);            \
      }                                                                                    \
      _Pragma("unroll") for (int ni = 0; ni < TN; ni++) {                                  \
        if constexpr (B_KC)                                                                \
          pbf[ks][ni] = frag_kc<BS::ld, BK>(Bs_, wn * WN + ni * 32 + (lane & 31), ks * 16 + (lane >> 5) * 8); \
        else                                                                               \
          pbf[ks][ni] = frag_mn<BS::ld>(Bs_, ks * 16, wn * WN + ni * 32, lane);            \
      }                                                                                    \
    }                                                                                      \
  } while (0)
#define MOE_MFMA()                                                                         \
  do {                                                                                     \
    _Pragma("unroll") for (int ks = 0; ks < BK / 16; ks++)                                 \
      _Pragma("unroll") for (int mi = 0; mi < TM; mi++)                                    \
        _Pragma("unroll") for (int ni = 0; ni < TN; ni++) acc[mi][ni] =                    \
            __builtin_amdgcn_mfma_f32_32x32x16_bf16(paf[ks][mi], pbf[ks][ni], acc[mi][ni], 0, 0, 0); \
  } while (0)
#define MOE_PP_BARRIER()                                                                   \
  do {                                                                                     \
    __builtin_amdgcn_sched_barrier(0);                                                     \
    __syncthreads();                                                                       \
    __builtin_amdgcn_sched_barrier(0);                                                     \
  } while (0)

  f32x16 acc[TM][TN];
  // Two LDS stages and two register sets: the tile stored into a stage was loaded
  // from memory two tiles earlier, so each global load has about two tiles of MFMA
  // work to arrive.
  u32x4 ra0[A_LD], rb0[B_LD], ra1[A_LD], rb1[B_LD];
  int ia0[A_LD], ib0[B_LD], ia1[A_LD], ib1[B_LD];  // varlen-K: rows of each set's next tile
  // Every load of the prologue and of the steady loop is unconditional (k offsets of
  // grouped-M are clamped to the last tile, varlen-K rows past the segment read as
  // zeros), so the memory wait counters stay exact across the loop.
  // The ping-pong schedule below is taken by the eight-wave grouped GEMMs: measured
  // 6-10% faster on the up and down projections and 2-7% on the backward ones.
  constexpr bool PP = MODE == GROUPED_M && WGM * WGN == 8;
  auto kof = [&](int t) { return (MODE == GROUPED_M ? min(t, nk - 1) : t) * BK; };
  // Grouped-M: the first k-tile of every tile after a workgroup's first is loaded
  // before the epilogue of the tile before it (one register set: the epilogues need
  // the rest of the registers; the DSWIGLU epilogue needs all of them).
  constexpr bool EARLY = MODE == GROUPED_M && EPI != EPI_DSWIGLU;
  if constexpr (EARLY) MOE_LOAD(ra0, rb0, ia0, ib0, 0);
  for (;;) {
  // The thread index passes through an empty asm at every tile, so the addresses
  // derived from it are recomputed per tile instead of being kept live (hoisted)
  // across the tile loop, which would cost registers the main loop needs.
  asm volatile("" : "+v"(tid));
  lane = tid & 63;
  wave = tid >> 6;
  wm = wave / WGN;
  wn = wave % WGN;
#pragma unroll
  for (int mi = 0; mi < TM; mi++)
#pragma unroll
    for (int ni = 0; ni < TN; ni++)
#pragma unroll
      for (int r = 0; r < 16; r++) acc[mi][ni][r] = 0.0f;
  // grouped-M: the next tile of this workgroup (the last one again after the last,
  // so the loads below stay unconditional); its A rows are fetched now and used
  // after the main loop
  const bool more = MODE == GROUPED_M && tl + tstep < tcnt;
  int e_n = e, nt_n = nt, row0_n = row0, rows_n = rows;
  if constexpr (MODE == GROUPED_M) {
    decode(tstart + min(tl + tstep, tcnt - 1), e_n, nt_n, row0_n, rows_n);
#pragma unroll
    for (int i = 0; i < A_LD; i++) arow[i] = a_mem(i, row0_n, rows_n);
  }
  if (nk > 0) {
    if constexpr (MODE == VARLEN_K) {
      MOE_ROWS(ia0, ib0, 0);
      MOE_ROWS(ia1, ib1, BK);
    }
    if constexpr (!EARLY) MOE_LOAD(ra0, rb0, ia0, ib0, 0);
    MOE_LOAD(ra1, rb1, ia1, ib1, kof(1));
    MOE_STORE(ra0, rb0, 0, 0);
    MOE_LOAD(ra0, rb0, ia0, ib0, kof(2));
    if constexpr (EPI == EPI_DSWIGLU) {
      for (int r = tid; r < BM; r += NT)
        s_wq[r] = r < rows ? g.scores[g.s_scatter[row0 + r]] : 0.0f;
    }
    __syncthreads();
  }
  if (PP && nk > 0) {
    // Waves 0-3 and 4-7 (one of each per SIMD) run half an iteration apart: between
    // two barriers one group multiplies tile j while the other reads tile j's
    // fragments, stores tile j+1 into the other stage and loads tile j+3. Two stages
    // suffice: a stage is rewritten two phases after both groups have read it.
    bf16x8 paf[BK / 16][TM], pbf[BK / 16][TN];
    const bool late = __builtin_amdgcn_readfirstlane(wave) >= 4;  // wave-uniform
    // a wave whose rows all lie past the segment (a tile of at most WM rows) skips its
    // fragment reads and MFMAs (it still stores its share of each stage for the other
    // group): its accumulators stay zero and its rows are never stored
    const bool mm = __builtin_amdgcn_readfirstlane(wm) * WM < rows;
    if (late) MOE_PP_BARRIER();
    int j = 0;
    for (; j + 2 < nk; j += 2) {  // loads past the end re-read the last tile
      if (mm) MOE_FRAGS(0);  // tile j
      MOE_STORE(ra1, rb1, 1, j + 1);
      MOE_LOAD(ra1, rb1, ia1, ib1, kof(j + 3));
      MOE_PP_BARRIER();
      if (mm) MOE_MFMA();
      MOE_PP_BARRIER();
      if (mm) MOE_FRAGS(1);  // tile j+1
      MOE_STORE(ra0, rb0, 0, j + 2);
      MOE_LOAD(ra0, rb0, ia0, ib0, kof(j + 4));
      MOE_PP_BARRIER();
      if (mm) MOE_MFMA();
      MOE_PP_BARRIER();
    }
    if (mm) MOE_FRAGS(0);  // tile j
    if (j + 1 < nk) MOE_STORE(ra1, rb1, 1, j + 1);
    MOE_PP_BARRIER();
    if (mm) MOE_MFMA();
    MOE_PP_BARRIER();
    if (j + 1 < nk) {  // tile j+1
      if (mm) MOE_FRAGS(1);
      MOE_PP_BARRIER();
      if (mm) MOE_MFMA();
      MOE_PP_BARRIER();
    }
    if (!late) MOE_PP_BARRIER();
  } else if (nk > 0) {
    int kt = 0;
    // steady state, free of branches: the wait before a stage store only holds back
    // the set being stored (loaded two tiles earlier), not the set loaded after it
    for (; kt + 4 < nk; kt += 2) {
      MOE_COMPUTE(0);  // tile kt
      MOE_STORE(ra1, rb1, 1, kt + 1);
      MOE_LOAD(ra1, rb1, ia1, ib1, (kt + 3) * BK);
      __syncthreads();
      MOE_COMPUTE(1);  // tile kt+1
      MOE_STORE(ra0, rb0, 0, kt + 2);
      MOE_LOAD(ra0, rb0, ia0, ib0, (kt + 4) * BK);
      __syncthreads();
    }
    // the last (at most four) tiles
    for (; kt < nk; kt += 2) {
      MOE_COMPUTE(0);
      if (kt + 1 < nk) {
        MOE_STORE(ra1, rb1, 1, kt + 1);
        if (kt + 3 < nk) MOE_LOAD(ra1, rb1, ia1, ib1, (kt + 3) * BK);
      }
      __syncthreads();
      if (kt + 1 < nk) {
        MOE_COMPUTE(1);
        if (kt + 2 < nk) {
          MOE_STORE(ra0, rb0, 0, kt + 2);
          if (kt + 4 < nk) MOE_LOAD(ra0, rb0, ia0, ib0, (kt + 4) * BK);
        }
        __syncthreads();
      }
    }
  }
  if constexpr (MODE == GROUPED_M) {  // the next tile's rows (and first k-tile)
    set_ptrs(arow, e_n, nt_n);
    if constexpr (EARLY) MOE_LOAD(ra0, rb0, ia0, ib0, 0);
  }
#undef MOE_LOAD
#undef MOE_ROWS
#undef MOE_STORE
#undef MOE_COMPUTE
#undef MOE_FRAGS
#undef MOE_MFMA
#undef MOE_PP_BARRIER

  // ---- epilogues. Accumulator (mi, ni, r) of lane l holds tile row
  // wm*WM + mi*32 + (r/4)*8 + (l/32)*4 + r%4 and column wn*WN + ni*32 + l%32.
  const int col_l = lane & 31;
  if constexpr (EPI == EPI_STORE) {
    // bf16 tile -> LDS [BM][BN+8] (adjacent lanes swap one value so each writes a
    // column pair), then whole rows -> memory in 16-byte chunks
    uint16_t *Cs = smem;
    const bool odd = lane & 1;
#pragma unroll
    for (int mi = 0; mi < TM; mi++)
#pragma unroll
      for (int ni = 0; ni < TN; ni++)
#pragma unroll
        for (int r = 0; r < 16; r += 2) {
          // The even lane of a pair writes row r, the odd lane row r+1, each as one
          // column pair; quad_perm [1,0,3,2] brings the neighbour's two values (no LDS
          // traffic). Both neighbour values are moved and the selects pick between
          // them and the lane's own: a select between acc[r] and acc[r+1] would be
          // folded into a lane-dependent vector index, lowered as a 16-way select.
          const float a0 = acc[mi][ni][r], a1 = acc[mi][ni][r + 1];
          const float n0 = __uint_as_float((uint32_t)__builtin_amdgcn_mov_dpp(
              (int)__float_as_uint(a0), 0xB1, 0xF, 0xF, false));
          const float n1 = __uint_as_float((uint32_t)__builtin_amdgcn_mov_dpp(
              (int)__float_as_uint(a1), 0xB1, 0xF, 0xF, false));
          const int row = wm * WM + mi * 32 + (r >> 2) * 8 + (lane >> 5) * 4 + (r & 3) + odd;
          const int col = wn * WN + ni * 32 + (col_l & ~1);
          const uint32_t v = pack_bf16x2(odd ? n1 : a0, odd ? a1 : n0);
          *(uint32_t *)(Cs + row * CLD + col) = v;
        }
    __syncthreads();
    uint16_t *C = (uint16_t *)g.C;
    constexpr int CPR = BN / 8;
#pragma unroll
    for (int i = 0; i < BM * CPR / NT; i++) {
      const int c = tid + NT * i;
      // grouped-M rows past the segment store the segment's last row again (the same
      // bytes): every store is issued, so the wait counters stay exact for the next
      // tile's loads already in flight
      int row = MODE == GROUPED_M ? min(c / CPR, rows - 1) : c / CPR, ch = c % CPR;
      if constexpr (RAG) {  // past an edge: the last in-range row / chunk again
        if constexpr (MODE == VARLEN_K) row = min(row, g.M - mt * BM - 1);
        ch = min(ch, (g.N - nt * BN) / 8 - 1);
      }
      int64_t off;
      if constexpr (MODE == GROUPED_M) {
        off = (int64_t)(row0 + row) * g.ldc;
      } else {
        off = (int64_t)e * g.c_es + (int64_t)(mt * BM + row) * g.ldc;
      }
      // streaming store: a whole-chip burst of output tiles would otherwise fill L2
      // with dirty lines ahead of the operands other tiles still read
      __builtin_nontemporal_store(*(const u32x4 *)(Cs + row * CLD + ch * 8),
                                  (u32x4 *)(C + off + (int64_t)nt * BN + ch * 8));
    }
  } else if constexpr (SWI) {
    // Both outputs are staged through LDS and leave as whole rows of 16-byte streaming
    // stores: h (interleaved (gate, up) pairs, [BM][BN]) first, then a ([BM][BN/2]).
    constexpr int HLD = BN + 8, ALD = BN / 2 + 8;  // staging row strides (elements)
    static_assert(BM * HLD <= SMEM && BM * ALD <= SMEM, "staging tiles fit");
    uint16_t *Hst = smem;
    uint16_t *Hs = (uint16_t *)g.C;  // may be null (inference); always interleaved
    uint16_t *Aout = (uint16_t *)g.C2;
    const bool odd = lane & 1;
    // (gate, up) of one row and pair -> f(tile row, local pair, gate, up)
    auto for_pairs = [&](auto &&f) {
      if constexpr (EPI == EPI_SWIGLU) {
        // Interleaved W_up columns: even accumulator columns are gates, odd ones the
        // matching ups. As in the plain-store epilogue, a quad_perm [1,0,3,2] move
        // gives the even lane of a pair (gate, up) of row r and the odd lane that of
        // row r+1.
#pragma unroll
        for (int mi = 0; mi < TM; mi++)
#pragma unroll
          for (int ni = 0; ni < TN; ni++) {
            const int jl = (wn * WN + ni * 32 + (col_l & ~1)) / 2;
#pragma unroll
            for (int r = 0; r < 16; r += 2) {
              const float a0 = acc[mi][ni][r], a1 = acc[mi][ni][r + 1];
              const float n0 = __uint_as_float((uint32_t)__builtin_amdgcn_mov_dpp(
                  (int)__float_as_uint(a0), 0xB1, 0xF, 0xF, false));
              const float n1 = __uint_as_float((uint32_t)__builtin_amdgcn_mov_dpp(
                  (int)__float_as_uint(a1), 0xB1, 0xF, 0xF, false));
              const int row = wm * WM + mi * 32 + (r >> 2) * 8 + (lane >> 5) * 4 + (r & 3) + odd;
              f(row, jl, odd ? n1 : a0, odd ? a1 : n0);
            }
          }
      } else {
        // concatenated W_up: the B tile holds per wave its gates, then its ups, so
        // acc[.][np] holds gates and acc[.][np + TN/2] the matching ups
#pragma unroll
        for (int mi = 0; mi < TM; mi++)
#pragma unroll
          for (int np = 0; np < TN / 2; np++) {
            const int jl = wn * (WN / 2) + np * 32 + col_l;
#pragma unroll
            for (int r = 0; r < 16; r++) {
              const int row = wm * WM + mi * 32 + (r >> 2) * 8 + (lane >> 5) * 4 + (r & 3);
              f(row, jl, acc[mi][np][r], acc[mi][np + TN / 2][r]);
            }
          }
      }
    };
    if (Hs) {
      for_pairs([&](int row, int jl, float gt, float up) {
        *(uint32_t *)(Hst + row * HLD + 2 * jl) = pack_bf16x2(gt, up);
      });
      __syncthreads();
      constexpr int CPR = BN / 8;
#pragma unroll
      for (int i = 0; i < BM * CPR / NT; i++) {
        // rows past the segment store its last row again (the same bytes), so every
        // store is issued and the wait counters stay exact
        const int c = tid + NT * i, row = min(c / CPR, rows - 1);
        const int ch = RAG ? min(c % CPR, (g.N - nt * BN) / 8 - 1) : c % CPR;
        __builtin_nontemporal_store(*(const u32x4 *)(Hst + row * HLD + ch * 8),
                                    (u32x4 *)(Hs + (int64_t)(row0 + row) * g.ldc +
                                              (int64_t)nt * BN + ch * 8));
      }
      __syncthreads();
    }
    for_pairs([&](int row, int jl, float gt, float up) {
      Hst[row * ALD + jl] = f32_to_bf16(silu_fast(gt) * up);
    });
    __syncthreads();
    constexpr int CPA = BN / 16;
#pragma unroll
    for (int i = 0; i < BM * CPA / NT; i++) {
      const int c = tid + NT * i, row = min(c / CPA, rows - 1);
      const int ch = RAG ? min(c % CPA, (g.N / 2 - nt * (BN / 2)) / 8 - 1) : c % CPA;
      __builtin_nontemporal_store(*(const u32x4 *)(Hst + row * ALD + ch * 8),
                                    (u32x4 *)(Aout + (int64_t)(row0 + row) * g.ldc2 +
                                              (int64_t)nt * (BN / 2) + ch * 8));
    }
  } else {  // EPI_DSWIGLU: acc = da_u = dout_g W_down^T for pair columns j
    uint16_t *__restrict__ dH = (uint16_t *)g.C;
    uint16_t *__restrict__ AW = (uint16_t *)g.C2;
    const uint16_t *__restrict__ Hs = (const uint16_t *)g.Hs;
    float *red = (float *)smem;  // [WGN][BM] row partials of the column waves (the
                                 // loop's final barrier has released the stages)
    // Adjacent lanes (one column each) exchange their values of rows r and r+1 with one
    // DPP quad_perm [1,0,3,2] move per value (as in the plain-store epilogue): the even
    // lane of a pair then holds columns (jb, jb+1) of row r, the odd lane those of row
    // r+1, so each lane loads the two columns' saved (gate, up) pairs as 8 bytes and
    // stores 8 bytes of dh and 4 of w*a per row pair. The saved pairs of the next
    // (mi, ni) block are loaded while the current block is computed (each register is
    // refilled right after its value is consumed). Rows past the segment read row 0 of
    // the tile and are never stored.
    const bool odd = lane & 1;
    u32x2 hv[8];
    auto h_addr = [&](int mi_, int ni_, int rp) {
      int jb_ = nt * BN + wn * WN + ni_ * 32 + (col_l & ~1);
      if constexpr (RAG) jb_ = min(jb_, g.N - 2);  // columns past N: never stored
      const int r = 2 * rp;
      const int row_ = wm * WM + mi_ * 32 + (r >> 2) * 8 + (lane >> 5) * 4 + (r & 3) + odd;
      const int64_t s_ = row0 + (row_ < rows ? row_ : 0);
      return (const u32x2 *)(Hs + s_ * g.ldh + 2 * jb_);
    };
#pragma unroll
    for (int rp = 0; rp < 8; rp++) hv[rp] = *h_addr(0, 0, rp);
#pragma unroll
    for (int mi = 0; mi < TM; mi++) {
      float pp[8];  // this lane's row of each row pair: its two columns' dscore terms
#pragma unroll
      for (int rp = 0; rp < 8; rp++) pp[rp] = 0.0f;
#pragma unroll
      for (int ni = 0; ni < TN; ni++) {
        constexpr int NB = TM * TN;
        const int b = mi * TN + ni;
        const int jb = nt * BN + wn * WN + ni * 32 + (col_l & ~1);
#pragma unroll
        for (int rp = 0; rp < 8; rp++) {
          const int r = 2 * rp;
          const float a0 = acc[mi][ni][r], a1 = acc[mi][ni][r + 1];
          const float n0 = __uint_as_float((uint32_t)__builtin_amdgcn_mov_dpp(
              (int)__float_as_uint(a0), 0xB1, 0xF, 0xF, false));
          const float n1 = __uint_as_float((uint32_t)__builtin_amdgcn_mov_dpp(
              (int)__float_as_uint(a1), 0xB1, 0xF, 0xF, false));
          const float dau0 = odd ? n1 : a0;  // column jb of this lane's row
          const float dau1 = odd ? a1 : n0;  // column jb + 1
          const int row = wm * WM + mi * 32 + (r >> 2) * 8 + (lane >> 5) * 4 + (r & 3) + odd;
          const int64_t srow = row0 + row;
          const float wq = s_wq[row];
          const u32x2 h4 = hv[rp];
          if (b + 1 < NB) hv[rp] = *h_addr((b + 1) / TN, (b + 1) % TN, rp);
          const float gt0 = bf16_to_f32((uint16_t)(h4[0] & 0xffffu));
          const float up0 = bf16_to_f32((uint16_t)(h4[0] >> 16));
          const float gt1 = bf16_to_f32((uint16_t)(h4[1] & 0xffffu));
          const float up1 = bf16_to_f32((uint16_t)(h4[1] >> 16));
          const float sg0 = sigmoid_fast(gt0), sg1 = sigmoid_fast(gt1);
          const float av0 = gt0 * sg0 * up0, av1 = gt1 * sg1 * up1;
          if (row < rows && (!RAG || jb < g.N)) {
            pp[rp] += dau0 * av0 + dau1 * av1;
            const float da0 = wq * dau0, da1 = wq * dau1;
            const float dg0 = da0 * up0 * sg0 * (1.0f + gt0 * (1.0f - sg0));
            const float dg1 = da1 * up1 * sg1 * (1.0f + gt1 * (1.0f - sg1));
            const float du0 = da0 * gt0 * sg0, du1 = da1 * gt1 * sg1;
            if (g.gu_concat) {  // dh in W_up's column order
              *(uint32_t *)(dH + srow * g.ldc + jb) = pack_bf16x2(dg0, dg1);
              *(uint32_t *)(dH + srow * g.ldc + g.N + jb) = pack_bf16x2(du0, du1);
            } else {
              *(u32x2 *)(dH + srow * g.ldc + 2 * jb) =
                  u32x2{pack_bf16x2(dg0, du0), pack_bf16x2(dg1, du1)};
            }
            *(uint32_t *)(AW + srow * g.ldc2 + jb) = pack_bf16x2(wq * av0, wq * av1);
          }
        }
      }
      // Row sums over the 32 columns: lanes of one parity hold the same row of each
      // pair, so the butterfly runs over lane bits 4, 3, 2 (halving the entries each
      // step) and then adds the lane two apart; lane l then holds the row sum of entry
      // (l % 32) / 4 for its parity.
#pragma unroll
      for (int n = 8, o = 16; n > 1; n >>= 1, o >>= 1) {
        const bool upper = (lane & o) != 0;
#pragma unroll
        for (int i = 0; i < n / 2; i++) {
          const float send = upper ? pp[i] : pp[i + n / 2];
          const float keep = upper ? pp[i + n / 2] : pp[i];
          pp[i] = keep + __shfl_xor(send, o, kWave);
        }
      }
      const float rsum = pp[0] + __uint_as_float((uint32_t)__builtin_amdgcn_update_dpp(
                                     0, (int)__float_as_uint(pp[0]), 0x4E, 0xF, 0xF, false));
      const int rr = 2 * ((lane & 31) >> 2) + odd;
      const int row = wm * WM + mi * 32 + (rr >> 2) * 8 + (lane >> 5) * 4 + (rr & 3);
      if ((lane & 2) == 0) red[wn * BM + row] = rsum;
    }
    __syncthreads();
    for (int r = tid; r < rows; r += NT) {
      float v = red[r];
#pragma unroll
      for (int w = 1; w < WGN; w++) v += red[w * BM + r];
      g.partial[(int64_t)(row0 + r) * g.n_ntiles + nt] = v;
    }
  }
  if (!more) break;
  __syncthreads();  // the epilogue's LDS reads are done before the next stage stores
  tl += tstep;
  e = e_n;
  nt = nt_n;
  row0 = row0_n;
  rows = rows_n;
  }  // tiles
}

template <int MODE, bool A_KC, bool B_KC, int EPI, int GA = 0>
hipError_t launch_tiles(int bm, int bn, int bk, bool rag, int grid, const GemmArgs &g,
                        hipStream_t st) {
  // grouped-M workgroups are persistent: as many as the chip holds at once (capped
  // by the tile count), rounded up to a multiple of the 8 XCDs
#define MOE_LAUNCH(BM_, BN_, BK_, WGM_, WGN_, RAG_)                                          \
  if (bm == BM_ && bn == BN_ && bk == BK_ && rag == RAG_) {                               \
    auto kern = gemm_bf16_kernel<MODE, A_KC, B_KC, EPI, BM_, BN_, BK_, WGM_, WGN_, GA, RAG_>; \
    int blocks = grid;                                                                    \
    if constexpr (MODE == GROUPED_M) {                                                    \
      /* workgroups per CU, a property of the kernel: queried once (a function-local     \
         static is initialised once even when host threads race to the first launch) */   \
      static const int occ = [&] {                                                        \
        int o = 0;                                                                        \
        return hipOccupancyMaxActiveBlocksPerMultiprocessor(&o, kern, 64 * WGM_ * WGN_, 0) == \
                       hipSuccess                                                         \
                   ? o                                                                    \
                   : -1;                                                                  \
      }();                                                                                \
      if (occ < 0) return hipErrorInvalidValue;                                           \
      int dev = 0, ncu = 0;                                                               \
      if (hipGetDevice(&dev) != hipSuccess ||                                             \
          hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev) !=      \
              hipSuccess)                                                                 \
        return hipErrorInvalidValue;                                                      \
      const int64_t cap = (int64_t)ncu * (occ > 0 ? occ : 1);                             \
      blocks = (int)(((grid < cap ? grid : cap) + kNumXcd - 1) / kNumXcd * kNumXcd);      \
    }                                                                                     \
    hipLaunchKernelGGL(kern, dim3(blocks), dim3(64 * WGM_ * WGN_), 0, st, g);             \
    return hipGetLastError();                                                             \
  }
  if constexpr (MODE == GROUPED_M) {
    MOE_LAUNCH(32, 128, 64, 1, 2, false)
  }
  MOE_LAUNCH(128, 128, 64, 2, 2, false)
  MOE_LAUNCH(128, 128, 32, 2, 2, false)
  MOE_LAUNCH(256, 256, 32, 2, 4, false)
  MOE_LAUNCH(128, 128, 32, 2, 2, true)
#undef MOE_LAUNCH
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_gemm_bf16(GemmKind kind, const GemmArgs &g, hipStream_t st) {
  const int grid = gemm_grid(kind, g);
  if (grid < 0) return hipErrorInvalidValue;
  if (grid == 0) return hipSuccess;
  int bm, bn, bk;
  gemm_tile(kind, g, &bm, &bn, &bk);
  const bool rag = gemm_ragged(kind, g);
  switch (kind) {
    // grouped-M: GA = 1 when the A rows are gathered (x_gather_idx), a compile-time
    // choice like the weight gradients' (the row loads then carry no condition)
    case kUpSwiGLU:
      if (!g.a_rows) return hipErrorInvalidValue;
      if (g.gu_concat)
        return launch_tiles<GROUPED_M, true, false, EPI_SWIGLU_CAT, 1>(bm, bn, bk, rag, grid, g, st);
      return launch_tiles<GROUPED_M, true, false, EPI_SWIGLU, 1>(bm, bn, bk, rag, grid, g, st);
    case kDown:
      if (g.a_rows) return hipErrorInvalidValue;
      return launch_tiles<GROUPED_M, true, false, EPI_STORE, 0>(bm, bn, bk, rag, grid, g, st);
    case kDownBwd:
      if (!g.a_rows) return hipErrorInvalidValue;
      return launch_tiles<GROUPED_M, true, true, EPI_DSWIGLU, 1>(bm, bn, bk, rag, grid, g, st);
    case kUpBwd:
      if (g.a_rows) return hipErrorInvalidValue;
      return launch_tiles<GROUPED_M, true, true, EPI_STORE, 0>(bm, bn, bk, rag, grid, g, st);
    case kWeightGrad:
      // the gathered operand is a compile-time choice: the row-index loads of the loop
      // then carry no condition. Each weight gradient gathers exactly one operand
      // (x rows for dW_up, dout rows for dW_down); other combinations are not built.
      if (g.a_rows && !g.b_rows)
        return launch_tiles<VARLEN_K, false, false, EPI_STORE, 1>(bm, bn, bk, rag, grid, g, st);
      if (g.b_rows && !g.a_rows)
        return launch_tiles<VARLEN_K, false, false, EPI_STORE, 2>(bm, bn, bk, rag, grid, g, st);
      return hipErrorInvalidValue;
    default:
      return hipErrorInvalidValue;
  }
}

}  // namespace moe
