// Host-side size arithmetic of the kernels: tile shapes and grid sizes of the grouped
// GEMMs and the router's workspace. Host code only (no kernels), so it can also be
// built for the CPU alone and checked there under sanitizers.
#include "kernels.h"

namespace moe {

// router workspace, in floats: per-chunk softmax sums [E][nblk], then their totals [E]
size_t route_ws_floats(int64_t NK, int E) { return (size_t)(meta_blocks(NK) + 1) * (size_t)E; }

// bf16 tiles: 256x256x32 with eight waves where the fixed dimensions allow it (half
// the bytes per flop of 128x128), else 128x128; 32x128x64 with two waves when the
// capacity averages at most 16 rows per expert (decode), so the matrix work per
// streamed weight byte matches the rows there are and more workgroups stream weights.
// At few tokens the 128x128 tiles also replace the 256x256 ones where those would
// number fewer than the CUs (grouped-M) or where the experts average fewer than 128
// rows (weight gradients).
// Shapes whose output columns (and, grouped-M, reduction; varlen-K, output rows) do
// not fill whole 128-wide tiles take the 128x128x32 tiles with edge handling; H and I
// are multiples of 8 (one 16-byte chunk) there.
bool gemm_ragged(GemmKind kind, const GemmArgs &g) {
  if (kind == kWeightGrad) return g.M % 128 != 0 || g.N % 128 != 0;
  return g.N % 128 != 0 || g.K % 32 != 0;
}

void gemm_tile(GemmKind kind, const GemmArgs &g, int *bm, int *bn, int *bk) {
  if (gemm_ragged(kind, g)) {
    *bm = *bn = 128;
    *bk = 32;
  } else if (kind == kWeightGrad) {
    // few rows per expert: each tile is a short reduction and then a store burst, and the
    // 128x128 tiles (several workgroups per CU) overlap one tile's stores with another's
    // loads
    const bool big = g.M % 256 == 0 && g.N % 256 == 0 &&
                     (int64_t)g.cap >= kWgradFewRows * (int64_t)g.E;
    *bm = big ? 256 : 128;
    *bn = big ? 256 : 128;
    *bk = 32;
  } else {
    const bool skinny = (int64_t)g.cap <= 16LL * g.E && g.N % 128 == 0 && g.K % 64 == 0;
    bool big = g.N % 256 == 0 && g.K % 32 == 0;
    if (big && !skinny) {
      // fewer 256x256 tiles than the chip has CUs (bounded from the capacity): the
      // 128x128 tiles, four times as many, keep more of the chip busy
      const int64_t mt = ((int64_t)g.cap + (int64_t)g.E * 255) / 256;
      if (mt * (g.N / 256) < kGemmFewTiles) big = false;
    }
    *bm = skinny ? 32 : big ? 256 : 128;
    *bn = skinny ? 128 : big ? 256 : 128;
    *bk = skinny ? 64 : big ? 32 : (g.K % 64 == 0 ? 64 : 32);
  }
}

// Launch size: varlen-K launches one workgroup per output tile of every expert (-1
// when that exceeds the grid limit); grouped-M returns an upper bound of its tiles
// (row tiles of every expert segment, bounded from the capacity, times column tiles,
// capped at INT_MAX), and the launch caps its persistent grid at what the chip holds.
// Partial edge tiles count as tiles.
int gemm_grid(GemmKind kind, const GemmArgs &g) {
  int bm, bn, bk;
  gemm_tile(kind, g, &bm, &bn, &bk);
  const int64_t ntn = ((int64_t)g.N + bn - 1) / bn;
  if (kind == kWeightGrad) {
    const int64_t grid = (int64_t)g.E * (((int64_t)g.M + bm - 1) / bm) * ntn;
    return grid > 0x7fffffff ? -1 : (int)grid;
  }
  const int64_t mt = ((int64_t)g.cap + (int64_t)g.E * (bm - 1)) / bm;
  const int64_t tiles = mt * ntn;
  return tiles > 0x7fffffff ? 0x7fffffff : (int)tiles;
}

// fp32 checking mode: one workgroup per 128x128 tile (grouped-M: row tiles of every
// expert segment, bounded from the capacity; varlen-K: every expert's output tiles);
// -1 when that exceeds the grid limit.
int gemm_grid_f32(GemmKind kind, const GemmArgs &g) {
  int64_t grid;
  const int64_t ntn = ((int64_t)g.N + kGemmBN - 1) / kGemmBN;
  if (kind == kWeightGrad) {
    grid = (int64_t)g.E * (((int64_t)g.M + kGemmBM - 1) / kGemmBM) * ntn;
  } else {
    const int64_t mt = ((int64_t)g.cap + (int64_t)g.E * (kGemmBM - 1)) / kGemmBM;
    grid = mt * ntn;
  }
  return grid > 0x7fffffff ? -1 : (int)grid;
}

}  // namespace moe
