// Device helpers shared by the gfx950 kernels of the local MoE expert layer.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
// 16 bytes as a native vector (HIP's uint4 struct is copied through memory by the
// optimizer; a native vector stays in registers)
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;
constexpr int kNumXcd = 8;  // gfx950: workgroups are dealt round-robin to 8 XCDs

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(((uint32_t)b) << 16);
}
// fp32 -> bf16, round to nearest even (the language conversion; gfx950 has it in hardware)
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  __bf16 h = (__bf16)f;
  return __builtin_bit_cast(uint16_t, h);
}
// two fp32 -> packed bf16 pair (lo in bits 0-15), round to nearest even: one
// v_cvt_pk_bf16_f32 on gfx950
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  typedef float f32x2_t __attribute__((ext_vector_type(2)));
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{lo, hi}, bf16x2_t));
}

__device__ __forceinline__ int lane_id() {
  return __builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0));
}
// number of set bits of m at lanes below the calling lane
__device__ __forceinline__ int popc_below(uint64_t m) {
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0));
}
__device__ __forceinline__ uint64_t ballot64(bool p) { return __ballot(p); }

// Inclusive prefix sum across the 64 lanes of a wave with DPP lane moves (no LDS
// traffic): Hillis-Steele shifts 1, 2, 4, 8 inside each row of 16 lanes, then
// lane 15 of rows 0 and 2 is added into rows 1 and 3, then lane 31 into rows 2
// and 3 (GFX9 DPP row_shr, row_bcast:15, row_bcast:31). All 64 lanes must be active.
__device__ __forceinline__ int wave_inclusive_scan_dpp(int v) {
  v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xf, 0xf, true);  // row_shr:1
  v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xf, 0xf, true);  // row_shr:2
  v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xf, 0xf, true);  // row_shr:4
  v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xf, 0xf, true);  // row_shr:8
  v += __builtin_amdgcn_update_dpp(0, v, 0x142, 0xa, 0xf, false); // row_bcast:15 -> rows 1, 3
  v += __builtin_amdgcn_update_dpp(0, v, 0x143, 0xc, 0xf, false); // row_bcast:31 -> rows 2, 3
  return v;
}

// Sum across the 64 lanes of a wave with the same DPP pattern (fixed association
// order, so deterministic); every lane receives lane 63's total. All lanes active.
__device__ __forceinline__ float wave_sum_dpp_f32(float v) {
#define MOE_DPP_ADD(C, R, B) \
  v += __uint_as_float((uint32_t)__builtin_amdgcn_update_dpp(0, (int)__float_as_uint(v), C, R, 0xf, B));
  MOE_DPP_ADD(0x111, 0xf, true)   // row_shr:1
  MOE_DPP_ADD(0x112, 0xf, true)   // row_shr:2
  MOE_DPP_ADD(0x114, 0xf, true)   // row_shr:4
  MOE_DPP_ADD(0x118, 0xf, true)   // row_shr:8
  MOE_DPP_ADD(0x142, 0xa, false)  // row_bcast:15 -> rows 1, 3
  MOE_DPP_ADD(0x143, 0xc, false)  // row_bcast:31 -> rows 2, 3
#undef MOE_DPP_ADD
  return __uint_as_float((uint32_t)__builtin_amdgcn_readlane((int)__float_as_uint(v), kWave - 1));
}

// In-place exclusive scan of a[0..n) in LDS by wave 0 of the block (n <= 64*16).
// Writes the total to a[n]. Caller synchronises before and after.
__device__ __forceinline__ void wave0_exclusive_scan(int *a, int n) {
  if (threadIdx.x >= kWave) return;
  const int lane = threadIdx.x;
  const int per = (n + kWave - 1) / kWave;
  const int lo = lane * per;
  const int hi = lo + per < n ? lo + per : n;
  int s = 0;
  for (int i = lo; i < hi; i++) s += a[i];
  const int incl = wave_inclusive_scan_dpp(s);
  int run = incl - s;
  for (int i = lo; i < hi; i++) {
    const int v = a[i];
    a[i] = run;
    run += v;
  }
  if (lane == kWave - 1) a[n] = incl;
}


__device__ __forceinline__ float silu_f(float g) { return g / (1.0f + __expf(-g)); }
__device__ __forceinline__ float sigmoid_f(float g) { return 1.0f / (1.0f + __expf(-g)); }
// bf16 epilogues: the quotient by the hardware reciprocal (v_rcp_f32, about 1 ulp),
// far below the bf16 rounding that follows. At g = -inf both forms give NaN; for any
// finite g the reciprocal of an infinite 1 + e^-g is 0, as with the division.
__device__ __forceinline__ float sigmoid_fast(float g) {
  return __builtin_amdgcn_rcpf(1.0f + __expf(-g));
}
__device__ __forceinline__ float silu_fast(float g) { return g * sigmoid_fast(g); }

}  // namespace moe
