// Building blocks of the swap-AB MFMA kernels (dense GEMV and MoE): row
// tiles, the LDS ring that stages activations, and the exact NVFP4 A
// fragment.
//
// v_mfma_f32_16x16x32_bf16 multiplies a 16 x 32 A operand (here 16 weight
// rows) by a 32 x 16 B operand (16 tokens).  Lane l holds row (or token)
// l % 16 and k = 8 * (l / 16) .. +7 of both operands, and receives C rows
// 4 * (l / 16) + i (i = 0..3) of token column l % 16.
#pragma once

#include "device_common.hpp"

namespace w4a16 {

// Row r (0..15) of 16-row tile `tile`.  NVFP4 tiles take rows
// {band*128 + 4q + (r&3) + 32(r>>2)} (q = tile % 8), whose scale words for a
// 64-k tile are 64 contiguous bytes of the 128x4-swizzled layout; BF16 tiles
// are 16 consecutive rows.
template <bool FP4>
__device__ __forceinline__ int64_t mfma_row(int64_t tile, int r) {
  if constexpr (FP4) return (tile >> 3) * 128 + (tile & 7) * 4 + (r & 3) + 32 * (r >> 2);
  else return tile * 16 + r;
}

// Ring position of activation chunk c (16 bytes) of token t (0..31) in its
// token segment of CPT chunks: the 8 or 16 lanes that one ds_read_b128 pass
// serves (same c, consecutive t) land in distinct banks.
template <int CPT>
__device__ __forceinline__ int xl_pos(int t, int c) {
  if constexpr (CPT == 16) return c ^ (t & 15);
  else return c ^ (((t >> 2) ^ (t >> 1)) & 3);
}

// Ring slot I of the staged activations, N chunks for all waves.  Each slot
// is an LDS allocation of its own: the compiler then knows that a read of
// one slot does not depend on the loads in flight into the others, and adds
// no wait of its own for them.
template <int I, int N>
__device__ __forceinline__ u32x4* xl_slot() {
  __shared__ u32x4 slot[N];
  return slot;
}

template <int N>
__device__ __forceinline__ u32x4* xl_slot(int d) {
  static_assert(N > 0);
  switch (d) {
    case 0: return xl_slot<0, N>();
    case 1: return xl_slot<1, N>();
    case 2: return xl_slot<2, N>();
    case 3: return xl_slot<3, N>();
    case 4: return xl_slot<4, N>();
    case 5: return xl_slot<5, N>();
    case 6: return xl_slot<6, N>();
    default: return xl_slot<7, N>();
  }
}

// A fragment j (0..3) of an NVFP4 step: lane (r, g) holds 32 codes of row r
// (k = 32g .. 32g+31 of the step) in `codes` and the row's scale word of the
// 64-k tile holding them; fragment j is k = 32g + 8j .. +7, dequantized
// exactly (e2m1 * e4m3 has at most 6 significant bits).
__device__ __forceinline__ bf16x8 fp4_a_fragment(const u32x4& codes, uint32_t scale_word, int g, int j) {
  const uint32_t sw = scale_word >> (16 * (g & 1));  // this lane's two block scales
  const float scale = (j < 2) ? e4m3_to_f32<0>(sw) : e4m3_to_f32<1>(sw);
  const uint32_t word = (j == 0) ? codes.x : (j == 1) ? codes.y : (j == 2) ? codes.z : codes.w;
  uint32_t pr[4];
  dequant_dword(word, scale, pr);
  return __builtin_bit_cast(bf16x8, u32x4{pr[0], pr[1], pr[2], pr[3]});
}

__device__ __forceinline__ f32x4 mfma_16x16x32(const bf16x8& a, const u32x4& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

}  // namespace w4a16
