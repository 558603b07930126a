// Building blocks of the 4x4 block MFMA kernels (dense GEMV and MoE).
//
// v_mfma_f32_4x4x4_16b_bf16 computes 16 independent 4x4x4 products, block b
// on lanes 4b..4b+3: lane 4b+i holds row i of block b's A operand (4 k),
// lane 4b+j column j of its B operand, and the result C[i][j] lands in item
// i of lane 4b+j.  The kernels make the 16 blocks 16 k ranges of the same 4
// weight rows (B) and 4 tokens (A), so that lane 4b+j can load 16 bytes of
// row j at byte 16b of a 256-byte stretch: every load of the wave reads 256
// contiguous bytes of each of 4 rows.
#pragma once

#include "device_common.hpp"

namespace w4a16 {

typedef short s16x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f32x4 mfma_4x4x4(u32x2 a, u32x2 b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_4x4x4bf16_1k(__builtin_bit_cast(s16x4, a), __builtin_bit_cast(s16x4, b), c, 0, 0,
                                                0);
}

// Sums V per-lane values over the 16 blocks of a wave and over the KS waves
// that split a unit's K: two half-wave swaps (permlane32 / permlane16) halve
// the values per lane, two DPP row rotations add the lanes 4 and 8 apart
// within each row of 16 (lanes of one quad row stay apart), and waves
// kw = 1..KS-1 of the unit hand their sums to wave kw = 0 through LDS, added
// in slice order.  Lane l of wave kw = 0 then holds, in v[0 .. V/4 - 1], the
// full sums of values base + 0 .. V/4 - 1 for quad row l % 4, base returned.
// Pairs (2t, 2t + 1) stay in one lane when V / 4 is even.  Contains a barrier
// of the workgroup when KS > 1.
template <int V, int KS>
__device__ __forceinline__ int blk_reduce(float (&v)[V], int lane, int wave, int kw) {
  static_assert(V % 4 == 0, "values come in groups of the 4 quad rows");
#pragma unroll
  for (int j = 0; j < V / 2; ++j) {
    const auto r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(uint32_t, v[j]),
                                                    __builtin_bit_cast(uint32_t, v[j + V / 2]), false, false);
    v[j] = __builtin_bit_cast(float, static_cast<uint32_t>(r[0])) + __builtin_bit_cast(float, static_cast<uint32_t>(r[1]));
  }
#pragma unroll
  for (int j = 0; j < V / 4; ++j) {
    const auto r = __builtin_amdgcn_permlane16_swap(__builtin_bit_cast(uint32_t, v[j]),
                                                    __builtin_bit_cast(uint32_t, v[j + V / 4]), false, false);
    v[j] = __builtin_bit_cast(float, static_cast<uint32_t>(r[0])) + __builtin_bit_cast(float, static_cast<uint32_t>(r[1]));
  }
#pragma unroll
  for (int j = 0; j < V / 4; ++j) {
    v[j] += dpp_f32<0x124>(v[j]);  // row_ror:4
    v[j] += dpp_f32<0x128>(v[j]);  // row_ror:8
  }
  if constexpr (KS > 1) {
    __shared__ float red[4][V / 4][64];
    if (kw > 0) {
#pragma unroll
      for (int j = 0; j < V / 4; ++j) red[wave][j][lane] = v[j];
    }
    __syncthreads();
    if (kw == 0) {
#pragma unroll
      for (int s2 = 1; s2 < KS; ++s2)
#pragma unroll
        for (int j = 0; j < V / 4; ++j) v[j] += red[wave + s2][j][lane];
    }
  }
  return (lane >> 5) * (V / 2) + ((lane >> 4) & 1) * (V / 4);
}

// The two bf16 codes-at-unit-scale pairs of MFMA step st (4 k) of a lane's
// 32 codes: bytes 2st, 2st + 1 of the 16 bytes (low nibble first).
__device__ __forceinline__ void blk_codes(const u32x4& w, u32x2 (&wb)[8]) {
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    const uint32_t x = w[d];
    wb[2 * d] = u32x2{__builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(x, 1.0f, 0)),
                      __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(x, 1.0f, 1))};
    wb[2 * d + 1] = u32x2{__builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(x, 1.0f, 2)),
                          __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(x, 1.0f, 3))};
  }
}

// acc += the lane's 32 codes (wb) times the 32 k of 4 tokens (xv, 4 x 16
// bytes), one MFMA chain per 16-k block scaled once by its E4M3 scale (s0,
// s1): the sum of x * (e2m1 * e4m3) with its own FP32 rounding sequence.
__device__ __forceinline__ void blk_mac(const u32x2 (&wb)[8], const u32x4 (&xv)[4], float s0, float s1, f32x4& acc) {
  f32x4 h0 = f32x4{0, 0, 0, 0}, h1 = f32x4{0, 0, 0, 0};
#pragma unroll
  for (int st = 0; st < 4; ++st) {
    const u32x4& xa = xv[st / 2];
    h0 = mfma_4x4x4(st % 2 ? u32x2{xa.z, xa.w} : u32x2{xa.x, xa.y}, wb[st], h0);
  }
#pragma unroll
  for (int st = 4; st < 8; ++st) {
    const u32x4& xa = xv[st / 2];
    h1 = mfma_4x4x4(st % 2 ? u32x2{xa.z, xa.w} : u32x2{xa.x, xa.y}, wb[st], h1);
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    acc[i] = __builtin_fmaf(h0[i], s0, acc[i]);
    acc[i] = __builtin_fmaf(h1[i], s1, acc[i]);
  }
}

}  // namespace w4a16
