// The VALU "unit" of the small-M dense GEMV kernels (the row-set helpers
// quad_rows / consecutive_rows also serve the MoE kernels).
//
// A unit is a set of R weight rows (4, or 8 = gate quad + up quad) that a
// group of LPQ lanes reduces over the whole K extent.  K is cut into tiles:
// an NVFP4 tile is 64 k (32 bytes of codes per row plus one 4-byte scale
// word per row); a BF16 tile is 16 k (32 bytes per row).  Lane li of the
// group owns tiles li, li + LPQ, ... and keeps FP32 partial sums for every
// (row, token); the group sum is formed afterwards with cross-lane adds.
//
// NVFP4 rows are taken as "quads" {r, r+32, r+64, r+96} of one 128-row band,
// whose scale words for a tile are one aligned 16-byte chunk of the 128x4
// swizzled buffer, so one 16-byte load brings all four scales.
#pragma once

#include "device_common.hpp"

namespace w4a16 {

// Rows of NVFP4 quad unit u within the first `limit` rows: band u / 32,
// rows band*128 + u%32 + 32j.
template <int R>
__device__ __forceinline__ void quad_rows(int64_t u, int64_t limit, int64_t second_offset,
                                          int64_t (&rows)[R], bool (&rv)[R]) {
  const int64_t base = (u >> 5) * 128 + (u & 31);
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    rows[j] = base + 32 * j;
    rv[j] = rows[j] < limit;
    if constexpr (R == 8) {
      rows[4 + j] = rows[j] + second_offset;
      rv[4 + j] = rv[j];
    }
  }
}

// Rows of a BF16 unit: 4 consecutive rows (plus the matching up rows).
template <int R>
__device__ __forceinline__ void consecutive_rows(int64_t u, int64_t limit, int64_t second_offset,
                                                 int64_t (&rows)[R], bool (&rv)[R]) {
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    rows[j] = 4 * u + j;
    rv[j] = rows[j] < limit;
    if constexpr (R == 8) {
      rows[4 + j] = rows[j] + second_offset;
      rv[4 + j] = rv[j];
    }
  }
}

}  // namespace w4a16

namespace w4a16 {

// ---------------------------------------------------------------------------
// Register-staged tile of one unit for the pipelined dense VALU kernel.
template <int R>
struct TileRegs {
  u32x4 w[R][2];   // 32 bytes per row
  uint32_t s[R];   // NVFP4 scale word per row (4 blocks of 16 k)
};

// Issues the loads of one (unit, tile) item: scale words first, then the rows
// in order, so that a row's compute can start when its own loads land.  All
// loads are unconditional buffer loads; rows that are not valid (past the
// matrix, inactive unit, tile past K) use an out-of-range offset and read 0.
template <bool FP4, int R>
__device__ __forceinline__ void tile_issue(TileRegs<R>& b, rsrc_t w, uint32_t row_bytes, rsrc_t s,
                                           uint32_t tiles_per_row, const int64_t (&rows)[R],
                                           const bool (&rv)[R], const bool (&quad_ok)[R / 4],
                                           uint32_t t, bool tv) {
  if constexpr (FP4) {
#pragma unroll
    for (int h = 0; h < R / 4; ++h) {
      if (quad_ok[h]) {
        const uint32_t off = (tv && rv[4 * h])
                                 ? static_cast<uint32_t>(scale_word_offset(rows[4 * h], t, tiles_per_row))
                                 : kOutOfRange;
        const u32x4 c = bload16(s, off);
        b.s[4 * h + 0] = c.x;
        b.s[4 * h + 1] = c.y;
        b.s[4 * h + 2] = c.z;
        b.s[4 * h + 3] = c.w;
      } else {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const uint32_t off = (tv && rv[4 * h + j])
                                   ? static_cast<uint32_t>(scale_word_offset(rows[4 * h + j], t, tiles_per_row))
                                   : kOutOfRange;
          b.s[4 * h + j] = bload4(s, off);
        }
      }
    }
  }
  uint32_t off[R];
#pragma unroll
  for (int i = 0; i < R; ++i)
    off[i] = (tv && rv[i]) ? static_cast<uint32_t>(rows[i]) * row_bytes + t * 32 : kOutOfRange;
  // first 16 bytes of every row, then the second 16: the first half of the
  // tile can be consumed while the second is still arriving
#pragma unroll
  for (int i = 0; i < R; ++i) b.w[i][0] = bload16_nt(w, off[i]);
#pragma unroll
  for (int i = 0; i < R; ++i) b.w[i][1] = bload16_nt(w, off[i] + 16);
}

// Position of 16-byte chunk q of a staged activation row in LDS.  Lanes read
// chunks 8 (NVFP4) or 2 (BF16) apart; XOR-ing the low 3 bits with bits 4..6
// spreads 16 consecutive lanes over all 16 bank groups.
__device__ __forceinline__ int64_t lds_chunk(int64_t q) { return q ^ ((q >> 4) & 7); }

template <int SEL>
__device__ __forceinline__ uint32_t e2m1x2_bf16(uint32_t word) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(word, 1.0f, SEL));
}

// Activation slice of one tile for MT tokens: NVFP4 tiles are 64 k (32 bf16
// pairs per token), BF16 tiles 16 k (8 pairs).
template <bool FP4, int MT>
struct TileX {
  uint32_t v[MT][FP4 ? 32 : 8];
};

// The slice of tile t from the LDS staging area (xs: token 0, xstride
// elements per token, 16-byte chunks placed by lds_chunk).
template <bool FP4, int MT>
__device__ __forceinline__ void tile_x_lds(TileX<FP4, MT>& x, const uint16_t* xs, uint32_t xstride,
                                           uint32_t t, int M) {
  constexpr int C = FP4 ? 8 : 2;  // 16-byte chunks per tile
#pragma unroll
  for (int m = 0; m < MT; ++m) {
    const u32x4* xrow = reinterpret_cast<const u32x4*>(xs + (m < M ? m : 0) * xstride);
#pragma unroll
    for (int c = 0; c < C; ++c) {
      const u32x4 v = xrow[lds_chunk(t * C + c)];
      x.v[m][4 * c + 0] = m < M ? v.x : 0u;
      x.v[m][4 * c + 1] = m < M ? v.y : 0u;
      x.v[m][4 * c + 2] = m < M ? v.z : 0u;
      x.v[m][4 * c + 3] = m < M ? v.w : 0u;
    }
  }
}

// The slice of tile t straight from global memory (buffer loads; tokens past
// M and tiles past K read zero).
template <bool FP4, int MT>
__device__ __forceinline__ void tile_x_global(TileX<FP4, MT>& x, rsrc_t rx, uint32_t ldx_bytes,
                                              uint32_t t, bool tv, int M) {
  constexpr int C = FP4 ? 8 : 2;
#pragma unroll
  for (int m = 0; m < MT; ++m) {
#pragma unroll
    for (int c = 0; c < C; ++c) {
      const uint32_t off = (tv && m < M) ? m * ldx_bytes + (t * C + c) * 16 : kOutOfRange;
      const u32x4 v = bload16(rx, off);
      x.v[m][4 * c + 0] = v.x;
      x.v[m][4 * c + 1] = v.y;
      x.v[m][4 * c + 2] = v.z;
      x.v[m][4 * c + 3] = v.w;
    }
  }
}

// Accumulates half H (0: k 0..31, 1: k 32..63 of an NVFP4 tile; 0: k 0..7,
// 1: k 8..15 of a BF16 tile) of one tile; rows are interleaved so that the
// per-row dot chains are independent.
//   NVFP4: per 16-k block, the E2M1 codes become exact BF16 pairs, the 16
//   products with x are summed in FP32 (v_dot2_f32_bf16) and the block sum is
//   multiplied by the block's E4M3 scale into the FP32 accumulator (x * e2m1
//   is exact, so this is the product sum x * (e2m1 * e4m3) with a different
//   FP32 rounding sequence).
//   BF16: plain dot2 products into the accumulator.
template <bool FP4, int R, int MT, int H>
__device__ __forceinline__ void tile_compute_half(const TileRegs<R>& b, const TileX<FP4, MT>& x,
                                                  float (&acc)[R][MT]) {
  if constexpr (FP4) {
#pragma unroll
    for (int bb = 0; bb < 2; ++bb) {
      const int blk = 2 * H + bb;
      float part[R][MT];
#pragma unroll
      for (int i = 0; i < R; ++i) {
        const uint32_t d0 = bb == 0 ? b.w[i][H].x : b.w[i][H].z;
        const uint32_t d1 = bb == 0 ? b.w[i][H].y : b.w[i][H].w;
        const uint32_t pr[8] = {e2m1x2_bf16<0>(d0), e2m1x2_bf16<1>(d0), e2m1x2_bf16<2>(d0), e2m1x2_bf16<3>(d0),
                                e2m1x2_bf16<0>(d1), e2m1x2_bf16<1>(d1), e2m1x2_bf16<2>(d1), e2m1x2_bf16<3>(d1)};
#pragma unroll
        for (int m = 0; m < MT; ++m) {
          float a = 0.0f;
#pragma unroll
          for (int q = 0; q < 8; ++q) a = dot2_bf16(pr[q], x.v[m][8 * blk + q], a);
          part[i][m] = a;
        }
      }
#pragma unroll
      for (int i = 0; i < R; ++i) {
        float sc;
        if (blk == 0) sc = e4m3_to_f32<0>(b.s[i]);
        else if (blk == 1) sc = e4m3_to_f32<1>(b.s[i]);
        else if (blk == 2) sc = e4m3_to_f32<2>(b.s[i]);
        else sc = e4m3_to_f32<3>(b.s[i]);
#pragma unroll
        for (int m = 0; m < MT; ++m) acc[i][m] = __builtin_fmaf(part[i][m], sc, acc[i][m]);
      }
    }
  } else {
#pragma unroll
    for (int i = 0; i < R; ++i) {
      const uint32_t wd[4] = {b.w[i][H].x, b.w[i][H].y, b.w[i][H].z, b.w[i][H].w};
#pragma unroll
      for (int m = 0; m < MT; ++m) {
        float a = acc[i][m];
#pragma unroll
        for (int q = 0; q < 4; ++q) a = dot2_bf16(wd[q], x.v[m][4 * H + q], a);
        acc[i][m] = a;
      }
    }
  }
}

template <bool FP4, int R, int MT>
__device__ __forceinline__ void tile_compute(const TileRegs<R>& b, const TileX<FP4, MT>& x, bool tv,
                                             float (&acc)[R][MT]) {
  if (!tv) return;
  tile_compute_half<FP4, R, MT, 0>(b, x, acc);
  tile_compute_half<FP4, R, MT, 1>(b, x, acc);
}

}  // namespace w4a16
