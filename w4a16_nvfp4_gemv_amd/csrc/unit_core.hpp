// The VALU "unit" used by the small-M dense GEMV and the MoE kernels.
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

// Loads and accumulates one tile of one unit.
//   w          base of the weight matrix, row_bytes per row
//   s          base of the flat scale buffer (NVFP4), tiles_per_row tiles
//   rows/rv    the R rows and their validity
//   quad_ok[h] rows 4h..4h+3 form a quad (their scale words are one chunk)
//   x, ldx, M  activations (M tokens, BF16 row stride ldx elements)
template <bool FP4, int R, int MT>
__device__ __forceinline__ void unit_tile(const uint8_t* __restrict__ w, int64_t row_bytes,
                                          const uint8_t* __restrict__ s, int64_t tiles_per_row,
                                          const int64_t (&rows)[R], const bool (&rv)[R],
                                          const bool (&quad_ok)[R / 4], int64_t t,
                                          const uint16_t* __restrict__ x, int64_t ldx, int M,
                                          float (&acc)[R][MT]) {
  // Weight codes / bf16 weights of this tile: 2 x 16 bytes per row.
  u32x4 wq[R][2];
#pragma unroll
  for (int i = 0; i < R; ++i) {
    if (rv[i]) {
      const uint8_t* p = w + rows[i] * row_bytes + t * 32;
      wq[i][0] = load16_nt(p);
      wq[i][1] = load16_nt(p + 16);
    } else {
      wq[i][0] = u32x4{0, 0, 0, 0};
      wq[i][1] = u32x4{0, 0, 0, 0};
    }
  }
  if constexpr (FP4) {
    uint32_t sw[R];
#pragma unroll
    for (int h = 0; h < R / 4; ++h) {
      if (quad_ok[h]) {
        if (rv[4 * h]) {
          u32x4 c = load16(s + scale_word_offset(rows[4 * h], t, tiles_per_row));
          sw[4 * h + 0] = c.x;
          sw[4 * h + 1] = c.y;
          sw[4 * h + 2] = c.z;
          sw[4 * h + 3] = c.w;
        } else {
#pragma unroll
          for (int j = 0; j < 4; ++j) sw[4 * h + j] = 0;
        }
      } else {
#pragma unroll
        for (int j = 0; j < 4; ++j)
          sw[4 * h + j] = rv[4 * h + j] ? load4(s + scale_word_offset(rows[4 * h + j], t, tiles_per_row)) : 0u;
      }
    }
    // 4 blocks of 16 k; block b uses code dwords 2b, 2b+1 and x dwords 8b..8b+7.
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      uint32_t xr[MT][8];
#pragma unroll
      for (int m = 0; m < MT; ++m) {
        if (m < M) {
          const uint16_t* xp = x + m * ldx + t * 64 + b * 16;
          u32x4 a = load16(xp), c = load16(xp + 8);
          xr[m][0] = a.x; xr[m][1] = a.y; xr[m][2] = a.z; xr[m][3] = a.w;
          xr[m][4] = c.x; xr[m][5] = c.y; xr[m][6] = c.z; xr[m][7] = c.w;
        } else {
#pragma unroll
          for (int q = 0; q < 8; ++q) xr[m][q] = 0;
        }
      }
#pragma unroll
      for (int i = 0; i < R; ++i) {
        float sc;
        if (b == 0) sc = e4m3_to_f32<0>(sw[i]);
        else if (b == 1) sc = e4m3_to_f32<1>(sw[i]);
        else if (b == 2) sc = e4m3_to_f32<2>(sw[i]);
        else sc = e4m3_to_f32<3>(sw[i]);
        const uint32_t d0 = (b < 2) ? ((b == 0) ? wq[i][0].x : wq[i][0].z) : ((b == 2) ? wq[i][1].x : wq[i][1].z);
        const uint32_t d1 = (b < 2) ? ((b == 0) ? wq[i][0].y : wq[i][0].w) : ((b == 2) ? wq[i][1].y : wq[i][1].w);
        uint32_t pr[8];
        dequant_dword(d0, sc, pr);
        dequant_dword(d1, sc, pr + 4);
#pragma unroll
        for (int m = 0; m < MT; ++m) {
          float a = acc[i][m];
#pragma unroll
          for (int q = 0; q < 8; ++q) a = dot2_bf16(pr[q], xr[m][q], a);
          acc[i][m] = a;
        }
      }
    }
  } else {
    uint32_t xr[MT][8];
#pragma unroll
    for (int m = 0; m < MT; ++m) {
      if (m < M) {
        const uint16_t* xp = x + m * ldx + t * 16;
        u32x4 a = load16(xp), c = load16(xp + 8);
        xr[m][0] = a.x; xr[m][1] = a.y; xr[m][2] = a.z; xr[m][3] = a.w;
        xr[m][4] = c.x; xr[m][5] = c.y; xr[m][6] = c.z; xr[m][7] = c.w;
      } else {
#pragma unroll
        for (int q = 0; q < 8; ++q) xr[m][q] = 0;
      }
    }
#pragma unroll
    for (int i = 0; i < R; ++i) {
      const uint32_t wd[8] = {wq[i][0].x, wq[i][0].y, wq[i][0].z, wq[i][0].w,
                              wq[i][1].x, wq[i][1].y, wq[i][1].z, wq[i][1].w};
#pragma unroll
      for (int m = 0; m < MT; ++m) {
        float a = acc[i][m];
#pragma unroll
        for (int q = 0; q < 8; ++q) a = dot2_bf16(wd[q], xr[m][q], a);
        acc[i][m] = a;
      }
    }
  }
}

// Whole-K accumulation of one unit by one lane of its LPQ-lane group,
// followed by the group reduction (every lane of the group gets the sums).
template <bool FP4, int R, int MT, int LPQ>
__device__ __forceinline__ void unit_dot(const uint8_t* __restrict__ w, int64_t row_bytes,
                                         const uint8_t* __restrict__ s, int64_t tiles,
                                         const int64_t (&rows)[R], const bool (&rv)[R],
                                         const bool (&quad_ok)[R / 4],
                                         const uint16_t* __restrict__ x, int64_t ldx, int M,
                                         int li, bool active, float (&acc)[R][MT]) {
#pragma unroll
  for (int i = 0; i < R; ++i)
#pragma unroll
    for (int m = 0; m < MT; ++m) acc[i][m] = 0.0f;
  if (active) {
    for (int64_t t = li; t < tiles; t += LPQ)
      unit_tile<FP4, R, MT>(w, row_bytes, s, tiles, rows, rv, quad_ok, t, x, ldx, M, acc);
  }
#pragma unroll
  for (int i = 0; i < R; ++i)
#pragma unroll
    for (int m = 0; m < MT; ++m) acc[i][m] = group_sum<LPQ>(acc[i][m]);
}

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
