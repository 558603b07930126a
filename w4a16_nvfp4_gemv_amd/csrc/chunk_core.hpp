// Chunk-interleaved NVFP4 row loads and dot products: the building block of
// the chunked VALU kernels (dense GEMV at small M, MoE decode pair).
//
// K is cut into 8-k chunks: 4 code bytes of a weight row and 16 activation
// bytes of a token row.  The C chunk positions of a lane are chosen by the
// caller (ch[c]); when lane l takes chunk base + l, a chunk load of the wave
// covers 256 contiguous bytes of a weight row or 1 KB of a token row.  The
// block scale of chunk ch is byte (ch/2) % 4 of its row's word in tile ch/8;
// with ch = base + l and base a multiple of 64 that byte index is (l/2) % 4
// for every position, so one fixed shift serves all of a lane's chunks.
//
// Numerics (nvfp4_gemv page, module docstring "Numerics", with the summation
// order left free): the E2M1 codes of a chunk become exact BF16 pairs at unit
// scale, the 8 products with x are summed in FP32 (v_dot2_f32_bf16), and the
// chunk sum is multiplied by the chunk's E4M3 scale into the FP32
// accumulator.  x * e2m1 is exact, so this is the sum of x * (e2m1 * e4m3)
// with its own FP32 rounding sequence.
#pragma once

#include "device_common.hpp"

namespace w4a16 {

// Codes and scale words of C chunk positions of R rows (R = 4: one quad of
// rows; R = 8: two quads).
template <int C, int R>
struct ChunkW {
  uint32_t w[C][R];
  uint32_t s[C][R];
};

// Activation chunks of MT token rows.
template <int C, int MT>
struct ChunkX {
  u32x4 x[MT][C];
};

// The two E2M1 codes of byte SEL of `word` as an exact BF16 pair.
template <int SEL>
__device__ __forceinline__ uint32_t e2m1x2_bf16_pair(uint32_t word) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(word, 1.0f, SEL));
}

// Issues the scale and code loads of one lane's chunk positions.
//   rows/rv     the R rows (byte offsets are taken relative to rw / rs)
//   quad_ok[h]  rows 4h..4h+3 are an aligned quad {r, r+32, r+64, r+96} of
//               one 128-row band, so their scale words are one 16-byte chunk
//   ch/ok       chunk index of each position and whether it is in range
// Every load is unconditional: positions or rows out of range use an
// out-of-range offset and read zeros.
template <int C, int R>
__device__ __forceinline__ void chunk_issue_w(ChunkW<C, R>& b, rsrc_t rw, uint32_t row_bytes, rsrc_t rs,
                                              uint32_t tiles, const int64_t (&rows)[R], const bool (&rv)[R],
                                              const bool (&quad_ok)[R / 4], const uint32_t (&ch)[C],
                                              const bool (&ok)[C]) {
#pragma unroll
  for (int c = 0; c < C; ++c) {
    const uint32_t t = ch[c] >> 3;
#pragma unroll
    for (int h = 0; h < R / 4; ++h) {
      if (quad_ok[h]) {
        const u32x4 sc =
            bload16(rs, off_if(ok[c] & rv[4 * h], static_cast<uint32_t>(scale_word_offset(rows[4 * h], t, tiles))));
        b.s[c][4 * h + 0] = sc.x;
        b.s[c][4 * h + 1] = sc.y;
        b.s[c][4 * h + 2] = sc.z;
        b.s[c][4 * h + 3] = sc.w;
      } else {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          b.s[c][4 * h + j] = bload4(
              rs, off_if(ok[c] & rv[4 * h + j], static_cast<uint32_t>(scale_word_offset(rows[4 * h + j], t, tiles))));
        }
      }
    }
  }
#pragma unroll
  for (int c = 0; c < C; ++c)
#pragma unroll
    for (int i = 0; i < R; ++i)
      b.w[c][i] = bload4_nt(rw, off_if(ok[c] & rv[i], static_cast<uint32_t>(rows[i]) * row_bytes + ch[c] * 4));
}

// Issues the activation loads: token m's row starts at byte xoff[m] of rx
// (kOutOfRange for an absent token; adding a chunk offset keeps it out of
// range).
template <int C, int MT>
__device__ __forceinline__ void chunk_issue_x(ChunkX<C, MT>& b, rsrc_t rx, const uint32_t (&xoff)[MT],
                                              const uint32_t (&ch)[C], const bool (&ok)[C]) {
#pragma unroll
  for (int c = 0; c < C; ++c)
#pragma unroll
    for (int m = 0; m < MT; ++m)
      b.x[m][c] = bload16(rx, off_if(ok[c], xoff[m] + ch[c] * 16));
}

// acc[i][m] += sum over the lane's chunks of row i times token m.  `shift`
// selects the lane's scale byte: 8 * ((lane / 2) % 4).
template <int C, int R, int MT>
__device__ __forceinline__ void chunk_compute(const ChunkW<C, R>& w, const ChunkX<C, MT>& x, uint32_t shift,
                                              float (&acc)[R][MT]) {
#pragma unroll
  for (int c = 0; c < C; ++c) {
#pragma unroll
    for (int i = 0; i < R; ++i) {
      const uint32_t pr[4] = {e2m1x2_bf16_pair<0>(w.w[c][i]), e2m1x2_bf16_pair<1>(w.w[c][i]),
                              e2m1x2_bf16_pair<2>(w.w[c][i]), e2m1x2_bf16_pair<3>(w.w[c][i])};
      const float sc = e4m3_to_f32<0>(w.s[c][i] >> shift);
#pragma unroll
      for (int m = 0; m < MT; ++m) {
        float a = dot2_bf16(pr[0], x.x[m][c].x, 0.0f);
        a = dot2_bf16(pr[1], x.x[m][c].y, a);
        a = dot2_bf16(pr[2], x.x[m][c].z, a);
        a = dot2_bf16(pr[3], x.x[m][c].w, a);
        acc[i][m] = __builtin_fmaf(a, sc, acc[i][m]);
      }
    }
  }
}

}  // namespace w4a16
