// Dense small-M GEMV kernels for gfx950: out = bf16(fp32(x @ W^T) * gs).
//
// Two kernel families serve the same entry points:
//   * k_gemv_valu  -- VALU dot path for the smallest M.  Lanes split K, every
//     lane keeps FP32 partial sums for all rows of its unit and all tokens,
//     and the lane group is reduced with cross-lane adds.  Weights are
//     dequantized exactly to BF16 pairs and consumed by v_dot2_f32_bf16.
//   * k_gemv_mfma  -- swap-AB MFMA path (v_mfma_f32_16x16x32_bf16): the 16
//     weight rows of a tile are the A operand, up to 16 tokens the B operand.
//     The four waves of a workgroup split K and reduce through LDS.
// Both stream every weight byte exactly once with 16-byte loads, and both
// apply the FP32 global scale to the FP32 sum before the single BF16 rounding
// (nvfp4_gemv page, module docstring "Numerics").
#include "device_common.hpp"
#include "launch.hpp"
#include "unit_core.hpp"

namespace w4a16 {

// ------------------------------------------------------------------ VALU
template <bool FP4, int MT, int LPQ, bool SILU>
__global__ __launch_bounds__(256) void k_gemv_valu(const GemvParams p) {
  constexpr int R = SILU ? 8 : 4;
  constexpr int G = kWave / LPQ;  // units a wave works on at once
  const int lane = threadIdx.x & 63;
  const int li = lane % LPQ;
  const int slot = lane / LPQ;
  const int wave = threadIdx.x >> 6;
  const int64_t gwave = static_cast<int64_t>(xcd_logical_block()) * 4 + wave;
  const int64_t stride = static_cast<int64_t>(gridDim.x) * 4 * G;
  const int64_t limit = SILU ? p.half : p.N;
  const int64_t row_bytes = FP4 ? p.K / 2 : static_cast<int64_t>(p.K) * 2;
  const float gs = FP4 ? *p.gs : 1.0f;
  const bool quad_b = FP4 && SILU && (p.half % 128 == 0);

  for (int64_t ubase = gwave * G; ubase < p.units; ubase += stride) {
    const int64_t u = ubase + slot;
    const bool active = u < p.units;
    int64_t rows[R];
    bool rv[R];
    if constexpr (FP4) quad_rows<R>(u, limit, p.half, rows, rv);
    else consecutive_rows<R>(u, limit, p.half, rows, rv);
    bool quad_ok[R / 4];
    quad_ok[0] = true;
    if constexpr (R == 8) quad_ok[1] = quad_b;
    float acc[R][MT];
    unit_dot<FP4, R, MT, LPQ>(p.w, row_bytes, p.s, p.tiles, rows, rv, quad_ok, p.x, p.ldx,
                              p.M, li, active, acc);
    if (!active) continue;
    // Each lane of the group writes the outputs whose index is li mod LPQ.
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
      for (int m = 0; m < MT; ++m) {
        if ((i * MT + m) % LPQ != li || m >= p.M || !rv[i]) continue;
        if constexpr (!SILU) {
          p.out[m * static_cast<int64_t>(p.N) + rows[i]] = f32_to_bf16_bits(acc[i][m] * gs);
        } else {
          const float g = bf16_bits_to_f32(f32_to_bf16_bits(acc[i][m] * gs));
          const float up = bf16_bits_to_f32(f32_to_bf16_bits(acc[4 + i][m] * gs));
          p.out[m * static_cast<int64_t>(p.half) + rows[i]] = f32_to_bf16_bits(silu_f32(g) * up);
        }
      }
    }
  }
}

// ------------------------------------------------------------------ MFMA
// Tile of 16 rows: NVFP4 rows {band*128 + 4q + (r&3) + 32(r>>2)} (q = tile % 8),
// whose scale words for one 64-k tile are 64 contiguous bytes; BF16 rows are
// 16 consecutive rows.  A step covers 128 k (NVFP4: 64 bytes per row, one
// 16-byte load per lane feeding 4 MFMAs) or 32 k (BF16: one 16-byte load per
// lane feeding 1 MFMA).  Lane l supplies row l%16 and k-group l/16.
template <bool FP4>
__device__ __forceinline__ int64_t mfma_row(int64_t tile, int r) {
  if constexpr (FP4) return (tile >> 3) * 128 + (tile & 7) * 4 + (r & 3) + 32 * (r >> 2);
  else return tile * 16 + r;
}

template <bool FP4, int NT, bool SILU>
__global__ __launch_bounds__(256) void k_gemv_mfma(const GemvParams p) {
  constexpr int NA = SILU ? 2 : 1;           // A operands per step (gate, up)
  constexpr int KSTEP = FP4 ? 128 : 32;       // k per step
  __shared__ f32x4 red[4][NA][NT][64];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int r = lane & 15;
  const int g = lane >> 4;
  const int64_t limit = SILU ? p.half : p.N;
  const int64_t row_bytes = FP4 ? p.K / 2 : static_cast<int64_t>(p.K) * 2;
  const float gs = FP4 ? *p.gs : 1.0f;
  const int64_t nsteps = (p.K + KSTEP - 1) / KSTEP;

  for (int64_t tile = xcd_logical_block(); tile < p.units; tile += gridDim.x) {
    int64_t rows[NA];
    bool rv[NA];
    rows[0] = mfma_row<FP4>(tile, r);
    rv[0] = rows[0] < limit;
    if constexpr (SILU) {
      rows[1] = rows[0] + p.half;
      rv[1] = rv[0];
    }
    f32x4 acc[NA][NT];
#pragma unroll
    for (int a = 0; a < NA; ++a)
#pragma unroll
      for (int n = 0; n < NT; ++n) acc[a][n] = f32x4{0, 0, 0, 0};

    for (int64_t st = wave; st < nsteps; st += 4) {
      if constexpr (FP4) {
        const int64_t k0 = st * 128 + g * 32;  // this lane's 32 k
        const bool kv = k0 < p.K;
        u32x4 wv[NA];
        uint32_t sw[NA];
#pragma unroll
        for (int a = 0; a < NA; ++a) {
          if (rv[a] && kv) {
            wv[a] = load16_nt(p.w + rows[a] * row_bytes + k0 / 2);
            sw[a] = load4(p.s + scale_word_offset(rows[a], k0 / 64, p.tiles)) >> (16 * (g & 1));
          } else {
            wv[a] = u32x4{0, 0, 0, 0};
            sw[a] = 0;
          }
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          // B fragments: tokens 16n + r, k0 + 8j .. +7
          bf16x8 bx[NT];
#pragma unroll
          for (int n = 0; n < NT; ++n) {
            const int m = 16 * n + r;
            u32x4 v = (m < p.M && kv) ? load16(p.x + m * p.ldx + k0 + 8 * j) : u32x4{0, 0, 0, 0};
            bx[n] = __builtin_bit_cast(bf16x8, v);
          }
#pragma unroll
          for (int a = 0; a < NA; ++a) {
            const float sc = (j < 2) ? e4m3_to_f32<0>(sw[a]) : e4m3_to_f32<1>(sw[a]);
            const uint32_t word = (j == 0) ? wv[a].x : (j == 1) ? wv[a].y : (j == 2) ? wv[a].z : wv[a].w;
            uint32_t pr[4];
            dequant_dword(word, sc, pr);
            const bf16x8 av = __builtin_bit_cast(bf16x8, u32x4{pr[0], pr[1], pr[2], pr[3]});
#pragma unroll
            for (int n = 0; n < NT; ++n)
              acc[a][n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, bx[n], acc[a][n], 0, 0, 0);
          }
        }
      } else {
        const int64_t k0 = st * 32 + g * 8;
        const bool kv = k0 < p.K;
        bf16x8 av[NA];
#pragma unroll
        for (int a = 0; a < NA; ++a) {
          u32x4 v = (rv[a] && kv) ? load16_nt(p.w + rows[a] * row_bytes + k0 * 2) : u32x4{0, 0, 0, 0};
          av[a] = __builtin_bit_cast(bf16x8, v);
        }
#pragma unroll
        for (int n = 0; n < NT; ++n) {
          const int m = 16 * n + r;
          u32x4 v = (m < p.M && kv) ? load16(p.x + m * p.ldx + k0) : u32x4{0, 0, 0, 0};
          const bf16x8 bx = __builtin_bit_cast(bf16x8, v);
#pragma unroll
          for (int a = 0; a < NA; ++a)
            acc[a][n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av[a], bx, acc[a][n], 0, 0, 0);
        }
      }
    }
    // Split-K reduction of the four waves through LDS.
#pragma unroll
    for (int a = 0; a < NA; ++a)
#pragma unroll
      for (int n = 0; n < NT; ++n) red[wave][a][n][lane] = acc[a][n];
    __syncthreads();
    if (wave == 0) {
#pragma unroll
      for (int a = 0; a < NA; ++a)
#pragma unroll
        for (int n = 0; n < NT; ++n)
          acc[a][n] = red[0][a][n][lane] + red[1][a][n][lane] + red[2][a][n][lane] + red[3][a][n][lane];
      // C layout: lane l holds rows 4(l/16)+i of the tile, token column l%16.
#pragma unroll
      for (int n = 0; n < NT; ++n) {
        const int m = 16 * n + (lane & 15);
        if (m >= p.M) continue;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int64_t row = mfma_row<FP4>(tile, 4 * (lane >> 4) + i);
          if (row >= limit) continue;
          if constexpr (!SILU) {
            p.out[m * static_cast<int64_t>(p.N) + row] = f32_to_bf16_bits(acc[0][n][i] * gs);
          } else {
            const float gv = bf16_bits_to_f32(f32_to_bf16_bits(acc[0][n][i] * gs));
            const float uv = bf16_bits_to_f32(f32_to_bf16_bits(acc[1][n][i] * gs));
            p.out[m * static_cast<int64_t>(p.half) + row] = f32_to_bf16_bits(silu_f32(gv) * uv);
          }
        }
      }
    }
    __syncthreads();
  }
}

// ------------------------------------------------------------------ launch
namespace {

int lanes_per_unit(int64_t tiles) {
  if (tiles > 32) return 64;
  if (tiles > 16) return 32;
  if (tiles > 8) return 16;
  return 8;
}

template <bool FP4, int MT, bool SILU>
hipError_t launch_valu(const GemvParams& p, int lpq, hipStream_t stream) {
  const int64_t g = kWave / lpq;
  const int64_t waves = (p.units + g - 1) / g;
  int64_t blocks = (waves + 3) / 4;
  if (blocks > 8192) blocks = 8192;
  const dim3 grid(static_cast<unsigned>(blocks)), block(256);
  switch (lpq) {
    case 64: hipLaunchKernelGGL((k_gemv_valu<FP4, MT, 64, SILU>), grid, block, 0, stream, p); break;
    case 32: hipLaunchKernelGGL((k_gemv_valu<FP4, MT, 32, SILU>), grid, block, 0, stream, p); break;
    case 16: hipLaunchKernelGGL((k_gemv_valu<FP4, MT, 16, SILU>), grid, block, 0, stream, p); break;
    default: hipLaunchKernelGGL((k_gemv_valu<FP4, MT, 8, SILU>), grid, block, 0, stream, p); break;
  }
  return hipGetLastError();
}

template <bool FP4, int NT, bool SILU>
hipError_t launch_mfma(const GemvParams& p, hipStream_t stream) {
  int64_t blocks = p.units;
  if (blocks > 16384) blocks = 16384;
  hipLaunchKernelGGL((k_gemv_mfma<FP4, NT, SILU>), dim3(static_cast<unsigned>(blocks)), dim3(256),
                     0, stream, p);
  return hipGetLastError();
}

template <bool FP4, bool SILU>
hipError_t dispatch(GemvParams p, int path, hipStream_t stream) {
  const int64_t limit = SILU ? p.half : p.N;
  if (path == kPathValu) {
    p.tiles = FP4 ? p.K / 64 : p.K / 16;
    p.units = FP4 ? ((limit + 127) / 128) * 32 : (limit + 3) / 4;
    const int lpq = lanes_per_unit(p.tiles);
    if (p.M <= 1) return launch_valu<FP4, 1, SILU>(p, lpq, stream);
    if (p.M <= 2) return launch_valu<FP4, 2, SILU>(p, lpq, stream);
    return launch_valu<FP4, 4, SILU>(p, lpq, stream);
  }
  p.tiles = p.K / 64;
  p.units = FP4 ? ((limit + 127) / 128) * 8 : (limit + 15) / 16;
  if (p.M <= 16) return launch_mfma<FP4, 1, SILU>(p, stream);
  return launch_mfma<FP4, 2, SILU>(p, stream);
}

}  // namespace

int choose_gemv_path(bool fp4, int64_t M, int64_t N, int64_t K) {
  (void)fp4;
  (void)N;
  (void)K;
  return M <= 4 ? kPathValu : kPathMfma;
}

hipError_t launch_gemv(bool fp4, const GemvParams& p, int silu, int path, hipStream_t stream) {
  if (fp4) return silu ? dispatch<true, true>(p, path, stream) : dispatch<true, false>(p, path, stream);
  return silu ? dispatch<false, true>(p, path, stream) : dispatch<false, false>(p, path, stream);
}

}  // namespace w4a16
