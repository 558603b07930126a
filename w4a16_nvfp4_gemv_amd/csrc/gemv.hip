// Dense small-M GEMV kernels for gfx950: out = bf16(fp32(x @ W^T) * gs).
//
// Four kernel families serve the same entry points:
//   * k_gemv_vchunk -- NVFP4 rows of up to 16384 columns at one token (two
//     for rows longer than 4096; up to 4 when the VALU path is forced).
//     VALU dot products over exactly decoded BF16 pairs (v_dot2_f32_bf16);
//     lanes own interleaved 8-k chunks so that every load instruction of a
//     wave reads one contiguous stretch, and a permlane reduce-scatter sums
//     the lanes.
//   * k_gemv_blk -- NVFP4 at 2..4 tokens, rows of up to 4096 columns (with
//     or without silu_mul): the same streaming as k_gemv_vchunk (256
//     contiguous bytes of a row per load, every load issued up front), with
//     the products on v_mfma_f32_4x4x4_16b_bf16, whose 16 blocks take 16 k
//     ranges of 4 rows.  k_gemv_blkh is its BF16-weight form (1..8 tokens,
//     without silu_mul; the activations go straight into the MFMA operands).
//   * k_gemv_valu1 / k_gemv_valu -- the same VALU scheme with lanes owning
//     whole 64-k (NVFP4) or 16-k (BF16) tiles: BF16 weights with silu_mul at
//     M = 1 beyond 8192 columns and NVFP4 rows longer than 16384 columns at
//     M <= 2.
//   * k_gemv_mfma -- swap-AB MFMA path (v_mfma_f32_16x16x32_bf16): the 16
//     weight rows of a tile are the A operand, up to 16 tokens the B operand,
//     staged through an LDS ring.  The waves of a workgroup split K and
//     reduce through LDS.
// All of them stream every weight byte exactly once with buffer loads, and
// all apply the FP32 global scale to the FP32 sum before the single BF16
// rounding (nvfp4_gemv page, module docstring "Numerics").
#include <atomic>
#include <cstdio>
#include <cstdlib>
#include <cstring>

#include "blk_core.hpp"
#include "device_common.hpp"
#include "launch.hpp"
#include "mfma_core.hpp"
#include "unit_core.hpp"

namespace w4a16 {

// ------------------------------------------------------------------ VALU
// A unit is a quad of rows (NVFP4) or 4 consecutive rows (BF16), plus the
// matching up rows with silu_mul; LPQ lanes split the unit's K tiles.  The
// workgroup first stages all M activation rows in LDS (their global loads are
// issued before any weight load, so waiting for them never waits behind the
// HBM stream), and every wave streams its (unit, tile) items with the next
// item's loads in flight while the current one is computed.
template <int R>
struct UnitRows {
  int64_t rows[R];
  bool rv[R];
  bool quad_ok[R / 4];
};

template <bool FP4, bool SILU, int R>
__device__ __forceinline__ UnitRows<R> unit_rows(const GemvParams& p, int64_t u) {
  UnitRows<R> r;
  const int64_t limit = SILU ? p.half : p.N;
  if constexpr (FP4) quad_rows<R>(u, limit, p.half, r.rows, r.rv);
  else consecutive_rows<R>(u, limit, p.half, r.rows, r.rv);
  if (u >= p.units) {
#pragma unroll
    for (int i = 0; i < R; ++i) r.rv[i] = false;
  }
  r.quad_ok[0] = true;
  if constexpr (R == 8) r.quad_ok[1] = FP4 && (p.half % 128 == 0);
  return r;
}

// Index (in 16-byte chunks) of the spare LDS chunk that absorbs the writes of
// staging slots past the end of the activations.
__device__ __forceinline__ uint32_t chunks_dummy(int M, uint32_t xstride) {
  return static_cast<uint32_t>(M) * (xstride / 8);
}

// Single-unit form: every wave-slot owns one unit and every lane exactly one
// tile (the tiles of a row fit in LPQ lanes), so the whole kernel is straight
// line code -- activation slice, scale words, the first and then the second
// 16 bytes of every row are issued back to back, and each half is consumed as
// soon as it has landed.
template <bool FP4, int MT, int LPQ, bool SILU>
__global__ __launch_bounds__(256) void k_gemv_valu1(const GemvParams p) {
  constexpr int R = SILU ? 8 : 4;
  constexpr int G = kWave / LPQ;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int li = lane % LPQ;
  const int slot = lane / LPQ;
  const int gwave = xcd_logical_block() * 4 + (tid >> 6);
  const uint32_t row_bytes = FP4 ? p.K / 2 : static_cast<uint32_t>(p.K) * 2;
  const int tiles = static_cast<int>(p.tiles);
  const int unit = gwave * G + slot;
  const bool tv = unit < static_cast<int>(p.units) && li < tiles;
  const rsrc_t rw = make_rsrc(p.w, p.w_bytes);
  const rsrc_t rs = make_rsrc(p.s, p.s_bytes);
  const rsrc_t rx = make_rsrc(p.x, p.x_bytes);

  // the global scale is read first: left to the epilogue, its load would add
  // a full memory round trip to the end of every wave
  const float gs = FP4 ? *p.gs : 1.0f;
  TileX<FP4, MT> xr;
  tile_x_global<FP4, MT>(xr, rx, static_cast<uint32_t>(p.ldx) * 2, li, tv, p.M);
  const UnitRows<R> ur = unit_rows<FP4, SILU, R>(p, unit);
  TileRegs<R> A;
  tile_issue<FP4, R>(A, rw, row_bytes, rs, p.tiles, ur.rows, ur.rv, ur.quad_ok, li, tv);
  // keep every load above ahead of all the arithmetic below
  __builtin_amdgcn_sched_barrier(0);

  float acc[R][MT];
#pragma unroll
  for (int i = 0; i < R; ++i)
#pragma unroll
    for (int m = 0; m < MT; ++m) acc[i][m] = 0.0f;
  tile_compute_half<FP4, R, MT, 0>(A, xr, acc);
  tile_compute_half<FP4, R, MT, 1>(A, xr, acc);

#pragma unroll
  for (int i = 0; i < R; ++i)
#pragma unroll
    for (int m = 0; m < MT; ++m) acc[i][m] = group_sum<LPQ>(acc[i][m]);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
#pragma unroll
    for (int m = 0; m < MT; ++m) {
      if ((i * MT + m) % LPQ == li && m < p.M && ur.rv[i]) {
        if constexpr (!SILU) {
          p.out[m * static_cast<int64_t>(p.N) + ur.rows[i]] = f32_to_bf16_bits(acc[i][m] * gs);
        } else {
          const float g = bf16_bits_to_f32(f32_to_bf16_bits(acc[i][m] * gs));
          const float up = bf16_bits_to_f32(f32_to_bf16_bits(acc[4 + i][m] * gs));
          p.out[m * static_cast<int64_t>(p.half) + ur.rows[i]] = f32_to_bf16_bits(silu_f32(g) * up);
        }
      }
    }
  }
}

// XREG: every lane owns exactly one tile (K <= 64 * LPQ tiles' worth), so its
// activation slice is loaded into registers once, before any weight load.
// Otherwise the workgroup stages all M activation rows in LDS first.
template <bool FP4, int MT, int LPQ, bool SILU, bool XREG>
__global__ __launch_bounds__(256) void k_gemv_valu(const GemvParams p) {
  constexpr int R = SILU ? 8 : 4;
  constexpr int G = kWave / LPQ;  // units a wave works on at once
  constexpr int XR = 8;           // 16-byte x chunks per thread issued before the weights
  extern __shared__ u32x4 xs_raw[];
  uint16_t* xs = reinterpret_cast<uint16_t*>(xs_raw);
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int li = lane % LPQ;
  const int slot = lane / LPQ;
  // 32-bit bookkeeping: units, tiles and items all stay far below 2^31
  const int nwaves = static_cast<int>(gridDim.x) * 4;
  const int gwave = xcd_logical_block() * 4 + (tid >> 6);
  const uint32_t row_bytes = FP4 ? p.K / 2 : static_cast<uint32_t>(p.K) * 2;
  const uint32_t xstride = (p.K + 63) / 64 * 64;  // LDS row stride (elements)
  const uint32_t ldx_bytes = static_cast<uint32_t>(p.ldx) * 2;
  const int tiles = static_cast<int>(p.tiles);
  const int units = static_cast<int>(p.units);
  const int ntl = (tiles + LPQ - 1) / LPQ;  // tiles per lane per unit
  const int first = gwave * G;
  const int nbatch = first < units ? (units - first + nwaves * G - 1) / (nwaves * G) : 0;
  const int n_items = nbatch * ntl;
  const rsrc_t rw = make_rsrc(p.w, p.w_bytes);
  const rsrc_t rs = make_rsrc(p.s, p.s_bytes);
  const rsrc_t rx = make_rsrc(p.x, p.x_bytes);

  // 1. activations, before any weight load
  TileX<FP4, MT> xa, xb;
  u32x4 xv[XR];
  uint32_t xdst[XR];
  const uint32_t kc = p.K / 8;
  const uint32_t chunks = static_cast<uint32_t>(p.M) * kc;
  if constexpr (XREG) {
    tile_x_global<FP4, MT>(xa, rx, ldx_bytes, li, n_items > 0 && li < tiles, p.M);
  } else {
#pragma unroll
    for (int r = 0; r < XR; ++r) {
      const uint32_t c = r * 256 + tid;
      const uint32_t m = c / kc, q = c - m * kc;
      const bool ok = c < chunks;
      xv[r] = bload16(rx, ok ? m * ldx_bytes + q * 16 : kOutOfRange);
      xdst[r] = ok ? m * (xstride / 8) + static_cast<uint32_t>(lds_chunk(q)) : chunks_dummy(p.M, xstride);
    }
  }

  // 2. first item's weight loads (issued unconditionally -- a wave without
  //    items reads out of range, i.e. nothing -- so that no branch separates
  //    them from the activation loads)
  TileRegs<R> A, B;
  UnitRows<R> ua, ub;
  bool ta = false, tb = false;
  uint32_t tA = 0, tB = 0;
  ua = unit_rows<FP4, SILU, R>(p, first + slot);
  tA = li;
  ta = n_items > 0 && static_cast<int>(tA) < tiles;
  tile_issue<FP4, R>(A, rw, row_bytes, rs, p.tiles, ua.rows, ua.rv, ua.quad_ok, tA, ta);

  // 3. staged activations into LDS (swizzled 16-byte chunks; unused slots
  //    write a spare chunk)
  if constexpr (!XREG) {
    u32x4* xs4 = reinterpret_cast<u32x4*>(xs);
#pragma unroll
    for (int r = 0; r < XR; ++r) xs4[xdst[r]] = xv[r];
    for (uint32_t c = XR * 256 + tid; c < chunks; c += 256) {
      const uint32_t m = c / kc, q = c - m * kc;
      xs4[m * (xstride / 8) + lds_chunk(q)] = bload16(rx, m * ldx_bytes + q * 16);
    }
    __syncthreads();
  }

  const float gs = FP4 ? *p.gs : 1.0f;
  float acc[R][MT];
#pragma unroll
  for (int i = 0; i < R; ++i)
#pragma unroll
    for (int m = 0; m < MT; ++m) acc[i][m] = 0.0f;

  auto finish_unit = [&](const UnitRows<R>& ur) {
#pragma unroll
    for (int i = 0; i < R; ++i)
#pragma unroll
      for (int m = 0; m < MT; ++m) acc[i][m] = group_sum<LPQ>(acc[i][m]);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
      for (int m = 0; m < MT; ++m) {
        if ((i * MT + m) % LPQ == li && m < p.M && ur.rv[i]) {
          if constexpr (!SILU) {
            p.out[m * static_cast<int64_t>(p.N) + ur.rows[i]] = f32_to_bf16_bits(acc[i][m] * gs);
          } else {
            const float g = bf16_bits_to_f32(f32_to_bf16_bits(acc[i][m] * gs));
            const float up = bf16_bits_to_f32(f32_to_bf16_bits(acc[4 + i][m] * gs));
            p.out[m * static_cast<int64_t>(p.half) + ur.rows[i]] = f32_to_bf16_bits(silu_f32(g) * up);
          }
        }
      }
    }
#pragma unroll
    for (int i = 0; i < R; ++i)
#pragma unroll
      for (int m = 0; m < MT; ++m) acc[i][m] = 0.0f;
  };

  // Items run unit batch by unit batch, tile by tile: (nb_unit, nb_tj) is the
  // next item to load, advanced without divisions.
  int nb_unit = first + slot, nb_tj = 0;
  auto advance = [&]() {
    if (++nb_tj == ntl) {
      nb_tj = 0;
      nb_unit += nwaves * G;
    }
  };
  advance();  // item 0 is already in A
  for (int it = 0; it < n_items; it += 2) {
    // A holds item it; bring item it+1 into B
    if (it + 1 < n_items) {
      ub = unit_rows<FP4, SILU, R>(p, nb_unit);
      tB = static_cast<uint32_t>(li + nb_tj * LPQ);
      tb = static_cast<int>(tB) < tiles;
      tile_issue<FP4, R>(B, rw, row_bytes, rs, p.tiles, ub.rows, ub.rv, ub.quad_ok, tB, tb);
      advance();
    }
    if constexpr (!XREG) tile_x_lds<FP4, MT>(xa, xs, xstride, tA, p.M);
    tile_compute<FP4, R, MT>(A, xa, ta && ua.rv[0], acc);
    if ((it % ntl) == ntl - 1) finish_unit(ua);
    if (it + 1 >= n_items) break;
    // B holds item it+1; bring item it+2 into A
    if (it + 2 < n_items) {
      ua = unit_rows<FP4, SILU, R>(p, nb_unit);
      tA = static_cast<uint32_t>(li + nb_tj * LPQ);
      ta = static_cast<int>(tA) < tiles;
      tile_issue<FP4, R>(A, rw, row_bytes, rs, p.tiles, ua.rows, ua.rv, ua.quad_ok, tA, ta);
      advance();
    }
    if constexpr (XREG) {
      tile_compute<FP4, R, MT>(B, xa, tb && ub.rv[0], acc);
    } else {
      tile_x_lds<FP4, MT>(xb, xs, xstride, tB, p.M);
      tile_compute<FP4, R, MT>(B, xb, tb && ub.rv[0], acc);
    }
    if (((it + 1) % ntl) == ntl - 1) finish_unit(ub);
  }
}

// ------------------------------------------------------------------ VALU, chunked
// NVFP4 form of the VALU path in which every load instruction of a wave reads
// one contiguous stretch of memory.  A unit is one quad (plus its up quad with
// silu_mul) and KS waves of a workgroup share it, each taking a contiguous
// slice of K.  K is cut into 8-k chunks -- 4 code bytes of a row, 16
// activation bytes of a token -- and lane l of slice s owns chunks
// (s*C + c)*64 + l for c < C, so a chunk load of the wave covers 256
// contiguous bytes of a weight row or 1 KB of an activation row.  The scale of
// chunk ch is byte (ch/2) % 4 = (l/2) % 4 of its row's word in tile ch/8: the
// lane reads the quad's 16-byte scale chunk of that tile and shifts by a fixed
// amount.  All loads are issued up front (activations, scales, then weights
// chunk by chunk), the 8 products of a chunk are summed in FP32 and scaled
// once, each wave's partial sums meet through a permlane reduce-scatter, and
// the KS slices are added in slice order through LDS.
// PAIR (without silu_mul): a unit is two adjacent quads (rows r and r + 1 of
// each quad position), so every activation chunk a wave loads serves 8 rows
// instead of 4 and the two quads' scale chunks share one cache line.
template <int MT, bool SILU, int C, int KS, bool PAIR>
__global__ __launch_bounds__(256) void k_gemv_vchunk(const GemvParams p) {
  static_assert(!(SILU && PAIR), "a pair unit has no up half");
  constexpr int R = (SILU || PAIR) ? 8 : 4;
  constexpr int NQ = R / 4;
  constexpr int P = (SILU || PAIR) ? 2 : 1;
  constexpr int V = MT * 4 * P;  // value index v = (m * 4 + q) * P + u
  using RS = ReduceScatter<V, P>;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform, and known to be
  const int kw = wave % KS;
  const int unit = xcd_logical_block() * (4 / KS) + wave / KS;
  const uint32_t row_bytes = p.K / 2;
  const uint32_t nch = p.K / 8;
  const uint32_t ch0 = static_cast<uint32_t>(kw * C) * 64 + lane;
  const uint32_t ldx_bytes = static_cast<uint32_t>(p.ldx) * 2;
  const rsrc_t rw = make_rsrc(p.w, p.w_bytes);
  const rsrc_t rs = make_rsrc(p.s, p.s_bytes);
  const rsrc_t rx = make_rsrc(p.x, p.x_bytes);

  const float gs = *p.gs;
  UnitRows<R> ur;
  if constexpr (PAIR) {
    // quads 2 unit and 2 unit + 1: the second quad's rows are the first's + 1
    quad_rows<R>(2 * static_cast<int64_t>(unit), p.N, 1, ur.rows, ur.rv);
#pragma unroll
    for (int i = 0; i < R; ++i) ur.rv[i] = ur.rv[i] && unit < p.units;
    ur.quad_ok[0] = true;
    ur.quad_ok[1] = true;
  } else {
    ur = unit_rows<true, SILU, R>(p, unit);
  }

  u32x4 xv[MT][C];
#pragma unroll
  for (int c = 0; c < C; ++c) {
    const uint32_t ch = ch0 + c * 64;
#pragma unroll
    for (int m = 0; m < MT; ++m)
      xv[m][c] = bload16(rx, (ch < nch && m < p.M) ? m * ldx_bytes + ch * 16 : kOutOfRange);
  }
  uint32_t sw[C][R];
#pragma unroll
  for (int c = 0; c < C; ++c) {
    const uint32_t ch = ch0 + c * 64;
    const uint32_t t = ch >> 3;
#pragma unroll
    for (int h = 0; h < NQ; ++h) {
      if (ur.quad_ok[h]) {
        const bool ok = ch < nch && ur.rv[4 * h];
        const u32x4 sc = bload16(rs, ok ? static_cast<uint32_t>(scale_word_offset(ur.rows[4 * h], t, p.tiles))
                                        : kOutOfRange);
        sw[c][4 * h + 0] = sc.x;
        sw[c][4 * h + 1] = sc.y;
        sw[c][4 * h + 2] = sc.z;
        sw[c][4 * h + 3] = sc.w;
      } else {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const bool ok = ch < nch && ur.rv[4 * h + j];
          sw[c][4 * h + j] =
              bload4(rs, ok ? static_cast<uint32_t>(scale_word_offset(ur.rows[4 * h + j], t, p.tiles)) : kOutOfRange);
        }
      }
    }
  }
  uint32_t wv[C][R];
#pragma unroll
  for (int c = 0; c < C; ++c) {
    const uint32_t ch = ch0 + c * 64;
#pragma unroll
    for (int i = 0; i < R; ++i)
      wv[c][i] = bload4_nt(rw, (ch < nch && ur.rv[i]) ? static_cast<uint32_t>(ur.rows[i]) * row_bytes + ch * 4
                                                    : kOutOfRange);
  }
  // every load above stays ahead of the arithmetic below
  __builtin_amdgcn_sched_barrier(0);

  const uint32_t shift = 8u * ((lane >> 1) & 3);
  float acc[R][MT];
#pragma unroll
  for (int i = 0; i < R; ++i)
#pragma unroll
    for (int m = 0; m < MT; ++m) acc[i][m] = 0.0f;
#pragma unroll
  for (int c = 0; c < C; ++c) {
#pragma unroll
    for (int i = 0; i < R; ++i) {
      const uint32_t pr[4] = {e2m1x2_bf16<0>(wv[c][i]), e2m1x2_bf16<1>(wv[c][i]), e2m1x2_bf16<2>(wv[c][i]),
                              e2m1x2_bf16<3>(wv[c][i])};
      const float sc = e4m3_to_f32<0>(sw[c][i] >> shift);
#pragma unroll
      for (int m = 0; m < MT; ++m) {
        float a = dot2_bf16(pr[0], xv[m][c].x, 0.0f);
        a = dot2_bf16(pr[1], xv[m][c].y, a);
        a = dot2_bf16(pr[2], xv[m][c].z, a);
        a = dot2_bf16(pr[3], xv[m][c].w, a);
        acc[i][m] = __builtin_fmaf(a, sc, acc[i][m]);
      }
    }
  }

  float v[V];
#pragma unroll
  for (int m = 0; m < MT; ++m)
#pragma unroll
    for (int q = 0; q < 4; ++q)
#pragma unroll
      for (int u = 0; u < P; ++u) v[(m * 4 + q) * P + u] = acc[4 * u + q][m];
  reduce_scatter<V, P>(v);
  if constexpr (KS > 1) {
    __shared__ float red[4][RS::LEFT][64];
    if (kw > 0) {
#pragma unroll
      for (int j = 0; j < RS::LEFT; ++j) red[wave][j][lane] = v[j];
    }
    __syncthreads();
    if (kw == 0) {
#pragma unroll
      for (int s2 = 1; s2 < KS; ++s2)
#pragma unroll
        for (int j = 0; j < RS::LEFT; ++j) v[j] += red[wave + s2][j][lane];
    }
  }
  const int base = reduce_scatter_base<V, P>(lane);
  // the row is computed, not looked up: a lane-dependent index into ur.rows
  // would move the array to LDS
  const int64_t limit = SILU ? p.half : p.N;
#pragma unroll
  for (int j = 0; j < RS::LEFT / P; ++j) {
    const int vi = base + j * P;
    const int m = vi / (4 * P), q = (vi / P) % 4;
    const int64_t qu = PAIR ? 2 * static_cast<int64_t>(unit) : unit;  // (first) quad of the unit
    const int64_t row = (qu >> 5) * 128 + (qu & 31) + 32 * q;
    if (kw == 0 && (lane & 15) == j && m < p.M && unit < p.units && row < limit) {
      if constexpr (PAIR) {
        // N % 16 == 0: row r < N (r even) implies r + 1 < N
        p.out[m * static_cast<int64_t>(p.N) + row] = f32_to_bf16_bits(v[j * P] * gs);
        p.out[m * static_cast<int64_t>(p.N) + row + 1] = f32_to_bf16_bits(v[j * P + 1] * gs);
      } else if constexpr (!SILU) {
        p.out[m * static_cast<int64_t>(p.N) + row] = f32_to_bf16_bits(v[j] * gs);
      } else {
        const float g = bf16_bits_to_f32(f32_to_bf16_bits(v[j * P] * gs));
        const float up = bf16_bits_to_f32(f32_to_bf16_bits(v[j * P + 1] * gs));
        p.out[m * static_cast<int64_t>(p.half) + row] = f32_to_bf16_bits(silu_f32(g) * up);
      }
    }
  }
}

// ------------------------------------------------------------------ 4x4 block MFMA (NVFP4, M <= 8)
// On v_mfma_f32_4x4x4_16b_bf16 (blk_core.hpp), a unit of quads {r, r+32,
// r+64, r+96} streams like the VALU kernel: lane 4b+j loads 16 bytes of row j
// at byte 16b of a 256-byte stretch (one load of the wave reads 256
// contiguous bytes of each of the 4 rows), i.e. 32 codes, k = 512s + 32b ..
// +31 of 512-k segment s.  Those codes are the B operand of 8 MFMAs (4 k
// each) against the A operand of tokens 4g..4g+3 (lane 4b+i: token 4g+i, the
// same 32 k: 64 contiguous activation bytes).  Each MFMA chain covers 16 k,
// one E4M3 block, and is scaled once into the FP32 accumulator, as the VALU
// kernel scales its chunk sums; the 16 blocks are added across lanes at the
// end.  NQ adjacent quads per unit (their scale chunks share cache lines), G
// groups of 4 tokens, C segments per lane, KS waves splitting K.  All loads
// are issued up front.
//
// The end of a dense 4x4 block kernel: acc[a][g] holds, in item i of lane
// 4b+j, block b's partial sum for row j of quad a and token 4g+i.  Sums the
// blocks and waves (blk_reduce; with silu_mul a gate value and its up value
// stay in one lane) and stores the rows (row[q], the lane's row of quad q).
template <int G, int NQ, int KS, bool SILU>
__device__ __forceinline__ void blk_finish(const GemvParams& p, const f32x4 (&acc)[SILU ? 2 * NQ : NQ][G],
                                           const int64_t (&row)[SILU ? 2 * NQ : NQ], const bool (&rv)[SILU ? 2 * NQ : NQ],
                                           float gs, int lane, int wave, int kw) {
  constexpr int P = SILU ? 2 : 1;
  constexpr int V = NQ * G * 4 * P;  // values per lane: v = ((q * G + g) * 4 + i) * P + u
  float v[V];
#pragma unroll
  for (int q = 0; q < NQ; ++q)
#pragma unroll
    for (int g = 0; g < G; ++g)
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int u = 0; u < P; ++u) v[((q * G + g) * 4 + i) * P + u] = acc[u * NQ + q][g][i];
  const int base = blk_reduce<V, KS>(v, lane, wave, kw);
  if (kw == 0 && (lane & 12) == 0) {
#pragma unroll
    for (int j = 0; j < V / 4 / P; ++j) {
      const int t = (base + j * P) / P;
      const int q = t / (4 * G), m = t % (4 * G);
      // the row is selected, not indexed: a lane-dependent index into row[]
      // would move the array to scratch
      int64_t r = row[0];
      bool ok = rv[0];
#pragma unroll
      for (int q2 = 1; q2 < NQ; ++q2)
        if (q == q2) {
          r = row[q2];
          ok = rv[q2];
        }
      if (!ok || m >= p.M) continue;
      if constexpr (!SILU) {
        p.out[m * static_cast<int64_t>(p.N) + r] = f32_to_bf16_bits(v[j] * gs);
      } else {
        const float gv = bf16_bits_to_f32(f32_to_bf16_bits(v[j * P] * gs));
        const float uv = bf16_bits_to_f32(f32_to_bf16_bits(v[j * P + 1] * gs));
        p.out[m * static_cast<int64_t>(p.half) + r] = f32_to_bf16_bits(silu_f32(gv) * uv);
      }
    }
  }
}

template <int G, int NQ, int C, int KS, bool SILU>
__global__ __launch_bounds__(256) void k_gemv_blk(const GemvParams p) {
  constexpr int NA = SILU ? 2 * NQ : NQ;  // quads per unit: NQ (gate) quads, then their up quads
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform, and known to be
  const int kw = wave % KS;
  const int64_t unit = static_cast<int64_t>(xcd_logical_block()) * (4 / KS) + wave / KS;
  const int jr = lane & 3;   // row of the quad (B column) / token of the group (A row)
  const int blk = lane >> 2;  // k range
  const int64_t limit = SILU ? p.half : p.N;
  const uint32_t row_bytes = p.K / 2;
  const uint32_t ldx_bytes = static_cast<uint32_t>(p.ldx) * 2;
  const rsrc_t rw = make_rsrc(p.w, p.w_bytes);
  const rsrc_t rs = make_rsrc(p.s, p.s_bytes);
  const rsrc_t rx = make_rsrc(p.x, p.x_bytes);
  const float gs = *p.gs;

  // This wave's activations: token t (< 4G) of segment c at chunk t * XS + c * 64 of
  // its LDS area, 1 KB per load; XS = 64C + 1 chunks per token, so the 16 lanes
  // of one ds_read_b128 pass (4 tokens, 4 k ranges 64 bytes apart) hit distinct banks.
  // These copies go out before any row arithmetic (measured: 6144x4096 at 4
  // tokens 5.55 -> 5.28 us, 4096x4096 at 8 tokens 5.08 -> 4.99 us).
  constexpr int XS = 64 * C + 1;
  __shared__ u32x4 xl[4][4 * G * XS];
  u32x4* xw = xl[wave];
#pragma unroll
  for (int c = 0; c < C; ++c) {
    const uint32_t ks = static_cast<uint32_t>(kw * C + c) * 512 + 8 * lane;  // this lane's 8 k
#pragma unroll
    for (int t = 0; t < 4 * G; ++t)
      bload16_lds(rx, xw + t * XS + c * 64,
                  off_if(ks < static_cast<uint32_t>(p.K) && t < p.M, static_cast<uint32_t>(t) * ldx_bytes + ks * 2));
  }
  __builtin_amdgcn_sched_barrier(0);  // every load below is issued after these (the wait counts them)

  // this lane's row in each quad of the unit
  int64_t row[NA];
  bool rv[NA];
#pragma unroll
  for (int q = 0; q < NQ; ++q) {
    const int64_t qi = unit * NQ + q;
    row[q] = (qi >> 5) * 128 + (qi & 31) + 32 * jr;
    rv[q] = row[q] < limit && unit < p.units;
    if constexpr (SILU) {
      row[NQ + q] = row[q] + p.half;
      rv[NQ + q] = rv[q];
    }
  }
  uint32_t k0[C];
  bool kv[C];
#pragma unroll
  for (int c = 0; c < C; ++c) {
    k0[c] = static_cast<uint32_t>(kw * C + c) * 512 + 32 * blk;
    kv[c] = k0[c] < static_cast<uint32_t>(p.K);
  }

  __builtin_amdgcn_sched_barrier(0);  // the scale and code loads go out together, after the row arithmetic
  uint32_t sw[C][NA];
#pragma unroll
  for (int c = 0; c < C; ++c)
#pragma unroll
    for (int a = 0; a < NA; ++a)
      sw[c][a] = bload4(rs, off_if(kv[c] && rv[a], static_cast<uint32_t>(scale_word_offset(row[a], k0[c] / 64, p.tiles))));
  u32x4 wv[C][NA];
#pragma unroll
  for (int c = 0; c < C; ++c)
#pragma unroll
    for (int a = 0; a < NA; ++a)
      wv[c][a] = bload16_nt(rw, off_if(kv[c] && rv[a], static_cast<uint32_t>(row[a]) * row_bytes + k0[c] / 2));
  __builtin_amdgcn_sched_barrier(0);

  vm_wait<C * NA * 2>();  // the activation loads (issued first) are in LDS
  u32x4 xv[C][G][4];
#pragma unroll
  for (int c = 0; c < C; ++c)
#pragma unroll
    for (int g = 0; g < G; ++g)
#pragma unroll
      for (int h = 0; h < 4; ++h) xv[c][g][h] = xw[(4 * g + jr) * XS + c * 64 + 4 * blk + h];
  __builtin_amdgcn_sched_barrier(0);  // the LDS reads go out before the wait for the codes

  const uint32_t shift = 16u * (blk & 1);  // scale bytes 2(b%2), 2(b%2)+1 of the word
  f32x4 acc[NA][G];
#pragma unroll
  for (int a = 0; a < NA; ++a)
#pragma unroll
    for (int g = 0; g < G; ++g) acc[a][g] = f32x4{0, 0, 0, 0};
#pragma unroll
  for (int c = 0; c < C; ++c) {
#pragma unroll
    for (int a = 0; a < NA; ++a) {
      u32x2 wb[8];
      blk_codes(wv[c][a], wb);
      const float s0 = e4m3_to_f32<0>(sw[c][a] >> shift);
      const float s1 = e4m3_to_f32<1>(sw[c][a] >> shift);
#pragma unroll
      for (int g = 0; g < G; ++g) blk_mac(wb, xv[c][g], s0, s1, acc[a][g]);
    }
  }

  blk_finish<G, NQ, KS, SILU>(p, acc, row, rv, gs, lane, wave, kw);
}

// The same 4x4 block scheme for BF16 weights (no dequant, no block scales):
// a unit is NQ groups of 4 consecutive rows; lane 4b+j loads 16 bytes of row
// j, k = 128s + 8b .. +7 of 128-k piece s (256 contiguous bytes of each of the
// 4 rows per load), the B operand of 2 MFMAs.  The activations go straight
// into the A operands: lane 4b+i of token group g loads token 4g+i's same 8
// k (one load of the wave reads 256 contiguous bytes of each of 4 token rows),
// so neither K nor the token count is bound by LDS (staging them in LDS, as
// the NVFP4 kernel must, measured up to 1 us slower).  G groups of 4 tokens;
// the KS waves split the pieces.  ONE: a wave's pieces (at most R) are all
// loaded up front and multiplied in order as they arrive; else R pieces per
// round, the next round's weights and activations in flight while the
// current one is multiplied.
template <int G, int NQ, int R, int KS, bool ONE>
__global__ __launch_bounds__(256) void k_gemv_blkh(const GemvParams p) {
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  // wave-uniform, and known to be: the K split's pieces and rounds then stay
  // in scalar registers and scalar branches
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int kw = wave % KS;
  const int64_t unit = static_cast<int64_t>(xcd_logical_block()) * (4 / KS) + wave / KS;
  const int jr = lane & 3;
  const int blk = lane >> 2;
  const uint32_t row_bytes = static_cast<uint32_t>(p.K) * 2;
  const uint32_t ldx_bytes = static_cast<uint32_t>(p.ldx) * 2;
  const rsrc_t rw = make_rsrc(p.w, p.w_bytes);
  const rsrc_t rx = make_rsrc(p.x, p.x_bytes);

  int64_t row[NQ];
  bool rv[NQ];
#pragma unroll
  for (int q = 0; q < NQ; ++q) {
    row[q] = unit * (4 * NQ) + 4 * q + jr;
    rv[q] = row[q] < p.N && unit < p.units;
  }
  const int pieces = (p.K + 127) / 128;
  const int pw = (pieces + KS - 1) / KS;  // pieces per wave
  const int pc0 = kw * pw;                // this wave's first piece
  const int npc = pc0 < pieces ? (pieces - pc0 < pw ? pieces - pc0 : pw) : 0;
  const int rounds = (npc + R - 1) / R;
  const uint32_t k0 = static_cast<uint32_t>(pc0) * 128;
  uint32_t xo[G];
  bool xok[G];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    xo[g] = static_cast<uint32_t>(4 * g + jr) * ldx_bytes;
    xok[g] = 4 * g + jr < p.M;
  }

  auto issue = [&](u32x4 (&w)[R][NQ], u32x4 (&x)[R][G], int r) {
#pragma unroll
    for (int i = 0; i < R; ++i) {
      const int pc = r * R + i;  // piece within the wave
      // K % 16 == 0: the lane's 8 k are all in the row or all past its end
      const uint32_t k = k0 + pc * 128 + 8 * blk;
      const bool ok = pc < npc && k < static_cast<uint32_t>(p.K);
#pragma unroll
      for (int g = 0; g < G; ++g) x[i][g] = bload16(rx, off_if(ok && xok[g], xo[g] + k * 2));
#pragma unroll
      for (int q = 0; q < NQ; ++q)
        w[i][q] = bload16_nt(rw, off_if(ok && rv[q], static_cast<uint32_t>(row[q]) * row_bytes + k * 2));
    }
  };
  f32x4 acc[NQ][G];
#pragma unroll
  for (int q = 0; q < NQ; ++q)
#pragma unroll
    for (int g = 0; g < G; ++g) acc[q][g] = f32x4{0, 0, 0, 0};
  auto compute = [&](const u32x4 (&w)[R][NQ], const u32x4 (&x)[R][G]) {
#pragma unroll
    for (int i = 0; i < R; ++i)
#pragma unroll
      for (int q = 0; q < NQ; ++q)
#pragma unroll
        for (int g = 0; g < G; ++g) {
          acc[q][g] = mfma_4x4x4(u32x2{x[i][g].x, x[i][g].y}, u32x2{w[i][q].x, w[i][q].y}, acc[q][g]);
          acc[q][g] = mfma_4x4x4(u32x2{x[i][g].z, x[i][g].w}, u32x2{w[i][q].z, w[i][q].w}, acc[q][g]);
        }
  };
  if constexpr (ONE) {  // the launcher picks it only when pw <= R
    u32x4 wa[R][NQ], xa[R][G];
    issue(wa, xa, 0);
    __builtin_amdgcn_sched_barrier(0);  // every load before any product
    compute(wa, xa);
  } else {
    u32x4 wa[R][NQ], xa[R][G], wb[R][NQ], xb[R][G];
    // more than 8 pieces per wave in this form, so every wave has a round:
    // no test ahead of the first loads (4096x14336 at 8 tokens 23.9 -> 22.9 us)
    issue(wa, xa, 0);
    int r = 0;
    do {
      if (r + 1 < rounds) issue(wb, xb, r + 1);
      compute(wa, xa);
      if (r + 1 >= rounds) break;
      if (r + 2 < rounds) issue(wa, xa, r + 2);
      compute(wb, xb);
      r += 2;
    } while (r < rounds);
  }
  blk_finish<G, NQ, KS, false>(p, acc, row, rv, 1.0f, lane, wave, kw);
}

// ------------------------------------------------------------------ MFMA
// Swap-AB MFMA path.  A row tile is 16 weight rows, the A operand of
// v_mfma_f32_16x16x32_bf16; the B operand holds up to 16 tokens (two token
// tiles for M > 16).  NVFP4 tile rows are {band*128 + 4q + (r&3) + 32(r>>2)}
// (q = tile % 8): their scale words for a 64-k tile are 64 contiguous bytes.
// BF16 tile rows are 16 consecutive rows.
//
// A workgroup takes RT row tiles (plus the matching up tiles with silu_mul);
// its mfma_waves(XT) waves split K into contiguous slices and meet in LDS at the
// end.  A step is 128 k and feeds 4 MFMAs per A operand and token tile.
// NVFP4: lane (r, g) loads 32 codes of row r, k = 32g .. 32g+31, in one
// 16-byte load; fragment j is k = 32g+8j .. +7.  BF16: lane (r, g) makes four
// 16-byte loads, fragment j = k 32j+8g .. +7, so that every load of the wave
// reads 64 contiguous bytes of each of its 16 rows.  Each wave keeps D steps in flight in a ring: while the
// ring has later steps to fetch, every slot is refilled as soon as it is
// consumed, so each wait is the same in-order count; the last round drains
// the ring without refilling it.
//
// Activations are staged through the ring in LDS.  Every workgroup reads all
// M*K*2 activation bytes, so at M >= 8 they are most of the bytes that reach
// a compute unit.  Loaded straight into B fragments, a 1 KB load would touch
// 16 token rows and 32 cache lines.  Here each 16-byte load goes straight
// into LDS and covers whole token segments of one step (4 tokens x 256
// bytes), and the fragments are then read with ds_read_b128.  Chunk c of a token's segment sits at position c ^ swz(token),
// so the 8 or 16 lanes that a fragment read serves in one LDS pass hit
// distinct banks.
constexpr int mfma_waves(int /*XT*/) { return 4; }

// Steps in flight per wave, measured: 4 up to 16 staged tokens (2 at 16 for
// BF16, whose four weight loads per step already keep 4 KB per wave in
// flight), 2 at 32 (a 128 KB ring would leave one workgroup per CU) and at 64
// (deeper rings were slower).  Bounded by vmcnt, which counts at most 63 outstanding loads, and by
// the LDS ring (128 KB per workgroup).  A depth that divides the steps of a
// wave wastes nothing in the last round; K = 4096 gives 8 steps per wave.
constexpr int mfma_depth_of(bool fp4, int xt, int na, int w) {
  const int per = fp4 ? 2 : 4;                   // loads per A operand and step
  const int cpt = 16;                            // 16-byte chunks per token and step
  const int load_x = xt * cpt / 64;              // staging loads per step
  int d = (xt >= 32 || (!fp4 && xt >= 16)) ? 2 : 4;
  while (d > 2 && (na * per + (d - 1) * (load_x + na * per) > 62 || w * d * xt * cpt * 16 > 128 * 1024)) d /= 2;
  return d;
}

template <bool FP4, int XT, int NA, int W>
constexpr int mfma_depth() { return mfma_depth_of(FP4, XT, NA, W); }

// Whether the MFMA kernel with na A operands per step fits a compute unit:
// the loads a full ring keeps in flight within vmcnt's count, and the ring
// plus the cross-wave partial sums within the 160 KB of LDS.
constexpr bool mfma_fits(bool fp4, int xt, int na) {
  const int w = mfma_waves(xt);
  const int d = mfma_depth_of(fp4, xt, na, w);
  const int per = fp4 ? 2 : 4;
  const int l = xt * 16 / 64 + na * per;
  const int nt = (xt + 15) / 16;
  return na * per + (d - 1) * l <= 62 && d * w * xt * 256 + (w - 1) * na * nt * 64 * 16 <= 160 * 1024;
}

// XT: token rows staged per step (4, 8, 16, 32 or 64).  With XT < 16 the fragment
// lanes of tokens XT..15 read the rows of tokens 0..XT-1 again: those MFMA
// columns are never stored.
//
// S > 1: cross-workgroup split-K.  Every workgroup streams all M*K*2 bytes
// of activations for its K range, so from 16 tokens on the activation bytes
// that reach the compute units exceed the weight bytes several times.  With
// S splits, S workgroups share a unit of RT row tiles, each taking 1/S of
// K, so the activation stream per workgroup shrinks S-fold for the same
// weight bytes.  Items are numbered split-major: the workgroups of one XCD
// share a K range (and its activations in their L2).  Each workgroup
// writes its FP32 partial sums to the workspace, and the last of the S to
// arrive at the unit's counter adds the S partials in split order (the same
// sum whatever the arrival order), applies the epilogue and clears the
// counter for the next call.
//
// Hand-off.  The partial sums are written and read with device-coherent
// (sc1) buffer accesses, which is how the compiler implements relaxed
// device-scope atomic loads and stores: they do not stop in an XCD's L2.
// A writer waits for its stores (vmcnt 0) before its counter increment, and
// the last arriver issues its loads only after the increment has returned,
// so it reads every other split's sums.  A __threadfence() here would write
// back and invalidate the whole L2 of the XCD on every arrival, which
// measured 2-4x slower than the call without a split.
constexpr int kCoherent = 16;  // cache policy bit sc1 of the buffer intrinsics

__device__ __forceinline__ void store16_coherent(rsrc_t r, uint32_t off, const f32x4& v) {
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), r, static_cast<int>(off), 0, kCoherent);
}
__device__ __forceinline__ f32x4 load16_coherent(rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(r, static_cast<int>(off), 0, kCoherent));
}

template <bool FP4, int XT, bool SILU, int RT, int S>
__global__ __launch_bounds__(mfma_waves(XT) * 64) void k_gemv_mfma(const GemvParams p) {
  constexpr int NT = (XT + 15) / 16;        // token tiles (B operands)
  constexpr int NA = (SILU ? 2 : 1) * RT;   // A operands per step: RT row tiles (x gate, up)
  constexpr int KSTEP = 128;                // k per step
  constexpr int NJ = 4;                     // MFMAs per step per A operand and token tile
  constexpr int W = mfma_waves(XT);
  constexpr int D = mfma_depth<FP4, XT, NA, W>();  // steps in flight per wave
  constexpr int CPT = KSTEP * 2 / 16;       // 16-byte activation chunks per token and step
  constexpr int LX = XT * CPT / 64;         // staging loads per step
  static_assert(XT * CPT % 64 == 0, "a staging load covers whole token segments");
  constexpr int PER = FP4 ? 2 : 4;          // weight-side loads per A operand and step
  constexpr int WL = FP4 ? 1 : 4;           // 16-byte weight loads per A operand and step
  constexpr int L = LX + NA * PER;          // loads per step
  // loads issued after a step's staging loads while it is the oldest in a full ring
  constexpr int FULL_AFTER = NA * PER + (D - 1) * L;
  __shared__ f32x4 red[W - 1][NA][NT][64];
  constexpr int SLOT = XT * CPT;             // ring chunks per wave and step
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int r = lane & 15;
  const int g = lane >> 4;
  const int64_t limit = SILU ? p.half : p.N;
  const uint32_t row_bytes = FP4 ? p.K / 2 : static_cast<uint32_t>(p.K) * 2;
  const int64_t steps_total = (p.K + KSTEP - 1) / KSTEP;
  const int64_t sps = S == 1 ? steps_total : (steps_total + S - 1) / S;  // steps per split
  const int64_t spw = (sps + W - 1) / W;               // steps per wave
  static_assert((W & (W - 1)) == 0, "the slice rotation below needs a power-of-two wave count");
  const rsrc_t rw = make_rsrc(p.w, p.w_bytes);
  const rsrc_t rs = make_rsrc(p.s, p.s_bytes);
  const rsrc_t rx = make_rsrc(p.x, p.x_bytes);
  const float gs = FP4 ? *p.gs : 1.0f;

  // Staging load i of a step: this lane fetches chunk skc[i] / 8 of token
  // i * (64 / CPT) + lane / CPT into ring position lane % CPT of that token.
  uint32_t sxo[LX], skc[LX];
#pragma unroll
  for (int i = 0; i < LX; ++i) {
    const int t = i * (64 / CPT) + lane / CPT;
    skc[i] = static_cast<uint32_t>(xl_pos<CPT>(t, lane % CPT)) * 8;  // the XOR is its own inverse
    sxo[i] = t < p.M ? static_cast<uint32_t>(t) * static_cast<uint32_t>(p.ldx) * 2 : kOutOfRange;
  }

  // The grid never exceeds the items, so the first item is taken without a
  // test: a loop test ahead of the body held the first loads behind another
  // wait for kernel arguments (4096x4096 at 16 tokens 6.26 -> 6.15 us).
  int64_t item = xcd_logical_block();
  do {
    const int64_t split = S == 1 ? 0 : item / p.units;
    const int64_t tile = S == 1 ? item : item - split * p.units;  // the unit of RT row tiles
    const int64_t s_first = split * sps;                          // this split's steps
    const int64_t s_count = s_first < steps_total ? (steps_total - s_first < sps ? steps_total - s_first : sps) : 0;
    // This wave's K slice.  From 8 staged tokens on, the slices rotate with
    // the tile, so that the workgroups of one die do not all stream the same
    // activation slice at the same time (measured 2-6% faster at 8..32 tokens,
    // and slower at 4).
    const int slice = XT >= 8 ? (wave + static_cast<int>(tile & (W - 1))) & (W - 1) : wave;
    const int64_t w0 = slice * spw;
    const int64_t st0 = s_first + w0;
    const int64_t nst = w0 < s_count ? (s_count - w0 < spw ? s_count - w0 : spw) : 0;
    // A operand a: row tile tile*RT + a % RT, the up half for a >= RT
    int64_t rows[NA];
    bool rv[NA];
#pragma unroll
    for (int a = 0; a < RT; ++a) {
      rows[a] = mfma_row<FP4>(tile * RT + a, r);
      rv[a] = rows[a] < limit;
      if constexpr (SILU) {
        rows[RT + a] = rows[a] + p.half;
        rv[RT + a] = rv[a];
      }
    }
    u32x4 wb[D][NA][WL];
    uint32_t sb[D][NA];
    auto issue = [&](int d, int64_t st) {
      const bool sv = st < nst;
      const uint32_t kb = static_cast<uint32_t>((st0 + st) * KSTEP);  // first k of the step
#pragma unroll
      for (int i = 0; i < LX; ++i) {
        const uint32_t k = kb + skc[i];
        bload16_lds(rx, xl_slot<W * SLOT>(d) + wave * SLOT + i * 64,
                    off_if(sv && k < static_cast<uint32_t>(p.K), sxo[i] + k * 2));
      }
      // The waits below count the loads issued after a slot's staging loads:
      // the scheduler keeps each step's staging loads, then its weight loads,
      // in the order written.
      __builtin_amdgcn_sched_barrier(0);
      const uint32_t k = kb + (FP4 ? g * 32 : g * 8);
      const bool kv = sv && k < static_cast<uint32_t>(p.K);
#pragma unroll
      for (int a = 0; a < NA; ++a) {
        const bool ok = rv[a] && kv;  // (a select here measured faster than off_if)
        if constexpr (FP4) {
          // K % 64 == 0: the lane's 32 codes are all in range or all out
          // (streaming scale loads measured 0.1-0.17 us faster at 4..32
          // tokens without silu_mul, slower with it)
          const uint32_t so = ok ? static_cast<uint32_t>(scale_word_offset(rows[a], k / 64, p.tiles)) : kOutOfRange;
          sb[d][a] = SILU ? bload4(rs, so) : bload4_nt(rs, so);
          wb[d][a][0] = bload16_nt(rw, ok ? static_cast<uint32_t>(rows[a]) * row_bytes + k / 2 : kOutOfRange);
        } else {
          // load j: 8 weights at k + 32j (each load of the wave reads 64
          // contiguous bytes of 16 rows); K % 16 == 0, so each 8-weight
          // fragment is in range or out as a whole
          sb[d][a] = 0;
#pragma unroll
          for (int j = 0; j < WL; ++j) {
            const bool okj = rv[a] && sv && k + 32 * j < static_cast<uint32_t>(p.K);
            wb[d][a][j] = bload16_nt(rw, okj ? static_cast<uint32_t>(rows[a]) * row_bytes + (k + 32 * j) * 2 : kOutOfRange);
          }
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    };
#pragma unroll
    for (int d = 0; d < D; ++d) issue(d, d);
    __builtin_amdgcn_sched_barrier(0);  // all D steps in flight before any arithmetic

    f32x4 acc[NA][NT];
#pragma unroll
    for (int a = 0; a < NA; ++a)
#pragma unroll
      for (int n = 0; n < NT; ++n) acc[a][n] = f32x4{0, 0, 0, 0};

    // Slot d of the ring holds step base + d.  `after` = loads issued after
    // the slot's staging loads (a compile-time count once d is unrolled).
    auto consume = [&](int d, int after) {
      u32x4 xf[NJ][NT];
      vm_wait_n(after);
#pragma unroll
      for (int j = 0; j < NJ; ++j)
#pragma unroll
        for (int n = 0; n < NT; ++n) {
          const int t = (16 * n + r) & (XT - 1);
          xf[j][n] = xl_slot<W * SLOT>(d)[wave * SLOT + t * CPT + xl_pos<CPT>(t, FP4 ? 4 * g + j : 4 * j + g)];
        }
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
#pragma unroll
        for (int a = 0; a < NA; ++a) {
          bf16x8 av;
          if constexpr (FP4) {
            av = fp4_a_fragment(wb[d][a][0], sb[d][a], g, j);
          } else {
            av = __builtin_bit_cast(bf16x8, wb[d][a][j]);
          }
#pragma unroll
          for (int n = 0; n < NT; ++n)
            acc[a][n] = mfma_16x16x32(av, xf[j][n], acc[a][n]);
        }
      }
    };

    // Rounds that have steps after them: consume each slot, then refill it
    // with the step D later (the ring stays full, so the wait is the same
    // for every slot).
    int64_t base = 0;
    for (; base + D < nst; base += D) {
#pragma unroll
      for (int d = 0; d < D; ++d) {
        consume(d, FULL_AFTER);
        lds_wait();  // the slot's fragment reads retire before it is refilled
        issue(d, base + d + D);
      }
    }
    // The last round drains the ring without refilling it (no loads past the
    // wave's share).  It runs even for a wave without steps: its waits retire
    // every load into LDS before the slots are reused or the wave ends.
#pragma unroll
    for (int d = 0; d < D; ++d) consume(d, NA * PER + (D - 1 - d) * L);

    // The W K slices meet in LDS; wave 0 adds them in slice order and writes.
    if (wave > 0) {
#pragma unroll
      for (int a = 0; a < NA; ++a)
#pragma unroll
        for (int n = 0; n < NT; ++n) red[wave - 1][a][n][lane] = acc[a][n];
    }
    __syncthreads();
    if (wave == 0) {
#pragma unroll
      for (int w = 0; w < W - 1; ++w)
#pragma unroll
        for (int a = 0; a < NA; ++a)
#pragma unroll
          for (int n = 0; n < NT; ++n) acc[a][n] += red[w][a][n][lane];
      bool last = true;
      if constexpr (S > 1) {
        // publish this split's partial sums, then count the arrival.  The
        // partials of (unit, split) are NA * NT * 64 f32x4, lane-minor.
        const rsrc_t rp = make_rsrc(p.part, p.part_bytes);
        auto part_off = [&](int64_t s2, int a, int n) {
          return static_cast<uint32_t>((((tile * S + s2) * NA + a) * NT + n) * 64 + lane) * 16u;
        };
#pragma unroll
        for (int a = 0; a < NA; ++a)
#pragma unroll
          for (int n = 0; n < NT; ++n) store16_coherent(rp, part_off(split, a, n), acc[a][n]);
        vm_wait<0>();  // the partial sums are visible device-wide before the count
        uint32_t before = 0;
        if (lane == 0) before = atomicAdd(p.cnt + tile, 1u);
        last = __builtin_amdgcn_readfirstlane(before) == S - 1;
        asm volatile("" ::: "memory");  // the loads below stay after the count
        if (last) {
          // the S partials in split order (this workgroup's own from registers)
#pragma unroll
          for (int a = 0; a < NA; ++a)
#pragma unroll
            for (int n = 0; n < NT; ++n) {
              f32x4 t = split == 0 ? acc[a][n] : load16_coherent(rp, part_off(0, a, n));
#pragma unroll
              for (int s2 = 1; s2 < S; ++s2) t += s2 == split ? acc[a][n] : load16_coherent(rp, part_off(s2, a, n));
              acc[a][n] = t;
            }
          if (lane == 0) __hip_atomic_store(p.cnt + tile, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
      }
      if (last) {
        // C layout: lane holds rows 4(l/16)+i of the tile, token column l%16
#pragma unroll
        for (int a = 0; a < RT; ++a) {
#pragma unroll
          for (int n = 0; n < NT; ++n) {
            const int m = 16 * n + (lane & 15);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const int64_t row = mfma_row<FP4>(tile * RT + a, 4 * (lane >> 4) + i);
              if (m >= p.M || row >= limit) continue;
              if constexpr (!SILU) {
                p.out[m * static_cast<int64_t>(p.N) + row] = f32_to_bf16_bits(acc[a][n][i] * gs);
              } else {
                const float gv = bf16_bits_to_f32(f32_to_bf16_bits(acc[a][n][i] * gs));
                const float uv = bf16_bits_to_f32(f32_to_bf16_bits(acc[RT + a][n][i] * gs));
                p.out[m * static_cast<int64_t>(p.half) + row] = f32_to_bf16_bits(silu_f32(gv) * uv);
              }
            }
          }
        }
      }
    }
    __syncthreads();
    item += gridDim.x;
  } while (item < p.units * S);
}

// ------------------------------------------------------------------ MFMA, block-diagonal (NVFP4, M <= 8)
// For row counts whose 16-row tiles outnumber the compute units without
// filling a second round (e.g. 6144 rows: 384 tiles on 256 units, where half
// the units did two tiles or, with two tiles per workgroup, a quarter of the
// units idled), this form gives each workgroup 24 consecutive rows (6144
// rows: 256 workgroups, one per unit).
// With TK <= 8 tokens, the swap-AB MFMA's 16 B columns would carry 16 - TK
// copies; here they carry a K split into KC = 16 / TK chunks instead:
//
//   A row    i = KC rho + c   row rho (0..TK-1) of a TK-row group, k chunk c
//   B column j = KC n + c'    token n (0..TK-1), k chunk c'
//
// Lane (i, g) loads the 32 codes k = S + 128c + 32g .. +31 of its row (S =
// first k of a super-step of 128 KC k), so the 4 KC lanes of a row read
// 64 KC contiguous bytes (256 for 4 tokens, 128 for 8) in one load; MFMA f
// (0..3) takes fragment f of those codes, k = S + 128c + 32g + 8f .. +7,
// against token n's k = S + 128c' + 32g + 8f .. +7.  The products with c = c'
// (the diagonal blocks) are the wanted ones.  Lane (col, g') of the C
// fragment holds rows i = 4g' + q; its diagonal entries are q = c' + KC u
// (u < 4 / KC), i.e. group rows 4g' / KC + u, and the KC lanes col % KC add
// theirs over the k chunks.  The activations (4 KB per super-step: TK
// tokens x 128 KC k) arrive by 4 loads straight into an LDS ring, token n's
// chunk ch at position ch ^ ((KC n + ch / 16) & 15), so the 16 lanes of one
// B-fragment read hit 16 distinct bank groups.  The 4 waves split K and meet
// in LDS.
constexpr int kBdWaves = 4;

template <int KC>
__device__ __forceinline__ int bd_pos(int n, int ch) { return ch ^ ((KC * n + (ch >> 4)) & 15); }

template <bool SILU, int TK, int R>
__global__ __launch_bounds__(kBdWaves * 64) void k_gemv_mfma_bd(const GemvParams p) {
  static_assert(TK == 4 || TK == 8, "4 or 8 tokens");
  static_assert(R % TK == 0, "whole groups per workgroup");
  constexpr int KC = 16 / TK;          // k chunks of the K split
  constexpr int G = R / TK;            // TK-row groups per workgroup (R rows)
  constexpr int W = kBdWaves;
  constexpr int D = 2;                 // super-steps in flight per wave
  constexpr int NG = SILU ? 2 * G : G; // groups (gate, then up)
  constexpr int SSK = 128 * KC;        // k per super-step
  constexpr int SEG = 16 * KC;         // ring chunks (16 B) per token and super-step
  constexpr int SLOT = TK * SEG;       // ring chunks per wave and super-step (256)
  constexpr int LX = SLOT / 64;        // staging loads per super-step (4)
  constexpr int PER = 2;               // loads per group and super-step: scale word, codes
  constexpr int L = LX + NG * PER;
  constexpr int FULL_AFTER = NG * PER + (D - 1) * L;
  static_assert(FULL_AFTER <= 62, "vmcnt waits count at most 62 loads");
  __shared__ f32x4 red[W - 1][NG][64];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 4;
  const int rho = (lane & 15) / KC;    // A: row of the group; B: token n
  const int c = lane % KC;             // A: k chunk c; B: k chunk c'
  const int64_t limit = SILU ? p.half : p.N;
  const uint32_t row_bytes = p.K / 2;
  const int64_t ss_total = (p.K + SSK - 1) / SSK;
  const int64_t spw = (ss_total + W - 1) / W;
  const int64_t st0 = wave * spw;
  const int64_t nst = st0 < ss_total ? (ss_total - st0 < spw ? ss_total - st0 : spw) : 0;
  const rsrc_t rw = make_rsrc(p.w, p.w_bytes);
  const rsrc_t rs = make_rsrc(p.s, p.s_bytes);
  const rsrc_t rx = make_rsrc(p.x, p.x_bytes);
  const float gs = *p.gs;

  // staging load q: ring positions 64 q + lane, i.e. token (64 q + lane) / SEG
  // and the chunk stored at that position
  uint32_t sxo[LX], sch[LX];
#pragma unroll
  for (int q = 0; q < LX; ++q) {
    const int n = (64 * q + lane) / SEG;
    sch[q] = static_cast<uint32_t>(bd_pos<KC>(n, (64 * q + lane) % SEG));  // bd_pos is its own inverse
    sxo[q] = n < p.M ? static_cast<uint32_t>(n) * static_cast<uint32_t>(p.ldx) * 2 : kOutOfRange;
  }

  {  // the grid is exactly one workgroup per unit (no test ahead of the first loads)
    const int64_t unit = xcd_logical_block();
    int64_t rows[NG];
    bool rv[NG];
#pragma unroll
    for (int a = 0; a < G; ++a) {
      rows[a] = unit * R + TK * a + rho;
      rv[a] = rows[a] < limit;
      if constexpr (SILU) {
        rows[G + a] = rows[a] + p.half;
        rv[G + a] = rv[a];
      }
    }
    u32x4 wb[D][NG];
    uint32_t sb[D][NG];
    auto issue = [&](int d, int64_t st) {
      const bool sv = st < nst;
      const uint32_t kb = static_cast<uint32_t>((st0 + st) * SSK);
#pragma unroll
      for (int q = 0; q < LX; ++q) {
        const uint32_t k = kb + sch[q] * 8;
        bload16_lds(rx, xl_slot<W * SLOT>(d) + wave * SLOT + q * 64,
                    off_if(sv && k < static_cast<uint32_t>(p.K), sxo[q] + k * 2));
      }
      // staging loads, then weight loads, in the order the waits count them
      __builtin_amdgcn_sched_barrier(0);
      // K % 64 == 0: the lane's 32 codes are all in range or all out
      const uint32_t k = kb + 128 * c + 32 * g;
      const bool kv = sv && k < static_cast<uint32_t>(p.K);
#pragma unroll
      for (int a = 0; a < NG; ++a) {
        const bool ok = rv[a] && kv;
        sb[d][a] = bload4(rs, ok ? static_cast<uint32_t>(scale_word_offset(rows[a], k / 64, p.tiles)) : kOutOfRange);
        wb[d][a] = bload16_nt(rw, ok ? static_cast<uint32_t>(rows[a]) * row_bytes + k / 2 : kOutOfRange);
      }
      __builtin_amdgcn_sched_barrier(0);
    };
#pragma unroll
    for (int d = 0; d < D; ++d) issue(d, d);
    __builtin_amdgcn_sched_barrier(0);

    f32x4 acc[NG];
#pragma unroll
    for (int a = 0; a < NG; ++a) acc[a] = f32x4{0, 0, 0, 0};

    auto consume = [&](int d, int after) {
      u32x4 xf[4];
      vm_wait_n(after);
#pragma unroll
      for (int f = 0; f < 4; ++f)
        xf[f] = xl_slot<W * SLOT>(d)[wave * SLOT + rho * SEG + bd_pos<KC>(rho, 16 * c + 4 * g + f)];
#pragma unroll
      for (int f = 0; f < 4; ++f)
#pragma unroll
        for (int a = 0; a < NG; ++a)
          acc[a] = mfma_16x16x32(fp4_a_fragment(wb[d][a], sb[d][a], g, f), xf[f], acc[a]);
    };

    int64_t base = 0;
    for (; base + D < nst; base += D) {
#pragma unroll
      for (int d = 0; d < D; ++d) {
        consume(d, FULL_AFTER);
        lds_wait();
        issue(d, base + d + D);
      }
    }
#pragma unroll
    for (int d = 0; d < D; ++d) consume(d, NG * PER + (D - 1 - d) * L);

    if (wave > 0) {
#pragma unroll
      for (int a = 0; a < NG; ++a) red[wave - 1][a][lane] = acc[a];
    }
    __syncthreads();
    if (wave == 0) {
      constexpr int U = 4 / KC;        // diagonal entries per lane
      float v[NG][U];
#pragma unroll
      for (int a = 0; a < NG; ++a) {
#pragma unroll
        for (int w = 0; w < W - 1; ++w) acc[a] += red[w][a][lane];
#pragma unroll
        for (int u = 0; u < U; ++u) {
          // component q = c' + KC u (c == c'), then the sum over the KC k chunks
          const int q = c + KC * u;
          float e = q == 0 ? acc[a][0] : q == 1 ? acc[a][1] : q == 2 ? acc[a][2] : acc[a][3];
#pragma unroll
          for (int sh = 1; sh < KC; sh <<= 1) e += __shfl_xor(e, sh);
          v[a][u] = e;
        }
      }
      const int n = rho;               // C column KC n + c'
      if (c == 0 && n < p.M) {
#pragma unroll
        for (int a = 0; a < G; ++a)
#pragma unroll
          for (int u = 0; u < U; ++u) {
            const int64_t row = unit * R + TK * a + (4 / KC) * g + u;  // C rows 4g' + q
            if (row >= limit) continue;
            if constexpr (!SILU) {
              p.out[n * static_cast<int64_t>(p.N) + row] = f32_to_bf16_bits(v[a][u] * gs);
            } else {
              const float gv = bf16_bits_to_f32(f32_to_bf16_bits(v[a][u] * gs));
              const float uv = bf16_bits_to_f32(f32_to_bf16_bits(v[G + a][u] * gs));
              p.out[n * static_cast<int64_t>(p.half) + row] = f32_to_bf16_bits(silu_f32(gv) * uv);
            }
          }
      }
    }
    __syncthreads();
  }
}

// ------------------------------------------------------------------ launch
namespace {

// When set, the launchers below write the name of the kernel they would
// launch here and launch nothing (describe_gemv).
thread_local char* t_describe = nullptr;
thread_local size_t t_describe_len = 0;

const char* tf(bool v) { return v ? "true" : "false"; }

int lanes_per_unit(int64_t tiles) {
  if (tiles > 32) return 64;
  if (tiles > 16) return 32;
  if (tiles > 8) return 16;
  return 8;
}

template <bool FP4, int MT, bool SILU, int LPQ>
hipError_t launch_valu_lpq(const GemvParams& p, hipStream_t stream) {
  const int64_t g = kWave / LPQ;
  const int64_t waves = (p.units + g - 1) / g;
  int64_t blocks = (waves + 3) / 4;
  if (blocks > 1024) blocks = 1024;
  const dim3 grid(static_cast<unsigned>(blocks)), block(256);
  if (t_describe) {
    if (p.tiles <= LPQ) std::snprintf(t_describe, t_describe_len, "k_gemv_valu1<%s, %d, %d, %s>", tf(FP4), MT, LPQ, tf(SILU));
    else std::snprintf(t_describe, t_describe_len, "k_gemv_valu<%s, %d, %d, %s, false>", tf(FP4), MT, LPQ, tf(SILU));
    return hipSuccess;
  }
  if (p.tiles <= LPQ) {  // one tile per lane: one unit per wave-slot, straight-line kernel
    const dim3 grid1(static_cast<unsigned>((waves + 3) / 4));
    hipLaunchKernelGGL((k_gemv_valu1<FP4, MT, LPQ, SILU>), grid1, block, 0, stream, p);
  } else {
    const size_t lds = static_cast<size_t>(p.M) * ((p.K + 63) / 64 * 64) * 2 + 16;  // + spare chunk
    hipLaunchKernelGGL((k_gemv_valu<FP4, MT, LPQ, SILU, false>), grid, block, lds, stream, p);
  }
  return hipGetLastError();
}

// Pair units (two adjacent quads) for one or two tokens without silu_mul
// (measured: 4096 x 4096 at 1 / 2 tokens 4.41 / 5.08 -> 4.17 / 4.80 us).
constexpr bool kVchunkPairs = true;

template <int MT, bool SILU, int C, int KS>
hipError_t launch_vchunk_c(GemvParams p, hipStream_t stream) {
  constexpr int upb = 4 / KS;
  constexpr bool PAIR = kVchunkPairs && !SILU && MT <= 2;
  if constexpr (PAIR) p.units = (p.units + 1) / 2;  // quads come 32 to a band, so this is exact
  if (t_describe) {
    std::snprintf(t_describe, t_describe_len, "k_gemv_vchunk<%d, %s, %d, %d, %s>", MT, tf(SILU), C, KS, tf(PAIR));
    return hipSuccess;
  }
  const dim3 grid(static_cast<unsigned>((p.units + upb - 1) / upb)), block(256);
  hipLaunchKernelGGL((k_gemv_vchunk<MT, SILU, C, KS, PAIR>), grid, block, 0, stream, p);
  return hipGetLastError();
}

// Largest M the NVFP4 GEMV sends to the VALU path by default.  The MFMA
// path costs about the same for every M up to 8 (weight stream and dequant),
// and from M = 3 it is the faster one.
constexpr int64_t kValuMaxMFp4 = 2;

// The 4x4 block MFMA kernel: rows of up to two 512-k segments per lane and
// 4 waves (K <= 4096), up to 8 tokens (two groups of 4).
constexpr int64_t kBlkMaxK = 4096;
constexpr int64_t kBlkMaxM = 8;
constexpr int64_t kBlkhMaxM = 8;  // BF16 weights: two groups of 4 tokens

// NVFP4 rows of at most kVchunkMaxK columns: 8-k chunks, at most 8 per lane
// and 4 waves per unit.
constexpr int64_t kVchunkMaxK = 64 * 8 * 8 * 4;

template <int MT, bool SILU, int KS>
hipError_t launch_vchunk_ks(const GemvParams& p, hipStream_t stream) {
  const int64_t per_lane = (p.K / 8 + 64 * KS - 1) / (64 * KS);
  if (per_lane <= 1) return launch_vchunk_c<MT, SILU, 1, KS>(p, stream);
  if (per_lane <= 2) return launch_vchunk_c<MT, SILU, 2, KS>(p, stream);
  if (per_lane <= 4) return launch_vchunk_c<MT, SILU, 4, KS>(p, stream);
  return launch_vchunk_c<MT, SILU, 8, KS>(p, stream);
}

// Waves per unit: four for one or two tokens, two for four tokens (whose
// activation registers would otherwise crowd out the loads in flight), fewer
// when K has too few 8-k chunks to give every lane of every wave one, more
// when a lane would need more than 8 chunks.
int vchunk_ks(int MT, int64_t K) {
  const int64_t chunks = K / 8;
  int ks = MT <= 2 ? 4 : 2;
  while (ks > 1 && 64 * ks > chunks) ks /= 2;
  while (ks < 4 && chunks > 512 * ks) ks *= 2;
  return ks;
}

template <int MT, bool SILU>
hipError_t launch_vchunk(const GemvParams& p, hipStream_t stream) {
  switch (vchunk_ks(MT, p.K)) {
    case 1: return launch_vchunk_ks<MT, SILU, 1>(p, stream);
    case 2: return launch_vchunk_ks<MT, SILU, 2>(p, stream);
    default: return launch_vchunk_ks<MT, SILU, 4>(p, stream);
  }
}

template <bool FP4, int MT, bool SILU>
hipError_t launch_valu(const GemvParams& p, int lpq, hipStream_t stream) {
  switch (lpq) {
    case 64: return launch_valu_lpq<FP4, MT, SILU, 64>(p, stream);
    case 32: return launch_valu_lpq<FP4, MT, SILU, 32>(p, stream);
    case 16: return launch_valu_lpq<FP4, MT, SILU, 16>(p, stream);
    default: return launch_valu_lpq<FP4, MT, SILU, 8>(p, stream);
  }
}

template <bool FP4, int XT, bool SILU, int RT, int S = 1>
hipError_t launch_mfma_rt(GemvParams p, hipStream_t stream) {
  const int64_t limit = SILU ? p.half : p.N;
  const int64_t tiles = FP4 ? ((limit + 127) / 128) * 8 : (limit + 15) / 16;
  p.units = (tiles + RT - 1) / RT;
  if (t_describe) {
    std::snprintf(t_describe, t_describe_len, "k_gemv_mfma<%s, %d, %s, %d, %d>", tf(FP4), XT, tf(SILU), RT, S);
    return hipSuccess;
  }
  int64_t blocks = p.units * S;
  if (blocks > 65536) blocks = 65536;  // never more than the items (the kernel relies on it)
  hipLaunchKernelGGL((k_gemv_mfma<FP4, XT, SILU, RT, S>), dim3(static_cast<unsigned>(blocks)),
                     dim3(mfma_waves(XT) * 64), 0, stream, p);
  return hipGetLastError();
}

// Compute units of the current device (queried once per device).
int device_cu_count() {
  constexpr int kMaxDevices = 64;
  static std::atomic<int> cached[kMaxDevices] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return 256;
  int n = cached[dev].load(std::memory_order_relaxed);
  if (n == 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    cached[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}

// The block-diagonal form with R-row units where the 16-row tiles outnumber
// the compute units but the R-row units do not (measured: 24 rows at 6144
// rows for 1..8 tokens; 56 rows at 14336 rows for 5..8 tokens, where at 4
// tokens it was slower than the 16-row tiles).
template <bool SILU, int TK, int R>
bool launch_mfma_bd(GemvParams p, hipStream_t stream, hipError_t* err) {
  const int64_t limit = SILU ? p.half : p.N;
  const int64_t tiles16 = (limit + 15) / 16;
  const int64_t units = (limit + R - 1) / R;
  const int cus = device_cu_count();
  if (!(tiles16 > cus && units <= cus)) return false;
  p.units = units;
  if (t_describe) {
    std::snprintf(t_describe, t_describe_len, "k_gemv_mfma_bd<%s, %d, %d>", tf(SILU), TK, R);
    *err = hipSuccess;
    return true;
  }
  // exactly one workgroup per unit: the kernel relies on it
  hipLaunchKernelGGL((k_gemv_mfma_bd<SILU, TK, R>), dim3(static_cast<unsigned>(units)), dim3(kBdWaves * 64), 0,
                     stream, p);
  *err = hipGetLastError();
  return true;
}

// Row tiles per workgroup.  One tile per workgroup while the tiles fit the
// compute units in one round; beyond that, two tiles share every activation
// fragment (half the activation traffic through L2) and the grid keeps one
// round instead of leaving some units with twice the work of the others.
int mfma_row_tiles(int64_t tiles) { return tiles > device_cu_count() ? 2 : 1; }

// Token rows the MFMA kernels stage per step for M tokens.
int mfma_xt(int64_t M) { return M <= 4 ? 4 : M <= 8 ? 8 : M <= 16 ? 16 : M <= 32 ? 32 : 64; }

// The split-K forms built into the library: (row tiles per unit, splits).
constexpr int kSplitForms[][2] = {{1, 2}, {2, 2}, {3, 2}, {4, 2}, {1, 4}, {2, 4}, {4, 4}};

template <bool FP4, int XT, bool SILU, int RT, int S>
bool launch_split_if(const GemvParams& p, int rt, int s, hipStream_t stream, hipError_t* err) {
  if (rt != RT || s != S) return false;
  if constexpr (mfma_fits(FP4, XT, (SILU ? 2 : 1) * RT)) {
    *err = launch_mfma_rt<FP4, XT, SILU, RT, S>(p, stream);
    return true;
  }
  return false;
}

template <bool FP4, int XT, bool SILU>
hipError_t launch_mfma(GemvParams p, hipStream_t stream) {
  const int64_t limit = SILU ? p.half : p.N;
  const int64_t tiles = FP4 ? ((limit + 127) / 128) * 8 : (limit + 15) / 16;
  if (p.part != nullptr) {
    const SplitPlan plan = gemv_split_plan(FP4, p.M, p.N, p.K, SILU);
    hipError_t err = hipSuccess;
    if (plan.s > 1 && (launch_split_if<FP4, XT, SILU, 1, 2>(p, plan.rt, plan.s, stream, &err) ||
                       launch_split_if<FP4, XT, SILU, 2, 2>(p, plan.rt, plan.s, stream, &err) ||
                       launch_split_if<FP4, XT, SILU, 3, 2>(p, plan.rt, plan.s, stream, &err) ||
                       launch_split_if<FP4, XT, SILU, 4, 2>(p, plan.rt, plan.s, stream, &err) ||
                       launch_split_if<FP4, XT, SILU, 1, 4>(p, plan.rt, plan.s, stream, &err) ||
                       launch_split_if<FP4, XT, SILU, 2, 4>(p, plan.rt, plan.s, stream, &err) ||
                       launch_split_if<FP4, XT, SILU, 4, 4>(p, plan.rt, plan.s, stream, &err)))
      return err;
  }
  // (one tile per workgroup at XT = 4, and for silu_mul up to XT = 8:
  // measured faster there; with silu_mul at XT = 64 a second tile's partial
  // sums would not fit in LDS beside the ring)
  if constexpr (XT < 64 || !SILU) {
    if (XT > 4 && !(SILU && XT <= 8) && mfma_row_tiles(tiles) == 2) return launch_mfma_rt<FP4, XT, SILU, 2>(p, stream);
  }
  return launch_mfma_rt<FP4, XT, SILU, 1>(p, stream);
}

template <int G, int NQ, int C, bool SILU>
hipError_t launch_blk_c(GemvParams p, hipStream_t stream) {
  constexpr int KS = 4;
  p.units = (p.units + NQ - 1) / NQ;
  if (t_describe) {
    std::snprintf(t_describe, t_describe_len, "k_gemv_blk<%d, %d, %d, %d, %s>", G, NQ, C, KS, tf(SILU));
    return hipSuccess;
  }
  hipLaunchKernelGGL((k_gemv_blk<G, NQ, C, KS, SILU>), dim3(static_cast<unsigned>(p.units)), dim3(64 * KS), 0, stream,
                     p);
  return hipGetLastError();
}

template <int G, int NQ, bool SILU>
hipError_t launch_blk_nq(const GemvParams& p, hipStream_t stream) {
  if ((p.K + 511) / 512 <= 4) return launch_blk_c<G, NQ, 1, SILU>(p, stream);
  return launch_blk_c<G, NQ, 2, SILU>(p, stream);
}

// Quads per unit: the busiest compute unit's rounds of units times the
// quads of a unit plus one (a unit's fixed cost, its activation reads and
// reduction, counted as one quad); ties go to the larger unit.  Measured at
// 2..4 tokens: 4096 rows (1024 quads) 4 per unit, 6144 rows 3 (2 or 4 were
// 0.1-0.2 us slower, 6 and 8 slower still), the fused silu call on 2 x 14336
// rows 4 (0.05-0.2 us ahead of 2, 1 was 1.8-3.7 us slower).
int blk_quads_per_unit(int64_t quads) {
  const int64_t cus = device_cu_count();
  int best = 0;
  int64_t best_cost = 0;
  for (int nq = 4; nq >= 1; --nq) {
    const int64_t units = (quads + nq - 1) / nq;
    const int64_t cost = (units + cus - 1) / cus * (nq + 1);
    if (best == 0 || cost < best_cost) {
      best = nq;
      best_cost = cost;
    }
  }
  return best;
}

template <int G, bool SILU>
hipError_t launch_blk(const GemvParams& p, hipStream_t stream) {
  switch (blk_quads_per_unit(p.units)) {
    case 1: return launch_blk_nq<G, 1, SILU>(p, stream);
    case 2: return launch_blk_nq<G, 2, SILU>(p, stream);
    case 3: return launch_blk_nq<G, 3, SILU>(p, stream);
    default: return launch_blk_nq<G, 4, SILU>(p, stream);
  }
}

template <int G, int NQ, int R, bool ONE>
hipError_t launch_blkh_r(GemvParams p, hipStream_t stream) {
  constexpr int KS = 4;
  p.units = (p.units + NQ - 1) / NQ;
  if (t_describe) {
    std::snprintf(t_describe, t_describe_len, "k_gemv_blkh<%d, %d, %d, %d, %s>", G, NQ, R, KS, tf(ONE));
    return hipSuccess;
  }
  hipLaunchKernelGGL((k_gemv_blkh<G, NQ, R, KS, ONE>), dim3(static_cast<unsigned>(p.units)), dim3(256), 0, stream,
                     p);
  return hipGetLastError();
}

// Up to 8 pieces of 128 k per wave (K <= 4096): all loaded up front.
template <int G, int NQ>
hipError_t launch_blkh_nq(const GemvParams& p, hipStream_t stream) {
  const int64_t pw = ((p.K + 127) / 128 + 3) / 4;  // pieces per wave
  if (pw <= 4) return launch_blkh_r<G, NQ, 4, true>(p, stream);
  if (pw <= 8) return launch_blkh_r<G, NQ, 8, true>(p, stream);
  return launch_blkh_r<G, NQ, 4, false>(p, stream);
}

template <int G>
hipError_t launch_blkh(const GemvParams& p, hipStream_t stream) {
  switch (blk_quads_per_unit(p.units)) {
    case 1: return launch_blkh_nq<G, 1>(p, stream);
    case 2: return launch_blkh_nq<G, 2>(p, stream);
    case 3: return launch_blkh_nq<G, 3>(p, stream);
    default: return launch_blkh_nq<G, 4>(p, stream);
  }
}

template <bool FP4, bool SILU>
hipError_t dispatch(GemvParams p, int path, hipStream_t stream) {
  const int64_t limit = SILU ? p.half : p.N;
  if (path == kPathBlk) {
    if constexpr (FP4) {
      p.tiles = p.K / 64;
      p.units = ((limit + 127) / 128) * 32;
      if (p.M <= 4) return launch_blk<1, SILU>(p, stream);
      return launch_blk<2, SILU>(p, stream);
    } else if constexpr (!SILU) {
      p.units = (p.N + 3) / 4;  // groups of 4 consecutive rows
      if (p.M <= 4) return launch_blkh<1>(p, stream);
      return launch_blkh<2>(p, stream);
    }
  }
  if (path == kPathValu) {
    p.tiles = FP4 ? p.K / 64 : p.K / 16;
    p.units = FP4 ? ((limit + 127) / 128) * 32 : (limit + 3) / 4;
    if constexpr (FP4) {
      if (p.K <= kVchunkMaxK) {
        if (p.M <= 1) return launch_vchunk<1, SILU>(p, stream);
        if (p.M <= 2) return launch_vchunk<2, SILU>(p, stream);
        return launch_vchunk<4, SILU>(p, stream);
      }
    }
    const int lpq = lanes_per_unit(p.tiles);
    if (p.M <= 1) return launch_valu<FP4, 1, SILU>(p, lpq, stream);
    return launch_valu<FP4, 2, SILU>(p, lpq, stream);
  }
  p.tiles = p.K / 64;
  if constexpr (FP4) {
    hipError_t err;
    if (p.M <= 4 && launch_mfma_bd<SILU, 4, 24>(p, stream, &err)) return err;
    if (p.M > 4 && p.M <= 8 && launch_mfma_bd<SILU, 8, 24>(p, stream, &err)) return err;
    if (p.M > 4 && p.M <= 8 && launch_mfma_bd<SILU, 8, 56>(p, stream, &err)) return err;
  }
  if (p.M <= 4) return launch_mfma<FP4, 4, SILU>(p, stream);
  if (p.M <= 8) return launch_mfma<FP4, 8, SILU>(p, stream);
  if (p.M <= 16) return launch_mfma<FP4, 16, SILU>(p, stream);
  if (p.M <= 32) return launch_mfma<FP4, 32, SILU>(p, stream);
  return launch_mfma<FP4, 64, SILU>(p, stream);
}

}  // namespace

SplitPlan gemv_split_plan(bool fp4, int64_t M, int64_t N, int64_t K, int silu) {
  SplitPlan none{1, 1, 0};
  if (M <= 0 || N <= 0 || K <= 0) return none;
  const int xt = mfma_xt(M);
  const int64_t limit = silu ? N / 2 : N;
  const int64_t tiles = fp4 ? ((limit + 127) / 128) * 8 : (limit + 15) / 16;
  int rt = 1, s = 1;
  const char* env = std::getenv("W4A16_SPLITK");
  if (env && std::strcmp(env, "off") == 0) return none;
  if (env && std::sscanf(env, "%d,%d", &rt, &s) == 2) {
    // a forced form (tests and measurements); it must be one of the built ones
    bool built = false;
    for (const auto& f : kSplitForms) built |= f[0] == rt && f[1] == s;
    if (!built) return none;
  } else {
    // Measured on the MI355X (graphs of 64 launches, rotating weights): the
    // hand-off of the partial sums costs about 1.2 us, so a split pays where
    // it either fills compute units that would idle or removes a large share
    // of the activation stream.
    //  * Fewer row tiles than half the compute units: one tile per unit and
    //    2 splits (4 where a quarter of the units would be busy and each
    //    split still streams >= 16 KB of weights), once a workgroup's weight
    //    and activation bytes reach 160 KB (128 KB with 4 splits).  E.g.
    //    1024 x 8192 NVFP4 at 32 tokens 11.9 -> 7.8 us, BF16 2048 x 8192
    //    13.5 -> 9.6 us at 4 tokens; 1024 x 4096 NVFP4 at 4 tokens stays.
    //  * Otherwise, when a workgroup would stream >= 768 KB of activations:
    //    2 splits over units of about 2 * tiles / (compute units) tiles.
    //    E.g. 4096 x 14336 NVFP4 at 32 tokens 21.4 -> 17.4 us, BF16 36.5 ->
    //    31.6 us; the 4096 x 4096 and 6144 x 4096 sweep shapes never split.
    // the VALU and 4x4 block kernels take these
    if ((fp4 && M <= kValuMaxMFp4) || default_gemv_path(fp4, M, N, K, silu) == kPathBlk) return none;
    const int64_t cus = device_cu_count();
    const double w_tile = 16.0 * (silu ? 2 : 1) * static_cast<double>(K) * (fp4 ? 0.5625 : 2.0);
    const double a_wg = static_cast<double>(xt) * static_cast<double>(K) * 2.0;
    if (tiles * 2 <= cus) {
      rt = 1;
      s = (tiles * 4 <= cus && w_tile / 4 >= 16384.0) ? 4 : 2;
      if (w_tile + a_wg < (s == 4 ? 131072.0 : 163840.0)) return none;
    } else if (a_wg >= 786432.0) {
      s = 2;
      const int64_t want = (tiles * s + cus - 1) / cus;
      rt = static_cast<int>(want < 1 ? 1 : want > 4 ? 4 : want);
    } else {
      return none;
    }
  }
  const int na = (silu ? 2 : 1) * rt;
  if (!mfma_fits(fp4, xt, na)) return none;
  const int64_t units = (tiles + rt - 1) / rt;
  if (units * 4 > kSplitCounterBytes) return none;
  const int64_t nt = (xt + 15) / 16;
  // The counters sit in a region of fixed size at the start of every
  // workspace, whatever the plan: partial sums of one call never overlap
  // counters of another, so a workspace moves between shapes with every
  // counter still zero.
  return SplitPlan{rt, s, kSplitCounterBytes, kSplitCounterBytes + units * s * na * nt * 64 * 16};
}

// NVFP4: the VALU kernel at one token (and at two for rows longer than
// kBlkMaxK columns), the 4x4 block MFMA kernel from 2 to 4 tokens (rows of
// up to kBlkMaxK columns), the 16x16 MFMA kernels above.  BF16 without
// silu_mul: the 4x4 block kernel from 1 to 4 tokens, and from 5 to 8 for
// rows longer than 2048 columns, else the MFMA kernels.  NVFP4 rows of up
// to kVchunkMaxK columns take the chunked VALU kernel (M <= 4 when forced);
// other VALU cases stage M <= 2 activation rows in a 64 KB LDS area.
// W4A16_GEMV_PATH=valu|mfma|blk forces a path where it applies (the tests
// use it to cover every family at every M).
namespace {

bool valu_fits(bool fp4, int64_t M, int64_t K) {
  return (fp4 && K <= kVchunkMaxK) ? M <= 4 : (M <= 2 && M * ((K + 63) / 64 * 64) * 2 <= 65536);
}
bool blk_fits(bool fp4, int64_t M, int64_t K, int silu) {
  return fp4 ? (K <= kBlkMaxK && M <= kBlkMaxM) : (!silu && M <= kBlkhMaxM);
}

}  // namespace

int default_gemv_path(bool fp4, int64_t M, int64_t N, int64_t K, int silu) {
  (void)N;
  // measured (µs, 4096 x 4096 / 6144 x 4096 / the fused silu call on
  // 2 x 14336 rows): 2 tokens 4.62 / 5.35 / 16.1 (VALU) -> 4.31 / 5.36 /
  // 14.4, 4 tokens 4.86 / 6.51 / 19.9 (16x16 MFMA) -> 4.42 / 5.58 / 14.9; at
  // 5..8 tokens the 16x16 MFMA kernels stay ahead (4x4x4 MFMAs are a
  // quarter of their rate per product, and 8 tokens' activations halve the
  // workgroups per compute unit).  BF16 weights (4096 x 4096 / 4096 x 14336
  // / 2048 x 8192): 1 token 7.95 / 23.5 / - (VALU) -> 7.08 / 19.9 / 8.2, 4
  // tokens 8.26 / 25.0 / - (16x16 MFMA) -> 7.59 / 21.3 / 8.9; 8 tokens, rows
  // longer than 2048 columns, 8.74 / 26.5 / 14.6 (16x16 MFMA) -> 8.37 / 23.8
  // / 10.6 (at 2048 columns equal, at 1024 4.41 -> 4.71)
  if (blk_fits(fp4, M, K, silu) && M >= (fp4 ? 2 : 1) && M <= 4) return kPathBlk;
  if (!fp4 && blk_fits(fp4, M, K, silu) && K > 2048) return kPathBlk;
  // NVFP4 without silu_mul at 5..8 tokens: the 4x4 kernel where its units fill
  // the compute units in one round (4096 x 4096: 5.13 -> 5.00 us at 8 tokens;
  // at 6144 x 4096, two units per compute unit, 6.43 -> 6.72)
  if (fp4 && !silu && blk_fits(fp4, M, K, silu) && M > 4) {
    const int64_t quads = (N + 127) / 128 * 32;
    const int nq = blk_quads_per_unit(quads);
    if ((quads + nq - 1) / nq <= device_cu_count()) return kPathBlk;
  }
  // BF16 with silu_mul at M = 1: the MFMA path up to K = 8192 (measured 5%
  // faster at 4096 without silu_mul), the VALU path beyond (2% faster at
  // 14336)
  const int64_t valu_max_m = fp4 ? kValuMaxMFp4 : (K <= 8192 ? 0 : 1);
  return (valu_fits(fp4, M, K) && M <= valu_max_m) ? kPathValu : kPathMfma;
}

int choose_gemv_path(bool fp4, int64_t M, int64_t N, int64_t K, int silu) {
  if (const char* env = std::getenv("W4A16_GEMV_PATH")) {
    if (std::strcmp(env, "mfma") == 0) return kPathMfma;
    if (std::strcmp(env, "valu") == 0 && valu_fits(fp4, M, K)) return kPathValu;
    if (std::strcmp(env, "blk") == 0 && blk_fits(fp4, M, K, silu)) return kPathBlk;
  }
  return default_gemv_path(fp4, M, N, K, silu);
}

void describe_gemv(bool fp4, const GemvParams& p, int silu, int path, char* name, size_t len) {
  name[0] = 0;
  t_describe = name;
  t_describe_len = len;
  (void)launch_gemv(fp4, p, silu, path, nullptr);  // p.part non-null: the form with a workspace
  t_describe = nullptr;
  t_describe_len = 0;
}

hipError_t launch_gemv(bool fp4, const GemvParams& p, int silu, int path, hipStream_t stream) {
  if (fp4) return silu ? dispatch<true, true>(p, path, stream) : dispatch<true, false>(p, path, stream);
  return silu ? dispatch<false, true>(p, path, stream) : dispatch<false, false>(p, path, stream);
}

}  // namespace w4a16
