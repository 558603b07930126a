// Expert-indexed MoE decode pair (moe_gemv page): gate_up, then
// down_combine, both built from the VALU unit of the dense GEMV.
//
// gate_up: one unit per (routed pair p, gate quad) and per (token, shared
// gate quad).  A unit reads the gate quad and the matching up quad (rows i and
// I + i of the expert's [gate; up] weight) over the whole hidden size and
// writes act[p][i] = bf16(silu(g) * u) with g, u = FP32 accumulator * alpha[e]
// (routed), or sact[t][i] = bf16(silu(bf16(g)) * bf16(u)) (shared expert, the
// dense silu_mul numerics).
//
// down_combine: one workgroup per (token, quad of output rows).  Its lane
// groups compute the topk routed down projections and the shared one at the
// same time (each over the whole intermediate size); the per-piece results
// meet in LDS, where the FP32 weighted sum is formed over j ascending and
// out = bf16(bf16(sum_j tw_j * y_j) + y_shared) is written.
#include "device_common.hpp"
#include "launch.hpp"
#include "unit_core.hpp"

namespace w4a16 {

__device__ __forceinline__ int64_t clamp_expert(int32_t id, int E) {
  return id < 0 ? 0 : (id >= E ? E - 1 : id);
}

template <int LPQ>
__global__ __launch_bounds__(256) void k_moe_gate_up(const MoeGateUpParams p) {
  constexpr int G = kWave / LPQ;
  const int lane = threadIdx.x & 63;
  const int li = lane % LPQ;
  const int slot = lane / LPQ;
  const int wave = threadIdx.x >> 6;
  const int64_t gwave = static_cast<int64_t>(xcd_logical_block()) * 4 + wave;
  const int64_t stride = static_cast<int64_t>(gridDim.x) * 4 * G;
  const int64_t total = p.routed_units + p.shared_units;
  const int64_t row_bytes = p.H / 2;
  const int64_t tiles = p.H / 64;

  for (int64_t ubase = gwave * G; ubase < total; ubase += stride) {
    const int64_t u = ubase + slot;
    const bool active = u < total;
    const bool routed = u < p.routed_units;
    const uint8_t* w;
    const uint8_t* s;
    int64_t t, q, half, dst_base;
    float scale;
    uint16_t* dst;
    if (routed) {
      const int64_t pair = u / p.units_per_pair;
      q = u - pair * p.units_per_pair;
      t = pair / p.topk;
      const int64_t e = clamp_expert(p.ids[pair], p.E);
      w = p.w1 + e * p.w1_expert_bytes;
      s = p.w1s + e * p.s1_expert_bytes;
      half = p.I;
      scale = p.alpha[e];
      dst = p.act;
      dst_base = pair * p.I;
    } else {
      const int64_t v = active ? u - p.routed_units : 0;
      t = v / p.units_per_token;
      q = v - t * p.units_per_token;
      w = p.wsh;
      s = p.ssh;
      half = p.SI;
      scale = *p.gssh;
      dst = p.sact;
      dst_base = t * p.SI;
    }
    int64_t rows[8];
    bool rv[8];
    quad_rows<8>(q, half, half, rows, rv);
    if (!active) {
#pragma unroll
      for (int i = 0; i < 8; ++i) rv[i] = false;
    }
    const bool quad_ok[2] = {true, half % 128 == 0};
    float acc[8][1];
    unit_dot<true, 8, 1, LPQ>(w, row_bytes, s, tiles, rows, rv, quad_ok, p.x + t * p.H, p.H, 1,
                              li, active, acc);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if (i % LPQ != li || !rv[i]) continue;
      float v;
      if (routed) {
        const float g = acc[i][0] * scale;
        const float up = acc[4 + i][0] * scale;
        v = silu_f32(g) * up;
      } else {
        const float g = bf16_bits_to_f32(f32_to_bf16_bits(acc[i][0] * scale));
        const float up = bf16_bits_to_f32(f32_to_bf16_bits(acc[4 + i][0] * scale));
        v = silu_f32(g) * up;
      }
      dst[dst_base + rows[i]] = f32_to_bf16_bits(v);
    }
  }
}

// One workgroup of `waves` waves per (token, output quad); piece j < topk is
// routed slot j, piece topk the shared expert.  G pieces per wave.
template <int LPQ>
__global__ __launch_bounds__(1024) void k_moe_down_combine(const MoeDownParams p) {
  constexpr int G = kWave / LPQ;
  __shared__ float part[17][4];
  const int lane = threadIdx.x & 63;
  const int li = lane % LPQ;
  const int wave = threadIdx.x >> 6;
  const int piece = wave * G + lane / LPQ;
  const int pieces = p.topk + 1;

  for (int64_t u = xcd_logical_block(); u < p.units; u += gridDim.x) {
    const int64_t t = u / p.units_per_token;
    const int64_t q = u - t * p.units_per_token;
    int64_t rows[4];
    bool rv[4];
    quad_rows<4>(q, p.H, 0, rows, rv);
    const bool active = piece < pieces;
    const bool routed = piece < p.topk;
    const uint8_t* w;
    const uint8_t* s;
    const uint16_t* xrow;
    int64_t kdim;
    float scale, weight;
    if (routed) {
      const int64_t pair = t * p.topk + piece;
      const int64_t e = clamp_expert(p.ids[pair], p.E);
      w = p.w2 + e * p.w2_expert_bytes;
      s = p.w2s + e * p.s2_expert_bytes;
      xrow = p.act + pair * p.I;
      kdim = p.I;
      scale = p.alpha2[e];
      weight = p.tw[pair];
    } else {
      w = p.wsd;
      s = p.ssd;
      xrow = p.sact + t * p.SI;
      kdim = p.SI;
      scale = *p.gssd;
      weight = 1.0f;
    }
    bool rva[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) rva[i] = rv[i] && active;
    const bool quad_ok[1] = {true};
    float acc[4][1];
    unit_dot<true, 4, 1, LPQ>(w, kdim / 2, s, kdim / 64, rows, rva, quad_ok, xrow, kdim, 1, li,
                              active, acc);
    if (active && li < 4) {
      float v = li == 0 ? acc[0][0] : li == 1 ? acc[1][0] : li == 2 ? acc[2][0] : acc[3][0];
      // y = bf16(acc * alpha); routed pieces contribute tw * y (FP32).
      const float y = bf16_bits_to_f32(f32_to_bf16_bits(v * scale));
      part[piece][li] = routed ? weight * y : y;
    }
    __syncthreads();
    if (threadIdx.x < 4) {
      const int i = threadIdx.x;
      float sum = 0.0f;
      for (int j = 0; j < p.topk; ++j) sum += part[j][i];
      const float sr = bf16_bits_to_f32(f32_to_bf16_bits(sum));
      const float v = sr + part[p.topk][i];
      const int64_t row = rows[i];
      if (row < p.H) p.out[t * p.H + row] = f32_to_bf16_bits(v);
    }
    __syncthreads();
  }
}

namespace {
int lanes_for_tiles(int64_t tiles) {
  if (tiles > 32) return 64;
  if (tiles > 16) return 32;
  if (tiles > 8) return 16;
  return 8;
}
}  // namespace

hipError_t launch_moe_gate_up(MoeGateUpParams p, hipStream_t stream) {
  const int lpq = lanes_for_tiles(p.H / 64);
  const int64_t g = kWave / lpq;
  const int64_t total = p.routed_units + p.shared_units;
  const int64_t waves = (total + g - 1) / g;
  int64_t blocks = (waves + 3) / 4;
  if (blocks > 16384) blocks = 16384;
  const dim3 grid(static_cast<unsigned>(blocks)), block(256);
  switch (lpq) {
    case 64: hipLaunchKernelGGL(k_moe_gate_up<64>, grid, block, 0, stream, p); break;
    case 32: hipLaunchKernelGGL(k_moe_gate_up<32>, grid, block, 0, stream, p); break;
    case 16: hipLaunchKernelGGL(k_moe_gate_up<16>, grid, block, 0, stream, p); break;
    default: hipLaunchKernelGGL(k_moe_gate_up<8>, grid, block, 0, stream, p); break;
  }
  return hipGetLastError();
}

hipError_t launch_moe_down_combine(MoeDownParams p, hipStream_t stream) {
  const int64_t kmax = p.I > p.SI ? p.I : p.SI;
  int lpq = lanes_for_tiles(kmax / 64);
  // at most 16 waves (1024 threads) per workgroup
  while (lpq > 8 && (p.topk + 1 + kWave / lpq - 1) / (kWave / lpq) > 16) lpq /= 2;
  const int g = kWave / lpq;
  const int waves = (p.topk + 1 + g - 1) / g;
  int64_t blocks = p.units;
  if (blocks > 65536) blocks = 65536;
  const dim3 grid(static_cast<unsigned>(blocks)), block(64 * waves);
  switch (lpq) {
    case 64: hipLaunchKernelGGL(k_moe_down_combine<64>, grid, block, 0, stream, p); break;
    case 32: hipLaunchKernelGGL(k_moe_down_combine<32>, grid, block, 0, stream, p); break;
    case 16: hipLaunchKernelGGL(k_moe_down_combine<16>, grid, block, 0, stream, p); break;
    default: hipLaunchKernelGGL(k_moe_down_combine<8>, grid, block, 0, stream, p); break;
  }
  return hipGetLastError();
}

}  // namespace w4a16
