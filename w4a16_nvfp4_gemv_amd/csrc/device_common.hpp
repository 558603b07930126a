// Device-side building blocks shared by the gfx950 kernels: element decode,
// 128x4 scale addressing, wave reductions and the XCD-aware block order.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace w4a16 {

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;

// ---------------------------------------------------------------- decode
// FP8 E4M3FN byte `sel` of `word` -> f32.  gfx950's v_cvt_f32_fp8 decodes the
// OCP E4M3FN format (bias 7, NaN at 0x7F/0xFF, no inf); every value is exact
// in f32.
template <int SEL>
__device__ __forceinline__ float e4m3_to_f32(uint32_t word) {
  return __builtin_amdgcn_cvt_f32_fp8(static_cast<int>(word), SEL);
}

// The two FP4 E2M1 codes of byte `SEL` of `word` (low nibble first) -> two
// exact f32 values.  The hardware conversion takes only the exponent of its
// scale operand, so it runs with scale 1 and the E4M3 block scale is applied
// by an ordinary f32 multiply (e2m1 * e4m3 has at most 6 significant bits:
// exact in f32 and in bf16).
template <int SEL>
__device__ __forceinline__ f32x2 e2m1x2_to_f32(uint32_t word) {
  return __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(word, 1.0f, SEL);
}

// Two f32 -> packed bf16 pair, round to nearest even (v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  f32x2 v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}

// Exactly dequantized weights of byte SEL of `word`, as a packed bf16 pair.
template <int SEL>
__device__ __forceinline__ uint32_t dequant_pair(uint32_t word, float scale) {
  f32x2 f = e2m1x2_to_f32<SEL>(word);
  return pack_bf16x2(f.x * scale, f.y * scale);
}

// Eight dequantized weights (one packed dword of codes) as bf16 pairs.
__device__ __forceinline__ void dequant_dword(uint32_t word, float scale, uint32_t out[4]) {
  out[0] = dequant_pair<0>(word, scale);
  out[1] = dequant_pair<1>(word, scale);
  out[2] = dequant_pair<2>(word, scale);
  out[3] = dequant_pair<3>(word, scale);
}

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t bits16) {
  return __builtin_bit_cast(float, bits16 << 16);
}

__device__ __forceinline__ uint16_t f32_to_bf16_bits(float v) {
  return static_cast<uint16_t>(pack_bf16x2(v, 0.0f) & 0xFFFFu);
}

// a.x*b.x + a.y*b.y + c on packed bf16 pairs, FP32 accumulate.
__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a),
                                         __builtin_bit_cast(bf16x2, b), c, false);
}

// SiLU in FP32 with the accurate exponential and IEEE division.
__device__ __forceinline__ float silu_f32(float g) {
  return g / (1.0f + expf(-g));
}

// ---------------------------------------------------------------- layout
// The flat 128x4-swizzled scale buffer is a sequence of 512-byte tiles of
// 128 rows x 4 scale columns (64 k), ordered by 128-row band then by column
// group.  Row r of a band lives in the 16-byte chunk r % 32 at byte
// (r / 32) * 4; the 4 bytes of that word are the 4 consecutive columns.
// So the scale words of rows {r, r+32, r+64, r+96} for one 64-k tile are one
// aligned 16-byte chunk: the "quad" the kernels are built around.
__device__ __forceinline__ int64_t scale_chunk_offset(int64_t band, int64_t tile,
                                                      int64_t tiles_per_row, int r32) {
  return (band * tiles_per_row + tile) * 512 + r32 * 16;
}

__device__ __forceinline__ int64_t scale_word_offset(int64_t row, int64_t tile,
                                                     int64_t tiles_per_row) {
  int64_t band = row >> 7;
  int r = static_cast<int>(row & 127);
  return (band * tiles_per_row + tile) * 512 + (r & 31) * 16 + (r >> 5) * 4;
}

// ---------------------------------------------------------------- loads
// Buffer-resource loads.  A load whose byte range reaches past the resource's
// size returns zeros (per dword) instead of touching memory, so rows or tiles
// past the end of a matrix are read as zeros without a branch: every load of
// a wave can be issued back to back and waited for in order.  Offsets are
// 32-bit, so one resource spans less than 2 GiB; kOutOfRange is an offset no
// resource reaches.
typedef __amdgpu_buffer_rsrc_t rsrc_t;
constexpr uint32_t kOutOfRange = 0x80000000u;
constexpr int kRsrcWord3 = 0x00020000;  // raw buffer, 32-bit data format

// `v` when `cond` holds, else an offset at or above kOutOfRange (v < 2^31).
// Plain bit arithmetic: unlike a ?: or && the compiler cannot turn it into a
// branch around the load that uses it.
__device__ __forceinline__ uint32_t off_if(bool cond, uint32_t v) {
  return v | (static_cast<uint32_t>(!cond) << 31);
}

__device__ __forceinline__ rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, static_cast<int>(bytes), kRsrcWord3);
}
__device__ __forceinline__ u32x4 bload16(rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, static_cast<int>(off), 0, 0));
}
// Streaming variant (non-temporal: the weights are read exactly once).
__device__ __forceinline__ u32x4 bload16_nt(rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, static_cast<int>(off), 0, 2));
}
__device__ __forceinline__ uint32_t bload4(rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b32(r, static_cast<int>(off), 0, 0);
}
// Streaming 4-byte variant (the VALU kernels' code loads: measured 0.2-1.1 us
// faster per call than cached loads, which evict the scale lines and
// activations that other workgroups still read from L2).
__device__ __forceinline__ uint32_t bload4_nt(rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b32(r, static_cast<int>(off), 0, 2);
}

// 16-byte buffer load straight into LDS: lane l's 16 bytes land at byte 16*l
// of `dst`, a wave-uniform LDS address; out-of-range dwords are written as
// zeros.  These loads count in vmcnt like any other, but the compiler does not
// order later LDS reads after them: a reader waits with vm_wait<N>() (N = the
// loads issued after the ones it needs), and a slot is refilled only after
// lds_wait() has retired the reads of its previous contents.
typedef __attribute__((address_space(3))) void lds_void;
__device__ __forceinline__ void bload16_lds(rsrc_t r, void* dst, uint32_t off) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)dst, 16, static_cast<int>(off), 0, 0, 0);
}
template <int N>
__device__ __forceinline__ void vm_wait() {
  static_assert(N >= 0 && N < 64, "vmcnt is a 6-bit counter");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}
// vm_wait<n>() for an n that is a constant once the caller is unrolled (the
// switch folds away).
__device__ __forceinline__ void vm_wait_n(int n) {
  switch (n) {
#define W4A16_VM_CASE(i) \
  case i:                \
    vm_wait<i>();        \
    break;
    W4A16_VM_CASE(0) W4A16_VM_CASE(1) W4A16_VM_CASE(2) W4A16_VM_CASE(3) W4A16_VM_CASE(4) W4A16_VM_CASE(5)
    W4A16_VM_CASE(6) W4A16_VM_CASE(7) W4A16_VM_CASE(8) W4A16_VM_CASE(9) W4A16_VM_CASE(10) W4A16_VM_CASE(11)
    W4A16_VM_CASE(12) W4A16_VM_CASE(13) W4A16_VM_CASE(14) W4A16_VM_CASE(15) W4A16_VM_CASE(16) W4A16_VM_CASE(17)
    W4A16_VM_CASE(18) W4A16_VM_CASE(19) W4A16_VM_CASE(20) W4A16_VM_CASE(21) W4A16_VM_CASE(22) W4A16_VM_CASE(23)
    W4A16_VM_CASE(24) W4A16_VM_CASE(25) W4A16_VM_CASE(26) W4A16_VM_CASE(27) W4A16_VM_CASE(28) W4A16_VM_CASE(29)
    W4A16_VM_CASE(30) W4A16_VM_CASE(31) W4A16_VM_CASE(32) W4A16_VM_CASE(33) W4A16_VM_CASE(34) W4A16_VM_CASE(35)
    W4A16_VM_CASE(36) W4A16_VM_CASE(37) W4A16_VM_CASE(38) W4A16_VM_CASE(39) W4A16_VM_CASE(40) W4A16_VM_CASE(41)
    W4A16_VM_CASE(42) W4A16_VM_CASE(43) W4A16_VM_CASE(44) W4A16_VM_CASE(45) W4A16_VM_CASE(46) W4A16_VM_CASE(47)
    W4A16_VM_CASE(48) W4A16_VM_CASE(49) W4A16_VM_CASE(50) W4A16_VM_CASE(51) W4A16_VM_CASE(52) W4A16_VM_CASE(53)
    W4A16_VM_CASE(54) W4A16_VM_CASE(55) W4A16_VM_CASE(56) W4A16_VM_CASE(57) W4A16_VM_CASE(58) W4A16_VM_CASE(59)
    W4A16_VM_CASE(60) W4A16_VM_CASE(61) W4A16_VM_CASE(62)
#undef W4A16_VM_CASE
    default:
      vm_wait<0>();
      break;
  }
}
// LDS accesses written as their own instructions, so that the compiler, which
// cannot tell LDS tables apart from ring slots that loads are still writing,
// adds no vmcnt wait in front of them.  Only for LDS data that those loads do
// not write.  lds_read_u32 retires before it returns; stores and adds retire
// with the next lds_wait(), which the caller issues before any barrier that
// publishes them.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return static_cast<uint32_t>(reinterpret_cast<uintptr_t>((const __attribute__((address_space(3))) uint32_t*)(p)));
}
__device__ __forceinline__ uint32_t lds_read_u32(const void* p) {
  uint32_t v;
  asm volatile("ds_read_b32 %0, %1\n\ts_waitcnt lgkmcnt(0)" : "=v"(v) : "v"(lds_addr(p)));
  return v;
}
__device__ __forceinline__ void lds_store_f32(float* p, float v) {
  asm volatile("ds_write_b32 %0, %1" ::"v"(lds_addr(p)), "v"(v));
}
__device__ __forceinline__ void lds_add_f32(float* p, float v) {
  asm volatile("ds_add_f32 %0, %1" ::"v"(lds_addr(p)), "v"(v));
}
__device__ __forceinline__ void lds_wait() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }

__device__ __forceinline__ u32x4 load16(const void* p) {
  return *reinterpret_cast<const u32x4*>(p);
}
__device__ __forceinline__ u32x4 load16_nt(const void* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}
__device__ __forceinline__ uint32_t load4(const void* p) {
  return *reinterpret_cast<const uint32_t*>(p);
}

// ---------------------------------------------------------------- reduce
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), CTRL, 0xF, 0xF, true));
}

// Sum over aligned groups of G lanes (G a power of two <= 64); every lane of
// the group ends up with the group sum.  Inside a row of 16 lanes the partner
// values come from DPP (quad_perm [1,0,3,2], [2,3,0,1], row_half_mirror,
// row_mirror: after each step every lane holds the sum of its 2, 4, 8, 16
// lanes); the 16- and 32-lane steps use cross-lane shuffles.
template <int G>
__device__ __forceinline__ float group_sum(float v) {
  if constexpr (G >= 2) v += dpp_f32<0xB1>(v);
  if constexpr (G >= 4) v += dpp_f32<0x4E>(v);
  if constexpr (G >= 8) v += dpp_f32<0x141>(v);
  if constexpr (G >= 16) v += dpp_f32<0x140>(v);
  if constexpr (G >= 32) v += __shfl_xor(v, 16, kWave);
  if constexpr (G >= 64) v += __shfl_xor(v, 32, kWave);
  return v;
}

// Reduce-scatter of V per-lane values over the 64 lanes of a wave, down to P
// values per lane (P = 1, or 2 to keep pairs such as gate/up together).
// v_permlane32_swap exchanges the upper half-wave of its first operand with the
// lower half-wave of its second, so one swap and one add sum value j over lanes
// {l, l^32} in the lower half-wave and value j + V/2 in the upper one;
// v_permlane16_swap does the same between odd and even 16-lane rows.  The
// values left are then summed over the remaining 16/32/64 lanes with
// group_sum.  On return lane l holds, in v[0..P'-1], the full sums of values
// base + 0..P'-1, base = reduce_scatter_base<V, P>(l).
template <int V, int P>
struct ReduceScatter {
  static constexpr bool S32 = V >= 2 * P;
  static constexpr bool S16 = V >= 4 * P;
  static constexpr int LEFT = S16 ? V / 4 : (S32 ? V / 2 : V);  // values per lane at the end
  static constexpr int SPAN = S16 ? 16 : (S32 ? 32 : 64);       // lanes still to sum over
};

template <int V, int P>
__device__ __forceinline__ int reduce_scatter_base(int lane) {
  using RS = ReduceScatter<V, P>;
  int base = 0;
  if constexpr (RS::S32) base += (lane >> 5) * (V / 2);
  if constexpr (RS::S16) base += ((lane >> 4) & 1) * (V / 4);
  return base;
}

template <int V, int P>
__device__ __forceinline__ void reduce_scatter(float (&v)[V]) {
  using RS = ReduceScatter<V, P>;
  if constexpr (RS::S32) {
#pragma unroll
    for (int j = 0; j < V / 2; ++j) {
      const auto r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(uint32_t, v[j]),
                                                      __builtin_bit_cast(uint32_t, v[j + V / 2]), false, false);
      v[j] = __builtin_bit_cast(float, static_cast<uint32_t>(r[0])) +
             __builtin_bit_cast(float, static_cast<uint32_t>(r[1]));
    }
  }
  if constexpr (RS::S16) {
#pragma unroll
    for (int j = 0; j < V / 4; ++j) {
      const auto r = __builtin_amdgcn_permlane16_swap(__builtin_bit_cast(uint32_t, v[j]),
                                                      __builtin_bit_cast(uint32_t, v[j + V / 4]), false, false);
      v[j] = __builtin_bit_cast(float, static_cast<uint32_t>(r[0])) +
             __builtin_bit_cast(float, static_cast<uint32_t>(r[1]));
    }
  }
#pragma unroll
  for (int j = 0; j < RS::LEFT; ++j) v[j] = group_sum<RS::SPAN>(v[j]);
}

// ---------------------------------------------------------------- XCD order
// Workgroups are dispatched round-robin over the 8 XCDs (hardware id b runs on
// XCD b % 8).  Renumbering them so that consecutive logical ids share an XCD
// keeps the blocks that read neighbouring scale chunks (and the same 128-byte
// L2 lines) on one L2.
__device__ __forceinline__ int xcd_logical_block() {
  const int b = blockIdx.x, g = gridDim.x;
  const int xcd = b & 7, idx = b >> 3;
  const int q = g >> 3, rem = g & 7;
  return xcd * q + (xcd < rem ? xcd : rem) + idx;
}

}  // namespace w4a16
