// dequantize_rows and the scale un-swizzle (bit-exact kernels).
//
// dequantize_rows (nvfp4_gemv page, function dequantize_rows): every weight
// becomes the BF16 value e2m1 * e4m3, which is exact, so the result does not
// depend on how it is computed; the global scale is not applied.  One thread
// decodes 16 bytes of codes (32 weights, two 16-k scale blocks) of one row and
// writes 64 bytes of BF16.
#include "device_common.hpp"
#include "launch.hpp"

namespace w4a16 {

__global__ __launch_bounds__(256) void k_dequantize_rows(const uint8_t* __restrict__ w,
                                                         const uint8_t* __restrict__ s,
                                                         uint16_t* __restrict__ out, int64_t rows,
                                                         int64_t K) {
  const int64_t per_row = K / 32;
  const int64_t total = rows * per_row;
  const int64_t tiles = K / 64;
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < total;
       i += static_cast<int64_t>(gridDim.x) * blockDim.x) {
    const int64_t row = i / per_row;
    const int64_t q = i - row * per_row;  // 32-k piece of the row
    const u32x4 wv = load16_nt(w + row * (K / 2) + q * 16);
    const uint32_t sw = load4(s + scale_word_offset(row, q >> 1, tiles)) >> (16 * (q & 1));
    const float s0 = e4m3_to_f32<0>(sw);
    const float s1 = e4m3_to_f32<1>(sw);
    uint32_t o[16];
    dequant_dword(wv.x, s0, o);
    dequant_dword(wv.y, s0, o + 4);
    dequant_dword(wv.z, s1, o + 8);
    dequant_dword(wv.w, s1, o + 12);
    u32x4* dst = reinterpret_cast<u32x4*>(out + row * K + q * 32);
    __builtin_nontemporal_store(u32x4{o[0], o[1], o[2], o[3]}, dst);
    __builtin_nontemporal_store(u32x4{o[4], o[5], o[6], o[7]}, dst + 1);
    __builtin_nontemporal_store(u32x4{o[8], o[9], o[10], o[11]}, dst + 2);
    __builtin_nontemporal_store(u32x4{o[12], o[13], o[14], o[15]}, dst + 3);
  }
}

// out[n][c] = scale byte of row n, column c, through the same addressing the
// GEMV kernels use (one 4-byte word = 4 consecutive columns of one row).
__global__ __launch_bounds__(256) void k_unswizzle(const uint8_t* __restrict__ s,
                                                   uint8_t* __restrict__ out, int64_t N,
                                                   int64_t K) {
  const int64_t cols = K / 16;
  const int64_t tiles = (cols + 3) / 4;
  const int64_t total = N * cols;
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < total;
       i += static_cast<int64_t>(gridDim.x) * blockDim.x) {
    const int64_t n = i / cols;
    const int64_t c = i - n * cols;
    out[i] = s[scale_word_offset(n, c >> 2, tiles) + (c & 3)];
  }
}

// Epilogue of the dequant + GEMM path: out = bf16(acc * gs) from the FP32
// GEMM result acc [M][N], or with silu_mul out[m][j] = bf16(silu(g) * u),
// g = bf16(acc[m][j] * gs), u = bf16(acc[m][N/2 + j] * gs) (the same
// epilogue as the GEMV kernels).
__global__ __launch_bounds__(256) void k_scale_epilogue(const float* __restrict__ acc,
                                                        const float* __restrict__ gs_ptr,
                                                        uint16_t* __restrict__ out, int64_t M, int64_t N,
                                                        int silu_mul) {
  const float gs = *gs_ptr;
  const int64_t cols = silu_mul ? N / 2 : N;
  const int64_t total = M * cols;
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < total;
       i += static_cast<int64_t>(gridDim.x) * blockDim.x) {
    const int64_t m = i / cols;
    const int64_t j = i - m * cols;
    if (!silu_mul) {
      out[i] = f32_to_bf16_bits(acc[m * N + j] * gs);
    } else {
      const float g = bf16_bits_to_f32(f32_to_bf16_bits(acc[m * N + j] * gs));
      const float u = bf16_bits_to_f32(f32_to_bf16_bits(acc[m * N + cols + j] * gs));
      out[i] = f32_to_bf16_bits(silu_f32(g) * u);
    }
  }
}

namespace {
unsigned grid_for(int64_t items) {
  int64_t b = (items + 255) / 256;
  if (b > 65536) b = 65536;
  if (b < 1) b = 1;
  return static_cast<unsigned>(b);
}
}  // namespace

hipError_t launch_dequantize_rows(const uint8_t* w, const uint8_t* s, int64_t rows, int64_t K,
                                  uint16_t* out, hipStream_t stream) {
  hipLaunchKernelGGL(k_dequantize_rows, dim3(grid_for(rows * (K / 32))), dim3(256), 0, stream, w, s,
                     out, rows, K);
  return hipGetLastError();
}

hipError_t launch_unswizzle(const uint8_t* s, int64_t N, int64_t K, uint8_t* out,
                            hipStream_t stream) {
  hipLaunchKernelGGL(k_unswizzle, dim3(grid_for(N * (K / 16))), dim3(256), 0, stream, s, out, N, K);
  return hipGetLastError();
}

hipError_t launch_scale_epilogue(const float* acc, const float* gs, uint16_t* out, int64_t M, int64_t N,
                                 int silu_mul, hipStream_t stream) {
  const int64_t items = M * (silu_mul ? N / 2 : N);
  hipLaunchKernelGGL(k_scale_epilogue, dim3(grid_for(items)), dim3(256), 0, stream, acc, gs, out, M, N, silu_mul);
  return hipGetLastError();
}

}  // namespace w4a16
