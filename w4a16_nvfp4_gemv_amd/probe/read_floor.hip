// Streaming-read reference for the benchmark (not part of the GEMV library):
// one launch reads the packed weight bytes and the scale bytes of a GEMV call
// exactly once and writes a little output, with nothing else in the way, so
// its time is what a launch that moves those bytes costs on this part.
//
// Each workgroup of 256 threads reads one contiguous region of NL * 4 KB:
// every thread issues its NL 16-byte streaming loads back to back (a wave's
// load covers 1 KB contiguous), then folds them with XOR and stores the
// result only if it equals a constant that random data almost never gives:
// every load's value is used, so none can be dropped, and the launch writes
// (next to) nothing.  (A store from some threads only would let the compiler
// drop the other threads' loads.)
// The first ceil(w_bytes / region) workgroups read the weight, the rest the
// scales; loads past either buffer's end return zeros (buffer resources).
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* p, uint32_t n) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), 0, static_cast<int>(n), 0x00020000);
}

template <int NL>
__global__ __launch_bounds__(256) void k_read_floor(const uint8_t* w, uint32_t w_bytes, const uint8_t* s,
                                                    uint32_t s_bytes, uint32_t w_blocks, uint16_t* out) {
  const bool on_w = blockIdx.x < w_blocks;
  const uint32_t blk = on_w ? blockIdx.x : blockIdx.x - w_blocks;
  const auto r = on_w ? rsrc(w, w_bytes) : rsrc(s, s_bytes);
  const uint32_t base = blk * NL * 4096u;
  u32x4 v[NL];
#pragma unroll
  for (int i = 0; i < NL; ++i)
    v[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                         r, static_cast<int>(base + (i * 256 + threadIdx.x) * 16), 0, 2));
  uint32_t x = 0;
#pragma unroll
  for (int i = 0; i < NL; ++i) x ^= v[i].x ^ v[i].y ^ v[i].z ^ v[i].w;
  if (x == 0x9E3779B9u) out[blockIdx.x * 64 + (threadIdx.x & 63)] = static_cast<uint16_t>(x);
}

}  // namespace

// Workgroups of one launch: regions of nl * 4 KB (nl = 1..16) over the
// w_bytes + s_bytes of one call (-1 for bad arguments).
extern "C" int64_t read_floor_blocks(int64_t w_bytes, int64_t s_bytes, int nl) {
  if (nl < 1 || nl > 16 || w_bytes < 0 || s_bytes < 0) return -1;
  const int64_t region = int64_t(nl) * 4096;
  return (w_bytes + region - 1) / region + (s_bytes + region - 1) / region;
}

// One launch; `out` holds at least read_floor_blocks(...) * 64 uint16.
// Returns 0, 1 for bad arguments, 2 for a launch error.
extern "C" int read_floor_launch(const uint8_t* w, int64_t w_bytes, const uint8_t* s, int64_t s_bytes, int nl,
                                 uint16_t* out, void* stream) {
  const int64_t blocks = read_floor_blocks(w_bytes, s_bytes, nl);
  if (blocks <= 0 || blocks > 65535 || w_bytes >= (int64_t(1) << 31) || s_bytes >= (int64_t(1) << 31)) return 1;
  const uint32_t w_blocks = static_cast<uint32_t>((w_bytes + int64_t(nl) * 4096 - 1) / (int64_t(nl) * 4096));
  const hipStream_t st = static_cast<hipStream_t>(stream);
  const dim3 grid(static_cast<unsigned>(blocks)), block(256);
  const uint32_t wb = static_cast<uint32_t>(w_bytes), sb = static_cast<uint32_t>(s_bytes);
  switch (nl) {
#define W4A16_RF(n) \
  case n: hipLaunchKernelGGL(k_read_floor<n>, grid, block, 0, st, w, wb, s, sb, w_blocks, out); break;
    W4A16_RF(1) W4A16_RF(2) W4A16_RF(3) W4A16_RF(4) W4A16_RF(5) W4A16_RF(6) W4A16_RF(7) W4A16_RF(8)
    W4A16_RF(9) W4A16_RF(10) W4A16_RF(11) W4A16_RF(12) W4A16_RF(13) W4A16_RF(14) W4A16_RF(15) W4A16_RF(16)
#undef W4A16_RF
    default: return 1;
  }
  return hipGetLastError() == hipSuccess ? 0 : 2;
}
