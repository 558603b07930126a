// The library GEMM of the dequant + GEMM path for token counts beyond the
// GEMV kernels (linear page, function _dequant_gemm): BF16 operands, FP32
// accumulation and FP32 output, through rocBLAS.  The global scale and the
// single BF16 rounding are applied afterwards by the library's own epilogue
// kernel, so the GEMM runs with host-side alpha = 1 and beta = 0 and never
// reads its output buffer.
//
// One rocBLAS handle per device, created on the first call on that device and
// kept until the process ends (rocBLAS manages its own device memory for it).
// Calls on one device are serialized on the handle, whose stream is set per
// call; atomics are disallowed so that the sums do not depend on timing.
#include <hip/hip_runtime.h>
#include <rocblas/rocblas.h>

#include <mutex>

#include "launch.hpp"

namespace w4a16 {
namespace {

constexpr int kMaxDevices = 64;
std::mutex g_blas_mu;
rocblas_handle g_blas[kMaxDevices] = {};

}  // namespace

hipError_t gemm_bf16_f32(const uint16_t* x, int64_t M, int64_t K, int64_t ldx, const uint16_t* w_bf16, int64_t N,
                         float* acc, hipStream_t stream, const char** why) {
  int dev = 0;
  const hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) {
    *why = "device index out of range";
    return hipErrorInvalidDevice;
  }
  std::lock_guard<std::mutex> lock(g_blas_mu);
  if (!g_blas[dev]) {
    rocblas_handle h = nullptr;
    if (rocblas_create_handle(&h) != rocblas_status_success) {
      *why = "rocblas_create_handle failed";
      return hipErrorUnknown;
    }
    if (rocblas_set_atomics_mode(h, rocblas_atomics_not_allowed) != rocblas_status_success ||
        rocblas_set_pointer_mode(h, rocblas_pointer_mode_host) != rocblas_status_success) {
      rocblas_destroy_handle(h);
      *why = "rocBLAS handle set-up failed";
      return hipErrorUnknown;
    }
    g_blas[dev] = h;
  }
  rocblas_handle h = g_blas[dev];
  if (rocblas_set_stream(h, stream) != rocblas_status_success) {
    *why = "rocblas_set_stream failed";
    return hipErrorUnknown;
  }
  const float one = 1.0f, zero = 0.0f;
  // Row-major acc[M][N] = x[M][K] * w[N][K]^T is, column-major, the N x M
  // matrix w^T (w read as K x N, transposed) times x^T (K x M, leading
  // dimension ldx).
  const rocblas_status st = rocblas_gemm_ex(
      h, rocblas_operation_transpose, rocblas_operation_none, static_cast<rocblas_int>(N),
      static_cast<rocblas_int>(M), static_cast<rocblas_int>(K), &one, w_bf16, rocblas_datatype_bf16_r,
      static_cast<rocblas_int>(K), x, rocblas_datatype_bf16_r, static_cast<rocblas_int>(ldx), &zero, acc,
      rocblas_datatype_f32_r, static_cast<rocblas_int>(N), acc, rocblas_datatype_f32_r,
      static_cast<rocblas_int>(N), rocblas_datatype_f32_r, rocblas_gemm_algo_standard, 0, 0);
  if (st != rocblas_status_success) {
    *why = rocblas_status_to_string(st);
    return hipErrorUnknown;
  }
  return hipSuccess;
}

}  // namespace w4a16
