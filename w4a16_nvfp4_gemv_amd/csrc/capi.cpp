// C ABI of the library: argument validation, path choice and launch.
// No entry point synchronizes or aborts; a call that cannot run returns a
// non-zero status and enqueues nothing.  None allocates device memory except
// nvfp4_dequant_gemm, through rocBLAS: its handle (created on the first call
// on a device, kept until the process ends) manages device memory of its own
// and may grow it for larger shapes.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <cstdio>
#include <string>

#include "w4a16_nvfp4_gemv.h"
#include "launch.hpp"

static_assert(W4A16_NOALLOC_SCRATCH_BYTES == w4a16::kNoAllocScratchBytes, "one scratch size");

namespace {

thread_local std::string g_last_error;

int fail(int status, const char* fmt, long long a = 0, long long b = 0) {
  char buf[256];
  std::snprintf(buf, sizeof buf, fmt, a, b);
  g_last_error = buf;
  return status;
}

int ok() {
  g_last_error.clear();
  return W4A16_OK;
}

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

constexpr int64_t kMaxDim = (int64_t(1) << 31) - 1;

int hip_status(hipError_t e) {
  if (e == hipSuccess) return ok();
  g_last_error = std::string("HIP launch failed: ") + hipGetErrorString(e);
  return W4A16_ERR_HIP;
}

int64_t flat_scale_bytes(int64_t n, int64_t k) {
  return (n + 127) / 128 * 128 * ((k / 16 + 3) / 4 * 4);
}

// Checks shared by the dense GEMV entry points.  Returns W4A16_OK to go on.
int check_dense(const uint16_t* x, int64_t M, int64_t K, int64_t ldx, const void* w, int64_t N,
                int silu_mul, const uint16_t* out, int64_t k_multiple) {
  if (M < 0 || K <= 0 || N <= 0 || ldx < K) return fail(W4A16_ERR_INVALID_ARG, "bad sizes M=%lld N=%lld", M, N);
  if (M > W4A16_MAX_M) return fail(W4A16_ERR_UNSUPPORTED, "M=%lld exceeds the %lld-token limit", M, W4A16_MAX_M);
  if (K > kMaxDim || N > kMaxDim || ldx > kMaxDim) return fail(W4A16_ERR_UNSUPPORTED, "size too large K=%lld N=%lld", K, N);
  if (K % k_multiple) return fail(W4A16_ERR_UNSUPPORTED, "K=%lld is not a multiple of %lld", K, k_multiple);
  if (N % 16) return fail(W4A16_ERR_UNSUPPORTED, "N=%lld is not a multiple of 16", N);
  if (silu_mul != 0 && silu_mul != 1) return fail(W4A16_ERR_INVALID_ARG, "silu_mul=%lld must be 0 or 1", silu_mul);
  if (silu_mul && N % 32) return fail(W4A16_ERR_UNSUPPORTED, "silu_mul needs N %% 32 == 0, N=%lld", N);
  if (M == 0) return ok();
  if (!x || !w || !out) return fail(W4A16_ERR_INVALID_ARG, "null pointer");
  if (!aligned(x, 16) || !aligned(w, 16) || ldx % 8) return fail(W4A16_ERR_MISALIGNED, "x/w must be 16-byte aligned, ldx %% 8 == 0 (ldx=%lld)", ldx);
  if (!aligned(out, 2)) return fail(W4A16_ERR_MISALIGNED, "out must be 2-byte aligned");
  return W4A16_OK;
}

// The dense GEMV entry points.  With `splitk`, the call may use the
// caller's workspace for the cross-workgroup split-K form (the plan for these
// sizes says whether and how much).
int run_gemv(bool fp4, const uint16_t* x, int64_t M, int64_t K, int64_t ldx, const void* w, const uint8_t* w_scale,
             const float* global_scale, int64_t N, int silu_mul, void* workspace, int64_t workspace_bytes,
             bool splitk, uint16_t* out, void* stream) {
  int st = check_dense(x, M, K, ldx, w, N, silu_mul, out, fp4 ? 64 : 16);
  if (st != W4A16_OK || M == 0) return st;
  if (fp4) {
    if (!w_scale || !global_scale) return fail(W4A16_ERR_INVALID_ARG, "null scale pointer");
    if (!aligned(w_scale, 4) || !aligned(global_scale, 4))
      return fail(W4A16_ERR_MISALIGNED, "w_scale and global_scale must be 4-byte aligned");
  }
  const int64_t w_bytes = fp4 ? N * (K / 2) : N * K * 2, s_bytes = fp4 ? flat_scale_bytes(N, K) : 0;
  const int64_t x_bytes = ((M - 1) * ldx + K) * 2;
  if (w_bytes > kMaxDim || s_bytes > kMaxDim || x_bytes > kMaxDim)
    return fail(W4A16_ERR_UNSUPPORTED, "tensors above 2 GiB are not supported (weight %lld bytes)", w_bytes);
  w4a16::GemvParams p{};
  p.x = x;
  p.w = static_cast<const uint8_t*>(w);
  p.s = fp4 ? w_scale : nullptr;
  p.gs = fp4 ? global_scale : nullptr;
  p.x_bytes = static_cast<uint32_t>(x_bytes);
  p.w_bytes = static_cast<uint32_t>(w_bytes);
  p.s_bytes = static_cast<uint32_t>(s_bytes);
  p.out = out;
  p.ldx = ldx;
  p.M = static_cast<int>(M);
  p.N = static_cast<int>(N);
  p.K = static_cast<int>(K);
  p.half = silu_mul ? static_cast<int>(N / 2) : 0;
  if (splitk) {
    const int64_t m_launch = M < W4A16_GEMV_TOKENS_PER_LAUNCH ? M : W4A16_GEMV_TOKENS_PER_LAUNCH;
    const w4a16::SplitPlan plan = w4a16::gemv_split_plan(fp4, m_launch, N, K, silu_mul);
    if (plan.s > 1) {
      if (!workspace) return fail(W4A16_ERR_INVALID_ARG, "null workspace (%lld bytes needed)", plan.bytes);
      if (workspace_bytes < plan.bytes)
        return fail(W4A16_ERR_INVALID_ARG, "workspace of %lld bytes, %lld needed", workspace_bytes, plan.bytes);
      if (!aligned(workspace, 256)) return fail(W4A16_ERR_MISALIGNED, "the workspace must be 256-byte aligned");
      if (plan.bytes > kMaxDim) return fail(W4A16_ERR_UNSUPPORTED, "split-K workspace above 2 GiB (%lld bytes)", plan.bytes);
      p.cnt = static_cast<uint32_t*>(workspace);
      p.part = reinterpret_cast<float*>(static_cast<char*>(workspace) + plan.cnt_bytes);
      p.part_bytes = static_cast<uint32_t>(plan.bytes - plan.cnt_bytes);
    }
  }
  // The VALU kernels read a quad's scale words as one 16-byte chunk; a scale
  // buffer that is only 4-byte aligned goes to the MFMA kernels, which read
  // one 4-byte word per row.
  const bool s16 = !fp4 || aligned(w_scale, 16);
  // Beyond 64 tokens, one launch per 64 tokens (stream-ordered, so the
  // split-K form's counters are free again for the next launch).
  const int64_t n_out = silu_mul ? N / 2 : N;
  for (int64_t m0 = 0; m0 < M; m0 += W4A16_GEMV_TOKENS_PER_LAUNCH) {
    const int64_t mc = M - m0 < W4A16_GEMV_TOKENS_PER_LAUNCH ? M - m0 : W4A16_GEMV_TOKENS_PER_LAUNCH;
    w4a16::GemvParams q = p;
    q.x = x + m0 * ldx;
    q.x_bytes = static_cast<uint32_t>(((mc - 1) * ldx + K) * 2);
    q.out = out + m0 * n_out;
    q.M = static_cast<int>(mc);
    const int path = s16 ? w4a16::choose_gemv_path(fp4, mc, N, K, silu_mul) : w4a16::kPathMfma;
    const int st2 = hip_status(w4a16::launch_gemv(fp4, q, silu_mul, path, static_cast<hipStream_t>(stream)));
    if (st2 != W4A16_OK) return st2;
  }
  return W4A16_OK;
}

const char* gemv_kernel_name_of(int weight_fp4, int64_t M, int64_t N, int64_t K, int silu_mul, bool splitk) {
  thread_local char name[128];
  name[0] = 0;
  if (weight_fp4 != 0 && weight_fp4 != 1) {
    fail(W4A16_ERR_INVALID_ARG, "weight_fp4=%lld must be 0 or 1", weight_fp4);
    return name;
  }
  // the size checks of the GEMV entry points, on stand-in aligned pointers
  const uint16_t* stand_in = reinterpret_cast<const uint16_t*>(uintptr_t(256));
  const int st = check_dense(stand_in, M, K, K, stand_in, N, silu_mul, reinterpret_cast<uint16_t*>(uintptr_t(256)),
                             weight_fp4 ? 64 : 16);
  if (st != W4A16_OK) return name;
  if (M == 0) {
    fail(W4A16_ERR_INVALID_ARG, "M=0 launches no kernel");
    return name;
  }
  // the kernel of the first launch (calls past 64 tokens launch once per 64)
  const int64_t m_launch = M < W4A16_GEMV_TOKENS_PER_LAUNCH ? M : W4A16_GEMV_TOKENS_PER_LAUNCH;
  w4a16::GemvParams p{};
  p.ldx = K;
  p.M = static_cast<int>(m_launch);
  p.N = static_cast<int>(N);
  p.K = static_cast<int>(K);
  p.half = silu_mul ? static_cast<int>(N / 2) : 0;
  const bool fp4 = weight_fp4 != 0;
  if (splitk && w4a16::gemv_split_plan(fp4, m_launch, N, K, silu_mul).s > 1) {
    // a stand-in workspace: the dispatch only checks that there is one
    p.part = reinterpret_cast<float*>(uintptr_t(256));
    p.cnt = reinterpret_cast<uint32_t*>(uintptr_t(256));
  }
  w4a16::describe_gemv(fp4, p, silu_mul, w4a16::choose_gemv_path(fp4, m_launch, N, K, silu_mul), name, sizeof name);
  ok();
  return name;
}


}  // namespace

extern "C" {

const char* w4a16_status_string(int status) {
  switch (status) {
    case W4A16_OK: return "ok";
    case W4A16_ERR_INVALID_ARG: return "invalid argument";
    case W4A16_ERR_MISALIGNED: return "misaligned pointer or stride";
    case W4A16_ERR_UNSUPPORTED: return "unsupported shape";
    case W4A16_ERR_HIP: return "HIP runtime error";
    default: return "unknown status";
  }
}

const char* nvfp4_status_string(int status) { return w4a16_status_string(status); }

const char* w4a16_last_error(void) { return g_last_error.c_str(); }

int nvfp4_gemv(const uint16_t* x, int64_t M, int64_t K, int64_t ldx, const uint8_t* w,
               const uint8_t* w_scale, const float* global_scale, int64_t N, int silu_mul,
               uint16_t* out, void* stream) {
  return run_gemv(true, x, M, K, ldx, w, w_scale, global_scale, N, silu_mul, nullptr, 0, false, out, stream);
}

int bf16_gemv(const uint16_t* x, int64_t M, int64_t K, int64_t ldx, const uint16_t* w, int64_t N,
              int silu_mul, uint16_t* out, void* stream) {
  return run_gemv(false, x, M, K, ldx, w, nullptr, nullptr, N, silu_mul, nullptr, 0, false, out, stream);
}

int64_t gemv_splitk_workspace_bytes(int weight_fp4, int64_t M, int64_t N, int64_t K, int silu_mul) {
  if (weight_fp4 != 0 && weight_fp4 != 1) return -1;
  const uint16_t* stand_in = reinterpret_cast<const uint16_t*>(uintptr_t(256));
  if (check_dense(stand_in, M, K, K, stand_in, N, silu_mul, reinterpret_cast<uint16_t*>(uintptr_t(256)),
                  weight_fp4 ? 64 : 16) != W4A16_OK)
    return -1;
  ok();
  const int64_t m_launch = M < W4A16_GEMV_TOKENS_PER_LAUNCH ? M : W4A16_GEMV_TOKENS_PER_LAUNCH;
  return M == 0 ? 0 : w4a16::gemv_split_plan(weight_fp4 != 0, m_launch, N, K, silu_mul).bytes;
}

int nvfp4_gemv_splitk(const uint16_t* x, int64_t M, int64_t K, int64_t ldx, const uint8_t* w,
                      const uint8_t* w_scale, const float* global_scale, int64_t N, int silu_mul,
                      void* workspace, int64_t workspace_bytes, uint16_t* out, void* stream) {
  return run_gemv(true, x, M, K, ldx, w, w_scale, global_scale, N, silu_mul, workspace, workspace_bytes, true, out,
                  stream);
}

int nvfp4_gemv_splitk_noalloc(const uint16_t* x, int64_t M, int64_t K, int64_t ldx, const uint8_t* w,
                              const uint8_t* w_scale, const float* global_scale, int64_t N, int silu_mul,
                              uint16_t* out, void* stream) {
  // the size checks of the GEMV entry points first (stand-in pointers), so
  // that the plan below is computed for valid sizes only
  const uint16_t* stand_in = reinterpret_cast<const uint16_t*>(uintptr_t(256));
  int st = check_dense(stand_in, M, K, K, stand_in, N, silu_mul, reinterpret_cast<uint16_t*>(uintptr_t(256)), 64);
  if (st != W4A16_OK || M == 0) return st;
  const int64_t m_launch = M < W4A16_GEMV_TOKENS_PER_LAUNCH ? M : W4A16_GEMV_TOKENS_PER_LAUNCH;
  const int64_t need = w4a16::gemv_split_plan(true, m_launch, N, K, silu_mul).bytes;
  if (need > W4A16_NOALLOC_SCRATCH_BYTES)
    return fail(W4A16_ERR_UNSUPPORTED, "the split-K plan needs %lld bytes of scratch, the library holds %lld", need,
                W4A16_NOALLOC_SCRATCH_BYTES);
  void* scratch = nullptr;
  if (need > 0) {
    const hipError_t e = w4a16::noalloc_scratch(&scratch);
    if (e != hipSuccess) return hip_status(e);
  }
  return run_gemv(true, x, M, K, ldx, w, w_scale, global_scale, N, silu_mul, scratch, W4A16_NOALLOC_SCRATCH_BYTES,
                  true, out, stream);
}

int bf16_gemv_splitk(const uint16_t* x, int64_t M, int64_t K, int64_t ldx, const uint16_t* w, int64_t N,
                     int silu_mul, void* workspace, int64_t workspace_bytes, uint16_t* out, void* stream) {
  return run_gemv(false, x, M, K, ldx, w, nullptr, nullptr, N, silu_mul, workspace, workspace_bytes, true, out,
                  stream);
}

const char* w4a16_gemv_kernel_name(int weight_fp4, int64_t M, int64_t N, int64_t K, int silu_mul) {
  return gemv_kernel_name_of(weight_fp4, M, N, K, silu_mul, false);
}

const char* w4a16_gemv_splitk_kernel_name(int weight_fp4, int64_t M, int64_t N, int64_t K, int silu_mul) {
  return gemv_kernel_name_of(weight_fp4, M, N, K, silu_mul, true);
}


int dequantize_rows(const uint8_t* w, const uint8_t* w_scale, int64_t rows, int64_t K,
                    uint16_t* out, void* stream) {
  if (rows < 0 || K <= 0) return fail(W4A16_ERR_INVALID_ARG, "bad sizes rows=%lld K=%lld", rows, K);
  if (rows % 16 || K % 256) return fail(W4A16_ERR_UNSUPPORTED, "needs rows %% 16 == 0 and K %% 256 == 0 (rows=%lld K=%lld)", rows, K);
  if (rows > kMaxDim || K > kMaxDim) return fail(W4A16_ERR_UNSUPPORTED, "size too large");
  if (rows == 0) return ok();
  if (!w || !w_scale || !out) return fail(W4A16_ERR_INVALID_ARG, "null pointer");
  if (!aligned(w, 16) || !aligned(out, 16) || !aligned(w_scale, 4)) return fail(W4A16_ERR_MISALIGNED, "w/out 16-byte, w_scale 4-byte alignment required");
  return hip_status(w4a16::launch_dequantize_rows(w, w_scale, rows, K, out, static_cast<hipStream_t>(stream)));
}

int64_t nvfp4_dequant_gemm_workspace_bytes(int64_t M, int64_t N, int64_t K) {
  if (M < 0 || N < 0 || K < 0 || M > kMaxDim || N > kMaxDim || K > kMaxDim) return -1;
  return (N * K * 2 + 255) / 256 * 256 + M * N * 4;
}

int nvfp4_dequant_gemm(const uint16_t* x, int64_t M, int64_t K, int64_t ldx, const uint8_t* w,
                       const uint8_t* w_scale, const float* global_scale, int64_t N, int silu_mul,
                       void* workspace, int64_t workspace_bytes, uint16_t* out, void* stream) {
  if (M < 0 || K <= 0 || N <= 0 || ldx < K) return fail(W4A16_ERR_INVALID_ARG, "bad sizes M=%lld N=%lld", M, N);
  if (silu_mul != 0 && silu_mul != 1) return fail(W4A16_ERR_INVALID_ARG, "silu_mul must be 0 or 1");
  if (N % 16 || K % 256) return fail(W4A16_ERR_UNSUPPORTED, "needs N %% 16 == 0 and K %% 256 == 0 (N=%lld K=%lld)", N, K);
  if (silu_mul && N % 32) return fail(W4A16_ERR_UNSUPPORTED, "silu_mul needs N %% 32 == 0 (N=%lld)", N);
  if (M > kMaxDim || N > kMaxDim || K > kMaxDim || ldx > kMaxDim || M * ldx > kMaxDim)
    return fail(W4A16_ERR_UNSUPPORTED, "size too large (M=%lld N=%lld)", M, N);
  if (M == 0) return ok();
  if (!x || !w || !w_scale || !global_scale || !workspace || !out) return fail(W4A16_ERR_INVALID_ARG, "null pointer");
  if (workspace_bytes < nvfp4_dequant_gemm_workspace_bytes(M, N, K))
    return fail(W4A16_ERR_INVALID_ARG, "workspace of %lld bytes, %lld needed", workspace_bytes,
                nvfp4_dequant_gemm_workspace_bytes(M, N, K));
  if (!aligned(x, 2) || !aligned(out, 2) || !aligned(w, 16) || !aligned(w_scale, 4) || !aligned(global_scale, 4) ||
      !aligned(workspace, 256))
    return fail(W4A16_ERR_MISALIGNED, "x/out 2-byte, w 16-byte, w_scale 4-byte, workspace 256-byte alignment required");
  const hipStream_t st = static_cast<hipStream_t>(stream);
  uint16_t* w_bf16 = static_cast<uint16_t*>(workspace);
  float* acc = reinterpret_cast<float*>(static_cast<char*>(workspace) + (N * K * 2 + 255) / 256 * 256);
  int status = hip_status(w4a16::launch_dequantize_rows(w, w_scale, N, K, w_bf16, st));
  if (status != W4A16_OK) return status;
  const char* why = "library GEMM failed";
  const hipError_t e = w4a16::gemm_bf16_f32(x, M, K, ldx, w_bf16, N, acc, st, &why);
  if (e != hipSuccess) {
    g_last_error = std::string("GEMM: ") + why;
    return W4A16_ERR_HIP;
  }
  return hip_status(w4a16::launch_scale_epilogue(acc, global_scale, out, M, N, silu_mul, st));
}

int nvfp4_unswizzle_scales(const uint8_t* w_scale, int64_t N, int64_t K, uint8_t* out,
                           void* stream) {
  if (N < 0 || K <= 0) return fail(W4A16_ERR_INVALID_ARG, "bad sizes N=%lld K=%lld", N, K);
  if (K % 16) return fail(W4A16_ERR_UNSUPPORTED, "K=%lld is not a multiple of 16", K);
  if (N > kMaxDim || K > kMaxDim) return fail(W4A16_ERR_UNSUPPORTED, "size too large");
  if (N == 0) return ok();
  if (!w_scale || !out) return fail(W4A16_ERR_INVALID_ARG, "null pointer");
  return hip_status(w4a16::launch_unswizzle(w_scale, N, K, out, static_cast<hipStream_t>(stream)));
}

int moe_gate_up(const uint16_t* x, int64_t M, int64_t H, const int32_t* ids, int64_t topk,
                int64_t E, const uint8_t* w1, const uint8_t* w1_scale, const float* alpha,
                int64_t I, uint16_t* act, const uint8_t* wsh, const uint8_t* ssh,
                const float* gssh, int64_t SI, uint16_t* sact, void* stream) {
  if (M < 0 || H <= 0 || topk <= 0 || E <= 0 || I <= 0 || SI <= 0) return fail(W4A16_ERR_INVALID_ARG, "bad sizes M=%lld H=%lld", M, H);
  if (M > W4A16_MOE_MAX_M || topk > 16) return fail(W4A16_ERR_UNSUPPORTED, "M=%lld topk=%lld outside limits", M, topk);
  if (H % 64 || I % 16 || SI % 16) return fail(W4A16_ERR_UNSUPPORTED, "needs H %% 64, I %% 16, SI %% 16 == 0 (H=%lld I=%lld)", H, I);
  if (H > kMaxDim || I > kMaxDim / 2 || SI > kMaxDim / 2 || E > kMaxDim) return fail(W4A16_ERR_UNSUPPORTED, "size too large");
  if (M == 0) return ok();
  if (!x || !ids || !w1 || !w1_scale || !alpha || !act || !wsh || !ssh || !gssh || !sact) return fail(W4A16_ERR_INVALID_ARG, "null pointer");
  if (!aligned(x, 16) || !aligned(w1, 16) || !aligned(wsh, 16) || !aligned(w1_scale, 4) || !aligned(ssh, 4))
    return fail(W4A16_ERR_MISALIGNED, "x and weights must be 16-byte aligned, scales 4-byte aligned");
  if (!aligned(ids, 4) || !aligned(alpha, 4) || !aligned(gssh, 4) || !aligned(act, 2) || !aligned(sact, 2))
    return fail(W4A16_ERR_MISALIGNED, "misaligned ids/alpha/outputs");
  w4a16::MoeGateUpParams p{};
  p.x = x;
  p.ids = ids;
  p.w1 = w1;
  p.w1s = w1_scale;
  p.alpha = alpha;
  p.act = act;
  p.wsh = wsh;
  p.ssh = ssh;
  p.gssh = gssh;
  p.sact = sact;
  p.w1_expert_bytes = 2 * I * (H / 2);
  p.s1_expert_bytes = flat_scale_bytes(2 * I, H);
  p.wsh_bytes = 2 * SI * (H / 2);
  p.ssh_bytes = flat_scale_bytes(2 * SI, H);
  if (p.w1_expert_bytes > kMaxDim || p.s1_expert_bytes > kMaxDim || p.wsh_bytes > kMaxDim ||
      M * H * 2 > kMaxDim || M * topk * I * 2 > kMaxDim)
    return fail(W4A16_ERR_UNSUPPORTED, "per-expert weights and activations must stay below 2 GiB (H=%lld I=%lld)", H, I);
  p.M = static_cast<int>(M);
  p.H = static_cast<int>(H);
  p.topk = static_cast<int>(topk);
  p.E = static_cast<int>(E);
  p.I = static_cast<int>(I);
  p.SI = static_cast<int>(SI);
  p.scales16 = aligned(w1_scale, 16) && aligned(ssh, 16);
  return hip_status(w4a16::launch_moe_gate_up(p, static_cast<hipStream_t>(stream)));
}

int moe_down_combine(const uint16_t* act, const int32_t* ids, const float* tw, int64_t M,
                     int64_t topk, int64_t E, const uint8_t* w2, const uint8_t* w2_scale,
                     const float* alpha2, int64_t H, int64_t I, const uint16_t* sact,
                     const uint8_t* wsd, const uint8_t* ssd, const float* gssd, int64_t SI,
                     uint16_t* out, void* stream) {
  if (M < 0 || H <= 0 || topk <= 0 || E <= 0 || I <= 0 || SI <= 0) return fail(W4A16_ERR_INVALID_ARG, "bad sizes M=%lld H=%lld", M, H);
  if (M > W4A16_MOE_MAX_M || topk > 16) return fail(W4A16_ERR_UNSUPPORTED, "M=%lld topk=%lld outside limits", M, topk);
  if (H % 16 || I % 64 || SI % 64) return fail(W4A16_ERR_UNSUPPORTED, "needs H %% 16, I %% 64, SI %% 64 == 0 (I=%lld SI=%lld)", I, SI);
  if (H > kMaxDim || I > kMaxDim || SI > kMaxDim || E > kMaxDim) return fail(W4A16_ERR_UNSUPPORTED, "size too large");
  if (M == 0) return ok();
  if (!act || !ids || !tw || !w2 || !w2_scale || !alpha2 || !sact || !wsd || !ssd || !gssd || !out)
    return fail(W4A16_ERR_INVALID_ARG, "null pointer");
  if (!aligned(act, 16) || !aligned(sact, 16) || !aligned(w2, 16) || !aligned(wsd, 16) || !aligned(w2_scale, 4) ||
      !aligned(ssd, 4))
    return fail(W4A16_ERR_MISALIGNED, "activations and weights must be 16-byte aligned, scales 4-byte aligned");
  if (!aligned(ids, 4) || !aligned(tw, 4) || !aligned(alpha2, 4) || !aligned(gssd, 4) || !aligned(out, 2))
    return fail(W4A16_ERR_MISALIGNED, "misaligned ids/tw/alpha2/out");
  w4a16::MoeDownParams p{};
  p.act = act;
  p.ids = ids;
  p.tw = tw;
  p.w2 = w2;
  p.w2s = w2_scale;
  p.alpha2 = alpha2;
  p.sact = sact;
  p.wsd = wsd;
  p.ssd = ssd;
  p.gssd = gssd;
  p.out = out;
  p.w2_expert_bytes = H * (I / 2);
  p.s2_expert_bytes = flat_scale_bytes(H, I);
  p.wsd_bytes = H * (SI / 2);
  p.ssd_bytes = flat_scale_bytes(H, SI);
  if (p.w2_expert_bytes > kMaxDim || p.s2_expert_bytes > kMaxDim || p.wsd_bytes > kMaxDim ||
      M * topk * I * 2 > kMaxDim || M * SI * 2 > kMaxDim)
    return fail(W4A16_ERR_UNSUPPORTED, "per-expert weights and activations must stay below 2 GiB (H=%lld I=%lld)", H, I);
  p.M = static_cast<int>(M);
  p.topk = static_cast<int>(topk);
  p.E = static_cast<int>(E);
  p.H = static_cast<int>(H);
  p.I = static_cast<int>(I);
  p.SI = static_cast<int>(SI);
  p.scales16 = aligned(w2_scale, 16) && aligned(ssd, 16);
  return hip_status(w4a16::launch_moe_down_combine(p, static_cast<hipStream_t>(stream)));
}

}  // extern "C"
