// Host-side interface between the C ABI (capi.cpp) and the kernel launchers.
// Arguments reaching these launchers have already been validated.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace w4a16 {

constexpr int kPathValu = 0;
constexpr int kPathMfma = 1;
constexpr int kPathBlk = 2;

struct GemvParams {
  const uint16_t* x;   // bf16 [M][ldx]
  const uint8_t* w;    // packed codes [N][K/2] or bf16 [N][K] (as bytes)
  const uint8_t* s;    // flat 128x4 scales (NVFP4), else unused
  const float* gs;     // device FP32 global scale (NVFP4), else unused
  uint16_t* out;       // bf16 [M][N] or [M][N/2]
  int64_t ldx;
  int64_t tiles;       // set by the launcher
  int64_t units;       // set by the launcher
  uint32_t x_bytes;     // byte extents of x, w and s (each below 2 GiB): the
  uint32_t w_bytes;     // kernels read them through buffer resources whose
  uint32_t s_bytes;     // out-of-range loads return zero
  int M, N, K;
  int half;            // N / 2 with silu_mul, else 0
  // Cross-workgroup split-K (MFMA kernels): FP32 partial sums and per-unit
  // arrival counters (zero between calls) in a caller-provided workspace;
  // null when the call has no workspace.
  float* part;
  uint32_t* cnt;
  uint32_t part_bytes;  // extent of part (below 2 GiB)
};

// The split-K form a GEMV call uses when it has a workspace: rt row tiles
// per unit and s workgroups per unit along K (s == 1: no split), and the
// workspace bytes that form needs (0 for s == 1).
struct SplitPlan {
  int rt, s;
  int64_t cnt_bytes;  // the counters, at the start of the workspace (kSplitCounterBytes)
  int64_t bytes;      // counters and partial sums
};
// Bytes of arrival counters at the start of every split-K workspace (one
// 32-bit counter per unit: plans with more units do not split).
constexpr int64_t kSplitCounterBytes = 65536;
SplitPlan gemv_split_plan(bool fp4, int64_t M, int64_t N, int64_t K, int silu);

// The library-owned scratch of nvfp4_gemv_splitk_noalloc (noalloc.hip): its
// device address on the current device (looked up on the first call there).
constexpr int64_t kNoAllocScratchBytes = int64_t(8) << 20;
hipError_t noalloc_scratch(void** ptr);

// The kernel family a GEMV call uses: the measured default, or the one that
// W4A16_GEMV_PATH forces where it applies.
int default_gemv_path(bool fp4, int64_t M, int64_t N, int64_t K, int silu);
int choose_gemv_path(bool fp4, int64_t M, int64_t N, int64_t K, int silu);
hipError_t launch_gemv(bool fp4, const GemvParams& p, int silu, int path, hipStream_t stream);
// Runs the GEMV dispatch without launching: writes the name of the kernel
// instantiation launch_gemv would launch for these sizes into name.
void describe_gemv(bool fp4, const GemvParams& p, int silu, int path, char* name, size_t len);

hipError_t launch_dequantize_rows(const uint8_t* w, const uint8_t* s, int64_t rows, int64_t K,
                                  uint16_t* out, hipStream_t stream);
hipError_t launch_unswizzle(const uint8_t* s, int64_t N, int64_t K, uint8_t* out,
                            hipStream_t stream);
hipError_t launch_scale_epilogue(const float* acc, const float* gs, uint16_t* out, int64_t M, int64_t N,
                                 int silu_mul, hipStream_t stream);
// out = x @ w_bf16^T as FP32 [M][N] by one BLAS GEMM (no scaling).
hipError_t gemm_bf16_f32(const uint16_t* x, int64_t M, int64_t K, int64_t ldx, const uint16_t* w_bf16, int64_t N,
                         float* acc, hipStream_t stream, const char** why);

struct MoeGateUpParams {
  const uint16_t* x;      // bf16 [M][H]
  const int32_t* ids;     // [M][topk]
  const uint8_t* w1;      // [E][2I][H/2]
  const uint8_t* w1s;     // E flat buffers
  const float* alpha;     // [E]
  uint16_t* act;          // [M*topk][I]
  const uint8_t* wsh;     // [2SI][H/2]
  const uint8_t* ssh;
  const float* gssh;      // [1]
  uint16_t* sact;         // [M][SI]
  int64_t w1_expert_bytes, s1_expert_bytes, wsh_bytes, ssh_bytes;
  int M, H, topk, E, I, SI;
  int slots_max;          // min(M * topk, E): workgroup rows of routed experts
  bool scales16;          // both scale buffers 16-byte aligned (the VALU forms need it)
};

struct MoeDownParams {
  const uint16_t* act;    // [M*topk][I]
  const int32_t* ids;     // [M][topk]
  const float* tw;        // [M][topk]
  const uint8_t* w2;      // [E][H][I/2]
  const uint8_t* w2s;
  const float* alpha2;    // [E]
  const uint16_t* sact;   // [M][SI]
  const uint8_t* wsd;     // [H][SI/2]
  const uint8_t* ssd;
  const float* gssd;      // [1]
  uint16_t* out;          // [M][H]
  int64_t w2_expert_bytes, s2_expert_bytes, wsd_bytes, ssd_bytes;
  int M, topk, E, H, I, SI;
  bool scales16;          // both scale buffers 16-byte aligned (the VALU forms need it)
};

hipError_t launch_moe_gate_up(MoeGateUpParams p, hipStream_t stream);
hipError_t launch_moe_down_combine(MoeDownParams p, hipStream_t stream);

}  // namespace w4a16
