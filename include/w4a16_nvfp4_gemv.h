/*
 * w4a16_nvfp4_gemv -- small-M BF16 x NVFP4 (W4A16) GEMV for AMD MI355X (gfx950).
 *
 * C ABI of libw4a16_nvfp4_gemv.so.  Every entry point takes plain device
 * pointers and sizes, enqueues its kernels asynchronously on `stream` (a
 * hipStream_t; NULL means the legacy default stream) and returns a status
 * code.  No entry point synchronizes the stream or aborts: a call that
 * cannot run returns a non-zero status and enqueues nothing.  No entry point
 * allocates device memory, with one exception: nvfp4_dequant_gemm runs its
 * GEMM through rocBLAS, whose handle (created on the first call on a device,
 * kept until the process ends) manages device memory of its own and may
 * grow it for larger shapes (make those calls outside HIP graph capture).
 * All buffers are owned by the caller and must
 * stay alive until the enqueued work has finished.
 *
 * Data formats (the "ModelOpt layout" of the pages vllm.models.flint.ops.
 * nvfp4_gemv, module docstring, and vllm.models.flint.ops.linear,
 * _swizzled_scale_buffer):
 *   bf16 tensors    uint16_t bit patterns of IEEE bfloat16.
 *   packed weight   uint8_t [N][K/2], two FP4 E2M1 codes per byte, the LOW
 *                   nibble holding the even k.
 *   block scales    one FP8 E4M3FN byte per 16 consecutive k of a row, in
 *                   the FLAT 128x4-swizzled buffer of
 *                   ceil(N/128)*128 * ceil(K/64)*4 bytes: 512-byte tiles of
 *                   128 rows x 4 scale columns, ordered by 128-row band and
 *                   then by column group; inside a tile, row r lives in the
 *                   16-byte chunk r%32 at byte (r/32)*4 + column%4.
 *   global scale    one FP32 value in DEVICE memory (read by the kernel).
 *
 * Numerics (nvfp4_gemv page, module docstring "Numerics"): each weight is
 * decoded exactly (e2m1 * e4m3 is always a BF16 value), products with the
 * BF16 activations are accumulated in FP32, the FP32 global scale multiplies
 * the FP32 accumulator and the result is rounded to BF16 once (round to
 * nearest even).  The FP32 summation order is unspecified.
 *
 * Shape limits shared by the GEMV entry points: 0 <= M <= W4A16_MAX_M tokens
 * (M == 0 is a successful no-op; the pages' kernels stop at 32 tokens, the
 * MFMA kernels here take up to four 16-token tiles per launch), K % 64 == 0,
 * N % 16 == 0, all sizes below 2^31.
 * Pointer alignment: activations and weights 16 bytes, scale buffers and
 * global scales 4 bytes (one 32-bit word holds a row's 4 scales of a 64-k
 * tile: the 4-byte divisibility of the moe_gemv page's fake tensor specs),
 * outputs 2 bytes; the row stride ldx of x is a multiple of 8 elements.  A
 * scale buffer that is 4- but not 16-byte aligned is served by the kernels
 * that read one scale word per row (the MFMA forms), with the same results.
 * Each of x, the weight and the scale buffer must span less than 2 GiB.
 *
 * The kernels read past-the-end rows and tiles through buffer resources that
 * return zeros, so no entry point reads outside the extents given here; the
 * results are deterministic (a fixed reduction order, no atomics).
 */
#ifndef W4A16_NVFP4_GEMV_H
#define W4A16_NVFP4_GEMV_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes. */
#define W4A16_OK 0
#define W4A16_ERR_INVALID_ARG 1   /* null pointer, negative or inconsistent size */
#define W4A16_ERR_MISALIGNED 2    /* a pointer or stride breaks the alignment rules */
#define W4A16_ERR_UNSUPPORTED 3   /* valid request outside the supported shapes */
#define W4A16_ERR_HIP 4           /* the HIP runtime refused a launch */

/* Largest token count of the GEMV entry points, and of the MoE pair.  The
 * GEMV kernels take up to 64 tokens per launch; from 65 tokens on a call
 * launches them once per 64 tokens (each launch reads the weight again),
 * which measured faster than the dequant + GEMM path up to 192 tokens. */
#define W4A16_MAX_M 192
#define W4A16_GEMV_TOKENS_PER_LAUNCH 64
#define W4A16_MOE_MAX_M 32

/*
 * nvfp4_gemv -- out[M][N] = bf16(fp32(x @ dequant(W)^T) * global_scale).
 * Defined on the nvfp4_gemv page (function nvfp4_gemv and the module
 * docstring).
 *   x            bf16 [M][ldx] (device), the first K columns are used.
 *   w            uint8 [N][K/2] packed E2M1 codes (device).
 *   w_scale      flat 128x4-swizzled E4M3 scales of the [N][K] weight (device).
 *   global_scale one FP32 value (device).
 *   silu_mul     0: out is bf16 [M][N].
 *                1: the N rows are [gate | up] halves; out is bf16 [M][N/2]
 *                   with out[m][j] = bf16(silu(g) * u), g and u the BF16
 *                   GEMV outputs of rows j and N/2 + j, SiLU in FP32.
 *                   Needs N % 32 == 0.
 *   out          bf16 output, contiguous (device).
 */
int nvfp4_gemv(const uint16_t *x, int64_t M, int64_t K, int64_t ldx,
               const uint8_t *w, const uint8_t *w_scale, const float *global_scale,
               int64_t N, int silu_mul, uint16_t *out, void *stream);

/*
 * bf16_gemv -- the same GEMV with a row-major BF16 weight w [N][K] (device)
 * and a global scale of one (nvfp4_gemv page, function bf16_gemv).
 * Arguments and limits as nvfp4_gemv, except that K % 16 == 0 suffices.
 */
int bf16_gemv(const uint16_t *x, int64_t M, int64_t K, int64_t ldx,
              const uint16_t *w, int64_t N, int silu_mul, uint16_t *out, void *stream);

/*
 * nvfp4_gemv_splitk, bf16_gemv_splitk -- the nvfp4_gemv and bf16_gemv
 * results, with a workspace that lets the library split K across
 * workgroups: the nvfp4_gemv page (module docstring) splits K across the
 * warps of a CTA and, with split > 1, across the CTAs of a cluster, reducing
 * through shared memory.  Here the workgroups of a unit of row tiles each
 * sum a K range in FP32, write the partial sums to the workspace, and the
 * last one to arrive adds them in split order (so the result does not depend
 * on timing) and applies the same epilogue (global scale, single BF16
 * rounding, silu_mul).  Used from 16 tokens on, where every workgroup would
 * otherwise stream all M*K*2 activation bytes.
 *   Arguments as nvfp4_gemv / bf16_gemv, plus:
 *   workspace        device memory owned by the caller, 256-byte aligned, of
 *                    at least gemv_splitk_workspace_bytes(...) bytes for these
 *                    sizes.  Its first 64 KiB hold per-unit arrival counters
 *                    (for every shape): they must be ZERO before the first
 *                    call (e.g. memset once after allocation), and every call
 *                    leaves them zero, so one workspace of the largest size
 *                    serves calls of any sizes.  Calls that share a workspace
 *                    must not overlap.
 *   workspace_bytes  its size.
 * When the plan for these sizes uses no split (the size query returns 0),
 * workspace may be NULL and the call is exactly nvfp4_gemv / bf16_gemv.
 * Errors as nvfp4_gemv; a missing or too small workspace returns
 * W4A16_ERR_INVALID_ARG, a workspace that is not 256-byte aligned
 * W4A16_ERR_MISALIGNED.
 * gemv_splitk_workspace_bytes(weight_fp4, ...) returns the bytes the call
 * needs on the current device (the plan depends on its compute units), 0
 * when it uses no split, and -1 for sizes the entry points reject.
 */
int64_t gemv_splitk_workspace_bytes(int weight_fp4, int64_t M, int64_t N, int64_t K, int silu_mul);
int nvfp4_gemv_splitk(const uint16_t *x, int64_t M, int64_t K, int64_t ldx,
                      const uint8_t *w, const uint8_t *w_scale, const float *global_scale,
                      int64_t N, int silu_mul, void *workspace, int64_t workspace_bytes,
                      uint16_t *out, void *stream);
int bf16_gemv_splitk(const uint16_t *x, int64_t M, int64_t K, int64_t ldx, const uint16_t *w,
                     int64_t N, int silu_mul, void *workspace, int64_t workspace_bytes,
                     uint16_t *out, void *stream);

/*
 * nvfp4_gemv_splitk_noalloc -- nvfp4_gemv_splitk for callers that cannot
 * allocate device memory (code under HIP graph capture, serving loops that
 * must not allocate, harnesses that forbid it): the same kernels and the same
 * results, with the split-K partial sums and counters in a scratch array
 * that the library holds on each GPU (W4A16_NOALLOC_SCRATCH_BYTES, created
 * with the library's code object on that device and kept until the process
 * ends).  No call allocates or frees memory.  Arguments as nvfp4_gemv.
 * All calls on one GPU share that GPU's scratch: calls that may overlap
 * (different streams without ordering between them) race and must not be
 * issued.  Every call leaves the scratch's counters zero for the next one.
 * Returns W4A16_ERR_UNSUPPORTED when the split plan for these sizes needs
 * more scratch than W4A16_NOALLOC_SCRATCH_BYTES (w4a16_last_error() gives
 * both sizes), otherwise the errors of nvfp4_gemv.
 */
#define W4A16_NOALLOC_SCRATCH_BYTES (8ll << 20)
int nvfp4_gemv_splitk_noalloc(const uint16_t *x, int64_t M, int64_t K, int64_t ldx,
                              const uint8_t *w, const uint8_t *w_scale, const float *global_scale,
                              int64_t N, int silu_mul, uint16_t *out, void *stream);

/*
 * dequantize_rows -- out[rows][K] = bf16(e2m1 * e4m3), bit-exact, global
 * scale not applied (nvfp4_gemv page, function dequantize_rows).
 * Needs rows % 16 == 0 and K % 256 == 0 (the page's assertion).
 *   w        uint8 [rows][K/2] (device), 16-byte aligned.
 *   w_scale  flat 128x4-swizzled scales of the [rows][K] weight (device).
 *   out      bf16 [rows][K] (device), 16-byte aligned.
 */
int dequantize_rows(const uint8_t *w, const uint8_t *w_scale, int64_t rows, int64_t K,
                    uint16_t *out, void *stream);

/*
 * nvfp4_dequant_gemm -- the nvfp4_gemv result for any number of tokens: the
 * weight is dequantized once into a BF16 copy (as dequantize_rows), one BLAS
 * GEMM forms the FP32 sums of x @ W^T, and the global scale is applied to
 * those sums before the single BF16 rounding (linear page, function
 * _dequant_gemm; there the scale is the GEMM's alpha).  The path beside the
 * GEMV kernels for M beyond W4A16_MAX_M.
 *   x, w, w_scale, global_scale, silu_mul, out   as nvfp4_gemv, any M >= 0;
 *                x and out need only 2-byte alignment, ldx >= K.
 *   workspace    device memory owned by the caller, 256-byte aligned, of at
 *                least nvfp4_dequant_gemm_workspace_bytes(M, N, K) bytes; it
 *                holds the BF16 weight copy and the FP32 sums, and its
 *                contents are undefined afterwards.  Calls that share a
 *                workspace must not overlap.
 *   Needs N % 16 == 0 and K % 256 == 0 (dequantize_rows), and N % 32 == 0
 *   with silu_mul.  The GEMM runs through rocBLAS: the first call on a device
 *   creates that device's rocBLAS handle, which keeps rocBLAS's own device
 *   memory until the process ends.  A GEMM failure returns W4A16_ERR_HIP.
 * nvfp4_dequant_gemm_workspace_bytes returns the workspace size in bytes
 * (-1 for negative or too large sizes).
 */
int64_t nvfp4_dequant_gemm_workspace_bytes(int64_t M, int64_t N, int64_t K);
int nvfp4_dequant_gemm(const uint16_t *x, int64_t M, int64_t K, int64_t ldx,
                       const uint8_t *w, const uint8_t *w_scale, const float *global_scale,
                       int64_t N, int silu_mul, void *workspace, int64_t workspace_bytes,
                       uint16_t *out, void *stream);

/*
 * nvfp4_unswizzle_scales -- out[n][c] = the scale of row n, column c (= k/16)
 * read from the flat 128x4-swizzled buffer; bit-exact.  Exposes the scale
 * addressing the GEMV kernels use (the 128x4 layout named on the
 * nvfp4_gemv page, nvfp4_gemv argument weight_scale).  Needs K % 16 == 0.
 *   out  uint8 [N][K/16] (device).
 */
int nvfp4_unswizzle_scales(const uint8_t *w_scale, int64_t N, int64_t K, uint8_t *out,
                           void *stream);

/*
 * moe_gate_up -- routed and shared expert gate/up projections of the MoE
 * decode block in one launch (moe_gemv page, function gate_up).
 *   x        bf16 [M][H] (device); ids int32 [M][topk] expert ids, each in
 *            [0, E) (device; not validated: ids outside the range are a
 *            caller error and are clamped into range by the kernel).
 *   w1       uint8 [E][2I][H/2]: expert e's [gate; up] rows; w1_scale holds
 *            E consecutive flat 128x4 buffers of the [2I][H] weight;
 *            alpha FP32 [E] (device).
 *   act      bf16 [M*topk][I] output: for pair p = t*topk + j and e = ids[p],
 *            act[p][i] = bf16(silu(g) * u) with g, u the FP32 accumulators of
 *            rows i and I+i of W1[e] times alpha[e] (not rounded to BF16).
 *   wsh      uint8 [2SI][H/2] shared [gate; up] weight, ssh its flat scales,
 *            gssh FP32 [1] (device).
 *   sact     bf16 [M][SI] output: the nvfp4_gemv silu_mul result of the
 *            shared expert.
 * Limits: 0 <= M <= W4A16_MOE_MAX_M (M == 0 is a no-op), 1 <= topk <= 16, E >= 1,
 * H % 64 == 0, I % 16 == 0, SI % 16 == 0.
 */
int moe_gate_up(const uint16_t *x, int64_t M, int64_t H, const int32_t *ids, int64_t topk,
                int64_t E, const uint8_t *w1, const uint8_t *w1_scale, const float *alpha,
                int64_t I, uint16_t *act, const uint8_t *wsh, const uint8_t *ssh,
                const float *gssh, int64_t SI, uint16_t *sact, void *stream);

/*
 * moe_down_combine -- top-k down projections, shared-expert down projection
 * and the weighted combine in one launch (moe_gemv page, function
 * down_combine):
 *   y_j   = bf16(act[t*topk+j] . W2[e_j][h] * alpha2[e_j])
 *   out   = bf16(bf16(sum_j tw[t][j] * y_j) + bf16(sact[t] . Wsd[h] * gssd))
 * with the sum over j in FP32.
 *   act bf16 [M*topk][I], ids int32 [M][topk], tw FP32 [M][topk] (device).
 *   w2 uint8 [E][H][I/2] with E consecutive flat scale buffers of the
 *   [H][I] weight in w2_scale; alpha2 FP32 [E].
 *   sact bf16 [M][SI]; wsd uint8 [H][SI/2], ssd its flat scales, gssd FP32 [1].
 *   out bf16 [M][H] (device).
 * Limits: as moe_gate_up, with H % 16 == 0, I % 64 == 0, SI % 64 == 0.
 */
int moe_down_combine(const uint16_t *act, const int32_t *ids, const float *tw, int64_t M,
                     int64_t topk, int64_t E, const uint8_t *w2, const uint8_t *w2_scale,
                     const float *alpha2, int64_t H, int64_t I, const uint16_t *sact,
                     const uint8_t *wsd, const uint8_t *ssd, const float *gssd, int64_t SI,
                     uint16_t *out, void *stream);

/*
 * w4a16_gemv_kernel_name -- host-only query, enqueues nothing: the name of
 * the kernel instantiation (as profilers print it, without the namespace and
 * parameter list) that nvfp4_gemv (weight_fp4 = 1) or bf16_gemv
 * (weight_fp4 = 0) launches for these sizes and silu_mul, under the current
 * W4A16_GEMV_PATH and W4A16_SPLITK settings.  Returns "" and records the reason in
 * w4a16_last_error() for sizes the entry point would reject or for M = 0.
 * The string lives in static per-thread storage until the next call.
 */
const char *w4a16_gemv_kernel_name(int weight_fp4, int64_t M, int64_t N, int64_t K, int silu_mul);
/* The same query for nvfp4_gemv_splitk / bf16_gemv_splitk. */
const char *w4a16_gemv_splitk_kernel_name(int weight_fp4, int64_t M, int64_t N, int64_t K, int silu_mul);

/* Human-readable name of a status code (static storage).  The two names are
 * the same function. */
const char *nvfp4_status_string(int status);
const char *w4a16_status_string(int status);

/* Detail of the last failed call on this host thread (static per-thread
 * storage; empty after a successful call). */
const char *w4a16_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* W4A16_NVFP4_GEMV_H */
