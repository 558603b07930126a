"""Python binding of the HIP library: argument marshalling only.

Each op checks dtypes and devices, allocates the outputs the pages' ops
return (nvfp4_gemv, bf16_gemv, dequantize_rows), and calls the C entry point
of the same name on the current HIP stream.  Every step of the computation
runs in the library's kernels; a non-zero status raises W4A16Error.
Signatures follow the pages (vllm.models.flint.ops.nvfp4_gemv and
vllm.models.flint.ops.moe_gemv); `pdl` is accepted for API parity and has
no effect (there is no programmatic dependent launch on ROCm).
"""
from __future__ import annotations

import torch

from . import _lib


class W4A16Error(ValueError):
    def __init__(self, status: int, op: str):
        lib = _lib.load()
        msg = lib.w4a16_status_string(status).decode()
        detail = lib.w4a16_last_error().decode()
        super().__init__(f"{op}: {msg} ({detail})")
        self.status = status


def _check(status: int, op: str) -> None:
    if status != 0:
        raise W4A16Error(status, op)


def _stream(t: torch.Tensor) -> int:
    return torch.cuda.current_stream(t.device).cuda_stream


def _flat_u8(t: torch.Tensor) -> torch.Tensor:
    """The contiguous byte storage behind a scale tensor (uint8 or float8_e4m3fn)."""
    if t.dtype != torch.uint8:
        t = t.view(torch.uint8)
    if not t.is_contiguous():
        raise ValueError("scale tensors must be contiguous flat 128x4-swizzled buffers")
    return t.reshape(-1)


def _x2d(x: torch.Tensor) -> torch.Tensor:
    if x.dtype != torch.bfloat16:
        raise ValueError(f"activations must be bfloat16, got {x.dtype}")
    if x.dim() != 2 or x.stride(1) != 1:
        raise ValueError("activations must be 2-D with unit inner stride")
    return x


def nvfp4_gemv(x: torch.Tensor, weight: torch.Tensor, weight_scale: torch.Tensor,
               global_scale: torch.Tensor, silu_mul: bool = False, pdl: bool = True) -> torch.Tensor:
    """bf16(fp32(x @ dequant(weight).T) * global_scale); [M, N/2] silu(gate)*up with silu_mul."""
    x = _x2d(x)
    if weight.dtype != torch.uint8 or weight.dim() != 2 or not weight.is_contiguous():
        raise ValueError("weight must be a contiguous uint8 [N, K/2] tensor")
    m, k = x.shape[0], weight.shape[1] * 2
    if x.shape[1] < k:
        raise ValueError(f"x has {x.shape[1]} columns, the weight needs K={k}")
    n = weight.shape[0]
    gs = global_scale.reshape(1)
    if gs.dtype != torch.float32:
        raise ValueError("global_scale must be float32")
    scale = _flat_u8(weight_scale)
    out = torch.empty((m, n // 2 if silu_mul else n), dtype=torch.bfloat16, device=x.device)
    st = _lib.load().nvfp4_gemv(x.data_ptr(), m, k, x.stride(0), weight.data_ptr(), scale.data_ptr(),
                                gs.data_ptr(), n, int(bool(silu_mul)), out.data_ptr(), _stream(x))
    _check(st, "nvfp4_gemv")
    return out


def bf16_gemv(x: torch.Tensor, weight: torch.Tensor, silu_mul: bool = False,
              pdl: bool = True) -> torch.Tensor:
    """x @ weight.T with FP32 accumulation, one BF16 rounding (same kernels, scale one)."""
    x = _x2d(x)
    if weight.dtype != torch.bfloat16 or weight.dim() != 2 or not weight.is_contiguous():
        raise ValueError("weight must be a contiguous bfloat16 [N, K] tensor")
    m, k = x.shape[0], weight.shape[1]
    if x.shape[1] < k:
        raise ValueError(f"x has {x.shape[1]} columns, the weight needs K={k}")
    n = weight.shape[0]
    out = torch.empty((m, n // 2 if silu_mul else n), dtype=torch.bfloat16, device=x.device)
    st = _lib.load().bf16_gemv(x.data_ptr(), m, k, x.stride(0), weight.data_ptr(), n,
                               int(bool(silu_mul)), out.data_ptr(), _stream(x))
    _check(st, "bf16_gemv")
    return out


def gemv_splitk_workspace(m: int, n: int, k: int, silu_mul: bool = False, weight_fp4: bool = True,
                          device="cuda") -> torch.Tensor:
    """A zero-filled workspace for nvfp4_gemv_splitk / bf16_gemv_splitk at
    these sizes (at least 256 bytes, so that one buffer also serves calls
    whose plan uses no split).  Every call leaves its counters zero, so the
    buffer can be reused by calls that do not overlap."""
    nbytes = _lib.load().gemv_splitk_workspace_bytes(int(weight_fp4), m, n, k, int(bool(silu_mul)))
    if nbytes < 0:
        raise W4A16Error(1, "gemv_splitk_workspace_bytes")
    return torch.zeros(max(nbytes, 256), dtype=torch.uint8, device=device)


def _workspace(ws: torch.Tensor):
    if ws.dtype != torch.uint8 or not ws.is_contiguous():
        raise ValueError("the workspace must be a contiguous uint8 tensor")
    return ws.data_ptr(), ws.numel()


def nvfp4_gemv_splitk(x: torch.Tensor, weight: torch.Tensor, weight_scale: torch.Tensor,
                      global_scale: torch.Tensor, silu_mul: bool = False,
                      workspace: torch.Tensor | None = None) -> torch.Tensor:
    """nvfp4_gemv with a workspace for the cross-workgroup K split (a fresh
    zeroed one when none is given)."""
    x = _x2d(x)
    if weight.dtype != torch.uint8 or weight.dim() != 2 or not weight.is_contiguous():
        raise ValueError("weight must be a contiguous uint8 [N, K/2] tensor")
    m, k = x.shape[0], weight.shape[1] * 2
    if x.shape[1] < k:
        raise ValueError(f"x has {x.shape[1]} columns, the weight needs K={k}")
    n = weight.shape[0]
    gs = global_scale.reshape(1)
    if gs.dtype != torch.float32:
        raise ValueError("global_scale must be float32")
    scale = _flat_u8(weight_scale)
    if workspace is None:
        workspace = gemv_splitk_workspace(m, n, k, silu_mul, True, x.device)
    wp, wn = _workspace(workspace)
    out = torch.empty((m, n // 2 if silu_mul else n), dtype=torch.bfloat16, device=x.device)
    st = _lib.load().nvfp4_gemv_splitk(x.data_ptr(), m, k, x.stride(0), weight.data_ptr(), scale.data_ptr(),
                                       gs.data_ptr(), n, int(bool(silu_mul)), wp, wn, out.data_ptr(), _stream(x))
    _check(st, "nvfp4_gemv_splitk")
    return out


def bf16_gemv_splitk(x: torch.Tensor, weight: torch.Tensor, silu_mul: bool = False,
                     workspace: torch.Tensor | None = None) -> torch.Tensor:
    """bf16_gemv with a workspace for the cross-workgroup K split."""
    x = _x2d(x)
    if weight.dtype != torch.bfloat16 or weight.dim() != 2 or not weight.is_contiguous():
        raise ValueError("weight must be a contiguous bfloat16 [N, K] tensor")
    m, k = x.shape[0], weight.shape[1]
    if x.shape[1] < k:
        raise ValueError(f"x has {x.shape[1]} columns, the weight needs K={k}")
    n = weight.shape[0]
    if workspace is None:
        workspace = gemv_splitk_workspace(m, n, k, silu_mul, False, x.device)
    wp, wn = _workspace(workspace)
    out = torch.empty((m, n // 2 if silu_mul else n), dtype=torch.bfloat16, device=x.device)
    st = _lib.load().bf16_gemv_splitk(x.data_ptr(), m, k, x.stride(0), weight.data_ptr(), n, int(bool(silu_mul)),
                                      wp, wn, out.data_ptr(), _stream(x))
    _check(st, "bf16_gemv_splitk")
    return out


def dequant_gemm(x: torch.Tensor, weight: torch.Tensor, weight_scale: torch.Tensor,
                 global_scale: torch.Tensor, silu_mul: bool = False) -> torch.Tensor:
    """The nvfp4_gemv result for any number of tokens, by dequantize + library GEMM."""
    x = _x2d(x)
    if weight.dtype != torch.uint8 or weight.dim() != 2 or not weight.is_contiguous():
        raise ValueError("weight must be a contiguous uint8 [N, K/2] tensor")
    m, k = x.shape[0], weight.shape[1] * 2
    if x.shape[1] < k:
        raise ValueError(f"x has {x.shape[1]} columns, the weight needs K={k}")
    n = weight.shape[0]
    gs = global_scale.reshape(1)
    if gs.dtype != torch.float32:
        raise ValueError("global_scale must be float32")
    scale = _flat_u8(weight_scale)
    lib = _lib.load()
    ws_bytes = lib.nvfp4_dequant_gemm_workspace_bytes(m, n, k)
    if ws_bytes < 0:
        raise ValueError(f"sizes out of range (M={m} N={n} K={k})")
    workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=x.device)
    out = torch.empty((m, n // 2 if silu_mul else n), dtype=torch.bfloat16, device=x.device)
    st = lib.nvfp4_dequant_gemm(x.data_ptr(), m, k, x.stride(0), weight.data_ptr(), scale.data_ptr(), gs.data_ptr(),
                                n, int(bool(silu_mul)), workspace.data_ptr(), ws_bytes, out.data_ptr(), _stream(x))
    _check(st, "nvfp4_dequant_gemm")
    return out


def dequantize_rows(weight: torch.Tensor, weight_scale: torch.Tensor) -> torch.Tensor:
    """Exact BF16 e2m1 * e4m3 of every weight row (global scale not applied)."""
    if weight.dtype != torch.uint8 or weight.dim() != 2 or not weight.is_contiguous():
        raise ValueError("weight must be a contiguous uint8 [rows, K/2] tensor")
    rows, k = weight.shape[0], weight.shape[1] * 2
    scale = _flat_u8(weight_scale)
    out = torch.empty((rows, k), dtype=torch.bfloat16, device=weight.device)
    st = _lib.load().dequantize_rows(weight.data_ptr(), scale.data_ptr(), rows, k, out.data_ptr(),
                                     _stream(weight))
    _check(st, "dequantize_rows")
    return out


def nvfp4_unswizzle_scales(weight_scale: torch.Tensor, n: int, k: int) -> torch.Tensor:
    """Logical [n, k/16] E4M3 scale bytes read from the flat 128x4 buffer."""
    scale = _flat_u8(weight_scale)
    out = torch.empty((n, k // 16), dtype=torch.uint8, device=scale.device)
    st = _lib.load().nvfp4_unswizzle_scales(scale.data_ptr(), n, k, out.data_ptr(), _stream(scale))
    _check(st, "nvfp4_unswizzle_scales")
    return out


def gemv_kernel_name(m: int, n: int, k: int, silu_mul: bool = False, weight_fp4: bool = True,
                     splitk: bool = False) -> str:
    """Name of the kernel nvfp4_gemv (or bf16_gemv; with splitk the _splitk
    entry points) launches for these sizes (host-only query; raises
    W4A16Error for sizes the entry point rejects)."""
    lib = _lib.load()
    query = lib.w4a16_gemv_splitk_kernel_name if splitk else lib.w4a16_gemv_kernel_name
    name = query(int(weight_fp4), m, n, k, int(silu_mul)).decode()
    if not name:
        raise W4A16Error(1, "gemv_kernel_name")
    return name


def moe_gate_up(x, ids, w1, w1_sf, alpha, act, wsh, ssh, gssh, sact) -> None:
    """act[p] = silu(g) * u of the routed experts, sact[t] of the shared one (in place)."""
    x = _x2d(x)
    m, h = x.shape
    topk = ids.shape[1]
    e, two_i, _ = w1.shape
    inter = two_i // 2
    si = wsh.shape[0] // 2
    for name, t, dt in (("ids", ids, torch.int32), ("alpha", alpha, torch.float32),
                        ("gssh", gssh, torch.float32), ("act", act, torch.bfloat16),
                        ("sact", sact, torch.bfloat16), ("w1", w1, torch.uint8)):
        if t.dtype != dt or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous {dt} tensor")
    if tuple(act.shape) != (m * topk, inter) or tuple(sact.shape) != (m, si):
        raise ValueError("act must be [M*topk, I] and sact [M, SI]")
    wsh_u8 = wsh.view(torch.uint8)
    st = _lib.load().moe_gate_up(x.data_ptr(), m, h, ids.data_ptr(), topk, e, w1.data_ptr(),
                                 _flat_u8(w1_sf).data_ptr(), alpha.data_ptr(), inter,
                                 act.data_ptr(), wsh_u8.data_ptr(), _flat_u8(ssh).data_ptr(),
                                 gssh.data_ptr(), si, sact.data_ptr(), _stream(x))
    _check(st, "moe_gate_up")


def moe_down_combine(act, ids, tw, w2, w2_sf, alpha2, sact, wsd, ssd, gssd, out) -> None:
    """out[t] = bf16(bf16(sum_j tw * y_j) + y_shared) (in place)."""
    m, topk = ids.shape
    e, h, half_i = w2.shape
    inter = half_i * 2
    si = wsd.shape[1] * 2
    for name, t, dt in (("act", act, torch.bfloat16), ("ids", ids, torch.int32),
                        ("tw", tw, torch.float32), ("w2", w2, torch.uint8),
                        ("alpha2", alpha2, torch.float32), ("sact", sact, torch.bfloat16),
                        ("wsd", wsd, torch.uint8), ("gssd", gssd, torch.float32),
                        ("out", out, torch.bfloat16)):
        if t.dtype != dt or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous {dt} tensor")
    if tuple(out.shape) != (m, h) or tuple(act.shape) != (m * topk, inter) or tuple(sact.shape) != (m, si):
        raise ValueError("out must be [M, H], act [M*topk, I], sact [M, SI]")
    st = _lib.load().moe_down_combine(act.data_ptr(), ids.data_ptr(), tw.data_ptr(), m, topk, e,
                                      w2.data_ptr(), _flat_u8(w2_sf).data_ptr(), alpha2.data_ptr(),
                                      h, inter, sact.data_ptr(), wsd.data_ptr(),
                                      _flat_u8(ssd).data_ptr(), gssd.data_ptr(), si, out.data_ptr(),
                                      _stream(act))
    _check(st, "moe_down_combine")


# The pages' names of the MoE pair.
gate_up = moe_gate_up
down_combine = moe_down_combine
