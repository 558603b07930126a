"""Seeded synthetic workloads for the W4A16 NVFP4 GEMV family.

Both the CPU oracle and the HIP path are fed from the host tensors made
here; nothing in this module computes any part of the method (no decoding,
no swizzling, no products).  All tensors are CPU torch tensors drawn from a
``torch.Generator`` seeded with the given seed.

Value distributions (the workloads of the design notes):
  * activations x ~ N(0, 1) rounded to BF16;
  * packed weights: uniform random bytes, so both nibbles are uniform over
    the 16 E2M1 codes (including the -0 code);
  * block scales: uniform over the 65 finite positive E4M3 codes whose
    values lie in [2^-4, 2^4] (codes 0x18..0x58), drawn i.i.d. for every
    byte of the flat 128x4-swizzled buffer.  A layout permutation of i.i.d.
    draws is again i.i.d., so drawing the flat buffer directly has the same
    distribution as drawing logical scales and swizzling them; padding
    bytes (rows past N, columns past K/16) are drawn too and are never read;
  * global scale 1/64;
  * BF16 weights ~ N(0, 0.02) rounded to BF16;
  * MoE: distinct uniform top-k expert ids per token, softmax(N(0,1))
    routing weights in FP32, per-expert alphas 2^-(5 + e mod 3) and
    2^-(5 + (e+1) mod 3).
"""
from __future__ import annotations

import torch

SCALE_CODE_LO = 0x18  # E4M3 2^-4
SCALE_CODE_HI = 0x58  # E4M3 2^4
GLOBAL_SCALE = 1.0 / 64.0


def seed_for(config: int, m: int, variant: int = 0) -> int:
    """Seed of one workload: 1000 * config + M + 100 * variant."""
    return 1000 * config + m + 100 * variant


def flat_scale_bytes(n: int, k: int) -> int:
    """Byte size of a flat 128x4-swizzled scale buffer for an [n, k] weight:
    rows rounded up to 128 times K/16 rounded up to 4."""
    return (n + 127) // 128 * 128 * ((k // 16 + 3) // 4 * 4)


def _gen(seed: int) -> torch.Generator:
    g = torch.Generator()
    g.manual_seed(int(seed))
    return g


def activations(m: int, k: int, g: torch.Generator) -> torch.Tensor:
    return torch.randn((m, k), generator=g, dtype=torch.float32).to(torch.bfloat16)


def packed_weight(n: int, k: int, g: torch.Generator) -> torch.Tensor:
    return torch.randint(0, 256, (n, k // 2), generator=g, dtype=torch.uint8)


def flat_scales(n: int, k: int, g: torch.Generator) -> torch.Tensor:
    return torch.randint(SCALE_CODE_LO, SCALE_CODE_HI + 1, (flat_scale_bytes(n, k),),
                         generator=g, dtype=torch.uint8)


def flat_scales_all_finite(n: int, k: int, g: torch.Generator) -> torch.Tensor:
    """Scale bytes uniform over all 254 finite E4M3FN codes: zero and
    subnormal codes (0x00-0x07), normal ones up to 448 (0x7E), and all their
    negatives (0x80-0xFE); the two NaN codes 0x7F / 0xFF are left out."""
    codes = torch.randint(0, 254, (flat_scale_bytes(n, k),), generator=g, dtype=torch.int32)
    codes = codes + (codes >= 0x7F).to(torch.int32)          # skip 0x7F
    return codes.to(torch.uint8)


def activations_wide(m: int, k: int, g: torch.Generator, lo: int, hi: int) -> torch.Tensor:
    """N(0, 1) values each multiplied by 2^e, e uniform over [lo, hi],
    rounded to BF16 (lo <= -127 reaches BF16 subnormals)."""
    x = torch.randn((m, k), generator=g, dtype=torch.float64)
    e = torch.randint(lo, hi + 1, (m, k), generator=g, dtype=torch.int64)
    return (x * torch.pow(2.0, e.to(torch.float64))).to(torch.float32).to(torch.bfloat16)


def dense_w4a16(m: int, n: int, k: int, seed: int, scales: str = "config", x_exp: tuple | None = None) -> dict:
    """x bf16 [m, k], w uint8 [n, k/2], s uint8 flat swizzled, gs fp32 [1].
    scales="all_finite" draws every finite E4M3 code (edge-case tests);
    x_exp=(lo, hi) scales each activation by 2^e, e uniform over [lo, hi]."""
    g = _gen(seed)
    x = activations(m, k, g) if x_exp is None else activations_wide(m, k, g, *x_exp)
    w = packed_weight(n, k, g)
    s = flat_scales(n, k, g) if scales == "config" else flat_scales_all_finite(n, k, g)
    gs = torch.tensor([GLOBAL_SCALE], dtype=torch.float32)
    return dict(x=x, w=w, s=s, gs=gs)


def dense_bf16(m: int, n: int, k: int, seed: int) -> dict:
    """x bf16 [m, k], w bf16 [n, k] ~ N(0, 0.02)."""
    g = _gen(seed)
    x = activations(m, k, g)
    w = (torch.randn((n, k), generator=g, dtype=torch.float32) * 0.02).to(torch.bfloat16)
    return dict(x=x, w=w)


def moe_routing(m: int, n_experts: int, topk: int, g: torch.Generator):
    ids = torch.stack([torch.randperm(n_experts, generator=g)[:topk] for _ in range(m)]).to(torch.int32)
    if m == 0:
        ids = torch.empty((0, topk), dtype=torch.int32)
    tw = torch.softmax(torch.randn((m, topk), generator=g, dtype=torch.float32), dim=-1)
    return ids.contiguous(), tw.contiguous()


def moe_alphas(n_experts: int):
    alpha = torch.tensor([2.0 ** -(5 + e % 3) for e in range(n_experts)], dtype=torch.float32)
    alpha2 = torch.tensor([2.0 ** -(5 + (e + 1) % 3) for e in range(n_experts)], dtype=torch.float32)
    return alpha, alpha2


def moe_weights(n_experts: int, hidden: int, inter: int, shared_inter: int, seed: int,
                scales: str = "config") -> dict:
    """Routed W1 [E, 2I, H/2] + flat scales [E, bytes(2I, H)], W2 [E, H, I/2] +
    flat scales [E, bytes(H, I)], shared Wsh [2SI, H/2] / Wsd [H, SI/2] with
    flat scales, per-expert alphas and the shared global scales
    (scales="all_finite": every finite E4M3 code, as dense_w4a16)."""
    g = _gen(seed)

    def expert_scales(rows, cols):
        if scales == "config":
            return torch.randint(SCALE_CODE_LO, SCALE_CODE_HI + 1, (n_experts, flat_scale_bytes(rows, cols)),
                                 generator=g, dtype=torch.uint8)
        return torch.stack([flat_scales_all_finite(rows, cols, g) for _ in range(n_experts)])

    def one_scales(rows, cols):
        return flat_scales(rows, cols, g) if scales == "config" else flat_scales_all_finite(rows, cols, g)
    w1 = torch.randint(0, 256, (n_experts, 2 * inter, hidden // 2), generator=g, dtype=torch.uint8)
    w1_sf = expert_scales(2 * inter, hidden)
    w2 = torch.randint(0, 256, (n_experts, hidden, inter // 2), generator=g, dtype=torch.uint8)
    w2_sf = expert_scales(hidden, inter)
    wsh = packed_weight(2 * shared_inter, hidden, g)
    ssh = one_scales(2 * shared_inter, hidden)
    wsd = packed_weight(hidden, shared_inter, g)
    ssd = one_scales(hidden, shared_inter)
    alpha, alpha2 = moe_alphas(n_experts)
    gssh = torch.tensor([GLOBAL_SCALE], dtype=torch.float32)
    gssd = torch.tensor([GLOBAL_SCALE], dtype=torch.float32)
    return dict(w1=w1, w1_sf=w1_sf, alpha=alpha, w2=w2, w2_sf=w2_sf, alpha2=alpha2,
                wsh=wsh, ssh=ssh, gssh=gssh, wsd=wsd, ssd=ssd, gssd=gssd)


def moe_tokens(m: int, hidden: int, n_experts: int, topk: int, seed: int) -> dict:
    """x bf16 [m, H], ids int32 [m, topk] (distinct per token), tw fp32 [m, topk]."""
    g = _gen(seed)
    x = activations(m, hidden, g)
    ids, tw = moe_routing(m, n_experts, topk, g)
    return dict(x=x, ids=ids, tw=tw)


# The MoE decode block measured here: 128 experts, top-8, hidden 4096,
# expert and shared-expert intermediate size 1536.
MOE_EXPERTS = 128
MOE_TOPK = 8
MOE_HIDDEN = 4096
MOE_INTER = 1536
MOE_SHARED_INTER = 1536
