"""Workload registry: the shapes, dtypes and distributions the forward pass is
exercised and measured on.

Shapes follow the MiniMind FFN/MoE pages: hidden size H, intermediate size
I = ceil(H*pi/64)*64 (MiniMind course lesson 13, section 3 step 1, config
excerpt; minimind3 chapter 4, section 4.1), E experts, k experts per token,
router aux coefficient ``coef``.  Token count N = batch * seq (lesson 13,
section 1.5, shape table).
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field


def intermediate_size(hidden: int) -> int:
    """MiniMind's default FFN width: ceil(hidden * pi / 64) * 64
    (lesson 13, section 3 step 1; minimind3 chapter 4, section 4.1)."""
    return int(math.ceil(hidden * math.pi / 64) * 64)


@dataclass(frozen=True)
class Workload:
    name: str
    kind: str            # "dense" or "moe"
    N: int               # tokens (B*S)
    H: int               # hidden size
    I: int               # intermediate size (per expert for MoE)
    E: int = 1           # experts (1 for dense)
    k: int = 1           # experts per token
    coef: float = 0.0    # router aux-loss coefficient
    dtype: str = "bf16"  # "fp32": everything fp32; "bf16": x, W, y bf16, router fp32
    batch: int = 1
    seq: int = 1
    # Skewed routing: per-expert logit offset b = bias_scale * z, z ~ N(0, bias_std).
    bias_std: float = 0.0
    bias_scale: float = 0.0
    # Block context: a residual stream [N, H] (dtype) that y is added to, and
    # the config's norm_topk_prob (False: alpha = the raw top-k probabilities).
    residual: bool = False
    norm_topk_prob: bool = True
    seed: int = 0
    note: str = ""
    extra: dict = field(default_factory=dict)

    @property
    def rows(self) -> int:
        """Rows the expert GEMMs process: one per (token, selected expert)."""
        return self.N * self.k

    def flops(self) -> float:
        """Algorithmic FLOPs of one forward pass: 6*N*k*H*I for the three
        projections of the selected experts, plus 2*N*H*E for the router."""
        f = 6.0 * self.N * self.k * self.H * self.I
        if self.kind == "moe":
            f += 2.0 * self.N * self.H * self.E
        return f

    def elem_bytes(self) -> int:
        return 4 if self.dtype == "fp32" else 2


_C4_BIAS_SCALE = 0.197  # calibrated so max/min expert load is about 10x (oracle/calibrate_skew.py)

WORKLOADS = {
    w.name: w
    for w in [
        Workload(
            name="dense_fp32_n100_h768_i2432", kind="dense", N=100, H=768,
            I=intermediate_size(768), dtype="fp32", batch=1, seq=100,
            note="dense SwiGLU FFN, fp32, MiniMind default width (small parity case)",
        ),
        Workload(
            name="moe_top1_n4096_h768_e4", kind="moe", N=4096, H=768,
            I=intermediate_size(768), E=4, k=1, coef=0.01, dtype="bf16",
            batch=8, seq=512,
            note="MoE FFN top-1, 4 experts, MiniMind default routing",
        ),
        Workload(
            name="dense_bf16_n16384_h2048_i6464", kind="dense", N=16384, H=2048,
            I=intermediate_size(2048), dtype="bf16", batch=32, seq=512,
            note="dense SwiGLU FFN, bf16 prefill",
        ),
        Workload(
            name="moe_top2_skew_n16384_h768_e8", kind="moe", N=16384, H=768,
            I=intermediate_size(768), E=8, k=2, coef=0.01, dtype="bf16",
            batch=32, seq=512, bias_std=1.5, bias_scale=_C4_BIAS_SCALE,
            note="MoE FFN top-2, 8 experts, per-expert logit offsets giving ~10x load skew",
        ),
        Workload(
            name="moe_top2_skew_literal_n16384_h768_e8", kind="moe", N=16384, H=768,
            I=intermediate_size(768), E=8, k=2, coef=0.01, dtype="bf16",
            batch=32, seq=512, bias_std=1.5, bias_scale=1.0,
            note="as the skewed top-2 case with unscaled N(0,1.5) offsets (empties experts; parity only)",
        ),
        Workload(
            name="moe_decode_n32_h2048_e16", kind="moe", N=32, H=2048, I=1408,
            E=16, k=2, coef=0.01, dtype="bf16", batch=32, seq=1,
            note="decode-shaped MoE FFN, weight-streaming bound",
        ),
    ]
}

# Short aliases used on the command line.
ALIASES = {
    "dense_fp32": "dense_fp32_n100_h768_i2432",
    "moe_top1": "moe_top1_n4096_h768_e4",
    "dense_bf16": "dense_bf16_n16384_h2048_i6464",
    "moe_skew": "moe_top2_skew_n16384_h768_e8",
    "moe_skew_literal": "moe_top2_skew_literal_n16384_h768_e8",
    "moe_decode": "moe_decode_n32_h2048_e16",
}


def get(name: str) -> Workload:
    return WORKLOADS[ALIASES.get(name, name)]
