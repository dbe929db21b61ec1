"""MI355X (gfx950) MiniMind FFN / top-k MoE forward and backward.

The compute lives in ``lib/libtopmoe.so`` (hand-written HIP kernels behind the
C ABI of include/topmoe.h).  This package only marshals torch tensors into
that ABI.  Importing it does not load the library; the first call does, and
fails loudly if the library has not been built.
"""
from ._binding import (  # noqa: F401
    DTYPE_BF16,
    DTYPE_FP32,
    FFN_BWD_STAGES,
    FFN_BWD_STAGE_NAMES,
    FFN_STAGES,
    FFN_STAGE_NAMES,
    MOE_BWD_STAGES,
    MOE_BWD_STAGE_NAMES,
    MOE_STAGES,
    MOE_STAGE_NAMES,
    LIB_PATH,
    StageEvents,
    TopmoeError,
    PATH_FIELDS,
    lib,
    moe_fwd_path,
    set_tile_override,
    strerror,
)


def __getattr__(name):
    # torch-level wrappers are imported lazily so that ``import top_moe_layer_amd``
    # stays cheap for tools that only need the raw binding.
    if name in ("ffn_swiglu_fwd", "moe_ffn_fwd", "ffn_workspace_bytes", "moe_workspace_bytes",
                "MoeOutput", "ffn_swiglu_bwd", "moe_ffn_bwd", "ffn_bwd_workspace_bytes",
                "moe_bwd_workspace_bytes", "FfnGrads", "MoeGrads"):
        from . import ops
        return getattr(ops, name)
    if name in ("swiglu_ffn", "moe_ffn"):
        from . import autograd
        return getattr(autograd, name)
    raise AttributeError(name)
