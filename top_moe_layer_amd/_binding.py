"""ctypes binding of ``lib/libtopmoe.so`` (declared in include/topmoe.h).

Argument marshalling only: every step of the forward pass runs in the HIP
kernels behind the C ABI.  PyTorch provides device memory and the stream.
There is no CPU fallback: if the library is missing, loading fails loudly.
"""
from __future__ import annotations

import ctypes
import os

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "lib", "libtopmoe.so")

# Must match include/topmoe.h
OK = 0
ERR_NULL_ARG = -1
ERR_BAD_SHAPE = -2
ERR_UNSUPPORTED_DTYPE = -3
ERR_WORKSPACE_TOO_SMALL = -4
ERR_HIP = -5
ERR_BAD_ARG = -6
ERR_SCRATCH_TOO_SMALL = -7
NOALLOC_SCRATCH_BYTES = 64 << 20
DTYPE_FP32 = 0
DTYPE_BF16 = 1
MOE_RAW_TOPK_WEIGHTS = 1
MOE_BWD_SAVED = 2
MOE_EVAL = 4
TILE_SLOTS = {"gateup": 0, "down": 1, "bwd_gu": 2, "bwd_dh": 3, "wgrad_gu": 4, "wgrad_d": 5}
FFN_STAGES = 2
MOE_STAGES = 5
FFN_BWD_STAGES = 7
MOE_BWD_STAGES = 12

FFN_STAGE_NAMES = ["gateup_gemm", "down_gemm"]
MOE_STAGE_NAMES = ["router", "permute", "gateup_gemm", "down_gemm", "combine"]
FFN_BWD_STAGE_NAMES = ["transpose_w", "transpose_act", "gu_gemm", "dh_gemm", "dx_gemm",
                       "dwgu_gemm", "dwd_gemm"]
MOE_BWD_STAGE_NAMES = ["router", "permute", "transpose_w", "transpose_act", "gu_gemm", "dh_gemm",
                       "dx_gemm", "router_bwd", "dx_combine", "dwr", "dwgu_gemm", "dwd_gemm"]

# Every function include/topmoe.h declares, with its ctypes signature.
_vp, _i64, _i32, _sz, _f32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_size_t, ctypes.c_float
SIGNATURES = {
    "ffn_workspace_bytes": (_sz, [_i64, _i64, _i64, _i32]),
    "ffn_swiglu_fwd": (_i32, [_vp, _vp, _vp, _vp, _vp, _vp, _i64, _i64, _i64, _i32, _vp, _sz, _vp,
                              _vp]),
    "moe_workspace_bytes": (_sz, [_i64, _i64, _i64, _i32, _i32, _i32]),
    "moe_ffn_fwd": (_i32, [_vp, _vp, _vp, _vp, _vp, _vp, _i64, _i64, _i64, _i32, _i32, _f32, _f32,
                           _f32, _i32, _i32, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _sz, _vp,
                           _vp]),
    "moe_ffn_fwd_noalloc": (_i32, [_vp, _vp, _vp, _vp, _vp, _vp, _i64, _i64, _i64, _i32, _i32,
                                   _f32, _f32, _f32, _i32, _i32, _vp, _vp, _vp, _vp, _vp, _vp,
                                   _vp, _vp, _vp]),
    "ffn_swiglu_fwd_train": (_i32, [_vp, _vp, _vp, _vp, _vp, _vp, _i64, _i64, _i64, _i32, _vp, _sz,
                                    _vp, _sz, _vp, _vp]),
    "moe_ffn_fwd_train": (_i32, [_vp, _vp, _vp, _vp, _vp, _vp, _i64, _i64, _i64, _i32, _i32, _f32,
                                 _f32, _f32, _i32, _i32, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                                 _sz, _vp, _sz, _vp, _vp]),
    "ffn_bwd_workspace_bytes": (_sz, [_i64, _i64, _i64, _i32]),
    "ffn_swiglu_bwd": (_i32, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i64, _i64, _i64, _i32,
                              _vp, _sz, _vp, _vp]),
    "ffn_swiglu_bwd_saved": (_i32, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i64, _i64, _i64,
                                    _i32, _vp, _sz, _vp, _vp]),
    "moe_bwd_workspace_bytes": (_sz, [_i64, _i64, _i64, _i32, _i32, _i32]),
    "moe_ffn_bwd": (_i32, [_vp, _vp, _vp, _vp, _vp, _vp, _f32, _f32, _vp, _vp, _i64, _i64, _i64,
                           _i32, _i32, _f32, _f32, _f32, _i32, _i32, _vp, _vp, _vp, _vp, _vp, _vp,
                           _sz, _vp, _vp]),
    "topmoe_strerror": (ctypes.c_char_p, [_i32]),
    "topmoe_version": (_i32, []),
    "topmoe_set_tile_override": (_i32, [_i32, _vp]),
    "moe_ffn_fwd_path": (_i32, [_i64, _i64, _i64, _i32, _i32, _f32, _i32, _vp, _i32]),
    "topmoe_events_create": (_i32, [_i32, _vp]),
    "topmoe_events_destroy": (_i32, [_i32, _vp]),
    "topmoe_event_elapsed_ms": (_i32, [_vp, _vp, ctypes.POINTER(ctypes.c_float)]),
}

_lib = None


class TopmoeError(RuntimeError):
    def __init__(self, status: int, what: str = ""):
        self.status = status
        msg = strerror(status)
        super().__init__(f"{what}: status {status}: {msg}" if what else f"status {status}: {msg}")


def lib() -> ctypes.CDLL:
    """Load the library (once).  Raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build it with `python -m top_moe_layer_amd.build` "
                "(there is no CPU fallback)")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


def strerror(status: int) -> str:
    return lib().topmoe_strerror(int(status)).decode()


def check(status: int, what: str = "") -> None:
    if status != OK:
        raise TopmoeError(status, what)


# ------------------------------------------------------------ raw calls
def raw_ffn_workspace_bytes(N, H, I, dtype) -> int:
    return int(lib().ffn_workspace_bytes(N, H, I, dtype))


def raw_moe_workspace_bytes(N, H, I, E, k, dtype) -> int:
    return int(lib().moe_workspace_bytes(N, H, I, E, k, dtype))


def raw_ffn_swiglu_fwd(x, Wg, Wu, Wd, residual, y, N, H, I, dtype, ws, ws_bytes, stream,
                       events) -> int:
    return int(lib().ffn_swiglu_fwd(x, Wg, Wu, Wd, residual, y, N, H, I, dtype, ws, ws_bytes,
                                    stream, events))


def raw_moe_ffn_fwd(x, Wr, Wg, Wu, Wd, residual, N, H, I, E, k, coef, z_coef, capacity_factor,
                    flags, dtype, y, topk_idx, alpha, aux, z_loss, offsets, sorted_ids, ws,
                    ws_bytes, stream, events) -> int:
    return int(lib().moe_ffn_fwd(x, Wr, Wg, Wu, Wd, residual, N, H, I, E, k, coef, z_coef,
                                 capacity_factor, flags, dtype, y, topk_idx, alpha, aux, z_loss,
                                 offsets, sorted_ids, ws, ws_bytes, stream, events))


def raw_moe_ffn_fwd_noalloc(x, Wr, Wg, Wu, Wd, residual, N, H, I, E, k, coef, z_coef,
                            capacity_factor, flags, dtype, y, topk_idx, alpha, aux, z_loss,
                            offsets, sorted_ids, stream, events) -> int:
    return int(lib().moe_ffn_fwd_noalloc(x, Wr, Wg, Wu, Wd, residual, N, H, I, E, k, coef,
                                         z_coef, capacity_factor, flags, dtype, y, topk_idx,
                                         alpha, aux, z_loss, offsets, sorted_ids, stream, events))


def raw_ffn_swiglu_fwd_train(x, Wg, Wu, Wd, residual, y, N, H, I, dtype, ws, ws_bytes, saved,
                             saved_bytes, stream, events) -> int:
    return int(lib().ffn_swiglu_fwd_train(x, Wg, Wu, Wd, residual, y, N, H, I, dtype, ws, ws_bytes,
                                          saved, saved_bytes, stream, events))


def raw_moe_ffn_fwd_train(x, Wr, Wg, Wu, Wd, residual, N, H, I, E, k, coef, z_coef,
                          capacity_factor, flags, dtype, y, topk_idx, alpha, aux, z_loss, offsets,
                          sorted_ids, ws, ws_bytes, saved, saved_bytes, stream, events) -> int:
    return int(lib().moe_ffn_fwd_train(x, Wr, Wg, Wu, Wd, residual, N, H, I, E, k, coef, z_coef,
                                       capacity_factor, flags, dtype, y, topk_idx, alpha, aux,
                                       z_loss, offsets, sorted_ids, ws, ws_bytes, saved,
                                       saved_bytes, stream, events))


def raw_ffn_bwd_workspace_bytes(N, H, I, dtype) -> int:
    return int(lib().ffn_bwd_workspace_bytes(N, H, I, dtype))


def raw_moe_bwd_workspace_bytes(N, H, I, E, k, dtype) -> int:
    return int(lib().moe_bwd_workspace_bytes(N, H, I, E, k, dtype))


def raw_ffn_swiglu_bwd(x, Wg, Wu, Wd, dy, dx, dWg, dWu, dWd, N, H, I, dtype, ws, ws_bytes, stream,
                       events) -> int:
    return int(lib().ffn_swiglu_bwd(x, Wg, Wu, Wd, dy, dx, dWg, dWu, dWd, N, H, I, dtype, ws,
                                    ws_bytes, stream, events))


def raw_ffn_swiglu_bwd_saved(x, Wg, Wu, Wd, dy, dx, dWg, dWu, dWd, N, H, I, dtype, ws, ws_bytes,
                             stream, events) -> int:
    return int(lib().ffn_swiglu_bwd_saved(x, Wg, Wu, Wd, dy, dx, dWg, dWu, dWd, N, H, I, dtype, ws,
                                          ws_bytes, stream, events))


def raw_moe_ffn_bwd(x, Wr, Wg, Wu, Wd, dy, aux_grad, z_grad, aux_grad_scale, z_grad_scale, N, H,
                    I, E, k, coef, z_coef, capacity_factor, flags, dtype, dx, dWr, dWg, dWu, dWd,
                    ws, ws_bytes, stream, events) -> int:
    return int(lib().moe_ffn_bwd(x, Wr, Wg, Wu, Wd, dy, aux_grad, z_grad, aux_grad_scale,
                                 z_grad_scale, N, H, I, E, k, coef, z_coef, capacity_factor, flags,
                                 dtype, dx, dWr, dWg, dWu, dWd, ws, ws_bytes, stream, events))


PATH_FIELDS = ["router_layout", "router_tokens", "router_blocks", "up_bm", "up_bn", "up_ring",
               "down_bm", "down_bn", "down_ring", "down_ksplit", "inblock", "router_in_up"]


def moe_fwd_path(N, H, I, E, k, dtype, capacity_factor=0.0) -> dict:
    """The launch plan of moe_ffn_fwd for a problem (host only, no GPU):
    a dict of PATH_FIELDS (include/topmoe.h, TOPMOE_PATH_*)."""
    info = (ctypes.c_int32 * len(PATH_FIELDS))()
    check(lib().moe_ffn_fwd_path(N, H, I, E, k, float(capacity_factor), dtype, info,
                                 len(PATH_FIELDS)), "moe_ffn_fwd_path")
    return dict(zip(PATH_FIELDS, (int(v) for v in info)))


def set_tile_override(gemm: str, shape=None) -> None:
    """Force the launch shape of one GEMM of the path (tuning sweeps, tests):
    ``gemm`` one of TILE_SLOTS; ``shape`` "BMxBNxWMxWNxRBxS" or a 6-tuple, None
    to clear.  Raises TopmoeError (bad argument) if it is not instantiated."""
    arr = None
    if shape is not None:
        vals = [int(v) for v in shape.split("x")] if isinstance(shape, str) else list(shape)
        if len(vals) != 6:
            raise ValueError(f"shape needs 6 values, got {shape!r}")
        arr = (ctypes.c_int * 6)(*vals)
    check(lib().topmoe_set_tile_override(TILE_SLOTS[gemm], arr), f"set_tile_override({gemm})")


class StageEvents:
    """Start / stop events of every stage (2 * stages) for ``stage_events``."""

    def __init__(self, stages: int):
        self.stages = stages
        self.n = 2 * stages
        self.arr = (ctypes.c_void_p * self.n)()
        check(lib().topmoe_events_create(self.n, self.arr), "topmoe_events_create")

    @property
    def ptr(self):
        return ctypes.cast(self.arr, ctypes.c_void_p)

    def elapsed_ms(self):
        """Kernel milliseconds of each stage of the last recorded call (waits for it)."""
        out = []
        ms = ctypes.c_float()
        for i in range(self.stages):
            check(lib().topmoe_event_elapsed_ms(self.arr[2 * i], self.arr[2 * i + 1],
                                                ctypes.byref(ms)),
                  "topmoe_event_elapsed_ms")
            out.append(ms.value)
        return out

    def close(self):
        if self.arr is not None:
            lib().topmoe_events_destroy(self.n, self.arr)
            self.arr = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
