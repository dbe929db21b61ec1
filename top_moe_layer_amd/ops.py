"""Torch-tensor front end of the C ABI: shape / dtype checks, output and
workspace allocation through PyTorch, the caller's HIP stream (the current one
by default).  Nothing here computes any part of the forward pass.

Every tensor these functions allocate (outputs and internal workspaces) is
allocated while the stream the kernels run on is torch's current stream, so
the caching allocator ties the memory to that stream: an internal workspace
released on return is only handed out again to work ordered after these
kernels on the same stream."""
from __future__ import annotations

import functools
from dataclasses import dataclass
from typing import Optional

import torch

from . import _binding as B


def _dtype_code(t: torch.dtype) -> int:
    if t == torch.float32:
        return B.DTYPE_FP32
    if t == torch.bfloat16:
        return B.DTYPE_BF16
    raise TypeError(f"unsupported dtype {t}; use float32 or bfloat16")


def _need(t: torch.Tensor, name: str, shape, dtype, device):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be a GPU tensor (got {t.device}); the library has no CPU path")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if t.dtype != dtype:
        raise TypeError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _ptr(t: Optional[torch.Tensor]) -> int:
    return 0 if t is None else t.data_ptr()


def _stream(device, stream) -> int:
    if stream is None:
        stream = torch.cuda.current_stream(device)
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _torch_stream(device, stream):
    """The torch stream object the kernels will run on: the current stream of
    ``device`` when ``stream`` is None, an ExternalStream for a raw handle."""
    if stream is None:
        return torch.cuda.current_stream(device)
    if isinstance(stream, torch.cuda.Stream):
        return stream
    return torch.cuda.ExternalStream(int(stream), device=device)


def _on_caller_stream(fn):
    """Run ``fn`` with the kernels' stream as torch's current stream, so that
    the tensors it allocates belong to that stream (see the module docstring).
    Tensors that are not on a GPU pass through to ``fn``'s own checks."""
    @functools.wraps(fn)
    def wrapped(x, *args, stream=None, **kw):
        if not isinstance(x, torch.Tensor) or x.device.type != "cuda":
            return fn(x, *args, stream=stream, **kw)
        ts = _torch_stream(x.device, stream)
        with torch.cuda.stream(ts):
            return fn(x, *args, stream=ts, **kw)
    return wrapped


def _buffer(t: torch.Tensor, name: str, nbytes: int, device) -> torch.Tensor:
    """A caller-provided byte buffer: on the device, contiguous, large enough."""
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device} (the library has no CPU path)")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if t.numel() * t.element_size() < nbytes:
        raise ValueError(f"{name} has {t.numel() * t.element_size()} bytes, needs {nbytes}")
    return t


def _workspace(nbytes: int, device, ws: Optional[torch.Tensor]) -> torch.Tensor:
    if ws is None:
        return torch.empty(max(nbytes, 256), dtype=torch.uint8, device=device)
    return _buffer(ws, "workspace", nbytes, device)


def ffn_workspace_bytes(N: int, H: int, I: int, dtype: torch.dtype) -> int:
    return B.raw_ffn_workspace_bytes(N, H, I, _dtype_code(dtype))


def moe_workspace_bytes(N: int, H: int, I: int, E: int, k: int, dtype: torch.dtype) -> int:
    return B.raw_moe_workspace_bytes(N, H, I, E, k, _dtype_code(dtype))


@_on_caller_stream
def ffn_swiglu_fwd(x: torch.Tensor, Wg: torch.Tensor, Wu: torch.Tensor, Wd: torch.Tensor, *,
                   residual: Optional[torch.Tensor] = None, y: Optional[torch.Tensor] = None,
                   workspace: Optional[torch.Tensor] = None,
                   saved: Optional[torch.Tensor] = None, stream=None,
                   stage_events: Optional[B.StageEvents] = None) -> torch.Tensor:
    """Dense SwiGLU FFN: y = residual + Wd (SiLU(Wg x) * Wu x) (residual
    optional, x's shape and dtype; it may be y itself).  x [..., H];
    Wg, Wu [I, H]; Wd [H, I].  Returns y with x's shape and dtype.
    ``saved`` (a backward workspace, ffn_bwd_workspace_bytes long): also keep
    g, u and h there for ``ffn_swiglu_bwd(..., workspace=saved,
    from_saved=True)``; y is the same either way."""
    dev = x.device
    H = x.shape[-1]
    I = Wg.shape[0]
    xf = x.reshape(-1, H)
    N = xf.shape[0]
    dt = x.dtype
    _need(xf, "x", (N, H), dt, dev)
    _need(Wg, "Wg", (I, H), dt, dev)
    _need(Wu, "Wu", (I, H), dt, dev)
    _need(Wd, "Wd", (H, I), dt, dev)
    rf = None if residual is None else residual.reshape(-1, H)
    if rf is not None:
        _need(rf, "residual", (N, H), dt, dev)
    if y is None:
        y = torch.empty((N, H), dtype=dt, device=dev)
    _need(y, "y", (N, H), dt, dev)
    code = _dtype_code(dt)
    nbytes = B.raw_ffn_workspace_bytes(N, H, I, code)
    if nbytes == 0:
        B.check(B.ERR_BAD_SHAPE, "ffn_swiglu_fwd")
    ws = _workspace(nbytes, dev, workspace)
    evp = stage_events.ptr if stage_events is not None else None
    if saved is not None:
        _buffer(saved, "saved", B.raw_ffn_bwd_workspace_bytes(N, H, I, code), dev)
        st = B.raw_ffn_swiglu_fwd_train(_ptr(xf), _ptr(Wg), _ptr(Wu), _ptr(Wd), _ptr(rf), _ptr(y),
                                        N, H, I, code, _ptr(ws), ws.numel() * ws.element_size(),
                                        _ptr(saved), saved.numel() * saved.element_size(),
                                        _stream(dev, stream), evp)
        B.check(st, "ffn_swiglu_fwd_train")
        return y.view(x.shape)
    st = B.raw_ffn_swiglu_fwd(_ptr(xf), _ptr(Wg), _ptr(Wu), _ptr(Wd), _ptr(rf), _ptr(y), N, H, I, code,
                              _ptr(ws), ws.numel() * ws.element_size(), _stream(dev, stream), evp)
    B.check(st, "ffn_swiglu_fwd")
    return y.view(x.shape)


@dataclass
class MoeOutput:
    y: torch.Tensor
    topk_idx: torch.Tensor
    alpha: torch.Tensor
    aux_loss: torch.Tensor
    expert_offsets: Optional[torch.Tensor]
    sorted_token_ids: Optional[torch.Tensor]
    z_loss: Optional[torch.Tensor] = None


@_on_caller_stream
def moe_ffn_fwd(x: torch.Tensor, Wr: torch.Tensor, Wg: torch.Tensor, Wu: torch.Tensor,
                Wd: torch.Tensor, k: int, aux_coef: float, *,
                residual: Optional[torch.Tensor] = None, norm_topk_prob: bool = True,
                z_coef: float = 0.0, capacity_factor: float = 0.0,
                y: Optional[torch.Tensor] = None, topk_idx: Optional[torch.Tensor] = None,
                alpha: Optional[torch.Tensor] = None, aux_loss: Optional[torch.Tensor] = None,
                expert_offsets: Optional[torch.Tensor] = None,
                sorted_token_ids: Optional[torch.Tensor] = None, return_lists: bool = True,
                workspace: Optional[torch.Tensor] = None, saved: Optional[torch.Tensor] = None,
                training: bool = True, stream=None,
                stage_events: Optional[B.StageEvents] = None) -> MoeOutput:
    """Top-k MoE FFN forward.  x [..., H]; Wr [E, H] float32; Wg, Wu [E, I, H];
    Wd [E, H, I].  Returns y (x's shape), topk_idx / alpha [N, k], aux_loss [1]
    and, when ``return_lists``, expert_offsets [E+1] and sorted_token_ids [N*k].
    ``residual`` (x's shape and dtype, may be y itself) is added to y;
    ``norm_topk_prob`` False keeps the raw top-k probabilities as alpha;
    ``z_coef`` > 0 also returns the router z-loss; ``capacity_factor`` > 0
    caps each expert at ceil(factor * N * k / E) tokens (offsets and lists
    then hold the kept tokens).  ``saved`` (a backward workspace,
    moe_bwd_workspace_bytes long): also keep the routing, g, u and h there
    for ``moe_ffn_bwd(..., workspace=saved, from_saved=True)``; the outputs
    are the same either way.  ``training`` False is the module outside
    training: aux_loss (and z_loss) are zero whatever the coefficients."""
    dev = x.device
    H = x.shape[-1]
    E, I = Wg.shape[0], Wg.shape[1]
    xf = x.reshape(-1, H)
    N = xf.shape[0]
    dt = x.dtype
    _need(xf, "x", (N, H), dt, dev)
    _need(Wr, "Wr", (E, H), torch.float32, dev)
    _need(Wg, "Wg", (E, I, H), dt, dev)
    _need(Wu, "Wu", (E, I, H), dt, dev)
    _need(Wd, "Wd", (E, H, I), dt, dev)
    new = lambda shape, d: torch.empty(shape, dtype=d, device=dev)
    y = new((N, H), dt) if y is None else y
    topk_idx = new((N, k), torch.int32) if topk_idx is None else topk_idx
    alpha = new((N, k), torch.float32) if alpha is None else alpha
    aux_loss = new((1,), torch.float32) if aux_loss is None else aux_loss
    z_loss = new((1,), torch.float32) if z_coef else None
    if return_lists:
        expert_offsets = new((E + 1,), torch.int32) if expert_offsets is None else expert_offsets
        sorted_token_ids = new((N * k,), torch.int32) if sorted_token_ids is None else sorted_token_ids
    _need(y, "y", (N, H), dt, dev)
    rf = None if residual is None else residual.reshape(-1, H)
    if rf is not None:
        _need(rf, "residual", (N, H), dt, dev)
    _need(topk_idx, "topk_idx", (N, k), torch.int32, dev)
    _need(alpha, "alpha", (N, k), torch.float32, dev)
    _need(aux_loss, "aux_loss", (1,), torch.float32, dev)
    if expert_offsets is not None:
        _need(expert_offsets, "expert_offsets", (E + 1,), torch.int32, dev)
    if sorted_token_ids is not None:
        _need(sorted_token_ids, "sorted_token_ids", (N * k,), torch.int32, dev)
    code = _dtype_code(dt)
    nbytes = B.raw_moe_workspace_bytes(N, H, I, E, k, code)
    if nbytes == 0:
        B.check(B.ERR_BAD_SHAPE, "moe_ffn_fwd")
    ws = _workspace(nbytes, dev, workspace)
    flags = (0 if norm_topk_prob else B.MOE_RAW_TOPK_WEIGHTS) | (0 if training else B.MOE_EVAL)
    args = (_ptr(xf), _ptr(Wr), _ptr(Wg), _ptr(Wu), _ptr(Wd), _ptr(rf), N, H, I, E, k,
            float(aux_coef), float(z_coef), float(capacity_factor), flags, code, _ptr(y),
            _ptr(topk_idx), _ptr(alpha), _ptr(aux_loss), _ptr(z_loss), _ptr(expert_offsets),
            _ptr(sorted_token_ids), _ptr(ws), ws.numel() * ws.element_size())
    evp = stage_events.ptr if stage_events is not None else None
    if saved is not None:
        _buffer(saved, "saved", B.raw_moe_bwd_workspace_bytes(N, H, I, E, k, code), dev)
        st = B.raw_moe_ffn_fwd_train(*args, _ptr(saved), saved.numel() * saved.element_size(),
                                     _stream(dev, stream), evp)
        B.check(st, "moe_ffn_fwd_train")
    else:
        st = B.raw_moe_ffn_fwd(*args, _stream(dev, stream), evp)
        B.check(st, "moe_ffn_fwd")
    return MoeOutput(y.view(x.shape), topk_idx, alpha, aux_loss, expert_offsets, sorted_token_ids,
                     z_loss)


def ffn_bwd_workspace_bytes(N: int, H: int, I: int, dtype: torch.dtype) -> int:
    return B.raw_ffn_bwd_workspace_bytes(N, H, I, _dtype_code(dtype))


def moe_bwd_workspace_bytes(N: int, H: int, I: int, E: int, k: int, dtype: torch.dtype) -> int:
    return B.raw_moe_bwd_workspace_bytes(N, H, I, E, k, _dtype_code(dtype))


@dataclass
class FfnGrads:
    dx: torch.Tensor
    dWg: torch.Tensor
    dWu: torch.Tensor
    dWd: torch.Tensor


@dataclass
class MoeGrads:
    dx: torch.Tensor
    dWr: torch.Tensor
    dWg: torch.Tensor
    dWu: torch.Tensor
    dWd: torch.Tensor


@_on_caller_stream
def ffn_swiglu_bwd(x: torch.Tensor, Wg: torch.Tensor, Wu: torch.Tensor, Wd: torch.Tensor,
                   dy: torch.Tensor, *, workspace: Optional[torch.Tensor] = None,
                   from_saved: bool = False, stream=None,
                   stage_events: Optional[B.StageEvents] = None) -> FfnGrads:
    """Gradients of the dense SwiGLU FFN for the upstream gradient dy (x's
    shape and dtype): dx (x's shape), dWg, dWu [I, H], dWd [H, I].
    ``from_saved``: ``workspace`` is the ``saved`` buffer of a training
    forward on the same inputs, and g, u are not recomputed."""
    dev = x.device
    H = x.shape[-1]
    I = Wg.shape[0]
    xf = x.reshape(-1, H)
    N = xf.shape[0]
    dt = x.dtype
    dyf = dy.reshape(-1, H)
    _need(xf, "x", (N, H), dt, dev)
    _need(Wg, "Wg", (I, H), dt, dev)
    _need(Wu, "Wu", (I, H), dt, dev)
    _need(Wd, "Wd", (H, I), dt, dev)
    _need(dyf, "dy", (N, H), dt, dev)
    new = lambda shape: torch.empty(shape, dtype=dt, device=dev)
    dx, dWg, dWu, dWd = new((N, H)), new((I, H)), new((I, H)), new((H, I))
    code = _dtype_code(dt)
    nbytes = B.raw_ffn_bwd_workspace_bytes(N, H, I, code)
    if nbytes == 0:
        B.check(B.ERR_BAD_SHAPE, "ffn_swiglu_bwd")
    if from_saved and workspace is None:
        raise ValueError("from_saved needs the training forward's saved buffer as workspace")
    ws = _workspace(nbytes, dev, workspace)
    fn = B.raw_ffn_swiglu_bwd_saved if from_saved else B.raw_ffn_swiglu_bwd
    st = fn(_ptr(xf), _ptr(Wg), _ptr(Wu), _ptr(Wd), _ptr(dyf), _ptr(dx),
            _ptr(dWg), _ptr(dWu), _ptr(dWd), N, H, I, code, _ptr(ws),
            ws.numel() * ws.element_size(), _stream(dev, stream),
            stage_events.ptr if stage_events is not None else None)
    B.check(st, "ffn_swiglu_bwd")
    return FfnGrads(dx.view(x.shape), dWg, dWu, dWd)


@_on_caller_stream
def moe_ffn_bwd(x: torch.Tensor, Wr: torch.Tensor, Wg: torch.Tensor, Wu: torch.Tensor,
                Wd: torch.Tensor, dy: torch.Tensor, k: int, aux_coef: float, *,
                aux_grad=1.0, norm_topk_prob: bool = True, z_coef: float = 0.0,
                z_grad=1.0, capacity_factor: float = 0.0,
                workspace: Optional[torch.Tensor] = None, from_saved: bool = False, stream=None,
                stage_events: Optional[B.StageEvents] = None) -> MoeGrads:
    """Gradients of the top-k MoE FFN (and of ``aux_grad`` * aux_loss and
    ``z_grad`` * z_loss) for the upstream gradient dy: dx (x's shape), dWr
    [E, H] float32, dWg, dWu [E, I, H], dWd [E, H, I].  The routing (with the
    same capacity) is recomputed from x and Wr.  ``from_saved``: ``workspace``
    is the ``saved`` buffer of a training forward on the same inputs and
    arguments, and neither the routing nor g, u are recomputed.  ``aux_grad``
    and ``z_grad`` are floats or one-element float32 device tensors (read by
    the kernel: no host synchronisation)."""
    dev = x.device
    H = x.shape[-1]
    E, I = Wg.shape[0], Wg.shape[1]
    xf = x.reshape(-1, H)
    N = xf.shape[0]
    dt = x.dtype
    dyf = dy.reshape(-1, H)
    _need(xf, "x", (N, H), dt, dev)
    _need(Wr, "Wr", (E, H), torch.float32, dev)
    _need(Wg, "Wg", (E, I, H), dt, dev)
    _need(Wu, "Wu", (E, I, H), dt, dev)
    _need(Wd, "Wd", (E, H, I), dt, dev)
    _need(dyf, "dy", (N, H), dt, dev)
    new = lambda shape, d=dt: torch.empty(shape, dtype=d, device=dev)
    dx, dWr = new((N, H)), new((E, H), torch.float32)
    dWg, dWu, dWd = new((E, I, H)), new((E, I, H)), new((E, H, I))
    code = _dtype_code(dt)
    nbytes = B.raw_moe_bwd_workspace_bytes(N, H, I, E, k, code)
    if nbytes == 0:
        B.check(B.ERR_BAD_SHAPE, "moe_ffn_bwd")
    if from_saved and workspace is None:
        raise ValueError("from_saved needs the training forward's saved buffer as workspace")
    ws = _workspace(nbytes, dev, workspace)
    flags = (0 if norm_topk_prob else B.MOE_RAW_TOPK_WEIGHTS) | (B.MOE_BWD_SAVED if from_saved else 0)

    def scalar(v, name):  # (host factor, device scalar or None)
        if isinstance(v, torch.Tensor):
            t = v.reshape(-1)
            _need(t, name, (1,), torch.float32, dev)
            return 1.0, t
        return float(v), None

    ag, ag_t = scalar(aux_grad, "aux_grad")
    zg, zg_t = scalar(z_grad, "z_grad")
    st = B.raw_moe_ffn_bwd(_ptr(xf), _ptr(Wr), _ptr(Wg), _ptr(Wu), _ptr(Wd), _ptr(dyf),
                           ag, zg, _ptr(ag_t), _ptr(zg_t), N, H, I, E, k, float(aux_coef),
                           float(z_coef), float(capacity_factor), flags, code,
                           _ptr(dx), _ptr(dWr), _ptr(dWg), _ptr(dWu), _ptr(dWd), _ptr(ws),
                           ws.numel() * ws.element_size(), _stream(dev, stream),
                           stage_events.ptr if stage_events is not None else None)
    B.check(st, "moe_ffn_bwd")
    return MoeGrads(dx.view(x.shape), dWr, dWg, dWu, dWd)
