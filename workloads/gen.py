"""Seeded input generation.

Recipe (shared by every consumer; all values drawn in float64, then rounded
once to the storage dtype with round-to-nearest-even):

* x ~ N(0, 1), shape [N, H].
* Expert weights in nn.Linear [out, in] layout, ~ U(-1/sqrt(fan_in), +1/sqrt(fan_in)):
  Wg, Wu [E, I, H] (fan_in H); Wd [E, H, I] (fan_in I).  Dense cases drop E.
* Router weight Wr [E, H] ~ U(+-1/sqrt(H)), always stored fp32.
* Skewed routing: the router is bias-free, so a per-expert logit offset b is
  realised as one shared mean shift of the tokens, m = Wr^T (Wr Wr^T)^-1 b,
  x = round(z + m), which gives logits Wr z + b.  b = bias_scale * N(0, bias_std).
* Upstream gradient for the backward (make_upstream): dy ~ N(0, 1), shape
  [N, H], in the storage dtype.
* Every tensor has its own random stream: SeedSequence(seed, spawn_key=(crc32(name),)).
  A token row that must be redrawn uses the stream keyed (crc32("x_redraw"), t, attempt).

Storage: "fp32" arrays are numpy float32; "bf16" arrays are numpy uint16 holding
bf16 bit patterns.
"""
from __future__ import annotations

import zlib

import numpy as np

from .registry import Workload


# ---------------------------------------------------------------- rounding
def bf16_bits_from_f64(a) -> np.ndarray:
    """Round float64 values to bf16 (round-to-nearest-even), return uint16 bits.

    Done without double rounding: float64 -> float32 with round-to-odd (truncate
    toward zero, then set the last bit if anything was dropped), then float32 ->
    bf16 with round-to-nearest-even on the 16 dropped bits.  Round-to-odd at 24
    bits is exact enough for a following rounding to 8 bits.  NaN/Inf are not
    produced by the generator and are not handled.
    """
    a = np.asarray(a, dtype=np.float64)
    f = a.astype(np.float32)  # RNE to float32
    # step back toward zero where RNE rounded away from zero
    away = np.abs(f.astype(np.float64)) > np.abs(a)
    f = np.where(away, np.nextafter(f, np.float32(0)), f)
    bits = f.view(np.uint32).copy()
    inexact = f.astype(np.float64) != a
    bits |= inexact.astype(np.uint32)
    # float32 -> bf16, round to nearest even
    lsb = (bits >> 16) & np.uint32(1)
    rounded = (bits + np.uint32(0x7FFF) + lsb) >> 16
    return rounded.astype(np.uint16)


def f64_from_bf16_bits(b) -> np.ndarray:
    """Widen bf16 bit patterns to float64 exactly."""
    b = np.asarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def round_to(a, dtype: str) -> np.ndarray:
    if dtype == "fp32":
        return np.asarray(a, dtype=np.float64).astype(np.float32)
    if dtype == "bf16":
        return bf16_bits_from_f64(a)
    raise ValueError(dtype)


def to_f64(a, dtype: str) -> np.ndarray:
    """Exact float64 view of a stored tensor."""
    if dtype == "fp32":
        return np.asarray(a, dtype=np.float32).astype(np.float64)
    if dtype == "bf16":
        return f64_from_bf16_bits(a)
    raise ValueError(dtype)


# ---------------------------------------------------------------- streams
def _rng(seed: int, *key) -> np.random.Generator:
    spawn = tuple(zlib.crc32(k.encode()) if isinstance(k, str) else int(k) for k in key)
    return np.random.default_rng(np.random.SeedSequence(entropy=seed, spawn_key=spawn))


def _uniform(seed, name, shape, bound):
    return _rng(seed, name).uniform(-bound, bound, size=shape)


# ---------------------------------------------------------------- inputs
def _mean_shift(Wr64: np.ndarray, b: np.ndarray) -> np.ndarray:
    """m with Wr m = b (minimum-norm solution): m = Wr^T (Wr Wr^T)^-1 b."""
    return Wr64.T @ np.linalg.solve(Wr64 @ Wr64.T, b)


def make_inputs(w: Workload, seed: int | None = None, N: int | None = None) -> dict:
    """Draw every input tensor of workload ``w``.

    Returns a dict with storage-dtype arrays ``x, Wg, Wu, Wd`` (+ ``Wr`` fp32 for
    MoE) and metadata.  ``N`` overrides the token count (weights unchanged).
    """
    seed = w.seed if seed is None else seed
    N = w.N if N is None else N
    H, I, E, dt = w.H, w.I, w.E, w.dtype
    out = {"workload": w, "seed": seed, "N": N, "dtype": dt}
    if w.kind == "dense":
        out["Wg"] = round_to(_uniform(seed, "Wg", (I, H), 1 / np.sqrt(H)), dt)
        out["Wu"] = round_to(_uniform(seed, "Wu", (I, H), 1 / np.sqrt(H)), dt)
        out["Wd"] = round_to(_uniform(seed, "Wd", (H, I), 1 / np.sqrt(I)), dt)
    else:
        out["Wr"] = _uniform(seed, "Wr", (E, H), 1 / np.sqrt(H)).astype(np.float32)
        out["Wg"] = round_to(_uniform(seed, "Wg", (E, I, H), 1 / np.sqrt(H)), dt)
        out["Wu"] = round_to(_uniform(seed, "Wu", (E, I, H), 1 / np.sqrt(H)), dt)
        out["Wd"] = round_to(_uniform(seed, "Wd", (E, H, I), 1 / np.sqrt(I)), dt)
    shift = np.zeros(H)
    if w.kind == "moe" and w.bias_scale != 0.0:
        b = w.bias_scale * _rng(seed, "router_offset").normal(0.0, w.bias_std, size=E)
        shift = _mean_shift(out["Wr"].astype(np.float64), b)
        out["router_offset"] = b
    out["shift"] = shift
    z = _rng(seed, "x").standard_normal((N, H))
    out["x"] = round_to(z + shift, dt)
    if w.residual:
        out["residual"] = round_to(_rng(seed, "residual").standard_normal((N, H)), dt)
    return out


def make_upstream(inputs: dict, seed: int | None = None) -> np.ndarray:
    """The upstream gradient dy [N, H] (storage dtype) for ``inputs``."""
    seed = inputs["seed"] if seed is None else seed
    N, H = inputs["x"].shape
    return round_to(_rng(seed, "dy").standard_normal((N, H)), inputs["dtype"])


def redraw_token_rows(inputs: dict, rows, attempt: int) -> None:
    """Replace token rows ``rows`` of ``inputs['x']`` in place with fresh draws
    from the per-(token, attempt) stream.  Weights are never redrawn."""
    seed, dt, shift = inputs["seed"], inputs["dtype"], inputs["shift"]
    H = inputs["x"].shape[1]
    for t in np.asarray(rows, dtype=np.int64).ravel():
        z = _rng(seed, "x_redraw", int(t), int(attempt)).standard_normal(H)
        inputs["x"][t] = round_to(z + shift, dt)
