"""C ABI checks that need no GPU: the library loads, exports every function
include/topmoe.h declares, sizes its workspace, and rejects bad arguments
before launching anything (every call here fails validation on the host)."""
import ctypes
import os
import re

import pytest

import top_moe_layer_amd as tm
from top_moe_layer_amd import _binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "topmoe.h")


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    names = re.findall(r"^[A-Za-z_][\w \*]*?\b([a-z_][a-z0-9_]*)\s*\(", src, flags=re.M)
    return sorted(set(n for n in names if n not in ("defined",)))


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(B.LIB_PATH):
        pytest.fail("libtopmoe.so is not built (run python -m top_moe_layer_amd.build)")
    return B.lib()


def test_header_declares_expected_functions():
    assert declared_functions() == sorted(B.SIGNATURES)


def test_library_exports_every_declared_symbol(L):
    for name in declared_functions():
        assert hasattr(L, name), name
    assert L.topmoe_version() == 151


def test_strerror_covers_codes(L):
    for code in (B.OK, B.ERR_NULL_ARG, B.ERR_BAD_SHAPE, B.ERR_UNSUPPORTED_DTYPE,
                 B.ERR_WORKSPACE_TOO_SMALL, B.ERR_HIP, B.ERR_BAD_ARG, B.ERR_SCRATCH_TOO_SMALL):
        assert B.strerror(code) != "unknown status"
    assert B.strerror(-99) == "unknown status"


def test_workspace_sizes(L):
    # dense: the [N, I] intermediate
    assert B.raw_ffn_workspace_bytes(100, 768, 2432, B.DTYPE_FP32) >= 100 * 2432 * 4
    assert B.raw_ffn_workspace_bytes(16384, 2048, 6464, B.DTYPE_BF16) >= 16384 * 6464 * 2
    # moe: intermediate [N*k, I] plus the k-slots [N*k, H] (dtype) when k >= 2
    # (none for k = 1: the down GEMM writes y, also under a capacity)
    w1 = B.raw_moe_workspace_bytes(4096, 768, 2432, 4, 1, B.DTYPE_BF16)
    assert 4096 * 2432 * 2 <= w1 < 4096 * 2432 * 2 + 4096 * 16 + 65536
    w2 = B.raw_moe_workspace_bytes(16384, 768, 2432, 8, 2, B.DTYPE_BF16)
    assert w2 >= 32768 * 2432 * 2 + 32768 * 768 * 2
    w3 = B.raw_moe_workspace_bytes(16384, 768, 2432, 8, 2, B.DTYPE_FP32)
    assert w3 >= 32768 * 2432 * 4 + 32768 * 768 * 4
    assert B.raw_moe_workspace_bytes(0, 64, 64, 4, 2, B.DTYPE_BF16) > 0
    for args in [(10, 65, 64, 4, 1), (10, 64, 96, 4, 1), (10, 64, 64, 0, 1), (10, 64, 64, 65, 1),
                 (10, 64, 64, 4, 5), (10, 64, 64, 4, 0), (-1, 64, 64, 4, 1), (2**31, 64, 64, 4, 1)]:
        assert B.raw_moe_workspace_bytes(*args, B.DTYPE_BF16) == 0, args
    assert B.raw_moe_workspace_bytes(10, 64, 64, 4, 1, 7) == 0
    assert B.raw_ffn_workspace_bytes(10, 64, 32, B.DTYPE_BF16) == 0


FAKE = 1 << 20  # 256-byte aligned, never dereferenced: validation fails first


def moe_call(**over):
    a = dict(x=FAKE, Wr=FAKE, Wg=FAKE, Wu=FAKE, Wd=FAKE, residual=None, N=8, H=64, I=64, E=4, k=2,
             coef=0.01, z_coef=0.0, capacity_factor=0.0, flags=0, dtype=B.DTYPE_BF16, y=FAKE,
             topk_idx=FAKE, alpha=FAKE, aux=FAKE, z_loss=None, offsets=None,
             sorted_ids=None, ws=FAKE, ws_bytes=0, stream=None, events=None)
    a.update(over)
    return B.raw_moe_ffn_fwd(*a.values())


def ffn_call(**over):
    a = dict(x=FAKE, Wg=FAKE, Wu=FAKE, Wd=FAKE, residual=None, y=FAKE, N=8, H=64, I=64,
             dtype=B.DTYPE_BF16,
             ws=FAKE, ws_bytes=0, stream=None, events=None)
    a.update(over)
    return B.raw_ffn_swiglu_fwd(*a.values())


def test_moe_validation_codes(L):
    assert moe_call(x=None) == B.ERR_NULL_ARG
    # N == 0: the zero-size tensors may be NULL (validation reaches the workspace check)
    assert moe_call(N=0, x=None, y=None, topk_idx=None, alpha=None) == B.ERR_WORKSPACE_TOO_SMALL
    assert moe_call(N=0, aux=None) == B.ERR_NULL_ARG
    assert moe_call(aux=None) == B.ERR_NULL_ARG
    assert moe_call(ws=None) == B.ERR_NULL_ARG
    assert moe_call(H=96) == B.ERR_BAD_SHAPE
    assert moe_call(I=32) == B.ERR_BAD_SHAPE
    assert moe_call(E=65, k=1) == B.ERR_BAD_SHAPE
    assert moe_call(k=5) == B.ERR_BAD_SHAPE
    assert moe_call(k=0) == B.ERR_BAD_SHAPE
    assert moe_call(N=-3) == B.ERR_BAD_SHAPE
    # every GEMM operand below 4 GiB: x (N*H), the intermediate (N*k*I), one expert's weights
    assert moe_call(N=1 << 21, H=1024, k=1) == B.ERR_BAD_SHAPE            # x = 4 GiB bf16
    assert moe_call(N=(1 << 21) - 1, H=1024, k=1) == B.ERR_WORKSPACE_TOO_SMALL
    assert moe_call(N=1 << 20, I=1024, k=2) == B.ERR_BAD_SHAPE            # h = 4 GiB bf16
    assert moe_call(H=1 << 16, I=1 << 15) == B.ERR_BAD_SHAPE              # W_e = 4 GiB bf16
    assert moe_call(H=1 << 16, I=(1 << 15) - 64) == B.ERR_WORKSPACE_TOO_SMALL
    assert moe_call(H=1 << 15, I=1 << 15, dtype=B.DTYPE_FP32) == B.ERR_BAD_SHAPE
    assert moe_call(dtype=2) == B.ERR_UNSUPPORTED_DTYPE
    assert moe_call(coef=-0.5) == B.ERR_BAD_ARG
    assert moe_call(coef=float("nan")) == B.ERR_BAD_ARG
    assert moe_call(coef=float("inf")) == B.ERR_BAD_ARG
    assert moe_call() == B.ERR_WORKSPACE_TOO_SMALL
    need = B.raw_moe_workspace_bytes(8, 64, 64, 4, 2, B.DTYPE_BF16)
    assert moe_call(ws_bytes=need - 1) == B.ERR_WORKSPACE_TOO_SMALL
    assert moe_call(ws_bytes=need, x=FAKE + 8) == B.ERR_BAD_ARG
    assert moe_call(ws_bytes=need, ws=FAKE + 64) == B.ERR_BAD_ARG
    assert moe_call(ws_bytes=need, alpha=FAKE + 2) == B.ERR_BAD_ARG
    assert moe_call(ws_bytes=need, residual=FAKE + 8) == B.ERR_BAD_ARG
    assert moe_call(ws_bytes=need, flags=2) == B.ERR_BAD_ARG
    assert moe_call(ws_bytes=need, flags=8) == B.ERR_BAD_ARG
    assert moe_call(flags=B.MOE_EVAL | B.MOE_RAW_TOPK_WEIGHTS) == B.ERR_WORKSPACE_TOO_SMALL
    assert moe_call(ws_bytes=need, flags=-1) == B.ERR_BAD_ARG
    assert moe_call(z_coef=-0.1) == B.ERR_BAD_ARG
    assert moe_call(z_coef=float("inf")) == B.ERR_BAD_ARG
    assert moe_call(capacity_factor=-1.0) == B.ERR_BAD_ARG
    assert moe_call(capacity_factor=float("nan")) == B.ERR_BAD_ARG
    assert moe_call(ws_bytes=need, z_loss=FAKE + 2) == B.ERR_BAD_ARG


def test_ffn_validation_codes(L):
    assert ffn_call(y=None) == B.ERR_NULL_ARG
    assert ffn_call(N=0, x=None, y=None) == B.ERR_WORKSPACE_TOO_SMALL
    assert ffn_call(H=0) == B.ERR_BAD_SHAPE
    assert ffn_call(I=100) == B.ERR_BAD_SHAPE
    assert ffn_call(N=1 << 20, I=2048) == B.ERR_BAD_SHAPE                  # h = 4 GiB bf16
    assert ffn_call(N=1 << 20, I=2048 - 64) == B.ERR_WORKSPACE_TOO_SMALL
    assert ffn_call(dtype=-1) == B.ERR_UNSUPPORTED_DTYPE
    assert ffn_call() == B.ERR_WORKSPACE_TOO_SMALL
    need = B.raw_ffn_workspace_bytes(8, 64, 64, B.DTYPE_BF16)
    assert ffn_call(ws_bytes=need, Wd=FAKE + 4) == B.ERR_BAD_ARG
    assert ffn_call(ws_bytes=need, residual=FAKE + 4) == B.ERR_BAD_ARG


def ffn_bwd_call(**over):
    a = dict(x=FAKE, Wg=FAKE, Wu=FAKE, Wd=FAKE, dy=FAKE, dx=FAKE, dWg=FAKE, dWu=FAKE, dWd=FAKE,
             N=8, H=64, I=64, dtype=B.DTYPE_BF16, ws=FAKE, ws_bytes=0, stream=None, events=None)
    a.update(over)
    return B.raw_ffn_swiglu_bwd(*a.values())


def moe_bwd_call(**over):
    a = dict(x=FAKE, Wr=FAKE, Wg=FAKE, Wu=FAKE, Wd=FAKE, dy=FAKE, aux_grad=1.0, z_grad=1.0,
             aux_grad_scale=None, z_grad_scale=None, N=8, H=64, I=64, E=4, k=2, coef=0.01, z_coef=0.0, capacity_factor=0.0, flags=0,
             dtype=B.DTYPE_BF16, dx=FAKE, dWr=FAKE, dWg=FAKE, dWu=FAKE, dWd=FAKE, ws=FAKE,
             ws_bytes=0, stream=None, events=None)
    a.update(over)
    return B.raw_moe_ffn_bwd(*a.values())


def test_bwd_workspace_sizes(L):
    # dense: [Wg|Wu]^T, Wd^T, x^T and dy^T [H, round64(N)], the (g, u) pairs [N, I],
    # [dg|du], dg^T / du^T / h^T
    N, H, I = 100, 128, 192
    w = B.raw_ffn_bwd_workspace_bytes(N, H, I, B.DTYPE_BF16)
    Np = 128
    floor = 2 * (3 * H * I + 2 * H * Np + 2 * N * I + 2 * N * I + 3 * I * Np)
    assert floor <= w < floor + 16 * 256
    assert B.raw_ffn_bwd_workspace_bytes(N, H, I, B.DTYPE_FP32) >= 2 * floor
    assert B.raw_ffn_bwd_workspace_bytes(0, H, I, B.DTYPE_BF16) > 0
    assert B.raw_ffn_bwd_workspace_bytes(N, 96, I, B.DTYPE_BF16) == 0
    # moe: at least the forward's routing plus the per-entry buffers
    N, H, I, E, k = 300, 128, 128, 8, 2
    wm = B.raw_moe_bwd_workspace_bytes(N, H, I, E, k, B.DTYPE_BF16)
    rows = N * k
    assert wm >= 2 * (3 * E * H * I + rows * 2 * I + rows * H) + 4 * N * E * 2
    assert B.raw_moe_bwd_workspace_bytes(0, H, I, E, k, B.DTYPE_BF16) > 0
    assert B.raw_moe_bwd_workspace_bytes(N, H, I, E, E + 1, B.DTYPE_BF16) == 0
    assert B.raw_moe_bwd_workspace_bytes(N, H, I, 65, 1, B.DTYPE_BF16) == 0


def test_bwd_validation_codes(L):
    assert ffn_bwd_call(dy=None) == B.ERR_NULL_ARG
    assert ffn_bwd_call(dWd=None) == B.ERR_NULL_ARG
    assert ffn_bwd_call(N=0, x=None, dy=None, dx=None) == B.ERR_WORKSPACE_TOO_SMALL
    assert ffn_bwd_call(N=0, dWg=None) == B.ERR_NULL_ARG
    assert ffn_bwd_call(I=100) == B.ERR_BAD_SHAPE
    assert ffn_bwd_call(N=1 << 20, I=1024) == B.ERR_BAD_SHAPE      # [dg|du] = 4 GiB bf16
    assert ffn_bwd_call(dtype=5) == B.ERR_UNSUPPORTED_DTYPE
    assert ffn_bwd_call() == B.ERR_WORKSPACE_TOO_SMALL
    need = B.raw_ffn_bwd_workspace_bytes(8, 64, 64, B.DTYPE_BF16)
    assert ffn_bwd_call(ws_bytes=need - 1) == B.ERR_WORKSPACE_TOO_SMALL
    assert ffn_bwd_call(ws_bytes=need, dy=FAKE + 8) == B.ERR_BAD_ARG
    assert ffn_bwd_call(ws_bytes=need, dWu=FAKE + 2) == B.ERR_BAD_ARG

    assert moe_bwd_call(dWr=None) == B.ERR_NULL_ARG
    assert moe_bwd_call(dy=None) == B.ERR_NULL_ARG
    assert moe_bwd_call(N=0, x=None, dy=None, dx=None) == B.ERR_WORKSPACE_TOO_SMALL
    assert moe_bwd_call(k=5) == B.ERR_BAD_SHAPE
    assert moe_bwd_call(N=1 << 20, I=1024) == B.ERR_BAD_SHAPE      # [dg|du] = 8 GiB bf16
    assert moe_bwd_call(coef=-1.0) == B.ERR_BAD_ARG
    assert moe_bwd_call(aux_grad=float("nan")) == B.ERR_BAD_ARG
    assert moe_bwd_call(aux_grad=float("inf")) == B.ERR_BAD_ARG
    assert moe_bwd_call(flags=8) == B.ERR_BAD_ARG
    assert moe_bwd_call(flags=B.MOE_EVAL) == B.ERR_WORKSPACE_TOO_SMALL  # a known flag
    assert moe_bwd_call(aux_grad_scale=FAKE + 2) == B.ERR_BAD_ARG
    assert moe_bwd_call(z_grad=float("nan")) == B.ERR_BAD_ARG
    assert moe_bwd_call(z_coef=-1.0) == B.ERR_BAD_ARG
    assert moe_bwd_call(capacity_factor=float("inf")) == B.ERR_BAD_ARG
    assert moe_bwd_call() == B.ERR_WORKSPACE_TOO_SMALL
    need = B.raw_moe_bwd_workspace_bytes(8, 64, 64, 4, 2, B.DTYPE_BF16)
    assert moe_bwd_call(ws_bytes=need - 1) == B.ERR_WORKSPACE_TOO_SMALL
    assert moe_bwd_call(ws_bytes=need, dWr=FAKE + 4) == B.ERR_BAD_ARG
    assert moe_bwd_call(ws_bytes=need, ws=FAKE + 16) == B.ERR_BAD_ARG


def ffn_train_call(**over):
    a = dict(x=FAKE, Wg=FAKE, Wu=FAKE, Wd=FAKE, residual=None, y=FAKE, N=8, H=64, I=64,
             dtype=B.DTYPE_BF16, ws=FAKE, ws_bytes=0, saved=FAKE, saved_bytes=0, stream=None,
             events=None)
    a.update(over)
    return B.raw_ffn_swiglu_fwd_train(*a.values())


def moe_train_call(**over):
    a = dict(x=FAKE, Wr=FAKE, Wg=FAKE, Wu=FAKE, Wd=FAKE, residual=None, N=8, H=64, I=64, E=4, k=2,
             coef=0.01, z_coef=0.0, capacity_factor=0.0, flags=0, dtype=B.DTYPE_BF16, y=FAKE,
             topk_idx=FAKE, alpha=FAKE, aux=FAKE, z_loss=None, offsets=None,
             sorted_ids=None, ws=FAKE, ws_bytes=0, saved=FAKE, saved_bytes=0, stream=None,
             events=None)
    a.update(over)
    return B.raw_moe_ffn_fwd_train(*a.values())


def test_train_forward_validation_codes(L):
    # the saved buffer is a backward workspace: its size, presence and alignment are checked
    # first, then everything the plain forward checks
    nb = B.raw_ffn_bwd_workspace_bytes(8, 64, 64, B.DTYPE_BF16)
    nf = B.raw_ffn_workspace_bytes(8, 64, 64, B.DTYPE_BF16)
    assert ffn_train_call(saved=None, saved_bytes=nb) == B.ERR_NULL_ARG
    assert ffn_train_call(saved_bytes=nb - 1) == B.ERR_WORKSPACE_TOO_SMALL
    assert ffn_train_call(saved_bytes=nb, saved=FAKE + 128) == B.ERR_BAD_ARG
    assert ffn_train_call(saved_bytes=nb) == B.ERR_WORKSPACE_TOO_SMALL
    assert ffn_train_call(saved_bytes=nb, ws_bytes=nf, y=None) == B.ERR_NULL_ARG
    assert ffn_train_call(saved_bytes=nb, ws_bytes=nf, Wd=FAKE + 4) == B.ERR_BAD_ARG
    assert ffn_train_call(H=96, saved_bytes=nb) == B.ERR_BAD_SHAPE
    assert ffn_train_call(dtype=3, saved_bytes=nb) == B.ERR_UNSUPPORTED_DTYPE

    mb = B.raw_moe_bwd_workspace_bytes(8, 64, 64, 4, 2, B.DTYPE_BF16)
    mf = B.raw_moe_workspace_bytes(8, 64, 64, 4, 2, B.DTYPE_BF16)
    assert moe_train_call(saved=None, saved_bytes=mb) == B.ERR_NULL_ARG
    assert moe_train_call(saved_bytes=mb - 1) == B.ERR_WORKSPACE_TOO_SMALL
    assert moe_train_call(saved_bytes=mb, saved=FAKE + 16) == B.ERR_BAD_ARG
    assert moe_train_call(saved_bytes=mb) == B.ERR_WORKSPACE_TOO_SMALL
    assert moe_train_call(saved_bytes=mb, ws_bytes=mf, alpha=None) == B.ERR_NULL_ARG
    assert moe_train_call(saved_bytes=mb, ws_bytes=mf, flags=B.MOE_BWD_SAVED) == B.ERR_BAD_ARG
    assert moe_train_call(saved_bytes=mb, ws_bytes=mf, coef=-1.0) == B.ERR_BAD_ARG
    assert moe_train_call(k=5, saved_bytes=mb) == B.ERR_BAD_SHAPE
    # the backward from the saved buffer validates as the recomputing one does
    fb = dict(x=FAKE, Wg=FAKE, Wu=FAKE, Wd=FAKE, dy=FAKE, dx=FAKE, dWg=FAKE, dWu=FAKE, dWd=FAKE,
              N=8, H=64, I=64, dtype=B.DTYPE_BF16, ws=FAKE, ws_bytes=nb - 1, stream=None,
              events=None)
    assert B.raw_ffn_swiglu_bwd_saved(*fb.values()) == B.ERR_WORKSPACE_TOO_SMALL
    fb.update(ws_bytes=nb, dy=None)
    assert B.raw_ffn_swiglu_bwd_saved(*fb.values()) == B.ERR_NULL_ARG
    assert moe_bwd_call(flags=B.MOE_BWD_SAVED) == B.ERR_WORKSPACE_TOO_SMALL
    assert moe_bwd_call(flags=B.MOE_BWD_SAVED | B.MOE_RAW_TOPK_WEIGHTS, ws_bytes=mb,
                        dWr=FAKE + 4) == B.ERR_BAD_ARG


def test_torch_front_end_rejects_bad_tensors():
    torch = pytest.importorskip("torch")
    x = torch.zeros(4, 64)
    w = torch.zeros(64, 64)
    with pytest.raises(ValueError, match="GPU tensor"):
        tm.ffn_swiglu_fwd(x, w, w, w)
    with pytest.raises(ValueError, match="GPU tensor"):
        tm.moe_ffn_fwd(x, torch.zeros(4, 64), torch.zeros(4, 64, 64), torch.zeros(4, 64, 64),
                       torch.zeros(4, 64, 64), 1, 0.01)


def test_torch_front_end_checks_caller_buffers():
    torch = pytest.importorskip("torch")
    from top_moe_layer_amd import ops

    cpu, gpu = torch.device("cpu"), torch.device("cuda:0")
    with pytest.raises(ValueError, match="expected cuda:0"):
        ops._buffer(torch.empty(64, dtype=torch.uint8), "saved", 16, gpu)
    with pytest.raises(ValueError, match="needs 128"):
        ops._buffer(torch.empty(64, dtype=torch.uint8), "workspace", 128, cpu)
    with pytest.raises(ValueError, match="contiguous"):
        ops._buffer(torch.empty(64, 2, dtype=torch.uint8).t(), "saved", 16, cpu)
    ok = torch.empty(32, dtype=torch.float32)
    assert ops._buffer(ok, "saved", 128, cpu) is ok


def test_tile_override_is_validated(L):
    """A launch-shape override must name a shape the library instantiates for
    that GEMM; a rejected one changes nothing."""
    try:
        with pytest.raises(B.TopmoeError, match="status -6"):
            B.set_tile_override("gateup", "96x96x2x2x128x2")            # not instantiated
        with pytest.raises(B.TopmoeError, match="status -6"):
            B.set_tile_override("gateup", "256x256x4x2x128x2")          # LDS ring too big here
        assert L.topmoe_set_tile_override(9, None) == B.ERR_BAD_ARG
        B.set_tile_override("down", "256x256x4x2x128x2")
        B.set_tile_override("gateup", (128, 128, 2, 4, 128, 3))
        assert B.raw_moe_workspace_bytes(300, 64, 64, 4, 2, B.DTYPE_BF16) > 0
    finally:
        for g in B.TILE_SLOTS:
            B.set_tile_override(g, None)


def test_invalid_environment_override_fails_before_launch():
    """The environment's overrides are read once; one that names a shape that
    is not instantiated makes the calls that would use it fail validation."""
    import subprocess
    import sys

    code = ("from top_moe_layer_amd import _binding as B\n"
            "print(B.raw_ffn_workspace_bytes(64, 64, 64, B.DTYPE_BF16),"
            " B.raw_moe_workspace_bytes(64, 64, 64, 4, 2, B.DTYPE_BF16))")
    env = dict(os.environ, TOPMOE_DOWN_TILE="100x100x2x2x128x2")
    r = subprocess.run([sys.executable, "-c", code], env=env, capture_output=True, text=True,
                       cwd=ROOT, timeout=60)
    assert r.returncode == 0, r.stderr
    assert r.stdout.split() == ["0", "0"]
    env = dict(os.environ, TOPMOE_DOWN_TILE="128x128x2x4x128x3")
    r = subprocess.run([sys.executable, "-c", code], env=env, capture_output=True, text=True,
                       cwd=ROOT, timeout=60)
    assert r.returncode == 0 and all(int(v) > 0 for v in r.stdout.split()), (r.stdout, r.stderr)


def test_front_end_allocates_on_the_kernels_stream(monkeypatch):
    """The torch front end makes the kernels' stream torch's current stream
    while it allocates outputs and workspaces, so the caching allocator ties
    them to that stream."""
    torch = pytest.importorskip("torch")
    from top_moe_layer_amd import ops

    entered = []

    class FakeCtx:
        def __init__(self, s):
            self.s = s

        def __enter__(self):
            entered.append(self.s)

        def __exit__(self, *a):
            entered.append("exit")

    class FakeDev:
        type = "cuda"

    class FakeTensor(torch.Tensor):
        pass

    x = torch.zeros(2).as_subclass(FakeTensor)
    monkeypatch.setattr(FakeTensor, "device", property(lambda self: FakeDev()))
    monkeypatch.setattr(ops.torch.cuda, "stream", FakeCtx)
    monkeypatch.setattr(ops, "_torch_stream", lambda dev, st: ("stream", st))
    seen = []

    @ops._on_caller_stream
    def fn(x, *, stream=None):
        seen.append((stream, list(entered)))
        return 7

    assert fn(x, stream=1234) == 7
    assert seen == [(("stream", 1234), [("stream", 1234)])]
    assert entered[-1] == "exit"


def test_noalloc_size_limit_checked_first(L):
    """The no-allocation forward rejects a problem whose workspace exceeds its
    fixed scratch before touching any device (shape errors come first)."""
    args = lambda N, k: (FAKE, FAKE, FAKE, FAKE, FAKE, None, N, 768, 2432, 8, k, 0.01, 0.0, 0.0, 0,
                         B.DTYPE_BF16, FAKE, FAKE, FAKE, FAKE, None, None, None, None, None)
    assert B.raw_moe_workspace_bytes(16384, 768, 2432, 8, 2, B.DTYPE_BF16) > B.NOALLOC_SCRATCH_BYTES
    assert B.raw_moe_ffn_fwd_noalloc(*args(16384, 2)) == B.ERR_SCRATCH_TOO_SMALL
    assert B.raw_moe_ffn_fwd_noalloc(*args(16384, 9)) == B.ERR_BAD_SHAPE


def test_forward_path(L):
    """The launch plan the forward follows (host logic): decode-sized calls
    route inside the GEMM launches, a capacity or a large batch does not."""
    dec = B.moe_fwd_path(32, 2048, 1408, 16, 2, B.DTYPE_BF16)
    assert dec == dict(router_layout=1, router_tokens=1, router_blocks=32, up_bm=64, up_bn=128,
                       up_ring=3, down_bm=64, down_bn=128, down_ring=3, down_ksplit=1, inblock=1,
                       router_in_up=1)
    capped = B.moe_fwd_path(32, 2048, 1408, 16, 2, B.DTYPE_BF16, capacity_factor=1.25)
    assert capped["inblock"] == 0 and capped["router_in_up"] == 0
    more_tokens = B.moe_fwd_path(200, 2048, 1408, 16, 2, B.DTYPE_BF16)
    assert more_tokens["inblock"] == 1 and more_tokens["router_in_up"] == 0
    many_experts = B.moe_fwd_path(37, 192, 320, 64, 6, B.DTYPE_BF16)
    assert many_experts["inblock"] == 1 and many_experts["router_in_up"] == 0
    top1 = B.moe_fwd_path(4096, 768, 2432, 4, 1, B.DTYPE_BF16)
    assert top1["inblock"] == 0 and top1["router_in_up"] == 0 and top1["router_blocks"] * top1[
        "router_tokens"] >= 4096
    # fields past the last read -1; errors as moe_ffn_fwd reports them
    info = (ctypes.c_int32 * (len(B.PATH_FIELDS) + 2))()
    assert L.moe_ffn_fwd_path(32, 2048, 1408, 16, 2, 0.0, B.DTYPE_BF16, info, len(info)) == B.OK
    assert list(info)[-2:] == [-1, -1]
    assert L.moe_ffn_fwd_path(32, 2048, 1408, 16, 2, -1.0, B.DTYPE_BF16, info, 4) == B.ERR_BAD_ARG
    assert L.moe_ffn_fwd_path(32, 2048, 1408, 16, 2, 0.0, B.DTYPE_BF16, None, 4) == B.ERR_NULL_ARG
    assert L.moe_ffn_fwd_path(32, 2048, 1408, 0, 2, 0.0, B.DTYPE_BF16, info, 4) == B.ERR_BAD_SHAPE
