"""moe_ffn_fwd_noalloc (the MoE forward whose workspace is the library's fixed
device scratch, for callers that cannot allocate) against moe_ffn_fwd on the
same inputs: every output bit for bit, on two calls in a row, the second with
a smaller input (the scratch keeps the first call's contents)."""
import numpy as np
import pytest

from oracle.cases import custom_workload, make_case
from workloads import get
from gpu_util import announce, to_dev, torch_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def env():
    torch, dev = torch_dev()
    import top_moe_layer_amd as tm

    tm.lib()
    return torch, dev, tm


def call_noalloc(torch, dev, d, w, cf=0.0, z_coef=0.0):
    from top_moe_layer_amd import _binding as B

    N, H = d["x"].shape
    E, I = d["Wg"].shape[0], d["Wg"].shape[1]
    k = w.k
    dt = d["x"].dtype
    y = torch.empty((N, H), dtype=dt, device=dev)
    idx = torch.empty((N, k), dtype=torch.int32, device=dev)
    alpha = torch.empty((N, k), dtype=torch.float32, device=dev)
    aux = torch.empty((1,), dtype=torch.float32, device=dev)
    z = torch.empty((1,), dtype=torch.float32, device=dev) if z_coef else None
    offs = torch.empty((E + 1,), dtype=torch.int32, device=dev)
    ids = torch.empty((N * k,), dtype=torch.int32, device=dev)
    code = B.DTYPE_BF16 if dt == torch.bfloat16 else B.DTYPE_FP32
    p = lambda t: 0 if t is None else t.data_ptr()
    st = B.raw_moe_ffn_fwd_noalloc(p(d["x"]), p(d["Wr"]), p(d["Wg"]), p(d["Wu"]), p(d["Wd"]), None,
                                   N, H, I, E, k, w.coef, z_coef, cf, 0, code, p(y), p(idx),
                                   p(alpha), p(aux), p(z), p(offs), p(ids),
                                   torch.cuda.current_stream(dev).cuda_stream, None)
    B.check(st, "moe_ffn_fwd_noalloc")
    return dict(y=y, topk_idx=idx, alpha=alpha, aux_loss=aux, z_loss=z, expert_offsets=offs,
                sorted_token_ids=ids)


def same_bits(torch, a, b):
    a, b = a.contiguous(), b.contiguous()
    return a.shape == b.shape and torch.equal(a.view(torch.uint8), b.view(torch.uint8))


def test_noalloc_matches_the_allocating_forward(env):
    torch, dev, tm = env
    cases = [
        (get("moe_top1_n4096_h768_e4"), 0.0, 0.0),                       # 20 MB of scratch
        (custom_workload(name="noalloc_small", N=777, H=256, I=320, E=6, k=2, coef=0.01,
                         seed=41), 1.25, 0.002),                          # smaller, capacity, z
    ]
    for w, cf, zc in cases:
        announce(f"moe_ffn_fwd_noalloc {w.name} N={w.N} H={w.H} I={w.I} E={w.E} k={w.k} "
                 f"capacity={cf} z={zc}")
        d = to_dev(make_case(w), dev)
        got = call_noalloc(torch, dev, d, w, cf, zc)
        ref = tm.moe_ffn_fwd(d["x"], d["Wr"], d["Wg"], d["Wu"], d["Wd"], w.k, w.coef,
                             capacity_factor=cf, z_coef=zc)
        torch.cuda.synchronize()
        for n in ("y", "topk_idx", "alpha", "aux_loss", "expert_offsets", "sorted_token_ids"):
            assert same_bits(torch, got[n], getattr(ref, n)), n
        if zc:
            assert same_bits(torch, got["z_loss"], ref.z_loss)


def test_noalloc_rejects_problems_beyond_the_scratch(env):
    torch, dev, tm = env
    from top_moe_layer_amd import _binding as B

    w = get("moe_top2_skew_n16384_h768_e8")   # needs about 212 MB
    assert B.raw_moe_workspace_bytes(w.N, w.H, w.I, w.E, w.k, B.DTYPE_BF16) > B.NOALLOC_SCRATCH_BYTES
    st = B.raw_moe_ffn_fwd_noalloc(1 << 20, 1 << 20, 1 << 20, 1 << 20, 1 << 20, None, w.N, w.H,
                                   w.I, w.E, w.k, 0.01, 0.0, 0.0, 0, B.DTYPE_BF16, 1 << 20,
                                   1 << 20, 1 << 20, 1 << 20, None, None, None, None, None)
    assert st == B.ERR_SCRATCH_TOO_SMALL
