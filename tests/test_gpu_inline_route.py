"""Decode-sized MoE calls (at most 512 entries on the 64 x 128 weight-streaming
tiles) group the entries by expert inside the two GEMM kernels instead of in
the permutation kernel; an extra block of one of the GEMM launches writes the
offsets, the token lists, aux and the z-loss.  With E <= 16 and one token per
router block the router itself runs as blocks of the gate/up launch, which
takes every token against every expert.  Every output against the oracle:
lists and offsets bit-exact, alpha / aux / z to 1e-5, y to the bf16 bar."""
import numpy as np
import pytest

from oracle import moe_ffn
from oracle.cases import custom_workload, make_case, widen
from gpu_util import (TOL_Y, announce, check_routing, rel_l2_per_token, to_dev, torch_dev,
                      y_to_f64)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def env():
    torch, dev = torch_dev()
    import top_moe_layer_amd as tm

    tm.lib()
    return torch, dev, tm


CASES = [  # N, H, I, E, k, z_coef, residual, (in-block routing, router in the gate/up launch)
    (32, 2048, 1408, 16, 2, 0.001, True, (1, 1)),
    (1, 256, 384, 8, 2, 0.0, False, (1, 1)),
    (5, 128, 256, 4, 1, 0.002, False, (1, 1)),      # k = 1: the down GEMM writes y
    (100, 256, 512, 8, 2, 0.0, True, (0, 0)),       # split-K down projection: permutation kernel
    (256, 128, 128, 16, 2, 0.001, False, (1, 0)),   # 512 entries, the most in-block routing
                                                    # takes; the LDS router layout
    (37, 192, 320, 64, 6, 0.0, False, (1, 0)),      # E > 16: the router launch stays
    (64, 1024, 512, 16, 1, 0.001, True, (1, 1)),    # one full row tile of tokens
    (16, 2048, 1408, 16, 4, 0.0, False, (1, 1)),
    (200, 2048, 1408, 16, 2, 0.0, True, (1, 0)),    # more tokens than one row tile
    (8, 256, 256, 1, 1, 0.001, True, (1, 1)),       # one expert
    (8, 256, 256, 2, 2, 0.0, False, (1, 1)),        # k = E
]


@pytest.mark.parametrize("N,H,I,E,k,zc,res,path", CASES)
def test_inline_routing(env, N, H, I, E, k, zc, res, path):
    torch, dev, tm = env
    from top_moe_layer_amd import _binding as B

    plan = B.moe_fwd_path(N, H, I, E, k, B.DTYPE_BF16)
    assert (plan["inblock"], plan["router_in_up"]) == path, plan

    w = custom_workload(name="inl", N=N, H=H, I=I, E=E, k=k, coef=0.01, residual=res,
                        seed=N * 7 + E)
    assert N * k <= 512 and N * k <= 32 * E  # the decode-sized plan
    inp = make_case(w)
    f = widen(inp)
    ref = moe_ffn(f["x"], f["Wr"], f["Wg"], f["Wu"], f["Wd"], k, w.coef,
                  residual=f.get("residual"), z_coef=zc)
    announce(f"moe_ffn_fwd in-block routing N={N} H={H} I={I} E={E} k={k} z={zc} res={res}")
    d = to_dev(inp, dev)
    out = tm.moe_ffn_fwd(d["x"], d["Wr"], d["Wg"], d["Wu"], d["Wd"], k, w.coef,
                         residual=d.get("residual"), z_coef=zc)
    torch.cuda.synchronize()
    check_routing(out, ref, k, E, exact_order=k < E)
    if zc:
        z = float(out.z_loss.cpu()[0])
        assert abs(z - ref["z_loss"]) <= 1e-5 * ref["z_loss"], (z, ref["z_loss"])
    err = rel_l2_per_token(y_to_f64(out.y), ref["y"])
    assert err <= TOL_Y["bf16"], err
    # the no-allocation entry point takes the same path: the same bits
    y2 = torch.empty_like(out.y)
    idx2 = torch.empty_like(out.topk_idx)
    al2 = torch.empty_like(out.alpha)
    aux2 = torch.empty_like(out.aux_loss)
    p = lambda t: 0 if t is None else t.data_ptr()
    r = d.get("residual")
    st = B.raw_moe_ffn_fwd_noalloc(p(d["x"]), p(d["Wr"]), p(d["Wg"]), p(d["Wu"]), p(d["Wd"]),
                                   p(r), N, H, I, E, k, w.coef, zc, 0.0, 0, B.DTYPE_BF16, p(y2),
                                   p(idx2), p(al2), p(aux2), None, None, None,
                                   torch.cuda.current_stream(dev).cuda_stream, None)
    B.check(st, "moe_ffn_fwd_noalloc")
    torch.cuda.synchronize()
    assert torch.equal(y2.view(torch.int16), out.y.view(torch.int16))
    assert torch.equal(aux2, out.aux_loss)


@pytest.mark.parametrize("N,H,I,E,k,norm,training", [
    (32, 2048, 1408, 16, 2, False, True),   # router inside the gate/up launch, alpha = p_S
    (32, 2048, 1408, 16, 2, True, False),   # the module outside training: aux = 0
    (37, 192, 320, 64, 6, False, True),     # in-block grouping with the router launch
])
def test_inline_routing_flags(env, N, H, I, E, k, norm, training):
    torch, dev, tm = env
    w = custom_workload(name="inl_flags", N=N, H=H, I=I, E=E, k=k, coef=0.01, seed=N * 5 + E)
    inp = make_case(w)
    f = widen(inp)
    ref = moe_ffn(f["x"], f["Wr"], f["Wg"], f["Wu"], f["Wd"], k, w.coef, norm_topk_prob=norm)
    announce(f"moe_ffn_fwd in-block routing flags N={N} E={E} k={k} norm={norm} training={training}")
    d = to_dev(inp, dev)
    out = tm.moe_ffn_fwd(d["x"], d["Wr"], d["Wg"], d["Wu"], d["Wd"], k, w.coef,
                         norm_topk_prob=norm, training=training)
    torch.cuda.synchronize()
    if training:
        check_routing(out, ref, k, E, exact_order=k < E)
    else:
        assert float(out.aux_loss.cpu()[0]) == 0.0
        assert np.array_equal(out.topk_idx.cpu().numpy(), ref["topk_idx"])
    err = rel_l2_per_token(y_to_f64(out.y), ref["y"])
    assert err <= TOL_Y["bf16"], err
