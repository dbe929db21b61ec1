"""The launch planner (host logic, no GPU): over a grid of shapes, every plan
moe_ffn_fwd_path reports keeps the invariants its kernels rely on."""
import itertools
import math

import pytest

from top_moe_layer_amd import _binding as B


@pytest.fixture(scope="module")
def lib():
    return B.lib()


def shapes():
    for N, H, I, E, k in itertools.product((1, 5, 32, 64, 65, 100, 255, 256, 1000, 4096),
                                           (128, 768, 2048), (128, 1408, 2432),
                                           (1, 4, 8, 16, 17, 64), (1, 2, 4)):
        if k <= E:
            yield N, H, I, E, k


@pytest.mark.parametrize("dtype", [B.DTYPE_BF16, B.DTYPE_FP32])
def test_plan_invariants(lib, dtype):
    elem = 2 if dtype == B.DTYPE_BF16 else 4
    seen = {"inblock": 0, "router_in_up": 0}
    for N, H, I, E, k in shapes():
        p = B.moe_fwd_path(N, H, I, E, k, dtype)
        rows = N * k
        assert p["router_blocks"] * p["router_tokens"] >= N, (N, p)
        assert (p["router_blocks"] - 1) * p["router_tokens"] < N, (N, p)
        if p["inblock"]:
            seen["inblock"] += 1
            assert rows <= 512
            assert (p["up_bm"], p["up_bn"], p["down_bm"], p["down_bn"]) == (64, 128, 64, 128)
            assert p["down_ksplit"] == 1
        if p["router_in_up"]:
            seen["router_in_up"] += 1
            assert p["inblock"] and E <= 16 and N <= p["up_bm"]
            assert p["router_layout"] == 1 and p["router_tokens"] == 1
            assert E * -(-I // p["up_bn"]) + p["router_blocks"] <= 256
        # the workspace holds h for every row the gate/up projection writes
        h_rows = max(E * N, rows) if p["router_in_up"] else rows
        assert B.raw_moe_workspace_bytes(N, H, I, E, k, dtype) >= h_rows * I * elem
        # a capacity that can drop entries (ceil(f N k / E) < N) turns the
        # in-block paths off, nothing else; one of N or more is no capacity
        q = B.moe_fwd_path(N, H, I, E, k, dtype, capacity_factor=1.0)
        if math.ceil(N * k / E) < N:
            assert q["inblock"] == 0 and q["router_in_up"] == 0
            assert {f: v for f, v in q.items() if f not in ("inblock", "router_in_up")} == \
                {f: v for f, v in p.items() if f not in ("inblock", "router_in_up")}
        else:
            assert q == p
    if dtype == B.DTYPE_BF16:
        assert seen["inblock"] > 0 and seen["router_in_up"] > 0, seen
