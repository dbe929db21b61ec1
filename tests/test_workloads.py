"""The seeded input generator: rounding, determinism, margins, skew."""
import numpy as np
import pytest

import workloads
from workloads import bf16_bits_from_f64, f64_from_bf16_bits, get, make_inputs, to_f64
from oracle.cases import enforce_margin, small_margin_rows, make_case
from oracle import router_probs, topk_canonical, expert_lists


def test_bf16_rne_known_patterns():
    one = 1.0
    cases = [
        (1.0, 0x3F80),
        (-1.0, 0xBF80),
        (0.0, 0x0000),
        (one + 2**-7, 0x3F81),             # representable
        (one + 2**-8, 0x3F80),             # halfway, ties to even (down)
        (one + 3 * 2**-8, 0x3F82),         # halfway, ties to even (up)
        (one + 2**-8 + 2**-30, 0x3F81),    # just above halfway: double rounding via fp32 would give 0x3F80
        (-(one + 2**-8 + 2**-30), 0xBF81),
        (3.0, 0x4040),
        (2.0**-10, 0x3A80),
    ]
    got = bf16_bits_from_f64(np.array([c[0] for c in cases]))
    assert got.tolist() == [c[1] for c in cases]


def test_bf16_widening_exact():
    assert f64_from_bf16_bits(np.array([0x3F81], np.uint16))[0] == 1 + 2**-7
    b = np.arange(0, 0x7F80, 7, dtype=np.uint16)
    assert np.array_equal(bf16_bits_from_f64(f64_from_bf16_bits(b)), b)


def test_generator_deterministic_and_seeded():
    w = get("moe_top1")
    a = make_inputs(w, N=64)
    b = make_inputs(w, N=64)
    for n in ("x", "Wr", "Wg", "Wu", "Wd"):
        assert np.array_equal(a[n], b[n])
    c = make_inputs(w, seed=1, N=64)
    assert not np.array_equal(a["x"], c["x"])
    # x rows are a prefix-stable stream: fewer tokens give the first rows
    full = make_inputs(w, N=128)
    assert np.array_equal(full["x"][:64], a["x"])


def test_generator_distributions():
    w = get("moe_top1")
    inp = make_inputs(w)
    x = to_f64(inp["x"], "bf16")
    assert abs(x.mean()) < 0.01 and abs(x.std() - 1) < 0.01
    for n, fan in (("Wg", w.H), ("Wu", w.H), ("Wd", w.I), ("Wr", w.H)):
        W = inp[n].astype(np.float64) if n == "Wr" else to_f64(inp[n], "bf16")
        assert np.abs(W).max() <= 1 / np.sqrt(fan) * (1 + 2**-8)
        assert np.abs(W).max() > 0.99 / np.sqrt(fan)
    assert inp["Wr"].dtype == np.float32 and inp["x"].dtype == np.uint16
    assert inp["Wg"].shape == (4, 2432, 768) and inp["Wd"].shape == (4, 768, 2432)


def test_dense_fp32_shapes():
    w = get("dense_fp32")
    inp = make_inputs(w)
    assert inp["x"].dtype == np.float32 and inp["x"].shape == (100, 768)
    assert inp["Wg"].shape == (2432, 768) and inp["Wd"].shape == (768, 2432)


@pytest.mark.parametrize("name", ["moe_top1", "moe_decode"])
def test_margin_enforced(name):
    w = get(name)
    inp = make_case(w)
    x = to_f64(inp["x"], inp["dtype"])
    assert small_margin_rows(x, inp["Wr"].astype(np.float64), w.k).size == 0
    assert inp["redrawn_rows"] < 0.05 * w.N + 2


def test_skewed_loads_about_10x():
    """The skewed top-2 workload: per-expert loads differ by about 10x."""
    w = get("moe_skew")
    inp = make_inputs(w)
    p = router_probs(to_f64(inp["x"], "bf16"), inp["Wr"].astype(np.float64))
    counts, _, _ = expert_lists(topk_canonical(p, w.k), w.E)
    ratio = counts.max() / counts.min()
    assert 8 <= ratio <= 12, counts


def test_skewed_literal_empties_or_starves_experts():
    w = get("moe_skew_literal")
    inp = make_inputs(w, N=4096)
    p = router_probs(to_f64(inp["x"], "bf16"), inp["Wr"].astype(np.float64))
    counts, _, _ = expert_lists(topk_canonical(p, w.k), w.E)
    assert counts.min() * 100 < counts.max()
