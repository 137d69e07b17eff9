"""Byte and FLOP accounting against the figures the FlashAttention pages print
(tests/golden/page_memory_numbers.txt, each line citing its page and diagram)
and against the workload table's closed forms."""
import os

import pytest

from exact_io_aware_60_amd import accounting as acc

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "page_memory_numbers.txt")
UNIT = {"GB": 1e9, "MB": 1e6, "scores": 1}


def golden_rows():
    rows = []
    for line in open(GOLDEN):
        if line.startswith("#") or not line.strip():
            continue
        name, inputs, value, unit, source = [f.strip() for f in line.split("|")]
        kv = dict(item.split("=") for item in inputs.split())
        rows.append((name, {k: int(v) for k, v in kv.items()}, value, unit, source))
    return rows


def compute(name, a):
    if name.startswith("naive_scores"):
        return acc.naive_score_bytes(a["N"], a.get("heads", 1), a["bytes_per_value"])
    if name == "flash_qkvo_one_head":
        return acc.flash_qkvo_bytes(a["N"], a["d"], 1, a["bytes_per_value"])
    if name == "flash_lse_one_head":
        assert a["bytes_per_value"] == acc.LSE_BYTES
        return acc.flash_lse_bytes(a["N"])
    if name == "flash_total_eight_heads":
        return acc.flash_total_bytes(a["N"], a["d"], a["heads"])
    if name == "score_count_2048":
        return acc.score_count(a["N"])
    raise KeyError(name)


@pytest.mark.parametrize("row", golden_rows(), ids=lambda r: r[0])
def test_page_figure(row):
    name, a, printed, unit, _ = row
    got = compute(name, a) / UNIT[unit]
    decimals = len(printed.split(".")[1]) if "." in printed else 0
    assert round(got, decimals) == float(printed), (name, got, printed)


def test_page_figure_8000_is_garbled():
    """The page prints N = 8,000 next to 1.07 GB; 8000 gives 1.02 GB, only 8192 gives 1.07."""
    assert round(acc.naive_score_bytes(8000, 8) / 1e9, 2) == 1.02
    assert round(acc.naive_score_bytes(8192, 8) / 1e9, 2) == 1.07


@pytest.mark.parametrize("B,Hq,N,d,causal,gflop", [
    (1, 1, 256, 64, False, 0.016777216),
    (4, 16, 2048, 64, True, 34.359738368),
    (1, 32, 8192, 128, True, 549.755813888),
    (2, 32, 16384, 128, True, 4398.046511104),
    (1, 8, 131072, 128, True, 35184.372088832),
])
def test_workload_flops(B, Hq, N, d, causal, gflop):
    assert acc.fwd_flop(B, Hq, N, d, causal) == pytest.approx(gflop * 1e9, rel=1e-12)
    assert acc.bwd_flop(B, Hq, N, d, causal) == pytest.approx(2.5 * gflop * 1e9, rel=1e-12)


def test_visible_pairs_brute_force():
    for N in (1, 2, 5, 17):
        assert acc.visible_pairs(N, True) == sum(1 for i in range(N) for j in range(N) if j <= i)
        assert acc.visible_pairs(N, False) == N * N


def test_long_context_footprint():
    """The 131072-token, 8-head, d = 128 workload keeps Q, K, V, O and LSE: about
    1.08 GB, against 275 GB for one bf16 score matrix per head."""
    assert acc.flash_total_bytes(131072, 128, 8) == 4 * 8 * 131072 * 128 * 2 + 8 * 131072 * 4
    assert round(acc.flash_total_bytes(131072, 128, 8) / 1e9, 2) == 1.08
    assert round(acc.naive_score_bytes(131072, 8) / 1e9) == 275


def test_tiny_input_rounding_deviation():
    """For information (the tiny workload draws its inputs in fp32 and both
    sides see them rounded to bf16): the fp64 oracle's output moves by about
    1.7e-3 in O and 1.5e-3 in LSE between the unrounded fp32 draws and the
    rounded inputs. That is the input rounding itself, not an error of either
    side. The bounds only check the order of magnitude: half a bf16 ulp
    (2^-9 relative) on each input."""
    import numpy as np
    import attn_inputs as ai
    import oracle
    w = ai.WORKLOADS["tiny"]
    inp = ai.make_inputs(w)
    f = ai.bf16_bits_to_f64
    o_r, l_r = oracle.fwd(f(inp["q"]), f(inp["k"]), f(inp["v"]), w.causal, w.scale)
    o_u, l_u = oracle.fwd(*(inp[t].astype(np.float64) for t in ("q32", "k32", "v32")), w.causal, w.scale)
    dev_o, dev_l = float(np.abs(o_r - o_u).max()), float(np.abs(l_r - l_u).max())
    print(f"tiny: oracle deviation from bf16 input rounding: O {dev_o:.2e}, LSE {dev_l:.2e}")
    assert 1e-4 < dev_o < 1e-2 and 1e-4 < dev_l < 1e-2
