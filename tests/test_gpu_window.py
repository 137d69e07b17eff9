"""GPU forward with a sliding-window (local) causal mask against the fp64 oracle.

Row i sees keys i - W < j <= i. The oracle applies the same band in its
definition (pinned against torch's SDPA with the band written out). Tolerances
are the forward pass's. The cases put the window's left edge at every kind of
place relative to the kernel's 32-key chunks, 64-key tiles and 256-row q-tiles
(W = 1, 2, 31, 32, 33, 64, 255, 256, 257, ...), with ragged sequence lengths,
both head dimensions, GQA and large logits; the full-size case compares sampled
rows.
"""
import math

import numpy as np
import pytest

import attn_inputs as ai
import oracle
from tests.gpu_util import TOL_LSE, TOL_O, excess_err, f64, from_dev_bf16, from_dev_f32, max_err, say, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def fa():
    import torch
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a GPU")
    import exact_io_aware_60_amd as fa
    fa.lib()
    return fa


def run(fa, inp, W, scale):
    import torch
    q, k, v = to_dev(inp["q"]), to_dev(inp["k"]), to_dev(inp["v"])
    o, lse = fa.fwd_window(q, k, v, W, scale=scale)
    torch.cuda.synchronize()
    return from_dev_bf16(o), from_dev_f32(lse)


def check(fa, inp, W, scale, tag):
    B, Hq, N, d = inp["q"].shape
    say(f"fwd window {tag}: B={B} Hq={Hq} Hkv={inp['k'].shape[1]} N={N} d={d} W={W}")
    o, lse = run(fa, inp, W, scale)
    ro, rl = oracle.fwd(f64(inp["q"]), f64(inp["k"]), f64(inp["v"]), True, scale, window=W)
    eo, el = excess_err(o, ro), max_err(lse, rl)
    assert eo <= TOL_O and el <= TOL_LSE, f"{tag}: O err {eo:.2e}, LSE err {el:.2e}"


CASES = [(300, W) for W in (1, 2, 31, 32, 33, 100, 300)] + \
        [(1000, W) for W in (64, 255, 256, 257, 999)] + [(2049, 128), (2049, 700)]


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("N,W", CASES, ids=[f"N{n}-W{w}" for n, w in CASES])
def test_windows(fa, N, W, d):
    inp = ai.make_case(1, 2, 2, N, d, seed=N + 3 * W + d, with_grad=False)
    check(fa, inp, W, 1.0 / math.sqrt(d), "window")


def test_gqa(fa):
    inp = ai.make_case(2, 8, 2, 777, 128, seed=31, with_grad=False)
    check(fa, inp, 200, 0.0883883, "gqa")


def test_large_logits(fa):
    """Spread scores: the reference max of a wave's first chunks must hold for
    every row, and later maxima rise past it."""
    inp = ai.make_case(1, 4, 4, 1500, 128, seed=32, with_grad=False, dist_scale=2.0)
    check(fa, inp, 333, 0.2, "large logits")


def test_window_covering_everything_is_causal(fa):
    import torch
    inp = ai.make_case(1, 4, 2, 600, 128, seed=33, with_grad=False)
    say("fwd window >= N vs causal")
    q, k, v = to_dev(inp["q"]), to_dev(inp["k"]), to_dev(inp["v"])
    ow, lw = fa.fwd_window(q, k, v, 600)
    oc, lc = fa.fwd(q, k, v, causal=True)
    torch.cuda.synchronize()
    assert (ow.float() - oc.float()).abs().max().item() <= 2 * TOL_O
    assert (lw - lc).abs().max().item() <= TOL_LSE


def test_full_size_sampled(fa):
    """gqa16k shapes (B=2, Hq=32, Hkv=8, N=16384, d=128) with a 4096-key window:
    256 seeded rows (with the first and last) on every head against the oracle."""
    import torch
    w = ai.WORKLOADS["gqa16k"]
    W = 4096
    inp = ai.make_inputs(w, with_grad=False)
    rows = ai.sample_rows(w.N, 256, w.cfg_id)
    say("fwd window gqa16k W=4096 (full size on GPU, sampled rows)")
    q, k, v = to_dev(inp["q"]), to_dev(inp["k"]), to_dev(inp["v"])
    o, lse = fa.fwd_window(q, k, v, W, scale=w.scale)
    torch.cuda.synchronize()
    rt = torch.as_tensor(rows, device=o.device)
    o_s, l_s = from_dev_bf16(o.index_select(2, rt)), from_dev_f32(lse.index_select(2, rt))
    del q, k, v, o, lse
    ro, rl = oracle.fwd(f64(inp["q"][:, :, rows]), f64(inp["k"]), f64(inp["v"]), True, w.scale, qpos=rows, window=W)
    eo, el = excess_err(o_s, ro), max_err(l_s, rl)
    assert eo <= TOL_O and el <= TOL_LSE, f"O err {eo:.2e}, LSE err {el:.2e}"
