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


@pytest.mark.parametrize("d", [64, 128, 256])
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


# ------------------------------------------------------------------ backward
TOL_GRAD = 2e-2


def check_bwd(fa, inp, W, scale, tag):
    import torch
    B, Hq, N, d = inp["q"].shape
    say(f"bwd window {tag}: B={B} Hq={Hq} Hkv={inp['k'].shape[1]} N={N} d={d} W={W}")
    q, k, v, do = to_dev(inp["q"]), to_dev(inp["k"]), to_dev(inp["v"]), to_dev(inp["do"])
    o, lse = fa.fwd_window(q, k, v, W, scale=scale)
    dq, dk, dv = fa.bwd_window(q, k, v, o, lse, do, W, scale=scale)
    torch.cuda.synchronize()
    ref = oracle.bwd(f64(inp["q"]), f64(inp["k"]), f64(inp["v"]), f64(inp["do"]), True, scale, window=W)
    errs = {n: excess_err(from_dev_bf16(g), ref[n]) for n, g in (("dq", dq), ("dk", dk), ("dv", dv))}
    assert all(e <= TOL_GRAD for e in errs.values()), f"{tag} W={W}: {errs}"


BWD_CASES = [(300, W) for W in (1, 31, 64, 100, 300)] + \
            [(1000, W) for W in (63, 64, 65, 127, 128, 129, 192, 256, 700)] + [(2049, 200), (2049, 1500)]


@pytest.mark.parametrize("N,W", BWD_CASES, ids=[f"N{n}-W{w}" for n, w in BWD_CASES])
def test_bwd_windows(fa, N, W):
    """Window edges against the backward's 64-row steps, 128-key workgroups and
    64-key dQ tiles: masked first tiles, a uniform middle and masked ends."""
    inp = ai.make_case(1, 4, 2, N, 128, seed=N + 5 * W)
    check_bwd(fa, inp, W, 0.0883883, "window")


@pytest.mark.parametrize("W", [33, 500])
def test_bwd_windows_d64(fa, W):
    inp = ai.make_case(2, 4, 4, 1100, 64, seed=40 + W)
    check_bwd(fa, inp, W, 0.125, "d64")


def test_bwd_large_logits(fa):
    inp = ai.make_case(1, 4, 2, 1500, 128, seed=41, dist_scale=2.0)
    check_bwd(fa, inp, 333, 0.2, "large logits")


def test_bwd_window_covering_everything_is_causal(fa):
    """W >= N: the same gradients as the plain causal backward (within rounding)."""
    import torch
    inp = ai.make_case(1, 4, 2, 700, 128, seed=42)
    say("bwd window >= N vs causal")
    q, k, v, do = to_dev(inp["q"]), to_dev(inp["k"]), to_dev(inp["v"]), to_dev(inp["do"])
    o, lse = fa.fwd(q, k, v, causal=True)
    g1 = fa.bwd_window(q, k, v, o, lse, do, 700)
    g2 = fa.bwd(q, k, v, o, lse, do, causal=True)
    torch.cuda.synchronize()
    for a, b_ in zip(g1, g2):
        assert (a.float() - b_.float()).abs().max().item() <= TOL_GRAD


def test_bwd_full_size_sampled(fa):
    """gqa16k shapes with a 4096-key window: full GPU forward and backward, then
    256 sampled dQ rows and dK/dV keys of one seeded (b, kv-head) group against
    the oracle."""
    import torch
    w = ai.WORKLOADS["gqa16k"]
    W = 4096
    inp = ai.make_inputs(w)
    say("bwd window gqa16k W=4096 (full size on GPU, one group)")
    q, k, v, do = to_dev(inp["q"]), to_dev(inp["k"]), to_dev(inp["v"]), to_dev(inp["do"])
    o, lse = fa.fwd_window(q, k, v, W, scale=w.scale)
    dq, dk, dv = fa.bwd_window(q, k, v, o, lse, do, W, scale=w.scale)
    torch.cuda.synchronize()
    rows = ai.sample_rows(w.N, 256, w.cfg_id)
    keys = ai.sample_rows(w.N, 256, w.cfg_id + 100)
    rt, kt = torch.as_tensor(rows, device=q.device), torch.as_tensor(keys, device=q.device)
    b, h, G = 1, 5, w.G
    hs = slice(h * G, (h + 1) * G)
    g = {"dq": from_dev_bf16(dq[b:b + 1, hs].index_select(2, rt)),
         "dk": from_dev_bf16(dk[b:b + 1, h:h + 1].index_select(2, kt)),
         "dv": from_dev_bf16(dv[b:b + 1, h:h + 1].index_select(2, kt))}
    del q, k, v, do, o, lse, dq, dk, dv
    ref = oracle.bwd_sampled(f64(inp["q"][b:b + 1, hs]), f64(inp["k"][b:b + 1, h:h + 1]),
                             f64(inp["v"][b:b + 1, h:h + 1]), f64(inp["do"][b:b + 1, hs]), True, w.scale, rows, keys,
                             window=W)
    errs = {n: excess_err(g[n], ref[n]) for n in g}
    assert all(e <= TOL_GRAD for e in errs.values()), errs


@pytest.mark.parametrize("d", [32, 96])
@pytest.mark.parametrize("N,W", [(300, 31), (1000, 129), (2049, 700)], ids=["N300-W31", "N1000-W129", "N2049-W700"])
def test_padded_headdim(fa, N, W, d):
    """Head dimensions below 64 / 128 with a window: forward and backward."""
    inp = ai.make_case(1, 4, 2, N, d, seed=7600 + N + W + d)
    check(fa, inp, W, 1.0 / math.sqrt(d), f"padded d={d}")
    check_bwd(fa, inp, W, 1.0 / math.sqrt(d), f"padded d={d}")


@pytest.mark.parametrize("N,W", [(300, 31), (1000, 129)], ids=["N300-W31", "N1000-W129"])
def test_wide_headdim_bwd(fa, N, W):
    """d = 256 with a window: the split gradient kernels with a bounded mask."""
    inp = ai.make_case(1, 4, 2, N, 256, seed=7900 + N + W)
    check_bwd(fa, inp, W, 0.0625, "wide d=256")


@pytest.mark.parametrize("W", [33, 1000])
def test_twelve_wave_workgroups(fa, W):
    """A grid large enough for the d = 64 forward's 12-wave (384-row)
    workgroups (the launch geometry confirms it), every row against the oracle."""
    g = fa.fwd_geometry(1, 64, 8, 4100, 64, True)
    assert g["threads"] == 768, g
    inp = ai.make_case(1, 64, 8, 4100, 64, seed=41 + W, with_grad=False)
    check(fa, inp, W, 0.125, f"12 waves W={W}")
