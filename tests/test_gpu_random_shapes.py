"""Seeded random shapes against the fp64 oracle: head counts and GQA ratios that
are not powers of two, ragged sequence lengths, both masks and every head
dimension, for the forward with backward, the forward alone at d = 256, and
decode. The shapes are drawn once from a fixed seed, so the cases are the
same on every run; each is small enough for the oracle to finish in well under
a second, and every output element is compared.
"""
import math

import numpy as np
import pytest

import attn_inputs as ai
import oracle
from tests.gpu_util import TOL_GRAD, TOL_LSE, TOL_O, excess_err, f64, from_dev_bf16, from_dev_f32, max_err, say, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def fa():
    import torch
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a GPU")
    import exact_io_aware_60_amd as fa
    fa.lib()
    return fa


def _draw(n, seed, decode=False):
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(n):
        hkv = int(rng.integers(1, 4))
        g = int(rng.choice([1, 2, 3, 5]))
        B = int(rng.integers(1, 3))
        causal = bool(rng.integers(0, 2))
        if decode:
            nk = int(rng.integers(1, 2500))
            nq = int(rng.integers(1, 20))
            if causal:
                nq = min(nq, nk)
            out.append((B, hkv * g, hkv, nq, nk, causal))
        else:
            out.append((B, hkv * g, hkv, int(rng.integers(1, 900)), causal))
    return out


def _seed(case, extra):
    """A seed made of the case's own numbers, the same in every process."""
    acc = extra
    for x in case:
        acc = (acc * 1000003 + int(x)) % 2147483647
    return acc


FWD_BWD = _draw(10, 5150)
FWD_256 = _draw(6, 5151)
DECODE = _draw(10, 5152, decode=True)


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("case", FWD_BWD, ids=[f"B{c[0]}Hq{c[1]}Hkv{c[2]}N{c[3]}{'c' if c[4] else 'n'}" for c in FWD_BWD])
def test_fwd_bwd(fa, case, d):
    import torch
    B, Hq, Hkv, N, causal = case
    scale = 1.0 / math.sqrt(d)
    inp = ai.make_case(B, Hq, Hkv, N, d, seed=_seed(case, d), with_grad=True)
    say(f"random fwd+bwd B={B} Hq={Hq} Hkv={Hkv} N={N} d={d} causal={causal}")
    q, k, v, do = to_dev(inp["q"]), to_dev(inp["k"]), to_dev(inp["v"]), to_dev(inp["do"])
    o, lse = fa.fwd(q, k, v, causal=causal, scale=scale)
    dq, dk, dv = fa.bwd(q, k, v, o, lse, do, causal=causal, scale=scale)
    torch.cuda.synchronize()
    ref = oracle.bwd(f64(inp["q"]), f64(inp["k"]), f64(inp["v"]), f64(inp["do"]), causal, scale)
    eo, el = excess_err(from_dev_bf16(o), ref["o"]), max_err(from_dev_f32(lse), ref["lse"])
    assert eo <= TOL_O and el <= TOL_LSE, (eo, el)
    for name, t in (("dq", dq), ("dk", dk), ("dv", dv)):
        e = excess_err(from_dev_bf16(t), ref[name])
        assert e <= TOL_GRAD, (name, e)


@pytest.mark.parametrize("case", FWD_256, ids=[f"B{c[0]}Hq{c[1]}Hkv{c[2]}N{c[3]}{'c' if c[4] else 'n'}" for c in FWD_256])
def test_fwd_d256(fa, case):
    import torch
    B, Hq, Hkv, N, causal = case
    inp = ai.make_case(B, Hq, Hkv, N, 256, seed=_seed(case, 256), with_grad=False)
    say(f"random fwd B={B} Hq={Hq} Hkv={Hkv} N={N} d=256 causal={causal}")
    q, k, v = to_dev(inp["q"]), to_dev(inp["k"]), to_dev(inp["v"])
    o, lse = fa.fwd(q, k, v, causal=causal, scale=0.0625)
    torch.cuda.synchronize()
    ro, rl = oracle.fwd(f64(inp["q"]), f64(inp["k"]), f64(inp["v"]), causal, 0.0625)
    eo, el = excess_err(from_dev_bf16(o), ro), max_err(from_dev_f32(lse), rl)
    assert eo <= TOL_O and el <= TOL_LSE, (eo, el)


@pytest.mark.parametrize("d", [64, 128, 256])
@pytest.mark.parametrize("case", DECODE, ids=[f"B{c[0]}Hq{c[1]}Hkv{c[2]}Nq{c[3]}Nk{c[4]}{'c' if c[5] else 'n'}"
                                              for c in DECODE])
def test_decode(fa, case, d):
    import torch
    B, Hq, Hkv, Nq, Nk, causal = case
    scale = 1.0 / math.sqrt(d)
    inp = ai.make_decode_case(B, Hq, Hkv, Nq, Nk, d, seed=_seed(case, 7 * d))
    say(f"random decode B={B} Hq={Hq} Hkv={Hkv} Nq={Nq} Nk={Nk} d={d} causal={causal}")
    q, k, v = to_dev(inp["q"]), to_dev(inp["k"]), to_dev(inp["v"])
    o, lse = fa.decode(q, k, v, causal=causal, scale=scale)
    torch.cuda.synchronize()
    pos = np.arange(Nk - Nq, Nk, dtype=np.int64) if causal else None
    ro, rl = oracle.fwd(f64(inp["q"]), f64(inp["k"]), f64(inp["v"]), causal, scale, qpos=pos)
    eo, el = excess_err(from_dev_bf16(o), ro), max_err(from_dev_f32(lse), rl)
    assert eo <= TOL_O and el <= TOL_LSE, (eo, el)
