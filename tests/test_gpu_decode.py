"""GPU decode (a few query rows over a long key/value cache) against the fp64 oracle.

The oracle runs the textbook definition with each query row placed at its
position among the keys: row i of Nq is token Nk - Nq + i under the causal mask.
Tolerances are the forward pass's: max abs error on O <= 1e-2 beyond the bf16
output rounding, and <= 1e-3 on the fp32 LSE. Every output element is compared.

The cases cover the kernel's layouts: one or two 32-row blocks per K/V head
(two waves per block, one per half tile), three and four blocks (one wave
each), more than 128 rows (several row blocks), a single key range (output
written directly) and many ranges (partial results merged by logsumexp), ragged
and tiny caches, both head dimensions and both masks, and per-sequence cache
lengths (seqlens_k), including entries with no key at all and rows that see
none (their O is 0 and LSE -inf, as in the oracle).
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


def run_decode(fa, inp, causal, scale, seqlens=None):
    import torch
    q, k, v = to_dev(inp["q"]), to_dev(inp["k"]), to_dev(inp["v"])
    sl = None if seqlens is None else torch.as_tensor(np.asarray(seqlens, np.int32)).cuda()
    o, lse = fa.decode(q, k, v, causal=causal, scale=scale, seqlens_k=sl)
    torch.cuda.synchronize()
    return from_dev_bf16(o), from_dev_f32(lse)


def oracle_decode_ragged(inp, causal, scale, seqlens):
    """Per batch entry b, the oracle over the first L_b = clamp(seqlens[b], 0, Nk)
    cache rows; an entry with no key gives O = 0 and LSE = -inf on every row."""
    B, Hq, Nq, d = inp["q"].shape
    Nk = inp["k"].shape[2]
    o = np.zeros((B, Hq, Nq, d))
    lse = np.full((B, Hq, Nq), -np.inf)
    for b in range(B):
        L = int(min(max(int(seqlens[b]), 0), Nk))
        if L == 0:
            continue
        pos = L - Nq + np.arange(Nq, dtype=np.int64) if causal else None
        o[b:b + 1], lse[b:b + 1] = oracle.fwd(f64(inp["q"][b:b + 1]), f64(inp["k"][b:b + 1, :, :L]),
                                              f64(inp["v"][b:b + 1, :, :L]), causal, scale, qpos=pos)
    return o, lse


def check_ragged(fa, inp, causal, scale, seqlens, tag):
    B, Hq, Nq, d = inp["q"].shape
    _, Hkv, Nk, _ = inp["k"].shape
    say(f"decode {tag}: B={B} Hq={Hq} Hkv={Hkv} Nq={Nq} Nk={Nk} d={d} causal={causal} seqlens={list(seqlens)[:8]}")
    o, lse = run_decode(fa, inp, causal, scale, seqlens)
    ro, rl = oracle_decode_ragged(inp, causal, scale, seqlens)
    empty = np.isneginf(rl)
    assert np.array_equal(np.isneginf(lse), empty), f"{tag}: rows without keys differ"
    assert np.all(o[empty] == 0.0), f"{tag}: rows without keys must give O = 0"
    eo = excess_err(o, ro)
    el = max_err(lse[~empty], rl[~empty]) if (~empty).any() else 0.0
    assert eo <= TOL_O and el <= TOL_LSE, f"{tag}: O err {eo:.2e}, LSE err {el:.2e}"


def oracle_decode(inp, causal, scale):
    Nq, Nk = inp["q"].shape[2], inp["k"].shape[2]
    pos = Nk - Nq + np.arange(Nq, dtype=np.int64) if causal else None
    return oracle.fwd(f64(inp["q"]), f64(inp["k"]), f64(inp["v"]), causal, scale, qpos=pos)


def check(fa, inp, causal, scale, tag):
    B, Hq, Nq, d = inp["q"].shape
    _, Hkv, Nk, _ = inp["k"].shape
    say(f"decode {tag}: B={B} Hq={Hq} Hkv={Hkv} Nq={Nq} Nk={Nk} d={d} causal={causal}")
    o, lse = run_decode(fa, inp, causal, scale)
    ro, rl = oracle_decode(inp, causal, scale)
    eo, el = excess_err(o, ro), max_err(lse, rl)
    assert eo <= TOL_O and el <= TOL_LSE, f"{tag}: O err {eo:.2e}, LSE err {el:.2e}"


# (B, Hq, Hkv, Nq, Nk): rows per K/V head M = (Hq / Hkv) * Nq
SHAPES = [
    (1, 1, 1, 1, 1),          # a single key
    (1, 4, 1, 1, 37),         # M = 4, one ragged tile
    (2, 8, 2, 1, 1000),       # M = 4, many ranges
    (1, 8, 2, 4, 4133),       # M = 16
    (1, 16, 2, 5, 2049),      # M = 40: two row blocks, two waves each
    (1, 8, 1, 8, 3001),       # M = 64
    (1, 6, 1, 16, 1500),      # M = 96: three blocks, one wave idle
    (1, 8, 1, 16, 2500),      # M = 128: four blocks
    (1, 10, 1, 16, 900),      # M = 160: two 128-row blocks
    (1, 3, 3, 40, 40),        # Nq = Nk: the square causal case
]


@pytest.mark.parametrize("d", [64, 128, 256])
@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("shape", SHAPES, ids=[f"B{s[0]}Hq{s[1]}Hkv{s[2]}Nq{s[3]}Nk{s[4]}" for s in SHAPES])
def test_shapes(fa, shape, causal, d):
    B, Hq, Hkv, Nq, Nk = shape
    inp = ai.make_decode_case(B, Hq, Hkv, Nq, Nk, d, seed=sum(shape) * 3 + d + int(causal))
    check(fa, inp, causal, 1.0 / math.sqrt(d), "shape")


def test_more_rows_than_keys_noncausal(fa):
    inp = ai.make_decode_case(1, 4, 2, 20, 7, 128, seed=90)
    check(fa, inp, False, 0.0883883, "Nq > Nk")


@pytest.mark.parametrize("d", [64, 128, 256])
def test_single_range_direct_output(fa, d):
    """512 (b, kv-head) groups fill the grid with one range each: no merge."""
    B, Hq, Hkv, Nq, Nk = 64, 16, 8, 1, 200
    assert fa.decode_workspace_size(B, Hq, Hkv, Nq, Nk, d, 1) == 0
    inp = ai.make_decode_case(B, Hq, Hkv, Nq, Nk, d, seed=91 + d)
    check(fa, inp, True, 1.0 / math.sqrt(d), "direct")


def test_large_logits(fa):
    """Scores spread by a factor of 4 and a larger scale: the running max rises
    inside ranges and differs widely between ranges."""
    inp = ai.make_decode_case(1, 8, 2, 3, 3000, 128, seed=92, dist_scale=2.0)
    check(fa, inp, True, 0.2, "large logits")


def test_late_maximum(fa):
    """The row max sits in the last keys of the cache: every earlier range is
    rescaled away in the merge."""
    inp = ai.make_decode_case(1, 4, 1, 2, 5000, 128, seed=93)
    k = f64(inp["k"])
    k[:, :, -3:] = np.sign(k[:, :, -3:]) * 4.0
    inp["k"] = ai.bf16_round_bits(k.astype(np.float32))
    inp["q"] = ai.bf16_round_bits((np.sign(f64(inp["q"])) * 1.0).astype(np.float32))
    check(fa, inp, True, 0.0883883, "late max")


def test_scale_zero_uniform(fa):
    """scale = 0: every visible key has the same weight, so O_i is the mean of
    v over keys 0 .. Nk - Nq + i and LSE_i = ln(Nk - Nq + i + 1)."""
    B, Hq, Hkv, Nq, Nk, d = 1, 4, 2, 5, 3333, 64
    inp = ai.make_decode_case(B, Hq, Hkv, Nq, Nk, d, seed=94)
    say("decode scale 0")
    o, lse = run_decode(fa, inp, True, 0.0)
    v = f64(inp["v"])
    cnt = Nk - Nq + np.arange(Nq) + 1
    ref = np.stack([v[:, :, :c].mean(axis=2) for c in cnt], axis=2)
    ref = np.repeat(ref, Hq // Hkv, axis=1)
    assert excess_err(o, ref) <= TOL_O
    assert max_err(lse, np.broadcast_to(np.log(cnt), lse.shape)) <= TOL_LSE


def test_matches_forward_when_square(fa):
    """Nq = Nk, causal: decode and the forward pass compute the same thing."""
    import torch
    inp = ai.make_decode_case(1, 4, 2, 300, 300, 128, seed=95)
    say("decode vs fwd, square")
    q, k, v = to_dev(inp["q"]), to_dev(inp["k"]), to_dev(inp["v"])
    od, ld = fa.decode(q, k, v, causal=True)
    of, lf = fa.fwd(q, k, v, causal=True)
    torch.cuda.synchronize()
    assert (od.float() - of.float()).abs().max().item() <= 2 * TOL_O
    assert (ld - lf).abs().max().item() <= TOL_LSE


def test_deterministic(fa):
    inp = ai.make_decode_case(2, 8, 2, 1, 7000, 128, seed=96)
    say("decode determinism")
    o1, l1 = run_decode(fa, inp, True, 0.0883883)
    o2, l2 = run_decode(fa, inp, True, 0.0883883)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


@pytest.mark.parametrize("d", [64, 128, 256])
@pytest.mark.parametrize("causal", [True, False])
def test_seqlens_ragged(fa, causal, d):
    """Entries with 0, 1, 2, 65 and all cache rows, one past the capacity
    (clamped) and a negative length (clamped to 0); with Nq = 3 and the causal
    mask the 1- and 2-key entries have rows that see no key."""
    inp = ai.make_decode_case(7, 4, 2, 3, 700, d, seed=97 + d + int(causal))
    check_ragged(fa, inp, causal, 1.0 / math.sqrt(d), [0, 1, 2, 65, 700, 5000, -3], "seqlens ragged")


def test_seqlens_many_ranges(fa):
    """Few groups, so the keys split into many ranges; the short entry leaves
    most of its ranges empty, which the merge must weigh 0."""
    inp = ai.make_decode_case(2, 8, 1, 2, 9000, 128, seed=98)
    check_ragged(fa, inp, True, 0.0883883, [150, 8999], "seqlens many ranges")


@pytest.mark.parametrize("d", [64, 128, 256])
def test_seqlens_direct(fa, d):
    """512 groups, one range each (no merge), random lengths including 0."""
    B, Hq, Hkv, Nq, Nk = 64, 16, 8, 1, 300
    assert fa.decode_workspace_size(B, Hq, Hkv, Nq, Nk, d, 1) == 0
    inp = ai.make_decode_case(B, Hq, Hkv, Nq, Nk, d, seed=99 + d)
    lens = np.random.default_rng(99 + d).integers(0, Nk, size=B, endpoint=True)
    lens[:3] = (0, 1, Nk)
    check_ragged(fa, inp, True, 1.0 / math.sqrt(d), lens, "seqlens direct")


def test_seqlens_full_is_default(fa):
    """seqlens_k equal to the capacity gives bit-identical results to no seqlens_k."""
    inp = ai.make_decode_case(3, 8, 2, 2, 3000, 128, seed=100)
    say("decode seqlens = Nk vs none")
    o1, l1 = run_decode(fa, inp, True, 0.0883883)
    o2, l2 = run_decode(fa, inp, True, 0.0883883, [3000, 3000, 3000])
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


@pytest.mark.parametrize("name", sorted(ai.DECODE_WORKLOADS))
def test_workload(fa, name):
    """The measured decode workloads at full size, every row against the oracle."""
    w = ai.DECODE_WORKLOADS[name]
    inp = ai.make_decode_inputs(w)
    lens = ai.decode_seqlens(w)
    if lens is None:
        check(fa, inp, w.causal, w.scale, name)
    else:
        check_ragged(fa, inp, w.causal, w.scale, lens, name)


def check_window(fa, inp, W, scale, tag, seqlens=None):
    import torch
    B, Hq, Nq, d = inp["q"].shape
    Nk = inp["k"].shape[2]
    say(f"decode window {tag}: B={B} Hq={Hq} Nq={Nq} Nk={Nk} d={d} W={W} seqlens={seqlens}")
    q, k, v = to_dev(inp["q"]), to_dev(inp["k"]), to_dev(inp["v"])
    sl = None if seqlens is None else torch.as_tensor(np.asarray(seqlens, np.int32)).cuda()
    o, lse = fa.decode(q, k, v, causal=True, scale=scale, seqlens_k=sl, window=W)
    torch.cuda.synchronize()
    o, lse = from_dev_bf16(o), from_dev_f32(lse)
    lens = [Nk] * B if seqlens is None else [int(min(max(x, 0), Nk)) for x in seqlens]
    for b, L in enumerate(lens):
        if L == 0:
            assert np.all(o[b] == 0) and np.all(np.isneginf(lse[b]))
            continue
        pos = L - Nq + np.arange(Nq, dtype=np.int64)
        ro, rl = oracle.fwd(f64(inp["q"][b:b + 1]), f64(inp["k"][b:b + 1, :, :L]), f64(inp["v"][b:b + 1, :, :L]),
                            True, scale, qpos=pos, window=W)
        empty = np.isneginf(rl)
        assert np.array_equal(np.isneginf(lse[b:b + 1]), empty)
        eo = excess_err(o[b:b + 1], ro)
        el = max_err(lse[b:b + 1][~empty], rl[~empty]) if (~empty).any() else 0.0
        assert eo <= TOL_O and el <= TOL_LSE, f"{tag} b={b}: O err {eo:.2e}, LSE err {el:.2e}"


@pytest.mark.parametrize("W", [1, 63, 64, 65, 100, 1000, 4999, 6000])
def test_window(fa, W):
    """Sliding window over a 5000-key cache: the window's first key falls in
    the middle of a tile, on a tile edge, or before the cache (W >= Nk)."""
    inp = ai.make_decode_case(2, 8, 2, 1, 5000, 128, seed=110 + W)
    check_window(fa, inp, W, 0.0883883, "W")


def test_window_short_queries_ragged(fa):
    """Nq = 4 rows with a 37-key window over ragged caches (lengths 0, 3, 500,
    3000), d = 64: rows whose window starts before the cache, inside it, and
    entries with no key."""
    inp = ai.make_decode_case(4, 8, 2, 4, 3000, 64, seed=120)
    check_window(fa, inp, 37, 0.125, "ragged", seqlens=[0, 3, 500, 3000])


def test_window_many_ranges(fa):
    """Few groups and a 4096-key window over a 60000-key cache: the ranges cover
    only the window's tiles."""
    inp = ai.make_decode_case(1, 4, 1, 2, 60000, 128, seed=121)
    assert fa.decode_workspace_size(1, 4, 1, 2, 60000, 128, 1, 4096) < fa.decode_workspace_size(1, 4, 1, 2, 60000,
                                                                                                 128, 1)
    check_window(fa, inp, 4096, 0.0883883, "many ranges")


# ------------------------------------------------------------------ head dimensions below 64 / 128 / 256
@pytest.mark.parametrize("d", [8, 32, 96, 200])
@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("shape", [(2, 8, 2, 1, 1000), (1, 16, 2, 5, 2049), (1, 8, 1, 16, 2500)],
                         ids=["M4", "M40", "M128"])
def test_padded_headdim(fa, shape, causal, d):
    """Rows of d values on the 64-, 128- or 256-wide instance (split ranges and
    the merge), every element against the oracle."""
    B, Hq, Hkv, Nq, Nk = shape
    inp = ai.make_decode_case(B, Hq, Hkv, Nq, Nk, d, seed=sum(shape) * 5 + d + int(causal))
    check(fa, inp, causal, 1.0 / math.sqrt(d), f"padded d={d}")


@pytest.mark.parametrize("d", [32, 96])
def test_padded_headdim_direct_and_seqlens(fa, d):
    """One range per group (the range kernel writes O itself) and ragged lengths."""
    B, Hq, Hkv, Nq, Nk = 64, 16, 8, 1, 200
    assert fa.decode_workspace_size(B, Hq, Hkv, Nq, Nk, d, 1) == 0
    inp = ai.make_decode_case(B, Hq, Hkv, Nq, Nk, d, seed=7400 + d)
    check(fa, inp, True, 1.0 / math.sqrt(d), f"padded direct d={d}")
    inp = ai.make_decode_case(7, 4, 2, 3, 700, d, seed=7500 + d)
    check_ragged(fa, inp, True, 1.0 / math.sqrt(d), [0, 1, 2, 65, 700, 5000, -3], f"padded seqlens d={d}")
