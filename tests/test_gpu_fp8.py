"""GPU parity of the FP8 path: the transposing E4M3 quantiser of V (bit-exact
against the oracle's quantiser), and the forward on E4M3 inputs against the
oracle's attention of the dequantised values code * scale.

Tolerance of the FP8 forward, derived from its arithmetic; neither the pages nor
the bf16 tolerances fix one for E4M3 inputs.

The E4M3 matrix instruction does not sum its products exactly. Measured on
gfx950 with exact operands: it adds its 64 products in groups of 8
consecutive k slots; inside a group every nonzero product is truncated toward
zero to a multiple of 2^(E - 13), E the group's largest exponent sum e_a + e_b
of nonzero codes (a code's exponent is its field minus 7, -6 for subnormals);
the group sums then go into the fp32 accumulator. In the score product the
slots of a group are 8 consecutive head columns, so the test computes the
scores exactly as the instruction does (mfma_scores) and takes P', O', LSE' of
those scores in fp64. LSE must match LSE' up to fp32 rounding of the scores,
the exp sum and the log. Against O' the remaining errors are bounded:

1. The rounding of P to E4M3. The kernel rounds a_j = P~_j r_j, where P~_j is
   the probability relative to its reference and r_j = s_v(j) / s_vmax <= 1 the
   key's V-scale ratio. Rounded to nearest, a normal E4M3 value (>= 2^-6) is
   within 2^-4 relative, a smaller one within min(a_j, 2^-10) (its spacing
   2^-9, halved; below 2^-10 it rounds to zero). O is
   normalised by the sum of the rounded values divided back by r_j, so with D_j
   that error bound over r_j, in units of P~, and L = sum_j P~_j:
       |dO| <= sum_j D_j |v_j - O| / (L - sum_j D_j).
2. The instruction's truncation in P.V and in the all-ones row sum: a product
   loses less than min(|product|, 2^(E - 13)) in its group of 8 keys (the
   kernel's key order in a 64-key tile fixes the groups), bounded with an
   upper bound on a_j.

The bound is widest when the reference is the row's exact max, since a stale
reference only makes P~ larger and the subnormal range emptier. So the test
takes P~_j = P'_j / max_k P'_k, which gives L = 1 / max_k P'_k. The bound holds
on every element of every row, plus half a bf16 ulp of O (its output
rounding), the fp32 rounding of the scores and 1e-4. The error against the
oracle's exact attention is reported beside it.
"""
import math

import numpy as np
import pytest

import attn_inputs as ai
import oracle
from tests.fp8_model import MFMA_GROUP, e4m3_exp, group_loss, mfma_scores, tile_groups
from tests.gpu_util import bf16_half_ulp, from_dev_bf16, say, to_dev

pytestmark = pytest.mark.gpu

E4M3_REL = 2.0 ** -4
E4M3_ABS = 2.0 ** -10
E4M3_MIN_NORMAL = 2.0 ** -6


@pytest.fixture(scope="module")
def fa():
    import torch
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a GPU")
    import exact_io_aware_60_amd as fa
    fa.lib()
    return fa


@pytest.fixture(scope="module")
def orc():
    return oracle.default()


def vt_key(p):
    """Key (within its group of 64) held at position p of a transposed row."""
    p = np.asarray(p)
    return ((p % 32) // 16) * 32 + ((p % 16) // 4) * 8 + (p // 32) * 4 + p % 4


# ------------------------------------------------------------------ quantiser, transposed
@pytest.mark.parametrize("BH,N,d,rows", [(1, 1, 64, 64), (3, 300, 128, 128), (2, 64, 64, 64), (2, 777, 128, 192),
                                         (4, 130, 24, 64), (1, 4100, 128, 256), (1, 1100, 128, 512),
                                         (2, 200, 256, 128)])
def test_quantize_vt_matches_oracle(fa, orc, BH, N, d, rows):
    """Every code and scale bit-exact with the oracle's quantiser, placed at the
    documented transposed position; positions past N hold 0. Runs up to 32768
    elements take the single-read path, (1, 1100, 128, 512) the two-sweep one."""
    import torch
    say(f"quantize_e4m3_vt BH={BH} N={N} d={d} rows={rows}")
    g = torch.Generator().manual_seed(31 * N + d + rows)
    x = (torch.randn((BH, N, d), generator=g) * torch.exp(torch.randn((BH, 1, 1), generator=g) * 2)).to(torch.bfloat16)
    if N > 100:
        x[0, 64:128] = 0.0                            # a zero group
    codes_t, scales = fa.quantize_e4m3_vt(x.cuda(), rows)
    torch.cuda.synchronize()
    want_c, want_s = orc.quantize_e4m3(x.float().numpy()[None], rows)
    Np = -(-N // 64) * 64
    keys = (np.arange(Np) // 64) * 64 + vt_key(np.arange(Np) % 64)
    inside = keys < N
    want_t = np.zeros((BH, d, Np), dtype=np.uint8)
    want_t[:, :, inside] = np.transpose(want_c[0], (0, 2, 1))[:, :, keys[inside]]
    got = codes_t.cpu().numpy()
    assert got.shape == (BH, d, Np)
    bad = np.flatnonzero(got.reshape(-1) != want_t.reshape(-1))
    assert bad.size == 0, f"{bad.size} codes differ"
    assert np.array_equal(scales.cpu().numpy().view(np.uint32), want_s[0].view(np.uint32))


def test_vt_positions_are_a_permutation():
    assert sorted(vt_key(np.arange(64)).tolist()) == list(range(64))


# ------------------------------------------------------------------ forward on E4M3 inputs
def fp8_case(orc, B, Hq, Hkv, N, d, rows, seed, dist_scale=1.0, v_spread=0.0):
    """Seeded bf16 draws (V runs optionally spread in magnitude), quantised on
    the host by the oracle; returns host codes, scales and dequantised values."""
    inp = ai.make_case(B, Hq, Hkv, N, d, seed=seed, with_grad=False, dist_scale=dist_scale)
    q, k, v = (ai.bf16_bits_to_f32(inp[t]) for t in ("q", "k", "v"))
    if v_spread:
        nr = -(-N // rows)
        f = np.exp2(ai.rng_for(9000 + seed, 0).uniform(-v_spread, 0, size=(B, Hkv, nr))).astype(np.float32)
        v = v * np.repeat(f, rows, axis=2)[:, :, :N, None]
    q8, qs = orc.quantize_e4m3(q, rows)
    k8, ks = orc.quantize_e4m3(k, rows)
    v8, vs = orc.quantize_e4m3(v, rows)
    deq = dict(q=orc.dequantize_e4m3(q8, qs, rows), k=orc.dequantize_e4m3(k8, ks, rows),
               v=orc.dequantize_e4m3(v8, vs, rows))
    return dict(q8=q8, qs=qs, k8=k8, ks=ks, v8=v8, vs=vs, v=v, deq=deq)


def vt_layout(v8):
    """Host transposition of row-major V codes into the forward's layout."""
    B, H, N, d = v8.shape
    Np = -(-N // 64) * 64
    keys = (np.arange(Np) // 64) * 64 + vt_key(np.arange(Np) % 64)
    out = np.zeros((B, H, d, Np), dtype=np.uint8)
    inside = keys < N
    out[:, :, :, inside] = np.transpose(v8, (0, 1, 3, 2))[:, :, :, keys[inside]]
    return out


def run_fp8(fa, c, rows, causal, scale, device_quant=None):
    import torch
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    v8t, vs = (vt_layout(c["v8"]), c["vs"]) if device_quant is None else device_quant
    o, lse = fa.fwd_e4m3(dev(c["q8"]), dev(c["qs"]), dev(c["k8"]), dev(c["ks"]),
                         v8t if isinstance(v8t, torch.Tensor) else dev(v8t),
                         vs if isinstance(vs, torch.Tensor) else dev(vs), rows, causal=causal, scale=scale)
    torch.cuda.synchronize()
    return from_dev_bf16(o), lse.double().cpu().numpy()


def head_reference(orc, q8, qs, k8, ks, v, rows_idx, rows, causal, scale):
    """P', O', LSE' and per-row max |scaled score| of query rows `rows_idx`
    of one head (codes [N, d], run scales, dequantised V [N, d]), all keys,
    with the scores as the instruction computes them."""
    N = k8.shape[0]
    sq = np.repeat(qs.astype(np.float64), rows)[:N][rows_idx]
    sk = np.repeat(ks.astype(np.float64), rows)[:N]
    x = scale * sq[:, None] * sk[None, :] * mfma_scores(orc, q8[rows_idx], k8)
    if causal:
        x = np.where(np.arange(N)[None, :] <= rows_idx[:, None], x, -np.inf)
    xabs = np.max(np.where(np.isfinite(x), np.abs(x), 0.0), axis=1)
    mx = x.max(axis=1, keepdims=True)
    e = np.exp(x - mx)
    se = e.sum(axis=1, keepdims=True)
    P = e / se
    return P, P @ v, mx[:, 0] + np.log(se[:, 0]), xabs


def emulated_reference(orc, c, rows, causal, scale):
    """head_reference for every row of every head, stacked [B, Hq, ...]."""
    d = c["deq"]
    B, Hq, N, _ = d["q"].shape
    G = Hq // d["v"].shape[1]
    P = np.empty((B, Hq, N, N))
    O = np.empty((B, Hq, N, d["v"].shape[3]))
    lse = np.empty((B, Hq, N))
    xabs = np.empty((B, Hq, N))
    rows_idx = np.arange(N)
    for b in range(B):
        for h in range(Hq):
            hk = h // G
            P[b, h], O[b, h], lse[b, h], xabs[b, h] = head_reference(
                orc, c["q8"][b, h], c["qs"][b, h], c["k8"][b, hk], c["ks"][b, hk], d["v"][b, hk], rows_idx, rows,
                causal, scale)
    return P, O, lse, xabs


def head_bound(orc, v8, vs_runs, v, rows, P, O, xabs, chunk=8):
    """Per element bound on |O_gpu - O'| (module docstring) for the rows of
    one head whose P' [R, N], O' [R, d] and max |x| are given; V as codes
    [N, d], run scales and dequantised values."""
    R, N = P.shape
    dd = O.shape[1]
    Np = -(-N // 64) * 64
    vs = np.repeat(vs_runs.astype(np.float64), rows)
    vs = np.concatenate([vs, np.full(Np, vs[-1])])[:Np]         # s_v per key, past N too
    r = vs / vs.max()                                             # V-scale ratio per key
    order = (np.arange(Np // 64)[:, None, None] * 64 + tile_groups()[None]).reshape(-1)   # keys by group
    r_g = r[order].reshape(-1, 8, MFMA_GROUP)[:, :, :1]          # one ratio per tile
    v8p = np.zeros((Np, dd), dtype=np.uint8)
    v8p[:N] = v8
    vv = np.abs(orc.e4m3_decode(v8p)[order].reshape(-1, 8, MFMA_GROUP, dd))          # [tiles, 8, 8, d]
    ev = np.where(vv != 0, e4m3_exp(v8p[order]).reshape(vv.shape), -1000)
    bound = np.empty_like(O)
    for i0 in range(0, R, chunk):
        p = P[i0:i0 + chunk]
        o = O[i0:i0 + chunk]
        n = p.shape[0]
        live = p > 0                                              # masked keys: exact zeros
        pt = p / p.max(axis=1, keepdims=True)                     # P~ under the exact max
        a = pt * r[None, :N]
        D = np.where(a >= E4M3_MIN_NORMAL, E4M3_REL * a, np.minimum(a, E4M3_ABS)) / r[None, :N]
        D = np.where(live, D, 0.0)
        den = pt.sum(axis=1) - D.sum(axis=1)
        dev = np.abs(v[None, :, :] - o[:, None, :])               # [n, N, d]
        rounding = np.einsum("ij,ijc->ic", D, dev) / den[:, None]
        # fp32 scores: relative error of the weights below 2^-20 |x| + 1e-6
        slack = (2.0 ** -19 * xabs[i0:i0 + chunk] + 2e-6)[:, None] * np.einsum("ij,ijc->ic", p, dev)
        # instruction truncation in P.V and in the ones-vector sum, keys in group order
        a_up = np.zeros((n, Np))
        a_up[:, :N] = np.where(live, a * (1 + E4M3_REL), 0.0)
        a_up = a_up[:, order].reshape(n, -1, 8, MFMA_GROUP)       # [n, tiles, 8, 8]
        ea = np.where(a_up > 0, np.maximum(np.floor(np.log2(np.where(a_up > 0, a_up, 1.0))), -6), -1000)
        ones = group_loss(a_up / r_g[None], ea).sum(axis=-1) / den   # relative, per row
        pv = np.empty((n, dd))
        for k0 in range(n):
            x = a_up[k0][..., None] * vv                          # [tiles, 8, 8, d]
            ex = np.where((ea[k0][..., None] > -1000) & (ev > -1000), ea[k0][..., None] + ev, -1000)
            pv[k0] = group_loss(np.moveaxis(x, -1, 0), np.moveaxis(ex, -1, 0)).sum(axis=-1)
        pv *= vs.max() / den[:, None]
        bound[i0:i0 + chunk] = rounding + slack + pv + 1.1 * np.abs(o) * ones[:, None]
    return bound + bf16_half_ulp(O) + 1e-4


def fp8_bound(orc, c, rows, P, O, xabs):
    """Per element bound on |O_gpu - O'| for every row of every head."""
    B, Hq = P.shape[:2]
    G = Hq // c["v8"].shape[1]
    bound = np.empty_like(O)
    for b in range(B):
        for h in range(Hq):
            hk = h // G
            bound[b, h] = head_bound(orc, c["v8"][b, hk], c["vs"][b, hk], c["deq"]["v"][b, hk], rows, P[b, h],
                                     O[b, h], xabs[b, h])
    return bound


def check_fp8(fa, orc, c, rows, causal, scale, tag, device_quant=None):
    say(f"fwd_e4m3 {tag}")
    o, lse = run_fp8(fa, c, rows, causal, scale, device_quant)
    ro, rl = orc.fwd_e4m3(c["q8"], c["k8"], c["v8"], c["qs"], c["ks"], c["vs"], rows, causal, scale)
    P, O, L, xabs = emulated_reference(orc, c, rows, causal, scale)
    bound = fp8_bound(orc, c, rows, P, O, xabs)
    N = O.shape[2]
    lbound = 1e-5 + 2.0 ** -19 * xabs + N * 2.0 ** -23
    assert np.all(np.isfinite(o)), "non-finite O"
    err = np.abs(o - O)
    ratio = float(np.max(err / bound))
    lerr = np.abs(lse - L)
    lratio = float(np.max(lerr / lbound))
    say(f"{tag}: max|O - O'| {err.max():.3e}, largest error / bound {ratio:.3f}; max|LSE - LSE'| {lerr.max():.2e} "
        f"({lratio:.3f} of its bound); against exact attention max|O - ref| {np.abs(o - ro).max():.3e}, "
        f"max|LSE - ref| {np.abs(lse - rl).max():.2e}")
    assert ratio <= 1.0, f"{tag}: O error beyond the E4M3 bound ({ratio:.3f} of it)"
    assert lratio <= 1.0, f"{tag}: LSE off the instruction's scores ({lratio:.3f} of the bound)"
    return ratio


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("N", [1, 17, 64, 65, 200, 300])
def test_ragged(fa, orc, d, causal, N):
    c = fp8_case(orc, 1, 2, 2, N, d, 64, seed=8100 + N + d + int(causal))
    check_fp8(fa, orc, c, 64, causal, 1.0 / math.sqrt(d), f"ragged N={N} d={d} causal={causal}")


@pytest.mark.parametrize("causal", [False, True])
def test_gqa_runs_and_spread_v_scales(fa, orc, causal):
    """GQA, 128-row runs, V runs spread over 2^-6 .. 1 in magnitude (so the V
    ratio folded into P matters), N with a ragged last run."""
    c = fp8_case(orc, 2, 8, 2, 450, 128, 128, seed=8200 + int(causal), v_spread=6.0)
    check_fp8(fa, orc, c, 128, causal, 0.0883883, f"gqa spread causal={causal}")


def test_large_logits(fa, orc):
    """Peaked rows (logits spread x4): the reference moves, P~ rounds near 1."""
    c = fp8_case(orc, 1, 4, 4, 700, 128, 64, seed=8300, dist_scale=2.0)
    check_fp8(fa, orc, c, 64, True, 0.2, "large logits")


def test_heads_multiple_of_eight_device_quantiser(fa, orc):
    """The whole FP8 path on the GPU: both quantisers, then the forward, with
    the XCD-grouped workgroup order (16 heads)."""
    import torch
    c = fp8_case(orc, 2, 8, 2, 520, 128, 128, seed=8400)
    inp = ai.make_case(2, 8, 2, 520, 128, seed=8400, with_grad=False)
    v = to_dev(inp["v"])
    q8, qs = fa.quantize_e4m3(to_dev(inp["q"]), 128)
    k8, ks = fa.quantize_e4m3(to_dev(inp["k"]), 128)
    v8t, vs = fa.quantize_e4m3_vt(v, 128)
    torch.cuda.synchronize()
    assert np.array_equal(q8.cpu().numpy(), c["q8"]) and np.array_equal(k8.cpu().numpy(), c["k8"])
    assert np.array_equal(v8t.cpu().numpy(), vt_layout(c["v8"]))
    check_fp8(fa, orc, c, 128, True, 0.0883883, "device quantisers", device_quant=(v8t, vs))


def test_constant_v(fa, orc):
    """Every V code equal (one run): O equals that value exactly up to the
    bf16 output rounding, whatever P rounds to."""
    import torch
    c = fp8_case(orc, 1, 2, 2, 300, 128, 64, seed=8500)
    c["v8"][:] = 0x3B                                               # 1.375
    c["vs"][:] = 0.5
    o, _ = run_fp8(fa, c, 64, True, 0.0883883)
    assert np.max(np.abs(o - 0.6875)) == 0.0


def test_full_size_gqa16k_sampled_rows(fa, orc):
    """The configuration bench.py --fp8 times (gqa16k: B=2, Hq=32, Hkv=8,
    N=16384, d=128, causal, 128-row runs, device quantisers), checked on 24
    seeded rows (always 0 and N-1) of two heads in different K/V groups, all
    16384 keys each, to the same bounds."""
    import torch
    w = ai.WORKLOADS["gqa16k"]
    rows = 128
    inp = ai.make_inputs(w, with_grad=False)
    q, k, v = (to_dev(inp[t]) for t in ("q", "k", "v"))
    q8, qs = fa.quantize_e4m3(q, rows)
    k8, ks = fa.quantize_e4m3(k, rows)
    v8t, vs = fa.quantize_e4m3_vt(v, rows)
    say("fwd_e4m3 gqa16k full size")
    o, lse = fa.fwd_e4m3(q8, qs, k8, ks, v8t, vs, rows, causal=w.causal, scale=w.scale)
    torch.cuda.synchronize()
    rows_idx = ai.sample_rows(w.N, 24, w.cfg_id)
    worst = 0.0
    for b, h in ((0, 0), (1, 29)):
        hk = h // w.G
        qh = ai.bf16_bits_to_f32(inp["q"][b, h])[None, None]
        kh = ai.bf16_bits_to_f32(inp["k"][b, hk])[None, None]
        vh = ai.bf16_bits_to_f32(inp["v"][b, hk])[None, None]
        q8h, qsh = orc.quantize_e4m3(qh, rows)
        k8h, ksh = orc.quantize_e4m3(kh, rows)
        v8h, vsh = orc.quantize_e4m3(vh, rows)
        # the device's codes and scales are the oracle's
        assert np.array_equal(q8[b, h].cpu().numpy(), q8h[0, 0]) and np.array_equal(k8[b, hk].cpu().numpy(), k8h[0, 0])
        assert np.array_equal(vs[b, hk].cpu().numpy().view(np.uint32), vsh[0, 0].view(np.uint32))
        vdeq = orc.dequantize_e4m3(v8h, vsh, rows)[0, 0]
        P, O, L, xabs = head_reference(orc, q8h[0, 0], qsh[0, 0], k8h[0, 0], ksh[0, 0], vdeq, rows_idx, rows,
                                       w.causal, w.scale)
        bound = head_bound(orc, v8h[0, 0], vsh[0, 0], vdeq, rows, P, O, xabs)
        og = from_dev_bf16(o[b, h])[rows_idx]
        lg = lse[b, h].double().cpu().numpy()[rows_idx]
        lb = 1e-5 + 2.0 ** -19 * xabs + w.N * 2.0 ** -23
        eo, el = np.abs(og - O), np.abs(lg - L)
        ratio, lratio = float((eo / bound).max()), float((el / lb).max())
        worst = max(worst, ratio)
        say(f"gqa16k head ({b}, {h}): max|O - O'| {eo.max():.3e} ({ratio:.3f} of the bound), "
            f"max|LSE - LSE'| {el.max():.2e} ({lratio:.3f} of its bound)")
        assert np.all(np.isfinite(og)) and ratio <= 1.0 and lratio <= 1.0, (b, h, ratio, lratio)
