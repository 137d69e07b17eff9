"""GPU forward over packed sequences of different lengths against the fp64 oracle.

Each sequence is an independent attention problem, so the oracle runs the
textbook definition on each sequence's rows alone. Tolerances are the forward
pass's (O <= 1e-2 beyond the bf16 output rounding, LSE <= 1e-3). Small cases
compare every element; the full-size packed workload compares seeded samples
of query rows in every sequence, which the oracle computes one by one.
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


def run_varlen(fa, inp, causal, scale, max_seqlen=None):
    import torch
    q, k, v = to_dev(inp["q"]), to_dev(inp["k"]), to_dev(inp["v"])
    cu = torch.as_tensor(inp["cu_seqlens"]).cuda()
    ms = int(max(inp["lengths"].max(), 1)) if max_seqlen is None else max_seqlen
    o, lse = fa.fwd_varlen(q, k, v, cu, ms, causal=causal, scale=scale)
    torch.cuda.synchronize()
    return from_dev_bf16(o), from_dev_f32(lse)


def check(fa, inp, causal, scale, tag, rows_per_seq=None, max_seqlen=None):
    lens, cu = inp["lengths"], inp["cu_seqlens"]
    Hq, total, d = inp["q"].shape
    say(f"varlen {tag}: B={len(lens)} Hq={Hq} Hkv={inp['k'].shape[0]} total={total} d={d} causal={causal}")
    o, lse = run_varlen(fa, inp, causal, scale, max_seqlen)
    eo = el = 0.0
    for b, n in enumerate(lens):
        if n == 0:
            continue
        s0, s1 = int(cu[b]), int(cu[b + 1])
        rows = np.arange(n, dtype=np.int64) if rows_per_seq is None else ai.sample_rows(int(n), rows_per_seq, 50 + b)
        qs = f64(inp["q"][None, :, s0:s1][:, :, rows])
        ks, vs = f64(inp["k"][None, :, s0:s1]), f64(inp["v"][None, :, s0:s1])
        ro, rl = oracle.fwd(qs, ks, vs, causal, scale, qpos=rows)
        eo = max(eo, excess_err(o[None, :, s0:s1][:, :, rows], ro))
        el = max(el, max_err(lse[None, :, s0:s1][:, :, rows], rl))
    assert eo <= TOL_O and el <= TOL_LSE, f"{tag}: O err {eo:.2e}, LSE err {el:.2e}"


LENGTHS = [
    [1],
    [300],
    [1, 17, 256, 257, 700],
    [0, 64, 0, 513, 5],          # empty sequences in between
    [1000, 999, 3, 1024],
]


@pytest.mark.parametrize("d", [64, 128, 256])
@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("lens", LENGTHS, ids=["-".join(map(str, x)) for x in LENGTHS])
def test_lengths(fa, lens, causal, d):
    inp = ai.make_varlen_case(lens, 4, 2, d, seed=sum(lens) % 997 + d + int(causal))
    check(fa, inp, causal, 1.0 / math.sqrt(d), f"lengths {lens}")


def test_grid_larger_than_longest(fa):
    """max_seqlen above every length: the extra q-tiles exit at once."""
    inp = ai.make_varlen_case([100, 333], 8, 2, 128, seed=7)
    check(fa, inp, True, 0.0883883, "max_seqlen 2000", max_seqlen=2000)


@pytest.mark.parametrize("causal", [True, False])
def test_equal_lengths_match_fixed(fa, causal):
    """B sequences of one length N give bit-identical results to flash_attn_fwd
    on the [B, H, N, d] layout of the same data."""
    import torch
    B, Hq, Hkv, N, d = 3, 8, 2, 600, 128
    inp = ai.make_varlen_case([N] * B, Hq, Hkv, d, seed=8 + int(causal))
    say(f"varlen equal lengths vs fixed causal={causal}")
    o_v, l_v = run_varlen(fa, inp, causal, 0.0883883)

    def fixed(x, H):
        return np.ascontiguousarray(x.reshape(H, B, N, d).transpose(1, 0, 2, 3))
    q, k, v = to_dev(fixed(inp["q"], Hq)), to_dev(fixed(inp["k"], Hkv)), to_dev(fixed(inp["v"], Hkv))
    o_f, l_f = fa.fwd(q, k, v, causal=causal, scale=0.0883883)
    torch.cuda.synchronize()
    o_f = from_dev_bf16(o_f).transpose(1, 0, 2, 3).reshape(Hq, B * N, d)
    l_f = from_dev_f32(l_f).transpose(1, 0, 2).reshape(Hq, B * N)
    assert np.array_equal(o_v, o_f) and np.array_equal(l_v, l_f)


@pytest.mark.parametrize("name", sorted(ai.VARLEN_WORKLOADS))
def test_workload_sampled(fa, name):
    """The measured packed workload at full size; 64 seeded rows per sequence
    (always the first and last) against the oracle."""
    w = ai.VARLEN_WORKLOADS[name]
    inp = ai.make_varlen_inputs(w)
    check(fa, inp, w.causal, w.scale, name, rows_per_seq=64)


# ------------------------------------------------------------------ backward
TOL_GRAD = 2e-2


def make_grad_case(lengths, Hq, Hkv, d, seed):
    inp = ai.make_varlen_case(lengths, Hq, Hkv, d, seed)
    inp["do"] = ai.normal_bf16(inp["q"].shape, 4000 + seed, ai.TENSOR_DO)
    return inp


def check_bwd(fa, inp, scale, tag, seqs=None, sample=None, causal=True):
    """GPU forward + backward on the packed batch, then per sequence (all, or
    the listed ones) the oracle's gradients of that sequence alone; `sample`
    rows/keys per sequence when given (sampled oracle), else every element."""
    import torch
    lens, cu = inp["lengths"], inp["cu_seqlens"]
    Hq, total, d = inp["q"].shape
    Hkv = inp["k"].shape[0]
    say(f"bwd varlen {tag}: B={len(lens)} Hq={Hq} Hkv={Hkv} total={total} d={d} causal={causal}")
    q, k, v, do = to_dev(inp["q"]), to_dev(inp["k"]), to_dev(inp["v"]), to_dev(inp["do"])
    cud = torch.as_tensor(cu).cuda()
    ms = int(max(lens.max(), 1))
    o, lse = fa.fwd_varlen(q, k, v, cud, ms, causal=causal, scale=scale)
    dq, dk, dv = fa.bwd_varlen(q, k, v, o, lse, do, cud, ms, causal=causal, scale=scale)
    torch.cuda.synchronize()
    dq, dk, dv = from_dev_bf16(dq), from_dev_bf16(dk), from_dev_bf16(dv)
    errs = {"dq": 0.0, "dk": 0.0, "dv": 0.0}
    for b in (range(len(lens)) if seqs is None else seqs):
        n = int(lens[b])
        if n == 0:
            continue
        s0, s1 = int(cu[b]), int(cu[b + 1])
        qs, ks, vs, ds = (f64(inp[t][None, :, s0:s1]) for t in ("q", "k", "v", "do"))
        if sample is None:
            ref = oracle.bwd(qs, ks, vs, ds, causal, scale)
            got = {"dq": dq[None, :, s0:s1], "dk": dk[None, :, s0:s1], "dv": dv[None, :, s0:s1]}
        else:
            rows = ai.sample_rows(n, sample, 60 + b)
            keys = ai.sample_rows(n, sample, 160 + b)
            ref = oracle.bwd_sampled(qs, ks, vs, ds, causal, scale, rows, keys)
            got = {"dq": dq[None, :, s0:s1][:, :, rows], "dk": dk[None, :, s0:s1][:, :, keys],
                   "dv": dv[None, :, s0:s1][:, :, keys]}
        for key in errs:
            errs[key] = max(errs[key], excess_err(got[key], ref[key]))
    assert all(e <= TOL_GRAD for e in errs.values()), f"{tag}: {errs}"


@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("lens", LENGTHS, ids=["-".join(map(str, x)) for x in LENGTHS])
def test_bwd_lengths(fa, lens, d, causal):
    """Sequence boundaries inside 32-row waves, 64-key tiles and 128-key
    workgroups, with empty sequences between them."""
    inp = make_grad_case(lens, 4, 2, d, seed=sum(lens) % 991 + d + 3 * int(not causal))
    check_bwd(fa, inp, 1.0 / math.sqrt(d), f"lengths {lens}", causal=causal)


@pytest.mark.parametrize("causal", [True, False])
def test_bwd_many_short(fa, causal):
    """40 sequences of 1..200 tokens: most tiles cross a boundary."""
    lens = np.random.default_rng(5).integers(1, 200, size=40)
    inp = make_grad_case(lens, 4, 2, 128, seed=77)
    check_bwd(fa, inp, 0.0883883, "many short", causal=causal)


@pytest.mark.parametrize("causal", [True, False])
def test_bwd_large_logits(fa, causal):
    inp = ai.make_varlen_case([700, 1300, 90], 4, 4, 128, seed=78)
    inp["q"] = ai.bf16_round_bits(f64(inp["q"]).astype(np.float32) * 2)
    inp["k"] = ai.bf16_round_bits(f64(inp["k"]).astype(np.float32) * 2)
    inp["do"] = ai.normal_bf16(inp["q"].shape, 4078, ai.TENSOR_DO)
    check_bwd(fa, inp, 0.2, "large logits", causal=causal)


@pytest.mark.parametrize("causal", [True, False])
def test_bwd_workload_sampled(fa, causal):
    """The packed workload (16 prompts of 512..16384 tokens) at full size; the
    shortest and the longest sequence checked on 128 sampled rows and keys."""
    w = ai.VARLEN_WORKLOADS["varlen_mix"]
    inp = ai.make_varlen_inputs(w)
    inp["do"] = ai.normal_bf16(inp["q"].shape, w.cfg_id, ai.TENSOR_DO)
    lens = inp["lengths"]
    check_bwd(fa, inp, w.scale, "varlen_mix", seqs=[int(np.argmin(lens)), int(np.argmax(lens))], sample=128,
              causal=causal)


def test_bwd_noncausal_equal_lengths_match_fixed(fa):
    """Equal lengths without the causal mask: the packed backward and the
    fixed-length non-causal backward (a separate kernel instantiation, itself
    checked against the oracle) agree within the gradient tolerance."""
    import torch
    B, Hq, Hkv, N, d = 3, 4, 2, 320, 128
    inp = make_grad_case([N] * B, Hq, Hkv, d, seed=91)
    say(f"bwd varlen equal lengths vs fixed, non-causal: B={B} N={N}")
    q, k, v, do = (to_dev(inp[t]) for t in ("q", "k", "v", "do"))
    cud = torch.as_tensor(inp["cu_seqlens"]).cuda()
    o, lse = fa.fwd_varlen(q, k, v, cud, N, causal=False, scale=0.0883883)
    dq, dk, dv = fa.bwd_varlen(q, k, v, o, lse, do, cud, N, causal=False, scale=0.0883883)

    def fixed(t):   # [H, B*N, d] -> [B, H, N, d]
        return t.reshape(t.shape[0], B, N, *t.shape[2:]).transpose(0, 1).contiguous()

    def packed(t):  # [B, H, N, d] -> [H, B*N, d]
        return t.transpose(0, 1).reshape(t.shape[1], B * N, *t.shape[3:]).contiguous()

    fq, fk, fv, fdo = fixed(q), fixed(k), fixed(v), fixed(do)
    fo, flse = fa.fwd(fq, fk, fv, causal=False, scale=0.0883883)
    gq, gk, gv = fa.bwd(fq, fk, fv, fo, flse, fdo, causal=False, scale=0.0883883)
    torch.cuda.synchronize()
    for a, b_, name in ((dq, packed(gq), "dq"), (dk, packed(gk), "dk"), (dv, packed(gv), "dv")):
        err = (a.float() - b_.float()).abs().max().item()
        assert err <= 2e-2, f"{name}: {err}"


@pytest.mark.parametrize("d", [32, 96])
@pytest.mark.parametrize("causal", [True, False])
def test_padded_headdim(fa, d, causal):
    """Packed sequences with head dimensions below 64 / 128: forward and backward."""
    lens = [0, 64, 0, 513, 5]
    inp = ai.make_varlen_case(lens, 4, 2, d, seed=7700 + d + int(causal))
    check(fa, inp, causal, 1.0 / math.sqrt(d), f"padded d={d} lengths {lens}")
    inp = make_grad_case([1, 17, 256, 257, 700], 4, 2, d, seed=7800 + d + int(causal))
    check_bwd(fa, inp, 1.0 / math.sqrt(d), f"padded d={d}", causal=causal)


@pytest.mark.parametrize("causal", [True, False])
def test_wide_headdim_bwd(fa, causal):
    """d = 256 packed sequences: the split gradient kernels with sequence bounds."""
    inp = make_grad_case([1, 17, 256, 257, 700], 4, 2, 256, seed=8000 + int(causal))
    check_bwd(fa, inp, 0.0625, "wide d=256", causal=causal)


def test_twelve_wave_workgroups(fa):
    """Packed sequences of up to 4100 rows with 64 query heads: the d = 64
    forward takes 12-wave workgroups (the launch geometry for B sequences of the
    longest length confirms it); 128 seeded rows per sequence against the
    oracle."""
    lens = [4100, 1, 3000, 2500, 0, 777]
    g = fa.fwd_geometry(len(lens), 64, 8, max(lens), 64, True)
    assert g["threads"] == 768, g
    for causal in (True, False):
        inp = ai.make_varlen_case(lens, 64, 8, 64, seed=12 + int(causal))
        check(fa, inp, causal, 0.125, f"12 waves causal={causal}", rows_per_seq=128)


@pytest.mark.parametrize("causal", [True, False])
def test_equal_lengths_match_fixed_twelve_waves(fa, causal):
    """As test_equal_lengths_match_fixed, at a size where both calls take the
    d = 64 forward's 12-wave workgroups: bit-identical results."""
    import torch
    B, Hq, Hkv, N, d = 2, 64, 8, 2100, 64
    assert fa.fwd_geometry(B, Hq, Hkv, N, d, causal)["threads"] == 768
    inp = ai.make_varlen_case([N] * B, Hq, Hkv, d, seed=9 + int(causal))
    say(f"varlen equal lengths vs fixed, 12 waves, causal={causal}")
    o_v, l_v = run_varlen(fa, inp, causal, 0.125)

    def fixed(x, H):
        return np.ascontiguousarray(x.reshape(H, B, N, d).transpose(1, 0, 2, 3))
    q, k, v = to_dev(fixed(inp["q"], Hq)), to_dev(fixed(inp["k"], Hkv)), to_dev(fixed(inp["v"], Hkv))
    o_f, l_f = fa.fwd(q, k, v, causal=causal, scale=0.125)
    torch.cuda.synchronize()
    o_f = from_dev_bf16(o_f).transpose(1, 0, 2, 3).reshape(Hq, B * N, d)
    l_f = from_dev_f32(l_f).transpose(1, 0, 2).reshape(Hq, B * N)
    assert np.array_equal(o_v, o_f) and np.array_equal(l_v, l_f)
