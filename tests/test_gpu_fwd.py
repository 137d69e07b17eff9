"""GPU forward pass against the fp64 oracle on identical seeded bf16 inputs.

Tolerances: max abs error on O <= 1e-2 beyond the rounding of the bf16 output
(half a bf16 ulp at the oracle's value), and on the fp32 LSE <= 1e-3. Small
cases are compared element by element on every output.
The spiky N = 8192 workload is compared on every row of every head; the other
full-size workloads on seeded samples of query rows that the oracle computes
one by one (every row of the GQA workload's two seeded groups is checked in the
backward tests). Failure messages carry the plain max abs error beside the error
beyond the output rounding. Closed forms (constant V, causal row 0, uniform attention
at scale 0) are checked on every row.
"""
import math

import numpy as np
import pytest

import attn_inputs as ai
import oracle
from tests.gpu_util import (TOL_LSE, TOL_O, check_outputs, excess_err, f64, from_dev_bf16, from_dev_f32, max_err,
                            say, to_dev)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def fa():
    import torch
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a GPU")
    import exact_io_aware_60_amd as fa
    fa.lib()
    return fa


def run_fwd(fa, inp, causal, scale):
    q, k, v = to_dev(inp["q"]), to_dev(inp["k"]), to_dev(inp["v"])
    o, lse = fa.fwd(q, k, v, causal=causal, scale=scale)
    import torch
    torch.cuda.synchronize()
    return from_dev_bf16(o), from_dev_f32(lse)


def check_full(fa, inp, causal, scale, tag):
    say(f"fwd {tag}")
    o, lse = run_fwd(fa, inp, causal, scale)
    ro, rl = oracle.fwd(f64(inp["q"]), f64(inp["k"]), f64(inp["v"]), causal, scale)
    errs = check_outputs(tag, {"o": (o, ro), "lse": (lse, rl)}, dict(o=TOL_O, lse=TOL_LSE))
    return errs["o"], errs["lse"]


def test_tiny_workload(fa):
    """The 1-head, N = 256, d = 64, non-causal workload with fp32-drawn inputs
    rounded to bf16; both sides see the same rounded values."""
    w = ai.WORKLOADS["tiny"]
    inp = ai.make_inputs(w)
    check_full(fa, inp, w.causal, w.scale, "tiny")


@pytest.mark.parametrize("d", [64, 128, 256])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("N", [1, 2, 3, 17, 63, 64, 65, 255, 256, 257, 300, 700])
def test_ragged(fa, d, causal, N):
    inp = ai.make_case(1, 2, 2, N, d, seed=N * 7 + d + int(causal), with_grad=False)
    check_full(fa, inp, causal, 1.0 / math.sqrt(d), f"ragged N={N} d={d} causal={causal}")


@pytest.mark.parametrize("d", [64, 128, 256])
def test_gqa_small(fa, d):
    inp = ai.make_case(2, 8, 2, 333, d, seed=400 + d, with_grad=False)
    check_full(fa, inp, True, 1.0 / math.sqrt(d), f"gqa d={d}")
    check_full(fa, inp, False, 1.0 / math.sqrt(d), f"gqa d={d} noncausal")


def test_head_count_multiple_of_eight(fa):
    """Head counts that are a multiple of 8 take the XCD-grouped workgroup order."""
    inp = ai.make_case(2, 8, 4, 520, 128, seed=77, with_grad=False)
    check_full(fa, inp, True, 0.0883883, "heads%8==0")


@pytest.mark.parametrize("d", [128, 256])
def test_large_logits(fa, d):
    """Scores spread by a factor of 4 on some keys and a larger scale: exercises
    the lazy reference-max rescale."""
    inp = ai.make_case(1, 4, 4, 1000, d, seed=5 + d, with_grad=False, dist_scale=2.0)
    check_full(fa, inp, True, 0.2 * math.sqrt(128 / d), f"large logits d={d}")


def test_d256_head_count_multiple_of_eight(fa):
    """d = 256 (four waves, 128-row workgroups) with the XCD-grouped order."""
    inp = ai.make_case(2, 8, 2, 600, 256, seed=78, with_grad=False)
    check_full(fa, inp, True, 0.0625, "d=256 heads%8==0")
    check_full(fa, inp, False, 0.0625, "d=256 heads%8==0 noncausal")


@pytest.mark.parametrize("causal", [False, True])
def test_constant_v(fa, causal):
    """Every v_j equal: O_i = v exactly for every row."""
    inp = ai.make_case(1, 2, 2, 500, 128, seed=11, with_grad=False)
    inp["v"] = np.broadcast_to(inp["v"][:, :, :1], inp["v"].shape).copy()
    say(f"fwd constant V causal={causal}")
    o, _ = run_fwd(fa, inp, causal, 0.0883883)
    assert excess_err(o, np.broadcast_to(f64(inp["v"][:, :, :1]), o.shape)) <= TOL_O


def test_causal_row_zero(fa):
    """Causal row 0 attends only to key 0: O_0 = v_0, LSE_0 = s q_0.k_0."""
    inp = ai.make_case(2, 4, 4, 300, 64, seed=12, with_grad=False)
    s = 0.125
    say("fwd causal row 0")
    o, lse = run_fwd(fa, inp, True, s)
    q, k, v = f64(inp["q"]), f64(inp["k"]), f64(inp["v"])
    assert excess_err(o[:, :, 0], v[:, :, 0]) <= TOL_O
    assert max_err(lse[:, :, 0], s * np.einsum("bhd,bhd->bh", q[:, :, 0], k[:, :, 0])) <= TOL_LSE


@pytest.mark.parametrize("d", [64, 128, 256])
def test_uniform_scale_zero(fa, d):
    """scale = 0: causal O_i is the prefix mean of V and LSE_i = ln(i + 1)."""
    inp = ai.make_case(1, 2, 1, 777, d, seed=13, with_grad=False)
    say(f"fwd scale 0 d={d}")
    o, lse = run_fwd(fa, inp, True, 0.0)
    v = f64(inp["v"])
    G = 2
    ref = np.repeat(np.cumsum(v, axis=2) / np.arange(1, 778)[None, None, :, None], G, axis=1)
    assert excess_err(o, ref) <= TOL_O
    assert max_err(lse, np.broadcast_to(np.log(np.arange(1, 778)), lse.shape)) <= TOL_LSE


def test_deterministic(fa):
    inp = ai.make_case(1, 4, 2, 1000, 128, seed=21, with_grad=False)
    say("fwd determinism")
    o1, l1 = run_fwd(fa, inp, True, 0.0883883)
    o2, l2 = run_fwd(fa, inp, True, 0.0883883)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


# ------------------------------------------------------------------ full-size workloads
def sampled_check(fa, w, inp, rows, heads_b=None):
    """Run the full GPU forward, then compare the sampled query rows (all heads, or
    the (b, kv-head) groups listed) with the oracle."""
    import torch
    say(f"fwd workload {w.name} (full size on GPU, {len(rows)} sampled rows)")
    q, k, v = to_dev(inp["q"]), to_dev(inp["k"]), to_dev(inp["v"])
    o, lse = fa.fwd(q, k, v, causal=w.causal, scale=w.scale)
    torch.cuda.synchronize()
    rows_t = torch.as_tensor(rows, device=o.device)
    o_s = from_dev_bf16(o.index_select(2, rows_t))
    l_s = from_dev_f32(lse.index_select(2, rows_t))
    del q, k, v, o, lse
    ro, rl = oracle.fwd(f64(inp["q"][:, :, rows]), f64(inp["k"]), f64(inp["v"]), w.causal, w.scale, qpos=rows)
    check_outputs(f"{w.name} ({len(rows)} rows)", {"o": (o_s, ro), "lse": (l_s, rl)}, dict(o=TOL_O, lse=TOL_LSE))


@pytest.mark.parametrize("name", ["mha2k", "spiky8k", "gqa16k", "long128k"])
def test_workload_sampled(fa, name):
    """The full-size forward on seeded rows of every head (every row at mha2k).
    The spiky and GQA workloads' forward outputs are also checked on every
    element of every head they cover in the backward tests."""
    w = ai.WORKLOADS[name]
    inp = ai.make_inputs(w, with_grad=False)
    rows = ai.sample_rows(w.N, 256 if name != "mha2k" else w.N, w.cfg_id)
    sampled_check(fa, w, inp, rows)


def test_workload_spiky8k_every_row(fa):
    """N = 8192, d = 128, causal, spiked K: O and LSE of every row of all 32
    heads against the oracle."""
    w = ai.WORKLOADS["spiky8k"]
    inp = ai.make_inputs(w, with_grad=False)
    check_full(fa, inp, w.causal, w.scale, "spiky8k (every row, every head)")


def test_d256_full_size_sampled(fa):
    """d = 256 at a prefill size (B=2, Hq=16, Hkv=4, N=16384, causal) on 128
    seeded rows of every head."""
    w = ai.WORKLOADS["gqa16k_d256"]
    inp = ai.make_inputs(w, with_grad=False)
    rows = ai.sample_rows(w.N, 128, w.cfg_id)
    sampled_check(fa, w, inp, rows)


def test_long_context_every_row_uniform(fa):
    """N = 131072, 8 heads, d = 128, causal, Q = 0: every row's output is the
    prefix mean of V and LSE_i = ln(i + 1). This checks all rows at full length."""
    import torch
    w = ai.WORKLOADS["long128k"]
    inp = ai.make_inputs(w, with_grad=False)
    say("fwd long128k with Q = 0 (all rows)")
    q = torch.zeros((w.B, w.Hq, w.N, w.d), dtype=torch.bfloat16, device="cuda")
    k, v = to_dev(inp["k"]), to_dev(inp["v"])
    o, lse = fa.fwd(q, k, v, causal=True, scale=w.scale)
    vf = v.float()
    ref = torch.cumsum(vf.double(), dim=2) / torch.arange(1, w.N + 1, device=v.device, dtype=torch.float64)[None, None, :, None]
    half_ulp = torch.exp2(torch.floor(torch.log2(ref.abs().clamp_min(2.0 ** -126))) - 8)
    err_o = ((o.double() - ref).abs() - half_ulp).max().item()
    err_l = (lse.double() - torch.log(torch.arange(1, w.N + 1, device=v.device, dtype=torch.float64))).abs().max().item()
    assert err_o <= TOL_O, err_o
    assert err_l <= TOL_LSE, err_l


def test_long_context_memory_footprint(fa):
    """O(N d) memory at N = 131072, 8 heads, d = 128: the forward allocates no
    device memory of its own (free device memory is the same before and after a
    call), and the tensors in use are Q, K, V, O and LSE, about 1.08 GB, where
    one bf16 score matrix per head would take 275 GB."""
    import torch
    w = ai.WORKLOADS["long128k"]
    say("fwd long128k memory footprint")
    q = torch.randn((w.B, w.Hq, w.N, w.d), device="cuda").bfloat16()
    k = torch.randn((w.B, w.Hkv, w.N, w.d), device="cuda").bfloat16()
    v = torch.randn((w.B, w.Hkv, w.N, w.d), device="cuda").bfloat16()
    o = torch.empty_like(q)
    lse = torch.empty((w.B, w.Hq, w.N), dtype=torch.float32, device="cuda")
    args = (q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(), w.B, w.Hq, w.Hkv, w.N, w.d,
            1, w.scale)
    assert fa.fwd_raw(*args) == 0                  # first call: code objects load
    torch.cuda.synchronize()
    free0, _ = torch.cuda.mem_get_info()
    torch.cuda.reset_peak_memory_stats()
    held = torch.cuda.memory_allocated()
    assert fa.fwd_raw(*args) == 0
    torch.cuda.synchronize()
    free1, _ = torch.cuda.mem_get_info()
    assert free1 == free0, (free0, free1)          # no device allocation during the call
    assert torch.cuda.max_memory_allocated() == held
    tensors = sum(t.numel() * t.element_size() for t in (q, k, v, o, lse))
    assert tensors == 4 * w.B * w.Hq * w.N * w.d * 2 + w.B * w.Hq * w.N * 4
    assert round(tensors / 1e9, 2) == 1.08
    assert w.B * w.Hq * w.N * w.N * 2 > 250 * tensors


# ------------------------------------------------------------------ head dimensions below 64 / 128 / 256
@pytest.mark.parametrize("d", [8, 32, 40, 96, 112, 200])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("N", [1, 17, 64, 129, 300])
def test_padded_headdim(fa, d, causal, N):
    """Rows of d values run on the 64-, 128- or 256-wide instance with zero
    columns past d: every element against the oracle at d itself."""
    inp = ai.make_case(1, 2, 2, N, d, seed=6000 + N * 3 + d + int(causal), with_grad=False)
    check_full(fa, inp, causal, 1.0 / math.sqrt(d), f"padded d={d} N={N} causal={causal}")


@pytest.mark.parametrize("d", [32, 96])
def test_padded_headdim_gqa(fa, d):
    inp = ai.make_case(2, 8, 2, 700, d, seed=6100 + d, with_grad=False)
    check_full(fa, inp, True, 1.0 / math.sqrt(d), f"padded gqa d={d}")
    check_full(fa, inp, False, 1.0 / math.sqrt(d), f"padded gqa d={d} noncausal")


@pytest.mark.parametrize("d", [64, 48])
@pytest.mark.parametrize("causal", [False, True])
def test_twelve_wave_workgroups(fa, d, causal):
    """64 query heads over 8 K/V heads, N = 4100: a grid large enough for the
    d <= 64 forward's 12-wave (384-row) workgroups, which the launch geometry
    confirms; every row against the oracle, ragged last q-tile and key tile."""
    g = fa.fwd_geometry(1, 64, 8, 4100, d, causal)
    assert g["threads"] == 768 and g["block_m"] == 384, g
    inp = ai.make_case(1, 64, 8, 4100, d, seed=4100 + d + int(causal), with_grad=False)
    check_full(fa, inp, causal, 1.0 / math.sqrt(d), f"12 waves d={d} causal={causal}")


@pytest.mark.parametrize("d", [64, 48])
def test_launch_shape_does_not_change_results(fa, d):
    """Both launch shapes of the d <= 64 forward group rows into the same
    32-row waves and walk the same chunks, so a 64-head call (12-wave
    workgroups) and eight calls of 8 heads each (8-wave workgroups) give the
    same bits."""
    import torch
    B, Hq, Hkv, N = 1, 64, 8, 4100
    assert fa.fwd_geometry(B, Hq, Hkv, N, d, True)["threads"] == 768
    assert fa.fwd_geometry(B, Hq // Hkv, 1, N, d, True)["threads"] == 512
    inp = ai.make_case(B, Hq, Hkv, N, d, seed=4242 + d, with_grad=False)
    say(f"fwd launch shapes d={d}")
    q, k, v = to_dev(inp["q"]), to_dev(inp["k"]), to_dev(inp["v"])
    o, lse = fa.fwd(q, k, v, causal=True, scale=0.125)
    G = Hq // Hkv
    for g in range(Hkv):
        qs = q[:, g * G:(g + 1) * G].contiguous()
        o_g, lse_g = fa.fwd(qs, k[:, g:g + 1].contiguous(), v[:, g:g + 1].contiguous(), causal=True, scale=0.125)
        torch.cuda.synchronize()
        assert torch.equal(o_g, o[:, g * G:(g + 1) * G]) and torch.equal(lse_g, lse[:, g * G:(g + 1) * G]), g


@pytest.mark.parametrize("causal", [False, True])
def test_d128_four_and_eight_wave_forwards_agree(fa, causal):
    """At d = 128 the forward runs 4-wave (128-row) workgroups up to 16384 rows
    per head and on small grids, 8-wave (256-row) ones otherwise. Both group
    rows into the same 32-row waves and walk the same chunks, so 8 heads of
    N = 16400 in one call (520 workgroups of 256 rows: 8 waves) and each head
    alone (65: 4 waves) give the same bits. The small-shape tests pin the
    4-wave form to the oracle; the long-context sample pins the 8-wave one."""
    import torch
    B, H, N = 1, 8, 16400
    assert fa.fwd_geometry(B, H, H, N, 128, causal)["threads"] == 512
    assert fa.fwd_geometry(B, 1, 1, N, 128, causal)["threads"] == 256
    inp = ai.make_case(B, H, H, N, 128, seed=16400 + int(causal), with_grad=False)
    say(f"fwd d=128 4- vs 8-wave causal={causal}")
    q, k, v = to_dev(inp["q"]), to_dev(inp["k"]), to_dev(inp["v"])
    o, lse = fa.fwd(q, k, v, causal=causal, scale=0.0883883)
    for h in range(H):
        sl = lambda t: t[:, h:h + 1].contiguous()
        o1, lse1 = fa.fwd(sl(q), sl(k), sl(v), causal=causal, scale=0.0883883)
        torch.cuda.synchronize()
        assert torch.equal(o1, o[:, h:h + 1]) and torch.equal(lse1, lse[:, h:h + 1]), h


@pytest.mark.parametrize("d", [64, 128, 256])
def test_value_scale_homogeneity(fa, d):
    """O is homogeneous in V and the forward's arithmetic on V is exact scaling
    by powers of two (products, sums and the final division), so V * 2^e gives
    O * 2^e bit for bit and the same LSE, as long as nothing overflows or
    underflows. e = +-60 with spread scores (the reference moves, and P stays
    up to 2^16 between moves) checks the accumulators' range at both ends."""
    import torch
    inp = ai.make_case(1, 4, 2, 900, d, seed=31 + d, with_grad=False, dist_scale=2.0)
    s = 0.2 * math.sqrt(128 / d)
    say(f"fwd value-scale homogeneity d={d}")
    o, lse = run_fwd(fa, inp, True, s)
    for e in (60, -60):
        v = torch.from_numpy(f64(inp["v"]) * 2.0 ** e).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
        o2, lse2 = run_fwd(fa, dict(inp, v=v), True, s)
        assert np.array_equal(o2, o * 2.0 ** e), e
        assert np.array_equal(lse2, lse), e
