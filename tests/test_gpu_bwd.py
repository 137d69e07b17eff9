"""GPU backward pass against the fp64 oracle on identical seeded bf16 inputs.

The GPU backward is fed the GPU forward's own O and LSE, as a caller would; the
oracle computes everything from the inputs in fp64 (exact D). Tolerance: max
abs error on
dQ, dK and dV <= 2e-2 beyond the rounding of the bf16 output (half a bf16 ulp at
the oracle's value). Small cases are compared element by element on every
output. The full-size workloads are compared on every element too: the spiky
N = 8192 workload on all 32 heads, the GQA N = 16384 workload on two seeded
(batch, K/V head) groups, each group's four query heads and one K/V head whole.
Failure messages carry the plain max abs error beside the error beyond the
output rounding.
"""
import math

import numpy as np
import pytest

import attn_inputs as ai
import oracle
from tests.gpu_util import (TOL_GRAD, TOL_LSE, TOL_O, check_outputs, excess_err, f64, from_dev_bf16,
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


def run_fwd_bwd(fa, inp, causal, scale):
    """GPU forward then backward on the same device tensors; returns host fp64 arrays."""
    import torch
    q, k, v, do = to_dev(inp["q"]), to_dev(inp["k"]), to_dev(inp["v"]), to_dev(inp["do"])
    o, lse = fa.fwd(q, k, v, causal=causal, scale=scale)
    dq, dk, dv = fa.bwd(q, k, v, o, lse, do, causal=causal, scale=scale)
    torch.cuda.synchronize()
    return from_dev_bf16(dq), from_dev_bf16(dk), from_dev_bf16(dv)


def check_full(fa, inp, causal, scale, tag):
    say(f"bwd {tag}")
    dq, dk, dv = run_fwd_bwd(fa, inp, causal, scale)
    ref = oracle.bwd(f64(inp["q"]), f64(inp["k"]), f64(inp["v"]), f64(inp["do"]), causal, scale)
    return check_outputs(tag, {"dq": (dq, ref["dq"]), "dk": (dk, ref["dk"]), "dv": (dv, ref["dv"])},
                         dict(dq=TOL_GRAD, dk=TOL_GRAD, dv=TOL_GRAD))


def test_workload_mha2k_full(fa):
    """B=4, H=16, N=2048, d=64, causal: every gradient element against the oracle."""
    w = ai.WORKLOADS["mha2k"]
    inp = ai.make_inputs(w)
    check_full(fa, inp, w.causal, w.scale, "mha2k (all elements)")


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("N", [1, 2, 3, 17, 31, 32, 33, 63, 64, 65, 127, 128, 129, 255, 256, 257, 300, 700])
def test_ragged(fa, d, causal, N):
    inp = ai.make_case(1, 2, 2, N, d, seed=N * 11 + d + int(causal))
    check_full(fa, inp, causal, 1.0 / math.sqrt(d), f"ragged N={N} d={d} causal={causal}")


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_gqa_small(fa, d, causal):
    """Four query heads per K/V head: dK and dV sum over the group."""
    inp = ai.make_case(2, 8, 2, 333, d, seed=500 + d + int(causal))
    check_full(fa, inp, causal, 1.0 / math.sqrt(d), f"gqa d={d} causal={causal}")


def test_head_count_multiple_of_eight(fa):
    """Unit counts that are a multiple of 8 take the XCD-grouped workgroup order
    (B*Hkv = 8 for the dK/dV kernel, B*Hq = 16 for the dQ kernel)."""
    inp = ai.make_case(2, 8, 4, 520, 128, seed=78)
    check_full(fa, inp, True, 0.0883883, "units%8==0")


@pytest.mark.parametrize("B,Hq,Hkv", [(8, 16, 16), (4, 32, 8), (8, 15, 15)])
def test_d128_wave_forms(fa, B, Hq, Hkv):
    """At d = 128 the gradient kernels come in an eight-wave form (256 keys or
    rows per workgroup) for grids of 512 such workgroups or more and a four-wave
    form below. N = 1000 (four 256-row blocks, ragged): 8 x 16 heads runs both
    passes eight-wave at exactly 512 workgroups; 4 x 32 query heads over 8 K/V
    heads runs dQ eight-wave (512) and dK/dV four-wave (128), so the row dot one
    form writes feeds the other; 8 x 15 heads (480) runs both four-wave."""
    inp = ai.make_case(B, Hq, Hkv, 1000, 128, seed=900 + B * Hq + Hkv)
    check_full(fa, inp, True, 1.0 / math.sqrt(128), f"wave forms B={B} Hq={Hq} Hkv={Hkv}")


def test_large_logits(fa):
    inp = ai.make_case(1, 4, 4, 1000, 128, seed=6, dist_scale=2.0)
    check_full(fa, inp, True, 0.2, "large logits")


@pytest.mark.parametrize("causal", [False, True])
def test_constant_v(fa, causal):
    """Every v_j equal: dP_ij = D_i, so dS = 0 and dQ = dK = 0 exactly in exact
    arithmetic; dV_j = sum_i P_ij dO_i (checked against the oracle)."""
    inp = ai.make_case(1, 2, 2, 500, 128, seed=14)
    inp["v"] = np.broadcast_to(inp["v"][:, :, :1], inp["v"].shape).copy()
    say(f"bwd constant V causal={causal}")
    dq, dk, dv = run_fwd_bwd(fa, inp, causal, 0.0883883)
    ref = oracle.bwd(f64(inp["q"]), f64(inp["k"]), f64(inp["v"]), f64(inp["do"]), causal, 0.0883883)
    assert np.max(np.abs(dq)) <= TOL_GRAD and np.max(np.abs(dk)) <= TOL_GRAD
    assert excess_err(dv, ref["dv"]) <= TOL_GRAD


def test_causal_row_zero_and_sums(fa):
    """Causal row 0 has one visible key, so dQ_0 = 0. Rows of dS sum to zero, so
    sum_j dK_j = 0; rows of P sum to one, so sum_j dV_j = sum over the group of dO."""
    inp = ai.make_case(1, 4, 2, 640, 64, seed=15)
    say("bwd causal row 0 and gradient sums")
    dq, dk, dv = run_fwd_bwd(fa, inp, True, 0.125)
    assert np.max(np.abs(dq[:, :, 0])) <= TOL_GRAD
    do = f64(inp["do"])
    sum_dv = dv.sum(axis=2)
    ref_dv = do.reshape(1, 2, 2, 640, 64).sum(axis=(2, 3))
    scale_ref = np.sqrt(640 * 2)   # the sums run over 1280 terms of unit size
    assert np.max(np.abs(sum_dv - ref_dv)) <= 2e-2 * scale_ref
    assert np.max(np.abs(dk.sum(axis=2))) <= 2e-2 * scale_ref


def test_deterministic(fa):
    inp = ai.make_case(1, 4, 2, 1000, 128, seed=22)
    say("bwd determinism")
    a = run_fwd_bwd(fa, inp, True, 0.0883883)
    b = run_fwd_bwd(fa, inp, True, 0.0883883)
    for x, y in zip(a, b):
        assert np.array_equal(x, y)


@pytest.mark.parametrize("d", [64, 128])
def test_power_of_two_homogeneity(fa, d):
    """Scaling inputs by powers of two scales the gradients exactly: the kernels
    re-derive their fp16 scales, so every intermediate has the same bits.
    V * 2^12 and dO * 2^-20 give dQ, dK * 2^-8 and dV * 2^-20; Q * 2^9 with
    K * 2^-9 give dQ * 2^-9 and dK * 2^9."""
    import torch
    inp = ai.make_case(1, 4, 2, 700, d, seed=24 + d)
    say(f"bwd power-of-two homogeneity d={d}")
    s = 1.0 / math.sqrt(d)
    base = run_fwd_bwd(fa, inp, True, s)

    def scaled(name, e):
        x = torch.from_numpy(f64(inp[name]) * 2.0 ** e).to(torch.bfloat16)
        return x.view(torch.int16).numpy().view(np.uint16)

    inp2 = dict(inp, v=scaled("v", 12), do=scaled("do", -20))
    dq, dk, dv = run_fwd_bwd(fa, inp2, True, s)
    assert np.array_equal(dq, base[0] * 2.0 ** -8) and np.array_equal(dk, base[1] * 2.0 ** -8)
    assert np.array_equal(dv, base[2] * 2.0 ** -20)
    inp3 = dict(inp, q=scaled("q", 9), k=scaled("k", -9))
    dq, dk, dv = run_fwd_bwd(fa, inp3, True, s)
    assert np.array_equal(dq, base[0] * 2.0 ** -9) and np.array_equal(dk, base[1] * 2.0 ** 9)
    assert np.array_equal(dv, base[2])


def test_stages_equal_full_call(fa):
    """preprocess, dkdv, dq called one by one give flash_attn_bwd's bits."""
    import torch
    inp = ai.make_case(1, 4, 2, 300, 64, seed=23)
    say("bwd stages vs full call")
    q, k, v, do = to_dev(inp["q"]), to_dev(inp["k"]), to_dev(inp["v"]), to_dev(inp["do"])
    o, lse = fa.fwd(q, k, v, causal=True, scale=0.125)
    dq, dk, dv = fa.bwd(q, k, v, o, lse, do, causal=True, scale=0.125)
    dq2, dk2, dv2 = torch.empty_like(dq), torch.empty_like(dk), torch.empty_like(dv)
    ws_bytes = fa.bwd_workspace_size(1, 4, 2, 300, 64, 1)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=q.device)
    stream = torch.cuda.current_stream().cuda_stream
    for stage in range(3):
        st = fa.bwd_stage_raw(stage, q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                              do.data_ptr(), dq2.data_ptr(), dk2.data_ptr(), dv2.data_ptr(), 1, 4, 2, 300, 64, 1,
                              0.125, ws.data_ptr(), ws_bytes, stream)
        assert st == 0
    torch.cuda.synchronize()
    for x, y in ((dq, dq2), (dk, dk2), (dv, dv2)):
        assert torch.equal(x.view(torch.int16), y.view(torch.int16))


# ------------------------------------------------------------------ full-size workloads
def group_bwd_check(fa, w, inp, groups):
    """Full GPU forward + backward at the workload's size, then every element of
    O, LSE, dQ, dK and dV of the listed (b, kv-head) groups against the oracle's
    full backward of those groups (every row, every key)."""
    import torch
    say(f"bwd workload {w.name} (full size on GPU; oracle on groups {groups}, all rows and keys)")
    q, k, v, do = to_dev(inp["q"]), to_dev(inp["k"]), to_dev(inp["v"]), to_dev(inp["do"])
    o, lse = fa.fwd(q, k, v, causal=w.causal, scale=w.scale)
    dq, dk, dv = fa.bwd(q, k, v, o, lse, do, causal=w.causal, scale=w.scale)
    torch.cuda.synchronize()
    G = w.G
    for (b, h) in groups:
        hs = slice(h * G, (h + 1) * G)
        got = dict(o=from_dev_bf16(o[b:b + 1, hs]), lse=lse[b:b + 1, hs].double().cpu().numpy(),
                   dq=from_dev_bf16(dq[b:b + 1, hs]), dk=from_dev_bf16(dk[b:b + 1, h:h + 1]),
                   dv=from_dev_bf16(dv[b:b + 1, h:h + 1]))
        say(f"oracle backward of group {(b, h)}")
        ref = oracle.bwd(f64(inp["q"][b:b + 1, hs]), f64(inp["k"][b:b + 1, h:h + 1]),
                         f64(inp["v"][b:b + 1, h:h + 1]), f64(inp["do"][b:b + 1, hs]), w.causal, w.scale)
        check_outputs(f"{w.name} group {(b, h)}", {n: (got[n], ref[n]) for n in got},
                      dict(o=TOL_O, lse=TOL_LSE, dq=TOL_GRAD, dk=TOL_GRAD, dv=TOL_GRAD))


def seeded_groups(w, count):
    rng = ai.rng_for(w.cfg_id, 7)
    flat = rng.choice(w.B * w.Hkv, size=min(count, w.B * w.Hkv), replace=False)
    return [(int(f) // w.Hkv, int(f) % w.Hkv) for f in sorted(flat)]


def test_workload_spiky8k(fa):
    """N=8192, d=128, causal, K rows x4 at 5% of positions: every element of
    every output of all 32 heads (forward O and LSE included) against the
    oracle's full backward."""
    import torch
    w = ai.WORKLOADS["spiky8k"]
    inp = ai.make_inputs(w)
    say(f"bwd workload {w.name} (full size, every head, row and key)")
    q, k, v, do = to_dev(inp["q"]), to_dev(inp["k"]), to_dev(inp["v"]), to_dev(inp["do"])
    o, lse = fa.fwd(q, k, v, causal=w.causal, scale=w.scale)
    dq, dk, dv = fa.bwd(q, k, v, o, lse, do, causal=w.causal, scale=w.scale)
    torch.cuda.synchronize()
    got = dict(o=from_dev_bf16(o), lse=lse.double().cpu().numpy(), dq=from_dev_bf16(dq),
               dk=from_dev_bf16(dk), dv=from_dev_bf16(dv))
    del q, k, v, do, o, lse, dq, dk, dv
    say("oracle backward of all 32 heads")
    ref = oracle.bwd(f64(inp["q"]), f64(inp["k"]), f64(inp["v"]), f64(inp["do"]), w.causal, w.scale)
    check_outputs(w.name, {n: (got[n], ref[n]) for n in got},
                  dict(o=TOL_O, lse=TOL_LSE, dq=TOL_GRAD, dk=TOL_GRAD, dv=TOL_GRAD))


def test_workload_gqa16k(fa):
    """B=2, Hq=32, Hkv=8, N=16384, d=128, causal: two seeded (b, kv-head) groups
    (8 of the 32 query heads' rows, 2 of the 8 K/V heads' keys) on every
    element of O, LSE, dQ, dK and dV."""
    w = ai.WORKLOADS["gqa16k"]
    inp = ai.make_inputs(w)
    group_bwd_check(fa, w, inp, seeded_groups(w, w.oracle_groups))


@pytest.mark.parametrize("d", [64, 128])
def test_dynamic_range_of_the_fp16_operands(fa, d):
    """The backward's products take fp16 operands scaled by one power of two per
    tensor (and one for dS, from the bound 2 d max|dO| max|V|). Four heads see
    the same Q, K and V, and dO times 2^0, 2^-8, 2^-24 and 2^-40: a dynamic range
    of 2^40 inside one dO tensor, beyond fp16's. The gradients are linear in dO,
    so head h's gradients are 2^e_h times head 0's.
      * Every head meets the absolute bound against the oracle.
      * Heads at 2^0 and 2^-8, divided by their factor, meet it too: relative
        accuracy holds there.
      * Further down, dS falls below fp16's normal range (2^-14 after its scale)
        and then below its subnormals, so dQ and dK of those heads lose their
        relative accuracy (their absolute error stays below 2^-20); dV, whose
        operands are P and dO alone, keeps it at 2^-24. The relative errors are
        printed."""
    import torch
    Hq = 4
    exps = (0, -8, -24, -40)
    base = ai.make_case(1, 1, 1, 640, d, seed=3100 + d)
    inp = {n: np.repeat(base[n], Hq, axis=1) for n in ("q", "k", "v", "do")}
    do = torch.from_numpy(f64(inp["do"]))
    for h, e in enumerate(exps):
        do[:, h] *= 2.0 ** e
    inp["do"] = do.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(f64(inp["do"][:, 1]) * 2.0 ** 8, f64(base["do"][:, 0])), "power-of-two scaling is exact"
    s = 1.0 / math.sqrt(d)
    say(f"bwd dynamic range of dO over heads d={d}")
    dq, dk, dv = run_fwd_bwd(fa, inp, True, s)
    ref = oracle.bwd(f64(inp["q"]), f64(inp["k"]), f64(inp["v"]), f64(inp["do"]), True, s)
    check_outputs(f"dynamic range d={d} (absolute, all heads)",
                  {"dq": (dq, ref["dq"]), "dk": (dk, ref["dk"]), "dv": (dv, ref["dv"])},
                  dict(dq=TOL_GRAD, dk=TOL_GRAD, dv=TOL_GRAD))
    rel = {}
    for h, e in enumerate(exps):
        f = 2.0 ** -e
        rel[e] = {n: excess_err(g[:, h] * f, ref[n][:, h] * f)
                  for n, g in (("dq", dq), ("dk", dk), ("dv", dv))}
    say(f"error beyond rounding, each head divided by its factor: {rel}")
    for e in (0, -8):
        assert all(x <= TOL_GRAD for x in rel[e].values()), f"head at 2^{e}: {rel[e]}"
    assert np.max(np.abs(dq[:, 2:])) <= 2.0 ** -20 and np.max(np.abs(dk[:, 2:])) <= 2.0 ** -20


@pytest.mark.parametrize("d", [8, 32, 40, 96, 112])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("N", [1, 33, 129, 300])
def test_padded_headdim(fa, d, causal, N):
    """Head dimensions below 64 and 128: the preparation writes the fp16 copies
    with zero columns past d, the epilogues write d columns."""
    inp = ai.make_case(1, 2, 2, N, d, seed=6200 + N * 3 + d + int(causal))
    check_full(fa, inp, causal, 1.0 / math.sqrt(d), f"padded d={d} N={N} causal={causal}")


@pytest.mark.parametrize("d", [32, 96])
@pytest.mark.parametrize("causal", [False, True])
def test_padded_headdim_gqa(fa, d, causal):
    inp = ai.make_case(2, 8, 2, 520, d, seed=6300 + d + int(causal))
    check_full(fa, inp, causal, 1.0 / math.sqrt(d), f"padded gqa d={d} causal={causal}")


# ------------------------------------------------------------------ head dimensions up to 256
@pytest.mark.parametrize("d", [256, 136, 200])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("N", [1, 17, 64, 129, 300, 700])
def test_wide_headdim(fa, d, causal, N):
    """d above 128 runs the split gradient kernels (each half of the columns
    in its own workgroup); every element against the oracle."""
    inp = ai.make_case(1, 2, 2, N, d, seed=6400 + N * 3 + d + int(causal))
    check_full(fa, inp, causal, 1.0 / math.sqrt(d), f"wide d={d} N={N} causal={causal}")


@pytest.mark.parametrize("causal", [False, True])
def test_wide_headdim_gqa(fa, causal):
    inp = ai.make_case(2, 8, 2, 520, 256, seed=6500 + int(causal))
    check_full(fa, inp, causal, 0.0625, f"wide gqa d=256 causal={causal}")


def test_wide_headdim_large_logits(fa):
    inp = ai.make_case(1, 4, 4, 1000, 256, seed=6600, dist_scale=2.0)
    check_full(fa, inp, True, 0.2 * math.sqrt(128 / 256), "wide large logits")


def test_wide_headdim_full_size(fa):
    """d = 256 at a prefill size (B = 2, Hq = 16, Hkv = 4, N = 16384, causal):
    one seeded (b, kv-head) group, every element of O, LSE, dQ, dK and dV."""
    w = ai.WORKLOADS["gqa16k_d256"]
    inp = ai.make_inputs(w, with_grad=True)
    group_bwd_check(fa, w, inp, seeded_groups(w, 1))
