"""flash_attn_decode_noalloc: the decode entry point for callers that cannot
allocate (its partial results live in a static per-GPU scratch array). It runs
the same kernels as flash_attn_decode, so its outputs must equal that entry
point's bit for bit; two calls in a row, the second smaller, check that the
shared scratch carries nothing from one call into the next. The oracle bound
(O within 1e-2 beyond the bf16 output rounding, LSE within 1e-3) is checked
as well."""
import math

import numpy as np
import pytest

import attn_inputs as ai
import oracle
from tests.gpu_util import TOL_LSE, TOL_O, check_outputs, f64, from_dev_bf16, say, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def fa():
    import torch
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a GPU")
    import exact_io_aware_60_amd as fa
    fa.lib()
    return fa


def _run_both(fa, B, Hq, Hkv, Nq, Nk, d, causal, seed, seqlens=None, window=0):
    import torch
    inp = ai.make_decode_case(B, Hq, Hkv, Nq, Nk, d, seed=seed)
    q, k, v = to_dev(inp["q"]), to_dev(inp["k"]), to_dev(inp["v"])
    sl = None if seqlens is None else torch.as_tensor(np.asarray(seqlens, np.int32), device=q.device)
    scale = 1.0 / math.sqrt(d)
    ws = fa.decode_workspace_size(B, Hq, Hkv, Nq, Nk, d, causal, window)
    assert 0 < ws <= fa.decode_noalloc_max_bytes(), "the case must split its keys and fit the scratch"
    say(f"decode_noalloc B={B} Hq={Hq} Hkv={Hkv} Nq={Nq} Nk={Nk} d={d} causal={causal} ws={ws}")
    o_ref, l_ref = fa.decode(q, k, v, causal=causal, scale=scale, seqlens_k=sl, window=window)
    o = torch.full_like(q, float("nan"))
    lse = torch.full((B, Hq, Nq), float("nan"), dtype=torch.float32, device=q.device)
    torch.cuda.synchronize()
    free0, _ = torch.cuda.mem_get_info()
    fa.decode_noalloc(q, k, v, o, lse, causal=causal, scale=scale, seqlens_k=sl, window=window)
    torch.cuda.synchronize()
    free1, _ = torch.cuda.mem_get_info()
    assert free1 == free0, "the no-allocation decode changed free device memory"
    assert torch.equal(o.view(torch.int16), o_ref.view(torch.int16)), "O differs from flash_attn_decode"
    assert torch.equal(lse.view(torch.int32), l_ref.view(torch.int32)), "LSE differs from flash_attn_decode"
    L = np.full(B, Nk) if seqlens is None else np.clip(np.asarray(seqlens), 0, Nk)
    for b in range(B):
        pos = L[b] - Nq + np.arange(Nq, dtype=np.int64) if causal else None
        ro, rl = oracle.fwd(f64(inp["q"][b:b + 1]), f64(inp["k"][b:b + 1, :, :L[b]]),
                            f64(inp["v"][b:b + 1, :, :L[b]]), causal, scale, qpos=pos, window=window)
        check_outputs(f"decode_noalloc entry {b}", {"o": (from_dev_bf16(o[b:b + 1]), ro),
                                                   "lse": (lse[b:b + 1].double().cpu().numpy(), rl)},
                      dict(o=TOL_O, lse=TOL_LSE))


@pytest.mark.parametrize("d", [64, 128, 256])
def test_two_calls_second_smaller(fa, d):
    """A large split decode, then a smaller one on the same scratch."""
    _run_both(fa, 2, 16, 4, 4, 3000, d, True, seed=7100 + d)
    _run_both(fa, 1, 8, 2, 1, 700, d, True, seed=7200 + d)


def test_seqlens_and_window(fa):
    _run_both(fa, 3, 8, 2, 2, 2048, 128, True, seed=7300, seqlens=[2048, 5, 1300])
    _run_both(fa, 2, 8, 8, 3, 1500, 128, True, seed=7301, window=200)
    _run_both(fa, 1, 4, 1, 5, 600, 64, False, seed=7302)


def test_rejects_a_plan_beyond_the_scratch(fa):
    """128 query rows per K/V head at d = 256 over one K/V head need about
    34 MB of partial results, more than the 32 MiB array: FA_ERR_SCRATCH, and
    nothing is written."""
    import torch
    B, Hq, Hkv, Nq, Nk, d = 1, 128, 1, 1, 32768, 256
    need = fa.decode_workspace_size(B, Hq, Hkv, Nq, Nk, d, True)
    assert need > fa.decode_noalloc_max_bytes()
    q = torch.zeros((B, Hq, Nq, d), dtype=torch.bfloat16, device="cuda")
    k = torch.zeros((B, Hkv, Nk, d), dtype=torch.bfloat16, device="cuda")
    o = torch.full_like(q, 7.0)
    lse = torch.full((B, Hq, Nq), 7.0, dtype=torch.float32, device="cuda")
    st = fa.decode_noalloc_raw(q.data_ptr(), k.data_ptr(), k.data_ptr(), o.data_ptr(), lse.data_ptr(), None, B, Hq,
                               Hkv, Nq, Nk, d, True, 0.0625)
    torch.cuda.synchronize()
    assert st == fa.FA_ERR_SCRATCH, st
    assert "scratch" in fa.strerror(st)
    assert bool((o == 7.0).all()) and bool((lse == 7.0).all()), "a rejected call wrote its outputs"
