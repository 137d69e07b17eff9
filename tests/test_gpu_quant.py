"""GPU parity of the E4M3 block quantiser against the oracle's quantiser.

The codes are bytes, so the comparison is bit-exact: codes and fp32 scales
must equal what the oracle computes from the same bf16 values (held exactly in
float32). The format and the fp32 steps follow the OCP E4M3 definition with one
scale per run of rows (FlashAttention-3's FP8 block scaling, mlapandio
"FlashAttention: IO-aware exact attention", Generations).
"""
import numpy as np
import pytest

import oracle
from tests.gpu_util import say

pytestmark = pytest.mark.gpu


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

CASES = [  # (BH, N, d, rows)
    (1, 1, 8, 1),
    (3, 300, 64, 128),
    (2, 257, 128, 64),
    (4, 1000, 256, 128),
    (2, 129, 128, 7),
    (1, 4100, 128, 100000),
    (5, 33, 24, 16),
]


def _input(BH, N, d, seed):
    import torch
    g = torch.Generator().manual_seed(seed)
    x = torch.randn((BH, N, d), generator=g) * torch.exp(torch.randn((BH, 1, 1), generator=g) * 3)
    x = x.to(torch.bfloat16)
    if N > 10:
        x[0, :min(N, 7)] = 0.0                       # zeros (a whole run when rows <= 7)
        x[-1, N // 2, d - 1] = 3e4                   # an outlier: many subnormal codes in its run
        x[-1, N // 3, 0] = -0.0
    return x


def _compare(fa, orc, x, rows):
    import torch
    codes, scales = fa.quantize_e4m3(x.cuda(), rows)
    torch.cuda.synchronize()
    x32 = x.float().numpy()
    want_c, want_s = orc.quantize_e4m3(x32[None], rows)
    got_c = codes.cpu().numpy()
    got_s = scales.cpu().numpy()
    bad = np.flatnonzero(got_c.reshape(-1) != want_c.reshape(-1))
    assert bad.size == 0, f"{bad.size} codes differ, first at {bad[:5]}: {got_c.reshape(-1)[bad[:5]]} vs {want_c.reshape(-1)[bad[:5]]}"
    assert np.array_equal(got_s.view(np.uint32), want_s[0].view(np.uint32)), "scales differ"
    return got_c


@pytest.mark.parametrize("BH,N,d,rows", CASES)
def test_quantize_matches_oracle(fa, orc, BH, N, d, rows):
    say(f"quantize_e4m3 BH={BH} N={N} d={d} rows={rows}")
    x = _input(BH, N, d, seed=BH * 7919 + N * 31 + d + rows)
    c = _compare(fa, orc, x, rows)
    assert not np.any((c & 0x7F) == 0x7F), "a NaN code was written"


@pytest.mark.parametrize("exp", [-64, -70, -100, -120, -126, -133])
def test_quantize_tiny_runs(fa, orc, exp):
    """Runs whose max is near or below 2^-64, where 448 / amax overflows fp32
    unless the run is scaled up first, down to bf16 subnormals (2^-133): codes
    and scales bit-exact with the oracle, no NaN code, the run's max at 448."""
    import torch
    say(f"quantize_e4m3 tiny runs 2^{exp}")
    g = torch.Generator().manual_seed(900 + (-exp))
    x = (torch.randn((3, 48, 64), generator=g) * 2.0 ** exp).to(torch.bfloat16)
    x[1, :16] = 0.0                                   # an all-zero run
    x[2, 32:] = (torch.randn((16, 64), generator=g) * 2.0 ** min(exp + 40, 0)).to(torch.bfloat16)
    c = _compare(fa, orc, x, 16)
    assert not np.any((c & 0x7F) == 0x7F), "a NaN code was written"
    mags = x.float().abs().numpy().reshape(3, -1, 16 * 64)
    codes = c.reshape(3, -1, 16 * 64)
    for bh in range(3):
        for r in range(mags.shape[1]):
            if mags[bh, r].max() > 0:
                assert np.all(codes[bh, r][mags[bh, r] == mags[bh, r].max()] & 0x7F == 0x7E)


def test_quantize_full_size_q_of_gqa16k(fa, orc):
    """Q of the gqa16k workload (B = 2, Hq = 32, N = 16384, d = 128), 128-row runs, every code."""
    import torch
    say("quantize_e4m3 full size [64, 16384, 128]")
    g = torch.Generator().manual_seed(20261)
    x = torch.randn((64, 16384, 128), generator=g).to(torch.bfloat16)
    _compare(fa, orc, x, 128)


def test_quantize_rejects_bad_arguments(fa):
    import torch
    x = torch.zeros((2, 64, 64), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(fa.FlashAttnError):
        fa.quantize_e4m3(x, 0)
    with pytest.raises(fa.FlashAttnError):
        fa.quantize_e4m3(torch.zeros((2, 64, 12), dtype=torch.bfloat16, device="cuda"), 64)
