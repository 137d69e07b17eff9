"""Helpers for the GPU parity tests: move seeded bf16 inputs to the device, run
the HIP library, and compare against the fp64 oracle."""
from __future__ import annotations

import sys

import numpy as np

import attn_inputs as ai


def say(msg: str) -> None:
    """Name the case before a GPU step, flushed, so a failing run shows where it was."""
    print(f"[gpu-case] {msg}", flush=True)
    sys.stdout.flush()


def to_dev(bits: np.ndarray):
    import torch
    t = torch.from_numpy(np.ascontiguousarray(bits, dtype=np.uint16).view(np.int16))
    return t.view(torch.bfloat16).cuda()


def from_dev_bf16(t) -> np.ndarray:
    """bf16 device tensor -> exact float64 numpy array."""
    import torch
    bits = t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
    return ai.bf16_bits_to_f64(bits)


def from_dev_f32(t) -> np.ndarray:
    return t.detach().cpu().numpy().astype(np.float64)


def f64(bits: np.ndarray) -> np.ndarray:
    return ai.bf16_bits_to_f64(bits)


def max_err(a, b) -> float:
    a, b = np.asarray(a, np.float64), np.asarray(b, np.float64)
    assert a.shape == b.shape, (a.shape, b.shape)
    if a.size == 0:
        return 0.0
    assert np.all(np.isfinite(a)), "non-finite values in the GPU result"
    return float(np.max(np.abs(a - b)))


def bf16_half_ulp(x) -> np.ndarray:
    """Half the spacing of the bf16 grid at |x| (8 significant bits: 2^(e-8) in [2^e, 2^(e+1)))."""
    ax = np.maximum(np.abs(np.asarray(x, np.float64)), 2.0 ** -126)
    return np.exp2(np.floor(np.log2(ax)) - 8)


def excess_err(gpu, ref) -> float:
    """Max over elements of |gpu - ref| minus the rounding to the bf16 output grid.

    A bf16 output can be no closer to the exact value than half a bf16 ulp, which
    is 0.0156 at |x| in [4, 8). The arithmetic tolerances below are therefore
    applied on top of that rounding."""
    gpu, ref = np.asarray(gpu, np.float64), np.asarray(ref, np.float64)
    assert gpu.shape == ref.shape, (gpu.shape, ref.shape)
    if gpu.size == 0:
        return 0.0
    assert np.all(np.isfinite(gpu)), "non-finite values in the GPU result"
    return float(np.max(np.abs(gpu - ref) - bf16_half_ulp(ref)))


def report(gpu, ref) -> str:
    """Both error figures of one output: the plain max abs error and the error
    beyond the bf16 output rounding (the quantity the tolerance applies to)."""
    return f"max|gpu-ref| {max_err(gpu, ref):.3e}, beyond rounding {excess_err(gpu, ref):.3e}"


def check_outputs(tag: str, pairs: dict, tol: dict) -> dict:
    """Compare several outputs at once. ``pairs`` maps a name to (gpu, ref);
    ``tol`` maps it to its bound. The LSE ("lse" in the name) is fp32 and is
    compared plainly; bf16 outputs beyond their rounding. The assertion message
    carries both figures of every output, so a failure shows how much of the
    margin the rounding allowance took."""
    errs, lines = {}, []
    for name, (g, r) in pairs.items():
        plain = max_err(g, r)
        errs[name] = plain if "lse" in name else excess_err(g, r)
        lines.append(f"{name}: max|gpu-ref| {plain:.3e}" + ("" if "lse" in name else
                                                             f", beyond rounding {errs[name]:.3e}"))
    say(f"{tag}: " + "; ".join(lines))
    bad = [n for n, e in errs.items() if not e <= tol[n]]
    assert not bad, f"{tag}: " + "; ".join(lines)
    return errs


# Tolerances for bf16 inputs/outputs with fp32 accumulation: max abs error beyond
# the bf16 output rounding for O and the gradients; plain max abs error for the
# fp32 LSE.
TOL_O = 1e-2
TOL_LSE = 1e-3
TOL_GRAD = 2e-2
