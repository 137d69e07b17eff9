"""Plant plausible mistakes in copies of the oracle (on the CPU) and check that
the pins catch every one of them.

Each mutant replaces one snippet of ``oracle/oracle.c``; the snippet must occur
exactly once, so an edit to the oracle that removes it fails loudly here rather
than silently weakening the check. The mutated source is compiled into a
temporary directory; the in-tree oracle is never touched.
"""
import os
import tempfile

import pytest

from oracle import Oracle
from oracle.build import SRC, compile_oracle
from tests.oracle_pins import PINS

MUTANTS = {
    "score scale dropped": ("S[j] = s * dot(qi, kh", "S[j] = dot(qi, kh"),
    "causal mask off by one": ("(int64_t)j <= pos_i", "(int64_t)j < pos_i"),
    "causal mask flipped": ("(int64_t)j <= pos_i", "(int64_t)j >= pos_i"),
    "max shift dropped": ("exp(S[j] - m)", "exp(S[j])"),
    "no normalisation": ("for (int j = 0; j < Nk; ++j) P[j] /= l;", ""),
    "O uses K for V": ("const double* vj = vh + (size_t)j * d;", "const double* vj = kh + (size_t)j * d;"),
    "LSE in log2": ("*lse_i = m + log(l);", "*lse_i = m + log2(l);"),
    "LSE drops max": ("*lse_i = m + log(l);", "*lse_i = log(l);"),
    "fwd GQA map modulo": ("const int hk = h / G;\n        const double* kh", "const int hk = h % Hkv;\n        const double* kh"),
    "window keeps one key too many": ("(int64_t)j > pos_i - window", "(int64_t)j >= pos_i - window"),
    "window ignored": ("(window <= 0 ||", "(1 ||"),
    "bwd softmax ignores window": ("attend_row(qi, kh, vh, N, d, i, causal, window, scale,", "attend_row(qi, kh, vh, N, d, i, causal, 0, scale,"),
    "fwd row position ignored": ("qpos ? qpos[i] : i, causal, window, scale, S, P,", "qpos ? qpos[i] : 0, causal, window, scale, S, P,"),
    "D uses dO.dO": ("const double Di = dot(doi, ostore, d);", "const double Di = dot(doi, doi, d);"),
    "D term dropped": ("const double dSij = P[j] * (dPij - Di);", "const double dSij = P[j] * dPij;"),
    "dS sign flipped": ("const double dSij = P[j] * (dPij - Di);", "const double dSij = P[j] * (Di - dPij);"),
    "dP uses K": ("const double dPij = dot(doi, vh + (size_t)j * d, d);", "const double dPij = dot(doi, kh + (size_t)j * d, d);"),
    "dQ uses Q": ("dqi[c] += scale * dSij * kj[c];", "dqi[c] += scale * dSij * qi[c];"),
    "dK scale dropped": ("dkj[c] += scale * dSij * qi[c];", "dkj[c] += dSij * qi[c];"),
    "dV uses dS": ("dvj[c] += P[j] * doi[c];", "dvj[c] += dSij * doi[c];"),
    "bwd KV head ignored": ("const double* kh = k + ((size_t)b * Hkv + hk) * head;", "const double* kh = k + ((size_t)b * Hkv) * head;"),
    "bwd head in group wrong": ("const int h = hk * G + g;", "const int h = hk + g * Hkv;"),
    "sampled key slot wrong": ("slot[keys[t]] = t;", "slot[keys[t]] = 0;"),
    "sampled row slot wrong": ("rslot[rows[t]] = t;", "rslot[rows[t]] = nrows - 1 - t;"),
    "stored O not rounded": ("ostore[c] = o_bf16 ? round_bf16(oi[c]) : oi[c];", "ostore[c] = oi[c];"),
    "stored O rounded to 9 bits": ("ldexp(nearbyint(ldexp(m, 8)), e - 8)", "ldexp(nearbyint(ldexp(m, 9)), e - 9)"),
    "stored O rounding truncates": ("ldexp(nearbyint(ldexp(m, 8)), e - 8)", "ldexp(trunc(ldexp(m, 8)), e - 8)"),
    "e4m3 exponent bias 8": ("ldexp(8.0 + m, e - 10)", "ldexp(8.0 + m, e - 11)"),
    "e4m3 subnormal spacing": ("ldexp((double)m, -9)", "ldexp((double)m, -10)"),
    "e4m3 encode truncates": ("double q = nearbyint(ldexp(a, 3 - ee));", "double q = floor(ldexp(a, 3 - ee));"),
    "e4m3 overflow to NaN": ("if (a >= 448.0) return sign | 0x7E;", "if (a >= 464.0) return sign | 0x7F;"),
    "e4m3 sign dropped": ("const uint8_t sign = signbit(x) ? 0x80 : 0;", "const uint8_t sign = 0;"),
    "e4m3 subnormal rounding truncates": ("return sign | (uint8_t)nearbyint(ldexp(a, 9));", "return sign | (uint8_t)trunc(ldexp(a, 9));"),
    "quantiser stores the inverse scale": ("volatile float sc = amax > 0.0f ? a / 448.0f : 1.0f;", "volatile float sc = amax > 0.0f ? 448.0f / a : 1.0f;"),
    "quantiser forgets the tiny-run factor on x": ("volatile float xs = xb[t] * up;", "volatile float xs = xb[t];"),
    "quantiser keeps the scale of the scaled-up run": ("volatile float sc_out = sc * (tiny ? 0x1p-64f : 1.0f);", "volatile float sc_out = sc;"),
    "quantiser amax of the first row": ("for (int64_t t = 0; t < cnt; ++t) {\n                const float a = fabsf(xb[t]);", "for (int64_t t = 0; t < d; ++t) {\n                const float a = fabsf(xb[t]);"),
    "bwd reduction drops a thread": ("for (int t = 0; t < nt; ++t) {\n                const double* dk_t", "for (int t = 1; t < nt; ++t) {\n                const double* dk_t"),
}


def _pins_fail(orc):
    failed = []
    for pin in PINS:
        try:
            pin(orc)
        except (AssertionError, ValueError, FloatingPointError) as e:
            failed.append((pin.__name__, str(e).splitlines()[0][:120]))
    return failed


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name):
    old, new = MUTANTS[name]
    src = open(SRC).read()
    assert src.count(old) == 1, f"mutation anchor for '{name}' not found exactly once"
    with tempfile.TemporaryDirectory() as tmp:
        path = os.path.join(tmp, "oracle_mutant.c")
        with open(path, "w") as f:
            f.write(src.replace(old, new))
        lib = os.path.join(tmp, "liboracle_mutant.so")
        compile_oracle(path, lib)
        failed = _pins_fail(Oracle(lib))
    assert failed, f"no pin caught the planted mistake '{name}'"
