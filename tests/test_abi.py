"""The C ABI without a GPU: the library loads, exports every function the header
declares, and rejects bad arguments with the documented status before any HIP call."""
import ctypes
import os
import re
import subprocess

import pytest

import exact_io_aware_60_amd as fa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "flash_attn.h")

# plausible, 16-byte-aligned fake device addresses: validation must fail before
# any of them is touched
P = [0x10000 * (i + 1) for i in range(12)]


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(flash_attn_\w+)\s*\(", text)))


def test_header_and_binding_agree():
    assert declared_functions() == sorted(fa.EXPORTED)


def test_library_exports_every_declared_symbol():
    out = subprocess.run(["nm", "-D", "--defined-only", fa.LIB_PATH], capture_output=True, text=True,
                         check=True).stdout
    exported = set(re.findall(r"\bT (flash_attn_\w+)", out))
    for name in declared_functions():
        assert name in exported, name
        assert hasattr(fa.lib(), name)


def test_version_names_target():
    assert "gfx950" in fa.version()


def test_strerror_covers_all_codes():
    for code in (fa.FA_OK, fa.FA_ERR_NULL, fa.FA_ERR_SHAPE, fa.FA_ERR_HEADDIM, fa.FA_ERR_ALIGN,
                 fa.FA_ERR_WORKSPACE, fa.FA_ERR_HIP, fa.FA_ERR_SCALE):
        assert fa.strerror(code)
    assert fa.strerror(12345) == "unknown status"


def fwd_call(**over):
    a = dict(q=P[0], k=P[1], v=P[2], o=P[3], lse=P[4], B=1, Hq=4, Hkv=2, N=128, d=128, causal=1, scale=0.088)
    a.update(over)
    return fa.fwd_raw(a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"], a["Hq"], a["Hkv"], a["N"], a["d"],
                      a["causal"], a["scale"])


def bwd_call(**over):
    a = dict(q=P[0], k=P[1], v=P[2], o=P[3], lse=P[4], do=P[5], dq=P[6], dk=P[7], dv=P[8], B=1, Hq=4,
             Hkv=2, N=128, d=128, causal=1, scale=0.088, ws=P[9], ws_bytes=1 << 20)
    a.update(over)
    return fa.bwd_raw(a["q"], a["k"], a["v"], a["o"], a["lse"], a["do"], a["dq"], a["dk"], a["dv"], a["B"],
                      a["Hq"], a["Hkv"], a["N"], a["d"], a["causal"], a["scale"], a["ws"], a["ws_bytes"])


@pytest.mark.parametrize("name", ["q", "k", "v", "o", "lse"])
def test_fwd_null(name):
    assert fwd_call(**{name: None}) == fa.FA_ERR_NULL


@pytest.mark.parametrize("over", [dict(B=0), dict(Hq=0), dict(Hkv=0), dict(N=0), dict(N=-5), dict(Hq=6, Hkv=4),
                                  dict(B=1 << 20, Hq=1 << 10, Hkv=1 << 10, N=1 << 20)])
def test_fwd_shape(over):
    assert fwd_call(**over) == fa.FA_ERR_SHAPE


@pytest.mark.parametrize("d", [0, -8, 4, 12, 63, 129, 250, 255, 257, 264, 512])
def test_fwd_headdim(d):
    """Head dimensions are multiples of 8 from 8 to 256 in the forward passes."""
    assert fwd_call(d=d) == fa.FA_ERR_HEADDIM


@pytest.mark.parametrize("d", [8, 16, 32, 40, 64, 80, 96, 112, 128, 136, 192, 256])
def test_fwd_headdim_accepted(d):
    """Multiples of 8 up to 256 pass the head-dimension check (the next check,
    the scale, is reached); they run on the 64-, 128- or 256-wide instance."""
    assert fwd_call(d=d, scale=-1.0) == fa.FA_ERR_SCALE
    assert dec_call(d=d, scale=-1.0) == fa.FA_ERR_SCALE
    assert varlen_call(d=d, scale=-1.0) == fa.FA_ERR_SCALE


@pytest.mark.parametrize("d", [8, 16, 32, 40, 64, 80, 96, 112, 128, 136, 200, 256])
def test_bwd_headdim_accepted(d):
    assert bwd_call(d=d, scale=-1.0) == fa.FA_ERR_SCALE
    pad = 64 if d <= 64 else (128 if d <= 128 else 256)
    # the copies hold the padded width; only the reduction scratch follows d
    ws, ws_pad = fa.bwd_workspace_size(1, 4, 2, 128, d, 1), fa.bwd_workspace_size(1, 4, 2, 128, pad, 1)
    assert 0 < ws <= ws_pad and ws_pad - ws < 8192


def test_d256_every_pass():
    """d = 256 passes every entry point's shape checks (the next check, the
    scale or the alignment, is reached)."""
    assert fwd_call(d=256, scale=-1.0) == fa.FA_ERR_SCALE
    assert fwd_call(d=256, o=P[3] + 2) == fa.FA_ERR_ALIGN
    assert bwd_call(d=256, scale=-1.0) == fa.FA_ERR_SCALE
    assert dec_call(d=256, scale=-1.0) == fa.FA_ERR_SCALE
    assert varlen_call(d=256, scale=-1.0) == fa.FA_ERR_SCALE
    assert fa.bwd_workspace_size(1, 4, 2, 128, 256, 1) > fa.bwd_workspace_size(1, 4, 2, 128, 128, 1)


@pytest.mark.parametrize("scale", [-0.1, float("nan"), float("inf"), float("-inf")])
def test_fwd_scale(scale):
    assert fwd_call(scale=scale) == fa.FA_ERR_SCALE


@pytest.mark.parametrize("name", ["q", "k", "v", "o", "lse"])
def test_fwd_align(name):
    assert fwd_call(**{name: P[10] + 2}) == fa.FA_ERR_ALIGN


@pytest.mark.parametrize("name", ["q", "k", "v", "o", "lse", "do", "dq", "dk", "dv"])
def test_bwd_null(name):
    assert bwd_call(**{name: None}) == fa.FA_ERR_NULL


def test_bwd_checks():
    assert bwd_call(Hq=3, Hkv=2) == fa.FA_ERR_SHAPE
    assert bwd_call(d=100) == fa.FA_ERR_HEADDIM
    assert bwd_call(d=264) == fa.FA_ERR_HEADDIM
    assert bwd_call(scale=float("nan")) == fa.FA_ERR_SCALE
    assert bwd_call(dk=P[7] + 8) == fa.FA_ERR_ALIGN
    assert bwd_call(ws=None) == fa.FA_ERR_WORKSPACE
    need = fa.bwd_workspace_size(1, 4, 2, 128, 128, 1)
    assert bwd_call(ws_bytes=need - 1) == fa.FA_ERR_WORKSPACE
    assert bwd_call(ws=P[9] + 4, ws_bytes=need) == fa.FA_ERR_ALIGN


@pytest.mark.parametrize("B,Hq,Hkv,N,d", [(1, 1, 1, 1, 64), (4, 16, 16, 2048, 64), (2, 32, 8, 16384, 128),
                                          (1, 8, 8, 131072, 128), (3, 5, 5, 77, 128)])
def test_workspace_size(B, Hq, Hkv, N, d):
    # Per head, rows padded to Np = N rounded up to 128: D and the log2-scaled
    # LSE (fp32 per query row), fp16 copies of q, k, v and dout, transposed
    # fp16 copies of q, dout and k, and at most 16 KiB of reduction scratch plus
    # 256 bytes of constants; every array rounded up to 256 bytes
    got = fa.bwd_workspace_size(B, Hq, Hkv, N, d, 1)

    def up(x):
        return x + (-x) % 256
    Np = -(-N // 128) * 128
    rows, nq, nk = B * Hq * Np, B * Hq * Np * d, B * Hkv * Np * d
    core = 2 * up(4 * rows) + 4 * up(2 * nq) + 3 * up(2 * nk)
    assert got % 256 == 0 and core + 256 < got <= core + 256 + up(16 * 1024)


@pytest.mark.parametrize("stage", [0, 1, 2])
def test_bwd_stages_validate(stage):
    """The stage entry points take flash_attn_bwd's arguments and checks."""
    a = dict(B=1, Hq=4, Hkv=2, N=128, d=128)
    need = fa.bwd_workspace_size(1, 4, 2, 128, 128, 1)
    args = [P[0], P[1], P[2], P[3], P[4], P[5], P[6], P[7], P[8], a["B"], a["Hq"], a["Hkv"], a["N"], a["d"], 1,
            0.088, P[9], need]
    bad = list(args)
    bad[0] = None
    assert fa.bwd_stage_raw(stage, *bad) == fa.FA_ERR_NULL
    bad = list(args)
    bad[17] = need - 1
    assert fa.bwd_stage_raw(stage, *bad) == fa.FA_ERR_WORKSPACE
    bad = list(args)
    bad[13] = 84
    assert fa.bwd_stage_raw(stage, *bad) == fa.FA_ERR_HEADDIM


def test_workspace_size_rejects_bad_shapes():
    assert fa.bwd_workspace_size(1, 3, 2, 64, 128, 1) == 0
    assert fa.bwd_workspace_size(1, 4, 2, 64, 100, 1) == 0
    assert fa.bwd_workspace_size(1, 4, 2, 64, 512, 1) == 0


def dec_call(**over):
    a = dict(q=P[0], k=P[1], v=P[2], o=P[3], lse=P[4], sl=None, B=2, Hq=32, Hkv=8, Nq=1, Nk=16384, d=128,
             causal=1, scale=0.088, ws=P[9], ws_bytes=1 << 30)
    a.update(over)
    return fa.decode_raw(a["q"], a["k"], a["v"], a["o"], a["lse"], a["sl"], a["B"], a["Hq"], a["Hkv"], a["Nq"],
                         a["Nk"], a["d"], a["causal"], a["scale"], a["ws"], a["ws_bytes"])


@pytest.mark.parametrize("name", ["q", "k", "v", "o", "lse"])
def test_decode_null(name):
    assert dec_call(**{name: None}) == fa.FA_ERR_NULL


@pytest.mark.parametrize("over", [dict(B=0), dict(Hq=0), dict(Hkv=0), dict(Nq=0), dict(Nk=0), dict(Hq=6, Hkv=4),
                                  dict(Nq=5, Nk=4), dict(Nk=1 << 23), dict(Hq=1 << 20, Hkv=1, Nq=1 << 12)])
def test_decode_shape(over):
    assert dec_call(**over) == fa.FA_ERR_SHAPE


def test_decode_checks():
    assert dec_call(d=97) == fa.FA_ERR_HEADDIM
    assert dec_call(d=264) == fa.FA_ERR_HEADDIM
    assert dec_call(scale=-1.0) == fa.FA_ERR_SCALE
    assert dec_call(o=P[3] + 2) == fa.FA_ERR_ALIGN
    assert dec_call(sl=P[11] + 2) == fa.FA_ERR_ALIGN
    need = fa.decode_workspace_size(2, 32, 8, 1, 16384, 128, 1)
    assert need > 0
    assert dec_call(ws=None) == fa.FA_ERR_WORKSPACE
    assert dec_call(ws_bytes=need - 1) == fa.FA_ERR_WORKSPACE
    assert dec_call(ws=P[9] + 4, ws_bytes=need) == fa.FA_ERR_ALIGN
    assert fa.decode_raw(P[0], P[1], P[2], P[3], P[4], None, 2, 32, 8, 1, 16384, 128, 1, 0.088, P[9], 1 << 30,
                         window=-1) == fa.FA_ERR_SHAPE
    assert fa.decode_raw(P[0], P[1], P[2], P[3], P[4], None, 2, 32, 8, 1, 16384, 128, 0, 0.088, P[9], 1 << 30,
                         window=64) == fa.FA_ERR_SHAPE
    assert fa.decode_workspace_size(2, 32, 8, 1, 16384, 128, 0, 64) == 0
    # a window shrinks the ranges to the tiles it covers
    assert 0 < fa.decode_workspace_size(1, 8, 8, 1, 131072, 128, 1, 4096) < fa.decode_workspace_size(
        1, 8, 8, 1, 131072, 128, 1)
    # more query rows than keys is only an error under the causal mask
    assert fa.decode_workspace_size(1, 4, 2, 9, 8, 64, 1) == 0
    assert fa.decode_workspace_size(1, 4, 2, 9, 8, 64, 0) == 0


@pytest.mark.parametrize("B,Hq,Hkv,Nq,Nk,d", [(2, 32, 8, 1, 16384, 128), (2, 32, 8, 16, 16384, 128),
                                               (1, 8, 8, 1, 131072, 128), (1, 4, 1, 3, 1000, 64),
                                               (1, 16, 1, 20, 5000, 128)])
def test_decode_workspace_size(B, Hq, Hkv, Nq, Nk, d):
    """With R key ranges per K/V head the workspace is one fp32 logsumexp and d
    fp32 outputs per (range, query row), each array rounded up to 256 bytes;
    the ranges are whole 64-key tiles, at most one range per tile."""
    got = fa.decode_workspace_size(B, Hq, Hkv, Nq, Nk, d, 1)
    rows = B * Hq * Nq

    def up(x):
        return x + (-x) % 256
    ranges = [R for R in range(2, -(-Nk // 64) + 1) if up(4 * rows * R) + up(4 * rows * R * d) == got]
    assert len(ranges) == 1, got


def test_decode_single_range_needs_no_workspace():
    """A grid that already fills the GPU (B * Hkv >= 512 groups) reads each head
    in one range and writes the output directly."""
    assert fa.decode_workspace_size(64, 32, 8, 1, 8192, 128, 1) == 0


def varlen_call(**over):
    a = dict(q=P[0], k=P[1], v=P[2], o=P[3], lse=P[4], cu=P[5], B=4, ms=4096, total=9000, Hq=32, Hkv=8, d=128,
             causal=1, scale=0.088)
    a.update(over)
    return fa.fwd_varlen_raw(a["q"], a["k"], a["v"], a["o"], a["lse"], a["cu"], a["B"], a["ms"], a["total"],
                             a["Hq"], a["Hkv"], a["d"], a["causal"], a["scale"])


@pytest.mark.parametrize("name", ["q", "k", "v", "o", "lse", "cu"])
def test_varlen_null(name):
    assert varlen_call(**{name: None}) == fa.FA_ERR_NULL


def test_varlen_checks():
    assert varlen_call(B=0) == fa.FA_ERR_SHAPE
    assert varlen_call(ms=0) == fa.FA_ERR_SHAPE
    assert varlen_call(total=0) == fa.FA_ERR_SHAPE
    assert varlen_call(Hq=6, Hkv=4) == fa.FA_ERR_SHAPE
    assert varlen_call(d=94) == fa.FA_ERR_HEADDIM
    assert varlen_call(scale=float("nan")) == fa.FA_ERR_SCALE
    assert varlen_call(cu=P[5] + 2) == fa.FA_ERR_ALIGN
    assert varlen_call(o=P[3] + 8) == fa.FA_ERR_ALIGN


def test_window_checks():
    def call(**over):
        a = dict(q=P[0], k=P[1], v=P[2], o=P[3], lse=P[4], B=1, Hq=4, Hkv=2, N=128, d=128, W=64, scale=0.088)
        a.update(over)
        return fa.fwd_window_raw(a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"], a["Hq"], a["Hkv"], a["N"],
                                 a["d"], a["W"], a["scale"])
    assert call(q=None) == fa.FA_ERR_NULL
    assert call(W=0) == fa.FA_ERR_SHAPE
    assert call(W=-4) == fa.FA_ERR_SHAPE
    assert call(Hq=3) == fa.FA_ERR_SHAPE
    assert call(d=36) == fa.FA_ERR_HEADDIM
    assert call(scale=-1.0) == fa.FA_ERR_SCALE
    assert call(d=256, scale=-1.0) == fa.FA_ERR_SCALE
    assert call(lse=P[4] + 4) == fa.FA_ERR_ALIGN


def test_bwd_window_checks():
    need = fa.bwd_workspace_size(1, 4, 2, 128, 128, 1)
    args = [P[0], P[1], P[2], P[3], P[4], P[5], P[6], P[7], P[8], 1, 4, 2, 128, 128, 64, 0.088, P[9], need]
    bad = list(args)
    bad[14] = 0
    assert fa.bwd_window_raw(*bad) == fa.FA_ERR_SHAPE
    bad = list(args)
    bad[0] = None
    assert fa.bwd_window_raw(*bad) == fa.FA_ERR_NULL
    bad = list(args)
    bad[17] = need - 1
    assert fa.bwd_window_raw(*bad) == fa.FA_ERR_WORKSPACE


def test_bwd_varlen_checks():
    need = fa.bwd_workspace_size(1, 4, 2, 1000, 128, 1)
    args = [P[0], P[1], P[2], P[3], P[4], P[5], P[6], P[7], P[8], P[9], 3, 512, 1000, 4, 2, 128, 1, 0.088, P[10],
            need]
    bad = list(args)
    bad[9] = None
    assert fa.bwd_varlen_raw(*bad) == fa.FA_ERR_NULL
    for i in (10, 11):                                     # no sequences; max_seqlen < 1
        bad = list(args)
        bad[i] = 0
        assert fa.bwd_varlen_raw(*bad) == fa.FA_ERR_SHAPE
    bad = list(args)
    bad[16] = 0                                            # non-causal: still checked before any launch
    bad[9] = None
    assert fa.bwd_varlen_raw(*bad) == fa.FA_ERR_NULL
    bad = list(args)
    bad[9] = P[9] + 2
    assert fa.bwd_varlen_raw(*bad) == fa.FA_ERR_ALIGN
    bad = list(args)
    bad[19] = need - 1
    assert fa.bwd_varlen_raw(*bad) == fa.FA_ERR_WORKSPACE


# (B, Hq, Hkv, N, d, waves): d <= 64 takes 12-wave (384-row) workgroups when the
# rounds of one workgroup per CU (256 when no GPU is current) times rows per
# workgroup, at 0.9 for a 12-wave row, come out below those of 8 waves. d = 128
# takes 4-wave (128-row) workgroups up to 16384 rows per head, and beyond that
# when 256-row ones would be fewer than two per CU.
WAVE_CASES = [
    (2, 64, 16, 16384, 64, 12),   # 8192 vs 5504 workgroups: 32 vs 22 rounds
    (4, 16, 16, 2048, 64, 8),     # 512 vs 384: 2 rounds either way, 384-row ones take longer
    (2, 16, 16, 4096, 64, 8),
    (1, 64, 8, 4100, 64, 12),     # 1088 vs 704: 5 vs 3 rounds
    (1, 64, 8, 4100, 48, 12),     # a padded head dimension runs the d = 64 kernels
    (1, 32, 8, 16384, 64, 8),     # 2048 vs 1376: 8 vs 6 rounds, 8 * 256 * 10 < 6 * 384 * 9
    (2, 32, 8, 16384, 128, 4),    # d = 128: 4 waves up to 16384 rows per head
    (1, 8, 8, 7900, 128, 4),
    (1, 8, 8, 131072, 128, 8),    # longer rows on 4096 workgroups of 256 rows: 8 waves
    (1, 4, 4, 65536, 128, 8),     # 1024 workgroups of 256 rows: 8 waves
    (1, 1, 1, 65536, 128, 4),     # 256 < 2 per CU: 4 waves
    (1, 16, 16, 1024, 128, 4),
    (1, 16, 16, 1024, 120, 4),    # a padded head dimension runs the d = 128 kernels
    (2, 16, 4, 16384, 256, 4),    # d = 256: 4 waves
]


@pytest.mark.parametrize("B,Hq,Hkv,N,d,waves", WAVE_CASES)
def test_fwd_geometry_wave_choice(B, Hq, Hkv, N, d, waves):
    g = fa.fwd_geometry(B, Hq, Hkv, N, d)
    assert g["threads"] == 64 * waves and g["block_m"] == 32 * waves, g
    assert g["block_n"] == 64
    assert g["grid"] == B * Hq * -(-N // g["block_m"])
    assert g["lds_bytes"] == 5 * 64 * 2 * (256 if d > 128 else 128 if d > 64 else 64)


def test_fwd_geometry_checks():
    out = (ctypes.c_int * 5)(*range(5))
    assert fa.lib().flash_attn_fwd_geometry(1, 4, 2, 128, 128, 1, None) == fa.FA_ERR_NULL
    assert fa.lib().flash_attn_fwd_geometry(1, 4, 2, 128, 132, 1, out) == fa.FA_ERR_HEADDIM
    assert fa.lib().flash_attn_fwd_geometry(1, 4, 3, 128, 128, 1, out) == fa.FA_ERR_SHAPE
    assert list(out) == [0, 1, 2, 3, 4]
