"""The decode kernel reads LDS fragments with inline-asm loads and waits for
them later (s_waitcnt lgkmcnt in a separate statement), so that copies of later
tiles can stay in flight across the reads. The compiler takes such a load's
output as written when the asm statement ends: it must not read, copy or reuse
a destination register before the wait retires the load. This test compiles
the decode source for gfx950 with the library's own flags and walks each
kernel's instructions in order, keeping the LDS loads not yet retired by an
s_waitcnt lgkmcnt. It fails if any instruction touches one of their
destination registers. (A first build of the 256-wide instance did so, at 350
places, and returned wrong outputs.)

CPU only: hipcc cross-compiles; nothing runs on a GPU.
"""
import os
import re
import shutil
import subprocess

import pytest

from exact_io_aware_60_amd import build as fa_build

HIPCC = fa_build.HIPCC


def _regs(text):
    out = set()
    for m in re.finditer(r"\b([va])\[(\d+):(\d+)\]|\b([va])(\d+)\b", text):
        if m.group(1):
            out.update(f"{m.group(1)}{r}" for r in range(int(m.group(2)), int(m.group(3)) + 1))
        else:
            out.add(f"{m.group(4)}{m.group(5)}")
    return out


def inflight_violations(lines):
    """(LDS loads seen, list of violations) for one kernel's instruction lines."""
    pending = []          # (line, destination registers) of loads not yet retired, in issue order
    bad, nloads = [], 0
    for i, raw in enumerate(lines):
        ins = raw.split(";")[0].strip()
        if not ins or ins.startswith(".") or ins.endswith(":"):
            continue
        op = ins.split()[0]
        wait = re.search(r"lgkmcnt\((\d+)\)", ins)
        if op == "s_waitcnt":
            if wait:
                while len(pending) > int(wait.group(1)):
                    pending.pop(0)
            continue
        args = ins[len(op):]
        used = _regs(args)
        for li, dst in pending:
            if dst & used:
                bad.append(f"{ins}  (load: {lines[li].strip()})")
        if op.startswith("ds_read") or op.startswith("ds_load"):
            pending.append((i, _regs(args.split(",")[0])))
            nloads += 1
    return nloads, bad


def kernels(asm):
    lines = asm.split("\n")
    starts = [i for i, l in enumerate(lines) if re.match(r"^_ZN\S+:", l)]
    for s in starts:
        # the next label, so a data symbol (the static scratch array) is no kernel
        nxt = next((i for i in range(s + 1, len(lines)) if re.match(r"^_ZN\S+:", lines[i])), len(lines))
        e = next((i for i in range(s, nxt) if "s_endpgm" in lines[i]), None)
        if e is None:
            continue
        yield lines[s].split(":")[0], lines[s + 1:e + 1]


@pytest.fixture(scope="module")
def decode_asm(tmp_path_factory):
    if not shutil.which(HIPCC) and not os.path.exists(HIPCC):
        pytest.skip("hipcc is not available")
    src = os.path.join(fa_build.CSRC, "fa_decode.hip")
    out = str(tmp_path_factory.mktemp("asm") / "fa_decode.s")
    cmd = [HIPCC, *fa_build.FLAGS, *fa_build.SOURCE_FLAGS.get("fa_decode.hip", []), "-x", "hip", "-S",
           "--cuda-device-only", src, "-o", out]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    with open(out) as fh:
        return fh.read()


def test_decode_inflight_loads_untouched(decode_asm):
    found = 0
    for name, lines in kernels(decode_asm):
        if "decode_split_kernel" not in name:
            continue
        found += 1
        nloads, bad = inflight_violations(lines)
        assert nloads > 0, name
        assert not bad, f"{name}: {len(bad)} instructions touch registers of LDS loads in flight, e.g. {bad[:3]}"
    assert found == 6            # d = 64, 128, 256, each with and without padded columns


def test_checker_catches_a_touched_register():
    """The walk itself: a use of a destination register before the wait is
    reported, and a wait that retires the load clears it."""
    bad_code = ["ds_read_b128 v[4:7], v1", "v_mov_b32 v9, v5", "s_waitcnt lgkmcnt(0)"]
    good_code = ["ds_read_b128 v[4:7], v1", "ds_read_b128 v[8:11], v2", "s_waitcnt lgkmcnt(1)",
                 "v_mov_b32 v12, v5", "s_waitcnt lgkmcnt(0)", "v_mov_b32 v13, v8"]
    assert len(inflight_violations(bad_code)[1]) == 1
    assert inflight_violations(good_code) == (2, [])
    # the second load is still in flight after lgkmcnt(1): touching it is reported
    early = good_code[:3] + ["v_mov_b32 v12, v9"]
    assert len(inflight_violations(early)[1]) == 1
