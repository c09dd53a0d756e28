"""Build check of the direct-to-LDS loads (CPU only).

The tiled GEMM and the flash-attention kernel issue their direct-to-LDS
buffer loads from inline asm that sets m0 (the LDS destination) right before
each load.  The compiler treats m0 as a register it may also use, so this
test compiles both sources to gfx950 assembly and checks that nothing else
touches m0: every textual m0 is the `s_mov_b32 m0, sN` of one such sequence
(followed by `s_nop 0` and a `buffer_load_dwordx4 ... lds`), every
direct-to-LDS load is preceded by one, and no instruction that reads m0
implicitly (message sends, relative moves, lane-id LDS ops, GWS, interpolation)
appears at all."""
import concurrent.futures as cf
import os
import re
import shutil
import subprocess
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "sparse_moe_transformer_group_amd", "csrc")
SOURCES = ["gemm_tiled.hip", "attention.hip"]
IMPLICIT_M0 = re.compile(r"\b(s_sendmsg\w*|s_movrel\w*|v_movrel\w*|\w+_addtid\w*|ds_gws\w*|"
                         r"v_interp\w*|lds_param_load\w*|lds_direct_load\w*)\b")


def hipcc():
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    pytest.skip("hipcc not available")


def device_asm(src, out_dir):
    out = os.path.join(out_dir, src + ".s")
    cmd = [hipcc(), "--offload-arch=gfx950", "-O3", "-std=c++17", "-Xclang", "-target-feature",
           "-Xclang", "-packed-fp32-ops", "--cuda-device-only", "-S",
           f"-I{os.path.join(ROOT, 'include')}", os.path.join(CSRC, src), "-o", out]
    subprocess.run(cmd, check=True, capture_output=True)
    with open(out) as f:
        return [ln.split(";")[0].strip() for ln in f]


def m0_violations(lines):
    code = [ln for ln in lines if ln and not ln.startswith((".", "#")) and not ln.endswith(":")]
    bad, sequences = [], 0
    for i, ln in enumerate(code):
        if IMPLICIT_M0.search(ln):
            bad.append(f"implicit m0 user: {ln}")
        if re.search(r"\bm0\b", ln):
            ok = (re.fullmatch(r"s_mov_b32 m0, s\d+", ln) is not None and i + 2 < len(code)
                  and code[i + 1] == "s_nop 0"
                  and re.match(r"buffer_load_dwordx4 .* offen lds$", code[i + 2]) is not None)
            if ok:
                sequences += 1
            else:
                bad.append(f"m0 outside the direct-to-LDS sequence: {ln}")
        if re.search(r"\blds$", ln) and ln.startswith(("buffer_", "global_")):
            if not (i >= 2 and re.fullmatch(r"s_mov_b32 m0, s\d+", code[i - 2])
                    and code[i - 1] == "s_nop 0"):
                bad.append(f"direct-to-LDS load without its own m0: {ln}")
    return bad, sequences


def test_m0_only_in_direct_to_lds_sequences():
    with tempfile.TemporaryDirectory() as d, cf.ThreadPoolExecutor(len(SOURCES)) as ex:
        asm = dict(zip(SOURCES, ex.map(lambda s: device_asm(s, d), SOURCES)))
    for src, lines in asm.items():
        bad, n = m0_violations(lines)
        assert n > 0, f"{src}: no direct-to-LDS sequence found"
        assert not bad, f"{src}: " + "; ".join(bad[:5])


def test_checker_flags_a_stray_m0_use():
    good = ["s_mov_b32 m0, s4", "s_nop 0", "buffer_load_dwordx4 v1, s[8:11], s5 offen lds"]
    assert m0_violations(good) == ([], 1)
    assert m0_violations(good + ["s_mov_b32 m0, -1"])[0]
    assert m0_violations(good + ["v_movrels_b32 v0, v1"])[0]
    assert m0_violations(["buffer_load_dwordx4 v1, s[8:11], s5 offen lds"])[0]
    assert m0_violations(["s_mov_b32 m0, s4", "v_add_u32 v0, v1, v2",
                          "buffer_load_dwordx4 v1, s[8:11], s5 offen lds"])[0]
