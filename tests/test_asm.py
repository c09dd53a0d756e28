"""Build checks on the kernels' gfx950 assembly (CPU only).

Direct-to-LDS loads.  The tiled GEMM and the flash-attention kernel issue their direct-to-LDS
buffer loads from inline asm that sets m0 (the LDS destination) right before
each load.  The compiler treats m0 as a register it may also use, so this
test compiles both sources to gfx950 assembly and checks that nothing else
touches m0: every textual m0 is the `s_mov_b32 m0, sN` of one such sequence
(followed by `s_nop 0` and a `buffer_load_dwordx4 ... lds`), every
direct-to-LDS load is preceded by one, and no instruction that reads m0
implicitly (message sends, relative moves, lane-id LDS ops, GWS, interpolation)
appears at all.

Register spills.  The tiled GEMM's gate/up instantiations spill a few
registers around the SwiGLU epilogue, where a tile's 2 x 320 accumulators per
lane meet the next tile's coordinates.  A spill reload is a vector-memory
load the compiler waits on with a full count, so one inside a k-loop would
stall every step behind the direct-to-LDS prefetches in flight.  The check
finds each innermost loop (a backward branch with no other loop inside) that
issues MFMAs, in every kernel of the GEMM and attention sources, and asserts
that no scratch access lies inside one.

Occupancy of the streaming GEMM.  At decode and verify sizes the streaming
kernel keeps one 8 KB step of weight loads in flight per wave and relies on
two waves per SIMD (8 per CU, 64 KB in flight: the per-CU optimum of the
vector-load path; 32 KB streams 10-13% slower).  Its instantiations for one or
two 16-token tiles must therefore fit 256 registers (arch + accumulation)
per lane, read from the code object metadata (`.vgpr_count`)."""
import concurrent.futures as cf
import os
import re
import shutil
import subprocess
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "sparse_moe_transformer_group_amd", "csrc")
M0_SOURCES = ["gemm_tiled.hip", "attention.hip"]
SOURCES = ["gemm_tiled.hip", "gemm_stream.hip", "attention.hip"]
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


@pytest.fixture(scope="module")
def asm():
    with tempfile.TemporaryDirectory() as d, cf.ThreadPoolExecutor(len(SOURCES)) as ex:
        return dict(zip(SOURCES, ex.map(lambda s: device_asm(s, d), SOURCES)))


def functions(lines):
    """Kernel name -> its body, from the label to its .Lfunc_end marker."""
    out, name = {}, None
    for ln in lines:
        m = re.fullmatch(r"(_Z\w+):", ln)
        if m:
            name, out[m.group(1)] = m.group(1), []
        elif name and ln.startswith(".Lfunc_end"):
            name = None
        elif name:
            out[name].append(ln)
    return out


def scratch_in_mfma_loops(body):
    """(innermost MFMA loops, scratch accesses, scratch accesses inside those loops)."""
    label = {m.group(1): i for i, ln in enumerate(body)
             if (m := re.fullmatch(r"(\.LBB\d+_\d+):", ln))}
    loops = [(label[m.group(1)], i) for i, ln in enumerate(body)
             if (m := re.fullmatch(r"s_c?branch\w*\s+(\.LBB\d+_\d+)", ln)) and label[m.group(1)] < i]
    inner = [(a, b) for a, b in loops
             if not any((c, d) != (a, b) and a <= c and d <= b for c, d in loops)]
    mfma = [(a, b) for a, b in inner if any(body[j].startswith("v_mfma") for j in range(a, b))]
    scratch = [i for i, ln in enumerate(body) if ln.startswith("scratch_")]
    inside = [i for i in scratch if any(a <= i <= b for a, b in mfma)]
    return mfma, scratch, inside


def test_m0_only_in_direct_to_lds_sequences(asm):
    for src in M0_SOURCES:
        bad, n = m0_violations(asm[src])
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


def test_no_spill_access_inside_mfma_loops(asm):
    for src, lines in asm.items():
        kernels = functions(lines)
        assert kernels, f"{src}: no kernel found"
        with_loops = 0
        for name, body in kernels.items():
            mfma, scratch, inside = scratch_in_mfma_loops(body)
            with_loops += bool(mfma)
            assert not inside, (f"{src} {name}: {len(inside)} of {len(scratch)} scratch accesses "
                                f"inside MFMA loops: {[body[i] for i in inside[:3]]}")
        assert with_loops, f"{src}: no MFMA loop found"


def test_loop_checker_flags_a_spill_in_a_loop():
    body = ["s_load_dword s0, s[0:1], 0x0", ".LBB0_1:", "v_mfma_f32_16x16x32_bf16 v[0:3], v[4:7], v[8:11], v[0:3]",
            "scratch_load_dword v12, off, s33", "s_cbranch_scc1 .LBB0_1", "scratch_store_dword off, v12, s33"]
    mfma, scratch, inside = scratch_in_mfma_loops(body)
    assert (mfma, scratch, inside) == ([(1, 4)], [3, 5], [3])
    # an outer loop around it does not count; its own scratch access is outside the inner loop
    outer = [".LBB0_0:"] + body + ["s_branch .LBB0_0"]
    assert scratch_in_mfma_loops(outer)[2] == [4]
    assert functions(["_ZN1k1fEv:", "v_nop", ".Lfunc_end0:", "_ZN1k1gEv:", "s_endpgm", ".Lfunc_end1:"]) == \
        {"_ZN1k1fEv": ["v_nop"], "_ZN1k1gEv": ["s_endpgm"]}


def register_counts(lines):
    """Kernel name -> .vgpr_count (arch + accumulation registers) from the
    code object metadata; entries there start with '- .'."""
    out, entry = {}, {}
    for ln in lines:
        if ln.startswith("- ."):
            entry = {}
        m = re.fullmatch(r"-?\s*\.(name|vgpr_count):\s+(\S+)", ln)
        if m:
            entry[m.group(1)] = m.group(2)
            if "name" in entry and "vgpr_count" in entry:
                out[entry["name"]] = int(entry["vgpr_count"])
    return out


def test_stream_kernels_keep_two_waves_per_simd(asm):
    regs = register_counts(asm["gemm_stream.hip"])
    stream = {n: v for n, v in regs.items() if "grouped_stream_kernel" in n}
    assert len(stream) >= 12, sorted(regs)
    # template arguments <MAT, RB, MT, W8>: MT is the third
    small = {n: v for n, v in stream.items()
             if re.search(r"grouped_stream_kernelILi\d+ELi\d+ELi([12])E", n)}
    assert len(small) >= 8, sorted(stream)
    too_big = {n: v for n, v in small.items() if v > 256}
    assert not too_big, f"fewer than two waves per SIMD: {too_big}"


def test_register_count_parser():
    meta = ["- .agpr_count:     8", ".name:           _ZN4beam1kILi1EEEv", ".vgpr_count:     196",
            "- .agpr_count:     0", ".vgpr_count:     40", ".name:           _ZN4beam1kILi2EEEv"]
    assert register_counts(meta) == {"_ZN4beam1kILi1EEEv": 196, "_ZN4beam1kILi2EEEv": 40}
