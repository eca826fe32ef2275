"""Register contract of the MLA kernel, checked on the generated gfx950 code.

The MLA kernel keeps its 256 output accumulators in a0 .. a255 and touches
them only from inline asm; the compiler does not know those registers hold
live values.  If its own register allocation ever placed a value in an AGPR
(it does so when VGPR pressure passes 256), that value and the accumulators
would overwrite each other.  This compiles the kernel (hipcc cross-compiles
for gfx950 without a GPU) and checks that every AGPR access in the decode
kernels sits inside an inline-asm block, and that nothing spills to scratch.

The kernels also load q and prefetch block-table entries and row ids with
global loads written as inline asm, which the compiler's own wait insertion does not
track: the kernel's explicit vmcnt waits cover them.  The compiler must not
read or overwrite such a load's destination register (a copy, a spill) before
the next vmcnt wait, or it would see the register's old contents; the last
test checks that on the generated code.
"""
import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "cross_cu_load_amd", "csrc", "decode_mla.hip")
AGPR = re.compile(r"\bv_accvgpr_|\ba\[\d+|\ba\d+\b")


def _hipcc():
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    return None


@pytest.fixture(scope="module")
def mla_asm(tmp_path_factory):
    hipcc = _hipcc()
    if hipcc is None:
        pytest.skip("hipcc not available")
    out = tmp_path_factory.mktemp("asm") / "decode_mla.s"
    cmd = [hipcc, "-O3", "-std=c++17", "--offload-arch=gfx950", "--cuda-device-only", "-S",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-o", str(out), SRC]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    return out.read_text()


def _kernel_body(asm, sparse):
    name = f"_ZN2cc3mla17mla_decode_kernelILb{1 if sparse else 0}EE"
    start = asm.index("\n" + name) + 1
    end = asm.index(".Lfunc_end", start)
    return asm[start:end]


@pytest.mark.parametrize("sparse", [False, True])
def test_agprs_touched_only_by_inline_asm(mla_asm, sparse):
    body = _kernel_body(mla_asm, sparse)
    inside, outside = False, []
    for line in body.splitlines():
        if ";;#ASMSTART" in line:
            inside = True
            continue
        if ";;#ASMEND" in line:
            inside = False
            continue
        code = line.split(";")[0]
        if not inside and AGPR.search(code):
            outside.append(line.strip())
    assert not outside, f"{len(outside)} compiler-generated AGPR accesses, e.g. {outside[:3]}"


def test_no_scratch_and_full_agpr_reservation(mla_asm):
    for sparse in (False, True):
        name = f"_ZN2cc3mla17mla_decode_kernelILb{1 if sparse else 0}EE"
        meta = mla_asm[mla_asm.index(".name:           " + name):]
        meta = meta[:meta.index(".wavefront_size")] if ".wavefront_size" in meta else meta[:4000]
        pre = mla_asm[:mla_asm.index(".name:           " + name)]
        block = pre[pre.rindex("- .agpr_count"):]
        assert re.search(r"\.agpr_count:\s+256", block), "the kernel must reserve a0..a255"
        assert re.search(r"\.private_segment_fixed_size:\s+0\b", block + meta), "scratch spills"
        assert re.search(r"\.vgpr_spill_count:\s+0\b", block + meta), "VGPR spills"


VREG = re.compile(r"\bv\[(\d+):(\d+)\]|\bv(\d+)\b")


def _vregs(code):
    regs = set()
    for m in VREG.finditer(code):
        if m.group(3) is not None:
            regs.add(int(m.group(3)))
        else:
            regs.update(range(int(m.group(1)), int(m.group(2)) + 1))
    return regs


@pytest.mark.parametrize("sparse", [False, True])
def test_untracked_loads_untouched_until_waited(mla_asm, sparse):
    """Between an inline-asm global load (the dword prefetches and the 16-byte
    q loads) and the next vmcnt wait (in code order), no instruction outside
    inline asm names its destination VGPRs."""
    body = _kernel_body(mla_asm, sparse).splitlines()
    inside, pending, found, bad = False, {}, 0, []
    for i, line in enumerate(body):
        if ";;#ASMSTART" in line:
            inside = True
            continue
        if ";;#ASMEND" in line:
            inside = False
            continue
        code = line.split(";")[0].strip()
        if not code or code.endswith(":"):
            continue
        if "s_waitcnt" in code and "vmcnt" in code:
            pending.clear()
            continue
        if inside:
            m = re.match(r"global_load_dword(?:x4)?\s+(v\[\d+:\d+\]|v\d+),", code)
            if m:
                for r in _vregs(m.group(1)):
                    pending[r] = i
                found += 1
            continue
        hit = _vregs(code) & set(pending)
        if hit:
            bad.append(f"line {i}: {code} (load at line {pending[min(hit)]})")
    assert found > 0, "no untracked dword loads found: the check no longer sees them"
    assert not bad, "destination of an untracked load used before a vmcnt wait: " + "; ".join(bad[:3])


@pytest.mark.parametrize("sparse", [False, True])
def test_wide_asm_stores_end_with_a_wait_state(mla_asm, sparse):
    """A VMEM store of more than 8 bytes needs one wait state before a VALU
    write of its data registers.  The compiler adds it only after stores it
    generates, so every such store written as inline asm must be followed by
    an s_nop inside its own asm block."""
    body = _kernel_body(mla_asm, sparse).splitlines()
    inside, bad, found = False, [], 0
    for i, line in enumerate(body):
        if ";;#ASMSTART" in line:
            inside = True
            continue
        if ";;#ASMEND" in line:
            inside = False
            continue
        code = line.split(";")[0].strip()
        if inside and re.match(r"(global|buffer|flat)_store_dwordx[34]\b", code):
            found += 1
            nxt = body[i + 1].split(";")[0].strip() if i + 1 < len(body) else ""
            if not nxt.startswith("s_nop"):
                bad.append(f"line {i}: {code} followed by {nxt!r}")
    assert not bad, "; ".join(bad[:3])


@pytest.mark.parametrize("sparse", [False, True])
def test_score_chain_carries_no_vmcnt_wait(mla_asm, sparse):
    """The score MFMAs (the chain accumulating in VGPRs) must not wait on
    vector memory: q, page and row-id loads are covered by the wait at the top
    of the step, and the tile's own transfers land before it.  A compiler that
    tracked a q load again would put vmcnt(N) waits in front of them (it did,
    with N counting down to the transfers in flight, before q was loaded
    untracked)."""
    lines = _kernel_body(mla_asm, sparse).splitlines()
    chain, waited = 0, []
    for i, line in enumerate(lines):
        if re.search(r"v_mfma_f32_32x32x16_bf16 v\[", line):
            chain += 1
            for j in range(i - 1, max(0, i - 4), -1):
                if "s_waitcnt" in lines[j]:
                    if "vmcnt" in lines[j]:
                        waited.append(f"line {j}: {lines[j].strip()}")
                    break
    assert chain >= 36, "the score chain's MFMAs were not found"
    assert not waited, "vmcnt waits in front of score MFMAs: " + "; ".join(waited[:3])
