"""The 576/512 attention kernel waits for every inline-assembly LDS read before
any instruction touches its destination registers, and no VALU instruction
writes a source of an inline-assembly MFMA without wait states in between
(see asm_lds_check). Builds
the kernel's device assembly with the library's own flags (hipcc
cross-compiles gfx950 without a GPU)."""
import os
import re
import subprocess
import tempfile

import pytest

from asm_lds_check import check, kernel_lines, loads_before_first_vm_wait, mfma_hazards

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _device_asm(src):
    from paged_absorbed_mla_amd import build as b
    try:
        hipcc = b.hipcc()
    except RuntimeError:
        pytest.skip("hipcc not available")
    per_file = [f for pre, fl in b.FILE_FLAGS.items() if os.path.basename(src).startswith(pre) for f in fl]
    flags = [f for f in b.HIPCC_FLAGS if f != "-c"]
    with tempfile.TemporaryDirectory() as d:
        out = os.path.join(d, "k.s")
        r = subprocess.run([hipcc, *flags, *per_file, "--cuda-device-only", "-S", "-o", out, src],
                           capture_output=True, text=True)
        assert r.returncode == 0, r.stderr[-2000:]
        return open(out).read()


@pytest.mark.parametrize("nt", [0, 1])
@pytest.mark.parametrize("inst", ["attnm_bf16_576_512.hip", "attnm_f16_576_512.hip"])
def test_mla_kernel_lds_reads_are_waited_for(inst, nt):
    """Both copy-policy variants of the 576/512 kernel (template flag NT)."""
    asm = _device_asm(os.path.join(ROOT, "paged_absorbed_mla_amd", "csrc", "inst", inst))
    syms = re.findall(r"^(_ZN2pa15attn_mla_kernel\S*?Lb%dE\S*):" % nt, asm, re.M)
    assert syms, "kernel symbol not found"
    lines = kernel_lines(asm, syms[0])
    assert len(lines) > 1000, "kernel body not found"
    found = check(lines)
    assert not found, "\n".join(f"line {a}: {b} uses {c} of the LDS read at line {d}" for a, b, c, d in found[:10])
    hz = mfma_hazards(lines)
    assert not hz, "\n".join(f"line {a}: {b} right after {c}" for a, b, c in hz[:10])
    # 576 channels = 36 k-steps of query loads, all issued while the first two
    # KV tiles are in flight.
    n, at = loads_before_first_vm_wait(lines)
    assert n >= 36, f"only {n} query loads before the vmcnt wait at line {at}"


def test_checker_flags_a_valu_write_right_before_an_asm_mfma():
    lines = ["v_mov_b32 v5, v1", "v_mfma_f32_32x32x16_bf16 a[0:15], v[2:5], v[6:9], a[0:15]",
             "v_mov_b32 v9, v1", "s_nop 3", "v_mfma_f32_32x32x16_bf16 a[0:15], v[2:5], v[6:9], a[0:15]"]
    assert [f[0] for f in mfma_hazards(lines)] == [2]


def test_checker_flags_a_copy_before_the_wait():
    """Negative control: a register copied while its LDS read is in flight."""
    lines = ["ds_read_b128 v[2:5], v1", "ds_read_b128 v[6:9], v1", "s_waitcnt lgkmcnt(1)",
             "v_mov_b32 v10, v6", "s_waitcnt lgkmcnt(0)", "v_mov_b32 v11, v7"]
    found = check(lines)
    assert [f[0] for f in found] == [4]


def test_checker_counts_loads_before_a_vm_wait():
    lines = ["buffer_load_dwordx4 v1, s[0:3], 0 offen lds", "scratch_load_dword v0, off, off",
             "s_waitcnt vmcnt(0)", "buffer_load_dwordx4 v[4:7], v2, s[4:7], 0 offen"]
    assert loads_before_first_vm_wait(lines) == (0, 3)
    lines = [lines[0], lines[3], lines[1], lines[2]]
    assert loads_before_first_vm_wait(lines) == (1, 4)
