"""Code-generation guard for the grouped GEMM (host only, no GPU).

The k-loop of every k_gemm instance streams its stages with
global_load_lds_dwordx4 and counts them with vmcnt. A register spilled into
that loop reloads from scratch memory, whose load shares vmcnt with the DMA:
the compiler then waits for vmcnt(0) right after the reload and drains the
whole ring every stage (the copying output projection ran 25-30% slower when
one fragment offset spilled). This test compiles gemm.hip for gfx950 to
assembly and checks that no instance touches scratch between its first and
last MFMA. Spills in the item set-up and the epilogue are allowed.
"""
import os
import re
import shutil
import subprocess

import pytest

from combine_overlap_amd import build as B


def _kernel_bodies(asm: str):
    for m in re.finditer(r"^(_Z\S*k_gemm\S*):\s*;.*?^\.Lfunc_end", asm, re.S | re.M):
        yield m.group(1), m.group(0).splitlines()


def mfma_region_scratch(asm: str):
    """{kernel symbol: (MFMA count, scratch accesses between the first and last MFMA)}."""
    out = {}
    for name, lines in _kernel_bodies(asm):
        code = [l.split(";")[0].strip() for l in lines]
        mf = [i for i, l in enumerate(code) if l.startswith("v_mfma")]
        sc = [i for i, l in enumerate(code) if l.startswith("scratch_")]
        inside = [i for i in sc if mf and mf[0] <= i <= mf[-1]]
        out[name] = (len(mf), len(inside))
    return out


def test_region_scan_finds_a_planted_reload():
    # the scanner itself, on a hand-written listing: a reload between two MFMAs
    asm = "\n".join([
        "_ZN3moe6k_gemmILi1EEEvNS_8GemmArgsE: ; @x",
        "  scratch_store_dword off, v1, off ; set-up spill",
        "  v_mfma_f32_16x16x32_bf16 v[0:3], v[4:7], v[8:11], v[0:3]",
        "  scratch_load_dword v2, off, off offset:4 ; 4-byte Folded Reload",
        "  v_mfma_f32_16x16x32_bf16 v[0:3], v[4:7], v[8:11], v[0:3]",
        "  scratch_load_dword v3, off, off ; epilogue",
        ".Lfunc_end0:",
    ])
    assert mfma_region_scratch(asm) == {"_ZN3moe6k_gemmILi1EEEvNS_8GemmArgsE": (2, 1)}


@pytest.mark.skipif(shutil.which(B.HIPCC) is None and not os.path.exists(B.HIPCC), reason="hipcc not found")
def test_no_scratch_access_inside_any_gemm_k_loop(tmp_path):
    out = tmp_path / "gemm.s"
    flags = [f for f in B.HIP_FLAGS if f != "-fPIC"]
    cmd = [B.HIPCC, *flags, "--cuda-device-only", "-S", os.path.join(B.CSRC, "gemm.hip"), "-o", str(out)]
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    assert r.returncode == 0, r.stdout[-2000:]
    regions = mfma_region_scratch(out.read_text())
    assert len(regions) >= 6, sorted(regions)
    for name, (n_mfma, n_scratch) in regions.items():
        assert n_mfma > 0, name
        assert n_scratch == 0, f"{name}: {n_scratch} scratch accesses inside the MFMA loop"
