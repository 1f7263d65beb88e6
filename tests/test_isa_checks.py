"""Checks on the gfx950 assembly of the HIP library (CPU only: hipcc
cross-compiles the device code to text).

- No packed-fp32 instruction (v_pk_add/mul/fma_f32) is emitted: the build
  disables the feature.
- No scalar-cache write (s_store*, s_buffer_store*, s_atomic*, s_buffer_atomic*,
  s_dcache_wb*, s_dcache_discard*) is emitted.
- No s_cselect reads an SCC left by an arithmetic instruction while a v_cmp
  sits between the two: the signature of the stale-SCC miscompile that
  uniform 64-bit comparisons are routed around (uniform_flag in the source).
- Every v_permlane16/32_swap follows an s_nop 3: the swaps are issued from
  inline asm, which gets no hazard wait states from the compiler.
- No v_fma_mixlo/mixhi_f16 adds a literal +0: the compiler forms that from
  an fp32 multiply followed by a conversion to fp16, and x * y + 0 turns a
  product of -0 into +0.
"""
from __future__ import annotations

import os
import re
import shutil
import subprocess
import tempfile

import pytest

from int4_row_wise_amd import build as qbuild

SCC_WRITERS = re.compile(
    r"^\s*(s_cmp|s_cmpk|s_and_|s_or_|s_xor_|s_andn2|s_orn2|s_nand|s_nor|s_xnor|s_add_|s_addc|"
    r"s_sub_|s_subb|s_lshl|s_lshr|s_ashr|s_bitcmp|s_min|s_max|s_abs|s_not|s_bfe|s_absdiff|"
    r"s_bcnt|s_ff|s_flbit)")
ARITH = re.compile(r"^\s*(s_add_|s_addc|s_sub_|s_subb|s_lshl|s_lshr|s_ashr|s_bcnt|s_min|s_max)")


@pytest.fixture(scope="module")
def asm():
    hipcc = qbuild.hipcc()
    if shutil.which(hipcc) is None and not os.path.exists(hipcc):
        pytest.skip("hipcc not available")
    flags = [f for f in qbuild.HIPCC_FLAGS if f not in ("-fPIC", "-shared")]
    with tempfile.TemporaryDirectory() as d:
        out = os.path.join(d, "qemb.s")
        cmd = [hipcc, *flags, "--cuda-device-only", "-S", "-I", os.path.join(qbuild.ROOT, "include"),
               "-o", out, qbuild.SRC]
        r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
        assert r.returncode == 0, r.stdout[-2000:]
        return open(out).read()


def instructions(asm):
    for line in asm.splitlines():
        t = line.strip()
        if t and not t.startswith((";", ".")) and not re.match(r"^\S+:", t):
            yield line


def test_no_packed_fp32(asm):
    bad = [l.strip() for l in instructions(asm) if re.match(r"\s*v_pk_(add|mul|fma)_f32", l)]
    assert not bad, bad[:5]


def test_no_scalar_cache_writes(asm):
    pat = re.compile(r"\s*s_(store|buffer_store|atomic|buffer_atomic|dcache_wb|dcache_discard)")
    bad = [l.strip() for l in instructions(asm) if pat.match(l)]
    assert not bad, bad[:5]


def test_no_stale_scc_select(asm):
    lines = asm.splitlines()
    bad = []
    for i, l in enumerate(lines):
        if "s_cselect" not in l:
            continue
        j, vcmp = i - 1, False
        while j > 0 and not SCC_WRITERS.match(lines[j]) and not re.match(r"^\S", lines[j]):
            if re.match(r"\s*v_cmp", lines[j]):
                vcmp = True
            j -= 1
        if vcmp and ARITH.match(lines[j]):
            bad.append((lines[j].strip(), l.strip()))
    assert not bad, bad[:5]


def test_swaps_have_wait_states(asm):
    lines = [l.strip() for l in instructions(asm)]
    swaps = [i for i, l in enumerate(lines) if l.startswith(("v_permlane16_swap", "v_permlane32_swap"))]
    assert swaps, "the lookup's reduce-scatter should use the swaps"
    bad = [lines[i] for i in swaps if lines[i - 1] != "s_nop 3"]
    assert not bad, bad[:5]


def test_no_fp16_mix_fma_with_plus_zero_addend(asm):
    pat = re.compile(r"\s*v_fma_mix(lo|hi)_f16\s+\S+,\s*\S+,\s*\S+,\s*0\s*$")
    bad = [l.strip() for l in instructions(asm) if pat.match(l)]
    assert not bad, bad[:5]
