"""Checks of the gfx950 code object that need no GPU: compile the kernels to
assembly and verify what the bit-exactness contract relies on.

* no fused or packed float32 arithmetic (v_fma/v_fmac/v_mad/v_pk_*_f32):
  the squared distance must round after every multiply and add;
* float32 denormals preserved in every kernel (denorm mode 3), IEEE mode on;
* no scratch memory: the register-resident FPS keeps its pulses in VGPRs.
"""
import os
import re

import pytest

from point_cloud_tokenization_amd import build as fbuild


@pytest.fixture(scope="module")
def asm(tmp_path_factory):
    out = str(tmp_path_factory.mktemp("asm") / "kernels.s")
    fbuild.device_asm(out)
    return open(out).read()


def test_no_fused_or_packed_fp32(asm):
    bad = re.findall(r"\b(v_(?:fma|fmac|mad|mac|pk_fma|pk_mul|pk_add)_f32\w*)", asm)
    assert bad == [], sorted(set(bad))


def test_denormals_and_ieee(asm):
    kernels = re.findall(r"\.amdhsa_kernel\s+(\S+)", asm)
    assert len(kernels) >= 8
    assert asm.count(".amdhsa_float_denorm_mode_32 3") == len(kernels)
    assert asm.count(".amdhsa_ieee_mode 1") == len(kernels)


def test_no_scratch(asm):
    sizes = re.findall(r"\.private_segment_fixed_size:\s+(\d+)", asm)
    assert sizes and all(int(s) == 0 for s in sizes), sizes
    assert "scratch_store" not in asm and "scratch_load" not in asm


def test_library_is_built_for_gfx950():
    if fbuild.is_stale():
        fbuild.build()
    data = open(fbuild.LIB, "rb").read()
    assert b"gfx950" in data


def _kernel_body(asm, prefix):
    m = re.search(r"^(%s\S*):" % re.escape(prefix), asm, re.M)
    assert m, prefix
    start = m.end()
    end = asm.index(".Lfunc_end", start)
    return asm[start:end]


def test_gang_poll_loads_issued_together(asm):
    """Every agent-scope (sc1) record load of the gang's poll spin is issued
    before any is waited for: hipcc waits for a load inside a divergent branch
    before leaving the branch, which made each spin cost one round trip per
    load.  In the work-list kernel no sc1 load may be followed by a full
    vmcnt(0) wait before the next sc1 load of the same run."""
    body = _kernel_body(asm, "_ZN6fpstok15tokenize_kernelILb0E")
    lines = [l.strip() for l in body.splitlines()]
    runs = 0
    for i, l in enumerate(lines):
        if not (l.startswith("global_load_dwordx2") and l.endswith("sc1")):
            continue
        # the next sc1 load within a few lines belongs to the same spin
        for k in range(i + 1, min(i + 24, len(lines))):
            if lines[k].startswith("global_load_dwordx2") and lines[k].endswith("sc1"):
                between = lines[i + 1:k]
                assert not any(b.startswith("s_waitcnt") and "vmcnt(0)" in b for b in between), \
                    "serialised record loads near line %d" % i
                runs += 1
                break
    assert runs > 0, "no poll spin found"
