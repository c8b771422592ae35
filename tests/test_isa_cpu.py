"""Checks on the gfx950 machine code of our own build (CPU only).

The built library's device code object is extracted and disassembled with
ROCm's llvm-objdump, then checked for:
* no scratch (private memory) traffic in the hot kernels: scratch loads share
  the in-order vector-memory counter with the K/V loads, so one stray spill
  serialises the prefetch pipeline;
* no packed-fp32 instructions anywhere (the build disables them);
* no stores or atomics through the scalar data cache, and no scalar cache
  write-back / discard.
"""
import os
import re
import shutil
import subprocess
import tempfile

import pytest

import paged_kv_cache_v2_amd as pa
from paged_kv_cache_v2_amd import binding

OBJDUMP = "/opt/rocm/llvm/bin/llvm-objdump"


@pytest.fixture(scope="module")
def kernels():
    if not os.path.exists(OBJDUMP):
        pytest.skip("llvm-objdump not available")
    pa.ensure_built()
    with tempfile.TemporaryDirectory() as d:
        lib = os.path.join(d, "lib.so")
        shutil.copy(binding.LIB_PATH, lib)
        subprocess.run([OBJDUMP, "--offloading", lib], cwd=d, check=True, capture_output=True)
        cos = sorted(f for f in os.listdir(d) if "gfx950" in f)
        assert cos, "no gfx950 code object in the library"
        # one code object per translation unit (host unit + instantiation units)
        out = {}
        for co in cos:
            dis = subprocess.run([OBJDUMP, "-d", "--mcpu=gfx950", os.path.join(d, co)],
                                 check=True, capture_output=True, text=True).stdout
            for m in re.finditer(r"\n[0-9a-f]+ <(\S+)>:\n(.*?)(?=\n\n|\Z)", dis, re.S):
                out[m.group(1)] = [l.split("//")[0].strip() for l in m.group(2).splitlines()]
    assert any("partition_mfma_kernel" in k for k in out)
    return out


def ops(lines):
    return [l.split()[0] for l in lines if l]


def spill_exempt(name):
    # fp32 caches with head_size 256 hold q in registers and spill; a known cost
    # of that rare combination, kept correct (tests cover it) rather than fast.
    return "partition_vec_kernelILi0ELi256" in name


def test_hot_kernels_use_no_scratch(kernels):
    bad = {k: sum(o.startswith("scratch_") for o in ops(v)) for k, v in kernels.items()
           if ("partition_" in k or "reduce_kernel" in k or "reduce_one_kernel" in k) and not spill_exempt(k)}
    bad = {k: v for k, v in bad.items() if v}
    assert not bad, f"scratch traffic in {bad}"


def test_no_packed_fp32(kernels):
    packed = ("v_pk_add_f32", "v_pk_mul_f32", "v_pk_fma_f32")
    hits = {k: [o for o in ops(v) if o.startswith(packed)] for k, v in kernels.items()}
    assert not {k: v for k, v in hits.items() if v}


def test_no_scalar_cache_writes(kernels):
    forbidden = re.compile(r"^(s_store|s_buffer_store|s_scratch_store|s_atomic|s_buffer_atomic|"
                           r"s_dcache_wb|s_dcache_discard)")
    hits = {k: [o for o in ops(v) if forbidden.match(o)] for k, v in kernels.items()}
    assert not {k: v for k, v in hits.items() if v}


def test_kv_loads_are_dwordx4_or_dwordx2_streaming(kernels):
    """K/V pages are fetched with 16-byte (K, vector-path V, 8-bit MFMA-path V) or
    8-byte (16-bit MFMA-path V, also in the rolling-merge instantiations) non-temporal loads; the 8-bit MFMA path then
    transposes its V words across lane rows with the gfx950 permlane swaps."""
    seen = 0
    for k, v in kernels.items():
        nt = [l for l in v if l.startswith("global_load") and l.endswith(" nt")]
        if "partition_mfma_kernelILi2ELi128ELi16ELb0" in k:
            assert any(l.startswith("global_load_dwordx4") for l in nt)
            assert any(l.startswith("global_load_dwordx2") for l in nt)
            seen += 1
        if "partition_mfma_kernelILi2ELi128ELi16ELb1" in k:
            assert any(l.startswith("global_load_dwordx4") for l in nt)
            assert not any(l.startswith(("global_load_dword ", "global_load_dwordx2")) for l in nt)
            assert {"v_permlane32_swap_b32_e32", "v_permlane16_swap_b32_e32"} <= set(ops(v))
            seen += 1
        if "partition_vec_kernelILi2ELi128ELi16ELi1ELb1" in k:
            assert any(l.startswith("global_load_dwordx4") for l in nt)
            seen += 1
    # each with ALiBi off and on; the MFMA ones (16-bit and 8-bit caches) with
    # one and two column tiles, with and without the rolling merge
    assert seen == 18


def test_fp8_kernels_convert_with_gfx950_instructions(kernels):
    """8-bit pages are widened in registers by the gfx950 conversions."""
    for k, v in kernels.items():
        o = set(ops(v))
        if "partition_mfma_kernelILi2ELi128ELi16ELb1" in k:
            assert "v_cvt_scalef32_pk_bf16_fp8" in o
        if "partition_mfma_kernelILi1ELi128ELi16ELb1" in k:
            assert "v_cvt_scalef32_pk_f16_fp8" in o
        if "partition_vec_kernelILi2ELi128ELi16ELi1ELb1" in k:
            assert "v_cvt_scalef32_pk_bf16_fp8" in o
            assert any(x.startswith("v_cvt_pk_f32_fp8") for x in o)
