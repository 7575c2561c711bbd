"""Register and scratch budgets of the decode kernels (CPU only: reads the
device assembly hipcc writes for gfx950, runs nothing).

Two budgets matter for speed, not for correctness, and a small source change
can break either without any test failing:

- 128 VGPRs at most for the select/attend kernel and for the R = 4 scan
  kernels: their blocks have 512 threads (8 waves), and two blocks per compute
  unit need 16 waves, 4 per SIMD, so 128 registers each.  The batched shapes
  run 512 blocks of either kernel on 256 compute units in one round only
  within that budget (at 129 the batch-16 select kernel went from 18.7 to
  23.5 us).
- no private (scratch) memory in any kernel: a spill to scratch turns register
  reads into memory round trips on every critical path.
"""
import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _device_asm(tmp_path, source):
    import importlib.util
    spec = importlib.util.spec_from_file_location("_adamas_build_flags",
                                                  os.path.join(ROOT, "sparse_attention_long_fwht_amd", "build.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    if not (os.path.exists(mod.HIPCC) or shutil.which(mod.HIPCC)):
        pytest.skip("no hipcc")
    flags = [f for f in mod.FLAGS if f not in ("-fPIC", "-shared")]
    out = str(tmp_path / (os.path.basename(source) + ".s"))
    res = subprocess.run([mod.HIPCC, *flags, "--cuda-device-only", "-S", os.path.join(mod.CSRC, source), "-o", out],
                         capture_output=True, text=True, timeout=600)
    assert res.returncode == 0, res.stderr[-3000:]
    return open(out).read()


def _resources(asm):
    """{kernel symbol: {"num_vgpr": n, "private_seg_size": n, ...}} from the .set lines."""
    res = {}
    for name, key, val in re.findall(r"^\s*\.set\s+(_Z\S+)\.(num_vgpr|num_agpr|private_seg_size),\s*(\d+)", asm, re.M):
        res.setdefault(name, {})[key] = int(val)
    return res


@pytest.fixture(scope="module")
def decode_resources(tmp_path_factory):
    return _resources(_device_asm(tmp_path_factory.mktemp("asm"), "decode.hip"))


def test_select_kernel_fits_two_blocks_per_compute_unit(decode_resources):
    sel = {k: v for k, v in decode_resources.items() if "select_attend_kernel" in k}
    assert len(sel) == 2, sorted(decode_resources)  # contiguous and paged caches
    for name, r in sel.items():
        assert r["num_vgpr"] + r.get("num_agpr", 0) <= 128, (name, r)


def test_r4_scan_kernels_fit_two_blocks_per_compute_unit(decode_resources):
    scans = {k: v for k, v in decode_resources.items() if re.search(r"scan_kernelILi4E", k)}
    assert len(scans) == 20, sorted(scans)  # forced x paged x passes 1, 2, 4, 8, 16
    for name, r in scans.items():
        assert r["num_vgpr"] + r.get("num_agpr", 0) <= 128, (name, r)


def test_no_decode_kernel_uses_scratch(decode_resources):
    kernels = {k: v for k, v in decode_resources.items() if "private_seg_size" in v}
    assert kernels
    for name, r in kernels.items():
        assert r["private_seg_size"] == 0, (name, r)


def test_no_encode_or_dense_kernel_uses_scratch(tmp_path):
    res = _resources(_device_asm(tmp_path, "kernels.hip"))
    assert any("encode_keys_kernel" in k for k in res) and any("dense_attend_kernel" in k for k in res)
    for name, r in res.items():
        if "private_seg_size" in r:
            assert r["private_seg_size"] == 0, (name, r)
