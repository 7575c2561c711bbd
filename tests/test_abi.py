"""The C ABI on the CPU: the library loads, exports every function that
include/adamas.h declares, sizes workspaces, and rejects invalid arguments with
the documented status before any HIP call (so no GPU is needed here).
"""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "adamas.h")
GLUE_HEADER = os.path.join(ROOT, "include", "llama_glue.h")


@pytest.fixture(scope="module")
def A():
    import sparse_attention_long_fwht_amd as A
    return A


def declared_functions(header=HEADER):
    text = open(header).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[A-Za-z_][A-Za-z0-9_]*\s*\*?\s*([a-z_][a-z0-9_]*)\s*\(", text, flags=re.M)
    return sorted(set(names))


def test_header_declares_the_boundary():
    names = declared_functions()
    for n in ("adamas_encode_keys", "adamas_decode_step", "adamas_append_decode_step", "adamas_forced_decode_step",
              "adamas_paged_encode_keys", "adamas_paged_decode_step", "dense_paged_decode_attention",
              "dense_decode_attention",
              "adamas_decode_workspace_size",
              "dense_decode_workspace_size", "adamas_status_string", "adamas_abi_version"):
        assert n in names


def test_library_exports_every_declared_symbol(A):
    lib = A.raw_library()
    for n in declared_functions():
        assert hasattr(lib, n), n
    assert sorted(A.EXPORTED_SYMBOLS) == declared_functions()


def test_version_and_status_strings(A):
    assert A.abi_version() == 1
    assert A.status_string(0) == "ok"
    for s in range(1, 5):
        assert A.status_string(s) not in ("ok", "unknown status")
    assert A.status_string(99) == "unknown status"


def test_workspace_sizes(A):
    s128 = A.decode_workspace_size(1, 32, 8, 32768, 128)
    assert s128 > 0 and s128 % 256 == 0
    assert A.decode_workspace_size(1, 32, 8, 65536, 128) > s128
    assert A.decode_workspace_size(2, 32, 8, 32768, 128) > s128
    assert A.dense_workspace_size(1, 32, 8, 32768) > 0
    # invalid shapes give 0
    assert A.decode_workspace_size(1, 32, 8, 32768, 0) == 0
    assert A.decode_workspace_size(1, 30, 8, 32768, 8) == 0
    assert A.decode_workspace_size(1, 32, 8, 32768, 8, head_dim=64) == 0
    assert A.decode_workspace_size(1, 48, 8, 32768, 8) == 0  # group of 6 is not supported
    assert A.decode_workspace_size(1, 32, 8, (1 << 20) + 1, 8) == 0
    # the largest capacity takes budgets up to what one block's on-chip selection state holds
    assert A.decode_workspace_size(1, 32, 8, 1 << 19, 1024) > 0
    assert A.decode_workspace_size(1, 32, 8, 1 << 19, 65536) > 0
    assert A.decode_workspace_size(1, 32, 8, 1 << 19, 1 << 19) == 0


FAKE = 0x100000  # aligned, never dereferenced: every call below fails validation first


def call_decode(A, d, budget=8, ws_bytes=1 << 30, ptrs=None, ws=FAKE):
    lib = A.raw_library()
    p = dict(q=FAKE, k=FAKE, v=FAKE, codes=FAKE, kv_len=FAKE, out=FAKE)
    if ptrs:
        p.update(ptrs)
    return lib.adamas_decode_step(ctypes.byref(d), p["q"], p["k"], p["v"], p["codes"], p["kv_len"], budget,
                                  ctypes.c_float(0.088), p["out"], None, None, None, ws, ws_bytes, None)


def test_decode_rejects_invalid_arguments(A):
    lib = A.raw_library()
    good = A.dims(1, 32, 8, 32768)
    assert lib.adamas_decode_step(None, FAKE, FAKE, FAKE, FAKE, FAKE, 8, ctypes.c_float(1.0), FAKE, None, None,
                                  None, FAKE, 1 << 30, None) == A.ERR_INVALID_ARGUMENT
    assert call_decode(A, good, budget=0) == A.ERR_INVALID_ARGUMENT
    assert call_decode(A, good, ptrs=dict(q=None)) == A.ERR_INVALID_ARGUMENT
    assert call_decode(A, good, ptrs=dict(out=None)) == A.ERR_INVALID_ARGUMENT
    assert call_decode(A, good, ptrs=dict(k=FAKE + 2)) == A.ERR_INVALID_ARGUMENT  # misaligned
    assert call_decode(A, A.dims(0, 32, 8, 32768)) == A.ERR_INVALID_ARGUMENT
    assert call_decode(A, A.dims(1, 30, 8, 32768)) == A.ERR_INVALID_ARGUMENT
    assert call_decode(A, A.dims(1, 32, 8, 0)) == A.ERR_INVALID_ARGUMENT
    assert call_decode(A, A.dims(1, 32, 8, 32768, head_dim=64)) == A.ERR_UNSUPPORTED
    assert call_decode(A, A.dims(1, 24, 2, 32768)) == A.ERR_UNSUPPORTED  # group of 12
    assert call_decode(A, A.dims(1, 32, 8, (1 << 20) + 1)) == A.ERR_UNSUPPORTED
    assert call_decode(A, A.dims(1, 32, 8, 1 << 19), budget=1 << 19) == A.ERR_UNSUPPORTED
    need = A.decode_workspace_size(1, 32, 8, 32768, 8)
    assert call_decode(A, good, ws_bytes=need - 1) == A.ERR_WORKSPACE
    assert call_decode(A, good, ws=None) == A.ERR_WORKSPACE
    assert call_decode(A, good, ws=FAKE + 128) == A.ERR_WORKSPACE  # not 256-byte aligned


def call_forced(A, f, append=0, budget=8, d=None):
    lib = A.raw_library()
    d = d or A.dims(1, 32, 8, 32768)
    fp = ctypes.byref(f) if f is not None else None
    return lib.adamas_forced_decode_step(ctypes.byref(d), fp, append, FAKE, FAKE, FAKE, FAKE, FAKE, budget,
                                         ctypes.c_float(0.088), FAKE, None, None, None, None, 0, None)


def test_forced_decode_rejects_invalid_arguments(A):
    """Checked before anything else runs (the workspace here is missing, so an
    accepted forced set reaches ERR_WORKSPACE and no launch)."""
    F = A.Forced
    assert call_forced(A, F(2, 6, None, 0)) == A.ERR_WORKSPACE  # valid: fails only on the workspace
    assert call_forced(A, F(4, 4, None, 0)) == A.ERR_WORKSPACE  # sink + recent == budget is allowed
    assert call_forced(A, None) == A.ERR_INVALID_ARGUMENT
    assert call_forced(A, F(0, 0, None, 0), append=2) == A.ERR_INVALID_ARGUMENT
    assert call_forced(A, F(-1, 0, None, 0)) == A.ERR_INVALID_ARGUMENT
    assert call_forced(A, F(0, -1, None, 0)) == A.ERR_INVALID_ARGUMENT
    assert call_forced(A, F(5, 4, None, 0)) == A.ERR_INVALID_ARGUMENT  # more than the budget
    assert call_forced(A, F(0, 0, FAKE, 1023)) == A.ERR_INVALID_ARGUMENT  # 1023 * 32 < 32768 positions
    assert call_forced(A, F(0, 0, FAKE, 1024)) == A.ERR_WORKSPACE
    assert call_forced(A, F(0, 0, FAKE + 2, 1024)) == A.ERR_INVALID_ARGUMENT  # misaligned mask


def test_paged_entry_points_reject_invalid_pages(A):
    """Page descriptions are checked before anything runs (a valid one reaches
    ERR_WORKSPACE here, since no workspace is given)."""
    lib = A.raw_library()
    d = A.dims(2, 32, 8, 32768)

    def dec(pages):
        pp = ctypes.byref(pages) if pages is not None else None
        return lib.adamas_paged_decode_step(ctypes.byref(d), pp, None, 0, FAKE, FAKE, FAKE, FAKE, FAKE, 128,
                                            ctypes.c_float(0.088), FAKE, None, None, None, None, 0, None)

    P = A._PagesC
    assert dec(P(FAKE, 512, 64, 1200)) == A.ERR_WORKSPACE    # 512 pages of 64 = 32768
    assert dec(None) == A.ERR_INVALID_ARGUMENT
    assert dec(P(None, 512, 64, 1200)) == A.ERR_INVALID_ARGUMENT
    assert dec(P(FAKE, 511, 64, 1200)) == A.ERR_INVALID_ARGUMENT  # 511 * 64 < capacity
    assert dec(P(FAKE, 700, 48, 1200)) == A.ERR_INVALID_ARGUMENT  # not a power of two
    assert dec(P(FAKE, 512, 64, 0)) == A.ERR_INVALID_ARGUMENT     # empty pool
    assert dec(P(FAKE + 2, 512, 64, 1200)) == A.ERR_INVALID_ARGUMENT  # misaligned table
    assert lib.adamas_paged_encode_keys(ctypes.byref(d), None, FAKE, None, FAKE, FAKE, None) == A.ERR_INVALID_ARGUMENT
    assert lib.adamas_paged_encode_keys(ctypes.byref(d), ctypes.byref(P(FAKE, 511, 64, 9)), FAKE, None, FAKE, FAKE,
                                        None) == A.ERR_INVALID_ARGUMENT
    assert lib.dense_paged_decode_attention(ctypes.byref(d), ctypes.byref(P(FAKE, 512, 64, 9)), FAKE, FAKE, FAKE,
                                            FAKE, ctypes.c_float(1.0), FAKE, None, 0, None) == A.ERR_WORKSPACE
    assert lib.dense_paged_decode_attention(ctypes.byref(d), None, FAKE, FAKE, FAKE, FAKE, ctypes.c_float(1.0), FAKE,
                                            FAKE, 1 << 30, None) == A.ERR_INVALID_ARGUMENT


def test_encode_and_dense_reject_invalid_arguments(A):
    lib = A.raw_library()
    d = A.dims(1, 8, 8, 1024)
    assert lib.adamas_encode_keys(ctypes.byref(d), None, None, FAKE, FAKE, None) == A.ERR_INVALID_ARGUMENT
    assert lib.adamas_encode_keys(ctypes.byref(d), FAKE, None, None, FAKE, None) == A.ERR_INVALID_ARGUMENT
    assert lib.adamas_encode_keys(ctypes.byref(A.dims(1, 8, 8, 1024, head_dim=256)), FAKE, None, FAKE, FAKE,
                                  None) == A.ERR_UNSUPPORTED
    # the bounded form: a bound below 1 is rejected, the other checks are the same
    for bad in (0, -1, -(1 << 31)):
        assert lib.adamas_encode_keys_bounded(ctypes.byref(d), FAKE, None, FAKE, bad, FAKE,
                                              None) == A.ERR_INVALID_ARGUMENT
    assert lib.adamas_encode_keys_bounded(ctypes.byref(d), None, None, FAKE, 1, FAKE, None) == A.ERR_INVALID_ARGUMENT
    assert lib.adamas_paged_encode_keys_bounded(ctypes.byref(d), None, FAKE, None, FAKE, 1, FAKE,
                                                None) == A.ERR_INVALID_ARGUMENT
    assert lib.dense_decode_attention(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, ctypes.c_float(1.0), FAKE, FAKE, 0,
                                      None) == A.ERR_WORKSPACE
    assert lib.dense_decode_attention(ctypes.byref(d), FAKE, None, FAKE, FAKE, ctypes.c_float(1.0), FAKE, FAKE,
                                      1 << 30, None) == A.ERR_INVALID_ARGUMENT


def test_glue_library_exports_and_rejects():
    """libllama_glue.so exports what include/llama_glue.h declares; invalid
    arguments return 1 before any launch."""
    from sparse_attention_long_fwht_amd import llama_glue as G
    lib = G.raw_library()
    assert sorted(G.EXPORTED_SYMBOLS) == declared_functions(GLUE_HEADER)
    for n in declared_functions(GLUE_HEADER):
        assert hasattr(lib, n), n
    f = ctypes.c_float(1e-5)
    assert lib.llama_add_rmsnorm(None, None, None, FAKE, FAKE, 1, 4096, f, None) == 1
    assert lib.llama_add_rmsnorm(FAKE, None, None, FAKE, FAKE, 1, 4100, f, None) == 1   # hidden % 8
    assert lib.llama_add_rmsnorm(FAKE, None, None, FAKE, FAKE, 1, 32768, f, None) == 2  # too wide
    assert lib.llama_add_rmsnorm(FAKE + 2, None, None, FAKE, FAKE, 1, 4096, f, None) == 1  # misaligned
    assert lib.llama_rope_append(FAKE, None, FAKE, FAKE, FAKE, FAKE, 1, 32, 8, 100, None) == 1
    assert lib.llama_rope_append(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 0, 32, 8, 100, None) == 1
    assert lib.llama_silu_mul(FAKE, FAKE, 1, 100, None) == 1  # ffn % 8
    assert lib.llama_silu_mul(None, FAKE, 1, 128, None) == 1
    # the binding rejects buffers that do not match the dims before any call
    import torch
    x = torch.zeros((2, 64), dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="gu must have shape"):
        G.silu_mul(torch.zeros((2, 64), dtype=torch.bfloat16), x)
    with pytest.raises(ValueError, match="w must have shape"):
        G.add_rmsnorm(x, None, x, torch.zeros(32, dtype=torch.bfloat16), x, 1e-5)
    kc = torch.zeros((2, 1, 16, 128), dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="qkv must have shape"):
        G.rope_append(torch.zeros((2, 128), dtype=torch.bfloat16), torch.zeros(2, dtype=torch.int32),
                      torch.zeros(64), torch.zeros((2, 2, 128), dtype=torch.bfloat16), kc, kc)


def test_package_has_no_cpu_fallback():
    """The product package must not reach the oracle or any host implementation."""
    pkg = os.path.join(ROOT, "sparse_attention_long_fwht_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".h", ".cpp")):
                text = open(os.path.join(dirpath, f), encoding="utf-8").read()
                assert "import oracle" not in text and "from oracle" not in text, f
                assert "liboracle" not in text, f


def test_bench_refuses_several_gpus():
    """bench.py measures one GPU: --gpus above 1 exits with status 2 and says so,
    before any GPU work."""
    import subprocess
    import sys
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=300)
    assert r.returncode == 2 and "one GPU" in r.stderr


def test_binding_rejects_host_and_misshapen_tensors(A):
    """The binding checks its tensors before any library call: host tensors,
    non-contiguous views, wrong element sizes and buffers whose shapes do not
    match the dims raise ValueError (no GPU needed)."""
    import torch
    q = torch.zeros((1, 4, 128), dtype=torch.bfloat16)
    k = torch.zeros((1, 2, 64, 128), dtype=torch.bfloat16)
    codes = torch.zeros((1, 2, 64, 32), dtype=torch.uint8)
    kv_len = torch.full((1,), 64, dtype=torch.int32)
    out = torch.zeros((1, 4, 128), dtype=torch.float32)
    ws = torch.zeros(1 << 20, dtype=torch.uint8)
    with pytest.raises(ValueError, match="device tensor"):
        A.decode_step(q, k, k, codes, kv_len, 8, 0.1, out, ws)
    with pytest.raises(ValueError, match="device tensor"):
        A.encode_keys(k, kv_len, codes)
    with pytest.raises(ValueError, match="device tensor"):
        A.dense_decode_attention(q, k, k, kv_len, 0.1, out, ws)
    with pytest.raises(ValueError):
        A.Pages(torch.zeros((1, 4), dtype=torch.int64), 16)  # block table must be int32 [B][pages]
    # buffers that do not match the dims are rejected before any pointer is taken
    # (the kernels would index past their ends)
    with pytest.raises(ValueError, match="out must have shape"):
        A.decode_step(q, k, k, codes, kv_len, 8, 0.1, torch.zeros((1, 2, 128)), ws)
    with pytest.raises(ValueError, match="sel_idx must have shape"):
        A.decode_step(q, k, k, codes, kv_len, 8, 0.1, out, ws, sel_idx=torch.zeros((1, 4, 4), dtype=torch.int32))
    with pytest.raises(ValueError, match="dist must have shape"):
        A.decode_step(q, k, k, codes, kv_len, 8, 0.1, out, ws, dist=torch.zeros((1, 4, 32), dtype=torch.int16))
    with pytest.raises(ValueError, match="q_codes must have shape"):
        A.decode_step(q, k, k, codes, kv_len, 8, 0.1, out, ws, q_codes=torch.zeros((1, 4, 16), dtype=torch.uint8))
    with pytest.raises(ValueError, match="codes must have shape"):
        A.decode_step(q, k, k, codes[:, :, :32], kv_len, 8, 0.1, out, ws)
    with pytest.raises(ValueError, match="v must have shape"):
        A.decode_step(q, k, k[:, :1], codes, kv_len, 8, 0.1, out, ws)
    with pytest.raises(ValueError, match="kv_len must have shape"):
        A.dense_decode_attention(q, k, k, torch.zeros((2,), dtype=torch.int32), 0.1, out, ws)
    with pytest.raises(ValueError, match="sequences"):
        A.decode_step(q, torch.zeros((2, 2, 64, 128), dtype=torch.bfloat16), torch.zeros((2, 2, 64, 128)),
                      torch.zeros((2, 2, 64, 32), dtype=torch.uint8), kv_len, 8, 0.1, out, ws)
    with pytest.raises(ValueError, match="codes must have shape"):
        A.encode_keys(k, kv_len, codes[:, :1])
    with pytest.raises(ValueError, match="mask must have shape"):
        A.decode_step(q, k, k, codes, kv_len, 8, 0.1, out, ws, mask=torch.zeros((2, 2), dtype=torch.int32))
    table = torch.zeros((1, 4), dtype=torch.int32)
    with pytest.raises(ValueError, match="pages of 64 positions"):
        A.decode_step(q, k, k, codes, kv_len, 8, 0.1, out, ws, pages=A.Pages(table, 16))
    with pytest.raises(ValueError, match="page table has 1 rows"):
        A.decode_step(torch.zeros((2, 4, 128), dtype=torch.bfloat16), k, k, codes, torch.zeros(2, dtype=torch.int32),
                      8, 0.1, torch.zeros((2, 4, 128)), ws, pages=A.Pages(table, 64))


def test_bench_reads_committed_counters():
    """bench.py takes `traffic` from the committed counter summaries while they
    match the kernel sources (a hash in the file), and None when they do not."""
    import importlib.util
    spec = importlib.util.spec_from_file_location("bench_mod", os.path.join(ROOT, "bench.py"))
    bench = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(bench)
    for workload in bench.PMC_ARGS:
        for kernel in ("scan", "select_attend"):
            path = bench.counters_path(kernel, workload)
            assert os.path.exists(path), path
            text = open(path).read()
            got = bench.read_traffic(kernel, workload)
            if bench.source_hash(kernel) in text:
                assert got is not None and got > 0
            else:
                assert got is None


def test_bench_summarizes_sq_counters(tmp_path, monkeypatch):
    """The SQ counter summary reads rocprofv3's counter CSV (two passes), sums
    the SQ counters over their dimensions, and derives the ratios it states."""
    import csv
    import importlib.util
    spec = importlib.util.spec_from_file_location("bench_mod_sq", os.path.join(ROOT, "bench.py"))
    bench = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(bench)
    cols = ["Dispatch_Id", "Kernel_Name", "Workgroup_Size", "Counter_Name", "Counter_Value", "Start_Timestamp",
            "End_Timestamp"]
    passes = {"a": {"SQ_WAVES": 64, "SQ_WAVE_CYCLES": 800, "SQ_BUSY_CU_CYCLES": 400, "SQ_ACTIVE_INST_VALU": 100,
                    "SQ_ACTIVE_INST_ANY": 200, "SQ_WAIT_INST_ANY": 400, "GRBM_GUI_ACTIVE": 9},
              "b": {"SQ_INSTS_VALU": 6400, "SQ_INSTS_LDS": 640, "SQ_LDS_BANK_CONFLICT": 320,
                    "SQ_LDS_IDX_ACTIVE": 1280, "GRBM_GUI_ACTIVE": 9}}
    dirs = []
    for p, counters in passes.items():
        d = tmp_path / p
        d.mkdir()
        with open(d / "pmc_counter_collection.csv", "w", newline="") as fh:
            w = csv.writer(fh)
            w.writerow(cols)
            for disp in (1, 2):
                for c, v in counters.items():
                    for half in (0.5, 0.5):  # two shader engines: summed
                        w.writerow([disp, "void adamas::scan_kernel<4, false, false>(adamas::ScanArgs)", 512, c,
                                    v * half if c != "GRBM_GUI_ACTIVE" else v, 1000, 8000])
                w.writerow([disp, "__amd_rocclr_copyBuffer", 512, "SQ_WAVES", 1, 0, 1])
        dirs.append(str(d))
    monkeypatch.setattr(bench, "PROFILE_DIR", str(tmp_path / "out"))
    bench.summarize_sq("llama32k_b128", *dirs)
    text = open(tmp_path / "out" / "sq_counters_llama32k_b128.txt").read()
    row = [line for line in text.splitlines() if line.startswith("scan_kernel<4, false, false>")]
    assert len(row) == 1 and "copyBuffer" not in text
    f = row[0].split()[-12:]
    # dispatches, waves, waves/block, us, w/SIMD, VALU/cy, ANY/cy, wait, VALU/w, LDS/w, cf/LDS, cf/act
    assert f == ["2", "64", "8", "7.00", "2.00", "0.250", "0.500", "0.500", "100.0", "10.0", "0.50", "0.250"], f
    assert "--only-workload" not in text and "--pmc SQ_WAVES" in text


def test_bench_summarizes_byte_counters(tmp_path, monkeypatch):
    """The HBM byte counter summary scales each kernel's FETCH_SIZE and
    WRITE_SIZE by the first device copies of the program (the calibration
    copies), not by larger copies made later, and records the command of the
    workload it covers."""
    import csv
    import importlib.util
    spec = importlib.util.spec_from_file_location("bench_mod_pmc", os.path.join(ROOT, "bench.py"))
    bench = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(bench)
    cols = ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"]
    dirs = []
    for counter, calib, big, sel, scan in (("FETCH_SIZE", 32768.0, 500000.0, 300.0, 1000.0),
                                           ("WRITE_SIZE", 16384.0, 250000.0, 2.0, 40.0)):
        d = tmp_path / counter
        d.mkdir()
        with open(d / "pmc_counter_collection.csv", "w", newline="") as fh:
            w = csv.writer(fh)
            w.writerow(cols)
            did = 1
            for _ in range(3):  # calibration copies, two XCD halves each
                for half in (0.5, 0.5):
                    w.writerow([did, "__amd_rocclr_copyBuffer", counter, calib * half])
                did += 1
            w.writerow([did, "__amd_rocclr_copyBuffer", counter, big])  # a later clone of a big tensor
            did += 1
            for _ in range(2):
                w.writerow([did, "void adamas::scan_kernel<4, false, false>(adamas::ScanArgs)", counter, scan])
                w.writerow([did + 1, "void adamas::select_attend_kernel<false>(adamas::SelectArgs)", counter, sel])
                did += 2
        dirs.append(str(d))
    monkeypatch.setattr(bench, "PROFILE_DIR", str(tmp_path / "out"))
    bench.summarize_counters("batched16_ragged16k-32k_b256", *dirs)
    text = open(tmp_path / "out" / "scan_kernel_batched16_ragged16k-32k_b256_counters.txt").read()
    # scale 2 for FETCH (65536 / 32768), 4 for WRITE (65536 / 16384)
    assert "hbm_bytes_per_launch: %d" % int((1000 * 2 + 40 * 4) * 1024) in text, text
    assert "--only-workload batched16_ragged16k-32k_b256 --calibrate-copy-mib 64" in text
    # read back for the bench line while the kernel sources are the ones hashed
    assert bench.read_traffic("scan", "batched16_ragged16k-32k_b256") == (1000 * 2 + 40 * 4) * 1024
    assert bench.read_traffic("scan", "long512k_b1024") is None


def test_workspace_for_any_int32_budget(A):
    """A budget past the capacity plans like budget = capacity (no step selects
    more rows), so every positive int32 budget gives a sane size and no
    arithmetic overflows; budgets the select kernel cannot hold give 0."""
    for B, Hq, Hkv, cap in ((1, 32, 8, 32768), (3, 8, 2, 3000), (1, 4, 1, 1)):
        at_cap = A.decode_workspace_size(B, Hq, Hkv, cap, cap)
        assert 0 < at_cap < (1 << 32)
        for budget in (cap + 1, 1 << 20, 1 << 30, 2 ** 31 - 1):
            assert A.decode_workspace_size(B, Hq, Hkv, cap, budget) == at_cap, (cap, budget)
    assert A.decode_workspace_size(1, 32, 8, 524288, 245760) > 0
    for budget in (245761, 1 << 30, 2 ** 31 - 1):
        assert A.decode_workspace_size(1, 32, 8, 524288, budget) == 0


def test_decoder_refuses_steps_past_capacity():
    """The Llama-shaped decode loop counts appended tokens on the host: a step or
    a graph replay that would write past the cache capacity raises before
    anything is issued (CPU tensors: nothing here reaches a kernel)."""
    import pytest
    from sparse_attention_long_fwht_amd.llama_decode import DecoderShape, LlamaShapedDecoder, _GuardedGraph
    shape = DecoderShape(layers=1, hidden=256, q_heads=2, kv_heads=1, ffn=64, vocab=32)
    m = LlamaShapedDecoder(shape, batch=2, capacity=10, attention="dense", device="cpu")
    m.len_hi = 9
    st = m.state()
    m.reserve(1)  # position 9, the last one, fits
    assert m.len_hi == 10
    with pytest.raises(RuntimeError, match="capacity"):
        m.step()  # raises before any launch
    assert m.len_hi == 10
    m.restore(st)
    assert m.len_hi == 9

    class FakeGraph:
        replays = 0

        def replay(self):
            FakeGraph.replays += 1

    g = _GuardedGraph(m, FakeGraph(), 1)
    g.replay()
    with pytest.raises(RuntimeError, match="capacity"):
        g.replay()
    assert FakeGraph.replays == 1
    m.len_hi = 8
    with pytest.raises(RuntimeError, match="cannot run"):
        m.capture(3)


def test_noalloc_decode_rejects_before_any_hip_call(A):
    """adamas_decode_step_noalloc checks its arguments and the scratch size
    before touching the GPU (these calls return without a device)."""
    lib = A.raw_library()

    def call(d, budget=128, q=FAKE, out=FAKE):
        return lib.adamas_decode_step_noalloc(ctypes.byref(d), q, FAKE, FAKE, FAKE, FAKE, budget,
                                              ctypes.c_float(0.088), out, None, None, None, None)

    assert lib.adamas_decode_step_noalloc(None, FAKE, FAKE, FAKE, FAKE, FAKE, 8, ctypes.c_float(0.1), FAKE, None,
                                          None, None, None) == A.ERR_INVALID_ARGUMENT
    assert call(A.dims(1, 32, 8, 32768), q=None) == A.ERR_INVALID_ARGUMENT
    assert call(A.dims(1, 32, 8, 32768), budget=0) == A.ERR_INVALID_ARGUMENT
    assert call(A.dims(1, 32, 8, 32768), q=FAKE + 2) == A.ERR_INVALID_ARGUMENT  # misaligned
    assert call(A.dims(1, 32, 8, 32768, head_dim=64)) == A.ERR_UNSUPPORTED
    # workspace beyond the 64 MiB static scratch: 64 sequences of 32K positions
    assert A.decode_workspace_size(64, 32, 8, 32768, 128) > A.NOALLOC_SCRATCH_BYTES
    assert call(A.dims(64, 32, 8, 32768)) == A.ERR_UNSUPPORTED
    # the largest configurations of the benchmark fit
    for dims, budget in (((1, 32, 8, 32768), 1024), ((16, 32, 8, 32768), 256), ((1, 32, 8, 524288), 1024)):
        assert 0 < A.decode_workspace_size(*dims, budget) <= A.NOALLOC_SCRATCH_BYTES
