"""CPU tests of the C ABI: every declared symbol is exported, and invalid arguments come back
as the documented status before any HIP call (so these run without a GPU)."""
import ctypes
import os
import re
import subprocess

import pytest
import torch

import bandwidth_bound_decode_amd as bbd
from bandwidth_bound_decode_amd._binding import DeviceDesc, PlanOpts, Segment, Status

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "gemv.h")
MI355X = (256, 8.0e12, 1.0e-6)
FAKE = 0x7F0000000000          # 16-byte aligned stand-in for a device address (never touched)


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(gemv_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_boundary():
    names = declared_functions()
    for required in ("gemv_plan", "gemv_run", "gemv_fused_run", "gemv_graph_begin",
                     "gemv_graph_end", "gemv_graph_launch", "gemv_graph_destroy",
                     "gemv_workspace_size", "gemv_plan_query", "gemv_plan_destroy",
                     "gemv_status_string", "gemv_last_hip_error"):
        assert required in names


def test_library_exports_every_declared_symbol():
    names = declared_functions()
    out = subprocess.run(["nm", "-D", "--defined-only", bbd.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r"\b[TW]\s+(\S+)$", out, flags=re.M))
    missing = [n for n in names if n not in exported]
    assert not missing, missing
    assert sorted(bbd.SIGNATURES) == names, "binding signatures out of sync with the header"
    for n in names:
        assert hasattr(bbd.lib(), n)


def test_library_targets_gfx950_only(tmp_path):
    """The device code object bundled in the library is for gfx950 and nothing else."""
    fatbin = tmp_path / "fatbin"
    # explicit output file: objcopy without one rewrites its input in place
    subprocess.run(["objcopy", "-O", "binary", "--only-section=.hip_fatbin", bbd.LIB_PATH,
                    str(fatbin)], check=True, capture_output=True)
    out = subprocess.run(["/opt/rocm/llvm/bin/clang-offload-bundler", "--list", "--type=o",
                          f"--input={fatbin}"], capture_output=True, text=True, check=True)
    targets = [t for t in out.stdout.split() if "amdgcn" in t]
    assert targets == ["hipv4-amdgcn-amd-amdhsa--gfx950"], targets


def test_status_strings():
    lib = bbd.lib()
    seen = set()
    for s in Status:
        text = lib.gemv_status_string(int(s)).decode()
        assert text and text != "unknown status"
        seen.add(text)
    assert len(seen) == len(Status)
    assert lib.gemv_status_string(99).decode() == "unknown status"


def host_plan(n, k, m=1, **opts):
    h = ctypes.c_void_p()
    o = PlanOpts(opts.get("splits", 0), opts.get("rows_per_wave", 0),
                 opts.get("waves_per_block", 0), opts.get("unroll", 0))
    d = DeviceDesc(*MI355X)
    st = bbd.lib().gemv_plan_for(ctypes.byref(h), n, k, m, ctypes.byref(d), ctypes.byref(o))
    return st, h


@pytest.fixture
def plan_split():
    st, h = host_plan(1024, 4096, 1, splits=4)      # k_proj shape, K split in 4
    assert st == Status.OK
    yield h
    bbd.lib().gemv_plan_destroy(h)


@pytest.fixture
def plan_m3():
    st, h = host_plan(64, 1000, 3, splits=1)
    assert st == Status.OK
    yield h
    bbd.lib().gemv_plan_destroy(h)


def run(h, W=FAKE, ldw=4096, X=FAKE, ldx=4096, Y=FAKE, ldy=1024, ws=FAKE, ws_bytes=1 << 20):
    return bbd.lib().gemv_run(h, W, ldw, X, ldx, Y, ldy, ws, ws_bytes, None)


def test_plan_arguments():
    for n, k, m in ((0, 8, 1), (8, 0, 1), (8, 8, 0), (8, 8, 17), (-1, 8, 1)):
        assert host_plan(n, k, m)[0] == Status.INVALID_ARG
    assert host_plan(8, 8, 1, splits=-1)[0] == Status.INVALID_ARG
    assert host_plan(8, 8, 1, rows_per_wave=3)[0] == Status.INVALID_ARG     # not compiled
    assert host_plan(8, 8, 16, unroll=8)[0] == Status.INVALID_ARG
    assert host_plan(8, 8, 1, waves_per_block=3)[0] == Status.INVALID_ARG
    assert host_plan(8, 8, 1, splits=65)[0] == Status.INVALID_ARG
    assert host_plan(8, 129, 1, splits=7)[0] == Status.INVALID_ARG         # empty slice
    lib = bbd.lib()
    d = DeviceDesc(0, 8e12, 1e-6)
    h = ctypes.c_void_p()
    assert lib.gemv_plan_for(ctypes.byref(h), 8, 8, 1, ctypes.byref(d), None) == Status.INVALID_ARG
    assert lib.gemv_plan_for(None, 8, 8, 1, ctypes.byref(DeviceDesc(*MI355X)), None) \
        == Status.INVALID_ARG
    # gemv_plan rejects bad sizes before asking the runtime about the device
    assert lib.gemv_plan(ctypes.byref(h), 0, 8, 1, 0, None) == Status.INVALID_ARG
    assert lib.gemv_plan(ctypes.byref(h), 8, 8, 17, 0, None) == Status.INVALID_ARG
    assert lib.gemv_plan_query(None, None) == Status.INVALID_ARG
    assert lib.gemv_workspace_size(None) == 0
    lib.gemv_plan_destroy(None)


@pytest.mark.skipif(torch.cuda.is_available(), reason="checks the no-GPU error path")
def test_plan_without_device_is_a_device_error():
    h = ctypes.c_void_p()
    assert bbd.lib().gemv_plan(ctypes.byref(h), 8, 8, 1, 0, None) == Status.DEVICE
    assert not h


def test_run_validation(plan_split, plan_m3):
    h = plan_split
    # a 4096-slot ticket region, then S=4 x M=1 x N=1024 fp32 partials
    assert bbd.lib().gemv_workspace_size(h) == 4096 * 4 + 4 * 1024 * 4
    assert run(None) == Status.INVALID_ARG
    assert run(h, W=None) == Status.INVALID_ARG
    assert run(h, X=None) == Status.INVALID_ARG
    assert run(h, Y=None) == Status.INVALID_ARG
    assert run(h, ldw=4095) == Status.INVALID_ARG
    assert run(h, ldy=1023) == Status.INVALID_ARG
    assert run(h, W=FAKE + 1) == Status.MISALIGNED
    assert run(h, X=FAKE + 3) == Status.MISALIGNED
    assert run(h, Y=FAKE + 2) == Status.MISALIGNED
    assert run(h, ws=None) == Status.WORKSPACE
    assert run(h, ws_bytes=4096 * 4 + 4 * 1024 * 4 - 1) == Status.WORKSPACE
    assert run(h, ws=FAKE + 2) == Status.MISALIGNED
    # batched plan: X rows need ldx >= k; ldx is not checked for a single vector
    assert run(plan_m3, ldw=1000, ldx=999, ldy=64, ws=None, ws_bytes=0) == Status.INVALID_ARG


def test_fused_validation(plan_split):
    lib = bbd.lib()
    h = plan_split

    def fused(segs, X=FAKE, ws=FAKE, ws_bytes=1 << 20, nseg=None):
        arr = (Segment * max(len(segs), 1))(*segs)
        return lib.gemv_fused_run(h, arr, len(segs) if nseg is None else nseg, X, 4096, ws,
                                  ws_bytes, None)

    good = [Segment(FAKE, 512, 4096, FAKE, 512), Segment(FAKE, 512, 4096, FAKE, 512)]
    assert fused(good, nseg=0) == Status.INVALID_ARG
    assert fused(good * 3, nseg=5) == Status.INVALID_ARG
    assert fused(good[:1]) == Status.INVALID_ARG                 # 512 rows != plan's 1024
    assert fused([Segment(FAKE, 1024, 4096, FAKE, 1024), Segment(FAKE, 0, 4096, FAKE, 1)]) \
        == Status.INVALID_ARG
    assert fused([good[0], Segment(FAKE, 512, 4000, FAKE, 512)]) == Status.INVALID_ARG
    assert fused([good[0], Segment(FAKE + 1, 512, 4096, FAKE, 512)]) == Status.MISALIGNED
    assert fused(good, ws=None) == Status.WORKSPACE
    assert lib.gemv_fused_run(h, None, 2, FAKE, 4096, FAKE, 1 << 20, None) == Status.INVALID_ARG


def test_graph_argument_errors():
    lib = bbd.lib()
    assert lib.gemv_graph_begin(None) == Status.CAPTURE          # legacy default stream
    assert lib.gemv_graph_end(None, None) == Status.INVALID_ARG
    out = ctypes.c_void_p()
    assert lib.gemv_graph_end(None, ctypes.byref(out)) == Status.CAPTURE
    assert lib.gemv_graph_launch(None, None) == Status.INVALID_ARG
    lib.gemv_graph_destroy(None)


def test_no_kernel_uses_scratch():
    """The build records the compiler's per-kernel resource usage and refuses scratch or VGPR
    spills; every kernel keeps enough occupancy for its loads in flight."""
    import json
    report = os.path.join(os.path.dirname(bbd.LIB_PATH), "kernel_resources.json")
    kernels = json.load(open(report))
    assert len(kernels) >= 2 * 2 * 13 + 2 * 2 * 16
    for name, r in kernels.items():
        assert r["ScratchSize [bytes/lane]"] == "0", name
        assert r["VGPRs Spill"] == "0", name
        assert int(r["Occupancy [waves/SIMD]"]) >= 2, name


def test_chain_validation_before_any_hip_call():
    from bandwidth_bound_decode_amd._binding import ChainLink
    lib = bbd.lib()
    h = ctypes.c_void_p()

    def create(links, n=None):
        arr = (ChainLink * max(len(links), 1))(*links)
        return lib.gemv_chain_create(ctypes.byref(h), arr, len(links) if n is None else n, 0,
                                     None)

    seg = (Segment * 2)(Segment(FAKE, 64, 4096, FAKE, 64), Segment(FAKE, 32, 4096, FAKE, 32))
    good = ChainLink(seg, 2, FAKE, 4096)
    assert lib.gemv_chain_create(None, None, 1, 0, None) == Status.INVALID_ARG
    assert create([good], n=0) == Status.INVALID_ARG
    assert create([ChainLink(seg, 0, FAKE, 4096)]) == Status.INVALID_ARG
    assert create([ChainLink(seg, 5, FAKE, 4096)]) == Status.INVALID_ARG
    assert create([ChainLink(seg, 2, None, 4096)]) == Status.INVALID_ARG
    assert create([ChainLink(seg, 2, FAKE, 0)]) == Status.INVALID_ARG
    assert create([ChainLink(seg, 2, FAKE, 7)]) == Status.INVALID_ARG          # k < 8
    assert create([ChainLink(seg, 2, FAKE, 4097)]) == Status.INVALID_ARG       # ldw < k
    assert create([ChainLink(seg, 2, FAKE + 8, 4096)]) == Status.MISALIGNED    # X
    bad_w = (Segment * 1)(Segment(FAKE + 2, 64, 4096, FAKE, 64))
    assert create([ChainLink(bad_w, 1, FAKE, 4096)]) == Status.MISALIGNED
    bad_ld = (Segment * 1)(Segment(FAKE, 64, 4100, FAKE, 64))
    assert create([ChainLink(bad_ld, 1, FAKE, 4096)]) == Status.MISALIGNED
    from bandwidth_bound_decode_amd._binding import ChainOpts
    for waves in (-1, 12):                                                      # 1..11 workers
        assert lib.gemv_chain_create(ctypes.byref(h), (ChainLink * 1)(good), 1, 0,
                                     ctypes.byref(ChainOpts(waves, 0))) == Status.INVALID_ARG
    assert not h
    assert lib.gemv_chain_run(None, None) == Status.INVALID_ARG
    assert lib.gemv_chain_check(None) == Status.INVALID_ARG
    lib.gemv_chain_destroy(None)


def test_binding_refuses_host_tensors_and_short_buffers():
    """The binding hands data pointers to the kernels as device pointers: host tensors and
    buffers smaller than the plan are refused before any call reaches the library."""
    import torch

    import bandwidth_bound_decode_amd as bbd

    plan = bbd.Plan(64, 256, 2, desc=(256, 8.0e12, 1.0e-6))   # host-only plan
    W = torch.zeros((64, 256), dtype=torch.bfloat16)
    X = torch.zeros((2, 256), dtype=torch.bfloat16)
    Y = torch.zeros((2, 64), dtype=torch.float32)
    with pytest.raises(ValueError, match="on the GPU"):
        bbd.run(plan, W, X, Y)
    with pytest.raises(ValueError, match="on the GPU"):
        bbd.fused_run(plan, [(W[:32], Y[:, :32]), (W[32:], Y[:, 32:])], X)
    with pytest.raises(TypeError):
        bbd.run(plan, W.float(), X, Y)
    # shape checks are exercised with the device check bypassed
    from bandwidth_bound_decode_amd import _binding as b
    with pytest.raises(ValueError, match="the plan needs"):
        b._need(X[:1], plan.m, plan.k, "X")
    with pytest.raises(ValueError, match="the plan needs"):
        b._need(Y[:, :63], plan.m, plan.n, "Y")
    b._need(X, plan.m, plan.k, "X")
    b._need(torch.zeros(256, dtype=torch.bfloat16), 1, 256, "X")


def test_package_fails_loudly_without_the_library(tmp_path):
    """With the compiled library absent the package refuses to import: there is no CPU or
    Python fallback path. Checked in a child process on a copy of the package whose lib/
    directory is empty."""
    import shutil
    import sys

    pkg = os.path.join(ROOT, "bandwidth_bound_decode_amd")
    copy = tmp_path / "bandwidth_bound_decode_amd"
    shutil.copytree(pkg, copy, ignore=shutil.ignore_patterns("lib", "__pycache__"))
    (copy / "lib").mkdir()
    proc = subprocess.run([sys.executable, "-c", "import bandwidth_bound_decode_amd"],
                          cwd=tmp_path, capture_output=True, text=True, timeout=300)
    assert proc.returncode != 0
    assert "ImportError" in proc.stderr and "no fallback" in proc.stderr, proc.stderr[-500:]


def test_binding_refuses_strided_rows():
    """A view whose elements along a row are not adjacent (buf[::2], M[:, j]) would be read
    by the kernels as if it were dense; the binding refuses it, for 1-D and 2-D operands and
    for the single-vector operands of the INT4, RMSNorm and chain calls."""
    from bandwidth_bound_decode_amd import _binding as b

    buf = torch.zeros(512, dtype=torch.bfloat16)
    mat = torch.zeros((64, 256), dtype=torch.bfloat16)
    assert buf[::2].stride() == (2,)
    with pytest.raises(ValueError, match="contiguous"):
        b._row_stride(buf[::2], "X")
    with pytest.raises(ValueError, match="contiguous"):
        b._row_stride(mat[:, 3], "X")
    with pytest.raises(ValueError, match="contiguous"):
        b._row_stride(mat[:, ::2], "W")
    with pytest.raises(ValueError, match="contiguous"):
        b._vector(buf[::2], "H")
    with pytest.raises(ValueError, match=r"\[k\] or \[1, k\]"):
        b._vector(mat[:2], "X")
    # dense operands and one-element rows pass, with the row stride the kernels expect
    assert b._row_stride(buf, "X") == 512
    assert b._row_stride(buf[:1], "X") == 1
    assert b._row_stride(mat, "W") == 256
    assert b._row_stride(mat[:, :100], "W") == 256
    assert b._row_stride(mat[:1, :100], "W") == 100
    assert b._row_stride(mat[:, :1], "W") == 256
    b._vector(mat[:1], "X")
    b._vector(buf, "X")


def test_static_entry_point_refuses_before_any_hip_call():
    """gemv_run_static validates like gemv_run and refuses a split plan whose partial sums
    exceed the static scratch array, all before any HIP call (host-only plans, fake
    pointers)."""
    lib = bbd.lib()
    desc = DeviceDesc(256, 8.0e12, 1.0e-6)
    h = ctypes.c_void_p()
    # 2 slices x 16 vectors x 40000 rows x 4 B = 5.1 MB of partial sums > 4 MiB
    opts = PlanOpts(2, 0, 0, 0, 0, -1, 0, 0)
    assert lib.gemv_plan_for(ctypes.byref(h), 40000, 14336, 16, ctypes.byref(desc),
                             ctypes.byref(opts)) == Status.OK
    try:
        assert lib.gemv_workspace_size(h) > 4 << 20
        assert lib.gemv_run_static(h, FAKE, 14336, FAKE, 14336, FAKE, 40000,
                                   None) == Status.WORKSPACE
        assert lib.gemv_run_static(h, None, 14336, FAKE, 14336, FAKE, 40000,
                                   None) == Status.INVALID_ARG
        assert lib.gemv_run_static(h, FAKE, 14335, FAKE, 14336, FAKE, 40000,
                                   None) == Status.INVALID_ARG
        assert lib.gemv_run_static(h, FAKE + 1, 14336, FAKE, 14336, FAKE, 40000,
                                   None) == Status.MISALIGNED
    finally:
        lib.gemv_plan_destroy(h)
    assert lib.gemv_run_static(None, FAKE, 4096, FAKE, 4096, FAKE, 64, None) == \
        Status.INVALID_ARG


def test_read_stream_validation_before_any_hip_call():
    lib = bbd.lib()
    sink = FAKE + 64
    ok = dict(buf=FAKE, rows=8, row_bytes=4096, unroll=4, waves=8, sink=sink)

    def call(**kw):
        a = dict(ok, **kw)
        return lib.gemv_read_stream(a["buf"], a["rows"], a["row_bytes"], a["unroll"],
                                    a["waves"], a["sink"], None)
    assert call(buf=None) == Status.INVALID_ARG
    assert call(sink=None) == Status.INVALID_ARG
    assert call(rows=0) == Status.INVALID_ARG
    assert call(row_bytes=4096 + 1024) == Status.INVALID_ARG     # not a multiple of 1 KiB * U
    assert call(unroll=3) == Status.INVALID_ARG
    assert call(waves=33) == Status.INVALID_ARG
    assert call(waves=-1) == Status.INVALID_ARG
    assert call(buf=FAKE + 8) == Status.MISALIGNED
    assert call(sink=sink + 2) == Status.MISALIGNED
