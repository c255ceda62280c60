"""CPU tests of the bench's arithmetic against the pages' worked numbers, and its contract."""
import json
import os
import subprocess
import sys

import pytest

import bench
import workloads

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
GOLDEN = json.load(open(os.path.join(ROOT, "tests", "golden", "pages_worked_numbers.json")))


def close(a, b, rel=None, abs_=None):
    if rel is not None:
        return abs(a - b) <= rel * abs(b)
    return abs(a - b) <= abs_


def test_k_proj_transfer_time():
    g = GOLDEN["k_proj_transfer_h100"]
    w_bytes = 2 * g["rows"] * g["k"]
    assert close(w_bytes, g["bytes"], rel=g["bytes_rel_tol"])
    assert close(bench.seconds_at(w_bytes, g["bandwidth_B_per_s"]), g["seconds"],
                 rel=g["seconds_rel_tol"])


def test_decode_step_mbu():
    g = GOLDEN["decode_step_mbu_h100"]
    assert close(bench.mbu(g["bytes"], g["step_s"], g["bandwidth_B_per_s"]), g["mbu_printed"],
                 abs_=g["mbu_abs_tol"])
    assert close(bench.mbu(g["bytes"], g["kernel_s"], g["bandwidth_B_per_s"]),
                 g["kernel_fraction_printed"], abs_=g["kernel_fraction_abs_tol"])


def test_wave_quantization():
    g = GOLDEN["wave_quantization_h100"]
    assert bench.waves(g["tiles"], g["sms"]) == g["waves"]
    assert close(bench.wave_efficiency(g["tiles"], g["sms"]), g["efficiency"],
                 abs_=g["efficiency_abs_tol"])


def test_ridge():
    g = GOLDEN["ridge_h100"]
    assert close(bench.ridge(g["bf16_flops"], g["bandwidth_B_per_s"]), g["ridge"],
                 abs_=g["ridge_abs_tol"])


def test_algorithmic_bytes_of_the_workloads():
    import workloads
    assert bench.alg_bytes(4096, 14336) == 117_485_568
    assert bench.alg_bytes(1024, 4096) == 8_400_896
    assert bench.alg_bytes(4097, 14337, 3) == 117_612_564
    step = sum(bench.alg_bytes(g.n, g.k, g.m) for g in workloads.decode_step_gemvs())
    assert step == 15_017_047_040
    for cfg in workloads.WORKLOADS:
        for g in cfg.gemvs:
            assert g.alg_bytes == bench.alg_bytes(g.n, g.k, g.m)


def test_more_than_one_gpu_is_refused():
    proc = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                          capture_output=True, text=True, timeout=120)
    assert proc.returncode == 2
    assert "one GPU" in proc.stderr
    assert proc.stdout == ""


def test_shard_shapes_cover_the_step():
    """One GPU's shares times G give back every projection: rows for QKV, gate_up and
    lm_head (every fused segment cut alike), K for o_proj and down_proj; the per-GPU step's
    weight bytes are the full step's divided by G."""
    full = {g.name: g for g in workloads.decode_step_gemvs(1)}
    lm = workloads.decode_step_gemvs(1)[-1]
    for gpus in workloads.SHARD_GPUS:
        qkv, o, gu, down, lm_s = workloads.shard_gemvs(gpus)
        assert (qkv.n * gpus, qkv.k) == (full["L0.qkv"].n, full["L0.qkv"].k)
        assert tuple(s * gpus for s in qkv.segments) == full["L0.qkv"].segments
        assert tuple(s * gpus for s in gu.segments) == full["L0.gate_up"].segments
        assert (o.n, o.k * gpus) == (full["L0.o"].n, full["L0.o"].k)
        assert (down.n, down.k * gpus) == (full["L0.down"].n, full["L0.down"].k)
        assert (lm_s.n * gpus, lm_s.k) == (lm.n, lm.k)
        step = workloads.shard_decode_step_gemvs(gpus)
        whole = workloads.decode_step_gemvs()
        assert len(step) == len(whole) == 129
        assert sum(2 * g.n * g.k for g in step) * gpus == sum(2 * g.n * g.k for g in whole)
    with pytest.raises(ValueError):
        workloads.shard_gemvs(3)
