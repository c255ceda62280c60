"""GPU parity of gemv_fused_run (fused QKV and gate_up): bitwise equal to gemv_run on the
row-concatenated weight on the same VALU kernels, and within tolerance of the oracle."""
import pytest
import torch

import bandwidth_bound_decode_amd as bbd
import workloads
from gpu_helpers import bits_equal, device_matrix, draw, oracle_check, output

pytestmark = pytest.mark.gpu


def fused_vs_concat(parts, x, ldws=None, ldys=None):
    n = sum(p.shape[0] for p in parts)
    k = x.shape[1]
    m = x.shape[0]
    ldws = ldws or [None] * len(parts)
    ldys = ldys or [None] * len(parts)
    Ws = [device_matrix(p, ld=ld) for p, ld in zip(parts, ldws)]
    X = device_matrix(x)
    plan = bbd.Plan(n, k, m)
    ws = plan.alloc_workspace()
    Ys = [output(m, p.shape[0], ld) for p, ld in zip(parts, ldys)]
    bbd.fused_run(plan, list(zip(Ws, Ys)), X, ws)
    Wcat = device_matrix(torch.cat(parts, 0))
    # A fused call always runs the VALU kernels the plan describes; a single-matrix batch
    # call of the same plan may take the matrix-core kernel, so the bitwise reference is
    # the concatenated run with that kernel switched off (the same VALU tile).
    ref_plan = plan
    if plan.info["mfma"]:
        ref_plan = bbd.Plan(n, k, m, mfma=-1)
        for key in ("splits", "rows_per_wave", "waves_per_block", "unroll", "slice"):
            assert ref_plan.info[key] == plan.info[key], key
        Ymf = output(m, n)
        bbd.run(plan, Wcat, X, Ymf, ws)
        torch.cuda.synchronize()
        oracle_check(Wcat, X, Ymf, f"concatenated, matrix cores, n={n} k={k}")
    Ycat = output(m, n)
    bbd.run(ref_plan, Wcat, X, Ycat, ref_plan.alloc_workspace())
    torch.cuda.synchronize()
    got = torch.cat([y for y in Ys], 1)
    assert bits_equal(got, Ycat), "fused result differs from the concatenated run"
    oracle_check(Wcat, X, got, f"fused n={n} k={k}")
    return plan


def test_qkv_and_gate_up():
    cfg = workloads.FUSED_PROJECTIONS
    for g, (w, x) in zip(cfg.gemvs, workloads.draw_config(cfg)):
        parts = list(torch.split(w, list(g.segments), 0))
        plan = fused_vs_concat(parts, x)
        print(g.name, plan.info, flush=True)


def test_strided_segments_and_odd_sizes():
    k = 4096
    sizes = [5, 100, 1, 1000]
    parts = [draw(s, k, 1, seed=s)[0] for s in sizes]
    x = draw(1, k, 1, seed=99)[1]
    fused_vs_concat(parts, x, ldws=[4096, 4104, 4096, 4160], ldys=[8, 100, 4, 1000])


def test_fused_batch():
    k = 2048
    parts = [draw(s, k, 1, seed=s)[0] for s in (64, 33)]
    x = draw(1, k, 5, seed=7)[1]
    fused_vs_concat(parts, x, ldys=[70, 40])
