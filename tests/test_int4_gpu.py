"""GPU parity of the INT4-weight GEMV (batch 1) against the fp64 INT4 oracle: the Llama
projection shapes at full size, small and ragged shapes (a short last group, one vector per
row), padded strides whose padding would poison the result if read, exact cases,
reproducibility, every compiled burst length bitwise equal, graph replay, and the calls the
library must refuse."""
import numpy as np
import pytest
import torch

import bandwidth_bound_decode_amd as bbd
import oracle
import workloads
from gpu_helpers import bits_equal, host_bits

pytestmark = pytest.mark.gpu


def draw(n, k, seed, **kw):
    packed, scales, q = workloads.draw_int4(n, k, workloads.generator(seed), **kw)
    x = workloads.bf16_normal((1, k), workloads.SIGMA_X, workloads.generator(seed + 1))
    return packed, scales, q, x


def run(packed, scales, x, plan=None, **opts):
    n, k = packed.shape[0], x.shape[1]
    p = plan or bbd.Plan(n, k, 1, weights="int4", **opts)
    Wq, S, X = packed.cuda(), scales.cuda(), x.cuda()
    Y = torch.full((1, n), float("nan"), dtype=torch.float32, device="cuda")
    bbd.run_int4(p, Wq, S, X, Y)
    torch.cuda.synchronize()
    return Y, p


def check(packed, scales, x, Y, what):
    y_ref, s_abs = oracle.gemv_q4(packed.cpu().numpy(), host_bits(scales), host_bits(x))
    rep = oracle.check(Y.cpu().numpy(), y_ref, s_abs)
    assert rep.ok, f"{what}: {rep}"
    return rep


@pytest.mark.parametrize("n,k", [(4096, 14336), (1024, 4096), (6144, 4096), (4096, 4096),
                                 (28672, 4096), (128256, 4096)])
def test_llama_shapes(n, k):
    packed, scales, _, x = draw(n, k, seed=n + k)
    Y, p = run(packed, scales, x)
    print(n, k, p.info, flush=True)
    check(packed, scales, x, Y, f"int4 {n}x{k}")


TILES = [dict(), dict(unroll=1), dict(unroll=2, rows_per_wave=1, waves_per_block=1),
         dict(unroll=4, rows_per_wave=1, waves_per_block=8), dict(unroll=1, rows_per_wave=2),
         dict(unroll=2, rows_per_wave=2, waves_per_block=2),
         dict(unroll=2, rows_per_wave=1, waves_per_block=16),
         # capped grids: workgroups loop over row blocks (their LDS holds only the staged x)
         dict(unroll=2, rows_per_wave=1, waves_per_block=8, waves_per_cu=8),
         dict(unroll=1, rows_per_wave=2, waves_per_block=16, waves_per_cu=16)]


@pytest.mark.parametrize("n,k", [(7, 128), (33, 1024), (300, 4128), (64, 32), (5, 96),
                                 (129, 2080), (37, 36864)])
def test_small_and_ragged(n, k):
    """Ragged row blocks, a short last group, one vector per row, and x too long for LDS
    (K = 36864), on every compiled tile."""
    packed, scales, _, x = draw(n, k, seed=3 * n + k)
    for opts in TILES:
        Y, p = run(packed, scales, x, **opts)
        check(packed, scales, x, Y, f"int4 {n}x{k} {opts} lds={p.info['lds_bytes']}")


@pytest.mark.parametrize("form", [-1, 1])
def test_padded_strides_and_every_tile_same_bits(form):
    """Every compiled tile gives the same bits for one staging form of x (bf16: -1, fp16:
    1), reproducibly; padding (0xEE bytes, NaN scales) is never read."""
    n, k = 100, 4128
    packed, scales, _, x = draw(n, k, seed=5, ldq=2096, lds=40)
    ref = None
    for opts in TILES:
        Y, p = run(packed, scales, x, int4_fp16=form, **opts)
        assert p.info["int4_fp16"] == (form > 0)
        check(packed, scales, x, Y, f"padded {opts} form {form}")
        if ref is None:
            ref = Y
        assert bits_equal(Y, ref), f"{opts} differs"
        Y2, _ = run(packed, scales, x, int4_fp16=form, **opts)
        assert bits_equal(Y, Y2), "not reproducible"


@pytest.mark.parametrize("n,k,form", [(4096, 14336, 1), (128256, 4096, -1), (28672, 4096, 1)])
def test_llama_shapes_other_staging_form(n, k, form):
    """The staging form the plan does not pick by default, at full size."""
    packed, scales, _, x = draw(n, k, seed=n + k)
    Y, p = run(packed, scales, x, int4_fp16=form)
    assert p.info["int4_fp16"] == (form > 0)
    check(packed, scales, x, Y, f"int4 {n}x{k} form {form}")


def test_exact_cases():
    n, k = 40, 1024
    # all-zero weights
    packed = torch.zeros((n, k // 2), dtype=torch.uint8)
    scales = torch.ones((n, k // 128), dtype=torch.bfloat16)
    _, _, _, x = draw(n, k, seed=7)
    Y, _ = run(packed, scales, x)
    assert (Y == 0).all()
    # one-hot x picks v * scale exactly, at every position in a vector and a group
    packed, scales, q, _ = draw(n, k, seed=8)
    deq = oracle.q4_dequant(packed.numpy(), host_bits(scales), k)
    for c in (0, 1, 7, 8, 31, 32, 127, 128, 511, 1023):
        xo = torch.zeros((1, k), dtype=torch.bfloat16)
        xo[0, c] = 1.0
        for form in (-1, 1):
            Y, _ = run(packed, scales, xo, int4_fp16=form)
            assert bits_equal(Y[0], torch.from_numpy(deq[:, c]).float()), \
                f"one-hot column {c}, form {form}"
    # every weight -8 with scale 2^-4 and x in {-2..2}: every partial sum is exact
    packed = torch.full((n, k // 2), 0x88, dtype=torch.uint8)
    scales = torch.full((n, k // 128), 2.0 ** -4, dtype=torch.bfloat16)
    xi = np.random.default_rng(9).integers(-2, 3, size=(1, k))
    x = torch.from_numpy(xi.astype(np.float32)).to(torch.bfloat16)
    want = float(-8 * 2.0 ** -4 * xi.sum())
    for form in (-1, 1):
        Y, _ = run(packed, scales, x, int4_fp16=form)
        assert bits_equal(Y, torch.full((1, n), want)), (form, Y[0, :3].tolist())


@pytest.mark.parametrize("case", ["wide_range", "tiny_odd", "all_subnormal", "one_huge",
                                  "boundary"])
def test_x_staging_paths(case):
    """x whose elements cannot all be staged as exact normal fp16 at one power-of-two scale
    sends the workgroups to the bf16 form, and x that can takes the fp16 form; both must
    meet the oracle, and the fp16 form must agree exactly where every sum is exact."""
    n, k = 96, 4096
    packed, scales, _, x = draw(n, k, seed=17)
    xf = x.float()
    if case == "wide_range":          # 2^40 next to O(1) values: the rest underflow in fp16
        xf[0, 5] = 2.0 ** 40
    elif case == "tiny_odd":          # an odd element 2^-26 below the largest (x 2^(s-4))
        xf[0, 1] = xf.abs().max() * 2.0 ** -26
    elif case == "all_subnormal":     # every element a bf16 subnormal
        xf = torch.sign(xf) * 2.0 ** -130
    elif case == "one_huge":          # a single huge element, zeros elsewhere: exact fp16
        xf = torch.zeros_like(xf)
        xf[0, 77] = 2.0 ** 100
    elif case == "boundary":          # smallest odd element exactly at the normal fp16 edge
        xf[0, 3] = xf.abs().max() * 2.0 ** -24
    xb = xf.to(torch.bfloat16)
    Y, _ = run(packed, scales, xb, int4_fp16=1)
    check(packed, scales, xb, Y, f"x staging {case}")
    if case == "one_huge":
        deq = oracle.q4_dequant(packed.numpy(), host_bits(scales), k)
        want = torch.from_numpy(deq[:, 77] * 2.0 ** 100).float()
        assert bits_equal(Y[0], want)


def test_graph_replay_matches_eager():
    n, k = 4096, 14336
    packed, scales, _, x = draw(n, k, seed=11)
    p = bbd.Plan(n, k, 1, weights="int4")
    Wq, S, X = packed.cuda(), scales.cuda(), x.cuda()
    Y = torch.empty((1, n), dtype=torch.float32, device="cuda")
    bbd.run_int4(p, Wq, S, X, Y)
    torch.cuda.synchronize()
    eager = Y.clone()
    stream = torch.cuda.Stream()
    Yg = torch.full((1, n), float("nan"), dtype=torch.float32, device="cuda")
    with bbd.Graph(stream) as g:
        bbd.run_int4(p, Wq, S, X, Yg, stream=stream)
    for _ in range(3):
        Yg.fill_(float("nan"))
        torch.cuda.synchronize()
        g.launch()
        stream.synchronize()
        assert bits_equal(Yg, eager), "graph replay differs from eager"


def test_refused_calls():
    n, k = 64, 1024
    packed, scales, _, x = draw(n, k, seed=13, ldq=528)
    p = bbd.Plan(n, k, 1, weights="int4")
    raw = torch.zeros(n * 528 + 16, dtype=torch.uint8, device="cuda")
    Wq_mis = raw[1:1 + n * 528].view(n, 528)                 # rows not 16-byte aligned
    S, X = scales.cuda(), x.cuda()
    Y = torch.empty((1, n), dtype=torch.float32, device="cuda")
    with pytest.raises(bbd.GemvError) as e:
        bbd.run_int4(p, Wq_mis, S, X, Y)
    assert e.value.status == bbd.Status.MISALIGNED
    odd = torch.zeros((n, 520), dtype=torch.uint8, device="cuda")   # ldq not a multiple of 16
    with pytest.raises(bbd.GemvError) as e:
        bbd.run_int4(p, odd, S, X, Y)
    assert e.value.status == bbd.Status.INVALID_ARG
    pb = bbd.Plan(n, k, 1)
    with pytest.raises(bbd.GemvError):
        bbd.run_int4(pb, packed.cuda(), S, X, Y)                  # bf16 plan
    W = torch.zeros((n, k), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(bbd.GemvError):
        bbd.run(p, W, X, Y)                                       # INT4 plan on gemv_run
