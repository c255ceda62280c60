"""GPU parity of the matrix-core batch kernel (its three instances: 16-row blocks staging 8 X
vectors for M <= 8, 16-row blocks staging 16 for larger M where 32-row blocks would split K,
32-row blocks otherwise): within tolerance of the oracle at the down_proj shape and on small
shapes that span several row blocks with a ragged last one,
unsplit and split over K; exact where every partial sum is exact (identity, one-hot, constant
W); reproducible bit for bit; unaligned calls with too few rows for the matrix-core form
of unaligned rows equal to the VALU plan; and that form itself (row classes of every
size, x at either 2-byte phase, edge-only and head-and-tail-only rows, the longest K its
depth bound allows) within tolerance of the oracle, reproducible, and not the VALU run."""
import numpy as np
import pytest
import torch

import bandwidth_bound_decode_amd as bbd
from gpu_helpers import bits_equal, device_matrix, draw, gemv, oracle_check, output

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("m", [8, 12, 16])
def test_down_proj_batches(m):
    """Full size: M = 8 and 12 on the 16-row form (unsplit; 8 and 16 X vectors), M = 16 on
    the 32-row form (two slices and the combine)."""
    w, x = draw(4096, 14336, m, seed=300 + m)
    W, X = device_matrix(w), device_matrix(x)
    Y, p = gemv(W, X)
    want = (16, 1) if m <= 14 else (32, 2)
    assert p.info["mfma"] == 1 and (p.info["mfma_rows"], p.info["mfma_splits"]) == want, p.info
    oracle_check(W, X, Y, f"mfma down m={m}")
    Y2, _ = gemv(W, X, plan=p)
    assert bits_equal(Y, Y2), "not reproducible"


@pytest.mark.parametrize("n,k", [(300, 5120), (33, 4096), (8200, 1024), (1, 64), (47, 192)])
def test_shapes_every_batch(n, k):
    """Ragged row blocks, one slice and split slices (the combine), every M from 2."""
    for m in range(2, 17):
        w, x = draw(n, k, m, seed=n + k + m)
        W, X = device_matrix(w), device_matrix(x)
        p = bbd.Plan(n, k, m, mfma=1)
        assert p.info["mfma"] == 1
        Y, _ = gemv(W, X, plan=p)
        oracle_check(W, X, Y, f"mfma n={n} k={k} m={m} S={p.info['mfma_splits']}")
        Y2, _ = gemv(W, X, plan=p)         # the tickets were left at zero for this call
        assert bits_equal(Y, Y2), f"n={n} k={k} m={m} not reproducible"


@pytest.mark.parametrize("m,rows", [(16, 32), (16, 16), (8, 16)])
def test_identity_and_one_hot_exact(m, rows):
    """Every form: K a multiple of 128 takes the 16-row form at these sizes, K = 576 and 4160
    (64 past a multiple of 128) the 32-row one. One-hot columns sit at the ends of K, on
    MFMA, piece and line edges of a chunk and on slice boundaries."""
    n = k = 512 if rows == 16 else 576
    _, x = draw(1, k, m, seed=7)
    eye = torch.eye(n, dtype=torch.bfloat16)
    Y, p = gemv(device_matrix(eye), device_matrix(x), mfma=1)
    assert p.info["mfma"] == 1 and p.info["mfma_rows"] == rows
    assert bits_equal(Y, x.float()), "W = I must return X exactly"
    kw = 4096 if rows == 16 else 4160
    w, _ = draw(300, kw, 1, seed=8)
    if rows == 32:       # 64-element chunks, slices of 576
        cols = [0, 1, 31, 32, 63, 64, 575, 576, 2047, 2048, 4032, 4159, 7, 100, 3000, 4158]
    else:                # 128-element chunks, slices of 1024 (both lines, every MFMA and piece)
        cols = [0, 33, 71, 127, 128, 1023, 2050, 4095, 1, 32, 64, 96, 1024, 3968, 2048, 2047]
    xo = torch.zeros(m, kw, dtype=torch.bfloat16)
    for i in range(m):
        xo[i, cols[i]] = 1.0
    Y, p = gemv(device_matrix(w), device_matrix(xo), mfma=1)
    assert p.info["mfma_rows"] == rows and p.info["mfma_splits"] > 1, p.info
    for i in range(m):
        assert bits_equal(Y[i], w[:, cols[i]].float()), f"one-hot column {cols[i]}"


def test_constant_w_exact():
    """W = 2^-6 and x in {-2..2}: every partial sum is an exact fp32 value in any order."""
    n, k, m = 300, 5120, 16
    w = torch.full((n, k), 2.0 ** -6, dtype=torch.bfloat16)
    rng = np.random.default_rng(n + k)
    xi = rng.integers(-2, 3, size=(m, k))
    x = torch.from_numpy(xi.astype(np.float32)).to(torch.bfloat16)
    Y, _ = gemv(device_matrix(w), device_matrix(x), mfma=1)
    want = torch.from_numpy((2.0 ** -6 * xi.sum(axis=1)).astype(np.float32))
    assert bits_equal(Y, want[:, None].expand(m, n))


def test_accumulator_rounded_once_per_mfma():
    """Pin of the depth model: the running accumulator enters an MFMA's sum once, not ahead
    of each product. K = 64 is one chunk (two MFMAs in order on one wave): the first gives
    exactly 1.0, the second adds 32 products of 2^-25. Summed exactly that is 1 + 2^-20; an
    accumulator rounded after every product would stay at 1.0."""
    n, k, m = 16, 64, 16
    w = torch.zeros(n, k, dtype=torch.bfloat16)
    w[:, 0] = 1.0
    w[:, 32:] = 2.0 ** -25
    x = torch.ones(m, k, dtype=torch.bfloat16)
    Y, p = gemv(device_matrix(w), device_matrix(x), mfma=1)
    assert p.info["mfma"] == 1 and p.info["mfma_splits"] == 1
    assert bits_equal(Y, torch.full((m, n), 1.0 + 2.0 ** -20)), Y[0, :4].tolist()


@pytest.mark.parametrize("m,k,rows", [(9, 1024, 16), (8, 1024, 16), (16, 1088, 32)])
def test_special_values(m, k, rows):
    n = 64
    w, x = draw(n, k, m, seed=10)
    w[3, 17] = float("inf")
    w[5, 900] = float("nan")
    x[:, 17] = 1.0
    Y, p = gemv(device_matrix(w), device_matrix(x), mfma=1)
    assert p.info["mfma_rows"] == rows, p.info
    assert torch.isinf(Y[:, 3]).all() and torch.isnan(Y[:, 5]).all()
    keep = [i for i in range(n) if i not in (3, 5)]
    assert torch.isfinite(Y[:, keep]).all()


@pytest.mark.parametrize("m", [8, 16])
def test_accumulator_rounded_once_per_mfma_narrow(m):
    """The same pin on the 16-row form (8 and 16 X vectors): K = 128 is one chunk, four MFMAs
    in order on one wave; the first gives exactly 1.0 and each later one adds 32 products of
    2^-25."""
    n, k = 16, 128
    w = torch.zeros(n, k, dtype=torch.bfloat16)
    w[:, 0] = 1.0
    w[:, 32:] = 2.0 ** -25
    x = torch.ones(m, k, dtype=torch.bfloat16)
    Y, p = gemv(device_matrix(w), device_matrix(x), mfma=1)
    assert (p.info["mfma_rows"], p.info["mfma_splits"]) == (16, 1), p.info
    assert bits_equal(Y, torch.full((m, n), 1.0 + 3 * 2.0 ** -20)), Y[0, :4].tolist()


def test_unaligned_call_takes_the_valu_kernels():
    n, k, m = 100, 2048, 16
    w, x = draw(n, k, m, seed=11)
    W = device_matrix(w, ld=2056, offset=1)          # rows not 16-byte aligned
    X = device_matrix(x)
    p = bbd.Plan(n, k, m)
    assert p.info["mfma"] == 1
    Y, _ = gemv(W, X, plan=p)
    oracle_check(W, X, Y, "unaligned fallback")
    Yv, _ = gemv(W, X, mfma=-1)
    assert bits_equal(Y, Yv), "fallback differs from the VALU plan"


# n, k, m, ldw, W offset, ldx, X offset (elements): 8 / gcd(ldw, 8) row classes, x phases
UNALIGNED = [
    (4097, 14337, 16, 14337, 0, 14340, 1),   # 8 classes, class 0 one row past its tiles
    (4097, 14337, 10, 14337, 1, 14337, 0),   # x rows at alternating 2-byte phases
    (4100, 2000, 16, 2002, 1, 2005, 2),      # 4 classes
    (4160, 1024, 14, 1028, 3, 1024, 0),      # 2 classes, x on the grid
    (4096, 4096, 16, 4096, 1, 4096, 0),      # 1 class, every row 7 elements off the grid
    (4096, 4096, 15, 4096, 0, 4096, 1),      # W on the grid, x off it: first chunk apart
    (4099, 100, 16, 101, 1, 103, 1),         # no whole chunk: edge and ragged chunks only
    (4096, 13, 16, 13, 1, 13, 0),            # head and tail elements only
    (4096, 29000, 13, 29001, 1, 29003, 1),   # depth bound 160, the longest allowed
]


@pytest.mark.parametrize("n,k,m,ldw,woff,ldx,xoff", UNALIGNED)
def test_unaligned_rows_on_the_matrix_cores(n, k, m, ldw, woff, ldx, xoff):
    """Rows off the 16-byte grid, M >= 10 by default: the class-tiled matrix-core kernel."""
    what = f"unaligned mfma n={n} k={k} m={m} ldw={ldw} offsets {woff}/{xoff}"
    print(what, flush=True)
    w, x = draw(n, k, m, seed=n + k + m)
    W = device_matrix(w, ld=ldw, offset=woff)
    X = device_matrix(x, ld=ldx, offset=xoff)
    p = bbd.Plan(n, k, m)
    assert 0 < p.info["mfma_unaligned_depth"] <= 160, p.info
    Y, _ = gemv(W, X, plan=p)
    oracle_check(W, X, Y, what)
    Y2, _ = gemv(W, X, plan=p)
    assert bits_equal(Y, Y2), "not reproducible"
    Yv, pv = gemv(W, X, mfma=-1)
    assert pv.info["mfma_unaligned_depth"] == 0
    oracle_check(W, X, Yv, what + " (VALU)")
    if k >= 1024:   # another summation order: some outputs round differently
        assert not bits_equal(Y, Yv), "the matrix-core kernel did not run"


def test_unaligned_rows_through_every_entry_point():
    """The same unaligned batch through gemv_run (with a strided Y), gemv_fused_run with one
    segment and gemv_run_static (no workspace): all run the matrix-core kernel for unaligned
    rows and agree bit for bit."""
    n, k, m = 4100, 6001, 12
    w, x = draw(n, k, m, seed=4242)
    W = device_matrix(w, ld=6003, offset=1)
    X = device_matrix(x, ld=6005, offset=1)
    p = bbd.Plan(n, k, m)
    assert p.info["mfma_unaligned_depth"] > 0, p.info
    Y, _ = gemv(W, X, plan=p, ldy=n + 5)
    oracle_check(W, X, Y, "unaligned mfma, strided Y")
    Yf = output(m, n)
    bbd.fused_run(p, [(W, Yf)], X, p.alloc_workspace())
    Ys = output(m, n)
    bbd.run_static(p, W, X, Ys)
    torch.cuda.synchronize()
    assert bits_equal(Yf, Y), "fused run differs"
    assert bits_equal(Ys, Y), "static run differs"
    Yv, _ = gemv(W, X, mfma=-1)
    assert not bits_equal(Y, Yv), "the matrix-core kernel did not run"
