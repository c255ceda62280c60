"""GPU parity of skinny batches (M = 1..16): within tolerance of the oracle, and, on the VALU
kernels, every row of Y bitwise equal to the batch-1 run on that row of X (their split count
and per-row summation order do not depend on M). Plans that take the matrix-core kernel
(M >= 2 with K a multiple of 64) meet the tolerance in another summation order; the
invariance is checked on the same inputs with that kernel switched off."""
import pytest
import torch

import bandwidth_bound_decode_amd as bbd
import workloads
from gpu_helpers import bits_equal, device_matrix, draw, gemv, oracle_check

pytestmark = pytest.mark.gpu


def rows_match_batch_one(W, X, Y):
    for i in range(X.shape[0]):
        y1, _ = gemv(W, X[i:i + 1])
        assert bits_equal(Y[i:i + 1], y1), f"batch row {i} differs from its batch-1 run"


def test_skinny_config():
    cfg = workloads.SKINNY_BATCH
    for g, (w, x) in zip(cfg.gemvs, workloads.draw_config(cfg)):
        W, X = device_matrix(w), device_matrix(x)
        Y, p = gemv(W, X)
        print(g.name, p.info, flush=True)
        oracle_check(W, X, Y, g.name)
        if p.info["mfma"]:
            Y, _ = gemv(W, X, mfma=-1)
            oracle_check(W, X, Y, g.name + " (VALU)")
        rows_match_batch_one(W, X, Y)


@pytest.mark.parametrize("m", range(1, 17))
def test_every_batch_size(m):
    n, k = 300, 5000
    w, x = draw(n, k, m, seed=100 + m)
    W, X = device_matrix(w), device_matrix(x)
    Y, _ = gemv(W, X)
    oracle_check(W, X, Y, f"m={m}")
    rows_match_batch_one(W, X, Y)


@pytest.mark.parametrize("m", [2, 3, 7, 16])
def test_batch_unaligned(m):
    n, k = 45, 3001
    w, x = draw(n, k, m, seed=200 + m)
    W = device_matrix(w, ld=3003, offset=1)
    X = device_matrix(x, ld=3005, offset=3)
    Y, _ = gemv(W, X)
    oracle_check(W, X, Y, f"unaligned m={m}")
    rows_match_batch_one(W, X, Y)


@pytest.mark.parametrize("m,ldw", [(5, 14339), (9, 14340), (16, 14337)])
def test_batch_unaligned_chunked(m, ldw):
    """Unaligned rows whose M shifted x rows exceed the LDS the kernel stages them in: x goes
    through in chunks, and every row of Y still equals its batch-1 run bitwise."""
    n, k = 37, 14337
    w, x = draw(n, k, m, seed=300 + m)
    W = device_matrix(w, ld=ldw, offset=1)
    X = device_matrix(x, ld=k + 3, offset=3)
    Y, _ = gemv(W, X)
    oracle_check(W, X, Y, f"unaligned chunked m={m}")
    rows_match_batch_one(W, X, Y)


@pytest.mark.parametrize("m", [1, 3, 7])
def test_batch_unaligned_many_rows(m):
    """More unaligned row blocks than the device holds at once: workgroups loop over row
    blocks with x staged once, and the results are those of the oracle."""
    n, k = 200_000, 301
    w, x = draw(n, k, m, seed=400 + m)
    W = device_matrix(w, ld=303, offset=1)
    X = device_matrix(x, ld=k + 1, offset=1)
    Y, _ = gemv(W, X)
    oracle_check(W, X, Y, f"unaligned many rows m={m}")
    rows_match_batch_one(W, X, Y)


@pytest.mark.parametrize("n,m", [(63, 1), (63, 3), (63, 6), (135, 1), (135, 3), (135, 6),
                                 (4097, 1), (4097, 3), (4097, 6), (4097, 16)])
def test_unaligned_tail_rows(n, m):
    """Rows of a row class past its last whole group of 8 are summed by a whole workgroup
    with K split over its waves: 63 rows in 8 classes leave one class of 7 rows (all tail
    rows) beside classes of 8, 135 rows one tail row in seven classes, 4097 one in class 0.
    Oracle parity and, since which rows are tail rows does not depend on M, every batch row
    bitwise equal to its batch-1 run; with x staged in chunks at M = 16 (the matrix cores,
    which take such calls from M = 10 by default, switched off)."""
    k = 2001 if m < 16 else 9001
    w, x = draw(n, k, m, seed=500 + n + m)
    W = device_matrix(w)                 # ldw = k, odd: every row at another 2-byte offset
    X = device_matrix(x, ld=k + 3, offset=1)
    Y, p = gemv(W, X, mfma=-1)
    assert p.info["splits"] == 1
    oracle_check(W, X, Y, f"unaligned tail rows n={n} m={m}")
    rows_match_batch_one(W, X, Y)
