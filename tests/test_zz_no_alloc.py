"""GPU tests of gemv_run_static, the entry point that allocates nothing: its split partial sums
and tickets live in the library's static per-GPU scratch array. Each call goes through the C
ABI and is compared with gemv_run on the same plan and inputs (bitwise) and with the fp64
oracle, on consecutive calls whose second input is smaller."""
import pytest
import torch

import bandwidth_bound_decode_amd as bbd
from gpu_helpers import bits_equal, device_matrix, draw, oracle_check, output

pytestmark = pytest.mark.gpu


def with_workspace(plan, W, X):
    Y = output(plan.m, plan.n)
    bbd.run(plan, W, X, Y, plan.alloc_workspace())
    return Y


def static(plan, W, X, stream=None):
    Y = output(plan.m, plan.n)
    bbd.run_static(plan, W, X, Y, stream)
    return Y


# (n, k, m, forced splits): a matrix-core batch split in two, a batch-1 VALU split, an
# unsplit batch-1 call (no scratch), a ragged split, then smaller inputs of the same kinds.
CASES = [(4096, 14336, 16, 0), (64, 14336, 1, 0), (1024, 4096, 1, 0), (300, 5000, 3, 4),
         (520, 2048, 8, 0), (33, 1000, 1, 3), (7, 129, 1, 2)]


def test_static_equals_workspace_run_on_consecutive_calls():
    """Every case twice in a row through gemv_run_static, each bitwise equal to gemv_run with
    a workspace of its own and within tolerance of the oracle; sizes shrink along the list,
    so later calls reuse scratch that larger calls left behind."""
    drawn = []
    for i, (n, k, m, splits) in enumerate(CASES):
        w, x = draw(n, k, m, seed=300 + i)
        W, X = device_matrix(w), device_matrix(x)
        plan = bbd.Plan(n, k, m, splits=splits)
        ws_size = plan.workspace_size
        assert ws_size <= 4 << 20
        drawn.append((plan, W, X))
        ref = with_workspace(plan, W, X)
        for rep in range(2):
            got = static(plan, W, X)
            torch.cuda.synchronize()
            info = plan.info
            what = f"{n}x{k} m={m} S={info['splits']} mfma S={info['mfma_splits']} call {rep}"
            assert bits_equal(got, ref), what
            oracle_check(W, X, got, what)
    # interleaved: plans alternate, every call still bitwise equal to its workspace run
    for rep in range(2):
        for plan, W, X in drawn:
            assert bits_equal(static(plan, W, X), with_workspace(plan, W, X))
    assert any(p.info["splits"] > 1 for p, _, _ in drawn)
    assert any(p.info["mfma_splits"] > 1 for p, _, _ in drawn)


def test_static_calls_captured_in_a_graph():
    """Static calls recorded into one graph (no allocation during capture): every replay,
    with eager calls of other plans on the same stream in between, equals the eager run."""
    stream = torch.cuda.Stream()
    calls = []
    for i, (n, k, m, splits) in enumerate([(4096, 14336, 16, 0), (64, 14336, 1, 0),
                                           (300, 5000, 3, 4)]):
        w, x = draw(n, k, m, seed=400 + i)
        W, X = device_matrix(w), device_matrix(x)
        plan = bbd.Plan(n, k, m, splits=splits)
        calls.append((plan, W, X, output(m, n)))
    with torch.cuda.stream(stream):
        for plan, W, X, Y in calls:
            bbd.run_static(plan, W, X, Y, stream)
    stream.synchronize()
    eager = [Y.clone() for _, _, _, Y in calls]
    g = bbd.Graph(stream)
    with torch.cuda.stream(stream):
        with g:
            for plan, W, X, Y in calls:
                bbd.run_static(plan, W, X, Y, stream)
    other_w, other_x = draw(520, 2048, 8, seed=499)
    OW, OX = device_matrix(other_w), device_matrix(other_x)
    other = bbd.Plan(520, 2048, 8)
    for rep in range(3):
        for _, _, _, Y in calls:
            Y.fill_(float("nan"))
        with torch.cuda.stream(stream):
            OY = static(other, OW, OX, stream)      # eager static call between replays
        g.launch(stream)
        stream.synchronize()
        for (plan, W, X, Y), ref in zip(calls, eager):
            assert bits_equal(Y, ref), f"replay {rep}: {plan.n}x{plan.k}"
        oracle_check(OW, OX, OY, "eager static call between replays")
    g.destroy()


def test_static_refuses_plans_beyond_the_scratch():
    """A split plan whose partial sums exceed the static array is refused before launch;
    the same plan still runs through gemv_run with a workspace of its own."""
    plan = bbd.Plan(40000, 14336, 16, splits=2, mfma=-1)   # 2 x 16 x 40000 x 4 B = 5.1 MB
    assert plan.workspace_size > 4 << 20
    W = torch.zeros((40000, 14336), dtype=torch.bfloat16, device="cuda")
    X = torch.zeros((16, 14336), dtype=torch.bfloat16, device="cuda")
    Y = torch.empty((16, 40000), dtype=torch.float32, device="cuda")
    with pytest.raises(bbd.GemvError) as e:
        bbd.run_static(plan, W, X, Y)
    assert e.value.status == bbd.Status.WORKSPACE
