"""GPU parity of gemv_run against the fp64 oracle: the workload shapes, closed forms (bitwise),
a brute-force sweep over small and ragged shapes, forced split counts, every compiled tile
variant, strided and misaligned layouts, determinism, and edge cases."""
import numpy as np
import pytest
import torch

import bandwidth_bound_decode_amd as bbd
import workloads
from gpu_helpers import (DEV, bits_equal, device_matrix, draw, gemv, host_bits, oracle_check,
                         output)

pytestmark = pytest.mark.gpu

ONE = 0x3F80
C_2M6 = 0x3C80          # 2^-6


def bf16_from_bits(bits) -> torch.Tensor:
    return torch.from_numpy(np.asarray(bits, dtype=np.uint16).view(np.int16).copy()).view(
        torch.bfloat16)


def small_ints(shape, seed):
    """x in {-2, ..., 2} as bf16, plus the integers."""
    rng = np.random.default_rng(seed)
    xi = rng.integers(-2, 3, size=shape)
    return torch.from_numpy(xi.astype(np.float32)).to(torch.bfloat16), xi


# ---------------------------------------------------------------------------- workloads
def test_k_proj_and_tails():
    """k_proj 1024x4096 with tails 7x129 and 33x1000, drawn in order from seed 1000."""
    cfg = workloads.K_PROJ_AND_TAILS
    for g, (w, x) in zip(cfg.gemvs, workloads.draw_config(cfg)):
        W, X = device_matrix(w), device_matrix(x)
        Y, p = gemv(W, X)
        print(g.name, p.info, flush=True)
        oracle_check(W, X, Y, g.name)


def test_down_proj_full_size():
    """The split-K stress shape, 4096x14336, in the launch configuration the bench times."""
    cfg = workloads.DOWN_PROJ
    (w, x), = workloads.draw_config(cfg)
    W, X = device_matrix(w), device_matrix(x)
    Y, p = gemv(W, X)
    oracle_check(W, X, Y, "down 4096x14336")
    Y2, _ = gemv(W, X, plan=p)
    assert bits_equal(Y, Y2), "two runs of one plan differ"


@pytest.mark.parametrize("name,n,k,unroll", [("o_proj", 4096, 4096, 2),
                                              ("lm_head", workloads.VOCAB, workloads.HIDDEN, 8)])
def test_single_matrix_decode_shapes_full_size(name, n, k, unroll):
    """The single-matrix K = 4096 decode shapes at full size, every output against the
    oracle: o_proj 4096x4096 (bursts of 2 steps: 16 waves per CU in one round) and the
    128256-row lm_head (one burst per row), in the plans the bench and the decode step use."""
    g = workloads.Gemv(name, n, k)
    w, x = workloads.draw_gemv(g, workloads.generator(8 if name == "lm_head" else 7, DEV), DEV)
    p = bbd.Plan(n, k, 1)
    info = p.info
    assert (info["splits"], info["rows_per_wave"], info["unroll"]) == (1, 1, unroll), info
    Y, _ = gemv(w, x, plan=p)
    rep = oracle_check(w, x, Y, f"{name} {n}x{k}")
    print(f"{name} {n}x{k}: {rep}", flush=True)
    Y2, _ = gemv(w, x, plan=p)
    assert bits_equal(Y, Y2), "two runs of one plan differ"


# ---------------------------------------------------------------------------- closed forms
@pytest.mark.parametrize("n", [129, 4096])
def test_identity_bitwise(n):
    w = torch.eye(n, dtype=torch.bfloat16)
    _, x = draw(1, n, 1, seed=n)
    W, X = device_matrix(w), device_matrix(x)
    Y, _ = gemv(W, X)
    assert bits_equal(Y, x.float()), "W = I must return x exactly"


@pytest.mark.parametrize("n,k,splits", [(1024, 4096, 0), (1024, 4096, 1), (1024, 4096, 3),
                                        (33, 1000, 2), (7, 129, 0), (64, 14337, 6)])
def test_one_hot_bitwise(n, k, splits):
    w, _ = draw(n, k, 1, seed=k)
    W = device_matrix(w)
    p = bbd.Plan(n, k, 1, splits=splits)
    slice_ = p.info["slice"]
    cols = {0, 1, 7, 8, 9, 511, 512, k // 2, k - 9, k - 8, k - 2, k - 1}
    for s in range(1, p.info["splits"]):
        cols |= {s * slice_ - 1, s * slice_}          # both sides of every split boundary
    cols = sorted(c for c in cols if 0 <= c < k)
    for c in cols:
        x = torch.zeros(1, k, dtype=torch.bfloat16)
        x[0, c] = 1.0
        Y, _ = gemv(W, device_matrix(x), plan=p)
        assert bits_equal(Y[0], w[:, c].float()), f"one-hot column {c} (n={n} k={k} S={splits})"


@pytest.mark.parametrize("n,k,m,splits", [(33, 1000, 1, 0), (4096, 14336, 1, 0),
                                          (4096, 14336, 1, 16), (7, 129, 1, 0),
                                          (4097, 14337, 3, 0), (300, 5000, 16, 3)])
def test_constant_w_bitwise(n, k, m, splits):
    """W = 2^-6 everywhere and x in {-2..2}: every partial sum is exact in fp32."""
    w = torch.full((n, k), 2.0 ** -6, dtype=torch.bfloat16)
    x, xi = small_ints((m, k), seed=n + k)
    Y, _ = gemv(device_matrix(w), device_matrix(x), splits=splits)
    want = torch.from_numpy((2.0 ** -6 * xi.sum(axis=1)).astype(np.float32))
    assert bits_equal(Y, want[:, None].expand(m, n)), f"constant W {n}x{k}x{m} S={splits}"


# ---------------------------------------------------------------------------- sweeps
SWEEP_K = sorted(set(list(range(1, 18)) + [31, 32, 33, 63, 64, 65, 127, 128, 129, 255, 256, 257,
                                           300, 511, 512, 513, 1023, 1024, 1025, 2049, 4100]))
SWEEP_N = [1, 2, 3, 5, 8, 17, 33, 40]


def test_brute_force_sweep():
    """Every K residue mod 8 and around each wave-step boundary, several N, the auto plan."""
    fails = []
    for n in SWEEP_N:
        for k in SWEEP_K:
            w, x = draw(n, k, 1, seed=7 * n + k)
            W, X = device_matrix(w), device_matrix(x)
            Y, _ = gemv(W, X)
            try:
                oracle_check(W, X, Y, f"n={n} k={k}")
            except AssertionError as e:
                fails.append(str(e))
    assert not fails, fails[:5]


def test_unaligned_layouts():
    """Row strides that are not multiples of 8 and base offsets that break 16-byte alignment
    run the unaligned path; the result must still meet the tolerance."""
    cases = [(7, 129, 1, 129, 0, 0), (33, 1000, 1, 1001, 0, 0), (33, 1000, 1, 1000, 3, 0),
             (40, 300, 2, 303, 1, 5), (5, 17, 3, 19, 7, 2), (64, 4100, 4, 4101, 2, 1),
             (17, 2049, 16, 2049, 0, 3), (4097, 14337, 3, 14337, 0, 0)]
    for n, k, m, ldw, woff, xoff in cases:
        w, x = draw(n, k, m, seed=n * k)
        W = device_matrix(w, ld=ldw, offset=woff)
        X = device_matrix(x, ld=k + (1 if m > 1 else 0), offset=xoff)
        Y, _ = gemv(W, X)
        oracle_check(W, X, Y, f"unaligned n={n} k={k} m={m} ldw={ldw} woff={woff} xoff={xoff}")


@pytest.mark.parametrize("n,k", [(1024, 4096), (4096, 14336), (33, 1000), (40, 2049)])
def test_forced_split_counts(n, k):
    w, x = draw(n, k, 1, seed=n + 3 * k)
    W, X = device_matrix(w), device_matrix(x)
    accepted = 0
    for s in (1, 2, 3, 4, 7, 16):
        try:
            p = bbd.Plan(n, k, 1, splits=s)
        except bbd.GemvError as e:
            assert e.status == bbd.Status.INVALID_ARG     # a slice would be empty
            continue
        accepted += 1
        Y, _ = gemv(W, X, plan=p)
        oracle_check(W, X, Y, f"n={n} k={k} S={s}")
        Y2, _ = gemv(W, X, plan=p)
        assert bits_equal(Y, Y2), f"S={s} not reproducible"
    assert accepted >= 4


def test_every_variant_same_bits():
    """The per-row summation order depends only on the K slice, so every compiled
    (rows per wave, unroll, waves per block) gives bitwise the same Y for a fixed split."""
    from bandwidth_bound_decode_amd._binding import lib  # noqa: F401  (loaded library)
    n, k = 300, 5000
    for m in (1, 2, 3, 8, 16):
        w, x = draw(n, k, m, seed=m)
        W, X = device_matrix(w), device_matrix(x)
        ref = None
        for r in (1, 2, 4):
            for u in (2, 4, 7, 8, 14):
                for waves in (1, 4, 8):
                    try:
                        p = bbd.Plan(n, k, m, splits=2, rows_per_wave=r, unroll=u,
                                     waves_per_block=waves)
                    except bbd.GemvError:
                        continue
                    Y, _ = gemv(W, X, plan=p)
                    if ref is None:
                        ref = Y
                        oracle_check(W, X, Y, f"m={m} r={r} u={u}")
                    assert bits_equal(Y, ref), f"m={m} r={r} u={u} waves={waves}"


# ---------------------------------------------------------------------------- layouts
def test_strided_output_and_padding_untouched():
    n, k, m = 100, 3000, 4
    w, x = draw(n, k, m, seed=5)
    W = device_matrix(w, ld=3008)
    X = device_matrix(x, ld=3016)
    Y, _ = gemv(W, X, ldy=104)
    oracle_check(W, X, Y, "strided")
    full = Y.as_strided((m, 104), (104, 1))
    assert torch.isnan(full[:, n:]).all(), "a store landed in Y's padding"


def test_misaligned_pointers_rejected():
    w, x = draw(8, 64, 1, seed=1)
    W, X = device_matrix(w), device_matrix(x)
    p = bbd.Plan(8, 64, 1)
    Y = output(1, 8)
    raw = torch.empty(64, dtype=torch.uint8, device="cuda")
    odd = raw.data_ptr() + 1                     # not 2-byte aligned
    st = bbd.lib().gemv_run(p.handle, odd, 64, X.data_ptr(), 64, Y.data_ptr(), 8, None, 0, None)
    assert st == bbd.Status.MISALIGNED
    st = bbd.lib().gemv_run(p.handle, W.data_ptr(), 64, X.data_ptr(), 64, Y.data_ptr() + 2, 8,
                            None, 0, None)
    assert st == bbd.Status.MISALIGNED
    torch.cuda.synchronize()
    assert torch.isnan(Y).all(), "a rejected call must enqueue nothing"


def test_workspace_checks_on_device():
    w, x = draw(1024, 4096, 1, seed=2)
    W, X = device_matrix(w), device_matrix(x)
    p = bbd.Plan(1024, 4096, 1, splits=4)
    assert p.workspace_size > 0
    Y = output(1, 1024)
    with pytest.raises(bbd.GemvError) as e:
        bbd.run(p, W, X, Y, None)
    assert e.value.status == bbd.Status.WORKSPACE
    small = torch.zeros(p.workspace_size - 4, dtype=torch.uint8, device="cuda")
    with pytest.raises(bbd.GemvError):
        bbd.run(p, W, X, Y, small)
    assert torch.isnan(Y).all(), "a rejected call must enqueue nothing"


def test_one_workspace_shared_by_two_plans():
    a = draw(1024, 4096, 1, seed=3)
    b = draw(4096, 14336, 1, seed=4)
    pa, pb = bbd.Plan(1024, 4096, 1, splits=2), bbd.Plan(4096, 14336, 1, splits=4)
    ws = torch.zeros(max(pa.workspace_size, pb.workspace_size), dtype=torch.uint8, device="cuda")
    Wa, Xa, Wb, Xb = (device_matrix(t) for t in (*a, *b))
    Ya, Yb = output(1, 1024), output(1, 4096)
    bbd.run(pa, Wa, Xa, Ya, ws)
    bbd.run(pb, Wb, Xb, Yb, ws)
    oracle_check(Wa, Xa, Ya, "first")
    oracle_check(Wb, Xb, Yb, "second")
    ya, yb = Ya.clone(), Yb.clone()
    for _ in range(3):                  # alternate: neither plan disturbs the other's tickets
        Ya.fill_(float("nan"))
        Yb.fill_(float("nan"))
        bbd.run(pb, Wb, Xb, Yb, ws)
        bbd.run(pa, Wa, Xa, Ya, ws)
        assert bits_equal(Ya, ya) and bits_equal(Yb, yb)
    assert not ws[:4 * 4096].any(), "tickets must be back at zero after the calls"


def test_one_plan_on_two_streams_at_once():
    """Calls on one split plan may run concurrently when each has its own workspace: two
    streams, each with its own workspace, input and output, launch the same plan in turn
    without synchronising, and every output is bitwise the sequential one."""
    p = bbd.Plan(512, 14336, 2, splits=4)
    assert p.info["splits"] == 4 and p.workspace_size > 0
    ins = [draw(512, 14336, 2, seed=40 + i) for i in range(2)]
    Ws = [device_matrix(w) for w, _ in ins]
    Xs = [device_matrix(x) for _, x in ins]
    ref = []
    for W, X in zip(Ws, Xs):
        Y, _ = gemv(W, X, plan=p)
        oracle_check(W, X, Y, "sequential")
        ref.append(Y.clone())
    streams = [torch.cuda.Stream() for _ in range(2)]
    wss = [p.alloc_workspace() for _ in range(2)]
    Ys = [output(2, 512) for _ in range(2)]
    torch.cuda.synchronize()
    for _ in range(20):
        for i in range(2):
            bbd.run(p, Ws[i], Xs[i], Ys[i], wss[i], stream=streams[i])
    torch.cuda.synchronize()
    for i in range(2):
        assert bits_equal(Ys[i], ref[i]), f"stream {i} differs from the sequential run"
        assert not wss[i][:4 * 4096].any(), "tickets must be back at zero"


# ---------------------------------------------------------------------------- edges
def test_degenerate_shapes():
    for n, k, m in ((1, 1, 1), (1, 8, 1), (1, 9, 2), (64, 1, 16), (1, 14336, 1), (2, 512, 1)):
        w, x = draw(n, k, m, seed=n + k + m)
        W, X = device_matrix(w), device_matrix(x)
        Y, _ = gemv(W, X)
        oracle_check(W, X, Y, f"degenerate n={n} k={k} m={m}")


def test_zero_and_special_values():
    n, k = 16, 1000
    w = torch.zeros(n, k, dtype=torch.bfloat16)
    _, x = draw(1, k, 1, seed=9)
    Y, _ = gemv(device_matrix(w), device_matrix(x))
    assert (Y == 0).all()
    w, x = draw(n, k, 1, seed=10)
    w[3, 17] = float("inf")
    w[5, 900] = float("nan")
    Y, _ = gemv(device_matrix(w), device_matrix(x))
    assert torch.isnan(Y[0, 5]) and torch.isinf(Y[0, 3]) and torch.isfinite(Y[0, :3]).all()


def test_maximum_batch_and_long_k():
    """M = 16 at the down_proj shape and a K long enough that accuracy forces a split."""
    w, x = draw(4096, 14336, 16, seed=11)
    W, X = device_matrix(w), device_matrix(x)
    Y, _ = gemv(W, X)
    oracle_check(W, X, Y, "M=16 down")
    k = 1 << 19
    w, x = draw(24, k, 2, seed=12)
    W, X = device_matrix(w), device_matrix(x)
    Y, p = gemv(W, X)
    assert p.info["splits"] >= 2
    oracle_check(W, X, Y, "K=2^19")


def test_large_x_stride():
    """Batch rows of X more than 2^31 / 16 elements apart: m * ldx must not wrap in 32 bits
    (aligned, unaligned and matrix-core paths)."""
    for k, ldx, m in ((1000, 150_000_000, 16), (1000, 150_000_001, 3), (1024, 150_000_000, 16)):
        w, x = draw(64, k, m, seed=k + m)
        W = device_matrix(w)
        X = device_matrix(x, ld=ldx)
        Y, p = gemv(W, X)
        oracle_check(W, X, Y, f"k={k} ldx={ldx} m={m} mfma={p.info['mfma']}")
        del X
        torch.cuda.empty_cache()


def test_a_million_rows():
    """N = 2^20 short rows: 131,072 eight-wave workgroups (one row per wave) at batch 1, and
    32,768 matrix-core blocks at batch 16, checked in full."""
    n, k = 1 << 20, 64
    for m in (1, 16):
        w, x = draw(n, k, m, seed=m)
        W, X = device_matrix(w), device_matrix(x)
        Y, p = gemv(W, X)
        print(m, p.info, flush=True)
        oracle_check(W, X, Y, f"n=2^20 m={m}")


@pytest.mark.parametrize("n,k", [(4096, 512), (8200, 1000), (5000, 3000), (9000, 3583)])
def test_short_rows_in_multi_wave_workgroups(n, k):
    """Batch-1 rows under 8 wave steps in numbers run in 8-wave workgroups: every output
    against the oracle, and bitwise equal to single-wave workgroups (each row is summed in
    the same order whatever the workgroup)."""
    w, x = draw(n, k, 1, seed=n + k)
    W, X = device_matrix(w), device_matrix(x)
    Y, p = gemv(W, X)
    assert p.info["waves_per_block"] == 8, p.info
    oracle_check(W, X, Y, f"{n}x{k} in 8-wave workgroups")
    Y1, p1 = gemv(W, X, waves_per_block=1)
    assert p1.info["waves_per_block"] == 1 and p1.info["splits"] == p.info["splits"]
    assert bits_equal(Y, Y1), "8-wave and single-wave workgroups differ"


def test_device_plans_equal_host_plans():
    """gemv_plan on the GPU describes the device as the host-only planner is told to (CU
    count from the runtime, 8 TB/s, the default latency): every workload shape, batch-1
    INT4 and the RMSNorm prologue get the same plan both ways. The one field allowed to
    differ is the LDS reserved only to cap resident workgroups (when a cap is set): the device plan confirms its size
    with the runtime's occupancy calculator (256-byte steps), the host plan assumes a 512-byte
    allocation unit; both must admit the same number of workgroups per CU."""
    import torch

    props = torch.cuda.get_device_properties(0)
    cus = props.multi_processor_count
    # the library's loaded-latency constant, read back from what a device plan reports
    latency = bbd.Plan(4096, 4096, 1).info["bytes_in_flight_needed"] * cus / 8.0e12
    assert 0.3e-6 < latency < 1.5e-6
    desc = (cus, 8.0e12, latency)
    lds_per_cu = 160 * 1024

    def same(a, b, what):
        a, b = dict(a), dict(b)
        la, lb = a.pop("lds_bytes"), b.pop("lds_bytes")
        assert a.pop("bytes_in_flight_needed") == pytest.approx(b.pop("bytes_in_flight_needed"))
        assert a == b, what
        # LDS that holds data (staged x: INT4, RMSNorm), or no cap: equal
        if not a["waves_per_cu"] or a["weights"] or a["prologue"]:
            assert la == lb, what
            return
        blocks = a["waves_per_cu"] // a["waves_per_block"]
        for lds in (la, lb):
            assert blocks * lds <= lds_per_cu < (blocks + 1) * lds, (what, lds, blocks)

    shapes = [(g.n, g.k, g.m) for cfg in workloads.WORKLOADS for g in cfg.gemvs]
    for n, k, m in sorted(set(shapes)):
        same(bbd.Plan(n, k, m).info, bbd.Plan(n, k, m, desc=desc).info, (n, k, m))
    for n in (4096, 28672, 128256):
        same(bbd.Plan(n, 4096, 1, weights="int4").info,
             bbd.Plan(n, 4096, 1, weights="int4", desc=desc).info, ("int4", n))
        same(bbd.Plan(n, 4096, 1, prologue="rmsnorm").info,
             bbd.Plan(n, 4096, 1, prologue="rmsnorm", desc=desc).info, ("rmsnorm", n))
