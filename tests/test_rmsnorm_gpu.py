"""GPU parity of the GEMV with its RMSNorm prologue against the fp64 oracle: the fused QKV and
gate_up projections and o_proj at full size, ragged shapes on every compiled burst length
and workgroup size, the exact reduction to gemv_run when rms_inv = 1, reproducibility, graph
replay, and the calls the library must refuse."""
import numpy as np
import pytest
import torch

import bandwidth_bound_decode_amd as bbd
import oracle
import workloads
from gpu_helpers import bits_equal, device_matrix, host_bits

pytestmark = pytest.mark.gpu
EPS = 1e-5


def draw(n, k, seed):
    gen = workloads.generator(seed)
    w = workloads.bf16_normal((n, k), workloads.SIGMA_W, gen)
    h = workloads.bf16_normal((k,), workloads.SIGMA_X, gen)
    gain = (1.0 + 0.1 * torch.randn((k,), generator=gen)).to(torch.bfloat16)
    return w, h, gain


def run(parts, h, gain, eps=EPS, plan=None, **opts):
    k = h.shape[-1]
    n = sum(p.shape[0] for p in parts)
    p = plan or bbd.Plan(n, k, 1, prologue="rmsnorm", **opts)
    Ws = [device_matrix(w) for w in parts]
    Ys = [torch.full((w.shape[0],), float("nan"), dtype=torch.float32, device="cuda")
          for w in parts]
    bbd.rmsnorm_run(p, list(zip(Ws, Ys)), h.cuda(), gain.cuda(), eps)
    torch.cuda.synchronize()
    return torch.cat(Ys)[None, :], p


def check(w, h, gain, Y, what, eps=EPS):
    y_ref, s_abs = oracle.gemv_rmsnorm(host_bits(w), host_bits(h), host_bits(gain), eps)
    rep = oracle.check(Y.cpu().numpy(), y_ref, s_abs)
    assert rep.ok, f"{what}: {rep}"
    return rep


@pytest.mark.parametrize("segments", [(4096, 1024, 1024), (14336, 14336), (4096,), (128256,)])
def test_llama_projections(segments):
    k = 4096
    w, h, gain = draw(sum(segments), k, seed=sum(segments))
    parts = list(torch.split(w, list(segments), 0))
    Y, p = run(parts, h, gain)
    print(segments, p.info, flush=True)
    check(w, h, gain, Y, f"rmsnorm {segments}")
    # The other grid form (looping workgroups, or one workgroup per row block) sums every row
    # in the same order, so it gives the same bits.
    blocks = -(-sum(segments) // 8)
    other = dict(waves_per_cu=-1) if p.info["grid_x"] < blocks else dict(waves_per_cu=8)
    Y2, p2 = run(parts, h, gain, **other)
    assert p2.info["grid_x"] != p.info["grid_x"]
    assert bits_equal(Y, Y2), f"grid {p2.info['grid_x']} differs from grid {p.info['grid_x']}"


@pytest.mark.parametrize("n,k", [(7, 8), (33, 1000), (129, 4104), (300, 2048), (17, 8192)])
def test_ragged_every_tile(n, k):
    w, h, gain = draw(n, k, seed=3 * n + k)
    for u in (1, 2, 4, 8):
        for waves in (1, 2, 8):
            Y, _ = run([w], h, gain, unroll=u, waves_per_block=waves)
            check(w, h, gain, Y, f"n={n} k={k} U={u} waves={waves}")
            Y2, _ = run([w], h, gain, unroll=u, waves_per_block=waves)
            assert bits_equal(Y, Y2), "not reproducible"


def test_longest_k():
    """K = 16368, the longest row the prologue accepts (its staging fills the 64 KiB of LDS a
    workgroup gets by default): every burst length on 8-wave workgroups meets the tolerance,
    and a single-wave workgroup, whose longer sum-of-squares chain would break the depth
    bound, is refused by the planner rather than run."""
    n, k = 65, 16368
    w, h, gain = draw(n, k, seed=3 * n + k)
    for u in (1, 2, 4, 8):
        Y, p = run([w], h, gain, unroll=u, waves_per_block=8)
        assert p.info["depth_bound"] <= 160
        check(w, h, gain, Y, f"k={k} U={u}")
    with pytest.raises(bbd.GemvError):
        bbd.Plan(n, k, 1, prologue="rmsnorm", waves_per_block=1)


def test_unit_scale_equals_gemv_run():
    """gamma = 1 and h in {+-1, +-1/2} with eps = 1 - mean(h^2): every step of the norm is
    exact, rms_inv = 1, and the result must be gemv_run's bit for bit."""
    n, k = 1024, 4096
    rng = np.random.default_rng(5)
    hv = rng.choice([-1.0, -0.5, 0.5, 1.0], size=k)
    eps = 1.0 - float(np.sum(hv * hv)) / k
    h = torch.from_numpy(hv.astype(np.float32)).to(torch.bfloat16)
    gain = torch.ones(k, dtype=torch.bfloat16)
    w, _, _ = draw(n, k, seed=6)
    Y, _ = run([w], h, gain, eps=eps)
    W = device_matrix(w)
    Yr = torch.empty((1, n), dtype=torch.float32, device="cuda")
    bbd.run(bbd.Plan(n, k, 1), W, h[None, :].cuda(), Yr)
    torch.cuda.synchronize()
    assert bits_equal(Y, Yr), "rms_inv = 1 must reproduce gemv_run"
    check(w, h, gain, Y, "unit scale", eps=eps)


def test_single_nonzero_and_zero_input():
    n, k = 64, 512
    w, _, gain = draw(n, k, seed=7)
    h = torch.zeros(k, dtype=torch.bfloat16)
    h[37] = 3.0
    Y, _ = run([w], h, gain)
    check(w, h, gain, Y, "one nonzero h")
    Y, _ = run([w], torch.zeros(k, dtype=torch.bfloat16), gain, eps=0.5)
    assert (Y == 0).all()


def test_graph_replay_matches_eager():
    k = 4096
    w, h, gain = draw(6144, k, seed=8)
    parts = list(torch.split(w, [4096, 1024, 1024], 0))
    p = bbd.Plan(6144, k, 1, prologue="rmsnorm")
    Ws = [device_matrix(x) for x in parts]
    Ys = [torch.empty((x.shape[0],), dtype=torch.float32, device="cuda") for x in parts]
    H, G = h.cuda(), gain.cuda()
    bbd.rmsnorm_run(p, list(zip(Ws, Ys)), H, G, EPS)
    torch.cuda.synchronize()
    eager = torch.cat(Ys).clone()
    stream = torch.cuda.Stream()
    with bbd.Graph(stream) as g:
        bbd.rmsnorm_run(p, list(zip(Ws, Ys)), H, G, EPS, stream=stream)
    for _ in range(3):
        for y in Ys:
            y.fill_(float("nan"))
        torch.cuda.synchronize()
        g.launch()
        stream.synchronize()
        assert bits_equal(torch.cat(Ys), eager), "graph replay differs from eager"


def test_refused_calls():
    n, k = 64, 1024
    w, h, gain = draw(n, k, seed=9)
    p = bbd.Plan(n, k, 1, prologue="rmsnorm")
    W = device_matrix(w)
    Y = torch.empty((n,), dtype=torch.float32, device="cuda")
    raw = torch.zeros(k + 8, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(bbd.GemvError) as e:
        bbd.rmsnorm_run(p, [(W, Y)], raw[1:1 + k], gain.cuda(), EPS)     # H not aligned
    assert e.value.status == bbd.Status.MISALIGNED
    with pytest.raises(bbd.GemvError):
        bbd.rmsnorm_run(p, [(W, Y)], h.cuda(), gain.cuda(), -1.0)         # eps < 0
    half = [device_matrix(w[:32]), device_matrix(w[32:], ld=1032)]        # two row strides
    with pytest.raises(bbd.GemvError):
        bbd.rmsnorm_run(p, [(half[0], Y[:32]), (half[1], Y[32:])], h.cuda(), gain.cuda(), EPS)
    with pytest.raises(bbd.GemvError):
        bbd.rmsnorm_run(bbd.Plan(n, k, 1), [(W, Y)], h.cuda(), gain.cuda(), EPS)   # plain plan
    with pytest.raises(bbd.GemvError):
        bbd.run(p, W, h[None, :].cuda(), Y[None, :])                      # norm plan on gemv_run
