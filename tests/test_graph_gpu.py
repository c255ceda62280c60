"""GPU parity of the graph-captured decode step: every replay bitwise equal to the eager
sequence, and every output of all 129 GEMVs within tolerance of the oracle."""
import numpy as np
import pytest
import torch

import bandwidth_bound_decode_amd as bbd
import oracle
import workloads
from bandwidth_bound_decode_amd.decode_step import Call, Sequence
from gpu_helpers import bits_equal, device_matrix, draw, host_bits, oracle_check

pytestmark = pytest.mark.gpu


def make_sequence(drawn):
    calls = []
    for g, parts, x in drawn:
        ys = [torch.full((x.shape[0], w.shape[0]), float("nan"), device="cuda") for w in parts]
        calls.append(Call(parts, x, ys))
    return Sequence(calls)


def snapshot(seq):
    return [torch.cat(c.ys, 1).clone() for c in seq.calls]


def replay_matches_eager(seq, replays=3):
    stream = torch.cuda.Stream()
    seq.run()                                   # eager, torch's current stream
    torch.cuda.synchronize()
    eager = snapshot(seq)
    seq.capture(stream)
    for r in range(replays):
        for c in seq.calls:                     # eager work between replays
            for y in c.ys:
                y.fill_(float("nan"))
        torch.cuda.synchronize()
        seq.replay(stream)
        stream.synchronize()
        got = snapshot(seq)
        for i, (a, b) in enumerate(zip(got, eager)):
            assert bits_equal(a, b), f"replay {r}: call {i} differs from eager"
    return eager


def test_small_graph():
    """A short mixed sequence: split and unsplit plans, a fused call, a batch of 3."""
    drawn = []
    for i, (n, k, m, segs) in enumerate([(1024, 4096, 1, ()), (600, 4096, 1, (100, 500)),
                                         (64, 14336, 1, ()), (4096, 14336, 1, ()),
                                         (77, 1000, 3, ())]):
        w, x = draw(n, k, m, seed=50 + i)
        parts = [device_matrix(p) for p in (torch.split(w, list(segs)) if segs else [w])]
        drawn.append((None, parts, device_matrix(x)))
    seq = make_sequence(drawn)
    assert any(c.plan.info["splits"] > 1 for c in seq.calls), "want a split-K call in the graph"
    eager = replay_matches_eager(seq)
    for (_, parts, x), y in zip(drawn, eager):
        oracle_check(torch.cat(parts, 0), x, y, "small graph")


def test_decode_step_full():
    """32 layers x [QKV, o_proj, gate_up, down] + lm_head, ~15 GB of bf16 weights."""
    drawn = workloads.draw_decode_step("cuda")
    seq = make_sequence(drawn)
    print(f"decode step: {len(seq.calls)} GEMVs, {seq.weight_bytes / 1e9:.2f} GB of weights",
          flush=True)
    assert len(seq.calls) == 129
    eager = replay_matches_eager(seq, replays=2)
    # the same step as one persistent chain launch, bitwise equal to the eager sequence
    chain = seq.chain()
    for rep in range(2):
        for c in seq.calls:
            for y in c.ys:
                y.fill_(float("nan"))
        chain.run()
        chain.check()
        for i, (a, b) in enumerate(zip(snapshot(seq), eager)):
            assert bits_equal(a, b), f"chain run {rep}: call {i} differs from eager"
    chain.destroy()
    # Every output of every GEMV against the oracle, one weight matrix on the host at a time
    # (at most the 1 GB lm_head).
    worst = 0.0
    for i, ((g, parts, x), y) in enumerate(zip(drawn, eager)):
        xb = host_bits(x)
        y_host = y.cpu().numpy()
        col = 0
        for j, part in enumerate(parts):
            n = part.shape[0]
            y_ref, s_abs = oracle.gemv(host_bits(part), xb)
            rep = oracle.check(y_host[:, col:col + n], y_ref, s_abs)
            assert rep.ok, f"call {i} ({g.name}) segment {j}: {rep}"
            worst = max(worst, rep.worst_ratio)
            col += n
        assert col == y_host.shape[1]
    print(f"decode step: all {sum(c.n for c in seq.calls)} outputs within tolerance, "
          f"worst error / allowance {worst:.3g}", flush=True)


def test_unaligned_and_matrix_core_calls_in_graph():
    """Unaligned calls on the class-staged kernel (x staged whole, x past 64 KiB of LDS, x in
    chunks), a matrix-core batch and an unaligned batch on the matrix cores, captured
    together: every replay bitwise equal to the eager run, and the eager run within
    tolerance of the oracle."""
    drawn = []
    for i, (n, k, m, ldw, off) in enumerate([(1000, 14337, 1, 14339, 1), (513, 14337, 4, 14337, 3),
                                             (300, 14337, 9, 14340, 1), (4096, 4096, 8, 4096, 0),
                                             (4097, 14337, 16, 14337, 1)]):
        w, x = draw(n, k, m, seed=70 + i)
        W = device_matrix(w, ld=ldw, offset=off)
        X = device_matrix(x, ld=k + (off & 1), offset=off & 1)
        drawn.append((None, [W], X))
    seq = make_sequence(drawn)
    assert seq.calls[3].plan.info["mfma"], "want a matrix-core call in the graph"
    assert seq.calls[4].plan.info["mfma_unaligned_depth"], "want an unaligned one on them"
    eager = replay_matches_eager(seq)
    for (_, parts, x), y in zip(drawn, eager):
        oracle_check(parts[0], x, y, "unaligned graph")
