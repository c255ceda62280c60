"""GPU parity of the persistent chain: bitwise equal to running its links one by one with
unsplit plans, within tolerance of the oracle, stable over repeated runs and graph replays,
and its bounded dependency wait reports a timeout instead of hanging."""
import pytest
import torch

import bandwidth_bound_decode_amd as bbd
from gpu_helpers import bits_equal, device_matrix, draw, oracle_check, output

pytestmark = pytest.mark.gpu

# (segment rows, K, ldw): single and fused links, one- and two-row items (2049 rows give an
# odd row count to two-row items), partial bursts, ragged K with padded rows (K = 4099: the
# k % 8 last elements lie past every wave step a burst reads)
LINKS = [((1024,), 4096, 4096), ((100, 500), 4096, 4096), ((4096,), 14336, 14336),
         ((64,), 14336, 14336), ((2049,), 14336, 14336), ((33,), 1000, 1008),
         ((7,), 129, 136), ((5, 3, 2, 9), 520, 520), ((300,), 4099, 4104)]


def build_links(seed=0):
    links, refs = [], []
    for i, (rows, k, ldw) in enumerate(LINKS):
        segs = []
        for j, n in enumerate(rows):
            w, _ = draw(n, k, 1, seed=seed + 10 * i + j)
            segs.append((device_matrix(w, ld=ldw), output(1, n)))
        _, x = draw(1, k, 1, seed=seed + 10 * i + 9)
        links.append((segs, device_matrix(x)))
    return links


def one_by_one(links):
    outs = []
    for segs, x in links:
        n = sum(w.shape[0] for w, _ in segs)
        plan = bbd.Plan(n, x.shape[1], 1, splits=1)
        ys = [output(1, w.shape[0]) for w, _ in segs]
        if len(segs) == 1:
            bbd.run(plan, segs[0][0], x, ys[0])
        else:
            bbd.fused_run(plan, [(w, y) for (w, _), y in zip(segs, ys)], x)
        outs.append(torch.cat(ys, 1))
    torch.cuda.synchronize()
    return outs


def outputs(links):
    return [torch.cat([y for _, y in segs], 1).clone() for segs, _ in links]


def clear(links):
    for segs, _ in links:
        for _, y in segs:
            y.fill_(float("nan"))


def test_chain_matches_links_one_by_one():
    links = build_links()
    ref = one_by_one(links)
    chain = bbd.Chain(links)
    for rep in range(3):                       # counters reset between launches
        clear(links)
        chain.run()
        chain.check()
        got = outputs(links)
        for i, (a, b) in enumerate(zip(got, ref)):
            assert bits_equal(a, b), f"run {rep}: link {i} differs from its gemv_run"
    for (segs, x), y in zip(links, got):
        oracle_check(torch.cat([w for w, _ in segs], 0), x, y, "chain link")


@pytest.mark.parametrize("waves_per_cu", [1, 3, 11])
def test_chain_grid_sizes_give_same_bits(waves_per_cu):
    links = build_links(seed=100)
    ref = one_by_one(links)
    chain = bbd.Chain(links, waves_per_cu=waves_per_cu)
    clear(links)
    chain.run()
    chain.check()
    for a, b in zip(outputs(links), ref):
        assert bits_equal(a, b), f"waves_per_cu={waves_per_cu}"


def test_chain_in_a_graph():
    links = build_links(seed=200)
    ref = one_by_one(links)
    chain = bbd.Chain(links)
    stream = torch.cuda.Stream()
    g = bbd.Graph(stream)
    with torch.cuda.stream(stream):
        with g:
            chain.run(stream)
    for rep in range(3):
        clear(links)
        torch.cuda.synchronize()
        g.launch(stream)
        stream.synchronize()
        for a, b in zip(outputs(links), ref):
            assert bits_equal(a, b), f"graph replay {rep}"
    chain.check()
    g.destroy()


def test_chain_timeout_is_reported_not_hung():
    """A tiny spin limit (set from the host) makes dependency waits give up: the launch
    still ends, check() reports the timeout once, and a healthy chain afterwards is exact."""
    links = build_links(seed=300)
    ref = one_by_one(links)
    impatient = bbd.Chain(links, spin_limit=1)
    impatient.run()
    with pytest.raises(bbd.GemvError) as e:
        impatient.check()
    assert e.value.status == bbd.Status.TIMEOUT
    impatient.check()                          # the flag was cleared
    healthy = bbd.Chain(links)
    clear(links)
    healthy.run()
    healthy.check()
    for a, b in zip(outputs(links), ref):
        assert bits_equal(a, b)
