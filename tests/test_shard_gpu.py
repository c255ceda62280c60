"""GPU parity of one GPU's share of each projection when the decode step is spread over G
GPUs (rows of QKV, gate_up and lm_head; K of o_proj and down_proj): every output against the
oracle at G = 2 and 8, the fused shares (QKV, gate_up) also bitwise equal to the same call on
the row-concatenated share."""
import pytest
import torch

import bandwidth_bound_decode_amd as bbd
import workloads
from gpu_helpers import bits_equal, device_matrix, draw, oracle_check, output

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("gpus", [8, 2])
def test_every_share(gpus):
    for i, g in enumerate(workloads.shard_gemvs(gpus)):
        w, x = draw(g.n, g.k, 1, seed=700 + 10 * gpus + i)
        W, X = device_matrix(w), device_matrix(x)
        plan = bbd.Plan(g.n, g.k, 1)
        ws = plan.alloc_workspace()
        Y = output(1, g.n)
        bbd.run(plan, W, X, Y, ws)
        torch.cuda.synchronize()
        print(g.name, g.n, g.k, plan.info["splits"], plan.info["unroll"], flush=True)
        oracle_check(W, X, Y, g.name)
        if g.segments:
            parts = list(torch.split(W, list(g.segments), 0))
            Ys = [output(1, p.shape[0]) for p in parts]
            bbd.fused_run(plan, list(zip(parts, Ys)), X, ws)
            torch.cuda.synchronize()
            assert bits_equal(torch.cat(Ys, 1), Y), f"{g.name}: fused differs from one call"
