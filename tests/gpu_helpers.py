"""Helpers for the GPU parity tests: padded/misaligned device buffers, one GEMV call through
the C ABI, and the oracle comparison on the exact bf16 bits the GPU consumed."""
from __future__ import annotations

import numpy as np
import torch

import bandwidth_bound_decode_amd as bbd
import oracle
import workloads

NAN_BF16 = 0x7FC0          # quiet NaN: any padding element that is read poisons the result
DEV = "cuda"


def device_matrix(t: torch.Tensor, ld: int | None = None, offset: int = 0) -> torch.Tensor:
    """Copy a bf16 [r, c] tensor to the GPU with row stride `ld` (>= c), starting `offset`
    elements into its allocation (offset % 8 != 0 breaks 16-byte alignment). Padding holds
    NaN bit patterns."""
    r, c = t.shape
    ld = c if ld is None else ld
    raw = torch.full((offset + r * ld + 16,), NAN_BF16, dtype=torch.int16, device=DEV)
    view = raw[offset:offset + r * ld].view(torch.bfloat16).view(r, ld)[:, :c]
    view.copy_(t.to(DEV))
    return view


def host_bits(t: torch.Tensor) -> np.ndarray:
    """Exact bf16 bits of a (possibly strided) tensor, as a contiguous host uint16 array."""
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def output(m: int, n: int, ldy: int | None = None) -> torch.Tensor:
    """fp32 [m, n] output view with row stride ldy, pre-filled with NaN (so a missed store
    shows), inside an allocation whose padding is NaN as well."""
    ldy = n if ldy is None else ldy
    raw = torch.full((m * ldy + 4,), float("nan"), dtype=torch.float32, device=DEV)
    return raw[:m * ldy].view(m, ldy)[:, :n]


def gemv(W: torch.Tensor, X: torch.Tensor, *, ldy=None, plan=None, stream=None, **opts):
    """Run one GEMV on device tensors; returns (Y on device, plan)."""
    n, k = W.shape
    m = X.shape[0]
    p = plan or bbd.Plan(n, k, m, **opts)
    Y = output(m, n, ldy)
    ws = p.alloc_workspace()
    bbd.run(p, W, X, Y, ws, stream=stream)
    return Y, p


def oracle_check(W: torch.Tensor, X: torch.Tensor, Y: torch.Tensor, what: str = ""):
    """Parity of Y (device or host fp32 [m, n]) against the fp64 oracle on W's and X's bits."""
    y_ref, s_abs = oracle.gemv(host_bits(W), host_bits(X))
    rep = oracle.check(Y.detach().cpu().numpy(), y_ref, s_abs)
    assert rep.ok, f"{what}: {rep}"
    return rep


def draw(n: int, k: int, m: int = 1, seed: int = 0):
    """Seeded CPU draw of (W [n, k], X [m, k]) with the workload distributions."""
    gen = workloads.generator(seed)
    return workloads.draw_gemv(workloads.Gemv("t", n, k, m), gen)


def bits_equal(a: torch.Tensor, b: torch.Tensor) -> bool:
    a = a.detach().cpu().contiguous()
    b = b.detach().cpu().contiguous()
    return a.shape == b.shape and torch.equal(a.view(torch.int32), b.view(torch.int32))
