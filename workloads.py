"""Seeded synthetic inputs for the decode GEMV, shared by the tests and the bench.

This module holds no arithmetic of the GEMV itself: it only names the workload shapes and
draws seeded bf16 tensors. Both the HIP path and the CPU oracle receive exactly the tensors
drawn here (the oracle always sees the bf16 bits copied back from wherever they were drawn),
so the generator affects reproducibility only, never correctness.

Shapes are the Llama 3.1 8B projection shapes the decode-GEMV page uses ("A strong answer",
causes 1 and 3, and the split-K reversal paragraph on the LM head). Values are dense and
unstructured: float32 normal samples scaled by sigma and rounded to bf16 (round to nearest
even), W with sigma 0.02 and x with sigma 1.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import torch

SIGMA_W = 0.02
SIGMA_X = 1.0

# Llama 3.1 8B projection shapes (rows N, reduction K).
HIDDEN = 4096
INTERMEDIATE = 14336
Q_ROWS = 4096
KV_ROWS = 1024
VOCAB = 128256
LAYERS = 32


@dataclass(frozen=True)
class Gemv:
    """One GEMV problem: y[m] = W . x[m] with W [n, k] and X [m, k]."""
    name: str
    n: int
    k: int
    m: int = 1
    segments: tuple[int, ...] = ()   # row split of a fused projection, sums to n

    @property
    def alg_bytes(self) -> int:
        """Bytes a perfect kernel moves: W and X read once (bf16), Y written once (fp32)."""
        return 2 * self.n * self.k + 2 * self.m * self.k + 4 * self.m * self.n


@dataclass(frozen=True)
class Config:
    seed: int
    title: str
    gemvs: tuple[Gemv, ...] = field(default_factory=tuple)


def decode_step_gemvs(layers: int = LAYERS) -> tuple[Gemv, ...]:
    """The GEMV sequence of one batch-1 decode step, in stream order."""
    seq = []
    for layer in range(layers):
        seq.append(Gemv(f"L{layer}.qkv", Q_ROWS + 2 * KV_ROWS, HIDDEN,
                        segments=(Q_ROWS, KV_ROWS, KV_ROWS)))
        seq.append(Gemv(f"L{layer}.o", HIDDEN, HIDDEN))
        seq.append(Gemv(f"L{layer}.gate_up", 2 * INTERMEDIATE, HIDDEN,
                        segments=(INTERMEDIATE, INTERMEDIATE)))
        seq.append(Gemv(f"L{layer}.down", HIDDEN, INTERMEDIATE))
    seq.append(Gemv("lm_head", VOCAB, HIDDEN))
    return tuple(seq)


K_PROJ_AND_TAILS = Config(
    1000, "k_proj GEMV 1024x4096 with tails 7x129 and 33x1000, batch 1",
    (Gemv("k_proj", KV_ROWS, HIDDEN), Gemv("tail_7x129", 7, 129), Gemv("tail_33x1000", 33, 1000)))
DOWN_PROJ = Config(
    1001, "split-K stress GEMV, down_proj 4096x14336, batch 1",
    (Gemv("down", HIDDEN, INTERMEDIATE),))
FUSED_PROJECTIONS = Config(
    1002, "fused projections at batch 1: QKV 6144x4096 and gate_up 28672x4096",
    (Gemv("qkv", Q_ROWS + 2 * KV_ROWS, HIDDEN, segments=(Q_ROWS, KV_ROWS, KV_ROWS)),
     Gemv("gate_up", 2 * INTERMEDIATE, HIDDEN, segments=(INTERMEDIATE, INTERMEDIATE))))
DECODE_STEP = Config(
    1003, "full batch-1 decode-step GEMV sequence (32 layers + lm_head) in one graph",
    decode_step_gemvs())
SKINNY_BATCH = Config(
    1004, "skinny-batch GEMV 4096x14336 at M in {1,2,4,8,16}, tail 4097x14337 at M=3",
    tuple(Gemv(f"skinny_m{m}", HIDDEN, INTERMEDIATE, m) for m in (1, 2, 4, 8, 16))
    + (Gemv("skinny_tail_m3", HIDDEN + 1, INTERMEDIATE + 1, 3),))

# One GPU's share of each projection when a decode step is spread over `gpus` GPUs: the
# row-independent projections (QKV, gate_up, lm_head) by rows, every segment of a fused one
# cut alike; o_proj and down_proj by K (each GPU then holds a partial y that a sum over the
# GPUs completes). Every dimension divides evenly for gpus in {1, 2, 4, 8}.
SHARD_GPUS = (2, 4, 8)


def shard_gemvs(gpus: int) -> tuple[Gemv, ...]:
    """The five projection shapes of one layer (and lm_head) on one of `gpus` GPUs."""
    if gpus < 1 or any(d % gpus for d in (Q_ROWS, KV_ROWS, HIDDEN, INTERMEDIATE, VOCAB)):
        raise ValueError(f"the Llama shapes do not split evenly over {gpus} GPUs")
    q, kv, i = Q_ROWS // gpus, KV_ROWS // gpus, INTERMEDIATE // gpus
    return (Gemv(f"qkv_g{gpus}", q + 2 * kv, HIDDEN, segments=(q, kv, kv)),
            Gemv(f"o_proj_g{gpus}", HIDDEN, HIDDEN // gpus),
            Gemv(f"gate_up_g{gpus}", 2 * i, HIDDEN, segments=(i, i)),
            Gemv(f"down_g{gpus}", HIDDEN, INTERMEDIATE // gpus),
            Gemv(f"lm_head_g{gpus}", VOCAB // gpus, HIDDEN))


def shard_decode_step_gemvs(gpus: int, layers: int = LAYERS) -> tuple[Gemv, ...]:
    """One GPU's GEMV sequence of a decode step spread over `gpus` GPUs, in stream order."""
    qkv, o, gu, down, lm = shard_gemvs(gpus)
    seq = []
    for layer in range(layers):
        seq += [Gemv(f"L{layer}.{g.name}", g.n, g.k, segments=g.segments) for g in (qkv, o, gu, down)]
    seq.append(lm)
    return tuple(seq)


# Every workload above, smallest first.
WORKLOADS: tuple[Config, ...] = (K_PROJ_AND_TAILS, DOWN_PROJ, FUSED_PROJECTIONS, DECODE_STEP,
                                 SKINNY_BATCH)


def generator(seed: int, device: str | torch.device = "cpu") -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def bf16_normal(shape, sigma: float, gen: torch.Generator,
                device: str | torch.device = "cpu") -> torch.Tensor:
    """float32 N(0, 1) samples times sigma, rounded to bf16."""
    t = torch.randn(shape, generator=gen, device=device, dtype=torch.float32)
    return t.mul_(sigma).to(torch.bfloat16)


def draw_gemv(g: Gemv, gen: torch.Generator, device: str | torch.device = "cpu"):
    """Draw (W [n, k], X [m, k]) for one GEMV, W first, from the given generator."""
    w = bf16_normal((g.n, g.k), SIGMA_W, gen, device)
    x = bf16_normal((g.m, g.k), SIGMA_X, gen, device)
    return w, x


def draw_config(cfg: Config, device: str | torch.device = "cpu"):
    """Draw every GEMV of a config in listed order from one generator seeded 1000 + index."""
    gen = generator(cfg.seed, device)
    return [draw_gemv(g, gen, device) for g in cfg.gemvs]


def bf16_bits(t: torch.Tensor):
    """The raw bf16 bit patterns of a tensor as a contiguous host uint16 numpy array."""
    assert t.dtype == torch.bfloat16
    return t.detach().contiguous().cpu().view(torch.int16).numpy().view("uint16")


def draw_decode_step(device: str | torch.device = "cuda", layers: int = LAYERS,
                     seed: int | None = None, gemvs: tuple[Gemv, ...] | None = None):
    """Draw the decode-step sequence: for each GEMV in stream order, its weight (as separate
    contiguous tensors, one per segment of a fused projection) and its input vector.

    Returns a list of (Gemv, [W parts], X). About 15 GB of weights at 32 layers, so draw on
    the GPU. `gemvs` replaces the sequence (e.g. one GPU's shard of it).
    """
    gen = generator(DECODE_STEP.seed if seed is None else seed, device)
    out = []
    for g in gemvs if gemvs is not None else decode_step_gemvs(layers):
        w, x = draw_gemv(g, gen, device)
        if g.segments:
            parts = [t.clone() for t in torch.split(w, list(g.segments), 0)]
            del w
        else:
            parts = [w]
        out.append((g, parts, x))
    return out


# --------------------------------------------------------------------------- INT4 weights
INT4_GROUP = 128


def draw_int4(n: int, k: int, gen: torch.Generator, device: str | torch.device = "cpu",
              ldq: int | None = None, lds: int | None = None):
    """Seeded INT4 weights in the packed format the INT4 GEMV reads, drawn the way a weight
    of the workloads above would be quantized: W ~ N(0, SIGMA_W) in bf16, then per row and
    run of 128 elements a bf16 scale absmax / 7 and integers round(W / scale) clamped to
    [-8, 7]. This only prepares inputs; the GEMV's own arithmetic (dequantize, multiply,
    sum) is not here.

    Returns (packed uint8 [n, ldq], bf16 scales [n, lds], the integer values int8 [n, k]):
    element k of a row is the low nibble of byte k/2 when k is even and the high nibble when
    odd, two's complement; padding bytes and scales beyond the last group are filled with
    0xEE / NaN so a read of them shows.
    """
    groups = (k + INT4_GROUP - 1) // INT4_GROUP
    ldq = (k + 1) // 2 if ldq is None else ldq
    lds = groups if lds is None else lds
    assert ldq >= (k + 1) // 2 and lds >= groups
    w = bf16_normal((n, k), SIGMA_W, gen, device).float()
    pad = groups * INT4_GROUP - k
    wg = torch.nn.functional.pad(w, (0, pad)).view(n, groups, INT4_GROUP)
    scale = (wg.abs().amax(dim=2) / 7.0).to(torch.bfloat16)
    scale = torch.where(scale == 0, torch.ones_like(scale), scale)
    q = torch.round(wg / scale.float()[:, :, None]).clamp_(-8, 7).view(n, -1)[:, :k]
    q = q.to(torch.int8)
    nib = (q.to(torch.int16) & 0xF).to(torch.uint8)
    if k % 2:
        nib = torch.nn.functional.pad(nib, (0, 1))
    packed = torch.full((n, ldq), 0xEE, dtype=torch.uint8, device=device)
    packed[:, :(k + 1) // 2] = nib[:, 0::2] | (nib[:, 1::2] << 4)
    scales = torch.full((n, lds), float("nan"), dtype=torch.bfloat16, device=device)
    scales[:, :groups] = scale
    return packed, scales, q
