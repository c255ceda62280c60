"""Pins that tie the CPU oracle to facts other than itself.

Each pin takes a loaded oracle library (ctypes handle) and raises AssertionError when the
oracle disagrees with:
  - the IEEE binary32 layout of bf16 (exhaustive over all 65,536 patterns, against
    torch's own bf16 -> float64 conversion, plus textbook values);
  - closed forms whose exact result is known without summing anything
    (identity W, one-hot x, constant W with small-integer x);
  - the exact rational value of the sum (fractions.Fraction brute force on tiny shapes,
    where fp64 summation must land within the standard recursive-summation bound
    gamma_K * sum|terms|, gamma_K = K u / (1 - K u), u = 2^-53);
  - an independent library routine (numpy float64 matmul) at the working shapes.

The mutation test in test_oracle.py compiles deliberately broken copies of the oracle and
checks that at least one pin rejects each of them.
"""
from __future__ import annotations

import math
import sys
from fractions import Fraction

import numpy as np
import torch

import oracle

U53 = 2.0 ** -53


def gamma(n: int, u: float = U53) -> float:
    return n * u / (1.0 - n * u)


def _rand_bits(rng: np.random.Generator, shape, scale=1.0, wide_exponents=False):
    """Finite bf16 bit patterns: normal values, optionally spread over many binades."""
    v = rng.standard_normal(shape).astype(np.float32) * np.float32(scale)
    if wide_exponents:
        v *= np.exp2(rng.integers(-24, 25, size=shape)).astype(np.float32)
    t = torch.from_numpy(v).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16).copy()


def _exact(bits) -> list:
    """Exact rational values of finite bf16 bits, via the binary32 layout by hand."""
    out = []
    for b in np.asarray(bits, dtype=np.uint16).ravel().tolist():
        sign = -1 if b & 0x8000 else 1
        e = (b >> 7) & 0xFF
        f = b & 0x7F
        assert e != 0xFF, "finite inputs only"
        if e == 0:
            val = Fraction(f, 1 << 7) * Fraction(1, 1 << 126)
        else:
            val = (1 + Fraction(f, 1 << 7)) * (Fraction(2) ** (e - 127))
        out.append(sign * val)
    return out


# --------------------------------------------------------------------------- decode
def pin_bf16_decode(so):
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    got = oracle.bf16_to_f64(bits, so=so)
    ref = torch.from_numpy(bits.view(np.int16).copy()).view(torch.bfloat16).double().numpy()
    nan_g, nan_r = np.isnan(got), np.isnan(ref)
    assert np.array_equal(nan_g, nan_r), "NaN patterns differ"
    ok = ~nan_r
    assert np.array_equal(got[ok], ref[ok]), "decoded values differ from torch"
    assert np.array_equal(np.signbit(got[ok]), np.signbit(ref[ok])), "signs of zero differ"
    textbook = {0x3F80: 1.0, 0xC000: -2.0, 0x3C80: 2.0 ** -6, 0x0001: 2.0 ** -133,
                0x0080: 2.0 ** -126, 0x7F7F: (2 - 2 ** -7) * 2.0 ** 127, 0x7F80: math.inf,
                0xFF80: -math.inf, 0x8000: -0.0}
    for b, v in textbook.items():
        g = got[b]
        assert g == v and math.copysign(1, g) == math.copysign(1, v), hex(b)


# --------------------------------------------------------------------------- closed forms
def pin_identity(so):
    rng = np.random.default_rng(11)
    for n in (1, 129, 1024):
        w = np.zeros((n, n), dtype=np.uint16)
        w[np.arange(n), np.arange(n)] = 0x3F80
        x = _rand_bits(rng, (n,))
        y, s = oracle.gemv(w, x, so=so)
        xv = oracle.bf16_to_f64(x, so=so)
        assert np.array_equal(y[0], xv), f"identity {n}"
        assert np.array_equal(s[0], np.abs(xv)), f"identity s_abs {n}"


def pin_one_hot(so):
    rng = np.random.default_rng(12)
    for n, k in ((7, 129), (33, 1000), (64, 4096)):
        w = _rand_bits(rng, (n, k), 0.02)
        wv = oracle.bf16_to_f64(w, so=so)
        js = sorted({0, 1, 7, 8, 63, 64, 127, 128, k // 2, k - 2, k - 1} & set(range(k)))
        x = np.zeros((len(js), k), dtype=np.uint16)
        for row, j in enumerate(js):
            x[row, j] = 0x3F80
        y, s = oracle.gemv(w, x, so=so)
        for row, j in enumerate(js):
            assert np.array_equal(y[row], wv[:, j]), f"one-hot {n}x{k} j={j}"
            assert np.array_equal(s[row], np.abs(wv[:, j])), f"one-hot s_abs j={j}"


def pin_constant_w(so):
    """W = c = 2^-6 everywhere, x in {-2..2}: y = c * sum(x), exact at every partial sum."""
    rng = np.random.default_rng(13)
    ints = {-2: 0xC000, -1: 0xBF80, 0: 0x0000, 1: 0x3F80, 2: 0x4000}
    for n, k, m in ((5, 129, 1), (33, 1000, 3), (16, 14337, 2)):
        w = np.full((n, k), 0x3C80, dtype=np.uint16)
        xi = rng.integers(-2, 3, size=(m, k))
        x = np.vectorize(ints.get)(xi).astype(np.uint16)
        y, s = oracle.gemv(w, x, so=so)
        want = (2.0 ** -6) * xi.sum(axis=1)
        want_abs = (2.0 ** -6) * np.abs(xi).sum(axis=1)
        assert np.array_equal(y, np.repeat(want[:, None], n, axis=1)), f"const {n}x{k}"
        assert np.array_equal(s, np.repeat(want_abs[:, None], n, axis=1)), "const s_abs"


# --------------------------------------------------------------------------- brute force
def pin_brute_force(so):
    """Exact rational sums on tiny strided problems whose padding holds NaN bits."""
    rng = np.random.default_rng(14)
    for n in (1, 2, 3, 5, 12):
        for k in (1, 2, 7, 8, 9, 63, 64, 65, 70):
            for m in (1, 2, 3):
                wide = (n + k + m) % 2 == 0
                ldw, ldx = k + 3, k + 5
                wbuf = np.full((n, ldw), 0x7FC0, dtype=np.uint16)   # NaN padding
                xbuf = np.full((m, ldx), 0x7FC0, dtype=np.uint16)
                wbuf[:, :k] = _rand_bits(rng, (n, k), 0.02, wide)
                xbuf[:, :k] = _rand_bits(rng, (m, k), 1.0, wide)
                y, s = oracle.gemv(wbuf, xbuf[:, :k], so=so)
                assert y.shape == (m, n)
                assert np.isfinite(y).all() and np.isfinite(s).all(), \
                    f"non-finite output (padding read?) n={n} k={k} m={m}"
                we = [_exact(wbuf[r, :k]) for r in range(n)]
                xe = [_exact(xbuf[i, :k]) for i in range(m)]
                for i in range(m):
                    for r in range(n):
                        terms = [a * b for a, b in zip(we[r], xe[i])]
                        exact = sum(terms, Fraction(0))
                        mag = sum((abs(t) for t in terms), Fraction(0))
                        bound = gamma(k) * float(mag)
                        assert abs(Fraction(y[i, r]) - exact) <= Fraction(bound), \
                            f"brute force n={n} k={k} m={m} ({i},{r})"
                        assert abs(Fraction(s[i, r]) - mag) <= Fraction(bound), \
                            f"brute force s_abs n={n} k={k} m={m}"


def pin_cancellation(so):
    """Terms chosen to cancel: +a, -a pairs around one small survivor; exact answer known."""
    rng = np.random.default_rng(15)
    k = 257
    big = _rand_bits(rng, (128,), 1.0, wide_exponents=True)
    w = np.concatenate([big, big ^ np.uint16(0x8000), np.array([0x3C80], np.uint16)])[None, :]
    x = np.full((1, k), 0x3F80, dtype=np.uint16)
    y, s = oracle.gemv(w, x, so=so)
    # every +a is added before its -a, so with exact products the fp64 result is within
    # gamma_K * s_abs of the exact 2^-6
    assert abs(y[0, 0] - 2.0 ** -6) <= gamma(k) * s[0, 0], "cancellation"


# --------------------------------------------------------------------------- library
def pin_numpy_matmul(so):
    rng = np.random.default_rng(16)
    for n, k, m in ((1024, 4096, 1), (7, 129, 1), (33, 1000, 1), (257, 14337, 3)):
        w = _rand_bits(rng, (n, k), 0.02)
        x = _rand_bits(rng, (m, k), 1.0)
        y, s = oracle.gemv(w, x, nthreads=4, so=so)
        wv = oracle.bf16_to_f64(w, so=so)
        xv = oracle.bf16_to_f64(x, so=so)
        ref = xv @ wv.T
        ref_abs = np.abs(xv) @ np.abs(wv).T
        tol = 2 * gamma(k) * ref_abs
        assert np.all(np.abs(y - ref) <= tol), f"numpy matmul {n}x{k}x{m}"
        assert np.all(np.abs(s - ref_abs) <= tol), f"numpy s_abs {n}x{k}x{m}"


def pin_thread_invariance(so):
    rng = np.random.default_rng(17)
    w = _rand_bits(rng, (301, 777), 0.02)
    x = _rand_bits(rng, (2, 777), 1.0)
    y1, s1 = oracle.gemv(w, x, nthreads=1, so=so)
    y4, s4 = oracle.gemv(w, x, nthreads=4, so=so)
    assert np.array_equal(y1, y4) and np.array_equal(s1, s4), "thread count changes result"


# --------------------------------------------------------------------------- INT4 weights
def _bf16_bits(values) -> np.ndarray:
    t = torch.tensor(np.asarray(values, dtype=np.float64)).to(torch.bfloat16)
    back = t.to(torch.float64).numpy()
    assert np.array_equal(back, np.asarray(values, dtype=np.float64)), "not exact in bf16"
    return t.view(torch.int16).numpy().view(np.uint16).copy()


def pin_q4_format(so):
    """Hand-decoded rows of the INT4 format: two's-complement nibbles, low nibble first,
    one bf16 scale per 128 elements."""
    # row 0: bytes 0x10 0x32 0x98 0xF7 -> nibbles 0,1,2,3,8,9,7,F -> 0,1,2,3,-8,-7,7,-1, x 0.5
    # row 1: bytes 0x8F 0x7F 0x00 0x00 -> F,8,F,7,0,0,0,0 -> -1,-8,-1,7,0,0,0,0, x -2
    wq = np.array([[0x10, 0x32, 0x98, 0xF7], [0x8F, 0x7F, 0x00, 0x00]], dtype=np.uint8)
    sc = _bf16_bits([[0.5], [-2.0]])
    want = np.array([[0, 0.5, 1, 1.5, -4, -3.5, 3.5, -0.5], [2, 16, 2, -14, 0, 0, 0, 0]])
    got = oracle.q4_dequant(wq, sc, 8, so=so)
    assert np.array_equal(got, want), f"format decode {got.tolist()}"
    # groups: K = 260 elements all +1 (nibble pairs 0x11), scales 1, 2, 4 for elements
    # 0..127, 128..255, 256..259; a padded row stride on both arrays
    raw = np.full((1, 140), 0xEE, dtype=np.uint8)
    raw[0, :130] = 0x11
    sraw = _bf16_bits([[1.0, 2.0, 4.0, 1024.0]])
    got = oracle.q4_dequant(raw, sraw, 260, so=so)[0]
    want = np.concatenate([np.full(128, 1.0), np.full(128, 2.0), np.full(4, 4.0)])
    assert np.array_equal(got, want), "group boundaries"
    x = _bf16_bits(np.ones((1, 260)))
    y, s = oracle.gemv_q4(raw, sraw, x, so=so)
    assert y[0, 0] == 128 + 256 + 16 and s[0, 0] == y[0, 0], "group sums"


def _q4_case(rng, n, k, ldq_pad=0, lds_pad=0):
    """Random nibbles and power-of-two scales (so every weight is exact in bf16)."""
    groups = (k + 127) // 128
    wq = rng.integers(0, 256, size=(n, (k + 1) // 2 + ldq_pad), dtype=np.uint8)
    scale = np.exp2(rng.integers(-12, 3, size=(n, groups + lds_pad)).astype(np.float64))
    scale *= np.where(rng.random((n, groups + lds_pad)) < 0.3, -1.0, 1.0)
    return wq, _bf16_bits(scale)


def pin_q4_equals_bf16_oracle(so):
    """With power-of-two scales every INT4 weight is a bf16 value, so the INT4 oracle must
    equal the (separately pinned) bf16 oracle on those values bit for bit: same products,
    same k-ascending sum. Odd K, a ragged last group, padded strides on every array."""
    rng = np.random.default_rng(31)
    for n, k, m in ((37, 300, 3), (5, 129, 1), (64, 1024, 2)):
        wq, sc = _q4_case(rng, n, k, ldq_pad=3, lds_pad=2)
        x = _rand_bits(rng, (m, k + 5), 1.0)[:, :k]
        wdeq = oracle.q4_dequant(wq, sc, k, so=so)
        y4, s4 = oracle.gemv_q4(wq, sc, x, so=so)
        y, s = oracle.gemv(_bf16_bits(wdeq), x, so=so)
        assert np.array_equal(y4, y) and np.array_equal(s4, s), f"q4 vs bf16 n={n} k={k}"


def pin_q4_brute_force(so):
    """Exact rational sums with weights decoded by hand from the nibbles, general scales."""
    rng = np.random.default_rng(37)
    n, k = 3, 200
    wq = rng.integers(0, 256, size=(n, 100), dtype=np.uint8)
    sc = _rand_bits(rng, (n, 2), 0.02)
    x = _rand_bits(rng, (2, k), 1.0)
    y, s = oracle.gemv_q4(wq, sc, x, so=so)
    xs = [_exact(x[i]) for i in range(2)]
    for r in range(n):
        scales = _exact(sc[r])
        w = []
        for j in range(k):
            b = int(wq[r, j // 2])
            nib = (b >> 4) if j % 2 else (b & 0xF)
            w.append((nib - 16 if nib >= 8 else nib) * scales[j // 128])
        for i in range(2):
            terms = [a * b for a, b in zip(w, xs[i])]
            exact = sum(terms)
            mag = sum(abs(t) for t in terms)
            assert abs(Fraction(y[i, r]) - exact) <= Fraction(gamma(k)) * mag, "q4 brute force"
            assert abs(Fraction(s[i, r]) - mag) <= Fraction(gamma(k)) * mag, "q4 s_abs"
    zero = np.zeros((4, 100), dtype=np.uint8)
    y, s = oracle.gemv_q4(zero, _bf16_bits(np.ones((4, 2))), x, so=so)
    assert not y.any() and not s.any(), "all-zero weights"


# --------------------------------------------------------------------------- RMSNorm prologue
def pin_rmsnorm_unit_scale_is_plain_gemv(so):
    """gamma = 1 and eps chosen so that mean(h^2) + eps = 1 exactly: rms_inv = 1 and the
    result must be the (separately pinned) plain GEMV bit for bit."""
    rng = np.random.default_rng(41)
    k = 256
    h = _bf16_bits(rng.choice([-1.0, -0.5, 0.5, 1.0], size=k))   # h^2 in {1/4, 1}
    hv = oracle.bf16_to_f64(h, so=so)
    mean = float(np.sum(hv * hv)) / k                          # exact: a multiple of 1/1024
    eps = 1.0 - mean
    assert 0.0 <= eps < 1.0
    w = _rand_bits(rng, (9, k + 3), 0.02)[:, :k]
    gain = _bf16_bits(np.ones(k))
    y, s = oracle.gemv_rmsnorm(w, h, gain, eps, so=so)
    y0, s0 = oracle.gemv(w, h, so=so)
    assert np.array_equal(y, y0) and np.array_equal(s, s0), "rms_inv = 1 must give the GEMV"


def pin_rmsnorm_closed_forms(so):
    """Constant h = c with eps = 0 gives rms_inv = 1/|c|; a single nonzero h_j = a gives
    mean(h^2) = a^2 / K; W = I gives y = gamma * h * rms_inv elementwise."""
    k = 64
    w = _bf16_bits(np.eye(k))
    gain = _bf16_bits(np.arange(1, k + 1) / 8.0)
    h = _bf16_bits(np.full(k, -4.0))
    y, _ = oracle.gemv_rmsnorm(w, h, gain, 0.0, so=so)
    gv = oracle.bf16_to_f64(gain, so=so)
    assert np.array_equal(y[0], gv * -4.0 / 4.0), "constant h"
    h1 = np.zeros(k)
    h1[5] = 8.0
    eps = 0.75                                   # mean = 64/64 = 1, + 0.75 -> rms = sqrt(1.75)
    y, _ = oracle.gemv_rmsnorm(w, _bf16_bits(h1), gain, eps, so=so)
    want = np.zeros(k)
    want[5] = gv[5] * 8.0 * (1.0 / math.sqrt(1.75))
    assert np.allclose(y[0], want, rtol=1e-15, atol=0), "one nonzero h"


def pin_rmsnorm_scale_invariance(so):
    """With eps = 0 the normalisation cancels any power-of-two scale of h exactly: the sum of
    squares scales by 4^j, its square root by 2^j and the dot product by 2^j, and scaling by
    powers of two commutes with fp64 rounding. So y(2^j h) equals y(h) bit for bit (a mean of
    |h| instead of h^2, a missing square root or a missing scale would all break it)."""
    rng = np.random.default_rng(77)
    n, k = 9, 200
    w = _rand_bits(rng, (n, k), 0.02)
    gain = _rand_bits(rng, (k,), 1.0)
    hv = torch.tensor(rng.standard_normal(k)).to(torch.bfloat16).to(torch.float64).numpy()
    base, _ = oracle.gemv_rmsnorm(w, _bf16_bits(hv), gain, 0.0, so=so)
    for j in (-3, 1, 5):
        y, _ = oracle.gemv_rmsnorm(w, _bf16_bits(hv * 2.0 ** j), gain, 0.0, so=so)
        assert np.array_equal(y, base), f"rmsnorm scale invariance 2^{j}"


def pin_rmsnorm_brute_force(so):
    """Exact rationals where eps makes mean(h^2) + eps a perfect square s^2: rms_inv = 1/s
    exactly, so the whole result is rational."""
    rng = np.random.default_rng(43)
    n, k = 4, 96
    w = _rand_bits(rng, (n, k), 0.02)
    h = _bf16_bits(rng.integers(-8, 9, size=k).astype(np.float64) / 4)
    gain = _rand_bits(rng, (k,), 1.0)
    hx = _exact(h)
    mean = sum(v * v for v in hx) / k
    root = Fraction(math.ceil(math.sqrt(mean)) + 1)
    eps = root * root - mean                     # exact in fp64: a multiple of 1/1536 < 2^53
    assert Fraction(float(eps)) == eps
    y, s = oracle.gemv_rmsnorm(w, h, gain, float(eps), so=so)
    gx = _exact(gain)
    for r in range(n):
        wx = _exact(w[r])
        terms = [a * b * c / root for a, b, c in zip(wx, gx, hx)]
        exact = sum(terms)
        mag = sum(abs(t) for t in terms)
        assert abs(Fraction(y[0, r]) - exact) <= Fraction(gamma(k + 4)) * mag, "rmsnorm brute force"
        assert abs(Fraction(s[0, r]) - mag) <= Fraction(gamma(k + 4)) * mag, "rmsnorm s_abs"


PINS = (pin_bf16_decode, pin_identity, pin_one_hot, pin_constant_w, pin_brute_force,
        pin_cancellation, pin_numpy_matmul, pin_thread_invariance, pin_q4_format,
        pin_q4_equals_bf16_oracle, pin_q4_brute_force, pin_rmsnorm_unit_scale_is_plain_gemv,
        pin_rmsnorm_closed_forms, pin_rmsnorm_scale_invariance, pin_rmsnorm_brute_force)


def run_all(lib_path: str) -> int:
    """Run every pin against the library at lib_path; exit status 0 only if all pass."""
    import ctypes
    so = oracle._bind(ctypes.CDLL(lib_path))
    for pin in PINS:
        try:
            pin(so)
        except AssertionError as e:
            print(f"REJECTED by {pin.__name__}: {e}")
            return 1
    print("all pins pass")
    return 0


if __name__ == "__main__":
    sys.exit(run_all(sys.argv[1]))
