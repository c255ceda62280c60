"""CPU tests of the parity oracle: every pin, the tolerance rule, and planted mistakes."""
import os
import subprocess
import sys

import numpy as np
import pytest

import oracle
import oracle_pins
from oracle.build import SOURCE, build

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def so():
    return oracle.lib()


@pytest.mark.parametrize("pin", oracle_pins.PINS, ids=lambda p: p.__name__)
def test_pin(so, pin):
    pin(so)


def test_check_boundary():
    """The tolerance rule: at the allowance passes, just past it fails, NaN always fails."""
    y_ref = np.array([[1.0, -2.0, 0.0, 5.0]])
    s_abs = np.array([[3.0, 4.0, 0.0, 1.0]])
    allow = 1e-5 * s_abs + 1e-6
    assert oracle.check(y_ref + 0.999 * allow, y_ref, s_abs).ok
    assert oracle.check(y_ref - 0.999 * allow, y_ref, s_abs).ok
    over = y_ref.copy()
    over[0, 1] += 1.01 * allow[0, 1]
    rep = oracle.check(over, y_ref, s_abs)
    assert not rep.ok and rep.n_fail == 1 and rep.first_fail == (0, 1)
    nan = y_ref.copy()
    nan[0, 2] = np.nan
    rep = oracle.check(nan, y_ref, s_abs)
    assert not rep.ok and rep.n_nan == 1
    # the absolute floor alone covers an output whose terms are all zero
    assert oracle.check(np.array([[9e-7]]), np.array([[0.0]]), np.array([[0.0]])).ok
    assert not oracle.check(np.array([[2e-6]]), np.array([[0.0]]), np.array([[0.0]])).ok


def test_bad_arguments(so):
    w = np.zeros((2, 4), dtype=np.uint16)
    with pytest.raises(TypeError):
        oracle.gemv(w.astype(np.float32), np.zeros(4, np.uint16), so=so)
    with pytest.raises(ValueError):
        oracle.gemv(w, np.zeros(5, np.uint16), so=so)   # X longer than W's rows


def test_empty_shapes(so):
    y, s = oracle.gemv(np.zeros((0, 8), np.uint16), np.zeros((1, 8), np.uint16), so=so)
    assert y.shape == (1, 0)
    y, s = oracle.gemv(np.zeros((3, 0), np.uint16), np.zeros((2, 0), np.uint16), so=so)
    assert y.shape == (2, 3) and not y.any() and not s.any()


# Each mutation is a plausible slip in writing the oracle. At least one pin must reject
# every one of them; a mutant that crashes is rejected too.
MUTATIONS = {
    "drop_last_term": ("k < K; ++k", "k < K - 1; ++k"),
    "skip_first_term": ("int64_t k = 0; k < K", "int64_t k = 1; k < K"),
    "wrong_sign": ("sum += p;", "sum -= p;"),
    "fp32_accumulator": ("double sum = 0.0;", "float sum = 0.0f;"),
    "ignore_ldw": ("W + n * ldw", "W + n * K"),
    "ignore_ldx": ("X + m * ldx", "X + m * K"),
    "transposed_output": ("Y[m * N + n] = sum;", "Y[n * M + m] = sum;"),
    "decode_shift": ("(uint32_t)bits << 16", "(uint32_t)bits << 15"),
    "decode_drops_sign": ("(uint32_t)bits << 16", "(uint32_t)(bits & 0x7fff) << 16"),
    "abs_without_fabs": ("mag += fabs(p);", "mag += p;"),
    "w_index_transposed": ("bf16_value(w[k])", "bf16_value(W[k * ldw + n])"),
    "x_index_by_row": ("bf16_value(x[k])", "bf16_value(x[n % K])"),
    "stale_row_pointer": ("const uint16_t *w = W + n * ldw;", "const uint16_t *w = W + m * ldw;"),
    "q4_unsigned_nibble": ("int v = nibble >= 8 ? nibble - 16 : nibble;", "int v = nibble;"),
    "q4_nibble_order": ("(j & 1) ? (row[j >> 1] >> 4) : (row[j >> 1] & 0x0F)",
                        "(j & 1) ? (row[j >> 1] & 0x0F) : (row[j >> 1] >> 4)"),
    "q4_group_64": ("#define ORACLE_Q4_GROUP 128", "#define ORACLE_Q4_GROUP 64"),
    "q4_scale_dropped": ("return (double)v * bf16_value(scales[j / ORACLE_Q4_GROUP]);",
                         "return (double)v;"),
    "q4_ignore_ldq": ("Wq + row * ldq", "Wq + row * ((K + 1) / 2)"),
    "q4_ignore_lds": ("Sc + row * lds", "Sc + row * ((K + 127) / 128)"),
    "q4_abs_without_fabs": ("magnitude += fabs(term);", "magnitude += term;"),
    "norm_eps_dropped": ("sqrt(squares / (double)K + eps)", "sqrt(squares / (double)K)"),
    "norm_mean_over_n": ("squares / (double)K", "squares / (double)(N > 0 ? N : 1)"),
    "norm_gamma_dropped": ("(bf16_value(G[i]) * bf16_value(H[i]))", "bf16_value(H[i])"),
    "norm_no_sqrt": ("1.0 / sqrt(squares / (double)K + eps)", "1.0 / (squares / (double)K + eps)"),
    "norm_scale_missing": ("Y[row] = rms_inv * dot;", "Y[row] = dot;"),
    "norm_abs_not_square": ("squares += hv * hv;", "squares += fabs(hv);"),
}


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_planted_mistake_is_caught(tmp_path, name):
    old, new = MUTATIONS[name]
    src = open(SOURCE).read()
    assert src.count(old) == 1, f"mutation anchor for {name} not unique"
    mutant_c = tmp_path / f"{name}.c"
    mutant_c.write_text(src.replace(old, new))
    mutant_so = build(str(mutant_c), str(tmp_path / f"lib{name}.so"), extra=["-Wno-error"])
    code = ("import sys; sys.path[:0] = [%r, %r]; import oracle_pins; "
            "sys.exit(oracle_pins.run_all(%r))" % (ROOT, os.path.join(ROOT, "tests"), mutant_so))
    proc = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True,
                          timeout=300, cwd=ROOT)
    assert proc.returncode != 0, f"mutant {name} passed every pin:\n{proc.stdout}{proc.stderr}"
