"""The CPU oracle against its pins, and the pins against planted mistakes."""
import os

import numpy as np
import shutil
import tempfile

import pytest

from oracle import oracle as O
from tests import oracle_pins as P


@pytest.fixture(scope="module")
def oracle():
    return O.default()


@pytest.mark.parametrize("pin", P.ALL_PINS, ids=lambda p: p.__name__)
def test_pin(oracle, pin):
    pin(oracle)


# Each mutant is a plausible slip in the oracle's C source; at least one pin must catch it.
MUTANTS = [
    ("q4k nibble halves swapped", "int q = (r < 32) ? (byte & 15) : (byte >> 4);",
     "int q = (r < 32) ? (byte >> 4) : (byte & 15);"),
    ("q4k scale high bits from wrong byte", "*sc = (s[j + 4] & 15) | ((s[j - 4] >> 6) << 4);",
     "*sc = (s[j + 4] & 15) | ((s[j] >> 6) << 4);"),
    ("q4k min low bits from scale nibble", "*m = (s[j + 4] >> 4) | ((s[j] >> 6) << 4);",
     "*m = (s[j + 4] & 15) | ((s[j] >> 6) << 4);"),
    ("dropped min term", "w[e] = d * sc * q - dmin * m;", "w[e] = d * sc * q;"),
    ("min term sign", "w[e] = d * sc * q - dmin * m;", "w[e] = d * sc * q + dmin * m;"),
    ("q5k wrong high bit", "q += ((qh[e % 32] >> g) & 1) << 4;", "q += ((qh[e % 32] >> (g ^ 1)) & 1) << 4;"),
    ("q6k offset", "w[e] = d * scales[e / 16] * (q - 32);", "w[e] = d * scales[e / 16] * (q - 31);"),
    ("q6k scale granularity", "w[e] = d * scales[e / 16] * (q - 32);", "w[e] = d * scales[e / 32] * (q - 32);"),
    ("q6k high bit shift", "int hi = (qh[32 * h + i] >> (2 * r)) & 3;", "int hi = (qh[32 * h + i] >> r) & 3;"),
    ("q6k low-byte index", "int lbyte = ql[64 * h + 32 * (r & 1) + i];", "int lbyte = ql[64 * h + 32 * (r >> 1) + i];"),
    ("fp16 subnormal exponent", "v = ldexp((double)man, -24);", "v = ldexp((double)man, -25);"),
    ("fp16 normal bias", "v = ldexp((double)(man | 0x400), exp - 25);", "v = ldexp((double)(man | 0x400), exp - 24);"),
    ("bf16 shift", "uint32_t u = (uint32_t)b << 16;", "uint32_t u = (uint32_t)b << 15;"),
    ("x row ignored", "const double *xb = xd + b * cols + s * 256;", "const double *xb = xd + s * 256;"),
    ("abs dropped", "magp[b] += fabs(p);", "magp[b] += p;"),
]


@pytest.mark.parametrize("name,orig,mut", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_pins_catch_planted_mistake(name, orig, mut):
    src = open(O._SRC).read()
    assert src.count(orig) == 1, f"mutation anchor not found: {orig}"
    d = tempfile.mkdtemp(prefix="kqo_mut_")
    try:
        path = os.path.join(d, "mut.c")
        open(path, "w").write(src.replace(orig, mut))
        so = os.path.join(d, "libmut.so")
        O.compile_c(path, so)
        bad = O.Oracle(so)
        caught = []
        for pin in P.ALL_PINS:
            try:
                pin(bad)
            except (AssertionError, ValueError) as e:
                caught.append(f"{pin.__name__}: {e}")
        assert caught, f"no pin caught mutant '{name}'"
    finally:
        shutil.rmtree(d, ignore_errors=True)


def test_silu_closed_forms():
    """silu pins that do not retype its formula: silu(0) = 0, the odd part silu(g) - silu(-g) = g,
    sigmoid(ln 3) = 3/4 so silu(ln 3) = 0.75 ln 3, the limits g and 0, and swiglu(g, u) = silu(g) u."""
    import math
    assert O.silu(0.0) == 0.0
    g = np.linspace(-30.0, 30.0, 601)
    assert np.allclose(O.silu(g) - O.silu(-g), g, rtol=0, atol=1e-13)
    assert abs(O.silu(math.log(3.0)) - 0.75 * math.log(3.0)) < 1e-15
    assert O.silu(800.0) == 800.0 and O.silu(-800.0) == 0.0
    assert abs(O.silu(40.0) - 40.0) < 1e-14 and abs(O.silu(-40.0)) < 1e-15
    assert np.array_equal(O.swiglu(g, 2.0 * np.ones_like(g)), 2.0 * O.silu(g))


def test_gather_is_rows_of_dequant():
    from quant_weight_streaming_amd import synth
    g = synth.gen_weights("q4k", 70, 512, 5).numpy()
    ids = [69, 0, 64, 5, 5]
    full = O.dequant_f32("q4k", 70, 512, g)
    assert np.array_equal(O.gather("q4k", 70, 512, g, ids), full[ids])


def test_sigmoid_closed_forms():
    """sigmoid(0) = 1/2, sigmoid(v) + sigmoid(-v) = 1, sigmoid(ln 3) = 3/4, the limits, and
    silu(v) = v sigmoid(v)."""
    import math
    assert O.sigmoid(0.0) == 0.5
    v = np.linspace(-40.0, 40.0, 801)
    assert np.allclose(O.sigmoid(v) + O.sigmoid(-v), 1.0, rtol=0, atol=1e-15)
    assert abs(O.sigmoid(math.log(3.0)) - 0.75) < 1e-15
    assert O.sigmoid(800.0) == 1.0 and O.sigmoid(-800.0) == 0.0
    assert np.allclose(O.silu(v), v * O.sigmoid(v), rtol=1e-15, atol=0)


def test_rmsnorm_pins():
    """Hand-computed values, the unit mean square at eps = 0, scale invariance and the eps term."""
    import math
    x = np.array([[3.0, 4.0]])
    assert np.allclose(O.rmsnorm(x, 0.0), [[3 / math.sqrt(12.5), 4 / math.sqrt(12.5)]], rtol=1e-15, atol=0)
    assert (O.rmsnorm(np.ones((1, 4)), 3.0) == 0.5).all()             # 1 / sqrt(1 + 3)
    assert (O.rmsnorm(np.full((2, 8), -2.0), 0.0) == -1.0).all()
    r = np.random.default_rng(1).standard_normal((3, 1000))
    n = O.rmsnorm(r, 0.0)
    assert np.allclose(np.mean(n * n, axis=1), 1.0, rtol=1e-13)
    assert np.allclose(O.rmsnorm(7.5 * r, 0.0), n, rtol=1e-13, atol=0)
    m = np.mean(r * r, axis=1)
    assert np.allclose(np.mean(O.rmsnorm(r, 0.25) ** 2, axis=1), m / (m + 0.25), rtol=1e-13)
    assert (O.rmsnorm(np.zeros((1, 16)), 1e-5) == 0.0).all()


def test_gemv_rmsnorm_is_the_scaled_gemv():
    """W rmsnorm(x) equals the oracle GEMV of x divided by rms(x) (the C oracle's own dot products), for bf16
    bits and fp32 x; and a zero x row gives y = a = 0."""
    import torch
    from quant_weight_streaming_amd import synth
    rows, cols = 70, 512
    g = synth.gen_weights("q6k", rows, cols, synth.seed_of("onorm"))
    xb = synth.gen_x(2, cols, synth.seed_of("onorm-x"), "bf16").view(torch.int16).numpy().view(np.uint16)
    y0, a0 = O.gemv("q6k", rows, cols, g.numpy(), xb)
    xd = (xb.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    rms = np.sqrt(np.mean(xd * xd, axis=1, keepdims=True) + 1e-5)
    y, a = O.gemv_rmsnorm("q6k", rows, cols, g.numpy(), xb, 1e-5)
    assert np.allclose(y, y0 / rms, rtol=0, atol=1e-12 * (a0 / rms).max())
    assert np.allclose(a, a0 / rms, rtol=1e-12)
    xf = synth.gen_x(1, cols, synth.seed_of("onorm-xf"), "f32").numpy()
    xf[0, :] = 0.0
    y, a = O.gemv_rmsnorm("q6k", rows, cols, g.numpy(), xf, 1e-8)
    assert (y == 0).all() and (a == 0).all()


def test_head_rmsnorm_pins():
    """Per-head closed forms: a constant head c maps to c / sqrt(c^2 + eps); heads are independent; every head of
    the output has mean square m / (m + eps) of its input's mean square m."""
    import math
    v = np.concatenate([np.full((1, 128), 3.0), np.full((1, 128), -0.5)], axis=1)
    out = O.head_rmsnorm(v, 0.25)
    assert np.allclose(out[0, :128], 3.0 / math.sqrt(9.25), rtol=1e-15)
    assert np.allclose(out[0, 128:], -0.5 / math.sqrt(0.5), rtol=1e-15)
    r = np.random.default_rng(2).standard_normal((2, 512))
    a = O.head_rmsnorm(r, 1e-3)
    r2 = r.copy()
    r2[:, 128:256] *= 100.0                        # only head 1 changes
    b = O.head_rmsnorm(r2, 1e-3)
    assert (a[:, :128] == b[:, :128]).all() and (a[:, 256:] == b[:, 256:]).all()
    m = np.mean(r.reshape(2, 4, 128) ** 2, axis=-1)
    got = np.mean(a.reshape(2, 4, 128) ** 2, axis=-1)
    assert np.allclose(got, m / (m + 1e-3), rtol=1e-13)
    with pytest.raises(ValueError):
        O.head_rmsnorm(np.ones((1, 100)), 1e-6)
