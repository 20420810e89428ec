"""Pins of the CPU oracle against facts that do not come from the oracle itself.

Each ``pin_*`` function takes an oracle object (``oracle.oracle.Oracle``) and
raises AssertionError when the oracle disagrees with:
  * hand-evaluated closed forms of the K-quant formulas
    (w = d*sc*q - dmin*m for Q4_K/Q5_K, w = d*sc*(q-32) for Q6_K);
  * numpy's IEEE binary16 decoder and the bf16 = top-half-of-binary32 rule;
  * the generator's independent field encoder, exhaustively over the 6-bit
    scale/min field;
  * exact rational arithmetic (fractions.Fraction) on tiny random blocks;
  * numpy's float64 matmul, and invariants of a linear map.
The same pins are run against deliberately broken copies of the oracle
(test_oracle.py) to show that each plausible mistake is caught.
"""
from __future__ import annotations

from fractions import Fraction

import numpy as np
import torch

from quant_weight_streaming_amd import synth

F16_ONE, F16_HALF, F16_QUARTER = 0x3C00, 0x3800, 0x3400


def _t(a, dtype=torch.int32):
    return torch.as_tensor(np.asarray(a), dtype=dtype)


def _frac_f16(bits: int) -> Fraction:
    return Fraction(float(np.array([bits], dtype=np.uint16).view(np.float16)[0]))


def pin_f16_exhaustive(O):
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = bits.view(np.float16).astype(np.float64)
    got = np.array([O.f16_to_double(int(b)) for b in bits])
    fin = np.isfinite(ref)
    assert np.array_equal(got[fin], ref[fin]), "fp16 decode mismatch"
    assert np.all(np.signbit(got[fin]) == np.signbit(ref[fin])), "fp16 sign of zero"
    assert np.all(np.isnan(got[~fin])), "fp16 inf/nan must decode to NaN (rejected)"


def pin_bf16_exhaustive(O):
    bits = np.arange(0, 65536, 7, dtype=np.uint32)
    with np.errstate(invalid="ignore"):
        ref = (bits << 16).astype(np.uint32).view(np.float32).astype(np.float64)
    got = np.array([O.bf16_to_double(int(b)) for b in bits])
    fin = np.isfinite(ref)
    assert np.array_equal(got[fin], ref[fin]), "bf16 decode mismatch"


def pin_q4k_hand_blocks(O):
    # d = 0.5, dmin = 0.25, sc = 2, m = 3, q = 5  ->  0.5*2*5 - 0.25*3 = 4.25 everywhere
    n = 1
    g = synth.pack_q4k(_t([F16_HALF]), _t([F16_QUARTER]), torch.full((n, 8), 2), torch.full((n, 8), 3),
                       torch.full((n, 256), 5))
    w = O.dequant("q4k", 1, 256, g.numpy())
    assert np.all(w == 4.25), "Q4_K closed form 4.25"
    # d = 1, dmin = 0, sc = 1, m = 0  ->  w = q, element by element
    q = torch.arange(256) % 16
    q = q[torch.randperm(256, generator=torch.Generator().manual_seed(1))]
    g = synth.pack_q4k(_t([F16_ONE]), _t([0]), torch.ones(1, 8), torch.zeros(1, 8), q[None])
    w = O.dequant("q4k", 1, 256, g.numpy())
    assert np.array_equal(w[0], q.numpy().astype(np.float64)), "Q4_K quant order"
    # d = 0 -> w = -dmin * m, independent of q
    g = synth.pack_q4k(_t([0]), _t([F16_ONE]), torch.full((1, 8), 63), _t([[0, 1, 2, 3, 60, 61, 62, 63]]),
                       torch.full((1, 256), 15))
    w = O.dequant("q4k", 1, 256, g.numpy())
    assert np.array_equal(w[0], -np.repeat([0, 1, 2, 3, 60, 61, 62, 63], 32).astype(float)), "Q4_K min term"


def pin_q4k_scale_field_exhaustive(O):
    """Every (sc, m) in 0..63 x 0..63 at every sub-block position j."""
    k = np.arange(4096)
    sc = np.stack([(k + 7 * j) % 64 for j in range(8)], 1)
    m = np.stack([(k // 64 + 11 * j) % 64 for j in range(8)], 1)
    q = np.zeros((4096, 256), dtype=np.int64)
    q.reshape(4096, 8, 32)[:, :, 16:] = 1            # first half of each sub-block q=0, second half q=1
    g = synth.pack_q4k(_t(np.full(4096, F16_ONE)), _t(np.full(4096, F16_ONE)), _t(sc), _t(m), _t(q))
    w = O.dequant("q4k", 4096, 256, g.numpy()).reshape(4096, 8, 32)
    assert np.array_equal(w[:, :, 0], -m.astype(float)), "6-bit min unpack"
    assert np.array_equal(w[:, :, 16], (sc - m).astype(float)), "6-bit scale unpack"


def pin_q5k_vs_q4k(O):
    rng = np.random.default_rng(5)
    n = 16
    d = _t(rng.integers(0x1000, 0x2C00, n)); dmin = _t(rng.integers(0x1000, 0x2C00, n))
    sc = _t(rng.integers(0, 64, (n, 8))); m = _t(rng.integers(0, 64, (n, 8)))
    q4 = rng.integers(0, 16, (n, 256))
    w4 = O.dequant("q4k", n, 256, synth.pack_q4k(d, dmin, sc, m, _t(q4)).numpy())
    w5 = O.dequant("q5k", n, 256, synth.pack_q5k(d, dmin, sc, m, _t(q4)).numpy())
    assert np.array_equal(w4, w5), "Q5_K with zero fifth bits must equal Q4_K"
    hb = rng.integers(0, 2, (n, 256))
    w5h = O.dequant("q5k", n, 256, synth.pack_q5k(d, dmin, sc, m, _t(q4 + 16 * hb)).numpy())
    dd = np.array([float(np.array([v], np.uint16).view(np.float16)[0]) for v in d.numpy()])
    extra = 16.0 * dd[:, None] * np.repeat(sc.numpy(), 32, axis=1) * hb
    assert np.array_equal(w5h, w4 + extra), "Q5_K fifth bit adds 16*d*sc"


def pin_q6k_hand_blocks(O):
    # d = 0.5, sc = -3, q = 40  ->  0.5 * -3 * 8 = -12 ; q = 32 -> 0
    g = synth.pack_q6k(_t([F16_HALF]), torch.full((1, 16), -3), torch.full((1, 256), 40))
    assert np.all(O.dequant("q6k", 1, 256, g.numpy()) == -12.0), "Q6_K closed form -12"
    g = synth.pack_q6k(_t([F16_HALF]), torch.full((1, 16), -3), torch.full((1, 256), 32))
    assert np.all(O.dequant("q6k", 1, 256, g.numpy()) == 0.0), "Q6_K q=32 gives 0"
    # d = 1, sc = 1: w = q - 32 element by element (pins the ql/qh bit positions)
    q = torch.arange(256) % 64
    q = q[torch.randperm(256, generator=torch.Generator().manual_seed(3))]
    g = synth.pack_q6k(_t([F16_ONE]), torch.ones(1, 16), q[None])
    assert np.array_equal(O.dequant("q6k", 1, 256, g.numpy())[0], q.numpy() - 32.0), "Q6_K quant order"
    # distinct scale per 16-element sub-block, q = 33 -> w = sc_g
    sc = torch.tensor([[-64, -50, -7, -1, 0, 1, 2, 3, 5, 8, 13, 21, 34, 55, 62, 63]])
    g = synth.pack_q6k(_t([F16_ONE]), sc, torch.full((1, 256), 33))
    assert np.array_equal(O.dequant("q6k", 1, 256, g.numpy())[0], np.repeat(sc.numpy()[0], 16).astype(float)), \
        "Q6_K scale per sub-block"


def _random_fields(qtype, n, rng, subnormal=True):
    lo = 1 if subnormal else 0x0400
    d = rng.integers(lo, 0x3000, n)
    dmin = rng.integers(lo, 0x3000, n)
    if qtype == "q6k":
        return dict(d=d, sc=rng.integers(-64, 64, (n, 16)), q=rng.integers(0, 64, (n, 256)))
    qmax = 16 if qtype == "q4k" else 32
    return dict(d=d, dmin=dmin, sc=rng.integers(0, 64, (n, 8)), m=rng.integers(0, 64, (n, 8)),
                q=rng.integers(0, qmax, (n, 256)))


def _pack(qtype, f):
    if qtype == "q6k":
        return synth.pack_q6k(_t(f["d"]), _t(f["sc"]), _t(f["q"]))
    p = synth.pack_q4k if qtype == "q4k" else synth.pack_q5k
    return p(_t(f["d"]), _t(f["dmin"]), _t(f["sc"]), _t(f["m"]), _t(f["q"]))


def _exact_w(qtype, f, i, e) -> Fraction:
    if qtype == "q6k":
        return _frac_f16(int(f["d"][i])) * int(f["sc"][i][e // 16]) * (int(f["q"][i][e]) - 32)
    g = e // 32
    return (_frac_f16(int(f["d"][i])) * int(f["sc"][i][g]) * int(f["q"][i][e])
            - _frac_f16(int(f["dmin"][i])) * int(f["m"][i][g]))


def pin_fraction_dequant(O):
    rng = np.random.default_rng(11)
    for qtype in ("q4k", "q5k", "q6k"):
        n = 4                                  # 2 rows x 512 cols = 4 super-blocks
        f = _random_fields(qtype, n, rng)
        w = O.dequant(qtype, 2, 512, _pack(qtype, f).numpy()).reshape(n, 256)
        for i in range(n):
            for e in range(256):
                assert Fraction(w[i, e]) == _exact_w(qtype, f, i, e), f"{qtype} exact value sb {i} el {e}"


def pin_fraction_gemv(O):
    rng = np.random.default_rng(12)
    for qtype in ("q4k", "q5k", "q6k"):
        rows, cols, batch = 3, 512, 3
        n = rows * cols // 256
        f = _random_fields(qtype, n, rng)
        g = _pack(qtype, f).numpy()
        xbits = (rng.normal(size=(batch, cols)).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
        y, a = O.gemv(qtype, rows, cols, g, xbits)
        xfr = [[Fraction(float((np.uint32(v) << 16).view(np.float32))) for v in row] for row in xbits]
        for b in range(batch):
            for r in range(rows):
                ex = Fraction(0)
                mag = Fraction(0)
                for k in range(cols):
                    i, e = r * (cols // 256) + k // 256, k % 256
                    t = _exact_w(qtype, f, i, e) * xfr[b][k]
                    ex += t
                    mag += abs(t)
                assert abs(Fraction(y[b, r]) - ex) <= Fraction(1, 10**12) * mag, f"{qtype} y[{b},{r}]"
                assert abs(Fraction(a[b, r]) - mag) <= Fraction(1, 10**12) * mag, f"{qtype} a[{b},{r}]"


def pin_matmul_and_invariants(O):
    w = synth.gen_weights("q4k", 256, 1024, 0)
    x = synth.gen_x(1, 1024, 0, "f32").numpy()
    W = O.dequant("q4k", 256, 1024, w.numpy())
    y, a = O.gemv("q4k", 256, 1024, w.numpy(), x)
    ref = W @ x[0].astype(np.float64)
    assert np.all(np.abs(y[0] - ref) <= 1e-12 * a[0]), "gemv vs numpy float64 matmul"
    assert np.allclose(a[0], np.abs(W) @ np.abs(x[0].astype(np.float64)), rtol=1e-12, atol=0), "sum |w x|"
    # one-hot x picks a column exactly; 2x doubles y exactly; x = 0 gives 0
    for qtype in ("q4k", "q5k", "q6k"):
        g = synth.gen_weights(qtype, 8, 512, 7)
        Wq = O.dequant(qtype, 8, 512, g.numpy())
        oh = np.zeros((3, 512), dtype=np.float32)
        cols = [0, 257, 511]
        for b, c in enumerate(cols):
            oh[b, c] = 1.0
        yo, _ = O.gemv(qtype, 8, 512, g.numpy(), oh)
        for b, c in enumerate(cols):
            assert np.array_equal(yo[b], Wq[:, c]), f"{qtype} one-hot column {c}"
        xr = synth.gen_x(2, 512, 9, "f32").numpy()
        y1, _ = O.gemv(qtype, 8, 512, g.numpy(), xr)
        y2, _ = O.gemv(qtype, 8, 512, g.numpy(), 2 * xr)
        assert np.array_equal(2 * y1, y2), f"{qtype} homogeneity"
        y0, a0 = O.gemv(qtype, 8, 512, g.numpy(), np.zeros((1, 512), np.float32))
        assert np.all(y0 == 0) and np.all(a0 == 0), f"{qtype} zero input"
        # bf16 path reads the same numbers as the fp32 path when x is bf16-representable
        xb = synth.gen_x(2, 512, 9, "bf16")
        yb, _ = O.gemv(qtype, 8, 512, g.numpy(), xb.view(torch.int16).numpy().view(np.uint16))
        yf, _ = O.gemv(qtype, 8, 512, g.numpy(), xb.float().numpy())
        assert np.array_equal(yb, yf), f"{qtype} bf16 x decode"


ALL_PINS = [pin_f16_exhaustive, pin_bf16_exhaustive, pin_q4k_hand_blocks, pin_q4k_scale_field_exhaustive,
            pin_q5k_vs_q4k, pin_q6k_hand_blocks, pin_fraction_dequant, pin_fraction_gemv,
            pin_matmul_and_invariants]
