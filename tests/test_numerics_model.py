"""A CPU model of the kernel's per-sub-block arithmetic (host logic, no GPU).

The GEMV forms, per sub-block of one row and one batch row, S = sum v * x with a chain of
v_dot2_f32_bf16 steps (two exact bf16 products added to the fp32 accumulator, one rounding per
step), and then acc += (d*sc) * S - (dmin*m) * X (Q4_K/Q5_K, X = sum x by the same chain with v = 1)
or acc += (d*sc/4) * S (Q6_K, v = 4(q - 32)), each an fp32 FMA.  This file models that order in
numpy and checks what the per-output bound 1e-4 * sum |w x| needs from it:

* with exact operands (v = q, or 4(q - 32)) the error stays within the bound on rows whose sum comes
  from one or two weights (near-empty rows: zero mins, Q6_K quants at 32), and on random rows;
* the model can see the failure this replaced: operands with an offset removed afterwards
  (S over 128 + q minus T over 128, Q6_K 160) break the bound on the same near-empty rows;
* for Q4_K/Q5_K the two-term form is bounded by sum (|d sc q| + |dmin m|) |x|, which is the only
  bound it has when the two terms cancel for every element of a sub-block (w = 0 with q, m != 0).
"""
import numpy as np

U = 2.0 ** -24
N = 4000            # trials (rows) per case


def bf16(v):
    """Round float64 values to bf16 (nearest even), returned as float64."""
    f = np.asarray(v, dtype=np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    u = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16) << 16
    return u.astype(np.uint32).view(np.float32).astype(np.float64)


def f32(v):
    return np.asarray(v, dtype=np.float64).astype(np.float32).astype(np.float64)


def dot2_chain(v, x):
    """[trials, n] operands and activations -> fp32 chain of pair steps, one rounding per step."""
    s = np.zeros(v.shape[0])
    for i in range(0, v.shape[1], 2):
        s = f32(s + v[:, i] * x[:, i] + v[:, i + 1] * x[:, i + 1])
    return s


def model_q45(d, sc, dmin, m, q, x, offset=0):
    """One sub-block of 32 (Q4_K/Q5_K): the kernel's order; offset > 0 models the replaced scheme."""
    ca, cm = f32(d * sc), f32(dmin * m)
    if offset:
        S = dot2_chain(q + offset, x)
        T = dot2_chain(np.full_like(q, offset), x)
        acc = f32(ca * f32(S - T))
        return f32(acc - f32(cm / offset) * T)
    S = dot2_chain(q, x)
    X = dot2_chain(np.ones_like(q), x)
    acc = f32(ca * S)
    return f32(acc - cm * X)


def model_q6(d, sc, q, x, offset=0):
    """One sub-block of 16 (Q6_K)."""
    if offset:
        S = dot2_chain(q + offset, x)
        T = dot2_chain(np.full_like(q, offset + 32), x)
        return f32(f32(d * sc) * f32(S - T))
    return f32(f32(d * sc / 4) * dot2_chain(4 * (q - 32), x))


def exact_q45(d, sc, dmin, m, q, x):
    w = d[:, None] * sc[:, None] * q - (dmin * m)[:, None]
    return (w * x).sum(1), np.abs(w * x).sum(1), ((np.abs(d * sc)[:, None] * q + np.abs(dmin * m)[:, None]) * np.abs(x)).sum(1)


def exact_q6(d, sc, q, x):
    w = (d * sc)[:, None] * (q - 32)
    return (w * x).sum(1), np.abs(w * x).sum(1)


def _fields(rng, n):
    d = np.abs(rng.standard_normal(n)).astype(np.float16).astype(np.float64) * 1e-2
    d = d.astype(np.float16).astype(np.float64)
    return d


def _x(rng, n, width, tiny_at=None):
    x = bf16(rng.standard_normal((n, width)))
    if tiny_at is not None:
        x[np.arange(n), tiny_at] = bf16(x[np.arange(n), tiny_at] * 2.0 ** -12)
    return x


def _near_empty(rng, width, qmax, zero):
    q = np.full((N, width), zero, dtype=np.float64)
    pos = rng.integers(0, width, N)
    val = rng.integers(0, qmax, N)
    val = np.where(val == zero, (val + 1) % qmax, val)
    q[np.arange(N), pos] = val
    return q, pos


def _ratio(y, ye, a):
    err = np.abs(y - ye)
    return np.where(a > 0, err / np.where(a > 0, a, 1.0), np.where(err > 0, np.inf, 0.0))


def test_q4_q5_near_empty_rows_within_bound():
    rng = np.random.default_rng(11)
    for qmax in (16, 32):
        q, pos = _near_empty(rng, 32, qmax, 0)
        x = _x(rng, N, 32, tiny_at=np.where(rng.random(N) < 0.5, pos, rng.integers(0, 32, N)))
        d = _fields(rng, N)
        sc = rng.integers(1, 64, N).astype(np.float64)
        dmin = _fields(rng, N)
        m = np.where(rng.random(N) < 0.5, 0.0, rng.integers(0, 64, N)).astype(np.float64)
        dmin = np.where(m == 0, dmin, 0.0)            # zero mins or zero dmin
        ye, a, _ = exact_q45(d, sc, dmin, m, q, x)
        assert _ratio(model_q45(d, sc, dmin, m, q, x), ye, a).max() <= 1e-4
        # the offset scheme the kernel replaced fails on the same rows
        assert _ratio(model_q45(d, sc, dmin, m, q, x, offset=128), ye, a).max() > 1e-4


def test_q6_near_empty_rows_within_bound():
    rng = np.random.default_rng(12)
    q, pos = _near_empty(rng, 16, 64, 32)
    x = _x(rng, N, 16, tiny_at=np.where(rng.random(N) < 0.5, pos, rng.integers(0, 16, N)))
    d = _fields(rng, N)
    sc = rng.integers(-64, 64, N).astype(np.float64)
    ye, a = exact_q6(d, sc, q, x)
    assert _ratio(model_q6(d, sc, q, x), ye, a).max() <= 1e-4
    assert _ratio(model_q6(d, sc, q, x, offset=128), ye, a).max() > 1e-4


def test_random_rows_within_bound():
    rng = np.random.default_rng(13)
    for qmax in (16, 32):
        q = rng.integers(0, qmax, (N, 32)).astype(np.float64)
        x = _x(rng, N, 32)
        d, dmin = _fields(rng, N), _fields(rng, N)
        sc, m = rng.integers(0, 64, N).astype(np.float64), rng.integers(0, 64, N).astype(np.float64)
        ye, a, _ = exact_q45(d, sc, dmin, m, q, x)
        assert _ratio(model_q45(d, sc, dmin, m, q, x), ye, a).max() <= 1e-5
    q = rng.integers(0, 64, (N, 16)).astype(np.float64)
    x = _x(rng, N, 16)
    d = _fields(rng, N)
    sc = rng.integers(-64, 64, N).astype(np.float64)
    ye, a = exact_q6(d, sc, q, x)
    assert _ratio(model_q6(d, sc, q, x), ye, a).max() <= 1e-5


def test_q4_two_term_bound_when_terms_cancel():
    """q constant c and dmin*m = d*sc*c: every w is 0, yet S and X are rounded separately.  The
    output is then bounded by sum (|d sc q| + |dmin m|) |x|, not by sum |w x| = 0."""
    rng = np.random.default_rng(14)
    c = rng.integers(1, 16, N).astype(np.float64)
    d = _fields(rng, N)
    sc = rng.integers(1, 4, N).astype(np.float64)
    m = sc * c                                      # < 64
    dmin = d                                        # so dmin * m == d * sc * c exactly
    q = np.repeat(c[:, None], 32, axis=1)
    x = _x(rng, N, 32)
    ye, a, ab = exact_q45(d, sc, dmin, m, q, x)
    assert np.all(a == 0)
    err = np.abs(model_q45(d, sc, dmin, m, q, x) - ye)
    assert err.max() > 0                            # the sum |w x| bound cannot hold here
    assert np.all(err <= 32 * U * ab)               # the two-term bound does
