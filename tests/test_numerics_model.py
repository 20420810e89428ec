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
  bound it has when the two terms cancel for every element of a sub-block (w = 0 with q, m != 0);
* on the matrix-core path (three or more staged rows) the mins' term is a product of its own: the
  staged sums as three bf16 parts (exact) times m scaled by dmin's power of two; it stays within the
  bound, also on near-empty rows and negative scales, and in range where the output is.
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


# ---- the matrix-core path (three or more staged rows), Q4_K/Q5_K super-blocks of 8 sub-blocks of 32
#
# Per sub-block g the products come from a chain of 4 matrix-core instructions, each adding 8 exact
# products to the fp32 accumulator with one rounding (modelled so), then acc += (d sc_g) S_g (an fp32
# FMA).  The mins' term is one more product: the staged sums X_g (fp32, a dot2 chain over the
# sub-block) split into three bf16 parts, times the row's m_g * p, p the signed power of two of dmin,
# chained over the three parts (one rounding each); then acc -= f * M with f = dmin / p (an FMA).

def bf16_parts(t):
    """fp32 values -> (hi, mid, lo): each the bf16 rounding of what the earlier parts leave."""
    hi = bf16(t)
    r1 = f32(t - hi)
    mid = bf16(r1)
    lo = bf16(f32(r1 - mid))
    return hi, mid, lo


def pow2_split(dmin):
    """dmin -> (p, f): p = sign * 2^floor(log2 |dmin|), f = dmin / p in [1, 2) (1 for a zero dmin)."""
    e = np.floor(np.log2(np.where(dmin != 0, np.abs(dmin), 1.0)))
    p = np.where(dmin != 0, np.sign(dmin) * 2.0 ** e, 0.0)
    return p, np.where(dmin != 0, dmin / np.where(p != 0, p, 1.0), 1.0)


def model_q45_mfma(d, sc, dmin, m, q, x):
    """[trials] super-blocks: d, dmin [n]; sc, m [n, 8]; q, x [n, 256] -> the kernel's order."""
    n = q.shape[0]
    acc = np.zeros(n)
    X = np.zeros((n, 8))
    for g in range(8):
        qs, xs = q[:, 32 * g:32 * g + 32], x[:, 32 * g:32 * g + 32]
        S = np.zeros(n)
        for kb in range(4):
            S = f32(S + (qs[:, 8 * kb:8 * kb + 8] * xs[:, 8 * kb:8 * kb + 8]).sum(1))
        acc = f32(acc + f32(d * sc[:, g]) * S)
        X[:, g] = dot2_chain(np.ones_like(xs), xs)
    p, f = pow2_split(dmin)
    mp = m * p[:, None]
    assert np.array_equal(bf16(mp), mp)                 # m * p is an exact bf16 operand
    M = np.zeros(n)
    for part in bf16_parts(X):
        M = f32(M + (mp * part).sum(1))
    return f32(acc - f * M), M


def exact_q45_sb(d, sc, dmin, m, q, x):
    w = np.repeat(d[:, None] * sc, 32, axis=1) * q - np.repeat(dmin[:, None] * m, 32, axis=1)
    return (w * x).sum(1), np.abs(w * x).sum(1)


def _sb_fields(rng, n, qmax, near_empty=False):
    d, dmin = _fields(rng, n), _fields(rng, n)
    sc = rng.integers(1, 64, (n, 8)).astype(np.float64)
    m = rng.integers(0, 64, (n, 8)).astype(np.float64)
    q = rng.integers(0, qmax, (n, 256)).astype(np.float64)
    if near_empty:                                       # one nonzero quant, zero mins or zero dmin
        q[:] = 0
        pos = rng.integers(0, 256, n)
        q[np.arange(n), pos] = rng.integers(1, qmax, n)
        zero_m = rng.random(n) < 0.5
        m[zero_m] = 0
        dmin = np.where(zero_m, dmin, 0.0)
    return d, sc, dmin, m, q


def test_three_bf16_parts_are_exact():
    """hi + mid + lo is the fp32 value exactly, over the normal fp32 range and both signs (up to the
    largest value whose bf16 rounding is finite, 2^128 - 2^119)."""
    rng = np.random.default_rng(21)
    t = f32(rng.standard_normal(200000) * 2.0 ** rng.integers(-100, 100, 200000))
    edge = [0.0, -0.0, 1.0, -1.0, 3.0e38, -3.0e38, 2.0 ** 128 - 2.0 ** 120, 2.0 ** -100, 1 + 2.0 ** -23]
    t = np.concatenate([t, f32(np.array(edge))])
    hi, mid, lo = bf16_parts(t)
    assert np.array_equal(hi + mid + lo, t)
    for part in (hi, mid, lo):
        assert np.array_equal(bf16(part), part)


def test_mfma_mins_product_within_bound():
    rng = np.random.default_rng(22)
    for qmax in (16, 32):
        for near_empty, tol in ((False, 1e-5), (True, 1e-4)):
            d, sc, dmin, m, q = _sb_fields(rng, N, qmax, near_empty)
            x = _x(rng, N, 256)
            neg = rng.random(N) < 0.3                    # negative fp16 d and dmin are legal
            d, dmin = np.where(neg, -d, d), np.where(rng.random(N) < 0.3, -dmin, dmin)
            ye, a = exact_q45_sb(d, sc, dmin, m, q, x)
            y, _ = model_q45_mfma(d, sc, dmin, m, q, x)
            assert _ratio(y, ye, a).max() <= tol, (qmax, near_empty)


def test_mfma_mins_product_stays_in_range():
    """Activations of 2^100 times 2^-20..2^20 (the GPU range test's mixed row) put outputs near 2^122.
    With dmin's power of two inside the operand the product keeps the magnitude of dmin * m * X and
    stays finite; with plain m (dmin applied after) it is about 1 / dmin times larger and overflows."""
    rng = np.random.default_rng(23)
    d, sc, dmin, m, q = _sb_fields(rng, 256, 16)
    x = _x(rng, 256, 256) * 2.0 ** (100 + rng.integers(-20, 21, (256, 256)))
    ye, a = exact_q45_sb(d, sc, dmin, m, q, x)
    y, M = model_q45_mfma(d, sc, dmin, m, q, x)
    assert np.all(np.isfinite(y)) and np.all(np.abs(M) < 3.4e38)
    assert _ratio(y, ye, a).max() <= 1e-5
    X = np.stack([x[:, 32 * g:32 * g + 32].sum(1) for g in range(8)], 1)
    assert np.any(np.abs((m * X).sum(1)) > np.finfo(np.float32).max)   # the plain-m product overflows
