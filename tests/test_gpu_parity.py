"""HIP path vs the CPU oracle, element by element, through the C ABI.

Dequantised weights must match bit-exactly; every output must satisfy
|y_gpu - y_oracle| <= 1e-4 * sum_k |w_k x_k| (so an output whose terms are all
zero must be exactly zero).  Small cases compare every output; the full-size
workloads (one launch each, as the benchmark issues them) compare sampled rows.
"""
import numpy as np
import pytest
import torch

from oracle import oracle as O
from quant_weight_streaming_amd import kq, synth
from tests.gpu_cases import check_dequant, check_y, oracle_rows, sample_rows, say, x_host

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]
DEV = "cuda:0"


def run_case(qtype, rows, cols, batch, xdtype, seed, merge=0.0, check_w=True):
    say(f"case {qtype} rows={rows} cols={cols} B={batch} x={xdtype} seed={seed}")
    g = synth.gen_weights(qtype, rows, cols, synth.seed_of("w", seed), merge_frac=merge)
    x = synth.gen_x(batch, cols, synth.seed_of("x", seed), xdtype)
    gd = g.to(DEV)
    w = kq.repack(qtype, gd, rows, cols)
    y = kq.gemv(qtype, w, rows, cols, x.to(DEV))
    torch.cuda.synchronize()
    yo, ao = O.gemv(qtype, rows, cols, g.numpy(), x_host(x))
    worst = check_y(y.cpu().numpy(), yo, ao, f"{qtype} {rows}x{cols} B={batch} {xdtype}")
    if check_w:
        check_dequant(qtype, w, rows, cols, g.numpy(), np.arange(rows), f"{qtype} {rows}x{cols}")
    return worst


def test_config0_exact():
    """Q4_K 256 x 1024, batch 1, fp32 x ~ N(0,1), seed 0."""
    run_case("q4k", 256, 1024, 1, "f32", 0)


@pytest.mark.parametrize("qtype", ["q4k", "q5k", "q6k"])
@pytest.mark.parametrize("xdtype", ["bf16", "f32"])
@pytest.mark.parametrize("batch", [1, 2, 3, 4, 5, 6, 7, 8])
def test_small_ragged(qtype, xdtype, batch):
    # 4 row tiles (the last one 17 rows), 5 super-block columns
    run_case(qtype, 3 * 64 + 17, 5 * 256, batch, xdtype, 100 + batch, check_w=(batch == 1))


@pytest.mark.parametrize("qtype", ["q4k", "q5k", "q6k"])
@pytest.mark.parametrize("batch", [1, 8])
def test_units_span_tiles(qtype, batch):
    # 301 tiles x 20 columns: each wavefront takes a run of units that starts and ends inside tiles
    run_case(qtype, 300 * 64 + 37, 20 * 256, batch, "bf16", 200 + batch, check_w=False)


@pytest.mark.parametrize("qtype", ["q4k", "q6k"])
@pytest.mark.parametrize("batch", [1, 8])
def test_runs_span_many_tiles(qtype, batch):
    # one super-block column and 3000 tiles: a wavefront's run covers several whole tiles
    run_case(qtype, 3000 * 64 + 5, 256, batch, "bf16", 250 + batch, check_w=False)


@pytest.mark.parametrize("qtype", ["q4k", "q5k", "q6k"])
@pytest.mark.parametrize("cols_sb", [26, 29])
@pytest.mark.parametrize("xdtype,batch", [("bf16", 8), ("f32", 4)])
def test_window_workgroups_smaller_than_their_wavefronts(qtype, cols_sb, xdtype, batch):
    """Eight staged rows and 26 or 29 super-block columns: column windows of 5 or 6 columns over 4 row tiles,
    one tile per workgroup, so a workgroup has fewer units than wavefronts; its wavefronts take parts of 1 or 0
    units (the longer ones first), and the tile sums still add in unit order."""
    run_case(qtype, 3 * 64 + 9, cols_sb * 256, batch, xdtype, 900 + cols_sb + batch, check_w=False)


@pytest.mark.parametrize("qtype", ["q4k", "q6k"])
def test_long_rows_split_many_ways(qtype):
    # 5 tiles x 122 columns (the down projection's K): one unit per wavefront, 122 partials per tile
    run_case(qtype, 300, 31232, 2, "bf16", 300)


@pytest.mark.parametrize("qtype", ["q4k", "q5k", "q6k"])
def test_single_row_single_column(qtype):
    run_case(qtype, 1, 256, 3, "bf16", 400)
    run_case(qtype, 1, 256, 1, "f32", 401)


@pytest.mark.parametrize("qtype", ["q4k", "q5k", "q6k"])
@pytest.mark.parametrize("xdtype", ["bf16", "f32"])
def test_multi_projection(qtype, xdtype):
    parts = [100, 64, 37]
    cols, batch = 1024, 3
    say(f"case multi {qtype} parts={parts} x={xdtype}")
    gs = [synth.gen_weights(qtype, r, cols, synth.seed_of("multi", qtype, i)) for i, r in enumerate(parts)]
    x = synth.gen_x(batch, cols, 7, xdtype)
    ws = [kq.repack(qtype, g.to(DEV), r, cols) for g, r in zip(gs, parts)]
    # outputs with padded strides to check ldy handling
    ys = [torch.full((batch, r + 5), float("nan"), device=DEV) for r in parts]
    kq.kq_gemv_multi(qtype, ws, parts, cols, x.to(DEV), ys)
    torch.cuda.synchronize()
    for g, r, y in zip(gs, parts, ys):
        yo, ao = O.gemv(qtype, r, cols, g.numpy(), x_host(x))
        check_y(y[:, :r].cpu().numpy(), yo, ao, f"multi {qtype} part {r}")
        assert torch.isnan(y[:, r:]).all(), "wrote outside [0, rows)"


def _fields(qtype, n, rng):
    d = torch.as_tensor(rng.integers(0x1000, 0x2C00, n))
    if qtype == "q6k":
        return dict(d=d, sc=torch.as_tensor(rng.integers(-64, 64, (n, 16))), q=torch.as_tensor(rng.integers(0, 64, (n, 256))))
    qmax = 16 if qtype == "q4k" else 32
    return dict(d=d, dmin=torch.as_tensor(rng.integers(0x1000, 0x2C00, n)), sc=torch.as_tensor(rng.integers(0, 64, (n, 8))),
                m=torch.as_tensor(rng.integers(0, 64, (n, 8))), q=torch.as_tensor(rng.integers(0, qmax, (n, 256))))


def _pack(qtype, f):
    if qtype == "q6k":
        return synth.pack_q6k(f["d"], f["sc"], f["q"])
    p = synth.pack_q4k if qtype == "q4k" else synth.pack_q5k
    return p(f["d"], f["dmin"], f["sc"], f["m"], f["q"])


def _run_fields(qtype, f, rows, cols, x, where):
    g = _pack(qtype, f).reshape(rows, -1)
    w = kq.repack(qtype, g.to(DEV), rows, cols)
    y = kq.gemv(qtype, w, rows, cols, x.to(DEV))
    torch.cuda.synchronize()
    yo, ao = O.gemv(qtype, rows, cols, g.numpy(), x_host(x))
    check_y(y.cpu().numpy(), yo, ao, where)
    check_dequant(qtype, w, rows, cols, g.numpy(), np.arange(rows), where)
    return y.cpu().numpy(), yo, ao


@pytest.mark.parametrize("qtype", ["q4k", "q5k", "q6k"])
@pytest.mark.parametrize("xdtype,batch,path", [("bf16", 2, "mfma"), ("bf16", 8, "mfma"), ("bf16", 2, "dot2"),
                                               ("bf16", 8, "dot2"), ("f32", 2, "dot2")])
def test_zero_rows_are_exactly_zero(qtype, xdtype, batch, path, monkeypatch):
    """Rows whose weights are all zero give exactly 0: zero super-blocks (d = dmin = 0),
    zero quants with zero mins (Q4_K/Q5_K), all quants 32 (Q6_K); on the matrix-core and the dot2 path."""
    monkeypatch.setenv("KQ_MATRIX_CORES_FROM", "2" if path == "mfma" else "9")
    rows, cols = 130, 768
    say(f"case zero rows {qtype} {xdtype} B={batch} {path}")
    rng = np.random.default_rng(1)
    f = _fields(qtype, rows * 3, rng)
    sb = lambda r: slice(3 * r, 3 * r + 3)
    zero_rows = [0, 5, 64, 129]
    f["d"][sb(0)] = 0
    if qtype != "q6k":
        f["dmin"][sb(0)] = 0
        f["q"][sb(5)] = 0; f["m"][sb(5)] = 0
        f["q"][sb(64)] = 0; f["m"][sb(64)] = 0
        f["d"][sb(129)] = 0; f["m"][sb(129)] = 0
    else:
        f["q"][sb(5)] = 32
        f["q"][sb(64)] = 32
        f["sc"][sb(129)] = 0
    x = synth.gen_x(batch, cols, 3, xdtype)
    y, yo, ao = _run_fields(qtype, f, rows, cols, x, f"zero rows {qtype} {xdtype}")
    for r in zero_rows:
        assert np.all(ao[:, r] == 0) and np.all(y[:, r] == 0), f"row {r} not exactly zero"


@pytest.mark.parametrize("qtype", ["q4k", "q5k", "q6k"])
def test_subnormal_and_extreme_scales(qtype):
    rows, cols = 70, 512
    say(f"case subnormal/extreme {qtype}")
    rng = np.random.default_rng(2)
    f = _fields(qtype, rows * 2, rng)
    f["d"][:40] = torch.as_tensor(rng.integers(1, 0x400, 40))          # fp16 subnormal d
    f["d"][40:50] = 0x7BFF                                             # 65504
    if qtype != "q6k":
        f["dmin"][20:60] = torch.as_tensor(rng.integers(1, 0x400, 40))
        f["dmin"][60:70] = 0x7BFF
    x = synth.gen_x(1, cols, 4, "bf16")
    _run_fields(qtype, f, rows, cols, x, f"subnormal {qtype}")


@pytest.mark.parametrize("qtype", ["q4k", "q5k", "q6k"])
@pytest.mark.parametrize("batch,path", [(1, "dot2"), (4, "mfma"), (8, "mfma"), (8, "dot2")])
def test_negative_scales(qtype, batch, path, monkeypatch):
    """Negative fp16 d and dmin (the format's sign bit), normal and subnormal, beside positive ones: the
    dot2 path and the matrix-core path (whose mins' product carries dmin's sign in its power of two)."""
    monkeypatch.setenv("KQ_MATRIX_CORES_FROM", "2" if path == "mfma" else "9")
    rows, cols = 70, 512
    say(f"case negative scales {qtype} B={batch} {path}")
    rng = np.random.default_rng(5)
    f = _fields(qtype, rows * 2, rng)
    f["d"][:50] |= 0x8000                                               # negative d
    f["d"][50:60] = torch.as_tensor(rng.integers(1, 0x400, 10)) | 0x8000   # negative subnormal d
    if qtype != "q6k":
        f["dmin"][30:100] |= 0x8000                                     # negative dmin
        f["dmin"][100:110] = torch.as_tensor(rng.integers(1, 0x400, 10)) | 0x8000
        f["dmin"][110:115] = 0x8000                                     # -0
    x = synth.gen_x(5, cols, batch, "bf16")
    _run_fields(qtype, f, rows, cols, x, f"negative scales {qtype} B={batch} {path}")


@pytest.mark.parametrize("qtype", ["q4k", "q5k", "q6k"])
@pytest.mark.parametrize("xdtype", ["bf16", "f32"])
def test_one_hot_picks_columns_exactly(qtype, xdtype):
    """x = e_k gives y = W[:, k] bit-exactly: each weight is rounded once, like the dequantised value."""
    rows, cols = 200, 1024
    say(f"case one-hot {qtype} {xdtype}")
    g = synth.gen_weights(qtype, rows, cols, 9)
    ks = [0, 31, 32, 255, 256, 700, 1023, 513]
    x = torch.zeros(len(ks), cols, dtype=torch.float32)
    for b, k in enumerate(ks):
        x[b, k] = 1.0
    x = x.to(torch.bfloat16) if xdtype == "bf16" else x
    w = kq.repack(qtype, g.to(DEV), rows, cols)
    y = kq.gemv(qtype, w, rows, cols, x.to(DEV)).cpu().numpy()
    W = O.dequant_f32(qtype, rows, cols, g.numpy())
    for b, k in enumerate(ks):
        assert np.array_equal(y[b], W[:, k]), f"column {k}"


@pytest.mark.parametrize("qtype", ["q4k", "q6k"])
@pytest.mark.parametrize("xdtype", ["bf16", "f32"])
def test_dynamic_units_deterministic(qtype, xdtype):
    """Batch 1: the wavefronts of a workgroup take units in whatever order they get to them, yet y is
    bitwise the same on every call (a tile's unit sums are added in unit order) and within tolerance."""
    rows, cols = 40 * 64 + 7, 48 * 256
    say(f"case dynamic units {qtype} {xdtype}")
    g = synth.gen_weights(qtype, rows, cols, synth.seed_of("dyn", qtype))
    x = synth.gen_x(1, cols, synth.seed_of("dyn-x", qtype), xdtype)
    w = kq.repack(qtype, g.to(DEV), rows, cols)
    xd = x.to(DEV)
    ys = [kq.gemv(qtype, w, rows, cols, xd) for _ in range(4)]
    torch.cuda.synchronize()
    for y in ys[1:]:
        assert torch.equal(y, ys[0]), "batch-1 results differ between calls"
    yo, ao = O.gemv(qtype, rows, cols, g.numpy(), x_host(x))
    check_y(ys[0].cpu().numpy(), yo, ao, f"dynamic units {qtype} {xdtype}")


def test_zero_x_and_determinism():
    rows, cols = 500, 2048
    say("case zero-x / determinism")
    g = synth.gen_weights("q6k", rows, cols, 10).to(DEV)
    w = kq.repack("q6k", g, rows, cols)
    y0 = kq.gemv("q6k", w, rows, cols, torch.zeros(4, cols, dtype=torch.bfloat16, device=DEV))
    assert torch.all(y0 == 0)
    x = synth.gen_x(8, cols, 11).to(DEV)
    y1 = kq.gemv("q6k", w, rows, cols, x)
    y2 = kq.gemv("q6k", w, rows, cols, x)
    assert torch.equal(y1, y2)


def test_strided_x():
    rows, cols, batch = 128, 1024, 3
    say("case strided x")
    g = synth.gen_weights("q4k", rows, cols, 12)
    xfull = synth.gen_x(batch, cols + 64, 13)
    x = xfull[:, :cols]                       # row stride cols + 64 (128 B multiple)
    w = kq.repack("q4k", g.to(DEV), rows, cols)
    y = kq.gemv("q4k", w, rows, cols, xfull.to(DEV)[:, :cols])
    yo, ao = O.gemv("q4k", rows, cols, g.numpy(), x_host(x))
    check_y(y.cpu().numpy(), yo, ao, "strided x")


@pytest.mark.parametrize("qtype", ["q4k", "q5k", "q6k"])
@pytest.mark.parametrize("batch", [1, 2, 5, 6, 7])
@pytest.mark.parametrize("waves", ["4", "8"])
def test_workgroup_sizes(qtype, batch, waves, monkeypatch):
    """Both workgroup shapes (4 and 8 wavefronts, KQ_WG_WAVES): at batch 1 the fixed runs and the
    dynamic unit distribution, from batch 2 the matrix-core path, including batches that leave some of
    an instruction's four result registers unread (5, 6, 7)."""
    monkeypatch.setenv("KQ_WG_WAVES", waves)
    monkeypatch.setenv("KQ_MATRIX_CORES_FROM", "2")
    run_case(qtype, 5 * 64 + 9, 7 * 256, batch, "bf16", 400 + batch, check_w=False)


@pytest.mark.parametrize("qtype", ["q4k", "q6k"])
@pytest.mark.parametrize("batch", [1, 8])
@pytest.mark.parametrize("waves,per_cu", [("4", "2"), ("4", "4"), ("4", "6"), ("4", "12"), ("8", "8"), ("8", "16")])
@pytest.mark.parametrize("cols", [20 * 256, 122 * 256])
def test_launch_geometries(qtype, batch, waves, per_cu, cols, monkeypatch):
    """Launch geometries (KQ_WG_WAVES x KQ_WAVES_PER_CU): runs of other lengths, so tiles split at other
    points between wavefronts and workgroups, fewer workgroups than CUs, and grids larger than what is
    resident at once; 41 ragged tiles of 20 columns (gate+up's K) and 5 of 122 (down's K)."""
    monkeypatch.setenv("KQ_WG_WAVES", waves)
    monkeypatch.setenv("KQ_WAVES_PER_CU", per_cu)
    rows = (41 if cols == 20 * 256 else 5) * 64 - 23
    run_case(qtype, rows, cols, batch, "bf16", 700 + batch, check_w=False)


@pytest.mark.parametrize("qtype", ["q4k", "q5k", "q6k"])
@pytest.mark.parametrize("batch,xdtype,windows_from", [(4, "bf16", None), (8, "bf16", None), (2, "bf16", "2"),
                                                       (4, "f32", None), (1, "bf16", "1")])
def test_column_windows(qtype, batch, xdtype, windows_from, monkeypatch):
    """Rows longer than the staging budget: each workgroup takes whole tiles of one column window and
    the windows' pieces of a tile are added in window order (K = 31232, the down projection's)."""
    if windows_from:
        monkeypatch.setenv("KQ_WINDOWS_FROM", windows_from)
    run_case(qtype, 5 * 64 + 9, 122 * 256, batch, xdtype, 500 + batch, check_w=False)


@pytest.mark.parametrize("qtype", ["q4k", "q5k", "q6k"])
@pytest.mark.parametrize("batch", [2, 3, 4, 5, 8])
@pytest.mark.parametrize("cols", [7 * 256, 122 * 256])
def test_vector_path_bf16(qtype, batch, cols, monkeypatch):
    """bf16 activations at batch >= 2 on the dot2 VALU path (KQ_MATRIX_CORES_FROM=9) instead of the
    matrix cores, with even unit runs (7 columns) and with column windows (122 columns)."""
    monkeypatch.setenv("KQ_MATRIX_CORES_FROM", "9")
    run_case(qtype, 5 * 64 + 9, cols, batch, "bf16", 600 + batch, check_w=False)



@pytest.mark.parametrize("qtype", ["q4k", "q5k", "q6k"])
@pytest.mark.parametrize("batch", [9, 12, 13, 16])
@pytest.mark.parametrize("shape", [(3 * 64 + 17, 5 * 256), (5 * 64 + 9, 122 * 256)], ids=["ragged", "windows"])
def test_verify_block_batches(qtype, batch, shape):
    """A speculative-verify block of up to 16 rows (bf16 x, matrix cores with three or four operand
    sets): a ragged tile, and long rows split into column windows."""
    rows, cols = shape
    run_case(qtype, rows, cols, batch, "bf16", 800 + batch, check_w=False)


@pytest.mark.parametrize("batch", [1, 2, 4, 8])
@pytest.mark.parametrize("scale", [2.0 ** -100, 1.0, 2.0 ** 100])
def test_fp32_activation_range(batch, scale):
    """fp32 activations run as two bf16 rows (hi = bf16(x), lo = bf16(x - hi)): within the GEMV bound over the
    documented range of row scales, also when one row mixes magnitudes from 2^-20 to 2^20."""
    rows, cols = 192, 1536
    say(f"case fp32 range 2^{int(np.log2(scale))} B={batch}")
    g = synth.gen_weights("q4k", rows, cols, synth.seed_of("f32range"))
    w = kq.repack("q4k", g.to(DEV), rows, cols)
    gen = torch.Generator().manual_seed(batch)
    x = torch.randn(batch, cols, generator=gen) * scale
    x[0] *= torch.exp2(torch.randint(-20, 21, (cols,), generator=gen).float())
    y = kq.gemv("q4k", w, rows, cols, x.float().to(DEV))
    torch.cuda.synchronize()
    yo, ao = O.gemv("q4k", rows, cols, g.numpy(), x.float().numpy())
    check_y(y.cpu().numpy(), yo, ao, f"fp32 x at scale 2^{int(np.log2(scale))}")
