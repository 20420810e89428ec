"""Weight-less RMSNorm folded into the GEMV (kq_gemv_fused with rms_eps > 0) against the oracle's
W rmsnorm(x) in fp64.

Tolerance, derived: the launch computes (W x) / rms(x).  W x is within 1e-4 sum|w x| of its exact value, which
scaled by 1/rms is 1e-4 a with a = sum|w xn| the oracle's bound for the normalised row.  sum x^2 is added in
fp32 with every term positive over at most ~80 rounding steps (16 in a sub-block, 4 across the sub-block
lanes, one per column of a piece, one per piece), so it is within 80 * 2^-24 relative; the mean, the
square root, the divide and the final product add a few more ulps.  Hence |dy| <= 1e-4 a + 2^-17 |y|.
"""
import numpy as np
import pytest
import torch

from oracle import oracle as O
from quant_weight_streaming_amd import kq, synth
from tests.gpu_cases import sample_rows, say, x_host

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]
DEV = "cuda:0"


def check_norm(yg, yo, ao, where):
    err = np.abs(yg.astype(np.float64) - yo)
    bound = 1e-4 * ao + 2.0 ** -17 * np.abs(yo)
    bad = err > bound
    if bad.any():
        i = tuple(np.argwhere(bad)[0])
        raise AssertionError(f"{where}: {int(bad.sum())} outputs over tolerance; first {i}: gpu {yg[i]!r} "
                             f"oracle {yo[i]!r} bound {bound[i]!r}")


CASES = [  # (qtype, rows, cols, batch, xdtype): hand-offs across tiles, column windows, ragged tiles
    ("q4k", 200, 1024, 1, "bf16"), ("q5k", 130, 2048, 2, "bf16"), ("q6k", 70, 768, 3, "bf16"),
    ("q4k", 300, 8192, 4, "bf16"), ("q6k", 190, 8192, 8, "bf16"), ("q4k", 129, 8192, 12, "bf16"),
    ("q5k", 64, 4096, 16, "bf16"), ("q4k", 250, 1536, 1, "f32"), ("q6k", 100, 8192, 5, "f32"),
    ("q5k", 77, 2560, 8, "f32"),
]


@pytest.mark.parametrize("qtype,rows,cols,batch,xdt", CASES)
def test_norm_against_oracle(qtype, rows, cols, batch, xdt):
    say(f"case norm {qtype} {rows}x{cols} B={batch} {xdt}")
    g = synth.gen_weights(qtype, rows, cols, synth.seed_of("norm", qtype, rows, cols))
    w = kq.repack(qtype, g.to(DEV), rows, cols)
    x = synth.gen_x(batch, cols, synth.seed_of("norm-x", batch, cols), xdt) * 3
    if batch > 1:
        x[1] = 0      # a zero row: y = 0 exactly
    y = torch.full((batch, rows + 3), 9.0, device=DEV)
    kq.kq_gemv_fused(qtype, [w], [rows], cols, x.to(DEV), [y], rms_eps=1e-5)
    torch.cuda.synchronize()
    yh = y.cpu().numpy()
    assert (yh[:, rows:] == 9.0).all()
    yo, ao = O.gemv_rmsnorm(qtype, rows, cols, g.numpy(), x_host(x), 1e-5)
    check_norm(yh[:, :rows], yo, ao, f"norm {qtype} B={batch}")
    if batch > 1:
        assert (yh[1, :rows] == 0).all(), "a zero activation row must give exactly 0"


def test_norm_multi_segments_and_epilogues():
    """Four QKVG-like segments with sigmoid and residual epilogues, eps 1e-8, batch 3."""
    parts, cols, batch = [128, 64, 70, 128], 1280, 3
    epis = [kq.KQ_EPI_NONE, kq.KQ_EPI_NONE, kq.KQ_EPI_RESIDUAL, kq.KQ_EPI_SIGMOID]
    say("case norm multi")
    gs = [synth.gen_weights("q4k", r, cols, synth.seed_of("norm-multi", i)) for i, r in enumerate(parts)]
    ws = [kq.repack("q4k", g.to(DEV), r, cols) for g, r in zip(gs, parts)]
    x = synth.gen_x(batch, cols, synth.seed_of("norm-multi-x"), "bf16")
    res = torch.randn(batch, parts[2], generator=torch.Generator().manual_seed(3))
    ys = [torch.empty(batch, r, device=DEV) for r in parts]
    ys[2].copy_(res)
    kq.kq_gemv_fused("q4k", ws, parts, cols, x.to(DEV), ys, epis, rms_eps=1e-8)
    torch.cuda.synchronize()
    for i, (g, r, y, e) in enumerate(zip(gs, parts, ys, epis)):
        yo, ao = O.gemv_rmsnorm("q4k", r, cols, g.numpy(), x_host(x), 1e-8)
        got = y.cpu().numpy().astype(np.float64)
        if e == kq.KQ_EPI_NONE:
            check_norm(got, yo, ao, f"segment {i}")
        elif e == kq.KQ_EPI_SIGMOID:
            want = O.sigmoid(yo)
            assert (np.abs(got - want) <= 0.25 * (1e-4 * ao + 2.0 ** -17 * np.abs(yo)) + 2.0 ** -21 * want).all()
        else:
            want = res.numpy().astype(np.float64) + yo
            assert (np.abs(got - want) <= 1e-4 * ao + 2.0 ** -17 * np.abs(yo) + 2.0 ** -24 * np.abs(want)).all()


def test_norm_swiglu():
    """The normalised x feeding the fused gate+up pair: silu(g) u with g, u from W rmsnorm(x)."""
    inter, cols, batch = 160, 2048, 2
    say("case norm swiglu")
    gg = synth.gen_weights("q4k", inter, cols, synth.seed_of("norm-sw", "g"))
    gu = synth.gen_weights("q4k", inter, cols, synth.seed_of("norm-sw", "u"))
    ws = kq.repack_swiglu("q4k", gg.to(DEV), gu.to(DEV), inter, cols)
    x = synth.gen_x(batch, cols, synth.seed_of("norm-sw-x"), "bf16")
    h = torch.empty(batch, inter, device=DEV)
    kq.kq_gemv_fused("q4k", [ws], [inter], cols, x.to(DEV), [h], [kq.KQ_EPI_SWIGLU], rms_eps=1e-5)
    torch.cuda.synchronize()
    go, ag = O.gemv_rmsnorm("q4k", inter, cols, gg.numpy(), x_host(x), 1e-5)
    uo, au = O.gemv_rmsnorm("q4k", inter, cols, gu.numpy(), x_host(x), 1e-5)
    eg = 1e-4 * ag + 2.0 ** -17 * np.abs(go)
    eu = 1e-4 * au + 2.0 ** -17 * np.abs(uo)
    s = np.abs(O.silu(go))
    bound = 1.1 * eg * (np.abs(uo) + eu) + eu * s + 2.0 ** -20 * (s + 1.1 * eg) * (np.abs(uo) + eu)
    assert (np.abs(h.cpu().numpy().astype(np.float64) - O.swiglu(go, uo)) <= bound).all()


@pytest.mark.parametrize("waves", ["4", "8"])
def test_norm_batch1_workgroup_shapes(monkeypatch, waves):
    """Batch 1 with fixed runs (4 wavefronts) and per-unit slots (8 wavefronts) agree with the oracle."""
    monkeypatch.setenv("KQ_WG_WAVES", waves)
    rows, cols = 4608, 5120
    say(f"case norm B=1 waves={waves}")
    g = synth.gen_weights("q4k", rows, cols, synth.seed_of("norm-b1"), device=DEV)
    w = kq.repack("q4k", g, rows, cols)
    x = synth.gen_x(1, cols, synth.seed_of("norm-b1-x"), "bf16", device=DEV)
    y = torch.empty(1, rows, device=DEV)
    kq.kq_gemv_fused("q4k", [w], [rows], cols, x, [y], rms_eps=1e-5)
    torch.cuda.synchronize()
    idx = sample_rows(rows, 200, 4)
    yo, ao = O.gemv_rmsnorm("q4k", len(idx), cols, g[torch.as_tensor(idx, device=DEV)].cpu().numpy(),
                            x_host(x), 1e-5)
    check_norm(y.cpu().numpy()[:, idx], yo, ao, f"B=1 waves={waves}")


@pytest.mark.parametrize("batch", [1, 8, 16])
def test_norm_full_size_qkvg(batch):
    """The 6,656-hidden decoder's fused QKVG projection (8,704 x 6,656) on the normalised x, sampled rows."""
    rows, cols = synth.QKVG_P4.rows, synth.QKVG_P4.cols
    say(f"case norm full-size qkvg B={batch}")
    g = synth.gen_weights("q4k", rows, cols, synth.seed_of("norm-full"), device=DEV)
    w = kq.repack("q4k", g, rows, cols)
    x = synth.gen_x(batch, cols, synth.seed_of("norm-full-x", batch), "bf16", device=DEV)
    y = torch.empty(batch, rows, device=DEV)
    kq.kq_gemv_fused("q4k", [w], [rows], cols, x, [y], rms_eps=1e-5)
    torch.cuda.synchronize()
    idx = sample_rows(rows, 150, batch)
    yo, ao = O.gemv_rmsnorm("q4k", len(idx), cols, g[torch.as_tensor(idx, device=DEV)].cpu().numpy(),
                            x_host(x), 1e-5)
    check_norm(y.cpu().numpy()[:, idx], yo, ao, f"full-size B={batch}")


def test_norm_chain_step_matches_launch():
    """A chain whose second step normalises the first step's output equals the two single launches bitwise."""
    hidden, batch = 1024, 4
    say("case norm chain")
    g0 = synth.gen_weights("q4k", hidden, 512, synth.seed_of("norm-chain", 0), device=DEV)
    g1 = synth.gen_weights("q6k", 384, hidden, synth.seed_of("norm-chain", 1), device=DEV)
    w0, w1 = kq.repack("q4k", g0, hidden, 512), kq.repack("q6k", g1, 384, hidden)
    x0 = synth.gen_x(batch, 512, synth.seed_of("norm-chain-x"), "f32", device=DEV)
    h = torch.full((batch, hidden), 1e30, device=DEV)
    y = torch.full((batch, 384), 1e30, device=DEV)
    ch = kq.Chain([("q4k", [w0], [hidden], 512, x0, [h]),
                   ("q6k", [w1], [384], hidden, h, [y], kq.KQ_EPI_NONE, 1e-8)], batch)
    ch.run()
    torch.cuda.synchronize()
    assert ch.status() == 0
    ch.close()
    h1 = kq.gemv("q4k", w0, hidden, 512, x0)
    y1 = torch.empty(batch, 384, device=DEV)
    kq.kq_gemv_fused("q6k", [w1], [384], hidden, h1, [y1], rms_eps=1e-8)
    torch.cuda.synchronize()
    assert torch.equal(h, h1) and torch.equal(y, y1), "the chain differs from the launches"
    yo, ao = O.gemv_rmsnorm("q6k", 384, hidden, g1.cpu().numpy(), h1.cpu().numpy(), 1e-8)
    check_norm(y.cpu().numpy(), yo, ao, "chain step")
