"""Per-head weight-less RMSNorm epilogue (KQ_EPI_HEADNORM, the Q/K norm) against the oracle.

Tolerance, derived.  The launch normalises its own v (each within e_i = 1e-4 a_i of the exact product) by
R = sqrt(S / 128 + eps), S = sum over the head of v^2.  |dS| <= sum (2 |v_i| e_i + e_i^2) + 2^-17 S (fp32 squares
added over two tiles by a butterfly), so dR / R <= dS / (2 (S + 128 eps)) + 2^-22, and
|dy_i| <= e_i / R + |y_i| (1.01 dR / R + 2^-20).
"""
import numpy as np
import pytest
import torch

from oracle import oracle as O
from quant_weight_streaming_amd import kq, synth
from tests.gpu_cases import check_y, sample_rows, say, x_host

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]
DEV = "cuda:0"
H = kq.KQ_HEAD_ROWS


def check_heads(got, v, a, eps, where):
    """got [B, rows] against the oracle's head norm of v (fp64 GEMV) with bound a (sum |w x|)."""
    b, r = v.shape
    vh, ah = v.reshape(b, r // H, H), a.reshape(b, r // H, H)
    e = 1e-4 * ah
    S = np.sum(vh * vh, axis=-1, keepdims=True)
    dS = np.sum(2 * np.abs(vh) * e + e * e, axis=-1, keepdims=True) + 2.0 ** -17 * S
    R = np.sqrt(S / H + eps)
    rel = dS / (2 * (S + H * eps)) + 2.0 ** -22
    want = vh / R
    bound = e / R + np.abs(want) * (1.01 * rel + 2.0 ** -20)
    err = np.abs(got.reshape(b, r // H, H).astype(np.float64) - want)
    bad = err > bound
    assert not bad.any(), (f"{where}: {int(bad.sum())} outputs over tolerance; worst ratio "
                           f"{float((err / bound).max()):.3g}")
    assert np.allclose(want.reshape(b, r), O.head_rmsnorm(v, eps), rtol=1e-12, atol=0)


@pytest.mark.parametrize("qtype", ["q4k", "q6k"])
@pytest.mark.parametrize("batch", [1, 3, 8, 16])
def test_qkvg_head_norm(qtype, batch):
    """q (4 heads) and k (2 heads) normalised per head, v plain, gate through the sigmoid, in one launch."""
    parts, cols, eps = [512, 256, 256, 512], 1536, 1e-6
    epis = [kq.KQ_EPI_HEADNORM, kq.KQ_EPI_HEADNORM, kq.KQ_EPI_NONE, kq.KQ_EPI_SIGMOID]
    say(f"case head norm {qtype} B={batch}")
    gs = [synth.gen_weights(qtype, r, cols, synth.seed_of("hn", qtype, i)) for i, r in enumerate(parts)]
    ws = [kq.repack(qtype, g.to(DEV), r, cols) for g, r in zip(gs, parts)]
    x = synth.gen_x(batch, cols, synth.seed_of("hn-x", qtype, batch), "bf16")
    ys = [torch.full((batch, r), 7.0, device=DEV) for r in parts]
    kq.kq_gemv_fused(qtype, ws, parts, cols, x.to(DEV), ys, epis, head_eps=eps)
    torch.cuda.synchronize()
    for i, (g, r, y, e) in enumerate(zip(gs, parts, ys, epis)):
        v, a = O.gemv(qtype, r, cols, g.numpy(), x_host(x))
        got = y.cpu().numpy()
        if e == kq.KQ_EPI_HEADNORM:
            check_heads(got, v, a, eps, f"segment {i}")
        elif e == kq.KQ_EPI_NONE:
            check_y(got, v, a, f"segment {i}")
        else:
            want = O.sigmoid(v)
            assert (np.abs(got - want) <= 0.25e-4 * a + 2.0 ** -21 * want).all()


@pytest.mark.parametrize("batch,xdt", [(1, "bf16"), (2, "f32"), (8, "bf16")])
def test_head_norm_long_rows(batch, xdt):
    """K = 8,192 columns: the heads' tiles are split over workgroups (hand-offs, and column windows from
    batch 4), so the two tiles of a head are finished by different workgroups in either order."""
    rows, cols, eps = 1024, 8192, 1e-5
    say(f"case head norm long B={batch} {xdt}")
    g = synth.gen_weights("q4k", rows, cols, synth.seed_of("hn-long"))
    w = kq.repack("q4k", g.to(DEV), rows, cols)
    x = synth.gen_x(batch, cols, synth.seed_of("hn-long-x", batch), xdt)
    y = torch.empty(batch, rows, device=DEV)
    for _ in range(2):   # the head counters are back at zero for the second call
        kq.kq_gemv_fused("q4k", [w], [rows], cols, x.to(DEV), [y], [kq.KQ_EPI_HEADNORM], head_eps=eps)
        torch.cuda.synchronize()
        v, a = O.gemv("q4k", rows, cols, g.numpy(), x_host(x))
        check_heads(y.cpu().numpy(), v, a, eps, "long rows")


def test_head_norm_with_input_norm():
    """The input RMSNorm and the head norm in the same launch: y = headnorm(W rmsnorm(x))."""
    rows, cols, batch = 256, 2048, 3
    say("case head norm + input norm")
    g = synth.gen_weights("q6k", rows, cols, synth.seed_of("hn-in"))
    w = kq.repack("q6k", g.to(DEV), rows, cols)
    x = synth.gen_x(batch, cols, synth.seed_of("hn-in-x"), "bf16") * 5
    y = torch.empty(batch, rows, device=DEV)
    kq.kq_gemv_fused("q6k", [w], [rows], cols, x.to(DEV), [y], [kq.KQ_EPI_HEADNORM], rms_eps=1e-5, head_eps=1e-6)
    torch.cuda.synchronize()
    v, a = O.gemv_rmsnorm("q6k", rows, cols, g.numpy(), x_host(x), 1e-5)
    # the input norm's own bound is 1e-4 a + 2^-17 |v|; fold it into e through a
    check_heads(y.cpu().numpy(), v, a + 2.0 ** -17 / 1e-4 * np.abs(v), 1e-6, "input and head norm")


@pytest.mark.parametrize("batch", [1, 8])
def test_head_norm_full_size_qkvg(batch):
    """The 6,656-hidden decoder's QKVG launch with q and k heads normalised (32 + 2 heads), sampled heads."""
    spec = synth.QKVG_P4
    parts, cols, eps = list(spec.parts), spec.cols, 1e-6
    say(f"case head norm full-size B={batch}")
    g = synth.gen_weights("q4k", spec.rows, cols, synth.seed_of("hn-full"), device=DEV)
    starts = np.cumsum([0] + parts)
    ws = [kq.repack("q4k", g[starts[i]:starts[i + 1]].contiguous(), r, cols) for i, r in enumerate(parts)]
    x = synth.gen_x(batch, cols, synth.seed_of("hn-full-x", batch), "bf16", device=DEV)
    ys = [torch.empty(batch, r, device=DEV) for r in parts]
    epis = [kq.KQ_EPI_HEADNORM, kq.KQ_EPI_HEADNORM, kq.KQ_EPI_NONE, kq.KQ_EPI_SIGMOID]
    kq.kq_gemv_fused("q4k", ws, parts, cols, x, ys, epis, head_eps=eps)
    torch.cuda.synchronize()
    for i in (0, 1):
        heads = sorted(set([0, parts[i] // H - 1] + list(np.random.default_rng(i).integers(0, parts[i] // H, 3))))
        for h in heads:
            r0 = int(starts[i] + h * H)
            v, a = O.gemv("q4k", H, cols, g[r0:r0 + H].cpu().numpy(), x_host(x))
            check_heads(ys[i].cpu().numpy()[:, h * H:(h + 1) * H], v, a, eps, f"segment {i} head {h}")


def test_head_norm_in_a_chain(monkeypatch):
    """A QKV step with the head norm inside a chain equals its single launch bitwise."""
    monkeypatch.setenv("KQ_WG_WAVES", "8")
    parts, cols, batch = [512, 256, 256], 1024, 2
    say("case head norm chain")
    gs = [synth.gen_weights("q4k", r, cols, synth.seed_of("hn-chain", i), device=DEV) for i, r in enumerate(parts)]
    ws = [kq.repack("q4k", g, r, cols) for g, r in zip(gs, parts)]
    x = synth.gen_x(batch, cols, synth.seed_of("hn-chain-x"), "f32", device=DEV)
    ys = [torch.full((batch, r), 1e30, device=DEV) for r in parts]
    packed = kq.KQ_EPI_HEADNORM | (kq.KQ_EPI_HEADNORM << 4)
    ch = kq.Chain([("q4k", ws, parts, cols, x, ys, packed, 0.0, 1e-6)], batch)
    ch.run()
    torch.cuda.synchronize()
    assert ch.status() == 0
    ch.close()
    ref = [torch.empty(batch, r, device=DEV) for r in parts]
    kq.kq_gemv_fused("q4k", ws, parts, cols, x, ref, [kq.KQ_EPI_HEADNORM, kq.KQ_EPI_HEADNORM, kq.KQ_EPI_NONE],
                     head_eps=1e-6)
    torch.cuda.synchronize()
    for a_, b_ in zip(ys, ref):
        assert torch.equal(a_, b_), "the chain differs from the launch"


@pytest.mark.parametrize("batch,xdt", [(1, "f32"), (4, "f32"), (8, "bf16")])
def test_head_norm_repeats_bitwise(batch, xdt):
    """The same launch gives the same bits every time, whichever tile of a head finishes second (the head's
    sum of squares is taken from one lane, so both halves add the same published values)."""
    parts, cols = [512, 256, 256], 1024
    say(f"case head norm repeats B={batch} {xdt}")
    gs = [synth.gen_weights("q4k", r, cols, synth.seed_of("hn-rep", i), device=DEV) for i, r in enumerate(parts)]
    ws = [kq.repack("q4k", g, r, cols) for g, r in zip(gs, parts)]
    x = synth.gen_x(batch, cols, synth.seed_of("hn-rep-x", batch), xdt, device=DEV)
    first = None
    for _ in range(8):
        ys = [torch.empty(batch, r, device=DEV) for r in parts]
        kq.kq_gemv_fused("q4k", ws, parts, cols, x, ys, [kq.KQ_EPI_HEADNORM, kq.KQ_EPI_HEADNORM, kq.KQ_EPI_NONE],
                         head_eps=1e-6)
        torch.cuda.synchronize()
        out = torch.cat(ys, 1)
        if first is None:
            first = out
        assert torch.equal(out, first), "a repeated launch gave different bits"
