"""bf16 copies of the outputs (kq_gemv_fused y16; chain steps' y16): each copy is the bf16 nearest (round to nearest
even) to the fp32 output written beside it, bit for bit, whatever the segment's epilogue; a chain whose steps read
those copies as their bf16 activations equals the same launches in order."""
import numpy as np
import pytest
import torch

from quant_weight_streaming_amd import kq, synth
from tests.gpu_cases import say

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]
DEV = "cuda:0"


def rne(y):
    """torch's fp32 -> bf16 conversion rounds to nearest even."""
    return y.to(torch.bfloat16)


@pytest.mark.parametrize("batch,xdt", [(1, "bf16"), (3, "bf16"), (8, "bf16"), (16, "bf16"), (2, "f32"), (8, "f32")])
def test_copies_equal_rounded_outputs(batch, xdt):
    parts, cols = [128, 64, 70, 256], 1536
    epis = [kq.KQ_EPI_NONE, kq.KQ_EPI_SIGMOID, kq.KQ_EPI_RESIDUAL, kq.KQ_EPI_HEADNORM]
    say(f"case bf16 copies B={batch} {xdt}")
    ws = [kq.repack("q4k", synth.gen_weights("q4k", r, cols, synth.seed_of("y16", i), device=DEV), r, cols)
          for i, r in enumerate(parts)]
    x = synth.gen_x(batch, cols, synth.seed_of("y16-x", batch), xdt, device=DEV)
    ys = [torch.randn(batch, r, device=DEV) for r in parts]
    y16 = [torch.zeros(batch, r + 5, dtype=torch.bfloat16, device=DEV) for r in parts]
    kq.kq_gemv_fused("q4k", ws, parts, cols, x, ys, epis, head_eps=1e-6, y16s=y16)
    torch.cuda.synchronize()
    for i, (y, c) in enumerate(zip(ys, y16)):
        assert torch.equal(c[:, :parts[i]].view(torch.int16), rne(y).view(torch.int16)), f"segment {i}"
        assert (c[:, parts[i]:] == 0).all(), f"segment {i}: wrote past its rows"


def test_swiglu_copy():
    inter, cols, batch = 96, 1024, 4
    say("case bf16 copy swiglu")
    g = synth.gen_weights("q4k", inter, cols, synth.seed_of("y16-sw", "g"), device=DEV)
    u = synth.gen_weights("q4k", inter, cols, synth.seed_of("y16-sw", "u"), device=DEV)
    w = kq.repack_swiglu("q4k", g, u, inter, cols)
    x = synth.gen_x(batch, cols, synth.seed_of("y16-sw-x"), "bf16", device=DEV)
    h = torch.empty(batch, inter, device=DEV)
    h16 = torch.empty(batch, inter, dtype=torch.bfloat16, device=DEV)
    kq.kq_gemv_fused("q4k", [w], [inter], cols, x, [h], [kq.KQ_EPI_SWIGLU], y16s=[h16])
    torch.cuda.synchronize()
    assert torch.equal(h16.view(torch.int16), rne(h).view(torch.int16))


@pytest.mark.parametrize("batch", [1, 4, 8, 16])
def test_bf16_activation_chain(batch, monkeypatch):
    """Three dependent steps whose activations are the previous step's bf16 copy; the chain equals the launches."""
    monkeypatch.setenv("KQ_WG_WAVES", "8")
    dims = [1024, 768, 512, 1280]
    say(f"case bf16 activation chain B={batch}")
    ws = [kq.repack("q4k", synth.gen_weights("q4k", dims[j + 1], dims[j], synth.seed_of("y16c", j), device=DEV),
                    dims[j + 1], dims[j]) for j in range(3)]
    x0 = synth.gen_x(batch, dims[0], synth.seed_of("y16c-x", batch), "bf16", device=DEV)

    def bufs():
        return ([torch.zeros(batch, d, device=DEV) for d in dims[1:]],
                [torch.zeros(batch, d, dtype=torch.bfloat16, device=DEV) for d in dims[1:]])
    ys, cs = bufs()
    xs = [x0] + cs[:2]
    ch = kq.Chain([("q4k", [ws[j]], [dims[j + 1]], dims[j], xs[j], [ys[j]], kq.KQ_EPI_NONE, 0.0, 0.0, [cs[j]])
                   for j in range(3)], batch)
    ch.run()
    torch.cuda.synchronize()
    assert ch.status() == 0
    ch.close()
    ys2, cs2 = bufs()
    xs2 = [x0] + cs2[:2]
    for j in range(3):
        kq.kq_gemv_fused("q4k", [ws[j]], [dims[j + 1]], dims[j], xs2[j], [ys2[j]], y16s=[cs2[j]])
    torch.cuda.synchronize()
    for j in range(3):
        assert torch.equal(ys[j], ys2[j]) and torch.equal(cs[j].view(torch.int16), cs2[j].view(torch.int16)), j
        assert torch.equal(cs[j].view(torch.int16), rne(ys[j]).view(torch.int16)), j


@pytest.mark.parametrize("batch", [1, 2, 3, 8])
def test_chain_rereads_a_rewritten_activation(batch, monkeypatch):
    """Step 0 reads A, step 1 overwrites A with the bf16 copy of its output, step 2 reads A again and must see the
    new values, not lines that step 0's reads left in a cache.  A second run's step 0 reads what the first run's
    step 1 wrote.  Every run equals the launches in order."""
    monkeypatch.setenv("KQ_WG_WAVES", "8")
    K = 1536
    say(f"case chain re-reads a rewritten activation B={batch}")
    ws = [kq.repack("q4k", synth.gen_weights("q4k", K, K, synth.seed_of("reread", j), device=DEV), K, K)
          for j in range(3)]
    a0 = synth.gen_x(batch, K, synth.seed_of("reread-a", batch), "bf16", device=DEV)
    c = synth.gen_x(batch, K, synth.seed_of("reread-c", batch), "bf16", device=DEV)

    def launches(a, n_runs):
        a = a.clone()
        ys = [torch.zeros(batch, K, device=DEV) for _ in range(3)]
        out = []
        for _ in range(n_runs):
            kq.kq_gemv_fused("q4k", [ws[0]], [K], K, a, [ys[0]])
            kq.kq_gemv_fused("q4k", [ws[1]], [K], K, c, [ys[1]], y16s=[a])
            kq.kq_gemv_fused("q4k", [ws[2]], [K], K, a, [ys[2]])
            torch.cuda.synchronize()
            out.append([y.clone() for y in ys] + [a.clone()])
        return out

    ref = launches(a0, 2)
    a = a0.clone()
    ys = [torch.zeros(batch, K, device=DEV) for _ in range(3)]
    ch = kq.Chain([("q4k", [ws[0]], [K], K, a, [ys[0]]),
                   ("q4k", [ws[1]], [K], K, c, [ys[1]], kq.KQ_EPI_NONE, 0.0, 0.0, [a]),
                   ("q4k", [ws[2]], [K], K, a, [ys[2]])], batch)
    for run in range(2):
        ch.run()
        torch.cuda.synchronize()
        assert ch.status() == 0
        got = [y.clone() for y in ys] + [a.clone()]
        for j, (g, r) in enumerate(zip(got, ref[run])):
            assert torch.equal(g.view(torch.int32) if g.dtype == torch.float32 else g.view(torch.int16),
                               r.view(torch.int32) if r.dtype == torch.float32 else r.view(torch.int16)), \
                f"run {run} output {j}"
    ch.close()
    assert not torch.equal(ref[0][0], ref[1][0]), "the second run's first step must read a different A"
