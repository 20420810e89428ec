"""Sigmoid-gate and residual epilogues (kq_gemv_fused) against the oracle.

sigmoid: |sigmoid'| <= 1/4, so |dy| <= 0.25e-4 a + 2^-21 sigmoid(y) (the GEMV tolerance carried
through, plus the fp32 exp, add and divide).  residual: |dy| <= 1e-4 a + 2^-24 |r + y| (one fp32 add).
"""
import numpy as np
import pytest
import torch

from oracle import oracle as O
from quant_weight_streaming_amd import kq, synth
from tests.gpu_cases import check_y, say, x_host

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]
DEV = "cuda:0"


@pytest.mark.parametrize("qtype", ["q4k", "q6k"])
@pytest.mark.parametrize("batch", [1, 3, 8, 16])
def test_qkvg_with_sigmoid_gate_and_residual(qtype, batch):
    """A fused launch of four segments: plain, plain, residual-added, sigmoid-gated."""
    parts, cols = [128, 64, 70, 128], 768
    epis = [kq.KQ_EPI_NONE, kq.KQ_EPI_NONE, kq.KQ_EPI_RESIDUAL, kq.KQ_EPI_SIGMOID]
    say(f"case epilogues {qtype} B={batch}")
    gs = [synth.gen_weights(qtype, r, cols, synth.seed_of("epi", qtype, i)) for i, r in enumerate(parts)]
    ws = [kq.repack(qtype, g.to(DEV), r, cols) for g, r in zip(gs, parts)]
    x = synth.gen_x(batch, cols, synth.seed_of("epi-x", qtype, batch), "bf16")
    res = torch.randn(batch, parts[2], generator=torch.Generator().manual_seed(5)) * 10
    ys = [torch.full((batch, r + 2), 7.0, device=DEV) for r in parts]
    ys[2][:, :parts[2]] = res.to(DEV)
    kq.kq_gemv_fused(qtype, ws, parts, cols, x.to(DEV), ys, epis)
    torch.cuda.synchronize()
    for i, (g, r, y, e) in enumerate(zip(gs, parts, ys, epis)):
        yh = y.cpu().numpy()
        assert (yh[:, r:] == 7.0).all(), f"segment {i}: wrote outside [0, rows)"
        yo, ao = O.gemv(qtype, r, cols, g.numpy(), x_host(x))
        got = yh[:, :r].astype(np.float64)
        if e == kq.KQ_EPI_NONE:
            check_y(yh[:, :r], yo, ao, f"segment {i}")
        elif e == kq.KQ_EPI_SIGMOID:
            want = O.sigmoid(yo)
            assert (np.abs(got - want) <= 0.25e-4 * ao + 2.0 ** -21 * want).all(), f"segment {i}: sigmoid off"
        else:
            want = res.numpy().astype(np.float64) + yo
            assert (np.abs(got - want) <= 1e-4 * ao + 2.0 ** -24 * np.abs(want)).all(), f"segment {i}: residual off"


def test_residual_in_a_chain():
    """O projection with the residual epilogue in a chain: the step reads the residual that the previous
    step wrote into the same buffer (fp32), through the device coherence point."""
    hidden, batch = 512, 2
    say("case residual chain")
    g0 = synth.gen_weights("q4k", hidden, 256, synth.seed_of("epi-chain", 0))
    g1 = synth.gen_weights("q4k", hidden, hidden, synth.seed_of("epi-chain", 1))
    w0, w1 = kq.repack("q4k", g0.to(DEV), hidden, 256), kq.repack("q4k", g1.to(DEV), hidden, hidden)
    x0 = synth.gen_x(batch, 256, synth.seed_of("epi-chain-x"), "f32").to(DEV)
    h = torch.full((batch, hidden), 1e30, device=DEV)
    r = torch.full((batch, hidden), 1e30, device=DEV)
    # step 0: h = W0 x0; step 1: r = W0 x0 again (the residual); step 2: r += W1 h
    ch = kq.Chain([("q4k", [w0], [hidden], 256, x0, [h]), ("q4k", [w0], [hidden], 256, x0, [r]),
                   ("q4k", [w1], [hidden], hidden, h, [r], kq.KQ_EPI_RESIDUAL)], batch)
    ch.run()
    torch.cuda.synchronize()
    assert ch.status() == 0
    h1 = kq.gemv("q4k", w0, hidden, 256, x0)
    r1 = h1.clone()
    kq.kq_gemv_fused("q4k", [w1], [hidden], hidden, h1, [r1], [kq.KQ_EPI_RESIDUAL])
    torch.cuda.synchronize()
    assert torch.equal(h, h1) and torch.equal(r, r1), "the chain differs from the launches"
    ch.close()
