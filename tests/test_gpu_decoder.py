"""Decoder layers as one chain, with the operations either side of each product fused into it: the QKV step
reads the residual stream through the weight-less input RMSNorm and normalises the Q and K heads; the O step reads
q (a stand-in for the attention output) and adds into the residual stream; gate+up reads the residual stream
through the input norm and writes silu(gate) * up; down adds into the residual stream.  Every activation is the
fp32 output of an earlier step.  The chain equals the same single launches in order bitwise, and every launch is
checked against the oracle on the inputs it actually read (each step's tolerance is derived in the test of that
operation: tests/test_gpu_norm.py, test_gpu_headnorm.py, test_gpu_epilogues.py, test_gpu_swiglu.py)."""
import numpy as np
import pytest
import torch

from oracle import oracle as O
from quant_weight_streaming_amd import kq, synth
from tests.gpu_cases import say
from tests.test_gpu_headnorm import check_heads

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]
DEV = "cuda:0"
HIDDEN, QROWS, KVROWS, INTER = 512, 512, 128, 1024
RMS_EPS, HEAD_EPS = 1e-5, 1e-6
HN = kq.KQ_EPI_HEADNORM


def _layer(tag):
    g = {}
    g["qkv"] = synth.gen_weights("q4k", QROWS + 2 * KVROWS, HIDDEN, synth.seed_of("dec", tag, "qkv"))
    g["o"] = synth.gen_weights("q4k", HIDDEN, QROWS, synth.seed_of("dec", tag, "o"))
    g["gate"] = synth.gen_weights("q4k", INTER, HIDDEN, synth.seed_of("dec", tag, "gate"))
    g["up"] = synth.gen_weights("q4k", INTER, HIDDEN, synth.seed_of("dec", tag, "up"))
    g["down"] = synth.gen_weights("q6k", HIDDEN, INTER, synth.seed_of("dec", tag, "down"))
    parts = [QROWS, KVROWS, KVROWS]
    starts = np.cumsum([0] + parts)
    w = {"qkv": [kq.repack("q4k", g["qkv"][starts[i]:starts[i + 1]].contiguous().to(DEV), r, HIDDEN)
                 for i, r in enumerate(parts)],
         "o": kq.repack("q4k", g["o"].to(DEV), HIDDEN, QROWS),
         "gu": kq.repack_swiglu("q4k", g["gate"].to(DEV), g["up"].to(DEV), INTER, HIDDEN),
         "down": kq.repack("q6k", g["down"].to(DEV), HIDDEN, INTER)}
    return g, w


def _steps(w, r, q, k, v, h):
    return [("q4k", w["qkv"], [QROWS, KVROWS, KVROWS], HIDDEN, r, [q, k, v], HN | (HN << 4), RMS_EPS, HEAD_EPS),
            ("q4k", [w["o"]], [HIDDEN], QROWS, q, [r], kq.KQ_EPI_RESIDUAL),
            ("q4k", [w["gu"]], [INTER], HIDDEN, r, [h], kq.KQ_EPI_SWIGLU, RMS_EPS),
            ("q6k", [w["down"]], [HIDDEN], INTER, h, [r], kq.KQ_EPI_RESIDUAL)]


def _steps16(w, r, q, k, v, h, r16, q16, h16):
    """The same layer with bf16 activations: every step also writes the bf16 copy the next product reads (the
    residual stream itself stays fp32)."""
    return [("q4k", w["qkv"], [QROWS, KVROWS, KVROWS], HIDDEN, r16, [q, k, v], HN | (HN << 4), RMS_EPS, HEAD_EPS,
             [q16, None, None]),
            ("q4k", [w["o"]], [HIDDEN], QROWS, q16, [r], kq.KQ_EPI_RESIDUAL, 0.0, 0.0, [r16]),
            ("q4k", [w["gu"]], [INTER], HIDDEN, r16, [h], kq.KQ_EPI_SWIGLU, RMS_EPS, 0.0, [h16]),
            ("q6k", [w["down"]], [HIDDEN], INTER, h16, [r], kq.KQ_EPI_RESIDUAL, 0.0, 0.0, [r16])]


@pytest.mark.parametrize("batch", [1, 8, 16])
def test_decoder_layers_chain_bf16(batch, monkeypatch):
    """bf16 activations (the bf16 copies of the fp32 outputs): the chain equals the launches bitwise, and the copies
    are the rounded fp32 outputs."""
    monkeypatch.setenv("KQ_WG_WAVES", "8")
    say(f"case decoder chain bf16 B={batch}")
    layers = [_layer(i) for i in range(2)]
    r0 = torch.randn(batch, HIDDEN, generator=torch.Generator().manual_seed(batch)) * 2

    def bufs():
        r = r0.clone().to(DEV)
        return (r, torch.zeros(batch, QROWS, device=DEV), torch.zeros(batch, KVROWS, device=DEV),
                torch.zeros(batch, KVROWS, device=DEV), torch.zeros(batch, INTER, device=DEV),
                r.to(torch.bfloat16), torch.zeros(batch, QROWS, dtype=torch.bfloat16, device=DEV),
                torch.zeros(batch, INTER, dtype=torch.bfloat16, device=DEV))
    b1 = bufs()
    ch = kq.Chain([s for _, w in layers for s in _steps16(w, *b1)], batch)
    ch.run()
    torch.cuda.synchronize()
    assert ch.status() == 0
    ch.close()
    b2 = bufs()
    for _, w in layers:
        for st in _steps16(w, *b2):
            qt, ws, rows, cols, x, ys, epi, reps, heps, y16 = st
            codes = [(epi >> (4 * i)) & 15 for i in range(len(ws))]
            kq.kq_gemv_fused(qt, ws, rows, cols, x, ys, codes, rms_eps=reps, head_eps=heps, y16s=y16)
    torch.cuda.synchronize()
    for i, (a_, b_) in enumerate(zip(b1, b2)):
        assert torch.equal(a_.view(torch.int16) if a_.dtype == torch.bfloat16 else a_,
                           b_.view(torch.int16) if b_.dtype == torch.bfloat16 else b_), f"buffer {i}"
    r, q, k, v, h, r16, q16, h16 = b1
    assert torch.equal(r16.view(torch.int16), r.to(torch.bfloat16).view(torch.int16))
    assert torch.equal(q16.view(torch.int16), q.to(torch.bfloat16).view(torch.int16))
    assert torch.equal(h16.view(torch.int16), h.to(torch.bfloat16).view(torch.int16))


@pytest.mark.parametrize("batch", [1, 3, 8])
def test_decoder_layers_chain(batch, monkeypatch):
    monkeypatch.setenv("KQ_WG_WAVES", "8")      # single launches with the chain's workgroup shape
    say(f"case decoder chain B={batch}")
    layers = [_layer(i) for i in range(2)]
    r0 = torch.randn(batch, HIDDEN, generator=torch.Generator().manual_seed(batch)) * 2
    bufs = lambda: (r0.clone().to(DEV), torch.zeros(batch, QROWS, device=DEV), torch.zeros(batch, KVROWS, device=DEV),
                    torch.zeros(batch, KVROWS, device=DEV), torch.zeros(batch, INTER, device=DEV))
    # the chain
    r, q, k, v, h = bufs()
    ch = kq.Chain([s for _, w in layers for s in _steps(w, r, q, k, v, h)], batch)
    ch.run()
    torch.cuda.synchronize()
    assert ch.status() == 0
    ch.close()
    # the same launches one by one, each checked against the oracle on its own inputs
    r2, q2, k2, v2, h2 = bufs()
    for li, (g, w) in enumerate(layers):
        where = f"layer {li}"
        rin = r2.cpu().numpy().copy()
        kq.kq_gemv_fused("q4k", w["qkv"], [QROWS, KVROWS, KVROWS], HIDDEN, r2, [q2, k2, v2], [HN, HN, 0],
                         rms_eps=RMS_EPS, head_eps=HEAD_EPS)
        torch.cuda.synchronize()
        yq, aq = O.gemv_rmsnorm("q4k", QROWS + 2 * KVROWS, HIDDEN, g["qkv"].numpy(), rin, RMS_EPS)
        loose = aq + 2.0 ** -17 / 1e-4 * np.abs(yq)        # the input norm's own bound, folded into a
        check_heads(q2.cpu().numpy(), yq[:, :QROWS], loose[:, :QROWS], HEAD_EPS, where + " q")
        check_heads(k2.cpu().numpy(), yq[:, QROWS:QROWS + KVROWS], loose[:, QROWS:QROWS + KVROWS], HEAD_EPS,
                    where + " k")
        vv = v2.cpu().numpy().astype(np.float64)
        assert (np.abs(vv - yq[:, QROWS + KVROWS:]) <= loose[:, QROWS + KVROWS:] * 1e-4).all(), where + " v"

        rin, qin = r2.cpu().numpy().astype(np.float64), q2.cpu().numpy()
        kq.kq_gemv_fused("q4k", [w["o"]], [HIDDEN], QROWS, q2, [r2], [kq.KQ_EPI_RESIDUAL])
        torch.cuda.synchronize()
        yo, ao = O.gemv("q4k", HIDDEN, QROWS, g["o"].numpy(), qin)
        want = rin + yo
        assert (np.abs(r2.cpu().numpy() - want) <= 1e-4 * ao + 2.0 ** -24 * np.abs(want)).all(), where + " o"

        rin = r2.cpu().numpy().copy()
        kq.kq_gemv_fused("q4k", [w["gu"]], [INTER], HIDDEN, r2, [h2], [kq.KQ_EPI_SWIGLU], rms_eps=RMS_EPS)
        torch.cuda.synchronize()
        go, ag = O.gemv_rmsnorm("q4k", INTER, HIDDEN, g["gate"].numpy(), rin, RMS_EPS)
        uo, au = O.gemv_rmsnorm("q4k", INTER, HIDDEN, g["up"].numpy(), rin, RMS_EPS)
        eg, eu = 1e-4 * ag + 2.0 ** -17 * np.abs(go), 1e-4 * au + 2.0 ** -17 * np.abs(uo)
        s = np.abs(O.silu(go))
        bound = 1.1 * eg * (np.abs(uo) + eu) + eu * s + 2.0 ** -20 * (s + 1.1 * eg) * (np.abs(uo) + eu)
        assert (np.abs(h2.cpu().numpy().astype(np.float64) - O.swiglu(go, uo)) <= bound).all(), where + " gate+up"

        rin, hin = r2.cpu().numpy().astype(np.float64), h2.cpu().numpy()
        kq.kq_gemv_fused("q6k", [w["down"]], [HIDDEN], INTER, h2, [r2], [kq.KQ_EPI_RESIDUAL])
        torch.cuda.synchronize()
        yd, ad = O.gemv("q6k", HIDDEN, INTER, g["down"].numpy(), hin)
        want = rin + yd
        assert (np.abs(r2.cpu().numpy() - want) <= 1e-4 * ad + 2.0 ** -24 * np.abs(want)).all(), where + " down"
    for name, a_, b_ in (("r", r, r2), ("q", q, q2), ("k", k, k2), ("v", v, v2), ("h", h, h2)):
        assert torch.equal(a_, b_), f"the chain's {name} differs from the launches"
