"""SwiGLU epilogue (kq_repack_swiglu + kq_gemv_swiglu) against the oracle.

The oracle gives the gate and up products g, u exactly (fp64) with a_g = sum |w_g x|, a_u = sum |w_u x|.
The GPU computes g and u within the GEMV tolerance (1e-4 * a) and then silu(g) * u in fp32.  Since
|silu'| <= 1.1, the output may be off by at most
    1.1e-4 a_g (|u| + 1e-4 a_u) + 1e-4 a_u |silu(g)| + 2^-20 (|silu(g)| + 1.1e-4 a_g)(|u| + 1e-4 a_u)
(the last term: exp, division and product rounding in fp32); with a_g = a_u = 0 it must be exactly 0.
"""
import numpy as np
import pytest
import torch

from oracle import oracle as O
from quant_weight_streaming_amd import kq, synth
from tests.gpu_cases import oracle_rows, sample_rows, say, x_host

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]
DEV = "cuda:0"


def check_swiglu(y, g, a_g, u, a_u, where):
    s = np.abs(O.silu(g))
    U = np.abs(u) + 1e-4 * a_u
    bound = 1.1e-4 * a_g * U + 1e-4 * a_u * s + 2.0 ** -20 * (s + 1.1e-4 * a_g) * U
    err = np.abs(y.astype(np.float64) - O.swiglu(g, u))
    bad = err > bound
    assert not bad.any(), f"{where}: {int(bad.sum())} outputs off, first {np.argwhere(bad)[0]}"


def pair(qtype, inter, cols, tag):
    gate = synth.gen_weights(qtype, inter, cols, synth.seed_of("swiglu", tag, "gate"))
    up = synth.gen_weights(qtype, inter, cols, synth.seed_of("swiglu", tag, "up"))
    w = kq.repack_swiglu(qtype, gate.to(DEV), up.to(DEV), inter, cols)
    return gate, up, w


@pytest.mark.parametrize("qtype", ["q4k", "q5k", "q6k"])
@pytest.mark.parametrize("batch,xdtype", [(1, "bf16"), (2, "bf16"), (3, "bf16"), (8, "bf16"), (1, "f32"), (5, "f32")])
def test_swiglu_small(qtype, batch, xdtype):
    inter, cols = 3 * 32 + 7, 1024                   # a ragged last tile (7 gate + 7 up rows)
    say(f"case swiglu {qtype} {inter}x{cols} B={batch} {xdtype}")
    gate, up, w = pair(qtype, inter, cols, qtype)
    x = synth.gen_x(batch, cols, synth.seed_of("swiglu-x", qtype, batch), xdtype)
    y = torch.full((batch, inter + 5), 7.0, device=DEV)
    kq.kq_gemv_swiglu(qtype, w, inter, cols, x.to(DEV), y)
    torch.cuda.synchronize()
    yh = y.cpu().numpy()
    assert (yh[:, inter:] == 7.0).all(), "wrote outside [0, inter)"
    g, a_g = O.gemv(qtype, inter, cols, gate.numpy(), x_host(x))
    u, a_u = O.gemv(qtype, inter, cols, up.numpy(), x_host(x))
    check_swiglu(yh[:, :inter], g, a_g, u, a_u, f"swiglu {qtype} B={batch} {xdtype}")


def test_swiglu_zero_and_deterministic():
    inter, cols = 64, 512
    say("case swiglu zero x / determinism")
    gate, up, w = pair("q4k", inter, cols, "det")
    z = kq.gemv_swiglu("q4k", w, inter, cols, torch.zeros(2, cols, dtype=torch.bfloat16, device=DEV))
    x = synth.gen_x(4, cols, 3).to(DEV)
    y1 = kq.gemv_swiglu("q4k", w, inter, cols, x)
    y2 = kq.gemv_swiglu("q4k", w, inter, cols, x)
    torch.cuda.synchronize()
    assert torch.all(z == 0)
    assert torch.equal(y1, y2)


@pytest.mark.parametrize("batch", [1, 8])
def test_swiglu_full_size(batch):
    """The 6656-hidden decoder's feed-forward (19968 x 6656 gate and up), sampled rows."""
    inter, cols = synth.INTER_P4, synth.HIDDEN_P4
    say(f"case swiglu full size B={batch}")
    gate = synth.gen_weights("q4k", inter, cols, synth.seed_of("swiglu-full", "gate"), device=DEV)
    up = synth.gen_weights("q4k", inter, cols, synth.seed_of("swiglu-full", "up"), device=DEV)
    w = kq.repack_swiglu("q4k", gate, up, inter, cols)
    x = synth.gen_x(batch, cols, synth.seed_of("swiglu-full-x", batch), device=DEV)
    y = kq.gemv_swiglu("q4k", w, inter, cols, x)
    torch.cuda.synchronize()
    idx = sample_rows(inter, 128, 77)
    _, g, a_g = oracle_rows("q4k", gate, idx, cols, x)
    _, u, a_u = oracle_rows("q4k", up, idx, cols, x)
    check_swiglu(y[:, torch.as_tensor(idx, device=DEV)].cpu().numpy(), g, a_g, u, a_u, f"swiglu full B={batch}")


def test_swiglu_in_a_chain():
    """gate+up with the SwiGLU epilogue feeding the down projection in one chain (fp32 activations): the
    down step reads the hidden activation only after the epilogue has written all of it."""
    inter, hidden, batch = 512, 768, 2
    say("case swiglu chain")
    gate, up, w = pair("q4k", inter, hidden, "chain")
    dn = synth.gen_weights("q6k", hidden, inter, synth.seed_of("swiglu", "chain", "down"))
    wd = kq.repack("q6k", dn.to(DEV), hidden, inter)
    x = synth.gen_x(batch, hidden, synth.seed_of("swiglu-chain-x"), "f32").to(DEV)
    h = torch.full((batch, inter), 1.0e30, device=DEV)
    y = torch.full((batch, hidden), 1.0e30, device=DEV)
    ch = kq.Chain([("q4k", [w], [inter], hidden, x, [h], kq.KQ_EPI_SWIGLU),
                   ("q6k", [wd], [hidden], inter, h, [y])], batch)
    ch.run()
    torch.cuda.synchronize()
    assert ch.status() == 0
    h1 = kq.gemv_swiglu("q4k", w, inter, hidden, x)
    y1 = kq.gemv("q6k", wd, hidden, inter, h1)
    torch.cuda.synchronize()
    assert torch.equal(h, h1) and torch.equal(y, y1), "the chain differs from the two launches"
    ch.close()
