"""Near-empty rows: every quant at the type's zero (Q4_K/Q5_K: q = 0 with zero mins; Q6_K: q = 32)
except one or two, so sum |w x| comes from one or two terms.  The bound 1e-4 * sum |w x| is per
output, so these rows check that the kernel's dot products carry no error proportional to the
other activations of the sub-block (an offset added to every quant and removed afterwards would).
Covered on the dot2 path (batch 1, 2), the matrix-core path (batch 3, 8, 16), and fp32 activations.
"""
import numpy as np
import pytest
import torch

from oracle import oracle as O
from quant_weight_streaming_amd import kq, synth
from tests.gpu_cases import check_dequant, check_y, say, x_host

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]
DEV = "cuda:0"
ROWS, COLS = 3 * 64 + 5, 4 * 256


def _near_empty_fields(qtype, rng):
    """Fields for ROWS x COLS: row r has nonzero weights only at positions picked below."""
    n = ROWS * (COLS // 256)
    d = torch.as_tensor(rng.integers(0x1000, 0x2C00, n))
    zero_q = 32 if qtype == "q6k" else 0
    q = torch.full((n, 256), zero_q, dtype=torch.int64)
    qmax = {"q4k": 16, "q5k": 32, "q6k": 64}[qtype]
    qv = q.view(ROWS, COLS)
    # rows cycle through: one nonzero quant, two in one sub-block, two in different super-blocks,
    # one nonzero quant at a column whose activations are tiny, and a fully random row
    for r in range(ROWS):
        kind = r % 5
        if kind == 4:
            qv[r] = torch.as_tensor(rng.integers(0, qmax, COLS))
            continue
        if kind == 0:
            cols = [int(rng.integers(0, COLS))]
        elif kind == 1:
            c0 = int(rng.integers(0, COLS - 16))
            cols = [c0, c0 + 1 + int(rng.integers(0, 15))]
        elif kind == 2:
            cols = [int(rng.integers(0, 256)), 512 + int(rng.integers(0, 512))]
        else:
            cols = [TINY_COLS[r % len(TINY_COLS)]]
        for c in cols:
            v = zero_q
            while v == zero_q:
                v = int(rng.integers(0, qmax))
            qv[r, c] = v
    if qtype == "q6k":
        return dict(d=d, sc=torch.as_tensor(rng.integers(-64, 64, (n, 16))), q=q)
    sc = torch.as_tensor(rng.integers(1, 64, (n, 8)))
    m = torch.as_tensor(rng.integers(0, 64, (n, 8)))
    dmin = torch.as_tensor(rng.integers(0x1000, 0x2C00, n))
    sbr = COLS // 256
    for r in range(ROWS):
        if r % 5 == 4:
            continue
        if r % 2 == 0:
            m[r * sbr:(r + 1) * sbr] = 0          # zero mins
        else:
            dmin[r * sbr:(r + 1) * sbr] = 0       # zero dmin
    return dict(d=d, dmin=dmin, sc=sc, m=m, q=q)


TINY_COLS = [3, 77, 300, 513, 1000]


def _x(batch, xdtype, seed):
    """N(0,1) activations, except columns TINY_COLS scaled by 2^-12 (the surviving term is then small
    next to the sub-block's other activations)."""
    x = synth.gen_x(batch, COLS, seed, "f32")
    x[:, TINY_COLS] *= 2.0 ** -12
    return x.to(torch.bfloat16) if xdtype == "bf16" else x


def _pack(qtype, f):
    if qtype == "q6k":
        return synth.pack_q6k(f["d"], f["sc"], f["q"])
    p = synth.pack_q4k if qtype == "q4k" else synth.pack_q5k
    return p(f["d"], f["dmin"], f["sc"], f["m"], f["q"])


@pytest.mark.parametrize("qtype", ["q4k", "q5k", "q6k"])
@pytest.mark.parametrize("xdtype,batch", [("bf16", 1), ("bf16", 2), ("bf16", 3), ("bf16", 8), ("bf16", 16),
                                          ("f32", 1), ("f32", 4)])
def test_near_empty_rows(qtype, xdtype, batch):
    say(f"case near-empty rows {qtype} {xdtype} B={batch}")
    rng = np.random.default_rng(1000 + batch)
    f = _near_empty_fields(qtype, rng)
    g = _pack(qtype, f).reshape(ROWS, -1)
    x = _x(batch, xdtype, synth.seed_of("near-empty", qtype, batch))
    w = kq.repack(qtype, g.to(DEV), ROWS, COLS)
    y = kq.gemv(qtype, w, ROWS, COLS, x.to(DEV))
    torch.cuda.synchronize()
    yo, ao = O.gemv(qtype, ROWS, COLS, g.numpy(), x_host(x))
    worst = check_y(y.cpu().numpy(), yo, ao, f"near-empty {qtype} {xdtype} B={batch}")
    say(f"  worst |err| / sum|wx| = {worst:.3g}")
    if batch == 1:
        check_dequant(qtype, w, ROWS, COLS, g.numpy(), np.arange(ROWS), f"near-empty {qtype}")


@pytest.mark.parametrize("qtype", ["q4k", "q6k"])
@pytest.mark.parametrize("batch", [1, 8])
def test_near_empty_rows_in_multi_and_chain(qtype, batch):
    """The same rows through a two-segment launch and a one-step chain (the chain kernels' paths)."""
    say(f"case near-empty multi/chain {qtype} B={batch}")
    rng = np.random.default_rng(2000 + batch)
    f = _near_empty_fields(qtype, rng)
    g = _pack(qtype, f).reshape(ROWS, -1)
    x = _x(batch, "bf16", synth.seed_of("near-empty-multi", qtype, batch))
    split = 128
    parts = [split, ROWS - split]
    ws = [kq.repack(qtype, g[:split].contiguous().to(DEV), split, COLS),
          kq.repack(qtype, g[split:].contiguous().to(DEV), ROWS - split, COLS)]
    ys = [torch.empty(batch, r, device=DEV) for r in parts]
    xd = x.to(DEV)
    kq.kq_gemv_multi(qtype, ws, parts, COLS, xd, ys)
    torch.cuda.synchronize()
    yo, ao = O.gemv(qtype, ROWS, COLS, g.numpy(), x_host(x))
    check_y(torch.cat(ys, 1).cpu().numpy(), yo, ao, f"near-empty multi {qtype} B={batch}")
    yc = [torch.empty(batch, r, device=DEV) for r in parts]
    ch = kq.Chain([(qtype, ws, parts, COLS, xd, yc)], batch)
    ch.run()
    torch.cuda.synchronize()
    assert ch.status() == 0
    check_y(torch.cat(yc, 1).cpu().numpy(), yo, ao, f"near-empty chain {qtype} B={batch}")
    ch.close()
