"""Mixed K-quant types inside one chain step (a QKV projection whose V rows are Q6_K and q/k rows Q4_K,
as in mixed-type GGUF builds).  Every segment must be within the oracle's bound, and each type's segments
bitwise equal to the kq_gemv_fused call over them (the chain's workgroup shape); the step reads x once
and its sub-steps run in the same launch.  A dependent second step checks the step's outputs are complete
before the next step reads them."""
import numpy as np
import pytest
import torch

from oracle import oracle as O
from quant_weight_streaming_amd import kq, synth
from tests.gpu_cases import check_y, oracle_rows, sample_rows, say, x_host

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]
DEV = "cuda:0"
SENTINEL = 1.0e30


@pytest.fixture(autouse=True)
def _chain_shape(monkeypatch):
    """Single launches with the chain's workgroup shape, so a sub-step and its single launch agree bitwise."""
    monkeypatch.setenv("KQ_WG_WAVES", "8")


def _segments(types, parts, cols, tag):
    gs = [synth.gen_weights(t, r, cols, synth.seed_of("mixed", tag, i)) for i, (t, r) in enumerate(zip(types, parts))]
    ws = [kq.repack(t, g.to(DEV), r, cols) for t, g, r in zip(types, gs, parts)]
    return gs, ws


def _by_type(types):
    order = []
    for t in types:
        if t not in order:
            order.append(t)
    return [(t, [i for i, u in enumerate(types) if u == t]) for t in order]


@pytest.mark.parametrize("batch,xdtype", [(1, "bf16"), (2, "bf16"), (3, "bf16"), (8, "bf16"), (16, "bf16"),
                                          (1, "f32"), (4, "f32")])
def test_mixed_step_matches_fused_launches(batch, xdtype):
    types = ["q4k", "q4k", "q6k", "q5k"]
    parts = [512, 128, 128, 200]
    epis = [kq.KQ_EPI_HEADNORM, kq.KQ_EPI_HEADNORM, kq.KQ_EPI_NONE, kq.KQ_EPI_SIGMOID]
    cols = 1024
    say(f"case mixed step B={batch} {xdtype}")
    gs, ws = _segments(types, parts, cols, f"m{batch}{xdtype}")
    x = synth.gen_x(batch, cols, synth.seed_of("mixed-x", batch, xdtype), xdtype)
    xd = x.to(DEV)
    ys = [torch.full((batch, r + 3), SENTINEL, device=DEV) for r in parts]
    packed = sum(e << (4 * i) for i, e in enumerate(epis))
    ch = kq.Chain([(types, ws, parts, cols, xd, ys, packed, 1e-5, 1e-6)], batch)
    ch.run()
    torch.cuda.synchronize()
    assert ch.status() == 0
    # each type's segments as one fused launch
    ref = [None] * len(parts)
    for t, idx in _by_type(types):
        yy = [torch.full((batch, parts[i] + 3), SENTINEL, device=DEV) for i in idx]
        kq.kq_gemv_fused(t, [ws[i] for i in idx], [parts[i] for i in idx], cols, xd, yy, [epis[i] for i in idx],
                         1e-5, None, 1e-6)
        for i, y in zip(idx, yy):
            ref[i] = y
    torch.cuda.synchronize()
    for i, (y, r) in enumerate(zip(ys, ref)):
        assert torch.equal(y, r), f"segment {i} ({types[i]}) differs from its fused launch"
        assert (y[:, parts[i]:] == SENTINEL).all(), f"segment {i} wrote outside [0, rows)"
    ch.close()


@pytest.mark.parametrize("batch", [1, 8])
def test_mixed_step_plain_against_oracle(batch):
    """Without epilogues every segment of a mixed step is checked element by element against the oracle."""
    types = ["q6k", "q4k", "q5k", "q4k"]
    parts = [70, 300, 129, 64]
    cols = 2048
    say(f"case mixed plain B={batch}")
    gs, ws = _segments(types, parts, cols, f"p{batch}")
    x = synth.gen_x(batch, cols, synth.seed_of("mixed-px", batch), "bf16")
    ys = [torch.empty((batch, r), device=DEV) for r in parts]
    ch = kq.Chain([(types, ws, parts, cols, x.to(DEV), ys)], batch)
    ch.run()
    torch.cuda.synchronize()
    assert ch.status() == 0
    for t, g, r, y in zip(types, gs, parts, ys):
        yo, ao = O.gemv(t, r, cols, g.numpy(), x_host(x))
        check_y(y.cpu().numpy(), yo, ao, f"mixed plain {t} {r} rows B={batch}")
    ch.close()


def test_mixed_step_then_dependent_step():
    """Step 1 (Q4_K) reads the q segment written by step 0 (mixed Q4_K/Q6_K): the barrier before step 1
    covers every sub-step of step 0."""
    batch, cols = 3, 1024
    types, parts = ["q4k", "q6k"], [1024, 256]
    say("case mixed then dependent")
    gs, ws = _segments(types, parts, cols, "dep")
    x = synth.gen_x(batch, cols, synth.seed_of("mixed-dep-x"), "f32").to(DEV)
    ys = [torch.empty((batch, r), device=DEV) for r in parts]
    g2 = synth.gen_weights("q4k", 500, 1024, synth.seed_of("mixed-dep-2"))
    w2 = kq.repack("q4k", g2.to(DEV), 500, 1024)
    y2 = torch.empty((batch, 500), device=DEV)
    ch = kq.Chain([(types, ws, parts, cols, x, ys), ("q4k", [w2], [500], 1024, ys[0], [y2])], batch)
    ch.run()
    torch.cuda.synchronize()
    assert ch.status() == 0
    yo, ao = O.gemv("q4k", 500, 1024, g2.numpy(), ys[0].cpu().numpy())
    check_y(y2.cpu().numpy(), yo, ao, "step reading a mixed step's output")
    ch.close()


@pytest.mark.parametrize("batch", [1, 8])
def test_q4km_qkv_full_size(batch):
    """The Q4_K_M-style QKV projection at full size (4096 + 256 rows Q4_K, 256 rows Q6_K, K = 5120): sampled
    rows of every segment against the oracle."""
    spec = synth.QKV_Q4KM
    say(f"case Q4_K_M QKV full size B={batch}")
    types, parts = spec.part_types(), list(spec.parts)
    gens = [synth.gen_weights(t, r, spec.cols, synth.seed_of("q4km", i), device=DEV)
            for i, (t, r) in enumerate(zip(types, parts))]
    ws = [kq.repack(t, g, r, spec.cols) for t, g, r in zip(types, gens, parts)]
    x = synth.gen_x(batch, spec.cols, synth.seed_of("q4km-x", batch), device=DEV)
    ys = [torch.empty((batch, r), device=DEV) for r in parts]
    ch = kq.Chain([(types, ws, parts, spec.cols, x, ys)], batch)
    ch.run()
    torch.cuda.synchronize()
    assert ch.status() == 0
    for i, (t, g, r, y) in enumerate(zip(types, gens, parts, ys)):
        idx = sample_rows(r, 48, 700 + i)
        _, yo, ao = oracle_rows(t, g, idx, spec.cols, x)
        check_y(y[:, torch.as_tensor(idx, device=DEV)].cpu().numpy(), yo, ao, f"Q4_K_M QKV segment {i} B={batch}")
    ch.close()


@pytest.mark.parametrize("batch", [1, 3])
def test_mixed_step_reads_previous_output(batch):
    """A mixed step whose x is the previous step's output: the workgroups of its later sub-steps (which start
    on the workgroups after the first sub-step's) must also wait until the previous step is complete, not
    only those of its first sub-step.  The previous step's output is reset to a sentinel before each run, so
    a read that comes too early shows."""
    say(f"case mixed step reading the previous output B={batch}")
    cols = 1024
    g0 = synth.gen_weights("q6k", cols, 64 * 256, synth.seed_of("mixed-prev-0"))
    w0 = kq.repack("q6k", g0.to(DEV), cols, 64 * 256)
    x0 = synth.gen_x(batch, 64 * 256, synth.seed_of("mixed-prev-x", batch), "f32").to(DEV)
    y0 = torch.empty((batch, cols), device=DEV)
    types, parts = ["q4k", "q6k"], [64, 64]
    gs, ws = _segments(types, parts, cols, f"prev{batch}")
    ys = [torch.empty((batch, r), device=DEV) for r in parts]
    ch = kq.Chain([("q6k", [w0], [cols], 64 * 256, x0, [y0]), (types, ws, parts, cols, y0, ys)], batch)
    for rep in range(4):
        y0.fill_(SENTINEL)
        for y in ys:
            y.fill_(SENTINEL)
        torch.cuda.synchronize()
        ch.run()
        torch.cuda.synchronize()
        assert ch.status() == 0
        for t, idx in _by_type(types):
            ref = [torch.empty((batch, parts[i]), device=DEV) for i in idx]
            kq.kq_gemv_fused(t, [ws[i] for i in idx], [parts[i] for i in idx], cols, y0, ref)
            torch.cuda.synchronize()
            for i, r in zip(idx, ref):
                assert torch.equal(ys[i], r), f"run {rep} segment {i} ({t}) read its x before it was complete"
    ch.close()
