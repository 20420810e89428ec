"""Chains (kq_chain_*): a dependent sequence of GEMV steps in one persistent launch.

Every step must give what the same kq_gemv_multi call gives on its own (same
partition, so bitwise), within the oracle tolerance; a step whose x is the
previous step's y must read it only after it is complete; a run may be replayed
from a HIP graph; and a wait that gives up is reported, not hung on.
"""
import os

import numpy as np
import pytest
import torch

from oracle import oracle as O
from quant_weight_streaming_amd import kq, synth
from tests.gpu_cases import check_y, say, x_host

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]
DEV = "cuda:0"


@pytest.fixture(autouse=True)
def _chain_shape(monkeypatch):
    """Single launches with the chain's workgroup shape (8 wavefronts; at batch 1 single launches default to one
    4-wavefront workgroup per CU), so a chain step and its single launch run the same arithmetic in the same order."""
    monkeypatch.setenv("KQ_WG_WAVES", "8")
SENTINEL = 1.0e30


def _weights(qtype, parts, cols, tag):
    gs = [synth.gen_weights(qtype, r, cols, synth.seed_of("chain", tag, i)) for i, r in enumerate(parts)]
    ws = [kq.repack(qtype, g.to(DEV), r, cols) for g, r in zip(gs, parts)]
    return gs, ws


def _singles(steps):
    """The same steps as separate kq_gemv_multi launches, into fresh outputs."""
    outs = []
    for qtype, ws, rows, cols, x, ys in steps:
        yy = [torch.full_like(y, SENTINEL) for y in ys]
        kq.kq_gemv_multi(qtype, ws, rows, cols, x, yy)
        outs.append(yy)
    torch.cuda.synchronize()
    return outs


def _independent_steps(specs, batch, xdtype, tag):
    """specs: (qtype, parts, cols); each step gets its own x."""
    steps, hosts = [], []
    for j, (qtype, parts, cols) in enumerate(specs):
        gs, ws = _weights(qtype, parts, cols, f"{tag}{j}")
        x = synth.gen_x(batch, cols, synth.seed_of("chain-x", tag, j), xdtype)
        ys = [torch.full((batch, r + 3), SENTINEL, device=DEV) for r in parts]
        steps.append((qtype, ws, list(parts), cols, x.to(DEV), ys))
        hosts.append((gs, x))
    return steps, hosts


def _check_steps(steps, hosts, singles, where):
    for j, ((qtype, ws, parts, cols, x, ys), (gs, xh), ref) in enumerate(zip(steps, hosts, singles)):
        for i, (g, r, y, y1) in enumerate(zip(gs, parts, ys, ref)):
            yc = y[:, :r].cpu()
            assert torch.equal(yc, y1[:, :r].cpu()), f"{where} step {j} part {i}: differs from its single launch"
            assert (y[:, r:].cpu() == SENTINEL).all(), f"{where} step {j} part {i}: wrote outside [0, rows)"
            yo, ao = O.gemv(qtype, r, cols, g.numpy(), x_host(xh))
            check_y(yc.numpy(), yo, ao, f"{where} step {j} part {i}")


MIXED = [("q4k", (100, 64, 37), 1024), ("q6k", (300,), 512), ("q5k", (129,), 2048),
         ("q4k", (64,), 256), ("q6k", (5 * 64 + 9,), 122 * 256), ("q4k", (1,), 256)]


@pytest.mark.parametrize("batch,xdtype", [(1, "bf16"), (2, "bf16"), (3, "bf16"), (5, "bf16"), (8, "bf16"),
                                          (12, "bf16"), (16, "bf16"), (1, "f32"), (4, "f32"),
                                          (6, "f32"), (8, "f32")])
def test_chain_matches_single_launches(batch, xdtype):
    say(f"case chain mixed B={batch} x={xdtype}")
    steps, hosts = _independent_steps(MIXED, batch, xdtype, f"mixed{batch}{xdtype}")
    ch = kq.Chain(steps, batch)
    for rep in range(2):                       # the second run starts from the counters the first left
        for s in steps:
            for y in s[5]:
                y.fill_(SENTINEL)
        ch.run()
        torch.cuda.synchronize()
        assert ch.status() == 0
        _check_steps(steps, hosts, _singles(steps), f"mixed B={batch} {xdtype} run {rep}")
    ch.close()


@pytest.mark.parametrize("batch", [1, 8])
def test_chain_sweep_layer(batch):
    """One decoder layer at full size plus the head, as the sweep runs them."""
    say(f"case chain sweep layer B={batch}")
    specs = [(s.qtype, tuple(s.parts) or (s.rows,), s.cols)
             for s in (synth.QKV, synth.O_PROJ, synth.GATE_UP, synth.DOWN, synth.HEAD)]
    steps = []
    for j, (qtype, parts, cols) in enumerate(specs):
        ws = []
        for i, r in enumerate(parts):
            g = synth.gen_weights(qtype, r, cols, synth.seed_of("chain-layer", j, i), device=DEV)
            ws.append(kq.repack(qtype, g, r, cols))
            del g
        x = synth.gen_x(batch, cols, synth.seed_of("chain-layer-x", j), device=DEV)
        steps.append((qtype, ws, list(parts), cols, x, [torch.empty((batch, r), device=DEV) for r in parts]))
    singles = _singles(steps)
    ch = kq.Chain(steps, batch)
    ch.run()
    torch.cuda.synchronize()
    assert ch.status() == 0
    for j, (s, ref) in enumerate(zip(steps, singles)):
        for i, (y, y1) in enumerate(zip(s[5], ref)):
            assert torch.equal(y, y1), f"layer step {j} part {i}: differs from its single launch"
    ch.close()


def _dependent_chain(batch):
    """fp32 chain where every step reads the previous step's y: K_{j+1} = M_j."""
    specs = [("q4k", (512,), 1024), ("q6k", (768,), 512), ("q5k", (256,), 768), ("q4k", (300, 212), 256)]
    x0 = synth.gen_x(batch, 1024, synth.seed_of("dep-x"), "f32").to(DEV)
    steps, gs_all, x = [], [], x0
    for j, (qtype, parts, cols) in enumerate(specs):
        gs, ws = _weights(qtype, parts, cols, f"dep{j}")
        ys = [torch.full((batch, r), SENTINEL, device=DEV) for r in parts]
        steps.append((qtype, ws, list(parts), cols, x, ys))
        gs_all.append(gs)
        x = ys[0]                                   # the next step reads this step's (first) output
    return steps, gs_all, x0


@pytest.mark.parametrize("batch", [1, 3])
def test_chain_reads_previous_output(batch):
    say(f"case chain dependent fp32 B={batch}")
    steps, gs_all, x0 = _dependent_chain(batch)
    ch = kq.Chain(steps, batch)
    for rep in range(3):
        for s in steps:
            for y in s[5]:
                y.fill_(SENTINEL)                   # a step that read too early would see these
        ch.run()
        torch.cuda.synchronize()
        assert ch.status() == 0
        # each step against a single launch on the chain's own input, bitwise
        for j, (qtype, ws, parts, cols, x, ys) in enumerate(steps):
            ref = [torch.empty_like(y) for y in ys]
            kq.kq_gemv_multi(qtype, ws, parts, cols, x, ref)
            torch.cuda.synchronize()
            for i, (y, y1) in enumerate(zip(ys, ref)):
                assert torch.equal(y, y1), f"dependent run {rep} step {j} part {i}: differs from a single launch"
    # against the oracle run step by step on its own outputs, with the error carried through: if the
    # input of a step is off by at most E, its output is off by at most |W| (1.0001 E + 2e-4 |x|)
    # (the inherited error, this step's 1e-4 * sum |w x| and the fp32 rounding of the oracle's input)
    xh = x_host(x0).astype(np.float64)
    e_prev = np.zeros_like(xh)
    for j, (qtype, ws, parts, cols, x, ys) in enumerate(steps):
        nxt = None
        for i, (g, r, y) in enumerate(zip(gs_all[j], parts, ys)):
            yo, ao = O.gemv(qtype, r, cols, g.numpy(), xh.astype(np.float32))
            W = np.abs(O.dequant_f32(qtype, r, cols, g.numpy()).astype(np.float64))
            bound = (1.0001 * e_prev + 2e-4 * np.abs(xh)) @ W.T
            err = np.abs(y.cpu().numpy().astype(np.float64) - yo)
            assert (err <= bound).all(), f"dependent step {j} part {i}: {int((err > bound).sum())} outputs off"
            if i == 0:
                nxt = (yo, bound)
        xh, e_prev = nxt
    ch.close()


def test_chain_graph_replay():
    """A captured run replayed several times, with eager work in between, equals the eager run."""
    batch = 2
    say("case chain graph replay")
    steps, gs_all, x0 = _dependent_chain(batch)
    ch = kq.Chain(steps, batch)
    ch.run()
    torch.cuda.synchronize()
    want = [[y.clone() for y in s[5]] for s in steps]
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            ch.run(s)
    torch.cuda.current_stream().wait_stream(s)
    for rep in range(3):
        for st in steps:
            for y in st[5]:
                y.fill_(SENTINEL)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for j, (st, w) in enumerate(zip(steps, want)):
            for i, (y, y1) in enumerate(zip(st[5], w)):
                assert torch.equal(y, y1), f"replay {rep} step {j} part {i} differs from the eager run"
    assert ch.status() == 0
    del g
    ch.close()


@pytest.mark.parametrize("batch", [1, 8])
def test_chain_wait_that_gives_up_is_reported(batch, monkeypatch):
    """With no polls allowed (KQ_CHAIN_SPIN=0, read at each run) a wait that finds the previous step unfinished
    gives up: the run's results are invalid, the host-visible flag says so without a device synchronisation
    (kq_chain_query), the next kq_chain_run is refused, and kq_chain_status reports it and resets the chain.
    The same chain then runs clean with the default limit and matches its single launches bitwise (so the
    time-out left no stale split-tile counters behind).  Step 1 gives every workgroup work, so every
    workgroup waits for step 0, and the first to finish step 0 finds it unfinished.  Batch 1 waits in two
    hops (collector, done word), batch 8 in one (every workgroup polls the arrivals)."""
    timeout = kq.STATUS_CODE["KQ_ERR_TIMEOUT"]
    say(f"case chain spin 0 B={batch}")
    specs = [("q6k", (64 * 64,), 122 * 256), ("q4k", (16384,), 4096), ("q4k", (256,), 1024)]
    steps, hosts = _independent_steps(specs, batch, "bf16", "spin")
    ch = kq.Chain(steps, batch)
    monkeypatch.setenv("KQ_CHAIN_SPIN", "0")
    ch.run()
    torch.cuda.synchronize()
    assert ch.query() == timeout               # host-visible, no synchronisation
    with pytest.raises(kq.KQError) as err:     # refused: nothing is enqueued until a reset
        ch.run()
    assert err.value.code == timeout
    assert ch.status() == timeout              # reports and resets
    assert ch.query() == 0 and ch.status() == 0
    monkeypatch.delenv("KQ_CHAIN_SPIN")
    for rep in range(2):
        for s in steps:
            for y in s[5]:
                y.fill_(SENTINEL)
        ch.run()
        torch.cuda.synchronize()
        assert ch.status() == 0
        _check_steps(steps, hosts, _singles(steps), f"the same chain after a time-out, run {rep}")
    ch.close()


def test_chain_dynamic_units(monkeypatch):
    """Batch 1 with 8-wavefront workgroups (KQ_WG_WAVES=8): the chain's steps take units dynamically
    and still match their single launches bitwise."""
    monkeypatch.setenv("KQ_WG_WAVES", "8")
    say("case chain dynamic units")
    steps, hosts = _independent_steps(MIXED, 1, "bf16", "dyn")
    ch = kq.Chain(steps, 1)
    ch.run()
    torch.cuda.synchronize()
    assert ch.status() == 0
    _check_steps(steps, hosts, _singles(steps), "chain dynamic units")
    ch.close()


@pytest.mark.parametrize("batch", [1, 3])
def test_chain_four_wave_workgroups(batch, monkeypatch):
    """KQ_WG_WAVES=4 forces 4-wavefront workgroups on chains and single launches alike (two per CU): the
    chain's steps still match their single launches bitwise."""
    monkeypatch.setenv("KQ_WG_WAVES", "4")
    say(f"case chain four-wave workgroups B={batch}")
    steps, hosts = _independent_steps(MIXED, batch, "bf16", f"w4{batch}")
    ch = kq.Chain(steps, batch)
    ch.run()
    torch.cuda.synchronize()
    assert ch.status() == 0
    _check_steps(steps, hosts, _singles(steps), "chain four-wave workgroups")
    ch.close()


@pytest.mark.parametrize("batch", [1, 8])
def test_chain_p4_layer(batch):
    """One layer and the head of the 6656-hidden decoder as a chain.  The resident grid forces longer
    runs than a single launch picks (the head at batch 8 takes 25 whole tiles of a column window per
    workgroup), so the steps are checked against the oracle on sampled rows."""
    from tests.gpu_cases import oracle_rows, sample_rows
    say(f"case chain p4 layer B={batch}")
    steps, gens = [], []
    for j, spec in enumerate((synth.QKVG_P4, synth.O_P4, synth.GATE_UP_P4, synth.DOWN_P4, synth.HEAD_P4)):
        parts = list(spec.parts) or [spec.rows]
        g = synth.gen_weights(spec.qtype, spec.rows, spec.cols, synth.seed_of("chain-p4", j), device=DEV)
        starts = np.cumsum([0] + parts)
        ws = [kq.repack(spec.qtype, g[starts[i]:starts[i + 1]].contiguous(), r, spec.cols) for i, r in enumerate(parts)]
        x = synth.gen_x(batch, spec.cols, synth.seed_of("chain-p4-x", j), device=DEV)
        steps.append((spec.qtype, ws, parts, spec.cols, x, [torch.empty((batch, r), device=DEV) for r in parts]))
        gens.append(g)
    ch = kq.Chain(steps, batch)
    ch.run()
    torch.cuda.synchronize()
    assert ch.status() == 0
    for j, ((qtype, ws, parts, cols, x, ys), g) in enumerate(zip(steps, gens)):
        rows = sum(parts)
        idx = sample_rows(rows, 96, 600 + j)
        y = torch.cat(ys, dim=1)[:, torch.as_tensor(idx, device=DEV)].cpu().numpy()
        _, yo, ao = oracle_rows(qtype, g, idx, cols, x)
        check_y(y, yo, ao, f"chain p4 step {j} B={batch}")
    ch.close()


@pytest.mark.parametrize("batch,xdtype", [(1, "bf16"), (2, "bf16"), (8, "bf16"), (16, "bf16"), (4, "f32")])
@pytest.mark.parametrize("same_plans", [True, False])
def test_chain_overlap_of_independent_steps(batch, xdtype, same_plans, monkeypatch):
    """KQ_STEP_OVERLAP on steps whose buffers are all distinct: no step after the first waits at the step
    barrier.  Overlapping steps with fewer than 8 units per CU (all of these) take whole tiles per
    workgroup; with KQ_WHOLE_TILES_BELOW=8 the single launches (and the chain's first step) are planned the
    same way, and every step gives its single launch's result bitwise.  Either way every output is within
    the oracle's bound, and two runs in a row give the same bits."""
    if same_plans:
        monkeypatch.setenv("KQ_WHOLE_TILES_BELOW", "8")
    say(f"case chain overlap independent B={batch} x={xdtype} same plans {same_plans}")
    steps, hosts = _independent_steps(MIXED + MIXED[:3], batch, xdtype, f"ovl{batch}{xdtype}")
    ch = kq.Chain(steps, batch, overlap=True)
    assert ch.waits() == [True] + [False] * (len(steps) - 1)
    first = None
    for rep in range(2):
        for s in steps:
            for y in s[5]:
                y.fill_(SENTINEL)
        ch.run()
        torch.cuda.synchronize()
        assert ch.status() == 0
        if same_plans:
            _check_steps(steps, hosts, _singles(steps), f"overlap B={batch} {xdtype} run {rep}")
        else:
            got = [[y.clone() for y in s[5]] for s in steps]
            if first is None:
                first = got
                for j, ((qtype, ws, parts, cols, x, ys), (gs, xh)) in enumerate(zip(steps, hosts)):
                    for i, (g, r, y) in enumerate(zip(gs, parts, ys)):
                        assert (y[:, r:].cpu() == SENTINEL).all(), f"overlap step {j} part {i}: wrote outside"
                        yo, ao = O.gemv(qtype, r, cols, g.numpy(), x_host(xh))
                        check_y(y[:, :r].cpu().numpy(), yo, ao, f"overlap B={batch} {xdtype} step {j} part {i}")
            else:
                for j, (a, b) in enumerate(zip(first, got)):
                    for i, (ya, yb) in enumerate(zip(a, b)):
                        assert torch.equal(ya, yb), f"overlap step {j} part {i}: runs differ"
    ch.close()


@pytest.mark.parametrize("batch", [1, 3])
def test_chain_overlap_keeps_dependencies(batch, monkeypatch):
    """KQ_STEP_OVERLAP with buffers shared between steps (fp32 activations, so an output can be a later
    step's input or overwrite an earlier step's input):
      A: own x -> yA;  B: own x -> yB;  C: x = yA (reads A's output: waits);
      D: own x -> yD (meets nothing still running: overlaps);  E: x = yB (B finished before C read: overlaps);
      F: own x -> writes D's x in place (D may still be reading it: waits).
    Each step must equal its single launch on the input it should have read (all steps planned with whole
    tiles per workgroup, as the overlapping ones are)."""
    monkeypatch.setenv("KQ_WHOLE_TILES_BELOW", "8")
    say(f"case chain overlap dependencies B={batch}")
    f32 = dict(dtype=torch.float32, device=DEV)

    def xg(cols, tag):
        return synth.gen_x(batch, cols, synth.seed_of("ovl-dep-x", tag, batch), "f32").to(DEV)

    specs = {"A": ("q4k", (512,), 1024), "B": ("q6k", (768,), 512), "C": ("q5k", (256,), 512),
             "D": ("q4k", (300, 212), 256), "E": ("q6k", (256,), 768), "F": ("q4k", (256,), 512)}
    W = {k: _weights(q, p, c, f"ovl-dep{k}")[1] for k, (q, p, c) in specs.items()}
    xa, xb, xd0, xf = xg(1024, "a"), xg(512, "b"), xg(256, "d"), xg(512, "f")
    xd = xd0.clone()
    Y = {k: [torch.full((batch, r), SENTINEL, **f32) for r in p] for k, (q, p, c) in specs.items() if k != "F"}
    Y["F"] = [xd]                                     # F overwrites D's input
    X = {"A": xa, "B": xb, "C": Y["A"][0], "D": xd, "E": Y["B"][0], "F": xf}
    order = "ABCDEF"
    steps = [(specs[k][0], W[k], list(specs[k][1]), specs[k][2], X[k], Y[k]) for k in order]
    ch = kq.Chain(steps, batch, overlap=True)
    assert ch.waits() == [True, False, True, False, False, True]
    for rep in range(3):
        xd.copy_(xd0)
        for k in "ABCDE":
            for y in Y[k]:
                y.fill_(SENTINEL)
        torch.cuda.synchronize()
        ch.run()
        torch.cuda.synchronize()
        assert ch.status() == 0
        inputs = {"A": xa, "B": xb, "C": Y["A"][0], "D": xd0, "E": Y["B"][0], "F": xf}
        for k in order:
            q, parts, cols = specs[k]
            ref = [torch.empty((batch, r), **f32) for r in parts]
            kq.kq_gemv_multi(q, W[k], list(parts), cols, inputs[k], ref)
            torch.cuda.synchronize()
            for i, (y, y1) in enumerate(zip(Y[k], ref)):
                assert torch.equal(y, y1), f"overlap with dependencies, run {rep} step {k} part {i}"
    ch.close()
