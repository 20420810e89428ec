"""The boundary's rules on the device: the library allocates nothing on a GEMV call, every call takes the
caller's workspace (the exact size the query reports is enough, less is refused), and calls on unordered
streams with their own workspaces are correct (each within the oracle's bound and bitwise equal to the same
call made alone)."""
import numpy as np
import pytest
import torch

from oracle import oracle as O
from quant_weight_streaming_amd import kq, synth
from tests.gpu_cases import check_y, say, x_host

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]
DEV = "cuda:0"

CASES = [  # (qtype, rows, cols, batch): hand-offs of split tiles, column windows, the dot2 and matrix-core paths
    ("q4k", 4096 + 17, 5120, 1),
    ("q6k", 640, 31232, 8),
    ("q5k", 1000, 2048, 3),
    ("q4k", 300, 31232, 16),
]


def _problem(qtype, rows, cols, batch, tag):
    g = synth.gen_weights(qtype, rows, cols, synth.seed_of("boundary", tag))
    x = synth.gen_x(batch, cols, synth.seed_of("boundary-x", tag), "bf16")
    return g, x, kq.repack(qtype, g.to(DEV), rows, cols), x.to(DEV)


def _workspace(nbytes):
    ws = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=DEV)
    kq.kq_workspace_init(ws)
    return ws


@pytest.mark.parametrize("case", range(len(CASES)))
def test_workspace_query_is_exact(case):
    qtype, rows, cols, batch = CASES[case]
    say(f"case workspace query {CASES[case]}")
    g, x, w, xd = _problem(qtype, rows, cols, batch, case)
    need = kq.kq_gemv_workspace_bytes(qtype, [rows], cols, kq.KQ_X_BF16, batch)
    assert 64 * 1024 <= need <= kq.KQ_WORKSPACE_BYTES
    exact = _workspace(need)
    y = kq.gemv(qtype, w, rows, cols, xd, work=exact)
    ref = kq.gemv(qtype, w, rows, cols, xd)            # the stream's own full-size workspace
    torch.cuda.synchronize()
    assert torch.equal(y, ref)
    yo, ao = O.gemv(qtype, rows, cols, g.numpy(), x_host(x))
    check_y(y.cpu().numpy(), yo, ao, f"exact workspace {CASES[case]}")
    with pytest.raises(kq.KQError) as err:
        kq.gemv(qtype, w, rows, cols, xd, work=exact[:need - 16])
    assert err.value.code == kq.STATUS_CODE["KQ_ERR_WORKSPACE"]


def test_no_device_allocation_on_the_call_path():
    """Device memory in use does not change across GEMV calls once their kernels are loaded: the library
    itself allocates nothing (outputs and workspace come from the caller)."""
    say("case no allocation on the call path")
    probs = [_problem(*c, 10 + i) for i, c in enumerate(CASES)]
    ws = _workspace(kq.KQ_WORKSPACE_BYTES)
    ys = [torch.empty((c[3], c[1]), device=DEV) for c in CASES]
    for (qtype, rows, cols, batch), (_, _, w, xd), y in zip(CASES, probs, ys):   # load every kernel once
        kq.GEMV[qtype](w, rows, cols, xd, y, None, ws)
    torch.cuda.synchronize()
    free0, _ = torch.cuda.mem_get_info()
    for _ in range(3):
        for (qtype, rows, cols, batch), (_, _, w, xd), y in zip(CASES, probs, ys):
            kq.GEMV[qtype](w, rows, cols, xd, y, None, ws)
    torch.cuda.synchronize()
    free1, _ = torch.cuda.mem_get_info()
    assert free1 == free0, f"device memory in use changed by {free0 - free1} bytes across GEMV calls"


def test_unordered_streams_with_their_own_workspaces():
    """Two streams with no ordering between them each run their own problem 12 times into 12 outputs, the
    launches interleaved on the host.  Each stream's calls use that stream's workspace (the binding keeps
    one per stream).  Every output must equal the same call made alone, and be within the oracle's bound."""
    say("case two unordered streams")
    a, b = CASES[0], CASES[1]
    pa, pb = _problem(*a, "sa"), _problem(*b, "sb")
    alone_a = kq.gemv(a[0], pa[2], a[1], a[2], pa[3])
    alone_b = kq.gemv(b[0], pb[2], b[1], b[2], pb[3])
    torch.cuda.synchronize()
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    s1.wait_stream(torch.cuda.current_stream())
    s2.wait_stream(torch.cuda.current_stream())
    ya = [torch.full((a[3], a[1]), float("nan"), device=DEV) for _ in range(12)]
    yb = [torch.full((b[3], b[1]), float("nan"), device=DEV) for _ in range(12)]
    torch.cuda.synchronize()
    for i in range(12):
        with torch.cuda.stream(s1):
            kq.gemv(a[0], pa[2], a[1], a[2], pa[3], ya[i], stream=s1)
        with torch.cuda.stream(s2):
            kq.gemv(b[0], pb[2], b[1], b[2], pb[3], yb[i], stream=s2)
    torch.cuda.synchronize()
    assert kq.workspace(s1).data_ptr() != kq.workspace(s2).data_ptr()
    for i in range(12):
        assert torch.equal(ya[i], alone_a), f"stream 1 call {i} differs from the call made alone"
        assert torch.equal(yb[i], alone_b), f"stream 2 call {i} differs from the call made alone"
    for (qtype, rows, cols, batch), (g, x, _, _), y in ((a, pa, alone_a), (b, pb, alone_b)):
        yo, ao = O.gemv(qtype, rows, cols, g.numpy(), x_host(x))
        check_y(y.cpu().numpy(), yo, ao, f"two streams {qtype}")
