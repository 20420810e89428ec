"""Row gather (the embedding lookup) against the oracle's dequantised rows, bit-exactly."""
import numpy as np
import pytest
import torch

from oracle import oracle as O
from quant_weight_streaming_amd import kq, synth
from tests.gpu_cases import say

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]
DEV = "cuda:0"


@pytest.mark.parametrize("qtype", ["q4k", "q5k", "q6k"])
def test_gather_matches_dequant(qtype):
    rows, cols = 5 * 64 + 11, 26 * 256              # ragged last tile, the 6656-hidden row length
    say(f"case gather {qtype} {rows}x{cols}")
    g = synth.gen_weights(qtype, rows, cols, synth.seed_of("gather", qtype))
    w = kq.repack(qtype, g.to(DEV), rows, cols)
    ids = np.array([0, rows - 1, 64, 63, 7, 7, rows - 11, 200, 0, 321, 65], dtype=np.int32)
    out = kq.gather_rows(qtype, w, rows, cols, torch.as_tensor(ids, device=DEV))
    torch.cuda.synchronize()
    want = O.gather(qtype, rows, cols, g.numpy(), ids)
    got = out.cpu().numpy()
    bad = got != want
    assert not bad.any(), f"{int(bad.sum())} gathered weights differ from the oracle, first at {np.argwhere(bad)[0]}"


def test_gather_strided_and_out_of_range():
    rows, cols = 130, 512
    say("case gather strided / out of range")
    g = synth.gen_weights("q6k", rows, cols, synth.seed_of("gather-oor"))
    w = kq.repack("q6k", g.to(DEV), rows, cols)
    ids = torch.tensor([3, -1, 130, 129, 1 << 30], dtype=torch.int32, device=DEV)
    out = torch.full((5, cols + 9), 7.0, device=DEV)
    kq.kq_gather_rows("q6k", w, rows, cols, ids, out)
    torch.cuda.synchronize()
    o = out.cpu().numpy()
    want = O.dequant_f32("q6k", rows, cols, g.numpy())
    assert (o[0, :cols] == want[3]).all() and (o[3, :cols] == want[129]).all()
    assert np.isnan(o[[1, 2, 4], :cols]).all(), "an id outside [0, rows) must give a row of NaNs"
    assert (o[:, cols:] == 7.0).all(), "wrote outside [0, cols)"


def test_gather_embedding_full_size():
    """The untied embedding of the 6656-hidden decoder (202048 x 6656), a decode step's eight tokens."""
    rows, cols = synth.VOCAB_P4, synth.HIDDEN_P4
    say("case gather 202048x6656")
    g = synth.gen_weights("q6k", rows, cols, synth.seed_of("gather-emb"), device=DEV)
    w = kq.repack("q6k", g, rows, cols)
    ids = np.array([0, 1, 12345, 202047, 99999, 64, 63, 150000], dtype=np.int32)
    out = kq.gather_rows("q6k", w, rows, cols, torch.as_tensor(ids, device=DEV))
    torch.cuda.synchronize()
    want = O.dequant_f32("q6k", len(ids), cols, g[torch.as_tensor(ids, device=DEV).long()].cpu().numpy())
    assert (out.cpu().numpy() == want).all()
