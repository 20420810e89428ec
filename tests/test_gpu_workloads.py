"""The measured workloads at full size, launched as the benchmark launches them,
checked on sampled rows against the CPU oracle (dequantised weights bit-exact,
outputs within 1e-4 * sum |w x|)."""
import numpy as np
import pytest
import torch

from quant_weight_streaming_amd import kq, synth
from tests.gpu_cases import check_dequant, check_y, oracle_rows, sample_rows, say

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]
DEV = "cuda:0"


def run_gemv(spec: synth.Gemv, batches, cfg, merge=0.0, nsample=160):
    rows, cols, qtype = spec.rows, spec.cols, spec.qtype
    say(f"workload cfg{cfg} {spec.name} {qtype} {rows}x{cols} B={batches} merge={merge}")
    g = synth.gen_weights(qtype, rows, cols, synth.seed_of(cfg, 0, spec.name), device=DEV,
                          merge_frac=merge if qtype == "q4k" else 0.0)
    parts = list(spec.parts) or [rows]
    ws, starts = [], np.cumsum([0] + parts)
    for i, r in enumerate(parts):
        ws.append(kq.repack(qtype, g[starts[i]:starts[i + 1]].contiguous(), r, cols))
    idx = sample_rows(rows, nsample, cfg)
    for B in batches:
        x = synth.gen_x(B, cols, synth.seed_of(cfg, 0, spec.name, "x", B), "bf16", device=DEV)
        ys = [torch.empty((B, r), dtype=torch.float32, device=DEV) for r in parts]
        if len(parts) > 1:
            kq.kq_gemv_multi(qtype, ws, parts, cols, x, ys)
        else:
            kq.GEMV[qtype](ws[0], rows, cols, x, ys[0])
        torch.cuda.synchronize()
        y = torch.cat(ys, dim=1)[:, torch.as_tensor(idx, device=DEV)].cpu().numpy()
        gh, yo, ao = oracle_rows(qtype, g, idx, cols, x)
        worst = check_y(y, yo, ao, f"cfg{cfg} {spec.name} B={B}")
        say(f"  B={B}: worst |err|/sum|wx| = {worst:.3e}")
    # bit-exact dequant of the sampled rows, per part
    for i, r in enumerate(parts):
        sel = idx[(idx >= starts[i]) & (idx < starts[i + 1])] - starts[i]
        if len(sel):
            check_dequant(qtype, ws[i], r, cols, g[starts[i]:starts[i + 1]][torch.as_tensor(sel, device=DEV)].cpu().numpy(),
                          sel, f"cfg{cfg} {spec.name} part {i}")
    del ws, g
    torch.cuda.empty_cache()


def test_config1_gate_up_q4k():
    run_gemv(synth.GATE_UP, [1], 1)


def test_config2_head_q6k():
    run_gemv(synth.HEAD, [1], 2)


@pytest.mark.parametrize("spec", [synth.QKV, synth.O_PROJ, synth.GATE_UP, synth.DOWN, synth.HEAD],
                         ids=lambda s: s.name)
def test_config3_sweep_gemvs(spec):
    run_gemv(spec, [1, 8], 3)


@pytest.mark.parametrize("spec", [synth.QKV, synth.O_PROJ, synth.GATE_UP, synth.DOWN, synth.HEAD],
                         ids=lambda s: s.name)
def test_config4_sweep_gemvs(spec):
    import dataclasses
    if spec.name == "gate_up":
        spec = dataclasses.replace(spec, qtype="q5k")
    run_gemv(spec, [2, 4, 8], 4, merge=0.25)


@pytest.mark.parametrize("spec", [synth.QKVG_P4, synth.O_P4, synth.GATE_UP_P4, synth.DOWN_P4, synth.HEAD_P4],
                         ids=lambda s: s.name)
def test_p4_sweep_gemvs(spec):
    """The 6656-hidden decoder's projections (K = 26, 16 and 78 super-blocks, a four-way fused qkvg)."""
    run_gemv(spec, [1, 3, 8], 5)


@pytest.mark.parametrize("spec", [synth.QKV, synth.GATE_UP, synth.DOWN, synth.HEAD], ids=lambda s: s.name)
def test_verify_block_full_size(spec):
    """The sweep's projections verifying a 16-token speculative block (and 12), sampled rows."""
    run_gemv(spec, [12, 16], 6)
