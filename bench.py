#!/usr/bin/env python3
"""Decode-step K-quant GEMV weight-streaming benchmark on one MI355X.

One step = one decode-equivalent token: the 209 GEMVs of a synthetic 52-layer
28B-class decoder, back to back on one stream:
  52 x { QKV Q4_K 4608x5120 (one launch over q/k/v), O Q4_K 5120x4096,
         gate+up Q4_K 62464x5120 (one launch over gate/up), down Q6_K 5120x31232 }
  + head Q6_K 131072x5120  =  18,029,690,880 weight bytes.
Weights are resident in HBM (repacked once, untimed); every GEMV has its own
seeded bf16 activations.  The headline value is weight GB/s of the
hipGraph-replayed sweep at batch 1; batch 8, plain stream launches, the
Q5_K gate+up variant with merged sub-blocks (batch 2/4/8), per-kernel times,
the roofline of the dominant kernel and the CPU oracle baseline are reported in
the same JSON line.  Decode priced as weight bytes per token follows the Core AI
card's decode table ("23.7 x 17.9 GB is 424 GB/s of traffic").

Also reported: per-step median/min/max, the three single-GEMV workloads (the small Q4_K GEMV's latency,
gate+up and the head over rotated weight copies), the CPU oracle on one thread for those three, the
achievable HBM read rate (kq_stream_read), GPU power and clocks under load before and after the timed
work (amd-smi), and the host CPU model.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu] [--no-c4]
       python bench.py --profile-kernel N     # only the dominant kernel, N launches (for rocprofv3)
       python bench.py --copy-calibration N   # N plain device copies of 1 GiB (counter calibration)
"""
from __future__ import annotations

import argparse
import ctypes
import dataclasses
import glob
import hashlib
import re
import json
import math
import os
import sys
import time

HBM_PEAK_GBS = 8000.0
METRIC = "K-quant GEMV weight GB/s (% of HBM peak) + decode-equiv tok/s, batch 1 and 8"
ROOT = os.path.dirname(os.path.abspath(__file__))


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def weight_gbs(weight_bytes: float, ms: float) -> float:
    """Weight bytes streamed per millisecond of device time, in GB/s (decimal)."""
    return weight_bytes / ms / 1e6


def tok_s(ms_per_step: float, batch: int = 1) -> float:
    """Decode-equivalent tokens per second when one step streams the whole weight set once for `batch` tokens."""
    return batch * 1e3 / ms_per_step


def code_text(src: str) -> str:
    """C/C++ source without comments and with whitespace runs collapsed: what the kernels are built from."""
    src = re.sub(r"/\*.*?\*/", " ", src, flags=re.S)
    src = re.sub(r"//[^\n]*", " ", src)
    return " ".join(src.split())


def kernel_source_hash() -> str:
    """Hash of the library's code (comments and layout ignored) and of its build script."""
    h = hashlib.sha256()
    for p in sorted(glob.glob(os.path.join(ROOT, "quant_weight_streaming_amd", "csrc", "*"))):
        h.update(code_text(open(p).read()).encode())
    h.update(open(os.path.join(ROOT, "quant_weight_streaming_amd", "build.py"), "rb").read())
    return h.hexdigest()[:16]


class Sweep:
    """Device-resident weights, activations and outputs of one sweep, with the launch list."""

    def __init__(self, cfg, gate_up_type: str, batches, merge: float, sample_frac: float, entries=None):
        import torch
        from quant_weight_streaming_amd import kq, synth
        self.torch, self.kq, self.synth = torch, kq, synth
        self.cfg, self.batches = cfg, list(batches)
        self.entries = []          # (layer, spec, [repacked part tensors], parts)
        self.samples = []          # (qtype, rows_sampled, cols, host gguf bytes, layer, spec name)
        self.weight_bytes = 0
        dev = "cuda:0"
        t0 = time.time()
        for layer, spec in (entries if entries is not None else synth.sweep(gate_up_type)):
            parts = list(spec.parts) or [spec.rows]
            if spec.types:       # a mixed-type projection: each part drawn and repacked in its own type
                reps = [kq.repack(t, synth.gen_weights(t, r, spec.cols, synth.seed_of(cfg, layer, spec.name, i),
                                                       device=dev), r, spec.cols)
                        for i, (t, r) in enumerate(zip(spec.part_types(), parts))]
                self.weight_bytes += spec.weight_bytes()
                self.entries.append((layer, spec, reps, parts))
                continue
            g = synth.gen_weights(spec.qtype, spec.rows, spec.cols, synth.seed_of(cfg, layer, spec.name),
                                  device=dev, merge_frac=merge if spec.qtype == "q4k" else 0.0)
            starts = [0]
            for r in parts:
                starts.append(starts[-1] + r)
            reps = [kq.repack(spec.qtype, g[starts[i]:starts[i + 1]].contiguous(), r, spec.cols)
                    for i, r in enumerate(parts)]
            if sample_frac > 0:
                rs = min(spec.rows, max(1, int(math.ceil(sample_frac * spec.rows))))
                self.samples.append((spec.qtype, rs, spec.cols, g[:rs].cpu().numpy(), layer, spec.name))
            self.weight_bytes += spec.rows * spec.cols // 256 * synth.SB_BYTES[spec.qtype]
            self.entries.append((layer, spec, reps, parts))
            del g
        torch.cuda.synchronize()
        log(f"[bench] cfg{cfg} sweep: {len(self.entries)} GEMVs, {self.weight_bytes} weight bytes, "
            f"generated+repacked in {time.time() - t0:.1f} s")
        self.x, self.y = {}, {}
        for B in self.batches:
            self.x[B] = [synth.gen_x(B, spec.cols, synth.seed_of(cfg, layer, spec.name, "x", B), "bf16", device=dev)
                         for layer, spec, _, _ in self.entries]
            self.y[B] = [[torch.empty((B, r), dtype=torch.float32, device=dev) for r in parts]
                         for _, _, _, parts in self.entries]
        self._keep = []
        # one workspace for every call of the sweep: they all run in order on one stream (eager or replayed)
        self.work = torch.empty(kq.KQ_WORKSPACE_BYTES, dtype=torch.uint8, device=dev)
        kq.kq_workspace_init(self.work)
        torch.cuda.synchronize()

    def calls(self, B: int, stream: int):
        """Pre-marshalled C-ABI calls of one step (minimal Python work per launch)."""
        L = self.kq.lib()
        wsp, wsb = self.work.data_ptr(), self.work.numel()
        out = []
        for i, (layer, spec, reps, parts) in enumerate(self.entries):
            x, ys = self.x[B][i], self.y[B][i]
            t = self.kq.TYPE_ID[spec.qtype]
            if spec.types:       # mixed types: one multi-projection launch per type
                pt = spec.part_types()
                for qt in dict.fromkeys(pt):
                    idx = [k for k, u in enumerate(pt) if u == qt]
                    n = len(idx)
                    W = (ctypes.c_void_p * n)(*[reps[k].data_ptr() for k in idx])
                    R = (ctypes.c_int64 * n)(*[parts[k] for k in idx])
                    Y = (ctypes.c_void_p * n)(*[ys[k].data_ptr() for k in idx])
                    LD = (ctypes.c_int64 * n)(*[ys[k].stride(0) for k in idx])
                    self._keep += [W, R, Y, LD]
                    out.append((L.kq_gemv_multi, (self.kq.TYPE_ID[qt], n, W, R, spec.cols, x.data_ptr(), 1,
                                                   x.stride(0), B, Y, LD, wsp, wsb, stream), spec.name))
                continue
            if len(parts) > 1:
                n = len(parts)
                W = (ctypes.c_void_p * n)(*[w.data_ptr() for w in reps])
                R = (ctypes.c_int64 * n)(*parts)
                Y = (ctypes.c_void_p * n)(*[y.data_ptr() for y in ys])
                LD = (ctypes.c_int64 * n)(*[y.stride(0) for y in ys])
                self._keep += [W, R, Y, LD]
                out.append((L.kq_gemv_multi, (t, n, W, R, spec.cols, x.data_ptr(), 1, x.stride(0), B, Y, LD, wsp, wsb,
                                               stream), spec.name))
            else:
                fn = getattr(L, {"q4k": "kq_gemv_q4k", "q5k": "kq_gemv_q5k", "q6k": "kq_gemv_q6k"}[spec.qtype])
                out.append((fn, (reps[0].data_ptr(), spec.rows, spec.cols, x.data_ptr(), 1, x.stride(0), B,
                                 ys[0].data_ptr(), ys[0].stride(0), wsp, wsb, stream), spec.name))
        return out


def step_stats(per_step_ms) -> dict:
    """Median, min and max of per-step times (ms)."""
    d = sorted(per_step_ms)
    return dict(median=round(d[len(d) // 2], 4), min=round(d[0], 4), max=round(d[-1], 4), n=len(d))


def timed_steps(run, steps: int, stream):
    """HIP events on `stream` around each of `steps` calls of run(): (mean ms, [ms per step])."""
    import torch
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    ev[0].record(stream)
    for i in range(steps):
        run()
        ev[i + 1].record(stream)
    torch.cuda.synchronize()
    per = [ev[i].elapsed_time(ev[i + 1]) for i in range(steps)]
    return ev[0].elapsed_time(ev[-1]) / steps, per


def time_chain(sw: Sweep, B: int, steps: int, warmup: int, per_step: dict = None, overlap: bool = False) -> float:
    """The whole sweep as one chain launch (step j+1 reads its x only after step j's y is complete);
    returns ms per step (per-step times in per_step['chain'] if given).  overlap: every step carries
    KQ_STEP_OVERLAP, so steps whose buffers are independent (every GEMV of the sweep has its own x and y)
    skip the step barrier and run back to back without it (key 'chain_overlap')."""
    torch, kq = sw.torch, sw.kq
    chain = kq.Chain([(spec.part_types() if spec.types else spec.qtype, reps, parts, spec.cols, sw.x[B][i], sw.y[B][i])
                      for i, (layer, spec, reps, parts) in enumerate(sw.entries)], B, overlap=overlap)
    if overlap and any(chain.waits()[1:]):
        raise RuntimeError("a step of the independent sweep waits at the step barrier")
    stream = torch.cuda.current_stream()
    for _ in range(warmup):
        chain.run(stream)
    torch.cuda.synchronize()
    ms, per = timed_steps(lambda: chain.run(stream), steps, stream)
    if chain.status() != 0:
        raise RuntimeError("a chain step's wait gave up: the chain timing is invalid")
    chain.close()
    if per_step is not None:
        per_step["chain_overlap" if overlap else "chain"] = step_stats(per)
    return ms


def time_gather(rows: int, cols: int, batches, reps: int = 64) -> dict:
    """Mean time of one embedding lookup (kq_gather_rows of `batch` token rows of a Q6_K rows x cols table),
    from HIP events around a graph of `reps` lookups."""
    import torch
    from quant_weight_streaming_amd import kq, synth
    g = synth.gen_weights("q6k", rows, cols, synth.seed_of("bench-emb"), device="cuda:0")
    w = kq.repack("q6k", g, rows, cols)
    del g
    out = {}
    for B in batches:
        ids = torch.randint(0, rows, (B,), dtype=torch.int32, device="cuda:0")
        o = torch.empty((B, cols), device="cuda:0")
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.stream(s):
            kq.kq_gather_rows("q6k", w, rows, cols, ids, o, s)
            with torch.cuda.graph(graph, stream=s):
                for _ in range(reps):
                    kq.kq_gather_rows("q6k", w, rows, cols, ids, o, s)
        torch.cuda.current_stream().wait_stream(s)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        graph.replay()
        e1.record()
        torch.cuda.synchronize()
        out[f"b{B}"] = round(e0.elapsed_time(e1) * 1e3 / reps, 2)
    return out


def time_swiglu(inter: int, cols: int, batches, copies: int = 6, reps: int = 4) -> dict:
    """Mean launch time of gate+up with the SwiGLU epilogue (kq_gemv_swiglu, Q4_K, one intermediate-size
    output), over `copies` distinct weight pairs so no launch reads another's weights from cache."""
    import torch
    from quant_weight_streaming_amd import kq, synth
    ws = []
    for i in range(copies):
        gate = synth.gen_weights("q4k", inter, cols, synth.seed_of("bench-swiglu", i, "gate"), device="cuda:0")
        up = synth.gen_weights("q4k", inter, cols, synth.seed_of("bench-swiglu", i, "up"), device="cuda:0")
        ws.append(kq.repack_swiglu("q4k", gate, up, inter, cols))
        del gate, up
    out = {}
    for B in batches:
        x = synth.gen_x(B, cols, synth.seed_of("bench-swiglu-x", B), device="cuda:0")
        y = torch.empty((B, inter), device="cuda:0")
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.stream(s):
            kq.kq_gemv_swiglu("q4k", ws[0], inter, cols, x, y, s)
            with torch.cuda.graph(graph, stream=s):
                for w in ws:
                    kq.kq_gemv_swiglu("q4k", w, inter, cols, x, y, s)
        torch.cuda.current_stream().wait_stream(s)
        graph.replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            graph.replay()
        e1.record()
        torch.cuda.synchronize()
        out[f"b{B}"] = round(e0.elapsed_time(e1) * 1e3 / (reps * copies), 2)
    return out


def time_fused(parts, cols: int, batches, variants, copies: int = 6, reps: int = 4) -> dict:
    """Mean launch time of one fused multi-projection launch (Q4_K, row segments `parts`) per variant
    (name -> (epilogue codes or None, rms_eps[, head_eps])), over `copies` distinct weight sets."""
    import torch
    from quant_weight_streaming_amd import kq, synth
    rows = sum(parts)
    sets = []
    for i in range(copies):
        g = synth.gen_weights("q4k", rows, cols, synth.seed_of("bench-fused", i), device="cuda:0")
        ws, r0 = [], 0
        for r in parts:
            ws.append(kq.repack("q4k", g[r0:r0 + r].contiguous(), r, cols))
            r0 += r
        sets.append(ws)
        del g
    out = {}
    for name, var in variants.items():
        epis, eps = var[0], var[1]
        heps = var[2] if len(var) > 2 else 0.0
        out[name] = {}
        for B in batches:
            x = synth.gen_x(B, cols, synth.seed_of("bench-fused-x", B), device="cuda:0")
            ys = [torch.zeros((B, r), device="cuda:0") for r in parts]
            s = torch.cuda.Stream()
            s.wait_stream(torch.cuda.current_stream())
            graph = torch.cuda.CUDAGraph()
            with torch.cuda.stream(s):
                kq.kq_gemv_fused("q4k", sets[0], list(parts), cols, x, ys, epis, eps, s, heps)
                with torch.cuda.graph(graph, stream=s):
                    for ws in sets:
                        kq.kq_gemv_fused("q4k", ws, list(parts), cols, x, ys, epis, eps, s, heps)
            torch.cuda.current_stream().wait_stream(s)
            graph.replay()
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(reps):
                graph.replay()
            e1.record()
            torch.cuda.synchronize()
            out[name][f"b{B}"] = round(e0.elapsed_time(e1) * 1e3 / (reps * copies), 2)
    return out


def time_decode_chain(batches, steps: int, warmup: int) -> dict:
    """A whole decode step as one chain in which every step reads what an earlier step wrote (fp32 activations),
    with the operations either side of each product fused into it: per layer, QKV reads the residual stream
    through the weight-less input RMSNorm and normalises the Q and K heads, O reads q (a stand-in for the attention
    output) and adds into the residual stream, gate+up reads the residual stream through the input norm and writes
    silu(gate) * up (one interleaved 62,464-row matrix), down adds into the residual stream; then the head through
    the input norm.  The first workload's shapes and types (52 layers, hidden 5,120, 18.03 GB of weights)."""
    import torch
    from quant_weight_streaming_amd import kq, synth
    H, Q, KV, I, V, L = synth.HIDDEN, 4096, 256, synth.INTER, synth.VOCAB, synth.N_LAYERS
    dev, hn = "cuda:0", kq.KQ_EPI_HEADNORM
    layers, nbytes = [], 0
    for li in range(L):
        g = synth.gen_weights("q4k", Q + 2 * KV, H, synth.seed_of("dec", li, "qkv"), device=dev)
        qkv = [kq.repack("q4k", g[a:b].contiguous(), b - a, H) for a, b in ((0, Q), (Q, Q + KV), (Q + KV, Q + 2 * KV))]
        o = kq.repack("q4k", synth.gen_weights("q4k", H, Q, synth.seed_of("dec", li, "o"), device=dev), H, Q)
        gate = synth.gen_weights("q4k", I, H, synth.seed_of("dec", li, "gate"), device=dev)
        up = synth.gen_weights("q4k", I, H, synth.seed_of("dec", li, "up"), device=dev)
        gu = kq.repack_swiglu("q4k", gate, up, I, H)
        del g, gate, up
        down = kq.repack("q6k", synth.gen_weights("q6k", H, I, synth.seed_of("dec", li, "down"), device=dev), H, I)
        layers.append((qkv, o, gu, down))
    head = kq.repack("q6k", synth.gen_weights("q6k", V, H, synth.seed_of("dec", "head"), device=dev), V, H)
    for spec in (synth.QKV, synth.O_PROJ, synth.GATE_UP, synth.DOWN):
        nbytes += L * spec.rows * spec.cols // 256 * synth.SB_BYTES[spec.qtype]
    nbytes += V * H // 256 * synth.SB_BYTES["q6k"]
    out = {"workload": "52 x {QKV + input RMSNorm + Q/K head norm, O + residual, gate+up + input RMSNorm + SwiGLU, "
                       "down + residual} + head + input RMSNorm, one chain; activations fp32 (the outputs) or bf16 "
                       "(the outputs' bf16 copies, the residual stream staying fp32)",
           "weight_bytes": nbytes}
    for act, B in [(a, b) for a in ("bf16", "f32") for b in batches]:
        r = torch.randn(B, H, device=dev)
        q, k, v = (torch.zeros(B, n, device=dev) for n in (Q, KV, KV))
        h, logits = torch.zeros(B, I, device=dev), torch.zeros(B, V, device=dev)
        st = []
        if act == "f32":
            for qkv, o, gu, down in layers:
                st += [("q4k", qkv, [Q, KV, KV], H, r, [q, k, v], hn | (hn << 4), 1e-5, 1e-6),
                       ("q4k", [o], [H], Q, q, [r], kq.KQ_EPI_RESIDUAL),
                       ("q4k", [gu], [I], H, r, [h], kq.KQ_EPI_SWIGLU, 1e-5),
                       ("q6k", [down], [H], I, h, [r], kq.KQ_EPI_RESIDUAL)]
            st.append(("q6k", [head], [V], H, r, [logits], kq.KQ_EPI_NONE, 1e-5))
        else:
            r16 = r.to(torch.bfloat16)
            q16 = torch.zeros(B, Q, dtype=torch.bfloat16, device=dev)
            h16 = torch.zeros(B, I, dtype=torch.bfloat16, device=dev)
            for qkv, o, gu, down in layers:
                st += [("q4k", qkv, [Q, KV, KV], H, r16, [q, k, v], hn | (hn << 4), 1e-5, 1e-6, [q16, None, None]),
                       ("q4k", [o], [H], Q, q16, [r], kq.KQ_EPI_RESIDUAL, 0.0, 0.0, [r16]),
                       ("q4k", [gu], [I], H, r16, [h], kq.KQ_EPI_SWIGLU, 1e-5, 0.0, [h16]),
                       ("q6k", [down], [H], I, h16, [r], kq.KQ_EPI_RESIDUAL, 0.0, 0.0, [r16])]
            st.append(("q6k", [head], [V], H, r16, [logits], kq.KQ_EPI_NONE, 1e-5))
        ch = kq.Chain(st, B)
        for _ in range(warmup):
            ch.run()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(steps):
            ch.run()
        e1.record()
        torch.cuda.synchronize()
        if ch.status() != 0:
            raise RuntimeError("a chain step's wait gave up: the decode-chain timing is invalid")
        ch.close()
        ms = e0.elapsed_time(e1) / steps
        out[f"{act}_b{B}"] = dict(ms=round(ms, 4), weight_gbs=round(nbytes / ms / 1e6, 1),
                                  tok_s=round(B * 1e3 / ms, 1))
    del layers, head
    torch.cuda.empty_cache()
    return out


def run_calls(calls):
    for fn, args, name in calls:
        rc = fn(*args)
        if rc:
            raise RuntimeError(f"{name}: GEMV launch failed with status {rc}")


def time_sweep(sw: Sweep, B: int, steps: int, warmup: int, per_step: dict = None):
    """Plain stream launches and hipGraph replay of the whole sweep; returns ms per step for both
    (per-step times in per_step['plain'] and per_step['graph'] if given)."""
    torch = sw.torch
    stream = torch.cuda.current_stream()
    calls = sw.calls(B, stream.cuda_stream)
    for _ in range(warmup):
        run_calls(calls)
    torch.cuda.synchronize()
    plain_ms, plain_per = timed_steps(lambda: run_calls(calls), steps, stream)
    ref = [[y.clone() for y in ys] for ys in sw.y[B]]

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run_calls(sw.calls(B, torch.cuda.current_stream().cuda_stream))
    for _ in range(warmup):
        g.replay()
    torch.cuda.synchronize()
    # every replay must reproduce the eager outputs bitwise (deterministic kernels)
    for i in (0, 1, 2, 3, len(ref) - 1):
        for y, r in zip(sw.y[B][i], ref[i]):
            if not torch.equal(y, r):
                raise RuntimeError(f"graph replay differs from eager launch (GEMV {i}, B={B})")
    torch.cuda.synchronize()
    graph_ms, graph_per = timed_steps(g.replay, steps, stream)
    del g
    if per_step is not None:
        per_step["plain"] = step_stats(plain_per)
        per_step["graph"] = step_stats(graph_per)
    return plain_ms, graph_ms


def kernel_time_in_sweep(sw: Sweep, B: int, name: str, reps: int = 9) -> float:
    """Mean cost (us) of one launch of class `name` as it runs inside the sweep: the replay time of the
    whole sweep's hipGraph minus that of the same graph without that class's launches, divided by the
    launches removed (HIP events on the launch stream; the two graphs replayed alternately, medians).
    The class's back-to-back graph (kernel_times) runs a launch right after another of the same shape,
    which is not how the sweep runs it."""
    import statistics
    torch = sw.torch
    stream = torch.cuda.current_stream()
    graphs = []
    for keep in (lambda c: True, lambda c: c[2] != name):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            run_calls([c for c in sw.calls(B, torch.cuda.current_stream().cuda_stream) if keep(c)])
        g.replay()
        graphs.append(g)
    torch.cuda.synchronize()
    n = sum(1 for c in sw.calls(B, stream.cuda_stream) if c[2] == name)
    times = ([], [])
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    for _ in range(reps):
        for k, g in enumerate(graphs):
            e0.record(stream)
            g.replay()
            e1.record(stream)
            torch.cuda.synchronize()
            times[k].append(e0.elapsed_time(e1))
    del graphs
    return (statistics.median(times[0]) - statistics.median(times[1])) / n * 1e3


def kernel_times(sw: Sweep, B: int, reps: int = 3):
    """Average launch duration per GEMV class, from HIP events on the launch stream around a hipGraph
    of all of that class's launches in the sweep (52 distinct weight tensors per layer class, so no
    launch re-reads another's weights from cache), replayed `reps` times: elapsed / launches."""
    torch = sw.torch
    stream = torch.cuda.current_stream()
    names = []
    for _, spec, _, _ in sw.entries:
        if spec.name not in names:
            names.append(spec.name)
    out = {}
    for name in names:
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            calls = [c for c in sw.calls(B, torch.cuda.current_stream().cuda_stream) if c[2] == name]
            run_calls(calls)
        g.replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        n_rep = max(reps, -(-26 // len(calls)))
        e0.record(stream)
        for _ in range(n_rep):
            g.replay()
        e1.record(stream)
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / (n_rep * len(calls))
        del g
        specs = [s for _, s, _, _ in sw.entries if s.name == name]
        spec = specs[0]
        wb = sum(s.weight_bytes() for s in specs) / len(specs)
        out[name] = dict(qtype=spec.qtype, rows=spec.rows, cols=spec.cols, launches=n_rep * len(calls),
                         avg_us=round(ms * 1e3, 2), weight_gbs=round(weight_gbs(wb, ms), 1),
                         weight_bytes=wb, x_bytes=B * spec.cols * 2, y_bytes=B * spec.rows * 4)
    return out


def host_info() -> dict:
    """The host CPU's model name (lscpu) and the cores this process may use."""
    import subprocess
    model = ""
    try:
        out = subprocess.run(["lscpu"], capture_output=True, text=True, timeout=20).stdout
        for line in out.splitlines():
            if line.lower().startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except Exception as e:          # no lscpu: say so in the record
        model = f"unknown ({type(e).__name__})"
    return dict(cpu_model=model, cores=len(os.sched_getaffinity(0)))


def smi_under_load(run, warm_s: float = 1.0, max_s: float = 6.0) -> dict:
    """GPU power and clocks read by amd-smi while run() keeps the GPU busy (an idle GPU reads its
    deep-sleep clocks): run() repeats for warm_s seconds, then amd-smi runs as a child process while run()
    keeps repeating until it returns."""
    import subprocess
    import torch
    t0 = time.time()
    while time.time() - t0 < warm_s:
        run()
        torch.cuda.synchronize()
    try:
        pr = subprocess.Popen(["amd-smi", "metric", "-p", "-c", "--json"], stdout=subprocess.PIPE,
                              stderr=subprocess.DEVNULL, text=True)
    except Exception as e:
        return dict(error=f"amd-smi not run: {type(e).__name__}")
    t0 = time.time()
    while pr.poll() is None and time.time() - t0 < max_s:
        run()
        torch.cuda.synchronize()
    try:
        out, _ = pr.communicate(timeout=30)
        d = json.loads(out)
        g = d["gpu_data"][0] if isinstance(d, dict) else d[0]
        gfx = [v["clk"]["value"] for k, v in g["clock"].items() if k.startswith("gfx_") and isinstance(v.get("clk"), dict)]
        return dict(power_w=g["power"]["socket_power"]["value"], gfx_mhz_mean=round(sum(gfx) / len(gfx), 1),
                    gfx_mhz_min=min(gfx), gfx_mhz_max=max(gfx), mem_mhz=g["clock"]["mem_0"]["clk"]["value"],
                    seconds_under_load=round(time.time() - t0, 2))
    except Exception as e:
        if pr.poll() is None:
            pr.kill()
        return dict(error=f"amd-smi output not read: {type(e).__name__}")


def read_ceiling(gib: int = 4, reps: int = 10) -> dict:
    """The achievable HBM read rate: kq_stream_read over `gib` GiB (far beyond the 256 MB Infinity
    Cache) with the GEMV's own loads, HIP events per read, median."""
    import torch
    from quant_weight_streaming_amd import kq
    buf = torch.empty(gib << 30, dtype=torch.uint8, device="cuda:0")
    sink = torch.zeros(1, dtype=torch.int32, device="cuda:0")
    stream = torch.cuda.current_stream()
    kq.kq_stream_read(buf, sink, stream)
    _, per = timed_steps(lambda: kq.kq_stream_read(buf, sink, stream), reps, stream)
    del buf
    med = sorted(per)[len(per) // 2]
    return dict(gbs=round((gib << 30) / med / 1e6, 1), best_gbs=round((gib << 30) / min(per) / 1e6, 1),
                bytes=gib << 30, median_ms=round(med, 4),
                how="kq_stream_read: every byte read once with 128-bit nontemporal buffer loads, 16 per "
                    "wavefront in flight, 16 workgroups of 4 wavefronts per CU; median of 10 reads")


def single_gemvs(sw: Sweep, kt1: dict, reps: int = 8) -> dict:
    """The three single-GEMV workloads: the small Q4_K 256x1024 GEMV with fp32 x (latency only: it fits in
    cache), gate+up alone over rotated weight copies, and the head alone over two rotated copies (so no
    launch finds its weights in the 256 MB Infinity Cache)."""
    import statistics
    torch, kq, synth = sw.torch, sw.kq, sw.synth
    stream = torch.cuda.current_stream()
    out = {}
    # config 0: latency of one launch, eager (launch overhead included) and inside a graph of 100
    c0 = synth.CONFIGS[0]["gemv"]
    g = synth.gen_weights("q4k", c0.rows, c0.cols, 0, device="cuda:0")
    w0 = kq.repack("q4k", g, c0.rows, c0.cols)
    x0 = synth.gen_x(1, c0.cols, 0, "f32", device="cuda:0")
    y0 = torch.empty((1, c0.rows), device="cuda:0")
    for _ in range(10):
        kq.gemv("q4k", w0, c0.rows, c0.cols, x0, y0, stream, sw.work)
    torch.cuda.synchronize()
    _, eager = timed_steps(lambda: kq.gemv("q4k", w0, c0.rows, c0.cols, x0, y0, stream, sw.work), 50, stream)
    gr = torch.cuda.CUDAGraph()
    with torch.cuda.graph(gr):
        for _ in range(100):
            kq.gemv("q4k", w0, c0.rows, c0.cols, x0, y0, torch.cuda.current_stream(), sw.work)
    gr.replay()
    torch.cuda.synchronize()
    _, per = timed_steps(gr.replay, 5, stream)
    out["c0_q4k_256x1024_b1_f32"] = dict(
        eager_us=dict(median=round(statistics.median(eager) * 1e3, 2), min=round(min(eager) * 1e3, 2),
                      max=round(max(eager) * 1e3, 2)),
        in_graph_us=round(statistics.median(per) * 1e3 / 100, 2),
        note="147,456 weight bytes: latency only, the matrix sits in cache")
    del gr
    # config 1: gate+up alone, 52 distinct weight copies back to back (the sweep's class graph)
    gu = kt1["gate_up"]
    out["c1_gate_up_q4k_62464x5120_b1"] = dict(avg_us=gu["avg_us"], weight_gbs=gu["weight_gbs"],
                                               pct_of_hbm_peak=round(100 * gu["weight_gbs"] / HBM_PEAK_GBS, 2),
                                               rotated_copies=52, launches=gu["launches"])
    # config 2: the head alone, two copies alternating
    head = [e for e in sw.entries if e[1].name == "head"][0]
    spec, reps0 = head[1], head[2]
    g2 = synth.gen_weights("q6k", spec.rows, spec.cols, synth.seed_of("bench-head-copy"), device="cuda:0")
    w2 = kq.repack("q6k", g2, spec.rows, spec.cols)
    del g2
    xh = synth.gen_x(1, spec.cols, 7, device="cuda:0")
    yh = torch.empty((1, spec.rows), device="cuda:0")
    copies = [reps0[0], w2]
    gr = torch.cuda.CUDAGraph()
    with torch.cuda.graph(gr):
        for i in range(2 * reps):
            kq.gemv("q6k", copies[i % 2], spec.rows, spec.cols, xh, yh, torch.cuda.current_stream(), sw.work)
    gr.replay()
    torch.cuda.synchronize()
    _, per = timed_steps(gr.replay, 3, stream)
    us = statistics.median(per) * 1e3 / (2 * reps)
    wb = spec.rows * spec.cols // 256 * 210
    out["c2_head_q6k_131072x5120_b1"] = dict(avg_us=round(us, 2), weight_gbs=round(wb / us / 1e3, 1),
                                             pct_of_hbm_peak=round(100 * wb / us / 1e3 / HBM_PEAK_GBS, 2),
                                             rotated_copies=2, launches=2 * reps * 3)
    del gr, w2
    torch.cuda.empty_cache()
    return out


def oracle_one_thread(frac1: float = 0.01, frac2: float = 0.005) -> dict:
    """The C oracle on ONE thread for the three single-GEMV workloads: the whole small GEMV, and the first
    rows of gate+up and of the head (fraction frac1 / frac2), extrapolated by rows to the whole GEMV (the
    oracle's time is linear in rows)."""
    import numpy as np
    import torch
    from oracle import oracle as O
    from quant_weight_streaming_amd import synth
    Or = O.default()
    try:
        gomp = ctypes.CDLL("libgomp.so.1")
        prev = gomp.omp_get_max_threads()
        gomp.omp_set_num_threads(1)
    except OSError:
        return dict(error="libgomp not found: thread count not set")
    out = {}
    try:
        for key, spec, xd, frac in (("c0_q4k_256x1024_b1_f32", synth.CONFIGS[0]["gemv"], "f32", 1.0),
                                    ("c1_gate_up_q4k_62464x5120_b1", synth.GATE_UP, "bf16", frac1),
                                    ("c2_head_q6k_131072x5120_b1", synth.HEAD, "bf16", frac2)):
            rs = max(1, int(round(spec.rows * frac)))
            g = synth.gen_weights(spec.qtype, rs, spec.cols, synth.seed_of("oracle-1t", key)).numpy()
            x = synth.gen_x(1, spec.cols, 3, xd)
            xh = x.numpy() if xd == "f32" else x.view(torch.int16).numpy().view(np.uint16)
            t = time.perf_counter()
            Or.gemv(spec.qtype, rs, spec.cols, g, xh)
            dt = time.perf_counter() - t
            full = dt * spec.rows / rs
            wb = spec.rows * spec.cols // 256 * synth.SB_BYTES[spec.qtype]
            out[key] = dict(rows_timed=rs, seconds_timed=round(dt, 4), seconds_whole_gemv=round(full, 4),
                            weight_gbs=round(wb / full / 1e9, 4))
    finally:
        gomp.omp_set_num_threads(prev)
    out["threads"] = 1
    return out


def profile_roofline() -> dict:
    """The roofline kernel's mean duration inside the sweep from the committed rocprofv3 kernel-trace summary,
    if it was taken of the current kernels."""
    p = os.path.join(ROOT, "profiles", "gemv_sweep52_kernel_trace.txt")
    if not os.path.exists(p):
        return None
    txt = open(p).read()
    m = re.search(r"kernel hash: ([0-9a-f]+)", txt)
    if not m or m.group(1) != kernel_source_hash():
        return None
    m = re.search(r"after another GEMV \(the sweep\)\s+(\d+) dispatches, mean\s+([0-9.]+)", txt)
    return dict(avg_launch_us=float(m.group(2)), dispatches=int(m.group(1))) if m else None


def cpu_baseline(sw: Sweep, frac: float):
    """The CPU oracle on the sampled rows of every sweep tensor, batch 1 (compute time only)."""
    from oracle import oracle as O
    import numpy as np
    torch = sw.torch
    Or = O.default()
    total_s, total_bytes = 0.0, 0
    for (qtype, rs, cols, g, layer, name), xs in zip(sw.samples, sw.x[1]):
        x = xs.cpu().contiguous().view(torch.int16).numpy().view(np.uint16)
        t = time.perf_counter()
        Or.gemv(qtype, rs, cols, g, x)
        total_s += time.perf_counter() - t
        total_bytes += g.nbytes
    try:
        threads = int(Or.L.omp_get_max_threads())
    except Exception:
        threads = int(os.environ.get("OMP_NUM_THREADS", len(os.sched_getaffinity(0))))
    gbs = total_bytes / total_s / 1e9
    return dict(value=round(gbs, 3), unit="GB/s", cores=threads, kind="oracle",
                sample=(f"first {frac:.3f} of the rows of each of the 209 sweep tensors at batch 1 "
                        f"({total_bytes} of {sw.weight_bytes} weight bytes), fp64 C oracle, {total_s:.1f} s"),
                seconds=round(total_s, 2), decode_equiv_tok_s=round(gbs * 1e9 / sw.weight_bytes, 3))


def oracle_rate_probe() -> float:
    """Weight GB/s of the CPU oracle on a small Q4_K + Q6_K probe (sizes the baseline sample)."""
    from oracle import oracle as O
    from quant_weight_streaming_amd import synth
    import numpy as np
    import torch
    t, nb = 0.0, 0
    for qt, rows, cols in (("q4k", 1024, 5120), ("q6k", 128, 31232)):
        g = synth.gen_weights(qt, rows, cols, 5).numpy()
        x = synth.gen_x(1, cols, 6).view(torch.int16).numpy().view(np.uint16)
        s = time.perf_counter()
        O.gemv(qt, rows, cols, g, x)
        t += time.perf_counter() - s
        nb += g.nbytes
    return nb / t / 1e9


def load_traffic(name: str):
    """Measured HBM bytes per launch from a committed rocprofv3 counter summary, if it matches these kernels."""
    p = os.path.join(ROOT, "profiles", f"{name}.json")
    if not os.path.exists(p):
        return None
    d = json.load(open(p))
    if d.get("kernel_hash") != kernel_source_hash():
        return None
    return d.get("hbm_bytes_per_launch")


def profile_kernel(n: int, batch: int = 1):
    """Only the dominant kernel (gate+up Q4_K, batch 1 unless asked otherwise): n launches over 8
    distinct weight copies."""
    import torch
    from quant_weight_streaming_amd import kq, synth
    spec = synth.GATE_UP
    kq.kq_init(0)
    copies = []
    for i in range(8):
        g = synth.gen_weights("q4k", spec.rows, spec.cols, synth.seed_of("prof", i), device="cuda:0")
        copies.append([kq.repack("q4k", g[:spec.parts[0]].contiguous(), spec.parts[0], spec.cols),
                       kq.repack("q4k", g[spec.parts[0]:].contiguous(), spec.parts[1], spec.cols)])
        del g
    x = synth.gen_x(batch, spec.cols, 1, device="cuda:0")
    ys = [torch.empty((batch, r), device="cuda:0") for r in spec.parts]
    for i in range(n):
        kq.kq_gemv_multi("q4k", copies[i % 8], list(spec.parts), spec.cols, x, ys)
    torch.cuda.synchronize()
    log(f"[bench] profile-kernel: {n} launches at batch {batch} done")


def copy_calibration(n: int):
    import torch
    a = torch.empty(1 << 30, dtype=torch.uint8, device="cuda:0").fill_(1)
    b = torch.empty_like(a)
    for _ in range(n):
        b.copy_(a)
    torch.cuda.synchronize()
    log(f"[bench] copy-calibration: {n} copies of {1 << 30} bytes")


def summarize_trace(src: str, cmd: str) -> str:
    """Text summary of a rocprofv3 --kernel-trace --stats run of this benchmark: the GEMV rows of the
    stats table, then every GEMV dispatch grouped by (kernel, grid) and named by sweep class (each timed
    sweep issues the 209 GEMVs in sweep order, so a key's first dispatch falls at its sweep position)."""
    import csv
    from quant_weight_streaming_amd import synth
    stats = [r for r in csv.DictReader(open(glob.glob(os.path.join(src, "*_kernel_stats.csv"))[0]))
             if "kq::" in r["Name"]]
    trace = [r for r in csv.DictReader(open(glob.glob(os.path.join(src, "*_kernel_trace.csv"))[0]))
             if "kq::gemv_kernel" in r["Kernel_Name"]]
    trace.sort(key=lambda r: int(r["Start_Timestamp"]))
    order = [spec.name for _, spec in synth.sweep("q4k")]
    groups, label = {}, {}
    for i, r in enumerate(trace):
        key = (r["Kernel_Name"].split("(")[0].replace("void ", ""), int(r["Grid_Size_X"]) // int(r["Workgroup_Size_X"]))
        if key not in label:
            label[key] = order[i % len(order)]
        groups.setdefault(key, []).append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
    out = [f"command: {cmd}", f"kernel hash: {kernel_source_hash()}", "",
           "rocprofv3 kernel stats (kq kernels; durations in us):",
           f"{'kernel':44s} {'calls':>6s} {'avg':>9s} {'min':>9s} {'max':>9s}"]
    for r in stats:
        out.append(f"{r['Name'].split('(')[0].replace('void ', ''):44s} {int(r['Calls']):6d} "
                   f"{float(r['AverageNs']) / 1e3:9.2f} {float(r['MinNs']) / 1e3:9.2f} {float(r['MaxNs']) / 1e3:9.2f}")
    out += ["", "GEMV dispatches by kernel and grid (from the kernel trace; durations in us):",
            f"{'kernel':36s} {'workgroups':>10s} {'class':>8s} {'calls':>6s} {'avg':>9s} {'median':>9s} {'min':>9s} {'max':>9s}"]
    for key, d in sorted(groups.items(), key=lambda kv: (kv[0][0], kv[0][1])):
        d = sorted(d)
        out.append(f"{key[0]:36s} {key[1]:10d} {label[key]:>8s} {len(d):6d} {sum(d) / len(d):9.2f} "
                   f"{d[len(d) // 2]:9.2f} {d[0]:9.2f} {d[-1]:9.2f}")
    # the roofline kernel (gate+up at batch 1: the batch-1 Q4_K kernel on gate+up's grid), split by what ran
    # just before a dispatch: another kernel (as in the sweep) or a gate+up (the back-to-back class graph)
    keys = [k for k, v in label.items() if v == "gate_up" and k[0].startswith("kq::gemv_kernel<1, 1, false")]
    if keys:
        gk = max(keys, key=lambda k: len(groups[k]))
        split = {True: [], False: []}
        prev = None
        for r in trace:
            key = (r["Kernel_Name"].split("(")[0].replace("void ", ""), int(r["Grid_Size_X"]) // int(r["Workgroup_Size_X"]))
            if key == gk:
                split[prev == gk].append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
            prev = key
        out += ["", f"gate+up at batch 1 ({gk[0]}, {gk[1]} workgroups), by what ran before it (durations in us).",
                "This is the roofline kernel: bench.py's roofline.avg_launch_us is its cost inside the sweep. The",
                "stats line above averages every launch of the template (QKV, O and gate+up alike)."]
        for b2b, name in ((False, "after another GEMV (the sweep)"), (True, "after another gate+up (class graph)")):
            d = sorted(split[b2b])
            if d:
                out.append(f"  {name:38s} {len(d):6d} dispatches, mean {sum(d) / len(d):7.2f}, median {d[len(d) // 2]:7.2f}")
    return "\n".join(out) + "\n"


def summarize_counters(kfetch: str, kwrite: str, cfetch: str, cwrite: str) -> dict:
    """HBM bytes per launch of the dominant GEMV from FETCH_SIZE / WRITE_SIZE passes (KiB per dispatch),
    each scaled by what the same counter reads for a plain 1 GiB device copy."""
    import csv

    def rows(d, pred):
        f = glob.glob(os.path.join(d, "*_counter_collection.csv"))[0]
        return [float(r["Counter_Value"]) for r in csv.DictReader(open(f)) if pred(r)]
    gemv = lambda r: "kq::gemv_kernel" in r["Kernel_Name"]
    copy = lambda r: "copyBuffer" in r["Kernel_Name"]
    kf, kw = rows(kfetch, gemv), rows(kwrite, gemv)
    cf, cw = rows(cfetch, copy), rows(cwrite, copy)
    gib_kib = float(1 << 20)
    f_fac, w_fac = gib_kib / (sum(cf) / len(cf)), gib_kib / (sum(cw) / len(cw))
    fetch_b = sum(kf) / len(kf) * 1024 * f_fac
    write_b = sum(kw) / len(kw) * 1024 * w_fac
    return dict(kernel_hash=kernel_source_hash(), dispatches=len(kf),
                fetch_kib_per_dispatch=sum(kf) / len(kf), write_kib_per_dispatch=sum(kw) / len(kw),
                copy_1gib_fetch_kib=sum(cf) / len(cf), copy_1gib_write_kib=sum(cw) / len(cw),
                fetch_scale=f_fac, write_scale=w_fac,
                hbm_fetch_bytes_per_launch=round(fetch_b), hbm_write_bytes_per_launch=round(write_b),
                hbm_bytes_per_launch=round(fetch_b + write_b))


def summarize_pmc(dirs: list) -> str:
    """Per-dispatch means of every counter of the GEMV dispatches in rocprofv3 --pmc runs (one column per
    run directory), plus the VALU issue floor: wavefront VALU instructions / (CUs x 1 per clock)."""
    import csv
    cols, names = [], set()
    for d in dirs:
        f = glob.glob(os.path.join(d, "*_counter_collection.csv"))[0]
        per, kname = {}, ""
        for r in csv.DictReader(open(f)):
            if "kq::gemv_kernel" not in r["Kernel_Name"]:
                continue
            kname = r["Kernel_Name"].split("(")[0].replace("void ", "")
            key = (r["Dispatch_Id"], r["Counter_Name"])
            per[key] = per.get(key, 0.0) + float(r["Counter_Value"])
        by = {}
        for (_, c), v in per.items():
            by.setdefault(c, []).append(v)
        cols.append((d, kname, {c: sum(v) / len(v) for c, v in by.items()}))
        names |= set(by)
    out = [f"{'counter':28s}" + "".join(f" {os.path.basename(d.rstrip('/')):>22s}" for d, _, _ in cols)]
    out.append(f"{'kernel':28s}" + "".join(f" {k.replace('kq::gemv_kernel', 'gemv'):>22s}" for _, k, _ in cols))
    for c in sorted(names):
        out.append(f"{c:28s}" + "".join(f" {m.get(c, float('nan')):22.0f}" for _, _, m in cols))
    cus = 256
    for ghz in (2.1, 2.4):
        out.append(f"{'VALU floor us @' + str(ghz) + ' GHz':28s}" +
                   "".join(f" {m.get('SQ_INSTS_VALU', 0) / cus / (ghz * 1e3):22.2f}" for _, _, m in cols))
    return "\n".join(out) + "\n"


def timeline_report(batches, runs: int = 3) -> str:
    """Per-step timeline of the B = 1 / B = 8 chain sweeps from libkq_timeline.so (the -DKQ_TIMELINE build, see
    include/kq_timeline.h): per projection class, medians over the 52 layers of where each step's time goes."""
    import ctypes
    import numpy as np
    import torch
    from quant_weight_streaming_amd import kq
    kq.LIB_PATH = os.path.join(ROOT, "quant_weight_streaming_amd", "libkq_timeline.so")
    kq._lib = None
    L = kq.lib()
    L.kq_chain_timeline.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t,
                                    ctypes.POINTER(ctypes.c_int), ctypes.POINTER(ctypes.c_int)]
    L.kq_chain_timeline.restype = ctypes.c_int
    kq.kq_init(0)
    sw = Sweep(3, "q4k", batches, 0.0, 0.0)
    names = [spec.name for (_, spec, _, _) in sw.entries]
    out = ["Per-step timeline of the chain sweep (52 x {QKV, O, gate+up, down} + head, Q4_K / Q6_K, bf16 x):",
           "device clock stamps (100 MHz) of every workgroup at six points of every step, last of "
           f"{runs} runs after warm-up.",
           "Per class, medians over the 52 layers of: span = last arrival of the step - last arrival of the",
           "step before; release = a workgroup's exit from the barrier wait - the previous step's last arrival",
           "(median / max over workgroups); stage, main, tail = staging, main loop, tile writes and hand-off",
           "(median over workgroups; main also max); drain = last arrival - slowest main loop end.", ""]
    for B in batches:
        chain = kq.Chain([(spec.part_types() if spec.types else spec.qtype, reps, parts, spec.cols, sw.x[B][i],
                           sw.y[B][i]) for i, (layer, spec, reps, parts) in enumerate(sw.entries)], B)
        s = torch.cuda.current_stream()
        for _ in range(3):
            chain.run(s)
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        ms = []
        for _ in range(runs):
            ev[0].record(s)
            chain.run(s)
            ev[1].record(s)
            torch.cuda.synchronize()
            ms.append(ev[0].elapsed_time(ev[1]))
        if chain.status() != 0:
            raise RuntimeError("a chain wait gave up during the timeline run")
        buf = np.zeros((len(names) + 8) * 256 * 8 * 4, dtype=np.uint64)
        g, n = ctypes.c_int(), ctypes.c_int()
        rc = L.kq_chain_timeline(ctypes.c_void_p(chain.handle), buf.ctypes.data, buf.nbytes, ctypes.byref(g),
                                 ctypes.byref(n))
        if rc != 0:
            raise RuntimeError(f"kq_chain_timeline failed: {rc}")
        G, N = g.value, n.value
        t = buf[:N * G * 8].reshape(N, G, 8).astype(np.int64)
        chain.close()
        xcc = t[0, :, 6].copy()
        us = (t[:, :, :6] - t[0, :, 0].min()) * 0.01
        act = t[:, :, 1] > 0
        rows = {}
        prev_end = us[0, :, 0].min()
        for j in range(N):
            v = act[j]
            r = us[j]
            end = r[:, 5].max()
            rel = r[v, 1] - prev_end
            main = r[v, 3] - r[v, 2]
            d = dict(span=end - prev_end, rel_med=np.median(rel), rel_max=rel.max(),
                     stage=np.median(r[v, 2] - r[v, 1]), main_med=np.median(main), main_max=main.max(),
                     tail=np.median(r[v, 4] - r[v, 3]), drain=end - r[v, 3].max(), groups=int(v.sum()))
            rows.setdefault(names[j] if j < len(names) else "?", []).append(d)
            prev_end = end
        out.append(f"batch {B}: chain run {np.median(ms):.3f} ms (event timing of the timeline build), "
                   f"{G} workgroups, {N} steps")
        out.append(f"  {'class':8s} {'steps':>5s} {'groups':>6s} {'span':>7s} {'rel med':>8s} {'rel max':>8s} "
                   f"{'stage':>7s} {'main med':>9s} {'main max':>9s} {'tail':>6s} {'drain':>6s}   (us)")
        for name, ds in rows.items():
            med = {k: float(np.median([d[k] for d in ds])) for k in ds[0]}
            out.append(f"  {name:8s} {len(ds):5d} {int(med['groups']):6d} {med['span']:7.2f} {med['rel_med']:8.2f} "
                       f"{med['rel_max']:8.2f} {med['stage']:7.2f} {med['main_med']:9.2f} {med['main_max']:9.2f} "
                       f"{med['tail']:6.2f} {med['drain']:6.2f}")
        tot = sum(float(np.sum([d["span"] for d in ds])) for ds in rows.values())
        out.append(f"  sum of spans {tot / 1e3:.3f} ms; per layer "
                   + ", ".join(f"{k} {np.median([d['span'] for d in ds]):.2f}" for k, ds in rows.items() if len(ds) > 1)
                   + " us")
        # main-loop time of each workgroup relative to its step's median, averaged over the big steps, by XCC
        big = [j for j in range(N) if j < len(names) and names[j] in ("gate_up", "down")]
        relm = []
        for j in big:
            v = act[j]
            m = us[j, :, 3] - us[j, :, 2]
            relm.append(np.where(v, m / np.median(m[v]), np.nan))
        relm = np.array(relm)
        per_xcc = [relm[:, xcc == x] for x in range(8)]
        out.append("  gate+up and down main loop relative to the step median, mean per XCC: "
                   + " ".join(f"{x}:{np.nanmean(m):.3f}" for x, m in enumerate(per_xcc) if np.isfinite(m).any()))
        out.append("")
    return "\n".join(out) + "\n"


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--no-c4", action="store_true", help="skip the Q5_K / merged-sub-block sweep")
    ap.add_argument("--no-p4", action="store_true", help="skip the 6656-hidden decoder's sweep")
    ap.add_argument("--no-q4km", action="store_true", help="skip the Q4_K_M-style mixed-type sweep")
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="target CPU work of the oracle sample")
    ap.add_argument("--profile-kernel", type=int, default=0)
    ap.add_argument("--profile-batch", type=int, default=1, help="batch of the --profile-kernel launches")
    ap.add_argument("--copy-calibration", type=int, default=0, help="N plain 1 GiB device copies")
    ap.add_argument("--summarize-trace", nargs=2, metavar=("ROCPROF_DIR", "COMMAND"),
                    help="print a text summary of a rocprofv3 kernel-trace run of this benchmark")
    ap.add_argument("--summarize-counters", nargs=4, metavar=("GEMV_FETCH", "GEMV_WRITE", "COPY_FETCH", "COPY_WRITE"),
                    help="print the HBM-traffic JSON of the dominant kernel from four rocprofv3 --pmc runs")
    ap.add_argument("--summarize-pmc", nargs="+", metavar="ROCPROF_DIR",
                    help="print per-dispatch counter means of the GEMV dispatches of rocprofv3 --pmc runs")
    ap.add_argument("--timeline", action="store_true",
                    help="print the per-step timeline of the B=1 and B=8 chain sweeps (needs libkq_timeline.so)")
    args = ap.parse_args()
    if args.summarize_pmc:
        sys.stdout.write(summarize_pmc(args.summarize_pmc))
        return
    if args.summarize_trace:
        sys.path.insert(0, ROOT)
        sys.stdout.write(summarize_trace(*args.summarize_trace))
        return
    if args.summarize_counters:
        print(json.dumps(summarize_counters(*args.summarize_counters), indent=1))
        return
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only (--gpus {args.gpus}, WORLD_SIZE {world}): the K-quant GEMV path "
              f"is built and timed on a single MI355X; multi-GPU sharding is a design note, not a run.",
              file=sys.stderr)
        sys.exit(2)
    sys.path.insert(0, ROOT)
    if args.profile_kernel:
        return profile_kernel(args.profile_kernel, args.profile_batch)
    if args.copy_calibration:
        return copy_calibration(args.copy_calibration)
    if args.timeline:
        sys.stdout.write(timeline_report((1, 8)))
        return

    import torch
    from quant_weight_streaming_amd import kq, synth
    kq.lib()                       # fails loudly if the HIP library is not built
    kq.kq_init(0)

    frac = 0.0
    if not args.no_cpu:
        rate = oracle_rate_probe()
        frac = min(1.0, args.cpu_seconds * rate * 1e9 / synth.sweep_bytes("q4k"))
        log(f"[bench] oracle probe {rate:.3f} GB/s -> sample fraction {frac:.3f}")

    VERIFY = (2, 3, 4, 12, 16)     # speculative-verify block sizes for the cost staircase
    host = host_info()
    sw = Sweep(3, "q4k", (1, 8) + VERIFY, 0.0, frac)
    # clocks and power under load, before the timed work (an idle GPU shows its deep-sleep clocks)
    smi_chain = sw.kq.Chain([(spec.qtype, reps, parts, spec.cols, sw.x[1][i], sw.y[1][i])
                             for i, (layer, spec, reps, parts) in enumerate(sw.entries)], 1)
    smi_before = smi_under_load(smi_chain.run)
    log(f"[bench] amd-smi under load before timing: {smi_before}")
    res, per_step = {}, {}
    for B in (1, 8):
        per_step[B] = {}
        plain, graph = time_sweep(sw, B, args.steps, args.warmup, per_step[B])
        chain = time_chain(sw, B, args.steps, args.warmup, per_step[B])
        overlap = time_chain(sw, B, args.steps, args.warmup, per_step[B], overlap=True)
        res[B] = dict(plain_ms=plain, graph_ms=graph, chain_ms=chain, overlap_ms=overlap)
        log(f"[bench] cfg3 B={B}: plain {plain:.3f} ms ({sw.weight_bytes / plain / 1e6:.0f} GB/s), "
            f"graph {graph:.3f} ms ({sw.weight_bytes / graph / 1e6:.0f} GB/s), "
            f"chain {chain:.3f} ms ({sw.weight_bytes / chain / 1e6:.0f} GB/s), "
            f"chain without barriers between independent GEMVs {overlap:.3f} ms "
            f"({sw.weight_bytes / overlap / 1e6:.0f} GB/s)")
    # verify cost: the sweep at S rows per call (a speculative block verified in one forward)
    for B in VERIFY:
        plain, graph = time_sweep(sw, B, max(3, args.steps // 2), args.warmup)
        chain = time_chain(sw, B, max(3, args.steps // 2), args.warmup)
        res[B] = dict(plain_ms=plain, graph_ms=graph, chain_ms=chain)
    stair = {}
    t1 = min(res[1]["graph_ms"], res[1]["chain_ms"])
    for B in sorted(res):
        t = min(res[B]["graph_ms"], res[B]["chain_ms"])
        stair[str(B)] = dict(ms=round(t, 4), vs_one_row=round(t / t1, 3), rows_per_s=round(tok_s(t, B), 1))
    log("[bench] verify cost (sweep time at S rows / at 1 row): " +
        ", ".join(f"S={k}: {v['vs_one_row']}x" for k, v in stair.items()))
    kt1 = kernel_times(sw, 1)
    kt8 = kernel_times(sw, 8)
    gu_in_sweep_us = kernel_time_in_sweep(sw, 1, "gate_up")
    singles = single_gemvs(sw, kt1)
    log(f"[bench] single GEMVs: {singles}")
    smi_after = smi_under_load(smi_chain.run)
    smi_chain.close()
    log(f"[bench] amd-smi under load after timing: {smi_after}")
    ceiling = read_ceiling()
    log(f"[bench] read ceiling: {ceiling['gbs']} GB/s")
    if not args.no_cpu:
        singles["oracle_one_thread"] = oracle_one_thread()
        log(f"[bench] oracle on one thread: {singles['oracle_one_thread']}")
    cpu = cpu_baseline(sw, frac) if not args.no_cpu else None
    swiglu_us = time_swiglu(synth.INTER, synth.HIDDEN, (1, 8))
    decode = time_decode_chain((1, 8), max(3, args.steps // 2), args.warmup)
    log(f"[bench] fused decode chain (norms, SwiGLU, residuals): "
        + ", ".join(f"{b} {v['ms']:.3f} ms ({v['weight_gbs']:.0f} GB/s)" for b, v in decode.items()
                    if isinstance(v, dict)))
    qkvg = synth.QKVG_P4
    fused_us = time_fused(qkvg.parts, qkvg.cols, (1, 8), {
        "plain": (None, 0.0),
        "rmsnorm_and_sigmoid_gate": ([kq.KQ_EPI_NONE] * 3 + [kq.KQ_EPI_SIGMOID], 1e-5),
        "rmsnorm_qk_head_norm_sigmoid_gate": ([kq.KQ_EPI_HEADNORM] * 2 + [kq.KQ_EPI_NONE, kq.KQ_EPI_SIGMOID],
                                              1e-5, 1e-6)})
    log(f"[bench] fused QKVG 8704x6656: {fused_us} us")
    log(f"[bench] gate+up with SwiGLU epilogue (Q4_K 2 x {synth.INTER}x{synth.HIDDEN}): {swiglu_us} us "
        f"(plain gate+up: {kt1['gate_up']['avg_us']} / {kt8['gate_up']['avg_us']} us)")
    if cpu:
        cpu["cpu_model"] = host["cpu_model"]
        log(f"[bench] cpu oracle: {cpu['value']} GB/s on {cpu['cores']} threads over {cpu['seconds']} s")

    # roofline of the dominant kernel (gate+up, batch 1): algorithmic bytes per launch / the mean cost of
    # one of its launches inside the sweep's graph; its back-to-back class graph time beside it
    gu = kt1["gate_up"]
    alg = gu["weight_bytes"] + gu["x_bytes"] + gu["y_bytes"]
    achieved = alg / (gu_in_sweep_us * 1e-6) / 1e9
    prof = profile_roofline()
    roofline = dict(bound="hbm", achieved=round(achieved, 1), peak=HBM_PEAK_GBS, unit="GB/s",
                    frac=round(achieved / HBM_PEAK_GBS, 4), traffic=load_traffic("gate_up_q4k_b1_traffic"),
                    kernel="gemv_kernel<Q4_K, B=1, bf16> (gate+up 62464x5120, one launch over both halves)",
                    algorithmic_bytes_per_launch=alg, avg_launch_us=round(gu_in_sweep_us, 2),
                    timing="sweep graph minus the same graph without the 52 gate+up launches, per launch "
                           "(HIP events, medians of 9 alternated replays)",
                    avg_launch_us_back_to_back=gu["avg_us"],
                    read_ceiling_gbs=ceiling["gbs"], frac_of_read_ceiling=round(achieved / ceiling["gbs"], 4),
                    profile=(dict(avg_launch_us=prof["avg_launch_us"], dispatches=prof["dispatches"],
                                  achieved=round(alg / (prof["avg_launch_us"] * 1e-6) / 1e9, 1),
                                  frac=round(alg / (prof["avg_launch_us"] * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
                                  source="profiles/gemv_sweep52_kernel_trace.txt (rocprofv3 kernel trace, gate+up "
                                         "dispatches that follow another GEMV)")
                             if prof else None))

    c4 = None
    if not args.no_c4:
        bytes3 = sw.weight_bytes
        del sw
        torch.cuda.empty_cache()
        sw4 = Sweep(4, "q5k", (2, 4, 8), 0.25, 0.0)
        c4 = {}
        for B in (2, 4, 8):
            plain, graph = time_sweep(sw4, B, max(3, args.steps // 2), args.warmup)
            chain = time_chain(sw4, B, max(3, args.steps // 2), args.warmup)
            best = min(graph, chain)
            c4[f"b{B}"] = dict(graph_ms=round(graph, 4), plain_ms=round(plain, 4), chain_ms=round(chain, 4),
                               weight_gbs=round(weight_gbs(sw4.weight_bytes, best), 1),
                               pct_of_hbm_peak=round(100 * weight_gbs(sw4.weight_bytes, best) / HBM_PEAK_GBS, 2),
                               tok_s=round(tok_s(best, B), 1))
            log(f"[bench] cfg4 B={B}: graph {graph:.3f} ms, chain {chain:.3f} ms "
                f"({sw4.weight_bytes / best / 1e6:.0f} GB/s)")
        c4["weight_bytes"] = sw4.weight_bytes
        c4["kernels_b8"] = kernel_times(sw4, 8)
        del sw4
        sw = None
    else:
        bytes3 = sw.weight_bytes

    # the 6656-hidden decoder of the Core AI card (its own sweep; not the headline workload)
    p4 = None
    if not args.no_p4:
        sw = None
        torch.cuda.empty_cache()
        swp = Sweep("p4", "q4k", (1, 8), 0.0, 0.0, entries=synth.sweep_p4())
        p4 = {"workload": "52 x {QKVG Q4_K 8704x6656, O Q4_K 6656x4096, gate+up Q4_K 39936x6656, down Q6_K "
                          "6656x19968} + head Q6_K 202048x6656", "weight_bytes": swp.weight_bytes}
        for B in (1, 8):
            plain, graph = time_sweep(swp, B, max(3, args.steps // 2), args.warmup)
            chain = time_chain(swp, B, max(3, args.steps // 2), args.warmup)
            best = min(graph, chain)
            p4[f"b{B}"] = dict(graph_ms=round(graph, 4), chain_ms=round(chain, 4), plain_ms=round(plain, 4),
                               weight_gbs=round(weight_gbs(swp.weight_bytes, best), 1),
                               pct_of_hbm_peak=round(100 * weight_gbs(swp.weight_bytes, best) / HBM_PEAK_GBS, 2),
                               tok_s=round(tok_s(best, B), 1))
            log(f"[bench] p4 B={B}: graph {graph:.3f} ms, chain {chain:.3f} ms "
                f"({swp.weight_bytes / best / 1e6:.0f} GB/s)")
        del swp
        p4["embedding_gather_us"] = time_gather(synth.VOCAB_P4, synth.HIDDEN_P4, (1, 8))
        log(f"[bench] p4 embedding gather: {p4['embedding_gather_us']}")

    # the Q4_K_M-style type mix: mixed-type QKV steps (Q4_K q/k, Q6_K v) and down alternating Q6_K / Q4_K
    q4km = None
    if not args.no_q4km:
        torch.cuda.empty_cache()
        swm = Sweep("q4km", "q4k", (1, 8), 0.0, 0.0, entries=synth.sweep_q4km())
        q4km = {"workload": "52 x {QKV 4608x5120 (q, k Q4_K; v Q6_K; one chain step), O Q4_K 5120x4096, gate+up "
                            "Q4_K 62464x5120, down 5120x31232 (Q6_K even layers, Q4_K odd)} + head Q6_K 131072x5120",
                "weight_bytes": swm.weight_bytes}
        for B in (1, 8):
            plain, graph = time_sweep(swm, B, max(3, args.steps // 2), args.warmup)
            chain = time_chain(swm, B, max(3, args.steps // 2), args.warmup)
            best = min(graph, chain)
            q4km[f"b{B}"] = dict(graph_ms=round(graph, 4), chain_ms=round(chain, 4), plain_ms=round(plain, 4),
                                 weight_gbs=round(weight_gbs(swm.weight_bytes, best), 1),
                                 pct_of_hbm_peak=round(100 * weight_gbs(swm.weight_bytes, best) / HBM_PEAK_GBS, 2),
                                 tok_s=round(tok_s(best, B), 1))
            log(f"[bench] q4km B={B}: graph {graph:.3f} ms, chain {chain:.3f} ms "
                f"({swm.weight_bytes / best / 1e6:.0f} GB/s)")
        del swm

    # the sweep's time per token: the faster of the two ways of running the same dependent sequence
    def best(r):
        return ("chain", r["chain_ms"]) if r["chain_ms"] < r["graph_ms"] else ("graph", r["graph_ms"])
    LAUNCH = {"chain": "one chain launch of the 209 GEMVs (each step reads its x only after the previous "
                       "step's y is complete)",
              "graph": "hipGraph replay of 209 GEMV launches"}
    how1, g1 = best(res[1])
    how8, g8 = best(res[8])
    gbs1 = weight_gbs(bytes3, g1)
    line = {
        "metric": METRIC,
        "value": round(gbs1, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(g1, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "sweep52_q4k_q6k: 52 x {QKV Q4_K 4608x5120, O Q4_K 5120x4096, gate+up Q4_K "
                               "62464x5120, down Q6_K 5120x31232} + head Q6_K 131072x5120",
                   "weight_bytes": bytes3, "batch": 1, "launch": LAUNCH[how1],
                   "x": "bf16 N(0,1), own seed per GEMV", "y": "fp32"},
        "pct_of_hbm_peak": round(100 * gbs1 / HBM_PEAK_GBS, 2),
        "decode_equiv_tok_s": round(tok_s(g1), 1),
        "batch8": {"ms": round(g8, 4), "launch": LAUNCH[how8], "graph_ms": round(res[8]["graph_ms"], 4),
                   "chain_ms": round(res[8]["chain_ms"], 4), "plain_ms": round(res[8]["plain_ms"], 4),
                   "weight_gbs": round(weight_gbs(bytes3, g8), 1),
                   "pct_of_hbm_peak": round(100 * weight_gbs(bytes3, g8) / HBM_PEAK_GBS, 2),
                   "tok_s": round(tok_s(g8, 8), 1)},
        "batch1_all": {"chain_ms": round(res[1]["chain_ms"], 4), "graph_ms": round(res[1]["graph_ms"], 4),
                       "plain_ms": round(res[1]["plain_ms"], 4),
                       "graph_weight_gbs": round(weight_gbs(bytes3, res[1]["graph_ms"]), 1)},
        "independent_gemvs_overlapped": {
            "what": "the same 209 GEMVs, each with its own x and y, in one chain launch whose steps carry "
                    "KQ_STEP_OVERLAP: no step depends on another, so none waits at the step barrier and each "
                    "starts while the one before drains (the sweep as 209 independent products run back to "
                    "back; not a decode, where every projection reads the previous one's output)",
            **{f"b{B}": {"ms": round(res[B]["overlap_ms"], 4),
                         "weight_gbs": round(weight_gbs(bytes3, res[B]["overlap_ms"]), 1),
                         "pct_of_hbm_peak": round(100 * weight_gbs(bytes3, res[B]["overlap_ms"]) / HBM_PEAK_GBS, 2)}
               for B in (1, 8)}},
        "per_step_ms": {f"b{B}": v for B, v in per_step.items()},
        "single_gemvs": singles,
        "read_ceiling": ceiling,
        "smi": {"before": smi_before, "after": smi_after},
        "host": host,
        "verify_cost_staircase": stair,
        "gate_up_swiglu_epilogue_us": swiglu_us,
        "qkvg_6656_fused_us": fused_us,
        "decode_chain_fused": decode,
        "kernels_b1": kt1,
        "kernels_b8": kt8,
        "c4_q5k_merged": c4,
        "hidden6656_sweep": p4,
        "q4km_mixed_sweep": q4km,
        "roofline": roofline,
        "cpu_baseline": cpu,
        "kernel_hash": kernel_source_hash(),
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
