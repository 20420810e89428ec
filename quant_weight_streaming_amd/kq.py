"""Thin Python binding of libkq.so (the C ABI in include/kq.h).

Argument marshalling only: torch tensors supply device memory and the current
HIP stream; every step of the computation runs in the library's HIP kernels.
There is no fallback: if libkq.so is missing or fails to load, every call
raises.
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libkq.so")

KQ_Q4_K, KQ_Q5_K, KQ_Q6_K = 1, 2, 3
KQ_X_F32, KQ_X_BF16 = 0, 1
KQ_MAX_BATCH, KQ_MAX_BATCH_F32, KQ_MAX_PROJ = 16, 8, 8
KQ_EPI_NONE, KQ_EPI_SWIGLU, KQ_EPI_SIGMOID, KQ_EPI_RESIDUAL, KQ_EPI_HEADNORM = 0, 1, 2, 3, 4
KQ_HEAD_ROWS = 128
KQ_STEP_OVERLAP = 1               # kq_chain_step.flags: skip the step barrier where buffers are independent
TYPE_ID = {"q4k": KQ_Q4_K, "q5k": KQ_Q5_K, "q6k": KQ_Q6_K}
SB_BYTES = {"q4k": 144, "q5k": 176, "q6k": 210}
STATUS = {0: "KQ_OK", 1: "KQ_ERR_NULL", 2: "KQ_ERR_SHAPE", 3: "KQ_ERR_ALIGN", 4: "KQ_ERR_BATCH",
          5: "KQ_ERR_TYPE", 6: "KQ_ERR_HIP", 7: "KQ_ERR_NOMEM", 8: "KQ_ERR_RANGE", 9: "KQ_ERR_TIMEOUT",
          10: "KQ_ERR_DEVICE", 11: "KQ_ERR_WORKSPACE"}
KQ_WORKSPACE_BYTES = 72417280     # enough for any GEMV call (kq.h)
KQ_NOALLOC_SCRATCH_BYTES = 8388608  # the static scratch of kq_gemv_fused_noalloc (kq.h)
STATUS_CODE = {v: k for k, v in STATUS.items()}
EXPORTS = ("kq_abi_version", "kq_status_str", "kq_init", "kq_gemv_workspace_bytes", "kq_workspace_init",
           "kq_repacked_bytes", "kq_repack", "kq_gemv_q4k",
           "kq_gemv_q5k", "kq_gemv_q6k", "kq_gemv_multi", "kq_gemv_fused", "kq_gemv_fused_noalloc", "kq_dequant",
           "kq_gather_rows", "kq_stream_read",
           "kq_repack_swiglu",
           "kq_gemv_swiglu", "kq_chain_create", "kq_chain_run",
           "kq_chain_waits", "kq_chain_query", "kq_chain_status", "kq_chain_destroy")


class ChainStep(ctypes.Structure):
    """Mirror of kq_chain_step."""
    _fields_ = [("type", ctypes.c_int32), ("n", ctypes.c_int32), ("cols", ctypes.c_int64),
                ("w", ctypes.c_void_p * KQ_MAX_PROJ), ("rows", ctypes.c_int64 * KQ_MAX_PROJ),
                ("y", ctypes.c_void_p * KQ_MAX_PROJ), ("ldy", ctypes.c_int64 * KQ_MAX_PROJ),
                ("y16", ctypes.c_void_p * KQ_MAX_PROJ), ("ldy16", ctypes.c_int64 * KQ_MAX_PROJ),
                ("x", ctypes.c_void_p), ("ldx", ctypes.c_int64), ("epilogue", ctypes.c_int32),
                ("rms_eps", ctypes.c_float), ("head_eps", ctypes.c_float), ("flags", ctypes.c_int32),
                ("types", ctypes.c_int32 * KQ_MAX_PROJ)]


class KQError(RuntimeError):
    def __init__(self, fn: str, code: int):
        super().__init__(f"{fn} failed: {STATUS.get(code, code)} ({lib().kq_status_str(code).decode()})")
        self.code = code


_lib = None


def lib() -> ctypes.CDLL:
    """Load libkq.so (raises if it is not built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is not built; run quant_weight_streaming_amd.build.build()")
        L = ctypes.CDLL(LIB_PATH)
        vp, i64, ci = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
        L.kq_abi_version.restype = ci
        L.kq_status_str.argtypes = [ci]
        L.kq_status_str.restype = ctypes.c_char_p
        L.kq_init.argtypes = [ci]
        L.kq_init.restype = ci
        L.kq_gemv_workspace_bytes.argtypes = [ci, ci, ctypes.POINTER(i64), i64, ci, ci,
                                              ctypes.POINTER(ctypes.c_int32), ctypes.c_float]
        L.kq_gemv_workspace_bytes.restype = ctypes.c_size_t
        L.kq_workspace_init.argtypes = [vp, ctypes.c_size_t, vp]
        L.kq_workspace_init.restype = ci
        L.kq_repacked_bytes.argtypes = [ci, i64, i64]
        L.kq_repacked_bytes.restype = ctypes.c_size_t
        L.kq_repack.argtypes = [ci, i64, i64, vp, vp, vp]
        L.kq_repack.restype = ci
        for n in ("kq_gemv_q4k", "kq_gemv_q5k", "kq_gemv_q6k"):
            f = getattr(L, n)
            f.argtypes = [vp, i64, i64, vp, ci, i64, ci, vp, i64, vp, ctypes.c_size_t, vp]
            f.restype = ci
        L.kq_gemv_multi.argtypes = [ci, ci, ctypes.POINTER(vp), ctypes.POINTER(i64), i64, vp, ci, i64, ci,
                                    ctypes.POINTER(vp), ctypes.POINTER(i64), vp, ctypes.c_size_t, vp]
        L.kq_gemv_multi.restype = ci
        L.kq_gemv_fused.argtypes = [ci, ci, ctypes.POINTER(vp), ctypes.POINTER(i64), i64, vp, ci, i64, ci,
                                    ctypes.POINTER(vp), ctypes.POINTER(i64), ctypes.POINTER(vp), ctypes.POINTER(i64),
                                    ctypes.POINTER(ctypes.c_int32), ctypes.c_float, ctypes.c_float, vp,
                                    ctypes.c_size_t, vp]
        L.kq_gemv_fused.restype = ci
        L.kq_gemv_fused_noalloc.argtypes = [ci, ci, ctypes.POINTER(vp), ctypes.POINTER(i64), i64, vp, ci, i64, ci,
                                            ctypes.POINTER(vp), ctypes.POINTER(i64), ctypes.POINTER(vp),
                                            ctypes.POINTER(i64), ctypes.POINTER(ctypes.c_int32), ctypes.c_float,
                                            ctypes.c_float, vp]
        L.kq_gemv_fused_noalloc.restype = ci
        L.kq_stream_read.argtypes = [vp, ctypes.c_size_t, vp, vp]
        L.kq_stream_read.restype = ci
        L.kq_dequant.argtypes = [ci, vp, i64, i64, vp, i64, vp]
        L.kq_dequant.restype = ci
        L.kq_gather_rows.argtypes = [ci, vp, i64, i64, vp, i64, vp, i64, vp]
        L.kq_gather_rows.restype = ci
        L.kq_repack_swiglu.argtypes = [ci, i64, i64, vp, vp, vp, vp]
        L.kq_repack_swiglu.restype = ci
        L.kq_gemv_swiglu.argtypes = [ci, vp, i64, i64, vp, ci, i64, ci, vp, i64, vp, ctypes.c_size_t, vp]
        L.kq_gemv_swiglu.restype = ci
        L.kq_chain_create.argtypes = [ci, ctypes.POINTER(ChainStep), ci, ci, ctypes.POINTER(vp)]
        L.kq_chain_create.restype = ci
        for n in ("kq_chain_query", "kq_chain_status", "kq_chain_destroy"):
            getattr(L, n).argtypes = [vp]
            getattr(L, n).restype = ci
        L.kq_chain_run.argtypes = [vp, vp]
        L.kq_chain_run.restype = ci
        L.kq_chain_waits.argtypes = [vp, ctypes.POINTER(ctypes.c_uint8), ci]
        L.kq_chain_waits.restype = ci
        _lib = L
    return _lib


def _stream(stream) -> int:
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _check(fn: str, rc: int) -> None:
    if rc != 0:
        raise KQError(fn, rc)


def _xtype(x: torch.Tensor) -> int:
    if x.dtype == torch.bfloat16:
        return KQ_X_BF16
    if x.dtype == torch.float32:
        return KQ_X_F32
    raise TypeError(f"x must be bfloat16 or float32, got {x.dtype}")


def _type(qtype) -> int:
    return TYPE_ID[qtype] if isinstance(qtype, str) else int(qtype)


# ---------------------------------------------------------------- C-ABI mirrors

def kq_abi_version() -> int:
    return lib().kq_abi_version()


def kq_init(device: int = 0) -> None:
    _check("kq_init", lib().kq_init(device))


def kq_gemv_workspace_bytes(qtype, rows, cols: int, xtype: int, batch: int, epis=None, rms_eps: float = 0.0) -> int:
    n = len(rows)
    R = (ctypes.c_int64 * n)(*rows)
    E = (ctypes.c_int32 * n)(*epis) if epis is not None else None
    return int(lib().kq_gemv_workspace_bytes(_type(qtype), n, R, cols, xtype, batch, E, rms_eps))


def kq_workspace_init(ws: torch.Tensor, stream=None) -> None:
    _check("kq_workspace_init", lib().kq_workspace_init(ws.data_ptr(), ws.numel() * ws.element_size(),
                                                        _stream(stream)))


_workspaces = {}


def workspace(stream=None) -> torch.Tensor:
    """This binding's workspace for `stream` (default: the current stream): KQ_WORKSPACE_BYTES of device
    memory that torch allocates on the stream's device the first time the stream is used, prepared with
    kq_workspace_init on that stream.  One per stream, so calls on unordered streams never share one."""
    h = _stream(stream)
    dev = torch.cuda.current_device()
    key = (dev, h)
    ws = _workspaces.get(key)
    if ws is None:
        ws = torch.empty(KQ_WORKSPACE_BYTES, dtype=torch.uint8, device=f"cuda:{dev}")
        kq_workspace_init(ws, h)
        _workspaces[key] = ws
    return ws


def _ws(ws, stream):
    """(pointer, bytes) of the caller's workspace tensor, or of the stream's own."""
    t = ws if ws is not None else workspace(stream)
    return t.data_ptr(), t.numel() * t.element_size()


def kq_repacked_bytes(qtype, rows: int, cols: int) -> int:
    return int(lib().kq_repacked_bytes(_type(qtype), rows, cols))


def kq_repack(qtype, rows: int, cols: int, gguf: torch.Tensor, out: torch.Tensor, stream=None) -> None:
    _check("kq_repack", lib().kq_repack(_type(qtype), rows, cols, gguf.data_ptr(), out.data_ptr(), _stream(stream)))


def _gemv(fn: str, w: torch.Tensor, rows: int, cols: int, x: torch.Tensor, y: torch.Tensor, stream=None,
          work=None) -> None:
    if x.dim() != 2 or y.dim() != 2:
        raise ValueError("x is [batch, ldx], y is [batch, ldy]")
    f = getattr(lib(), fn)
    _check(fn, f(w.data_ptr(), rows, cols, x.data_ptr(), _xtype(x), x.stride(0), x.shape[0], y.data_ptr(),
                 y.stride(0), *_ws(work, stream), _stream(stream)))


def kq_gemv_q4k(w, rows, cols, x, y, stream=None, work=None):
    _gemv("kq_gemv_q4k", w, rows, cols, x, y, stream, work)


def kq_gemv_q5k(w, rows, cols, x, y, stream=None, work=None):
    _gemv("kq_gemv_q5k", w, rows, cols, x, y, stream, work)


def kq_gemv_q6k(w, rows, cols, x, y, stream=None, work=None):
    _gemv("kq_gemv_q6k", w, rows, cols, x, y, stream, work)


def kq_gemv_multi(qtype, ws, rows, cols: int, x: torch.Tensor, ys, stream=None, work=None) -> None:
    n = len(ws)
    if len(rows) != n or len(ys) != n:
        raise ValueError("ws, rows and ys must have the same length")
    W = (ctypes.c_void_p * n)(*[w.data_ptr() for w in ws])
    R = (ctypes.c_int64 * n)(*rows)
    Y = (ctypes.c_void_p * n)(*[y.data_ptr() for y in ys])
    LD = (ctypes.c_int64 * n)(*[y.stride(0) for y in ys])
    _check("kq_gemv_multi", lib().kq_gemv_multi(_type(qtype), n, W, R, cols, x.data_ptr(), _xtype(x), x.stride(0),
                                                x.shape[0], Y, LD, *_ws(work, stream), _stream(stream)))


def kq_gemv_fused(qtype, ws, rows, cols: int, x: torch.Tensor, ys, epis=None, rms_eps: float = 0.0,
                  stream=None, head_eps: float = 0.0, y16s=None, work=None) -> None:
    """kq_gemv_multi with a weight-less RMSNorm of x first (rms_eps > 0), an epilogue code per segment
    (epis: None for none; KQ_EPI_HEADNORM segments use head_eps) and optional bf16 copies of the outputs
    (y16s: None, or one bf16 tensor or None per segment)."""
    n = len(ws)
    if len(rows) != n or len(ys) != n or (epis is not None and len(epis) != n) or (y16s is not None and len(y16s) != n):
        raise ValueError("ws, rows, ys, epis and y16s must have the same length")
    W = (ctypes.c_void_p * n)(*[w.data_ptr() for w in ws])
    R = (ctypes.c_int64 * n)(*rows)
    Y = (ctypes.c_void_p * n)(*[y.data_ptr() for y in ys])
    LD = (ctypes.c_int64 * n)(*[y.stride(0) for y in ys])
    E = (ctypes.c_int32 * n)(*epis) if epis is not None else None
    Y16 = LD16 = None
    if y16s is not None:
        Y16 = (ctypes.c_void_p * n)(*[t.data_ptr() if t is not None else None for t in y16s])
        LD16 = (ctypes.c_int64 * n)(*[t.stride(0) if t is not None else 0 for t in y16s])
    _check("kq_gemv_fused", lib().kq_gemv_fused(_type(qtype), n, W, R, cols, x.data_ptr(), _xtype(x), x.stride(0),
                                                x.shape[0], Y, LD, Y16, LD16, E, rms_eps, head_eps, *_ws(work, stream),
                                                _stream(stream)))


def kq_gemv_fused_noalloc(qtype, ws, rows, cols: int, x: torch.Tensor, ys, epis=None, rms_eps: float = 0.0,
                          stream=None, head_eps: float = 0.0, y16s=None) -> None:
    """kq_gemv_fused on the library's static scratch: no workspace argument, no allocation."""
    n = len(ws)
    if len(rows) != n or len(ys) != n or (epis is not None and len(epis) != n) or (y16s is not None and len(y16s) != n):
        raise ValueError("ws, rows, ys, epis and y16s must have the same length")
    W = (ctypes.c_void_p * n)(*[w.data_ptr() for w in ws])
    R = (ctypes.c_int64 * n)(*rows)
    Y = (ctypes.c_void_p * n)(*[y.data_ptr() for y in ys])
    LD = (ctypes.c_int64 * n)(*[y.stride(0) for y in ys])
    E = (ctypes.c_int32 * n)(*epis) if epis is not None else None
    Y16 = LD16 = None
    if y16s is not None:
        Y16 = (ctypes.c_void_p * n)(*[t.data_ptr() if t is not None else None for t in y16s])
        LD16 = (ctypes.c_int64 * n)(*[t.stride(0) if t is not None else 0 for t in y16s])
    _check("kq_gemv_fused_noalloc",
           lib().kq_gemv_fused_noalloc(_type(qtype), n, W, R, cols, x.data_ptr(), _xtype(x), x.stride(0), x.shape[0],
                                       Y, LD, Y16, LD16, E, rms_eps, head_eps, _stream(stream)))


def kq_stream_read(buf: torch.Tensor, sink: torch.Tensor, stream=None) -> None:
    """Read every byte of `buf` once with the GEMV's loads (the achievable read rate)."""
    _check("kq_stream_read", lib().kq_stream_read(buf.data_ptr(), buf.numel() * buf.element_size(),
                                                  sink.data_ptr(), _stream(stream)))


def kq_dequant(qtype, w: torch.Tensor, rows: int, cols: int, out: torch.Tensor, stream=None) -> None:
    _check("kq_dequant", lib().kq_dequant(_type(qtype), w.data_ptr(), rows, cols, out.data_ptr(), out.stride(0),
                                          _stream(stream)))


def kq_repack_swiglu(qtype, inter: int, cols: int, gate: torch.Tensor, up: torch.Tensor, out: torch.Tensor,
                     stream=None) -> None:
    _check("kq_repack_swiglu", lib().kq_repack_swiglu(_type(qtype), inter, cols, gate.data_ptr(), up.data_ptr(),
                                                      out.data_ptr(), _stream(stream)))


def kq_gemv_swiglu(qtype, w: torch.Tensor, inter: int, cols: int, x: torch.Tensor, y: torch.Tensor,
                   stream=None, work=None) -> None:
    _check("kq_gemv_swiglu", lib().kq_gemv_swiglu(_type(qtype), w.data_ptr(), inter, cols, x.data_ptr(), _xtype(x),
                                                  x.stride(0), x.shape[0], y.data_ptr(), y.stride(0),
                                                  *_ws(work, stream), _stream(stream)))


def kq_gather_rows(qtype, w: torch.Tensor, rows: int, cols: int, ids: torch.Tensor, out: torch.Tensor,
                   stream=None) -> None:
    if ids.dtype != torch.int32:
        raise TypeError("ids must be int32")
    _check("kq_gather_rows", lib().kq_gather_rows(_type(qtype), w.data_ptr(), rows, cols, ids.data_ptr(), ids.numel(),
                                                  out.data_ptr(), out.stride(0), _stream(stream)))


def kq_chain_create(steps, xtype: int, batch: int, overlap: bool = False) -> int:
    """steps: sequence of (qtype, ws, rows, cols, x, ys[, epilogue[, rms_eps[, head_eps[, y16s[, types]]]]]) as
    kq_gemv_multi and kq_gemv_fused take them, the epilogue packed four bits per segment; qtype may be a list
    of per-segment types (a mixed-type step), or `types` gives them; overlap: every step carries
    KQ_STEP_OVERLAP (it skips the step barrier where its buffers are independent); returns the handle."""
    arr = (ChainStep * len(steps))()
    for st, step in zip(arr, steps):
        st.flags = KQ_STEP_OVERLAP if overlap else 0
        qtype, ws, rows, cols, x, ys = step[:6]
        st.epilogue = step[6] if len(step) > 6 else KQ_EPI_NONE
        st.rms_eps = step[7] if len(step) > 7 else 0.0
        st.head_eps = step[8] if len(step) > 8 else 0.0
        y16s = step[9] if len(step) > 9 else None
        types = step[10] if len(step) > 10 else None
        if isinstance(qtype, (list, tuple)):
            qtype, types = qtype[0], qtype
        n = len(ws)
        if len(rows) != n or len(ys) != n or n > KQ_MAX_PROJ or (types is not None and len(types) != n):
            raise ValueError("ws, rows, ys (and types) must have the same length, at most KQ_MAX_PROJ")
        st.type, st.n, st.cols = _type(qtype), n, cols
        if types is not None:
            for i, t in enumerate(types):
                st.types[i] = _type(t)
        for i in range(n):
            st.w[i], st.rows[i], st.y[i], st.ldy[i] = ws[i].data_ptr(), rows[i], ys[i].data_ptr(), ys[i].stride(0)
            if y16s is not None and y16s[i] is not None:
                st.y16[i], st.ldy16[i] = y16s[i].data_ptr(), y16s[i].stride(0)
        st.x, st.ldx = x.data_ptr(), x.stride(0)
    h = ctypes.c_void_p()
    _check("kq_chain_create", lib().kq_chain_create(len(steps), arr, xtype, batch, ctypes.byref(h)))
    return h.value


def kq_chain_run(handle: int, stream=None) -> None:
    _check("kq_chain_run", lib().kq_chain_run(handle, _stream(stream)))


def kq_chain_waits(handle: int, n_steps: int) -> list:
    """Per step: True if it waits at the step barrier, False if it overlaps the steps before it."""
    w = (ctypes.c_uint8 * n_steps)()
    _check("kq_chain_waits", lib().kq_chain_waits(handle, w, n_steps))
    return [bool(v) for v in w]


def kq_chain_query(handle: int) -> int:
    """KQ_OK, or KQ_ERR_TIMEOUT once a run's wait has given up (no device synchronisation); does not raise."""
    return lib().kq_chain_query(handle)


def kq_chain_status(handle: int) -> int:
    """KQ_OK, or the status code (KQ_ERR_TIMEOUT when a wait gave up); does not raise."""
    return lib().kq_chain_status(handle)


def kq_chain_destroy(handle: int) -> None:
    _check("kq_chain_destroy", lib().kq_chain_destroy(handle))


# ---------------------------------------------------------------- conveniences


class Chain:
    """A chain plan that keeps the tensors of its steps alive; run() enqueues one run."""

    def __init__(self, steps, batch: int, overlap: bool = False):
        self.steps = list(steps)
        xt = {_xtype(s[4]) for s in self.steps}
        if len(xt) != 1:
            raise ValueError("every step of a chain takes the same activation type")
        self.handle = kq_chain_create(self.steps, xt.pop(), batch, overlap)

    def run(self, stream=None) -> None:
        kq_chain_run(self.handle, stream)

    def status(self) -> int:
        return kq_chain_status(self.handle)

    def waits(self) -> list:
        return kq_chain_waits(self.handle, len(self.steps))

    def query(self) -> int:
        return kq_chain_query(self.handle)

    def close(self) -> None:
        if self.handle:
            kq_chain_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

GEMV = {"q4k": kq_gemv_q4k, "q5k": kq_gemv_q5k, "q6k": kq_gemv_q6k}


def repack(qtype: str, gguf: torch.Tensor, rows: int, cols: int, stream=None) -> torch.Tensor:
    """GGUF bytes on the device -> new repacked uint8 tensor."""
    out = torch.empty(kq_repacked_bytes(qtype, rows, cols), dtype=torch.uint8, device=gguf.device)
    kq_repack(qtype, rows, cols, gguf, out, stream)
    return out


def gemv(qtype: str, w: torch.Tensor, rows: int, cols: int, x: torch.Tensor, y: torch.Tensor = None,
         stream=None, work=None) -> torch.Tensor:
    if y is None:
        y = torch.empty((x.shape[0], rows), dtype=torch.float32, device=x.device)
    GEMV[qtype](w, rows, cols, x, y, stream, work)
    return y


def repack_swiglu(qtype: str, gate: torch.Tensor, up: torch.Tensor, inter: int, cols: int, stream=None) -> torch.Tensor:
    """GGUF bytes of the gate and up matrices on the device -> the interleaved repacked pair."""
    out = torch.empty(kq_repacked_bytes(qtype, 64 * ((inter + 31) // 32), cols), dtype=torch.uint8, device=gate.device)
    kq_repack_swiglu(qtype, inter, cols, gate, up, out, stream)
    return out


def gemv_swiglu(qtype: str, w: torch.Tensor, inter: int, cols: int, x: torch.Tensor, y: torch.Tensor = None,
                stream=None) -> torch.Tensor:
    if y is None:
        y = torch.empty((x.shape[0], inter), dtype=torch.float32, device=x.device)
    kq_gemv_swiglu(qtype, w, inter, cols, x, y, stream)
    return y


def gather_rows(qtype: str, w: torch.Tensor, rows: int, cols: int, ids: torch.Tensor, stream=None) -> torch.Tensor:
    out = torch.empty((ids.numel(), cols), dtype=torch.float32, device=w.device)
    kq_gather_rows(qtype, w, rows, cols, ids, out, stream)
    return out


def dequant(qtype: str, w: torch.Tensor, rows: int, cols: int, stream=None) -> torch.Tensor:
    out = torch.empty((rows, cols), dtype=torch.float32, device=w.device)
    kq_dequant(qtype, w, rows, cols, out, stream)
    return out
