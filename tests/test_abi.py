"""The C-ABI library: it loads, exports every symbol include/kq.h declares, and
rejects invalid arguments on the host (no device work, so this runs without a GPU)."""
import ctypes
import os
import re

import pytest

from quant_weight_streaming_amd import kq

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_symbols():
    src = open(os.path.join(ROOT, "include", "kq.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(kq_[a-z0-9_]+)\s*\(", src)))


def test_header_matches_binding():
    assert declared_symbols() == sorted(kq.EXPORTS)


def test_library_exports_every_declared_symbol():
    L = kq.lib()
    for name in declared_symbols():
        assert hasattr(L, name), name


def test_timeline_symbol_only_in_the_measurement_build(tmp_path):
    """kq_timeline.h compiles as C99; its one symbol is exported by libkq_timeline.so (when built) and not by the
    product library, whose chain kernel records nothing."""
    import subprocess
    src = tmp_path / "tl.c"
    src.write_text('#include "kq_timeline.h"\nint main(void) { return kq_chain_timeline != 0 ? 0 : 1; }\n')
    subprocess.run(["gcc", "-std=c99", "-fsyntax-only", "-I", os.path.join(ROOT, "include"), str(src)], check=True)
    assert not hasattr(kq.lib(), "kq_chain_timeline")
    tl = os.path.join(ROOT, "quant_weight_streaming_amd", "libkq_timeline.so")
    if os.path.exists(tl):
        assert hasattr(ctypes.CDLL(tl), "kq_chain_timeline")


def test_missing_library_fails_loudly(monkeypatch, tmp_path):
    """No fallback path: without the built library every entry point raises instead of computing on the CPU."""
    monkeypatch.setattr(kq, "LIB_PATH", str(tmp_path / "libkq.so"))
    monkeypatch.setattr(kq, "_lib", None)
    with pytest.raises(ImportError):
        kq.lib()
    with pytest.raises(ImportError):
        kq.kq_repacked_bytes("q4k", 64, 256)


def test_version_and_sizes():
    assert kq.kq_abi_version() == 2
    assert kq.kq_repacked_bytes("q4k", 256, 1024) == 256 * 4 * 144
    assert kq.kq_repacked_bytes("q5k", 1, 256) == 64 * 176          # one zero-padded tile
    assert kq.kq_repacked_bytes("q6k", 65, 512) == 2 * 2 * 64 * 210
    assert kq.kq_repacked_bytes("q4k", 64, 300) == 0                 # cols not a multiple of 256
    assert kq.kq_repacked_bytes(9, 64, 256) == 0
    assert kq.kq_repacked_bytes("q4k", 0, 256) == 0


A16 = 0x10000  # a fake, 16-byte aligned "device" address: validation fails before any use
WS = (A16, kq.KQ_WORKSPACE_BYTES)   # a fake workspace of the documented size


@pytest.mark.parametrize("args,code", [
    # (w, rows, cols, x, xtype, ldx, batch, y, ldy)
    ((None, 64, 256, A16, 1, 256, 1, A16, 64), 1),
    ((A16, 64, 256, None, 1, 256, 1, A16, 64), 1),
    ((A16, 64, 256, A16, 1, 256, 1, None, 64), 1),
    ((A16, 64, 300, A16, 1, 300, 1, A16, 64), 2),       # cols % 256
    ((A16, 0, 256, A16, 1, 256, 1, A16, 64), 2),        # rows < 1
    ((A16, 64, 256, A16, 1, 128, 1, A16, 64), 2),       # ldx < cols
    ((A16, 64, 256, A16, 1, 256, 1, A16, 32), 2),       # ldy < rows
    ((A16 + 4, 64, 256, A16, 1, 256, 1, A16, 64), 3),   # w misaligned
    ((A16, 64, 256, A16 + 2, 1, 256, 1, A16, 64), 3),   # x misaligned
    ((A16, 64, 256, A16, 1, 260, 1, A16, 64), 3),       # bf16 row stride not 16 B
    ((A16, 64, 256, A16, 1, 256, 0, A16, 64), 4),       # batch 0
    ((A16, 64, 256, A16, 1, 256, 17, A16, 64), 4),      # batch 17 (bf16 x allows 16)
    ((A16, 64, 256, A16, 0, 256, 9, A16, 64), 4),       # batch 9 with fp32 x (fp32 allows 8)
    ((A16, 64, 256, A16, 7, 256, 1, A16, 64), 5),       # xtype
])
def test_gemv_rejects(args, code):
    for fn in ("kq_gemv_q4k", "kq_gemv_q5k", "kq_gemv_q6k"):
        assert getattr(kq.lib(), fn)(*args, *WS, None) == code


def test_multi_and_others_reject():
    L = kq.lib()
    vp, i64 = ctypes.c_void_p, ctypes.c_int64
    W = (vp * 2)(A16, A16)
    R = (i64 * 2)(64, 64)
    Y = (vp * 2)(A16, A16)
    LD = (i64 * 2)(64, 64)
    assert L.kq_gemv_multi(9, 2, W, R, 256, A16, 1, 256, 1, Y, LD, *WS, None) == 5
    assert L.kq_gemv_multi(1, 0, W, R, 256, A16, 1, 256, 1, Y, LD, *WS, None) == 4
    assert L.kq_gemv_multi(1, 9, W, R, 256, A16, 1, 256, 1, Y, LD, *WS, None) == 4
    Yb = (vp * 2)(A16, None)
    assert L.kq_gemv_multi(1, 2, W, R, 256, A16, 1, 256, 1, Yb, LD, *WS, None) == 1
    Rb = (i64 * 2)(64, 0)
    assert L.kq_gemv_multi(1, 2, W, Rb, 256, A16, 1, 256, 1, Y, LD, *WS, None) == 2
    assert L.kq_repack(1, 64, 256, None, A16, None) == 1
    assert L.kq_repack(1, 64, 300, A16, A16, None) == 2
    assert L.kq_repack(1, 64, 256, A16 + 2, A16, None) == 3       # Q4_K input needs 4-byte alignment
    assert L.kq_repack(4, 64, 256, A16, A16, None) == 5
    assert L.kq_dequant(1, A16, 64, 256, A16, 100, None) == 2     # ldo < cols
    assert L.kq_dequant(3, A16 + 8, 64, 256, A16, 256, None) == 3
    assert kq.lib().kq_status_str(3) == b"misaligned pointer or stride"


def test_chain_step_layout_matches_header(tmp_path):
    """The ctypes mirror of kq_chain_step has the C layout (size and every field offset)."""
    import subprocess
    fields = [f[0] for f in kq.ChainStep._fields_]
    src = tmp_path / "layout.c"
    src.write_text('#include <stddef.h>\n#include <stdio.h>\n#include "kq.h"\nint main(void) {\n'
                   '  printf("%zu", sizeof(kq_chain_step));\n' +
                   "".join(f'  printf(" %zu", offsetof(kq_chain_step, {f}));\n' for f in fields) +
                   "  return 0;\n}\n")
    exe = tmp_path / "layout"
    subprocess.run(["gcc", "-std=c99", "-I", os.path.join(ROOT, "include"), str(src), "-o", str(exe)], check=True)
    got = [int(v) for v in subprocess.run([str(exe)], capture_output=True, text=True, check=True).stdout.split()]
    assert got == [ctypes.sizeof(kq.ChainStep)] + [getattr(kq.ChainStep, f).offset for f in fields]


def _step(**kw):
    st = kq.ChainStep()
    st.type, st.n, st.cols, st.x, st.ldx = 1, 1, 256, A16, 256
    st.w[0], st.rows[0], st.y[0], st.ldy[0] = A16, 64, A16, 64
    for k, v in kw.items():
        setattr(st, k, v)
    return st


@pytest.mark.parametrize("step,xtype,batch,code", [
    (dict(type=9), 1, 1, 5),                 # weight type
    (dict(), 7, 1, 5),                       # activation type
    (dict(), 1, 0, 4),                       # batch
    (dict(), 1, 17, 4),
    (dict(), 0, 9, 4),                       # fp32 x: at most 8
    (dict(n=0), 1, 1, 4),                    # segments
    (dict(cols=300, ldx=300), 1, 1, 2),      # cols % 256
    (dict(ldx=128), 1, 1, 2),                # ldx < cols
    (dict(x=None), 1, 1, 1),
    (dict(x=A16 + 2), 1, 1, 3),
    (dict(ldx=1 << 30), 1, 2, 8),            # x rows beyond 31-bit offsets
])
def test_chain_create_rejects(step, xtype, batch, code):
    arr = (kq.ChainStep * 2)(_step(), _step(**step))
    h = ctypes.c_void_p(1234)
    assert kq.lib().kq_chain_create(2, arr, xtype, batch, ctypes.byref(h)) == code
    assert h.value is None                   # nothing was created


def test_chain_other_rejects():
    L = kq.lib()
    arr = (kq.ChainStep * 1)(_step())
    h = ctypes.c_void_p()
    assert L.kq_chain_create(0, arr, 1, 1, ctypes.byref(h)) == 4
    assert L.kq_chain_create(1, None, 1, 1, ctypes.byref(h)) == 1
    assert L.kq_chain_create(1, arr, 1, 1, None) == 1
    assert L.kq_chain_run(None, None) == 1
    assert L.kq_chain_status(None) == 1
    assert L.kq_chain_query(None) == 1
    assert L.kq_chain_destroy(None) == 0
    assert L.kq_status_str(9) == b"a chain step's wait for the previous step gave up"


def test_gather_rejects():
    L = kq.lib()
    ids = A16
    assert L.kq_gather_rows(9, A16, 64, 256, ids, 4, A16, 256, None) == 5       # type
    assert L.kq_gather_rows(1, None, 64, 256, ids, 4, A16, 256, None) == 1      # w
    assert L.kq_gather_rows(1, A16, 64, 256, None, 4, A16, 256, None) == 1      # ids
    assert L.kq_gather_rows(1, A16, 64, 256, ids, 4, None, 256, None) == 1      # out
    assert L.kq_gather_rows(1, A16, 64, 300, ids, 4, A16, 300, None) == 2       # cols % 256
    assert L.kq_gather_rows(1, A16, 0, 256, ids, 4, A16, 256, None) == 2        # rows
    assert L.kq_gather_rows(1, A16, 64, 256, ids, 4, A16, 128, None) == 2       # ldo < cols
    assert L.kq_gather_rows(1, A16 + 4, 64, 256, ids, 4, A16, 256, None) == 3   # w alignment
    assert L.kq_gather_rows(1, A16, 64, 256, ids + 2, 4, A16, 256, None) == 3   # ids alignment
    assert L.kq_gather_rows(1, A16, 64, 256, ids, -1, A16, 256, None) == 4      # n < 0
    assert L.kq_gather_rows(1, A16, 64, 256, None, 0, None, 256, None) == 0     # n = 0: nothing to do


def test_swiglu_rejects():
    L = kq.lib()
    assert L.kq_repack_swiglu(9, 64, 256, A16, A16, A16, None) == 5
    assert L.kq_repack_swiglu(1, 64, 256, None, A16, A16, None) == 1
    assert L.kq_repack_swiglu(1, 64, 256, A16, None, A16, None) == 1
    assert L.kq_repack_swiglu(1, 0, 256, A16, A16, A16, None) == 2
    assert L.kq_repack_swiglu(1, 64, 300, A16, A16, A16, None) == 2
    assert L.kq_repack_swiglu(1, 64, 256, A16, A16, A16 + 4, None) == 3
    assert L.kq_gemv_swiglu(1, A16, 64, 256, A16, 1, 256, 17, A16, 64, *WS, None) == 4
    assert L.kq_gemv_swiglu(1, A16, 64, 256, A16, 1, 128, 1, A16, 64, *WS, None) == 2
    assert L.kq_gemv_swiglu(1, None, 64, 256, A16, 1, 256, 1, A16, 64, *WS, None) == 1


def test_chain_rejects_bad_epilogue():
    bad = _step()
    bad.epilogue = 7
    arr = (kq.ChainStep * 1)(bad)
    h = ctypes.c_void_p()
    assert kq.lib().kq_chain_create(1, arr, 1, 1, ctypes.byref(h)) == 5
    two = _step(n=2)
    two.w[1], two.rows[1], two.y[1], two.ldy[1] = A16, 64, A16, 64
    two.epilogue = 1                              # SwiGLU takes one matrix
    arr = (kq.ChainStep * 1)(two)
    assert kq.lib().kq_chain_create(1, arr, 1, 1, ctypes.byref(h)) == 5


def test_fused_rejects():
    L = kq.lib()
    vp, i64 = ctypes.c_void_p, ctypes.c_int64
    W = (vp * 2)(A16, A16)
    R = (i64 * 2)(64, 64)
    Y = (vp * 2)(A16, A16)
    LD = (i64 * 2)(64, 64)
    E = (ctypes.c_int32 * 2)(2, 9)
    assert L.kq_gemv_fused(1, 2, W, R, 256, A16, 1, 256, 1, Y, LD, None, None, E, 0.0, 0.0, *WS, None) == 5      # unknown code
    E = (ctypes.c_int32 * 2)(1, 0)
    assert L.kq_gemv_fused(1, 2, W, R, 256, A16, 1, 256, 1, Y, LD, None, None, E, 0.0, 0.0, *WS, None) == 5      # SwiGLU needs n = 1
    for eps in (-1e-5, float("inf"), float("nan")):
        assert L.kq_gemv_fused(1, 2, W, R, 256, A16, 1, 256, 1, Y, LD, None, None, None, eps, 0.0, *WS, None) == 2
    assert L.kq_gemv_fused(1, 0, W, R, 256, A16, 1, 256, 1, Y, LD, None, None, None, 0.0, 0.0, *WS, None) == 4
    # head norm: rows a multiple of KQ_HEAD_ROWS, head_eps finite and > 0
    E = (ctypes.c_int32 * 2)(4, 0)
    assert L.kq_gemv_fused(1, 2, W, R, 256, A16, 1, 256, 1, Y, LD, None, None, E, 0.0, 1e-6, *WS, None) == 2    # 64 rows
    R2 = (i64 * 2)(128, 64)
    LD2 = (i64 * 2)(128, 64)
    for eps in (0.0, -1.0, float("inf"), float("nan")):
        assert L.kq_gemv_fused(1, 2, W, R2, 256, A16, 1, 256, 1, Y, LD2, None, None, E, 0.0, eps, *WS, None) == 2
    # bf16 copies: a stride for every copy, at least the segment's rows, 2-byte aligned
    Y16 = (vp * 2)(A16, None)
    assert L.kq_gemv_fused(1, 2, W, R, 256, A16, 1, 256, 1, Y, LD, Y16, None, None, 0.0, 0.0, *WS, None) == 1
    LD16 = (i64 * 2)(63, 0)
    assert L.kq_gemv_fused(1, 2, W, R, 256, A16, 1, 256, 1, Y, LD, Y16, LD16, None, 0.0, 0.0, *WS, None) == 2
    Y16 = (vp * 2)(A16 + 1, None)
    LD16 = (i64 * 2)(64, 0)
    assert L.kq_gemv_fused(1, 2, W, R, 256, A16, 1, 256, 1, Y, LD, Y16, LD16, None, 0.0, 0.0, *WS, None) == 3
    st = _step()
    st.y16[0], st.ldy16[0] = A16, 32
    arr = (kq.ChainStep * 1)(st)
    assert L.kq_chain_create(1, arr, 1, 1, ctypes.byref(h := ctypes.c_void_p())) == 2
    st = _step()
    st.epilogue = 3 | (2 << 4)                    # a code for a segment the step does not have
    arr = (kq.ChainStep * 1)(st)
    h = ctypes.c_void_p()
    assert L.kq_chain_create(1, arr, 1, 1, ctypes.byref(h)) == 5
    st = _step()
    st.rms_eps = -1.0
    arr = (kq.ChainStep * 1)(st)
    assert L.kq_chain_create(1, arr, 1, 1, ctypes.byref(h)) == 2
    st = _step(epilogue=4, head_eps=1e-6)           # a head-norm segment of 64 rows
    arr = (kq.ChainStep * 1)(st)
    assert L.kq_chain_create(1, arr, 1, 1, ctypes.byref(h)) == 2


def test_workspace_rules():
    """The library allocates nothing: a GEMV call without a usable workspace is refused on the host."""
    L = kq.lib()
    args = (A16, 64, 256, A16, 1, 256, 1, A16, 64)
    for fn in ("kq_gemv_q4k", "kq_gemv_q5k", "kq_gemv_q6k"):
        assert getattr(L, fn)(*args, None, kq.KQ_WORKSPACE_BYTES, None) == 11          # no workspace
        assert getattr(L, fn)(*args, A16 + 8, kq.KQ_WORKSPACE_BYTES, None) == 11       # misaligned
        assert getattr(L, fn)(A16, 64, 300, A16, 1, 300, 1, A16, 64, None, 0, None) == 2   # arguments first
    vp, i64 = ctypes.c_void_p, ctypes.c_int64
    W, R, Y, LD = (vp * 1)(A16), (i64 * 1)(64), (vp * 1)(A16), (i64 * 1)(64)
    assert L.kq_gemv_multi(1, 1, W, R, 256, A16, 1, 256, 1, Y, LD, None, 0, None) == 11
    assert L.kq_gemv_fused(1, 1, W, R, 256, A16, 1, 256, 1, Y, LD, None, None, None, 0.0, 0.0, None, 0, None) == 11
    assert L.kq_gemv_swiglu(1, A16, 64, 256, A16, 1, 256, 1, A16, 64, None, 0, None) == 11
    assert L.kq_workspace_init(None, kq.KQ_WORKSPACE_BYTES, None) == 1
    assert L.kq_workspace_init(A16 + 4, kq.KQ_WORKSPACE_BYTES, None) == 11
    assert L.kq_workspace_init(A16, 65535, None) == 11                               # smaller than the counters
    assert L.kq_status_str(11) == b"workspace missing, misaligned or smaller than the call needs"
    # the size query returns 0 for invalid arguments
    assert kq.kq_gemv_workspace_bytes("q4k", [64], 300, kq.KQ_X_BF16, 1) == 0
    assert kq.kq_gemv_workspace_bytes("q4k", [64], 256, kq.KQ_X_BF16, 17) == 0
    assert kq.kq_gemv_workspace_bytes(9, [64], 256, kq.KQ_X_BF16, 1) == 0


def test_workspace_bound_matches_layout():
    """KQ_WORKSPACE_BYTES = the counter block + two slots of 16 batch rows per workgroup for the largest grid
    + the heads' sums of squares (the layout the library documents)."""
    counters = 2 * 8192 * 4
    slots = 2 * 8192 * (16 * 64 + 64) * 4
    heads = 8192 * 2 * 16 * 4
    assert kq.KQ_WORKSPACE_BYTES == counters + slots + heads
    src = open(os.path.join(ROOT, "include", "kq.h")).read()
    assert re.search(r"#define KQ_WORKSPACE_BYTES (\d+)u", src).group(1) == str(kq.KQ_WORKSPACE_BYTES)


def test_stream_read_rejects():
    L = kq.lib()
    assert L.kq_stream_read(None, 1024, A16, None) == 1
    assert L.kq_stream_read(A16, 1024, None, None) == 1
    assert L.kq_stream_read(A16 + 8, 1024, A16, None) == 3
    assert L.kq_stream_read(A16, 1000, A16, None) == 3
    assert L.kq_stream_read(A16, 0, A16, None) == 0          # nothing to read: nothing enqueued
