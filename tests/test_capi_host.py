"""The C ABI on the host (no GPU needed): libswa.so loads, exports every
function include/swa.h declares, and rejects bad arguments before any HIP
call (every check below returns without touching a device)."""
import ctypes
import os
import re

import pytest

from sliding_window_gqa_swa_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared_functions():
    names = []
    for f in os.listdir(os.path.join(ROOT, "include")):
        if f.endswith(".h"):
            src = open(os.path.join(ROOT, "include", f)).read()
            names += re.findall(r"SWA_API\s+[\w\s\*]+?\b(swa_\w+)\s*\(", src)
    return sorted(set(names))


def test_library_exports_every_declared_symbol():
    names = _declared_functions()
    assert len(names) >= 7
    lib = ctypes.CDLL(_lib.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(_lib.SIGNATURES), "binding and header disagree"


def test_strerror_codes():
    L = _lib.lib()
    for code in (0, -1, -2, -3, -4, -5, -99):
        assert len(L.swa_strerror(code)) > 0


# fake 16-byte-aligned "device" addresses: the calls below must fail in
# host-side validation, before any pointer is dereferenced or any kernel runs
A = 0x10000
B = 0x20000


def _prefill(**kw):
    args = dict(q=A, k=A, v=A, cu=B, ids=None, window=16, mode=0, out=A, T=10, nd=1, hq=4,
                hkv=2, d=128, dtype=0, scale=0.0)
    args.update(kw)
    return _lib.lib().swa_prefill(args["q"], args["k"], args["v"], args["cu"], args["ids"],
                                  args["window"], args["mode"], args["out"], args["T"], args["nd"],
                                  args["hq"], args["hkv"], args["d"], args["dtype"], args["scale"],
                                  None)


@pytest.mark.parametrize("kw,code", [
    (dict(d=100), _lib.SWA_EUNSUPPORTED),
    (dict(d=96), _lib.SWA_EUNSUPPORTED),
    (dict(d=576), _lib.SWA_EUNSUPPORTED),
    (dict(d=0), _lib.SWA_EUNSUPPORTED),
    (dict(dtype=7), _lib.SWA_EUNSUPPORTED),
    (dict(mode=2), _lib.SWA_EUNSUPPORTED),
    (dict(hq=3, hkv=2), _lib.SWA_EINVAL),
    (dict(hkv=0), _lib.SWA_EINVAL),
    (dict(T=-1), _lib.SWA_EINVAL),
    (dict(nd=0), _lib.SWA_EINVAL),
    (dict(q=None), _lib.SWA_EINVAL),
    (dict(out=A + 8), _lib.SWA_EINVAL),
    (dict(cu=None), _lib.SWA_EINVAL),
    (dict(mode=1, ids=None), _lib.SWA_EINVAL),
])
def test_prefill_rejects(kw, code):
    assert _prefill(**kw) == code


def _prefill_chunk(**kw):
    a = dict(q=A, k=A, v=A, cuq=B, cuk=B, ids=None, window=0, mode=0, out=A, Tq=10, Tk=20,
             nd=1, hq=4, hkv=2, d=128, dtype=0)
    a.update(kw)
    return _lib.lib().swa_prefill_chunk(a["q"], a["k"], a["v"], a["cuq"], a["cuk"], a["ids"],
                                        a["window"], a["mode"], a["out"], a["Tq"], a["Tk"],
                                        a["nd"], a["hq"], a["hkv"], a["d"], a["dtype"], 0.0, None)


@pytest.mark.parametrize("kw,code", [
    (dict(cuk=None), _lib.SWA_EINVAL),
    (dict(cuq=None), _lib.SWA_EINVAL),
    (dict(Tk=0), _lib.SWA_EINVAL),
    (dict(Tk=-1), _lib.SWA_EINVAL),
    (dict(d=96), _lib.SWA_EUNSUPPORTED),
    (dict(mode=1), _lib.SWA_EINVAL),
    (dict(mode=2), _lib.SWA_EUNSUPPORTED),
    (dict(k=A + 2), _lib.SWA_EINVAL),
])
def test_prefill_chunk_rejects(kw, code):
    assert _prefill_chunk(**kw) == code


@pytest.mark.parametrize("d", (64, 128, 192, 256, 320, 384, 448, 512))
def test_every_multiple_of_64_passes_every_size_check(d):
    """Every multiple of 64 from 64 to 512 passes the head-size checks of
    every entry point (each call below fails on a later check, or is an
    empty no-op)."""
    assert _prefill_chunk(d=d, Tq=0, q=None, out=None) == _lib.SWA_OK
    assert _prefill_chunk(d=d, cuk=None) == _lib.SWA_EINVAL  # checked past the size
    assert _decode(d=d, ws=None) == _lib.SWA_EWORKSPACE
    assert _decode_step(d=d, ws=None) == _lib.SWA_EWORKSPACE
    assert _noalloc(d=d, out=None) == _lib.SWA_EINVAL
    L = _lib.lib()
    assert L.swa_decode_workspace_bytes(2, 8, 4, d, 1088) > 0
    assert L.swa_cache_append(A, A, A, A, B, 0, 1088, 4, d, 0, None) == _lib.SWA_OK
    assert L.swa_cache_roll(A, A, B, 1024, 0, 1088, 4, d, 0, None) == _lib.SWA_OK


@pytest.mark.parametrize("d", (32, 96, 100, 160, 200, 480, 576, 640, 1024))
def test_other_head_sizes_are_rejected_everywhere(d):
    """Sizes that are not a multiple of 64, or above 512, are refused by
    every entry point with SWA_EUNSUPPORTED."""
    L = _lib.lib()
    for call in (_decode, _decode_step, _noalloc):
        assert call(d=d) == _lib.SWA_EUNSUPPORTED
    assert _prefill_chunk(d=d) == _lib.SWA_EUNSUPPORTED
    assert L.swa_decode_workspace_bytes(2, 8, 4, d, 1088) == 0
    assert L.swa_cache_append(A, A, A, A, B, 2, 1088, 4, d, 0, None) == _lib.SWA_EUNSUPPORTED
    assert L.swa_cache_roll(A, A, B, 1024, 2, 1088, 4, d, 0, None) == _lib.SWA_EUNSUPPORTED


def test_prefill_chunk_empty_is_a_no_op():
    assert _prefill_chunk(Tq=0, q=None, out=None) == _lib.SWA_OK


def test_prefill_empty_is_a_no_op():
    assert _prefill(T=0, q=None, k=None, v=None, out=None, cu=None) == _lib.SWA_OK


def _backward(**kw):
    a = dict(q=A, k=A, v=A, out=A, dout=A, cu=B, ids=None, window=16, mode=0, lse=None, dq=A,
             dk=A, dv=A,
             T=10, nd=1, hq=4, hkv=2, d=128, dtype=0, ws=A, wsb=1 << 30)
    a.update(kw)
    return _lib.lib().swa_prefill_backward(
        a["q"], a["k"], a["v"], a["out"], a["dout"], a["cu"], a["ids"], a["window"], a["mode"],
        a["lse"], a["dq"], a["dk"], a["dv"], a["T"], a["nd"], a["hq"], a["hkv"], a["d"], a["dtype"], 0.0,
        a["ws"], a["wsb"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(d=96), _lib.SWA_EUNSUPPORTED),
    (dict(d=576), _lib.SWA_EUNSUPPORTED),
    (dict(d=0), _lib.SWA_EUNSUPPORTED),
    (dict(dtype=7), _lib.SWA_EUNSUPPORTED),
    (dict(mode=2), _lib.SWA_EUNSUPPORTED),
    (dict(hq=3, hkv=2), _lib.SWA_EINVAL),
    (dict(T=-1), _lib.SWA_EINVAL),
    (dict(nd=0), _lib.SWA_EINVAL),
    (dict(dout=None), _lib.SWA_EINVAL),
    (dict(out=A + 4), _lib.SWA_EINVAL),
    (dict(dk=None), _lib.SWA_EINVAL),
    (dict(cu=None), _lib.SWA_EINVAL),
    (dict(mode=1, ids=None), _lib.SWA_EINVAL),
    (dict(ws=None), _lib.SWA_EWORKSPACE),
    (dict(wsb=16), _lib.SWA_EWORKSPACE),
    (dict(ws=A + 8), _lib.SWA_EWORKSPACE),
    (dict(lse=B + 2), _lib.SWA_EINVAL),
])
def test_prefill_backward_rejects(kw, code):
    assert _backward(**kw) == code


def test_prefill_backward_sizes():
    """Empty input is a no-op; every supported head size passes the size
    checks (a call with too little workspace gets past them); the
    workspace holds two fp32 rows of statistics per head and two int32
    intervals per token."""
    assert _backward(T=0, q=None, dq=None, ws=None) == _lib.SWA_OK
    for d in (64, 128, 192, 256, 320, 384, 448, 512):
        assert _backward(d=d, wsb=0) == _lib.SWA_EWORKSPACE
    for d in (64, 128, 192, 256, 320, 384, 448, 512):
        assert _backward(d=d, dtype=1, wsb=0) == _lib.SWA_EWORKSPACE
    for d in (96, 160, 576):
        assert _backward(d=d) == _lib.SWA_EUNSUPPORTED
    L = _lib.lib()
    for T, hq in ((1, 1), (4096, 32), (16384, 16)):
        n = L.swa_prefill_backward_workspace_bytes(T, hq)
        assert n >= 8 * T * hq + 8 * T and n % 256 == 0
    assert L.swa_prefill_backward_workspace_bytes(-1, 4) == 0


def test_prefill_lse_rejects():
    L = _lib.lib()

    def call(lse, T=10, d=128):
        return L.swa_prefill_lse(A, A, A, B, None, 16, 0, A, lse, T, 1, 4, 2, d, 0, 0.0, None)
    assert call(None) == _lib.SWA_EINVAL
    assert call(B + 2) == _lib.SWA_EINVAL
    assert call(B, d=96) == _lib.SWA_EUNSUPPORTED
    assert call(None, T=0) == _lib.SWA_OK


def _decode(**kw):
    a = dict(q=A, k=A, v=A, meta=B, window=1024, out=A, b=2, R=1088, hq=8, hkv=4, d=256,
             dtype=0, ws=A, wsb=1 << 30)
    a.update(kw)
    return _lib.lib().swa_decode(a["q"], a["k"], a["v"], a["meta"], a["window"], a["out"], a["b"],
                                 a["R"], a["hq"], a["hkv"], a["d"], a["dtype"], 0.0, a["ws"],
                                 a["wsb"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(window=0), _lib.SWA_EINVAL),
    (dict(R=1024), _lib.SWA_EINVAL),
    (dict(R=70000, window=1024), _lib.SWA_EUNSUPPORTED),
    (dict(d=96), _lib.SWA_EUNSUPPORTED),
    (dict(meta=None), _lib.SWA_EINVAL),
    (dict(ws=None), _lib.SWA_EWORKSPACE),
    (dict(wsb=16), _lib.SWA_EWORKSPACE),
    (dict(hq=6, hkv=4), _lib.SWA_EINVAL),
])
def test_decode_rejects(kw, code):
    assert _decode(**kw) == code


def _decode_step(**kw):
    a = dict(q=A, kn=A, vn=A, k=A, v=A, meta=B, window=1024, out=A, b=2, R=1088, hq=8, hkv=4,
             d=256, dtype=0, ws=A, wsb=1 << 30)
    a.update(kw)
    return _lib.lib().swa_decode_step(a["q"], a["kn"], a["vn"], a["k"], a["v"], a["meta"],
                                      a["window"], a["out"], a["b"], a["R"], a["hq"], a["hkv"],
                                      a["d"], a["dtype"], 0.0, a["ws"], a["wsb"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(window=0), _lib.SWA_EINVAL),
    (dict(R=1024), _lib.SWA_EINVAL),
    (dict(R=70000, window=1024), _lib.SWA_EUNSUPPORTED),
    (dict(d=96), _lib.SWA_EUNSUPPORTED),
    (dict(dtype=3), _lib.SWA_EUNSUPPORTED),
    (dict(kn=None), _lib.SWA_EINVAL),
    (dict(vn=A + 4), _lib.SWA_EINVAL),
    (dict(meta=None), _lib.SWA_EINVAL),
    (dict(ws=None), _lib.SWA_EWORKSPACE),
    (dict(wsb=16), _lib.SWA_EWORKSPACE),
    (dict(hq=6, hkv=4), _lib.SWA_EINVAL),
])
def test_decode_step_rejects(kw, code):
    assert _decode_step(**kw) == code


def test_decode_step_empty_batch_is_a_no_op():
    assert _decode_step(b=0, q=None, kn=None, vn=None, k=None, v=None, meta=None, out=None,
                        ws=None, wsb=0) == _lib.SWA_OK


def test_decode_workspace_depends_only_on_sizes():
    L = _lib.lib()
    a = L.swa_decode_workspace_bytes(64, 8, 4, 256, 1088)
    assert a > 0 and a == L.swa_decode_workspace_bytes(64, 8, 4, 256, 1088)
    assert L.swa_decode_workspace_bytes(0, 8, 4, 256, 1088) == 0
    assert L.swa_decode_workspace_bytes(1, 8, 4, 100, 1088) == 0


def _decode_ws(batch, hq, hkv, d, splits, head_blocks=1):
    """Workspace of a decode plan with the given splits per ring: the
    counters (one per sequence, kv head and head block, plus one per
    sequence, rounded up to 256 bytes), then (m, l, o[d]) in fp32 per
    sequence, query head and split."""
    counters = (batch * (hkv * head_blocks + 1) * 4 + 255) // 256 * 256
    return counters + batch * hq * splits * (d + 2) * 4


def test_decode_plan_splits():
    """The split plan, read back through the workspace size: 64 sequences
    of 4 kv heads (256 blocks) take one split per 1088-row ring; a single
    sequence takes 64-row splits (17 per ring); a 65536-row ring takes at
    most 2048 rows per split (32)."""
    L = _lib.lib()
    assert L.swa_decode_workspace_bytes(64, 8, 4, 256, 1088) == _decode_ws(64, 8, 4, 256, 1)
    assert L.swa_decode_workspace_bytes(1, 4, 2, 256, 1088) == _decode_ws(1, 4, 2, 256, 17)
    assert L.swa_decode_workspace_bytes(2, 8, 4, 256, 65536) == _decode_ws(2, 8, 4, 256, 32)


def test_ring_ops_reject():
    L = _lib.lib()
    # append: bad d / null meta
    assert L.swa_cache_append(A, A, A, A, B, 2, 1088, 4, 100, 0, None) == _lib.SWA_EUNSUPPORTED
    assert L.swa_cache_append(A, A, A, A, None, 2, 1088, 4, 256, 0, None) == _lib.SWA_EINVAL
    assert L.swa_cache_append(A, A, A, A, B, 0, 1088, 4, 256, 0, None) == _lib.SWA_OK
    # compact: ring no larger than the window
    assert L.swa_cache_compact(A, A, B, None, None, 10, A, A, B, 1088, 2, 1088, 4, 256, 0,
                               None) == _lib.SWA_EINVAL
    assert L.swa_cache_compact(A, A, None, None, None, 10, A, A, B, 1024, 2, 1088, 4, 256, 0,
                               None) == _lib.SWA_EINVAL
    # roll: window < 1
    assert L.swa_cache_roll(A, A, B, 0, 2, 1088, 4, 256, 0, None) == _lib.SWA_EINVAL
    assert L.swa_cache_roll(A, A, B, 1024, 2, 1088, 4, 256, 5, None) == _lib.SWA_EUNSUPPORTED


def test_binding_refuses_cpu_tensors():
    import torch
    from sliding_window_gqa_swa_amd import api
    q = torch.zeros(4, 2, 64, dtype=torch.bfloat16)
    cu = torch.tensor([0, 4], dtype=torch.int32)
    with pytest.raises(ValueError, match="GPU"):
        api.prefill(q, q[:, :1].contiguous(), q[:, :1].contiguous(), cu)


def _noalloc(**kw):
    a = dict(q=A, kn=A, vn=A, kr=A, vr=A, meta=B, W=1024, out=A, B=1, R=1088, hq=4, hkv=2, d=256,
             dtype=0)
    a.update(kw)
    return _lib.lib().swa_decode_step_noalloc(a["q"], a["kn"], a["vn"], a["kr"], a["vr"], a["meta"],
                                              a["W"], a["out"], a["B"], a["R"], a["hq"], a["hkv"],
                                              a["d"], a["dtype"], 0.0, None)


@pytest.mark.parametrize("kw,code", [
    (dict(d=160), _lib.SWA_EUNSUPPORTED),
    (dict(R=1024), _lib.SWA_EINVAL),
    (dict(hq=3), _lib.SWA_EINVAL),
    (dict(out=None), _lib.SWA_EINVAL),
    (dict(meta=B + 4), _lib.SWA_EINVAL),
    # partials of 256 sequences x 32 heads x 2 splits x 514 floats: 16.8 MB,
    # more than the 8 MiB static scratch
    (dict(B=256, hq=32, hkv=8, d=512), _lib.SWA_ESCRATCH),
])
def test_decode_step_noalloc_rejects(kw, code):
    assert _noalloc(**kw) == code
