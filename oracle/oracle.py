"""Python face of the CPU oracle (fp64).  TEST INFRASTRUCTURE ONLY.

Only ``tests/``, the smoke check and the CPU-baseline leg of ``bench.py`` may
import this module.  It shares no code with the GPU library: it takes numpy
arrays (bf16 bit patterns as ``uint16`` or ``float32``) and returns float64.

Pages cited (title; section):
  [SPYRE]  "Enable compact sliding-window attention for Gemma 3 and Gemma 4
           variants" (torch-spyre/hf-adapters pull request 496)
  [BONSAI] "Gemma3 Local Attention Cache" (jax-ml/bonsai issue 124)
  [SDPA]   "Add SDPA attention implementation" (Fast-LLM pull request 512)
"""
import ctypes
import os

import numpy as np

from . import build as _build

CAUSAL = 0
BLOCKWISE = 1

_lib = None


def _load():
    global _lib
    if _lib is None:
        path = _build.build(force=False)
        lib = ctypes.CDLL(path)
        P, I, D = ctypes.c_void_p, ctypes.c_int, ctypes.c_double
        lib.oracle_prefill_rows.argtypes = [P, P, P, I, P, I, P, I, I, I, I, I, I, D, P, I, P, P, I]
        lib.oracle_prefill_rows.restype = I
        lib.oracle_decode_linear.argtypes = [P, P, P, I, P, P, P, P, P, I, I, I, I, I, D, P, I]
        lib.oracle_decode_linear.restype = I
        lib.oracle_prefill_backward.argtypes = [P, P, P, P, I, P, I, P, I, I, I, I, I, I, D,
                                                P, I, P, I, P, P, P, I]
        lib.oracle_prefill_backward.restype = I
        lib.oracle_count_allowed.argtypes = [P, I, P, I, I, I, I]
        lib.oracle_count_allowed.restype = ctypes.c_longlong
        lib.oracle_allowed.argtypes = [P, I, P, I, I, I, I]
        lib.oracle_allowed.restype = I
        lib.oracle_max_threads.argtypes = []
        lib.oracle_max_threads.restype = I
        _lib = lib
    return _lib


def _dtype_code(a):
    if a.dtype == np.uint16:
        return 0
    if a.dtype == np.float32:
        return 1
    raise TypeError("oracle inputs are bf16 bit patterns (uint16) or float32, got %s" % a.dtype)


def _ptr(a):
    return a.ctypes.data_as(ctypes.c_void_p) if a is not None else None


def max_threads() -> int:
    return _load().oracle_max_threads()


def prefill(q, k, v, cu_seqlens, ids=None, window=0, mode=CAUSAL, scale=None,
            rows=None, nthreads=0, return_lse=False):
    """Packed varlen SWA prefill in fp64.

    q [T, Hq, D], k/v [T, Hkv, D] (uint16 bf16 bits or float32); cu_seqlens
    int32 [ndocs+1].  ``rows`` selects packed query indices (default: all).
    Returns float64 [len(rows), Hq, D]; with ``return_lse`` also each row's
    log-sum-exp log(sum_j exp(scale * <q, k_j>)) over its allowed keys,
    float64 [len(rows), Hq].  ``scale`` defaults to 1/sqrt(D).
    """
    q = np.ascontiguousarray(q)
    k = np.ascontiguousarray(k)
    v = np.ascontiguousarray(v)
    dt = _dtype_code(q)
    assert _dtype_code(k) == dt and _dtype_code(v) == dt
    T, hq, d = q.shape
    hkv = k.shape[1]
    assert k.shape == (T, hkv, d) and v.shape == (T, hkv, d)
    cu = np.ascontiguousarray(cu_seqlens, dtype=np.int32)
    ids_a = None if ids is None else np.ascontiguousarray(ids, dtype=np.int32)
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    rows_a = None if rows is None else np.ascontiguousarray(rows, dtype=np.int32)
    n = T if rows_a is None else rows_a.size
    out = np.empty((n, hq, d), dtype=np.float64)
    lse = np.empty((n, hq), dtype=np.float64) if return_lse else None
    rc = _load().oracle_prefill_rows(
        _ptr(q), _ptr(k), _ptr(v), dt, _ptr(cu), cu.size - 1, _ptr(ids_a),
        int(window), int(mode), T, hq, hkv, d, float(scale), _ptr(rows_a), n,
        _ptr(out), _ptr(lse), int(nthreads))
    if rc != 0:
        raise ValueError("oracle_prefill_rows rejected its arguments (rc=%d)" % rc)
    return (out, lse) if return_lse else out


def prefill_chunk(q, k, v, cu_q, cu_k, ids=None, window=0, mode=CAUSAL, scale=None,
                  rows=None, nthreads=0):
    """Prefill of a chunk of each document against its cache so far, fp64.

    [SPYRE] Summary: chunked prefill is preserved.  Document b's keys are
    its first len_k = cu_k[b+1] - cu_k[b] positions and its queries the last
    len_q = cu_q[b+1] - cu_q[b] of them; the mask is the prefill mask over
    positions 0 .. len_k - 1 of the document.  That is, by definition, the
    prefill of the documents cut at len_k, read at the chunk's rows: the
    chunk rows are placed at their key positions of a key-length query array
    (other rows unused) and only they are computed.  ids are key-indexed.
    ``rows`` selects packed chunk rows (default: all).
    Returns float64 [len(rows), Hq, D]."""
    q = np.ascontiguousarray(q)
    cq = np.asarray(cu_q, dtype=np.int64)
    ck = np.asarray(cu_k, dtype=np.int64)
    Tk = int(ck[-1])
    _, hq, d = q.shape
    full = np.zeros((Tk, hq, d), dtype=q.dtype)
    keyrow = np.empty(q.shape[0], np.int64)  # key row of every chunk row
    for b in range(cq.size - 1):
        nq, ke = int(cq[b + 1] - cq[b]), int(ck[b + 1])
        if nq > ke - int(ck[b]):
            raise ValueError("document %d: more queries than keys" % b)
        full[ke - nq:ke] = q[cq[b]:cq[b + 1]]
        keyrow[cq[b]:cq[b + 1]] = np.arange(ke - nq, ke)
    sel = keyrow if rows is None else keyrow[np.asarray(rows, dtype=np.int64)]
    if sel.size == 0:
        return np.zeros((0, hq, d), dtype=np.float64)
    return prefill(full, k, v, ck.astype(np.int32), ids, window, mode, scale,
                   rows=sel.astype(np.int32), nthreads=nthreads)


def prefill_backward(q, k, v, dout, cu_seqlens, ids=None, window=0, mode=CAUSAL,
                     scale=None, rows=None, keys=None, nthreads=0):
    """Gradients of the packed varlen SWA prefill, fp64.

    For the loss sum(dout * out) (dout [T, Hq, D], the gradient arriving at
    the output) returns (dq [len(rows), Hq, D], dk [len(keys), Hkv, D],
    dv [len(keys), Hkv, D]) as float64, by the chain rule through the
    prefill's definition (the forward recomputed per row in fp64).  ``rows``
    selects the packed query rows of dq and ``keys`` the packed key rows of
    dk and dv (default: all).  Inputs as for ``prefill``; dout has q's dtype.
    """
    q = np.ascontiguousarray(q)
    k = np.ascontiguousarray(k)
    v = np.ascontiguousarray(v)
    dout = np.ascontiguousarray(dout)
    dt = _dtype_code(q)
    assert _dtype_code(k) == dt and _dtype_code(v) == dt and _dtype_code(dout) == dt
    T, hq, d = q.shape
    hkv = k.shape[1]
    assert k.shape == (T, hkv, d) and v.shape == (T, hkv, d) and dout.shape == q.shape
    cu = np.ascontiguousarray(cu_seqlens, dtype=np.int32)
    ids_a = None if ids is None else np.ascontiguousarray(ids, dtype=np.int32)
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    rows_a = None if rows is None else np.ascontiguousarray(rows, dtype=np.int32)
    keys_a = None if keys is None else np.ascontiguousarray(keys, dtype=np.int32)
    nr = T if rows_a is None else rows_a.size
    nk = T if keys_a is None else keys_a.size
    # an empty selection still passes a (dummy) array: NULL means "all"
    if rows_a is not None and nr == 0:
        rows_a = np.zeros(1, np.int32)
    if keys_a is not None and nk == 0:
        keys_a = np.zeros(1, np.int32)
    dq = np.empty((nr, hq, d), dtype=np.float64)
    dk = np.empty((nk, hkv, d), dtype=np.float64)
    dv = np.empty((nk, hkv, d), dtype=np.float64)
    rc = _load().oracle_prefill_backward(
        _ptr(q), _ptr(k), _ptr(v), _ptr(dout), dt, _ptr(cu), cu.size - 1, _ptr(ids_a),
        int(window), int(mode), T, hq, hkv, d, float(scale), _ptr(rows_a), nr,
        _ptr(keys_a), nk, _ptr(dq), _ptr(dk), _ptr(dv), int(nthreads))
    if rc != 0:
        raise ValueError("oracle_prefill_backward rejected its arguments (rc=%d)" % rc)
    return dq, dk, dv


def decode_linear(q, k_hist, v_hist, hist_off, first_pos, hist_len, pos, lo,
                  window, scale=None, nthreads=0):
    """One-token decode per sequence on linear histories, fp64.

    q [B, Hq, D]; k_hist/v_hist [rows, Hkv, D]; sequence b owns rows
    hist_off[b] .. hist_off[b]+hist_len[b]-1 holding positions first_pos[b]..
    Returns float64 [B, Hq, D].
    """
    q = np.ascontiguousarray(q)
    k_hist = np.ascontiguousarray(k_hist)
    v_hist = np.ascontiguousarray(v_hist)
    dt = _dtype_code(q)
    B, hq, d = q.shape
    hkv = k_hist.shape[1]
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    off = np.ascontiguousarray(hist_off, dtype=np.int64)
    fp = np.ascontiguousarray(first_pos, dtype=np.int32)
    hl = np.ascontiguousarray(hist_len, dtype=np.int32)
    ps = np.ascontiguousarray(pos, dtype=np.int32)
    lo_a = np.ascontiguousarray(lo, dtype=np.int32)
    out = np.empty((B, hq, d), dtype=np.float64)
    rc = _load().oracle_decode_linear(
        _ptr(q), _ptr(k_hist), _ptr(v_hist), dt, _ptr(off), _ptr(fp), _ptr(hl),
        _ptr(ps), _ptr(lo_a), int(window), B, hq, hkv, d, float(scale), _ptr(out),
        int(nthreads))
    if rc != 0:
        raise ValueError("oracle_decode_linear rejected its arguments (rc=%d)" % rc)
    return out


def count_allowed(cu_seqlens, ids=None, window=0, mode=CAUSAL, nthreads=0):
    """Number of admitted (query, key) pairs, counted pair by pair."""
    cu = np.ascontiguousarray(cu_seqlens, dtype=np.int32)
    ids_a = None if ids is None else np.ascontiguousarray(ids, dtype=np.int32)
    return int(_load().oracle_count_allowed(_ptr(cu), cu.size - 1, _ptr(ids_a),
                                            int(window), int(mode), int(cu[-1]),
                                            int(nthreads)))


def allowed(cu_seqlens, ids, window, mode, i, j):
    """The oracle's mask for one (query i, key j) pair, as a bool."""
    cu = np.ascontiguousarray(cu_seqlens, dtype=np.int32)
    ids_a = None if ids is None else np.ascontiguousarray(ids, dtype=np.int32)
    return bool(_load().oracle_allowed(_ptr(cu), cu.size - 1, _ptr(ids_a), int(window),
                                       int(mode), int(i), int(j)))
