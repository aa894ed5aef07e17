"""Python face of libswa: the C entry points under the same names, taking
``torch.Tensor`` arguments.

Argument marshalling only -- every step of attention and of the ring cache
runs in the HIP kernels behind the C ABI.  torch supplies device memory and
the current stream; nothing here computes on the host.  Tensors must be
contiguous, on a ROCm device, and of the element type the call names
(bfloat16 or float32; int32 for lengths, ids and ring_meta).
"""
import torch

from . import _lib
from ._lib import SWA_BF16, SWA_BLOCKWISE, SWA_CAUSAL, SWA_F32, SWA_META_ERR  # noqa: F401

CAUSAL = SWA_CAUSAL
BLOCKWISE = SWA_BLOCKWISE


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return SWA_BF16
    if t.dtype == torch.float32:
        return SWA_F32
    raise TypeError("expected bfloat16 or float32, got %s" % t.dtype)


def _dev(t: torch.Tensor, name: str, dtype=None) -> int:
    """Device pointer of a contiguous GPU tensor (0 for None)."""
    if t is None:
        return 0
    if not t.is_cuda:
        raise ValueError("%s must be a GPU tensor (libswa has no CPU path)" % name)
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    if dtype is not None and t.dtype != dtype:
        raise TypeError("%s must be %s, got %s" % (name, dtype, t.dtype))
    return t.data_ptr()


def _stream(t: torch.Tensor) -> int:
    return torch.cuda.current_stream(t.device).cuda_stream


def prefill(q, k, v, cu_seqlens, doc_or_block_ids=None, window=0, causal_mode=CAUSAL,
            out=None, scale=0.0):
    """Packed varlen sliding-window GQA prefill; see swa_prefill in swa.h.

    q [T, Hq, D], k/v [T, Hkv, D] (bf16 or fp32), cu_seqlens int32 [ndocs+1],
    doc_or_block_ids int32 [T] (BLOCKWISE only).  Returns out [T, Hq, D]."""
    T, hq, d = q.shape
    hkv = k.shape[1]
    if k.shape != (T, hkv, d) or v.shape != (T, hkv, d):
        raise ValueError("k and v must be [T, Hkv, D] matching q")
    if out is None:
        out = torch.empty_like(q)
    dt = _dtype_code(q)
    for name, t in (("k", k), ("v", v), ("out", out)):
        if t.dtype != q.dtype:
            raise TypeError("%s dtype differs from q" % name)
    rc = _lib.lib().swa_prefill(
        _dev(q, "q"), _dev(k, "k"), _dev(v, "v"), _dev(cu_seqlens, "cu_seqlens", torch.int32),
        _dev(doc_or_block_ids, "doc_or_block_ids", torch.int32), int(window), int(causal_mode),
        _dev(out, "out"), T, cu_seqlens.numel() - 1, hq, hkv, d, dt, float(scale), _stream(q))
    _lib.check("swa_prefill", rc)
    return out


def prefill_lse(q, k, v, cu_seqlens, doc_or_block_ids=None, window=0, causal_mode=CAUSAL,
                out=None, lse=None, scale=0.0):
    """prefill that also returns each row's log-sum-exp; see swa_prefill_lse
    in swa.h.  Returns (out [T, Hq, D], lse float32 [Hq, T])."""
    T, hq, d = q.shape
    hkv = k.shape[1]
    if k.shape != (T, hkv, d) or v.shape != (T, hkv, d):
        raise ValueError("k and v must be [T, Hkv, D] matching q")
    out = torch.empty_like(q) if out is None else out
    lse = torch.empty((hq, T), dtype=torch.float32, device=q.device) if lse is None else lse
    if lse.shape != (hq, T):
        raise ValueError("lse must be [Hq, T]")
    dt = _dtype_code(q)
    for name, t in (("k", k), ("v", v), ("out", out)):
        if t.dtype != q.dtype:
            raise TypeError("%s dtype differs from q" % name)
    rc = _lib.lib().swa_prefill_lse(
        _dev(q, "q"), _dev(k, "k"), _dev(v, "v"), _dev(cu_seqlens, "cu_seqlens", torch.int32),
        _dev(doc_or_block_ids, "doc_or_block_ids", torch.int32), int(window), int(causal_mode),
        _dev(out, "out"), _dev(lse, "lse", torch.float32), T, cu_seqlens.numel() - 1, hq, hkv, d,
        dt, float(scale), _stream(q))
    _lib.check("swa_prefill_lse", rc)
    return out, lse


def prefill_chunk(q, k, v, cu_seqlens_q, cu_seqlens_k, doc_or_block_ids=None, window=0,
                  causal_mode=CAUSAL, out=None, scale=0.0):
    """Prefill of one chunk of each document against its cache so far; see
    swa_prefill_chunk in swa.h.

    q [Tq, Hq, D] (document b's rows are the last cu_q[b+1]-cu_q[b] of its
    cu_k[b+1]-cu_k[b] key positions); k/v [Tk, Hkv, D]; doc_or_block_ids
    int32 [Tk] (BLOCKWISE only).  Returns out [Tq, Hq, D]."""
    Tq, hq, d = q.shape
    Tk, hkv = k.shape[0], k.shape[1]
    if k.shape != (Tk, hkv, d) or v.shape != (Tk, hkv, d):
        raise ValueError("k and v must be [Tk, Hkv, D] with q's D")
    if cu_seqlens_q.numel() != cu_seqlens_k.numel():
        raise ValueError("cu_seqlens_q and cu_seqlens_k must have one entry per document + 1")
    if out is None:
        out = torch.empty_like(q)
    dt = _dtype_code(q)
    for name, t in (("k", k), ("v", v), ("out", out)):
        if t.dtype != q.dtype:
            raise TypeError("%s dtype differs from q" % name)
    rc = _lib.lib().swa_prefill_chunk(
        _dev(q, "q"), _dev(k, "k"), _dev(v, "v"), _dev(cu_seqlens_q, "cu_seqlens_q", torch.int32),
        _dev(cu_seqlens_k, "cu_seqlens_k", torch.int32),
        _dev(doc_or_block_ids, "doc_or_block_ids", torch.int32), int(window), int(causal_mode),
        _dev(out, "out"), Tq, Tk, cu_seqlens_q.numel() - 1, hq, hkv, d, dt, float(scale),
        _stream(q))
    _lib.check("swa_prefill_chunk", rc)
    return out


def prefill_backward_workspace_bytes(total_tokens, hq) -> int:
    return int(_lib.lib().swa_prefill_backward_workspace_bytes(total_tokens, hq))


def prefill_backward(q, k, v, out, dout, cu_seqlens, doc_or_block_ids=None, window=0,
                     causal_mode=CAUSAL, dq=None, dk=None, dv=None, workspace=None, scale=0.0,
                     lse=None):
    """Gradients (dq, dk, dv) of prefill for the loss sum(dout * out); see
    swa_prefill_backward in swa.h.  out is prefill's output for the same
    arguments, dout the gradient at out (both [T, Hq, D]); lse optionally
    the forward's row log-sum-exp from prefill_lse ([Hq, T] float32).
    Returns (dq [T, Hq, D], dk [T, Hkv, D], dv [T, Hkv, D])."""
    T, hq, d = q.shape
    hkv = k.shape[1]
    if k.shape != (T, hkv, d) or v.shape != (T, hkv, d):
        raise ValueError("k and v must be [T, Hkv, D] matching q")
    if out.shape != q.shape or dout.shape != q.shape:
        raise ValueError("out and dout must be [T, Hq, D] like q")
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    dt = _dtype_code(q)
    for name, t in (("k", k), ("v", v), ("out", out), ("dout", dout), ("dq", dq), ("dk", dk),
                    ("dv", dv)):
        if t.dtype != q.dtype:
            raise TypeError("%s dtype differs from q" % name)
    nbytes = prefill_backward_workspace_bytes(T, hq)
    if workspace is None:
        workspace = torch.empty(max(nbytes, 16), dtype=torch.uint8, device=q.device)
    rc = _lib.lib().swa_prefill_backward(
        _dev(q, "q"), _dev(k, "k"), _dev(v, "v"), _dev(out, "out"), _dev(dout, "dout"),
        _dev(cu_seqlens, "cu_seqlens", torch.int32),
        _dev(doc_or_block_ids, "doc_or_block_ids", torch.int32), int(window), int(causal_mode),
        _dev(lse, "lse", torch.float32),
        _dev(dq, "dq"), _dev(dk, "dk"), _dev(dv, "dv"), T, cu_seqlens.numel() - 1, hq, hkv, d, dt,
        float(scale), _dev(workspace, "workspace"), workspace.numel() * workspace.element_size(),
        _stream(q))
    _lib.check("swa_prefill_backward", rc)
    return dq, dk, dv


def decode_workspace_bytes(batch, hq, hkv, d, ring_rows) -> int:
    return int(_lib.lib().swa_decode_workspace_bytes(batch, hq, hkv, d, ring_rows))


def decode_workspace(q, k_ring) -> torch.Tensor:
    """A zero-filled workspace of the size swa_decode needs for these shapes
    (zero once; swa_decode leaves its counters at zero after every call)."""
    B, hq, d = q.shape
    nbytes = decode_workspace_bytes(B, hq, k_ring.shape[1], d, k_ring.shape[2])
    return torch.zeros(max(nbytes, 16) // 4 + 4, dtype=torch.float32, device=q.device)


def decode(q, k_ring, v_ring, ring_meta, window, out=None, workspace=None, scale=0.0):
    """One-token decode against compact rings; see swa_decode in swa.h.

    q [B, Hq, D]; k_ring/v_ring [B, Hkv, R, D]; ring_meta int32 [B, 4]."""
    B, hq, d = q.shape
    _, hkv, R, _ = k_ring.shape
    if out is None:
        out = torch.empty_like(q)
    if workspace is None:
        workspace = decode_workspace(q, k_ring)
    rc = _lib.lib().swa_decode(
        _dev(q, "q"), _dev(k_ring, "k_ring"), _dev(v_ring, "v_ring"),
        _dev(ring_meta, "ring_meta", torch.int32), int(window), _dev(out, "out"), B, R, hq, hkv, d,
        _dtype_code(q), float(scale), _dev(workspace, "workspace"),
        workspace.numel() * workspace.element_size(), _stream(q))
    _lib.check("swa_decode", rc)
    return out


def decode_step(q, k_new, v_new, k_ring, v_ring, ring_meta, window, out=None, workspace=None,
                scale=0.0):
    """Roll (by metadata, when a ring is full), append and decode in one
    launch; see swa_decode_step in swa.h.

    q [B, Hq, D]; k_new/v_new [B, Hkv, D]; k_ring/v_ring [B, Hkv, R, D];
    ring_meta int32 [B, 4] (updated in place).  Returns out [B, Hq, D]."""
    B, hq, d = q.shape
    _, hkv, R, _ = k_ring.shape
    if k_new.shape != (B, hkv, d) or v_new.shape != (B, hkv, d):
        raise ValueError("k_new and v_new must be [B, Hkv, D]")
    if out is None:
        out = torch.empty_like(q)
    if workspace is None:
        workspace = decode_workspace(q, k_ring)
    rc = _lib.lib().swa_decode_step(
        _dev(q, "q"), _dev(k_new, "k_new"), _dev(v_new, "v_new"), _dev(k_ring, "k_ring"),
        _dev(v_ring, "v_ring"), _dev(ring_meta, "ring_meta", torch.int32), int(window),
        _dev(out, "out"), B, R, hq, hkv, d, _dtype_code(q), float(scale),
        _dev(workspace, "workspace"), workspace.numel() * workspace.element_size(), _stream(q))
    _lib.check("swa_decode_step", rc)
    return out


def decode_step_noalloc(q, k_new, v_new, k_ring, v_ring, ring_meta, window, out=None, scale=0.0):
    """decode_step with the library's static scratch instead of a workspace
    (nothing is allocated when `out` is given); see swa_decode_step_noalloc
    in swa.h.  Raises with SWA_ESCRATCH for sizes beyond the scratch."""
    B, hq, d = q.shape
    _, hkv, R, _ = k_ring.shape
    if k_new.shape != (B, hkv, d) or v_new.shape != (B, hkv, d):
        raise ValueError("k_new and v_new must be [B, Hkv, D]")
    if out is None:
        out = torch.empty_like(q)
    rc = _lib.lib().swa_decode_step_noalloc(
        _dev(q, "q"), _dev(k_new, "k_new"), _dev(v_new, "v_new"), _dev(k_ring, "k_ring"),
        _dev(v_ring, "v_ring"), _dev(ring_meta, "ring_meta", torch.int32), int(window),
        _dev(out, "out"), B, R, hq, hkv, d, _dtype_code(q), float(scale), _stream(q))
    _lib.check("swa_decode_step_noalloc", rc)
    return out


def cache_append(k_new, v_new, k_ring, v_ring, ring_meta):
    """Write one token per sequence at position pos + 1; see swa_cache_append."""
    B, hkv, R, d = k_ring.shape
    rc = _lib.lib().swa_cache_append(
        _dev(k_new, "k_new"), _dev(v_new, "v_new"), _dev(k_ring, "k_ring"), _dev(v_ring, "v_ring"),
        _dev(ring_meta, "ring_meta", torch.int32), B, R, hkv, d, _dtype_code(k_ring),
        _stream(k_ring))
    _lib.check("swa_cache_append", rc)


def cache_compact(k_src, v_src, cu_seqlens, k_ring, v_ring, ring_meta, window,
                  prompt_lens=None, left_pad=None):
    """Build rings from packed prompt rows; see swa_cache_compact."""
    B, hkv, R, d = k_ring.shape
    rc = _lib.lib().swa_cache_compact(
        _dev(k_src, "k_src"), _dev(v_src, "v_src"), _dev(cu_seqlens, "cu_seqlens", torch.int32),
        _dev(prompt_lens, "prompt_lens", torch.int32), _dev(left_pad, "left_pad", torch.int32),
        k_src.shape[0], _dev(k_ring, "k_ring"), _dev(v_ring, "v_ring"),
        _dev(ring_meta, "ring_meta", torch.int32), int(window), B, R, hkv, d,
        _dtype_code(k_ring), _stream(k_ring))
    _lib.check("swa_cache_compact", rc)


def cache_roll(k_ring, v_ring, ring_meta, window):
    """Roll every full ring by ring_rows - window rows; see swa_cache_roll."""
    B, hkv, R, d = k_ring.shape
    rc = _lib.lib().swa_cache_roll(
        _dev(k_ring, "k_ring"), _dev(v_ring, "v_ring"), _dev(ring_meta, "ring_meta", torch.int32),
        int(window), B, R, hkv, d, _dtype_code(k_ring), _stream(k_ring))
    _lib.check("swa_cache_roll", rc)
