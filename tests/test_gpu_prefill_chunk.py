"""GPU chunked prefill (a chunk of each document's queries against the
document's keys so far) against the fp64 oracle, through the C ABI."""
import numpy as np
import pytest
import torch

import swa_inputs as si
from oracle import oracle as orc
from sliding_window_gqa_swa_amd import api

from gpu_util import as_f64, assert_close, dev, host, log, require_gpu
from test_gpu_prefill import _ids_for

pytestmark = pytest.mark.gpu

CAUSAL, BLOCKWISE = si.CAUSAL, si.BLOCKWISE


def _chunk(q, k, v, cu_q, cu_k, ids, W, mode):
    out = api.prefill_chunk(dev(q), dev(k), dev(v), dev(cu_q), dev(cu_k),
                            None if ids is None else dev(ids), W, mode)
    torch.cuda.synchronize()
    return host(out)


def _ragged_chunks(rng, d):
    """Documents of ragged key lengths; chunks of 0, 1, all, and random
    lengths, spanning several query and key tiles."""
    lk = np.array([1, 130, 7, 300, 257, 64] if d <= 256 else [1, 90, 7, 200, 65], np.int64)
    lq = np.array([1, 0, 7, 129, 100, 64] if d <= 256 else [1, 0, 7, 77, 33], np.int64)
    cu_k = np.concatenate([[0], np.cumsum(lk)]).astype(np.int32)
    cu_q = np.concatenate([[0], np.cumsum(lq)]).astype(np.int32)
    return cu_q, cu_k


# (kv heads, query heads per kv head) per head size: groups of 2, 4 and 8
# (4 or 8 heads share each K/V tile in one work-group)
GROUPS = {64: (1, 8), 128: (1, 4), 192: (2, 2), 256: (2, 2), 320: (1, 4), 384: (2, 2), 448: (1, 4),
          512: (1, 4)}

CASES = [(d, dt, m) for d in (64, 128, 192, 256, 320, 384, 448, 512) for dt in ("bf16", "f32")
         for m in (CAUSAL, BLOCKWISE)]


@pytest.mark.parametrize("d,dtype,mode", CASES)
def test_chunk_small_ragged(d, dtype, mode):
    require_gpu()
    rng = si.rng_for(30 * d + (dtype == "f32") * 7 + mode)
    cu_q, cu_k = _ragged_chunks(rng, d)
    Tq, Tk = int(cu_q[-1]), int(cu_k[-1])
    hkv, g = GROUPS[d]
    q = si.normal(rng, (Tq, hkv * g, d), dtype)
    k = si.normal(rng, (Tk, hkv, d), dtype)
    v = si.normal(rng, (Tk, hkv, d), dtype)
    ids = _ids_for(Tk, cu_k, 40 + d) if mode == BLOCKWISE else None
    for W in (0, 37, 200):
        log("chunk small d=%d %s mode=%d W=%d Tq=%d Tk=%d" % (d, dtype, mode, W, Tq, Tk))
        got = _chunk(q, k, v, cu_q, cu_k, ids, W, mode)
        want = orc.prefill_chunk(q, k, v, cu_q, cu_k, ids, W, mode)
        assert_close(got, want, dtype, "chunk d=%d %s mode=%d W=%d" % (d, dtype, mode, W))


@pytest.mark.parametrize("d", [128, 512])
def test_causal_chunks_equal_whole_prompt_rows(d):
    """A prompt prefilled in chunks gives, chunk by chunk, the rows of the
    whole-prompt prefill (to the bf16 tolerance of each other: tiles differ)."""
    require_gpu()
    rng = si.rng_for(600 + d)
    L, hkv, g, W = 700, 2, 2, 150
    q = si.normal(rng, (L, hkv * g, d), "bf16")
    k = si.normal(rng, (L, hkv, d), "bf16")
    v = si.normal(rng, (L, hkv, d), "bf16")
    whole = as_f64(host(api.prefill(dev(q), dev(k), dev(v), dev(np.array([0, L], np.int32)),
                                    None, W, CAUSAL)))
    for o, c in ((0, 256), (256, 256), (512, 188)):
        log("chunk vs whole d=%d chunk %d..%d" % (d, o, o + c))
        got = _chunk(q[o:o + c], k[:o + c], v[:o + c], np.array([0, c], np.int32),
                     np.array([0, o + c], np.int32), None, W, CAUSAL)
        err = np.abs(as_f64(got) - whole[o:o + c])
        assert err.max() <= 2e-2 and err.mean() <= 2e-3, (o, err.max(), err.mean())


def test_chunk_cuts_image_at_cache_end():
    """An image that continues past the cached keys: chunk rows inside it see
    only its cached part (the oracle's reading), not its later tokens."""
    require_gpu()
    rng = si.rng_for(77)
    L, hkv, g, d = 300, 1, 2, 128
    ids = np.full(L, -1, np.int32)
    ids[100:260] = 0
    q = si.normal(rng, (L, hkv * g, d), "f32")
    k = si.normal(rng, (L, hkv, d), "f32")
    v = si.normal(rng, (L, hkv, d), "f32")
    o, c = 64, 128  # queries 64..191, keys 0..191: the image is cut at 191
    got = _chunk(q[o:o + c], k[:o + c], v[:o + c], np.array([0, c], np.int32),
                 np.array([0, o + c], np.int32), ids[:o + c], 0, BLOCKWISE)
    want = orc.prefill_chunk(q[o:o + c], k[:o + c], v[:o + c], [0, c], [0, o + c], ids[:o + c],
                             0, BLOCKWISE)
    assert_close(got, want, "f32", "image cut")


def test_chunk_of_16k_gqa_d512_window_4096_sampled_rows():
    """The 16384-token D=512 GQA workload's last 2048 tokens as one chunk
    against all 16384 keys, on sampled rows (chunk start, window edges,
    random rows)."""
    require_gpu()
    c = si.PREFILL_WORKLOADS["prefill_16k_gqa_d512"]()
    q, k, v = c.tensors("bf16")
    o = c.T - 2048
    qc = np.ascontiguousarray(q[o:])
    cu_q = np.array([0, 2048], np.int32)
    log("chunk 16k d512 last 2048")
    got = _chunk(qc, k, v, cu_q, c.cu_seqlens, None, c.window, CAUSAL)
    rng = si.rng_for(8)
    rows = np.array(sorted({0, 1, 2047, 1024, 1023} | set(int(x) for x in rng.integers(0, 2048, 12))),
                    np.int32)
    want = orc.prefill_chunk(qc, k, v, cu_q, c.cu_seqlens, None, c.window, CAUSAL, rows=rows)
    assert_close(got[rows], want, "bf16", "16k chunk")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_chunked_prefill_then_compact_then_decode(dtype):
    """The serving flow of [SPYRE] Summary end to end on the GPU: three
    prompts of ragged lengths are prefilled in 256-token chunks into one
    packed prompt-sized cache (each chunk against its document's keys so
    far), the rings are compacted directly from that cache, and fused decode
    steps run past a roll.  Every chunk's rows are checked against the
    oracle's whole-prompt prefill rows, every step against the oracle's
    decode on the linear history."""
    require_gpu()
    rng = si.rng_for(4242)
    lens = [700, 1200, 301]
    hq, hkv, d, W, A, C = 4, 2, 128, 512, 64, 256
    R = W + A
    B = len(lens)
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    T = int(cu[-1])
    q = si.normal(rng, (T, hq, d), dtype)
    k = si.normal(rng, (T, hkv, d), dtype)
    v = si.normal(rng, (T, hkv, d), dtype)
    kd, vd = dev(k), dev(v)
    # chunk j of every prompt that still has rows: queries [j C, min((j+1) C, L))
    want_all = orc.prefill(q, k, v, cu, None, W, CAUSAL)
    for j in range((max(lens) + C - 1) // C):
        rows, cuq, cuk = [], [0], [0]
        for b, L in enumerate(lens):
            a, e = min(j * C, L), min((j + 1) * C, L)
            rows += list(range(int(cu[b]) + a, int(cu[b]) + e))
            cuq.append(cuq[-1] + (e - a))
            cuk.append(cuk[-1] + e)
        if not rows:
            break
        rows = np.array(rows, np.int64)
        # each document's keys so far, packed: its first e rows
        kidx = np.concatenate([np.arange(int(cu[b]), int(cu[b]) + min((j + 1) * C, L))
                               for b, L in enumerate(lens)])
        log("chunk %d %s rows %d" % (j, dtype, rows.size))
        out = api.prefill_chunk(dev(q[rows]), dev(k[kidx]), dev(v[kidx]),
                                dev(np.array(cuq, np.int32)), dev(np.array(cuk, np.int32)),
                                None, W, CAUSAL)
        assert_close(host(out), want_all[rows], dtype, "chunk %d" % j)
    # compaction straight from the packed prompt cache, then decode steps
    kr = torch.zeros((B, hkv, R, d), dtype=kd.dtype, device="cuda")
    vr = torch.zeros_like(kr)
    meta = torch.zeros((B, 4), dtype=torch.int32, device="cuda")
    api.cache_compact(kd, vd, dev(cu), kr, vr, meta, W, dev(np.array(lens, np.int32)), None)
    hist_k = [k[cu[b]:cu[b + 1]] for b in range(B)]
    hist_v = [v[cu[b]:cu[b + 1]] for b in range(B)]
    pos = np.array(lens, np.int64) - 1
    for s in range(A + 6):  # the 64th append after compaction needs the roll
        qn = si.normal(rng, (B, hq, d), dtype)
        kn = si.normal(rng, (B, hkv, d), dtype)
        vn = si.normal(rng, (B, hkv, d), dtype)
        log("decode step %d %s" % (s, dtype))
        out = api.decode_step(dev(qn), dev(kn), dev(vn), kr, vr, meta, W)
        pos += 1
        for b in range(B):
            hist_k[b] = np.concatenate([hist_k[b], kn[b:b + 1]])
            hist_v[b] = np.concatenate([hist_v[b], vn[b:b + 1]])
        off = np.concatenate([[0], np.cumsum([h.shape[0] for h in hist_k])[:-1]])
        want = orc.decode_linear(qn, np.concatenate(hist_k), np.concatenate(hist_v), off,
                                 [0] * B, [h.shape[0] for h in hist_k], pos, [0] * B, W)
        assert_close(host(out), want, dtype, "decode step %d" % s)
    m = host(meta)
    assert not (m[:, 3] < 0).any(), "a sequence overflowed its ring"
    assert (m[:, 0] == pos).all()
