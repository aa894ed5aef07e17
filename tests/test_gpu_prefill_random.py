"""Seeded random sweep of prefill and chunked-prefill shapes against the
fp64 oracle, every output element compared.

Each case draws its own head size (every supported multiple of 64), GQA
group (1, 2, 3, 4 or 8 query heads per kv head), document lengths (empty,
one-token and ragged documents, up to 3000 tokens in all, 1600 from head
size 320),
window (unlimited, 1, tile-edge values around 64 and 128, or random), mask
mode and element type, so that shapes the hand-written cases do not name
(odd groups with blockwise masks, windows one key either side of a tile
edge, chunks that start inside a tile) are still covered.  The draws are a
function of the case number only, and each case is logged before it runs.
"""
import numpy as np
import pytest
import torch

import swa_inputs as si
from oracle import oracle as orc
from sliding_window_gqa_swa_amd import api

from gpu_util import assert_close, dev, host, log, require_gpu

pytestmark = pytest.mark.gpu

CAUSAL, BLOCKWISE = si.CAUSAL, si.BLOCKWISE
HEAD_SIZES = (64, 128, 192, 256, 320, 384, 448, 512)
WINDOWS = (0, 1, 63, 64, 65, 127, 128, 129)


def _draw(case: int):
    rng = si.rng_for(7000 + case)
    d = HEAD_SIZES[case % len(HEAD_SIZES)]
    g = int(rng.choice([1, 2, 3, 4, 8]))
    hkv = int(rng.integers(1, 3))
    ndocs = int(rng.integers(1, 6))
    cap = 3000 if d <= 256 else 1600  # tokens in all (the oracle takes < 1 s)
    lens = rng.integers(0, cap // ndocs + 1, size=ndocs)
    if case % 3 == 0:
        lens[int(rng.integers(0, ndocs))] = 1
    W = int(WINDOWS[int(rng.integers(0, len(WINDOWS)))]) if rng.random() < 0.6 \
        else int(rng.integers(2, 1500))
    mode = BLOCKWISE if rng.random() < 0.4 else CAUSAL
    dtype = "f32" if rng.random() < 0.25 else "bf16"
    return rng, d, g, hkv, lens.astype(np.int64), W, mode, dtype


def _ids(rng, T):
    """Image runs of random lengths at random places (ids distinct per run)."""
    ids = np.full(T, -1, np.int32)
    pos, nid = 0, 0
    while pos < T:
        pos += int(rng.integers(0, 60))
        ln = int(rng.integers(1, 140))
        if pos >= T:
            break
        ids[pos:pos + ln] = nid
        nid += 1
        pos += ln
    return ids


def _name(case, d, g, hkv, lens, W, mode, dtype):
    return "case %d: d=%d hq=%d hkv=%d docs=%s W=%d mode=%d %s" % (
        case, d, g * hkv, hkv, lens.tolist(), W, mode, dtype)


@pytest.mark.parametrize("case", range(32))
def test_prefill_random_shapes(case):
    require_gpu()
    rng, d, g, hkv, lens, W, mode, dtype = _draw(case)
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    T = int(cu[-1])
    if T == 0:
        lens[0] = 1
        cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
        T = 1
    hq = g * hkv
    q = si.normal(rng, (T, hq, d), dtype)
    k = si.normal(rng, (T, hkv, d), dtype)
    v = si.normal(rng, (T, hkv, d), dtype)
    ids = _ids(rng, T) if mode == BLOCKWISE else None
    what = _name(case, d, g, hkv, lens, W, mode, dtype)
    log("prefill random " + what)
    out = api.prefill(dev(q), dev(k), dev(v), dev(cu), None if ids is None else dev(ids), W, mode)
    torch.cuda.synchronize()
    want = orc.prefill(q, k, v, cu, ids, W, mode)
    assert_close(host(out), want, dtype, what)


@pytest.mark.parametrize("case", range(16))
def test_prefill_chunk_random_shapes(case):
    """Each document's last len_q positions against its first len_k keys
    (a chunk of 0 .. len_k rows that may start inside a tile)."""
    require_gpu()
    rng, d, g, hkv, lens, W, mode, dtype = _draw(100 + case)
    lens = np.maximum(lens, 1)
    lq = np.array([int(rng.integers(0, int(n) + 1)) for n in lens], np.int64)
    cu_k = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    cu_q = np.concatenate([[0], np.cumsum(lq)]).astype(np.int32)
    Tk, Tq = int(cu_k[-1]), int(cu_q[-1])
    if Tq == 0:
        lq[0] = 1
        cu_q = np.concatenate([[0], np.cumsum(lq)]).astype(np.int32)
        Tq = 1
    hq = g * hkv
    q = si.normal(rng, (Tq, hq, d), dtype)
    k = si.normal(rng, (Tk, hkv, d), dtype)
    v = si.normal(rng, (Tk, hkv, d), dtype)
    ids = _ids(rng, Tk) if mode == BLOCKWISE else None
    what = _name(100 + case, d, g, hkv, lens, W, mode, dtype) + " chunks=%s" % lq.tolist()
    log("prefill chunk random " + what)
    out = api.prefill_chunk(dev(q), dev(k), dev(v), dev(cu_q), dev(cu_k),
                            None if ids is None else dev(ids), W, mode)
    torch.cuda.synchronize()
    want = orc.prefill_chunk(q, k, v, cu_q, cu_k, ids, W, mode)
    assert_close(host(out), want, dtype, what)
