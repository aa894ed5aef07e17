"""Pins of the CPU oracle to things other than itself (CPU only).

Each test fixes the oracle against what the pages or mathematics determine:
closed forms, a library routine (torch SDPA on CPU in fp64), brute force on
tiny inputs and hand-derived worked examples in tests/golden/.  The mistakes
each one catches are named in its docstring.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import swa_inputs as si
from oracle import oracle as orc

CAUSAL, BLOCKWISE = orc.CAUSAL, orc.BLOCKWISE


def _f64(a):
    return si.bf16_bits_to_f32(a).astype(np.float64) if a.dtype == np.uint16 else a.astype(np.float64)


def _rand(shape, seed, dtype="f32"):
    return si.normal(si.rng_for(seed), shape, dtype)


# ----------------------------------------------------------------- mask
def test_vlm_mask_golden(golden_dir):
    """Hand-listed allowed sets: catches a symmetric window, a missing
    future same-image allowance, a same-image key beyond the window being
    admitted, merging two runs of one id, and cross-document leakage."""
    fx = json.load(open(os.path.join(golden_dir, "vlm_mask_small.json")))
    for case in fx["cases"]:
        cu = np.array(case["cu_seqlens"], np.int32)
        ids = np.array(case["ids"], np.int32)
        T = int(cu[-1])
        for mode, key in ((BLOCKWISE, "blockwise_allowed"), (CAUSAL, "causal_allowed")):
            for i in range(T):
                got = [j for j in range(T) if orc.allowed(cu, ids, case["window"], mode, i, j)]
                assert got == case[key][i], (case["name"], key, i)


def test_vlm_mask_golden_through_attention(golden_dir):
    """With K = 0 every admitted key gets the same weight, so each output row
    is the plain mean of V over the hand-listed set (catches a mask that is
    right in oracle_allowed but not used by the attention path)."""
    fx = json.load(open(os.path.join(golden_dir, "vlm_mask_small.json")))
    for case in fx["cases"]:
        cu = np.array(case["cu_seqlens"], np.int32)
        ids = np.array(case["ids"], np.int32)
        T = int(cu[-1])
        q = _rand((T, 2, 8), 11)
        k = np.zeros((T, 1, 8), np.float32)
        v = _rand((T, 1, 8), 12)
        for mode, key in ((BLOCKWISE, "blockwise_allowed"), (CAUSAL, "causal_allowed")):
            out = orc.prefill(q, k, v, cu, ids, case["window"], mode)
            for i in range(T):
                want = v[case[key][i], 0, :].astype(np.float64).mean(axis=0)
                for h in range(2):
                    np.testing.assert_allclose(out[i, h], want, rtol=0, atol=1e-14)


def _causal_window_pairs(n, W):
    """Closed form of sum_{i<n} min(i+1, W) (W <= 0: no window)."""
    if W <= 0 or W >= n:
        return n * (n + 1) // 2
    return W * (W + 1) // 2 + (n - W) * W


def test_allowed_pair_counts_closed_form():
    """Pair counts of the three prefill workloads against closed forms:
    catches an inclusive window (i - j <= W), a two-sided window on future
    image keys, and documents leaking into each other."""
    c2 = si.prefill_4x1024_mha_d128()
    assert orc.count_allowed(c2.cu_seqlens, None, c2.window, CAUSAL) == 4 * 524800
    assert 4 * _causal_window_pairs(1024, 1024) == 4 * 524800
    c5 = si.prefill_vlm_4096_d256()
    future_in_blocks = 8 * (256 * 255 // 2)
    want5 = _causal_window_pairs(4096, 1024) + future_in_blocks
    assert want5 == 3931648
    assert orc.count_allowed(c5.cu_seqlens, c5.ids, c5.window, BLOCKWISE) == want5
    assert orc.count_allowed(c5.cu_seqlens, c5.ids, c5.window, CAUSAL) == _causal_window_pairs(4096, 1024)
    # the 16384-token, W=4096 document: 58,722,304 pairs per head
    assert _causal_window_pairs(16384, 4096) == 58722304
    cu = np.array([0, 16384], np.int32)
    assert orc.count_allowed(cu, None, 4096, CAUSAL) == 58722304
    # ragged documents with a window shorter than some of them
    cu = np.array([0, 5, 5, 40, 41, 100], np.int32)
    for W in (0, 1, 3, 7, 64):
        want = sum(_causal_window_pairs(int(b - a), W) for a, b in zip(cu[:-1], cu[1:]))
        assert orc.count_allowed(cu, None, W, CAUSAL) == want


# ----------------------------------------------------------------- attention closed forms
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_window_one_is_identity(dtype):
    """W = 1 admits only the query itself: O[i, h] = V[i, h // g] exactly
    (weight 1, sum 1).  Catches an inclusive window and a wrong GQA map."""
    cu = np.array([0, 7, 20, 21, 33], np.int32)
    T = 33
    q = _rand((T, 4, 16), 1, dtype)
    k = _rand((T, 2, 16), 2, dtype)
    v = _rand((T, 2, 16), 3, dtype)
    out = orc.prefill(q, k, v, cu, None, 1, CAUSAL)
    vf = _f64(v)
    for h in range(4):
        np.testing.assert_array_equal(out[:, h, :], vf[:, h // 2, :])


def test_zero_keys_give_window_mean():
    """K = 0 makes the softmax uniform, so O[i] = mean of V over keys
    max(doc_start, i - W + 1) .. i, a closed form.  Catches window and
    document boundary errors and a wrong normaliser."""
    cu = np.array([0, 9, 30, 31, 64], np.int32)
    T = 64
    q = _rand((T, 2, 8), 4)
    k = np.zeros((T, 2, 8), np.float32)
    v = _rand((T, 2, 8), 5)
    for W in (0, 1, 2, 5, 16, 100):
        out = orc.prefill(q, k, v, cu, None, W, CAUSAL)
        for dd in range(4):
            s, e = int(cu[dd]), int(cu[dd + 1])
            for i in range(s, e):
                a = s if W <= 0 else max(s, i - W + 1)
                want = v[a:i + 1].astype(np.float64).mean(axis=0)
                np.testing.assert_allclose(out[i], want, rtol=0, atol=1e-14)


def test_two_key_softmax_closed_form():
    """Two keys with scores 0 and s: weights 1/(1+e^s) and e^s/(1+e^s),
    s = <q, k1> / sqrt(D).  Catches a wrong scale (1/D, none) and a sign
    error in the exponent."""
    D = 4
    q = np.zeros((2, 1, D), np.float32)
    q[1, 0, 0] = 3.0
    k = np.zeros((2, 1, D), np.float32)
    k[1, 0, 0] = 0.5  # token 1's key: score = 3 * 0.5 / 2 = 0.75
    v = np.zeros((2, 1, D), np.float32)
    v[0, 0, :] = [1, 0, 0, 0]
    v[1, 0, :] = [0, 1, 0, 0]
    out = orc.prefill(q, k, v, np.array([0, 2], np.int32), None, 0, CAUSAL)
    s = 0.75
    w1 = math.exp(s) / (1 + math.exp(s))
    np.testing.assert_allclose(out[1, 0], [1 - w1, w1, 0, 0], rtol=0, atol=1e-15)
    np.testing.assert_allclose(out[0, 0], [1, 0, 0, 0], rtol=0, atol=0)


def _sdpa_causal_fp64(q, k, v):
    """torch SDPA (CPU, fp64, is_causal) on one document; K/V repeated per
    query head with repeat_interleave, the GQA form the SDPA page uses."""
    g = q.shape[1] // k.shape[1]
    qt = torch.from_numpy(_f64(q)).permute(1, 0, 2).unsqueeze(0)
    kt = torch.from_numpy(_f64(k)).repeat_interleave(g, dim=1).permute(1, 0, 2).unsqueeze(0)
    vt = torch.from_numpy(_f64(v)).repeat_interleave(g, dim=1).permute(1, 0, 2).unsqueeze(0)
    o = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, is_causal=True)
    return o.squeeze(0).permute(1, 0, 2).numpy()


@pytest.mark.parametrize("hq,hkv,D", [(2, 2, 16), (4, 2, 32), (8, 2, 8)])
def test_wide_window_equals_torch_causal(hq, hkv, D):
    """A window at least as long as every document equals textbook causal
    attention per document (library routine: torch SDPA, fp64).  Catches a
    dropped or misindexed term in the dot product or the weighted sum, and a
    transposed operand."""
    cu = np.array([0, 17, 50, 51, 96], np.int32)
    T = 96
    q = _rand((T, hq, D), 21, "bf16")
    k = _rand((T, hkv, D), 22, "bf16")
    v = _rand((T, hkv, D), 23, "bf16")
    for W in (0, 45, 1000):
        out = orc.prefill(q, k, v, cu, None, W, CAUSAL)
        for dd in range(4):
            s, e = int(cu[dd]), int(cu[dd + 1])
            want = _sdpa_causal_fp64(q[s:e], k[s:e], v[s:e])
            np.testing.assert_allclose(out[s:e], want, rtol=0, atol=1e-12)


def test_packed_equals_separate_documents():
    """Packing documents must not change any row: the packed result equals
    each document run alone, bit for bit (both modes)."""
    rng = si.rng_for(31)
    cu = np.array([0, 13, 14, 40, 64], np.int32)
    ids = np.full(64, -1, np.int32)
    ids[3:8] = 0
    ids[20:30] = 1
    ids[41:50] = 2
    q = _rand((64, 4, 8), 32, "bf16")
    k = _rand((64, 2, 8), 33, "bf16")
    v = _rand((64, 2, 8), 34, "bf16")
    for mode in (CAUSAL, BLOCKWISE):
        packed = orc.prefill(q, k, v, cu, ids, 6, mode)
        for dd in range(4):
            s, e = int(cu[dd]), int(cu[dd + 1])
            one = orc.prefill(q[s:e], k[s:e], v[s:e], np.array([0, e - s], np.int32), ids[s:e], 6, mode)
            np.testing.assert_array_equal(packed[s:e], one)
    del rng


def test_gqa_equals_repeated_mha():
    """Grouped heads equal multi-head attention on K/V repeated with
    repeat_interleave (query head h reads kv head h // g), bit for bit."""
    cu = np.array([0, 30, 50], np.int32)
    q = _rand((50, 6, 8), 41, "bf16")
    k = _rand((50, 2, 8), 42, "bf16")
    v = _rand((50, 2, 8), 43, "bf16")
    ids = np.full(50, -1, np.int32)
    ids[10:20] = 4
    for mode in (CAUSAL, BLOCKWISE):
        gqa = orc.prefill(q, k, v, cu, ids, 7, mode)
        mha = orc.prefill(q, np.repeat(k, 3, axis=1), np.repeat(v, 3, axis=1), cu, ids, 7, mode)
        np.testing.assert_array_equal(gqa, mha)


def _brute_force(q, k, v, cu, ids, W, mode):
    """Dense T x T boolean mask and a dense fp64 softmax over all keys."""
    T, hq, D = q.shape
    g = hq // k.shape[1]
    doc = np.searchsorted(cu, np.arange(T), side="right") - 1
    run = np.zeros(T, np.int64)
    for t in range(1, T):
        run[t] = run[t - 1] + int(ids[t] != ids[t - 1] or doc[t] != doc[t - 1])
    i = np.arange(T)[:, None]
    j = np.arange(T)[None, :]
    m = doc[:, None] == doc[None, :]
    if W > 0:
        m &= (i - j) < W
    fut = np.zeros((T, T), bool)
    if mode == BLOCKWISE:
        fut = (ids[:, None] >= 0) & (run[:, None] == run[None, :])
    m &= (j <= i) | fut
    qf, kf, vf = _f64(q), _f64(k), _f64(v)
    out = np.zeros((T, hq, D))
    for h in range(hq):
        s = qf[:, h, :] @ kf[:, h // g, :].T / math.sqrt(D)
        s = np.where(m, s, -np.inf)
        mx = s.max(axis=1, keepdims=True)
        mx = np.where(np.isfinite(mx), mx, 0.0)
        p = np.exp(s - mx)
        l = p.sum(axis=1, keepdims=True)
        out[:, h, :] = np.where(l > 0, (p @ vf[:, h // g, :]) / np.where(l > 0, l, 1), 0.0)
    return out


@pytest.mark.parametrize("trial", range(12))
def test_brute_force_random_tiny(trial):
    """Random tiny shapes, both modes, several windows and group sizes:
    oracle == explicit-mask dense softmax within 1e-12."""
    rng = si.rng_for(1000 + trial)
    T = int(rng.integers(1, 64))
    nd = int(rng.integers(1, 5))
    cu = si.ragged_cu_seqlens(rng, T, nd)
    hkv = int(rng.choice([1, 2]))
    g = int(rng.choice([1, 2, 4]))
    D = int(rng.choice([4, 8, 16]))
    ids = np.full(T, -1, np.int32)
    for b in range(int(rng.integers(0, 4))):
        s = int(rng.integers(0, T))
        e = min(T, s + int(rng.integers(1, 12)))
        ids[s:e] = b
    q = _rand((T, hkv * g, D), 2000 + trial, "bf16")
    k = _rand((T, hkv, D), 3000 + trial, "bf16")
    v = _rand((T, hkv, D), 4000 + trial, "bf16")
    for W in (1, 2, 3, 5, T, T + 7, 0):
        for mode in (CAUSAL, BLOCKWISE):
            got = orc.prefill(q, k, v, cu, ids, W, mode)
            want = _brute_force(q, k, v, cu, ids, W, mode)
            np.testing.assert_allclose(got, want, rtol=0, atol=1e-12)


def test_rows_subset_equals_full():
    """Computing selected rows gives the same bits as the full run."""
    c = si.PrefillCase("t", np.array([0, 40, 90], np.int32), 4, 2, 16, 9, CAUSAL, seed=7)
    q, k, v = c.tensors("bf16")
    full = orc.prefill(q, k, v, c.cu_seqlens, None, c.window, CAUSAL)
    rows = np.array([0, 39, 40, 41, 89, 5], np.int32)
    np.testing.assert_array_equal(orc.prefill(q, k, v, c.cu_seqlens, None, c.window, CAUSAL, rows=rows), full[rows])


# ----------------------------------------------------------------- chunked prefill
def _brute_force_chunk(q, k, v, cu_q, cu_k, ids, W, mode):
    """Dense (query row x key row) mask in key positions: query row i of
    document b sits at position len_k - len_q + i of b; a dense fp64 softmax
    over all key rows."""
    Tq, hq, D = q.shape
    Tk = k.shape[0]
    g = hq // k.shape[1]
    cu_q, cu_k = np.asarray(cu_q), np.asarray(cu_k)
    kdoc = np.searchsorted(cu_k, np.arange(Tk), side="right") - 1
    qdoc = np.searchsorted(cu_q, np.arange(Tq), side="right") - 1
    qpos = np.arange(Tq) - cu_q[qdoc] + (cu_k[qdoc + 1] - cu_k[qdoc]) - (cu_q[qdoc + 1] - cu_q[qdoc])
    qkey = cu_k[qdoc] + qpos  # key row of each query
    run = np.zeros(Tk, np.int64)
    for t in range(1, Tk):
        run[t] = run[t - 1] + int(ids[t] != ids[t - 1] or kdoc[t] != kdoc[t - 1])
    i = qkey[:, None]
    j = np.arange(Tk)[None, :]
    m = qdoc[:, None] == kdoc[None, :]
    if W > 0:
        m &= (i - j) < W
    fut = np.zeros((Tq, Tk), bool)
    if mode == BLOCKWISE:
        fut = (ids[qkey][:, None] >= 0) & (run[qkey][:, None] == run[None, :])
    m &= (j <= i) | fut
    qf, kf, vf = _f64(q), _f64(k), _f64(v)
    out = np.zeros((Tq, hq, D))
    for h in range(hq):
        s = qf[:, h, :] @ kf[:, h // g, :].T / math.sqrt(D)
        s = np.where(m, s, -np.inf)
        mx = s.max(axis=1, keepdims=True)
        mx = np.where(np.isfinite(mx), mx, 0.0)
        p = np.exp(s - mx)
        l = p.sum(axis=1, keepdims=True)
        out[:, h, :] = np.where(l > 0, (p @ vf[:, h // g, :]) / np.where(l > 0, l, 1), 0.0)
    return out


@pytest.mark.parametrize("trial", range(8))
def test_chunk_brute_force_random_tiny(trial):
    """Chunks of random length (0 .. len_k) of random documents, both modes:
    the chunk oracle == a dense key-position mask within 1e-12."""
    rng = si.rng_for(5000 + trial)
    nd = int(rng.integers(1, 4))
    lk = rng.integers(1, 30, size=nd)
    lq = np.array([int(rng.integers(0, x + 1)) for x in lk])
    cu_k = np.concatenate([[0], np.cumsum(lk)]).astype(np.int32)
    cu_q = np.concatenate([[0], np.cumsum(lq)]).astype(np.int32)
    Tk, Tq = int(cu_k[-1]), int(cu_q[-1])
    hkv, g, D = int(rng.choice([1, 2])), int(rng.choice([1, 2])), 8
    ids = np.full(Tk, -1, np.int32)
    for b in range(int(rng.integers(0, 4))):
        s0 = int(rng.integers(0, Tk))
        ids[s0:min(Tk, s0 + int(rng.integers(1, 10)))] = b
    q = _rand((Tq, hkv * g, D), 6000 + trial, "bf16")
    k = _rand((Tk, hkv, D), 7000 + trial, "bf16")
    v = _rand((Tk, hkv, D), 8000 + trial, "bf16")
    for W in (1, 3, 7, 0):
        for mode in (CAUSAL, BLOCKWISE):
            got = orc.prefill_chunk(q, k, v, cu_q, cu_k, ids, W, mode)
            want = _brute_force_chunk(q, k, v, cu_q, cu_k, ids, W, mode)
            np.testing.assert_allclose(got, want, rtol=0, atol=1e-12)


def test_causal_chunk_equals_rows_of_the_whole_document():
    """CAUSAL: a chunk at positions o .. o+c-1 of a document, against keys
    0 .. o+c-1, gives the rows o .. o+c-1 of the prefill of the WHOLE
    document (the later keys are never allowed), for any window."""
    hq, hkv, D = 4, 2, 16
    L = 70
    q = _rand((L, hq, D), 91, "bf16")
    k = _rand((L, hkv, D), 92, "bf16")
    v = _rand((L, hkv, D), 93, "bf16")
    for W in (0, 1, 9, 33):
        whole = orc.prefill(q, k, v, np.array([0, L], np.int32), None, W, CAUSAL)
        for o, c in ((0, 70), (0, 10), (10, 25), (50, 20), (69, 1)):
            got = orc.prefill_chunk(q[o:o + c], k[:o + c], v[:o + c], [0, c], [0, o + c],
                                    None, W, CAUSAL)
            np.testing.assert_array_equal(got, whole[o:o + c])


def test_chunk_blockwise_cuts_image_at_cache_end():
    """BLOCKWISE: a chunk whose last image run continues past the cached keys
    sees only the cached part of it: its rows equal those of the prefill of
    the document cut at the cache end, and differ from the whole document's
    rows (which see the image's later tokens)."""
    hq, hkv, D, W = 2, 1, 8, 0
    L = 20
    ids = np.full(L, -1, np.int32)
    ids[8:16] = 0  # one image, tokens 8..15
    q = _rand((L, hq, D), 94, "bf16")
    k = _rand((L, hkv, D), 95, "bf16")
    v = _rand((L, hkv, D), 96, "bf16")
    o, c = 6, 6  # queries 6..11, keys 0..11: the image is cut after token 11
    got = orc.prefill_chunk(q[o:o + c], k[:o + c], v[:o + c], [0, c], [0, o + c], ids[:o + c],
                            W, BLOCKWISE)
    cut = orc.prefill(q[:o + c], k[:o + c], v[:o + c], np.array([0, o + c], np.int32),
                      ids[:o + c], W, BLOCKWISE)
    whole = orc.prefill(q, k, v, np.array([0, L], np.int32), ids, W, BLOCKWISE)
    np.testing.assert_array_equal(got, cut[o:])
    assert np.abs(got[2:] - whole[o + 2:o + c]).max() > 1e-3  # image rows 8..11 differ
    np.testing.assert_array_equal(got[:2], whole[o:o + 2])  # text rows 6, 7 do not


# ----------------------------------------------------------------- decode on a linear cache
def test_decode_linear_equals_prefill_last_row():
    """Decode of the token at position pos with left pad lo equals the
    prefill row of that token over a document holding positions lo..pos
    (window distances do not change under the shift)."""
    hq, hkv, D, W = 4, 2, 16, 9
    n = 40
    q = _rand((n, hq, D), 51, "bf16")
    k = _rand((n, hkv, D), 52, "bf16")
    v = _rand((n, hkv, D), 53, "bf16")
    for pos in (0, 3, 8, 9, 25, 39):
        for lo in (0, 2, 7):
            if lo > pos:
                continue
            pre = orc.prefill(q[lo:pos + 1], k[lo:pos + 1], v[lo:pos + 1],
                              np.array([0, pos + 1 - lo], np.int32), None, W, CAUSAL)[-1]
            dec = orc.decode_linear(q[pos:pos + 1], k, v, [0], [0], [n], [pos], [lo], W)[0]
            np.testing.assert_array_equal(dec, pre)


def test_decode_linear_closed_forms():
    """W = 1 gives V[pos] exactly; K = 0 gives the mean of V over
    max(lo, pos - W + 1, 0) .. pos."""
    B, hq, hkv, D, n = 3, 4, 2, 8, 30
    q = _rand((B, hq, D), 61)
    k = _rand((B * n, hkv, D), 62)
    v = _rand((B * n, hkv, D), 63)
    off = [0, n, 2 * n]
    first = [0, 0, 0]
    lens = [n, n, n]
    pos = [29, 4, 17]
    lo = [0, 3, 16]
    out = orc.decode_linear(q, k, v, off, first, lens, pos, lo, 1)
    for b in range(B):
        for h in range(hq):
            np.testing.assert_array_equal(out[b, h], v[off[b] + pos[b], h // 2].astype(np.float64))
    kz = np.zeros_like(k)
    for W in (0, 3, 12):
        out = orc.decode_linear(q, kz, v, off, first, lens, pos, lo, W)
        for b in range(B):
            a = max(lo[b], 0) if W <= 0 else max(lo[b], pos[b] - W + 1, 0)
            want = v[off[b] + a: off[b] + pos[b] + 1].astype(np.float64).mean(axis=0)
            for h in range(hq):
                np.testing.assert_allclose(out[b, h], want[h // 2], rtol=0, atol=1e-14)


def test_decode_linear_rejects_short_history():
    q = _rand((1, 2, 8), 1)
    k = _rand((10, 1, 8), 2)
    with pytest.raises(ValueError):
        orc.decode_linear(q, k, k, [0], [5], [5], [12], [0], 4)
