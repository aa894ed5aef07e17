"""Pins of the oracle's prefill backward to things other than itself (CPU only).

The backward (dq, dk, dv of the loss sum(dout * out)) is fixed against:
central finite differences of the oracle's forward (itself pinned in
test_oracle_pins.py), torch autograd through an explicit-mask dense fp64
attention, a closed form (window 1) and two invariants of the softmax.
The mistakes each test catches are named in its docstring.
"""
import math

import numpy as np
import pytest
import torch

import swa_inputs as si
from oracle import oracle as orc

CAUSAL, BLOCKWISE = orc.CAUSAL, orc.BLOCKWISE


def _f64(a):
    return si.bf16_bits_to_f32(a).astype(np.float64) if a.dtype == np.uint16 else a.astype(np.float64)


def _dense_mask(cu, ids, W, mode, T):
    """Explicit T x T mask from the definition: same document, window
    i - j < W (W <= 0: none), and causal or (blockwise: same image run)."""
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
    return m & ((j <= i) | fut)


def _autograd(q, k, v, dout, cu, ids, W, mode):
    """torch autograd through a dense masked fp64 attention (CPU)."""
    T, hq, D = q.shape
    g = hq // k.shape[1]
    mask = torch.from_numpy(_dense_mask(cu, ids, W, mode, T))
    qt = torch.tensor(_f64(q), requires_grad=True)
    kt = torch.tensor(_f64(k), requires_grad=True)
    vt = torch.tensor(_f64(v), requires_grad=True)
    kr = kt.repeat_interleave(g, dim=1)
    vr = vt.repeat_interleave(g, dim=1)
    s = torch.einsum("ihd,jhd->hij", qt, kr) / math.sqrt(D)
    s = s.masked_fill(~mask, float("-inf"))
    p = torch.softmax(s, dim=-1)
    out = torch.einsum("hij,jhd->ihd", p, vr)
    (out * torch.from_numpy(_f64(dout))).sum().backward()
    return qt.grad.numpy(), kt.grad.numpy(), vt.grad.numpy()


@pytest.mark.parametrize("trial", range(10))
def test_backward_matches_autograd_on_dense_mask(trial):
    """Random tiny packed shapes, both modes, windows 1..T+7 and none, group
    sizes 1/2/4: the oracle's chain rule equals autograd of the explicit-mask
    dense attention within 1e-12.  Catches a dropped softmax-Jacobian term
    (delta), a missing scale, a transposed product, GQA contributions not
    summed over the group, and a mask that differs between forward and
    backward."""
    rng = si.rng_for(5000 + trial)
    T = int(rng.integers(2, 40))
    cu = si.ragged_cu_seqlens(rng, T, int(rng.integers(1, 4)))
    hkv = int(rng.choice([1, 2]))
    g = int(rng.choice([1, 2, 4]))
    D = int(rng.choice([4, 8]))
    ids = np.full(T, -1, np.int32)
    for b in range(int(rng.integers(0, 3))):
        s = int(rng.integers(0, T))
        ids[s:min(T, s + int(rng.integers(1, 10)))] = b
    q = si.normal(rng, (T, hkv * g, D), "bf16")
    k = si.normal(rng, (T, hkv, D), "bf16")
    v = si.normal(rng, (T, hkv, D), "bf16")
    do = si.normal(rng, (T, hkv * g, D), "bf16")
    for W in (1, 3, T, T + 7, 0):
        for mode in (CAUSAL, BLOCKWISE):
            got = orc.prefill_backward(q, k, v, do, cu, ids, W, mode)
            want = _autograd(q, k, v, do, cu, ids, W, mode)
            for a, b in zip(got, want):
                np.testing.assert_allclose(a, b, rtol=0, atol=1e-12)


def _grid(rng, shape):
    """fp32 values on a 2^-6 grid in [-4, 4): x +- 2^-12 stays exact in fp32."""
    return (np.round(np.clip(rng.standard_normal(shape), -3.9, 3.9) * 64) / 64).astype(np.float32)


@pytest.mark.parametrize("mode,W", [(CAUSAL, 3), (BLOCKWISE, 4), (CAUSAL, 0)])
def test_backward_central_differences(mode, W):
    """Every element of dq, dk and dv equals the central difference
    (L(x + h) - L(x - h)) / 2h of L = sum(dout * prefill(q, k, v)), taken
    with the oracle's forward, within 1e-7 (the O(h^2) truncation error).
    A derivative by perturbation shares nothing with the chain rule, so any
    wrong term, sign or index in the backward fails here."""
    rng = si.rng_for(77 + W)
    T, hq, hkv, D = 11, 4, 2, 4
    cu = np.array([0, 4, 11], np.int32)
    ids = np.array([-1, 0, 0, -1, 1, 1, 1, -1, 2, 2, -1], np.int32)
    q, k, v, do = (_grid(rng, s) for s in [(T, hq, D), (T, hkv, D), (T, hkv, D), (T, hq, D)])
    h = 2.0 ** -12

    def loss(qq, kk, vv):
        return float((orc.prefill(qq, kk, vv, cu, ids, W, mode) * do.astype(np.float64)).sum())

    dq, dk, dv = orc.prefill_backward(q, k, v, do, cu, ids, W, mode)
    for which, grad in ((0, dq), (1, dk), (2, dv)):
        base = [q, k, v]
        x = base[which]
        num = np.empty(x.shape)
        for idx in np.ndindex(x.shape):
            xp, xm = x.copy(), x.copy()
            xp[idx] += np.float32(h)
            xm[idx] -= np.float32(h)
            assert float(xp[idx]) - float(x[idx]) == h  # the step is exact
            ap, am = list(base), list(base)
            ap[which], am[which] = xp, xm
            num[idx] = (loss(*ap) - loss(*am)) / (2 * h)
        np.testing.assert_allclose(grad, num, rtol=0, atol=1e-7)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_backward_window_one_closed_form(dtype):
    """W = 1 (causal): every row attends only itself with weight exactly 1,
    so out = v and the scores do not matter: dq = dk = 0 exactly and
    dv[j] = sum of dout[j, h] over the heads h of the group, exactly."""
    rng = si.rng_for(91)
    T, hq, hkv, D = 20, 6, 2, 8
    cu = np.array([0, 7, 20], np.int32)
    q, k, v, do = (si.normal(rng, s, dtype) for s in [(T, hq, D), (T, hkv, D), (T, hkv, D), (T, hq, D)])
    dq, dk, dv = orc.prefill_backward(q, k, v, do, cu, None, 1, CAUSAL)
    assert not dq.any() and not dk.any()
    want = _f64(do).reshape(T, hkv, hq // hkv, D).sum(axis=2)
    np.testing.assert_allclose(dv, want, rtol=0, atol=1e-14)


@pytest.mark.parametrize("mode,W", [(CAUSAL, 5), (BLOCKWISE, 6), (CAUSAL, 0)])
def test_backward_document_sum_invariants(mode, W):
    """Moving every key of a document by one vector c adds <q_i, c> * scale
    to all of row i's scores, which leaves each softmax unchanged: the keys'
    gradients of a document sum to 0 per K/V head.  Moving every value by c
    moves every output row of the document by c (the weights sum to 1): the
    values' gradients of a document sum to the document's dout, summed over
    the heads of the group.  Catches a gradient routed to the wrong key row
    or document, and a row whose weights do not sum to one."""
    rng = si.rng_for(123 + W)
    T, hq, hkv, D = 48, 4, 2, 8
    cu = np.array([0, 13, 30, 48], np.int32)
    ids = np.full(T, -1, np.int32)
    ids[3:9] = 0
    ids[15:22] = 1
    ids[35:47] = 2
    q, k, v, do = (si.normal(rng, s, "bf16") for s in [(T, hq, D), (T, hkv, D), (T, hkv, D), (T, hq, D)])
    _, dk, dv = orc.prefill_backward(q, k, v, do, cu, ids, W, mode)
    dof = _f64(do).reshape(T, hkv, hq // hkv, D).sum(axis=2)
    for b in range(cu.size - 1):
        s, e = cu[b], cu[b + 1]
        np.testing.assert_allclose(dk[s:e].sum(axis=0), 0.0, rtol=0, atol=1e-12)
        np.testing.assert_allclose(dv[s:e].sum(axis=0), dof[s:e].sum(axis=0), rtol=0, atol=1e-12)


def test_backward_subsets_equal_full():
    """Selected rows of dq give the same bits as the full computation;
    selected key rows of dk, dv (gathered key by key over the rows that
    admit them) equal the full computation (scattered row by row) within
    rounding: two summation orders of the same terms."""
    rng = si.rng_for(5)
    T, hq, hkv, D = 40, 4, 2, 8
    cu = np.array([0, 17, 40], np.int32)
    q, k, v, do = (si.normal(rng, s, "bf16") for s in [(T, hq, D), (T, hkv, D), (T, hkv, D), (T, hq, D)])
    full = orc.prefill_backward(q, k, v, do, cu, None, 6, CAUSAL)
    rows = np.array([0, 16, 17, 39, 3], np.int32)
    keys = np.array([39, 0, 20, 16], np.int32)
    dq, dk, dv = orc.prefill_backward(q, k, v, do, cu, None, 6, CAUSAL, rows=rows, keys=keys)
    np.testing.assert_array_equal(dq, full[0][rows])
    np.testing.assert_allclose(dk, full[1][keys], rtol=0, atol=1e-13)
    np.testing.assert_allclose(dv, full[2][keys], rtol=0, atol=1e-13)


# ----------------------------------------------------------------- row log-sum-exp
@pytest.mark.parametrize("trial", range(6))
def test_lse_matches_dense_logsumexp(trial):
    """The forward's per-row log-sum-exp equals logsumexp over the row of
    an explicit-mask dense score matrix (scipy), within 1e-12."""
    from scipy.special import logsumexp
    rng = si.rng_for(8000 + trial)
    T = int(rng.integers(2, 50))
    cu = si.ragged_cu_seqlens(rng, T, int(rng.integers(1, 4)))
    hkv, g, D = 2, int(rng.choice([1, 2])), 8
    ids = np.full(T, -1, np.int32)
    s0 = int(rng.integers(0, T))
    ids[s0:min(T, s0 + 9)] = 0
    q = si.normal(rng, (T, hkv * g, D), "bf16")
    k = si.normal(rng, (T, hkv, D), "bf16")
    v = si.normal(rng, (T, hkv, D), "bf16")
    for W in (1, 4, 0):
        for mode in (CAUSAL, BLOCKWISE):
            _, lse = orc.prefill(q, k, v, cu, ids, W, mode, return_lse=True)
            m = _dense_mask(cu, ids, W, mode, T)
            for h in range(hkv * g):
                s = _f64(q)[:, h] @ _f64(k)[:, h // g].T / math.sqrt(D)
                want = logsumexp(np.where(m, s, -np.inf), axis=1)
                np.testing.assert_allclose(lse[:, h], want, rtol=0, atol=1e-12)


def test_lse_closed_forms():
    """W = 1: the row's only key is itself, lse = scale <q_i, k_i>.  K = 0:
    every score is 0, lse = log of the number of allowed keys, which for a
    causal window is min(W, position in the document + 1)."""
    rng = si.rng_for(17)
    T, hq, hkv, D = 30, 4, 2, 16
    cu = np.array([0, 11, 30], np.int32)
    q, k, v = (si.normal(rng, s, "f32") for s in [(T, hq, D), (T, hkv, D), (T, hkv, D)])
    _, lse = orc.prefill(q, k, v, cu, None, 1, CAUSAL, return_lse=True)
    dots = np.einsum("thd,thd->th", q.astype(np.float64), np.repeat(k, 2, axis=1).astype(np.float64))
    np.testing.assert_allclose(lse, dots / math.sqrt(D), rtol=0, atol=1e-13)
    for W in (5, 0):
        _, lse = orc.prefill(q, np.zeros_like(k), v, cu, None, W, CAUSAL, return_lse=True)
        pos = np.concatenate([np.arange(11), np.arange(19)])
        n = pos + 1 if W <= 0 else np.minimum(W, pos + 1)
        np.testing.assert_allclose(lse, np.log(n)[:, None] * np.ones((1, hq)), rtol=0, atol=1e-14)
