"""GPU parity of swa_prefill_backward against the fp64 CPU oracle.

Small ragged cases span several query and key tiles (and the 64-key dk/dv
tiles) with empty, one-token and ragged documents and are compared element
by element; the full-size prefill workloads are compared on sampled rows and
keys in the launch configuration the benchmark times, plus two properties
that hold at any size (the key gradients of a document sum to zero; the
value gradients of a document sum to its dout).

Tolerances (gradients have no natural unit, so they scale with the largest
reference magnitude m of each tensor): bf16 max-abs 2e-2 m and mean-abs
2e-3 m (the softmax weights and dS are rounded to bf16 for the matrix
products, the outputs to bf16: relative errors of a few 1e-3); fp32 max-abs
1e-5 m.  A small absolute floor covers tensors that are exactly zero in the
reference (window 1: dq = dk = 0) where the kernel leaves rounding residue.
"""
import numpy as np
import pytest
import torch

import swa_inputs as si
from oracle import oracle as orc
from sliding_window_gqa_swa_amd import api

from gpu_util import as_f64, dev, host, log, require_gpu

pytestmark = pytest.mark.gpu

CAUSAL, BLOCKWISE = si.CAUSAL, si.BLOCKWISE


def assert_grad_close(got, want, dtype, what):
    g = as_f64(got)
    assert g.shape == want.shape, (what, g.shape, want.shape)
    assert np.isfinite(g).all(), "%s: non-finite gradient" % what
    m = float(np.abs(want).max(initial=0.0))
    err = np.abs(g - want)
    mx, mean = float(err.max(initial=0.0)), float(err.mean()) if err.size else 0.0
    if m == 0.0 and err.size:
        # an exactly zero reference (every row admits only keys whose weight
        # is 1, e.g. window 1): only the rounding residue of dP - delta
        # remains, the window-1 floor 1e-5 sqrt(D / 128) (see
        # test_backward_window_one)
        floor = 1e-5 * np.sqrt(g.shape[-1] / 128.0)
        assert mx <= floor, "%s: max-abs %.3g where the reference is 0 (floor %.3g)" % (what, mx, floor)
        return mx, mean
    if dtype == "bf16":
        tmax, tmean = 2e-2 * m + 1e-5, 2e-3 * m + 1e-6
        assert mx <= tmax and mean <= tmean, \
            "%s: max-abs %.3g (tol %.3g), mean-abs %.3g (tol %.3g), ref max %.3g" % (
                what, mx, tmax, mean, tmean, m)
    else:
        tmax = 1e-5 * m + 1e-6
        assert mx <= tmax, "%s: max-abs %.3g (tol %.3g), ref max %.3g" % (what, mx, tmax, m)
    return mx / m if m > 0 else mx, mean / m if m > 0 else mean


def _round_out(out64, dtype):
    """The forward output handed to the backward, in the input dtype."""
    f = out64.astype(np.float32)
    return si.f32_to_bf16_bits(f) if dtype == "bf16" else f


def _run(q, k, v, out, do, cu, ids, W, mode):
    dq, dk, dv = api.prefill_backward(dev(q), dev(k), dev(v), dev(out), dev(do), dev(cu),
                                      None if ids is None else dev(ids), W, mode)
    torch.cuda.synchronize()
    return host(dq), host(dk), host(dv)


def _ids_for(T, cu, seed):
    """A few image runs per document, including ones crossing many rows."""
    rng = si.rng_for(seed)
    ids = np.full(T, -1, np.int32)
    nid = 0
    for a, b in zip(cu[:-1], cu[1:]):
        pos = int(a)
        while pos < int(b):
            s = pos + int(rng.integers(0, 40))
            e = min(int(b), s + int(rng.integers(1, 150)))
            if s >= int(b):
                break
            ids[s:e] = nid
            nid += 1
            pos = e
    return ids


CASES = [(d, dtype, mode) for d in (64, 128, 192, 256, 320, 384, 448, 512) for dtype in ("bf16", "f32")
         for mode in (CAUSAL, BLOCKWISE)]


@pytest.mark.parametrize("d,dtype,mode", CASES)
def test_backward_small_ragged(d, dtype, mode):
    require_gpu()
    rng = si.rng_for(31 * d + (dtype == "f32") * 7 + mode)
    T = 613 if d <= 256 else 389
    cu = np.array([0, 1, 130, 130, 401, T], np.int32) if d <= 256 else np.array([0, 77, 78, 300, T], np.int32)
    hkv, g = (2, 2) if d != 128 else (1, 4)
    hq = hkv * g
    q, k, v, do = (si.normal(rng, s, dtype) for s in [(T, hq, d), (T, hkv, d), (T, hkv, d), (T, hq, d)])
    ids = _ids_for(T, cu, 3 * d + mode) if mode == BLOCKWISE else None
    for W in (0, 37, 200):
        out = _round_out(orc.prefill(q, k, v, cu, ids, W, mode), dtype)
        log("backward small d=%d %s mode=%d W=%d T=%d hq=%d hkv=%d" % (d, dtype, mode, W, T, hq, hkv))
        got = _run(q, k, v, out, do, cu, ids, W, mode)
        want = orc.prefill_backward(q, k, v, do, cu, ids, W, mode)
        for name, a, b in zip(("dq", "dk", "dv"), got, want):
            assert_grad_close(a, b, dtype, "%s d=%d %s mode=%d W=%d" % (name, d, dtype, mode, W))


@pytest.mark.parametrize("d", [128, 256])
@pytest.mark.parametrize("mode", [CAUSAL, BLOCKWISE])
def test_backward_odd_group(d, mode):
    """Three query heads per K/V head: the dk/dv work-groups walk three
    heads' query tiles and sum their contributions."""
    require_gpu()
    rng = si.rng_for(700 + d + mode)
    T, hkv, g = 301, 1, 3
    cu = np.array([0, 150, 151, T], np.int32)
    q, k, v, do = (si.normal(rng, s, "bf16") for s in [(T, hkv * g, d), (T, hkv, d), (T, hkv, d), (T, hkv * g, d)])
    ids = _ids_for(T, cu, 750 + d) if mode == BLOCKWISE else None
    for W in (0, 45):
        out = _round_out(orc.prefill(q, k, v, cu, ids, W, mode), "bf16")
        log("backward odd group d=%d mode=%d W=%d" % (d, mode, W))
        got = _run(q, k, v, out, do, cu, ids, W, mode)
        want = orc.prefill_backward(q, k, v, do, cu, ids, W, mode)
        for name, a, b in zip(("dq", "dk", "dv"), got, want):
            assert_grad_close(a, b, "bf16", "%s odd group d=%d mode=%d W=%d" % (name, d, mode, W))


@pytest.mark.parametrize("d", [64, 128, 256, 512])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_backward_window_one(d, dtype):
    """W = 1: every row attends only itself with weight 1, so dq = dk = 0
    and dv[j] = the sum of dout[j] over the group's heads."""
    require_gpu()
    rng = si.rng_for(40 + d)
    T, hkv, g = 333, 2, 2
    cu = np.array([0, 100, 101, T], np.int32)
    q, k, v, do = (si.normal(rng, s, dtype) for s in [(T, hkv * g, d), (T, hkv, d), (T, hkv, d), (T, hkv * g, d)])
    out = np.repeat(v, g, axis=1)  # the forward at W = 1, exactly
    log("backward W=1 d=%d %s" % (d, dtype))
    dq, dk, dv = _run(q, k, v, out, do, cu, None, 1, CAUSAL)
    # dS = P (dP - delta) with dP from the matrix cores and delta from a
    # vector sum: their fp32 rounding differs by ~1e-6 |dP| (|dP| grows as
    # sqrt(D)), which leaves dq, dk of order 1e-6 .. 1e-5 where the exact
    # value is 0 (a wrongly admitted key would give O(0.1))
    floor = 1e-5 * np.sqrt(d / 128.0)
    assert np.abs(as_f64(dq)).max() <= floor and np.abs(as_f64(dk)).max() <= floor
    want = as_f64(do).reshape(T, hkv, g, d).sum(axis=2)
    assert_grad_close(dv, want, dtype, "dv W=1 d=%d %s" % (d, dtype))


@pytest.mark.parametrize("ndocs", [300, 1500])
@pytest.mark.parametrize("mode", [CAUSAL, BLOCKWISE])
def test_backward_many_documents(ndocs, mode):
    """Hundreds of short documents (empty ones among them), more than the
    forward keeps in LDS at 1500: every row interval ends at a document
    boundary, so most tiles are split between documents."""
    require_gpu()
    rng = si.rng_for(7300 + ndocs + mode)
    lens = rng.integers(0, 25, size=ndocs)
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    T = int(cu[-1])
    hq, hkv, d = 4, 2, 128
    q, k, v, do = (si.normal(rng, s, "bf16") for s in [(T, hq, d), (T, hkv, d), (T, hkv, d), (T, hq, d)])
    ids = _ids_for(T, cu, 7400 + ndocs) if mode == BLOCKWISE else None
    for W in (0, 7):
        out = _round_out(orc.prefill(q, k, v, cu, ids, W, mode), "bf16")
        log("backward many docs ndocs=%d T=%d mode=%d W=%d" % (ndocs, T, mode, W))
        got = _run(q, k, v, out, do, cu, ids, W, mode)
        want = orc.prefill_backward(q, k, v, do, cu, ids, W, mode)
        for name, a, b in zip(("dq", "dk", "dv"), got, want):
            assert_grad_close(a, b, "bf16", "%s many docs %d mode=%d W=%d" % (name, ndocs, mode, W))


def test_backward_is_deterministic():
    """Every output element has one writer and a fixed summation order:
    two runs give the same bits."""
    require_gpu()
    rng = si.rng_for(3)
    T, hq, hkv, d = 700, 4, 2, 128
    cu = np.array([0, 300, T], np.int32)
    q, k, v, do = (si.normal(rng, s, "bf16") for s in [(T, hq, d), (T, hkv, d), (T, hkv, d), (T, hq, d)])
    args = [dev(x) for x in (q, k, v)]
    out = api.prefill(*args, dev(cu), None, 100, CAUSAL)
    log("backward determinism")
    a = [host(x) for x in api.prefill_backward(*args, out, dev(do), dev(cu), None, 100, CAUSAL)]
    b = [host(x) for x in api.prefill_backward(*args, out, dev(do), dev(cu), None, 100, CAUSAL)]
    for x, y in zip(a, b):
        np.testing.assert_array_equal(x, y)


def test_backward_empty_is_a_no_op():
    require_gpu()
    q = torch.zeros((0, 2, 128), dtype=torch.bfloat16, device="cuda")
    k = torch.zeros((0, 1, 128), dtype=torch.bfloat16, device="cuda")
    cu = torch.zeros(2, dtype=torch.int32, device="cuda")
    dq, dk, dv = api.prefill_backward(q, k, k, q, q, cu)
    assert dq.shape == (0, 2, 128) and dk.shape == (0, 1, 128)


def _sum_properties(case, dk, dv, do):
    """Per document and K/V head: sum_j dk_j = 0 and sum_j dv_j = sum of the
    document's dout over the group's heads (both exact in real arithmetic;
    bounded here by the rounding of the summed bf16 gradients)."""
    dkf, dvf, dof = as_f64(dk), as_f64(dv), as_f64(do)
    T, hkv, d = dkf.shape
    g = dof.shape[1] // hkv
    dos = dof.reshape(T, hkv, g, d).sum(axis=2)
    cu = case.cu_seqlens
    for b in range(cu.size - 1):
        s, e = int(cu[b]), int(cu[b + 1])
        ks = dkf[s:e].sum(axis=0)
        kn = np.abs(dkf[s:e]).sum(axis=0).max()
        assert np.abs(ks).max() <= 2e-3 * kn, "doc %d: sum of dk %.3g vs scale %.3g" % (b, np.abs(ks).max(), kn)
        vs = dvf[s:e].sum(axis=0) - dos[s:e].sum(axis=0)
        vn = np.abs(dvf[s:e]).sum(axis=0).max()
        assert np.abs(vs).max() <= 2e-3 * vn, "doc %d: sum of dv - dout %.3g vs scale %.3g" % (b, np.abs(vs).max(), vn)


FULL = [("prefill_4x1024_mha_d128", [0, 1, 1023, 1024, 2047, 3000, 4095], [0, 1023, 1024, 4095]),
        ("prefill_vlm_4096_d256", [0, 700, 2048, 4095], None),
        ("prefill_16k_gqa_d512", [0, 4096, 16383], None)]


@pytest.mark.parametrize("name,rows,keys", FULL)
def test_backward_full_size_sampled(name, rows, keys):
    """The prefill workloads at full size, in the benchmark's launch
    configuration: dq on sampled rows (and dk, dv on sampled keys where the
    oracle's per-key gather finishes in seconds) against the oracle, and
    the document-sum properties of dk and dv over every key."""
    require_gpu()
    case = si.PREFILL_WORKLOADS[name]()
    q, k, v = case.tensors("bf16")
    do = si.normal(si.rng_for(case.seed + 500), q.shape, "bf16")
    rows_a = np.array(rows, np.int32)
    # the forward output enters only through delta_i = <dout_i, out_i>: the
    # GPU forward supplies it (its own parity is the forward tests'); the
    # oracle recomputes its forward and needs none
    o = api.prefill(dev(q), dev(k), dev(v), dev(case.cu_seqlens),
                    None if case.ids is None else dev(case.ids), case.window, case.mode)
    torch.cuda.synchronize()
    out = host(o)
    log("backward full size %s" % name)
    dq, dk, dv = _run(q, k, v, out, do, case.cu_seqlens, case.ids, case.window, case.mode)
    wq, wk, wv = orc.prefill_backward(q, k, v, do, case.cu_seqlens, case.ids, case.window, case.mode,
                                      rows=rows_a, keys=np.array(keys or [], np.int32))
    rel = assert_grad_close(dq[rows_a], wq, "bf16", "%s dq rows" % name)
    log("  %s dq, %d rows: max-abs %.3g, mean-abs %.3g of the largest |dq|" % ((name, len(rows_a)) + rel))
    if keys is not None:
        ka = np.array(keys, np.int32)
        for nm, g, w in (("dk", dk, wk), ("dv", dv, wv)):
            rel = assert_grad_close(g[ka], w, "bf16", "%s %s keys" % (name, nm))
            log("  %s %s, %d keys: max-abs %.3g, mean-abs %.3g of the largest |%s|"
                % ((name, nm, len(ka)) + rel + (nm,)))
    _sum_properties(case, dk, dv, do)


def test_long_document_forward_and_backward_sampled():
    """One 65536-token document (window 4096, 8 MHA heads, D = 128): the
    forward, its log-sum-exp and the backward at a length four times the
    largest benchmark workload, on sampled rows against the oracle and with
    the document-sum properties of dk and dv over every key."""
    require_gpu()
    rng = si.rng_for(65536)
    T, h, d, W = 65536, 8, 128, 4096
    cu = np.array([0, T], np.int32)
    q, k, v, do = (si.normal(rng, (T, h, d), "bf16") for _ in range(4))
    qd, kd, vd, dod, cud = dev(q), dev(k), dev(v), dev(do), dev(cu)
    log("long document forward T=%d" % T)
    out, lse = api.prefill_lse(qd, kd, vd, cud, None, W, CAUSAL)
    torch.cuda.synchronize()
    rows = np.array([0, 1, 4095, 4096, 4097, 30000, 65534, 65535], np.int32)
    want_o, want_l = orc.prefill(q, k, v, cu, None, W, CAUSAL, rows=rows, return_lse=True)
    got_o = as_f64(host(out))[rows]
    assert np.abs(got_o - want_o).max() <= 2e-2
    assert np.abs(host(lse).astype(np.float64).T[rows] - want_l).max() <= 1e-2
    log("long document backward T=%d" % T)
    dq, dk, dv = api.prefill_backward(qd, kd, vd, out, dod, cud, None, W, CAUSAL, lse=lse)
    torch.cuda.synchronize()
    wq, _, _ = orc.prefill_backward(q, k, v, do, cu, None, W, CAUSAL, rows=rows,
                                    keys=np.array([], np.int32))
    assert_grad_close(host(dq)[rows], wq, "bf16", "long document dq rows")
    case = si.PrefillCase("long", cu, h, h, d, W, CAUSAL, seed=0)
    _sum_properties(case, host(dk), host(dv), do)


WINDOWS_R = (0, 1, 15, 16, 17, 31, 32, 33, 63, 64, 65)


@pytest.mark.parametrize("case", range(24))
def test_backward_random_shapes(case):
    """Seeded random sweep: head size (every supported one), group (1, 2,
    3, 4, 8), ragged and empty documents (up to 900 tokens in all), windows
    on either side of the 16-, 32- and 64-key tile edges or random, mask
    and element type drawn per case; dq, dk, dv compared element by
    element."""
    require_gpu()
    rng = si.rng_for(9000 + case)
    d = (64, 128, 192, 256, 320, 384, 448, 512)[case % 8]
    g = int(rng.choice([1, 2, 3, 4, 8]))
    hkv = int(rng.integers(1, 3))
    ndocs = int(rng.integers(1, 5))
    cap = 900 if d <= 256 else 500
    lens = rng.integers(0, cap // ndocs + 1, size=ndocs)
    lens[int(rng.integers(0, ndocs))] = max(1, int(lens.max()))
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    T = int(cu[-1])
    W = int(WINDOWS_R[int(rng.integers(0, len(WINDOWS_R)))]) if rng.random() < 0.6 \
        else int(rng.integers(2, 700))
    mode = BLOCKWISE if rng.random() < 0.4 else CAUSAL
    dtype = "f32" if rng.random() < 0.25 else "bf16"
    hq = g * hkv
    q, k, v, do = (si.normal(rng, s, dtype) for s in [(T, hq, d), (T, hkv, d), (T, hkv, d), (T, hq, d)])
    ids = _ids_for(T, cu, 11 * case + 1) if mode == BLOCKWISE else None
    out = _round_out(orc.prefill(q, k, v, cu, ids, W, mode), dtype)
    what = "case %d: d=%d hq=%d hkv=%d docs=%s W=%d mode=%d %s" % (
        case, d, hq, hkv, lens.tolist(), W, mode, dtype)
    log("backward random " + what)
    got = _run(q, k, v, out, do, cu, ids, W, mode)
    want = orc.prefill_backward(q, k, v, do, cu, ids, W, mode)
    for name, a, b in zip(("dq", "dk", "dv"), got, want):
        assert_grad_close(a, b, dtype, "%s %s" % (name, what))
