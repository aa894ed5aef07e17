"""GPU parity of swa_prefill_lse (the forward's row log-sum-exp) and of the
backward that takes it.

out must equal swa_prefill's bit for bit (the same kernel, one more store);
lse is compared with the oracle's fp64 log-sum-exp: fp32 inputs within
2e-5 (fp32 rounding of a value of order 10), bf16 within 1e-2 (the D = 128
kernel scales Q by scale * log2(e) and rounds it to bf16 before the
products, which moves each score by ~2^-9 of its size; the row sum adds the
bf16-rounded weights).  The backward given this lse must meet the same
gradient tolerances as the one that recomputes it.
"""
import numpy as np
import pytest
import torch

import swa_inputs as si
from oracle import oracle as orc
from sliding_window_gqa_swa_amd import api

from gpu_util import dev, host, log, require_gpu
from test_gpu_prefill_backward import _ids_for, _round_out, assert_grad_close

pytestmark = pytest.mark.gpu

CAUSAL, BLOCKWISE = si.CAUSAL, si.BLOCKWISE

# (kv heads, query heads per kv head) per head size: groups of 2, 4 and 8
# (4 or 8 heads share each K/V tile in one work-group)
GROUPS = {64: (1, 8), 128: (1, 4), 192: (2, 2), 256: (2, 2), 320: (1, 4), 384: (2, 2), 448: (1, 4),
          512: (1, 4)}

CASES = [(d, dtype, mode) for d in (64, 128, 192, 256, 320, 384, 448, 512) for dtype in ("bf16", "f32")
         for mode in (CAUSAL, BLOCKWISE)]


@pytest.mark.parametrize("d,dtype,mode", CASES)
def test_prefill_lse(d, dtype, mode):
    require_gpu()
    rng = si.rng_for(55 * d + (dtype == "f32") * 5 + mode)
    T = 613 if d <= 256 else 389
    cu = np.array([0, 1, 130, 130, 401, T], np.int32) if d <= 256 else np.array([0, 77, 78, 300, T], np.int32)
    hkv, g = GROUPS[d]
    hq = hkv * g
    q, k, v = (si.normal(rng, s, dtype) for s in [(T, hq, d), (T, hkv, d), (T, hkv, d)])
    ids = _ids_for(T, cu, 7 * d + mode) if mode == BLOCKWISE else None
    for W in (0, 37):
        log("prefill lse d=%d %s mode=%d W=%d" % (d, dtype, mode, W))
        args = (dev(q), dev(k), dev(v), dev(cu), None if ids is None else dev(ids), W, mode)
        out, lse = api.prefill_lse(*args)
        ref_out = api.prefill(*args)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(host(out), host(ref_out))
        _, want = orc.prefill(q, k, v, cu, ids, W, mode, return_lse=True)
        got = host(lse).astype(np.float64).T  # [T, hq]
        tol = 1e-2 if dtype == "bf16" else 2e-5
        err = np.abs(got - want).max()
        assert err <= tol, "lse d=%d %s mode=%d W=%d: max-abs %.3g (tol %.3g)" % (d, dtype, mode, W, err, tol)


@pytest.mark.parametrize("d,dtype", [(64, "bf16"), (128, "bf16"), (128, "f32"), (192, "bf16"),
                                     (256, "bf16"), (320, "bf16"), (384, "bf16"), (448, "bf16"),
                                     (512, "bf16")])
@pytest.mark.parametrize("mode", [CAUSAL, BLOCKWISE])
def test_backward_with_forward_lse(d, dtype, mode):
    """The backward that takes the forward's lse (and skips its own pass
    over the keys) against the oracle."""
    require_gpu()
    rng = si.rng_for(66 * d + mode)
    T = 613 if d <= 256 else 389
    cu = np.array([0, 1, 130, 130, 401, T], np.int32) if d <= 256 else np.array([0, 77, 78, 300, T], np.int32)
    hkv, g = (2, 2) if d != 128 else (1, 4)
    hq = hkv * g
    q, k, v, do = (si.normal(rng, s, dtype) for s in [(T, hq, d), (T, hkv, d), (T, hkv, d), (T, hq, d)])
    ids = _ids_for(T, cu, 9 * d + mode) if mode == BLOCKWISE else None
    W = 37
    log("backward with forward lse d=%d %s mode=%d" % (d, dtype, mode))
    idsd = None if ids is None else dev(ids)
    qd, kd, vd, cud = dev(q), dev(k), dev(v), dev(cu)
    out, lse = api.prefill_lse(qd, kd, vd, cud, idsd, W, mode)
    dq, dk, dv = api.prefill_backward(qd, kd, vd, out, dev(do), cud, idsd, W, mode, lse=lse)
    torch.cuda.synchronize()
    want = orc.prefill_backward(q, k, v, do, cu, ids, W, mode)
    for name, a, b in zip(("dq", "dk", "dv"), (host(dq), host(dk), host(dv)), want):
        assert_grad_close(a, b, dtype, "%s (forward lse) d=%d %s mode=%d" % (name, d, dtype, mode))
