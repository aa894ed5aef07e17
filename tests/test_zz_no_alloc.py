"""swa_decode_step_noalloc, whose split-K scratch is a static device array
of the library, against swa_decode_step with a caller workspace.  Both run
the same kernels, so outputs, ring bytes and ring_meta must agree bit for
bit.  Calls follow one another on the one shared scratch: a batch of 12
sequences over 18 steps (across a roll), then a smaller batch of 3, then a
float32 batch of 5, then head size 448 with groups of 4, so each call finds
the scratch as the previous, larger or differently laid out, call left
it."""
import numpy as np
import pytest
import torch

import swa_inputs as si
from sliding_window_gqa_swa_amd import api

from gpu_util import dev, host, log, require_gpu

pytestmark = pytest.mark.gpu


def _case(B, dtype_seed, W=64, A=16, d=256, hq=8, hkv=4):
    rng = si.rng_for(4000 + dtype_seed + B)
    L = rng.integers(1, 3 * W, size=B).astype(np.int32)
    L[0] = 1
    lo = np.array([rng.integers(0, min(int(x), 5)) for x in L], np.int32)
    tail = np.minimum(L, W).astype(np.int32)
    return si.DecodeCase("noalloc", batch=B, hq=hq, hkv=hkv, d=d, window=W, ring_rows=W + A,
                         prompt_lens=L, left_pad=lo, tail_lens=tail, steps=0,
                         seed=4100 + dtype_seed + B)


def _two_rings(case, dtype):
    ks, vs = case.prompt_tail(dtype)
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    out = []
    for _ in range(2):
        k = torch.zeros((case.batch, case.hkv, case.ring_rows, case.d), dtype=tdt, device="cuda")
        v = torch.zeros_like(k)
        meta = torch.zeros((case.batch, 4), dtype=torch.int32, device="cuda")
        api.cache_compact(dev(ks), dev(vs), dev(case.cu_tail), k, v, meta, case.window,
                          dev(case.prompt_lens), dev(case.left_pad))
        out.append((k, v, meta))
    return out


def test_noalloc_step_matches_workspace_step():
    require_gpu()
    for B, steps, dtype, d, hq, hkv in ((12, 18, "bf16", 256, 8, 4), (3, 2, "bf16", 256, 8, 4),
                                        (5, 3, "f32", 256, 8, 4), (4, 3, "bf16", 448, 8, 2)):
        case = _case(B, 0 if dtype == "bf16" else 1, d=d, hq=hq, hkv=hkv)
        (ka, va, ma), (kb, vb, mb) = _two_rings(case, dtype)
        ws = api.decode_workspace(torch.empty((B, case.hq, case.d), dtype=ka.dtype, device="cuda"), ka)
        for s in range(steps):
            q, kn, vn = case.step_inputs(s, dtype)
            log("noalloc B=%d %s d=%d step %d" % (B, dtype, d, s))
            ref = api.decode_step(dev(q), dev(kn), dev(vn), ka, va, ma, case.window, workspace=ws)
            got = api.decode_step_noalloc(dev(q), dev(kn), dev(vn), kb, vb, mb, case.window)
            torch.cuda.synchronize()
            np.testing.assert_array_equal(host(got), host(ref))
            np.testing.assert_array_equal(host(mb), host(ma))
        np.testing.assert_array_equal(host(kb), host(ka))
        np.testing.assert_array_equal(host(vb), host(va))
        m = host(ma)
        assert not (m[:, 3] < 0).any(), "a sequence overflowed its ring"
        if steps > case.ring_rows - case.window:
            # the roll by metadata happened: anchor moved by A for every sequence
            np.testing.assert_array_equal(
                m[:, 1], case.prompt_lens - case.window + (case.ring_rows - case.window))
