"""GPU ring-cache kernels (compact, append, roll) against the byte-exact ring
model of the oracle: ring bytes and ring_meta must match bit for bit."""
import json
import os

import numpy as np
import pytest
import torch

import swa_inputs as si
from oracle.ring_model import ERR_BIT, RingModel
from sliding_window_gqa_swa_amd import api

from gpu_util import dev, host, log, require_gpu

pytestmark = pytest.mark.gpu


class GpuRing:
    def __init__(self, B, hkv, R, d, W, dtype):
        tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
        self.W = W
        # garbage-filled, so compaction must write every row
        self.k = torch.full((B, hkv, R, d), 7.0, dtype=tdt, device="cuda")
        self.v = torch.full((B, hkv, R, d), -3.0, dtype=tdt, device="cuda")
        self.meta = torch.full((B, 4), 12345, dtype=torch.int32, device="cuda")

    def compact(self, ks, vs, cu, L=None, lo=None):
        api.cache_compact(dev(ks), dev(vs), dev(cu), self.k, self.v, self.meta, self.W,
                          None if L is None else dev(np.asarray(L, np.int32)),
                          None if lo is None else dev(np.asarray(lo, np.int32)))

    def append(self, kn, vn):
        api.cache_append(dev(kn), dev(vn), self.k, self.v, self.meta)

    def roll(self):
        api.cache_roll(self.k, self.v, self.meta, self.W)

    def check(self, model, what):
        torch.cuda.synchronize()
        np.testing.assert_array_equal(host(self.meta), model.meta, err_msg=what)
        np.testing.assert_array_equal(host(self.k), model.k, err_msg=what)
        np.testing.assert_array_equal(host(self.v), model.v, err_msg=what)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("d,W,A", [(64, 12, 4), (256, 24, 8), (512, 9, 3), (128, 64, 64),
                                   (320, 20, 6), (192, 16, 4), (384, 12, 6), (448, 10, 6)])
def test_ring_ops_bit_exact_against_model(dtype, d, W, A):
    require_gpu()
    rng = si.rng_for(d + W + A)
    B, hkv = 5, 2
    R = W + A
    L = rng.integers(1, 3 * W, size=B).astype(np.int32)
    lo = np.array([rng.integers(0, min(int(l), 9)) for l in L], np.int32)
    n = np.minimum(L, W + int(rng.integers(0, 3))).astype(np.int32)
    n = np.minimum(n, L)
    cu = np.concatenate([[0], np.cumsum(n)]).astype(np.int32)
    ks = si.normal(rng, (int(cu[-1]), hkv, d), dtype)
    vs = si.normal(rng, (int(cu[-1]), hkv, d), dtype)
    model = RingModel(B, hkv, R, d, W, dtype=ks.dtype)
    ring = GpuRing(B, hkv, R, d, W, dtype)
    log("ring compact d=%d W=%d A=%d %s" % (d, W, A, dtype))
    model.compact(ks, vs, cu, L, lo)
    ring.compact(ks, vs, cu, L, lo)
    ring.check(model, "compact")
    for step in range(3 * A + 5):
        kn = si.normal(rng, (B, hkv, d), dtype)
        vn = si.normal(rng, (B, hkv, d), dtype)
        log("ring step %d" % step)
        model.roll()
        ring.roll()
        ring.check(model, "roll %d" % step)
        model.append(kn, vn)
        ring.append(kn, vn)
        ring.check(model, "append %d" % step)
    assert not (model.meta[:, 3] & ERR_BIT).any()


def test_ring_tiny_worked_example_on_gpu(golden_dir):
    require_gpu()
    fx = json.load(open(os.path.join(golden_dir, "ring_tiny.json")))
    W, R, L = fx["window"], fx["ring_rows"], fx["prompt_len"]
    d = 64
    ring = GpuRing(1, 1, R, d, W, "f32")

    def rows(ps):
        a = np.zeros((len(ps), 1, d), np.float32)
        a[:, 0, 0] = np.asarray(ps, np.float32) + 1  # 0 = never written
        return a

    src = rows(range(L))
    for st in fx["steps"]:
        log("tiny ring %s" % st["op"])
        if st["op"] == "compact":
            ring.compact(src, src, np.array([0, L], np.int32), [L], [fx["left_pad"]])
        elif st["op"] == "append":
            r = rows([st["position"]])
            ring.append(r, r)
        else:
            ring.roll()
        torch.cuda.synchronize()
        assert host(ring.meta)[0].tolist() == st["meta"]
        held = host(ring.k)[0, 0, :, 0]
        assert [None if x == 0 else int(x) - 1 for x in held] == st["row_positions"]


def test_append_on_full_ring_sets_flag_and_writes_nothing():
    require_gpu()
    W, A, d = 4, 2, 64
    ring = GpuRing(1, 1, W + A, d, W, "bf16")
    src = si.normal(si.rng_for(1), (5, 1, d), "bf16")
    ring.compact(src, src, np.array([0, 5], np.int32))
    for _ in range(2):
        kn = si.normal(si.rng_for(2), (1, 1, d), "bf16")
        ring.append(kn, kn)
    torch.cuda.synchronize()
    before_k, before_m = host(ring.k).copy(), host(ring.meta).copy()
    log("ring overflow append")
    ring.append(kn, kn)  # no roll first: the ring is full
    torch.cuda.synchronize()
    m = host(ring.meta)
    assert m[0, 3] & ERR_BIT
    assert m[0, 0] == before_m[0, 0]
    np.testing.assert_array_equal(host(ring.k), before_k)


def test_compact_rejects_uncovered_prompt():
    """A source that does not cover the first decode's window yields a zero
    ring and the error flag (no read outside the source)."""
    require_gpu()
    W, A, d = 8, 4, 64
    ring = GpuRing(2, 1, W + A, d, W, "bf16")
    src = si.normal(si.rng_for(3), (6, 1, d), "bf16")
    # sequence 0: 3 rows of a 10-token prompt (needs 7); sequence 1: fine
    ring.compact(src, src, np.array([0, 3, 6], np.int32), [10, 3], [0, 0])
    torch.cuda.synchronize()
    m = host(ring.meta)
    assert m[0, 3] & ERR_BIT and not (m[1, 3] & ERR_BIT)
    assert (host(ring.k)[0] == 0).all()


def test_decode_single_state_matches_worked_example(golden_dir):
    """The single-sequence decode workload reaches the hand-derived ring
    state (anchor 1920, start 832, position 3000 at row 824)."""
    require_gpu()
    fx = json.load(open(os.path.join(golden_dir, "ring_decode_single.json")))
    c = si.decode_single_d256()
    ks, vs = c.prompt_tail("bf16")
    ring = GpuRing(1, c.hkv, c.ring_rows, c.d, c.window, "bf16")
    ring.compact(ks, vs, c.cu_tail, c.prompt_lens, c.left_pad)
    for s in range(-c.pre_appends, c.steps):
        _, kn, vn = c.step_inputs(s)
        ring.roll()
        ring.append(kn, vn)
    torch.cuda.synchronize()
    assert host(ring.meta)[0].tolist() == fx["meta"]
    # the last appended K row sits at row 824
    np.testing.assert_array_equal(host(ring.k)[0, :, fx["slot_of_final"], :], kn[0])
