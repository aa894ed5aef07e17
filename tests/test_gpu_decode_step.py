"""GPU decode step (metadata roll + append + decode in one launch) against
the oracle: ring bytes and ring_meta bit for bit against the byte-exact ring
model (its metadata-only roll, then its append), attention against the fp64
oracle's decode on a LINEAR cache, at every step of runs that span rolls."""
import numpy as np
import pytest
import torch

import swa_inputs as si
from oracle.ring_model import ERR_BIT, RingModel
from sliding_window_gqa_swa_amd import api

from gpu_util import assert_close, dev, host, log, require_gpu
from test_gpu_decode import DecodeRun, _small_case

pytestmark = pytest.mark.gpu


class StepRun(DecodeRun):
    """The decode run of test_gpu_decode, advanced by swa_decode_step, with
    a ring model that follows the same cache operations on the host."""

    def __init__(self, case, dtype, model=True):
        super().__init__(case, dtype)
        self.model = None
        if model:
            ks, vs = case.prompt_tail(dtype)
            self.model = RingModel(case.batch, case.hkv, case.ring_rows, case.d, case.window,
                                   dtype=ks.dtype)
            self.model.compact(ks, vs, case.cu_tail, case.prompt_lens, case.left_pad)

    def step(self, s, check_seqs=None):
        c = self.c
        q, kn, vn = c.step_inputs(s, self.dtype)
        qd = dev(q)
        if self.ws is None:
            self.ws = api.decode_workspace(qd, self.k)
        out = host(api.decode_step(qd, dev(kn), dev(vn), self.k, self.v, self.meta, c.window,
                                   workspace=self.ws))
        if self.model is not None:
            self.model.roll(copy=False)
            self.model.append(kn, vn)
        self.pos += 1
        for b in range(c.batch):
            self.hist_k[b] = np.concatenate([self.hist_k[b], kn[b:b + 1]])
            self.hist_v[b] = np.concatenate([self.hist_v[b], vn[b:b + 1]])
        seqs = range(c.batch) if check_seqs is None else check_seqs
        return q, out, list(seqs)

    def check_ring(self, what):
        torch.cuda.synchronize()
        np.testing.assert_array_equal(host(self.meta), self.model.meta, err_msg=what)
        np.testing.assert_array_equal(host(self.k), self.model.k, err_msg=what)
        np.testing.assert_array_equal(host(self.v), self.model.v, err_msg=what)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("d,g,W,A", [(64, 1, 40, 8), (128, 4, 100, 16), (256, 2, 50, 64),
                                     (512, 2, 30, 8), (256, 8, 33, 5), (320, 2, 60, 16),
                                     (320, 4, 31, 7), (192, 8, 40, 8), (384, 4, 50, 16),
                                     (448, 2, 30, 8)])
def test_decode_step_matches_model_and_linear_decode(dtype, d, g, W, A):
    require_gpu()
    case = _small_case(d, g, W, A, seed=500 + d + g + W)
    run = StepRun(case, dtype)
    run.check_ring("compact")
    for s in range(case.steps):
        log("decode step d=%d g=%d W=%d A=%d %s step %d" % (d, g, W, A, dtype, s))
        q, out, seqs = run.step(s)
        run.check_ring("step %d" % s)
        assert_close(out, run.oracle(q, seqs), dtype, "step %d" % s)
    m = host(run.meta)
    assert not (m[:, 3] < 0).any(), "a sequence overflowed its ring"
    # at least one roll happened (anchor moved past its compaction value)
    assert (m[:, 1] > case.prompt_lens - W).any()


def test_decode_step_equals_separate_calls():
    """Step by step, one state advanced by roll (copy) + append + decode and
    one by swa_decode_step give the same attention (to bf16 tolerance of
    each other: only the physical rows and so the summation order differ)
    and the same pos and anchor; start differs after a roll."""
    require_gpu()
    case = _small_case(256, 2, 48, 16, seed=77, B=5)
    sep = DecodeRun(case, "bf16")
    fused = StepRun(case, "bf16", model=False)
    for s in range(case.steps):
        log("decode step vs separate step %d" % s)
        q, a, _ = sep.step(s)
        _, b, _ = fused.step(s)
        ga = si.bf16_bits_to_f32(a).astype(np.float64)
        gb = si.bf16_bits_to_f32(b).astype(np.float64)
        assert np.abs(ga - gb).max() <= 2e-2 and np.abs(ga - gb).mean() <= 2e-3, s
    ms, mf = host(sep.meta), host(fused.meta)
    np.testing.assert_array_equal(ms[:, :2], mf[:, :2])
    np.testing.assert_array_equal(ms[:, 3], mf[:, 3])


def test_decode_step_window_one_is_exact():
    require_gpu()
    case = _small_case(128, 2, 1, 3, seed=41, steps=8)
    run = StepRun(case, "bf16")
    for s in range(case.steps):
        q, out, _ = run.step(s)
        _, kn, vn = case.step_inputs(s, "bf16")
        np.testing.assert_array_equal(out, np.repeat(vn, 2, axis=1))
        run.check_ring("W=1 step %d" % s)


def test_decode_step_refuses_an_overfull_ring():
    """A state two rolls behind (p - anchor >= R + A): one metadata roll is
    not enough, so nothing is written, pos is kept and the flag is set, as
    in the ring model; decode still runs on the kept state."""
    require_gpu()
    case = _small_case(64, 2, 20, 4, seed=13, B=3, steps=1)
    run = StepRun(case, "f32")
    m = host(run.meta).copy()
    m[1, 1] -= 2 * (case.ring_rows - case.window)  # sequence 1: anchor far behind
    run.meta.copy_(torch.from_numpy(m))
    run.model.meta[:] = m
    q, kn, vn = case.step_inputs(0, "f32")
    api.decode_step(dev(q), dev(kn), dev(vn), run.k, run.v, run.meta, case.window,
                    workspace=api.decode_workspace(dev(q), run.k))
    run.model.roll(copy=False)
    run.model.append(kn, vn)
    run.check_ring("overfull")
    assert host(run.meta)[1, 3] & ERR_BIT
    assert not (host(run.meta)[[0, 2], 3] & ERR_BIT).any()


def test_decode_step_b64_70_steps():
    """The 64-sequence workload advanced by decode steps across the roll, in
    the launch configuration the benchmark times: sampled sequences against
    the linear-cache oracle, the whole batch on the steps around the roll,
    ring bytes against the model at the end."""
    require_gpu()
    case = si.decode_b64_d256()
    run = StepRun(case, "bf16")
    for s in range(case.steps):
        full = s in (0, 63, 64, 65, 69)
        seqs = None if full else [(s * 8 + i) % case.batch for i in range(8)]
        log("decode step b64 step %d" % s)
        q, out, seqs = run.step(s, seqs)
        assert_close(out[seqs], run.oracle(q, seqs), "bf16", "b64 step %d" % s)
    run.check_ring("b64 end")
    m = host(run.meta)
    np.testing.assert_array_equal(m[:, 1], case.prompt_lens - case.window + 64)
    np.testing.assert_array_equal(m[:, 2], (case.prompt_lens - case.window + 64) % case.ring_rows)


def test_decode_step_graph_replays_match_eager():
    """One decode step captured in a HIP graph and replayed step after step
    (inputs copied into the captured buffers, eager work and a host
    synchronisation between replays) gives, at every replay, the bytes the
    eager calls give, and leaves the same rings and ring_meta."""
    require_gpu()
    case = _small_case(128, 2, 24, 8, seed=61, B=4, steps=20)
    eager = StepRun(case, "bf16", model=False)
    want = [eager.step(s)[1] for s in range(case.steps)]
    g = StepRun(case, "bf16", model=False)
    q0, k0, v0 = case.step_inputs(0, "bf16")
    gq, gk, gv = dev(q0), dev(k0), dev(v0)
    gout = torch.empty_like(gq)
    ws = api.decode_workspace(gq, g.k)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        api.decode_step(gq, gk, gv, g.k, g.v, g.meta, case.window, out=gout, workspace=ws)
    for s in range(case.steps):
        log("decode step graph replay %d" % s)
        q, kn, vn = case.step_inputs(s, "bf16")
        gq.copy_(dev(q))
        gk.copy_(dev(kn))
        gv.copy_(dev(vn))
        graph.replay()
        torch.cuda.synchronize()
        np.testing.assert_array_equal(host(gout), want[s], err_msg="replay %d" % s)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(host(g.meta), host(eager.meta))
    np.testing.assert_array_equal(host(g.k), host(eager.k))
    np.testing.assert_array_equal(host(g.v), host(eager.v))


@pytest.mark.parametrize("case", range(12))
def test_decode_step_random_shapes(case):
    """Seeded random sweep of the fused step: batch (1 to 128, so that both
    the small-grid launch and the one-split-per-ring launch run), kv heads,
    group, head size, window, slack rows and element type per case; ring
    bytes and ring_meta bit for bit against the ring model and every
    sequence's attention against the linear-cache oracle at every step
    across the first roll."""
    require_gpu()
    rng = si.rng_for(8600 + case)
    d = (64, 128, 192, 256, 320, 384, 448, 512)[case % 8]
    B = int(rng.choice([1, 5, 64, 128]))
    hkv = int(rng.choice([1, 2, 4]))
    g = int(rng.choice([1, 2, 3, 4, 8]))
    W = int(rng.integers(1, 200))
    A = int(rng.choice([1, 4, 64]))
    dtype = "f32" if rng.random() < 0.25 else "bf16"
    L = rng.integers(1, 3 * W + 2, size=B).astype(np.int32)
    lo = np.array([rng.integers(0, min(int(x), 7)) for x in L], np.int32)
    c = si.DecodeCase("random step", batch=B, hq=g * hkv, hkv=hkv, d=d, window=W,
                      ring_rows=W + A, prompt_lens=L, left_pad=lo,
                      tail_lens=np.minimum(L, W).astype(np.int32), steps=A + 2, seed=8600 + case)
    what = "case %d: B=%d hq=%d hkv=%d d=%d W=%d A=%d %s" % (case, B, g * hkv, hkv, d, W, A, dtype)
    run = StepRun(c, dtype)
    for s in range(c.steps):
        log("decode step random %s step %d" % (what, s))
        q, out, seqs = run.step(s)
        run.check_ring("%s step %d" % (what, s))
        assert_close(out, run.oracle(q, seqs), dtype, "%s step %d" % (what, s))
