"""GPU ring decode against the fp64 oracle's decode on a LINEAR cache, at
every step of runs that span rolls, plus the two decode workloads at full
size in the launch configuration the benchmark times."""
import numpy as np
import pytest
import torch

import swa_inputs as si
from oracle import oracle as orc
from sliding_window_gqa_swa_amd import api

from gpu_util import assert_close, dev, host, log, require_gpu

pytestmark = pytest.mark.gpu


class DecodeRun:
    """Compacts rings on the GPU from a prompt tail and keeps the linear
    history (prompt tail + every appended token) on the host for the oracle."""

    def __init__(self, case: si.DecodeCase, dtype: str):
        self.c, self.dtype = case, dtype
        ks, vs = case.prompt_tail(dtype)
        tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
        B, hkv, R, d = case.batch, case.hkv, case.ring_rows, case.d
        self.k = torch.zeros((B, hkv, R, d), dtype=tdt, device="cuda")
        self.v = torch.zeros_like(self.k)
        self.meta = torch.zeros((B, 4), dtype=torch.int32, device="cuda")
        api.cache_compact(dev(ks), dev(vs), dev(case.cu_tail), self.k, self.v, self.meta,
                          case.window, dev(case.prompt_lens), dev(case.left_pad))
        cu = case.cu_tail
        self.hist_k = [ks[cu[b]:cu[b + 1]] for b in range(B)]
        self.hist_v = [vs[cu[b]:cu[b + 1]] for b in range(B)]
        self.first = (case.prompt_lens - case.tail_lens).astype(np.int32)
        self.pos = case.prompt_lens.astype(np.int64) - 1
        self.ws = None

    def step(self, s, check_seqs=None):
        c = self.c
        q, kn, vn = c.step_inputs(s, self.dtype)
        api.cache_roll(self.k, self.v, self.meta, c.window)
        api.cache_append(dev(kn), dev(vn), self.k, self.v, self.meta)
        qd = dev(q)
        if self.ws is None:
            self.ws = api.decode_workspace(qd, self.k)
        out = host(api.decode(qd, self.k, self.v, self.meta, c.window, workspace=self.ws))
        self.pos += 1
        for b in range(c.batch):
            self.hist_k[b] = np.concatenate([self.hist_k[b], kn[b:b + 1]])
            self.hist_v[b] = np.concatenate([self.hist_v[b], vn[b:b + 1]])
        seqs = range(c.batch) if check_seqs is None else check_seqs
        return q, out, list(seqs)

    def oracle(self, q, seqs):
        ks = np.concatenate([self.hist_k[b] for b in seqs])
        vs = np.concatenate([self.hist_v[b] for b in seqs])
        lens = np.array([self.hist_k[b].shape[0] for b in seqs], np.int32)
        off = np.concatenate([[0], np.cumsum(lens)[:-1]]).astype(np.int64)
        return orc.decode_linear(q[seqs], ks, vs, off, self.first[seqs], lens,
                                 self.pos[seqs].astype(np.int32), self.c.left_pad[seqs],
                                 self.c.window)


def _small_case(d, g, W, A, seed, B=6, steps=None):
    rng = si.rng_for(seed)
    L = rng.integers(1, 4 * W, size=B).astype(np.int32)
    L[0] = 1
    L[1] = W - 1 if W > 1 else 1
    lo = np.array([rng.integers(0, min(int(l), 7)) for l in L], np.int32)
    tail = np.minimum(L, W).astype(np.int32)
    return si.DecodeCase("small", batch=B, hq=2 * g, hkv=2, d=d, window=W, ring_rows=W + A,
                         prompt_lens=L, left_pad=lo, tail_lens=tail,
                         steps=steps or 2 * A + 3, seed=seed)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("d,g,W,A", [(64, 1, 40, 8), (128, 4, 100, 16), (256, 2, 50, 64),
                                     (512, 2, 30, 8), (256, 8, 33, 5), (320, 2, 60, 16),
                                     (320, 4, 31, 7), (192, 8, 40, 8), (384, 4, 50, 16),
                                     (448, 2, 30, 8)])
def test_ring_decode_equals_linear_decode_every_step(dtype, d, g, W, A):
    require_gpu()
    case = _small_case(d, g, W, A, seed=d + g + W)
    run = DecodeRun(case, dtype)
    for s in range(case.steps):
        log("decode small d=%d g=%d W=%d A=%d %s step %d" % (d, g, W, A, dtype, s))
        q, out, seqs = run.step(s)
        want = run.oracle(q, seqs)
        assert_close(out, want, dtype, "step %d" % s)
    m = host(run.meta)
    assert not (m[:, 3] < 0).any(), "a sequence overflowed its ring"


def test_decode_window_one_is_exact():
    """W = 1: the query reads only its own freshly appended row."""
    require_gpu()
    case = _small_case(256, 2, 1, 4, seed=9, steps=7)
    run = DecodeRun(case, "bf16")
    for s in range(case.steps):
        q, out, _ = run.step(s)
        _, kn, vn = case.step_inputs(s, "bf16")
        np.testing.assert_array_equal(out, np.repeat(vn, 2, axis=1))


def test_decode_needle_follows_the_window():
    """fp32 sharpness: a dominant key is seen while inside the window and
    dropped exactly when it leaves it (one-key errors move O by O(1))."""
    require_gpu()
    d, W, A = 128, 16, 4
    case = si.DecodeCase("needle", batch=1, hq=2, hkv=1, d=d, window=W, ring_rows=W + A,
                         prompt_lens=np.array([W], np.int32), left_pad=np.array([0], np.int32),
                         tail_lens=np.array([W], np.int32), steps=1, seed=4)
    run = DecodeRun(case, "f32")
    direction = np.ones(d, np.float32) / np.sqrt(d)
    for s in range(2 * W):
        q, kn, vn = case.step_inputs(s, "f32")
        q = (q * 0.1 + 4.0 * direction).astype(np.float32)
        kn = (kn * 0.1).astype(np.float32)
        if s == 0:
            kn[0, 0] = 40.0 * direction  # the needle at position W
        api.cache_roll(run.k, run.v, run.meta, W)
        api.cache_append(dev(kn), dev(vn), run.k, run.v, run.meta)
        out = host(api.decode(dev(q), run.k, run.v, run.meta, W))
        run.pos += 1
        run.hist_k[0] = np.concatenate([run.hist_k[0], kn])
        run.hist_v[0] = np.concatenate([run.hist_v[0], vn])
        want = run.oracle(q, [0])
        assert_close(out, want, "f32", "needle step %d" % s)
        needle_v = run.hist_v[0][W, 0].astype(np.float64)
        sees = np.abs(out[0, 0] - needle_v).max() < 0.05
        assert sees == (s < W), s


def test_decode_batched_b64_70_steps():
    """64 sequences at random positions in [1, 32768] with left pad 0..63,
    70 steps spanning the roll: all sequences checked on the steps around
    the roll, a rotating sample of 8 on every other step."""
    require_gpu()
    case = si.decode_b64_d256()
    run = DecodeRun(case, "bf16")
    rolled = False
    worst = (0.0, 0.0)
    for s in range(case.steps):
        full = s in (0, 1, 62, 63, 64, 65, 69)
        seqs = None if full else [(s * 8 + i) % case.batch for i in range(8)]
        log("decode b64 step %d" % s)
        q, out, seqs = run.step(s, seqs)
        if s == 64:
            rolled = True
        want = run.oracle(q, seqs)
        mx, mean = assert_close(out[seqs], want, "bf16", "b64 step %d" % s)
        worst = (max(worst[0], mx), max(worst[1], mean))
    log("  decode b64, worst step: max-abs %.3g, mean-abs %.3g" % worst)
    assert rolled
    m = host(run.meta)
    assert not (m[:, 3] < 0).any()
    # the roll happened exactly once, at step 64: anchor = L - W + 64
    np.testing.assert_array_equal(m[:, 1], case.prompt_lens - case.window + 64)


def test_decode_one_split_per_ring_is_deterministic():
    """The 64-sequence workload's launch (one split per ring: every block
    writes its outputs itself, no partials): two decodes of one state are
    bit-identical and match the oracle."""
    require_gpu()
    case = si.decode_b64_d256()
    run = DecodeRun(case, "bf16")
    log("decode b64 determinism")
    q, out, seqs = run.step(0)
    out2 = host(api.decode(dev(q), run.k, run.v, run.meta, case.window, workspace=run.ws))
    np.testing.assert_array_equal(out, out2)
    assert_close(out, run.oracle(q, seqs), "bf16", "b64 one split")


def test_decode_single_sequence_position_3000():
    require_gpu()
    c = si.decode_single_d256()
    for dtype in ("bf16", "f32"):
        run = DecodeRun(c, dtype)
        for s in range(-c.pre_appends, c.steps):
            q, out, seqs = run.step(s)
        assert host(run.meta)[0].tolist() == [3000, 1920, 832, 0]
        want = run.oracle(q, seqs)
        mx, mean = assert_close(out, want, dtype, "single %s" % dtype)
        log("  decode single %s: max-abs %.3g, mean-abs %.3g" % (dtype, mx, mean))


def test_decode_deterministic_and_position_independent_launch():
    """Two decodes of one state are bit-identical; one workspace, sized from
    the shapes alone, serves ring states at very different positions (the
    launch never depends on positions), each matching the oracle."""
    require_gpu()
    case = _small_case(256, 2, 64, 64, seed=3, B=4, steps=1)
    run = DecodeRun(case, "bf16")
    q, out, seqs = run.step(0)
    out2 = host(api.decode(dev(q), run.k, run.v, run.meta, case.window, workspace=run.ws))
    np.testing.assert_array_equal(out, out2)
    assert_close(out, run.oracle(q, seqs), "bf16", "near start")
    # same sizes, positions around 30000 instead of below 256, same workspace
    far = si.DecodeCase("far", batch=case.batch, hq=case.hq, hkv=case.hkv, d=case.d,
                        window=case.window, ring_rows=case.ring_rows,
                        prompt_lens=case.prompt_lens + 30000, left_pad=case.left_pad,
                        tail_lens=np.full(case.batch, case.window, np.int32), steps=1, seed=5)
    run_far = DecodeRun(far, "bf16")
    run_far.ws = run.ws
    log("decode far positions, shared workspace")
    q, out, seqs = run_far.step(0)
    assert host(run_far.meta)[:, 0].min() >= 30000
    assert_close(out, run_far.oracle(q, seqs), "bf16", "far positions")


def test_decode_batched_d320_across_a_roll():
    """Head size 320 (640-byte rows: 40 chunks over 64 lanes) on the large
    grid of the batched decode: 64 sequences at seeded positions up to 8192,
    W = 1024, 1088-row rings, 70 steps across the roll, sampled sequences
    checked on every fifth step and all of them around the roll."""
    require_gpu()
    rng = si.rng_for(320)
    B = 64
    pos = rng.integers(1, 8192 + 1, size=B).astype(np.int32)
    lo = np.array([rng.integers(0, min(63, int(p) - 1) + 1) for p in pos], np.int32)
    case = si.DecodeCase("b64_d320", batch=B, hq=8, hkv=4, d=320, window=1024, ring_rows=1088,
                         prompt_lens=pos, left_pad=lo, tail_lens=np.minimum(pos, 1024).astype(np.int32),
                         steps=70, seed=320)
    run = DecodeRun(case, "bf16")
    for s in range(case.steps):
        full = s in (0, 63, 64, 65, 69)
        seqs = None if full else [(s * 8 + i) % B for i in range(8)]
        q, out, seqs = run.step(s, seqs)
        if full or s % 5 == 0:
            log("decode b64 d320 step %d" % s)
            assert_close(out[seqs], run.oracle(q, seqs), "bf16", "b64 d320 step %d" % s)
    assert not (host(run.meta)[:, 3] < 0).any()


def test_decode_at_the_largest_ring():
    """The largest ring the calls accept (SWA_MAX_RING_ROWS = 65536 rows:
    W = 65472 plus the 64 slack rows), two sequences whose prompts are
    longer than the window, decoded across the roll that the 64th step
    brings, against the linear-cache oracle at the steps around it."""
    require_gpu()
    W, A = 65536 - 64, 64
    L = np.array([70001, 66000], np.int32)
    case = si.DecodeCase("max_ring", batch=2, hq=4, hkv=2, d=64, window=W, ring_rows=W + A,
                         prompt_lens=L, left_pad=np.array([0, 5], np.int32),
                         tail_lens=np.minimum(L, W).astype(np.int32), steps=66, seed=65536)
    run = DecodeRun(case, "bf16")
    for s in range(case.steps):
        log("decode largest ring step %d" % s)
        q, out, seqs = run.step(s)
        if s in (0, 1, 62, 63, 64, 65):
            assert_close(out, run.oracle(q, seqs), "bf16", "largest ring step %d" % s)
    m = host(run.meta)
    assert not (m[:, 3] < 0).any(), "a sequence overflowed its ring"
    assert (m[:, 1] == L.astype(np.int64) - W + A).all(), "one roll moved each anchor by 64"


@pytest.mark.parametrize("case", range(16))
def test_decode_random_shapes_across_a_roll(case):
    """Seeded random sweep of decode shapes: batch (1 to 128, so that both
    the small-grid path and the one-split-per-ring path of large grids
    run), kv heads, group (1, 2, 3, 4, 8), head size, window, slack rows
    and element type per case; every sequence checked against the
    linear-cache oracle at every step across the first roll."""
    require_gpu()
    rng = si.rng_for(8800 + case)
    d = (64, 128, 192, 256, 320, 384, 448, 512)[case % 8]
    B = int(rng.choice([1, 3, 17, 64, 128]))
    hkv = int(rng.choice([1, 2, 4]))
    g = int(rng.choice([1, 2, 3, 4, 8]))
    W = int(rng.integers(1, 300))
    A = int(rng.choice([1, 5, 64]))
    dtype = "f32" if rng.random() < 0.25 else "bf16"
    L = rng.integers(1, 3 * W + 2, size=B).astype(np.int32)
    lo = np.array([rng.integers(0, min(int(x), 7)) for x in L], np.int32)
    c = si.DecodeCase("random", batch=B, hq=g * hkv, hkv=hkv, d=d, window=W, ring_rows=W + A,
                      prompt_lens=L, left_pad=lo, tail_lens=np.minimum(L, W).astype(np.int32),
                      steps=A + 2, seed=8800 + case)
    what = "case %d: B=%d hq=%d hkv=%d d=%d W=%d A=%d %s" % (case, B, g * hkv, hkv, d, W, A, dtype)
    run = DecodeRun(c, dtype)
    for s in range(c.steps):
        log("decode random %s step %d" % (what, s))
        q, out, seqs = run.step(s)
        assert_close(out, run.oracle(q, seqs), dtype, "%s step %d" % (what, s))
    assert not (host(run.meta)[:, 3] < 0).any(), what
