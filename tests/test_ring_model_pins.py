"""Pins of the byte-exact ring-cache model (CPU only).

The model is checked against hand-derived worked examples (tests/golden/),
against marker rows that encode their own position, and against decode on a
linear (never wrapped) cache at every step across several rolls.
"""
import json
import os

import numpy as np
import pytest

import swa_inputs as si
from oracle import oracle as orc
from oracle.ring_model import ERR_BIT, RingModel


def _marker_rows(positions, hkv, d):
    """K/V rows whose first two uint16 words encode the position."""
    n = len(positions)
    rows = np.zeros((n, hkv, d), np.uint16)
    p = np.asarray(positions, np.int64) + 1  # 0 stays "never written"
    rows[:, :, 0] = (p & 0xFFFF)[:, None]
    rows[:, :, 1] = (p >> 16)[:, None]
    return rows


def _row_positions(model, b):
    k = model.k[b, 0]
    p = k[:, 0].astype(np.int64) + (k[:, 1].astype(np.int64) << 16)
    return [None if x == 0 else int(x - 1) for x in p]


def test_ring_tiny_worked_example(golden_dir):
    fx = json.load(open(os.path.join(golden_dir, "ring_tiny.json")))
    W, R, L = fx["window"], fx["ring_rows"], fx["prompt_len"]
    m = RingModel(1, 1, R, 2, W)
    src = _marker_rows(range(L), 1, 2)
    for st in fx["steps"]:
        if st["op"] == "compact":
            m.compact(src, src, [0, L], [L], [fx["left_pad"]])
        elif st["op"] == "append":
            row = _marker_rows([st["position"]], 1, 2)
            m.append(row, row)
        else:
            m.roll()
        assert m.meta[0].tolist() == st["meta"], st
        assert _row_positions(m, 0) == st["row_positions"], st
        assert [r for r, _ in m.valid_rows(0)] == st["decode_rows"], st

    # the metadata-only roll alternative from the state after the 2nd append
    alt = fx["metadata_roll_after_step_3"]
    m = RingModel(1, 1, R, 2, W)
    m.compact(src, src, [0, L], [L], [0])
    for p in (5, 6):
        row = _marker_rows([p], 1, 2)
        m.append(row, row)
    m.roll(copy=False)
    assert m.meta[0].tolist() == alt["meta"]
    row = _marker_rows([7], 1, 2)
    m.append(row, row)
    assert m.slot(0, 7) == alt["append_7_row"]
    assert [r for r, _ in m.valid_rows(0)] == alt["decode_rows_after_append_7"]


def test_ring_single_sequence_state(golden_dir):
    fx = json.load(open(os.path.join(golden_dir, "ring_decode_single.json")))
    W, R, L = fx["attention_window"], fx["ring_rows"], fx["prompt_len"]
    m = RingModel(1, 1, R, 2, W)
    src = _marker_rows(range(L - 1024, L), 1, 2)
    m.compact(src, src, [0, 1024], [L], [0])
    for p in range(L, fx["final_position"] + 1):
        m.roll()
        row = _marker_rows([p], 1, 2)
        m.append(row, row)
    assert m.meta[0].tolist() == fx["meta"]
    assert m.slot(0, fx["final_position"]) == fx["slot_of_final"]
    rows = [r for r, _ in m.valid_rows(0)]
    (a0, a1), (b0, b1) = fx["decode_row_ranges"]
    assert rows == list(range(a0, a1 + 1)) + list(range(b0, b1 + 1))
    pos = _row_positions(m, 0)
    u0, u1 = fx["unwritten_rows"]
    assert all(pos[r] is None for r in range(u0, u1 + 1))
    s0, s1 = fx["stale_rows"]
    assert [pos[r] for r in range(s0, s1 + 1)] == list(range(1920, 1977))


@pytest.mark.parametrize("seed", range(6))
def test_marker_rows_recover_slot_map(seed):
    """After random compact/append/roll sequences every position the ring
    claims to hold sits at slot(p), and decode reads exactly the window."""
    rng = si.rng_for(500 + seed)
    B, W = 5, int(rng.integers(2, 9))
    A = int(rng.integers(1, 5))
    R = W + A
    L = rng.integers(1, 40, size=B)
    lo = np.array([rng.integers(0, l) for l in L])
    n = np.minimum(L, W)
    cu = np.concatenate([[0], np.cumsum(n)])
    src = np.concatenate([_marker_rows(range(l - nn, l), 1, 2) for l, nn in zip(L, n)])
    m = RingModel(B, 1, R, 2, W)
    m.compact(src, src, cu, L, lo)
    for step in range(60):
        m.roll()
        newp = m.meta[:, 0] + 1
        rows = np.concatenate([_marker_rows([p], 1, 2) for p in newp])
        m.append(rows, rows)
        assert not (m.meta[:, 3] & ERR_BIT).any()
        for b in range(B):
            pos, anchor = int(m.meta[b, 0]), int(m.meta[b, 1])
            held = _row_positions(m, b)
            for p in range(max(anchor, 0, int(L[b]) - int(n[b])), pos + 1):
                assert held[m.slot(b, p)] == p
            low = max(int(lo[b]), pos - W + 1, 0)
            assert [a for _, a in m.valid_rows(b)] == list(range(low, pos + 1))
            assert all(held[r] == a for r, a in m.valid_rows(b))


def test_roll_is_a_rotation_and_preserves_rows():
    m = RingModel(2, 3, 12, 4, 8)
    rng = si.rng_for(9)
    src = si.normal(rng, (16, 3, 4), "bf16")
    m.compact(src, src, [0, 8, 16], [8, 8], [0, 0])
    for _ in range(4):
        m.append(src[:2], src[:2])
    before = m.k.copy()
    m.roll()
    assert (m.meta[:, 1] == 4).all()
    for b in range(2):
        np.testing.assert_array_equal(m.k[b], np.roll(before[b], -4, axis=1))
        assert sorted(map(bytes, m.k[b].reshape(-1, 4))) == sorted(map(bytes, before[b].reshape(-1, 4)))


def test_append_overflow_sets_flag_and_writes_nothing():
    m = RingModel(1, 1, 6, 2, 4)
    src = _marker_rows(range(5), 1, 2)
    m.compact(src, src, [0, 5], [5], [0])
    for p in (5, 6):
        row = _marker_rows([p], 1, 2)
        m.append(row, row)
    before = m.k.copy()
    row = _marker_rows([7], 1, 2)
    m.append(row, row)  # no roll: position 7 would need row anchor + 6
    assert m.meta[0, 3] & ERR_BIT
    assert m.meta[0, 0] == 6
    np.testing.assert_array_equal(m.k, before)


@pytest.mark.parametrize("copy", [True, False])
def test_ring_decode_equals_linear_decode_every_step(copy):
    """Decode through the ring equals decode on the linear history at every
    step of a run spanning several rolls (copying and metadata-only roll),
    bit for bit in fp64."""
    B, hq, hkv, D, W, A = 4, 4, 2, 8, 10, 3
    R = W + A
    rng = si.rng_for(77)
    L = np.array([1, 5, 12, 30], np.int32)
    lo = np.array([0, 2, 0, 7], np.int32)
    steps = 25
    total = int(L.max()) + steps + 1
    k_lin = si.normal(rng, (B, total, hkv, D), "bf16")
    v_lin = si.normal(rng, (B, total, hkv, D), "bf16")
    n = np.minimum(L, W)
    cu = np.concatenate([[0], np.cumsum(n)]).astype(np.int32)
    ks = np.concatenate([k_lin[b, L[b] - n[b]:L[b]] for b in range(B)])
    vs = np.concatenate([v_lin[b, L[b] - n[b]:L[b]] for b in range(B)])
    m = RingModel(B, hkv, R, D, W)
    m.compact(ks, vs, cu, L, lo)
    flat_k = k_lin.reshape(B * total, hkv, D)
    flat_v = v_lin.reshape(B * total, hkv, D)
    rolls = 0
    for step in range(steps):
        anchors = m.meta[:, 1].copy()
        m.roll(copy=copy)
        rolls += int((m.meta[:, 1] != anchors).any())
        p = m.meta[:, 0] + 1
        m.append(np.stack([k_lin[b, p[b]] for b in range(B)]),
                 np.stack([v_lin[b, p[b]] for b in range(B)]))
        q = si.normal(si.rng_for(900 + step), (B, hq, D), "bf16")
        want = orc.decode_linear(q, flat_k, flat_v, [b * total for b in range(B)], [0] * B,
                                 [total] * B, m.meta[:, 0], lo, W)
        for b in range(B):
            kr, vr, first = m.gather_linear(b)
            got = orc.decode_linear(q[b:b + 1], kr, vr, [0], [first], [kr.shape[0]],
                                    [m.meta[b, 0]], [lo[b]], W)
            np.testing.assert_array_equal(got[0], want[b])
    assert rolls >= 5
