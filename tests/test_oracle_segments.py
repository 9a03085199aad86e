"""Pins of the segment post-processing oracle (oracle/segments.py).

The pages fix the output format (a list of [begin_seconds, end_seconds,
speaker_index], or {"Start", "End", "Speaker"} dictionaries) and that it comes
from thresholding and smoothing the per-frame probabilities; the parameter
order is the reading stated in the oracle. Checked here: hand-worked
examples, an independent run finder for the default parameters, and the
invariants every output must satisfy.
"""
import numpy as np
import pytest

from oracle import segments as SG

DT = 0.08  # Sortformer output frame (80 ms)


def _np_runs(mask):
    """Independent run finder: edges of the 0/1 sequence via np.diff."""
    d = np.diff(np.concatenate([[0], mask.astype(np.int8), [0]]))
    return list(zip(np.flatnonzero(d == 1), np.flatnonzero(d == -1)))


def test_default_segments_are_the_runs_above_one_half():
    rng = np.random.default_rng(0)
    for trial in range(20):
        T, S = int(rng.integers(1, 300)), 4
        probs = rng.random((T, S)).astype(np.float32)
        probs[rng.random((T, S)) < 0.3] = 0.5  # exactly at the threshold: off
        got = SG.segments(probs, DT)
        ref = sorted([[f0 * DT, f1 * DT, s] for s in range(S)
                      for f0, f1 in _np_runs(probs[:, s] > np.float32(0.5))],
                     key=lambda x: (x[0], x[2], x[1]))
        assert got == ref


def test_hysteresis_hand_example():
    p = [0.2, 0.7, 0.45, 0.45, 0.3, 0.8, 0.6, 0.1]
    act = SG.activity(p, onset=0.6, offset=0.4)
    assert act.tolist() == [False, True, True, True, False, True, True, False]
    assert SG.runs(act) == [(1, 4), (5, 7)]
    assert SG.track_segments(p, DT, onset=0.6, offset=0.4) == [(1 * DT, 4 * DT), (5 * DT, 7 * DT)]


def test_padding_merges_overlaps_and_clips():
    p = [0.2, 0.7, 0.45, 0.45, 0.3, 0.8, 0.6, 0.1]
    got = SG.track_segments(p, DT, onset=0.6, offset=0.4, pad_onset=0.05, pad_offset=0.1)
    # [0.03, 0.42] and [0.35, 0.66] overlap; the end is clipped to T*dt = 0.64
    assert got == [(1 * DT - 0.05, 8 * DT)]
    got = SG.track_segments([0.9, 0.9, 0.1, 0.9], DT, pad_onset=0.5, pad_offset=0.5)
    assert got == [(0.0, 4 * DT)]  # clipped to [0, T*dt]


def test_minimum_durations():
    p = [0.2, 0.7, 0.45, 0.45, 0.3, 0.8, 0.6, 0.1]
    kw = dict(onset=0.6, offset=0.4)
    # 0.24 s kept, 0.16 s dropped
    assert SG.track_segments(p, DT, min_duration_on=0.2, **kw) == [(1 * DT, 4 * DT)]
    # the 0.08 s gap is filled
    assert SG.track_segments(p, DT, min_duration_off=0.1, **kw) == [(1 * DT, 7 * DT)]
    # merging happens before dropping: two short runs joined survive
    assert SG.track_segments(p, DT, min_duration_off=0.1, min_duration_on=0.4, **kw) == \
        [(1 * DT, 7 * DT)]


def test_edges_all_on_all_off_last_frame():
    assert SG.track_segments(np.ones(10), DT) == [(0.0, 10 * DT)]
    assert SG.track_segments(np.zeros(10), DT) == []
    assert SG.track_segments([0.1, 0.1, 0.9], DT) == [(2 * DT, 3 * DT)]
    assert SG.segments(np.zeros((0, 4)), DT) == []


@pytest.mark.parametrize("params", [dict(), dict(onset=0.7, offset=0.3),
                                    dict(pad_onset=0.1, pad_offset=0.05, min_duration_on=0.3,
                                         min_duration_off=0.2)])
def test_invariants(params):
    rng = np.random.default_rng(1)
    # smooth-ish tracks: a random walk squashed to (0, 1)
    T, S = 500, 4
    z = np.cumsum(rng.standard_normal((T, S)) * 0.6, axis=0)
    probs = (1 / (1 + np.exp(-z))).astype(np.float32)
    prm = dict(SG.DEFAULTS, **params)
    out = SG.segments(probs, DT, **params)
    assert out == sorted(out, key=lambda x: (x[0], x[2], x[1]))
    for s in range(S):
        segs = [(a, b) for a, b, k in out if k == s]
        for a, b in segs:
            assert 0.0 <= a < b <= T * DT + 1e-12
            assert b - a >= prm["min_duration_on"]
        for (a0, b0), (a1, b1) in zip(segs, segs[1:]):
            assert a1 - b0 >= prm["min_duration_off"]  # sorted, disjoint, gaps respected
    dicts = SG.speaker_dicts(probs, DT, **params)
    assert [[d["Start"], d["End"], d["Speaker"]] for d in dicts] == out
