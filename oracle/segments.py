"""Speaker-activity probabilities -> speech segments (test infrastructure only).

The pages describe the user-facing output of diarization as a list of
[begin_seconds, end_seconds, speaker_index] segments obtained from the
per-frame sigmoid probabilities by VAD-style thresholding and smoothing
("Streaming Sortformer Diarizer" model card, Output; NeMo API docs,
`diarize()` Returns; Transformers docs, `extract_speaker_dict`). They do not
print the smoothing parameters or their order; the reading used here (and in
the library) is, per stream and speaker:

1. hysteresis thresholding in fp32: a frame turns the speaker on when
   p > onset and off when p <= offset (onset >= offset), otherwise it keeps
   the previous frame's state; the state before the first frame is off;
2. every maximal run of "on" frames [f0, f1) becomes [f0*dt, f1*dt] seconds;
3. padding: start - pad_onset and end + pad_offset, clipped to [0, T*dt];
4. segments (in time order) whose gap to the previous kept segment is below
   min_duration_off are merged into it (overlaps always merge);
5. segments shorter than min_duration_on are dropped.

With the defaults (onset = offset = 0.5, no padding, no minimum durations)
the segments are exactly the runs of frames with p > 0.5.
Plain Python loops: small inputs only.
"""
from __future__ import annotations

import numpy as np

DEFAULTS = dict(onset=0.5, offset=0.5, pad_onset=0.0, pad_offset=0.0, min_duration_on=0.0,
                min_duration_off=0.0)


def activity(p, onset=0.5, offset=0.5):
    """Per-frame on/off state of one speaker track (hysteresis, fp32 compares)."""
    p = np.asarray(p, dtype=np.float32)
    on_t, off_t = np.float32(onset), np.float32(offset)
    state, out = False, np.zeros(len(p), dtype=bool)
    for t, v in enumerate(p):
        if v > on_t:
            state = True
        elif v <= off_t:
            state = False
        out[t] = state
    return out


def runs(active):
    """Maximal runs of True as (f0, f1) with f1 exclusive."""
    out, start = [], None
    for t, a in enumerate(active):
        if a and start is None:
            start = t
        elif not a and start is not None:
            out.append((start, t))
            start = None
    if start is not None:
        out.append((start, len(active)))
    return out


def track_segments(p, frame_s, onset=0.5, offset=0.5, pad_onset=0.0, pad_offset=0.0,
                   min_duration_on=0.0, min_duration_off=0.0):
    """One speaker's segments [(start_s, end_s), ...] in time order (fp64)."""
    T = len(p)
    total = T * frame_s
    kept, pending = [], None
    for f0, f1 in runs(activity(p, onset, offset)):
        s = max(0.0, f0 * frame_s - pad_onset)
        e = min(total, f1 * frame_s + pad_offset)
        if pending is not None and s - pending[1] < min_duration_off:
            pending = (pending[0], max(pending[1], e))
            continue
        if pending is not None and pending[1] - pending[0] >= min_duration_on:
            kept.append(pending)
        pending = (s, e)
    if pending is not None and pending[1] - pending[0] >= min_duration_on:
        kept.append(pending)
    return kept


def segments(probs, frame_s, **params):
    """probs (T, S) of one stream -> [[start_s, end_s, speaker], ...] sorted by
    start time, then speaker."""
    prm = dict(DEFAULTS, **params)
    probs = np.asarray(probs)
    out = []
    for spk in range(probs.shape[1]):
        out += [[s, e, spk] for s, e in track_segments(probs[:, spk], frame_s, **prm)]
    return sorted(out, key=lambda x: (x[0], x[2], x[1]))


def speaker_dicts(probs, frame_s, **params):
    """The same segments as {"Start", "End", "Speaker"} dictionaries."""
    return [{"Start": s, "End": e, "Speaker": k} for s, e, k in segments(probs, frame_s, **params)]
