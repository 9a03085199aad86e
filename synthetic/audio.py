"""Meeting-like synthetic 16 kHz mono audio.

Stands in for the recordings the pages evaluate on (AMI, ES2004a, an 8 s
regression clip, a 488 s recording), none of which is available here.

Recipe (one reading of the workload description; every draw comes from
``numpy.random.Generator(PCG64(seed))`` in the order listed):

* per speaker s (in index order): f0_s ~ U(100, 250) Hz; five harmonic
  phases ~ U(0, 2*pi); initial state on/off with probability 1/2; then
  alternating on/off runs with durations ~ U(0.5, 2) s until the clip ends;
* every harmonic h = 1..5 has amplitude 0.3 (so a speaker's voice is
  sum_h 0.3 * sin(2*pi*h*f0*t + phase_h));
* at most two speakers sound at once: at each sample the two lowest-index
  active speakers are kept;
* white noise N(0, 0.01^2) over the whole clip, drawn last;
* ``arrival_order=True`` relabels speakers by first onset (speakers that
  never speak go last, by index) — used for the 8-speaker workload whose
  outputs are ordered by first arrival. The audio is unchanged by it.

Output is float32 with no clipping.
"""
from __future__ import annotations

import numpy as np

SAMPLE_RATE = 16000


def _activity(rng: np.random.Generator, n: int, sr: int) -> np.ndarray:
    on = rng.random() < 0.5
    act = np.zeros(n, dtype=bool)
    pos = 0
    while pos < n:
        run = int(round(rng.uniform(0.5, 2.0) * sr))
        run = max(run, 1)
        if on:
            act[pos:pos + run] = True
        pos += run
        on = not on
    return act


def meeting_audio(seconds: float, n_speakers: int, seed: int,
                  max_overlap: int = 2, arrival_order: bool = False,
                  sr: int = SAMPLE_RATE, return_labels: bool = False):
    """Return float32 audio of ``round(seconds*sr)`` samples (and labels)."""
    n = int(round(seconds * sr))
    rng = np.random.Generator(np.random.PCG64(seed))
    t = np.arange(n, dtype=np.float64) / sr
    voices = []
    acts = []
    for _ in range(n_speakers):
        f0 = rng.uniform(100.0, 250.0)
        phases = rng.uniform(0.0, 2.0 * np.pi, size=5)
        acts.append(_activity(rng, n, sr))
        v = np.zeros(n, dtype=np.float64)
        for h in range(5):
            v += 0.3 * np.sin(2.0 * np.pi * (h + 1) * f0 * t + phases[h])
        voices.append(v)
    act = np.stack(acts) if n_speakers else np.zeros((0, n), dtype=bool)
    # keep the lowest-index active speakers, at most max_overlap per sample
    kept = np.zeros_like(act)
    count = np.zeros(n, dtype=np.int32)
    for s in range(n_speakers):
        k = act[s] & (count < max_overlap)
        kept[s] = k
        count += k
    x = np.zeros(n, dtype=np.float64)
    for s in range(n_speakers):
        x += np.where(kept[s], voices[s], 0.0)
    x += rng.normal(0.0, 0.01, size=n)
    audio = x.astype(np.float32)
    if arrival_order and n_speakers:
        first = [int(np.argmax(kept[s])) if kept[s].any() else n + s
                 for s in range(n_speakers)]
        order = np.argsort(np.asarray(first), kind="stable")
        kept = kept[order]
    if return_labels:
        return audio, kept
    return audio


# The five measured workloads: (seconds, speakers, audio seed(s), arrival order).
WORKLOADS = {
    "offline8s": dict(seconds=8.0, n_speakers=2, seed=101),
    "low60s": dict(seconds=60.0, n_speakers=4, seed=102),
    "veryhigh600s": dict(seconds=600.0, n_speakers=4, seed=103),
    "ultralow64x120s": dict(seconds=120.0, n_speakers=4, seed=104000, streams=64),
    "nemotron1800s": dict(seconds=1800.0, n_speakers=8, seed=105,
                          arrival_order=True),
}


def workload_audio(name: str, stream: int = 0, seconds: float | None = None):
    """Audio for one stream of a named workload (optionally truncated)."""
    w = dict(WORKLOADS[name])
    streams = w.pop("streams", 1)
    if stream >= streams:
        raise ValueError(f"{name} has {streams} streams")
    seed = w.pop("seed") + stream
    if seconds is not None:
        w["seconds"] = seconds
    return meeting_audio(seed=seed, **w)
