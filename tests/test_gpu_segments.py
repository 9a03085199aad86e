"""GPU parity of the probabilities -> segments kernel against the oracle
(oracle/segments.py): every segment time must be identical (fp64, same
operations in the same order), for random tracks of every length class
around the 64-frame chunking, three parameter sets, the model's own output
on the low60s workload and the 10 ms Nemotron output of the 30-minute
workload."""
import os

import numpy as np
import pytest
import torch

from oracle import segments as SG

pytestmark = pytest.mark.gpu
GOLD = os.path.join(os.path.dirname(__file__), "golden")
PARAMS = [dict(), dict(onset=0.7, offset=0.3),
          dict(pad_onset=0.1, pad_offset=0.05, min_duration_on=0.3, min_duration_off=0.2)]


@pytest.fixture(scope="module")
def rt():
    from streaming_speaker_diarization_amd import runtime
    return runtime


def _tracks(B, T, S, seed):
    rng = np.random.default_rng(seed)
    z = np.cumsum(rng.standard_normal((B, T, S)) * 0.6, axis=1)
    p = (1 / (1 + np.exp(-z))).astype(np.float32)
    p[:, ::7] = 0.5  # exactly on the default thresholds
    p[:, 3::11] = 0.7
    return p


@pytest.mark.parametrize("T", [1, 2, 63, 64, 65, 128, 129, 1000])
@pytest.mark.parametrize("k", range(len(PARAMS)))
def test_segments_match_oracle(rt, T, k):
    B, S = 3, 4
    probs = _tracks(B, T, S, 100 * T + k)
    got = rt.segments(torch.from_numpy(probs).cuda(), 0.08, **PARAMS[k])
    for b in range(B):
        assert got[b] == SG.segments(probs[b], 0.08, **PARAMS[k]), (T, k, b)


def test_segments_of_model_outputs(rt):
    low = np.load(os.path.join(GOLD, "low60s_bf16.npy")).astype(np.float32)
    got = rt.segments(torch.from_numpy(low[None]).cuda(), 0.08)[0]
    assert got == SG.segments(low, 0.08) and len(got) > 0
    nm = np.load(os.path.join(GOLD, "nemotron1800s_bf16.npy")).astype(np.float32)
    x = torch.from_numpy(nm[None]).cuda()
    prm = dict(pad_onset=0.02, pad_offset=0.02, min_duration_on=0.1, min_duration_off=0.05)
    got = rt.segments(x, 0.01, **prm)[0]
    ref = SG.segments(nm, 0.01, **prm)
    print(f"[segments] nemotron 1800 s: {len(got)} segments", flush=True)
    assert got == ref
    d = rt.speaker_dicts(x, 0.01, **prm)[0]
    assert [[e["Start"], e["End"], e["Speaker"]] for e in d] == ref
    # kernel time for the whole 30-minute output (180 000 frames x 8 speakers)
    from streaming_speaker_diarization_amd import sortformer as sf
    cap = sf.sortformer_segments_capacity(nm.shape[0])
    out = torch.empty(8 * cap * sf.SEGMENT_BYTES, dtype=torch.uint8, device="cuda")
    cnt = torch.empty(8, dtype=torch.int64, device="cuda")
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    sf.sortformer_segments(x, 0.01, None, out, cap, cnt)
    e0.record()
    for _ in range(10):
        sf.sortformer_segments(x, 0.01, None, out, cap, cnt)
    e1.record()
    torch.cuda.synchronize()
    print(f"[segments] 180000 x 8 frames: {e0.elapsed_time(e1) / 10 * 1e3:.1f} us per call",
          flush=True)


def test_segments_argument_checks(rt):
    from streaming_speaker_diarization_amd import sortformer as sf
    x = torch.rand(1, 10, 4, device="cuda")
    with pytest.raises(sf.SortformerError):
        rt.segments(x, 0.08, onset=0.3, offset=0.6)  # onset below offset
    with pytest.raises(sf.SortformerError):
        rt.segments(x, 0.08, pad_onset=-1.0)
    out = torch.empty(4 * 2 * sf.SEGMENT_BYTES, dtype=torch.uint8, device="cuda")
    cnt = torch.empty(4, dtype=torch.int64, device="cuda")
    with pytest.raises(sf.SortformerError):  # capacity 2 < (10 + 1) // 2
        sf.sortformer_segments(x, 0.08, None, out, 2, cnt)
    assert rt.segments(torch.zeros(2, 0, 4, device="cuda"), 0.08) == [[], []]
