"""Audio tails and presets beyond the benchmark workloads, against the oracle.

Every clip length class the streaming front end can see: the mel frame count
takes all 16 remainders modulo 16 (so the encoder frame count ceil(T/8) takes
both parities and the last 80 ms frame is partial), plus a sub-hop sample
remainder. For the Low, 0.64 s and Ultra-low presets the live stream (the
clip fed as it arrives) is compared with the oracle's live schedule, output
lengths are checked, and a reset stream replays identically; the Nemotron
variant runs its 30.4 s offline configuration on the same lengths. The High
preset runs once over a longer clip. bf16 bar: max|dp| <= 2e-2 and >= 99.5%
agreement of p > 0.5.
"""
import numpy as np
import pytest
import torch

from oracle import run as OR
from oracle import streaming as OST
from oracle.weights import make_weights
from synthetic import meeting_audio

pytestmark = pytest.mark.gpu


def _cuda(x):
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).cuda()


def _check(name, got, ref):
    err = float(np.abs(got - ref).max()) if got.size else 0.0
    agree = float(np.mean((got > 0.5) == (ref > 0.5))) if got.size else 1.0
    print(f"[{name}] shape {got.shape} max|dp| {err:.3e} agree {agree:.5f}", flush=True)
    assert err <= 2e-2 and agree >= 0.995, name


def _clip(r, q, seed):
    T = 16 * q + r                 # mel frames
    n = 160 * T + (37 * r) % 160   # plus a partial hop
    return meeting_audio(n / 16000, 3, seed)[:n], T


@pytest.fixture(scope="module")
def sfbf():
    from streaming_speaker_diarization_amd import runtime
    return runtime.Model("sortformer", "bf16", seed=0)


@pytest.fixture(scope="module")
def wbf():
    return make_weights("sortformer", 0, bf16=True)


@pytest.mark.parametrize("preset", ["low", "very_low", "ultra_low"])
def test_stream_tails_all_remainders(sfbf, wbf, preset):
    cfg = OST.StreamConfig.preset(preset)
    for r in range(16):
        audio, T = _clip(r, 12, 900 + r)
        st = sfbf.stream(preset)
        got = st.run(_cuda(audio)[None])[0].cpu().numpy()
        ref, _ = OR.sortformer_stream(audio, wbf, cfg, live=True)
        assert got.shape == ref.shape == ((T + 7) // 8, 4), (preset, r)
        _check(f"{preset} tail T={T} N={len(audio)}", got, ref)
        st.reset()
        again = st.run(_cuda(audio)[None])[0].cpu().numpy()
        assert np.array_equal(again, got), (preset, r)


def test_short_inputs(sfbf, wbf):
    """Clips of a single encoder frame or less: one final step."""
    for n in (160, 1000, 1280, 1400):
        audio = meeting_audio(n / 16000, 2, 950 + n)[:n]
        got = sfbf.stream("low").run(_cuda(audio)[None])[0].cpu().numpy()
        ref, _ = OR.sortformer_stream(audio, wbf, OST.StreamConfig.preset("low"), live=True)
        assert got.shape == ref.shape == (((n // 160) + 7) // 8, 4)
        _check(f"short N={n}", got, ref)


def test_nemotron_offline_tails():
    from streaming_speaker_diarization_amd import runtime
    m = runtime.Model("nemotron", "bf16", seed=1)
    w = make_weights("nemotron", 1, bf16=True)
    for r in range(0, 16, 3):
        audio, T = _clip(r, 12, 970 + r)
        got = m.offline(_cuda(audio)[None])[0].cpu().numpy()
        ref, _ = OR.nemotron_offline(audio, w)
        assert got.shape == ref.shape == (8 * ((T + 7) // 8), 8)
        _check(f"nemotron offline tail T={T}", got, ref)


def test_high_preset(sfbf, wbf):
    audio = meeting_audio(22.3, 4, 990)
    cfg = OST.StreamConfig.preset("high")
    got = sfbf.stream("high").run(_cuda(audio)[None])[0].cpu().numpy()
    ref, _ = OR.sortformer_stream(audio, wbf, cfg, live=True)
    assert got.shape == ref.shape
    _check("high 22.3 s", got, ref)


def test_very_high_tails_all_remainders(sfbf, wbf):
    """'very high' (340 + 40 frames per step): clips of 3200-3215 mel frames
    give one full step and a final step of 60-62 frames, over all 16 mel-frame
    remainders."""
    cfg = OST.StreamConfig.preset("very_high")
    for r in range(16):
        audio, T = _clip(r, 200, 1100 + r)
        got = sfbf.stream("very_high").run(_cuda(audio)[None])[0].cpu().numpy()
        ref, _ = OR.sortformer_stream(audio, wbf, cfg, live=True)
        assert got.shape == ref.shape == ((T + 7) // 8, 4), r
        _check(f"very_high tail T={T} N={len(audio)}", got, ref)
