"""Nemotron-style output resolution (Transformers docs "Nemotron 3
Diarization", Overview: output frames configurable in 10 ms steps; 10 ms by
default per the model-card summary): frames of r x 10 ms, r in {1, 2, 4, 8},
each the mean of r consecutive 10 ms probabilities. Offline fp32 against the
oracle's pooled output (max|dp| <= 1e-4), a stream against its own 10 ms run
pooled, and the option's refusals."""
import numpy as np
import pytest
import torch

from oracle import nemotron as ON
from oracle import run as OR
from oracle.weights import make_weights
from synthetic import meeting_audio

pytestmark = pytest.mark.gpu


def _cuda(x):
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).cuda()


@pytest.fixture(scope="module")
def nm32():
    from streaming_speaker_diarization_amd import runtime
    return runtime.Model("nemotron", "f32", seed=1)


def test_offline_strides_vs_oracle(nm32):
    audio = meeting_audio(35.0, 5, 401, arrival_order=True)
    ref10, _ = OR.nemotron_offline(audio, make_weights("nemotron", 1))
    Te = (len(audio) // 160 + 7) // 8
    for r in (1, 2, 4, 8):
        nm32.set_output_stride(r)
        got = nm32.offline(_cuda(audio)[None])[0].cpu().numpy()
        ref = ON.pool_output(ref10, r)
        assert got.shape == ref.shape == (8 // r * Te, 8)
        err = float(np.abs(got - ref).max())
        print(f"[nemotron offline f32 stride {r} ({10 * r} ms)] max|dp| {err:.3e}", flush=True)
        assert err <= 1e-4
    nm32.set_output_stride(1)


def test_stream_stride_is_the_pooled_10ms_stream(nm32):
    from streaming_speaker_diarization_amd import sortformer as sf
    c = sf.sf_stream_config(20, 4, 40, 20, 48, 3)
    audio = _cuda(meeting_audio(9.0, 4, 402))[None]
    nm32.set_output_stride(1)
    p10 = nm32.stream(config=c).run(audio)[0].cpu().numpy()
    for r in (2, 8):
        nm32.set_output_stride(r)
        st = nm32.stream(config=c)
        assert sf.sortformer_stream_max_emit(st.handle) == 8 // r * 24
        got = st.run(audio)[0].cpu().numpy()
        ref = ON.pool_output(p10.astype(np.float64), r)
        assert got.shape == ref.shape
        assert float(np.abs(got - ref).max()) <= 1e-6
    nm32.set_output_stride(1)


def test_stride_option_refusals(nm32):
    from streaming_speaker_diarization_amd import runtime
    from streaming_speaker_diarization_amd import sortformer as sf
    for bad in (0, 3, 16):
        with pytest.raises(sf.SortformerError) as e:
            nm32.set_output_stride(bad)
        assert e.value.status == sf.SF_EINVAL
    m = runtime.Model("sortformer", "f32", seed=0)
    with pytest.raises(sf.SortformerError) as e:
        m.set_output_stride(2)
    assert e.value.status == sf.SF_EUNSUPPORTED
    m.set_output_stride(1)
    assert m.output_stride() == 1 and nm32.output_stride() == 1
