"""The allocation-free stream step (static scratch workspace) against the
regular step with a caller workspace: bit-identical outputs on two streams run
back to back, the second with a smaller batch and a shorter clip (so the
scratch holds the first stream's contents when the second starts), and a
refusal for streams whose workspace exceeds the scratch."""
import numpy as np
import pytest
import torch

from synthetic import meeting_audio

pytestmark = pytest.mark.gpu


def _cuda(x):
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).cuda()


def _run(st, audio, noalloc):
    from streaming_speaker_diarization_amd import sortformer as sf
    outs, pos, N = [], 0, audio.shape[1]
    while True:
        need = st.samples_needed()
        last = pos + need > N
        k = N - pos if last else need
        piece = audio[:, pos:pos + k].contiguous()
        if noalloc:
            n = sf.sortformer_stream_step_noalloc(st.handle, piece, k, last, st.out)
        else:
            n = sf.sortformer_stream_step(st.handle, piece, k, last, st.out, st.ws)
        outs.append(st.out.view(-1)[:st.B * n * 4].view(st.B, n, 4).clone())
        pos += k
        if last:
            return torch.cat(outs, dim=1)


def test_noalloc_step_matches_workspace_step():
    from streaming_speaker_diarization_amd import runtime
    from streaming_speaker_diarization_amd import sortformer as sf
    m = runtime.Model("sortformer", "bf16", seed=0)
    cases = [("low", 2, 21.7, 400), ("ultra_low", 1, 9.3, 401)]   # second: smaller input
    for preset, B, secs, seed in cases:
        print(f"[noalloc] preset {preset} B={B} {secs} s", flush=True)
        audio = _cuda(np.stack([meeting_audio(secs, 3, seed + b) for b in range(B)]))
        ref = _run(m.stream(preset, batch=B), audio, noalloc=False)
        got = _run(m.stream(preset, batch=B), audio, noalloc=True)
        assert got.shape == ref.shape and torch.equal(got, ref), preset
    for preset in ("low", "ultra_low", "very_low", "high"):
        c = sf.sortformer_stream_preset(preset)
        assert sf.sortformer_stream_workspace_bytes(m.handle, c, 1) <= sf.SF_NOALLOC_SCRATCH_BYTES
    big = m.stream("very_high")
    assert sf.sortformer_stream_workspace_bytes(m.handle, big.scfg, 1) > sf.SF_NOALLOC_SCRATCH_BYTES
    a = _cuda(meeting_audio(31.0, 2, 402))[None]
    with pytest.raises(sf.SortformerError) as e:
        sf.sortformer_stream_step_noalloc(big.handle, a[:, :big.samples_needed()].contiguous(),
                                          big.samples_needed(), False, big.out)
    assert e.value.status == sf.SF_ENOMEM
    assert big.info()[0]["steps"] == 0
