"""GPU checks of the boundary's stream-state calls: the model metadata, full
checkpoint / resume (NeMo API docs, SortformerStreamingState; Transformers
speaker_cache), the streaming feed of arbitrary sample counts and the final
flush (ExecuTorch issue, Proposed scope: the runner feeds audio as it comes,
resets between recordings and flushes the last chunk), and the refusals that
keep a stream's counters consistent."""
import numpy as np
import pytest
import torch

from oracle import run as OR
from oracle import streaming as OST
from oracle.weights import make_weights
from synthetic import meeting_audio, workload_audio

pytestmark = pytest.mark.gpu


def _cuda(x):
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).cuda()


@pytest.fixture(scope="module")
def rt():
    from streaming_speaker_diarization_amd import runtime
    return runtime


@pytest.fixture(scope="module")
def sf():
    from streaming_speaker_diarization_amd import sortformer
    return sortformer


@pytest.fixture(scope="module")
def sfbf(rt):
    return rt.Model("sortformer", "bf16", seed=0)


@pytest.fixture(scope="module")
def sf32(rt):
    return rt.Model("sortformer", "f32", seed=0)


def test_metadata_constants(rt, sfbf):
    """Exported Methods, Metadata of the model card: 16 kHz, 10 ms mel stride,
    8x subsampling, FastConformer 512, Transformer 192, 4 speakers, cache 188."""
    md = sfbf.metadata()
    assert (md["sample_rate"], md["subsampling_factor"], md["fc_d_model"], md["tf_d_model"],
            md["max_num_of_spks"], md["spkcache_len"]) == (16000, 8, 512, 192, 4, 188)
    assert md["window_stride"] == 0.01 and md["output_frame_s"] == 0.08
    assert (md["n_mels"], md["n_fft"], md["win_length"], md["hop_length"]) == (128, 512, 400, 160)
    assert (md["n_conformer_layers"], md["n_transformer_layers"], md["n_heads"]) == (17, 18, 8)
    nm = rt.Model("nemotron", "f32", seed=1).metadata()
    assert (nm["max_num_of_spks"], nm["fc_d_model"], nm["tf_d_model"], nm["output_frame_s"],
            nm["n_transformer_layers"]) == (8, 0, 512, 0.01, 31)


def _run_steps(st, audio, pos, n_steps=None):
    """Fixed-size steps from sample pos (final step when the clip ends) -> (outputs, pos)."""
    outs, N, k = [], audio.shape[1], 0
    while (n_steps is None or k < n_steps) and not st.info()[0]["finished"]:
        need = st.samples_needed()
        last = pos + need > N
        n = N - pos if last else need
        outs.append(st.step(audio[:, pos:pos + n], is_last=last).clone())
        pos += n
        k += 1
    return outs, pos


@pytest.mark.parametrize("k", [20, 31, 60, 123])
def test_checkpoint_resume_bit_identical(sfbf, k):
    """Export after k steps of the 60 s 'low' stream (before the first pop, at
    it, after the first compression, before the final step), import into a
    fresh stream object and finish there: identical to the uninterrupted run.
    The exporting stream, rewound by importing its own checkpoint after
    running to the end, replays the same rest."""
    audio = _cuda(workload_audio("low60s"))[None]
    ref = sfbf.stream("low").run(audio)
    a = sfbf.stream("low")
    head, pos = _run_steps(a, audio, 0, k)
    blob = a.export()
    info_a = a.info()[0]
    b = sfbf.stream("low")
    b.import_(blob)
    assert b.info()[0] == info_a
    tail, _ = _run_steps(b, audio, pos)
    got = torch.cat(head + tail, dim=1)
    assert got.shape == ref.shape and torch.equal(got, ref), k
    rest_a, _ = _run_steps(a, audio, pos)
    a.import_(blob)
    again, _ = _run_steps(a, audio, pos)
    assert torch.equal(torch.cat(again, dim=1), torch.cat(tail, dim=1))
    assert torch.equal(torch.cat(rest_a, dim=1), torch.cat(tail, dim=1))


def test_checkpoint_batched_with_pending_samples(sfbf):
    """Three lockstep streams fed in uneven pieces; the checkpoint taken with
    samples pending in the ring resumes bit-identically."""
    audio = _cuda(np.stack([meeting_audio(14.0, 3, 300 + b) for b in range(3)]))
    ref = sfbf.stream("ultra_low", batch=3).run(audio)
    a = sfbf.stream("ultra_low", batch=3)
    cut = 70_001
    head = a.feed(audio[:, :cut])
    assert a.info()[0]["pending"] > 0
    blob = a.export()
    b = sfbf.stream("ultra_low", batch=3)
    b.import_(blob)
    tail = b.feed(audio[:, cut:], is_last=True)
    got = torch.cat([head, tail], dim=1)
    assert got.shape == ref.shape and torch.equal(got, ref)


def test_import_rejects_foreign_or_corrupt_blobs(sf, sfbf):
    audio = _cuda(meeting_audio(6.0, 2, 310))[None]
    a = sfbf.stream("low")
    _run_steps(a, audio, 0, 5)
    blob = a.export()
    fresh_ref = sfbf.stream("low").run(audio)
    for bad, what in [(sfbf.stream("ultra_low"), "other configuration"),
                      (sfbf.stream("low", batch=2), "other batch")]:
        with pytest.raises(sf.SortformerError) as e:
            bad.import_(blob)
        assert e.value.status == sf.SF_EINVAL, what
    b = sfbf.stream("low")
    for corrupt in (np.concatenate([np.zeros(8, np.uint8), blob[8:]]),  # magic
                    blob[:200],                                         # truncated header
                    blob[:-4096]):                                      # truncated body
        with pytest.raises(sf.SortformerError) as e:
            b.import_(corrupt)
        assert e.value.status == sf.SF_EINVAL
    # a refused import leaves the stream as it was: it still runs a fresh clip
    assert torch.equal(b.run(audio), fresh_ref)


def test_rows_only_stream_refuses_steps(sf, sfbf):
    """Rows written by the set_rows test hook leave the step counters alone:
    steps, feeds and exports are refused before any work until a reset."""
    st = sfbf.stream("low")
    rows = 40
    rng = np.random.default_rng(5)
    sf.sortformer_stream_set_rows(st.handle, 20, 20, 0, rng.normal(size=(1, rows, 512)),
                                  rng.random((1, rows, 4)), np.zeros((1, rows), np.int32),
                                  np.zeros((1, 512)), np.zeros(1, np.int32))
    audio = _cuda(meeting_audio(2.0, 2, 320))[None]
    need = st.samples_needed()
    for call in (lambda: st.step(audio[:, :need]), lambda: st.feed(audio), lambda: st.export()):
        with pytest.raises(sf.SortformerError) as e:
            call()
        assert e.value.status == sf.SF_ESTATE
    assert st.info()[0]["steps"] == 0
    st.reset()
    assert st.run(audio).shape == (1, 25, 4)


def test_step_refused_while_feed_samples_pending(sf, sfbf):
    st = sfbf.stream("low")
    audio = _cuda(meeting_audio(3.0, 2, 330))[None]
    assert st.feed(audio[:, :1000]).shape[1] == 0
    with pytest.raises(sf.SortformerError) as e:
        st.step(audio[:, :st.samples_needed()])
    assert e.value.status == sf.SF_ESTATE


@pytest.mark.parametrize("model,preset,B", [("bf16", "low", 1), ("bf16", "ultra_low", 2),
                                            ("bf16", "very_low", 1)])
def test_feed_any_sizes_equals_fixed_steps(sfbf, model, preset, B):
    """The same samples fed in random pieces (empty, sub-hop, several steps at
    once) give the fixed-step outputs bit for bit, and the final flush scores
    every remaining frame."""
    audio = _cuda(np.stack([meeting_audio(17.3, 3, 340 + b) for b in range(B)]))
    N = audio.shape[1]
    ref = sfbf.stream(preset, batch=B).run(audio)
    rng = np.random.default_rng(7)
    st = sfbf.stream(preset, batch=B)
    outs, pos = [], 0
    while pos < N:
        n = int(rng.choice([0, 37, 160, 1279, 1280, 3841, 9000, 40000]))
        n = min(n, N - pos)
        outs.append(st.feed(audio[:, pos:pos + n]))
        pos += n
    outs.append(st.feed(audio[:, N:], is_last=True))
    got = torch.cat(outs, dim=1)
    assert got.shape == ref.shape == (B, (N // 160 + 7) // 8, 4)
    assert torch.equal(got, ref)
    assert st.info()[0]["finished"] == 1


def test_feed_random_sizes_vs_oracle_live_schedule(sf32):
    """fp32, a small configuration: random feed sizes against the oracle's
    live schedule at the fp32 bar (max|dp| <= 1e-4)."""
    oc = OST.StreamConfig(chunk_len=4, right_context=2, fifo_len=20, update_period=8,
                          spkcache_len=24, n_sil=3)
    from streaming_speaker_diarization_amd import sortformer as sf
    c = sf.sf_stream_config(oc.chunk_len, oc.right_context, oc.fifo_len, oc.update_period,
                            oc.spkcache_len, oc.n_sil)
    audio = meeting_audio(12.0, 3, 350)
    st = sf32.stream(config=c)
    rng = np.random.default_rng(8)
    outs, pos, N = [], 0, len(audio)
    a = _cuda(audio)[None]
    while pos < N:
        n = min(int(rng.integers(0, 12000)), N - pos)
        outs.append(st.feed(a[:, pos:pos + n]))
        pos += n
    outs.append(st.feed(a[:, N:], is_last=True))
    got = torch.cat(outs, dim=1)[0].cpu().numpy()
    ref, _ = OR.sortformer_stream(audio, make_weights("sortformer", 0), oc)
    assert got.shape == ref.shape == (150, 4)
    err = float(np.abs(got - ref).max())
    print(f"[feed fp32 small cfg] max|dp| {err:.3e}", flush=True)
    assert err <= 1e-4


def test_feed_nemotron_rate(rt):
    """The Nemotron-style stream emits 8 rows per scored frame through feed too."""
    m = rt.Model("nemotron", "bf16", seed=1)
    from streaming_speaker_diarization_amd import sortformer as sf
    c = sf.sf_stream_config(20, 4, 40, 20, 48, 3)
    audio = _cuda(meeting_audio(9.0, 4, 360))[None]
    ref = m.stream(config=c).run(audio)
    st = m.stream(config=c)
    got = torch.cat([st.feed(audio[:, :33333]), st.feed(audio[:, 33333:], is_last=True)], dim=1)
    assert got.shape == ref.shape == (1, 8 * ((audio.shape[1] // 160 + 7) // 8), 8)
    assert torch.equal(got, ref)
