"""GPU parity of the streaming path: FIFO/cache update bit-exact against the
oracle when both are fed identical embeddings and probabilities, free-running
streams against the oracle's live schedule, lockstep batches, the
Nemotron-style chunked offline forward, and error/reset handling."""
import os

import numpy as np
import pytest
import torch

from oracle import frontend as OF
from oracle import nemotron as ON
from oracle import run as OR
from oracle import sortformer as OS
from oracle import streaming as OST
from oracle.weights import make_weights
from synthetic import meeting_audio, random_embeddings, random_probs, workload_audio

pytestmark = pytest.mark.gpu
GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _cuda(x):
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).cuda()


def _report(name, got, ref):
    err = float(np.abs(got - ref).max())
    agree = float(np.mean((got > 0.5) == (ref > 0.5)))
    print(f"[{name}] shape {got.shape} max|dp| {err:.3e} agree {agree:.5f}", flush=True)
    if not err <= 3e-2:  # say what the output looked like
        bad = np.argwhere(np.abs(got - ref) > 3e-2)
        print(f"  got range [{np.nanmin(got):.4g}, {np.nanmax(got):.4g}] nan {np.isnan(got).sum()}"
              f" | ref range [{ref.min():.4g}, {ref.max():.4g}] | {len(bad)} entries off, first"
              f" {bad[:4].tolist()} last {bad[-4:].tolist()}", flush=True)
    return err, agree


@pytest.fixture(scope="module")
def rt():
    from streaming_speaker_diarization_amd import runtime
    return runtime


@pytest.fixture(scope="module")
def sf():
    from streaming_speaker_diarization_amd import sortformer
    return sortformer


@pytest.fixture(scope="module")
def sf32(rt):
    return rt.Model("sortformer", "f32", seed=0)


@pytest.fixture(scope="module")
def sfbf(rt):
    return rt.Model("sortformer", "bf16", seed=0)


@pytest.fixture(scope="module")
def nmbf(rt):
    return rt.Model("nemotron", "bf16", seed=1)


# ------------------------------------------------------------- cache update
def _random_state(B, Lc, Lf, Lp, S, seed, kind, n_ph):
    emb = np.stack([random_embeddings(Lc + Lf + Lp, 512, seed + b) for b in range(B)])
    probs = np.stack([random_probs(Lc + Lf + Lp, S, seed + 100 + b, kind) for b in range(B)])
    flags = np.zeros((B, Lc + Lf + Lp), np.int32)
    flags[:, :n_ph] = 1
    probs[:, :n_ph] = 0.0
    sil_sum = np.stack([random_embeddings(1, 512, seed + 200 + b)[0].astype(np.float64) * 3
                        for b in range(B)])
    sil_cnt = np.arange(B, dtype=np.int32) + 2
    wprobs = np.stack([random_probs(Lc + Lf + Lp, S, seed + 300 + b, kind) for b in range(B)])
    return emb, probs, flags, sil_sum, sil_cnt, wprobs


@pytest.mark.parametrize("case", [
    # (model, preset, Lc, Lf, Lp, n_chunk, kind)
    ("sortformer", "low", 150, 186, 13, 6, "uniform"),      # pop 144 + compress (M = 294)
    ("sortformer", "low", 150, 186, 13, 6, "q256"),         # heavy ties
    ("sortformer", "low", 150, 186, 13, 6, "coarse"),       # exact 0.5 and ties
    ("sortformer", "low", 150, 186, 13, 6, "equal"),        # every key ties
    ("sortformer", "low", 20, 180, 13, 6, "uniform"),       # no pop
    ("sortformer", "very_high", 188, 40, 380, 340, "uniform"),  # pop 300, compress M = 488
    ("sortformer", "ultra_low", 0, 186, 4, 3, "uniform"),   # pop without compression
    ("nemotron", "nemotron_offline", 188, 188, 380, 380, "uniform"),  # S = 8, M = 568
    ("nemotron", "nemotron_offline", 188, 188, 380, 380, "q256"),
])
def test_cache_update_bit_exact(rt, sf, sfbf, nmbf, case):
    arch, preset, Lc, Lf, Lp, n_chunk, kind = case
    model = sfbf if arch == "sortformer" else nmbf
    S = model.n_spk
    B = 2
    st = model.stream(preset, batch=B)
    cfg = OST.StreamConfig.preset(preset)
    emb, probs, flags, sil_sum, sil_cnt, wprobs = _random_state(B, Lc, Lf, Lp, S, 11, kind, 5)
    sf.sortformer_stream_set_rows(st.handle, Lc, Lf, Lp, emb, probs, flags, sil_sum, sil_cnt)
    back = sf.sortformer_stream_get_rows(st.handle, S)
    assert np.array_equal(back["emb"], emb) and np.array_equal(back["probs"], probs)
    sf.sortformer_stream_update(st.handle, _cuda(wprobs), n_chunk, st.ws)
    got = sf.sortformer_stream_get_rows(st.handle, S)
    for b in range(B):
        o = OST.State(emb[b, :Lc].copy(), probs[b, :Lc].copy(), flags[b, :Lc].astype(bool),
                      emb[b, Lc:Lc + Lf].copy(), probs[b, Lc:Lc + Lf].copy(), sil_sum[b].copy(),
                      int(sil_cnt[b]))
        OST.fifo_update(o, wprobs[b], emb[b, Lc + Lf:], n_chunk, cfg, S)
        lc, lf = o.cache_emb.shape[0], o.fifo_emb.shape[0]
        assert (got["cache_len"], got["fifo_len"], got["lookahead_len"]) == (lc, lf, Lp - n_chunk)
        ref_emb = np.concatenate([o.cache_emb, o.fifo_emb, emb[b, Lc + Lf + n_chunk:]])
        assert np.array_equal(got["emb"][b], ref_emb)
        assert np.array_equal(got["probs"][b, :lc + lf],
                              np.concatenate([o.cache_probs, o.fifo_probs]).astype(np.float32))
        assert np.array_equal(got["flags"][b, :lc].astype(bool), o.cache_ph)
        assert not got["flags"][b, lc:lc + lf].any()
        assert np.array_equal(got["sil_sum"][b], o.sil_sum)
        assert got["sil_cnt"][b] == o.sil_count


# ------------------------------------------------------------- free running
def _small_cfg():
    return OST.StreamConfig(chunk_len=4, right_context=2, fifo_len=20, update_period=8,
                            spkcache_len=24, n_sil=3)


def test_stream_fp32_small_config_free_running(rt, sf, sf32):
    oc = _small_cfg()
    c = sf.sf_stream_config(oc.chunk_len, oc.right_context, oc.fifo_len, oc.update_period,
                            oc.spkcache_len, oc.n_sil)
    audio = meeting_audio(20.0, 3, 51)
    st = sf32.stream(config=c)
    got = st.run(_cuda(audio)[None])[0].cpu().numpy()
    ref, ost = OR.sortformer_stream(audio, make_weights("sortformer", 0), oc)
    assert got.shape == ref.shape == (250, 4)
    err, _ = _report("stream f32 small cfg", got, ref)
    assert err <= 1e-4
    info = st.info()[0]
    assert info["finished"] == 1 and info["frames_emitted"] == 250
    assert info["cache_len"] == ost.cache_emb.shape[0] and info["fifo_len"] == ost.fifo_emb.shape[0]


def test_stream_single_final_step_equals_offline(rt, sf, sf32):
    audio = workload_audio("offline8s")
    c = sf.sf_stream_config(100, 0, 0, 1, 188, 3)
    st = sf32.stream(config=c)
    got = st.run(_cuda(audio)[None]).cpu().numpy()
    off = sf32.offline(_cuda(audio)[None]).cpu().numpy()
    assert got.shape == off.shape == (1, 100, 4)
    assert np.array_equal(got, off)


def test_stream_errors_reset_and_determinism(rt, sf, sfbf):
    audio = _cuda(meeting_audio(6.0, 2, 61))[None]
    st = sfbf.stream("low")
    need = st.samples_needed()
    assert need == 1280 * 13 + 40
    with pytest.raises(sf.SortformerError) as e:
        st.step(audio[:, :need - 1])
    assert e.value.status == sf.SF_ESHAPE
    a = st.run(audio).cpu().numpy()
    with pytest.raises(sf.SortformerError) as e:
        st.step(audio[:, :10], is_last=True)
    assert e.value.status == sf.SF_ESTATE
    st.reset()
    b = st.run(audio).cpu().numpy()
    assert np.array_equal(a, b)


def _lockstep(sfbf, B, steps, check):
    n = 1280 * (steps * 3 + 1) + 40
    audio = np.stack([workload_audio("ultralow64x120s", stream=b, seconds=n / 16000 + 1)[:n]
                      for b in range(B)])
    st = sfbf.stream("ultra_low", batch=B)
    outs, pos = [], 0
    for s in range(steps):
        k = st.samples_needed()
        outs.append(st.step(_cuda(audio[:, pos:pos + k])).clone())
        pos += k
    got = torch.cat(outs, 1).cpu().numpy()
    for b in check:
        one = sfbf.stream("ultra_low", batch=1)
        o, pos = [], 0
        for s in range(steps):
            k = one.samples_needed()
            o.append(one.step(_cuda(audio[b:b + 1, pos:pos + k])).clone())
            pos += k
        single = torch.cat(o, 1)[0].cpu().numpy()
        yield b, got[b], single


def test_lockstep_small_batch_is_bit_exact(rt, sfbf):
    """Ultra-low preset, 6 streams in lockstep (every window under 4096 rows,
    the GEMMs' K slicing is the single-stream one): each stream equals the
    same stream run alone, bit for bit."""
    for b, got, single in _lockstep(sfbf, 6, 30, (0, 5)):
        err, _ = _report(f"lockstep B=6 b={b}", got, single)
        assert err == 0.0


def test_lockstep_batch_matches_single_streams(rt, sfbf):
    """Ultra-low preset, 64 streams in lockstep (30 steps): once the batched
    window exceeds 4096 rows the GEMMs run the whole K in one loop instead of
    the single stream's K slices, so each stream agrees with its solo run to
    the bf16 parity bar rather than bit for bit."""
    for b, got, single in _lockstep(sfbf, 64, 30, (0, 37, 63)):
        err, agree = _report(f"lockstep B=64 b={b}", got, single)
        assert err <= 2e-2 and agree >= 0.995


def test_state_forced_full_windows(rt, sfbf):
    """The full-size window of the very-high preset (W = 608), fed the same
    embeddings on both sides (the 64-stream workload's windows are checked
    on real oracle states in test_gpu_ultralow.py)."""
    w = make_weights("sortformer", 0, bf16=True)
    emb = OR.pre_encode_all(w, OF.log_mel(workload_audio("veryhigh600s", seconds=60.0)))
    x = emb[100:708]
    got = sfbf.encode_window(_cuda(x)[None])[0].cpu().numpy()
    err, agree = _report("state-forced very_high W=608", got, OS.encode_window(w, x))
    assert err <= 2e-2 and agree >= 0.995


def test_nemotron_offline_fp32_two_chunks(rt):
    m = rt.Model("nemotron", "f32", seed=1)
    audio = meeting_audio(50.0, 5, 71, arrival_order=True)
    got = m.offline(_cuda(audio)[None])[0].cpu().numpy()
    ref, _ = OR.nemotron_offline(audio, make_weights("nemotron", 1))
    assert got.shape == ref.shape == (8 * 625, 8)
    err, _ = _report("nemotron offline f32 50 s", got, ref)
    assert err <= 1e-4


def test_nemotron_state_forced_full_window(nmbf):
    w = make_weights("nemotron", 1, bf16=True)
    emb = ON.pre_encode(w, OF.log_mel(workload_audio("nemotron1800s", seconds=70.0)))[:756]
    p80, p10 = nmbf.encode_window(_cuda(emb)[None])
    r80, r10 = ON.encode_window(w, emb)
    err, agree = _report("nemotron state-forced W=756", p10[0].cpu().numpy(), r10)
    assert err <= 2e-2 and agree >= 0.995


@pytest.mark.parametrize("name,preset", [("low60s", "low"), ("veryhigh600s", "very_high")])
def test_full_stream_vs_golden(rt, sfbf, name, preset):
    path = os.path.join(GOLD, f"{name}_bf16.npy")
    ref = np.load(path)
    st = sfbf.stream(preset)
    got = st.run(_cuda(workload_audio(name))[None])[0].cpu().numpy()
    assert got.shape == ref.shape
    err, agree = _report(f"free-running {name} bf16", got, ref)
    assert err <= 2e-2 and agree >= 0.995


def test_nemotron_1800s_vs_golden(nmbf):
    ref = np.load(os.path.join(GOLD, "nemotron1800s_bf16.npy"))
    got = nmbf.offline(_cuda(workload_audio("nemotron1800s"))[None])[0].cpu().numpy()
    assert got.shape == ref.shape == (180000, 8)
    err, agree = _report("nemotron 1800 s bf16", got, ref)
    assert err <= 2e-2 and agree >= 0.995


def test_graph_replays_match_direct_launches(rt, sf, sfbf):
    """Window forwards replayed from captured HIP graphs equal the direct
    launches bit for bit, on every replay (three passes, eager work and
    synchronisations between them)."""
    audio = _cuda(meeting_audio(25.0, 4, 81))[None]
    st = sfbf.stream("low")
    sf.sortformer_stream_set_option(st.handle, sf.SF_STREAM_OPT_GRAPHS, 0)
    ref = st.run(audio).cpu().numpy()
    sf.sortformer_stream_set_option(st.handle, sf.SF_STREAM_OPT_GRAPHS, 1)
    for rep in range(3):
        st.reset()
        got = st.run(audio).cpu().numpy()
        torch.cuda.synchronize()
        _ = (torch.randn(1000, device="cuda") * 2).sum().item()   # eager work in between
        assert np.array_equal(got, ref), f"replay {rep}"
    # a step with another workspace releases the cached graphs and captures
    # new ones; the workspace holds nothing across steps: results unchanged
    st.reset()
    ws_a, ws_b = st.ws, torch.full_like(st.ws, 0x7F)
    outs, pos, n, k = [], 0, audio.shape[1], 0
    while True:
        st.ws = ws_b if (k // 5) % 2 else ws_a
        need = st.samples_needed()
        if pos + need > n:
            outs.append(st.step(audio[:, pos:n], is_last=True).clone())
            break
        outs.append(st.step(audio[:, pos:pos + need]).clone())
        pos += need
        k += 1
    st.ws = ws_a
    assert k > 10
    assert np.array_equal(torch.cat(outs, dim=1).cpu().numpy(), ref), "workspace switches"
    b = sfbf.stream("ultra_low", batch=3)
    a3 = _cuda(np.stack([meeting_audio(8.0, 2, 90 + i) for i in range(3)]))
    sf.sortformer_stream_set_option(b.handle, sf.SF_STREAM_OPT_GRAPHS, 0)
    r3 = b.run(a3).cpu().numpy()
    sf.sortformer_stream_set_option(b.handle, sf.SF_STREAM_OPT_GRAPHS, 1)
    for rep in range(2):
        b.reset()
        assert np.array_equal(b.run(a3).cpu().numpy(), r3), f"batched replay {rep}"


def test_sortformer_offline_beyond_one_window(rt, sfbf):
    """A 100 s clip (1250 encoder frames, past the 1024-frame single window)
    runs in 'very high' chunks: two clips batched against the oracle's
    chunked offline forward at the bf16 bar, and the batch against each clip
    run alone, bit for bit."""
    w = make_weights("sortformer", 0, bf16=True)
    clips = [meeting_audio(100.0, 4, 600 + i) for i in range(2)]
    got = sfbf.offline(_cuda(np.stack(clips))).cpu().numpy()
    assert got.shape == (2, 1250, 4)
    ref = OR.sortformer_offline(clips[0], w)
    err, agree = _report("offline 100 s bf16 (chunked)", got[0], ref)
    assert err <= 2e-2 and agree >= 0.995
    for i in range(2):
        one = sfbf.offline(_cuda(clips[i])[None])[0].cpu().numpy()
        assert np.array_equal(one, got[i])
