"""Pins of the oracle's streaming schedule, FIFO and cache compression:
page-stated presets/latencies, brute force and invariants."""
import json
import os

import numpy as np
import pytest

from oracle import streaming as S
from synthetic import random_embeddings, random_probs

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "page_facts.json")))


def test_presets_and_latency():
    for row in GOLD["presets"]["rows"]:
        cfg = S.StreamConfig.preset(row["name"])
        assert (cfg.chunk_len, cfg.right_context, cfg.fifo_len, cfg.update_period,
                cfg.spkcache_len) == (row["chunk_len"], row["right_context"], row["fifo_len"],
                                      row["update_period"], row["spkcache_len"])
        assert cfg.latency_ms() == round(row["latency_s"] * 1000)
    assert S.StreamConfig.preset("low").latency_ms() / 1000 == \
        GOLD["transformers_streaming_modes_s"]["low_latency"]
    assert S.StreamConfig.preset("ultra_low").latency_ms() / 1000 == \
        GOLD["transformers_streaming_modes_s"]["ultra_low_latency"]
    # the 0.64 s mode (its chunk / look-ahead split is a reading; the total is the page's)
    assert S.StreamConfig.preset("very_low").latency_ms() / 1000 == \
        GOLD["transformers_streaming_modes_s"]["very_low_latency"]
    assert S.StreamConfig.preset("nemotron_offline").latency_ms() / 1000 == \
        GOLD["nemotron_offline_buffer_s"]["value"]


def test_schedule_covers_frames_once():
    for Te in (1, 2, 5, 13, 750, 7500, 7501):
        for name in ("very_high", "high", "low", "ultra_low", "nemotron_offline"):
            cfg = S.StreamConfig.preset(name)
            sch = S.schedule(Te, cfg)
            covered = np.concatenate([np.arange(c0, c0 + n) for c0, n, _, _ in sch])
            assert np.array_equal(covered, np.arange(Te))
            assert sch[-1][3] and sch[-1][2] == 0 and not any(s[3] for s in sch[:-1])
            for c0, n, rc, last in sch:
                assert c0 + n + rc <= Te


def _simulate(Te, cfg, n_spk=4, seed=0):
    """Drive the FIFO/cache with random probabilities; record lengths."""
    st = S.State.empty(8, n_spk)
    rng = np.random.default_rng(seed)
    log = []
    for si, (c0, n, rc, last) in enumerate(S.schedule(Te, cfg)):
        Lc, Lf = st.cache_emb.shape[0], st.fifo_emb.shape[0]
        W = Lc + Lf + n + rc
        probs = rng.random((W, n_spk))
        emb = np.full((n + rc, 8), float(c0))[:, :] + np.arange(n + rc)[:, None]
        popped, comp = S.fifo_update(st, probs, emb, n, cfg, n_spk)
        log.append((si, W, Lc, Lf, popped, comp))
    return log, st


def test_pop_and_compression_cadence():
    log, _ = _simulate(750, S.StreamConfig.preset("low"))
    assert [s for s, *_, p, c in log if p] == [31, 55, 79, 103]
    assert [s for s, *_, c in log if c] == [55, 79, 103]
    assert max(W for _, W, *_ in log) == 387 and len(log) == 125
    log, _ = _simulate(1500, S.StreamConfig.preset("ultra_low"))
    comp = [s for s, *_, c in log if c]
    assert comp[0] == 110 and len(comp) == 9 and len(log) == 500
    assert max(W for _, W, *_ in log) == 378
    log, _ = _simulate(7500, S.StreamConfig.preset("very_high"))
    assert len(log) == 23 and log[0][1] == 380 and max(W for _, W, *_ in log) == 608
    assert all(c for *_, c in log[1:])
    log, _ = _simulate(22500, S.StreamConfig.preset("nemotron_offline"), n_spk=8)
    assert len(log) == 60 and log[0][1] == 380 and max(W for _, W, *_ in log) == 756


def test_live_schedule():
    cfg = S.StreamConfig.preset("low")
    sch = S.live_schedule(60 * 16000, cfg)
    assert len(sch) == 124 and sch[-1] == (738, 12, 0, True)
    assert all(s[1:] == (6, 7, False) for s in sch[:-1])
    # samples needed accumulate to what each non-final step consumes
    got = 0
    for i, (c0, n, rc, last) in enumerate(sch[:-1]):
        got += S.samples_needed(i, cfg)
        assert got == 1280 * (c0 + n + rc) + 40
    assert len(S.live_schedule(120 * 16000, S.StreamConfig.preset("ultra_low"))) == 500
    vh = S.live_schedule(600 * 16000, S.StreamConfig.preset("very_high"))
    assert len(vh) == 22 and vh[-1] == (7140, 360, 0, True)
    # a clip shorter than the first window is one final step
    assert S.live_schedule(1280 * 5, cfg) == [(0, 5, 0, True)]
    # every frame is scored exactly once
    for n in (1280 * 13 + 39, 1280 * 13 + 40, 1280 * 40 + 500, 160 * 7):
        sch = S.live_schedule(n, cfg)
        Te = (n // 160 + 7) // 8
        cov = np.concatenate([np.arange(c0, c0 + k) for c0, k, _, _ in sch])
        assert np.array_equal(cov, np.arange(Te))


def test_fifo_conservation():
    cfg = S.StreamConfig(chunk_len=5, right_context=2, fifo_len=12, update_period=7,
                         spkcache_len=10_000)
    st = S.State.empty(1, 2)
    popped = []
    rng = np.random.default_rng(1)
    Te = 97
    for c0, n, rc, last in S.schedule(Te, cfg):
        Lc, Lf = st.cache_emb.shape[0], st.fifo_emb.shape[0]
        W = Lc + Lf + n + rc
        emb = np.arange(c0, c0 + n + rc, dtype=float)[:, None]
        S.fifo_update(st, rng.random((W, 2)), emb, n, cfg, 2)
        assert st.fifo_emb.shape[0] <= max(cfg.fifo_len, 0) + cfg.chunk_len
    seq = np.concatenate([st.cache_emb[:, 0], st.fifo_emb[:, 0]])
    assert np.array_equal(seq, np.arange(Te, dtype=float))


def test_fifo_probs_refresh_and_cache_frozen():
    cfg = S.StreamConfig(chunk_len=2, right_context=0, fifo_len=3, update_period=2,
                         spkcache_len=100)
    st = S.State.empty(1, 1)
    S.fifo_update(st, np.array([[0.1], [0.2]]), np.zeros((2, 1)), 2, cfg, 1)
    S.fifo_update(st, np.array([[0.3], [0.4], [0.5], [0.6]]), np.ones((2, 1)), 2, cfg, 1)
    # fifo (4 > 3) pops max(2, 1) = 2 frames with their refreshed probs 0.3, 0.4
    assert np.allclose(st.cache_probs[:, 0], [0.3, 0.4])
    assert np.allclose(st.fifo_probs[:, 0], [0.5, 0.6])
    S.fifo_update(st, np.array([[0.9], [0.9], [0.7], [0.8], [0.1], [0.1]]), 2 * np.ones((2, 1)),
                  2, cfg, 1)
    assert np.allclose(st.cache_probs[:, 0], [0.3, 0.4, 0.7, 0.8])   # frozen entries kept


def test_score_key_is_monotone_in_log_odds_score():
    p = random_probs(4000, 4, 3).astype(np.float64)
    p = np.clip(p, S.CLAMP, 1 - S.CLAMP)
    keys = S.score_keys(p)
    for s in range(4):
        logscore = np.log(p[:, s]) - np.log(1 - p[:, s]) + sum(
            np.log(1 - p[:, j]) for j in range(4) if j != s)
        assert np.allclose(np.log(keys[:, s]), logscore, atol=1e-12)
        order_k = np.argsort(-keys[:, s], kind="stable")
        order_l = np.argsort(-logscore, kind="stable")
        gap = np.abs(np.diff(np.sort(logscore)))
        if gap.min() > 1e-10:
            assert np.array_equal(order_k, order_l)


def _brute_force(emb, probs, ph, sil, cfg, n_spk):
    C = cfg.spkcache_len
    per = C // n_spk
    k = per - cfg.n_sil
    M = emb.shape[0]
    p = np.clip(probs.astype(np.float64), S.CLAMP, 1 - S.CLAMP)
    rows = []
    for s in range(n_spk):
        elig = [m for m in range(M) if probs[m, s] > 0.5 and not ph[m]]
        # full sort by (score desc, index asc) with the log score; ties resolved by index
        sc = {m: np.log(p[m, s] / (1 - p[m, s])) + sum(np.log(1 - p[m, j]) for j in range(n_spk)
                                                       if j != s) for m in elig}
        ranked = sorted(elig, key=lambda m: (-sc[m], m))
        chosen = sorted(ranked[:k])
        rows += chosen + [-1] * (per - len(chosen))
    rows += [-1] * (C - n_spk * per)
    return rows


@pytest.mark.parametrize("kind", ["uniform", "coarse", "q256", "equal"])
@pytest.mark.parametrize("n_spk", [4, 8])
def test_compress_brute_force_and_invariants(kind, n_spk):
    cfg = S.StreamConfig(chunk_len=1, right_context=0, fifo_len=1, update_period=1,
                         spkcache_len=188)
    M = 332
    emb = random_embeddings(M, 16, 5)
    emb[:, 0] = np.arange(M)                       # row id travels with the frame
    probs = random_probs(M, n_spk, 6, kind)
    ph = np.zeros(M, bool)
    ph[::17] = True
    st = S.State(emb.copy(), probs.copy(), ph.copy(), np.zeros((0, 16), np.float32),
                 np.zeros((0, n_spk), np.float32), np.arange(16, dtype=np.float64) * 3.0, 4)
    S.compress(st, cfg, n_spk)
    assert st.cache_emb.shape == (188, 16) and st.cache_emb.dtype == np.float32
    per = 188 // n_spk
    k = per - 3
    got_rows = [int(st.cache_emb[r, 0]) if not st.cache_ph[r] else -1 for r in range(188)]
    if kind in ("uniform",):
        assert got_rows == _brute_force(emb, probs, ph, None, cfg, n_spk)
    keys = S.score_keys(probs)
    sil = (np.arange(16) * 3.0 / 4).astype(np.float32)
    for s in range(n_spk):
        blk = got_rows[s * per:(s + 1) * per]
        real = [m for m in blk if m >= 0]
        assert len(real) <= k and real == sorted(real)
        assert blk[:len(real)] == real                  # winners first, then placeholders
        elig = [m for m in range(M) if probs[m, s] > 0.5 and not ph[m]]
        assert all(m in elig for m in real)
        assert len(real) == min(k, len(elig))
        lost = [m for m in elig if m not in real]
        if real and lost:
            kmin = min(keys[m, s] for m in real)
            assert all(keys[m, s] <= kmin for m in lost)
            # ties at the boundary go to the earlier frame
            tied = [m for m in lost if keys[m, s] == kmin]
            assert all(m > max(r for r in real if keys[r, s] == kmin) for m in tied)
    for r in range(188):
        if st.cache_ph[r]:
            assert np.array_equal(st.cache_emb[r], sil) and np.all(st.cache_probs[r] == 0)


def test_compress_idempotent_on_single_speaker_frames():
    """With at most one speaker above 0.5 per frame no frame can sit in two
    blocks, so compressing a compressed cache again changes nothing."""
    cfg = S.StreamConfig(1, 0, 1, 1, 188)
    M = 400
    probs = random_probs(M, 4, 12)
    top = np.argmax(probs, axis=1)
    probs = np.where(np.arange(4)[None, :] == top[:, None], probs, probs * 0.5).astype(np.float32)
    st = S.State(random_embeddings(M, 8, 13), probs, np.zeros(M, bool), np.zeros((0, 8)),
                 np.zeros((0, 4)), np.ones(8), 3)
    S.compress(st, cfg, 4)
    again = st.copy()
    S.compress(again, cfg, 4)
    assert np.array_equal(again.cache_emb, st.cache_emb)
    assert np.array_equal(again.cache_probs, st.cache_probs)
    assert np.array_equal(again.cache_ph, st.cache_ph)


def test_compress_speaker_relabel_permutes_blocks():
    cfg = S.StreamConfig(1, 0, 1, 1, 188)
    M = 300
    emb = random_embeddings(M, 4, 7)
    probs = random_probs(M, 4, 8)
    perm = np.array([2, 0, 3, 1])
    a = S.State(emb.copy(), probs.copy(), np.zeros(M, bool), np.zeros((0, 4)), np.zeros((0, 4)),
                np.zeros(4), 0)
    b = S.State(emb.copy(), probs[:, perm].copy(), np.zeros(M, bool), np.zeros((0, 4)),
                np.zeros((0, 4)), np.zeros(4), 0)
    S.compress(a, cfg, 4)
    S.compress(b, cfg, 4)
    for s in range(4):
        # new speaker s is old speaker perm[s]
        assert np.array_equal(b.cache_emb[47 * s:47 * s + 47], a.cache_emb[47 * perm[s]:47 * perm[s] + 47])


def test_silence_mean_from_popped_frames():
    cfg = S.StreamConfig(chunk_len=4, right_context=0, fifo_len=2, update_period=3,
                         spkcache_len=4)
    st = S.State.empty(2, 2, dtype=np.float32)
    probs = np.array([[0.2, 0.4], [0.9, 0.1], [0.5, 0.5], [0.3, 0.6]])
    emb = np.array([[1, 2], [3, 4], [5, 6], [7, 8]], np.float32)
    S.fifo_update(st, probs, emb, 4, cfg, 2)
    # 4 > 2: pop max(3, 2) = 3 frames; frames 0 and 2 are silent (max p <= 0.5)
    assert st.sil_count == 2 and np.array_equal(st.sil_sum, [6.0, 8.0])
    assert st.cache_emb.shape[0] == 3
