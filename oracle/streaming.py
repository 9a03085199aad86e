"""Streaming schedule, FIFO and speaker-cache compression, float64 / exact.

"Streaming Sortformer Diarizer" model card, Streaming Architecture: each
step runs the encoder, transformer and head over [speaker_cache | FIFO |
current_chunk] and keeps the chunk's predictions; the FIFO holds recent
embeddings and its oldest frames are popped into the speaker cache when it
fills; the cache (188 frames) is compressed on overflow by keeping the
highest log-odds-scored frames per speaker plus silence placeholders; only
the new chunk is pre-encoded. Streaming Configurations: the four presets and
latency = (chunk_len + right_context) x 80 ms. Transformers docs "Nemotron 3
Diarization", streaming usage: look-ahead frames are attended but not
scored; the last chunk has no look-ahead and all remaining frames are
scored. NeMo API docs, SortformerStreamingState: the state holds the cache,
FIFO, their lengths and their predictions.

Readings (pages silent):
* known-length schedule (offline chunking, where the clip length is known):
  step s covers encoder frames [sL, min(Te,(s+1)L)); look-ahead is the next
  min(R, rest) frames, none on the last step;
* live schedule (streaming, where the end is only known at the final call,
  as in the Transformers streaming loop that yields full chunks while audio
  remains and then the rest with is_last_audio_chunk): a non-final step s
  needs the audio of encoder frames up to (s+1)L+R, i.e. 1280((s+1)L+R)+40
  samples (the last mel frame's window reaches 40 samples past its frame);
  the final step scores every remaining frame and has no look-ahead;
* FIFO predictions are refreshed from every step's window; cache
  predictions are frozen when frames enter the cache;
* pop rule: when the FIFO exceeds fifo_len, pop
  n = min(len, max(update_period, len - fifo_len)) oldest frames;
* popped frames whose max_s p <= 0.5 feed a running silence mean (float64
  sum in frame order, one division, rounded to the storage dtype);
* compression score: the workload's log p_s - log(1-p_s) + sum_{j!=s}
  log(1-p_j), evaluated as the monotone-equivalent product key
  K_s = (p_s/(1-p_s)) * prod_{j!=s, ascending}(1-p_j) with p clamped to
  [2^-24, 1-2^-24], every operation a correctly rounded float64 op;
  eligible frames have p_s > 0.5 and are not placeholders; per speaker the
  k = floor(C/S) - 3 largest keys win (ties -> earlier frame); block s of
  the new cache holds the winners in time order then placeholders; trailing
  C - S*floor(C/S) slots are placeholders (embedding = silence mean or 0,
  probabilities 0).
"""
from __future__ import annotations

import dataclasses

import numpy as np

CLAMP = 2.0 ** -24
PRESETS = {
    # chunk_len, right_context, fifo_len, update_period, spkcache_len (80 ms frames)
    "very_high": (340, 40, 40, 300, 188),
    "high": (124, 1, 124, 124, 188),
    "low": (6, 7, 188, 144, 188),
    "ultra_low": (3, 1, 188, 144, 188),
    # 0.64 s input-buffer latency (the Transformers very_low_latency mode): the
    # pages give only the total of 8 frames; read as the Low preset's 6-frame
    # chunk with a 2-frame look-ahead
    "very_low": (6, 2, 188, 144, 188),
    "nemotron_offline": (380, 0, 188, 192, 188),
}


@dataclasses.dataclass
class StreamConfig:
    chunk_len: int
    right_context: int
    fifo_len: int
    update_period: int
    spkcache_len: int = 188
    n_sil: int = 3

    @classmethod
    def preset(cls, name):
        return cls(*PRESETS[name])

    def latency_ms(self) -> int:
        return (self.chunk_len + self.right_context) * 80


def schedule(Te: int, cfg: StreamConfig):
    """List of (chunk_start, chunk_n, rc_n, is_last) over Te encoder frames."""
    steps = []
    s = 0
    while s * cfg.chunk_len < Te:
        c0 = s * cfg.chunk_len
        c1 = min(Te, c0 + cfg.chunk_len)
        last = c1 == Te
        rc = 0 if last else min(cfg.right_context, Te - c1)
        steps.append((c0, c1 - c0, rc, last))
        s += 1
    return steps


def live_schedule(n_samples: int, cfg: StreamConfig, hop: int = 160, sub: int = 8):
    """Schedule of a live stream of n_samples samples: (start, n, rc, last)."""
    T = n_samples // hop
    Te = (T + sub - 1) // sub
    L, R = cfg.chunk_len, cfg.right_context
    steps = []
    s = 0
    while hop * sub * ((s + 1) * L + R) + 40 <= n_samples:
        steps.append((s * L, L, R, False))
        s += 1
    steps.append((s * L, Te - s * L, 0, True))
    return steps


def samples_needed(step: int, cfg: StreamConfig) -> int:
    """Samples the live stream must have received before non-final step s."""
    if step == 0:
        return 1280 * (cfg.chunk_len + cfg.right_context) + 40
    return 1280 * cfg.chunk_len


@dataclasses.dataclass
class State:
    cache_emb: np.ndarray
    cache_probs: np.ndarray
    cache_ph: np.ndarray          # placeholder flags
    fifo_emb: np.ndarray
    fifo_probs: np.ndarray
    sil_sum: np.ndarray           # float64 (D,)
    sil_count: int

    @classmethod
    def empty(cls, d: int, n_spk: int, dtype=np.float64):
        return cls(np.zeros((0, d), dtype), np.zeros((0, n_spk), dtype), np.zeros(0, bool),
                   np.zeros((0, d), dtype), np.zeros((0, n_spk), dtype),
                   np.zeros(d, np.float64), 0)

    def copy(self):
        return dataclasses.replace(self, **{f.name: np.copy(getattr(self, f.name))
                                            for f in dataclasses.fields(self)
                                            if f.name != "sil_count"})


def score_keys(probs):
    """(M,S) probabilities -> (M,S) float64 keys K_s (exact IEEE sequence)."""
    p = np.clip(np.asarray(probs, dtype=np.float64), CLAMP, 1.0 - CLAMP)
    M, S = p.shape
    one_minus = 1.0 - p
    keys = np.empty((M, S))
    for s in range(S):
        k = p[:, s] / one_minus[:, s]
        for j in range(S):
            if j != s:
                k = k * one_minus[:, j]
        keys[:, s] = k
    return keys


def compress(state: State, cfg: StreamConfig, n_spk: int):
    """Compress the speaker cache to exactly spkcache_len frames (in place)."""
    C = cfg.spkcache_len
    per = C // n_spk
    k = per - cfg.n_sil
    M, d = state.cache_emb.shape
    dtype = state.cache_emb.dtype
    keys = score_keys(state.cache_probs)
    eligible = (np.asarray(state.cache_probs, dtype=np.float64) > 0.5) & ~state.cache_ph[:, None]
    if state.sil_count > 0:
        sil = (state.sil_sum / state.sil_count).astype(dtype)
    else:
        sil = np.zeros(d, dtype)
    emb = np.empty((C, d), dtype)
    probs = np.zeros((C, n_spk), state.cache_probs.dtype)
    ph = np.ones(C, bool)
    emb[:] = sil
    for s in range(n_spk):
        cand = [m for m in range(M) if eligible[m, s]]
        cand.sort(key=lambda m: (-keys[m, s], m))
        chosen = sorted(cand[:k])
        for slot, m in enumerate(chosen):
            r = s * per + slot
            emb[r] = state.cache_emb[m]
            probs[r] = state.cache_probs[m]
            ph[r] = False
    state.cache_emb, state.cache_probs, state.cache_ph = emb, probs, ph


def fifo_update(state: State, window_probs, chunk_emb, n_chunk: int, cfg: StreamConfig,
                n_spk: int):
    """Refresh FIFO predictions, append the chunk, pop into the cache and
    compress when needed. Returns (popped count, compressed?)."""
    Lc = state.cache_emb.shape[0]
    Lf = state.fifo_emb.shape[0]
    dt_e, dt_p = state.fifo_emb.dtype, state.fifo_probs.dtype
    state.fifo_probs = np.asarray(window_probs[Lc:Lc + Lf], dtype=dt_p).copy()
    state.fifo_emb = np.concatenate([state.fifo_emb, np.asarray(chunk_emb[:n_chunk], dt_e)])
    state.fifo_probs = np.concatenate(
        [state.fifo_probs, np.asarray(window_probs[Lc + Lf:Lc + Lf + n_chunk], dt_p)])
    Lf = state.fifo_emb.shape[0]
    popped = 0
    if Lf > cfg.fifo_len:
        n = min(Lf, max(cfg.update_period, Lf - cfg.fifo_len))
        pe, pp = state.fifo_emb[:n], state.fifo_probs[:n]
        for r in range(n):
            if np.max(np.asarray(pp[r], dtype=np.float64)) <= 0.5:
                state.sil_sum = state.sil_sum + np.asarray(pe[r], dtype=np.float64)
                state.sil_count += 1
        state.cache_emb = np.concatenate([state.cache_emb, pe])
        state.cache_probs = np.concatenate([state.cache_probs, pp])
        state.cache_ph = np.concatenate([state.cache_ph, np.zeros(n, bool)])
        state.fifo_emb, state.fifo_probs = state.fifo_emb[n:].copy(), state.fifo_probs[n:].copy()
        popped = n
    compressed = False
    if state.cache_emb.shape[0] > cfg.spkcache_len:
        compress(state, cfg, n_spk)
        compressed = True
    return popped, compressed


def stream_step(state: State, emb_new, n_chunk: int, cfg: StreamConfig, encode, n_spk: int):
    """One step. emb_new: (n_chunk + n_rc, D) pre-encoded chunk and
    look-ahead. ``encode(window) -> (probs80 (W,S), emitted-rate probs)``.
    Returns the chunk's emitted probabilities."""
    window = np.concatenate([np.asarray(state.cache_emb, np.float64),
                             np.asarray(state.fifo_emb, np.float64),
                             np.asarray(emb_new, np.float64)])
    p80, pout = encode(window)
    Lc, Lf = state.cache_emb.shape[0], state.fifo_emb.shape[0]
    rate = pout.shape[0] // p80.shape[0]
    out = pout[rate * (Lc + Lf):rate * (Lc + Lf + n_chunk)]
    fifo_update(state, p80, emb_new, n_chunk, cfg, n_spk)
    return out


def run_stream(emb, cfg: StreamConfig, encode, n_spk: int, state: State | None = None,
               steps=None, on_step=None, sched=None):
    """Run a schedule (default: known-length) over pre-encoded embeddings (Te, D)."""
    Te, d = emb.shape
    if state is None:
        state = State.empty(d, n_spk)
    if sched is None:
        sched = schedule(Te, cfg)
    outs = []
    for si, (c0, cn, rc, last) in enumerate(sched):
        if cn == 0:
            break
        if steps is not None and si >= steps:
            break
        if on_step is not None:
            on_step(si, state)
        outs.append(stream_step(state, emb[c0:c0 + cn + rc], cn, cfg, encode, n_spk))
    return np.concatenate(outs) if outs else np.zeros((0, n_spk)), state
