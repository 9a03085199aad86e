"""Whole-workload drivers of the oracle (audio in, probabilities out)."""
from __future__ import annotations

import numpy as np

from . import frontend, nemotron, sortformer, streaming
from .weights import make_weights


def pre_encode_all(w, mel, block: int = 64):
    """Sortformer pre_encode over the whole utterance, computed block by
    block of encoder frames (each block is an exact slice of the definition:
    per-layer padding sits at the utterance's absolute edges)."""
    T = mel.shape[0]
    Te = sortformer.subsampled_lengths(T)[2]
    out = [sortformer.pre_encode(w, mel, j0, min(Te, j0 + block), T=T)
           for j0 in range(0, Te, block)]
    return np.concatenate(out) if out else np.zeros((0, sortformer.D_FC))


# Longest clip (encoder frames) the offline forward takes as one window.
MAX_WINDOW = 1024


def sortformer_offline(audio, w):
    """Offline forward. A clip of at most MAX_WINDOW encoder frames is one
    window. Reading for longer clips (the pages' Sortformer offline forward has
    no stated limit, and the Nemotron-style variant processes long offline
    input in chunks with its cache and FIFO): the 'very high' streaming
    configuration on the known-length schedule."""
    mel = frontend.log_mel(audio)
    emb = pre_encode_all(w, mel)
    if emb.shape[0] <= MAX_WINDOW:
        return sortformer.encode_window(w, emb)
    p, _ = streaming.run_stream(emb, streaming.StreamConfig.preset("very_high"),
                                sortformer_encoder(w), 4)
    return p


def sortformer_encoder(w):
    def enc(window):
        p = sortformer.encode_window(w, window)
        return p, p
    return enc


def nemotron_encoder(w):
    return lambda window: nemotron.encode_window(w, window)


def sortformer_stream(audio, w, cfg: streaming.StreamConfig, steps=None, on_step=None,
                      live=True):
    """Streaming Sortformer over a clip delivered live (the end is known only
    at the final call); ``live=False`` uses the known-length schedule."""
    mel = frontend.log_mel(audio)
    emb = pre_encode_all(w, mel)
    sched = streaming.live_schedule(len(audio), cfg) if live else None
    return streaming.run_stream(emb, cfg, sortformer_encoder(w), 4, steps=steps,
                                on_step=on_step, sched=sched)


def nemotron_offline(audio, w, cfg: streaming.StreamConfig | None = None, steps=None,
                     on_step=None):
    """The Nemotron-style offline forward processes the clip in 30.4 s chunks
    with the arrival-order speaker cache and a 188-frame FIFO."""
    if cfg is None:
        cfg = streaming.StreamConfig.preset("nemotron_offline")
    mel = frontend.log_mel(audio)
    emb = nemotron.pre_encode(w, mel)
    return streaming.run_stream(emb, cfg, nemotron_encoder(w), 8, steps=steps,
                                on_step=on_step)


def weights_for(arch: str, dtype: str, seed: int | None = None, full_random=False):
    if seed is None:
        seed = 0 if arch == "sortformer" else 1
    return make_weights(arch, seed, full_random=full_random, bf16=(dtype == "bf16"))
