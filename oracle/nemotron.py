"""Nemotron-3-style variant, float64.

ExecuTorch issue "Enable Nemotron-3-Diarization ...", model-card summary:
~100M parameters, up to eight speakers ordered by first arrival, 128-bin mel
features stacked to an 80 ms encoder frame rate, a 31-layer Transformer with
RoPE, and a Conv1D upsampling head giving per-speaker probabilities at 10 ms.
Transformers docs "Nemotron 3 Diarization", fixed-window section: positions
restart at every chunk, so right padding does not change valid frames.

Readings: stacking concatenates mel frames 8t..8t+7 (feature 128r + m),
zero-padding the tail to a multiple of 8; input Linear 1024->512; pre-LN
layers x += Wo MHA(RoPE(q), RoPE(k), v)(LN1 x); x += W2 GELU(W1 LN2 x) with
exact (erf) GELU, FFN 2048, 8 heads of 64, scale 1/8; RoPE rotate-half with
base 10000 and positions 0..W-1 of the window; final LN; head Linear 512->8
(80 ms logits) then ConvTranspose1d(8, 8, kernel 8, stride 8) to 10 ms and
a sigmoid. The speaker cache is scored with sigmoid of the 80 ms logits.

Output resolution (Transformers docs "Nemotron 3 Diarization", Overview: one
checkpoint, output frame resolution configurable in 10 ms steps; the
model-card summary: 10 ms by default). Reading: a resolution of r x 10 ms
with r in {1, 2, 4, 8} (so an 80 ms encoder frame holds a whole number of
output frames) gives output frame k the mean of the head's 10 ms
probabilities r k .. r k + r - 1.
"""
from __future__ import annotations

import numpy as np
from scipy.special import erf

from .sortformer import layer_norm, linear, sigmoid, softmax_masked

D = 512
N_HEADS = 8
N_LAYERS = 31


def stack_frames(mel):
    """(T,128) -> (ceil(T/8), 1024), row t = [mel[8t], ..., mel[8t+7]]."""
    T = mel.shape[0]
    Te = (T + 7) // 8
    m = np.zeros((8 * Te, mel.shape[1]))
    m[:T] = mel
    return m.reshape(Te, 8 * mel.shape[1])


def pre_encode(w, mel):
    return linear(stack_frames(np.asarray(mel, dtype=np.float64)), w["in.w"], w["in.b"])


def rope(x, pos, base=10000.0):
    """Rotate-half rotary embedding of (H, W, 64) at positions pos (W,)."""
    half = x.shape[-1] // 2
    inv = base ** (-np.arange(half, dtype=np.float64) / half)
    ang = pos[:, None].astype(np.float64) * inv[None, :]
    c, s = np.cos(ang), np.sin(ang)
    x1, x2 = x[..., :half], x[..., half:]
    return np.concatenate([x1 * c - x2 * s, x2 * c + x1 * s], axis=-1)


def gelu(x):
    return 0.5 * x * (1.0 + erf(x / np.sqrt(2.0)))


def rope_context(w, l, x, n_valid):
    """Attention context (W, 512) of RoPE layer l before the output
    projection, given the residual stream x entering the layer."""
    p = f"rl{l}."
    W = x.shape[0]
    dk = D // N_HEADS
    h = layer_norm(x, w[p + "ln1.g"], w[p + "ln1.b"])
    q = linear(h, w[p + "wq"], w[p + "bq"]).reshape(W, N_HEADS, dk).transpose(1, 0, 2)
    k = linear(h, w[p + "wk"], w[p + "bk"]).reshape(W, N_HEADS, dk).transpose(1, 0, 2)
    v = linear(h, w[p + "wv"], w[p + "bv"]).reshape(W, N_HEADS, dk).transpose(1, 0, 2)
    pos = np.arange(W)
    q, k = rope(q, pos), rope(k, pos)
    a = softmax_masked(q @ k.transpose(0, 2, 1) / np.sqrt(dk), n_valid)
    return (a @ v).transpose(1, 0, 2).reshape(W, D)


def rope_layer(w, l, x, n_valid):
    p = f"rl{l}."
    x = x + linear(rope_context(w, l, x, n_valid), w[p + "wo"], w[p + "bo"])
    h = layer_norm(x, w[p + "ln2.g"], w[p + "ln2.b"])
    return x + linear(gelu(linear(h, w[p + "w1"], w[p + "b1"])), w[p + "w2"], w[p + "b2"])


def upsample_head(w, logits80):
    """ConvTranspose1d(S, S, k=8, s=8): out[8t+r, o] = b[o] + sum_i z[t,i] W[i,o,r]."""
    W, S = logits80.shape
    up = np.einsum("ti,ior->tro", logits80, w["up.w"]) + w["up.b"]
    return up.reshape(8 * W, S)


OUTPUT_STRIDES = (1, 2, 4, 8)


def pool_output(probs10, r):
    """(8W, S) probabilities at 10 ms -> (8W / r, S) at r x 10 ms: the mean of
    each run of r consecutive frames."""
    if r not in OUTPUT_STRIDES:
        raise ValueError(f"output stride {r} not in {OUTPUT_STRIDES}")
    n, S = probs10.shape
    assert n % r == 0
    return probs10.reshape(n // r, r, S).mean(axis=1)


def encode_window(w, emb, n_valid=None, n_layers=N_LAYERS):
    """(W,512) window embeddings -> (probs80 (W,S), probs10 (8W,S))."""
    x = np.asarray(emb, dtype=np.float64)
    if n_valid is None:
        n_valid = x.shape[0]
    for l in range(n_layers):
        x = rope_layer(w, l, x, n_valid)
    x = layer_norm(x, w["final_ln.g"], w["final_ln.b"])
    z = linear(x, w["head.w"], w["head.b"])
    return sigmoid(z), sigmoid(upsample_head(w, z))
