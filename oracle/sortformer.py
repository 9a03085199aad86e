"""Sortformer frame-classification forward, float64, one GEMM per Linear.

"Streaming Sortformer Diarizer" model card:
* Pipeline: mel (T,128) -> ConvSubsampling 8x (pre_encode) -> 17 conformer
  layers (rel-pos self-attention + conv + FFN, d_model 512) -> encoder_proj
  Linear 512->192 -> 18-layer Transformer encoder (hidden 192, 8 heads) ->
  head Linear 192->192, ReLU, Linear 192->4, Sigmoid. One output frame per
  80 ms.
* Exported Methods: pre_encode maps (4000,128) mel frames to (500,512);
  output length 1+((L-1)//8).
* torch.export Fixes 4: the subsampling output (b,c,t,f) is permuted to
  (b,t,c,f) and flattened, so feature index = c*16 + f.
* torch.export Fixes 6: rel_shift turns the query-by-position score matrix
  into the score of relative distance i-j; here it is written out directly as
  (q_i + v) . p(i-j) for every pair.

Readings (pages silent): dw-striding subsampling (conv0 1->256 3x3 stride 2
pad 1, ReLU, then twice [depthwise 3x3 stride 2 pad 1, pointwise 256->256,
ReLU]), which gives the card's 117M parameters; macaron conformer layer
x += FF/2; x += MHSA; x += Conv; x += FF/2; x = LN(x) with Swish FFNs,
LN eps 1e-5, no input scaling, eval mode; interleaved sinusoidal relative
positions pe[2k] = sin(d w_k), pe[2k+1] = cos(d w_k), w_k = 10000^(-2k/512),
bias-free positional projection, per-layer u/v biases; conv module
pw 512->1024, GLU (first half * sigmoid(second half)), depthwise k=9 pad 4,
BatchNorm (eval statistics, eps 1e-5), Swish, pw 512->512; post-LN
transformer layers x = LN(x + MHA(x)); x = LN(x + W2 relu(W1 x)); no ReLU
before the head's first Linear (the card's head order is authoritative).
"""
from __future__ import annotations

import numpy as np

D_FC = 512
D_TF = 192
N_HEADS = 8
LN_EPS = 1e-5
BN_EPS = 1e-5


# ----------------------------------------------------------------- helpers
def layer_norm(x, g, b, eps=LN_EPS):
    mu = x.mean(axis=-1, keepdims=True)
    var = ((x - mu) ** 2).mean(axis=-1, keepdims=True)
    return (x - mu) / np.sqrt(var + eps) * g + b


def sigmoid(x):
    return 1.0 / (1.0 + np.exp(-x))


def swish(x):
    return x * sigmoid(x)


def softmax_masked(s, n_valid_keys):
    """Softmax over the last axis; keys at index >= n_valid_keys are padding."""
    s = s.copy()
    if n_valid_keys < s.shape[-1]:
        s[..., n_valid_keys:] = -np.inf
    m = s.max(axis=-1, keepdims=True)
    e = np.exp(s - m)
    return e / e.sum(axis=-1, keepdims=True)


def linear(x, w, b=None):
    y = x @ w.T
    return y if b is None else y + b


# --------------------------------------------------------- pre_encode (a2)
def subsampled_lengths(T: int):
    """Lengths after each stride-2 (kernel 3, pad 1) layer: ceil(L/2) each."""
    l1 = (T + 1) // 2
    l2 = (l1 + 1) // 2
    l3 = (l2 + 1) // 2
    return l1, l2, l3


def _patches(x, start, len_in, out_lo, out_hi, f_in):
    """Gather the 3x3 stride-2 neighbourhoods of output rows [out_lo,out_hi).

    x: (C, n, f_in) holding absolute rows start..start+n-1 of a layer of
    total length len_in. Rows outside [0, len_in) and columns outside
    [0, f_in) are the convolution's zero padding. Returns (C, rows, f_out, 3, 3).
    """
    C = x.shape[0]
    f_out = (f_in + 1) // 2
    o = np.arange(out_lo, out_hi)
    rows = 2 * o[:, None] + np.arange(-1, 2)[None, :]            # (R,3)
    cols = 2 * np.arange(f_out)[:, None] + np.arange(-1, 2)[None, :]  # (F,3)
    rvalid = (rows >= 0) & (rows < len_in)
    cvalid = (cols >= 0) & (cols < f_in)
    ri = rows - start
    if rvalid.any():
        assert ri[rvalid].min() >= 0 and ri[rvalid].max() < x.shape[1], "missing input rows"
    ri = np.clip(ri, 0, max(x.shape[1] - 1, 0))
    ci = np.clip(cols, 0, f_in - 1)
    p = x[:, ri[:, None, :, None], ci[None, :, None, :]]         # (C,R,F,3,3)
    mask = rvalid[:, None, :, None] & cvalid[None, :, None, :]
    return p * mask[None]


def pre_encode(w, mel, j0=0, j1=None, T=None, mel_start=0):
    """Encoder frames [j0, j1) of the 8x ConvSubsampling.

    mel: (n, 128) holding absolute mel frames mel_start..mel_start+n-1 of an
    utterance of T frames (T defaults to mel_start+n). Each layer's padding
    is applied at the absolute edges of that layer, so any range of outputs
    equals the same rows of the whole-utterance result.
    """
    if T is None:
        T = mel_start + mel.shape[0]
    l1, l2, l3 = subsampled_lengths(T)
    if j1 is None:
        j1 = l3
    assert 0 <= j0 <= j1 <= l3
    if j1 == j0:
        return np.zeros((0, D_FC))
    a1 = (max(0, 4 * j0 - 3), min(l1, 4 * j1))
    a2 = (max(0, 2 * j0 - 1), min(l2, 2 * j1))
    x0 = np.asarray(mel, dtype=np.float64)[None]                   # (1,n,128)
    p = _patches(x0, mel_start, T, a1[0], a1[1], 128)              # (1,R,64,3,3)
    k0 = w["pre.conv0.w"][:, 0]                                    # (256,3,3)
    y1 = np.einsum("rfab,cab->crf", p[0], k0) + w["pre.conv0.b"][:, None, None]
    y1 = np.maximum(y1, 0.0)
    y2 = _dw_pw(w, 1, y1, a1[0], l1, a2[0], a2[1])
    y3 = _dw_pw(w, 2, y2, a2[0], l2, j0, j1)                       # (256,R,16)
    flat = y3.transpose(1, 0, 2).reshape(j1 - j0, 256 * 16)        # feature c*16+f
    return linear(flat, w["pre.out.w"], w["pre.out.b"])


def _dw_pw(w, k, x, start, len_in, lo, hi):
    p = _patches(x, start, len_in, lo, hi, x.shape[2])              # (C,R,F,3,3)
    dw = w[f"pre.dw{k}.w"][:, 0]                                   # (256,3,3)
    y = np.einsum("crfab,cab->crf", p, dw) + w[f"pre.dw{k}.b"][:, None, None]
    pw = w[f"pre.pw{k}.w"][:, :, 0, 0]                             # (256,256)
    y = np.einsum("dc,crf->drf", pw, y) + w[f"pre.pw{k}.b"][:, None, None]
    return np.maximum(y, 0.0)


# ------------------------------------------------------ conformer (a4)
def rel_pos_table(W: int, d: int = D_FC):
    """Sinusoid rows for relative distances delta = -(W-1) .. W-1 (row
    delta + W - 1), interleaved sin/cos."""
    delta = np.arange(-(W - 1), W, dtype=np.float64)
    k = np.arange(d // 2, dtype=np.float64)
    omega = 10000.0 ** (-2.0 * k / d)
    ang = delta[:, None] * omega[None, :]
    pe = np.zeros((2 * W - 1, d))
    pe[:, 0::2] = np.sin(ang)
    pe[:, 1::2] = np.cos(ang)
    return pe


def rel_pos_context(w, p, h, n_valid):
    """Relative-position multi-head attention context with u/v biases, all
    heads concatenated (W, 512), before the output projection.

    score(i,j) = [(q_i+u).k_j + (q_i+v).p(i-j)] / sqrt(64), softmax over the
    n_valid real keys, times V.
    """
    W = h.shape[0]
    H, dk = N_HEADS, D_FC // N_HEADS
    q = linear(h, w[p + "att.wq"], w[p + "att.bq"]).reshape(W, H, dk).transpose(1, 0, 2)
    k = linear(h, w[p + "att.wk"], w[p + "att.bk"]).reshape(W, H, dk).transpose(1, 0, 2)
    v = linear(h, w[p + "att.wv"], w[p + "att.bv"]).reshape(W, H, dk).transpose(1, 0, 2)
    pos = linear(rel_pos_table(W), w[p + "att.wpos"])                # (2W-1, 512)
    pos = pos.reshape(2 * W - 1, H, dk).transpose(1, 0, 2)          # (H,2W-1,dk)
    qu = q + w[p + "att.u"][:, None, :]
    qv = q + w[p + "att.v"][:, None, :]
    ac = qu @ k.transpose(0, 2, 1)                                  # (H,W,W)
    g = qv @ pos.transpose(0, 2, 1)                                 # (H,W,2W-1)
    i = np.arange(W)[:, None]
    j = np.arange(W)[None, :]
    bd = g[:, i, i - j + W - 1]                                     # (q_i+v).p(i-j)
    a = softmax_masked((ac + bd) / np.sqrt(dk), n_valid)
    return (a @ v).transpose(1, 0, 2).reshape(W, D_FC)


def rel_pos_mhsa(w, p, h, n_valid):
    """Relative-position self-attention: the context above, output projection."""
    return linear(rel_pos_context(w, p, h, n_valid), w[p + "att.wo"], w[p + "att.bo"])


def conv_module(w, p, h, n_valid):
    a = linear(h, w[p + "conv.pw1.w"], w[p + "conv.pw1.b"])
    g = a[:, :D_FC] * sigmoid(a[:, D_FC:])
    g[n_valid:] = 0.0                                                # padded frames
    W = g.shape[0]
    gp = np.concatenate([np.zeros((4, D_FC)), g, np.zeros((4, D_FC))])
    dw = w[p + "conv.dw.w"]                                         # (512, 9)
    d = np.zeros_like(g) + w[p + "conv.dw.b"]
    for t in range(9):
        d += gp[t:t + W] * dw[:, t]
    bn = (d - w[p + "conv.bn.mean"]) / np.sqrt(w[p + "conv.bn.var"] + BN_EPS) \
        * w[p + "conv.bn.g"] + w[p + "conv.bn.b"]
    return linear(swish(bn), w[p + "conv.pw2.w"], w[p + "conv.pw2.b"])


def feed_forward(w, p, h):
    return linear(swish(linear(h, w[p + "w1"], w[p + "b1"])), w[p + "w2"], w[p + "b2"])


def conformer_layer(w, l, x, n_valid):
    p = f"conf{l}."
    x = x + 0.5 * feed_forward(w, p + "ff1.", layer_norm(x, w[p + "ff1.ln.g"], w[p + "ff1.ln.b"]))
    x = x + rel_pos_mhsa(w, p, layer_norm(x, w[p + "att.ln.g"], w[p + "att.ln.b"]), n_valid)
    x = x + conv_module(w, p, layer_norm(x, w[p + "conv.ln.g"], w[p + "conv.ln.b"]), n_valid)
    x = x + 0.5 * feed_forward(w, p + "ff2.", layer_norm(x, w[p + "ff2.ln.g"], w[p + "ff2.ln.b"]))
    return layer_norm(x, w[p + "out_ln.g"], w[p + "out_ln.b"])


def conformer_attention_context(w, l, x, n_valid):
    """Attention context (before W_o) of conformer layer l, given the residual
    stream x entering the layer: the first half-step FFN, LN, then
    rel_pos_context."""
    p = f"conf{l}."
    x = x + 0.5 * feed_forward(w, p + "ff1.", layer_norm(x, w[p + "ff1.ln.g"], w[p + "ff1.ln.b"]))
    return rel_pos_context(w, p, layer_norm(x, w[p + "att.ln.g"], w[p + "att.ln.b"]), n_valid)


# ---------------------------------------------------- transformer (a6)
def mha_context(w, p, x, n_valid, n_heads=N_HEADS):
    """Softmax attention context of all heads (W, d), before the output
    projection."""
    W, d = x.shape
    dk = d // n_heads
    q = linear(x, w[p + "wq"], w[p + "bq"]).reshape(W, n_heads, dk).transpose(1, 0, 2)
    k = linear(x, w[p + "wk"], w[p + "bk"]).reshape(W, n_heads, dk).transpose(1, 0, 2)
    v = linear(x, w[p + "wv"], w[p + "bv"]).reshape(W, n_heads, dk).transpose(1, 0, 2)
    a = softmax_masked(q @ k.transpose(0, 2, 1) / np.sqrt(dk), n_valid)
    return (a @ v).transpose(1, 0, 2).reshape(W, d)


def mha(w, p, x, n_valid, n_heads=N_HEADS):
    return linear(mha_context(w, p, x, n_valid, n_heads), w[p + "wo"], w[p + "bo"])


def transformer_layer(w, l, x, n_valid):
    p = f"tf{l}."
    x = layer_norm(x + mha(w, p, x, n_valid), w[p + "ln1.g"], w[p + "ln1.b"])
    f = linear(np.maximum(linear(x, w[p + "w1"], w[p + "b1"]), 0.0), w[p + "w2"], w[p + "b2"])
    return layer_norm(x + f, w[p + "ln2.g"], w[p + "ln2.b"])


# ----------------------------------------------------------- head (a7)
def speaker_head(w, x):
    h = np.maximum(linear(x, w["head.w1"], w["head.b1"]), 0.0)
    return sigmoid(linear(h, w["head.w2"], w["head.b2"]))


# ------------------------------------------------------------- forward
def encode_window(w, emb, n_valid=None, n_conformer=17, n_transformer=18):
    """[speaker_cache | FIFO | chunk | look-ahead] embeddings (W,512) ->
    probabilities (W, n_spk). Rows >= n_valid are right padding: masked as
    keys and zeroed before the depthwise convolution, so valid rows do not
    depend on them."""
    x = np.asarray(emb, dtype=np.float64)
    if n_valid is None:
        n_valid = x.shape[0]
    for l in range(n_conformer):
        x = conformer_layer(w, l, x, n_valid)
    x = linear(x, w["proj.w"], w["proj.b"])
    for l in range(n_transformer):
        x = transformer_layer(w, l, x, n_valid)
    return speaker_head(w, x)


def forward_offline(w, audio):
    """Offline forward: audio (N,) -> probabilities (ceil(floor(N/160)/8), 4)."""
    from .frontend import log_mel
    mel = log_mel(audio)
    emb = pre_encode(w, mel)
    return encode_window(w, emb)
