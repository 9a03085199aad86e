"""Pins of the oracle's layer compositions against independent torch chains.

"Streaming Sortformer Diarizer" model card, Pipeline and Streaming
Architecture: a conformer layer is the macaron pair of half-step feed-forward
modules around the relative-position self-attention and the convolution
module, closed by a LayerNorm; the encoder projects 512 -> 192 into the
Transformer; the head is Linear, ReLU, Linear, Sigmoid; a streaming step
emits the rows of its chunk only. Each reference below is written with
``torch.nn.functional`` (grouped conv1d, batch_norm, glu, silu, layer_norm)
and, for the relative-position scores, the pad -> view -> slice shift
(torch.export Fixes 6), not with the oracle's own helpers. Every pin is
checked twice: the oracle passes it, and a copy of the oracle with a planted
mistake (a dropped 1/2, a swapped module order, a missing output LayerNorm, a
misplaced ReLU, an emission slice off by one row) fails it by orders of
magnitude more than the tolerance.
"""
import numpy as np
import pytest
import torch
import torch.nn.functional as TF

from oracle import sortformer as SF
from oracle import streaming as S

TOL = 1e-10


def _t(x):
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float64))


# ---------------------------------------------------------------- torch chains
def _ln(x, w, key):
    return TF.layer_norm(x, (x.shape[-1],), _t(w[key + ".g"]), _t(w[key + ".b"]), eps=1e-5)


def _ffn(w, p, h):
    return TF.linear(TF.silu(TF.linear(h, _t(w[p + "w1"]), _t(w[p + "b1"]))),
                     _t(w[p + "w2"]), _t(w[p + "b2"]))


def _sinusoids_desc(W, d=512):
    """Positions W-1, W-2, ..., -(W-1), interleaved sin / cos of d * 10000^(-2k/d)."""
    dist = torch.arange(W - 1, -W, -1, dtype=torch.float64)
    om = torch.pow(torch.tensor(10000.0, dtype=torch.float64),
                   -2.0 * torch.arange(d // 2, dtype=torch.float64) / d)
    ang = dist[:, None] * om[None, :]
    return torch.stack([torch.sin(ang), torch.cos(ang)], dim=-1).reshape(2 * W - 1, d)


def _rel_shift(x):
    """(H, W, 2W-1) scores against descending positions -> column j holds the
    score of distance i - j (pad one column, view, drop a row, view, slice)."""
    H, W, P = x.shape
    x = TF.pad(x, (1, 0))
    x = x.view(H, P + 1, W)[:, 1:].reshape(H, W, P)
    return x[:, :, :W]


def _relpos_attention(w, p, h, n_valid):
    W = h.shape[0]
    q = TF.linear(h, _t(w[p + "att.wq"]), _t(w[p + "att.bq"])).view(W, 8, 64).transpose(0, 1)
    k = TF.linear(h, _t(w[p + "att.wk"]), _t(w[p + "att.bk"])).view(W, 8, 64).transpose(0, 1)
    v = TF.linear(h, _t(w[p + "att.wv"]), _t(w[p + "att.bv"])).view(W, 8, 64).transpose(0, 1)
    pos = TF.linear(_sinusoids_desc(W), _t(w[p + "att.wpos"])).view(2 * W - 1, 8, 64).transpose(0, 1)
    u, vb = _t(w[p + "att.u"])[:, None, :], _t(w[p + "att.v"])[:, None, :]
    ac = torch.matmul(q + u, k.transpose(1, 2))
    bd = _rel_shift(torch.matmul(q + vb, pos.transpose(1, 2)))
    s = (ac + bd) / 8.0
    mask = torch.arange(W) >= n_valid
    s = s.masked_fill(mask[None, None, :], float("-inf"))
    ctx = torch.matmul(torch.softmax(s, dim=-1), v).transpose(0, 1).reshape(W, 512)
    return TF.linear(ctx, _t(w[p + "att.wo"]), _t(w[p + "att.bo"]))


def _conv_module(w, p, h, n_valid):
    W = h.shape[0]
    g = TF.glu(TF.linear(h, _t(w[p + "conv.pw1.w"]), _t(w[p + "conv.pw1.b"])), dim=-1)
    g = g.masked_fill((torch.arange(W) >= n_valid)[:, None], 0.0)
    d = TF.conv1d(g.T[None], _t(w[p + "conv.dw.w"]).view(512, 1, 9), _t(w[p + "conv.dw.b"]),
                  padding=4, groups=512)
    bn = TF.batch_norm(d, _t(w[p + "conv.bn.mean"]), _t(w[p + "conv.bn.var"]),
                       _t(w[p + "conv.bn.g"]), _t(w[p + "conv.bn.b"]), training=False, eps=1e-5)
    return TF.linear(TF.silu(bn)[0].T, _t(w[p + "conv.pw2.w"]), _t(w[p + "conv.pw2.b"]))


def _conformer(w, l, x, n_valid):
    p = f"conf{l}."
    x = x + 0.5 * _ffn(w, p + "ff1.", _ln(x, w, p + "ff1.ln"))
    x = x + _relpos_attention(w, p, _ln(x, w, p + "att.ln"), n_valid)
    x = x + _conv_module(w, p, _ln(x, w, p + "conv.ln"), n_valid)
    x = x + 0.5 * _ffn(w, p + "ff2.", _ln(x, w, p + "ff2.ln"))
    return _ln(x, w, p + "out_ln")


def _transformer(w, l, x, n_valid):
    p = f"tf{l}."
    W = x.shape[0]
    q = TF.linear(x, _t(w[p + "wq"]), _t(w[p + "bq"])).view(W, 8, 24).transpose(0, 1)
    k = TF.linear(x, _t(w[p + "wk"]), _t(w[p + "bk"])).view(W, 8, 24).transpose(0, 1)
    v = TF.linear(x, _t(w[p + "wv"]), _t(w[p + "bv"])).view(W, 8, 24).transpose(0, 1)
    keep = (torch.arange(W) < n_valid)[None, :].expand(W, W)
    ctx = TF.scaled_dot_product_attention(q, k, v, attn_mask=keep).transpose(0, 1).reshape(W, 192)
    x = _ln(x + TF.linear(ctx, _t(w[p + "wo"]), _t(w[p + "bo"])), w, p + "ln1")
    f = TF.linear(TF.relu(TF.linear(x, _t(w[p + "w1"]), _t(w[p + "b1"]))), _t(w[p + "w2"]),
                  _t(w[p + "b2"]))
    return _ln(x + f, w, p + "ln2")


def _head(w, x):
    h = TF.relu(TF.linear(x, _t(w["head.w1"]), _t(w["head.b1"])))
    return torch.sigmoid(TF.linear(h, _t(w["head.w2"]), _t(w["head.b2"])))


# ------------------------------------------------------------------ helpers
def _err(a, b):
    return float(np.abs(np.asarray(a) - np.asarray(b)).max())


@pytest.fixture(scope="module")
def rows():
    rng = np.random.default_rng(20)
    return rng.normal(size=(11, 512))


def _planted(monkeypatch, kind, w):
    """Plant one mistake into the oracle module (restored after the test)."""
    if kind == "dropped_half":           # x + FF instead of x + FF/2
        ff = SF.feed_forward
        monkeypatch.setattr(SF, "feed_forward", lambda w_, p, h: 2.0 * ff(w_, p, h))
    elif kind == "conv_before_attention":
        att, conv = SF.rel_pos_mhsa, SF.conv_module
        monkeypatch.setattr(SF, "rel_pos_mhsa", conv)
        monkeypatch.setattr(SF, "conv_module", att)
    elif kind == "no_output_ln":
        ln = SF.layer_norm
        targets = [id(w[f"conf{l}.out_ln.g"]) for l in range(17)]
        monkeypatch.setattr(SF, "layer_norm",
                            lambda x, g, b, eps=SF.LN_EPS: x if id(g) in targets else ln(x, g, b, eps))
    elif kind == "relu_before_head":
        lin = SF.linear
        monkeypatch.setattr(SF, "speaker_head", lambda w_, x: SF.sigmoid(
            lin(lin(np.maximum(x, 0.0), w_["head.w1"], w_["head.b1"]), w_["head.w2"], w_["head.b2"])))
    elif kind == "no_head_relu":
        lin = SF.linear
        monkeypatch.setattr(SF, "speaker_head", lambda w_, x: SF.sigmoid(
            lin(lin(x, w_["head.w1"], w_["head.b1"]), w_["head.w2"], w_["head.b2"])))
    elif kind == "swish_ffn_as_relu":
        lin = SF.linear
        monkeypatch.setattr(SF, "feed_forward", lambda w_, p, h: lin(
            np.maximum(lin(h, w_[p + "w1"], w_[p + "b1"]), 0.0), w_[p + "w2"], w_[p + "b2"]))
    else:
        raise ValueError(kind)


# -------------------------------------------------------------------- pins
def test_feed_forward_vs_torch(sf_weights_full, rows, monkeypatch):
    w = sf_weights_full
    for p in ("conf0.ff1.", "conf5.ff2."):
        ref = _ffn(w, p, _t(rows)).numpy()
        assert _err(SF.feed_forward(w, p, rows), ref) < TOL
    _planted(monkeypatch, "swish_ffn_as_relu", w)
    assert _err(SF.feed_forward(w, "conf0.ff1.", rows), _ffn(w, "conf0.ff1.", _t(rows)).numpy()) > 1e-3


@pytest.mark.parametrize("n_valid", [11, 8])
def test_conformer_layer_vs_torch(sf_weights_full, rows, n_valid):
    w = sf_weights_full
    for l in (0, 9):
        got = SF.conformer_layer(w, l, rows, n_valid)
        ref = _conformer(w, l, _t(rows), n_valid).numpy()
        assert _err(got[:n_valid], ref[:n_valid]) < TOL


@pytest.mark.parametrize("kind", ["dropped_half", "conv_before_attention", "no_output_ln",
                                  "swish_ffn_as_relu"])
def test_conformer_pin_catches_planted_mistakes(sf_weights_full, rows, monkeypatch, kind):
    w = sf_weights_full
    ref = _conformer(w, 3, _t(rows), 11).numpy()
    assert _err(SF.conformer_layer(w, 3, rows, 11), ref) < TOL
    _planted(monkeypatch, kind, w)
    assert _err(SF.conformer_layer(w, 3, rows, 11), ref) > 1e-3


def test_speaker_head_vs_torch(sf_weights_full, monkeypatch):
    w = sf_weights_full
    x = np.random.default_rng(21).normal(size=(13, 192))
    ref = _head(w, _t(x)).numpy()
    got = SF.speaker_head(w, x)
    assert got.shape == (13, 4) and _err(got, ref) < 1e-13
    for kind in ("relu_before_head", "no_head_relu"):
        with monkeypatch.context() as mp:
            _planted(mp, kind, w)
            assert _err(SF.speaker_head(w, x), ref) > 1e-4


@pytest.mark.parametrize("n_valid", [10, 7])
def test_encode_window_chain_vs_torch(sf_weights_full, monkeypatch, n_valid):
    """One conformer layer, encoder_proj, one transformer layer and the head."""
    w = sf_weights_full
    emb = np.random.default_rng(22).normal(size=(10, 512))
    x = _conformer(w, 0, _t(emb), n_valid)
    x = TF.linear(x, _t(w["proj.w"]), _t(w["proj.b"]))
    ref = _head(w, _transformer(w, 0, x, n_valid)).numpy()
    got = SF.encode_window(w, emb, n_valid=n_valid, n_conformer=1, n_transformer=1)
    assert got.shape == (10, 4) and _err(got[:n_valid], ref[:n_valid]) < TOL
    for kind in ("no_output_ln", "relu_before_head", "dropped_half"):
        with monkeypatch.context() as mp:
            _planted(mp, kind, w)
            bad = SF.encode_window(w, emb, n_valid=n_valid, n_conformer=1, n_transformer=1)
            assert _err(bad[:n_valid], ref[:n_valid]) > 1e-5


# ------------------------------------------------------- emitted rows of a step
def _tagged_encoder(rate):
    """Fake encoder: window row r carries its tag in column 0; the 80 ms
    probabilities of that row are (tag mod 1000) / 1000 per speaker s shifted
    by s / 10^4, and the emitted-rate rows 8r + q add q / 10^6."""
    def enc(window):
        tag = window[:, 0]
        base = (tag % 1000.0) / 1000.0
        p80 = base[:, None] + np.arange(4)[None, :] * 1e-4
        if rate == 1:
            return p80, p80
        pout = np.repeat(p80, rate, axis=0) + np.tile(np.arange(rate), len(tag))[:, None] * 1e-6
        return p80, pout
    return enc


def _expected_rows(tags, rate):
    base = (np.asarray(tags) % 1000.0) / 1000.0
    p = base[:, None] + np.arange(4)[None, :] * 1e-4
    if rate == 1:
        return p
    return np.repeat(p, rate, axis=0) + np.tile(np.arange(rate), len(tags))[:, None] * 1e-6


def _tagged_state(Lc, Lf, d=8, seed=0):
    rng = np.random.default_rng(seed)
    ce = rng.normal(size=(Lc, d))
    ce[:, 0] = 100 + np.arange(Lc)
    fe = rng.normal(size=(Lf, d))
    fe[:, 0] = 400 + np.arange(Lf)
    return S.State(ce, rng.random((Lc, 4)), np.zeros(Lc, bool), fe, rng.random((Lf, 4)),
                   np.zeros(d), 0)


def _step_shifted(state, emb_new, n_chunk, cfg, encode, n_spk):
    """stream_step with its emission window moved one row late (a planted mistake)."""
    window = np.concatenate([state.cache_emb, state.fifo_emb, emb_new])
    p80, pout = encode(window)
    Lc, Lf = state.cache_emb.shape[0], state.fifo_emb.shape[0]
    rate = pout.shape[0] // p80.shape[0]
    out = pout[rate * (Lc + Lf + 1):rate * (Lc + Lf + 1 + n_chunk)]
    S.fifo_update(state, p80, emb_new, n_chunk, cfg, n_spk)
    return out


@pytest.mark.parametrize("rate", [1, 8])
@pytest.mark.parametrize("Lc,Lf,n,rc", [(188, 100, 3, 1), (150, 188, 6, 7), (0, 0, 6, 7),
                                        (188, 188, 4, 0)])
def test_stream_step_emits_chunk_rows(rate, Lc, Lf, n, rc):
    cfg = S.StreamConfig(chunk_len=n, right_context=rc, fifo_len=188, update_period=144)
    d = 8
    new = np.random.default_rng(1).normal(size=(n + rc, d))
    new[:, 0] = 800 + np.arange(n + rc)
    enc = _tagged_encoder(rate)
    want = _expected_rows(new[:n, 0], rate)
    st = _tagged_state(Lc, Lf, d)
    out = S.stream_step(st, new, n, cfg, enc, 4)
    assert out.shape == (rate * n, 4) and np.array_equal(out, want)
    # the FIFO (or, after a pop, the cache and FIFO together) now ends with the chunk rows
    seq = np.concatenate([st.cache_emb[:, 0], st.fifo_emb[:, 0]])
    assert np.array_equal(seq[-n:], new[:n, 0])
    bad = _step_shifted(_tagged_state(Lc, Lf, d), new, n, cfg, enc, 4)
    assert bad.shape != want.shape or not np.array_equal(bad, want)
