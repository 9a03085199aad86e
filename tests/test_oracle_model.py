"""Pins of the oracle's subsampling, conformer, transformer, head and the
Nemotron-style layers: library routines (torch CPU float64), brute force,
page-given shapes and invariants."""
import json
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as TF

from oracle import nemotron as NM
from oracle import sortformer as SF
from oracle import run, streaming

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "page_facts.json")))


def _t(x):
    return torch.from_numpy(np.ascontiguousarray(x))


def test_subsampling_lengths_rule():
    for T in range(1, 65):
        assert SF.subsampled_lengths(T)[2] == 1 + (T - 1) // 8   # page formula


def test_pre_encode_page_shape(sf_weights_full):
    fin, fout = GOLD["pre_encode_io"]["in"], GOLD["pre_encode_io"]["out"]
    mel = np.random.default_rng(1).normal(size=fin)
    out = run.pre_encode_all(sf_weights_full, mel, block=100)
    assert list(out.shape) == fout


def test_pre_encode_matches_torch_convs(sf_weights_full):
    w = sf_weights_full
    rng = np.random.default_rng(2)
    for T in (1, 7, 8, 9, 23, 40):
        mel = rng.normal(size=(T, 128))
        got = SF.pre_encode(w, mel)
        x = _t(mel)[None, None]
        x = TF.relu(TF.conv2d(x, _t(w["pre.conv0.w"]), _t(w["pre.conv0.b"]), stride=2, padding=1))
        for k in (1, 2):
            x = TF.conv2d(x, _t(w[f"pre.dw{k}.w"]), _t(w[f"pre.dw{k}.b"]), stride=2, padding=1,
                          groups=256)
            x = TF.relu(TF.conv2d(x, _t(w[f"pre.pw{k}.w"]), _t(w[f"pre.pw{k}.b"])))
        x = x.permute(0, 2, 1, 3).flatten(2)                     # (b,t,c*f)
        ref = TF.linear(x, _t(w["pre.out.w"]), _t(w["pre.out.b"]))[0].numpy()
        assert got.shape == ref.shape == (1 + (T - 1) // 8, 512)
        assert np.abs(got - ref).max() < 1e-10


def test_pre_encode_ranges_and_receptive_field(sf_weights_full):
    w = sf_weights_full
    rng = np.random.default_rng(3)
    T = 75
    mel = rng.normal(size=(T, 128))
    full = SF.pre_encode(w, mel)
    for j0, j1 in ((0, 3), (2, 5), (4, 10), (9, 10)):
        lo = max(0, 8 * j0 - 8)
        part = SF.pre_encode(w, mel[lo:8 * j1 if j1 < 10 else T], j0, j1, T=T, mel_start=lo)
        assert np.abs(part - full[j0:j1]).max() < 1e-13   # same values, BLAS order aside
    j = 4
    mel2 = mel.copy()
    mel2[8 * j + 8:] += 1.0
    assert np.array_equal(SF.pre_encode(w, mel2)[:j + 1], full[:j + 1])
    mel3 = mel.copy()
    mel3[8 * j + 7] += 1.0
    assert not np.array_equal(SF.pre_encode(w, mel3)[j], full[j])


def _attn_textbook(q, k, v, scale):
    """Brute-force softmax attention with Python loops (tiny sizes)."""
    H, W, d = q.shape
    out = np.zeros_like(q)
    for h in range(H):
        for i in range(W):
            s = [sum(q[h, i, c] * k[h, j, c] for c in range(d)) * scale for j in range(W)]
            m = max(s)
            e = [np.exp(x - m) for x in s]
            z = sum(e)
            for j in range(W):
                out[h, i] += e[j] / z * v[h, j]
    return out


def test_rel_pos_mhsa_reduces_to_softmax_attention(sf_weights_full):
    w = dict(sf_weights_full)
    p = "conf0."
    w[p + "att.wpos"] = np.zeros_like(w[p + "att.wpos"])
    w[p + "att.u"] = np.zeros_like(w[p + "att.u"])
    w[p + "att.v"] = np.zeros_like(w[p + "att.v"])
    rng = np.random.default_rng(4)
    W = 5
    h = rng.normal(size=(W, 512))
    got = SF.rel_pos_mhsa(w, p, h, W)
    q = SF.linear(h, w[p + "att.wq"], w[p + "att.bq"]).reshape(W, 8, 64).transpose(1, 0, 2)
    k = SF.linear(h, w[p + "att.wk"], w[p + "att.bk"]).reshape(W, 8, 64).transpose(1, 0, 2)
    v = SF.linear(h, w[p + "att.wv"], w[p + "att.bv"]).reshape(W, 8, 64).transpose(1, 0, 2)
    ctx = TF.scaled_dot_product_attention(_t(q), _t(k), _t(v)).numpy()
    ctx_bf = _attn_textbook(q, k, v, 1 / 8)
    assert np.abs(ctx - ctx_bf).max() < 1e-12
    ref = SF.linear(ctx.transpose(1, 0, 2).reshape(W, 512), w[p + "att.wo"], w[p + "att.bo"])
    assert np.abs(got - ref).max() < 1e-12


def test_rel_shift_pad_view_slice_equivalence():
    """The oracle's direct (q_i+v).p(i-j) equals the pad -> view -> slice ->
    view shift applied to scores against positions ordered W-1 ... -(W-1)."""
    rng = np.random.default_rng(5)
    W, d = 7, 16
    qv = rng.normal(size=(W, d))
    pe = rng.normal(size=(2 * W - 1, d))        # row r = relative distance r-(W-1)
    g = qv @ pe.T
    i = np.arange(W)[:, None]
    j = np.arange(W)[None, :]
    direct = g[i, i - j + W - 1]
    # second implementation: descending positions + the shift trick
    desc = qv @ pe[::-1].T                      # column c = distance W-1-c
    x = np.concatenate([np.zeros((W, 1)), desc], axis=1)   # pad one column left
    x = x.reshape(2 * W, W)[1:].reshape(W, 2 * W - 1)       # view, drop row, view
    shifted = x[:, :W]
    assert np.allclose(shifted, direct, atol=1e-13)


def test_rel_pos_table_values():
    pe = SF.rel_pos_table(4)
    assert pe.shape == (7, 512)
    assert np.allclose(pe[3, 0::2], 0) and np.allclose(pe[3, 1::2], 1)   # distance 0
    assert abs(pe[4, 0] - np.sin(1.0)) < 1e-15 and abs(pe[4, 2] - np.sin(10000 ** (-2 / 512))) < 1e-15
    assert np.allclose(pe[2, 0::2], -pe[4, 0::2]) and np.allclose(pe[2, 1::2], pe[4, 1::2])


def test_conv_module_against_np_convolve_and_bn(sf_weights_full):
    w = sf_weights_full
    p = "conf2."
    rng = np.random.default_rng(6)
    W = 13
    h = rng.normal(size=(W, 512))
    got = SF.conv_module(w, p, h, W)
    a = h @ w[p + "conv.pw1.w"].T + w[p + "conv.pw1.b"]
    g = TF.glu(_t(a), dim=-1).numpy()
    d = np.stack([np.convolve(g[:, c], w[p + "conv.dw.w"][c, ::-1], mode="same")
                  for c in range(512)], axis=1) + w[p + "conv.dw.b"]
    bn = TF.batch_norm(_t(d), _t(w[p + "conv.bn.mean"]), _t(w[p + "conv.bn.var"]),
                       _t(w[p + "conv.bn.g"]), _t(w[p + "conv.bn.b"]), training=False,
                       eps=1e-5).numpy()
    ref = TF.silu(_t(bn)).numpy() @ w[p + "conv.pw2.w"].T + w[p + "conv.pw2.b"]
    assert np.abs(got - ref).max() < 1e-11


def test_layernorm_ffn_and_transformer_layer_vs_torch(sf_weights_full):
    w = sf_weights_full
    rng = np.random.default_rng(7)
    x = rng.normal(size=(9, 192))
    p = "tf3."
    got = SF.transformer_layer(w, 3, x, 9)
    xt = _t(x)
    q = TF.linear(xt, _t(w[p + "wq"]), _t(w[p + "bq"])).view(9, 8, 24).transpose(0, 1)
    k = TF.linear(xt, _t(w[p + "wk"]), _t(w[p + "bk"])).view(9, 8, 24).transpose(0, 1)
    v = TF.linear(xt, _t(w[p + "wv"]), _t(w[p + "bv"])).view(9, 8, 24).transpose(0, 1)
    ctx = TF.scaled_dot_product_attention(q, k, v).transpose(0, 1).reshape(9, 192)
    y = TF.layer_norm(xt + TF.linear(ctx, _t(w[p + "wo"]), _t(w[p + "bo"])), (192,),
                      _t(w[p + "ln1.g"]), _t(w[p + "ln1.b"]), eps=1e-5)
    f = TF.linear(TF.relu(TF.linear(y, _t(w[p + "w1"]), _t(w[p + "b1"]))), _t(w[p + "w2"]),
                  _t(w[p + "b2"]))
    ref = TF.layer_norm(y + f, (192,), _t(w[p + "ln2.g"]), _t(w[p + "ln2.b"]), eps=1e-5).numpy()
    assert np.abs(got - ref).max() < 1e-11


def test_key_mask_matches_torch(sf_weights_full):
    rng = np.random.default_rng(8)
    q, k, v = (rng.normal(size=(2, 6, 5)) for _ in range(3))
    s = q @ k.transpose(0, 2, 1)
    a = SF.softmax_masked(s, 4)
    mask = torch.zeros(6, 6, dtype=torch.bool)
    mask[:, :4] = True
    ref = TF.scaled_dot_product_attention(_t(q), _t(k), _t(v), attn_mask=mask, scale=1.0).numpy()
    assert np.abs(a @ v - ref).max() < 1e-12


def test_offline_output_shape_and_range(sf_weights_f32):
    from synthetic import workload_audio
    audio = workload_audio("offline8s")
    p = run.sortformer_offline(audio, sf_weights_f32)
    assert list((1,) + p.shape) == GOLD["offline_8s_output_shape"]["value"]
    assert np.all((p > 0) & (p < 1))


@pytest.mark.parametrize("model", ["sortformer", "nemotron"])
def test_right_padding_invariance(model, sf_weights_full, nm_weights_full):
    rng = np.random.default_rng(9)
    W, P = 11, 5
    emb = rng.normal(size=(W, 512))
    pad = np.concatenate([emb, rng.normal(size=(P, 512)) * 3])
    if model == "sortformer":
        a = SF.encode_window(sf_weights_full, emb, n_conformer=3, n_transformer=3)
        b = SF.encode_window(sf_weights_full, pad, n_valid=W, n_conformer=3, n_transformer=3)
        assert np.abs(a - b[:W]).max() < 1e-12
    else:
        a = NM.encode_window(nm_weights_full, emb, n_layers=3)[0]
        b = NM.encode_window(nm_weights_full, pad, n_valid=W, n_layers=3)[0]
        assert np.abs(a - b[:W]).max() < 1e-12


def test_stream_single_chunk_equals_offline(sf_weights_f32):
    from synthetic import meeting_audio
    audio = meeting_audio(3.2, 2, 11)
    off = run.sortformer_offline(audio, sf_weights_f32)
    cfg = streaming.StreamConfig(chunk_len=10_000, right_context=0, fifo_len=188, update_period=144)
    st, _ = run.sortformer_stream(audio, sf_weights_f32, cfg)
    assert st.shape == off.shape == (40, 4)
    assert np.abs(st - off).max() < 1e-13


# ---------------------------------------------------------------- Nemotron
def test_rope_properties():
    rng = np.random.default_rng(10)
    q = rng.normal(size=(1, 6, 64))
    k = rng.normal(size=(1, 6, 64))
    pos = np.arange(6)
    qr, kr = NM.rope(q, pos), NM.rope(k, pos)
    assert np.allclose(np.linalg.norm(qr, axis=-1), np.linalg.norm(q, axis=-1))
    assert np.allclose(NM.rope(q, np.zeros(6))[0], q[0])
    # scores depend on relative position only
    qq = np.repeat(q[:, :1], 6, axis=1)
    kk = np.repeat(k[:, :1], 6, axis=1)
    s = np.einsum("hid,hjd->hij", NM.rope(qq, pos), NM.rope(kk, pos))[0]
    for dlt in range(-3, 4):
        diag = np.diagonal(s, offset=dlt)
        assert np.allclose(diag, diag[0])


def test_rope_matches_complex_rotation():
    rng = np.random.default_rng(11)
    x = rng.normal(size=(1, 3, 64))
    pos = np.array([0, 5, 17])
    z = x[..., :32] + 1j * x[..., 32:]
    theta = pos[:, None] * 10000.0 ** (-np.arange(32) / 32)
    zr = z * np.exp(1j * theta)
    ref = np.concatenate([zr.real, zr.imag], axis=-1)
    assert np.allclose(NM.rope(x, pos), ref, atol=1e-13)


def test_nemotron_parts_vs_torch(nm_weights_full):
    w = nm_weights_full
    rng = np.random.default_rng(12)
    z = rng.normal(size=(5, 8))
    up = NM.upsample_head(w, z)
    ref = TF.conv_transpose1d(_t(z.T)[None], _t(w["up.w"]), _t(w["up.b"]), stride=8)[0].numpy().T
    assert up.shape == (40, 8) and np.abs(up - ref).max() < 1e-13
    x = rng.normal(size=(100,))
    assert np.abs(NM.gelu(x) - TF.gelu(_t(x)).numpy()).max() < 1e-14
    mel = rng.normal(size=(19, 128))
    st = NM.stack_frames(mel)
    assert st.shape == (3, 1024) and np.array_equal(st[1, 128 * 3:128 * 4], mel[11])
    assert np.all(st[2, 128 * 3:] == 0)


def test_nemotron_layer_vs_torch(nm_weights_full):
    w = nm_weights_full
    rng = np.random.default_rng(13)
    W = 7
    x = rng.normal(size=(W, 512))
    got = NM.rope_layer(w, 4, x, W)
    p = "rl4."
    xt = _t(x)
    h = TF.layer_norm(xt, (512,), _t(w[p + "ln1.g"]), _t(w[p + "ln1.b"]), eps=1e-5)

    def heads(m):
        return TF.linear(h, _t(w[p + f"w{m}"]), _t(w[p + f"b{m}"])).view(W, 8, 64).transpose(0, 1)

    q, k, v = heads("q"), heads("k"), heads("v")
    # rotary applied as complex multiplication (an independent formulation)
    f64 = torch.float64  # every tensor here is fp64 (no process-wide default is set)
    ang = torch.arange(W, dtype=f64)[:, None] * 10000.0 ** (-torch.arange(32, dtype=f64) / 32)
    rot = torch.polar(torch.ones_like(ang), ang)

    def rope_c(t):
        zc = torch.complex(t[..., :32], t[..., 32:]) * rot
        return torch.cat([zc.real, zc.imag], dim=-1)

    ctx = TF.scaled_dot_product_attention(rope_c(q), rope_c(k), v).transpose(0, 1).reshape(W, 512)
    y = xt + TF.linear(ctx, _t(w[p + "wo"]), _t(w[p + "bo"]))
    h2 = TF.layer_norm(y, (512,), _t(w[p + "ln2.g"]), _t(w[p + "ln2.b"]), eps=1e-5)
    ref = y + TF.linear(TF.gelu(TF.linear(h2, _t(w[p + "w1"]), _t(w[p + "b1"]))),
                        _t(w[p + "w2"]), _t(w[p + "b2"]))
    assert np.abs(got - ref.numpy()).max() < 1e-11


def test_nemotron_output_pooling_definition():
    """Output frames of r x 10 ms: the mean of r consecutive 10 ms frames,
    checked against an explicit loop; r = 1 is the identity; a constant track
    stays constant; the mean over the clip is unchanged."""
    rng = np.random.default_rng(14)
    p = rng.random((8 * 7, 8))
    assert np.array_equal(NM.pool_output(p, 1), p)
    for r in (2, 4, 8):
        got = NM.pool_output(p, r)
        ref = np.array([[sum(p[r * k + q, s] for q in range(r)) / r for s in range(8)]
                        for k in range(p.shape[0] // r)])
        assert got.shape == (p.shape[0] // r, 8) and np.abs(got - ref).max() < 1e-15
        assert abs(got.mean() - p.mean()) < 1e-15
        assert np.allclose(NM.pool_output(np.full((16, 8), 0.3), r), 0.3)
    with pytest.raises(ValueError):
        NM.pool_output(p, 3)
