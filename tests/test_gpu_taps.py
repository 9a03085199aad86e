"""Per-layer GPU parity through the encoder taps (sortformer_debug_tap).

The end-to-end probabilities of randomly initialised models sit close to 0.5
and react little to any one layer, so these tests check every layer kind on
its own: the activation entering a tapped layer is read back from the GPU and
the oracle computes, from that same input, the layer's attention context
(softmax(scores) V before W_o) and its output. Inputs are i.i.d. unit-normal
frames, so attention weights differ strongly between keys and an error in the
scores shows up in the context.

Tolerances. fp32 path: every operation rounds to fp32 (unit roundoff 2^-24)
over sums of at most a few thousand terms, so the relative error of a layer
is ~1e-6; bounds: relative RMS 1e-5, max |error| / max |ref| 1e-4. bf16 path:
GEMM operands, the attention probabilities and the context are rounded to
bf16 (relative error <= 2^-9 each, RMS 2^-9/sqrt(3) ~ 1.1e-3), about six
roundings in sequence per layer, so the relative RMS error is a few 1e-3;
bounds: relative RMS 1e-2, max |error| / max |ref| 3e-2. The planted-mistake
check shows the bound separates a one-frame shift of the relative positions
(computed by the oracle on the CPU).
"""
import numpy as np
import pytest
import torch

from oracle import nemotron as ON
from oracle import sortformer as OS
from oracle.weights import make_weights

pytestmark = pytest.mark.gpu

IN, CTX, OUT = 0, 1, 2
TOL = {"f32": (1e-5, 1e-4), "bf16": (1e-2, 3e-2)}


def _cuda(x):
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).cuda()


def _metrics(got, ref):
    d = got - ref
    return (float(np.linalg.norm(d) / np.linalg.norm(ref)),
            float(np.abs(d).max() / np.abs(ref).max()))


def _check(name, got, ref, dtype):
    rr, rm = _metrics(got, ref)
    print(f"[{name}] rel_rms {rr:.3e} rel_max {rm:.3e}", flush=True)
    assert np.isfinite(got).all()
    assert rr <= TOL[dtype][0] and rm <= TOL[dtype][1], name
    return rr


def _run_taps(model, emb, n_valid, taps, width):
    """encode_window with the (layer, point) taps; returns {(layer, point): (B, W, d)}."""
    B, W, _ = emb.shape
    bufs = {}
    model.clear_taps()
    for lp in taps:
        bufs[lp] = torch.full((B, W, width(lp[0])), float("nan"), device="cuda")
        model.tap(lp[0], lp[1], bufs[lp])
    model.encode_window(_cuda(emb), n_valid=n_valid)
    torch.cuda.synchronize()
    model.clear_taps()
    return {k: v.cpu().numpy().astype(np.float64) for k, v in bufs.items()}


def _sf_width(layer):
    return 512 if layer < 17 else 192


@pytest.fixture(scope="module")
def rt():
    from streaming_speaker_diarization_amd import runtime
    return runtime


def _sortformer_layers(w, got, b, layers, n_valid, tag):
    dtype = tag.split()[0]
    for L in layers:
        x = got[(L, IN)][b]
        if L < 17:
            ctx = OS.conformer_attention_context(w, L, x, n_valid)
            out = OS.conformer_layer(w, L, x, n_valid)
        else:
            ctx = OS.mha_context(w, f"tf{L - 17}.", x, n_valid)
            out = OS.transformer_layer(w, L - 17, x, n_valid)
        _check(f"{tag} b={b} layer {L} ctx", got[(L, CTX)][b, :n_valid], ctx[:n_valid], dtype)
        _check(f"{tag} b={b} layer {L} out", got[(L, OUT)][b, :n_valid], out[:n_valid], dtype)


def test_sortformer_bf16_layers_single_window(rt):
    """One window of the 'low' preset's largest size (387 frames, 380 valid):
    the latency-form kernels."""
    m = rt.Model("sortformer", "bf16", seed=0)
    w = make_weights("sortformer", 0, bf16=True)
    W, nv = 387, 380
    emb = np.random.default_rng(11).standard_normal((1, W, 512))
    layers = [0, 8, 16, 17, 34]
    got = _run_taps(m, emb, nv, [(L, p) for L in layers for p in (IN, CTX, OUT)], _sf_width)
    _sortformer_layers(w, got, 0, layers, nv, "bf16 W=387")


def test_sortformer_bf16_layers_batched_throughput_form(rt):
    """11 windows of 390 frames, 333 valid (4290 rows: the batched GEMM and
    attention forms)."""
    m = rt.Model("sortformer", "bf16", seed=0)
    w = make_weights("sortformer", 0, bf16=True)
    B, W, nv = 11, 390, 333
    emb = np.random.default_rng(12).standard_normal((B, W, 512))
    layers = [0, 16, 17, 34]
    got = _run_taps(m, emb, nv, [(L, p) for L in layers for p in (IN, CTX, OUT)], _sf_width)
    for b in (0, 5, 10):
        _sortformer_layers(w, got, b, layers, nv, f"bf16 B={B} W={W}")


def test_sortformer_bf16_layers_batched_latency_form(rt):
    """5 windows of 203 frames, 190 valid (1015 rows: the latency forms, with
    the output projection fused into the attention epilogue): each stream
    against the oracle, and one stream bit-identical to the same window
    encoded alone (a row's arithmetic does not depend on the batch)."""
    m = rt.Model("sortformer", "bf16", seed=0)
    w = make_weights("sortformer", 0, bf16=True)
    B, W, nv = 5, 203, 190
    emb = np.random.default_rng(16).standard_normal((B, W, 512))
    layers = [0, 16, 17, 34]
    taps = [(L, p) for L in layers for p in (IN, CTX, OUT)]
    got = _run_taps(m, emb, nv, taps, _sf_width)
    for b in (0, 2, 4):
        _sortformer_layers(w, got, b, layers, nv, f"bf16 B={B} W={W}")
    alone = _run_taps(m, emb[3:4], nv, taps, _sf_width)
    for k in taps:
        assert np.array_equal(alone[k][0, :nv], got[k][3, :nv]), k


def test_nemotron_bf16_layers_batched(rt):
    """3 windows of 150 frames, 140 valid, through the rotary layers' fused
    output projection."""
    m = rt.Model("nemotron", "bf16", seed=1)
    w = make_weights("nemotron", 1, bf16=True)
    B, W, nv = 3, 150, 140
    emb = np.random.default_rng(17).standard_normal((B, W, 512))
    layers = [0, 30]
    got = _run_taps(m, emb, nv, [(L, p) for L in layers for p in (IN, CTX, OUT)], lambda L: 512)
    for b in range(B):
        for L in layers:
            x = got[(L, IN)][b]
            ctx = ON.rope_context(w, L, x, nv)
            out = ON.rope_layer(w, L, x, nv)
            if L == 30:
                out = ON.layer_norm(out, w["final_ln.g"], w["final_ln.b"])
            _check(f"nemotron bf16 B={B} b={b} layer {L} ctx", got[(L, CTX)][b, :nv], ctx[:nv], "bf16")
            _check(f"nemotron bf16 B={B} b={b} layer {L} out", got[(L, OUT)][b, :nv], out[:nv], "bf16")


def test_bf16_tolerance_separates_a_relative_position_shift(rt, monkeypatch):
    """Planted mistake, in the oracle: p(i-j+1) instead of p(i-j). The GPU
    context must sit inside the bf16 bound of the true oracle and far outside
    it for the shifted one."""
    m = rt.Model("sortformer", "bf16", seed=0)
    w = make_weights("sortformer", 0, bf16=True)
    for B, W, nv in ((1, 387, 380), (11, 390, 333)):
        emb = np.random.default_rng(13).standard_normal((B, W, 512))
        got = _run_taps(m, emb, nv, [(0, IN), (0, CTX)], _sf_width)
        x = got[(0, IN)][B - 1]
        true_ctx = OS.conformer_attention_context(w, 0, x, nv)[:nv]
        table = OS.rel_pos_table
        monkeypatch.setattr(OS, "rel_pos_table", lambda n, d=512: np.roll(table(n, d), -1, axis=0))
        shifted = OS.conformer_attention_context(w, 0, x, nv)[:nv]
        monkeypatch.setattr(OS, "rel_pos_table", table)
        g = got[(0, CTX)][B - 1, :nv]
        rr_true, _ = _metrics(g, true_ctx)
        rr_shift, _ = _metrics(g, shifted)
        print(f"[B={B}] rel_rms vs oracle {rr_true:.3e}, vs shifted oracle {rr_shift:.3e}",
              flush=True)
        assert rr_true <= TOL["bf16"][0] and rr_shift >= 2 * TOL["bf16"][0]


def test_sortformer_fp32_layers(rt):
    m = rt.Model("sortformer", "f32", seed=0)
    w = make_weights("sortformer", 0)
    W, nv = 200, 190
    emb = np.random.default_rng(14).standard_normal((1, W, 512))
    layers = [0, 16, 17, 34]
    got = _run_taps(m, emb, nv, [(L, p) for L in layers for p in (IN, CTX, OUT)], _sf_width)
    _sortformer_layers(w, got, 0, layers, nv, "f32 W=200")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_nemotron_layers(rt, dtype):
    m = rt.Model("nemotron", dtype, seed=1)
    w = make_weights("nemotron", 1, bf16=dtype == "bf16")
    W, nv = 300, 290
    emb = np.random.default_rng(15).standard_normal((1, W, 512))
    layers = [0, 15, 30]
    got = _run_taps(m, emb, nv, [(L, p) for L in layers for p in (IN, CTX, OUT)], lambda L: 512)
    for L in layers:
        x = got[(L, IN)][0]
        ctx = ON.rope_context(w, L, x, nv)
        out = ON.rope_layer(w, L, x, nv)
        if L == 30:
            out = ON.layer_norm(out, w["final_ln.g"], w["final_ln.b"])
        _check(f"nemotron {dtype} layer {L} ctx", got[(L, CTX)][0, :nv], ctx[:nv], dtype)
        _check(f"nemotron {dtype} layer {L} out", got[(L, OUT)][0, :nv], out[:nv], dtype)


def test_tap_registration_errors(rt):
    from streaming_speaker_diarization_amd import sortformer as sf
    m = rt.Model("sortformer", "bf16", seed=0)
    buf = torch.zeros(4 * 512, device="cuda")
    with pytest.raises(sf.SortformerError):
        m.tap(35, IN, buf)       # SORTFORMER has layers 0..34
    with pytest.raises(sf.SortformerError):
        m.tap(0, 3, buf)         # no such point
    for L in range(sf.SF_MAX_TAPS):
        m.tap(L, IN, buf)
    with pytest.raises(sf.SortformerError):
        m.tap(16, CTX, buf)      # one tap too many
    m.tap(3, IN, None)           # removing one makes room
    m.tap(16, CTX, buf)
    m.clear_taps()
    # a tap too small for the call: nothing is launched, the call fails
    m.tap(0, CTX, buf)
    with pytest.raises(sf.SortformerError):
        m.encode_window(torch.zeros(1, 8, 512, device="cuda"))
    m.clear_taps()
    p = m.encode_window(torch.zeros(1, 8, 512, device="cuda"))
    assert p.shape == (1, 8, 4)
