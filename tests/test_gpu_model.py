"""GPU parity of the frontend, pre_encode and encoder against the fp64 oracle.

Tolerances (stated in the workload description): fp32 path max|dp| <= 1e-4;
bf16 path max|dp| <= 2e-2 with >= 99.5% agreement of p > 0.5. Feature-level
checks (mel, embeddings) use bounds derived from fp32 rounding of sums of a
few hundred to a few thousand terms (relative ~1e-5 of the value scale).
"""
import numpy as np
import pytest
import torch

from oracle import frontend as OF
from oracle import nemotron as ON
from oracle import run as OR
from oracle import sortformer as OS
from oracle.weights import make_weights
from synthetic import meeting_audio, workload_audio

pytestmark = pytest.mark.gpu


def _cuda(x):
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).cuda()


def _report(name, got, ref):
    err = float(np.abs(got - ref).max())
    agree = float(np.mean((got > 0.5) == (ref > 0.5)))
    print(f"[{name}] shape {got.shape} max|dp| {err:.3e} agree {agree:.5f}", flush=True)
    if not err <= 1e-3:  # say what the output looked like
        bad = np.argwhere(np.abs(got - ref) > 1e-3)
        print(f"  got range [{np.nanmin(got):.4g}, {np.nanmax(got):.4g}] nan {np.isnan(got).sum()}"
              f" | ref range [{ref.min():.4g}, {ref.max():.4g}] | {len(bad)} entries off, first"
              f" {bad[:4].tolist()} last {bad[-4:].tolist()}", flush=True)
    return err, agree


@pytest.fixture(scope="module")
def rt():
    from streaming_speaker_diarization_amd import runtime
    return runtime


@pytest.fixture(scope="module")
def sf32(rt):
    return rt.Model("sortformer", "f32", seed=0)


@pytest.fixture(scope="module")
def w32():
    return make_weights("sortformer", 0)


@pytest.fixture(scope="module")
def sfbf(rt):
    return rt.Model("sortformer", "bf16", seed=0)


@pytest.fixture(scope="module")
def wbf():
    return make_weights("sortformer", 0, bf16=True)


@pytest.fixture(scope="module")
def emb20(w32):
    """Oracle pre-encoded embeddings of a 40 s clip (500 frames)."""
    return OR.pre_encode_all(w32, OF.log_mel(meeting_audio(40.0, 3, 31)))


def test_offline_8s_fp32(sf32, w32):
    audio = workload_audio("offline8s")
    got = sf32.offline(_cuda(audio)[None])[0].cpu().numpy()
    ref = OR.sortformer_offline(audio, w32)
    assert got.shape == (100, 4)
    err, _ = _report("offline8s f32", got, ref)
    assert err <= 1e-4


def test_frontend_and_pre_encode_fp32_ragged(sf32, w32):
    audio = meeting_audio(8.0, 2, 21)[:128000 - 4321]   # T = 772, not a multiple of 8
    mel, emb = sf32.pre_encode(_cuda(audio)[None])
    mel, emb = mel[0].cpu().numpy(), emb[0].cpu().numpy()
    ref_mel = OF.log_mel(audio)
    assert mel.shape == ref_mel.shape == (772, 128)
    em = float(np.abs(mel - ref_mel).max())
    ref_emb = OR.pre_encode_all(w32, ref_mel)
    assert emb.shape == ref_emb.shape == (97, 512)
    ee = float(np.abs(emb - ref_emb).max())
    scale = float(np.abs(ref_emb).max())
    p999 = float(np.quantile(np.abs(mel - ref_mel), 0.999))
    print(f"[pre_encode f32] mel max|d| {em:.2e} (99.9% {p999:.2e})  emb max|d| {ee:.2e} "
          f"(scale {scale:.2e})")
    # fp32 DFT of 400 terms: absolute error ~ sqrt(400) 2^-24 sum|x w|, so a
    # bin 30 dB below its frame's energy carries ~1e-4 relative power error;
    # the log-mel error is that relative error.
    assert em <= 2e-3 and p999 <= 1e-4
    assert ee <= 1e-4 * max(scale, 1.0)


@pytest.mark.parametrize("W", [1, 5, 64, 65, 130])
def test_encode_window_fp32(sf32, w32, emb20, W):
    x = emb20[:W]
    got = sf32.encode_window(_cuda(x)[None])[0].cpu().numpy()
    ref = OS.encode_window(w32, x)
    err, _ = _report(f"window f32 W={W}", got, ref)
    assert err <= 1e-4


def test_encode_window_full_random_padded_batched(rt, emb20):
    m = rt.Model("sortformer", "f32", seed=7, full_random=True)
    w = make_weights("sortformer", 7, full_random=True)
    W, nv = 77, 60
    xs = np.stack([emb20[0:W], emb20[100:100 + W], emb20[300:300 + W]])
    got = m.encode_window(_cuda(xs), n_valid=nv).cpu().numpy()
    for b in range(3):
        ref = OS.encode_window(w, xs[b], n_valid=nv)
        err, _ = _report(f"window f32 full-random padded b={b}", got[b, :nv], ref[:nv])
        assert err <= 1e-4


def test_encode_window_bf16_full_size(sfbf, wbf):
    """Largest window of the 'low' preset (cache 188 + FIFO 186 + 6 + 7)."""
    emb = OR.pre_encode_all(make_weights("sortformer", 0, bf16=True),
                            OF.log_mel(workload_audio("low60s")))[:387]
    got = sfbf.encode_window(_cuda(emb)[None])[0].cpu().numpy()
    ref = OS.encode_window(wbf, emb)
    err, agree = _report("window bf16 W=387", got, ref)
    assert err <= 2e-2 and agree >= 0.995


def test_encode_window_bf16_batched_throughput_regime(sfbf, wbf):
    """11 padded windows of 390 frames (4290 rows: the batched GEMM and
    attention forms), 333 valid frames each: valid rows match the oracle per
    stream and rows past n_valid do not change them."""
    B, W, nv = 11, 390, 333
    full = OR.pre_encode_all(make_weights("sortformer", 0, bf16=True),
                             OF.log_mel(workload_audio("low60s")))
    xs = np.stack([full[17 * b:17 * b + W] for b in range(B)])
    xs[:, nv:] = np.random.default_rng(5).standard_normal((B, W - nv, 512))  # padding garbage
    got = sfbf.encode_window(_cuda(xs), n_valid=nv).cpu().numpy()
    for b in (0, 6, 10):
        ref = OS.encode_window(wbf, xs[b], n_valid=nv)
        err, agree = _report(f"window bf16 batched B={B} W={W} valid={nv} b={b}", got[b, :nv],
                             ref[:nv])
        assert err <= 2e-2 and agree >= 0.995


@pytest.mark.parametrize("B,W,nv", [(160, 30, 27), (45, 100, 93)])
def test_encode_window_bf16_batched_short_windows(sfbf, wbf, B, W, nv):
    """Batches of short windows above 4096 rows: the batched kernels' paths for
    windows shorter than their row tiles (V^T stores of the Q/K/V GEMM below
    128 rows per window, of the transformer tail below 48) against the oracle
    on sampled streams; rows past n_valid hold garbage."""
    full = OR.pre_encode_all(make_weights("sortformer", 0, bf16=True),
                             OF.log_mel(workload_audio("low60s")))
    span = full.shape[0] - W
    xs = np.stack([full[(17 * b) % span:(17 * b) % span + W] for b in range(B)])
    xs[:, nv:] = np.random.default_rng(B).standard_normal((B, W - nv, 512))
    got = sfbf.encode_window(_cuda(xs), n_valid=nv).cpu().numpy()
    for b in (0, B // 2 + 1, B - 1):
        ref = OS.encode_window(wbf, xs[b], n_valid=nv)
        err, agree = _report(f"window bf16 batched B={B} W={W} valid={nv} b={b}", got[b, :nv],
                             ref[:nv])
        assert err <= 2e-2 and agree >= 0.995


def test_nemotron_window_fp32_and_bf16(rt, emb20):
    m = rt.Model("nemotron", "f32", seed=1)
    w = make_weights("nemotron", 1)
    x = emb20[:100]
    p80, p10 = m.encode_window(_cuda(x)[None])
    r80, r10 = ON.encode_window(w, x)
    e1, _ = _report("nemotron f32 p80", p80[0].cpu().numpy(), r80)
    e2, _ = _report("nemotron f32 p10", p10[0].cpu().numpy(), r10)
    assert e1 <= 1e-4 and e2 <= 1e-4
    mb = rt.Model("nemotron", "bf16", seed=1)
    wb = make_weights("nemotron", 1, bf16=True)
    x = emb20[:130]
    p80, p10 = mb.encode_window(_cuda(x)[None])
    r80, r10 = ON.encode_window(wb, x)
    e3, a3 = _report("nemotron bf16 p10", p10[0].cpu().numpy(), r10)
    assert e3 <= 2e-2 and a3 >= 0.995


def test_offline_fp32_batched_matches_single(sf32):
    a = np.stack([meeting_audio(4.0, 2, 41), meeting_audio(4.0, 3, 42)])
    both = sf32.offline(_cuda(a)).cpu().numpy()
    one = sf32.offline(_cuda(a[1:])).cpu().numpy()
    assert np.array_equal(both[1], one[0])   # same kernels, same order: bit-identical


def test_binding_checks_and_default_dtype_independence(sf32):
    """The runtime allocates float32 whatever torch's default dtype is, and the
    binding refuses mistyped or short buffers before launching anything."""
    from streaming_speaker_diarization_amd import sortformer as sf
    audio = _cuda(meeting_audio(3.0, 2, 11))[None]
    ref = sf32.offline(audio).cpu()
    old = torch.get_default_dtype()
    torch.set_default_dtype(torch.float64)
    try:
        got = sf32.offline(audio).cpu()
    finally:
        torch.set_default_dtype(old)
    assert got.dtype == torch.float32 and torch.equal(got, ref)
    ws = sf32.workspace(sf.sortformer_offline_workspace_bytes(sf32.handle, 1, audio.shape[1]))
    with pytest.raises(TypeError):
        sf.sortformer_forward_offline(sf32.handle, audio.double(), torch.empty(1, 38, 4).cuda(), ws)
    with pytest.raises(ValueError):
        sf.sortformer_forward_offline(sf32.handle, audio,
                                      torch.empty(1, 10, 4, dtype=torch.float32).cuda(), ws)
