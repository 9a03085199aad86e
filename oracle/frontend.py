"""Log-mel frontend, float64.

"Streaming Sortformer Diarizer" model card, Pipeline and Model Parameters:
16 kHz audio -> mel spectrogram with 128 bins, 25 ms window, 10 ms stride.
The workload description fixes n_fft 512, Hann window 400, hop 160, 128
Slaney mel bands over 0-8 kHz and log(x + 2^-24).

Readings (the pages leave these open): periodic Hann of length 400 centred
inside the 512-point frame (56 zeros each side); centred STFT with 256 zero
samples of padding at both ends of the signal; power spectrum |X|^2; natural
log; no dither, pre-emphasis or feature normalisation; no pad-to-16 (the
ExecuTorch issue's Progress section reports it removed). The centred STFT
yields floor(N/160)+1 frames; the last ("extra") frame is dropped, so
T = floor(N/160) frames are produced.
"""
from __future__ import annotations

import numpy as np

SR = 16000
N_FFT = 512
WIN = 400
HOP = 160
N_MELS = 128
LOG_GUARD = 2.0 ** -24


def hz_to_mel_slaney(f):
    """Slaney mel scale: linear (3 mel per 200 Hz) below 1 kHz, logarithmic
    (27 mel per factor 6.4) above."""
    f = np.asarray(f, dtype=np.float64)
    lin = 3.0 * f / 200.0
    log = 15.0 + np.log(np.maximum(f, 1e-300) / 1000.0) * (27.0 / np.log(6.4))
    return np.where(f >= 1000.0, log, lin)


def mel_to_hz_slaney(m):
    m = np.asarray(m, dtype=np.float64)
    lin = 200.0 * m / 3.0
    log = 1000.0 * np.exp((m - 15.0) * (np.log(6.4) / 27.0))
    return np.where(m >= 15.0, log, lin)


def mel_filterbank(n_mels: int = N_MELS, n_fft: int = N_FFT, sr: int = SR,
                   fmin: float = 0.0, fmax: float = 8000.0) -> np.ndarray:
    """(n_mels, n_fft//2+1) triangular Slaney filters with area normalisation
    2/(f_{m+2}-f_m)."""
    edges = mel_to_hz_slaney(np.linspace(hz_to_mel_slaney(fmin), hz_to_mel_slaney(fmax),
                                         n_mels + 2))
    freqs = np.arange(n_fft // 2 + 1, dtype=np.float64) * sr / n_fft
    fb = np.zeros((n_mels, freqs.size))
    for m in range(n_mels):
        lo, ce, hi = edges[m], edges[m + 1], edges[m + 2]
        up = (freqs - lo) / (ce - lo)
        down = (hi - freqs) / (hi - ce)
        fb[m] = np.maximum(0.0, np.minimum(up, down)) * (2.0 / (hi - lo))
    return fb


def frame_window() -> np.ndarray:
    """512-point analysis window: periodic Hann(400) centred in the frame."""
    n = np.arange(WIN, dtype=np.float64)
    hann = 0.5 - 0.5 * np.cos(2.0 * np.pi * n / WIN)
    w = np.zeros(N_FFT)
    off = (N_FFT - WIN) // 2
    w[off:off + WIN] = hann
    return w


def n_frames(n_samples: int) -> int:
    return n_samples // HOP


def power_spectrum(audio: np.ndarray) -> np.ndarray:
    """(T, 257) |rfft(window * frame)|^2 for the T = floor(N/160) frames;
    frame t covers samples 160t-256 ... 160t+255 (zeros outside the clip)."""
    x = np.asarray(audio, dtype=np.float64)
    T = n_frames(x.size)
    pad = N_FFT // 2
    xp = np.concatenate([np.zeros(pad), x, np.zeros(pad + N_FFT)])
    idx = np.arange(T)[:, None] * HOP + np.arange(N_FFT)[None, :]
    frames = xp[idx] * frame_window()[None, :]
    spec = np.fft.rfft(frames, n=N_FFT, axis=1)
    return spec.real ** 2 + spec.imag ** 2


def log_mel(audio: np.ndarray) -> np.ndarray:
    """(T, 128) time-major log-mel features."""
    p = power_spectrum(audio)
    return np.log(p @ mel_filterbank().T + LOG_GUARD)
