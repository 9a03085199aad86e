"""Buffer management around the C ABI: allocates the weight, workspace and
state buffers with PyTorch on the current device and calls the library.
No arithmetic of the method happens here."""
from __future__ import annotations

import torch

from . import sortformer as sf


def _bytes(n: int, device) -> torch.Tensor:
    return torch.empty(max(int(n), 1), dtype=torch.uint8, device=device)


class Model:
    def __init__(self, arch: str = "sortformer", dtype: str = "bf16", seed: int | None = None,
                 full_random: bool = False, device: str = "cuda"):
        if not torch.cuda.is_available():
            raise RuntimeError("the HIP library needs a GPU")
        self.arch, self.dtype = arch, dtype
        self.cfg = sf.model_config(arch, dtype, full_random)
        self.seed = (0 if arch == "sortformer" else 1) if seed is None else seed
        self.device = torch.device(device)
        nbytes = sf.sortformer_weight_bytes(self.cfg)
        if nbytes == 0:
            raise ValueError("invalid model configuration")
        self.weights = _bytes(nbytes, self.device)
        self.handle = sf.sortformer_init(self.cfg, self.seed, self.weights)
        self.n_spk = self.cfg.n_spk
        self._ws = None
        self._taps = {}  # keeps registered tap buffers alive

    def __del__(self):
        h = getattr(self, "handle", None)
        if h and sf is not None and sf.sortformer_free is not None:
            sf.sortformer_free(h)
            self.handle = None

    def set_output_stride(self, r: int):
        """Nemotron: output frames of r x 10 ms (r in 1, 2, 4, 8)."""
        sf.sortformer_set_option(self.handle, sf.SF_OPT_OUTPUT_STRIDE, r)

    def output_stride(self) -> int:
        return sf.sortformer_get_option(self.handle, sf.SF_OPT_OUTPUT_STRIDE)

    def metadata(self) -> dict:
        return sf.sortformer_get_metadata(self.handle)

    def workspace(self, nbytes: int) -> torch.Tensor:
        if self._ws is None or self._ws.numel() < nbytes:
            self._ws = _bytes(nbytes, self.device)
        return self._ws

    def offline(self, audio: torch.Tensor) -> torch.Tensor:
        B, N = audio.shape
        ws = self.workspace(sf.sortformer_offline_workspace_bytes(self.handle, B, N))
        te = (N // 160 + 7) // 8
        n_out = te if self.arch == "sortformer" else 8 // self.output_stride() * te
        out = torch.empty(B, max(n_out, 1), self.n_spk, dtype=torch.float32, device=self.device)
        got = sf.sortformer_forward_offline(self.handle, audio.contiguous(), out, ws)
        return out[:, :got]

    def encode_window(self, emb: torch.Tensor, n_valid: int | None = None):
        B, W, _ = emb.shape
        ws = self.workspace(sf.sortformer_encode_workspace_bytes(self.handle, B, W))
        p = torch.empty(B, W, self.n_spk, dtype=torch.float32, device=self.device)
        p10 = torch.empty(B, 8 * W, self.n_spk, dtype=torch.float32, device=self.device) \
            if self.arch == "nemotron" else None
        sf.sortformer_encode_window(self.handle, emb.contiguous(), W if n_valid is None else n_valid,
                                    p, p10, ws)
        return p if p10 is None else (p, p10)

    def tap(self, layer: int, point: int, out: torch.Tensor | None):
        """Have encode_window also write the (layer, point) activation into
        `out` (float32, at least batch x window x width elements); None
        removes the tap. The tensor must outlive the registration."""
        sf.sortformer_debug_tap(self.handle, layer, point, out)
        if out is None:
            self._taps.pop((layer, point), None)
        else:
            self._taps[(layer, point)] = out

    def clear_taps(self):
        sf.sortformer_debug_tap(self.handle, -1, 0, None)
        self._taps.clear()

    def pre_encode(self, audio: torch.Tensor):
        B, N = audio.shape
        T = N // 160
        te = (T + 7) // 8
        ws = self.workspace(sf.sortformer_pre_encode_workspace_bytes(self.handle, B, N))
        mel = torch.empty(B, max(T, 1), 128, dtype=torch.float32, device=self.device)
        emb = torch.empty(B, max(te, 1), 512, dtype=torch.float32, device=self.device)
        sf.sortformer_pre_encode(self.handle, audio.contiguous(), mel, emb, ws)
        return mel[:, :T], emb[:, :te]

    def stream(self, preset="low", batch: int = 1, config: sf.sf_stream_config | None = None):
        return Stream(self, config if config is not None else sf.sortformer_stream_preset(preset),
                      batch)


class Stream:
    def __init__(self, model: Model, scfg, batch: int = 1):
        self.model, self.scfg, self.B = model, scfg, batch
        nbytes = sf.sortformer_state_bytes(model.handle, scfg, batch)
        if nbytes == 0:
            raise ValueError("unsupported stream configuration")
        self.state = _bytes(nbytes, model.device)
        self.ws = _bytes(sf.sortformer_stream_workspace_bytes(model.handle, scfg, batch),
                         model.device)
        self.handle = sf.sortformer_stream_create(model.handle, scfg, batch, self.state)
        self.out = torch.empty(batch, sf.sortformer_stream_max_emit(self.handle), model.n_spk,
                               dtype=torch.float32, device=model.device)

    def __del__(self):
        h = getattr(self, "handle", None)
        if h and sf is not None and sf.sortformer_stream_destroy is not None:
            sf.sortformer_stream_destroy(h)
            self.handle = None

    def samples_needed(self) -> int:
        return sf.sortformer_stream_samples_needed(self.handle)

    def step(self, audio_new: torch.Tensor, is_last: bool = False) -> torch.Tensor:
        """audio_new (B, n) on the device -> this step's probabilities (B, n_emit, S)
        (a view of a buffer the next step overwrites)."""
        n = sf.sortformer_stream_step(self.handle, audio_new.contiguous(), audio_new.shape[1],
                                      is_last, self.out, self.ws)
        # the library writes the emitted rows densely as (B, n, S)
        return self.out.view(-1)[:self.B * n * self.model.n_spk].view(self.B, n, self.model.n_spk)

    def feed(self, audio_new: torch.Tensor, is_last: bool = False) -> torch.Tensor:
        """Any number of new samples (B, n) on the device -> the probabilities
        (B, frames, S) of every step they completed (possibly none); the rest
        waits in the stream's audio ring. A fresh tensor each call."""
        n = audio_new.shape[1]
        frames = sf.sortformer_stream_feed_frames(self.handle, n, is_last)
        if frames < 0:
            raise sf.SortformerError(sf.SF_ESTATE, "stream_feed")
        out = torch.empty(self.B, max(frames, 1), self.model.n_spk, dtype=torch.float32,
                          device=self.model.device)
        got = sf.sortformer_stream_feed(self.handle, audio_new.contiguous(), is_last, out, self.ws)
        return out[:, :got]

    def export(self):
        """The whole stream state (cache, FIFO, look-ahead, silence statistics,
        audio ring, counters) as a host byte array."""
        return sf.sortformer_stream_export(self.handle)

    def import_(self, blob):
        sf.sortformer_stream_import(self.handle, blob)

    def reset(self):
        sf.sortformer_stream_reset(self.handle)

    def info(self):
        return sf.sortformer_stream_get_info(self.handle)

    def run(self, audio: torch.Tensor) -> torch.Tensor:
        """Feed a whole clip (B, N) the way a live stream would and return the
        concatenated emitted probabilities."""
        outs = []
        pos, N = 0, audio.shape[1]
        while True:
            need = self.samples_needed()
            if pos + need > N:  # the clip ends within this step's audio
                outs.append(self.step(audio[:, pos:N], is_last=True).clone())
                break
            outs.append(self.step(audio[:, pos:pos + need]).clone())
            pos += need
        return torch.cat(outs, dim=1)


# numpy view of the library's sf_segment records
SEGMENT_DTYPE = [("start_s", "<f8"), ("end_s", "<f8"), ("speaker", "<i4"), ("stream", "<i4")]


def segments(probs: torch.Tensor, frame_s: float = 0.08, **params):
    """Per-frame speaker probabilities (B, T, S) on the device -> for each
    stream a list of [start_s, end_s, speaker] segments sorted by start time
    (then speaker). The thresholding and smoothing run in the library's
    kernel; this only formats its per-track lists. Keyword parameters:
    onset, offset, pad_onset, pad_offset, min_duration_on, min_duration_off."""
    import numpy as np
    prm = sf.sortformer_segment_defaults()
    for k, v in params.items():
        if not hasattr(prm, k):
            raise TypeError(f"unknown segment parameter {k}")
        setattr(prm, k, v)
    probs = probs.contiguous()
    B, T, S = probs.shape
    if T == 0:
        return [[] for _ in range(B)]
    cap = sf.sortformer_segments_capacity(T)
    out = _bytes(B * S * cap * sf.SEGMENT_BYTES, probs.device)
    counts = torch.empty(B * S, dtype=torch.int64, device=probs.device)
    sf.sortformer_segments(probs, frame_s, prm, out, cap, counts)
    recs = out[:B * S * cap * sf.SEGMENT_BYTES].cpu().numpy().view(SEGMENT_DTYPE).reshape(B * S, cap)
    n = counts.cpu().numpy()
    result = []
    for b in range(B):
        segs = [[float(r["start_s"]), float(r["end_s"]), int(r["speaker"])]
                for s in range(S) for r in recs[b * S + s, :n[b * S + s]]]
        result.append(sorted(segs, key=lambda x: (x[0], x[2], x[1])))
    return result


def speaker_dicts(probs: torch.Tensor, frame_s: float = 0.08, **params):
    """The same segments as {"Start", "End", "Speaker"} dictionaries."""
    return [[{"Start": a, "End": e, "Speaker": k} for a, e, k in segs]
            for segs in segments(probs, frame_s, **params)]
