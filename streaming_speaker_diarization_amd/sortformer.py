"""ctypes binding of libsortformer.so (argument marshalling only).

Every compute step runs in the library's HIP kernels; PyTorch only provides
device memory (tensors) and the stream handle. Functions keep the C names.
There is no fallback: if the library is missing, loading raises.
"""
from __future__ import annotations

import ctypes as C
import os

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libsortformer.so")

SF_OK, SF_EINVAL, SF_ESHAPE, SF_ENOMEM, SF_EHIP, SF_ESTATE, SF_EUNSUPPORTED = 0, -1, -2, -3, -4, -5, -6
SF_ARCH_SORTFORMER, SF_ARCH_NEMOTRON = 0, 1
SF_DTYPE_F32, SF_DTYPE_BF16 = 0, 1
SF_INIT_SPEC, SF_INIT_FULL_RANDOM = 0, 1
SF_MAX_WINDOW = 1024

# every symbol include/sortformer.h declares
EXPORTS = [
    "sortformer_status_string", "sortformer_stream_preset", "sortformer_weight_bytes",
    "sortformer_init", "sortformer_free", "sortformer_get_config", "sortformer_num_tensors",
    "sortformer_tensor_info", "sortformer_get_weights", "sortformer_offline_workspace_bytes",
    "sortformer_forward_offline", "sortformer_state_bytes", "sortformer_stream_workspace_bytes",
    "sortformer_stream_create", "sortformer_stream_destroy", "sortformer_stream_reset",
    "sortformer_stream_samples_needed", "sortformer_stream_max_emit", "sortformer_stream_step",
    "sortformer_stream_get_info", "sortformer_stream_export", "sortformer_stream_import",
    "sortformer_stream_checkpoint_bytes", "sortformer_stream_get_rows", "sortformer_stream_set_rows",
    "sortformer_stream_feed", "sortformer_stream_feed_frames", "sortformer_get_metadata",
    "sortformer_stream_step_noalloc", "sortformer_set_option", "sortformer_get_option",
    "sortformer_stream_update",
    "sortformer_encode_workspace_bytes", "sortformer_encode_window", "sortformer_pre_encode",
    "sortformer_pre_encode_workspace_bytes", "sortformer_config_num_tensors",
    "sortformer_config_tensor", "sortformer_profile_begin", "sortformer_profile_end",
    "sortformer_stream_set_option", "sortformer_segment_defaults", "sortformer_segments_capacity",
    "sortformer_segments", "sortformer_debug_tap",
]
SF_STREAM_OPT_GRAPHS = 1
SF_STREAM_OPT_FIXED_WINDOW = 2
SF_OPT_OUTPUT_STRIDE = 1
SF_NOALLOC_SCRATCH_BYTES = 64 << 20
SF_TAP_LAYER_IN, SF_TAP_ATTN_CTX, SF_TAP_LAYER_OUT = 0, 1, 2
SF_MAX_TAPS = 16
SF_PROF = {"gemm": 1, "attn": 2, "ln": 3, "conv": 4, "frontend": 5, "cache": 6}


class sf_model_config(C.Structure):
    _fields_ = [("arch", C.c_int32), ("dtype", C.c_int32), ("init_mode", C.c_int32),
                ("n_spk", C.c_int32)]


class sf_stream_config(C.Structure):
    _fields_ = [("chunk_len", C.c_int32), ("right_context", C.c_int32),
                ("fifo_len", C.c_int32), ("update_period", C.c_int32),
                ("spkcache_len", C.c_int32), ("n_sil_per_spk", C.c_int32)]


class sf_model_metadata(C.Structure):
    _fields_ = [("window_stride", C.c_double), ("output_frame_s", C.c_double),
                ("sample_rate", C.c_int32), ("subsampling_factor", C.c_int32),
                ("fc_d_model", C.c_int32), ("tf_d_model", C.c_int32),
                ("max_num_of_spks", C.c_int32), ("spkcache_len", C.c_int32),
                ("n_mels", C.c_int32), ("n_fft", C.c_int32), ("win_length", C.c_int32),
                ("hop_length", C.c_int32), ("n_conformer_layers", C.c_int32),
                ("n_transformer_layers", C.c_int32), ("n_heads", C.c_int32),
                ("max_window", C.c_int32)]


class sf_segment_params(C.Structure):
    _fields_ = [("onset", C.c_float), ("offset", C.c_float), ("pad_onset", C.c_double),
                ("pad_offset", C.c_double), ("min_duration_on", C.c_double),
                ("min_duration_off", C.c_double)]


class sf_segment(C.Structure):
    _fields_ = [("start_s", C.c_double), ("end_s", C.c_double), ("speaker", C.c_int32),
                ("stream", C.c_int32)]


SEGMENT_BYTES = C.sizeof(sf_segment)  # 24


class SortformerError(RuntimeError):
    def __init__(self, status, what):
        super().__init__(f"{what}: {status_string(status)} ({status})")
        self.status = status


_lib = None


def load(path: str = LIB_PATH):
    """Load the HIP library (raises if it was not built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} not found: build it first (__graft_entry__.build())")
    lib = C.CDLL(path)
    P, I32, I64, SZ, U64 = C.c_void_p, C.c_int32, C.c_int64, C.c_size_t, C.c_uint64
    cfgp, scfgp = C.POINTER(sf_model_config), C.POINTER(sf_stream_config)
    sig = {
        "sortformer_status_string": (C.c_char_p, [I32]),
        "sortformer_stream_preset": (I32, [C.c_char_p, scfgp]),
        "sortformer_weight_bytes": (SZ, [cfgp]),
        "sortformer_init": (I32, [cfgp, U64, P, SZ, P, C.POINTER(P)]),
        "sortformer_free": (None, [P]),
        "sortformer_get_config": (I32, [P, cfgp]),
        "sortformer_num_tensors": (I32, [P]),
        "sortformer_tensor_info": (I32, [P, I32, C.c_char_p, I32, C.POINTER(I64)]),
        "sortformer_get_weights": (I32, [P, I32, P]),
        "sortformer_offline_workspace_bytes": (SZ, [P, I32, I64]),
        "sortformer_forward_offline": (I32, [P, P, I32, I64, P, C.POINTER(I64), P, SZ, P]),
        "sortformer_state_bytes": (SZ, [P, scfgp, I32]),
        "sortformer_stream_workspace_bytes": (SZ, [P, scfgp, I32]),
        "sortformer_stream_create": (I32, [P, scfgp, I32, P, SZ, P, C.POINTER(P)]),
        "sortformer_stream_destroy": (None, [P]),
        "sortformer_stream_reset": (I32, [P, P]),
        "sortformer_stream_samples_needed": (I64, [P]),
        "sortformer_stream_max_emit": (I32, [P]),
        "sortformer_stream_step": (I32, [P, P, I64, I32, P, C.POINTER(I32), P, SZ, P]),
        "sortformer_stream_get_info": (I32, [P, C.POINTER(I64), C.POINTER(P)]),
        "sortformer_stream_checkpoint_bytes": (SZ, [P]),
        "sortformer_stream_export": (I32, [P, P, SZ, P]),
        "sortformer_stream_import": (I32, [P, P, SZ, P]),
        "sortformer_stream_get_rows": (I32, [P, P, P, P, P, P, P]),
        "sortformer_stream_set_rows": (I32, [P, I32, I32, I32, P, P, P, P, P, P]),
        "sortformer_stream_feed": (I32, [P, P, I64, I32, P, I64, C.POINTER(I64), P, SZ, P]),
        "sortformer_stream_feed_frames": (I64, [P, I64, I32]),
        "sortformer_stream_step_noalloc": (I32, [P, P, I64, I32, P, C.POINTER(I32), P]),
        "sortformer_set_option": (I32, [P, I32, I32]),
        "sortformer_get_option": (I32, [P, I32]),
        "sortformer_get_metadata": (I32, [P, C.POINTER(sf_model_metadata)]),
        "sortformer_stream_update": (I32, [P, P, I32, P, SZ, P]),
        "sortformer_encode_workspace_bytes": (SZ, [P, I32, I32]),
        "sortformer_encode_window": (I32, [P, P, I32, I32, I32, P, P, P, SZ, P]),
        "sortformer_debug_tap": (I32, [P, I32, I32, P, SZ]),
        "sortformer_pre_encode": (I32, [P, P, I32, I64, P, P, P, SZ, P]),
        "sortformer_pre_encode_workspace_bytes": (SZ, [P, I32, I64]),
        "sortformer_config_num_tensors": (I32, [cfgp]),
        "sortformer_config_tensor": (I32, [cfgp, U64, I32, C.c_char_p, I32, C.POINTER(I64), P]),
        "sortformer_profile_begin": (I32, [I32, I32]),
        "sortformer_stream_set_option": (I32, [P, I32, I32]),
        "sortformer_segment_defaults": (None, [C.POINTER(sf_segment_params)]),
        "sortformer_segments_capacity": (I64, [I64]),
        "sortformer_segments": (I32, [P, I32, I64, I32, C.c_double, C.POINTER(sf_segment_params),
                                      P, I64, P, P]),
        "sortformer_profile_end": (I32, [C.POINTER(C.c_double), C.POINTER(I64),
                                         C.POINTER(C.c_double), C.POINTER(C.c_double)]),
    }
    for name, (res, args) in sig.items():
        f = getattr(lib, name)
        f.restype = res
        f.argtypes = args
    _lib = lib
    return lib


def _check(st, what):
    if st != SF_OK:
        raise SortformerError(st, what)


def _ptr(t, min_numel=0):
    """Device address of a contiguous float32 tensor on the GPU (None passes
    through); raises before anything is launched when the tensor is on the
    host, strided, of another dtype or shorter than min_numel elements."""
    import torch
    if t is None:
        return None
    if not t.is_cuda:
        raise TypeError("expected a tensor in device memory")
    if not t.is_contiguous():
        raise ValueError("expected a contiguous tensor")
    if t.dtype != torch.float32:
        raise TypeError(f"expected a float32 tensor, got {t.dtype}")
    if t.numel() < min_numel:
        raise ValueError(f"buffer holds {t.numel()} elements, {min_numel} needed")
    return C.c_void_p(t.data_ptr())


def _buf(t):
    """(address, size in bytes) of a contiguous device byte buffer (workspace,
    stream state or weight arena) of any dtype."""
    if not t.is_cuda:
        raise TypeError("expected a buffer in device memory")
    if not t.is_contiguous():
        raise ValueError("expected a contiguous buffer")
    return C.c_void_p(t.data_ptr()), t.numel() * t.element_size()


def _stream(s):
    import torch
    if s is None:
        s = torch.cuda.current_stream()
    return C.c_void_p(s.cuda_stream)


# ---------------------------------------------------------------- C names
def status_string(st: int) -> str:
    return load().sortformer_status_string(st).decode()


def sortformer_stream_preset(name: str) -> sf_stream_config:
    c = sf_stream_config()
    _check(load().sortformer_stream_preset(name.encode(), C.byref(c)), "stream_preset")
    return c


def model_config(arch: str = "sortformer", dtype: str = "bf16", full_random: bool = False):
    a = SF_ARCH_SORTFORMER if arch == "sortformer" else SF_ARCH_NEMOTRON
    return sf_model_config(a, SF_DTYPE_BF16 if dtype == "bf16" else SF_DTYPE_F32,
                           SF_INIT_FULL_RANDOM if full_random else SF_INIT_SPEC,
                           4 if a == SF_ARCH_SORTFORMER else 8)


def sortformer_weight_bytes(cfg: sf_model_config) -> int:
    return load().sortformer_weight_bytes(C.byref(cfg))


def sortformer_init(cfg, seed, d_weights, stream=None):
    h = C.c_void_p()
    _check(load().sortformer_init(C.byref(cfg), seed, *_buf(d_weights), _stream(stream),
                                  C.byref(h)), "init")
    return h


def sortformer_free(h):
    load().sortformer_free(h)


def sortformer_set_option(h, option, value):
    _check(load().sortformer_set_option(h, option, int(value)), "set_option")


def sortformer_get_option(h, option) -> int:
    return load().sortformer_get_option(h, option)


def sortformer_get_metadata(h) -> dict:
    md = sf_model_metadata()
    _check(load().sortformer_get_metadata(h, C.byref(md)), "get_metadata")
    return {k: getattr(md, k) for k, _ in sf_model_metadata._fields_}


def sortformer_num_tensors(h) -> int:
    return load().sortformer_num_tensors(h)


def sortformer_tensor_info(h, i):
    buf = C.create_string_buffer(128)
    n = C.c_int64()
    _check(load().sortformer_tensor_info(h, i, buf, 128, C.byref(n)), "tensor_info")
    return buf.value.decode(), n.value


def sortformer_get_weights(h, i):
    import numpy as np
    _, n = sortformer_tensor_info(h, i)
    out = np.empty(n, np.float32)
    _check(load().sortformer_get_weights(h, i, out.ctypes.data_as(C.c_void_p)), "get_weights")
    return out


def sortformer_config_num_tensors(cfg) -> int:
    return load().sortformer_config_num_tensors(C.byref(cfg))


def sortformer_config_tensor(cfg, seed, index, values=True):
    """(name, float32 values or element count) of one generated tensor, host only."""
    import numpy as np
    buf = C.create_string_buffer(128)
    n = C.c_int64()
    _check(load().sortformer_config_tensor(C.byref(cfg), seed, index, buf, 128, C.byref(n), None),
           "config_tensor")
    if not values:
        return buf.value.decode(), n.value
    out = np.empty(n.value, np.float32)
    _check(load().sortformer_config_tensor(C.byref(cfg), seed, index, None, 0, None,
                                           out.ctypes.data_as(C.c_void_p)), "config_tensor")
    return buf.value.decode(), out


def sortformer_offline_workspace_bytes(h, batch, n_samples) -> int:
    return load().sortformer_offline_workspace_bytes(h, batch, n_samples)


def sortformer_forward_offline(h, d_audio, d_probs, d_ws, stream=None) -> int:
    B, N = d_audio.shape
    n_out = C.c_int64()
    cfg = sf_model_config()
    _check(load().sortformer_get_config(h, C.byref(cfg)), "get_config")
    te = (N // 160 + 7) // 8
    rows = te if cfg.arch == SF_ARCH_SORTFORMER else \
        8 // sortformer_get_option(h, SF_OPT_OUTPUT_STRIDE) * te
    _check(load().sortformer_forward_offline(h, _ptr(d_audio), B, N,
                                             _ptr(d_probs, B * rows * cfg.n_spk),
                                             C.byref(n_out), *_buf(d_ws), _stream(stream)),
           "forward_offline")
    return n_out.value


def sortformer_state_bytes(h, scfg, batch) -> int:
    return load().sortformer_state_bytes(h, C.byref(scfg), batch)


def sortformer_stream_workspace_bytes(h, scfg, batch) -> int:
    return load().sortformer_stream_workspace_bytes(h, C.byref(scfg), batch)


def sortformer_stream_create(h, scfg, batch, d_state, stream=None):
    st = C.c_void_p()
    cfg = sf_model_config()
    _check(load().sortformer_get_config(h, C.byref(cfg)), "get_config")
    _check(load().sortformer_stream_create(h, C.byref(scfg), batch, *_buf(d_state),
                                           _stream(stream), C.byref(st)),
           "stream_create")
    _STREAMS[st.value] = (batch, cfg.n_spk)
    return st


def sortformer_stream_destroy(st):
    load().sortformer_stream_destroy(st)
    _STREAMS.pop(getattr(st, "value", st), None)


def sortformer_stream_set_option(st, option, value):
    _check(load().sortformer_stream_set_option(st, option, int(value)), "stream_set_option")


def sortformer_stream_reset(st, stream=None):
    _check(load().sortformer_stream_reset(st, _stream(stream)), "stream_reset")


def sortformer_stream_samples_needed(st) -> int:
    return load().sortformer_stream_samples_needed(st)


def sortformer_stream_max_emit(st) -> int:
    return load().sortformer_stream_max_emit(st)


def sortformer_stream_step(st, d_audio_new, n_new, is_last, d_probs_out, d_ws, stream=None) -> int:
    n = C.c_int32()
    B, S = _STREAMS[st.value]
    _check(load().sortformer_stream_step(st, _ptr(d_audio_new, B * n_new), n_new, int(is_last),
                                         _ptr(d_probs_out, B * sortformer_stream_max_emit(st) * S),
                                         C.byref(n), *_buf(d_ws),
                                         _stream(stream)), "stream_step")
    return n.value


def sortformer_stream_step_noalloc(st, d_audio_new, n_new, is_last, d_probs_out, stream=None) -> int:
    """sortformer_stream_step with the library's static scratch as workspace."""
    n = C.c_int32()
    B, S = _STREAMS[st.value]
    _check(load().sortformer_stream_step_noalloc(
        st, _ptr(d_audio_new, B * n_new), n_new, int(is_last),
        _ptr(d_probs_out, B * sortformer_stream_max_emit(st) * S), C.byref(n), _stream(stream)),
        "stream_step_noalloc")
    return n.value


def sortformer_stream_feed_frames(st, n_new, is_last=False) -> int:
    return load().sortformer_stream_feed_frames(st, n_new, int(is_last))


def sortformer_stream_feed(st, d_audio_new, is_last, d_probs_out, d_ws, stream=None) -> int:
    """Feed d_audio_new (B, n) (any n) -> frames per stream written to d_probs_out
    (B, out_frames, S), row 0 onwards."""
    B, S = _STREAMS[st.value]
    n_new = d_audio_new.shape[1]
    out_frames = d_probs_out.shape[1]
    n = C.c_int64()
    _check(load().sortformer_stream_feed(st, _ptr(d_audio_new, B * n_new), n_new, int(is_last),
                                         _ptr(d_probs_out, B * out_frames * S), out_frames,
                                         C.byref(n), *_buf(d_ws), _stream(stream)), "stream_feed")
    return n.value


def sortformer_stream_get_info(st):
    info = (C.c_int64 * 9)()
    ptrs = (C.c_void_p * 6)()
    _check(load().sortformer_stream_get_info(st, info, ptrs), "stream_get_info")
    keys = ["cache_len", "fifo_len", "lookahead_len", "capacity", "steps", "frames_emitted",
            "samples_received", "finished", "pending"]
    return dict(zip(keys, list(info))), [p or 0 for p in ptrs]


def _np(a):
    return None if a is None else a.ctypes.data_as(C.c_void_p)


def sortformer_stream_checkpoint_bytes(st) -> int:
    return load().sortformer_stream_checkpoint_bytes(st)


def sortformer_stream_export(st, stream=None):
    """-> the whole streaming state as a host byte array (numpy uint8)."""
    import numpy as np
    blob = np.zeros(sortformer_stream_checkpoint_bytes(st), np.uint8)
    _check(load().sortformer_stream_export(st, _np(blob), blob.nbytes, _stream(stream)),
           "stream_export")
    return blob


def sortformer_stream_import(st, blob, stream=None):
    import numpy as np
    blob = np.ascontiguousarray(blob, np.uint8)
    _check(load().sortformer_stream_import(st, _np(blob), blob.nbytes, _stream(stream)),
           "stream_import")


def sortformer_stream_get_rows(st, n_spk, stream=None):
    """-> dict of host arrays (emb, probs, flags, sil_sum, sil_cnt) and lengths."""
    import numpy as np
    info, ptrs = sortformer_stream_get_info(st)
    rows = info["cache_len"] + info["fifo_len"] + info["lookahead_len"]
    D = int(ptrs[5])
    B = _stream_batch(st)
    out = dict(emb=np.empty((B, rows, D), np.float32), probs=np.empty((B, rows, n_spk), np.float32),
               flags=np.empty((B, rows), np.int32), sil_sum=np.empty((B, D), np.float64),
               sil_cnt=np.empty(B, np.int32))
    _check(load().sortformer_stream_get_rows(st, _np(out["emb"]), _np(out["probs"]),
                                             _np(out["flags"]), _np(out["sil_sum"]),
                                             _np(out["sil_cnt"]), _stream(stream)), "stream_get_rows")
    out.update(info)
    return out


def sortformer_stream_set_rows(st, cache_len, fifo_len, lookahead_len, emb, probs, flags, sil_sum,
                               sil_cnt, stream=None):
    import numpy as np
    arrs = [np.ascontiguousarray(emb, np.float32), np.ascontiguousarray(probs, np.float32),
            np.ascontiguousarray(flags, np.int32), np.ascontiguousarray(sil_sum, np.float64),
            np.ascontiguousarray(sil_cnt, np.int32)]
    _check(load().sortformer_stream_set_rows(st, cache_len, fifo_len, lookahead_len,
                                             *[_np(a) for a in arrs], _stream(stream)),
           "stream_set_rows")


_STREAMS = {}  # stream handle -> (batch, speakers)


def _stream_batch(st):
    return _STREAMS[st.value][0]


def sortformer_stream_update(st, d_window_probs, n_chunk, d_ws, stream=None):
    _check(load().sortformer_stream_update(st, _ptr(d_window_probs), n_chunk, *_buf(d_ws),
                                           _stream(stream)), "stream_update")


def sortformer_encode_workspace_bytes(h, batch, window) -> int:
    return load().sortformer_encode_workspace_bytes(h, batch, window)


def sortformer_encode_window(h, d_emb, n_valid, d_probs, d_probs10, d_ws, stream=None):
    B, W, D = d_emb.shape
    cfg = sf_model_config()
    _check(load().sortformer_get_config(h, C.byref(cfg)), "get_config")
    if D != 512:
        raise ValueError("embeddings must have 512 features")
    _check(load().sortformer_encode_window(h, _ptr(d_emb), B, W, n_valid,
                                           _ptr(d_probs, B * W * cfg.n_spk),
                                           _ptr(d_probs10, 8 * B * W * cfg.n_spk),
                                           *_buf(d_ws), _stream(stream)), "encode_window")


def sortformer_debug_tap(h, layer, point, d_out):
    """Register (d_out a float32 GPU tensor) or remove (d_out None) a tap;
    layer -1 with d_out None removes every tap."""
    n = 0 if d_out is None else d_out.numel()
    _check(load().sortformer_debug_tap(h, layer, point, _ptr(d_out), n), "debug_tap")


def sortformer_pre_encode_workspace_bytes(h, batch, n_samples) -> int:
    return load().sortformer_pre_encode_workspace_bytes(h, batch, n_samples)


def sortformer_pre_encode(h, d_audio, d_mel, d_emb, d_ws, stream=None):
    B, N = d_audio.shape
    T = N // 160
    _check(load().sortformer_pre_encode(h, _ptr(d_audio), B, N, _ptr(d_mel, B * T * 128),
                                        _ptr(d_emb, B * ((T + 7) // 8) * 512), *_buf(d_ws),
                                        _stream(stream)), "pre_encode")


def sortformer_profile_begin(kind: str, max_launches: int = 20000):
    _check(load().sortformer_profile_begin(SF_PROF[kind], max_launches), "profile_begin")


def sortformer_profile_end():
    ms, fl, by = C.c_double(), C.c_double(), C.c_double()
    n = C.c_int64()
    _check(load().sortformer_profile_end(C.byref(ms), C.byref(n), C.byref(fl), C.byref(by)),
           "profile_end")
    return dict(ms=ms.value, launches=n.value, flops=fl.value, bytes=by.value)


def sortformer_segment_defaults() -> sf_segment_params:
    p = sf_segment_params()
    load().sortformer_segment_defaults(C.byref(p))
    return p


def sortformer_segments_capacity(n_frames) -> int:
    return load().sortformer_segments_capacity(n_frames)


def sortformer_segments(d_probs, frame_s, params, d_out, capacity, d_counts, stream=None):
    """d_probs (B, T, S) float32 device tensor; d_out a device byte buffer of
    B*S*capacity segments (SEGMENT_BYTES each); d_counts int64 (B*S,)."""
    import torch
    B, T, S = d_probs.shape
    out_ptr, out_bytes = _buf(d_out)
    if out_bytes < B * S * capacity * SEGMENT_BYTES:
        raise ValueError("segment buffer smaller than batch x speakers x capacity")
    if not (d_counts.is_cuda and d_counts.dtype == torch.int64 and d_counts.is_contiguous()
            and d_counts.numel() >= B * S):
        raise TypeError("counts must be a contiguous int64 device tensor of batch x speakers")
    _check(load().sortformer_segments(_ptr(d_probs), B, T, S, frame_s,
                                      None if params is None else C.byref(params), out_ptr,
                                      capacity, C.c_void_p(d_counts.data_ptr()), _stream(stream)),
           "segments")
