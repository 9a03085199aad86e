"""Host-side checks of the C ABI (no GPU): the library loads, exports every
symbol the header declares, validates configurations, and its host weight
generator reproduces the oracle's weights."""
import os
import re

import numpy as np
import pytest

from oracle import weights as OW
from oracle.streaming import PRESETS

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def sf():
    from streaming_speaker_diarization_amd import sortformer
    if not os.path.exists(sortformer.LIB_PATH):
        import __graft_entry__
        __graft_entry__.build()
    sortformer.load()
    return sortformer


def _header_functions():
    src = open(os.path.join(ROOT, "include", "sortformer.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(sortformer_\w+)\s*\(", src)))


def test_exports_every_declared_symbol(sf):
    lib = sf.load()
    names = _header_functions()
    assert len(names) >= 25
    for n in names:
        assert hasattr(lib, n), n
    assert sorted(sf.EXPORTS) == names


def test_status_strings_and_presets(sf):
    assert sf.status_string(0) == "ok"
    assert "invalid" in sf.status_string(-1)
    for name, vals in PRESETS.items():
        c = sf.sortformer_stream_preset(name)
        assert (c.chunk_len, c.right_context, c.fifo_len, c.update_period, c.spkcache_len) == vals
        assert c.n_sil_per_spk == 3
    with pytest.raises(sf.SortformerError):
        sf.sortformer_stream_preset("nope")


def test_config_validation(sf):
    assert sf.sortformer_weight_bytes(sf.model_config("sortformer", "bf16")) > 200e6
    assert sf.sortformer_weight_bytes(sf.model_config("sortformer", "f32")) > 450e6
    assert sf.sortformer_weight_bytes(sf.model_config("nemotron", "bf16")) > 190e6
    bad = sf.model_config("sortformer", "bf16")
    bad.n_spk = 8
    assert sf.sortformer_weight_bytes(bad) == 0
    bad = sf.model_config("sortformer", "bf16")
    bad.dtype = 7
    assert sf.sortformer_weight_bytes(bad) == 0


@pytest.mark.parametrize("arch", ["sortformer", "nemotron"])
def test_tensor_list_matches_oracle(sf, arch):
    cfg = sf.model_config(arch, "f32")
    tl = OW.sortformer_tensors() if arch == "sortformer" else OW.nemotron_tensors()
    assert sf.sortformer_config_num_tensors(cfg) == len(tl)
    for i, (name, shape, _) in enumerate(tl):
        got = sf.sortformer_config_tensor(cfg, 0, i, values=False)
        assert got == (name, int(np.prod(shape)))


@pytest.mark.parametrize("arch,full", [("sortformer", False), ("sortformer", True),
                                       ("nemotron", False)])
def test_weight_generator_matches_oracle(sf, arch, full):
    """The library's host generator and the oracle's are independent
    implementations of the same published generator; compare every element of
    a sample of tensors (large and small, every kind)."""
    seed = 5 if arch == "sortformer" else 1
    cfg = sf.model_config(arch, "f32", full)
    tl = OW.sortformer_tensors() if arch == "sortformer" else OW.nemotron_tensors()
    ref = OW.make_weights(arch, seed, full_random=full)
    idx = [0, 1, 7, 12, 13, 30, 41, len(tl) - 1, len(tl) - 3]
    mism = 0
    total = 0
    for i in idx:
        name, vals = sf.sortformer_config_tensor(cfg, seed, i)
        r = ref[name].astype(np.float32).ravel()
        mism += int(np.sum(vals != r))
        total += r.size
        assert np.max(np.abs(vals - r)) <= 1e-9 + 2 ** -22 * np.max(np.abs(r))
    # libm differences may flip a rare last-bit rounding; none are expected
    assert mism <= total * 1e-6, (mism, total)


def test_no_cpu_fallback_in_product_path():
    """The binding refuses to run without the HIP library and never imports
    the oracle."""
    pkg = os.path.join(ROOT, "streaming_speaker_diarization_amd")
    for f in os.listdir(pkg):
        if f.endswith(".py"):
            txt = open(os.path.join(pkg, f)).read()
            assert "import oracle" not in txt and "from oracle" not in txt, f


def test_binding_rejects_host_strided_or_mistyped_tensors():
    import torch
    from streaming_speaker_diarization_amd import sortformer
    with pytest.raises(TypeError):
        sortformer._ptr(torch.zeros(4, dtype=torch.float32))  # host memory
    with pytest.raises(TypeError):
        sortformer._buf(torch.zeros(4, dtype=torch.uint8))
    assert sortformer._ptr(None) is None


def test_segment_defaults_and_capacity(sf):
    p = sf.sortformer_segment_defaults()
    assert (p.onset, p.offset, p.pad_onset, p.pad_offset, p.min_duration_on,
            p.min_duration_off) == (0.5, 0.5, 0.0, 0.0, 0.0, 0.0)
    assert [sf.sortformer_segments_capacity(t) for t in (0, 1, 2, 3, 64, 65)] == [0, 1, 1, 2, 32, 33]
    assert sf.SEGMENT_BYTES == 24
