"""MI355X (gfx950) Streaming Sortformer / Nemotron-3-style diarization forward.

The compute path lives in ``libsortformer.so`` (hand-written HIP kernels
behind the C ABI of ``include/sortformer.h``); ``sortformer`` is its ctypes
binding and ``runtime`` a small helper that allocates the library's buffers
with PyTorch.
"""
from . import sortformer  # noqa: F401
