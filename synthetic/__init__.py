"""Seeded synthetic inputs shared by the oracle and the HIP path.

This package only draws inputs (audio, probability tables, embeddings). It
holds none of the diarization method's arithmetic, so both sides can use it
without sharing any computation.
"""
from .audio import meeting_audio, workload_audio, WORKLOADS  # noqa: F401
from .tables import random_probs, random_embeddings  # noqa: F401
