"""Write the oracle's outputs for the full-size streaming workloads.

Calls only the oracle (and the shared synthetic-input generator); the GPU
path never writes these files. Run from the repository root:
    python tests/golden/make_golden.py [name ...]
Outputs float32 .npy files next to this script.
"""
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

from oracle import run, streaming  # noqa: E402
from oracle.weights import make_weights  # noqa: E402
from synthetic import workload_audio  # noqa: E402

HERE = os.path.dirname(os.path.abspath(__file__))


def low60s():
    w = make_weights("sortformer", 0, bf16=True)
    p, _ = run.sortformer_stream(workload_audio("low60s"), w, streaming.StreamConfig.preset("low"))
    return p


def veryhigh600s():
    w = make_weights("sortformer", 0, bf16=True)
    p, _ = run.sortformer_stream(workload_audio("veryhigh600s"), w,
                                 streaming.StreamConfig.preset("very_high"))
    return p


def nemotron1800s():
    w = make_weights("nemotron", 1, bf16=True)
    p, _ = run.nemotron_offline(workload_audio("nemotron1800s"), w)
    return p


JOBS = {"low60s_bf16": low60s, "veryhigh600s_bf16": veryhigh600s,
        "nemotron1800s_bf16": nemotron1800s}

if __name__ == "__main__":
    names = sys.argv[1:] or list(JOBS)
    for n in names:
        t = time.time()
        p = JOBS[n]().astype(np.float32)
        np.save(os.path.join(HERE, n + ".npy"), p)
        print(f"{n}: {p.shape} in {time.time() - t:.1f} s", flush=True)
