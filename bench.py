"""Benchmark of the streaming diarization forward on one MI355X.

One benchmark step = one pass of the whole hot path over one synthetic
workload: for the default workload (Streaming Sortformer, 'low' preset,
60 s of 4-speaker meeting-like audio, bf16) that is the live stream of 124
steps, each running the log-mel frontend and pre_encode on the new audio,
the encoder over [cache | FIFO | chunk | look-ahead], the head, the FIFO
update and (when the cache overflows) the compression.

value = RTFx = audio seconds processed / wall seconds, with the audio already
resident in device memory. The JSON line also carries the dominant kernel
class's roofline figures (algorithmic FLOPs per launch over its average
launch time, measured with HIP events on the launch stream in a separate
profiled pass) and the CPU oracle timed on a bounded sample.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK = {"bf16_tflops": 2516.6, "f32_tflops": 157.3, "hbm_gbs": 8000.0}
METRIC = "RTFx (audio s / wall s) of Sortformer forward bf16; % of MFMA bf16 peak"

WORKLOADS = {
    "low60s": dict(arch="sortformer", dtype="bf16", mode="stream", preset="low", batch=1,
                   desc="Streaming Sortformer 4-spk, 'low' preset 6/7/188/144/188, 60 s, B=1"),
    "veryhigh600s": dict(arch="sortformer", dtype="bf16", mode="stream", preset="very_high",
                         batch=1, desc="Streaming Sortformer, 'very high' 340/40/40/300/188, 600 s"),
    "ultralow64x120s": dict(arch="sortformer", dtype="bf16", mode="stream", preset="ultra_low",
                            batch=64, desc="64 lockstep streams, 'ultra low' 3/1/188/144/188, 120 s"),
    "offline8s": dict(arch="sortformer", dtype="f32", mode="offline", batch=1,
                      desc="offline Sortformer, 8 s clip, fp32"),
    "nemotron1800s": dict(arch="nemotron", dtype="bf16", mode="offline", batch=1,
                          desc="Nemotron-3-style, 30 min, 30.4 s chunks, AOSC 188 + FIFO 188"),
}


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=5)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--workload", default="low60s", choices=sorted(WORKLOADS))
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU-oracle baselines")
    ap.add_argument("--no-cpu-1thread", action="store_true",
                    help="skip the single-thread CPU-oracle baseline")
    ap.add_argument("--no-profile", action="store_true", help="skip the profiled pass")
    ap.add_argument("--no-graphs", action="store_true",
                    help="launch the stream window forward kernel by kernel (no HIP graphs)")
    ap.add_argument("--window-probe", type=int, default=0, metavar="W",
                    help="only run the encoder over one steady-state window of W frames of the "
                         "workload's model twice (a short program for counter collection) and exit")
    ap.add_argument("--copy-probe", type=int, default=0, metavar="MIB",
                    help="only run a plain device-to-device copy of MIB MiB three times (the "
                         "calibration kernel for the HBM byte counters) and exit")
    return ap.parse_args()


# HBM traffic of the dominant kernel class from the FETCH_SIZE / WRITE_SIZE
# counter runs, stored beside the rocprofv3 summaries together with a hash of
# the kernel sources it was measured on; reported only while they match.
PMC_FILE = os.path.join(ROOT, "profiles", "gemm_low60s_pmc.txt")
PMC_SOURCES = ["gemm.hip", "tftail.hip", "kernels.h", "common.h"]


def kernel_source_hash():
    import hashlib
    h = hashlib.sha256()
    for f in PMC_SOURCES:
        with open(os.path.join(ROOT, "streaming_speaker_diarization_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic(workload, kernel):
    """HBM bytes per launch (calibrated FETCH_SIZE + WRITE_SIZE), or None."""
    try:
        kv = dict(line.split(":", 1) for line in open(PMC_FILE) if ":" in line)
    except OSError:
        return None
    kv = {k.strip(): v.strip() for k, v in kv.items()}
    if (kv.get("workload") != workload or kv.get("kernel_class") != kernel
            or kv.get("kernel_sources_sha256") != kernel_source_hash()):
        return None
    return float(kv["hbm_bytes_per_launch"])


def window_probe(name, wl, W):
    import torch
    from streaming_speaker_diarization_amd import runtime
    m = runtime.Model(wl["arch"], wl["dtype"])
    g = torch.Generator().manual_seed(W)
    emb = torch.randn(wl["batch"], W, 512, generator=g).cuda()
    for _ in range(2):
        m.encode_window(emb)
    torch.cuda.synchronize()
    print(json.dumps({"window_probe": name, "frames": W, "passes": 2}), flush=True)


def copy_probe(mib):
    import torch
    n = mib * (1 << 20) // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_probe_bytes_per_copy": n * 4, "copies": 3}), flush=True)


def load_audio(name, wl):
    import numpy as np
    from synthetic import workload_audio
    if wl["batch"] == 1:
        return workload_audio(name)[None]
    return np.stack([workload_audio(name, stream=b) for b in range(wl["batch"])])


class Runner:
    """One pass of a workload through the library (no arithmetic here)."""

    def __init__(self, name, wl, audio_gpu):
        import torch
        from streaming_speaker_diarization_amd import runtime
        from streaming_speaker_diarization_amd import sortformer as sf
        self.sf, self.torch = sf, torch
        self.wl = wl
        self.model = runtime.Model(wl["arch"], wl["dtype"])
        self.audio = audio_gpu
        B, N = audio_gpu.shape
        self.B, self.N = B, N
        te = (N // 160 + 7) // 8
        S = self.model.n_spk
        if wl["mode"] == "stream":
            self.stream = self.model.stream(wl["preset"], batch=B)
            # slack of one step's maximum emission: a step may be handed the
            # tail of this buffer directly (B == 1)
            max_emit = sf.sortformer_stream_max_emit(self.stream.handle)
            self.out = torch.empty(B, te + max_emit, S, dtype=torch.float32, device="cuda")
        else:
            self.ws = self.model.workspace(
                sf.sortformer_offline_workspace_bytes(self.model.handle, B, N))
            n_out = te if wl["arch"] == "sortformer" else 8 * te
            self.out = torch.empty(B, n_out, S, dtype=torch.float32, device="cuda")

    def chunks(self):
        """The live schedule's audio pieces as contiguous (B, k) device tensors,
        prepared once outside the timed region (a column slice of a batch is
        strided). For B == 1 the slices are views."""
        if getattr(self, "_chunks", None) is None:
            sf, st = self.sf, self.stream
            st.reset()
            plan, pos, N = [], 0, self.N
            while True:
                need = sf.sortformer_stream_samples_needed(st.handle)
                last = pos + need > N
                k = N - pos if last else need
                plan.append((pos, k, last))
                sf.sortformer_stream_step(st.handle, self.audio[:, pos:pos + k].contiguous(), k,
                                          last, st.out, st.ws)
                pos += k
                if last:
                    break
            self._chunks = [(self.audio[:, p:p + k] if self.B == 1 else
                             self.audio[:, p:p + k].contiguous(), k, last) for p, k, last in plan]
        return self._chunks

    def step_latency(self):
        """Device time of each stream step of one pass (events on the launch
        stream between steps): p50 / p95 / max in ms, or None offline."""
        import numpy as np
        import torch
        if self.wl["mode"] != "stream":
            return None
        sf = self.sf
        steps = self.chunks()
        st = self.stream
        st.reset()
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(len(steps) + 1)]
        e0 = 0
        ev[0].record()
        for i, (piece, k, last) in enumerate(steps):
            buf = self.out[:, e0:] if self.B == 1 else st.out
            e0 += sf.sortformer_stream_step(st.handle, piece, k, last, buf, st.ws)
            ev[i + 1].record()
        torch.cuda.synchronize()
        t = np.array([ev[i].elapsed_time(ev[i + 1]) for i in range(len(steps))])
        return {"p50": round(float(np.percentile(t, 50)), 4), "p95": round(float(np.percentile(t, 95)), 4),
                "max": round(float(t.max()), 4), "steps": len(steps)}

    def one_pass(self):
        sf = self.sf
        if self.wl["mode"] == "offline":
            sf.sortformer_forward_offline(self.model.handle, self.audio, self.out, self.ws)
            return
        steps = self.chunks()
        st = self.stream
        st.reset()
        e0 = 0
        h = st.handle
        for piece, k, last in steps:
            buf = self.out[:, e0:] if self.B == 1 else st.out
            n = sf.sortformer_stream_step(h, piece, k, last, buf, st.ws)
            if self.B > 1 and n:
                S = self.out.shape[2]
                self.out[:, e0:e0 + n].copy_(st.out.view(-1)[:self.B * n * S].view(self.B, n, S))
            e0 += n


def cpu_baseline(name, wl, audio_np, one_thread=False):
    """The oracle as it stands on a bounded sample of the same workload (BLAS
    on every host core, or on one)."""
    if one_thread:
        from threadpoolctl import threadpool_limits
        with threadpool_limits(limits=1):
            return cpu_baseline(name, wl, audio_np)
    import numpy as np
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # threadpoolctl absent: report the affinity size
        threads = len(os.sched_getaffinity(0))
    from oracle import frontend, run, streaming
    from oracle.weights import make_weights
    if not (wl["mode"] == "stream" and wl["arch"] == "sortformer"):
        return None
    w = make_weights("sortformer", 0, bf16=(wl["dtype"] == "bf16"))
    cfg = streaming.StreamConfig.preset(wl["preset"])
    audio = audio_np[0]
    t0 = time.perf_counter()
    emb = run.pre_encode_all(w, frontend.log_mel(audio))
    t_pre = time.perf_counter() - t0
    sched = streaming.live_schedule(len(audio), cfg)
    # steady state: start from a full cache/FIFO built from earlier frames
    k0 = max(0, len(sched) - 12)
    c0 = sched[k0][0]
    Lc = min(cfg.spkcache_len, max(0, c0 - cfg.fifo_len))
    Lf = min(cfg.fifo_len - 2, c0 - Lc)
    rng = np.random.default_rng(0)
    st = streaming.State(emb[c0 - Lf - Lc:c0 - Lf].copy(), rng.random((Lc, 4)), np.zeros(Lc, bool),
                         emb[c0 - Lf:c0].copy(), rng.random((Lf, 4)), np.zeros(512), 0)
    n_steps = min(8, len(sched) - k0)
    enc = run.sortformer_encoder(w)
    t0 = time.perf_counter()
    for c0_, n, rc, last in sched[k0:k0 + n_steps]:
        streaming.stream_step(st, emb[c0_:c0_ + n + rc], n, cfg, enc, 4)
    t_step = (time.perf_counter() - t0) / n_steps
    audio_s = len(audio) / 16000.0
    total = t_pre + len(sched) * t_step
    return {"value": audio_s / total, "unit": "x realtime (audio s / wall s)", "cores": threads,
            "kind": "oracle",
            "sample": (f"oracle frontend+pre_encode of the whole {audio_s:.0f} s clip ({t_pre:.2f} s) "
                       f"plus {n_steps} steady-state stream steps (W~{Lc + Lf + cfg.chunk_len + cfg.right_context}, "
                       f"{t_step:.2f} s/step) extrapolated to the {len(sched)} steps of one pass")}


def main():
    args = parse()
    if args.copy_probe:
        copy_probe(args.copy_probe)
        return
    if args.window_probe:
        window_probe(args.workload, WORKLOADS[args.workload], args.window_probe)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(streams shard across GPUs with no per-step exchange; see the design notes).")
        sys.exit(2)
    import numpy as np
    import torch
    wl = WORKLOADS[args.workload]
    audio_np = load_audio(args.workload, wl)
    audio = torch.from_numpy(audio_np.astype(np.float32)).cuda().contiguous()
    r = Runner(args.workload, wl, audio)
    if args.no_graphs and wl["mode"] == "stream":
        r.sf.sortformer_stream_set_option(r.stream.handle, r.sf.SF_STREAM_OPT_GRAPHS, 0)
    if wl["mode"] == "stream":
        r.chunks()  # the schedule's audio pieces, before any timing
    for _ in range(args.warmup):
        r.one_pass()
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    ev0.record()
    for _ in range(args.steps):
        r.one_pass()
    ev1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    gpu_ms = ev0.elapsed_time(ev1)
    ms_per_step = 1e3 * wall / args.steps
    audio_s = audio_np.shape[0] * audio_np.shape[1] / 16000.0
    value = audio_s / (ms_per_step / 1e3)

    lat = r.step_latency()
    prof = {}
    if not args.no_profile:
        sf = r.sf
        for kind in ("gemm", "attn", "ln", "conv", "frontend", "cache"):
            sf.sortformer_profile_begin(kind, 200000)
            r.one_pass()
            prof[kind] = sf.sortformer_profile_end()
        torch.cuda.synchronize()
    roof = None
    total_flops = sum(p["flops"] for p in prof.values())
    if prof:
        dom = max(prof, key=lambda k: prof[k]["ms"])
        p = prof[dom]
        avg_ms = p["ms"] / max(p["launches"], 1)
        mfma = dom in ("gemm", "attn")
        peak = PEAK["bf16_tflops"] if wl["dtype"] == "bf16" else PEAK["f32_tflops"]
        if mfma:
            ach = p["flops"] / max(p["launches"], 1) / (avg_ms / 1e3) / 1e12
            roof = {"bound": "mfma", "kernel": dom, "achieved": round(ach, 3), "peak": peak,
                    "unit": "TFLOP/s", "frac": round(ach / peak, 5),
                    "traffic": measured_traffic(args.workload, dom),
                    "launches": p["launches"], "avg_launch_us": round(1e3 * avg_ms, 3),
                    "share_of_pass": round(p["ms"] / ms_per_step, 4)}
        else:
            ach = p["bytes"] / max(p["launches"], 1) / (avg_ms / 1e3) / 1e9
            roof = {"bound": "hbm", "kernel": dom, "achieved": round(ach, 2),
                    "peak": PEAK["hbm_gbs"], "unit": "GB/s", "frac": round(ach / PEAK["hbm_gbs"], 5),
                    "traffic": measured_traffic(args.workload, dom), "launches": p["launches"], "avg_launch_us": round(1e3 * avg_ms, 3)}
    line = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "x realtime (audio s / wall s)",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 3),
        "gpu_ms_per_step": round(gpu_ms / args.steps, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": wl["dtype"],
        "data": "synthetic",
        "config": {"workload": f"{args.workload}: {wl['desc']}", "batch_streams": wl["batch"],
                   "audio_s_per_step": audio_s},
        "tflops_whole_pass": round(total_flops / (ms_per_step / 1e3) / 1e12, 3) if prof else None,
        "pct_bf16_peak_whole_pass": round(100 * total_flops / (ms_per_step / 1e3) / 1e12 /
                                          PEAK["bf16_tflops"], 4) if prof else None,
        "kernel_classes": {k: {"ms": round(v["ms"], 3), "launches": v["launches"],
                               "tflops": round(v["flops"] / max(v["ms"], 1e-9) / 1e9, 3),
                               "gbs": round(v["bytes"] / max(v["ms"], 1e-9) / 1e6, 1)}
                           for k, v in prof.items()},
        "roofline": roof,
        "step_latency_ms": lat,
        "cpu_baseline": None if args.no_cpu else cpu_baseline(args.workload, wl, audio_np),
        "cpu_baseline_1thread": (None if args.no_cpu or args.no_cpu_1thread else
                                 cpu_baseline(args.workload, wl, audio_np, one_thread=True)),
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
