"""Benchmark of the streaming diarization forward on one MI355X.

One benchmark step = one pass of the whole hot path over one synthetic
workload. For the default workload (64 independent streams of 120 s of
4-speaker meeting-like audio, Streaming Sortformer 'ultra low' preset
3/1/188/144/188, bf16, the streams in lockstep) that is the live stream of
500 steps, each running, for all 64 streams at once, the log-mel frontend
and pre_encode on the new audio, the encoder over [cache | FIFO | chunk |
look-ahead] (64 windows of up to 378 frames), the head, the FIFO update and
(when the cache overflows) the compression.

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
    ap.add_argument("--workload", default="ultralow64x120s", choices=sorted(WORKLOADS))
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU-oracle baselines")
    ap.add_argument("--cpu-1thread", action="store_true",
                    help="also time the CPU oracle with one BLAS thread")
    ap.add_argument("--no-profile", action="store_true", help="skip the profiled pass")
    ap.add_argument("--no-graphs", action="store_true",
                    help="launch the stream window forward kernel by kernel (no HIP graphs)")
    ap.add_argument("--fixed-window", action="store_true",
                    help="pad every stream window to the preset's capacity (one graph per stream)")
    ap.add_argument("--window-probe", type=int, default=0, metavar="W",
                    help="only run the encoder over one steady-state window of W frames of the "
                         "workload's model twice (a short program for counter collection) and exit")
    ap.add_argument("--copy-probe", type=int, default=0, metavar="MIB",
                    help="only run a plain device-to-device copy of MIB MiB three times (the "
                         "calibration kernel for the HBM byte counters) and exit")
    ap.add_argument("--pmc-summary", nargs=3, metavar=("FETCH_DIR", "WRITE_DIR", "COPY_DIR"),
                    help="write the GEMM-class HBM-traffic summary of the workload from "
                         "rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE runs of --window-probe and "
                         "of --copy-probe (COPY_DIR holds copy_fetch/ and copy_write/) and exit")
    return ap.parse_args()


def progress(msg):
    """Progress of the run on stderr (the JSON line stays alone on stdout)."""
    print(f"[bench {time.strftime('%H:%M:%S')}] {msg}", file=sys.stderr, flush=True)


# HBM traffic of the dominant kernel class from the FETCH_SIZE / WRITE_SIZE
# counter runs, stored beside the rocprofv3 summaries together with a hash of
# the kernel sources it was measured on; reported only while they match.
def pmc_file(workload):
    return os.path.join(ROOT, "profiles", f"gemm_{workload}_pmc.txt")


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
        kv = dict(line.split(":", 1) for line in open(pmc_file(workload)) if ":" in line)
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
            n_out = te if wl["arch"] == "sortformer" else 8 * te
            self.out = torch.empty(B, n_out, S, dtype=torch.float32, device="cuda")
        else:
            self.ws = self.model.workspace(
                sf.sortformer_offline_workspace_bytes(self.model.handle, B, N))
            n_out = te if wl["arch"] == "sortformer" else 8 * te
            self.out = torch.empty(B, n_out, S, dtype=torch.float32, device="cuda")

    def steps(self):
        """The live schedule's audio pieces (start, count, is_last): the first
        step needs 1280 * (chunk + look-ahead) + 40 samples, later ones 1280 *
        chunk; the clip's end goes into the final step."""
        c = self.stream.scfg
        plan, pos = [], 0
        while True:
            need = 1280 * (c.chunk_len + c.right_context) + 40 if not plan else 1280 * c.chunk_len
            if pos + need > self.N:
                plan.append((pos, self.N - pos, True))
                return plan
            plan.append((pos, need, False))
            pos += need

    def step_latency(self):
        """Device time of each stream step of one pass (events on the launch
        stream between steps): p50 / p95 / max in ms, or None offline."""
        import numpy as np
        import torch
        if self.wl["mode"] != "stream":
            return None
        sf, st = self.sf, self.stream
        plan = self.steps()
        pieces = [self.audio[:, p:p + k].contiguous() for p, k, _ in plan]
        st.reset()
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(len(plan) + 1)]
        ev[0].record()
        for i, (piece, (_, k, last)) in enumerate(zip(pieces, plan)):
            sf.sortformer_stream_step(st.handle, piece, k, last, st.out, st.ws)
            ev[i + 1].record()
        torch.cuda.synchronize()
        t = np.array([ev[i].elapsed_time(ev[i + 1]) for i in range(len(plan))])
        return {"p50": round(float(np.percentile(t, 50)), 4), "p95": round(float(np.percentile(t, 95)), 4),
                "max": round(float(t.max()), 4), "steps": len(plan)}

    def one_pass(self):
        """The whole clip of every stream fed at once: the library runs the
        live schedule's steps back to back, writing each step's emitted
        frames into the output in order."""
        sf = self.sf
        if self.wl["mode"] == "offline":
            sf.sortformer_forward_offline(self.model.handle, self.audio, self.out, self.ws)
            return
        st = self.stream
        st.reset()
        n = sf.sortformer_stream_feed(st.handle, self.audio, True, self.out, st.ws)
        assert n == self.out.shape[1]


def cpu_baseline(name, wl, audio_np, one_thread=False):
    """The oracle as it stands on a bounded sample of the same workload (BLAS
    on every host core, or on one): frontend + pre_encode of one stream's clip
    and a few steady-state stream steps, extrapolated to every step of every
    stream of one pass."""
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
    B = audio_np.shape[0]
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
    n_steps = min(8 if B == 1 else 4, len(sched) - k0)
    enc = run.sortformer_encoder(w)
    t0 = time.perf_counter()
    for c0_, n, rc, last in sched[k0:k0 + n_steps]:
        streaming.stream_step(st, emb[c0_:c0_ + n + rc], n, cfg, enc, 4)
    t_step = (time.perf_counter() - t0) / n_steps
    audio_s = B * len(audio) / 16000.0
    total = B * (t_pre + len(sched) * t_step)
    per = "" if B == 1 else f" per stream, times {B} streams"
    return {"value": audio_s / total, "unit": "x realtime (audio s / wall s)", "cores": threads,
            "kind": "oracle",
            "sample": (f"oracle frontend+pre_encode of one {len(audio) / 16000:.0f} s clip "
                       f"({t_pre:.2f} s) plus {n_steps} steady-state stream steps (W~"
                       f"{Lc + Lf + cfg.chunk_len + cfg.right_context}, {t_step:.2f} s/step), "
                       f"extrapolated to the {len(sched)} steps of one pass{per}")}


def pmc_summary(name, fetch_dir, write_dir, copy_dir):
    """GEMM-class HBM traffic per launch from rocprofv3 --pmc counter CSVs of
    the window probe, calibrated by the same counters on a plain copy of
    known size. Writes the summary that measured_traffic() reads."""
    import csv
    import glob

    def rows(d, counter):
        out = []
        for f in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
            for r in csv.DictReader(open(f)):
                if r.get("Counter_Name") == counter:
                    out.append((r["Kernel_Name"], float(r["Counter_Value"])))
        return out

    def per_kernel(d, counter):
        acc = {}
        for k, v in rows(d, counter):
            n, t = acc.get(k, (0, 0.0))
            acc[k] = (n + 1, t + v)
        return acc

    cf = per_kernel(os.path.join(copy_dir, "copy_fetch"), "FETCH_SIZE")
    cw = per_kernel(os.path.join(copy_dir, "copy_write"), "WRITE_SIZE")
    copy_kib = 1024 * 1024  # the 1 GiB copy probe
    ck = [k for k in cf if "copy" in k.lower()]
    f_scale = copy_kib / (cf[ck[0]][1] / cf[ck[0]][0])
    w_scale = copy_kib / (cw[ck[0]][1] / cw[ck[0]][0])
    fe, wr = per_kernel(fetch_dir, "FETCH_SIZE"), per_kernel(write_dir, "WRITE_SIZE")

    def is_gemm(k):
        n = k.split("(")[0].replace("void ", "").replace("sf::", "")
        # the fp32 relative-position table GEMM and its split-K reduction run
        # once while the model initialises, before the probed windows
        init = n.startswith("gemm_slice_kernel<float") or n.startswith("splitk_epi")
        return n.startswith(("gemm_", "splitk_epi", "tf_tail", "tf_layer_tp")) and not init

    n = sum(v[0] for k, v in fe.items() if is_gemm(k))
    rd = sum(v[1] for k, v in fe.items() if is_gemm(k)) * 1024 * f_scale / max(n, 1)
    wt = sum(v[1] for k, v in wr.items() if is_gemm(k)) * 1024 * w_scale / max(n, 1)
    wl = WORKLOADS[name]
    W = {"ultralow64x120s": 380, "low60s": 387, "veryhigh600s": 608}.get(name, 380)
    wk = "" if name == "ultralow64x120s" else f" --workload {name}"
    lines = [f"# GEMM kernel class: HBM traffic from FETCH_SIZE / WRITE_SIZE counters", "",
             f"Workload: {name} ({wl['desc']}); counters taken on the encoder window probe",
             f"(bench.py --window-probe {W}): one steady-state window of {W} frames per stream, "
             f"{wl['batch']} streams, encoded twice.", "",
             "Commands (from /tmp, TMPDIR=/tmp; R = repository root):",
             f"  timeout -s KILL 240 rocprofv3 --pmc FETCH_SIZE -f csv -d FETCH -o run -- python3 R/bench.py{wk} --window-probe {W}",
             f"  timeout -s KILL 240 rocprofv3 --pmc WRITE_SIZE -f csv -d WRITE -o run -- python3 R/bench.py{wk} --window-probe {W}",
             "  timeout -s KILL 120 rocprofv3 --pmc FETCH_SIZE -f csv -d COPY/copy_fetch -o run -- python3 R/bench.py --copy-probe 1024",
             "  timeout -s KILL 120 rocprofv3 --pmc WRITE_SIZE -f csv -d COPY/copy_write -o run -- python3 R/bench.py --copy-probe 1024",
             f"  python3 R/bench.py{wk} --pmc-summary FETCH WRITE COPY", "",
             "GEMM class: every gemm_*, splitk_epi, tf_tail and tf_layer_tp dispatch of the probed windows (the",
             "relative-position table GEMM and its reduction, run once at model initialisation, excluded).", "",
             f"Calibration (1 GiB device copy {ck[0]}): FETCH_SIZE scale {f_scale:.4f}, "
             f"WRITE_SIZE scale {w_scale:.4f}", "",
             "Per kernel (KiB per dispatch, raw counter values):",
             f"  {'kernel':60s} {'n':>5s} {'FETCH':>10s} {'WRITE':>10s}"]
    for k in sorted(fe, key=lambda k: -fe[k][1]):
        wv = wr.get(k, (1, 0.0))
        lines.append(f"  {k[:60]:60s} {fe[k][0]:5d} {fe[k][1] / fe[k][0]:10.1f} "
                     f"{wv[1] / max(wv[0], 1):10.1f}")
    lines += ["", f"GEMM-class launches: {n}",
              f"calibrated HBM read bytes per launch: {rd:.0f}",
              f"calibrated HBM write bytes per launch: {wt:.0f}", "",
              f"workload: {name}", "kernel_class: gemm",
              f"kernel_sources_sha256: {kernel_source_hash()}",
              f"hbm_bytes_per_launch: {rd + wt:.0f}"]
    return "\n".join(lines) + "\n"


def main():
    args = parse()
    if args.copy_probe:
        copy_probe(args.copy_probe)
        return
    if args.pmc_summary:
        text = pmc_summary(args.workload, *args.pmc_summary)
        with open(pmc_file(args.workload), "w") as f:
            f.write(text)
        print(text)
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
    progress(f"workload {args.workload}: generating audio")
    audio_np = load_audio(args.workload, wl)
    audio = torch.from_numpy(audio_np.astype(np.float32)).cuda().contiguous()
    progress("model init")
    r = Runner(args.workload, wl, audio)
    if args.no_graphs and wl["mode"] == "stream":
        r.sf.sortformer_stream_set_option(r.stream.handle, r.sf.SF_STREAM_OPT_GRAPHS, 0)
    if args.fixed_window and wl["mode"] == "stream":
        r.sf.sortformer_stream_set_option(r.stream.handle, r.sf.SF_STREAM_OPT_FIXED_WINDOW, 1)
    for i in range(args.warmup):
        r.one_pass()
        torch.cuda.synchronize()
        progress(f"warm-up pass {i + 1}/{args.warmup} done")
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    ev0.record()
    for i in range(args.steps):
        r.one_pass()
        if i % 5 == 4:
            progress(f"timed pass {i + 1}/{args.steps} enqueued")
    ev1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    gpu_ms = ev0.elapsed_time(ev1)
    ms_per_step = 1e3 * wall / args.steps
    audio_s = audio_np.shape[0] * audio_np.shape[1] / 16000.0
    value = audio_s / (ms_per_step / 1e3)
    progress(f"timed: {ms_per_step:.1f} ms per pass, {value:.1f} x real time")

    lat = r.step_latency()
    prof = {}
    if not args.no_profile:
        sf = r.sf
        for kind in ("gemm", "attn", "ln", "conv", "frontend", "cache"):
            sf.sortformer_profile_begin(kind, 400000)
            r.one_pass()
            prof[kind] = sf.sortformer_profile_end()
            progress(f"profiled pass ({kind}) done")
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
                    "traffic": measured_traffic(args.workload, dom), "launches": p["launches"],
                    "avg_launch_us": round(1e3 * avg_ms, 3)}
    cpu = None
    if not args.no_cpu:
        progress("CPU oracle sample")
        cpu = cpu_baseline(args.workload, wl, audio_np)
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
        "cpu_baseline": cpu,
        "cpu_baseline_1thread": (cpu_baseline(args.workload, wl, audio_np, one_thread=True)
                                 if args.cpu_1thread and not args.no_cpu else None),
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
