"""Throughput of the audio-tower forward pass on one MI355X.

One step = one forward pass of the whole path (log-mel -> conv stack -> 32 windowed layers ->
head -> SwiGLU adapter) over one batch of synthetic PCM already resident in HBM.  Default
workload: the full-size bf16 tower on 16 clips of 30 s (6000 tokens per step).

Prints ONE JSON line: audio-seconds encoded per second, TFLOP/s and % of the bf16 MFMA peak,
the roofline of the dominant kernel (timed live with HIP events on the forward's stream) and
the float64 CPU oracle timed on a bounded sample on this host.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_F32_TFLOPS = 157.3
PEAK_HBM_GBS = 8000.0

WORKLOADS = {
    "c2": "16 x 30 s clips (mixed pink noise / tones / chords / harmonic bursts, peak 0.5), "
          "full-size tower, bf16",
    "c1": "1 x 30 s clip (pink noise + harmonic bursts, peak 0.5), full-size tower, bf16",
    "c3": "512 s stream as 8 x 64 s pieces in one pass, full-size tower, bf16",
    "c4": "60 min recording as 57 sequential 64 s pieces, full-size tower, bf16",
    "ragged": "16 clips of 5-60 s (lengths seeded, mixed content, peak 0.5) in one ragged call, "
              "full-size tower, bf16",
}


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def work_model(cfg: dict, lengths: list) -> dict:
    """Algorithmic work per step for each kernel role: FLOPs (2 per MAC over valid positions and
    in-window attention only) or HBM bytes for the bandwidth-bound roles."""
    from audio_encoder_amd import binding as B
    tab = B.encoder_plan_windows_ragged(cfg, lengths)
    C, d, F, O, A = (cfg[k] for k in ("conv_channels", "d_model", "d_ffn", "d_out", "d_adapter"))
    Lh = cfg["n_layers"]
    L1, L2, L3 = (tab[:, i].astype(float) for i in (3, 4, 5))
    ntok = L3.sum()
    es = 2 if cfg["dtype"] == "bf16" else 4
    w = {
        "conv1": 2 * (L1 * 64).sum() * C * 9,
        "conv2": 2 * (L2 * 32).sum() * C * C * 9,
        "conv3": 2 * (L3 * 16).sum() * C * C * 9,
        "conv_out": 2 * ntok * d * 16 * C,
        "qkv": 2 * ntok * 3 * d * d * Lh,
        "attention": 2 * 2 * (L3 ** 2).sum() * d * Lh,
        "o_proj": 2 * ntok * d * d * Lh,
        "ffn1": 2 * ntok * F * d * Lh,
        "ffn2": 2 * ntok * d * F * Lh,
        "proj1": 2 * ntok * d * d,
        "proj2": 2 * ntok * O * d,
        "gate_up": 2 * ntok * 2 * A * O,
        "down": 2 * ntok * O * A,
    }
    flops = float(sum(w.values()))
    bytes_ = {
        "mel": float(sum(4.0 * n + 512.0 * (n // 160) for n in lengths)),
        "layernorm": (2 * Lh + 1) * ntok * d * (4 + es),
    }
    return {"flops": w, "total_flops": flops, "bytes": bytes_, "ntok": int(ntok)}


RAGGED_SECONDS = (5.0, 60.0)


def ragged_lengths(n_clips: int = 16, seed: int = 500) -> list:
    import numpy as np
    rng = np.random.default_rng(seed)
    return [int(round(16000 * rng.uniform(*RAGGED_SECONDS))) for _ in range(n_clips)]


def make_input(workload: str):
    from audio_encoder_amd import synth as S
    if workload == "ragged":
        import numpy as np
        lens = ragged_lengths()
        pcm = np.concatenate([S.mixed_clip(501 + i, n) for i, n in enumerate(lens)])
        return pcm, sum(lens) / 16000.0
    if workload == "c2":
        return S.mixed_batch(range(101, 117)), 480.0
    if workload == "c1":
        return S.pink_plus_bursts(seed=1)[None], 30.0
    if workload == "c3":
        return S.long_stream_512s()[None], 512.0
    if workload == "c4":
        return S.hour_stream()[None], 3600.0
    raise ValueError(workload)


def measured_traffic(role: str, launches_per_step: int):
    """HBM bytes per launch of `role` from the committed counter summary, or None when the GEMM
    source changed since the counters were taken, when they were taken on launches of another
    size, or when no summary exists."""
    import hashlib
    path = os.path.join(ROOT, "profiles", "hbm_traffic_full_16x30s.json")
    src = os.path.join(ROOT, "audio_encoder_amd", "csrc", "ae_gemm.hip")
    try:
        with open(path) as f:
            rec = json.load(f)
        with open(src, "rb") as f:
            sha = hashlib.sha256(f.read()).hexdigest()
    except OSError:
        return None
    if rec.get("gemm_source_sha256") != sha or role not in rec.get("per_launch", {}):
        return None
    if rec.get("launches_per_step", {}).get(role) != launches_per_step:
        return None
    t = rec["per_launch"][role]
    return round(t["fetch_bytes"] + t["write_bytes"])


def cpu_baseline(pcm, weights, cfg, max_windows: int = 24, int4: bool = False) -> dict:
    """The float64 oracle on the first `max_windows` 8 s windows of the batch (clip by clip;
    about 10-30 s of CPU work), scaled to audio-seconds per second."""
    import numpy as np

    import oracle as O
    Wt = O.unpack_weights(weights, O.FULL)
    if int4:
        Wt = O.int4_weights(Wt, O.FULL)
    W = cfg["window_tokens"]
    t0 = time.perf_counter()
    frames = nwin = clips = 0
    for clip in pcm:
        mel = O.log_mel(clip)
        clips += 1
        for w in O.window_plan(mel.shape[0], W):
            O.encode_mel(mel[w["start"]:w["start"] + w["L0"]], Wt, O.FULL)
            frames += w["L0"]
            nwin += 1
            if nwin >= max_windows:
                break
        if nwin >= max_windows:
            break
    dt = time.perf_counter() - t0
    audio_s = frames * 160 / 16000.0
    cores = len(os.sched_getaffinity(0))
    return {"value": audio_s / dt, "unit": "audio-s/s", "cores": cores, "kind": "oracle",
            "sample": f"first {nwin} windows of the batch ({clips} clips, {audio_s:.0f} s of "
                      f"audio), float64 NumPy, {dt:.1f} s wall",
            "cpu": host_cpu_model(), "blas": blas_vendor()}


def host_cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def blas_vendor() -> str:
    import numpy as np
    try:
        cfg = np.show_config(mode="dicts")
        b = cfg["Build Dependencies"]["blas"]
        return f"{b.get('name', '?')} {b.get('version', '')}".strip()
    except Exception:
        return "unknown"


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="c2", choices=sorted(WORKLOADS))
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--weight-bits", type=int, default=16, choices=(16, 4),
                    help="4: int4 weight-only linear layers, head and adapter (dequantised in the "
                         "GEMM loader); the CPU baseline then runs on the dequantised weights")
    ap.add_argument("--split-small-gemms", action="store_true",
                    help="split K of GEMMs too small to fill the GPU (single clips); their rows then "
                         "round differently from the same rows in a large call")
    ap.add_argument("--pieces-per-pass", type=int, default=0,
                    help="long-audio workloads: 64 s pieces per pass (default 8 for c3, 1 for c4)")
    ap.add_argument("--roofline-steps", type=int, default=3)
    ap.add_argument("--copy-probe-mb", type=int, default=0,
                    help="after the run, launch one plain device copy of this many MiB (a "
                         "known-size reference for HBM byte counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for {args.gpus}); windows are independent, "
              "so several GPUs would each run this same step on their own share of clips.",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    from audio_encoder_amd import binding as B
    from audio_encoder_amd import synth as S

    cfg = dict(B.FULL, weight_bits=args.weight_bits, split_small_gemms=int(args.split_small_gemms))
    log("generating weights and input")
    weights = S.make_weights(cfg, seed=0)
    pcm_np, audio_s = make_input(args.workload)
    free_before, _ = torch.cuda.mem_get_info()
    enc = B.Encoder(weights, cfg)
    pcm = torch.from_numpy(pcm_np).cuda()
    long_mode = args.workload in ("c3", "c4")
    ragged = args.workload == "ragged"
    ppp = args.pieces_per_pass or (8 if args.workload == "c3" else 1)
    if ragged:
        lengths = ragged_lengths()
        n_clips, n_samples = len(lengths), max(lengths)
        out = torch.empty((sum(enc.output_frames(n) for n in lengths), cfg["d_out"]),
                          dtype=torch.bfloat16, device="cuda")
    else:
        n_clips, n_samples = pcm.shape[0], pcm.shape[1]
        lengths = [n_samples] * n_clips
        out = torch.empty((n_clips, enc.output_frames(n_samples), cfg["d_out"]),
                          dtype=torch.bfloat16, device="cuda")
    wm = work_model(cfg, lengths)

    def step():
        if ragged:
            enc.forward_ragged(pcm, lengths, out=out)
        elif long_mode:
            enc.forward_long(pcm[0], pieces_per_pass=ppp, out=out[0])
        else:
            enc.forward(pcm, out=out)

    log(f"warmup {args.warmup}")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    log(f"timing {args.steps} steps")
    # one event between consecutive steps: the total gives the mean, the gaps the median
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    torch.cuda.synchronize()
    t_wall = time.perf_counter()
    evs[0].record()
    for i in range(args.steps):
        step()
        evs[i + 1].record()
    torch.cuda.synchronize()
    t_wall = time.perf_counter() - t_wall
    ms = evs[0].elapsed_time(evs[-1]) / args.steps
    ms_median = float(np.median([evs[i].elapsed_time(evs[i + 1]) for i in range(args.steps)]))
    free_after, _ = torch.cuda.mem_get_info()
    tflops = wm["total_flops"] / (ms * 1e-3) / 1e12
    log(f"{ms:.3f} ms/step, {audio_s / (ms * 1e-3):.0f} audio-s/s, {tflops:.1f} TFLOP/s "
        f"({100 * tflops / PEAK_BF16_TFLOPS:.1f}% of bf16 peak); wall {t_wall:.2f} s")

    # Per-kernel timing on the forward's own stream, in extra steps run kernel by kernel on one
    # stream.  Mode 1 runs the passes of the timed steps (a 6000-token call: two 3000-token
    # halves) one after another; mode 2 runs a call that fits one pass as that single pass.  A
    # one-element int16 fill before each marks where these steps begin in a profiler's kernel
    # trace.
    R = args.roofline_steps

    def role_times(mode):
        torch.full((1,), 7, dtype=torch.int16, device="cuda")
        torch.cuda.synchronize()
        enc.timing_enable(mode)
        enc.timing_read(reset=True)
        for _ in range(R):
            step()
        tm = enc.timing_read(reset=True)
        enc.timing_enable(0)
        return tm

    def roofline(tm, dom, passes):
        dom_ms, dom_n = tm[dom]
        avg_ms = dom_ms / dom_n
        per_launch = wm["flops"][dom] / (dom_n / R)
        achieved = per_launch / (avg_ms * 1e-3) / 1e12
        return {"bound": "mfma", "kernel": dom, "achieved": round(achieved, 2),
                "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                "frac": round(achieved / PEAK_BF16_TFLOPS, 4), "avg_launch_ms": round(avg_ms, 5),
                "launches_per_step": dom_n // R, "algorithmic_unit": "FLOP per launch",
                "algorithmic_per_launch": per_launch,
                "method": "HIP events around each launch on the forward's stream, in extra steps "
                          f"run kernel by kernel on one stream ({passes})"}

    tm = role_times(1)
    stage_ms = {k: round(v[0] / R, 4) for k, v in tm.items() if v[1]}
    dom = max((k for k in tm if k in wm["flops"]), key=lambda k: tm[k][0])
    roof = roofline(tm, dom, "the passes of the timed steps, one after another")
    roof["traffic"] = measured_traffic(dom, roof["launches_per_step"]) if args.workload == "c2" else None
    tm2 = role_times(2)
    roof_single = roofline(tm2, dom, "a call that fits one pass run as that one pass")
    for k, v in stage_ms.items():
        log(f"  {k:10s} {v:8.3f} ms/step")
    log(f"dominant kernel {dom}: {roof['frac']:.4f} of peak in the timed passes, "
        f"{roof_single['frac']:.4f} as one pass")

    cpu = None
    if not args.no_cpu_baseline:
        log("timing the CPU oracle")
        clips = ([pcm_np[o:o + n] for o, n in zip(np.cumsum([0] + lengths[:-1]), lengths)]
                 if ragged else list(pcm_np))
        cpu = cpu_baseline(clips, weights, cfg, int4=args.weight_bits == 4)
        log(f"oracle: {cpu['value']:.2f} audio-s/s on {cpu['cores']} cores")

    wbytes, ws = enc.memory_stats()
    line = {
        "metric": "audio-seconds encoded/sec (bf16, 1 GPU) + % of bf16 MFMA peak",
        "value": round(audio_s / (ms * 1e-3), 1),
        "unit": "audio-s/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "median_ms_per_step": round(ms_median, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if args.weight_bits == 16 else "bf16 (int4 weights)",
        "data": "synthetic",
        "config": {"workload": WORKLOADS[args.workload], "clips": int(n_clips),
                   "samples_per_clip": int(n_samples) if not ragged else lengths,
                   "tokens_per_step": wm["ntok"], "audio_seconds_per_step": audio_s,
                   **({"pieces_per_pass": ppp} if long_mode else {})},
        "tflops": round(tflops, 2),
        "pct_bf16_peak": round(100 * tflops / PEAK_BF16_TFLOPS, 2),
        "roofline": roof,
        "roofline_single_pass": roof_single,
        "cpu_baseline": cpu,
        "stage_ms": stage_ms,
        # device memory: the library's weights and workspace high-water mark, and the drop in
        # free device memory (hipMemGetInfo) from before the encoder was created to the end of
        # the timed run (inputs and outputs included)
        "hbm_bytes": {"weights": wbytes, "workspace_high_water": ws,
                      "device_used_delta": int(free_before - free_after)},
    }
    print(json.dumps(line), flush=True)
    if args.copy_probe_mb:
        n = args.copy_probe_mb * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        log(f"copy probe: {4 * n} bytes read, {4 * n} bytes written")


if __name__ == "__main__":
    main()
