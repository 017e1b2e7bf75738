"""Benchmark of the VDA linear-branch hot path on one MI355X.

One step = the whole path for one layer of the H3-shaped workload (24 heads,
d = 128, 102 latent frames of which 2 are anchors, U = 1008 tokens per frame,
512 text tokens, bf16 inputs, float32 state, bf16 output):

    vda_prepare_frames -> vda_scan_fwd || vda_scan_rev -> vda_readout

Inputs are seeded synthetic draws (frame_wise_delta_amd.inputs) resident in
HBM before timing starts.  Prints one JSON line: latent frames/s (value),
algorithmic TFLOP/s and the fraction of the bf16 MFMA peak, a roofline entry
for the dominant kernel timed with HIP events on its own stream, and the
float64 oracle timed on this host's cores on the same inputs.

    python bench.py [--steps K] [--warmup W] [--config h3] [--no-cpu-baseline]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2516.6   # MI355X dense bf16/f16 MFMA
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E


def algorithmic_work(cfg):
    """Algorithmic FLOPs and HBM bytes of one step.  Per scanned frame-head:
    2Ud^2 (A) + 2Ud^2 (B) + d^3 (solve) + 2 * 2d^3 (two scan directions)
    + 2 * 2Ud^2 (forward and reverse reads; one read without window
    exclusion); bytes: Q, K, V (16-bit), beta, alpha, O (16-bit).  Text
    state once per head: 4 N_text d^2 + d^3 + 2d^3 FLOPs, k_T, v_T, beta_T."""
    U, d, n, H, Nt = cfg.tokens, cfg.d, cfg.scanned, cfg.heads, cfg.text_tokens
    ib = 4 if cfg.in_dtype == "f32" else 2
    ob = {"f32": 4, "bf16": 2, "f16": 2}[cfg.out_dtype]
    reads = 2 if cfg.window >= 0 else 1
    fl_fh = 4 * U * d * d + d ** 3 + 4 * d ** 3 + reads * 2 * U * d * d
    by_fh = 3 * U * d * ib + 4 * U + 4 * d + U * d * ob
    fl_text = (4 * Nt * d * d + 3 * d ** 3) if Nt else 0
    by_text = (2 * Nt * d * ib + 4 * Nt) if Nt else 0
    return H * (n * fl_fh + fl_text), H * (n * by_fh + by_text)


def kernel_bytes(cfg):
    """Algorithmic HBM bytes of one launch of each kernel."""
    U, d, n, H, Nt, T = cfg.tokens, cfg.d, cfg.scanned, cfg.heads, cfg.text_tokens, cfg.frames
    ib = 4 if cfg.in_dtype == "f32" else 2
    ob = {"f32": 4, "bf16": 2, "f16": 2}[cfg.out_dtype]
    prep = H * (n * (2 * U * d * ib + 4 * U) + (2 * Nt * d * ib + 4 * Nt))
    read = H * n * (U * d * ib + U * d * ob + 4 * d)
    return {"prepare": prep, "readout": read}


def _src_hash():
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "frame_wise_delta_amd", "csrc")
    for name in sorted(os.listdir(csrc)):
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(name.encode() + f.read())
    return h.hexdigest()[:16]


def _traffic(kernel):
    """HBM traffic per launch measured with rocprofv3 counters (committed
    under profiles/), or None if the kernels changed since."""
    p = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        with open(p) as f:
            t = json.load(f)
    except OSError:
        return None
    if t.get("src_hash") != _src_hash():
        return None
    k = t.get("kernels", {}).get(kernel)
    return None if k is None else k.get("bytes_per_launch")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", default="h3")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-heads", type=int, default=None,
                    help="heads the oracle runs for the CPU baseline (default: all)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (--gpus {args.gpus} requested): the VDA path is "
              "built and measured on a single MI355X; heads would shard across GPUs with no "
              "communication, which this build does not run.", file=sys.stderr)
        sys.exit(2)

    import torch
    from frame_wise_delta_amd import inputs as inp
    from frame_wise_delta_amd import runner, vda

    cfg = inp.CONFIG_BY_NAME[args.config]
    t0 = time.time()
    heads_in = inp.all_heads(cfg)
    t_gen = time.time() - t0
    print(f"[bench] inputs for {cfg.name} drawn in {t_gen:.1f}s", file=sys.stderr, flush=True)
    desc = vda.desc_for(cfg)
    dev = runner.upload(cfg, heads_in, "cuda")
    bufs = runner.allocate(desc, cfg.out_dtype, "cuda")
    path = runner.Path(desc, dev, bufs)
    main_s, side_s = path.main, path.side

    # events around each kernel, on the stream it runs on
    names = ["prepare", "scan_fwd", "scan_rev", "readout"]
    ev = {k: [] for k in names}

    def step(record):
        pairs = {}
        if record:
            for k in names:
                pairs[k] = (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
        x, b = dev, bufs
        if record:
            pairs["prepare"][0].record(main_s)
        vda.vda_prepare_frames(desc, x.k, x.v, x.beta, x.kt, x.vt, x.bt, b.ws, b.ws_bytes, stream=main_s)
        if record:
            pairs["prepare"][1].record(main_s)
        path.ev_prep.record(main_s)
        side_s.wait_event(path.ev_prep)
        if record:
            pairs["scan_rev"][0].record(side_s)
        vda.vda_scan_rev(desc, b.ws, x.alpha, None, b.states_r, stream=side_s)
        if record:
            pairs["scan_rev"][1].record(side_s)
        path.ev_rev.record(side_s)
        if record:
            pairs["scan_fwd"][0].record(main_s)
        vda.vda_scan_fwd(desc, b.ws, x.alpha, None, b.states_f, stream=main_s)
        if record:
            pairs["scan_fwd"][1].record(main_s)
        main_s.wait_event(path.ev_rev)
        if record:
            pairs["readout"][0].record(main_s)
        vda.vda_readout(desc, x.q, x.alpha, b.states_f, b.states_r, b.out, stream=main_s)
        if record:
            pairs["readout"][1].record(main_s)
            for k in names:
                ev[k].append(pairs[k])

    for _ in range(args.warmup):
        step(False)
    torch.cuda.synchronize()
    print(f"[bench] warmup {args.warmup} steps done", file=sys.stderr, flush=True)
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step(True)
    torch.cuda.synchronize()
    t_total = time.perf_counter() - t0
    status = vda.vda_device_status(desc, bufs.ws)
    ms_step = 1e3 * t_total / args.steps
    kms = {k: float(np.mean([a.elapsed_time(b) for a, b in ev[k]])) for k in names}
    print(f"[bench] {args.steps} steps: {ms_step:.3f} ms/step; kernels {kms}", file=sys.stderr, flush=True)

    flops, nbytes = algorithmic_work(cfg)
    t_s = ms_step / 1e3
    frames_s = cfg.frames / t_s
    tflops = flops / t_s / 1e12
    kb = kernel_bytes(cfg)
    dom = max(("prepare", "readout"), key=lambda k: kms[k])
    ach = kb[dom] / (kms[dom] / 1e3) / 1e9
    roofline = {"kernel": dom, "bound": "hbm", "achieved": round(ach, 1), "peak": PEAK_HBM_GBS,
                "unit": "GB/s", "frac": round(ach / PEAK_HBM_GBS, 4), "traffic": _traffic(dom),
                "algorithmic_bytes": kb[dom], "avg_ms": round(kms[dom], 4)}

    cpu = None
    rel = None
    if not args.no_cpu_baseline:
        from oracle import vda_oracle as orc
        try:
            from threadpoolctl import threadpool_info
            cores = max(x.get("num_threads", 1) for x in threadpool_info()) if threadpool_info() else 1
        except Exception:
            cores = len(os.sched_getaffinity(0))
        hs = list(range(cfg.heads if args.cpu_heads is None else min(args.cpu_heads, cfg.heads)))
        O0 = bufs.out[0].float().cpu().numpy().astype(np.float64)
        t_cpu = 0.0
        errs = []
        for h in hs:
            f = heads_in[h].f64
            text = cfg.text_tokens > 0
            a = [f(x) for x in ("q", "k", "v", "beta", "alpha")]
            tt = [f(x) if text else None for x in ("kt", "vt", "bt")]
            c0 = time.perf_counter()
            ref = orc.run_head(cfg.frames, cfg.chunk, cfg.window, cfg.anchors, *a, *tt)
            t_cpu += time.perf_counter() - c0
            if h == 0:
                sl = slice(cfg.anchors, cfg.frames - cfg.anchors)
                errs.append(orc.rel_l2(O0[sl], ref["O"][sl]))
        frac = len(hs) / cfg.heads
        cpu = {"value": round(cfg.frames * frac / t_cpu, 4), "unit": "frames/s", "cores": int(cores),
               "kind": "oracle",
               "sample": f"{len(hs)} of {cfg.heads} heads of the same workload (all {cfg.frames} frames), "
                         f"float64 NumPy/LAPACK, {t_cpu:.1f}s; frames/s scaled by heads fraction"}
        rel = errs[0] if errs else None

    out = {
        "metric": "VDA scan+readout latent frames/s and % of MI355X bf16 MFMA peak",
        "value": round(frames_s, 2),
        "unit": "frames/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"{cfg.name}: {cfg.heads} heads, d={cfg.d}, {cfg.frames} latent frames "
                               f"({cfg.anchors * 2} anchors, chunks of {cfg.chunk}, window +-{cfg.window} "
                               f"chunk), U={cfg.tokens}, {cfg.text_tokens} text tokens",
                   "heads": cfg.heads, "d": cfg.d, "frames": cfg.frames, "tokens": cfg.tokens,
                   "text_tokens": cfg.text_tokens, "in_dtype": cfg.in_dtype, "out_dtype": cfg.out_dtype,
                   "state_dtype": "f32", "global_batch": 1, "seq_len": cfg.frames * cfg.tokens,
                   "parallelism": "single GPU"},
        "tflops_algorithmic": round(tflops, 2),
        "mfma_peak_frac": round(tflops / PEAK_BF16_TFLOPS, 4),
        "hbm_frac_path": round(nbytes / t_s / 1e9 / PEAK_HBM_GBS, 4),
        "kernel_ms": {k: round(v, 4) for k, v in kms.items()},
        "roofline": roofline,
        "cpu_baseline": cpu,
        "rel_l2_head0": rel,
        "device_status": status,
    }
    print(json.dumps(out))


if __name__ == "__main__":
    main()
