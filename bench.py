"""Benchmark of the VDA linear-branch hot path on one MI355X.

One step = the whole path for one attention layer of the H3-shaped workload
(24 heads, d = 128, 102 latent frames of which 2 are anchors, U = 1008
tokens per frame, 512 text tokens, bf16 inputs, float32 state, bf16 output):

    vda_prepare_frames -> vda_scan_bidir -> vda_readout

(the same kernels, in the same order, as one vda_forward call).  Inputs are
seeded synthetic draws (frame_wise_delta_amd.inputs) resident in HBM before
timing starts.  The timed region is K steps back to back (ms_per_step, the
headline); a second pass of K steps brackets every call with HIP events on
the stream it runs on, for the per-call times and the roofline of the
dominant HBM-bound kernel (the events add ~30 us per step, so that pass is
not the step time); a third pass times each step with the caches flushed
first (a 512 MiB buffer written between steps, outside the events); and a
plain streaming read of a 4 GiB buffer (the best of four grid sizes) gives
the read bandwidth the device reaches without any arithmetic.  Prints one JSON line: latent frames/s,
algorithmic TFLOP/s, the roofline entry, and the float64 oracle timed on
this host's cores.

    python bench.py [--steps K] [--warmup W] [--config h3|long|hires] [--no-cpu-baseline] [--epilogue] [--prep]
                    [--chunk-scan] [--sana-wm] [--newton]
    python bench.py --softmax [--steps K] [--warmup W]

--epilogue replaces the readout by vda_readout_gated (the readout followed by
the RMSNorm + sigmoid-gate epilogue of the linear branch, with seeded gate
logits and norm weights); --prep feeds raw projections (q, k not normalised,
beta and alpha as logits) and sets VDA_PREP, so the kernels normalise and
gate them.  Both measure next steps of the path; neither is the default line.
--chunk-scan sets VDA_CHUNK_SCAN: vda_compose_chunks after the factorisation,
then the scans at chunk level (S <- S M_c + J_c once per chunk).
--sana-wm sets VDA_SANA_WM: the SANA-WM batched additive update as a
comparator (the prepare call then forms -A/U and B/sqrt(U)).
--newton sets VDA_NEWTON: (I + A)^-1 by Newton iteration in the prepare
call instead of Gauss-Jordan.
--config long / hires time the long-video (202 frames) and high-resolution
(402 frames, U = 2016) workloads; the oracle baseline then covers the
heads it finishes in its time budget.
--softmax times the softmax window + anchor + text branch (vda_softmax_branch)
on the same workload instead: an MFMA-bound kernel, reported against the
bf16 MFMA peak.

Measurement helpers (used to make the files under profiles/):

    python bench.py --copy-calibration
        copies a 512 MiB device buffer three times (a plain copy of known
        size, profiled with rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE)
    python bench.py --traffic FETCH.csv WRITE.csv COPY_FETCH.csv COPY_WRITE.csv
        turns the four rocprofv3 counter_collection files into
        profiles/traffic.json: HBM bytes per launch of each kernel, with both
        counters scaled by the factor that maps the copy's counts to its size
"""
from __future__ import annotations

import argparse
import csv
import hashlib
import json
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2516.6   # MI355X dense bf16/f16 MFMA
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
COPY_BYTES = 512 * 1024 * 1024
KERNELS = ("frame_kernel", "stats_kernel", "ns_kernel", "sana_kernel", "scan_kernel", "compose_kernel",
           "readout_kernel", "readout_gated")
EPS = 1e-6  # RMSNorm epsilon of the epilogue


def algorithmic_work(cfg, epilogue=False):
    """Algorithmic FLOPs and HBM bytes of one step.  Per scanned frame-head:
    2Ud^2 (A) + 2Ud^2 (B) + d^3 (solve) + 2 * 2d^3 (two scan directions)
    + 2Ud^2 (the readout: the forward and reverse reads are one product with
    the merged operand W_t = S^f Diag(b_f) + S^r Diag(b_r), formed in 2d^2);
    bytes: Q, K, V (16-bit), beta, alpha, O (16-bit), plus the gate logits
    with the epilogue (its few elementwise FLOPs are not counted).  Text
    state once per head: 4 N_text d^2 + d^3 + 2d^3 FLOPs, k_T, v_T, beta_T.
    Returns (flops, bytes, flops counting the two reads as two products)."""
    U, d, n, H, Nt = cfg.tokens, cfg.d, cfg.scanned, cfg.heads, cfg.text_tokens
    ib = 4 if cfg.in_dtype == "f32" else 2
    ob = {"f32": 4, "bf16": 2, "f16": 2}[cfg.out_dtype]
    reads = 2 if cfg.window >= 0 else 1
    base = 4 * U * d * d + d ** 3 + 4 * d ** 3
    fl_fh = base + 2 * U * d * d + (2 * d * d if reads == 2 else 0)
    fl_fh_two = base + reads * 2 * U * d * d
    by_fh = 3 * U * d * ib + 4 * U + 4 * d + U * d * ob + (U * d * ib if epilogue else 0)
    fl_text = (4 * Nt * d * d + 3 * d ** 3) if Nt else 0
    by_text = (2 * Nt * d * ib + 4 * Nt) if Nt else 0
    return H * (n * fl_fh + fl_text), H * (n * by_fh + by_text), H * (n * fl_fh_two + fl_text)


def kernel_bytes(cfg):
    """Algorithmic HBM bytes of one launch of the HBM-bound kernels: the
    statistics (with the factorisation in frame_kernel) read K, V (16-bit)
    and beta of every scanned frame and the text tokens; the readout reads
    Q and alpha of every scanned frame and writes every output row (anchor
    rows are zeros); the gated readout also reads the gate logits of every
    scanned frame."""
    U, d, n, H, Nt, T = cfg.tokens, cfg.d, cfg.scanned, cfg.heads, cfg.text_tokens, cfg.frames
    ib = 4 if cfg.in_dtype == "f32" else 2
    ob = {"f32": 4, "bf16": 2, "f16": 2}[cfg.out_dtype]
    stats = H * (n * (2 * U * d * ib + 4 * U) + (2 * Nt * d * ib + 4 * Nt))
    read = H * (n * (U * d * ib + 4 * d) + T * U * d * ob)
    gated = read + H * n * U * d * ib + H * d * 4
    return {"frame_kernel": stats, "stats_kernel": stats, "readout_kernel": read, "readout_gated": gated}


KERNEL_SRC = {"frame_kernel": "vda_prepare.hip", "stats_kernel": "vda_prepare.hip",
              "ns_kernel": "vda_prepare.hip", "sana_kernel": "vda_prepare.hip",
              "scan_kernel": "vda_scan.hip", "compose_kernel": "vda_scan.hip", "readout_kernel": "vda_readout.hip",
              "readout_gated": "vda_readout.hip"}


def _code_only(text):
    """C++ source without comments and blank lines, so that a change to
    comments alone does not count as a change of the kernel."""
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    text = re.sub(r"//[^\n]*", "", text)
    return "\n".join(l.rstrip() for l in text.splitlines() if l.strip())


def _src_hash(kernel):
    """Hash of the code a kernel is compiled from (its file and the shared
    headers, comments left out)."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "frame_wise_delta_amd", "csrc")
    for name in (KERNEL_SRC[kernel], "vda_common.h", "vda_kernels.h"):
        with open(os.path.join(csrc, name), encoding="utf-8") as f:
            h.update(name.encode() + _code_only(f.read()).encode())
    return h.hexdigest()[:16]


TRAFFIC_JSON = os.path.join(ROOT, "profiles", "traffic.json")


def _traffic(kernel):
    """HBM bytes per launch measured with rocprofv3 counters (profiles/
    traffic.json), or None if the kernel's sources changed since."""
    try:
        with open(TRAFFIC_JSON) as f:
            t = json.load(f)
    except OSError:
        return None
    k = t.get("kernels", {}).get(kernel)
    if k is None or k.get("src_hash") != _src_hash(kernel):
        return None
    return k.get("bytes_per_launch")


# ------------------------------------------------------------- helpers --

def copy_calibration():
    import torch
    x = torch.ones(COPY_BYTES // 4, device="cuda")
    y = torch.empty_like(x)
    torch.cuda.synchronize()
    for _ in range(3):
        y.copy_(x)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes": COPY_BYTES, "copies": 3}))


def _short(name):
    """Short name of a profiled kernel; the gated readout is the
    readout_kernel instantiation whose fourth template argument (GATED) is
    true: readout_kernel<D, TIN, OUT, GATED, PREP>."""
    if "readout_kernel" in name:
        m = re.search(r"readout_kernel<([^>]*)>", name)
        args = [x.strip() for x in m.group(1).split(",")] if m else []
        return "readout_gated" if len(args) >= 4 and args[3] == "true" else "readout_kernel"
    for k in KERNELS:
        if k in name:
            return k
    return None


def _counter_means(path, counter):
    """Mean counter value (KiB) per dispatch of each kernel in a
    counter_collection file; for the copy, only the copy dispatches."""
    sums, counts = {}, {}
    with open(path) as f:
        for r in csv.DictReader(f):
            if r["Counter_Name"] != counter:
                continue
            name = r["Kernel_Name"]
            key = _short(name) or ("copy" if "copyBuffer" in name else None)
            if key is None:
                continue
            sums[key] = sums.get(key, 0.0) + float(r["Counter_Value"])
            counts[key] = counts.get(key, 0) + 1
    return {k: sums[k] / counts[k] for k in sums}


def write_traffic(fetch_csv, write_csv, cal_fetch_csv, cal_write_csv):
    f = _counter_means(fetch_csv, "FETCH_SIZE")
    w = _counter_means(write_csv, "WRITE_SIZE")
    cf = _counter_means(cal_fetch_csv, "FETCH_SIZE")["copy"]
    cw = _counter_means(cal_write_csv, "WRITE_SIZE")["copy"]
    ff = COPY_BYTES / (cf * 1024.0)
    wf = COPY_BYTES / (cw * 1024.0)
    # kernels profiled in other runs (e.g. the gated readout) stay as they were
    try:
        with open(TRAFFIC_JSON) as fh:
            kept = json.load(fh).get("kernels", {})
    except (OSError, ValueError):
        kept = {}
    # (entries whose sources have changed since are dropped)
    out = {"calibration": {"copy_bytes": COPY_BYTES, "fetch_kib": cf, "write_kib": cw,
                           "fetch_factor": round(ff, 4), "write_factor": round(wf, 4)},
           "kernels": {k: v for k, v in kept.items()
                       if k in KERNELS and not (k in f and k in w) and v.get("src_hash") == _src_hash(k)}}
    for k in KERNELS:
        if k in f and k in w:
            fb, wb = f[k] * 1024.0 * ff, w[k] * 1024.0 * wf
            out["kernels"][k] = {"fetch_bytes": round(fb), "write_bytes": round(wb),
                                 "bytes_per_launch": round(fb + wb), "src_hash": _src_hash(k)}
    os.makedirs(os.path.dirname(TRAFFIC_JSON), exist_ok=True)
    with open(TRAFFIC_JSON, "w") as fh:
        json.dump(out, fh, indent=1)
    print(json.dumps(out))


# ---------------------------------------------------------------- bench --

def cpu_baseline(cfg, heads_in, out0, budget_s=15.0, epi_in=None, prep=False, update="vda"):
    """The float64 oracle, as it stands, on whole heads of the same workload
    until about budget_s seconds of CPU time are spent (at least one head);
    with epi_in, followed by the oracle's readout epilogue; update selects
    the frame update rule ("sana": the SANA-WM comparator)."""
    from oracle import vda_oracle as orc
    try:
        from threadpoolctl import threadpool_info
        info = threadpool_info()
        cores = max(x.get("num_threads", 1) for x in info) if info else 1
    except Exception:
        cores = len(os.sched_getaffinity(0))
    text = cfg.text_tokens > 0
    t_cpu, done, rel = 0.0, 0, None
    for h in range(cfg.heads):
        f = heads_in[h].f64
        args = [f(x) for x in ("q", "k", "v", "beta", "alpha")] + [f(x) if text else None for x in ("kt", "vt", "bt")]
        c0 = time.perf_counter()
        if prep:
            q, k, v, b, a, kt, vt, bt = args
            q, k, b, a, kt, bt = orc.prep(q, k, b, a, kt, bt, eps=1e-6)
            args = [q, k, v, b, a, kt, vt, bt]
        ref = orc.run_head(cfg.frames, cfg.chunk, cfg.window, cfg.anchors, *args, update=update)
        if epi_in is not None:
            ref["O"] = orc.rmsnorm_gate(ref["O"], epi_in[h].f64("weight"), epi_in[h].f64("gate"), EPS)
        t_cpu += time.perf_counter() - c0
        done += 1
        if h == 0:
            sl = slice(cfg.anchors, cfg.frames - cfg.anchors)
            rel = orc.rel_l2(out0[sl], ref["O"][sl])
        if t_cpu >= budget_s:
            break
    frac = done / cfg.heads
    return ({"value": round(cfg.frames * frac / t_cpu, 4), "unit": "frames/s", "cores": int(cores),
             "kind": "oracle",
             "sample": f"{done} of {cfg.heads} heads of the same workload (all {cfg.frames} frames of each), "
                       f"float64 NumPy/LAPACK{' with the prep' if prep else ''}"
                       f"{' with the SANA-WM update' if update == 'sana' else ''}"
                       f"{' with the readout epilogue' if epi_in is not None else ''}, "
                       f"{t_cpu:.1f} s; frames/s scaled by the fraction of heads"},
            rel)


def softmax_work(cfg):
    """Algorithmic FLOPs and HBM bytes of the softmax branch: 4d FLOPs per
    (query, visible key) pair (q.k and p.v), and Q, K, V (bf16), text K, V
    and O (bf16) once."""
    T, P, w = cfg.frames, cfg.chunk, cfg.window
    a = 1 if cfg.anchors else 0
    n = T - 2 * a
    C = -(-n // P)
    visible = 0
    for t in range(T):
        if a and t in (0, T - 1):
            visible += T                       # an anchor frame sees every frame
        else:
            c = (t - a) // P                   # window: chunks c-w .. c+w, clipped
            lo, hi = max(c - w, 0), min(c + w, C - 1)
            visible += min(a + P * (hi + 1), T - a) - (a + P * lo) + 2 * a
    pairs = (visible * cfg.tokens + T * cfg.text_tokens) * cfg.tokens
    flops = 4 * cfg.d * pairs * cfg.heads
    nbytes = cfg.heads * (4 * cfg.frames * cfg.tokens * cfg.d * 2 + 2 * cfg.text_tokens * cfg.d * 2)
    return flops, nbytes


def softmax_bench(args):
    """The softmax branch on the H3-shaped workload: seeded bf16 q, k, f16 v
    (the same draws, exactly representable), resident in HBM; K timed calls."""
    import torch
    from frame_wise_delta_amd import inputs as inp
    from frame_wise_delta_amd import runner, vda
    cfg = inp.CONFIG_BY_NAME[args.config]
    if cfg.window < 0:
        sys.exit(f"bench.py --softmax: config {cfg.name} has no window (the softmax branch needs one)")
    t0 = time.time()
    ins = [inp.softmax_inputs(cfg, h) for h in range(cfg.heads)]
    dev = lambda name: runner._dev(np.stack([getattr(x, name) for x in ins]), "cuda")
    q, k = dev("q"), dev("k")
    v = dev("v").view(torch.bfloat16).to(torch.float16)
    kt, vt = dev("kt"), dev("vt").view(torch.bfloat16).to(torch.float16)
    print(f"[bench] softmax inputs drawn in {time.time() - t0:.1f}s", file=sys.stderr, flush=True)
    out = torch.empty((cfg.heads, cfg.frames, cfg.tokens, cfg.d), dtype=torch.bfloat16, device="cuda")
    desc = vda.desc_for(cfg)
    scale = 1.0 / np.sqrt(cfg.d)
    st = torch.cuda.current_stream()
    call = lambda: vda.vda_softmax_branch(desc, q, k, v, kt, vt, scale, out, v_dtype="f16", stream=st)
    for _ in range(args.warmup):
        call()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record(st)
    for _ in range(args.steps):
        call()
    e1.record(st)
    torch.cuda.synchronize()
    ms = 1e3 * (time.perf_counter() - t0) / args.steps
    ms_ev = e0.elapsed_time(e1) / args.steps
    flops, nbytes = softmax_work(cfg)
    tf = flops / (ms_ev / 1e3) / 1e12
    res = {
        "metric": "softmax window + anchor + text branch TFLOP/s and % of MI355X bf16 MFMA peak",
        "value": round(tf, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms, 4), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic",
        "config": {"workload": f"{cfg.name}: {cfg.heads} heads, d={cfg.d}, {cfg.frames} latent frames, "
                               f"U={cfg.tokens}, window +-{cfg.window} chunk of {cfg.chunk}, 2 anchors, "
                               f"{cfg.text_tokens} text tokens; q, k bf16, v f16, bf16 out"},
        "roofline": {"kernel": "attn_kernel", "bound": "mfma", "achieved": round(tf, 1), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(tf / PEAK_BF16_TFLOPS, 4), "traffic": None,
                     "algorithmic_flops_per_launch": flops, "avg_ms": round(ms_ev, 4)},
        "hbm_bytes_algorithmic": nbytes,
    }
    print(json.dumps(res))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=20,
                    help="untimed steps first (the clock settles over the first ~20 steps)")
    ap.add_argument("--config", default="h3")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=15.0,
                    help="CPU time budget of the oracle baseline (whole heads)")
    ap.add_argument("--epilogue", action="store_true",
                    help="time the readout with the RMSNorm + sigmoid-gate epilogue (vda_readout_gated)")
    ap.add_argument("--prep", action="store_true",
                    help="raw inputs prepared inside the kernels (VDA_PREP: L2 normalisation, sigmoid gates)")
    ap.add_argument("--chunk-scan", action="store_true",
                    help="scans at chunk level from composed chunk maps (VDA_CHUNK_SCAN)")
    ap.add_argument("--sana-wm", action="store_true",
                    help="the SANA-WM batched additive update in place of the VDA write (VDA_SANA_WM)")
    ap.add_argument("--newton", action="store_true",
                    help="(I + A)^-1 by Newton iteration instead of Gauss-Jordan (VDA_NEWTON)")
    ap.add_argument("--softmax", action="store_true",
                    help="time the softmax window + anchor + text branch instead of the linear branch")
    ap.add_argument("--copy-calibration", action="store_true")
    ap.add_argument("--traffic", nargs=4, metavar=("FETCH", "WRITE", "COPY_FETCH", "COPY_WRITE"))
    args = ap.parse_args()
    if args.traffic:
        write_traffic(*args.traffic)
        return
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (--gpus {args.gpus} requested): libvda runs and is "
              "measured on a single MI355X; heads would shard across GPUs with no communication, "
              "but no multi-GPU path exists here.", file=sys.stderr)
        sys.exit(2)
    if args.copy_calibration:
        copy_calibration()
        return
    if args.softmax:
        softmax_bench(args)
        return

    import torch
    from frame_wise_delta_amd import inputs as inp
    from frame_wise_delta_amd import runner, vda

    cfg = inp.CONFIG_BY_NAME[args.config]
    t0 = time.time()
    heads_in = inp.all_raw_heads(cfg) if args.prep else inp.all_heads(cfg)
    print(f"[bench] inputs for {cfg.name} drawn in {time.time() - t0:.1f}s", file=sys.stderr, flush=True)
    desc = vda.desc_for(cfg, prep=args.prep, chunk_scan=args.chunk_scan, sana_wm=args.sana_wm,
                        newton=args.newton)
    dev = runner.upload(cfg, heads_in, "cuda")
    bufs = runner.allocate(desc, cfg.out_dtype, "cuda")
    epi_in, gate, norm_w = None, None, None
    if args.epilogue:
        epi_in = [inp.epilogue_inputs(cfg, h) for h in range(cfg.heads)]
        gate, norm_w = runner.upload_epilogue(cfg, epi_in)
    main_s = torch.cuda.current_stream()

    # the calls of a step, as named in call_ms
    names = ["prepare"] + (["compose"] if args.chunk_scan else []) + ["scans", "readout"]

    def step(pairs=None):
        """One step; with pairs (event pairs per call) each call is bracketed
        by HIP events recorded on the stream it runs on."""
        x, b = dev, bufs

        def mark(k, i):
            if pairs is not None:
                pairs[k][i].record(main_s)
        mark("prepare", 0)
        vda.vda_prepare_frames(desc, x.k, x.v, x.beta, x.kt, x.vt, x.bt, b.ws, b.ws_bytes, stream=main_s)
        mark("prepare", 1)
        if args.chunk_scan:
            mark("compose", 0)
            vda.vda_compose_chunks(desc, b.ws, x.alpha, ws_bytes=b.ws_bytes, stream=main_s)
            mark("compose", 1)
        mark("scans", 0)
        vda.vda_scan_bidir(desc, b.ws, x.alpha, None, b.states_f, b.states_r, stream=main_s)
        mark("scans", 1)
        mark("readout", 0)
        if args.epilogue:
            vda.vda_readout_gated(desc, x.q, x.alpha, b.states_f, b.states_r, gate, norm_w, EPS, b.out,
                                  stream=main_s)
        else:
            vda.vda_readout(desc, x.q, x.alpha, b.states_f, b.states_r, b.out, stream=main_s)
        mark("readout", 1)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    print(f"[bench] warmup {args.warmup} steps done", file=sys.stderr, flush=True)
    # the timed region: K steps back to back, nothing else on the stream
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    t_total = time.perf_counter() - t0
    status = vda.vda_device_status(desc, bufs.ws)
    ms_step = 1e3 * t_total / args.steps
    # per-call times: K more steps with an event pair (created beforehand)
    # around every call; the events themselves cost ~30 us per step, so this
    # pass gives the kernels' durations, not the step time
    pairs = [{k: (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for k in names}
             for _ in range(args.steps)]
    for i in range(args.steps):
        step(pairs[i])
    torch.cuda.synchronize()
    kms = {k: float(np.mean([pr[k][0].elapsed_time(pr[k][1]) for pr in pairs])) for k in names}
    print(f"[bench] {args.steps} steps: {ms_step:.3f} ms/step; calls {kms}", file=sys.stderr, flush=True)

    # cold steps: a 512 MiB buffer is written before each step (outside the
    # events), so the L2s and the 256 MB MALL hold none of the step's data
    flush = torch.empty(512 * 1024 * 1024 // 4, dtype=torch.float32, device="cuda")
    cold = []
    for i in range(min(args.steps, 20)):
        flush.fill_(float(i))
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(main_s)
        step()
        e1.record(main_s)
        torch.cuda.synchronize()
        cold.append(e0.elapsed_time(e1))
    del flush
    # the read bandwidth of a plain streaming kernel on this device: 4 GiB,
    # the best of four grid sizes (2 to 128 workgroups of 256 threads per CU)
    src = torch.ones(4 * 1024 * 1024 * 1024 // 4, dtype=torch.float32, device="cuda")
    stream_gbs = 0.0
    for blocks in (512, 2048, 8192, 32768):
        sink = torch.empty(blocks, dtype=torch.int32, device="cuda")
        vda.vda_stream_read(src, sink, blocks)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(main_s)
        for _ in range(5):
            vda.vda_stream_read(src, sink, blocks)
        e1.record(main_s)
        torch.cuda.synchronize()
        stream_gbs = max(stream_gbs, 5 * src.numel() * 4 / (e0.elapsed_time(e1) / 1e3) / 1e9)
        del sink
    del src
    print(f"[bench] cold steps median {np.median(cold):.3f} ms; stream read {stream_gbs:.0f} GB/s", file=sys.stderr,
          flush=True)

    flops, nbytes, flops_two = algorithmic_work(cfg, args.epilogue)
    t_s = ms_step / 1e3
    kb = kernel_bytes(cfg)
    rk = "readout_gated" if args.epilogue else "readout_kernel"
    # the prepare call is one kernel (frame_kernel) on the path; for the
    # comparators it is the statistics kernel followed by their own kernel
    pk = "stats_kernel" if (args.sana_wm or args.newton) else "frame_kernel"
    kb = {k: kb[k] for k in (pk, rk)}
    call_of = {pk: "prepare", rk: "readout"}
    dom = max(kb, key=lambda k: kms[call_of[k]])
    ach = kb[dom] / (kms[call_of[dom]] / 1e3) / 1e9
    roofline = {"kernel": dom, "bound": "hbm", "achieved": round(ach, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": round(ach / PEAK_HBM_GBS, 4), "traffic": None if args.prep else _traffic(dom),
                "algorithmic_bytes_per_launch": kb[dom], "avg_ms": round(kms[call_of[dom]], 4)}

    cpu, rel = None, None
    if not args.no_cpu_baseline:
        out0 = bufs.out[0].float().cpu().numpy().astype(np.float64)
        cpu, rel = cpu_baseline(cfg, heads_in, out0, args.cpu_seconds, epi_in, args.prep,
                                "sana" if args.sana_wm else "vda")

    out = {
        "metric": "VDA scan+readout latent frames/s and % of MI355X bf16 MFMA peak",
        "value": round(cfg.frames / t_s, 2),
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
                               f"chunk), U={cfg.tokens}, {cfg.text_tokens} text tokens"
                               + (", readout epilogue (RMSNorm + sigmoid gate)" if args.epilogue else "")
                               + (", raw inputs prepared in the kernels" if args.prep else "")
                               + (", chunk-level scans from composed chunk maps" if args.chunk_scan else "")
                               + (", SANA-WM batched additive update (comparator)" if args.sana_wm else "")
                               + (", Newton-iteration inverse" if args.newton else ""),
                   "epilogue": bool(args.epilogue), "prep": bool(args.prep), "chunk_scan": bool(args.chunk_scan),
                   "sana_wm": bool(args.sana_wm), "newton": bool(args.newton),
                   "heads": cfg.heads, "d": cfg.d, "frames": cfg.frames, "tokens": cfg.tokens,
                   "text_tokens": cfg.text_tokens, "in_dtype": cfg.in_dtype, "out_dtype": cfg.out_dtype,
                   "state_dtype": "f32", "global_batch": 1, "seq_len": cfg.frames * cfg.tokens,
                   "parallelism": "single GPU"},
        "tflops_algorithmic": round(flops / t_s / 1e12, 2),
        "mfma_peak_frac": round(flops / t_s / 1e12 / PEAK_BF16_TFLOPS, 4),
        "flop_count": "readout as one product with the merged operand (2Ud^2 per frame-head)",
        "tflops_algorithmic_two_reads": round(flops_two / t_s / 1e12, 2),
        "mfma_peak_frac_two_reads": round(flops_two / t_s / 1e12 / PEAK_BF16_TFLOPS, 4),
        "hbm_frac_path": round(nbytes / t_s / 1e9 / PEAK_HBM_GBS, 4),
        "call_ms": {k: round(v, 4) for k, v in kms.items()},
        "cold": {"ms_per_step_median": round(float(np.median(cold)), 4),
                 "ms_per_step_min": round(float(np.min(cold)), 4), "steps": len(cold),
                 "frames_per_s": round(cfg.frames / (float(np.median(cold)) / 1e3), 2),
                 "flush": "512 MiB written before each step, outside the timed events"},
        "stream_read_gbs": round(stream_gbs, 1),
        "roofline": roofline,
        "cpu_baseline": cpu,
        "rel_l2_head0": rel,
        "device_status": status,
    }
    print(json.dumps(out))


if __name__ == "__main__":
    main()
