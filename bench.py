#!/usr/bin/env python3
"""Benchmark of the SSD chunked forward on one MI355X.

One "step" is one ssd_forward over one batch of the 2.7B-shaped workload
(b = 1, L = 64K tokens, H = 80 heads, P = 64, N = 128, one group, bf16 inputs,
fp32 decay/accumulation), with every input already resident in HBM.  The timed
region is exactly --steps forward calls bracketed by device synchronisation, after
--warmup untimed ones (50 and 50 by default).

The printed JSON line also carries
  * roofline     -- the dominant kernel's algorithmic bytes (or flops) per launch
                    over its average launch duration, timed with HIP events on the
                    stream it runs on, against the MI355X peak;
  * cpu_baseline -- the fp64 oracle timed on this host on a bounded sample;
  * decode       -- 64 back-to-back ssd_step calls on the 2.7B decode shape, the same 64 steps
                    replayed as one graph, and as one ssd_step_multi call (state kept on chip);
  * backward     -- ssd_backward (all gradients) on the same 2.7B workload;
  * selective_scan -- the Mamba-1 selective scan (ssd_selective_scan) on the same width
                    (5120 channels, N = 16, 64K tokens, zero-order hold), with its own ALU
                    roofline and oracle baseline.
"""

from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0  # MI355X HBM3E
PEAK_BF16_TFLOPS = 2500.0  # dense bf16 MFMA
PEAK_FP32_MFMA_TFLOPS = 157.3  # dense fp32 MFMA (the backward's scans with fp32 inputs)
# backward FLOP per token-head in its recurrence form: state recompute (3PN), adjoint update (3PN) and
# the four contractions G.B, G^T.x, S^T.dy and <G, S> (2PN each)
BWD_FLOP_PER_TOKEN_HEAD_PN = 14
# fp32 VALU issue rate without packed math: 256 CUs x 4 SIMDs x 16 lanes x 2.4 GHz, in G lane-ops/s
PEAK_VALU_GOPS = 256 * 4 * 16 * 2.4
# lane operations of one selective-scan element update (token, channel, state entry) in its
# cheapest form: delta*A, exp2, B*x, add, fma (state), C/A scale, fma (output)
SEL_OPS_PER_ELEMENT = 7
# fp32 lane operations per state element and decode step: decay multiply, input fma, output fma
STEP_OPS = 3
METRIC = "SSD fwd tokens/s + % MFMA/HBM roofline (2.7B heads, L 1K–256K, N 64–512)"


def backward_section(ssd, torch, dev, timed, args, cfg, x, dt, A, B, C, D, tokens):
    """Time ssd_backward (every gradient) on the forward's workload; returns the bench object."""
    b, L, H, P = x.shape
    N, G = B.shape[3], B.shape[2]
    tdt = x.dtype
    gen = torch.Generator(device=dev).manual_seed(11)
    gdy = torch.randn(x.shape, generator=gen, device=dev, dtype=torch.float32).to(tdt)
    gdf = torch.randn((b, H, P, N), generator=gen, device=dev, dtype=torch.float32)
    bws = torch.empty(max(ssd.backward_workspace_bytes(x, B, 0), 1), dtype=torch.uint8, device=dev)

    def bwd():
        ssd.backward(x, dt, A, B, C, D, None, gdy, gdf, workspace=bws)

    bwd_ms = timed(bwd, max(3, args.steps // 4))
    bflop = BWD_FLOP_PER_TOKEN_HEAD_PN * P * N * tokens * H
    btf = bflop / (bwd_ms / 1e3) / 1e12
    # bf16 inputs run on the bf16 MFMA kernels (the decay gradient chunk by chunk); fp32 inputs on fp32 MFMA
    peak = PEAK_BF16_TFLOPS if tdt == torch.bfloat16 else PEAK_FP32_MFMA_TFLOPS
    es = x.element_size()
    # minimum bytes: x, dy, dt read and dx, ddt written per token-head; B, C read and dB, dC written per
    # token-group; the final-state gradient and dh0
    min_bytes = b * L * (H * (3 * P * es + 2 * es) + 4 * G * N * es) + 2 * b * H * P * N * 4
    out = {
        "workload": f"{args.workload}: ssd_backward b={b} L={L} H={H} P={P} N={N} G={G} {cfg['dtype']} io, "
                    f"every gradient (dx, ddt, dA, dB, dC, dD, dh0), final-state gradient given",
        "ms_per_call": bwd_ms,
        "tokens_per_s": tokens / (bwd_ms / 1e3),
        "workspace_bytes": int(bws.numel()),
        "roofline": {"kernel": "ssd_backward (whole call: the adjoint and two transposed chunked scans, the "
                               "chunk-local decay gradient, the combine kernels)",
                     "bound": "mfma", "achieved": btf, "peak": peak, "unit": "TFLOP/s",
                     "frac": btf / peak,
                     "flop_per_token_head": BWD_FLOP_PER_TOKEN_HEAD_PN * P * N,
                     "flop_count": "recurrence form: state recompute 3PN, adjoint 3PN, G.B, G^T.x, S^T.dy, <G,S> "
                                   "2PN each, per token-head",
                     "hbm_frac_min_bytes": min_bytes / (bwd_ms / 1e3) / 1e9 / PEAK_HBM_GBS,
                     "min_bytes_per_call": min_bytes},
    }
    log(f"backward: {bwd_ms:.3f} ms/call, {tokens / (bwd_ms / 1e3) / 1e6:.1f} M tok/s, {btf:.1f} TFLOP/s "
        f"(recurrence-form count, {btf / peak:.3f} of the {'bf16' if peak == PEAK_BF16_TFLOPS else 'fp32'} "
        f"MFMA peak), {min_bytes / (bwd_ms / 1e3) / 1e9:.0f} GB/s on the minimum bytes")
    del gdy, gdf, bws
    torch.cuda.empty_cache()
    return out


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    # the GPU's clocks settle within a few tens of milliseconds of steady work: 5 warm-up steps
    # leave the timed forward ~7% slower than 50 do (0.89 against 0.83 ms at 2.7B/64K)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--workload", default="cfg2_64k", help="a forward workload name from synth.CONFIGS")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-selective", action="store_true")
    ap.add_argument("--no-backward", action="store_true")
    ap.add_argument("--backward-only", action="store_true",
                    help="time only ssd_backward on the workload (kernel-trace profiling); prints its object")
    ap.add_argument("--cpu-heads", type=int, default=0, help="heads in the oracle's timed sample (0 = all)")
    ap.add_argument("--sweep", action="store_true",
                    help="time ssd_forward on every forward workload (tiny, 130M, 2.7B at 1K-64K, the long-context "
                         "state-size grid) and print one JSON line with all of them; nothing else runs")
    ap.add_argument("--calib-copy", type=int, default=0, metavar="MIB",
                    help="also run a plain device copy of this many MiB (hardware-counter calibration)")
    return ap.parse_args()


def cpu_model() -> str:
    """The host CPU's model name (lscpu's "Model name", read from /proc/cpuinfo)."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.lower().startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def cold_ms(torch, stream, fn, reps, flush):
    """Median time of fn alone when the 256 MB Infinity Cache holds none of its data: a 512 MiB
    buffer is written before every rep (outside the event pair)."""
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
    for i, (e0, e1) in enumerate(evs):
        flush.fill_(float(i))
        e0.record(stream)
        fn()
        e1.record(stream)
    torch.cuda.synchronize()
    return float(np.median([e0.elapsed_time(e1) for e0, e1 in evs]))


def fwd_flops_per_token(H, P, N, G, Q):
    """Causal algorithmic FLOP per token at chunk Q: H((Q+1)P + 4NP) + G(Q+1)N."""
    return H * ((Q + 1) * P + 4 * N * P) + G * (Q + 1) * N


def fwd_bytes_per_token(H, P, N, G, s_io):
    """Minimum HBM bytes per token: x and y, dt, and B and C once per group."""
    return H * (P * 2 * s_io + s_io) + 2 * G * N * s_io


def kernel_sources_sha(paths) -> str:
    """sha256 over the concatenated kernel sources (the .hip file and the headers it includes)."""
    import hashlib

    h = hashlib.sha256()
    for path in paths:
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()


# the kernels one ssd_forward call launches at dstate <= 128, in order
FWD_LAUNCHES = ["subchunk_decay_kernel", "chunk_state_fast_kernel", "state_passing_kernel", "chunk_scan_fast_kernel"]
# the sources of every kernel the forward launches at the 2.7B shape (dstate 128)
FWD_SOURCES = [os.path.join(ROOT, "mamba_ssd_chunked_05_amd", "csrc", f)
               for f in ("fused.hip", "state_passing.hip", "tiles.hpp", "common.hpp")]


def measured_traffic(kernel_sources, summary: str):
    """HBM bytes per launch from a committed counter summary, or None if the kernel changed since.

    The summary records FETCH_SIZE and WRITE_SIZE per dispatch, already scaled by the factors a
    plain device copy of known size gives for the same counters, and the sha256 of the kernel
    sources they were taken on.
    """
    try:
        fields = {}
        with open(summary) as f:
            for line in f:
                if ":" in line and not line.startswith("#"):
                    k, v = line.split(":", 1)
                    fields[k.strip()] = v.strip()
        if fields.get("source_sha256") != kernel_sources_sha(kernel_sources):
            return None
        return float(fields["traffic_bytes_per_launch"])
    except (OSError, KeyError, ValueError):
        return None


def device_inputs(torch, dev, cfg, seed):
    """The workload's inputs drawn on the device (the recipe of the synthetic inputs, in torch's
    generator instead of NumPy's: the sweep times shapes far too large to draw on the host)."""
    b, L, H, P, N, G = cfg["batch"], cfg["seqlen"], cfg["nheads"], cfg["headdim"], cfg["dstate"], cfg["ngroups"]
    tdt = torch.bfloat16 if cfg["dtype"] == "bf16" else torch.float32
    gen = torch.Generator(device=dev).manual_seed(seed)
    f32 = dict(device=dev, dtype=torch.float32, generator=gen)
    x = torch.randn((b, L, H, P), **f32).to(tdt)
    # dt log-uniform on [1e-3, 0.1], A = -exp(U(0, ln 16)), B, C ~ N(0, 1/N), D ~ N(0, 1)
    dt = torch.exp(torch.empty((b, L, H), device=dev, dtype=torch.float32)
                   .uniform_(math.log(1e-3), math.log(0.1), generator=gen)).to(tdt)
    A = -torch.exp(torch.empty(H, device=dev, dtype=torch.float32).uniform_(0.0, math.log(16.0), generator=gen))
    Bm = (torch.randn((b, L, G, N), **f32) / math.sqrt(N)).to(tdt)
    Cm = (torch.randn((b, L, G, N), **f32) / math.sqrt(N)).to(tdt)
    D = torch.randn(H, **f32)
    return x, dt, A, Bm, Cm, D


def sweep(args, torch, ssd, dev):
    """ssd_forward on every forward workload, warm and cold, each with its roofline fraction."""
    from synth import CONFIGS, seed_for
    stream = torch.cuda.current_stream(dev)
    flush = torch.empty(128 << 20, dtype=torch.float32, device=dev)
    out = []
    names = [n for n in CONFIGS if n != "cfg4"]
    for name in names:
        cfg = CONFIGS[name]
        b, L, H, P, N, G = (cfg[k] for k in ("batch", "seqlen", "nheads", "headdim", "dstate", "ngroups"))
        s_io = 2 if cfg["dtype"] == "bf16" else 4
        x, dt, A, Bm, Cm, D = device_inputs(torch, dev, cfg, seed_for(name))
        y = torch.empty_like(x)
        fin = torch.empty((b, H, P, N), dtype=torch.float32, device=dev)
        ws = torch.empty(max(ssd.forward_workspace_bytes(x, Bm, 0), 1), dtype=torch.uint8, device=dev)

        def fwd():
            ssd.forward(x, dt, A, Bm, Cm, D, None, chunk=0, y=y, final_state=fin, workspace=ws)

        for _ in range(10):
            fwd()
        torch.cuda.synchronize()
        # enough reps for about half a second, at least 10
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        fwd()
        e1.record(stream)
        torch.cuda.synchronize()
        reps = max(10, min(2000, int(500.0 / max(e0.elapsed_time(e1), 1e-3))))
        e0.record(stream)
        for _ in range(reps):
            fwd()
        e1.record(stream)
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / reps
        cold = cold_ms(torch, stream, fwd, 10, flush)
        tokens = b * L
        flop = fwd_flops_per_token(H, P, N, G, cfg["chunk"]) * tokens
        nbytes = fwd_bytes_per_token(H, P, N, G, s_io) * tokens + b * H * P * N * 4
        peak_flop = (PEAK_BF16_TFLOPS if s_io == 2 else PEAK_FP32_MFMA_TFLOPS) * 1e12
        ceiling = min(peak_flop, flop / nbytes * PEAK_HBM_GBS * 1e9)  # flop/s the roofline allows
        rate = flop / (ms / 1e3)
        out.append({
            "workload": name, "shape": dict(b=b, L=L, H=H, P=P, N=N, G=G, dtype=cfg["dtype"]),
            "chunk": ssd.query_config(b, L, H, P, N, G, 0, x.dtype)["chunk"],
            "ms": ms, "cold_ms": cold, "tokens_per_s": tokens / (ms / 1e3),
            "tflops_algorithmic": rate / 1e12, "mfma_frac": rate / peak_flop,
            "gbs_min_bytes": nbytes / (ms / 1e3) / 1e9, "hbm_frac": nbytes / (ms / 1e3) / 1e9 / PEAK_HBM_GBS,
            "intensity_flop_per_byte": flop / nbytes,
            "bound": "mfma" if ceiling >= peak_flop else "hbm",
            "roofline_frac": rate / ceiling,
        })
        log(f"{name}: {ms:.3f} ms (cold {cold:.3f}), {tokens / (ms / 1e3) / 1e6:.1f} M tok/s, "
            f"{rate / 1e12:.1f} TFLOP/s, roofline {rate / ceiling:.3f} ({out[-1]['bound']})")
        del x, dt, A, Bm, Cm, D, y, fin, ws
        torch.cuda.empty_cache()
    print(json.dumps({"sweep": out, "method": "ssd_forward (chunk chosen by the library), inputs drawn on the "
                      "device with the synthetic recipe; warm: mean over about 0.5 s of back-to-back calls; cold: "
                      "median of 10 calls each after a 512 MiB cache-evicting write; FLOP at the workload's "
                      "chunk of 256 (causal), bytes = x, y, dt, B, C once plus the final state"}), flush=True)


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              f"(the forward shards over batch, heads or sequence segments, see the design notes)",
              file=sys.stderr)
        sys.exit(2)

    import torch

    import mamba_ssd_chunked_05_amd as ssd
    from synth import CONFIGS, make_config_inputs, make_step_inputs, seed_for

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    ssd.load()
    dev = torch.device("cuda:0")
    if args.sweep:
        sweep(args, torch, ssd, dev)
        return
    cfg = CONFIGS[args.workload]
    b, L, H, P, N, G = cfg["batch"], cfg["seqlen"], cfg["nheads"], cfg["headdim"], cfg["dstate"], cfg["ngroups"]
    tdt = torch.bfloat16 if cfg["dtype"] == "bf16" else torch.float32
    s_io = 2 if cfg["dtype"] == "bf16" else 4

    log(f"generating {args.workload}: b={b} L={L} H={H} P={P} N={N} G={G} {cfg['dtype']}")
    t0 = time.time()
    fi = make_config_inputs(args.workload)

    def t(a, dtype=tdt):
        return None if a is None else torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(dtype).to(dev)

    x, dt, B, C = t(fi.x), t(fi.dt), t(fi.B), t(fi.C)
    A, D = t(fi.A, torch.float32), t(fi.D, torch.float32)
    log(f"inputs resident in HBM ({time.time() - t0:.1f}s)")
    if args.backward_only:
        stream0 = torch.cuda.current_stream(dev)

        def timed0(fn, reps):
            for _ in range(min(args.warmup, 3)):
                fn()
            ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            ev0.record(stream0)
            for _ in range(reps):
                fn()
            ev1.record(stream0)
            torch.cuda.synchronize()
            return ev0.elapsed_time(ev1) / reps

        print(json.dumps({"backward": backward_section(ssd, torch, dev, timed0, args, cfg, x, dt, A, B, C, D, b * L)}),
              flush=True)
        return
    if args.calib_copy:
        nbytes = args.calib_copy << 20
        src = torch.empty(nbytes // 4, dtype=torch.float32, device=dev).fill_(1.0)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        log(f"calibration copy: 3 x {args.calib_copy} MiB read + written")
        del src, dst

    qcfg = ssd.query_config(b, L, H, P, N, G, 0, tdt)
    Q = qcfg["chunk"]
    y = torch.empty_like(x)
    fin = torch.empty((b, H, P, N), dtype=torch.float32, device=dev)
    ws = torch.empty(max(ssd.forward_workspace_bytes(x, B, 0), 1), dtype=torch.uint8, device=dev)

    def step():
        ssd.forward(x, dt, A, B, C, D, None, chunk=0, y=y, final_state=fin, workspace=ws)

    stream_f = torch.cuda.current_stream(dev)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    ev_a, ev_b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t_start = time.perf_counter()
    ev_a.record(stream_f)  # the forward's kernels all run on this stream
    for _ in range(args.steps):
        step()
    ev_b.record(stream_f)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t_start
    ms = elapsed * 1e3 / args.steps
    ev_ms = ev_a.elapsed_time(ev_b) / args.steps  # HIP events over the timed region, per forward
    # per-call spread, after the timed region: each call bracketed by its own HIP events
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(30)]
    for e0, e1 in evs:
        e0.record(stream_f)
        step()
        e1.record(stream_f)
    torch.cuda.synchronize()
    per_call = sorted(e0.elapsed_time(e1) for e0, e1 in evs)
    tokens = b * L
    tok_s = tokens / (ms / 1e3)
    flops = fwd_flops_per_token(H, P, N, G, cfg["chunk"]) * tokens
    min_bytes = fwd_bytes_per_token(H, P, N, G, s_io) * tokens + b * H * P * N * 4
    log(f"forward: {ms:.3f} ms/step, {tok_s / 1e6:.1f} M tok/s, {flops / (ms / 1e3) / 1e12:.1f} TFLOP/s algorithmic; "
        f"per call median {per_call[len(per_call) // 2]:.3f}, min {per_call[0]:.3f} ms")

    # ---- the forward's stages, each timed alone on the stream it runs on ----------------------
    # ssd_forward is exactly these four calls at chunk Q; the chunk scan dominates.
    stream = torch.cuda.current_stream(dev)
    dt_t, cs = ssd.chunk_cumsum(dt, A, Q)
    states = ssd.chunk_state(x, B, dt_t, cs, Q)
    ssd.state_passing(states, cs, None, seqlen=L, chunk=Q, io=tdt)
    ys = torch.empty_like(x)

    def timed(fn, reps):
        for _ in range(min(args.warmup, 3)):
            fn()
        ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        ev0.record(stream)
        for _ in range(reps):
            fn()
        ev1.record(stream)
        torch.cuda.synchronize()
        return ev0.elapsed_time(ev1) / reps

    scan_ms = timed(lambda: ssd.chunk_scan(x, B, C, dt_t, cs, states, D, chunk=Q, y=ys), args.steps)
    # the forward with a cold Infinity Cache (a 512 MiB write before each rep)
    flush = torch.empty(128 << 20, dtype=torch.float32, device=dev)
    cold = {"method": "a 512 MiB buffer written before every rep (evicts the 256 MB Infinity Cache); "
                      "median over the reps, each rep timed alone with HIP events on the call's stream"}
    cold["forward_ms"] = cold_ms(torch, stream, step, 10, flush)
    stage_ms = {
        "chunk_cumsum": timed(lambda: ssd.chunk_cumsum(dt, A, Q), args.steps),
        "chunk_state": timed(lambda: ssd.chunk_state(x, B, dt_t, cs, Q), args.steps),
        "chunk_scan": scan_ms,
    }
    scratch = states.clone()
    stage_ms["state_passing"] = timed(lambda: ssd.state_passing(scratch, cs, None, seqlen=L, chunk=Q, io=tdt),
                                      args.steps)
    log(f"staged calls at the forward's chunk, each alone (ms): " + ", ".join(f"{k} {v:.3f}" for k, v in stage_ms.items()))
    cold["forward_tokens_per_s"] = tokens / (cold["forward_ms"] / 1e3)
    cold["forward_hbm_frac_min_bytes"] = min_bytes / (cold["forward_ms"] / 1e3) / 1e9 / PEAK_HBM_GBS
    log(f"cold cache: forward {cold['forward_ms']:.3f} ms")
    del states, dt_t, cs, ys, scratch
    torch.cuda.empty_cache()

    result = {
        "metric": METRIC,
        "value": tok_s,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": cfg["dtype"],
        "data": "synthetic (seeded; x~N(0,1), dt log-uniform [1e-3,0.1], A=-exp(U(0,ln16)), B,C~N(0,1)/sqrt(N), D~N(0,1))",
        "config": {"workload": f"{args.workload}: SSD forward b={b} L={L} H={H} P={P} N={N} G={G} "
                               f"{cfg['dtype']} (Mamba-2 2.7B heads)" if args.workload.startswith("cfg2")
                   else f"{args.workload}: SSD forward b={b} L={L} H={H} P={P} N={N} G={G} {cfg['dtype']}",
                   "chunk": Q, "global_batch": b, "seq_len": L, "parallelism": "single GPU"},
        "throughput": {
            "tflops_algorithmic": flops / (ms / 1e3) / 1e12,
            "mfma_frac_algorithmic": flops / (ms / 1e3) / 1e12 / PEAK_BF16_TFLOPS,
            "gbs_min_bytes": min_bytes / (ms / 1e3) / 1e9,
            "hbm_frac_min_bytes": min_bytes / (ms / 1e3) / 1e9 / PEAK_HBM_GBS,
            "flop_per_token": fwd_flops_per_token(H, P, N, G, cfg["chunk"]),
            "min_bytes_per_token": fwd_bytes_per_token(H, P, N, G, s_io),
        },
        "forward_ms_per_call": {"median": per_call[len(per_call) // 2], "min": per_call[0], "max": per_call[-1],
                                "calls": len(per_call)},
        "stage_ms": stage_ms,
        "cold": cold,
        "roofline": {
            "kernel": "ssd_forward (the whole call)",
            "launches": FWD_LAUNCHES,
            "bound": "hbm",
            "achieved": min_bytes / (ev_ms / 1e3) / 1e9,
            "peak": PEAK_HBM_GBS,
            "unit": "GB/s",
            "frac": min_bytes / (ev_ms / 1e3) / 1e9 / PEAK_HBM_GBS,
            "traffic": measured_traffic(FWD_SOURCES,
                                        os.path.join(ROOT, "profiles", f"forward_{args.workload}_traffic.txt")),
            "avg_launch_ms": ev_ms,
            "algorithmic_bytes_per_launch": min_bytes,
            "algorithmic_bytes": "x, y, dt, B, C once each plus the fp32 final state: "
                                 "H(P(s_x+s_y)+s_dt) + 2GN s_bc bytes per token, + b H P N 4",
            "mfma_frac_algorithmic": flops / (ev_ms / 1e3) / 1e12 / PEAK_BF16_TFLOPS,
        },
    }

    # ---- decode: 64 back-to-back ssd_step calls on the 2.7B decode shape ------------------------
    if not args.no_decode:
        c4 = CONFIGS["cfg4"]
        si = make_step_inputs(c4["batch"], c4["nheads"], c4["headdim"], c4["dstate"], c4["ngroups"],
                              steps=c4["steps"], dtype=c4["dtype"], seed=seed_for("cfg4"))
        S = t(si.state0, torch.float32)
        sx = [t(si.x[i]) for i in range(c4["steps"])]
        sdt = [t(si.dt[i]) for i in range(c4["steps"])]
        sB = [t(si.B[i]) for i in range(c4["steps"])]
        sC = [t(si.C[i]) for i in range(c4["steps"])]
        sA, sD = t(si.A, torch.float32), t(si.D, torch.float32)
        yo = [torch.empty_like(sx[0]) for _ in range(c4["steps"])]
        for i in range(8):
            ssd.step(S, sx[i], sdt[i], sA, sB[i], sC[i], sD, y=yo[i])
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for i in range(c4["steps"]):
            ssd.step(S, sx[i], sdt[i], sA, sB[i], sC[i], sD, y=yo[i])
        e1.record(stream)
        torch.cuda.synchronize()
        step_ms = e0.elapsed_time(e1) / c4["steps"]
        bb, hh, pp, nn, gg = c4["batch"], c4["nheads"], c4["headdim"], c4["dstate"], c4["ngroups"]
        step_bytes = 2 * bb * hh * pp * nn * 4 + bb * hh * (pp * 2 * 2 + 2) + 2 * bb * gg * nn * 2
        gbs = step_bytes / (step_ms / 1e3) / 1e9
        nst = c4["steps"]
        # the same 64 steps as one CUDA/HIP graph of ssd_step launches (no host work between steps)
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            for i in range(nst):
                ssd.step(S, sx[i], sdt[i], sA, sB[i], sC[i], sD, y=yo[i])
        graph.replay()
        torch.cuda.synchronize()
        e0.record(stream)
        for _ in range(3):
            graph.replay()
        e1.record(stream)
        torch.cuda.synchronize()
        graph_ms = e0.elapsed_time(e1) / (3 * nst)
        # ... and as one ssd_step_multi call over the pre-staged inputs, the state kept on chip
        xm, dtm = torch.stack(sx, dim=1).contiguous(), torch.stack(sdt, dim=1).contiguous()
        Bm, Cm = torch.stack(sB, dim=1).contiguous(), torch.stack(sC, dim=1).contiguous()
        ym = torch.empty_like(xm)
        for _ in range(2):
            ssd.step_multi(S, xm, dtm, sA, Bm, Cm, sD, y=ym)
        reps = 10
        e0.record(stream)
        for _ in range(reps):
            ssd.step_multi(S, xm, dtm, sA, Bm, Cm, sD, y=ym)
        e1.record(stream)
        torch.cuda.synchronize()
        multi_ms = e0.elapsed_time(e1) / reps
        multi_bytes = 2 * bb * hh * pp * nn * 4 + nst * (step_bytes - 2 * bb * hh * pp * nn * 4)
        # one step with a cold Infinity Cache: the state streams from HBM
        ic = [0]

        def one_step():
            i = ic[0] % nst
            ic[0] += 1
            ssd.step(S, sx[i], sdt[i], sA, sB[i], sC[i], sD, y=yo[i])

        # cold, interleaved rep by rep with the same in-place read-modify-write of a buffer of the
        # state's size (ssd_bench_rmw_stream: the step's state bytes and nothing else), so both see the
        # same clocks: the rate this chip achieves for the step's access pattern
        rmw_buf = torch.zeros_like(S)
        st_evs, rmw_evs = [], []
        for i in range(32):
            for fn, evl in ((one_step, st_evs), (lambda: ssd.bench_rmw_stream(rmw_buf), rmw_evs)):
                flush.fill_(float(i))
                e_a, e_b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e_a.record(stream)
                fn()
                e_b.record(stream)
                evl.append((e_a, e_b))
        torch.cuda.synchronize()
        cold_step_ms = float(np.median([a.elapsed_time(b) for a, b in st_evs]))
        rmw_ms = float(np.median([a.elapsed_time(b) for a, b in rmw_evs]))
        rmw_min_ms = float(np.min([a.elapsed_time(b) for a, b in rmw_evs]))
        rmw_bytes = 2 * rmw_buf.numel() * 4
        del rmw_buf
        cold_gbs = step_bytes / (cold_step_ms / 1e3) / 1e9
        multi_gbs = multi_bytes / (multi_ms / 1e3) / 1e9
        multi_gops = STEP_OPS * bb * hh * pp * nn * nst / (multi_ms / 1e3) / 1e9
        result["decode"] = {
            "workload": f"cfg4: ssd_step b={bb} H={hh} P={pp} N={nn} bf16 io, fp32 state, 64 steps",
            "us_per_step": step_ms * 1e3,
            "tokens_per_s": bb / (step_ms / 1e3),
            "roofline": {"kernel": "step_lane_kernel<bf16> (dstate 128: 32 lanes per state row)", "bound": "hbm", "achieved": gbs, "peak": PEAK_HBM_GBS,
                         "unit": "GB/s", "frac": gbs / PEAK_HBM_GBS, "algorithmic_bytes_per_launch": step_bytes},
            "note": "the 168 MB state fits the 256 MB Infinity Cache, so back-to-back steps can exceed HBM rate; "
                    "the cold object times single steps after a 512 MiB cache-evicting write",
            "cold": {"us_per_step": cold_step_ms * 1e3, "achieved_gbs": cold_gbs,
                     "frac": cold_gbs / PEAK_HBM_GBS,
                     "rmw_ceiling": {
                         "what": "ssd_bench_rmw_stream: in-place fp32 read-modify-write of a buffer the size of "
                                 "the state (the step's state bytes, none of its other work), timed cold, "
                                 "interleaved rep by rep with the step",
                         "us_median": rmw_ms * 1e3, "us_min": rmw_min_ms * 1e3,
                         "gbs_median": rmw_bytes / (rmw_ms / 1e3) / 1e9,
                         "frac_of_hbm_peak": rmw_bytes / (rmw_ms / 1e3) / 1e9 / PEAK_HBM_GBS,
                         "step_time_over_ceiling": cold_step_ms / rmw_ms}},
            "graph_us_per_step": graph_ms * 1e3,
            "multi_step": {
                "call": f"ssd_step_multi, {nst} pre-staged steps per call, state in registers across steps",
                "us_per_call": multi_ms * 1e3,
                "us_per_step": multi_ms * 1e3 / nst,
                "tokens_per_s": bb * nst / (multi_ms / 1e3),
                "hbm_gbs_algorithmic": multi_gbs,
                "roofline": {"kernel": "step_multi_kernel (state in registers across the steps)", "bound": "alu",
                             "achieved": multi_gops, "peak": PEAK_VALU_GOPS, "unit": "Gop/s",
                             "frac": multi_gops / PEAK_VALU_GOPS, "ops_per_state_element_step": STEP_OPS,
                             "traffic": None},
            },
        }
        log(f"decode cold: {cold_step_ms * 1e3:.1f} us/step, {cold_gbs:.0f} GB/s algorithmic; read-modify-write "
            f"ceiling {rmw_ms * 1e3:.1f} us ({rmw_bytes / (rmw_ms / 1e3) / 1e9:.0f} GB/s)")
        log(f"decode: {step_ms * 1e3:.1f} us/step, {gbs:.0f} GB/s algorithmic; graph {graph_ms * 1e3:.1f} us/step; "
            f"multi-step {multi_ms * 1e3 / nst:.2f} us/step ({multi_gbs:.0f} GB/s algorithmic)")

    # ---- backward pass on the same workload --------------------------------------------------------
    if not args.no_backward:
        result["backward"] = backward_section(ssd, torch, dev, timed, args, cfg, x, dt, A, B, C, D, tokens)

    # ---- Mamba-1 selective scan on the same width ------------------------------------------------
    if not args.no_selective:
        from synth import SELECTIVE_CONFIGS, make_selective_config_inputs

        sname = "mamba1_5120ch_64k"
        sc = SELECTIVE_CONFIGS[sname]
        t0 = time.time()
        si = make_selective_config_inputs(sname)
        sdt_ = torch.bfloat16 if sc["dtype"] == "bf16" else torch.float32
        ux, ud, uB, uC = t(si.x, sdt_), t(si.delta, sdt_), t(si.B, sdt_), t(si.C, sdt_)
        uA, uD = t(si.A, torch.float32), t(si.D, torch.float32)
        log(f"selective workload resident ({time.time() - t0:.1f}s)")
        sb, sL, sDc = ux.shape
        sN = uB.shape[-1]
        fe = ssd.Frontend(zoh=True)
        uy = torch.empty_like(ux)
        ufin = torch.empty((sb, sDc, sN), dtype=torch.float32, device=dev)
        uws_n = ssd.selective_scan_workspace_bytes(sb, sL, sDc, sN, uB.shape[2], dtype=sdt_)
        uws = torch.empty(max(uws_n, 1), dtype=torch.uint8, device=dev)

        def sel():
            ssd.selective_scan(ux, ud, uA, uB, uC, uD, None, y=uy, final_state=ufin, workspace=uws, frontend=fe)

        sel_ms = timed(sel, args.steps)
        elems = sb * sL * sDc * sN
        gops = elems * SEL_OPS_PER_ELEMENT / (sel_ms / 1e3) / 1e9
        sel_bytes = sb * sL * sDc * 3 * (2 if sc["dtype"] == "bf16" else 4) + 2 * sb * sL * uB.shape[2] * sN * 2
        result["selective_scan"] = {
            "workload": f"{sname}: Mamba-1 selective scan b={sb} L={sL} channels={sDc} N={sN} G={uB.shape[2]} "
                        f"{sc['dtype']} io, fp32 state, zero-order hold",
            "ms_per_call": sel_ms,
            "tokens_per_s": sb * sL / (sel_ms / 1e3),
            "element_updates_per_s": elems / (sel_ms / 1e3),
            "hbm_gbs_min_bytes": sel_bytes / (sel_ms / 1e3) / 1e9,
            "roofline": {"kernel": "ssd_selective_scan (whole call: first pass, carry, output pass)",
                         "bound": "alu", "achieved": gops, "peak": PEAK_VALU_GOPS, "unit": "Gop/s",
                         "frac": gops / PEAK_VALU_GOPS, "ops_per_element": SEL_OPS_PER_ELEMENT,
                         "traffic": None},
        }
        log(f"selective scan: {sel_ms:.3f} ms/call, {elems / (sel_ms / 1e3) / 1e12:.2f} T element updates/s, "
            f"{gops / PEAK_VALU_GOPS:.2f} of the VALU issue rate")
        if not args.no_cpu_baseline:
            import oracle

            ch = list(range(0, sDc, max(1, sDc // 256)))[:256]
            t1 = time.perf_counter()
            oracle.selective_scan(si.x[:, :, ch], si.delta[:, :, ch], si.A[ch], si.B, si.C, si.D[ch], None, zoh=True)
            cpu_s = time.perf_counter() - t1
            result["selective_scan"]["cpu_baseline"] = {
                "value": sb * sL * len(ch) / sDc / cpu_s, "unit": "tokens/s", "cores": oracle.max_threads(),
                "kind": "oracle",
                "sample": f"{len(ch)} of {sDc} channels over all {sL} tokens; tokens/s scaled to all channels "
                          f"({cpu_s:.1f} s, fp64 recurrence, OpenMP over (b, channel))",
            }
        del si, ux, ud, uB, uC, uy, uws
        torch.cuda.empty_cache()

    # ---- CPU baseline: the fp64 oracle on a bounded sample of the same workload ----------------
    if not args.no_cpu_baseline:
        import oracle

        hs = list(range(min(args.cpu_heads, H) if args.cpu_heads > 0 else H))
        xs, dts = fi.x[:, :, hs], fi.dt[:, :, hs]
        t1 = time.perf_counter()
        oracle.forward(xs, dts, fi.A[hs], fi.B, fi.C, fi.D[hs], None)
        cpu_s = time.perf_counter() - t1
        frac = len(hs) / H
        result["cpu_baseline"] = {
            "value": tokens * frac / cpu_s,
            "unit": "tokens/s",
            "cores": oracle.max_threads(),
            "kind": "oracle",
            "sample": f"{len(hs)} of {H} heads over all {L} tokens (b={b}); tokens/s scaled to all heads "
                      f"({cpu_s:.1f} s, fp64 token recurrence, OpenMP over (b, h))",
        }
        log(f"cpu oracle: {cpu_s:.1f}s for {len(hs)} heads on {oracle.max_threads()} threads")
        result["cpu_baseline"]["model"] = cpu_model()
        # one thread: the tiny and 130M workloads whole, and one head of this workload
        one = {}
        for name in ("cfg0", "cfg1"):
            f1 = make_config_inputs(name)
            t1 = time.perf_counter()
            oracle.forward(f1.x, f1.dt, f1.A, f1.B, f1.C, f1.D, f1.h0, threads=1)
            one[name] = {"tokens_per_s": f1.x.shape[0] * f1.x.shape[1] / (time.perf_counter() - t1),
                         "seconds": time.perf_counter() - t1}
        t1 = time.perf_counter()
        oracle.forward(fi.x[:, :, :1], fi.dt[:, :, :1], fi.A[:1], fi.B, fi.C, fi.D[:1], None, threads=1)
        one_s = time.perf_counter() - t1
        one[f"{args.workload}_1_head"] = {"token_heads_per_s": tokens / one_s, "seconds": one_s}
        result["cpu_baseline"]["one_thread"] = one
        log(f"cpu oracle, one thread: " + ", ".join(f"{k} {v['seconds']:.2f}s" for k, v in one.items()))

    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
