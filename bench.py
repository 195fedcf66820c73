"""Benchmark of the Orthros per-layer attention step on one MI355X.

A step is one orthros_prefill call over the 128K-token, batch-2,
32/8-head workload, with every input already resident in HBM: one pass of
the streaming kernel (base-stream sliding-window attention, the fused
cache write, and the output copy's global query folded in as one partial
per segment), then the LSE merge of those partials.  value = prefill
tokens per second (B * T / time per step).  The decode step latency
(batch 16, lengths U[8192, 131072], 1024 steps) is reported beside it.

Timing: W untimed warm-up calls (30 by default: from idle the GPU's clocks
need about 20 back-to-back calls of this step to ramp up, and calls during
the ramp run 15-20% slower), then K calls bracketed by
torch.cuda.synchronize() and HIP events on the stream the kernels run on
(the library queues its work on torch's current stream).  The roofline figure is for the step's
dominant kernel, the fused streaming kernel: the step's algorithmic bytes
over the step time (the merge that follows it in the same call takes a few
microseconds of that).  The separate entry points orthros_swa_prefill and
orthros_global_xattn are timed too, as a breakdown.  The fp64 CPU oracle is
timed on the same workload on this machine's host cores (cpu_baseline).

Every other workload the library is checked on gets its own leg in
`configs` (rate, algorithmic GB/s and MFMA TFLOP/s, fractions of the
vendor peaks, and the oracle's time on this host, measured in full or
extrapolated from a measured part and labelled so):

  tiny_fp32_prefill     fp32, B1, 4/4 heads, d64, T2048 (a parity workload)
  mha_1p3b_prefill_8k   bf16, B1, 16/16 heads (MHA), d128, T8192
  gqa_8b_prefill_128k   the headline step above
  gqa_8b_prefill_1m     bf16, B1, 32/8, d128, T2^20, 36 layers whose caches
                        (144 GiB) stay resident: the 36-layer total and the
                        per-layer rate
  gqa_8b_decode_b16     the decode step

The projections either side of the attention (orthros_project: the shared
W_Q over the base and copy rows, K/V written into the cache; d_model 4096)
are timed over the same 128K batch as an MFMA-bound leg, the many-copy
modes (orthros_copies) at an SFT span and a PT sequence, and the
multi-layer decode step over 36 resident layers, eager and as one captured
HIP graph.  hbm_practical measures what plain streaming kernels reach on
this GPU (library copy / GEMV / fill, and the read and copy kernels of
libhbmprobe.so swept over unroll and grid sizes).

  python bench.py [--gpus 1] [--steps K] [--warmup W] [--only LEG] [--skip LEG ...]
"""
import argparse
import ctypes
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "prefill attn tokens/s at 128K (SWA w=128 + 1 global query); decode us/step"
PROFILES = os.path.join(ROOT, "profiles")
HBM_PEAK_GBS = 8000.0
BF16_PEAK_TFLOPS = 2500.0
FP32_PEAK_TFLOPS = 157.3
LEGS = ["prefill", "swa", "xattn", "tiny", "mha8k", "prefill1m", "copies", "project", "layers", "decode"]


def swa_bytes(B, T, Hq, Hkv, d, es=2):
    """Algorithmic HBM bytes of one orthros_swa_prefill launch: q read, o
    written, k and v read once, the cache written once."""
    return B * T * (2 * Hq + 4 * Hkv) * d * es


def swa_flops(B, T, Hq, d, w):
    """Algorithmic flops: 4 d per (query, admissible key) (QK^T and PV)."""
    keys = sum(min(t + 1, w) for t in range(min(T, w))) + max(0, T - w) * w
    return 4 * d * B * Hq * keys


def prefill_bytes(B, T, Hq, Hkv, d, es=2):
    """Algorithmic bytes of one orthros_prefill step: those of the SWA pass
    (which also serves the copy's key reads: one pass over K/V), plus the
    copy's query read and its output written."""
    return swa_bytes(B, T, Hq, Hkv, d, es) + 2 * B * Hq * d * es


def xattn_bytes(B, pos_plus_1, Hkv, d, es=2):
    """Algorithmic bytes of the copy's global read: K and V of keys [0, P]."""
    return B * pos_plus_1 * Hkv * d * 2 * es


def prefill_flops(B, T, Hq, d, w):
    """SWA flops plus the copy's 4 d flops per key per query head."""
    return swa_flops(B, T, Hq, d, w) + 4 * d * B * Hq * T


def project_flops(c):
    """Algorithmic flops of orthros_project: 2 d_model per output element;
    base rows against W_Q, W_K and W_V, copy rows against W_Q."""
    nq, nk = c["n_q_heads"] * c["head_dim"], c["n_kv_heads"] * c["head_dim"]
    return 2 * c["d_model"] * c["batch"] * (c["T"] * (nq + 2 * nk) + c["T_out"] * nq)


def measured_traffic(summary):
    """HBM bytes per launch from a committed rocprofv3 counter summary
    (FETCH_SIZE and WRITE_SIZE scaled by a copy kernel's reading), or None
    when the kernel sources changed since those counters were taken."""
    path = os.path.join(PROFILES, summary)
    if not os.path.exists(path):
        return None
    fields = {}
    for line in open(path):
        if ":" in line and not line.startswith(("|", "#", " ")):
            k, v = line.split(":", 1)
            fields[k.strip()] = v.strip()
    if "traffic_bytes_per_launch" not in fields or "sources" not in fields:
        return None
    h = hashlib.sha256()
    for f in fields["sources"].split():
        h.update(open(os.path.join(ROOT, f), "rb").read())
    if h.hexdigest()[:16] != fields.get("source_sha256_16"):
        return None
    return float(fields["traffic_bytes_per_launch"])


def timed(fn, steps, warmup):
    import torch
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    start.record()
    for _ in range(steps):
        fn()
    end.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    return start.elapsed_time(end) / 1e3, wall


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def hbm_fracs(nbytes, flops, sec, peak_tflops=BF16_PEAK_TFLOPS):
    """Algorithmic GB/s and TFLOP/s of `sec` seconds, with the fractions of
    the vendor peaks and of the attainable roofline min(P, I x BW)."""
    gbs = nbytes / sec / 1e9
    tfl = flops / sec / 1e12
    attain = min(peak_tflops, flops / nbytes * HBM_PEAK_GBS / 1e3)
    return {"GBps": gbs, "hbm_frac": gbs / HBM_PEAK_GBS, "TFLOPs": tfl, "mfma_frac": tfl / peak_tflops,
            "intensity_flop_per_byte": flops / nbytes, "attainable_TFLOPs": attain,
            "attainable_frac": tfl / attain}


# ---------------------------------------------------------------- oracle legs

def cpu_baseline(cfg, x_dev, one_thread_rows=128):
    """The fp64 oracle on the whole workload (Eq. (4) for every token and
    head, the cache, and each sequence's global query over all its keys) on
    this host's cores; plus the Eq. (4) rate of a single thread on a short
    run of rows."""
    import torch

    import oracle
    B, T, Hq = cfg["batch"], cfg["T"], cfg["n_q_heads"]
    w = cfg["window"]
    nthreads = oracle.default_threads()
    q = x_dev["q"].cpu().contiguous()
    k = x_dev["k"].cpu().contiguous()
    v = x_dev["v"].cpu().contiguous()
    a, b = x_dev["alpha"].cpu(), x_dev["beta"].cpu()
    s = time.perf_counter()
    oracle.prefill(q, x_dev["q_out"].cpu().contiguous(), [T - 1] * B, k, v, a, b, x_dev["alpha_out"].cpu(),
                   x_dev["beta_out"].cpu(), w, nthreads=nthreads)
    t_all = time.perf_counter() - s
    t0 = T // 2
    n1 = min(one_thread_rows, T - t0)
    rows = torch.tensor([(0, t, h) for t in range(t0, t0 + n1) for h in range(Hq)])
    s = time.perf_counter()
    oracle.swa_rows(q[:1], k[:1], v[:1], a, b, w, rows, nthreads=1)
    t_row1 = (time.perf_counter() - s) / n1            # seconds per token, 1 thread
    return {"value": B * T / t_all, "unit": "tokens/s", "cores": nthreads, "kind": "oracle",
            "seconds": t_all, "extrapolated": False, "cpu_model": cpu_model(),
            "one_thread_swa_tokens_per_s": 1.0 / t_row1,
            "sample": f"fp64 oracle, {nthreads} threads, the whole workload (B={B} x T={T}: Eq. (4) for every "
                      f"token x {Hq} heads, the cache, and the global query over all {T} keys) in {t_all:.2f} s; "
                      f"one thread: Eq. (4) for {n1} tokens x {Hq} heads"}


def cpu_baseline_1m(cfg, x_dev, n_rows=2048):
    """The fp64 oracle on one layer of the 1M workload, measured in part and
    extrapolated: the global query over all 2^20 keys (in full), and Eq. (4)
    on n_rows consecutive mid-sequence tokens x every head, scaled to all T
    tokens; the 36-layer figure is 36 such layers."""
    import torch

    import oracle
    B, T, Hq, d, w, L = (cfg[k] for k in ("batch", "T", "n_q_heads", "head_dim", "window", "layers"))
    nthreads = oracle.default_threads()
    k = x_dev["k"].cpu()
    v = x_dev["v"].cpu()
    ab = [x_dev[n].cpu() for n in ("alpha", "beta", "alpha_out", "beta_out")]
    kc = torch.empty(B, k.shape[2], T, d, dtype=k.dtype)
    vc = torch.empty_like(kc)
    s = time.perf_counter()
    oracle.prefill(None, x_dev["q_out"].cpu(), [T - 1] * B, k, v, *ab, w, swa=False, k_cache=kc, v_cache=vc,
                   nthreads=nthreads)
    t_glob = time.perf_counter() - s
    t0 = T // 2
    ts = torch.arange(t0, t0 + n_rows)
    qrows = x_dev["q"][0, ts.cuda()].reshape(-1, d).cpu()
    rows = torch.stack([torch.zeros_like(ts).repeat_interleave(Hq), ts.repeat_interleave(Hq),
                        torch.arange(Hq).repeat(n_rows)], dim=1)
    s = time.perf_counter()
    oracle.swa_rows_given_q(qrows, k, v, ab[0], ab[1], w, rows, n_q_heads=Hq, nthreads=nthreads)
    t_rows = time.perf_counter() - s
    per_layer = t_glob + t_rows / n_rows * T * B
    return {"value": B * T * L / (per_layer * L), "unit": "tokens/s (per layer)", "cores": nthreads,
            "kind": "oracle", "extrapolated": True, "seconds_per_layer": per_layer,
            "seconds_36_layers": per_layer * L, "cpu_model": cpu_model(),
            "sample": f"fp64 oracle, {nthreads} threads, one layer: the global query over all {T} keys x {Hq} heads "
                      f"measured in full ({t_glob:.2f} s, the cache copy included) and Eq. (4) measured on "
                      f"{n_rows} tokens x {Hq} heads ({t_rows:.2f} s), extrapolated to {T} tokens and to {L} layers"}


def cpu_baseline_decode(cfg, xd, len0, steps=8):
    """The fp64 oracle on the decode workload: a contiguous block of `steps`
    steps from the starting lengths (every sequence's base token over its
    window and its copy over the whole history), on this machine's host
    cores, extrapolated to the workload's step count."""
    import oracle
    steps = min(steps, xd["q"].shape[0])
    kc, vc = xd["k_cache"].cpu(), xd["v_cache"].cpu()
    lc = len0.cpu().to(dtype=len0.dtype).clone()
    a = {k: xd[k].cpu() for k in ("alpha", "beta", "alpha_out", "beta_out")}
    nthreads = oracle.default_threads()
    s = time.perf_counter()
    for i in range(steps):
        oracle.decode_step(xd["q"][i].cpu(), xd["q_out"][i].cpu(), xd["k_new"][i].cpu(), xd["v_new"][i].cpu(),
                           a["alpha"], a["beta"], a["alpha_out"], a["beta_out"], cfg["window"], kc, vc, lc,
                           nthreads=nthreads)
    t = (time.perf_counter() - s) / steps
    total = cfg["steps"]
    return {"value": t * 1e6, "unit": "us/step", "cores": nthreads, "kind": "oracle", "extrapolated": True,
            "measured_steps": steps, "seconds_all_steps_extrapolated": t * total, "cpu_model": cpu_model(),
            "sample": f"fp64 oracle, {nthreads} threads, the first {steps} consecutive steps of the workload "
                      f"(batch {cfg['batch']}, every sequence's window and whole-history copy) measured, "
                      f"{t:.2f} s per step; the {total}-step total ({t * total:.0f} s) is extrapolated from them"}


# ------------------------------------------------------------ practical HBM

def practical_ceilings():
    """HBM rates plain streaming kernels reach on this GPU over 4 GiB:
    PyTorch's copy (read + write), a bf16 matrix-vector product (read) and
    fill (write); and the hand-written read and copy kernels of
    libhbmprobe.so, swept over unroll (16-byte loads in flight per lane) and
    grid size, best of the sweep.  Context for the rooflines, which price
    against the 8 TB/s vendor figure."""
    import torch
    n = 4 << 30
    a = torch.empty(n, dtype=torch.uint8, device="cuda")
    b = torch.empty_like(a)
    a.fill_(1)
    mat = a.view(torch.bfloat16).view(-1, 4096)
    vec = torch.ones(4096, 1, device="cuda", dtype=torch.bfloat16)
    out = {}
    sec, _ = timed(lambda: b.copy_(a), 5, 2)
    out["torch_copy_read_plus_write_GBps"] = 2 * n * 5 / sec / 1e9
    sec, _ = timed(lambda: mat @ vec, 5, 2)
    out["torch_gemv_read_GBps"] = n * 5 / sec / 1e9
    sec, _ = timed(lambda: b.fill_(1), 5, 2)
    out["torch_fill_write_GBps"] = n * 5 / sec / 1e9
    lib = ctypes.CDLL(os.path.join(ROOT, "phase_aware_swa_amd", "libhbmprobe.so"))
    vp, i64, ci = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
    lib.hbm_probe_read.argtypes = [vp, i64, vp, ci, ci, vp]
    lib.hbm_probe_copy.argtypes = [vp, vp, i64, ci, ci, vp]
    grids = (256, 512, 1024, 2048, 4096, 8192)
    sink = torch.empty(max(grids) * 256, dtype=torch.int32, device="cuda")
    stream = lambda: ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    best = {"read": (0.0, None), "copy": (0.0, None)}
    half = n // 2
    for unroll in (4, 8, 16):
        for grid in grids:
            def rd():
                assert lib.hbm_probe_read(a.data_ptr(), n, sink.data_ptr(), unroll, grid, stream()) == 0

            def cp():
                assert lib.hbm_probe_copy(b.data_ptr(), a.data_ptr(), half, unroll, grid, stream()) == 0
            sec, _ = timed(rd, 5, 1)
            r = n * 5 / sec / 1e9
            if r > best["read"][0]:
                best["read"] = (r, f"unroll {unroll}, grid {grid}")
            sec, _ = timed(cp, 5, 1)
            r = 2 * half * 5 / sec / 1e9
            if r > best["copy"][0]:
                best["copy"] = (r, f"unroll {unroll}, grid {grid}")
    out["probe_read_GBps"], out["probe_read_best_launch"] = best["read"]
    out["probe_copy_read_plus_write_GBps"], out["probe_copy_best_launch"] = best["copy"]
    del a, b, mat, vec, sink
    torch.cuda.empty_cache()
    return out


# ------------------------------------------------------------------- main

def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    # untimed calls before each timed leg: the GPU's clocks take about 20
    # back-to-back calls of the 128K step (~30 ms of load) to ramp up from
    # idle, and a few idle seconds undo it
    ap.add_argument("--warmup", type=int, default=30)
    ap.add_argument("--only", default="all", choices=["all", "copy", "ceilings"] + LEGS)
    ap.add_argument("--decode-steps", type=int, default=1024)
    ap.add_argument("--skip", nargs="*", default=[], choices=LEGS + ["ceilings"],
                    help="legs to leave out of a full run (e.g. to keep a profiled run's trace small)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the Orthros layer here runs on a single MI355X with no "
              "sharding or collectives; run it with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch

    from phase_aware_swa_amd import inputs
    from phase_aware_swa_amd.runner import Copies, Decode, LayerStack, Prefill, Project

    torch.cuda.set_device(0)
    out, configs = {}, {}
    cpu_ok = not args.no_cpu_baseline
    run_leg = lambda leg: (args.only in ("all", leg)) and leg not in args.skip
    progress = lambda *a: print("[bench]", *a, file=sys.stderr, flush=True)

    if args.only == "copy":
        # plain copy kernel of known size: calibrates the FETCH_SIZE / WRITE_SIZE counters
        n = 1 << 30
        src = torch.empty(n, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        sec, _ = timed(lambda: dst.copy_(src), args.steps, args.warmup)
        print(json.dumps({"copy_bytes_each_way": n, "copy_GBps": 2 * n * args.steps / sec / 1e9}), flush=True)
        return
    if args.only == "ceilings":
        print(json.dumps({"hbm_practical": practical_ceilings()}), flush=True)
        return

    cfg = dict(inputs.WORKLOADS["gqa_8b_prefill_128k"])
    B, T, Hq, Hkv, d, w = (cfg[k] for k in ("batch", "T", "n_q_heads", "n_kv_heads", "head_dim", "window"))
    result = None
    if run_leg("prefill") or run_leg("swa") or run_leg("xattn"):
        progress("gqa_8b_prefill_128k")
        x = inputs.prefill_inputs(seed=2, device="cuda", **cfg)
        run = Prefill(cfg, x)
        run.run()
        torch.cuda.synchronize()
        if run_leg("prefill"):
            sec, wall = timed(run.run, args.steps, args.warmup)
            ms = sec / args.steps * 1e3
            nbytes = prefill_bytes(B, T, Hq, Hkv, d)
            fl = prefill_flops(B, T, Hq, d, w)
            out["prefill"] = {"kernel": "orthros_prefill", "us": ms * 1e3, "bytes": nbytes, "flops": fl,
                              "GBps": nbytes / (ms * 1e-3) / 1e9, "TFLOPs": fl / (ms * 1e-3) / 1e12}
            result = {"metric": METRIC, "value": B * T * args.steps / sec, "unit": "tokens/s", "n_gpus": 1,
                      "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms, "higher_is_better": True,
                      "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
                      "config": {"workload": "gqa_8b_prefill_128k", "global_batch": B, "seq_len": T,
                                 "n_q_heads": Hq, "n_kv_heads": Hkv, "head_dim": d, "window": w,
                                 "parallelism": "single-gpu"},
                      "wall_s_timed": wall}
            configs["gqa_8b_prefill_128k"] = {"us_per_call": ms * 1e3, "tokens_per_s": B * T / (ms * 1e-3),
                                              **hbm_fracs(nbytes, fl, ms * 1e-3)}
        if run_leg("swa"):
            sec, _ = timed(run.run_swa, args.steps, args.warmup)
            t_swa = sec / args.steps
            nbytes = swa_bytes(B, T, Hq, Hkv, d)
            fl = swa_flops(B, T, Hq, d, w)
            out["swa"] = {"kernel": "orthros_swa_prefill", "us": t_swa * 1e6, "bytes": nbytes, "flops": fl,
                          "GBps": nbytes / t_swa / 1e9, "TFLOPs": fl / t_swa / 1e12}
        if run_leg("xattn"):
            sec, _ = timed(run.run_xattn, args.steps, args.warmup)
            t_x = sec / args.steps
            nbytes = xattn_bytes(B, T, Hkv, d)
            out["xattn"] = {"kernel": "orthros_global_xattn", "us": t_x * 1e6, "bytes": nbytes,
                            "GBps": nbytes / t_x / 1e9}
        if result is not None and cpu_ok:
            progress("gqa_8b_prefill_128k: oracle")
            result["cpu_baseline"] = cpu_baseline(cfg, x)
            configs["gqa_8b_prefill_128k"]["cpu_baseline"] = result["cpu_baseline"]
        del run, x
        torch.cuda.empty_cache()

    for leg, name in (("tiny", "tiny_fp32_prefill"), ("mha8k", "mha_1p3b_prefill_8k")):
        if not run_leg(leg):
            continue
        progress(name)
        c = dict(inputs.WORKLOADS[name])
        cB, cT, cHq, cHkv, cd, cw = (c[k] for k in ("batch", "T", "n_q_heads", "n_kv_heads", "head_dim", "window"))
        es = 4 if c["dtype"] == torch.float32 else 2
        x = inputs.prefill_inputs(seed=1, device="cuda", **c)
        run = Prefill(c, x)
        n = max(50, args.steps * 10)
        sec, _ = timed(run.run, n, args.warmup)
        t = sec / n
        nbytes = prefill_bytes(cB, cT, cHq, cHkv, cd, es)
        fl = prefill_flops(cB, cT, cHq, cd, cw)
        peak = FP32_PEAK_TFLOPS if es == 4 else BF16_PEAK_TFLOPS
        configs[name] = {"us_per_call": t * 1e6, "tokens_per_s": cB * cT / t, "dtype": "f32" if es == 4 else "bf16",
                         "kernels": "swa_f32_kernel + xattn_split_kernel + merge_kernel" if es == 4 else
                                    "swa_ring_kernel<128, true, 1, 2> (the copy fused; one head a block, "
                                    "the head dims split over the waves) + merge_kernel",
                         "bytes": nbytes, "flops": fl, **hbm_fracs(nbytes, fl, t, peak),
                         "note": f"{nbytes / 2**20:.0f} MiB per call: much of it can be served from the 256 MB "
                                 "last-level cache between back-to-back calls, so GB/s is an effective rate"}
        if cpu_ok:
            configs[name]["cpu_baseline"] = cpu_baseline(c, x)
        del run, x
        torch.cuda.empty_cache()

    if run_leg("prefill1m"):
        # 36 layers whose caches all stay resident; each layer's inputs are
        # drawn (untimed) before its timed call
        c = dict(inputs.WORKLOADS["gqa_8b_prefill_1m"])
        cT, nl = c["T"], c["layers"]
        progress(f"gqa_8b_prefill_1m: {nl} resident caches")
        kc_all = torch.empty(nl, 1, c["n_kv_heads"], cT, c["head_dim"], dtype=torch.bfloat16, device="cuda")
        vc_all = torch.empty_like(kc_all)
        times = []
        for layer in range(nl):
            x = inputs.prefill_inputs(seed=1000 + layer, device="cuda", **c)
            run = Prefill(c, x, k_cache=kc_all[layer], v_cache=vc_all[layer])
            if layer == 0:
                for _ in range(5):                 # warm-up calls (clock ramp)
                    run.run()
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            run.run()
            e1.record()
            torch.cuda.synchronize()
            times.append(e0.elapsed_time(e1) / 1e3)
            if layer < nl - 1:
                del run, x
        total = sum(times)
        per = total / nl
        nbytes = prefill_bytes(1, cT, c["n_q_heads"], c["n_kv_heads"], c["head_dim"])
        fl = prefill_flops(1, cT, c["n_q_heads"], c["head_dim"], c["window"])
        configs["gqa_8b_prefill_1m"] = {"layers": nl, "ms_36_layers": total * 1e3, "ms_per_layer": per * 1e3,
                                        "ms_per_layer_min": min(times) * 1e3, "ms_per_layer_max": max(times) * 1e3,
                                        "tokens_per_s_per_layer": cT / per, "tokens_per_s_36_layers": cT / total,
                                        "bytes_per_layer": nbytes, "flops_per_layer": fl,
                                        **hbm_fracs(nbytes, fl, per)}
        if cpu_ok:
            progress("gqa_8b_prefill_1m: oracle (one layer, extrapolated)")
            configs["gqa_8b_prefill_1m"]["cpu_baseline"] = cpu_baseline_1m(c, x)
        del run, x, kc_all, vc_all
        torch.cuda.empty_cache()

    if run_leg("copies"):
        # output copies at many positions (SFT answer span, PT every position): MFMA-bound
        for name in ("gqa_8b_sft_32k", "gqa_8b_pt_16k"):
            progress(name)
            ccfg = dict(inputs.WORKLOADS[name])
            cB, cT, cTo = ccfg["batch"], ccfg["T"], ccfg["T_out"]
            xc = inputs.prefill_inputs(seed=7, device="cuda", **ccfg)
            pre = Prefill(ccfg, xc)
            pre.run_swa()                       # fills the caches, not timed
            q_out, pos = inputs.copies_inputs(cB, Hq, d, cT, cTo, torch.bfloat16, seed=8, device="cuda")
            cp = Copies(ccfg, cT, q_out, pos, xc["alpha_out"], xc["beta_out"], pre.k_cache, pre.v_cache)
            n = max(3, args.steps // 4)
            sec, _ = timed(cp.run, n, args.warmup)
            t = sec / n
            keys = float((pos.double() + 1).sum().item())           # admissible (copy, key) pairs per head
            fl = 4 * d * Hq * keys
            nbytes = cB * cT * Hkv * d * 2 * 2 + 2 * cB * cTo * Hq * d * 2
            out[name] = {"kernel": "orthros_copies (copies_flash_kernel<128>)", "us": t * 1e6, "T": cT,
                         "T_out": cTo, "copies_per_s": cB * cTo / t, "flops": fl, "TFLOPs": fl / t / 1e12,
                         "bytes": nbytes, "GBps": nbytes / t / 1e9,
                         "roofline": {"bound": "mfma", "achieved": fl / t / 1e12, "peak": BF16_PEAK_TFLOPS,
                                      "unit": "TFLOP/s", "frac": fl / t / 1e12 / BF16_PEAK_TFLOPS, "traffic": None,
                                      "kernel": f"orthros_copies at {name}"}}
            del pre, cp, xc, q_out, pos
            torch.cuda.empty_cache()

    if run_leg("project"):
        # the projections either side of the attention over the 128K batch: MFMA-bound
        progress("gqa_8b_project_128k")
        pcfg = dict(inputs.WORKLOADS["gqa_8b_project_128k"])
        xp = inputs.project_inputs(seed=9, device="cuda", **pcfg)
        pr = Project(pcfg, xp, cap=pcfg["T"])
        n_p = max(3, args.steps // 4)
        sec, _ = timed(pr.run, n_p, args.warmup)
        t = sec / n_p
        fl = project_flops(pcfg)
        out["project"] = {"kernel": "orthros_project (project_kernel<8, 4>)", "workload": "gqa_8b_project_128k",
                          "us": t * 1e6, "flops": fl, "TFLOPs": fl / t / 1e12,
                          "roofline": {"bound": "mfma", "achieved": fl / t / 1e12, "peak": BF16_PEAK_TFLOPS,
                                       "unit": "TFLOP/s", "frac": fl / t / 1e12 / BF16_PEAK_TFLOPS,
                                       "traffic": None, "kernel": "orthros_project at gqa_8b_project_128k"}}
        del pr, xp
        torch.cuda.empty_cache()

    for lname in ("gqa_8b_decode_36l_b4", "gqa_8b_decode_36l_b1_short"):
        if not run_leg("layers"):
            break
        # one decode step over 36 resident layers: eager launches vs one HIP graph
        progress(lname)
        lcfg = dict(inputs.WORKLOADS[lname])
        nl, ns = lcfg["layers"], lcfg["steps"]
        layers = [inputs.decode_inputs(seed=100 + l, device="cuda", **lcfg) for l in range(nl)]
        len0 = [x["cache_len"].clone() for x in layers]
        stack = LayerStack(lcfg, layers, ns)
        stack.set_inputs(0)
        graph = stack.capture()

        def reset():
            for x, l0 in zip(layers, len0):
                x["cache_len"].copy_(l0)

        def eager_pass():
            for _ in range(ns):
                stack.step()

        def graph_pass():
            for _ in range(ns):
                graph.replay()

        res = {}
        for name, fn in (("eager", eager_pass), ("graph", graph_pass)):
            reset()
            fn()                                   # warm-up pass
            reset()
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            fn()
            e1.record()
            torch.cuda.synchronize()
            res[name] = e0.elapsed_time(e1) * 1e3 / ns
        lens = torch.stack([l0.double() for l0 in len0])
        step_bytes = float(((lens + ns / 2).sum() * lcfg["n_kv_heads"] * lcfg["head_dim"] * 2 * 2).item())
        out["decode_layers_" + lname] = {"workload": lname, "layers": nl, "steps": ns,
                                         "eager_us_per_step": res["eager"], "graph_us_per_step": res["graph"],
                                         "bytes_per_step": step_bytes,
                                         "GBps_graph": step_bytes / (res["graph"] * 1e-6) / 1e9}
        del stack, graph, layers
        torch.cuda.empty_cache()

    if run_leg("decode"):
        progress("gqa_8b_decode_b16")
        dcfg = dict(inputs.WORKLOADS["gqa_8b_decode_b16"])
        nsteps = args.decode_steps
        dcfg["steps"] = nsteps
        xd = inputs.decode_inputs(seed=4, device="cuda", **dcfg)
        len0 = xd["cache_len"].clone()
        hint = int(len0.max().item()) + nsteps - 1
        dec = Decode(dcfg, xd["k_cache"], xd["v_cache"], xd["cache_len"], hint, xd["alpha"], xd["beta"],
                     xd["alpha_out"], xd["beta_out"])

        def one_pass():
            dec.cache_len.copy_(len0)
            for s in range(nsteps):
                dec.step(xd["q"][s], xd["q_out"][s], xd["k_new"][s], xd["v_new"][s])

        sec, _ = timed(one_pass, 2, 1)
        us = sec / 2 / nsteps * 1e6
        # one more pass with an event pair around every step: the per-step distribution
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(nsteps)]
        dec.cache_len.copy_(len0)
        for s_, (e0, e1) in enumerate(evs):
            e0.record()
            dec.step(xd["q"][s_], xd["q_out"][s_], xd["k_new"][s_], xd["v_new"][s_])
            e1.record()
        torch.cuda.synchronize()
        per = sorted(e0.elapsed_time(e1) * 1e3 for e0, e1 in evs)
        lens = len0.double()
        step_bytes = float(((lens + nsteps / 2).sum() * Hkv * d * 2 * 2).item())   # mean history K+V per step
        out["decode"] = {"workload": "gqa_8b_decode_b16", "us_per_step": us, "steps": nsteps,
                         "bytes_per_step": step_bytes, "GBps": step_bytes / (us * 1e-6) / 1e9,
                         "p50_us": per[len(per) // 2], "p99_us": per[min(len(per) - 1, (99 * len(per)) // 100)]}
        configs["gqa_8b_decode_b16"] = {"us_per_step": us, "steps": nsteps, "bytes_per_step": step_bytes,
                                        "GBps": step_bytes / (us * 1e-6) / 1e9,
                                        "hbm_frac": step_bytes / (us * 1e-6) / 1e9 / HBM_PEAK_GBS}
        if cpu_ok:
            progress("gqa_8b_decode_b16: oracle")
            dcfg["steps"] = 1024
            cb = cpu_baseline_decode(dcfg, xd, len0)
            out["decode"]["cpu_baseline"] = cb
            configs["gqa_8b_decode_b16"]["cpu_baseline"] = cb
        if result is None:
            result = {"metric": METRIC, "value": us, "unit": "us/step", "n_gpus": 1, "steps": nsteps,
                      "warmup": 1, "ms_per_step": us / 1e3, "higher_is_better": False, "scaling": "weak",
                      "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
                      "config": {"workload": "gqa_8b_decode_b16", "global_batch": 16,
                                 "parallelism": "single-gpu"}}
        del dec, xd
        torch.cuda.empty_cache()

    if result is None:
        result = {"metric": METRIC, "value": None, "unit": "tokens/s", "n_gpus": 1, "data": "synthetic",
                  "dtype": "bf16", "config": {"workload": "gqa_8b_prefill_128k"}}
    if "prefill" in out:
        s = out["prefill"]
        # the same step priced as two passes (SWA + writer, then the copy's
        # read of the whole cache): 1 GiB more than the one fused pass moves
        two_pass = s["bytes"] + xattn_bytes(B, T, Hkv, d)
        result["roofline"] = {"bound": "hbm", "achieved": s["GBps"], "peak": HBM_PEAK_GBS, "unit": "GB/s",
                              "frac": s["GBps"] / HBM_PEAK_GBS,
                              "traffic": measured_traffic("traffic_prefill_fused_gqa_8b_128k.md"),
                              "kernel": "orthros_prefill: swa_ring_kernel<128, true, 2, 1> (+ merge_kernel)",
                              "algorithmic_bytes": s["bytes"],
                              "two_pass_bytes": two_pass,
                              "achieved_two_pass_bytes": two_pass / (s["us"] * 1e-6) / 1e9,
                              "frac_two_pass_bytes": two_pass / (s["us"] * 1e-6) / 1e9 / HBM_PEAK_GBS,
                              "mfma_algorithmic_TFLOPs": s["TFLOPs"],
                              "mfma_algorithmic_frac": s["TFLOPs"] / BF16_PEAK_TFLOPS,
                              # the attainable roofline min(MFMA peak, intensity x HBM peak) at this
                              # step's algorithmic intensity, and the fraction of it reached
                              "intensity_flop_per_byte": s["flops"] / s["bytes"],
                              "attainable_TFLOPs": min(BF16_PEAK_TFLOPS, s["flops"] / s["bytes"] * HBM_PEAK_GBS / 1e3),
                              "attainable_frac": s["TFLOPs"] / min(BF16_PEAK_TFLOPS,
                                                                   s["flops"] / s["bytes"] * HBM_PEAK_GBS / 1e3)}
    if "swa" in out:
        s = out["swa"]
        result["roofline_swa"] = {"bound": "hbm", "achieved": s["GBps"], "peak": HBM_PEAK_GBS, "unit": "GB/s",
                                  "frac": s["GBps"] / HBM_PEAK_GBS,
                                  "traffic": measured_traffic("traffic_swa_prefill_gqa_8b_128k.md"),
                                  "kernel": "orthros_swa_prefill: swa_ring_kernel<128, false, 2, 1>"}
    if "xattn" in out:
        x = out["xattn"]
        result["roofline_xattn"] = {"bound": "hbm", "achieved": x["GBps"], "peak": HBM_PEAK_GBS, "unit": "GB/s",
                                    "frac": x["GBps"] / HBM_PEAK_GBS,
                                    "traffic": measured_traffic("traffic_global_xattn_gqa_8b_128k.md"),
                                    "kernel": "orthros_global_xattn (split-K + merge)"}
    if "decode" in out:
        dd = out["decode"]
        result["decode_us_per_step"] = dd["us_per_step"]
        result["roofline_decode"] = {"bound": "hbm", "achieved": dd["GBps"], "peak": HBM_PEAK_GBS, "unit": "GB/s",
                                     "frac": dd["GBps"] / HBM_PEAK_GBS,
                                     "traffic": measured_traffic("traffic_decode_gqa_8b_b16.md"),
                                     "kernel": "orthros_decode_step: "
                                               "xattn_lds_kernel<128, DecodeParams> + lds_decode_merge_kernel (per step)"}
    if args.only == "all" and "ceilings" not in args.skip:
        progress("practical HBM ceilings")
        result["hbm_practical"] = practical_ceilings()
    result["configs"] = configs
    result["kernels"] = out
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
