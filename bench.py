#!/usr/bin/env python3
"""Throughput of libgdn's frame-wise GDN forward on one MI355X.

One step = one gdn_forward over one GDN layer at the one-minute 720p shape
(B = 1, 20 heads, D = 112, 121 latent frames x 880 tokens = 106,480 tokens,
bf16 Q/K/V/O, fp32 gates and state), inputs resident in HBM.

Before the W warm-up steps the forward runs untimed for --ramp-seconds so
that the GPU's clocks have settled; the K timed steps are plain gdn_forward
calls between two device synchronisations.  A separate, untimed pass with
the library's phase events (gdn_forward_events, HIP events on the stream the
kernels run on) gives each kernel's average duration, from which the
roofline of the dominant kernel is computed.  Prints one JSON line:
tokens/s, that roofline, and the float64 CPU oracle timed on a bounded
sample of the same workloads.  Extras: forward + backward at the same shape,
121 streaming gdn_step calls, chunk-causal streaming by windows of latent
frames, token-wise GDN (one token per frame) in the token form, and the
fused block prologue.
"""

import argparse
import ctypes
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "GDN tokens/s per layer (20 heads, D=112) at 1-min 720p shape; % MFMA peak"
HBM_PEAK_GBS = 8000.0           # MI355X HBM3E
BF16_PEAK_TFLOPS = 2500.0       # MI355X dense bf16 MFMA
SHAPE = dict(B=1, H=20, D=112, T=121, N=880)
PROFILE_TRAFFIC = os.path.join(ROOT, "profiles", "traffic.json")


def algorithmic(kernel, B, H, D, T, N):
    """Bytes and dense-equivalent FLOPs the method must move / do in one
    launch of each kernel (inputs read once, outputs written once; the
    per-frame intermediates A_t, U_t, S_t are not counted)."""
    tokens = B * T * N
    heads_frames = B * H * T
    if kernel == "gram":      # read K, V (bf16) and beta (fp32)
        return tokens * H * (2 * D * 2 + 4), heads_frames * 2 * (2 * D * D * N)
    if kernel == "output":    # read Q, write O (bf16)
        return tokens * H * (2 * D * 2), heads_frames * 2 * D * D * N
    if kernel == "scan":      # intermediates only
        return 0, heads_frames * 2 * D * D * D
    if kernel == "forward":
        return tokens * H * (4 * D * 2 + 4), heads_frames * (3 * 2 * D * D * N + 2 * D * D * D)
    raise KeyError(kernel)


class HipEvents:
    def __init__(self, n):
        self.hip = ctypes.CDLL("libamdhip64.so")
        self.hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float),
                                                  ctypes.c_void_p, ctypes.c_void_p]
        self.hip.hipEventSynchronize.argtypes = [ctypes.c_void_p]
        self.ev = []
        for _ in range(n):
            e = ctypes.c_void_p()
            if self.hip.hipEventCreate(ctypes.byref(e)) != 0:
                raise RuntimeError("hipEventCreate failed")
            self.ev.append(e.value)

    def elapsed(self, i, j):
        self.hip.hipEventSynchronize(ctypes.c_void_p(self.ev[j]))
        ms = ctypes.c_float()
        if self.hip.hipEventElapsedTime(ctypes.byref(ms), ctypes.c_void_p(self.ev[i]),
                                        ctypes.c_void_p(self.ev[j])) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return ms.value


def load_traffic(kernel):
    """HBM bytes per launch from the committed rocprofv3 counter summary,
    if it was taken on the kernel's current source."""
    from gated_deltanet_recurrence_frame_amd.rocprof_summary import source_sha
    try:
        with open(PROFILE_TRAFFIC) as f:
            tr = json.load(f)
    except (OSError, ValueError):
        return None
    rec = tr.get(kernel)
    if not rec or rec.get("source_sha") != source_sha(kernel):
        return None
    return rec.get("bytes_per_launch")


def _blas_threads():
    try:
        from threadpoolctl import threadpool_info
        return sum(p.get("num_threads", 1) for p in threadpool_info()
                   if p.get("user_api") == "blas") or 1
    except Exception:
        return 1


def _oracle_heads(inp, fn, budget_s, T):
    """Call fn(per-head float64 tensors) on whole heads in turn (again from
    the first head while the budget lasts); returns one-layer tokens/s
    (heads scaled to the layer) and the sample's description."""
    from gated_deltanet_recurrence_frame_amd import inputs as gin
    H, N = SHAPE["H"], SHAPE["N"]
    done, t_total = 0, 0.0
    while t_total < budget_s:
        sl = slice(done % H, done % H + 1)
        x = {n: gin.as_f64(inp[n][:, :T * N, sl]) for n in ("q", "k", "v", "beta", "d_o")
             if n in inp}
        x["gamma"] = gin.as_f64(inp["gamma"][:, :T, sl])
        t0 = time.perf_counter()
        fn(x)
        t_total += time.perf_counter() - t0
        done += 1
    tokens = SHAPE["B"] * T * N
    return tokens * (done / H) / t_total, done, t_total


def cpu_baseline(inp, budget_s):
    """The float64 oracle, untouched, on whole heads of the workloads until
    each leg's share of the time budget is spent, scaled to one layer's
    tokens/s.  The headline value is the one-minute forward on all the BLAS
    threads the host gives; beside it the same forward on one thread, the
    short clip, the 121 streaming steps and forward + backward."""
    import oracle
    from threadpoolctl import threadpool_limits
    N = SHAPE["N"]
    T = SHAPE["T"]
    fwd = lambda x: oracle.forward(x["q"], x["k"], x["v"], x["gamma"], x["beta"], N)

    def stream(x):
        S = None                        # frame 0 from a zero state
        for t in range(T):
            sl = slice(t * N, (t + 1) * N)
            _, S = oracle.step(x["q"][:, sl], x["k"][:, sl], x["v"][:, sl],
                               x["gamma"][:, t:t + 1], x["beta"][:, sl], S)

    def train(x):
        fwd(x)
        oracle.backward(x["q"], x["k"], x["v"], x["gamma"], x["beta"], N, x["d_o"])

    threads = _blas_threads()
    # dense-equivalent FLOPs per token of one layer (the GPU legs' count)
    H, D = SHAPE["H"], SHAPE["D"]
    fwd_ft = H * (3 * 2 * D * D * N + 2 * D ** 3) / N
    flops_per_token = {"forward_minute": fwd_ft, "forward_minute_1thread": fwd_ft,
                       "forward_short": fwd_ft, "stream_minute": fwd_ft,
                       "train_minute": H * (8 * 2 * D * D * N + 3 * 2 * D ** 3) / N}
    legs = {}
    share = {"forward_minute": 0.4, "forward_minute_1thread": 0.15, "forward_short": 0.1,
             "stream_minute": 0.15, "train_minute": 0.2}
    for name, fn, frames, one in (("forward_minute", fwd, T, False),
                                  ("forward_minute_1thread", fwd, T, True),
                                  ("forward_short", fwd, 21, False),
                                  ("stream_minute", stream, T, False),
                                  ("train_minute", train, T, False)):
        if name == "train_minute" and "d_o" not in inp:
            continue
        if one:
            with threadpool_limits(limits=1):
                v, done, secs = _oracle_heads(inp, fn, budget_s * share[name], frames)
        else:
            v, done, secs = _oracle_heads(inp, fn, budget_s * share[name], frames)
        legs[name] = {"tokens_per_s": round(v, 1),
                      "gflops": round(v * flops_per_token[name] / 1e9, 2),
                      "head_passes": done, "seconds": round(secs, 2),
                      "threads": 1 if one else threads}
    main = legs["forward_minute"]
    return {"value": main["tokens_per_s"], "unit": "tokens/s", "cores": threads,
            "nproc": os.cpu_count(), "affinity_cores": len(os.sched_getaffinity(0)),
            "omp_num_threads": os.environ.get("OMP_NUM_THREADS"),
            "kind": "oracle",
            "sample": "float64 oracle (numpy, %d BLAS threads) forward on %d whole heads of the "
                      "1-min shape (121 x 880 tokens each, the 20 heads in turn), %.1f s, scaled "
                      "by heads to one-layer tokens/s; legs: the same on one thread, the short "
                      "clip (21 frames), 121 oracle steps, forward + backward"
                      % (threads, main["head_passes"], main["seconds"]),
            "legs": legs}


def main():
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--scan-chunk", type=int, default=0)
    ap.add_argument("--ramp-seconds", type=float, default=1.0,
                    help="untimed forwards before the warm-up steps (GPU clocks settle)")
    ap.add_argument("--cpu-seconds", type=float, default=24.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extras", action="store_true")
    ap.add_argument("--extras", default="train,stream,windows,tokenwise,prologue",
                    help="comma-separated extra legs to run")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU: libgdn runs on one GPU per process "
              "(--gpus %d requested)" % args.gpus, file=sys.stderr)
        sys.exit(2)

    import torch
    from gated_deltanet_recurrence_frame_amd import binding as gb
    from gated_deltanet_recurrence_frame_amd import inputs as gin

    dev = torch.device("cuda:0")
    B, H, D, T, N = (SHAPE[k] for k in ("B", "H", "D", "T", "N"))
    print("[bench] generating inputs", file=sys.stderr, flush=True)
    inp = gin.make_inputs(B=B, H=H, T=T, N=N, D=D, io="bf16", gamma="uniform", seed=0,
                          with_do=True)
    d = {k: v.to(dev) for k, v in inp.items()}
    torch.cuda.synchronize()

    plan = gb.ForwardPlan(B, H, T, N, D, "bf16", dev, scan_chunk=args.scan_chunk)
    fwd = lambda: plan(d["q"], d["k"], d["v"], d["gamma"], d["beta"])
    print("[bench] clock ramp (%.1f s) and %d warm-up steps" % (args.ramp_seconds, args.warmup),
          file=sys.stderr, flush=True)
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < args.ramp_seconds:
        for _ in range(20):
            fwd()
        torch.cuda.synchronize()
    for _ in range(args.warmup):
        fwd()
    torch.cuda.synchronize()
    print("[bench] timing %d steps" % args.steps, file=sys.stderr, flush=True)
    t0 = time.perf_counter()
    for _ in range(args.steps):
        fwd()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_step = wall * 1e3 / args.steps
    tokens = B * T * N
    value = tokens / (ms_step * 1e-3)

    # phases: a separate, untimed pass with the library's events
    nph = max(10, min(args.steps, 50))
    ev = HipEvents(4 * nph)
    for i in range(nph):
        plan(d["q"], d["k"], d["v"], d["gamma"], d["beta"], events=ev.ev[4 * i:4 * i + 4])
    torch.cuda.synchronize()
    phases = {"gram": 0.0, "scan": 0.0, "output": 0.0}
    for i in range(nph):
        phases["gram"] += ev.elapsed(4 * i, 4 * i + 1)
        phases["scan"] += ev.elapsed(4 * i + 1, 4 * i + 2)
        phases["output"] += ev.elapsed(4 * i + 2, 4 * i + 3)
    phases = {k: v / nph for k, v in phases.items()}

    dom = max(("gram", "output"), key=lambda k: phases[k])
    abytes, aflops = algorithmic(dom, B, H, D, T, N)
    achieved = abytes / (phases[dom] * 1e-3) / 1e9
    roof = {"bound": "hbm", "kernel": dom, "achieved": round(achieved, 1),
            "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": load_traffic(dom), "algorithmic_bytes": abytes,
            "avg_ms": round(phases[dom], 4), "timing": "phase events, separate pass of %d "
                                                      "forwards" % nph}
    copy_gbs = copy_ceiling()
    roof["copy_gbs"] = round(copy_gbs, 1)
    roof["frac_of_copy"] = round(achieved / copy_gbs, 4)
    if roof["traffic"]:
        roof["traffic_gbs"] = round(roof["traffic"] / (phases[dom] * 1e-3) / 1e9, 1)
        roof["traffic_frac_of_copy"] = round(roof["traffic_gbs"] / copy_gbs, 4)
    fbytes, fflops = algorithmic("forward", B, H, D, T, N)
    step_roof = {"bound": "hbm", "achieved": round(fbytes / (ms_step * 1e-3) / 1e9, 1),
                 "peak": HBM_PEAK_GBS, "unit": "GB/s",
                 "frac": round(fbytes / (ms_step * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                 "algorithmic_bytes": fbytes,
                 "tflops": round(fflops / (ms_step * 1e-3) / 1e12, 2),
                 "mfma_frac": round(fflops / (ms_step * 1e-3) / 1e12 / BF16_PEAK_TFLOPS, 4)}

    extra = {}
    legs = set() if args.no_extras else set(x for x in args.extras.split(",") if x)
    if "train" in legs:
        print("[bench] forward+backward", file=sys.stderr, flush=True)
        extra["train"] = bench_train(gb, d, B, H, D, T, N, max(3, args.steps // 4))
    if "stream" in legs:
        print("[bench] streaming steps", file=sys.stderr, flush=True)
        extra["stream"] = bench_stream(gb, d, B, H, D, T, N)
    if "windows" in legs:
        print("[bench] streaming windows", file=sys.stderr, flush=True)
        extra["windows"] = [bench_windows(gb, d, B, H, D, T, N, k) for k in (2, 8, 15)]
    if "tokenwise" in legs:
        print("[bench] token-wise GDN (token form)", file=sys.stderr, flush=True)
        extra["tokenwise"] = bench_tokenwise(gb, d, B, H, D, T * N)
    if "prologue" in legs:
        print("[bench] block prologue", file=sys.stderr, flush=True)
        extra["prologue"] = bench_prologue(gb, d, B, H, D, T, N)

    out = {
        "metric": METRIC, "value": round(value, 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "gdn_forward, one GDN layer at the 1-min 720p latent shape",
                   "B": B, "H": H, "D": D, "T": T, "N": N, "tokens": tokens,
                   "io": "bf16", "state": "fp32", "scan_chunk": args.scan_chunk},
        "roofline": roof,
        "step_roofline": step_roof,
        "phases_ms": {k: round(v, 4) for k, v in phases.items()},
        "extra": extra,
    }
    if not args.no_cpu_baseline:
        print("[bench] cpu baseline (oracle)", file=sys.stderr, flush=True)
        out["cpu_baseline"] = cpu_baseline(inp, args.cpu_seconds)
    print(json.dumps(out), flush=True)


def copy_ceiling(nbytes=1 << 30, reps=10):
    """Device-to-device copy bandwidth (read + write bytes / time) of a plain
    torch copy of `nbytes`: the practical HBM ceiling the kernels are also
    set against."""
    import torch
    src = torch.empty(nbytes // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(reps):
        dst.copy_(src)
    e1.record()
    torch.cuda.synchronize()
    gbs = 2.0 * nbytes * reps / (e0.elapsed_time(e1) * 1e-3) / 1e9
    del src, dst
    torch.cuda.empty_cache()
    return gbs


def bench_train(gb, d, B, H, D, T, N, steps):
    import torch
    plan = gb.ForwardPlan(B, H, T, N, D, "bf16", d["q"].device, saved=True)
    prob = plan.prob
    ws = torch.empty(gb.workspace_size(prob, gb.GDN_OP_BACKWARD), dtype=torch.uint8,
                     device=d["q"].device)
    grads = None

    def one():
        nonlocal grads
        plan(d["q"], d["k"], d["v"], d["gamma"], d["beta"])
        grads = gb.backward(d["q"], d["k"], d["v"], d["gamma"], d["beta"], N, d["d_o"],
                            saved=plan.saved, workspace=ws)
    one()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        one()
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / steps
    tokens = B * T * N
    # algorithmic bytes of forward + backward: the forward's Q, K, V read, O
    # written (bf16), beta read (fp32); the backward's Q, K, V, dO read,
    # dQ, dK, dV written (bf16), beta read, dbeta written (fp32)
    nbytes = tokens * H * ((4 * D * 2 + 4) + (7 * D * 2 + 8))
    return {"workload": "gdn_forward + gdn_backward (saved A_t, S_t), 1-min shape",
            "ms_per_step": round(ms, 4), "tokens_per_s": round(tokens / (ms * 1e-3), 1),
            "algorithmic_bytes": nbytes,
            "hbm_frac": round(nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4), "steps": steps}


def bench_stream(gb, d, B, H, D, T, N):
    import torch
    dev = d["q"].device
    state = torch.zeros((B, H, D, D), dtype=torch.float32, device=dev)
    plan = gb.StepPlan(B, H, N, D, "bf16", dev)
    frames = [(d["q"][:, t * N:(t + 1) * N], d["k"][:, t * N:(t + 1) * N],
               d["v"][:, t * N:(t + 1) * N], d["gamma"][:, t:t + 1], d["beta"][:, t * N:(t + 1) * N])
              for t in range(T)]
    for f in frames[:3]:
        plan(*f, state)
    state.zero_()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream(dev)
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(T + 1)]
    evs[0].record(stream)
    t0 = time.perf_counter()
    for t, f in enumerate(frames):
        plan(*f, state)
        evs[t + 1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    lat = sorted(evs[t].elapsed_time(evs[t + 1]) for t in range(T))
    # the same chain with no event between the calls: GPU time per frame
    state.zero_()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    for f in frames:
        plan(*f, state)
    e1.record(stream)
    torch.cuda.synchronize()
    chain = e0.elapsed_time(e1)
    return {"workload": "frame 0 then 120 gdn_step calls (state carried), 880 tokens each",
            "calls": T, "per_frame_ms_median": round(lat[T // 2], 4),
            "per_frame_ms_p90": round(lat[int(T * 0.9)], 4),
            "per_frame_ms_back_to_back": round(chain / T, 4),
            "tokens_per_s": round(B * T * N / wall, 1),
            "timing": "per-frame figures from an event after every call; back_to_back from "
                      "two events around the whole chain"}


def bench_tokenwise(gb, d, B, H, D, L):
    """Token-wise GDN (one token per step, N = 1) over the same 106,480 tokens
    per head, in the token form (chunks of 64 one-token frames); the frame
    form is timed beside it on the first 8192 tokens (its per-frame D x D
    intermediates for all 106,480 steps would take 160 GB)."""
    import torch
    dev = d["q"].device
    gen = torch.Generator(device="cpu").manual_seed(5)
    gam = (0.9 + 0.1 * torch.rand((B, L, H), generator=gen)).to(dev)
    out = {"workload": "token-wise GDN: %d one-token frames, %d heads, D=%d, bf16" % (L, H, D)}
    for name, T, algo in (("token_form", L, "token"), ("token_form_8192", 8192, "token"),
                          ("frame_form_8192", 8192, "frame")):
        plan = gb.ForwardPlan(B, H, T, 1, D, "bf16", dev, algorithm=algo)
        args = (d["q"][:, :T], d["k"][:, :T], d["v"][:, :T], gam[:, :T].contiguous(),
                d["beta"][:, :T])
        plan(*args)
        torch.cuda.synchronize()
        reps = 3
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            plan(*args)
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / reps
        out[name] = {"tokens": B * T, "ms": round(ms, 4), "tokens_per_s": round(B * T / (ms * 1e-3), 1)}
        # algorithmic HBM bytes: q, k, v, o (bf16) and the two gates (fp32, one
        # of each per token and head, the frames being single tokens)
        nbytes = B * T * H * (4 * D * 2 + 4 + 4)
        out[name]["algorithmic_bytes"] = nbytes
        out[name]["hbm_frac"] = round(nbytes / (ms * 1e-3) / (HBM_PEAK_GBS * 1e9), 4)
        del plan
    return out


def bench_prologue(gb, d, B, H, D, T, N):
    """The block's prologue at the 1-min shape: gdn_forward with the query /
    key normalisation and gate logits fused (GDN_FLAG_*), the same forward
    behind a separate normalisation pass (torch ops, for comparison only),
    and forward + backward with the prologue."""
    import torch
    dev = d["q"].device
    args = (d["q"], d["k"], d["v"], d["gamma"], d["beta"])
    fused = gb.ForwardPlan(B, H, T, N, D, "bf16", dev, flags=3)
    plain = gb.ForwardPlan(B, H, T, N, D, "bf16", dev)
    sv = gb.ForwardPlan(B, H, T, N, D, "bf16", dev, flags=3, saved=True)
    ws = torch.empty(gb.workspace_size(sv.prob, gb.GDN_OP_BACKWARD), dtype=torch.uint8,
                     device=dev)

    def separate():
        q = torch.nn.functional.normalize(d["q"].float(), dim=-1).to(torch.bfloat16)
        k = torch.nn.functional.normalize(d["k"].float(), dim=-1).to(torch.bfloat16)
        plain(q, k, d["v"], torch.sigmoid(d["gamma"]), torch.sigmoid(d["beta"]))

    def train():
        sv(*args)
        gb.backward(*args, N, d["d_o"], saved=sv.saved, workspace=ws, normalize_qk=True,
                    gate_logits=True)

    out = {"workload": "gdn_forward with normalised q, k and gate logits, 1-min shape"}
    tokens = B * T * N
    for name, fn, reps in (("fused_forward", lambda: fused(*args), 10),
                           ("plain_forward", lambda: plain(*args), 10),
                           ("separate_pass_forward", separate, 5),
                           ("fused_forward_backward", train, 3)):
        fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / reps
        out[name] = {"ms": round(ms, 4), "tokens_per_s": round(tokens / (ms * 1e-3), 1)}
    del fused, plain, sv, ws
    return out


def bench_windows(gb, d, B, H, D, T, N, k):
    """Chunk-causal streaming: the first latent frame alone, then windows of
    k latent frames (8k raw frames each), every window one gdn_forward that
    carries the state in place."""
    import torch
    dev = d["q"].device
    bounds = [(0, 1)] + [(t, min(t + k, T)) for t in range(1, T, k)]
    plans = {}
    for t0, t1 in bounds:
        if t1 - t0 not in plans:
            plans[t1 - t0] = gb.ForwardPlan(B, H, t1 - t0, N, D, "bf16", dev)
    state = torch.zeros((B, H, D, D), dtype=torch.float32, device=dev)
    wins = [(plans[t1 - t0], d["q"][:, t0 * N:t1 * N], d["k"][:, t0 * N:t1 * N],
             d["v"][:, t0 * N:t1 * N], d["gamma"][:, t0:t1], d["beta"][:, t0 * N:t1 * N])
            for t0, t1 in bounds]
    for w in wins[:3]:
        w[0](*w[1:], state_in=state, state_out=state)
    state.zero_()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream(dev)
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(len(wins) + 1)]
    evs[0].record(stream)
    t0 = time.perf_counter()
    for i, w in enumerate(wins):
        w[0](*w[1:], state_in=state, state_out=state)
        evs[i + 1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    lat = sorted(evs[i].elapsed_time(evs[i + 1]) for i in range(1, len(wins)))
    n = len(lat)
    return {"workload": "frame 0, then windows of %d latent frames (gdn_forward, state carried)"
                        % k,
            "calls": len(wins), "per_window_ms_median": round(lat[n // 2], 4),
            "per_window_ms_max": round(lat[-1], 4), "tokens_per_s": round(B * T * N / wall, 1)}


if __name__ == "__main__":
    main()
