"""Benchmark: denoising steps/s and tokens/s of the SureLock step engine at the
LLaDA-8B shape (32 layers, d=4096, 32x128 MHA, SwiGLU 12288, vocab 126464,
bf16), one sequence of N=512 (128 random prompt tokens + 384 masked), on one
GPU, with synthetic random-init weights.

A "step" is one denoising iteration of the whole hot path: dlm_step (active
set compaction, per-layer projections / rotary / K-V scatter / attention over
all cached positions / FFN on the active rows, LM head, vocabulary
statistics) + dlm_lock_update (top-k unmasking and the lock test).  The timed
steps follow a decoding run from its first step (a new run starts every
128 steps).  `value` is the configured lock setting (KL <= 1e-3, max-prob >=
0.9, 2 consecutive steps); the scheduled-lock and vanilla (no locking) runs,
the configured lock test with the SlowFast sampler in place of the
semi-autoregressive top-k, and the scheduled lock test with the drift-aware
refresh of locked positions (8 recomputed per step, unlocked above a drift of
1e-3) are reported alongside.

Per-kernel times come from HIP events recorded on the engine's stream in a
second pass over the same steps; the roofline entry is for the kernel class
with the largest share of that time.  The CPU baseline times the oracle on a
bounded sample (see cpu_baseline.sample).
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "denoising steps/s + tokens/s, LLaDA-8B shape N=512, 1 GPU; MFMA% / HBM%"
PEAK_BF16_TFLOPS = 2500.0
PEAK_HBM_GBS = 8000.0
RIDGE = PEAK_BF16_TFLOPS * 1e12 / (PEAK_HBM_GBS * 1e9)  # FLOP per byte


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def run_steps(eng_factory, K, timing=False, flops_out=None):
    """K steps from the start of a run (new run every `steps` steps).
    Returns (seconds, decoded tokens, list of M, engine-timing dict or None);
    decoded tokens are counted from the engines' token arrays after the
    timed region (positions past the prompt no longer holding the mask).
    flops_out (a list), if given, receives each step's algorithmic FLOPs as
    the engine counts them (dlm_last_step_info)."""
    import torch
    acc = {}

    def absorb(e):
        for k, v in e.read_timing().items():
            a = acc.setdefault(k, dict(ms=0.0, launches=0, bytes=0.0, flops=0.0))
            for f in a:
                a[f] += v[f]

    eng = eng_factory()
    if timing:
        eng.set_timing(True)
    run = eng.run
    used = [eng]
    ms = []
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(K):
        if eng.t >= run.steps:
            eng = eng_factory()
            used.append(eng)
            if timing:
                eng.set_timing(True)
        ms.append(eng.step())
        if flops_out is not None:
            flops_out.append(eng.last_step_info()[2])
        eng.lock_update()
    torch.cuda.synchronize()
    dt = time.perf_counter() - t0
    toks = 0
    for e in used:
        if timing:
            absorb(e)
        toks += int((e.tokens()[:, run.prompt_len:] != e.shape.mask_id).sum())
        e.close()
    return dt, toks, ms, (acc if timing else None)


def roofline_entry(tim, setting_ms):
    """Roofline of the kernel class with the largest event time: the class's
    algorithmic FLOPs / bytes per launch over its average launch duration,
    both from the engine's HIP events around each launch (the events include
    the few microseconds between back-to-back dispatches on one queue, which
    a kernel trace's durations do not)."""
    name = max(tim, key=lambda k: tim[k]["ms"])
    t = tim[name]
    avg_s = t["ms"] / 1e3 / max(t["launches"], 1)
    flops = t["flops"] / max(t["launches"], 1)
    byts = t["bytes"] / max(t["launches"], 1)
    mean_m = sum(setting_ms) / len(setting_ms)
    timing = "engine HIP events around each launch over the timed steps"
    if flops > 0 and flops / max(byts, 1.0) >= RIDGE:
        ach = flops / avg_s / 1e12
        return name, dict(bound="mfma", achieved=round(ach, 2), peak=PEAK_BF16_TFLOPS,
                          unit="TFLOP/s", frac=round(ach / PEAK_BF16_TFLOPS, 4), traffic=None,
                          kernel=name, avg_launch_us=round(avg_s * 1e6, 2),
                          flops_per_launch=flops, bytes_per_launch=byts,
                          launches=t["launches"], mean_active_rows=round(mean_m, 1),
                          timing=timing)
    ach = byts / avg_s / 1e9
    return name, dict(bound="hbm", achieved=round(ach, 1), peak=PEAK_HBM_GBS, unit="GB/s",
                      frac=round(ach / PEAK_HBM_GBS, 4), traffic=None, kernel=name,
                      avg_launch_us=round(avg_s * 1e6, 2), flops_per_launch=flops,
                      bytes_per_launch=byts, launches=t["launches"],
                      mean_active_rows=round(mean_m, 1), timing=timing)


TRAFFIC_SOURCES = ("selective_token_recompute_amd/csrc/k_gemm.hip",
                   "selective_token_recompute_amd/csrc/common.h",
                   "selective_token_recompute_amd/csrc/vocab_part.h")


def sources_sha256(paths=TRAFFIC_SOURCES):
    import hashlib
    h = hashlib.sha256()
    for p in paths:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def measured_traffic(kernel_class):
    """HBM bytes per launch of a kernel class from the committed counter
    summary profiles/<class>_traffic.md (lines 'key: value'), or None when
    the summary is missing or the kernel sources changed since the counters
    were taken (sha256 over TRAFFIC_SOURCES)."""
    path = os.path.join(ROOT, "profiles", f"{kernel_class}_traffic.md")
    if not os.path.exists(path):
        return None
    kv = {}
    for line in open(path):
        if ":" in line and not line.startswith(("#", "|", " ")):
            k, v = line.split(":", 1)
            kv[k.strip()] = v.strip()
    if kv.get("sources_sha256") != sources_sha256():
        return None
    try:
        return float(kv["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def copy_calibration(nbytes=1 << 30, reps=3):
    """A plain device-to-device copy of nbytes (torch's copy kernel), reps
    times: the reference for scaling the FETCH_SIZE / WRITE_SIZE counters."""
    import torch
    src = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    log(f"copy calibration: {reps} copies of {nbytes} bytes")


def graph_timed(calls, reps=5):
    """Seconds per call of a list of zero-argument launch functions, captured
    once in a HIP graph (after one eager warm-up pass) and replayed reps
    times, so that the host's launch overhead is not in the time; falls back
    to eager launches between events when the capture fails."""
    import torch
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        for f in calls:
            f()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    try:
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=s):
            for f in calls:
                f()
        g.replay()
        torch.cuda.synchronize()
        e0.record()
        for _ in range(reps):
            g.replay()
        e1.record()
        torch.cuda.synchronize()
        del g
    except Exception:  # capture not supported by a call: eager launches
        torch.cuda.synchronize()
        e0.record()
        for _ in range(reps):
            for f in calls:
                f()
        e1.record()
        torch.cuda.synchronize()
    return e0.elapsed_time(e1) / 1e3 / (reps * len(calls))


# GEMM shapes of one LLaDA-8B step (N, K) and their epilogue in the engine
STEP_GEMMS = {"gemm_qkv": (12288, 4096), "gemm_o": (4096, 4096), "gemm_gate_up": (12288, 4096),
              "gemm_down": (4096, 12288), "gemm_lm_head": (126464, 4096)}


def measured_ceilings(step_m=384):
    """Ceilings measured on this GPU:
    * a plain 1 GiB device-to-device copy (read + write bytes over its time);
    * device copies moving 8.4 MB and 16.8 MB (one layer's K/V cache at
      N = 512 and 1024), 32 buffers rotated, back to back in a HIP graph: the
      bandwidth a kernel of that size reaches, launch and first DRAM round
      trip included;
    * hipBLASLt (torch.mm, bf16 in and out) on 8192 x 8192 x 8192, and this
      library's GEMM (default plan, fp32 store) on the same problem;
    * hipBLASLt against this library on each GEMM shape of the step at
      M = step_m active rows (gate/up as one 2 d_ff-wide GEMM for hipBLASLt,
      the SwiGLU epilogue here), both graph-timed."""
    import torch
    from selective_token_recompute_amd import ops, _lib as L
    n = 1 << 28
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    t_copy = graph_timed([lambda: dst.copy_(src)] * 4, reps=3)
    del src, dst
    small = {}
    for traffic in (8388608, 16777216):
        m = traffic // 2 // 4
        bufs = [(torch.ones(m, device="cuda"), torch.empty(m, device="cuda")) for _ in range(32)]
        t = graph_timed([lambda a=a, b=b: b.copy_(a) for a, b in bufs], reps=5)
        small[f"{traffic / 1e6:.1f}MB"] = round(traffic / t / 1e9, 1)
        del bufs
    S = 8192
    A = torch.randn(S, S, device="cuda").to(torch.bfloat16)
    W = torch.randn(S, S, device="cuda").mul_(0.02).to(torch.bfloat16)
    Wt = W.t().contiguous()
    C = torch.empty(S, S, device="cuda")
    Cb = torch.empty(S, S, device="cuda", dtype=torch.bfloat16)
    t_ours = graph_timed([lambda: ops.gemm(L.DLM_EPI_STORE_F32, A, W, C=C)] * 4, reps=3)
    t_blas = graph_timed([lambda: torch.mm(A, Wt, out=Cb)] * 4, reps=3)
    del A, W, Wt, C, Cb
    per_shape = {}
    for name, (N, K) in STEP_GEMMS.items():
        A = torch.randn(step_m, K, device="cuda").to(torch.bfloat16)
        W = torch.randn(N, K, device="cuda").mul_(0.02).to(torch.bfloat16)
        dual = name == "gemm_gate_up"
        Wb = torch.randn(2 * N if dual else N, K, device="cuda").mul_(0.02).to(torch.bfloat16)
        Wbt = Wb.t().contiguous()
        Cb = torch.empty(step_m, Wb.shape[0], device="cuda", dtype=torch.bfloat16)
        t_b = graph_timed([lambda: torch.mm(A, Wbt, out=Cb)] * 8)
        if dual:
            W2 = torch.randn(N, K, device="cuda").mul_(0.02).to(torch.bfloat16)
            U = torch.empty(step_m, N, device="cuda", dtype=torch.bfloat16)
            t_o = graph_timed([lambda: ops.gemm(L.DLM_EPI_SWIGLU, A, W, W2=W2, C=U)] * 8)
        else:
            Co = torch.empty(step_m, N, device="cuda")
            t_o = graph_timed([lambda: ops.gemm(L.DLM_EPI_STORE_F32, A, W, C=Co)] * 8)
        fl = 2.0 * step_m * Wb.shape[0] * K
        per_shape[name] = dict(hipblaslt_us=round(t_b * 1e6, 2), ours_us=round(t_o * 1e6, 2),
                               hipblaslt_tflops=round(fl / t_b / 1e12, 1),
                               ours_tflops=round(fl / t_o / 1e12, 1))
        del A, W, Wb, Wbt, Cb
    torch.cuda.empty_cache()
    return dict(hbm_copy_gbs=round(2 * 4 * n / t_copy / 1e9, 1),
                small_copy_gbs=small,
                gemm_bf16_tflops_hipblaslt=round(2.0 * S ** 3 / t_blas / 1e12, 1),
                gemm_bf16_tflops_ours=round(2.0 * S ** 3 / t_ours / 1e12, 1),
                step_gemms_at_m=step_m, step_gemms=per_shape,
                note="copies: read + write bytes; GEMMs graph-timed, 8192^3 bf16 "
                     "(hipBLASLt via torch.mm, bf16 out; ours fp32 out)")


def cpu_baseline(shape, run):
    """Oracle on a bounded sample: one full-width layer at step 0 (M = 512
    active rows, attention over N = 512) plus the LM head and statistics for
    8 sampled rows, extrapolated to one configured-setting step (M = 384,
    32 layers, LM head on 384 rows)."""
    import dataclasses
    import numpy as np
    import oracle
    import synth
    one = dataclasses.replace(shape, n_layers=1)
    W = synth.gen_weights(one)
    pr = synth.gen_prompts(one, run)
    o = oracle.Oracle(one, W, run, synth.LOCK_SETTINGS["natural"], pr)
    t0 = time.perf_counter()
    o.step(sample_rows=list(range(8)))
    t_all = time.perf_counter() - t0
    # split the sample's time into its layer part and LM-head part by FLOPs
    d, V, N = one.d_model, one.vocab, run.seq_len
    f_layer = oracle.closed_form_flops(one, [N], N) - 2.0 * N * d * V
    f_head8 = 2.0 * 8 * d * V
    rate = (f_layer + f_head8) / t_all  # FLOP/s of the oracle on this sample
    M = run.seq_len - run.prompt_len
    f_step = oracle.closed_form_flops(shape, [M], N)
    step_s = f_step / rate
    return dict(value=round(1.0 / step_s, 6), unit="steps/s", cores=oracle.num_threads(),
                kind="oracle",
                sample=(f"oracle (C++ fp64, OpenMP) on 1 of 32 layers at full width for all 512 "
                        f"rows of step 0 plus the LM head for 8 rows: {t_all:.1f} s, "
                        f"{rate / 1e9:.1f} GFLOP/s; extrapolated by closed-form FLOPs to a "
                        f"384-row, 32-layer step ({f_step / 1e12:.2f} TFLOP)"),
                sample_seconds=round(t_all, 2))


GEMM_CLASSES = ("gemm_qkv", "gemm_o", "gemm_gate_up", "gemm_down")


def layer_isolation(n_caches=32, launches=100, warmup=10):
    """One bf16 layer at LLaDA-8B width over an N=1024 cache, at M = 1024,
    512, 256, 102 and 20 active rows (a sorted uniform random subset, seed
    2).  Runs through the engine with a one-layer model and a 256-entry
    vocabulary (so the LM head and statistics are negligible and not
    reported); n_caches engines with their own cache (K, V ~ N(0, 1) bf16)
    are stepped round-robin so the 16.8 MB caches (537 MB in all) and the
    436 MB of layer weights are not served from the 256 MB Infinity Cache.
    Per-kernel times come from the engine's HIP events."""
    import dataclasses
    import numpy as np
    import torch
    import synth
    from selective_token_recompute_amd import engine as E

    cfg = synth.LAYER_ISOLATION
    shape = dataclasses.replace(cfg["shape"], vocab=256)
    N = cfg["cache_len"]
    run = synth.RunShape(1, N, N // 2, 4 * launches, N // 2)
    lock = synth.LOCK_SETTINGS["vanilla"]
    dev = torch.device("cuda:0")
    dw = E.random_device_weights(shape, seed=0, device=dev)
    prompts = torch.from_numpy(synth.gen_prompts(shape, run)).to(dev)
    g = torch.Generator(device=dev)
    g.manual_seed(3)
    points = []
    for frac in cfg["active_fractions"]:
        M = int(round(frac * N))
        act = np.sort(np.random.default_rng(2).choice(N, size=M, replace=False))
        locked = np.ones(N, dtype=bool)
        locked[act] = False
        words = np.zeros((1, (N + 63) // 64), dtype=np.uint64)
        for p_ in np.nonzero(locked)[0]:
            words[0, p_ // 64] |= np.uint64(1) << np.uint64(p_ % 64)
        bits = torch.from_numpy(words.view(np.int64)).to(dev)
        engs = []
        for _ in range(n_caches):
            e = E.Engine(shape, dw, run, lock, prompts)
            kc, vc = e.kv_cache()
            kc.copy_(torch.randn(kc.shape, generator=g, device=dev).to(kc.dtype))
            vc.copy_(torch.randn(vc.shape, generator=g, device=dev).to(vc.dtype))
            e.lock_bits().copy_(bits)
            engs.append(e)

        def go(n):
            for i in range(n):
                e = engs[i % n_caches]
                assert e.step() == M
                e.lock_update()

        go(warmup)
        for e in engs:
            e.set_timing(True)
        go(launches)
        tot = {}
        for e in engs:
            for k, v in e.read_timing().items():
                a = tot.setdefault(k, dict(ms=0.0, launches=0, bytes=0.0, flops=0.0))
                for f in a:
                    a[f] += v[f]
            e.close()
        gem = [tot[c] for c in GEMM_CLASSES]
        g_s = sum(x["ms"] for x in gem) / 1e3 / launches
        g_fl = sum(x["flops"] for x in gem) / launches
        g_by = sum(x["bytes"] for x in gem) / launches
        at = tot["attention"]
        a_s = at["ms"] / 1e3 / max(at["launches"], 1)
        a_by = at["bytes"] / max(at["launches"], 1)
        a_fl = at["flops"] / max(at["launches"], 1)
        pt = dict(M=M, gemm_us=round(g_s * 1e6, 2),
                  gemm_tflops=round(g_fl / g_s / 1e12, 1),
                  gemm_mfma_frac=round(g_fl / g_s / 1e12 / PEAK_BF16_TFLOPS, 4),
                  gemm_weight_stream_gbs=round(g_by / g_s / 1e9, 1),
                  gemm_hbm_frac=round(g_by / g_s / 1e9 / PEAK_HBM_GBS, 4),
                  attention_us=round(a_s * 1e6, 2),
                  attention_gbs=round(a_by / a_s / 1e9, 1),
                  attention_hbm_frac=round(a_by / a_s / 1e9 / PEAK_HBM_GBS, 4),
                  attention_tflops=round(a_fl / a_s / 1e12, 1))
        pt.update({f"{c}_us": round(tot[c]["ms"] * 1e3 / max(tot[c]["launches"], 1), 2)
                   for c in GEMM_CLASSES + ("rmsnorm",)})
        log(f"[layer M={M}] {pt}")
        points.append(pt)
        del engs
        torch.cuda.empty_cache()
    return dict(workload=("one bf16 LLaDA-8B-width layer (d=4096, 32x128 MHA, SwiGLU 12288) "
                          f"over an N={N} cache, {n_caches} caches stepped round-robin, "
                          f"{launches} timed launches per point"),
                points=points)


EXTRA_CONFIGS = {
    "dream7b": "Dream-7B shape (28 layers, d=3584, 28 query / 4 K-V heads x128, SwiGLU 18944, "
               "vocab 152064, bf16), B=8 sequences of N=1024 (256 prompt + 768 masked), 256-step "
               "runs, one semi-AR block",
    "longctx": "LLaDA-8B shape, B=4 sequences of N=4096 (1024 prompt + 3072 masked), 512-step runs "
               "in 12 semi-AR blocks of 256",
}


def extra_config(name, K, full_run=False, settings=("natural", "scheduled")):
    """Steps/s and tokens/s of another configured shape: the first K steps of
    a run (M at its largest), or whole runs with full_run."""
    import torch
    import synth
    from selective_token_recompute_amd import engine as E
    shape, run = synth.CONFIGS[name]
    dev = torch.device("cuda:0")
    dw = E.random_device_weights(shape, seed=0, device=dev)
    prompts = torch.from_numpy(synth.gen_prompts(shape, run)).to(dev)
    out = dict(workload=EXTRA_CONFIGS[name], batch=run.batch, seq_len=run.seq_len)
    steps = run.steps if full_run else K
    for st in settings:
        def factory():
            return E.Engine(shape, dw, run, synth.LOCK_SETTINGS[st], prompts)
        run_steps(factory, 2)
        dt, toks, ms, _ = run_steps(factory, steps)
        out[st] = dict(steps=steps, from_run_start=True, steps_per_s=round(steps / dt, 3),
                       tokens_per_s=round(toks / dt, 2), ms_per_step=round(dt * 1e3 / steps, 2),
                       mean_active_rows=round(sum(ms) / len(ms), 1), first_m=ms[0])
        log(f"[{name}/{st}] {steps} steps in {dt:.2f} s -> {steps / dt:.2f} steps/s, "
            f"{toks / dt:.1f} tokens/s, mean M {sum(ms) / len(ms):.1f}")
    del dw
    torch.cuda.empty_cache()
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=128)
    ap.add_argument("--warmup", type=int, default=128)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extra-settings", action="store_true")
    ap.add_argument("--no-layer-sweep", action="store_true")
    ap.add_argument("--extra-configs", default="dream7b,longctx",
                    help="other configured shapes to time ('' for none)")
    ap.add_argument("--extra-steps", type=int, default=16)
    ap.add_argument("--full-runs", action="store_true",
                    help="time whole runs of the extra configurations")
    ap.add_argument("--repeats", type=int, default=3,
                    help="extra timed regions of the configured setting (spread only)")
    ap.add_argument("--no-ceilings", action="store_true",
                    help="skip the measured copy / GEMM ceilings")
    ap.add_argument("--no-whole-runs", action="store_true",
                    help="skip the whole 128-step runs of the lock settings")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run 1 GiB device copies (counter calibration for profiles)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on exactly one GPU: the step engine has no multi-GPU path "
              "(data parallelism over sequences would need no per-step exchange).",
              file=sys.stderr)
        sys.exit(2)

    import torch
    import synth
    from selective_token_recompute_amd import engine as E

    shape, run = synth.CONFIGS["llada8b"]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    log("generating random-init weights on the device ...")
    dw = E.random_device_weights(shape, seed=0, device=dev)
    prompts = torch.from_numpy(synth.gen_prompts(shape, run)).to(dev)

    def factory(setting):
        return lambda: E.Engine(shape, dw, run, synth.LOCK_SETTINGS[setting], prompts)

    K, Wm = args.steps, args.warmup
    results = {}
    settings = ["natural"] + ([] if args.no_extra_settings
                              else ["scheduled", "vanilla", "slowfast", "refresh"])
    for s in settings:
        if Wm > 0:
            run_steps(factory(s), Wm)
        dt, toks, ms, _ = run_steps(factory(s), K)
        log(f"[{s}] {K} steps in {dt * 1e3:.1f} ms -> {K / dt:.1f} steps/s, "
            f"{toks / dt:.1f} tokens/s, mean M {sum(ms) / len(ms):.1f}")
        results[s] = dict(seconds=dt, tokens=toks, ms=ms)

    # whole 128-step runs of the lock settings, whatever --steps is: the
    # scheduled setting's locking shows only over a whole run
    whole = {}
    if not args.no_whole_runs:
        for s in ("natural", "scheduled", "refresh", "vanilla"):
            run_steps(factory(s), run.steps)
            fls = []
            dt, toks, ms, _ = run_steps(factory(s), run.steps, flops_out=fls)
            fl = sum(fls)
            whole[s] = dict(steps=run.steps, seconds=round(dt, 4),
                            steps_per_s=round(run.steps / dt, 3), tokens_per_s=round(toks / dt, 2),
                            mean_active_rows=round(sum(ms) / len(ms), 1), tflop=round(fl / 1e12, 3))
            log(f"[whole run/{s}] {run.steps} steps in {dt:.3f} s -> {run.steps / dt:.1f} steps/s, "
                f"mean M {sum(ms) / len(ms):.1f}")
        v = whole["vanilla"]
        for s in ("natural", "scheduled", "refresh"):
            whole[s]["speedup_vs_vanilla"] = round(v["seconds"] / whole[s]["seconds"], 3)
            whole[s]["flop_saving_vs_vanilla"] = round(1.0 - whole[s]["tflop"] / v["tflop"], 4)

    # the configured setting's timed region again, for its run-to-run spread
    spread = [K / nat_dt for nat_dt in (run_steps(factory("natural"), K)[0]
                                        for _ in range(args.repeats))]
    regions = sorted([K / results["natural"]["seconds"]] + spread)

    # per-kernel event timing over the same steps (configured setting)
    _, _, ms_nat, tim = run_steps(factory("natural"), K, timing=True)
    dom, roof = roofline_entry(tim, ms_nat)
    roof["traffic"] = measured_traffic(dom)
    kernels = {k: dict(ms_total=round(v["ms"], 3), launches=v["launches"],
                       us_avg=round(v["ms"] * 1e3 / max(v["launches"], 1), 2))
               for k, v in tim.items() if v["launches"]}
    for k, v in tim.items():
        if v["launches"] and v["ms"] > 0:
            avg = v["ms"] / 1e3 / v["launches"]
            if v["flops"] > 0:
                kernels[k]["tflops"] = round(v["flops"] / v["launches"] / avg / 1e12, 1)
            if v["bytes"] > 0:
                kernels[k]["gbs"] = round(v["bytes"] / v["launches"] / avg / 1e9, 1)
    log(f"dominant kernel: {dom} {roof}")

    nat = results["natural"]
    out = {
        "metric": METRIC,
        "value": round(K / nat["seconds"], 3),
        "unit": "steps/s",
        "tokens_per_s": round(nat["tokens"] / nat["seconds"], 2),
        "n_gpus": 1,
        "steps": K,
        "warmup": Wm,
        "ms_per_step": round(nat["seconds"] * 1e3 / K, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (random-init weights N(0,0.02), random prompts)",
        "config": {"workload": "LLaDA-8B-shaped denoising step, B=1, N=512 (128 prompt + 384 "
                               "masked), 128-step runs, lock: KL<=1e-3 & max-prob>=0.9 x2",
                   "global_batch": run.batch, "seq_len": run.seq_len, "parallelism": "none"},
        "mean_active_rows": round(sum(nat["ms"]) / len(nat["ms"]), 1),
        "repeats": dict(steps_per_s=[round(v, 3) for v in spread],
                        median=round(regions[len(regions) // 2], 3), min=round(regions[0], 3),
                        max=round(regions[-1], 3),
                        note="the same K timed steps run again after the timed region "
                             "(not part of value); median / min / max over all regions"),
        "roofline": roof,
        "kernels": kernels,
    }
    if whole:
        out["whole_run"] = dict(whole, note="one whole run per setting (timed after one whole "
                                             "warm-up run); FLOPs as the engine counts them per "
                                             "step (projections, FFN, attention, LM head on the "
                                             "active rows)")
    for s in settings[1:]:
        r = results[s]
        out[f"{s}_lock"] = dict(steps_per_s=round(K / r["seconds"], 3),
                                tokens_per_s=round(r["tokens"] / r["seconds"], 2),
                                mean_active_rows=round(sum(r["ms"]) / len(r["ms"]), 1))
    for name in [c for c in args.extra_configs.split(",") if c]:
        log(f"{name} ...")
        out[name] = extra_config(name, args.extra_steps, args.full_runs)
    if not args.no_ceilings:
        log("measured ceilings ...")
        out["ceilings"] = measured_ceilings()
        ach = out["roofline"]["achieved"]
        ceil = out["ceilings"]["gemm_bf16_tflops_hipblaslt" if out["roofline"]["bound"] == "mfma"
                               else "hbm_copy_gbs"]
        out["roofline"]["frac_of_measured_ceiling"] = round(ach / ceil, 4) if ceil else None
        out["roofline"]["measured_ceiling"] = ("hipBLASLt 8192^3 bf16" if
                                               out["roofline"]["bound"] == "mfma" else
                                               "1 GiB device copy")
    if not args.no_layer_sweep:
        log("single-layer roofline sweep ...")
        out["layer_isolation"] = layer_isolation()
        floor = out.get("ceilings", {}).get("small_copy_gbs", {}).get("16.8MB")
        if floor:
            for pt in out["layer_isolation"]["points"]:
                pt["attention_frac_of_small_copy"] = round(pt["attention_gbs"] / floor, 4)
            out["layer_isolation"]["small_copy_gbs"] = floor
    if not args.no_cpu_baseline:
        log("timing the oracle on a bounded sample ...")
        out["cpu_baseline"] = cpu_baseline(shape, run)
    if args.copy_calibration:
        copy_calibration()
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
