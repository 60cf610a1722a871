"""Benchmark of the attention hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline] [--no-decode]
                    [--no-projections] [--no-extra-workloads]

One step is one attn_prefill call (rotary embedding of k + cache append, then causal GQA
flash attention with q rotated in the kernel prologue) over the 28-layer, T = 1024,
12q/2kv x 128 prefill workload, with every input already resident in HBM.  `value` is
the prefill attention throughput in TFLOP/s, counting 4 * head_dim FLOPs per unmasked
(query, key) pair per query head (the two GEMMs; softmax and rotation not counted).

The same run also measures the decode side of the metric -- KV-cache GB/s of one
attn_decode step on the 28-layer batch-32 (4096-row) workload and on the 4-layer
batch-64 YaRN long-context workload -- with the 256 MB Infinity Cache flushed (a full
read of a 512 MB buffer) before every timed step; decode bytes count the cache rows read plus the new k/v read, the
appended row written and q read / out written.

Unless --no-extra-workloads is given, it also reports the prefill_kv workload (32 layers,
256 new tokens after 3840 cached rows, 32q/2kv; `prefill_kv`, TFLOP/s as above) and the
single-sequence decode workloads (28 layers, caches to 1024 and to 4096 rows; extra
`decode` entries, launch-dominated).

`roofline` describes the dominant kernel (the prefill flash kernel), timed per launch
with HIP events the library records around it on the launch stream (timestamp-only
events: created with hipEventDisableSystemFence, so recording one flushes no cache);
`cpu_baseline` is
the CPU oracle timed on a bounded sample of the same prefill workload.
Rank 0 prints one JSON line on stdout; progress goes to stderr.
"""
import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "prefill attn TFLOP/s (% MFMA peak) + decode KV-cache GB/s (% HBM peak)"
PEAK_F16_TFLOPS = 2500.0   # MI355X dense f16 MFMA
PEAK_HBM_GBS = 8000.0      # MI355X HBM3E

# HBM bytes per launch from rocprofv3 --pmc FETCH_SIZE and WRITE_SIZE passes of this script,
# scaled by what the same counters read for a plain 1 GiB device copy (FETCH_SIZE x 2.0,
# WRITE_SIZE x 1.0; profiles/hbm_traffic_counters.md).  `src` is the sha256 of the kernel
# source and the shared device headers at measurement time: once any changes, the
# figure no longer describes the kernel and `traffic` is reported as null.
TRAFFIC = {
    "prefill_attn:qwen1p5b_prefill_t1024": {
        "bytes": 2.7341e+08,
        "src": ("5e7ebc778f48f6ce2728ebcb49602a016a0580024a7e0c10b8b7ddf2ce7276ba",
                "a6d9dc8cd7255542c7eebeaa1756c1c71e09d777b53c8423adfc8fdfbedf5469",
                "3ebd6c561bb7e991ea26ae7ef7503854843410a2f2f1c272b5aca5cf584d513d")},
    "prefill_attn:h4096_prefill_kv_3840p256": {
        "bytes": 2.6894e+08,
        "src": ("5e7ebc778f48f6ce2728ebcb49602a016a0580024a7e0c10b8b7ddf2ce7276ba",
                "a6d9dc8cd7255542c7eebeaa1756c1c71e09d777b53c8423adfc8fdfbedf5469",
                "3ebd6c561bb7e991ea26ae7ef7503854843410a2f2f1c272b5aca5cf584d513d")},
    "decode_attn:qwen1p5b_decode_l4096_b32": {
        "bytes": 2.8411e+09,
        "src": ("6a983c6e07b32f232012d0e5df5d4bccc196a7216bb1dc9218f3accee79e27e4",
                "a6d9dc8cd7255542c7eebeaa1756c1c71e09d777b53c8423adfc8fdfbedf5469",
                "3ebd6c561bb7e991ea26ae7ef7503854843410a2f2f1c272b5aca5cf584d513d")},
    "decode_attn:yarn_decode_l32k_b64": {
        "bytes": 2.3069e+10,
        "src": ("6a983c6e07b32f232012d0e5df5d4bccc196a7216bb1dc9218f3accee79e27e4",
                "a6d9dc8cd7255542c7eebeaa1756c1c71e09d777b53c8423adfc8fdfbedf5469",
                "3ebd6c561bb7e991ea26ae7ef7503854843410a2f2f1c272b5aca5cf584d513d")},
    "decode_attn:qwen1p5b_decode_l1024_b1": {
        "bytes": 2.9481e+07,
        "src": ("6a983c6e07b32f232012d0e5df5d4bccc196a7216bb1dc9218f3accee79e27e4",
                "a6d9dc8cd7255542c7eebeaa1756c1c71e09d777b53c8423adfc8fdfbedf5469",
                "3ebd6c561bb7e991ea26ae7ef7503854843410a2f2f1c272b5aca5cf584d513d")},
    "decode_attn:qwen1p5b_decode_l4096_b1": {
        "bytes": 7.2235e+07,
        "src": ("6a983c6e07b32f232012d0e5df5d4bccc196a7216bb1dc9218f3accee79e27e4",
                "a6d9dc8cd7255542c7eebeaa1756c1c71e09d777b53c8423adfc8fdfbedf5469",
                "3ebd6c561bb7e991ea26ae7ef7503854843410a2f2f1c272b5aca5cf584d513d")},
}
KERNEL_SOURCES = {"prefill_attn": "prefill.hip", "decode_attn": "decode.hip"}


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def prefill_flops(n, t, hq, d, hist):
    """4*d FLOPs per unmasked (query, key) pair per query head."""
    pairs = 0
    for h0 in hist:
        pairs += t * (t + 1) // 2 + int(h0) * t
    return 4.0 * d * hq * pairs


def decode_bytes(lens, hq, hkv, d):
    lens = [int(x) for x in lens]
    per_unit_fixed = 2 * hkv * d * 2 + 2 * hkv * d * 2 + 2 * hq * d * 2
    return sum(2 * hkv * d * 2 * L for L in lens) + per_unit_fixed * len(lens)


def traffic(kernel, workload):
    """Counter-measured HBM bytes per launch, or None when the
    kernel source has changed since the counters were taken."""
    import hashlib
    rec = TRAFFIC.get(f"{kernel}:{workload}")
    if rec is None:
        return None
    csrc = os.path.join(ROOT, "kv_cache_causal_rope_amd", "csrc")
    now = tuple(hashlib.sha256(open(os.path.join(csrc, f), "rb").read()).hexdigest()
                for f in (KERNEL_SOURCES[kernel], "device_common.h", "rope_device.h"))
    return rec["bytes"] if now == rec["src"] else None


def make_events(n):
    import torch
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(n)]
    for e in evs:
        e.record()   # creates the underlying hipEvent
    torch.cuda.synchronize()
    return evs


class TimingEvent:
    """A HIP event that only takes a timestamp (hipEventDisableSystemFence): recording it
    neither writes back nor invalidates caches.  A default event does both when it is
    recorded, which, placed between two kernels, slows the kernel that follows (the T=1024
    flash kernel by ~10 % in kernel traces).  Used for the events the library records right
    before and after a kernel; read after a device synchronize."""
    _hip = None
    DISABLE_SYSTEM_FENCE = 0x20000000

    @classmethod
    def hip(cls):
        import ctypes
        if cls._hip is None:
            with open("/proc/self/maps") as f:   # the HIP runtime torch has loaded
                path = next(line.split()[-1] for line in f if "libamdhip64" in line)
            h = ctypes.CDLL(path)
            h.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
            h.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
            h.hipEventDestroy.argtypes = [ctypes.c_void_p]
            cls._hip = h
        return cls._hip

    def __init__(self):
        import ctypes
        ev = ctypes.c_void_p()
        if self.hip().hipEventCreateWithFlags(ctypes.byref(ev), self.DISABLE_SYSTEM_FENCE) != 0:
            raise RuntimeError("hipEventCreateWithFlags failed")
        self.cuda_event = ev.value

    def elapsed_time(self, end):
        import ctypes
        ms = ctypes.c_float()
        if self.hip().hipEventElapsedTime(ctypes.byref(ms), ctypes.c_void_p(self.cuda_event),
                                          ctypes.c_void_p(end.cuda_event)) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return ms.value

    def __del__(self):
        import ctypes
        if self._hip is not None and getattr(self, "cuda_event", None):
            self._hip.hipEventDestroy(ctypes.c_void_p(self.cuda_event))


def timing_events(n):
    return [TimingEvent() for _ in range(n)]


def bench_prefill(kv, W, name, steps, warmup):
    import torch
    cfg = W.CONFIGS[name]
    inp = W.make_inputs(cfg, device="cuda")
    rp = kv.RopeParams.from_fields(cfg.rope)
    out = torch.empty_like(inp.q)
    hist = inp.lens.cpu().numpy()
    call = (lambda: kv.prefill(inp.q, inp.k, inp.v, inp.positions, inp.cache_k, inp.cache_v, rp,
                               scale=cfg.scale, out=out)) if cfg.phase == "prefill" else \
        (lambda: kv.prefill_kv(inp.q, inp.k, inp.v, inp.positions, inp.cache_k, inp.cache_v,
                               inp.lens, int(hist.max()), rp, scale=cfg.scale, out=out))
    for _ in range(warmup):
        call()
    torch.cuda.synchronize()
    # whole-step throughput: K back-to-back steps
    t0, t1 = make_events(2)
    t0.record()
    for _ in range(steps):
        call()
    t1.record()
    torch.cuda.synchronize()
    ms_step = t0.elapsed_time(t1) / steps
    # per-launch duration of the flash kernel (timestamp-only events recorded by the library)
    evb, eva = timing_events(steps), timing_events(steps)
    for i in range(steps):
        kv.set_profile_events(evb[i], eva[i])
        call()
    torch.cuda.synchronize()
    k_ms = sum(evb[i].elapsed_time(eva[i]) for i in range(steps)) / steps
    flops = prefill_flops(cfg.n, cfg.t, cfg.hq, cfg.d, hist)
    return cfg, ms_step, k_ms, flops


def bench_decode(kv, W, name, steps, warmup):
    import numpy as np
    import torch
    cfg = W.CONFIGS[name]
    inp = W.make_inputs(cfg, device="cuda")
    rp = kv.RopeParams.from_fields(cfg.rope)
    lens = inp.lens.cpu().numpy()
    max_len = int(lens.max())
    ws = torch.empty(max(kv.workspace_size(cfg.n, cfg.hq, cfg.hkv, max_len), 16), dtype=torch.uint8,
                     device="cuda")
    out = torch.empty_like(inp.q)
    # Infinity Cache (256 MB) eviction between timed steps: a full read of a 512 MB buffer.
    # A read leaves the cache holding clean lines of that buffer, so the timed kernel reads
    # the KV cache from HBM and pays no write-back of the eviction traffic (filling the
    # buffer instead leaves 256 MB of dirty lines that drain to HBM inside the timed
    # kernel: measured 8-10 % lower GB/s on the 28-layer batch-32 cache).
    flush = torch.zeros(128 << 20, dtype=torch.int32, device="cuda")

    def call():
        kv.decode(inp.q, inp.k, inp.v, inp.positions, inp.cache_k, inp.cache_v, inp.lens, max_len,
                  rp, scale=cfg.scale, out=out, workspace=ws)

    for _ in range(warmup):
        call()
    torch.cuda.synchronize()
    # whole step (rotation + append + attention kernel, then the combine kernel): events
    # around the call only
    ca, cb = make_events(steps), make_events(steps)
    for i in range(steps):
        flush.sum()                    # evict the Infinity Cache between steps
        ca[i].record()
        call()
        cb[i].record()
    torch.cuda.synchronize()
    call_ms = sum(ca[i].elapsed_time(cb[i]) for i in range(steps)) / steps
    # the attention kernel alone, in a pass of its own: the library's (timestamp-only)
    # events around it
    evb, eva = timing_events(steps), timing_events(steps)
    for i in range(steps):
        flush.sum()
        kv.set_profile_events(evb[i], eva[i])
        call()
    torch.cuda.synchronize()
    k_ms = sum(evb[i].elapsed_time(eva[i]) for i in range(steps)) / steps
    nbytes = decode_bytes(lens, cfg.hq, cfg.hkv, cfg.d)
    # the attention kernel moves all of it except the output rows, which the combine
    # kernel writes
    kbytes = nbytes - cfg.n * cfg.hq * cfg.d * 2
    # measured ceiling of this access pattern: a kernel that only reads the same cache
    # rows (rows 0..len of K and V), split into chunks exactly as the decode kernel splits
    # them for this shape, timed the same way
    chunk = kv.decode_chunk_keys(cfg.n, cfg.hq, cfg.hkv, max_len)
    sink = torch.zeros(16, dtype=torch.uint8, device="cuda")
    pa, pb = make_events(steps), make_events(steps)
    for i in range(steps):
        flush.sum()
        pa[i].record()
        probes.stream_rows(inp.cache_k, inp.cache_v, inp.lens, max_len, chunk, sink)
        pb[i].record()
    torch.cuda.synchronize()
    probe_ms = sum(pa[i].elapsed_time(pb[i]) for i in range(steps)) / steps
    probe_bytes = 2 * cfg.hkv * cfg.d * 2 * int((lens.astype(np.int64) + 1).sum())
    del inp, flush, ws
    torch.cuda.empty_cache()
    return cfg, call_ms, k_ms, nbytes, kbytes, probe_bytes / probe_ms / 1e6, chunk


def measured_hbm_read():
    """The plain HBM read ceiling: a 4 GiB buffer read once front to back with 16-byte lane
    loads (Infinity Cache evicted first), best of a few grid sizes and repeats."""
    import torch
    buf = torch.ones(4 << 30, dtype=torch.uint8, device="cuda")
    flush = torch.zeros(128 << 20, dtype=torch.int32, device="cuda")
    sink = torch.zeros(16, dtype=torch.uint8, device="cuda")
    best = (0.0, 0)
    for blocks in (256, 1024, 4096, 8192):
        for _ in range(3):
            flush.sum()
            e0, e1 = make_events(2)
            e0.record()
            probes.read(buf, blocks, sink)
            e1.record()
            torch.cuda.synchronize()
            gbs = buf.numel() / (e0.elapsed_time(e1) * 1e-3) / 1e9
            best = max(best, (gbs, blocks))
    del buf, flush
    torch.cuda.empty_cache()
    return {"hbm_read_gbs": round(best[0], 1),
            "what": f"4 GiB read once with 16-byte lane loads, best of 4 grid sizes x 3 runs "
                    f"({best[1]} workgroups); Infinity Cache evicted before each run"}


def measured_mfma(kv):
    """f16 MFMA throughput a plain chain of independent 32x32x16 MFMAs reaches (two waves
    per SIMD on every CU), and the shader clock the matrix cores ran at meanwhile."""
    import torch
    ncu = torch.cuda.get_device_properties(0).multi_processor_count
    blocks, iters = 2 * ncu, 4096
    sink = torch.zeros(4 + 4 * blocks, dtype=torch.int64, device="cuda")
    probes.mfma(blocks, 64, sink)                   # warm-up
    torch.cuda.synchronize()
    e0, e1 = make_events(2)
    e0.record()
    probes.mfma(blocks, iters, sink)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1)
    flops = blocks * 4 * iters * 4 * (2 * 32 * 32 * 16)
    c = sink[4:].view(blocks, 4).cpu().double()
    mhz = float(((c[:, 3] - c[:, 2]) / (c[:, 1] - c[:, 0])).mean()) * 100.0
    return {"mfma_f16_tflops": round(flops / ms / 1e9, 1), "sclk_mhz": round(mhz, 0),
            "what": f"{blocks} workgroups x 4 waves x {iters} rounds of 4 independent "
                    f"v_mfma_f32_32x32x16_f16; clock from the shader and 100 MHz counters"}


def bench_projections(kv, steps, warmup):
    """The projections either side of attention on the 28-layer T=1024 Qwen-1.5B-style
    prefill (hidden 1536, 12q/2kv x 128, one weight matrix per layer): the fused QKV
    projection (k rotated and appended in its epilogue) and the output projection with the
    residual, each as TFLOP/s over its 2 * tokens * N * K FLOPs."""
    import torch
    layers, t, hidden, hq, hkv, d = 28, 1024, 1536, 12, 2, 128
    g = torch.Generator(device="cuda").manual_seed(5)
    rn = lambda *shape, s=1.0: (torch.randn(shape, generator=g, device="cuda") * s).half()
    x = rn(layers, t, hidden)
    w_qkv = rn(layers, (hq + 2 * hkv) * d, hidden, s=hidden ** -0.5)
    w_o = rn(layers, hidden, hq * d, s=(hq * d) ** -0.5)
    ck = torch.zeros(layers, hkv, t, d, dtype=torch.float16, device="cuda")
    cv = torch.zeros_like(ck)
    pos = torch.arange(t, dtype=torch.int32, device="cuda").repeat(layers, 1).contiguous()
    lens = torch.zeros(layers, dtype=torch.int32, device="cuda")
    q = torch.empty(layers, t, hq, d, dtype=torch.float16, device="cuda")
    attn = rn(layers, t, hq, d)
    out = torch.empty_like(x)
    rp = kv.RopeParams.plain()
    res = {}
    for name, call, flops in [
            ("qkv_project", lambda: kv.qkv_project(x, w_qkv, pos, ck, cv, lens, 0, rp, hq, hkv, q_out=q),
             2.0 * layers * t * (hq + 2 * hkv) * d * hidden),
            ("out_project", lambda: kv.out_project(attn, w_o, x, out=out), 2.0 * layers * t * hidden * hq * d)]:
        for _ in range(warmup):
            call()
        torch.cuda.synchronize()
        e0, e1 = make_events(2)
        e0.record()
        for _ in range(steps):
            call()
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / steps
        tf = flops / (ms * 1e-3) / 1e12
        res[name] = {"tflops": round(tf, 1), "us": round(ms * 1e3, 1), "flops": flops,
                     "frac_of_f16_peak": round(tf / PEAK_F16_TFLOPS, 4)}
    del x, w_qkv, w_o, ck, cv, q, attn, out
    torch.cuda.empty_cache()
    res["workload"] = "28 layers x T=1024, hidden 1536, 12q/2kv x 128, per-layer weights"
    return res


def oracle_time(W, name, units, threads, min_sec=0.0, max_runs=1):
    """Seconds the oracle (untuned, fp64, OpenMP on `threads` threads) takes for `units`
    layers of a prefill workload, run in this process (which touches no GPU): the mean of
    repeated runs until `min_sec` of work or `max_runs` runs (each run appends the same rows
    again, so every run does the same work); prints one JSON line."""
    import numpy as np
    import torch
    import oracle
    cfg = W.CONFIGS[name]
    inp = W.make_inputs(cfg, n=units)
    bits = lambda x: x.contiguous().view(torch.int16).numpy().view(np.uint16)
    ck, cv = bits(inp.cache_k).copy(), bits(inp.cache_v).copy()
    r = cfg.rope
    rp = oracle.RopeParams(base=r.base, n_rot=r.n_rot, yarn=r.yarn, freq_scale=r.freq_scale,
                           ext_factor=r.ext_factor, n_ctx_orig=r.n_ctx_orig, beta_fast=r.beta_fast,
                           beta_slow=r.beta_slow, mscale=r.mscale)
    oracle.set_num_threads(threads)
    args = (bits(inp.q), bits(inp.k), bits(inp.v), inp.positions.numpy(), ck, cv, inp.lens.numpy(), cfg.scale, rp)
    total, runs = 0.0, 0
    while runs < max(1, max_runs) and (runs == 0 or total < min_sec):
        t0 = time.perf_counter()
        oracle.prefill_kv(*args)
        total += time.perf_counter() - t0
        runs += 1
    flops = prefill_flops(units, cfg.t, cfg.hq, cfg.d, inp.lens.numpy())
    print(json.dumps({"sec": total / runs, "runs": runs, "total_sec": total, "flops": flops,
                      "threads": oracle.num_threads()}), flush=True)


def cpu_baseline(name, st_units):
    """The oracle on the whole prefill workload with every host thread, and single-threaded
    on the tiny T = 64 workload and on `st_units` layers of the prefill workload; each run
    in a child process that touches no GPU."""
    import subprocess
    threads = int(os.environ.get("OMP_NUM_THREADS", "0")) or len(os.sched_getaffinity(0))

    def run(workload, units, nthreads, min_sec=0.0, max_runs=1):
        out = subprocess.run([sys.executable, os.path.abspath(__file__), "--oracle-time", workload, str(units),
                              str(nthreads), str(min_sec), str(max_runs)],
                             capture_output=True, text=True, check=True).stdout
        return json.loads(out.strip().splitlines()[-1])

    model = "unknown"
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    full = run(name, 28, threads, min_sec=10.0, max_runs=30)  # about 10 s of work
    tiny = run("tiny_prefill_t64", 1, 1)
    one = run(name, st_units, 1)
    return {"value": full["flops"] / full["sec"] / 1e12, "unit": "TFLOP/s", "cores": full["threads"],
            "kind": "oracle",
            "sample": f"all 28 layers of {name} (T=1024, 12q/2kv x 128), full causal prefill incl. "
                      f"rotary + append, {full['sec']:.2f} s per run on {full['threads']} threads, "
                      f"mean of {full['runs']} runs ({full['total_sec']:.1f} s)",
            "cpu_model": model,
            "single_thread": {
                "threads": one["threads"],
                "tiny_prefill_t64_s": round(tiny["sec"], 4),
                "tiny_prefill_t64_tflops": tiny["flops"] / tiny["sec"] / 1e12,
                f"{name}_{st_units}_layers_s": round(one["sec"], 2),
                f"{name}_tflops": one["flops"] / one["sec"] / 1e12}}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="qwen1p5b_prefill_t1024")
    ap.add_argument("--cpu-single-thread-units", type=int, default=4,
                    help="layers of the prefill workload the single-thread oracle run takes")
    ap.add_argument("--oracle-time", nargs=5, metavar=("WORKLOAD", "UNITS", "THREADS", "MIN_SEC", "MAX_RUNS"),
                    help=argparse.SUPPRESS)  # child process of the CPU baseline
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-projections", action="store_true")
    ap.add_argument("--no-extra-workloads", action="store_true",
                    help="skip the prefill_kv workload (32 layers, 256 new tokens after 3840 cached "
                         "rows) and the single-sequence decode workloads")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain 1 GiB device copy (the reference for HBM byte counters)")
    args = ap.parse_args()
    if args.oracle_time:
        from kv_cache_causal_rope_amd import workloads as W
        oracle_time(W, args.oracle_time[0], int(args.oracle_time[1]), int(args.oracle_time[2]),
                    float(args.oracle_time[3]), int(args.oracle_time[4]))
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this attention path runs on a single MI355X "
              "(no collectives); rerun with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch
    import kv_cache_causal_rope_amd as kv
    from kv_cache_causal_rope_amd import workloads as W
    global probes
    from kv_cache_causal_rope_amd import probes

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    kv.lib()

    if args.copy_calibration:
        # a plain copy of known size: what FETCH_SIZE / WRITE_SIZE read for 1 GiB each way
        src = torch.empty(1 << 30, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
        torch.cuda.empty_cache()

    log(f"[bench] prefill {args.workload}: warmup {args.warmup}, steps {args.steps}")
    cfg, ms_step, k_ms, flops = bench_prefill(kv, W, args.workload, args.steps, args.warmup)
    value = flops / (ms_step * 1e-3) / 1e12
    achieved = flops / (k_ms * 1e-3) / 1e12
    log(f"[bench] prefill: {ms_step * 1e3:.1f} us/step, flash kernel {k_ms * 1e3:.1f} us, "
        f"{value:.1f} TFLOP/s step, {achieved:.1f} TFLOP/s kernel")
    torch.cuda.empty_cache()

    pkv = None
    if not args.no_extra_workloads:
        name = "h4096_prefill_kv_3840p256"
        log(f"[bench] prefill_kv {name}")
        pcfg, p_ms, pk_ms, pflops = bench_prefill(kv, W, name, max(5, args.steps // 2), min(args.warmup, 3))
        pkv = {"workload": name, "value": round(pflops / (p_ms * 1e-3) / 1e12, 2), "unit": "TFLOP/s",
               "ms_per_step": round(p_ms, 5), "flops_per_step": pflops,
               "roofline": {"bound": "mfma", "achieved": round(pflops / (pk_ms * 1e-3) / 1e12, 2),
                            "peak": PEAK_F16_TFLOPS, "unit": "TFLOP/s",
                            "frac": round(pflops / (pk_ms * 1e-3) / 1e12 / PEAK_F16_TFLOPS, 4),
                            "traffic": traffic("prefill_attn", name)}}
        log(f"[bench] prefill_kv: {p_ms * 1e3:.1f} us/step, flash kernel {pk_ms * 1e3:.1f} us, "
            f"{pkv['value']:.1f} TFLOP/s step, {pkv['roofline']['achieved']:.1f} TFLOP/s kernel")
        torch.cuda.empty_cache()

    decode = []
    if not args.no_decode:
        # the two large decode workloads, then the single-sequence ones (launch-dominated)
        names = ["qwen1p5b_decode_l4096_b32", "yarn_decode_l32k_b64"]
        if not args.no_extra_workloads:
            names += ["qwen1p5b_decode_l1024_b1", "qwen1p5b_decode_l4096_b1"]
        for name in names:
            log(f"[bench] decode {name}")
            dcfg, call_ms, dk_ms, nbytes, kbytes, ceil_gbs, chunk = bench_decode(
                kv, W, name, max(3, args.steps // 2), min(args.warmup, 3))
            gbs = nbytes / (call_ms * 1e-3) / 1e9
            kgbs = kbytes / (dk_ms * 1e-3) / 1e9
            log(f"[bench] decode {name}: {call_ms * 1e3:.1f} us/step, split kernel "
                f"{dk_ms * 1e3:.1f} us, {gbs:.0f} GB/s step, {kgbs:.0f} GB/s kernel; "
                f"read-only stream of the same rows {ceil_gbs:.0f} GB/s")
            decode.append({"workload": name, "value": round(gbs, 1), "unit": "GB/s",
                           "ms_per_step": round(call_ms, 4), "bytes_per_step": nbytes,
                           "frac_of_hbm_peak": round(gbs / PEAK_HBM_GBS, 4),
                           "roofline": {"bound": "hbm", "achieved": round(kgbs, 1),
                                        "peak": PEAK_HBM_GBS, "unit": "GB/s",
                                        "frac": round(kgbs / PEAK_HBM_GBS, 4),
                                        "traffic": traffic("decode_attn", name),
                                        "kernel_bytes": kbytes,
                                        "what": "attention kernel (rotation, append, split-key "
                                                "attention); its bytes exclude the output rows"},
                           "stream_ceiling": {"value": round(ceil_gbs, 1), "unit": "GB/s",
                                              "what": f"read-only kernel over the same cache rows, "
                                                      f"same split ({chunk}-key chunks at most)",
                                              "kernel_frac": round(kgbs / ceil_gbs, 4)}})

    proj = None
    if not args.no_projections:
        proj = bench_projections(kv, max(5, args.steps // 2), min(args.warmup, 3))
        log(f"[bench] projections: QKV {proj['qkv_project']['tflops']:.0f} TFLOP/s "
            f"({proj['qkv_project']['us']:.1f} us), out {proj['out_project']['tflops']:.0f} TFLOP/s "
            f"({proj['out_project']['us']:.1f} us)")

    ceilings = measured_mfma(kv)
    ceilings.update(measured_hbm_read())
    log(f"[bench] plain HBM read: {ceilings['hbm_read_gbs']:.0f} GB/s")
    log(f"[bench] f16 MFMA microbenchmark: {ceilings['mfma_f16_tflops']:.0f} TFLOP/s at "
        f"{ceilings['sclk_mhz']:.0f} MHz shader clock")

    cpu = None
    if not args.no_cpu_baseline:
        log(f"[bench] cpu baseline: oracle on all 28 layers, then single-threaded runs")
        cpu = cpu_baseline(args.workload, args.cpu_single_thread_units)
        log(f"[bench] cpu baseline: {cpu['value'] * 1e3:.2f} GFLOP/s on {cpu['cores']} threads "
            f"({cpu['cpu_model']}); single thread {cpu['single_thread']}")

    line = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic",
        "config": {"workload": cfg.name, "layers": cfg.layers, "batch": cfg.batch, "t": cfg.t,
                   "hq": cfg.hq, "hkv": cfg.hkv, "head_dim": cfg.d, "rope": "plain base 1e4",
                   "flops_per_step": flops},
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_F16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(achieved / PEAK_F16_TFLOPS, 4),
                     "traffic": traffic("prefill_attn", cfg.name)},
        "prefill_kv": pkv,
        "decode": decode,
        "projections": proj,
        "measured_ceilings": ceilings,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
