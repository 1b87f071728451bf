"""Benchmark: MoE grouped GEMM forward + backward on one MI355X.

One step = the whole grouped-GEMM hot path over one batch of the balanced
bf16 workload (E=8 experts, M=1024 token rows split 128 per expert with the
group sizes resident on the device, K=4096, N=6400; X and W uniform[0,1),
dY = ones, the gradient of the output's sum):
    Y  = X_g . W_g          (gmm_fwd)
    dX = dY_g . W_g^T       (gmm_bwd)
    dW = X_g^T . dY_g       (gmm_bwd, dynamic K)
Each product is one kernel launch (the device argument builder runs in the
kernel prologue).  Inputs are resident in HBM before the timed region.

Also reported: the dominant kernel against its roofline (HIP events around
every launch in the timed region), the fp64 CPU oracle timed on a bounded
sample of the same workload, and the sparse-M latency of the F8I4 grouped
GEMM (one routed token over 128 experts, K=5120, N=8192) next to the same
call with a single expert.

Usage: python bench.py [--gpus 1] [--steps 100] [--warmup 200] [--no-cpu]
(The GPU's clocks settle only after some tens of milliseconds of sustained
work: with 5 warmup steps, 1.5 ms, the timed steps of the balanced step ran
at 487-497 TFLOP/s, with 200 at 645-653 on the same box; the defaults
measure the steady state.)
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "grouped-GEMM TFLOP/s & % MFMA peak; µs latency at total_M=1, 128 groups"
PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0          # MI355X HBM3E
PEAK_FP8_TFLOPS = 5000.0       # MI355X dense fp8 MFMA


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def balanced_inputs(torch, mg, E=8, M=1024, K=4096, N=6400, seed=0):
    import numpy as np
    import workloads as wl
    c = wl.balanced_bf16(seed=seed, E=E, M=M, K=K, N=N)
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()
    return dict(x=t(c["X"]), w=t(c["W"]), dy=t(c["dY"]), sizes=torch.from_numpy(c["sizes"]).cuda(), host=c)


def algorithmic_bytes(E, M, K, N):
    """Bytes each GEMM must move at least once (bf16): forward reads W, X and
    writes Y; dX reads W, dY and writes dX; dW reads X, dY and writes dW."""
    w = E * K * N * 2
    return {"fwd": w + M * K * 2 + M * N * 2, "dx": w + M * N * 2 + M * K * 2, "dw": w + M * K * 2 + M * N * 2}


KERNEL_SOURCES = ["moe_grouped_gemm_device_amd/csrc/gmm.hip", "moe_grouped_gemm_device_amd/csrc/gemm_dev.h",
                  "moe_grouped_gemm_device_amd/csrc/worklist.h", "moe_grouped_gemm_device_amd/csrc/common.h",
                  "moe_grouped_gemm_device_amd/csrc/kernels.h"]
TRAFFIC_PROFILE = "profiles/gmm_bf16_balanced_traffic.md"


def kernel_source_digest():
    """SHA-256 over the sources the GEMM kernel is built from."""
    import hashlib
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def measured_traffic(which):
    """HBM bytes per launch of `which` from the committed rocprofv3 counter
    summary (FETCH_SIZE + WRITE_SIZE, each scaled by the factor a plain copy
    of known size gives), or None when that summary was taken on other kernel
    sources than the ones in the tree."""
    path = os.path.join(ROOT, TRAFFIC_PROFILE)
    if not os.path.exists(path):
        return None
    vals = {}
    for line in open(path):
        line = line.strip().strip("`")
        if "=" in line and line.split("=")[0].strip().replace("_", "").replace(".", "").isalnum():
            k, v = line.split("=", 1)
            vals[k.strip()] = v.strip()
    if vals.get("kernel_source_sha256") != kernel_source_digest():
        return None
    key = f"traffic_bytes.{which}"
    return int(vals[key]) if key in vals else None


def traffic_probe(torch, mg):
    """Runs each product of the step a few times and a plain copy of known
    size, for rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE passes (no timing)."""
    E, M, K, N = 8, 1024, 4096, 6400
    d = balanced_inputs(torch, mg, E, M, K, N)
    x, w, dy, sizes = d["x"], d["w"], d["dy"], d["sizes"]
    y = torch.empty(M, N, dtype=torch.bfloat16, device="cuda")
    dx = torch.empty(M, K, dtype=torch.bfloat16, device="cuda")
    dw = torch.empty_like(w)
    ws = mg.workspace(E, M)
    src = torch.ones(256 << 20, dtype=torch.uint8, device="cuda")   # copy calibration: 256 MiB each way
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
        mg.gmm_fwd(x, w, sizes, out=y, ws=ws)
        mg.gmm_bwd(dy, x, w, sizes, need_dw=False, dx=dx, ws=ws)
        mg.gmm_bwd(dy, x, w, sizes, need_dx=False, dw=dw, ws=ws)
    torch.cuda.synchronize()
    log("traffic probe done; kernel source sha256 " + kernel_source_digest())


def run_gpu(args, torch, mg):
    E, M, K, N = 8, 1024, 4096, 6400
    log("generating inputs")
    d = balanced_inputs(torch, mg, E, M, K, N)
    x, w, dy, sizes = d["x"], d["w"], d["dy"], d["sizes"]
    y = torch.empty(M, N, dtype=torch.bfloat16, device="cuda")
    dx = torch.empty(M, K, dtype=torch.bfloat16, device="cuda")
    dw = torch.empty_like(w)
    ws = mg.workspace(E, M)

    products = {
        "fwd": lambda: mg.gmm_fwd(x, w, sizes, out=y, ws=ws),
        "dx": lambda: mg.gmm_bwd(dy, x, w, sizes, need_dw=False, dx=dx, ws=ws),
        "dw": lambda: mg.gmm_bwd(dy, x, w, sizes, need_dx=False, dw=dw, ws=ws),
    }

    def step():
        for fn in products.values():
            fn()

    log(f"warmup {args.warmup}")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    # The timed steps carry no per-launch events: an event marker between two
    # kernels costs several microseconds of idle GPU on ROCm.
    log(f"timing {args.steps} steps")
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    # Per-kernel durations: the same K steps once more, with a HIP event pair
    # around every launch (on the stream the library launches on), so each
    # product's average launch duration is measured in the step it belongs
    # to.  (The timed steps above carry no events: an event marker between
    # two kernels leaves the GPU idle for a few microseconds.)
    samples = {name: [] for name in products}
    pairs = []
    for _ in range(args.steps):
        for name, fn in products.items():
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            fn()
            e1.record()
            pairs.append((name, e0, e1))
    torch.cuda.synchronize()
    for name, e0, e1 in pairs:
        samples[name].append(e0.elapsed_time(e1))
    step_ms = {name: sum(v) / len(v) for name, v in samples.items()}
    # R launches of one product back to back, one event pair around them
    # (only the dispatch gap between identical kernels is counted besides the
    # kernels themselves): the average the roofline uses
    R = max(args.steps, 5)
    b2b_ms = {}
    for name, fn in products.items():
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(R):
            fn()
        e1.record()
        e1.synchronize()
        b2b_ms[name] = e0.elapsed_time(e1) / R
    avg_ms = b2b_ms
    launch_stats = {name: launch_percentiles(torch, fn, reps=20) for name, fn in products.items()}
    # the pages' A100 figure is the total kernel time of 30 forward + backward
    # iterations: the same 30 steps here, back to back, HIP events around them
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(30):
        step()
    e1.record()
    e1.synchronize()
    total30_ms = e0.elapsed_time(e1)
    flops_step = 3 * 2.0 * M * K * N
    ms_step = elapsed * 1e3 / args.steps
    tflops = flops_step / (ms_step * 1e-3) / 1e12
    bytes_per = algorithmic_bytes(E, M, K, N)
    dom = max(avg_ms, key=avg_ms.get)
    achieved = bytes_per[dom] / (avg_ms[dom] * 1e-3) / 1e9
    kernel_names = {"fwd": "gmm_kernel<128,256,3,true,false,FIXED_M,bf16,8 waves> (forward: X rows k-contiguous, W [K,N])",
                    "dx": "gmm_kernel<128,256,3,true,true,FIXED_M,bf16,8 waves> (dX: dY rows, W rows contraction-contiguous)",
                    "dw": "gmm_kernel<256,256,2,false,false,DYNAMIC_K,bf16,8 waves> (dW: X and dY row-contiguous)"}
    roofline = {
        "bound": "hbm",
        "kernel": kernel_names[dom],
        "achieved": round(achieved, 1),
        "peak": PEAK_HBM_GBS,
        "unit": "GB/s",
        "frac": round(achieved / PEAK_HBM_GBS, 4),
        "traffic": measured_traffic(dom),
        "algorithmic_bytes_per_launch": bytes_per[dom],
        "avg_launch_us": {k: round(v * 1e3, 2) for k, v in avg_ms.items()},
        "avg_launch_us_how": f"{R} launches of each product back to back between one HIP event pair",
        "avg_launch_us_in_steps": {k: round(v * 1e3, 2) for k, v in step_ms.items()},
        "avg_launch_us_in_steps_how": f"HIP event pair around every launch of {args.steps} more steps "
                                      "(fwd, dX, dW in turn)",
        "launch_us_percentiles": launch_stats,
        "mfma_frac": {k: round(2.0 * M * K * N / (v * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4) for k, v in avg_ms.items()},
    }
    return dict(value=tflops, ms_per_step=ms_step, roofline=roofline, E=E, M=M, K=K, N=N, host=d["host"],
                total30_ms=total30_ms)


_FLUSH = None


def _flush_caches(torch):
    """Writes 1 GiB, four times the 256 MB Infinity Cache, so the next kernel
    finds none of its operands cached (L2 and the Infinity Cache)."""
    global _FLUSH
    if _FLUSH is None:
        _FLUSH = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
    _FLUSH.fill_(1)


def launch_percentiles(torch, fn, reps=20):
    """Median, p10 and p90 of single-launch durations (a HIP event pair
    around each launch), warm (launches back to back) and cold (caches
    flushed before each launch, outside the events)."""
    out = {}
    for cold in (False, True):
        times = []
        fn()
        torch.cuda.synchronize()
        for _ in range(reps):
            if cold:
                _flush_caches(torch)
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            fn()
            b.record()
            b.synchronize()
            times.append(a.elapsed_time(b) * 1e3)
        times.sort()
        q = lambda f: times[min(len(times) - 1, int(round(f * (len(times) - 1))))]
        out["cold" if cold else "warm"] = {"median": round(q(0.5), 2), "p10": round(q(0.1), 2), "p90": round(q(0.9), 2)}
    return out


def tiny_latency(torch, mg):
    """The tiny grouped GEMM (E=4, K=64, N=48, group sizes [0, 20, 9, 8]):
    forward and backward latency per launch (median, p10, p90)."""
    import numpy as np
    import workloads as wl
    c = wl.tiny_bf16(seed=0)
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()
    x, w, gs = t(c["X"]), t(c["W"]), torch.from_numpy(c["sizes"]).cuda()
    dy = t(wl.normal_bf16((c["M"], c["N"]), 1.0, 0, wl.T_DY))
    y = torch.empty(c["M"], c["N"], dtype=torch.bfloat16, device="cuda")
    dx, dw = torch.empty_like(x), torch.empty_like(w)
    ws = mg.workspace(4, c["M"])
    return {"workload": "E=4, K=64, N=48, group sizes [0,20,9,8] (total_M=37), bf16",
            "fwd_us": launch_percentiles(torch, lambda: mg.gmm_fwd(x, w, gs, out=y, ws=ws))["warm"],
            "dx_us": launch_percentiles(torch, lambda: mg.gmm_bwd(dy, x, w, gs, need_dw=False, dx=dx, ws=ws))["warm"],
            "dw_us": launch_percentiles(torch, lambda: mg.gmm_bwd(dy, x, w, gs, need_dx=False, dw=dw, ws=ws))["warm"]}


def measured_peaks(torch):
    """What this GPU sustains, measured beside the published peaks: device
    memory streams through torch (copy, read-only sum, write-only fill of
    1 GiB), and dense GEMMs through the vendor BLAS (torch.matmul in bf16,
    torch._scaled_mm in e4m3) at 8192 x 8192 x 8192.  Context only: none of
    these runs any part of the grouped-GEMM path."""
    def t(fn, reps=10):
        fn()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(reps):
            fn()
        b.record()
        b.synchronize()
        return a.elapsed_time(b) / reps * 1e3
    n = 1 << 30
    src = torch.ones(n // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    res = {"copy_GBps": round(2 * n / t(lambda: dst.copy_(src)) / 1e3, 1),
           "read_GBps": round(n / t(lambda: src.sum()) / 1e3, 1),
           "write_GBps": round(n / t(lambda: dst.fill_(2.0)) / 1e3, 1)}
    del src, dst
    S = 8192
    a = torch.randn(S, S, device="cuda").to(torch.bfloat16)
    b = torch.randn(S, S, device="cuda").to(torch.bfloat16)
    res["bf16_gemm_TFLOPs"] = round(2.0 * S ** 3 / t(lambda: torch.matmul(a, b)) / 1e6, 1)
    try:
        a8, b8 = a.to(torch.float8_e4m3fn), b.t().contiguous().to(torch.float8_e4m3fn).t()
        one = torch.ones((), device="cuda")
        res["fp8_gemm_TFLOPs"] = round(2.0 * S ** 3 / t(lambda: torch._scaled_mm(a8, b8, scale_a=one, scale_b=one,
                                                                             out_dtype=torch.bfloat16)) / 1e6, 1)
    except Exception as e:   # a torch build without the fp8 product
        res["fp8_gemm_TFLOPs"] = None
        res["fp8_gemm_error"] = str(e)[:160]
    res["what"] = ("sustained on this GPU: 1 GiB copy / fp32 sum / fill through torch, and the vendor BLAS at "
                   "8192^3 (bf16 matmul, e4m3 scaled_mm); published peaks: HBM 8000 GB/s, bf16 2500, fp8 5000 TFLOP/s")
    return res


def graph_replay_latency(torch, fn, reps=50):
    """Median of the event-timed replay of fn captured in a HIP graph."""
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    times = []
    for _ in range(5):
        g.replay()
    torch.cuda.synchronize()
    for _ in range(reps):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        g.replay()
        b.record()
        b.synchronize()
        times.append(a.elapsed_time(b) * 1e3)
    times.sort()
    return round(times[len(times) // 2], 2)


def sparse_m_latency(torch, mg, reps=50):
    """F8I4 grouped GEMM latency (hipEvent pairs, median) for one routed row
    among 128 experts vs the same row and weights with a single expert;
    K=5120, N=8192, W ~ N(0, 0.02) quantized to int4 by the library, X ~ N(0,1)
    quantized rowwise to e4m3."""
    E, K, N = 128, 5120, 8192
    g = torch.Generator(device="cuda")
    g.manual_seed(0)
    w4 = torch.empty(E, N, K // 2, dtype=torch.uint8, device="cuda")
    sw = torch.empty(E, K // 128, N, dtype=torch.bfloat16, device="cuda")
    for e in range(E):
        we = (torch.randn(1, K, N, generator=g, device="cuda") * 0.02).to(torch.bfloat16)
        q, s = mg.quantize_int4_weights(we)
        w4[e].copy_(q[0])
        sw[e].copy_(s[0])
    x = torch.randn(1, K, generator=g, device="cuda").to(torch.bfloat16)
    xq, sx = mg.quantize_rowwise_fp8(x)
    expert = int(torch.randint(0, E, (1,), generator=g, device="cuda").item())
    sizes128 = torch.zeros(E, dtype=torch.int32, device="cuda")
    sizes128[expert] = 1
    sizes1 = torch.ones(1, dtype=torch.int32, device="cuda")
    w4_1 = w4[expert:expert + 1].clone()
    sw_1 = sw[expert:expert + 1].clone()
    y = torch.empty(1, N, dtype=torch.bfloat16, device="cuda")
    ws = mg.workspace(E, 1)
    flush = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")

    def timed(fn, cold):
        times = []
        for _ in range(5):
            fn()
        for _ in range(reps):
            if cold:
                flush.fill_(1)
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            fn()
            b.record()
            b.synchronize()
            times.append(a.elapsed_time(b) * 1e3)
        times.sort()
        return times[len(times) // 2]

    run128 = lambda: mg.gmm_fwd_f8i4(xq, sx, w4, sw, sizes128, out=y, ws=ws)
    run1 = lambda: mg.gmm_fwd_f8i4(xq, sx, w4_1, sw_1, sizes1, out=y, ws=ws)
    res = {}
    for cold in (False, True):
        t128, t1 = timed(run128, cold), timed(run1, cold)
        key = "cold" if cold else "warm"
        res[key] = {"us_total_M1_E128": round(t128, 2), "us_total_M1_E1": round(t1, 2),
                    "ratio": round(t128 / t1, 3)}
    bytes_expert = N * K // 2 + (K // 128) * N * 2
    res["cold"]["hbm_frac"] = round(bytes_expert / (res["cold"]["us_total_M1_E128"] * 1e-6) / 1e9 / PEAK_HBM_GBS, 4)
    # total_M = 16 and 128 routed rows on uniformly random experts (warm):
    # weight bytes of the experts that have rows against HBM peak
    gen = torch.Generator()
    gen.manual_seed(1)
    for tm in (16, 128):
        picks = torch.randint(0, E, (tm,), generator=gen)
        sz = torch.bincount(picks, minlength=E).to(torch.int32).cuda()
        xm = torch.randn(tm, K, generator=g, device="cuda").to(torch.bfloat16)
        xqm, sxm = mg.quantize_rowwise_fp8(xm)
        ym = torch.empty(tm, N, dtype=torch.bfloat16, device="cuda")
        wsm = mg.workspace(E, tm)
        t = timed(lambda: mg.gmm_fwd_f8i4(xqm, sxm, w4, sw, sz, out=ym, ws=wsm), False)
        touched = int((sz > 0).sum().item())
        res[f"warm_total_M{tm}"] = {"us": round(t, 2), "experts_with_rows": touched,
                                    "hbm_frac": round(touched * bytes_expert / (t * 1e-6) / 1e9 / PEAK_HBM_GBS, 4)}
    res["graph_replay_us_total_M1_E128"] = graph_replay_latency(torch, run128)
    res["graph_replay_us_total_M1_E1"] = graph_replay_latency(torch, run1)
    res["workload"] = "F8I4: E=128, total_M=1 (one routed row), K=5120, N=8192; int4 per-128-K bf16 scales"
    return res


def _timeit(torch, fn, reps=10, settle_ms=30.0):
    """Average microseconds of fn over reps back-to-back launches (HIP events),
    after untimed launches covering about settle_ms of GPU time (at most
    200): the clocks settle only after some tens of milliseconds of
    sustained work, and each row starts after its inputs were made."""
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    fn()
    e1.record()
    e1.synchronize()
    one_ms = max(e0.elapsed_time(e1), 1e-3)
    for _ in range(min(200, int(settle_ms / one_ms))):
        fn()
    torch.cuda.synchronize()
    e0.record()
    for _ in range(reps):
        fn()
    e1.record()
    e1.synchronize()
    return e0.elapsed_time(e1) / reps * 1e3


def _row(what, us, amount, unit, peak):
    """One measured row: achieved = amount / time against the peak in unit."""
    scale = 1e3 if unit == "GB/s" else 1e6   # bytes/us -> GB/s, flops/us -> TFLOP/s
    achieved = amount / us / scale
    return {"what": what, "us": round(us, 2), "achieved": round(achieved, 1), "unit": unit, "peak": peak,
            "frac": round(achieved / peak, 4)}


def _row_cases(torch, mg):
    """The hot-path steps of the fp8 training layer (DeepSeek-MoE-16B share:
    16384 tokens, 64 experts, top-6 with Zipf(1.1) loads, hidden 2048,
    expert intermediate 1408) and of the token-sorted Mixtral-8x7B expert FFN
    (T=4096, top-2 of 8, hidden 4096, intermediate 14336), one at a time.
    Yields (key, what, fn, amount, unit, peak, reps); fn runs the step once
    and must be used before the next case is drawn (later cases may free or
    overwrite its inputs).  Inputs: seeded synthetic bf16 N(0,1) activations
    and N(0,0.02) weights."""
    import numpy as np
    import workloads as wl
    g = torch.Generator(device="cuda")
    g.manual_seed(0)
    # ---- fp8 layer share (configuration: DeepSeek-MoE-16B-shaped) ----------
    T, E, k, H, I = 16384, 64, 6, 2048, 1408
    ids = wl.zipf_topk_routing(T, E, k, 1.1, seed=0)
    sizes_np = np.bincount(ids.ravel(), minlength=E).astype(np.int32)
    M = T * k
    sizes = torch.from_numpy(sizes_np).cuda()
    X = torch.randn(M, H, generator=g, device="cuda").to(torch.bfloat16)
    dY = torch.randn(M, I, generator=g, device="cuda").to(torch.bfloat16)
    W = (torch.randn(E, H, I, generator=g, device="cuda") * 0.02).to(torch.bfloat16)
    ws = mg.workspace(E, M)
    xq = torch.empty(M, H, dtype=torch.uint8, device="cuda")
    sx = torch.empty(M, dtype=torch.float32, device="cuda")
    yield ("A5_quantize_rowwise_fp8", f"X [{M},{H}] bf16 -> e4m3 + row scales",
           lambda: mg.quantize_rowwise_fp8(X, q=xq, scales=sx), M * H * 3 + M * 4, "GB/s", PEAK_HBM_GBS, 10)
    ldc = mg.colwise_ld(M)   # code rows of the column-major operands, padded as the library pads them
    cq = (torch.zeros(I, ldc, dtype=torch.uint8, device="cuda")[:, :M],
          torch.empty(E, I, dtype=torch.float32, device="cuda"),
          torch.zeros(H, ldc, dtype=torch.uint8, device="cuda")[:, :M],
          torch.empty(E, H, dtype=torch.float32, device="cuda"))
    yield ("A6_quantize_colwise_dual", f"dY [{M},{I}] and X [{M},{H}], {E} Zipf groups -> column-major e4m3",
           lambda: mg.quantize_colwise_per_group_fp8(dY, sizes, b=X, out=cq),
           M * (I + H) * 3 + E * (I + H) * 4, "GB/s", PEAK_HBM_GBS, 10)
    dyc, sdyc, xc, sxc = cq
    wq_c, sw_c = mg.quantize_fp8_expert_weights(W)
    y = torch.empty(M, I, dtype=torch.bfloat16, device="cuda")
    yield ("A7_fp8_gmm_fwd", f"Y [{M},{I}] = Xq . Wq_g, K={H}",
           lambda: mg.gmm_fwd_fp8(xq, sx, wq_c, sw_c, None, H, sizes, I, out=y, ws=ws),
           2.0 * M * H * I, "TFLOP/s", PEAK_FP8_TFLOPS, 10)
    dyq = torch.empty(M, I, dtype=torch.uint8, device="cuda")
    sdy = torch.empty(M, dtype=torch.float32, device="cuda")
    mg.quantize_rowwise_fp8(dY, q=dyq, scales=sdy)
    wq_r, sw_r = mg.quantize_rowwise_fp8(W.reshape(E * H, I))
    dxo = torch.empty(M, H, dtype=torch.bfloat16, device="cuda")
    yield ("A7_fp8_gmm_dx", f"dX [{M},{H}] = dYq . Wq_g^T, contraction {I}",
           lambda: mg.gmm_bwd_fp8(sizes, H, I, dyq=dyq, sdy=sdy, wq=wq_r, sw=sw_r, w_ld=I,
                                  w_expert_stride=H * I, need_dw=False, dx=dxo, ws=ws),
           2.0 * M * H * I, "TFLOP/s", PEAK_FP8_TFLOPS, 10)
    dwo = torch.empty(E, H, I, dtype=torch.bfloat16, device="cuda")
    yield ("A7_fp8_gmm_dw", f"dW [{E},{H},{I}] = Xq_g^T . dYq_g (dynamic K)",
           lambda: mg.gmm_bwd_fp8(sizes, H, I, xc=xc, sxc=sxc, dyc=dyc, sdyc=sdyc, need_dx=False, dw=dwo, ws=ws),
           2.0 * M * H * I, "TFLOP/s", PEAK_FP8_TFLOPS, 10)
    yield ("A1_builder", f"work list for {E} groups, total_M={M}, 128-row tiles (own launch)",
           lambda: mg.build_worklist(mg.MG_WL_FIXED_M, sizes, M, 128), None, None, None, 10)
    del X, dY, W, xq, dyq, cq, wq_c, wq_r, y, dxo, dwo
    torch.cuda.empty_cache()
    # ---- the torchao page's colwise shapes: M=16640 rows, 2048 or 5120
    # columns, 64 or 128 groups cut at multiples of 16, randn bf16 input
    for Cp, Gp in ((2048, 64), (5120, 64), (2048, 128), (5120, 128)):
        Mp = 16640
        szp = torch.from_numpy(wl.jagged_sizes_multiple_of(Gp, Mp, 16, 0)).cuda()
        xp = torch.randn(Mp, Cp, generator=g, device="cuda").to(torch.bfloat16)
        outp = (torch.empty(Cp, Mp, dtype=torch.uint8, device="cuda"),
                torch.empty(Gp, Cp, dtype=torch.float32, device="cuda"))
        yield (f"A6_colwise_M{Mp}_C{Cp}_G{Gp}", f"single tensor [{Mp},{Cp}] bf16, {Gp} groups -> column-major e4m3",
               lambda: mg.quantize_colwise_per_group_fp8(xp, szp, out=outp),
               Mp * Cp * 3 + Gp * Cp * 4, "GB/s", PEAK_HBM_GBS, 10)
        del xp, outp
    del ws
    torch.cuda.empty_cache()
    # ---- token-sorted fused FFN (configuration: Mixtral-8x7B-shaped) -------
    T, E, k, H, I = 4096, 8, 2, 4096, 14336
    ids_np, wts_np = wl.softmax_topk_routing(T, E, k, seed=0)
    ids = torch.from_numpy(ids_np).cuda()
    wts = torch.from_numpy(wts_np).cuda()
    x = torch.randn(T, H, generator=g, device="cuda").to(torch.bfloat16)
    w1 = (torch.randn(E, H, 2 * I, generator=g, device="cuda") * 0.02).to(torch.bfloat16)
    w2 = (torch.randn(E, I, H, generator=g, device="cuda") * 0.02).to(torch.bfloat16)
    # the bf16 expert GEMMs take the weights in the (E, N, K) layout of the
    # applied-ai page's fused_moe_kernel: W1 as [E, 2I, H], W2 as [E, H, I]
    w1n, w2n = w1.transpose(1, 2).contiguous(), w2.transpose(1, 2).contiguous()
    logits = torch.randn(T, E, generator=g, device="cuda")
    yield ("A0_route_topk", f"router: fp32 softmax + top-{k} of {T}x{E} logits (renormalized)",
           lambda: mg.route_topk(logits, k, renormalize=True), T * E * 4 + T * k * 8, "GB/s", PEAK_HBM_GBS, 10)
    bm = 128
    p = mg.moe_permute(ids, E, bm, x=x)
    ntpp = int(p["num_tokens_post_padded"].item())
    yield ("A9_moe_permute", f"align + gather of {T}x{k} routed rows, hidden {H}, block_m {bm}",
           lambda: mg.moe_permute(ids, E, bm, x=x), T * H * 2 + ntpp * H * 2 + T * k * 8, "GB/s", PEAK_HBM_GBS, 10)
    yield ("A9_moe_align", f"align only (what the fused path runs): {T}x{k} routed rows, block_m {bm}",
           lambda: mg.moe_permute(ids, E, bm), T * k * 4 * 3 + ntpp * 4, "GB/s", PEAK_HBM_GBS, 10)
    xs, psz, sids = p["x_sorted"], p["padded_sizes"], p["sorted_token_ids"]
    wsf = mg.workspace(E, xs.shape[0])
    h1 = torch.empty(xs.shape[0], 2 * I, dtype=torch.bfloat16, device="cuda")
    yield ("A10_gemm1", f"H1 = X[sorted_ids / {k}] . W1_e (gather in the A load; W1 as [E, 2I, H]), {ntpp} padded "
                        f"rows, K={H}, N={2 * I} (useful flops of {T * k} rows)",
           lambda: mg.gmm_fwd_gather(x, sids, k, w1n, psz, trans_b=True, out=h1, ws=wsf), 2.0 * T * k * H * 2 * I,
           "TFLOP/s", PEAK_BF16_TFLOPS, 5)
    act = torch.empty(xs.shape[0], I, dtype=torch.bfloat16, device="cuda")
    yield ("A10_A11_gemm1_silu_fused", f"act = silu*mul(X[sorted_ids / {k}] . W1_e) in one kernel (what the fused path "
                                       f"runs; W1 as [E, 2I, H]), {ntpp} padded rows, K={H}, 2I={2 * I} (useful flops "
                                       f"of {T * k} rows)",
           lambda: mg.gmm_fwd_silu_mul(x, w1n, psz, sorted_token_ids=sids, top_k=k, trans_b=True, out=act, ws=wsf),
           2.0 * T * k * H * 2 * I, "TFLOP/s", PEAK_BF16_TFLOPS, 5)
    yield ("A11_silu_mul", f"silu(H1[:, :I]) * H1[:, I:], {xs.shape[0]} rows, I={I}",
           lambda: mg.silu_mul(h1, out=act), xs.shape[0] * I * 6, "GB/s", PEAK_HBM_GBS, 10)
    y2 = torch.empty(xs.shape[0], H, dtype=torch.bfloat16, device="cuda")
    yield ("A12_gemm2", f"Y2 = act . W2_e (W2 as [E, H, I]), K={I}, N={H} (useful flops of {T * k} rows)",
           lambda: mg.gmm_fwd(act, w2n, psz, trans_b=True, out=y2, ws=wsf), 2.0 * T * k * I * H, "TFLOP/s",
           PEAK_BF16_TFLOPS, 5)
    out = torch.empty(T, H, dtype=torch.bfloat16, device="cuda")
    yield ("A13_moe_unpermute", f"top-{k} weighted combine of {T * k} rows, hidden {H}",
           lambda: mg.moe_unpermute(y2, p["inv"], wts, T, k, out=out),
           T * k * H * 2 + T * H * 2 + T * k * 8, "GB/s", PEAK_HBM_GBS, 10)
    yield ("C3_fused_ffn_T4096", "align -> gathered GEMM1 with SiLU*mul epilogue -> GEMM2 -> combine, end to end "
                                 "(weights in the (E, N, K) layout)",
           lambda: mg.fused_moe(x, w1n, w2n, ids, wts, block_m=bm, ws=wsf, trans_b=True), 2.0 * T * k * H * 3 * I,
           "TFLOP/s", PEAK_BF16_TFLOPS, 3)
    for Tsmall in (1, 64):
        sub_ids, sub_w = ids[:Tsmall].contiguous(), wts[:Tsmall].contiguous()
        xsub = x[:Tsmall].contiguous()
        experts = int(torch.unique(sub_ids).numel())
        yield (f"C3_fused_ffn_T{Tsmall}", f"end to end, {experts} experts touched: weight bytes of those experts",
               lambda: mg.fused_moe(xsub, w1n, w2n, sub_ids, sub_w, ws=wsf, trans_b=True),
               experts * (H * 2 * I + I * H) * 2, "GB/s", PEAK_HBM_GBS, 5)
    # the same FFN with e4m3 expert weights (one scale per expert and output
    # column) and e4m3 activations
    w1q, s1q = mg.quantize_fp8_expert_weights(w1)
    w2q, s2q = mg.quantize_fp8_expert_weights(w2)
    yield ("C3_fused_ffn_fp8_T4096", "fp8-weight FFN end to end: align -> e4m3 of the token rows in sorted order "
                                     "-> fp8 GEMM1 -> SiLU*mul -> e4m3 -> fp8 GEMM2 -> combine",
           lambda: mg.fused_moe_fp8(x, w1q, s1q, w2q, s2q, ids, wts, ws=wsf), 2.0 * T * k * H * 3 * I,
           "TFLOP/s", PEAK_FP8_TFLOPS, 3)
    for Tsmall in (1, 64):
        sub_ids, sub_w = ids[:Tsmall].contiguous(), wts[:Tsmall].contiguous()
        xsub = x[:Tsmall].contiguous()
        experts = int(torch.unique(sub_ids).numel())
        yield (f"C3_fused_ffn_fp8_T{Tsmall}",
               f"fp8-weight FFN end to end, {experts} experts touched: e4m3 weight bytes of those experts",
               lambda: mg.fused_moe_fp8(xsub, w1q, s1q, w2q, s2q, sub_ids, sub_w, ws=wsf),
               experts * (H * 2 * I + I * H), "GB/s", PEAK_HBM_GBS, 5)
    del w1q, w2q
    torch.cuda.empty_cache()
    # the same FFN with int4 expert weights (per-128-K bf16 scales) and fp8
    # activations, decode-sized token counts
    w1_4, s1 = mg.quantize_int4_weights(w1)
    w2_4, s2 = mg.quantize_int4_weights(w2)
    del w1, w2
    torch.cuda.empty_cache()
    for Tsmall in (1, 64):
        sub_ids, sub_w = ids[:Tsmall].contiguous(), wts[:Tsmall].contiguous()
        xsub = x[:Tsmall].contiguous()
        experts = int(torch.unique(sub_ids).numel())
        int4_bytes = experts * ((H * 2 * I + I * H) // 2 + (H // 128 * 2 * I + I // 128 * H) * 2)
        yield (f"C3xC4_fused_ffn_f8i4_T{Tsmall}",
               f"int4-weight FFN end to end, {experts} experts touched: int4 weight and scale bytes of those experts",
               lambda: mg.fused_moe_f8i4(xsub, w1_4, s1, w2_4, s2, sub_ids, sub_w, ws=wsf),
               int4_bytes, "GB/s", PEAK_HBM_GBS, 5)


def row_measurements(torch, mg):
    """Each case of _row_cases timed on its own against its roofline: the
    average of back-to-back launches, and for the HBM-bound steps also the
    median of single launches with the caches flushed before each (cold)."""
    rows = {}
    for key, what, fn, amount, unit, peak, reps in _row_cases(torch, mg):
        us = _timeit(torch, fn, reps=reps)
        rows[key] = _row(what, us, amount, unit, peak) if amount is not None else {"what": what, "us": round(us, 2)}
        if unit == "GB/s":
            cold = launch_percentiles(torch, fn, reps=10)["cold"]
            rows[key]["cold_us"] = cold
            rows[key]["cold_frac"] = round(amount / cold["median"] / 1e3 / peak, 4)
    return rows


def counter_probe(torch, mg):
    """Runs every hot-path step three times, untimed, for rocprofv3 counter
    passes (--pmc): the balanced step's three products, a 256 MiB device copy
    (the calibration of FETCH_SIZE / WRITE_SIZE), then every case of
    _row_cases.  Before each batch a one-element fill (torch's FillFunctor)
    marks where the batch starts in the dispatch sequence (no other fp64
    fill runs here); the batch names are printed in order."""
    names = []
    marker = torch.empty(1, dtype=torch.float64, device="cuda")

    def batch(name, fn):
        marker.fill_(len(names))
        names.append(name)
        for _ in range(3):
            fn()

    E, M, K, N = 8, 1024, 4096, 6400
    d = balanced_inputs(torch, mg, E, M, K, N)
    x, w, dy, sizes = d["x"], d["w"], d["dy"], d["sizes"]
    y = torch.empty(M, N, dtype=torch.bfloat16, device="cuda")
    dx = torch.empty(M, K, dtype=torch.bfloat16, device="cuda")
    dw = torch.empty_like(w)
    ws = mg.workspace(E, M)
    batch("C2_fwd", lambda: mg.gmm_fwd(x, w, sizes, out=y, ws=ws))
    batch("C2_dx", lambda: mg.gmm_bwd(dy, x, w, sizes, need_dw=False, dx=dx, ws=ws))
    batch("C2_dw", lambda: mg.gmm_bwd(dy, x, w, sizes, need_dx=False, dw=dw, ws=ws))
    src = torch.ones(256 << 20, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    batch("copy_256MiB", lambda: dst.copy_(src))
    del d, x, w, dy, y, dx, dw, src, dst
    torch.cuda.empty_cache()
    for key, what, fn, amount, unit, peak, reps in _row_cases(torch, mg):
        batch(key, fn)
    torch.cuda.synchronize()
    log("counter probe batches: " + ",".join(names))


def _cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def cpu_baseline(host):
    """The fp64 oracle (unchanged, OpenMP over output rows) timed on the host
    cores on a bounded sample of the same workload: with every core of the
    process (up to 16, the GPU machine's share), the whole step -- forward, dX
    and dW -- once; with one thread, the forward of one group (128 of the
    1024 rows), the rest of the step being the same loops."""
    import oracle
    nproc = os.cpu_count() or 1
    affinity = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else nproc
    threads = min(affinity, 16)
    X, W, dY, s = host["X"], host["W"], host["dY"], host["sizes"]
    M, K = X.shape
    N = dY.shape[1]
    used = oracle.set_threads(threads)
    t0 = time.perf_counter()
    oracle.gmm_fwd_bf16(X, W, s)
    oracle.gmm_dx_bf16(dY, W, s)
    oracle.gmm_dw_bf16(X, dY, s)
    dt = time.perf_counter() - t0
    flops = 3 * 2.0 * M * K * N
    oracle.set_threads(1)
    r1 = int(s[0])
    t1 = time.perf_counter()
    oracle.gmm_fwd_bf16(X[:r1], W[:1], s[:1])
    dt1 = time.perf_counter() - t1
    oracle.set_threads(used)
    return {"value": round(flops / dt / 1e12, 6), "unit": "TFLOP/s", "cores": used, "kind": "oracle",
            "seconds": round(dt, 2),
            "sample": f"the whole step once (fwd + dX + dW, M={M}, K={K}, N={N}, E={len(s)}) in fp64 on {used} "
                      "threads, including the bf16 -> fp64 decode of the operands",
            "single_thread": {"value": round(2.0 * r1 * K * N / dt1 / 1e12, 6), "unit": "TFLOP/s", "cores": 1,
                              "seconds": round(dt1, 2),
                              "sample": f"the forward of one group ({r1} rows, K={K}, N={N}) in fp64 on one thread"},
            "host_cpus": nproc, "process_cpus": affinity, "cpu_model": _cpu_model()}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=200)
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--no-sparse", action="store_true", help="skip the sparse-M latency measurement")
    ap.add_argument("--no-rows", action="store_true", help="skip the per-step measurements of the other configurations")
    ap.add_argument("--no-peaks", action="store_true", help="skip the measured memory and vendor-BLAS rates")
    ap.add_argument("--traffic-probe", action="store_true",
                    help="only run each product and a known-size copy (for rocprofv3 --pmc passes)")
    ap.add_argument("--counter-probe", action="store_true",
                    help="only run every hot-path step three times, with batch markers (for rocprofv3 passes)")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(the grouped GEMM runs on one device's share); run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch
    import moe_grouped_gemm_device_amd as mg
    mg.lib()   # fails loudly if the HIP library is missing
    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        sys.exit(1)

    if args.traffic_probe:
        traffic_probe(torch, mg)
        return
    if args.counter_probe:
        counter_probe(torch, mg)
        return
    r = run_gpu(args, torch, mg)
    out = {
        "metric": METRIC,
        "value": round(r["value"], 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(r["ms_per_step"], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "balanced bf16 grouped GEMM fwd+dX+dW: E=8, M=1024 (128 rows per group, "
                               "sizes on device), K=4096, N=6400, X,W~U[0,1), dY=ones",
                   "E": r["E"], "M": r["M"], "K": r["K"], "N": r["N"]},
        "mfma_frac": round(r["value"] / PEAK_BF16_TFLOPS, 4),
        "roofline": r["roofline"],
        "context": "pages: 60 ms total kernel time for 30 fwd+bwd iterations of this workload on A100 (2.0 ms/iter); "
                   "here: total_kernel_ms_30_iterations",
    }
    out["total_kernel_ms_30_iterations"] = round(r["total30_ms"], 3)
    log("tiny-configuration latency")
    out["tiny_config"] = tiny_latency(torch, mg)
    if not args.no_sparse:
        log("sparse-M latency")
        out["sparse_m"] = sparse_m_latency(torch, mg)
    if not args.no_rows:
        log("per-step rows (fp8 layer share, fused FFN)")
        out["rows"] = row_measurements(torch, mg)
    if not args.no_peaks:
        log("measured peaks")
        out["measured_peaks"] = measured_peaks(torch)
    if not args.no_cpu:
        log("cpu baseline (oracle)")
        out["cpu_baseline"] = cpu_baseline(r["host"])
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
