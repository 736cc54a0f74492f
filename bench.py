"""Benchmark of the LFM2 ShortConv hot path on one MI355X.

A step is one pass of the whole training hot path over one batch of seeded
synthetic input: lfm2sc_prefill_ragged (forward: B*xv, causal depthwise conv,
C gate) followed by lfm2sc_backward (dB, dC, dxv and the deterministic dW
reduction), on one sequence of T=65536 tokens, H=2048, K=3, bf16 I/O with fp32
accumulation, zero initial state.  Inputs are resident in HBM before timing.

Prints ONE JSON line.  `value` is the step's algorithmic HBM bytes divided by
the measured step time (GB/s); the roofline object reports the backward call
(its dominant launch) against the MI355X HBM peak; cpu_baseline times the fp64
oracle on a bounded channel sample of the same workload.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu] [--no-extra]
       python bench.py --calibrate-copy   (plain device copy of known size, for counter scaling)
"""
import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0   # MI355X HBM3E, AMD public specification
MFMA_BF16_PEAK_TFLOPS = 2500.0   # MI355X dense bf16 matrix-core peak, AMD public specification
METRIC = "ShortConv GB/s and % of HBM peak; fwd+bwd ms at T=65536, H=2048, K=3"


def algo_bytes_fwd(T, H, K, e):
    """Forward: read B, C, xv (3H) and write y (H) per token, plus the weight."""
    return T * 4 * H * e + H * K * e


def algo_bytes_bwd(T, H, K, e):
    """Backward: read dy (H) and B, C, xv (3H), write dB, dC, dxv (3H) per token, plus weight and fp32 dW."""
    return T * 7 * H * e + H * K * e + H * K * 4


def algo_bytes_decode(N, H, K, e):
    """Per sequence: read B, C, xv and the [H,K] state, write y and the state; plus weight and slot ids."""
    return N * (3 * H * e + H * e + 2 * H * K * e) + H * K * e + 4 * N


def algo_bytes_prefill(total_T, N, H, K, e):
    """Read in_proj (3H), write y (H) per token; read + write each sequence's state; weight; offsets and slots."""
    return total_T * 4 * H * e + N * 2 * H * K * e + H * K * e + 4 * (2 * N + 1)


def algo_bytes_verify(N, L, H, K, e):
    """Read in_proj rows and the states, write y and the per-step tape; weight and slot ids."""
    return N * L * (3 * H * e + H * e + H * K * e) + N * H * K * e + H * K * e + 4 * N


def algo_bytes_conv_update(N, L, H, K, e):
    """Read bx and write out (H per token), write the tape (H*K per token), read each state; weight, slot ids."""
    return N * L * (2 * H * e + H * K * e) + N * H * K * e + H * K * e + 4 * N


def kernel_source_hash():
    h = hashlib.sha256()
    for f in ("bwd.hip", "common.hpp", "kernels.hpp"):
        with open(os.path.join(ROOT, "gated_short_causal_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def read_traffic(per_launch_algo_bytes):
    """HBM bytes of one backward launch from the committed counter summary, if it matches the current source."""
    path = os.path.join(ROOT, "profiles", "backward_T65536_counters.txt")
    if not os.path.exists(path):
        return None
    vals = {}
    for line in open(path):
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            vals[k.strip()] = v.strip()
    if vals.get("kernel_source_sha256_16") != kernel_source_hash():
        return None
    try:
        return float(vals["hbm_bytes_per_backward_call"])
    except (KeyError, ValueError):
        return None


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for ln in f:
                if ln.startswith("model name"):
                    return ln.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def host_cpus():
    """CPUs this process may run on (the machine's CPU share for one GPU is 16; the oracle uses at most that)."""
    try:
        return len(os.sched_getaffinity(0))
    except AttributeError:
        return os.cpu_count() or 1


def cpu_baseline(wl_mod, T, H, K, n_channels, min_seconds=10.0, single_channels=64):
    """The fp64 oracle (as it stands) on the same workload restricted to n_channels channels
    (channels are independent, so this is the same arithmetic on a slice).  Whole passes with
    min(16, host CPUs) OpenMP threads (16 = one GPU's share of the host) until min_seconds have elapsed
    (value: median pass), then three single-threaded passes over the first `single_channels` channels
    (median); then every other workload (cpu_baseline_configs)."""
    import statistics
    import torch
    import oracle
    c = wl_mod.train_lfm2(T=T)

    def sample(n):
        chans = torch.arange(n)
        cols = torch.cat([chans, chans + H, chans + 2 * H])
        return oracle.f64(c.inp[:, cols]), oracle.f64(c.w[chans]), oracle.f64(c.dy[:, chans])

    def one_pass(inp, w, dy):
        t = time.perf_counter()
        oracle.prefill(inp, c.cu, w)
        oracle.backward(inp, c.cu, w, dy)
        return time.perf_counter() - t

    threads = min(16, host_cpus())
    oracle.set_threads(threads)
    inp, w, dy = sample(n_channels)
    times, t0 = [], time.perf_counter()
    while True:
        times.append(one_pass(inp, w, dy))
        if time.perf_counter() - t0 >= min_seconds:
            break
    dt = time.perf_counter() - t0
    pass_bytes = algo_bytes_fwd(T, n_channels, K, 2) + algo_bytes_bwd(T, n_channels, K, 2)
    med = statistics.median(times)
    oracle.set_threads(1)
    inp1, w1, dy1 = sample(single_channels)
    t1 = statistics.median([one_pass(inp1, w1, dy1) for _ in range(3)])
    oracle.set_threads(threads)
    bytes1 = algo_bytes_fwd(T, single_channels, K, 2) + algo_bytes_bwd(T, single_channels, K, 2)
    return {"value": round(pass_bytes / med / 1e9, 4), "unit": "GB/s", "cores": threads, "kind": "oracle",
            "sample": f"fwd+bwd, T={T}, first {n_channels} of {H} channels, K={K}, bf16 inputs widened to fp64; "
                      f"median of {len(times)} passes ({dt:.2f} s wall)",
            "seconds": round(dt, 3), "passes": len(times), "pass_s_median": round(med, 4),
            "cpu_model": cpu_model(), "host_cpus": host_cpus(),
            "configs": cpu_baseline_configs(wl_mod, threads),
            "single_thread": {"value": round(bytes1 / t1 / 1e9, 4), "unit": "GB/s", "cores": 1,
                              "sample": f"first {single_channels} channels, median of 3 passes",
                              "pass_s_median": round(t1, 4)}}


def cpu_baseline_configs(wl_mod, threads, min_seconds=0.5):
    """The fp64 oracle (as it stands) on the other workloads, each at `threads` OpenMP threads and single
    threaded: calls repeated until `min_seconds` have elapsed, median call time, GB/s at the same algorithmic
    bytes as the GPU figures.  Config 1 (tiny fp32) is its 64-token forward + backward; config 2 one decode
    step; config 3 one ragged prefill; config 4 one verify window; config 5 at T=4096 the forward + backward."""
    import statistics
    import oracle

    def timed(fn):
        ts, t0 = [], time.perf_counter()
        while True:
            t = time.perf_counter()
            fn()
            ts.append(time.perf_counter() - t)
            if time.perf_counter() - t0 >= min_seconds and len(ts) >= 3:
                return statistics.median(ts), len(ts)

    c1 = wl_mod.tiny_fp32()
    c2 = wl_mod.decode_lfm2()
    c3 = wl_mod.ragged_prefill_lfm2()
    c4 = wl_mod.verify_lfm2()
    c5 = wl_mod.train_lfm2(T=4096)
    T3 = c3.inp.shape[0]
    cases = {
        "cfg1_tiny_fp32_fwd_bwd": (lambda: (oracle.prefill(c1.inp, c1.cu, c1.w),
                                            oracle.backward(c1.inp, c1.cu, c1.w, c1.dy)),
                                   algo_bytes_fwd(64, 256, 3, 4) + algo_bytes_bwd(64, 256, 3, 4)),
        "cfg2_decode_N256": (lambda: oracle.decode(c2.inp, c2.w, c2.pool, c2.slot_idx),
                             algo_bytes_decode(256, 2048, 3, 2)),
        "cfg3_ragged_prefill_N8": (lambda: oracle.prefill(c3.inp, c3.cu, c3.w, c3.pool, c3.slot_idx),
                                   algo_bytes_prefill(T3, 8, 2048, 3, 2)),
        "cfg4_verify_64x8": (lambda: oracle.verify(c4.inp, c4.w, c4.pool, c4.slot_idx, 8),
                             algo_bytes_verify(64, 8, 2048, 3, 2)),
        "cfg5_train_T4096": (lambda: (oracle.prefill(c5.inp, c5.cu, c5.w),
                                      oracle.backward(c5.inp, c5.cu, c5.w, c5.dy)),
                             algo_bytes_fwd(4096, 2048, 3, 2) + algo_bytes_bwd(4096, 2048, 3, 2)),
    }
    out = {}
    for name, (fn, nbytes) in cases.items():
        row = {}
        for n in (threads, 1):
            oracle.set_threads(n)
            med, calls = timed(fn)
            row["threads_%d" % n] = {"ms": round(1e3 * med, 4), "GB/s": round(nbytes / med / 1e9, 4), "calls": calls}
        row["bytes"] = int(nbytes)
        out[name] = row
    oracle.set_threads(threads)
    return out


def copy_ceiling(reps=10):
    """Measured device-copy ceiling: a plain 1 GiB device-to-device copy (torch's copy kernel), bytes read +
    written per copy over its event time, median of `reps`."""
    import statistics
    import torch
    n = 1 << 30
    src = torch.empty(n, dtype=torch.uint8, device="cuda").random_(0, 255)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    ts = []
    for _ in range(reps):
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record()
        dst.copy_(src)
        b.record()
        torch.cuda.synchronize()
        ts.append(a.elapsed_time(b))
    ms = statistics.median(ts)
    del src, dst
    torch.cuda.empty_cache()
    return {"GB/s": round(2 * n / ms / 1e6, 1), "bytes_per_copy": 2 * n, "ms": round(ms, 5),
            "kernel": "torch copy_ of 1 GiB, device to device", "reps": reps}


def mix_reference(reps=10):
    """The runtime's own elementwise kernels at several shares of written bytes (torch fill_, copy_, add,
    addcmul over 1 GiB-scale buffers), GB/s read + written, median of `reps`: how fast this box streams a
    plain read/write mix, beside which the ShortConv kernels' own shares (forward 1/4, decode 2/5, backward
    3/7 of their bytes written) can be read.  Context, not a ceiling."""
    import statistics
    import torch

    def med(fn):
        for _ in range(3):
            fn()
        ts = []
        for _ in range(reps):
            a = torch.cuda.Event(enable_timing=True)
            b = torch.cuda.Event(enable_timing=True)
            a.record()
            fn()
            b.record()
            torch.cuda.synchronize()
            ts.append(a.elapsed_time(b))
        return statistics.median(ts)

    n = 1 << 28   # bf16 elements per operand (512 MiB)
    x = torch.randn(n, dtype=torch.bfloat16, device="cuda")
    y = torch.randn_like(x)
    z = torch.randn_like(x)
    o = torch.empty_like(x)
    e = 2 * n
    out = {}
    for name, w, nbytes, fn in (("fill_", 1.0, e, lambda: o.fill_(1.0)),
                                ("copy_", 0.5, 2 * e, lambda: o.copy_(x)),
                                ("add", 1 / 3, 3 * e, lambda: torch.add(x, y, out=o)),
                                ("addcmul", 0.25, 4 * e, lambda: torch.addcmul(x, y, z, out=o))):
        ms = med(fn)
        out[name] = {"written_share": round(w, 3), "GB/s": round(nbytes / ms / 1e6, 1)}
    del x, y, z, o
    torch.cuda.empty_cache()
    return out


def timed_loop(fn, steps, warmup):
    import torch
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record()
    for _ in range(steps):
        fn()
    t1.record()
    torch.cuda.synchronize()
    return t0.elapsed_time(t1) / steps


def graph_time(calls, replays):
    """GPU time per call with host launch overhead removed: the calls are captured once into a HIP graph
    (torch.cuda.CUDAGraph; the library launches on the capturing stream) and the graph is replayed."""
    import torch
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for c in calls:
            c()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for c in calls:
            c()
    g.replay()
    torch.cuda.synchronize()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record()
    for _ in range(replays):
        g.replay()
    t1.record()
    torch.cuda.synchronize()
    return t0.elapsed_time(t1) / (replays * len(calls))


def extra_measurements(wl_mod, steps, fused=True):
    """Decode, ragged prefill and verify at their LFM2-1.2B shapes.  Input sets are rotated so that one pass
    touches more than 2 x 256 MB (past the Infinity Cache): these are HBM figures.  `ms` is GPU time per call
    from graph replay; `eager_ms` is the back-to-back eager rate, which includes host launch overhead."""
    import torch
    from gated_short_causal_amd import lfm2sc_decode_step, lfm2sc_prefill_ragged, lfm2sc_verify_window
    dev = torch.device("cuda")
    out = {}

    def record(name, calls, nbytes):
        eager = timed_loop(lambda: [c() for c in calls], steps, 2) / len(calls)
        ms = graph_time(calls, steps)
        out[name] = {"ms": round(ms, 5), "GB/s": round(nbytes / ms / 1e6, 1), "pct_of_hbm_peak":
                     round(100 * nbytes / ms / 1e6 / HBM_PEAK_GBS, 1), "eager_ms": round(eager, 5), "bytes": int(nbytes)}

    # decode: 10.5 MB per call, 64 rotated sets (672 MB)
    sets = [wl_mod.decode_lfm2(seed=200 + i).to(dev) for i in range(64)]
    ys = [torch.empty(256, 2048, dtype=torch.bfloat16, device=dev) for _ in sets]
    calls = [(lambda s=s, y=y: lfm2sc_decode_step(s.inp, s.w, s.pool, s.slot_idx, y)) for s, y in zip(sets, ys)]
    record("decode_N256", calls, algo_bytes_decode(256, 2048, 3, 2))
    del sets, ys, calls
    # decode at a larger batch (N=4096 of a 8192-slot pool, 168 MB per call, 4 rotated sets): launch latency amortised
    sets = [wl_mod.decode_lfm2(seed=250 + i, N=4096, slots=8192).to(dev) for i in range(4)]
    ys = [torch.empty(4096, 2048, dtype=torch.bfloat16, device=dev) for _ in sets]
    calls = [(lambda s=s, y=y: lfm2sc_decode_step(s.inp, s.w, s.pool, s.slot_idx, y)) for s, y in zip(sets, ys)]
    record("decode_N4096", calls, algo_bytes_decode(4096, 2048, 3, 2))
    del sets, ys, calls
    # ragged prefill: ~141 MB per call, 5 rotated sets (705 MB)
    sets = [wl_mod.ragged_prefill_lfm2(seed=300 + i).to(dev) for i in range(5)]
    ys = [torch.empty(s.inp.shape[0], 2048, dtype=torch.bfloat16, device=dev) for s in sets]
    calls = [(lambda s=s, y=y: lfm2sc_prefill_ragged(s.inp, s.cu, s.w, y, s.pool, s.slot_idx)) for s, y in zip(sets, ys)]
    record("ragged_prefill_N8", calls, sum(algo_bytes_prefill(s.inp.shape[0], 8, 2048, 3, 2) for s in sets) / len(sets))
    del sets, ys, calls
    # verify: 15.5 MB per call, 48 rotated sets (743 MB)
    sets = [wl_mod.verify_lfm2(seed=400 + i).to(dev) for i in range(48)]
    outs = [(torch.empty(512, 2048, dtype=torch.bfloat16, device=dev),
             torch.empty(64, 8, 2048, 3, dtype=torch.bfloat16, device=dev)) for _ in sets]
    calls = [(lambda s=s, o=o: lfm2sc_verify_window(s.inp, s.w, s.pool, s.slot_idx, 8, o[1], o[0]))
             for s, o in zip(sets, outs)]
    record("verify_64x8", calls, algo_bytes_verify(64, 8, 2048, 3, 2))
    del sets, outs, calls
    # conv update of gated inputs at the verify shape, in the transposed-view layout of token-major rows
    # (vector path) and as a dense [N][H][L] tensor (per-element path): bx, out, tape and the read of the state
    from gated_short_causal_amd import lfm2sc_conv_update
    for kind in ("view", "dense"):
        sets = [wl_mod.verify_lfm2(seed=450 + i).to(dev) for i in range(48)]
        bxs, outs, tapes = [], [], []
        for st in sets:
            rows = st.inp[:, :2048]                                   # stands in for gated B*xv rows
            if kind == "view":
                bxs.append(rows.contiguous().view(64, 8, 2048).transpose(1, 2))
                outs.append(torch.empty(64, 8, 2048, dtype=torch.bfloat16, device=dev).transpose(1, 2))
            else:
                bxs.append(rows.view(64, 8, 2048).transpose(1, 2).contiguous())
                outs.append(torch.empty(64, 2048, 8, dtype=torch.bfloat16, device=dev))
            tapes.append(torch.empty(64, 8, 2048, 3, dtype=torch.bfloat16, device=dev))
        calls = [(lambda st=st, b=b, o=o, t=t: lfm2sc_conv_update(b, st.w, st.pool, st.slot_idx, o, windows=t))
                 for st, b, o, t in zip(sets, bxs, outs, tapes)]
        record(f"conv_update_64x8_{kind}", calls, algo_bytes_conv_update(64, 8, 2048, 3, 2))
        del sets, bxs, outs, tapes, calls
    out.update(train_t4096_measurement(wl_mod, steps))
    if fused:
        out.update(fused_measurements(wl_mod, steps))
        out.update(shape_measurements(wl_mod, steps))
    return out


def train_t4096_measurement(wl_mod, steps, nsets=5):
    """The training step (prefill forward + backward) at T=4096, H=2048, K=3, bf16: `nsets` independent input
    sets (~134 MB each with outputs, 670 MB per pass, past the 256 MB Infinity Cache) taken in turn, so each
    step reads from HBM.  `ms` per step by graph replay (launch overhead removed), `eager_ms` back to back."""
    import torch
    from gated_short_causal_amd import lfm2sc_backward, lfm2sc_backward_workspace_bytes, lfm2sc_prefill_ragged
    dev = torch.device("cuda")
    T, H, K = 4096, 2048, 3
    sets = [wl_mod.train_lfm2(seed=510 + i, T=T).to(dev) for i in range(nsets)]
    ws = torch.empty(max(16, lfm2sc_backward_workspace_bytes(torch.bfloat16, H, K, T, 1)), dtype=torch.uint8,
                     device=dev)
    dW = torch.empty(H, K, dtype=torch.float32, device=dev)
    calls = []
    for c in sets:
        y = torch.empty(T, H, dtype=torch.bfloat16, device=dev)
        d_in = torch.empty(T, 3 * H, dtype=torch.bfloat16, device=dev)
        calls.append(lambda c=c, y=y: lfm2sc_prefill_ragged(c.inp, c.cu, c.w, y))
        calls.append(lambda c=c, d_in=d_in: lfm2sc_backward(c.inp, c.cu, c.w, c.dy, d_in, dW, ws))
    eager = timed_loop(lambda: [f() for f in calls], steps, 2) / nsets
    ms = 2 * graph_time(calls, steps)
    nbytes = algo_bytes_fwd(T, H, K, 2) + algo_bytes_bwd(T, H, K, 2)
    return {"train_T4096": {"ms": round(ms, 5), "GB/s": round(nbytes / ms / 1e6, 1),
                            "pct_of_hbm_peak": round(100 * nbytes / ms / 1e6 / HBM_PEAK_GBS, 1),
                            "eager_ms": round(eager, 5), "bytes": int(nbytes), "input_sets": nsets,
                            "pages_mi325x_liger_fwd_bwd_ms": 0.463}}


def shape_measurements(wl_mod, steps):
    """The training step (prefill forward + backward, T=65536, one sequence) at other channel counts and tap
    counts, and with fp32 I/O: GB/s of the step's algorithmic bytes and % of the HBM peak."""
    import torch
    from gated_short_causal_amd import lfm2sc_backward, lfm2sc_backward_workspace_bytes, lfm2sc_prefill_ragged
    dev = torch.device("cuda")
    out = {}
    for H, K, dt in ((1024, 3, torch.bfloat16), (1536, 3, torch.bfloat16), (2048, 2, torch.bfloat16),
                     (2048, 4, torch.bfloat16), (2048, 3, torch.float32)):
        T = 65536
        e = 2 if dt == torch.bfloat16 else 4
        c = wl_mod.train_lfm2(seed=5, T=T, H=H, K=K, dtype=dt).to(dev)
        y = torch.empty(T, H, dtype=dt, device=dev)
        d_in = torch.empty(T, 3 * H, dtype=dt, device=dev)
        dW = torch.empty(H, K, dtype=torch.float32, device=dev)
        ws = torch.empty(max(16, lfm2sc_backward_workspace_bytes(dt, H, K, T, 1)), dtype=torch.uint8, device=dev)

        def step():
            lfm2sc_prefill_ragged(c.inp, c.cu, c.w, y)
            lfm2sc_backward(c.inp, c.cu, c.w, c.dy, d_in, dW, ws)

        ms = timed_loop(step, steps, 3)
        nbytes = algo_bytes_fwd(T, H, K, e) + algo_bytes_bwd(T, H, K, e)
        name = f"train_T65536_H{H}_K{K}_{'bf16' if e == 2 else 'fp32'}"
        out[name] = {"ms": round(ms, 5), "GB/s": round(nbytes / ms / 1e6, 1),
                     "pct_of_hbm_peak": round(100 * nbytes / ms / 1e6 / HBM_PEAK_GBS, 1), "bytes": int(nbytes)}
        del c, y, d_in, dW, ws
    return out


def fused_measurements(wl_mod, steps):
    """The fused in_proj + ShortConv forward (lfm2sc_fused_prefill) at the LFM2-1.2B layer shape (D = H = 2048):
    the training forward at T=65536 (y only, and with the in_proj output the backward takes), the ragged
    prefill, short forwards (T=4096: one round of halo tiles; T=1024: mid tiles; T=256 and 256 one-token
    sequences with a pool: split tiles).  Matrix-core bound: FLOPs = 2 * T * D * 3H
    per call against the bf16 dense peak.  `unfused_ms` is the two-step path it replaces, a bf16 GEMM into
    in_proj (torch.matmul) then lfm2sc_prefill_ragged: context, not a lower bound."""
    import torch
    from gated_short_causal_amd import (lfm2sc_fused_prefill, lfm2sc_fused_prefill_plan,
                                        lfm2sc_fused_prefill_workspace_bytes, lfm2sc_prefill_ragged)
    dev = torch.device("cuda")
    out = {}
    tilings = {1: "wide", 2: "wide, halo rows", 3: "4-wave", 32: "split, 32 channels", 64: "split, 64 channels",
               128: "mid"}

    def one(name, c, with_io, graph):
        g = c.to(dev)
        T, H, D = c.x.shape[0], c.H, c.D
        N = c.cu.numel() - 1
        y = torch.empty(T, H, dtype=torch.bfloat16, device=dev)
        io = torch.empty(T, 3 * H, dtype=torch.bfloat16, device=dev) if with_io else None
        ws = torch.empty(max(16, lfm2sc_fused_prefill_workspace_bytes(torch.bfloat16, H, c.K, N, c.pool is not None)),
                         dtype=torch.uint8, device=dev)
        ip = torch.empty(T, 3 * H, dtype=torch.bfloat16, device=dev)
        fused = lambda: lfm2sc_fused_prefill(g.x, g.W_in, g.cu, g.w, y, g.pool, g.slot_idx, in_proj_out=io,
                                             workspace=ws)
        gemm = lambda: torch.matmul(g.x, g.W_in.t(), out=ip)
        conv = lambda: lfm2sc_prefill_ragged(ip, g.cu, g.w, y, g.pool, g.slot_idx)
        if graph:
            # 8 back-to-back calls per graph (per pair of calls for the two-step path), so that the gap
            # between graph replays is spread over them as it is over the calls of a serving loop
            ms = graph_time([fused] * 8, steps)
            unf = 2 * graph_time([gemm, conv] * 8, steps)
        else:
            # the inputs were just generated on the host with the GPU idle: warm up long enough for the
            # long calls to reach their steady rate (the same for both paths)
            warm = max(10, steps)
            ms = timed_loop(fused, steps, warm)
            unf = timed_loop(gemm, steps, warm) + timed_loop(conv, steps, warm)
        flops = 2.0 * T * D * 3 * H
        tf = flops / ms / 1e9
        out[name] = {"ms": round(ms, 5), "TFLOP/s": round(tf, 1),
                     "roofline": {"bound": "mfma", "achieved": round(tf, 1), "peak": MFMA_BF16_PEAK_TFLOPS,
                                  "unit": "TFLOP/s", "frac": round(tf / MFMA_BF16_PEAK_TFLOPS, 4)},
                     "unfused_ms": round(unf, 5), "T": T, "flops": flops,
                     "tiling": tilings.get(lfm2sc_fused_prefill_plan(H, c.K, D, T), "?")}

    one("fused_train_T65536", wl_mod.fused_train_lfm2(T=65536), False, False)
    one("fused_train_T65536_with_in_proj", wl_mod.fused_train_lfm2(T=65536), True, False)
    one("fused_ragged_prefill_N8", wl_mod.fused_ragged_lfm2(), False, True)
    one("fused_train_T4096", wl_mod.fused_train_lfm2(T=4096), False, True)
    one("fused_short_T1024", wl_mod.fused_train_lfm2(T=1024), False, True)
    one("fused_short_T256", wl_mod.fused_train_lfm2(T=256), False, True)
    one("fused_one_token_N256", wl_mod.fused_one_token_lfm2(), False, True)
    return out


def fused_only(args):
    """The fused in_proj + ShortConv training forward at D = H = 2048, T = args.T (y only): `warmup` untimed
    calls, then `steps` timed ones; one JSON line with the time and the algorithmic bytes of a call (x rows
    read, W_in read once, y written, the weight)."""
    import torch
    from gated_short_causal_amd import lfm2sc_fused_prefill
    from gated_short_causal_amd import workloads as wl_mod
    c = wl_mod.fused_train_lfm2(T=args.T).to(torch.device("cuda"))
    T, H, D = c.x.shape[0], c.H, c.D
    y = torch.empty(T, H, dtype=torch.bfloat16, device="cuda")
    call = lambda: lfm2sc_fused_prefill(c.x, c.W_in, c.cu, c.w, y)
    ms = timed_loop(call, args.steps, args.warmup)
    algo = T * D * 2 + 3 * H * D * 2 + T * H * 2 + H * c.K * 2
    print(json.dumps({"fused_only": {"T": T, "ms": round(ms, 5), "TFLOP/s": round(2.0 * T * D * 3 * H / ms / 1e9, 1),
                                     "algorithmic_bytes_per_call": algo}}), flush=True)


def calibrate_copy():
    """A plain device-to-device copy of 1 GiB, 5 times: the FETCH_SIZE / WRITE_SIZE readings of this kernel
    under rocprofv3 give the counter-to-bytes factor (1 GiB read and 1 GiB written per dispatch)."""
    import torch
    n = 1 << 30
    src = torch.empty(n, dtype=torch.uint8, device="cuda").random_(0, 255)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"calibrate_copy_bytes": n, "dispatches": 5}))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--T", type=int, default=65536)
    ap.add_argument("--no-cpu", action="store_true", help="skip the oracle CPU baseline")
    ap.add_argument("--cpu-channels", type=int, default=2048)
    ap.add_argument("--no-extra", dest="extra", action="store_false",
                    help="skip the decode, ragged prefill and verify figures (graph replay, a few seconds)")
    ap.add_argument("--extra", dest="extra", action="store_true", help=argparse.SUPPRESS)
    ap.add_argument("--no-fused", dest="fused", action="store_false",
                    help="in the extra figures, skip the fused forward and the other-shape training steps")
    ap.add_argument("--calibrate-copy", action="store_true")
    ap.add_argument("--fused-only", action="store_true",
                    help="only the fused in_proj + ShortConv training forward (y only), for counter passes")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only; the ShortConv path is sharded by channels or "
              "sequences with no collective on the hot path, and no multi-GPU figure is produced.", file=sys.stderr)
        sys.exit(2)

    import torch
    if args.calibrate_copy:
        calibrate_copy()
        return
    if args.fused_only:
        fused_only(args)
        return
    from gated_short_causal_amd import lfm2sc_backward, lfm2sc_backward_workspace_bytes, lfm2sc_prefill_ragged
    from gated_short_causal_amd import workloads as wl

    T, H, K, e = args.T, 2048, 3, 2
    dev = torch.device("cuda")
    print(f"bench: generating T={T} inputs", file=sys.stderr, flush=True)
    c = wl.train_lfm2(T=T).to(dev)
    y = torch.empty(T, H, dtype=torch.bfloat16, device=dev)
    d_in = torch.empty(T, 3 * H, dtype=torch.bfloat16, device=dev)
    dW = torch.empty(H, K, dtype=torch.float32, device=dev)
    ws = torch.empty(max(16, lfm2sc_backward_workspace_bytes(torch.bfloat16, H, K, T, 1)), dtype=torch.uint8,
                     device=dev)

    def fwd():
        lfm2sc_prefill_ragged(c.inp, c.cu, c.w, y)

    def bwd():
        lfm2sc_backward(c.inp, c.cu, c.w, c.dy, d_in, dW, ws)

    for _ in range(args.warmup):
        fwd()
        bwd()
    torch.cuda.synchronize()
    # the timed region: exactly `steps` steps back to back, events only at its two ends (an event recorded
    # between two calls costs several microseconds of stream time of its own)
    start = torch.cuda.Event(enable_timing=True)
    stop = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record()
    for _ in range(args.steps):
        fwd()
        bwd()
    stop.record()
    torch.cuda.synchronize()
    ms_step = start.elapsed_time(stop) / args.steps
    # average duration of one backward call (the dominant launch), from `steps` back-to-back calls on the
    # stream the library launches on; and of one forward call the same way
    bwd_ms = timed_loop(bwd, args.steps, 2)
    fwd_ms = timed_loop(fwd, args.steps, 2)
    # the median protocol beside the timed loop: 50 more steps, each call bracketed by events (so each call's
    # figure includes the cost of its events)
    import statistics
    ev50 = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(50)]
    for s in range(50):
        ev50[s][0].record()
        fwd()
        ev50[s][1].record()
        bwd()
        ev50[s][2].record()
    torch.cuda.synchronize()
    median50 = {"fwd_ms": round(statistics.median(a.elapsed_time(b) for a, b, _ in ev50), 5),
                "bwd_ms": round(statistics.median(b.elapsed_time(cc) for _, b, cc in ev50), 5),
                "step_ms": round(statistics.median(a.elapsed_time(cc) for a, _, cc in ev50), 5), "reps": 50,
                "note": "events around every call"}
    step_bytes = algo_bytes_fwd(T, H, K, e) + algo_bytes_bwd(T, H, K, e)
    bwd_bytes = algo_bytes_bwd(T, H, K, e)
    value = step_bytes / ms_step / 1e6
    bwd_gbs = bwd_bytes / bwd_ms / 1e6
    traffic = read_traffic(bwd_bytes)

    line = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) inputs and dy, U(-0.5,0.5) weight)",
        "config": {"workload": f"ShortConv training step (prefill forward + backward), 1 sequence, T={T}, "
                               f"H={H}, K={K}, bf16 I/O, fp32 accumulation, zero initial state",
                   "T": T, "H": H, "K": K, "seqs": 1},
        "pct_of_hbm_peak": round(100 * value / HBM_PEAK_GBS, 2),
        "fwd_ms": round(fwd_ms, 5),
        "bwd_ms": round(bwd_ms, 5),
        "step_algorithmic_bytes": step_bytes,
        "roofline": {"bound": "hbm", "achieved": round(bwd_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(bwd_gbs / HBM_PEAK_GBS, 4), "traffic": traffic,
                     "kernel": "lfm2sc_backward (backward_kernel + dw_finish_kernel, one call; average of "
                               "back-to-back calls)",
                     "algorithmic_bytes_per_launch": bwd_bytes},
        "median_of_50": median50,
        "context": {"pages_mi325x_liger_fwd_bwd_ms": {"T=4096": 0.463, "T=65536": 8.083}},
    }
    cc = copy_ceiling()
    cc["step_frac"] = round(value / cc["GB/s"], 4)
    cc["backward_frac"] = round(bwd_gbs / cc["GB/s"], 4)
    line["copy_ceiling"] = cc
    line["mix_reference"] = mix_reference()
    if args.extra:
        line["extra"] = extra_measurements(wl, max(2, args.steps // 2), args.fused)
    if not args.no_cpu:
        print("bench: timing the oracle CPU baseline", file=sys.stderr, flush=True)
        line["cpu_baseline"] = cpu_baseline(wl, T, H, K, args.cpu_channels)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
