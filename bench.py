"""Benchmark of the dense-GEMM hot path on one MI355X.

One step is one fp16 GEMM C = A @ B at M = N = K = 4096 (row-major A and B,
fp16 output, fp32 accumulation, alpha = 1, beta = 0) through the C ABI.
Prints ONE JSON line: TFLOP/s of that GEMM (whole job, one GPU), the
roofline of its kernel (algorithmic FLOPs over the kernel's average duration,
measured with HIP events on the stream it is launched on, against the
2.5 PFLOP/s dense fp16 MFMA peak), the CPU oracle timed on a bounded sample
of the same product, and the other workloads' figures: the 2048-token q4
prefill projections in tokens/s (dequant per call and GEMM only), the fp32
ladder, and the tall-skinny fused-epilogue shapes as HBM roofline fractions.

Inputs are synthetic and seeded (dense_gemm_engineering_amd.inputs); they are
resident in HBM before any timed region starts.
"""
import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK = {"f16": 2500.0, "bf16": 2500.0, "f32": 157.3}  # TFLOP/s, dense MFMA
HBM_PEAK_GBS = 8000.0

# ------------------------------------------------------------ accounting

def gemm_flops(M, N, K):
    """2MNK: one multiply and one add per term of every dot product."""
    return 2.0 * M * N * K


def gemm_alg_bytes(M, N, K, s_in, s_out, beta_read=False, bias_bytes=0):
    """Least traffic any kernel can have: read A and B once, write C once
    (plus C's old value when beta != 0, plus the bias vector)."""
    b = s_in * (M * K + K * N) + s_out * M * N + bias_bytes
    if beta_read:
        b += s_out * M * N
    return float(b)


def ideal_intensity(M, N, K, s):
    """Best-case FLOP/byte of an M x K by K x N product with s-byte numbers."""
    return gemm_flops(M, N, K) / (s * (M * K + K * N + M * N))


def dequant_alg_bytes(rows, cols):
    """q4 -> fp16: 18 bytes per 32 weights read, 2 bytes per weight written."""
    return rows * cols / 32 * 18 + rows * cols * 2.0


KQ_BLOCK = {"q4_k": (256, 144), "q6_k": (256, 210)}


def kquant_alg_bytes(qtype, rows, cols):
    """Super-block format -> fp16: the block bytes read once, 2 bytes per
    weight written."""
    w, nb = KQ_BLOCK[qtype]
    return rows * cols / w * nb + rows * cols * 2.0


def prefill_stack_tokens_per_s(t_attn, t_up, t_down, tokens=2048, layers=32):
    """tokens / (layers x [4 square projections + 2 up-projections + 1 down]).

    A 7B-like decoder layer with hidden 4096 and FFN 11008 has four 4096 x 4096
    projections (q, k, v, o), two 11008 x 4096 (gate, up) and one 4096 x 11008
    (down): 6.5e9 projection weights over 32 layers."""
    return tokens / (layers * (4 * t_attn + 2 * t_up + t_down))


# ------------------------------------------------------------ timing
#
# Protocol: every figure is the median of several windows of back-to-back
# launches, each window bracketed by HIP events on the launch stream (GPU
# time) and by host synchronisation (wall time); before its first window a
# leg runs back to back for a while without host syncs (the engine clock
# needs a few hundred ms of load to settle).  The headline legs run
# interleaved in a shuffled order, three times over, so that slow drift of
# the clock or the machine affects every leg alike.

MIN_TIMED_S = 0.05  # timed work per leg and repeat (windows are added to reach it)


def _prewarm(fn, torch, seconds, est_s):
    n = max(1, int(seconds / max(est_s, 1e-6)))
    for _ in range(n):
        fn()
    torch.cuda.synchronize()


def time_windows(fn, steps, windows, torch, min_timed_s=MIN_TIMED_S):
    """`windows` (or more, to reach min_timed_s) windows of `steps`
    back-to-back calls.  Returns a list of (GPU seconds, wall seconds) per
    window (per window, not per call)."""
    out = []
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    total = 0.0
    while len(out) < windows or total < min_timed_s:
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        e0.record()
        for _ in range(steps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        gpu = e0.elapsed_time(e1) * 1e-3
        out.append((gpu, wall))
        total += gpu
        if len(out) >= 1000:
            break
    return out


def summarize(wins, steps):
    """Per-call figures of a list of (gpu, wall) windows."""
    g = np.array([w[0] for w in wins]) / steps
    h = np.array([w[1] for w in wins]) / steps
    med = float(np.median(g))
    return {"us": med * 1e6, "us_min": float(g.min()) * 1e6, "us_max": float(g.max()) * 1e6,
            "spread_pct": float((g.max() - g.min()) / med * 100.0), "windows": len(wins),
            "steps_per_window": steps, "wall_us": float(np.median(h)) * 1e6}


def time_leg(fn, steps, torch, windows=5, warm_seconds=0.3, warmup=3):
    """Warm-up calls, a settling period, then the median of the windows."""
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    fn()
    torch.cuda.synchronize()
    _prewarm(fn, torch, warm_seconds, time.perf_counter() - t0)
    return summarize(time_windows(fn, steps, windows, torch), steps)


def time_graph(fn, steps, torch, warm_seconds=0.3, windows=5):
    """Per-call figures of kernels too short for host launches to keep the
    GPU busy: `steps` calls captured in one HIP graph (on torch's capture
    stream, which the binding launches on), replayed back to back for
    warm_seconds, then one replay per window."""
    fn()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _ in range(steps):
            fn()
    torch.cuda.synchronize()
    t_end = time.perf_counter() + warm_seconds
    while time.perf_counter() < t_end:
        for _ in range(4):
            g.replay()
        torch.cuda.synchronize()
    res = summarize(time_windows(g.replay, 1, windows, torch), steps)
    del g
    return res


def _strip_comments(src):
    """C/C++ source without its comments and blank lines (string and
    character literals kept), so that comment edits leave the hash alone."""
    out, i, n = [], 0, len(src)
    while i < n:
        c = src[i]
        if c in "\"'":
            j = i + 1
            while j < n and src[j] != c:
                j += 2 if src[j] == "\\" else 1
            out.append(src[i:j + 1])
            i = j + 1
        elif src.startswith("//", i):
            while i < n and src[i] != "\n":
                i += 1
        elif src.startswith("/*", i):
            j = src.find("*/", i + 2)
            i = n if j < 0 else j + 2
        else:
            out.append(c)
            i += 1
    lines = (l.rstrip() for l in "".join(out).split("\n"))
    return "\n".join(l for l in lines if l)


# the files that define the headline kernel (a committed traffic summary is
# only used while they are unchanged)
HEADLINE_KERNEL_FILES = ("device_common.h", "mfma_gemm.h", "mfma_direct.h", "mfma_instances.inc",
                         "kernels_direct_f16_nn.hip")


def _src_hash(files=HEADLINE_KERNEL_FILES):
    """Hash of the kernel sources, comments left out."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "dense_gemm_engineering_amd", "csrc")
    for f in sorted(files):
        with open(os.path.join(csrc, f), encoding="utf-8") as fh:
            h.update(f.encode() + _strip_comments(fh.read()).encode())
    return h.hexdigest()[:16]


def _traffic(kernel_key):
    """HBM bytes per launch from a committed rocprofv3 counter summary, if it
    was taken on the current kernel sources; else None."""
    path = os.path.join(ROOT, "profiles", "traffic_%s.md" % kernel_key)
    if not os.path.exists(path):
        return None
    vals = {}
    with open(path) as f:
        for line in f:
            if ":" in line and line.strip().startswith("- "):
                k, v = line.strip()[2:].split(":", 1)
                vals[k.strip()] = v.strip()
    if vals.get("source_hash") != _src_hash():
        return None
    try:
        return float(vals["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


# ------------------------------------------------------------ workloads

def _dev(bits, dtype, torch):
    bits = np.ascontiguousarray(bits)
    if dtype == "f32":
        return torch.from_numpy(bits.view(np.int32).copy()).view(torch.float32).cuda()
    tdt = {"f16": torch.float16, "bf16": torch.bfloat16}[dtype]
    return torch.from_numpy(bits.view(np.int16).copy()).view(tdt).cuda()


def clock_of(clk):
    """Engine clock from per-workgroup records (shader-clock and 100 MHz
    real-time counters at start and end): the mean over workgroups of
    shader cycles / real time, in MHz, and the launch's span in us."""
    c = clk.view(-1, 4).cpu().numpy().astype(np.float64)
    c = c[c[:, 3] > c[:, 1]]
    if len(c) == 0:
        return None, None
    mhz = float(np.mean((c[:, 2] - c[:, 0]) / (c[:, 3] - c[:, 1]) * 100.0))
    span_us = float((c[:, 3].max() - c[:, 1].min()) / 100.0)
    return mhz, span_us


def bench_headline(dge, inputs, torch, steps, windows, repeats, warmup, dtype, seed=0):
    """The 4096^3 legs, interleaved: the headline GEMM (fp16 out), the same
    product with fp32 output, the bf16-operand product, the GEMM with clock
    records, and the MFMA-only probe on the same operands.  Returns per-leg
    window lists and the clock records."""
    M = N = K = 4096
    A, B = inputs.square4096(dtype)
    dA, dB = _dev(A, dtype, torch), _dev(B, dtype, torch)
    Ab, Bb = inputs.square4096("bf16")
    dAb, dBb = _dev(Ab, "bf16", torch), _dev(Bb, "bf16", torch)
    C = torch.empty((M, N), dtype=torch.float16, device="cuda")
    C32 = torch.empty((M, N), dtype=torch.float32, device="cuda")
    wsz = dge.gemm_workspace_size(M, N, K, dA.dtype)
    work = torch.empty(max(wsz // 4, 1), dtype=torch.float32, device="cuda") if wsz else None
    gemm = dge.gemm_f16 if dtype == "f16" else dge.gemm_bf16
    clk = torch.zeros(4 * 1024, dtype=torch.int64, device="cuda")
    clk_mfma = torch.zeros(4 * dge.PROBE_MFMA_GRID, dtype=torch.int64, device="cuda")
    probe_out = torch.empty(dge.PROBE_MFMA_GRID * 512, dtype=torch.float32, device="cuda")
    # the MFMA probe reads B as rows (the N x K view): a transposed copy of B
    dBt = dB.t().contiguous()
    legs = {
        "gemm": lambda: gemm(dA, dB, C, workspace=work),
        "gemm_f32out": lambda: gemm(dA, dB, C32, workspace=work),
        "bf16": lambda: dge.gemm_bf16(dAb, dBb, C, workspace=work),
        "gemm_clock": lambda: dge.probe_clock(dA, dB, C, clk),
        "mfma_only": lambda: dge.probe_mfma(dA, dBt, 128, probe_out, clk_mfma),
    }
    # launches per leg invocation, in launch order, so that a kernel trace of
    # this run can be split by leg
    launch_log = []

    def counted(k, fn):
        def call():
            if launch_log and launch_log[-1][0] == k:
                launch_log[-1][1] += 1
            else:
                launch_log.append([k, 1])
            fn()
        return call

    legs = {k: counted(k, fn) for k, fn in legs.items()}
    for fn in legs.values():
        for _ in range(warmup):
            fn()
    torch.cuda.synchronize()
    rng = np.random.Generator(np.random.PCG64(seed))
    wins = {k: [] for k in legs}
    clocks = {"gemm_clock": [], "mfma_only": []}
    names = list(legs)
    order = []
    for _ in range(repeats):
        for k in [names[i] for i in rng.permutation(len(names))]:
            order.append(k)
            fn = legs[k]
            t0 = time.perf_counter()
            fn()
            torch.cuda.synchronize()
            _prewarm(fn, torch, 0.2, time.perf_counter() - t0)
            w = time_windows(fn, steps, windows, torch)
            wins[k] += w
            if k in clocks:
                clocks[k].append(clock_of(clk if k == "gemm_clock" else clk_mfma))
    del dA, dB, dAb, dBb, C, C32, work, dBt
    return wins, clocks, A, B, order, launch_log


def bench_ksweep(dge, torch, steps, Ks=(1024, 2048, 4096, 8192)):
    """M = N = 4096 fp16 GEMMs (K x N B, fp16 out) over K: per-launch time,
    the engine clock and the spread of workgroup start and end times from the
    kernel's clock records, and a least-squares line time = fixed + per-stage
    x stages whose intercept is the per-launch cost that does not scale with
    K (launch, prologue, epilogue store burst)."""
    out = {}
    for K in Ks:
        a = (torch.randn(4096, K, device="cuda") / 64).half()
        b = (torch.randn(K, 4096, device="cuda") / 64).half()
        C = torch.empty(4096, 4096, device="cuda", dtype=torch.float16)
        clk = torch.zeros(4 * 1024, dtype=torch.int64, device="cuda")
        t = time_leg(lambda: dge.gemm_f16(a, b, C), steps, torch, windows=5, warm_seconds=0.2)
        dge.probe_clock(a, b, C, clk)
        torch.cuda.synchronize()
        c = clk.view(-1, 4)[:256].cpu().numpy().astype(np.float64)
        st, en = (c[:, 1] - c[:, 1].min()) / 100.0, (c[:, 3] - c[:, 1].min()) / 100.0
        out["K%d" % K] = {"us": t["us"], "sclk_mhz": float(np.mean((c[:, 2] - c[:, 0]) /
                                                                   (c[:, 3] - c[:, 1]) * 100.0)),
                          "wg_start_max_us": float(st.max()), "wg_end_min_us": float(en.min()),
                          "wg_end_max_us": float(en.max())}
        del a, b, C
    x = np.array([K / 64 for K in Ks])
    y = np.array([out["K%d" % K]["us"] for K in Ks])
    slope, icpt = np.polyfit(x, y, 1)
    out["fit"] = {"fixed_us": float(icpt), "us_per_stage": float(slope)}
    return out


def bench_stream_peaks(dge, torch, windows=5, nbytes=1 << 30, grids=(2048, 4096, 8192, 16384, 32768)):
    """Measured HBM ceilings: the best streaming read of 1 GiB and the best
    copy of 1 GiB (2 GiB moved) over a few grid sizes, both well beyond the
    256 MB Infinity Cache."""
    src = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    out = torch.empty(max(grids) * 256, dtype=torch.int32, device="cuda")
    read, copy = {}, {}
    for g in grids:
        r = time_leg(lambda: dge.probe_read(src, out, g), 1, torch, windows=windows,
                     warm_seconds=0.1)
        c = time_leg(lambda: dge.probe_copy(src, dst, g), 1, torch, windows=windows,
                     warm_seconds=0.1)
        read[g] = nbytes / (r["us"] * 1e-6) / 1e9
        copy[g] = 2 * nbytes / (c["us"] * 1e-6) / 1e9
    del src, dst
    return {"read_GBs": max(read.values()), "copy_GBs": max(copy.values()),
            "read_GBs_by_grid": read, "copy_GBs_by_grid": copy, "bytes": nbytes}


def bench_prefill(dge, inputs, torch, steps, peaks, rotate_bytes=300e6):
    """Per shape: dequant (HBM-cold by rotating weight sets), GEMM, the fused
    q4 GEMM (gemm_q4_f16), tok/s."""
    out = {}
    for shape in ("up", "attn", "down"):
        A, q, N, K = inputs.prefill_projection(shape)
        dA = _dev(A, "f16", torch)
        nset = max(1, int(np.ceil(rotate_bytes / dequant_alg_bytes(N, K))))
        qs = [torch.from_numpy(q).cuda() for _ in range(nset)]
        ws = [torch.empty((N, K), dtype=torch.float16, device="cuda") for _ in range(nset)]
        C = torch.empty((2048, N), dtype=torch.float16, device="cuda")
        wsz = dge.gemm_workspace_size(2048, N, K, torch.float16)
        work = torch.empty(max(wsz // 4, 1), dtype=torch.float32, device="cuda") if wsz else None
        it = [0]

        def deq():
            i = it[0] % nset
            it[0] += 1
            dge.dequant_q4_f16(qs[i], N, K, out=ws[i])

        def gem():
            dge.gemm_f16(dA, ws[0], C, trans_b=True, workspace=work)

        def fused():
            i = it[0] % nset
            it[0] += 1
            dge.gemm_q4_f16(dA, qs[i], N, K, C, workspace=work)

        td = time_graph(deq, max(steps, nset), torch)
        tg = time_leg(gem, steps, torch)
        tf = time_leg(fused, steps, torch)
        dq_gbs = dequant_alg_bytes(N, K) / (td["us"] * 1e-6) / 1e9
        fl = gemm_flops(2048, N, K)
        out[shape] = {"N": N, "K": K, "dequant_us": td["us"], "gemm_us": tg["us"],
                      "fused_us": tf["us"], "dequant_timing": td, "gemm_timing": tg,
                      "fused_timing": tf,
                      "dequant_GBs": dq_gbs, "dequant_hbm_frac": dq_gbs / HBM_PEAK_GBS,
                      "dequant_frac_of_measured_copy": dq_gbs / peaks["copy_GBs"],
                      "gemm_TFLOPs": fl / tg["us"] / 1e6,
                      "gemm_mfma_frac": fl / tg["us"] / 1e6 / PEAK["f16"],
                      "fused_TFLOPs": fl / tf["us"] / 1e6,
                      "tok_s_dequant_per_call": 2048 / ((td["us"] + tg["us"]) * 1e-6),
                      "tok_s_gemm_only": 2048 / (tg["us"] * 1e-6),
                      "tok_s_fused": 2048 / (tf["us"] * 1e-6)}
        del qs, ws, C, work, dA
    t = {k: (out[k]["dequant_us"] + out[k]["gemm_us"]) * 1e-6 for k in out}
    g = {k: out[k]["gemm_us"] * 1e-6 for k in out}
    f = {k: out[k]["fused_us"] * 1e-6 for k in out}
    out["stack_7b_like"] = {
        "tok_s_dequant_per_call": prefill_stack_tokens_per_s(t["attn"], t["up"], t["down"]),
        "tok_s_gemm_only": prefill_stack_tokens_per_s(g["attn"], g["up"], g["down"]),
        "tok_s_fused": prefill_stack_tokens_per_s(f["attn"], f["up"], f["down"])}
    return out


def bench_kquant(dge, inputs, torch, steps, prefill, peaks, rotate_bytes=300e6):
    """The super-block formats: dequant_f16 per prefill shape (HBM-cold by
    rotating weight sets); two-pass tok/s with the fp16 GEMM time measured by
    the prefill leg (the GEMM is the same one)."""
    out = {}
    for qtype in ("q4_k", "q6_k"):
        res = {}
        for shape in ("up", "attn", "down"):
            _, q, N, K = inputs.kquant_projection(qtype, shape, M=1)
            alg = kquant_alg_bytes(qtype, N, K)
            nset = max(1, int(np.ceil(rotate_bytes / alg)))
            qs = [torch.from_numpy(q).cuda() for _ in range(nset)]
            ws = [torch.empty((N, K), dtype=torch.float16, device="cuda") for _ in range(nset)]
            it = [0]

            def deq():
                i = it[0] % nset
                it[0] += 1
                dge.dequant_f16(qtype, qs[i], N, K, out=ws[i])

            td = time_graph(deq, max(steps, nset), torch)
            gbs = alg / (td["us"] * 1e-6) / 1e9
            tg = prefill[shape]["gemm_us"]
            res[shape] = {"dequant_us": td["us"], "dequant_timing": td, "dequant_GBs": gbs,
                          "dequant_hbm_frac": gbs / HBM_PEAK_GBS,
                          "dequant_frac_of_measured_copy": gbs / peaks["copy_GBs"],
                          "tok_s_dequant_per_call": 2048 / ((td["us"] + tg) * 1e-6)}
            del qs, ws
        t = {k: (res[k]["dequant_us"] + prefill[k]["gemm_us"]) * 1e-6 for k in res}
        res["stack_7b_like"] = {
            "tok_s_dequant_per_call": prefill_stack_tokens_per_s(t["attn"], t["up"], t["down"])}
        out[qtype] = res
    return out


def bench_streamk(dge, torch, steps):
    """The persistent schedule with a stream-K tail (algo "streamk", tile
    chosen by its model) beside the default schedule, fp16 N x K weights."""
    out = {}
    shapes = {"square_4096": (4096, 4096, 4096), "up": (2048, 11008, 4096),
              "attn": (2048, 4096, 4096), "down": (2048, 4096, 11008)}
    for name, (M, N, K) in shapes.items():
        A = torch.randn(M, K, device="cuda", dtype=torch.float16) / K ** 0.5
        B = torch.randn(N, K, device="cuda", dtype=torch.float16) / K ** 0.5
        C = torch.empty(M, N, device="cuda", dtype=torch.float16)
        n = max(dge.gemm_workspace_size(M, N, K, torch.float16),
                dge.gemm_workspace_size_streamk(M, N, K))
        ws = torch.empty(n // 4 + 1, dtype=torch.float32, device="cuda")
        td = time_leg(lambda: dge.gemm_f16(A, B, C, trans_b=True, workspace=ws), steps, torch)
        ts = time_leg(lambda: dge.gemm_ex(A, B, C, trans_b=True, workspace=ws, algo="streamk"),
                      steps, torch)
        fl = gemm_flops(M, N, K)
        out[name] = {"default_us": td["us"], "streamk_us": ts["us"],
                     "default_TFLOPs": fl / td["us"] / 1e6, "streamk_TFLOPs": fl / ts["us"] / 1e6,
                     "default_timing": td, "streamk_timing": ts}
        del A, B, C, ws
    return out


def bench_square256(dge, inputs, torch, steps):
    """The 256^3 fp16 correctness configuration (uniform inputs, fp32 out):
    launch-bound, so its time is reported and no roofline fraction claimed;
    per call from host-launched windows and from graph replays."""
    A, B = inputs.square256()
    dA, dB = _dev(A, "f16", torch), _dev(B, "f16", torch)
    C = torch.empty((256, 256), dtype=torch.float32, device="cuda")
    fn = lambda: dge.gemm_ex(dA, dB, C, out_dtype=torch.float32)
    te = time_leg(fn, steps, torch, warm_seconds=0.1)
    tg = time_graph(fn, steps, torch, warm_seconds=0.1)
    return {"us_host_launched": te["us"], "us_graph": tg["us"],
            "TFLOPs_graph": gemm_flops(256, 256, 256) / tg["us"] / 1e6,
            "timing": te, "graph_timing": tg}


def bench_library_context(dge, torch, steps):
    """Context only: torch.matmul (the vendor BLAS, hipBLASLt on ROCm) on the
    4096^3 fp16 product, K x N and N x K B, beside this library's gemm_f16 on
    the same operands.  Never used by the library."""
    n = 4096
    A = torch.randn(n, n, device="cuda", dtype=torch.float16) / n ** 0.5
    B = torch.randn(n, n, device="cuda", dtype=torch.float16) / n ** 0.5  # K x N
    Bt = B.t().contiguous()                                              # N x K
    C = torch.empty(n, n, device="cuda", dtype=torch.float16)
    fl = gemm_flops(n, n, n)
    out = {}
    for name, lib_fn, own_fn in (
            ("kxn_b", lambda: torch.matmul(A, B, out=C), lambda: dge.gemm_f16(A, B, C)),
            ("nxk_b", lambda: torch.matmul(A, Bt.t(), out=C),
             lambda: dge.gemm_f16(A, Bt, C, trans_b=True))):
        tl = time_leg(lib_fn, steps, torch)
        to = time_leg(own_fn, steps, torch)
        out[name] = {"torch_matmul_us": tl["us"], "gemm_f16_us": to["us"],
                     "torch_matmul_TFLOPs": fl / tl["us"] / 1e6,
                     "gemm_f16_TFLOPs": fl / to["us"] / 1e6,
                     "torch_matmul_timing": tl, "gemm_f16_timing": to}
    del A, B, Bt, C
    return out


def bench_decode(dge, inputs, torch, steps, peaks, rotate_bytes=300e6):
    """The decode shape: M input rows against one 4096 x 4096 fp16 weight
    (HBM-cold by rotating weight copies); bound by reading W once."""
    out = {}
    N = K = 4096
    _, W = inputs.decode_shape(1)
    nset = max(1, int(np.ceil(rotate_bytes / (N * K * 2))))
    Ws = [_dev(W, "f16", torch) for _ in range(nset)]
    for M in inputs.DECODE_ROWS:
        X, _ = inputs.decode_shape(M)
        dX = _dev(X, "f16", torch)
        C = torch.empty((M, N), dtype=torch.float16, device="cuda")
        wsz = dge.gemm_workspace_size(M, N, K, torch.float16)
        work = torch.empty(max(wsz // 4, 1), dtype=torch.float32, device="cuda") if wsz else None
        it = [0]

        def run():
            i = it[0] % nset
            it[0] += 1
            dge.gemm_f16(dX, Ws[i], C, trans_b=True, workspace=work)

        t = time_graph(run, max(steps, nset), torch)
        alg = gemm_alg_bytes(M, N, K, 2, 2)
        gbs = alg / (t["us"] * 1e-6) / 1e9
        out["M%d" % M] = {"us": t["us"], "timing": t, "GBs": gbs,
                          "hbm_frac": gbs / HBM_PEAK_GBS,
                          "frac_of_measured_read": gbs / peaks["read_GBs"],
                          "tokens_per_s": M / (t["us"] * 1e-6)}
    del Ws
    return out


def bench_skinny(dge, inputs, torch, steps, peaks, rotate_bytes=300e6):
    out = {}
    for N in (160, 32):
        X, W, bias = inputs.tall_skinny(N)
        alg = gemm_alg_bytes(65536, N, 160, 2, 2, bias_bytes=2 * N)
        nset = max(1, int(np.ceil(rotate_bytes / alg)))
        Xs = [_dev(X, "f16", torch) for _ in range(nset)]
        Cs = [torch.empty((65536, N), dtype=torch.float16, device="cuda") for _ in range(nset)]
        dW, db = _dev(W, "f16", torch), _dev(bias, "f16", torch)
        it = [0]

        def run():
            i = it[0] % nset
            it[0] += 1
            dge.gemm_f16(Xs[i], dW, Cs[i], epi="bias_gelu", bias=db)

        t = time_graph(run, max(steps, nset), torch)
        # the same call on one input set: its 25-42 MB stay in the Infinity Cache
        t_warm = time_graph(lambda: dge.gemm_f16(Xs[0], dW, Cs[0], epi="bias_gelu", bias=db),
                            steps, torch)
        gbs = alg / (t["us"] * 1e-6) / 1e9
        out["N%d" % N] = {"us": t["us"], "timing": t, "GBs": gbs,
                          "hbm_frac": gbs / HBM_PEAK_GBS,
                          "frac_of_measured_copy": gbs / peaks["copy_GBs"],
                          "TFLOPs": gemm_flops(65536, N, 160) / (t["us"] * 1e-6) / 1e12,
                          "us_cache_warm": t_warm["us"]}
        del Xs, Cs
    return out


def bench_ladder(dge, inputs, torch, steps):
    out = {}
    for n in (1024, 2048, 4096):
        A, B = inputs.fp32_square(n)
        dA, dB = _dev(A, "f32", torch), _dev(B, "f32", torch)
        C = torch.empty((n, n), dtype=torch.float32, device="cuda")
        # the MFMA rung gets the workspace the library asks for (a K split
        # fills the CUs at n = 1024)
        wsz = dge.gemm_workspace_size(n, n, n, torch.float32)
        ws = torch.empty(max(wsz // 4, 1), dtype=torch.float32, device="cuda") if wsz else None
        row = {}
        algos = ["naive", "lds_tiled", "mfma"] if n <= 2048 else ["lds_tiled", "mfma"]
        for algo in algos:
            s = max(2, steps // 10) if algo != "mfma" else steps
            w = ws if algo == "mfma" else None
            t = time_leg(lambda: dge.gemm_ex(dA, dB, C, algo=algo, workspace=w), s, torch,
                         warm_seconds=0.1)
            tf = gemm_flops(n, n, n) / (t["us"] * 1e-6) / 1e12
            row[algo] = {"us": t["us"], "TFLOPs": tf, "fp32_mfma_frac": tf / PEAK["f32"],
                         "timing": t}
        out["n%d" % n] = row
    return out


# ------------------------------------------------------------ CPU oracle

def _oracle_rate(fn, flops, threads):
    t0 = time.perf_counter()
    fn(threads)
    t = time.perf_counter() - t0
    return {"seconds": t, "GFLOPs": flops / t / 1e9, "threads": threads}


def cpu_baseline(A, B, inputs, seconds_target=15.0):
    """The oracle, untuned (binary64 i-k-j loops), on the host cores: the
    headline figure on the first rows of the 4096^3 product (all of them when
    that takes at most about 2x seconds_target), and per workload a bounded
    sample on all cores, plus one thread for the 256^3 and 1024^3 products."""
    import oracle
    cores = oracle.default_threads()
    probe = max(cores, 64)
    t0 = time.perf_counter()
    oracle.gemm(A[:probe], B, "f16", want_U=False, threads=cores)
    tp = time.perf_counter() - t0
    est_full = tp * 4096 / probe
    rows = 4096 if est_full <= 2 * seconds_target else int(4096 * seconds_target / est_full)
    rows = max(probe, rows - rows % cores)
    t0 = time.perf_counter()
    oracle.gemm(A[:rows], B, "f16", want_U=False, threads=cores)
    t = time.perf_counter() - t0
    res = {"value": gemm_flops(rows, 4096, 4096) / t / 1e12, "unit": "TFLOP/s", "cores": cores,
           "kind": "oracle", "seconds": t,
           "sample": "rows 0..%d of the 4096^3 fp16 product (%.1f GFLOP), binary64 "
                     "accumulation, row-parallel over %d threads"
                     % (rows - 1, gemm_flops(rows, 4096, 4096) / 1e9, cores)}
    per = {}
    a1, b1 = inputs.square256()
    for th in (cores, 1):
        per["square256_threads%d" % th] = _oracle_rate(
            lambda t: oracle.gemm(a1, b1, "f16", want_U=False, threads=t), gemm_flops(256, 256, 256), th)
    a3, b3 = inputs.fp32_square(1024)
    for th in (cores, 1):
        per["fp32_1024_threads%d" % th] = _oracle_rate(
            lambda t: oracle.gemm(a3, b3, "f32", want_U=False, threads=t), gemm_flops(1024, 1024, 1024), th)
    for n in (2048, 4096):
        a, b = inputs.fp32_square(n)
        r = 256
        per["fp32_%d_rows%d" % (n, r)] = _oracle_rate(
            lambda t: oracle.gemm(a[:r], b, "f32", want_U=False, threads=t), gemm_flops(r, n, n), cores)
    for shape in ("up", "attn", "down"):
        a, q, N, K = inputs.prefill_projection(shape)
        r = 64
        W16 = oracle.dequant_q4(q, N, K)
        per["prefill_%s_rows%d" % (shape, r)] = _oracle_rate(
            lambda t: oracle.gemm(a[:r], W16, "f16", trans_b=True, want_U=False, threads=t),
            gemm_flops(r, N, K), cores)
        t0 = time.perf_counter()
        oracle.dequant_q4(q, N, K)
        dt = time.perf_counter() - t0
        per["dequant_%s" % shape] = {"seconds": dt, "threads": 1,
                                     "GBs": dequant_alg_bytes(N, K) / dt / 1e9}
    for N in (160, 32):
        x, w, bias = inputs.tall_skinny(N)
        bd = oracle.decode(bias, "f16")
        per["skinny_N%d" % N] = _oracle_rate(
            lambda t: oracle.gemm(x, w, "f16", epi="bias_gelu", bias=bd, want_U=False, threads=t),
            gemm_flops(65536, N, 160), cores)
    res["per_workload"] = per
    return res


# ------------------------------------------------------------ profiler runs

def _kernel_set_calls(name, dge, inputs, torch):
    """(label, call) pairs of one workload's kernels on its full-size inputs."""
    calls = []
    if name == "square4096":
        A, B = inputs.square4096("f16")
        dA, dB = _dev(A, "f16", torch), _dev(B, "f16", torch)
        C = torch.empty((4096, 4096), dtype=torch.float16, device="cuda")
        calls.append(("gemm_f16 4096^3", lambda: dge.gemm_f16(dA, dB, C)))
    elif name == "prefill":
        for shape in ("attn", "up", "down"):
            A, q, N, K = inputs.prefill_projection(shape)
            dA, dq = _dev(A, "f16", torch), torch.from_numpy(q).cuda()
            w16 = torch.empty((N, K), dtype=torch.float16, device="cuda")
            C = torch.empty((2048, N), dtype=torch.float16, device="cuda")
            wsz = dge.gemm_workspace_size(2048, N, K, torch.float16)
            ws = torch.empty(max(wsz // 4, 1), dtype=torch.float32, device="cuda")
            dge.dequant_q4_f16(dq, N, K, out=w16)
            calls.append(("dequant_q4_f16 %s" % shape,
                          lambda dq=dq, N=N, K=K, w16=w16: dge.dequant_q4_f16(dq, N, K, out=w16)))
            calls.append(("gemm_f16 %s" % shape,
                          lambda dA=dA, w16=w16, C=C, ws=ws: dge.gemm_f16(dA, w16, C, trans_b=True,
                                                                         workspace=ws)))
            calls.append(("gemm_q4_f16 %s" % shape,
                          lambda dA=dA, dq=dq, N=N, K=K, C=C, ws=ws: dge.gemm_q4_f16(
                              dA, dq, N, K, C, workspace=ws)))
    elif name == "skinny":
        for N in (160, 32):
            X, W, bias = inputs.tall_skinny(N)
            dX, dW, db = _dev(X, "f16", torch), _dev(W, "f16", torch), _dev(bias, "f16", torch)
            C = torch.empty((65536, N), dtype=torch.float16, device="cuda")
            calls.append(("skinny N=%d" % N, lambda dX=dX, dW=dW, C=C, db=db: dge.gemm_f16(
                dX, dW, C, epi="bias_gelu", bias=db)))
    elif name == "decode":
        _, W = inputs.decode_shape(1)
        dW = _dev(W, "f16", torch)
        for M in inputs.DECODE_ROWS:
            X, _ = inputs.decode_shape(M)
            dX = _dev(X, "f16", torch)
            C = torch.empty((M, 4096), dtype=torch.float16, device="cuda")
            wsz = dge.gemm_workspace_size(M, 4096, 4096, torch.float16)
            ws = torch.empty(max(wsz // 4, 1), dtype=torch.float32, device="cuda")
            calls.append(("decode M=%d" % M, lambda dX=dX, C=C, ws=ws: dge.gemm_f16(
                dX, dW, C, trans_b=True, workspace=ws)))
    elif name == "streamk":
        shapes = {"square_4096": (4096, 4096, 4096), "up": (2048, 11008, 4096),
                  "attn": (2048, 4096, 4096), "down": (2048, 4096, 11008)}
        for label, (M, N, K) in shapes.items():
            A = torch.randn(M, K, device="cuda", dtype=torch.float16) / K ** 0.5
            B = torch.randn(N, K, device="cuda", dtype=torch.float16) / K ** 0.5
            C = torch.empty(M, N, device="cuda", dtype=torch.float16)
            n = max(dge.gemm_workspace_size(M, N, K, torch.float16),
                    dge.gemm_workspace_size_streamk(M, N, K))
            ws = torch.empty(n // 4 + 1, dtype=torch.float32, device="cuda")
            calls.append(("default %s" % label, lambda A=A, B=B, C=C, ws=ws: dge.gemm_f16(
                A, B, C, trans_b=True, workspace=ws)))
            calls.append(("streamk %s" % label, lambda A=A, B=B, C=C, ws=ws: dge.gemm_ex(
                A, B, C, trans_b=True, workspace=ws, algo="streamk")))
    return calls


KERNEL_SETS = ("square4096", "prefill", "skinny", "decode", "streamk")


def run_phases(dge, inputs, torch, steps, repeats=5):
    """Phase records (gemm_probe_phases: 100 MHz real-time counter, per
    workgroup) of the split decode at M = 32 and 64 and the tall-skinny
    bias+GELU at N = 160 and 32.  Each record follows `steps` back-to-back
    calls of the same shape (HBM-cold weight / input sets, so the clock and
    caches are in their steady state); per phase the median and maximum over
    workgroups, relative to the earliest workgroup start, medians over
    `repeats` records."""
    out = {}

    def summarize_rec(recs, names):
        rows = []
        for r in recs:
            r = r[r[:, 0] > 0].astype(np.float64)
            r = (r - r[:, 0].min()) / 100.0
            rows.append([[float(np.median(r[:, i])), float(r[:, i].max())] for i in range(4)])
        a = np.median(np.array(rows), axis=0)
        return {n: {"median_us": round(float(a[i][0]), 3), "max_us": round(float(a[i][1]), 3)}
                for i, n in enumerate(names)}

    _, W = inputs.decode_shape(1)
    nset = max(1, int(np.ceil(300e6 / (4096 * 4096 * 2))))
    Ws = [_dev(W, "f16", torch) for _ in range(nset)]
    for M in (32, 64):
        X, _ = inputs.decode_shape(M)
        dX = _dev(X, "f16", torch)
        C = torch.empty((M, 4096), dtype=torch.float16, device="cuda")
        ws = torch.empty(dge.gemm_workspace_size(M, 4096, 4096, torch.float16) // 4 + 1,
                         dtype=torch.float32, device="cuda")
        rec = torch.zeros(4 * 512, dtype=torch.int64, device="cuda")
        recs = []
        for rep in range(repeats):
            for i in range(steps):
                dge.gemm_f16(dX, Ws[i % nset], C, trans_b=True, workspace=ws)
            rec.zero_()
            dge.probe_phases(dX, Ws[(steps + rep) % nset], C, rec, trans_b=True, workspace=ws)
            torch.cuda.synchronize()
            recs.append(rec.view(-1, 4).cpu().numpy())
        out["decode_M%d" % M] = summarize_rec(
            recs, ("start", "first_span_landed_wave0", "loads_and_mfma_done", "partial_issued"))
    del Ws
    for N in (160, 32):
        X, Wk, bias = inputs.tall_skinny(N)
        nset = max(1, int(np.ceil(300e6 / (65536 * (160 + N) * 2))))
        Xs = [_dev(X, "f16", torch) for _ in range(nset)]
        dW, db = _dev(Wk, "f16", torch), _dev(bias, "f16", torch)
        C = torch.empty((65536, N), dtype=torch.float16, device="cuda")
        rec = torch.zeros(4 * 512, dtype=torch.int64, device="cuda")
        recs = []
        for rep in range(repeats):
            for i in range(steps):
                dge.gemm_f16(Xs[i % nset], dW, C, epi="bias_gelu", bias=db)
            rec.zero_()
            dge.probe_phases(Xs[(steps + rep) % nset], dW, C, rec, epi="bias_gelu", bias=db)
            torch.cuda.synchronize()
            recs.append(rec.view(-1, 4).cpu().numpy())
        out["skinny_N%d" % N] = summarize_rec(
            recs, ("start", "w_staged", "first_rows_landed_wave0", "wave0_done"))
        del Xs
    return out


def run_kernel_set(name, dge, inputs, torch, steps, warmup):
    calls = _kernel_set_calls(name, dge, inputs, torch)
    for label, fn in calls:
        for _ in range(warmup):
            fn()
        torch.cuda.synchronize()
        for _ in range(steps):
            fn()
        torch.cuda.synchronize()
        print(json.dumps({"kernel_set": name, "call": label, "launches": steps}), flush=True)


# ------------------------------------------------------------ main

def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    # launches per timed window (each leg: the median of at least --windows
    # windows, more when they add up to under 50 ms)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--windows", type=int, default=7)
    ap.add_argument("--repeats", type=int, default=3)
    ap.add_argument("--dtype", default="f16", choices=["f16", "bf16"])
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--no-extra", action="store_true", help="only the 4096^3 legs")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only a plain 256 MiB device-to-device copy, 5 times (the reference "
                         "for scaling HBM byte counters)")
    ap.add_argument("--phases", action="store_true",
                    help="only the phase records of the split decode and tall-skinny kernels")
    ap.add_argument("--kernel-set", choices=sorted(KERNEL_SETS),
                    help="only launch one workload's kernels --steps times each, after "
                         "--warmup launches, and print their names (for profiler runs)")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU: the library has no multi-GPU path "
              "(requested --gpus %d)" % args.gpus, file=sys.stderr)
        sys.exit(2)

    import torch
    import dense_gemm_engineering_amd.binding as dge
    from dense_gemm_engineering_amd import inputs

    if args.phases:
        dge.gemm_init()
        print(json.dumps({"phases": run_phases(dge, inputs, torch, max(args.steps, 30))}), flush=True)
        return
    if args.kernel_set:
        run_kernel_set(args.kernel_set, dge, inputs, torch, args.steps, args.warmup)
        return

    if args.copy_calibration:
        n = 256 << 20
        src = torch.ones(n // 2, dtype=torch.float16, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_read_per_launch": n, "copy_bytes_written_per_launch": n,
                          "launches": 5}), flush=True)
        return

    dge.gemm_init()
    M = N = K = 4096
    flops = gemm_flops(M, N, K)
    wins, clocks, A, B, order, launch_log = bench_headline(dge, inputs, torch, args.steps, args.windows,
                                               args.repeats, args.warmup, args.dtype)
    head = summarize(wins["gemm"], args.steps)
    ms_per_step = head["wall_us"] * 1e-3
    value = flops / (head["wall_us"] * 1e-6) / 1e12
    achieved = flops / (head["us"] * 1e-6) / 1e12
    legs = {k: summarize(w, args.steps) for k, w in wins.items()}
    mfma_only = flops / (legs["mfma_only"]["us"] * 1e-6) / 1e12

    def med_clock(k):
        v = [c[0] for c in clocks[k] if c[0]]
        return float(np.median(v)) if v else None

    sclk = med_clock("gemm_clock")
    sclk_mfma = med_clock("mfma_only")
    spans = [c[1] for c in clocks["gemm_clock"] if c[1]]
    peaks = bench_stream_peaks(dge, torch)
    traffic = _traffic("gemm_%s_4096" % args.dtype)
    peak = PEAK[args.dtype]
    line = {
        "metric": "TFLOP/s fp16 GEMM 4096^3 (% of MFMA peak); 2K-token prefill GEMM tok/s",
        "value": value, "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms_per_step, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": args.dtype, "data": "synthetic",
        "config": {"workload": "%s GEMM M=N=K=4096, row-major A (MxK) and B (KxN), entries "
                               "N(0,1)/sqrt(K), fp32 accumulate, fp16 output, alpha=1, beta=0"
                               % args.dtype, "M": M, "N": N, "K": K, "accumulate": "f32",
                   "output": "f16", "parallelism": "single GPU"},
        "roofline": {
            "bound": "mfma", "achieved": achieved, "peak": peak, "unit": "TFLOP/s",
            "frac": achieved / peak, "traffic": traffic,
            "kernel_us_median": head["us"], "kernel_us_min": head["us_min"],
            "kernel_us_max": head["us_max"], "windows": head["windows"],
            "steps_per_window": args.steps, "repeats": args.repeats,
            "alg_bytes": gemm_alg_bytes(M, N, K, 2, 2),
            "kernel": "gemm_direct_kernel<%s, 256x256 tile, 8 waves, 16x16x32 MFMA, K x N B>"
                      % args.dtype,
            # the engine clock over the same kernel (its own clock records) and
            # the measured ceilings at the workload's data
            "sclk_mhz": sclk,
            "frac_at_sclk": achieved / (peak * sclk / 2400.0) if sclk else None,
            "clock_launch_span_us": float(np.median(spans)) if spans else None,
            "measured_peak": {"mfma_only_TFLOPs": mfma_only, "mfma_only_sclk_mhz": sclk_mfma,
                              "mfma_only_us": legs["mfma_only"]["us"],
                              "frac_of_mfma_only": achieved / mfma_only,
                              "hbm_read_GBs": peaks["read_GBs"],
                              "hbm_copy_GBs": peaks["copy_GBs"]},
        },
        "legs_4096": {
            "gemm_f16out": legs["gemm"],
            "gemm_f32out": dict(legs["gemm_f32out"], TFLOPs=flops / legs["gemm_f32out"]["us"] / 1e6),
            "bf16_f16out": dict(legs["bf16"], TFLOPs=flops / legs["bf16"]["us"] / 1e6,
                                mfma_frac=flops / legs["bf16"]["us"] / 1e6 / PEAK["bf16"]),
            "gemm_with_clock_records": legs["gemm_clock"],
            "mfma_only_probe": legs["mfma_only"],
            # the order the legs ran in (warm-up calls, a settling period and
            # the windows of each); the fp16-out, fp32-out and clock-record
            # legs launch the same kernel
            "order": order,
            "launch_log": launch_log,
        },
        "hbm_peaks": peaks,
    }
    if not args.no_extra:
        extra_steps = max(10, min(args.steps, 30))
        line["ksweep_4096"] = bench_ksweep(dge, torch, extra_steps)
        line["prefill_2048"] = bench_prefill(dge, inputs, torch, extra_steps, peaks)
        line["prefill_kquant"] = bench_kquant(dge, inputs, torch, extra_steps,
                                              line["prefill_2048"], peaks)
        line["streamk_vs_default"] = bench_streamk(dge, torch, extra_steps)
        line["skinny_bias_gelu"] = bench_skinny(dge, inputs, torch, extra_steps, peaks)
        line["decode_4096"] = bench_decode(dge, inputs, torch, extra_steps, peaks)
        line["fp32_ladder"] = bench_ladder(dge, inputs, torch, extra_steps)
        line["library_context"] = bench_library_context(dge, torch, extra_steps)
        line["square256_f32out"] = bench_square256(dge, inputs, torch, extra_steps)
    if not args.no_cpu:
        line["cpu_baseline"] = cpu_baseline(A, B, inputs, args.cpu_seconds)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
