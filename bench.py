"""Benchmark: NVFP4 four-over-six quantize throughput on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--warmup-ms T]
                    [--err mae|mse] [--no-cpu] [--no-extra] [--no-pages]
                    [--only WORKLOAD] [--copy-calib]

Workload (the metric's configuration): row-scaled four-over-six NVFP4
quantize of an 8192x7168 bf16 activation (N(0,1) with a log-uniform per-row
std in [1e-2, 1e2]), MAE selection, e4m3 scale bound 256, per-row global amax
computed in the same kernel.  One step = one launch of that fused kernel
(nvfp4_quantize_4over6) over one input buffer set; four buffer sets rotate so
the 600 MB footprint exceeds the 256 MB Infinity Cache.  GB/s counts
algorithmic bytes in + out: bf16 input + packed e2m1 codes + e4m3 scale bytes
(2.5625 B/element, 150,470,656 B per step), the pages' convention.

Timing: HIP events recorded on the stream the C ABI launches on (torch's
current stream) bracket the K timed steps.  Each step is exactly one launch
of the dominant kernel, so region time / K bounds that kernel's average
duration from above; `value` and `roofline.achieved` both come from it.

Before timing, the GPU output is checked bit for bit against the CPU oracle on
a sample of rows.  The line also carries the roofline (8 TB/s HBM peak; HBM
traffic from the committed rocprofv3 counter summary while it matches the
current kernel source) and the CPU oracle timed over a process pool of every
core this process may use.  Unless --no-extra, the other workloads are timed
too (each parity-checked on a sample first) and reported under "extra".
Every timed region follows an untimed warmup of at least W steps (W/4 for
the extras) and at least --warmup-ms (30) of GPU time.
`--only NAME` runs one workload's steps alone (for rocprofv3 runs).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
N_SETS = 4
CSRC = os.path.join(ROOT, "fp4_block_quantization_nvfp4_amd", "csrc")
PROFILES = os.path.join(ROOT, "profiles")
METRIC = "act_rows_8192x7168_4over6_mae"

# Committed HBM-traffic summaries (profiles/), each valid while the hash of
# its kernel's sources matches: workload -> (summary file, source files).
_COMMON = ["nvfp4_device.hpp", "nvfp4_plan.hpp"]
TRAFFIC = {
    METRIC: ("traffic_4over6_act_rows_8192x7168.txt", ["k_4over6.hip", "nvfp4_fos.hpp"] + _COMMON),
    "weight_2d_7168x18432_quantize_2d_sr": ("traffic_quant2d_sr_weight_7168x18432.txt",
                                            ["k_2d.hip", "nvfp4_strip.hpp"] + _COMMON),
    "weight_2d_7168x18432_4over6_16x16_mae": ("traffic_4over6_2d_weight_7168x18432.txt",
                                              ["k_rowcol.hip", "nvfp4_fos.hpp"] + _COMMON),
    "weight_2d_7168x18432_rowcol_1x16_standard": ("traffic_rowcol_standard_weight_7168x18432.txt",
                                                  ["k_rowcol.hip", "nvfp4_fos.hpp"] + _COMMON),
    "weight_2d_7168x18432_rowcol_1x16_4over6_mae": ("traffic_rowcol_4over6_weight_7168x18432.txt",
                                                    ["k_rowcol.hip", "nvfp4_fos.hpp"] + _COMMON),
    "heavy_16384x8192_qdq_sr_ef": ("traffic_qdq_sr_ef_heavy_16384x8192.txt", ["k_1x16.hip"] + _COMMON),
    "ef_weight_4096x4096_qdq_step_rtn_ef": ("traffic_qdq_ef_fp32_4096x4096.txt", ["k_1x16.hip"] + _COMMON),
    "weight_2d_7168x18432_amax": ("traffic_amax_weight_7168x18432.txt", ["k_amax.hip"] + _COMMON),
}


def src_hash(workload=METRIC):
    h = hashlib.sha256()
    for f in TRAFFIC[workload][1]:
        h.update(open(os.path.join(CSRC, f), "rb").read())
    return h.hexdigest()[:16]


def traffic_file(workload):
    return os.path.join(PROFILES, TRAFFIC[workload][0])


def read_traffic(workload=METRIC, path=None):
    """HBM bytes per launch from the committed counter summary, or None when
    absent or taken on a different kernel source."""
    path = path or traffic_file(workload)
    if not os.path.exists(path):
        return None
    kv = {}
    for line in open(path):
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            kv[k.strip()] = v.strip()
    if kv.get("kernel_src_sha256_16") != src_hash(workload):
        return None
    try:
        return int(float(kv["hbm_bytes_per_launch"]))
    except (KeyError, ValueError):
        return None


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def dev_bf16(torch, np, bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


def time_ms(torch, fn, warmup, steps, host=None):
    """Average ms per step over `steps` steps on torch's current stream (the
    stream every C-ABI call here is issued on), after `warmup` steps: events
    bracket the whole timed region, with a synchronization on both sides.
    If `host` is a dict, host["us_per_call"] receives the host-side time to
    submit one step (the loop without the final synchronization)."""
    for i in range(warmup):
        fn(i)
    torch.cuda.synchronize()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record()
    h0 = time.perf_counter()
    for i in range(steps):
        fn(i)
    h1 = time.perf_counter()
    t1.record()
    torch.cuda.synchronize()
    if host is not None:
        host["us_per_call"] = (h1 - h0) * 1e6 / steps
    return t0.elapsed_time(t1) / steps


def warm(torch, fn, min_steps, min_ms, cap=4000):
    """Untimed warmup: at least `min_steps` steps and at least `min_ms` of GPU
    time (batches of 8 steps timed by events; exactly `min_steps` when
    `min_ms` is 0), at most `cap` steps.  Back-to-back launches that follow
    an idle GPU (the parity check runs on the CPU) run well below their
    steady rate for several milliseconds (the four-over-six row kernel: 33
    -> 42 -> 35 us per launch over its first ~7 ms); a fixed handful of
    warmup steps would fold that transient into the timed region.  Returns
    the steps run."""
    if min_ms <= 0:
        for i in range(min_steps):
            fn(i)
        torch.cuda.synchronize()
        return min_steps
    n, t = 0, 0.0
    while (n < min_steps or t < min_ms) and n < cap:
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        for k in range(8):
            fn(n + k)
        e1.record()
        torch.cuda.synchronize()
        t += e0.elapsed_time(e1)
        n += 8
    return n


def copy_ceiling_gbs(torch, nbytes=1 << 30, reps=10):
    """Plain device-to-device copy throughput (bytes read + written per
    second) over two alternating pairs of buffers larger than the Infinity
    Cache: the practical ceiling of a streaming kernel on this machine."""
    n = nbytes // 4
    bufs = [torch.empty(n, dtype=torch.float32, device="cuda") for _ in range(4)]
    for b in bufs:
        b.fill_(1.0)
    for i in range(3):
        bufs[2 * (i % 2) + 1].copy_(bufs[2 * (i % 2)])
    torch.cuda.synchronize()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record()
    for i in range(reps):
        bufs[2 * (i % 2) + 1].copy_(bufs[2 * (i % 2)])
    t1.record()
    torch.cuda.synchronize()
    ms = t0.elapsed_time(t1) / reps
    del bufs
    torch.cuda.empty_cache()
    return 2 * nbytes / (ms * 1e-3) / 1e9


def check_rows(np, got, want, what):
    g, w = np.ascontiguousarray(got), np.ascontiguousarray(want)
    if g.dtype == np.float32:
        g, w = g.view(np.uint32), w.view(np.uint32)
    if not np.array_equal(g, w):
        raise SystemExit(f"bench: parity check failed for {what}")


# ------------------------------------------------------------- CPU baseline
def _cpu_task(x, err):
    """One chunk of rows through the oracle: per-row amax, then four-over-six
    (runs in a spawned worker process)."""
    import oracle

    A = oracle.amax(x, mode="row")
    oracle.quantize_4over6(x, A, err_mode=err, bound=256.0)
    return x.size


def cpu_baseline(np, x_bits, err, seconds):
    """The oracle on the metric workload over a pool of every core this
    process may use (one single-threaded worker per core), whole passes over
    the tensor until `seconds` of wall time; GB/s in the metric's bytes."""
    import multiprocessing as mp

    cores = len(os.sched_getaffinity(0))
    os.environ["OMP_NUM_THREADS"] = "1"
    M = x_bits.shape[0]
    step = max(1, M // (cores * 4))
    chunks = [(x_bits[a:a + step], err) for a in range(0, M, step)]
    with mp.get_context("spawn").Pool(cores) as pool:
        pool.starmap(_cpu_task, chunks[:cores])  # workers up and warm
        n, passes, t0 = 0, 0, time.perf_counter()
        while True:
            n += sum(pool.starmap(_cpu_task, chunks))
            passes += 1
            dt = time.perf_counter() - t0
            if dt >= seconds or passes >= 20:
                break
    return {
        "value": round(n * 2.5625 / dt / 1e9, 5),
        "unit": "GB/s",
        "cores": cores,
        "kind": "oracle",
        "sample": f"{passes} whole pass(es) over the {M}x{x_bits.shape[1]} tensor ({n} elements), per-row amax + "
                  f"four-over-six {err.upper()} bound 256, numpy float32, {cores} single-threaded worker "
                  f"processes ({cpu_model()}); {dt:.2f} s wall, {n / dt / 1e6:.2f} M elements/s",
    }


# ---------------------------------------------------------------- workloads
class Ctx:
    """Shared handles for the workload builders."""

    def __init__(self, np, torch, L, lib, stream, workloads, oracle):
        self.np, self.torch, self.L, self.lib, self.stream = np, torch, L, lib, stream
        self.workloads, self.oracle = workloads, oracle


def _call(c, what, status):
    if status:
        c.L.check(status, what)


def build_metric(c, err):
    """Row-scaled four-over-six on 8192x7168 bf16 (per-row amax in the pass)."""
    np, torch, L = c.np, c.torch, c.L
    M, K = c.workloads.ACT_ROWS_SHAPE
    x_bits = c.workloads.act_rows_input()
    xs = [dev_bf16(torch, np, x_bits) for _ in range(N_SETS)]
    packed = [torch.empty((M, K // 2), dtype=torch.uint8, device="cuda") for _ in range(N_SETS)]
    scales = [torch.empty((M, K // 16), dtype=torch.uint8, device="cuda") for _ in range(N_SETS)]
    amaxes = [torch.empty(M, dtype=torch.float32, device="cuda") for _ in range(N_SETS)]
    e = L.MAE if err == "mae" else L.MSE
    args = [(xs[j].data_ptr(), L.BF16, M, K, amaxes[j].data_ptr(), L.SCALE_ROW, 0, e, 256.0,
             packed[j].data_ptr(), scales[j].data_ptr(), c.stream) for j in range(N_SETS)]

    def step(i):
        _call(c, "nvfp4_quantize_4over6", c.lib.nvfp4_quantize_4over6(*args[i % N_SETS]))

    def check():
        step(0)
        torch.cuda.synchronize()
        rows = np.unique(np.concatenate([np.arange(16), np.random.default_rng(0).integers(0, M, 48), [M - 1]]))
        A = c.oracle.amax(x_bits[rows], mode="row")
        wp, ws = c.oracle.quantize_4over6(x_bits[rows], A, err_mode=err, bound=256.0)
        check_rows(np, amaxes[0].cpu().numpy()[rows], A, "row amax")
        check_rows(np, packed[0].cpu().numpy()[rows], wp, f"codes ({err})")
        check_rows(np, scales[0].cpu().numpy()[rows], ws, f"scales ({err})")

    return dict(step=step, check=check, bytes=M * K * 2 + M * K // 2 + M * K // 16, x_bits=x_bits,
                kernel="k_4over6_rows", note=f"the metric workload with err_mode {err}; per-row amax in-pass")


def build_small(c, kind):
    np, torch, L = c.np, c.torch, c.L
    x = c.workloads.small_input()
    xd = torch.from_numpy(x).cuda()
    p = torch.empty((256, 128), dtype=torch.uint8, device="cuda")
    s = torch.empty((256, 16), dtype=torch.uint8, device="cuda")
    o = torch.empty((256, 256), dtype=torch.bfloat16, device="cuda")
    if kind == "dequantize":
        c.lib.nvfp4_quantize(xd.data_ptr(), L.F32, 256, 256, None, None, 0, 0, 0, p.data_ptr(), s.data_ptr(), c.stream)

        def step(i):
            _call(c, "nvfp4_dequantize", c.lib.nvfp4_dequantize(p.data_ptr(), s.data_ptr(), 256, 256, 0, None, 0,
                                                                 448.0, o.data_ptr(), L.BF16, c.stream))

        def check():
            step(0)
            wp, ws = c.oracle.quantize(x)
            check_rows(np, o.cpu().view(torch.int16).numpy().view(np.uint16),
                       c.oracle.dequantize(wp, ws, 256, 256), "small dequantize")

        return dict(step=step, check=check, bytes=256 * 128 + 256 * 16 + 256 * 256 * 2, kernel="k_dequant",
                    note="launch-bound")
    sr = int(kind == "sr")

    def step(i):
        _call(c, "nvfp4_quantize", c.lib.nvfp4_quantize(xd.data_ptr(), L.F32, 256, 256, None, None, sr, 0, 0,
                                                         p.data_ptr(), s.data_ptr(), c.stream))

    def check():
        step(0)
        wp, ws = c.oracle.quantize(x, stochastic=bool(sr))
        check_rows(np, p.cpu().numpy(), wp, "small codes")
        check_rows(np, s.cpu().numpy(), ws, "small scales")

    return dict(step=step, check=check, bytes=256 * 256 * 4 + 256 * 128 + 256 * 16, kernel="k_quant1x16",
                note="launch-bound")


def build_ef(c, sr):
    np, torch, L = c.np, c.torch, c.L
    Mw, Kw = c.workloads.EF_SHAPE
    w = torch.from_numpy(c.workloads.ef_weight0().view(np.int16)).view(torch.bfloat16).cuda().float()
    xs = [w.clone() for _ in range(N_SETS)]
    rs = [torch.zeros_like(w) for _ in range(N_SETS)]
    outs = [torch.empty((Mw, Kw), dtype=torch.bfloat16, device="cuda") for _ in range(N_SETS)]

    def step(i):
        j = i % N_SETS
        _call(c, "nvfp4_qdq", c.lib.nvfp4_qdq(xs[j].data_ptr(), L.F32, Mw, Kw, rs[j].data_ptr(), None, sr, 0, i,
                                               outs[j].data_ptr(), L.BF16, None, None, c.stream))

    def check():
        r0 = np.zeros((32, Kw), np.float32)
        rd = torch.zeros((32, Kw), dtype=torch.float32, device="cuda")
        od = torch.empty((32, Kw), dtype=torch.bfloat16, device="cuda")
        x32 = np.ascontiguousarray(xs[0][:32].cpu().numpy())
        c.lib.nvfp4_qdq(xs[0].data_ptr(), L.F32, 32, Kw, rd.data_ptr(), None, sr, 0, 3, od.data_ptr(), L.BF16,
                        None, None, c.stream)
        wo = c.oracle.qdq(x32, stochastic=bool(sr), residual=r0, seed=0, step=3)[0]
        check_rows(np, od.cpu().view(torch.int16).numpy().view(np.uint16), wo, "ef qdq out")
        check_rows(np, rd.cpu().numpy(), r0, "ef residual")

    return dict(step=step, check=check, bytes=Mw * Kw * 14, kernel="k_quant1x16",
                note="fp32 x in + fp32 residual in/out + bf16 out")


class Weight2D:
    """The 7168x18432 bf16 weight, its per-tensor amax and output buffers,
    shared by the 16x16 and row + column workloads."""

    def __init__(self, c):
        np, torch, L = c.np, c.torch, c.L
        self.M, self.K = M, K = c.workloads.WEIGHT_2D_SHAPE
        self.wb = c.workloads.weight_2d_input()
        self.wd = [dev_bf16(torch, np, self.wb) for _ in range(2)]
        self.ga = torch.empty(1, dtype=torch.float32, device="cuda")
        self.wsz = c.lib.nvfp4_amax_workspace_bytes(M, K)
        self.ws = torch.empty(self.wsz, dtype=torch.uint8, device="cuda")
        self.pr = [torch.empty((M, K // 2), dtype=torch.uint8, device="cuda") for _ in range(2)]
        self.pc = [torch.empty((K, M // 2), dtype=torch.uint8, device="cuda") for _ in range(2)]
        self.ts = [torch.empty((M // 16, K // 16), dtype=torch.uint8, device="cuda") for _ in range(2)]
        self.srow = torch.empty((M, K // 16), dtype=torch.uint8, device="cuda")
        self.scol = torch.empty((K, M // 16), dtype=torch.uint8, device="cuda")
        _call(c, "nvfp4_amax", c.lib.nvfp4_amax(self.wd[0].data_ptr(), L.BF16, M, K, None, L.SCALE_TENSOR,
                                                 self.ga.data_ptr(), self.ws.data_ptr(), self.wsz, c.stream))
        self.A = c.oracle.amax(self.wb)
        check_rows(np, self.ga.cpu().numpy(), np.array([self.A], np.float32), "2d amax")


def build_2d(c, W, kind):
    np, L = c.np, c.L
    M, K = W.M, W.K
    n2 = M * K
    rows = slice(0, 64)
    if kind in ("sr", "truncfree"):
        tf = int(kind == "truncfree")

        def step(i):
            j = i % 2
            _call(c, "nvfp4_quantize_2d", c.lib.nvfp4_quantize_2d(
                W.wd[j].data_ptr(), L.BF16, M, K, W.ga.data_ptr(), 1, 0, 0, tf, W.pr[j].data_ptr(),
                W.pc[j].data_ptr(), W.ts[j].data_ptr(), c.stream))

        def check():
            step(1)
            wr, wc, wt = c.oracle.quantize_2d(W.wb[rows], stochastic=True, global_amax=W.A, truncation_free=bool(tf))
            check_rows(np, W.pr[1].cpu().numpy()[rows], wr, "2d rowwise")
            check_rows(np, W.ts[1].cpu().numpy()[:4], wt, "2d tiles")
            check_rows(np, W.pc[1].cpu().numpy()[:, :32], wc, "2d columnwise")

        return dict(step=step, check=check, bytes=n2 * 2 + n2 // 2 + n2 // 2 + n2 // 256, kernel="k_quant2d",
                    note="fused pass: bf16 in, rowwise + columnwise codes, tile scales" +
                         (" (tile scale rounded up)" if tf else ""))
    if kind == "4over6":
        def step(i):
            j = i % 2
            _call(c, "nvfp4_quantize_4over6_2d", c.lib.nvfp4_quantize_4over6_2d(
                W.wd[j].data_ptr(), L.BF16, M, K, W.ga.data_ptr(), L.MAE, 256.0, W.pr[j].data_ptr(),
                W.pc[j].data_ptr(), W.ts[j].data_ptr(), c.stream))

        def check():
            step(1)
            wr, wc, wt = c.oracle.quantize_4over6_2d(W.wb[rows], W.A, err_mode="mae", bound=256.0)
            check_rows(np, W.pr[1].cpu().numpy()[rows], wr, "4over6 2d rowwise")
            check_rows(np, W.ts[1].cpu().numpy()[:4], wt, "4over6 2d tiles")

        return dict(step=step, check=check, bytes=n2 * 2 + n2 // 2 + n2 // 2 + n2 // 256, kernel="k_4over6_2d",
                    note="four-over-six on 16x16 tiles, rowwise + columnwise codes, tile scales")
    if kind in ("rowcol", "rowcol4over6"):
        fos = int(kind == "rowcol4over6")
        bnd = 256.0 if fos else 448.0

        def step(i):
            j = i % 2
            _call(c, "nvfp4_quantize_rowcol", c.lib.nvfp4_quantize_rowcol(
                W.wd[j].data_ptr(), L.BF16, M, K, W.ga.data_ptr(), fos, L.MAE, bnd, W.pr[j].data_ptr(),
                W.srow.data_ptr(), W.pc[j].data_ptr(), W.scol.data_ptr(), c.stream))

        def check():
            step(1)
            wpr, wsr, wpc, wsc = c.oracle.quantize_rowcol(W.wb[rows], W.A, four_over_six=bool(fos), bound=bnd)
            check_rows(np, W.pr[1].cpu().numpy()[rows], wpr, "rowcol rowwise")
            check_rows(np, W.scol.cpu().numpy()[:, :4], wsc, "rowcol col scales")

        return dict(step=step, check=check, bytes=n2 * 2 + n2 + n2 // 8, kernel="k_rowcol",
                    note="bf16 in, rowwise + columnwise codes and 1x16 scales")
    if kind == "amax":
        def step(i):
            _call(c, "nvfp4_amax", c.lib.nvfp4_amax(W.wd[i % 2].data_ptr(), L.BF16, M, K, None, L.SCALE_TENSOR,
                                                     W.ga.data_ptr(), W.ws.data_ptr(), W.wsz, c.stream))

        return dict(step=step, check=lambda: None, bytes=n2 * 2, kernel="k_amax_partial + k_amax_final",
                    note="per-tensor amax, two passes")

    def step(i):  # amax then 2D on the same tensor
        j = i % 2
        c.lib.nvfp4_amax(W.wd[j].data_ptr(), L.BF16, M, K, None, L.SCALE_TENSOR, W.ga.data_ptr(),
                         W.ws.data_ptr(), W.wsz, c.stream)
        c.lib.nvfp4_quantize_2d(W.wd[j].data_ptr(), L.BF16, M, K, W.ga.data_ptr(), 1, 0, 0, 0, W.pr[j].data_ptr(),
                                W.pc[j].data_ptr(), W.ts[j].data_ptr(), c.stream)

    return dict(step=step, check=lambda: None, bytes=n2 * 2 * 2 + n2 + n2 // 256, kernel="amax + k_quant2d",
                note="end to end: the amax pass then the 2D + SR pass on the same tensor, back to back")


def build_heavy(c):
    np, torch, L = c.np, c.torch, c.L
    Mh, Kh = c.workloads.HEAVY_SHAPE
    hb = c.workloads.heavy_input()
    hd = dev_bf16(torch, np, hb)
    r0 = torch.zeros((Mh, Kh), dtype=torch.float32, device="cuda")
    ho = torch.empty((Mh, Kh), dtype=torch.bfloat16, device="cuda")
    seed, stp = c.workloads.HEAVY_SEED, c.workloads.HEAVY_STEP

    def step(i):
        _call(c, "nvfp4_qdq", c.lib.nvfp4_qdq(hd.data_ptr(), L.BF16, Mh, Kh, r0.data_ptr(), None, 1, seed, stp,
                                               ho.data_ptr(), L.BF16, None, None, c.stream))

    def check():
        step(0)
        rr = np.zeros((64, Kh), np.float32)
        wo = c.oracle.qdq(hb[:64], stochastic=True, residual=rr, seed=seed, step=stp)[0]
        check_rows(np, ho[:64].cpu().view(torch.int16).numpy().view(np.uint16), wo, "heavy qdq out")
        check_rows(np, r0[:64].cpu().numpy(), rr, "heavy residual")

    return dict(step=step, check=check, bytes=Mh * Kh * 12, kernel="k_quant1x16",
                note="bf16 in, fp32 residual in/out, bf16 out")


# The four-over-six pull request's Bench table (bf16 input, MAE, bound 256,
# bytes in + out): shape -> CuTe DSL kernel microseconds on GB200 for the
# 1x16 per-tensor, 1x16 row-scaled and 16x16 rows (other hardware: context).
PAGES_BENCH_GB200_US = {
    (8192, 2048): (127.0, 127.0, 131.1),
    (8192, 7168): (409.6, 413.7, 423.9),
    (32768, 2048): (464.9, 470.0, 481.3),
    (32768, 7168): (1572.2, 1592.3, 1631.2),
    (131072, 2048): (1793.1, 1815.6, 1860.6),
    (131072, 7168): (6222.9, 6300.8, 6460.5),
}


def pages_bench(c, warmup, steps, warmup_ms):
    """The pages' benchmark shapes on this GPU: four-over-six MAE, bound 256,
    bf16 rows N(0,1) with a log-uniform row std in [1e-2, 1e2] drawn on the
    device (seeded).  Per shape: 1x16 with the per-tensor amax given, 1x16
    row-scaled with the row amax computed in the pass, and 16x16 per tensor
    (rowwise output, as the table).  Each variant is checked bit for bit
    against the oracle on sampled rows (whole 16-row strips for 16x16), then
    timed like the extras; buffer sets rotate until the footprint passes
    600 MB."""
    np, torch, L = c.np, c.torch, c.L
    out = {}
    for si, ((M, K), gb200) in enumerate(PAGES_BENCH_GB200_US.items()):
        g = torch.Generator(device="cuda")
        g.manual_seed(1000 + si)
        std = torch.pow(10.0, 4.0 * torch.rand(M, 1, generator=g, device="cuda") - 2.0)
        x0 = (torch.randn(M, K, generator=g, device="cuda") * std).to(torch.bfloat16)
        del std
        nb = M * K * 2 + M * K // 2 + M * K // 16
        nsets = max(1, min(16, -(-600_000_000 // nb)))
        xs = [x0] + [x0.clone() for _ in range(nsets - 1)]
        pk = [torch.empty((M, K // 2), dtype=torch.uint8, device="cuda") for _ in range(nsets)]
        sc = [torch.empty((M, K // 16), dtype=torch.uint8, device="cuda") for _ in range(nsets)]
        ts = torch.empty((M // 16, K // 16), dtype=torch.uint8, device="cuda")
        ra = [torch.empty(M, dtype=torch.float32, device="cuda") for _ in range(nsets)]
        ga = torch.empty(1, dtype=torch.float32, device="cuda")
        wsz = c.lib.nvfp4_amax_workspace_bytes(M, K)
        ws = torch.empty(max(wsz, 1), dtype=torch.uint8, device="cuda")
        _call(c, "nvfp4_amax", c.lib.nvfp4_amax(x0.data_ptr(), L.BF16, M, K, None, L.SCALE_TENSOR, ga.data_ptr(),
                                                 ws.data_ptr(), wsz, c.stream))
        A = np.float32(ga.cpu().numpy()[0])
        assert A == np.float32(x0.abs().max().float().item()), "per-tensor amax"
        rows = np.unique(np.concatenate([np.arange(16), np.arange(M - 16, M), [M // 2]]))
        strips = np.concatenate([np.arange(16), np.arange(M - 16, M)])
        host = lambda r: x0[torch.from_numpy(r).cuda()].cpu().view(torch.int16).numpy().view(np.uint16)
        xr, xt = host(rows), host(strips)
        res = {}
        for vi, name in enumerate(("1x16", "1x16_row_scaled", "16x16")):
            if name == "16x16":
                def step(i):
                    j = i % nsets
                    _call(c, "nvfp4_quantize_4over6_2d", c.lib.nvfp4_quantize_4over6_2d(
                        xs[j].data_ptr(), L.BF16, M, K, ga.data_ptr(), L.MAE, 256.0, pk[j].data_ptr(), None,
                        ts.data_ptr(), c.stream))
                step(0)
                torch.cuda.synchronize()
                wp, wt = c.oracle.quantize_4over6(xt, A, err_mode="mae", bound=256.0, block="16x16")
                check_rows(np, pk[0].cpu().numpy()[strips], wp, f"pages {M}x{K} 16x16 codes")
                check_rows(np, ts.cpu().numpy()[[0, M // 16 - 1]], wt, f"pages {M}x{K} 16x16 tile scales")
                nbytes = M * K * 2 + M * K // 2 + M * K // 256
            else:
                row = name != "1x16"
                def step(i, row=row):
                    j = i % nsets
                    a = ra[j].data_ptr() if row else ga.data_ptr()
                    _call(c, "nvfp4_quantize_4over6", c.lib.nvfp4_quantize_4over6(
                        xs[j].data_ptr(), L.BF16, M, K, a, L.SCALE_ROW if row else L.SCALE_TENSOR, 0 if row else 1, L.MAE,
                        256.0, pk[j].data_ptr(), sc[j].data_ptr(), c.stream))
                step(0)
                torch.cuda.synchronize()
                Ar = c.oracle.amax(xr, mode="row") if row else A
                wp, wsc = c.oracle.quantize_4over6(xr, Ar, err_mode="mae", bound=256.0)
                if row:
                    check_rows(np, ra[0].cpu().numpy()[rows], Ar, f"pages {M}x{K} row amax")
                check_rows(np, pk[0].cpu().numpy()[rows], wp, f"pages {M}x{K} {name} codes")
                check_rows(np, sc[0].cpu().numpy()[rows], wsc, f"pages {M}x{K} {name} scales")
                nbytes = nb
            warm(torch, step, warmup, warmup_ms)
            ms = time_ms(torch, step, 0, steps)
            res[name] = {"us": round(ms * 1e3, 3), "GB/s": round(nbytes / (ms * 1e-3) / 1e9, 2),
                         "frac_hbm": round(nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                         "gb200_us": gb200[vi]}
        out[f"{M}x{K}"] = res
        del xs, pk, sc, ts, ra, x0, ws
        torch.cuda.empty_cache()
    return out


def builders(c, W):
    """Workload name -> builder (the extra workloads and the metric's MSE form)."""
    w2 = lambda kind: (lambda: build_2d(c, W(), kind))
    return {
        "act_rows_8192x7168_4over6_mse": lambda: build_metric(c, "mse"),
        "small_256x256_fp32_quantize_rtn": lambda: build_small(c, "rtn"),
        "small_256x256_fp32_quantize_sr": lambda: build_small(c, "sr"),
        "small_256x256_dequantize_bf16": lambda: build_small(c, "dequantize"),
        "ef_weight_4096x4096_qdq_step_rtn_ef": lambda: build_ef(c, 0),
        "ef_weight_4096x4096_qdq_step_sr_ef": lambda: build_ef(c, 1),
        "weight_2d_7168x18432_quantize_2d_sr": w2("sr"),
        "weight_2d_7168x18432_quantize_2d_sr_truncation_free": w2("truncfree"),
        "weight_2d_7168x18432_4over6_16x16_mae": w2("4over6"),
        "weight_2d_7168x18432_rowcol_1x16_standard": w2("rowcol"),
        "weight_2d_7168x18432_rowcol_1x16_4over6_mae": w2("rowcol4over6"),
        "weight_2d_7168x18432_amax": w2("amax"),
        "weight_2d_7168x18432_amax_plus_2d": w2("pair"),
        "heavy_16384x8192_qdq_sr_ef": lambda: build_heavy(c),
    }


def roofline(bytes_, ms, workload, kernel):
    gbs = bytes_ / (ms * 1e-3) / 1e9
    return {"bound": "hbm", "achieved": round(gbs, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": read_traffic(workload) if workload in TRAFFIC else None,
            "kernel": kernel, "algorithmic_bytes_per_launch": bytes_, "avg_launch_us": round(ms * 1e3, 3)}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--warmup-ms", type=float, default=30.0,
                    help="untimed warmup also lasts at least this much GPU time (0: exactly --warmup steps)")
    ap.add_argument("--err", choices=["mae", "mse"], default="mae")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU-oracle baseline")
    ap.add_argument("--no-extra", action="store_true", help="time only the metric workload")
    ap.add_argument("--no-pages", action="store_true", help="skip the pages' benchmark shapes")
    ap.add_argument("--only", default=None, help="run only this workload's steps (for profiling)")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--copy-calib", action="store_true",
                    help="only run a plain 1 GiB device copy (counter calibration) and exit")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py: the library runs on one GPU; --gpus {args.gpus} is not supported "
              "(the path would shard by rows, its only exchange a 4-byte max all-reduce of the "
              "per-tensor amax, with the generator keyed by global element indices).", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    from fp4_block_quantization_nvfp4_amd import _lib as L
    import workloads

    torch.cuda.set_device(0)
    if args.copy_calib:
        a = torch.empty(1 << 28, dtype=torch.float32, device="cuda")
        b = torch.empty_like(a)
        a.fill_(1.0)
        for _ in range(5):
            b.copy_(a)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calib_bytes_each_way": a.numel() * 4, "launches": 5}))
        return

    import oracle

    lib = L.lib()
    stream = torch.cuda.current_stream().cuda_stream
    c = Ctx(np, torch, L, lib, stream, workloads, oracle)
    w2d = []

    def W():
        if not w2d:
            w2d.append(Weight2D(c))
        return w2d[0]

    if args.only:
        b = build_metric(c, args.err) if args.only == METRIC else builders(c, W)[args.only]()
        b["check"]()
        ms = time_ms(torch, b["step"], args.warmup, args.steps)
        print(json.dumps({"workload": args.only, "us_per_step": round(ms * 1e3, 3), "steps": args.steps,
                          "GB/s": round(b["bytes"] / (ms * 1e-3) / 1e9, 2)}), flush=True)
        return

    m = build_metric(c, args.err)
    m["check"]()  # parity before timing (sampled rows; rows are independent on this path)
    host = {}
    # untimed: at least W steps and at least --warmup-ms of GPU time, so the
    # timed region starts in the steady state (see warm())
    nwarm = warm(torch, m["step"], args.warmup, args.warmup_ms)
    ms = time_ms(torch, m["step"], 0, args.steps, host)
    algo = m["bytes"]
    gbs = algo / (ms * 1e-3) / 1e9
    metric_name = f"act_rows_8192x7168_4over6_{args.err}"
    rl = roofline(algo, ms, metric_name, "k_4over6_rows (row amax computed in-pass)")
    rl.update({"timing": "HIP events on the launch stream around the timed region; one launch of the kernel "
                         "per step, so region time / steps bounds its average duration from above; untimed "
                         f"warmup of at least {args.warmup} steps and {args.warmup_ms:g} ms of GPU time first",
               "host_submit_us_per_launch": round(host["us_per_call"], 3),
               "copy_ceiling_GBs": round(copy_ceiling_gbs(torch), 1)})
    line = {
        "metric": "NVFP4 quantize GB/s (bytes in+out) and % of HBM peak, 8192x7168 bf16",
        "value": round(gbs, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "warmup_steps_run": nwarm,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": "four-over-six NVFP4 1x16 quantize, row-scaled (per-row amax fused), "
                        f"{args.err.upper()}, e4m3 bound 256, 8192x7168 bf16 N(0,1) x per-row "
                        "log-uniform std [1e-2,1e2]",
            "M": workloads.ACT_ROWS_SHAPE[0], "K": workloads.ACT_ROWS_SHAPE[1], "block": "1x16",
            "err_mode": args.err, "bound": 256, "bytes_per_step": algo, "buffer_sets": N_SETS,
            "parity": "bitwise vs CPU oracle on 65 sampled rows (codes, scales, row amax) before timing",
        },
        "pct_of_hbm_peak": round(100.0 * gbs / HBM_PEAK_GBS, 2),
        "roofline": rl,
    }

    if not args.no_extra:
        steps, warmup = max(args.steps // 4, 10), max(args.warmup // 4, 3)
        extra = {}
        for name, build in builders(c, W).items():
            if name == metric_name:
                continue
            b = build()
            b["check"]()
            nw = warm(torch, b["step"], warmup, args.warmup_ms)
            ms_b = time_ms(torch, b["step"], 0, steps)
            r = roofline(b["bytes"], ms_b, name, b["kernel"])
            extra[name] = {"us": r["avg_launch_us"], "GB/s": r["achieved"], "frac_hbm": r["frac"],
                           "bytes": b["bytes"], "traffic": r["traffic"], "steps": steps, "warmup": nw,
                           "note": b["note"]}
            del b
        line["extra"] = extra

    if not args.no_pages:
        line["pages_bench"] = {
            "note": "the four-over-six pull request's Bench shapes: bf16 rows N(0,1) x log-uniform row std "
                    "[1e-2,1e2] (seeded, drawn on the device), MAE, bound 256, checked bit for bit on sampled "
                    "rows first; GB/s = bytes in + out as there; 16x16 rowwise output; gb200_us = the pages' "
                    "CuTe DSL kernel on GB200 (other hardware, context only)",
            "shapes": pages_bench(c, max(args.warmup // 4, 3), max(args.steps // 4, 10), args.warmup_ms)}

    if not args.no_cpu:
        line["cpu_baseline"] = cpu_baseline(np, m["x_bits"], args.err, args.cpu_seconds)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
