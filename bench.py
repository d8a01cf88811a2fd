"""Benchmark: NVFP4 four-over-six quantize throughput on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu] [--no-extra]

Workload (the metric's configuration): row-scaled four-over-six NVFP4
quantize of an 8192x7168 bf16 activation (N(0,1) with a log-uniform per-row
std in [1e-2, 1e2]), MAE selection, e4m3 scale bound 256, per-row global amax
computed in the same kernel.  One step = one pass of that fused kernel
(nvfp4_quantize_4over6) over one input buffer set; four buffer sets rotate so
the 600 MB footprint exceeds the 256 MB Infinity Cache.  GB/s counts
algorithmic bytes in + out: bf16 input + packed e2m1 codes + e4m3 scale bytes
(2.5625 B/element, 150,470,656 B per step), the pages' convention.

Before timing, the GPU output is checked bit for bit against the CPU oracle on
a sample of rows.  The line also carries the dominant kernel's roofline
(bytes / average launch time vs the 8 TB/s HBM peak; HBM traffic from the
committed rocprofv3 counter summary when it matches the current kernel
source) and the CPU oracle timed on a bounded row sample.  Unless --no-extra,
the other quantization workloads are timed too and reported under "extra".
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
KERNEL_SRC = os.path.join(ROOT, "fp4_block_quantization_nvfp4_amd", "csrc", "k_4over6.hip")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_4over6_act_rows_8192x7168.txt")


def src_hash(path=KERNEL_SRC):
    h = hashlib.sha256()
    d = os.path.dirname(path)
    for p in (path, os.path.join(d, "nvfp4_device.hpp"), os.path.join(d, "nvfp4_fos.hpp")):
        h.update(open(p, "rb").read())
    return h.hexdigest()[:16]


def read_traffic(algo_bytes):
    """HBM bytes per launch from the committed counter summary, or None when
    absent or taken on a different kernel source."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    kv = {}
    for line in open(TRAFFIC_FILE):
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            kv[k.strip()] = v.strip()
    if kv.get("kernel_src_sha256_16") != src_hash():
        return None
    try:
        return int(float(kv["hbm_bytes_per_launch"]))
    except (KeyError, ValueError):
        return None


def dev_bf16(torch, np, bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


def time_ms(torch, fn, warmup, steps, host=None):
    """Average ms per call over `steps` calls on torch's current stream
    (the stream every C-ABI call here is issued on), after `warmup` calls.
    If `host` is a dict, host["us_per_call"] receives the host-side time to
    submit one call (the loop without the final synchronization)."""
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


def time_each_ms(torch, fn, warmup, steps, each=None):
    """Average ms of one call measured with a pair of events around each call
    on the launch stream (the kernel's own duration, without the gaps
    between back-to-back launches).  If `each` is a list, it receives every
    call's ms."""
    for i in range(warmup):
        fn(i)
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    for i in range(steps):
        ev[i][0].record()
        fn(i)
        ev[i][1].record()
    torch.cuda.synchronize()
    d = [a.elapsed_time(b) for a, b in ev]
    if each is not None:
        each.extend(d)
    return sum(d) / steps


def percentile(v, q):
    """q-th percentile (0..100) of a list, nearest rank."""
    s = sorted(v)
    return s[min(len(s) - 1, max(0, int(round(q / 100.0 * (len(s) - 1)))))]


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


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--err", choices=["mae", "mse"], default="mae")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU-oracle baseline")
    ap.add_argument("--no-extra", action="store_true", help="time only the metric workload")
    ap.add_argument("--cpu-rows", type=int, default=8192)
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--copy-calib", action="store_true",
                    help="only run a plain 1 GiB device copy (counter calibration) and exit")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py: this build runs on one GPU only; --gpus {args.gpus} is not supported "
              "(the path shards by rows with no exchange except a 4-byte amax max-reduce; "
              "see the sharding note in the design document).", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import fp4_block_quantization_nvfp4_amd as nv
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

    lib = L.lib()
    stream = torch.cuda.current_stream().cuda_stream
    M, K = workloads.ACT_ROWS_SHAPE
    err = L.MAE if args.err == "mae" else L.MSE
    bound = 256.0
    x_bits = workloads.act_rows_input()
    xs = [dev_bf16(torch, np, x_bits) for _ in range(N_SETS)]
    packed = [torch.empty((M, K // 2), dtype=torch.uint8, device="cuda") for _ in range(N_SETS)]
    scales = [torch.empty((M, K // 16), dtype=torch.uint8, device="cuda") for _ in range(N_SETS)]
    amaxes = [torch.empty(M, dtype=torch.float32, device="cuda") for _ in range(N_SETS)]

    fn = lib.nvfp4_quantize_4over6
    call_args = [(xs[j].data_ptr(), L.BF16, M, K, amaxes[j].data_ptr(), L.SCALE_ROW, 0, err, bound,
                  packed[j].data_ptr(), scales[j].data_ptr(), stream) for j in range(N_SETS)]

    def step(i):
        status = fn(*call_args[i % N_SETS])
        if status:
            L.check(status, "nvfp4_quantize_4over6")

    # parity before timing (sampled rows; rows are independent on this path)
    import oracle

    step(0)
    torch.cuda.synchronize()
    rows = np.unique(np.concatenate([np.arange(16), np.random.default_rng(0).integers(0, M, 48), [M - 1]]))
    A = oracle.amax(x_bits[rows], mode="row")
    wp, ws = oracle.quantize_4over6(x_bits[rows], A, err_mode=args.err, bound=bound)
    check_rows(np, amaxes[0].cpu().numpy()[rows], A, "row amax")
    check_rows(np, packed[0].cpu().numpy()[rows], wp, "codes")
    check_rows(np, scales[0].cpu().numpy()[rows], ws, "scales")

    host = {}
    ms = time_ms(torch, step, args.warmup, args.steps, host)
    each = []
    ms_kernel = time_each_ms(torch, step, args.warmup, args.steps, each)
    algo = M * K * 2 + M * K // 2 + M * K // 16  # 150,470,656 B
    gbs = algo / (ms * 1e-3) / 1e9
    kgbs = algo / (ms_kernel * 1e-3) / 1e9
    traffic = read_traffic(algo)
    line = {
        "metric": "NVFP4 quantize GB/s (bytes in+out) and % of HBM peak, 8192x7168 bf16",
        "value": round(gbs, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
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
            "M": M, "K": K, "block": "1x16", "err_mode": args.err, "bound": 256,
            "bytes_per_step": algo, "buffer_sets": N_SETS,
            "parity": "bitwise vs CPU oracle on 65 sampled rows (codes, scales, row amax)",
        },
        "pct_of_hbm_peak": round(100.0 * gbs / HBM_PEAK_GBS, 2),
        "roofline": {
            "bound": "hbm",
            "achieved": round(kgbs, 2),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(kgbs / HBM_PEAK_GBS, 4),
            "traffic": traffic,
            "kernel": "k_4over6 (row amax computed in-pass)",
            "algorithmic_bytes_per_launch": algo,
            "avg_launch_us": round(ms_kernel * 1e3, 3),
            "timing": "events around each launch on the launch stream; value uses the whole timed region",
            "host_submit_us_per_launch": round(host["us_per_call"], 3),
            "launch_us_p10_median_p90": [round(percentile(each, q) * 1e3, 3) for q in (10, 50, 90)],
            "copy_ceiling_GBs": round(copy_ceiling_gbs(torch), 1),
        },
    }

    if not args.no_extra:
        line["extra"] = extra_workloads(np, torch, nv, L, lib, stream, workloads, oracle,
                                        max(args.steps // 4, 10), max(args.warmup // 4, 3))
        # the same workload with the other error measure (the configuration
        # names both), parity-checked on the same sampled rows
        other = "mse" if args.err == "mae" else "mae"
        err_o = L.MSE if other == "mse" else L.MAE
        args_o = [(a[:7] + (err_o,) + a[8:]) for a in call_args]

        def step_o(i):
            status = fn(*args_o[i % N_SETS])
            if status:
                L.check(status, "nvfp4_quantize_4over6")

        step_o(0)
        torch.cuda.synchronize()
        wp, ws = oracle.quantize_4over6(x_bits[rows], A, err_mode=other, bound=bound)
        check_rows(np, packed[0].cpu().numpy()[rows], wp, f"codes ({other})")
        check_rows(np, scales[0].cpu().numpy()[rows], ws, f"scales ({other})")
        ms_o = time_ms(torch, step_o, args.warmup, args.steps)
        ms_ok = time_each_ms(torch, step_o, args.warmup, args.steps)
        line["extra"][f"act_rows_8192x7168_4over6_{other}"] = {
            "us": round(ms_o * 1e3, 3), "GB/s": round(algo / (ms_o * 1e-3) / 1e9, 2),
            "frac_hbm": round(algo / (ms_o * 1e-3) / 1e9 / HBM_PEAK_GBS, 4), "bytes": algo,
            "kernel_us": round(ms_ok * 1e3, 3),
            "note": f"the metric workload with err_mode {other}; per-row amax computed in-pass"}

    if not args.no_cpu:
        # the oracle over whole rows of the same tensor, repeated until about
        # args.cpu_seconds of CPU time (one process, one core)
        R = min(args.cpu_rows, M)
        xr = x_bits[:R]
        n_pass, dt = 0, 0.0
        while dt < args.cpu_seconds and n_pass < 8:
            t = time.perf_counter()
            Ar = oracle.amax(xr, mode="row")
            oracle.quantize_4over6(xr, Ar, err_mode=args.err, bound=bound)
            dt += time.perf_counter() - t
            n_pass += 1
        n = R * K * n_pass
        line["cpu_baseline"] = {
            "value": round(n * 2.5625 / dt / 1e9, 5),
            "unit": "GB/s",
            "cores": 1,
            "kind": "oracle",
            "sample": f"{n_pass} pass(es) over {R} of {M} rows ({R * K} elements each), per-row amax + "
                      f"four-over-six {args.err.upper()} bound 256, numpy float32 single process; "
                      f"{dt:.2f} s, {n / dt / 1e6:.3f} M elements/s",
        }
    print(json.dumps(line), flush=True)


def extra_workloads(np, torch, nv, L, lib, stream, workloads, oracle, steps, warmup):
    """Time the other quantization workloads (GPU only), each parity-checked
    on a sample first; time per call over the whole timed region (kernel
    durations of the same runs are in the committed all-workload kernel
    trace).  Returns {name: {...}}."""
    out = {}

    def rec(name, ms, algo, note):
        gbs = algo / (ms * 1e-3) / 1e9
        out[name] = {"us": round(ms * 1e3, 3), "GB/s": round(gbs, 2),
                     "frac_hbm": round(gbs / HBM_PEAK_GBS, 4), "bytes": algo, "note": note}

    # 256x256 fp32 quantize (RTN and SR) and dequantize: launch-bound
    x = workloads.small_input()
    xd = torch.from_numpy(x).cuda()
    p = torch.empty((256, 128), dtype=torch.uint8, device="cuda")
    s = torch.empty((256, 16), dtype=torch.uint8, device="cuda")
    o = torch.empty((256, 256), dtype=torch.bfloat16, device="cuda")
    for sr in (0, 1):
        ms = time_ms(torch, lambda i: lib.nvfp4_quantize(xd.data_ptr(), L.F32, 256, 256, None, None, sr, 0, 0,
                                                          p.data_ptr(), s.data_ptr(), stream), warmup, steps)
        wp, ws = oracle.quantize(x, stochastic=bool(sr))
        check_rows(np, p.cpu().numpy(), wp, "small codes")
        rec(f"small_256x256_fp32_quantize_{'sr' if sr else 'rtn'}", ms, 256 * 256 * 4 + 256 * 128 + 256 * 16,
            "launch-bound")
    ms = time_ms(torch, lambda i: lib.nvfp4_dequantize(p.data_ptr(), s.data_ptr(), 256, 256, 0, None, 0, 448.0,
                                                        o.data_ptr(), L.BF16, stream), warmup, steps)
    rec("small_256x256_dequantize_bf16", ms, 256 * 128 + 256 * 16 + 256 * 256 * 2, "launch-bound")

    # 4096x4096 stored weight, one error-feedback qdq step (fp32 x in, residual in/out, bf16 out)
    Mw, Kw = workloads.EF_SHAPE
    w = torch.from_numpy(workloads.ef_weight0().view(np.int16)).view(torch.bfloat16).cuda().float()
    xs = [w.clone() for _ in range(N_SETS)]
    rs = [torch.zeros_like(w) for _ in range(N_SETS)]
    outs = [torch.empty((Mw, Kw), dtype=torch.bfloat16, device="cuda") for _ in range(N_SETS)]
    for sr in (0, 1):
        ms = time_ms(torch, lambda i: lib.nvfp4_qdq(xs[i % N_SETS].data_ptr(), L.F32, Mw, Kw, rs[i % N_SETS].data_ptr(),
                                                     None, sr, 0, i, outs[i % N_SETS].data_ptr(), L.BF16, None, None,
                                                     stream), warmup, steps)
        rec(f"ef_weight_4096x4096_qdq_step_{'sr' if sr else 'rtn'}_ef", ms, Mw * Kw * 14,
            "fp32 x in + fp32 residual in/out + bf16 out")

    # 7168x18432 bf16 2D 16x16 + SR, per-tensor amax
    Mt, Kt = workloads.WEIGHT_2D_SHAPE
    wb = workloads.weight_2d_input()
    wd = [torch.from_numpy(wb.view(np.int16)).view(torch.bfloat16).cuda() for _ in range(2)]
    ga = torch.empty(1, dtype=torch.float32, device="cuda")
    wsz = lib.nvfp4_amax_workspace_bytes(Mt, Kt)
    wsb = torch.empty(wsz, dtype=torch.uint8, device="cuda")
    pr = [torch.empty((Mt, Kt // 2), dtype=torch.uint8, device="cuda") for _ in range(2)]
    pc = [torch.empty((Kt, Mt // 2), dtype=torch.uint8, device="cuda") for _ in range(2)]
    ts = [torch.empty((Mt // 16, Kt // 16), dtype=torch.uint8, device="cuda") for _ in range(2)]
    lib.nvfp4_amax(wd[0].data_ptr(), L.BF16, Mt, Kt, None, L.SCALE_TENSOR, ga.data_ptr(), wsb.data_ptr(), wsz, stream)
    ms_amax = time_ms(torch, lambda i: lib.nvfp4_amax(wd[i % 2].data_ptr(), L.BF16, Mt, Kt, None, L.SCALE_TENSOR,
                                                       ga.data_ptr(), wsb.data_ptr(), wsz, stream), warmup, steps)
    ms_2d = time_ms(torch, lambda i: lib.nvfp4_quantize_2d(wd[i % 2].data_ptr(), L.BF16, Mt, Kt, ga.data_ptr(), 1, 0, 0, 0,
                                                            pr[i % 2].data_ptr(), pc[i % 2].data_ptr(),
                                                            ts[i % 2].data_ptr(), stream), warmup, steps)
    A = oracle.amax(wb)
    check_rows(np, ga.cpu().numpy(), np.array([A], np.float32), "2d amax")
    rows = slice(0, 64)
    wr, wc, wt = oracle.quantize_2d(wb[rows], stochastic=True, global_amax=A)
    check_rows(np, pr[1].cpu().numpy()[rows], wr, "2d rowwise")
    check_rows(np, ts[1].cpu().numpy()[:4], wt, "2d tiles")
    check_rows(np, pc[1].cpu().numpy()[:, :32], wc, "2d columnwise")
    n2 = Mt * Kt
    rec("weight_2d_7168x18432_quantize_2d_sr", ms_2d, n2 * 2 + n2 // 2 + n2 // 2 + n2 // 256,
        "fused pass: bf16 in, rowwise + columnwise codes, tile scales")
    ms_tf = time_ms(torch, lambda i: lib.nvfp4_quantize_2d(wd[i % 2].data_ptr(), L.BF16, Mt, Kt, ga.data_ptr(), 1, 0, 0, 1,
                                                            pr[i % 2].data_ptr(), pc[i % 2].data_ptr(),
                                                            ts[i % 2].data_ptr(), stream), warmup, steps)
    rec("weight_2d_7168x18432_quantize_2d_sr_truncation_free", ms_tf, n2 * 2 + n2 // 2 + n2 // 2 + n2 // 256,
        "as above, tile scale rounded up")
    ms_46 = time_ms(torch, lambda i: lib.nvfp4_quantize_4over6_2d(wd[i % 2].data_ptr(), L.BF16, Mt, Kt, ga.data_ptr(),
                                                                   L.MAE, 256.0, pr[i % 2].data_ptr(),
                                                                   pc[i % 2].data_ptr(), ts[i % 2].data_ptr(),
                                                                   stream), warmup, steps)
    wr, wc, wt = oracle.quantize_4over6_2d(wb[rows], A, err_mode="mae", bound=256.0)
    check_rows(np, pr[1].cpu().numpy()[rows], wr, "4over6 2d rowwise")
    check_rows(np, ts[1].cpu().numpy()[:4], wt, "4over6 2d tiles")
    rec("weight_2d_7168x18432_4over6_16x16_mae", ms_46, n2 * 2 + n2 // 2 + n2 // 2 + n2 // 256,
        "four-over-six on 16x16 tiles, rowwise + columnwise codes, tile scales")
    srow = torch.empty((Mt, Kt // 16), dtype=torch.uint8, device="cuda")
    scol = torch.empty((Kt, Mt // 16), dtype=torch.uint8, device="cuda")
    for fos in (0, 1):
        bnd = 256.0 if fos else 448.0
        ms_rc = time_ms(torch, lambda i: lib.nvfp4_quantize_rowcol(wd[i % 2].data_ptr(), L.BF16, Mt, Kt, ga.data_ptr(),
                                                                    fos, L.MAE, bnd, pr[i % 2].data_ptr(),
                                                                    srow.data_ptr(), pc[i % 2].data_ptr(),
                                                                    scol.data_ptr(), stream), warmup, steps)
        wpr, wsr, wpc, wsc = oracle.quantize_rowcol(wb[rows], A, four_over_six=bool(fos), bound=bnd)
        check_rows(np, pr[1].cpu().numpy()[rows], wpr, "rowcol rowwise")
        check_rows(np, scol.cpu().numpy()[:, :4], wsc, "rowcol col scales")
        rec(f"weight_2d_7168x18432_rowcol_1x16_{'4over6_mae' if fos else 'standard'}", ms_rc,
            n2 * 2 + n2 + n2 // 8, "bf16 in, rowwise + columnwise codes and 1x16 scales")
    rec("weight_2d_7168x18432_amax", ms_amax, n2 * 2, "per-tensor amax, two passes")
    def amax_then_2d(i):
        j = i % 2
        lib.nvfp4_amax(wd[j].data_ptr(), L.BF16, Mt, Kt, None, L.SCALE_TENSOR, ga.data_ptr(), wsb.data_ptr(),
                       wsz, stream)
        lib.nvfp4_quantize_2d(wd[j].data_ptr(), L.BF16, Mt, Kt, ga.data_ptr(), 1, 0, 0, 0, pr[j].data_ptr(),
                              pc[j].data_ptr(), ts[j].data_ptr(), stream)

    ms_pair = time_ms(torch, amax_then_2d, warmup, steps)
    rec("weight_2d_7168x18432_amax_plus_2d", ms_pair, n2 * 2 * 2 + n2 + n2 // 256,
        "end to end: the amax pass then the 2D + SR pass on the same tensor, back to back")
    del wd, pr, pc, ts

    # 16384x8192 bf16 heavy-tailed qdq with SR + EF (residual in place), seed 7 step 123
    Mh, Kh = workloads.HEAVY_SHAPE
    hb = workloads.heavy_input()
    hd = torch.from_numpy(hb.view(np.int16)).view(torch.bfloat16).cuda()
    r0 = torch.zeros((Mh, Kh), dtype=torch.float32, device="cuda")
    ho = torch.empty((Mh, Kh), dtype=torch.bfloat16, device="cuda")
    lib.nvfp4_qdq(hd.data_ptr(), L.BF16, Mh, Kh, r0.data_ptr(), None, 1, 7, 123, ho.data_ptr(), L.BF16, None, None,
                  stream)
    rr = np.zeros((64, Kh), np.float32)
    wo = oracle.qdq(hb[:64], stochastic=True, residual=rr, seed=7, step=123)[0]
    check_rows(np, ho[:64].cpu().view(torch.int16).numpy().view(np.uint16), wo, "heavy qdq out")
    check_rows(np, r0[:64].cpu().numpy(), rr, "heavy residual")
    ms = time_ms(torch, lambda i: lib.nvfp4_qdq(hd.data_ptr(), L.BF16, Mh, Kh, r0.data_ptr(), None, 1, 7, 123,
                                                 ho.data_ptr(), L.BF16, None, None, stream), warmup, steps)
    rec("heavy_16384x8192_qdq_sr_ef", ms, Mh * Kh * 12, "bf16 in, fp32 residual in/out, bf16 out")
    return out


if __name__ == "__main__":
    main()
