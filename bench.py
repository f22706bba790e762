"""Benchmark of the MXNorm forward hot path on one MI355X.

A step is one mxnorm_fwd call (p = 2, E4M3 elements, bf16 gain) over the
16384 x 4096 bf16 activation matrix (Llama-3 8B hidden size, 4 x 4096 tokens,
per-row log-normal scale times outlier-Gaussian channels).  Inputs are
synthetic and resident in HBM before timing starts; R distinct input/output
buffer sets are rotated so that the 256 MB Infinity Cache cannot serve a step
from the previous one.  Before the W warm-up steps the same calls run for a
fixed 0.1 s of GPU time, which brings the GPU from idle to its steady clocks
(it needs ~30 ms of back-to-back work); then the K steps, captured as calls
through the C ABI in one HIP graph, are replayed once on the current stream:
one HIP event pair on that stream brackets the replay, and the wall clock
between two synchronisations.  (A graph launch is one host call: K direct
calls from Python, in `extras`, carry the interpreter's jitter, which at the
short K = 20 measured 33.7-37.8 us per step against 33.5 us replayed.)

Printed: one JSON line with the achieved algorithmic HBM throughput (GB/s),
a roofline object for the kernel, the CPU oracle timed on the host as a
reference baseline, and context figures in `extras`.  Context legs are timed
as HIP graphs of many captured calls (the same kernels, without the host's
per-call launch cost, which exceeds the kernel time of the small workloads):
  * the byte-pattern references (libmxq_measure.so) at this shape and at the
    8192 x 2048 workload, and a rows sweep (8192 ... 65536 x 4096) of the
    kernel and the patterns with a least-squares fit t = a + bytes / B;
  * a device copy of the same byte count;
  * the two-pass RMSNorm + MX cast baseline, the straight-through backward
    (beside the backward's byte pattern at this shape), MXNormLinear (the
    MXFP8 matmul), the other workloads and the variants.

`python bench.py --counters NAME` only runs one kernel 20 times and a 256 MiB
device copy (the calibration of the HBM byte counters), for rocprofv3 --pmc;
NAME is one of headline, c2, c4, h16, h32, two_pass, bwd, bwd_no_gain,
bwd_2048x32768, matmul.
"""
import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0            # MI355X HBM3E peak, 8 TB/s
FP8_DENSE_PEAK = 5.0e15          # MI355X dense fp8 matrix peak, FLOP/s
HEADLINE = 3                     # workload number of the headline line
METRIC = "MXNorm fwd HBM GB/s (% of MI355X peak), hidden=4096, 16k rows bf16"
KERNEL_SOURCES = ["mx_quantised_tensor_amd/csrc/mxnorm_kernels.hip",
                  "mx_quantised_tensor_amd/csrc/mx_device.h"]  # the headline kernel's sources
PMC_SUMMARY = os.path.join(ROOT, "profiles", "mxnorm_fwd_16384x4096_e4m3_pmc.txt")
C_P2 = float.fromhex("0x1.c1ed54p+0")  # the library's default c(2, 32)
CLOCK_RAMP_S = 0.1               # GPU time of untimed calls before the warm-up steps
COUNTER_RUNS = ("headline", "c2", "c4", "h16", "h32", "two_pass", "bwd", "bwd_no_gain",
                "bwd_2048x32768", "matmul")


def algorithmic_bytes(rows, hidden, elem, gamma=True, with_rrms=True):
    """Bytes the operation must move: read x (2 B/elem) and gamma (2 B per
    column), write codes (1 or 0.5 B/elem), scales (1 B per 32) and rho
    (4 B per row)."""
    code_bytes = rows * hidden if elem == 0 else rows * hidden // 2
    return (2 * rows * hidden + (2 * hidden if gamma else 0) + code_bytes
            + rows * (hidden // 32) + (4 * rows if with_rrms else 0))


def two_pass_bytes(rows, hidden, elem):
    """RMSNorm pass (read x, gamma; write bf16 y, rstd) + MX cast of y."""
    code_bytes = rows * hidden if elem == 0 else rows * hidden // 2
    return (2 * rows * hidden + 2 * hidden + 2 * rows * hidden + 4 * rows
            + 2 * rows * hidden + code_bytes + rows * (hidden // 32))


def bwd_bytes(rows, hidden, gain=True):
    """Straight-through backward: read x, dy (2 B/elem each) and rho (4 B per
    row), write dx (2 B/elem); with the gain also read gamma and write dgamma
    (fp32).  The dgamma partial rows (workspace) are not counted."""
    return 6 * rows * hidden + 4 * rows + ((2 + 4) * hidden if gain else 0)


def kernel_hash():
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def read_traffic():
    """HBM bytes per launch from the committed rocprofv3 counter summary,
    valid only while the kernel sources are unchanged since it was taken."""
    if not os.path.exists(PMC_SUMMARY):
        return None
    text = open(PMC_SUMMARY).read()
    m_hash = re.search(r"kernel_source_hash:\s*(\w+)", text)
    m_bytes = re.search(r"hbm_bytes_per_launch:\s*([0-9.eE+]+)", text)
    if not m_hash or not m_bytes or m_hash.group(1) != kernel_hash():
        return None
    return float(m_bytes.group(1))


def fit_line(xs, ys):
    """Least-squares t = a + b * bytes: (a, b)."""
    n = len(xs)
    mx, my = sum(xs) / n, sum(ys) / n
    b = sum((x - mx) * (y - my) for x, y in zip(xs, ys)) / sum((x - mx) ** 2 for x in xs)
    return my - b * mx, b


def main():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=1000)
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--buffers", type=int, default=6, help="rotated buffer sets")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--no-extras", action="store_true", help="headline workload only")
    ap.add_argument("--counters", choices=COUNTER_RUNS,
                    help="run one kernel 20 times and a calibration copy (for --pmc)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the MXNorm path is per-row independent and this "
              "build runs on a single MI355X; --gpus %d is not supported." % args.gpus,
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch
    import mx_quantised_tensor_amd as mxq
    from mx_quantised_tensor_amd import measure
    from mx_quantised_tensor_amd import workloads as W

    assert torch.cuda.is_available(), "bench.py needs a ROCm GPU"
    L = mxq.lib()
    M = measure.lib()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream()
    sp = stream.cuda_stream

    def dptr(t):
        return None if t is None else t.data_ptr()

    def device_sets(xb, gb, elem, nsets, two_pass=False):
        rows, hidden = xb.shape
        x0 = torch.from_numpy(xb.view(np.int16)).to(dev).view(torch.bfloat16)
        g = torch.from_numpy(gb.view(np.int16)).to(dev).view(torch.bfloat16)
        return g, make_sets(x0, elem, nsets, two_pass)

    def make_sets(x0, elem, nsets, two_pass=False):
        rows, hidden = x0.shape
        sets = []
        for i in range(nsets):
            x = x0 if i == 0 else x0.clone()
            ccols = hidden if elem == 0 else hidden // 2
            s = dict(x=x, codes=torch.empty((rows, ccols), dtype=torch.uint8, device=dev),
                     scales=torch.empty((rows, hidden // 32), dtype=torch.uint8, device=dev),
                     rrms=torch.empty((rows,), dtype=torch.float32, device=dev))
            if two_pass:
                s["y"] = torch.empty((rows, hidden), dtype=torch.bfloat16, device=dev)
            sets.append(s)
        return sets

    # A call is fn(stream) -> status, with the pointers resolved once, so the
    # host keeps ahead of the GPU and the steps run back to back.
    def mxnorm_calls(sets, g, p, elem, had=0, gain=True):
        calls = []
        for s in sets:
            rows, hidden = s["x"].shape
            a = (s["x"].data_ptr(), dptr(g) if gain else None, rows, hidden, p, 0.0)
            o = (s["codes"].data_ptr(), s["scales"].data_ptr(), s["rrms"].data_ptr())
            if had:
                calls.append(lambda st, a=a, o=o: L.mxnorm_hadamard_fwd(*a, had, elem, *o, st))
            else:
                calls.append(lambda st, a=a, o=o: L.mxnorm_fwd(*a, elem, *o, st))
        return calls

    def pattern_calls(sets, layout):
        calls = []
        for s in sets:
            rows, hidden = s["x"].shape
            a = (layout, s["x"].data_ptr(), rows, hidden, s["codes"].data_ptr(),
                 s["scales"].data_ptr(), s["rrms"].data_ptr())
            calls.append(lambda st, a=a: M.mxq_measure_pattern(*a, st))
        return calls

    def two_pass_calls(sets, g, elem):
        calls = []
        for s in sets:
            rows, hidden = s["x"].shape
            a = (s["x"].data_ptr(), g.data_ptr(), rows, hidden, 1e-5, elem, s["y"].data_ptr(),
                 s["codes"].data_ptr(), s["scales"].data_ptr(), s["rrms"].data_ptr())
            calls.append(lambda st, a=a: L.rmsnorm_mxquant_fwd(*a, st))
        return calls

    def run(calls, n, st=sp):
        for i in range(n):
            rc = calls[i % len(calls)](st)
            if rc != 0:
                raise RuntimeError("call failed with status %d" % rc)

    def gpu_time(calls, n):
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        run(calls, n)
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e-3

    def clock_ramp(calls, seconds=CLOCK_RAMP_S):
        """Back-to-back calls for about `seconds` of GPU time (clock ramp)."""
        per = max(gpu_time(calls, 10) / 10, 1e-6)
        run(calls, int(seconds / per) + 1)

    def time_steps(calls, steps, warmup):
        """Clock ramp, `warmup` untimed steps, then the wall time and GPU time
        (one event pair on the launch stream) of `steps` back-to-back calls,
        synchronised on both sides."""
        clock_ramp(calls)
        run(calls, warmup)
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        e0.record(stream)
        run(calls, steps)
        e1.record(stream)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        return wall, e0.elapsed_time(e1) * 1e-3

    def time_steps_graph(calls, steps, warmup):
        """The timed region of the headline: clock ramp and `warmup` untimed
        steps as direct calls, then the `steps` calls captured in one HIP graph
        (capture runs nothing; one untimed replay uploads it), then one timed
        replay: wall time between two synchronisations and GPU time from one
        event pair on the replay stream."""
        clock_ramp(calls)
        run(calls, warmup)
        gr = torch.cuda.CUDAGraph()
        cap = torch.cuda.Stream()
        with torch.cuda.graph(gr, stream=cap):
            run(calls, steps, torch.cuda.current_stream().cuda_stream)
        gr.replay()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        e0.record(stream)
        gr.replay()
        e1.record(stream)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        del gr
        return wall, e0.elapsed_time(e1) * 1e-3

    def graph_us(calls, n=200, seconds=0.06):
        """Mean GPU time per call (us) of n calls captured in one HIP graph,
        replayed back to back for ~`seconds` before one timed replay."""
        g = torch.cuda.CUDAGraph()
        cap = torch.cuda.Stream()
        with torch.cuda.graph(g, stream=cap):
            run(calls, n, torch.cuda.current_stream().cuda_stream)
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        g.replay()
        e1.record(stream)
        torch.cuda.synchronize()
        per = max(e0.elapsed_time(e1) * 1e-3, 1e-6)
        for _ in range(int(seconds / per) + 1):
            g.replay()
        e0.record(stream)
        g.replay()
        e1.record(stream)
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / n
        del g
        return us

    def launch_spread(calls, n):
        """Per-launch event durations (context: spread across single launches)."""
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(n)]
        for i in range(n):
            ev[i][0].record(stream)
            run([calls[i % len(calls)]], 1)
            ev[i][1].record(stream)
        torch.cuda.synchronize()
        return np.array([a.elapsed_time(b) for a, b in ev]) * 1e-3

    def calibration_copy():
        src = torch.empty(256 << 20, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(20):
            dst.copy_(src)
        torch.cuda.synchronize()

    xb, gb = W.workload_inputs(HEADLINE)
    rows, hidden = xb.shape

    # ----------------------------------------------------- counter runs only
    if args.counters:
        name = args.counters
        if name in ("headline", "c2", "c4", "h16", "h32", "two_pass"):
            cfg = {"headline": 3, "c2": 2, "c4": 4, "h16": 5, "h32": 5, "two_pass": 3}[name]
            wl = W.WORKLOADS[cfg]
            xc, gc = (xb, gb) if cfg == HEADLINE else W.workload_inputs(cfg)
            elem = wl.elem
            gd, sc = device_sets(xc, gc, elem, 2, two_pass=(name == "two_pass"))
            if name == "two_pass":
                cl = two_pass_calls(sc, gd, elem)
            else:
                cl = mxnorm_calls(sc, gd, 2, elem, 32 if name == "h32" else wl.had)
            run(cl, 20)
        elif name.startswith("bwd"):
            br, bh = (2048, 32768) if name == "bwd_2048x32768" else (rows, hidden)
            if br == rows:
                bx, bg = xb, gb
            else:
                bx = W.to_bf16_bits(W.random_rows(br, bh, 77))
                bg = W.to_bf16_bits(np.float32(1.0) + np.float32(0.02) *
                                    W.random_rows(1, bh, 78)[0])
            x = torch.from_numpy(bx.view(np.int16)).to(dev)
            gd = torch.from_numpy(bg.view(np.int16)).to(dev)
            dy = torch.from_numpy(W.grad_output(br, bh, HEADLINE).view(np.int16)).to(dev)
            rr = mxq.mxnorm_fwd(x.view(torch.bfloat16), gd.view(torch.bfloat16), p=2)[2]
            gain = name != "bwd_no_gain"
            for _ in range(20):
                mxq.mxnorm_bwd(x.view(torch.bfloat16), dy.view(torch.bfloat16), rr,
                               gd.view(torch.bfloat16) if gain else None)
        else:  # matmul
            xt = torch.from_numpy(xb.view(np.int16)).to(dev).view(torch.bfloat16)
            xc_, xs_ = mxq.mxnorm_fwd(xt, None, p=2)[:2]
            wt = torch.from_numpy(W.linear_weight(hidden, hidden, HEADLINE).view(np.int16)).to(dev)
            gt_ = torch.from_numpy(gb.view(np.int16)).to(dev)
            wc, wsc = mxq.mx_quant_gain(wt.view(torch.bfloat16), gt_.view(torch.bfloat16))
            out = torch.empty((rows, hidden), dtype=torch.float32, device=dev)
            for _ in range(20):
                mxq.mx_matmul(xc_, xs_, wc, wsc, c=out)
        torch.cuda.synchronize()
        calibration_copy()
        print("counters run: 20 x %s, 20 x 256 MiB copy" % name)
        return

    # ---------------------------------------------------------------- headline
    w = W.WORKLOADS[HEADLINE]
    g, sets = device_sets(xb, gb, w.elem, args.buffers)
    calls = mxnorm_calls(sets, g, 2, w.elem)
    nbytes = algorithmic_bytes(rows, hidden, w.elem)

    wall, gpu_s = time_steps_graph(calls, args.steps, args.warmup)
    value = nbytes * args.steps / wall / 1e9
    kern_s = gpu_s / args.steps
    achieved = nbytes / kern_s / 1e9
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS,
                "unit": "GB/s", "frac": round(achieved / PEAK_HBM_GBS, 4),
                "traffic": read_traffic()}
    spread = launch_spread(calls, 60)
    extras = {"algorithmic_bytes_per_launch": nbytes,
              "kernel_us_mean_timed_region": round(kern_s * 1e6, 3),
              "single_launch_event_us_p10_p50_p90": [
                  round(float(np.percentile(spread, q)) * 1e6, 2) for q in (10, 50, 90)],
              "rows_per_s": round(rows * args.steps / wall, 1),
              "pct_of_peak_wall": round(100 * value / PEAK_HBM_GBS, 2),
              "buffer_sets": args.buffers,
              "timed_region": "one replay of a HIP graph of the K captured calls",
              "clock_ramp_s_before_warmup": CLOCK_RAMP_S,
              "kernel_source_hash": kernel_hash()}

    # the same K steps as direct calls through the C ABI (context: per-call host
    # work in Python, whose jitter shows at small K)
    dwall, dgpu = time_steps(calls, args.steps, 0)
    extras["direct_calls_kernel_us_mean"] = round(dgpu / args.steps * 1e6, 3)
    extras["direct_calls_wall_GBps"] = round(nbytes * args.steps / dwall / 1e9, 1)

    if not args.no_extras:
        head_us = graph_us(calls, 300)
        extras["headline_graph_us_per_call"] = round(head_us, 3)
        # the practical ceiling of this byte traffic: the measurement library's
        # patterns (no arithmetic) on the same buffers
        pat_bytes = algorithmic_bytes(rows, hidden, w.elem, gamma=False)
        pats = {}
        for lay, lname in measure.LAYOUTS.items():
            us = graph_us(pattern_calls(sets, lay), 300)
            pats[lname] = {"us": round(us, 3), "GBps": round(pat_bytes / us / 1e3, 1)}
        best = min(v["us"] for v in pats.values())
        extras["patterns_16384x4096"] = pats
        extras["headline_graph_over_best_pattern"] = round(head_us / best, 4)
        extras["best_pattern_frac_of_peak"] = round(pat_bytes / best / 1e3 / PEAK_HBM_GBS, 4)
        # the same workload without a gain (MXNormLinear mode)
        us = graph_us(mxnorm_calls(sets, g, 2, w.elem, gain=False), 300)
        extras["headline_no_gain_us_per_call"] = round(us, 3)
        extras["headline_no_gain_algorithmic_GBps"] = round(
            algorithmic_bytes(rows, hidden, w.elem, gamma=False) / us / 1e3, 1)
        # warm-cache context: one buffer set reused every step
        us = graph_us(calls[:1], 300)
        extras["headline_one_buffer_set_us_per_call"] = round(us, 3)
        del sets, calls
        torch.cuda.empty_cache()

        # rows sweep at hidden 4096: the headline matrix tiled; fit t = a + bytes/B
        x16 = torch.from_numpy(xb.view(np.int16)).to(dev).view(torch.bfloat16)
        sweep = {"rows": [8192, 16384, 32768, 65536], "kernel_us": []}
        sweep_layouts = (measure.ONE_WAVE_CHUNK8, measure.TWO_WAVES_CHUNK8,
                         measure.ONE_WAVE_LANE16X)
        for lay in sweep_layouts:
            sweep["pattern_%s_us" % measure.LAYOUTS[lay]] = []
        for r in sweep["rows"]:
            xr = x16[:r] if r <= rows else x16.repeat(r // rows, 1)
            ss = make_sets(xr, w.elem, 2 if r >= 32768 else 3)
            sweep["kernel_us"].append(round(graph_us(mxnorm_calls(ss, g, 2, w.elem), 100), 3))
            for lay in sweep_layouts:
                sweep["pattern_%s_us" % measure.LAYOUTS[lay]].append(
                    round(graph_us(pattern_calls(ss, lay), 100), 3))
            del ss, xr
            torch.cuda.empty_cache()
        bx = [algorithmic_bytes(r, hidden, w.elem) for r in sweep["rows"]]
        fits = {}
        for key in [k for k in sweep if k.endswith("_us")]:
            a, b = fit_line(bx, sweep[key])
            fits[key[:-3]] = {"intercept_us": round(a, 3),
                              "asymptotic_GBps": round(1e-3 / b, 1),
                              "asymptotic_frac_of_peak": round(1e-3 / b / PEAK_HBM_GBS, 4)}
        sweep["fit_t_equals_a_plus_bytes_over_B"] = fits
        extras["rows_sweep_hidden4096"] = sweep
        del x16

        # a device-to-device copy moving the headline's byte count (read + write
        # = the algorithmic bytes), two rotated pairs, and of 1 GiB
        for label, cbytes in (("same_bytes", nbytes // 2), ("1GiB", 1 << 30)):
            pairs = [(torch.empty(cbytes, dtype=torch.uint8, device=dev),
                      torch.empty(cbytes, dtype=torch.uint8, device=dev)) for _ in range(2)]
            cc = [lambda st, p=p: (p[1].copy_(p[0]), 0)[1] for p in pairs]
            n = 200 if label == "same_bytes" else 20
            us = graph_us(cc, n)
            extras["device_copy_%s_GBps" % label] = round(2 * cbytes / us / 1e3, 1)
            if label == "same_bytes":
                extras["device_copy_same_bytes_us"] = round(us, 3)
            del pairs, cc
            torch.cuda.empty_cache()

        # two-pass baseline on the same workload
        g2, sets2 = device_sets(xb, gb, w.elem, max(2, args.buffers // 2), two_pass=True)
        us = graph_us(two_pass_calls(sets2, g2, w.elem), 200)
        extras["two_pass_us_per_call"] = round(us, 3)
        extras["speedup_vs_two_pass"] = round(us / head_us, 3)
        extras["two_pass_algorithmic_GBps"] = round(two_pass_bytes(rows, hidden, w.elem)
                                                    / us / 1e3, 1)
        del sets2
        torch.cuda.empty_cache()

        # straight-through backward (dy seeded, rho from the forward): with the
        # gain (dx + dgamma, two launches) and without it, on the headline
        # matrix, and with the gain on wider rows of the same element count
        dyb = W.grad_output(rows, hidden, HEADLINE)
        for (br, bh) in ((rows, hidden), (8192, 8192), (2048, 32768)):
            if br == rows:
                bx, bg, bd = xb, gb, dyb
            else:
                bx = W.to_bf16_bits(W.random_rows(br, bh, 77))
                bg = W.to_bf16_bits(np.float32(1.0) + np.float32(0.02) *
                                    W.random_rows(1, bh, 78)[0])
                bd = W.grad_output(br, bh, 77)
            gd = torch.from_numpy(bg.view(np.int16)).to(dev)
            bsets = []
            for i in range(3):
                x = torch.from_numpy(bx.view(np.int16)).to(dev)
                rr = mxq.mxnorm_fwd(x.view(torch.bfloat16), gd.view(torch.bfloat16), p=2)[2]
                bsets.append(dict(x=x, dy=torch.from_numpy(bd.view(np.int16)).to(dev), r=rr,
                                  dx=torch.empty_like(x),
                                  dg=torch.empty((bh,), dtype=torch.float32, device=dev),
                                  ws=torch.empty((mxq.mxnorm_bwd_workspace_bytes(br, bh) // 4,),
                                                 dtype=torch.float32, device=dev)))
            for gain in ((True, False) if br == rows else (True,)):
                bc = [lambda st, s=s, gain=gain: L.mxnorm_bwd(
                    s["x"].data_ptr(), s["dy"].data_ptr(), gd.data_ptr() if gain else None,
                    s["r"].data_ptr(), br, bh, s["dx"].data_ptr(),
                    s["dg"].data_ptr() if gain else None, s["ws"].data_ptr() if gain else None,
                    st) for s in bsets]
                us = graph_us(bc, 100)
                key = "mxnorm_bwd" + ("" if gain else "_no_gain")
                if br != rows:
                    key += "_%dx%d" % (br, bh)
                extras[key + "_us_per_call"] = round(us, 3)
                extras[key + "_algorithmic_GBps"] = round(bwd_bytes(br, bh, gain) / us / 1e3, 1)
            if br == rows:
                # the backward's byte pattern (libmxq_measure.so: x and dy read,
                # dx written, each store waiting for its whole row) in the
                # backward's layouts, 2 and 8 waves per row
                pats = {}
                for wv in (2, 8):
                    if not M.mxq_bwd_pattern_supported(wv, bh):
                        continue
                    pc = [lambda st, s=s, wv=wv: M.mxq_measure_bwd_pattern(
                        wv, s["x"].data_ptr(), s["dy"].data_ptr(), br, bh, s["dx"].data_ptr(), st)
                        for s in bsets]
                    us = graph_us(pc, 100)
                    pats["waves_%d" % wv] = {"us": round(us, 3),
                                             "GBps": round(bwd_bytes(br, bh, False) / us / 1e3, 1)}
                if pats:
                    best = min(v["us"] for v in pats.values())
                    extras["bwd_patterns_%dx%d" % (br, bh)] = pats
                    extras["bwd_best_pattern_frac_of_peak"] = round(
                        bwd_bytes(br, bh, False) / best / 1e3 / PEAK_HBM_GBS, 4)
                    for key in ("mxnorm_bwd", "mxnorm_bwd_no_gain"):
                        extras[key + "_over_best_bwd_pattern"] = round(
                            extras[key + "_us_per_call"] / best, 4)
            del bsets
            torch.cuda.empty_cache()

        # MXNormLinear on the headline matrix: the gain folded into a square
        # weight (hidden x hidden, cast once), then per step mxnorm_fwd with no
        # gain into MXFP8 + the MXFP8 matmul (fp32 out).  The matmul alone is
        # priced against the fp8 dense matrix peak.
        gb_dev = torch.from_numpy(gb.view(np.int16)).to(dev)
        wbits = W.linear_weight(hidden, hidden, HEADLINE)
        wdev = torch.from_numpy(wbits.view(np.int16)).to(dev)
        wc = torch.empty((hidden, hidden), dtype=torch.uint8, device=dev)
        wsc = torch.empty((hidden, hidden // 32), dtype=torch.uint8, device=dev)
        mxq.mx_quant_gain(wdev.view(torch.bfloat16), gb_dev.view(torch.bfloat16), codes=wc,
                          scales=wsc)
        lsets = []
        for i in range(2):
            lsets.append(dict(x=torch.from_numpy(xb.view(np.int16)).to(dev),
                              xc=torch.empty((rows, hidden), dtype=torch.uint8, device=dev),
                              xs=torch.empty((rows, hidden // 32), dtype=torch.uint8, device=dev),
                              out=torch.empty((rows, hidden), dtype=torch.float32, device=dev),
                              outh=torch.empty((rows, hidden), dtype=torch.bfloat16, device=dev)))
        for s in lsets:
            mxq.mxnorm_fwd(s["x"].view(torch.bfloat16), None, p=2, codes=s["xc"], scales=s["xs"])
        flops = 2.0 * rows * hidden * hidden
        for otype, okey, sfx in ((mxq.OUT_F32, "out", ""), (mxq.OUT_BF16, "outh", "_bf16_out")):
            mm = [lambda st, s=s: L.mx_matmul(s["xc"].data_ptr(), s["xs"].data_ptr(),
                                              wc.data_ptr(), wsc.data_ptr(), rows, hidden,
                                              hidden, s[okey].data_ptr(), otype, st)
                  for s in lsets]
            us = graph_us(mm, 20, seconds=0.1)
            extras["mx_matmul%s_us_per_call" % sfx] = round(us, 3)
            extras["mx_matmul%s_TFLOPs" % sfx] = round(flops / us / 1e6, 1)
            if not sfx:
                extras["mx_matmul_shape"] = [rows, hidden, hidden]
                extras["mx_matmul_frac_of_fp8_dense_peak"] = round(
                    flops / us / 1e-6 / FP8_DENSE_PEAK, 4)
        lin = [lambda st, s=s: L.mxnorm_linear_fwd(s["x"].data_ptr(), rows, hidden, 2, C_P2,
                                                   wc.data_ptr(), wsc.data_ptr(), hidden,
                                                   s["xc"].data_ptr(), s["xs"].data_ptr(), None,
                                                   s["out"].data_ptr(), mxq.OUT_F32, st)
               for s in lsets]
        extras["mxnorm_linear_fwd_us_per_call"] = round(graph_us(lin, 20, seconds=0.1), 3)
        # The unfused layer MXNormLinear replaces: RMSNorm with its gain to a
        # bf16 y, the MX cast of y (the two-pass baseline), then the matmul
        # with the plain MX cast of W.
        wpc = torch.empty((hidden, hidden), dtype=torch.uint8, device=dev)
        wps = torch.empty((hidden, hidden // 32), dtype=torch.uint8, device=dev)
        mxq.mx_quant(wdev.view(torch.bfloat16), codes=wpc, scales=wps)
        ys = [torch.empty((rows, hidden), dtype=torch.bfloat16, device=dev) for _ in lsets]

        def unfused(st, s, y):
            rc = L.rmsnorm_mxquant_fwd(s["x"].data_ptr(), gb_dev.data_ptr(), rows, hidden, 1e-5,
                                       mxq.E4M3, y.data_ptr(), s["xc"].data_ptr(),
                                       s["xs"].data_ptr(), None, st)
            return rc or L.mx_matmul(s["xc"].data_ptr(), s["xs"].data_ptr(), wpc.data_ptr(),
                                     wps.data_ptr(), rows, hidden, hidden, s["out"].data_ptr(),
                                     mxq.OUT_F32, st)
        unf = [lambda st, s=s, y=y: unfused(st, s, y) for s, y in zip(lsets, ys)]
        extras["rmsnorm_mxquant_then_matmul_us_per_call"] = round(
            graph_us(unf, 20, seconds=0.1), 3)
        extras["mxnorm_linear_speedup_vs_unfused"] = round(
            extras["rmsnorm_mxquant_then_matmul_us_per_call"]
            / extras["mxnorm_linear_fwd_us_per_call"], 3)
        del ys, wpc, wps, lsets, wdev, wc, wsc
        torch.cuda.empty_cache()

        # the other workloads (context; the headline is workload 3), and the
        # byte patterns at the 8192 x 2048 workload
        others = {}
        for cfg in (1, 2, 4, 5):
            wc_ = W.WORKLOADS[cfg]
            xc, gc = W.workload_inputs(cfg)
            r, d = xc.shape
            nset = 2 if r * d <= 256 * 1024 else max(2, args.buffers // 2)
            gdev, sc = device_sets(xc, gc, wc_.elem, nset, two_pass=(cfg == 2))
            b = algorithmic_bytes(r, d, wc_.elem)
            for p in wc_.ps:
                cl = mxnorm_calls(sc, gdev, p, wc_.elem, wc_.had)
                us = graph_us(cl, 400 if cfg <= 2 else 200)
                st_wall, _ = time_steps(cl, 200, 10)
                others["%s_p%d" % (wc_.name, p)] = {
                    "kernel_us_graph": round(us, 3),
                    "GBps_kernel": round(b / us / 1e3, 1),
                    "frac_of_peak": round(b / us / 1e3 / PEAK_HBM_GBS, 4),
                    "us_per_call_direct_launches_wall": round(st_wall / 200 * 1e6, 3)}
            if cfg == 2:
                # this workload is defined against the two-pass RMSNorm + MX cast
                us2 = graph_us(two_pass_calls(sc, gdev, wc_.elem), 400)
                others["%s_two_pass" % wc_.name] = {
                    "kernel_us_graph": round(us2, 3),
                    "GBps_kernel": round(two_pass_bytes(r, d, wc_.elem) / us2 / 1e3, 1)}
                for p in wc_.ps:
                    k = "%s_p%d" % (wc_.name, p)
                    others[k]["speedup_vs_two_pass"] = round(us2 / others[k]["kernel_us_graph"], 3)
                pb = algorithmic_bytes(r, d, wc_.elem, gamma=False)
                pats2 = {}
                for lay, lname in measure.LAYOUTS.items():
                    if M.mxq_pattern_supported(lay, d):
                        us = graph_us(pattern_calls(sc, lay), 400)
                        pats2[lname] = {"us": round(us, 3), "GBps": round(pb / us / 1e3, 1)}
                others["patterns_%dx%d" % (r, d)] = pats2
                bestp = min(v["us"] for v in pats2.values())
                for p in wc_.ps:
                    k = "%s_p%d" % (wc_.name, p)
                    others[k]["over_best_pattern"] = round(others[k]["kernel_us_graph"] / bestp, 4)
            del sc
            torch.cuda.empty_cache()
        extras["other_workloads"] = others

        # the variants beside the method's main path (context): H32 -> E2M1 and
        # H16 -> E4M3 on workload 5's matrix, and the exact-absmax block
        # magnitude (mxnorm_fwd_ex) on the headline matrix
        variants = {}
        xc, gc = W.workload_inputs(5)
        r, d = xc.shape
        for had, elem, name in ((32, mxq.E2M1, "h32_e2m1"), (16, mxq.E4M3, "h16_e4m3")):
            gdev, sc = device_sets(xc, gc, elem, max(2, args.buffers // 2))
            us = graph_us(mxnorm_calls(sc, gdev, 2, elem, had), 200)
            b = algorithmic_bytes(r, d, elem)
            variants["%s_%dx%d_p2" % (name, r, d)] = {
                "kernel_us_graph": round(us, 3), "GBps_kernel": round(b / us / 1e3, 1),
                "frac_of_peak": round(b / us / 1e3 / PEAK_HBM_GBS, 4)}
            del sc
            torch.cuda.empty_cache()
        gdev, sc = device_sets(xb, gb, w.elem, max(2, args.buffers // 2))
        cl = []
        for s_ in sc:
            a_ = (s_["x"].data_ptr(), gdev.data_ptr(), rows, hidden, 2, 0.0, mxq.SRC_ABSMAX, 0,
                  w.elem, s_["codes"].data_ptr(), s_["scales"].data_ptr(), s_["rrms"].data_ptr())
            cl.append(lambda st, a_=a_: L.mxnorm_fwd_ex(*a_, st))
        us = graph_us(cl, 200)
        b = algorithmic_bytes(rows, hidden, w.elem)
        variants["absmax_e4m3_%dx%d_p2" % (rows, hidden)] = {
            "kernel_us_graph": round(us, 3), "GBps_kernel": round(b / us / 1e3, 1)}
        del sc
        torch.cuda.empty_cache()
        extras["variants"] = variants

    # ------------------------------------------------------- CPU oracle baseline
    cpu = None
    if not args.no_cpu:
        import oracle as O
        O.lib()
        threads = O.max_threads()

        def oracle_runs(n):
            reps = []
            for _ in range(n):
                t0 = time.perf_counter()
                O.mxnorm_fwd(xb, gb, 2, C_P2, w.elem)
                reps.append(time.perf_counter() - t0)
            return sorted(reps)[len(reps) // 2]

        t = oracle_runs(3)
        cpu = {"value": round(nbytes / t / 1e9, 3), "unit": "GB/s",
               "cores": threads, "kind": "oracle",
               "sample": "the full 16384x4096 headline matrix, median of 3 runs "
                         "(%.2f s), OpenMP over rows on %d threads" % (t, threads)}
        O.set_threads(1)
        t1 = oracle_runs(3)
        O.set_threads(threads)
        extras["cpu_oracle_single_thread_GBps"] = round(nbytes / t1 / 1e9, 4)
        extras["cpu_oracle_single_thread_s"] = round(t1, 3)
        extras["cpu_oracle_rows_per_s"] = round(rows / t, 1)
        extras["host_nproc"] = os.cpu_count()
        model = None
        try:
            with open("/proc/cpuinfo") as f:
                for line in f:
                    if line.startswith("model name"):
                        model = line.split(":", 1)[1].strip()
                        break
        except OSError:
            pass
        extras["host_cpu_model"] = model

    out = {"metric": METRIC, "value": round(value, 1), "unit": "GB/s", "n_gpus": 1,
           "steps": args.steps, "warmup": args.warmup,
           "ms_per_step": round(wall / args.steps * 1e3, 5),
           "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
           "dtype": "f32", "data": "synthetic",
           "config": {"workload": w.name, "rows": rows, "hidden": hidden, "p": 2,
                      "elem": "e4m3", "gamma": True, "block": 32,
                      "inputs": "bf16 N(0,1), 1% outlier channels x20, per-row lognormal "
                                "scale (sigma 1), seed 3"},
           "roofline": roofline, "cpu_baseline": cpu, "extras": extras}
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
