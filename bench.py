#!/usr/bin/env python3
"""Benchmark of the dense GEMM on one MI355X.

One step is one call of the library's GEMM (grid decomposition, global->LDS
staging, MFMA main loop, edge handling and epilogue, and for the split-K class
the reduce) on a seeded synthetic workload whose operands are already resident
in HBM.  Prints ONE JSON line (last line of stdout):

  metric / value / unit   GEMM TFLOP/s of --workload (default fp32 4096^3):
                          2*M*N*K per step over the timed steps
  roofline                the GEMM kernel against the MI355X dense matrix peak
                          of its input type (the tall-skinny shape: achieved
                          HBM GB/s against 8 TB/s), from HIP events on the
                          stream the kernel runs on; `traffic` is the HBM bytes
                          per launch read from the committed rocprofv3 counter
                          summary (profiles/traffic.json) when it was taken on
                          the current sources, else null -- it is a stored
                          reading, not measured in this run
  per_call_ms             median, minimum and maximum of single calls (HIP events
                          between consecutive calls, up to 50 calls after the
                          timed steps; likewise in each 'also' entry)
  sclk_sustained          the graphics clock, memory clock, board power and
                          temperatures the GPU holds over 2.5 s of the headline
                          workload run back to back after the timed steps
                          (amdsmi GPU metrics, when readable; likewise for every
                          configuration in 'also', as sclk_sustained_mhz,
                          socket_power_w, mclk_mhz, hotspot_c and hbm_c -- for
                          the shortest calls the host's launch rate, not the
                          GPU, can bound that back-to-back run)
  cpu_baseline            the oracle (CPU, fp64) timed on a bounded sample of the
                          same workload on this host
  also                    the same measurement, in short form, for the other
                          configurations: bf16 8192^3, the im2col and
                          tall-skinny shapes, fp32 1000^3 and the ragged
                          4097 x 4095 x 4099 (all measured before the headline
                          workload, each with its own warm-up); with --all
                          also the generalised-GEMM variants (transposed
                          operands, alpha/beta, bf16 C)

With --all the convolution routes (im2col + GEMM, implicit GEMM with each
address form, the im2col kernel against HBM; 2-D, 3-D and 4-D workloads) are
timed too and printed as a separate JSON line before the last one.

Usage:  python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--all]
                       [--operand-values workload|small-int|zero]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_TFLOPS = {"f32": 157.3, "bf16": 2516.6}   # MI355X dense matrix peaks
HBM_PEAK_GBS = 8000.0
PRIMARY = "fp32-4096"
SECONDARY = ["bf16-8192", "im2col", "tall", "fp32-1000", "fp32-rag"]
EXTRA = ["bf16-8192-nt-bf16c", "bf16-8192-tn-acc", "fp32-4096-tt-ab"]
# Judged on HBM bandwidth rather than matrix throughput (its MFMA-limited time
# at the fp32 peak caps the achievable rate below 8 TB/s).
HBM_BOUND = {"tall"}
CONV = ["conv-64c-31k", "conv-64c-31k-bf16", "conv3d-32c-k7", "conv3d-32c-k7-bf16",
        "conv4d-16c-k5"]


def log(msg: str) -> None:
    print(msg, file=sys.stderr, flush=True)


# Sources that define each kernel family's device code (and, for the
# convolution routes, the dispatcher that picks their GEMM kernels): stored
# counter readings are used only while these are unchanged.
KERNEL_SOURCES = {
    "gemm": ["gemm_kernel.hpp", "gemm_launch.hpp", "gemm_instances.hip"],
    "im2col": ["conv.hip"],
    # a convolution route: im2col and/or the GEMM kernels, the reduce, the
    # implicit loaders and their table and pad kernels
    "conv": ["conv.hip", "gemm_kernel.hpp", "gemm_launch.hpp", "gemm_instances.hip",
             "gemm_aux.hip", "gemm_api.hip"],
}


def source_digest(family: str = "gemm") -> str:
    """Hash of the HIP sources of one kernel family."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "dense_gemm_03_amd", "csrc")
    for name in sorted(KERNEL_SOURCES[family]):
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(name.encode() + b"\0" + f.read())
    return h.hexdigest()[:16]


def stored_traffic(workload: str, family: str = "gemm", config: str | None = None):
    """HBM bytes per launch from profiles/traffic.json, if taken on these
    sources (and, for a GEMM, on the tile configuration dispatched now)."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        with open(path) as f:
            data = json.load(f)
    except (OSError, ValueError):
        return None
    entry = data.get(workload)
    if not entry or entry.get("sources") != source_digest(family):
        return None
    if config is not None and entry.get("config") != config:
        return None
    return entry.get("bytes_per_launch")


def sustained_clock(step, seconds: float = 2.5):
    """The graphics clock the GPU holds while running `step` back to back:
    the workload runs for `seconds` while a thread samples amdsmi's GPU
    metrics; the SMU refreshes that table too slowly for the timed steps
    themselves, and readings lag by up to about a second), and the median of
    the samples of the last second is reported.  Outside the timed steps."""
    import threading

    import torch
    try:
        import amdsmi
        amdsmi.amdsmi_init()
        handles = amdsmi.amdsmi_get_processor_handles()
        if len(handles) != 1:
            raise RuntimeError("%d GPUs visible to amdsmi" % len(handles))
        handle = handles[0]
    except Exception as e:  # noqa: BLE001 - reported, not fatal
        return {"mhz": None, "error": "%s: %s" % (type(e).__name__, e)}

    def num(v):
        return float(v) if isinstance(v, (int, float)) and not isinstance(v, bool) else None

    def read():
        m = amdsmi.amdsmi_get_gpu_metrics_info(handle)
        clks = [c for c in (m.get("current_gfxclks") or []) if isinstance(c, (int, float)) and c > 0]
        mhz = float(sum(clks)) / len(clks) if clks else float(m.get("current_gfxclk") or 0)
        return (mhz, num(m.get("current_socket_power")), num(m.get("current_uclk")),
                num(m.get("temperature_hotspot")), num(m.get("temperature_mem")))

    samples, stop, err = [], threading.Event(), []

    def loop():
        while not stop.is_set():
            try:
                samples.append((time.perf_counter(),) + read())
            except Exception as e:  # noqa: BLE001
                err.append("%s: %s" % (type(e).__name__, e))
                return
            time.sleep(0.002)

    th = threading.Thread(target=loop, daemon=True)
    t0 = time.perf_counter()
    th.start()
    while time.perf_counter() - t0 < seconds:
        for _ in range(8):
            step()
        torch.cuda.synchronize()
    stop.set()
    th.join()
    tail = [x for x in samples if x[0] - t0 >= seconds - 1.0]

    def median(i):
        v = sorted(x[i] for x in tail if x[i] is not None)
        return v[len(v) // 2] if v else None

    late = sorted(x[1] for x in tail)
    if not late:
        return {"mhz": None, "error": err[0] if err else "no sample"}
    return {"mhz": late[len(late) // 2], "min_mhz": late[0], "max_mhz": late[-1],
            "socket_power_w": median(2), "mclk_mhz": median(3),
            "hotspot_c": median(4), "hbm_c": median(5),
            "samples": len(late), "window_s": seconds,
            "source": "amdsmi gpu_metrics current_gfxclks (mean over XCDs), current_uclk, "
                      "current_socket_power, temperature_hotspot and temperature_mem, medians "
                      "over the last second of a %.1f s back-to-back run of this workload"
                      % seconds}


def _workload(name: str):
    from dense_gemm_03_amd.workloads import VARIANTS, WORKLOADS
    return WORKLOADS[name] if name in WORKLOADS else VARIANTS[name]


def _operands(w, values: str):
    """The workload's operands (values "workload"), or arrays of the same
    shapes and types holding small integers in [-3, 3] or zeros: the same
    calls and instructions on other data, to show how the operand values move
    the board's power and so its clock."""
    from dense_gemm_03_amd import workloads as wl
    if values == "workload":
        return w.operands()
    shapes = [(w.K, w.M) if w.transa else (w.M, w.K), (w.N, w.K) if w.transb else (w.K, w.N)]
    bf16 = w.dtype == "bf16"
    if values == "small-int":
        gen = wl.small_int_bf16_bits if bf16 else wl.small_int_f32
        return tuple(gen(sh, w.seed + 1 + i) for i, sh in enumerate(shapes))
    return tuple(np.zeros(sh, dtype=np.uint16 if bf16 else np.float32) for sh in shapes)


OPERAND_VALUES = "workload"


def prepare(name: str):
    """Draw workload `name`'s operands on the host and copy them to the GPU;
    returns what measure() needs."""
    import torch

    import dense_gemm_03_amd as dg

    w = _workload(name)
    log("[bench] %s: drawing operands %dx%dx%d (%s, values: %s)" % (
        name, w.M, w.N, w.K, w.dtype, OPERAND_VALUES))

    def dev(x):
        if x.dtype == np.uint16:
            return torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).to("cuda:0")
        return torch.from_numpy(x).to("cuda:0")

    A_np, B_np = _operands(w, OPERAND_VALUES)
    A, B = dev(A_np), dev(B_np)
    del A_np, B_np
    if w.beta != 0.0:
        C = dev(w.initial_c())
    else:
        C = torch.empty((w.M, w.N), dtype=torch.float32 if w.out == "f32" else torch.bfloat16,
                        device="cuda:0")
    # Workloads judged on HBM bandwidth whose operands would fit the 256 MB
    # MALL (Infinity Cache) across back-to-back steps rotate over three copies
    # of A and B, so every step streams its operands from HBM.  (The im2col
    # shape's 4 GB B cannot stay cached; the compute-bound shapes are not
    # judged on bandwidth.)
    operands = [(A, B)]
    if name == "tall":
        operands += [(A.clone(), B.clone()) for _ in range(2)]
    torch.cuda.synchronize()
    return {"name": name, "w": w, "operands": operands, "C": C}


def measure(ctx, steps: int, warmup: int):
    """Time `steps` GEMM calls on a prepared workload; returns a result dict."""
    import torch

    import dense_gemm_03_amd as dg

    name, w, operands, C = ctx["name"], ctx["w"], ctx["operands"], ctx["C"]
    stream = torch.cuda.current_stream()
    dtype_id = dg.GEMM_DTYPE_F32 if w.dtype == "f32" else dg.GEMM_DTYPE_BF16
    ta, tb = int(w.transa), int(w.transb)
    cfg = dg.gemm_select_config_ex(dtype_id, ta, tb, w.M, w.N, w.K)
    splits = dg.gemm_split_k_ex(dtype_id, cfg, ta, tb, w.M, w.N, w.K)
    turn = [0]

    def step():
        # with beta != 0 every step accumulates into C again: same work, the
        # values only grow (they stay finite over these step counts)
        a_op, b_op = operands[turn[0] % len(operands)]
        turn[0] += 1
        dg.gemm(a_op, b_op, out=C, alpha=w.alpha, beta=w.beta, transa=w.transa, transb=w.transb)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    log("[bench] %s: warmup done (%d), timing %d steps with %s" % (
        name, warmup, steps, dg.gemm_config_name(dtype_id, cfg)))

    # HIP events on the stream the library launches on (torch's current
    # stream, passed to the C ABI), bracketing the timed region.
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev0.record(stream)
    for _ in range(steps):
        step()
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    event_ms = ev0.elapsed_time(ev1) / steps

    # Spread of single calls, outside the timed region: HIP events recorded
    # between consecutive calls on the same stream, median and minimum.
    n_calls = min(steps, 50)
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(n_calls + 1)]
    evs[0].record(stream)
    for i in range(n_calls):
        step()
        evs[i + 1].record(stream)
    torch.cuda.synchronize()
    per_call = sorted(evs[i].elapsed_time(evs[i + 1]) for i in range(n_calls))
    per_call_ms = {"median": per_call[n_calls // 2], "min": per_call[0], "max": per_call[-1],
                   "calls": n_calls}
    ms_per_step = wall * 1e3 / steps
    tflops = w.flops * steps / wall / 1e12
    achieved = w.flops / (event_ms * 1e-3) / 1e12
    peak = PEAK_TFLOPS[w.dtype]
    traffic = stored_traffic(name, "gemm", dg.gemm_config_name(dtype_id, cfg))
    hbm_gbs = w.algorithmic_bytes / (event_ms * 1e-3) / 1e9
    if name in HBM_BOUND:
        # the shape is judged on HBM bandwidth; at the fp32 matrix peak its
        # flops alone take w.flops / peak, which caps the reachable rate
        roofline = {"bound": "hbm", "achieved": hbm_gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                    "frac": hbm_gbs / HBM_PEAK_GBS, "traffic": traffic,
                    "mfma_cap_gbs": w.algorithmic_bytes / (w.flops / (peak * 1e12)) / 1e9,
                    "tflops": achieved}
    else:
        roofline = {"bound": "mfma", "achieved": achieved, "peak": peak, "unit": "TFLOP/s",
                    "frac": achieved / peak, "traffic": traffic}
    roofline["traffic_source"] = ("stored rocprofv3 FETCH_SIZE/WRITE_SIZE reading "
                                  "(profiles/traffic.json), not measured in this run"
                                  if traffic is not None else None)
    res = {
        "workload": name,
        "M": w.M, "N": w.N, "K": w.K,
        "dtype": w.dtype,
        "op": ("A^T" if w.transa else "A") + "." + ("B^T" if w.transb else "B"),
        "alpha": w.alpha, "beta": w.beta, "c_dtype": w.out,
        "value": tflops,
        "ms_per_step": ms_per_step,
        "kernel_config": dg.gemm_config_name(dtype_id, cfg),
        "split_k": splits,
        "roofline": roofline,
        "hbm_gbs": hbm_gbs,
        "per_call_ms": per_call_ms,
        "operand_sets": len(operands),
        "step": step,
    }
    return res


def measure_conv(name: str, steps: int, warmup: int, only: str | None = None):
    """Time the convolution `name`: forward pass and filter gradient through
    im2col + GEMM and through the implicit GEMM (one to four dimensions), and
    the im2col kernel alone (its HBM roofline).  `only` names one of these
    measurements (for per-route profiler passes)."""
    import torch

    import dense_gemm_03_amd as dg
    from dense_gemm_03_amd.workloads import CONV_WORKLOADS, CONVND_WORKLOADS

    nd = name in CONVND_WORKLOADS
    c = CONVND_WORKLOADS[name] if nd else CONV_WORKLOADS[name]
    x_shape = (c.batch, c.cin) + (tuple(c.size) if nd else (c.h, c.w))
    w_shape = (c.cout, c.cin) + (tuple(c.kernel) if nd else (c.r, c.s))
    out = c.out if nd else (c.p, c.q)
    log("[bench] %s: drawing x %s, filters and output gradient" % (name, x_shape))

    def dev(a):
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to("cuda:0")
        return torch.from_numpy(a).to("cuda:0")

    x, w, dy = dev(c.x()), dev(c.weights()), dev(c.dy())
    dtype = dg.GEMM_DTYPE_F32 if c.dtype == "f32" else dg.GEMM_DTYPE_BF16
    F32 = dg.GEMM_DTYPE_F32
    if nd:
        params = dg.convnd_params(c.batch, c.cin, c.cout, c.size, c.kernel, c.pad, c.stride,
                                  c.dilation)
        api = {"ws": dg.convnd_workspace_size, "fwd": dg.convnd_fwd,
               "wgrad": dg.convnd_bwd_weight, "im2col": dg.convnd_im2col}
    else:
        params = dg.conv2d_params(c.batch, c.cin, c.h, c.w, c.cout, c.r, c.s, (c.pad, c.pad),
                                  (c.stride, c.stride), (c.dilation, c.dilation))
        api = {"ws": dg.conv2d_workspace_size, "fwd": dg.conv2d_fwd,
               "wgrad": dg.conv2d_bwd_weight, "im2col": dg.conv2d_im2col}
    need = api["ws"](dtype, params)
    ws = torch.empty(need, dtype=torch.uint8, device="cuda:0")
    y = torch.empty((c.batch, c.cout) + tuple(out), dtype=torch.float32, device="cuda:0")
    dw = torch.empty(w_shape, dtype=torch.float32, device="cuda:0")
    stream = torch.cuda.current_stream()
    sp = stream.cuda_stream
    ld = need // (c.crs * c.in_bytes)

    def fwd():
        assert api["fwd"](dtype, F32, params, x.data_ptr(), w.data_ptr(), y.data_ptr(),
                          ws.data_ptr(), need, sp) == dg.GEMM_OK

    def wgrad():
        assert api["wgrad"](dtype, params, x.data_ptr(), dy.data_ptr(), dw.data_ptr(),
                            ws.data_ptr(), need, sp) == dg.GEMM_OK

    def im2col():
        assert api["im2col"](dtype, params, 0, x.data_ptr(), ws.data_ptr(), ld, sp) == dg.GEMM_OK

    def implicit_fwd(mode):
        def run():
            assert dg.conv2d_fwd_implicit_ex(dtype, F32, params, mode, x.data_ptr(), w.data_ptr(),
                                             y.data_ptr(), sp) == dg.GEMM_OK
        return run

    def implicit_wgrad(mode):
        def run():
            assert dg.conv2d_bwd_weight_implicit_ex(dtype, params, mode, x.data_ptr(),
                                                    dy.data_ptr(), dw.data_ptr(), sp) == dg.GEMM_OK
        return run

    def timed(fn, n):
        for _ in range(warmup):
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0 = time.perf_counter()
        e0.record(stream)
        for _ in range(n):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return (time.perf_counter() - t0) * 1e3 / n, e0.elapsed_time(e1) / n

    res = {}
    peak = PEAK_TFLOPS[c.dtype]
    routes = [("fwd", fwd), ("wgrad", wgrad)]
    A, T, PD = dg.CONV_ADDR_ANALYTIC, dg.CONV_ADDR_TABLE, dg.CONV_ADDR_PADDED
    if nd:
        def fwd_nd_implicit(mode):
            def run():
                assert dg.convnd_fwd_implicit_ex(dtype, F32, params, mode, x.data_ptr(),
                                                 w.data_ptr(), y.data_ptr(), sp) == dg.GEMM_OK
            return run

        def wgrad_nd_implicit(mode):
            def run():
                assert dg.convnd_bwd_weight_implicit_ex(dtype, params, mode, x.data_ptr(),
                                                        dy.data_ptr(), dw.data_ptr(),
                                                        sp) == dg.GEMM_OK
            return run
        routes += [("fwd_implicit", fwd_nd_implicit(A)), ("wgrad_implicit", wgrad_nd_implicit(A)),
                   ("fwd_implicit_padded", fwd_nd_implicit(PD)),
                   ("wgrad_implicit_padded", wgrad_nd_implicit(PD))]
    if not nd:
        routes += [("fwd_implicit", implicit_fwd(A)), ("wgrad_implicit", implicit_wgrad(A)),
                   ("fwd_implicit_table", implicit_fwd(T)), ("wgrad_implicit_table", implicit_wgrad(T)),
                   ("fwd_implicit_padded", implicit_fwd(PD)),
                   ("wgrad_implicit_padded", implicit_wgrad(PD)),
                   ("fwd_implicit_window", implicit_fwd(dg.CONV_ADDR_WINDOW)),
                   ("wgrad_implicit_window", implicit_wgrad(dg.CONV_ADDR_WINDOW))]
    if only is not None and only not in [r[0] for r in routes] + ["im2col"]:
        raise SystemExit("unknown route %r for %s" % (only, name))
    for label, fn in routes:
        if only is not None and label != only:
            continue
        wall_ms, ev_ms = timed(fn, steps)
        log("[bench] %s %s: %.3f ms per call" % (name, label, ev_ms))
        ach = c.flops / (ev_ms * 1e-3) / 1e12
        # traffic: HBM bytes of one call of the route (all its kernels)
        res[label] = {"value": c.flops / (wall_ms * 1e-3) / 1e12, "ms_per_step": wall_ms,
                      "roofline": {"bound": "mfma", "achieved": ach, "peak": peak,
                                   "unit": "TFLOP/s", "frac": ach / peak,
                                   "traffic": stored_traffic(name + "-" + label, "conv")}}
    if only is None or only == "im2col":
        _, ev_ms = timed(im2col, steps)
        gbs = c.im2col_bytes / (ev_ms * 1e-3) / 1e9
        traffic = stored_traffic(name + "-im2col", "im2col")
        res["im2col"] = {"ms_per_call": ev_ms,
                         "roofline": {"bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS,
                                      "unit": "GB/s", "frac": gbs / HBM_PEAK_GBS,
                                      "traffic": traffic}}
        log("[bench] %s im2col: %.3f ms, %.0f GB/s" % (name, ev_ms, gbs))
    vol_out = int(np.prod(out))
    result = {"workload": name, "dtype": c.dtype,
              "shape": {"batch": c.batch, "cin": c.cin, "size": list(x_shape[2:]),
                        "cout": c.cout, "kernel": list(w_shape[2:]),
                        "pad": list(c.pad) if nd else c.pad,
                        "stride": list(c.stride) if nd else c.stride,
                        "dilation": list(c.dilation) if nd else c.dilation},
              "gemm_fwd": [c.cout, vol_out, c.crs], "gemm_wgrad": [c.cout, c.crs, vol_out]}
    result.update(res)
    del x, w, dy, ws, y, dw
    torch.cuda.empty_cache()
    return result


def cpu_baseline(name: str, budget_s: float = 10.0):
    """The oracle on a bounded row sample of the workload, scaled to TFLOP/s."""
    import oracle

    w = _workload(name)
    threads = oracle.default_threads()
    A, B = w.operands()
    C0 = w.initial_c() if w.beta != 0.0 else None
    kind = "f32" if w.dtype == "f32" else "bf16"

    def run(rows):
        # rows of op(A): leading rows of A, or leading columns of A^T's storage
        a = np.ascontiguousarray(A[:, :rows] if w.transa else A[:rows])
        c0 = None
        if C0 is not None:
            c0 = C0[:rows].astype(np.float64) if w.out == "f32" else oracle.bf16_bits_to_f64(C0[:rows])
        t = time.perf_counter()
        if w.plain:
            # the plain product alone (no tolerance scale S)
            (oracle.gemm_f32 if kind == "f32" else oracle.gemm_bf16)(a, B, threads=threads,
                                                                     with_s=False)
        else:
            oracle.gemm_general(a, B, w.alpha, w.beta, c0, w.transa, w.transb, kind=kind,
                                threads=threads)
        return time.perf_counter() - t

    rows = min(w.M, max(threads, 16))
    dt = run(rows)
    # grow the sample towards budget_s seconds of wall time (the whole
    # product when it takes less); small first samples overestimate the
    # per-row time, so re-estimate up to three times
    for _ in range(3):
        if rows >= w.M or dt >= budget_s / 2:
            break
        target = int(rows * budget_s / max(dt, 1e-3))
        rows2 = max(rows, min(w.M, target - target % threads if target > threads else target))
        if rows2 == rows:
            break
        dt = run(rows2)
        rows = rows2
    flops = 2.0 * rows * w.N * w.K
    return {
        "value": flops / dt / 1e12,
        "unit": "TFLOP/s",
        "cores": threads,
        "kind": "oracle",
        "sample": "first %d of %d rows of op(A) times all of op(B) (%dx%dx%d, fp64 accumulation), %.1f s"
                  % (rows, w.M, rows, w.N, w.K, dt),
    }


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--workload", default=PRIMARY)
    ap.add_argument("--all", action="store_true",
                    help="also time the generalised-GEMM variants and the convolution routes")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-also", action="store_true",
                    help="time only --workload (for per-kernel profiler passes)")
    ap.add_argument("--conv", default=None, metavar="NAME",
                    help="only time the convolution workload NAME (for per-kernel profiler "
                         "passes) and print its result")
    ap.add_argument("--conv-route", default=None, metavar="ROUTE",
                    help="with --conv: time only this route (fwd, wgrad, fwd_implicit, "
                         "wgrad_implicit, fwd_implicit_table, wgrad_implicit_table, "
                         "fwd_implicit_padded, wgrad_implicit_padded, fwd_implicit_window, "
                         "wgrad_implicit_window, im2col), "
                         "for per-route profiler passes")
    ap.add_argument("--operand-values", choices=("workload", "small-int", "zero"),
                    default="workload",
                    help="operand values of the GEMM workloads: the workloads' own seeded "
                         "distributions (default), integers in [-3, 3], or zeros -- the same "
                         "calls on other data, to show how the values move power and clock "
                         "(the CPU baseline keeps the workloads' values)")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="only run a plain device-to-device copy of MIB MiB (reference kernel "
                         "for the HBM byte counters) and exit")
    args = ap.parse_args()
    global OPERAND_VALUES
    OPERAND_VALUES = args.operand_values

    if args.gpus != 1:
        print("bench.py measures one GPU: this GEMM is built and timed on a single MI355X, "
              "--gpus %d is not supported" % args.gpus, file=sys.stderr)
        return 2

    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU (none visible)", file=sys.stderr)
        return 1
    if args.calibrate_copy:
        n = args.calibrate_copy * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device="cuda:0")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_per_launch": n * 4, "launches": 3}), flush=True)
        return 0

    import dense_gemm_03_amd as dg
    dg.load_library()
    if args.conv:
        print(json.dumps({"convolution": {args.conv: measure_conv(
            args.conv, args.steps, args.warmup, args.conv_route)}}), flush=True)
        return 0

    # Every workload's operands are drawn and copied to the GPU first; then the
    # other configurations are timed, each with its own warm-up, and the
    # headline workload last (W warm-up steps, K timed steps), so that the
    # timed steps run back to back on a GPU that is already busy rather than
    # after seconds of host-side drawing with the GPU idle.
    others = [] if args.no_also else [
        n for n in SECONDARY + (EXTRA if args.all else []) if n != args.workload]
    ctxs = {n: prepare(n) for n in others + [args.workload]}
    if args.all and not args.no_also:
        conv = {}
        for n in CONV:
            conv[n] = measure_conv(n, max(10, args.steps // 5), max(5, args.warmup // 5))
        # its own line, before the result line
        print(json.dumps({"convolution": conv}), flush=True)
    also = {}
    for n in others:
        also[n] = measure(ctxs[n], max(10, args.steps // 2), max(20, args.warmup))
    main_res = measure(ctxs[args.workload], args.steps, args.warmup)

    # the clock each headline workload sustains (outside the timed steps)
    clocks = {}
    if not args.no_also:
        for n, r in [(args.workload, main_res)] + [(n, also[n]) for n in also]:
            clocks[n] = sustained_clock(r["step"])
            log("[bench] %s sustained clock: %s MHz" % (n, clocks[n].get("mhz")))
    del ctxs

    cpu = None
    if not args.no_cpu_baseline:
        log("[bench] oracle baseline on the host")
        cpu = cpu_baseline(args.workload)

    def short(r):
        rf = dict(r["roofline"])
        rf.pop("traffic_source", None)
        for k in ("achieved", "frac", "mfma_cap_gbs", "tflops"):
            if rf.get(k) is not None:
                rf[k] = round(rf[k], 4 if k == "frac" else 1)
        if rf.get("traffic") is not None:
            rf["traffic"] = int(rf["traffic"])
        out = {"shape": "%s %dx%dx%d %s" % (r["dtype"], r["M"], r["N"], r["K"], r["op"]),
               "value": round(r["value"], 2), "ms_per_step": round(r["ms_per_step"], 4),
               "kernel_config": r["kernel_config"], "split_k": r["split_k"], "roofline": rf,
               "per_call_ms": {k: round(v, 4) if k != "calls" else v
                               for k, v in r["per_call_ms"].items()}}
        if r["workload"] in clocks:
            ck = clocks[r["workload"]]
            out["sclk_sustained_mhz"] = ck.get("mhz")
            out["socket_power_w"] = ck.get("socket_power_w")
            for k in ("mclk_mhz", "hotspot_c", "hbm_c"):
                if ck.get(k) is not None:
                    out[k] = ck[k]
        if r["alpha"] != 1.0 or r["beta"] != 0.0 or r["c_dtype"] != "f32":
            out["alpha"], out["beta"], out["c_dtype"] = r["alpha"], r["beta"], r["c_dtype"]
        return out

    w = main_res
    import torch
    prop = torch.cuda.get_device_properties(0)
    line = {
        "metric": "GEMM TFLOP/s and % of MI355X matrix peak (fp32 4096^3, bf16 8192^3)",
        "value": w["value"],
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": w["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w["dtype"],
        "data": "synthetic (seeded uniform[-1,1] fp32 / normal(0,1) rounded to bf16)"
                if OPERAND_VALUES == "workload" else
                "synthetic (%s operands: the workloads' shapes with %s)" % (
                    OPERAND_VALUES, "integers in [-3, 3]" if OPERAND_VALUES == "small-int"
                    else "zeros"),
        "config": {
            "workload": "%s GEMM %dx%dx%d" % (w["dtype"], w["M"], w["N"], w["K"]),
            "name": w["workload"],
            "kernel_config": w["kernel_config"],
            "split_k": w["split_k"],
            "parallelism": "single GPU",
        },
        "roofline": w["roofline"],
        "per_call_ms": w["per_call_ms"],
        "sclk_sustained": clocks.get(args.workload),
        "cpu_baseline": cpu,
        "also": {n: short(r) for n, r in also.items()},
        "device": {"name": prop.name, "arch": getattr(prop, "gcnArchName", None),
                   "compute_units": prop.multi_processor_count,
                   "memory_gib": round(prop.total_memory / 2**30, 1), "hip": torch.version.hip},
    }
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
