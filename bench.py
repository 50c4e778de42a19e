"""Benchmark of the NVFP4 W4A4 quantized-linear hot path on one MI355X.

One step = one pass of the whole path over one batch: online NVFP4 quantization of the activations
X [32768, 5120] (bf16, heavy-tailed synthetic data) followed by the fused Gated DeltaNet input
projection GEMM against six separately calibrated NVFP4 weight segments (q 2048, k 2048, v 4096,
z 4096, b 32, a 32; N = 12352), with per-segment global scales, bf16 outputs for q/k/v/z, the
sigmoid gate for b and the decay gate for a (FP32). Weights are quantized once, before timing, as
they would be offline; the activation global scale is a static calibration input, also set up
before timing. Inputs are resident in HBM when the timed region starts.

Prints one JSON line. `value` is the step's throughput in GEMM TFLOP/s (2 M N K per step time);
`roofline` describes the dominant kernel (the GEMM) against the dense FP16 MFMA peak it runs on;
`roofline_quantize` the quantizer against HBM bandwidth, timed over three rotating copies of the
activation (1 GB of input per round, more than the last-level cache); `cpu_baseline` the CPU oracle on
a bounded sample of the same step, extrapolated linearly in M, on all host threads and on one;
`other_configs` the GEMMs of the other workloads (prefill projection, fused MLP gate+up, the six
decode GEMMs, and the four decode GEMMs with M > 1 again with the weights in the decode layout,
`*_packed`), each over rotating weight copies, with its own roofline.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import nvfp4_w4a4_quantized_quantize_amd as nv  # noqa: E402
import workloads as wl  # noqa: E402

PEAK_F16_MFMA_TFLOPS = 2500.0  # MI355X dense FP16/BF16 matrix peak
PEAK_HBM_GBPS = 8000.0         # MI355X HBM3E
QUANT_BYTES_PER_ELEM = 2.0 + 0.5 + 1.0 / 16.0  # read bf16, write codes + scales


def sources_digest(paths) -> str:
    """sha256 over the given source files, in order (a kernel's file and the headers it includes)."""
    import hashlib
    h = hashlib.sha256()
    for p in paths:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def measured_traffic(kernel: str, workload: str):
    """HBM bytes per launch recorded from rocprofv3 counters for this kernel's sources, else None."""
    try:
        with open(os.path.join(ROOT, "profiles", "traffic.json")) as f:
            rec = json.load(f)[kernel]
        same = sources_digest(rec["sources"]) == rec["sha256"]
    except (OSError, KeyError, ValueError):
        return None
    if not same or rec["workload"] != workload:
        return None
    return rec["read_bytes"] + rec["write_bytes"], {"read_bytes": rec["read_bytes"], "write_bytes": rec["write_bytes"],
                                                    "from": rec["summary"]}


def log(msg: str) -> None:
    print(msg, file=sys.stderr, flush=True)


PEAK_GFX_MHZ = 2400.0  # MI355X peak engine clock, at which the matrix peak above is quoted


def _gfx_mhz(amdsmi, dev):
    """The graphics clock now (MHz): the mean over the XCDs from the GPU metrics table, else the
    driver's current clock level; None when neither reads."""
    try:
        m = amdsmi.amdsmi_get_gpu_metrics_info(dev)
        per_xcd = [v for v in (m.get("current_gfxclks") or []) if isinstance(v, int) and 0 < v < 0xFFFF]
        if per_xcd:
            return float(np.mean(per_xcd))
        v = m.get("current_gfxclk")
        if isinstance(v, int) and 0 < v < 0xFFFF:
            return float(v)
    except Exception:  # noqa: BLE001 - a missing field or an unsupported query leaves the next source
        pass
    try:
        v = amdsmi.amdsmi_get_clock_info(dev, amdsmi.AmdSmiClkType.GFX).get("clk")
        return float(v) if isinstance(v, (int, float)) and v > 0 else None
    except Exception:  # noqa: BLE001
        return None


def clock_under_load(fn, seconds: float = 2.0, period: float = 0.02) -> dict | None:
    """Runs fn back to back for about `seconds` (untimed) while a thread reads the GPU metrics table
    through amdsmi; returns the graphics clock (mean over the XCDs) and socket power over the second
    half of the run, when the clock has settled under the load (the table refreshes about once a
    second), or None when amdsmi cannot read them."""
    import threading
    try:
        import amdsmi
        amdsmi.amdsmi_init()
        devs = amdsmi.amdsmi_get_processor_handles()
    except Exception:  # noqa: BLE001 - no amdsmi, or no access: the line reports no clock
        return None
    if len(devs) != 1:  # more than one GPU visible: which handle is cuda:0 is not known here
        amdsmi.amdsmi_shut_down()
        return None
    samples, done = [], threading.Event()

    def sample():
        t_start = time.perf_counter()
        while not done.is_set():
            v = _gfx_mhz(amdsmi, devs[0])
            try:
                pw = amdsmi.amdsmi_get_gpu_metrics_info(devs[0]).get("current_socket_power")
            except Exception:  # noqa: BLE001
                pw = None
            if v is not None:
                samples.append((time.perf_counter() - t_start, v, pw if isinstance(pw, (int, float)) else None))
            time.sleep(period)

    th = threading.Thread(target=sample, daemon=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    th.start()
    n = 0
    while time.perf_counter() - t0 < seconds:
        for _ in range(4):
            fn()
        n += 4
        torch.cuda.synchronize()
    done.set()
    th.join()
    amdsmi.amdsmi_shut_down()
    late = [x for x in samples if x[0] >= seconds / 2]
    if len(late) < 5:
        return None
    mhz = [x[1] for x in late]
    pw = [x[2] for x in late if x[2] is not None]
    return {"mean_mhz": float(np.mean(mhz)), "min_mhz": float(np.min(mhz)), "max_mhz": float(np.max(mhz)),
            "socket_power_w": float(np.mean(pw)) if pw else None, "launches": n, "seconds": seconds,
            "source": "amdsmi GPU metrics table (graphics clock, mean over the XCDs; refreshed about once a "
                      "second), second half of a run of back-to-back launches"}


def to_dev_bf16(bits: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(bits.view(np.int16)).cuda().view(torch.bfloat16)


class Step:
    """Device buffers and the launches of one step of the fused GDN input projection."""

    def __init__(self, case: wl.GemmCase, seed: int = 0, copies: int = 1, packed: bool = False):
        self.case = case
        self.packed = packed
        M, K, N = case.M, case.K, case.N
        dev = torch.device("cuda")
        t0 = time.time()
        self.x_bits = wl.draw_x(case, seed)
        self.x = to_dev_bf16(self.x_bits)
        log(f"[setup] X {self.x_bits.shape} drawn and uploaded in {time.time() - t0:.1f}s")
        # offline: weights per segment -> global scale -> NVFP4, concatenated along N
        self.w_codes, self.w_scales = nv.alloc_nvfp4(N, K, dev)
        self.g_w, self.w_bits = [], []
        n0 = 0
        for s, seg in enumerate(case.segments):
            wb = wl.draw_w(case, s, seed)
            self.w_bits.append(wb)
            wt = to_dev_bf16(wb)
            g = float(nv.global_scale(wt).item())
            nv.quantize(wt, g, self.w_codes[n0:n0 + seg.n], self.w_scales[n0:n0 + seg.n])
            self.g_w.append(g)
            n0 += seg.n
        # extra copies of the quantized weights, used in turn by consecutive steps (as consecutive
        # layers would), so that a small working set is still read from HBM
        self.w_copies = [(self.w_codes, self.w_scales)]
        for _ in range(copies - 1):
            self.w_copies.append((self.w_codes.clone(), self.w_scales.clone()))
        # the decode weight layout of each copy, repacked once (offline) for gemm_packed
        self.w_packed = [nv.pack_weights(c, sc) for c, sc in self.w_copies] if packed else []
        self.calls = 0
        # static activation calibration
        self.g_a = float(nv.global_scale(self.x).item())
        self.a_codes, self.a_scales = nv.alloc_nvfp4(M, K, dev)
        self.segments = []
        for s, seg in enumerate(case.segments):
            dt = torch.float32 if seg.out_dtype == wl.OUT_F32 else torch.bfloat16
            epi = {wl.EPI_NONE: "none", wl.EPI_SIGMOID: "sigmoid", wl.EPI_GDN_DECAY: "gdn_decay"}[seg.epilogue]
            a_log = dt_bias = None
            if seg.epilogue == wl.EPI_GDN_DECAY:
                al, db = wl.draw_gate_params(case, s, seed)
                a_log, dt_bias = torch.from_numpy(al).cuda(), torch.from_numpy(db).cuda()
            out = torch.empty((M, seg.n), dtype=dt, device=dev)
            self.segments.append(nv.Segment(seg.n, self.g_w[s], epi, dt, a_log, dt_bias, out))
        need = nv.lib().nvfp4_gemm_workspace_bytes(M, case.N, K)
        self.workspace = torch.empty(need, dtype=torch.uint8, device=dev) if need else None
        torch.cuda.synchronize()
        log(f"[setup] weights quantized, g_a = {self.g_a:.6g}, setup {time.time() - t0:.1f}s")

    def quantize(self):
        nv.quantize(self.x, self.g_a, self.a_codes, self.a_scales)

    def gemm(self):
        i = self.calls % len(self.w_copies)
        self.calls += 1
        if self.packed:
            nv.gemm_packed(self.a_codes, self.a_scales, self.g_a, self.w_packed[i], self.case.N, self.segments,
                           workspace=self.workspace)
        else:
            wc, ws = self.w_copies[i]
            nv.gemm(self.a_codes, self.a_scales, self.g_a, wc, ws, self.segments, workspace=self.workspace)


def run_gpu(step: Step, steps: int, warmup: int, flush_mb: int) -> dict:
    """Time `steps` steps with HIP events on the library's stream. With flush_mb > 0 a buffer of that
    size is overwritten before every step (outside the timed kernels) so that a working set smaller
    than the 256 MB last-level cache is read from HBM, and the step time is the sum of the kernels."""
    flush = torch.empty(flush_mb * (1 << 20) // 4, dtype=torch.float32, device="cuda") if flush_mb else None
    for _ in range(warmup):
        step.quantize()
        step.gemm()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()  # the library launches on this stream
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        if flush is not None:
            flush.zero_()
        ev[i][0].record(stream)
        step.quantize()
        ev[i][1].record(stream)
        step.gemm()
        ev[i][2].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    q_ms = [ev[i][0].elapsed_time(ev[i][1]) for i in range(steps)]
    g_ms = [ev[i][1].elapsed_time(ev[i][2]) for i in range(steps)]
    # the quantizer alone, 20 back-to-back launches (its event time inside a step also holds the gap
    # after the previous step's GEMM); the 335 MB activation does not fit the 256 MB last-level cache
    qa, qb = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    qa.record(stream)
    for _ in range(20):
        step.quantize()
    qb.record(stream)
    torch.cuda.synchronize()
    quant_iso_ms = qa.elapsed_time(qb) / 20
    # the GEMM alone, back to back over the weight copies (only meaningful when there are several:
    # a single copy would be served from the last-level cache)
    n_iso = max(steps, 4 * len(step.w_copies))
    qa.record(stream)
    for _ in range(n_iso):
        step.gemm()
    qb.record(stream)
    torch.cuda.synchronize()
    gemm_iso_ms = qa.elapsed_time(qb) / n_iso
    if flush is None:
        step_ms = ev[0][0].elapsed_time(ev[-1][2]) / steps
    else:
        step_ms = float(np.mean(np.array(q_ms) + np.array(g_ms)))
    return {"wall_s": wall, "step_ms": step_ms, "quant_ms": float(np.mean(q_ms)), "quant_iso_ms": quant_iso_ms,
            "gemm_iso_ms": gemm_iso_ms,
            "gemm_ms": float(np.mean(g_ms)), "quant_ms_med": float(np.median(q_ms)),
            "gemm_ms_med": float(np.median(g_ms)),
            "gemm_ms_p10_p90": [float(np.percentile(g_ms, 10)), float(np.percentile(g_ms, 90))],
            "quant_ms_p10_p90": [float(np.percentile(q_ms, 10)), float(np.percentile(q_ms, 90))]}


def time_quantizer_rotating(step: Step, copies: int = 3, reps: int = 10) -> dict:
    """The quantizer over `copies` distinct activation tensors (and as many output buffers) in turn,
    back to back: with three copies of the 32K-token activation that is 1.0 GB of input per round,
    four times the 256 MB last-level cache, so every launch streams its input from HBM."""
    xs = [step.x] + [step.x.clone() for _ in range(copies - 1)]
    outs = [(step.a_codes, step.a_scales)] + [nv.alloc_nvfp4(step.case.M, step.case.K, "cuda")
                                              for _ in range(copies - 1)]
    fn = lambda i: nv.quantize(xs[i % copies], step.g_a, *outs[i % copies])  # noqa: E731
    for i in range(2 * copies):
        fn(i)
    torch.cuda.synchronize()
    ms = _time_loop(fn, reps * copies)
    in_bytes = copies * step.case.M * step.case.K * 2
    del xs, outs
    torch.cuda.empty_cache()
    return {"ms": ms, "rotation_bytes": in_bytes, "copies": copies, "launches": reps * copies}


def decode_kernel_name(M: int, K: int, packed: bool = False) -> str:
    """The kernel the library runs for M <= 32 activation rows: with row-major weights the
    weight-streaming GEMV for one row (K from 16 to 32768), else (and always with packed weights) the
    skinny kernel."""
    if packed:
        return "gemm_skinny_kernel (packed weights)"
    return "gemm_gemv_kernel" if M == 1 and 16 <= K <= 32768 else "gemm_skinny_kernel"


def gemm_roofline(case: wl.GemmCase, ms: float, packed: bool = False) -> dict:
    """TFLOP/s, GB/s and the roofline the GEMM of `case` runs against: the dense FP16 MFMA peak above
    the ridge point (peak FLOP/s per HBM byte/s), HBM bandwidth below it."""
    M, N, K = case.M, case.N, case.K
    flops = 2.0 * M * N * K
    out_bytes = sum(M * s.n * (4 if s.out_dtype == wl.OUT_F32 else 2) for s in case.segments)
    nbytes = 0.5625 * (M + N) * K + out_bytes  # codes + scales of A and W, plus the outputs
    tflops = flops / (ms * 1e-3) / 1e12
    gbps = nbytes / (ms * 1e-3) / 1e9
    if flops / nbytes >= PEAK_F16_MFMA_TFLOPS * 1e12 / (PEAK_HBM_GBPS * 1e9):
        roof = {"bound": "mfma", "achieved": tflops, "peak": PEAK_F16_MFMA_TFLOPS, "unit": "TFLOP/s",
                "frac": tflops / PEAK_F16_MFMA_TFLOPS}
    else:
        roof = {"bound": "hbm", "achieved": gbps, "peak": PEAK_HBM_GBPS, "unit": "GB/s", "frac": gbps / PEAK_HBM_GBPS}
    if M > 64:
        kernel = "gemm_kernel"
    elif M > 32:
        kernel = "gemm_wide_kernel" + (" + gemm_wide_reduce_kernel" if nv.lib().nvfp4_gemm_workspace_bytes(M, N, K)
                                       else "") + (" (packed weights)" if packed else "")
    else:
        kernel = decode_kernel_name(M, K, packed)
    roof.update({"kernel": kernel, "avg_ms": ms, "algorithmic_flop": flops, "algorithmic_bytes": nbytes})
    return {"ms": ms, "tflops": tflops, "gbps": gbps, "roofline": roof}


def weight_copies(case: wl.GemmCase) -> int:
    """Copies of the quantized weights a timing rotates through: 1 when a step's working set exceeds
    1 GiB, else enough copies for 1 GiB of weights (as consecutive layers would), at most 64."""
    work_mb = (case.M * case.K * 2.5625 + (case.M + case.N) * case.K * 0.5625 +
               sum(case.M * sg.n * 4 for sg in case.segments)) / 2 ** 20
    w_mb = case.N * case.K * 0.5625 / 2 ** 20
    return 1 if work_mb > 1024 else int(min(64, max(2, np.ceil(1024 / w_mb))))


OTHER_CONFIGS = ("C2", "C4", "C3_up_1", "C3_up_16", "C3_up_64", "C3_down_1", "C3_down_16", "C3_down_64")
# decode GEMMs also timed with the weights in the decode layout (nvfp4_gemm_packed)
PACKED_CONFIGS = ("C3_up_16", "C3_up_64", "C3_down_16", "C3_down_64")


def bench_other_configs(reps: int) -> dict:
    """The GEMMs of the other workloads, each timed back to back over rotating weight copies (HIP
    events on the library's stream, after a few untimed calls): prefill projection 4096x5120x5120,
    fused MLP gate+up 8192x34816x5120, and the six decode GEMMs (HBM-bound weight streaming)."""
    res = {}
    for key, packed in [(k, False) for k in OTHER_CONFIGS] + [(k, True) for k in PACKED_CONFIGS]:
        case = wl.ALL[key]
        step = Step(case, copies=weight_copies(case), packed=packed)
        step.quantize()
        n = max(reps, 4 * len(step.w_copies))
        _settle(lambda i: step.gemm(), 0.1)
        ms = _time_loop(lambda i: step.gemm(), n)
        r = gemm_roofline(case, ms, packed)
        r.update({"workload": case.name + ("_packed" if packed else ""), "M": case.M, "N": case.N, "K": case.K,
                  "weight_copies": len(step.w_copies), "launches": n})
        if r["roofline"]["bound"] == "mfma":
            clk = clock_under_load(step.gemm, 1.5)
            if clk is not None:
                r["roofline"]["clock"] = clk
                r["roofline"]["frac_at_clock"] = r["tflops"] / (PEAK_F16_MFMA_TFLOPS * clk["mean_mhz"] / PEAK_GFX_MHZ)
        res[key + ("_packed" if packed else "")] = r
        log(f"[gpu] {case.name}: {ms * 1e3:.1f} us, {r['tflops']:.1f} TFLOP/s, {r['gbps']:.0f} GB/s "
            f"({r['roofline']['bound']} {100 * r['roofline']['frac']:.1f}%)")
        del step
        torch.cuda.empty_cache()
    return res


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def run_cpu_baseline(step: Step, rows_quant: int, rows_gemm: int) -> dict:
    """The CPU oracle on a bounded sample of the same step, extrapolated linearly in M."""
    import oracle
    case = step.case
    M, N, K = case.M, case.N, case.K
    # oracle-side operands: weights quantized by the oracle itself (offline, untimed)
    wq = [oracle.quantize(wb, oracle.global_scale(wb)) for wb in step.w_bits]
    w_codes = np.concatenate([c for c, _ in wq])
    w_scales = np.concatenate([s for _, s in wq])
    g_w = np.array([oracle.global_scale(wb) for wb in step.w_bits], np.float32)
    g_a = oracle.global_scale(step.x_bits)
    bounds = case.seg_bounds
    xs = step.x_bits[:rows_quant]
    t0 = time.perf_counter()
    a_codes, a_scales = oracle.quantize(xs, g_a)
    t_quant = time.perf_counter() - t0
    rows = np.arange(rows_gemm)
    t0 = time.perf_counter()
    oracle.gemm_rows(a_codes, a_scales, g_a, w_codes, w_scales, bounds, g_w, rows[:1])
    t_one = time.perf_counter() - t0
    t0 = time.perf_counter()
    y, T = oracle.gemm_rows(a_codes, a_scales, g_a, w_codes, w_scales, bounds, g_w, rows)
    t_many = time.perf_counter() - t0
    per_row = max(t_many - t_one, 1e-9) / max(rows_gemm - 1, 1)
    fixed = max(t_one - per_row, 0.0)
    t_full = t_quant / rows_quant * M + fixed + per_row * M
    # sanity: the timed GPU step's outputs on the sampled rows against the oracle (FP32 segments)
    checks = {}
    for s, seg in enumerate(step.segments):
        lo, hi = bounds[s], bounds[s + 1]
        got = step.segments[s].out[:rows_gemm].float().cpu().numpy().astype(np.float64)
        ys, Ts = y[:, lo:hi], T[:, lo:hi]
        if seg.epilogue == "none":
            tol = 2.0 ** -20 * Ts + (2.0 ** -8 * (np.abs(ys) + 2.0 ** -20 * Ts) if seg.out_dtype == torch.bfloat16 else 0)
            checks[case.segments[s].name] = bool((np.abs(got - ys) <= tol).all())
        elif seg.epilogue == "sigmoid":
            b = oracle.sigmoid(ys)
            checks[case.segments[s].name] = bool((np.abs(got - b) <= b * (1 - b) * 2.0 ** -20 * Ts + 2.0 ** -20 * b + 2.0 ** -126).all())
        else:
            al = seg.A_log.cpu().numpy()
            db = seg.dt_bias.cpu().numpy()
            a = oracle.gdn_decay(ys, al, db)
            sig = 1 / (1 + np.exp(-(ys + db.astype(np.float64))))
            bound = a * np.exp(al.astype(np.float64)) * sig * 2.0 ** -20 * Ts + 2.0 ** -20 * a * (1 + np.abs(np.log(np.maximum(a, 1e-300)))) + 2.0 ** -126
            checks[case.segments[s].name] = bool((np.abs(got - a) <= bound).all())
    codes_ok = bool((step.a_codes[:rows_quant].cpu().numpy() == a_codes).all()
                    and (step.a_scales[:rows_quant].cpu().numpy() == a_scales).all())
    threads = oracle.num_threads()
    # the same oracle on one thread: quantizer on 2048 rows, GEMM on 32 rows (all N), extrapolated
    oracle.set_num_threads(1)
    try:
        q1_rows, g1_rows = min(2048, rows_quant), min(32, rows_gemm)
        t0 = time.perf_counter()
        oracle.quantize(xs[:q1_rows], g_a)
        t_q1 = time.perf_counter() - t0
        t0 = time.perf_counter()
        oracle.gemm_rows(a_codes, a_scales, g_a, w_codes, w_scales, bounds, g_w, rows[:g1_rows])
        t_g1 = time.perf_counter() - t0
    finally:
        oracle.set_num_threads(threads)
    t_full1 = t_q1 / q1_rows * M + t_g1 / g1_rows * M
    q_bytes_row = K * QUANT_BYTES_PER_ELEM
    return {
        "value": 2.0 * M * N * K / t_full / 1e12, "unit": "TFLOP/s", "cores": threads,
        "kind": "oracle",
        "sample": (f"oracle quantize of {rows_quant} rows + exact GEMM of {rows_gemm} rows (all N) of the "
                   f"{M}x{N}x{K} step, extrapolated linearly to M={M}; measured "
                   f"{t_quant:.2f}s + {t_many:.2f}s, extrapolated full step {t_full:.1f}s"),
        "cpu_model": cpu_model(), "os_cpu_count": os.cpu_count(),
        "quantize_gbps": q_bytes_row * rows_quant / t_quant / 1e9,
        "single_thread": {
            "value": 2.0 * M * N * K / t_full1 / 1e12, "unit": "TFLOP/s", "cores": 1,
            "quantize_gbps": q_bytes_row * q1_rows / t_q1 / 1e9,
            "gemm_tflops": 2.0 * g1_rows * N * K / t_g1 / 1e12,
            "sample": (f"one thread: oracle quantize of {q1_rows} rows ({t_q1:.2f}s) + exact GEMM of {g1_rows} rows "
                       f"({t_g1:.2f}s), extrapolated to the full step: {t_full1:.0f}s")},
        "parity_sample": {"codes_scales_bit_exact": codes_ok, **checks},
    }


# ----------------------------------------------------------------------- serving-path companions
COMPANIONS = ("kv_cache", "rmsnorm_quantize", "gdn_prefill", "gdn_decode")
PEAK_F32_VALU_TFLOPS = 157.3  # MI355X FP32 vector peak (256 CUs, 2.4 GHz)


def _time_loop(fn, n: int) -> float:
    """Milliseconds per call of fn(i) over n back-to-back calls on the current stream (HIP events)."""
    stream = torch.cuda.current_stream()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record(stream)
    for i in range(n):
        fn(i)
    b.record(stream)
    torch.cuda.synchronize()
    return a.elapsed_time(b) / n


def _settle(fn, seconds: float = 0.2) -> None:
    """Untimed: call fn(i) back to back for about `seconds` of wall time, so that the GPU's clocks have
    left their idle state before a kernel of a fraction of a millisecond is timed."""
    t0, i = time.perf_counter(), 0
    while time.perf_counter() - t0 < seconds:
        fn(i)
        i += 1
        if i % 64 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()


def library_gemm(step: Step, M: int, N: int, K: int, rounds: int = 4, reps: int = 10) -> dict:
    """Dense FP16 and BF16 GEMMs of the same shape through torch.matmul (hipBLASLt on ROCm), timed in
    rounds alternating with the NVFP4 GEMM of `step`: a same-process, same-clock comparison. The dense
    operands are random normal; the library GEMMs dequantize nothing and have no segment epilogue."""
    a16 = torch.randn(M, K, device="cuda", dtype=torch.float16)
    w16 = torch.randn(N, K, device="cuda", dtype=torch.float16)
    y16 = torch.empty(M, N, device="cuda", dtype=torch.float16)
    abf, wbf = a16.to(torch.bfloat16), w16.to(torch.bfloat16)
    ybf = torch.empty(M, N, device="cuda", dtype=torch.bfloat16)
    runs = {"nvfp4_gemm": lambda i: step.gemm(),
            "fp16_matmul": lambda i: torch.matmul(a16, w16.t(), out=y16),
            "bf16_matmul": lambda i: torch.matmul(abf, wbf.t(), out=ybf)}
    times = {k: [] for k in runs}
    for _ in range(rounds):
        for k, fn in runs.items():
            for i in range(3):
                fn(i)
            torch.cuda.synchronize()
            times[k].append(_time_loop(fn, reps))
    flops = 2.0 * M * N * K
    res = {k: {"best_ms": min(v), "tflops": flops / (min(v) * 1e-3) / 1e12} for k, v in times.items()}
    log("[gpu] same process: " + ", ".join(f"{k} {v['best_ms']:.3f} ms ({v['tflops']:.0f} TFLOP/s)"
                                           for k, v in res.items()))
    del a16, w16, y16, abf, wbf, ybf
    torch.cuda.empty_cache()
    res["note"] = "best of 4 rounds of 10 back-to-back calls; torch.matmul on dense random operands"
    return res


def copy_ceiling_gbps(mb: int = 1024, reps: int = 10) -> float:
    """Bytes moved (read + write) per second by a plain device-to-device copy of `mb` MiB: the
    practical streaming ceiling of HBM on this machine, reported beside the nominal peak."""
    n = mb * (1 << 20) // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    ms = _time_loop(lambda i: dst.copy_(src), reps)
    del src, dst
    return 2.0 * n * 4 / (ms * 1e-3) / 1e9


def bench_kv_cache(steps: int, warmup: int, cpu: bool) -> dict:
    """One step = the FP8 KV-cache write of a 32K-token prefill for every attention layer (K and V
    of 16 layers, each quantized with its own static scale), then the read of all of it back to
    bf16. Layer l's tensors are the two seeded base draws times 2^(l/4 - 2) (rounded to bf16), so
    the 32 tensors (3.2 GB with their codes) stream from HBM."""
    import oracle
    case = wl.KV
    rows, cols = case.tokens, case.cols
    base = [to_dev_bf16(wl.draw_kv(case, w)) for w in (0, 1)]
    xs, ss, qs, ys = [], [], [], []
    for layer in range(case.layers):
        for w in (0, 1):
            x = (base[w].float() * float(2.0 ** (layer / 4 - 2))).to(torch.bfloat16)
            xs.append(x)
            ss.append(float(nv.kv_scale(x).item()))  # static calibration, shipped with the model
            qs.append(torch.empty((rows, cols), dtype=torch.uint8, device="cuda"))
            ys.append(torch.empty((rows, cols), dtype=torch.bfloat16, device="cuda"))
    del base
    n = len(xs)
    quant = lambda i: nv.kv_quantize(xs[i % n], ss[i % n], out=qs[i % n])  # noqa: E731
    deq = lambda i: nv.kv_dequantize(qs[i % n], ss[i % n], out=ys[i % n])  # noqa: E731
    for i in range(warmup * n):
        quant(i)
        deq(i)
    torch.cuda.synchronize()
    q_ms = _time_loop(quant, steps * n)
    d_ms = _time_loop(deq, steps * n)
    elems = rows * cols
    q_gbps = 3.0 * elems / (q_ms * 1e-3) / 1e9
    d_gbps = 3.0 * elems / (d_ms * 1e-3) / 1e9
    log(f"[gpu] kv_quantize {q_ms * 1e3:.1f} us/tensor ({q_gbps:.0f} GB/s), "
        f"kv_dequantize {d_ms * 1e3:.1f} us/tensor ({d_gbps:.0f} GB/s)")
    # sampled parity: layer 0's K cache, first 2048 tokens, against the oracle from the same input
    xb = xs[0][:2048].contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
    parity = bool((qs[0][:2048].cpu().numpy() == oracle.kv_quantize(xb, np.float32(ss[0]))).all())
    out = {
        "metric": "FP8 E4M3 KV-cache quantize GB/s (static per-tensor scales), % of HBM roofline",
        "value": q_gbps, "unit": "GB/s", "n_gpus": 1, "steps": steps, "warmup": warmup,
        "ms_per_step": (q_ms + d_ms) * n, "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16 in, e4m3 out (f32 arithmetic)", "data": "synthetic (seeded normal K/V, hot key channels)",
        "config": {"workload": case.name, "tensors": n, "rows": rows, "cols": cols},
        "kv_dequantize_gbps": d_gbps,
        "roofline": {"bound": "hbm", "achieved": q_gbps, "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                     "frac": q_gbps / PEAK_HBM_GBPS, "traffic": None, "kernel": "kv_quantize_kernel",
                     "avg_ms": q_ms, "algorithmic_bytes": 3 * elems},
        "roofline_dequantize": {"bound": "hbm", "achieved": d_gbps, "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                                "frac": d_gbps / PEAK_HBM_GBPS, "kernel": "kv_dequantize_kernel", "avg_ms": d_ms,
                                "algorithmic_bytes": 3 * elems},
        "parity_sample": {"layer0_K_first_2048_tokens_bit_exact": parity},
    }
    if cpu:
        rows_cpu = 8192
        xb = xs[0][:rows_cpu].contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
        t0 = time.perf_counter()
        oracle.kv_quantize(xb, np.float32(ss[0]))
        t = time.perf_counter() - t0
        out["cpu_baseline"] = {"value": 3.0 * rows_cpu * cols / t / 1e9, "unit": "GB/s",
                               "cores": oracle.num_threads(), "kind": "oracle",
                               "sample": f"oracle kv_quantize of {rows_cpu} x {cols} (one tensor's first "
                                         f"{rows_cpu} tokens), {t:.2f}s"}
    return out


def bench_rmsnorm_quantize(steps: int, warmup: int, cpu: bool) -> dict:
    """One step = RMSNorm of X [32768, 5120] fused with the NVFP4 quantizer of its output (static g,
    calibrated before timing); also timed: the same two steps as separate kernels (norm writing bf16
    y, then the quantizer reading it)."""
    import oracle
    case = wl.NORM
    rows, K = case.rows, case.K
    x_bits = wl.draw_norm_x(case)
    w_bits = wl.draw_norm_weight(case)
    x, w = to_dev_bf16(x_bits), to_dev_bf16(w_bits)
    eps = 1e-6
    y = torch.empty((rows, K), dtype=torch.bfloat16, device="cuda")
    codes, scales = nv.alloc_nvfp4(rows, K, "cuda")
    g0 = 1.0
    nv.rmsnorm_quantize(x, w, eps, g0, codes, scales, y=y)
    g = float(nv.global_scale(y).item())  # static calibration of the consuming module
    fused = lambda i: nv.rmsnorm_quantize(x, w, eps, g, codes, scales)  # noqa: E731

    def unfused(i):
        nv.rmsnorm_quantize(x, w, eps, g, codes, scales, y=y)
        nv.quantize(y, g, codes, scales)
    for i in range(warmup):
        fused(i)
        unfused(i)
    torch.cuda.synchronize()
    _settle(fused)
    f_ms = _time_loop(fused, steps)
    _settle(unfused)
    u_ms = _time_loop(unfused, steps)
    alg = rows * K * (2.0 + 0.5625) + 2 * K
    f_gbps = alg / (f_ms * 1e-3) / 1e9
    log(f"[gpu] rmsnorm+quantize fused {f_ms:.3f} ms ({f_gbps:.0f} GB/s), as two kernels {u_ms:.3f} ms")
    yb = oracle.rmsnorm(x_bits[:256], w_bits, np.float32(eps))[0]
    c_ref, s_ref = oracle.quantize(yb, np.float32(g))
    parity = bool((codes[:256].cpu().numpy() == c_ref).all() and (scales[:256].cpu().numpy() == s_ref).all())
    out = {
        "metric": "RMSNorm + NVFP4 quantize (fused) GB/s, % of HBM roofline",
        "value": f_gbps, "unit": "GB/s", "n_gpus": 1, "steps": steps, "warmup": warmup, "ms_per_step": f_ms,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16 in, NVFP4 out (f64 row sums, f32 rounding steps)",
        "data": "synthetic (seeded heavy-tailed activations with outlier channels)",
        "config": {"workload": case.name, "rows": rows, "K": K},
        "two_kernel_ms": u_ms, "fused_speedup": u_ms / f_ms,
        "roofline": {"bound": "hbm", "achieved": f_gbps, "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                     "frac": f_gbps / PEAK_HBM_GBPS, "traffic": None, "kernel": "rmsnorm_quantize_kernel",
                     "avg_ms": f_ms, "algorithmic_bytes": alg},
        "parity_sample": {"first_256_rows_bit_exact": parity},
    }
    if cpu:
        rows_cpu = 4096
        t0 = time.perf_counter()
        yb = oracle.rmsnorm(x_bits[:rows_cpu], w_bits, np.float32(eps))[0]
        oracle.quantize(yb, np.float32(g))
        t = time.perf_counter() - t0
        out["cpu_baseline"] = {"value": (rows_cpu * K * 2.5625) / t / 1e9, "unit": "GB/s",
                               "cores": oracle.num_threads(), "kind": "oracle",
                               "sample": f"oracle rmsnorm + quantize of the first {rows_cpu} rows, {t:.2f}s"}
    return out


def bench_gdn(case, steps: int, warmup: int, cpu: bool) -> dict:
    """The Gated DeltaNet recurrence over one batch: gdn_prefill = one sequence of 32768 tokens, all 32
    value heads (FP32-accurate arithmetic, counted as the recurrence's 6 D^2 flops per token and head:
    S^T k, the update, S^T q; timed over the whole call, both kernels of the chunked form);
    gdn_decode = one token for each of 64 sequences, which streams every head's 64 KB state in and out."""
    import oracle
    B, T, Hv, D = case.B, case.T, case.Hv, case.D
    q, k, v, a, b = wl.draw_gdn(case)
    qd, kd, vd = to_dev_bf16(q), to_dev_bf16(k), to_dev_bf16(v)
    ad, bd = torch.from_numpy(a).cuda(), torch.from_numpy(b).cuda()
    # decode: rotate 4 state buffers (4 x 268 MB) so each step streams its state from HBM
    copies = 1 if T > 1 else 4
    states = [torch.zeros((B, Hv, D, D), dtype=torch.float32, device="cuda") for _ in range(copies)]
    o = torch.empty((B * T, Hv * D), dtype=torch.float32, device="cuda")
    need = nv.lib().nvfp4_gdn_workspace_bytes(B, T, Hv, case.Hk, D)
    ws = torch.empty(max(need, 1), dtype=torch.uint8, device="cuda")
    run = lambda i: nv.gdn_recurrence(qd, kd, vd, ad, bd, states[i % copies], B, T, o=o, workspace=ws)  # noqa: E731
    for i in range(warmup):
        run(i)
    torch.cuda.synchronize()
    ms = _time_loop(run, steps)
    flops = 6.0 * D * D * Hv * B * T
    tflops = flops / (ms * 1e-3) / 1e12
    state_bytes = 2.0 * B * Hv * D * D * 4
    in_bytes = B * T * (2 * 16 * D * 2 + Hv * D * 2 + 2 * Hv * 4) + B * T * Hv * D * 4
    gbps = (state_bytes + in_bytes) / (ms * 1e-3) / 1e9
    log(f"[gpu] gdn {case.name}: {ms:.3f} ms per call, {B * T / (ms * 1e-3) / 1e6:.2f} M tokens/s, "
        f"{tflops:.2f} TFLOP/s, {gbps:.0f} GB/s")
    # sampled parity: the first 64 tokens of sequence 0, all heads, from a zero state
    n = min(T, 64)
    st = torch.zeros((1, Hv, D, D), dtype=torch.float32, device="cuda")
    og = nv.gdn_recurrence(qd[:n], kd[:n], vd[:n], ad[:n], bd[:n], st, 1, n).cpu().numpy().astype(np.float64)
    o64, _ = oracle.gdn_recurrence(q[:n], k[:n], v[:n], a[:n], b[:n], 1, n)
    o32, _ = oracle.gdn_recurrence(q[:n], k[:n], v[:n], a[:n], b[:n], 1, n, f32=True)
    parity = bool(np.abs(og - o64).max() <= 8 * np.abs(o32 - o64).max() + 2.0 ** -22 * np.abs(o64).max())
    if T > 1:
        # the recurrence's FP32 work against the FP32 peak (matrix and vector alike on MI355X); calls of
        # 32 tokens or more run the chunked form (a parallel pre-pass, then the chunk-sequential kernel)
        chunked = nv.lib().nvfp4_gdn_workspace_bytes(B, T, Hv, case.Hk, D) > 0
        roof = {"bound": "mfma" if chunked else "alu", "achieved": tflops, "peak": PEAK_F32_VALU_TFLOPS,
                "unit": "TFLOP/s", "frac": tflops / PEAK_F32_VALU_TFLOPS, "traffic": None,
                "kernel": "gdn_chunk_prep_kernel + gdn_chunk_kernel" if chunked else "gdn_recurrence_kernel",
                "avg_ms": ms, "algorithmic_flop": flops}
        metric, value, unit = "Gated DeltaNet recurrence tokens/s (FP32, 32 heads)", B * T / (ms * 1e-3), "tokens/s"
    else:
        roof = {"bound": "hbm", "achieved": gbps, "peak": PEAK_HBM_GBPS, "unit": "GB/s", "frac": gbps / PEAK_HBM_GBPS,
                "traffic": None, "kernel": "gdn_recurrence_kernel", "avg_ms": ms,
                "algorithmic_bytes": state_bytes + in_bytes}
        metric, value, unit = "Gated DeltaNet decode step GB/s (state in + out), % of HBM roofline", gbps, "GB/s"
    out = {"metric": metric, "value": value, "unit": unit, "n_gpus": 1, "steps": steps, "warmup": warmup,
           "ms_per_step": ms, "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32",
           "data": "synthetic (seeded unit-norm q/k, normal v, decays over horizons 3..1e5 tokens)",
           "config": {"workload": case.name, "B": B, "T": T, "Hv": Hv, "Hk": case.Hk, "D": D},
           "tflops": tflops, "gbps": gbps, "roofline": roof,
           "parity_sample": {"first_64_tokens_within_fp32_bound": parity}}
    if cpu:
        Tc = T  # the whole batch: a few seconds of the double-precision recurrence
        t0 = time.perf_counter()
        oracle.gdn_recurrence(q[:Tc * B], k[:Tc * B], v[:Tc * B], a[:Tc * B], b[:Tc * B], B, Tc) if T == 1 else \
            oracle.gdn_recurrence(q[:Tc], k[:Tc], v[:Tc], a[:Tc], b[:Tc], 1, Tc)
        t = time.perf_counter() - t0
        toks = Tc * B if T == 1 else Tc
        cpu_v = toks / t if T > 1 else 6.0 * D * D * Hv * toks / t / 1e12
        out["cpu_baseline"] = {"value": cpu_v if T > 1 else (state_bytes / B * toks) / t / 1e9,
                               "unit": "tokens/s" if T > 1 else "GB/s", "cores": oracle.num_threads(),
                               "kind": "oracle",
                               "sample": f"oracle recurrence (double) over {toks} tokens x {Hv} heads, {t:.2f}s"}
    return out


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="C5", choices=sorted(wl.ALL) + list(COMPANIONS))
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--packed", action="store_true",
                    help="decode GEMM workloads (M <= 64): weights in the decode layout (nvfp4_gemm_packed)")
    ap.add_argument("--cpu-rows-quant", type=int, default=32768)
    ap.add_argument("--cpu-rows-gemm", type=int, default=4096)
    ap.add_argument("--flush-mb", type=int, default=-1,
                    help="overwrite a buffer of this size before each step (-1: none)")
    ap.add_argument("--calib-copy-mb", type=int, default=0,
                    help="also run one device copy of this many MiB (counter calibration runs)")
    ap.add_argument("--no-extras", action="store_true",
                    help="skip the other configurations' GEMM timings (profiling runs)")
    ap.add_argument("--library-gemm", action="store_true",
                    help="also time torch.matmul (hipBLASLt) on dense FP16 and BF16 operands of the same "
                         "shape, alternating with the NVFP4 GEMM in this process")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU: the hot path has no multi-GPU part here (asked for --gpus {args.gpus}).",
              file=sys.stderr)
        return 2
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 2
    nv.lib()  # fail loudly if the HIP library is missing
    if args.workload in COMPANIONS:
        fn = {"kv_cache": bench_kv_cache, "rmsnorm_quantize": bench_rmsnorm_quantize,
              "gdn_prefill": lambda *a: bench_gdn(wl.GDN_PREFILL, *a),
              "gdn_decode": lambda *a: bench_gdn(wl.GDN_DECODE, *a)}[args.workload]
        print(json.dumps(fn(args.steps, args.warmup, not args.no_cpu_baseline)), flush=True)
        return 0
    case = wl.ALL[args.workload]
    # a step whose working set fits the 256 MB last-level cache would be served from it: such steps
    # rotate through copies of the weights, 1 GiB in all
    copies = weight_copies(case)
    if args.packed and case.M > 64:
        print("--packed serves the decode GEMMs (M <= 64)", file=sys.stderr)
        return 2
    step = Step(case, copies=copies, packed=args.packed)
    if args.calib_copy_mb:
        n = args.calib_copy_mb * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    log(f"[gpu] warmup {args.warmup}, timing {args.steps} steps")
    flush_mb = max(args.flush_mb, 0)
    r = run_gpu(step, args.steps, args.warmup, flush_mb)
    # the GEMM's average launch duration: inside the step when the weights are not rotated, else
    # back to back over the copies (a few microseconds of event overhead per step would count)
    gemm_ms = r["gemm_ms"] if copies == 1 else r["gemm_iso_ms"]
    M, N, K = case.M, case.N, case.K
    flops = 2.0 * M * N * K
    gemm_tflops = flops / (gemm_ms * 1e-3) / 1e12
    q_bytes = QUANT_BYTES_PER_ELEM * M * K
    qrot = time_quantizer_rotating(step)
    q_gbps = q_bytes / (qrot["ms"] * 1e-3) / 1e9
    q_gbps_same_x = q_bytes / (r["quant_iso_ms"] * 1e-3) / 1e9
    out_bytes = sum(M * s.n * (4 if s.out_dtype == wl.OUT_F32 else 2) for s in case.segments)
    gemm_bytes = 0.5625 * (M + N) * K + out_bytes  # codes + scales of A and W, plus the outputs
    gemm_gbps = gemm_bytes / (gemm_ms * 1e-3) / 1e9
    # the GEMM's bound: dense FP16 MFMA above the ridge point (peak FLOP/s per HBM byte/s), HBM below
    mfma_bound = flops / gemm_bytes >= PEAK_F16_MFMA_TFLOPS * 1e12 / (PEAK_HBM_GBPS * 1e9)
    log(f"[gpu] step {r['step_ms']:.3f} ms: quantize {qrot['ms']:.4f} ms over {qrot['copies']} rotating inputs "
        f"({q_gbps:.0f} GB/s; {q_gbps_same_x:.0f} GB/s on one input), "
        f"gemm {gemm_ms:.4f} ms ({gemm_tflops:.0f} TFLOP/s, {gemm_gbps:.0f} GB/s), weight copies {copies}")
    if mfma_bound:
        roof = {"bound": "mfma", "achieved": gemm_tflops, "peak": PEAK_F16_MFMA_TFLOPS, "unit": "TFLOP/s",
                "frac": gemm_tflops / PEAK_F16_MFMA_TFLOPS}
    else:
        roof = {"bound": "hbm", "achieved": gemm_gbps, "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                "frac": gemm_gbps / PEAK_HBM_GBPS}
    if M > 64:
        kernel = "gemm_kernel"
    elif M > 32:  # the reduce kernel runs only when K is split over workgroups (the workspace holds the parts)
        kernel = "gemm_wide_kernel" + (" + gemm_wide_reduce_kernel" if step.workspace is not None else "") + \
            (" (packed weights)" if args.packed else "")
    else:
        kernel = decode_kernel_name(M, K, args.packed)
    tr = measured_traffic(kernel, case.name)
    roof.update({"traffic": tr[0] if tr else None, "traffic_detail": tr[1] if tr else None,
                 "kernel": kernel, "avg_ms": gemm_ms, "algorithmic_flop": flops,
                 "algorithmic_bytes": gemm_bytes})
    # per-step event times of the timed steps (each GEMM interval also holds the event overhead)
    roof["step_events_ms"] = {"gemm_median": r["gemm_ms_med"], "gemm_p10_p90": r["gemm_ms_p10_p90"],
                              "quantize_median": r["quant_ms_med"], "quantize_p10_p90": r["quant_ms_p10_p90"]}
    clk = clock_under_load(step.gemm)
    if clk is not None:
        roof["clock"] = clk
        if mfma_bound:  # the matrix peak scales with the engine clock
            roof["peak_at_clock"] = PEAK_F16_MFMA_TFLOPS * clk["mean_mhz"] / PEAK_GFX_MHZ
            roof["frac_at_clock"] = gemm_tflops / roof["peak_at_clock"]
        log(f"[gpu] graphics clock during the GEMM: {clk['mean_mhz']:.0f} MHz "
            f"({clk['min_mhz']:.0f}-{clk['max_mhz']:.0f}), socket power {clk['socket_power_w']} W")
    trq = measured_traffic("quantize_kernel", f"x_{M}x{K}")
    copy_gbps = copy_ceiling_gbps()
    log(f"[gpu] plain device copy: {copy_gbps:.0f} GB/s (read + write)")
    out = {
        "metric": "NVFP4 W4A4 GEMM TFLOPS at 32K-token prefill + quantize GB/s, % of roofline",
        "value": flops / (r["step_ms"] * 1e-3) / 1e12,
        "unit": "TFLOP/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": r["step_ms"],
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "f16 MFMA operands (exact NVFP4 decode), f32 accumulate",
        "data": "synthetic (seeded; heavy-tailed activations with outlier channels, per-segment weight spreads)",
        "config": {"workload": case.name, "M": M, "N": N, "K": K,
                   "segments": ",".join(f"{s.name}{s.n}" for s in case.segments),
                   "epilogues": ";".join(f"{s.name}:{['none', 'sigmoid', 'gdn_decay'][s.epilogue]}/"
                                         f"{['f32', 'bf16'][s.out_dtype]}" for s in case.segments)},
        "gemm_tflops": gemm_tflops,
        "gemm_gbps": gemm_gbps,
        "quantize_gbps": q_gbps,
        "roofline": roof,
        "roofline_quantize": {"bound": "hbm", "achieved": q_gbps, "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                              "frac": q_gbps / PEAK_HBM_GBPS, "traffic": trq[0] if trq else None,
                              "traffic_detail": trq[1] if trq else None, "kernel": "quantize_kernel",
                              "avg_ms": qrot["ms"], "rotation": {k: v for k, v in qrot.items() if k != "ms"},
                              "avg_ms_one_input": r["quant_iso_ms"], "avg_ms_in_step": r["quant_ms"],
                              "algorithmic_bytes": q_bytes, "copy_ceiling_gbps": copy_gbps,
                              "frac_of_copy_ceiling": q_gbps / copy_gbps},
    }

    if args.library_gemm:
        out["library_gemm"] = library_gemm(step, M, N, K)
    if not args.no_cpu_baseline:
        log("[cpu] timing the oracle on a sample")
        out["cpu_baseline"] = run_cpu_baseline(step, min(args.cpu_rows_quant, M), min(args.cpu_rows_gemm, M))
    if not args.no_extras and args.workload == "C5":
        del step
        torch.cuda.empty_cache()
        log("[gpu] other configurations")
        out["other_configs"] = bench_other_configs(max(args.steps, 20))
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
