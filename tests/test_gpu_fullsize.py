"""GPU parity at the full workload sizes, in the launch configuration the benchmark times.

The whole activation tensor is quantized on the GPU and compared with the oracle bit for bit; the
GEMM is compared with the oracle's exact result on sampled rows across all N columns: one seeded
row per 128-row M tile, the first and last rows, and the rows holding the largest activations.
Every input is drawn by the seeded workload generator; g is calibrated on the GPU and checked
against the oracle's value.
"""
import numpy as np
import pytest
import torch

import nvfp4_w4a4_quantized_quantize_amd as nv
import oracle
import workloads as wl
from gpu_common import DEV, check_bf16, check_decay, check_fp32, check_sigmoid, dev_bf16, host

pytestmark = pytest.mark.gpu


def gpu_g(bits_dev: torch.Tensor, bits_np: np.ndarray) -> float:
    g = np.float32(host(nv.global_scale(bits_dev))[0])
    assert g.view(np.uint32) == oracle.global_scale(bits_np).view(np.uint32)
    return float(g)


def sample_rows(x_bits: np.ndarray, M: int, seed: int) -> np.ndarray:
    rng = np.random.default_rng(seed)
    rows = {0, M - 1}
    for t in range(0, M, 128):
        rows.add(int(rng.integers(t, min(t + 128, M))))
    amax_row = np.abs(wl.bf16_bits_to_f32(x_bits)).max(axis=1)
    rows.update(int(r) for r in np.argsort(amax_row)[-4:])
    return np.array(sorted(rows), dtype=np.int64)


def run_case(case: wl.GemmCase, out_dtype_plain, check_unfused: bool):
    print(f"{case.name}: drawing inputs", flush=True)
    x = wl.draw_x(case)
    xd = dev_bf16(x)
    g_a = gpu_g(xd, x)
    ac, as_ = nv.quantize(xd, g_a)
    # the whole activation tensor, bit for bit
    rac, ras = oracle.quantize(x, g_a)
    assert (host(as_) == ras).all() and (host(ac) == rac).all(), "activation codes/scales differ"
    del xd
    # weights: per segment global scale, quantized on the GPU into one concatenated tensor
    N, K = case.N, case.K
    wc, ws = nv.alloc_nvfp4(N, K, DEV)
    segs, g_w, rw_c, rw_s = [], [], [], []
    n0 = 0
    for s, seg in enumerate(case.segments):
        wb = wl.draw_w(case, s)
        wd = dev_bf16(wb)
        g = gpu_g(wd, wb)
        nv.quantize(wd, g, wc[n0:n0 + seg.n], ws[n0:n0 + seg.n])
        c, sc = oracle.quantize(wb, g)
        rw_c.append(c)
        rw_s.append(sc)
        g_w.append(g)
        epi = {wl.EPI_NONE: "none", wl.EPI_SIGMOID: "sigmoid", wl.EPI_GDN_DECAY: "gdn_decay"}[seg.epilogue]
        dt = torch.float32 if seg.epilogue != wl.EPI_NONE else out_dtype_plain
        a_log = dt_bias = None
        if seg.epilogue == wl.EPI_GDN_DECAY:
            al, db = wl.draw_gate_params(case, s)
            a_log, dt_bias = torch.from_numpy(al).to(DEV), torch.from_numpy(db).to(DEV)
        segs.append(nv.Segment(seg.n, g, epi, dt, a_log, dt_bias))
        n0 += seg.n
    rw_c, rw_s = np.concatenate(rw_c), np.concatenate(rw_s)
    assert (host(wc) == rw_c).all() and (host(ws) == rw_s).all(), "weight codes/scales differ"
    print(f"{case.name}: GEMM {case.M}x{N}x{K}", flush=True)
    outs = nv.gemm(ac, as_, g_a, wc, ws, segs)
    rows = sample_rows(x, case.M, case.cfg_id)
    y, T = oracle.gemm_rows(rac, ras, g_a, rw_c, rw_s, case.seg_bounds, np.array(g_w, np.float32), rows)
    rows_t = torch.from_numpy(rows).to(DEV)
    worst = 0.0
    for s, seg in enumerate(case.segments):
        lo, hi = case.seg_bounds[s], case.seg_bounds[s + 1]
        got = outs[s].index_select(0, rows_t)
        ys, Ts = y[:, lo:hi], T[:, lo:hi]
        if seg.epilogue == wl.EPI_SIGMOID:
            check_sigmoid(host(got), ys, Ts, oracle.sigmoid(ys))
        elif seg.epilogue == wl.EPI_GDN_DECAY:
            al, db = wl.draw_gate_params(case, s)
            check_decay(host(got), ys, Ts, oracle.gdn_decay(ys, al, db), al, db)
        elif segs[s].out_dtype == torch.float32:
            worst = max(worst, check_fp32(host(got), ys, Ts, f"{case.name} {seg.name}"))
        else:
            check_bf16(got, ys, Ts, f"{case.name} {seg.name}")
    print(f"{case.name}: {len(rows)} sampled rows within tolerance (max |err|/T {worst:.3g})", flush=True)
    if check_unfused:
        # each module alone gives bitwise the same columns as the fused GEMM
        n0 = 0
        for s, seg in enumerate(case.segments):
            alone = nv.Segment(seg.n, segs[s].g_w, segs[s].epilogue, segs[s].out_dtype, segs[s].A_log, segs[s].dt_bias)
            (u,) = nv.gemm(ac, as_, g_a, wc[n0:n0 + seg.n], ws[n0:n0 + seg.n], [alone])
            assert torch.equal(u, outs[s]), f"{case.name}: segment {seg.name} fused != unfused"
            n0 += seg.n


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_prefill_projection(dtype):
    run_case(wl.C2, dtype, check_unfused=False)


def test_fused_mlp_gate_up():
    run_case(wl.C4, torch.float32, check_unfused=True)


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_fused_gdn_in_proj_32k(dtype):
    run_case(wl.C5, dtype, check_unfused=dtype == torch.bfloat16)
