"""GPU parity at the full workload sizes, in the launch configuration the benchmark times.

The whole activation tensor is quantized on the GPU and compared with the oracle bit for bit; the
GEMM is compared with the oracle's exact result on every output of the single prefill projection
(4096 x 5120 x 5120, in FP32 and bf16), and on sampled rows across all N columns of the larger fused
GEMMs: one seeded row per 128-row M tile, the first and last rows, and the rows holding the largest
activations.
Every input is drawn by the seeded workload generator; g is calibrated on the GPU and checked
against the oracle's value.
"""
import numpy as np
import pytest
import torch

import nvfp4_w4a4_quantized_quantize_amd as nv
import oracle
import workloads as wl
from gpu_common import DEV, check_bf16, check_decay, check_fp32, check_sigmoid, dev_bf16, host, padded_u8

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


def run_case(case: wl.GemmCase, out_dtype_plain, check_unfused: bool, all_rows: bool = False):
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
    rows = np.arange(case.M, dtype=np.int64) if all_rows else sample_rows(x, case.M, case.cfg_id)
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
    print(f"{case.name}: {len(rows)} {'(all)' if all_rows else 'sampled'} rows within tolerance "
          f"(max |err|/T {worst:.3g})", flush=True)
    if check_unfused:
        # each module alone gives bitwise the same columns as the fused GEMM
        n0 = 0
        for s, seg in enumerate(case.segments):
            alone = nv.Segment(seg.n, segs[s].g_w, segs[s].epilogue, segs[s].out_dtype, segs[s].A_log, segs[s].dt_bias)
            (u,) = nv.gemm(ac, as_, g_a, wc[n0:n0 + seg.n], ws[n0:n0 + seg.n], [alone])
            assert torch.equal(u, outs[s]), f"{case.name}: segment {seg.name} fused != unfused"
            n0 += seg.n
    return dict(ac=ac, as_=as_, wc=wc, ws=ws, g_a=g_a, g_w=g_w, rows=rows, y=y, T=T, outs=outs)


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_prefill_projection(dtype):
    """Every one of the 4096 x 5120 outputs against the oracle's exact result."""
    run_case(wl.C2, dtype, check_unfused=False, all_rows=True)


def test_fused_mlp_gate_up():
    """The fused gate+up GEMM at full size, then the pages' fused-module trap ("Trap 1") on the same
    operands: one global scale (the first module's) for both modules mis-scales every output of the
    second module by g_w1 / g_w2, a relative error of |1 - g_w1 / g_w2| (about 0.67 here, the size of
    the pages' 0.35 / 0.57), while the first module stays within the FP32 bound."""
    case = wl.C4
    r = run_case(case, torch.float32, check_unfused=True)
    n1 = case.segments[0].n
    g1, g2 = r["g_w"]
    (bad,) = nv.gemm(r["ac"], r["as_"], r["g_a"], r["wc"], r["ws"], [nv.Segment(case.N, g1)])
    got = host(bad.index_select(0, torch.from_numpy(r["rows"]).to(DEV))).astype(np.float64)
    y, T = r["y"], r["T"]
    check_fp32(got[:, :n1], y[:, :n1], T[:, :n1], "first module under its own scale")
    rel = np.abs(got[:, n1:] - y[:, n1:]).sum() / np.abs(y[:, n1:]).sum()
    expect = abs(1.0 - float(g1) / float(g2))
    print(f"single global scale: second module relative error {rel:.4f} (expected {expect:.4f})", flush=True)
    assert expect > 0.3 and abs(rel - expect) < 1e-4 * expect


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_fused_gdn_in_proj_32k(dtype):
    run_case(wl.C5, dtype, check_unfused=dtype == torch.bfloat16)


def test_rmsnorm_quantize_full_size():
    """RMSNorm + NVFP4 quantization of the full 32768 x 5120 activation, bit-exact with the oracle."""
    case = wl.NORM
    x, w = wl.draw_norm_x(case), wl.draw_norm_weight(case)
    y_ref, _ = oracle.rmsnorm(x, w, np.float32(1e-6))
    g = oracle.global_scale(y_ref)
    c_ref, s_ref = oracle.quantize(y_ref, g)
    print(f"{case.name}: GPU", flush=True)
    codes, scales = nv.rmsnorm_quantize(dev_bf16(x), dev_bf16(w), 1e-6, float(g))
    assert (host(codes) == c_ref).all() and (host(scales) == s_ref).all()


def test_fold_in_repair_on_the_gdn_in_proj():
    """The pages' own repair on the full GDN in_proj weights: folded scales bit-exact with the oracle;
    the fused GEMM with the common scale against the exact per-segment result on sampled rows, which
    must stay within 2^-4 of sum |a w| (the E4M3 re-rounding bound); the observed error is printed."""
    case = wl.C5
    M = 4096
    x = wl.draw_x(case, M=M)
    g_a = gpu_g(dev_bf16(x), x)
    ac, as_ = oracle.quantize(x, g_a)
    wcs, wss, gs = [], [], []
    for s in range(len(case.segments)):
        wb = wl.draw_w(case, s)
        g = oracle.global_scale(wb)
        c, sc = oracle.quantize(wb, g)
        wcs.append(c)
        wss.append(sc)
        gs.append(g)
    wc, ws = np.concatenate(wcs), np.concatenate(wss)
    G_ref, folded = oracle.fold_group(wss, gs)
    d_scales = padded_u8(ws)
    G = nv.fold_group(d_scales, [s.n for s in case.segments], [float(g) for g in gs])
    assert np.float32(G) == G_ref and (host(d_scales) == np.concatenate(folded)).all()
    (out,) = nv.gemm(padded_u8(ac), padded_u8(as_), float(g_a), padded_u8(wc), d_scales, [nv.Segment(case.N, G)])
    rows = sample_rows(x, M, 5)
    y, T = oracle.gemm_rows(ac, as_, g_a, wc, ws, case.seg_bounds, np.array(gs, np.float32), rows)
    got = host(out.index_select(0, torch.from_numpy(rows).to(DEV))).astype(np.float64)
    err = np.abs(got - y)
    assert (err <= (2.0 ** -4 + 2.0 ** -19) * T).all()
    rel = np.linalg.norm(got - y) / np.linalg.norm(y)
    print(f"fold-in vs per-segment scales on {len(rows)} rows: max |err|/T = {(err / T).max():.3g}, "
          f"relative Frobenius error = {rel:.3g}", flush=True)
