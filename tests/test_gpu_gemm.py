"""GPU parity of nvfp4_gemm against the oracle: FP32 outputs within 2^-20 * sum|a w| * g_a * g_w,
bf16 outputs within that plus half a bf16 ulp, gate epilogues within the propagated bound; fused ==
unfused bitwise; repeatability; guard bands; the single-global-scale negative control; and the
workload shapes (tiny, ragged multi-tile, skinny decode)."""
import numpy as np
import pytest
import torch

import nvfp4_w4a4_quantized_quantize_amd as nv
import oracle
import workloads as wl
from gpu_common import (DEV, check_bf16, check_decay, check_fp32, check_sigmoid, dev_bf16, dev_u8, host,
                        padded_u8)

pytestmark = pytest.mark.gpu


def gpu_global_scale(bits: np.ndarray) -> np.float32:
    """Global scale computed on the GPU, checked bit-exact against the oracle's."""
    g = np.float32(host(nv.global_scale(dev_bf16(bits)))[0])
    assert g.view(np.uint32) == oracle.global_scale(bits).view(np.uint32)
    return g


def random_nvfp4(rng, rows, K, lo=0x01, hi=0x7F):
    codes = rng.integers(0, 256, size=(rows, K // 2), dtype=np.uint8)
    scales = rng.integers(lo, hi, size=(rows, K // 16), dtype=np.uint8)
    return codes, scales


def run_gemm(a, w, g_a, seg_specs, K):
    """a, w: (codes, scales) numpy; seg_specs: list of (n, g_w, epilogue, out_dtype, a_log, dt_bias)."""
    ac, as_ = padded_u8(a[0]), padded_u8(a[1])
    wc, ws = padded_u8(w[0]), padded_u8(w[1])
    segs = []
    for n, gw, epi, dt, al, db in seg_specs:
        segs.append(nv.Segment(n, gw, epi, dt, None if al is None else torch.from_numpy(al).to(DEV),
                               None if db is None else torch.from_numpy(db).to(DEV)))
    return nv.gemm(ac, as_, g_a, wc, ws, segs)


def oracle_y(a, w, g_a, seg_specs, rows):
    bounds = np.concatenate([[0], np.cumsum([s[0] for s in seg_specs])])
    g_w = np.array([s[1] for s in seg_specs], np.float32)
    return oracle.gemm_rows(a[0], a[1], np.float32(g_a), w[0], w[1], bounds, g_w, rows), bounds


@pytest.mark.parametrize("M,N,K", [(16, 128, 256), (1, 1, 16), (1, 300, 48), (300, 520, 272), (257, 259, 1040),
                                   (513, 64, 128), (64, 1024, 5120), (40, 96, 17408)])
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_random_codes_single_segment(M, N, K, dtype):
    rng = np.random.default_rng(M * 1000 + N + K)
    a, w = random_nvfp4(rng, M, K), random_nvfp4(rng, N, K)
    g_a, g_w = np.float32(0.0123), np.float32(3.5)
    spec = [(N, g_w, "none", dtype, None, None)]
    (out,) = run_gemm(a, w, g_a, spec, K)
    (y, T), _ = oracle_y(a, w, g_a, spec, np.arange(M))
    if dtype == torch.float32:
        check_fp32(host(out), y, T, f"M={M} N={N} K={K}")
    else:
        check_bf16(out, y, T, f"M={M} N={N} K={K}")


def test_multi_segment_ragged_boundaries_and_gates():
    rng = np.random.default_rng(42)
    M, K = 300, 512
    sizes = [5, 100, 3, 130, 33, 32]
    N = sum(sizes)
    a, w = random_nvfp4(rng, M, K, 0x20, 0x48), random_nvfp4(rng, N, K, 0x20, 0x48)
    a_log = (rng.standard_normal(33) * 0.5).astype(np.float32)
    dt_b = (rng.standard_normal(33) * 0.5).astype(np.float32)
    g_a = np.float32(2.0 ** -7)
    spec = [(5, 0.5, "none", torch.float32, None, None),
            (100, 1.82, "none", torch.bfloat16, None, None),
            (3, 0.01, "none", torch.float32, None, None),
            (130, 2.75, "sigmoid", torch.float32, None, None),
            (33, 0.37, "gdn_decay", torch.float32, a_log, dt_b),
            (32, 1.0, "none", torch.bfloat16, None, None)]
    outs = run_gemm(a, w, g_a, spec, K)
    (y, T), bounds = oracle_y(a, w, g_a, spec, np.arange(M))
    for s, out in enumerate(outs):
        lo, hi = bounds[s], bounds[s + 1]
        ys, Ts = y[:, lo:hi], T[:, lo:hi]
        epi, dt = spec[s][2], spec[s][3]
        if epi == "sigmoid":
            check_sigmoid(host(out), ys, Ts, oracle.sigmoid(ys))
        elif epi == "gdn_decay":
            check_decay(host(out), ys, Ts, oracle.gdn_decay(ys, a_log, dt_b), a_log, dt_b)
        elif dt == torch.float32:
            check_fp32(host(out), ys, Ts, f"segment {s}")
        else:
            check_bf16(out, ys, Ts, f"segment {s}")


# Partial last tile columns of every width class, with and without gate columns in them: the prefill
# kernel stacks its waves along M when a tile has at most 128 columns (64 or 128 of them per wave) and
# keeps 2 x 2 waves otherwise (the second column pair with 32 or 64 columns); tiles whose fragments all
# lie in plain vector-aligned segments are written straight from the registers, the others (gates,
# unaligned boundaries, a ragged N tail) element by element in a second launch.
_LAYOUTS = {
    "gates_in_64_col_tail": [(256, 1.5, "none", torch.bfloat16), (32, 0.7, "sigmoid", torch.float32),
                             (32, 0.9, "gdn_decay", torch.float32)],
    "gates_in_104_col_tail": [(512, 1.5, "none", torch.bfloat16), (40, 2.0, "none", torch.float32),
                              (32, 0.7, "sigmoid", torch.float32), (32, 0.9, "gdn_decay", torch.float32)],
    "direct_96_col_tail": [(352, 1.25, "none", torch.bfloat16)],
    "direct_192_col_tail": [(448, 0.5, "none", torch.float32)],
    "direct_160_col_tail": [(160, 0.75, "none", torch.bfloat16), (256, 3.0, "none", torch.float32)],
    "ragged_72_col_tail": [(256, 1.0, "none", torch.bfloat16), (72, 2.5, "none", torch.bfloat16)],
    "gates_mid_n": [(256, 1.0, "none", torch.bfloat16), (64, 0.6, "sigmoid", torch.float32),
                    (256, 1.1, "none", torch.bfloat16), (64, 0.8, "gdn_decay", torch.float32),
                    (256, 1.2, "none", torch.float32)],
}


@pytest.mark.parametrize("name", sorted(_LAYOUTS))
def test_tile_layouts_and_epilogue_kernels(name):
    rng = np.random.default_rng(sum(map(ord, name)))
    M, K = 300, 528  # a ragged second M tile and a K tail of one block
    layout = _LAYOUTS[name]
    N = sum(n for n, *_ in layout)
    a, w = random_nvfp4(rng, M, K, 0x20, 0x50), random_nvfp4(rng, N, K, 0x20, 0x50)
    spec = []
    for n, gw, epi, dt in layout:
        al = db = None
        if epi == "gdn_decay":
            al = (rng.standard_normal(n) * 0.5).astype(np.float32)
            db = (rng.standard_normal(n) * 0.5).astype(np.float32)
        spec.append((n, gw, epi, dt, al, db))
    g_a = np.float32(2.0 ** -6)
    outs = run_gemm(a, w, g_a, spec, K)
    (y, T), bounds = oracle_y(a, w, g_a, spec, np.arange(M))
    for s, out in enumerate(outs):
        lo, hi = bounds[s], bounds[s + 1]
        ys, Ts = y[:, lo:hi], T[:, lo:hi]
        n, _, epi, dt, al, db = spec[s]
        if epi == "sigmoid":
            check_sigmoid(host(out), ys, Ts, oracle.sigmoid(ys))
        elif epi == "gdn_decay":
            check_decay(host(out), ys, Ts, oracle.gdn_decay(ys, al, db), al, db)
        elif dt == torch.float32:
            check_fp32(host(out), ys, Ts, f"{name} segment {s}")
        else:
            check_bf16(out, ys, Ts, f"{name} segment {s}")


def _check_outputs(outs, spec, y, T, bounds, tag):
    for s, out in enumerate(outs):
        lo, hi = bounds[s], bounds[s + 1]
        ys, Ts = y[:, lo:hi], T[:, lo:hi]
        n, _, epi, dt, al, db = spec[s]
        if epi == "sigmoid":
            check_sigmoid(host(out), ys, Ts, oracle.sigmoid(ys))
        elif epi == "gdn_decay":
            check_decay(host(out), ys, Ts, oracle.gdn_decay(ys, al, db), al, db)
        elif dt == torch.float32:
            check_fp32(host(out), ys, Ts, f"{tag} segment {s}")
        else:
            check_bf16(out, ys, Ts, f"{tag} segment {s}")


def _spec_from(layout, rng):
    spec = []
    for n, gw, epi, dt in layout:
        al = db = None
        if epi == "gdn_decay":
            al = (rng.standard_normal(n) * 0.5).astype(np.float32)
            db = (rng.standard_normal(n) * 0.5).astype(np.float32)
        spec.append((n, gw, epi, dt, al, db))
    return spec


def test_full_tiles_with_gates_mid_n():
    """Gate and plain segments inside full 256 x 256 tiles (2 x 2 waves). 9 M-tiles x 15 full tile
    columns are 135 tiles, too many for their pieces to fit one round of 256 CUs, so no column is
    split; the 64-column tail holds a gate segment."""
    rng = np.random.default_rng(2100)
    M, K = 2100, 528
    layout = [(1024, 1.0, "none", torch.bfloat16), (64, 0.6, "sigmoid", torch.float32),
              (1000, 1.1, "none", torch.bfloat16), (88, 0.8, "gdn_decay", torch.float32),
              (1664, 1.2, "none", torch.float32), (64, 0.9, "sigmoid", torch.float32)]
    N = sum(n for n, *_ in layout)
    a, w = random_nvfp4(rng, M, K, 0x20, 0x50), random_nvfp4(rng, N, K, 0x20, 0x50)
    spec = _spec_from(layout, rng)
    g_a = np.float32(2.0 ** -6)
    outs = run_gemm(a, w, g_a, spec, K)
    (y, T), bounds = oracle_y(a, w, g_a, spec, np.arange(M))
    _check_outputs(outs, spec, y, T, bounds, "full tiles")


# Shapes whose full tiles leave most CUs idle in their last round (on 256 CUs): trailing tile columns
# run as 128-column (1000 x 6450, 2048 x 2148, 4096 x 5184) or 64-column (512 x 1000) pieces, next to
# the partial last column; segment boundaries and gates fall inside and across the pieces.
@pytest.mark.parametrize("M,N,K", [(1000, 6450, 272), (2048, 2148, 528), (512, 1000, 1040), (4096, 5184, 256)])
def test_split_tail_tile_columns(M, N, K):
    rng = np.random.default_rng(M + 7 * N + K)
    n1 = (N // 3) | 1
    layout = [(n1, 0.75, "none", torch.bfloat16), (40, 1.3, "sigmoid", torch.float32),
              (72, 0.9, "gdn_decay", torch.float32), (N - n1 - 112, 1.5, "none", torch.float32)]
    a, w = random_nvfp4(rng, M, K, 0x20, 0x58), random_nvfp4(rng, N, K, 0x20, 0x58)
    spec = _spec_from(layout, rng)
    g_a = np.float32(0.03)
    outs = run_gemm(a, w, g_a, spec, K)
    (y, T), bounds = oracle_y(a, w, g_a, spec, np.arange(M))
    _check_outputs(outs, spec, y, T, bounds, f"M={M} N={N} K={K}")


def test_fused_equals_unfused_bitwise_and_repeatable():
    rng = np.random.default_rng(7)
    M, K = 200, 640
    sizes = [96, 40, 256, 8]
    N = sum(sizes)
    a = random_nvfp4(rng, M, K)
    ws = [random_nvfp4(rng, n, K) for n in sizes]
    w = (np.concatenate([x[0] for x in ws]), np.concatenate([x[1] for x in ws]))
    g_w = [0.25, 1.82, 0.5, 2.75]
    spec = [(n, gw, "none", torch.float32, None, None) for n, gw in zip(sizes, g_w)]
    fused = [host(o) for o in run_gemm(a, w, 0.1, spec, K)]
    fused2 = [host(o) for o in run_gemm(a, w, 0.1, spec, K)]
    for f, f2 in zip(fused, fused2):
        assert (f.view(np.uint32) == f2.view(np.uint32)).all()
    for i, (n, gw) in enumerate(zip(sizes, g_w)):
        (u,) = run_gemm(a, ws[i], 0.1, [(n, gw, "none", torch.float32, None, None)], K)
        assert (host(u).view(np.uint32) == fused[i].view(np.uint32)).all(), f"segment {i}"


def test_single_global_scale_negative_control():
    """One global scale for two separately calibrated modules (the pages' "Trap 1") mis-scales the
    second module by the ratio of their scales; per-segment scales match the oracle."""
    rng = np.random.default_rng(8)
    M, K, n = 64, 256, 64
    a = random_nvfp4(rng, M, K)
    w = random_nvfp4(rng, 2 * n, K)
    g1, g2 = 0.01, 0.0275
    good_spec = [(n, g1, "none", torch.float32, None, None), (n, g2, "none", torch.float32, None, None)]
    good = np.concatenate([host(o) for o in run_gemm(a, w, 1.0, good_spec, K)], axis=1)
    (bad,) = run_gemm(a, w, 1.0, [(2 * n, g1, "none", torch.float32, None, None)], K)
    bad = host(bad)
    (y, T), _ = oracle_y(a, w, 1.0, good_spec, np.arange(M))
    check_fp32(good, y, T, "per-segment scales")
    rel = np.abs(bad[:, n:] - y[:, n:]).sum() / np.abs(y[:, n:]).sum()
    assert abs(rel - (1 - g1 / g2)) < 1e-5
    assert np.abs(bad[:, :n] - y[:, :n]).max() <= (2.0 ** -20 * T[:, :n]).max()


def test_output_guard_bands_and_strides():
    rng = np.random.default_rng(9)
    M, N, K = 70, 90, 160
    a, w = random_nvfp4(rng, M, K), random_nvfp4(rng, N, K)
    buf = torch.full((M + 2, 128), float("nan"), dtype=torch.float32, device=DEV)
    out = buf[1:M + 1, 4:4 + N]
    ac, as_, wc, ws = padded_u8(a[0]), padded_u8(a[1]), padded_u8(w[0]), padded_u8(w[1])
    nv.gemm(ac, as_, 0.5, wc, ws, [nv.Segment(N, 2.0, out=out)])
    b = host(buf)
    assert np.isnan(b[0]).all() and np.isnan(b[-1]).all()
    assert np.isnan(b[:, :4]).all() and np.isnan(b[:, 4 + N:]).all()
    (y, T), _ = oracle_y(a, w, 0.5, [(N, 2.0, "none", torch.float32, None, None)], np.arange(M))
    check_fp32(b[1:M + 1, 4:4 + N], y, T, "strided output")


def test_row_strides_just_below_the_limit():
    """Codes and scale rows of both operands strided by 2^23 - 16 bytes, the largest stride accepted:
    the prefill kernel's 32-bit buffer offsets (up to 255 strides inside a tile) and record counts
    stay in range. The padding holds 0xFF bytes (NaN as an E4M3 scale), read in the chunk that
    crosses K and masked there."""
    rng = np.random.default_rng(23)
    M, N, K = 300, 70, 272  # a ragged second M tile, a ragged N tile, a K tail of one block
    a, w = random_nvfp4(rng, M, K), random_nvfp4(rng, N, K)
    ld = (1 << 23) - 16

    def strided(x):
        rows, cols = x.shape
        buf = torch.full((rows, ld), 0xFF, dtype=torch.uint8, device=DEV)
        buf[:, :cols] = torch.from_numpy(np.ascontiguousarray(x)).to(DEV)
        return buf[:, :cols]
    ac, as_, wc, ws = strided(a[0]), strided(a[1]), strided(w[0]), strided(w[1])
    assert ac.stride(0) == ld and ws.stride(0) == ld
    (out,) = nv.gemm(ac, as_, 0.25, wc, ws, [nv.Segment(N, 3.0)])
    (y, T), _ = oracle_y(a, w, 0.25, [(N, 3.0, "none", torch.float32, None, None)], np.arange(M))
    check_fp32(host(out), y, T, "strides 2^23 - 16")
    del ac, as_, wc, ws
    torch.cuda.empty_cache()


def sweep_shapes():
    """Seeded shapes across the three GEMM kernels: M in the skinny (<= 32), wide (33..64) and tiled
    (> 64) ranges, N ragged against every column grouping (16, 32, 64, 80, 128, 256), K with tails
    and, for the wide kernel, long enough to be split over workgroups."""
    rng = np.random.default_rng(2026)
    shapes = []
    for i in range(36):
        M = int(rng.choice([1, 3, 17, 32, 33, 47, 64, 65, 130, 257]))
        N = int(rng.integers(1, 400)) if i % 3 else int(rng.integers(400, 2600))
        K = 16 * int(rng.integers(1, 160)) if i % 4 else 16 * int(rng.integers(300, 420))
        shapes.append((M, N, K))
    return shapes


@pytest.mark.parametrize("M,N,K", sweep_shapes())
def test_random_shape_sweep(M, N, K):
    rng = np.random.default_rng(M * 7919 + N * 31 + K)
    a, w = random_nvfp4(rng, M, K, 0x20, 0x58), random_nvfp4(rng, N, K, 0x20, 0x58)
    n1 = max(1, N // 3)
    spec = [(n1, 0.75, "none", torch.bfloat16, None, None)]
    if N - n1 > 0:
        spec.append((N - n1, 1.5, "none", torch.float32, None, None))
    outs = run_gemm(a, w, np.float32(0.03), spec, K)
    (y, T), bounds = oracle_y(a, w, np.float32(0.03), spec, np.arange(M))
    for s, out in enumerate(outs):
        lo, hi = bounds[s], bounds[s + 1]
        if spec[s][3] == torch.float32:
            check_fp32(host(out), y[:, lo:hi], T[:, lo:hi], f"M={M} N={N} K={K} segment {s}")
        else:
            check_bf16(out, y[:, lo:hi], T[:, lo:hi], f"M={M} N={N} K={K} segment {s}")


@pytest.mark.parametrize("M", [5, 40, 70])
def test_k_zero_writes_zero_and_empty_shapes(M):
    """K = 0 on each kernel (skinny, split-K decode, tiled): the epilogue of y = 0."""
    N = 7
    a = torch.empty((M, 0), dtype=torch.uint8, device=DEV)
    w = torch.empty((N, 0), dtype=torch.uint8, device=DEV)
    (out,) = nv.gemm(a, a, 1.0, w, w, [nv.Segment(N, 1.0)])
    assert (host(out) == 0).all()
    e = torch.empty((0, 8), dtype=torch.uint8, device=DEV)
    e2 = torch.empty((0, 1), dtype=torch.uint8, device=DEV)
    wc = padded_u8(np.zeros((N, 8), np.uint8))
    ws = padded_u8(np.zeros((N, 1), np.uint8))
    (out,) = nv.gemm(e, e2, 1.0, wc, ws, [nv.Segment(N, 1.0)])
    assert out.shape == (0, N)


@pytest.mark.parametrize("M", [5, 40, 300])
def test_k_zero_gates_see_zero(M):
    """K = 0 with gate segments, on each kernel: the gates of y = 0 (sigmoid 1/2, decay of dt_bias)."""
    rng = np.random.default_rng(M)
    a_log = (rng.standard_normal(32) * 0.5).astype(np.float32)
    dt_b = (rng.standard_normal(32) * 0.5).astype(np.float32)
    a = torch.empty((M, 0), dtype=torch.uint8, device=DEV)
    w = torch.empty((64, 0), dtype=torch.uint8, device=DEV)
    sig, dec = nv.gemm(a, a, 1.0, w, w, [nv.Segment(32, 1.0, "sigmoid"),
                                         nv.Segment(32, 1.0, "gdn_decay", torch.float32,
                                                    torch.from_numpy(a_log).to(DEV), torch.from_numpy(dt_b).to(DEV))])
    y = np.zeros((M, 32))
    check_sigmoid(host(sig), y, y, oracle.sigmoid(y))
    check_decay(host(dec), y, y, oracle.gdn_decay(y, a_log, dt_b), a_log, dt_b)


def test_tiny_workload_end_to_end():
    """Tiny config: both operands quantized on the GPU from bf16, single segment, FP32 out."""
    case = wl.C1
    x, w = wl.draw_x(case), wl.draw_w(case, 0)
    g_a, g_w = gpu_global_scale(x), gpu_global_scale(w)
    ac, as_ = nv.quantize(dev_bf16(x), float(g_a))
    wc, ws = nv.quantize(dev_bf16(w), float(g_w))
    (out,) = nv.gemm(ac, as_, float(g_a), wc, ws, [nv.Segment(case.N, float(g_w))])
    rac, ras = oracle.quantize(x, g_a)
    rwc, rws = oracle.quantize(w, g_w)
    assert (host(ac) == rac).all() and (host(wc) == rwc).all()
    y, T = oracle.gemm_rows(rac, ras, g_a, rwc, rws, [0, case.N], np.array([g_w], np.float32), np.arange(case.M))
    e = check_fp32(host(out), y, T, "tiny")
    print(f"tiny: max |err| / T = {e:.3g}")


@pytest.mark.parametrize("M", [1, 16, 64])
@pytest.mark.parametrize("direction", ["up", "down"])
def test_decode_shapes(M, direction):
    case = wl.C3(M, direction)
    x = wl.draw_x(case)
    w = wl.draw_w(case, 0)
    print(f"{case.name}: X {x.shape} W {w.shape}", flush=True)
    g_a, g_w = gpu_global_scale(x), gpu_global_scale(w)
    ac, as_ = nv.quantize(dev_bf16(x), float(g_a))
    wc, ws = nv.quantize(dev_bf16(w), float(g_w))
    (out,) = nv.gemm(ac, as_, float(g_a), wc, ws, [nv.Segment(case.N, float(g_w), out_dtype=torch.float32)])
    rac, ras = oracle.quantize(x, g_a)
    rwc, rws = oracle.quantize(w, g_w)
    assert (host(ac) == rac).all() and (host(as_) == ras).all()
    assert (host(wc) == rwc).all() and (host(ws) == rws).all()
    y, T = oracle.gemm_rows(rac, ras, g_a, rwc, rws, [0, case.N], np.array([g_w], np.float32), np.arange(M))
    check_fp32(host(out), y, T, case.name)
