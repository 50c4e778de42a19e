"""GPU parity of the decode (M <= 64) GEMM path against the oracle.

One activation row runs on the weight-streaming GEMV kernel (K up to 32768), up to 32 rows on the
skinny kernel, 33 .. 64 on the wide (split-K) kernel:
these tests cover every activation-tile count (M = 1 .. 64, ragged), both weight-tile widths of the
skinny kernel (1 tile per wave for M <= 4, 2 above) at large N, K-splits over 1 .. 4 waves and over
1 .. 8 workgroups with ragged chunk counts and a ragged final chunk, padded input strides, a reused
workspace, multi-segment tables with gate epilogues, bitwise agreement of a fused call with the same
modules called one by one, repeatability, and the switch to the tiled kernel at M = 65. Acceptance
is the bound stated in gpu_common.
"""
import numpy as np
import pytest
import torch

import nvfp4_w4a4_quantized_quantize_amd as nv
import oracle
import workloads as wl
from gpu_common import DEV, check_bf16, check_decay, check_fp32, check_sigmoid, dev_bf16, host, padded_u8

pytestmark = pytest.mark.gpu


def random_nvfp4(rng, rows, K, lo=0x01, hi=0x7F):
    codes = rng.integers(0, 256, size=(rows, K // 2), dtype=np.uint8)
    scales = rng.integers(lo, hi, size=(rows, K // 16), dtype=np.uint8)
    return codes, scales


def upload(t):
    return padded_u8(t[0]), padded_u8(t[1])


def run_single(a, w, g_a, g_w, dtype=torch.float32):
    ac, as_ = upload(a)
    wc, ws = upload(w)
    (out,) = nv.gemm(ac, as_, g_a, wc, ws, [nv.Segment(w[0].shape[0], g_w, out_dtype=dtype)])
    return out


def expect(a, w, g_a, g_w):
    N = w[0].shape[0]
    return oracle.gemm_rows(a[0], a[1], np.float32(g_a), w[0], w[1], [0, N], np.array([g_w], np.float32),
                            np.arange(a[0].shape[0]))


@pytest.mark.parametrize("M", [1, 2, 15, 16, 17, 33, 48, 63, 64])
@pytest.mark.parametrize("N,K", [(1, 16), (17, 48), (100, 272), (1000, 1040), (300, 4112)])
def test_skinny_random_codes(M, N, K):
    rng = np.random.default_rng(M * 7919 + N * 31 + K)
    a, w = random_nvfp4(rng, M, K), random_nvfp4(rng, N, K)
    out = run_single(a, w, 0.375, 1.25)
    y, T = expect(a, w, 0.375, 1.25)
    check_fp32(host(out), y, T, f"M={M} N={N} K={K}")


@pytest.mark.parametrize("M", [1, 2, 4, 5, 20, 40, 64])
def test_skinny_wide_weight_tiles(M):
    """Large N: the skinny kernel with one weight tile per wave (M <= 4) and two (M > 4), and the wide
    kernel."""
    rng = np.random.default_rng(100 + M)
    for N in (16400, 32800 + 48):
        a, w = random_nvfp4(rng, M, 96), random_nvfp4(rng, N, 96)
        out = run_single(a, w, 0.5, 0.75, torch.bfloat16)
        y, T = expect(a, w, 0.5, 0.75)
        check_bf16(out, y, T, f"M={M} N={N}")


@pytest.mark.parametrize("M", [1, 2, 9, 40, 64])
@pytest.mark.parametrize("K", [2048 + 16, 3072 + 16, 3840, 8192 + 128, 17408, 17408 + 16 * 7])
def test_skinny_long_k_splits(M, K):
    """Long K: 2, 3 or 4 waves per column tile (M <= 32; 9, 13, 15 and more chunks) or up to 8
    workgroup K-splits (M > 32), uneven chunk counts, a partial last chunk."""
    rng = np.random.default_rng(K + M)
    N = 70 if M <= 32 else 200
    a, w = random_nvfp4(rng, M, K), random_nvfp4(rng, N, K)
    out = run_single(a, w, 2.0 ** -7, 3.0)
    y, T = expect(a, w, 2.0 ** -7, 3.0)
    check_fp32(host(out), y, T, f"M={M} K={K}")


@pytest.mark.parametrize("direction", ["up", "down"])
def test_wide_workgroup_shapes_agree_bitwise(direction):
    """For 32 < M <= 64 the rows per workgroup follow N and the K split count (128, 80 or 64): on a
    256-CU MI355X the MLP up projection (N = 17408, one split) takes 80-row workgroups, the down
    projection (N = 5120, six splits) 128-row ones, and their first 300 weight rows as a GEMM of
    their own 64-row ones. Every column's sum runs in the same order in all shapes, so the shared
    columns agree bit for bit; the full result also meets the oracle's bound on sampled rows."""
    M = 64
    N, K = (17408, 5120) if direction == "up" else (5120, 17408)
    rng = np.random.default_rng(N + K)
    a = random_nvfp4(rng, M, K, 0x30, 0x70)
    w = random_nvfp4(rng, N, K, 0x30, 0x70)
    full = run_single(a, w, 0.02, 0.5)
    part = run_single(a, (w[0][:300], w[1][:300]), 0.02, 0.5)
    assert torch.equal(full[:, :300].contiguous().view(torch.int32), part.contiguous().view(torch.int32))
    rows = np.array([0, 31, 63])
    y, T = oracle.gemm_rows(a[0], a[1], np.float32(0.02), w[0], w[1], [0, N], np.array([0.5], np.float32), rows)
    check_fp32(host(full)[rows], y, T, f"{direction} M=64 sampled rows")


def test_wide_decode_workspace_contents_do_not_matter():
    """M in (32, 64] with K long enough for two K splits: the partial sums go to the caller's workspace.
    One workspace, filled with NaN first, serves two calls in a row (the second with fewer rows,
    columns and chunks); each call matches the oracle."""
    rng = np.random.default_rng(91)
    ws = torch.full((nv.lib().nvfp4_gemm_workspace_bytes(64, 300, 8320) // 4,), float("nan"),
                    dtype=torch.float32, device=DEV)
    assert ws.numel() > 0
    for M, N, K in ((64, 300, 8320), (35, 130, 6160)):
        assert nv.lib().nvfp4_gemm_workspace_bytes(M, N, K) <= ws.numel() * 4
        a, w = random_nvfp4(rng, M, K), random_nvfp4(rng, N, K)
        ac, as_ = upload(a)
        wc, wsc = upload(w)
        (out,) = nv.gemm(ac, as_, 0.5, wc, wsc, [nv.Segment(N, 2.0)], workspace=ws.view(torch.uint8))
        y, T = expect(a, w, 0.5, 2.0)
        check_fp32(host(out), y, T, f"M={M} N={N} K={K}")


@pytest.mark.parametrize("M", [2, 23, 41])
def test_skinny_padded_strides_and_offsets(M):
    """Inputs that are row slices of wider buffers (strides beyond the row), output with a stride."""
    rng = np.random.default_rng(77 + M)
    N, K = 130, 528
    a, w = random_nvfp4(rng, M, K), random_nvfp4(rng, N, K)

    def wide(x, extra16):
        """x inside a buffer whose row stride is the row rounded up to 16 bytes plus 16 * extra16."""
        rows, cols = x.shape
        buf = torch.full((rows, (cols + 15) // 16 * 16 + 16 * extra16), 0x77, dtype=torch.uint8, device=DEV)
        buf[:, :cols] = torch.from_numpy(x).to(DEV)
        return buf[:, :cols]

    ac, as_ = wide(a[0], 3), wide(a[1], 2)
    wc, ws = wide(w[0], 1), wide(w[1], 1)
    buf = torch.full((M, N + 10), float("nan"), dtype=torch.float32, device=DEV)
    nv.gemm(ac, as_, 0.25, wc, ws, [nv.Segment(N, 0.5, out=buf[:, 3:3 + N])])
    b = host(buf)
    assert np.isnan(b[:, :3]).all() and np.isnan(b[:, 3 + N:]).all()
    y, T = expect(a, w, 0.25, 0.5)
    check_fp32(b[:, 3:3 + N], y, T, "padded strides")


@pytest.mark.parametrize("M", [1, 7, 64])
def test_skinny_gdn_segments_fused_equals_unfused(M):
    """The GDN input projection layout at decode: six segments, sigmoid and decay gates; each module
    called alone gives the same bits as the fused call, and a second call repeats them."""
    case = wl.C5
    K = case.K
    rng = np.random.default_rng(M)
    a = random_nvfp4(rng, M, K, 0x30, 0x70)
    sizes = [s.n for s in case.segments]
    ws = [random_nvfp4(rng, n, K, 0x30, 0x70) for n in sizes]
    g_w = [0.003 * (1 + s) for s in range(len(sizes))]
    g_a = 0.02
    ac, as_ = upload(a)
    wc = padded_u8(np.concatenate([x[0] for x in ws]))
    wsc = padded_u8(np.concatenate([x[1] for x in ws]))
    segs, gates = [], {}
    for s, seg in enumerate(case.segments):
        if seg.epilogue == wl.EPI_SIGMOID:
            segs.append(nv.Segment(seg.n, g_w[s], "sigmoid", torch.float32))
        elif seg.epilogue == wl.EPI_GDN_DECAY:
            al, db = wl.draw_gate_params(case, s)
            gates[s] = (al, db)
            segs.append(nv.Segment(seg.n, g_w[s], "gdn_decay", torch.float32, torch.from_numpy(al).to(DEV),
                                   torch.from_numpy(db).to(DEV)))
        else:
            segs.append(nv.Segment(seg.n, g_w[s], "none", torch.bfloat16 if s % 2 else torch.float32))
    outs = nv.gemm(ac, as_, g_a, wc, wsc, segs)
    again = nv.gemm(ac, as_, g_a, wc, wsc, segs)
    for o, o2 in zip(outs, again):
        assert torch.equal(o, o2)
    y, T = oracle.gemm_rows(a[0], a[1], np.float32(g_a), np.concatenate([x[0] for x in ws]),
                            np.concatenate([x[1] for x in ws]), case.seg_bounds, np.array(g_w, np.float32),
                            np.arange(M))
    n0 = 0
    for s, seg in enumerate(case.segments):
        lo, hi = case.seg_bounds[s], case.seg_bounds[s + 1]
        ys, Ts = y[:, lo:hi], T[:, lo:hi]
        if seg.epilogue == wl.EPI_SIGMOID:
            check_sigmoid(host(outs[s]), ys, Ts, oracle.sigmoid(ys))
        elif seg.epilogue == wl.EPI_GDN_DECAY:
            al, db = gates[s]
            check_decay(host(outs[s]), ys, Ts, oracle.gdn_decay(ys, al, db), al, db)
        elif segs[s].out_dtype == torch.float32:
            check_fp32(host(outs[s]), ys, Ts, seg.name)
        else:
            check_bf16(outs[s], ys, Ts, seg.name)
        (u,) = nv.gemm(ac, as_, g_a, wc[n0:n0 + seg.n], wsc[n0:n0 + seg.n], [segs[s]])
        assert torch.equal(u, outs[s]), f"M={M}: segment {seg.name} fused != unfused"
        n0 += seg.n


def test_path_switch_at_65_rows():
    """Rows 0..63 computed with M = 64 (skinny) and M = 65 (tiled) both meet the bound."""
    rng = np.random.default_rng(65)
    N, K = 200, 784
    a, w = random_nvfp4(rng, 65, K), random_nvfp4(rng, N, K)
    y, T = expect(a, w, 1.0, 1.0)
    big = host(run_single(a, w, 1.0, 1.0))
    small = host(run_single((a[0][:64], a[1][:64]), w, 1.0, 1.0))
    check_fp32(big, y, T, "M=65")
    check_fp32(small, y[:64], T[:64], "M=64")


@pytest.mark.parametrize("M", [1, 16, 64])
@pytest.mark.parametrize("direction", ["up", "down"])
def test_decode_bf16_activation_pipeline(direction, M):
    """The decode workloads at full size (up 5120 -> 17408, down 17408 -> 5120) from bf16: GPU global
    scales and quantizer, then the decode GEMM (skinny kernel at M = 1 and 16, split-K wide kernel at
    M = 64), BF16 out; every output checked."""
    case = wl.C3(M, direction)
    x, w = wl.draw_x(case), wl.draw_w(case, 0)
    g_a = np.float32(host(nv.global_scale(dev_bf16(x)))[0])
    g_w = np.float32(host(nv.global_scale(dev_bf16(w)))[0])
    ac, as_ = nv.quantize(dev_bf16(x), float(g_a))
    wc, ws = nv.quantize(dev_bf16(w), float(g_w))
    (out,) = nv.gemm(ac, as_, float(g_a), wc, ws, [nv.Segment(case.N, float(g_w), out_dtype=torch.bfloat16)])
    rac, ras = oracle.quantize(x, g_a)
    rwc, rws = oracle.quantize(w, g_w)
    assert (host(ac) == rac).all() and (host(as_) == ras).all()
    y, T = oracle.gemm_rows(rac, ras, g_a, rwc, rws, [0, case.N], np.array([g_w], np.float32), np.arange(M))
    check_bf16(out, y, T, case.name)


@pytest.mark.parametrize("M", [1, 2])
@pytest.mark.parametrize("K", [16, 1024 + 16, 32768, 32768 + 16])
def test_gemv_rows_and_k_limits(M, K):
    """One activation row runs on the weight-streaming kernel up to K = 32768 (a lane's share of
    blocks ragged below that) and on the skinny kernel above, as do two rows; N not a multiple of the
    4 rows of a workgroup."""
    rng = np.random.default_rng(K * 3 + M)
    N = 37
    a, w = random_nvfp4(rng, M, K), random_nvfp4(rng, N, K)
    out = run_single(a, w, 0.125, 2.5)
    y, T = expect(a, w, 0.125, 2.5)
    check_fp32(host(out), y, T, f"M={M} K={K}")
