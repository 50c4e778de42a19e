"""GPU parity of the decode weight layout (nvfp4_pack_weights, nvfp4_gemm_packed).

The packed bytes are checked against a NumPy packing written here from the layout's definition in the C
header; the GEMM with packed weights against nvfp4_gemm with the same weights row-major (bitwise for
2 <= M <= 64: the same decode kernels, fed the same operand values in the same order) and against the
oracle (M = 1, where nvfp4_gemm takes another kernel, and a full-size sample). Acceptance is the bound
stated in gpu_common.
"""
import numpy as np
import pytest
import torch

import nvfp4_w4a4_quantized_quantize_amd as nv
import oracle
import workloads as wl
from gpu_common import DEV, check_fp32, host, padded_u8

pytestmark = pytest.mark.gpu


def random_nvfp4(rng, rows, K, lo=0x01, hi=0x7F):
    codes = rng.integers(0, 256, size=(rows, K // 2), dtype=np.uint8)
    scales = rng.integers(lo, hi, size=(rows, K // 16), dtype=np.uint8)
    return codes, scales


def pack_np(codes: np.ndarray, scales: np.ndarray, N: int, K: int) -> np.ndarray:
    """The decode layout by its definition: tile t, chunk c; codes piece h, lane r + 16 g holds code
    bytes 64 h + 16 g .. + 15 of chunk c of row 16 t + r; the scale dword of that lane holds the scale
    bytes of blocks 2g, 2g + 1, 8 + 2g, 9 + 2g of that row and chunk; zeros past N and K."""
    T, C = -(-N // 16), -(-K // 256)
    cz = np.zeros((T * 16, C * 128), np.uint8)
    cz[:N, :K // 2] = codes
    sz = np.zeros((T * 16, C * 16), np.uint8)
    sz[:N, :K // 16] = scales
    cr = cz.reshape(T, 16, C, 128)
    sr = sz.reshape(T, 16, C, 16)
    pc = np.zeros((T, C, 2, 64, 16), np.uint8)
    ps = np.zeros((T, C, 64, 4), np.uint8)
    for g in range(4):
        for r in range(16):
            lane = r + 16 * g
            for h in range(2):
                pc[:, :, h, lane, :] = cr[:, r, :, 64 * h + 16 * g:64 * h + 16 * g + 16]
            for e, b in enumerate((2 * g, 2 * g + 1, 8 + 2 * g, 9 + 2 * g)):
                ps[:, :, lane, e] = sr[:, r, :, b]
    return np.concatenate([pc.ravel(), ps.ravel()])


@pytest.mark.parametrize("N,K", [(1, 16), (17, 48), (100, 272), (300, 4112), (33, 5120), (64, 512)])
def test_pack_layout_matches_its_definition(N, K):
    rng = np.random.default_rng(N * 131 + K)
    w = random_nvfp4(rng, N, K)
    assert nv.lib().nvfp4_packed_weight_bytes(N, K) == -(-N // 16) * -(-K // 256) * 2304
    packed = nv.pack_weights(padded_u8(w[0]), padded_u8(w[1]))
    got = host(packed)[:nv.lib().nvfp4_packed_weight_bytes(N, K)]
    assert np.array_equal(got, pack_np(w[0], w[1], N, K)), f"N={N} K={K}"


def both(a, w, g_a, g_w, dtype=torch.float32):
    ac, as_ = padded_u8(a[0]), padded_u8(a[1])
    wc, ws = padded_u8(w[0]), padded_u8(w[1])
    N = w[0].shape[0]
    (ref,) = nv.gemm(ac, as_, g_a, wc, ws, [nv.Segment(N, g_w, out_dtype=dtype)])
    packed = nv.pack_weights(wc, ws)
    (got,) = nv.gemm_packed(ac, as_, g_a, packed, N, [nv.Segment(N, g_w, out_dtype=dtype)])
    return got, ref


@pytest.mark.parametrize("M", [2, 5, 16, 17, 32, 33, 48, 64])
@pytest.mark.parametrize("N,K", [(17, 48), (100, 272), (1000, 1040), (90, 3072 + 16), (300, 4112)])
def test_gemm_packed_equals_row_major_bitwise(M, N, K):
    rng = np.random.default_rng(M * 7919 + N * 31 + K + 1)
    a, w = random_nvfp4(rng, M, K), random_nvfp4(rng, N, K)
    got, ref = both(a, w, 0.375, 1.25)
    assert torch.equal(got.view(torch.int32), ref.view(torch.int32)), f"M={M} N={N} K={K}"
    if N == 300:
        y, T = oracle.gemm_rows(a[0], a[1], np.float32(0.375), w[0], w[1], [0, N], np.array([1.25], np.float32),
                                np.arange(M))
        check_fp32(host(got), y, T, f"M={M} N={N} K={K}")


@pytest.mark.parametrize("N,K", [(1, 16), (100, 272), (300, 4112)])
def test_gemm_packed_one_row_meets_bound(N, K):
    rng = np.random.default_rng(N + K)
    a, w = random_nvfp4(rng, 1, K), random_nvfp4(rng, N, K)
    got, _ = both(a, w, 0.5, 2.0)
    y, T = oracle.gemm_rows(a[0], a[1], np.float32(0.5), w[0], w[1], [0, N], np.array([2.0], np.float32),
                            np.arange(1))
    check_fp32(host(got), y, T, f"M=1 N={N} K={K}")


@pytest.mark.parametrize("M", [7, 64])
def test_gemm_packed_gdn_segments_equal_row_major(M):
    """The GDN input projection layout (six segments, sigmoid and decay gates, bf16 and FP32 outputs)."""
    case = wl.C5
    K = case.K
    rng = np.random.default_rng(100 + M)
    a = random_nvfp4(rng, M, K, 0x30, 0x70)
    w = random_nvfp4(rng, case.N, K, 0x30, 0x70)
    g_w = [0.003 * (1 + s) for s in range(len(case.segments))]
    segs = []
    for s, seg in enumerate(case.segments):
        if seg.epilogue == wl.EPI_SIGMOID:
            segs.append(nv.Segment(seg.n, g_w[s], "sigmoid", torch.float32))
        elif seg.epilogue == wl.EPI_GDN_DECAY:
            al, db = wl.draw_gate_params(case, s)
            segs.append(nv.Segment(seg.n, g_w[s], "gdn_decay", torch.float32, torch.from_numpy(al).to(DEV),
                                   torch.from_numpy(db).to(DEV)))
        else:
            segs.append(nv.Segment(seg.n, g_w[s], "none", torch.bfloat16 if s % 2 else torch.float32))
    ac, as_ = padded_u8(a[0]), padded_u8(a[1])
    wc, ws = padded_u8(w[0]), padded_u8(w[1])
    ref = nv.gemm(ac, as_, 0.02, wc, ws, segs)
    packed = nv.pack_weights(wc, ws)
    got = nv.gemm_packed(ac, as_, 0.02, packed, case.N, segs)
    for s, (o, r) in enumerate(zip(got, ref)):
        assert torch.equal(o.view(torch.uint8), r.view(torch.uint8)), f"M={M}: segment {case.segments[s].name}"


@pytest.mark.parametrize("M", [16, 64])
@pytest.mark.parametrize("direction", ["up", "down"])
def test_gemm_packed_decode_full_size(direction, M):
    """The decode projections at full size (up 5120 -> 17408, down 17408 -> 5120; the down projection
    at M = 64 splits K over workgroups): bitwise equal to the row-major call."""
    N, K = (17408, 5120) if direction == "up" else (5120, 17408)
    g = torch.Generator(device=DEV)
    g.manual_seed(M + (0 if direction == "up" else 1))
    wc, ws = nv.alloc_nvfp4(N, K, DEV)
    wc.copy_(torch.randint(0, 256, wc.shape, device=DEV, dtype=torch.uint8, generator=g))
    ws.copy_(torch.randint(0x28, 0x48, ws.shape, device=DEV, dtype=torch.uint8, generator=g))
    ac, as_ = nv.alloc_nvfp4(M, K, DEV)
    ac.copy_(torch.randint(0, 256, ac.shape, device=DEV, dtype=torch.uint8, generator=g))
    as_.copy_(torch.randint(0x30, 0x38, as_.shape, device=DEV, dtype=torch.uint8, generator=g))
    seg = [nv.Segment(N, 0.01, out_dtype=torch.bfloat16)]
    (ref,) = nv.gemm(ac, as_, 0.5, wc, ws, seg)
    packed = nv.pack_weights(wc, ws)
    (got,) = nv.gemm_packed(ac, as_, 0.5, packed, N, seg)
    assert torch.equal(got.view(torch.int16), ref.view(torch.int16))


def test_gemm_packed_k_zero_and_empty():
    """K = 0 writes the epilogue of y = 0 (no weight byte is read)."""
    ac = torch.zeros((3, 0), dtype=torch.uint8, device=DEV)
    out = torch.full((3, 20), 7.0, dtype=torch.float32, device=DEV)
    packed = torch.zeros(16, dtype=torch.uint8, device=DEV)
    nv.gemm_packed(ac, ac.clone(), 1.0, packed, 20, [nv.Segment(20, 1.0, out=out)])
    assert torch.equal(out, torch.zeros_like(out))
    assert nv.lib().nvfp4_packed_weight_bytes(20, 0) == 0
