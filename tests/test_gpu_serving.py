"""GPU parity of the serving-path companions against the oracle, bit for bit: the FP8 E4M3 KV-cache
codec (quantize, dequantize, static scale), the fold-in repair (single scale arrays and whole fused
groups, then the GEMM on the folded weights), and RMSNorm fused with the NVFP4 quantizer."""
import numpy as np
import pytest
import torch

import nvfp4_w4a4_quantized_quantize_amd as nv
import oracle
import workloads as wl
from gpu_common import DEV, check_fp32, dev_bf16, dev_u8, host, padded_u8

pytestmark = pytest.mark.gpu


def bf16_bits(a) -> np.ndarray:
    return wl.f32_to_bf16_bits(np.asarray(a, dtype=np.float32))


def specials_mixed(rng, rows, cols, spread=6.0):
    """Heavy-tailed bf16 bits with infinities, NaN, signed zeros and subnormals sprinkled in."""
    x = rng.standard_normal((rows, cols)) * np.exp(rng.uniform(-spread, spread, (rows, 1)))
    bits = bf16_bits(x)
    n = bits.size
    idx = rng.choice(n, size=min(n, 64), replace=False)
    pool = np.array([0x7F80, 0xFF80, 0x7FC0, 0x8000, 0x0000, 0x0001, 0x8001, 0x7F7F, 0xFF7F], np.uint16)
    bits.reshape(-1)[idx] = pool[np.arange(len(idx)) % len(pool)]
    return bits


def strided_bf16(bits: np.ndarray, extra: int = 8) -> torch.Tensor:
    rows, cols = bits.shape
    buf = torch.zeros((rows, cols + extra), dtype=torch.bfloat16, device=DEV)
    buf[:, :cols] = dev_bf16(bits)
    return buf[:, :cols]


def bits_of(t: torch.Tensor) -> np.ndarray:
    return host(t.contiguous().view(torch.int16)).view(np.uint16)


# ------------------------------------------------------------------ FP8 KV codec
@pytest.mark.parametrize("rows,cols,strided", [(1, 16, False), (3, 144, True), (257, 1024, False),
                                               (64, 128, True), (4096, 1024, False), (1, 48, False)])
@pytest.mark.parametrize("s", [0.0123, 2.0 ** -110, 2.0 ** -85, 2.0 ** -79, 3.0e30])
def test_kv_quantize_bit_exact(rows, cols, strided, s):
    rng = np.random.default_rng(rows * 31 + cols)
    x = specials_mixed(rng, rows, cols, spread=8.0 if s < 1 else 40.0)
    xd = strided_bf16(x) if strided else dev_bf16(x)
    s = float(np.float32(s))
    q = nv.kv_quantize(xd, s)
    ref = oracle.kv_quantize(x, s)
    got = host(q)
    bad = got != ref
    assert not bad.any(), f"{bad.sum()} codes differ, e.g. x={x[bad][:4]} got={got[bad][:4]} want={ref[bad][:4]}"


@pytest.mark.parametrize("s", [0.0123, 1.0, 2.0 ** -120, 1.5e36])
def test_kv_dequantize_all_codes(s):
    q = np.tile(np.arange(256, dtype=np.uint8), (3, 1))
    s = float(np.float32(s))
    y = nv.kv_dequantize(dev_u8(q), s)
    assert (bits_of(y) == oracle.kv_dequantize(q, s)).all()


def test_kv_dequantize_strided_and_scale():
    rng = np.random.default_rng(11)
    rows, cols = 37, 208
    q = rng.integers(0, 256, size=(rows, cols), dtype=np.uint8)
    qbuf = torch.zeros((rows, 224), dtype=torch.uint8, device=DEV)
    qbuf[:, :cols] = dev_u8(q)
    ybuf = torch.full((rows, 216), float("nan"), dtype=torch.bfloat16, device=DEV)
    nv.kv_dequantize(qbuf[:, :cols], 0.07, out=ybuf[:, :cols])
    assert (bits_of(ybuf[:, :cols]) == oracle.kv_dequantize(q, np.float32(0.07))).all()
    assert torch.isnan(ybuf[:, cols:]).all()
    x = bf16_bits(rng.standard_normal((512, 128)) * 5)
    s = host(nv.kv_scale(dev_bf16(x)))[0]
    assert np.float32(s).view(np.uint32) == oracle.kv_scale(x).view(np.uint32)


def test_kv_cache_full_size_round_trip():
    """A 32K-token prefill's K cache of one attention layer: 32768 tokens x 8 KV heads x 128 dims, with
    a scale calibrated on another draw (static, shipped); codes and the dequantized cache bit-exact."""
    rng = np.random.default_rng(32768)
    calib = bf16_bits(rng.standard_normal((4096, 1024)) * 2.0)
    s = float(oracle.kv_scale(calib))
    x = bf16_bits(rng.standard_normal((32768, 1024)) * 2.0)
    q = nv.kv_quantize(dev_bf16(x), s)
    ref = oracle.kv_quantize(x, s)
    assert (host(q) == ref).all()
    y = nv.kv_dequantize(q, s)
    assert (bits_of(y) == oracle.kv_dequantize(ref, s)).all()


# ------------------------------------------------------------------ fold-in repair
@pytest.mark.parametrize("ratio", [1.0, 1 / 1.82, 1 / 2.75, 0.37, 2.0 ** -7, 2.0 ** -20])
def test_fold_scales_all_bytes(ratio):
    b = np.tile(np.arange(256, dtype=np.uint8), (5, 2))
    r = np.float32(ratio)
    d = dev_u8(b)
    nv.fold_scales(d, float(r))
    assert (host(d) == oracle.fold_scales(b, r)).all()


def test_fold_group_then_gemm():
    """The pages' repair on the GDN in_proj layout (six modules, separately calibrated), then the fused
    GEMM with the one common scale: folded scales bit-exact with the oracle, GEMM within the FP32
    bound of the oracle's exact result on the folded weights, and within 2^-4 of the exact
    per-segment result (the A/B of the two repairs)."""
    case = wl.C5
    K, M = case.K, 96
    rng = np.random.default_rng(7)
    seg_rows = [s.n // 16 for s in case.segments]  # the layout at 1/16 of the width
    ws, gs = [], []
    for i, n in enumerate(seg_rows):
        wb = bf16_bits(rng.standard_normal((n, K)) * [1.0, 1.25, 1.82, 1.0, 2.75, 1.0][i])
        g = oracle.global_scale(wb)
        ws.append(oracle.quantize(wb, g))
        gs.append(g)
    wc = np.concatenate([c for c, _ in ws])
    wsc = np.concatenate([s for _, s in ws])
    G_ref, folded = oracle.fold_group([s for _, s in ws], gs)
    d_scales = padded_u8(wsc)
    G = nv.fold_group(d_scales, seg_rows, [float(g) for g in gs])
    assert np.float32(G) == G_ref
    assert (host(d_scales) == np.concatenate(folded)).all()
    # GEMM on the folded weights, one segment with G
    xb = bf16_bits(rng.standard_normal((M, K)))
    g_a = oracle.global_scale(xb)
    ac, as_ = oracle.quantize(xb, g_a)
    (out,) = nv.gemm(padded_u8(ac), padded_u8(as_), float(g_a), padded_u8(wc), d_scales,
                     [nv.Segment(wc.shape[0], G)])
    y, T = oracle.gemm_rows(ac, as_, g_a, wc, np.concatenate(folded), [0, wc.shape[0]],
                            np.array([G_ref], np.float32), np.arange(M))
    check_fp32(host(out), y, T, "folded GEMM")
    bounds = np.concatenate([[0], np.cumsum(seg_rows)])
    y_exact, T_exact = oracle.gemm_rows(ac, as_, g_a, wc, wsc, bounds, np.array(gs, np.float32), np.arange(M))
    err = np.abs(host(out).astype(np.float64) - y_exact)
    assert (err <= (2.0 ** -4 + 2.0 ** -19) * T_exact + 1e-30).all()


# ------------------------------------------------------------------ RMSNorm + quantize
@pytest.mark.parametrize("rows,K", [(1, 16), (7, 5120), (300, 1040), (1024, 5120), (5, 48), (65, 17408)])
def test_rmsnorm_quantize_bit_exact(rows, K):
    rng = np.random.default_rng(rows + K)
    x = bf16_bits(rng.standard_normal((rows, K)) * np.exp(rng.uniform(-3, 3, (rows, 1))))
    hot = rng.choice(K, size=max(1, K // 1000), replace=False)
    x[:, hot] = bf16_bits(wl.bf16_bits_to_f32(x[:, hot]) * 50)
    w = bf16_bits(rng.uniform(0.2, 2.0, K))
    eps = np.float32(1e-6)
    y_ref, _ = oracle.rmsnorm(x, w, eps)
    # the static global scale of the consuming module, from the normalized activations
    g = oracle.global_scale(y_ref)
    c_ref, s_ref = oracle.quantize(y_ref, g)
    xd, wd = dev_bf16(x), dev_bf16(w)
    y = torch.empty((rows, K), dtype=torch.bfloat16, device=DEV)
    codes, scales = nv.rmsnorm_quantize(xd, wd, float(eps), float(g), y=y)
    yb = bits_of(y)
    bad = yb != y_ref
    assert not bad.any(), f"{bad.sum()} normalized values differ"
    assert (host(codes) == c_ref).all() and (host(scales) == s_ref).all()
    # without the optional output, the same codes
    c2, s2 = nv.rmsnorm_quantize(xd, wd, float(eps), float(g))
    assert torch.equal(c2, codes) and torch.equal(s2, scales)


def test_rmsnorm_quantize_strided_rows():
    rng = np.random.default_rng(3)
    rows, K = 33, 256
    x = bf16_bits(rng.standard_normal((rows, K)))
    w = bf16_bits(rng.uniform(0.5, 1.5, K))
    y_ref, _ = oracle.rmsnorm(x, w, np.float32(1e-5))
    g = oracle.global_scale(y_ref)
    c_ref, s_ref = oracle.quantize(y_ref, g)
    codes, scales = nv.rmsnorm_quantize(strided_bf16(x, 24), dev_bf16(w), 1e-5, float(g))
    assert (host(codes) == c_ref).all() and (host(scales) == s_ref).all()
