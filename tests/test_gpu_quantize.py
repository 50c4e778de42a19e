"""GPU parity of nvfp4_global_scale and nvfp4_quantize against the oracle: bit-exact codes, scales
and global scales on the workload tensors, on every finite bf16 value over a grid of block scales,
and on edge shapes and extreme global scales."""
import numpy as np
import pytest
import torch

import nvfp4_w4a4_quantized_quantize_amd as nv
import oracle
import workloads as wl
from conftest import read_golden
from gpu_common import DEV, dev_bf16, host

pytestmark = pytest.mark.gpu


def gpu_quantize(bits: np.ndarray, g) -> tuple[np.ndarray, np.ndarray]:
    c, s = nv.quantize(dev_bf16(bits), float(np.float32(g)))
    return host(c), host(s)


def assert_same_quant(bits: np.ndarray, g, what: str):
    gc, gs = gpu_quantize(bits, g)
    rc, rs = oracle.quantize(bits, np.float32(g))
    bad_s = np.argwhere(gs != rs)
    assert bad_s.size == 0, f"{what}: {len(bad_s)} scale bytes differ, first {bad_s[:3]}"
    bad_c = np.argwhere(gc != rc)
    assert bad_c.size == 0, f"{what}: {len(bad_c)} code bytes differ, first {bad_c[:3]}"


def test_library_loads_and_exports():
    L = nv.lib()
    for name in nv.EXPORTED:
        assert hasattr(L, name)


def test_worked_blocks_golden():
    for ln in read_golden("worked_blocks.txt"):
        name, g, xs, sc, cb = [p.strip() for p in ln.split("|")]
        bits = wl.f32_to_bf16_bits(np.array([float(v) for v in xs.split()], np.float32))[None, :]
        c, s = gpu_quantize(bits, np.float32(float(g)))
        assert s[0, 0] == int(sc, 16), name
        assert list(c[0]) == [int(b, 16) for b in cb.split()], name


@pytest.mark.parametrize("which", ["C1_x", "C1_w", "C2_x_head", "zeros", "heavy_odd_K", "tiny_values"])
def test_global_scale_bit_exact(which):
    rng = np.random.default_rng(3)
    if which == "C1_x":
        bits = wl.draw_x(wl.C1)
    elif which == "C1_w":
        bits = wl.draw_w(wl.C1, 0)
    elif which == "C2_x_head":
        bits = wl.draw_x(wl.C2, 0, 0, 512)
    elif which == "zeros":
        bits = np.zeros((7, 64), np.uint16)
    elif which == "heavy_odd_K":
        bits = wl.f32_to_bf16_bits(rng.standard_t(3, (33, 100)).astype(np.float32) * 7)
    else:
        bits = wl.f32_to_bf16_bits(rng.standard_normal((5, 24)).astype(np.float32) * np.float32(1e-38))
    K = bits.shape[1]
    buf = torch.zeros((bits.shape[0], (K + 7) // 8 * 8), dtype=torch.bfloat16, device=DEV)
    buf[:, :K] = dev_bf16(bits)
    g = host(nv.global_scale(buf[:, :K]))[0]
    assert np.float32(g).view(np.uint32) == oracle.global_scale(bits).view(np.uint32)


@pytest.mark.parametrize("name,rows", [("C1_x", None), ("C1_w", None), ("C2_x", None), ("C3_down_64_x", None),
                                       ("C5_x_head", 2048), ("C5_w_b", None)])
def test_workload_tensors_bit_exact(name, rows):
    if name == "C1_x":
        bits = wl.draw_x(wl.C1)
    elif name == "C1_w":
        bits = wl.draw_w(wl.C1, 0)
    elif name == "C2_x":
        bits = wl.draw_x(wl.C2)
    elif name == "C3_down_64_x":
        bits = wl.draw_x(wl.C3(64, "down"))
    elif name == "C5_x_head":
        bits = wl.draw_x(wl.C5, 0, 0, rows)
    else:
        bits = wl.draw_w(wl.C5, 4)
    g = oracle.global_scale(bits)
    print(f"{name}: shape {bits.shape}, g = {g!r}", flush=True)
    assert_same_quant(bits, g, name)


def _grid_blocks(g: float) -> np.ndarray:
    """Blocks [anchor, 15 values] where the anchor fixes the block maximum and the values run over every
    bf16 value within 5 binades below it, for anchors spanning all 128 bf16 significands at four scale
    levels (subnormal, small, mid and saturating E4M3 scales)."""
    blocks = []
    for s_target in (2.0 ** -8, 1.0, 100.0, 1000.0):
        for m in range(0, 128, 1):
            a = 6.0 * g * s_target * (1 + m / 128.0)
            ab = int(wl.f32_to_bf16_bits(np.array([a], np.float32))[0])
            lo = int(wl.f32_to_bf16_bits(np.array([a * 2.0 ** -5], np.float32))[0])
            vals = np.arange(lo, ab + 1, dtype=np.uint16)
            vals = np.concatenate([vals, vals | np.uint16(0x8000)])
            pad = (-len(vals)) % 15
            vals = np.concatenate([vals, np.zeros(pad, np.uint16)]).reshape(-1, 15)
            blocks.append(np.concatenate([np.full((vals.shape[0], 1), ab, np.uint16), vals], axis=1))
    out = np.concatenate(blocks)
    pad = (-out.shape[0]) % 64
    out = np.concatenate([out, np.zeros((pad, 16), np.uint16)])
    return out.reshape(-1, 64 * 16)


# the last two put block scales s * g on both sides of the fast division's lower edge (2^-80)
@pytest.mark.parametrize("g", [2.0 ** -6, 0.0173, 1.0 / 3.0, 3.14159e-3, 7.77e-8, 12.34, 2.0 ** -85, 3.7e-26])
def test_every_bf16_value_over_scale_grid(g):
    g = np.float32(g)
    bits = _grid_blocks(float(g))
    assert_same_quant(bits, g, f"grid g={g}")


def test_all_finite_bf16_patterns():
    # every finite bf16 pattern, shuffled into blocks, for several global scales
    pats = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    finite = (pats & 0x7F80) != 0x7F80
    pats = pats[finite]
    rng = np.random.default_rng(0)
    pats = pats[rng.permutation(pats.size)]
    pats = np.concatenate([pats, np.zeros((-pats.size) % 1024, np.uint16)]).reshape(-1, 1024)
    for g in [1e-30, 2.0 ** -100, 1e-3, 1.0, 1e30, 1e37]:
        assert_same_quant(pats, np.float32(g), f"all patterns g={g}")
    # sorted order: neighbouring magnitudes share blocks, so most values sit near the block maximum
    srt = np.sort(pats.ravel().view(np.uint16) & 0x7FFF).reshape(pats.shape)
    srt = srt | (np.arange(srt.size, dtype=np.uint16).reshape(srt.shape) % 3 == 0).astype(np.uint16) << 15
    for g in [2.0 ** -20, 0.37, 1e20]:
        assert_same_quant(srt, np.float32(g), f"sorted patterns g={g}")


@pytest.mark.parametrize("rows,K", [(1, 16), (3, 48), (5, 1040), (7, 1024 + 16), (64, 4096 + 32), (130, 17408)])
def test_edge_shapes(rows, K):
    rng = np.random.default_rng(rows * 7 + K)
    v = rng.standard_t(3, (rows, K)).astype(np.float32)
    v[rng.random((rows, K)) < 0.05] = 0.0
    v[rng.random((rows, K)) < 0.02] *= -0.0
    bits = wl.f32_to_bf16_bits(v)
    for g in [oracle.global_scale(bits), np.float32(1e-3), np.float32(50.0)]:
        assert_same_quant(bits, g, f"rows={rows} K={K} g={g}")


def test_strided_input_and_guard_bands():
    rows, K, ldx = 9, 96, 136
    rng = np.random.default_rng(1)
    full = wl.f32_to_bf16_bits(rng.standard_normal((rows, ldx)).astype(np.float32))
    x = dev_bf16(full)[:, :K]
    g = oracle.global_scale(full[:, :K])
    cbuf = torch.full((rows + 2, 64), 0xAB, dtype=torch.uint8, device=DEV)
    sbuf = torch.full((rows + 2, 32), 0xCD, dtype=torch.uint8, device=DEV)
    codes, scales = cbuf[1:rows + 1, :K // 2], sbuf[1:rows + 1, :K // 16]
    nv.quantize(x, float(g), codes, scales)
    cb, sb = host(cbuf), host(sbuf)
    rc, rs = oracle.quantize(full[:, :K], g)
    assert (cb[1:rows + 1, :K // 2] == rc).all() and (sb[1:rows + 1, :K // 16] == rs).all()
    assert (cb[0] == 0xAB).all() and (cb[-1] == 0xAB).all() and (cb[:, K // 2:] == 0xAB).all()
    assert (sb[0] == 0xCD).all() and (sb[-1] == 0xCD).all() and (sb[:, K // 16:] == 0xCD).all()


def test_zero_rows_is_a_no_op():
    x = torch.empty((0, 64), dtype=torch.bfloat16, device=DEV)
    c, s = nv.quantize(x, 1.0)
    assert c.shape == (0, 32) and s.shape == (0, 4)


def test_repeatable():
    bits = wl.draw_x(wl.C1)
    a = gpu_quantize(bits, 0.01)
    b = gpu_quantize(bits, 0.01)
    assert (a[0] == b[0]).all() and (a[1] == b[1]).all()
