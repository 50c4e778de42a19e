"""Storage-size closed form (pinned to the weight-memory figures the pages print) and the seeded
input generator's contract (CPU only)."""
import numpy as np

import oracle
import workloads
from conftest import read_golden

FIG = {ln.split()[0]: float(ln.split()[1]) for ln in read_golden("page_figures.txt")}


def test_nvfp4_storage_is_4_5_bits_per_weight():
    rng = np.random.default_rng(0)
    N, K = 48, 320
    x = workloads.f32_to_bf16_bits(rng.standard_normal((N, K)).astype(np.float32))
    codes, scales = oracle.quantize(x, oracle.global_scale(x))
    assert codes.nbytes + scales.nbytes == N * K * 9 // 16  # 0.5625 B = 4.5 bits per element
    assert FIG["block_size"] == 16


def test_page_weight_memory_is_consistent_with_4_5_bits():
    # Linear layers in NVFP4 (0.5625 B/param) and the rest in BF16 (2 B/param) must explain
    # 50.13 GiB -> 17.53 GiB with a fraction of linear parameters in (0, 1).
    bf16, nv = FIG["weights_bf16_gib"], FIG["weights_nvfp4_gib"]
    total_params = bf16 / 2.0
    linear = (bf16 - nv) / (2.0 - 0.5625)
    frac = linear / total_params
    assert 0.85 < frac < 0.95  # about 24.4e9 of 26.9e9 parameters
    assert FIG["linear_layers_total"] == FIG["linear_layers_gdn"] + FIG["linear_layers_attention"] + FIG["linear_layers_mlp"]


def test_generator_is_deterministic_and_chunk_independent():
    case = workloads.C2
    a = workloads.draw_x(case, 0, 250, 600)
    b = np.concatenate([workloads.draw_x(case, 0, 250, 256), workloads.draw_x(case, 0, 256, 600)])
    assert (a == b).all()
    assert (workloads.draw_x(case, 1, 0, 10) != workloads.draw_x(case, 0, 0, 10)).any()


def test_generator_statistics():
    case = workloads.C2
    x = workloads.bf16_bits_to_f32(workloads.draw_x(case, 0, 0, 512)).astype(np.float64)
    cols = np.argsort(np.abs(x).mean(axis=0))[-5:]
    assert workloads.n_outliers(5120) == 5 and workloads.n_outliers(17408) == 17
    assert np.abs(x[:, cols]).mean() > 20 * np.median(np.abs(x))  # hot channels
    assert np.abs(x).max() / np.sqrt((x ** 2).mean()) > 30        # heavy tail
    w = workloads.bf16_bits_to_f32(workloads.draw_w(workloads.C5, 4, 0)).astype(np.float64)
    assert abs(w.std() * np.sqrt(5120) - 2.75) < 0.05
    assert workloads.C5.N == 12352 and list(workloads.C5.seg_bounds) == [0, 2048, 4096, 8192, 12288, 12320, 12352]
    a_log, dt = workloads.draw_gate_params(workloads.C5, 5)
    assert a_log.shape == (32,) and dt.dtype == np.float32


def test_bf16_rounding_is_nearest_even():
    f = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -2.5, 1.0 + 2 ** -8 + 2 ** -20], dtype=np.float32)
    b = workloads.f32_to_bf16_bits(f)
    assert list(workloads.bf16_bits_to_f32(b)) == [1.0, 1.0, 1.0 + 2 ** -6, -2.5, 1.0 + 2 ** -7]


def test_bench_refuses_more_than_one_gpu():
    """bench.py measures one GPU; asked for more it says so and exits non-zero before touching a GPU."""
    import os
    import subprocess
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    res = subprocess.run([sys.executable, os.path.join(root, "bench.py"), "--gpus", "2"], capture_output=True,
                         text=True, timeout=300)
    assert res.returncode != 0
    assert "one GPU" in res.stderr and res.stdout == ""
