"""nvfp4_gemm_noalloc (the allocation-free GEMM entry point) against nvfp4_gemm, through the C
interface: two calls in a row on shapes whose decode kernel splits K over workgroups (so the partial
sums live in the library's per-GPU scratch array), the second smaller than the first. Each call must
give bitwise the outputs of nvfp4_gemm with a caller workspace, and those are checked against the
oracle within the FP32 bound; a third call checks that a smaller call after a larger one does not
read the larger one's leftovers. Shapes needing more scratch than the fixed array are rejected."""
import numpy as np
import pytest
import torch

import nvfp4_w4a4_quantized_quantize_amd as nv
import oracle
from gpu_common import DEV, check_fp32, host, padded_u8

pytestmark = pytest.mark.gpu


def random_nvfp4(rng, rows, K):
    return (rng.integers(0, 256, size=(rows, K // 2), dtype=np.uint8),
            rng.integers(0x01, 0x7F, size=(rows, K // 16), dtype=np.uint8))


def operands(seed, M, N, K):
    rng = np.random.default_rng(seed)
    a, w = random_nvfp4(rng, M, K), random_nvfp4(rng, N, K)
    return a, w, [padded_u8(x) for x in (*a, *w)]


def segments(N, dtype=torch.float32):
    # two modules with their own global scales and a gate, as in the fused projections
    n1 = N // 2
    return [nv.Segment(n1, 0.37), nv.Segment(N - n1 - 32, 1.91, out_dtype=dtype),
            nv.Segment(32, 0.8, "sigmoid", torch.float32)]


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_noalloc_matches_gemm_on_two_calls_second_smaller(dtype):
    shapes = [(64, 5120, 17408, 11), (48, 2048, 8192, 12), (40, 1024, 5632, 13)]
    for M, N, K, seed in shapes:
        need = nv.lib().nvfp4_gemm_workspace_bytes(M, N, K)
        assert 0 < need <= nv.NOALLOC_SCRATCH_BYTES, (M, N, K, need)
        print(f"noalloc M={M} N={N} K={K}: {need} bytes of scratch", flush=True)
        a, w, (ac, as_, wc, ws) = operands(seed, M, N, K)
        ref = nv.gemm(ac, as_, 0.05, wc, ws, segments(N, dtype))
        got = nv.gemm_noalloc(ac, as_, 0.05, wc, ws, segments(N, dtype))
        torch.cuda.synchronize()
        for r, g in zip(ref, got):
            assert torch.equal(r.view(torch.int16 if r.dtype == torch.bfloat16 else torch.int32),
                               g.view(torch.int16 if g.dtype == torch.bfloat16 else torch.int32)), (M, N, K)
        if dtype == torch.float32:
            bounds = np.array([0, N // 2, N - 32, N])
            y, T = oracle.gemm_rows(a[0], a[1], np.float32(0.05), w[0], w[1], bounds,
                                    np.array([0.37, 1.91, 0.8], np.float32), np.arange(M))
            check_fp32(np.concatenate([host(got[0]), host(got[1])], axis=1), y[:, :N - 32], T[:, :N - 32],
                       f"noalloc M={M} N={N} K={K}")


def test_noalloc_rejects_shapes_beyond_its_scratch():
    M, N, K = 64, 40960, 17408  # 6 K splits x 40960 columns x 64 rows of FP32 = 60 MiB
    assert nv.lib().nvfp4_gemm_workspace_bytes(M, N, K) > nv.NOALLOC_SCRATCH_BYTES
    ac, as_ = nv.alloc_nvfp4(M, K, DEV)
    wc, ws = nv.alloc_nvfp4(N, K, DEV)
    with pytest.raises(nv.Nvfp4Error) as e:
        nv.gemm_noalloc(ac, as_, 1.0, wc, ws, [nv.Segment(N, 1.0)])
    assert e.value.status == 7 and "scratch" in str(e.value)


def test_noalloc_prefill_and_skinny_paths():
    """Shapes that need no scratch (prefill tiles, M <= 32) run through the same entry point."""
    for M, N, K, seed in [(300, 520, 272, 21), (16, 1000, 5120, 22)]:
        a, w, (ac, as_, wc, ws) = operands(seed, M, N, K)
        ref = nv.gemm(ac, as_, 0.5, wc, ws, [nv.Segment(N, 2.0)])[0]
        got = nv.gemm_noalloc(ac, as_, 0.5, wc, ws, [nv.Segment(N, 2.0)])[0]
        assert torch.equal(ref.view(torch.int32), got.view(torch.int32))
