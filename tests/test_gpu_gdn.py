"""GPU parity of the Gated DeltaNet recurrence (FP32 on the GPU) against the oracle (double).

Tolerance: the GPU result must be within 8 times the error of the oracle's own float32 twin (the
same recurrence in binary32, sequential sums) on the same input, plus 2^-22 of the output scale.
Both are FP32 evaluations of a contractive recurrence (unit keys, decay and write strength in
(0, 1]); they differ only in summation order, so their errors are of the same size."""
import numpy as np
import pytest
import torch

import nvfp4_w4a4_quantized_quantize_amd as nv
import oracle
import workloads as wl
from gpu_common import DEV, dev_bf16, host

pytestmark = pytest.mark.gpu


def to_value_major(S):
    """[B, Hv, D key, D value] -> the library's value-major state layout (each head's S^T)."""
    return np.ascontiguousarray(np.swapaxes(np.asarray(S), 2, 3))


def run_gpu(q, k, v, alpha, beta, B, T, Hv, S0=None):
    state = torch.zeros((B, Hv, 128, 128), dtype=torch.float32, device=DEV)
    if S0 is not None:
        state.copy_(torch.from_numpy(to_value_major(np.asarray(S0, np.float32))))
    o = nv.gdn_recurrence(dev_bf16(q), dev_bf16(k), dev_bf16(v), torch.from_numpy(alpha).to(DEV),
                          torch.from_numpy(beta).to(DEV), state, B, T)
    return host(o).astype(np.float64), to_value_major(host(state).astype(np.float64))


def check(o, S, q, k, v, alpha, beta, B, T, S0=None, what=""):
    o64, S64 = oracle.gdn_recurrence(q, k, v, alpha, beta, B, T, S0=S0)
    o32, S32 = oracle.gdn_recurrence(q, k, v, alpha, beta, B, T, S0=S0, f32=True)
    for got, ref, twin, name in ((o, o64, o32, "o"), (S, S64, S32, "state")):
        tol = 8 * np.abs(twin - ref).max() + 2.0 ** -22 * np.abs(ref).max()
        err = np.abs(got - ref).max()
        assert err <= tol, f"{what} {name}: max error {err:.3g} > tolerance {tol:.3g}"
    return np.abs(o - o64).max() / max(np.abs(o64).max(), 1e-30)


@pytest.mark.parametrize("B,T", [(1, 1), (2, 7), (1, 8), (3, 37), (1, 1000)])
def test_small_shapes(B, T):
    case = wl.GdnCase("t", 70, B, T, Hv=4, Hk=2)
    q, k, v, a, b = wl.draw_gdn(case)
    o, S = run_gpu(q, k, v, a, b, B, T, 4)
    check(o, S, q, k, v, a, b, B, T, what=f"B={B} T={T}")


def test_decode_step_batch_with_state():
    """One decode step for 64 sequences, all 32 value heads, from a state built by 24 earlier tokens."""
    case = wl.GDN_DECODE
    q0, k0, v0, a0, b0 = wl.draw_gdn(case, seed=1, T=24)
    _, S0 = oracle.gdn_recurrence(q0, k0, v0, a0, b0, case.B, 24)
    q, k, v, a, b = wl.draw_gdn(case)
    o, S = run_gpu(q, k, v, a, b, case.B, 1, case.Hv, S0=S0.astype(np.float32))
    check(o, S, q, k, v, a, b, case.B, 1, S0=S0.astype(np.float32).astype(np.float64), what="decode")


def run_split(q, k, v, a, b, B, T, Hv, cuts):
    """The B sequences of T tokens fed in consecutive calls of the given lengths, carrying the state on
    the GPU; returns the outputs re-assembled in [b][t] order and the final state."""
    state = torch.zeros((B, Hv, 128, 128), dtype=torch.float32, device=DEV)
    bounds = np.concatenate([[0], np.cumsum(cuts)])
    assert bounds[-1] == T
    sel = lambda x, lo, hi: np.concatenate([x[s * T + lo:s * T + hi] for s in range(B)])  # noqa: E731
    parts = []
    for lo, hi in zip(bounds[:-1], bounds[1:]):
        parts.append(host(nv.gdn_recurrence(dev_bf16(sel(q, lo, hi)), dev_bf16(sel(k, lo, hi)),
                                            dev_bf16(sel(v, lo, hi)), torch.from_numpy(sel(a, lo, hi)).to(DEV),
                                            torch.from_numpy(sel(b, lo, hi)).to(DEV), state, B, int(hi - lo))))
    o = np.concatenate([np.concatenate([p[s * n:(s + 1) * n] for p, n in zip(parts, np.diff(bounds))])
                        for s in range(B)])
    return o, to_value_major(host(state))


@pytest.mark.parametrize("T,cuts", [(24, (11, 13)), (192, (64, 128)), (200, (128, 64, 8)), (256, (64, 64, 128))])
def test_state_carries_across_calls_bitwise(T, cuts):
    """Calls that split a sequence where the kernel's own blocking splits it give the same bits as one
    call: under 32 tokens the token-by-token kernel, at chunk (64-token) boundaries the chunked one
    (the last call of the (128, 64, 8) split is token by token, so only the first 192 tokens and the
    outputs of that prefix are compared bitwise; the rest within the bound)."""
    case = wl.GdnCase("t", 71, 2, T, Hv=4, Hk=2)
    q, k, v, a, b = wl.draw_gdn(case)
    o, S = run_gpu(q, k, v, a, b, 2, T, 4)
    o2, S2 = run_split(q, k, v, a, b, 2, T, 4, cuts)
    if cuts[-1] >= 32:
        assert (o2 == o.astype(np.float32)).all() and (S2 == S.astype(np.float32)).all()
    else:
        head = T - cuts[-1]
        rows = np.concatenate([np.arange(s * T, s * T + head) for s in range(2)])
        assert (o2[rows] == o.astype(np.float32)[rows]).all()
        check(o2.astype(np.float64), S2.astype(np.float64), q, k, v, a, b, 2, T, what=f"split {cuts}")


@pytest.mark.parametrize("cuts", [(19, 21), (1, 39), (33, 7)])
def test_state_carries_across_calls(cuts):
    """Any split (calls that take either kernel, chunks that start anywhere) meets the bound of one call."""
    B, T = 2, 40
    case = wl.GdnCase("t", 74, B, T, Hv=4, Hk=2)
    q, k, v, a, b = wl.draw_gdn(case)
    o, S = run_split(q, k, v, a, b, B, T, 4, cuts)
    check(o.astype(np.float64), S.astype(np.float64), q, k, v, a, b, B, T, what=f"split {cuts}")


@pytest.mark.parametrize("T", [32, 33, 63, 64, 65, 127, 129])
def test_chunk_boundaries_from_a_state(T):
    """Lengths around the 64-token chunk (half a chunk, one full chunk, a one-token tail, ...), two sequences, starting
    from states built by 20 earlier tokens."""
    B, Hv = 2, 4
    case = wl.GdnCase("t", 75, B, T, Hv=Hv, Hk=2)
    q0, k0, v0, a0, b0 = wl.draw_gdn(case, seed=5, T=20)
    _, S0 = oracle.gdn_recurrence(q0, k0, v0, a0, b0, B, 20)
    S0 = S0.astype(np.float32).astype(np.float64)
    q, k, v, a, b = wl.draw_gdn(case)
    o, S = run_gpu(q, k, v, a, b, B, T, Hv, S0=S0)
    check(o, S, q, k, v, a, b, B, T, S0=S0, what=f"T={T}")


@pytest.mark.parametrize("Hv,Hk", [(4, 4), (8, 2), (3, 1)])
def test_chunked_head_grouping(Hv, Hk):
    T = 70
    case = wl.GdnCase("t", 76, 1, T, Hv=Hv, Hk=Hk)
    q, k, v, a, b = wl.draw_gdn(case)
    o, S = run_gpu(q, k, v, a, b, 1, T, Hv)
    check(o, S, q, k, v, a, b, 1, T, what=f"Hv={Hv} Hk={Hk}")


def test_chunked_extreme_gates_and_repeated_keys():
    """Decays of exactly 0 and 1 and products that underflow inside a chunk (alpha = 1e-30), write
    strengths 0 and 1, and runs of one repeated key (the delta rule then overwrites the same slot;
    the triangular system has its largest off-diagonal weights)."""
    B, T, Hv = 1, 96, 4
    case = wl.GdnCase("t", 77, B, T, Hv=Hv, Hk=2)
    q, k, v, a, b = wl.draw_gdn(case)
    rng = np.random.default_rng(77)
    a = a.copy()
    b = b.copy()
    a[rng.random(a.shape) < 0.05] = 0.0
    a[rng.random(a.shape) < 0.05] = 1e-30
    a[rng.random(a.shape) < 0.2] = 1.0
    b[rng.random(b.shape) < 0.1] = 0.0
    b[rng.random(b.shape) < 0.2] = 1.0
    k = k.copy()
    k[10:30] = k[10]
    k[40:72:2] = k[40]
    o, S = run_gpu(q, k, v, a, b, B, T, Hv)
    assert np.isfinite(o).all() and np.isfinite(S).all()
    check(o, S, q, k, v, a, b, B, T, what="extreme gates")


def test_inputs_as_slices_of_the_fused_projection_output():
    """q, k, v as column slices of the fused in_proj output (row stride 12352) and the gates as the two
    columns blocks of one [T, 64] FP32 buffer, exactly as the GEMM's segments would leave them."""
    T = 50
    case = wl.GdnCase("t", 72, 1, T)
    q, k, v, a, b = wl.draw_gdn(case)
    fused = torch.zeros((T, 12352), dtype=torch.bfloat16, device=DEV)
    fused[:, :2048], fused[:, 2048:4096], fused[:, 4096:8192] = dev_bf16(q), dev_bf16(k), dev_bf16(v)
    gates = torch.zeros((T, 64), dtype=torch.float32, device=DEV)
    gates[:, :32], gates[:, 32:] = torch.from_numpy(b).to(DEV), torch.from_numpy(a).to(DEV)
    state = torch.zeros((1, 32, 128, 128), dtype=torch.float32, device=DEV)
    o = nv.gdn_recurrence(fused[:, :2048], fused[:, 2048:4096], fused[:, 4096:8192], gates[:, 32:], gates[:, :32],
                          state, 1, T)
    check(host(o).astype(np.float64), to_value_major(host(state).astype(np.float64)), q, k, v, a, b, 1, T,
          what="slices")


def test_prefill_8192_tokens_all_heads():
    case = wl.GdnCase("t", 73, 1, 8192)
    q, k, v, a, b = wl.draw_gdn(case)
    o, S = run_gpu(q, k, v, a, b, 1, 8192, 32)
    rel = check(o, S, q, k, v, a, b, 1, 8192, what="prefill 8192")
    print(f"prefill 8192: max |o - exact| / max |o| = {rel:.3g}")


def test_prefill_32768_tokens_all_heads():
    """The 32768-token prefill the companion benchmark times (same seeded inputs), every token, head
    and state entry against the double oracle; on top of the global bound, no stretch of the sequence
    may be worse than 8 times the float32 twin's error over a window of 512 tokens around it."""
    case = wl.GDN_PREFILL
    q, k, v, a, b = wl.draw_gdn(case)
    T = case.T
    print(f"{case.name}: GPU", flush=True)
    o, S = run_gpu(q, k, v, a, b, 1, T, case.Hv)
    print(f"{case.name}: oracle (double and float32 twin)", flush=True)
    o64, S64 = oracle.gdn_recurrence(q, k, v, a, b, 1, T)
    o32, S32 = oracle.gdn_recurrence(q, k, v, a, b, 1, T, f32=True)
    for got, ref, twin, name in ((o, o64, o32, "o"), (S, S64, S32, "state")):
        tol = 8 * np.abs(twin - ref).max() + 2.0 ** -22 * np.abs(ref).max()
        err = np.abs(got - ref).max()
        assert err <= tol, f"prefill 32768 {name}: max error {err:.3g} > tolerance {tol:.3g}"
    floor = 2.0 ** -22 * np.abs(o64).max()
    err_t = np.abs(o - o64).max(axis=1)
    twin_t = np.abs(o32 - o64).max(axis=1)
    win = 512
    pad = np.concatenate([np.zeros(win // 2), twin_t, np.zeros(win // 2)])
    local = np.lib.stride_tricks.sliding_window_view(pad, win)[:T].max(axis=1)
    bad = np.nonzero(err_t > 8 * local + floor)[0]
    assert bad.size == 0, f"tokens {bad[:8]} exceed 8x the local float32 error"
    rel = np.abs(o - o64).max() / np.abs(o64).max()
    print(f"prefill 32768: max |o - exact| / max |o| = {rel:.3g}", flush=True)
