"""Helpers shared by the GPU parity tests: device upload and the acceptance bounds.

Acceptance (stated once here, used by every GEMM parity test):
  * codes, scale bytes and global scales: bit-exact with the oracle;
  * FP32 GEMM output: |gpu - y| <= 2^-20 * T, with y the oracle's exact result and
    T = g_a * g_w * sum_k |a_k w_k| (the FP32-accumulation bound the method is held to);
  * bf16 output: |gpu - y| <= tol + 2^-8 (|y| + tol) (plus half a bf16 ulp of rounding);
  * gates (FP32): first-order propagation of tol through the gate plus 2^-20 relative for the
    GPU's own exp/log1p and an underflow floor.
"""
import numpy as np
import torch

DEV = "cuda"


def dev_bf16(bits: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits, dtype=np.uint16).view(np.int16)).to(DEV).view(torch.bfloat16)


def dev_u8(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.uint8)).to(DEV)


def host(t: torch.Tensor) -> np.ndarray:
    torch.cuda.synchronize()
    return t.contiguous().cpu().numpy()


def padded_u8(a: np.ndarray) -> torch.Tensor:
    """Upload a uint8 [rows, cols] array into a device buffer whose row stride is a multiple of 16."""
    rows, cols = a.shape
    buf = torch.zeros((rows, (cols + 15) // 16 * 16), dtype=torch.uint8, device=DEV)
    buf[:, :cols] = torch.from_numpy(np.ascontiguousarray(a, dtype=np.uint8)).to(DEV)
    return buf[:, :cols]


def tol_fp32(T: np.ndarray) -> np.ndarray:
    return 2.0 ** -20 * T


def check_fp32(gpu: np.ndarray, y: np.ndarray, T: np.ndarray, what: str = "") -> float:
    err = np.abs(gpu.astype(np.float64) - y)
    bad = err > tol_fp32(T)
    assert not bad.any(), f"{what}: {bad.sum()} of {bad.size} outside 2^-20*T; worst at {np.argwhere(bad)[:3]}"
    return float(np.max(err / np.maximum(T, 1e-300)))


def check_bf16(gpu_bf16: torch.Tensor, y: np.ndarray, T: np.ndarray, what: str = "") -> None:
    g = host(gpu_bf16.float()).astype(np.float64)
    tol = tol_fp32(T)
    bad = np.abs(g - y) > tol + 2.0 ** -8 * (np.abs(y) + tol)
    assert not bad.any(), f"{what}: {bad.sum()} bf16 outputs outside tolerance"


def check_sigmoid(gpu: np.ndarray, y: np.ndarray, T: np.ndarray, oracle_beta: np.ndarray) -> None:
    b = oracle_beta
    bound = b * (1 - b) * tol_fp32(T) + 2.0 ** -20 * b + 2.0 ** -126
    bad = np.abs(gpu.astype(np.float64) - b) > bound
    assert not bad.any(), f"{bad.sum()} sigmoid outputs outside tolerance"


def check_decay(gpu: np.ndarray, y: np.ndarray, T: np.ndarray, oracle_alpha: np.ndarray,
                a_log: np.ndarray, dt_bias: np.ndarray) -> None:
    a = oracle_alpha
    z = y + dt_bias.astype(np.float64)[None, :]
    sig = np.exp(-np.logaddexp(0.0, -z))  # logistic(z) without overflow for large |z|
    ln_a = np.log(np.maximum(a, 1e-300))
    bound = a * np.exp(a_log.astype(np.float64))[None, :] * sig * tol_fp32(T) + 2.0 ** -20 * a * (1 + np.abs(ln_a)) + 2.0 ** -126
    bad = np.abs(gpu.astype(np.float64) - a) > bound
    assert not bad.any(), f"{bad.sum()} decay outputs outside tolerance"
