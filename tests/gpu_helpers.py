"""Shared helpers for the GPU parity tests (moving seeded inputs to the device,
normwise error).  Expected values come only from the oracle or the golden
fixtures; nothing the GPU produced is fed back into the oracle."""

import sys

import numpy as np
import pytest
import torch

import oracle


def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda:0")


def announce(msg):
    print(f"[gpu-test] {msg}", flush=True)
    sys.stdout.flush()


def bf16_to_dev(bits: np.ndarray) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16)
    return t.to(dev())


def u8_to_dev(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.uint8)).to(dev())


def f32_to_dev(v) -> torch.Tensor:
    return torch.tensor([float(np.float32(v))], dtype=torch.float32, device=dev())


def to_bits(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().view(torch.int16).numpy().view(np.uint16)


def to_np(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().numpy()


def normwise(c_bits: np.ndarray, ref64: np.ndarray) -> float:
    c = oracle.bf16_bits_to_f32(c_bits).astype(np.float64)
    den = np.linalg.norm(ref64)
    return float(np.linalg.norm(c - ref64) / den) if den > 0 else float(np.linalg.norm(c))


def gemm_errors(c_bits, c64, c_ref_bits):
    """(‖C−C_ref‖/‖C_ref‖, ‖C−C64‖/‖C64‖) with C_ref the bf16-rounded oracle."""
    ref = oracle.bf16_bits_to_f32(c_ref_bits).astype(np.float64)
    return normwise(c_bits, ref), normwise(c_bits, c64)


#: normwise tolerance on GEMM outputs, from the required relative error bound
GEMM_TOL = 2e-3
