"""Helpers for the GPU parity tests: moving seeded numpy inputs to the device and
comparing results with the oracle."""
from __future__ import annotations

import sys

import numpy as np
import torch

DEV = "cuda:0"


def say(msg: str) -> None:
    """Name the case about to run on the GPU (flushed, so a hang or fault still shows it)."""
    print(f"[gpu] {msg}", flush=True)
    sys.stdout.flush()


def u8(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.uint8)).to(DEV)


def bf16(bits: np.ndarray) -> torch.Tensor:
    b = np.ascontiguousarray(bits, dtype=np.uint16).view(np.int16)
    return torch.from_numpy(b).view(torch.bfloat16).to(DEV)


def f32(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(DEV)


def i64(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int64)).to(DEV)


def i32(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(DEV)


def words(a: np.ndarray) -> torch.Tensor:
    """uint32 words as an int32 device tensor (same bits)."""
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.uint32).view(np.int32)).to(DEV)


def bits(t: torch.Tensor) -> np.ndarray:
    """bf16 / int16 device tensor -> uint16 bit patterns on the host."""
    torch.cuda.synchronize()
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def host_f32(t: torch.Tensor) -> np.ndarray:
    torch.cuda.synchronize()
    return t.float().cpu().numpy()


def rel_l2(got: np.ndarray, want: np.ndarray) -> float:
    got = np.asarray(got, dtype=np.float64)
    want = np.asarray(want, dtype=np.float64)
    den = np.linalg.norm(want)
    num = np.linalg.norm(got - want)
    return float(num / den) if den > 0 else float(num)


def bf16_values(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)
