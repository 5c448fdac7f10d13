"""Helpers for the GPU parity tests: moving seeded host arrays to the device as
the same bytes, and reading results back as bytes or float64."""

import sys

import numpy as np
import torch

DEV = "cuda"


def say(*a):
    """Name the case before a GPU step (flushed, so a fault still leaves it)."""
    print("[case]", *a, flush=True)
    sys.stdout.flush()


def to_dev(arr: np.ndarray) -> torch.Tensor:
    """float32 -> float32 tensor; uint16 (bf16 patterns) -> bfloat16 tensor; uint8 -> uint8."""
    t = torch.from_numpy(np.ascontiguousarray(arr))
    if arr.dtype == np.uint16:
        t = t.view(torch.bfloat16)
    return t.to(DEV)


def raw(t: torch.Tensor) -> np.ndarray:
    """Device tensor -> host array of the same bytes (bf16 as uint16)."""
    t = t.detach().contiguous().cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def f64(a: np.ndarray) -> np.ndarray:
    """uint16 bf16 patterns or float32 -> float64 (exact), for comparisons."""
    if a.dtype == np.uint16:
        return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return a.astype(np.float64)


def sentinel_like(shape, dtype) -> torch.Tensor:
    """Output buffer prefilled with NaN bytes (0xFF), so unwritten elements show."""
    t = torch.empty(shape, dtype=dtype, device=DEV)
    t.view(torch.uint8).fill_(0xFF)
    return t


def rand_bits(rng, shape, dtype: str) -> np.ndarray:
    """Seeded N(0,1) values in storage form (uint16 bf16 patterns or float32)."""
    from sequence_attention_video_amd.workloads import f32_to_bf16_bits
    x = rng.standard_normal(shape).astype(np.float32)
    return f32_to_bf16_bits(x) if dtype == "bf16" else x
