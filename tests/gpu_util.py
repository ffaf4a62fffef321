"""Helpers shared by the GPU parity tests (device transfer of bf16 bits)."""
import numpy as np


def to_dev_bf16(bits: np.ndarray):
    import torch
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16))
    return t.to("cuda").view(torch.bfloat16)


def to_dev_u8(arr: np.ndarray):
    import torch
    return torch.from_numpy(np.ascontiguousarray(arr, dtype=np.uint8)).to("cuda")


def gpu_available() -> bool:
    try:
        import torch
        return torch.cuda.is_available()
    except Exception:
        return False
