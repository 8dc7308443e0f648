"""Helpers of the GPU parity tests: moving seeded host inputs to the device and
comparing results with the oracle.  Nothing here computes the decode step."""
import numpy as np
import pytest
import torch

DEV = "cuda:0"


def require_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")


def bf16_dev(bits: np.ndarray) -> torch.Tensor:
    """uint16 bf16 bit patterns -> device bfloat16 tensor."""
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(DEV).view(torch.bfloat16)


def f16_dev(bits: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(DEV).view(torch.float16)


def bits_host(t: torch.Tensor) -> np.ndarray:
    """Device 16-bit tensor -> uint16 bit patterns on the host."""
    torch.cuda.synchronize()
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def bytes_host(t: torch.Tensor) -> np.ndarray:
    torch.cuda.synchronize()
    return t.contiguous().view(torch.uint8).cpu().numpy().reshape(-1)


def sentinel_dev(shape, dtype) -> torch.Tensor:
    t = torch.empty(shape, dtype=dtype, device=DEV)
    t.view(torch.uint8).fill_(0xA5)
    return t


def rel_err_rows(got: np.ndarray, ref: np.ndarray) -> float:
    """Max over rows (last axis = head dim) of max_d |got - ref| / max_d |ref|."""
    got = np.asarray(got, dtype=np.float64).reshape(-1, ref.shape[-1])
    ref = np.asarray(ref, dtype=np.float64).reshape(-1, ref.shape[-1])
    num = np.abs(got - ref).max(axis=1)
    den = np.maximum(np.abs(ref).max(axis=1), 1e-30)
    return float((num / den).max())


def workspace(nbytes: int) -> torch.Tensor:
    return torch.empty(max(int(nbytes), 256), dtype=torch.uint8, device=DEV)
