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


U_BF16 = 2.0 ** -8      # bf16 unit roundoff (8 significant bits, round to nearest even)


def assert_bf16_pv_bound(got: np.ndarray, ref: np.ndarray, s: np.ndarray, V: np.ndarray):
    """Elementwise error bound of an attention output whose probabilities enter P.V as bf16 and whose result
    is rounded to bf16 (the MFMA chunk kernel).  s: [..., n] scaled scores (-inf where a key is not
    visible), V: [..., n, D] the values, ref / got: [..., D].  Rounding each p_k to bf16 (relative error
    <= u) while the denominator sums the unrounded p gives |o~ - o| <= u * w, w = sum_k p_k |v_k| /
    sum_k p_k; the bf16 output adds u * |o~|.  So |got - ref| <= u (1 + u) (w + |ref|), plus float32
    noise.  A key dropped or counted twice moves an element by p_k |v_k - o| / sum p, which this catches
    on short rows; the planted-key tests catch it on long ones."""
    p = np.exp(s - s.max(axis=-1, keepdims=True))
    w = np.einsum("...k,...kd->...d", p, np.abs(V)) / p.sum(axis=-1)[..., None]
    bound = U_BF16 * (1 + U_BF16) * (w + np.abs(ref)) + 1e-6 * np.abs(ref).max()
    err = np.abs(got - ref)
    assert (err <= bound).all(), float((err / bound).max())
