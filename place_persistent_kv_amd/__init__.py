"""Python binding of libpkv (include/pkv.h): argument marshalling only.

Every function here has the name of its C entry point without the ``pkv_``
prefix, converts torch tensors (or :class:`Raw` descriptors) to ``pkv_tensor``
structs, passes the current HIP stream and raises :class:`PkvError` on a
non-zero status.  Every step of the decode path runs in the HIP library; this
module computes nothing and never copies or converts tensors (non-contiguous
inputs are rejected).  If ``libpkv.so`` is missing, importing this package
raises: there is no fallback.

Build the library first:  ``python place_persistent_kv_amd/build.py``.
"""
from __future__ import annotations

import ctypes as C
import struct
import os
from dataclasses import dataclass
from typing import Optional, Sequence

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libpkv.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is missing: build it with `python place_persistent_kv_amd/build.py` "
                      "(the decode path has no CPU fallback)")

# torch supplies device memory and streams and ships its own HIP runtime.  It
# is imported first so that libpkv's dependency on libamdhip64.so.7 resolves
# to that same, already loaded runtime (same SONAME): two HIP runtimes in one
# process would not share streams, synchronisation or allocations.
import torch  # noqa: E402,F401

_lib = C.CDLL(LIB_PATH)


def _hip_runtimes_loaded() -> list[str]:
    try:
        with open("/proc/self/maps") as f:
            return sorted({ln.split()[-1] for ln in f if "libamdhip64" in ln and "/" in ln})
    except OSError:
        return []


if len(_hip_runtimes_loaded()) > 1:
    raise ImportError("two HIP runtimes are loaded in this process " + str(_hip_runtimes_loaded()) +
                      "; import torch before anything that links /opt/rocm's libamdhip64")

# ---------------------------------------------------------------------------
# C types
# ---------------------------------------------------------------------------
MAX_DIMS = 6
F32, BF16, F16, U8, I32, I64, F64 = range(7)
_ESIZE = {F32: 4, BF16: 2, F16: 2, U8: 1, I32: 4, I64: 8, F64: 8}

OK, E_ARG, E_CAPACITY, E_READONLY, E_ALIAS, E_BUSY, E_PAGE, E_NOMEM, E_DTYPE, E_LAYOUT, E_HIP = range(11)
STATUS_NAMES = {OK: "OK", E_ARG: "E_ARG", E_CAPACITY: "E_CAPACITY", E_READONLY: "E_READONLY",
                E_ALIAS: "E_ALIAS", E_BUSY: "E_BUSY", E_PAGE: "E_PAGE", E_NOMEM: "E_NOMEM",
                E_DTYPE: "E_DTYPE", E_LAYOUT: "E_LAYOUT", E_HIP: "E_HIP"}


class PkvTensor(C.Structure):
    _fields_ = [("data", C.c_void_p), ("dtype", C.c_int32), ("ndim", C.c_int32),
                ("shape", C.c_int64 * MAX_DIMS)]


class PageFormat(C.Structure):
    """``pkv_page_format``: storage code, scale and zero point of new or converted pages."""
    _fields_ = [("storage", C.c_int32), ("scale", C.c_float), ("zero_point", C.c_int32)]


PAGE_BF16, PAGE_F16, PAGE_INT8, PAGE_UINT8, PAGE_INT4, PAGE_UINT4, PAGE_INT2, PAGE_UINT2 = range(8)
PAGE_STORAGES = {"BF16": PAGE_BF16, "F16": PAGE_F16, "INT8": PAGE_INT8, "UINT8": PAGE_UINT8,
                 "INT4": PAGE_INT4, "UINT4": PAGE_UINT4, "INT2": PAGE_INT2, "UINT2": PAGE_UINT2}


def page_format(storage, scale: float = 1.0, zero_point: int = 0) -> PageFormat:
    """A :class:`PageFormat` from a storage name (``"INT8"``) or code."""
    code = PAGE_STORAGES[storage] if isinstance(storage, str) else int(storage)
    return PageFormat(code, float(scale), int(zero_point))


class LengthThresholdSelector:
    """A format selector: one (K, V) format pair while fewer than ``threshold``
    tokens are retained, another afterwards ("Persistent input/output feedback",
    "Optional heterogeneous paged KV": a selector picks the formats of the pages
    an append creates from the retained length)."""

    def __init__(self, threshold: int, early: tuple, late: tuple):
        self.threshold, self.early, self.late = int(threshold), early, late

    def __call__(self, retained: int) -> tuple:
        return self.early if retained < self.threshold else self.late


class PkvError(RuntimeError):
    """A libpkv call returned a non-zero status; ``.status`` holds it."""

    def __init__(self, status: int, func: str, msg: str):
        super().__init__(f"{func}: {STATUS_NAMES.get(status, status)}: {msg}")
        self.status = status


_P = C.POINTER
_T = C.c_void_p          # const pkv_tensor*: the packed bytes of _d()
_VP = C.c_void_p
_I32P = _P(C.c_int32)
_SIG = {
    "pkv_last_error": (C.c_char_p, []),
    "pkv_abi_version": (C.c_int32, []),
    "pkv_bind_writable": (C.c_int, [_VP, C.c_size_t, _P(_VP)]),
    "pkv_unbind": (C.c_int, [_VP]),
    "pkv_cache_update": (C.c_int, [_T, _T, _I32P, C.c_int32, _P(_VP), _VP]),
    "pkv_pool_create": (C.c_int, [C.c_int32, C.c_int32, C.c_int32, C.c_int32, _I32P, _P(_VP)]),
    "pkv_pool_destroy": (C.c_int, [_VP]),
    "pkv_pool_reserve": (C.c_int, [_VP, C.c_int32, _I32P, _I32P, _VP, _VP]),
    "pkv_pool_release": (C.c_int, [_VP, C.c_int32, _VP, _VP]),
    "pkv_pool_query": (C.c_int, [_VP, C.c_int32, _I32P, _I32P]),
    "pkv_pool_free_count": (C.c_int, [_VP, _I32P]),
    "pkv_pool_table": (C.c_int, [_VP, _I32P]),
    "pkv_paged_cache_update": (C.c_int, [_VP, _T, _VP, _T, _I32P, C.c_int32, _P(_VP), _VP]),
    "pkv_paged_cache_update_kv": (C.c_int, [_VP, _T, _T, _VP, _T, _T, _I32P, C.c_int32, _VP]),
    "pkv_cache_update_kv": (C.c_int, [_T, _T, _T, _T, _I32P, C.c_int32, _VP]),
    "pkv_paged_cache_update_int4": (C.c_int, [_VP, _T, _T, _VP, _T, C.c_uint16, C.c_uint16, _I32P,
                                              C.c_int32, _P(_VP), _P(_VP), _VP]),
    "pkv_paged_gather": (C.c_int, [_T, _VP, C.c_int32, C.c_int32, C.c_int32, _T, _VP]),
    "pkv_decode_workspace_size": (C.c_size_t, [C.c_int32] * 6),
    "pkv_decode_attention": (C.c_int, [_T, _T, _T, _I32P, C.c_float, C.c_int32, _T, _VP, C.c_size_t, C.c_int32,
                                       _VP]),
    "pkv_decode_step": (C.c_int, [_T, _T, _T, _T, _I32P, C.c_int32, _T, C.c_float, C.c_int32, _T, _VP, C.c_size_t,
                                  C.c_int32, _VP]),
    "pkv_decode_step_dev": (C.c_int, [_T, _T, _T, _T, _VP, C.c_int32, _T, C.c_int32, C.c_float, C.c_int32, _T,
                                      _VP, C.c_size_t, C.c_int32, _VP, _VP]),
    "pkv_paged_decode_attention": (C.c_int, [_T, _T, _T, _VP, C.c_int32, C.c_int32, _VP, _I32P, C.c_float,
                                             C.c_int32, _T, _VP, C.c_size_t, C.c_int32, _VP]),
    "pkv_paged_decode_attention_noalloc": (C.c_int, [_T, _T, _T, _VP, C.c_int32, C.c_int32, _VP, _I32P, C.c_float,
                                                     C.c_int32, _T, C.c_int32, _VP]),
    "pkv_paged_decode_attention_int4": (C.c_int, [_T, _T, _T, _T, _T, _VP, C.c_int32, C.c_int32, _VP, _I32P,
                                                  C.c_float, C.c_int32, _T, _VP, C.c_size_t, C.c_int32, _VP]),
    "pkv_chunk_attention": (C.c_int, [_T, _T, _T, _VP, C.c_int32, C.c_int32, _VP, _I32P, C.c_float, C.c_int32,
                                      _T, _VP]),
    "pkv_chunk_workspace_size": (C.c_size_t, [C.c_int32] * 5),
    "pkv_chunk_attention_split": (C.c_int, [_T, _T, _T, _VP, C.c_int32, C.c_int32, _VP, _I32P, C.c_float,
                                            C.c_int32, _T, _VP, C.c_size_t, C.c_int32, _VP]),
    "pkv_mixed_cache_update": (C.c_int, [_VP, _T, _T, _T, _VP, _T, _T, _I32P, C.c_int32, PageFormat, PageFormat,
                                         _VP]),
    "pkv_mixed_convert_pages": (C.c_int, [_T, _T, _T, _I32P, _I32P, C.c_int32, _P(PageFormat), _P(PageFormat),
                                          _VP]),
    "pkv_paged_decode_attention_mixed": (C.c_int, [_T, _T, _T, _T, _VP, C.c_int32, C.c_int32, _VP, _I32P,
                                                   C.c_float, C.c_int32, _T, _VP, C.c_size_t, C.c_int32, _VP]),
    "pkv_generate_step_seed": (C.c_uint64, [C.c_uint64, C.c_int64, C.c_int32, C.c_int64]),
    "pkv_generate_finish": (C.c_int, [_VP, _VP, _VP, C.c_int64, C.c_int32, C.c_int32, C.c_int64, C.c_int64, _VP,
                                      _VP, _VP]),
    "pkv_sample_workspace_size": (C.c_size_t, [C.c_int32, C.c_int64]),
    "pkv_sample": (C.c_int, [_T, C.c_float, C.c_uint64, _VP, _VP, C.c_size_t, _VP]),
    "pkv_sample_dev": (C.c_int, [_T, C.c_float, C.c_uint64, _VP, _VP, _VP, C.c_size_t, _VP]),
    "pkv_cache_update_kv_dev": (C.c_int, [_T, _T, _T, _T, _VP, C.c_int32, _VP, _VP]),
    "pkv_paged_cache_update_kv_dev": (C.c_int, [_VP, _T, _T, _VP, _T, _T, _VP, C.c_int32, _VP, _VP]),
    "pkv_advance": (C.c_int, [_VP, C.c_int32, C.c_int32, _VP, _VP]),
    "pkv_decode_attention_dev": (C.c_int, [_T, _T, _T, _VP, C.c_int32, C.c_float, C.c_int32, _T, _VP, C.c_size_t,
                                           C.c_int32, _VP, _VP]),
    "pkv_paged_decode_attention_dev": (C.c_int, [_T, _T, _T, _VP, C.c_int32, C.c_int32, _VP, _VP, C.c_int32,
                                                 C.c_float, C.c_int32, _T, _VP, C.c_size_t, C.c_int32, _VP, _VP]),
}

for _name, (_res, _args) in _SIG.items():
    _fn = getattr(_lib, _name, None)
    if _fn is not None:
        _fn.restype = _res
        _fn.argtypes = _args


ABI_VERSION = 10      # the argument lists above follow this version of include/pkv.h
if _lib.pkv_abi_version() != ABI_VERSION:
    raise ImportError(f"libpkv.so has ABI version {_lib.pkv_abi_version()}, the binding expects {ABI_VERSION}; "
                      "rebuild it (python place_persistent_kv_amd/build.py)")


def exported_symbols() -> list[str]:
    """Names from the signature table that the loaded library exports."""
    return [n for n in _SIG if getattr(_lib, n, None) is not None]


def last_error() -> str:
    return _lib.pkv_last_error().decode()


def abi_version() -> int:
    return int(_lib.pkv_abi_version())


def _check(status: int, func: str) -> None:
    if status != OK:
        raise PkvError(status, func, last_error())


# ---------------------------------------------------------------------------
# Descriptors
# ---------------------------------------------------------------------------
@dataclass
class Raw:
    """A tensor described by address, dtype code and shape (no torch needed)."""
    ptr: int
    dtype: int
    shape: Sequence[int]

    @property
    def nbytes(self) -> int:
        n = 1
        for s in self.shape:
            n *= int(s)
        return n * _ESIZE[self.dtype]


_DTYPE_CODES = None
_SHAPE_T = C.c_int64 * MAX_DIMS


def _torch_dtype_code(t) -> int:
    global _DTYPE_CODES
    if _DTYPE_CODES is None:
        import torch
        _DTYPE_CODES = {torch.float32: F32, torch.bfloat16: BF16, torch.float16: F16, torch.uint8: U8,
                        torch.int32: I32, torch.int64: I64, torch.float64: F64}
    code = _DTYPE_CODES.get(t.dtype)
    if code is None:
        raise TypeError(f"unsupported dtype {t.dtype}")
    return code


def desc(x) -> PkvTensor:
    """``pkv_tensor`` for a torch tensor (contiguous, any device) or a :class:`Raw`."""
    if isinstance(x, Raw):
        ptr, code, shape = x.ptr, x.dtype, tuple(int(s) for s in x.shape)
    else:
        if not x.is_contiguous():
            raise ValueError("tensor must be contiguous (libpkv never copies inputs)")
        ptr, code, shape = x.data_ptr(), _torch_dtype_code(x), x.shape
    n = len(shape)
    if not 1 <= n <= MAX_DIMS:
        raise ValueError(f"rank {n} not supported")
    return PkvTensor(ptr, code, n, _SHAPE_T(*shape))


# pkv_tensor as packed bytes (data, dtype, ndim, shape[6]); built with one
# struct.pack instead of a ctypes structure, which costs about ten times as
# much per call and adds up on the short, launch-bound calls
_DESC = struct.Struct("<Qii%dq" % MAX_DIMS)
_ZEROS = (0,) * MAX_DIMS
assert _DESC.size == C.sizeof(PkvTensor)


def _d(x) -> bytes:
    if isinstance(x, Raw):
        ptr, code, shape = x.ptr, x.dtype, tuple(int(s) for s in x.shape)
    else:
        if not x.is_contiguous():
            raise ValueError("tensor must be contiguous (libpkv never copies inputs)")
        ptr, code, shape = x.data_ptr(), _torch_dtype_code(x), x.shape
    n = len(shape)
    if not 1 <= n <= MAX_DIMS:
        raise ValueError(f"rank {n} not supported")
    return _DESC.pack(ptr, code, n, *shape, *_ZEROS[n:])


def _ptr(x) -> Optional[int]:
    if x is None:
        return None
    if isinstance(x, int):
        return x
    if isinstance(x, Raw):
        return x.ptr
    return x.data_ptr()


def _nbytes(x) -> int:
    if isinstance(x, Raw):
        return x.nbytes
    return x.numel() * x.element_size()


def _i32_array(values) -> C.Array:
    vals = [int(v) for v in values]
    return (C.c_int32 * (len(vals) or 1))(*vals)


_GPU = None


def current_stream() -> Optional[int]:
    """Handle of torch's current HIP stream (None when no GPU is visible)."""
    global _GPU
    import torch
    if _GPU is None:
        _GPU = torch.cuda.is_available()
    if not _GPU:
        return None
    return torch.cuda.current_stream().cuda_stream


def _stream(stream) -> Optional[int]:
    if stream is None:
        return current_stream()
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


# ---------------------------------------------------------------------------
# Writable bindings
# ---------------------------------------------------------------------------
class Binding:
    """Writable binding of a cache's storage ("Mutable execution cache", "Runtime contract")."""

    def __init__(self, storage, nbytes: Optional[int] = None):
        h = C.c_void_p()
        n = _nbytes(storage) if nbytes is None else int(nbytes)
        _check(_lib.pkv_bind_writable(_ptr(storage), n, C.byref(h)), "pkv_bind_writable")
        self._h = h

    def close(self) -> None:
        if self._h is not None and self._h.value:
            _check(_lib.pkv_unbind(self._h), "pkv_unbind")
        self._h = None

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        self.close()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def bind_writable(storage, nbytes: Optional[int] = None) -> Binding:
    return Binding(storage, nbytes)


def unbind(binding: Binding) -> None:
    binding.close()


# ---------------------------------------------------------------------------
# Cache updates
# ---------------------------------------------------------------------------
def cache_update(cache, values, position, update_length: int, stream=None) -> int:
    """In-place ``CacheUpdate``; returns the address of the updated cache (== cache's)."""
    out = C.c_void_p()
    _check(_lib.pkv_cache_update(_d(cache), _d(values), _i32_array(position),
                                 int(update_length), C.byref(out), _stream(stream)), "pkv_cache_update")
    return out.value


class Pool:
    """Host bookkeeping of a fixed page pool (``pkv_pool_*``)."""

    def __init__(self, num_blocks: int, block_size: int, max_seqs: int, max_blocks_per_seq: int,
                 initial_free_order=None):
        h = C.c_void_p()
        order = None if initial_free_order is None else _i32_array(initial_free_order)
        _check(_lib.pkv_pool_create(num_blocks, block_size, max_seqs, max_blocks_per_seq, order, C.byref(h)),
               "pkv_pool_create")
        self._h = h
        self.num_blocks, self.block_size = num_blocks, block_size
        self.max_seqs, self.max_blocks_per_seq = max_seqs, max_blocks_per_seq

    @property
    def handle(self):
        return self._h

    def reserve(self, seqs, new_lens, page_table=None, stream=None) -> None:
        seqs, new_lens = list(seqs), list(new_lens)
        _check(_lib.pkv_pool_reserve(self._h, len(seqs), _i32_array(seqs), _i32_array(new_lens),
                                     _ptr(page_table), _stream(stream) if page_table is not None else None),
               "pkv_pool_reserve")

    def release(self, seq: int, page_table=None, stream=None) -> None:
        _check(_lib.pkv_pool_release(self._h, seq, _ptr(page_table),
                                     _stream(stream) if page_table is not None else None), "pkv_pool_release")

    def query(self, seq: int) -> tuple[int, int]:
        held, length = C.c_int32(), C.c_int32()
        _check(_lib.pkv_pool_query(self._h, seq, C.byref(held), C.byref(length)), "pkv_pool_query")
        return held.value, length.value

    def free_count(self) -> int:
        n = C.c_int32()
        _check(_lib.pkv_pool_free_count(self._h, C.byref(n)), "pkv_pool_free_count")
        return n.value

    def table(self):
        import numpy as np
        out = np.empty((self.max_seqs, self.max_blocks_per_seq), dtype=np.int32)
        _check(_lib.pkv_pool_table(self._h, out.ctypes.data_as(_I32P)), "pkv_pool_table")
        return out

    def close(self) -> None:
        if self._h is not None and self._h.value:
            _check(_lib.pkv_pool_destroy(self._h), "pkv_pool_destroy")
        self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def _pool_handle(pool):
    return None if pool is None else pool.handle


def paged_cache_update(pool: Pool, pool_kv, page_table, values, position, update_length: int,
                       stream=None) -> int:
    out = C.c_void_p()
    _check(_lib.pkv_paged_cache_update(_pool_handle(pool), _d(pool_kv), _ptr(page_table),
                                       _d(values), _i32_array(position), int(update_length),
                                       C.byref(out), _stream(stream)), "pkv_paged_cache_update")
    return out.value


def cache_update_kv(k_cache, v_cache, k_values, v_values, position, update_length: int, stream=None) -> None:
    """``pkv_cache_update_kv``: K and V appended to contiguous caches at host positions in one launch."""
    _check(_lib.pkv_cache_update_kv(_d(k_cache), _d(v_cache), _d(k_values),
                                    _d(v_values), _i32_array(position), int(update_length),
                                    _stream(stream)), "pkv_cache_update_kv")


def paged_cache_update_kv(pool: Pool, k_pool, v_pool, page_table, k_values, v_values, position,
                          update_length: int, stream=None) -> None:
    """``pkv_paged_cache_update_kv``: K and V appended at host positions in one launch."""
    _check(_lib.pkv_paged_cache_update_kv(_pool_handle(pool), _d(k_pool), _d(v_pool),
                                          _ptr(page_table), _d(k_values), _d(v_values),
                                          _i32_array(position), int(update_length), _stream(stream)),
           "pkv_paged_cache_update_kv")


def paged_cache_update_int4(pool: Pool, codes_pool, params_pool, page_table, values, scale_f16_bits: int,
                            zero_point_f16_bits: int, position, update_length: int, stream=None):
    oc, op = C.c_void_p(), C.c_void_p()
    _check(_lib.pkv_paged_cache_update_int4(_pool_handle(pool), _d(codes_pool),
                                            _d(params_pool), _ptr(page_table), _d(values),
                                            int(scale_f16_bits), int(zero_point_f16_bits), _i32_array(position),
                                            int(update_length), C.byref(oc), C.byref(op), _stream(stream)),
           "pkv_paged_cache_update_int4")
    return oc.value, op.value


def paged_gather(pool_kv, page_table, max_blocks_per_seq: int, seq: int, length: int, out, stream=None) -> None:
    _check(_lib.pkv_paged_gather(_d(pool_kv), _ptr(page_table), max_blocks_per_seq, seq, length,
                                 _d(out), _stream(stream)), "pkv_paged_gather")


# ---------------------------------------------------------------------------
# Attention
# ---------------------------------------------------------------------------
def decode_workspace_size(B: int, Hq: int, Hkv: int, D: int, max_len: int, num_splits: int = 0) -> int:
    return int(_lib.pkv_decode_workspace_size(B, Hq, Hkv, D, max_len, num_splits))


def decode_step(k_cache, v_cache, k_values, v_values, position, update_length: int, q, out, workspace=None,
                scale: float = 0.0, num_splits: int = 0, stream=None, left_window: int = -1) -> None:
    """``cache_update_kv`` then ``decode_attention`` at ``position + update_length``, in one launch."""
    _check(_lib.pkv_decode_step(_d(k_cache), _d(v_cache), _d(k_values),
                                _d(v_values), _i32_array(position), int(update_length), _d(q),
                                float(scale), int(left_window), _d(out), _ptr(workspace),
                                0 if workspace is None else _nbytes(workspace), int(num_splits), _stream(stream)),
           "pkv_decode_step")


def decode_step_dev(k_cache, v_cache, k_values, v_values, position, update_length: int, q, max_len: int, out,
                    status, workspace=None, scale: float = 0.0, num_splits: int = 0, stream=None,
                    left_window: int = -1) -> None:
    """``decode_step`` at the device positions ``position`` (int32 [B]); they are not advanced."""
    _check(_lib.pkv_decode_step_dev(_d(k_cache), _d(v_cache), _d(k_values), _d(v_values), _ptr(position),
                                    int(update_length), _d(q), int(max_len), float(scale), int(left_window),
                                    _d(out), _ptr(workspace), 0 if workspace is None else _nbytes(workspace),
                                    int(num_splits), _ptr(status), _stream(stream)), "pkv_decode_step_dev")


def decode_attention(q, k_cache, v_cache, valid_len, out, workspace=None, scale: float = 0.0,
                     num_splits: int = 0, stream=None, left_window: int = -1) -> None:
    ws = _ptr(workspace)
    _check(_lib.pkv_decode_attention(_d(q), _d(k_cache), _d(v_cache),
                                     _i32_array(valid_len), float(scale), int(left_window), _d(out), ws,
                                     0 if workspace is None else _nbytes(workspace), int(num_splits),
                                     _stream(stream)), "pkv_decode_attention")


def paged_decode_attention(q, k_pool, v_pool, page_table, max_blocks_per_seq: int, block_size: int, valid_len,
                           out, workspace=None, pool: Optional[Pool] = None, scale: float = 0.0,
                           num_splits: int = 0, stream=None, left_window: int = -1) -> None:
    _check(_lib.pkv_paged_decode_attention(_d(q), _d(k_pool), _d(v_pool),
                                           _ptr(page_table), int(max_blocks_per_seq), int(block_size),
                                           _pool_handle(pool), _i32_array(valid_len), float(scale),
                                           int(left_window), _d(out), _ptr(workspace),
                                           0 if workspace is None else _nbytes(workspace), int(num_splits),
                                           _stream(stream)), "pkv_paged_decode_attention")


NOALLOC_SCRATCH_BYTES = 16 << 20      # PKV_NOALLOC_SCRATCH_BYTES


def paged_decode_attention_noalloc(q, k_pool, v_pool, page_table, max_blocks_per_seq: int, block_size: int,
                                   valid_len, out, pool: Optional[Pool] = None, scale: float = 0.0,
                                   num_splits: int = 0, stream=None, left_window: int = -1) -> None:
    """``pkv_paged_decode_attention_noalloc``: the paged decode with its split partials in the library's
    static device scratch (no workspace argument, nothing allocated)."""
    _check(_lib.pkv_paged_decode_attention_noalloc(
        _d(q), _d(k_pool), _d(v_pool), _ptr(page_table), int(max_blocks_per_seq),
        int(block_size), _pool_handle(pool), _i32_array(valid_len), float(scale), int(left_window),
        _d(out), int(num_splits), _stream(stream)), "pkv_paged_decode_attention_noalloc")


def paged_decode_attention_int4(q, k_codes, k_params, v_codes, v_params, page_table, max_blocks_per_seq: int,
                                block_size: int, valid_len, out, workspace=None, pool: Optional[Pool] = None,
                                scale: float = 0.0, num_splits: int = 0, stream=None,
                                left_window: int = -1) -> None:
    _check(_lib.pkv_paged_decode_attention_int4(
        _d(q), _d(k_codes), _d(k_params), _d(v_codes),
        _d(v_params), _ptr(page_table), int(max_blocks_per_seq), int(block_size), _pool_handle(pool),
        _i32_array(valid_len), float(scale), int(left_window), _d(out), _ptr(workspace),
        0 if workspace is None else _nbytes(workspace), int(num_splits), _stream(stream)),
        "pkv_paged_decode_attention_int4")


def chunk_workspace_size(B: int, Hq: int, Hkv: int, C: int, num_splits: int = 0) -> int:
    return int(_lib.pkv_chunk_workspace_size(B, Hq, Hkv, C, num_splits))


def chunk_attention(q, k_pool, v_pool, page_table, max_blocks_per_seq: int, block_size: int, p0, out,
                    pool: Optional[Pool] = None, scale: float = 0.0, stream=None, left_window: int = -1,
                    workspace=None, num_splits: int = 1) -> None:
    """Causal chunk attention; with ``num_splits`` other than 1 (0 = library choice) the key range of every
    workgroup is split into parts whose partials ``workspace`` (``chunk_workspace_size`` bytes) holds."""
    if num_splits == 1 and workspace is None:
        _check(_lib.pkv_chunk_attention(_d(q), _d(k_pool), _d(v_pool),
                                        _ptr(page_table), int(max_blocks_per_seq), int(block_size),
                                        _pool_handle(pool), _i32_array(p0), float(scale), int(left_window),
                                        _d(out), _stream(stream)),
               "pkv_chunk_attention")
        return
    _check(_lib.pkv_chunk_attention_split(_d(q), _d(k_pool), _d(v_pool),
                                          _ptr(page_table), int(max_blocks_per_seq), int(block_size),
                                          _pool_handle(pool), _i32_array(p0), float(scale), int(left_window),
                                          _d(out), _ptr(workspace),
                                          0 if workspace is None else _nbytes(workspace), int(num_splits),
                                          _stream(stream)),
           "pkv_chunk_attention_split")


# ---------------------------------------------------------------------------
# Mixed-format pages
# ---------------------------------------------------------------------------
def mixed_page_desc(num_blocks: int, device="cuda"):
    """A zeroed descriptor table ``u8 [num_blocks, 16]`` (every page BF16)."""
    import torch
    return torch.zeros((num_blocks, 16), dtype=torch.uint8, device=device)


def mixed_cache_update(pool: Pool, k_pool, v_pool, page_desc, page_table, k_values, v_values, position,
                       update_length: int, k_format: PageFormat, v_format: PageFormat, stream=None) -> None:
    _check(_lib.pkv_mixed_cache_update(_pool_handle(pool), _d(k_pool), _d(v_pool),
                                       _d(page_desc), _ptr(page_table), _d(k_values),
                                       _d(v_values), _i32_array(position), int(update_length),
                                       k_format, v_format, _stream(stream)), "pkv_mixed_cache_update")


def mixed_convert_pages(k_pool, v_pool, page_desc, pages, valid_rows, k_format: Optional[PageFormat] = None,
                        v_format: Optional[PageFormat] = None, stream=None) -> None:
    pages, valid_rows = list(pages), list(valid_rows)
    _check(_lib.pkv_mixed_convert_pages(_d(k_pool), _d(v_pool), _d(page_desc),
                                        _i32_array(pages), _i32_array(valid_rows), len(pages),
                                        None if k_format is None else C.byref(k_format),
                                        None if v_format is None else C.byref(v_format), _stream(stream)),
           "pkv_mixed_convert_pages")


def paged_decode_attention_mixed(q, k_pool, v_pool, page_desc, page_table, max_blocks_per_seq: int,
                                 block_size: int, valid_len, out, workspace=None, pool: Optional[Pool] = None,
                                 scale: float = 0.0, num_splits: int = 0, stream=None,
                                 left_window: int = -1) -> None:
    _check(_lib.pkv_paged_decode_attention_mixed(
        _d(q), _d(k_pool), _d(v_pool), _d(page_desc), _ptr(page_table),
        int(max_blocks_per_seq), int(block_size), _pool_handle(pool), _i32_array(valid_len), float(scale),
        int(left_window), _d(out), _ptr(workspace), 0 if workspace is None else _nbytes(workspace),
        int(num_splits), _stream(stream)), "pkv_paged_decode_attention_mixed")


# ---------------------------------------------------------------------------
# Sampling
# ---------------------------------------------------------------------------
def sample_workspace_size(B: int, V: int) -> int:
    return int(_lib.pkv_sample_workspace_size(B, V))


def sample(logits, temperature: float, seed: int, out_ids, workspace=None, stream=None) -> None:
    _check(_lib.pkv_sample(_d(logits), float(temperature), C.c_uint64(seed & (2 ** 64 - 1)),
                           _ptr(out_ids), _ptr(workspace), 0 if workspace is None else _nbytes(workspace),
                           _stream(stream)), "pkv_sample")


def sample_dev(logits, temperature: float, seed: int, step, out_ids, workspace=None, stream=None) -> None:
    """``pkv_sample_dev``: the seed of the iteration held in the device int64 counter ``step``."""
    _check(_lib.pkv_sample_dev(_d(logits), float(temperature), C.c_uint64(seed & (2 ** 64 - 1)),
                               _ptr(step), _ptr(out_ids), _ptr(workspace), 0 if workspace is None else _nbytes(workspace),
                               _stream(stream)), "pkv_sample_dev")


# ---------------------------------------------------------------------------
# Device-driven step: positions, lengths and the sampling step in device memory
# ---------------------------------------------------------------------------
def cache_update_kv_dev(k_cache, v_cache, k_values, v_values, position, update_length: int, status,
                        stream=None) -> None:
    """``pkv_cache_update_kv_dev``: K and V appended at the device positions ``position`` (int32 [B])."""
    _check(_lib.pkv_cache_update_kv_dev(_d(k_cache), _d(v_cache), _d(k_values),
                                        _d(v_values), _ptr(position), int(update_length), _ptr(status),
                                        _stream(stream)), "pkv_cache_update_kv_dev")


def paged_cache_update_kv_dev(pool: Pool, k_pool, v_pool, page_table, k_values, v_values, position,
                              update_length: int, status, stream=None) -> None:
    """``pkv_paged_cache_update_kv_dev``: the paged form."""
    _check(_lib.pkv_paged_cache_update_kv_dev(_pool_handle(pool), _d(k_pool), _d(v_pool),
                                              _ptr(page_table), _d(k_values), _d(v_values),
                                              _ptr(position), int(update_length), _ptr(status), _stream(stream)),
           "pkv_paged_cache_update_kv_dev")


def advance(values, delta: int, step=None, stream=None, n: Optional[int] = None) -> None:
    """``pkv_advance``: ``values[:n] += delta`` (device int32) and ``step += 1`` (device int64) when given."""
    count = int(n) if n is not None else (values.numel() if values is not None else 0)
    _check(_lib.pkv_advance(_ptr(values), count, int(delta), _ptr(step), _stream(stream)), "pkv_advance")


def decode_attention_dev(q, k_cache, v_cache, valid_len, max_len: int, out, status, workspace=None,
                         scale: float = 0.0, num_splits: int = 0, stream=None, left_window: int = -1) -> None:
    """``pkv_decode_attention_dev``: valid lengths from the device int32 tensor ``valid_len``."""
    _check(_lib.pkv_decode_attention_dev(_d(q), _d(k_cache), _d(v_cache),
                                         _ptr(valid_len), int(max_len), float(scale), int(left_window),
                                         _d(out), _ptr(workspace),
                                         0 if workspace is None else _nbytes(workspace), int(num_splits),
                                         _ptr(status), _stream(stream)), "pkv_decode_attention_dev")


def paged_decode_attention_dev(q, k_pool, v_pool, page_table, max_blocks_per_seq: int, block_size: int, valid_len,
                               max_len: int, out, status, workspace=None, pool: Optional[Pool] = None,
                               scale: float = 0.0, num_splits: int = 0, stream=None, left_window: int = -1) -> None:
    """``pkv_paged_decode_attention_dev``: the paged form."""
    _check(_lib.pkv_paged_decode_attention_dev(
        _d(q), _d(k_pool), _d(v_pool), _ptr(page_table), int(max_blocks_per_seq),
        int(block_size), _pool_handle(pool), _ptr(valid_len), int(max_len), float(scale), int(left_window),
        _d(out), _ptr(workspace), 0 if workspace is None else _nbytes(workspace), int(num_splits),
        _ptr(status), _stream(stream)), "pkv_paged_decode_attention_dev")


# ---------------------------------------------------------------------------
# Generation loop
# ---------------------------------------------------------------------------
def generate_step_seed(seed: int, step: int, B: int, V: int) -> int:
    return int(_lib.pkv_generate_step_seed(C.c_uint64(seed & (2 ** 64 - 1)), int(step), int(B), int(V)))


def generate_finish(sampled, finished, tokens, column: int, eos_token_id, pad_token_id, next_ids, unfinished,
                    stream=None) -> None:
    """One iteration's bookkeeping (``pkv_generate_finish``); ``eos_token_id`` None means no EOS."""
    B, row_stride = tokens.shape
    eos = -1 if eos_token_id is None else int(eos_token_id)
    pad = 0 if pad_token_id is None else int(pad_token_id)
    _check(_lib.pkv_generate_finish(_ptr(sampled), _ptr(finished), _ptr(tokens), int(row_stride), int(column), int(B),
                                    eos, pad, _ptr(next_ids), _ptr(unfinished), _stream(stream)),
           "pkv_generate_finish")


def generate(forward, prompt_ids, max_new_tokens: int, temperature: float = 0.0, seed: int = 0,
             eos_token_id=None, pad_token_id=None, stream=None):
    """Token loop ("Persistent input/output feedback", "Autoregressive generation").

    ``forward(step, input_ids)`` is the caller's model: it receives the prompt
    (device int64 ``[B, P]``) at step 0 and then the previous step's tokens
    (device int64 ``[B]``), and returns device logits ``[B, V]`` or
    ``[B, S, V]``.  Each iteration samples (``pkv_sample``) and books the
    tokens (``pkv_generate_finish``) in the library; the loop stops at
    ``max_new_tokens`` or once every row has emitted EOS (one host read of a
    device counter per iteration).  Returns device int64 ``[B, P + generated]``.
    """
    import torch
    B, P = prompt_ids.shape
    dev = prompt_ids.device
    pad = eos_token_id if pad_token_id is None else pad_token_id
    tokens = torch.empty((B, P + max_new_tokens), dtype=torch.int64, device=dev)
    tokens[:, :P].copy_(prompt_ids)
    finished = torch.zeros(B, dtype=torch.uint8, device=dev)
    ids = torch.empty(B, dtype=torch.int64, device=dev)
    nxt = torch.empty(B, dtype=torch.int64, device=dev)
    unfinished = torch.empty(1, dtype=torch.int32, device=dev)
    ws = None
    inputs = prompt_ids
    done = 0
    for t in range(int(max_new_tokens)):
        logits = forward(t, inputs)
        V = logits.shape[-1]
        if ws is None:
            ws = torch.empty(sample_workspace_size(B, V), dtype=torch.uint8, device=dev)
        sample(logits, temperature, generate_step_seed(seed, t, B, V), ids, ws, stream=stream)
        generate_finish(ids, finished, tokens, P + t, eos_token_id, pad, nxt, unfinished, stream=stream)
        done = t + 1
        inputs = nxt
        if eos_token_id is not None and int(unfinished.item()) == 0:
            break
    return tokens[:, :P + done]
