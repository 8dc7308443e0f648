"""In-place cache update, the fixed page pool and the paged mapping.

Contiguous update -- "Mutable execution cache", sections "Value model",
"ShapesContext", "Required alias", "Model example" and "Runtime contract":
``updated_cache = CacheUpdate(cache, values, position)`` writes ``values`` into
the range starting at ``position``, the result *is* the input storage, the
capacity check ``position + update_length <= capacity`` happens before any
write, and overflow is an error (no growth, no copy of the cache).

Paged update -- same page, "Heterogeneous paged cache" and "Runtime contract":
existing pages are written in place, only a missing page is allocated, page
table growth never duplicates payloads; the fixed physical block pool with a
per-request block table is the layout of "Existing implementations / ONNX
Runtime GenAI" (backing tensors never grow; once the free pool is empty no
more capacity exists).

Readings where the pages leave a step open (listed in the design doc):

* ``position`` is one value per batch row (a scalar position is B equal
  entries);
* a partially filled last page is filled in place (the mutable-cache page says
  existing pages are updated in place; the how-to's sealed-block policy is the
  CPU kernel's, not this contract's);
* pages are laid out head-major, ``pool[block, head, slot, :]``, the page
  shape ``[heads, page_size, head_size]`` of the paged-cache example (one pool
  per K and per V);
* logical token ``p`` of row ``b`` lives at
  ``(page_table[b, p // block_size], p % block_size)``.
"""
from __future__ import annotations

import numpy as np


class CapacityError(ValueError):
    """position + update_length exceeds the capacity (no write happened)."""


class PageError(ValueError):
    """A page needed by the update is not reserved, or an id is invalid."""


class PoolExhausted(MemoryError):
    """The free pool cannot satisfy a reservation (nothing was taken)."""


# ----------------------------------------------------------------------------
# Contiguous CacheUpdate
# ----------------------------------------------------------------------------

def check_capacity(position, update_length: int, capacity: int) -> None:
    """Capacity rule: every row needs 0 <= position and position + n <= capacity."""
    position = np.asarray(position, dtype=np.int64).reshape(-1)
    if update_length < 0:
        raise ValueError("update_length must be >= 0")
    for b, p in enumerate(position):
        if p < 0 or p + update_length > capacity:
            raise CapacityError(f"row {b}: position {p} + update_length {update_length} "
                                f"> capacity {capacity}")


def cache_update(cache: np.ndarray, values: np.ndarray, position, update_length: int) -> np.ndarray:
    """Write ``values[b, h, t, :]`` to ``cache[b, h, position[b] + t, :]`` in place.

    ``cache`` is ``[B, H, capacity, D]`` and ``values`` is ``[B, H, n, D]`` with
    ``n == update_length``; any element type (the update is a byte copy).
    Returns ``cache`` itself (the output aliases the input).  Raises
    :class:`CapacityError` before touching anything when a row would overflow.
    """
    B, H, cap, D = cache.shape
    n = int(update_length)
    if values.shape != (B, H, n, D):
        raise ValueError(f"values shape {values.shape} != {(B, H, n, D)}")
    if values.dtype != cache.dtype:
        raise ValueError("values and cache element types differ")
    position = np.asarray(position, dtype=np.int64).reshape(-1)
    if position.shape[0] != B:
        raise ValueError("one position per batch row")
    check_capacity(position, n, cap)
    for b in range(B):
        for t in range(n):
            cache[b, :, position[b] + t, :] = values[b, :, t, :]   # every head of the token row
    return cache


# ----------------------------------------------------------------------------
# Fixed page pool (host metadata) and the paged update
# ----------------------------------------------------------------------------

def pages_for(length: int, block_size: int) -> int:
    """Number of logical pages that hold ``length`` tokens."""
    return -(-int(length) // int(block_size))


class PagePool:
    """Fixed pool of ``num_blocks`` physical pages shared by ``max_seqs`` requests.

    The free list starts as ``initial_free_order`` (default ``0..num_blocks-1``)
    and pages are handed out from its front.  ``reserve(seq, new_len)`` takes
    exactly the pages that logical positions ``[0, new_len)`` need and the
    request does not hold yet, all or nothing.  ``release(seq)`` returns every
    page of the request to the back of the free list.
    """

    def __init__(self, num_blocks: int, block_size: int, max_seqs: int,
                 max_blocks_per_seq: int, initial_free_order=None):
        if num_blocks <= 0 or block_size <= 0 or max_seqs <= 0 or max_blocks_per_seq <= 0:
            raise ValueError("pool dimensions must be positive")
        self.num_blocks = int(num_blocks)
        self.block_size = int(block_size)
        self.max_seqs = int(max_seqs)
        self.max_blocks_per_seq = int(max_blocks_per_seq)
        if initial_free_order is None:
            order = list(range(self.num_blocks))
        else:
            order = [int(x) for x in np.asarray(initial_free_order).reshape(-1)]
            if sorted(order) != list(range(self.num_blocks)):
                raise ValueError("initial_free_order must be a permutation of 0..num_blocks-1")
        self.free = list(order)
        self.table = np.full((self.max_seqs, self.max_blocks_per_seq), -1, dtype=np.int32)
        self.held = [0] * self.max_seqs        # pages held per request
        self.length = [0] * self.max_seqs      # reserved logical length per request

    def reserve(self, seq: int, new_len: int) -> list[int]:
        """Make positions ``[0, new_len)`` of ``seq`` backed by pages.

        Returns the newly taken physical ids (possibly empty).  Raises
        :class:`PoolExhausted` or :class:`PageError` with nothing changed.
        """
        if not (0 <= seq < self.max_seqs):
            raise PageError(f"sequence {seq} out of range")
        need = pages_for(new_len, self.block_size)
        if need > self.max_blocks_per_seq:
            raise PageError(f"{need} pages exceed max_blocks_per_seq {self.max_blocks_per_seq}")
        missing = max(0, need - self.held[seq])
        if missing > len(self.free):
            raise PoolExhausted(f"need {missing} pages, {len(self.free)} free")
        taken = self.free[:missing]
        del self.free[:missing]
        for i, phys in enumerate(taken):
            self.table[seq, self.held[seq] + i] = phys
        self.held[seq] += missing
        self.length[seq] = max(self.length[seq], int(new_len))
        return taken

    def release(self, seq: int) -> None:
        n = self.held[seq]
        self.free.extend(int(x) for x in self.table[seq, :n])
        self.table[seq, :] = -1
        self.held[seq] = 0
        self.length[seq] = 0

    def used(self) -> int:
        return sum(self.held)


def physical_slot(page_table_row: np.ndarray, p: int, block_size: int) -> tuple[int, int]:
    """Logical position ``p`` -> (physical page id, slot within the page)."""
    return int(page_table_row[p // block_size]), p % block_size


def paged_cache_update(pool: np.ndarray, page_table: np.ndarray, values: np.ndarray,
                       position, update_length: int, block_size: int,
                       held_pages=None) -> np.ndarray:
    """Write ``values[b, h, t, :]`` to logical position ``position[b] + t`` of row b.

    ``pool`` is ``[num_blocks, H, block_size, D]`` and is written in place and
    returned.  ``held_pages[b]`` (when given) is how many pages row b holds;
    a write past them raises :class:`PageError` before anything is written.
    """
    NB, H, bs, D = pool.shape
    if bs != block_size:
        raise ValueError("pool slot count != block_size")
    B = values.shape[0]
    n = int(update_length)
    if values.shape != (B, H, n, D):
        raise ValueError(f"values shape {values.shape} != {(B, H, n, D)}")
    position = np.asarray(position, dtype=np.int64).reshape(-1)
    for b in range(B):
        if position[b] < 0:
            raise PageError(f"row {b}: negative position")
        if n == 0:
            continue
        last_page = (position[b] + n - 1) // bs
        if held_pages is not None and last_page >= held_pages[b]:
            raise PageError(f"row {b}: logical page {last_page} not reserved")
        for j in range(position[b] // bs, last_page + 1):
            if not (0 <= page_table[b, j] < NB):
                raise PageError(f"row {b}: page id {page_table[b, j]} out of range")
    for b in range(B):
        for t in range(n):
            phys, slot = physical_slot(page_table[b], int(position[b]) + t, bs)
            pool[phys, :, slot, :] = values[b, :, t, :]       # every head of the token row
    return pool


def paged_gather(pool: np.ndarray, page_table_row: np.ndarray, length: int, block_size: int) -> np.ndarray:
    """Logical ``[H, length, D]`` view of one request, assembled token by token."""
    NB, H, bs, D = pool.shape
    out = np.empty((H, length, D), dtype=pool.dtype)
    for p in range(length):
        phys, slot = physical_slot(page_table_row, p, block_size)
        out[:, p, :] = pool[phys, :, slot, :]
    return out
