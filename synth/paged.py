"""Seeded paged layouts of a synthetic case's KV caches.

Layout only: the dense caches of a case are cut into pages of `block_size`
slots, the pages are scattered over a pool in a random order (a fragmented
pool, as after many allocations and releases), and a block table records
where each sequence's pages went.  Pool pages nobody uses, and the rows of a
sequence's last page past its slots in use, hold NaN, so any read of a slot
that is not visible shows up in the output.

Pool: [num_blocks, Hkv, block_size, D]; table: [B, capacity / block_size],
-1 for pages never allocated (past the slots in use).
"""
from __future__ import annotations

import dataclasses
from typing import Optional, Tuple

import numpy as np

from .inputs import Case


@dataclasses.dataclass
class PagedKV:
    k_pool: np.ndarray        # [NB, Hkv, BS, D] fp32 or bf16 bits
    v_pool: np.ndarray
    block_table: np.ndarray   # [B, capacity // BS] int32
    block_size: int
    capacity: int             # slots per sequence the table can address

    @property
    def num_blocks(self) -> int:
        return self.k_pool.shape[0]


def _nan_fill(dtype) -> np.generic:
    return np.uint16(0x7FC0) if dtype == np.uint16 else np.float32(np.nan)


def page_case(case: Case, block_size: int, *, spare: int = 7, share_prefix_pages: int = 0,
              seed: Tuple[int, ...] = (0,)) -> Tuple[Case, PagedKV]:
    """Paged copy of case's caches.  Returns (case, paged): with share_prefix_pages = m,
    every sequence's first m pages are sequence 0's (the returned case has those
    prefix slots copied from sequence 0, so both views agree); needs m * block_size
    <= every kv_len.  `spare` extra NaN pages are mixed into the pool."""
    B, Hkv, Lcap, D = case.k_cache.shape
    T = case.nodes
    nbt = -(-Lcap // block_size)
    capacity = nbt * block_size
    kv_len = case.kv_len.astype(np.int64)
    m = share_prefix_pages
    k_dense, v_dense = case.k_cache, case.v_cache
    if m:
        assert (kv_len >= m * block_size).all(), "shared prefix pages must hold prefix slots only"
        k_dense = k_dense.copy()
        v_dense = v_dense.copy()
        k_dense[1:, :, :m * block_size] = k_dense[0, :, :m * block_size]
        v_dense[1:, :, :m * block_size] = v_dense[0, :, :m * block_size]
        case = dataclasses.replace(case, k_cache=k_dense, v_cache=v_dense)
    used = [int(-(-min(int(kv_len[b]) + T, capacity) // block_size)) if kv_len[b] >= 0 else 0 for b in range(B)]
    owned = [(b, j) for b in range(B) for j in range(used[b]) if not (m and b > 0 and j < m)]
    nb = len(owned) + spare
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence(list(seed) + [99])))
    slots = rng.permutation(nb)
    fill = _nan_fill(k_dense.dtype)
    k_pool = np.full((nb, Hkv, block_size, D), fill, dtype=k_dense.dtype)
    v_pool = np.full((nb, Hkv, block_size, D), fill, dtype=v_dense.dtype)
    table = np.full((B, nbt), -1, dtype=np.int32)
    for n, (b, j) in enumerate(owned):
        page = int(slots[n])
        table[b, j] = page
        lo = j * block_size
        hi = min(lo + block_size, int(kv_len[b]) + T, Lcap)
        k_pool[page, :, :hi - lo, :] = k_dense[b, :, lo:hi, :]
        v_pool[page, :, :hi - lo, :] = v_dense[b, :, lo:hi, :]
    if m:
        table[1:, :m] = table[0, :m]
    return case, PagedKV(k_pool, v_pool, table, block_size, capacity)
