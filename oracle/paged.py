"""Paged KV cache: a block table maps each sequence's slots to pages of a pool.

TEST INFRASTRUCTURE ONLY (the oracle; see the package docstring).

The pages ask that the verify step's extra KV live in page-based KV memory
([P1] section 4.2 on the memory cost of the candidates' KV; section 6.3: the
speculative KV is given pages and released page by page, rejected paths at
once).  They fix no layout.  Reading taken here:

  * k_pool, v_pool: [num_blocks, Hkv, BS, D]; one page holds BS consecutive
    slots of one sequence for every KV head.
  * Slot s of sequence b (prefix slots 0..L_b-1, tree node i at L_b + i) is
    row s % BS of page block_table[b, s // BS].  The table has capacity / BS
    entries per sequence.
  * The entries of the slots in use, 0..L_b+T-1, must name pages of the pool
    (0 <= page < num_blocks); otherwise the sequence's KV is invalid exactly
    like an out-of-range length: status bit 8 and no attention output.
    Entries past the slots in use are never read.
  * Several sequences may share pages (a common prefix); the verify step only
    reads.  The commit writes slots L_b..L_b+accept_len, which the caller
    keeps in pages of that sequence alone.

Everything else (the attention, the commit rule) is the dense definition
applied to the slots gathered through the table.
"""
from __future__ import annotations

from typing import Dict, Tuple

import numpy as np

from .attention import tree_attention_sequence
from .commit import commit_kv
from .tree import check_parent
from .verify import verify, widen


def slot_page_row(table_row: np.ndarray, s: int, block_size: int) -> Tuple[int, int]:
    """(page, row) of slot s of one sequence."""
    return int(table_row[s // block_size]), s % block_size


def pages_valid(table_row: np.ndarray, n_slots: int, block_size: int, num_blocks: int) -> bool:
    """Whether every table entry of slots 0..n_slots-1 names a page of the pool."""
    used = -(-n_slots // block_size)
    if used > len(table_row):
        return False
    entries = np.asarray(table_row[:used], dtype=np.int64)
    return bool(((entries >= 0) & (entries < num_blocks)).all())


def gather_slots(pool: np.ndarray, table_row: np.ndarray, n_slots: int, block_size: int) -> np.ndarray:
    """Slots 0..n_slots-1 of one sequence, in slot order: [Hkv, n_slots, D] (pool dtype)."""
    out = np.empty((pool.shape[1], n_slots, pool.shape[3]), dtype=pool.dtype)
    for s in range(n_slots):
        page, row = slot_page_row(table_row, s, block_size)
        out[:, s, :] = pool[page, :, row, :]
    return out


def kv_valid(kv_len: int, nodes: int, capacity: int, table_row: np.ndarray, block_size: int,
             num_blocks: int) -> bool:
    """Length in range and every used table entry inside the pool."""
    if kv_len < 0 or kv_len + nodes > capacity:
        return False
    return pages_valid(table_row, kv_len + nodes, block_size, num_blocks)


def verify_paged(case, paged, *, seqs=None, **kw) -> Dict[str, np.ndarray]:
    """The verify step with the caches read through the block table.

    `case` supplies everything but the caches; `paged` holds k_pool, v_pool,
    block_table, block_size and capacity.  Outputs as `verify`.
    """
    spec = case.spec
    seqs = list(range(case.parent.shape[0])) if seqs is None else list(seqs)
    out = verify(case, attention=False, seqs=seqs, **kw)
    T = case.parent.shape[1]
    nb = paged.k_pool.shape[0]
    attn = np.full((len(seqs),) + case.q.shape[1:], np.nan)
    kv_status = np.zeros(len(seqs), dtype=np.int32)
    for n, b in enumerate(seqs):
        L = int(case.kv_len[b])
        row = paged.block_table[b]
        if not kv_valid(L, T, paged.capacity, row, paged.block_size, nb):
            kv_status[n] = 8
            continue
        if not check_parent(case.parent[b]):
            continue
        k = gather_slots(paged.k_pool, row, L + T, paged.block_size)
        v = gather_slots(paged.v_pool, row, L + T, paged.block_size)
        attn[n] = tree_attention_sequence(widen(case.q[b], spec.dtype), widen(k, spec.dtype),
                                          widen(v, spec.dtype), L, case.parent[b])
    out["attn_out"] = attn
    out["status"] = out["status"] | kv_status
    return out


def commit_kv_paged(k_pool: np.ndarray, v_pool: np.ndarray, block_table: np.ndarray, kv_len: np.ndarray,
                    path: np.ndarray, accept_len: np.ndarray, final_node: np.ndarray, nodes: int,
                    block_size: int, capacity: int):
    """KV commit through the block table: returns (k_pool, v_pool, kv_len); inputs unchanged.

    Per sequence the rule of `commit_kv` on the slots 0..L_b+T-1 gathered
    through the table, written back to the same pages.  A sequence whose used
    table entries leave the pool is skipped as well.
    """
    k = np.array(k_pool, copy=True)
    v = np.array(v_pool, copy=True)
    new_len = np.array(kv_len, copy=True)
    T = nodes
    nb = k_pool.shape[0]
    for b in range(block_table.shape[0]):
        L = int(kv_len[b])
        row = block_table[b]
        if not kv_valid(L, T, capacity, row, block_size, nb):
            continue
        n = L + T
        dk = gather_slots(k_pool, row, n, block_size)[None]
        dv = gather_slots(v_pool, row, n, block_size)[None]
        ck, cv, cl = commit_kv(dk, dv, np.array([L]), path[b:b + 1], accept_len[b:b + 1], final_node[b:b + 1], T)
        if int(cl[0]) == L:
            continue
        for s in range(L, int(cl[0])):
            page, r = slot_page_row(row, s, block_size)
            k[page, :, r, :] = ck[0, :, s, :]
            v[page, :, r, :] = cv[0, :, s, :]
        new_len[b] = cl[0]
    return k, v, new_len
