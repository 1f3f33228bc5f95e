"""Cache append, in plain numpy (exact copies).

Test infrastructure only (see the package docstring).

"Flash Decoding" explainer, section 3: every generated token appends its key
and value rows to the KV cache; a paged cache keeps the rows in fixed-size
pages, found through the sequence's block table.  The oracle writes the new
rows with plain indexing, one position at a time.
"""
from __future__ import annotations

import numpy as np


def append_contiguous(cache: np.ndarray, new: np.ndarray, t: int) -> np.ndarray:
    """cache [B, Hkv, L_cap, d], new [B, Hkv, M, d]: rows t..t+M-1 replaced."""
    out = cache.copy()
    M = new.shape[2]
    for m in range(M):
        out[:, :, t + m] = new[:, :, m]
    return out


def append_paged(pool: np.ndarray, table: np.ndarray, pos: np.ndarray,
                 new: np.ndarray) -> np.ndarray:
    """pool [P, Hkv, page, d], table [B, max_pages], pos [B], new [B, Hkv, M, d].

    Position p of sequence b goes to slot p % page of page table[b, p // page].
    A position below 0, past the table row, or whose entry is not a page of
    the pool is skipped.
    """
    out = pool.copy()
    P, _, page, _ = pool.shape
    B, _, M, _ = new.shape
    for b in range(B):
        for m in range(M):
            p = int(pos[b]) + m
            if p < 0 or p // page >= table.shape[1]:
                continue
            pg = int(table[b, p // page])
            if pg < 0 or pg >= P:
                continue
            out[pg, :, p % page] = new[b, :, m]
    return out
