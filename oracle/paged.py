"""Decode attention over a paged KV cache, in float64.

Test infrastructure only (see the package docstring).

"Flash Decoding" explainer, section 3: the cache is cut into fixed-size pages
allocated on demand (the PagedAttention idea).  Paging changes where a
token's K and V live, not what attention computes, so the oracle gathers each
sequence's logical cache through its block table with plain indexing and
applies the dense definition.
"""
from __future__ import annotations

import numpy as np

from .flash_decoding import attention_row


def gather_sequence(pool: np.ndarray, table_row: np.ndarray, L: int, page: int):
    """pool [P, Hkv, page, d], table_row [max_pages]  ->  [Hkv, L, d].

    Token t of the sequence sits in page table_row[t // page], slot t % page.
    """
    t = np.arange(L)
    rows = pool[table_row[t // page], :, t % page]      # [L, Hkv, d]
    return np.ascontiguousarray(rows.transpose(1, 0, 2)).astype(np.float64)


def paged_attention(q, k_pool, v_pool, block_table, seq_lens, page, scale,
                    rows=None):
    """q [B, Hq, d]; pools [P, Hkv, page, d]; block_table [B, max_pages];
    seq_lens [B]  ->  out [B, Hq, d], lse [B, Hq].

    A sequence of length 0 has no keys: out = 0, lse = -inf (the pages are
    silent; this is the value of an empty softmax sum).  ``rows`` optionally
    restricts the work to a list of (b, h); other entries are left NaN.
    """
    B, Hq, d = q.shape
    Hkv = k_pool.shape[1]
    G = Hq // Hkv
    out = np.full((B, Hq, d), np.nan)
    lse = np.full((B, Hq), np.nan)
    want = None if rows is None else set(map(tuple, rows))
    for b in range(B):
        hs = [h for h in range(Hq) if want is None or (b, h) in want]
        if not hs:
            continue
        L = int(seq_lens[b])
        K = gather_sequence(k_pool, block_table[b], L, page)
        V = gather_sequence(v_pool, block_table[b], L, page)
        for h in hs:
            out[b, h], lse[b, h] = attention_row(q[b, h], K[h // G], V[h // G],
                                                 scale)
    return out, lse


def paged_multi_row_attention(q, k_pool, v_pool, block_table, seq_lens, page, scale,
                              rows=None):
    """Several new tokens per sequence over a paged cache: q [B, M, Hq, d];
    pools [P, Hkv, page, d]; block_table [B, max_pages]; seq_lens [B]
    ->  out [B, M, Hq, d], lse [B, M, Hq].

    Sequence b holds L_b = seq_lens[b] positions, its M new tokens' keys and
    values among them at L_b-M .. L_b-1; token r attends to positions
    0 .. L_b-M+r ("Flash Decoding" explainer, section 1), through the block
    table (section 3).  A token with no position to attend to (L_b-M+r < 0)
    gets the empty softmax: out = 0, lse = -inf.  ``rows`` optionally
    restricts the work to a list of (b, r, h); other entries are left NaN.
    """
    B, M, Hq, d = q.shape
    Hkv = k_pool.shape[1]
    G = Hq // Hkv
    out = np.full((B, M, Hq, d), np.nan)
    lse = np.full((B, M, Hq), np.nan)
    want = None if rows is None else set(map(tuple, rows))
    for b in range(B):
        todo = [(r, h) for r in range(M) for h in range(Hq)
                if want is None or (b, r, h) in want]
        if not todo:
            continue
        L = int(seq_lens[b])
        K = gather_sequence(k_pool, block_table[b], L, page)
        V = gather_sequence(v_pool, block_table[b], L, page)
        for r, h in todo:
            n = max(L - M + r + 1, 0)
            out[b, r, h], lse[b, r, h] = attention_row(q[b, r, h], K[h // G, :n],
                                                       V[h // G, :n], scale)
    return out, lse
