"""Multi-row decode attention: several new query tokens per sequence, float64.

Test infrastructure only (see the package docstring).

"Flash Decoding" explainer, section 1: a token's query attends to the keys of
every position up to and including its own.  With M new tokens whose keys
and values are already appended at the end of the cache (positions
L-M .. L-1), token r (0-based) sees positions 0 .. L-M+r.  The
"FlashDecoding" deployment blog, section 1 (flat GEMM for queries with few
rows): the rows of the M tokens and of the G query heads of a kv-head share
one read of K and V.  The oracle applies the plain definition to each
(sequence, token, head), one row at a time.
"""
from __future__ import annotations

import numpy as np

from .flash_decoding import attention_row


def visible(L: int, M: int, r: int) -> int:
    """Number of cache positions token r of M new tokens attends to."""
    return L - M + r + 1


def multi_row_attention(q, k, v, scale, rows=None):
    """q [B, M, Hq, d]; k, v [B, Hkv, L, d]  ->  out [B, M, Hq, d], lse [B, M, Hq].

    ``rows`` optionally restricts the work to a list of (b, r, h); other
    entries are left NaN.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    B, M, Hq, d = q.shape
    Hkv, L = k.shape[1], k.shape[2]
    G = Hq // Hkv
    assert L >= M
    out = np.full((B, M, Hq, d), np.nan)
    lse = np.full((B, M, Hq), np.nan)
    todo = rows if rows is not None else [(b, r, h) for b in range(B) for r in range(M)
                                          for h in range(Hq)]
    for b, r, h in todo:
        n = visible(L, M, r)
        out[b, r, h], lse[b, r, h] = attention_row(q[b, r, h], k[b, h // G, :n],
                                                   v[b, h // G, :n], scale)
    return out, lse
