"""Dense decode attention and the split-KV identity, in float64.

Test infrastructure only (see the package docstring).

The target of every dense entry point is the plain definition of attention
("Flash Decoding" explainer, section 1): scores S = q K^T, scaled by
1/sqrt(d_k), turned into weights by softmax, and used to average V.  Split-KV
decoding reaches exactly this (section 2 calls the merge an identity, not an
approximation), so the GPU is compared with the definition itself and not
with a chunked replay.  The chunked routines below exist to pin that identity
and the merge formula.
"""
from __future__ import annotations

import numpy as np


def attention_row(qh: np.ndarray, K: np.ndarray, V: np.ndarray, scale: float):
    """Attention of one query vector over one head's cache.

    qh [d], K [L, d], V [L, d]  ->  (out [d], lse)

    Section 1, steps 1-4: s = scale * K qh; softmax taken with the maximum
    subtracted first (the numpy demonstration's step 2, which keeps exp from
    overflowing and leaves the weights unchanged); out = sum_j w_j V_j.
    lse = m + ln sum_j exp(s_j - m) is the log of the softmax denominator,
    returned so merges can be checked.  L = 0 gives out = 0, lse = -inf.
    """
    L = K.shape[0]
    if L == 0:
        return np.zeros(V.shape[1]), -np.inf
    s = scale * (K @ qh)
    m = s.max()
    w = np.exp(s - m)
    den = w.sum()
    return (w @ V) / den, m + np.log(den)


def dense_attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, scale: float):
    """q [B, Hq, d], k/v [B, Hkv, L, d]  ->  out [B, Hq, d], lse [B, Hq].

    Grouped-query heads: query head h reads kv-head h // (Hq // Hkv) (heads
    of a group are consecutive).  The pages never mention head grouping; this
    is the plain reading of a cache with fewer kv-heads than query heads.
    """
    B, Hq, d = q.shape
    Hkv = k.shape[1]
    assert Hq % Hkv == 0
    G = Hq // Hkv
    out = np.empty((B, Hq, d))
    lse = np.empty((B, Hq))
    for b in range(B):
        for h in range(Hq):
            out[b, h], lse[b, h] = attention_row(q[b, h], k[b, h // G],
                                                 v[b, h // G], scale)
    return out, lse


def chunk_bounds(L: int, chunk: int):
    """Chunk c covers [c*chunk, min((c+1)*chunk, L)); no empty chunks.

    Section 2 cuts the cache along the sequence into B blocks; its
    demonstration assumes the length divides evenly.  The plain reading for a
    ragged tail: the last block is shorter.
    """
    return [(a, min(a + chunk, L)) for a in range(0, L, chunk)]


def partials(s: np.ndarray, V: np.ndarray, bounds):
    """Per-block statistics of section 2, step 1.

    For block i over positions [a, b): m_i = max s, l_i = sum exp(s - m_i),
    O_i = sum exp(s - m_i) V  (O_i is NOT normalised by l_i).
    """
    ms, ls, Os = [], [], []
    for a, b in bounds:
        si = s[a:b]
        mi = si.max()
        p = np.exp(si - mi)
        ms.append(mi)
        ls.append(p.sum())
        Os.append(p @ V[a:b])
    return np.array(ms), np.array(ls), np.array(Os)


def merge(ms: np.ndarray, ls: np.ndarray, Os: np.ndarray):
    """Exact merge of unnormalised block partials (section 2, steps 2-4).

    m = max_i m_i; w_i = exp(m_i - m); out = sum_i w_i O_i / sum_i w_i l_i;
    lse = m + ln sum_i w_i l_i.

    Reading taken: the section's displayed merge multiplies each block's
    output by exp(m_i - m) * l_i, which is right when O_i is the block's
    NORMALISED output, but its step 1 (and the demonstration) define O_i
    unnormalised; combining the two as printed is wrong.  With unnormalised
    O_i the weight on O_i is exp(m_i - m) alone, while the denominator keeps
    exp(m_i - m) * l_i.  Both consistent readings give the same result; the
    test suite checks that the as-printed combination does not.
    """
    m = ms.max()
    w = np.exp(ms - m)
    den = (w * ls).sum()
    return (w @ Os) / den, m + np.log(den)


def split_kv_row(qh, K, V, scale, bounds):
    """Flash-Decoding for one query head: block partials, then the merge."""
    s = scale * (K @ qh)
    return merge(*partials(s, V, bounds))
