"""Fixed ("unified") maximum decode attention with overflow fallback, float64.

Test infrastructure only (see the package docstring).

"FlashDecoding" deployment blog, section 1 and the settings of section 3:
every partial softmax is taken against one fixed maximum phi chosen in
advance from the spread of the softmax inputs, so blocks need no shared
running maximum and the merge needs no rescale; the fixed maximum only holds
with high probability, so a block whose inputs leave the expected range falls
back to the original (exact) computation, or the numbers blow up (section 5,
item four, which also quotes [-16.8, 6.5] as one model's input range).

Softmax is shift invariant, so with the fallback in place the result is the
plain definition of attention: the entry point's target is the dense oracle.
This module adds the per-chunk range flags and a float64 replay of the
fixed-maximum algorithm used to pin that identity.

Readings taken where the pages are silent:

* phi and both margins are in scaled-score units (the units of q.K/sqrt(d)).
* "Out of range" for chunk c means max_{j in c} s_j > phi + margin_hi (the
  exponent could overflow) or max_{j in c} s_j < phi - margin_lo (every
  exponent of the chunk is tiny, so its sum would lose precision or vanish).
  The range quoted by the blog has two ends; the high one is the one the
  blog names.
* The fallback recomputes only the flagged chunks, with their own maximum,
  and merges them with the unflagged chunks taken at maximum phi; a
  whole-row recompute gives the same value.
"""
from __future__ import annotations

import numpy as np

from .flash_decoding import chunk_bounds, dense_attention, partials, merge


def chunk_flags_row(s: np.ndarray, bounds, phi, margin_hi, margin_lo):
    """Range flag of every chunk of one head's scaled scores s."""
    out = []
    for a, b in bounds:
        mx = s[a:b].max()
        out.append(bool(mx > phi + margin_hi or mx < phi - margin_lo))
    return np.array(out, dtype=bool)


def chunk_flags(q, k, scale, phi, margin_hi, margin_lo, chunk):
    """flags [B, Hq, n_chunks] (uint8) for a contiguous cache k [B, Hkv, L, d]."""
    B, Hq, d = q.shape
    Hkv, L = k.shape[1], k.shape[2]
    G = Hq // Hkv
    bounds = chunk_bounds(L, chunk)
    flags = np.zeros((B, Hq, len(bounds)), dtype=np.uint8)
    for b in range(B):
        for h in range(Hq):
            s = scale * (k[b, h // G] @ q[b, h])
            flags[b, h] = chunk_flags_row(s, bounds, phi, margin_hi, margin_lo)
    return flags


def unified_attention(q, k, v, scale, phi, margin_hi, margin_lo, chunk):
    """(out, lse, flags): out and lse are the dense definition (the fixed
    maximum plus fallback must reach it); flags are the chunk range flags."""
    out, lse = dense_attention(q, k, v, scale)
    return out, lse, chunk_flags(q, k, scale, phi, margin_hi, margin_lo, chunk)


def fixed_max_partials(s: np.ndarray, V: np.ndarray, phi: float, bounds):
    """Partials against the fixed maximum: l_c = sum exp(s - phi),
    O_c = sum exp(s - phi) V over each chunk (no per-chunk maximum)."""
    ls, Os = [], []
    for a, b in bounds:
        p = np.exp(s[a:b] - phi)
        ls.append(p.sum())
        Os.append(p @ V[a:b])
    return np.array(ls), np.array(Os)


def fixed_max_merge(ls: np.ndarray, Os: np.ndarray, phi: float):
    """No rescale: out = sum_c O_c / sum_c l_c, lse = phi + ln sum_c l_c."""
    den = ls.sum()
    return Os.sum(0) / den, phi + np.log(den)


def unified_row(qh, K, V, scale, phi, margin_hi, margin_lo, bounds):
    """Replay of the fixed-maximum algorithm with per-chunk fallback.

    Unflagged chunks contribute (phi, l_c, O_c) from ``fixed_max_partials``;
    flagged chunks are recomputed with their own maximum (``partials``); the
    pieces are merged exactly.  Returns (out, lse, flags).
    """
    s = scale * (K @ qh)
    flags = chunk_flags_row(s, bounds, phi, margin_hi, margin_lo)
    ms, ls, Os = [], [], []
    for c, (a, b) in enumerate(bounds):
        if flags[c]:
            m1, l1, O1 = partials(s, V, [(a, b)])
            ms.append(m1[0]); ls.append(l1[0]); Os.append(O1[0])
        else:
            l1, O1 = fixed_max_partials(s, V, phi, [(a, b)])
            ms.append(phi); ls.append(l1[0]); Os.append(O1[0])
    out, lse = merge(np.array(ms), np.array(ls), np.array(Os))
    return out, lse, flags
