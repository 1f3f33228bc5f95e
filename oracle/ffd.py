"""FFD sparse decode attention (2-bit scan, pseudo-max, top-delta, 8-bit
refine, exact attention over the candidates), float64.

Test infrastructure only (see the package docstring).

Source: the "Faster Than Flash" digest (longzhangge.com).
* Section 5 and Fig. 2: each key is stored as a 2-bit main part, scanned for
  every position, plus an 8-bit residual, read only for candidates.
* Section 4: a pseudo-maximum is the largest quickly-computed score over a
  few anchor positions: the attention-sink tokens at the start and a local
  window of recent tokens.
* Section 3: top-delta keeps position j for query i iff s_ij >= m_i - delta,
  i.e. exp(s_ij) / exp(m_i) >= exp(-delta); no sort.
* Fig. 2 / section 6: after the selection the candidates' scores are refined
  with the residual and exact attention is taken over them.

FFD approximates dense attention, so this oracle replays the algorithm on the
exact stored (packed) values instead of comparing with the dense result.

Storage format (the pages name only "2-bit main part plus 8-bit residual";
the grouping is per token, 32 consecutive dimensions per group, asymmetric):

* zero z = fp16(min over the group), step s = fp16((max - min) / 3);
* code c = clamp(rne((x - z) / s), 0, 3), and c = 0 when s = 0;
* residual r = x - (z + s*c); rs = fp16(max_group |r| / 127);
  r8 = clamp(rne(r / rs), -127, 127), and r8 = 0 when rs = 0;
* the 2-bit key is z + s*c; the refined key is z + s*c + rs*r8.

The integer decisions (c, r8) and the stored fp16 values are computed in
float32 with each operation rounded to nearest even, the precision the GPU
packer uses; z + s*c is formed with a single rounding (as a fused
multiply-add).  Inputs must be finite with |x| < 65504.

Bit layout of the codes: one uint32 word per 16 consecutive dimensions
[16w, 16w + 16); dimension 16w + 2p (p = 0..7) sits at bits 2p..2p+1 and
dimension 16w + 2p + 1 at bits 16 + 2p..17 + 2p.  (Even dimensions fill the
low half-word, odd dimensions the high half-word.)  Arrays:
    codes uint32 [..., d/16]
    zs    fp16   [..., d/32, 2]   (zero, step) per group
    res   int8   [..., d]
    rs    fp16   [..., d/32]
"""
from __future__ import annotations

import numpy as np

GROUP = 32


def pack_keys(k: np.ndarray):
    """Quantise keys k [..., d] (float32-representable) -> dict of arrays."""
    k = np.asarray(k, dtype=np.float32)
    d = k.shape[-1]
    assert d % GROUP == 0
    lead = k.shape[:-1]
    x = k.reshape(*lead, d // GROUP, GROUP)
    mn = x.min(-1)
    mx = x.max(-1)
    z16 = mn.astype(np.float16)
    s16 = ((mx - mn) / np.float32(3.0)).astype(np.float16)
    z = z16.astype(np.float32)[..., None]
    s = s16.astype(np.float32)[..., None]
    with np.errstate(divide="ignore", invalid="ignore"):
        t = (x - z) / s
        code = np.where(s == 0, 0.0, np.clip(np.rint(t), 0, 3))
    code = np.nan_to_num(code).astype(np.uint32)
    # z + s*code with one rounding: the float64 product and sum are exact for
    # fp16 operands and a 2-bit code, so rounding once to float32 is an fma.
    base = (s.astype(np.float64) * code + z.astype(np.float64)).astype(np.float32)
    r = x - base
    rs16 = (np.abs(r).max(-1) / np.float32(127.0)).astype(np.float16)
    rs = rs16.astype(np.float32)[..., None]
    with np.errstate(divide="ignore", invalid="ignore"):
        u = r / rs
        r8 = np.where(rs == 0, 0.0, np.clip(np.rint(u), -127, 127))
    r8 = np.nan_to_num(r8).astype(np.int8)

    c = code.reshape(*lead, d // 16, 8, 2)
    shifts = (2 * np.arange(8)).astype(np.uint32)
    words = ((c[..., 0] << shifts).sum(-1, dtype=np.uint32)
             | (c[..., 1] << (shifts + 16)).sum(-1, dtype=np.uint32))
    zs = np.stack([z16, s16], axis=-1)
    return dict(codes=words.astype(np.uint32), zs=zs, res=r8.reshape(*lead, d),
                rs=rs16)


def unpack_codes(words: np.ndarray, d: int) -> np.ndarray:
    """uint32 [..., d/16] -> integer codes [..., d] (inverse of the layout)."""
    words = np.asarray(words, dtype=np.uint32)
    lead = words.shape[:-1]
    p = np.arange(8, dtype=np.uint32)
    even = (words[..., None] >> (2 * p)) & 3
    odd = (words[..., None] >> (16 + 2 * p)) & 3
    return np.stack([even, odd], axis=-1).reshape(*lead, d).astype(np.int64)


def dequant(packed, d: int):
    """Exact float64 values of the stored keys: (2-bit key, refined key)."""
    c = unpack_codes(packed["codes"], d).astype(np.float64)
    lead = c.shape[:-1]
    zs = packed["zs"].astype(np.float64)
    z = np.repeat(zs[..., 0], GROUP, axis=-1).reshape(*lead, d)
    s = np.repeat(zs[..., 1], GROUP, axis=-1).reshape(*lead, d)
    rs = np.repeat(packed["rs"].astype(np.float64), GROUP, axis=-1).reshape(*lead, d)
    k2 = z + s * c
    return k2, k2 + rs * packed["res"].astype(np.float64)


def anchors(L: int, n_sink: int, n_local: int) -> np.ndarray:
    """Anchor positions: the first n_sink and the last n_local positions
    (section 4), as a sorted set (they overlap when L < n_sink + n_local)."""
    a = set(range(min(n_sink, L))) | set(range(max(0, L - n_local), L))
    return np.array(sorted(a), dtype=np.int64)


def ffd_row(qh, K2, Khat, V, scale, delta, n_sink, n_local):
    """FFD for one query head over one kv-head's cache.

    qh [d]; K2, Khat, V [L, d] (2-bit keys, refined keys, values).
    Returns dict(out, lse, cand (bool [L]), mhat, jstar, scan, refined).

    1. scan[j] = scale * qh . K2[j]           (2-bit scores, every position)
    2. refined[j] = scale * qh . Khat[j]      (needed only at anchors and
       candidates; all computed here, which changes nothing)
    3. mhat = max over anchors of refined; jstar = lowest anchor attaining it.
       Reading: anchors are scored with the most precise key the format
       holds.
    4. cand = {j : scan[j] >= mhat - delta} plus jstar (reading: the anchor
       that set the threshold is always kept, so the set is never empty).
    5. Exact softmax over cand with the refined scores and its own maximum.
    """
    L = K2.shape[0]
    scan = scale * (K2 @ qh)
    refined = scale * (Khat @ qh)
    A = anchors(L, n_sink, n_local)
    mhat = refined[A].max()
    jstar = int(A[np.nonzero(refined[A] == mhat)[0][0]])
    cand = scan >= mhat - delta
    cand[jstar] = True
    sc = refined[cand]
    M = sc.max()
    w = np.exp(sc - M)
    den = w.sum()
    return dict(out=(w @ V[cand]) / den, lse=M + np.log(den), cand=cand,
                mhat=mhat, jstar=jstar, scan=scan, refined=refined)


def ffd_attention(q, packed, v, scale, delta, n_sink, n_local, rows=None):
    """Batched FFD.  q [B, Hq, d]; packed arrays [B, Hkv, L, ...];
    v [B, Hkv, L, d].  Returns out [B, Hq, d], lse [B, Hq], cand [B, Hq, L],
    mhat [B, Hq]; entries outside ``rows`` (list of (b, h)) stay NaN/False.
    """
    B, Hq, d = q.shape
    Hkv, L = v.shape[1], v.shape[2]
    G = Hq // Hkv
    out = np.full((B, Hq, d), np.nan)
    lse = np.full((B, Hq), np.nan)
    mhat = np.full((B, Hq), np.nan)
    cand = np.zeros((B, Hq, L), dtype=bool)
    want = None if rows is None else set(map(tuple, rows))
    for b in range(B):
        for g in range(Hkv):
            hs = [h for h in range(g * G, (g + 1) * G)
                  if want is None or (b, h) in want]
            if not hs:
                continue
            sub = {key: arr[b, g] for key, arr in packed.items()}
            K2, Khat = dequant(sub, d)
            for h in hs:
                r = ffd_row(q[b, h], K2, Khat, v[b, g], scale, delta, n_sink,
                            n_local)
                out[b, h], lse[b, h], mhat[b, h] = r["out"], r["lse"], r["mhat"]
                cand[b, h] = r["cand"]
    return out, lse, cand, mhat
