"""Seeded synthetic decode-attention inputs.

Recipes follow the workloads the Flash-Decoding explainer and the FFD digest
talk about (one new query token per sequence attending over a long cached
history, grouped-query heads, contiguous or paged caches).  The pages measure
on trained models (Llama-3.1-8B, Qwen2.5-7B) and on RULER/LongBench; none of
those are available here, so every input is iid Gaussian with the planted
structure described on each function.

Randomness comes from two seeded sources:

* structural choices (sequence lengths, page permutation, planted positions,
  which heads overflow) from ``numpy.random.default_rng(seed)`` on the host,
  so they are the same whatever device builds the tensors;
* Gaussian values from a ``torch.Generator`` seeded with ``seed`` on the
  device that builds the case (CPU Mersenne-Twister or GPU Philox).  A case is
  reproducible for a given (seed, device); the oracle always receives a copy
  of the very tensors the GPU path reads.

Rounding to bf16 is torch's round-to-nearest-even conversion.  Plants are
added in float32/float64 *before* that rounding, using the bf16-rounded query.
Nothing here computes attention outputs; the only score evaluation is the
calibration of the fixed maximum (a constant chosen before either side runs).
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np
import torch

__all__ = [
    "DenseCase", "PagedCase", "UnifiedCase", "FfdCase",
    "dense_case", "paged_case", "unified_case", "ffd_case", "multi_case",
    "config_case", "CONFIGS",
]


# The five workloads, sized as the decode-attention configurations this
# library is measured on.  ``kind`` selects the entry point that consumes it.
CONFIGS = {
    1: dict(kind="dense", B=1, Hq=8, Hkv=8, L=4096, d=64, dtype="f32",
            chunk=1024, seed=101),
    2: dict(kind="dense", B=8, Hq=32, Hkv=8, L=32768, d=128, dtype="bf16",
            chunk=512, seed=102),
    # chunk 1024 for the ragged paged batch: 7 units per resident wave, the
    # best of a sweep over 256 .. 2048 (512: 614 us, 1024: 578 us on MI355X)
    3: dict(kind="paged", B=16, Hq=32, Hkv=8, d=128, len_lo=1024,
            len_hi=131072, page=16, chunk=1024, seed=103),
    4: dict(kind="unified", B=4, Hq=32, Hkv=8, L=65536, d=128, chunk=512,
            plant_frac=0.02, plant_coef=0.5, over_frac=0.01, over_shift=15.0,
            margin_hi=10.0, margin_lo=40.0, seed=104, cal_seed=1104),
    5: dict(kind="ffd", B=4, Hq=32, Hkv=8, L=65536, d=128, n_sink=4,
            n_local=64, deltas=(5.0, 7.0), sink_shift=3.0, plant_frac=0.01,
            plant_shift=5.0, chunk=1024, seed=105),
    # Peaked queries (sharper softmax, heads of a group alike): per-head
    # sparsity ~83 % at delta 5 and ~73 % at delta 7, the levels the FFD digest
    # reports; the union over a group of 4 keeps ~29 % / ~41 % of positions.
    6: dict(kind="ffd", B=4, Hq=32, Hkv=8, L=65536, d=128, n_sink=4,
            n_local=64, deltas=(5.0, 7.0), sink_shift=3.0, plant_frac=0.01,
            plant_shift=5.0, chunk=1024, seed=106, q_scale=5.0, q_shared=0.95),
}


def _gen(seed: int, device) -> torch.Generator:
    g = torch.Generator(device=torch.device(device))
    g.manual_seed(int(seed))
    return g


def _randn(shape, gen, device) -> torch.Tensor:
    return torch.randn(tuple(shape), generator=gen, device=device,
                       dtype=torch.float32)


def _store(x: torch.Tensor, dtype: str) -> torch.Tensor:
    if dtype == "bf16":
        return x.to(torch.bfloat16)
    if dtype == "f32":
        return x.to(torch.float32)
    raise ValueError(f"unknown storage dtype {dtype!r}")


def _group_plant(qg: np.ndarray, targets: np.ndarray) -> np.ndarray:
    """Minimum-norm key offset D with qg[h] . D = targets[h] for every head h.

    qg is the [G, d] block of (bf16-rounded) queries that share one kv-head.
    D = qg^T (qg qg^T)^-1 t.  For G = 1 and t = c*|q|^2 this is c*q.
    """
    gram = qg @ qg.T
    return qg.T @ np.linalg.solve(gram, targets)


@dataclass
class DenseCase:
    q: torch.Tensor          # [B, Hq, d]
    k: torch.Tensor          # [B, Hkv, L, d]
    v: torch.Tensor          # [B, Hkv, L, d]
    scale: float
    chunk: int
    meta: dict = field(default_factory=dict)


@dataclass
class PagedCase:
    q: torch.Tensor           # [B, Hq, d], or [B, M, Hq, d] for several tokens
    k_pool: torch.Tensor      # [P, Hkv, page, d]
    v_pool: torch.Tensor      # [P, Hkv, page, d]
    block_table: torch.Tensor  # int32 [B, max_pages]; unused entries -1
    seq_lens: torch.Tensor    # int32 [B]
    page: int
    scale: float
    chunk: int
    meta: dict = field(default_factory=dict)


@dataclass
class UnifiedCase:
    q: torch.Tensor
    k: torch.Tensor
    v: torch.Tensor
    scale: float
    chunk: int
    phi: float
    margin_hi: float
    margin_lo: float
    overflow_heads: list      # [(b, hq, position)] planted above phi
    meta: dict = field(default_factory=dict)


@dataclass
class FfdCase:
    q: torch.Tensor           # bf16 [B, Hq, d]
    k: torch.Tensor           # bf16 [B, Hkv, L, d] (unpacked keys)
    v: torch.Tensor           # bf16 [B, Hkv, L, d]
    scale: float
    chunk: int
    n_sink: int
    n_local: int
    deltas: tuple
    meta: dict = field(default_factory=dict)


def dense_case(B, Hq, Hkv, L, d, dtype="bf16", chunk=512, seed=0,
               device="cpu") -> DenseCase:
    """q, K, V iid N(0, 1), drawn in that order, then stored as ``dtype``."""
    g = _gen(seed, device)
    q = _store(_randn((B, Hq, d), g, device), dtype)
    k = _store(_randn((B, Hkv, L, d), g, device), dtype)
    v = _store(_randn((B, Hkv, L, d), g, device), dtype)
    return DenseCase(q, k, v, 1.0 / math.sqrt(d), int(chunk),
                     dict(B=B, Hq=Hq, Hkv=Hkv, L=L, d=d, dtype=dtype, seed=seed))


def multi_case(B, M, Hq, Hkv, L, d, chunk=512, seed=0, device="cpu",
               q_scale=1.0) -> DenseCase:
    """Several new query tokens per sequence: q [B, M, Hq, d] (times
    ``q_scale`` for sharper scores), K, V [B, Hkv, L, d], the M tokens' keys
    and values being the last M positions; all iid N(0, 1), drawn in that
    order, stored as bf16."""
    g = _gen(seed, device)
    q = (q_scale * _randn((B, M, Hq, d), g, device)).to(torch.bfloat16)
    k = _randn((B, Hkv, L, d), g, device).to(torch.bfloat16)
    v = _randn((B, Hkv, L, d), g, device).to(torch.bfloat16)
    return DenseCase(q, k, v, 1.0 / math.sqrt(d), int(chunk),
                     dict(B=B, M=M, Hq=Hq, Hkv=Hkv, L=L, d=d, dtype="bf16", seed=seed,
                          q_scale=q_scale))


def paged_case(B, Hq, Hkv, d, len_lo, len_hi, page=16, chunk=512, seed=0,
               device="cpu", lens=None, max_pages=None, M=None) -> PagedCase:
    """Ragged sequences in a shared page pool.

    M: several new query tokens per sequence, q [B, M, Hq, d] (their keys
    and values are each sequence's last M positions); None: q [B, Hq, d].

    Lengths are uniform integers in [len_lo, len_hi] (unless ``lens`` is
    given).  The pool holds exactly the pages the sequences need; a random
    permutation of the pool's page ids is dealt out to the sequences in order,
    so every sequence's pages are scattered through the pool.  Unused slots of
    a sequence's last page are zero; unused block-table entries are -1.
    Values: q first, then per sequence K_b [Hkv, L_b, d] and V_b.
    """
    rs = np.random.default_rng(seed)
    if lens is None:
        lens = rs.integers(len_lo, len_hi, size=B, endpoint=True)
    lens = np.asarray(lens, dtype=np.int64)
    assert lens.shape == (B,)
    n_pages = (lens + page - 1) // page
    total = int(n_pages.sum())
    perm = rs.permutation(total) if total > 0 else np.zeros(0, np.int64)
    if max_pages is None:
        max_pages = max(1, (int(len_hi) + page - 1) // page)
    assert int(n_pages.max(initial=0)) <= max_pages
    table = np.full((B, max_pages), -1, dtype=np.int32)
    off = 0
    for b in range(B):
        table[b, :n_pages[b]] = perm[off:off + n_pages[b]]
        off += int(n_pages[b])

    g = _gen(seed, device)
    q = _randn((B, Hq, d) if M is None else (B, M, Hq, d), g, device).to(torch.bfloat16)
    k_pool = torch.zeros((max(total, 1), Hkv, page, d), dtype=torch.bfloat16,
                         device=device)
    v_pool = torch.zeros_like(k_pool)
    for b in range(B):
        Lb, nb = int(lens[b]), int(n_pages[b])
        if Lb == 0:
            continue
        ids = torch.as_tensor(table[b, :nb].astype(np.int64), device=device)
        for pool in (k_pool, v_pool):
            x = torch.zeros((Hkv, nb * page, d), dtype=torch.bfloat16,
                            device=device)
            x[:, :Lb] = _randn((Hkv, Lb, d), g, device).to(torch.bfloat16)
            pool[ids] = x.view(Hkv, nb, page, d).permute(1, 0, 2, 3)
    return PagedCase(q, k_pool, v_pool,
                     torch.as_tensor(table, device=device),
                     torch.as_tensor(lens.astype(np.int32), device=device),
                     int(page), 1.0 / math.sqrt(d), int(chunk),
                     dict(B=B, Hq=Hq, Hkv=Hkv, d=d, lens=lens.tolist(),
                          pages=total, max_pages=max_pages, seed=seed))


def _calibrate_phi(Hq, Hkv, L, d, plant_frac, plant_coef, seed, device) -> float:
    """Fixed maximum for the unified-max path: the largest scaled score on a
    separate calibration draw of the same recipe (one sequence, at most 8192
    positions, no overflow plants), rounded up to a multiple of 1/16."""
    Lc = min(L, 8192)
    g = _gen(seed, device)
    rs = np.random.default_rng(seed)
    G = Hq // Hkv
    q = _randn((1, Hq, d), g, device).to(torch.bfloat16)
    k = _randn((1, Hkv, Lc, d), g, device)
    qd = q.double().cpu().numpy()
    n_plant = int(round(plant_frac * Lc))
    for gi in range(Hkv):
        qg = qd[0, gi * G:(gi + 1) * G]
        delta = _group_plant(qg, plant_coef * (qg * qg).sum(1))
        pos = torch.as_tensor(rs.choice(Lc, n_plant, replace=False), device=device)
        k[0, gi, pos] += torch.as_tensor(delta, dtype=torch.float32, device=device)
    kd = k.to(torch.bfloat16).double()[0]                   # [Hkv, Lc, d]
    qh = q.double()[0].view(Hkv, G, d).transpose(1, 2).contiguous()  # [Hkv, d, G]
    smax = float(torch.matmul(kd, qh).max()) / math.sqrt(d)
    return math.ceil(smax * 16.0) / 16.0


def unified_case(B, Hq, Hkv, L, d, chunk=512, plant_frac=0.02, plant_coef=0.5,
                 over_frac=0.01, over_shift=15.0, margin_hi=10.0, margin_lo=40.0,
                 seed=0, cal_seed=None, device="cpu", phi=None) -> UnifiedCase:
    """Concentrated scores for the fixed-maximum path.

    On round(plant_frac*L) random positions per (sequence, kv-head) the key
    gets the minimum-norm offset that raises every query head of the group by
    plant_coef*|q_h|^2 in q.K (the key is pulled 0.5 along q when G = 1).
    phi comes from a calibration draw (``_calibrate_phi``) unless given.
    Then ceil(over_frac*B*Hq) query heads each get one position whose key is
    replaced by (phi + over_shift) * sqrt(d) * q_h / |q_h|^2, so that head's
    scaled score there is phi + over_shift (before bf16 rounding of the key):
    those heads must take the overflow fallback.
    """
    G = Hq // Hkv
    rs = np.random.default_rng(seed)
    g = _gen(seed, device)
    q = _randn((B, Hq, d), g, device).to(torch.bfloat16)
    k = _randn((B, Hkv, L, d), g, device)
    v = _randn((B, Hkv, L, d), g, device).to(torch.bfloat16)
    qd = q.double().cpu().numpy()
    n_plant = int(round(plant_frac * L))
    for b in range(B):
        for gi in range(Hkv):
            qg = qd[b, gi * G:(gi + 1) * G]
            delta = _group_plant(qg, plant_coef * (qg * qg).sum(1))
            pos = torch.as_tensor(rs.choice(L, n_plant, replace=False), device=device)
            k[b, gi, pos] += torch.as_tensor(delta, dtype=torch.float32, device=device)
    if phi is None:
        phi = _calibrate_phi(Hq, Hkv, L, d, plant_frac, plant_coef,
                             seed if cal_seed is None else cal_seed, device)
    n_over = int(math.ceil(over_frac * B * Hq)) if over_frac > 0 else 0
    over = []
    if n_over:
        for flat in rs.choice(B * Hq, n_over, replace=False):
            b, h = divmod(int(flat), Hq)
            j = int(rs.integers(L))
            qh = qd[b, h]
            key = (phi + over_shift) * math.sqrt(d) * qh / float(qh @ qh)
            k[b, h // G, j] = torch.as_tensor(key, dtype=torch.float32, device=device)
            over.append((b, h, j))
    k = k.to(torch.bfloat16)
    return UnifiedCase(q, k, v, 1.0 / math.sqrt(d), int(chunk), float(phi),
                       float(margin_hi), float(margin_lo), over,
                       dict(B=B, Hq=Hq, Hkv=Hkv, L=L, d=d, seed=seed))


def ffd_case(B, Hq, Hkv, L, d, n_sink=4, n_local=64, deltas=(5.0, 7.0),
             sink_shift=3.0, plant_frac=0.01, plant_shift=5.0, chunk=1024,
             seed=0, device="cpu", q_scale=1.0, q_shared=0.0) -> FfdCase:
    """Keys with attention-sink and needle structure for the sparse path.

    The first n_sink keys of every (sequence, kv-head) get the minimum-norm
    offset that raises each head's scaled score by sink_shift; round(
    plant_frac*L) keys drawn from positions [n_sink, L - n_local) get one that
    raises it by plant_shift (kept out of the anchor window, so the
    pseudo-maximum taken from the anchors sits below the true maximum).

    Peaked variant: q = q_scale * (rho * u_g + sqrt(1 - rho^2) * e_h) with
    rho = q_shared, one u_g per kv-head group and one e_h per head (all
    N(0, 1)): scores spread by q_scale (sharper softmax) and the heads of a
    group attend to similar positions.  q_scale = 1, q_shared = 0 is plain iid.
    """
    G = Hq // Hkv
    rs = np.random.default_rng(seed)
    g = _gen(seed, device)
    q = _randn((B, Hq, d), g, device)
    if q_shared != 0.0:
        u = _randn((B, Hkv, 1, d), g, device).expand(B, Hkv, G, d).reshape(B, Hq, d)
        q = q_shared * u + math.sqrt(1.0 - q_shared * q_shared) * q
    q = (q_scale * q).to(torch.bfloat16)
    k = _randn((B, Hkv, L, d), g, device)
    v = _randn((B, Hkv, L, d), g, device).to(torch.bfloat16)
    qd = q.double().cpu().numpy()
    n_plant = int(round(plant_frac * L))
    lo, hi = min(n_sink, L), max(min(n_sink, L), L - n_local)
    n_plant = min(n_plant, hi - lo)
    for b in range(B):
        for gi in range(Hkv):
            qg = qd[b, gi * G:(gi + 1) * G]
            unit = np.full(G, math.sqrt(d))
            if n_sink > 0 and sink_shift != 0:
                dk = torch.as_tensor(_group_plant(qg, sink_shift * unit),
                                     dtype=torch.float32, device=device)
                k[b, gi, :min(n_sink, L)] += dk
            if n_plant > 0 and plant_shift != 0:
                dk = torch.as_tensor(_group_plant(qg, plant_shift * unit),
                                     dtype=torch.float32, device=device)
                pos = rs.choice(np.arange(lo, hi), n_plant, replace=False)
                k[b, gi, torch.as_tensor(pos, device=device)] += dk
    k = k.to(torch.bfloat16)
    return FfdCase(q, k, v, 1.0 / math.sqrt(d), int(chunk), int(n_sink),
                   int(n_local), tuple(float(x) for x in deltas),
                   dict(B=B, Hq=Hq, Hkv=Hkv, L=L, d=d, seed=seed))


def config_case(i: int, device="cpu", **override):
    """Build workload ``i`` (1-5) at its full size, or with ``override``."""
    cfg = dict(CONFIGS[i])
    cfg.update(override)
    kind = cfg.pop("kind")
    if kind == "dense":
        return dense_case(device=device, **cfg)
    if kind == "paged":
        return paged_case(device=device, **cfg)
    if kind == "unified":
        return unified_case(device=device, **cfg)
    if kind == "ffd":
        return ffd_case(device=device, **cfg)
    raise ValueError(kind)
