"""Pins for the FFD oracle: key format, top-delta selection, exact attention
over the candidates (CPU only)."""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import ffd
from oracle import flash_decoding as fd

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _bf16(x):
    return torch.from_numpy(np.asarray(x, np.float32)).to(torch.bfloat16).float().numpy()


def _keys(shape, seed, scale=1.0):
    return _bf16(scale * np.random.default_rng(seed).standard_normal(shape))


def test_golden_layout_and_rounding():
    g = json.load(open(os.path.join(GOLDEN, "ffd_pack_layout.json")))
    for case in g["cases"]:
        x = np.array(case["x"], np.float32)[None]
        p = ffd.pack_keys(x)
        assert p["codes"][0].tolist() == case["words"], case["name"]
        assert float(p["zs"][0, 0, 0]) == case["zero"], case["name"]
        assert float(p["zs"][0, 0, 1]) == case["step"], case["name"]
        assert float(p["rs"][0, 0]) == case["res_step"], case["name"]
        assert p["res"][0].tolist() == case["res"], case["name"]


def test_unpack_inverts_layout():
    rs = np.random.default_rng(1)
    codes = rs.integers(0, 4, size=(5, 128))
    words = np.zeros((5, 8), np.uint32)
    for t in range(5):
        for i in range(128):
            w, j = divmod(i, 16)
            bit = 2 * (j // 2) + (16 if j % 2 else 0)
            words[t, w] |= np.uint32(codes[t, i]) << np.uint32(bit)
    assert np.array_equal(ffd.unpack_codes(words, 128), codes)


@pytest.mark.parametrize("scale", [1.0, 0.01, 30.0])
def test_pack_error_bounds(scale):
    x = _keys((300, 128), 2, scale).astype(np.float64)
    p = ffd.pack_keys(x)
    k2, kh = ffd.dequant(p, 128)
    c = ffd.unpack_codes(p["codes"], 128)
    assert c.min() >= 0 and c.max() <= 3
    z = np.repeat(p["zs"][..., 0].astype(np.float64), 32, -1)
    s = np.repeat(p["zs"][..., 1].astype(np.float64), 32, -1)
    rs = np.repeat(p["rs"].astype(np.float64), 32, -1)
    eps16 = 2.0 ** -11
    fudge = 2.0 ** -22 * np.abs(x).max()
    assert np.all(np.abs(x - k2) <= s / 2 + eps16 * (np.abs(z) + 3 * s) + fudge)
    r = (x - k2).reshape(300, 4, 32)
    rmax = np.repeat(np.abs(r).max(-1), 32, -1)
    assert np.all(np.abs(x - kh) <= rs / 2 + eps16 * rmax + 2 * fudge)
    # the refined key is much closer than the 2-bit key
    assert np.abs(x - kh).max() < 0.05 * np.abs(x - k2).max()
    assert np.abs(p["res"]).max() <= 127


def test_constant_group():
    x = np.full((1, 64), 0.375, np.float32)
    p = ffd.pack_keys(x)
    k2, kh = ffd.dequant(p, 64)
    assert np.all(p["codes"] == 0) and np.all(p["zs"][..., 1] == 0)
    assert np.all(k2 == 0.375) and np.all(kh == 0.375)


def test_anchor_set():
    assert ffd.anchors(100, 4, 8).tolist() == [0, 1, 2, 3] + list(range(92, 100))
    assert ffd.anchors(10, 4, 8).tolist() == list(range(10))
    assert ffd.anchors(3, 4, 64).tolist() == [0, 1, 2]
    assert ffd.anchors(70, 4, 64).tolist() == [0, 1, 2, 3] + list(range(6, 70))
    assert ffd.anchors(68, 4, 64).tolist() == list(range(68))


def _exact(v):
    return Fraction(float(v))


@pytest.mark.parametrize("seed,delta", [(3, 0.5), (4, 1.0), (5, 2.0), (6, 0.0)])
def test_candidates_brute_force_exact_arithmetic(seed, delta):
    # Tiny cache: enumerate every position and decide the top-delta rule in
    # exact rational arithmetic on the stored values (d = 64 -> scale 1/8).
    L, d, n_sink, n_local = 40, 64, 3, 5
    q = _keys(d, seed)
    x = _keys((L, d), seed + 100)
    V = _keys((L, d), seed + 200).astype(np.float64)
    p = ffd.pack_keys(x)
    k2, kh = ffd.dequant(p, d)
    r = ffd.ffd_row(q.astype(np.float64), k2, kh, V, 1 / 8, delta, n_sink, n_local)
    qf = [_exact(v) for v in q]
    scan = [sum(qf[i] * _exact(k2[j, i]) for i in range(d)) / 8 for j in range(L)]
    ref = [sum(qf[i] * _exact(kh[j, i]) for i in range(d)) / 8 for j in range(L)]
    A = sorted(set(range(n_sink)) | set(range(L - n_local, L)))
    mhat = max(ref[j] for j in A)
    jstar = min(j for j in A if ref[j] == mhat)
    want = [scan[j] >= mhat - _exact(delta) or j == jstar for j in range(L)]
    assert r["cand"].tolist() == want
    assert r["jstar"] == jstar
    assert r["mhat"] == pytest.approx(float(mhat), abs=1e-13)
    # the result is the softmax over exactly those positions
    idx = [j for j in range(L) if want[j]]
    sc = np.array([float(ref[j]) for j in idx])
    w = np.exp(sc - sc.max())
    np.testing.assert_allclose(r["out"], w @ V[idx] / w.sum(), atol=1e-12)


def test_selection_is_ratio_rule_and_monotone():
    L, d = 3000, 128
    q = _keys(d, 7).astype(np.float64)
    x = _keys((L, d), 8)
    V = _keys((L, d), 9).astype(np.float64)
    k2, kh = ffd.dequant(ffd.pack_keys(x), d)
    scale = 1 / math.sqrt(d)
    prev = None
    for delta in [0.5, 1.0, 2.0, 3.0, 5.0, 7.0]:
        r = ffd.ffd_row(q, k2, kh, V, scale, delta, 4, 64)
        ratio = np.exp(r["scan"] - r["mhat"]) >= math.exp(-delta)
        ratio[r["jstar"]] = True
        near = np.abs(r["scan"] - (r["mhat"] - delta)) < 1e-12
        assert np.array_equal(r["cand"][~near], ratio[~near])
        if prev is not None:
            assert np.all(r["cand"] >= prev)      # larger delta keeps a superset
        prev = r["cand"]
    # a higher pseudo-maximum (a stronger sink) keeps a subset
    r0 = ffd.ffd_row(q, k2, kh, V, scale, 3.0, 4, 64)
    x2 = x.copy()
    x2[0] = _bf16(6.0 * math.sqrt(d) * q / (q @ q))
    k2b, khb = ffd.dequant(ffd.pack_keys(x2), d)
    r1 = ffd.ffd_row(q, k2b, khb, V, scale, 3.0, 4, 64)
    assert r1["mhat"] > r0["mhat"]
    assert np.all(r1["cand"][1:] <= r0["cand"][1:])
    assert r1["cand"].sum() < r0["cand"].sum()


def test_huge_delta_is_dense_attention_on_refined_keys():
    B, Hq, Hkv, L, d = 1, 4, 2, 500, 64
    rs = np.random.default_rng(10)
    q = _bf16(rs.standard_normal((B, Hq, d))).astype(np.float64)
    x = _bf16(rs.standard_normal((B, Hkv, L, d)))
    v = _bf16(rs.standard_normal((B, Hkv, L, d))).astype(np.float64)
    p = ffd.pack_keys(x)
    out, lse, cand, _ = ffd.ffd_attention(q, p, v, 1 / 8, 1e30, 4, 64)
    assert cand.all()
    _, kh = ffd.dequant(p, d)
    kt = torch.from_numpy(kh).repeat_interleave(2, dim=1)
    vt = torch.from_numpy(v).repeat_interleave(2, dim=1)
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q)[:, :, None], kt, vt, scale=1 / 8)[:, :, 0]
    np.testing.assert_allclose(out, ref.numpy(), atol=1e-12)


def test_anchor_always_kept():
    # Threshold above every 2-bit score: only the anchor that set the
    # pseudo-maximum survives, so the output is its value row.
    L, d = 20, 64
    q = np.zeros(d); q[0] = 1.0
    x = np.zeros((L, d), np.float32)
    x[:, 1] = 8.0                                   # group max, so step > 0
    x[2, 0] = 1.0                                   # refined-only gain at j=2
    V = _keys((L, d), 11).astype(np.float64)
    p = ffd.pack_keys(x)
    k2, kh = ffd.dequant(p, d)
    r = ffd.ffd_row(q, k2, kh, V, 1 / 8, 0.0, 4, 4)
    assert r["jstar"] == 2
    assert r["scan"][2] < r["mhat"]                 # would be dropped by the rule
    assert r["cand"].tolist() == [j == 2 for j in range(L)]
    np.testing.assert_allclose(r["out"], V[2], atol=1e-15)
    # threshold exactly at the 2-bit scores (mhat - delta == 0 == scan[j]):
    # the rule is inclusive, so every position is kept
    r2 = ffd.ffd_row(q, k2, kh, V, 1 / 8, float(r["mhat"]), 4, 4)
    assert r2["cand"].all()
