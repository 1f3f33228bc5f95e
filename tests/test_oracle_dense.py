"""Pins for the dense oracle and the split-KV identity (CPU only).

Each test ties the oracle to something other than itself: a library routine
(torch's scaled_dot_product_attention in float64), hand-derived values,
closed forms, or invariants the "Flash Decoding" explainer states (section 2:
the block merge is an exact identity; the numpy demonstration subtracts the
maximum before exp).
"""
import json
import math
import os

import numpy as np
import pytest
import torch

from oracle import flash_decoding as fd

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


def test_hand_worked_softmax():
    g = json.load(open(os.path.join(GOLDEN, "hand_softmax.json")))
    out, lse = fd.attention_row(np.array(g["q"]), np.array(g["K"]),
                                np.array(g["V"]), g["scale"])
    np.testing.assert_allclose(out, g["out"], atol=1e-14)
    assert abs(lse - g["lse"]) < 1e-14


@pytest.mark.parametrize("B,Hq,Hkv,L,d", [(2, 8, 8, 300, 64), (2, 8, 2, 257, 128),
                                          (1, 4, 1, 1000, 32)])
def test_matches_torch_sdpa(B, Hq, Hkv, L, d):
    q = _rand((B, Hq, d), 1)
    k = _rand((B, Hkv, L, d), 2)
    v = _rand((B, Hkv, L, d), 3)
    scale = 1 / math.sqrt(d)
    out, lse = fd.dense_attention(q, k, v, scale)
    G = Hq // Hkv
    kt = torch.from_numpy(k).repeat_interleave(G, dim=1)
    vt = torch.from_numpy(v).repeat_interleave(G, dim=1)
    qt = torch.from_numpy(q)[:, :, None, :]
    ref = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, scale=scale)
    np.testing.assert_allclose(out, ref[:, :, 0].numpy(), atol=1e-12)
    s = torch.matmul(qt, kt.transpose(-1, -2).contiguous())[:, :, 0] * scale
    np.testing.assert_allclose(lse, torch.logsumexp(s, -1).numpy(), atol=1e-12)


def test_gqa_head_mapping():
    # V of kv-head g is the constant g everywhere: query head h must read
    # kv-head h // G, so its output is exactly h // G.
    B, Hq, Hkv, L, d = 2, 8, 2, 50, 16
    q = _rand((B, Hq, d), 4)
    k = _rand((B, Hkv, L, d), 5)
    v = np.zeros((B, Hkv, L, d))
    for g in range(Hkv):
        v[:, g] = g
    out, _ = fd.dense_attention(q, k, v, 0.25)
    for h in range(Hq):
        np.testing.assert_allclose(out[:, h], h // (Hq // Hkv), atol=1e-12)


def test_single_key_returns_value():
    q, K, V = _rand(64, 6), _rand((1, 64), 7), _rand((1, 64), 8)
    out, lse = fd.attention_row(q, K, V, 0.125)
    assert np.array_equal(out, V[0])
    assert lse == pytest.approx(0.125 * float(K[0] @ q), abs=1e-14)


def test_equal_scores_return_mean():
    K, V = _rand((777, 32), 9), _rand((777, 32), 10)
    out, lse = fd.attention_row(np.zeros(32), K, V, 0.3)
    np.testing.assert_allclose(out, V.mean(0), atol=1e-13)
    assert lse == pytest.approx(math.log(777), abs=1e-12)
    # every key identical: same conclusion for any query
    Kc = np.repeat(K[:1], 777, axis=0)
    out2, _ = fd.attention_row(_rand(32, 11), Kc, V, 0.3)
    np.testing.assert_allclose(out2, V.mean(0), atol=1e-13)


def test_two_keys_closed_form():
    q, K, V = _rand(16, 12), _rand((2, 16), 13), _rand((2, 16), 14)
    s = 0.25 * (K @ q)
    sig = 1 / (1 + math.exp(-(s[0] - s[1])))
    out, lse = fd.attention_row(q, K, V, 0.25)
    np.testing.assert_allclose(out, sig * V[0] + (1 - sig) * V[1], atol=1e-14)
    assert lse == pytest.approx(math.log(math.exp(s[0]) + math.exp(s[1])), abs=1e-13)


@pytest.mark.parametrize("c", [0.0, 30.0, 1000.0])
def test_shift_invariance(c):
    # K_j += w with scale*q.w = c raises every score by c: softmax weights and
    # output unchanged, lse up by c.  At c = 1000 exp without the maximum
    # subtracted would overflow.
    d, L, scale = 32, 400, 1 / math.sqrt(32)
    q, K, V = _rand(d, 15), _rand((L, d), 16), _rand((L, d), 17)
    w = c * q / (scale * (q @ q))
    o0, l0 = fd.attention_row(q, K, V, scale)
    o1, l1 = fd.attention_row(q, K + w, V, scale)
    np.testing.assert_allclose(o1, o0, atol=1e-9)
    assert l1 - c == pytest.approx(l0, abs=1e-9)
    assert np.all(np.isfinite(o1))


@pytest.mark.parametrize("chunk", [1, 16, 64, 512, 1024, 4096])
def test_split_kv_equals_definition(chunk):
    d, L, scale = 64, 4096, 1 / 8
    q, K, V = _rand(d, 18), _rand((L, d), 19), _rand((L, d), 20)
    ref, lse_ref = fd.attention_row(q, K, V, scale)
    out, lse = fd.split_kv_row(q, K, V, scale, fd.chunk_bounds(L, chunk))
    np.testing.assert_allclose(out, ref, atol=1e-13)
    assert lse == pytest.approx(lse_ref, abs=1e-12)


def test_split_kv_uneven_cuts_and_ragged_tail():
    d, L, scale = 32, 1000, 0.2
    q, K, V = _rand(d, 21), _rand((L, d), 22), _rand((L, d), 23)
    ref, lse_ref = fd.attention_row(q, K, V, scale)
    rs = np.random.default_rng(24)
    for _ in range(5):
        cuts = np.sort(rs.choice(np.arange(1, L), 7, replace=False))
        edges = [0, *cuts.tolist(), L]
        out, lse = fd.split_kv_row(q, K, V, scale, list(zip(edges[:-1], edges[1:])))
        np.testing.assert_allclose(out, ref, atol=1e-13)
        assert lse == pytest.approx(lse_ref, abs=1e-12)
    assert fd.chunk_bounds(1000, 256)[-1] == (768, 1000)
    assert fd.chunk_bounds(1024, 256)[-1] == (768, 1024)


def test_merge_independent_of_order_and_associative():
    d, L, scale = 32, 900, 0.3
    q, K, V = _rand(d, 25), 3 * _rand((L, d), 26), _rand((L, d), 27)
    s = scale * (K @ q)
    ms, ls, Os = fd.partials(s, V, fd.chunk_bounds(L, 100))
    ref, lse_ref = fd.merge(ms, ls, Os)
    perm = np.random.default_rng(28).permutation(len(ms))
    out, lse = fd.merge(ms[perm], ls[perm], Os[perm])
    np.testing.assert_allclose(out, ref, atol=1e-13)
    # merged pieces are partials again: (m = lse, l = 1, O = out)
    oa, la = fd.merge(ms[:4], ls[:4], Os[:4])
    ob, lb = fd.merge(ms[4:], ls[4:], Os[4:])
    out2, lse2 = fd.merge(np.array([la, lb]), np.ones(2), np.array([oa, ob]))
    np.testing.assert_allclose(out2, ref, atol=1e-13)
    assert lse2 == pytest.approx(lse_ref, abs=1e-12)


def test_merge_as_printed_is_wrong():
    # The explainer's displayed merge weights each block output by
    # exp(m_i - m) * l_i; with the unnormalised block outputs of its step 1
    # and its numpy demonstration (d = 64, n = 16384, 4 blocks, seed-style
    # randn inputs) that is far from attention.  The corrected merge is not.
    d, L, scale = 64, 16384, 1 / 8
    rs = np.random.default_rng(42)
    q = rs.standard_normal(d).astype(np.float32).astype(np.float64)
    K = rs.standard_normal((L, d)).astype(np.float32).astype(np.float64)
    V = rs.standard_normal((L, d)).astype(np.float32).astype(np.float64)
    ref, _ = fd.attention_row(q, K, V, scale)
    ms, ls, Os = fd.partials(scale * (K @ q), V, fd.chunk_bounds(L, L // 4))
    w = np.exp(ms - ms.max()) * ls
    printed = (w @ Os) / w.sum()
    assert np.abs(printed - ref).max() > 1.0
    out, _ = fd.merge(ms, ls, Os)
    assert np.abs(out - ref).max() < 1e-12
    # the other consistent reading: normalised block outputs with the
    # printed weights
    normed = (w @ (Os / ls[:, None])) / w.sum()
    assert np.abs(normed - ref).max() < 1e-12
