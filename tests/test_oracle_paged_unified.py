"""Pins for the paged and fixed-maximum oracles (CPU only)."""
import math

import numpy as np
import pytest

from oracle import flash_decoding as fd
from oracle import paged, unified


def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


def _scatter_into_pool(k, lens, page, seed):
    """Test-side paging (independent of the oracle's gather): put sequence b's
    pages at a random permutation of pool slots, return pool and table."""
    B, Hkv, Lmax, d = k.shape
    n = [(L + page - 1) // page for L in lens]
    perm = np.random.default_rng(seed).permutation(sum(n))
    pool = np.zeros((sum(n), Hkv, page, d))
    table = np.full((B, max(n)), -1, dtype=np.int32)
    off = 0
    for b, L in enumerate(lens):
        for i in range(n[b]):
            pid = perm[off + i]
            table[b, i] = pid
            lo, hi = i * page, min((i + 1) * page, L)
            pool[pid, :, :hi - lo] = k[b, :, lo:hi]
        off += n[b]
    return pool, table


def test_paged_equals_dense_on_gathered_copy():
    B, Hq, Hkv, d, page = 3, 8, 2, 32, 16
    lens = [37, 16, 130]
    q = _rand((B, Hq, d), 1)
    k = _rand((B, Hkv, max(lens), d), 2)
    v = _rand((B, Hkv, max(lens), d), 3)
    kp, table = _scatter_into_pool(k, lens, page, 4)
    vp, _ = _scatter_into_pool(v, lens, page, 4)
    out, lse = paged.paged_attention(q, kp, vp, table, lens, page, 0.2)
    for b, L in enumerate(lens):
        ref, lref = fd.dense_attention(q[b:b + 1], k[b:b + 1, :, :L],
                                       v[b:b + 1, :, :L], 0.2)
        np.testing.assert_allclose(out[b], ref[0], atol=1e-13)
        np.testing.assert_allclose(lse[b], lref[0], atol=1e-13)
    # relabelling the pool's pages changes nothing
    relabel = np.random.default_rng(5).permutation(kp.shape[0])
    inv = np.argsort(relabel)
    t2 = np.where(table >= 0, inv[np.maximum(table, 0)], -1)
    out2, _ = paged.paged_attention(q, kp[relabel], vp[relabel], t2, lens, page, 0.2)
    np.testing.assert_allclose(out2, out, atol=1e-15)


def test_paged_empty_sequence():
    q = _rand((1, 2, 8), 6)
    pool = np.zeros((1, 1, 16, 8))
    out, lse = paged.paged_attention(q, pool, pool, np.full((1, 1), -1), [0], 16, 1.0)
    assert np.all(out == 0) and np.all(lse == -np.inf)


def test_flags_by_brute_force():
    B, Hq, Hkv, L, d, chunk = 1, 4, 2, 200, 16, 64
    q, k = _rand((B, Hq, d), 7), _rand((B, Hkv, L, d), 8)
    flags = unified.chunk_flags(q, k, 0.25, 1.0, 0.5, 2.0, chunk)
    for h in range(Hq):
        for c, (a, b) in enumerate(fd.chunk_bounds(L, chunk)):
            mx = max(0.25 * float(k[0, h // 2, j] @ q[0, h]) for j in range(a, b))
            assert flags[0, h, c] == (mx > 1.5 or mx < -1.0)


@pytest.mark.parametrize("phi", [-3.0, 0.0, 2.5, 6.0])
def test_fixed_max_without_flags_is_exact(phi):
    d, L, scale = 64, 2048, 1 / 8
    q, K, V = _rand(d, 9), _rand((L, d), 10), _rand((L, d), 11)
    bounds = fd.chunk_bounds(L, 256)
    s = scale * (K @ q)
    assert not unified.chunk_flags_row(s, bounds, phi, 10.0, 40.0).any()
    ref, lref = fd.attention_row(q, K, V, scale)
    out, lse = unified.fixed_max_merge(*unified.fixed_max_partials(s, V, phi, bounds), phi)
    np.testing.assert_allclose(out, ref, atol=1e-12)
    assert lse == pytest.approx(lref, abs=1e-12)


def test_overflow_needs_fallback():
    # One key planted 100 above phi: exp(100) is inf in float32, so the
    # fixed-maximum sums overflow without the fallback; the replay with the
    # fallback equals attention and flags exactly the planted chunk.
    d, L, scale, phi = 64, 1024, 1 / 8, 3.0
    q, K, V = _rand(d, 12), _rand((L, d), 13), _rand((L, d), 14)
    j = 700
    K[j] = (phi + 100.0) / scale * q / (q @ q)
    s = scale * (K @ q)
    assert s[j] == pytest.approx(phi + 100.0)
    p32 = np.exp((s - phi).astype(np.float32))
    assert np.isinf(p32.sum(dtype=np.float32))
    bounds = fd.chunk_bounds(L, 128)
    out, lse, flags = unified.unified_row(q, K, V, scale, phi, 10.0, 40.0, bounds)
    assert flags.tolist() == [c == j // 128 for c in range(8)]
    ref, lref = fd.attention_row(q, K, V, scale)
    np.testing.assert_allclose(out, ref, atol=1e-12)
    assert lse == pytest.approx(lref, abs=1e-12)


def test_low_side_flag_and_replay():
    # Every score far below phi: all chunks are flagged low, and the replay
    # (which then recomputes everything) still equals attention.
    d, L, scale = 32, 500, 0.2
    q, K, V = _rand(d, 15), _rand((L, d), 16), _rand((L, d), 17)
    bounds = fd.chunk_bounds(L, 100)
    out, lse, flags = unified.unified_row(q, K, V, scale, 200.0, 10.0, 40.0, bounds)
    assert flags.all()
    ref, lref = fd.attention_row(q, K, V, scale)
    np.testing.assert_allclose(out, ref, atol=1e-12)
    assert lse == pytest.approx(lref, abs=1e-12)


def test_unified_attention_target_is_dense():
    B, Hq, Hkv, L, d = 2, 4, 1, 300, 16
    q, k, v = _rand((B, Hq, d), 18), _rand((B, Hkv, L, d), 19), _rand((B, Hkv, L, d), 20)
    out, lse, flags = unified.unified_attention(q, k, v, 0.25, 0.5, 1.0, 40.0, 64)
    ref, lref = fd.dense_attention(q, k, v, 0.25)
    assert np.array_equal(out, ref) and np.array_equal(lse, lref)
    assert flags.shape == (B, Hq, math.ceil(L / 64))
    # margins this tight flag some chunks; the replay still matches
    assert flags.any()
    for b in range(B):
        for h in range(Hq):
            o, l, f = unified.unified_row(q[b, h], k[b, 0], v[b, 0], 0.25, 0.5, 1.0,
                                          40.0, fd.chunk_bounds(L, 64))
            np.testing.assert_allclose(o, ref[b, h], atol=1e-12)
            assert np.array_equal(f, flags[b, h].astype(bool))


def test_paged_multi_row_matches_contiguous_multi_row():
    """Several new tokens over a scattered page pool equal the contiguous
    multi-row oracle on each sequence's own cache (pinned on its own), and
    relabelling the pool's pages changes nothing."""
    from oracle import multi_row
    B, M, Hq, Hkv, d, page = 3, 4, 6, 2, 16, 8
    lens = [37, 9, 130]
    q = _rand((B, M, Hq, d), 11)
    k = _rand((B, Hkv, max(lens), d), 12)
    v = _rand((B, Hkv, max(lens), d), 13)
    kp, table = _scatter_into_pool(k, lens, page, 4)
    vp, _ = _scatter_into_pool(v, lens, page, 4)
    out, lse = paged.paged_multi_row_attention(q, kp, vp, table, lens, page, 0.3)
    for b, L in enumerate(lens):
        ref, lref = multi_row.multi_row_attention(q[b:b + 1], k[b:b + 1, :, :L],
                                                  v[b:b + 1, :, :L], 0.3)
        np.testing.assert_allclose(out[b], ref[0], atol=1e-13)
        np.testing.assert_allclose(lse[b], lref[0], atol=1e-13)
    relabel = np.random.default_rng(6).permutation(kp.shape[0])
    inv = np.argsort(relabel)
    t2 = np.where(table >= 0, inv[np.maximum(table, 0)], -1)
    out2, _ = paged.paged_multi_row_attention(q, kp[relabel], vp[relabel], t2, lens, page, 0.3)
    np.testing.assert_allclose(out2, out, atol=1e-15)


def test_paged_multi_row_one_token_is_paged_decode():
    B, Hq, Hkv, d, page = 2, 4, 1, 8, 16
    lens = [50, 0]
    q = _rand((B, 1, Hq, d), 14)
    k, v = _rand((B, Hkv, 50, d), 15), _rand((B, Hkv, 50, d), 16)
    kp, table = _scatter_into_pool(k, lens, page, 2)
    vp, _ = _scatter_into_pool(v, lens, page, 2)
    out, lse = paged.paged_multi_row_attention(q, kp, vp, table, lens, page, 0.5)
    ref, lref = paged.paged_attention(q[:, 0], kp, vp, table, lens, page, 0.5)
    np.testing.assert_array_equal(out[:, 0], ref)
    np.testing.assert_array_equal(lse[:, 0], lref)


def test_paged_multi_row_short_sequences_by_brute_force():
    """Sequences shorter than the token count: token r sees the first
    L - M + r + 1 positions, none when that is not positive (out 0, lse
    -inf); the rest by an explicit softmax sum over the visible keys."""
    M, Hq, Hkv, d, page = 5, 2, 1, 4, 8
    lens = [3, 5, 0]
    B = len(lens)
    q = _rand((B, M, Hq, d), 17)
    k, v = _rand((B, Hkv, 8, d), 18), _rand((B, Hkv, 8, d), 19)
    kp, table = _scatter_into_pool(k, lens, page, 1)
    vp, _ = _scatter_into_pool(v, lens, page, 1)
    out, lse = paged.paged_multi_row_attention(q, kp, vp, table, lens, page, 0.7)
    for b, L in enumerate(lens):
        for r in range(M):
            n = L - M + r + 1
            for h in range(Hq):
                if n <= 0:
                    assert np.all(out[b, r, h] == 0) and lse[b, r, h] == -np.inf
                    continue
                s = [0.7 * sum(k[b, 0, j, i] * q[b, r, h, i] for i in range(d)) for j in range(n)]
                e = [math.exp(x) for x in s]
                want = [sum(e[j] * v[b, 0, j, i] for j in range(n)) / sum(e) for i in range(d)]
                np.testing.assert_allclose(out[b, r, h], want, atol=1e-12)
                assert abs(lse[b, r, h] - math.log(sum(e))) < 1e-12
