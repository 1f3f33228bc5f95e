"""Pins of the cache-append oracle (CPU).

The placement is checked through the paged oracle's own gather (an
independent function of the block-table addressing), and the composition
append -> attention against attention over the concatenated cache.
"""
import numpy as np

from oracle import append as oap
from oracle import flash_decoding as ofd
from oracle import paged as opg


def _pool_case(seed=0, B=3, Hkv=2, page=8, d=16, lens=(5, 16, 0), max_pages=4):
    rs = np.random.default_rng(seed)
    n = [(L + page - 1) // page for L in lens]
    P = 12
    table = np.full((B, max_pages), -1, dtype=np.int32)
    free = list(rs.permutation(P))
    for b in range(B):
        for i in range(max_pages):          # every sequence owns all its table slots
            table[b, i] = free.pop()
    pool = rs.standard_normal((P, Hkv, page, d))
    return pool, table, np.asarray(lens), rs


def test_paged_append_lands_where_the_gather_reads():
    pool, table, lens, rs = _pool_case()
    B, Hkv, d = 3, 2, 16
    M = 3
    new = rs.standard_normal((B, Hkv, M, d))
    out = oap.append_paged(pool, table, lens, new)
    for b in range(B):
        L = int(lens[b])
        before = opg.gather_sequence(pool, table[b], L, 8)
        after = opg.gather_sequence(out, table[b], L + M, 8)
        assert np.array_equal(after[:, :L], before)          # old rows untouched
        assert np.array_equal(after[:, L:], new[b])           # new rows at L..L+M-1
    # rows the appends did not target are unchanged
    touched = set()
    for b in range(B):
        for m in range(M):
            p = int(lens[b]) + m
            touched.add((int(table[b, p // 8]), p % 8))
    for pg in range(pool.shape[0]):
        for s in range(8):
            if (pg, s) not in touched:
                assert np.array_equal(out[pg, :, s], pool[pg, :, s])


def test_paged_append_skips_positions_without_a_page():
    pool, table, lens, rs = _pool_case()
    new = rs.standard_normal((3, 2, 2, 16))
    t2 = table.copy()
    t2[0, 0] = -1                  # sequence 0 writes into page slot 0: no page
    pos = np.array([3, 31, -5])    # seq 1 runs past its 4-page row; seq 2 starts below 0
    out = oap.append_paged(pool, t2, pos, new)
    assert np.array_equal(out[t2[1, 3], :, 7], new[1, :, 0])   # position 31 fits
    # seq 0: page slot 0 has no page; seq 1: position 32 is past its row;
    # seq 2: positions -5 and -4 are below 0 -- only position 31 is written
    diff = np.argwhere(np.any(out != pool, axis=(1, 3)))
    assert {tuple(x) for x in diff} == {(int(t2[1, 3]), 7)}


def test_contiguous_append_then_attention_equals_concatenation():
    rs = np.random.default_rng(3)
    B, Hkv, G, L_cap, d, t, M = 2, 2, 2, 12, 16, 7, 3
    k = rs.standard_normal((B, Hkv, L_cap, d))
    v = rs.standard_normal((B, Hkv, L_cap, d))
    kn = rs.standard_normal((B, Hkv, M, d))
    vn = rs.standard_normal((B, Hkv, M, d))
    k2 = oap.append_contiguous(k, kn, t)
    v2 = oap.append_contiguous(v, vn, t)
    assert np.array_equal(k2[:, :, :t], k[:, :, :t]) and np.array_equal(k2[:, :, t + M:], k[:, :, t + M:])
    q = rs.standard_normal((B, Hkv * G, d))
    for b in range(B):
        for h in range(Hkv * G):
            kc = np.concatenate([k[b, h // G, :t], kn[b, h // G]])
            vc = np.concatenate([v[b, h // G, :t], vn[b, h // G]])
            o1, l1 = ofd.attention_row(q[b, h], k2[b, h // G, :t + M], v2[b, h // G, :t + M], 0.25)
            o2, l2 = ofd.attention_row(q[b, h], kc, vc, 0.25)
            assert np.array_equal(o1, o2) and l1 == l2
