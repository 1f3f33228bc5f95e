"""Run-to-run bitwise determinism of every kernel that exchanges data across
lanes, waves or workgroups (LDS tiles behind barriers, cross-lane swaps,
split-column merges).  A race on shared memory shows up as a result that
changes between two identical calls; every summation order here is fixed, so
the bits must not change.  Each entry point runs three times on the same
inputs with other work in between (the dense headline shape), so a race that
depends on timing gets several chances to show."""
import numpy as np
import pytest
import torch

import long_context_decode_fd_amd as fd
import workloads as W
from oracle import ffd as offd
from tests.helpers import banner, f64, packed_to_device

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _filler():
    # unrelated work on the same stream between the repeats
    c = W.dense_case(2, 32, 8, 8192, 128, "bf16", 512, seed=900, device=DEV)
    return lambda: fd.decode_attn(c.q, c.k, c.v, chunk=512)


def _same_every_time(run, n=3):
    other = _filler()
    first = [t.clone() for t in run() if t is not None]
    for _ in range(n - 1):
        other()
        again = [t for t in run() if t is not None]
        torch.cuda.synchronize()
        for a, b in zip(first, again):
            assert torch.equal(a, b)


@pytest.mark.parametrize("d,G,chunk", [(128, 4, 1024), (128, 8, 512), (128, 4, 96),
                                       (64, 1, 256), (64, 2, 2048)])
def test_ffd_repeatable(d, G, chunk):
    """The FFD kernel: scan scores, candidate masks and the compacted list in
    LDS behind barriers; the matrix-core form (d 128, G 4/8) and the
    dot-product form."""
    banner(f"determinism ffd d={d} G={G} chunk={chunk}")
    Hq = 8 * G if G < 8 else 16
    c = W.ffd_case(2, Hq, Hq // G, 5000, d, chunk=chunk, seed=910 + G, device=DEV)
    pk = packed_to_device(offd.pack_keys(f64(c.k).astype(np.float32)), DEV)
    for delta in (0.5, 5.0):
        _same_every_time(lambda: fd.ffd_sparse_decode(c.q, pk, c.v, delta, c.n_sink, c.n_local,
                                                      chunk=chunk, want_mask=True,
                                                      want_pseudo_max=True))


@pytest.mark.parametrize("M", [2, 4, 8])
def test_multi_repeatable(M):
    """Multi-row kernels: one query tile per wave (M 2, 4: per-wave LDS
    tiles) and the wave pair (M 8: tiles shared through LDS behind barriers),
    with the transposing read."""
    banner(f"determinism multi M={M}")
    c = W.multi_case(2, M, 32, 8, 6000, 128, seed=920 + M, device=DEV)
    _same_every_time(lambda: fd.decode_attn_multi(c.q, c.k, c.v, chunk=512))
    _same_every_time(lambda: fd.decode_attn_multi(c.q, c.k, c.v, chunk=48))


@pytest.mark.parametrize("M", [4, 8])
def test_multi_many_units_repeatable(M):
    """More (sequence, kv-head) rows than wave slots (256 sequences x 32
    kv-heads): each wave, or wave pair, takes 8 units in a row, so partials
    are held, staged through LDS and written between units, and the next
    unit's query and keys are requested across the boundary."""
    banner(f"determinism multi many units M={M}")
    c = W.multi_case(256, M, 128, 32, 100, 128, seed=960 + M, device=DEV)
    _same_every_time(lambda: fd.decode_attn_multi(c.q, c.k, c.v, chunk=128))


def test_paged_repeatable():
    banner("determinism paged")
    lens = [0, 17, 1000, 5000, 16 * 300 + 3, 64]
    c = W.paged_case(len(lens), 32, 8, 128, 0, max(lens), page=16, chunk=256, seed=930,
                     device=DEV, lens=lens)
    _same_every_time(lambda: fd.decode_attn_paged(c.q, c.k_pool, c.v_pool, c.block_table,
                                                  c.seq_lens, max(lens), chunk=256))


def test_fixed_max_repeatable():
    """Fixed maximum with tight margins: some chunks switch to the exact path
    in flight, others do not."""
    banner("determinism fixed max")
    c = W.dense_case(2, 32, 8, 20000, 128, "bf16", 256, seed=940, device=DEV)
    _same_every_time(lambda: fd.decode_attn_unified_max(c.q, c.k, c.v, 1.0, chunk=256,
                                                        margin_hi=1.0, margin_lo=1.5))


@pytest.mark.parametrize("nc", [30, 64, 100, 200, 300])
def test_split_column_merges_repeatable(nc):
    """Every merge tier: rows of up to 256 chunks on single wavefronts (the
    columns over 1, 2, 4 or 8 of them, several chunks' (m, l) per lane past
    64), longer rows on 4-wave workgroups that reduce through LDS behind
    barriers."""
    banner(f"determinism merge nc={nc}")
    c = W.dense_case(2, 16, 4, 16 * (nc - 1) + 5, 128, "bf16", 16, seed=950 + nc, device=DEV)
    _same_every_time(lambda: fd.decode_attn(c.q, c.k, c.v, chunk=16))
