"""The library keeps no state between calls (besides the no-alloc buffer), so
calls on different streams with their own workspaces run side by side, and
a captured HIP graph of calls replays the same results.  Graph replays are
checked one by one against eager results, with other eager work and
synchronisations between them; every input is static and every output and
workspace allocated before the capture."""
import pytest
import torch

import long_context_decode_fd_amd as fd
import workloads as W

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _cases():
    dense = W.dense_case(4, 32, 8, 20000, 128, "bf16", 512, seed=1601, device=DEV)
    g8 = W.dense_case(8, 64, 8, 8187, 128, "bf16", 512, seed=1602, device=DEV)
    pm = W.paged_case(6, 32, 8, 128, 1, 9000, page=16, chunk=512, seed=1603, device=DEV, M=4)
    return dense, g8, pm


def _preallocated(dense, g8, pm):
    """(calls, outputs): each call writes into fixed buffers with a fixed
    workspace, allocating nothing."""
    outs, calls = [], []
    for c in (dense, g8):
        B, Hq, d = c.q.shape
        Hkv, L = c.k.shape[1], c.k.shape[2]
        o = torch.empty((B, Hq, d), dtype=torch.float32, device=DEV)
        l = torch.empty((B, Hq), dtype=torch.float32, device=DEV)
        ws = torch.empty(fd.workspace_bytes("fd_decode_attn", B=B, Hq=Hq, Hkv=Hkv, L=L, d=d,
                                            chunk=512), dtype=torch.uint8, device=DEV)
        calls.append(lambda c=c, o=o, l=l, ws=ws: fd.decode_attn(c.q, c.k, c.v, chunk=512, out=o,
                                                                 lse=l, workspace=ws))
        outs += [o, l]
    B, M, Hq, d = pm.q.shape
    maxl = int(max(pm.meta["lens"]))
    o = torch.empty((B, M, Hq, d), dtype=torch.float32, device=DEV)
    l = torch.empty((B, M, Hq), dtype=torch.float32, device=DEV)
    ws = torch.empty(fd.workspace_bytes("fd_decode_attn_multi_paged", B=B, M=M, Hq=Hq, Hkv=8, d=d,
                                        page=pm.page, max_pages=pm.block_table.shape[1],
                                        max_seq_len=maxl, chunk=512),
                     dtype=torch.uint8, device=DEV)
    calls.append(lambda: fd.decode_attn_multi_paged(pm.q, pm.k_pool, pm.v_pool, pm.block_table,
                                                    pm.seq_lens, maxl, chunk=512, out=o, lse=l,
                                                    workspace=ws))
    outs += [o, l]
    # the no-alloc entry point: its library-owned buffer, no workspace
    od = torch.empty_like(outs[0])
    ld = torch.empty_like(outs[1])
    calls.append(lambda: fd.decode_attn_noalloc(dense.q, dense.k, dense.v, chunk=512, out=od,
                                                lse=ld))
    outs += [od, ld]
    return calls, outs


def test_calls_on_two_streams_match_eager():
    dense, g8, pm = _cases()
    calls, outs = _preallocated(dense, g8, pm)
    for call in calls:
        call()
    torch.cuda.synchronize()
    ref = [t.clone() for t in outs]
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    for rep in range(4):
        for t in outs:
            t.fill_(float("nan"))
        torch.cuda.synchronize()
        with torch.cuda.stream(s1):
            calls[0]()
            calls[2]()
        with torch.cuda.stream(s2):
            calls[1]()
        torch.cuda.synchronize()
        for i in range(6):
            assert torch.equal(outs[i], ref[i]), (rep, i)


def _more_calls(calls, outs):
    """Fixed maximum (with its flags) and FFD on fixed buffers."""
    c = W.dense_case(4, 32, 8, 16384, 128, "bf16", 512, seed=1604, device=DEV)
    o = torch.empty((4, 32, 128), dtype=torch.float32, device=DEV)
    l = torch.empty((4, 32), dtype=torch.float32, device=DEV)
    f = torch.empty((4, 32, 32), dtype=torch.uint8, device=DEV)
    ws = torch.empty(fd.workspace_bytes("fd_decode_attn_unified_max", B=4, Hq=32, Hkv=8, L=16384,
                                        d=128, chunk=512), dtype=torch.uint8, device=DEV)
    calls.append(lambda: fd.decode_attn_unified_max(c.q, c.k, c.v, 3.0, chunk=512, margin_hi=0.5,
                                                    margin_lo=0.5, out=o, lse=l, flags=f,
                                                    workspace=ws))
    outs += [o, l, f]
    fc = W.ffd_case(2, 32, 8, 8192, 128, seed=1605, device=DEV)
    pk = fd.ffd_pack(fc.k)
    o2 = torch.empty((2, 32, 128), dtype=torch.float32, device=DEV)
    l2 = torch.empty((2, 32), dtype=torch.float32, device=DEV)
    ws2 = torch.empty(fd.workspace_bytes("fd_ffd_sparse_decode", B=2, Hq=32, Hkv=8, L=8192,
                                         d=128, chunk=1024), dtype=torch.uint8, device=DEV)
    calls.append(lambda: fd.ffd_sparse_decode(fc.q, pk, fc.v, 5.0, chunk=1024, out=o2, lse=l2,
                                              workspace=ws2))
    outs += [o2, l2]
    return c, fc, pk


def test_graph_replays_match_eager():
    dense, g8, pm = _cases()
    calls, outs = _preallocated(dense, g8, pm)
    keep = _more_calls(calls, outs)   # noqa: F841 (inputs stay alive for the replays)
    for call in calls:
        call()
    torch.cuda.synchronize()
    ref = [t.clone() for t in outs]
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for call in calls:
            call()
    for rep in range(3):
        for t in outs:
            t.fill_(float("nan") if t.is_floating_point() else 255)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for i, (t, r) in enumerate(zip(outs, ref)):
            assert torch.equal(t, r), (rep, i)
        # eager work between replays: the same calls, then something else
        for call in calls:
            call()
        torch.cuda.synchronize()
        x = torch.randn(1 << 20, device=DEV)
        assert torch.isfinite(x.sum())
