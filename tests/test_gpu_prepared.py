"""Prepared calls (arguments checked and marshalled once) launch exactly what
the plain binding functions launch: same output bits, the tensors' current
contents at each call, and the same results when captured into a HIP graph
and replayed."""

import numpy as np
import pytest
import torch

import paged_kv_cache_scatter_amd as pkv
from workloads import make_workload

from _gpu_util import PoolCase, bits, note, to_dev, to_host

pytestmark = pytest.mark.gpu


def test_prepared_decode_matches_plain_and_follows_contents():
    wl = make_workload(3)
    pc = PoolCase(wl)
    plain = to_host(pc.decode())
    out = torch.empty_like(pc.q)
    prep = pkv.prepare_decode(pc.q, pc.k_pool, pc.v_pool, pc.tables, pc.ctx, wl.scale,
                              pc.max_ctx, out=out)
    note("prepared pkv_decode, 8 x 2048 Llama-3.2-1B shape")
    prep()
    torch.cuda.synchronize()
    assert np.array_equal(bits(to_host(out)), bits(plain))
    # new contents of the same tensors: shorter contexts and another query
    pc.ctx.copy_(torch.full_like(pc.ctx, 1000))
    pc.q.mul_(0.5)
    prep()
    torch.cuda.synchronize()
    again = pkv.decode(pc.q, pc.k_pool, pc.v_pool, pc.tables, pc.ctx, wl.scale, pc.max_ctx)
    torch.cuda.synchronize()
    assert np.array_equal(bits(to_host(out)), bits(to_host(again)))


def test_prepared_step_matches_plain_step():
    wl = make_workload(5, num_seqs=8)
    rows = np.array([r[-1] for r in wl.seq_rows], dtype=np.int64)
    outs, pools = [], []
    for prepared in (False, True):
        pc = PoolCase(wl, exclude_last=True)
        kn, vn = to_dev(wl.k_rows[rows]), to_dev(wl.v_rows[rows])
        out = torch.empty_like(pc.q)
        note(f"pkv_decode_step, prepared={prepared}")
        if prepared:
            pkv.prepare_decode_step(pc.q, kn, vn, pc.k_pool, pc.v_pool, pc.tables, pc.ctx,
                                    wl.scale, pc.max_ctx, out=out)()
        else:
            pkv.decode_step(pc.q, kn, vn, pc.k_pool, pc.v_pool, pc.tables, pc.ctx, wl.scale,
                            pc.max_ctx, out=out)
        torch.cuda.synchronize()
        outs.append(to_host(out))
        pools.append((to_host(pc.k_pool), to_host(pc.v_pool)))
    assert np.array_equal(bits(outs[0]), bits(outs[1]))
    assert np.array_equal(bits(pools[0][0]), bits(pools[1][0]))
    assert np.array_equal(bits(pools[0][1]), bits(pools[1][1]))


def test_prepared_decode_in_a_graph():
    """Captured on a side stream (the call takes the current stream at each
    call), replayed three times with eager work in between: every replay
    gives the eager result."""
    wl = make_workload(4, num_seqs=48)
    pc = PoolCase(wl)
    out = torch.empty_like(pc.q)
    ws = torch.zeros(max(16, pkv.decode_workspace_bytes(wl.num_seqs, wl.num_q_heads, pc.max_ctx,
                                                        pc.k_pool)),
                     dtype=torch.uint8, device=pc.q.device)
    prep = pkv.prepare_decode(pc.q, pc.k_pool, pc.v_pool, pc.tables, pc.ctx, wl.scale,
                              pc.max_ctx, out=out, workspace=ws)
    prep()
    torch.cuda.synchronize()
    eager = to_host(out).copy()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        prep()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        prep()
    for _ in range(3):
        out.zero_()
        pkv.decode(pc.q, pc.k_pool, pc.v_pool, pc.tables, pc.ctx, wl.scale, pc.max_ctx)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert np.array_equal(bits(to_host(out)), bits(eager))
