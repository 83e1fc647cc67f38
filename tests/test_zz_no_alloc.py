"""pkv_decode_step_noalloc (no workspace, nothing allocated) against
pkv_decode_step with a workspace, through the C ABI: two calls in a row on
one GPU, the second with a smaller input, each bit-identical to the
workspace form (same kernels, same plan) and within the oracle's tolerance."""

import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_scatter_amd as pkv
from workloads import make_workload

from _gpu_util import PoolCase, bits, check_close, note, to_dev, to_host

pytestmark = pytest.mark.gpu


def _rows(wl):
    return np.array([r[-1] if len(r) else 0 for r in wl.seq_rows], dtype=np.int64)


def _step_pair(wl):
    """(out, k_pool, v_pool) of the workspace form and of the no-alloc form,
    each on its own copy of the bulk-filled pools, and the oracle's output."""
    rows = _rows(wl)
    kn, vn = to_dev(wl.k_rows[rows]), to_dev(wl.v_rows[rows])
    res = []
    for form in ("workspace", "noalloc"):
        pc = PoolCase(wl, exclude_last=True)
        need = pkv.decode_workspace_bytes(wl.num_seqs, wl.num_q_heads, pc.max_ctx, pc.k_pool)
        out = torch.full_like(pc.q, float("nan"))
        note(f"{wl.name}: pkv_decode_step ({form}), {wl.num_seqs} sequences, "
             f"{need} bytes of workspace or scratch")
        assert need <= pkv.NOALLOC_SCRATCH_BYTES
        if form == "workspace":
            pkv.decode_step(pc.q, kn, vn, pc.k_pool, pc.v_pool, pc.tables, pc.ctx, wl.scale,
                            pc.max_ctx, out=out)
        else:
            pkv.decode_step_noalloc(pc.q, kn, vn, pc.k_pool, pc.v_pool, pc.tables, pc.ctx,
                                    wl.scale, pc.max_ctx, out=out)
        torch.cuda.synchronize()
        res.append((to_host(out), to_host(pc.k_pool), to_host(pc.v_pool)))
    kp, vp = pc.ref_pools()
    tabs, first, cu, srows = wl.step_segments()
    kp, vp = oracle.write(kp, vp, wl.k_rows[srows], wl.v_rows[srows],
                          oracle.slot_mapping(tabs, first, cu, wl.block_size, wl.num_blocks))
    ref = oracle.decode(wl.q, kp, vp, wl.block_tables, wl.context_lens, wl.scale, wl.dtype)
    return res, ref


@pytest.mark.parametrize("cfg,sizes", [(5, (64, 9)), (4, (192, 40))])
def test_noalloc_step_matches_workspace_step(cfg, sizes):
    """The LLaMA-2-70B layer splits both calls (64 then 9 sequences); the
    Llama-3.2-1B shape runs 192 sequences unsplit (no scratch needed), then 40
    sequences split."""
    for S in sizes:
        wl = make_workload(cfg, num_seqs=S)
        ((o_ws, k_ws, v_ws), (o_na, k_na, v_na)), ref = _step_pair(wl)
        assert np.array_equal(bits(o_na), bits(o_ws)), "outputs differ from pkv_decode_step"
        assert np.array_equal(bits(k_na), bits(k_ws)), "k_pool differs"
        assert np.array_equal(bits(v_na), bits(v_ws)), "v_pool differs"
        err = check_close(oracle.storage_to_f64(o_na, wl.dtype), ref, wl.dtype, wl.name)
        note(f"{wl.name}: {S} sequences bit-identical to the workspace form, "
             f"max error {err:.3e}")


def test_noalloc_step_replays_from_a_captured_graph():
    """The callers the no-alloc entry point is for include code under HIP graph
    capture: after one eager call (which locates the scratch array on this
    device), the step is captured and replayed, with eager calls on other
    inputs in between, and every replay reproduces the eager bits."""
    wl = make_workload(5, num_seqs=16)
    rows = _rows(wl)
    kn, vn = to_dev(wl.k_rows[rows]), to_dev(wl.v_rows[rows])
    pc = PoolCase(wl, exclude_last=True)

    def step(out):
        return pkv.decode_step_noalloc(pc.q, kn, vn, pc.k_pool, pc.v_pool, pc.tables, pc.ctx,
                                       wl.scale, pc.max_ctx, out=out)

    eager = torch.full_like(pc.q, float("nan"))
    step(eager)
    torch.cuda.synchronize()
    other = make_workload(5, num_seqs=5, seed=77)     # a different call sharing the scratch
    po = PoolCase(other, exclude_last=True)
    orows = _rows(other)
    okn, ovn = to_dev(other.k_rows[orows]), to_dev(other.v_rows[orows])
    out_g = torch.full_like(pc.q, float("nan"))
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(side):
        note(f"{wl.name}: capturing pkv_decode_step_noalloc")
        with torch.cuda.graph(g):
            step(out_g)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    for r in range(3):
        out_g.fill_(float("nan"))
        note(f"{wl.name}: replay {r}")
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(bits(to_host(out_g)), bits(to_host(eager))), f"replay {r}"
        o2 = torch.empty_like(po.q)
        pkv.decode_step_noalloc(po.q, okn, ovn, po.k_pool, po.v_pool, po.tables, po.ctx,
                                other.scale, po.max_ctx, out=o2)
        torch.cuda.synchronize()
