"""GPU parity of the stream-K cut of the decode (each KV head's sequences laid
end to end and cut into one range per workgroup, two workgroups per CU): the
planner picks it for long automatic-partition launches; every output equals
the oracle within tolerance, repeated calls give the same bits and leave the
merge counters at zero, and the piece schedule (a forced partition) agrees.

Tolerances as in test_gpu_decode: fp32 row-relative 1e-5, bf16 absolute 2e-2.
"""

import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_scatter_amd as pkv
from workloads import make_custom

from _gpu_util import PoolCase, bits, check_close, note, out_f64, to_dev, to_host

pytestmark = pytest.mark.gpu

COUNTER_AREA = 65536 * 4


def _tables(lens, bs, rng, spare=3):
    need = sum(-(-int(L) // bs) for L in lens)
    perm = (rng.permutation(need + spare) + 1).tolist()
    tabs, k = [], 0
    for L in lens:
        n = -(-int(L) // bs)
        tabs.append(perm[k:k + n])
        k += n
    return tabs, need + spare + 1


def _lens(kind, rng):
    """(lengths, dtype, Hq, Hkv, head_dim, block_size) of each mix."""
    if kind == "mixed":
        lens = rng.integers(0, 3000, size=32)
        lens[[3, 9]] = [0, 1]
        lens[17] = 12000
        return lens, "bf16", 64, 8, 128, 16
    if kind == "mostly-empty":
        lens = np.zeros(40, np.int64)
        lens[[0, 13, 39]] = [16384, 700, 5]
        return lens, "bf16", 64, 8, 128, 16
    if kind == "short-and-one-long":
        lens = rng.integers(1, 4, size=48)
        lens[30] = 9001
        return lens, "bf16", 32, 8, 128, 16
    if kind == "fp32":
        lens = rng.integers(0, 2500, size=16)
        lens[5] = 9000
        return lens, "f32", 16, 4, 128, 16
    if kind == "block-32":
        lens = rng.integers(0, 2000, size=24)
        lens[0] = 10000
        return lens, "bf16", 64, 8, 128, 32
    if kind == "1000-seqs":
        lens = rng.integers(0, 600, size=1000)
        lens[[1, 500, 999]] = 4096
        return lens, "bf16", 8, 1, 128, 16
    raise ValueError(kind)


KINDS = ["mixed", "mostly-empty", "short-and-one-long", "fp32", "block-32", "1000-seqs"]


@pytest.mark.parametrize("kind", KINDS)
def test_stream_k_matches_the_oracle(kind):
    rng = np.random.default_rng(100 + KINDS.index(kind))
    lens, dtype, hq, hkv, hd, bs = _lens(kind, rng)
    tabs, nb = _tables(lens, bs, rng)
    wl = make_custom(tabs, lens, dtype=dtype, num_q_heads=hq, num_kv_heads=hkv, head_dim=hd,
                     block_size=bs, num_blocks=nb, seed=7, name=f"stream-k-{kind}")
    pc = PoolCase(wl)
    S, mc = wl.num_seqs, pc.max_ctx
    assert pkv.decode_schedule(S, hq, mc, pc.k_pool) == "stream_k"
    part = pkv.decode_partition(S, mc, pc.k_pool)
    assert pkv.decode_schedule(S, hq, mc, pc.k_pool, part) != "stream_k"
    need = pkv.decode_workspace_bytes(S, hq, mc, pc.k_pool)
    ws = torch.zeros(max(need, 16), dtype=torch.uint8, device=pc.q.device)
    note(f"{wl.name}: {S} sequences, {int(np.sum(lens))} tokens, stream-K")
    first = pkv.decode(pc.q, pc.k_pool, pc.v_pool, pc.tables, pc.ctx, wl.scale, mc,
                       workspace=ws)
    torch.cuda.synchronize()
    first = to_host(first)
    ref = pc.ref_decode()
    err = check_close(oracle.storage_to_f64(first, dtype), ref, dtype, f"{kind}, stream-K")
    assert not to_host(ws[:COUNTER_AREA]).any(), "merge counters not back to zero"
    again = pkv.decode(pc.q, pc.k_pool, pc.v_pool, pc.tables, pc.ctx, wl.scale, mc,
                       workspace=ws)
    torch.cuda.synchronize()
    assert np.array_equal(bits(to_host(again)), bits(first)), "repeated call differs"
    assert not to_host(ws[:COUNTER_AREA]).any()
    pieces = out_f64(pc.decode(partition=part), dtype)
    check_close(pieces, ref, dtype, f"{kind}, piece schedule")
    assert not oracle.storage_to_f64(first, dtype)[np.asarray(lens) == 0].any()
    note(f"{wl.name}: max error {err:.3e}")


def test_stream_k_fused_step():
    """pkv_decode_step under the stream-K cut: the pools bit for bit against
    the oracle's write of each sequence's new token at position ctx - 1, and
    every output against the oracle's decode."""
    rng = np.random.default_rng(77)
    lens, dtype, hq, hkv, hd, bs = _lens("mixed", rng)
    tabs, nb = _tables(lens, bs, rng)
    wl = make_custom(tabs, lens, dtype=dtype, num_q_heads=hq, num_kv_heads=hkv, head_dim=hd,
                     block_size=bs, num_blocks=nb, seed=8, name="stream-k-step")
    pc = PoolCase(wl, exclude_last=True)
    S, mc = wl.num_seqs, pc.max_ctx
    assert pkv.decode_schedule(S, hq, mc, pc.k_pool) == "stream_k"
    rows = np.array([r[-1] if len(r) else 0 for r in wl.seq_rows], dtype=np.int64)
    ws = torch.zeros(max(pkv.decode_workspace_bytes(S, hq, mc, pc.k_pool), 16),
                     dtype=torch.uint8, device=pc.q.device)
    out = torch.empty_like(pc.q)
    note(f"{wl.name}: pkv_decode_step, stream-K")
    pkv.decode_step(pc.q, to_dev(wl.k_rows[rows]), to_dev(wl.v_rows[rows]), pc.k_pool,
                    pc.v_pool, pc.tables, pc.ctx, wl.scale, mc, out=out, workspace=ws)
    torch.cuda.synchronize()
    kp, vp = pc.ref_pools()
    tabs2, first, cu, srows = wl.step_segments()
    kp, vp = oracle.write(kp, vp, wl.k_rows[srows], wl.v_rows[srows],
                          oracle.slot_mapping(tabs2, first, cu, wl.block_size, wl.num_blocks))
    assert np.array_equal(bits(to_host(pc.k_pool)), bits(kp)), "k_pool differs from the oracle"
    assert np.array_equal(bits(to_host(pc.v_pool)), bits(vp)), "v_pool differs from the oracle"
    ref = oracle.decode(wl.q, kp, vp, wl.block_tables, wl.context_lens, wl.scale, dtype)
    check_close(out_f64(out, dtype), ref, dtype, "stream-K step")
    assert not to_host(ws[:COUNTER_AREA]).any()
