"""GPU parity of the fused decode step (write of the new token + decode) against
the separate slot mapping + write + decode, and against the oracle."""

import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_scatter_amd as pkv
from workloads import make_custom, make_workload

from _gpu_util import PoolCase, bits, check_close, note, out_f64, to_dev, to_host

pytestmark = pytest.mark.gpu


def _new_rows(wl):
    """Row index of k_new / v_new [S, Hkv, hd]: each sequence's last position
    (any row for an empty sequence; it is neither written nor read)."""
    return np.array([r[-1] if len(r) else 0 for r in wl.seq_rows], dtype=np.int64)


def _separate(pc, partition):
    wl = pc.wl
    tabs, first, cu, rows = wl.step_segments()
    n = int(cu[-1])
    slots = pkv.slot_mapping(to_dev(tabs), to_dev(first), to_dev(cu), n, wl.block_size,
                             wl.num_blocks)
    pkv.write(to_dev(wl.k_rows[rows]), to_dev(wl.v_rows[rows]), slots, pc.k_pool, pc.v_pool)
    return pc.decode(partition=partition)


def _ref_step(pc):
    """Oracle: the bulk fill, then the step's write, then attention."""
    wl = pc.wl
    kp, vp = pc.ref_pools()
    tabs, first, cu, rows = wl.step_segments()
    kp, vp = oracle.write(kp, vp, wl.k_rows[rows], wl.v_rows[rows],
                          oracle.slot_mapping(tabs, first, cu, wl.block_size, wl.num_blocks))
    return oracle.decode(wl.q, kp, vp, wl.block_tables, wl.context_lens, wl.scale, wl.dtype)


def _fused(pc, rows, partition, phase="both"):
    wl = pc.wl
    note(f"{wl.name}: pkv_decode_step partition={partition or 'auto'} phase={phase}")
    if phase == "both":
        out = pkv.decode_step(pc.q, to_dev(wl.k_rows[rows]), to_dev(wl.v_rows[rows]), pc.k_pool,
                              pc.v_pool, pc.tables, pc.ctx, wl.scale, pc.max_ctx,
                              partition=partition)
    else:
        ws = torch.zeros(max(16, pkv.decode_workspace_bytes(wl.num_seqs, wl.num_q_heads,
                                                            pc.max_ctx, pc.k_pool, partition)),
                         dtype=torch.uint8, device=pc.q.device)
        out = torch.empty_like(pc.q)
        kn, vn = to_dev(wl.k_rows[rows]), to_dev(wl.v_rows[rows])
        pkv.decode_step(pc.q, kn, vn, pc.k_pool, pc.v_pool, pc.tables, pc.ctx, wl.scale,
                        pc.max_ctx, out=out, partition=partition, workspace=ws, phase="partials")
        pkv.decode(pc.q, pc.k_pool, pc.v_pool, pc.tables, pc.ctx, wl.scale, pc.max_ctx, out=out,
                   partition=partition, workspace=ws, phase="reduce")
    torch.cuda.synchronize()
    return out


def _compare(wl, partition=0):
    rows = _new_rows(wl)
    a = PoolCase(wl, exclude_last=True)
    b = PoolCase(wl, exclude_last=True)
    out_sep = to_host(_separate(a, partition))
    out_fused = to_host(_fused(b, rows, partition))
    assert np.array_equal(bits(out_fused), bits(out_sep)), "fused step differs from write + decode"
    assert np.array_equal(bits(to_host(b.k_pool)), bits(to_host(a.k_pool)))
    assert np.array_equal(bits(to_host(b.v_pool)), bits(to_host(a.v_pool)))
    return b, out_fused


@pytest.mark.parametrize("cfg,S", [(1, None), (3, 2), (4, 32), (5, 8)])
def test_step_equals_write_then_decode(cfg, S):
    wl = make_workload(cfg, num_seqs=S)
    b, out = _compare(wl)
    check_close(oracle.storage_to_f64(out, wl.dtype), _ref_step(b), wl.dtype, f"config {cfg}")


@pytest.mark.parametrize("bs", [1, 8, 32])
def test_step_block_sizes(bs):
    lens = [1, 9, 70, 129]
    need = sum(-(-L // bs) for L in lens)
    rng = np.random.default_rng(bs + 40)
    perm = (rng.permutation(need) + 1).tolist()
    tabs, k = [], 0
    for L in lens:
        n = -(-L // bs)
        tabs.append(perm[k:k + n])
        k += n
    wl = make_custom(tabs, lens, dtype="bf16", num_q_heads=8, num_kv_heads=2, head_dim=128,
                     block_size=bs, num_blocks=need + 1, seed=bs)
    b, out = _compare(wl)
    check_close(oracle.storage_to_f64(out, "bf16"), _ref_step(b), "bf16", f"bs={bs}")


def test_step_partition_and_phases():
    """Multi-split sequences (the new token in the last split) and the
    partials + reduce phases give the same bits."""
    wl = make_workload(5, num_seqs=6)
    rows = _new_rows(wl)
    outs = []
    for part, phase in ((256, "both"), (256, "partials"), (0, "both")):
        pc = PoolCase(wl, exclude_last=True)
        outs.append(to_host(_fused(pc, rows, part, phase)))
    assert np.array_equal(bits(outs[0]), bits(outs[1]))
    check_close(oracle.storage_to_f64(outs[2], "bf16"), _ref_step(pc), "bf16")
    check_close(oracle.storage_to_f64(outs[0], "bf16"), _ref_step(pc), "bf16")


def test_step_tile_aligned_lengths():
    """Lengths that end exactly on a tile / block / split boundary, and an
    empty sequence (no write, zero output)."""
    lens = [16, 32, 256, 512, 0, 1]
    tabs = []
    k = 1
    for L in lens:
        n = -(-L // 16)
        tabs.append(list(range(k, k + n)))
        k += n
    wl = make_custom(tabs, lens, dtype="bf16", num_q_heads=16, num_kv_heads=2, head_dim=128,
                     block_size=16, num_blocks=k + 1, seed=77)
    for part in (0, 256):
        b, out = _compare(wl, part)
        assert not out[4].any()
        check_close(oracle.storage_to_f64(out, "bf16"), _ref_step(b), "bf16")


def test_step_piece_boundaries():
    """The fused step on the piece schedule: the new token is written by the
    piece that ends the context, be it a full piece, a full piece with a short
    rest joined to it, or a tail piece."""
    lens = [0, 1, 100, 200, 255, 256, 257, 319, 320, 351, 352, 383, 384, 385, 511, 512, 513,
            1088, 1224, 2047, 2048]
    need = sum(-(-L // 16) for L in lens)
    perm = (np.random.default_rng(91).permutation(need) + 1).tolist()
    tabs, k = [], 0
    for L in lens:
        n = -(-L // 16)
        tabs.append(perm[k:k + n])
        k += n
    wl = make_custom(tabs, lens, dtype="bf16", num_q_heads=16, num_kv_heads=2, head_dim=128,
                     block_size=16, num_blocks=need + 1, seed=92)
    for part in (256, 64):
        b, out = _compare(wl, part)
        assert not out[0].any()
        check_close(oracle.storage_to_f64(out, "bf16"), _ref_step(b), "bf16", f"partition {part}")


def test_step_invalid_block_for_new_token():
    """The new token's table entry is out of range: nothing is written and the
    token is left out, as with a skipped slot."""
    wl = make_custom([[1, 2, 3], [4, 5]], [40, 30], num_q_heads=8, num_kv_heads=2, head_dim=64,
                     block_size=16, num_blocks=6, seed=81)
    rows = _new_rows(wl)
    pc = PoolCase(wl, exclude_last=True)
    bad = wl.block_tables.copy()
    bad[0, 2] = 1 << 20          # position 39 lives in table entry 2
    tables = to_dev(bad)
    before = to_host(pc.k_pool).copy()
    note("decode step with the new token's block out of range")
    out = pkv.decode_step(pc.q, to_dev(wl.k_rows[rows]), to_dev(wl.v_rows[rows]), pc.k_pool,
                          pc.v_pool, tables, pc.ctx, wl.scale, pc.max_ctx)
    torch.cuda.synchronize()
    after = to_host(pc.k_pool)
    # sequence 1's new token (position 29, block 5) is written; nothing else changes
    kp, vp = pc.ref_pools()
    slot1 = 5 * 16 + 29 % 16
    flat_a = after.reshape(-1, wl.num_kv_heads, wl.head_dim)
    flat_b = before.reshape(-1, wl.num_kv_heads, wl.head_dim)
    changed = np.nonzero((bits(flat_a) != bits(flat_b)).any(axis=(1, 2)))[0].tolist()
    assert changed == [slot1], changed
    assert np.array_equal(bits(flat_a[slot1]), bits(wl.k_rows[rows[1]]))
    # attention: the written pools, with the bad table
    stabs, sfirst, scu, srows = wl.step_segments()
    kp2, vp2 = oracle.write(kp, vp, wl.k_rows[srows], wl.v_rows[srows],
                            oracle.slot_mapping(stabs, sfirst, scu, wl.block_size, wl.num_blocks))
    ref = oracle.decode(wl.q, kp2, vp2, bad, wl.context_lens, wl.scale, "f32")
    check_close(out_f64(out, "f32"), ref, "f32")


@pytest.mark.parametrize("cfg,cut", [(4, "auto"), (5, "auto"), (5, "pieces")])
def test_step_full_size_as_benchmarked(cfg, cut):
    """The benchmark's timed call at full size: pkv_decode_step on every
    sequence of the workload with partition 0 (the library's own cut: the
    stream-K ranges for the 70B layer, longest-first single pieces for the
    192 sequences) and a zero-filled workspace, the new token of each sequence
    at position ctx - 1; "pieces" passes the automatic partition explicitly,
    which keeps the piece schedule. Both pools are compared bit for bit with
    the oracle's bulk write followed by the step's write, and every output
    element with the oracle's decode."""
    wl = make_workload(cfg)
    rows = _new_rows(wl)
    pc = PoolCase(wl, exclude_last=True)
    part = 0 if cut == "auto" else pkv.decode_partition(wl.num_seqs, pc.max_ctx, pc.k_pool)
    schedule = pkv.decode_schedule(wl.num_seqs, wl.num_q_heads, pc.max_ctx, pc.k_pool, part)
    assert schedule == {(4, "auto"): "longest_first", (5, "auto"): "stream_k",
                        (5, "pieces"): "pieces"}[(cfg, cut)]
    ws = torch.zeros(max(16, pkv.decode_workspace_bytes(wl.num_seqs, wl.num_q_heads,
                                                        pc.max_ctx, pc.k_pool, part)),
                     dtype=torch.uint8, device=pc.q.device)
    out = torch.empty_like(pc.q)
    note(f"{wl.name}: full-size pkv_decode_step, partition {part or 'auto'}, {schedule}")
    pkv.decode_step(pc.q, to_dev(wl.k_rows[rows]), to_dev(wl.v_rows[rows]), pc.k_pool,
                    pc.v_pool, pc.tables, pc.ctx, wl.scale, pc.max_ctx, out=out,
                    partition=part, workspace=ws)
    torch.cuda.synchronize()
    kp, vp = pc.ref_pools()
    tabs, first, cu, srows = wl.step_segments()
    kp, vp = oracle.write(kp, vp, wl.k_rows[srows], wl.v_rows[srows],
                          oracle.slot_mapping(tabs, first, cu, wl.block_size, wl.num_blocks))
    assert np.array_equal(bits(to_host(pc.k_pool)), bits(kp)), "k_pool differs from the oracle"
    assert np.array_equal(bits(to_host(pc.v_pool)), bits(vp)), "v_pool differs from the oracle"
    ref = oracle.decode(wl.q, kp, vp, wl.block_tables, wl.context_lens, wl.scale, wl.dtype)
    err = check_close(oracle.storage_to_f64(to_host(out), wl.dtype), ref, wl.dtype, wl.name)
    # the merge counters are back to zero for the next call
    assert not to_host(ws[:256 << 10]).any()
    note(f"{wl.name}: pools bit-exact, all {wl.num_seqs} sequences within tolerance "
         f"(max error {err:.3e})")
