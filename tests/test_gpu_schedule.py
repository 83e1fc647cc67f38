"""GPU parity of the decode launch orders: the piece schedule (full pieces,
tail pieces, a short rest joined to the last full piece), the longest-first
order of single-piece launches, the plain split grid they fall back to, and
the in-launch merge with its per-(sequence, KV head) counters.

Tolerances as in test_gpu_decode: fp32 row-relative 1e-5, bf16 absolute 2e-2.
"""

import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_scatter_amd as pkv
from workloads import make_custom

from _gpu_util import PoolCase, bits, check_close, note, out_f64, to_host

pytestmark = pytest.mark.gpu

SCHED_MAX_SEQS = 1024   # the piece schedule and the longest-first order stop here


def _tables(lens, bs, rng, spare=3):
    """Block tables of randomly permuted distinct blocks (block 0 unused)."""
    need = sum(-(-int(L) // bs) for L in lens)
    perm = (rng.permutation(need + spare) + 1).tolist()
    tabs, k = [], 0
    for L in lens:
        n = -(-int(L) // bs)
        tabs.append(perm[k:k + n])
        k += n
    return tabs, need + spare + 1


def _ws(pc, partition):
    need = pkv.decode_workspace_bytes(pc.wl.num_seqs, pc.wl.num_q_heads, pc.max_ctx, pc.k_pool,
                                      partition)
    return need, torch.zeros(max(need, 16), dtype=torch.uint8, device=pc.q.device)


COUNTER_AREA = 65536 * 4   # merge counters, at the start of every decode workspace


def _counters_zero(ws, need):
    """The merge counter area of a workspace is all zero again."""
    if need == 0:
        return True
    return not to_host(ws[:COUNTER_AREA]).any()


def _decode(pc, partition, ws=None, phase="both", **kw):
    S = kw.get("q", pc.q).shape[0]
    note(f"{pc.wl.name}: S={S} partition={partition or 'auto'} phase={phase}")
    out = pkv.decode(kw.get("q", pc.q), pc.k_pool, pc.v_pool, kw.get("tables", pc.tables),
                     kw.get("ctx", pc.ctx), pc.wl.scale, kw.get("max_ctx", pc.max_ctx),
                     out=kw.get("out"), partition=partition, workspace=ws, phase=phase)
    torch.cuda.synchronize()
    return out


# ------------------------------------------------------------ piece boundaries
# partition 256 with 16-token alignment: tail pieces of at most 128 tokens, a
# rest under 64 joins the last full piece, tails of 96 or more run first
BOUNDARY_LENS = [0, 1, 100, 200, 255, 256, 257, 319, 320, 351, 352, 383, 384, 385, 511, 512,
                 513, 1088, 1224, 2047, 2048]


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_piece_boundaries(dtype):
    """Lengths on and around every boundary of the piece schedule: equal to
    the oracle; the same lengths on the plain split grid (a partition that is
    not a power of two) too; repeated calls give the same bits and leave the
    counters at zero; the two phases called separately give those bits."""
    lens = BOUNDARY_LENS
    tabs, nb = _tables(lens, 16, np.random.default_rng(11))
    wl = make_custom(tabs, lens, dtype=dtype, num_q_heads=16, num_kv_heads=2, head_dim=128,
                     block_size=16, num_blocks=nb, seed=12, name=f"boundaries-{dtype}")
    pc = PoolCase(wl)
    ref = pc.ref_decode()
    need, ws = _ws(pc, 256)
    first = to_host(_decode(pc, 256, ws))
    check_close(oracle.storage_to_f64(first, dtype), ref, dtype, "piece schedule")
    assert _counters_zero(ws, need)
    for _ in range(2):
        again = to_host(_decode(pc, 256, ws))
        assert np.array_equal(bits(again), bits(first)), "repeated call differs"
        assert _counters_zero(ws, need)
    out = torch.empty_like(pc.q)
    for ph in ("partials", "reduce"):
        _decode(pc, 256, ws, phase=ph, out=out)
    assert np.array_equal(bits(to_host(out)), bits(first)), "two phases differ"
    assert _counters_zero(ws, need)
    for part in (240, 64, 0):   # plain grid; many small pieces; automatic
        got = out_f64(_decode(pc, part), dtype)
        check_close(got, ref, dtype, f"partition {part}")


def test_clamped_lengths_under_the_schedule():
    """Context lengths above max_context_len are clamped before the pieces
    are counted (the slot count follows max_context_len); 256-token pieces
    (128 KiB of K and V) take the piece schedule, smaller ones the plain grid."""
    lens = [40, 700, 300, 5, 321, 0]
    tabs, nb = _tables(lens, 16, np.random.default_rng(13))
    wl = make_custom(tabs, lens, dtype="f32", num_q_heads=4, num_kv_heads=2, head_dim=64,
                     block_size=16, num_blocks=nb, seed=14, name="clamped")
    pc = PoolCase(wl)
    kp, vp = pc.ref_pools()
    cap = 320
    ref = oracle.decode(wl.q, kp, vp, wl.block_tables,
                        np.minimum(wl.context_lens, cap).astype(np.int32), wl.scale, "f32")
    for part in (256, 128, 64, 0):
        got = out_f64(_decode(pc, part, max_ctx=cap), "f32")
        check_close(got, ref, "f32", f"clamped, partition {part}")


# ------------------------------------------------------------ the sequence limit
def _many(S, lo, hi, seed, dtype="bf16", hd=64, hq=4, hkv=1):
    rng = np.random.default_rng(seed)
    lens = rng.integers(lo, hi + 1, size=S)
    lens[rng.choice(S, size=S // 50, replace=False)] = 0
    lens[rng.choice(S, size=S // 50, replace=False)] = hi
    tabs, nb = _tables(lens, 16, rng)
    wl = make_custom(tabs, lens, dtype=dtype, num_q_heads=hq, num_kv_heads=hkv, head_dim=hd,
                     block_size=16, num_blocks=nb, seed=seed, name=f"many-{S}")
    return PoolCase(wl)


def test_schedule_and_plain_grid_at_the_sequence_limit():
    """1025 sequences split into 256-token pieces run on the plain grid; their
    first 1024 run on the piece schedule. Both equal the oracle."""
    pc = _many(SCHED_MAX_SEQS + 1, 1, 700, seed=21, hd=128)
    ref = pc.ref_decode()
    got = out_f64(_decode(pc, 256), "bf16")
    check_close(got, ref, "bf16", "1025 sequences, plain grid")
    S = SCHED_MAX_SEQS
    need = pkv.decode_workspace_bytes(S, pc.wl.num_q_heads, pc.max_ctx, pc.k_pool, 256)
    ws = torch.zeros(need, dtype=torch.uint8, device=pc.q.device)
    part = _decode(pc, 256, ws, q=pc.q[:S], tables=pc.tables[:S], ctx=pc.ctx[:S])
    check_close(out_f64(part, "bf16"), ref[:S], "bf16", "1024 sequences, piece schedule")
    assert _counters_zero(ws, need)


def test_longest_first_order_changes_no_bit():
    """Single-piece launches: 1025 sequences run in index order, their first
    1024 in longest-first order; every output bit is the same, and both equal
    the oracle. Lengths fill all four length classes."""
    pc = _many(SCHED_MAX_SEQS + 1, 1, 400, seed=22, hkv=2, hq=8)
    S = SCHED_MAX_SEQS
    assert pkv.decode_workspace_bytes(S + 1, 8, pc.max_ctx, pc.k_pool, 0) == 0   # one piece
    full = to_host(_decode(pc, 0))
    head = to_host(_decode(pc, 0, q=pc.q[:S], tables=pc.tables[:S], ctx=pc.ctx[:S]))
    assert np.array_equal(bits(head), bits(full[:S]))
    check_close(oracle.storage_to_f64(full, "bf16"), pc.ref_decode(), "bf16", "index order")


@pytest.mark.parametrize("kind", ["equal", "one-long", "classes", "all-empty-but-one"])
def test_longest_first_length_mixes(kind):
    """Longest-first order on length mixes that load the classes unevenly;
    a partition covering max_context_len makes every sequence one piece."""
    rng = np.random.default_rng(31)
    S, top = 300, 1000   # max_context_len is the longest length
    if kind == "equal":
        lens = np.full(S, 777)
    elif kind == "one-long":
        lens = rng.integers(1, 40, size=S)
        lens[137] = top
    elif kind == "classes":   # every class, both ends of each
        edges = [0, 1, 249, 250, 251, 499, 500, 501, 749, 750, 751, 999, 1000]
        lens = np.array((edges * (S // len(edges) + 1))[:S])
        rng.shuffle(lens)
    else:
        lens = np.zeros(S, np.int64)
        lens[S - 1] = 513
    tabs, nb = _tables(lens, 16, rng)
    wl = make_custom(tabs, lens, dtype="f32", num_q_heads=6, num_kv_heads=2, head_dim=32,
                     block_size=16, num_blocks=nb, seed=32, name=f"lpt-{kind}")
    pc = PoolCase(wl)
    got = out_f64(_decode(pc, 1024), "f32")   # one piece per sequence
    kp, vp = pc.ref_pools()
    ref = oracle.decode(wl.q, kp, vp, wl.block_tables, wl.context_lens, wl.scale, "f32")
    check_close(got, ref, "f32", kind)
    assert not got[np.asarray(lens) == 0].any()


# ------------------------------------------------------------ workspace reuse
def test_one_workspace_across_calls_of_different_sizes():
    """A workspace reused by calls of different sizes and partitions (in
    stream order) gives the bits of a fresh workspace each time: every call
    leaves the merge counters at zero."""
    big = _many(600, 1, 900, seed=41)
    small = _many(70, 1, 2000, seed=42)
    calls = ((big, 64), (small, 256), (big, 128), (small, 0), (big, 64))

    def need(c, p):
        return pkv.decode_workspace_bytes(c.wl.num_seqs, c.wl.num_q_heads, c.max_ctx, c.k_pool,
                                          p)
    ws = torch.zeros(max(need(c, p) for c, p in calls), dtype=torch.uint8, device=big.q.device)
    for c, p in calls:
        shared = to_host(_decode(c, p, ws))
        assert _counters_zero(ws, need(c, p)), (c.wl.name, p)
        fresh = to_host(_decode(c, p))
        assert np.array_equal(bits(shared), bits(fresh)), (c.wl.name, p)
    for c in (big, small):
        check_close(out_f64(_decode(c, 0, ws), "bf16"), c.ref_decode(), "bf16", c.wl.name)


def test_merge_counter_area_limit():
    """1024 sequences x 64 KV heads fill the 65536 merge counters exactly (the
    merge runs in the launch); 1025 sequences exceed them and merge in a
    second kernel. A few long contexts make several pieces; both equal the
    oracle."""
    rng = np.random.default_rng(51)
    S = SCHED_MAX_SEQS + 1
    lens = rng.integers(0, 9, size=S)
    longs = rng.choice(S - 1, size=24, replace=False)
    lens[longs] = rng.integers(65, 200, size=24)
    tabs, nb = _tables(lens, 16, rng)
    wl = make_custom(tabs, lens, dtype="bf16", num_q_heads=64, num_kv_heads=64, head_dim=16,
                     block_size=16, num_blocks=nb, seed=52, name="counter-limit")
    pc = PoolCase(wl)
    ref = pc.ref_decode()
    for n in (S, S - 1):
        need = pkv.decode_workspace_bytes(n, 64, pc.max_ctx, pc.k_pool, 64)
        ws = torch.zeros(need, dtype=torch.uint8, device=pc.q.device)
        got = _decode(pc, 64, ws, q=pc.q[:n], tables=pc.tables[:n], ctx=pc.ctx[:n])
        check_close(out_f64(got, "bf16"), ref[:n], "bf16", f"{n} sequences x 64 KV heads")
        assert _counters_zero(ws, COUNTER_AREA)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_more_than_64_pieces_per_sequence(dtype):
    """Contexts of 20,000 and 12,000 tokens: 78 partials per (sequence, head)
    on the piece schedule (256-token pieces), 313 and 417 on the plain grid
    (64 and 48), so the merge walks its partials in several batches of 64
    lanes, in the launch and in the two-phase reduce kernel."""
    lens = [20000, 12000, 4500, 70, 1, 0]
    tabs, nb = _tables(lens, 16, np.random.default_rng(61))
    wl = make_custom(tabs, lens, dtype=dtype, num_q_heads=8, num_kv_heads=2, head_dim=128,
                     block_size=16, num_blocks=nb, seed=62, name=f"long-{dtype}")
    pc = PoolCase(wl)
    ref = pc.ref_decode()
    for part in (256, 64, 48):
        need, ws = _ws(pc, part)
        both = to_host(_decode(pc, part, ws))
        check_close(oracle.storage_to_f64(both, dtype), ref, dtype, f"partition {part}")
        assert _counters_zero(ws, need)
        out = torch.empty_like(pc.q)
        for ph in ("partials", "reduce"):
            _decode(pc, part, ws, phase=ph, out=out)
        assert np.array_equal(bits(to_host(out)), bits(both)), part


def test_most_sequences_the_grid_takes():
    """65,535 sequences (the most a launch takes): one piece each in index
    order, and pieces of 32 tokens merged in the launch (65,535 counters)."""
    rng = np.random.default_rng(71)
    S = 65535
    lens = rng.integers(0, 81, size=S)
    tabs, nb = _tables(lens, 16, rng)
    wl = make_custom(tabs, lens, dtype="bf16", num_q_heads=2, num_kv_heads=1, head_dim=64,
                     block_size=16, num_blocks=nb, seed=72, name="most-sequences")
    pc = PoolCase(wl)
    note("oracle over 65,535 sequences (about 15 s)")
    ref = pc.ref_decode()
    for part in (0, 32):
        need, ws = _ws(pc, part)
        got = out_f64(_decode(pc, part, ws), "bf16")
        check_close(got, ref, "bf16", f"{S} sequences, partition {part}")
        assert _counters_zero(ws, need)
