"""GPU parity of paged decode attention against the fp64 oracle.

Tolerances: fp32 -- per (sequence, head) row, max |gpu - ref| <= 1e-5 * max |ref|;
bf16 -- elementwise |gpu - ref| <= 2e-2 against the unrounded fp64 reference.
"""

import functools

import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_scatter_amd as pkv
from workloads import make_custom, make_tp_shard, make_workload

from _gpu_util import PoolCase, bits, check_close, note, out_f64, to_dev, to_host

pytestmark = pytest.mark.gpu


@functools.lru_cache(maxsize=3)
def _case(cfg, S=None, fill="nan"):
    return PoolCase(make_workload(cfg, num_seqs=S), fill=fill)


# ---------------------------------------------------------------- the five configs
@pytest.mark.parametrize("cfg,S", [(1, None), (2, None), (3, None), (4, 24), (5, 6)])
def test_decode_config_all_outputs(cfg, S):
    pc = _case(cfg, S)
    got = out_f64(pc.decode(), pc.wl.dtype)
    ref = pc.ref_decode()
    err = check_close(got, ref, pc.wl.dtype, pc.wl.name)
    note(f"{pc.wl.name}: max error {err:.3e}")


@pytest.mark.parametrize("cfg", [3, 4, 5])
def test_decode_full_size_every_sequence(cfg):
    """Full-size configuration in the default launch (automatic partition, the
    piece schedule or paired heads the planner picks, as the benchmark times
    it): every output element of every sequence against the oracle."""
    pc = _case(cfg)
    got = out_f64(pc.decode(), pc.wl.dtype)
    ref = pc.ref_decode()
    err = check_close(got, ref, pc.wl.dtype, pc.wl.name)
    note(f"{pc.wl.name}: all {pc.wl.num_seqs} sequences, max error {err:.3e}")


def test_tp8_shard_of_the_70b_layer_every_sequence():
    """One rank's share of the 70B layer with its 8 KV heads split over 8 GPUs
    (1 KV head, 8 query heads, head_dim 128, the layer's lengths and tables):
    only 64 (sequence, KV head) units, so the planner splits every long
    context. Every output of every sequence against the oracle."""
    pc = PoolCase(make_tp_shard(5, 8))
    got = out_f64(pc.decode(), pc.wl.dtype)
    err = check_close(got, pc.ref_decode(), pc.wl.dtype, pc.wl.name)
    note(f"{pc.wl.name}: all {pc.wl.num_seqs} sequences, max error {err:.3e}")


@pytest.mark.parametrize("hd,hq,S", [(128, 64, 128), (128, 64, 167), (128, 64, 300),
                                     (64, 32, 200)])
def test_longest_first_dealt_over_cu_passes(hd, hq, S):
    """One piece per sequence, longest first, the ranks dealt over the passes
    in which the CUs take the grid (one workgroup per CU: 32 sequences at 8
    KV heads of 128 dims, 64 at head_dim 64 read as 4 paired heads). Four full
    passes (reversed pairs); five and a partial one (a reversed pair, then the
    three-pass deal); nine and a partial one; paired heads with three full
    passes and a partial one. Each sequence must run exactly once: the output
    starts as NaN, so a rank map that is not a permutation leaves rows NaN."""
    rng = np.random.default_rng(7000 + S)
    bs = 16
    ctx = rng.integers(64, 2049, S).astype(np.int32)
    ctx[rng.integers(0, S)] = 2048
    nb = -(-ctx // bs)
    perm = rng.permutation(int(nb.sum())) + 1
    tables, k = [], 0
    for n in nb:
        tables.append(list(perm[k:k + n]))
        k += int(n)
    wl = make_custom(tables, ctx, dtype="bf16", num_q_heads=hq, num_kv_heads=8, head_dim=hd,
                     block_size=bs, num_blocks=int(nb.sum()) + 1, seed=S,
                     name=f"longest-first hd{hd} {S} seqs")
    pc = PoolCase(wl)
    assert pkv.decode_schedule(S, hq, int(ctx.max()), pc.k_pool) == "longest_first"
    out = torch.full(wl.q.shape, float("nan"), dtype=torch.bfloat16, device="cuda")
    got = out_f64(pc.decode(out=out), "bf16")
    err = check_close(got, pc.ref_decode(), "bf16", wl.name)
    note(f"{wl.name}: all sequences, max error {err:.3e}")


@pytest.mark.parametrize("cfg,S,parts", [(2, None, [64, 128, 256]),
                                         (3, None, [256, 512, 2048]),
                                         (5, 6, [256, 1024, 4096, 8192])])
def test_partition_sweep(cfg, S, parts):
    """Different split sizes (one split, several, many) all meet the tolerance,
    and the two phases called separately give the same bits as pkv_decode."""
    pc = _case(cfg, S)
    ref = pc.ref_decode()
    for p in parts:
        got = out_f64(pc.decode(partition=p), pc.wl.dtype)
        check_close(got, ref, pc.wl.dtype, f"{pc.wl.name} partition {p}")
    p = parts[0]
    both = to_host(pc.decode(partition=p))
    out = torch.empty_like(pc.q)
    ws = torch.zeros(pkv.decode_workspace_bytes(pc.wl.num_seqs, pc.wl.num_q_heads, pc.max_ctx,
                                                pc.k_pool, p) or 1,
                     dtype=torch.uint8, device=pc.q.device)
    for ph in ("partials", "reduce"):
        pkv.decode(pc.q, pc.k_pool, pc.v_pool, pc.tables, pc.ctx, pc.wl.scale, pc.max_ctx,
                   out=out, partition=p, workspace=ws, phase=ph)
    torch.cuda.synchronize()
    assert np.array_equal(bits(to_host(out)), bits(both))


# ---------------------------------------------------------------- exact cases
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("hd,hq,hkv", [(16, 8, 4), (64, 9, 3), (128, 64, 8), (256, 4, 4)])
def test_ctx1_is_exactly_v0(dtype, hd, hq, hkv):
    wl = make_custom([[3], [1], [2]], [1, 1, 1], dtype=dtype, num_q_heads=hq,
                     num_kv_heads=hkv, head_dim=hd, block_size=16, num_blocks=4, seed=hd)
    pc = PoolCase(wl)
    got = to_host(pc.decode())
    rep = hq // hkv
    for s in range(3):
        v0 = wl.v_rows[wl.seq_rows[s][0]]
        for h in range(hq):
            assert np.array_equal(bits(got[s, h]), bits(v0[h // rep])), (s, h)


def test_ctx0_gives_zeros():
    wl = make_custom([[1, 2], [3, 0]], [0, 20], num_q_heads=4, num_kv_heads=2, head_dim=64,
                     block_size=16, num_blocks=4, seed=2)
    pc = PoolCase(wl)
    got = to_host(pc.decode())
    assert not got[0].any()
    check_close(oracle.storage_to_f64(got, "f32"), pc.ref_decode(), "f32")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_poison_is_bitwise_invisible(dtype):
    rng = np.random.default_rng(4)
    lens = [1, 15, 17, 64, 100, 333]
    perm = (rng.permutation(60) + 1).tolist()
    tabs, k = [], 0
    for L in lens:
        n = -(-L // 16)
        tabs.append(perm[k:k + n])
        k += n
    outs = []
    for fill in ("zero", "nan", "huge"):
        wl = make_custom(tabs, lens, dtype=dtype, num_q_heads=8, num_kv_heads=2, head_dim=128,
                         block_size=16, num_blocks=61, seed=5)
        pc = PoolCase(wl, fill=fill)
        outs.append(to_host(pc.decode(partition=64)))
        outs.append(to_host(pc.decode()))
    # outs alternates (partition 64, auto partition) for zero, NaN and huge fills
    for i in (2, 4):
        assert np.array_equal(bits(outs[i]), bits(outs[0]))
        assert np.array_equal(bits(outs[i + 1]), bits(outs[1]))
    check_close(oracle.storage_to_f64(outs[1], dtype), pc.ref_decode(), dtype)
    check_close(oracle.storage_to_f64(outs[0], dtype), pc.ref_decode(), dtype)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_block_relabeling_is_bitwise_invisible(dtype):
    """Same logical content under other physical block ids ([2, 0] vs [1, 2],
    and a random relabeling): identical output bits."""
    outs = []
    for tabs in ([[2, 0]], [[1, 2]], [[7, 4]]):
        wl = make_custom(tabs, [29], dtype=dtype, num_q_heads=4, num_kv_heads=1, head_dim=64,
                         block_size=16, num_blocks=8, seed=6)
        outs.append(to_host(PoolCase(wl).decode()))
    assert np.array_equal(bits(outs[0]), bits(outs[1]))
    assert np.array_equal(bits(outs[0]), bits(outs[2]))


def test_shared_prefix_tables_bitwise():
    wl = make_custom([[1, 2, 5], [1, 2, 6]], [30, 30], num_q_heads=9, num_kv_heads=3,
                     head_dim=64, block_size=16, num_blocks=8, prefix_tokens=32, seed=7)
    q = wl.q.copy()
    q[1] = q[0]
    pc = PoolCase(wl)
    got = to_host(pc.decode(q=to_dev(q)))
    assert np.array_equal(bits(got[0]), bits(got[1]))
    wl2 = make_custom([[1, 2, 5], [1, 2, 6]], [40, 47], num_q_heads=9, num_kv_heads=3,
                      head_dim=64, block_size=16, num_blocks=8, prefix_tokens=32, seed=7)
    pc2 = PoolCase(wl2)
    check_close(out_f64(pc2.decode(), "f32"), pc2.ref_decode(), "f32")


def test_invalid_block_id_is_excluded():
    wl = make_custom([[1, 2, 3], [4, 5]], [40, 30], num_q_heads=8, num_kv_heads=2,
                     head_dim=64, block_size=16, num_blocks=6, seed=8)
    pc = PoolCase(wl)
    bad = wl.block_tables.copy()
    bad[0, 1] = 1 << 20
    bad[1, 0] = -3
    tables = to_dev(bad)
    note("decode with out-of-range block ids")
    out = pkv.decode(pc.q, pc.k_pool, pc.v_pool, tables, pc.ctx, wl.scale, pc.max_ctx)
    torch.cuda.synchronize()
    kp, vp = pc.ref_pools()
    ref = oracle.decode(wl.q, kp, vp, bad, wl.context_lens, wl.scale, "f32")
    check_close(out_f64(out, "f32"), ref, "f32")


def test_context_beyond_max_context_len_is_clamped():
    wl = make_custom([[1, 2, 3]], [40], num_q_heads=2, num_kv_heads=1, head_dim=64,
                     block_size=16, num_blocks=4, seed=9)
    pc = PoolCase(wl)
    note("decode with max_context_len below the real length")
    out = pkv.decode(pc.q, pc.k_pool, pc.v_pool, pc.tables, pc.ctx, wl.scale, 20)
    torch.cuda.synchronize()
    kp, vp = pc.ref_pools()
    ref = oracle.decode(wl.q, kp, vp, wl.block_tables, np.array([20], np.int32), wl.scale,
                        "f32")
    check_close(out_f64(out, "f32"), ref, "f32")


# ---------------------------------------------------------------- every compiled kernel
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("hd", [16, 32, 64, 128, 256])
def test_every_compiled_variant(dtype, hd):
    """Each (dtype, head_dim, group size) kernel on ragged lengths that span
    several tiles, a partial last block and a multi-split sequence."""
    lens = [1, 13, 48, 97, 700]
    for rep in range(1, 9):
        hkv = 2
        rng = np.random.default_rng(rep)
        need = sum(-(-L // 16) for L in lens)
        perm = (rng.permutation(need + 5) + 1).tolist()
        tabs, k = [], 0
        for L in lens:
            n = -(-L // 16)
            tabs.append(perm[k:k + n])
            k += n
        wl = make_custom(tabs, lens, dtype=dtype, num_q_heads=hkv * rep, num_kv_heads=hkv,
                         head_dim=hd, block_size=16, num_blocks=need + 6, seed=rep)
        pc = PoolCase(wl)
        ref = pc.ref_decode()
        for part in (0, 256):
            got = out_f64(pc.decode(partition=part), dtype)
            check_close(got, ref, dtype, f"{dtype} hd={hd} rep={rep} partition={part}")


@pytest.mark.parametrize("bs", [1, 8, 32, 64])
def test_other_block_sizes(bs):
    lens = [3, 70, 129]
    need = sum(-(-L // bs) for L in lens)
    rng = np.random.default_rng(bs)
    perm = (rng.permutation(need) + 1).tolist()
    tabs, k = [], 0
    for L in lens:
        n = -(-L // bs)
        tabs.append(perm[k:k + n])
        k += n
    wl = make_custom(tabs, lens, dtype="bf16", num_q_heads=8, num_kv_heads=2, head_dim=64,
                     block_size=bs, num_blocks=need + 1, seed=bs)
    pc = PoolCase(wl)
    check_close(out_f64(pc.decode(), "bf16"), pc.ref_decode(), "bf16", f"bs={bs}")


def test_step_write_then_decode_llama1b_192_sequences():
    """The decode step of the 192-sequence Llama-3.2-1B workload: slot mapping
    and write of the new token at position ctx-1, then attention over the
    whole context."""
    wl = make_workload(4, num_seqs=32)
    pc = PoolCase(wl, exclude_last=True)
    tabs, first, cu, rows = wl.step_segments()
    note(f"{wl.name}: step write + decode")
    slots = pkv.slot_mapping(to_dev(tabs), to_dev(first), to_dev(cu), int(cu[-1]),
                             wl.block_size, wl.num_blocks)
    pkv.write(to_dev(wl.k_rows[rows]), to_dev(wl.v_rows[rows]), slots, pc.k_pool, pc.v_pool)
    got = out_f64(pc.decode(), "bf16")
    full = PoolCase.__new__(PoolCase)
    full.wl, full.kp0, full.vp0 = wl, pc.kp0, pc.vp0
    full.tabs, full.first, full.cu, full.rows = wl.bulk_segments()
    full._ref_pools = None
    check_close(got, full.ref_decode(), "bf16", wl.name)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("hd,hq,hkv,partition", [(64, 9, 3, 0), (64, 32, 8, 0), (128, 64, 8, 0),
                                                 (128, 64, 8, 64)])
def test_zero_queries_average_v(dtype, hd, hq, hkv, partition):
    """q = 0 makes every score 0, so the softmax weights are equal and each
    head's output is the plain mean of its KV head's V rows over the context:
    a closed form computed here from the written rows, not by the oracle.
    Automatic and forced (many-split) partitions."""
    lens = [1, 17, 200, 513]
    rng = np.random.default_rng(hd + hq)
    need = [-(-L // 16) for L in lens]
    perm = (rng.permutation(sum(need) + 5) + 1).tolist()
    tabs, k = [], 0
    for n in need:
        tabs.append(perm[k:k + n])
        k += n
    wl = make_custom(tabs, lens, dtype=dtype, num_q_heads=hq, num_kv_heads=hkv, head_dim=hd,
                     block_size=16, num_blocks=sum(need) + 6, seed=hd)
    pc = PoolCase(wl)
    got = out_f64(pc.decode(partition=partition, q=torch.zeros_like(pc.q)), dtype)
    v = oracle.storage_to_f64(wl.v_rows, dtype)          # [rows, Hkv, hd]
    heads = np.arange(hq) // (hq // hkv)
    want = np.stack([v[wl.seq_rows[s]].mean(axis=0)[heads] for s in range(len(lens))])
    err = check_close(got, want, dtype, f"zero queries hd={hd} partition={partition}")
    note(f"zero queries, {dtype} hd={hd}: max error {err:.2e} against the mean of V")
