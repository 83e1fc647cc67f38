"""GPU parity of causal (chunked) prefill over the paged pool against the oracle."""

import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_scatter_amd as pkv
from workloads import make_custom, make_workload

from _gpu_util import PoolCase, bits, check_close, note, out_f64, to_dev, to_host

pytestmark = pytest.mark.gpu


def _run(pc, q_rows, cu_q, max_q_len):
    wl = pc.wl
    note(f"{wl.name}: pkv_prefill rows={q_rows.shape[0]} max_q_len={max_q_len}")
    out = pkv.prefill(to_dev(q_rows), to_dev(cu_q), pc.k_pool, pc.v_pool, pc.tables, pc.ctx,
                      wl.scale, max_q_len, pc.max_ctx)
    torch.cuda.synchronize()
    return out


def _rand_rows(n, wl, seed):
    g = torch.Generator().manual_seed(seed)
    x = torch.randn((n, wl.num_q_heads, wl.head_dim), generator=g)
    if wl.dtype == "f32":
        return x.numpy()
    return x.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_prefill_chunks_small(dtype):
    """Chunks of several lengths: the whole sequence, a short tail, one row,
    and a chunk longer than the context (its leading rows are zero)."""
    lens = [37, 70, 16, 5]
    qlens = [37, 20, 1, 9]
    rng = np.random.default_rng(3)
    need = sum(-(-L // 16) for L in lens)
    perm = (rng.permutation(need + 3) + 1).tolist()
    tabs, k = [], 0
    for L in lens:
        n = -(-L // 16)
        tabs.append(perm[k:k + n])
        k += n
    wl = make_custom(tabs, lens, dtype=dtype, num_q_heads=8, num_kv_heads=2, head_dim=64,
                     block_size=16, num_blocks=need + 4, seed=7)
    pc = PoolCase(wl)
    cu = np.concatenate([[0], np.cumsum(qlens)]).astype(np.int32)
    q_rows = _rand_rows(int(cu[-1]), wl, 11)
    got = out_f64(_run(pc, q_rows, cu, max(qlens)), dtype)
    kp, vp = pc.ref_pools()
    ref = oracle.prefill(q_rows, cu, kp, vp, wl.block_tables, wl.context_lens, wl.scale, dtype)
    check_close(got, ref, dtype, "prefill small")
    assert not got[int(cu[3]):int(cu[3]) + 4].any(), "rows before position 0 are zero"


def _tables(lens, bs, rng, spare=3):
    need = sum(-(-L // bs) for L in lens)
    perm = (rng.permutation(need + spare) + 1).tolist()
    tabs, k = [], 0
    for L in lens:
        n = -(-L // bs)
        tabs.append(perm[k:k + n])
        k += n
    return tabs, need + spare + 1


def _case(lens, qlens, dtype, hd, rep, hkv=2, bs=16, seed=0, fill="nan"):
    rng = np.random.default_rng(seed)
    tabs, nb = _tables(lens, bs, rng)
    wl = make_custom(tabs, lens, dtype=dtype, num_q_heads=hkv * rep, num_kv_heads=hkv,
                     head_dim=hd, block_size=bs, num_blocks=nb, seed=seed)
    pc = PoolCase(wl, fill=fill)
    cu = np.concatenate([[0], np.cumsum(qlens)]).astype(np.int32)
    q_rows = _rand_rows(int(cu[-1]), wl, seed + 100)
    return pc, cu, q_rows


def _ref(pc, q_rows, cu, tables=None, ctx=None):
    wl = pc.wl
    kp, vp = pc.ref_pools()
    return oracle.prefill(q_rows, cu, kp, vp, wl.block_tables if tables is None else tables,
                          wl.context_lens if ctx is None else ctx, wl.scale, wl.dtype)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("hd", [64, 128])
def test_prefill_matrix_core_variants(hd, dtype):
    """Chunks on every compiled group size (bf16 and fp32 matrix cores):
    chunks spanning several query tiles with ragged ends, a one-row chunk, and
    a chunk longer than its context (leading rows zero); K/V ranges spanning
    several key tiles."""
    lens = [150, 70, 33, 300, 1]
    qlens = [150, 20, 40, 130, 1]
    for rep in range(1, 9):
        pc, cu, q_rows = _case(lens, qlens, dtype, hd, rep, seed=rep)
        got = out_f64(_run(pc, q_rows, cu, max(qlens)), dtype)
        check_close(got, _ref(pc, q_rows, cu), dtype, f"hd={hd} rep={rep}")
        z0 = int(cu[2])
        assert not got[z0:z0 + 7].any(), "rows before position 0 are zero"


@pytest.mark.parametrize("bs", [1, 8, 32, 64])
def test_prefill_block_sizes(bs):
    lens = [3, 70, 129, 260]
    qlens = [3, 70, 50, 200]
    pc, cu, q_rows = _case(lens, qlens, "bf16", 128, 4, bs=bs, seed=bs)
    got = out_f64(_run(pc, q_rows, cu, max(qlens)), "bf16")
    check_close(got, _ref(pc, q_rows, cu), "bf16", f"bs={bs}")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_prefill_poison_is_bitwise_invisible(dtype):
    """Slots no token was written to (zero, NaN or huge values) never reach
    the output: identical bits for all three fills."""
    lens = [17, 64, 100, 333]
    qlens = [17, 30, 100, 77]
    outs = []
    for fill in ("zero", "nan", "huge"):
        pc, cu, q_rows = _case(lens, qlens, dtype, 64, 4, seed=21, fill=fill)
        outs.append(to_host(_run(pc, q_rows, cu, max(qlens))))
    assert np.array_equal(bits(outs[1]), bits(outs[0]))
    assert np.array_equal(bits(outs[2]), bits(outs[0]))
    check_close(oracle.storage_to_f64(outs[1], dtype), _ref(pc, q_rows, cu), dtype)


def test_prefill_invalid_block_id_is_excluded():
    lens = [100, 64]
    qlens = [60, 64]
    pc, cu, q_rows = _case(lens, qlens, "bf16", 128, 8, seed=31)
    bad = pc.wl.block_tables.copy()
    bad[0, 2] = 1 << 20
    bad[1, 0] = -3
    note("prefill with out-of-range block ids")
    wl = pc.wl
    out = pkv.prefill(to_dev(q_rows), to_dev(cu), pc.k_pool, pc.v_pool, to_dev(bad), pc.ctx,
                      wl.scale, max(qlens), pc.max_ctx)
    torch.cuda.synchronize()
    check_close(out_f64(out, "bf16"), _ref(pc, q_rows, cu, tables=bad), "bf16")


def test_prefill_context_beyond_max_context_len_is_clamped():
    lens = [200, 90]
    qlens = [40, 40]
    pc, cu, q_rows = _case(lens, qlens, "bf16", 64, 2, seed=41)
    wl = pc.wl
    note("prefill with max_context_len below the real lengths")
    out = pkv.prefill(to_dev(q_rows), to_dev(cu), pc.k_pool, pc.v_pool, pc.tables, pc.ctx,
                      wl.scale, max(qlens), 120)
    torch.cuda.synchronize()
    ctx = np.minimum(wl.context_lens, 120).astype(np.int32)
    check_close(out_f64(out, "bf16"), _ref(pc, q_rows, cu, ctx=ctx), "bf16")


def test_prefill_long_table_takes_row_path():
    """Block size 1 with a 2,100-token context: more table entries than the
    matrix-core path stages, so the row path runs; same results."""
    lens = [2100, 40]
    qlens = [24, 40]
    pc, cu, q_rows = _case(lens, qlens, "bf16", 64, 2, bs=1, seed=51)
    got = out_f64(_run(pc, q_rows, cu, max(qlens)), "bf16")
    check_close(got, _ref(pc, q_rows, cu), "bf16", "bs=1 long table")


def test_prefill_one_row_equals_decode_row_path():
    """A one-row chunk at each sequence's last position is that sequence's
    decode step. head_dim 16 prefill runs the decode kernel's row mode, so with
    the same single split the bits are identical."""
    wl = make_workload(1)
    pc = PoolCase(wl)
    cu = np.arange(wl.num_seqs + 1, dtype=np.int32)
    got = _run(pc, wl.q, cu, 1)
    whole = -(-pc.max_ctx // 64) * 64
    dec = pc.decode(partition=whole)
    assert torch.equal(got.view(torch.int32), dec.view(torch.int32))
    check_close(out_f64(got, "f32"), pc.ref_decode(), "f32")


def test_prefill_one_row_fp32_matrix_cores():
    """The SmolLM2-shape workload's shapes (fp32, head_dim 64: fp32 matrix
    cores): a one-row chunk agrees with the oracle's decode and with
    pkv_decode."""
    wl = make_workload(2, num_seqs=12)
    pc = PoolCase(wl)
    cu = np.arange(wl.num_seqs + 1, dtype=np.int32)
    got = out_f64(_run(pc, wl.q, cu, 1), "f32")
    ref = pc.ref_decode()
    check_close(got, ref, "f32", "prefill")
    check_close(got, out_f64(pc.decode(), "f32"), "f32", "vs decode")


def test_prefill_one_row_matches_decode_matrix_cores():
    """The same on the LLaMA-2-70B layer's shapes (bf16, matrix-core path):
    both agree with the oracle's decode."""
    wl = make_workload(5, num_seqs=3)
    pc = PoolCase(wl)
    cu = np.arange(4, dtype=np.int32)
    got = out_f64(_run(pc, wl.q, cu, 1), "bf16")
    ref = pc.ref_decode()
    check_close(got, ref, "bf16", "prefill")
    check_close(out_f64(pc.decode(), "bf16"), ref, "bf16", "decode")


def test_prefill_llama70b_layer_chunks():
    """The LLaMA-2-70B layer workload's chunked prefill at full size (64
    sequences x 512 rows at each sequence's last 512 positions), in the launch
    the benchmark times. The oracle checks the whole chunks of the three
    shortest and two more sequences, and of the longest sequence the first and
    last row of every query tile (128 (row, head) pairs = 128 / group-size
    rows per tile), plus 40 random rows of the others."""
    wl = make_workload(5)
    pc = PoolCase(wl)
    q_pre, cu = wl.prefill_queries()
    n = wl.prefill_chunk
    got = out_f64(_run(pc, q_pre, cu, n), "bf16")
    kp, vp = pc.ref_pools()
    lens = wl.context_lens
    order = np.argsort(lens, kind="stable")
    rng = np.random.default_rng(5)
    whole = [int(x) for x in order[:3]] + [int(x) for x in rng.choice(order[3:-1], 2,
                                                                      replace=False)]
    for s in whole:
        a, b = int(cu[s]), int(cu[s + 1])
        ref = oracle.prefill_one(q_pre[a:b], kp, vp, wl.block_tables[s], int(lens[s]),
                                 wl.scale, "bf16")
        check_close(got[a:b], ref, "bf16", f"sequence {s} (ctx {int(lens[s])}), whole chunk")
    longest = int(order[-1])
    tile_rows = 128 // (wl.num_q_heads // wl.num_kv_heads)
    rows = [int(cu[longest]) + i for t in range(0, n, tile_rows) for i in (t, t + tile_rows - 1)]
    others = [r for r in rng.choice(q_pre.shape[0], 60, replace=False).tolist()
              if int(np.searchsorted(cu, r, side="right") - 1) not in whole + [longest]][:40]
    for r in rows + sorted(others):
        s = int(np.searchsorted(cu, r, side="right") - 1)
        a = int(lens[s]) - n + (r - int(cu[s]))      # the row's absolute position
        ref = oracle.prefill_one(q_pre[r:r + 1], kp, vp, wl.block_tables[s], a + 1,
                                 wl.scale, "bf16")
        check_close(got[r:r + 1], ref, "bf16", f"row {r} (sequence {s}, position {a})")
    note(f"checked {len(whole)} whole chunks and {len(rows) + len(others)} more rows")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("hd", [64, 128])
def test_prefill_zero_queries_average_the_visible_v(dtype, hd):
    """q = 0 gives every visible key the same weight: row i of a chunk (its
    position a = ctx - q_len + i) is the mean of V over positions 0 .. a, a
    closed form of the causal mask computed from the written rows (rows before
    position 0 are zero). Matrix-core path, several query and key tiles."""
    lens = [150, 70, 33, 300]
    qlens = [150, 20, 40, 130]
    rep = 4
    pc, cu, q_rows = _case(lens, qlens, dtype, hd, rep, seed=hd)
    got = out_f64(_run(pc, np.zeros_like(q_rows), cu, max(qlens)), dtype)
    wl = pc.wl
    v = oracle.storage_to_f64(wl.v_rows, dtype)
    heads = np.arange(wl.num_q_heads) // rep
    want = np.zeros_like(got)
    for s, (L, n) in enumerate(zip(lens, qlens)):
        for i in range(n):
            a = L - n + i
            if a >= 0:
                want[cu[s] + i] = v[wl.seq_rows[s][:a + 1]].mean(axis=0)[heads]
    err = check_close(got, want, dtype, f"prefill zero queries hd={hd}")
    note(f"prefill zero queries, {dtype} hd={hd}: max error {err:.2e} against the mean of V")
