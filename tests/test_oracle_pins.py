"""Pins of the CPU oracle to facts other than itself (no GPU needed).

Each test ties one part of the oracle to something independent: a figure the
pages print, a closed form, a library routine (torch's fp64
scaled_dot_product_attention), brute force with Python loops, or an invariant
the pages state (paged attention over table-ordered K/V equals contiguous
attention, "Build a Mini vLLM", "Key Takeaways" item 3 and section 4).
"""

import json
import math
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
from workloads import kv_bytes, make_custom
from workloads.gen import POISON_HUGE, POISON_NAN, poison_pool

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _gold(name):
    with open(os.path.join(GOLD, name)) as f:
        return json.load(f)


def _fill_pool(wl, bits=None, zero=False):
    """Pools holding every token row of ``wl`` at its table slots; all other
    slots hold ``bits`` (NaN by default) or zeros."""
    if zero:
        kp = np.zeros(wl.pool_shape, dtype=wl.storage_np_dtype)
        vp = np.zeros(wl.pool_shape, dtype=wl.storage_np_dtype)
    else:
        kp = poison_pool(wl, bits)
        vp = poison_pool(wl, bits)
    tabs, first, cu, rows = wl.bulk_segments()
    slots = oracle.slot_mapping(tabs, first, cu, wl.block_size, wl.num_blocks)
    return oracle.write(kp, vp, wl.k_rows[rows], wl.v_rows[rows], slots)


def _contig(wl, s):
    """Sequence s's K, V as contiguous float64 [ctx, Hkv, hd] (no pool involved)."""
    r = wl.seq_rows[s]
    return (oracle.storage_to_f64(wl.k_rows[r], wl.dtype),
            oracle.storage_to_f64(wl.v_rows[r], wl.dtype))


# ---------------------------------------------------------------- byte counts
def test_kv_bytes_match_pages():
    g = _gold("kv_bytes.json")
    for e in g["per_token"]:
        assert kv_bytes(1, e["layers"], e["kv_heads"], e["head_dim"], e["itemsize"]) == e["bytes"], e
    for e in g["per_block"]:
        assert kv_bytes(e["block_size"], e["layers"], e["kv_heads"], e["head_dim"],
                        e["itemsize"]) == e["bytes"], e
    blk = g["per_block"][0]
    per_block = kv_bytes(blk["block_size"], blk["layers"], blk["kv_heads"], blk["head_dim"],
                         blk["itemsize"])
    assert (1 << 30) // per_block == g["gib"]["blocks"]
    assert g["gib"]["blocks"] * blk["block_size"] == g["gib"]["tokens"]


# ---------------------------------------------------------------- slot mapping
def test_slot_mapping_out_of_order_blocks():
    g = _gold("block_ids_2_0.json")
    slots = oracle.slot_mapping([g["table"]], [0], [0, g["ctx"]], g["block_size"], 3)
    assert slots.tolist() == g["slots"]


def test_slot_mapping_shared_prefix_tables():
    g = _gold("shared_prefix_tables.json")
    bs = g["block_size"]
    for user, table in g["tables"].items():
        slots = oracle.slot_mapping([table], [0], [0, 48], bs, 8)
        for pos, slot in g["slots_at_positions"][user].items():
            assert slots[int(pos)] == slot
        assert g["dummy_block"] not in table


def test_slot_mapping_interleaved_allocation():
    g = _gold("interleaved_alloc.json")
    for name in ("A", "B"):
        s = oracle.slot_mapping([g["tables"][name]], [0], [0, g["lengths"][name]],
                                g["block_size"], 12)
        assert s.tolist() == g["slots"][name]


class _BlockManager:
    """Brute-force on-demand allocator: a sequence takes a new block from the
    free list whenever its next position starts a block, and each appended
    token gets (block, offset) of that position ("Build a Mini vLLM",
    section 2, append_slot)."""

    def __init__(self, num_blocks, bs, rng):
        self.free = list(range(num_blocks))
        rng.shuffle(self.free)
        self.bs = bs
        self.table, self.length = {}, {}

    def append_slot(self, sid):
        pos = self.length.setdefault(sid, 0)
        t = self.table.setdefault(sid, [])
        if pos % self.bs == 0:
            t.append(self.free.pop())
        self.length[sid] = pos + 1
        return t[pos // self.bs], pos % self.bs


def test_slot_mapping_matches_incremental_allocator():
    rng = np.random.default_rng(5)
    bs, nb = 8, 200
    bm = _BlockManager(nb, bs, rng)
    lens = [int(x) for x in rng.integers(1, 90, size=7)]
    got = {s: [] for s in range(len(lens))}
    # interleaved appends, as during real decode
    for step in range(max(lens)):
        for s, n in enumerate(lens):
            if step < n:
                b, o = bm.append_slot(s)
                got[s].append(b * bs + o)
    for s, n in enumerate(lens):
        slots = oracle.slot_mapping([bm.table[s]], [0], [0, n], bs, nb)
        assert slots.tolist() == got[s]
    # a write that starts mid-sequence (decode step at position n-1)
    for s, n in enumerate(lens):
        slots = oracle.slot_mapping([bm.table[s]], [n - 1], [0, 1], bs, nb)
        assert slots.tolist() == [got[s][-1]]


def test_slot_mapping_out_of_range_is_minus_one():
    # past the table, a negative id, an id beyond the pool
    s = oracle.slot_mapping([[3, -1, 9]], [0], [0, 12], 4, 8)
    assert s[:4].tolist() == [12, 13, 14, 15]
    assert s[4:8].tolist() == [-1] * 4
    assert s[8:12].tolist() == [-1] * 4
    s = oracle.slot_mapping([[1]], [2], [0, 4], 4, 8)   # positions 2..5: 5 is past the table
    assert s.tolist() == [6, 7, -1, -1]


# ---------------------------------------------------------------- write
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_write_reads_back_exactly_and_touches_nothing_else(dtype):
    wl = make_custom([[3, 1, 7]], [40], dtype=dtype, num_q_heads=4, num_kv_heads=2,
                     head_dim=16, block_size=16, num_blocks=9, seed=3)
    kp0 = poison_pool(wl)
    vp0 = poison_pool(wl, POISON_HUGE[dtype])
    tabs, first, cu, rows = wl.bulk_segments()
    slots = oracle.slot_mapping(tabs, first, cu, 16, 9)
    kp, vp = oracle.write(kp0, vp0, wl.k_rows[rows], wl.v_rows[rows], slots)
    u = np.uint32 if dtype == "f32" else np.uint16
    kb, vb = kp.view(u).reshape(-1, 2, 16), vp.view(u).reshape(-1, 2, 16)
    # read back through the table, position by position
    for p in range(40):
        blk, off = wl.block_tables[0][p // 16], p % 16
        assert np.array_equal(kp[blk, off].view(u), wl.k_rows[p].view(u))
        assert np.array_equal(vp[blk, off].view(u), wl.v_rows[p].view(u))
    untouched = np.ones(9 * 16, dtype=bool)
    untouched[slots] = False
    assert np.array_equal(kb[untouched], kp0.view(u).reshape(-1, 2, 16)[untouched])
    assert np.array_equal(vb[untouched], vp0.view(u).reshape(-1, 2, 16)[untouched])


def test_write_skips_out_of_range_slots():
    kp0 = np.zeros((2, 4, 1, 2), dtype=np.float32)
    vp0 = np.zeros_like(kp0)
    k = np.arange(8, dtype=np.float32).reshape(4, 1, 2) + 1
    kp, vp = oracle.write(kp0, vp0, k, -k, np.array([-1, 8, 3, 100]))
    flat = kp.reshape(8, 2)
    assert flat[3].tolist() == [5.0, 6.0]
    flat[3] = 0
    assert not flat.any()


# ---------------------------------------------------------------- dtype handling
def test_bf16_upcast_and_round():
    bits = np.array([0x3F80, 0xC000, 0x3E00, 0x0001, 0x7F80, 0xFF80, 0x4049], dtype=np.uint16)
    x = oracle.storage_to_f64(bits, "bf16")
    assert x[:4].tolist() == [1.0, -2.0, 0.125, 2.0 ** -133]
    assert x[4] == math.inf and x[5] == -math.inf
    assert x[6] == 3.140625
    # round to nearest even: 1 + 2^-8 is a tie between 1 and 1 + 2^-7 -> even (1.0)
    r = oracle.bf16_bits_from_f64(np.array([1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -3.140625]))
    assert r.tolist() == [0x3F80, 0x3F82, 0xC049]


# ---------------------------------------------------------------- attention math
def _sdpa(q, K, V, scale, causal=False):
    """torch fp64 SDPA with grouped KV heads; q [n, Hq, hd], K/V [L, Hkv, hd]."""
    qt = torch.from_numpy(q).permute(1, 0, 2)[None]
    kt = torch.from_numpy(K).permute(1, 0, 2)[None]
    vt = torch.from_numpy(V).permute(1, 0, 2)[None]
    o = F.scaled_dot_product_attention(qt, kt, vt, scale=scale, enable_gqa=True,
                                       is_causal=causal)
    return o[0].permute(1, 0, 2).numpy()


@pytest.mark.parametrize("Hq,Hkv,hd,L,scale_mult", [
    (8, 4, 16, 37, 1.0), (9, 3, 64, 130, 1.0), (32, 8, 64, 300, 1.0),
    (8, 8, 32, 5, 1.0), (6, 2, 16, 50, 40.0),   # last: scores in the hundreds
])
def test_attend_equals_library_sdpa(Hq, Hkv, hd, L, scale_mult):
    rng = np.random.default_rng(Hq * 1000 + L)
    q = rng.standard_normal((Hq, hd))
    K = rng.standard_normal((L, Hkv, hd))
    V = rng.standard_normal((L, Hkv, hd))
    scale = scale_mult / math.sqrt(hd)
    got = oracle.attention(q, K, V, scale)
    ref = _sdpa(q[None], K, V, scale)[0]
    assert np.isfinite(got).all()
    np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-12)


def test_ctx1_closed_form():
    # one key: the softmax weight is exactly 1, so out[h] = V[0, h // rep]
    rng = np.random.default_rng(1)
    q = rng.standard_normal((8, 16))
    K = rng.standard_normal((1, 4, 16))
    V = rng.standard_normal((1, 4, 16))
    out = oracle.attention(q, K, V, 0.25)
    for h in range(8):
        assert np.array_equal(out[h], V[0, h // 2])


def test_uniform_keys_give_mean_of_values():
    rng = np.random.default_rng(2)
    L = 23
    K = np.repeat(rng.standard_normal((1, 2, 16)), L, axis=0)
    V = rng.standard_normal((L, 2, 16))
    q = rng.standard_normal((6, 16))
    out = oracle.attention(q, K, V, 0.3)
    for h in range(6):
        np.testing.assert_allclose(out[h], V[:, h // 3].mean(axis=0), rtol=0, atol=1e-14)
    # q = 0: every score 0, same mean whatever K is
    K2 = rng.standard_normal((L, 2, 16))
    out2 = oracle.attention(np.zeros((6, 16)), K2, V, 0.3)
    for h in range(6):
        np.testing.assert_allclose(out2[h], V[:, h // 3].mean(axis=0), rtol=0, atol=1e-14)


def test_single_block_brute_force_loops():
    # one sequence inside one block, pool ids [5]; attention by explicit loops
    wl = make_custom([[5]], [13], num_q_heads=4, num_kv_heads=2, head_dim=8,
                     block_size=16, num_blocks=7, seed=11)
    kp, vp = _fill_pool(wl)
    got = oracle.decode(wl.q, kp, vp, wl.block_tables, wl.context_lens, wl.scale, "f32")
    for h in range(4):
        g = h // 2
        sc = []
        for p in range(13):
            dot = 0.0
            for d in range(8):
                dot += float(wl.q[0, h, d]) * float(kp[5, p, g, d])
            sc.append(dot * wl.scale)
        mx = max(sc)
        e = [math.exp(x - mx) for x in sc]
        tot = sum(e)
        for d in range(8):
            ref = sum(e[p] * float(vp[5, p, g, d]) for p in range(13)) / tot
            assert abs(got[0, h, d] - ref) <= 1e-13 * max(1.0, abs(ref))


# ---------------------------------------------------------------- paged == contiguous
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_paged_equals_contiguous_bit_exact(dtype):
    # scattered, out-of-order tables; lengths off block boundaries
    rng = np.random.default_rng(7)
    perm = (rng.permutation(40) + 1).tolist()
    lens = [1, 16, 17, 33, 70, 5]
    tabs, k = [], 0
    for L in lens:
        n = -(-L // 16)
        tabs.append(perm[k:k + n])
        k += n
    wl = make_custom(tabs, lens, dtype=dtype, num_q_heads=8, num_kv_heads=4, head_dim=16,
                     block_size=16, num_blocks=41, seed=4)
    kp, vp = _fill_pool(wl)
    out = oracle.decode(wl.q, kp, vp, wl.block_tables, wl.context_lens, wl.scale, dtype)
    for s in range(len(lens)):
        K, V = _contig(wl, s)
        ref = oracle.attention(oracle.storage_to_f64(wl.q[s], dtype), K, V, wl.scale)
        assert np.array_equal(out[s], ref), s


def test_block_ids_2_0_equals_contiguous_and_relabeling_is_invisible():
    g = _gold("block_ids_2_0.json")
    bs = g["block_size"]
    wl = make_custom([g["table"]], [g["ctx"]], num_q_heads=4, num_kv_heads=2, head_dim=16,
                     block_size=bs, num_blocks=3, seed=9)
    kp, vp = _fill_pool(wl)
    out = oracle.decode(wl.q, kp, vp, wl.block_tables, wl.context_lens, wl.scale, "f32")
    K, V = _contig(wl, 0)
    assert np.array_equal(out[0], oracle.attention(wl.q[0].astype(np.float64), K, V, wl.scale))
    # same logical content under another physical placement
    wl2 = make_custom([[1, 2]], [g["ctx"]], num_q_heads=4, num_kv_heads=2, head_dim=16,
                      block_size=bs, num_blocks=3, seed=9)
    kp2, vp2 = _fill_pool(wl2)
    out2 = oracle.decode(wl2.q, kp2, vp2, wl2.block_tables, wl2.context_lens, wl2.scale, "f32")
    assert np.array_equal(out, out2)


@pytest.mark.parametrize("ctx_a,ctx_b", [(20, 20), (32, 32), (9, 9), (40, 47)])
def test_prefix_shared_tables(ctx_a, ctx_b):
    g = _gold("shared_prefix_tables.json")
    tabs = [g["tables"]["A"], g["tables"]["B"]]
    wl = make_custom(tabs, [ctx_a, ctx_b], num_q_heads=6, num_kv_heads=3, head_dim=16,
                     block_size=16, num_blocks=7, prefix_tokens=g["prefix_tokens"], seed=12)
    q = wl.q.copy()
    q[1] = q[0]
    kp, vp = _fill_pool(wl)
    out = oracle.decode(q, kp, vp, wl.block_tables, wl.context_lens, wl.scale, "f32")
    if ctx_a <= 32 and ctx_a == ctx_b:
        assert np.array_equal(out[0], out[1])
    for s in range(2):
        K, V = _contig(wl, s)
        assert np.array_equal(out[s], oracle.attention(q[s].astype(np.float64), K, V, wl.scale))
    # the shared blocks were written once and hold the prefix rows
    assert np.array_equal(kp[1].reshape(16, -1), wl.k_rows[:16].reshape(16, -1))


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_poison_in_unowned_slots_changes_nothing(dtype):
    rng = np.random.default_rng(3)
    perm = (rng.permutation(20) + 1).tolist()
    lens = [3, 17, 31, 40]
    tabs, k = [], 0
    for L in lens:
        n = -(-L // 16)
        tabs.append(perm[k:k + n] + [0, 0])   # padded with the dummy block
        k += n
    wl = make_custom(tabs, lens, dtype=dtype, num_q_heads=4, num_kv_heads=2, head_dim=16,
                     block_size=16, num_blocks=21, seed=21)
    outs = []
    for kind in ("zero", "nan", "huge"):
        if kind == "zero":
            kp, vp = _fill_pool(wl, zero=True)
        else:
            bits = (POISON_NAN if kind == "nan" else POISON_HUGE)[dtype]
            kp, vp = _fill_pool(wl, bits)
        outs.append(oracle.decode(wl.q, kp, vp, wl.block_tables, wl.context_lens,
                                  wl.scale, dtype))
    assert np.isfinite(outs[0]).all()
    assert np.array_equal(outs[0], outs[1])
    assert np.array_equal(outs[0], outs[2])


def test_ctx0_gives_zeros_and_clamps():
    wl = make_custom([[1, 2], [3]], [0, 16], num_q_heads=2, num_kv_heads=1, head_dim=16,
                     block_size=16, num_blocks=4, seed=1)
    kp, vp = _fill_pool(wl, zero=True)
    out = oracle.decode(wl.q, kp, vp, wl.block_tables, wl.context_lens, wl.scale, "f32")
    assert not out[0].any() and out[1].any()
    # a length past the table is clamped to the table's reach (2 entries x 16)
    far = oracle.decode(wl.q, kp, vp, wl.block_tables, np.array([-5, 500], np.int32),
                        wl.scale, "f32")
    reach = oracle.decode(wl.q, kp, vp, wl.block_tables, np.array([0, 32], np.int32),
                          wl.scale, "f32")
    assert np.array_equal(far, reach)
    assert not far[0].any()


def test_invalid_block_id_excludes_its_tokens():
    wl = make_custom([[1, 2, 3]], [40], num_q_heads=2, num_kv_heads=1, head_dim=16,
                     block_size=16, num_blocks=4, seed=8)
    kp, vp = _fill_pool(wl)
    bad = wl.block_tables.copy()
    bad[0, 1] = 99
    out = oracle.decode(wl.q, kp, vp, bad, wl.context_lens, wl.scale, "f32")
    K, V = _contig(wl, 0)
    keep = np.r_[0:16, 32:40]
    ref = oracle.attention(wl.q[0].astype(np.float64), K[keep], V[keep], wl.scale)
    assert np.array_equal(out[0], ref)


# ---------------------------------------------------------------- split-K identity
@pytest.mark.parametrize("partition", [16, 64, 100, 1000])
def test_split_combine_equals_unsplit(partition):
    rng = np.random.default_rng(partition)
    q = rng.standard_normal((8, 32))
    K = rng.standard_normal((333, 2, 32)) * 3.0
    V = rng.standard_normal((333, 2, 32))
    ms, ls, os_ = oracle.split_partials(q, K, V, 0.2, partition)
    assert len(ms) == -(-333 // partition)
    got = oracle.combine_partials(ms, ls, os_)
    ref = oracle.attention(q, K, V, 0.2)
    np.testing.assert_allclose(got, ref, rtol=1e-13, atol=1e-13)
    # and against the library routine, so the identity is not only self-consistent
    np.testing.assert_allclose(got, _sdpa(q[None], K, V, 0.2)[0], rtol=1e-12, atol=1e-12)


# ---------------------------------------------------------------- causal prefill
def _one_seq_pool(L, Hq, Hkv, hd, seed, dtype="f32"):
    rng = np.random.default_rng(seed)
    nb = -(-L // 16)
    table = (rng.permutation(nb + 3) + 1)[:nb].tolist()
    wl = make_custom([table], [L], dtype=dtype, num_q_heads=Hq, num_kv_heads=Hkv,
                     head_dim=hd, block_size=16, num_blocks=nb + 4, seed=seed)
    kp, vp = _fill_pool(wl)
    return wl, kp, vp


@pytest.mark.parametrize("L,Hq,Hkv", [(1, 2, 1), (37, 8, 4), (70, 6, 2)])
def test_prefill_whole_sequence_equals_causal_sdpa(L, Hq, Hkv):
    wl, kp, vp = _one_seq_pool(L, Hq, Hkv, 16, L)
    rng = np.random.default_rng(L + 1)
    qr = rng.standard_normal((L, Hq, 16)).astype(np.float32)
    out = oracle.prefill(qr, np.array([0, L]), kp, vp, wl.block_tables, wl.context_lens,
                         wl.scale, "f32")
    K, V = _contig(wl, 0)
    ref = _sdpa(qr.astype(np.float64), K, V, wl.scale, causal=True)
    np.testing.assert_allclose(out, ref, rtol=1e-12, atol=1e-12)


def test_prefill_chunk_matches_full_rows_and_last_row_matches_decode():
    L, Hq, Hkv = 75, 8, 2
    wl, kp, vp = _one_seq_pool(L, Hq, Hkv, 16, 5)
    rng = np.random.default_rng(6)
    qr = rng.standard_normal((L, Hq, 16)).astype(np.float32)
    full = oracle.prefill(qr, np.array([0, L]), kp, vp, wl.block_tables, wl.context_lens,
                          wl.scale, "f32")
    for n in (1, 16, 30):
        chunk = oracle.prefill(qr[L - n:], np.array([0, n]), kp, vp, wl.block_tables,
                               wl.context_lens, wl.scale, "f32")
        np.testing.assert_allclose(chunk, full[L - n:], rtol=1e-14, atol=1e-14)
    dec = oracle.decode(qr[L - 1:], kp, vp, wl.block_tables, wl.context_lens, wl.scale, "f32")
    np.testing.assert_allclose(full[L - 1], dec[0], rtol=1e-13, atol=1e-13)


def test_prefill_rows_before_position_zero_are_zero():
    wl, kp, vp = _one_seq_pool(5, 2, 1, 16, 3)
    qr = np.ones((8, 2, 16), dtype=np.float32)
    out = oracle.prefill(qr, np.array([0, 8]), kp, vp, wl.block_tables, wl.context_lens,
                         wl.scale, "f32")
    assert not out[:3].any()
    assert np.isfinite(out).all() and out[3:].any()


def test_index_errors_worked_example():
    # pool of 64 blocks x 16 slots = 1024 slots, counted by hand:
    # slots: -1 (negative), 3 three times (two duplicates), 1024 and 5000 (past
    # the pool), 100 and 1023 (fine)
    slots = [-1, 3, 3, 3, 1024, 100, 5000, 1023]
    # tables: row 0 needs 3 blocks for ctx 40 and its third entry (70) is past
    # the pool; row 1 needs 2 blocks for ctx 20, its second entry is negative;
    # row 2's ctx 49 is past its 3-block reach (48), its entries are fine;
    # row 3's ctx -2 is negative and needs no block; row 4 needs 1 block for
    # ctx 1 and the bad entry after it is never needed
    tables = [[0, 1, 70], [2, -4, 9], [5, 6, 7], [-1, -1, -1], [8, 99, 99]]
    ctx = [40, 20, 49, -2, 1]
    assert oracle.index_errors(slots, tables, ctx, 64, 16) == {
        "negative_slots": 1, "slots_past_pool": 2, "duplicate_slots": 2,
        "invalid_table_entries": 2, "context_past_table": 2}
    assert oracle.index_errors(None, tables, ctx, 64, 16)["duplicate_slots"] == 0
    assert oracle.index_errors(slots, None, None, 64, 16)["invalid_table_entries"] == 0


def test_index_errors_on_shared_prefix_tables():
    # "nano-vLLM" "How it works": two sequences whose tables [1, 2, 5] and
    # [1, 2, 6] share a 32-token prompt (block 16). Writing the prompt once and
    # each sequence's own tokens is clean; writing the prompt for both
    # sequences sends 32 tokens to slots already named: 32 duplicates.
    tables = np.array([[1, 2, 5], [1, 2, 6]], np.int32)
    own = oracle.slot_mapping(tables, np.array([32, 32]), np.array([0, 8, 16]), 16, 8)
    prompt = oracle.slot_mapping(tables[:1], np.array([0]), np.array([0, 32]), 16, 8)
    clean = np.concatenate([prompt, own])
    assert oracle.index_errors(clean, tables, [40, 40], 8, 16) == {
        "negative_slots": 0, "slots_past_pool": 0, "duplicate_slots": 0,
        "invalid_table_entries": 0, "context_past_table": 0}
    twice = oracle.slot_mapping(tables, np.array([0, 0]), np.array([0, 40, 80]), 16, 8)
    assert oracle.index_errors(twice, tables, [40, 40], 8, 16)["duplicate_slots"] == 32
