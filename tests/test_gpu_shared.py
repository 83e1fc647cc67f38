"""GPU parity of the shared-prefix decode (pkv_decode_shared): groups of
sequences whose tables begin with the same prompt blocks attend them in one
shared pass, their tails in the decode kernel; the result is the decode of
every sequence, checked against the oracle and against pkv_decode."""

import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_scatter_amd as pkv
from workloads import make_shared, make_workload
from workloads.gen import BF16, F32

from _gpu_util import PoolCase, bits, check_close, note, out_f64, to_dev, to_host

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _always_share(monkeypatch):
    """These cases are far smaller than the 64 MiB of saved reads at which the
    planner starts using the shared pass; run the shared pass on them anyway
    (the planner's choice itself is checked in test_default_rule_*)."""
    monkeypatch.setenv("PKV_SHARED_MIN_SAVED_BYTES", "0")


def _groups(wl, extra=0):
    """group_start [G+1] and prefix_lens [G] of the workload's groups (every
    sequence in one group; ``extra`` is added to each prefix length)."""
    gs = [0]
    pl = []
    for (s0, s1, p) in wl.groups:
        assert s0 == gs[-1]
        gs.append(s1)
        pl.append(p + extra)
    if not wl.groups:
        gs = [0, wl.num_seqs]
        pl = [0]
    assert gs[-1] == wl.num_seqs
    return np.array(gs, np.int32), np.array(pl, np.int32)


def _shared(pc, gs, pl, partition=0, max_tail=-1, max_prefix=None):
    wl = pc.wl
    sizes = np.diff(gs)
    mp = int(pl.max()) if max_prefix is None else max_prefix
    mp = min(mp, pc.max_ctx)
    note(f"{wl.name}: pkv_decode_shared groups={len(pl)} max_group={sizes.max()} "
         f"max_prefix={mp} max_tail={max_tail} partition={partition or 'auto'}")
    out = pkv.decode_shared(pc.q, pc.k_pool, pc.v_pool, pc.tables, pc.ctx, to_dev(gs),
                            to_dev(pl), wl.scale, pc.max_ctx, int(sizes.max()), mp,
                            max_tail_len=max_tail, partition=partition)
    torch.cuda.synchronize()
    return out


def _max_tail(wl, pl, gs):
    t = 0
    for i in range(len(pl)):
        for s in range(gs[i], gs[i + 1]):
            c = int(wl.context_lens[s])
            p = (int(pl[i]) // wl.block_size) * wl.block_size
            t = max(t, c - min(c, p))
    return t


def _check(wl, extra=0, partition=0, exact_tail=True, fill="nan"):
    pc = PoolCase(wl, fill=fill)
    gs, pl = _groups(wl, extra)
    mt = _max_tail(wl, pl, gs) if exact_tail else -1
    got = out_f64(_shared(pc, gs, pl, partition, mt), wl.dtype)
    ref = pc.ref_decode()
    err = check_close(got, ref, wl.dtype, wl.name)
    note(f"{wl.name}: worst error {err:.3e}")
    return pc, got


def test_smollm2_shape_shared_32_token_prompt():
    """Every table of the 30-sequence SmolLM2-shape workload starts with the
    same two blocks (the 32-token prompt written once); a sequence shorter
    than 32 reads only its part."""
    wl = make_workload(2)
    assert wl.groups == [(0, 30, 32)]
    _check(wl)


def test_500_token_shared_prompt_fp32():
    """30 users of a ~500-token system prompt: its 31 full blocks (496 tokens)
    are shared, each user's own tail is the prompt's last 4 tokens plus a
    question and answer of 8..200 tokens (SmolLM2-135M shape, fp32)."""
    wl = make_shared([30], [496], ("uniform", 12, 204), dtype=F32, num_q_heads=9,
                     num_kv_heads=3, head_dim=64, seed=21, name="smollm2-500-shared")
    pc, got = _check(wl)
    # and the same numbers as the plain decode within fp32 rounding
    plain = out_f64(pc.decode(), wl.dtype)
    check_close(got, plain, wl.dtype, "vs pkv_decode")


@pytest.mark.parametrize("hq,hkv,hd", [(64, 8, 128), (32, 8, 64), (8, 8, 128), (12, 2, 64)])
def test_bf16_groups(hq, hkv, hd):
    """Several groups of different sizes and prompt lengths (one without a
    prompt, one of a single member), 70B-layer and 1B shapes."""
    wl = make_shared([5, 1, 7, 3, 2], [256, 64, 0, 1024, 16], ("uniform", 0, 300),
                     dtype=BF16, num_q_heads=hq, num_kv_heads=hkv, head_dim=hd, seed=hq + hd,
                     name=f"bf16-groups-{hq}x{hkv}x{hd}")
    _check(wl)


@pytest.mark.parametrize("hq,hkv,hd", [(9, 3, 64), (4, 2, 128), (8, 1, 64)])
def test_fp32_groups(hq, hkv, hd):
    wl = make_shared([4, 9, 2], [128, 48, 320], ("uniform", 1, 150), dtype=F32,
                     num_q_heads=hq, num_kv_heads=hkv, head_dim=hd, seed=3 * hq + hd,
                     name=f"fp32-groups-{hq}x{hkv}x{hd}")
    _check(wl)


def test_large_group_several_row_tiles():
    """40 members x 8 heads = 320 (member, head) rows: three row tiles of the
    shared pass over a 2048-token prompt (70B-layer shape)."""
    wl = make_shared([40], [2048], ("uniform", 1, 512), dtype=BF16, num_q_heads=64,
                     num_kv_heads=8, head_dim=128, seed=5, name="bf16-40x2048")
    _check(wl)


def test_short_members_and_unaligned_prefix_lengths():
    """Members whose context ends inside the prompt read only their part of it
    (C13); prefix lengths that are not whole blocks are rounded down."""
    wl = make_shared([6, 5], [160, 96], ("uniform", 1, 80), dtype=BF16, num_q_heads=16,
                     num_kv_heads=2, head_dim=128, short_members=3, seed=8, name="short")
    _check(wl, extra=7)
    wl = make_shared([6, 5], [160, 96], ("uniform", 1, 80), dtype=F32, num_q_heads=6,
                     num_kv_heads=3, head_dim=64, short_members=2, seed=9, name="short-fp32")
    _check(wl, extra=15)


@pytest.mark.parametrize("bs", [1, 8, 32, 64])
def test_block_sizes(bs):
    wl = make_shared([4, 3], [8 * 64, 4 * 64], ("uniform", 1, 100), dtype=BF16,
                     num_q_heads=8, num_kv_heads=2, head_dim=64, block_size=bs, seed=bs,
                     name=f"bs{bs}")
    _check(wl)


@pytest.mark.parametrize("partition", [0, 64, 256])
def test_partitions_and_loose_tail_bound(partition):
    wl = make_shared([8, 8], [512, 256], ("uniform", 1, 700), dtype=BF16, num_q_heads=32,
                     num_kv_heads=8, head_dim=64, seed=11, name="partitions")
    _check(wl, partition=partition)
    _check(wl, partition=partition, exact_tail=False)


def test_garbage_pool_is_invisible():
    """Unowned slots at 1e30 and at NaN give bit-identical results."""
    wl = make_shared([5, 4], [128, 64], ("uniform", 1, 90), dtype=BF16, num_q_heads=16,
                     num_kv_heads=4, head_dim=128, seed=13, name="garbage")
    outs = []
    for fill in ("nan", "huge"):
        pc = PoolCase(wl, fill=fill)
        gs, pl = _groups(wl)
        outs.append(to_host(_shared(pc, gs, pl)))
    assert np.array_equal(bits(outs[0]), bits(outs[1]))


def test_invalid_block_in_prompt_is_excluded():
    """An out-of-range id among the shared blocks removes those tokens for
    every member, as in pkv_decode."""
    wl = make_shared([6], [256], ("uniform", 1, 60), dtype=F32, num_q_heads=6,
                     num_kv_heads=3, head_dim=64, seed=17, name="bad-id")
    wl.block_tables[:, 3] = wl.num_blocks + 9
    pc = PoolCase(wl)
    gs, pl = _groups(wl)
    got = out_f64(_shared(pc, gs, pl), wl.dtype)
    check_close(got, pc.ref_decode(), wl.dtype, "bad id")


def test_empty_and_prompt_only_members():
    """Members of length 0 get zeros; members whose context is exactly the
    prompt have an empty tail (only the shared pass's partials)."""
    wl = make_shared([5], [128], ("uniform", 0, 0), dtype=BF16, num_q_heads=8,
                     num_kv_heads=1, head_dim=128, seed=19, name="prompt-only")
    wl.context_lens[1] = 0
    wl.context_lens[2] = 64
    pc = PoolCase(wl)
    gs, pl = _groups(wl)
    got = out_f64(_shared(pc, gs, pl, max_tail=0), wl.dtype)
    ref = pc.ref_decode()
    assert not got[1].any()
    check_close(got, ref, wl.dtype, "prompt-only")


def test_no_groups_is_plain_decode():
    """num_groups == 0 (and prompts shorter than a block) run pkv_decode itself."""
    wl = make_workload(4, num_seqs=16)
    pc = PoolCase(wl)
    plain = to_host(pc.decode())
    out = pkv.decode_shared(pc.q, pc.k_pool, pc.v_pool, pc.tables, pc.ctx,
                            to_dev(np.zeros(1, np.int32)), to_dev(np.zeros(0, np.int32)),
                            wl.scale, pc.max_ctx, 1, 0)
    torch.cuda.synchronize()
    assert np.array_equal(bits(to_host(out)), bits(plain))
    gs = np.array([0, 16], np.int32)
    out = pkv.decode_shared(pc.q, pc.k_pool, pc.v_pool, pc.tables, pc.ctx, to_dev(gs),
                            to_dev(np.array([8], np.int32)), wl.scale, pc.max_ctx, 16, 8)
    torch.cuda.synchronize()
    assert np.array_equal(bits(to_host(out)), bits(plain))


def test_70b_layer_64_users_of_one_prompt():
    """Full size: 64 sequences of the 70B-layer shape sharing a 4096-token
    prompt with own tails of 1..4096 tokens; every sequence against the
    oracle (and against pkv_decode)."""
    wl = make_shared([64], [4096], ("uniform", 1, 4096), dtype=BF16, num_q_heads=64,
                     num_kv_heads=8, head_dim=128, seed=23, name="70b-64x4096-shared")
    pc = PoolCase(wl)
    gs, pl = _groups(wl)
    got = out_f64(_shared(pc, gs, pl, max_tail=_max_tail(wl, pl, gs)), wl.dtype)
    err = check_close(got, pc.ref_decode(), wl.dtype, "vs oracle")
    plain = out_f64(pc.decode(), wl.dtype)
    check_close(got, plain, wl.dtype, "vs pkv_decode")
    note(f"{wl.name}: all 64 sequences, max error {err:.3e}")


@pytest.mark.parametrize("dtype,hd,hkv,hq", [(BF16, 128, 1, 8), (BF16, 128, 8, 64), (F32, 64, 2, 8)])
def test_stream_k_tails(dtype, hd, hkv, hq):
    """Tails long enough for stream-K ranges (at least 256 KiB of K/V per range
    at the longest tail): three groups with prompts of 1024, 2048 and 512
    tokens; members of length 0, members whose context is exactly the prompt
    (empty tail: only the shared pass's partials) or inside it, and tails up
    to 6000 tokens laid end to end. Every sequence against the oracle."""
    wl = make_shared([20, 30, 14], [1024, 2048, 512], ("uniform", 1, 6000), dtype=dtype,
                     num_q_heads=hq, num_kv_heads=hkv, head_dim=hd, seed=41 + hkv,
                     name=f"stream-k tails {dtype} hd{hd} hkv{hkv}")
    wl.context_lens[1] = 0
    wl.context_lens[2] = 1024
    wl.context_lens[25] = 2048
    wl.context_lens[26] = 700
    wl.context_lens[60] = 512
    pc = PoolCase(wl)
    gs, pl = _groups(wl)
    mt = _max_tail(wl, pl, gs)
    assert pkv.decode_schedule(wl.num_seqs, hq, mt, pc.k_pool) == "stream_k"
    got = out_f64(_shared(pc, gs, pl, max_tail=mt), wl.dtype)
    assert not got[1].any()
    err = check_close(got, pc.ref_decode(), wl.dtype, wl.name)
    note(f"{wl.name}: all {wl.num_seqs} sequences, max error {err:.3e}")


def test_default_rule_runs_plain_decode_at_the_pages_scale(monkeypatch):
    """With the default bound, 30 users of a 496-token shared prompt at the
    SmolLM2-135M shape (at most 22 MB of reads saved) run plain decode: the
    same bits as pkv_decode; with the bound at 0 they take the shared pass and
    stay within tolerance of the oracle."""
    monkeypatch.delenv("PKV_SHARED_MIN_SAVED_BYTES")
    wl = make_shared([30], [496], ("uniform", 12, 204), dtype=F32, num_q_heads=9,
                     num_kv_heads=3, head_dim=64, seed=21, name="smollm2-500-shared")
    pc = PoolCase(wl)
    gs, pl = _groups(wl)
    plain = to_host(pc.decode())
    got = to_host(_shared(pc, gs, pl, max_tail=_max_tail(wl, pl, gs)))
    assert np.array_equal(bits(got), bits(plain))
    monkeypatch.setenv("PKV_SHARED_MIN_SAVED_BYTES", "0")
    shared = out_f64(_shared(pc, gs, pl, max_tail=_max_tail(wl, pl, gs)), wl.dtype)
    check_close(shared, pc.ref_decode(), wl.dtype, "forced shared pass")
