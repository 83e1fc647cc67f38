"""GPU parity of the debug index check (pkv_validate) against the oracle's
definition of the same counts, and the PKV_DEBUG checks of the binding."""

import functools

import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_scatter_amd as pkv
from workloads import make_custom, make_workload

from _gpu_util import note, to_dev, to_host

pytestmark = pytest.mark.gpu


@functools.lru_cache(maxsize=1)
def _wl(cfg):
    return make_workload(cfg)


def _planted(seed, T, S, maxb, nb, bs):
    """Seeded slots and tables with every kind of error planted at random."""
    rng = np.random.default_rng(seed)
    n_slots = nb * bs
    slots = rng.integers(0, n_slots, T).astype(np.int64)
    kind = rng.integers(0, 10, T)
    slots[kind == 0] = -1 - rng.integers(0, 5, (kind == 0).sum())
    slots[kind == 1] = n_slots + rng.integers(0, 1000, (kind == 1).sum())
    dup_src = rng.integers(0, max(T, 1), (kind == 2).sum())
    slots[kind == 2] = slots[dup_src]   # duplicates of other tokens (or of themselves)
    slots = np.clip(slots, -(2**31), 2**31 - 1).astype(np.int32)
    tables = rng.integers(0, nb, (S, maxb)).astype(np.int32)
    bad = rng.random((S, maxb)) < 0.05
    tables[bad] = rng.choice(np.array([-7, -1, nb, nb + 3, 2**31 - 1], np.int32), bad.sum())
    ctx = rng.integers(0, maxb * bs + 1, S).astype(np.int32)
    out = rng.random(S)
    ctx[out < 0.05] = -rng.integers(1, 100, (out < 0.05).sum())
    ctx[out > 0.95] = maxb * bs + rng.integers(1, 100, (out > 0.95).sum())
    return slots, tables, ctx


@pytest.mark.parametrize("seed,T,S,maxb,nb,bs", [
    (0, 1, 1, 1, 1, 1), (1, 257, 3, 5, 64, 16), (2, 5000, 77, 33, 1000, 16),
    (3, 70001, 1025, 129, 4096, 64), (4, 300, 40, 9, 7, 256)])
def test_counts_match_the_oracle(seed, T, S, maxb, nb, bs):
    slots, tables, ctx = _planted(seed, T, S, maxb, nb, bs)
    ref = oracle.index_errors(slots, tables, ctx, nb, bs)
    note(f"validate seed {seed}: {T} slots, {S} tables; oracle {ref}")
    got = pkv.validate(to_dev(slots), to_dev(tables), to_dev(ctx), num_blocks=nb, block_size=bs)
    assert got == ref
    assert sum(ref.values()) > 0 or T < 10


def test_each_part_alone_and_the_workspace_left_zero():
    slots, tables, ctx = _planted(9, 4000, 50, 17, 300, 16)
    ref = oracle.index_errors(slots, tables, ctx, 300, 16)
    ws = torch.zeros((pkv.load().pkv_validate_workspace_bytes(300, 16) + 3) // 4,
                     dtype=torch.int32, device="cuda")
    s_only = pkv.validate(to_dev(slots), num_blocks=300, block_size=16, workspace=ws)
    assert not to_host(ws).any(), "bitmap cleared after the call"
    t_only = pkv.validate(block_tables=to_dev(tables), context_lens=to_dev(ctx), num_blocks=300,
                          block_size=16)
    again = pkv.validate(to_dev(slots), num_blocks=300, block_size=16, workspace=ws)
    assert s_only == again, "one workspace serves consecutive calls"
    for k in ("negative_slots", "slots_past_pool", "duplicate_slots"):
        assert s_only[k] == ref[k] and t_only[k] == 0
    for k in ("invalid_table_entries", "context_past_table"):
        assert t_only[k] == ref[k] and s_only[k] == 0


@pytest.mark.parametrize("cfg", [2, 5])
def test_the_pages_workloads_are_clean(cfg):
    """The configs' own writes and tables hold none of these errors."""
    wl = _wl(cfg)
    slots = pkv.slot_mapping(to_dev(wl.w_tables), to_dev(wl.w_first_pos), to_dev(wl.w_cu),
                             int(wl.w_cu[-1]), wl.block_size, wl.num_blocks)
    got = pkv.validate(slots, to_dev(wl.block_tables), to_dev(wl.context_lens),
                       num_blocks=wl.num_blocks, block_size=wl.block_size)
    assert got == oracle.index_errors(to_host(slots), wl.block_tables, wl.context_lens,
                                      wl.num_blocks, wl.block_size)
    assert not any(got.values()), got


def test_pkv_debug_raises_on_caller_errors(monkeypatch):
    monkeypatch.setenv("PKV_DEBUG", "1")
    wl = make_custom([[1, 2, 0, 0], [3, 4, 5, 0]], [20, 40], num_q_heads=4, num_kv_heads=2,
                     head_dim=64, block_size=16, num_blocks=8)
    kp = torch.zeros(wl.pool_shape, device="cuda")
    vp = torch.zeros_like(kp)
    k = torch.ones(3, 2, 64, device="cuda")
    with pytest.raises(pkv.PkvError, match="duplicate_slots 1"):
        pkv.write(k, k, to_dev(np.array([5, 9, 5], np.int32)), kp, vp)
    with pytest.raises(pkv.PkvError, match="slots_past_pool 1"):
        pkv.write(k, k, to_dev(np.array([5, 9, 128], np.int32)), kp, vp)
    pkv.write(k, k, to_dev(np.array([5, 9, -1], np.int32)), kp, vp)   # a skipped row is fine
    q = torch.ones(2, 4, 64, device="cuda")
    tb, ctx = to_dev(wl.block_tables), to_dev(wl.context_lens)
    pkv.decode(q, kp, vp, tb, ctx, wl.scale, 40)
    bad = wl.block_tables.copy()
    bad[1, 2] = 8                                              # needed, past the pool
    with pytest.raises(pkv.PkvError, match="invalid_table_entries 1"):
        pkv.decode(q, kp, vp, to_dev(bad), ctx, wl.scale, 40)
    with pytest.raises(pkv.PkvError, match="context_past_table 1"):
        pkv.decode_step(q, k[:2], k[:2], kp, vp, tb, to_dev(np.array([20, 65], np.int32)),
                        wl.scale, 64)
    monkeypatch.setenv("PKV_DEBUG", "0")
    pkv.decode(q, kp, vp, to_dev(bad), ctx, wl.scale, 40)      # unchecked: tokens masked
