"""GPU parity of the slot mapping and the KV write: bit-exact against the oracle."""

import functools

import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_scatter_amd as pkv
from workloads import make_custom, make_workload

from _gpu_util import PoolCase, bits, note, to_dev, to_host

pytestmark = pytest.mark.gpu


@functools.lru_cache(maxsize=2)
def _wl(cfg):
    return make_workload(cfg)


@pytest.mark.parametrize("cfg", [1, 2, 3, 4, 5])
def test_bulk_write_bit_exact(cfg):
    wl = _wl(cfg)
    pc = PoolCase(wl, fill="nan")
    got_slots = to_host(pc.slots)
    assert np.array_equal(got_slots, pc.ref_slots()), "slot mapping"
    kref, vref = pc.ref_pools()
    note(f"{wl.name}: comparing pools bit for bit")
    assert np.array_equal(bits(to_host(pc.k_pool)), bits(kref)), "k_pool"
    assert np.array_equal(bits(to_host(pc.v_pool)), bits(vref)), "v_pool"


@pytest.mark.parametrize("cfg", [4, 5])
def test_paired_decode_step_write_bit_exact(cfg):
    """Bulk fill of positions 0..ctx-2, then the step write of position ctx-1
    (1 token per sequence): the pools equal the oracle's full write."""
    wl = _wl(cfg)
    pc = PoolCase(wl, fill="nan", exclude_last=True)
    tabs, first, cu, rows = wl.step_segments()
    note(f"{wl.name}: step slot mapping + write of {int(cu[-1])} tokens")
    slots = pkv.slot_mapping(to_dev(tabs), to_dev(first), to_dev(cu), int(cu[-1]),
                             wl.block_size, wl.num_blocks)
    pkv.write(to_dev(wl.k_rows[rows]), to_dev(wl.v_rows[rows]), slots, pc.k_pool, pc.v_pool)
    torch.cuda.synchronize()
    ref_slots = oracle.slot_mapping(tabs, first, cu, wl.block_size, wl.num_blocks)
    assert np.array_equal(to_host(slots), ref_slots)
    full = PoolCase.__new__(PoolCase)
    full.wl, full.kp0, full.vp0 = wl, pc.kp0, pc.vp0
    full.tabs, full.first, full.cu, full.rows = wl.bulk_segments()
    full._ref_pools = None
    kref, vref = full.ref_pools()
    assert np.array_equal(bits(to_host(pc.k_pool)), bits(kref))
    assert np.array_equal(bits(to_host(pc.v_pool)), bits(vref))


@pytest.mark.parametrize("dtype,hkv,hd", [("f32", 1, 6), ("bf16", 1, 6), ("bf16", 3, 8),
                                          ("f32", 2, 64)])
def test_write_element_path_and_skipped_slots(dtype, hkv, hd):
    """Rows that are not a multiple of 16 bytes take the element path; slots
    outside the pool are skipped."""
    rng = np.random.default_rng(hd)
    nb, bs = 6, 4
    T = 10
    if dtype == "f32":
        pool = rng.standard_normal((nb, bs, hkv, hd)).astype(np.float32)
        new = rng.standard_normal((T, hkv, hd)).astype(np.float32)
    else:
        pool = rng.integers(0, 65535, (nb, bs, hkv, hd)).astype(np.uint16)
        new = rng.integers(0, 65535, (T, hkv, hd)).astype(np.uint16)
    slots = np.array([3, -1, 23, 24, 0, 1000, 7, -5, 12, 22], dtype=np.int32)
    kp, vp = to_dev(pool), to_dev(pool.copy())
    note(f"write element path {dtype} hkv={hkv} hd={hd}")
    pkv.write(to_dev(new), to_dev(new[::-1].copy()), to_dev(slots), kp, vp)
    torch.cuda.synchronize()
    kref, vref = oracle.write(pool, pool.copy(), new, new[::-1].copy(), slots)
    assert np.array_equal(bits(to_host(kp)), bits(kref))
    assert np.array_equal(bits(to_host(vp)), bits(vref))


def test_slot_mapping_edges():
    # out-of-order blocks [2, 0]; a table entry out of range; positions past the table
    tabs = np.array([[2, 0, 0], [5, 99, 1], [3, 4, -2]], dtype=np.int32)
    first = np.array([0, 0, 6], dtype=np.int32)
    cu = np.array([0, 7, 19, 24], dtype=np.int32)
    note("slot mapping edge cases")
    got = pkv.slot_mapping(to_dev(tabs), to_dev(first), to_dev(cu), 24, 4, 8)
    torch.cuda.synchronize()
    ref = oracle.slot_mapping(tabs, first, cu, 4, 8)
    assert np.array_equal(to_host(got), ref)
    assert ref[:7].tolist() == [8, 9, 10, 11, 0, 1, 2]


def test_shared_prefix_written_once():
    wl = make_custom([[1, 2, 5], [1, 2, 6]], [40, 47], num_q_heads=6, num_kv_heads=3,
                     head_dim=64, block_size=16, num_blocks=8, prefix_tokens=32, seed=1)
    pc = PoolCase(wl)
    kref, vref = pc.ref_pools()
    assert np.array_equal(bits(to_host(pc.k_pool)), bits(kref))
    assert np.array_equal(bits(to_host(pc.v_pool)), bits(vref))
