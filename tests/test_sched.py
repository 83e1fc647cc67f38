"""The native scheduler (include/pkv_sched.h) against the engine runs the
"Build a Mini vLLM" page prints for its 24-request workload (section 5's
make_workload, numpy seed 7): sections 6, 7 and 8."""

import numpy as np
import pytest

import paged_kv_cache_scatter_amd as pkv
from paged_kv_cache_scatter_amd.sched import Scheduler
from workloads import engine_requests


def _run(num_blocks, continuous=True, max_batch=8):
    s = Scheduler(num_blocks, 16, max_batch, continuous, max_blocks_per_seq=16)
    for r in engine_requests():
        s.submit(*r)
    return s, s.run()


def test_continuous_vs_static_steps():
    """Section 7: 891 tokens either way; static 187 steps, continuous 128."""
    sc, st_c = _run(96, True)
    ss, st_s = _run(96, False)
    assert st_c["tokens_generated"] == 891 and st_s["tokens_generated"] == 891
    assert st_c["requests_done"] == 24 and st_s["requests_done"] == 24
    assert st_s["steps"] == 187
    assert st_c["steps"] == 128


def test_memory_waste_naive_vs_paged():
    """Section 6: wasted KV memory -- naive slabs 48%, paged blocks 13%."""
    s, _ = _run(96, True)
    h = s.history()
    waste_naive = 1 - h["used"].sum() / h["naive"].sum()
    waste_paged = 1 - h["used"].sum() / h["allocated"].sum()
    assert round(100 * waste_naive) == 48, waste_naive
    assert round(100 * waste_paged) == 13, waste_paged
    # block-tail fragmentation is under one block per running sequence
    assert np.all(h["allocated"] - h["used"] <= 15 * h["running"])


def test_starved_pool_preempts_and_completes():
    """Section 8: a 24-block (384-token) pool completes all 24 requests with
    16 preemptions."""
    _, st = _run(24, True)
    assert st["requests_done"] == 24
    assert st["preemptions"] == 16


def test_occupancy_never_exceeds_batch_or_pool():
    s, st = _run(24, True)
    h = s.history()
    assert h["running"].max() <= 8
    assert h["allocated"].max() <= 24 * 16
    assert np.all(h["used"] <= h["allocated"])


def test_submit_and_capacity_errors():
    s = Scheduler(4, 16, 8, True, max_blocks_per_seq=2)
    with pytest.raises(pkv.PkvError) as e:
        s.submit(0, 20, 10, 20)           # 40 tokens > 2 blocks of 16
    assert e.value.status_name == "PKV_ERR_CAPACITY"
    with pytest.raises(pkv.PkvError):
        s.submit(1, 0, 10, 5)             # empty prompt
    s.submit(2, 10, 10, 5)
    with pytest.raises(pkv.PkvError):
        s.submit(2, 10, 10, 5)            # rid reused
    tiny = Scheduler(1, 16, 8, True, max_blocks_per_seq=8)
    tiny.submit(0, 40, 10, 5)            # needs 3 blocks to be admitted, the pool has 1
    with pytest.raises(pkv.PkvError) as e:
        tiny.step()
    assert e.value.status_name == "PKV_ERR_CAPACITY"
