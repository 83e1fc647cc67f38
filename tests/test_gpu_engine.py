"""The scheduler driving the kernels: the page's 24-request workload in a
starved 24-block pool (16 preemptions, blocks reused across requests) and in
a 96-block pool. Every decode output of every step is checked against plain
contiguous attention over that request's rows (the oracle), and so is every
prefill row (the prompt at admission, and prompt plus generated tokens after a
recompute preemption), so the paged pool must stay consistent through
admission, recompute preemption and reuse."""

import numpy as np
import pytest

import oracle
from paged_kv_cache_scatter_amd.sched import run_engine
from workloads import TokenRows, engine_requests

from _gpu_util import BF16_ABS_TOL, note, to_host

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("num_blocks,continuous,preemptions", [(24, True, 16), (96, True, 0),
                                                               (96, False, 0)])
def test_engine_runs_the_kernels(num_blocks, continuous, preemptions):
    reqs = engine_requests()
    rows = TokenRows(len(reqs), 128, num_q_heads=8, num_kv_heads=2, head_dim=64, dtype="bf16")
    scale = 1.0 / np.sqrt(64)
    worst = [0.0, 0]

    def check(step, out):
        got = oracle.storage_to_f64(to_host(out), "bf16")
        for i, (rid, pos) in enumerate(zip(step["decode_rid"], step["decode_pos"])):
            K = oracle.storage_to_f64(rows.k[rid, :pos + 1], "bf16")
            V = oracle.storage_to_f64(rows.v[rid, :pos + 1], "bf16")
            q = oracle.storage_to_f64(rows.q[rid, pos], "bf16")
            ref = oracle.attention(q, K, V, scale)
            err = float(np.abs(got[i] - ref).max())
            worst[0] = max(worst[0], err)
            worst[1] += 1
            assert err <= BF16_ABS_TOL, f"request {rid} position {pos}: {err}"

    pworst = [0.0, 0]

    def check_prefill(step, out, rid_rows, pos_rows):
        got = oracle.storage_to_f64(to_host(out), "bf16")
        for i, (rid, pos) in enumerate(zip(rid_rows, pos_rows)):
            K = oracle.storage_to_f64(rows.k[rid, :pos + 1], "bf16")
            V = oracle.storage_to_f64(rows.v[rid, :pos + 1], "bf16")
            q = oracle.storage_to_f64(rows.q[rid, pos], "bf16")
            err = float(np.abs(got[i] - oracle.attention(q, K, V, scale)).max())
            pworst[0] = max(pworst[0], err)
            pworst[1] += 1
            assert err <= BF16_ABS_TOL, f"prefill of request {rid} position {pos}: {err}"

    note(f"engine: {num_blocks} blocks, continuous={continuous}")
    st = run_engine(reqs, rows, num_blocks, continuous=continuous, max_blocks_per_seq=16,
                    check=check, check_prefill=check_prefill)
    note(f"engine stats {st}; {worst[1]} decode rows checked, worst error {worst[0]:.2e}; "
         f"{pworst[1]} prefill rows checked, worst error {pworst[0]:.2e}")
    assert pworst[1] > 0
    assert st["requests_done"] == 24 and st["preemptions"] == preemptions
    if not preemptions:
        assert st["tokens_generated"] == 891   # a re-prefill after preemption adds tokens
