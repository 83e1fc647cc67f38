"""The seeded input generator: determinism and the structure each config promises."""

import numpy as np
import pytest

from workloads import CONFIGS, make_workload


def _needed(wl, s):
    return wl.block_tables[s, : -(-int(wl.context_lens[s]) // wl.block_size)]


@pytest.mark.parametrize("cfg", [1, 2, 3])
def test_deterministic(cfg):
    a, b = make_workload(cfg), make_workload(cfg)
    for f in ("context_lens", "block_tables", "k_rows", "v_rows", "q"):
        assert np.array_equal(getattr(a, f), getattr(b, f)), f


@pytest.mark.parametrize("cfg,S", [(1, None), (2, None), (3, None), (4, 24), (5, 6)])
def test_structure(cfg, S):
    spec = CONFIGS[cfg]
    wl = make_workload(cfg, num_seqs=S)
    lens = wl.context_lens
    kind = spec.ctx_dist[0]
    if kind == "uniform":
        assert lens.min() >= spec.ctx_dist[1] and lens.max() <= spec.ctx_dist[2]
    elif kind == "const":
        assert (lens == spec.ctx_dist[1]).all()
    else:
        assert lens.min() >= spec.ctx_dist[1] and lens.max() < spec.ctx_dist[2]
    assert wl.block_tables.shape == (wl.num_seqs, spec.max_blocks_per_seq)
    assert lens.max() <= spec.max_blocks_per_seq * spec.block_size
    owned = []
    for s in range(wl.num_seqs):
        need = _needed(wl, s)
        assert 0 not in need, "block 0 is the never-assigned dummy"
        assert (need < spec.num_blocks).all()
        assert not wl.block_tables[s, len(need):].any(), "padding is the dummy block"
        owned.extend(need[spec.prefix_blocks:].tolist())
        if spec.prefix_blocks:
            assert wl.block_tables[s, :spec.prefix_blocks].tolist() == [1, 2]
        assert len(wl.seq_rows[s]) == lens[s]
    assert len(owned) == len(set(owned)), "no block belongs to two sequences"
    assert wl.k_rows.shape[0] == int(wl.w_cu[-1])
    assert wl.q.shape == (wl.num_seqs, spec.num_q_heads, spec.head_dim)


def test_llama1b_8x2048_reads_exactly_32_mib():
    wl = make_workload(3)
    assert wl.kv_bytes_per_call() == 33554432


def test_paired_write_split_covers_every_row_once():
    wl = make_workload(4, num_seqs=10)
    _, _, cu_b, rows_b = wl.bulk_segments(exclude_last=True)
    _, first, cu_s, rows_s = wl.step_segments()
    allrows = np.sort(np.concatenate([rows_b, rows_s]))
    assert np.array_equal(allrows, np.arange(wl.k_rows.shape[0]))
    assert (first == wl.context_lens - 1).all()
    assert int(cu_b[-1]) == wl.total_ctx - wl.num_seqs


def test_prefill_queries_shape():
    wl = make_workload(5, num_seqs=2)
    qp, cu = wl.prefill_queries()
    assert qp.shape == (2 * 512, 64, 128) and cu.tolist() == [0, 512, 1024]
    assert (wl.context_lens >= 512).all()
