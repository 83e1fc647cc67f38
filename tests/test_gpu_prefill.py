"""GPU parity of causal (chunked) prefill over the paged pool against the oracle."""

import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_scatter_amd as pkv
from workloads import make_custom, make_workload

from _gpu_util import DEV, PoolCase, check_close, note, out_f64, to_dev

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


def test_prefill_one_row_equals_decode():
    """A one-row chunk at each sequence's last position is that sequence's
    decode step; with the same single split the bits are identical."""
    wl = make_workload(5, num_seqs=3)
    pc = PoolCase(wl)
    cu = np.arange(4, dtype=np.int32)
    got = _run(pc, wl.q, cu, 1)
    whole = -(-pc.max_ctx // 16) * 16
    dec = pc.decode(partition=whole)
    assert torch.equal(got.view(torch.int16), dec.view(torch.int16))
    check_close(out_f64(got, "bf16"), pc.ref_decode(), "bf16")


def test_prefill_config5_variant_sampled():
    """Config 5's chunked-prefill variant at full size (64 sequences x 512 rows
    at each sequence's last 512 positions); the oracle checks sampled rows."""
    wl = make_workload(5)
    pc = PoolCase(wl)
    q_pre, cu = wl.prefill_queries()
    got = out_f64(_run(pc, q_pre, cu, wl.prefill_chunk), "bf16")
    kp, vp = pc.ref_pools()
    rng = np.random.default_rng(5)
    rows = sorted(set(rng.choice(q_pre.shape[0], 40, replace=False).tolist()) |
                  {0, 511, q_pre.shape[0] - 1})
    for r in rows:
        s = int(np.searchsorted(cu, r, side="right") - 1)
        n = int(cu[s + 1] - cu[s])
        a = int(wl.context_lens[s]) - n + (r - int(cu[s]))
        ref = oracle.prefill_one(q_pre[r:r + 1], kp, vp, wl.block_tables[s], a + 1,
                                 wl.scale, "bf16")
        check_close(got[r:r + 1], ref, "bf16", f"row {r}")
    note(f"checked {len(rows)} sampled prefill rows")
