"""GPU parity of decode with paired KV heads: bf16 pools of head_dim 64 with at
least 1024 (sequence, KV head) pairs are read two adjacent KV heads at a time
(256-byte rows). Each query head must still see only its own KV head.

Tolerance as in test_gpu_decode: bf16 absolute 2e-2 against the fp64 oracle.
"""

import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_scatter_amd as pkv
from workloads import make_custom

from _gpu_util import PoolCase, bits, check_close, note, out_f64, to_dev, to_host

pytestmark = pytest.mark.gpu

S_PAIRED = 512     # x 2 KV heads = 1024 pairs: the smallest launch that pairs
BF16_INF, BF16_NAN = 0x7F80, 0x7FC0


def _workload(rep, seed, S=S_PAIRED, hi=600):
    rng = np.random.default_rng(seed)
    lens = rng.integers(1, hi + 1, size=S)
    lens[rng.choice(S, size=8, replace=False)] = 0
    need = int(sum(-(-int(L) // 16) for L in lens))
    perm = (rng.permutation(need + 4) + 1).tolist()
    tabs, k = [], 0
    for L in lens:
        n = -(-int(L) // 16)
        tabs.append(perm[k:k + n])
        k += n
    wl = make_custom(tabs, lens, dtype="bf16", num_q_heads=2 * rep, num_kv_heads=2, head_dim=64,
                     block_size=16, num_blocks=need + 5, seed=seed, name=f"paired-rep{rep}")
    return wl


@pytest.mark.parametrize("rep", [1, 2, 3, 4])
def test_paired_decode_matches_oracle(rep):
    """One piece per sequence (automatic partition, longest first), pieces of
    256 tokens on the piece schedule, pieces of 96 and 32 on the plain grid,
    and the two phases called apart (bit-equal to the one-launch call)."""
    pc = PoolCase(_workload(rep, seed=60 + rep))
    ref = pc.ref_decode()
    for part in (0, 256, 96, 32):
        got = out_f64(pc.decode(partition=part), "bf16")
        check_close(got, ref, "bf16", f"rep {rep}, partition {part}")
    both = to_host(pc.decode(partition=256))
    ws = torch.zeros(pkv.decode_workspace_bytes(pc.wl.num_seqs, pc.wl.num_q_heads, pc.max_ctx,
                                                pc.k_pool, 256),
                     dtype=torch.uint8, device=pc.q.device)
    out = torch.empty_like(pc.q)
    for ph in ("partials", "reduce"):
        pkv.decode(pc.q, pc.k_pool, pc.v_pool, pc.tables, pc.ctx, pc.wl.scale, pc.max_ctx,
                   out=out, partition=256, workspace=ws, phase=ph)
    torch.cuda.synchronize()
    assert np.array_equal(bits(to_host(out)), bits(both))


def test_paired_heads_stay_independent():
    """An infinite K element and a NaN V element in KV head 1 of sequence 0
    leave every output of KV head 0's query heads bit-identical (the paired
    kernel forms no product across heads and stores only a head's own half)."""
    pc = PoolCase(_workload(2, seed=71))
    wl = pc.wl
    clean = [to_host(pc.decode(partition=p)) for p in (0, 256)]
    L = int(wl.context_lens[0])
    assert L >= 2
    for pool, pos, val in ((pc.k_pool, 0, BF16_INF), (pc.v_pool, L - 1, BF16_NAN)):
        blk = int(wl.block_tables[0, pos // 16])
        pool.view(torch.int16)[blk, pos % 16, 1, 5] = val
    torch.cuda.synchronize()
    note("decode with Inf / NaN in KV head 1 of sequence 0")
    for p, ref in zip((0, 256), clean):
        got = to_host(pc.decode(partition=p))
        # query heads 0, 1 read KV head 0; 2, 3 read KV head 1
        assert np.array_equal(bits(got[:, :2]), bits(ref[:, :2])), p
        assert np.array_equal(bits(got[1:]), bits(ref[1:])), p
        assert not np.isfinite(oracle.storage_to_f64(got[0, 2:], "bf16")).all()


def test_paired_fused_step():
    """The fused step (write of each sequence's last token, then decode) on
    paired heads: the same bits and pools as write + decode, and the oracle."""
    wl = _workload(4, seed=81)
    pcs = [PoolCase(wl, exclude_last=True) for _ in range(2)]
    rows = np.array([r[-1] if len(r) else 0 for r in wl.seq_rows], dtype=np.int64)
    tabs, first, cu, srows = wl.step_segments()
    a, b = pcs
    slots = pkv.slot_mapping(to_dev(tabs), to_dev(first), to_dev(cu), int(cu[-1]),
                             wl.block_size, wl.num_blocks)
    pkv.write(to_dev(wl.k_rows[srows]), to_dev(wl.v_rows[srows]), slots, a.k_pool, a.v_pool)
    sep = to_host(a.decode(partition=256))
    note("paired fused step")
    fused = pkv.decode_step(b.q, to_dev(wl.k_rows[rows]), to_dev(wl.v_rows[rows]), b.k_pool,
                            b.v_pool, b.tables, b.ctx, wl.scale, b.max_ctx, partition=256)
    torch.cuda.synchronize()
    fused = to_host(fused)
    assert np.array_equal(bits(fused), bits(sep))
    assert np.array_equal(bits(to_host(b.k_pool)), bits(to_host(a.k_pool)))
    assert np.array_equal(bits(to_host(b.v_pool)), bits(to_host(a.v_pool)))
    kp, vp = b.ref_pools()
    kp, vp = oracle.write(kp, vp, wl.k_rows[srows], wl.v_rows[srows],
                          oracle.slot_mapping(tabs, first, cu, wl.block_size, wl.num_blocks))
    ref = oracle.decode(wl.q, kp, vp, wl.block_tables, wl.context_lens, wl.scale, "bf16")
    check_close(oracle.storage_to_f64(fused, "bf16"), ref, "bf16", "paired fused step")
