"""The layered decode step captured as one HIP graph: every replay equals the
layer-by-layer eager launches bit for bit (outputs and pools), and each
layer's output equals the oracle's write-then-decode of that layer."""

import numpy as np
import pytest
import torch

import oracle
from paged_kv_cache_scatter_amd.graph import LayerSteps
from workloads import make_layers, make_shared, make_workload

from _gpu_util import PoolCase, bits, check_close, note, out_f64, to_dev, to_host

pytestmark = pytest.mark.gpu


BASES = {
    # Llama-3.2-1B attention shape, 12 sequences (compact pool)
    "llama-1b": lambda: make_shared([12], [0], ("uniform", 1, 600), dtype="bf16",
                                    num_q_heads=32, num_kv_heads=8, head_dim=64, seed=41,
                                    name="llama-3.2-1b-shape"),
    # the same shape with 128 sequences: 1024 (sequence, KV head) pairs read
    # two KV heads at a time, one piece per sequence in longest-first order
    "llama-1b-paired": lambda: make_shared([128], [0], ("uniform", 1, 600), dtype="bf16",
                                           num_q_heads=32, num_kv_heads=8, head_dim=64,
                                           seed=43, name="llama-3.2-1b-shape-128"),
    # LLaMA-2-70B layer shape, 4 sequences
    "llama-70b": lambda: make_shared([4], [0], ("uniform", 1, 3000), dtype="bf16",
                                     num_q_heads=64, num_kv_heads=8, head_dim=128, seed=42,
                                     name="llama-2-70b-layer-shape"),
    # the toy fp32 model (4 sequences, head_dim 16)
    "tiny": lambda: make_workload(1),
}


def _layers(name, L, seed):
    base = BASES[name]()
    layers = make_layers(base, L, seed=seed)
    cases = [PoolCase(w, exclude_last=True) for w in layers]
    rows = np.array([r[-1] if len(r) else 0 for r in base.seq_rows], dtype=np.int64)
    q = torch.stack([to_dev(w.q) for w in layers])
    kn = torch.stack([to_dev(w.k_rows[rows]) for w in layers])
    vn = torch.stack([to_dev(w.v_rows[rows]) for w in layers])
    kp = torch.stack([c.k_pool for c in cases])
    vp = torch.stack([c.v_pool for c in cases])
    return base, layers, cases, q, kn, vn, kp, vp


def _ref_layer(pc):
    wl = pc.wl
    kp, vp = pc.ref_pools()
    tabs, first, cu, rows = wl.step_segments()
    kp, vp = oracle.write(kp, vp, wl.k_rows[rows], wl.v_rows[rows],
                          oracle.slot_mapping(tabs, first, cu, wl.block_size, wl.num_blocks))
    return oracle.decode(wl.q, kp, vp, wl.block_tables, wl.context_lens, wl.scale, wl.dtype)


@pytest.mark.parametrize("name,L", [("llama-1b", 16), ("tiny", 3), ("llama-70b", 2),
                                    ("llama-1b-paired", 4)])
def test_graph_replays_equal_eager(name, L):
    base, layers, cases, q, kn, vn, kp, vp = _layers(name, L, seed=L)
    kp0, vp0 = kp.clone(), vp.clone()
    tables, ctx = to_dev(base.block_tables), to_dev(base.context_lens)
    max_ctx = int(base.context_lens.max())
    note(f"{base.name}: {L} layers eager")
    st = LayerSteps(q, kn, vn, kp, vp, tables, ctx, base.scale, max_ctx)
    eager = to_host(st.run().clone())
    torch.cuda.synchronize()
    kp_e, vp_e = to_host(kp.clone()), to_host(vp.clone())
    for layer, pc in enumerate(cases):
        check_close(oracle.storage_to_f64(eager[layer], base.dtype), _ref_layer(pc), base.dtype,
                    f"layer {layer}")
    # back to the pre-step pools, then capture and replay
    kp.copy_(kp0)
    vp.copy_(vp0)
    st.out.zero_()
    torch.cuda.synchronize()
    note(f"{base.name}: capture + replays")
    st.capture()
    for rep in range(3):
        st.out.zero_()
        st.replay()
        torch.cuda.synchronize()
        assert np.array_equal(bits(to_host(st.out)), bits(eager)), f"replay {rep}: outputs"
        assert np.array_equal(bits(to_host(kp)), bits(kp_e)), f"replay {rep}: k pool"
        assert np.array_equal(bits(to_host(vp)), bits(vp_e)), f"replay {rep}: v pool"
        # eager work of the program between replays
        other = st.run().clone()
        torch.cuda.synchronize()
        assert np.array_equal(bits(to_host(other)), bits(eager))
