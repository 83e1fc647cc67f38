"""A decode step over all layers of a model as one captured HIP graph.

Each layer runs the library's fused step (pkv_decode_step: the new token's
K/V write, the decode partials, then the split merge) on its own slice of a
layered pool ``[layers, num_blocks, block_size, Hkv, hd]``; every layer uses
the same block tables and lengths ("Build a Mini vLLM" section 2 keeps one
pool per layer behind one table; "Day 16" grows that table once per step for
all layers). Launched one by one, a step of small layers is dominated by
fixed launch costs ("nano-vLLM" "Where the time went": a one-user step takes
about four times what its weight reads need, the rest being the many small
per-layer operations; fusion or graph replay is the stated remedy).
``LayerSteps.capture`` records the whole layer loop once
into a graph on torch's current stream; ``replay`` re-issues it with a single
launch call. The library allocates nothing and never synchronises, so its
entry points can be captured; every buffer (outputs, workspace) is allocated
here before capture. Argument marshalling only: all arithmetic is in the
library's kernels.
"""

from __future__ import annotations

import torch

from . import _binding as _b


class LayerSteps:
    """Layered decode step: q [L, S, Hq, hd], k_new / v_new [L, S, Hkv, hd]
    (the new token of each sequence and layer, position context_lens - 1),
    k_pools / v_pools [L, NB, bs, Hkv, hd]; tables [S, maxb] and context_lens
    [S] are shared by every layer. ``out`` [L, S, Hq, hd] holds the results."""

    def __init__(self, q, k_new, v_new, k_pools, v_pools, tables, context_lens, scale: float,
                 max_context_len: int, partition: int = 0):
        _b._need(q.dim() == 4 and k_pools.dim() == 5 and v_pools.shape == k_pools.shape,
                 "q must be [L, S, Hq, hd] and the pools [L, NB, bs, Hkv, hd]")
        L = q.shape[0]
        _b._need(k_new.shape[0] == L and v_new.shape[0] == L and k_pools.shape[0] == L,
                 "every per-layer tensor needs the same leading layer count")
        self.q, self.k_new, self.v_new = q, k_new, v_new
        self.k_pools, self.v_pools = k_pools, v_pools
        self.tables, self.ctx = tables, context_lens
        self.scale, self.max_ctx = float(scale), int(max_context_len)
        S, Hq = q.shape[1], q.shape[2]
        # 0 leaves the cut to the library (it may then use stream-K ranges)
        self.partition = int(partition)
        nws = _b.decode_workspace_bytes(S, Hq, self.max_ctx, k_pools[0], self.partition)
        # one workspace serves every layer: the layers run in stream order
        self.ws = torch.zeros(max(nws, 16), dtype=torch.uint8, device=q.device)
        self.out = torch.empty_like(q)
        self.graph = None

    @property
    def num_layers(self) -> int:
        return self.q.shape[0]

    def run(self):
        """Every layer's step, launched one by one on the current stream."""
        for layer in range(self.num_layers):
            _b.decode_step(self.q[layer], self.k_new[layer], self.v_new[layer],
                           self.k_pools[layer], self.v_pools[layer], self.tables, self.ctx,
                           self.scale, self.max_ctx, out=self.out[layer],
                           partition=self.partition, workspace=self.ws)
        return self.out

    def capture(self):
        """Record ``run`` into a graph. The library's kernels are loaded by one
        eager pass first (a first launch may load code objects)."""
        self.run()
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            self.run()
        torch.cuda.synchronize()
        self.graph = g
        return self

    def replay(self):
        _b._need(self.graph is not None, "capture() first")
        self.graph.replay()
        return self.out
