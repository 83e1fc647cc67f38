"""Seeded request streams for the continuous-batching scheduler, and the
per-(request, position) K/V/q rows a synthetic model would produce.

The request lengths follow the draw order of the engine workload in "Build a
Mini vLLM" section 5 (numpy default_rng(seed): the generation cap, then the
prompt length, then the stop length of each request), so the scheduler runs
the very request set whose step and preemption counts the page prints. Token
values are not drawn from a model: every (request, position) has fixed N(0,1)
K, V and q rows, which is what recomputation after a preemption reproduces.
"""

from __future__ import annotations

import numpy as np
import torch


def engine_requests(n: int = 24, seed: int = 7):
    """[(rid, prompt_len, max_new, stop_after)] in the page's draw order."""
    rng = np.random.default_rng(seed)
    reqs = []
    for i in range(n):
        max_new = int(rng.integers(48, 80))
        prompt_len = int(rng.integers(8, 48))
        stop_after = int(rng.integers(5, max_new))
        reqs.append((i, prompt_len, max_new, stop_after))
    return reqs


class TokenRows:
    """K/V rows [Hkv, hd] and q rows [Hq, hd] for every (request, position),
    stored as bf16 bits (uint16) or fp32."""

    def __init__(self, num_requests: int, max_len: int, num_q_heads: int, num_kv_heads: int,
                 head_dim: int, dtype: str = "bf16", seed: int = 11):
        g = torch.Generator().manual_seed(seed)
        shape_kv = (num_requests, max_len, num_kv_heads, head_dim)
        shape_q = (num_requests, max_len, num_q_heads, head_dim)
        k = torch.randn(shape_kv, generator=g)
        v = torch.randn(shape_kv, generator=g)
        q = torch.randn(shape_q, generator=g)
        if dtype == "bf16":
            conv = lambda x: x.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
        else:
            conv = lambda x: x.numpy()
        self.k, self.v, self.q = conv(k), conv(v), conv(q)
        self.dtype = dtype
        self.max_len = max_len
