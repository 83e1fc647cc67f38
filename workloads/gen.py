"""Seeded synthetic workloads at the shapes of the five decode configurations.

Shapes come from the pages' models (per attention layer):
  * toy GQA model of "Build a Mini vLLM" (section 1 code: 8 query heads, 4 KV
    heads, head_dim 16, block 16),
  * SmolLM2-135M of "nano-vLLM" ("How it works": 3 KV heads of 64, query
    heads grouped 3 to a KV head, blocks of 16, a shared 32-token prompt),
  * Llama-3.2-1B of "Day 38: how many blocks fit" ("Why it matters": 8 KV
    heads, block 16, bf16, 24,645-block pool at 8 x 2048),
  * LLaMA-2-70B per-layer shape (GQA 8, head_dim 128) of "Build a Mini vLLM"
    section 1.
Values are N(0,1) drawn in fp32 and cast to the data type (torch's
round-to-nearest-even), standing in for real activations.

Draw order per configuration, from ``torch.Generator().manual_seed(1000+i)``:
context lengths, block-id permutation, K rows, V rows, q, then extras.

Nothing here computes a slot, gathers, or attends: this module only draws
numbers and lays out which token rows a write covers.
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field, replace

import numpy as np
import torch

F32 = "f32"
BF16 = "bf16"

# Bit patterns used to fill pool slots no sequence owns ("garbage pool").
POISON_NAN = {F32: 0x7FC00000, BF16: 0x7FC0}
POISON_HUGE = {F32: 0x7149F2CA, BF16: 0x7149}  # ~1e30 in fp32 / ~9.9e29 in bf16


@dataclass(frozen=True)
class ConfigSpec:
    cfg_id: int
    name: str
    dtype: str
    num_seqs: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    block_size: int
    num_blocks: int
    max_blocks_per_seq: int
    ctx_dist: tuple          # ("uniform", lo, hi) | ("const", n) | ("loguniform", lo, hi)
    prefix_blocks: int = 0   # leading table entries shared by every sequence
    paired_write: bool = False
    prefill_chunk: int = 0


CONFIGS = {
    1: ConfigSpec(1, "tiny-gqa-fp32", F32, 4, 8, 4, 16, 16, 64, 4, ("uniform", 1, 64)),
    2: ConfigSpec(2, "smollm2-135m-fp32", F32, 30, 9, 3, 64, 16, 512, 13,
                  ("uniform", 8, 200), prefix_blocks=2),
    3: ConfigSpec(3, "llama-3.2-1b-bf16-8x2048", BF16, 8, 32, 8, 64, 16, 24645, 128,
                  ("const", 2048)),
    4: ConfigSpec(4, "llama-3.2-1b-bf16-192seq", BF16, 192, 32, 8, 64, 16, 32768, 128,
                  ("uniform", 128, 2048), paired_write=True),
    5: ConfigSpec(5, "llama-2-70b-layer-bf16", BF16, 64, 64, 8, 128, 16, 32769, 512,
                  ("loguniform", 512, 8192), paired_write=True, prefill_chunk=512),
}


def kv_bytes(tokens: int, layers: int, kv_heads: int, head_dim: int, itemsize: int) -> int:
    """Bytes of K plus V for ``tokens`` tokens over ``layers`` layers: two
    tensors (K and V) x layers x KV heads x head_dim x itemsize per token
    ("Build a Mini vLLM", section 1; "Day 38: how many blocks fit", "Why it
    matters", where a block is ``block_size`` such tokens)."""
    return 2 * int(tokens) * int(layers) * int(kv_heads) * int(head_dim) * int(itemsize)


def _to_storage(x: torch.Tensor, dtype: str) -> np.ndarray:
    """fp32 tensor -> numpy storage: float32 values, or bf16 bit patterns (uint16)."""
    if dtype == F32:
        return x.to(torch.float32).numpy().copy()
    return x.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16).copy()


@dataclass
class Workload:
    """One batch of decode inputs.

    Token rows: ``k_rows``/``v_rows`` hold ``[T_all, Hkv, hd]`` values, one row
    per distinct token. A write segment ``w`` puts rows
    ``w_cu[w] .. w_cu[w+1]-1`` at consecutive logical positions starting at
    ``w_first_pos[w]`` of the sequence whose block table is ``w_tables[w]``.
    A shared prefix is one segment, written once.
    """

    name: str
    cfg_id: int | None
    dtype: str
    num_seqs: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    block_size: int
    num_blocks: int
    max_blocks_per_seq: int
    scale: float
    context_lens: np.ndarray      # int32 [S]
    block_tables: np.ndarray      # int32 [S, maxb], padded with 0
    k_rows: np.ndarray            # storage [T_all, Hkv, hd]
    v_rows: np.ndarray
    q: np.ndarray                 # storage [S, Hq, hd]
    w_tables: np.ndarray          # int32 [W, maxb]
    w_first_pos: np.ndarray       # int32 [W]
    w_cu: np.ndarray              # int32 [W+1]
    seq_rows: list                # per sequence: int64 row index of each position 0..ctx-1
    prefix_tokens: int = 0
    # shared-prefix groups: (first sequence, end sequence, shared tokens);
    # one group of every sequence when prefix_tokens > 0
    groups: list = field(default_factory=list)
    paired_write: bool = False
    prefill_chunk: int = 0
    _extra_gen: torch.Generator | None = field(default=None, repr=False)
    _prefill_q: np.ndarray | None = field(default=None, repr=False)

    # ---- sizes -------------------------------------------------------------
    @property
    def itemsize(self) -> int:
        return 4 if self.dtype == F32 else 2

    @property
    def storage_np_dtype(self):
        return np.float32 if self.dtype == F32 else np.uint16

    @property
    def pool_shape(self):
        return (self.num_blocks, self.block_size, self.num_kv_heads, self.head_dim)

    @property
    def total_ctx(self) -> int:
        return int(self.context_lens.astype(np.int64).sum())

    def kv_bytes_per_call(self) -> int:
        """K and V bytes a decode call must read: ctx rows per KV head, K and V."""
        return kv_bytes(self.total_ctx, 1, self.num_kv_heads, self.head_dim, self.itemsize)

    # ---- write descriptions ------------------------------------------------
    def bulk_segments(self, exclude_last: bool = False):
        """(tables, first_pos, cu, row_index) describing the bulk fill.

        With ``exclude_last`` every sequence's final position is left out (it is
        written by the paired decode-step write instead). Only valid without a
        shared prefix.
        """
        if not exclude_last:
            rows = np.arange(int(self.w_cu[-1]), dtype=np.int64)
            return self.w_tables, self.w_first_pos, self.w_cu, rows
        assert self.prefix_tokens == 0, "paired write needs unshared last tokens"
        counts = np.maximum(self.context_lens.astype(np.int64) - 1, 0)
        cu = np.zeros(self.num_seqs + 1, dtype=np.int32)
        cu[1:] = np.cumsum(counts)
        rows = np.concatenate([r[:-1] for r in self.seq_rows if len(r) > 0]
                              + [np.zeros(0, np.int64)]).astype(np.int64)
        return self.block_tables, np.zeros(self.num_seqs, np.int32), cu, rows

    def step_segments(self):
        """(tables, first_pos, cu, row_index) of the paired 1-token-per-sequence write."""
        assert self.prefix_tokens == 0
        live = self.context_lens > 0
        first = np.where(live, self.context_lens - 1, 0).astype(np.int32)
        counts = live.astype(np.int64)
        cu = np.zeros(self.num_seqs + 1, dtype=np.int32)
        cu[1:] = np.cumsum(counts)
        rows = np.array([r[-1] for r in self.seq_rows if len(r) > 0], dtype=np.int64)
        return self.block_tables, first, cu, rows

    # ---- extras ------------------------------------------------------------
    def prefill_queries(self):
        """Chunked-prefill queries: ``chunk`` rows per sequence at its last
        ``chunk`` positions. Returns (q_pre storage [S*chunk, Hq, hd], cu_q int32)."""
        assert self.prefill_chunk > 0
        if self._prefill_q is None:
            n = self.num_seqs * self.prefill_chunk
            x = torch.randn((n, self.num_q_heads, self.head_dim), generator=self._extra_gen)
            self._prefill_q = _to_storage(x, self.dtype)
        cu = np.arange(0, self.num_seqs * self.prefill_chunk + 1, self.prefill_chunk,
                       dtype=np.int32)
        return self._prefill_q, cu


def _draw_ctx(spec: ConfigSpec, S: int, g: torch.Generator) -> np.ndarray:
    kind = spec.ctx_dist[0]
    if kind == "uniform":
        lo, hi = spec.ctx_dist[1], spec.ctx_dist[2]
        return torch.randint(lo, hi + 1, (S,), generator=g).numpy().astype(np.int32)
    if kind == "const":
        return np.full(S, spec.ctx_dist[1], dtype=np.int32)
    if kind == "loguniform":
        lo, hi = spec.ctx_dist[1], spec.ctx_dist[2]
        u = torch.rand((S,), generator=g, dtype=torch.float64).numpy()
        x = np.floor(np.exp(math.log(lo) + (math.log(hi) - math.log(lo)) * u))
        return np.clip(x, lo, hi - 1).astype(np.int32)
    raise ValueError(kind)


def _fill_tables(ctx: np.ndarray, bs: int, maxb: int, order: np.ndarray,
                 prefix_ids: list) -> np.ndarray:
    """Block tables filled consecutively from ``order`` sequence by sequence,
    after the shared ``prefix_ids``; padded with the dummy block 0."""
    S = len(ctx)
    tables = np.zeros((S, maxb), dtype=np.int32)
    nxt = 0
    for s in range(S):
        need = -(-int(ctx[s]) // bs)
        tables[s, :len(prefix_ids)] = prefix_ids
        own = max(0, need - len(prefix_ids))
        if nxt + own > len(order):
            raise ValueError("pool too small for the drawn context lengths")
        tables[s, len(prefix_ids):len(prefix_ids) + own] = order[nxt:nxt + own]
        nxt += own
    return tables


def _build(name, cfg_id, dtype, Hq, Hkv, hd, bs, NB, maxb, scale, ctx, tables,
           prefix_tokens, g, paired_write=False, prefill_chunk=0, groups=None) -> Workload:
    S = len(ctx)
    ctx = np.asarray(ctx, dtype=np.int32)
    if groups is None:
        groups = [(0, S, prefix_tokens)] if prefix_tokens > 0 else []
    opens = {s0: (s1, p) for (s0, s1, p) in groups}
    # rows: each group's shared prefix (once), then its sequences' own positions
    seq_rows, w_first, w_counts, w_tabs = [], [], [], []
    n_rows = 0
    p, end, prow0 = 0, 0, 0
    for s in range(S):
        if s in opens:
            end, p = opens[s]
            nbp = -(-p // bs)
            t0 = np.zeros(maxb, dtype=np.int32)
            t0[:nbp] = tables[s, :nbp]
            for m in range(s, end):
                assert np.array_equal(tables[m, :nbp], t0[:nbp]), "prefix blocks must be shared"
            w_tabs.append(t0)
            w_first.append(0)
            w_counts.append(p)
            prow0 = n_rows
            n_rows += p
        elif s >= end:
            p = 0
        L = int(ctx[s])
        own = max(0, L - p)
        shared = min(L, p)
        seq_rows.append(np.concatenate([prow0 + np.arange(shared, dtype=np.int64),
                                        n_rows + np.arange(own, dtype=np.int64)]))
        w_tabs.append(tables[s].copy())
        w_first.append(p)
        w_counts.append(own)
        n_rows += own
    w_cu = np.zeros(len(w_counts) + 1, dtype=np.int32)
    w_cu[1:] = np.cumsum(w_counts)
    k = torch.randn((n_rows, Hkv, hd), generator=g)
    v = torch.randn((n_rows, Hkv, hd), generator=g)
    q = torch.randn((S, Hq, hd), generator=g)
    return Workload(
        name=name, cfg_id=cfg_id, dtype=dtype, num_seqs=S, num_q_heads=Hq,
        num_kv_heads=Hkv, head_dim=hd, block_size=bs, num_blocks=NB,
        max_blocks_per_seq=maxb, scale=scale, context_lens=ctx,
        block_tables=np.ascontiguousarray(tables, dtype=np.int32),
        k_rows=_to_storage(k, dtype), v_rows=_to_storage(v, dtype), q=_to_storage(q, dtype),
        w_tables=np.stack(w_tabs).astype(np.int32), w_first_pos=np.array(w_first, np.int32),
        w_cu=w_cu, seq_rows=seq_rows, prefix_tokens=prefix_tokens, groups=list(groups),
        paired_write=paired_write, prefill_chunk=prefill_chunk, _extra_gen=g)


def make_workload(cfg_id: int, num_seqs: int | None = None, seed: int | None = None) -> Workload:
    """Configuration ``cfg_id`` (1..5). ``num_seqs`` shrinks the batch while
    keeping shapes and distributions (a reduced parity case)."""
    spec = CONFIGS[cfg_id]
    S = spec.num_seqs if num_seqs is None else int(num_seqs)
    g = torch.Generator().manual_seed(1000 + cfg_id if seed is None else seed)
    ctx = _draw_ctx(spec, S, g)
    first_free = 1 + spec.prefix_blocks
    order = (torch.randperm(spec.num_blocks - first_free, generator=g).numpy()
             + first_free).astype(np.int32)
    prefix_ids = list(range(1, 1 + spec.prefix_blocks))
    tables = _fill_tables(ctx, spec.block_size, spec.max_blocks_per_seq, order, prefix_ids)
    scale = 1.0 / math.sqrt(spec.head_dim)
    name = spec.name if num_seqs is None else f"{spec.name}[S={S}]"
    return _build(name, cfg_id, spec.dtype, spec.num_q_heads, spec.num_kv_heads,
                  spec.head_dim, spec.block_size, spec.num_blocks,
                  spec.max_blocks_per_seq, scale, ctx, tables,
                  spec.prefix_blocks * spec.block_size, g,
                  paired_write=spec.paired_write, prefill_chunk=spec.prefill_chunk)


def make_tp_shard(cfg_id: int = 5, tp: int = 8) -> Workload:
    """One rank's share of configuration ``cfg_id`` when its KV heads are split
    over ``tp`` GPUs: the same context lengths and block tables (one table
    serves every rank), ``num_kv_heads / tp`` KV heads and their query heads,
    fresh N(0,1) values at that shape. For the 70B layer (8 KV heads) and
    tp = 8 this is 1 KV head and 8 query heads, head_dim 128."""
    spec = CONFIGS[cfg_id]
    assert spec.num_kv_heads % tp == 0, "tp must divide the KV heads"
    g = torch.Generator().manual_seed(1000 + cfg_id)
    ctx = _draw_ctx(spec, spec.num_seqs, g)
    first_free = 1 + spec.prefix_blocks
    order = (torch.randperm(spec.num_blocks - first_free, generator=g).numpy()
             + first_free).astype(np.int32)
    prefix_ids = list(range(1, 1 + spec.prefix_blocks))
    tables = _fill_tables(ctx, spec.block_size, spec.max_blocks_per_seq, order, prefix_ids)
    hkv = spec.num_kv_heads // tp
    hq = spec.num_q_heads // tp
    # cfg_id names the configuration whose lengths and tables the shard keeps
    return _build(f"{spec.name}-tp{tp}-shard", cfg_id, spec.dtype, hq, hkv, spec.head_dim,
                  spec.block_size, spec.num_blocks, spec.max_blocks_per_seq,
                  1.0 / math.sqrt(spec.head_dim), ctx, tables,
                  spec.prefix_blocks * spec.block_size, g, paired_write=spec.paired_write)


def make_custom(tables, context_lens, *, dtype=F32, num_q_heads=2, num_kv_heads=1,
                head_dim=16, block_size=16, num_blocks=None, prefix_tokens=0,
                scale=None, seed=0, name="custom") -> Workload:
    """Hand-built case: explicit block tables and lengths, fresh N(0,1) values."""
    tables = [list(t) for t in tables]
    maxb = max(1, max(len(t) for t in tables))
    tab = np.zeros((len(tables), maxb), dtype=np.int32)
    for i, t in enumerate(tables):
        tab[i, :len(t)] = t
    if num_blocks is None:
        num_blocks = int(tab.max()) + 1
    g = torch.Generator().manual_seed(seed)
    sc = 1.0 / math.sqrt(head_dim) if scale is None else float(scale)
    return _build(name, None, dtype, num_q_heads, num_kv_heads, head_dim, block_size,
                  num_blocks, maxb, sc, np.asarray(context_lens, np.int32), tab,
                  prefix_tokens, g)


def poison_pool(wl: Workload, bits: int | None = None) -> np.ndarray:
    """A pool-shaped storage array filled with one bit pattern (NaN by default)."""
    if bits is None:
        bits = POISON_NAN[wl.dtype]
    if wl.dtype == F32:
        return np.full(wl.pool_shape, bits, dtype=np.uint32).view(np.float32)
    return np.full(wl.pool_shape, bits, dtype=np.uint16)


def make_shared(group_sizes, prefix_tokens, tail=("uniform", 1, 64), *, dtype=BF16,
                num_q_heads=8, num_kv_heads=1, head_dim=128, block_size=16,
                short_members=0, num_blocks=None, seed=0, name="shared") -> Workload:
    """Groups of consecutive sequences sharing a prompt: group i has
    ``group_sizes[i]`` members whose tables start with the same
    ``prefix_tokens[i] // block_size`` blocks (the prompt, written once); each
    member adds its own tail of lengths drawn from ``tail`` (as ``ctx_dist``).
    The first ``short_members`` members of each group instead stop inside the
    prompt (context drawn from 1 .. prompt). Prompts are whole blocks. Draw
    order: tails, short lengths, block permutation, K rows, V rows, q."""
    assert len(group_sizes) == len(prefix_tokens)
    assert all(p % block_size == 0 for p in prefix_tokens), "prompts are whole blocks"
    g = torch.Generator().manual_seed(seed)
    S = int(sum(group_sizes))
    spec = ConfigSpec(0, name, dtype, S, num_q_heads, num_kv_heads, head_dim, block_size,
                      1, 1, tail)
    tails = _draw_ctx(spec, S, g).astype(np.int64)
    shorts = torch.rand((S,), generator=g, dtype=torch.float64).numpy()
    ctx = np.zeros(S, np.int64)
    groups, s = [], 0
    for n, p in zip(group_sizes, prefix_tokens):
        for i in range(n):
            if i < short_members and p > 0:
                ctx[s + i] = 1 + int(shorts[s + i] * p) if p > 1 else 1
            else:
                ctx[s + i] = p + tails[s + i]
        groups.append((s, s + n, int(p)))
        s += n
    need = sum(p // block_size for p in prefix_tokens) + sum(
        max(0, -(-int(ctx[m]) // block_size) - prefix_tokens[gi] // block_size)
        for gi, (s0, s1, _) in enumerate(groups) for m in range(s0, s1))
    NB = int(num_blocks) if num_blocks is not None else need + 1
    assert NB >= need + 1, "pool too small"
    order = (torch.randperm(NB - 1, generator=g).numpy() + 1).astype(np.int32)
    maxb = max([1] + [-(-int(c) // block_size) for c in ctx]
               + [p // block_size for p in prefix_tokens])
    tables = np.zeros((S, maxb), np.int32)
    nxt = 0
    for (s0, s1, p) in groups:
        # every member's table starts with the whole prompt, also a short
        # member's (which reads only the blocks its context reaches)
        nbp = p // block_size
        pre = order[nxt:nxt + nbp]
        nxt += nbp
        for m in range(s0, s1):
            nb = -(-int(ctx[m]) // block_size)
            tables[m, :nbp] = pre
            own = max(0, nb - nbp)
            tables[m, nbp:nbp + own] = order[nxt:nxt + own]
            nxt += own
    scale = 1.0 / math.sqrt(head_dim)
    return _build(name, None, dtype, num_q_heads, num_kv_heads, head_dim, block_size, NB, maxb,
                  scale, ctx.astype(np.int32), tables, 0, g, groups=groups)


def make_layers(wl: Workload, num_layers: int, seed: int = 0) -> list:
    """``num_layers`` workloads sharing ``wl``'s tables, lengths and write
    segments (one table serves every layer), each with its own K/V rows and
    queries drawn N(0,1) from ``manual_seed(seed * 1000 + layer)`` (K, V, q)."""
    out = []
    for layer in range(num_layers):
        g = torch.Generator().manual_seed(seed * 1000 + layer)
        shp = wl.k_rows.shape
        k = torch.randn(shp, generator=g)
        v = torch.randn(shp, generator=g)
        q = torch.randn(wl.q.shape, generator=g)
        out.append(replace(wl, name=f"{wl.name}[layer {layer}]", k_rows=_to_storage(k, wl.dtype),
                           v_rows=_to_storage(v, wl.dtype), q=_to_storage(q, wl.dtype),
                           _extra_gen=None, _prefill_q=None))
    return out
