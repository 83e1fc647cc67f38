"""Plain, slow fp64 oracle of the paged KV write and paged attention.

TEST INFRASTRUCTURE. Nothing on the product path imports this module; only the
tests, the smoke check and the CPU-baseline leg of the benchmark do.

What it computes, and where the pages define it:

* Slot of a token -- "Build a Mini vLLM", section 2 "The paged KV cache"
  (``append_slot`` returns ``(table[pos // BLOCK], pos % BLOCK)``); "Day 16:
  the paged KV cache, real K/V through scattered blocks", "What I added
  today" (a flat slot per token in a ``[num_blocks * block_size, n_kv, hd]``
  pool); "nano-vLLM", "How it works" (write into ``table[n // 16]``, slot
  ``n % 16``).
* Write = scatter -- "Day 16", "What I learned" item 3 (``pool[slots] = k``);
  "Build a Mini vLLM", section 4 (prefill/decode write each token's K/V into
  ``pool.k[layer, blk, off]``).
* Read = gather through the table, then plain attention -- "Build a Mini
  vLLM", section 3 "PagedAttention" (``gather_kv``: the table's blocks,
  reshaped to ``(-1, n_kv, hd)``, sliced to the sequence length;
  ``paged_attention``: ``repeat_interleave`` of the KV heads onto the query
  heads, scores ``q.k / sqrt(hd)``, softmax, weighted sum of V). Short tables
  are padded with the dummy block 0, which is never read ("nano-vLLM", "How it
  works").
* Causal prefill -- "Build a Mini vLLM", section 4 (``full((T,T), -inf)
  .triu(1)`` added to the scores before the softmax), applied at an offset for
  a query chunk that ends at the sequence's last position.

Readings where the pages are silent (each also listed in the design notes):
  - ``scale`` is an argument; the pages use ``1/sqrt(head_dim)``.
  - query head ``h`` uses KV head ``h // (Hq // Hkv)`` (``repeat_interleave``).
  - context length 0 gives an all-zero output row.
  - a slot outside ``[0, num_blocks*block_size)`` is skipped by the write.
  - a table entry outside ``[0, num_blocks)`` that a sequence needs makes that
    block's tokens absent (they take no part in the softmax); a slot mapping
    through such an entry, or past the end of the table, is -1.
  - a context length larger than the table covers is clamped to
    ``max_blocks_per_seq * block_size``; a negative one counts as 0.
  - the split-K partial/combine identity is the standard log-sum-exp merge;
    the pages have no split, so it is pinned by the fp64 identity
    combine(split(x)) == unsplit(x).
All arithmetic is float64 on values upcast exactly from fp32 or bf16.
"""

from __future__ import annotations

import numpy as np

F32 = "f32"
BF16 = "bf16"


# --------------------------------------------------------------------------
# storage <-> float64
# --------------------------------------------------------------------------
def storage_to_f64(a: np.ndarray, dtype: str) -> np.ndarray:
    """Exact upcast: fp32 values, or bf16 bit patterns held as uint16."""
    if dtype == F32:
        return np.asarray(a, dtype=np.float32).astype(np.float64)
    if dtype == BF16:
        bits = np.asarray(a).view(np.uint16).astype(np.uint32) << 16
        return bits.view(np.float32).astype(np.float64)
    raise ValueError(dtype)


def bf16_bits_from_f64(x: np.ndarray) -> np.ndarray:
    """Round float64 to bf16 with round-to-nearest-even (via fp32; used for
    reporting ulp distances, not for pass/fail)."""
    f = np.asarray(x, dtype=np.float64).astype(np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    r = ((u + 0x7FFF + lsb) >> 16).astype(np.uint16)
    nan = np.isnan(f)
    r[nan] = 0x7FC0
    return r


# --------------------------------------------------------------------------
# slot mapping and write
# --------------------------------------------------------------------------
def slot_mapping(tables, first_pos, cu, block_size: int, num_blocks: int) -> np.ndarray:
    """Flat slot of every written token, segment by segment.

    Token ``i`` of segment ``w`` sits at logical position ``p = first_pos[w] + i``
    of the sequence with table ``tables[w]``; its slot is
    ``tables[w][p // block_size] * block_size + p % block_size``, or -1 when
    the table has no entry there or the entry is not a pool block.
    """
    tables = np.asarray(tables)
    out = []
    for w in range(len(first_pos)):
        n = int(cu[w + 1]) - int(cu[w])
        row = tables[w]
        for i in range(n):
            p = int(first_pos[w]) + i
            bi = p // block_size
            if p < 0 or bi >= len(row):
                out.append(-1)
                continue
            b = int(row[bi])
            if b < 0 or b >= num_blocks:
                out.append(-1)
                continue
            out.append(b * block_size + p % block_size)
    return np.array(out, dtype=np.int32)


def write(k_pool: np.ndarray, v_pool: np.ndarray, k_new: np.ndarray, v_new: np.ndarray,
          slots: np.ndarray):
    """Scatter: returns copies of the pools with ``pool.flat_slots[slot_t] = new[t]``.

    Pools are ``[NB, bs, Hkv, hd]`` storage arrays (any element type; values
    are copied bit for bit). Slots outside the pool are skipped.
    """
    NB, bs, Hkv, hd = k_pool.shape
    kp = k_pool.copy()
    vp = v_pool.copy()
    kf = kp.reshape(NB * bs, Hkv, hd)
    vf = vp.reshape(NB * bs, Hkv, hd)
    for t, s in enumerate(np.asarray(slots, dtype=np.int64)):
        if 0 <= s < NB * bs:
            kf[s] = k_new[t]
            vf[s] = v_new[t]
    return kp, vp


# --------------------------------------------------------------------------
# gather + attention
# --------------------------------------------------------------------------
def _clamp_ctx(ctx: int, table_len: int, block_size: int) -> int:
    return max(0, min(int(ctx), table_len * block_size))


def gather_kv(pool: np.ndarray, table_row, ctx: int, dtype: str):
    """Table -> (K or V as float64 ``[L, Hkv, hd]``, keep mask ``[L]``).

    The first ``ceil(ctx / bs)`` table entries name the sequence's blocks in
    logical order; the rows are their concatenation cut to ``ctx``. Tokens in a
    block whose id is not a pool block are returned as zeros with keep=False.
    """
    NB, bs, Hkv, hd = pool.shape
    table_row = np.asarray(table_row)
    L = _clamp_ctx(ctx, len(table_row), bs)
    n = -(-L // bs)
    blocks = table_row[:n].astype(np.int64)
    ok = (blocks >= 0) & (blocks < NB)
    safe = np.where(ok, blocks, 0)
    x = storage_to_f64(pool[safe], dtype).reshape(-1, Hkv, hd)[:L]
    keep = np.repeat(ok, bs)[:L]
    x[~keep] = 0.0
    return x, keep


def attend(q: np.ndarray, K: np.ndarray, V: np.ndarray, scale: float, keep=None) -> np.ndarray:
    """One query token per head against contiguous K/V (all float64).

    q ``[Hq, hd]``; K, V ``[L, Hkv, hd]``. KV heads are repeated onto the query
    heads (query head h reads KV head h // rep), scores are ``scale * q.k``,
    the softmax subtracts the row max, and the output is the weighted sum of V.
    """
    Hq = q.shape[0]
    L, Hkv, _ = K.shape
    if keep is None:
        keep = np.ones(L, dtype=bool)
    if L == 0 or not keep.any():
        return np.zeros_like(q, dtype=np.float64)
    rep = Hq // Hkv
    Kr = np.repeat(K[keep], rep, axis=1)
    Vr = np.repeat(V[keep], rep, axis=1)
    scores = np.einsum("hd,lhd->hl", q, Kr) * scale
    z = scores - scores.max(axis=-1, keepdims=True)
    e = np.exp(z)
    w = e / e.sum(axis=-1, keepdims=True)
    return np.einsum("hl,lhd->hd", w, Vr)


def decode_one(q_s: np.ndarray, k_pool, v_pool, table_row, ctx: int, scale: float,
               dtype: str) -> np.ndarray:
    """Decode output ``[Hq, hd]`` (float64) of one sequence: gather, then attend."""
    K, keep = gather_kv(k_pool, table_row, ctx, dtype)
    V, _ = gather_kv(v_pool, table_row, ctx, dtype)
    return attend(storage_to_f64(q_s, dtype), K, V, scale, keep)


def decode(q, k_pool, v_pool, block_tables, context_lens, scale: float, dtype: str,
           seqs=None) -> np.ndarray:
    """Decode outputs ``[S, Hq, hd]`` float64 (only rows in ``seqs`` if given)."""
    S = q.shape[0]
    out = np.zeros(q.shape, dtype=np.float64)
    for s in (range(S) if seqs is None else seqs):
        out[s] = decode_one(q[s], k_pool, v_pool, block_tables[s], int(context_lens[s]),
                            scale, dtype)
    return out


# --------------------------------------------------------------------------
# split-K partials and their combine
# --------------------------------------------------------------------------
def split_partials(q: np.ndarray, K: np.ndarray, V: np.ndarray, scale: float,
                   partition: int):
    """Per-split (m, l, o) for one sequence, float64.

    Split j covers tokens ``[j*partition, (j+1)*partition)``. For every query
    head: ``m_j`` = max score in the split, ``l_j = sum exp(score - m_j)``,
    ``o_j = sum exp(score - m_j) * v`` (unnormalised).
    """
    Hq = q.shape[0]
    L, Hkv, _ = K.shape
    rep = Hq // Hkv
    ms, ls, os_ = [], [], []
    for j0 in range(0, L, partition):
        Kr = np.repeat(K[j0:j0 + partition], rep, axis=1)
        Vr = np.repeat(V[j0:j0 + partition], rep, axis=1)
        sc = np.einsum("hd,lhd->hl", q, Kr) * scale
        m = sc.max(axis=-1)
        e = np.exp(sc - m[:, None])
        ms.append(m)
        ls.append(e.sum(axis=-1))
        os_.append(np.einsum("hl,lhd->hd", e, Vr))
    return np.array(ms), np.array(ls), np.array(os_)


def combine_partials(ms: np.ndarray, ls: np.ndarray, os_: np.ndarray) -> np.ndarray:
    """Merge split partials: ``M = max_j m_j``, ``L = sum_j l_j e^(m_j - M)``,
    ``out = sum_j e^(m_j - M) o_j / L``."""
    M = ms.max(axis=0)
    w = np.exp(ms - M[None, :])
    Lsum = (ls * w).sum(axis=0)
    return (os_ * w[:, :, None]).sum(axis=0) / Lsum[:, None]


# --------------------------------------------------------------------------
# causal prefill over the pool
# --------------------------------------------------------------------------
def prefill_one(q_rows: np.ndarray, k_pool, v_pool, table_row, ctx: int, scale: float,
                dtype: str) -> np.ndarray:
    """Causal attention for the last ``n = len(q_rows)`` positions of a sequence.

    Row i sits at absolute position ``a = ctx - n + i`` and attends keys
    ``0..a``: the causal mask (``-inf`` above the diagonal) shifted by
    ``ctx - n``. Rows with ``a < 0`` attend nothing and are zero.
    """
    K, keep = gather_kv(k_pool, table_row, ctx, dtype)
    V, _ = gather_kv(v_pool, table_row, ctx, dtype)
    L = K.shape[0]
    qf = storage_to_f64(q_rows, dtype)
    n, Hq, hd = qf.shape
    out = np.zeros((n, Hq, hd), dtype=np.float64)
    if L == 0:
        return out
    Hkv = K.shape[1]
    rep = Hq // Hkv
    Kr = np.repeat(K, rep, axis=1)
    Vr = np.repeat(V, rep, axis=1)
    scores = np.einsum("qhd,khd->hqk", qf, Kr) * scale          # [Hq, n, L]
    a = (int(ctx) - n) + np.arange(n)
    allowed = (np.arange(L)[None, :] <= a[:, None]) & keep[None, :]   # [n, L]
    mask = np.where(allowed, 0.0, -np.inf)
    scores = scores + mask[None, :, :]
    has = allowed.any(axis=1)                                     # rows with a key
    mx = np.where(has[None, :, None], scores.max(axis=-1, keepdims=True), 0.0)
    e = np.where(allowed[None], np.exp(scores - mx), 0.0)
    den = e.sum(axis=-1, keepdims=True)
    w = np.divide(e, den, out=np.zeros_like(e), where=den > 0)
    out[:] = np.einsum("hqk,khd->qhd", w, Vr)
    return out


def prefill(q, cu_q, k_pool, v_pool, block_tables, context_lens, scale: float,
            dtype: str, seqs=None) -> np.ndarray:
    """Prefill outputs for packed queries ``q [sum n_s, Hq, hd]`` (float64)."""
    out = np.zeros(q.shape, dtype=np.float64)
    S = len(cu_q) - 1
    for s in (range(S) if seqs is None else seqs):
        a, b = int(cu_q[s]), int(cu_q[s + 1])
        if b > a:
            out[a:b] = prefill_one(q[a:b], k_pool, v_pool, block_tables[s],
                                   int(context_lens[s]), scale, dtype)
    return out
