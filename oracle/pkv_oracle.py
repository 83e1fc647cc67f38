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
* Read through the table, then plain attention -- "Build a Mini vLLM",
  section 3 "PagedAttention": the sequence's K/V are its positions in
  logical order, position p sitting at offset ``p % block`` of the block the
  table lists at ``p // block``; every query head attends the KV head of its
  group (grouped-query attention), scores are ``q.k / sqrt(hd)``, and the
  output is the softmax-weighted sum of the V rows. Short tables are padded
  with the dummy block 0, which is never read ("nano-vLLM", "How it works").
  Here the rows are looked up position by position and each query head's
  softmax is computed on its own; the result is the same definition.
* Index errors (for the debug check) -- counts of negative, past-the-pool and
  duplicate slots of one write, of table entries outside the pool among the
  blocks a sequence needs, and of context lengths outside the table's reach
  (each token is written once: "Build a Mini vLLM", section 4; tables name
  pool blocks: "nano-vLLM", "How it works").
* Causal prefill -- "Build a Mini vLLM", section 4: a query sees only keys at
  positions up to its own (later positions are masked out before the
  softmax), applied at an offset for a query chunk that ends at the
  sequence's last position.

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


def index_errors(slots, tables, context_lens, num_blocks: int, block_size: int) -> dict:
    """What a debug check of the index data counts, by definition.

    Each token is written once ("Build a Mini vLLM", section 4) and a table
    names pool blocks ("nano-vLLM", "How it works"); the kernels skip or mask
    whatever breaks this, so these counts name the caller's errors:
    slots below 0, slots at or past ``num_blocks * block_size``, duplicate
    slots (a slot named by k tokens adds k - 1), table entries outside
    ``[0, num_blocks)`` among the ``ceil(ctx / block_size)`` blocks a sequence
    needs (its context clamped to the table), and context lengths below 0 or
    past the table's reach. ``slots`` or ``tables`` may be None.
    """
    n_slots = num_blocks * block_size
    neg = past = dup = 0
    seen = {}
    for s in ([] if slots is None else [int(x) for x in np.asarray(slots).ravel()]):
        if s < 0:
            neg += 1
        elif s >= n_slots:
            past += 1
        else:
            seen[s] = seen.get(s, 0) + 1
    dup = sum(c - 1 for c in seen.values())
    bad = outside = 0
    if tables is not None:
        tables = np.asarray(tables)
        for row, c in zip(tables, np.asarray(context_lens).ravel()):
            c = int(c)
            if c < 0 or c > len(row) * block_size:
                outside += 1
            need = -(-_clamp_ctx(c, len(row), block_size) // block_size)
            bad += sum(1 for b in row[:need] if not 0 <= int(b) < num_blocks)
    return {"negative_slots": neg, "slots_past_pool": past, "duplicate_slots": dup,
            "invalid_table_entries": bad, "context_past_table": outside}


# --------------------------------------------------------------------------
# reading K/V through the table, and attention
# --------------------------------------------------------------------------
def _clamp_ctx(ctx: int, table_len: int, block_size: int) -> int:
    return max(0, min(int(ctx), table_len * block_size))


def token_rows(pool: np.ndarray, table_row, ctx: int, dtype: str):
    """The K (or V) rows of one sequence, looked up position by position.

    Returns ``(rows, valid)``: ``rows[p]`` (float64 ``[Hkv, hd]``) is row
    ``p % bs`` of block ``table_row[p // bs]`` for every logical position
    ``p < L`` (``L`` = ``ctx`` clamped to the table's reach), and ``valid[p]``
    says whether that table entry names a pool block. Positions in a block
    that is not in the pool have ``valid = False`` and zero rows; they take no
    part in any softmax. Table entries past the last needed one are not read.
    """
    NB, bs, Hkv, hd = pool.shape
    table_row = np.asarray(table_row, dtype=np.int64)
    L = _clamp_ctx(ctx, len(table_row), bs)
    p = np.arange(L)
    blk = table_row[p // bs]
    valid = (blk >= 0) & (blk < NB)
    rows = np.zeros((L, Hkv, hd), dtype=np.float64)
    rows[valid] = storage_to_f64(pool[blk[valid], p[valid] % bs], dtype)
    return rows, valid


def _softmax_weighted_sum(z: np.ndarray, vals: np.ndarray) -> np.ndarray:
    """``sum_p w_p vals[p]`` with ``w = exp(z - max z) / sum exp(z - max z)``
    along the last axis of ``z``; entries of ``z`` equal to ``-inf`` get weight 0."""
    m = z.max(axis=-1, keepdims=True)
    e = np.exp(z - m)
    return (e @ vals) / e.sum(axis=-1, keepdims=True)


def attention(q: np.ndarray, K: np.ndarray, V: np.ndarray, scale: float,
              valid=None) -> np.ndarray:
    """Decode attention of one token, all float64.

    ``q [Hq, hd]``; ``K, V [L, Hkv, hd]``; ``valid [L]`` (default: all).
    The query heads form ``Hkv`` groups of ``rep = Hq / Hkv`` consecutive heads;
    head ``h`` attends KV head ``h // rep``. For each head the scores of the
    valid positions are ``scale * (q[h] . K[p, g])``, their softmax weights the
    rows ``V[p, g]``, and the output is that weighted sum. No valid position:
    the output is zero.
    """
    Hq, hd = q.shape
    L, Hkv, _ = K.shape
    out = np.zeros((Hq, hd), dtype=np.float64)
    keep = np.arange(L) if valid is None else np.nonzero(valid)[0]
    if keep.size == 0:
        return out
    rep = Hq // Hkv
    for g in range(Hkv):
        Kg = K[keep, g, :]
        Vg = V[keep, g, :]
        for h in range(g * rep, (g + 1) * rep):
            out[h] = _softmax_weighted_sum(scale * (Kg @ q[h]), Vg)
    return out


def decode_one(q_s: np.ndarray, k_pool, v_pool, table_row, ctx: int, scale: float,
               dtype: str) -> np.ndarray:
    """Decode output ``[Hq, hd]`` (float64) of one sequence: its rows through
    the table, then attention over them."""
    K, valid = token_rows(k_pool, table_row, ctx, dtype)
    V, _ = token_rows(v_pool, table_row, ctx, dtype)
    return attention(storage_to_f64(q_s, dtype), K, V, scale, valid)


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
    """Per-split ``(m, l, o)`` for one sequence, float64.

    Split j covers positions ``[j*partition, (j+1)*partition)``. For every
    query head h (KV head ``g = h // rep``), with ``z_p = scale * q[h].K[p, g]``
    over the split: ``m`` = the largest ``z_p``, ``l = sum_p exp(z_p - m)``,
    ``o = sum_p exp(z_p - m) V[p, g]`` (not normalised).
    Returns arrays ``[J, Hq]``, ``[J, Hq]``, ``[J, Hq, hd]``.
    """
    Hq, hd = q.shape
    L, Hkv, _ = K.shape
    rep = Hq // Hkv
    ms, ls, os_ = [], [], []
    for j0 in range(0, L, partition):
        m = np.zeros(Hq)
        lsum = np.zeros(Hq)
        o = np.zeros((Hq, hd))
        for h in range(Hq):
            g = h // rep
            z = scale * (K[j0:j0 + partition, g, :] @ q[h])
            m[h] = z.max()
            e = np.exp(z - m[h])
            lsum[h] = e.sum()
            o[h] = e @ V[j0:j0 + partition, g, :]
        ms.append(m)
        ls.append(lsum)
        os_.append(o)
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

    Row i is the query at absolute position ``a_i = ctx - n + i``. It sees
    key position p when ``p <= a_i`` (never a later position) and p lies in a
    valid block. Each row is then decode attention over the keys it sees.
    Rows that see no key (``a_i < 0``) are zero.
    """
    K, valid = token_rows(k_pool, table_row, ctx, dtype)
    V, _ = token_rows(v_pool, table_row, ctx, dtype)
    qf = storage_to_f64(q_rows, dtype)
    n, Hq, hd = qf.shape
    out = np.zeros((n, Hq, hd), dtype=np.float64)
    L, Hkv = K.shape[0], K.shape[1]
    pos = int(ctx) - n + np.arange(n)
    sees = (np.arange(L)[None, :] <= pos[:, None]) & valid[None, :]     # [n, L]
    rows = np.nonzero(sees.any(axis=1))[0]
    if rows.size == 0:
        return out
    rep = Hq // Hkv
    hidden = ~sees[rows]
    for h in range(Hq):
        g = h // rep
        z = scale * (qf[rows, h, :] @ K[:, g, :].T)                     # [rows, L]
        z[hidden] = -np.inf
        out[rows, h, :] = _softmax_weighted_sum(z, V[:, g, :])
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
