"""The C ABI without a GPU: the library loads, exports what include/*.h
declare, and rejects bad arguments before touching the GPU."""

import ctypes
import os
import re

import pytest

import glob

import paged_kv_cache_scatter_amd as pkv
from paged_kv_cache_scatter_amd._binding import PoolDesc
from paged_kv_cache_scatter_amd.sched import SCHED_EXPORTS

INCLUDE = os.path.join(os.path.dirname(os.path.dirname(__file__)), "include")
HEADER = os.path.join(INCLUDE, "pkv.h")
COUNTER_AREA = 65536 * 4   # merge counters at the start of every decode workspace


@pytest.fixture(scope="module")
def lib():
    return pkv.load()


def _declared(path):
    src = open(path).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(pkv_[a-z_0-9]+)\s*\(", src)))


def test_every_declared_symbol_is_exported(lib):
    headers = sorted(glob.glob(os.path.join(INCLUDE, "*.h")))
    assert len(headers) >= 2
    every = set()
    for h in headers:
        names = _declared(h)
        assert names, h
        for n in names:
            assert hasattr(lib, n), f"{n} ({os.path.basename(h)})"
        every |= set(names)
    assert sorted(pkv.EXPORTS) == _declared(HEADER)
    assert sorted(SCHED_EXPORTS) == _declared(os.path.join(INCLUDE, "pkv_sched.h"))
    assert every == set(pkv.EXPORTS) | set(SCHED_EXPORTS)


def test_abi_version_and_strings(lib):
    assert lib.pkv_abi_version() == 1
    for code, name in [(0, b"PKV_OK"), (3, b"PKV_ERR_SHAPE"), (7, b"PKV_ERR_ALIGN")]:
        assert lib.pkv_status_string(code) == name


def _desc(nb=64, bs=16, hkv=8, hd=128, dtype=1):
    return PoolDesc(nb, bs, hkv, hd, dtype)


def _dec(lib, desc, q=16, S=4, Hq=64, maxb=8, max_ctx=100, part=0, out=16, ws=None, wsb=0,
         scale=0.1):
    return lib.pkv_decode(q, S, Hq, 16, 16, ctypes.byref(desc), 16, maxb, 16, max_ctx, scale,
                          part, out, ws, wsb, None)


def _err(lib):
    return lib.pkv_last_error().decode()


def test_decode_argument_errors(lib):
    d = _desc()
    assert _dec(lib, _desc(dtype=5)) == 2 and "dtype" in _err(lib)
    assert _dec(lib, d, Hq=60) == 3 and "multiple" in _err(lib)
    assert _dec(lib, _desc(hd=96)) == 4 and "head_dim" in _err(lib)
    assert _dec(lib, d, Hq=8 * 16) == 4              # group of 16 not compiled
    assert _dec(lib, _desc(bs=12)) == 4 and "power of two" in _err(lib)
    assert _dec(lib, d, max_ctx=200, maxb=8) == 3 and "max_context_len" in _err(lib)
    assert _dec(lib, d, part=100) == 3 and "partition" in _err(lib)
    assert _dec(lib, d, q=None) == 1 and "NULL" in _err(lib)
    assert _dec(lib, d, q=8) == 7 and "aligned" in _err(lib)
    assert _dec(lib, d, scale=float("inf")) == 3
    # two splits of 64 tokens need a workspace
    assert _dec(lib, d, part=64, max_ctx=100) == 5 and "workspace" in _err(lib)
    need = lib.pkv_decode_workspace_bytes(4, 64, 100, 64, ctypes.byref(d))
    assert _dec(lib, d, part=64, ws=16, wsb=need - 1) == 5
    assert lib.pkv_decode(None, 0, 64, None, None, ctypes.byref(d), None, 8, None, 0, 1.0, 0,
                          None, None, 0, None) == 0      # nothing to do


def test_workspace_bytes(lib):
    d = _desc(nb=32769, bs=16, hkv=8, hd=128)
    # 64 sequences x 64 heads x 9 partial slots: a context of up to 8192
    # tokens has at most 8 pieces of 1024 tokens and 1 tail piece of less than
    # 1024 (slots: 8192 / 1024 + ceil(1023 / 1024)); the fixed merge counter
    # area (65536 int32), then (m, l), then o[128], each part 256-byte aligned
    rows = 64 * 64 * 9
    assert lib.pkv_decode_workspace_bytes(64, 64, 8192, 1024, ctypes.byref(d)) == \
        COUNTER_AREA + rows * 2 * 4 + rows * 128 * 4
    assert lib.pkv_decode_workspace_bytes(64, 64, 1024, 1024, ctypes.byref(d)) == 0
    p = lib.pkv_decode_partition(64, 8192, ctypes.byref(d))
    assert p > 0 and p % 32 == 0 and p % 16 == 0
    # invalid arguments give 0 bytes
    assert lib.pkv_decode_workspace_bytes(64, 60, 8192, 0, ctypes.byref(d)) == 0


def test_write_and_slot_mapping_argument_errors(lib):
    d = _desc()
    assert lib.pkv_write(16, 16, 16, -1, 16, 16, ctypes.byref(d), None) == 3
    assert lib.pkv_write(16, None, 16, 4, 16, 16, ctypes.byref(d), None) == 1
    assert lib.pkv_write(16, 16, 16, 4, 16, 16, None, None) == 1
    assert lib.pkv_write(16, 16, 16, 4, 16, 17, ctypes.byref(d), None) == 7
    assert lib.pkv_write(16, 16, 16, 0, 16, 16, ctypes.byref(d), None) == 0
    assert lib.pkv_write(16, 16, 16, 4, 16, 16, ctypes.byref(_desc(nb=1 << 28)), None) == 4
    assert lib.pkv_slot_mapping(16, 4, 2, 16, 16, 8, 12, 64, 16, None) == 4   # bs 12
    assert lib.pkv_slot_mapping(16, 0, 2, 16, 16, 8, 16, 64, 16, None) == 3
    assert lib.pkv_slot_mapping(None, 4, 2, 16, 16, 8, 16, 64, 16, None) == 1
    assert lib.pkv_slot_mapping(None, 4, 0, None, None, 0, 16, 64, None, None) == 0


def test_prefill_argument_errors(lib):
    d = _desc()
    args = dict(q=16, cu=16, S=2, Hq=64, mq=8, tq=16)

    def call(desc, **kw):
        a = {**args, **kw}
        return lib.pkv_prefill(a["q"], a["cu"], a["S"], a["Hq"], a["mq"], a["tq"], 16, 16,
                               ctypes.byref(desc), 16, 8, 16, 100, 0.1, 16, None)
    assert call(_desc(dtype=3)) == 2
    assert call(d, Hq=63) == 3
    assert call(d, S=-1) == 3


def test_binding_checks_shapes_before_calling():
    import torch
    k = torch.zeros(2, 3)
    with pytest.raises(ValueError):
        pkv.write(k, k, torch.zeros(2, dtype=torch.int32), torch.zeros(1, 16, 1, 3),
                  torch.zeros(1, 16, 1, 3))


def _shared_ws(lib, d, S=64, Hq=64, max_ctx=4096, G=1, mg=64, mp=2048, mt=2048, part=1024):
    return lib.pkv_decode_shared_workspace_bytes(S, Hq, max_ctx, G, mg, mp, mt, part,
                                                 ctypes.byref(d))


def test_shared_prefix_plan(lib, monkeypatch):
    monkeypatch.delenv("PKV_SHARED_MIN_SAVED_BYTES", raising=False)
    d = _desc(nb=32769, bs=16, hkv=8, hd=128)
    # tails: 2 splits of 1024 tokens; shared pass: 1 group x 8 KV heads x 4 row
    # tiles (64 members x 8 heads / 128 rows) = 32 units, so 8 key splits of
    # 256 tokens for about one workgroup per CU
    rows = 64 * 64 * (8 + 2)
    assert _shared_ws(lib, d) == COUNTER_AREA + rows * 2 * 4 + rows * 128 * 4
    # no groups, a prompt shorter than a block, an uncompiled head size: plain decode
    plain = lib.pkv_decode_workspace_bytes(64, 64, 4096, 1024, ctypes.byref(d))
    assert _shared_ws(lib, d, G=0) == plain
    assert _shared_ws(lib, d, mp=15) == plain
    d32 = _desc(nb=32769, bs=16, hkv=8, hd=32)
    assert _shared_ws(lib, d32) == lib.pkv_decode_workspace_bytes(64, 64, 4096, 1024,
                                                                  ctypes.byref(d32))
    # the tail partition follows max_tail_len; < 0 means max_context_len
    assert _shared_ws(lib, d, mt=-1) == COUNTER_AREA + 64 * 64 * (8 + 4) * (2 + 128) * 4
    # inconsistent sizes give 0 bytes
    for kw in (dict(mp=5000), dict(G=65), dict(mg=0), dict(mg=65), dict(mt=5000), dict(G=-1)):
        assert _shared_ws(lib, d, **kw) == 0, kw


def test_shared_prefix_argument_errors(lib, monkeypatch):
    monkeypatch.setenv("PKV_SHARED_MIN_SAVED_BYTES", "0")   # small sizes: still share
    d = _desc(nb=64, bs=16, hkv=8, hd=128)

    def call(gs=16, pl=16, G=1, mg=4, mp=64, mt=-1, S=4, ws=16, wsb=1 << 30):
        return lib.pkv_decode_shared(16, S, 64, 16, 16, ctypes.byref(d), 16, 8, 16, 100, gs, pl,
                                     G, mg, mp, mt, 0.1, 0, 16, ws, wsb, None)
    assert call(gs=None) == 1 and "NULL" in _err(lib)
    assert call(pl=None) == 1
    assert call(G=5) == 3 and "shared-prefix" in _err(lib)
    assert call(mp=101) == 3
    assert call(mg=0) == 3
    assert call(ws=None, wsb=0) == 5 and "workspace" in _err(lib)
    assert call(S=0, G=0, mg=0) == 0      # nothing to do


def test_paired_heads_show_in_the_workspace(lib):
    """bf16 pools of head_dim 64 with at least 1024 (sequence, KV head) pairs
    are read two KV heads at a time: the partial o rows are 128 floats wide."""
    def ws(S, hkv=2, hq=8, dtype=1, hd=64, part=32, max_ctx=100):
        d = _desc(nb=4096, bs=16, hkv=hkv, hd=hd, dtype=dtype)
        return lib.pkv_decode_workspace_bytes(S, hq, max_ctx, part, ctypes.byref(d))

    def expect(S, hq, slots, width):
        rows = S * hq * slots
        return COUNTER_AREA + -(-rows * 8 // 256) * 256 + -(-rows * width * 4 // 256) * 256

    # 100 tokens in pieces of 32 (at most 32 KiB of K/V, too little to be worth
    # the piece schedule's lookup): the plain grid's 4 slots
    assert ws(512) == expect(512, 8, 4, 128)
    # 1022 pairs, fp32, odd KV heads, groups over 4: plain rows of 64
    assert ws(511) == expect(511, 8, 4, 64)
    assert ws(512, dtype=0) == expect(512, 8, 4, 64)
    assert ws(1024, hkv=1, hq=4) == expect(1024, 4, 4, 64)
    assert ws(512, hq=10) == expect(512, 10, 4, 64)


def test_too_many_sequences_is_refused(lib):
    d = _desc()
    assert _dec(lib, d, S=65536) == 4 and "65535" in _err(lib)


def test_piece_schedule_needs_large_pieces(lib):
    """The piece schedule (full pieces, then tail pieces: more slots than the
    plain grid's ceil(max_context_len / partition)) is used only when a piece
    carries at least 128 KiB of K and V."""
    d = _desc(nb=32769, bs=16, hkv=8, hd=128)    # bf16 rows: 512 bytes of K+V per token

    # (a multiple of the partition, so that the schedule's one slot for a
    # tail piece shows against the plain grid's ceil(max_ctx / partition))
    def slots(part, max_ctx=4096):
        rows = 64 * 64
        b = lib.pkv_decode_workspace_bytes(64, 64, max_ctx, part, ctypes.byref(d))
        return (b - COUNTER_AREA) // (rows * (2 + 128) * 4)
    assert slots(128) == 4096 // 128               # 64 KiB pieces: plain grid
    assert slots(256) == 4096 // 256 + 1           # 128 KiB pieces: schedule, one tail slot
    assert slots(1024) == 4096 // 1024 + 1


def test_decode_schedule_choice(lib):
    """pkv_decode_schedule: with partition 0, the 70B layer shape (64
    sequences, 8 KV heads of 128 bf16 dims, contexts up to 8192) takes the
    stream-K ranges, and so does its TP=8 shard (one KV head: 256 MiB of K/V
    at the largest contexts, 512 KiB per range of 512); 32 of the shard's
    sequences sit on the 256 KiB bound (8192: ranges, 8191: pieces). The
    explicit automatic partition, 192
    Llama-3.2-1B sequences (one piece each, longest first) and 8 x 2048 (the
    plain grid) do not. The workspace size covers both cuts."""
    d70 = _desc(nb=32769, bs=16, hkv=8, hd=128)
    sched = lib.pkv_decode_schedule
    assert sched(64, 64, 8192, 0, ctypes.byref(d70)) == 3
    part = lib.pkv_decode_partition(64, 8192, ctypes.byref(d70))
    assert part == 1024
    assert sched(64, 64, 8192, part, ctypes.byref(d70)) == 1
    # stream-K slots: ceil(512 units / 64) + 1 = 9, as the piece schedule's
    rows = 64 * 64 * 9
    assert lib.pkv_decode_workspace_bytes(64, 64, 8192, 0, ctypes.byref(d70)) == \
        COUNTER_AREA + rows * 2 * 4 + rows * 128 * 4
    shard = _desc(nb=32769, bs=16, hkv=1, hd=128)
    assert sched(64, 8, 8192, 0, ctypes.byref(shard)) == 3
    assert sched(32, 8, 8192, 0, ctypes.byref(shard)) == 3
    assert sched(32, 8, 8191, 0, ctypes.byref(shard)) == 1
    d1b = _desc(nb=32768, bs=16, hkv=8, hd=64)
    assert sched(192, 32, 2048, 0, ctypes.byref(d1b)) == 2
    assert sched(8, 32, 2048, 0, ctypes.byref(d1b)) == 0
    # a tile wider than a block (bf16 head_dim 128 reads 8-token tiles) keeps the pieces
    d_bs4 = _desc(nb=1 << 18, bs=4, hkv=8, hd=128)
    assert sched(64, 64, 8192, 0, ctypes.byref(d_bs4)) == 1
    # more sequences than the scan takes: the plain grid
    assert sched(1025, 8, 4096, 0, ctypes.byref(shard)) == 0
    assert sched(64, 60, 8192, 0, ctypes.byref(d70)) == -1 and "multiple" in _err(lib)
    assert sched(64, 64, 8192, 0, None) == -1


def test_partition_validity_does_not_depend_on_pairing(lib):
    """bf16 rows of 64 dims take 32-token tiles, so a partition must be a
    multiple of 32 whether or not the launch reads its KV heads in pairs
    (paired rows would allow 16)."""
    d = _desc(nb=4096, bs=16, hkv=2, hd=64, dtype=1)
    for S in (100, 512):                       # 200 pairs: unpaired; 1024: paired
        assert lib.pkv_decode_workspace_bytes(S, 8, 100, 16, ctypes.byref(d)) == 0, S
        assert lib.pkv_decode_workspace_bytes(S, 8, 100, 32, ctypes.byref(d)) > 0, S


def test_noalloc_step_refuses_plans_beyond_its_scratch(lib):
    """pkv_decode_step_noalloc checks the scratch its plan needs against the
    fixed area before any device call (PKV_ERR_WORKSPACE), and reports the
    other argument errors as pkv_decode_step does."""
    d = _desc(nb=1 << 20, bs=16, hkv=8, hd=128)
    cap = pkv.NOALLOC_SCRATCH_BYTES

    def call(S, max_ctx, part=0, q=16, kn=16):
        maxb = -(-max_ctx // 16)
        return lib.pkv_decode_step_noalloc(q, kn, 16, S, 64, 16, 16, ctypes.byref(d), 16, maxb,
                                           16, max_ctx, 0.1, part, 16, None)

    # 2048 sequences of 8192 tokens in 256-token pieces: far beyond 32 MiB
    need = lib.pkv_decode_workspace_bytes(2048, 64, 8192, 256, ctypes.byref(d))
    assert need > cap
    assert call(2048, 8192, part=256) == 5 and "scratch" in _err(lib)
    assert call(4, 100, q=None) == 1
    assert call(4, 100, kn=8) == 7
    assert call(4, 100, part=100) == 3 and "partition" in _err(lib)


def test_shared_prefix_planner_falls_back_below_the_saved_bytes_bound(lib, monkeypatch):
    """pkv_decode_shared plans plain decode (the same workspace as
    pkv_decode) when the reads a shared pass could save, (S - G) * prefix *
    2 * Hkv * hd * itemsize, are under 64 MiB or PKV_SHARED_MIN_SAVED_BYTES."""
    monkeypatch.delenv("PKV_SHARED_MIN_SAVED_BYTES", raising=False)
    d = _desc(nb=4096, bs=16, hkv=3, hd=64, dtype=0)      # SmolLM2-135M shape, fp32
    plain = lib.pkv_decode_workspace_bytes(30, 9, 704, 0, ctypes.byref(d))
    shared = lambda: lib.pkv_decode_shared_workspace_bytes(30, 9, 704, 1, 30, 496, 208, 0,
                                                           ctypes.byref(d))
    # 29 * 496 * 2 * 3 * 64 * 4 = 22,093,824 bytes: plain decode
    assert shared() == plain
    monkeypatch.setenv("PKV_SHARED_MIN_SAVED_BYTES", "0")
    assert shared() > plain
    monkeypatch.setenv("PKV_SHARED_MIN_SAVED_BYTES", str(22093824))     # exactly the bound
    assert shared() > plain
    monkeypatch.setenv("PKV_SHARED_MIN_SAVED_BYTES", str(22093825))
    assert shared() == plain


def test_missing_library_fails_loudly():
    """Without libpkv.so the binding raises on load and on any call; there is
    no CPU fallback. Run in a fresh interpreter (the handle is cached)."""
    import subprocess
    import sys
    code = (
        "import paged_kv_cache_scatter_amd._binding as b\n"
        "b.LIB_PATH = '/nonexistent/libpkv.so'\n"
        "for f in (b.load, lambda: b.block_bytes(1, 16, 8, 128, 2)):\n"
        "    try:\n"
        "        f()\n"
        "        print('no error')\n"
        "    except RuntimeError as e:\n"
        "        print('raised', 'not built' in str(e))\n")
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, cwd=root,
                       timeout=300)
    assert r.stdout.split("\n")[:2] == ["raised True", "raised True"], r.stdout + r.stderr
