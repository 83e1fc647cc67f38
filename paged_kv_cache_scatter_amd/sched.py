"""ctypes binding of the host scheduler (include/pkv_sched.h) and a driver that
runs its steps through the library's kernels.

The scheduler (native, in libpkv.so) decides admissions, preemptions and the
block tables; ``run_engine`` turns each step into kernel launches: the prompt
writes of newly admitted requests (pkv_slot_mapping + pkv_write) with their
causal prefill (pkv_prefill), then one fused decode step (pkv_decode_step) for
every running request. Argument marshalling only; no arithmetic of the path
happens here.
"""

from __future__ import annotations

import ctypes

import numpy as np
import torch

from . import _binding as _b

_P = ctypes.c_void_p
_I = ctypes.c_int32
_I64 = ctypes.c_int64
_IP = ctypes.POINTER(ctypes.c_int32)

SCHED_EXPORTS = ("pkv_sched_create", "pkv_sched_destroy", "pkv_sched_submit",
                 "pkv_sched_pending", "pkv_sched_step", "pkv_sched_get_stats",
                 "pkv_sched_history")


class _StepOut(ctypes.Structure):
    _fields_ = [("num_prefill", _I), ("num_decode", _I), ("num_preempted", _I),
                ("num_finished", _I), ("prefill_rid", _IP), ("prefill_len", _IP),
                ("prefill_tables", _IP), ("decode_rid", _IP), ("decode_pos", _IP),
                ("decode_tables", _IP)]


class _Stats(ctypes.Structure):
    _fields_ = [(n, _I64) for n in ("steps", "preemptions", "tokens_generated", "requests_done",
                                    "sum_running", "sum_naive_tokens", "sum_allocated_tokens",
                                    "sum_used_tokens")]


_ready = False


def _lib():
    global _ready
    lib = _b.load()
    if not _ready:
        lib.pkv_sched_create.argtypes = [_I, _I, _I, _I, _I]
        lib.pkv_sched_create.restype = _P
        lib.pkv_sched_destroy.argtypes = [_P]
        lib.pkv_sched_destroy.restype = None
        lib.pkv_sched_submit.argtypes = [_P, _I, _I, _I, _I]
        lib.pkv_sched_submit.restype = ctypes.c_int
        lib.pkv_sched_pending.argtypes = [_P]
        lib.pkv_sched_pending.restype = _I
        lib.pkv_sched_step.argtypes = [_P, ctypes.POINTER(_StepOut)]
        lib.pkv_sched_step.restype = ctypes.c_int
        lib.pkv_sched_get_stats.argtypes = [_P, ctypes.POINTER(_Stats)]
        lib.pkv_sched_get_stats.restype = ctypes.c_int
        lib.pkv_sched_history.argtypes = [_P, _IP, ctypes.POINTER(_I64), ctypes.POINTER(_I64),
                                          ctypes.POINTER(_I64), _I64]
        lib.pkv_sched_history.restype = _I64
        _ready = True
    return lib


class Scheduler:
    """Block manager + continuous (or static) batching over ``num_blocks`` blocks."""

    def __init__(self, num_blocks: int, block_size: int = 16, max_batch: int = 8,
                 continuous: bool = True, max_blocks_per_seq: int = 64):
        self._lib = _lib()
        self._h = self._lib.pkv_sched_create(num_blocks, block_size, max_batch,
                                             1 if continuous else 0, max_blocks_per_seq)
        if not self._h:
            raise _b.PkvError(3, self._lib.pkv_last_error().decode())
        self.block_size, self.max_batch, self.max_blocks = block_size, max_batch, max_blocks_per_seq
        mb = max_batch
        self._arr = {k: np.zeros(mb, np.int32) for k in ("prid", "plen", "drid", "dpos")}
        self._arr["ptab"] = np.zeros(mb * max_blocks_per_seq, np.int32)
        self._arr["dtab"] = np.zeros(mb * max_blocks_per_seq, np.int32)
        ptr = lambda a: a.ctypes.data_as(_IP)
        self._out = _StepOut(0, 0, 0, 0, ptr(self._arr["prid"]), ptr(self._arr["plen"]),
                             ptr(self._arr["ptab"]), ptr(self._arr["drid"]),
                             ptr(self._arr["dpos"]), ptr(self._arr["dtab"]))

    def __del__(self):
        h = getattr(self, "_h", None)
        if h:
            self._lib.pkv_sched_destroy(h)
            self._h = None

    def submit(self, rid: int, prompt_len: int, max_new: int, stop_after: int):
        _b._check(self._lib.pkv_sched_submit(self._h, rid, prompt_len, max_new, stop_after))

    def pending(self) -> int:
        return int(self._lib.pkv_sched_pending(self._h))

    def step(self) -> dict:
        _b._check(self._lib.pkv_sched_step(self._h, ctypes.byref(self._out)))
        o, a, mb = self._out, self._arr, self.max_blocks
        n_p, n_d = o.num_prefill, o.num_decode
        return {"prefill_rid": a["prid"][:n_p].copy(), "prefill_len": a["plen"][:n_p].copy(),
                "prefill_tables": a["ptab"][:n_p * mb].reshape(n_p, mb).copy(),
                "decode_rid": a["drid"][:n_d].copy(), "decode_pos": a["dpos"][:n_d].copy(),
                "decode_tables": a["dtab"][:n_d * mb].reshape(n_d, mb).copy(),
                "preempted": o.num_preempted, "finished": o.num_finished}

    def stats(self) -> dict:
        st = _Stats()
        _b._check(self._lib.pkv_sched_get_stats(self._h, ctypes.byref(st)))
        return {n: int(getattr(st, n)) for n, _ in _Stats._fields_}

    def history(self) -> dict:
        n = self.stats()["steps"]
        run = np.zeros(n, np.int32)
        naive, alloc, used = (np.zeros(n, np.int64) for _ in range(3))
        p64 = lambda a: a.ctypes.data_as(ctypes.POINTER(_I64))
        self._lib.pkv_sched_history(self._h, run.ctypes.data_as(_IP), p64(naive), p64(alloc),
                                    p64(used), n)
        return {"running": run, "naive": naive, "allocated": alloc, "used": used}

    def run(self, on_step=None) -> dict:
        """Step until every request is done; ``on_step(step_dict)`` runs each step's work."""
        while self.pending():
            s = self.step()
            if on_step is not None and (len(s["decode_rid"]) or len(s["prefill_rid"])):
                on_step(s)
        return self.stats()


def run_engine(requests, rows, num_blocks: int, block_size: int = 16, max_batch: int = 8,
               continuous: bool = True, max_blocks_per_seq: int = 64, check=None,
               check_prefill=None, device="cuda:0"):
    """Serve ``requests`` [(rid, prompt_len, max_new, stop_after)] through the
    scheduler and the GPU kernels. ``rows`` (workloads.TokenRows) gives the K/V/q
    of every (request, position). ``check(step, out)`` may inspect each step's
    decode output; ``check_prefill(step, out, rid_rows, pos_rows)`` each step's
    prefill output (row i is request rid_rows[i] at position pos_rows[i]).
    Returns the scheduler's stats."""
    dev = torch.device(device)
    dt = torch.bfloat16 if rows.dtype == "bf16" else torch.float32
    Hkv, hd = rows.k.shape[2], rows.k.shape[3]
    Hq = rows.q.shape[2]
    k_pool = torch.zeros((num_blocks, block_size, Hkv, hd), dtype=dt, device=dev)
    v_pool = torch.zeros_like(k_pool)
    scale = 1.0 / float(np.sqrt(hd))
    sched = Scheduler(num_blocks, block_size, max_batch, continuous, max_blocks_per_seq)
    for r in requests:
        sched.submit(*r)

    def tdev(a):
        a = np.ascontiguousarray(a)
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).to(dev).view(torch.bfloat16)
        return torch.from_numpy(a).to(dev)

    def on_step(s):
        n_p = len(s["prefill_rid"])
        if n_p:
            lens = s["prefill_len"].astype(np.int64)
            cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
            rid_rows = np.repeat(s["prefill_rid"], lens)
            pos_rows = np.concatenate([np.arange(n) for n in lens])
            slots = _b.slot_mapping(tdev(s["prefill_tables"]), tdev(np.zeros(n_p, np.int32)),
                                    tdev(cu), int(cu[-1]), block_size, num_blocks)
            _b.write(tdev(rows.k[rid_rows, pos_rows]), tdev(rows.v[rid_rows, pos_rows]), slots,
                     k_pool, v_pool)
            out_p = _b.prefill(tdev(rows.q[rid_rows, pos_rows]), tdev(cu), k_pool, v_pool,
                               tdev(s["prefill_tables"]), tdev(lens.astype(np.int32)), scale,
                               int(lens.max()), int(lens.max()))
            if check_prefill is not None:
                check_prefill(s, out_p, rid_rows, pos_rows)
        rid, pos = s["decode_rid"], s["decode_pos"]
        if not len(rid):
            return
        ctx = (pos + 1).astype(np.int32)
        out = _b.decode_step(tdev(rows.q[rid, pos]), tdev(rows.k[rid, pos]),
                             tdev(rows.v[rid, pos]), k_pool, v_pool, tdev(s["decode_tables"]),
                             tdev(ctx), scale, int(ctx.max()))
        if check is not None:
            check(s, out)

    _ = Hq
    return sched.run(on_step)
