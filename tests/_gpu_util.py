"""Shared helpers of the GPU parity tests (no tests here)."""

from __future__ import annotations

import sys

import numpy as np
import torch

import oracle
import paged_kv_cache_scatter_amd as pkv
from workloads.gen import poison_pool

DEV = torch.device("cuda:0")

FP32_REL_TOL = 1e-5    # per (sequence, head) row, relative to the row's max |ref|
BF16_ABS_TOL = 2e-2    # elementwise, against the unrounded fp64 reference


def note(msg: str) -> None:
    print(f"[gpu] {msg}", flush=True)
    sys.stdout.flush()


def to_dev(a: np.ndarray, dtype: str | None = None) -> torch.Tensor:
    """numpy -> cuda tensor; bf16 storage (uint16 bits) becomes torch.bfloat16."""
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16 or dtype == "bf16":
        return torch.from_numpy(a.view(np.int16)).to(DEV).view(torch.bfloat16)
    return torch.from_numpy(a).to(DEV)


def to_host(t: torch.Tensor) -> np.ndarray:
    t = t.detach().cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def bits(a: np.ndarray) -> np.ndarray:
    return a.view(np.uint32) if a.dtype == np.float32 else a.view(np.uint16)


def out_f64(t: torch.Tensor, dtype: str) -> np.ndarray:
    return oracle.storage_to_f64(to_host(t), dtype)


def check_close(got: np.ndarray, ref: np.ndarray, dtype: str, what: str = "") -> float:
    """Assert the decode/prefill tolerance; returns the measured error figure."""
    assert got.shape == ref.shape, (got.shape, ref.shape)
    assert np.isfinite(got).all(), f"{what}: non-finite output"
    if dtype == "f32":
        rowmax = np.abs(ref).max(axis=-1)
        err = np.abs(got - ref).max(axis=-1)
        zero = rowmax == 0
        assert not got[zero].any(), f"{what}: rows whose reference is 0 must be exactly 0"
        rel = np.where(zero, 0.0, err / np.where(zero, 1.0, rowmax))
        worst = float(rel.max()) if rel.size else 0.0
        assert worst <= FP32_REL_TOL, f"{what}: fp32 row-relative error {worst:.3e}"
        return worst
    err = float(np.abs(got - ref).max()) if got.size else 0.0
    assert err <= BF16_ABS_TOL, f"{what}: bf16 abs error {err:.3e}"
    return err


class PoolCase:
    """A workload written into device pools through the library.

    ``fill`` = "nan" | "huge" | "zero" for the slots no token is written to.
    ``exclude_last`` leaves each sequence's last position for a paired write.
    """

    def __init__(self, wl, fill: str = "nan", exclude_last: bool = False):
        from workloads.gen import POISON_HUGE
        self.wl = wl
        if fill == "zero":
            kp = np.zeros(wl.pool_shape, wl.storage_np_dtype)
            vp = np.zeros(wl.pool_shape, wl.storage_np_dtype)
        else:
            b = None if fill == "nan" else POISON_HUGE[wl.dtype]
            kp, vp = poison_pool(wl, b), poison_pool(wl, b)
        self.kp0, self.vp0 = kp, vp
        self.k_pool = to_dev(kp)
        self.v_pool = to_dev(vp)
        self.tabs, self.first, self.cu, self.rows = wl.bulk_segments(exclude_last=exclude_last)
        self.n_tok = int(self.cu[-1])
        note(f"{wl.name}: slot mapping + bulk write of {self.n_tok} tokens")
        self.slots = pkv.slot_mapping(to_dev(self.tabs), to_dev(self.first), to_dev(self.cu),
                                      self.n_tok, wl.block_size, wl.num_blocks)
        if self.n_tok:
            pkv.write(to_dev(wl.k_rows[self.rows]), to_dev(wl.v_rows[self.rows]), self.slots,
                      self.k_pool, self.v_pool)
        self.q = to_dev(wl.q)
        self.tables = to_dev(wl.block_tables)
        self.ctx = to_dev(wl.context_lens)
        self.max_ctx = int(wl.context_lens.max()) if wl.num_seqs else 0
        torch.cuda.synchronize()
        self._ref_pools = None

    def ref_slots(self):
        return oracle.slot_mapping(self.tabs, self.first, self.cu, self.wl.block_size,
                                   self.wl.num_blocks)

    def ref_pools(self):
        if self._ref_pools is None:
            wl = self.wl
            self._ref_pools = oracle.write(self.kp0, self.vp0, wl.k_rows[self.rows],
                                           wl.v_rows[self.rows], self.ref_slots())
        return self._ref_pools

    def decode(self, partition: int = 0, q=None, out=None, phase="both"):
        note(f"{self.wl.name}: pkv_decode partition={partition or 'auto'}")
        o = pkv.decode(self.q if q is None else q, self.k_pool, self.v_pool, self.tables,
                       self.ctx, self.wl.scale, self.max_ctx, out=out, partition=partition,
                       phase=phase)
        torch.cuda.synchronize()
        return o

    def ref_decode(self, seqs=None, q=None):
        kp, vp = self.ref_pools()
        return oracle.decode(self.wl.q if q is None else q, kp, vp, self.wl.block_tables,
                             self.wl.context_lens, self.wl.scale, self.wl.dtype, seqs=seqs)
