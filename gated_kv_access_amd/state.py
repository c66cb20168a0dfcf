"""Device memory for one ODA decode run: caches, rings, tables and workspace.

PyTorch only allocates and owns the buffers here; every step of the method
runs in liboda.so.  Buffers the kernels must never read before writing (cache
blocks and ring slots beyond the committed positions) are filled with NaN, so
a stray read shows up in the outputs instead of passing silently.
"""
from __future__ import annotations

import ctypes
from typing import Optional

import numpy as np
import torch

from . import binding as B
from .workloads import Workload, gen_block_table, gen_focus, gen_sequence


def _raw(x: torch.Tensor) -> torch.Tensor:
    """E4M3 tensors are moved as their bytes."""
    return x.view(torch.uint8) if x.dtype == torch.float8_e4m3fn else x


def _raw_fill(fill: float, dt: torch.dtype):
    """The fill value as the raw element of a host buffer filled through _raw()."""
    if dt == torch.float8_e4m3fn:
        return int(torch.tensor([fill]).to(dt).view(torch.uint8).item())
    return fill


def make_dims(wl: Workload, full_splits: int = 0, local_splits: int = 0,
              focus: Optional[bool] = None, recall_flops: int = 0) -> B.OdaDims:
    d = B.OdaDims()
    d.num_layers = wl.num_layers
    d.num_q_heads = wl.num_q_heads
    d.num_kv_heads = wl.num_kv_heads
    d.head_dim = wl.head_dim
    d.sink = wl.sink
    d.window = wl.window
    d.sw_window = wl.sw_window
    d.block_size = wl.block_size
    d.max_batch = wl.batch
    d.max_blocks_per_seq = wl.max_blocks_per_seq
    d.kv_dtype = {"bf16": B.BF16, "f32": B.F32, "fp8": B.FP8_E4M3}[wl.dtype]
    d.focus = int(wl.focus if focus is None else focus)
    d.full_splits = full_splits
    d.local_splits = local_splits
    d.softmax_scale = 0.0
    d.k_scale = wl.k_scale
    d.v_scale = wl.v_scale
    d.reserved0 = 0
    d.recall_flops = recall_flops
    kinds = np.ascontiguousarray(np.array(wl.kinds, dtype=np.uint8))
    d._kinds = kinds  # keep the host array alive with the struct
    d.layer_kind = kinds.ctypes.data
    return d


class DecodeState:
    """All device buffers of a run sized for workload `wl`."""

    def __init__(self, wl: Workload, device="cuda", dims: Optional[B.OdaDims] = None,
                 spare_blocks: int = 0, fill: float = float("nan"), gen_device=None,
                 host_cache: bool = False):
        self.wl = wl
        self.device = torch.device(device)
        # Where the seeded generator draws: the device itself (fast), or "cpu" so
        # that a CPU-side check can redraw exactly the same values.
        self.gen_device = torch.device(gen_device) if gen_device is not None else self.device
        self.dims = dims if dims is not None else make_dims(wl)
        dt = wl.torch_dtype
        Lg, Ls = len(wl.gated_layers), len(wl.sliding_layers)
        Hkv, d, Bn = wl.num_kv_heads, wl.head_dim, wl.batch
        table, nblocks = gen_block_table(wl, spare_blocks)
        self.num_blocks = nblocks
        self.block_table = torch.from_numpy(table).to(self.device)
        R = wl.sink + wl.window
        # host_cache: the paged history in pinned host memory (read by the Full
        # pass over the host link); the rings stay in HBM.
        self.host_cache = host_cache
        if Lg and host_cache:
            shape = (Lg, Hkv, nblocks, wl.block_size, d)
            self.k_cache = torch.empty(shape, dtype=dt, pin_memory=True)
            self.v_cache = torch.empty(shape, dtype=dt, pin_memory=True)
            _raw(self.k_cache).view(-1).fill_(_raw_fill(fill, dt))
            _raw(self.v_cache).view(-1).fill_(_raw_fill(fill, dt))
        else:
            self.k_cache = torch.full((Lg, Hkv, nblocks, wl.block_size, d), fill, dtype=dt, device=self.device) if Lg else None
            self.v_cache = torch.full_like(self.k_cache, fill) if Lg else None
        self.k_ring = torch.full((Lg, Bn, Hkv, R, d), fill, dtype=dt, device=self.device) if Lg else None
        self.v_ring = torch.full_like(self.k_ring, fill) if Lg else None
        self.ring_pos = torch.full((Bn, R), -7, dtype=torch.int32, device=self.device) if Lg else None
        W = wl.sw_window
        self.k_swring = torch.full((Ls, Bn, Hkv, W, d), fill, dtype=dt, device=self.device) if Ls else None
        self.v_swring = torch.full_like(self.k_swring, fill) if Ls else None
        self.swring_pos = torch.full((Bn, W), -7, dtype=torch.int32, device=self.device) if Ls else None
        self.seq_len = torch.tensor(list(wl.prefill), dtype=torch.int32, device=self.device)
        self.focus_range = torch.from_numpy(gen_focus(wl)).to(self.device)
        self.ws_bytes = B.workspace_size(self.dims, Bn)
        if self.ws_bytes == 0:
            raise ValueError("liboda rejected the dims of this workload")
        self.workspace = torch.zeros(self.ws_bytes, dtype=torch.uint8, device=self.device)
        self.kv = B.OdaKV()
        kv = self.kv
        if Lg and host_cache:
            kv.k_cache = B.host_kv_pointer(self.k_cache)
            kv.v_cache = B.host_kv_pointer(self.v_cache)
        else:
            kv.k_cache = B._p(self.k_cache) if Lg else None
            kv.v_cache = B._p(self.v_cache) if Lg else None
        kv.k_ring = B._p(self.k_ring) if Lg else None
        kv.v_ring = B._p(self.v_ring) if Lg else None
        kv.k_swring = B._p(self.k_swring) if Ls else None
        kv.v_swring = B._p(self.v_swring) if Ls else None
        kv.ring_pos = B._p(self.ring_pos) if Lg else None
        kv.swring_pos = B._p(self.swring_pos) if Ls else None
        kv.block_table = B._p(self.block_table)
        kv.seq_len = B._p(self.seq_len)
        kv.focus_range = B._p(self.focus_range)
        kv.num_blocks = nblocks
        B.workspace_init(self.dims, Bn, self.workspace)

    # ------------------------------------------------------------------ setup
    def sequence(self, layer: int, b: int, which: str) -> torch.Tensor:
        """Request b's K or V rows of `layer`, drawn by the seeded generator, on the device."""
        return gen_sequence(self.wl, layer, b, which, self.gen_device).to(self.device)

    def shifted_kv(self, b0: int) -> B.OdaKV:
        """A copy of the kv struct whose request 0 is request b0 (rings, tables and
        per-request arrays offset; caches unchanged since block ids are global)."""
        wl, kv = self.wl, B.OdaKV()
        ctypes.memmove(ctypes.byref(kv), ctypes.byref(self.kv), ctypes.sizeof(B.OdaKV))
        es = wl.esize
        R, W = wl.sink + wl.window, wl.sw_window
        if self.k_ring is not None:
            step = wl.num_kv_heads * R * wl.head_dim * es
            kv.k_ring, kv.v_ring = self.kv.k_ring + b0 * step, self.kv.v_ring + b0 * step
            kv.ring_pos = self.kv.ring_pos + b0 * R * 4
        if self.k_swring is not None:
            step = wl.num_kv_heads * W * wl.head_dim * es
            kv.k_swring, kv.v_swring = self.kv.k_swring + b0 * step, self.kv.v_swring + b0 * step
            kv.swring_pos = self.kv.swring_pos + b0 * W * 4
        kv.block_table = self.kv.block_table + b0 * wl.max_blocks_per_seq * 4
        kv.seq_len = self.kv.seq_len + b0 * 4
        kv.focus_range = self.kv.focus_range + b0 * 16
        return kv

    def prefill(self) -> None:
        """Commits each request's prefill positions for every layer, from the
        seeded generator, through oda_prefill_kv -- one request per call so the
        dense source holds a single request's rows."""
        wl = self.wl
        for b in range(wl.batch):
            P = wl.prefill[b]
            kv_b = self.shifted_kv(b)
            for layer in range(wl.num_layers):
                k_src = _raw(self.sequence(layer, b, "k"))[:max(P, 1)].unsqueeze(0).contiguous()
                v_src = _raw(self.sequence(layer, b, "v"))[:max(P, 1)].unsqueeze(0).contiguous()
                B.prefill_kv(self.dims, kv_b, 1, layer, k_src, v_src, k_src.shape[1], self.workspace)
                del k_src, v_src
        torch.cuda.synchronize(self.device)

    def decode_inputs(self, steps: Optional[int] = None):
        """k_new / v_new [steps][L][B][Hkv][d] for the decode steps (generator rows
        prefill_b .. prefill_b + steps - 1)."""
        wl = self.wl
        n = wl.steps if steps is None else steps
        k_new = torch.empty((n, wl.num_layers, wl.batch, wl.num_kv_heads, wl.head_dim), dtype=wl.torch_dtype,
                            device=self.device)
        v_new = torch.empty_like(k_new)
        for layer in range(wl.num_layers):
            for b in range(wl.batch):
                P = wl.prefill[b]
                _raw(k_new)[:, layer, b] = _raw(self.sequence(layer, b, "k"))[P:P + n]
                _raw(v_new)[:, layer, b] = _raw(self.sequence(layer, b, "v"))[P:P + n]
        return k_new, v_new

    def device_error(self) -> int:
        return int(self.workspace[:4].view(torch.int32).item())
