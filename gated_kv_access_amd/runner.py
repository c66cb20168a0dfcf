"""Replays whole ODA decode steps from pre-generated per-step inputs.

One replayed step is: oda_stage_step (copy step k's q / k_new / v_new / score
into fixed buffers, k read from a device counter that the same kernel then
advances) and oda_step (Local pass of every layer, gate, gated Full pass of
every layer, fused commit).  Captured once into a HIP graph (through
torch.cuda.CUDAGraph, which records the library's launches on the capture
stream), the step then runs with no host round trip: the gate decision never
leaves the device, and skipped requests launch no Full work beyond the
workgroups that read the empty call list and exit.
"""
from __future__ import annotations

from typing import Optional

import torch

from . import binding as B
from .state import DecodeState


class StepRunner:
    def __init__(self, st: DecodeState, q_local: torch.Tensor, k_new: torch.Tensor, v_new: torch.Tensor,
                 scores: torch.Tensor, theta: float = 0.0, q_full: Optional[torch.Tensor] = None,
                 want_lse: bool = True, counters: bool = True):
        wl = st.wl
        self.st = st
        self.theta = float(theta)
        n = q_local.shape[0]
        L, Bn = wl.num_layers, wl.batch
        assert q_local.shape == (n, L, Bn, wl.num_q_heads, wl.head_dim)
        assert k_new.shape == (n, L, Bn, wl.num_kv_heads, wl.head_dim) and v_new.shape == k_new.shape
        assert scores.shape == (n, Bn) and scores.dtype == torch.float32
        dev = st.device
        self.num_steps = n
        self.src = [q_local, k_new, v_new, scores] + ([q_full] if q_full is not None else [])
        self.q_buf = torch.empty_like(q_local[0])
        self.k_buf = torch.empty_like(k_new[0])
        self.v_buf = torch.empty_like(v_new[0])
        # stage copies in 16-byte vectors: pad the score buffer to a multiple of 4 floats
        pad = (-Bn) % 4
        if pad:
            self.src[3] = torch.cat([scores, torch.zeros((n, pad), dtype=torch.float32, device=dev)], 1).contiguous()
        self.score_buf = torch.empty(Bn + pad, dtype=torch.float32, device=dev)
        self.qf_buf = torch.empty_like(q_full[0]) if q_full is not None else None
        self.dst = [self.q_buf, self.k_buf, self.v_buf, self.score_buf] + ([self.qf_buf] if q_full is not None else [])
        self.out = torch.zeros((L, Bn, wl.num_q_heads, wl.head_dim), dtype=torch.float32, device=dev)
        self.lse = torch.zeros((L, Bn, wl.num_q_heads), dtype=torch.float32, device=dev) if want_lse else None
        self.call_list = torch.zeros(Bn, dtype=torch.int32, device=dev)
        self.call_count = torch.zeros(4, dtype=torch.int32, device=dev)
        self.full_calls = torch.zeros(Bn, dtype=torch.int64, device=dev)
        self.counters = torch.zeros((Bn, len(B.ACCT_FIELDS)), dtype=torch.int64, device=dev) if counters else None
        self.step_counter = torch.zeros(2, dtype=torch.int64, device=dev)
        self.graph: Optional[torch.cuda.CUDAGraph] = None

    def _step(self) -> None:
        st = self.st
        B.stage_step(self.src, self.dst, self.step_counter, self.num_steps)  # also advances the counter
        B.step(st.dims, st.kv, st.wl.batch, self.q_buf, self.qf_buf, self.k_buf, self.v_buf, self.score_buf,
               self.theta, self.out, self.lse, self.call_list, self.call_count, self.full_calls, self.counters,
               st.workspace)

    def step_eager(self) -> None:
        self._step()

    def capture(self) -> None:
        """Records one whole step into a HIP graph.  Capture does not execute it."""
        g = torch.cuda.CUDAGraph()
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            with torch.cuda.graph(g, stream=s):
                self._step()
        torch.cuda.current_stream().wait_stream(s)
        self.graph = g

    def replay(self, n: int = 1) -> None:
        if self.graph is None:
            raise RuntimeError("capture() first")
        for _ in range(n):
            self.graph.replay()
