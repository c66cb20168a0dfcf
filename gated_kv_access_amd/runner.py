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


class RecallHead:
    """Device weights of the recall-head stand-in, its descriptor and workspace."""

    def __init__(self, w1: torch.Tensor, b1: torch.Tensor, w2: torch.Tensor, b2: float, batch: int):
        self.w1, self.b1, self.w2, self.b2 = w1.contiguous(), b1.contiguous(), w2.contiguous(), float(b2)
        self.desc = B.make_head(self.w1, self.b1, self.w2, self.b2)
        n = B.recall_workspace_size(self.desc, batch)
        if n == 0:
            raise ValueError("liboda rejected the recall head")
        self.workspace = torch.zeros(n, dtype=torch.uint8, device=w1.device)
        B.recall_workspace_init(self.desc, batch, self.workspace)

    @property
    def in_dim(self) -> int:
        return int(self.desc.in_dim)

    @property
    def params(self) -> int:
        return self.w1.numel() + self.b1.numel() + self.w2.numel() + 1

    @property
    def flops(self) -> int:
        """Multiply-adds of one evaluation, 2 FLOPs each (biases and ReLU not counted)."""
        return 2 * (self.w1.numel() + self.w2.numel())


class StepRunner:
    def __init__(self, st: DecodeState, q_local: torch.Tensor, k_new: torch.Tensor, v_new: torch.Tensor,
                 scores: Optional[torch.Tensor], theta: float = 0.0, q_full: Optional[torch.Tensor] = None,
                 want_lse: bool = True, counters: bool = True, head: Optional[RecallHead] = None,
                 head_x: Optional[torch.Tensor] = None):
        """scores [n][B]: staged recall scores; or head + head_x [n][B][in_dim]:
        the scores are computed on the device each step by the recall head."""
        wl = st.wl
        self.st = st
        self.theta = float(theta)
        n = q_local.shape[0]
        L, Bn = wl.num_layers, wl.batch
        assert q_local.shape == (n, L, Bn, wl.num_q_heads, wl.head_dim)
        assert k_new.shape == (n, L, Bn, wl.num_kv_heads, wl.head_dim) and v_new.shape == k_new.shape
        dev = st.device
        self.num_steps = n
        self.head = head
        self.q_buf = torch.empty_like(q_local[0])
        self.k_buf = torch.empty_like(k_new[0])
        self.v_buf = torch.empty_like(v_new[0])
        # stage copies in 16-byte vectors: pad the score buffer to a multiple of 4 floats
        pad = (-Bn) % 4
        self.score_buf = torch.zeros(Bn + pad, dtype=torch.float32, device=dev)
        self.qf_buf = torch.empty_like(q_full[0]) if q_full is not None else None
        self.src = [q_local, k_new, v_new]
        self.dst = [self.q_buf, self.k_buf, self.v_buf]
        if head is None:
            assert scores.shape == (n, Bn) and scores.dtype == torch.float32
            if pad:
                scores = torch.cat([scores, torch.zeros((n, pad), dtype=torch.float32, device=dev)], 1)
            self.src.append(scores.contiguous())
            self.dst.append(self.score_buf)
            self.hx_buf = None
        else:
            assert head_x is not None and head_x.shape == (n, Bn, head.in_dim) and head_x.dtype == torch.bfloat16
            self.hx_buf = torch.empty_like(head_x[0])
            self.src.append(head_x)
            self.dst.append(self.hx_buf)
        if q_full is not None:
            self.src.append(q_full)
            self.dst.append(self.qf_buf)
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
        if self.head is None:
            B.step(st.dims, st.kv, st.wl.batch, self.q_buf, self.qf_buf, self.k_buf, self.v_buf, self.score_buf,
                   self.theta, self.out, self.lse, self.call_list, self.call_count, self.full_calls, self.counters,
                   st.workspace)
        else:
            B.step_recall(st.dims, st.kv, st.wl.batch, self.q_buf, self.qf_buf, self.k_buf, self.v_buf,
                          self.head.desc, self.hx_buf, self.score_buf, self.theta, self.out, self.lse,
                          self.call_list, self.call_count, self.full_calls, self.counters, st.workspace,
                          self.head.workspace)

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
