"""Seeded synthetic workloads for the ODA decode path.

This module only draws inputs: shapes, seeds and random values.  It contains
none of the method's arithmetic (no access sets, no attention, no gate), so
both the HIP path and the CPU oracle may take their inputs from it.

The shapes follow the runtime setting of the On-Demand Attention pages
(learnaivisually explainer, runtime section: 128K input, 1K output, batch 1,
12.5% global-call rate; picx.dev summary, RULER16K call rate of about 41%),
with a Qwen3-1.7B-like attention shape (28 layers, 16 query / 8 KV heads of
128, bf16).  No dataset or trained weight is involved: keys, values and
queries are N(0,1) draws rounded to the storage type, and recall scores are
drawn so that the Full-call rate is the stated rho.  FP8 E4M3 variants of a
workload (``Workload.fp8()``) store K/V as E4M3 codes of N(0, 16^2) draws with
per-tensor scales 1/16, so that the dequantised values are again about N(0,1);
their queries stay bf16.
"""
from __future__ import annotations

from dataclasses import dataclass, replace
from typing import Optional, Tuple

import numpy as np
import torch

GATED, SLIDING = 0, 1


@dataclass(frozen=True)
class Workload:
    name: str
    num_layers: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    dtype: str                      # K/V storage: "bf16", "f32" or "fp8" (E4M3; queries then bf16)
    batch: int
    prefill: Tuple[int, ...]        # committed positions per request before step 1
    steps: int
    sink: int
    window: int
    block_size: int = 16
    sw_window: int = 0
    layer_kind: Optional[Tuple[int, ...]] = None   # GATED / SLIDING per layer
    focus: bool = False
    score_mode: str = "normal"      # "normal" | "rho_minus_u" | "exact"
    rho: Tuple[float, ...] = (0.5,)  # per request (one value = all requests)
    seed: int = 0
    block_order: str = "shuffled"   # physical block ids: "shuffled" (seeded permutation) or "sequential"
    k_scale: float = 1.0            # K = k_scale * stored value
    v_scale: float = 1.0
    kv_code_std: float = 1.0        # standard deviation of the stored K/V draws

    @property
    def torch_dtype(self) -> torch.dtype:
        """Storage type of K and V."""
        return {"bf16": torch.bfloat16, "f32": torch.float32, "fp8": torch.float8_e4m3fn}[self.dtype]

    @property
    def q_torch_dtype(self) -> torch.dtype:
        return torch.float32 if self.dtype == "f32" else torch.bfloat16

    @property
    def esize(self) -> int:
        """Bytes per stored K/V element."""
        return {"bf16": 2, "f32": 4, "fp8": 1}[self.dtype]

    def fp8(self, k_scale: float = 0.0625, v_scale: float = 0.0625, code_std: float = 16.0) -> "Workload":
        """The same workload with an FP8 E4M3 KV cache."""
        return replace(self, name=self.name + "_fp8e4m3", dtype="fp8", k_scale=k_scale, v_scale=v_scale,
                       kv_code_std=code_std)

    @property
    def kinds(self) -> Tuple[int, ...]:
        return self.layer_kind if self.layer_kind is not None else (GATED,) * self.num_layers

    @property
    def gated_layers(self) -> Tuple[int, ...]:
        return tuple(i for i, k in enumerate(self.kinds) if k == GATED)

    @property
    def sliding_layers(self) -> Tuple[int, ...]:
        return tuple(i for i, k in enumerate(self.kinds) if k == SLIDING)

    def rows(self, b: int) -> int:
        """Sequence rows request b needs: its prefill plus one position per step."""
        return self.prefill[b] + self.steps

    @property
    def max_rows(self) -> int:
        return max(self.rows(b) for b in range(self.batch))

    def blocks_for(self, b: int) -> int:
        return -(-self.rows(b) // self.block_size)

    @property
    def max_blocks_per_seq(self) -> int:
        return max(self.blocks_for(b) for b in range(self.batch))

    def with_(self, **kw) -> "Workload":
        return replace(self, **kw)


def _hybrid_kinds(n: int) -> Tuple[int, ...]:
    # 3:1 interleave: three sliding-window layers, then one gated global layer.
    return tuple(GATED if i % 4 == 3 else SLIDING for i in range(n))


def _mixed_prefill(seed: int, batch: int, lo: int, hi: int, steps: int, cap_bytes: float,
                   bytes_per_pos: int) -> Tuple[int, ...]:
    """Uniform lengths in [lo, hi]; redraws (seed, seed+1, ...) until the whole
    paged cache fits cap_bytes."""
    for k in range(1000):
        rng = np.random.default_rng([seed, 77, k])
        lens = rng.integers(lo, hi + 1, size=batch)
        if float((lens + steps).sum()) * bytes_per_pos <= cap_bytes:
            return tuple(int(x) for x in lens)
    raise RuntimeError("no length draw fits the memory cap")


def config(index: int) -> Workload:
    """The five workloads: tiny CPU-checkable, 16K, 128K, batched mixed, hybrid+focus."""
    if index == 0:
        return Workload("tiny_f32_ctx300", 1, 2, 1, 64, "f32", 1, (300,), 50, 4, 64,
                        score_mode="normal", seed=0)
    if index == 1:
        return Workload("qwen3_1.7b_ctx16k_rho0.41", 28, 16, 8, 128, "bf16", 1, (16384,), 256,
                        4, 2048, score_mode="rho_minus_u", rho=(0.41,), seed=1)
    if index == 2:
        return Workload("qwen3_1.7b_ctx128k_rho0.125", 28, 16, 8, 128, "bf16", 1, (131072,), 1024,
                        4, 2048, score_mode="exact", rho=(0.125,), seed=2)
    if index == 3:
        steps = 512
        bytes_per_pos = 28 * 8 * 128 * 2 * 2
        pre = _mixed_prefill(3, 32, 4096, 131072, steps, 240e9, bytes_per_pos)
        rng = np.random.default_rng([3, 99])
        rho = tuple(float(x) for x in rng.choice([0.0, 0.125, 0.41, 1.0], size=32))
        return Workload("batched32_mixed_4k_128k", 28, 16, 8, 128, "bf16", 32, pre, steps, 4, 2048,
                        score_mode="rho_minus_u", rho=rho, seed=3)
    if index == 4:
        return Workload("hybrid32_sw1024_focus4096_ctx64k", 32, 16, 8, 128, "bf16", 8, (65536,) * 8,
                        512, 4, 2048, sw_window=1024, layer_kind=_hybrid_kinds(32), focus=True,
                        score_mode="rho_minus_u", rho=(0.25,), seed=4)
    raise IndexError(index)


def _seed(*parts: int) -> int:
    return int(np.random.SeedSequence([int(p) for p in parts]).generate_state(1)[0])


def _normal(shape, seed: int, device, dtype: torch.dtype, std: float = 1.0) -> torch.Tensor:
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    x = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    if std != 1.0:
        x = x * std
    return x.to(dtype)  # round-to-nearest-even (bf16, E4M3)


def gen_sequence(wl: Workload, layer: int, b: int, which: str, device="cpu") -> torch.Tensor:
    """K ('k') or V ('v') rows of request b in layer `layer`: [rows(b)][Hkv][d].
    Row p-1 holds position p; rows >= prefill[b] are the tokens decoded at steps 1.."""
    tag = {"k": 1, "v": 2}[which]
    return _normal((wl.rows(b), wl.num_kv_heads, wl.head_dim),
                   _seed(wl.seed, 11, layer, b, tag), device, wl.torch_dtype, wl.kv_code_std)


def gen_queries(wl: Workload, device="cpu", steps: Optional[int] = None, tag: int = 3) -> torch.Tensor:
    """Per-step queries [steps][L][B][Hq][d]."""
    n = wl.steps if steps is None else steps
    return _normal((n, wl.num_layers, wl.batch, wl.num_q_heads, wl.head_dim),
                   _seed(wl.seed, 13, tag), device, wl.q_torch_dtype)


def gen_scores(wl: Workload, steps: Optional[int] = None, rho: Optional[Tuple[float, ...]] = None) -> np.ndarray:
    """Recall scores [steps][B] float32.

    normal      : N(0,1) (about half of the steps fire at theta = 0)
    rho_minus_u : rho_b - U[0,1), so a step fires with probability rho_b
    exact       : round(rho*steps) steps chosen by a seeded permutation get +1,
                  the others -1 (batch 1 timing runs)."""
    n = wl.steps if steps is None else steps
    r = wl.rho if rho is None else rho
    rho_b = np.array([r[b % len(r)] for b in range(wl.batch)], dtype=np.float64)
    rng = np.random.default_rng([wl.seed, 17, n])
    if wl.score_mode == "normal":
        return rng.standard_normal((n, wl.batch)).astype(np.float32)
    if wl.score_mode == "rho_minus_u":
        u = rng.random((n, wl.batch))
        return (rho_b[None, :] - u).astype(np.float32)
    if wl.score_mode == "exact":
        out = -np.ones((n, wl.batch), dtype=np.float32)
        for b in range(wl.batch):
            k = int(round(rho_b[b] * n))
            chosen = rng.permutation(n)[:k]
            out[chosen, b] = 1.0
        return out
    raise ValueError(wl.score_mode)


def gen_focus(wl: Workload) -> np.ndarray:
    """Per-request focus region [a, b) of 4096 positions inside the prefill: int64 [B][2]."""
    rng = np.random.default_rng([wl.seed, 19])
    width = 4096
    out = np.zeros((wl.batch, 2), dtype=np.int64)
    for b in range(wl.batch):
        hi = max(1, wl.prefill[b] - width + 1)
        a = int(rng.integers(1, hi + 1))
        out[b] = (a, a + width)
    return out


def gen_block_table(wl: Workload, spare_blocks: int = 0) -> Tuple[np.ndarray, int]:
    """Block table int32 [B][max_blocks_per_seq] mapping each request's logical
    blocks to a seeded permutation of physical blocks; unused entries are -1.
    Returns (table, num_blocks)."""
    need = [wl.blocks_for(b) for b in range(wl.batch)]
    total = int(sum(need)) + spare_blocks
    rng = np.random.default_rng([wl.seed, 23])
    if wl.block_order == "sequential":
        perm = np.arange(total, dtype=np.int32)
    else:
        perm = rng.permutation(total).astype(np.int32)
    table = -np.ones((wl.batch, wl.max_blocks_per_seq), dtype=np.int32)
    off = 0
    for b in range(wl.batch):
        table[b, :need[b]] = perm[off:off + need[b]]
        off += need[b]
    return table, total


# Recall-head stand-in: the pages give R_psi's inputs (h_{t-1}, E(x_t), h^L_t
# of a 2048-wide model) and its size on Qwen3-1.7B (28,325,889 parameters),
# not its layers.  One hidden ReLU layer 6144 -> 4608 -> 1 holds 28,320,769.
HEAD_IN_DIM, HEAD_HIDDEN = 3 * 2048, 4608


def gen_recall_head(in_dim: int = HEAD_IN_DIM, hidden: int = HEAD_HIDDEN, seed: int = 7, device="cpu"):
    """Seeded stand-in weights (no trained values exist here): W1 bf16 with
    N(0, 1/in_dim) entries, b1 ~ N(0, 0.1^2), w2 ~ N(0, 2/hidden), all f32 but W1."""
    g = torch.Generator(device=device)
    g.manual_seed(_seed(seed, 29, in_dim, hidden))
    w1 = (torch.randn((hidden, in_dim), generator=g, device=device) * in_dim ** -0.5).to(torch.bfloat16)
    b1 = torch.randn(hidden, generator=g, device=device) * 0.1
    w2 = torch.randn(hidden, generator=g, device=device) * (2.0 / hidden) ** 0.5
    return w1.contiguous(), b1.contiguous(), w2.contiguous()


def gen_head_inputs(wl: Workload, in_dim: int = HEAD_IN_DIM, device="cpu", steps: Optional[int] = None) -> torch.Tensor:
    """Per-step decoding-state inputs [steps][B][in_dim] of the recall head:
    [h_{t-1}; E(x_t); h^L_t] drawn N(0,1) and rounded to bf16."""
    n = wl.steps if steps is None else steps
    return _normal((n, wl.batch, in_dim), _seed(wl.seed, 31, in_dim), device, torch.bfloat16)
