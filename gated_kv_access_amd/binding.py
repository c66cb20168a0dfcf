"""ctypes binding of liboda.so (include/oda.h) -- argument marshalling only.

Every function here has the C name without the ``oda_`` prefix, takes torch
tensors (device memory) or ctypes structs, passes their pointers and the
current HIP stream to the library, and raises :class:`OdaError` on a negative
status.  There is no fallback: if the library is missing the import of a
wrapper fails loudly.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "liboda.so")

BF16, F32, FP8_E4M3 = 0, 1, 2
LAYER_GATED, LAYER_SLIDING = 0, 1
ACCT_FIELDS = ("steps", "full_calls", "f_local", "f_full_taken", "f_full_always",
               "delta_f", "kv_bytes", "f_recall")
DEVERR_CAPACITY, DEVERR_BLOCK_ID, DEVERR_OUT_CAPACITY, DEVERR_MERGE_WAIT = 1, 2, 4, 8

# Every symbol include/oda.h declares.
EXPORTS = ("oda_workspace_size", "oda_workspace_init", "oda_prefill_kv", "oda_ring_init",
           "oda_commit_kv", "oda_decode_local", "oda_decode_full_gated", "oda_gate", "oda_step",
           "oda_step_static",
           "oda_access_set", "oda_stage_step", "oda_advance_counter", "oda_host_kv_pointer",
           "oda_recall_workspace_size", "oda_recall_workspace_init", "oda_recall_scores", "oda_step_recall",
           "oda_test_merge_wait", "oda_status_string")


class OdaError(RuntimeError):
    def __init__(self, fn: str, status: int):
        super().__init__(f"{fn} failed: {status_string(status)} ({status})")
        self.status = status


class OdaDims(ctypes.Structure):
    _fields_ = [
        ("num_layers", ctypes.c_int32), ("num_q_heads", ctypes.c_int32),
        ("num_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
        ("sink", ctypes.c_int32), ("window", ctypes.c_int32), ("sw_window", ctypes.c_int32),
        ("block_size", ctypes.c_int32), ("max_batch", ctypes.c_int32),
        ("max_blocks_per_seq", ctypes.c_int32), ("kv_dtype", ctypes.c_int32),
        ("focus", ctypes.c_int32), ("full_splits", ctypes.c_int32),
        ("local_splits", ctypes.c_int32), ("softmax_scale", ctypes.c_float),
        ("k_scale", ctypes.c_float), ("v_scale", ctypes.c_float),
        ("reserved0", ctypes.c_int32), ("recall_flops", ctypes.c_int64),
        ("layer_kind", ctypes.c_void_p),
    ]


class OdaRecallHead(ctypes.Structure):
    _fields_ = [
        ("in_dim", ctypes.c_int32), ("hidden", ctypes.c_int32),
        ("w1", ctypes.c_void_p), ("b1", ctypes.c_void_p), ("w2", ctypes.c_void_p),
        ("b2", ctypes.c_float), ("reserved0", ctypes.c_int32),
    ]


class OdaKV(ctypes.Structure):
    _fields_ = [
        ("k_cache", ctypes.c_void_p), ("v_cache", ctypes.c_void_p),
        ("k_ring", ctypes.c_void_p), ("v_ring", ctypes.c_void_p),
        ("k_swring", ctypes.c_void_p), ("v_swring", ctypes.c_void_p),
        ("ring_pos", ctypes.c_void_p), ("swring_pos", ctypes.c_void_p),
        ("block_table", ctypes.c_void_p), ("seq_len", ctypes.c_void_p),
        ("focus_range", ctypes.c_void_p), ("num_blocks", ctypes.c_int64),
    ]


_lib = None


def load(path: str = LIB_PATH):
    """Loads liboda.so (built by __graft_entry__.build()); raises if absent."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise FileNotFoundError(f"{path} is missing: build it with __graft_entry__.build()")
    L = ctypes.CDLL(path)
    P, I32, I64, SZ, F = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t, ctypes.c_float
    D, K = ctypes.POINTER(OdaDims), ctypes.POINTER(OdaKV)
    sig = {
        "oda_workspace_size": (SZ, [D, I32]),
        "oda_workspace_init": (I32, [D, I32, P, SZ, P]),
        "oda_prefill_kv": (I32, [D, K, I32, I32, P, P, I64, P, SZ, P]),
        "oda_ring_init": (I32, [D, K, I32, P, SZ, P]),
        "oda_commit_kv": (I32, [D, K, I32, P, P, P, SZ, P]),
        "oda_decode_local": (I32, [D, K, I32, I32, P, P, P, P, P, P, SZ, P]),
        "oda_decode_full_gated": (I32, [D, K, I32, I32, P, P, P, P, F, P, P, P, P, P, SZ, P]),
        "oda_gate": (I32, [D, K, I32, P, F, P, P, P, P, P]),
        "oda_step": (I32, [D, K, I32, P, P, P, P, P, F, P, P, P, P, P, P, P, SZ, P]),
        "oda_step_static": (I32, [D, K, I32, P, P, P, P, P, F, P, P, P, P, P, P, P]),
        "oda_access_set": (I32, [D, K, I32, I32, I32, P, I64, P, P, SZ, P]),
        "oda_stage_step": (I32, [I32, P, P, P, P, I64, P]),
        "oda_advance_counter": (I32, [P, P]),
        "oda_host_kv_pointer": (I32, [P, ctypes.POINTER(ctypes.c_void_p)]),
        "oda_recall_workspace_size": (SZ, [ctypes.POINTER(OdaRecallHead), I32]),
        "oda_recall_workspace_init": (I32, [ctypes.POINTER(OdaRecallHead), I32, P, SZ, P]),
        "oda_recall_scores": (I32, [ctypes.POINTER(OdaRecallHead), I32, P, P, P, SZ, P]),
        "oda_step_recall": (I32, [D, K, I32, P, P, P, P, ctypes.POINTER(OdaRecallHead), P, P, F, P, P, P, P,
                                  P, P, P, SZ, P, SZ, P]),
        "oda_test_merge_wait": (I32, [D, K, I32, I32, P, P, P, P, P, I32, I32, P, SZ, P]),
        "oda_status_string": (ctypes.c_char_p, [I32]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(L, name)
        fn.restype = res
        fn.argtypes = args
    _lib = L
    return L


def status_string(status: int) -> str:
    return load().oda_status_string(int(status)).decode()


def _p(t: Optional[torch.Tensor]):
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError("expected a torch tensor")
    if not t.is_contiguous():
        raise ValueError("tensors passed to liboda must be contiguous")
    return t.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream if torch.cuda.is_available() else None
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _check(fn: str, rc: int) -> None:
    if rc != 0:
        raise OdaError(fn, rc)


def workspace_size(dims: OdaDims, batch: int) -> int:
    return int(load().oda_workspace_size(ctypes.byref(dims), batch))


def workspace_init(dims: OdaDims, batch: int, ws: torch.Tensor, stream=None) -> None:
    _check("oda_workspace_init", load().oda_workspace_init(ctypes.byref(dims), batch, _p(ws),
                                                           ws.numel() * ws.element_size(), _stream(stream)))


def prefill_kv(dims, kv, batch, layer, k_src, v_src, src_rows, ws, stream=None) -> None:
    _check("oda_prefill_kv", load().oda_prefill_kv(ctypes.byref(dims), ctypes.byref(kv), batch, layer,
                                                   _p(k_src), _p(v_src), src_rows, _p(ws),
                                                   ws.numel() * ws.element_size(), _stream(stream)))


def ring_init(dims, kv, batch, ws, stream=None) -> None:
    _check("oda_ring_init", load().oda_ring_init(ctypes.byref(dims), ctypes.byref(kv), batch, _p(ws),
                                                 ws.numel() * ws.element_size(), _stream(stream)))


def commit_kv(dims, kv, batch, k_new, v_new, ws, stream=None) -> None:
    _check("oda_commit_kv", load().oda_commit_kv(ctypes.byref(dims), ctypes.byref(kv), batch, _p(k_new),
                                                 _p(v_new), _p(ws), ws.numel() * ws.element_size(),
                                                 _stream(stream)))


def decode_local(dims, kv, layer, batch, q, k_cur, v_cur, out, lse, ws, stream=None) -> None:
    _check("oda_decode_local", load().oda_decode_local(
        ctypes.byref(dims), ctypes.byref(kv), layer, batch, _p(q), _p(k_cur), _p(v_cur), _p(out),
        _p(lse), _p(ws), ws.numel() * ws.element_size(), _stream(stream)))


def test_merge_wait(dims, kv, layer, batch, q, k_cur, v_cur, out, lse, withheld_split, spin_limit, ws,
                    stream=None) -> None:
    _check("oda_test_merge_wait", load().oda_test_merge_wait(
        ctypes.byref(dims), ctypes.byref(kv), layer, batch, _p(q), _p(k_cur), _p(v_cur), _p(out), _p(lse),
        int(withheld_split), int(spin_limit), _p(ws), ws.numel() * ws.element_size(), _stream(stream)))


def decode_full_gated(dims, kv, layer, batch, q, k_cur, v_cur, recall_score, theta, out, lse,
                      call_list, call_count, ws, stream=None) -> None:
    _check("oda_decode_full_gated", load().oda_decode_full_gated(
        ctypes.byref(dims), ctypes.byref(kv), layer, batch, _p(q), _p(k_cur), _p(v_cur),
        _p(recall_score), float(theta), _p(out), _p(lse), _p(call_list), _p(call_count), _p(ws),
        ws.numel() * ws.element_size(), _stream(stream)))


def gate(dims, kv, batch, recall_score, theta, call_list=None, call_count=None, full_calls=None,
         counters=None, stream=None) -> None:
    _check("oda_gate", load().oda_gate(ctypes.byref(dims), ctypes.byref(kv), batch, _p(recall_score),
                                       float(theta), _p(call_list), _p(call_count), _p(full_calls),
                                       _p(counters), _stream(stream)))


def step(dims, kv, batch, q_local, q_full, k_new, v_new, recall_score, theta, out, lse, call_list,
         call_count, full_calls, counters, ws, stream=None) -> None:
    _check("oda_step", load().oda_step(
        ctypes.byref(dims), ctypes.byref(kv), batch, _p(q_local), _p(q_full), _p(k_new), _p(v_new),
        _p(recall_score), float(theta), _p(out), _p(lse), _p(call_list), _p(call_count),
        _p(full_calls), _p(counters), _p(ws), ws.numel() * ws.element_size(), _stream(stream)))


def step_static(dims, kv, batch, q_local, q_full, k_new, v_new, recall_score, theta, out, lse, call_list,
                call_count, full_calls, counters, stream=None) -> None:
    _check("oda_step_static", load().oda_step_static(
        ctypes.byref(dims), ctypes.byref(kv), batch, _p(q_local), _p(q_full), _p(k_new), _p(v_new),
        _p(recall_score), float(theta), _p(out), _p(lse), _p(call_list), _p(call_count),
        _p(full_calls), _p(counters), _stream(stream)))


def access_set(dims, kv, layer, b, mode, positions, count, ws, stream=None) -> None:
    _check("oda_access_set", load().oda_access_set(
        ctypes.byref(dims), ctypes.byref(kv), layer, b, mode, _p(positions), positions.numel(),
        _p(count), _p(ws), ws.numel() * ws.element_size(), _stream(stream)))


def stage_step(srcs: Sequence[torch.Tensor], dsts: Sequence[torch.Tensor], step_counter: torch.Tensor,
               num_steps: int, stream=None) -> None:
    n = len(srcs)
    src_arr = (ctypes.c_void_p * n)(*[_p(s) for s in srcs])
    dst_arr = (ctypes.c_void_p * n)(*[_p(d) for d in dsts])
    by = (ctypes.c_int64 * n)(*[d.numel() * d.element_size() for d in dsts])
    _check("oda_stage_step", load().oda_stage_step(n, src_arr, dst_arr, by, _p(step_counter), num_steps,
                                                   _stream(stream)))


def advance_counter(step_counter: torch.Tensor, stream=None) -> None:
    _check("oda_advance_counter", load().oda_advance_counter(_p(step_counter), _stream(stream)))


def make_head(w1: torch.Tensor, b1: torch.Tensor, w2: torch.Tensor, b2: float) -> OdaRecallHead:
    """Recall-head descriptor over device tensors (kept alive by the caller)."""
    h = OdaRecallHead()
    h.hidden, h.in_dim = int(w1.shape[0]), int(w1.shape[1])
    h.w1, h.b1, h.w2 = _p(w1), _p(b1), _p(w2)
    h.b2 = float(b2)
    h.reserved0 = 0
    return h


def recall_workspace_size(head: OdaRecallHead, batch: int) -> int:
    return int(load().oda_recall_workspace_size(ctypes.byref(head), batch))


def recall_workspace_init(head: OdaRecallHead, batch: int, ws: torch.Tensor, stream=None) -> None:
    _check("oda_recall_workspace_init", load().oda_recall_workspace_init(
        ctypes.byref(head), batch, _p(ws), ws.numel() * ws.element_size(), _stream(stream)))


def recall_scores(head: OdaRecallHead, batch: int, x: torch.Tensor, scores: torch.Tensor, ws: torch.Tensor,
                  stream=None) -> None:
    _check("oda_recall_scores", load().oda_recall_scores(ctypes.byref(head), batch, _p(x), _p(scores), _p(ws),
                                                         ws.numel() * ws.element_size(), _stream(stream)))


def step_recall(dims, kv, batch, q_local, q_full, k_new, v_new, head, head_x, recall_score, theta, out, lse,
                call_list, call_count, full_calls, counters, ws, head_ws, stream=None) -> None:
    _check("oda_step_recall", load().oda_step_recall(
        ctypes.byref(dims), ctypes.byref(kv), batch, _p(q_local), _p(q_full), _p(k_new), _p(v_new),
        ctypes.byref(head), _p(head_x), _p(recall_score), float(theta), _p(out), _p(lse), _p(call_list),
        _p(call_count), _p(full_calls), _p(counters), _p(ws), ws.numel() * ws.element_size(), _p(head_ws),
        head_ws.numel() * head_ws.element_size(), _stream(stream)))


def host_kv_pointer(t: torch.Tensor) -> int:
    """Device address of a pinned host tensor (for host-resident paged caches)."""
    out = ctypes.c_void_p()
    _check("oda_host_kv_pointer", load().oda_host_kv_pointer(ctypes.c_void_p(t.data_ptr()), ctypes.byref(out)))
    return out.value
