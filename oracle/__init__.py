"""CPU fp64 oracle for the On-Demand Attention decode step -- TEST INFRASTRUCTURE.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The HIP library never calls it, and it
never calls the HIP library: the two share no code.

The arithmetic lives in ``oda_oracle.c`` (plain C, fp64, libm); this module
only marshals numpy arrays through ctypes.  Sources followed:

* picx.dev summary of "On-Demand Attention", section "Local-First Decoding":
  the access sets S^F_t and S^L_t, the Local pass / recall score, and the gate
  q_t > theta with theta = 0;
* same page, section "Computational Savings": the per-step savings equation;
* the Declarative Attention pages ("Three Attention Modes"): focus reads one
  contiguous region; sliding-window layers keep a fixed recent window;
* the recall score q_t = R_psi(h_{t-1}, E(x_t), h^L_t) of "Local-First
  Decoding", with a one-hidden-layer stand-in for R_psi (the pages give its
  inputs and size, not its layers).
"""
from __future__ import annotations

import contextlib
import ctypes
import os
from dataclasses import dataclass, field
from typing import Optional, Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "liboda_oracle.so")

BF16, F32, FP8 = 0, 1, 2
GATED, SLIDING = 0, 1
LOCAL, FULL = 0, 1
ACCT_FIELDS = ("steps", "full_calls", "f_local", "f_full_taken", "f_full_always",
               "delta_f", "kv_bytes", "f_recall")


class _Cfg(ctypes.Structure):
    _fields_ = [
        ("num_layers", ctypes.c_int32), ("num_q_heads", ctypes.c_int32),
        ("num_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
        ("sink", ctypes.c_int32), ("window", ctypes.c_int32),
        ("sw_window", ctypes.c_int32), ("dtype", ctypes.c_int32),
        ("focus", ctypes.c_int32), ("pad_", ctypes.c_int32),
        ("scale", ctypes.c_double), ("recall_flops", ctypes.c_int64),
        ("k_scale", ctypes.c_double), ("v_scale", ctypes.c_double),
        ("layer_kind", ctypes.c_void_p),
    ]


@dataclass
class OracleConfig:
    num_layers: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    sink: int = 4
    window: int = 2048
    sw_window: int = 0
    dtype: int = BF16
    focus: bool = False
    scale: float = 0.0
    recall_flops: int = 0
    layer_kind: Optional[Sequence[int]] = None
    k_scale: float = 1.0
    v_scale: float = 1.0
    _kinds: Optional[np.ndarray] = field(default=None, repr=False)

    def to_c(self) -> _Cfg:
        c = _Cfg()
        c.num_layers, c.num_q_heads = self.num_layers, self.num_q_heads
        c.num_kv_heads, c.head_dim = self.num_kv_heads, self.head_dim
        c.sink, c.window, c.sw_window = self.sink, self.window, self.sw_window
        c.dtype, c.focus, c.pad_ = self.dtype, int(bool(self.focus)), 0
        c.scale, c.recall_flops = float(self.scale), int(self.recall_flops)
        c.k_scale, c.v_scale = float(self.k_scale), float(self.v_scale)
        if self.layer_kind is not None:
            self._kinds = np.ascontiguousarray(np.asarray(self.layer_kind, dtype=np.uint8))
            assert self._kinds.shape == (self.num_layers,)
            c.layer_kind = self._kinds.ctypes.data
        else:
            c.layer_kind = None
        return c


_lib = None


def _bind(path: str):
    L = ctypes.CDLL(path)
    P = ctypes.c_void_p
    L.oracle_in_set.argtypes = [ctypes.POINTER(_Cfg), ctypes.c_int32, ctypes.c_int32,
                                ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64]
    L.oracle_in_set.restype = ctypes.c_int
    L.oracle_access_set.argtypes = [ctypes.POINTER(_Cfg), ctypes.c_int32, ctypes.c_int32,
                                    ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, P]
    L.oracle_access_set.restype = ctypes.c_int64
    L.oracle_attention.argtypes = [P, P, P, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                   ctypes.c_int32, ctypes.c_double, ctypes.c_double, ctypes.c_double, P,
                                   ctypes.c_int64, P, P]
    L.oracle_recall_head.argtypes = [ctypes.c_int32, ctypes.c_int32, P, P, P, ctypes.c_float, P, ctypes.c_int32, P]
    L.oracle_recall_head.restype = None
    L.oracle_fp8_e4m3.argtypes = [ctypes.c_uint8]
    L.oracle_fp8_e4m3.restype = ctypes.c_double
    L.oracle_attention.restype = ctypes.c_double
    L.oracle_gate.argtypes = [ctypes.c_float, ctypes.c_float]
    L.oracle_gate.restype = ctypes.c_int
    L.oracle_step_accounting.argtypes = [ctypes.POINTER(_Cfg), ctypes.c_int64, ctypes.c_int32,
                                         ctypes.c_int64, ctypes.c_int64, P]
    L.oracle_step_accounting.restype = None
    L.oracle_decode_run.argtypes = [ctypes.POINTER(_Cfg), ctypes.c_int32, ctypes.c_int32, P,
                                    ctypes.c_int64, P, P, P, P, P, ctypes.c_float, P, P,
                                    P, P, P, P, P, P, P]
    L.oracle_decode_run.restype = ctypes.c_int
    L.oracle_set_threads.argtypes = [ctypes.c_int32]
    L.oracle_set_threads.restype = None
    L.oracle_get_threads.argtypes = []
    L.oracle_get_threads.restype = ctypes.c_int32
    return L


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            from . import build as _b
            _b.build()
        _lib = _bind(_LIB_PATH)
    return _lib


@contextlib.contextmanager
def using_library(path: str):
    """Temporarily route every call through another build of the oracle source
    (the mutation tests use this to show the pins reject planted mistakes)."""
    global _lib
    saved = lib()
    _lib = _bind(path)
    try:
        yield
    finally:
        _lib = saved


def _ptr(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data


def _raw(a: np.ndarray, dtype: int) -> np.ndarray:
    """Input arrays travel as raw element words: uint16 for bf16, float32 for f32,
    uint8 for FP8 E4M3."""
    want = {BF16: np.uint16, F32: np.float32, FP8: np.uint8}[dtype]
    if a.dtype != want:
        raise TypeError(f"expected {want} array for dtype {dtype}, got {a.dtype}")
    return np.ascontiguousarray(a)


def set_threads(n: int) -> None:
    lib().oracle_set_threads(int(n))


def get_threads() -> int:
    return int(lib().oracle_get_threads())


def in_set(cfg: OracleConfig, kind: int, mode: int, t: int, p: int, fa: int = 0, fb: int = 0) -> bool:
    c = cfg.to_c()
    return bool(lib().oracle_in_set(ctypes.byref(c), kind, mode, t, p, fa, fb))


def access_set(cfg: OracleConfig, kind: int, mode: int, t: int, fa: int = 0, fb: int = 0) -> np.ndarray:
    c = cfg.to_c()
    out = np.zeros(max(int(t), 1), dtype=np.int64)
    n = lib().oracle_access_set(ctypes.byref(c), kind, mode, t, fa, fb, _ptr(out))
    return out[:n].copy()


def gate(score: float, theta: float = 0.0) -> bool:
    return bool(lib().oracle_gate(score, theta))


def _qtype(dtype: int) -> int:
    return BF16 if dtype == FP8 else dtype


def fp8_e4m3(code: int) -> float:
    return float(lib().oracle_fp8_e4m3(int(code)))


def attention(q: np.ndarray, kseq: np.ndarray, vseq: np.ndarray, g: int, positions: np.ndarray,
              dtype: int, scale: float = 0.0, k_scale: float = 1.0, v_scale: float = 1.0):
    """One query head over one request's sequence rows.

    q: [d] (bf16 words when K/V are FP8); kseq, vseq: [T][Hkv][d] raw words;
    positions: 1-based int64.  Returns (out[d] float64, lse float)."""
    q, kseq, vseq = _raw(q, _qtype(dtype)), _raw(kseq, dtype), _raw(vseq, dtype)
    T, Hkv, d = kseq.shape
    pos = np.ascontiguousarray(positions, dtype=np.int64)
    assert pos.size == 0 or (pos.min() >= 1 and pos.max() <= T)
    out = np.zeros(d, dtype=np.float64)
    z = np.zeros(max(pos.size, 1), dtype=np.float64)
    sc = scale if scale > 0 else 1.0 / np.sqrt(d)
    lse = lib().oracle_attention(_ptr(q), _ptr(kseq), _ptr(vseq), Hkv, d, g, dtype, sc, k_scale, v_scale,
                                 _ptr(pos), pos.size, _ptr(out), _ptr(z))
    return out, float(lse)


def step_accounting(cfg: OracleConfig, t: int, fired: bool, fa: int = 0, fb: int = 0) -> dict:
    c = cfg.to_c()
    acct = np.zeros(len(ACCT_FIELDS), dtype=np.int64)
    lib().oracle_step_accounting(ctypes.byref(c), t, int(bool(fired)), fa, fb, _ptr(acct))
    return dict(zip(ACCT_FIELDS, (int(x) for x in acct)))


def decode_run(cfg: OracleConfig, prefill: Sequence[int], kseq: np.ndarray, vseq: np.ndarray,
               q_local: np.ndarray, score: np.ndarray, theta: float = 0.0,
               q_full: Optional[np.ndarray] = None, focus: Optional[np.ndarray] = None,
               active: Optional[np.ndarray] = None) -> dict:
    """Runs K decode steps for B requests.

    kseq, vseq: [L][B][T][Hkv][d] raw words holding every position of the run;
    q_local (and q_full): [K][L][B][Hq][d]; score: [K][B] float32."""
    kseq, vseq = _raw(kseq, cfg.dtype), _raw(vseq, cfg.dtype)
    q_local = _raw(q_local, _qtype(cfg.dtype))
    q_full = None if q_full is None else _raw(q_full, _qtype(cfg.dtype))
    L, B, T, Hkv, d = kseq.shape
    K = q_local.shape[0]
    Hq = cfg.num_q_heads
    assert q_local.shape == (K, L, B, Hq, d), q_local.shape
    score = np.ascontiguousarray(score, dtype=np.float32)
    assert score.shape == (K, B)
    pre = np.ascontiguousarray(np.asarray(prefill, dtype=np.int64))
    foc = None if focus is None else np.ascontiguousarray(focus, dtype=np.int64)
    act = None if active is None else np.ascontiguousarray(active, dtype=np.uint8)
    out = np.zeros((K, L, B, Hq, d), dtype=np.float64)
    lse = np.zeros((K, L, B, Hq), dtype=np.float64)
    fire = np.zeros((K, B), dtype=np.uint8)
    call_list = np.zeros((K, B), dtype=np.int32)
    call_count = np.zeros(K, dtype=np.int32)
    full_calls = np.zeros(B, dtype=np.int64)
    acct = np.zeros((B, len(ACCT_FIELDS)), dtype=np.int64)
    c = cfg.to_c()
    rc = lib().oracle_decode_run(ctypes.byref(c), B, K, _ptr(pre), T, _ptr(kseq), _ptr(vseq),
                                 _ptr(q_local), _ptr(q_full), _ptr(score), float(theta), _ptr(foc),
                                 _ptr(act), _ptr(out), _ptr(lse), _ptr(fire), _ptr(call_list),
                                 _ptr(call_count), _ptr(full_calls), _ptr(acct))
    if rc != 0:
        raise ValueError("oracle_decode_run rejected its arguments")
    return dict(out=out, lse=lse, fire=fire, call_list=call_list, call_count=call_count,
                full_calls=full_calls, acct=acct)


def recall_head(w1: np.ndarray, b1: np.ndarray, w2: np.ndarray, b2: float, x: np.ndarray) -> np.ndarray:
    """Recall scores q [batch] (float64) of the one-hidden-layer stand-in head.

    w1: bf16 words [hidden][in_dim]; b1, w2: float32 [hidden]; x: bf16 words [batch][in_dim]."""
    w1 = np.ascontiguousarray(w1, dtype=np.uint16)
    x = np.ascontiguousarray(np.atleast_2d(x), dtype=np.uint16)
    b1 = np.ascontiguousarray(b1, dtype=np.float32)
    w2 = np.ascontiguousarray(w2, dtype=np.float32)
    hidden, in_dim = w1.shape
    assert x.shape[1] == in_dim and b1.shape == (hidden,) and w2.shape == (hidden,)
    q = np.zeros(x.shape[0], dtype=np.float64)
    lib().oracle_recall_head(in_dim, hidden, _ptr(w1), _ptr(b1), _ptr(w2), float(b2), _ptr(x), x.shape[0], _ptr(q))
    return q


def bf16_to_f64(w: np.ndarray) -> np.ndarray:
    return (np.asarray(w, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)
