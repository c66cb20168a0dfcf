"""The C-ABI library loads, exports every symbol include/oda.h declares, and
rejects bad arguments on the host before any HIP call (no GPU needed)."""
import ctypes
import os
import re

import pytest

from gated_kv_access_amd import binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "oda.h")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(B.LIB_PATH):
        from gated_kv_access_amd import build
        build.build()
    return B.load()


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(oda_[a-z_]+)\s*\(", text)))


def test_header_declarations_match_binding_list():
    assert _declared() == sorted(B.EXPORTS)


def test_every_declared_symbol_is_exported(lib):
    for name in _declared():
        assert hasattr(lib, name), name


def _dims(**kw):
    d = B.OdaDims()
    base = dict(num_layers=2, num_q_heads=4, num_kv_heads=2, head_dim=128, sink=4, window=64,
                sw_window=0, block_size=16, max_batch=3, max_blocks_per_seq=40, kv_dtype=B.BF16,
                focus=0, full_splits=0, local_splits=0, softmax_scale=0.0, k_scale=0.0, v_scale=0.0,
                reserved0=0, recall_flops=0)
    base.update(kw)
    for k, v in base.items():
        setattr(d, k, v)
    d.layer_kind = None
    return d


FAKE = 0x10000  # 16-byte aligned stand-in; never dereferenced by the cases below


def _kv():
    kv = B.OdaKV()
    for f, _ in B.OdaKV._fields_:
        if f != "num_blocks":
            setattr(kv, f, FAKE)
    kv.num_blocks = 100
    return kv


def test_workspace_size_valid_and_invalid(lib):
    d = _dims()
    n = lib.oda_workspace_size(ctypes.byref(d), 3)
    assert n > 256 and n % 256 == 0
    assert lib.oda_workspace_size(None, 1) == 0
    assert lib.oda_workspace_size(ctypes.byref(_dims(num_q_heads=5)), 1) == 0      # Hq % Hkv
    assert lib.oda_workspace_size(ctypes.byref(_dims(block_size=12)), 1) == 0      # not a power of two
    assert lib.oda_workspace_size(ctypes.byref(_dims(window=0)), 1) == 0
    assert lib.oda_workspace_size(ctypes.byref(_dims()), 4) == 0                   # batch > max_batch
    assert lib.oda_workspace_size(ctypes.byref(_dims(reserved0=1)), 1) == 0
    assert lib.oda_workspace_size(ctypes.byref(_dims(head_dim=96)), 1) == 0        # not built
    assert lib.oda_workspace_size(ctypes.byref(_dims(num_q_heads=32, num_kv_heads=2)), 1) == 0  # group 16
    assert lib.oda_workspace_size(ctypes.byref(_dims(num_q_heads=6, num_kv_heads=2)), 1) == 0   # group 3
    # group 8: built for bf16, FP8 and f32 with d = 64
    assert lib.oda_workspace_size(ctypes.byref(_dims(num_q_heads=16, num_kv_heads=2)), 1) > 0
    assert lib.oda_workspace_size(ctypes.byref(_dims(num_q_heads=16, num_kv_heads=2, kv_dtype=B.F32,
                                                     head_dim=64)), 1) > 0
    assert lib.oda_workspace_size(ctypes.byref(_dims(num_q_heads=16, num_kv_heads=2, kv_dtype=B.F32)), 1) == 0
    assert lib.oda_workspace_size(ctypes.byref(_dims(num_q_heads=16, num_kv_heads=2, kv_dtype=B.FP8_E4M3)),
                                  1) > 0
    assert lib.oda_workspace_size(ctypes.byref(_dims(kv_dtype=3)), 1) == 0
    for bad in (-1.0, float("nan"), float("inf")):
        assert lib.oda_workspace_size(ctypes.byref(_dims(k_scale=bad)), 1) == 0
        assert lib.oda_workspace_size(ctypes.byref(_dims(v_scale=bad)), 1) == 0


def test_fp8_dims_accepted_and_workspace_independent_of_kv_dtype(lib):
    """The split partials are f32 whatever the stored type, so the workspace
    of an FP8 E4M3 cache differs from bf16 only through the split counts."""
    for d in (128, 64):
        n8 = lib.oda_workspace_size(ctypes.byref(_dims(kv_dtype=B.FP8_E4M3, head_dim=d, k_scale=0.05, v_scale=3.0)), 3)
        assert n8 > 256 and n8 % 256 == 0


def _ws(lib, d, batch=3):
    return lib.oda_workspace_size(ctypes.byref(d), batch)


def test_decode_calls_reject_bad_arguments(lib):
    d, kv = _dims(), _kv()
    ws = _ws(lib, d, 1)
    call = lambda *a: lib.oda_decode_local(ctypes.byref(d), ctypes.byref(kv), *a)
    # layer out of range
    assert call(2, 1, FAKE, FAKE, FAKE, FAKE, None, FAKE, ws, None) == -1
    assert call(-1, 1, FAKE, FAKE, FAKE, FAKE, None, FAKE, ws, None) == -1
    # null query / output
    assert call(0, 1, None, FAKE, FAKE, FAKE, None, FAKE, ws, None) == -1
    assert call(0, 1, FAKE, FAKE, FAKE, None, None, FAKE, ws, None) == -1
    # batch beyond max_batch
    assert call(0, 4, FAKE, FAKE, FAKE, FAKE, None, FAKE, ws, None) == -1
    # workspace missing, too small, misaligned
    assert call(0, 1, FAKE, FAKE, FAKE, FAKE, None, None, ws, None) == -4
    assert call(0, 1, FAKE, FAKE, FAKE, FAKE, None, FAKE, ws - 1, None) == -4
    assert call(0, 1, FAKE, FAKE, FAKE, FAKE, None, FAKE + 16, ws, None) == -4
    # misaligned query
    assert call(0, 1, FAKE + 2, FAKE, FAKE, FAKE, None, FAKE, ws, None) == -1
    # unsupported head dim / group (groups 1, 2, 4 and, for bf16, 8 are built)
    for d2 in (_dims(head_dim=96), _dims(num_q_heads=32, num_kv_heads=2), _dims(num_q_heads=6, num_kv_heads=2)):
        assert lib.oda_decode_local(ctypes.byref(d2), ctypes.byref(kv), 0, 1, FAKE, FAKE, FAKE, FAKE, None,
                                    FAKE, 1 << 30, None) == -2
    assert lib.oda_workspace_size(ctypes.byref(_dims(num_q_heads=8, num_kv_heads=2)), 1) > 0
    assert lib.oda_workspace_size(ctypes.byref(_dims(num_q_heads=16, num_kv_heads=2)), 1) > 0
    # missing ring
    kv2 = _kv()
    kv2.k_ring = None
    assert lib.oda_decode_local(ctypes.byref(d), ctypes.byref(kv2), 0, 1, FAKE, FAKE, FAKE, FAKE, None,
                                FAKE, ws, None) == -1


def test_full_gated_and_step_reject_bad_arguments(lib):
    d, kv = _dims(), _kv()
    ws = _ws(lib, d, 1)
    nan = float("nan")
    f = lib.oda_decode_full_gated
    # theta NaN, score missing, missing paged cache
    assert f(ctypes.byref(d), ctypes.byref(kv), 0, 1, FAKE, FAKE, FAKE, FAKE, nan, FAKE, None, None, None,
             FAKE, ws, None) == -1
    assert f(ctypes.byref(d), ctypes.byref(kv), 0, 1, FAKE, FAKE, FAKE, None, 0.0, FAKE, None, None, None,
             FAKE, ws, None) == -1
    kv2 = _kv()
    kv2.block_table = None
    assert f(ctypes.byref(d), ctypes.byref(kv2), 0, 1, FAKE, FAKE, FAKE, FAKE, 0.0, FAKE, None, None, None,
             FAKE, ws, None) == -1
    # focus without focus ranges
    d3 = _dims(focus=1)
    kv3 = _kv()
    kv3.focus_range = None
    assert f(ctypes.byref(d3), ctypes.byref(kv3), 0, 1, FAKE, FAKE, FAKE, FAKE, 0.0, FAKE, None, None,
             None, FAKE, _ws(lib, d3, 1), None) == -1
    s = lib.oda_step
    assert s(ctypes.byref(d), ctypes.byref(kv), 1, None, None, FAKE, FAKE, FAKE, 0.0, FAKE, None, None,
             None, None, None, FAKE, ws, None) == -1
    assert s(ctypes.byref(d), ctypes.byref(kv), 1, FAKE, None, FAKE, FAKE, FAKE, 0.0, FAKE, None, None,
             None, None, None, FAKE, 0, None) == -4
    assert s(ctypes.byref(d), ctypes.byref(kv), 1, FAKE, FAKE + 8, FAKE, FAKE, FAKE, 0.0, FAKE, None, None,
             None, None, None, FAKE, ws, None) == -1


def test_helpers_reject_bad_arguments(lib):
    d, kv = _dims(), _kv()
    ws = _ws(lib, d, 1)
    assert lib.oda_access_set(ctypes.byref(d), ctypes.byref(kv), 0, 3, 0, FAKE, 10, FAKE, FAKE, ws, None) == -1
    assert lib.oda_access_set(ctypes.byref(d), ctypes.byref(kv), 0, 0, 2, FAKE, 10, FAKE, FAKE, ws, None) == -1
    assert lib.oda_access_set(ctypes.byref(d), ctypes.byref(kv), 0, 0, 0, FAKE, 0, FAKE, FAKE, ws, None) == -1
    assert lib.oda_prefill_kv(ctypes.byref(d), ctypes.byref(kv), 1, 5, FAKE, FAKE, 10, FAKE, ws, None) == -1
    assert lib.oda_prefill_kv(ctypes.byref(d), ctypes.byref(kv), 1, 0, FAKE, FAKE, -1, FAKE, ws, None) == -1
    assert lib.oda_commit_kv(ctypes.byref(d), ctypes.byref(kv), 1, None, FAKE, FAKE, ws, None) == -1
    assert lib.oda_gate(ctypes.byref(d), ctypes.byref(kv), 1, None, 0.0, None, None, None, None, None) == -1
    assert lib.oda_gate(ctypes.byref(d), None, 1, FAKE, 0.0, None, None, None, None, None) == -1
    arr = (ctypes.c_void_p * 1)(FAKE)
    by = (ctypes.c_int64 * 1)(24)  # not a multiple of 16
    assert lib.oda_stage_step(1, arr, arr, by, FAKE, 4, None) == -1
    assert lib.oda_stage_step(0, arr, arr, by, FAKE, 4, None) == -1
    assert lib.oda_advance_counter(None, None) == -1
    out = ctypes.c_void_p()
    assert lib.oda_host_kv_pointer(None, ctypes.byref(out)) == -1
    assert lib.oda_host_kv_pointer(FAKE, None) == -1


def test_status_strings(lib):
    for code, name in [(0, "ODA_OK"), (-1, "ODA_ERR_INVALID_ARG"), (-2, "ODA_ERR_UNSUPPORTED"),
                       (-3, "ODA_ERR_HIP"), (-4, "ODA_ERR_WORKSPACE")]:
        assert B.status_string(code) == name


def test_workspace_size_is_deterministic_and_monotone_in_batch(lib):
    d = _dims(max_batch=64)
    sizes = [lib.oda_workspace_size(ctypes.byref(d), b) for b in (1, 2, 8, 64)]
    assert all(s > 0 for s in sizes)
    assert sizes == [lib.oda_workspace_size(ctypes.byref(d), b) for b in (1, 2, 8, 64)]


def test_empty_batch_is_a_no_op(lib):
    """batch 0: every call validates and returns ODA_OK without launching (no GPU here)."""
    d, kv = _dims(), _kv()
    ws = _ws(lib, d, 0)
    assert ws > 0
    assert lib.oda_step(ctypes.byref(d), ctypes.byref(kv), 0, FAKE, None, FAKE, FAKE, FAKE, 0.0, FAKE, None,
                        None, None, None, None, FAKE, ws, None) == 0


def test_step_static_rejects_bad_arguments_before_any_launch(lib):
    """The entry point without a workspace validates like oda_step and refuses
    dims whose workspace exceeds its static scratch, all on the host."""
    d, kv = _dims(), _kv()
    s = lib.oda_step_static
    args = lambda **o: [o.get(k, v) for k, v in (("q", FAKE), ("qf", None), ("k", FAKE), ("v", FAKE),
                                                 ("sc", FAKE), ("th", 0.0), ("out", FAKE))]
    call = lambda dims, batch, **o: s(ctypes.byref(dims), ctypes.byref(kv), batch, *args(**o), None, None,
                                      None, None, None, None)
    assert call(d, 1, q=None) == -1
    assert call(d, 1, sc=None) == -1
    assert call(d, 1, out=None) == -1
    assert call(d, 1, th=float("nan")) == -1
    assert call(d, 1, qf=FAKE + 8) == -1
    assert call(d, 4) == -1                                  # batch > max_batch
    assert call(_dims(head_dim=96), 1) == -2                 # not built
    assert call(d, 0) == 0                                   # empty batch: nothing launched
    # a workspace above the 4 MiB of static scratch is refused
    big = _dims(max_batch=4096, max_blocks_per_seq=8192, num_q_heads=64, num_kv_heads=8)
    assert lib.oda_workspace_size(ctypes.byref(big), 4096) > 4 << 20
    assert call(big, 4096) == -4
    kv2 = _kv()
    kv2.k_ring = None
    assert s(ctypes.byref(d), ctypes.byref(kv2), 1, *args(), None, None, None, None, None, None) == -1


def test_profiling_build_exports_the_phase_calls():
    """liboda_phases.so (the profiling build) exports what include/oda_phases.h
    declares on top of every oda.h symbol; the product library exports none of it."""
    from gated_kv_access_amd.build import PHASES_LIB
    if not os.path.exists(PHASES_LIB):
        from gated_kv_access_amd import build
        build.build(phases=True)
    text = re.sub(r"/\*.*?\*/", "", open(os.path.join(ROOT, "include", "oda_phases.h")).read(), flags=re.S)
    declared = sorted(set(re.findall(r"\b(oda_[a-z_]+)\s*\(", text)))
    assert declared == ["oda_phase_stamps_clear", "oda_phase_stamps_read"]
    prof = ctypes.CDLL(PHASES_LIB)
    for name in declared + _declared():
        assert hasattr(prof, name), name
    product = ctypes.CDLL(B.LIB_PATH)
    for name in declared:
        assert not hasattr(product, name), name
