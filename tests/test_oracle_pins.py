"""Pins of the CPU oracle against what the pages and the mathematics fix.

Every check here compares the oracle with something other than itself:
hand-worked fixtures (tests/golden/), closed forms of set sizes, a textbook
library routine (torch scaled_dot_product_attention in float64 on the CPU),
special cases with known answers, and brute-force counts done by numpy.
Sources: picx.dev summary of On-Demand Attention, sections "Local-First
Decoding" (access sets, Local pass, gate q_t > theta, theta = 0) and
"Computational Savings" (per-step savings equation).
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle as orc

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _cfg(**kw):
    base = dict(num_layers=1, num_q_heads=1, num_kv_heads=1, head_dim=1, sink=4, window=3)
    base.update(kw)
    return orc.OracleConfig(**base)


# --------------------------------------------------------------------------- access sets

@pytest.mark.parametrize("case", _load("access_sets.json")["local"])
def test_local_set_worked_examples(case):
    got = orc.access_set(_cfg(sink=case["s"], window=case["w"]), orc.GATED, orc.LOCAL, case["t"])
    assert got.tolist() == case["expect"]


def test_local_set_summary_example():
    for case in _load("access_sets.json")["local_summary"]:
        got = orc.access_set(_cfg(sink=case["s"], window=case["w"]), orc.GATED, orc.LOCAL, case["t"])
        assert got.size == case["count"]
        assert got[: len(case["head"])].tolist() == case["head"]
        assert got[-1] == case["last"]


@pytest.mark.parametrize("case", _load("access_sets.json")["sliding"])
def test_sliding_set_worked_examples(case):
    cfg = _cfg(sw_window=case["W"])
    got = orc.access_set(cfg, orc.SLIDING, orc.LOCAL, case["t"])
    full = orc.access_set(cfg, orc.SLIDING, orc.FULL, case["t"])
    assert got.tolist() == full.tolist(), "a sliding-window layer reads the same window in both modes"
    if "expect" in case:
        assert got.tolist() == case["expect"]
    else:
        assert got.size == case["expect_count"] and got[-1] == case["t"]


@pytest.mark.parametrize("case", _load("access_sets.json")["focus"])
def test_focus_set_worked_examples(case):
    cfg = _cfg(sink=case["s"], window=case["w"], focus=True)
    got = orc.access_set(cfg, orc.GATED, orc.FULL, case["t"], case["a"], case["b"])
    assert got.tolist() == case["expect"]


@pytest.mark.parametrize("s", [0, 1, 4])
@pytest.mark.parametrize("w", [1, 64, 2048])
def test_local_set_size_closed_form(s, w):
    """|S^L_t| = min(t, s+w): the two ranges of the equation are disjoint once
    t > s+w and cover {1..t} otherwise."""
    cfg = _cfg(sink=s, window=w)
    ts = sorted(set(list(range(1, min(3 * (s + w), 300) + 1)) + [s + w - 1, s + w, s + w + 1, 3 * (s + w)]))
    for t in ts:
        if t < 1:
            continue
        got = orc.access_set(cfg, orc.GATED, orc.LOCAL, t)
        assert got.size == min(t, s + w), (t, got.size)
        assert got[-1] == t, "the current token is always attended"
        assert np.all(np.diff(got) > 0)
        # the most recent min(w, t) positions are all present
        assert set(range(max(1, t - w + 1), t + 1)) <= set(got.tolist())
        full = orc.access_set(cfg, orc.GATED, orc.FULL, t)
        assert full.tolist() == list(range(1, t + 1))
        assert (got.tolist() == full.tolist()) == (t <= s + w)


def test_full_set_is_all_positions():
    cfg = _cfg(sink=4, window=2048)
    for t in (1, 2, 2052, 2053, 10000):
        assert orc.access_set(cfg, orc.GATED, orc.FULL, t).tolist() == list(range(1, t + 1))


# --------------------------------------------------------------------------- attention

@pytest.mark.parametrize("case", _load("attention_worked.json")["cases"])
def test_attention_worked_examples(case):
    d = case["d"]
    q = np.array(case["q"], dtype=np.float32)
    K = np.array(case["K"], dtype=np.float32).reshape(-1, 1, d)
    V = np.array(case["V"], dtype=np.float32).reshape(-1, 1, d)
    pos = np.arange(1, K.shape[0] + 1, dtype=np.int64)
    out, lse = orc.attention(q, K, V, 0, pos, orc.F32)
    np.testing.assert_allclose(out, case["expect_out"], atol=case["tol"], rtol=0)
    assert abs(lse - case["expect_lse"]) <= case["tol"]


def _words(x: torch.Tensor, dtype: int) -> np.ndarray:
    if dtype == orc.BF16:
        return x.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    return x.to(torch.float32).numpy()


def _as_f64(x: torch.Tensor, dtype: int) -> torch.Tensor:
    return (x.to(torch.bfloat16) if dtype == orc.BF16 else x.to(torch.float32)).to(torch.float64)


@pytest.mark.parametrize("dtype", [orc.F32, orc.BF16])
@pytest.mark.parametrize("d", [64, 128])
def test_attention_matches_torch_sdpa_float64(dtype, d):
    """Textbook cross-check: torch's scaled_dot_product_attention in float64 on
    the gathered positions equals the oracle within 1e-12."""
    g = torch.Generator().manual_seed(1234 + d + dtype)
    T, Hkv = 700, 2
    K = torch.randn(T, Hkv, d, generator=g)
    V = torch.randn(T, Hkv, d, generator=g)
    q = torch.randn(d, generator=g) * 2.0
    cfg = _cfg(sink=4, window=64)
    for t in (1, 5, 68, 69, 700):
        for mode in (orc.LOCAL, orc.FULL):
            pos = orc.access_set(cfg, orc.GATED, mode, t)
            for kvh in range(Hkv):
                out, lse = orc.attention(_words(q, dtype), _words(K, dtype), _words(V, dtype), kvh, pos, dtype)
                idx = torch.from_numpy(pos - 1)
                k64 = _as_f64(K, dtype)[idx, kvh]
                v64 = _as_f64(V, dtype)[idx, kvh]
                q64 = _as_f64(q, dtype)
                ref = torch.nn.functional.scaled_dot_product_attention(
                    q64.view(1, 1, 1, d), k64.view(1, 1, -1, d), v64.view(1, 1, -1, d))
                np.testing.assert_allclose(out, ref.view(d).numpy(), atol=1e-12, rtol=0)
                z = (k64 @ q64) / math.sqrt(d)
                assert abs(lse - torch.logsumexp(z, 0).item()) < 1e-12


# --------------------------------------------------------------------------- FP8 E4M3 KV

@pytest.mark.parametrize("case", _load("fp8_e4m3.json")["codes"], ids=lambda c: c["code"])
def test_fp8_e4m3_worked_codes(case):
    got = orc.fp8_e4m3(int(case["code"], 16))
    if case["value"] == "nan":
        assert math.isnan(got)
    else:
        assert got == case["value"] and math.copysign(1.0, got) == math.copysign(1.0, case["value"])


def test_fp8_e4m3_all_codes_match_torch_float8_e4m3fn():
    """Library cross-check over the whole code space: torch's float8_e4m3fn
    decoding of each byte, widened to float64."""
    want = torch.arange(256, dtype=torch.int16).to(torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = np.array([orc.fp8_e4m3(c) for c in range(256)])
    assert np.array_equal(np.isnan(got), np.isnan(want))
    ok = ~np.isnan(want)
    assert np.array_equal(got[ok], want[ok])
    assert np.array_equal(np.signbit(got[ok]), np.signbit(want[ok]))


@pytest.mark.parametrize("d", [64, 128])
def test_fp8_attention_matches_torch_sdpa_on_dequantised_values(d):
    """FP8 K/V with per-tensor scales: the oracle equals float64 SDPA over
    k_scale * decode(K) and v_scale * decode(V), with bf16 queries."""
    g = torch.Generator().manual_seed(99 + d)
    T, Hkv = 500, 2
    k_scale, v_scale = 0.0625, 3.0
    K8 = (torch.randn(T, Hkv, d, generator=g) * 4).to(torch.float8_e4m3fn)
    V8 = (torch.randn(T, Hkv, d, generator=g) * 0.5).to(torch.float8_e4m3fn)
    q = torch.randn(d, generator=g) * 2.0
    qw = q.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    kw, vw = K8.view(torch.uint8).numpy(), V8.view(torch.uint8).numpy()
    cfg = _cfg(sink=4, window=64)
    for t in (3, 68, 500):
        for mode in (orc.LOCAL, orc.FULL):
            pos = orc.access_set(cfg, orc.GATED, mode, t)
            idx = torch.from_numpy(pos - 1)
            for kvh in range(Hkv):
                out, lse = orc.attention(qw, kw, vw, kvh, pos, orc.FP8, k_scale=k_scale, v_scale=v_scale)
                k64 = K8.to(torch.float64)[idx, kvh] * k_scale
                v64 = V8.to(torch.float64)[idx, kvh] * v_scale
                q64 = q.to(torch.bfloat16).to(torch.float64)
                ref = torch.nn.functional.scaled_dot_product_attention(
                    q64.view(1, 1, 1, d), k64.view(1, 1, -1, d), v64.view(1, 1, -1, d))
                np.testing.assert_allclose(out, ref.view(d).numpy(), atol=1e-12, rtol=0)
                z = (k64 @ q64) / math.sqrt(d)
                assert abs(lse - torch.logsumexp(z, 0).item()) < 1e-12


def test_fp8_run_equals_bf16_run_on_exactly_representable_values():
    """Every E4M3 value is exact in bf16, so a decode run over FP8 codes with
    unit scales equals the same run over the bf16 words of the decoded values."""
    L, B, Hq, Hkv, d, P, K = 1, 2, 2, 1, 64, 90, 6
    T = P + K
    g = torch.Generator().manual_seed(7)
    k8 = torch.randn(L, B, T, Hkv, d, generator=g).to(torch.float8_e4m3fn)
    v8 = torch.randn(L, B, T, Hkv, d, generator=g).to(torch.float8_e4m3fn)
    q = torch.randn(K, L, B, Hq, d, generator=g).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    score = np.where(np.arange(K * B).reshape(K, B) % 3 == 0, 1.0, -1.0).astype(np.float32)
    prefill = np.full(B, P, np.int64)
    base = dict(num_layers=L, num_q_heads=Hq, num_kv_heads=Hkv, head_dim=d, sink=4, window=32)
    r8 = orc.decode_run(orc.OracleConfig(dtype=orc.FP8, **base), prefill, k8.view(torch.uint8).numpy(),
                        v8.view(torch.uint8).numpy(), q, score)
    kb = k8.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    vb = v8.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    rb = orc.decode_run(orc.OracleConfig(dtype=orc.BF16, **base), prefill, kb, vb, q, score)
    np.testing.assert_array_equal(r8["out"], rb["out"])
    np.testing.assert_array_equal(r8["lse"], rb["lse"])


def test_attention_special_cases():
    rng = np.random.default_rng(5)
    d, T = 64, 300
    K = rng.standard_normal((T, 1, d)).astype(np.float32)
    pos = np.arange(1, T + 1, dtype=np.int64)
    q = rng.standard_normal(d).astype(np.float32)
    # constant values: every convex combination is that constant
    V = np.full((T, 1, d), 0.75, dtype=np.float32)
    out, _ = orc.attention(q, K, V, 0, pos, orc.F32)
    np.testing.assert_allclose(out, 0.75, atol=1e-14)
    # zero query: uniform weights, the mean of V over the set
    V = rng.standard_normal((T, 1, d)).astype(np.float32)
    sub = pos[::7]
    out, lse = orc.attention(np.zeros(d, np.float32), K, V, 0, sub, orc.F32)
    np.testing.assert_allclose(out, V[sub - 1, 0].astype(np.float64).mean(0), atol=1e-13)
    assert abs(lse - math.log(sub.size)) < 1e-13
    # one dominant key: its value comes out
    K2 = K.copy()
    K2[41, 0] = q * 40.0
    out, _ = orc.attention(q, K2, V, 0, pos, orc.F32)
    np.testing.assert_allclose(out, V[41, 0], atol=1e-9)
    # softmax weights sum to one: attention over V = e_j basis recovers the weights
    n = 50
    Vb = np.zeros((n, 1, d), np.float32)
    for i in range(n):
        Vb[i, 0, i] = 1.0
    out, _ = orc.attention(q, K[:n], Vb, 0, np.arange(1, n + 1, dtype=np.int64), orc.F32)
    assert abs(out[:n].sum() - 1.0) < 1e-12 and np.all(out[:n] > 0)


# --------------------------------------------------------------------------- gate

def test_gate_strict_threshold():
    assert orc.gate(1e-45, 0.0)          # smallest positive fp32 (denormal) fires
    assert not orc.gate(0.0, 0.0)        # q_t = theta accepts Local (strict >)
    assert not orc.gate(-0.0, 0.0)
    assert not orc.gate(float("nan"), 0.0)
    assert not orc.gate(-1e-45, 0.0)
    assert orc.gate(float("inf"), 0.0)
    assert not orc.gate(0.5, 0.5) and orc.gate(0.5000001, 0.5)


# --------------------------------------------------------------------------- whole runs

def _run_inputs(L, B, Hq, Hkv, d, P, K, dtype, seed):
    g = torch.Generator().manual_seed(seed)
    T = max(P) + K
    kseq = torch.randn(L, B, T, Hkv, d, generator=g)
    vseq = torch.randn(L, B, T, Hkv, d, generator=g)
    q = torch.randn(K, L, B, Hq, d, generator=g)
    return kseq, vseq, q


def test_run_outputs_match_sdpa_per_decision():
    """A fired request's output is attention over {1..t}; otherwise over S^L_t
    (checked per step, layer and head against torch SDPA in float64)."""
    L, B, Hq, Hkv, d, K = 2, 3, 4, 2, 32, 6
    P = [3, 70, 140]
    s, w = 4, 64
    dtype = orc.BF16
    kseq, vseq, q = _run_inputs(L, B, Hq, Hkv, d, P, K, dtype, 7)
    score = np.random.default_rng(3).standard_normal((K, B)).astype(np.float32)
    score[0, :] = [1.0, -1.0, 0.0]
    cfg = orc.OracleConfig(L, Hq, Hkv, d, sink=s, window=w, dtype=dtype)
    res = orc.decode_run(cfg, P, _words(kseq, dtype), _words(vseq, dtype), _words(q, dtype), score)
    k64, v64, q64 = _as_f64(kseq, dtype), _as_f64(vseq, dtype), _as_f64(q, dtype)
    for k in range(K):
        fired = score[k] > 0
        assert res["fire"][k].tolist() == fired.astype(np.uint8).tolist()
        for l in range(L):
            for b in range(B):
                t = P[b] + k + 1
                if fired[b]:
                    pos = np.arange(1, t + 1)
                else:
                    pos = np.array([p for p in range(1, t + 1) if p <= s or p >= t - w + 1])
                idx = torch.from_numpy(pos - 1)
                for h in range(Hq):
                    gq = h // (Hq // Hkv)
                    ref = torch.nn.functional.scaled_dot_product_attention(
                        q64[k, l, b, h].view(1, 1, 1, d), k64[l, b, idx, gq].view(1, 1, -1, d),
                        v64[l, b, idx, gq].view(1, 1, -1, d)).view(d)
                    np.testing.assert_allclose(res["out"][k, l, b, h], ref.numpy(), atol=1e-12, rtol=0)


def test_run_local_equals_full_while_t_within_s_plus_w():
    L, B, Hq, Hkv, d, K = 1, 2, 2, 1, 64, 10
    P = [0, 55]                      # t runs 1..10 and 56..65, all <= s+w = 68
    kseq, vseq, q = _run_inputs(L, B, Hq, Hkv, d, P, K, orc.F32, 9)
    cfg = orc.OracleConfig(L, Hq, Hkv, d, sink=4, window=64, dtype=orc.F32)
    args = (cfg, P, _words(kseq, orc.F32), _words(vseq, orc.F32), _words(q, orc.F32))
    r_local = orc.decode_run(*args, -np.ones((K, B), np.float32))
    r_full = orc.decode_run(*args, np.ones((K, B), np.float32))
    assert np.array_equal(r_local["out"], r_full["out"])
    assert r_full["fire"].all() and not r_local["fire"].any()


def test_run_gqa_head_grouping():
    """Query head h reads KV head floor(h / (Hq/Hkv)): with constant values per
    KV head the outputs name the head each query head used."""
    L, B, Hq, Hkv, d, K, P = 1, 1, 8, 2, 16, 3, [20]
    kseq, _, q = _run_inputs(L, B, Hq, Hkv, d, P, K, orc.F32, 11)
    vseq = torch.zeros_like(kseq)
    vseq[:, :, :, 0] = 3.0
    vseq[:, :, :, 1] = 7.0
    cfg = orc.OracleConfig(L, Hq, Hkv, d, sink=2, window=4, dtype=orc.F32)
    res = orc.decode_run(cfg, P, _words(kseq, orc.F32), _words(vseq, orc.F32), _words(q, orc.F32),
                         np.zeros((K, B), np.float32))
    np.testing.assert_allclose(res["out"][:, 0, 0, :4], 3.0, atol=1e-14)
    np.testing.assert_allclose(res["out"][:, 0, 0, 4:], 7.0, atol=1e-14)


def test_run_gate_lists_and_counts():
    L, B, Hq, Hkv, d, K = 1, 9, 2, 1, 8, 40
    P = [10] * B
    kseq, vseq, q = _run_inputs(L, B, Hq, Hkv, d, P, K, orc.F32, 13)
    score = np.random.default_rng(4).standard_normal((K, B)).astype(np.float32)
    score[3, 2] = 0.0
    score[5, 4] = np.nan
    active = np.ones(B, np.uint8)
    active[7] = 0
    cfg = orc.OracleConfig(L, Hq, Hkv, d, sink=1, window=4, dtype=orc.F32)
    res = orc.decode_run(cfg, P, _words(kseq, orc.F32), _words(vseq, orc.F32), _words(q, orc.F32),
                         score, active=active)
    with np.errstate(invalid="ignore"):
        fired = (score > 0) & (active[None, :] == 1)
    assert np.array_equal(res["fire"].astype(bool), fired)
    assert res["call_count"].tolist() == fired.sum(1).tolist()
    for k in range(K):
        want = np.flatnonzero(fired[k]).tolist()
        assert res["call_list"][k].tolist() == want + [-1] * (B - len(want))
    assert res["full_calls"].tolist() == fired.sum(0).tolist()
    assert not res["fire"][3, 2] and not res["fire"][5, 4]
    assert np.all(res["out"][:, :, 7] == 0.0), "inactive request untouched"


# --------------------------------------------------------------------------- accounting

@pytest.mark.parametrize("case", _load("accounting.json")["cases"])
def test_accounting_worked_examples(case):
    c = dict(case["cfg"])
    c["dtype"] = orc.BF16 if c["dtype"] == "bf16" else orc.F32
    got = orc.step_accounting(orc.OracleConfig(**c), case["t"], case["fired"])
    assert got == case["expect"]


def test_accounting_closed_form_over_runs():
    """Summed over a run: at rho = 0 the savings are sum_t 4*Hq*d*L*(t - min(t, s+w))
    (minus F_Recall per step); at rho = 1 they are -sum_t F_Local(t) - F_Recall."""
    L, Hq, Hkv, d, s, w, rec = 3, 4, 2, 8, 2, 5, 11
    cfg = orc.OracleConfig(L, Hq, Hkv, d, sink=s, window=w, dtype=orc.BF16, recall_flops=rec)
    P, K = 4, 12
    kseq, vseq, q = _run_inputs(L, 1, Hq, Hkv, d, [P], K, orc.BF16, 17)
    args = (cfg, [P], _words(kseq, orc.BF16), _words(vseq, orc.BF16), _words(q, orc.BF16))
    ts = [P + k for k in range(1, K + 1)]
    per = 4 * Hq * d * L
    r0 = orc.decode_run(*args, -np.ones((K, 1), np.float32))
    r1 = orc.decode_run(*args, np.ones((K, 1), np.float32))
    a0 = dict(zip(orc.ACCT_FIELDS, r0["acct"][0].tolist()))
    a1 = dict(zip(orc.ACCT_FIELDS, r1["acct"][0].tolist()))
    assert a0["delta_f"] == sum(per * (t - min(t, s + w)) - rec for t in ts)
    assert a1["delta_f"] == sum(-per * min(t, s + w) - rec for t in ts)
    assert a1["kv_bytes"] == sum(Hkv * d * 2 * 2 * L * (min(t, s + w) + t) for t in ts)
    assert a0["steps"] == a1["steps"] == K and a1["full_calls"] == K and a0["full_calls"] == 0


def test_local_to_full_flop_ratio_at_long_context():
    """F_Local/F_Full = (s+w)/n for a gated stack once n > s+w: 2052/131073 at a
    131072-token prefill (about 1.57%, the Local attempt's share of a Full step)."""
    cfg = orc.OracleConfig(28, 16, 8, 128, sink=4, window=2048, dtype=orc.BF16)
    a = orc.step_accounting(cfg, 131073, False)
    assert a["f_local"] * 131073 == a["f_full_always"] * 2052


# --------------------------------------------------------------------------- recall head stand-in

def _bf16_words(a) -> np.ndarray:
    return torch.tensor(a, dtype=torch.float32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def test_recall_head_worked_example():
    g = _load("recall_head_worked.json")
    q = orc.recall_head(_bf16_words(g["W1"]), np.array(g["b1"], np.float32), np.array(g["w2"], np.float32),
                        g["b2"], _bf16_words(g["x"]))
    assert q.tolist() == g["expect_q"]


def test_recall_head_matches_torch_float64():
    """Library cross-check: relu(x W1^T + b1) w2 + b2 with torch in float64 on
    the same bf16-rounded weights and inputs."""
    gen = torch.Generator().manual_seed(31)
    H, I, Bn = 48, 96, 5
    W1 = (torch.randn(H, I, generator=gen) * 0.2).to(torch.bfloat16)
    x = torch.randn(Bn, I, generator=gen).to(torch.bfloat16)
    b1 = torch.randn(H, generator=gen) * 0.1
    w2 = torch.randn(H, generator=gen)
    b2 = 0.3125  # exact in f32, the type the head's output bias is stored in
    q = orc.recall_head(W1.view(torch.int16).numpy().view(np.uint16), b1.numpy(), w2.numpy(), b2,
                        x.view(torch.int16).numpy().view(np.uint16))
    ref = torch.relu(x.double() @ W1.double().T + b1.double()) @ w2.double() + b2
    np.testing.assert_allclose(q, ref.numpy(), atol=1e-12, rtol=0)
    assert (ref.numpy() > 0).any() and (ref.numpy() < 0).any()


def test_recall_head_hidden_units_commute():
    """Permuting the hidden units (rows of W1 with b1 and w2) leaves q unchanged."""
    rng = np.random.default_rng(8)
    H, I = 17, 40
    W1 = _bf16_words(rng.standard_normal((H, I)) * 0.3)
    b1 = rng.standard_normal(H).astype(np.float32)
    w2 = rng.standard_normal(H).astype(np.float32)
    x = _bf16_words(rng.standard_normal((3, I)))
    perm = rng.permutation(H)
    q0 = orc.recall_head(W1, b1, w2, -0.1, x)
    q1 = orc.recall_head(W1[perm], b1[perm], w2[perm], -0.1, x)
    np.testing.assert_allclose(q0, q1, atol=1e-12, rtol=0)
