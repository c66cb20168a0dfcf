"""Parity at the workloads' full sizes, in the launch configuration the
benchmark uses (default splits, captured-graph step replay), on sampled
outputs the oracle computes one by one.

For each sampled (step, layer, request) every query head's accepted output
is recomputed by the oracle over the access set the gate selected; the
Full-call totals and accounting counters of every request are compared bit
for bit with the oracle's per-step accounting over all steps run.
"""
import concurrent.futures as cf
import os

import numpy as np
import pytest
import torch

import oracle as orc
from gated_kv_access_amd import workloads as W
from gated_kv_access_amd.runner import StepRunner
from gated_kv_access_amd.state import DecodeState
from tests.gpu_helpers import TOL, oracle_cfg, say, words

pytestmark = pytest.mark.gpu

_POOL = min(16, os.cpu_count() or 4)


def _run_and_sample(wl, steps, sample_steps, sample_layers, sample_requests, host_cache=False):
    wl = wl.with_(steps=steps)
    say(f"{wl.name}: batch {wl.batch}, {wl.num_layers} layers, max prefill {max(wl.prefill)}, {steps} steps")
    st = DecodeState(wl, gen_device="cuda", host_cache=host_cache)
    st.prefill()
    q = W.gen_queries(wl, "cuda")
    k_new, v_new = st.decode_inputs()
    scores = W.gen_scores(wl)
    r = StepRunner(st, q, k_new, v_new, torch.from_numpy(scores).cuda(), want_lse=True)
    r.capture()
    rec = {}
    for k in range(steps):
        r.replay(1)
        if k in sample_steps:
            torch.cuda.synchronize()
            rec[k] = (r.out[list(sample_layers)][:, list(sample_requests)].cpu().numpy(),
                      int(r.call_count[0].item()), r.call_list.cpu().numpy().copy())
    torch.cuda.synchronize()
    assert st.device_error() == 0
    return wl, st, q, scores, r, rec


def _check(wl, st, q, scores, r, rec, sample_layers, sample_requests, each_request_both=True):
    """each_request_both: every sampled request must have at least one fired and
    one unfired sampled step (else: the samples as a whole must), so that both
    the Full pass over the paged cache and the accepted Local pass are compared
    with the oracle whatever the seeds."""
    cfg = oracle_cfg(wl)
    focus = st.focus_range.cpu().numpy()
    steps = wl.steps
    # integer results over every step: gate decisions, totals, counters
    fired = scores > 0
    ks_sampled = sorted(rec)
    per_req = [(int(fired[ks_sampled, b].sum()), int((~fired[ks_sampled, b]).sum())) for b in sample_requests]
    if each_request_both:
        for b, (nf, nu) in zip(sample_requests, per_req):
            assert nf >= 1 and nu >= 1, (wl.name, "request", b, "sampled steps", ks_sampled, "fired", nf, "unfired", nu)
    else:
        assert sum(n for n, _ in per_req) >= 1 and sum(n for _, n in per_req) >= 1, (wl.name, ks_sampled, per_req)
    for k, (_, count, clist) in rec.items():
        want = np.flatnonzero(fired[k])
        assert count == want.size
        assert clist[:count].tolist() == want.tolist()
    assert r.full_calls.cpu().numpy().tolist() == fired.sum(0).tolist()
    got_c = r.counters.cpu().numpy()
    for b in range(wl.batch):
        acc = {f: 0 for f in orc.ACCT_FIELDS}
        for k in range(steps):
            a = orc.step_accounting(cfg, wl.prefill[b] + k + 1, bool(fired[k, b]), int(focus[b, 0]), int(focus[b, 1]))
            for f in acc:
                acc[f] += a[f]
        assert got_c[b].tolist() == [acc[f] for f in orc.ACCT_FIELDS], b
    # sampled outputs
    qh = words(q)
    G = wl.num_q_heads // wl.num_kv_heads
    atol, rtol = TOL[wl.dtype]
    worst = 0.0
    n_fired = n_unfired = 0
    for li, l in enumerate(sample_layers):
        kind = wl.kinds[l]
        for bi, b in enumerate(sample_requests):
            ks = words(W.gen_sequence(wl, l, b, "k", "cuda"))
            vs = words(W.gen_sequence(wl, l, b, "v", "cuda"))
            jobs = {}
            with cf.ThreadPoolExecutor(_POOL) as ex:
                for k in rec:
                    t = wl.prefill[b] + k + 1
                    mode = orc.FULL if fired[k, b] else orc.LOCAL
                    pos = orc.access_set(cfg, kind, mode, t, int(focus[b, 0]), int(focus[b, 1]))
                    for h in range(wl.num_q_heads):
                        jobs[(k, h)] = ex.submit(orc.attention, qh[k, l, b, h], ks, vs, h // G, pos, cfg.dtype,
                                                 0.0, cfg.k_scale, cfg.v_scale)
                for k in rec:
                    want = np.stack([jobs[(k, h)].result()[0] for h in range(wl.num_q_heads)])
                    got = rec[k][0][li, bi].astype(np.float64)
                    diff = got - want
                    mabs = float(np.abs(diff).max())
                    rel = float(np.linalg.norm(diff) / np.linalg.norm(want))
                    worst = max(worst, mabs)
                    assert mabs <= atol and rel <= rtol, (wl.name, k, l, b, bool(fired[k, b]), mabs, rel)
                    if fired[k, b]:
                        n_fired += 1
                    else:
                        n_unfired += 1
    say(f"{wl.name}: sampled outputs within bars, worst max-abs {worst:.3e}; "
        f"{n_fired} fired (Full-pass) and {n_unfired} unfired (Local-pass) (step, layer, request) samples")


def test_ctx16k_rho041_every_step_run_sampled_outputs():
    wl = W.config(1)
    steps = wl.steps
    samp = {0, 1, 2, 57, 128, steps - 1}  # steps 1 and 2 fire
    out = _run_and_sample(wl, steps, samp, (0, 13, 27), (0,))
    _check(*out, (0, 13, 27), (0,))


def test_ctx128k_rho0125_sampled():
    wl = W.config(2)
    steps = 48
    # with these seeds steps 2, 8, 13, 36, 44 and 46 fire
    out = _run_and_sample(wl, steps, {0, 2, 8, 23, 46, steps - 1}, (0, 27), (0,))
    _check(*out, (0, 27), (0,))


def test_batched32_mixed_lengths_sampled():
    wl = W.config(3)
    steps = 12
    lens = np.array(wl.prefill)
    rho = np.array(wl.rho)
    picks = sorted({int(lens.argmin()), int(lens.argmax()), int(np.flatnonzero(rho == 1.0)[0]),
                    int(np.flatnonzero(rho == 0.0)[0])})
    free = torch.cuda.mem_get_info()[0]
    need = float((lens + steps).sum()) * 28 * 8 * 128 * 2 * 2
    if need > 0.92 * free:
        pytest.skip(f"paged cache of {need / 1e9:.0f} GB does not fit the {free / 1e9:.0f} GB free")
    out = _run_and_sample(wl, steps, {0, 1, steps - 1}, (0, 27), tuple(picks))
    # the picks include a request that never fires and one that always does
    _check(*out, (0, 27), tuple(picks), each_request_both=False)


@pytest.mark.parametrize("focus", [True, False], ids=["fire_focus", "fire_full"])
def test_hybrid_sliding_and_focus_sampled(focus):
    wl = W.config(4).with_(focus=focus)
    steps = 10
    out = _run_and_sample(wl, steps, {0, 3, steps - 1}, (2, 3, 31), (0, 5))  # request 0 fires at 3, 9; 5 at 3
    _check(*out, (2, 3, 31), (0, 5))


def test_ctx128k_rho0125_fp8_kv_sampled():
    """The 128K workload with an E4M3 KV cache (per-tensor scales 1/16)."""
    wl = W.config(2).fp8()
    steps = 48
    out = _run_and_sample(wl, steps, {0, 2, 7, 13, steps - 1}, (0, 27), (0,))  # 2 and 13 fire
    _check(*out, (0, 27), (0,))


@pytest.mark.parametrize("group,kv", [(4, "bf16"), (4, "fp8"), (8, "bf16"), (8, "fp8")])
def test_ctx128k_gqa_groups_sampled(group, kv):
    """The 128K workload with 32 or 64 query heads over the 8 KV heads (GQA
    groups of 4 and 8, bf16 and FP8: paged and ring passes on MFMA, the tail
    pool for bf16)."""
    wl = W.config(2).with_(num_q_heads=8 * group, rho=(0.5,))
    if kv == "fp8":
        wl = wl.fp8()
    steps = 6
    out = _run_and_sample(wl, steps, {0, 3, steps - 1}, (0, 27), (0,))
    _check(*out, (0, 27), (0,))


def test_hybrid_focus_fp8_kv_sampled():
    wl = W.config(4).fp8()
    steps = 8
    out = _run_and_sample(wl, steps, {0, 1, 4, steps - 1}, (3, 31), (0, 7))  # request 0 fires at 1, 7 at 4
    _check(*out, (3, 31), (0, 7))


def test_ctx128k_host_resident_history_sampled():
    """The 128K workload with the paged history in pinned host memory: 4 steps,
    two of them firing (Full passes read 15 GB over the host link)."""
    wl = W.config(2).with_(score_mode="exact", rho=(0.5,))
    steps = 4
    out = _run_and_sample(wl, steps, {0, 1, 2, 3}, (0, 27), (0,), host_cache=True)
    _check(*out, (0, 27), (0,))
