"""GPU parity of the HIP path (through the C ABI) against the CPU fp64 oracle.

Integer results -- gate decisions, compacted call lists, counts, Full-call
totals, accounting counters, access sets, ring slot contents -- must match
bit for bit; attention outputs within the bars of tests/gpu_helpers.TOL.
Inputs are seeded synthetic draws; sizes span several tiles, ragged tails,
ring wrap-around, the t <= s+w regime and empty prefixes.
"""
import numpy as np
import pytest
import torch

import oracle as orc
from gated_kv_access_amd import binding as B
from gated_kv_access_amd import workloads as W
from gated_kv_access_amd.state import DecodeState, make_dims
from tests.gpu_helpers import (assert_outputs_close, oracle_cfg, oracle_sequences, run_steps, say,
                               words, LSE_TOL)

pytestmark = pytest.mark.gpu


def _small(name, **kw):
    base = dict(num_layers=2, num_q_heads=4, num_kv_heads=2, head_dim=128, dtype="bf16", batch=3,
                prefill=(0, 700, 3001), steps=10, sink=4, window=256, score_mode="normal", seed=101)
    base.update(kw)
    return W.Workload(name, **base)


SMALL = [
    _small("bf16_d128_g2"),
    _small("bf16_d64_g1", head_dim=64, num_q_heads=2, num_kv_heads=2, seed=102),
    _small("bf16_d128_g4", num_q_heads=8, num_kv_heads=2, seed=103),
    _small("f32_d128_g2", dtype="f32", seed=104),
    _small("f32_d64_g4_bs8", dtype="f32", head_dim=64, num_q_heads=4, num_kv_heads=1, block_size=8, seed=105),
    _small("bf16_ring_wrap_bs64", sink=2, window=16, prefill=(100, 37, 5), steps=40, block_size=64, seed=106),
    _small("bf16_no_sinks", sink=0, window=33, prefill=(64, 1, 200), steps=12, seed=107),
]


def _check_run(wl, graph=False, q_full=False, host_cache=False, dims=None):
    say(f"{wl.name}: prefill {wl.prefill}, {wl.steps} steps, graph={graph}, host_cache={host_cache}")
    st = DecodeState(wl, gen_device="cpu", host_cache=host_cache, dims=dims)
    st.prefill()
    q = W.gen_queries(wl, "cpu")
    qf = W.gen_queries(wl, "cpu", tag=4) if q_full else None
    scores = W.gen_scores(wl)
    got = run_steps(st, q, scores, graph=graph, q_full=qf)
    assert st.device_error() == 0
    ks, vs = oracle_sequences(st)
    want = orc.decode_run(oracle_cfg(wl), wl.prefill, ks, vs, words(q), scores,
                          q_full=None if qf is None else words(qf),
                          focus=st.focus_range.cpu().numpy() if wl.focus else None)
    # integer results: bit-exact
    assert np.array_equal(got.call_count, want["call_count"])
    assert np.array_equal(got.call_list, want["call_list"])
    assert np.array_equal(got.full_calls, want["full_calls"])
    assert np.array_equal(got.counters, want["acct"])
    assert_outputs_close(got.out, want["out"], wl.dtype, wl.name)
    lse_err = float(np.abs(got.lse - want["lse"]).max())
    assert lse_err <= LSE_TOL[wl.dtype], lse_err
    return st, got, want


@pytest.mark.parametrize("wl", SMALL, ids=[w.name for w in SMALL])
def test_small_runs_match_oracle(wl):
    _check_run(wl)


def test_tiny_config_every_step():
    """The 1-layer fp32 workload (300-token prefill, 50 steps, s=4, w=64) step by step."""
    _check_run(W.config(0))


def test_graph_replay_matches_oracle_and_eager():
    wl = _small("graph_bf16", prefill=(50, 900, 2100), steps=16, seed=111)
    _, g_run, _ = _check_run(wl, graph=True)
    _, e_run, _ = _check_run(wl, graph=False)
    assert np.array_equal(g_run.out, e_run.out), "graph replay differs from eager launches"
    assert np.array_equal(g_run.counters, e_run.counters)


def test_separate_full_pass_queries():
    _check_run(_small("q_full_bf16", prefill=(10, 400, 1500), steps=8, seed=112), q_full=True)


def test_local_equals_full_while_t_within_s_plus_w():
    """t <= s+w: S^L_t = S^F_t, so the ring pass and the paged pass agree."""
    wl = _small("short_ctx", prefill=(0, 20, 200), steps=8, window=256, seed=113)
    st = DecodeState(wl, gen_device="cpu")
    st.prefill()
    q = W.gen_queries(wl, "cpu")
    never = np.full((wl.steps, wl.batch), -1.0, np.float32)
    always = np.full((wl.steps, wl.batch), 1.0, np.float32)
    r_local = run_steps(st, q, never)
    st2 = DecodeState(wl, gen_device="cpu")
    st2.prefill()
    r_full = run_steps(st2, q, always)
    diff = np.abs(r_local.out - r_full.out).max()
    say(f"ring vs paged max diff {diff:.3e}")
    assert diff <= 1e-5
    assert r_full.full_calls.tolist() == [wl.steps] * wl.batch


EDGE = [
    _small("block_size_1", block_size=1, prefill=(0, 40, 301), steps=6, seed=161),
    _small("block_size_2_fp8", block_size=2, prefill=(3, 90, 513), steps=6, seed=162).fp8(),
    _small("window_1", sink=4, window=1, prefill=(0, 3, 700), steps=8, seed=163),
    _small("sinks_over_window", sink=40, window=8, prefill=(0, 30, 60), steps=20, seed=164),
    _small("ring_exactly_one_tile", sink=4, window=124, prefill=(120, 127, 128), steps=6, seed=165),
    _small("one_request_f32_d64", dtype="f32", head_dim=64, num_q_heads=1, num_kv_heads=1, batch=1,
           prefill=(2049,), steps=4, seed=166),
    # GQA groups of 4 stream paged rows with half the vectors per lane (the
    # other two head sizes / types of that geometry are in SMALL and FP8)
    _small("bf16_d64_g4", head_dim=64, num_q_heads=8, num_kv_heads=2, seed=167),
    _small("f32_d128_g4", dtype="f32", num_q_heads=4, num_kv_heads=1, seed=168),
    # GQA groups of 8: the paged passes on MFMA for bf16 (one chunk per lane
    # and row, tiles half as tall, for f32 and in the ring passes); the merge
    # serves two outputs per thread at d = 128
    _small("bf16_d128_g8", num_q_heads=16, num_kv_heads=2, seed=169),
    _small("bf16_d64_g8", head_dim=64, num_q_heads=8, num_kv_heads=1, seed=170),
    _small("f32_d64_g8", dtype="f32", head_dim=64, num_q_heads=8, num_kv_heads=1, seed=171),
    # MFMA ring passes over a ring that wraps many times (slots of older
    # positions inside a pass), and a short request that never fills it
    _small("ring_wrap_g8", num_q_heads=16, num_kv_heads=2, sink=2, window=16, prefill=(100, 37, 5),
           steps=40, block_size=64, seed=172),
]


@pytest.mark.parametrize("wl", EDGE, ids=[w.name for w in EDGE])
def test_edge_shapes_match_oracle(wl):
    """Every row its own block, a one-slot window, more sinks than window
    slots, a ring of exactly one tile (plus the current token), GQA group 1."""
    _check_run(wl)


HYBRID = [
    _small("hybrid_full", num_layers=8, sw_window=64, sink=4, window=128, batch=2, prefill=(1000, 2500),
           steps=10, layer_kind=tuple(0 if i % 4 == 3 else 1 for i in range(8)), seed=121),
    _small("hybrid_focus", num_layers=8, sw_window=64, sink=4, window=128, batch=3,
           prefill=(1000, 2500, 6000), steps=10, layer_kind=tuple(0 if i % 4 == 3 else 1 for i in range(8)),
           focus=True, seed=122),
    _small("focus_only_gated", num_layers=2, batch=3, prefill=(5000, 300, 4300), steps=6, focus=True, seed=123),
]


@pytest.mark.parametrize("wl", HYBRID, ids=[w.name for w in HYBRID])
def test_hybrid_and_focus_runs_match_oracle(wl):
    _check_run(wl)


def test_focus_region_overlapping_window_and_sinks():
    wl = _small("focus_overlap", num_layers=1, batch=3, prefill=(4500, 4500, 4500), steps=4, focus=True,
                sink=4, window=256, seed=124)
    st = DecodeState(wl, gen_device="cpu")
    # regions: overlapping the window, covering the sinks, straddling nothing
    st.focus_range.copy_(torch.tensor([[4300, 4400 + 4096], [1, 4097], [2000, 2000 + 4096]], dtype=torch.int64))
    st.prefill()
    q = W.gen_queries(wl, "cpu")
    scores = np.ones((wl.steps, wl.batch), np.float32)
    got = run_steps(st, q, scores)
    ks, vs = oracle_sequences(st)
    want = orc.decode_run(oracle_cfg(wl), wl.prefill, ks, vs, words(q), scores,
                          focus=st.focus_range.cpu().numpy())
    assert np.array_equal(got.counters, want["acct"])
    assert_outputs_close(got.out, want["out"], wl.dtype, wl.name)


# ---------------------------------------------------------------- integer exports

def _ring_slot(p, s, w):
    return p - 1 if p <= s else s + (p - s - 1) % w


@pytest.mark.parametrize("wl", [SMALL[5], SMALL[6], HYBRID[1]], ids=["wrap", "nosink", "hybrid"])
def test_access_sets_and_ring_slots_bit_exact(wl):
    st = DecodeState(wl, gen_device="cpu")
    st.prefill()
    q = W.gen_queries(wl, "cpu")
    scores = W.gen_scores(wl)
    k_new, v_new = st.decode_inputs()
    cfg = oracle_cfg(wl)
    pos = torch.zeros(wl.max_rows + 8, dtype=torch.int32, device="cuda")
    cnt = torch.zeros(2, dtype=torch.int64, device="cuda")
    from gated_kv_access_amd.runner import StepRunner
    r = StepRunner(st, q.cuda(), k_new, v_new, torch.from_numpy(scores).cuda())
    for k in range(wl.steps + 1):
        for b in range(wl.batch):
            t = wl.prefill[b] + k + 1
            fa, fb = (int(x) for x in st.focus_range[b].tolist())
            for layer in range(wl.num_layers):
                kind = wl.kinds[layer]
                for mode in (0, 1):
                    B.access_set(st.dims, st.kv, layer, b, mode, pos, cnt, st.workspace)
                    torch.cuda.synchronize()
                    n = int(cnt[0].item())
                    got = np.sort(pos[:n].cpu().numpy().astype(np.int64))
                    want = orc.access_set(cfg, kind, mode, t, fa, fb)
                    assert np.array_equal(got, want), (wl.name, k, b, layer, mode, t)
            # ring slot contents: what one-by-one commits of 1..t-1 leave
            if wl.gated_layers:
                s, w = wl.sink, wl.window
                ring = np.zeros(s + w, np.int64)
                for p in range(1, t):
                    ring[_ring_slot(p, s, w)] = p
                assert np.array_equal(st.ring_pos[b].cpu().numpy(), ring), (k, b)
            if wl.sliding_layers:
                ring = np.zeros(wl.sw_window, np.int64)
                for p in range(1, t):
                    ring[(p - 1) % wl.sw_window] = p
                assert np.array_equal(st.swring_pos[b].cpu().numpy(), ring), (k, b)
        if k < wl.steps:
            r.step_eager()
    assert st.device_error() == 0


def test_commit_writes_paged_cache_and_ring_bit_exact():
    wl = _small("commit", prefill=(3, 31, 70), steps=20, sink=2, window=8, block_size=16, seed=131)
    st = DecodeState(wl, gen_device="cpu")
    st.prefill()
    q = W.gen_queries(wl, "cpu")
    run_steps(st, q, W.gen_scores(wl))
    bt = st.block_table.cpu().numpy()
    for layer in range(wl.num_layers):
        for b in range(wl.batch):
            k_all = st.sequence(layer, b, "k")
            v_all = st.sequence(layer, b, "v")
            t_end = wl.prefill[b] + wl.steps
            for p in range(1, t_end + 1):
                blk = bt[b, (p - 1) // wl.block_size]
                row = (p - 1) % wl.block_size
                assert torch.equal(st.k_cache[layer, :, blk, row], k_all[p - 1])
                assert torch.equal(st.v_cache[layer, :, blk, row], v_all[p - 1])
            for j in range(wl.sink + wl.window):
                p = int(st.ring_pos[b, j].item())
                if p:
                    assert torch.equal(st.k_ring[layer, b, :, j], k_all[p - 1])
                    assert torch.equal(st.v_ring[layer, b, :, j], v_all[p - 1])
    assert st.seq_len.cpu().tolist() == [p + wl.steps for p in wl.prefill]


def test_gate_and_accounting_bit_exact():
    wl = _small("gate", batch=1100, prefill=tuple([100] * 1100), num_layers=3, steps=1, seed=141)
    dims = __import__("gated_kv_access_amd.state", fromlist=["make_dims"]).make_dims(wl, recall_flops=1234)
    seq = torch.tensor(list(range(0, 2200, 2)), dtype=torch.int32, device="cuda")
    seq[7] = -1   # inactive slot
    kv = B.OdaKV()
    kv.seq_len = seq.data_ptr()
    rng = np.random.default_rng(5)
    score = rng.standard_normal(1100).astype(np.float32)
    score[[3, 64, 65, 1023, 1024]] = [0.0, -0.0, np.nan, np.inf, 1e-45]
    sc = torch.from_numpy(score).cuda()
    call_list = torch.full((1100,), 77, dtype=torch.int32, device="cuda")
    call_count = torch.zeros(4, dtype=torch.int32, device="cuda")
    full_calls = torch.zeros(1100, dtype=torch.int64, device="cuda")
    counters = torch.zeros((1100, 8), dtype=torch.int64, device="cuda")
    B.gate(dims, kv, 1100, sc, 0.0, call_list, call_count, full_calls, counters)
    torch.cuda.synchronize()
    seq_h = seq.cpu().numpy()
    fired = np.array([seq_h[b] >= 0 and orc.gate(float(score[b]), 0.0) for b in range(1100)])
    want_list = np.flatnonzero(fired)
    got_count = int(call_count[0].item())
    assert got_count == want_list.size
    assert np.array_equal(call_list[:got_count].cpu().numpy(), want_list)
    assert np.all(call_list[got_count:].cpu().numpy() == -1)
    assert np.array_equal(full_calls.cpu().numpy(), fired.astype(np.int64))
    cfg = oracle_cfg(wl, recall_flops=1234)
    got_c = counters.cpu().numpy()
    for b in range(1100):
        if seq_h[b] < 0:
            assert np.all(got_c[b] == 0)
            continue
        want = orc.step_accounting(cfg, int(seq_h[b]) + 1, bool(fired[b]))
        assert got_c[b].tolist() == [want[f] for f in orc.ACCT_FIELDS], b


# ---------------------------------------------------------------- standalone per-layer calls

EMPTY_SLOT = 0x7FA5A5A5  # what an unused split-partial word of the workspace holds


def _empty_words(st) -> int:
    torch.cuda.synchronize()
    return int((st.workspace.cpu().numpy().view(np.uint32) == EMPTY_SLOT).sum())


@pytest.mark.parametrize("full_splits,local_splits", [(50, 17), (24, 48), (50, 48)],
                         ids=["full_ticket", "local_ticket", "both_ticket"])
def test_ticket_and_polling_merges_share_one_workspace(full_splits, local_splits):
    """A launch whose workgroups all fit on the chip at once (at most 256)
    merges by re-reading the partial slots until none is empty; a larger one by
    the last ticket.  With batch 3 and 2 KV heads, 50 or 48 splits make the
    Full or the Local passes take tickets while the other kind polls, on the
    same partial slots.  Outputs match the oracle, and after every step each
    partial word of the workspace reads empty again (as after initialisation)."""
    wl = _small("merge_modes", window=1024, steps=6, seed=171)
    dims = make_dims(wl, full_splits=full_splits, local_splits=local_splits)
    ms = max(full_splits, local_splits)
    slots = wl.batch * wl.num_q_heads * ms * (wl.head_dim + 2 * (wl.head_dim // 64))
    st = DecodeState(wl, gen_device="cpu", dims=dims)
    at_init = _empty_words(st)
    assert slots <= at_init < slots + 128  # plus the padding that aligns the partial arrays
    st, got, want = _check_run(wl, dims=dims)
    assert _empty_words(st) == at_init


def test_polling_merge_over_several_rounds_of_partials():
    """The merging split reads the partial slots in rounds of 32; with one
    request and 2 KV heads, 64 ring splits (63 partials besides its own: two
    rounds) and 100 Full splits (four rounds) still fit the chip at once, so
    both merge by polling.  Outputs match the oracle and the slots read empty
    again afterwards."""
    wl = _small("poll_rounds", batch=1, prefill=(5000,), window=1024, steps=4, seed=173)
    dims = make_dims(wl, full_splits=100, local_splits=64)
    slots = wl.batch * wl.num_q_heads * 100 * (wl.head_dim + 2 * (wl.head_dim // 64))
    st = DecodeState(wl, gen_device="cpu", dims=dims)
    at_init = _empty_words(st)
    assert slots <= at_init < slots + 128
    st, got, want = _check_run(wl, dims=dims)
    assert _empty_words(st) == at_init


@pytest.mark.parametrize("group", [2, 4, 8])
def test_full_pass_tail_pool_matches_oracle(group):
    """With 2 Full splits per (request, KV head) the Full passes of contexts of
    4096 rows and more keep a pool of 4 tail tiles that the splits take one at
    a time (at the 128K workload the pool is 64 tiles of 32 splits).  Request 0
    stays below the threshold (static splits only), 1 and 2 use the pool, the
    last one with a ragged final pool tile.  Results match the oracle at every
    step; every launch reuses the claim counters, so a counter its merge did
    not reset would drop pool tiles from the next launch's result.  Groups 4
    and 8 run the paged geometries with fewer vectors per lane (and, at 8, a
    tile half as tall)."""
    wl = _small(f"tail_pool_g{group}", num_q_heads=2 * group, prefill=(3000, 4500, 6151), steps=5, seed=172)
    dims = make_dims(wl, full_splits=2)
    st, got, want = _check_run(wl, dims=dims)
    assert int(got.call_count.sum()) > 0, "some steps must fire"


def test_standalone_local_and_gated_full_calls():
    wl = _small("standalone", prefill=(0, 1200, 2600), steps=1, seed=151)
    st = DecodeState(wl, gen_device="cpu")
    st.prefill()
    q = W.gen_queries(wl, "cpu")[0].cuda()          # [L][B][Hq][d]
    k_new, v_new = st.decode_inputs()
    score = torch.tensor([0.5, -0.25, 2.0], dtype=torch.float32, device="cuda")
    ks, vs = oracle_sequences(st)
    want = orc.decode_run(oracle_cfg(wl), wl.prefill, ks, vs, words(q.unsqueeze(0)),
                          score.cpu().numpy()[None, :])
    for layer in range(wl.num_layers):
        out = torch.full((wl.batch, wl.num_q_heads, wl.head_dim), 5.0, device="cuda")
        lse = torch.zeros((wl.batch, wl.num_q_heads), device="cuda")
        B.decode_local(st.dims, st.kv, layer, wl.batch, q[layer].contiguous(), k_new[0, layer].contiguous(),
                       v_new[0, layer].contiguous(), out, lse, st.workspace)
        local = out.clone()
        call_list = torch.zeros(wl.batch, dtype=torch.int32, device="cuda")
        call_count = torch.zeros(4, dtype=torch.int32, device="cuda")
        B.decode_full_gated(st.dims, st.kv, layer, wl.batch, q[layer].contiguous(), k_new[0, layer].contiguous(),
                            v_new[0, layer].contiguous(), score, 0.0, out, lse, call_list, call_count,
                            st.workspace)
        torch.cuda.synchronize()
        assert call_list.cpu().tolist() == [0, 2, -1] and int(call_count[0]) == 2
        assert torch.equal(out[1], local[1]), "a request that did not fire keeps its Local row"
        assert_outputs_close(out.cpu().numpy()[None, None], want["out"][:, layer:layer + 1], wl.dtype,
                             f"standalone layer {layer}")


def test_device_errors_skip_and_flag_without_touching_other_requests():
    """Inputs that only the device can see are caught by the kernels' own
    checks: a block id outside the cache skips the rows it would address, a
    context longer than the block table skips the request; each sets its bit in
    the workspace's error word, and the other requests' outputs still match the
    oracle."""
    wl = _small("deverr", prefill=(300, 1200, 2600), steps=1, seed=181)
    st = DecodeState(wl, gen_device="cpu")
    st.prefill()
    q = W.gen_queries(wl, "cpu")[0].cuda()
    k_new, v_new = st.decode_inputs()
    score = torch.ones(wl.batch, dtype=torch.float32, device="cuda")  # every request fires
    ks, vs = oracle_sequences(st)
    want = orc.decode_run(oracle_cfg(wl), wl.prefill, ks, vs, words(q.unsqueeze(0)),
                          score.cpu().numpy()[None, :])["out"][0, 0]
    args = (q[0].contiguous(), k_new[0, 0].contiguous(), v_new[0, 0].contiguous())

    def full_pass():
        out = torch.full((wl.batch, wl.num_q_heads, wl.head_dim), 7.0, device="cuda")
        B.decode_full_gated(st.dims, st.kv, 0, wl.batch, *args, score, 0.0, out, None, None, None, st.workspace)
        torch.cuda.synchronize()
        err = st.device_error()
        st.workspace[:4].zero_()
        return out.cpu().numpy(), err

    out, err = full_pass()
    assert err == 0
    assert_outputs_close(out[None, None], want[None, None], wl.dtype, "clean")
    # a physical block id past the cache in request 1's table row
    saved = int(st.block_table[1, 10].item())
    st.block_table[1, 10] = st.num_blocks + 7
    out, err = full_pass()
    st.block_table[1, 10] = saved
    say(f"bad block id: error word {err}")
    assert err == B.DEVERR_BLOCK_ID
    assert np.isfinite(out[1]).all()
    for b in (0, 2):
        assert_outputs_close(out[None, None, b:b + 1], want[None, None, b:b + 1], wl.dtype, f"bad block, request {b}")
    # a committed length past the block table's capacity for request 2
    cap = st.dims.max_blocks_per_seq * wl.block_size
    st.seq_len[2] = cap + 5
    out, err = full_pass()
    st.seq_len[2] = wl.prefill[2]
    say(f"context beyond capacity: error word {err}")
    assert err == B.DEVERR_CAPACITY
    assert (out[2] == 7.0).all(), "the request is skipped: its output rows stay untouched"
    for b in (0, 1):
        assert_outputs_close(out[None, None, b:b + 1], want[None, None, b:b + 1], wl.dtype, f"capacity, request {b}")
    out, err = full_pass()
    assert err == 0
    assert_outputs_close(out[None, None], want[None, None], wl.dtype, "clean again")


# ---------------------------------------------------------------- FP8 E4M3 KV cache

FP8 = [
    _small("d128_g2", seed=131).fp8(),
    _small("d64_g1", head_dim=64, num_q_heads=2, num_kv_heads=2, seed=132).fp8(),
    _small("d128_g4", num_q_heads=8, num_kv_heads=2, seed=133).fp8(),
    _small("d64_g4_bs8_odd_scales", head_dim=64, num_q_heads=4, num_kv_heads=1, block_size=8,
           seed=134).fp8(k_scale=0.0371, v_scale=2.5, code_std=8.0),
    _small("d128_g8", num_q_heads=16, num_kv_heads=2, seed=139).fp8(),
    _small("d64_g8_bs8_odd_scales", head_dim=64, num_q_heads=8, num_kv_heads=1, block_size=8,
           seed=140).fp8(k_scale=0.0517, v_scale=1.75, code_std=8.0),
    _small("ring_wrap_bs64", sink=2, window=16, prefill=(100, 37, 5), steps=40, block_size=64, seed=135).fp8(),
    _small("ring_wrap_g4", num_q_heads=8, num_kv_heads=2, sink=2, window=16, prefill=(100, 37, 5), steps=40,
           block_size=64, seed=141).fp8(),
    _small("hybrid_focus", num_layers=8, sw_window=64, sink=4, window=128, batch=3,
           prefill=(1000, 2500, 6000), steps=10, layer_kind=tuple(0 if i % 4 == 3 else 1 for i in range(8)),
           focus=True, seed=136).fp8(),
]


def test_polling_merge_gives_up_and_flags_when_a_partial_never_arrives():
    """The merging workgroup of a polling pass waits a bounded time for the
    other splits' partials.  oda_test_merge_wait runs a Local pass in which
    split 0 of every (request, KV head) stores no partial, and caps the wait at
    a few re-reads: the call returns, every workgroup exits, the workspace's
    error word carries ODA_DEVERR_MERGE_WAIT and no output or lse is written.
    Once the workspace is prepared again, the same pass matches the oracle with
    a clean error word."""
    wl = _small("merge_wait", prefill=(300, 1200, 2600), steps=1, seed=191)
    st = DecodeState(wl, gen_device="cpu")
    st.prefill()
    q = W.gen_queries(wl, "cpu")[0].cuda()
    k_new, v_new = st.decode_inputs()
    score = np.full((1, wl.batch), -1.0, np.float32)  # nothing fires: the outputs are the Local pass's
    ks, vs = oracle_sequences(st)
    want = orc.decode_run(oracle_cfg(wl), wl.prefill, ks, vs, words(q.unsqueeze(0)), score)
    layer = 1
    args = (q[layer].contiguous(), k_new[0, layer].contiguous(), v_new[0, layer].contiguous())
    shape = (wl.batch, wl.num_q_heads, wl.head_dim)
    out = torch.full(shape, 7.0, device="cuda")
    lse = torch.full(shape[:2], 7.0, device="cuda")
    with pytest.raises(B.OdaError):  # the last split merges; it cannot be the withheld one
        B.test_merge_wait(st.dims, st.kv, layer, wl.batch, *args, out, lse, 10_000, 4, st.workspace)
    B.test_merge_wait(st.dims, st.kv, layer, wl.batch, *args, out, lse, 0, 4, st.workspace)
    torch.cuda.synchronize()
    err = st.device_error()
    say(f"withheld partial: error word {err}")
    assert err == B.DEVERR_MERGE_WAIT
    assert bool((out == 7.0).all()) and bool((lse == 7.0).all()), "a merge that gave up writes nothing"
    B.workspace_init(st.dims, wl.batch, st.workspace)
    B.decode_local(st.dims, st.kv, layer, wl.batch, *args, out, lse, st.workspace)
    torch.cuda.synchronize()
    assert st.device_error() == 0
    assert_outputs_close(out.cpu().numpy()[None, None], want["out"][:, layer:layer + 1], wl.dtype,
                         "after the workspace is prepared again")
    lse_err = float(np.abs(lse.cpu().numpy() - want["lse"][0, layer]).max())
    assert lse_err <= LSE_TOL[wl.dtype], lse_err


@pytest.mark.parametrize("wl", FP8, ids=[w.name for w in FP8])
def test_fp8_kv_runs_match_oracle(wl):
    """E4M3 codes in the caches, rings and new-token inputs, bf16 queries,
    per-tensor dequantisation scales; outputs to the bf16 bars."""
    _check_run(wl)


def test_fp8_graph_replay_matches_eager():
    wl = _small("graph", prefill=(50, 900, 2100), steps=12, seed=137).fp8()
    _, g_run, _ = _check_run(wl, graph=True)
    _, e_run, _ = _check_run(wl, graph=False)
    assert np.array_equal(g_run.out, e_run.out)


def test_fp8_equals_bf16_path_on_the_same_values():
    """Every E4M3 value is exact in bf16: the FP8 path with unit scales and
    the bf16 path over the decoded values see the same numbers, so their
    outputs agree to fp32 summation-order rounding."""
    wl8 = _small("same_values", prefill=(0, 700, 3001), steps=6, seed=138).fp8(k_scale=1.0, v_scale=1.0,
                                                                              code_std=1.0)
    st8 = DecodeState(wl8, gen_device="cpu")
    st8.prefill()
    q = W.gen_queries(wl8, "cpu")
    scores = W.gen_scores(wl8)
    r8 = run_steps(st8, q, scores)
    # the bf16 state holds the decoded values of the same codes
    wlb = wl8.with_(dtype="bf16", name="same_values_bf16")
    stb = DecodeState(wlb, gen_device="cpu")
    stb.sequence = lambda layer, b, which: W.gen_sequence(wl8, layer, b, which, "cpu").to(torch.bfloat16).to(stb.device)
    stb.prefill()
    rb = run_steps(stb, q, scores)
    assert np.array_equal(r8.counters[:, :6], rb.counters[:, :6])
    diff = float(np.abs(r8.out - rb.out).max())
    say(f"fp8 vs bf16 path on identical values: max diff {diff:.3e}")
    assert diff <= 2e-5


# ---------------------------------------------------------------- host-resident paged history

HOST = [
    _small("host_bf16_d128_g2", seed=141),
    _small("host_fp8_d64_g1", head_dim=64, num_q_heads=2, num_kv_heads=2, seed=142).fp8(),
    _small("host_hybrid_focus", num_layers=8, sw_window=64, sink=4, window=128, batch=3,
           prefill=(1000, 2500, 6000), steps=10, layer_kind=tuple(0 if i % 4 == 3 else 1 for i in range(8)),
           focus=True, seed=143),
]


@pytest.mark.parametrize("wl", HOST, ids=[w.name for w in HOST])
def test_host_resident_paged_history_matches_oracle(wl):
    """Paged caches in pinned host memory (prefill, commit and Full pass reach
    them over the host link), rings in HBM, replayed from a graph."""
    _check_run(wl, host_cache=True, graph=True)


def test_host_kv_pointer_rejects_device_and_pageable_memory():
    dev = torch.empty(1024, dtype=torch.uint8, device="cuda")
    pageable = torch.empty(1024, dtype=torch.uint8)
    for t in (dev, pageable):
        with pytest.raises(B.OdaError) as e:
            B.host_kv_pointer(t)
        assert e.value.status == -1
    pinned = torch.empty(1024, dtype=torch.uint8, pin_memory=True)
    assert B.host_kv_pointer(pinned) != 0
    torch.cuda.synchronize()
