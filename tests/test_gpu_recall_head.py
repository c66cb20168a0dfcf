"""GPU parity of the recall-head stand-in and of the step that computes its
recall scores on the device (oda_recall_scores, oda_step_recall) against the
CPU fp64 oracle.

Bar for the scores: the forward error bound of floating-point summation,
evaluated per request on the data, with the depth of the kernel's summation
trees -- |q_gpu - q| <= g(h1) S1 (1 + g(h2)) + g(h2) S2, where
S1 = sum_j |w2_j| (sum_i |W1_ji x_i| + |b1_j|), S2 = sum_j |w2_j max(u_j,0)| + |b2|,
g(h) = h u / (1 - h u), u = 2^-24 (bf16 products are exact in f32).  A term of
u_j passes at most h1 = 8 ceil(in_dim / 512) + 7 roundings (a lane's chain of
two-product dot steps, six lane-exchange additions, b1); a term of q at most
h2 = 17 + 8 ceil(groups / 512) (two fused adds per wave, eight wave partials,
the last workgroup's per-lane and lane-exchange additions, b2).  ReLU is
1-Lipschitz.  The step test's inputs are chosen so that every |q| exceeds its
bound: the oracle's own fp64 scores then fix every gate decision.
"""
import numpy as np
import pytest
import torch

import oracle as orc
from gated_kv_access_amd import binding as B
from gated_kv_access_amd import workloads as W
from gated_kv_access_amd.runner import RecallHead, StepRunner
from gated_kv_access_amd.state import DecodeState, make_dims
from tests.gpu_helpers import assert_outputs_close, oracle_cfg, oracle_sequences, say, words

pytestmark = pytest.mark.gpu

U = 2.0 ** -24


def _gamma(n):
    return n * U / (1 - n * U)


def _bound(w1, b1, w2, b2, x):
    """Per-request error bound of the head's output (see the module docstring)."""
    W1 = orc.bf16_to_f64(w1)
    X = orc.bf16_to_f64(np.atleast_2d(x))
    hidden, in_dim = W1.shape
    groups = -(-hidden // 16)
    h1 = 8 * -(-in_dim // 512) + 7
    h2 = 17 + 8 * -(-groups // 512)
    b1, w2 = b1.astype(np.float64), w2.astype(np.float64)
    u = X @ W1.T + b1
    s1 = (np.abs(X) @ np.abs(W1).T + np.abs(b1)) @ np.abs(w2)
    s2 = np.maximum(u, 0) @ np.abs(w2) + abs(b2)
    return _gamma(h1) * s1 * (1 + _gamma(h2)) + _gamma(h2) * s2


def _head(in_dim, hidden, seed, batch, b2=0.0):
    w1, b1, w2 = W.gen_recall_head(in_dim, hidden, seed=seed)
    return RecallHead(w1.cuda(), b1.cuda(), w2.cuda(), b2, batch), (w1, b1, w2)


@pytest.mark.parametrize("in_dim,hidden,batch", [(W.HEAD_IN_DIM, W.HEAD_HIDDEN, 1), (W.HEAD_IN_DIM, W.HEAD_HIDDEN, 5),
                                                 (W.HEAD_IN_DIM, W.HEAD_HIDDEN, 13), (64, 20, 3), (520, 37, 9)])
def test_recall_scores_match_oracle(in_dim, hidden, batch):
    say(f"recall head {in_dim} -> {hidden} -> 1, batch {batch}")
    b2 = -0.0625
    head, (w1, b1, w2) = _head(in_dim, hidden, 11 + batch, batch, b2)
    gen = torch.Generator().manual_seed(5 + batch)
    x = torch.randn((batch, in_dim), generator=gen).to(torch.bfloat16)
    scores = torch.full((batch + 3,), float("nan"), device="cuda")
    for _ in range(2):  # twice: the ticket word must be back at zero after a launch
        B.recall_scores(head.desc, batch, x.cuda(), scores, head.workspace)
        torch.cuda.synchronize()
        got = scores[:batch].cpu().numpy().astype(np.float64)
        want = orc.recall_head(words(w1), b1.numpy(), w2.numpy(), b2, words(x))
        bound = _bound(words(w1), b1.numpy(), w2.numpy(), b2, words(x))
        assert np.all(np.abs(got - want) <= bound), (np.abs(got - want) / bound).max()
        assert np.isnan(scores[batch:].cpu().numpy()).all()  # nothing written past the batch
    say(f"worst |dq| / bound {float((np.abs(got - want) / bound).max()):.3e}")


def test_recall_head_rejects_bad_descriptors():
    head, _ = _head(64, 20, 3, 2)
    bad = B.OdaRecallHead()
    for f, _ in B.OdaRecallHead._fields_:
        setattr(bad, f, getattr(head.desc, f))
    bad.in_dim = 60  # not a multiple of 8
    assert B.recall_workspace_size(bad, 2) == 0
    x = torch.zeros((2, 64), dtype=torch.bfloat16, device="cuda")
    s = torch.zeros(4, device="cuda")
    with pytest.raises(B.OdaError):
        B.recall_scores(head.desc, 2, x, s, head.workspace[:128])  # workspace too small


def test_step_with_device_recall_head_matches_oracle():
    """oda_step_recall: the gate reads the scores the head computed on the
    device from the staged decoding state; outputs, decisions and counters
    (F_Recall charged per step) against the oracle."""
    wl = W.Workload("head_step", 2, 4, 2, 128, "bf16", 3, (0, 700, 3001), 12, 4, 256, seed=154)
    hw1, hb1, hw2 = W.gen_recall_head(seed=9)
    b2 = -1.375  # centres the scores of these inputs: about half of the decisions fire
    head = RecallHead(hw1.cuda(), hb1.cuda(), hw2.cuda(), b2, wl.batch)
    dims = make_dims(wl, recall_flops=head.flops)
    st = DecodeState(wl, dims=dims, gen_device="cpu")
    st.prefill()
    q = W.gen_queries(wl, "cpu")
    hx = W.gen_head_inputs(wl, device="cpu")
    k_new, v_new = st.decode_inputs()
    r = StepRunner(st, q.cuda(), k_new, v_new, None, head=head, head_x=hx.cuda().contiguous())
    r.capture()
    outs, qs = [], []
    for _ in range(wl.steps):
        r.replay(1)
        torch.cuda.synchronize()
        outs.append(r.out.cpu().numpy().copy())
        qs.append(r.score_buf[:wl.batch].cpu().numpy().astype(np.float64))
    assert st.device_error() == 0
    got_q = np.stack(qs)
    want_q = np.stack([orc.recall_head(words(hw1), hb1.numpy(), hw2.numpy(), b2, words(hx[k]))
                       for k in range(wl.steps)])
    bound = np.stack([_bound(words(hw1), hb1.numpy(), hw2.numpy(), b2, words(hx[k])) for k in range(wl.steps)])
    assert np.all(np.abs(want_q) > bound), "inputs must leave no decision within the error bound"
    assert np.all(np.abs(got_q - want_q) <= bound)
    fired = got_q > 0
    assert np.array_equal(fired, want_q > 0)
    assert 0 < fired.sum() < fired.size
    say(f"device recall head: {int(fired.sum())} of {fired.size} decisions fire")
    scores = want_q.astype(np.float32)
    ks, vs = oracle_sequences(st)
    cfg = oracle_cfg(wl, recall_flops=head.flops)
    want = orc.decode_run(cfg, wl.prefill, ks, vs, words(q), scores)
    assert np.array_equal(r.full_calls.cpu().numpy(), want["full_calls"])
    assert np.array_equal(r.counters.cpu().numpy(), want["acct"])
    assert_outputs_close(np.stack(outs), want["out"], wl.dtype, wl.name)
