"""oda_step_static (the step entry point that allocates nothing: its workspace
is a static device array per GPU) against oda_step with a caller workspace,
through the C ABI.  Two identical decode states take the same two calls in a
row, the second with a smaller batch, so the second static call runs on the
scratch the first one left behind.  Outputs meet the bars of the parity tests
(the static entry point merges every pass by ticket, oda_step polls where a
launch fits the chip, so the last bits may differ); call lists, counts,
Full-call totals, accounting counters, committed caches, rings and lengths
are compared bit for bit."""
import numpy as np
import pytest
import torch

from gated_kv_access_amd import binding as B
from gated_kv_access_amd import workloads as W
from gated_kv_access_amd.state import DecodeState, make_dims
from tests.gpu_helpers import LSE_TOL, TOL, say

pytestmark = pytest.mark.gpu

CASES = {
    "small_bf16_g2": W.Workload("noalloc_small_bf16", 2, 4, 2, 128, "bf16", 3, (130, 70, 200), 2, 4, 64,
                                score_mode="normal", seed=41),
    "small_fp8_g4": W.Workload("noalloc_small_fp8", 2, 8, 2, 128, "bf16", 3, (300, 40, 95), 2, 4, 64,
                               score_mode="normal", seed=42).fp8(),
    "ctx16k_bf16_g2": W.Workload("noalloc_16k", 28, 16, 8, 128, "bf16", 2, (16384, 9000), 2, 4, 2048,
                                 score_mode="normal", seed=43),
}
# call 1: all requests, requests 0 and 2 fire; call 2: the first two, request 1 fires
SCORES = ([1.0, -1.0, 0.5], [-0.5, 2.0])


def _bytes(t):
    return t.view(torch.uint8).cpu().numpy() if t is not None else None


def _state_arrays(st):
    return {n: _bytes(getattr(st, n)) for n in ("k_cache", "v_cache", "k_ring", "v_ring", "ring_pos", "seq_len")}


@pytest.mark.parametrize("case", sorted(CASES))
def test_step_static_matches_step_on_two_calls(gpu_lib, case):
    wl = CASES[case]
    say(f"no-alloc {case}: batch {wl.batch}, {wl.num_layers} layers, prefill {wl.prefill}")
    dims = make_dims(wl)
    need = B.workspace_size(dims, wl.batch)
    assert 0 < need <= 4 << 20, need
    sa = DecodeState(wl, gen_device="cuda", dims=dims)
    sb = DecodeState(wl, gen_device="cuda", dims=make_dims(wl))
    sa.prefill()
    sb.prefill()
    q = W.gen_queries(wl, "cuda")
    k_new, v_new = sa.decode_inputs()
    L, Hq, Hkv, d = wl.num_layers, wl.num_q_heads, wl.num_kv_heads, wl.head_dim
    for call, n in enumerate((wl.batch, wl.batch - 1)):
        qs = q[call, :, :n].contiguous()
        ks = k_new[call, :, :n].contiguous()
        vs = v_new[call, :, :n].contiguous()
        sc = torch.tensor(SCORES[call] + [0.0] * ((-n) % 4), dtype=torch.float32, device="cuda")
        res = []
        for st, static in ((sa, False), (sb, True)):
            out = torch.full((L, n, Hq, d), float("nan"), dtype=torch.float32, device="cuda")
            lse = torch.full((L, n, Hq), float("nan"), dtype=torch.float32, device="cuda")
            clist = torch.full((n,), -9, dtype=torch.int32, device="cuda")
            ccount = torch.full((4,), -9, dtype=torch.int32, device="cuda")
            fcalls = torch.zeros(n, dtype=torch.int64, device="cuda")
            ctr = torch.zeros((n, len(B.ACCT_FIELDS)), dtype=torch.int64, device="cuda")
            if static:
                B.step_static(st.dims, st.kv, n, qs, None, ks, vs, sc, 0.0, out, lse, clist, ccount, fcalls, ctr)
            else:
                B.step(st.dims, st.kv, n, qs, None, ks, vs, sc, 0.0, out, lse, clist, ccount, fcalls, ctr,
                       st.workspace)
            torch.cuda.synchronize()
            res.append(dict(out=out.cpu().numpy(), lse=lse.cpu().numpy(), clist=clist.cpu().numpy(),
                            ccount=int(ccount[0].item()), fcalls=fcalls.cpu().numpy(), ctr=ctr.cpu().numpy()))
        ref, got = res
        fired = [b for b in range(n) if SCORES[call][b] > 0]
        assert ref["ccount"] == got["ccount"] == len(fired)
        assert ref["clist"].tolist() == got["clist"].tolist() == fired + [-1] * (n - len(fired))
        assert np.array_equal(ref["fcalls"], got["fcalls"]) and np.array_equal(ref["ctr"], got["ctr"])
        assert np.all(np.isfinite(got["out"])) and np.all(np.isfinite(got["lse"]))
        atol, rtol = TOL[wl.dtype]
        worst = 0.0
        for l in range(L):
            diff = got["out"][l].astype(np.float64) - ref["out"][l]
            mabs = float(np.abs(diff).max())
            rel = float(np.linalg.norm(diff) / np.linalg.norm(ref["out"][l]))
            worst = max(worst, mabs)
            assert mabs <= atol and rel <= rtol, (case, call, l, mabs, rel)
            assert float(np.abs(got["lse"][l] - ref["lse"][l]).max()) <= LSE_TOL[wl.dtype], (case, call, l)
        arrs_a, arrs_b = _state_arrays(sa), _state_arrays(sb)
        for name in arrs_a:
            if arrs_a[name] is not None:
                assert np.array_equal(arrs_a[name], arrs_b[name]), (case, call, name)
        say(f"no-alloc {case}: call {call + 1} (batch {n}, fired {fired}) matches oda_step, "
            f"worst max-abs {worst:.3e}")
