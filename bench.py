"""Decode-step throughput of the ODA hot path on one MI355X.

Workload (default): 28 layers, 16 query / 8 KV heads of 128, bf16 K/V
(--kv-dtype fp8: E4M3 K/V codes with per-tensor scales, bf16 queries),
batch 1, 131072-token prefilled context, s = 4, w = 2048, paged blocks of 16,
recall scores drawn so exactly 12.5% of the timed steps fire.  One step is
the whole hot path -- Local pass of every layer, device gate, gated Full pass
of every layer, fused commit -- replayed from a captured HIP graph.
--config selects another of the five workloads for an extra measurement line
(1: 16K context, 3: 32 requests of mixed length, 4: hybrid sliding/gated
layers with a focus region).

Prints one JSON line: steps/s (value), effective KV GB/s and its share of
HBM peak and of a plain device copy measured in the same run, the roofline of
the dominant kernel (the Full-pass attention kernel, timed with HIP events on
its launch stream), and the CPU oracle timed on a bounded sample as a
reported baseline.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0
TRAFFIC_FILE = {"bf16": os.path.join(ROOT, "profiles", "traffic_full_attention_ctx128k.json"),
                "fp8": os.path.join(ROOT, "profiles", "traffic_full_attention_ctx128k_fp8.json")}
DTYPE_LABEL = {"bf16": "bf16", "fp8": "fp8_e4m3 K/V, bf16 q"}
KERNEL_SRC = os.path.join(ROOT, "gated_kv_access_amd", "csrc", "oda_kernels.hip")
METRIC = "decode steps/s and effective KV GB/s (% HBM peak) at 128K ctx, rho=0.125"
ROOFLINE_WARM_REPLAYS = 4   # untimed replays of the roofline graph
ROOFLINE_TIMED_REPLAYS = 3  # timed replays


def log(msg: str) -> None:
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None, help="timed steps (default: 1024, or the workload's)")
    ap.add_argument("--warmup", type=int, default=8)
    ap.add_argument("--config", type=int, default=2, choices=(1, 2, 3, 4),
                    help="workload: 1 16K, 2 128K (headline), 3 batched mixed, 4 hybrid + focus")
    ap.add_argument("--focus", type=int, default=None, choices=(0, 1),
                    help="workload 4: a fired gated layer reads the focus set (1, default) or all positions (0)")
    ap.add_argument("--rho", type=float, default=None, help="override the Full-call rate")
    ap.add_argument("--q-heads", type=int, default=None,
                    help="override the query heads (a multiple of the KV heads: GQA group 1, 2 or 4)")
    ap.add_argument("--kv-dtype", choices=("bf16", "fp8"), default="bf16",
                    help="KV cache storage: bf16, or FP8 E4M3 codes with per-tensor scales")
    ap.add_argument("--host-kv", action="store_true",
                    help="paged history in pinned host memory (rings in HBM); the Full pass reads it over the host link")
    ap.add_argument("--recall-head", action="store_true",
                    help="compute the recall scores on the device with the recall-head stand-in "
                         "(6144 -> 4608 -> 1, seeded weights, b2 set so that about rho of the steps fire)")
    ap.add_argument("--reps", type=int, default=1,
                    help="timed repetitions of the whole measurement from the same state (value: the median)")
    ap.add_argument("--roofline-launches", type=int, default=56)
    ap.add_argument("--full-splits", type=int, default=0,
                    help="split-K ranges per (request, KV head) of Full passes (0: the library's choice)")
    ap.add_argument("--local-splits", type=int, default=0,
                    help="split-K ranges per (request, KV head) of ring passes (0: the library's choice)")
    ap.add_argument("--sweep", action="store_true",
                    help="also time rho=0, rho=1 and always-Full for the savings check (always done for "
                         "the 128K workload)")
    ap.add_argument("--no-delta-f", action="store_true",
                    help="skip the rho=0 / rho=1 / always-Full legs of the savings check")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-layers", type=int, default=4, help="layers in the oracle sample")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run a plain 1 GiB device copy 8 times (reference for HBM byte counters)")
    return ap.parse_args()


def copy_rate(n: int = 1 << 30, launches: int = 8):
    """A plain device copy of n bytes: returns (us per launch, read+write GB/s)."""
    import torch
    src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(launches):
        dst.copy_(src)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / launches
    del src, dst
    torch.cuda.empty_cache()
    return ms * 1e3, 2 * n / (ms * 1e-3) / 1e9


def host_copy_rate(n: int = 1 << 30, launches: int = 4) -> float:
    """Pinned host to device copy of n bytes (DMA): GB/s."""
    import torch
    src = torch.empty(n, dtype=torch.uint8, pin_memory=True)
    dst = torch.empty(n, dtype=torch.uint8, device="cuda")
    dst.copy_(src, non_blocking=True)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(launches):
        dst.copy_(src, non_blocking=True)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / launches
    del src, dst
    return n / (ms * 1e-3) / 1e9


def calibrate_copy() -> int:
    n = 1 << 30
    us, gbps = copy_rate(n)
    print(json.dumps({"calibration": "device copy", "bytes_read_per_launch": n, "bytes_written_per_launch": n,
                      "launches": 8, "us_per_launch": round(us, 2), "gbps_read_plus_write": round(gbps, 1)}),
          flush=True)
    return 0


def kernel_sha() -> str:
    """Hash of the kernel source's code: comments, blank lines and trailing
    spaces are dropped, so a change of comments keeps the recorded counters."""
    import re
    with open(KERNEL_SRC) as f:
        text = f.read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    lines = [re.sub(r"//.*$", "", ln).rstrip() for ln in text.splitlines()]
    code = "\n".join(ln for ln in lines if ln.strip())
    return hashlib.sha256(code.encode()).hexdigest()[:16]


def exact_rate_blocks(wl, K: int, max_blocks: int = 64) -> int:
    """Blocks of K steps needed so that exactly rho of all timed steps fire
    (scores drawn by the 'exact' mode: a seeded choice of round(rho * n) of n
    steps).  rho * K need not be whole: with r blocks the choice is made over
    r * K steps, r the least for which rho * r * K is whole (rho = 1/8 and
    K = 20: two blocks, 5 of 40 steps fire).  1 for the other score modes."""
    from fractions import Fraction
    if wl.score_mode != "exact" or len(set(wl.rho)) != 1:
        return 1
    fr = Fraction(wl.rho[0]).limit_denominator(10 ** 6)
    for r in range(1, max_blocks + 1):
        if (fr * r * K).denominator == 1:
            return r
    return 1


def build_workload(args):
    from gated_kv_access_amd import workloads as W
    base = W.config(args.config)
    if args.config == 4 and args.focus is not None:
        base = base.with_(focus=bool(args.focus))
    if args.kv_dtype == "fp8":
        base = base.fp8()
    if args.rho is not None:
        base = base.with_(rho=(args.rho,))
    if args.q_heads is not None:
        base = base.with_(name=f"{base.name}_q{args.q_heads}", num_q_heads=args.q_heads)
    K = args.steps if args.steps is not None else (1024 if args.config == 2 else base.steps)
    return base, K


def main() -> int:
    args = parse()
    if args.calibrate_copy:
        return calibrate_copy()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the path shards by request or KV head with no exchange; see the design notes)",
              file=sys.stderr)
        return 2
    import numpy as np
    import torch

    from gated_kv_access_amd import binding as B
    from gated_kv_access_amd import workloads as W
    from gated_kv_access_amd.runner import RecallHead, StepRunner
    from gated_kv_access_amd.state import DecodeState, make_dims

    B.load()
    base, K = build_workload(args)
    Wm = args.warmup
    # Timed: r blocks of K steps, so that exactly rho of them fire.
    nblk = exact_rate_blocks(base, K)
    T = nblk * K
    wl = base.with_(steps=Wm + T)
    pre = np.array(wl.prefill, dtype=np.int64)
    log(f"workload {wl.name}: batch {wl.batch}, prefill {pre.min()}..{pre.max()}, warmup {Wm}, timed {T} "
        f"({nblk} block(s) of {K}), rho {wl.rho if len(wl.rho) < 5 else 'per request'}")
    if args.config == 3:
        free = torch.cuda.mem_get_info()[0]
        need = float((pre + Wm + T).sum()) * wl.num_layers * wl.num_kv_heads * wl.head_dim * 2 * wl.esize
        if need > 0.92 * free:
            log(f"paged cache of {need / 1e9:.0f} GB does not fit the {free / 1e9:.0f} GB free")
            return 1
    t0 = time.time()
    head = head_x = None
    if args.recall_head:
        head, head_x = make_head(wl, Wm + T)
    dims = make_dims(wl, full_splits=args.full_splits, local_splits=args.local_splits,
                     recall_flops=head.flops if head else 0)
    st = DecodeState(wl, gen_device="cuda", host_cache=args.host_kv, dims=dims)
    st.prefill()
    q = W.gen_queries(wl, "cuda")
    k_new, v_new = st.decode_inputs()
    sc = np.concatenate([W.gen_scores(wl.with_(steps=Wm)), W.gen_scores(wl.with_(steps=T))], 0) \
        if Wm > 0 else W.gen_scores(wl.with_(steps=T))
    scores = torch.from_numpy(sc).cuda()
    log(f"setup {time.time() - t0:.1f}s")

    r = StepRunner(st, q, k_new, v_new, None if head else scores, want_lse=False, head=head, head_x=head_x)
    r.capture()
    r.replay(Wm)
    torch.cuda.synchronize()
    start_len = st.seq_len.clone()

    def restore():
        st.seq_len.copy_(start_len)
        B.ring_init(st.dims, st.kv, wl.batch, st.workspace)  # ring state of the restored context
        r.step_counter[0] = Wm
        torch.cuda.synchronize()

    times = []
    block_ms = []
    acct = None
    for rep in range(max(1, args.reps)):
        if rep:
            restore()
        acct0 = r.counters.clone()
        blocks = []
        for _ in range(nblk):
            start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            torch.cuda.synchronize()
            start.record()
            r.replay(K)
            end.record()
            torch.cuda.synchronize()
            blocks.append(start.elapsed_time(end))
        times.append(sum(blocks))
        if acct is None:
            acct = (r.counters - acct0).cpu().numpy().sum(0)
            block_ms = blocks
    if st.device_error() != 0:
        log(f"device error word {st.device_error()}")
        return 1
    ms = statistics.median(times)  # for T steps
    f = dict(zip(B.ACCT_FIELDS, acct.tolist()))
    steps_per_s = T / (ms / 1e3)
    kv_gbps = f["kv_bytes"] / (ms / 1e3) / 1e9
    rho_realised = f["full_calls"] / (T * wl.batch)
    log(f"timed {T} steps in {ms:.1f} ms (median of {len(times)}): {steps_per_s:.1f} steps/s, "
        f"{kv_gbps:.0f} GB/s effective KV, {f['full_calls']} Full calls (rho realised {rho_realised:.4f})")

    roofline = roofline_leg(args, st, wl, q, k_new, v_new)
    copy_us, copy_gbps = copy_rate()
    log(f"device copy reference: {copy_gbps:.0f} GB/s read+write")
    host_gbps = None
    if args.host_kv:
        host_gbps = host_copy_rate()
        log(f"host-to-device DMA reference: {host_gbps:.1f} GB/s")
        # the ceiling of this line is the host link, measured here as a DMA copy
        roofline["bound"] = "host_link"
        roofline["peak"] = round(host_gbps, 1)
        roofline["peak_kind"] = "measured pinned-host-to-device DMA"
        roofline["frac"] = round(roofline["achieved"] / host_gbps, 4)

    extra = {}
    if head is not None:
        extra["recall_head"] = recall_head_leg(head, head_x, wl.batch)
    if (args.sweep or args.config == 2) and not args.no_delta_f:
        legs = sweep(st, wl, q, k_new, v_new, K, Wm, start_len)
        extra["delta_f"] = delta_f_check(legs, ms / T * 1e3, f, wl, rho_realised, kv_gbps, roofline)

    cpu = None
    if not args.no_cpu_baseline:
        if wl.batch == 1 and not wl.sliding_layers:
            cpu = cpu_baseline(st, wl, q, float(wl.rho[0]), args.cpu_layers)
        else:
            log("cpu baseline: timed on the single-request workloads only")

    res = {
        "metric": METRIC,
        "value": round(steps_per_s, 2),
        "unit": "steps/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": Wm,
        "ms_per_step": round(ms / T, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": DTYPE_LABEL[args.kv_dtype],
        "data": "synthetic",
        "config": {"workload": wl.name, "layers": wl.num_layers, "q_heads": wl.num_q_heads,
                   "kv_heads": wl.num_kv_heads, "head_dim": wl.head_dim, "batch": wl.batch,
                   "prefill": int(pre[0]) if wl.batch == 1 else [int(pre.min()), int(pre.max())],
                   "sink": wl.sink, "window": wl.window, "block_size": wl.block_size,
                   "rho": list(wl.rho) if len(wl.rho) > 1 else wl.rho[0],
                   "rho_realised": round(rho_realised, 6), "timed_steps": T, "timed_blocks": nblk,
                   "kv_dtype": wl.dtype,
                   "sliding_layers": len(wl.sliding_layers), "focus": bool(wl.focus),
                   "paged_history": "pinned host memory" if args.host_kv else "HBM",
                   "recall_score": "device recall head" if head is not None else "staged input",
                   "full_calls_timed": int(f["full_calls"]), "parallelism": "single GPU"},
        "tokens_per_s": round(steps_per_s * wl.batch, 2),
        "effective_kv_gbps": round(kv_gbps, 1),
        "pct_hbm_peak": round(100 * kv_gbps / HBM_PEAK_GBPS, 2),
        "device_copy_gbps": round(copy_gbps, 1),
        "pct_device_copy": round(100 * kv_gbps / copy_gbps, 2),
        "flops_ratio_vs_full": round((f["f_local"] + f["f_full_taken"] + f["f_recall"]) / f["f_full_always"], 5),
        "roofline": roofline,
        "cpu_baseline": cpu,
    }
    res["ms_per_block"] = [round(t, 3) for t in block_ms]
    if len(times) > 1:
        res["ms_per_rep"] = [round(t, 3) for t in times]
    res.update(extra)
    print(json.dumps(res), flush=True)
    return 0


def make_head(wl, steps):
    """The recall-head stand-in with seeded weights and per-step inputs; b2 is the
    (1 - rho) quantile of the scores without it, computed with torch in float32
    (a calibration of the synthetic input, not part of the timed path)."""
    import torch

    from gated_kv_access_amd import workloads as W
    from gated_kv_access_amd.runner import RecallHead

    w1, b1, w2 = W.gen_recall_head(device="cuda")
    hx = W.gen_head_inputs(wl, device="cuda", steps=steps).contiguous()
    q0 = torch.relu(hx.float().reshape(-1, hx.shape[-1]) @ w1.float().T + b1) @ w2
    rho = float(sum(wl.rho) / len(wl.rho))
    b2 = -float(torch.quantile(q0, 1.0 - rho)) if 0.0 < rho < 1.0 else (-1e30 if rho <= 0 else 1e30)
    head = RecallHead(w1, b1, w2, b2, wl.batch)
    log(f"recall head: {head.params} parameters, b2 = {b2:.4f} for rho {rho}")
    return head, hx


def recall_head_leg(head, hx, batch, launches=50):
    """The recall-head kernel on its own: launch time and weight-streaming rate."""
    import torch

    from gated_kv_access_amd import binding as B

    s = torch.zeros(batch + 4, dtype=torch.float32, device="cuda")
    x = hx[0].contiguous()
    B.recall_scores(head.desc, batch, x, s, head.workspace)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(launches):
        B.recall_scores(head.desc, batch, x, s, head.workspace)
    e1.record()
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / launches
    wbytes = head.w1.numel() * 2 + (head.b1.numel() + head.w2.numel()) * 4
    log(f"recall head kernel: {us:.1f} us/launch, {wbytes / (us * 1e-6) / 1e9:.0f} GB/s of weights")
    return {"params": head.params, "flops_per_request": head.flops, "us_per_launch": round(us, 2),
            "weight_bytes": wbytes, "weight_gbps": round(wbytes / (us * 1e-6) / 1e9, 1), "launches": launches}


def roofline_leg(args, st, wl, q, k_new, v_new):
    """The dominant kernel: the Full-pass attention kernel (split-K over the paged
    cache + merge), one launch per oda_decode_full_gated call on a gated layer,
    every request firing.  The launches are captured into a HIP graph and
    replayed, as in the decode step: after ROOFLINE_WARM_REPLAYS untimed
    replays, ROOFLINE_TIMED_REPLAYS replays are timed with HIP events on the
    stream the graph replays on (torch's current stream)."""
    import torch

    from gated_kv_access_amd import binding as B

    Bn, Hkv, d = wl.batch, wl.num_kv_heads, wl.head_dim
    gated = list(wl.gated_layers)
    fire = torch.ones(max(4, Bn + (-Bn) % 4), dtype=torch.float32, device="cuda")
    out = torch.empty((Bn, wl.num_q_heads, d), dtype=torch.float32, device="cuda")
    # rows each launch streams from the paged cache: the library's own Full set, minus t
    cap = max(wl.rows(b) for b in range(Bn)) + 8
    pos = torch.empty(cap, dtype=torch.int32, device="cuda")
    cnt = torch.zeros(1, dtype=torch.int64, device="cuda")
    rows = 0
    for b in range(Bn):
        B.access_set(st.dims, st.kv, gated[0], b, 1, pos, cnt, st.workspace)
        rows += int(cnt.item()) - 1
    bytes_per_launch = rows * Hkv * d * 2 * wl.esize  # K and V rows streamed from the paged cache
    qs = [q[-1, l].contiguous() for l in gated]
    ks = [k_new[-1, l].contiguous() for l in gated]
    vs = [v_new[-1, l].contiguous() for l in gated]
    R = args.roofline_launches
    # The launches are replayed from a HIP graph, as the decode step runs them.
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        with torch.cuda.graph(g, stream=side):
            for i in range(R):
                j = i % len(gated)
                B.decode_full_gated(st.dims, st.kv, gated[j], Bn, qs[j], ks[j], vs[j], fire, 0.0, out, None, None,
                                    None, st.workspace)
    torch.cuda.current_stream().wait_stream(side)
    # The first replays after the light Local-only steps run slower (they
    # settle within about four replays of 56 launches): warm up, then time.
    for _ in range(ROOFLINE_WARM_REPLAYS):
        g.replay()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(ROOFLINE_TIMED_REPLAYS):
        g.replay()
    e1.record()
    torch.cuda.synchronize()
    avg_us = e0.elapsed_time(e1) * 1e3 / (R * ROOFLINE_TIMED_REPLAYS)
    achieved = bytes_per_launch / (avg_us * 1e-6) / 1e9
    R = R * ROOFLINE_TIMED_REPLAYS  # launches timed
    kernel = f"attention_kernel<{args.kv_dtype},{d},G{wl.num_q_heads // Hkv},paged,ballot>"
    # The committed counters hold for the profiled kernel and workload only: the
    # same kernel source, build variant and 128K workload, history in HBM.
    traffic = None
    tf = TRAFFIC_FILE[args.kv_dtype]
    if args.config == 2 and not args.host_kv and os.path.exists(tf):
        with open(tf) as fh:
            tr = json.load(fh)
        if tr.get("kernel_sha") == kernel_sha() and tr.get("kernel") == kernel:
            traffic = tr.get("hbm_bytes_per_launch")
    log(f"roofline: Full-pass kernel {avg_us:.1f} us/launch, {achieved:.0f} GB/s = "
        f"{100 * achieved / HBM_PEAK_GBPS:.1f}% of HBM peak")
    return {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBPS, 4), "traffic": traffic, "kernel": kernel,
            "avg_launch_us": round(avg_us, 2), "bytes_per_launch": bytes_per_launch, "launches": R}


def sweep(st, wl, q, k_new, v_new, K, Wm, start_len):
    """rho = 0, rho = 1 and always-Full over K steps from the timed run's start,
    for the step-time ratio against the FLOP prediction of the per-step savings
    equation.  Returns microseconds per step of each leg."""
    import torch

    from gated_kv_access_amd import binding as B
    from gated_kv_access_amd.runner import StepRunner

    Bn = wl.batch
    out = {}

    def time_runner(r, label):
        st.seq_len.copy_(start_len)
        B.ring_init(st.dims, st.kv, Bn, st.workspace)  # ring state of the reset context
        r.capture()
        s0, s1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        s0.record()
        r.replay(K)
        s1.record()
        torch.cuda.synchronize()
        ms = s0.elapsed_time(s1)
        log(f"sweep {label}: {K / (ms / 1e3):.1f} steps/s ({ms / K * 1e3:.1f} us/step)")
        return ms / K

    for label, val in (("rho0", -1.0), ("rho1", 1.0)):
        sc = torch.full((q.shape[0], Bn), val, dtype=torch.float32, device="cuda")
        r = StepRunner(st, q, k_new, v_new, sc, want_lse=False)
        r.step_counter[0] = Wm
        out[f"us_per_step_{label}"] = round(time_runner(r, label) * 1e3, 2)
    # Always-Full: every layer's Full pass and the commit, no Local attempt, no gate.
    fire = torch.ones(max(4, Bn + (-Bn) % 4), dtype=torch.float32, device="cuda")
    L = wl.num_layers
    o = torch.empty((L, Bn, wl.num_q_heads, wl.head_dim), dtype=torch.float32, device="cuda")
    ctr = torch.tensor([Wm, 0], dtype=torch.int64, device="cuda")
    qb, kb, vb = torch.empty_like(q[0]), torch.empty_like(k_new[0]), torch.empty_like(v_new[0])

    class FullOnly:
        def capture(self):
            g = torch.cuda.CUDAGraph()
            s = torch.cuda.Stream()
            s.wait_stream(torch.cuda.current_stream())
            with torch.cuda.stream(s):
                with torch.cuda.graph(g, stream=s):
                    B.stage_step([q, k_new, v_new], [qb, kb, vb], ctr, q.shape[0])
                    for l in range(L):
                        B.decode_full_gated(st.dims, st.kv, l, Bn, qb[l], kb[l], vb[l], fire, 0.0, o[l], None,
                                            None, None, st.workspace)
                    B.commit_kv(st.dims, st.kv, Bn, kb, vb, st.workspace)
            torch.cuda.current_stream().wait_stream(s)
            self.g = g

        def replay(self, n):
            for _ in range(n):
                self.g.replay()

    ms_full = time_runner(FullOnly(), "always-Full")
    out["us_per_step_full_only"] = round(ms_full * 1e3, 2)
    return out


def delta_f_check(legs, us_rho, f, wl, rho_realised, kv_gbps, roofline):
    """The savings check of the per-step savings equation (picx.dev summary,
    "Computational Savings"): the measured step-time ratio against always-Full,
    R = T(rho) / T(always-Full), beside the FLOP ratio the counters give,
    R_hat = sum(F_Local + F_Recall + a_t F_Full(t)) / sum(F_Full(t)); the affine
    model T(rho) = T(0) + rho (T(1) - T(0)); and the shortfall against 70% of
    HBM peak on the KV bytes read, at always-Full, rho = 1 and the timed rho."""
    t0, t1, tf = legs["us_per_step_rho0"], legs["us_per_step_rho1"], legs["us_per_step_full_only"]
    r_hat = (f["f_local"] + f["f_recall"] + f["f_full_taken"]) / f["f_full_always"]
    r_meas = us_rho / tf
    affine = t0 + rho_realised * (t1 - t0)
    # KV bytes per step of the legs, from the counters' attended positions
    # (F counts 4 * Hq * d per attended position and layer; a position and
    # layer is Hkv * d * 2 * element-size bytes of K and V)
    per_step = wl.batch / f["steps"]
    per_pos = wl.num_kv_heads * wl.head_dim * 2 * wl.esize
    fpp = 4 * wl.num_q_heads * wl.head_dim
    full_b = f["f_full_always"] / fpp * per_pos * per_step
    loc_b = f["f_local"] / fpp * per_pos * per_step
    frac = {"always_full": full_b / (tf * 1e-6) / 1e9 / HBM_PEAK_GBPS,
            "rho1": (full_b + loc_b) / (t1 * 1e-6) / 1e9 / HBM_PEAK_GBPS,
            "timed_rho": kv_gbps / HBM_PEAK_GBPS,
            "full_pass_kernel": roofline["frac"]}
    out = {"us_per_step_rho0": t0, "us_per_step_rho1": t1, "us_per_step_full_only": tf,
           "us_per_step_timed": round(us_rho, 2), "rho_realised": round(rho_realised, 6),
           "R_measured": round(r_meas, 5), "R_hat": round(r_hat, 5),
           "R_over_R_hat": round(r_meas / r_hat, 4),
           "fixed_cost_us": round(us_rho - r_hat * tf, 2),
           "affine_predicted_us": round(affine, 2), "affine_residual_us": round(us_rho - affine, 2),
           "hbm_frac": {k: round(v, 4) for k, v in frac.items()},
           "target_hbm_frac": 0.70,
           "target_met": {k: bool(v >= 0.70) for k, v in frac.items()}}
    log(f"delta-F: R = {r_meas:.4f} vs R_hat = {r_hat:.4f}; T(0) {t0:.1f} us, T(1) {t1:.1f} us, "
        f"always-Full {tf:.1f} us; affine residual {us_rho - affine:+.1f} us; "
        f"HBM fractions {', '.join(f'{k} {v:.3f}' for k, v in frac.items())} (target 0.70)")
    return out


def cpu_baseline(st, wl, q, rho, n_layers):
    """The fp64 oracle on the host cores over a bounded sample: n_layers of the
    layers, 2 Local-only and 2 fired steps at the end of the timed context,
    scaled linearly to all layers and combined as T(rho) = (1-rho) T_L + rho T_F;
    then the same with one thread on one layer and one step of each kind."""
    import numpy as np
    import torch

    import oracle as orc
    from gated_kv_access_amd import workloads as W

    t_end = int(st.seq_len[0].item())  # positions committed by the end of the run
    fp8 = wl.dtype == "fp8"
    kv_words = (lambda x: x.view(torch.uint8).cpu().numpy()) if fp8 else \
        (lambda x: x.view(torch.int16).cpu().numpy().view(np.uint16))
    ks = np.zeros((n_layers, 1, t_end, wl.num_kv_heads, wl.head_dim), np.uint8 if fp8 else np.uint16)
    vs = np.zeros_like(ks)
    for l in range(n_layers):
        ks[l, 0] = kv_words(W.gen_sequence(wl, l, 0, "k", "cuda")[:t_end])
        vs[l, 0] = kv_words(W.gen_sequence(wl, l, 0, "v", "cuda")[:t_end])
    qq = q[:2, :n_layers].contiguous().view(torch.int16).cpu().numpy().view(np.uint16)

    def run(layers, k, threads):
        orc.set_threads(threads)
        cfg = orc.OracleConfig(layers, wl.num_q_heads, wl.num_kv_heads, wl.head_dim, sink=wl.sink,
                               window=wl.window, dtype=orc.FP8 if fp8 else orc.BF16,
                               k_scale=wl.k_scale, v_scale=wl.v_scale)
        tm = {}
        for label, val in (("local", -1.0), ("full", 1.0)):
            s = np.full((k, 1), val, np.float32)
            t0 = time.perf_counter()
            orc.decode_run(cfg, [t_end - k], ks[:layers], vs[:layers],
                           np.ascontiguousarray(qq[:k, :layers]), s)
            tm[label] = (time.perf_counter() - t0) / k * (wl.num_layers / layers)
        return tm

    threads = orc.get_threads()
    tm = run(n_layers, 2, threads)
    t_step = (1 - rho) * tm["local"] + rho * tm["full"]
    log(f"cpu oracle ({threads} threads): Local step {tm['local']:.3f}s, Full step {tm['full']:.3f}s "
        f"(scaled to {wl.num_layers} layers)")
    tm1 = run(1, 1, 1)
    orc.set_threads(threads)
    t1 = (1 - rho) * tm1["local"] + rho * tm1["full"]
    log(f"cpu oracle (1 thread): Local step {tm1['local']:.3f}s, Full step {tm1['full']:.3f}s")
    return {"value": round(1.0 / t_step, 4), "unit": "steps/s", "cores": threads, "kind": "oracle",
            "sample": f"{n_layers} of {wl.num_layers} layers, 2 Local-only + 2 fired steps at "
                      f"t={t_end - 1}..{t_end}, scaled linearly to all layers, "
                      f"T(rho)=(1-rho)T_L+rho*T_F with rho={rho}",
            "value_1thread": round(1.0 / t1, 5),
            "sample_1thread": f"1 layer, 1 Local-only + 1 fired step at t={t_end}, 1 thread, same scaling"}


if __name__ == "__main__":
    sys.exit(main())
