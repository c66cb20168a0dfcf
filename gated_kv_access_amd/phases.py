"""Phase timings and workgroup balance of one attention launch, from the
profiling build liboda_phases.so (include/oda_phases.h).

    python -m gated_kv_access_amd.phases --config 3 --pass full

Sets up a workload's decode state, records the pass of layers 0..3 (Full:
every request firing, through oda_decode_full_gated; Local: oda_decode_local)
into a HIP graph, replays it, clears the stamps and replays it once more, then
reads the stamps of that replay's last launch.  Prints per-phase percentiles
(us from the first workgroup's entry), static-phase ends per XCD, and the
launch's use of the 256 compute units: the CU-time its workgroups were
running, and the idle CU-time after the last workgroup was dispatched.
"""
from __future__ import annotations

import argparse
import ctypes
import os
import sys

import numpy as np

PHASES = ("entry", "state", "tile0", "static", "pool", "fold", "stored", "merged")
COMPUTE_UNITS = 256


def load_phases_lib():
    from . import binding as B
    from .build import PHASES_LIB
    if not os.path.exists(PHASES_LIB):
        raise FileNotFoundError(f"{PHASES_LIB} is missing: build it with __graft_entry__.build()")
    B.LIB_PATH = PHASES_LIB
    B.load.__defaults__ = (PHASES_LIB,)
    lib = B.load()
    lib.oda_phase_stamps_read.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t]
    lib.oda_phase_stamps_clear.argtypes = []
    return lib


def summarize(stamps: np.ndarray, xcc: np.ndarray, groups: int, event_us: float, label: str) -> dict:
    """stamps [n][8] raw counter values of one launch (phase 0 > 0 for the
    workgroups that ran); returns and prints the figures."""
    run = stamps[:groups, 0] > 0
    st = stamps[:groups][run].astype(np.int64)
    xc = xcc[:groups][run]
    t0 = st[:, 0].min()
    # a phase counts for this launch only if it is not before the workgroup's entry
    valid = st >= st[:, :1]
    rel = np.where(valid, (st - t0) / 100.0, np.nan)
    end = np.nanmax(rel, axis=1)
    start = rel[:, 0]
    span = float(end.max())
    print(f"== {label}: {st.shape[0]} workgroups; {event_us:.2f} us per launch by HIP events; "
          f"stamped span {span:.2f} us")
    for k, nm in enumerate(PHASES):
        col = rel[:, k]
        col = col[~np.isnan(col)]
        if col.size:
            print(f"  {nm:7s} n {col.size:5d}  min {col.min():8.2f}  p10 {np.percentile(col, 10):8.2f}  "
                  f"med {np.median(col):8.2f}  p90 {np.percentile(col, 90):8.2f}  max {col.max():8.2f}")
    stat = rel[:, 3]
    by_xcc = {int(x): float(np.nanmedian(stat[xc == x])) for x in sorted(set(xc.tolist())) if np.any(~np.isnan(stat[xc == x]))}
    if by_xcc:
        print("  static rows done, median by XCD: " + " ".join(f"{x}:{v:.1f}" for x, v in by_xcc.items()))
    busy = float((end - start).sum())
    last_start = float(start.max())
    tail_busy = float(np.clip(end - np.maximum(start, last_start), 0, None).sum())
    idle_tail = COMPUTE_UNITS * (span - last_start) - tail_busy
    out = {"workgroups": int(st.shape[0]), "event_us": round(event_us, 2), "span_us": round(span, 2),
           "busy_frac": round(busy / (COMPUTE_UNITS * span), 4), "last_dispatch_us": round(last_start, 2),
           "tail_us": round(span - last_start, 2),
           "idle_after_last_dispatch_frac": round(idle_tail / (COMPUTE_UNITS * span), 4),
           "workgroup_end_us": {"p50": round(float(np.median(end)), 2), "p90": round(float(np.percentile(end, 90)), 2),
                                "max": round(span, 2)}}
    print(f"  compute units busy {100 * out['busy_frac']:.1f}% of the span; last workgroup dispatched at "
          f"{last_start:.1f} us; idle CU-time after it: {100 * out['idle_after_last_dispatch_frac']:.1f}% of the launch")
    print(f"  workgroup ends: p50 {out['workgroup_end_us']['p50']:.1f}  p90 {out['workgroup_end_us']['p90']:.1f}  "
          f"max {span:.1f} us")
    return out


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--config", type=int, default=2, choices=(1, 2, 3, 4))
    ap.add_argument("--pass", dest="which", choices=("full", "local"), default="full")
    ap.add_argument("--kv-dtype", choices=("bf16", "fp8"), default="bf16")
    ap.add_argument("--q-heads", type=int, default=None)
    ap.add_argument("--replays", type=int, default=5, help="graph replays timed by HIP events")
    args = ap.parse_args(argv)

    import torch

    lib = load_phases_lib()
    from . import binding as B
    from . import workloads as W
    from .state import DecodeState

    wl = W.config(args.config).with_(steps=4)
    if args.kv_dtype == "fp8":
        wl = wl.fp8()
    if args.q_heads is not None:
        wl = wl.with_(num_q_heads=args.q_heads)
    st = DecodeState(wl, gen_device="cuda")
    st.prefill()
    q = W.gen_queries(wl, "cuda")
    k_new, v_new = st.decode_inputs()
    Bn = wl.batch
    layers = [l for l in wl.gated_layers][:4] if args.which == "full" else list(range(min(4, wl.num_layers)))
    out = torch.empty((Bn, wl.num_q_heads, wl.head_dim), dtype=torch.float32, device="cuda")
    qs = [q[0, l].contiguous() for l in layers]
    ks = [k_new[0, l].contiguous() for l in layers]
    vs = [v_new[0, l].contiguous() for l in layers]
    fire = torch.ones(Bn + (-Bn) % 4, dtype=torch.float32, device="cuda")

    def launches():
        for i, l in enumerate(layers):
            if args.which == "full":
                B.decode_full_gated(st.dims, st.kv, l, Bn, qs[i], ks[i], vs[i], fire, 0.0, out, None, None, None,
                                    st.workspace)
            else:
                B.decode_local(st.dims, st.kv, l, Bn, qs[i], ks[i], vs[i], out, None, st.workspace)

    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            launches()
    torch.cuda.current_stream().wait_stream(s)
    g.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(args.replays):
        g.replay()
    e1.record()
    torch.cuda.synchronize()
    event_us = e0.elapsed_time(e1) * 1e3 / (args.replays * len(layers))
    if lib.oda_phase_stamps_clear() != 0:
        raise RuntimeError("oda_phase_stamps_clear failed")
    torch.cuda.synchronize()
    g.replay()
    torch.cuda.synchronize()
    if st.device_error() != 0:
        raise RuntimeError(f"device error word {st.device_error()}")
    groups = 65536
    stamps = np.zeros((groups, 8), dtype=np.uint64)
    xcc = np.zeros(groups, dtype=np.uint32)
    rc = lib.oda_phase_stamps_read(stamps.ctypes.data, xcc.ctypes.data, groups)
    if rc != 0:
        raise RuntimeError(f"oda_phase_stamps_read: HIP error {rc}")
    label = f"{wl.name} {args.which} pass"
    summarize(stamps, xcc, groups, event_us, label)
    return 0


if __name__ == "__main__":
    sys.exit(main())
