"""LCSA forward benchmark on one MI355X.

One step = one LCSA forward over one streaming chunk: lcsa_pool -> lcsa_score_select ->
lcsa_attn_fwd through the C ABI, inputs resident in HBM. Default workload: one 768x1408 streaming
chunk (2 query latent frames over 6, 12 heads, d = 128, bf16, 13.6% of blocks kept).

Prints one JSON line. `value` is the effective TFLOP/s on the selected blocks over the whole step
(sum over kept (head, i, j) pairs of 4*128*128*d FLOP / step time); `ms_per_step` is the time per
8-frame chunk. `roofline` is for the dominant kernel (lcsa_attn_fwd) against the dense bf16 MFMA
peak; its duration is measured with HIP events on the launch stream. `cpu_baseline` times the fp64
oracle on the host cores on the same workload.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
CSRC = os.path.join(ROOT, "block_sparse_causal_lcsa_amd", "csrc")
# the sources of the attention kernel whose HBM traffic the committed counter summary records
KERNEL_SRCS = ["attn_fwd_impl.h", "attn_fwd_block.hip", "attn_fwd.hip", "lcsa_geom.h"]


def kernel_hash() -> str:
    h = hashlib.sha256()
    for name in KERNEL_SRCS:
        with open(os.path.join(CSRC, name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def traffic_from_profile(workload: str):
    """HBM bytes per attn_fwd launch from the committed rocprofv3 counter summary, or None when
    the summary is missing or was taken on a different kernel source."""
    path = os.path.join(ROOT, "profiles", f"attn_fwd_{workload}_hbm_traffic.txt")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    h = re.search(r"kernel_source_sha256_16:\s*([0-9a-f]+)", text)
    t = re.search(r"hbm_bytes_per_launch:\s*([0-9.eE+]+)", text)
    if not h or not t or h.group(1) != kernel_hash():
        return None
    return float(t.group(1))


def mfma_busy_from_profile(workload: str):
    """SQ_VALU_MFMA_BUSY_CYCLES over the SIMD cycles of lcsa_attn_fwd from the committed rocprofv3 counter
    summary, or None when it is missing or was taken on different attention sources."""
    path = os.path.join(ROOT, "profiles", f"lcsa_forward_{workload}_counters.txt")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    h = re.search(r"attn_fwd \([^)]*\) ([0-9a-f]{16})", text)
    m = re.search(r"== lcsa_attn_fwd.*?SQ_VALU_MFMA_BUSY_CYCLES / [^=]*= ([0-9.]+)", text, re.S)
    if not h or not m or h.group(1) != kernel_hash():
        return None
    return float(m.group(1))


def cold_leg(reps, cold_pool, cold_sel, pool_bytes, sel_bytes):
    """The cold-cache figures, or None when the leg was skipped (--cold-reps 0)."""
    import numpy as np
    if not reps:
        return None
    mp, ms = float(np.median(cold_pool)), float(np.median(cold_sel))
    return {"flush": "read sweep of 1 GiB before each timed call", "reps": reps,
            "lcsa_pool_ms_median": round(mp, 4), "lcsa_score_select_ms_median": round(ms, 4),
            "pool_gbs_cold": round(pool_bytes / (mp * 1e-3) / 1e9, 1),
            "pool_frac_of_hbm_peak": round(pool_bytes / (mp * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
            "score_select_gbs_cold": round(sel_bytes / (ms * 1e-3) / 1e9, 1)}


def settle(run, seconds: float) -> float:
    """Untimed steps until at least `seconds` of wall time have passed (synchronising every 10 steps),
    so that clocks and caches reach their steady state whatever --warmup says. Returns the time spent."""
    import torch

    t0 = time.perf_counter()
    while True:
        for _ in range(10):
            run()
        torch.cuda.synchronize()
        dt = time.perf_counter() - t0
        if dt >= seconds:
            return dt


def pct(a, q: float) -> float:
    import numpy as np
    return round(float(np.percentile(np.asarray(a, dtype=np.float64), q)), 4)


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or "unknown"


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="chunk_768x1408_q2_kv6")
    ap.add_argument("--settle", type=float, default=1.5, metavar="SECONDS",
                    help="untimed steps for at least this wall time after the warmup steps, before any "
                         "timing (reported as settle_s)")
    ap.add_argument("--cold-reps", type=int, default=20,
                    help="repetitions of the cold-cache leg: pool and score_select each timed right after "
                         "a 1 GiB device write that evicts L2 and the Infinity Cache")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-sample-blocks", type=int, default=0,
                    help="query blocks per head in the oracle sample (0 = all)")
    ap.add_argument("--graph", action="store_true",
                    help="replay one captured HIP graph of the three calls per step instead of eager launches "
                         "(measured no faster on this path: the launches are already queued ahead)")
    ap.add_argument("--backward", action="store_true",
                    help="time lcsa_attn_bwd (gradients for the selection of one forward) instead of the "
                         "forward step; prints its own JSON line")
    ap.add_argument("--stream", type=int, default=0, metavar="CACHE",
                    help="time chunk-by-chunk streaming with a K/V cache of CACHE temporal blocks "
                         "(lcsa_stream_push + pool(q) + score_select + attn_fwd per chunk); prints its own JSON line")
    ap.add_argument("--layer", type=int, default=0, metavar="CACHE",
                    help="time a DiT self-attention layer with random weights around streaming LCSA "
                         "(QKV GEMM, 3D RoPE, stream push, pool/select/attention, output GEMM) per chunk, "
                         "cache of CACHE temporal blocks; prints its own JSON line with LCSA's share")
    ap.add_argument("--profile", action="store_true",
                    help="for rocprofv3 counter runs: warmup + `steps` steps, then one plain device copy "
                         "of 256 MiB (the byte-counter calibration kernel); prints a short line")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the LCSA forward here runs on a single MI355X, and "
              "sharding over several GPUs is not implemented (use --gpus 1).", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    from block_sparse_causal_lcsa_amd import inputs, lcsa
    from block_sparse_causal_lcsa_amd import workloads as W

    w = W.BY_NAME[args.workload]
    if args.stream:
        stream_bench(args, w)
        return
    if args.layer:
        layer_bench(args, w)
        return
    p = lcsa.problem(w)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    x = inputs.make_inputs(w, seed=0)

    def dev_t(a):
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(dev)
        return torch.from_numpy(a).to(dev)

    q, k, v = dev_t(x["q"]), dev_t(x["k"]), dev_t(x["v"])
    nqb, nkb, nnz, rp = lcsa.lcsa_csr_layout(p)
    row_ptr = torch.from_numpy(rp).to(dev)
    qp = torch.empty((w.batch, w.heads, nqb, w.head_dim), dtype=torch.float32, device=dev)
    kp = torch.empty((w.batch, w.heads, nkb, w.head_dim), dtype=torch.float32, device=dev)
    col = torch.empty((w.batch, w.heads, nnz), dtype=torch.int32, device=dev)
    o = torch.empty_like(q)
    lse = torch.empty((w.batch, w.heads, w.nq_tokens), dtype=torch.float32, device=dev)

    pairs = w.batch * w.heads * nnz
    flop = pairs * 4.0 * 128 * 128 * w.head_dim
    esz = 2 if w.dtype == "bf16" else 4
    pool_bytes = w.batch * w.heads * ((w.nq_tokens + w.nk_tokens) * w.head_dim * esz + (nqb + nkb) * w.head_dim * 4)
    sel_bytes = w.batch * w.heads * ((nqb + nkb) * w.head_dim * 4 + nnz * 4)

    def step(ev=None):
        # every call goes to the current stream (the capture stream while a graph is recorded)
        stream = torch.cuda.current_stream()
        if ev:
            ev[0].record(stream)
        lcsa.lcsa_pool(p, q, k, qp, kp, stream=stream)
        if ev:
            ev[1].record(stream)
        lcsa.lcsa_score_select(p, qp, kp, row_ptr, col, stream=stream)
        if ev:
            ev[2].record(stream)
        lcsa.lcsa_attn_fwd(p, q, k, v, row_ptr, col, o, lse, stream=stream)
        if ev:
            ev[3].record(stream)

    if args.backward:
        backward_bench(args, w, p, x, dev, step, dict(q=q, k=k, v=v, o=o, lse=lse, row_ptr=row_ptr, col=col, nnz=nnz))
        return

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    settle_s = settle(step, args.settle)

    # optionally, one step captured as a HIP graph and replayed
    run_step = step
    if args.graph and not args.profile:
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            step()
        torch.cuda.current_stream().wait_stream(side)
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            step()
        graph.replay()
        torch.cuda.synchronize()
        run_step = graph.replay

    if args.profile:
        for _ in range(args.steps):
            step()
        src = torch.empty(256 << 20, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        src.fill_(1)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        print(f"profile run: {args.steps} steps of {w.name}; calibration copy 268435456 bytes", flush=True)
        return

    # whole-step timing: K back-to-back steps between two synchronisations
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        run_step()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = wall * 1e3 / args.steps

    # per-kernel durations with HIP events on the launch stream (a second timed pass). It runs in
    # blocks of 25 steps with a synchronisation between blocks and one untimed step at the head of
    # each, so the launch queue never fills and no interval includes time the GPU spent waiting for
    # the host.
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
    for b0 in range(0, args.steps, 25):
        step()
        for e in evs[b0:b0 + 25]:
            step(e)
        torch.cuda.synchronize()
    t_pool = [e[0].elapsed_time(e[1]) for e in evs]
    t_sel = [e[1].elapsed_time(e[2]) for e in evs]
    t_attn = [e[2].elapsed_time(e[3]) for e in evs]
    t_step_ev = [e[0].elapsed_time(e[3]) for e in evs]
    med = lambda a: float(np.median(a))
    # mean launch duration; an interval above 3x the median holds time the GPU sat idle waiting for a
    # stalled host (seen once in 200 as a 35 ms gap), not kernel time: such intervals are dropped and
    # counted
    ta = np.array(t_attn)
    keep = ta <= 3.0 * np.median(ta)
    attn_ms = float(np.mean(ta[keep]))
    achieved = flop / (attn_ms * 1e-3) / 1e12
    traffic = traffic_from_profile(w.name)

    # cold-cache leg: each pool and each score_select is timed right after a read sweep over a 1 GiB
    # buffer (written once, before the leg), which evicts the 4 MB L2s and the 256 MB Infinity Cache
    # without leaving dirty lines whose write-back would share HBM with the timed kernel; the bytes
    # the timed kernel reads come from HBM
    flush = torch.ones(1 << 28, dtype=torch.int32, device=dev)
    torch.cuda.synchronize()
    cold_pool, cold_sel = [], []
    stream = torch.cuda.current_stream()
    for _ in range(args.cold_reps):
        e = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
        flush.sum()
        e[0].record(stream)
        lcsa.lcsa_pool(p, q, k, qp, kp, stream=stream)
        e[1].record(stream)
        flush.sum()
        e[2].record(stream)
        lcsa.lcsa_score_select(p, qp, kp, row_ptr, col, stream=stream)
        e[3].record(stream)
        torch.cuda.synchronize()
        cold_pool.append(e[0].elapsed_time(e[1]))
        cold_sel.append(e[2].elapsed_time(e[3]))
    del flush

    # matrix-core probe: the dense bf16 MFMA rate this GPU sustains right now (every CU busy), beside
    # which the attention kernel's rate is also given; the roofline's peak stays the published one
    probe_wgs, probe_iters = 2048, 1000
    sink = torch.empty(probe_wgs * 256, dtype=torch.float32, device=dev)
    probe_ms, probe_flop = [], 0.0
    for _ in range(6):
        e = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        e[0].record(stream)
        probe_flop = lcsa.lcsa_mfma_probe(probe_wgs, probe_iters, sink, stream=stream)
        e[1].record(stream)
        torch.cuda.synchronize()
        probe_ms.append(e[0].elapsed_time(e[1]))
    probe_tflops = probe_flop / (float(np.median(probe_ms[1:])) * 1e-3) / 1e12
    del sink

    out = {
        "metric": "LCSA fwd effective TFLOP/s on selected blocks + ms per 8-frame chunk",
        "value": round(flop / (ms_per_step * 1e-3) / 1e12, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if w.dtype == "bf16" else "f32",
        "data": "synthetic: seeded smooth sinusoidal Q/K fields + 0.5 N(0,1), V ~ N(0,1)",
        "config": {"workload": w.name, "batch": w.batch, "heads": w.heads, "head_dim": w.head_dim,
                   "grid": [w.grid_h, w.grid_w], "q_frames": [w.q_frame0, w.q_frame0 + w.q_frames],
                   "kv_frames": w.kv_frames, "keep_ratio": w.keep_ratio if not w.topk else None,
                   "topk": w.topk or None, "window": ["none", "truncated", "preserving"][w.win_mode],
                   "selected_pairs": pairs, "selected_gflop": round(flop / 1e9, 2)},
        "ms_per_chunk": round(ms_per_step, 4),
        "launch": "eager" if run_step is step else "hip_graph",
        "settle_s": round(settle_s, 2),
        "kernels_ms_median": {"lcsa_pool": round(med(t_pool), 4), "lcsa_score_select": round(med(t_sel), 4),
                              "lcsa_attn_fwd": round(med(t_attn), 4), "step_events": round(med(t_step_ev), 4)},
        "kernels_ms_p10": {"lcsa_pool": pct(t_pool, 10), "lcsa_score_select": pct(t_sel, 10),
                           "lcsa_attn_fwd": pct(t_attn, 10), "step_events": pct(t_step_ev, 10)},
        "kernels_ms_p90": {"lcsa_pool": pct(t_pool, 90), "lcsa_score_select": pct(t_sel, 90),
                           "lcsa_attn_fwd": pct(t_attn, 90), "step_events": pct(t_step_ev, 90)},
        "pool_gbs": round(pool_bytes / (med(t_pool) * 1e-3) / 1e9, 1),
        "score_select_gbs": round(sel_bytes / (med(t_sel) * 1e-3) / 1e9, 1),
        "cold_cache": cold_leg(args.cold_reps, cold_pool, cold_sel, pool_bytes, sel_bytes),
        "mfma_probe": {"tflops": round(probe_tflops, 1), "frac_of_spec_peak": round(probe_tflops / PEAK_BF16_TFLOPS, 4),
                       "workgroups": probe_wgs, "iters": probe_iters,
                       "what": "back-to-back v_mfma_f32_32x32x16_bf16, operands in registers, workgroups of 4 waves"},
        "roofline": {"bound": "mfma", "kernel": "lcsa_attn_fwd", "achieved": round(achieved, 2),
                     "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                     "traffic": traffic, "flop_per_launch": flop, "avg_launch_ms": round(attn_ms, 4),
                     "mfma_busy": mfma_busy_from_profile(w.name),
                     "frac_of_probe": round(achieved / probe_tflops, 4),
                     "event_intervals": int(ta.size), "event_outliers_dropped": int((~keep).sum())},
    }

    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(w, x, args.cpu_sample_blocks)
    print(json.dumps(out), flush=True)


def backward_bench(args, w, p, x, dev, step, t):
    """Times lcsa_attn_bwd on the selection, O and lse of one forward step (inputs resident in HBM).
    FLOP per kept (head, i, j) pair: 5 products of 128 x 128 x d (S recomputed, dP, dV, dK, dQ), the
    usual convention for attention backward; the kernels execute 7 (S and dP once in each of the dQ
    and dK/dV kernels), reported as executed_tflops."""
    import numpy as np
    import torch

    from block_sparse_causal_lcsa_amd import inputs, lcsa

    step()
    g = inputs.make_grad(w, seed=0)
    d_o = torch.from_numpy(g.view(np.int16)).view(torch.bfloat16).to(dev)
    ws = torch.empty(lcsa.lcsa_attn_bwd_workspace_size(p), dtype=torch.uint8, device=dev)
    hw = w.grid_h * w.grid_w
    dq = torch.empty((w.batch, w.heads, w.q_frames * hw, w.head_dim), dtype=torch.float32, device=dev)
    dk = torch.empty((w.batch, w.heads, w.kv_frames * hw, w.head_dim), dtype=torch.float32, device=dev)
    dv = torch.empty_like(dk)

    def bwd():
        lcsa.lcsa_attn_bwd(p, t["q"], t["k"], t["v"], t["o"], d_o, t["lse"], t["row_ptr"], t["col"], dq, dk, dv,
                           workspace=ws, stream=torch.cuda.current_stream())

    for _ in range(args.warmup):
        bwd()
    torch.cuda.synchronize()
    settle_s = settle(bwd, args.settle)
    t0 = time.perf_counter()
    for _ in range(args.steps):
        bwd()
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / args.steps
    stream = torch.cuda.current_stream()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    for e0, e1 in evs:
        e0.record(stream)
        bwd()
        e1.record(stream)
    torch.cuda.synchronize()
    call_t = [e0.elapsed_time(e1) for e0, e1 in evs]
    call_ms = float(np.mean(call_t))
    pairs = w.batch * w.heads * t["nnz"]
    flop = pairs * 10.0 * 128 * 128 * w.head_dim
    executed = pairs * 14.0 * 128 * 128 * w.head_dim
    out = {
        "metric": "LCSA attention backward effective TFLOP/s on selected blocks (5 GEMMs per kept pair)",
        "value": round(flop / (ms * 1e-3) / 1e12, 2),
        "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic: the forward's inputs; dO ~ N(0,1) rounded to bf16",
        "settle_s": round(settle_s, 2),
        "call_ms": {"p10": pct(call_t, 10), "median": pct(call_t, 50), "p90": pct(call_t, 90)},
        "config": {"workload": w.name, "batch": w.batch, "heads": w.heads, "head_dim": w.head_dim,
                   "grid": [w.grid_h, w.grid_w], "selected_pairs": pairs},
        "roofline": {"bound": "mfma", "kernel": "lcsa_attn_bwd (delta, csc, dq, dkdv launches)",
                     "achieved": round(executed / (call_ms * 1e-3) / 1e12, 2), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(executed / (call_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
                     "traffic": None, "flop_per_launch": executed, "avg_launch_ms": round(call_ms, 4)},
    }
    print(json.dumps(out), flush=True)


def stream_bench(args, w):
    """Steady-state chunk time of streaming LCSA at the workload's frame size, heads and keep ratio:
    a sequence of 8 temporal blocks resident in HBM is streamed through a cache of args.stream blocks
    (cycling), every chunk = lcsa_stream_push(K, V of the new block) + lcsa_pool(q) + lcsa_score_select
    + lcsa_attn_fwd on the cache window. Timing starts once the cache is full."""
    import numpy as np
    import torch

    from block_sparse_causal_lcsa_amd import inputs, lcsa

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    nblk = 8
    seq = w.replace(kv_frames=2 * nblk, q_frame0=0, q_frames=2 * nblk)
    chunk = w.replace(kv_frames=2, q_frame0=0, q_frames=2)
    x = inputs.make_inputs(seq, seed=0)
    q, k, v = (torch.from_numpy(x[n].view(np.int16)).view(torch.bfloat16).to(dev) for n in "qkv")
    del x
    tbt = 2 * w.grid_h * w.grid_w
    views = [(q[:, :, c * tbt:(c + 1) * tbt], k[:, :, c * tbt:(c + 1) * tbt], v[:, :, c * tbt:(c + 1) * tbt])
             for c in range(nblk)]
    s = lcsa.Stream(lcsa.problem(chunk), args.stream)

    def one(c, ev=None):
        qc, kc, vc = views[c % nblk]
        stream = torch.cuda.current_stream()
        if ev:
            ev[0].record(stream)
        s.push(kc, vc, stream=stream)
        if ev:
            ev[1].record(stream)
        out = s.forward(qc, stream=stream)
        if ev:
            ev[2].record(stream)
        return out

    c = 0
    for _ in range(max(args.warmup, args.stream)):
        one(c)
        c += 1
    torch.cuda.synchronize()

    def one_next():
        nonlocal c
        one(c)
        c += 1

    settle_s = settle(one_next, args.settle)
    t0 = time.perf_counter()
    for _ in range(args.steps):
        out = one(c)
        c += 1
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / args.steps
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    for e in evs:
        out = one(c, e)
        c += 1
    torch.cuda.synchronize()
    push_ms = float(np.median([e[0].elapsed_time(e[1]) for e in evs]))
    fwd_ms = float(np.median([e[1].elapsed_time(e[2]) for e in evs]))
    pw = out["problem"]
    nnz = int(out["row_ptr"][-1])
    flop = w.batch * w.heads * nnz * 4.0 * 128 * 128 * w.head_dim
    res = {
        "metric": "LCSA streaming ms per chunk (push K/V + pool q + score_select + attn_fwd), cache full",
        "value": round(ms, 4), "unit": "ms", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms, 4), "higher_is_better": False, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic: seeded smooth sinusoidal Q/K fields + 0.5 N(0,1), V ~ N(0,1)",
        "settle_s": round(settle_s, 2),
        "config": {"workload": f"{w.name} streamed, cache {args.stream} temporal blocks", "heads": w.heads,
                   "head_dim": w.head_dim, "grid": [w.grid_h, w.grid_w], "window_kv_frames": pw.kv_frames},
        "kernels_ms_median": {"lcsa_stream_push": round(push_ms, 4), "pool_select_attn": round(fwd_ms, 4)},
        "attention_tflops_per_chunk": round(flop / (ms * 1e-3) / 1e12, 2),
    }
    print(json.dumps(res), flush=True)


def layer_bench(args, w):
    """Steady-state chunk time of DitLcsaLayer (random weights, C = heads * head_dim) at the workload's
    frame size, with per-stage HIP-event times and LCSA's share (stream push + pool/select/attention)
    of the layer."""
    import numpy as np
    import torch

    from block_sparse_causal_lcsa_amd import lcsa
    from block_sparse_causal_lcsa_amd.layer import DitLcsaLayer

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    chunk = w.replace(kv_frames=2, q_frame0=0, q_frames=2)
    layer = DitLcsaLayer(lcsa.problem(chunk), args.layer, seed=0, device=dev)
    N, C = 2 * w.grid_h * w.grid_w, w.heads * w.head_dim
    g = torch.Generator(device="cpu").manual_seed(1)
    xs = [torch.randn(w.batch, N, C, generator=g).to(torch.bfloat16).to(dev) for _ in range(4)]
    c = 0
    for _ in range(max(args.warmup, args.layer)):
        layer.step(xs[c % 4])
        c += 1
    torch.cuda.synchronize()

    def one_next():
        nonlocal c
        layer.step(xs[c % 4])
        c += 1

    settle_s = settle(one_next, args.settle)
    t0 = time.perf_counter()
    for _ in range(args.steps):
        layer.step(xs[c % 4])
        c += 1
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / args.steps
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(6)] for _ in range(args.steps)]
    for e in evs:
        _, res = layer.step(xs[c % 4], timing=e)
        c += 1
    torch.cuda.synchronize()
    names = ["qkv_gemm", "rope_qkv", "stream_push", "pool_select_attn", "out_gemm"]
    med = {n: float(np.median([e[i].elapsed_time(e[i + 1]) for e in evs])) for i, n in enumerate(names)}
    tot = float(np.median([e[0].elapsed_time(e[5]) for e in evs]))
    lcsa_ms = med["stream_push"] + med["pool_select_attn"]
    nnz = int(res["row_ptr"][-1])
    gemm_flop = 2.0 * w.batch * N * C * 4 * C
    res_out = {
        "metric": "DiT attention layer ms per chunk with streaming LCSA (random weights), LCSA share",
        "value": round(ms, 4), "unit": "ms", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms, 4), "higher_is_better": False, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic: x ~ N(0,1), weights ~ N(0, 1/C), bf16", "settle_s": round(settle_s, 2),
        "config": {"workload": f"{w.name} as a DiT layer, cache {args.layer} temporal blocks", "heads": w.heads,
                   "head_dim": w.head_dim, "model_dim": C, "tokens_per_chunk": N, "rope_dims": [44, 42, 42],
                   "selected_pairs": w.batch * w.heads * nnz},
        "stages_ms_median": {k: round(v, 4) for k, v in med.items()},
        "layer_events_ms": round(tot, 4),
        "lcsa_share": round(lcsa_ms / tot, 4),
        "gemm_tflops": round(gemm_flop / ((med["qkv_gemm"] + med["out_gemm"]) * 1e-3) / 1e12, 1),
        "rope_gbs": round(2 * w.batch * N * 3 * C * 2 / (med["rope_qkv"] * 1e-3) / 1e9, 1),
    }
    print(json.dumps(res_out), flush=True)


def cpu_baseline(w, x, sample_blocks):
    """The fp64 oracle, unchanged, on this host: pool + score + select over the whole chunk and
    exact attention over a sample of query blocks (every head), scaled to TFLOP/s on the selected
    blocks it computed."""
    import numpy as np
    from threadpoolctl import threadpool_info

    from block_sparse_causal_lcsa_amd import inputs
    from oracle import lcsa_oracle as O

    q64, k64, v64 = (inputs.to_f64(x[n]) for n in "qkv")
    nqb = w.nqb
    qblocks = list(range(nqb)) if sample_blocks <= 0 else list(np.linspace(0, nqb - 1, sample_blocks).astype(int))
    times = []
    for _ in range(3):
        t0 = time.perf_counter()
        vis = O.visible(w)
        qbar, kbar = O.pool(w, q64, "q"), O.pool(w, k64, "k")
        s = O.block_scores(w, qbar, kbar, vis)
        rp, col = O.select(w, s, vis)
        O.attend(w, q64, k64, v64, rp, col, qblocks=qblocks)
        times.append(time.perf_counter() - t0)
    dt = float(np.median(times))
    kept = sum(int(rp[i + 1] - rp[i]) for i in qblocks) * w.batch * w.heads
    flop = kept * 4.0 * 128 * 128 * w.head_dim
    blas = [t for t in threadpool_info() if t.get("user_api") == "blas"]
    cores = max([t.get("num_threads", 1) for t in blas] or [1])
    vendor = ", ".join(sorted({f"{t.get('internal_api')} {t.get('version')}" for t in blas})) or "unknown"
    return {"value": round(flop / dt / 1e12, 5), "unit": "TFLOP/s", "cores": cores, "kind": "oracle",
            "seconds": round(dt, 2), "cpu_model": cpu_model(), "blas": vendor,
            "host_cpus_visible": len(os.sched_getaffinity(0)),
            "sample": f"median of 3 runs; {w.name}: pool+score+select of all {nqb} query blocks, attention of "
                      f"{len(qblocks)} query blocks x {w.batch * w.heads} heads ({kept} kept pairs); "
                      f"numpy fp64, BLAS threads={cores}, elementwise single-threaded"}


if __name__ == "__main__":
    main()
