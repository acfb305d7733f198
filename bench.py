"""Throughput of the masked second-order HLA forward on one MI355X.

  python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--no-cpu-baseline]

A step is one pass of the chunk-parallel forward over the whole workload:
segment summaries -> exclusive Blelloch scan -> outputs (three C-ABI calls
on one stream; inputs already resident in HBM).  The decode workload times
one streaming decode step for every (sequence, head); the unmasked_* and
ahla_* workloads time the two further operators' calls on the same shapes;
the bwd_* workload times the backward pass (one hla_bwd call).
Prints one JSON line.
"""

import argparse
import ctypes
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "HLA fwd tokens/s (B·H·T/s) at 1 MI355X; % MFMA peak (chunk) / % HBM peak (decode)"
HBM_PEAK_GBS = 8000.0
BF16_PEAK_TFLOPS = 2500.0
DEFAULT_WORKLOAD = "fwd_decay_bf16_b4h16t16384d128"
BWD_WORKLOAD = "bwd_decay_bf16_b4h16t16384d128"
BWD_CHUNK = 2048          # segment length of the backward's first-order sums
BWD_TILE = 64             # tokens per tile of its kernels (bf16 inputs)
HLA3_WORKLOAD = "hla3_decay_bf16_b4h16t16384d128"
HLA3_CHUNK = 2048         # segment length of the third-order forward


def credited_flops_per_token(c, d, dv):
    """Credited (algorithmic) flops per token of the masked chunk algorithm at
    chunk length c: exact multiply-adds x 2 with triangles and the symmetry of
    K^T K exploited, one combine per chunk."""
    f = (c * d * (d + 1) + 2 * c * d * dv + 2 * c * c * d + c * (c - 1) * dv + 2 * c * d * dv
         + 2 * d * d * dv + 2 * c * d * d + c * (c + 1) * d + c * (c + 1) * (c + 2) / 3
         + c * (c + 1) * dv + min(2 * d * d * dv + 2 * c * d * dv, 4 * c * d * dv))
    return f / c


def credited_flops_per_token_unmasked(c, d, dv):
    """Credited flops per token of the unmasked variant at chunk length c:
    K^T K (symmetric) and Q^T V, Q S_P, the lower triangles of Q K^T, A' K,
    P Q^T and B V, and P C_P; the combine has no cross term."""
    f = (c * d * (d + 1) + 2 * c * d * dv + 2 * c * d * d + 3 * c * (c + 1) * d
         + c * (c + 1) * dv + 2 * c * d * dv)
    return f / c


def credited_flops_per_token_ahla(c, d, dv):
    """Credited flops per token of AHLA at chunk length c: the lower triangles
    of Q K^T, A' V and A' R, the products Q P, Q E, K^T V, K^T R, the segment
    moment X = K^T Q, and one combine per chunk (X_B P_A)."""
    f = (c * (c + 1) * d + 2 * c * (c + 1) * dv + 8 * c * d * dv + 2 * c * d * d
         + 2 * d * d * dv)
    return f / c


def measured_traffic(key):
    """HBM bytes per launch measured with rocprofv3 counters for `key`, or None
    if the kernel's sources changed since the counters were taken."""
    import hashlib
    path = os.path.join(ROOT, "profiles", "hbm_traffic.json")
    try:
        entry = json.load(open(path))["kernels"][key]
    except (OSError, KeyError, ValueError):
        return None
    m = hashlib.sha256()
    for f in entry["sources"]:
        m.update(open(os.path.join(ROOT, "causal_prefix_scan_amd", "csrc", f), "rb").read())
    return entry["traffic_bytes"] if m.hexdigest() == entry["source_sha256"] else None


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    # 50 warm-up steps: the GPU leaves its idle clock state during the first
    # tens of milliseconds of work, and 20 steps of 0.6 ms would be timed inside
    # that ramp (measured: 0.69 against 0.60 ms per forward step)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--chunk", type=int, default=0, help="override the segment length")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-tokens", type=int, default=3072,
                    help="tokens per unit in the oracle sample (forward workloads)")
    ap.add_argument("--cpu-steps", type=int, default=40,
                    help="decode steps in the oracle sample (decode workload)")
    return ap.parse_args()


# Per-call HIP events are recorded on every KERNEL_EVENT_EVERY-th timed step
# only: each record is a marker in the stream that costs a few microseconds,
# which the step time would otherwise carry (14 us of a 65 us step at B2 H8
# T4096 d64; still 1.5 us per step on average with every 10th step sampled).
# The step time comes from one event pair around all timed steps.
KERNEL_EVENT_EVERY = 25


def timing_events(torch, steps):
    """Start and end events of the timed region, and the four per-call events
    of the sampled steps (a dict by step index)."""
    E = lambda: torch.cuda.Event(enable_timing=True)
    sampled = [i for i in range(steps) if i % KERNEL_EVENT_EVERY == KERNEL_EVENT_EVERY // 2] or [steps // 2]
    return E(), E(), {i: [E() for _ in range(4)] for i in sampled}


def cpu_threads():
    """Threads the oracle may use: this process's CPU affinity, capped by the
    host's thread budget for the job (OMP_NUM_THREADS when set)."""
    n = len(os.sched_getaffinity(0))
    cap = os.environ.get("OMP_NUM_THREADS")
    if cap and cap.isdigit() and int(cap) > 0:
        n = min(n, int(cap))
    return max(n, 1)


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline_fwd(inp, ntok):
    """The oracle's serial recurrence on a bounded sample: every unit, first ntok tokens."""
    import numpy as np
    from threadpoolctl import threadpool_limits
    from oracle import hla_oracle as O
    uq, uk, uv, ug = inp.units()
    nt = cpu_threads()
    with threadpool_limits(limits=nt):
        t0 = time.perf_counter()
        O.serial(uq[:, :ntok], uk[:, :ntok], uv[:, :ntok], ug)
        dt = time.perf_counter() - t0
    U = uq.shape[0]
    return {"value": U * ntok / dt, "unit": "tokens/s", "cores": nt, "kind": "oracle",
            "sample": f"fp64 serial recurrence, all {U} (batch, head) units, first {ntok} of "
                      f"{uq.shape[1]} tokens ({dt:.1f} s)", "seconds": round(dt, 2),
            "cpu_model": cpu_model()}


def cpu_baseline_decode(states64, toks, steps):
    from threadpoolctl import threadpool_limits
    from oracle import hla_oracle as O
    U = toks[0][0].shape[0]
    nt = cpu_threads()
    with threadpool_limits(limits=nt):
        t0 = time.perf_counter()
        st = states64
        for s in range(steps):
            _, _, st = O.decode_step(st, *toks[s])
        dt = time.perf_counter() - t0
    return {"value": U * steps / dt, "unit": "unit-tokens/s", "cores": nt, "kind": "oracle",
            "sample": f"fp64 decode steps, {U} units x {steps} steps ({dt:.1f} s)",
            "seconds": round(dt, 2), "cpu_model": cpu_model()}


def bench_fwd(args, torch, np):
    from causal_prefix_scan_amd import hla, synth
    cfg = dict(synth.FWD_WORKLOADS[args.workload])
    if args.chunk:
        cfg["chunk"] = args.chunk
    B, H, T, d, dv, chunk = (cfg[x] for x in ("B", "H", "T", "d", "dv", "chunk"))
    inp = synth.make_fwd_inputs(B, H, T, d, dv, cfg["dtype"], cfg["seed"],
                                k_l2norm=cfg["k_l2norm"], decay=cfg["decay"])
    if cfg["dtype"] == "bf16":
        cv = lambda b: torch.from_numpy(b.view(np.int16)).view(torch.bfloat16).cuda()
        q, k, v = cv(inp.q_bits), cv(inp.k_bits), cv(inp.v_bits)
    else:
        q, k, v = (torch.from_numpy(x).cuda() for x in (inp.q, inp.k, inp.v))
    g = None if inp.gamma is None else torch.from_numpy(inp.gamma).cuda()
    dcode = hla.HLA_BF16 if cfg["dtype"] == "bf16" else hla.HLA_F32
    L = hla.lib()
    # hla_fwd's plan: each workgroup walks a span of R chunks (forming and
    # combining their summaries in order), the scan runs over the span totals
    # (out of place), and the outputs walk each span from its prefix
    p0 = hla.make_problem(q, v, chunk, g, cfg["normalize"], cfg["eps"])
    R = L.hla_fwd_span_chunks(ctypes.byref(p0))
    span = chunk * R
    n = T // span
    summ = hla.alloc_state((B, H, n), d, dv, "cuda")
    o = torch.empty(B, H, T, dv, dtype=torch.float32, device="cuda")
    den = torch.empty(B, H, T, dtype=torch.float32, device="cuda") if cfg["normalize"] else None
    p = hla.make_problem(q, v, span, g, cfg["normalize"], cfg["eps"])
    st = hla._state_struct(summ)
    ws_bytes = L.hla_scan_workspace_bytes(ctypes.byref(p))
    ws = torch.empty(max(ws_bytes, 16), dtype=torch.uint8, device="cuda")
    # the shapes that have it (bf16, d = dv = 128) take hla_fwd's segment-local
    # p path: the summary kernel also writes p = S q, the outputs come from it
    p_bytes = L.hla_fwd_p_bytes(ctypes.byref(p))
    plocal = torch.empty(max(p_bytes, 16), dtype=torch.uint8, device="cuda") if p_bytes else None
    name_s = "hla_fwd_chunk_summaries_p" if p_bytes else "hla_fwd_chunk_summaries"
    name_o = "hla_fwd_output_from_p" if p_bytes else "hla_fwd_output"
    stream = torch.cuda.current_stream()
    sp = ctypes.c_void_p(stream.cuda_stream)
    ptr = lambda t: None if t is None else ctypes.c_void_p(t.data_ptr())
    # the scan out of place, as hla_fwd's fastest plan runs it: the rescan
    # writes every prefix itself (no separate C, m pass)
    pre = hla.alloc_state((B, H, n), d, dv, "cuda")
    st_pre = hla._state_struct(pre)
    name_scan = "hla_scan_into"

    def step(ev=None):
        if ev:
            ev[0].record(stream)
        if p_bytes:
            r1 = L.hla_fwd_chunk_summaries_p(ctypes.byref(p), ptr(q), ptr(k), ptr(v), ctypes.byref(st),
                                             ptr(plocal), sp)
        else:
            r1 = L.hla_fwd_chunk_summaries(ctypes.byref(p), ptr(q), ptr(k), ptr(v), ctypes.byref(st), sp)
        if ev:
            ev[1].record(stream)
        r2 = L.hla_scan_into(ctypes.byref(p), ctypes.byref(st), ctypes.byref(st_pre), None, ptr(ws),
                             ctypes.c_size_t(ws_bytes), sp)
        if ev:
            ev[2].record(stream)
        if p_bytes:
            r3 = L.hla_fwd_output_from_p(ctypes.byref(p), ptr(q), ptr(v), ptr(plocal), ctypes.byref(st_pre),
                                         ptr(o), ptr(den), sp)
        else:
            r3 = L.hla_fwd_output(ctypes.byref(p), ptr(q), ptr(k), ptr(v), ctypes.byref(st_pre), ptr(o),
                                  ptr(den), None, ctypes.c_size_t(0), sp)
        if ev:
            ev[3].record(stream)
        if r1 or r2 or r3:
            raise RuntimeError(f"HLA call failed: {r1} {r2} {r3}")

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    e0, e1, evs = timing_events(torch, args.steps)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    e0.record(stream)
    for i in range(args.steps):
        step(evs.get(i))
    e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    k1 = [e[0].elapsed_time(e[1]) for e in evs.values()]
    k2 = [e[1].elapsed_time(e[2]) for e in evs.values()]
    k3 = [e[2].elapsed_time(e[3]) for e in evs.values()]
    step_ms = e0.elapsed_time(e1) / args.steps
    tokens = B * H * T
    value = tokens / (step_ms / 1e3)

    U = B * H
    es = 2 if cfg["dtype"] == "bf16" else 4
    summ_bytes = U * n * (d * d + 2 * d * dv + 2 * d) * 4
    prefix_bytes = summ_bytes                                    # prefixes the output kernel reads
    io_bytes = tokens * ((2 * d + dv) * es)
    # the segment-local p: written by the summaries, read by the outputs in
    # place of k (bf16, 64-token tiles)
    kernels = {
        name_s: dict(ms=sum(k1) / len(k1), bytes=io_bytes + summ_bytes + p_bytes),
        name_scan: dict(ms=sum(k2) / len(k2), bytes=None),
        name_o: dict(ms=sum(k3) / len(k3),
                     bytes=io_bytes - (tokens * d * es if p_bytes else 0) + p_bytes + prefix_bytes
                     + tokens * dv * 4 + (tokens * 4 if den is not None else 0)),
    }
    dom = max((name_s, name_o), key=lambda kname: kernels[kname]["ms"])
    kd = kernels[dom]
    achieved = kd["bytes"] / (kd["ms"] / 1e3) / 1e9
    f_tok = credited_flops_per_token(cfg["credit_chunk"], d, dv)
    roofline = {"bound": "hbm", "kernel": dom, "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                "traffic": measured_traffic(f"{dom}@{args.workload}") if not args.chunk else None,
                "bytes_per_launch": kd["bytes"], "avg_launch_ms": round(kd["ms"], 4)}
    out = {
        "metric": METRIC, "value": round(value, 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(step_ms, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": cfg["dtype"], "data": "synthetic",
        "config": {"workload": args.workload, "B": B, "H": H, "T": T, "d": d, "dv": dv,
                   "chunk": chunk, "span_chunks": R, "decay": cfg["decay"],
                   "normalize": cfg["normalize"],
                   "path": (f"hla_fwd's plan: {name_s} over spans of {R} chunk(s) "
                            f"({span} tokens; each workgroup forms its chunks' summaries and "
                            f"combines them in order), {name_scan} over the {n} span totals per "
                            f"(b, h), {name_o} walking each span from its prefix")},
        "mfma_credited": {"flops_per_token": round(f_tok), "credit_chunk": cfg["credit_chunk"],
                          "tflops": round(value * f_tok / 1e12, 1),
                          "peak_tflops": BF16_PEAK_TFLOPS,
                          "frac": round(value * f_tok / 1e12 / BF16_PEAK_TFLOPS, 4)},
        "kernels_ms": {kname: round(kv["ms"], 4) for kname, kv in kernels.items()},
        "wall_ms_per_step": round(wall * 1e3 / args.steps, 4),
        "kernel_events": f"per-call HIP events on {len(evs)} of the {args.steps} timed steps",
        "roofline": roofline,
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline_fwd(inp, min(args.cpu_tokens, T))
    return out


def bench_decode(args, torch, np):
    from causal_prefix_scan_amd import hla, synth
    name, cfg = synth.DECODE_WORKLOAD
    Nq, H, d, dv, P, seed = (cfg[x] for x in ("n_seq", "H", "d", "dv", "prefix_len", "seed"))
    U = Nq * H
    steps = args.steps
    # prefill on the GPU: one segment summary of the 2048-token prefix is the
    # state after the prefix (hla_fwd with chunk = prefix length)
    pre = synth.make_fwd_inputs(Nq, H, P, d, dv, "bf16", seed)
    cv = lambda b: torch.from_numpy(np.ascontiguousarray(b).view(np.int16)).view(torch.bfloat16).cuda()
    pq, pk, pv = cv(pre.q_bits), cv(pre.k_bits), cv(pre.v_bits)
    _, _, state = hla.fwd(pq, pk, pv, P, None, want_state=True)
    del pq, pk, pv
    n_tok = args.warmup + steps
    toks_host = [synth.make_decode_step(Nq, H, d, dv, seed, s) for s in range(n_tok)]
    tq = torch.stack([cv(t[3][0]).reshape(Nq, H, d) for t in toks_host])
    tk = torch.stack([cv(t[3][1]).reshape(Nq, H, d) for t in toks_host])
    tv = torch.stack([cv(t[3][2]).reshape(Nq, H, dv) for t in toks_host])
    o = torch.empty(Nq, H, dv, dtype=torch.float32, device="cuda")
    den = torch.empty(Nq, H, dtype=torch.float32, device="cuda")
    states64 = None
    if not args.no_cpu_baseline:
        states64 = {key: val.double().cpu().numpy().reshape(U, *val.shape[2:])
                    for key, val in state.items()}
    for s in range(args.warmup):
        hla.decode_step(tq[s], tk[s], tv[s], state, None, True, cfg["eps"], o=o, den=den)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record(stream)
    for s in range(args.warmup, n_tok):
        hla.decode_step(tq[s], tk[s], tv[s], state, None, True, cfg["eps"], o=o, den=den)
    e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    step_ms = e0.elapsed_time(e1) / steps
    value = U / (step_ms / 1e3)
    state_bytes = (d * d + 2 * d * dv + 2 * d) * 4
    bytes_step = U * (2 * state_bytes + (2 * d + dv) * 2 + dv * 4 + 4)
    achieved = bytes_step / (step_ms / 1e3) / 1e9
    out = {
        "metric": METRIC, "value": round(value, 1), "unit": "unit-tokens/s", "n_gpus": 1,
        "steps": steps, "warmup": args.warmup, "ms_per_step": round(step_ms, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": name, "n_seq": Nq, "H": H, "d": d, "dv": dv, "prefix_len": P,
                   "normalize": True, "path": "hla_decode_step"},
        "wall_ms_per_step": round(wall * 1e3 / steps, 4),
        "roofline": {"bound": "hbm", "kernel": "hla_decode_step", "achieved": round(achieved, 1),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": measured_traffic(f"hla_decode_step@{name}"), "bytes_per_launch": bytes_step,
                     "avg_launch_ms": round(step_ms, 4)},
    }
    if states64 is not None:
        nb = min(args.cpu_steps, len(toks_host))
        toks = [(t[0], t[1], t[2]) for t in toks_host[:nb]]
        out["cpu_baseline"] = cpu_baseline_decode(states64, toks, nb)
    return out


# The two further operators on the same machinery: segment summaries, scan and
# outputs through three C-ABI calls named <prefix>_chunk_summaries, _scan and
# _output, and a decode step.
def _variants():
    from causal_prefix_scan_amd import hla
    return {
        "unmasked": dict(
            prefix="hla_unmasked", keys=("S", "C", "m"), oracle="serial_unmasked",
            alloc=hla.alloc_moments, struct=hla._state_struct,
            summaries=hla.unmasked_chunk_summaries, decode=hla.unmasked_decode_step,
            summary_floats=lambda d, dv: d * d + d * dv + d,
            prefix_floats=lambda d, dv: d * d + d * dv + d,
            flops=credited_flops_per_token_unmasked, name="unmasked variant"),
        "ahla": dict(
            prefix="hla_ahla", keys=("P", "m", "E", "n"), oracle="serial_ahla",
            alloc=hla.alloc_ahla_state, struct=hla._ahla_struct,
            summaries=hla.ahla_chunk_summaries, decode=hla.ahla_decode_step,
            summary_floats=lambda d, dv: 2 * d * dv + 2 * d + d * d,
            prefix_floats=lambda d, dv: 2 * d * dv + 2 * d,
            flops=credited_flops_per_token_ahla, name="AHLA"),
    }


# variant workloads: name -> (variant, forward inputs they run on)
VARIANT_FWD = {"unmasked_decay_bf16_b4h16t16384d128": ("unmasked", "fwd_decay_bf16_b4h16t16384d128"),
               "ahla_decay_bf16_b4h16t16384d128": ("ahla", "fwd_decay_bf16_b4h16t16384d128")}
VARIANT_DECODE = {"unmasked_decode_n64h32d128": "unmasked", "ahla_decode_n64h32d128": "ahla"}


def bench_variant_fwd(args, torch, np):
    """A variant on the inputs of a forward workload: segment summaries ->
    scan -> outputs (three C-ABI calls on one stream), each timed with HIP events."""
    import ctypes
    from causal_prefix_scan_amd import hla, synth
    vname, base = VARIANT_FWD[args.workload]
    V = _variants()[vname]
    cfg = dict(synth.FWD_WORKLOADS[base])
    if args.chunk:
        cfg["chunk"] = args.chunk
    B, H, T, d, dv, chunk = (cfg[x] for x in ("B", "H", "T", "d", "dv", "chunk"))
    inp = synth.make_fwd_inputs(B, H, T, d, dv, cfg["dtype"], cfg["seed"],
                                k_l2norm=cfg["k_l2norm"], decay=cfg["decay"])
    cv = lambda b: torch.from_numpy(b.view(np.int16)).view(torch.bfloat16).cuda()
    q, k, v = cv(inp.q_bits), cv(inp.k_bits), cv(inp.v_bits)
    g = None if inp.gamma is None else torch.from_numpy(inp.gamma).cuda()
    n = T // chunk
    st = V["alloc"]((B, H, n), d, dv, "cuda")
    o = torch.empty(B, H, T, dv, dtype=torch.float32, device="cuda")
    L = hla.lib()
    f_sum = getattr(L, V["prefix"] + "_chunk_summaries")
    f_scan = getattr(L, V["prefix"] + "_scan")
    f_out = getattr(L, V["prefix"] + "_output")
    p = hla.make_problem(q, v, chunk, g, cfg["normalize"], cfg["eps"])
    sst = V["struct"](st)
    stream = torch.cuda.current_stream()
    sp = ctypes.c_void_p(stream.cuda_stream)
    ptr = lambda t: ctypes.c_void_p(t.data_ptr())

    def step(ev=None):
        if ev:
            ev[0].record(stream)
        r1 = f_sum(ctypes.byref(p), ptr(q), ptr(k), ptr(v), ctypes.byref(sst), sp)
        if ev:
            ev[1].record(stream)
        r2 = f_scan(ctypes.byref(p), ctypes.byref(sst), sp)
        if ev:
            ev[2].record(stream)
        r3 = f_out(ctypes.byref(p), ptr(q), ptr(k), ptr(v), ctypes.byref(sst), ptr(o), None, sp)
        if ev:
            ev[3].record(stream)
        if r1 or r2 or r3:
            raise RuntimeError(f"HLA call failed: {r1} {r2} {r3}")

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    e0, e1, evs = timing_events(torch, args.steps)
    t0 = time.perf_counter()
    e0.record(stream)
    for i in range(args.steps):
        step(evs.get(i))
    e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = [sum(e[i].elapsed_time(e[i + 1]) for e in evs.values()) / len(evs) for i in range(3)]
    step_ms = e0.elapsed_time(e1) / args.steps
    tokens = B * H * T
    value = tokens / (step_ms / 1e3)
    U = B * H
    summ_bytes = U * n * V["summary_floats"](d, dv) * 4
    pre_bytes = U * n * V["prefix_floats"](d, dv) * 4
    io_bytes = tokens * (2 * d + dv) * 2
    names = [V["prefix"] + x for x in ("_chunk_summaries", "_scan", "_output")]
    kernels = {
        names[0]: dict(ms=ms[0], bytes=io_bytes + summ_bytes),
        names[1]: dict(ms=ms[1], bytes=summ_bytes + pre_bytes),
        names[2]: dict(ms=ms[2], bytes=io_bytes + pre_bytes + tokens * dv * 4),
    }
    dom = max(kernels, key=lambda kname: kernels[kname]["ms"])
    kd = kernels[dom]
    achieved = kd["bytes"] / (kd["ms"] / 1e3) / 1e9
    f_tok = V["flops"](64, d, dv)
    out = {
        "metric": METRIC, "value": round(value, 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(step_ms, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": cfg["dtype"], "data": "synthetic",
        "config": {"workload": args.workload, "B": B, "H": H, "T": T, "d": d, "dv": dv,
                   "chunk": chunk, "decay": cfg["decay"], "normalize": cfg["normalize"],
                   "path": " + ".join(names)},
        "mfma_credited": {"flops_per_token": round(f_tok), "tflops": round(value * f_tok / 1e12, 1),
                          "peak_tflops": BF16_PEAK_TFLOPS,
                          "frac": round(value * f_tok / 1e12 / BF16_PEAK_TFLOPS, 4)},
        "kernels_ms": {kname: round(kv["ms"], 4) for kname, kv in kernels.items()},
        "wall_ms_per_step": round(wall * 1e3 / args.steps, 4),
        "kernel_events": f"per-call HIP events on {len(evs)} of the {args.steps} timed steps",
        "roofline": {"bound": "hbm", "kernel": dom, "achieved": round(achieved, 1),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": measured_traffic(f"{dom}@{args.workload}") if not args.chunk else None,
                     "bytes_per_launch": kd["bytes"], "avg_launch_ms": round(kd["ms"], 4)},
    }
    if not args.no_cpu_baseline:
        from threadpoolctl import threadpool_limits
        from oracle import hla_oracle as O
        uq, uk, uv, ug = inp.units()
        ntok = min(args.cpu_tokens, T)
        nt = cpu_threads()
        with threadpool_limits(limits=nt):
            t0 = time.perf_counter()
            getattr(O, V["oracle"])(uq[:, :ntok], uk[:, :ntok], uv[:, :ntok], ug)
            dt = time.perf_counter() - t0
        out["cpu_baseline"] = {"value": U * ntok / dt, "unit": "tokens/s", "cores": nt, "kind": "oracle",
                               "sample": f"fp64 serial recurrence of the {V['name']}, all {U} "
                                         f"(batch, head) units, first {ntok} of {T} tokens ({dt:.1f} s)",
                               "seconds": round(dt, 2), "cpu_model": cpu_model()}
    return out


def bench_variant_decode(args, torch, np):
    """Decode steps of a variant on the decode workload's shapes; the prefix
    state is the summary of the prefix as one segment."""
    from causal_prefix_scan_amd import synth
    V = _variants()[VARIANT_DECODE[args.workload]]
    _, cfg = synth.DECODE_WORKLOAD
    Nq, H, d, dv, P, seed = (cfg[x] for x in ("n_seq", "H", "d", "dv", "prefix_len", "seed"))
    U = Nq * H
    steps = args.steps
    pre = synth.make_fwd_inputs(Nq, H, P, d, dv, "bf16", seed)
    cv = lambda b: torch.from_numpy(np.ascontiguousarray(b).view(np.int16)).view(torch.bfloat16).cuda()
    pq, pk, pv = cv(pre.q_bits), cv(pre.k_bits), cv(pre.v_bits)
    sm = V["summaries"](pq, pk, pv, P)
    state = {key: sm[key][:, :, 0].contiguous() for key in V["keys"]}
    del pq, pk, pv, sm
    n_tok = args.warmup + steps
    toks_host = [synth.make_decode_step(Nq, H, d, dv, seed, s) for s in range(n_tok)]
    tq = torch.stack([cv(t[3][0]).reshape(Nq, H, d) for t in toks_host])
    tk = torch.stack([cv(t[3][1]).reshape(Nq, H, d) for t in toks_host])
    tv = torch.stack([cv(t[3][2]).reshape(Nq, H, dv) for t in toks_host])
    o = torch.empty(Nq, H, dv, dtype=torch.float32, device="cuda")
    den = torch.empty(Nq, H, dtype=torch.float32, device="cuda")
    states64 = None
    if not args.no_cpu_baseline:
        states64 = {key: val.double().cpu().numpy().reshape(U, *val.shape[2:]) for key, val in state.items()}
    dec = V["decode"]
    for s in range(args.warmup):
        dec(tq[s], tk[s], tv[s], state, None, True, cfg["eps"], o=o, den=den)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record(stream)
    for s in range(args.warmup, n_tok):
        dec(tq[s], tk[s], tv[s], state, None, True, cfg["eps"], o=o, den=den)
    e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    step_ms = e0.elapsed_time(e1) / steps
    value = U / (step_ms / 1e3)
    state_bytes = V["prefix_floats"](d, dv) * 4
    bytes_step = U * (2 * state_bytes + (2 * d + dv) * 2 + dv * 4 + 4)
    achieved = bytes_step / (step_ms / 1e3) / 1e9
    kname = V["prefix"] + "_decode_step"
    out = {
        "metric": METRIC, "value": round(value, 1), "unit": "unit-tokens/s", "n_gpus": 1,
        "steps": steps, "warmup": args.warmup, "ms_per_step": round(step_ms, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": args.workload, "n_seq": Nq, "H": H, "d": d, "dv": dv,
                   "prefix_len": P, "normalize": True, "path": kname},
        "wall_ms_per_step": round(wall * 1e3 / steps, 4),
        "roofline": {"bound": "hbm", "kernel": kname, "achieved": round(achieved, 1),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": measured_traffic(f"{kname}@{args.workload}"),
                     "bytes_per_launch": bytes_step, "avg_launch_ms": round(step_ms, 4)},
    }
    if states64 is not None:
        from threadpoolctl import threadpool_limits
        from oracle import hla_oracle as O
        serial = getattr(O, V["oracle"])
        nb = min(args.cpu_steps, len(toks_host))
        nt = cpu_threads()
        with threadpool_limits(limits=nt):
            t0 = time.perf_counter()
            st = states64
            for s in range(nb):
                tq_, tk_, tv_ = toks_host[s][:3]
                _, _, st = serial(tq_[:, None], tk_[:, None], tv_[:, None], None, st)
            dt = time.perf_counter() - t0
        out["cpu_baseline"] = {"value": U * nb / dt, "unit": "unit-tokens/s", "cores": nt,
                               "kind": "oracle",
                               "sample": f"fp64 {V['name']} decode steps, {U} units x {nb} steps ({dt:.1f} s)",
                               "seconds": round(dt, 2), "cpu_model": cpu_model()}
    return out


def credited_flops_per_token_bwd(c, d, dv):
    """Credited flops per token of the backward: seven first-order sums
    y = sum lam^(t-s) (a_t.b_s) c_s with (width of a and b, width of c) =
    (d, d) for p, (dv, d) for dp, (d, dv) for dv, (dv, d) and (d, d) for dq,
    2 x (d, d) for dk.  Each costs, per token, the state product and the
    state update (2 Da Dc each) and the causal c-token tile's scores and
    score-value product (c + 1 terms of Da and of Dc on average, 2 flops
    each, halved by the mask)."""
    pairs = [(d, d), (dv, d), (d, dv), (dv, d), (d, d), (d, d), (d, d)]
    return sum(4 * a * b + (c + 1) * (a + b) for a, b in pairs)


def bwd_bytes_per_token(d, dv, ib, chunk):
    """Algorithmic HBM bytes per token of one hla_bwd call: for each of the
    six sums (operands a, b, c and output y; ib bytes per input element and
    per element of the intermediates p and dp, fp32 for dO and the outputs
    dq, dk, dv), the summary pass reads b and c, the output pass
    reads a, b, c and writes y (accumulating sums also read y), and the
    segment states are written, read and rewritten by the scan and read by
    the output pass (4 Da Dc fp32 per segment).  The S dp sum reuses the
    prefixes of the p sum (the same states) and the dv sum those of the dp
    sum (their transposes), so neither has a summary pass; the two dk sums
    are one sum over the symmetric states (q dp^T + dp q^T).  Where b and c
    are the same tensor (k in p = S q and S dp) it is read once.  With bf16
    inputs the dp summary pass reads dO in fp32 and writes it rounded to
    bf16; every later pass reads that copy."""
    f = 4
    do = dv * ib                       # dO as the later passes read it
    cp = dv * 2 if ib == 2 else 0      # the bf16 copy's write (bf16 inputs)
    sums = [  # (a, b (summary pass), b (output pass), c, y, Da, Dc, accumulate, summary pass)
        (d * ib, d * ib, d * ib, 0, d * ib, d, d, False, True),          # p = S q (b = c = k)
        (dv * ib, dv * f + cp, do, d * ib, d * ib, dv, d, False, True),  # dp (+ the dO copy)
        (d * ib, 0, d * ib, do, dv * f, d, dv, False, False),            # dv (dp's prefixes, transposed)
        (do, dv * ib, dv * ib, d * ib, d * f, dv, d, False, True),       # dq = M dO
        (d * ib, 0, d * ib, 0, d * f, d, d, True, False),                # dq += S dp (b = c = k)
        (d * ib, d * ib, d * ib, d * ib, d * f, d, d, False, True),      # dk (q, dp) + (dp, q)
    ]
    return sum(((bs + c) + 3 * Da * Dc * f / chunk if summ else 0) + (a + bo + c) + Da * Dc * f / chunk
               + y * (2 if acc else 1) for a, bs, bo, c, y, Da, Dc, acc, summ in sums)


def bench_bwd(args, torch, np):
    """The backward pass on the B4 H16 T16384 d128 decayed inputs: one
    hla_bwd call per step (14 kernel launches on one stream), HIP events."""
    import ctypes
    from causal_prefix_scan_amd import hla, synth
    cfg = dict(synth.FWD_WORKLOADS["fwd_decay_bf16_b4h16t16384d128"])
    chunk = args.chunk or BWD_CHUNK
    B, H, T, d, dv = (cfg[x] for x in ("B", "H", "T", "d", "dv"))
    inp = synth.make_fwd_inputs(B, H, T, d, dv, cfg["dtype"], cfg["seed"], decay=cfg["decay"])
    cv = lambda b: torch.from_numpy(b.view(np.int16)).view(torch.bfloat16).cuda()
    q, k, v = cv(inp.q_bits), cv(inp.k_bits), cv(inp.v_bits)
    g = torch.from_numpy(inp.gamma).cuda()
    do = torch.from_numpy(synth.make_upstream_grad(B, H, T, dv, cfg["seed"])).cuda()
    dq = torch.empty(B, H, T, d, dtype=torch.float32, device="cuda")
    dk = torch.empty_like(dq)
    dvv = torch.empty(B, H, T, dv, dtype=torch.float32, device="cuda")
    L = hla.lib()
    p = hla.make_problem(q, v, chunk, g, False, 0.0)
    ws = torch.empty(L.hla_bwd_workspace_bytes(ctypes.byref(p)), dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream()
    sp = ctypes.c_void_p(stream.cuda_stream)
    ptr = lambda t: ctypes.c_void_p(t.data_ptr())

    def step():
        r = L.hla_bwd(ctypes.byref(p), ptr(q), ptr(k), ptr(v), ptr(do), ptr(dq), ptr(dk), ptr(dvv),
                      ptr(ws), ctypes.c_size_t(ws.numel()), sp)
        if r:
            raise RuntimeError(f"hla_bwd failed: {hla.status_string(r)}")

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record(stream)
    for _ in range(args.steps):
        step()
    e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    step_ms = e0.elapsed_time(e1) / args.steps
    tokens = B * H * T
    value = tokens / (step_ms / 1e3)
    f_tok = credited_flops_per_token_bwd(BWD_TILE, d, dv)
    tflops = value * f_tok / 1e12
    b_tok = bwd_bytes_per_token(d, dv, 2, chunk)
    achieved = b_tok * tokens / (step_ms / 1e3) / 1e9
    out = {
        "metric": "HLA backward tokens/s (B·H·T/s) at 1 MI355X", "value": round(value, 1),
        "unit": "tokens/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(step_ms, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": BWD_WORKLOAD, "B": B, "H": H, "T": T, "d": d, "dv": dv,
                   "chunk": chunk, "decay": True, "normalize": False, "path": "hla_bwd"},
        "wall_ms_per_step": round(wall * 1e3 / args.steps, 4),
        "mfma_credited": {"flops_per_token": round(f_tok), "tflops": round(tflops, 1),
                          "peak_tflops": BF16_PEAK_TFLOPS, "frac": round(tflops / BF16_PEAK_TFLOPS, 4)},
        "roofline": {"bound": "hbm", "kernel": "hla_bwd (the 14 launches of one call)",
                     "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": measured_traffic(f"hla_bwd@{BWD_WORKLOAD}") if not args.chunk else None,
                     "bytes_per_launch": round(b_tok * tokens), "avg_launch_ms": round(step_ms, 4)},
    }
    if not args.no_cpu_baseline:
        from threadpoolctl import threadpool_limits
        from oracle import hla_backward_oracle as BO
        uq, uk, uv, ug = inp.units()
        dou = do.cpu().numpy().reshape(B * H, T, dv)
        ntok = min(2048, T)
        nt = cpu_threads()
        with threadpool_limits(limits=nt):
            t0 = time.perf_counter()
            BO.grad_states(uq[:, :ntok], uk[:, :ntok], uv[:, :ntok], dou[:, :ntok], ug)
            dt = time.perf_counter() - t0
        out["cpu_baseline"] = {"value": B * H * ntok / dt, "unit": "tokens/s", "cores": nt,
                               "cpu_model": cpu_model(),
                               "kind": "oracle",
                               "sample": f"fp64 serial forward/reverse state recurrences, all {B * H} "
                                         f"(batch, head) units, first {ntok} of {T} tokens ({dt:.1f} s)",
                               "seconds": round(dt, 2)}
    return out


def hla3_bytes_per_token(d, dv, es, chunk):
    """Algorithmic HBM bytes per token of one hla3_fwd call: every pass reads
    its operand rows and writes its outputs once (a pass whose value operand
    is its key operand stages it once), and the segment summaries (9 arrays,
    m, z, r 16 floats wide) go through HBM four times (written, read and
    written by the scan, read by the output passes), spread over the
    segment's tokens."""
    one = 16 * es
    passes = [
        # local p, u, q.m: read q, k (and v), write the result (the unit
        # channel is formed, not read; the S^K, P^KV, m^K summaries are
        # counted with the states below)
        2 * d * es + d * es, 2 * d * es + dv * es + dv * es, 2 * d * es + one,
        # the other summaries: read the operands of each state (S^Q: q once;
        # z and r ride on Z's and R's passes, which read q.m besides)
        d * es, 2 * d * es, d * es + dv * es + one, d * es + dv * es + one,
        # global p, u, q.m: read q, read and rewrite the local p, u, q.m
        d * es + 2 * d * es + 2 * dv * es + 2 * one,
        # num (fp32 out), den16 (fp32 out), den
        2 * d * es + dv * es + dv * 4, 2 * d * es + one + 16 * 4, 16 * 4 + 4,
    ]
    state = (3 * d * d + 3 * d * dv + 3 * 16 * d) * 4
    return sum(passes) + 4 * state / chunk


def bench_hla3(args, torch, np):
    """The third-order forward (one hla3_fwd call per step) on the decayed
    B4 H16 T16384 d128 inputs."""
    from causal_prefix_scan_amd import hla, synth
    cfg = synth.FWD_WORKLOADS["fwd_decay_bf16_b4h16t16384d128"]
    B, H, T, d, dv = (cfg[x] for x in ("B", "H", "T", "d", "dv"))
    chunk = args.chunk or HLA3_CHUNK
    inp = synth.make_fwd_inputs(B, H, T, d, dv, "bf16", cfg["seed"], decay=True)
    cv = lambda b: torch.from_numpy(b.view(np.int16)).view(torch.bfloat16).cuda()
    q, k, v = cv(inp.q_bits), cv(inp.k_bits), cv(inp.v_bits)
    g = torch.from_numpy(inp.gamma).cuda()
    L = hla.lib()
    p = hla.make_problem(q, v, chunk, g)
    ws_bytes = L.hla3_workspace_bytes(ctypes.byref(p))
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device="cuda")
    o = torch.empty(B, H, T, dv, dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream()
    sp = ctypes.c_void_p(stream.cuda_stream)
    ptr = lambda t: ctypes.c_void_p(t.data_ptr())

    def step():
        r = L.hla3_fwd(ctypes.byref(p), ptr(q), ptr(k), ptr(v), ptr(o), None, None, ptr(ws),
                       ctypes.c_size_t(ws_bytes), sp)
        if r:
            raise RuntimeError(f"hla3_fwd failed: {r}")

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record(stream)
    for _ in range(args.steps):
        step()
    e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    step_ms = e0.elapsed_time(e1) / args.steps
    tokens = B * H * T
    value = tokens / (step_ms / 1e3)
    b_tok = hla3_bytes_per_token(d, dv, 2, chunk)
    achieved = b_tok * tokens / (step_ms / 1e3) / 1e9
    out = {
        "metric": METRIC, "value": round(value, 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(step_ms, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": HLA3_WORKLOAD, "B": B, "H": H, "T": T, "d": d, "dv": dv,
                   "chunk": chunk, "decay": True, "normalize": False,
                   "path": "hla3_fwd: local p, u, q.m; segment summaries; moment scan and R, r "
                           "scan with the segment map; p, u, q.m and num, den from the prefixes"},
        "wall_ms_per_step": round(wall * 1e3 / args.steps, 4),
        "roofline": {"bound": "hbm", "kernel": "hla3_fwd (whole call)", "achieved": round(achieved, 1),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": None, "bytes_per_launch": round(b_tok * tokens),
                     "avg_launch_ms": round(step_ms, 4)},
    }
    if not args.no_cpu_baseline:
        from threadpoolctl import threadpool_limits
        from oracle import hla3_oracle as O3
        uq, uk, uv, ug = inp.units()
        ntok = min(2048, T)
        nt = cpu_threads()
        with threadpool_limits(limits=nt):
            t1 = time.perf_counter()
            O3.serial3(uq[:, :ntok], uk[:, :ntok], uv[:, :ntok], ug)
            dt = time.perf_counter() - t1
        out["cpu_baseline"] = {"value": B * H * ntok / dt, "unit": "tokens/s", "cores": nt,
                               "kind": "oracle", "cpu_model": cpu_model(),
                               "sample": f"fp64 pages-form serial recurrence of the third order, all "
                                         f"{B * H} (batch, head) units, first {ntok} of {T} tokens "
                                         f"({dt:.1f} s)", "seconds": round(dt, 2)}
    return out


def bench_hla3_decode(args, torch, np):
    """Third-order decode steps on the decode workload's shapes (64 sequences
    x 32 heads, d = dv = 128), from the state after the 2048-token prefix
    (hla3_fwd with one segment per prefix and a final state)."""
    from causal_prefix_scan_amd import hla, synth
    _, cfg = synth.DECODE_WORKLOAD
    Nq, H, d, dv, P, seed = (cfg[x] for x in ("n_seq", "H", "d", "dv", "prefix_len", "seed"))
    U = Nq * H
    steps = args.steps
    pre = synth.make_fwd_inputs(Nq, H, P, d, dv, "bf16", seed)
    cv = lambda b: torch.from_numpy(np.ascontiguousarray(b).view(np.int16)).view(torch.bfloat16).cuda()
    pq, pk, pv = cv(pre.q_bits), cv(pre.k_bits), cv(pre.v_bits)
    _, _, state = hla.hla3_fwd(pq, pk, pv, P, None, want_state=True)
    del pq, pk, pv
    n_tok = args.warmup + steps
    toks_host = [synth.make_decode_step(Nq, H, d, dv, seed, s) for s in range(n_tok)]
    tq = torch.stack([cv(t[3][0]).reshape(Nq, H, d) for t in toks_host])
    tk = torch.stack([cv(t[3][1]).reshape(Nq, H, d) for t in toks_host])
    tv = torch.stack([cv(t[3][2]).reshape(Nq, H, dv) for t in toks_host])
    o = torch.empty(Nq, H, dv, dtype=torch.float32, device="cuda")
    den = torch.empty(Nq, H, dtype=torch.float32, device="cuda")
    states64 = None
    if not args.no_cpu_baseline:
        states64 = {key: val.double().cpu().numpy().reshape(U, *val.shape[2:]) for key, val in state.items()}
    for s in range(args.warmup):
        hla.hla3_decode_step(tq[s], tk[s], tv[s], state, None, True, cfg["eps"], o=o, den=den)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record(stream)
    for s in range(args.warmup, n_tok):
        hla.hla3_decode_step(tq[s], tk[s], tv[s], state, None, True, cfg["eps"], o=o, den=den)
    e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    step_ms = e0.elapsed_time(e1) / steps
    value = U / (step_ms / 1e3)
    state_bytes = (d * d + 2 * d * dv + 2 * d) * 4
    bytes_step = U * (2 * state_bytes + (2 * d + dv) * 2 + dv * 4 + 4)
    achieved = bytes_step / (step_ms / 1e3) / 1e9
    out = {
        "metric": METRIC, "value": round(value, 1), "unit": "unit-tokens/s", "n_gpus": 1,
        "steps": steps, "warmup": args.warmup, "ms_per_step": round(step_ms, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": "hla3_decode_n64h32d128", "n_seq": Nq, "H": H, "d": d, "dv": dv,
                   "prefix_len": P, "normalize": True, "path": "hla3_decode_step"},
        "wall_ms_per_step": round(wall * 1e3 / steps, 4),
        "roofline": {"bound": "hbm", "kernel": "hla3_decode_step", "achieved": round(achieved, 1),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": measured_traffic("hla3_decode_step@hla3_decode_n64h32d128"),
                     "bytes_per_launch": bytes_step, "avg_launch_ms": round(step_ms, 4)},
    }
    if states64 is not None:
        from threadpoolctl import threadpool_limits
        from oracle import hla3_oracle as O3
        nb = min(args.cpu_steps, len(toks_host))
        nt = cpu_threads()
        with threadpool_limits(limits=nt):
            t1 = time.perf_counter()
            st = states64
            for s in range(nb):
                _, _, st = O3.decode_step3(st, *toks_host[s][:3])
            dt = time.perf_counter() - t1
        out["cpu_baseline"] = {"value": U * nb / dt, "unit": "unit-tokens/s", "cores": nt,
                               "kind": "oracle", "cpu_model": cpu_model(),
                               "sample": f"fp64 third-order decode steps, {U} units x {nb} steps ({dt:.1f} s)",
                               "seconds": round(dt, 2)}
    return out


def bench_copy(args, torch):
    """A plain device-to-device copy of a known size: the reference the HBM
    traffic counters (FETCH_SIZE, WRITE_SIZE) are scaled by."""
    nbytes = 1 << 30
    x = torch.empty(nbytes // 4, dtype=torch.float32, device="cuda").fill_(1.0)
    y = torch.empty_like(x)
    for _ in range(args.warmup):
        y.copy_(x)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(args.steps):
        y.copy_(x)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.steps
    return {"metric": "device copy (counter calibration)", "value": round(2 * nbytes / ms / 1e6, 1),
            "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
            "ms_per_step": round(ms, 4), "higher_is_better": True, "scaling": "weak",
            "vs_baseline": None, "dtype": "f32", "data": "synthetic",
            "config": {"workload": "copy", "bytes_read": nbytes, "bytes_written": nbytes}}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures a single GPU (got --gpus {args.gpus}): the kernels run per "
              "GPU with no collectives, so there is no multi-GPU step to time", file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    torch.cuda.set_device(0)
    if args.workload == "copy":
        out = bench_copy(args, torch)
    elif args.workload.startswith("decode"):
        out = bench_decode(args, torch, np)
    elif args.workload in VARIANT_FWD:
        out = bench_variant_fwd(args, torch, np)
    elif args.workload in VARIANT_DECODE:
        out = bench_variant_decode(args, torch, np)
    elif args.workload == HLA3_WORKLOAD:
        out = bench_hla3(args, torch, np)
    elif args.workload == "hla3_decode_n64h32d128":
        out = bench_hla3_decode(args, torch, np)
    elif args.workload == BWD_WORKLOAD:
        out = bench_bwd(args, torch, np)
    else:
        out = bench_fwd(args, torch, np)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
