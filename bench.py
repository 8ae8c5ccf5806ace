"""MonarchAttention forward benchmark on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload n16k] [--warm]
                    [--fast-aggregate] [--fused]

A step is one monarch_attn_forward call (the whole hot path: layout gather,
stage 1, stage 2, step loop, output scatter) over one batch of seeded
synthetic input already resident in HBM.  The default workload is
N=16384 as a 128x128 grid, d=64, 12 heads, T=1, bf16 (the configuration the
headline metric names); --workload picks another of the five workloads
(n256, n4k_t3, n16k, video, video_tiled).

Timing: W untimed warm-up calls, then exactly K calls bracketed by
torch.cuda.synchronize().  Each call records HIP events before its first
kernel and after every kernel on the launch stream (through the library's
timed entry point), giving the per-call and per-kernel GPU time.  By default
the K calls rotate over enough copies of Q, K, V, Y to exceed twice the
256 MB Infinity Cache (cold mode: inputs come from HBM); --warm reuses one.

Prints one JSON line: value = effective TFLOP/s (algorithmic flops of the
method over the measured time), plus the dominant kernel's roofline (its share
of the method's bytes Q, K, V in and Y out over its measured time; the design's
bytes with the stage exchange and the counted HBM traffic as separate fields),
the CPU oracle timed on this host as a baseline, and the error of Y against
exact softmax attention.
"""

import argparse
import ctypes
import glob
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MonarchAttention fwd ms/call + effective TFLOP/s (frac. of roofline), N=16K d=64"
HBM_PEAK_GBS = 8000.0
MFMA_PEAK_TFLOPS = {"bf16": 2500.0, "f32": 157.3}
MALL_BYTES = 256 * 1024 * 1024


def source_hash():
    h = hashlib.sha256()
    for p in sorted(glob.glob(os.path.join(ROOT, "structured_sub_quadratic_amd", "csrc", "*"))):
        with open(p, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def method_bytes(cfg, name):
    """HBM bytes the method itself makes a launch move, whatever the design:
    its share of Q, K, V read and Y written (the whole call's algorithmic bytes
    split over the launches that touch them).  Stage 1 reads Q (its first-step
    queries) and the keys (and on the last step the values) of every block;
    stage 2 reads Q and, on the last step, writes Y.  The exchange between the
    stages is the design's, not the method's, and is not counted here."""
    S, N, d = cfg.slices, cfg.seq_len, cfg.head_dim
    e = 4 if cfg.dtype == "f32" else 2
    t = N * d * e                 # one [N, d] tensor of one slice
    kv = t / cfg.kv_group         # K or V, read once per K/V head
    per = {"stage1_last": t + 2 * kv, "stage1": t + kv, "stage2_last": 2 * t,
           "stage2_stats": t, "alpha": t, "stage2_alpha": t, "qbar": t,
           "fused_t1": 2 * t + 2 * kv}.get(name)
    return None if per is None else per * S


def method_flops(cfg, causal=0):
    """Algorithmic flops of the call.  With a block-causal mask a stage-2 row
    l meets only the allowed key blocks, min(b1, (l // g + 1) * g) of them,
    so b1 in the stage-2 terms becomes their mean over the rows."""
    if not causal:
        return cfg.algorithmic_flops()
    N, d, b1, b2, c1, c2, T = (cfg.seq_len, cfg.head_dim, cfg.b1, cfg.b2, cfg.c1, cfg.c2,
                               cfg.steps)
    kb = sum(min(b1, (l // causal + 1) * causal) for l in range(b1)) / b1
    per = 2 * N * d * (3 * c1 * b2 + 2 * c2 * kb + (T - 1) * 2 * (c1 * b2 + c2 * kb))
    return per * cfg.slices


def design_bytes(cfg, name, precise):
    """HBM bytes of one launch as designed: every operand the kernel reads
    once and every result it writes once, including the stage-1 -> stage-2
    exchange (c, u, entropies, normalisers) and the next-step queries."""
    S, N, d = cfg.slices, cfg.seq_len, cfg.head_dim
    e = 4 if cfg.dtype == "f32" else 2
    xc = 4 if (precise or cfg.dtype == "f32") else 2
    rows = cfg.b1 * cfg.b2 * cfg.c1 * cfg.c2         # exchange rows per slice (grid positions)
    qkv = (1 + 2 / cfg.kv_group) * N * d * e         # Q, and K, V once per K/V head
    if name == "stage1_last":
        b = qkv + rows * d * (xc + e) + rows * 8
    elif name == "stage1":
        b = qkv + rows * d * xc + rows * 8
    elif name == "stage2_last":
        b = N * d * e + rows * d * (xc + e) + rows * 4 + N * d * e + N * 4
    elif name == "stage2_stats":
        b = N * d * e + rows * d * xc + rows * 4 + N * 4
    elif name == "alpha":
        b = N * d * e + rows * d * xc + rows * 4 + N * 4 + rows * d * 4
    elif name == "stage2_alpha":
        # Q, c and the entropies in; the normalisers and the next queries out
        b = N * d * e + rows * d * xc + rows * 4 + N * 4 + rows * d * 4
    elif name == "fused_t1":
        # the whole T = 1 pass in one launch: Q, K, V in and Y out, plus the
        # exchange written and read back
        b = qkv + N * d * e + 2 * rows * d * (xc + e) + rows * 12
    elif name == "qbar":
        b = N * d * e + cfg.c1 * cfg.b2 * d * 4
    else:
        return None
    return b * S


def host_description():
    """CPU model (from /proc/cpuinfo) and the BLAS library NumPy links."""
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    blas = "unknown"
    try:
        import numpy as np
        info = np.show_config(mode="dicts")["Build Dependencies"]["blas"]
        blas = f"{info.get('name', '?')} {info.get('version', '')}".strip()
    except Exception:
        pass
    return model, blas


def exact_attention_error(cfg, Q, K, V, y, rows_per_head=None, seed=4242, causal=0):
    """P9, reported only: the relative Frobenius error ||Y - Y_exact|| /
    ||Y_exact|| of the method's output against exact softmax attention
    softmax(Q K^T / sqrt(d)) V, computed in float64 on the host in row
    chunks.  Every row when rows_per_head is None, else that many seeded
    query rows per head (the same rows for every head).  With a block-causal
    mask (layouts whose blocks are runs of b2 consecutive tokens) the exact
    product is masked the same way: token n attends to n' iff
    unit(n') <= unit(n), unit = grid block // g."""
    import numpy as np
    B, H, N, d = Q.shape
    unit = None
    if causal:
        if cfg.layout not in ("flat", "fh_w", "f_hw"):
            return None
        pre = cfg.b1 * cfg.b2 - N if cfg.pad == "pre" else 0
        unit = ((np.arange(N) + pre) // cfg.b2) // causal
    group = H // K.shape[1]
    scale = 1.0 / math.sqrt(d)
    rows = np.arange(N) if rows_per_head is None else \
        np.sort(np.random.default_rng(seed).choice(N, size=min(rows_per_head, N), replace=False))
    num = den = 0.0
    for b in range(B):
        for h in range(H):
            k = K[b, h // group].astype(np.float64)
            v = V[b, h // group].astype(np.float64)
            for c0 in range(0, rows.size, 2048):
                r = rows[c0:c0 + 2048]
                s_ = scale * (Q[b, h, r].astype(np.float64) @ k.T)
                if unit is not None:
                    s_ = np.where(unit[None, :] <= unit[r][:, None], s_, -np.inf)
                s_ -= s_.max(axis=1, keepdims=True)
                p = np.exp(s_)
                ex = (p @ v) / p.sum(axis=1, keepdims=True)
                num += float(np.sum((y[b, h, r].astype(np.float64) - ex) ** 2))
                den += float(np.sum(ex ** 2))
    return {"value": math.sqrt(num / den), "rows": "all" if rows_per_head is None else
            f"{rows.size} seeded query rows per head (seed {seed})",
            "measure": "||Y - Y_exact||_F / ||Y_exact||_F, Y_exact = softmax(QK^T/sqrt(d))V in "
                       "float64 on the host"}


def cpu_baseline(cfg, causal=0):
    """The oracle as it stands, on this host, over the whole workload (or a
    bounded number of slices), in the metric's unit."""
    import numpy as np
    import oracle
    from workloads import make_inputs
    cores = len(os.sched_getaffinity(0))
    per_slice = method_flops(cfg, causal) / cfg.slices
    budget_s, spent, done = 20.0, 0.0, 0
    slices = [(b, h) for b in range(cfg.batch) for h in range(cfg.heads)]
    for sl in slices:
        Q, K, V = make_inputs(cfg, slices=[sl])
        t0 = time.perf_counter()
        oracle.forward(Q, K, V, cfg.b1, cfg.b2, cfg.steps, cfg.c1, cfg.c2,
                       layout=cfg.layout, fhw=cfg.fhw, slices=[sl], pad=cfg.pad, causal=causal)
        spent += time.perf_counter() - t0
        done += 1
        if spent > budget_s:
            break
    tflops = per_slice * done / spent / 1e12
    model, blas = host_description()
    return {"value": tflops, "unit": "TFLOP/s", "cores": cores, "kind": "oracle",
            "sample": f"{done} of {len(slices)} slices of the same workload, NumPy float64, "
                      f"{spent:.2f} s ({spent / done * 1e3:.0f} ms/slice; full call "
                      f"would take {spent / done * len(slices):.1f} s)",
            "cpu_model": model, "blas": blas}


def sampled_parity(cfg, Q, K, V, y, causal=0):
    """Y, L, R of one slice at four columns against the oracle (quick check)."""
    import numpy as np
    import oracle
    cols = sorted({0, cfg.b2 // 3, cfg.b2 // 2, cfg.b2 - 1})
    ref = oracle.forward(Q[:1, :1], K[:1, :1], V[:1, :1], cfg.b1, cfg.b2, cfg.steps, cfg.c1,
                         cfg.c2, layout=cfg.layout, fhw=cfg.fhw, cols=cols, pad=cfg.pad,
                         causal=causal)
    tok = ref["grid"][:, cols].reshape(-1)
    tok = tok[tok >= 0]
    a, r = y[0, 0][tok].astype(np.float64), ref["y"][0, 0][tok]
    return float(np.abs(a - r).max() / np.abs(r).max())


def backward_flops(cfg, rebuilt=True):
    """Products of the backward as computed (per slice, untiled).  Last step:
    stage 2 forms P, dP, dQ, dc, du over b1 x b1 per column (5), stage 1
    forms R, dR (two products), dQ, dK (two products), dV over b2 x b2 per
    block (7).  Each earlier step of T > 1: stage 2 forms P, dP, dQ, the
    direct P dalpha term and dc (5 over b1), stage 1 R, dR, dq~ and dK (two
    products; 5 over b2).  The rebuilt forward: per step c (2 over b2) and
    the stage-2 normalisers (1 over b1), u once (1 over b2), and the next
    queries of every step but the last (2 over b1).  With row tiles and key
    segments a stage-2 query meets b1 * c2 keys and a key c1 * b2 stage-1
    queries, which take the places of b1 and b2.  rebuilt=False: the forward
    state was kept, so the rebuilt forward's products are not counted."""
    N, d, T = cfg.seq_len, cfg.head_dim, cfg.steps
    b1, b2 = cfg.b1 * cfg.c2, cfg.c1 * cfg.b2
    per = (5 * b1 + 7 * b2) + (T - 1) * (5 * b1 + 5 * b2)
    if rebuilt:
        per += T * (2 * b2 + b1) + b2 + (T - 1) * 2 * b1
    return 2 * N * d * per * cfg.slices


def bench_backward(args, cfg, dev):
    """One JSON line: the backward call's time and effective TFLOP/s."""
    import numpy as np
    import torch
    import structured_sub_quadratic_amd as ma
    from workloads import make_inputs
    from workloads.generators import round_to_bf16
    tdt = torch.float32 if cfg.dtype == "f32" else torch.bfloat16
    Q, K, V = make_inputs(cfg)
    dY = np.random.default_rng(77).standard_normal(Q.shape).astype(np.float32)
    if cfg.dtype == "bf16":
        dY = round_to_bf16(dY)
    set_bytes = 7 * Q.size * (4 if cfg.dtype == "f32" else 2)
    n_sets = 1 if args.warm else max(2, math.ceil(2.5 * MALL_BYTES / set_bytes))
    base = [torch.from_numpy(x).to(dev).to(tdt) for x in (Q, K, V, dY)]
    sets = [tuple(x.clone() for x in base) + tuple(torch.empty_like(base[0]) for _ in range(3))
            for _ in range(n_sets)]
    del base
    prob = ma.make_problem(cfg.batch, cfg.heads, cfg.seq_len, cfg.head_dim, cfg.b1, cfg.b2,
                           cfg.steps, cfg.c1, cfg.c2, None, cfg.dtype, cfg.layout, cfg.fhw, 0)
    nws = n_sets if args.reuse_state else 1
    wss = [torch.empty(max(ma.backward_workspace_size(prob), 1), dtype=torch.uint8, device=dev)
           for _ in range(nws)]
    ys = [None] * n_sets
    if args.reuse_state:      # each set's forward state stays in its own workspace, with its Y
        for j, ((q, k, v, *_), w) in enumerate(zip(sets, wss)):
            ys[j] = ma.forward(q, k, v, cfg.b1, cfg.b2, cfg.steps, cfg.c1, cfg.c2, layout=cfg.layout,
                               fhw=cfg.fhw, workspace=w)

    def call(i):
        q, k, v, dy, dq, dk, dv = sets[i % n_sets]
        ma.backward(q, k, v, dy, cfg.b1, cfg.b2, cfg.steps, cfg.c1, cfg.c2, layout=cfg.layout,
                    fhw=cfg.fhw, workspace=wss[i % nws], out=(dq, dk, dv),
                    reuse_forward_state=args.reuse_state, y=ys[i % n_sets])
    for i in range(args.warmup):
        call(i)
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    for i in range(args.steps):
        call(i)
    end.record()
    torch.cuda.synchronize()
    ms = start.elapsed_time(end) / args.steps
    flops = backward_flops(cfg, rebuilt=not args.reuse_state)
    out = {
        "metric": "MonarchAttention bwd ms/call + effective TFLOP/s", "value":
            round(flops / (ms * 1e-3) / 1e12, 3), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 5),
        "higher_is_better": True, "dtype": cfg.dtype, "data": "synthetic",
        "config": {"workload": cfg.name,
                   "pass": "backward (dQ, dK, dV), forward state " +
                           ("and output Y kept from the forward call" if args.reuse_state
                            else "rebuilt"),
                   "inputs": "warm (one set)" if args.warm else f"cold ({n_sets} rotating sets)"},
        "flops_counted": flops,
        "mfma_frac_of_call": round(flops / (ms * 1e-3) / 1e12 / MFMA_PEAK_TFLOPS[cfg.dtype], 4),
    }
    print(json.dumps(out))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="n16k",
                    choices=["n256", "n4k_t3", "n16k", "video", "video_tiled", "n16k_pad",
                             "n16k_gqa"])
    ap.add_argument("--warm", action="store_true", help="reuse one input set (MALL-resident)")
    ap.add_argument("--fast-aggregate", action="store_true",
                    help="plain bf16 c = R K path (the default for T = 1)")
    ap.add_argument("--precise-aggregate", action="store_true",
                    help="split bf16 hi+lo c = R K path (the default for T > 1)")
    ap.add_argument("--fused", action="store_true",
                    help="T = 1 as one cooperative launch instead of separate stage launches")
    ap.add_argument("--reuse-state", action="store_true",
                    help="with --backward (T = 1): each input set's forward call leaves its state in "
                         "the workspace and its output Y, and the timed backward calls reuse both")
    ap.add_argument("--backward", action="store_true",
                    help="time monarch_attn_backward (dQ, dK, dV for a seeded dY) instead of "
                         "the forward")
    ap.add_argument("--causal", type=int, default=0,
                    help="block-causal use: g grid blocks per causal unit (0: bidirectional)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-p9", action="store_true",
                    help="skip the error of Y against exact softmax attention (host float64)")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="first run a plain 256 MiB device copy 3 times (reference for the "
                         "FETCH_SIZE / WRITE_SIZE counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (got --gpus {args.gpus}); the slices are "
              "independent and would shard across GPUs with no communication, but no "
              "multi-GPU figure is produced here.", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch
    import structured_sub_quadratic_amd as ma
    from structured_sub_quadratic_amd import _lib
    from workloads import get_workload, make_inputs

    cfg = get_workload(args.workload)
    dev = torch.device("cuda:0")
    if args.backward:
        bench_backward(args, cfg, dev)
        return
    if args.calibrate_copy:
        src = torch.empty(256 * 1024 * 1024 // 4, dtype=torch.float32, device=dev).fill_(1.0)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    tdt = torch.float32 if cfg.dtype == "f32" else torch.bfloat16
    Q, K, V = make_inputs(cfg)
    set_bytes = (2 * Q.size + K.size + V.size) * (4 if cfg.dtype == "f32" else 2)
    n_sets = 1 if args.warm else max(2, math.ceil(2.5 * MALL_BYTES / set_bytes))
    base = [torch.from_numpy(x).to(dev).to(tdt) for x in (Q, K, V)]
    sets = [(base[0].clone(), base[1].clone(), base[2].clone(), torch.empty_like(base[0]))
            for _ in range(n_sets)]
    del base

    flags = (ma.MA_FLAG_FAST_AGGREGATE if args.fast_aggregate else 0) | \
        (ma.MA_FLAG_PRECISE_AGGREGATE if args.precise_aggregate else 0)
    precise = cfg.dtype == "f32" or args.precise_aggregate or \
        (not args.fast_aggregate and cfg.steps > 1)
    if args.fused:
        flags |= ma.MA_FLAG_FORCE_FUSED
    if cfg.pad == "pre":
        flags |= ma.MA_FLAG_PAD_FRONT
    prob = ma.make_problem(cfg.batch, cfg.heads, cfg.seq_len, cfg.head_dim, cfg.b1, cfg.b2,
                           cfg.steps, cfg.c1, cfg.c2, None, cfg.dtype, cfg.layout, cfg.fhw, flags,
                           kv_heads=cfg.kv_heads, causal=args.causal)
    names = ma.launch_names(prob)
    nl = len(names)
    ws_bytes = ma.workspace_size(prob)
    ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=dev)
    lib = _lib.load()
    stream = torch.cuda.current_stream(dev).cuda_stream
    nev = 2 * nl            # start and end of every launch
    events = [[ma.Event() for _ in range(nev)] for _ in range(args.steps)]
    ev_arrays = [(ctypes.c_void_p * nev)(*[e.ptr.value for e in row]) for row in events]
    cex = _lib.MAExports(None, None, None, None)
    pprob = ctypes.byref(prob)
    pcex = ctypes.byref(cex)
    call_args = [(s[0].data_ptr(), s[1].data_ptr(), s[2].data_ptr(), s[3].data_ptr()) for s in sets]

    def call(i, evs=None, n=0):
        q, k, v, y = call_args[i % n_sets]
        if evs is None:
            st = lib.monarch_attn_forward(pprob, q, k, v, y, pcex, ws.data_ptr(), ws_bytes, stream)
        else:
            st = lib.monarch_attn_forward_timed(pprob, q, k, v, y, pcex, ws.data_ptr(), ws_bytes,
                                                stream, evs, n)
        if st != 0:
            raise RuntimeError(f"monarch_attn_forward failed: {st}")

    for i in range(args.warmup):
        call(i)
    # the timed region: K calls of the product entry point, bracketed by a
    # synchronisation and a HIP event pair on the launch stream
    t_start, t_end = ma.Event(), ma.Event()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    _lib.check(lib.monarch_attn_event_record(t_start.ptr, stream), "monarch_attn_event_record")
    for i in range(args.steps):
        call(i)
    _lib.check(lib.monarch_attn_event_record(t_end.ptr, stream), "monarch_attn_event_record")
    torch.cuda.synchronize()
    wall_ms = (time.perf_counter() - t0) * 1e3 / args.steps
    span_ms = t_start.elapsed_ms(t_end) / args.steps

    # per-launch durations: the same K calls again through the timed entry
    # point, whose events take each kernel's own start and end time stamps
    # (kept out of the timed region all the same)
    for i in range(args.steps):
        call(i, ev_arrays[i], nev)
    torch.cuda.synchronize()
    per_kernel = {n: [] for n in names}
    for i in range(args.steps):
        row = events[i]
        for j, n in enumerate(names):
            per_kernel[n].append(row[2 * j].elapsed_ms(row[2 * j + 1]))
    call_ms = float(np.mean([events[i][0].elapsed_ms(events[i][-1]) for i in range(args.steps)]))
    kern_ms = {n: float(np.mean(v)) for n, v in per_kernel.items()}

    flops = method_flops(cfg, args.causal)
    ms = span_ms
    value = flops / (ms * 1e-3) / 1e12

    dom = max(set(names), key=lambda n: kern_ms[n])
    kb = method_bytes(cfg, dom)
    db = design_bytes(cfg, dom, precise)
    achieved = kb / (kern_ms[dom] * 1e-3) / 1e9
    traffic = None
    tfile = os.path.join(ROOT, "profiles", "traffic.json")
    if os.path.exists(tfile):
        with open(tfile) as fh:
            tr = json.load(fh)
        key = f"{cfg.key}{'' if precise else '_plain'}:{dom}"
        ent = tr.get(key)
        if ent and ent.get("source_hash") == source_hash():
            traffic = ent["hbm_bytes_per_launch"]
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic,
                "kernel": dom, "algorithmic_bytes": kb, "kernel_ms": round(kern_ms[dom], 5),
                "design_bytes": db,
                "design_frac": round(db / (kern_ms[dom] * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                "traffic_over_algorithmic": round(traffic / kb, 3) if traffic else None,
                "traffic_over_design": round(traffic / db, 3) if traffic else None}
    whole = {"algorithmic_bytes": cfg.algorithmic_bytes(),
             "hbm_frac_of_call": round(cfg.algorithmic_bytes() / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
             "mfma_frac_of_call": round(value / MFMA_PEAK_TFLOPS[cfg.dtype], 4)}

    y = sets[(args.steps - 1) % n_sets][3].float().cpu().numpy()
    parity = sampled_parity(cfg, Q, K, V, y, args.causal)
    cpu = None if args.no_cpu_baseline else cpu_baseline(cfg, args.causal)
    p9 = None
    if not args.no_p9:
        # every row where the exact product fits a few seconds of host time,
        # 4096 seeded rows per head for the video latents
        p9 = exact_attention_error(cfg, Q, K, V, y,
                                   rows_per_head=4096 if cfg.seq_len > 16384 else None,
                                   causal=args.causal)

    out = {
        "metric": METRIC, "value": round(value, 3), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": cfg.dtype, "data": "synthetic",
        "config": {"workload": cfg.name, "batch": cfg.batch, "heads": cfg.heads,
                   "seq_len": cfg.seq_len, "head_dim": cfg.head_dim, "b1": cfg.b1, "b2": cfg.b2,
                   "T": cfg.steps, "tiles": [cfg.c1, cfg.c2], "layout": cfg.layout,
                   "kv_heads": cfg.kv_heads or cfg.heads,
                   "padding": (f"{cfg.b1 * cfg.b2 - cfg.seq_len} positions, {cfg.pad}"
                               if cfg.b1 * cfg.b2 > cfg.seq_len else None),
                   "inputs": "warm (one set)" if args.warm else f"cold ({n_sets} rotating sets)",
                   "aggregate": "split bf16 hi+lo" if precise and cfg.dtype != "f32" else
                                ("fp32" if cfg.dtype == "f32" else "plain bf16"),
                   "launches": names,
                   "block_causal_units": args.causal or None},
        "roofline": roofline,
        "cpu_baseline": cpu,
        "whole_call": whole,
        "kernels_ms": {n: round(v, 5) for n, v in kern_ms.items()},
        "call_ms_kernel_span": round(call_ms, 5),
        "wall_ms_per_call": round(wall_ms, 5),
        "parity_sampled_Y_rel_err": parity,
        "error_vs_exact_attention": p9,
        "source_hash": source_hash(),
    }
    print(json.dumps(out))


if __name__ == "__main__":
    main()
