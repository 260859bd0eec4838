"""Benchmark of the DMA forward on one MI355X.

A step is one whole forward over one batch of seeded synthetic input already
resident in HBM: dynamic weights, causal top-w keep mask with skip lists, and
the masked attention.  The default workload is the 16K-token GQA prefill
(B=1, Hq=32, Hkv=8, S=16384, D=128, w=2048, bf16).

Prints one JSON line:
  value          effective TFLOP/s of the whole forward, counting 4*D flops per
                 kept (query head, query row, key) triple
  ms_per_step    wall time per forward (synchronised on both sides of K steps)
  roofline       the attention kernel (dominant) against the bf16 dense MFMA peak;
                 its duration comes from HIP events on the launch stream
  cpu_baseline   the fp64 oracle on a bounded sample of the same workload
  stages_ms      event-timed weights / mask / attention per step, from a second
                 pass of K steps after the timed one (an event record costs GPU
                 time, so the timed steps carry only the two events around the
                 attention that the roofline uses; its stage time is theirs)
"""
import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "effective TFLOP/s (kept pairs) + ms/fwd, 16K-token DMA prefill, 1 MI355X"
PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0
# HBM bytes per launch of the attention kernel, from two counter passes (FETCH_SIZE and
# WRITE_SIZE) scaled by the same counters on a plain copy of known size.  The file carries
# the hash of the kernel sources it was taken on; a stale file reports null.
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "attn_prefill_bf16_kernel.prefill_16k.traffic.txt")
ATTN_SOURCES = ("trainable_dynamic_mask_amd/csrc/attn_prefill.hip",
                "trainable_dynamic_mask_amd/csrc/common.h",
                "trainable_dynamic_mask_amd/csrc/lds_dma.h")


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10, help="untimed steps before the timed ones")
    ap.add_argument("--clock-ramp-ms", type=float, default=300.0,
                    help="run untimed steps for this long before the warm-up: the shader clock "
                         "takes ~0.1-0.3 s of load to reach its sustained level, so without it "
                         "a short run times the kernels at a lower clock")
    ap.add_argument("--workload", default="prefill_16k")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="CPU time budget of the oracle sample")
    ap.add_argument("--backward", action="store_true",
                    help="time the training backward instead (attention and weights "
                         "gradients after a training forward); prints its own JSON line")
    ap.add_argument("--hbm-stages", action="store_true",
                    help="time the HBM-bound stages of the workload one at a time, each "
                         "repetition after a 512 MiB flush of the caches, and print their "
                         "achieved GB/s against the algorithmic bytes (own JSON line)")
    ap.add_argument("--reps", type=int, default=20, help="repetitions per stage (--hbm-stages)")
    ap.add_argument("--vproj", action="store_true",
                    help="the value projection with delta fused into its epilogue, against "
                         "the projection alone followed by the weights call (hidden = Hq*D)")
    ap.add_argument("--natural-ab", action="store_true",
                    help="time the attention on the gathered keep lists against natural-order "
                         "block skipping (the mask's key-tile lists, per-element keep test)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run a plain device copy of MIB MiB five times (the reference "
                         "reading of the FETCH_SIZE / WRITE_SIZE counters) and exit")
    return ap.parse_args()


def attn_source_hash():
    h = hashlib.sha256()
    for f in ATTN_SOURCES:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic(workload):
    """Counter-measured HBM bytes per attention launch, or None when no reading was
    taken on this workload with the current kernel sources."""
    if workload != "prefill_16k" or not os.path.exists(TRAFFIC_FILE):
        return None
    kv = {}
    with open(TRAFFIC_FILE) as fh:
        for line in fh:
            if ":" in line and not line.startswith((" ", "#")):
                k, v = line.split(":", 1)
                kv[k.strip()] = v.strip()
    if kv.get("kernel_source_sha256") != attn_source_hash():
        return None
    try:
        return float(kv["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def clock_ramp(step, ms):
    """Untimed steps for `ms` milliseconds of wall time (the GPU busy throughout):
    the shader clock ramps up under load, and the timed steps should see the
    clock a sustained workload runs at."""
    import torch
    t0 = time.perf_counter()
    while (time.perf_counter() - t0) * 1e3 < ms:
        for _ in range(4):
            step()
        torch.cuda.synchronize()


def copy_calibration(mib):
    import torch
    n = mib << 20
    src = torch.ones(n // 4, dtype=torch.float32, device="cuda:0")
    dst = torch.empty_like(src)
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes_read": n, "copy_calibration_bytes_written": n,
                      "launches": 5}), flush=True)


def cpu_baseline(x, wl, budget_s):
    """The fp64 oracle on a bounded sample: delta for every key plus the keep
    set and attention of randomly drawn query rows; the delta time is prorated
    to the sampled share of rows."""
    import numpy as np
    import oracle

    t0 = time.perf_counter()
    d64 = oracle.weights(x["V"], x["Delta"], x["A"])
    t_w = time.perf_counter() - t0
    Qc, Kc, Vc = (x[k].float().cpu() for k in ("Q", "K", "V"))
    rng = np.random.default_rng(wl.seed)
    total_rows = wl.B * wl.Hq * wl.Sq

    def draw(n):
        return np.stack([rng.integers(0, wl.B, n), rng.integers(0, wl.Hq, n),
                         rng.integers(0, wl.Sq, n)], 1).astype(np.int64)

    probe = draw(256)
    t0 = time.perf_counter()
    oracle.attn_rows(Qc, Kc, Vc, d64, wl.q_offset, wl.w, probe)
    per_row = (time.perf_counter() - t0) / len(probe)
    n = int(min(total_rows, max(256, (budget_s - t_w) / max(per_row, 1e-9))))
    rows = draw(n)
    t0 = time.perf_counter()
    oracle.attn_rows(Qc, Kc, Vc, d64, wl.q_offset, wl.w, rows)
    t_rows = time.perf_counter() - t0
    kept = np.minimum(wl.q_offset + rows[:, 2] + 1, wl.w).sum()
    t = t_rows + t_w * n / total_rows
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as fh:
            model = next(l.split(":", 1)[1].strip() for l in fh if l.startswith("model name"))
    except (OSError, StopIteration):
        pass
    return {"value": float(4 * wl.D * kept / t / 1e12), "unit": "TFLOP/s",
            "cores": oracle.num_threads(), "cpu_model": model, "kind": "oracle",
            "sample": f"fp64 oracle: delta of all {wl.B * wl.Hkv * wl.Sk} keys ({t_w:.2f} s, "
                      f"prorated) + keep set and attention of {n} random query rows of "
                      f"{total_rows} ({t_rows:.2f} s)",
            "seconds": round(t_w + t_rows, 2)}


def backward_bench(args, wl, x, dev):
    """Backward of the DMA forward: attention gradients (dQ, dK, dV, ddelta) then the
    weights gradients (dDelta, dA, the value-row part of dV), timed with events on the
    launch stream.  Effective FLOPs: 8*D per kept pair (the dQ, dK, dV and dP
    products; the recomputed scores are not counted)."""
    import torch
    import trainable_dynamic_mask_amd as dma
    from trainable_dynamic_mask_amd.inputs import make_grad

    dO = make_grad(wl, device=dev)
    delta = dma.weights(x["V"], x["Delta"], x["A"])
    mask = dma.topk_mask(delta, wl.Sq, wl.q_offset, wl.w)
    O, lse, Ores = dma.attn_fwd_train(x["Q"], x["K"], x["V"], delta, mask)
    lib = dma.load()
    ws = torch.empty(max(256, lib.dma_attn_bwd_workspace_bytes(wl.B, wl.Hq, wl.Hkv, wl.Sq,
                                                                 wl.Sk, wl.w)),
                     dtype=torch.uint8, device=dev)
    wsw = torch.empty(max(16, lib.dma_weights_bwd_workspace_bytes(wl.B, wl.Sk, wl.Hkv)),
                      dtype=torch.uint8, device=dev)
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]

    def step(e=None):
        if e:
            e[0].record()
        dQ, dK, dV, dd = dma.attn_bwd(x["Q"], x["K"], x["V"], delta, mask, O, lse, dO,
                                      O_res=Ores, workspace=ws)
        if e:
            e[1].record()
        dma.weights_bwd(x["V"], x["Delta"], x["A"], dd, dV=dV, workspace=wsw)
        if e:
            e[2].record()
        return dQ

    clock_ramp(step, args.clock_ramp_ms)
    for _ in range(max(3, args.warmup // 10)):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(args.steps):
        dQ = step(ev[k])
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / args.steps
    ta = sum(e[0].elapsed_time(e[1]) for e in ev) / args.steps
    tw = sum(e[1].elapsed_time(e[2]) for e in ev) / args.steps
    assert torch.isfinite(dQ).all(), "non-finite gradient"
    flops = 2 * wl.effective_flops()
    out = {"metric": "effective TFLOP/s (kept pairs) of the DMA backward, 1 MI355X",
           "value": round(flops / (ms * 1e-3) / 1e12, 3), "unit": "TFLOP/s",
           "ms_per_step": round(ms, 4), "steps": args.steps, "dtype": wl.dtype,
           "data": "synthetic", "config": {"workload": wl.name, "effective_flop": flops},
           "stages_ms": {"attention_bwd": round(ta, 4), "weights_bwd": round(tw, 4)},
           "attention_bwd_tflops": round(flops / (ta * 1e-3) / 1e12, 2)}
    print(json.dumps(out), flush=True)


def vproj_bench(args, wl, x, dev):
    """Fused value projection + weights (dma_vproj_weights with Delta) against the
    same projection without the epilogue followed by dma_weights, which re-reads V.
    X [B, Sk, Hq*D] and Wv [Hq*D, Hkv*D] are seeded bf16 normals (Wv scaled by
    1/sqrt(Cin)), Delta and A the workload's."""
    import statistics
    import torch
    import trainable_dynamic_mask_amd as dma
    B, Sk, Hkv, D = wl.B, wl.Sk, wl.Hkv, wl.D
    Cin = wl.Hq * wl.D
    g = torch.Generator(device=dev).manual_seed(wl.seed + 31)
    X = torch.randn(B, Sk, Cin, generator=g, device=dev).to(torch.bfloat16)
    Wv = (torch.randn(Cin, Hkv * D, generator=g, device=dev) / Cin ** 0.5).to(torch.bfloat16)
    V = torch.empty(B, Sk, Hkv, D, dtype=torch.bfloat16, device=dev)
    delta = torch.empty(B, Hkv, Sk, dtype=torch.float32, device=dev)
    lib = dma.load()
    ws = torch.empty(max(16, lib.dma_vproj_workspace_bytes(B, Sk, Hkv, D)), dtype=torch.uint8,
                     device=dev)

    def fused():
        dma.vproj_weights(X, Wv, Hkv, x["Delta"], x["A"], V=V, delta=delta, workspace=ws)

    def proj():
        dma.vproj_weights(X, Wv, Hkv, V=V)

    def wts():
        dma.weights(V, x["Delta"], x["A"], out=delta)

    def separate():
        proj()
        wts()

    def timed(f):
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(args.reps)]
        for a, b in ev:
            a.record()
            f()
            b.record()
        torch.cuda.synchronize()
        return statistics.median(a.elapsed_time(b) for a, b in ev)

    clock_ramp(separate, args.clock_ramp_ms)
    res = {}
    for _ in range(2):  # interleaved twice: the median of each over both passes
        for name, f in (("fused", fused), ("separate", separate), ("projection", proj),
                        ("weights", wts)):
            for _ in range(3):
                f()
            res.setdefault(name, []).append(timed(f))
    ms = {k: round(statistics.median(v), 4) for k, v in res.items()}
    flop = 2.0 * B * Sk * Cin * Hkv * D
    out = {"mode": "vproj", "workload": wl.name, "B": B, "Sk": Sk, "Cin": Cin, "N": Hkv * D,
           "reps": args.reps, "ms": ms,
           "tflops_fused": round(flop / (ms["fused"] * 1e-3) / 1e12, 1),
           "tflops_projection": round(flop / (ms["projection"] * 1e-3) / 1e12, 1),
           "saved_ms": round(ms["separate"] - ms["fused"], 4),
           "v_bytes_not_reread": B * Sk * Hkv * D * 2}
    print(json.dumps(out), flush=True)


def natural_ab(args, wl, x, dev):
    """The gathered-list attention against natural-order block skipping on the
    same kernel: the natural-order lists hold every key of each query tile's
    active 64-key tiles (the mask step's block-skip list) under the per-element
    keep test, so both compute the same outputs; the ratio of their times is
    what gathering the kept keys saves."""
    import statistics
    import torch
    import trainable_dynamic_mask_amd as dma
    from trainable_dynamic_mask_amd.blockskip import chunk_counts, natural_order_mask
    delta = dma.weights(x["V"], x["Delta"], x["A"])
    mask = dma.topk_mask(delta, wl.Sq, wl.q_offset, wl.w, kt_lists=True)
    nat = natural_order_mask(mask)
    O_g = torch.empty_like(x["Q"])
    O_n = torch.empty_like(x["Q"])

    def gathered():
        dma.attn_fwd(x["Q"], x["K"], x["V"], delta, mask, out=O_g)

    def natural():
        dma.attn_fwd(x["Q"], x["K"], x["V"], delta, nat, out=O_n)

    def timed(f):
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(args.reps)]
        for a, b in ev:
            a.record()
            f()
            b.record()
        torch.cuda.synchronize()
        return statistics.median(a.elapsed_time(b) for a, b in ev)

    clock_ramp(gathered, args.clock_ramp_ms)
    res = {}
    for _ in range(2):  # interleaved twice: the median of each over both passes
        for name, f in (("gathered", gathered), ("natural", natural)):
            for _ in range(3):
                f()
            res.setdefault(name, []).append(timed(f))
    ms = {k: round(statistics.median(v), 4) for k, v in res.items()}
    torch.cuda.synchronize()
    diff = (O_g.float() - O_n.float()).abs().max().item()
    cg, cn = chunk_counts(mask, nat)
    flop = wl.effective_flops()
    out = {"mode": "natural_ab", "workload": wl.name, "reps": args.reps, "ms": ms,
           "speedup": round(ms["natural"] / ms["gathered"], 3),
           "chunks": {"gathered": cg, "natural": cn}, "work_ratio": round(cn / cg, 3),
           "effective_tflops": {k: round(flop / (v * 1e-3) / 1e12, 1) for k, v in ms.items()},
           "max_abs_diff_outputs": diff}
    print(json.dumps(out), flush=True)


def hbm_stages(args, wl, x, dev):
    """The HBM-bound stages one at a time.  Before every repetition a 512 MiB
    buffer is read and written, which evicts the 256 MB Infinity Cache and the
    L2s, so each repetition reads its inputs from HBM.  Algorithmic bytes:
      weights    V read + delta written
      mask       prefill: delta read + eviction rows and the kept-key / key-tile
                 lists written (their actual lengths); decode (one row): delta
                 of the row's keys read + the w indices written
      attention  decode only (prefill attention is MFMA bound): the kept K and V
                 rows gathered + Q read + O written + indices and their delta
    """
    import statistics
    import torch
    import trainable_dynamic_mask_amd as dma

    lib = dma.load()
    es = x["V"].element_size()
    delta = torch.empty(wl.B, wl.Hkv, wl.Sk, dtype=torch.float32, device=dev)
    mask = dma.alloc_mask(wl.B, wl.Hkv, wl.Sq, wl.Sk, wl.q_offset, wl.w, dev)
    ws_t = torch.empty(max(16, lib.dma_topk_workspace_bytes(wl.B, wl.Hkv, wl.Sq, wl.Sk, wl.w)),
                       dtype=torch.uint8, device=dev)
    O = torch.empty_like(x["Q"])
    ws_a = torch.empty(max(16, lib.dma_attn_workspace_bytes(wl.B, wl.Hq, wl.Sq, wl.D, wl.w)),
                       dtype=torch.uint8, device=dev)
    flush = torch.zeros(512 << 20, dtype=torch.uint8, device=dev)

    def run_w():
        dma.weights(x["V"], x["Delta"], x["A"], out=delta)

    def run_t():
        dma.topk_mask(delta, wl.Sq, wl.q_offset, wl.w, mask=mask, workspace=ws_t)

    def run_a():
        dma.attn_fwd(x["Q"], x["K"], x["V"], delta, mask, out=O, workspace=ws_a)

    def all_stages():
        run_w()
        run_t()
        run_a()

    clock_ramp(all_stages, args.clock_ramp_ms)  # also leaves delta and the mask set
    all_stages()
    torch.cuda.synchronize()
    n_keys = wl.B * wl.Hkv * wl.Sk
    w_bytes = n_keys * wl.D * es + n_keys * 4  # V is [B, Sk, Hkv, D]
    n = mask.dims["n_tiles_total"]
    if wl.Sq == 1:
        rows = wl.B * wl.Hkv
        t_bytes = rows * (wl.q_offset + 1) * 4 + int(mask.u_cnt[:n].sum().item()) * 4
    else:
        t_bytes = (2 * n_keys * 4 + int(mask.u_cnt[:n].sum().item()) * 4
                   + int(mask.kt_cnt[:n].sum().item()) * 4)
    stages = [("weights", run_w, w_bytes), ("mask", run_t, t_bytes)]
    if wl.Sq == 1:
        kept = int(mask.u_cnt[:n].sum().item())
        a_bytes = (kept * 2 * wl.D * es + 2 * wl.B * wl.Hq * wl.D * es + kept * 8)
        stages.append(("attention", run_a, a_bytes))
    out = {"mode": "hbm_stages", "workload": wl.name, "flush_mib": 512, "reps": args.reps,
           "peak_GBps": PEAK_HBM_GBS, "stages": {}}
    for name, fn, nbytes in stages:
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(args.reps)]
        for e0, e1 in ev:
            flush.add_(1)
            e0.record()
            fn()
            e1.record()
        torch.cuda.synchronize()
        ms = [e0.elapsed_time(e1) for e0, e1 in ev]
        med = statistics.median(ms)
        gbs = nbytes / (med * 1e-3) / 1e9
        out["stages"][name] = {"ms_median": round(med, 4), "ms_min": round(min(ms), 4),
                               "bytes": nbytes, "GBps": round(gbs, 1),
                               "frac": round(gbs / PEAK_HBM_GBS, 4)}
    print(json.dumps(out), flush=True)


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}): this build of "
              "the DMA forward is the single-GPU hot path; across GPUs a prefill would shard "
              "by kv-head group and a decode batch by sequence.", file=sys.stderr)
        sys.exit(2)
    if args.copy_calibration:
        copy_calibration(args.copy_calibration)
        return
    import torch
    import trainable_dynamic_mask_amd as dma
    from trainable_dynamic_mask_amd.configs import WORKLOADS
    from trainable_dynamic_mask_amd.inputs import make_inputs

    wl = WORKLOADS[args.workload]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    lib = dma.load()
    x = make_inputs(wl, device=dev)
    if args.backward:
        backward_bench(args, wl, x, dev)
        return
    if args.hbm_stages:
        hbm_stages(args, wl, x, dev)
        return
    if args.vproj:
        vproj_bench(args, wl, x, dev)
        return
    if args.natural_ab:
        natural_ab(args, wl, x, dev)
        return
    delta = torch.empty(wl.B, wl.Hkv, wl.Sk, dtype=torch.float32, device=dev)
    mask = dma.alloc_mask(wl.B, wl.Hkv, wl.Sq, wl.Sk, wl.q_offset, wl.w, dev)
    ws_t = torch.empty(max(16, lib.dma_topk_workspace_bytes(wl.B, wl.Hkv, wl.Sq, wl.Sk, wl.w)),
                       dtype=torch.uint8, device=dev)
    O = torch.empty_like(x["Q"])
    nbytes_a = lib.dma_attn_workspace_bytes(wl.B, wl.Hq, wl.Sq, wl.D, wl.w)
    ws_a = torch.empty(max(16, nbytes_a), dtype=torch.uint8, device=dev)

    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
    ev_stage = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]

    # one query row per sequence (decode): delta of the cache is setup, computed once
    # (a serving loop computes it for each key as the key enters the cache); the
    # timed step is the keep set and the attention
    decode = wl.Sq == 1
    if decode:
        dma.weights(x["V"], x["Delta"], x["A"], out=delta)

    # e: events around the attention (the timed steps: each event record also
    # costs GPU time, so the timed loop records only the two the roofline
    # needs); stage_e: events around every stage (a separate, untimed pass)
    def step(e=None, stage_e=None):
        if stage_e:
            stage_e[0].record()
        if not decode:
            dma.weights(x["V"], x["Delta"], x["A"], out=delta)
        if stage_e:
            stage_e[1].record()
        dma.topk_mask(delta, wl.Sq, wl.q_offset, wl.w, mask=mask, workspace=ws_t)
        if stage_e:
            stage_e[2].record()
        if e:
            e[2].record()
        dma.attn_fwd(x["Q"], x["K"], x["V"], delta, mask, out=O, workspace=ws_a)
        if e:
            e[3].record()
        if stage_e:
            stage_e[3].record()

    clock_ramp(step, args.clock_ramp_ms)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(args.steps):
        step(ev[k])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_step = wall * 1e3 / args.steps
    attn_timed = sum(e[2].elapsed_time(e[3]) for e in ev) / len(ev)
    for k in range(args.steps):
        step(stage_e=ev_stage[k])
    torch.cuda.synchronize()
    import statistics
    per = {"weights": [e[0].elapsed_time(e[1]) for e in ev_stage],
           "mask": [e[1].elapsed_time(e[2]) for e in ev_stage],
           "attention": [e[2].elapsed_time(e[3]) for e in ev_stage]}
    st = {k: sum(v) / len(v) for k, v in per.items()}
    st["attention"] = attn_timed  # the timed steps' own events
    assert torch.isfinite(O.float()).all(), "non-finite output"

    flops = wl.effective_flops()
    value = flops / (ms_step * 1e-3) / 1e12
    attn_tflops = flops / (st["attention"] * 1e-3) / 1e12
    out = {
        "metric": METRIC,
        "value": round(value, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "clock_ramp_ms": args.clock_ramp_ms,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": wl.dtype,
        "data": "synthetic",
        "config": {"workload": wl.name, "B": wl.B, "Hq": wl.Hq, "Hkv": wl.Hkv, "Sq": wl.Sq,
                   "Sk": wl.Sk, "D": wl.D, "w": wl.w, "kept_pairs": wl.kept_pairs(),
                   "effective_flop": flops},
        "roofline": {"bound": "mfma", "kernel": "attn_prefill_bf16_kernel",
                     "achieved": round(attn_tflops, 2), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(attn_tflops / PEAK_BF16_TFLOPS, 4),
                     "traffic": measured_traffic(wl.name)},
        "stages_ms": {k: round(v, 4) for k, v in st.items()},
        "stages_ms_median": {k: round(statistics.median(v), 4) for k, v in per.items()},
        "stages_ms_min": {k: round(min(v), 4) for k, v in per.items()},
    }
    if decode:
        # one query row per sequence: the attention is bound by the HBM gather of the
        # kept K/V rows (plus Q, O, the indices and their delta); the stage covers the
        # gathering kernel and the merge of its splits
        kept = int(mask.u_cnt[:mask.dims["n_tiles_total"]].sum().item())
        es = x["V"].element_size()
        a_bytes = kept * 2 * wl.D * es + 2 * wl.B * wl.Hq * wl.D * es + kept * 8
        gbs = a_bytes / (st["attention"] * 1e-3) / 1e9
        out["roofline"] = {"bound": "hbm", "kernel": "decode_mfma_kernel",
                           "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                           "frac": round(gbs / PEAK_HBM_GBS, 4), "traffic": None}
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(x, wl, args.cpu_seconds)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
