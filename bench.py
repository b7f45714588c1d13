"""Benchmark of the segmented varlen attention forward on one MI355X.

Default workload: BF16 causal gapped replay, 64 segments of capacity 2048,
used q/k lengths uniform in [0, 2048] (4 segments without keys), 32 q heads /
8 KV heads, d = 128, bottom-right causal.  A step is one gvattn_fwd call
(device plan + attention) over the resident inputs.  The metric is TFLOP/s
over used rows: every visible (query, key) pair costs 4*d FLOPs per query
head; masked, gap and padding work is never counted.

Prints one JSON line.  ``--workload NAME`` benches another workload:
cfg_cross_attention (2 CFG samples of 4096 queries over right-padded text
of 24 and 700 keys), multiview_partitions (8 x 8190 queries over two key
partitions of 16380, the two partition launches plus the LSE merge, or with
``--fused`` one key-range launch over both), large_head_d256 (16 segments
of 16384, d = 256), ulysses_joint (the Ulysses rank-major joint attention of
issue #18687 through the key-range entry point) and decode_batch (32
segments of 4 query rows over 4096-16384 keys, which the plan splits along
the keys; reported against the HBM roofline).
``--dtype fp16`` runs the same workload through the fp16 matrix-core path
(the bf16-exact draws converted to fp16).
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2516.6   # MI355X dense bf16 matrix peak
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
CSRC = os.path.join(ROOT, "segmented_varlen_attention_amd", "csrc")
PMC_SUMMARY = os.path.join(ROOT, "profiles", "fwd_mfma_bf16_causal_replay_64x2048_pmc.md")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


# the sources of the attention forward kernel and of the plan that orders
# its work, which the counters cover
FWD_SOURCES = ("gvattn_fwd_mfma.hip", "gvattn_plan.hip", "gvattn_mfma.h", "gvattn_internal.h")


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for f in FWD_SOURCES:
        with open(os.path.join(CSRC, f), "rb") as fh:
            h.update(f.encode() + b"\0" + fh.read())
    with open(os.path.join(ROOT, "include", "gvattn.h"), "rb") as fh:
        h.update(b"gvattn.h\0" + fh.read())
    return h.hexdigest()[:16]


def recorded_traffic():
    """HBM bytes per launch of the main kernel from the committed rocprofv3
    --pmc summary, if it was taken on the current kernel sources."""
    try:
        text = open(PMC_SUMMARY).read()
    except OSError:
        return None
    for line in text.splitlines():
        if line.startswith("traffic_json:"):
            rec = json.loads(line.split(":", 1)[1])
            if rec.get("kernel_source_sha") == kernel_source_hash():
                return rec
    return None


def algorithmic_bytes(geom, elem=2, keys=None) -> int:
    """Used Q + used O + LSE + used K + used V, each once (``keys``: the
    per-segment key counts when they are not geom.used_k)."""
    uq = int(np.sum(geom.used_q))
    ks = np.asarray(geom.used_k if keys is None else keys)
    uk = int(np.sum(ks[geom.used_q > 0]))
    return (uq * geom.hq * geom.d * elem * 2 + uq * geom.hq * 4
            + uk * geom.hkv * geom.d * elem * 2)


def cpu_baseline(wl, flops_fn, seconds: float, gpu_out=None, gpu_lse=None):
    """The oracle, as it stands, on the same workload: whole passes over all
    segments, repeated until about ``seconds`` of CPU work have run.  The
    first pass's result also gives this run's parity record: the GPU output
    of the timed steps against the oracle over every used row."""
    import oracle
    g = wl.geom
    workers = oracle.host_cores()
    passes, dt = 0, 0.0
    ref = None
    while dt < seconds and passes < 20:
        t0 = time.perf_counter()
        r = oracle.attention_fwd(wl.q, wl.k, wl.v, g.cu_q, g.cu_k, g.used_q, g.used_k,
                                 float(g.scale), g.causal, workers=workers)
        dt += time.perf_counter() - t0
        passes += 1
        if ref is None:
            ref = r
    fl = flops_fn(g.used_q, g.used_k) * passes
    rec = {"value": round(fl / dt / 1e12, 6), "unit": "TFLOP/s", "cores": workers,
           "kind": "oracle",
           "sample": f"{passes} full pass(es) over all {g.nseg} segments and {g.hq} heads of "
                     f"the same workload, {fl / 1e9:.1f} GFLOP in {dt:.1f} s, FP64 NumPy, "
                     f"{workers} worker threads"}
    if gpu_out is not None:
        rec["parity"] = parity_record(wl, ref, gpu_out, gpu_lse)
    return rec


def parity_record(wl, ref, out, lse) -> dict:
    """Per-element comparison of the GPU result with the oracle's on every
    used row: literal max-abs output error, the output-rounding floor
    max|round(O_ref) - O_ref|, the excess over that floor, the LSE error and
    the count of elements whose literal error passes 5e-3."""
    from segmented_varlen_attention_amd import workloads as W
    g = wl.geom
    o_ref, l_ref = ref
    m = np.zeros(g.total_q, bool)
    for s in range(g.nseg):
        m[g.cu_q[s]:g.cu_q[s] + g.used_q[s]] = True
    o_gpu = out.float().cpu().numpy()[m].astype(np.float64)
    l_gpu = lse.cpu().numpy()[:, m].astype(np.float64)
    o_ref, l_ref = o_ref[m], l_ref[:, m]
    err = np.abs(o_gpu - o_ref)
    floor = np.abs(W.round_to(g.dtype, o_ref.astype(np.float32)).astype(np.float64) - o_ref)
    fin = np.isfinite(l_ref)
    return {"rows": int(m.sum()), "max_abs_out_err": float(err.max(initial=0.0)),
            "rounding_floor": float(floor.max(initial=0.0)),
            "excess_over_floor": float((err - floor).max(initial=0.0)),
            "elements_over_5e-3": int(np.count_nonzero(err > 5e-3)),
            "max_abs_lse_err": float(np.abs(l_gpu[fin] - l_ref[fin]).max(initial=0.0)),
            "neg_inf_rows_match": bool(np.array_equal(np.isneginf(l_gpu), np.isneginf(l_ref)))}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=None,
                    help="untimed warmup steps (default: as many as fill --warmup-seconds, "
                         "at least 5)")
    ap.add_argument("--warmup-seconds", type=float, default=0.2,
                    help="default warmup length: after the inputs are written the shader "
                         "clock takes about 50 ms of load to settle")
    ap.add_argument("--settle-seconds", type=float, default=0.25,
                    help="before the warmup, run the step back to back for this long so "
                         "that the timed steps see the steady-state clock (reported as "
                         "'settle'; 0 disables)")
    ap.add_argument("--evict", action="store_true",
                    help="also time launches one by one, each after writing a 512 MiB "
                         "buffer (evicts the 256 MB Infinity Cache)")
    ap.add_argument("--workload", default="causal_replay",
                    choices=["causal_replay", "cfg_cross_attention", "multiview_partitions",
                             "large_head_d256", "ulysses_joint", "decode_batch"])
    ap.add_argument("--fused", action="store_true",
                    help="multiview_partitions: both partitions as key ranges of one launch")
    ap.add_argument("--dtype", default="bf16", choices=["bf16", "fp16"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-bwd", action="store_true",
                    help="skip the backward (gvattn_bwd) record")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run a plain device-to-device copy of MIB MiB (5 times), the "
                         "reference for scaling rocprofv3 FETCH_SIZE / WRITE_SIZE")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: there is no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import torch

    import segmented_varlen_attention_amd as gv
    from segmented_varlen_attention_amd import workloads as W

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    gv.load_library()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    if args.copy_calibration:
        n = args.copy_calibration << 20
        src = torch.ones(n, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes": n, "launches": 5}))
        return

    t0 = time.time()
    wk = args.workload
    wl = (W.ulysses_joint() if wk == "ulysses_joint" else
          W.decode_batch() if wk == "decode_batch" else W.WORKLOADS[wk]())
    g = wl.geom
    fused = wk == "multiview_partitions" and args.fused
    if fused:
        (cu_a, used_a), (cu_b, used_b) = wl.partitions
        wl.key_ranges = (np.arange(0, 2 * g.nseg + 1, 2, dtype=np.int32),
                         np.stack([cu_a[:-1], cu_b[:-1]], 1).reshape(-1).astype(np.int32),
                         np.stack([used_a, used_b], 1).reshape(-1).astype(np.int32))
    log(f"[bench] workload {wl.name} generated in {time.time() - t0:.1f}s")

    def flops_of(uq, uk):
        pairs = 0
        for a, b in zip(uq, uk):
            a, b = int(a), int(b)
            if a == 0 or b == 0:
                continue
            if g.causal:
                i = np.arange(a)
                pairs += int(np.clip(i + b - a + 1, 0, b).sum())
            else:
                pairs += a * b
        return pairs * g.hq * (2 * g.d + 2 * g.dv)

    if wl.key_ranges is not None:
        kr_lens = [int(np.sum(wl.key_ranges[2][wl.key_ranges[0][s]:wl.key_ranges[0][s + 1]]))
                   for s in range(g.nseg)]
        flops = flops_of(g.used_q, kr_lens)
    else:
        flops = flops_of(g.used_q, g.used_k)
    tdt = torch.bfloat16 if args.dtype == "bf16" else torch.float16
    dcode = gv.GVATTN_BF16 if args.dtype == "bf16" else gv.GVATTN_FP16
    up = lambda x: torch.from_numpy(np.ascontiguousarray(x)).to(dev)  # noqa: E731
    q, k, v = up(wl.q).to(tdt), up(wl.k).to(tdt), up(wl.v).to(tdt)
    cu_q, used_q = up(g.cu_q), up(g.used_q)
    out = torch.full((g.total_q, g.hq, g.dv), W.SENTINEL, dtype=tdt, device=dev)
    lse = torch.full((g.hq, g.total_q), W.SENTINEL, dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream()

    if wl.key_ranges is not None:
        kr = tuple(up(x) for x in wl.key_ranges)
        launches = []
        parts = [(out, lse)]
        wss = [gv.alloc_workspace(g.nseg, g.total_q, g.hq, g.hkv, g.d, dcode, d_v=g.dv)]
    elif wk == "multiview_partitions":
        launches = [(up(cu), up(u)) for cu, u in wl.partitions]
        parts = [(torch.empty_like(out), torch.empty_like(lse)) for _ in launches]
        wss = [gv.alloc_workspace(g.nseg, g.total_q, g.hq, g.hkv, g.d, dcode, d_v=g.dv)
               for _ in launches]
    else:
        launches = [(up(g.cu_k), up(g.used_k))]
        parts = [(out, lse)]
        wss = [gv.alloc_workspace(g.nseg, g.total_q, g.hq, g.hkv, g.d, dcode, d_v=g.dv)]

    def step():
        if wl.key_ranges is not None:
            gv.gvattn_fwd_ranges(q, k, v, cu_q, used_q, *kr, out, lse, float(g.scale), g.causal,
                                 workspace=wss[0])
            return
        for (cu_k, used_k), (o, l), ws in zip(launches, parts, wss):
            gv.gvattn_fwd(q, k, v, cu_q, cu_k, used_q, used_k, o, l, float(g.scale), g.causal,
                          workspace=ws)
        if wk == "multiview_partitions":
            gv.gvattn_lse_merge([p[0] for p in parts], [p[1] for p in parts], cu_q, used_q, out,
                                lse)

    def run_only():
        if wl.key_ranges is not None:  # no separate plan: the whole call
            step()
            return
        (cu_k, used_k), (o, l), ws = launches[0], parts[0], wss[0]
        gv.gvattn_fwd_run(q, k, v, cu_q, cu_k, used_q, used_k, o, l, float(g.scale), g.causal,
                          ws)

    if wk == "multiview_partitions" and not fused:
        flops = sum(flops_of(g.used_q, u) for _, u in wl.partitions)

    # Clock settle.  Right after the input upload and the sentinel fills (or
    # any idle gap) the part's power management holds the shader clock low:
    # the first 50-75 steps run up to 35% slower.  The settle phase runs the
    # same step back to back for --settle-seconds before the warmup, so that
    # the W warmup steps and the K timed steps see the steady-state clock;
    # the record reports it separately from "warmup".
    settle_steps, t_s = 0, time.perf_counter()
    while args.settle_seconds > 0 and time.perf_counter() - t_s < args.settle_seconds:
        for _ in range(5):
            step()
        settle_steps += 5
        torch.cuda.synchronize()
    settle_s = time.perf_counter() - t_s
    if args.warmup is not None:
        for _ in range(args.warmup):
            step()
        torch.cuda.synchronize()
    else:
        args.warmup, t_w = 0, time.perf_counter()
        while args.warmup < 5 or time.perf_counter() - t_w < args.warmup_seconds:
            for _ in range(5):
                step()
            args.warmup += 5
            torch.cuda.synchronize()
    log(f"[bench] settle {settle_steps} steps ({settle_s:.2f} s), {args.warmup} warmup steps")

    def timed(fn, n):
        """n back-to-back calls with an event on the stream before each one
        and after the last: (mean, median, min) ms per call."""
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(n + 1)]
        ev[0].record(stream)
        for i in range(n):
            fn()
            ev[i + 1].record(stream)
        torch.cuda.synchronize()
        per = np.array([ev[i].elapsed_time(ev[i + 1]) for i in range(n)])
        return ev[0].elapsed_time(ev[n]) / n, float(np.median(per)), float(per.min())

    torch.cuda.synchronize()
    t_wall = time.perf_counter()
    ms, med_ms, min_ms = timed(step, args.steps)
    wall = time.perf_counter() - t_wall
    log(f"[bench] {args.steps} steps: {ms:.4f} ms/step (events; median {med_ms:.4f}, "
        f"min {min_ms:.4f}), wall {wall * 1e3 / args.steps:.4f} ms/step")

    # main attention kernel alone: the plan stays in the workspace; the
    # host-side gap after the timed steps (event readout) is bridged by a
    # short settle of the same launch
    t_s = time.perf_counter()
    while time.perf_counter() - t_s < min(0.1, args.settle_seconds):
        for _ in range(5):
            run_only()
        torch.cuda.synchronize()
    run_only()
    kern_ms, kern_med, kern_min = timed(run_only, args.steps)
    kern_flops = (flops_of(g.used_q, launches[0][1].cpu().numpy())
                  if (wk == "multiview_partitions" and not fused) else flops)
    log(f"[bench] main kernel alone: {kern_ms:.4f} ms/launch (median {kern_med:.4f}, "
        f"min {kern_min:.4f})")

    evict_rec = None
    if args.evict:
        # one launch at a time after a 512 MiB write: the step as seen from
        # a cold Infinity Cache (and after memory-heavy work, which also
        # lowers the clock for the next tens of ms)
        scratch = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
        per = []
        for _ in range(args.steps):
            scratch.fill_(1)
            a0, a1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a0.record(stream)
            step()
            a1.record(stream)
            torch.cuda.synchronize()
            per.append(a0.elapsed_time(a1))
        per = np.array(per)
        evict_rec = {"launches": args.steps, "mean_ms": round(float(per.mean()), 5),
                     "median_ms": round(float(np.median(per)), 5),
                     "min_ms": round(float(per.min()), 5),
                     "median_TFLOP_per_s": round(flops / (np.median(per) * 1e-3) / 1e12, 3)}
        log(f"[bench] after 512 MiB eviction: median {evict_rec['median_ms']:.4f} ms")
        del scratch

    merge_rec = None
    if wk == "multiview_partitions" and not fused:
        # the LSE merge alone: algorithmic bytes = both partials, the output
        # and the LSEs, used rows only
        pouts, plses = [p[0] for p in parts], [p[1] for p in parts]
        merge_ms, merge_med, merge_min = timed(
            lambda: gv.gvattn_lse_merge(pouts, plses, cu_q, used_q, out, lse), args.steps)
        uq = int(np.sum(g.used_q))
        mbytes = uq * g.hq * (len(parts) * (g.dv * 2 + 4) + g.dv * 2 + 4)
        merge_rec = {"ms": round(merge_ms, 5), "median_ms": round(merge_med, 5),
                     "min_ms": round(merge_min, 5), "algorithmic_bytes": mbytes,
                     "GB_per_s": round(mbytes / (merge_ms * 1e-3) / 1e9, 1),
                     "frac_of_hbm_peak": round(mbytes / (merge_ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)}
        log(f"[bench] LSE merge alone: {merge_ms:.4f} ms, {merge_rec['GB_per_s']} GB/s")

    bwd_rec = None
    if (not args.no_bwd and wl.key_ranges is None and wk != "multiview_partitions" and g.d <= 128
            and g.dv <= 128):
        # gradients of the same step: dO seeded, O / LSE from the forward
        # above; FLOPs counted as the five products of the calculus (S, dP,
        # dV, dQ, dK), although the kernels recompute S and dP once more
        dout = up(W.normal_tensor(wl.seed, 7, (g.total_q, g.hq, g.dv), 1.0, args.dtype)).to(tdt)
        dq, dk, dvv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
        (cu_k0, used_k0), (o0, l0), _ = launches[0], parts[0], wss[0]
        step()
        bws = gv.gvattn_bwd(q, k, v, o0, dout, l0, cu_q, cu_k0, used_q, used_k0, dq, dk, dvv,
                            float(g.scale), g.causal)
        for _ in range(max(1, args.warmup)):
            gv.gvattn_bwd(q, k, v, o0, dout, l0, cu_q, cu_k0, used_q, used_k0, dq, dk, dvv,
                          float(g.scale), g.causal, workspace=bws)
        bwd_ms, bwd_med, bwd_min = timed(
            lambda: gv.gvattn_bwd(q, k, v, o0, dout, l0, cu_q, cu_k0, used_q, used_k0, dq, dk,
                                  dvv, float(g.scale), g.causal, workspace=bws), args.steps)
        bflops = flops // (2 * g.d + 2 * g.dv) * (6 * g.d + 4 * g.dv)
        btf = bflops / (bwd_ms * 1e-3) / 1e12
        bwd_rec = {"ms": round(bwd_ms, 5), "median_ms": round(bwd_med, 5),
                   "min_ms": round(bwd_min, 5), "flop": bflops, "TFLOP_per_s": round(btf, 3),
                   "frac_of_peak": round(btf / PEAK_BF16_TFLOPS, 4)}
        log(f"[bench] backward: {bwd_ms:.4f} ms, {btf:.1f} TFLOP/s")
        del dout, dq, dk, dvv, bws

    tflops = flops / (ms * 1e-3) / 1e12
    achieved = kern_flops / (kern_ms * 1e-3) / 1e12
    traffic_rec = recorded_traffic() if (wk == "causal_replay" and args.dtype == "bf16") else None
    roofline = {"bound": "mfma", "achieved": round(achieved, 3), "peak": PEAK_BF16_TFLOPS,
                "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                "traffic": (traffic_rec["bytes_per_launch"] if traffic_rec else None)}
    if wk == "decode_batch":  # memory-bound: algorithmic bytes over the whole call
        gbs = algorithmic_bytes(g) / (kern_ms * 1e-3) / 1e9
        roofline = {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS,
                    "unit": "GB/s", "frac": round(gbs / PEAK_HBM_GBS, 4), "traffic": None}
    alg_bytes = algorithmic_bytes(g, keys=kr_lens if wl.key_ranges is not None else None)
    names = {"cfg_cross_attention": "bf16_cfg_cross_attn_b2_4096q_text24_700_gqa32x8_d128",
             "causal_replay": "bf16_causal_gapped_replay_64x2048_gqa32x8_d128",
             "multiview_partitions": "bf16_multiview_8x8190q_32760k_2partitions_merge_gqa24x8_d128",
             "large_head_d256": "bf16_gapped_16x16384_gqa16x4_d256",
             "ulysses_joint": "bf16_ulysses2_rank_major_joint_b2_4096q_text4096_video4096_keyranges",
             "decode_batch": "bf16_decode_b32x4_k4096_16384_gqa32x8_d128_causal_splitk"}
    res = {
        "metric": "gapped varlen attn fwd TFLOP/s (used rows) + % of MI355X bf16 MFMA peak",
        "value": round(tflops, 3), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 5), "median_ms": round(med_ms, 5),
        "min_ms": round(min_ms, 5),
        "settle": {"steps": settle_steps, "seconds": round(settle_s, 3)},
        "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": args.dtype, "data": "synthetic",
        "config": {"workload": names[wk].replace("bf16", args.dtype, 1)
                   + ("_fused_keyranges" if fused else ""),
                   "segments": g.nseg,
                   "used_q_rows": int(np.sum(g.used_q)), "hq": g.hq, "hkv": g.hkv, "d": g.d,
                   "causal": bool(g.causal), "flop_per_step": flops,
                   "pct_of_bf16_peak": round(100 * tflops / PEAK_BF16_TFLOPS, 2),
                   "algorithmic_hbm_bytes": alg_bytes},
        "roofline": roofline,
        "kernel_alone": {"ms": round(kern_ms, 5), "median_ms": round(kern_med, 5),
                         "min_ms": round(kern_min, 5),
                         # the same launch against the HBM roofline: used inputs and
                         # outputs, each once, over the mean launch time
                         "hbm_GB_per_s": round(alg_bytes / (kern_ms * 1e-3) / 1e9, 1),
                         "frac_of_hbm_peak": round(alg_bytes / (kern_ms * 1e-3) / 1e9
                                                   / PEAK_HBM_GBS, 4)},
    }
    if evict_rec is not None:
        res["evict"] = evict_rec
    if merge_rec is not None:
        res["merge"] = merge_rec
    if bwd_rec is not None:
        res["backward"] = bwd_rec
    if not args.no_cpu_baseline and wk == "causal_replay" and args.dtype == "bf16":
        log("[bench] timing the oracle on a bounded sample ...")
        # the output buffers hold the last timed launch's result
        res["cpu_baseline"] = cpu_baseline(wl, flops_of, args.cpu_seconds, out, lse)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
