"""Benchmark of the deterministic gradient-reduction hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W]

A step is one pass of all four det_* entry points, each on its synthetic
workload with inputs resident in HBM:
  colsum     gate backward, T = 4 x 2048 x 2 = 16384 tokens, H = 32, bf16, strided dg view
  index_add  4096 query rows x top-k 512 ids (Zipf 1.1 over 8192 keys, 5% padding)
             into an [8192, 128] fp32 dK, bf16 src ~ N(0, 0.02)
  dprob      E = 8 experts, 16384 x 2048 bf16 dY and C, tokens ~ 256 + multinomial
  wgrad      E = 8 experts, T_e ~ U{1024..8192}, main_grad[e] [1408 x 2048] fp32 += G_e^T X_e
The timed region is exactly K steps between two device synchronisations;
``value`` is the step's algorithmic bytes divided by the step time (GB/s).
Per-kernel figures (absolute GB/s or TFLOP/s, fraction of peak, deterministic
over atomic time ratio with a bootstrap 95% CI, 20-replay bit identity) are
measured after the step loop. One JSON line goes to stdout; progress goes to
stderr.
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

HBM_PEAK_GBS = 8000.0
COPY_BYTES = 256 * 1024 * 1024
BF16_MFMA_PEAK_TFLOPS = 2500.0


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--reps", type=int, default=50, help="timed repetitions per kernel for the per-kernel stats")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="after the measurements, copy a 256 MiB buffer three times (a kernel of known traffic, "
                         "against which hardware byte counters are scaled)")
    ap.add_argument("--cpu-seconds", type=float, default=15.0, help="target CPU time of the oracle sample")
    return ap.parse_args()


# ----------------------------------------------------------------- workloads
class Workload:
    """Device inputs and algorithmic cost of one entry point."""

    def __init__(self, name, call_det, call_atomic, reset, read_out, nbytes, flops=0.0, bound="hbm"):
        self.name, self.call_det, self.call_atomic = name, call_det, call_atomic
        self.reset, self.read_out = reset, read_out
        self.nbytes, self.flops, self.bound = nbytes, flops, bound


def build_workloads():
    import torch
    import deterministic_gradient_reductions_amd as dg
    import workloads as W

    def bf(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).cuda().view(torch.bfloat16)

    def f32(x):
        return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).cuda()

    def i32(x):
        return torch.from_numpy(np.ascontiguousarray(x, dtype=np.int32)).cuda()

    out = []
    # colsum: 4 microbatches x 2048 tokens x 2 sequences, 32 heads, strided dg
    g = W.gate_inputs(16384, 32, seed=2, out_init="normal")
    a, dgv = bf(g.a), bf(g.dg_base)[:, 32:]
    Al, db = f32(g.A_log), f32(g.dt_bias)
    o1, o2 = f32(g.dA_log0), f32(g.ddt_bias0)
    o10, o20 = o1.clone(), o2.clone()
    ccfg = dg.det_colsum_select_cfg(16384, 32)
    cws = dg.Workspace(dg.det_colsum_workspace_size(16384, 32, ccfg))
    out.append(Workload(
        "colsum",
        lambda: dg.det_colsum(a, dgv, Al, db, o1, o2, cfg=ccfg, ws=cws),
        lambda: dg.det_colsum(a, dgv, Al, db, o1, o2, cfg=ccfg, atomic=True),
        lambda: (o1.copy_(o10), o2.copy_(o20)),
        lambda: torch.cat([o1, o2]).cpu().numpy(),
        nbytes=16384 * 32 * 4 + 32 * 4 * 6, bound="alu"))
    # index_add
    ia = W.index_add_inputs(seed=3, out_init="normal")
    ids, src, o = i32(ia.ids), bf(ia.src), f32(ia.out0)
    o0 = o.clone()
    icfg = dg.IndexAddCfg(256)
    iws = dg.Workspace(dg.det_index_add_workspace_size(ids.numel(), 128, 8192, icfg))
    n_valid = int(np.count_nonzero(ia.ids >= 0))
    n_touched = int(np.count_nonzero(np.bincount(ia.ids[ia.ids >= 0], minlength=8192)))
    out.append(Workload(
        "index_add",
        lambda: dg.det_index_add(o, ids, src, cfg=icfg, ws=iws),
        lambda: dg.det_index_add(o, ids, src, atomic=True),
        lambda: o.copy_(o0),
        lambda: o.cpu().numpy(),
        nbytes=ids.numel() * 4 + n_valid * 128 * 2 + n_touched * 128 * 4 * 2))
    # dprob
    dp = W.dprob_inputs(seed=4, out_init="normal")
    dY, C, offs, d = bf(dp.dY), bf(dp.C), i32(dp.offs), f32(dp.dprob0)
    d0 = d.clone()
    out.append(Workload(
        "dprob",
        lambda: dg.det_grouped_dprob(d, dY, C, offs),
        lambda: dg.det_grouped_dprob(d, dY, C, offs, atomic=True),
        lambda: d.copy_(d0),
        lambda: d.cpu().numpy(),
        nbytes=16384 * 2048 * 4 + 16384 * 8))
    # wgrad
    wg = W.wgrad_inputs(seed=5, out_init="normal")
    T_total = int(wg.offs[-1])
    G, X, woffs, mg = bf(wg.G), bf(wg.X), i32(wg.offs), f32(wg.main_grad0)
    mg0 = mg.clone()
    wws = dg.Workspace(dg.det_grouped_wgrad_acc_workspace_size(T_total, 8, 1408, 2048))
    out.append(Workload(
        "wgrad",
        lambda: dg.det_grouped_wgrad_acc(mg, G, X, woffs, ws=wws),
        lambda: dg.det_grouped_wgrad_acc(mg, G, X, woffs, atomic=True),
        lambda: mg.copy_(mg0),
        lambda: mg.cpu().numpy(),
        nbytes=T_total * (1408 + 2048) * 2 + 8 * 1408 * 2048 * 4 * 2,
        flops=2.0 * 1408 * 2048 * T_total, bound="mfma"))
    return out


def build_extra_workloads():
    """Entry points measured beside the step (not part of it): grouped dbias at the dprob shapes
    and the canonical compact top-k."""
    import torch
    import deterministic_gradient_reductions_amd as dg
    import workloads as W
    db = W.dbias_inputs(seed=6, out_init="normal")
    dA = torch.from_numpy(np.ascontiguousarray(db.dA).view(np.int16)).cuda().view(torch.bfloat16)
    offs = torch.from_numpy(np.ascontiguousarray(db.offs, dtype=np.int32)).cuda()
    d = torch.from_numpy(db.dbias0).cuda()
    d0 = d.clone()
    dws = dg.Workspace(dg.det_grouped_dbias_workspace_size(db.M, db.N, 8))
    return [Workload(
        "dbias",
        lambda: dg.det_grouped_dbias(d, dA, offs, ws=dws),
        lambda: dg.det_grouped_dbias(d, dA, offs, atomic=True),
        lambda: d.copy_(d0),
        lambda: d.cpu().numpy(),
        nbytes=db.M * db.N * 2 + 8 * db.N * 4 * 2),
        topk_workload()]


def topk_workload():
    """Canonical compact top-k, 4096 rows x 512 slots (deterministic by construction: its
    comparison arm is the same call)."""
    import torch
    import deterministic_gradient_reductions_amd as dg
    import workloads as W
    tk = W.topk_inputs(seed=7)
    ids = torch.from_numpy(tk.ids).cuda()
    lg = torch.from_numpy(tk.logits).cuda()
    io, lo, po = torch.empty_like(ids), torch.empty_like(lg), torch.empty_like(lg)
    call = lambda: dg.det_topk_canonicalize(ids, lg, io, lo, po)
    return Workload("topk_canon", call, call, lambda: po.zero_(),
                    lambda: torch.cat([io.view(torch.float32).flatten(), lo.flatten(), po.flatten()]).cpu().numpy(),
                    nbytes=tk.ids.size * (4 + 4 + 4 + 4 + 4))


# ------------------------------------------------------------------- timing
def bootstrap_ratio_ci(det, atom, n=2000, seed=0):
    rng = np.random.default_rng(seed)
    det, atom = np.asarray(det), np.asarray(atom)
    k = len(det)
    r = [np.median(det[rng.integers(0, k, k)]) / np.median(atom[rng.integers(0, k, k)]) for _ in range(n)]
    return float(np.percentile(r, 2.5)), float(np.percentile(r, 97.5))


def per_kernel(wl, reps, flush):
    import torch
    det_t, atom_t = [], []
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
    for _ in range(3):
        wl.call_det(); wl.call_atomic()
    torch.cuda.synchronize()
    for r in range(reps):
        flush()
        ev[0].record(); wl.call_det(); ev[1].record()
        flush()
        ev[2].record(); wl.call_atomic(); ev[3].record()
        torch.cuda.synchronize()
        det_t.append(ev[0].elapsed_time(ev[1]) * 1e3)
        atom_t.append(ev[2].elapsed_time(ev[3]) * 1e3)
    return np.array(det_t), np.array(atom_t)


def replay_check(wl, n=20):
    """n deterministic replays from the same start state under side-stream load: all bit patterns equal?"""
    import torch
    side = torch.cuda.Stream()
    a = torch.empty(64 * 1024 * 1024, dtype=torch.float32, device="cuda")
    pats, apats = set(), set()
    for i in range(n):
        with torch.cuda.stream(side):
            for _ in range(4):
                a.mul_(1.0000001)
        wl.reset(); wl.call_det()
        torch.cuda.synchronize()
        pats.add(hashlib.sha1(wl.read_out().view(np.uint32).tobytes()).hexdigest())
        with torch.cuda.stream(side):
            for _ in range(4):
                a.mul_(1.0000001)
        wl.reset(); wl.call_atomic()
        torch.cuda.synchronize()
        apats.add(hashlib.sha1(wl.read_out().view(np.uint32).tobytes()).hexdigest())
    wl.reset()
    return len(pats) == 1, len(apats)


# ------------------------------------------------------------- CPU baseline
def cpu_baseline(target_s):
    """Time the CPU oracle, single-threaded, on bounded samples of the same workloads."""
    try:
        from threadpoolctl import threadpool_limits
    except Exception:  # pragma: no cover
        threadpool_limits = None
    import workloads as W
    from oracle import colsum as oc, dprob as od, index_add as oi, wgrad as ow
    samples = []
    ctx = threadpool_limits(1) if threadpool_limits else None
    try:
        t0 = time.perf_counter()
        spent = 0.0
        g = W.gate_inputs(16384, 32, seed=2)
        t = time.perf_counter(); oc.colsum(g.a, g.dg, g.A_log, g.dt_bias, g.dA_log0, g.ddt_bias0, 64)
        samples.append(("colsum T=16384 H=32 (full)", 16384 * 32 * 4, time.perf_counter() - t))
        dp = W.dprob_inputs(seed=4)
        t = time.perf_counter(); od.grouped_dprob(dp.dprob0, dp.dY, dp.C, dp.offs)
        samples.append(("dprob 16384x2048 (full)", 16384 * 2048 * 4 + 16384 * 8, time.perf_counter() - t))
        del dp
        ia = W.index_add_inputs(seed=3)
        nv = int(np.count_nonzero(ia.ids >= 0))
        t = time.perf_counter(); oi.index_add(ia.out0, ia.ids, ia.src, 256)
        samples.append(("index_add 4096x512 -> 8192x128 (full)", ia.ids.size * 4 + nv * 256 + 8192 * 128 * 8,
                        time.perf_counter() - t))
        del ia
        spent = sum(x[2] for x in samples)
        # wgrad: as many experts of the full workload as fit in the remaining compute budget
        wg = W.wgrad_inputs(seed=5)
        done_e, done_tok, t_w = 0, 0, 0.0
        for e in range(8):
            if spent + t_w > target_s:
                break
            t = time.perf_counter()
            ow.grouped_wgrad_acc(wg.main_grad0, wg.G, wg.X, wg.offs, experts=[e])
            t_w += time.perf_counter() - t
            done_e += 1
            done_tok += int(wg.offs[e + 1] - wg.offs[e])
        if done_e:
            samples.append(("wgrad %d of 8 experts, %d tokens (float64 matrix-product chain)" % (done_e, done_tok),
                            done_tok * 3456 * 2 + done_e * 1408 * 2048 * 8, t_w))
        log("cpu oracle: %.1f s of compute, %.1f s with input generation" % (
            sum(x[2] for x in samples), time.perf_counter() - t0))
    finally:
        if ctx is not None:
            ctx.__exit__(None, None, None)
    nbytes = sum(s[1] for s in samples)
    secs = sum(s[2] for s in samples)
    return {"value": round(nbytes / secs / 1e9, 4), "unit": "GB/s", "cores": 1, "kind": "oracle",
            "sample": "; ".join("%s: %.2f s" % (s[0], s[2]) for s in samples)}


def traffic_for(kernel_name):
    """HBM bytes per launch from committed rocprofv3 counter runs, if the kernel source is unchanged."""
    p = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(p):
        return None
    try:
        rec = json.load(open(p)).get(kernel_name)
        src = os.path.join(ROOT, "deterministic_gradient_reductions_amd", "csrc", rec["source"])
        if hashlib.sha1(open(src, "rb").read()).hexdigest() != rec["source_sha1"]:
            return None
        return rec["bytes_per_launch"]
    except Exception:
        return None


# --------------------------------------------------------------------- main
def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py measures one GPU only: this build's reductions run on a single MI355X; "
              "--gpus %d is not supported" % args.gpus, file=sys.stderr)
        sys.exit(2)
    import torch
    torch.cuda.init()
    wls = build_workloads()
    # Cold cache: read a 1 GiB buffer (4x the 256 MB last-level cache) between
    # timed runs. A read leaves only clean lines behind, so the timed kernel
    # pays no write-back of someone else's dirty data.
    flush_buf = torch.ones(1024 * 1024 * 1024 // 4, dtype=torch.float32, device="cuda")
    flush_sink = torch.empty((), dtype=torch.float32, device="cuda")

    def flush():
        torch.sum(flush_buf, dim=0, out=flush_sink)

    log("workloads ready: %s" % [w.name for w in wls])
    stream = torch.cuda.current_stream()
    for _ in range(args.warmup):
        for w in wls:
            w.call_det()
    torch.cuda.synchronize()
    n_ev = args.steps * len(wls)
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n_ev)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    i = 0
    for _ in range(args.steps):
        for w in wls:
            evs[i][0].record(stream); w.call_det(); evs[i][1].record(stream)
            i += 1
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = wall * 1e3 / args.steps
    in_step = {w.name: [] for w in wls}
    for k in range(n_ev):
        in_step[wls[k % len(wls)].name].append(evs[k][0].elapsed_time(evs[k][1]) * 1e3)
    step_bytes = sum(w.nbytes for w in wls)
    log("timed %d steps: %.3f ms/step" % (args.steps, ms_per_step))

    kernels, outside = {}, {}
    extra = build_extra_workloads()
    for w in wls + extra:
        det_cold, atom_cold = per_kernel(w, args.reps, flush)
        det_warm, atom_warm = per_kernel(w, args.reps, lambda: None)
        same, apats = replay_check(w)
        lo, hi = bootstrap_ratio_ci(det_cold, atom_cold)
        med = float(np.median(det_cold))
        k = {
            "us_in_step": round(float(np.mean(in_step[w.name])), 3) if w.name in in_step else None,
            "us_det_cold_median": round(med, 3),
            "us_det_cold_p10_p90": [round(float(np.percentile(det_cold, 10)), 3),
                                    round(float(np.percentile(det_cold, 90)), 3)],
            "us_atomic_cold_median": round(float(np.median(atom_cold)), 3),
            "us_det_warm_median": round(float(np.median(det_warm)), 3),
            "us_atomic_warm_median": round(float(np.median(atom_warm)), 3),
            "det_over_atomic": round(med / float(np.median(atom_cold)), 4),
            "det_over_atomic_ci95": [round(lo, 4), round(hi, 4)],
            "GB_per_s_cold": round(w.nbytes / med / 1e3, 2),
            "frac_hbm_peak_cold": round(w.nbytes / med / 1e3 / HBM_PEAK_GBS, 4),
            "algorithmic_bytes": int(w.nbytes),
            "replay_bit_identical_20": bool(same),
            "atomic_distinct_patterns_20": int(apats),
        }
        if w.flops:
            k["TFLOP_per_s_cold"] = round(w.flops / med / 1e6, 2)
            k["frac_mfma_peak_cold"] = round(w.flops / med / 1e6 / BF16_MFMA_PEAK_TFLOPS, 4)
        (kernels if w.name in in_step else outside)[w.name] = k
        log("%-9s %s" % (w.name, json.dumps(k)))

    # roofline of the dominant kernel: the entry point with the largest share of the step
    dom = max(wls, key=lambda w: np.mean(in_step[w.name]))
    avg_us = float(np.mean(in_step[dom.name]))
    if dom.bound == "mfma":
        roof = {"bound": "mfma", "achieved": round(dom.flops / avg_us / 1e6, 2), "peak": BF16_MFMA_PEAK_TFLOPS,
                "unit": "TFLOP/s"}
    else:
        roof = {"bound": "hbm", "achieved": round(dom.nbytes / avg_us / 1e3, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s"}
    roof["frac"] = round(roof["achieved"] / roof["peak"], 4)
    roof["traffic"] = traffic_for(dom.name)
    roof["kernel"] = dom.name
    roof["avg_launch_us"] = round(avg_us, 3)

    res = {
        "metric": "GB/s (%HBM peak) per det_* kernel; det/atomic time ratio; bitwise replay",
        "value": round(step_bytes / (ms_per_step * 1e-3) / 1e9, 2),
        "unit": "GB/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "f32", "data": "synthetic",
        "config": {"workload": "det_* hot path step: colsum gate bwd T=16384 H=32 (strided dg); "
                               "index_add 4096x512 Zipf(1.1) ids -> 8192x128; dprob E=8 16384x2048; "
                               "wgrad E=8 T_e~U{1024..8192} 1408x2048 fp32 main_grad",
                   "kernels_in_step": [w.name for w in wls], "step_algorithmic_bytes": int(step_bytes),
                   "parallelism": "single GPU"},
        "roofline": roof,
        "kernels": kernels,
        "kernels_outside_step": outside,
    }
    if args.copy_calibration:
        # a plain copy of known size: reads and writes exactly COPY_BYTES each
        src = torch.ones(COPY_BYTES // 4, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        log("copy calibration: 3 copies of %d bytes" % COPY_BYTES)
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(args.cpu_seconds)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
