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
over atomic time ratio with a bootstrap 95% CI, 20-replay bit identity and the
atomic arm's count of distinct results) are measured after the step loop, and
beside the step: grouped dbias, the canonical top-k, the gate backward at
T = 4096 x H = 16 and at T = 4,194,304 x H = 32 (a bandwidth-sized companion)
and every gate tile configuration. One JSON line goes to stdout; progress goes
to stderr.

    python bench.py --only wgrad --steps 20   # one entry point, K timed calls (for profilers)
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
    ap.add_argument("--only", default="", help="comma-separated entry points: run only their deterministic calls "
                    "(warmup + steps), print their mean times and exit (for profiler runs)")
    return ap.parse_args()


# ----------------------------------------------------------------- workloads
class Workload:
    """Device inputs and algorithmic cost of one entry point."""

    def __init__(self, name, call_det, call_atomic, reset, read_out, nbytes, flops=0.0, bound="hbm", note="",
                 extra_arms=None, valu_ops=0.0):
        self.name, self.call_det, self.call_atomic = name, call_det, call_atomic
        self.reset, self.read_out = reset, read_out
        self.nbytes, self.flops, self.bound = nbytes, flops, bound
        self.note = note                    # what the atomic arm is
        self.extra_arms = extra_arms or {}  # label -> (det call, atomic call) timed the same way
        self.valu_ops = valu_ops            # VALU lane-operations per call (ALU-bound kernels)


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
    # The comparison arm is split-K with float atomics, 4 K tiles (2048 rows) per split: with one split per
    # expert every element receives a single atomic add per call and the arm is bit-stable, so the smallest
    # splits whose results vary from run to run (1, 2 or 4 K tiles; 4 is the fastest) are the honest arm.
    split4 = dg.WgradCfg(256, 256, 512, 4)
    ws4 = dg.Workspace(dg.det_grouped_wgrad_acc_workspace_size(T_total, 8, 1408, 2048, split4))
    out.append(Workload(
        "wgrad",
        lambda: dg.det_grouped_wgrad_acc(mg, G, X, woffs, ws=wws),
        lambda: dg.det_grouped_wgrad_acc(mg, G, X, woffs, cfg=split4, atomic=True),
        lambda: mg.copy_(mg0),
        lambda: mg.cpu().numpy(),
        nbytes=T_total * (1408 + 2048) * 2 + 8 * 1408 * 2048 * 4 * 2,
        flops=2.0 * 1408 * 2048 * T_total, bound="mfma",
        note="deterministic: default call (one split per expert); atomic: split-K with 4 K tiles per split",
        extra_arms={"same_split_4": (lambda: dg.det_grouped_wgrad_acc(mg, G, X, woffs, cfg=split4, ws=ws4),
                                     lambda: dg.det_grouped_wgrad_acc(mg, G, X, woffs, cfg=split4, atomic=True))}))
    return out


def build_extra_workloads():
    """Entry points measured beside the step (not part of it): grouped dbias at the dprob shapes, the
    canonical compact top-k, and the gate backward at the small size and at the bandwidth companion."""
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
        topk_workload(), indexer_dk_workload(), colsum_workload(4096, 16, "colsum_tiny"),
        colsum_workload(4 * 1024 * 1024, 32, "colsum_companion", device_inputs=True)]


# VALU lane-operations per (t, h) element of the gate backward: the VALU instructions the colsum kernel
# executes per element (the detmath sequences of exp, log1p and two divisions, the two products and the
# pairwise tree), measured with the SQ_INSTS_VALU counter at the bandwidth-sized companion: 173,080,576 wave
# instructions x 64 lanes / (4,194,304 x 32) elements. The fold kernel's are not included; the rate below
# divides by the whole call (both kernels).
COLSUM_VALU_OPS_PER_ELEM = 82.5
# fp32 VALU lane-operations per second: the published fp32 vector rate, 157.3 TFLOP/s with an FMA counted as
# two flops, is 78.6 T lane-operations/s (256 CUs x 128 lanes per clock x 2.4 GHz). Non-packed code reaches
# more than half of it (the gate kernel issues 46.8 T/s by SQ_INSTS_VALU), so the wave64 VALU instruction
# takes two cycles, not four, on these compute units.
VALU_PEAK_TOPS = 256 * 128 * 2.4e9 / 1e12


def colsum_workload(T, H, name, device_inputs=False, cfg=None):
    """The gate backward at another size (beside the step). ``device_inputs`` draws a and dg on the GPU
    (the bandwidth companion has 512 MiB of inputs; its results are timed, not compared)."""
    import torch
    import deterministic_gradient_reductions_amd as dg
    import workloads as W
    if device_inputs:
        gen = torch.Generator(device="cuda").manual_seed(11)
        a = torch.randn((T, H), generator=gen, device="cuda").to(torch.bfloat16)
        dgv = torch.randn((T, 2 * H), generator=gen, device="cuda").to(torch.bfloat16)[:, H:]
        Al = torch.empty(H, device="cuda").uniform_(-2.0, 1.0, generator=gen)
        db = torch.empty(H, device="cuda").uniform_(-1.0, 1.0, generator=gen)
        o1, o2 = torch.zeros(H, device="cuda"), torch.zeros(H, device="cuda")
    else:
        g = W.gate_inputs(T, H, seed=1, out_init="normal")
        bf = lambda b: torch.from_numpy(np.ascontiguousarray(b).view(np.int16)).cuda().view(torch.bfloat16)
        a, dgv = bf(g.a), bf(g.dg_base)[:, H:]
        Al, db = torch.from_numpy(g.A_log).cuda(), torch.from_numpy(g.dt_bias).cuda()
        o1, o2 = torch.from_numpy(g.dA_log0).cuda(), torch.from_numpy(g.ddt_bias0).cuda()
    o10, o20 = o1.clone(), o2.clone()
    c = cfg or dg.det_colsum_select_cfg(T, H)
    ws = dg.Workspace(dg.det_colsum_workspace_size(T, H, c))
    return Workload(
        name,
        lambda: dg.det_colsum(a, dgv, Al, db, o1, o2, cfg=c, ws=ws),
        lambda: dg.det_colsum(a, dgv, Al, db, o1, o2, cfg=c, atomic=True),
        lambda: (o1.copy_(o10), o2.copy_(o20)),
        lambda: torch.cat([o1, o2]).cpu().numpy(),
        nbytes=T * H * 4 + H * 4 * 6, bound="alu", note="tile %dx%d" % (c.block_t, c.block_h),
        valu_ops=COLSUM_VALU_OPS_PER_ELEM * T * H)


def indexer_dk_workload():
    """The fused sparse-indexer dK: 4096 query rows x top-k 512 Zipf ids into 8192 x 128, source rows made
    from the clipped-KL score gradient and the bf16 query rows (no stored source rows)."""
    import torch
    import deterministic_gradient_reductions_amd as dg
    import workloads as W
    x = W.indexer_dk_inputs(seed=8, out_init="normal")
    ids = torch.from_numpy(x.ids).cuda()
    p, t = torch.from_numpy(x.predict).cuda(), torch.from_numpy(x.target).cuda()
    q = torch.from_numpy(np.ascontiguousarray(x.q).view(np.int16)).cuda().view(torch.bfloat16)
    dk = torch.from_numpy(x.dk0).cuda()
    dk0 = dk.clone()
    cfg = dg.IndexAddCfg(256)
    ws = dg.Workspace(dg.det_indexer_dk_workspace_size(4096, 512, 128, 8192, cfg))
    wsa = dg.Workspace(dg.det_indexer_dk_workspace_size(4096, 512, 128, 8192, cfg, atomic=True))
    n_touched = int(np.count_nonzero(np.bincount(x.ids[x.ids >= 0], minlength=8192)))
    return Workload(
        "indexer_dk",
        lambda: dg.det_indexer_dk(dk, ids, p, t, q, x.scale, cfg=cfg, ws=ws),
        lambda: dg.det_indexer_dk(dk, ids, p, t, q, x.scale, cfg=cfg, atomic=True, ws=wsa),
        lambda: dk.copy_(dk0),
        lambda: dk.cpu().numpy(),
        nbytes=x.ids.size * 12 + 4096 * 128 * 2 + n_touched * 128 * 8,
        note="ids, predict, target per slot + the query rows once + touched dK rows read and written")


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
    return Workload("topk_canon", call, None, lambda: po.zero_(),
                    lambda: torch.cat([io.view(torch.float32).flatten(), lo.flatten(), po.flatten()]).cpu().numpy(),
                    nbytes=tk.ids.size * (4 + 4 + 4 + 4 + 4))


# ------------------------------------------------------------------- timing
def bootstrap_ratio_ci(det, atom, n=2000, seed=0):
    rng = np.random.default_rng(seed)
    det, atom = np.asarray(det), np.asarray(atom)
    k = len(det)
    r = [np.median(det[rng.integers(0, k, k)]) / np.median(atom[rng.integers(0, k, k)]) for _ in range(n)]
    return float(np.percentile(r, 2.5)), float(np.percentile(r, 97.5))


def time_pairs(call_det, call_atomic, reps, flush):
    """HIP-event times (us) of both arms, interleaved in pairs; call_atomic may be None."""
    import torch
    det_t, atom_t = [], []
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
    for _ in range(3):
        call_det()
        if call_atomic:
            call_atomic()
    torch.cuda.synchronize()
    for r in range(reps):
        flush()
        ev[0].record(); call_det(); ev[1].record()
        if call_atomic:
            flush()
            ev[2].record(); call_atomic(); ev[3].record()
        torch.cuda.synchronize()
        det_t.append(ev[0].elapsed_time(ev[1]) * 1e3)
        if call_atomic:
            atom_t.append(ev[2].elapsed_time(ev[3]) * 1e3)
    return np.array(det_t), np.array(atom_t)


def replay_check(wl, n=20):
    """n deterministic replays from the same start state under side-stream load: all bit patterns equal?
    Also the number of distinct results of the atomic arm over n runs (None without an atomic arm)."""
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
        if wl.call_atomic is None:
            continue
        with torch.cuda.stream(side):
            for _ in range(4):
                a.mul_(1.0000001)
        wl.reset(); wl.call_atomic()
        torch.cuda.synchronize()
        apats.add(hashlib.sha1(wl.read_out().view(np.uint32).tobytes()).hexdigest())
    wl.reset()
    return len(pats) == 1, (len(apats) if wl.call_atomic is not None else None)


def kernel_record(w, reps, flush, in_step_us=None):
    det_cold, atom_cold = time_pairs(w.call_det, w.call_atomic, reps, flush)
    det_warm, atom_warm = time_pairs(w.call_det, w.call_atomic, reps, lambda: None)
    same, apats = replay_check(w)
    med = float(np.median(det_cold))
    k = {
        "us_in_step": round(float(in_step_us), 3) if in_step_us is not None else None,
        "us_det_cold_median": round(med, 3),
        "us_det_cold_p10_p90": [round(float(np.percentile(det_cold, 10)), 3),
                                round(float(np.percentile(det_cold, 90)), 3)],
        "us_det_warm_median": round(float(np.median(det_warm)), 3),
        "GB_per_s_cold": round(w.nbytes / med / 1e3, 2),
        "frac_hbm_peak_cold": round(w.nbytes / med / 1e3 / HBM_PEAK_GBS, 4),
        "algorithmic_bytes": int(w.nbytes),
        "replay_bit_identical_20": bool(same),
    }
    if w.call_atomic is not None:
        lo, hi = bootstrap_ratio_ci(det_cold, atom_cold)
        k.update({
            "us_atomic_cold_median": round(float(np.median(atom_cold)), 3),
            "us_atomic_warm_median": round(float(np.median(atom_warm)), 3),
            "det_over_atomic": round(med / float(np.median(atom_cold)), 4),
            "det_over_atomic_ci95": [round(lo, 4), round(hi, 4)],
            "atomic_distinct_patterns_20": int(apats),
        })
    else:
        k["atomic_arm"] = None  # deterministic by construction, nothing is accumulated
    if w.note:
        k["note"] = w.note
    if w.flops:
        k["TFLOP_per_s_cold"] = round(w.flops / med / 1e6, 2)
        k["frac_mfma_peak_cold"] = round(w.flops / med / 1e6 / BF16_MFMA_PEAK_TFLOPS, 4)
    if w.valu_ops:
        k["valu_Tops_cold"] = round(w.valu_ops / med / 1e6, 2)
        k["frac_valu_peak_cold"] = round(w.valu_ops / med / 1e6 / VALU_PEAK_TOPS, 4)
    for label, (cd, ca) in w.extra_arms.items():
        d2, a2 = time_pairs(cd, ca, reps, flush)
        lo, hi = bootstrap_ratio_ci(d2, a2)
        k[label] = {"us_det_cold_median": round(float(np.median(d2)), 3),
                    "us_atomic_cold_median": round(float(np.median(a2)), 3),
                    "det_over_atomic": round(float(np.median(d2) / np.median(a2)), 4),
                    "det_over_atomic_ci95": [round(lo, 4), round(hi, 4)]}
    return k


def colsum_tile_sweep(reps, flush):
    """Cold median (us) of the deterministic gate backward at T = 16384, H = 32 (strided dg) for every tile
    configuration block_t x block_h in {64, 128, 256} x {8, 16, 32}."""
    import deterministic_gradient_reductions_amd as dg
    out = {}
    for bt in (64, 128, 256):
        for bh in (8, 16, 32):
            w = colsum_workload(16384, 32, "sweep", cfg=dg.ColsumCfg(bt, bh))
            d, _ = time_pairs(w.call_det, None, reps, flush)
            out["%dx%d" % (bt, bh)] = round(float(np.median(d)), 3)
    return out


def library_reference(reps, flush):
    """Context for the weight-gradient fraction (not a comparison arm): the library GEMM (torch.mm, which
    runs hipBLASLt) in bf16 on the same expert products one expert at a time (G_e^T made contiguous
    beforehand; a bf16 result and no accumulate, so it does less work than the entry point), and on a
    square 8192 x 8192 x 8192 product, with operands of the workload's magnitude (N(0, 0.02) bf16)."""
    import torch
    import workloads as W
    wg = W.wgrad_inputs(seed=5)
    offs = [int(v) for v in wg.offs]
    G = torch.from_numpy(np.ascontiguousarray(wg.G).view(np.int16)).cuda().view(torch.bfloat16)
    X = torch.from_numpy(np.ascontiguousarray(wg.X).view(np.int16)).cuda().view(torch.bfloat16)
    E = len(offs) - 1
    Gt = [G[offs[e]:offs[e + 1]].t().contiguous() for e in range(E)]
    Xe = [X[offs[e]:offs[e + 1]] for e in range(E)]
    outs = [torch.empty((wg.M, wg.N), dtype=torch.bfloat16, device="cuda") for _ in range(E)]

    def experts():
        for e in range(E):
            torch.mm(Gt[e], Xe[e], out=outs[e])
    d, _ = time_pairs(experts, None, reps, flush)
    f = 2.0 * wg.M * wg.N * offs[-1]
    gen = torch.Generator(device="cuda").manual_seed(12)
    A = (torch.randn((8192, 8192), generator=gen, device="cuda") * 0.02).to(torch.bfloat16)
    B = (torch.randn((8192, 8192), generator=gen, device="cuda") * 0.02).to(torch.bfloat16)
    C = torch.empty((8192, 8192), dtype=torch.bfloat16, device="cuda")
    d2, _ = time_pairs(lambda: torch.mm(A, B, out=C), None, max(5, reps // 5), flush)
    f2 = 2.0 * 8192 ** 3
    m, m2 = float(np.median(d)), float(np.median(d2))
    return {"library": "torch.mm (hipBLASLt), bf16 operands N(0, 0.02), bf16 result",
            "wgrad_experts_one_at_a_time_us": round(m, 3),
            "wgrad_experts_frac_mfma_peak": round(f / m / 1e6 / BF16_MFMA_PEAK_TFLOPS, 4),
            "square_8192_us": round(m2, 3),
            "square_8192_frac_mfma_peak": round(f2 / m2 / 1e6 / BF16_MFMA_PEAK_TFLOPS, 4)}


def measured_ceilings(flush, reps=5):
    """What this machine delivers, measured beside the kernels (context for the fractions of the published
    peaks): the matrix cores alone (det_mfma_rate: the weight gradient's 4 x 4 MFMA pattern from registers,
    one workgroup per compute unit, about 5 ms per launch) on operands of the workload's magnitude
    (N(0, 0.02) bf16) and on constant operands (every value 1.0); and a plain device copy (cold) of the
    dprob workload's size (134 MB) and of 1 GiB, counting the bytes read and written."""
    import torch
    import deterministic_gradient_reductions_amd as dg
    blocks = torch.cuda.get_device_properties(0).multi_processor_count
    iters = 16384
    flops = float(blocks) * 4 * iters * 16 * 32768
    out = torch.empty(blocks * 256, dtype=torch.float32, device="cuda")
    gen = torch.Generator(device="cuda").manual_seed(13)
    n_ops = 64 * 64 * 64
    res = {}
    for name, ops in (("mfma_random_bf16", (torch.randn(n_ops, generator=gen, device="cuda") * 0.02).to(torch.bfloat16)),
                      ("mfma_constant_bf16", torch.ones(n_ops, dtype=torch.bfloat16, device="cuda"))):
        d, _ = time_pairs(lambda: dg.det_mfma_rate(ops, out, blocks, iters), None, reps, lambda: None)
        med = float(np.median(d))
        res[name] = {"TFLOP_per_s": round(flops / med / 1e6, 1),
                     "frac_mfma_peak": round(flops / med / 1e6 / BF16_MFMA_PEAK_TFLOPS, 4)}
    for name, n in (("hbm_copy_134MB", 16384 * 2048), ("hbm_copy_1GiB", 256 * 1024 * 1024)):
        x = torch.ones(n, dtype=torch.float32, device="cuda")
        y = torch.empty_like(x)
        d, _ = time_pairs(lambda: y.copy_(x), None, max(reps, 10), flush)
        med = float(np.median(d))
        res[name] = {"GB_per_s": round(2 * n * 4 / med / 1e3, 1),
                     "frac_hbm_peak": round(2 * n * 4 / med / 1e3 / HBM_PEAK_GBS, 4)}
        del x, y
    res["note"] = ("matrix cores: the weight gradient's MFMA pattern from registers with no memory traffic; "
                   "copies: a cold float32 device copy, read plus written bytes")
    return res


# ------------------------------------------------------------- CPU baseline
def _cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(target_s):
    """Time the CPU oracle on the host's cores, on bounded samples of the step's workloads.

    The oracle is run as it stands; independent parts go to a thread pool (numpy releases the GIL): gate
    heads and dprob rows are independent, index_add is one call (its stable sort spans all ids), and the
    matrix-core chains of the weight gradient run in the oracle's C file on OpenMP threads. The weight gradient is sampled (output rows of
    every expert) and scaled to the full problem by the sampled fraction of its chains."""
    import concurrent.futures as cf
    import workloads as W
    from oracle import _cmodel, colsum as oc, dprob as od, index_add as oi, wgrad as ow
    n = _cmodel.threads()
    pool = cf.ThreadPoolExecutor(n)
    samples = []   # (label, algorithmic bytes of the full problem, CPU seconds for the full problem)

    def split(k):
        return [(i * k // n, (i + 1) * k // n) for i in range(n) if (i + 1) * k // n > i * k // n]

    t0 = time.perf_counter()
    g = W.gate_inputs(16384, 32, seed=2)
    t = time.perf_counter()
    list(pool.map(lambda r: oc.colsum(g.a[:, r[0]:r[1]], g.dg[:, r[0]:r[1]], g.A_log[r[0]:r[1]],
                                      g.dt_bias[r[0]:r[1]], g.dA_log0[r[0]:r[1]], g.ddt_bias0[r[0]:r[1]], 64),
                  split(32)))
    samples.append(("colsum T=16384 H=32 (full, heads split)", 16384 * 32 * 4 + 32 * 4 * 6, time.perf_counter() - t))
    dp = W.dprob_inputs(seed=4)
    t = time.perf_counter()
    list(pool.map(lambda r: od.grouped_dprob(dp.dprob0[r[0]:r[1]], dp.dY[r[0]:r[1]], dp.C[r[0]:r[1]],
                                             np.array([0, r[1] - r[0]], np.int32)), split(16384)))
    samples.append(("dprob 16384x2048 (full, rows split)", 16384 * 2048 * 4 + 16384 * 8, time.perf_counter() - t))
    del dp
    ia = W.index_add_inputs(seed=3)
    nv = int(np.count_nonzero(ia.ids >= 0))
    nt = int(np.count_nonzero(np.bincount(ia.ids[ia.ids >= 0], minlength=8192)))
    t = time.perf_counter()
    oi.index_add(ia.out0, ia.ids, ia.src, 256)   # one call: its stable sort is over all ids
    samples.append(("index_add 4096x512 -> 8192x128 (full, one thread)", ia.ids.size * 4 + nv * 256 + nt * 128 * 8,
                    time.perf_counter() - t))
    del ia
    spent = sum(x[2] for x in samples)
    wg = W.wgrad_inputs(seed=5)
    T_total = int(wg.offs[-1])
    rows = 8
    t = time.perf_counter()
    ow.grouped_wgrad_acc(wg.main_grad0, wg.G, wg.X, wg.offs, rows=np.arange(rows))
    tw = time.perf_counter() - t
    if spent + tw < target_s:   # a larger sample while the budget allows
        rows = int(min(1408, max(rows, rows * (target_s - spent) / max(tw, 1e-3) * 0.8)))
        t = time.perf_counter()
        ow.grouped_wgrad_acc(wg.main_grad0, wg.G, wg.X, wg.offs, rows=np.arange(rows))
        tw = time.perf_counter() - t
    samples.append(("wgrad E=8 %d tokens: %d of 1408 output rows of every expert (matrix-core model chains), "
                    "scaled x%.1f" % (T_total, rows, 1408 / rows),
                    T_total * (1408 + 2048) * 2 + 8 * 1408 * 2048 * 8, tw * 1408 / rows))
    pool.shutdown()
    log("cpu oracle: %.1f s of compute, %.1f s with input generation, %d threads" % (
        spent + tw, time.perf_counter() - t0, n))
    nbytes = sum(s[1] for s in samples)
    secs = sum(s[2] for s in samples)
    return {"value": round(nbytes / secs / 1e9, 4), "unit": "GB/s", "cores": n, "kind": "oracle",
            "sample": "%s; threads %d on %s" % ("; ".join("%s: %.2f s" % (s[0], s[2]) for s in samples), n,
                                               _cpu_model())}


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


def copy_calibration():
    """A plain copy of known size (reads and writes exactly COPY_BYTES each), three times: the kernel against
    which hardware byte counters are scaled."""
    import torch
    src = torch.ones(COPY_BYTES // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    log("copy calibration: 3 copies of %d bytes" % COPY_BYTES)


# --------------------------------------------------------------------- main
def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py measures one GPU only: this build's reductions run on a single MI355X; "
              "--gpus %d is not supported" % args.gpus, file=sys.stderr)
        sys.exit(2)
    import torch
    torch.cuda.init()
    only = set(x for x in args.only.split(",") if x)
    wls = build_workloads()
    if only:
        pool = wls + (build_extra_workloads() if only - {w.name for w in wls} else [])
        unknown = only - {w.name for w in pool}
        if unknown:
            print("--only: unknown entry points %s" % sorted(unknown), file=sys.stderr)
            sys.exit(2)
        wls = [w for w in pool if w.name in only]
        del pool
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
    if only:
        print(json.dumps({"only": sorted(only), "steps": args.steps, "ms_per_step": round(ms_per_step, 4),
                          "us_per_call": {k: round(float(np.mean(v)), 3) for k, v in in_step.items()}}), flush=True)
        if args.copy_calibration:
            copy_calibration()
        return

    kernels, outside = {}, {}
    for w in wls:
        kernels[w.name] = kernel_record(w, args.reps, flush, float(np.mean(in_step[w.name])))
        log("%-9s %s" % (w.name, json.dumps(kernels[w.name])))
    for w in build_extra_workloads():
        outside[w.name] = kernel_record(w, args.reps, flush)
        log("%-9s %s" % (w.name, json.dumps(outside[w.name])))
        del w
    outside["colsum_tile_sweep_us"] = colsum_tile_sweep(args.reps, flush)
    log("colsum sweep %s" % json.dumps(outside["colsum_tile_sweep_us"]))
    libref = library_reference(args.reps, flush)
    log("library reference %s" % json.dumps(libref))
    ceil = measured_ceilings(flush)
    log("measured ceilings %s" % json.dumps(ceil))

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
    # the same kernel against what this box measured beside it (measured_ceilings): the matrix cores on
    # operands of the workload's magnitude, or a device copy
    c = ceil["mfma_random_bf16"]["TFLOP_per_s"] if dom.bound == "mfma" else ceil["hbm_copy_1GiB"]["GB_per_s"]
    roof["measured_ceiling"] = c
    roof["frac_of_measured_ceiling"] = round(roof["achieved"] / c, 4)

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
        "library_reference": libref,
        "measured_ceilings": ceil,
    }
    if args.copy_calibration:
        copy_calibration()
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(args.cpu_seconds)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
