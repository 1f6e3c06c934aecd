"""Calls keep no state between them: deterministic calls running at the same time
on two streams, each with its own workspace, give the bits they give one after
the other."""
import numpy as np
import pytest

import deterministic_gradient_reductions_amd as dg
import workloads as W
from tests.gpu_util import dev_bf16, dev_f32, dev_i32, host, note

pytestmark = pytest.mark.gpu

ROUNDS = 5


def concurrent(calls):
    """calls: [(run, out, out0)]; run(stream) enqueues one call into `out` on that stream. Every call first
    runs alone (the reference bits), then all of them run ROUNDS times, each on its own stream, enqueued
    back to back with no synchronisation between the streams; every result must equal its reference."""
    import torch
    want = []
    for run, out, out0 in calls:
        out.copy_(out0)
        run(torch.cuda.current_stream())
        want.append(host(out).copy())
    streams = [torch.cuda.Stream() for _ in calls]
    for r in range(ROUNDS):
        torch.cuda.synchronize()
        for (run, out, out0), s in zip(calls, streams):
            with torch.cuda.stream(s):
                out.copy_(out0)
                run(s)
        torch.cuda.synchronize()
        for i, ((run, out, out0), w) in enumerate(zip(calls, want)):
            got = host(out)
            assert np.array_equal(got.view(np.uint32), w.view(np.uint32)), "call %d, round %d: %d elements differ" % (
                i, r, int((got != w).sum()))


def index_add_call(seed):
    ia = W.index_add_inputs(Q=1024, K=512, n_rows=8192, dim=128, seed=seed, out_init="normal")
    ids, src, o, o0 = dev_i32(ia.ids), dev_bf16(ia.src), dev_f32(ia.out0), dev_f32(ia.out0)
    ws = dg.Workspace(dg.det_index_add_workspace_size(ia.ids.size, 128, 8192))
    return (lambda s: dg.det_index_add(o, ids, src, ws=ws, stream=s)), o, o0


def test_same_entry_point_on_two_streams():
    concurrent([index_add_call(3), index_add_call(4)])
    note("index_add on two streams: %d rounds bitwise equal to the calls alone" % ROUNDS)


def test_four_entry_points_on_four_streams():
    wg = W.wgrad_inputs(E=4, M=640, N=1024, tokens=[3000, 1500, 0, 2600], seed=5, out_init="normal")
    G, X, offs = dev_bf16(wg.G), dev_bf16(wg.X), dev_i32(wg.offs)
    mg, mg0 = dev_f32(wg.main_grad0), dev_f32(wg.main_grad0)
    cfg = dg.WgradCfg(256, 256, 512, 2)
    wws = dg.Workspace(dg.det_grouped_wgrad_acc_workspace_size(int(wg.offs[-1]), 4, 640, 1024, cfg))
    dp = W.dprob_inputs(M=4000, N=2048, E=5, min_tokens=1, seed=1, out_init="normal")
    dY, C, doffs, d, d0 = dev_bf16(dp.dY), dev_bf16(dp.C), dev_i32(dp.offs), dev_f32(dp.dprob0), dev_f32(dp.dprob0)
    g = W.gate_inputs(16323, 32, seed=2, out_init="normal")
    a, dgv, Al, db = dev_bf16(g.a), dev_bf16(g.dg_base)[:, 32:], dev_f32(g.A_log), dev_f32(g.dt_bias)
    both = dev_f32(np.concatenate([g.dA_log0, g.ddt_bias0]))
    both0 = both.clone()
    ccfg = dg.ColsumCfg(64, 8)
    cws = dg.Workspace(dg.det_colsum_workspace_size(16323, 32, ccfg))
    o1, o2 = both[:32], both[32:]
    concurrent([
        (lambda s: dg.det_grouped_wgrad_acc(mg, G, X, offs, cfg=cfg, ws=wws, stream=s), mg, mg0),
        (lambda s: dg.det_grouped_dprob(d, dY, C, doffs, stream=s), d, d0),
        (lambda s: dg.det_colsum(a, dgv, Al, db, o1, o2, cfg=ccfg, ws=cws, stream=s), both, both0),
        index_add_call(5),
    ])
    note("wgrad (split-K), dprob, colsum and index_add on four streams: %d rounds bitwise equal" % ROUNDS)
