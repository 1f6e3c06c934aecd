"""Every deterministic entry point can be captured into a HIP graph: a call
only enqueues kernels on the caller's stream (no allocation, no host
synchronisation, no memset node). Each case captures one call with a
workspace allocated beforehand, then replays the graph several times with the
program's own eager work and synchronisations between the replays; every
replay, started from the same output values, must give the bits of the eager
call."""
import numpy as np
import pytest

import deterministic_gradient_reductions_amd as dg
import workloads as W
from tests.gpu_util import dev_bf16, dev_f32, dev_i32, host, note

pytestmark = pytest.mark.gpu

REPLAYS = 5


def graph_check(call, outs, what):
    """call(): one entry-point call accumulating into the tensors `outs`. The graph is captured from
    the same start values; before each replay the outputs are reset eagerly and a side computation
    runs, then the replay's outputs are compared bit for bit with the eager call's."""
    import torch
    start = [o.clone() for o in outs]

    def reset():
        for o, s in zip(outs, start):
            o.copy_(s)

    reset()
    call()
    want = [host(o).copy() for o in outs]
    # warm-up on a side stream, as graph capture asks, then capture on it
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        reset()
        call()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    reset()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call()
    busy = torch.ones(1 << 22, device="cuda")
    for r in range(REPLAYS):
        reset()
        busy.mul_(1.0000001)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for o, w in zip(outs, want):
            got = host(o)
            assert np.array_equal(got.view(np.uint8), w.view(np.uint8)), (
                "%s graph replay %d differs from the eager call in %d elements" % (what, r, int((got != w).sum())))
    note("%s: %d graph replays bitwise equal to the eager call" % (what, REPLAYS))


def test_colsum_and_da():
    import torch
    g = W.gate_inputs(16323, 32, seed=2, out_init="normal")
    a, dgv = dev_bf16(g.a), dev_bf16(g.dg_base)[:, 32:]
    Al, db = dev_f32(g.A_log), dev_f32(g.dt_bias)
    o1, o2 = dev_f32(g.dA_log0), dev_f32(g.ddt_bias0)
    cfg = dg.ColsumCfg(128, 16)
    ws = dg.Workspace(dg.det_colsum_workspace_size(16323, 32, cfg))
    graph_check(lambda: dg.det_colsum(a, dgv, Al, db, o1, o2, cfg=cfg, ws=ws), [o1, o2], "colsum")
    da = torch.empty_like(a)
    graph_check(lambda: dg.det_colsum(a, dgv, Al, db, o1, o2, cfg=cfg, ws=ws, da=da), [o1, o2, da.view(torch.int16)],
                "colsum_da")


def test_colsum_noalloc():
    g = W.gate_inputs(4096, 16, seed=3, out_init="normal")
    a, dgv = dev_bf16(g.a), dev_bf16(g.dg_base)[:, 16:]
    Al, db = dev_f32(g.A_log), dev_f32(g.dt_bias)
    o1, o2 = dev_f32(g.dA_log0), dev_f32(g.ddt_bias0)
    graph_check(lambda: dg.det_colsum_noalloc(a, dgv, Al, db, o1, o2), [o1, o2], "colsum_noalloc")


@pytest.mark.parametrize("L", [7, 256])
def test_index_add(L):
    ia = W.index_add_inputs(Q=512, K=512, n_rows=4096, dim=128, seed=3, out_init="normal")
    ids, src, o = dev_i32(ia.ids), dev_bf16(ia.src), dev_f32(ia.out0)
    cfg = dg.IndexAddCfg(L)
    ws = dg.Workspace(dg.det_index_add_workspace_size(ia.ids.size, 128, 4096, cfg))
    graph_check(lambda: dg.det_index_add(o, ids, src, cfg=cfg, ws=ws), [o], "index_add L=%d" % L)


def test_indexer_dk():
    x = W.indexer_dk_inputs(Q=512, K=512, n_rows=4096, dim=128, seed=4, out_init="normal")
    ids, p, t, q, o = dev_i32(x.ids), dev_f32(x.predict), dev_f32(x.target), dev_bf16(x.q), dev_f32(x.dk0)
    cfg = dg.IndexAddCfg(256)
    ws = dg.Workspace(dg.det_indexer_dk_workspace_size(512, 512, 128, 4096, cfg))
    graph_check(lambda: dg.det_indexer_dk(o, ids, p, t, q, x.scale, cfg=cfg, ws=ws), [o], "indexer_dk")


def test_dprob():
    dp = W.dprob_inputs(M=3000, N=2048, E=5, min_tokens=1, seed=1, out_init="normal")
    dY, C, offs, d = dev_bf16(dp.dY), dev_bf16(dp.C), dev_i32(dp.offs), dev_f32(dp.dprob0)
    graph_check(lambda: dg.det_grouped_dprob(d, dY, C, offs), [d], "dprob")


def test_dbias():
    db = W.dbias_inputs(M=3000, N=1024, E=5, min_tokens=1, seed=6, out_init="normal")
    dA, offs, d = dev_bf16(db.dA), dev_i32(db.offs), dev_f32(db.dbias0)
    cfg = dg.DbiasCfg(128, 512)
    ws = dg.Workspace(dg.det_grouped_dbias_workspace_size(3000, 1024, 5, cfg))
    graph_check(lambda: dg.det_grouped_dbias(d, dA, offs, cfg=cfg, ws=ws), [d], "dbias")


@pytest.mark.parametrize("C", [0, 2])
def test_wgrad(C):
    import torch
    inp = W.wgrad_inputs(E=4, M=640, N=768, tokens=[1500, 0, 700, 2049], seed=7, out_init="normal")
    T = int(inp.offs[-1])
    G, X, offs, mg = dev_bf16(inp.G), dev_bf16(inp.X), dev_i32(inp.offs), dev_f32(inp.main_grad0)
    cfg = dg.WgradCfg(256, 256, 512, C)
    ws = dg.Workspace(dg.det_grouped_wgrad_acc_workspace_size(T, 4, 640, 768, cfg))
    graph_check(lambda: dg.det_grouped_wgrad_acc(mg, G, X, offs, cfg=cfg, ws=ws), [mg], "wgrad C=%d" % C)
    if C == 0:
        mg16 = torch.from_numpy((inp.main_grad0.view(np.uint32) >> 16).astype(np.uint16).view(np.int16)).cuda()
        b16 = mg16.view(torch.bfloat16)
        ws16 = dg.Workspace(dg.det_grouped_wgrad_acc_bf16_workspace_size(T, 4, 640, 768, cfg))
        graph_check(lambda: dg.det_grouped_wgrad_acc_bf16(b16, G, X, offs, cfg=cfg, ws=ws16), [mg16],
                    "wgrad bf16 main_grad")


def test_topk():
    import torch
    tk = W.topk_inputs(Q=256, K=512, seed=7)
    ids, lg = dev_i32(tk.ids), dev_f32(tk.logits)
    io, lo, po = torch.empty_like(ids), torch.empty_like(lg), torch.empty_like(lg)
    graph_check(lambda: dg.det_topk_canonicalize(ids, lg, io, lo, po), [io, lo, po], "topk")
