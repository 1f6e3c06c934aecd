"""Every workspace slot is written before it is read in the same call: a
workspace whose area behind the 256-byte header is filled with NaN bytes
(then the header initialised) gives the same bits as a fresh zeroed one, for
every entry point that takes a workspace."""
import numpy as np
import pytest

import deterministic_gradient_reductions_amd as dg
import workloads as W
from tests.gpu_util import assert_bitwise, dev_bf16, dev_f32, dev_i32, host, note

pytestmark = pytest.mark.gpu


def workspaces(nbytes):
    """(zeroed, poisoned) workspaces of nbytes."""
    import torch
    z = dg.Workspace(nbytes)
    z._buf.zero_()
    dg.det_workspace_init(z)
    p = dg.Workspace(nbytes)
    p._buf.fill_(0xFF)          # 0xFFFFFFFF: a NaN in every float32 slot, -1 in every integer one
    dg.det_workspace_init(p)   # the header's counters start at zero, as the contract asks
    torch.cuda.synchronize()
    return z, p


def both(call, nbytes):
    z, p = workspaces(nbytes)
    a = call(z)
    b = call(p)
    return a, b


def test_colsum():
    g = W.gate_inputs(16323, 32, seed=2, out_init="normal")
    for cfg in (dg.ColsumCfg(64, 8), dg.ColsumCfg(256, 32)):
        def call(ws):
            o1, o2 = dev_f32(g.dA_log0), dev_f32(g.ddt_bias0)
            dg.det_colsum(dev_bf16(g.a), dev_bf16(g.dg_base)[:, 32:], dev_f32(g.A_log), dev_f32(g.dt_bias), o1, o2,
                          cfg=cfg, ws=ws)
            return np.concatenate([host(o1), host(o2)])
        a, b = both(call, dg.det_colsum_workspace_size(16323, 32, cfg))
        assert_bitwise(b, a, "colsum")


def test_index_add_and_indexer_dk():
    ia = W.index_add_inputs(Q=512, K=512, n_rows=4096, dim=128, seed=3, out_init="normal")
    for L in (7, 256, 1024):
        cfg = dg.IndexAddCfg(L)

        def call(ws):
            o = dev_f32(ia.out0)
            dg.det_index_add(o, dev_i32(ia.ids), dev_bf16(ia.src), cfg=cfg, ws=ws)
            return host(o)
        a, b = both(call, dg.det_index_add_workspace_size(ia.ids.size, 128, 4096, cfg))
        assert_bitwise(b, a, "index_add L=%d" % L)
    x = W.indexer_dk_inputs(Q=512, K=512, n_rows=4096, dim=128, seed=4, out_init="normal")

    def call(ws):
        o = dev_f32(x.dk0)
        dg.det_indexer_dk(o, dev_i32(x.ids), dev_f32(x.predict), dev_f32(x.target), dev_bf16(x.q), x.scale,
                          cfg=dg.IndexAddCfg(256), ws=ws)
        return host(o)
    a, b = both(call, dg.det_indexer_dk_workspace_size(512, 512, 128, 4096, dg.IndexAddCfg(256)))
    assert_bitwise(b, a, "indexer_dk")


def test_dbias():
    db = W.dbias_inputs(M=3000, N=1024, E=5, min_tokens=1, seed=6, out_init="normal")
    for bm in (64, 256):
        cfg = dg.DbiasCfg(bm, 512)

        def call(ws):
            d = dev_f32(db.dbias0)
            dg.det_grouped_dbias(d, dev_bf16(db.dA), dev_i32(db.offs), cfg=cfg, ws=ws)
            return host(d)
        a, b = both(call, dg.det_grouped_dbias_workspace_size(3000, 1024, 5, cfg))
        assert_bitwise(b, a, "dbias block_m=%d" % bm)


def test_wgrad_split_and_bf16():
    import torch
    inp = W.wgrad_inputs(E=4, M=256, N=512, tokens=[1500, 0, 700, 2049], seed=7, out_init="normal")
    T = int(inp.offs[-1])
    for C in (1, 3):
        cfg = dg.WgradCfg(256, 256, 512, C)

        def call(ws):
            mg = dev_f32(inp.main_grad0)
            dg.det_grouped_wgrad_acc(mg, dev_bf16(inp.G), dev_bf16(inp.X), dev_i32(inp.offs), cfg=cfg, ws=ws)
            return host(mg)
        a, b = both(call, dg.det_grouped_wgrad_acc_workspace_size(T, 4, 256, 512, cfg))
        assert_bitwise(b, a, "wgrad C=%d" % C)
    mg16 = (np.random.default_rng(1).standard_normal((4, 256, 512)).astype(np.float32).view(np.uint32) >> 16
            ).astype(np.uint16)

    def call16(ws):
        mg = torch.from_numpy(mg16.view(np.int16).copy()).cuda().view(torch.bfloat16)
        dg.det_grouped_wgrad_acc_bf16(mg, dev_bf16(inp.G), dev_bf16(inp.X), dev_i32(inp.offs),
                                      cfg=dg.WgradCfg(256, 256, 512, 0), ws=ws)
        torch.cuda.synchronize()
        return mg.view(torch.int16).cpu().numpy()
    a, b = both(call16, dg.det_grouped_wgrad_acc_bf16_workspace_size(T, 4, 256, 512, dg.WgradCfg(256, 256, 512, 0)))
    note("wgrad bf16 poisoned workspace")
    assert np.array_equal(a, b)
