"""det_colsum_noalloc (slots in the library's static device scratch) against
det_colsum (slots in a caller workspace): bitwise on two calls in a row, the
second with a smaller input, and against the oracle; a problem too large for
the static scratch is refused before any launch."""
import numpy as np
import pytest

import deterministic_gradient_reductions_amd as dg
import workloads as W
from oracle import colsum as oc
from tests.gpu_util import assert_bitwise, dev_bf16, dev_f32, host, note

pytestmark = pytest.mark.gpu


def both(g, T, H, cfg):
    a = dev_bf16(g.a)
    dgv = dev_bf16(g.dg_base)[:, H:]
    outs = []
    for fn in (dg.det_colsum, dg.det_colsum_noalloc):
        o1, o2 = dev_f32(g.dA_log0), dev_f32(g.ddt_bias0)
        fn(a, dgv, dev_f32(g.A_log), dev_f32(g.dt_bias), o1, o2, cfg=cfg)
        outs.append((host(o1), host(o2)))
    return outs


def test_noalloc_matches_the_workspace_call_twice_then_smaller():
    for T, H in ((16384, 32), (1000, 16)):
        g = W.gate_inputs(T, H, seed=2, out_init="normal")
        cfg = dg.det_colsum_select_cfg(T, H)
        note("colsum_noalloc T=%d H=%d cfg %dx%d" % (T, H, cfg.block_t, cfg.block_h))
        (w1, w2), (n1, n2) = both(g, T, H, cfg)
        assert_bitwise(n1, w1, "dA_log")
        assert_bitwise(n2, w2, "ddt_bias")
        r1, r2 = oc.colsum(g.a, g.dg, g.A_log, g.dt_bias, g.dA_log0, g.ddt_bias0, cfg.block_t)
        assert_bitwise(n1, r1, "dA_log vs oracle")
        assert_bitwise(n2, r2, "ddt_bias vs oracle")


def test_noalloc_refuses_a_problem_beyond_its_scratch():
    import torch
    T, H = 4 << 20, 32  # block_t 64 would need 2 x 8 MiB of slots
    a = torch.zeros((T, H), dtype=torch.bfloat16, device="cuda")
    p = torch.zeros(H, dtype=torch.float32, device="cuda")
    o1, o2 = p.clone(), p.clone()
    with pytest.raises(dg.DetError) as e:
        dg.det_colsum_noalloc(a, a, p, p, o1, o2, cfg=dg.ColsumCfg(64, 8))
    assert e.value.status == dg.DET_ERR_WORKSPACE
    assert not o1.any() and not o2.any()
