"""The C-ABI library loads, exports every declared symbol and rejects bad
arguments on the host before any HIP call (CPU only, no kernel launches)."""
import ctypes
import os
import re

import pytest

import deterministic_gradient_reductions_amd as dg

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "detgrad.h")

pytestmark = pytest.mark.skipif(not os.path.exists(dg.library_path), reason="libdetgrad.so not built")


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(det_[a-z0-9_]+)\s*\(", src)))


def test_exports_every_declared_symbol():
    L = ctypes.CDLL(dg.library_path)
    names = declared_functions()
    assert len(names) >= 14
    for n in names:
        assert hasattr(L, n), n


def test_abi_version():
    assert dg.det_abi_version() == 1


def lib():
    return dg.lib()


def err():
    return lib().det_last_error().decode()


P = ctypes.c_void_p
FAKE = P(0x10000)  # never dereferenced: every case below fails validation first


def test_atomic_flag_must_be_0_or_1():
    n = ctypes.c_size_t()
    for bad in (2, -1, 7):
        assert lib().det_grouped_dprob_workspace_size(16, 16, None, bad, ctypes.byref(n)) == dg.DET_ERR_INVALID_ARG
        assert "atomic" in err()
        assert lib().det_grouped_dprob(FAKE, FAKE, 16, FAKE, 16, 16, 16, FAKE, 1, None, None, 0, bad, None) == \
            dg.DET_ERR_INVALID_ARG
        assert lib().det_colsum(FAKE, 16, 1, FAKE, 16, 1, 0, FAKE, FAKE, 16, 16, FAKE, FAKE, None, None, 0, bad,
                                None) == dg.DET_ERR_INVALID_ARG
        assert lib().det_index_add_workspace_size(16, 8, 16, None, bad, ctypes.byref(n)) == dg.DET_ERR_INVALID_ARG
        assert lib().det_grouped_wgrad_acc_workspace_size(16, 1, 16, 16, None, bad, ctypes.byref(n)) == \
            dg.DET_ERR_INVALID_ARG


def test_dprob_validation():
    L = lib()
    # negative sizes
    assert L.det_grouped_dprob(FAKE, FAKE, 16, FAKE, 16, -1, 16, FAKE, 1, None, None, 0, 0, None) == \
        dg.DET_ERR_INVALID_ARG
    # ld < N
    assert L.det_grouped_dprob(FAKE, FAKE, 8, FAKE, 16, 4, 16, FAKE, 1, None, None, 0, 0, None) == \
        dg.DET_ERR_INVALID_ARG
    # illegal tile
    cfg = dg.DprobCfg(64, 16)
    assert L.det_grouped_dprob(FAKE, FAKE, 16, FAKE, 16, 4, 16, FAKE, 1, ctypes.byref(cfg), None, 0, 0, None) == \
        dg.DET_ERR_INVALID_ARG
    cfg = dg.DprobCfg(128, 0)
    assert L.det_grouped_dprob(FAKE, FAKE, 16, FAKE, 16, 4, 16, FAKE, 1, ctypes.byref(cfg), None, 0, 0, None) == \
        dg.DET_ERR_INVALID_ARG
    # output overlapping an input
    base = 0x200000
    assert L.det_grouped_dprob(P(base + 8), P(base), 16, P(base + 4096), 16, 4, 16, P(base + 8192), 1, None, None, 0,
                               0, None) == dg.DET_ERR_OVERLAP
    # NULL pointers
    assert L.det_grouped_dprob(None, FAKE, 16, FAKE, 16, 4, 16, FAKE, 1, None, None, 0, 0, None) == \
        dg.DET_ERR_INVALID_ARG
    # empty problem: OK with nothing launched, even with NULL pointers
    assert L.det_grouped_dprob(None, None, 0, None, 0, 0, 16, None, 1, None, None, 0, 0, None) == dg.DET_OK
    n = ctypes.c_size_t(123)
    assert L.det_grouped_dprob_workspace_size(16384, 2048, None, 0, ctypes.byref(n)) == dg.DET_OK and n.value == 0


def test_dbias_validation():
    L = lib()
    n = ctypes.c_size_t(0)
    # workspace: header + tile starts + (ceil(M/128) + E) x N slots; none for the atomic arm
    assert L.det_grouped_dbias_workspace_size(16384, 2048, 8, None, 0, ctypes.byref(n)) == dg.DET_OK
    assert n.value == 256 + 256 + (128 + 8) * 2048 * 4
    assert L.det_grouped_dbias_workspace_size(16384, 2048, 8, None, 1, ctypes.byref(n)) == dg.DET_OK and n.value == 0
    assert L.det_grouped_dbias_workspace_size(16384, 2048, 8, None, 2, ctypes.byref(n)) == dg.DET_ERR_INVALID_ARG
    for cfg in (dg.DbiasCfg(96, 512), dg.DbiasCfg(128, 384), dg.DbiasCfg(128, 64)):
        assert L.det_grouped_dbias_workspace_size(64, 64, 2, ctypes.byref(cfg), 0, ctypes.byref(n)) == \
            dg.DET_ERR_INVALID_ARG
    big = 1 << 22
    # negative sizes, ld < N, N not a multiple of 8, NULL pointers, workspace too small
    assert L.det_grouped_dbias(FAKE, 64, FAKE, 64, -1, 64, FAKE, 2, None, FAKE, big, 0, None) == dg.DET_ERR_INVALID_ARG
    assert L.det_grouped_dbias(FAKE, 32, FAKE, 64, 16, 64, FAKE, 2, None, FAKE, big, 0, None) == dg.DET_ERR_INVALID_ARG
    assert L.det_grouped_dbias(FAKE, 64, FAKE, 60, 16, 60, FAKE, 2, None, FAKE, big, 0, None) == dg.DET_ERR_UNSUPPORTED
    assert L.det_grouped_dbias(None, 64, FAKE, 64, 16, 64, FAKE, 2, None, FAKE, big, 0, None) == dg.DET_ERR_INVALID_ARG
    assert L.det_grouped_dbias(FAKE, 64, FAKE, 64, 16, 64, FAKE, 2, None, FAKE, 512, 0, None) == dg.DET_ERR_WORKSPACE
    # output overlapping an input
    base = 0x400000
    assert L.det_grouped_dbias(P(base + 64), 64, P(base), 64, 16, 64, P(base + 65536), 2, None, None, 0, 1, None) == \
        dg.DET_ERR_OVERLAP
    # empty problems: OK with nothing launched
    assert L.det_grouped_dbias(None, 64, None, 64, 0, 64, None, 2, None, None, 0, 0, None) == dg.DET_OK
    assert L.det_grouped_dbias(None, 64, None, 64, 16, 64, None, 0, None, None, 0, 0, None) == dg.DET_OK


def test_topk_validation():
    L = lib()
    Z = P(0x500000)
    assert L.det_topk_canonicalize(FAKE, FAKE, -1, 8, 8, FAKE, FAKE, FAKE, 8, None) == dg.DET_ERR_INVALID_ARG
    assert L.det_topk_canonicalize(FAKE, FAKE, 4, 1025, 1025, FAKE, FAKE, FAKE, 1025, None) == dg.DET_ERR_UNSUPPORTED
    assert L.det_topk_canonicalize(FAKE, FAKE, 4, 8, 4, FAKE, FAKE, FAKE, 8, None) == dg.DET_ERR_INVALID_ARG
    assert L.det_topk_canonicalize(None, FAKE, 4, 8, 8, FAKE, FAKE, FAKE, 8, None) == dg.DET_ERR_INVALID_ARG
    # an output overlapping an input, or two outputs overlapping
    assert L.det_topk_canonicalize(P(0x600000), P(0x610000), 4, 8, 8, P(0x600010), Z, P(0x520000), 8, None) == \
        dg.DET_ERR_OVERLAP
    assert L.det_topk_canonicalize(P(0x600000), P(0x610000), 4, 8, 8, Z, P(0x500010), P(0x520000), 8, None) == \
        dg.DET_ERR_OVERLAP
    # empty problems: OK with nothing launched
    assert L.det_topk_canonicalize(None, None, 0, 8, 8, None, None, None, 8, None) == dg.DET_OK


def test_colsum_validation_and_selector():
    L = lib()
    # shape-only rule: block_h = 8; block_t the largest of 256/128 that still
    # gives >= 1024 workgroups, else 64
    c = dg.det_colsum_select_cfg(16384, 32)
    assert (c.block_t, c.block_h) == (64, 8)
    c = dg.det_colsum_select_cfg(4096, 16)
    assert (c.block_t, c.block_h) == (64, 8)
    c = dg.det_colsum_select_cfg(16384 * 4, 32)
    assert (c.block_t, c.block_h) == (256, 8)
    c = dg.det_colsum_select_cfg(16384 * 2, 32)
    assert (c.block_t, c.block_h) == (128, 8)
    c = dg.det_colsum_select_cfg(32768, 5)
    assert (c.block_t, c.block_h) == (64, 8)
    c = dg.det_colsum_select_cfg(1000, 100)
    assert (c.block_t, c.block_h) == (64, 8)
    bad = dg.ColsumCfg(96, 16)
    assert L.det_colsum(FAKE, 16, 1, FAKE, 16, 1, 0, FAKE, FAKE, 16, 16, FAKE, FAKE, ctypes.byref(bad), None, 0, 0,
                        None) == dg.DET_ERR_INVALID_ARG
    # unknown input dtype; fp32 inputs pass validation (a missing workspace is the first error here)
    assert L.det_colsum(FAKE, 16, 1, FAKE, 16, 1, 7, FAKE, FAKE, 16, 16, FAKE, FAKE, None, None, 0, 0, None) == \
        dg.DET_ERR_INVALID_ARG
    assert L.det_colsum(FAKE, 16, 1, FAKE, 16, 1, 1, FAKE, FAKE, 16, 16, FAKE, FAKE, None, None, 0, 0, None) == \
        dg.DET_ERR_WORKSPACE
    # workspace too small / missing / misaligned
    n = dg.det_colsum_workspace_size(1000, 16)
    assert n >= 256 + 2 * 16 * 4 * (1000 // 256)
    assert L.det_colsum(FAKE, 16, 1, FAKE, 16, 1, 0, FAKE, FAKE, 1000, 16, P(0x900000), P(0x900100), None, None, 0, 0,
                        None) == dg.DET_ERR_WORKSPACE
    assert L.det_colsum(FAKE, 16, 1, FAKE, 16, 1, 0, FAKE, FAKE, 1000, 16, P(0x900000), P(0x900100), None,
                        P(0xA00000), n - 4, 0, None) == dg.DET_ERR_WORKSPACE
    assert L.det_colsum(FAKE, 16, 1, FAKE, 16, 1, 0, FAKE, FAKE, 1000, 16, P(0x900000), P(0x900100), None,
                        P(0xA00010), n, 0, None) == dg.DET_ERR_WORKSPACE
    # outputs overlapping each other
    assert L.det_colsum(FAKE, 16, 1, FAKE, 16, 1, 0, FAKE, FAKE, 1000, 16, P(0x900000), P(0x900010), None,
                        P(0xA00000), n, 0, None) == dg.DET_ERR_OVERLAP
    # zero strides
    assert L.det_colsum(FAKE, 0, 1, FAKE, 16, 1, 0, FAKE, FAKE, 1000, 16, P(0x900000), P(0x900100), None,
                        P(0xA00000), n, 0, None) == dg.DET_ERR_INVALID_ARG


def test_workspace_init_validation():
    L = lib()
    assert L.det_workspace_init(None, 256, None) == dg.DET_ERR_WORKSPACE
    assert L.det_workspace_init(P(0x10010), 256, None) == dg.DET_ERR_WORKSPACE
    assert L.det_workspace_init(P(0x10000), 64, None) == dg.DET_ERR_WORKSPACE


def test_index_add_validation():
    L = lib()
    n = ctypes.c_size_t()
    assert L.det_index_add_workspace_size(2 ** 21, 128, 8192, None, 0, ctypes.byref(n)) == dg.DET_OK
    assert n.value > 2 ** 21 * 4  # holds at least the permutation
    assert L.det_index_add_workspace_size(2 ** 21, 128, 8192, None, 1, ctypes.byref(n)) == dg.DET_OK and n.value == 0
    # dim not a multiple of 8, too many rows, bad chunk size
    assert L.det_index_add_workspace_size(100, 12, 10, None, 0, ctypes.byref(n)) == dg.DET_ERR_UNSUPPORTED
    assert L.det_index_add_workspace_size(100, 16, 16385, None, 0, ctypes.byref(n)) == dg.DET_ERR_UNSUPPORTED
    bad = dg.IndexAddCfg(0)
    assert L.det_index_add_workspace_size(100, 16, 10, ctypes.byref(bad), 0, ctypes.byref(n)) == dg.DET_ERR_INVALID_ARG
    # out_ld < dim; misaligned src; overlap; unknown src dtype; workspace missing (bf16 and fp32 src)
    O, I, S = P(0x100000), P(0x200000), P(0x300000)
    assert L.det_index_add(O, 10, 16, 8, I, 100, S, 16, 0, None, None, 0, 1, None) == dg.DET_ERR_INVALID_ARG
    assert L.det_index_add(O, 10, 16, 16, I, 100, P(0x300008), 16, 0, None, None, 0, 1, None) == dg.DET_ERR_UNSUPPORTED
    assert L.det_index_add(O, 10, 16, 16, P(0x100010), 100, S, 16, 0, None, None, 0, 1, None) == dg.DET_ERR_OVERLAP
    assert L.det_index_add(O, 10, 16, 16, I, 100, S, 16, 5, None, None, 0, 1, None) == dg.DET_ERR_INVALID_ARG
    assert L.det_index_add(O, 10, 16, 16, I, 100, S, 16, 0, None, None, 0, 0, None) == dg.DET_ERR_WORKSPACE
    assert L.det_index_add(O, 10, 16, 16, I, 100, S, 16, 1, None, None, 0, 0, None) == dg.DET_ERR_WORKSPACE
    # empty problems return OK without touching anything
    assert L.det_index_add(None, 10, 16, 16, None, 0, None, 16, 0, None, None, 0, 0, None) == dg.DET_OK


def test_wgrad_validation():
    L = lib()
    n = ctypes.c_size_t()
    # one split per expert needs no workspace; split-K needs max_splits * M * N * 4 bytes
    assert L.det_grouped_wgrad_acc_workspace_size(36864, 8, 1408, 2048, None, 0, ctypes.byref(n)) == dg.DET_OK
    assert n.value == 0
    c = dg.WgradCfg(128, 512, 512, 4)
    assert L.det_grouped_wgrad_acc_workspace_size(36864, 8, 1408, 2048, ctypes.byref(c), 0, ctypes.byref(n)) == dg.DET_OK
    assert n.value == 256 + (36864 // 2048 + 8) * 1408 * 2048 * 4
    assert L.det_grouped_wgrad_acc_workspace_size(36864, 8, 1408, 2048, ctypes.byref(c), 1, ctypes.byref(n)) == dg.DET_OK
    assert n.value == 0
    bad = dg.WgradCfg(128, 512, 256, 0)
    assert L.det_grouped_wgrad_acc_workspace_size(100, 1, 128, 512, ctypes.byref(bad), 0, ctypes.byref(n)) == \
        dg.DET_ERR_INVALID_ARG
    bad = dg.WgradCfg(64, 512, 512, 0)
    assert L.det_grouped_wgrad_acc_workspace_size(100, 1, 128, 512, ctypes.byref(bad), 0, ctypes.byref(n)) == \
        dg.DET_ERR_UNSUPPORTED
    assert L.det_grouped_wgrad_acc_workspace_size(100, 1, 100, 512, None, 0, ctypes.byref(n)) == dg.DET_ERR_UNSUPPORTED
    assert L.det_grouped_wgrad_acc_workspace_size(100, 1, 128, 384, None, 0, ctypes.byref(n)) == dg.DET_ERR_UNSUPPORTED
    # the default 256 x 256 workgroup tile (like 128 x 256) takes N in multiples of 256, the 128 x 512 tile
    # in multiples of 512; other widths are refused
    wide = dg.WgradCfg(128, 512, 512, 0)
    assert L.det_grouped_wgrad_acc_workspace_size(100, 1, 128, 768, None, 0, ctypes.byref(n)) == dg.DET_OK
    assert L.det_grouped_wgrad_acc_workspace_size(100, 1, 128, 768, ctypes.byref(wide), 0, ctypes.byref(n)) == \
        dg.DET_ERR_UNSUPPORTED
    square = dg.WgradCfg(256, 256, 512, 0)
    assert L.det_grouped_wgrad_acc_workspace_size(100, 1, 384, 768, ctypes.byref(square), 0, ctypes.byref(n)) == \
        dg.DET_OK
    odd = dg.WgradCfg(128, 384, 512, 0)
    assert L.det_grouped_wgrad_acc_workspace_size(100, 1, 128, 768, ctypes.byref(odd), 0, ctypes.byref(n)) == \
        dg.DET_ERR_UNSUPPORTED
    MG, G, X, O = P(0x1000000), P(0x9000000), P(0xA000000), P(0xB000000)
    # an expanded main_grad (expert stride 0) is rejected
    assert L.det_grouped_wgrad_acc(MG, 0, 512, G, 128, X, 512, O, 2, 64, 128, 512, None, None, 0, 0, None) == \
        dg.DET_ERR_INVALID_ARG
    # ld_m < N
    assert L.det_grouped_wgrad_acc(MG, 128 * 512, 256, G, 128, X, 512, O, 2, 64, 128, 512, None, None, 0, 0,
                                   None) == dg.DET_ERR_INVALID_ARG
    # main_grad overlapping G
    assert L.det_grouped_wgrad_acc(P(0x9000100), 128 * 512, 512, G, 128, X, 512, O, 2, 64, 128, 512, None, None, 0,
                                   0, None) == dg.DET_ERR_OVERLAP
    # split-K without a workspace
    assert L.det_grouped_wgrad_acc(MG, 128 * 512, 512, G, 128, X, 512, O, 2, 64, 128, 512, ctypes.byref(c), None, 0,
                                   0, None) == dg.DET_ERR_WORKSPACE
    # misaligned G rows
    assert L.det_grouped_wgrad_acc(MG, 128 * 512, 512, G, 132, X, 512, O, 2, 64, 128, 512, None, None, 0, 0,
                                   None) == dg.DET_ERR_UNSUPPORTED
    # empty problems are OK and touch nothing
    assert L.det_grouped_wgrad_acc(None, 0, 0, None, 0, None, 0, None, 0, 0, 128, 512, None, None, 0, 0, None) == \
        dg.DET_OK


def test_colsum_da_validation():
    """det_colsum_da rejects a missing da, bad strides, strides that send two
    elements to one address, and overlaps (no case reaches a launch)."""
    L = lib()
    o1, o2 = P(0x900000), P(0x900100)

    def call(da, st, sh, T=16, H=16):
        return L.det_colsum_da(FAKE, 16, 1, FAKE, 16, 1, 0, FAKE, FAKE, T, H, o1, o2, da, st, sh, None, None, 0, 1,
                               None)
    assert call(None, 16, 1) == dg.DET_ERR_INVALID_ARG
    assert call(P(0xA00000), 0, 1) == dg.DET_ERR_INVALID_ARG
    assert call(P(0xA00000), 1, 1) == dg.DET_ERR_INVALID_ARG and "address" in err()
    assert call(P(0xA00000), 8, 1) == dg.DET_ERR_INVALID_ARG   # rows of 16 heads 8 elements apart
    assert call(FAKE, 16, 1) == dg.DET_ERR_OVERLAP              # da over a
    assert call(P(0x900000 - 64), 16, 1) == dg.DET_ERR_OVERLAP  # da over dA_log


def test_wgrad_bf16_validation_and_workspace():
    L = lib()
    n = dg.det_grouped_wgrad_acc_bf16_workspace_size(38346, 8, 1408, 2048)
    assert n >= 8 * 1408 * 2048 * 4  # every expert's partial, also with one split per expert
    assert dg.det_grouped_wgrad_acc_bf16_workspace_size(0, 8, 1408, 2048) == 0
    # missing workspace, misaligned main_grad, bad shape (no case reaches a launch)
    assert L.det_grouped_wgrad_acc_bf16(P(0x900000), 512 * 256, 512, FAKE, 256, FAKE, 512, FAKE, 2, 1000, 256, 512,
                                        None, None, 0, None) == dg.DET_ERR_WORKSPACE
    assert L.det_grouped_wgrad_acc_bf16(P(0x900002), 512 * 256, 512, FAKE, 256, FAKE, 512, FAKE, 2, 1000, 256, 512,
                                        None, None, 0, None) == dg.DET_ERR_UNSUPPORTED
    assert L.det_grouped_wgrad_acc_bf16(P(0x900000), 512 * 256, 512, FAKE, 256, FAKE, 512, FAKE, 2, 1000, 200, 512,
                                        None, None, 0, None) == dg.DET_ERR_UNSUPPORTED


def test_binding_rejects_wrong_dtypes_and_layouts():
    """The Python binding checks dtypes and layouts before any library call (CPU tensors suffice): an int64
    ids or offs tensor, a float64 output or a column-strided operand would otherwise be read as other words."""
    import torch
    f32, bf, i32, i64 = torch.float32, torch.bfloat16, torch.int32, torch.int64
    out = torch.zeros(8, 16, dtype=f32)
    src = torch.zeros(10, 16, dtype=bf)
    with pytest.raises(TypeError):
        dg.det_index_add(out, torch.zeros(10, dtype=i64), src)
    with pytest.raises(TypeError):
        dg.det_index_add(out.double(), torch.zeros(10, dtype=i32), src)
    with pytest.raises(ValueError):
        dg.det_index_add(out, torch.zeros(10, dtype=i32), torch.zeros(10, 32, dtype=bf)[:, ::2])
    with pytest.raises(ValueError):
        dg.det_index_add(out, torch.zeros(20, dtype=i32)[::2], src)
    dY = torch.zeros(4, 16, dtype=bf)
    with pytest.raises(TypeError):
        dg.det_grouped_dprob(torch.zeros(4, dtype=f32), dY, dY, torch.tensor([0, 4], dtype=i64))
    with pytest.raises(TypeError):
        dg.det_grouped_dprob(torch.zeros(4, dtype=torch.float64), dY, dY, torch.tensor([0, 4], dtype=i32))
    with pytest.raises(ValueError):
        dg.det_grouped_dprob(torch.zeros(4, dtype=f32), dY, torch.zeros(4, 32, dtype=bf)[:, ::2],
                             torch.tensor([0, 4], dtype=i32))
    with pytest.raises(TypeError):
        dg.det_grouped_dbias(torch.zeros(1, 16, dtype=f32), dY, torch.tensor([0, 4], dtype=i64))
    with pytest.raises(ValueError):
        dg.det_grouped_dbias(torch.zeros(2, 16, dtype=f32), dY, torch.tensor([0, 4], dtype=i32))
    G, X = torch.zeros(8, 128, dtype=bf), torch.zeros(8, 256, dtype=bf)
    mg = torch.zeros(1, 128, 256, dtype=f32)
    with pytest.raises(TypeError):
        dg.det_grouped_wgrad_acc(mg, G, X, torch.tensor([0, 8], dtype=i64))
    with pytest.raises(TypeError):
        dg.det_grouped_wgrad_acc(mg, G.float(), X, torch.tensor([0, 8], dtype=i32))
    with pytest.raises(TypeError):
        dg.det_grouped_wgrad_acc(mg.double(), G, X, torch.tensor([0, 8], dtype=i32))
    with pytest.raises(ValueError):
        dg.det_grouped_wgrad_acc(mg, G, X, torch.tensor([0, 4, 8], dtype=i32))
    with pytest.raises(TypeError):
        dg.det_grouped_wgrad_acc_bf16(mg, G, X, torch.tensor([0, 8], dtype=i32))
    a = torch.zeros(4, 2, dtype=bf)
    p = torch.zeros(2, dtype=f32)
    with pytest.raises(TypeError):
        dg.det_colsum(a, a.float(), p, p, p.clone(), p.clone())
    with pytest.raises(TypeError):
        dg.det_colsum(a, a, p.double(), p, p.clone(), p.clone())
    ids = torch.zeros(2, 4, dtype=i32)
    lg = torch.zeros(2, 4, dtype=f32)
    with pytest.raises(TypeError):
        dg.det_topk_canonicalize(ids.long(), lg, ids.clone(), lg.clone(), lg.clone())
    with pytest.raises(TypeError):
        dg.det_topk_canonicalize(ids, lg, ids.clone(), lg.clone(), lg.double())


def test_indexer_dk_validation():
    import ctypes
    L = lib()
    P = ctypes.c_void_p
    n = ctypes.c_size_t()
    f = ctypes.c_float(0.1)
    assert L.det_indexer_dk_workspace_size(64, 2048, 128, 100, None, 0, ctypes.byref(n)) == dg.DET_ERR_UNSUPPORTED
    assert L.det_indexer_dk_workspace_size(64, 512, 96, 100, None, 0, ctypes.byref(n)) == dg.DET_ERR_UNSUPPORTED
    c = dg.IndexAddCfg(2048)
    assert L.det_indexer_dk_workspace_size(64, 512, 128, 100, ctypes.byref(c), 0, ctypes.byref(n)) == \
        dg.DET_ERR_UNSUPPORTED
    assert L.det_indexer_dk_workspace_size(64, 512, 128, 100, None, 2, ctypes.byref(n)) == dg.DET_ERR_INVALID_ARG
    assert L.det_indexer_dk_workspace_size(64, 512, 128, 100, None, 1, ctypes.byref(n)) == 0
    assert n.value == 256 + 64 * 512 * 4
    assert L.det_indexer_dk_workspace_size(64, 512, 128, 100, None, 0, ctypes.byref(n)) == 0
    full = n.value
    assert L.det_index_add_workspace_size(64 * 512, 128, 100, None, 0, ctypes.byref(n)) == 0
    assert full == n.value + 3 * 64 * 512 * 4  # the coefficients by slot, then (slot, coefficient) pairs in sorted order
    dk, ids, pr, tg, q = P(0x10000000), P(0x20000000), P(0x30000000), P(0x40000000), P(0x50000000)
    ws = P(0x60000000)
    # float32 q, a NULL pointer, a short workspace, dk overlapping q: all refused before any launch
    assert L.det_indexer_dk(dk, 100, 128, 128, ids, pr, tg, 64, 512, q, 128, 1, f, None, ws, full, 0, None) == \
        dg.DET_ERR_UNSUPPORTED
    assert L.det_indexer_dk(dk, 100, 128, 128, None, pr, tg, 64, 512, q, 128, 0, f, None, ws, full, 0, None) == \
        dg.DET_ERR_INVALID_ARG
    assert L.det_indexer_dk(dk, 100, 128, 128, ids, pr, tg, 64, 512, q, 128, 0, f, None, ws, full - 256, 0, None) == \
        dg.DET_ERR_WORKSPACE
    assert L.det_indexer_dk(P(0x50000100), 100, 128, 128, ids, pr, tg, 64, 512, q, 128, 0, f, None, ws, full, 0,
                            None) == dg.DET_ERR_OVERLAP
    # empty problems are legal and launch nothing
    assert L.det_indexer_dk(None, 100, 128, 128, None, None, None, 0, 512, None, 128, 0, f, None, None, 0, 0, None) == 0


def test_mfma_rate_validation():
    L = lib()
    ops = 64 * 64 * 64
    assert L.det_mfma_rate(FAKE, ops, P(0x900000), 256, 0, 1, None) == dg.DET_ERR_INVALID_ARG    # no blocks
    assert L.det_mfma_rate(FAKE, ops, P(0x900000), 256, 1, -1, None) == dg.DET_ERR_INVALID_ARG   # negative iters
    assert L.det_mfma_rate(None, ops, P(0x900000), 256, 1, 1, None) == dg.DET_ERR_INVALID_ARG    # NULL ops
    assert L.det_mfma_rate(FAKE, ops - 1, P(0x900000), 256, 1, 1, None) == dg.DET_ERR_INVALID_ARG  # ops too short
    assert L.det_mfma_rate(FAKE, ops, P(0x900000), 511, 2, 1, None) == dg.DET_ERR_INVALID_ARG    # out too short
    assert L.det_mfma_rate(P(0x800000), ops, P(0x800100), 256, 1, 1, None) == dg.DET_ERR_OVERLAP  # out inside ops
