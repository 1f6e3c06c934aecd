"""The matrix-core step model of the oracle against the instruction itself.

det_mfma_eval runs the weight gradient's instruction (v_mfma_f32_32x32x16_bf16)
on plain operands; oracle/mfma_model.c computes the model of oracle/mfma.py on
the same inputs. More than 10^8 output elements of single instructions (each an
independent sixteen-product step into its own accumulator) and a set of long
chains must agree bit for bit: this is what lets the weight-gradient parity
tests compare the GPU with the oracle bitwise on general inputs.
"""
import time

import numpy as np
import pytest

import deterministic_gradient_reductions_amd as dg
from oracle import mfma
from tests.gpu_util import note

pytestmark = pytest.mark.gpu

CHUNK = 8192                       # instructions per chunk (8.4M output elements)
KINDS = ["normal", "realistic", "wide20", "wide60", "cancel", "subnormal", "zeros", "bits", "acc_dominant",
         "normal_c0", "realistic_big_acc", "mixed"]
N_CHUNKS = len(KINDS)              # 12 x 8192 x 1024 = 100,663,296 elements


def rne_bf16(x):
    u = np.asarray(x, np.float32).view(np.uint32).astype(np.uint64)
    return ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)


def rand_bf16(rng, shape, lo, hi):
    e = (rng.integers(lo, hi + 1, shape) + 127).astype(np.uint16)
    return (rng.integers(0, 2, shape).astype(np.uint16) << 15) | (e << 7) | rng.integers(0, 128, shape).astype(np.uint16)


def rand_f32(rng, shape, lo, hi):
    e = (rng.integers(lo, hi + 1, shape) + 127).astype(np.uint32)
    return ((rng.integers(0, 2, shape).astype(np.uint32) << 31) | (e << 23) |
            rng.integers(0, 1 << 23, shape).astype(np.uint32)).view(np.float32)


def inputs(kind, n, K, seed):
    rng = np.random.default_rng([seed, KINDS.index(kind)])
    sa, sb, sc = (n, 32, K), (n, K, 32), (n, 32, 32)
    if kind in ("normal", "normal_c0"):
        A = rne_bf16(rng.standard_normal(sa, np.float32)); B = rne_bf16(rng.standard_normal(sb, np.float32))
        C = np.zeros(sc, np.float32) if kind == "normal_c0" else rng.standard_normal(sc, np.float32) * 4
    elif kind in ("realistic", "realistic_big_acc"):
        A = rne_bf16(rng.standard_normal(sa, np.float32) * 0.02); B = rne_bf16(rng.standard_normal(sb, np.float32) * 0.02)
        C = rng.standard_normal(sc, np.float32) * (0.01 if kind == "realistic" else 1e3)
    elif kind == "wide20":
        A = rand_bf16(rng, sa, -20, 20); B = rand_bf16(rng, sb, -20, 20); C = rand_f32(rng, sc, -40, 40)
    elif kind == "wide60":
        A = rand_bf16(rng, sa, -60, 60); B = rand_bf16(rng, sb, -60, 60); C = rand_f32(rng, sc, -100, 100)
    elif kind == "cancel":
        A = rne_bf16(rng.standard_normal(sa, np.float32)); B = rne_bf16(rng.standard_normal(sb, np.float32))
        # inside every 16-wide block: the second half cancels the first, then the second quarter the first
        a4 = A.reshape(n, 32, K // 16, 16); b4 = B.reshape(n, K // 16, 16, 32)
        a4[..., 8:] = a4[..., :8] ^ np.uint16(0x8000); b4[:, :, 8:, :] = b4[:, :, :8, :]
        a4[..., 4:8] = a4[..., 0:4] ^ np.uint16(0x8000); b4[:, :, 4:8, :] = b4[:, :, 0:4, :]
        flip = rng.random(sa) < 0.2
        A[flip] ^= np.uint16(1)
        C = rng.standard_normal(sc, np.float32) * np.exp2(rng.integers(-30, 5, sc)).astype(np.float32)
    elif kind == "subnormal":
        A = rand_bf16(rng, sa, -75, -55); B = rand_bf16(rng, sb, -75, -55)
        C = (rng.integers(0, 1 << 23, sc).astype(np.uint32) | (rng.integers(0, 2, sc).astype(np.uint32) << 31)).view(np.float32)
    elif kind == "zeros":
        A = rne_bf16(rng.standard_normal(sa, np.float32)); B = rne_bf16(rng.standard_normal(sb, np.float32))
        A[rng.random(sa) < 0.7] = 0; B[rng.random(sb) < 0.3] = 0x8000
        C = np.where(rng.random(sc) < 0.5, np.float32(0.0), np.float32(-0.0)).astype(np.float32)
        m = rng.random(sc) < 0.3
        C[m] = rng.standard_normal(int(m.sum())).astype(np.float32)
    elif kind == "bits":  # any finite bf16 with exponents low enough that nothing overflows
        A = rng.integers(0, 1 << 16, sa).astype(np.uint16); B = rng.integers(0, 1 << 16, sb).astype(np.uint16)
        for X in (A, B):
            X &= np.uint16(0xBFFF)       # field exponent <= 127: |x| < 2^1
        C = rand_f32(rng, sc, -126, 4)
    elif kind == "acc_dominant":
        A = rand_bf16(rng, sa, -40, -20); B = rand_bf16(rng, sb, -40, -20); C = rand_f32(rng, sc, -30, 100)
    else:  # mixed: half normal, half wide, random zeros
        A = rand_bf16(rng, sa, -8, 8); B = rne_bf16(rng.standard_normal(sb, np.float32))
        A[rng.random(sa) < 0.1] = 0
        C = rand_f32(rng, sc, -20, 20)
    return A, B, C.astype(np.float32)


def gpu_eval(A, B, C):
    import torch
    Ad = torch.from_numpy(A.view(np.int16)).cuda().view(torch.bfloat16)
    Bd = torch.from_numpy(B.view(np.int16)).cuda().view(torch.bfloat16)
    Cd = torch.from_numpy(C).cuda()
    Dd = torch.empty_like(Cd)
    dg.det_mfma_eval(Ad, Bd, Cd, Dd)
    torch.cuda.synchronize()
    return Dd.cpu().numpy()


@pytest.mark.parametrize("kind", KINDS)
def test_single_instructions_match_the_model(kind):
    t0 = time.time()
    A, B, C = inputs(kind, CHUNK, 16, 1)
    got = gpu_eval(A, B, C).view(np.uint32)
    want = mfma.eval_c(A, B, C).view(np.uint32)
    assert ((want & 0x7F800000) != 0x7F800000).all(), "the model covers finite results only"
    bad = np.nonzero(got != want)
    note("mfma model %-18s %d elements, %d differ (%.1f s)" % (kind, got.size, len(bad[0]), time.time() - t0))
    if len(bad[0]):
        q, i, j = bad[0][0], bad[1][0], bad[2][0]
        raise AssertionError("%s: instruction %d element (%d, %d): gpu %#x model %#x" % (kind, q, i, j, got[q, i, j],
                                                                                        want[q, i, j]))


def test_element_count_is_at_least_1e8():
    assert N_CHUNKS * CHUNK * 1024 >= 10 ** 8


@pytest.mark.parametrize("kind,K", [("realistic", 512), ("normal", 256), ("wide20", 128), ("cancel", 64),
                                    ("realistic", 8192)])
def test_chains_match_the_model(kind, K):
    n = 256 if K <= 512 else 16
    A, B, C = inputs(kind, n, K, 2)
    if kind == "realistic":
        C[:] = 0.0  # weight-gradient chains start from +0
    got = gpu_eval(A, B, C).view(np.uint32)
    want = mfma.eval_c(A, B, C).view(np.uint32)
    note("mfma chains %s K=%d: %d differ of %d" % (kind, K, int((got != want).sum()), got.size))
    assert np.array_equal(got, want)


def test_rate_probe_runs_the_pattern():
    """det_mfma_rate (the measurement aid for the matrix-core ceiling) runs every MFMA it is asked for:
    with every operand 1.0, each of the 16 accumulators of a wave gains 16 per element and round, so a
    lane's sum after `iters` rounds is 16 x 16 x 16 x iters (exact in float32)."""
    import torch
    ops = torch.ones(64 * 64 * 64, dtype=torch.bfloat16, device="cuda")
    out = torch.full((3 * 256,), -1.0, dtype=torch.float32, device="cuda")
    for iters in (0, 1, 7):
        dg.det_mfma_rate(ops, out, 3, iters)
        torch.cuda.synchronize()
        assert (out == float(4096 * iters)).all(), (iters, out.unique())
