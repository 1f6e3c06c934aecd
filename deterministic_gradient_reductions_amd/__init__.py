"""Python binding of libdetgrad: deterministic, atomic-free gradient reductions on MI355X.

Argument marshalling only. Each function takes torch device tensors, passes
their data pointers, strides and the current HIP stream to the C ABI of
``libdetgrad.so`` (declared in include/detgrad.h) and raises RuntimeError with
the library's message on a non-OK status. All arithmetic runs in the HIP
kernels; there is no CPU or PyTorch fallback: if the library is not built,
every call raises.

Functions (same names as the C ABI):
    det_colsum(a, dg, A_log, dt_bias, dA_log, ddt_bias, cfg=None, atomic=False)
    det_index_add(out, ids, src, cfg=None, atomic=False)
    det_indexer_dk(dk, ids, predict, target, q, scale, cfg=None, atomic=False)
    det_grouped_dprob(dprob, dY, C, offs, cfg=None, atomic=False)
    det_grouped_wgrad_acc(main_grad, G, X, offs, cfg=None, atomic=False)
    det_grouped_dbias(dbias, dA, offs, cfg=None, atomic=False)
    det_topk_canonicalize(ids, logits, ids_out, logits_out, probs)
Every function accepts ``ws=`` (a Workspace or a uint8 device tensor) and
``stream=`` (a torch.cuda.Stream); by default a cached per-stream workspace
and torch's current stream are used.
"""
from __future__ import annotations

import ctypes
import os
import threading

__all__ = [
    "lib", "library_path", "DetError", "ColsumCfg", "IndexAddCfg", "DprobCfg", "WgradCfg", "Workspace",
    "det_abi_version", "det_colsum", "det_colsum_da", "det_colsum_noalloc", "det_colsum_select_cfg", "det_colsum_workspace_size", "det_index_add",
    "det_index_add_workspace_size", "det_index_add_bad_ids", "det_indexer_dk", "det_indexer_dk_workspace_size", "det_grouped_dprob", "det_grouped_dprob_workspace_size",
    "det_grouped_wgrad_acc", "det_grouped_wgrad_acc_workspace_size", "det_grouped_wgrad_acc_bf16",
    "det_grouped_wgrad_acc_bf16_workspace_size", "det_grouped_dbias",
    "det_grouped_dbias_workspace_size", "det_topk_canonicalize", "det_workspace_init", "det_detmath_eval", "det_mfma_eval",
    "det_mfma_rate", "DET_OK", "DET_ERR_INVALID_ARG", "DET_ERR_UNSUPPORTED", "DET_ERR_WORKSPACE", "DET_ERR_OVERLAP", "DET_ERR_HIP",
]

DET_OK, DET_ERR_INVALID_ARG, DET_ERR_UNSUPPORTED, DET_ERR_WORKSPACE, DET_ERR_OVERLAP, DET_ERR_HIP = 0, -1, -2, -3, -4, -5
DET_BF16, DET_F32 = 0, 1
WS_HEADER_BYTES = 256

library_path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libdetgrad.so")


class DetError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__("detgrad status %d: %s" % (status, msg))
        self.status = status


class ColsumCfg(ctypes.Structure):
    _fields_ = [("block_t", ctypes.c_int32), ("block_h", ctypes.c_int32)]


class IndexAddCfg(ctypes.Structure):
    _fields_ = [("chunk_rows", ctypes.c_int32)]


class DprobCfg(ctypes.Structure):
    _fields_ = [("tile_n", ctypes.c_int32), ("rows_per_wg", ctypes.c_int32)]


class DbiasCfg(ctypes.Structure):
    _fields_ = [("block_m", ctypes.c_int32), ("block_n", ctypes.c_int32)]


class WgradCfg(ctypes.Structure):
    _fields_ = [("block_m", ctypes.c_int32), ("block_n", ctypes.c_int32), ("k_tile", ctypes.c_int32),
                ("ktiles_per_split", ctypes.c_int32)]


_P = ctypes.c_void_p
_I64 = ctypes.c_int64
_I32 = ctypes.c_int32
_INT = ctypes.c_int
_SZ = ctypes.c_size_t

_SIGS = {
    "det_abi_version": ([], _INT),
    "det_last_error": ([], ctypes.c_char_p),
    "det_workspace_init": ([_P, _SZ, _P], _INT),
    "det_colsum_select_cfg": ([_I64, _I64, ctypes.POINTER(ColsumCfg)], _INT),
    "det_colsum_workspace_size": ([_I64, _I64, ctypes.POINTER(ColsumCfg), _INT, ctypes.POINTER(_SZ)], _INT),
    "det_colsum": ([_P, _I64, _I64, _P, _I64, _I64, _INT, _P, _P, _I64, _I64, _P, _P, ctypes.POINTER(ColsumCfg),
                    _P, _SZ, _INT, _P], _INT),
    "det_colsum_da": ([_P, _I64, _I64, _P, _I64, _I64, _INT, _P, _P, _I64, _I64, _P, _P, _P, _I64, _I64,
                       ctypes.POINTER(ColsumCfg), _P, _SZ, _INT, _P], _INT),
    "det_colsum_noalloc": ([_P, _I64, _I64, _P, _I64, _I64, _INT, _P, _P, _I64, _I64, _P, _P,
                            ctypes.POINTER(ColsumCfg), _INT, _P], _INT),
    "det_index_add_workspace_size": ([_I64, _I64, _I64, ctypes.POINTER(IndexAddCfg), _INT, ctypes.POINTER(_SZ)], _INT),
    "det_index_add": ([_P, _I64, _I64, _I64, _P, _I64, _P, _I64, _INT, ctypes.POINTER(IndexAddCfg), _P, _SZ, _INT,
                       _P], _INT),
    "det_index_add_bad_ids": ([_P, _SZ, ctypes.POINTER(_I64), _P], _INT),
    "det_indexer_dk_workspace_size": ([_I64, _I64, _I64, _I64, ctypes.POINTER(IndexAddCfg), _INT, ctypes.POINTER(_SZ)],
                                      _INT),
    "det_indexer_dk": ([_P, _I64, _I64, _I64, _P, _P, _P, _I64, _I64, _P, _I64, _INT, ctypes.c_float,
                        ctypes.POINTER(IndexAddCfg), _P, _SZ, _INT, _P], _INT),
    "det_grouped_dprob_workspace_size": ([_I64, _I64, ctypes.POINTER(DprobCfg), _INT, ctypes.POINTER(_SZ)], _INT),
    "det_grouped_dprob": ([_P, _P, _I64, _P, _I64, _I64, _I64, _P, _I32, ctypes.POINTER(DprobCfg), _P, _SZ, _INT,
                           _P], _INT),
    "det_grouped_wgrad_acc_workspace_size": ([_I64, _I32, _I64, _I64, ctypes.POINTER(WgradCfg), _INT,
                                              ctypes.POINTER(_SZ)], _INT),
    "det_detmath_eval": ([_P, _P, _I64, _INT, _P], _INT),
    "det_mfma_eval": ([_P, _P, _P, _P, _I64, _INT, _P], _INT),
    "det_mfma_rate": ([_P, _I64, _P, _I64, _INT, _INT, _P], _INT),
    "det_topk_canonicalize": ([_P, _P, _I64, _I64, _I64, _P, _P, _P, _I64, _P], _INT),
    "det_grouped_dbias_workspace_size": ([_I64, _I64, _I32, ctypes.POINTER(DbiasCfg), _INT, ctypes.POINTER(_SZ)],
                                         _INT),
    "det_grouped_dbias": ([_P, _I64, _P, _I64, _I64, _I64, _P, _I32, ctypes.POINTER(DbiasCfg), _P, _SZ, _INT, _P],
                          _INT),
    "det_grouped_wgrad_acc": ([_P, _I64, _I64, _P, _I64, _P, _I64, _P, _I32, _I64, _I64, _I64,
                               ctypes.POINTER(WgradCfg), _P, _SZ, _INT, _P], _INT),
    "det_grouped_wgrad_acc_bf16_workspace_size": ([_I64, _I32, _I64, _I64, ctypes.POINTER(WgradCfg),
                                                   ctypes.POINTER(_SZ)], _INT),
    "det_grouped_wgrad_acc_bf16": ([_P, _I64, _I64, _P, _I64, _P, _I64, _P, _I32, _I64, _I64, _I64,
                                    ctypes.POINTER(WgradCfg), _P, _SZ, _P], _INT),
}

_lib = None
_lock = threading.Lock()


def lib() -> ctypes.CDLL:
    """Load libdetgrad.so from the package directory (raises if it is not built)."""
    global _lib
    if _lib is None:
        with _lock:
            if _lib is None:
                if not os.path.exists(library_path):
                    raise RuntimeError("libdetgrad.so is not built; run "
                                       "`python -m deterministic_gradient_reductions_amd.build`")
                L = ctypes.CDLL(library_path)
                for name, (args, res) in _SIGS.items():
                    fn = getattr(L, name)
                    fn.argtypes = args
                    fn.restype = res
                _lib = L
    return _lib


def _check(status: int) -> None:
    if status != DET_OK:
        raise DetError(status, lib().det_last_error().decode())


def _atomic_flag(atomic) -> int:
    # bools map to 0/1; any other value goes to the library, which rejects it
    return int(atomic) if isinstance(atomic, bool) else atomic


def _stream_handle(stream):
    import torch
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else ctypes.c_void_p(0)


def det_abi_version() -> int:
    return lib().det_abi_version()


# ------------------------------------------------------------------ workspace
class Workspace:
    """A device scratch buffer with an initialised counter header.

    Owned by the caller; reused across calls on one stream. Calls that may run
    at the same time must not share a Workspace.
    """

    def __init__(self, nbytes: int, device=None, stream=None):
        import torch
        self.nbytes = max(int(nbytes), WS_HEADER_BYTES)
        # 256 extra bytes so that the start can be aligned to 256 bytes
        self._buf = torch.empty(self.nbytes + 256, dtype=torch.uint8, device=device or "cuda")
        base = self._buf.data_ptr()
        self.ptr = (base + 255) // 256 * 256
        _check(lib().det_workspace_init(ctypes.c_void_p(self.ptr), self.nbytes, _stream_handle(stream)))

    def ensure(self, nbytes: int, stream=None) -> "Workspace":
        return self if nbytes <= self.nbytes else Workspace(max(nbytes, 2 * self.nbytes), self._buf.device, stream)


_ws_cache = {}


def _workspace(need: int, ws, stream):
    if need == 0 and ws is None:
        return ctypes.c_void_p(0), 0
    if ws is None:
        import torch
        s = stream if stream is not None else torch.cuda.current_stream()
        key = (s.device.index if s.device.index is not None else torch.cuda.current_device(), s.cuda_stream)
        cur = _ws_cache.get(key)
        if cur is None or cur.nbytes < need:
            cur = Workspace(max(need, 2 * (cur.nbytes if cur else 0)), device=s.device, stream=s)
            _ws_cache[key] = cur
        ws = cur
    if isinstance(ws, Workspace):
        return ctypes.c_void_p(ws.ptr), ws.nbytes
    return ctypes.c_void_p(ws.data_ptr()), ws.numel() * ws.element_size()


def det_workspace_init(ws, stream=None) -> None:
    p, n = (ctypes.c_void_p(ws.ptr), ws.nbytes) if isinstance(ws, Workspace) else (_ptr(ws), ws.numel())
    _check(lib().det_workspace_init(p, n, _stream_handle(stream)))


def _require(t, dtype, name: str, contiguous: bool = False, unit_col: bool = False) -> None:
    """Raise TypeError/ValueError before any call when a tensor's dtype or layout does not match the C ABI."""
    import torch
    want = {"f32": torch.float32, "i32": torch.int32, "bf16": torch.bfloat16}[dtype]
    if t.dtype != want:
        raise TypeError("%s must be %s, got %s" % (name, want, t.dtype))
    if contiguous and not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    if unit_col and t.dim() >= 1 and t.shape[-1] > 1 and t.stride(-1) != 1:
        raise ValueError("%s must have unit innermost stride" % name)


def _dtype_code(t) -> int:
    import torch
    if t.dtype == torch.bfloat16:
        return DET_BF16
    if t.dtype == torch.float32:
        return DET_F32
    raise TypeError("unsupported dtype %s" % t.dtype)


# --------------------------------------------------------------------- colsum
def det_colsum_select_cfg(T: int, H: int) -> ColsumCfg:
    c = ColsumCfg()
    _check(lib().det_colsum_select_cfg(T, H, ctypes.byref(c)))
    return c


def det_colsum_workspace_size(T: int, H: int, cfg: ColsumCfg | None = None, atomic=False) -> int:
    n = _SZ()
    _check(lib().det_colsum_workspace_size(T, H, ctypes.byref(cfg) if cfg else None, _atomic_flag(atomic),
                                           ctypes.byref(n)))
    return n.value


def det_colsum(a, dg, A_log, dt_bias, dA_log, ddt_bias, cfg: ColsumCfg | None = None, atomic=False, ws=None,
               stream=None, da=None) -> None:
    """dA_log[h] += sum_t dg*g, ddt_bias[h] += sum_t dg*(-exp(A_log))*sigmoid(a+dt_bias). a, dg: [T, H].
    With ``da`` ([T, H], the dtype of ``a``), also da = dg*(-exp(A_log))*sigmoid(a+dt_bias) per element
    (det_colsum_da)."""
    T, H = a.shape
    if dg.dtype != a.dtype or tuple(dg.shape) != (T, H):
        raise TypeError("dg must have the shape and dtype of a")
    for t, n in ((A_log, "A_log"), (dt_bias, "dt_bias"), (dA_log, "dA_log"), (ddt_bias, "ddt_bias")):
        _require(t, "f32", n, contiguous=True)
    need = det_colsum_workspace_size(T, H, cfg, atomic) if atomic in (0, 1, False, True) else 0
    wp, wn = _workspace(need, ws, stream)
    head = (_ptr(a), a.stride(0), a.stride(1), _ptr(dg), dg.stride(0), dg.stride(1), _dtype_code(a),
            _ptr(A_log), _ptr(dt_bias), T, H, _ptr(dA_log), _ptr(ddt_bias))
    tail = (ctypes.byref(cfg) if cfg else None, wp, wn, _atomic_flag(atomic), _stream_handle(stream))
    if da is None:
        _check(lib().det_colsum(*head, *tail))
        return
    if da.dtype != a.dtype or tuple(da.shape) != (T, H):
        raise ValueError("da must have the shape and dtype of a")
    _check(lib().det_colsum_da(*head, _ptr(da), da.stride(0), da.stride(1), *tail))


def det_colsum_da(a, dg, A_log, dt_bias, dA_log, ddt_bias, da, **kw) -> None:
    """det_colsum plus the elementwise da [T, H] (dtype of ``a``), overwritten."""
    det_colsum(a, dg, A_log, dt_bias, dA_log, ddt_bias, da=da, **kw)


def det_colsum_noalloc(a, dg, A_log, dt_bias, dA_log, ddt_bias, cfg: ColsumCfg | None = None, atomic=False,
                       stream=None) -> None:
    """det_colsum with its slots in the library's static device scratch (no workspace, no allocation)."""
    T, H = a.shape
    if dg.dtype != a.dtype or tuple(dg.shape) != (T, H):
        raise TypeError("dg must have the shape and dtype of a")
    for t, n in ((A_log, "A_log"), (dt_bias, "dt_bias"), (dA_log, "dA_log"), (ddt_bias, "ddt_bias")):
        _require(t, "f32", n, contiguous=True)
    _check(lib().det_colsum_noalloc(_ptr(a), a.stride(0), a.stride(1), _ptr(dg), dg.stride(0), dg.stride(1),
                                    _dtype_code(a), _ptr(A_log), _ptr(dt_bias), T, H, _ptr(dA_log), _ptr(ddt_bias),
                                    ctypes.byref(cfg) if cfg else None, _atomic_flag(atomic), _stream_handle(stream)))


# ------------------------------------------------------------------ index_add
def det_index_add_workspace_size(n_src: int, dim: int, n_rows: int, cfg: IndexAddCfg | None = None,
                                 atomic=False) -> int:
    n = _SZ()
    _check(lib().det_index_add_workspace_size(n_src, dim, n_rows, ctypes.byref(cfg) if cfg else None,
                                              _atomic_flag(atomic), ctypes.byref(n)))
    return n.value


def det_index_add(out, ids, src, cfg: IndexAddCfg | None = None, atomic=False, ws=None, stream=None) -> None:
    """out[ids[p]] += src[p] for 0 <= ids[p] < out.shape[0]; out float32 [R, D], src bf16 [P, D]."""
    n_rows, dim = out.shape
    _require(out, "f32", "out", unit_col=True)
    _require(ids, "i32", "ids", contiguous=True)
    if src.dtype not in _src_dtypes():
        raise TypeError("src must be bfloat16 or float32, got %s" % src.dtype)
    _require(src, "bf16" if src.dtype == _src_dtypes()[0] else "f32", "src", unit_col=True)
    n_src = ids.numel()
    if src.dim() != 2 or src.shape[0] != n_src or src.shape[1] != dim:
        raise ValueError("src must be [ids.numel(), out.shape[1]]")
    need = det_index_add_workspace_size(n_src, dim, n_rows, cfg, atomic) if atomic in (0, 1, False, True) else 0
    wp, wn = _workspace(need, ws, stream)
    _check(lib().det_index_add(_ptr(out), n_rows, dim, out.stride(0), _ptr(ids), n_src, _ptr(src), src.stride(0),
                               _dtype_code(src), ctypes.byref(cfg) if cfg else None, wp, wn, _atomic_flag(atomic),
                               _stream_handle(stream)))


def _src_dtypes():
    import torch
    return (torch.bfloat16, torch.float32)


def det_index_add_bad_ids(ws=None, stream=None) -> int:
    wp, wn = _workspace(WS_HEADER_BYTES, ws, stream)
    c = _I64()
    _check(lib().det_index_add_bad_ids(wp, wn, ctypes.byref(c), _stream_handle(stream)))
    return c.value


# --------------------------------------------------------- fused indexer dK
def det_indexer_dk_workspace_size(Q: int, K: int, dim: int, n_rows: int, cfg: IndexAddCfg | None = None,
                                  atomic=False) -> int:
    n = _SZ()
    _check(lib().det_indexer_dk_workspace_size(Q, K, dim, n_rows, ctypes.byref(cfg) if cfg else None,
                                               _atomic_flag(atomic), ctypes.byref(n)))
    return n.value


def det_indexer_dk(dk, ids, predict, target, q, scale: float, cfg: IndexAddCfg | None = None, atomic=False,
                   ws=None, stream=None) -> None:
    """dk[ids] += the clipped-KL score gradient times the query rows, in det_index_add's canonical order.
    ids int32 [Q, K], predict and target float32 [Q, K] (contiguous), q bf16 [Q, D], dk float32 [R, D]."""
    n_rows, dim = dk.shape
    _require(dk, "f32", "dk", unit_col=True)
    _require(ids, "i32", "ids", contiguous=True)
    _require(predict, "f32", "predict", contiguous=True)
    _require(target, "f32", "target", contiguous=True)
    _require(q, "bf16", "q", unit_col=True)
    Q, K = ids.shape
    if tuple(predict.shape) != (Q, K) or tuple(target.shape) != (Q, K) or q.dim() != 2 or q.shape[0] != Q or \
            q.shape[1] != dim:
        raise ValueError("need ids, predict, target [Q, K], q [Q, D] and dk [R, D]")
    need = det_indexer_dk_workspace_size(Q, K, dim, n_rows, cfg, atomic) if atomic in (0, 1, False, True) else 0
    wp, wn = _workspace(need, ws, stream)
    _check(lib().det_indexer_dk(_ptr(dk), n_rows, dim, dk.stride(0), _ptr(ids), _ptr(predict), _ptr(target), Q, K,
                                _ptr(q), q.stride(0), DET_BF16, ctypes.c_float(float(scale)),
                                ctypes.byref(cfg) if cfg else None, wp, wn, _atomic_flag(atomic),
                                _stream_handle(stream)))


# ---------------------------------------------------------------------- dprob
def det_grouped_dprob_workspace_size(M: int, N: int, cfg: DprobCfg | None = None, atomic=False) -> int:
    n = _SZ()
    _check(lib().det_grouped_dprob_workspace_size(M, N, ctypes.byref(cfg) if cfg else None, _atomic_flag(atomic),
                                                  ctypes.byref(n)))
    return n.value


def det_grouped_dprob(dprob, dY, C, offs, cfg: DprobCfg | None = None, atomic=False, ws=None, stream=None) -> None:
    """dprob[m] += sum_n dY[m,n]*relu(C[m,n])^2 for offs[0] <= m < offs[E]; dY, C bf16 [M, N]."""
    M, N = dY.shape
    _require(dY, "bf16", "dY", unit_col=True)
    _require(C, "bf16", "C", unit_col=True)
    _require(dprob, "f32", "dprob", contiguous=True)
    _require(offs, "i32", "offs", contiguous=True)
    if tuple(C.shape) != (M, N) or dprob.numel() != M:
        raise ValueError("C must be [M, N] like dY and dprob [M]")
    need = det_grouped_dprob_workspace_size(M, N, cfg, atomic) if atomic in (0, 1, False, True) else 0
    wp, wn = _workspace(need, ws, stream)
    _check(lib().det_grouped_dprob(_ptr(dprob), _ptr(dY), dY.stride(0), _ptr(C), C.stride(0), M, N, _ptr(offs),
                                   offs.numel() - 1, ctypes.byref(cfg) if cfg else None, wp, wn,
                                   _atomic_flag(atomic), _stream_handle(stream)))


# ---------------------------------------------------------------------- dbias
def det_grouped_dbias_workspace_size(M: int, N: int, E: int, cfg: DbiasCfg | None = None, atomic=False) -> int:
    n = _SZ()
    _check(lib().det_grouped_dbias_workspace_size(M, N, E, ctypes.byref(cfg) if cfg else None, _atomic_flag(atomic),
                                                  ctypes.byref(n)))
    return n.value


def det_grouped_dbias(dbias, dA, offs, cfg: DbiasCfg | None = None, atomic=False, ws=None, stream=None) -> None:
    """dbias[e] += column sums of dA[offs[e]:offs[e+1]]; dA bf16 [M, N], dbias fp32 [E, N]."""
    M, N = dA.shape
    E = offs.numel() - 1
    _require(dA, "bf16", "dA", unit_col=True)
    _require(dbias, "f32", "dbias", unit_col=True)
    _require(offs, "i32", "offs", contiguous=True)
    if tuple(dbias.shape) != (E, N):
        raise ValueError("dbias must be [E, N] with E = offs.numel() - 1")
    need = det_grouped_dbias_workspace_size(M, N, E, cfg, atomic) if atomic in (0, 1, False, True) else 0
    wp, wn = _workspace(need, ws, stream)
    _check(lib().det_grouped_dbias(_ptr(dbias), dbias.stride(0), _ptr(dA), dA.stride(0), M, N, _ptr(offs), E,
                                   ctypes.byref(cfg) if cfg else None, wp, wn, _atomic_flag(atomic),
                                   _stream_handle(stream)))


# ------------------------------------------------------------- compact top-k
def det_topk_canonicalize(ids, logits, ids_out, logits_out, probs, stream=None) -> None:
    """Per row of the [Q, K] compact top-k: ids sorted (padding last), logits permuted alike,
    softmax recomputed in that order. ids int32, logits and outputs float32 (ids_out int32)."""
    Q, K = ids.shape
    _require(ids, "i32", "ids")
    _require(ids_out, "i32", "ids_out")
    for t, n in ((logits, "logits"), (logits_out, "logits_out"), (probs, "probs")):
        _require(t, "f32", n)
    if ids.stride(1) != 1 or logits.stride(1) != 1 or ids.stride(0) != logits.stride(0):
        raise ValueError("ids and logits need unit column stride and one row stride")
    if not (ids_out.stride(0) == logits_out.stride(0) == probs.stride(0)) or \
            ids_out.stride(1) != 1 or logits_out.stride(1) != 1 or probs.stride(1) != 1:
        raise ValueError("outputs need unit column stride and one row stride")
    _check(lib().det_topk_canonicalize(_ptr(ids), _ptr(logits), Q, K, ids.stride(0), _ptr(ids_out),
                                       _ptr(logits_out), _ptr(probs), probs.stride(0), _stream_handle(stream)))


# ---------------------------------------------------------------------- wgrad
def det_grouped_wgrad_acc_workspace_size(T_total: int, E: int, M: int, N: int, cfg: WgradCfg | None = None,
                                         atomic=False) -> int:
    n = _SZ()
    _check(lib().det_grouped_wgrad_acc_workspace_size(T_total, E, M, N, ctypes.byref(cfg) if cfg else None,
                                                      _atomic_flag(atomic), ctypes.byref(n)))
    return n.value


def _wgrad_operands(G, X, offs, E, M, N) -> None:
    _require(G, "bf16", "G", unit_col=True)
    _require(X, "bf16", "X", unit_col=True)
    _require(offs, "i32", "offs", contiguous=True)
    if G.dim() != 2 or X.dim() != 2 or G.shape[1] != M or X.shape[1] != N or X.shape[0] != G.shape[0]:
        raise ValueError("G must be [T, M] and X [T, N] for main_grad [E, M, N]")
    if offs.numel() != E + 1:
        raise ValueError("offs must hold E + 1 offsets")


def det_grouped_wgrad_acc(main_grad, G, X, offs, cfg: WgradCfg | None = None, atomic=False, ws=None,
                          stream=None) -> None:
    """main_grad[e] += G[offs[e]:offs[e+1]]^T X[offs[e]:offs[e+1]]; main_grad fp32 [E, M, N]."""
    E, M, N = main_grad.shape
    T_total = G.shape[0]
    _require(main_grad, "f32", "main_grad", unit_col=True)
    _wgrad_operands(G, X, offs, E, M, N)
    need = det_grouped_wgrad_acc_workspace_size(T_total, E, M, N, cfg, atomic) if atomic in (0, 1, False, True) else 0
    wp, wn = _workspace(need, ws, stream)
    _check(lib().det_grouped_wgrad_acc(_ptr(main_grad), main_grad.stride(0), main_grad.stride(1), _ptr(G), G.stride(0),
                                       _ptr(X), X.stride(0), _ptr(offs), E, T_total, M, N,
                                       ctypes.byref(cfg) if cfg else None, wp, wn, _atomic_flag(atomic),
                                       _stream_handle(stream)))


def det_grouped_wgrad_acc_bf16_workspace_size(T_total: int, E: int, M: int, N: int,
                                              cfg: WgradCfg | None = None) -> int:
    n = _SZ()
    _check(lib().det_grouped_wgrad_acc_bf16_workspace_size(T_total, E, M, N, ctypes.byref(cfg) if cfg else None,
                                                           ctypes.byref(n)))
    return n.value


def det_grouped_wgrad_acc_bf16(main_grad, G, X, offs, cfg: WgradCfg | None = None, ws=None, stream=None) -> None:
    """bf16 main_grad [E, M, N]: main_grad[e] <- bf16(main_grad[e] + bf16(G_e^T X_e)), deterministic only."""
    import torch
    if main_grad.dtype != torch.bfloat16:
        raise TypeError("main_grad must be bfloat16")
    E, M, N = main_grad.shape
    T_total = G.shape[0]
    _require(main_grad, "bf16", "main_grad", unit_col=True)
    _wgrad_operands(G, X, offs, E, M, N)
    wp, wn = _workspace(det_grouped_wgrad_acc_bf16_workspace_size(T_total, E, M, N, cfg), ws, stream)
    _check(lib().det_grouped_wgrad_acc_bf16(_ptr(main_grad), main_grad.stride(0), main_grad.stride(1), _ptr(G),
                                            G.stride(0), _ptr(X), X.stride(0), _ptr(offs), E, T_total, M, N,
                                            ctypes.byref(cfg) if cfg else None, wp, wn, _stream_handle(stream)))


# ---------------------------------------------------------------- diagnostics
DETMATH_FN = {"exp32": 0, "log1p32": 1, "softplus32": 2, "sigmoid32": 3}


def det_detmath_eval(x, y, fn: str, stream=None) -> None:
    """y = fn(x) elementwise on the GPU with the gate's detmath sequences (tests only)."""
    _check(lib().det_detmath_eval(_ptr(x), _ptr(y), x.numel(), DETMATH_FN[fn], _stream_handle(stream)))


def det_mfma_eval(A, B, C, D, stream=None) -> None:
    """D[q] = chain of the weight gradient's matrix-core instruction over the 16-wide k blocks of
    A[q] [32, K] and B[q] [K, 32] (bf16), starting from C[q] [32, 32] float32 (tests only)."""
    import torch
    n, m, K = A.shape
    if A.dtype != torch.bfloat16 or B.dtype != torch.bfloat16 or C.dtype != torch.float32 or D.dtype != torch.float32:
        raise TypeError("A, B must be bfloat16 and C, D float32")
    if m != 32 or K % 16 or tuple(B.shape) != (n, K, 32) or tuple(C.shape) != (n, 32, 32) or \
            tuple(D.shape) != (n, 32, 32):
        raise ValueError("shapes must be A [n,32,K], B [n,K,32], C and D [n,32,32] with K a multiple of 16")
    if not (A.is_contiguous() and B.is_contiguous() and C.is_contiguous() and D.is_contiguous()):
        raise ValueError("A, B, C and D must be contiguous")
    _check(lib().det_mfma_eval(_ptr(A), _ptr(B), _ptr(C), _ptr(D), n, K // 16, _stream_handle(stream)))


def det_mfma_rate(ops, out, blocks: int, iters: int, stream=None) -> None:
    """Measurement aid: `blocks` workgroups run `iters` rounds of the weight gradient's 4 x 4 MFMA pattern on
    operand values taken from ops (bf16, >= 64*64*64 values), 16 * 32768 flops per wave and round; out
    (float32, >= 256 * blocks) receives each lane's accumulator sum."""
    import torch
    if ops.dtype != torch.bfloat16 or out.dtype != torch.float32:
        raise TypeError("ops must be bfloat16 and out float32")
    if not (ops.is_contiguous() and out.is_contiguous()):
        raise ValueError("ops and out must be contiguous")
    _check(lib().det_mfma_rate(_ptr(ops), ops.numel(), _ptr(out), out.numel(), blocks, iters, _stream_handle(stream)))
