"""Python binding of libgptq_mi355x.so (argument marshalling only).

Every step of the hot path runs in the library's HIP kernels. PyTorch supplies
device memory (torch.empty on a ROCm device) and the current stream. There is
no CPU fallback: if the library is missing, loading raises.

Entry points (same names as include/gptq.h):
    accumulate_hessian(H, X, accumulate)      H (+)= 2 X^T X, lower triangle
    prepare_hinv(H, damp)                      U = chol_upper((H + lambda I)^-1)
    quantize_layer(W, U, bits, group_size, grid)
    act_order(H)                               column order of descending diag(H)
    permute_hessian(H, perm)                   H gathered into that order
    quantize_layer_ordered(W, U, perm, bits, group_size, grid, static_groups)
    dequant_gemv(qcodes, scales, zeros, bits, group_size, x)   y = W_hat x, one token
    pack_codes(codes, bits)
    trace_start(), trace_stop()                device time per kernel family (instrumentation)
and quantize(W, x_chunks, ...) which runs the stages of one layer (natural
order, or act-order with act_order=True).
"""

from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
# GPTQ_MI355X_LIB may name another build of the library (the debug build,
# libgptq_mi355x_debug.so, for instance)
LIB_PATH = os.environ.get("GPTQ_MI355X_LIB") or os.path.join(_HERE, "libgptq_mi355x.so")

GPTQ_OK, GPTQ_ERR_INVALID_ARG, GPTQ_ERR_WORKSPACE, GPTQ_ERR_HIP, GPTQ_ERR_UNSUPPORTED = range(5)
GPTQ_F16, GPTQ_F32, GPTQ_F64 = 0, 1, 2
GPTQ_GRID_ASYM_MINMAX, GPTQ_GRID_TERNARY, GPTQ_GRID_SYM_MINMAX = 0, 1, 2
WS_ACCUMULATE_HESSIAN, WS_PREPARE_HINV, WS_QUANTIZE_LAYER = 0, 1, 2

EXPORTED = ["gptq_abi_version", "gptq_status_string", "gptq_workspace_bytes", "gptq_accumulate_hessian",
            "gptq_prepare_hinv", "gptq_quantize_layer", "gptq_act_order", "gptq_permute_hessian",
            "gptq_quantize_layer_ordered", "gptq_dequant_gemv", "gptq_pack_codes", "gptq_trace_start",
            "gptq_trace_stop", "gptq_trace_family", "gptq_accumulate_hessian_noalloc", "gptq_prepare_hchol",
            "gptq_gemv_prepare_act_order", "gptq_dequant_gemv_perm"]
TRACE_FAMILIES = 15


GPTQ_FACTOR_HINV_CHOL, GPTQ_FACTOR_H_CHOL = 0, 1
_FACTOR = {"U": GPTQ_FACTOR_HINV_CHOL, "R": GPTQ_FACTOR_H_CHOL}


class QCfg(ctypes.Structure):
    _fields_ = [("bits", ctypes.c_int32), ("grid", ctypes.c_int32), ("group_size", ctypes.c_int32),
                ("block_size", ctypes.c_int32), ("factor", ctypes.c_int32)]


_lib = None


def load_library(path: str = LIB_PATH):
    """Load the HIP library (raises when it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with `python -m post_weight_quantization_18_amd.build`")
    lib = ctypes.CDLL(path)
    vp, i32, i64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
    lib.gptq_abi_version.restype = i32
    lib.gptq_abi_version.argtypes = []
    lib.gptq_status_string.restype = ctypes.c_char_p
    lib.gptq_status_string.argtypes = [i32]
    lib.gptq_workspace_bytes.restype = sz
    lib.gptq_workspace_bytes.argtypes = [i32, i64, i64, i64, ctypes.POINTER(QCfg)]
    lib.gptq_accumulate_hessian.restype = i32
    lib.gptq_accumulate_hessian.argtypes = [vp, i32, i64, i64, vp, i64, i64, i32, vp, sz, vp]
    lib.gptq_prepare_hinv.restype = i32
    lib.gptq_prepare_hinv.argtypes = [vp, i32, i64, i64, ctypes.c_double, vp, i32, i64, vp, vp, vp, sz, vp]
    lib.gptq_prepare_hchol.restype = i32
    lib.gptq_prepare_hchol.argtypes = [vp, i32, i64, i64, ctypes.c_double, vp, i32, i64, vp, vp, vp, sz, vp]
    lib.gptq_quantize_layer.restype = i32
    lib.gptq_quantize_layer.argtypes = [vp, i32, i64, i64, i64, vp, i32, i64, ctypes.POINTER(QCfg), vp, vp, vp, vp,
                                        vp, vp, sz, vp]
    lib.gptq_act_order.restype = i32
    lib.gptq_act_order.argtypes = [vp, i32, i64, i64, vp, vp]
    lib.gptq_permute_hessian.restype = i32
    lib.gptq_permute_hessian.argtypes = [vp, i32, i64, i64, vp, vp, i64, vp]
    lib.gptq_quantize_layer_ordered.restype = i32
    lib.gptq_quantize_layer_ordered.argtypes = [vp, i32, i64, i64, i64, vp, i32, i64, ctypes.POINTER(QCfg), vp, i32,
                                                vp, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.gptq_dequant_gemv.restype = i32
    lib.gptq_dequant_gemv.argtypes = [vp, vp, vp, i64, i64, i32, i32, vp, vp, vp]
    lib.gptq_gemv_prepare_act_order.restype = i32
    lib.gptq_gemv_prepare_act_order.argtypes = [vp, vp, i64, i64, i32, i32, vp, vp, vp, vp]
    lib.gptq_dequant_gemv_perm.restype = i32
    lib.gptq_dequant_gemv_perm.argtypes = [vp, vp, vp, i64, i64, i32, i32, vp, vp, vp, vp, vp]
    lib.gptq_pack_codes.restype = i32
    lib.gptq_pack_codes.argtypes = [vp, i64, i64, i32, vp, vp]
    lib.gptq_accumulate_hessian_noalloc.restype = i32
    lib.gptq_accumulate_hessian_noalloc.argtypes = [vp, i32, i64, i64, vp, i64, i64, i32, vp]
    lib.gptq_trace_start.restype = i32
    lib.gptq_trace_start.argtypes = []
    lib.gptq_trace_stop.restype = i32
    lib.gptq_trace_stop.argtypes = [vp, vp, vp, i32]
    lib.gptq_trace_family.restype = ctypes.c_char_p
    lib.gptq_trace_family.argtypes = [i32]
    _lib = lib
    return lib


class GPTQError(RuntimeError):
    def __init__(self, status: int, what: str):
        msg = load_library().gptq_status_string(status).decode()
        super().__init__(f"{what}: {msg}")
        self.status = status


def _check(status: int, what: str):
    if status != GPTQ_OK:
        raise GPTQError(status, what)


_DT = {torch.float16: GPTQ_F16, torch.float32: GPTQ_F32, torch.float64: GPTQ_F64}


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else ctypes.c_void_p(0)


def _stream(device) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _need_cuda(t, name):
    if not isinstance(t, torch.Tensor) or t.device.type != "cuda":
        raise ValueError(f"{name} must be a tensor on a ROCm device")


def _rowmajor_ld(t, name):
    if t.dim() != 2 or t.stride(1) != 1:
        raise ValueError(f"{name} must be a row-major 2-D tensor (unit column stride)")
    return t.stride(0)


def make_qcfg(bits: int, group_size: int = 0, grid: str = "asym", block_size: int = 128,
              factor: str = "U") -> QCfg:
    g = {"asym": GPTQ_GRID_ASYM_MINMAX, "ternary": GPTQ_GRID_TERNARY, "sym": GPTQ_GRID_SYM_MINMAX}[grid]
    return QCfg(bits, g, group_size, block_size, _FACTOR[factor])


def workspace_bytes(which: int, m: int = 0, d: int = 0, n: int = 0, cfg: QCfg | None = None) -> int:
    lib = load_library()
    return int(lib.gptq_workspace_bytes(which, m, d, n, ctypes.byref(cfg) if cfg is not None else None))


def _workspace(nbytes: int, device, workspace):
    if nbytes == 0:
        return None
    if workspace is not None and workspace.numel() * workspace.element_size() >= nbytes:
        return workspace
    return torch.empty(nbytes, dtype=torch.uint8, device=device)


def accumulate_hessian(H: torch.Tensor, X: torch.Tensor, accumulate: bool = True, workspace=None):
    """H[i][j] (+)= 2 sum_t X[t][i] X[t][j] for i >= j. H fp64 or fp32 [d, d]; X fp16 [n, d]."""
    lib = load_library()
    _need_cuda(H, "H")
    _need_cuda(X, "X")
    if X.dtype != torch.float16:
        raise ValueError("X must be fp16")
    d = H.shape[0]
    ldh = _rowmajor_ld(H, "H")
    ldx = _rowmajor_ld(X, "X") if X.shape[0] > 0 else d
    n = X.shape[0]
    # a caller's workspace is passed as it is: the call accepts any size (a
    # smaller one selects the token-major form, then fewer split partials)
    ws = workspace if workspace is not None else _workspace(workspace_bytes(WS_ACCUMULATE_HESSIAN, 0, d, n),
                                                           H.device, None)
    nbytes = 0 if ws is None else ws.numel() * ws.element_size()
    _check(lib.gptq_accumulate_hessian(_ptr(H), _DT[H.dtype], d, ldh, _ptr(X) if n else ctypes.c_void_p(0), n, ldx,
                                       int(bool(accumulate)), _ptr(ws), nbytes, _stream(H.device)),
           "gptq_accumulate_hessian")
    return H


def prepare_hinv(H: torch.Tensor, damp: float = 0.01, U: torch.Tensor | None = None,
                 u_dtype: torch.dtype = torch.float32, workspace=None):
    """Returns (U, info, lam): U upper [d, d] with U^T U = (H + lam I)^-1, info a
    1-element int32 device tensor (0 = ok), lam a 1-element fp64 device tensor."""
    lib = load_library()
    _need_cuda(H, "H")
    d = H.shape[0]
    if U is None:
        U = torch.empty(d, d, dtype=u_dtype, device=H.device)
    info = torch.empty(1, dtype=torch.int32, device=H.device)
    lam = torch.empty(1, dtype=torch.float64, device=H.device)
    ws = _workspace(workspace_bytes(WS_PREPARE_HINV, 0, d), H.device, workspace)
    _check(lib.gptq_prepare_hinv(_ptr(H), _DT[H.dtype], d, _rowmajor_ld(H, "H"), float(damp), _ptr(U), _DT[U.dtype],
                                 _rowmajor_ld(U, "U"), _ptr(info), _ptr(lam), _ptr(ws), ws.numel(),
                                 _stream(H.device)), "gptq_prepare_hinv")
    return U, info, lam


def prepare_hchol(H: torch.Tensor, damp: float = 0.01, R: torch.Tensor | None = None,
                  r_dtype: torch.dtype = torch.float64, workspace=None):
    """Returns (R, info, lam): R upper [d, d] with R R^T = H + lam I (R = U^-1), info
    and lam as prepare_hinv. Pass R to the quantize calls with factor="R"."""
    lib = load_library()
    _need_cuda(H, "H")
    d = H.shape[0]
    if R is None:
        R = torch.empty(d, d, dtype=r_dtype, device=H.device)
    info = torch.empty(1, dtype=torch.int32, device=H.device)
    lam = torch.empty(1, dtype=torch.float64, device=H.device)
    ws = _workspace(workspace_bytes(WS_PREPARE_HINV, 0, d), H.device, workspace)
    _check(lib.gptq_prepare_hchol(_ptr(H), _DT[H.dtype], d, _rowmajor_ld(H, "H"), float(damp), _ptr(R), _DT[R.dtype],
                                  _rowmajor_ld(R, "R"), _ptr(info), _ptr(lam), _ptr(ws), ws.numel(),
                                  _stream(H.device)), "gptq_prepare_hchol")
    return R, info, lam


def quantize_layer(W: torch.Tensor, U: torch.Tensor, bits: int, group_size: int = 0, grid: str = "asym",
                   block_size: int = 128, want_w_hat: bool = True, workspace=None, out=None, factor: str = "U"):
    """Returns dict(qcodes uint32 [m, d*bits/32] (as int32 storage), scales fp32 [m, ng],
    zeros uint8 [m, ng], w_hat fp32 [m, d] or None, err_sq fp32 [m]). factor "U": U =
    chol(H_d^-1) from prepare_hinv; "R": R from prepare_hchol (passed as U)."""
    lib = load_library()
    _need_cuda(W, "W")
    _need_cuda(U, "U")
    m, d = W.shape
    cfg = make_qcfg(bits, group_size, grid, block_size, factor)
    ng = d // group_size if group_size else 1
    dev = W.device
    if out is None:
        out = {
            "qcodes": torch.empty(m, d * bits // 32, dtype=torch.int32, device=dev),
            "scales": torch.empty(m, ng, dtype=torch.float32, device=dev),
            "zeros": torch.empty(m, ng, dtype=torch.uint8, device=dev),
            "w_hat": torch.empty(m, d, dtype=torch.float32, device=dev) if want_w_hat else None,
            "err_sq": torch.empty(m, dtype=torch.float32, device=dev),
        }
    ws = _workspace(workspace_bytes(WS_QUANTIZE_LAYER, m, d, 0, cfg), dev, workspace)
    _check(lib.gptq_quantize_layer(_ptr(W), _DT[W.dtype], m, d, _rowmajor_ld(W, "W"), _ptr(U), _DT[U.dtype],
                                   _rowmajor_ld(U, "U"), ctypes.byref(cfg), _ptr(out["qcodes"]), _ptr(out["scales"]),
                                   _ptr(out["zeros"]), _ptr(out["w_hat"]), _ptr(out["err_sq"]), _ptr(ws), ws.numel(),
                                   _stream(dev)), "gptq_quantize_layer")
    return out


def act_order(H: torch.Tensor, perm: torch.Tensor | None = None) -> torch.Tensor:
    """int32 device [d]: perm[j] = the column with the j-th largest H_jj (ties in index order)."""
    lib = load_library()
    _need_cuda(H, "H")
    d = H.shape[0]
    if perm is None:
        perm = torch.empty(d, dtype=torch.int32, device=H.device)
    elif perm.dtype != torch.int32 or not perm.is_contiguous() or perm.numel() != d:
        raise ValueError("perm must be contiguous int32 [d]")
    _check(lib.gptq_act_order(_ptr(H), _DT[H.dtype], d, _rowmajor_ld(H, "H"), _ptr(perm), _stream(H.device)),
           "gptq_act_order")
    return perm


_act_order = act_order  # `quantize` takes a flag of the same name


def permute_hessian(H: torch.Tensor, perm: torch.Tensor, Hp: torch.Tensor | None = None) -> torch.Tensor:
    """Hp[i][j] = H[perm[i]][perm[j]] for j <= i (lower triangles), same dtype as H."""
    lib = load_library()
    _need_cuda(H, "H")
    _need_cuda(perm, "perm")
    if perm.dtype != torch.int32 or not perm.is_contiguous():
        raise ValueError("perm must be contiguous int32")
    d = H.shape[0]
    if Hp is None:
        Hp = torch.empty(d, d, dtype=H.dtype, device=H.device)
    _check(lib.gptq_permute_hessian(_ptr(H), _DT[H.dtype], d, _rowmajor_ld(H, "H"), _ptr(perm), _ptr(Hp),
                                    _rowmajor_ld(Hp, "Hp"), _stream(H.device)), "gptq_permute_hessian")
    return Hp


def quantize_layer_ordered(W: torch.Tensor, U: torch.Tensor, perm: torch.Tensor, bits: int, group_size: int = 0,
                           grid: str = "asym", static_groups: bool = False, block_size: int = 128,
                           want_w_hat: bool = True, workspace=None, out=None, factor: str = "U"):
    """quantize_layer with the columns quantized in the order perm (U: the factor of
    the Hessian in that order). Outputs in natural column order, plus g_idx int32 [d]."""
    lib = load_library()
    _need_cuda(W, "W")
    _need_cuda(U, "U")
    _need_cuda(perm, "perm")
    if perm.dtype != torch.int32 or not perm.is_contiguous():
        raise ValueError("perm must be contiguous int32")
    m, d = W.shape
    cfg = make_qcfg(bits, group_size, grid, block_size, factor)
    ng = d // group_size if group_size else 1
    dev = W.device
    if out is None:
        out = {
            "qcodes": torch.empty(m, d * bits // 32, dtype=torch.int32, device=dev),
            "scales": torch.empty(m, ng, dtype=torch.float32, device=dev),
            "zeros": torch.empty(m, ng, dtype=torch.uint8, device=dev),
            "g_idx": torch.empty(d, dtype=torch.int32, device=dev),
            "w_hat": torch.empty(m, d, dtype=torch.float32, device=dev) if want_w_hat else None,
            "err_sq": torch.empty(m, dtype=torch.float32, device=dev),
        }
    ws = _workspace(workspace_bytes(WS_QUANTIZE_LAYER, m, d, 0, cfg), dev, workspace)
    _check(lib.gptq_quantize_layer_ordered(_ptr(W), _DT[W.dtype], m, d, _rowmajor_ld(W, "W"), _ptr(U), _DT[U.dtype],
                                           _rowmajor_ld(U, "U"), ctypes.byref(cfg), _ptr(perm),
                                           int(bool(static_groups)), _ptr(out["qcodes"]), _ptr(out["scales"]),
                                           _ptr(out["zeros"]), _ptr(out["g_idx"]), _ptr(out["w_hat"]),
                                           _ptr(out["err_sq"]), _ptr(ws), ws.numel(), _stream(dev)),
           "gptq_quantize_layer_ordered")
    return out


def dequant_gemv(qcodes: torch.Tensor, scales: torch.Tensor, zeros: torch.Tensor, bits: int, group_size: int,
                 x: torch.Tensor, y: torch.Tensor | None = None) -> torch.Tensor:
    """y fp32 [m] = W_hat x with W_hat dequantized on the fly from the packed
    codes (the quantize_layer outputs); x fp16 [d]."""
    lib = load_library()
    for t, n in ((qcodes, "qcodes"), (scales, "scales"), (zeros, "zeros"), (x, "x")):
        _need_cuda(t, n)
        if not t.is_contiguous():
            raise ValueError(f"{n} must be contiguous")
    if x.dtype != torch.float16 or scales.dtype != torch.float32 or zeros.dtype != torch.uint8:
        raise ValueError("x fp16, scales fp32, zeros uint8")
    m, d = qcodes.shape[0], x.shape[0]
    if y is None:
        y = torch.empty(m, dtype=torch.float32, device=x.device)
    _check(lib.gptq_dequant_gemv(_ptr(qcodes), _ptr(scales), _ptr(zeros), m, d, bits, group_size, _ptr(x), _ptr(y),
                                 _stream(x.device)), "gptq_dequant_gemv")
    return y


def gemv_prepare_act_order(qcodes: torch.Tensor, g_idx: torch.Tensor, bits: int, group_size: int):
    """Act-order codes (natural column order, group index g_idx) rewritten with
    the columns sorted by group. Returns (qcodes in col_perm order, col_perm
    int32 [d], info int32 device scalar: 0 when every group holds group_size
    columns)."""
    lib = load_library()
    for t, n in ((qcodes, "qcodes"), (g_idx, "g_idx")):
        _need_cuda(t, n)
        if not t.is_contiguous():
            raise ValueError(f"{n} must be contiguous")
    if g_idx.dtype != torch.int32:
        raise ValueError("g_idx must be int32")
    m, d = qcodes.shape[0], g_idx.shape[0]
    out = torch.empty_like(qcodes)
    col_perm = torch.empty(d, dtype=torch.int32, device=qcodes.device)
    info = torch.empty(1, dtype=torch.int32, device=qcodes.device)
    _check(lib.gptq_gemv_prepare_act_order(_ptr(qcodes), _ptr(g_idx), m, d, bits, group_size, _ptr(out),
                                           _ptr(col_perm), _ptr(info), _stream(qcodes.device)),
           "gptq_gemv_prepare_act_order")
    return out, col_perm, info


def dequant_gemv_perm(qcodes: torch.Tensor, scales: torch.Tensor, zeros: torch.Tensor, bits: int, group_size: int,
                      col_perm: torch.Tensor, x: torch.Tensor, x_perm: torch.Tensor | None = None,
                      y: torch.Tensor | None = None) -> torch.Tensor:
    """y fp32 [m] = W x for codes in col_perm order (gemv_prepare_act_order), x
    fp16 [d] in natural order; x_perm is the fp16 [d] buffer the gather uses."""
    lib = load_library()
    for t, n in ((qcodes, "qcodes"), (scales, "scales"), (zeros, "zeros"), (col_perm, "col_perm"), (x, "x")):
        _need_cuda(t, n)
        if not t.is_contiguous():
            raise ValueError(f"{n} must be contiguous")
    if x.dtype != torch.float16 or scales.dtype != torch.float32 or zeros.dtype != torch.uint8:
        raise ValueError("x fp16, scales fp32, zeros uint8")
    m, d = qcodes.shape[0], x.shape[0]
    if x_perm is None:
        x_perm = torch.empty(d, dtype=torch.float16, device=x.device)
    if y is None:
        y = torch.empty(m, dtype=torch.float32, device=x.device)
    _check(lib.gptq_dequant_gemv_perm(_ptr(qcodes), _ptr(scales), _ptr(zeros), m, d, bits, group_size,
                                      _ptr(col_perm), _ptr(x), _ptr(x_perm), _ptr(y), _stream(x.device)),
           "gptq_dequant_gemv_perm")
    return y


def pack_codes(codes: torch.Tensor, bits: int) -> torch.Tensor:
    """codes uint8 [m, d] -> int32 storage of the uint32 bitstream [m, d*bits/32]."""
    lib = load_library()
    _need_cuda(codes, "codes")
    if codes.dtype != torch.uint8 or not codes.is_contiguous():
        raise ValueError("codes must be contiguous uint8")
    m, d = codes.shape
    out = torch.empty(m, d * bits // 32, dtype=torch.int32, device=codes.device)
    _check(lib.gptq_pack_codes(_ptr(codes), m, d, bits, _ptr(out), _stream(codes.device)), "gptq_pack_codes")
    return out


def trace_start():
    """Start recording HIP events around every library launch from this thread."""
    _check(load_library().gptq_trace_start(), "gptq_trace_start")


def trace_stop() -> dict:
    """End the trace; {family: {"launches": n, "ms": summed device ms, "work": executed
    matrix-core flops}} for the families that launched anything."""
    lib = load_library()
    n = TRACE_FAMILIES
    launches = (ctypes.c_int64 * n)()
    ms = (ctypes.c_double * n)()
    work = (ctypes.c_double * n)()
    _check(lib.gptq_trace_stop(ctypes.cast(launches, ctypes.c_void_p), ctypes.cast(ms, ctypes.c_void_p),
                               ctypes.cast(work, ctypes.c_void_p), n), "gptq_trace_stop")
    return {lib.gptq_trace_family(k).decode(): {"launches": int(launches[k]), "ms": float(ms[k]),
                                                   "work": float(work[k])}
            for k in range(n) if launches[k]}


def quantize(W: torch.Tensor, x_chunks, bits: int, group_size: int = 0, grid: str = "asym", damp: float = 0.01,
             h_dtype: torch.dtype = torch.float64, u_dtype: torch.dtype = torch.float32, want_w_hat: bool = True,
             act_order: bool = False, static_groups: bool = False, factor: str = "U"):
    """The whole hot path of one layer: H over the chunks, U, then the column loop.
    Returns (result dict, H, U, lam). Raises when H + lam I is not positive definite.
    With act_order the columns go in descending diag(H) (result["perm"]), U is the
    factor of the permuted H, and the outputs are still in natural column order."""
    if isinstance(x_chunks, torch.Tensor):
        x_chunks = [x_chunks]
    d = W.shape[1]
    H = torch.empty(d, d, dtype=h_dtype, device=W.device)
    for i, xc in enumerate(x_chunks):
        accumulate_hessian(H, xc, accumulate=i > 0)
    perm = None
    prep = prepare_hchol if factor == "R" else prepare_hinv
    kw = {"r_dtype": torch.float64} if factor == "R" else {"u_dtype": u_dtype}
    if act_order:
        perm = _act_order(H)
        U, info, lam = prep(permute_hessian(H, perm), damp, **kw)
    else:
        U, info, lam = prep(H, damp, **kw)
    bad = int(info.item())
    if bad:
        raise GPTQError(GPTQ_ERR_INVALID_ARG, f"H + lambda I is not positive definite (reversed minor {bad})")
    if act_order:
        res = quantize_layer_ordered(W, U, perm, bits, group_size, grid, static_groups, want_w_hat=want_w_hat,
                                     factor=factor)
        res["perm"] = perm
    else:
        res = quantize_layer(W, U, bits, group_size, grid, want_w_hat=want_w_hat, factor=factor)
    return res, H, U, lam
