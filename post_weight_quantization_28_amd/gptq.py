"""Python binding of libgptq (ctypes): argument marshalling only.

Every step of the computation runs in the HIP kernels of libgptq.so; PyTorch
provides device memory and the current stream. There is no fallback: if the
library is not built, or a tensor is not on the GPU, the calls raise.
The names mirror include/gptq.h.
"""
import ctypes
import os
from dataclasses import dataclass

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libgptq.so")

OK, EINVAL, ENOTPD, ENONFINITE, EHIP, EWORKSPACE = 0, -1, -2, -3, -4, -5
BF16, F32 = 0, 1
PROF_CLASSES = ["hessian_syrk", "hessian_reduce", "quantize", "factor", "prep_finish", "sweep", "far_field",
                "inverse_x6"]


class GPTQError(RuntimeError):
    def __init__(self, status, message, fail_col=None):
        super().__init__(f"{message} (status {status})"
                         + ("" if fail_col is None or fail_col < 0 else f", column {fail_col}"))
        self.status = status
        self.fail_col = fail_col


class _Params(ctypes.Structure):
    _fields_ = [("struct_size", ctypes.c_uint32), ("bits", ctypes.c_int32),
                ("group", ctypes.c_int32), ("damp", ctypes.c_float),
                ("block", ctypes.c_int32), ("act_order", ctypes.c_int32),
                ("n_quant", ctypes.c_int64), ("sym", ctypes.c_int32), ("scale_fp16", ctypes.c_int32),
                ("reserved", ctypes.c_int32)]


class _Outputs(ctypes.Structure):
    _fields_ = [("qweight", ctypes.c_void_p), ("codes", ctypes.c_void_p),
                ("scales", ctypes.c_void_p), ("zeros", ctypes.c_void_p),
                ("g_idx", ctypes.c_void_p), ("w_hat", ctypes.c_void_p),
                ("row_loss", ctypes.c_void_p)]


_lib = None


def load():
    """Load libgptq.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is not built; run __graft_entry__.build() "
                           "or python post_weight_quantization_28_amd/build_lib.py")
    lib = ctypes.CDLL(LIB_PATH)
    c_i64, c_vp, c_sz = ctypes.c_int64, ctypes.c_void_p, ctypes.c_size_t
    sigs = {
        "gptq_hessian_workspace_bytes": [c_i64, c_i64, ctypes.c_int, ctypes.POINTER(c_sz)],
        "gptq_accumulate_hessian": [c_vp, c_vp, ctypes.c_int, c_i64, c_i64, c_i64, c_vp,
                                    ctypes.c_int, c_vp, c_sz],
        "gptq_workspace_bytes": [c_i64, c_i64, ctypes.POINTER(_Params), ctypes.POINTER(c_sz)],
        "gptq_quantize_layer": [c_vp, c_vp, ctypes.c_int, c_i64, c_i64, c_i64, c_vp,
                                ctypes.POINTER(_Params), c_vp, c_sz, ctypes.POINTER(_Outputs),
                                ctypes.POINTER(c_i64)],
        "gptq_factor_hinv": [c_vp, c_vp, c_i64, ctypes.POINTER(_Params), c_vp, c_sz, c_vp, c_vp,
                             ctypes.POINTER(c_i64)],
        "gptq_pack_codes": [c_vp, c_vp, c_i64, c_i64, ctypes.c_int32, c_vp],
        "gptq_unpack_codes": [c_vp, c_vp, c_i64, c_i64, ctypes.c_int32, c_vp],
        "gptq_dequant_matmul_workspace_bytes": [c_i64, c_i64, c_i64, ctypes.c_int32, ctypes.c_int32,
                                                ctypes.c_int32, ctypes.POINTER(c_sz)],
        "gptq_dequant_matmul": [c_vp, c_vp, ctypes.c_int32, c_i64, c_i64, c_i64, c_vp, c_vp, c_vp, c_vp,
                                c_i64, ctypes.c_int32, ctypes.c_int32, c_vp, c_i64, c_vp, c_sz],
        "gptq_dequant_matmul_noalloc": [c_vp, c_vp, ctypes.c_int32, c_i64, c_i64, c_i64, c_vp, c_vp, c_vp,
                                        c_vp, c_i64, ctypes.c_int32, ctypes.c_int32, c_vp, c_i64],
        "gptq_repack_act_order_workspace_bytes": [c_i64, c_i64, ctypes.POINTER(c_sz)],
        "gptq_repack_act_order": [c_vp, c_vp, c_vp, c_i64, c_i64, ctypes.c_int32, ctypes.c_int32, c_vp, c_vp,
                                  c_vp, c_sz],
        "gptq_eora_workspace_bytes": [c_i64, c_i64, ctypes.c_int32, ctypes.c_int32, ctypes.POINTER(c_sz)],
        "gptq_eora": [c_vp, c_vp, ctypes.c_int, c_vp, c_i64, c_i64, c_i64, c_vp, ctypes.c_int32, ctypes.c_int32,
                      c_vp, c_vp, c_vp, c_vp, c_sz],
        "gptq_refine_workspace_bytes": [c_i64, c_i64, ctypes.c_int32, ctypes.POINTER(c_sz)],
        "gptq_refine_lowrank": [c_vp, c_vp, ctypes.c_int, c_i64, c_i64, c_i64, c_vp, ctypes.c_int32, ctypes.c_int32,
                                c_vp, c_vp, c_vp, c_vp, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, c_vp, c_vp,
                                c_vp, c_vp, c_sz],
        "gptq_quantize_rtn": [c_vp, c_vp, c_i64, c_i64, c_i64, ctypes.c_int32, ctypes.c_int32, c_vp, c_vp, c_vp,
                              c_vp],
        "gptq_profile_enable": [ctypes.c_int],
        "gptq_profile_collect": [ctypes.POINTER(ctypes.c_double), ctypes.POINTER(c_i64)],
    }
    for name, args in sigs.items():
        f = getattr(lib, name)
        f.argtypes = args
        f.restype = ctypes.c_int
    lib.gptq_status_string.argtypes = [ctypes.c_int]
    lib.gptq_status_string.restype = ctypes.c_char_p
    lib.gptq_last_error.argtypes = []
    lib.gptq_last_error.restype = ctypes.c_char_p
    _lib = lib
    return lib


def _check(st, fail_col=None):
    if st != OK:
        lib = load()
        msg = lib.gptq_last_error().decode() or lib.gptq_status_string(st).decode()
        raise GPTQError(st, msg, fail_col)


def _dev(t, name):
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError(f"{name} must be a CUDA (HIP) tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _dtype_code(t):
    if t.dtype == torch.bfloat16:
        return BF16
    if t.dtype == torch.float32:
        return F32
    raise TypeError("tensor must be bfloat16 or float32")


def _workspace(nbytes, device, workspace):
    if nbytes == 0:
        return None, ctypes.c_void_p(0)
    if workspace is not None:
        if workspace.numel() * workspace.element_size() < nbytes:
            raise ValueError("workspace too small")
        return workspace, _dev(workspace, "workspace")
    ws = torch.empty(nbytes, dtype=torch.uint8, device=device)
    return ws, _dev(ws, "workspace")


def make_params(bits=4, group=128, damp=0.01, block=128, act_order=False, n_quant=None, n=None, sym=False,
                scale_fp16=False):
    nq = n if n_quant is None else n_quant
    return _Params(ctypes.sizeof(_Params), int(bits), int(group), float(damp), int(block),
                   int(bool(act_order)), int(nq), int(bool(sym)), int(bool(scale_fp16)), 0)


# ---------------------------------------------------------------- Hessian
def hessian_workspace_bytes(T, n, dtype=torch.bfloat16):
    lib = load()
    out = ctypes.c_size_t(0)
    _check(lib.gptq_hessian_workspace_bytes(int(T), int(n), BF16 if dtype == torch.bfloat16 else F32,
                                            ctypes.byref(out)))
    return out.value


def accumulate_hessian(X, H=None, zero_first=None, workspace=None):
    """H (n x n fp32) += 2 X^T X on the GPU; a new zeroed H when None."""
    lib = load()
    _dev(X, "X")
    T, n = X.shape
    if H is None:
        H = torch.empty((n, n), dtype=torch.float32, device=X.device)
        zero_first = True
    zero_first = bool(zero_first)
    need = hessian_workspace_bytes(T, n, X.dtype)
    ws, wsp = _workspace(need, X.device, workspace)
    _check(lib.gptq_accumulate_hessian(_stream(), _dev(X, "X"), _dtype_code(X), T, n, X.stride(0),
                                       _dev(H, "H"), int(zero_first), wsp, need))
    return H


# ---------------------------------------------------------------- quantize
@dataclass
class QuantResult:
    qweight: torch.Tensor
    scales: torch.Tensor
    zeros: torch.Tensor
    g_idx: torch.Tensor
    w_hat: torch.Tensor
    row_loss: torch.Tensor
    codes: torch.Tensor = None


def workspace_bytes(d_out, n, params):
    lib = load()
    out = ctypes.c_size_t(0)
    _check(lib.gptq_workspace_bytes(int(d_out), int(n), ctypes.byref(params), ctypes.byref(out)))
    return out.value


def quantize_layer(W, H=None, X=None, bits=4, group=128, damp=0.01, block=128, act_order=False,
                   n_quant=None, want_codes=False, workspace=None, outputs=None, sym=False, scale_fp16=False):
    """GPTQ of W (d_out x n, bf16 or fp32) against H = 2 X^T X (given, or
    accumulated from X first). Returns a QuantResult of device tensors.
    ``outputs`` may hold preallocated tensors (same names as QuantResult)."""
    lib = load()
    _dev(W, "W")
    if H is None:
        if X is None:
            raise ValueError("need H or X")
        H = accumulate_hessian(X)
    _dev(H, "H")
    d_out, n = W.shape
    p = make_params(bits, group, damp, block, act_order, n_quant, n, sym, scale_fp16)
    nq = p.n_quant
    dev = W.device
    o = outputs or {}
    wpr = (nq * bits + 31) // 32
    res = QuantResult(
        qweight=o.get("qweight", torch.empty((d_out, wpr), dtype=torch.int32, device=dev)),
        scales=o.get("scales", torch.empty((d_out, nq // group), dtype=torch.float32, device=dev)),
        zeros=o.get("zeros", torch.empty((d_out, nq // group), dtype=torch.uint8, device=dev)),
        g_idx=o.get("g_idx", torch.empty((nq,), dtype=torch.int32, device=dev)),
        w_hat=o.get("w_hat", torch.empty((d_out, n), dtype=torch.float32, device=dev)),
        row_loss=o.get("row_loss", torch.empty((d_out,), dtype=torch.float32, device=dev)),
        codes=o.get("codes", torch.empty((d_out, nq), dtype=torch.uint8, device=dev)) if want_codes else None)
    need = workspace_bytes(d_out, n, p)
    ws, wsp = _workspace(need, dev, workspace)
    outs = _Outputs(res.qweight.data_ptr(), res.codes.data_ptr() if want_codes else None,
                    res.scales.data_ptr(), res.zeros.data_ptr(), res.g_idx.data_ptr(),
                    res.w_hat.data_ptr(), res.row_loss.data_ptr())
    for name in ("qweight", "scales", "zeros", "g_idx", "w_hat", "row_loss"):
        _dev(getattr(res, name), name)
    fail = ctypes.c_int64(-1)
    st = lib.gptq_quantize_layer(_stream(), _dev(W, "W"), _dtype_code(W), d_out, n, W.stride(0),
                                 _dev(H, "H"), ctypes.byref(p), wsp, need, ctypes.byref(outs),
                                 ctypes.byref(fail))
    _check(st, fail.value)
    return res


def factor_hinv(H, damp=0.01, act_order=False, n_quant=None, workspace=None):
    """(U, perm): upper Cholesky factor of the damped Hessian's inverse in
    processing order, and the processing-order permutation."""
    lib = load()
    n = H.shape[0]
    p = make_params(4, 128, damp, 128, act_order, n_quant, n)
    need = workspace_bytes(0, n, p)
    ws, wsp = _workspace(need, H.device, workspace)
    U = torch.empty((n, n), dtype=torch.float32, device=H.device)
    perm = torch.empty((n,), dtype=torch.int32, device=H.device)
    fail = ctypes.c_int64(-1)
    st = lib.gptq_factor_hinv(_stream(), _dev(H, "H"), n, ctypes.byref(p), wsp, need, _dev(U, "U"),
                              _dev(perm, "perm"), ctypes.byref(fail))
    _check(st, fail.value)
    return U, perm


# ---------------------------------------------------------------- inference
def dequant_matmul_workspace_bytes(M, n, d_out, bits, group, permuted=False):
    lib = load()
    out = ctypes.c_size_t(0)
    _check(lib.gptq_dequant_matmul_workspace_bytes(int(M), int(n), int(d_out), int(bits), int(group),
                                                   int(bool(permuted)), ctypes.byref(out)))
    return out.value


def dequant_matmul(X, qweight, scales, zeros, bits, group, perm=None, out=None, workspace=None):
    """Y = X W_hat^T (M x d_out fp32) from a packed layer: X (M x n bf16),
    qweight (d_out x n*bits/32 int32/uint32 words), scales (d_out x n/group
    fp32), zeros (d_out x n/group uint8). With perm (from repack_act_order)
    the layer is in that column order and X's columns are gathered by it."""
    lib = load()
    _dev(X, "X")
    if X.dtype != torch.bfloat16:
        raise TypeError("X must be bfloat16")
    M, n = X.shape
    d_out = qweight.shape[0]
    Y = out if out is not None else torch.empty((M, d_out), dtype=torch.float32, device=X.device)
    _dev(Y, "Y")
    need = dequant_matmul_workspace_bytes(M, n, d_out, bits, group, perm is not None)
    ws, wsp = _workspace(need, X.device, workspace)
    pp = _dev(perm, "perm") if perm is not None else ctypes.c_void_p(0)
    _check(lib.gptq_dequant_matmul(_stream(), _dev(X, "X"), BF16, M, n, n, _dev(qweight, "qweight"),
                                   _dev(scales, "scales"), _dev(zeros, "zeros"), pp, d_out, int(bits),
                                   int(group), _dev(Y, "Y"), d_out, wsp, need))
    return Y


NOALLOC_SCRATCH_BYTES = 64 * 1024 * 1024


def dequant_matmul_noalloc(X, qweight, scales, zeros, bits, group, perm=None, out=None):
    """dequant_matmul without a workspace: the library's static per-GPU
    scratch holds the gathered activations and partials (at most
    NOALLOC_SCRATCH_BYTES; larger products raise). ``out`` (M x d_out fp32)
    lets a caller that cannot allocate pass Y as well. Calls that may overlap
    on one GPU race."""
    lib = load()
    _dev(X, "X")
    if X.dtype != torch.bfloat16:
        raise TypeError("X must be bfloat16")
    M, n = X.shape
    d_out = qweight.shape[0]
    Y = out if out is not None else torch.empty((M, d_out), dtype=torch.float32, device=X.device)
    _dev(Y, "Y")
    pp = _dev(perm, "perm") if perm is not None else ctypes.c_void_p(0)
    _check(lib.gptq_dequant_matmul_noalloc(_stream(), _dev(X, "X"), BF16, M, n, n, _dev(qweight, "qweight"),
                                           _dev(scales, "scales"), _dev(zeros, "zeros"), pp, d_out, int(bits),
                                           int(group), _dev(Y, "Y"), d_out))
    return Y


def repack_act_order(qweight, g_idx, n, bits, group, workspace=None):
    """(qweight in group-contiguous column order, perm): see gptq_repack_act_order."""
    lib = load()
    d_out = qweight.shape[0]
    out = torch.empty_like(qweight)
    perm = torch.empty((n,), dtype=torch.int32, device=qweight.device)
    c = ctypes.c_size_t(0)
    _check(lib.gptq_repack_act_order_workspace_bytes(d_out, n, ctypes.byref(c)))
    ws, wsp = _workspace(c.value, qweight.device, workspace)
    _check(lib.gptq_repack_act_order(_stream(), _dev(qweight, "qweight"), _dev(g_idx, "g_idx"), d_out, n,
                                     int(bits), int(group), _dev(out, "qweight_out"), _dev(perm, "perm"),
                                     wsp, c.value))
    return out, perm


# ---------------------------------------------------------------- EoRA
def eora_workspace_bytes(d_out, n, rank, with_h=True):
    lib = load()
    out = ctypes.c_size_t(0)
    _check(lib.gptq_eora_workspace_bytes(int(d_out), int(n), int(rank), int(bool(with_h)), ctypes.byref(out)))
    return out.value


def eora(W, W_hat, H=None, rank=32, iters=0, workspace=None):
    """(B, A, sigma): the rank-r EoRA adapter of W - W_hat in the eigenspace
    of H (plain SVD of W - W_hat when H is None); W_hat + B A is the
    compensated layer. W bf16 or fp32 (d_out x n), W_hat fp32, H fp32 n x n."""
    lib = load()
    _dev(W, "W")
    _dev(W_hat, "W_hat")
    if W_hat.dtype != torch.float32:
        raise TypeError("W_hat must be float32")
    d_out, n = W.shape
    if H is not None:
        _dev(H, "H")
        if H.dtype != torch.float32:
            raise TypeError("H must be float32")
    dev = W.device
    B = torch.empty((d_out, rank), dtype=torch.float32, device=dev)
    A = torch.empty((rank, n), dtype=torch.float32, device=dev)
    sigma = torch.empty((rank,), dtype=torch.float32, device=dev)
    need = eora_workspace_bytes(d_out, n, rank, H is not None)
    ws, wsp = _workspace(need, dev, workspace)
    _check(lib.gptq_eora(_stream(), _dev(W, "W"), _dtype_code(W), _dev(W_hat, "W_hat"), d_out, n, W.stride(0),
                         _dev(H, "H") if H is not None else ctypes.c_void_p(0), int(rank), int(iters),
                         _dev(B, "B"), _dev(A, "A"), _dev(sigma, "sigma"), wsp, need))
    return B, A, sigma


# ---------------------------------------------------------------- OLrC / Bid-Up
def refine_workspace_bytes(d_out, n, rank):
    lib = load()
    out = ctypes.c_size_t(0)
    _check(lib.gptq_refine_workspace_bytes(int(d_out), int(n), int(rank), ctypes.byref(out)))
    return out.value


def refine_lowrank(W, H, codes, scales, zeros, g_idx, bits, group, rank=32, cycles=1, passes=1, workspace=None):
    """OLrC / Bid-Up cycles on a quantized layer: returns (codes, B, A,
    w_hat) with the codes refined on their fixed grid (a new tensor; the
    input is not modified), W ~ w_hat + B A."""
    lib = load()
    for t, nm in ((W, "W"), (H, "H"), (codes, "codes"), (scales, "scales"), (zeros, "zeros"), (g_idx, "g_idx")):
        _dev(t, nm)
    d_out, n = W.shape
    dev = W.device
    c = codes.clone()
    B = torch.empty((d_out, rank), dtype=torch.float32, device=dev)
    A = torch.empty((rank, n), dtype=torch.float32, device=dev)
    w_hat = torch.empty((d_out, n), dtype=torch.float32, device=dev)
    need = refine_workspace_bytes(d_out, n, rank)
    ws, wsp = _workspace(need, dev, workspace)
    _check(lib.gptq_refine_lowrank(_stream(), _dev(W, "W"), _dtype_code(W), d_out, n, W.stride(0), _dev(H, "H"),
                                   int(bits), int(group), _dev(g_idx, "g_idx"), _dev(scales, "scales"),
                                   _dev(zeros, "zeros"), _dev(c, "codes"), int(rank), int(cycles), int(passes),
                                   _dev(B, "B"), _dev(A, "A"), _dev(w_hat, "w_hat"), wsp, need))
    return c, B, A, w_hat


# ---------------------------------------------------------------- round-to-nearest
def quantize_rtn(X, bits, group):
    """(codes, scales, zeros, x_hat) of X (rows x cols fp32) on the affine
    grid, groups of `group` columns, no feedback."""
    lib = load()
    _dev(X, "X")
    if X.dtype != torch.float32:
        raise TypeError("X must be float32")
    rows, cols = X.shape
    dev = X.device
    codes = torch.empty((rows, cols), dtype=torch.uint8, device=dev)
    scales = torch.empty((rows, cols // group), dtype=torch.float32, device=dev)
    zeros = torch.empty((rows, cols // group), dtype=torch.uint8, device=dev)
    xh = torch.empty((rows, cols), dtype=torch.float32, device=dev)
    _check(lib.gptq_quantize_rtn(_stream(), _dev(X, "X"), rows, cols, X.stride(0), int(bits), int(group),
                                 _dev(codes, "codes"), _dev(scales, "scales"), _dev(zeros, "zeros"), _dev(xh, "x_hat")))
    return codes, scales, zeros, xh


# ---------------------------------------------------------------- packing
def pack_codes(codes, bits):
    lib = load()
    _dev(codes, "codes")
    d_out, nq = codes.shape
    qw = torch.empty((d_out, (nq * bits + 31) // 32), dtype=torch.int32, device=codes.device)
    _check(lib.gptq_pack_codes(_stream(), _dev(codes, "codes"), d_out, nq, bits, _dev(qw, "qweight")))
    return qw


def unpack_codes(qweight, n_quant, bits):
    lib = load()
    _dev(qweight, "qweight")
    d_out = qweight.shape[0]
    codes = torch.empty((d_out, n_quant), dtype=torch.uint8, device=qweight.device)
    _check(lib.gptq_unpack_codes(_stream(), _dev(qweight, "qweight"), d_out, n_quant, bits,
                                 _dev(codes, "codes")))
    return codes


# ---------------------------------------------------------------- timing
def profile_enable(on=True, phases=False):
    """Start (clearing) or stop event timing; phases=True also times the
    phases of quantize_layer (for an untimed breakdown pass)."""
    _check(load().gptq_profile_enable(0 if not on else (2 if phases else 1)))


def profile_collect():
    """{kernel class: (total ms, launches)} since profile_enable."""
    lib = load()
    n = len(PROF_CLASSES)
    ms = (ctypes.c_double * n)()
    cnt = (ctypes.c_int64 * n)()
    _check(lib.gptq_profile_collect(ms, cnt))
    return {c: (ms[i], cnt[i]) for i, c in enumerate(PROF_CLASSES)}
