"""ctypes binding of the C ABI in include/fp8_linear.h.

Argument marshalling only: every step of the computation runs in the HIP
library ``_lib/libfp8linear.so``.  torch supplies device memory
(``torch.empty``) and the current stream; nothing here computes on tensor
data, and there is no fallback: if the library is missing, loading raises.

Names follow the C entry points.  Tensors are passed as ``data_ptr()``; the
caller's tensors must be contiguous CUDA (HIP) tensors of the documented
dtypes (bf16 for x / outputs, uint8 for the fp8 codes, float32 for scales).
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Tuple

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "_lib", "libfp8linear.so")

FP8L_OK, FP8L_EINVAL, FP8L_ESHAPE, FP8L_EALIGN, FP8L_EWORKSPACE, FP8L_EHIP = range(6)
FP8L_TENSORWISE, FP8L_ROWWISE, FP8L_E5M2 = 0, 1, 2
EXPORTS = ("fp8_linear_workspace_bytes", "fp8_linear_quantize",
           "fp8_linear_quantize_noalloc", "fp8_linear_amax",
           "fp8_linear_quantize_scaled", "fp8_linear_fwd", "fp8_linear_bwd",
           "fp8_linear_bwd_w_f32", "fp8_linear_bwd_x_acc", "fp8_linear_gemm_grouped",
           "fp8_linear_encode_e4m3",
           "fp8_linear_encode_e5m2", "fp8_swiglu_workspace_bytes", "fp8_swiglu_fwd",
           "fp8_swiglu_bwd", "fp8_linear_status_string", "fp8_linear_version")


FP8L_MAX_GROUP = 4


class GemmProblem(ctypes.Structure):
    """fp8l_gemm_problem of the C ABI."""
    _fields_ = [("a", ctypes.c_void_p), ("sa", ctypes.c_void_p), ("b", ctypes.c_void_p),
                ("sb", ctypes.c_void_p), ("c", ctypes.c_void_p), ("m", ctypes.c_int64),
                ("n", ctypes.c_int64), ("k", ctypes.c_int64)]


class Fp8LinearError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__("%s failed: %s (status %d)" % (where, status_string(status), status))


_lib = None


def lib() -> ctypes.CDLL:
    """Load the HIP library (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError("fp8 linear HIP library not built: %s is missing "
                           "(run __graft_entry__.build())" % LIB_PATH)
    L = ctypes.CDLL(LIB_PATH)
    P, i64, I = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
    L.fp8_linear_workspace_bytes.restype = ctypes.c_size_t
    L.fp8_linear_workspace_bytes.argtypes = [i64, i64, I]
    L.fp8_linear_quantize.restype = I
    L.fp8_linear_quantize.argtypes = [P, i64, i64, I, P, P, P, P, P, P, ctypes.c_size_t, P]
    L.fp8_linear_quantize_noalloc.restype = I
    L.fp8_linear_quantize_noalloc.argtypes = [P, i64, i64, I, P, P, P, P, P, P]
    L.fp8_linear_fwd.restype = I
    L.fp8_linear_fwd.argtypes = [P, P, P, P, i64, i64, i64, I, P, P]
    L.fp8_linear_bwd.restype = I
    L.fp8_linear_bwd.argtypes = [P, P, P, P, P, P, P, P, i64, i64, i64, I, P, P, P]
    L.fp8_linear_amax.restype = I
    L.fp8_linear_amax.argtypes = [P, i64, i64, P, P, ctypes.c_size_t, P]
    L.fp8_linear_quantize_scaled.restype = I
    L.fp8_linear_quantize_scaled.argtypes = [P, i64, i64, P, P, P, P]
    L.fp8_linear_bwd_w_f32.restype = I
    L.fp8_linear_bwd_w_f32.argtypes = [P, P, P, P, i64, i64, i64, I, P, P]
    L.fp8_linear_gemm_grouped.restype = I
    L.fp8_linear_gemm_grouped.argtypes = [ctypes.POINTER(GemmProblem), I, I, P]
    L.fp8_linear_bwd_x_acc.restype = I
    L.fp8_linear_bwd_x_acc.argtypes = [P, P, P, P, i64, i64, i64, I, P, P]
    L.fp8_swiglu_workspace_bytes.restype = ctypes.c_size_t
    L.fp8_swiglu_workspace_bytes.argtypes = [i64, i64, I]
    L.fp8_swiglu_fwd.restype = I
    L.fp8_swiglu_fwd.argtypes = [P, P, i64, i64, I, P, P, P, P, P, P, P, ctypes.c_size_t, P]
    L.fp8_swiglu_bwd.restype = I
    L.fp8_swiglu_bwd.argtypes = ([P, P, P, i64, i64, I, P, P] + [P] * 10
                                 + [P, ctypes.c_size_t, P])
    L.fp8_linear_encode_e4m3.restype = I
    L.fp8_linear_encode_e4m3.argtypes = [P, P, i64, P]
    L.fp8_linear_encode_e5m2.restype = I
    L.fp8_linear_encode_e5m2.argtypes = [P, P, i64, P]
    L.fp8_linear_status_string.restype = ctypes.c_char_p
    L.fp8_linear_status_string.argtypes = [I]
    L.fp8_linear_version.restype = ctypes.c_char_p
    L.fp8_linear_version.argtypes = []
    _lib = L
    return L


def status_string(status: int) -> str:
    return lib().fp8_linear_status_string(int(status)).decode()


def _check(status: int, where: str) -> None:
    if status != FP8L_OK:
        raise Fp8LinearError(status, where)


def _p(t: Optional[torch.Tensor]):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else None


def _stream(stream=None):
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def _scaling(rowwise: bool, e5m2: bool = False) -> int:
    return (FP8L_ROWWISE if rowwise else FP8L_TENSORWISE) | (FP8L_E5M2 if e5m2 else 0)


# ----------------------------------------------------------- entry points --

def fp8_linear_workspace_bytes(rows: int, cols: int, rowwise: bool = False) -> int:
    return int(lib().fp8_linear_workspace_bytes(rows, cols, _scaling(rowwise)))


class Quantized:
    """Outputs of fp8_linear_quantize for one bf16 matrix x [rows, cols]."""

    __slots__ = ("q", "qt", "scale", "scale_t", "amax")

    def __init__(self, q, qt, scale, scale_t, amax):
        self.q, self.qt, self.scale, self.scale_t, self.amax = q, qt, scale, scale_t, amax


def alloc_quantized(rows: int, cols: int, rowwise: bool, device) -> Quantized:
    ns, nst, na = (rows, cols, rows + cols) if rowwise else (1, 1, 1)
    return Quantized(torch.empty((rows, cols), dtype=torch.uint8, device=device),
                     torch.empty((cols, rows), dtype=torch.uint8, device=device),
                     torch.empty(ns, dtype=torch.float32, device=device),
                     torch.empty(nst, dtype=torch.float32, device=device),
                     torch.empty(na, dtype=torch.float32, device=device))


def alloc_workspace(rows: int, cols: int, rowwise: bool, device) -> torch.Tensor:
    """Zero-filled, as fp8_linear_quantize requires of a new workspace."""
    return torch.zeros(max(fp8_linear_workspace_bytes(rows, cols, rowwise), 256),
                       dtype=torch.uint8, device=device)


def fp8_linear_quantize(x: torch.Tensor, rowwise: bool = False,
                        out: Optional[Quantized] = None,
                        workspace: Optional[torch.Tensor] = None,
                        stream=None, e5m2: bool = False) -> Quantized:
    """Quantize bf16 x [rows, cols] -> (q, qt, scale, scale_t, amax); E5M2
    codes (scale onto 57344) when e5m2."""
    assert x.dtype == torch.bfloat16 and x.dim() == 2 and x.is_contiguous()
    rows, cols = x.shape
    if out is None:
        out = alloc_quantized(rows, cols, rowwise, x.device)
    if workspace is None:
        workspace = alloc_workspace(rows, cols, rowwise, x.device)
    _check(lib().fp8_linear_quantize(
        _p(x), rows, cols, _scaling(rowwise, e5m2), _p(out.q), _p(out.qt), _p(out.scale),
        _p(out.scale_t), _p(out.amax), _p(workspace), workspace.numel(), _stream(stream)),
        "fp8_linear_quantize")
    return out


FP8L_NOALLOC_MAX_WORKSPACE = 16 << 20


def fp8_linear_quantize_noalloc(x: torch.Tensor, rowwise: bool = False,
                                out: Optional[Quantized] = None, stream=None,
                                e5m2: bool = False) -> Quantized:
    """fp8_linear_quantize with the library's per-GPU scratch array in place
    of a workspace (the entry point allocates nothing; pass ``out`` to keep
    this call free of allocations too)."""
    assert x.dtype == torch.bfloat16 and x.dim() == 2 and x.is_contiguous()
    rows, cols = x.shape
    if out is None:
        out = alloc_quantized(rows, cols, rowwise, x.device)
    _check(lib().fp8_linear_quantize_noalloc(
        _p(x), rows, cols, _scaling(rowwise, e5m2), _p(out.q), _p(out.qt), _p(out.scale),
        _p(out.scale_t), _p(out.amax), _stream(stream)), "fp8_linear_quantize_noalloc")
    return out


def fp8_linear_fwd(xq: torch.Tensor, sx: torch.Tensor, wq: torch.Tensor,
                   sw: torch.Tensor, rowwise: bool = False,
                   out: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """out [M, N] bf16 = (xq [M, K] . wq [N, K]^T) / (sx * sw)."""
    M, K = xq.shape
    N = wq.shape[0]
    if out is None:
        out = torch.empty((M, N), dtype=torch.bfloat16, device=xq.device)
    _check(lib().fp8_linear_fwd(_p(xq), _p(sx), _p(wq), _p(sw), M, N, K,
                                _scaling(rowwise), _p(out), _stream(stream)),
           "fp8_linear_fwd")
    return out


def fp8_linear_bwd(dyq, sdy, dytq, sdyt, wtq, swt, xtq, sxt, M: int, N: int, K: int,
                   rowwise: bool = False, grad_x: Optional[torch.Tensor] = None,
                   grad_w: Optional[torch.Tensor] = None, want_x: bool = True,
                   want_w: bool = True, stream=None,
                   e5m2: bool = False) -> Tuple[torch.Tensor, torch.Tensor]:
    """grad_x [M, K] = dY . W and grad_w [N, K] = dY^T . X from the fp8 copies
    (dY's copies in E5M2 when e5m2)."""
    dev = (dyq if dyq is not None else dytq).device
    if want_x and grad_x is None:
        grad_x = torch.empty((M, K), dtype=torch.bfloat16, device=dev)
    if want_w and grad_w is None:
        grad_w = torch.empty((N, K), dtype=torch.bfloat16, device=dev)
    _check(lib().fp8_linear_bwd(_p(dyq), _p(sdy), _p(dytq), _p(sdyt), _p(wtq), _p(swt),
                                _p(xtq), _p(sxt), M, N, K, _scaling(rowwise, e5m2),
                                _p(grad_x if want_x else None),
                                _p(grad_w if want_w else None), _stream(stream)),
           "fp8_linear_bwd")
    return grad_x, grad_w


def fp8_linear_amax(x: torch.Tensor, out: Optional[torch.Tensor] = None,
                    workspace: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """[1] fp32 max |x| of a bf16 matrix (one shard's share of a global amax)."""
    assert x.dtype == torch.bfloat16 and x.dim() == 2 and x.is_contiguous()
    rows, cols = x.shape
    if out is None:
        out = torch.empty(1, dtype=torch.float32, device=x.device)
    if workspace is None:
        workspace = alloc_workspace(rows, cols, False, x.device)
    _check(lib().fp8_linear_amax(_p(x), rows, cols, _p(out), _p(workspace), workspace.numel(),
                                 _stream(stream)), "fp8_linear_amax")
    return out


def fp8_linear_quantize_scaled(x: torch.Tensor, scale: torch.Tensor,
                               q: Optional[torch.Tensor] = None,
                               qt: Optional[torch.Tensor] = None,
                               stream=None) -> Tuple[torch.Tensor, torch.Tensor]:
    """(q [rows, cols], qt [cols, rows]) E4M3 codes of x * scale[0]."""
    assert x.dtype == torch.bfloat16 and x.dim() == 2 and x.is_contiguous()
    assert scale.dtype == torch.float32 and scale.numel() >= 1
    rows, cols = x.shape
    if q is None:
        q = torch.empty((rows, cols), dtype=torch.uint8, device=x.device)
    if qt is None:
        qt = torch.empty((cols, rows), dtype=torch.uint8, device=x.device)
    _check(lib().fp8_linear_quantize_scaled(_p(x), rows, cols, _p(scale), _p(q), _p(qt),
                                            _stream(stream)), "fp8_linear_quantize_scaled")
    return q, qt


def fp8_linear_bwd_w_f32(dytq, sdyt, xtq, sxt, M: int, N: int, K: int,
                         rowwise: bool = False, grad_w: Optional[torch.Tensor] = None,
                         stream=None, e5m2: bool = False) -> torch.Tensor:
    """grad_w [N, K] fp32 = dY^T . X from the fp8 copies (no bf16 rounding)."""
    if grad_w is None:
        grad_w = torch.empty((N, K), dtype=torch.float32, device=dytq.device)
    _check(lib().fp8_linear_bwd_w_f32(_p(dytq), _p(sdyt), _p(xtq), _p(sxt), M, N, K,
                                      _scaling(rowwise, e5m2), _p(grad_w), _stream(stream)),
           "fp8_linear_bwd_w_f32")
    return grad_w


def fp8_linear_gemm_grouped(problems, rowwise: bool = False, stream=None,
                            e5m2: bool = False) -> None:
    """One launch of up to FP8L_MAX_GROUP GEMMs c = (a . b^T) / (sa * sb):
    problems is a sequence of (a [m, k], sa, b [n, k], sb, c [m, n] bf16)."""
    arr = (GemmProblem * len(problems))()
    for i, (a, sa, b, sb, c) in enumerate(problems):
        m, k = a.shape
        n = b.shape[0]
        assert c.shape == (m, n) and c.dtype == torch.bfloat16
        arr[i] = GemmProblem(a.data_ptr(), sa.data_ptr(), b.data_ptr(), sb.data_ptr(),
                             c.data_ptr(), m, n, k)
    _check(lib().fp8_linear_gemm_grouped(arr, len(problems), _scaling(rowwise, e5m2),
                                         _stream(stream)), "fp8_linear_gemm_grouped")


def fp8_linear_bwd_x_acc(dyq, sdy, wtq, swt, M: int, N: int, K: int, grad_x: torch.Tensor,
                         rowwise: bool = False, stream=None, e5m2: bool = False) -> torch.Tensor:
    """grad_x [M, K] (bf16, in place) = bf16(grad_x + bf16(dY . W)): the second
    gradient contribution of an x that feeds two linears."""
    _check(lib().fp8_linear_bwd_x_acc(_p(dyq), _p(sdy), _p(wtq), _p(swt), M, N, K,
                                      _scaling(rowwise, e5m2), _p(grad_x), _stream(stream)),
           "fp8_linear_bwd_x_acc")
    return grad_x


def fp8_swiglu_workspace_bytes(rows: int, hidden: int, rowwise: bool = False,
                               e5m2: bool = False) -> int:
    return int(lib().fp8_swiglu_workspace_bytes(rows, hidden, _scaling(rowwise, e5m2)))


def alloc_swiglu_workspace(rows: int, hidden: int, rowwise: bool, device) -> torch.Tensor:
    return torch.zeros(max(fp8_swiglu_workspace_bytes(rows, hidden, rowwise), 256),
                       dtype=torch.uint8, device=device)


def fp8_swiglu_fwd(a: torch.Tensor, b: torch.Tensor, rowwise: bool = False,
                   h: Optional[torch.Tensor] = None, out: Optional[Quantized] = None,
                   workspace: Optional[torch.Tensor] = None,
                   stream=None) -> Tuple[torch.Tensor, Quantized]:
    """h = silu(a) * b (bf16 [rows, hidden]) and the E4M3 quantize of h."""
    assert a.dtype == b.dtype == torch.bfloat16 and a.shape == b.shape and a.dim() == 2
    assert a.is_contiguous() and b.is_contiguous()
    rows, hidden = a.shape
    if h is None:
        h = torch.empty_like(a)
    if out is None:
        out = alloc_quantized(rows, hidden, rowwise, a.device)
    if workspace is None:
        workspace = alloc_swiglu_workspace(rows, hidden, rowwise, a.device)
    _check(lib().fp8_swiglu_fwd(_p(a), _p(b), rows, hidden, _scaling(rowwise), _p(h),
                                _p(out.q), _p(out.qt), _p(out.scale), _p(out.scale_t),
                                _p(out.amax), _p(workspace), workspace.numel(),
                                _stream(stream)), "fp8_swiglu_fwd")
    return h, out


def fp8_swiglu_bwd(dh: torch.Tensor, a: torch.Tensor, b: torch.Tensor, rowwise: bool = False,
                   da: Optional[torch.Tensor] = None, db: Optional[torch.Tensor] = None,
                   qa: Optional[Quantized] = None, qb: Optional[Quantized] = None,
                   workspace: Optional[torch.Tensor] = None, stream=None,
                   e5m2: bool = False):
    """(da, db, quantize of da, quantize of db) for h = silu(a) * b and the
    gradient dh; codes E5M2 when e5m2."""
    assert dh.shape == a.shape == b.shape and a.dim() == 2
    assert dh.dtype == a.dtype == b.dtype == torch.bfloat16
    assert dh.is_contiguous() and a.is_contiguous() and b.is_contiguous()
    rows, hidden = a.shape
    dev = a.device
    da = torch.empty_like(a) if da is None else da
    db = torch.empty_like(a) if db is None else db
    qa = alloc_quantized(rows, hidden, rowwise, dev) if qa is None else qa
    qb = alloc_quantized(rows, hidden, rowwise, dev) if qb is None else qb
    if workspace is None:
        workspace = alloc_swiglu_workspace(rows, hidden, rowwise, dev)
    _check(lib().fp8_swiglu_bwd(_p(dh), _p(a), _p(b), rows, hidden, _scaling(rowwise, e5m2),
                                _p(da), _p(db), _p(qa.q), _p(qa.qt), _p(qa.scale),
                                _p(qa.scale_t), _p(qa.amax), _p(qb.q), _p(qb.qt), _p(qb.scale),
                                _p(qb.scale_t), _p(qb.amax), _p(workspace), workspace.numel(),
                                _stream(stream)), "fp8_swiglu_bwd")
    return da, db, qa, qb


def fp8_linear_encode_e4m3(x: torch.Tensor, out: Optional[torch.Tensor] = None,
                           stream=None) -> torch.Tensor:
    """Device E4M3 saturating RNE codes of fp32 values."""
    assert x.dtype == torch.float32 and x.is_contiguous()
    if out is None:
        out = torch.empty(x.shape, dtype=torch.uint8, device=x.device)
    _check(lib().fp8_linear_encode_e4m3(_p(x), _p(out), x.numel(), _stream(stream)),
           "fp8_linear_encode_e4m3")
    return out


def fp8_linear_encode_e5m2(x: torch.Tensor, out: Optional[torch.Tensor] = None,
                           stream=None) -> torch.Tensor:
    """Device E5M2 saturating RNE codes of fp32 values."""
    assert x.dtype == torch.float32 and x.is_contiguous()
    if out is None:
        out = torch.empty(x.shape, dtype=torch.uint8, device=x.device)
    _check(lib().fp8_linear_encode_e5m2(_p(x), _p(out), x.numel(), _stream(stream)),
           "fp8_linear_encode_e5m2")
    return out


def fp8_linear_version() -> str:
    return lib().fp8_linear_version().decode()


# ------------------------------------------------------------ one linear --

class LinearStep:
    """One Float8 linear fwd+bwd on preallocated device buffers.

    Holds the bf16 inputs X [M, K], W [N, K], dY [M, N] and every output; a
    call to ``run()`` enqueues quantize(X), quantize(W), quantize(dY), the
    forward GEMM and both backward GEMMs on the current stream.  With
    ``e5m2_grad`` dY is quantized to E5M2 and the backward GEMMs read it so.
    """

    def __init__(self, x: torch.Tensor, w: torch.Tensor, dy: torch.Tensor,
                 rowwise: bool = False, e5m2_grad: bool = False,
                 qx: Optional[Quantized] = None):
        self.x, self.w, self.dy, self.rowwise = x, w, dy, rowwise
        self.e5m2_grad = e5m2_grad
        self.M, self.K = x.shape
        self.N = w.shape[0]
        dev = x.device
        # qx given: X's quantize belongs to another linear reading the same
        # X (w1 and w3 of the SwiGLU feed-forward), which runs it first
        self.owns_qx = qx is None
        self.qx = alloc_quantized(self.M, self.K, rowwise, dev) if qx is None else qx
        self.qw = alloc_quantized(self.N, self.K, rowwise, dev)
        self.qdy = alloc_quantized(self.M, self.N, rowwise, dev)
        ws = max(fp8_linear_workspace_bytes(self.M, self.K, rowwise),
                 fp8_linear_workspace_bytes(self.N, self.K, rowwise),
                 fp8_linear_workspace_bytes(self.M, self.N, rowwise), 256)
        self.ws = torch.zeros(ws, dtype=torch.uint8, device=dev)
        self.out = torch.empty((self.M, self.N), dtype=torch.bfloat16, device=dev)
        self.grad_x = torch.empty((self.M, self.K), dtype=torch.bfloat16, device=dev)
        self.grad_w = torch.empty((self.N, self.K), dtype=torch.bfloat16, device=dev)

    @property
    def quantize_bytes(self) -> int:
        """Algorithmic bytes of quantize(): 6 per element of each tensor."""
        return 6 * ((self.M * self.K if self.owns_qx else 0) + self.N * self.K + self.M * self.N)

    def quantize(self, stream=None):
        if self.owns_qx:
            fp8_linear_quantize(self.x, self.rowwise, self.qx, self.ws, stream)
        fp8_linear_quantize(self.w, self.rowwise, self.qw, self.ws, stream)
        fp8_linear_quantize(self.dy, self.rowwise, self.qdy, self.ws, stream,
                            e5m2=self.e5m2_grad)

    def gemms(self, stream=None):
        fp8_linear_fwd(self.qx.q, self.qx.scale, self.qw.q, self.qw.scale, self.rowwise,
                       self.out, stream)
        fp8_linear_bwd(self.qdy.q, self.qdy.scale, self.qdy.qt, self.qdy.scale_t,
                       self.qw.qt, self.qw.scale_t, self.qx.qt, self.qx.scale_t,
                       self.M, self.N, self.K, self.rowwise, self.grad_x, self.grad_w,
                       stream=stream, e5m2=self.e5m2_grad)

    def gemms_fwd_x(self, stream=None):
        """The forward GEMM and grad_X (grad_W left to a grouped launch)."""
        fp8_linear_fwd(self.qx.q, self.qx.scale, self.qw.q, self.qw.scale, self.rowwise,
                       self.out, stream)
        fp8_linear_bwd(self.qdy.q, self.qdy.scale, None, None, self.qw.qt, self.qw.scale_t,
                       None, None, self.M, self.N, self.K, self.rowwise, grad_x=self.grad_x,
                       want_w=False, stream=stream, e5m2=self.e5m2_grad)

    def grad_w_problem(self):
        """grad_W [N, K] = dY^T . X as a fp8_linear_gemm_grouped problem."""
        return (self.qdy.qt, self.qdy.scale_t, self.qx.qt, self.qx.scale_t, self.grad_w)

    def run(self, stream=None):
        self.quantize(stream)
        self.gemms(stream)


class GroupedStep:
    """The linears of one step on one stream, their GEMMs in few launches.

    Per linear: its quantizes, then one fp8_linear_gemm_grouped launch of
    its GEMMs (forward, grad_X, grad_W) ordered by contraction length,
    longest first, so that the short tiles fill in behind the long ones and
    every compute unit finishes at about the same time.  A grad_W whose
    shape equals the next linear's is deferred into the next launch (w1's
    and w3's, 896 tiles each, fill 7 rounds of 256 compute units together).
    For the Llama FFN that is 3 launches for 9 GEMMs.  A launch reads
    every problem's A operand in one code format, so with E5M2 gradients
    the forward GEMM (E4M3 X) gets a launch of its own, apart from the
    GEMMs that read dY (``launches()``).  Results equal each LinearStep's
    run() in turn.

    ``plan`` lists, per linear, the GEMMs of its launch as (kind, linear)
    with kind "fwd", "grad_x" or "grad_w".  ``run(record=True)`` brackets
    each linear's quantizes and its GEMM launch with timing events and
    returns (kind, launches, work, start, end) per group (kind "quantize"
    with work in bytes, or "gemm" with work in flops).
    """

    def __init__(self, steps):
        self.steps = list(steps)
        shape = lambda ls: (ls.N, ls.K, ls.M, ls.rowwise, ls.e5m2_grad)
        contraction = {"fwd": lambda ls: ls.K, "grad_x": lambda ls: ls.N,
                       "grad_w": lambda ls: ls.M}
        self.plan = []
        deferred = []
        for i, ls in enumerate(self.steps):
            probs = [("fwd", i), ("grad_x", i)]
            nxt = self.steps[i + 1] if i + 1 < len(self.steps) else None
            if nxt is not None and not deferred and shape(nxt) == shape(ls):
                deferred.append(("grad_w", i))
            else:
                probs += deferred + [("grad_w", i)]
                deferred = []
            probs.sort(key=lambda p: -contraction[p[0]](self.steps[p[1]]))
            self.plan.append(probs)

    def _problem(self, kind, i):
        ls = self.steps[i]
        if kind == "fwd":
            return (ls.qx.q, ls.qx.scale, ls.qw.q, ls.qw.scale, ls.out)
        if kind == "grad_x":
            return (ls.qdy.q, ls.qdy.scale, ls.qw.qt, ls.qw.scale_t, ls.grad_x)
        return ls.grad_w_problem()

    def run(self, stream=None, record: bool = False):
        st = stream if stream is not None else torch.cuda.current_stream()
        groups = []

        def timed(kind, n, work, fn):
            if record:
                e0 = torch.cuda.Event(enable_timing=True)
                e1 = torch.cuda.Event(enable_timing=True)
                e0.record(st)
                fn()
                e1.record(st)
                groups.append((kind, n, work, e0, e1))
            else:
                fn()

        for ls, probs in zip(self.steps, self.plan):
            timed("quantize", 3 if ls.owns_qx else 2, ls.quantize_bytes,
                  lambda: ls.quantize(st))
            for e5, chunk in self.launches(probs):
                flops = sum(2 * self.steps[i].M * self.steps[i].N * self.steps[i].K
                            for _, i in chunk)
                timed("gemm", 1, flops,
                      lambda: fp8_linear_gemm_grouped([self._problem(k, i) for k, i in chunk],
                                                      ls.rowwise, st, e5m2=e5))
        return groups

    def a_is_e5m2(self, kind, i) -> bool:
        """Whether problem (kind, i) reads its A operand as E5M2: the
        backward GEMMs read dY's copies, which are E5M2 under e5m2_grad;
        the forward GEMM reads X's, always E4M3."""
        return kind != "fwd" and self.steps[i].e5m2_grad

    def launches(self, probs):
        """The fp8_linear_gemm_grouped launches of one linear's problems:
        (e5m2, chunk) pairs.  The code format of A is one per launch, so
        problems are split by it (in the order of first appearance, each
        part keeping the longest-contraction-first order), and each part
        into chunks of at most FP8L_MAX_GROUP."""
        parts = {}
        for p in probs:
            parts.setdefault(self.a_is_e5m2(*p), []).append(p)
        return [(e5, part[c:c + FP8L_MAX_GROUP]) for e5, part in parts.items()
                for c in range(0, len(part), FP8L_MAX_GROUP)]


class PipelinedStep:
    """The linears of one step with their quantizes on a side stream.

    The GEMMs are compute-bound and the quantizes bandwidth-bound, and the
    quantizes of linear i+1 do not depend on the GEMMs of linear i: they are
    issued on ``side`` (a second stream at the default priority) ahead of
    the GEMMs on ``main``.  Ordering: ``run()`` first makes the side stream
    wait for all work already issued on ``main`` (so inputs written there,
    and the previous step's GEMMs that read the fp8 copies, come first);
    linear i's GEMMs wait for its quantizes.  The results are those of
    running each LinearStep in turn on ``main``.

    ``run(record=True)`` also brackets each linear's quantize group and
    GEMM group with timing events and returns (kind, launches, work, start,
    end) per group: kind "quantize" (3 quantizes, work = bytes) or "gemm"
    (fwd, grad_x, grad_w; work = flops).
    """

    def __init__(self, steps, main=None, side=None):
        self.steps = list(steps)
        self.main = main if main is not None else torch.cuda.current_stream()
        self.side = side if side is not None else torch.cuda.Stream(device=self.main.device)
        self.start = torch.cuda.Event()
        self.q_done = [torch.cuda.Event() for _ in self.steps]

    def run(self, record: bool = False):
        groups = []

        def timed(kind, n, work, stream, fn):
            if record:
                e0 = torch.cuda.Event(enable_timing=True)
                e1 = torch.cuda.Event(enable_timing=True)
                e0.record(stream)
                fn()
                e1.record(stream)
                groups.append((kind, n, work, e0, e1))
            else:
                fn()

        self.start.record(self.main)
        self.side.wait_event(self.start)
        for i, ls in enumerate(self.steps):
            timed("quantize", 3 if ls.owns_qx else 2, ls.quantize_bytes, self.side,
                  lambda: ls.quantize(self.side))
            self.q_done[i].record(self.side)
        for i, ls in enumerate(self.steps):
            self.main.wait_event(self.q_done[i])
            timed("gemm", 3, 6 * ls.M * ls.N * ls.K, self.main, lambda: ls.gemms(self.main))
        return groups


# ------------------------------------------------------ SwiGLU FFN block --

class SwiGLUFFNStep:
    """One Float8 SwiGLU feed-forward block fwd+bwd on preallocated buffers.

    x [M, D], w1 and w3 [H, D], w2 [D, H], d_out [M, D] (bf16).  ``run()``
    enqueues, on the current stream (the quantizes of the weights and of
    d_out on ``side`` when a second stream is given):

      quantize x once (read by w1 and w3), quantize w1, w3, w2
      a = x.w1^T, b = x.w3^T                       (one grouped launch)
      h = silu(a) * b and its quantize             (fp8_swiglu_fwd)
      out = h.w2^T
      quantize d_out
      dh = d_out.w2, grad_w2 = d_out^T.h           (one grouped launch)
      da, db and their quantizes                   (fp8_swiglu_bwd)
      grad_x = da.w1, grad_w1 = da^T.x, grad_w3 = db^T.x   (one grouped launch)
      grad_x += db.w3                              (fp8_linear_bwd_x_acc)

    With ``e5m2_grad`` the gradient operands (d_out, da, db) are E5M2.
    """

    def __init__(self, x, w1, w3, w2, d_out, rowwise: bool = False, e5m2_grad: bool = False):
        self.x, self.w1, self.w3, self.w2, self.d_out = x, w1, w3, w2, d_out
        self.rowwise, self.e5m2_grad = rowwise, e5m2_grad
        self.M, self.D = x.shape
        self.H = w1.shape[0]
        assert w1.shape == w3.shape == (self.H, self.D) and w2.shape == (self.D, self.H)
        assert d_out.shape == (self.M, self.D)
        M, D, H, dev = self.M, self.D, self.H, x.device
        bf = dict(dtype=torch.bfloat16, device=dev)
        self.qx = alloc_quantized(M, D, rowwise, dev)
        self.qw1 = alloc_quantized(H, D, rowwise, dev)
        self.qw3 = alloc_quantized(H, D, rowwise, dev)
        self.qw2 = alloc_quantized(D, H, rowwise, dev)
        self.qh = alloc_quantized(M, H, rowwise, dev)
        self.qdy = alloc_quantized(M, D, rowwise, dev)
        self.qda = alloc_quantized(M, H, rowwise, dev)
        self.qdb = alloc_quantized(M, H, rowwise, dev)
        ws = max(fp8_linear_workspace_bytes(r, c, rowwise) for r, c in
                 ((M, D), (H, D), (D, H)))
        self.ws = torch.zeros(max(ws, 256), dtype=torch.uint8, device=dev)
        self.ws_side = torch.zeros_like(self.ws)     # quantizes on a second stream
        self.ws_sw = alloc_swiglu_workspace(M, H, rowwise, dev)
        self._start = torch.cuda.Event()
        self._side_events = {n: torch.cuda.Event() for n in ("qw1", "qw3", "qw2", "qdy")}
        self.a = torch.empty((M, H), **bf)
        self.b = torch.empty((M, H), **bf)
        self.h = torch.empty((M, H), **bf)
        self.out = torch.empty((M, D), **bf)
        self.dh = torch.empty((M, H), **bf)
        self.da = torch.empty((M, H), **bf)
        self.db = torch.empty((M, H), **bf)
        self.grad_x = torch.empty((M, D), **bf)
        self.grad_w1 = torch.empty((H, D), **bf)
        self.grad_w3 = torch.empty((H, D), **bf)
        self.grad_w2 = torch.empty((D, H), **bf)

    @property
    def flops(self) -> int:
        """Nine GEMMs of 2*M*D*H each."""
        return 18 * self.M * self.D * self.H

    def ops(self):
        """The launches of one step, in order: (name, kind, work, side,
        needs, fn) with kind one of "quantize", "swiglu", "gemm"; work the
        algorithmic bytes (quantize / swiglu) or flops (gemm) of the launch;
        side True for the launches that depend on no other launch of the
        step (the quantizes of the weights and of d_out); needs the names
        of the side launches this one reads; fn(stream) the call."""
        M, D, H, rw, e5 = self.M, self.D, self.H, self.rowwise, self.e5m2_grad
        g = 2 * M * D * H
        return (
            ("qw1", "quantize", 6 * H * D, True, (),
             lambda st: fp8_linear_quantize(self.w1, rw, self.qw1, self.ws_side, st)),
            ("qw3", "quantize", 6 * H * D, True, (),
             lambda st: fp8_linear_quantize(self.w3, rw, self.qw3, self.ws_side, st)),
            ("qw2", "quantize", 6 * D * H, True, (),
             lambda st: fp8_linear_quantize(self.w2, rw, self.qw2, self.ws_side, st)),
            ("qdy", "quantize", 6 * M * D, True, (),
             lambda st: fp8_linear_quantize(self.d_out, rw, self.qdy, self.ws_side, st,
                                            e5m2=e5)),
            ("qx", "quantize", 6 * M * D, False, (),
             lambda st: fp8_linear_quantize(self.x, rw, self.qx, self.ws, st)),
            # a and b in one launch
            ("ab", "gemm", 2 * g, False, ("qw1", "qw3"), lambda st: fp8_linear_gemm_grouped(
                [(self.qx.q, self.qx.scale, self.qw1.q, self.qw1.scale, self.a),
                 (self.qx.q, self.qx.scale, self.qw3.q, self.qw3.scale, self.b)], rw, st)),
            # a, b read twice (elementwise pass, then h read by the cast),
            # h written once; q and qt written
            ("swiglu_fwd", "swiglu", 10 * M * H, False, (),
             lambda st: fp8_swiglu_fwd(self.a, self.b, rw, self.h, self.qh, self.ws_sw, st)),
            ("out", "gemm", g, False, ("qw2",),
             lambda st: fp8_linear_fwd(self.qh.q, self.qh.scale, self.qw2.q, self.qw2.scale, rw,
                                       self.out, st)),
            # grad_W2 (896 tiles, contraction M) and dh (1792 tiles,
            # contraction D) in one launch, the longer tiles first
            ("grad_w2_dh", "gemm", 2 * g, False, ("qw2", "qdy"),
             lambda st: fp8_linear_gemm_grouped(
                 [(self.qdy.qt, self.qdy.scale_t, self.qh.qt, self.qh.scale_t, self.grad_w2),
                  (self.qdy.q, self.qdy.scale, self.qw2.qt, self.qw2.scale_t, self.dh)],
                 rw, st, e5m2=e5)),
            # dh, a, b read; da, db written; each read again by its cast,
            # whose q and qt are written
            ("swiglu_bwd", "swiglu", 18 * M * H, False, (),
             lambda st: fp8_swiglu_bwd(self.dh, self.a, self.b, rw, self.da, self.db, self.qda,
                                       self.qdb, self.ws_sw, st, e5m2=e5)),
            # grad_x = da.w1 (512 tiles, contraction H) with the grad_W of w1
            # and w3 (2 x 896 tiles, contraction M) in one launch; then
            # grad_x += db.w3
            ("grad_x_w13", "gemm", 3 * g, False, ("qw1",), lambda st: fp8_linear_gemm_grouped(
                [(self.qda.q, self.qda.scale, self.qw1.qt, self.qw1.scale_t, self.grad_x),
                 (self.qda.qt, self.qda.scale_t, self.qx.qt, self.qx.scale_t, self.grad_w1),
                 (self.qdb.qt, self.qdb.scale_t, self.qx.qt, self.qx.scale_t, self.grad_w3)],
                rw, st, e5m2=e5)),
            ("grad_x_acc", "gemm", g, False, ("qw3",), lambda st: fp8_linear_bwd_x_acc(
                self.qdb.q, self.qdb.scale, self.qw3.qt, self.qw3.scale_t, M, H, D,
                self.grad_x, rw, st, e5m2=e5)),
        )

    def run(self, side=None, record: bool = False):
        """Enqueue one step on the current stream.  With ``side`` (a second
        stream) the launches marked side run there, after all work already
        issued on the current stream, and each launch on the current stream
        first waits for the side launches it reads; the results are those of
        the single-stream order.  record: timing events around every launch,
        returned as (kind, work, start, end)."""
        main = torch.cuda.current_stream()
        if side is not None:
            self._start.record(main)
            side.wait_event(self._start)
        rec = []
        done = {}
        for name, kind, work, on_side, needs, fn in self.ops():
            st = side if (on_side and side is not None) else main
            for n in needs:
                if n in done:
                    main.wait_event(done.pop(n))
            if record:
                e0 = torch.cuda.Event(enable_timing=True)
                e1 = torch.cuda.Event(enable_timing=True)
                e0.record(st)
                fn(st)
                e1.record(st)
                rec.append((kind, work, e0, e1))
            else:
                fn(st)
            if st is not main:
                ev = self._side_events[name]
                ev.record(st)
                done[name] = ev
        for ev in done.values():      # the step ends with the side stream joined
            main.wait_event(ev)
        return rec
