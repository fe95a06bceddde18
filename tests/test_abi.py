"""The C ABI library: it loads, exports every symbol include/fp8_linear.h
declares, and rejects bad arguments on the host with the documented status
codes before anything is enqueued.  No compute calls: every case here fails
validation, so no kernel is launched."""
import ctypes
import os
import re
import subprocess

import pytest

from float8_mixed_precision_amd import ops

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fp8_linear.h")


def declared_symbols():
    src = open(HEADER).read()
    return sorted(set(re.findall(r"FP8L_API\s+[\w\s\*]*?\b(fp8_\w+)\s*\(", src)))


def test_header_declares_the_boundary():
    assert declared_symbols() == sorted(ops.EXPORTS)


def test_library_exports_every_declared_symbol():
    out = subprocess.run(["nm", "-D", "--defined-only", ops.LIB_PATH],
                         capture_output=True, text=True, check=True).stdout
    exported = set(re.findall(r"\bT\s+(fp8_\w+)", out))
    assert set(declared_symbols()) <= exported
    L = ops.lib()
    for s in declared_symbols():
        assert getattr(L, s) is not None


def test_status_strings_and_version():
    assert ops.status_string(0) == "ok"
    for s in range(1, 6):
        assert ops.status_string(s) and ops.status_string(s) != "unknown status"
    assert ops.status_string(99) == "unknown status"
    assert "gfx950" in ops.fp8_linear_version()


def test_workspace_bytes():
    assert ops.fp8_linear_workspace_bytes(0, 0) == 0
    assert ops.fp8_linear_workspace_bytes(17, 16) == 0            # invalid shape
    assert ops.lib().fp8_linear_workspace_bytes(16, 16, 5) == 0    # invalid mode
    tw = ops.fp8_linear_workspace_bytes(8192, 14336, False)
    rw = ops.fp8_linear_workspace_bytes(8192, 14336, True)
    assert 0 < tw < rw and tw % 256 == 0 and rw % 256 == 0


# Fake device addresses: validation must reject these calls before any
# pointer is used.  These tests only run where no GPU is visible.
A16 = 0x10000          # 16-byte aligned
A_BAD = 0x10004        # misaligned


def _no_gpu():
    import torch
    return torch.cuda.device_count() == 0


pytestmark_cpu = pytest.mark.skipif(not _no_gpu(), reason="fake-pointer cases run without a GPU only")


def q_call(x=A16, rows=16, cols=16, scaling=0, q=A16, qt=A16, s=A16, st=A16,
           amax=None, ws=A16, wsb=1 << 20):
    P = ctypes.c_void_p
    return ops.lib().fp8_linear_quantize(P(x) if x else None, rows, cols, scaling,
                                         P(q) if q else None, P(qt) if qt else None,
                                         P(s) if s else None, P(st) if st else None,
                                         P(amax) if amax else None, P(ws) if ws else None,
                                         wsb, None)


@pytestmark_cpu
def test_quantize_rejects_bad_arguments():
    E = ops
    assert q_call(scaling=4) == E.FP8L_EINVAL               # unknown flag
    assert q_call(scaling=-1) == E.FP8L_EINVAL
    assert q_call(rows=17) == E.FP8L_ESHAPE
    assert q_call(cols=-16) == E.FP8L_ESHAPE
    assert q_call(rows=1 << 31) == E.FP8L_ESHAPE
    assert q_call(x=None) == E.FP8L_EINVAL
    assert q_call(q=None) == E.FP8L_EINVAL
    assert q_call(qt=None) == E.FP8L_EINVAL
    assert q_call(s=None) == E.FP8L_EINVAL
    assert q_call(st=None) == E.FP8L_EINVAL
    assert q_call(ws=None) == E.FP8L_EINVAL
    assert q_call(wsb=0) == E.FP8L_EWORKSPACE
    assert q_call(rows=8192, cols=4096, wsb=100) == E.FP8L_EWORKSPACE
    assert q_call(x=A_BAD) == E.FP8L_EALIGN
    assert q_call(q=A_BAD) == E.FP8L_EALIGN
    assert q_call(qt=A_BAD) == E.FP8L_EALIGN
    assert q_call(ws=A_BAD) == E.FP8L_EALIGN
    assert q_call(s=A16 + 2) == E.FP8L_EALIGN
    assert q_call(amax=A16 + 1) == E.FP8L_EALIGN


@pytestmark_cpu
def test_quantize_noalloc_rejects_bad_arguments():
    """The same argument rules as fp8_linear_quantize, and requests beyond the
    scratch array's size rejected on the host (no HIP call is made)."""
    E = ops
    P = ctypes.c_void_p

    def call(x=A16, rows=16, cols=16, scaling=0, q=A16, qt=A16, s=A16, st=A16, amax=None):
        return ops.lib().fp8_linear_quantize_noalloc(
            P(x) if x else None, rows, cols, scaling, P(q) if q else None,
            P(qt) if qt else None, P(s) if s else None, P(st) if st else None,
            P(amax) if amax else None, None)

    assert call(scaling=4) == E.FP8L_EINVAL
    assert call(rows=17) == E.FP8L_ESHAPE
    assert call(x=None) == E.FP8L_EINVAL
    assert call(st=None) == E.FP8L_EINVAL
    assert call(qt=A_BAD) == E.FP8L_EALIGN
    assert call(amax=A16 + 1) == E.FP8L_EALIGN
    limit = ops.FP8L_NOALLOC_MAX_WORKSPACE
    # rowwise [65536, 32768] needs ~84 MB of partial maxima
    assert ops.fp8_linear_workspace_bytes(65536, 32768, True) > limit
    assert call(rows=65536, cols=32768, scaling=E.FP8L_ROWWISE) == E.FP8L_EWORKSPACE
    # the largest rowwise workloads fit
    assert ops.fp8_linear_workspace_bytes(8192, 28672, True) <= limit
    assert ops.fp8_linear_workspace_bytes(28672, 8192, True) <= limit
    assert ops.fp8_linear_workspace_bytes(1 << 20, 1 << 20, False) <= limit


@pytestmark_cpu
def test_gemm_entry_points_reject_bad_arguments():
    E = ops
    L = ops.lib()
    P = ctypes.c_void_p

    def fwd(xq=A16, sx=A16, wq=A16, sw=A16, M=16, N=16, K=16, scaling=0, out=A16):
        return L.fp8_linear_fwd(P(xq) if xq else None, P(sx) if sx else None,
                                P(wq) if wq else None, P(sw) if sw else None,
                                M, N, K, scaling, P(out) if out else None, None)

    assert fwd(scaling=-1) == E.FP8L_EINVAL
    assert fwd(scaling=E.FP8L_E5M2) == E.FP8L_EINVAL       # the forward takes E4M3 only
    assert fwd(M=8) == E.FP8L_ESHAPE
    assert fwd(K=-16) == E.FP8L_ESHAPE
    assert fwd(xq=None) == E.FP8L_EINVAL
    assert fwd(sw=None) == E.FP8L_EINVAL
    assert fwd(out=None) == E.FP8L_EINVAL
    assert fwd(wq=A_BAD) == E.FP8L_EALIGN
    assert fwd(out=A_BAD) == E.FP8L_EALIGN
    assert fwd(sx=A16 + 1) == E.FP8L_EALIGN
    # operands and outputs are addressed with 32-bit byte offsets: a matrix
    # of 2^31 bytes is rejected, one row less gets past the size check (and
    # stops at the misaligned output, before any launch)
    assert fwd(M=32768, N=32768, K=16) == E.FP8L_ESHAPE          # bf16 out: 2^31 B
    assert fwd(M=32752, N=32768, K=16, out=A_BAD) == E.FP8L_EALIGN
    assert fwd(M=65536, N=16, K=32768) == E.FP8L_ESHAPE          # xq: 2^31 B
    assert fwd(M=65520, N=16, K=32768, out=A_BAD) == E.FP8L_EALIGN
    assert fwd(M=16, N=65536, K=32768) == E.FP8L_ESHAPE          # wq: 2^31 B
    assert fwd(M=1 << 31, N=16, K=16) == E.FP8L_ESHAPE           # dimension cap

    def bwd(gx=A16, gw=A16, dyq=A16, wtq=A_BAD, **kw):
        return L.fp8_linear_bwd(P(dyq) if dyq else None, P(A16), P(A16), P(A16),
                                P(wtq) if wtq else None, P(A16), P(A16), P(A16),
                                kw.get("M", 16), kw.get("N", 16), kw.get("K", 16),
                                kw.get("scaling", 0), P(gx) if gx else None,
                                P(gw) if gw else None, None)

    assert bwd(gx=None, gw=None) == E.FP8L_EINVAL
    assert bwd(N=24) == E.FP8L_ESHAPE
    assert bwd() == E.FP8L_EALIGN                    # grad_x operands checked
    assert bwd(wtq=None) == E.FP8L_EINVAL
    assert bwd(gw=A_BAD, wtq=A16) == E.FP8L_EALIGN   # grad_w output checked
    assert bwd(scaling=4) == E.FP8L_EINVAL
    assert bwd(M=32768, N=16, K=32768) == E.FP8L_ESHAPE     # grad_x bf16 [M, K]: 2^31 B
    assert bwd(M=65536, N=32768, K=16) == E.FP8L_ESHAPE     # dyq [M, N]: 2^31 B


@pytestmark_cpu
def test_encode_rejects_bad_arguments():
    L = ops.lib()
    P = ctypes.c_void_p
    assert L.fp8_linear_encode_e4m3(P(A16), P(A16), -1, None) == ops.FP8L_ESHAPE
    assert L.fp8_linear_encode_e4m3(None, P(A16), 4, None) == ops.FP8L_EINVAL
    assert L.fp8_linear_encode_e4m3(P(A_BAD), P(A16), 4, None) == ops.FP8L_EALIGN
    assert L.fp8_linear_encode_e4m3(None, None, 0, None) == ops.FP8L_OK   # empty


@pytestmark_cpu
def test_amax_scaled_and_f32_entry_points_reject_bad_arguments():
    E = ops
    L = ops.lib()
    P = ctypes.c_void_p

    def amax(x=A16, rows=16, cols=16, out=A16, ws=A16, wsb=1 << 20):
        return L.fp8_linear_amax(P(x) if x else None, rows, cols, P(out) if out else None,
                                 P(ws) if ws else None, wsb, None)

    assert amax(rows=24) == E.FP8L_ESHAPE
    assert amax(out=None) == E.FP8L_EINVAL
    assert amax(x=None) == E.FP8L_EINVAL
    assert amax(ws=None) == E.FP8L_EINVAL
    assert amax(wsb=0) == E.FP8L_EWORKSPACE
    assert amax(x=A_BAD) == E.FP8L_EALIGN
    assert amax(out=A16 + 2) == E.FP8L_EALIGN

    def qs(x=A16, rows=16, cols=16, s=A16, q=A16, qt=A16):
        return L.fp8_linear_quantize_scaled(P(x) if x else None, rows, cols,
                                            P(s) if s else None, P(q) if q else None,
                                            P(qt) if qt else None, None)

    assert qs(cols=8) == E.FP8L_ESHAPE
    assert qs(rows=0, x=None, s=None, q=None, qt=None) == E.FP8L_OK   # empty: nothing to do
    assert qs(s=None) == E.FP8L_EINVAL
    assert qs(q=None) == E.FP8L_EINVAL
    assert qs(qt=A_BAD) == E.FP8L_EALIGN
    assert qs(s=A16 + 1) == E.FP8L_EALIGN

    def bw(dyt=A16, sdyt=A16, xt=A16, sxt=A16, M=16, N=16, K=16, scaling=0, gw=A16):
        return L.fp8_linear_bwd_w_f32(P(dyt) if dyt else None, P(sdyt) if sdyt else None,
                                      P(xt) if xt else None, P(sxt) if sxt else None,
                                      M, N, K, scaling, P(gw) if gw else None, None)

    assert bw(scaling=8) == E.FP8L_EINVAL
    assert bw(N=40) == E.FP8L_ESHAPE
    assert bw(N=32768, K=32768) == E.FP8L_ESHAPE        # 4 GiB of fp32 output
    assert bw(gw=None) == E.FP8L_EINVAL
    assert bw(sxt=None) == E.FP8L_EINVAL
    assert bw(gw=A_BAD) == E.FP8L_EALIGN


@pytestmark_cpu
def test_swiglu_and_accumulate_entry_points_reject_bad_arguments():
    E = ops
    L = ops.lib()
    P = ctypes.c_void_p
    assert L.fp8_swiglu_workspace_bytes(24, 16, 0) == 0
    assert L.fp8_swiglu_workspace_bytes(16, 16, 4) == 0
    assert 0 < L.fp8_swiglu_workspace_bytes(8192, 14336, 0) < \
        L.fp8_swiglu_workspace_bytes(8192, 14336, 1)

    def fwd(a=A16, b=A16, rows=16, hidden=16, scaling=0, h=A16, q=A16, qt=A16, s=A16,
            st=A16, amax=None, ws=A16, wsb=1 << 20):
        v = lambda x: P(x) if x else None
        return L.fp8_swiglu_fwd(v(a), v(b), rows, hidden, scaling, v(h), v(q), v(qt), v(s),
                                v(st), v(amax), v(ws), wsb, None)

    assert fwd(scaling=E.FP8L_E5M2) == E.FP8L_EINVAL      # h is an activation: E4M3 only
    assert fwd(scaling=4) == E.FP8L_EINVAL
    assert fwd(hidden=40) == E.FP8L_ESHAPE
    assert fwd(rows=-16) == E.FP8L_ESHAPE
    for k in ("a", "b", "h", "q", "qt", "s", "st", "ws"):
        assert fwd(**{k: None}) == E.FP8L_EINVAL, k
    assert fwd(wsb=16) == E.FP8L_EWORKSPACE
    for k in ("a", "b", "h", "q", "qt", "ws"):
        assert fwd(**{k: A_BAD}) == E.FP8L_EALIGN, k
    assert fwd(s=A16 + 2) == E.FP8L_EALIGN

    names = ("dh", "a", "b", "da", "db", "daq", "daqt", "das", "dast", "daam", "dbq", "dbqt",
             "dbs", "dbst", "dbam", "ws")

    def bwd(rows=16, hidden=16, scaling=0, wsb=1 << 20, **kw):
        ptr = {n: kw.get(n, A16 if not n.endswith("am") else None) for n in names}
        v = lambda x: P(x) if x else None
        return L.fp8_swiglu_bwd(v(ptr["dh"]), v(ptr["a"]), v(ptr["b"]), rows, hidden, scaling,
                                *[v(ptr[n]) for n in names[3:15]], v(ptr["ws"]), wsb, None)

    assert bwd(scaling=8) == E.FP8L_EINVAL
    assert bwd(rows=8) == E.FP8L_ESHAPE
    for n in names:
        if not n.endswith("am"):
            assert bwd(**{n: None}) == E.FP8L_EINVAL, n
    assert bwd(wsb=0) == E.FP8L_EWORKSPACE
    for n in ("dh", "a", "b", "da", "db", "daq", "dbqt", "ws"):
        assert bwd(**{n: A_BAD}) == E.FP8L_EALIGN, n
    assert bwd(dbam=A16 + 1) == E.FP8L_EALIGN

    def acc(dyq=A16, sdy=A16, wtq=A16, swt=A16, M=16, N=16, K=16, scaling=0, gx=A16):
        v = lambda x: P(x) if x else None
        return L.fp8_linear_bwd_x_acc(v(dyq), v(sdy), v(wtq), v(swt), M, N, K, scaling, v(gx),
                                      None)

    assert acc(scaling=4) == E.FP8L_EINVAL
    assert acc(K=20) == E.FP8L_ESHAPE
    assert acc(gx=None) == E.FP8L_EINVAL
    assert acc(swt=None) == E.FP8L_EINVAL
    assert acc(gx=A_BAD) == E.FP8L_EALIGN


@pytestmark_cpu
def test_gemm_grouped_rejects_bad_arguments():
    E = ops
    L = ops.lib()

    def prob(c=A16, m=16, n=16, k=16, a=A16, sa=A16, b=A16, sb=A16):
        return ops.GemmProblem(a, sa, b, sb, c, m, n, k)

    def call(probs, count=None, scaling=0):
        arr = (ops.GemmProblem * max(len(probs), 1))(*probs)
        return L.fp8_linear_gemm_grouped(arr, len(probs) if count is None else count,
                                         scaling, None)

    assert L.fp8_linear_gemm_grouped(None, 1, 0, None) == E.FP8L_EINVAL
    assert call([prob()], count=0) == E.FP8L_EINVAL
    assert call([prob()] * 5) == E.FP8L_EINVAL                 # more than FP8L_MAX_GROUP
    assert call([prob()], scaling=4) == E.FP8L_EINVAL
    assert call([prob(m=24)]) == E.FP8L_ESHAPE
    assert call([prob(), prob(c=0x20000, k=-16)]) == E.FP8L_ESHAPE
    assert call([prob(a=None)]) == E.FP8L_EINVAL
    assert call([prob(sb=None)]) == E.FP8L_EINVAL
    assert call([prob(c=A_BAD)]) == E.FP8L_EALIGN
    # outputs overlapping: [A16, A16 + 512) and [A16 + 256, ...)
    assert call([prob(), prob(c=A16 + 256)]) == E.FP8L_EINVAL


@pytestmark_cpu
def test_mfma_probe_library_rejects_bad_arguments():
    """The measurement-only MFMA probe (bench.py's mfma_ceiling) loads and
    validates its arguments before launching anything."""
    import ctypes
    from float8_mixed_precision_amd import build as B
    L = ctypes.CDLL(B.PROBE_PATH)
    P, i64, I = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
    f = L.fp8_probe_mfma_loop
    f.restype = I
    f.argtypes = [P, i64, I, I, P, P]
    assert f(None, 1 << 20, 1, 1, A16, None) == 1
    assert f(A16, 1 << 20, 1, 1, None, None) == 1
    assert f(A16, 1 << 14, 1, 1, A16, None) == 1          # below one 32 KB slice
    assert f(A16, 1 << 20, 0, 1, A16, None) == 1
    assert f(A16, 1 << 20, 1, 0, A16, None) == 1
    assert f(A16 + 16, 1 << 20, 1, 1, A16, None) == 1     # codes not 32-byte aligned
