"""Python binding of libcsa (ctypes).  Argument marshalling only.

Each function has the name of the C entry point it calls and takes torch
tensors that already live on the GPU; it passes their device pointers,
sizes and strides, plus the current torch stream, to the library.  All
computation happens in the library's HIP kernels.  If ``libcsa.so`` is not
built, the first call raises ``CSAError``: there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os
import re
from typing import Optional

import torch

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libcsa.so")
HEADER_PATH = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "csa.h")

CSA_OK, CSA_ERR_INVALID_ARG, CSA_ERR_UNSUPPORTED, CSA_ERR_WORKSPACE, CSA_ERR_HIP = range(5)
CSA_F32, CSA_BF16 = 0, 1
_STATUS = {0: "CSA_OK", 1: "CSA_ERR_INVALID_ARG", 2: "CSA_ERR_UNSUPPORTED", 3: "CSA_ERR_WORKSPACE",
           4: "CSA_ERR_HIP"}


class CSAError(RuntimeError):
    def __init__(self, msg, status=None):
        super().__init__(msg)
        self.status = status


_lib = None

_i32, _i64, _f32, _vp, _sz = ctypes.c_int32, ctypes.c_int64, ctypes.c_float, ctypes.c_void_p, ctypes.c_size_t
_SIGS = {
    "csa_abi_version": (ctypes.c_int, []),
    "csa_last_error": (ctypes.c_char_p, []),
    "csa_project": (ctypes.c_int, [ctypes.c_int, ctypes.c_int, _i64, _i64, _i64, _vp, _i64, _vp, _i64, _vp,
                                   _i64, _vp]),
    "csa_project_pair": (ctypes.c_int, [ctypes.c_int, _i64, _i64, _vp, _i64, ctypes.c_int, _i64, _vp, _i64, _vp,
                                         _i64, ctypes.c_int, _i64, _vp, _i64, _vp, _i64, _vp]),
    "csa_project_backward_workspace": (ctypes.c_int, [ctypes.c_int, _i64, _i64, _i64, ctypes.c_int, ctypes.c_int,
                                                      ctypes.POINTER(_sz)]),
    "csa_project_backward": (ctypes.c_int, [ctypes.c_int, ctypes.c_int, _i64, _i64, _i64, _vp, _i64, _vp, _i64, _vp,
                                            _i64, _vp, _i64, _vp, _i64, _vp, _sz, _vp]),
    "csa_compress": (ctypes.c_int, [ctypes.c_int, _i64, _i32, _i32, _vp, _vp, _vp, _vp, _i64, _vp, _vp, _vp,
                                    _i64, _vp]),
    "csa_compress_append": (ctypes.c_int, [ctypes.c_int, _i64, _i32, _i32, _vp, _i64, _vp, _vp, _vp, _vp, _vp,
                                           _vp, _i64, _vp]),
    "csa_compress_append_pair": (ctypes.c_int, [ctypes.c_int, _i64, _i32, _vp, _vp, _i32, _vp, _i64, _vp, _vp, _vp,
                                                _vp, _i64, _i32, _vp, _i64, _vp, _vp, _vp, _vp, _i64, _vp]),
    "csa_compress_backward_workspace": (ctypes.c_int, [_i64, _i32, _i32, ctypes.POINTER(_sz)]),
    "csa_compress_backward": (ctypes.c_int, [ctypes.c_int, _i64, _i32, _i32, _vp, _vp, _vp, _vp, _i64, _vp, _vp,
                                             _vp, _i64, _vp, _vp, _vp, _vp, _i64, _vp, _vp, _vp, _sz, _vp]),
    "csa_index_topk_workspace": (ctypes.c_int, [_i64, _i64, _i32, _i32, ctypes.POINTER(_sz)]),
    "csa_index_topk": (ctypes.c_int, [ctypes.c_int, _i64, _i32, _i32, _i32, _i32, _vp, _vp, _vp, _vp, _vp,
                                      _vp, _i64, _vp, _vp, _vp, _sz, _vp]),
    "csa_index_topk_stream_workspace": (ctypes.c_int, [_i64, _i64, ctypes.POINTER(_sz)]),
    "csa_index_topk_stream": (ctypes.c_int, [ctypes.c_int, _i64, _i32, _i32, _i32, _i32, _vp, _vp, _vp, _i64, _vp,
                                             _vp, _vp, _sz, _vp]),
    "csa_sparse_mqa_workspace": (ctypes.c_int, [_i64, _i32, _i32, _i32, ctypes.POINTER(_sz)]),
    "csa_sparse_mqa": (ctypes.c_int, [ctypes.c_int, _i64, _i32, _i32, _i32, _f32, _vp, _vp, _vp, _vp, _vp,
                                      _vp, _vp, _vp, _sz, _vp]),
    "csa_sparse_mqa_backward_workspace": (ctypes.c_int, [_i64, _i32, _i32, _i32, _i64, ctypes.POINTER(_sz)]),
    "csa_sparse_mqa_backward": (ctypes.c_int, [ctypes.c_int, _i64, _i32, _i32, _i32, _f32, _vp, _vp, _i64, _vp, _vp,
                                               _vp, _vp, _vp, _vp, _vp, _vp, _vp, _sz, _vp]),
    "csa_compress_varlen": (ctypes.c_int, [ctypes.c_int, _i64, _i32, _i32, _vp, _vp, _vp, _vp, _i64, _vp, _vp, _vp,
                                           _vp, _i64, _vp, _i64, _vp]),
    "csa_compress_backward_varlen_workspace": (ctypes.c_int, [_i64, _i64, _i32, _i32, ctypes.POINTER(_sz)]),
    "csa_compress_backward_varlen": (ctypes.c_int, [ctypes.c_int, _i64, _i32, _i32, _vp, _vp, _vp, _vp, _i64, _vp,
                                                    _vp, _vp, _vp, _i64, _vp, _i64, _vp, _vp, _vp, _vp, _i64, _vp,
                                                    _vp, _vp, _sz, _vp]),
    "csa_index_topk_varlen_workspace": (ctypes.c_int, [_i64, _i64, _i64, _i32, ctypes.POINTER(_sz)]),
    "csa_index_topk_varlen": (ctypes.c_int, [ctypes.c_int, _i64, _i64, _i32, _i32, _i32, _i32, _vp, _vp, _vp, _vp,
                                             _vp, _i64, _vp, _vp, _vp, _vp, _sz, _vp]),
    "csa_decode_workspace": (ctypes.c_int, [_i64, _i64, _i32, _i32, _i32, _i32, ctypes.POINTER(_sz)]),
    "csa_decode": (ctypes.c_int, [ctypes.c_int, _i64, _i32, _i32, _i32, _i32, _i32, _i32, _f32, _vp, _vp, _vp, _vp,
                                  _vp, _vp, _vp, _vp, _i64, _vp, _vp, _vp, _vp, _vp, _sz, _vp]),
    "csa_decode_noalloc": (ctypes.c_int, [ctypes.c_int, _i64, _i32, _i32, _i32, _i32, _i32, _i32, _f32, _vp, _vp,
                                          _vp, _vp, _vp, _vp, _vp, _vp, _i64, _vp, _vp, _vp, _vp, _vp]),
    "csa_timing_enable": (ctypes.c_int, [ctypes.c_int]),
    "csa_timing_reset": (ctypes.c_int, []),
    "csa_timing_read": (ctypes.c_int, [ctypes.c_char_p, ctypes.POINTER(ctypes.c_double),
                                       ctypes.POINTER(_i64)]),
}


def header_functions():
    """Names of the functions declared in include/csa.h."""
    with open(HEADER_PATH) as f:
        text = f.read()
    return sorted(set(re.findall(r"^\s*(?:csa_status|int|const char\*)\s+(csa_\w+)\s*\(", text, re.M)))


def lib():
    """Load libcsa.so (once).  Raises CSAError if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise CSAError(f"{LIB_PATH} is missing: build it with "
                           "`python -m compressed_sparse_attention_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


def _check(status, what):
    if status != CSA_OK:
        msg = lib().csa_last_error().decode(errors="replace")
        raise CSAError(f"{what} failed with {_STATUS.get(status, status)}: {msg}", status)


def _dt(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return CSA_F32
    if t.dtype == torch.bfloat16:
        return CSA_BF16
    raise CSAError(f"unsupported dtype {t.dtype}")


def _ptr(t: Optional[torch.Tensor]):
    if t is None:
        return None
    if not t.is_cuda:
        raise CSAError("tensor must live on the GPU")
    return ctypes.c_void_p(t.data_ptr())


def _stream(device) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _rowmajor(t: torch.Tensor, name: str) -> int:
    """Leading dimension of a 2-D row-major view (unit column stride; any layout when empty)."""
    if t.dim() == 2 and t.numel() == 0:
        return max(t.shape[1], 1)
    if t.dim() != 2 or t.stride(1) != 1:
        raise CSAError(f"{name} must be a 2-D view with unit column stride")
    return t.stride(0)


def _contig(t: torch.Tensor, name: str):
    if not t.is_contiguous():
        raise CSAError(f"{name} must be contiguous")


# ---------------------------------------------------------------------------
# entry points
# ---------------------------------------------------------------------------


def csa_abi_version() -> int:
    return lib().csa_abi_version()


def csa_project(X: torch.Tensor, Wt: torch.Tensor, Y: torch.Tensor) -> torch.Tensor:
    """Y = X . Wt^T  (X [M,K], Wt [N,K] = W transposed, Y [M,N]; views allowed)."""
    M, K = X.shape
    N = Wt.shape[0]
    if Wt.shape[1] != K or tuple(Y.shape) != (M, N):
        raise CSAError("csa_project: shape mismatch")
    if X.dtype != Wt.dtype:
        raise CSAError("csa_project: X and Wt dtypes differ")
    _check(lib().csa_project(_dt(X), _dt(Y), M, N, K, _ptr(X), _rowmajor(X, "X"), _ptr(Wt),
                             _rowmajor(Wt, "Wt"), _ptr(Y), _rowmajor(Y, "Y"), _stream(X.device)),
           "csa_project")
    return Y


def csa_project_pair(X: torch.Tensor, Wt1: torch.Tensor, Y1: torch.Tensor, Wt2: torch.Tensor,
                     Y2: torch.Tensor) -> None:
    """Y1 = X . Wt1^T and Y2 = X . Wt2^T, one launch when X has at most 16 bf16 rows (views allowed)."""
    M, K = X.shape
    N1, N2 = Wt1.shape[0], Wt2.shape[0]
    if Wt1.shape[1] != K or Wt2.shape[1] != K or tuple(Y1.shape) != (M, N1) or tuple(Y2.shape) != (M, N2):
        raise CSAError("csa_project_pair: shape mismatch")
    if X.dtype != Wt1.dtype or X.dtype != Wt2.dtype:
        raise CSAError("csa_project_pair: X and weight dtypes differ")
    _check(lib().csa_project_pair(_dt(X), M, K, _ptr(X), _rowmajor(X, "X"), _dt(Y1), N1, _ptr(Wt1),
                                  _rowmajor(Wt1, "Wt1"), _ptr(Y1), _rowmajor(Y1, "Y1"), _dt(Y2), N2, _ptr(Wt2),
                                  _rowmajor(Wt2, "Wt2"), _ptr(Y2), _rowmajor(Y2, "Y2"), _stream(X.device)),
           "csa_project_pair")


def csa_project_backward_workspace(dtype, M: int, N: int, K: int, want_dx: bool, want_dw: bool) -> int:
    b = _sz(0)
    dt = CSA_F32 if dtype == torch.float32 else CSA_BF16
    _check(lib().csa_project_backward_workspace(dt, M, N, K, int(want_dx), int(want_dw), ctypes.byref(b)),
           "csa_project_backward_workspace")
    return b.value


def csa_project_backward(X, Wt, dY, dX=None, dWt=None, workspace=None):
    """Gradients of Y = X . Wt^T: dX [M, K] = dY . Wt, dWt [N, K] = dY^T . X (either may be None; views allowed)."""
    M, K = X.shape
    N = Wt.shape[0]
    if Wt.shape[1] != K or tuple(dY.shape) != (M, N) or X.dtype != Wt.dtype or dY.dtype != X.dtype:
        raise CSAError("csa_project_backward: shape or dtype mismatch")
    out = dX if dX is not None else dWt
    if out is None:
        return dX, dWt
    if dX is not None and (tuple(dX.shape) != (M, K) or dX.dtype != out.dtype):
        raise CSAError("csa_project_backward: dX must be [M, K]")
    if dWt is not None and (tuple(dWt.shape) != (N, K) or dWt.dtype != out.dtype):
        raise CSAError("csa_project_backward: dWt must be [N, K] of the dX dtype")
    need = csa_project_backward_workspace(X.dtype, M, N, K, dX is not None, dWt is not None)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=X.device)
    _check(lib().csa_project_backward(_dt(X), _dt(out), M, N, K, _ptr(X), _rowmajor(X, "X"), _ptr(Wt),
                                      _rowmajor(Wt, "Wt"), _ptr(dY), _rowmajor(dY, "dY"), _ptr(dX),
                                      _rowmajor(dX, "dX") if dX is not None else K, _ptr(dWt),
                                      _rowmajor(dWt, "dWt") if dWt is not None else K, _ptr(workspace),
                                      workspace.numel(), _stream(X.device)),
           "csa_project_backward")
    return dX, dWt


def csa_compress(Ca, Cb, Za, Zb, Ba, Bb, m: int, Ccomp: torch.Tensor) -> torch.Tensor:
    """Eqs 3-4.  Ca/Cb/Za/Zb: [n, c] views sharing one leading dimension; Ba/Bb [m, c]."""
    n, c = Ca.shape
    ld = _rowmajor(Ca, "Ca")
    for t, nm in ((Cb, "Cb"), (Za, "Za"), (Zb, "Zb")):
        if tuple(t.shape) != (n, c) or _rowmajor(t, nm) != ld or t.dtype != Ca.dtype:
            raise CSAError("csa_compress: Ca, Cb, Za, Zb must share shape, dtype and leading dimension")
    for t, nm in ((Ba, "Ba"), (Bb, "Bb")):
        _contig(t, nm)
        if tuple(t.shape) != (m, c):
            raise CSAError(f"csa_compress: {nm} must be [m, c]")
    if tuple(Ccomp.shape) != (n // m, c):
        raise CSAError("csa_compress: Ccomp must be [n // m, c]")
    _check(lib().csa_compress(_dt(Ca), n, m, c, _ptr(Ca), _ptr(Cb), _ptr(Za), _ptr(Zb), ld, _ptr(Ba),
                              _ptr(Bb), _ptr(Ccomp), _rowmajor(Ccomp, "Ccomp"), _stream(Ca.device)),
           "csa_compress")
    return Ccomp


def csa_compress_append(new_rows, ring, Ba, Bb, m: int, t_new, kv_offset, Ccomp) -> torch.Tensor:
    """Eqs 3-4 for one new token per sequence.  new_rows [B, >= 4c] (C^a|C^b|Z^a|Z^b), ring [B, 2m, 4c],
    Ba/Bb [m, c], t_new/kv_offset [B] int64 (device), Ccomp [rows, c] (row kv_offset[b] + t_new[b] // m is
    written when t_new[b] completes a block)."""
    B = new_rows.shape[0]
    c = Ccomp.shape[1]
    _contig(ring, "ring")
    if tuple(ring.shape) != (B, 2 * m, 4 * c) or ring.dtype != Ccomp.dtype or new_rows.dtype != Ccomp.dtype:
        raise CSAError("csa_compress_append: ring must be [B, 2m, 4c] of the cache dtype")
    for t, nm in ((Ba, "Ba"), (Bb, "Bb")):
        _contig(t, nm)
        if tuple(t.shape) != (m, c):
            raise CSAError(f"csa_compress_append: {nm} must be [m, c]")
    for t, nm in ((t_new, "t_new"), (kv_offset, "kv_offset")):
        if t.dtype != torch.int64 or tuple(t.shape) != (B,):
            raise CSAError(f"csa_compress_append: {nm} must be int64 [B]")
    _check(lib().csa_compress_append(_dt(Ccomp), B, m, c, _ptr(new_rows), _rowmajor(new_rows, "new_rows"),
                                     _ptr(ring), _ptr(Ba), _ptr(Bb), _ptr(t_new), _ptr(kv_offset), _ptr(Ccomp),
                                     _rowmajor(Ccomp, "Ccomp"), _stream(Ccomp.device)),
           "csa_compress_append")
    return Ccomp


def csa_compress_append_pair(rows1, ring1, Ba1, Bb1, Ccomp1, rows2, ring2, Ba2, Bb2, Ccomp2, m: int, t_new,
                             kv_offset):
    """csa_compress_append on two caches of the same sequences (same t_new, kv_offset) in one launch."""
    B = rows1.shape[0]
    args = []
    for x, (rows, ring, Ba, Bb, Ccomp) in enumerate(((rows1, ring1, Ba1, Bb1, Ccomp1), (rows2, ring2, Ba2, Bb2, Ccomp2))):
        c = Ccomp.shape[1]
        _contig(ring, "ring")
        if rows.shape[0] != B or tuple(ring.shape) != (B, 2 * m, 4 * c) or ring.dtype != Ccomp1.dtype \
                or rows.dtype != Ccomp1.dtype or Ccomp.dtype != Ccomp1.dtype:
            raise CSAError(f"csa_compress_append_pair: cache {x + 1}: ring must be [B, 2m, 4c] of the cache dtype")
        for t, nm in ((Ba, "Ba"), (Bb, "Bb")):
            _contig(t, nm)
            if tuple(t.shape) != (m, c) or t.dtype != Ccomp1.dtype:
                raise CSAError(f"csa_compress_append_pair: cache {x + 1}: {nm} must be [m, c]")
        args += [c, _ptr(rows), _rowmajor(rows, "new_rows"), _ptr(ring), _ptr(Ba), _ptr(Bb), _ptr(Ccomp),
                 _rowmajor(Ccomp, "Ccomp")]
    for t, nm in ((t_new, "t_new"), (kv_offset, "kv_offset")):
        if t.dtype != torch.int64 or tuple(t.shape) != (B,):
            raise CSAError(f"csa_compress_append_pair: {nm} must be int64 [B]")
    _check(lib().csa_compress_append_pair(_dt(Ccomp1), B, m, _ptr(t_new), _ptr(kv_offset), *args,
                                          _stream(Ccomp1.device)), "csa_compress_append_pair")
    return Ccomp1, Ccomp2


def csa_compress_backward_workspace(n: int, m: int, c: int) -> int:
    b = _sz(0)
    _check(lib().csa_compress_backward_workspace(n, m, c, ctypes.byref(b)), "csa_compress_backward_workspace")
    return b.value


def csa_compress_backward(Ca, Cb, Za, Zb, Ba, Bb, m: int, dCcomp, dCa, dCb, dZa, dZb, dBa, dBb, workspace=None):
    """Gradients of eqs 3-4.  Forward inputs as csa_compress; dCcomp [n // m, c] fp32; outputs dCa/dCb/dZa/dZb
    [n, c] views of the inputs' dtype sharing one leading dimension, dBa/dBb [m, c] fp32 (overwritten)."""
    n, c = Ca.shape
    ld = _rowmajor(Ca, "Ca")
    for t, nm in ((Cb, "Cb"), (Za, "Za"), (Zb, "Zb")):
        if tuple(t.shape) != (n, c) or _rowmajor(t, nm) != ld or t.dtype != Ca.dtype:
            raise CSAError("csa_compress_backward: Ca, Cb, Za, Zb must share shape, dtype and leading dimension")
    ldo = _rowmajor(dCa, "dCa")
    for t, nm in ((dCa, "dCa"), (dCb, "dCb"), (dZa, "dZa"), (dZb, "dZb")):
        if tuple(t.shape) != (n, c) or _rowmajor(t, nm) != ldo or t.dtype != Ca.dtype:
            raise CSAError("csa_compress_backward: dCa, dCb, dZa, dZb must be [n, c] of the input dtype "
                           "sharing one leading dimension")
    for t, nm in ((Ba, "Ba"), (Bb, "Bb"), (dBa, "dBa"), (dBb, "dBb")):
        _contig(t, nm)
        if tuple(t.shape) != (m, c):
            raise CSAError(f"csa_compress_backward: {nm} must be [m, c]")
    if dBa.dtype != torch.float32 or dBb.dtype != torch.float32 or dCcomp.dtype != torch.float32:
        raise CSAError("csa_compress_backward: dCcomp, dBa and dBb are fp32")
    if tuple(dCcomp.shape) != (n // m, c):
        raise CSAError("csa_compress_backward: dCcomp must be [n // m, c]")
    need = csa_compress_backward_workspace(n, m, c)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=Ca.device)
    _check(lib().csa_compress_backward(_dt(Ca), n, m, c, _ptr(Ca), _ptr(Cb), _ptr(Za), _ptr(Zb), ld, _ptr(Ba),
                                       _ptr(Bb), _ptr(dCcomp), _rowmajor(dCcomp, "dCcomp") if n // m else c,
                                       _ptr(dCa), _ptr(dCb), _ptr(dZa), _ptr(dZb), ldo, _ptr(dBa), _ptr(dBb),
                                       _ptr(workspace), workspace.numel(), _stream(Ca.device)),
           "csa_compress_backward")
    return dCa, dCb, dZa, dZb, dBa, dBb


def csa_index_topk_workspace(n_queries: int, max_cand: int, n_hI: int, k: int) -> int:
    b = _sz(0)
    _check(lib().csa_index_topk_workspace(n_queries, max_cand, n_hI, k, ctypes.byref(b)),
           "csa_index_topk_workspace")
    return b.value


def csa_index_topk_stream_workspace(n_queries: int, max_cand: int) -> int:
    b = _sz(0)
    _check(lib().csa_index_topk_stream_workspace(n_queries, max_cand, ctypes.byref(b)),
           "csa_index_topk_stream_workspace")
    return b.value


def csa_index_topk_stream(qI, wI, KIcomp, m: int, k: int, max_cand: int, idx_out, score_out=None,
                          workspace=None):
    """Eqs 8-9 for one sequence's prefill (query t at position t) without the causal score matrix.
    qI [n, n_hI, cI], wI [n, n_hI] fp32, KIcomp [rows, cI] -> idx_out [n, k] (each row in index order)."""
    nq, nhI, cI = qI.shape
    for t, nm in ((qI, "qI"), (wI, "wI"), (KIcomp, "KIcomp"), (idx_out, "idx_out")):
        _contig(t, nm)
    if wI.dtype != torch.float32 or tuple(wI.shape) != (nq, nhI):
        raise CSAError("csa_index_topk_stream: wI must be fp32 [n_queries, n_hI]")
    if idx_out.dtype != torch.int32 or tuple(idx_out.shape) != (nq, k):
        raise CSAError("csa_index_topk_stream: idx_out must be int32 [n_queries, k]")
    if score_out is not None:
        _contig(score_out, "score_out")
        if score_out.dtype != torch.float32 or tuple(score_out.shape) != (nq, k):
            raise CSAError("csa_index_topk_stream: score_out must be fp32 [n_queries, k]")
    need = csa_index_topk_stream_workspace(nq, max_cand)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=qI.device)
    _check(lib().csa_index_topk_stream(_dt(qI), nq, nhI, cI, m, k, _ptr(qI), _ptr(wI), _ptr(KIcomp), max_cand,
                                       _ptr(idx_out), _ptr(score_out), _ptr(workspace),
                                       workspace.numel() * workspace.element_size(), _stream(qI.device)),
           "csa_index_topk_stream")
    return idx_out


def csa_index_topk(qI, wI, KIcomp, m: int, k: int, max_cand: int, idx_out, score_out=None,
                   q_seq=None, q_pos=None, kv_offset=None, workspace=None):
    """Eqs 8-9.  qI [nq, n_hI, cI], wI [nq, n_hI] fp32, KIcomp [rows, cI] -> idx_out [nq, k]."""
    nq, nhI, cI = qI.shape
    for t, nm in ((qI, "qI"), (wI, "wI"), (KIcomp, "KIcomp"), (idx_out, "idx_out")):
        _contig(t, nm)
    if wI.dtype != torch.float32 or tuple(wI.shape) != (nq, nhI):
        raise CSAError("csa_index_topk: wI must be fp32 [n_queries, n_hI]")
    if idx_out.dtype != torch.int32 or tuple(idx_out.shape) != (nq, k):
        raise CSAError("csa_index_topk: idx_out must be int32 [n_queries, k]")
    if score_out is not None:
        _contig(score_out, "score_out")
        if score_out.dtype != torch.float32 or tuple(score_out.shape) != (nq, k):
            raise CSAError("csa_index_topk: score_out must be fp32 [n_queries, k]")
    if q_seq is not None and (q_seq.dtype != torch.int32 or q_seq.numel() != nq):
        raise CSAError("csa_index_topk: q_seq must be int32 [n_queries]")
    if q_pos is not None and (q_pos.dtype != torch.int64 or q_pos.numel() != nq):
        raise CSAError("csa_index_topk: q_pos must be int64 [n_queries]")
    if kv_offset is not None and kv_offset.dtype != torch.int64:
        raise CSAError("csa_index_topk: kv_offset must be int64")
    need = csa_index_topk_workspace(nq, max_cand, nhI, k)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=qI.device)
    _check(lib().csa_index_topk(_dt(qI), nq, nhI, cI, m, k, _ptr(qI), _ptr(wI), _ptr(KIcomp), _ptr(q_seq),
                                _ptr(q_pos), _ptr(kv_offset), max_cand, _ptr(idx_out), _ptr(score_out),
                                _ptr(workspace), workspace.numel() * workspace.element_size(),
                                _stream(qI.device)),
           "csa_index_topk")
    return idx_out


def csa_sparse_mqa_workspace(n_queries: int, n_h: int, c: int, k: int) -> int:
    b = _sz(0)
    _check(lib().csa_sparse_mqa_workspace(n_queries, n_h, c, k, ctypes.byref(b)), "csa_sparse_mqa_workspace")
    return b.value


def csa_sparse_mqa(q, Ccomp, idx, scale: float, o, lse=None, q_seq=None, kv_offset=None, workspace=None):
    """Eq 11.  q [nq, n_h, c], Ccomp [rows, c], idx [nq, k] int32 -> o [nq, n_h, c] (+ lse [nq, n_h])."""
    nq, nh, c = q.shape
    k = idx.shape[1]
    for t, nm in ((q, "q"), (Ccomp, "Ccomp"), (idx, "idx"), (o, "o")):
        _contig(t, nm)
    if idx.dtype != torch.int32 or idx.shape[0] != nq:
        raise CSAError("csa_sparse_mqa: idx must be int32 [n_queries, k]")
    if o.dtype != q.dtype or tuple(o.shape) != (nq, nh, c) or Ccomp.dtype != q.dtype:
        raise CSAError("csa_sparse_mqa: o/Ccomp must match q's dtype and o q's shape")
    if lse is not None:
        _contig(lse, "lse")
        if lse.dtype != torch.float32 or tuple(lse.shape) != (nq, nh):
            raise CSAError("csa_sparse_mqa: lse must be fp32 [n_queries, n_h]")
    if q_seq is not None and (q_seq.dtype != torch.int32 or q_seq.numel() != nq):
        raise CSAError("csa_sparse_mqa: q_seq must be int32 [n_queries]")
    if kv_offset is not None and kv_offset.dtype != torch.int64:
        raise CSAError("csa_sparse_mqa: kv_offset must be int64")
    need = csa_sparse_mqa_workspace(nq, nh, c, k)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    _check(lib().csa_sparse_mqa(_dt(q), nq, nh, c, k, float(scale), _ptr(q), _ptr(Ccomp), _ptr(q_seq),
                                _ptr(kv_offset), _ptr(idx), _ptr(o), _ptr(lse), _ptr(workspace),
                                workspace.numel() * workspace.element_size(), _stream(q.device)),
           "csa_sparse_mqa")
    return o


def csa_sparse_mqa_backward_workspace(n_queries: int, n_h: int, c: int, k: int, n_rows: int) -> int:
    b = _sz(0)
    _check(lib().csa_sparse_mqa_backward_workspace(n_queries, n_h, c, k, n_rows, ctypes.byref(b)),
           "csa_sparse_mqa_backward_workspace")
    return b.value


def csa_sparse_mqa_backward(q, Ccomp, idx, scale: float, o, lse, dO, dq, dCcomp, q_seq=None, kv_offset=None,
                            workspace=None):
    """Gradients of eq 11: q/o/dO/dq [n, n_h, c] bf16, Ccomp [rows, c] bf16, idx [n, k] int32, lse [n, n_h] fp32,
    dCcomp [rows, c] fp32 (overwritten)."""
    n, nh, c = q.shape
    k = idx.shape[1]
    rows = Ccomp.shape[0]
    for t, nm in ((q, "q"), (o, "o"), (dO, "dO"), (dq, "dq")):
        _contig(t, nm)
        if tuple(t.shape) != (n, nh, c) or t.dtype != Ccomp.dtype:
            raise CSAError(f"csa_sparse_mqa_backward: {nm} must be [n, n_h, c] of the Ccomp dtype")
    _contig(Ccomp, "Ccomp")
    _contig(idx, "idx")
    _contig(lse, "lse")
    _contig(dCcomp, "dCcomp")
    if idx.dtype != torch.int32 or idx.shape[0] != n:
        raise CSAError("csa_sparse_mqa_backward: idx must be int32 [n, k]")
    if lse.dtype != torch.float32 or tuple(lse.shape) != (n, nh):
        raise CSAError("csa_sparse_mqa_backward: lse must be fp32 [n, n_h]")
    if dCcomp.dtype != torch.float32 or tuple(dCcomp.shape) != (rows, c):
        raise CSAError("csa_sparse_mqa_backward: dCcomp must be fp32 [rows, c]")
    need = csa_sparse_mqa_backward_workspace(n, nh, c, k, rows)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    _check(lib().csa_sparse_mqa_backward(_dt(q), n, nh, c, k, scale, _ptr(q), _ptr(Ccomp), rows, _ptr(q_seq),
                                         _ptr(kv_offset), _ptr(idx), _ptr(o), _ptr(lse), _ptr(dO), _ptr(dq),
                                         _ptr(dCcomp), _ptr(workspace), workspace.numel(), _stream(q.device)),
           "csa_sparse_mqa_backward")
    return dq, dCcomp


def csa_compress_varlen(Ca, Cb, Za, Zb, Ba, Bb, m: int, cu_seqlens, block_offset, n_blocks: int, Ccomp):
    """Eqs 3-4 for packed sequences: sequence b's rows cu_seqlens[b] .. cu_seqlens[b+1]-1 of the [n, c] column
    slices Ca/Cb/Za/Zb (one shared leading dimension) -> Ccomp rows block_offset[b] .. block_offset[b+1]-1."""
    c = Ca.shape[1]
    ld = _rowmajor(Ca, "Ca")
    for t, nm in ((Cb, "Cb"), (Za, "Za"), (Zb, "Zb")):
        if _rowmajor(t, nm) != ld or tuple(t.shape) != tuple(Ca.shape) or t.dtype != Ca.dtype:
            raise CSAError("csa_compress_varlen: Ca, Cb, Za, Zb must share shape, dtype and row stride")
    for t, nm in ((Ba, "Ba"), (Bb, "Bb")):
        _contig(t, nm)
        if tuple(t.shape) != (m, c) or t.dtype != Ca.dtype:
            raise CSAError(f"csa_compress_varlen: {nm} must be [m, c] of Ca's dtype")
    nseq = cu_seqlens.numel() - 1
    for t, nm in ((cu_seqlens, "cu_seqlens"), (block_offset, "block_offset")):
        if t.dtype != torch.int64 or t.numel() != nseq + 1:
            raise CSAError(f"csa_compress_varlen: {nm} must be int64 [n_seqs + 1]")
    if Ccomp.shape[0] < n_blocks or Ccomp.shape[1] != c or Ccomp.dtype != Ca.dtype:
        raise CSAError("csa_compress_varlen: Ccomp must be [>= n_blocks, c] of Ca's dtype")
    _check(lib().csa_compress_varlen(_dt(Ca), nseq, m, c, _ptr(Ca), _ptr(Cb), _ptr(Za), _ptr(Zb), ld, _ptr(Ba),
                                     _ptr(Bb), _ptr(cu_seqlens), _ptr(block_offset), n_blocks, _ptr(Ccomp),
                                     _rowmajor(Ccomp, "Ccomp"), _stream(Ca.device)),
           "csa_compress_varlen")
    return Ccomp


def csa_compress_backward_varlen_workspace(n_seqs: int, n_blocks: int, m: int, c: int) -> int:
    b = _sz(0)
    _check(lib().csa_compress_backward_varlen_workspace(n_seqs, n_blocks, m, c, ctypes.byref(b)),
           "csa_compress_backward_varlen_workspace")
    return b.value


def csa_compress_backward_varlen(Ca, Cb, Za, Zb, Ba, Bb, m: int, cu_seqlens, block_offset, n_blocks: int, dCcomp,
                                 dCa, dCb, dZa, dZb, dBa, dBb, workspace=None):
    """Gradients of eqs 3-4 for packed sequences (the layout of csa_compress_varlen): dCcomp [>= n_blocks, c] fp32;
    dCa/dCb/dZa/dZb shaped like Ca and sharing one leading dimension; dBa/dBb [m, c] fp32 summed over every
    sequence's blocks (overwritten)."""
    n, c = Ca.shape
    ld = _rowmajor(Ca, "Ca")
    for t, nm in ((Cb, "Cb"), (Za, "Za"), (Zb, "Zb")):
        if tuple(t.shape) != (n, c) or _rowmajor(t, nm) != ld or t.dtype != Ca.dtype:
            raise CSAError("csa_compress_backward_varlen: Ca, Cb, Za, Zb must share shape, dtype and row stride")
    ldo = _rowmajor(dCa, "dCa")
    for t, nm in ((dCa, "dCa"), (dCb, "dCb"), (dZa, "dZa"), (dZb, "dZb")):
        if tuple(t.shape) != (n, c) or _rowmajor(t, nm) != ldo or t.dtype != Ca.dtype:
            raise CSAError("csa_compress_backward_varlen: dCa, dCb, dZa, dZb must be shaped like Ca, of its dtype, "
                           "sharing one leading dimension")
    for t, nm in ((Ba, "Ba"), (Bb, "Bb"), (dBa, "dBa"), (dBb, "dBb")):
        _contig(t, nm)
        if tuple(t.shape) != (m, c):
            raise CSAError(f"csa_compress_backward_varlen: {nm} must be [m, c]")
    if dBa.dtype != torch.float32 or dBb.dtype != torch.float32 or dCcomp.dtype != torch.float32:
        raise CSAError("csa_compress_backward_varlen: dCcomp, dBa and dBb are fp32")
    nseq = cu_seqlens.numel() - 1
    for t, nm in ((cu_seqlens, "cu_seqlens"), (block_offset, "block_offset")):
        if t.dtype != torch.int64 or t.numel() != nseq + 1:
            raise CSAError(f"csa_compress_backward_varlen: {nm} must be int64 [n_seqs + 1]")
    if dCcomp.dim() != 2 or dCcomp.shape[0] < n_blocks or dCcomp.shape[1] != c:
        raise CSAError("csa_compress_backward_varlen: dCcomp must be [>= n_blocks, c]")
    need = csa_compress_backward_varlen_workspace(nseq, n_blocks, m, c)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=Ca.device)
    _check(lib().csa_compress_backward_varlen(
        _dt(Ca), nseq, m, c, _ptr(Ca), _ptr(Cb), _ptr(Za), _ptr(Zb), ld, _ptr(Ba), _ptr(Bb), _ptr(cu_seqlens),
        _ptr(block_offset), n_blocks, _ptr(dCcomp), _rowmajor(dCcomp, "dCcomp") if dCcomp.shape[0] else c,
        _ptr(dCa), _ptr(dCb), _ptr(dZa), _ptr(dZb), ldo, _ptr(dBa), _ptr(dBb), _ptr(workspace), workspace.numel(),
        _stream(Ca.device)), "csa_compress_backward_varlen")
    return dCa, dCb, dZa, dZb, dBa, dBb


def csa_index_topk_varlen_workspace(n_seqs: int, n_tokens: int, max_cand: int, k: int) -> int:
    b = _sz(0)
    _check(lib().csa_index_topk_varlen_workspace(n_seqs, n_tokens, max_cand, k, ctypes.byref(b)),
           "csa_index_topk_varlen_workspace")
    return b.value


def csa_index_topk_varlen(qI, wI, KIcomp, m: int, k: int, max_cand: int, cu_seqlens, kv_offset, idx_out,
                          score_out=None, q_seq_out=None, workspace=None):
    """Eqs 8-9 for every token of packed sequences.  qI [n, n_hI, cI], wI [n, n_hI] fp32 -> idx_out [n, k]."""
    n, nhI, cI = qI.shape
    for t, nm in ((qI, "qI"), (wI, "wI"), (KIcomp, "KIcomp"), (idx_out, "idx_out")):
        _contig(t, nm)
    if wI.dtype != torch.float32 or tuple(wI.shape) != (n, nhI):
        raise CSAError("csa_index_topk_varlen: wI must be fp32 [n_tokens, n_hI]")
    if idx_out.dtype != torch.int32 or tuple(idx_out.shape) != (n, k):
        raise CSAError("csa_index_topk_varlen: idx_out must be int32 [n_tokens, k]")
    if score_out is not None:
        _contig(score_out, "score_out")
        if score_out.dtype != torch.float32 or tuple(score_out.shape) != (n, k):
            raise CSAError("csa_index_topk_varlen: score_out must be fp32 [n_tokens, k]")
    if q_seq_out is not None and (q_seq_out.dtype != torch.int32 or q_seq_out.numel() != n):
        raise CSAError("csa_index_topk_varlen: q_seq_out must be int32 [n_tokens]")
    nseq = cu_seqlens.numel() - 1
    if cu_seqlens.dtype != torch.int64 or kv_offset.dtype != torch.int64 or kv_offset.numel() < nseq:
        raise CSAError("csa_index_topk_varlen: cu_seqlens [n_seqs + 1] and kv_offset [>= n_seqs] must be int64")
    need = csa_index_topk_varlen_workspace(nseq, n, max_cand, k)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=qI.device)
    _check(lib().csa_index_topk_varlen(_dt(qI), nseq, n, nhI, cI, m, k, _ptr(qI), _ptr(wI), _ptr(KIcomp),
                                       _ptr(cu_seqlens), _ptr(kv_offset), max_cand, _ptr(idx_out), _ptr(score_out),
                                       _ptr(q_seq_out), _ptr(workspace), workspace.numel() * workspace.element_size(),
                                       _stream(qI.device)),
           "csa_index_topk_varlen")
    return idx_out


def csa_decode_workspace(n_queries: int, max_cand: int, n_hI: int, n_h: int, c: int, k: int) -> int:
    b = _sz(0)
    _check(lib().csa_decode_workspace(n_queries, max_cand, n_hI, n_h, c, k, ctypes.byref(b)), "csa_decode_workspace")
    return b.value


def _decode_args(fn, qI, wI, KIcomp, q, Ccomp, k, q_pos, idx_out, o, lse, score_out, q_seq, kv_offset,
                 workspace=None):
    """Checks shared by csa_decode and csa_decode_noalloc."""
    nq, nhI, cI = qI.shape
    _, nh, c = q.shape
    for t, nm in ((qI, "qI"), (wI, "wI"), (KIcomp, "KIcomp"), (q, "q"), (Ccomp, "Ccomp"), (idx_out, "idx_out"),
                  (o, "o")) + (((workspace, "workspace"),) if workspace is not None else ()):
        _contig(t, nm)
    if wI.dtype != torch.float32 or tuple(wI.shape) != (nq, nhI):
        raise CSAError(f"{fn}: wI must be fp32 [n_queries, n_hI]")
    if idx_out.dtype != torch.int32 or tuple(idx_out.shape) != (nq, k):
        raise CSAError(f"{fn}: idx_out must be int32 [n_queries, k]")
    if tuple(q.shape[:1]) != (nq,) or o.dtype != q.dtype or tuple(o.shape) != (nq, nh, c):
        raise CSAError(f"{fn}: o must match q [n_queries, n_h, c]")
    if KIcomp.dtype != qI.dtype or Ccomp.dtype != q.dtype or q.dtype != qI.dtype:
        raise CSAError(f"{fn}: caches and queries must share one dtype")
    if q_pos is None or q_pos.dtype != torch.int64 or q_pos.numel() != nq:
        raise CSAError(f"{fn}: q_pos must be int64 [n_queries]")
    if q_seq is not None and (q_seq.dtype != torch.int32 or q_seq.numel() != nq):
        raise CSAError(f"{fn}: q_seq must be int32 [n_queries]")
    if kv_offset is not None and kv_offset.dtype != torch.int64:
        raise CSAError(f"{fn}: kv_offset must be int64")
    for t, nm, shape in ((lse, "lse", (nq, nh)), (score_out, "score_out", (nq, k))):
        if t is not None:
            _contig(t, nm)
            if t.dtype != torch.float32 or tuple(t.shape) != shape:
                raise CSAError(f"{fn}: {nm} must be fp32 {list(shape)}")
    return nq, nhI, cI, nh, c


def csa_decode_noalloc(qI, wI, KIcomp, q, Ccomp, m: int, k: int, max_cand: int, scale: float, q_pos, idx_out, o,
                       lse=None, score_out=None, q_seq=None, kv_offset=None):
    """csa_decode with the library's static per-GPU scratch instead of a workspace (for callers that cannot
    allocate); calls that overlap on one GPU race on that scratch."""
    nq, nhI, cI, nh, c = _decode_args("csa_decode_noalloc", qI, wI, KIcomp, q, Ccomp, k, q_pos, idx_out, o, lse,
                                      score_out, q_seq, kv_offset)
    _check(lib().csa_decode_noalloc(_dt(q), nq, nhI, cI, nh, c, m, k, float(scale), _ptr(qI), _ptr(wI),
                                    _ptr(KIcomp), _ptr(q), _ptr(Ccomp), _ptr(q_seq), _ptr(q_pos), _ptr(kv_offset),
                                    max_cand, _ptr(idx_out), _ptr(score_out), _ptr(o), _ptr(lse),
                                    _stream(q.device)),
           "csa_decode_noalloc")
    return o


def csa_decode(qI, wI, KIcomp, q, Ccomp, m: int, k: int, max_cand: int, scale: float, q_pos, idx_out, o,
               workspace, lse=None, score_out=None, q_seq=None, kv_offset=None):
    """Eqs 8, 9 and 11 for a batch of decode queries in one call.  `workspace` (uint8, at least
    csa_decode_workspace bytes) must be zero-filled before its first use and again whenever the
    sizes change; every call leaves it ready for the next."""
    nq, nhI, cI, nh, c = _decode_args("csa_decode", qI, wI, KIcomp, q, Ccomp, k, q_pos, idx_out, o, lse,
                                      score_out, q_seq, kv_offset, workspace)
    _check(lib().csa_decode(_dt(q), nq, nhI, cI, nh, c, m, k, float(scale), _ptr(qI), _ptr(wI), _ptr(KIcomp),
                            _ptr(q), _ptr(Ccomp), _ptr(q_seq), _ptr(q_pos), _ptr(kv_offset), max_cand,
                            _ptr(idx_out), _ptr(score_out), _ptr(o), _ptr(lse), _ptr(workspace),
                            workspace.numel() * workspace.element_size(), _stream(q.device)),
           "csa_decode")
    return o


def csa_timing_enable(on: bool = True):
    _check(lib().csa_timing_enable(1 if on else 0), "csa_timing_enable")


def csa_timing_reset():
    _check(lib().csa_timing_reset(), "csa_timing_reset")


def csa_timing_read(name: str):
    ms = ctypes.c_double(0)
    n = _i64(0)
    _check(lib().csa_timing_read(name.encode(), ctypes.byref(ms), ctypes.byref(n)), "csa_timing_read")
    return ms.value, n.value
