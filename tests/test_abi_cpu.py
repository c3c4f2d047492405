"""The C-ABI library on the CPU: it loads, exports every declared entry point,
and rejects bad arguments before touching any device (no compute calls)."""
import ctypes
import os
import re
import subprocess

import pytest

from compressed_sparse_attention_amd import api

HERE = os.path.dirname(os.path.abspath(__file__))


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(api.LIB_PATH):
        pytest.fail("libcsa.so is not built (run __graft_entry__.build())")
    return api.lib()


def test_exports_every_declared_symbol(L):
    declared = api.header_functions()
    assert {"csa_project", "csa_compress", "csa_index_topk", "csa_sparse_mqa"} <= set(declared)
    out = subprocess.run(["nm", "-D", "--defined-only", api.LIB_PATH], capture_output=True, text=True,
                         check=True).stdout
    exported = set(re.findall(r"\bT\s+(csa_\w+)$", out, re.M))
    missing = set(declared) - exported
    assert not missing, f"declared but not exported: {sorted(missing)}"
    for name in declared:
        assert hasattr(L, name)


def test_abi_version(L):
    assert api.csa_abi_version() == 1


def _err():
    return api.lib().csa_last_error().decode()


def test_project_rejects_bad_args(L):
    p = ctypes.c_void_p(16)
    assert L.csa_project(1, 1, 0, 8, 8, p, 8, p, 8, p, 8, None) == api.CSA_ERR_INVALID_ARG
    assert "positive" in _err()
    assert L.csa_project(1, 1, 8, 8, 12, p, 16, p, 16, p, 8, None) == api.CSA_ERR_INVALID_ARG
    assert "multiple of 8" in _err()
    assert L.csa_project(1, 1, 8, 8, 8, None, 8, p, 8, p, 8, None) == api.CSA_ERR_INVALID_ARG
    assert L.csa_project(1, 1, 8, 8, 8, ctypes.c_void_p(18), 8, p, 8, p, 8, None) == api.CSA_ERR_INVALID_ARG
    assert "aligned" in _err()
    assert L.csa_project(0, 1, 8, 8, 8, p, 8, p, 8, p, 8, None) == api.CSA_ERR_INVALID_ARG
    assert L.csa_project(7, 1, 8, 8, 8, p, 8, p, 8, p, 8, None) == api.CSA_ERR_INVALID_ARG
    assert L.csa_project(1, 1, 8, 8, 8, p, 4, p, 8, p, 8, None) == api.CSA_ERR_INVALID_ARG


def test_project_pair_rejects_bad_args(L):
    p = ctypes.c_void_p(16)

    def call(ind=1, M=8, K=8, X=p, ldx=8, o1=1, N1=8, W1=p, ldw1=8, Y1=p, ldy1=8, o2=1, N2=8, W2=p, ldw2=8, Y2=p,
             ldy2=8):
        return L.csa_project_pair(ind, M, K, X, ldx, o1, N1, W1, ldw1, Y1, ldy1, o2, N2, W2, ldw2, Y2, ldy2, None)

    assert call(N2=0) == api.CSA_ERR_INVALID_ARG
    assert "positive" in _err()
    assert call(K=12, ldx=16, ldw1=16, ldw2=16) == api.CSA_ERR_INVALID_ARG
    assert "multiple of 8" in _err()
    assert call(W2=None) == api.CSA_ERR_INVALID_ARG
    assert call(Y2=ctypes.c_void_p(18)) == api.CSA_ERR_INVALID_ARG
    assert "aligned" in _err()
    assert call(ind=0, o1=0, o2=1) == api.CSA_ERR_INVALID_ARG
    assert call(o2=7) == api.CSA_ERR_INVALID_ARG
    assert call(ldw2=4) == api.CSA_ERR_INVALID_ARG
    assert call(ldy1=4, N1=8) == api.CSA_ERR_INVALID_ARG


def test_compress_rejects_bad_args(L):
    p = ctypes.c_void_p(16)
    assert L.csa_compress(1, 64, 0, 64, p, p, p, p, 256, p, p, p, 64, None) == api.CSA_ERR_INVALID_ARG
    assert L.csa_compress(1, 64, 4, 6, p, p, p, p, 256, p, p, p, 64, None) == api.CSA_ERR_INVALID_ARG
    assert L.csa_compress(1, 64, 4, 64, p, None, p, p, 256, p, p, p, 64, None) == api.CSA_ERR_INVALID_ARG
    assert L.csa_compress(1, 64, 4, 64, p, p, p, p, 60, p, p, p, 64, None) == api.CSA_ERR_INVALID_ARG
    # fewer rows than one block: nothing to do, succeeds without touching pointers or the device
    assert L.csa_compress(1, 3, 4, 64, None, None, None, None, 64, None, None, None, 64, None) == api.CSA_OK


def test_compress_append_rejects_bad_args(L):
    p = ctypes.c_void_p(16)

    def call(dt=1, B=2, m=4, c=64, new=p, ldn=256, ring=p, Ba=p, Bb=p, t=p, off=p, C=p, ldo=64):
        return L.csa_compress_append(dt, B, m, c, new, ldn, ring, Ba, Bb, t, off, C, ldo, None)
    assert call(dt=7) == api.CSA_ERR_INVALID_ARG
    assert call(m=0) == api.CSA_ERR_INVALID_ARG
    assert call(m=65) == api.CSA_ERR_INVALID_ARG
    assert call(c=6) == api.CSA_ERR_INVALID_ARG
    assert call(t=None) == api.CSA_ERR_INVALID_ARG
    assert call(ring=None) == api.CSA_ERR_INVALID_ARG
    assert call(ldn=255) == api.CSA_ERR_INVALID_ARG  # a row of new_rows holds C^a|C^b|Z^a|Z^b: 4c wide
    assert call(ldo=60) == api.CSA_ERR_INVALID_ARG
    assert call(new=ctypes.c_void_p(18)) == api.CSA_ERR_INVALID_ARG
    assert "aligned" in _err()
    assert call(B=0, new=None, ring=None) == api.CSA_OK  # no sequences: nothing enqueued


def test_compress_append_pair_rejects_bad_args(L):
    p = ctypes.c_void_p(16)

    def call(dt=1, B=2, m=4, t=p, off=p, c1=64, new1=p, ldn1=256, ring1=p, C1=p, ldo1=64, c2=32, new2=p, ldn2=128,
             ring2=p, Ba2=p, C2=p, ldo2=32):
        return L.csa_compress_append_pair(dt, B, m, t, off, c1, new1, ldn1, ring1, p, p, C1, ldo1, c2, new2, ldn2,
                                          ring2, Ba2, p, C2, ldo2, None)
    assert call(dt=7) == api.CSA_ERR_INVALID_ARG
    assert call(m=0) == api.CSA_ERR_INVALID_ARG
    assert call(c1=6) == api.CSA_ERR_INVALID_ARG
    assert call(c2=0) == api.CSA_ERR_INVALID_ARG
    assert call(t=None) == api.CSA_ERR_INVALID_ARG
    assert call(ring2=None) == api.CSA_ERR_INVALID_ARG
    assert "cache 2" in _err()
    assert call(Ba2=None) == api.CSA_ERR_INVALID_ARG
    assert call(ldn1=255) == api.CSA_ERR_INVALID_ARG
    assert call(ldo2=31) == api.CSA_ERR_INVALID_ARG
    assert call(new2=ctypes.c_void_p(18)) == api.CSA_ERR_INVALID_ARG
    assert "aligned" in _err()
    assert call(B=0, new1=None, ring2=None) == api.CSA_OK  # no sequences: nothing enqueued


def test_decode_rejects_bad_args(L):
    p = ctypes.c_void_p(16)

    def call(nq=2, q_pos=p, ws=p, wsb=1 << 30, k=64, c=128):
        return L.csa_decode(1, nq, 8, 64, 16, c, 4, k, 0.1, p, p, p, p, p, None, q_pos, None, 1000, p, None, p, None,
                            ws, wsb, None)
    assert call(q_pos=None) == api.CSA_ERR_INVALID_ARG
    assert "q_pos" in _err()
    assert call(k=0) == api.CSA_ERR_INVALID_ARG
    assert call(wsb=10) == api.CSA_ERR_WORKSPACE
    assert call(ws=None) == api.CSA_ERR_WORKSPACE
    assert call(nq=0, q_pos=None) == api.CSA_OK  # empty batch: nothing enqueued
    assert api.csa_decode_workspace(2, 1000, 8, 16, 128, 64) >= api.csa_index_topk_workspace(2, 1000, 8, 64)
    assert api.csa_sparse_mqa_workspace(0, 64, 512, 1024) == 0  # an empty batch needs no workspace


def test_varlen_calls_reject_bad_args(L):
    p = ctypes.c_void_p(16)

    def comp(dt=1, ns=3, m=4, c=64, ld=256, nb=10, cu=p, bo=p, ldo=64):
        return L.csa_compress_varlen(dt, ns, m, c, p, p, p, p, ld, p, p, cu, bo, nb, p, ldo, None)
    assert comp(m=0) == api.CSA_ERR_INVALID_ARG
    assert comp(c=6) == api.CSA_ERR_INVALID_ARG
    assert comp(cu=None) == api.CSA_ERR_INVALID_ARG
    assert comp(ld=60) == api.CSA_ERR_INVALID_ARG
    assert comp(nb=0, cu=None, bo=None) == api.CSA_OK  # no complete block anywhere: nothing to do

    def idx(ns=2, nt=100, nhI=8, cI=64, k=16, cu=p, ws=p, wsb=1 << 30):
        return L.csa_index_topk_varlen(1, ns, nt, nhI, cI, 4, k, p, p, p, cu, p, 30, p, None, None, ws, wsb, None)
    assert idx(cI=96) == api.CSA_ERR_INVALID_ARG
    assert idx(nhI=65) == api.CSA_ERR_INVALID_ARG
    assert idx(cu=None) == api.CSA_ERR_INVALID_ARG
    assert idx(ns=0) == api.CSA_ERR_INVALID_ARG  # tokens without sequences
    assert idx(wsb=8) == api.CSA_ERR_WORKSPACE
    assert idx(nt=0, cu=None) == api.CSA_OK
    assert api.csa_index_topk_varlen_workspace(2, 100, 30, 16) >= 100 * 32 * 4


def test_index_topk_rejects_bad_args(L):
    p = ctypes.c_void_p(16)
    args = dict(dt=1, nq=4, nhI=64, cI=128, m=4, k=16, qI=p, wI=p, K=p, seq=None, pos=None, off=None,
                maxc=100, idx=p, sc=None, ws=p, wsb=1 << 20)

    def call(**over):
        a = dict(args, **over)
        return L.csa_index_topk(a["dt"], a["nq"], a["nhI"], a["cI"], a["m"], a["k"], a["qI"], a["wI"], a["K"],
                                a["seq"], a["pos"], a["off"], a["maxc"], a["idx"], a["sc"], a["ws"], a["wsb"],
                                None)
    assert call(nhI=65) == api.CSA_ERR_INVALID_ARG
    assert call(cI=96) == api.CSA_ERR_INVALID_ARG
    assert call(k=0) == api.CSA_ERR_INVALID_ARG
    assert call(m=0) == api.CSA_ERR_INVALID_ARG
    assert call(qI=None) == api.CSA_ERR_INVALID_ARG
    assert call(wsb=10) == api.CSA_ERR_WORKSPACE
    assert "workspace" in _err()
    assert call(ws=None) == api.CSA_ERR_WORKSPACE
    assert call(nq=0, qI=None) == api.CSA_OK  # empty batch: nothing enqueued


def test_sparse_mqa_rejects_bad_args(L):
    p = ctypes.c_void_p(16)

    def call(dt=1, nq=2, nh=64, c=512, k=1024, scale=0.04, q=p, C=p, idx=p, o=p, ws=p, wsb=1 << 30):
        return L.csa_sparse_mqa(dt, nq, nh, c, k, scale, q, C, None, None, idx, o, None, ws, wsb, None)
    assert call(c=96) == api.CSA_ERR_INVALID_ARG
    assert call(nh=0) == api.CSA_ERR_INVALID_ARG
    assert call(scale=-1.0) == api.CSA_ERR_INVALID_ARG
    assert call(scale=float("nan")) == api.CSA_ERR_INVALID_ARG
    assert call(o=None) == api.CSA_ERR_INVALID_ARG
    assert call(wsb=64) == api.CSA_ERR_WORKSPACE
    # large batches need no workspace: the size query says 0 bytes
    assert api.csa_sparse_mqa_workspace(32768, 64, 512, 512) == 0


def test_workspace_queries(L):
    assert api.csa_index_topk_workspace(8, 32768, 64, 1024) >= 8 * 32768 * 4
    b1 = api.csa_sparse_mqa_workspace(8, 64, 512, 1024)
    b2 = api.csa_sparse_mqa_workspace(16, 64, 512, 1024)
    assert 0 < b1 < b2
    with pytest.raises(api.CSAError):
        api.csa_index_topk_workspace(-1, 10, 4, 4)


def test_timing_interface(L):
    api.csa_timing_reset()
    assert api.csa_timing_read("gemm") == (0.0, 0)
    api.csa_timing_enable(False)


def test_backward_calls_reject_bad_args(L):
    p = ctypes.c_void_p(16)

    def mqa(dt=1, nq=4, nh=64, c=512, k=64, scale=0.05, rows=100, dC=p, ws=p, wsb=1 << 30):
        return L.csa_sparse_mqa_backward(dt, nq, nh, c, k, scale, p, p, rows, None, None, p, p, p, p, p, dC, ws, wsb,
                                         None)
    assert mqa(dt=0) == api.CSA_ERR_UNSUPPORTED  # fp32 attention backward is not built
    assert mqa(c=256) == api.CSA_ERR_INVALID_ARG
    assert "512" in _err()
    assert mqa(nh=0) == api.CSA_ERR_INVALID_ARG
    assert mqa(k=0) == api.CSA_ERR_INVALID_ARG
    assert mqa(scale=0.0) == api.CSA_ERR_INVALID_ARG
    assert mqa(dC=None) == api.CSA_ERR_INVALID_ARG
    assert mqa(wsb=100) == api.CSA_ERR_WORKSPACE
    assert mqa(nq=0, rows=0, ws=None) == api.CSA_OK  # nothing to do
    # the share rows of one pass: at most 2^21 (query, slot) pairs of c bf16 values per head group
    assert api.csa_sparse_mqa_backward_workspace(4096, 64, 512, 512, 8192) >= (1 << 21) * 512 * 2
    assert api.csa_sparse_mqa_backward_workspace(100000, 64, 512, 512, 8192) < (1 << 21) * 512 * 2 + (64 << 20)

    def comp(dt=1, n=64, m=4, c=64, ldi=256, ldd=64, ldo=256, ws=p, wsb=1 << 30):
        return L.csa_compress_backward(dt, n, m, c, p, p, p, p, ldi, p, p, p, ldd, p, p, p, p, ldo, p, p, ws, wsb,
                                       None)
    assert comp(m=0) == api.CSA_ERR_INVALID_ARG
    assert comp(m=17) == api.CSA_ERR_INVALID_ARG  # the bias sums live in LDS: m <= 16
    assert comp(c=6) == api.CSA_ERR_INVALID_ARG
    assert comp(ldi=60) == api.CSA_ERR_INVALID_ARG
    assert comp(ldd=62) == api.CSA_ERR_INVALID_ARG
    assert comp(wsb=8) == api.CSA_ERR_INVALID_ARG
    assert "workspace" in _err()

    def compv(dt=1, ns=3, m=4, c=64, nb=10, cu=p, ldd=64, ws=p, wsb=1 << 30):
        return L.csa_compress_backward_varlen(dt, ns, m, c, p, p, p, p, 256, p, p, cu, p, nb, p, ldd, p, p, p, p, 256,
                                              p, p, ws, wsb, None)
    assert compv(m=17) == api.CSA_ERR_INVALID_ARG
    assert compv(ns=-1) == api.CSA_ERR_INVALID_ARG
    assert compv(ns=0, nb=3) == api.CSA_ERR_INVALID_ARG  # blocks without sequences
    assert compv(cu=None) == api.CSA_ERR_INVALID_ARG
    assert compv(ldd=60) == api.CSA_ERR_INVALID_ARG
    assert compv(wsb=8) == api.CSA_ERR_INVALID_ARG
    assert "workspace" in _err()
    # one partial-sum row of 2m x c fp32 per workgroup row, at least one row even with nothing to do
    assert api.csa_compress_backward_varlen_workspace(0, 0, 4, 64) == 2 * 4 * 64 * 4
    assert api.csa_compress_backward_varlen_workspace(300, 3000, 4, 64) >= 2 * 4 * 64 * 4

    def proj(M=64, N=64, K=64, dX=p, dW=p, ws=p, wsb=1 << 30, ind=1, outd=1):
        return L.csa_project_backward(ind, outd, M, N, K, p, K, p, K, p, N, dX, K, dW, K, ws, wsb, None)
    assert proj(N=60) == api.CSA_ERR_INVALID_ARG
    assert proj(K=12) == api.CSA_ERR_INVALID_ARG
    assert proj(M=0) == api.CSA_ERR_INVALID_ARG  # dW needs tokens
    assert proj(ind=0, outd=1) == api.CSA_ERR_INVALID_ARG  # fp32 in, bf16 out is not a GEMM combination
    assert proj(wsb=16) == api.CSA_ERR_WORKSPACE
    # workspace: W^T for dX, dY^T and X^T (tokens padded to 8) for dW
    assert api.csa_project_backward_workspace(torch_bf16(), 10, 64, 32, True, False) >= 64 * 32 * 2
    assert api.csa_project_backward_workspace(torch_bf16(), 10, 64, 32, False, True) >= (64 + 32) * 16 * 2


def torch_bf16():
    import torch
    return torch.bfloat16
