"""The oracle's gradients against their pins, and planted mistakes that the pins must catch.

Every mutant is a slip one could make in the chain rule of eqs 3-4 and 11 of
"Compressed Sparse Attention": a dropped term, a wrong sign, a b-row gradient
sent to the wrong block, a missing accumulation over queries.
"""
import zlib
from types import SimpleNamespace

import numpy as np
import pytest

from oracle import csa_oracle as O
from pins_backward import ALL_BACKWARD_CHECKS, backward_ns


def _rng(name):
    return np.random.Generator(np.random.PCG64(zlib.crc32(name.encode())))


@pytest.mark.parametrize("name,check", ALL_BACKWARD_CHECKS, ids=[n for n, _ in ALL_BACKWARD_CHECKS])
def test_backward_pin(name, check):
    check(backward_ns(), _rng(name))


def _mqa_bwd(drop_D=False, drop_q_term=False, sign=1.0):
    def f(q_t, C_sel, scale, dO_t):
        q, C, dO = (np.asarray(x, float) for x in (q_t, C_sel, dO_t))
        if C.shape[0] == 0:
            return np.zeros_like(q), np.zeros((0, q.shape[1]))
        lg = scale * (q @ C.T)
        P = np.exp(lg - lg.max(1, keepdims=True))
        P /= P.sum(1, keepdims=True)
        o = P @ C
        D = 0.0 if drop_D else (dO * o).sum(1, keepdims=True)
        dS = sign * P * (dO @ C.T - D)
        dC = P.T @ dO + (0.0 if drop_q_term else scale * dS.T @ q)
        return scale * dS @ C, dC
    return f


def _compress_bwd(mutate):
    def f(Ca, Cb, Za, Zb, Ba, Bb, m, dCcomp):
        g = list(O.compress_backward(Ca, Cb, Za, Zb, Ba, Bb, m, dCcomp))
        Ca_, Cb_, dC = (np.asarray(x, float) for x in (Ca, Cb, dCcomp))
        n, c = Ca_.shape
        N = n // m
        out, S = O.compress(Ca, Cb, Za, Zb, Ba, Bb, m, return_weights=True)
        if mutate == "b_rows_same_block":  # b-row gradient of block i sent to rows of block i
            dCb = np.zeros((n, c))
            dCb[: N * m] = (S * dC[:, None, :])[:, m:].reshape(N * m, c)
            g[1] = dCb
        elif mutate == "logit_sign":  # (out - v) in place of (v - out)
            g[2], g[3], g[4], g[5] = -g[2], -g[3], -g[4], -g[5]
        elif mutate == "logit_no_center":  # dlogit = S * dC * v (the softmax's own term dropped)
            va = Ca_[: N * m].reshape(N, m, c)
            dl = S[:, :m] * dC[:, None, :] * va
            g[2] = np.zeros((n, c))
            g[2][: N * m] = dl.reshape(N * m, c)
            g[4] = dl.sum(0)
        elif mutate == "bias_mean":  # bias gradient averaged over blocks
            g[4], g[5] = g[4] / max(N, 1), g[5] / max(N - 1, 1)
        return tuple(g)
    return f


def _sparse_overwrite(q, Ccomp, idx, row_offset, scale, dO):  # last query's share wins
    dq = np.zeros_like(np.asarray(q, float))
    dC = np.zeros_like(np.asarray(Ccomp, float))
    for r in range(dq.shape[0]):
        sel = np.asarray(idx[r])
        sel = sel[sel >= 0]
        rows = int(row_offset[r]) + sel
        dq[r], dC[rows] = O.mqa_backward(q[r], np.asarray(Ccomp, float)[rows], scale, dO[r])
    return dq, dC


def _project_token_mean(X, W, dY):  # weight gradient averaged over tokens instead of summed
    dX, dW = O.project_backward(X, W, dY)
    return dX, dW / np.shape(X)[0]


def _prefill_no_query_weight(P, m, k, nh, nhI, dO, scale=None):  # W_DQ's gradient dropped
    g = dict(O.prefill_backward(P, m, k, nh, nhI, dO, scale))
    g["W_DQ"] = np.zeros_like(g["W_DQ"])
    return g


MUTANTS = {
    "mqa_drop_D": dict(mqa_backward=_mqa_bwd(drop_D=True)),
    "mqa_drop_q_term": dict(mqa_backward=_mqa_bwd(drop_q_term=True)),
    "mqa_sign": dict(mqa_backward=_mqa_bwd(sign=-1.0)),
    "compress_b_rows_same_block": dict(compress_backward=_compress_bwd("b_rows_same_block")),
    "compress_logit_sign": dict(compress_backward=_compress_bwd("logit_sign")),
    "compress_logit_no_center": dict(compress_backward=_compress_bwd("logit_no_center")),
    "compress_bias_mean": dict(compress_backward=_compress_bwd("bias_mean")),
    "sparse_overwrite": dict(sparse_mqa_backward=_sparse_overwrite),
    "project_token_mean": dict(project_backward=_project_token_mean),
    "prefill_no_query_weight": dict(prefill_backward=_prefill_no_query_weight),
}


@pytest.mark.parametrize("mutant", sorted(MUTANTS))
def test_backward_pins_catch(mutant):
    d = dict(vars(backward_ns()))
    if "mqa_backward" in MUTANTS[mutant]:  # the batch form is built on the per-query one
        mb = MUTANTS[mutant]["mqa_backward"]

        def sparse(q, Ccomp, idx, row_offset, scale, dO):
            dq = np.zeros_like(np.asarray(q, float))
            dC = np.zeros_like(np.asarray(Ccomp, float))
            for r in range(dq.shape[0]):
                sel = np.asarray(idx[r])
                rows = int(row_offset[r]) + sel[sel >= 0]
                dq[r], dc = mb(q[r], np.asarray(Ccomp, float)[rows], scale, dO[r])
                np.add.at(dC, rows, dc)
            return dq, dC
        d["sparse_mqa_backward"] = sparse
    d.update(MUTANTS[mutant])
    ns = SimpleNamespace(**d)
    caught = []
    for name, check in ALL_BACKWARD_CHECKS:
        try:
            check(ns, _rng(name))
        except (AssertionError, ValueError, IndexError):
            caught.append(name)
    assert caught, f"no pin catches mutant {mutant}"
