"""Pins for the oracle's gradients (CPU only).

The backward functions are the chain rule of the forward definitions; none of
the checks here re-derives that chain rule.  They use central finite
differences of the (separately pinned) forward oracle, identities that hold
for any differentiable function of the given form (homogeneity, shift
invariance of a softmax), closed forms of special cases, and torch's autograd
through its own scaled-dot-product attention.

Source for every statement: page "Compressed Sparse Attention (压缩稀疏注意力)",
eqs 1-4 (projections and compression) and eq 11 (the core attention).
"""
from __future__ import annotations

import math
from types import SimpleNamespace

import numpy as np


def backward_ns():
    from oracle import csa_oracle as O
    return SimpleNamespace(compress=O.compress, mqa=O.mqa, project=O.project, prefill=O.prefill,
                           compress_backward=O.compress_backward, mqa_backward=O.mqa_backward,
                           sparse_mqa_backward=O.sparse_mqa_backward, project_backward=O.project_backward,
                           prefill_backward=O.prefill_backward)


def _fd_grad(loss, args, which, h=1e-5):
    """Central differences of loss(*args) w.r.t. args[which] (every element)."""
    x = np.array(args[which], dtype=np.float64)
    g = np.zeros_like(x)
    flat, gflat = x.reshape(-1), g.reshape(-1)
    for i in range(flat.size):
        keep = flat[i]
        a = list(args)
        flat[i] = keep + h
        a[which] = x.copy()
        up = loss(*a)
        flat[i] = keep - h
        a[which] = x.copy()
        dn = loss(*a)
        flat[i] = keep
        gflat[i] = (up - dn) / (2 * h)
    return g


def _close(got, want, what):
    np.testing.assert_allclose(got, want, rtol=1e-6, atol=1e-8, err_msg=what)


# ---------------------------------------------------------------------------
# compression, eqs 3-4 (block 0 sees only its own a-rows)
# ---------------------------------------------------------------------------


def _compress_inputs(rng, n, c, m):
    return [rng.standard_normal((n, c)) for _ in range(4)] + [rng.standard_normal((m, c)) * 0.5
                                                              for _ in range(2)]


def check_compress_backward_fd(ns, rng):
    """Every input's gradient equals central differences of sum(dC * compress(...)); n = 11 with
    m = 3 covers block 0, interior blocks and a ragged tail of two rows."""
    n, c, m = 11, 2, 3
    args = _compress_inputs(rng, n, c, m)
    dC = rng.standard_normal((n // m, c))

    def loss(*a):
        return float((dC * ns.compress(*a, m)).sum())

    grads = ns.compress_backward(*args, m, dC)
    for w, name in enumerate(["Ca", "Cb", "Za", "Zb", "Ba", "Bb"]):
        _close(grads[w], _fd_grad(loss, args, w), f"d{name}")


def check_compress_backward_identities(ns, rng):
    """Homogeneity in the values, shift invariance of the softmax, and the mean-pool closed form."""
    n, c, m = 26, 3, 4
    N = n // m
    Ca, Cb, Za, Zb, Ba, Bb = _compress_inputs(rng, n, c, m)
    dC = rng.standard_normal((N, c))
    out = ns.compress(Ca, Cb, Za, Zb, Ba, Bb, m)
    dCa, dCb, dZa, dZb, dBa, dBb = ns.compress_backward(Ca, Cb, Za, Zb, Ba, Bb, m, dC)
    # the output is 1-homogeneous in the values (Ca, Cb) jointly
    _close((dCa * Ca).sum() + (dCb * Cb).sum(), (dC * out).sum(), "Euler identity")
    # adding one constant to every logit of every block changes nothing: the logit
    # gradients (through Z and through B alike) sum to zero per channel
    _close(dZa.sum(0) + dZb.sum(0), np.zeros(c), "shift invariance (Z)")
    _close(dBa.sum(0) + dBb.sum(0), np.zeros(c), "shift invariance (B)")
    # the biases add to every block's logits, so their gradients are the per-position sums of Z's
    _close(dBa, dZa[: N * m].reshape(N, m, c).sum(0), "dBa = sum over blocks of dZa")
    _close(dBb, dZb[: N * m].reshape(N, m, c).sum(0), "dBb = sum over blocks of dZb")
    # rows with no complete block, and the b-rows of the last block, get nothing
    assert np.all(dCa[N * m:] == 0) and np.all(dZa[N * m:] == 0)
    assert np.all(dCb[(N - 1) * m:] == 0) and np.all(dZb[(N - 1) * m:] == 0)
    # equal logits: mean pooling, value gradient dC/(2m) (dC/m for block 0's a-rows)
    Z = np.zeros((n, c))
    B = np.zeros((m, c))
    g = ns.compress_backward(Ca, Cb, Z, Z, B, B, m, dC)
    want_a = np.repeat(dC, m, axis=0) / (2 * m)
    want_a[:m] *= 2
    _close(g[0][: N * m], want_a, "mean-pool dCa")
    _close(g[1][: (N - 1) * m], np.repeat(dC[1:], m, axis=0) / (2 * m), "mean-pool dCb")
    # constant values: the output does not depend on the logits at all
    v = rng.standard_normal(c)
    g = ns.compress_backward(np.broadcast_to(v, (n, c)), np.broadcast_to(v, (n, c)), Za, Zb, Ba, Bb, m, dC)
    for t in g[2:]:
        np.testing.assert_allclose(t, 0.0, atol=1e-12)
    # fewer rows than one block: all gradients zero
    g = ns.compress_backward(Ca[:m - 1], Cb[:m - 1], Za[:m - 1], Zb[:m - 1], Ba, Bb, m, np.zeros((0, c)))
    assert all(np.all(t == 0) for t in g) and g[0].shape == (m - 1, c) and g[4].shape == (m, c)


# ---------------------------------------------------------------------------
# core attention, eq 11
# ---------------------------------------------------------------------------


def check_mqa_backward_fd(ns, rng):
    nh, c, k = 3, 4, 5
    q = rng.standard_normal((nh, c))
    C = rng.standard_normal((k, c))
    dO = rng.standard_normal((nh, c))
    scale = 0.7

    def loss(q_, C_):
        return float((dO * ns.mqa(q_, C_, scale)[0]).sum())

    dq, dCs = ns.mqa_backward(q, C, scale, dO)
    _close(dq, _fd_grad(loss, [q, C], 0), "dq")
    _close(dCs, _fd_grad(loss, [q, C], 1), "dC_sel")


def check_mqa_backward_sdpa(ns, rng):
    """torch autograd through scaled_dot_product_attention with key = value = the selected rows."""
    import torch
    nh, c, k = 4, 16, 19
    q = rng.standard_normal((nh, c))
    C = rng.standard_normal((k, c))
    dO = rng.standard_normal((nh, c))
    scale = 1.0 / math.sqrt(c)
    qt = torch.from_numpy(q.copy())[None, :, None, :].requires_grad_()
    Kt = torch.from_numpy(C.copy())[None, None].requires_grad_()
    Vt = torch.from_numpy(C.copy())[None, None].requires_grad_()
    o = torch.nn.functional.scaled_dot_product_attention(qt, Kt, Vt, scale=scale)
    o.backward(torch.from_numpy(dO)[None, :, None, :])
    dq, dCs = ns.mqa_backward(q, C, scale, dO)
    np.testing.assert_allclose(dq, qt.grad[0, :, 0].numpy(), rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(dCs, (Kt.grad + Vt.grad)[0, 0].numpy(), rtol=1e-10, atol=1e-12)


def check_mqa_backward_special(ns, rng):
    nh, c = 3, 6
    q = rng.standard_normal((nh, c))
    dO = rng.standard_normal((nh, c))
    C = rng.standard_normal((7, c))
    # one selected row: the output is that row whatever q is
    dq, dC1 = ns.mqa_backward(q, C[2:3], 0.4, dO)
    np.testing.assert_allclose(dq, 0.0, atol=1e-12)
    np.testing.assert_allclose(dC1, dO.sum(0, keepdims=True), rtol=1e-12, atol=1e-12)
    # scale 0: uniform weights, output the mean row
    dq, dC0 = ns.mqa_backward(q, C, 0.0, dO)
    np.testing.assert_allclose(dq, 0.0, atol=1e-12)
    np.testing.assert_allclose(dC0, np.broadcast_to(dO.sum(0) / 7, C.shape), rtol=1e-12, atol=1e-12)
    # o(q / l, l C) = l o(q, C): d/dl at l = 1 gives <dC, C> - <dq, q> = <dO, o>
    dq, dC = ns.mqa_backward(q, C, 0.4, dO)
    o, _ = ns.mqa(q, C, 0.4)
    _close((dC * C).sum() - (dq * q).sum(), (dO * o).sum(), "scaling identity")
    # heads are independent: a head's gradient depends only on its own dO row
    dq1, dC1 = ns.mqa_backward(q[1:2], C, 0.4, dO[1:2])
    dO_only1 = np.zeros_like(dO)
    dO_only1[1] = dO[1]
    dqa, dCa = ns.mqa_backward(q, C, 0.4, dO_only1)
    _close(dqa[1], dq1[0], "dq of one head")
    _close(dCa, dC1, "dC of one head")
    # an empty selection contributes nothing
    dqe, dCe = ns.mqa_backward(q, np.zeros((0, c)), 0.4, dO)
    assert np.all(dqe == 0) and dCe.shape == (0, c)


def check_sparse_mqa_backward(ns, rng):
    """A batch with shared, repeated-across-queries and padded (-1) selections: the gradient of
    each compressed row collects every query's share (central differences of the batch loss)."""
    n, nh, c, rows = 4, 2, 3, 6
    q = rng.standard_normal((n, nh, c))
    Cc = rng.standard_normal((rows, c))
    dO = rng.standard_normal((n, nh, c))
    idx = np.array([[0, 1, -1], [0, 2, 1], [-1, -1, -1], [1, 0, 3]])
    off = np.array([0, 0, 2, 2])
    scale = 0.6

    def loss(q_, C_):
        tot = 0.0
        for r in range(n):
            sel = idx[r][idx[r] >= 0]
            tot += float((dO[r] * ns.mqa(q_[r], C_[off[r] + sel], scale)[0]).sum())
        return tot

    dq, dC = ns.sparse_mqa_backward(q, Cc, idx, off, scale, dO)
    _close(dq, _fd_grad(loss, [q, Cc], 0), "dq")
    _close(dC, _fd_grad(loss, [q, Cc], 1), "dCcomp")
    assert np.all(dq[2] == 0) and np.all(dC[4] == 0)  # query 2 selects nothing; row 4 is never selected


# ---------------------------------------------------------------------------
# projections, eqs 1, 2, 5, 6, 7, 10
# ---------------------------------------------------------------------------


def check_project_backward(ns, rng):
    X = rng.standard_normal((5, 4))
    W = rng.standard_normal((4, 3))
    dY = rng.standard_normal((5, 3))

    def loss(X_, W_):
        return float((dY * ns.project(X_, W_)).sum())

    dX, dW = ns.project_backward(X, W, dY)
    _close(dX, _fd_grad(loss, [X, W], 0), "dX")
    _close(dW, _fd_grad(loss, [X, W], 1), "dW")
    # bilinear: <dY, XW> = <dX, X> = <dW, W>
    s = (dY * ns.project(X, W)).sum()
    _close((dX * X).sum(), s, "bilinear (X)")
    _close((dW * W).sum(), s, "bilinear (W)")


# ---------------------------------------------------------------------------
# whole layer: the composed gradient against central differences of the prefill
# ---------------------------------------------------------------------------


def check_prefill_backward_fd(ns, rng):
    """Every parameter that reaches the output, perturbed element by element; the selection must not
    move under the perturbation (it is piecewise constant), which the check verifies."""
    from pins import tiny_params
    n, d, c, cI, m, dc, nh, nhI, k = 13, 4, 3, 2, 2, 3, 2, 2, 3
    P = tiny_params(rng, n, d, c, cI, m, dc, nh, nhI)
    dO = rng.standard_normal((n, nh, c))
    base = ns.prefill(P, m, k, nh, nhI)
    g = ns.prefill_backward(P, m, k, nh, nhI, dO)

    def loss_for(name):
        def loss(x):
            Q = dict(P)
            Q[name] = x
            out = ns.prefill(Q, m, k, nh, nhI)
            assert np.array_equal(out["idx"], base["idx"]), "selection moved under the perturbation"
            return float((dO * out["o"]).sum())
        return loss

    for name in ("H", "W_aKV", "W_bKV", "W_aZ", "W_bZ", "B_a", "B_b", "W_DQ", "W_UQ"):
        fd = _fd_grad(lambda x: loss_for(name)(x), [P[name]], 0, h=1e-6)
        np.testing.assert_allclose(g[name], fd, rtol=1e-5, atol=1e-7, err_msg=name)
    # the indexer's parameters do not reach the output (the selection is piecewise constant)
    for name in ("W_UQI", "W_w", "W_aKV_I"):
        fd = _fd_grad(lambda x: loss_for(name)(x), [P[name]], 0, h=1e-6)
        np.testing.assert_allclose(fd, 0.0, atol=1e-7, err_msg=name)


ALL_BACKWARD_CHECKS = [
    ("compress_backward_fd", check_compress_backward_fd),
    ("compress_backward_identities", check_compress_backward_identities),
    ("mqa_backward_fd", check_mqa_backward_fd),
    ("mqa_backward_sdpa", check_mqa_backward_sdpa),
    ("mqa_backward_special", check_mqa_backward_special),
    ("sparse_mqa_backward", check_sparse_mqa_backward),
    ("project_backward", check_project_backward),
    ("prefill_backward_fd", check_prefill_backward_fd),
]
