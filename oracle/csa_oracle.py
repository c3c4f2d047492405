"""CSA oracle: a plain, slow, float64 NumPy evaluation of the CSA definition.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or
execute this module: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code, constant or
helper with the HIP implementation and imports nothing from it.

Source: the web page "Compressed Sparse Attention (压缩稀疏注意力)" (cnblogs),
sections "Compressed Key-Value Entries" (eqs 1-4), "Lightning Indexer for
Sparse Selection" (eqs 5-9) and "Shared Key-Value MQA" (eqs 10-11).

Every input is widened to float64 (bf16 and fp32 values convert exactly) and
every step is evaluated in float64.  Readings taken where the page is silent
(each is also declared in the design notes):

* softmax of eq 3 runs independently per channel over the 2m stacked logits
  (the only reading under which S_j is a c-vector, as eq 4's Hadamard product
  needs);
* only floor(n/m) complete blocks are compressed;
* block 0 uses the page's padding literally: its Z^b logits are -inf and its
  C^b values are 0, so the b-weights are exactly 0;
* the indexer keys use their own parameter set of the same shape as the main
  one ("the same compression operation"), and W^UQ of eq 6 (indexer) and of
  eq 10 (attention) are two different matrices;
* head h of a projected query takes columns [h*dim, (h+1)*dim);
* token t (0-based) may select blocks s < floor(t/m); a decode query appended
  after L context tokens is token t = L, so all floor(L/m) blocks are
  candidates;
* eq 9 keeps exactly min(k, number of candidates) blocks; equal scores are
  ordered by lower block index (-0.0 equals +0.0);
* CoreAttn of eq 11 is softmax(scale * q K^T) V with K = V = the selected
  compressed entries and scale = 1/sqrt(c) unless given; an empty selection
  gives o = 0 and lse = -inf.

Backward functions (gradients of eqs 1-4 and 11 for training; the top-k of
eq 9 passes no gradient, and the indexer's training objective is not on the
page) are the chain rule of the forward definitions written out, pinned by
central finite differences.

Parity status: every function here is pinned by the CPU tests (closed forms,
invariants, brute force and a library routine); there is no trained-model
value to compare with, so absolute behaviour on trained weights is
"parity unpinned".
"""
from __future__ import annotations

import math
from typing import Dict, List, Optional, Sequence, Tuple

import numpy as np

__all__ = [
    "project", "compress", "compress_weights", "n_candidates", "index_scores",
    "index_scores_row", "topk", "topk_rows", "mqa", "prefill", "prefill_rows",
    "decode", "project_backward", "compress_backward", "mqa_backward", "sparse_mqa_backward",
    "prefill_backward",
]


def _f64(x) -> np.ndarray:
    return np.asarray(x, dtype=np.float64)


# ---------------------------------------------------------------------------
# eqs 1, 2, 5, 6, 7, 10: linear projections
# ---------------------------------------------------------------------------


def project(X, W) -> np.ndarray:
    """Row-vector projection Y = X . W (eqs 1, 2, 5, 6, 7 and 10 all have this form)."""
    return _f64(X) @ _f64(W)


# ---------------------------------------------------------------------------
# eqs 3, 4: softmax-gated overlapping compression
# ---------------------------------------------------------------------------


def compress_weights(Za, Zb, Ba, Bb, m: int) -> np.ndarray:
    """Eq 3: the 2m softmax weights of every block and channel.

    Returns S with shape [N, 2m, c], N = floor(n/m).  S[i, r] for r < m is the
    weight of row m*i + r of C^a; S[i, m + r] is the weight of row m*(i-1) + r
    of C^b.  For block 0 the b-logits are padded with -inf (page's rule).
    """
    Za, Zb, Ba, Bb = _f64(Za), _f64(Zb), _f64(Ba), _f64(Bb)
    n, c = Za.shape
    N = n // m
    if N == 0:
        return np.zeros((0, 2 * m, c))
    la = Za[: N * m].reshape(N, m, c) + Ba[None]  # block i: rows m*i .. m*i+m-1
    lb = np.full((N, m, c), -np.inf)
    if N > 1:
        lb[1:] = Zb[: (N - 1) * m].reshape(N - 1, m, c) + Bb[None]  # block i: rows m*(i-1) ..
    lam = np.concatenate([la, lb], axis=1)  # [N, 2m, c]
    mx = lam.max(axis=1, keepdims=True)  # finite: the a-logits always are
    e = np.exp(lam - mx)
    return e / e.sum(axis=1, keepdims=True)


def compress(Ca, Cb, Za, Zb, Ba, Bb, m: int, return_weights: bool = False):
    """Eqs 3-4: C^Comp[i] = sum_r S^a_r (.) C^a_{mi+r} + sum_r S^b_r (.) C^b_{m(i-1)+r}.

    Inputs are [n, c] (Ca, Cb, Za, Zb) and [m, c] (Ba, Bb).  Block 0's C^b rows
    are zeros (page's padding rule).  Output [floor(n/m), c].
    """
    Ca, Cb = _f64(Ca), _f64(Cb)
    n, c = Ca.shape
    N = n // m
    S = compress_weights(Za, Zb, Ba, Bb, m)
    va = Ca[: N * m].reshape(N, m, c)
    vb = np.zeros((N, m, c))
    if N > 1:
        vb[1:] = Cb[: (N - 1) * m].reshape(N - 1, m, c)
    vals = np.concatenate([va, vb], axis=1)  # [N, 2m, c]
    out = (S * vals).sum(axis=1)
    if return_weights:
        return out, S
    return out


# ---------------------------------------------------------------------------
# eq 8: lightning indexer
# ---------------------------------------------------------------------------


def n_candidates(t, m: int):
    """Number of compressed blocks token t may select: floor(t/m) (blocks s < floor(t/m))."""
    return np.asarray(t, dtype=np.int64) // m


def index_scores_row(qI_t, wI_t, KIcomp, n_cand: int) -> np.ndarray:
    """Eq 8 for one query: I[s] = sum_h w[h] * ReLU(q^I[h] . K^IComp[s]), s < n_cand.

    qI_t [n_hI, cI], wI_t [n_hI], KIcomp [>= n_cand, cI] -> [n_cand].
    """
    q = _f64(qI_t)
    w = _f64(wI_t)
    K = _f64(KIcomp)[:n_cand]
    dots = q @ K.T  # [n_hI, n_cand]: per-head q^I_{t,h} . K^IComp_s
    return w @ np.maximum(dots, 0.0)


def index_scores(qI, wI, KIcomp, n_cand: Sequence[int]) -> List[np.ndarray]:
    """Eq 8 for a list of queries; row r has n_cand[r] candidates."""
    return [index_scores_row(qI[r], wI[r], KIcomp, int(n_cand[r])) for r in range(len(n_cand))]


# ---------------------------------------------------------------------------
# eq 9: top-k selector
# ---------------------------------------------------------------------------


def topk(scores, k: int) -> np.ndarray:
    """Eq 9: indices of the min(k, len) largest scores, ties to the lower index.

    Sorting key: score descending, then index ascending (NumPy compares -0.0
    and +0.0 as equal).  Returned in ascending index order.
    """
    s = _f64(scores)
    n = s.shape[0]
    order = np.lexsort((np.arange(n), -s))
    return np.sort(order[: min(k, n)])


def topk_rows(score_rows: Sequence[np.ndarray], k: int) -> np.ndarray:
    """Eq 9 per row, padded with -1 to width k."""
    out = np.full((len(score_rows), k), -1, dtype=np.int64)
    for r, s in enumerate(score_rows):
        sel = topk(s, k)
        out[r, : sel.shape[0]] = sel
    return out


# ---------------------------------------------------------------------------
# eq 11: shared-KV multi-query attention
# ---------------------------------------------------------------------------


def mqa(q_t, C_sel, scale: float) -> Tuple[np.ndarray, np.ndarray]:
    """Eq 11 for one query token: each selected entry is both key and value.

    q_t [n_h, c], C_sel [k_sel, c] -> (o [n_h, c], lse [n_h]), where
    o[i] = softmax(scale * q_t[i] . C_sel^T) . C_sel and lse is the natural
    log of the softmax denominator (including the running max).
    """
    q = _f64(q_t)
    C = _f64(C_sel)
    nh, c = q.shape
    if C.shape[0] == 0:
        return np.zeros((nh, c)), np.full(nh, -np.inf)
    logits = scale * (q @ C.T)  # [n_h, k_sel]
    mx = logits.max(axis=1, keepdims=True)
    p = np.exp(logits - mx)
    den = p.sum(axis=1, keepdims=True)
    o = (p / den) @ C
    lse = (mx + np.log(den))[:, 0]
    return o, lse


def _mqa_rows(q, Ccomp, idx, row_offset, scale):
    n = q.shape[0]
    nh, c = q.shape[1], q.shape[2]
    o = np.zeros((n, nh, c))
    lse = np.full((n, nh), -np.inf)
    for r in range(n):
        sel = idx[r]
        sel = sel[sel >= 0]
        o[r], lse[r] = mqa(q[r], _f64(Ccomp)[int(row_offset[r]) + sel], scale)
    return o, lse


# ---------------------------------------------------------------------------
# whole layer
# ---------------------------------------------------------------------------


def default_scale(c: int) -> float:
    return 1.0 / math.sqrt(c)


def prefill(P: Dict[str, np.ndarray], m: int, k: int, n_h: int, n_hI: int,
            scale: Optional[float] = None) -> Dict[str, np.ndarray]:
    """Eqs 1-11 for one sequence; every token t is a query.

    P holds H [n, d] and the parameters named W_aKV, W_bKV, W_aZ, W_bZ, B_a,
    B_b (main compression), W_aKV_I, W_bKV_I, W_aZ_I, W_bZ_I, B_aI, B_bI
    (indexer-key compression), W_DQ, W_UQI (eq 6), W_w (eq 7), W_UQ (eq 10).
    """
    H = _f64(P["H"])
    n = H.shape[0]
    Ca, Cb = project(H, P["W_aKV"]), project(H, P["W_bKV"])  # eq 1
    Za, Zb = project(H, P["W_aZ"]), project(H, P["W_bZ"])  # eq 2
    Ccomp = compress(Ca, Cb, Za, Zb, P["B_a"], P["B_b"], m)  # eqs 3-4
    KIcomp = compress(project(H, P["W_aKV_I"]), project(H, P["W_bKV_I"]),
                      project(H, P["W_aZ_I"]), project(H, P["W_bZ_I"]),
                      P["B_aI"], P["B_bI"], m)  # same operation, indexer keys
    cQ = project(H, P["W_DQ"])  # eq 5
    cI = KIcomp.shape[1]
    qI = project(cQ, P["W_UQI"]).reshape(n, n_hI, cI)  # eq 6
    wI = project(H, P["W_w"])  # eq 7
    c = Ccomp.shape[1]
    q = project(cQ, P["W_UQ"]).reshape(n, n_h, c)  # eq 10
    ncand = n_candidates(np.arange(n), m)
    scores = index_scores(qI, wI, KIcomp, ncand)  # eq 8
    idx = topk_rows(scores, k)  # eq 9
    sc = default_scale(c) if scale is None else scale
    o, lse = _mqa_rows(q, Ccomp, idx, np.zeros(n, np.int64), sc)  # eq 11
    return {"Ccomp": Ccomp, "KIcomp": KIcomp, "cQ": cQ, "qI": qI, "wI": wI, "q": q,
            "scores": scores, "idx": idx, "o": o, "lse": lse}


def prefill_rows(P: Dict[str, np.ndarray], m: int, k: int, n_h: int, n_hI: int,
                 rows: Sequence[int], scale: Optional[float] = None) -> Dict[str, np.ndarray]:
    """Eqs 1-11 for selected query tokens of one sequence.

    Compression needs every hidden state (all blocks are candidates of late
    tokens), the query side only the selected rows.  Same readings as
    ``prefill``; used where the whole layer is too large for the CPU.
    """
    H = _f64(P["H"])
    n = H.shape[0]
    rows = np.asarray(rows, dtype=np.int64)
    n_used = (int(rows.max()) // m) * m if rows.size else 0
    Hc = H[:n_used]
    Ccomp = compress(project(Hc, P["W_aKV"]), project(Hc, P["W_bKV"]),
                     project(Hc, P["W_aZ"]), project(Hc, P["W_bZ"]), P["B_a"], P["B_b"], m)
    KIcomp = compress(project(Hc, P["W_aKV_I"]), project(Hc, P["W_bKV_I"]),
                      project(Hc, P["W_aZ_I"]), project(Hc, P["W_bZ_I"]), P["B_aI"], P["B_bI"], m)
    Hr = H[rows]
    cQ = project(Hr, P["W_DQ"])
    cI = _f64(P["B_aI"]).shape[1]
    c = _f64(P["B_a"]).shape[1]
    qI = project(cQ, P["W_UQI"]).reshape(len(rows), n_hI, cI)
    wI = project(Hr, P["W_w"])
    q = project(cQ, P["W_UQ"]).reshape(len(rows), n_h, c)
    ncand = n_candidates(rows, m)
    scores = index_scores(qI, wI, KIcomp, ncand)
    idx = topk_rows(scores, k)
    sc = default_scale(c) if scale is None else scale
    o, lse = _mqa_rows(q, Ccomp, idx, np.zeros(len(rows), np.int64), sc)
    return {"Ccomp": Ccomp, "KIcomp": KIcomp, "qI": qI, "wI": wI, "q": q,
            "scores": scores, "idx": idx, "o": o, "lse": lse}


def decode(q, qI, wI, Ccomp, KIcomp, seq_len, kv_offset, m: int, k: int,
           scale: Optional[float] = None, seqs: Optional[Sequence[int]] = None
           ) -> Dict[str, object]:
    """Eqs 8, 9, 11 for one query per sequence, appended after seq_len[b] tokens.

    Sequence b's compressed entries are rows kv_offset[b] .. kv_offset[b] +
    floor(seq_len[b]/m) - 1 of the shared cache buffers; all of them are
    candidates.  ``seqs`` restricts the work to some sequences.
    """
    seq_len = np.asarray(seq_len, dtype=np.int64)
    kv_offset = np.asarray(kv_offset, dtype=np.int64)
    B = seq_len.shape[0]
    seqs = list(range(B)) if seqs is None else list(seqs)
    c = q.shape[2]
    sc = default_scale(c) if scale is None else scale
    scores, idx, o, lse = [], [], [], []
    for b in seqs:
        nc = int(n_candidates(seq_len[b], m))
        off = int(kv_offset[b])
        s = index_scores_row(qI[b], wI[b], _f64(KIcomp)[off: off + nc], nc)
        sel = topk(s, k)
        ob, lb = mqa(q[b], _f64(Ccomp)[off + sel], sc)
        row = np.full(k, -1, dtype=np.int64)
        row[: sel.shape[0]] = sel
        scores.append(s)
        idx.append(row)
        o.append(ob)
        lse.append(lb)
    return {"scores": scores, "idx": np.stack(idx), "o": np.stack(o), "lse": np.stack(lse),
            "seqs": seqs}


# ---------------------------------------------------------------------------
# backward (gradients of a scalar loss whose gradient w.r.t. the outputs is given)
# ---------------------------------------------------------------------------


def project_backward(X, W, dY) -> Tuple[np.ndarray, np.ndarray]:
    """Eqs 1, 2, 5, 6, 7, 10 (Y = X W): dX = dY W^T, dW = X^T dY."""
    X, W, dY = _f64(X), _f64(W), _f64(dY)
    return dY @ W.T, X.T @ dY


def compress_backward(Ca, Cb, Za, Zb, Ba, Bb, m: int, dCcomp):
    """Gradients of eqs 3-4 given dCcomp [floor(n/m), c].

    For block i and channel ch, with weights S_j (the per-channel softmax of
    eq 3 over the 2m stacked logits) and values v_j (the C^a and C^b rows),
    out = sum_j S_j v_j; then dv_j = S_j * dout and the logit gradient is
    dlogit_j = S_j * dout * (v_j - out).  Each projected row is an a-row of one
    block and a b-row of the next, so its gradients come from one block each;
    B^a and B^b collect dlogit over all blocks.  Rows past the last complete
    block, and the b-rows of the last block, get zero gradient.
    Returns (dCa, dCb, dZa, dZb) [n, c] and (dBa, dBb) [m, c].
    """
    Ca, Cb, dC = _f64(Ca), _f64(Cb), _f64(dCcomp)
    n, c = Ca.shape
    N = n // m
    out, S = compress(Ca, Cb, Za, Zb, Ba, Bb, m, return_weights=True)
    grads = [np.zeros((n, c)) for _ in range(4)]
    dBa, dBb = np.zeros((m, c)), np.zeros((m, c))
    if N == 0:
        return (*grads, dBa, dBb)
    va = Ca[: N * m].reshape(N, m, c)
    vb = np.zeros((N, m, c))
    if N > 1:
        vb[1:] = Cb[: (N - 1) * m].reshape(N - 1, m, c)
    vals = np.concatenate([va, vb], axis=1)  # [N, 2m, c]
    dv = S * dC[:, None, :]
    dl = S * dC[:, None, :] * (vals - out[:, None, :])
    dCa, dCb, dZa, dZb = grads
    dCa[: N * m] = dv[:, :m].reshape(N * m, c)
    dZa[: N * m] = dl[:, :m].reshape(N * m, c)
    if N > 1:
        dCb[: (N - 1) * m] = dv[1:, m:].reshape((N - 1) * m, c)
        dZb[: (N - 1) * m] = dl[1:, m:].reshape((N - 1) * m, c)
    dBa = dl[:, :m].sum(axis=0)
    dBb = dl[1:, m:].sum(axis=0) if N > 1 else dBb
    return dCa, dCb, dZa, dZb, dBa, dBb


def mqa_backward(q_t, C_sel, scale: float, dO_t) -> Tuple[np.ndarray, np.ndarray]:
    """Gradients of eq 11 for one query token: (dq [n_h, c], dC_sel [k_sel, c]).

    With P = softmax(scale q C^T) (per head), o = P C and the selected entries
    serving as both keys and values: dP = dO C^T, D = rowsum(dO * o),
    dS = P * (dP - D), dq = scale dS C, dC = P^T dO + scale dS^T q.
    """
    q, C, dO = _f64(q_t), _f64(C_sel), _f64(dO_t)
    if C.shape[0] == 0:
        return np.zeros_like(q), np.zeros((0, q.shape[1]))
    logits = scale * (q @ C.T)
    P = np.exp(logits - logits.max(axis=1, keepdims=True))
    P /= P.sum(axis=1, keepdims=True)
    o = P @ C
    dP = dO @ C.T
    D = (dO * o).sum(axis=1, keepdims=True)
    dS = P * (dP - D)
    return scale * dS @ C, P.T @ dO + scale * dS.T @ q


def sparse_mqa_backward(q, Ccomp, idx, row_offset, scale: float, dO) -> Tuple[np.ndarray, np.ndarray]:
    """Gradients of eq 11 over a batch: dq [n, n_h, c] and dCcomp [rows, c], where
    every selection of a compressed row (by any query) adds its share."""
    q, dO, Cc = _f64(q), _f64(dO), _f64(Ccomp)
    dq = np.zeros_like(q)
    dC = np.zeros_like(Cc)
    for r in range(q.shape[0]):
        sel = np.asarray(idx[r])
        sel = sel[sel >= 0]
        rows = int(row_offset[r]) + sel
        dq[r], dc = mqa_backward(q[r], Cc[rows], scale, dO[r])
        np.add.at(dC, rows, dc)
    return dq, dC


def prefill_backward(P: Dict[str, np.ndarray], m: int, k: int, n_h: int, n_hI: int, dO,
                     scale: Optional[float] = None) -> Dict[str, np.ndarray]:
    """Gradients of sum(dO * o) for the prefill of ``prefill`` (eqs 1-11).

    The selection of eq 9 is piecewise constant in every input, so no
    gradient flows through eqs 6-9 (the indexer's own training objective is
    not part of the method as described): the indexer weights get none, and
    H collects the gradients of eqs 1-2 (through compression, eqs 3-4) and of
    eq 5 (through the attention queries, eq 10).  Returns dH, the gradients of
    W_aKV, W_bKV, W_aZ, W_bZ, B_a, B_b, W_DQ and W_UQ, plus dq and dCcomp.
    """
    H = _f64(P["H"])
    n = H.shape[0]
    fwd = prefill(P, m, k, n_h, n_hI, scale)
    c = fwd["Ccomp"].shape[1]
    sc = default_scale(c) if scale is None else scale
    dq, dCcomp = sparse_mqa_backward(fwd["q"], fwd["Ccomp"], fwd["idx"], np.zeros(n, np.int64), sc, dO)
    proj = {name: project(H, P[name]) for name in ("W_aKV", "W_bKV", "W_aZ", "W_bZ")}
    dCa, dCb, dZa, dZb, dBa, dBb = compress_backward(proj["W_aKV"], proj["W_bKV"], proj["W_aZ"], proj["W_bZ"],
                                                     P["B_a"], P["B_b"], m, dCcomp)
    dcQ, dW_UQ = project_backward(fwd["cQ"], P["W_UQ"], dq.reshape(n, n_h * c))
    g = {"dq": dq, "dCcomp": dCcomp, "B_a": dBa, "B_b": dBb, "W_UQ": dW_UQ}
    dH = np.zeros_like(H)
    for name, dY in (("W_aKV", dCa), ("W_bKV", dCb), ("W_aZ", dZa), ("W_bZ", dZb), ("W_DQ", dcQ)):
        dX, dW = project_backward(H, P[name], dY)
        dH += dX
        g[name] = dW
    g["H"] = dH
    return g

