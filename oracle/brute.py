"""Brute-force CSA in pure Python loops (no NumPy), for tiny inputs only.

TEST INFRASTRUCTURE ONLY (same rule as ``csa_oracle``).  It restates the
page "Compressed Sparse Attention (压缩稀疏注意力)", eqs 1-11, as scalar loops
over Python floats (IEEE double) and exists to pin the vectorised oracle:
a different code shape for the same definition, written without reshapes,
broadcasting or library sorting.

Inputs are nested lists (or anything indexable as ``x[i][j]``) of floats.
Readings are the same as in ``csa_oracle``; block 0 is handled here by
leaving its b-terms out of the sum, which is what -inf logits and zero values
contribute, so the two formulations check each other.
"""
from __future__ import annotations

import math


def matmul(X, W):
    rows, inner, cols = len(X), len(W), len(W[0])
    out = []
    for i in range(rows):
        r = []
        for j in range(cols):
            acc = 0.0
            for t in range(inner):
                acc += float(X[i][t]) * float(W[t][j])
            r.append(acc)
        out.append(r)
    return out


def compress(Ca, Cb, Za, Zb, Ba, Bb, m):
    n, c = len(Ca), len(Ca[0])
    out = []
    for i in range(n // m):
        row = []
        for j in range(c):
            logits, vals = [], []
            for r in range(m):
                logits.append(float(Za[m * i + r][j]) + float(Ba[r][j]))
                vals.append(float(Ca[m * i + r][j]))
            if i > 0:
                for r in range(m):
                    logits.append(float(Zb[m * (i - 1) + r][j]) + float(Bb[r][j]))
                    vals.append(float(Cb[m * (i - 1) + r][j]))
            top = max(logits)
            ws = [math.exp(x - top) for x in logits]
            tot = sum(ws)
            acc = 0.0
            for wgt, v in zip(ws, vals):
                acc += (wgt / tot) * v
            row.append(acc)
        out.append(row)
    return out


def index_score(qI_t, wI_t, K, s):
    total = 0.0
    for h in range(len(qI_t)):
        dot = 0.0
        for j in range(len(K[s])):
            dot += float(qI_t[h][j]) * float(K[s][j])
        total += float(wI_t[h]) * (dot if dot > 0.0 else 0.0)
    return total


def topk(scores, k):
    """Repeatedly take the best remaining candidate (largest score, then lowest index)."""
    remaining = list(range(len(scores)))
    chosen = []
    while remaining and len(chosen) < k:
        best = remaining[0]
        for s in remaining[1:]:
            if scores[s] > scores[best]:
                best = s
        chosen.append(best)
        remaining.remove(best)
    return sorted(chosen)


def attention(q_t, rows, scale):
    """One query token, all heads: softmax(scale * q . K^T) V with K = V = rows."""
    out, lses = [], []
    for qh in q_t:
        if not rows:
            out.append([0.0] * len(qh))
            lses.append(-math.inf)
            continue
        logits = []
        for r in rows:
            dot = 0.0
            for a, b in zip(qh, r):
                dot += float(a) * float(b)
            logits.append(scale * dot)
        top = max(logits)
        ws = [math.exp(x - top) for x in logits]
        tot = sum(ws)
        o = [0.0] * len(qh)
        for wgt, r in zip(ws, rows):
            for j in range(len(o)):
                o[j] += wgt / tot * float(r[j])
        out.append(o)
        lses.append(top + math.log(tot))
    return out, lses


def prefill(P, m, k, n_h, n_hI, scale=None):
    H = P["H"]
    n = len(H)
    C = compress(matmul(H, P["W_aKV"]), matmul(H, P["W_bKV"]), matmul(H, P["W_aZ"]),
                 matmul(H, P["W_bZ"]), P["B_a"], P["B_b"], m)
    K = compress(matmul(H, P["W_aKV_I"]), matmul(H, P["W_bKV_I"]), matmul(H, P["W_aZ_I"]),
                 matmul(H, P["W_bZ_I"]), P["B_aI"], P["B_bI"], m)
    cQ = matmul(H, P["W_DQ"])
    qI_flat = matmul(cQ, P["W_UQI"])
    wI = matmul(H, P["W_w"])
    q_flat = matmul(cQ, P["W_UQ"])
    c = len(P["B_a"][0])
    cI = len(P["B_aI"][0])
    sc = 1.0 / math.sqrt(c) if scale is None else scale
    idx_all, o_all, lse_all, scores_all = [], [], [], []
    for t in range(n):
        qI_t = [qI_flat[t][h * cI:(h + 1) * cI] for h in range(n_hI)]
        q_t = [q_flat[t][h * c:(h + 1) * c] for h in range(n_h)]
        nc = t // m
        scores = [index_score(qI_t, wI[t], K, s) for s in range(nc)]
        sel = topk(scores, k)
        o, lse = attention(q_t, [C[s] for s in sel], sc)
        idx_all.append(sel)
        o_all.append(o)
        lse_all.append(lse)
        scores_all.append(scores)
    return {"Ccomp": C, "KIcomp": K, "scores": scores_all, "idx": idx_all, "o": o_all,
            "lse": lse_all}
