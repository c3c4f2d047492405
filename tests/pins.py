"""Pins for the CSA oracle: checks against what the page and mathematics fix.

Each ``check_*`` takes the functions under test as arguments (normally the
real oracle's; the mutation tests pass copies with planted mistakes) and
raises AssertionError on a mismatch.  None of them re-types the oracle's
formula: they use hand-derived worked cases (``tests/golden``), closed forms,
invariants stated on the page, a library routine the definition reduces to,
or the independent pure-loop implementation in ``oracle.brute``.

Source for every statement: page "Compressed Sparse Attention (压缩稀疏注意力)".
"""
from __future__ import annotations

import heapq
import json
import math
import os
from types import SimpleNamespace

import numpy as np

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def load_golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def oracle_ns():
    from oracle import csa_oracle as O
    return SimpleNamespace(compress=O.compress, compress_weights=O.compress_weights,
                           index_scores_row=O.index_scores_row, topk=O.topk, mqa=O.mqa,
                           prefill=O.prefill, prefill_rows=O.prefill_rows, decode=O.decode,
                           project=O.project)


# ---------------------------------------------------------------------------
# compression (eqs 3-4 and the block-0 rule)
# ---------------------------------------------------------------------------


def check_compress_golden(ns):
    g = load_golden("compress_m2_c2.json")
    out, S = ns.compress(g["Ca"], g["Cb"], g["Za"], g["Zb"], g["Ba"], g["Bb"], g["m"],
                         return_weights=True)
    np.testing.assert_allclose(out, g["expected_Ccomp"], rtol=0, atol=g["tol"])
    np.testing.assert_allclose(S[1, :, 0], g["expected_weights_block1_ch0"], rtol=0, atol=g["tol"])


def _rand_compress_inputs(rng, n, c, m, scale=1.0):
    return [rng.standard_normal((n, c)) * scale for _ in range(4)] + \
        [rng.standard_normal((m, c)) * 0.3 for _ in range(2)]


def check_compress_constant_rows(ns, rng):
    """All 2m weights of a block sum to 1, so constant value rows are reproduced."""
    n, c, m = 24, 5, 4
    Ca, Cb, Za, Zb, Ba, Bb = _rand_compress_inputs(rng, n, c, m)
    v = rng.standard_normal(c)
    Ca[:] = v
    Cb[:] = v
    out = ns.compress(Ca, Cb, Za, Zb, Ba, Bb, m)
    np.testing.assert_allclose(out, np.broadcast_to(v, out.shape), rtol=0, atol=1e-12)


def check_compress_mean_pool(ns, rng):
    """Equal logits: weights are 1/(2m) (1/m for block 0), i.e. mean pooling.

    Integer values and m a power of two make every sum exact, so the result
    must equal the closed form bit for bit.
    """
    n, c, m = 32, 3, 4
    Ca = rng.integers(-50, 50, size=(n, c)).astype(np.float64)
    Cb = rng.integers(-50, 50, size=(n, c)).astype(np.float64)
    Z = np.full((n, c), 0.75)
    B = np.zeros((m, c))
    out = ns.compress(Ca, Cb, Z, Z, B, B, m)
    N = n // m
    exp = np.empty((N, c))
    for i in range(N):
        a = Ca[m * i:m * i + m].sum(0)
        if i == 0:
            exp[i] = a / m
        else:
            exp[i] = (a + Cb[m * (i - 1):m * i].sum(0)) / (2 * m)
    assert np.array_equal(out, exp), np.abs(out - exp).max()


def check_compress_weights(ns, rng):
    """Each channel's 2m weights sum to 1; block 0's b-weights are exactly 0."""
    n, c, m = 40, 6, 4
    Ca, Cb, Za, Zb, Ba, Bb = _rand_compress_inputs(rng, n, c, m, scale=3.0)
    S = ns.compress_weights(Za, Zb, Ba, Bb, m)
    assert S.shape == (n // m, 2 * m, c)
    np.testing.assert_allclose(S.sum(axis=1), 1.0, rtol=0, atol=1e-12)
    assert np.all(S[0, m:] == 0.0)
    assert np.all(S[1:] > 0.0)


def check_compress_overlap(ns, rng):
    """Row j of C^a/Z^a feeds only block floor(j/m); row j of C^b/Z^b only block floor(j/m)+1.

    This is the overlap the page points out (C^b rows of block i are the C^a
    rows of block i-1), so each token feeds two blocks and N = n/m.
    """
    n, c, m = 24, 4, 4
    base = _rand_compress_inputs(rng, n, c, m)
    ref = ns.compress(*base, m)
    N = n // m
    assert ref.shape == (N, c)
    for which in range(4):  # Ca, Cb, Za, Zb
        for j in (0, 3, 5, 13, n - 1):
            pert = [x.copy() for x in base]
            pert[which][j] += 1.7
            out = ns.compress(*pert, m)
            changed = set(np.nonzero(np.abs(out - ref).max(axis=1) > 0)[0].tolist())
            if which in (0, 2):
                assert changed == {j // m}, (which, j, changed)
            else:
                blk = j // m + 1
                assert changed == ({blk} if blk < N else set()), (which, j, changed)


def check_compress_convex(ns, rng):
    """Each output lies between the min and max of its 2m inputs (convex combination)."""
    n, c, m = 48, 7, 3
    Ca, Cb, Za, Zb, Ba, Bb = _rand_compress_inputs(rng, n, c, m, scale=2.0)
    out = ns.compress(Ca, Cb, Za, Zb, Ba, Bb, m)
    for i in range(n // m):
        vals = Ca[m * i:m * i + m]
        if i > 0:
            vals = np.concatenate([vals, Cb[m * (i - 1):m * i]])
        assert np.all(out[i] >= vals.min(0) - 1e-12) and np.all(out[i] <= vals.max(0) + 1e-12)


def check_compress_no_overlap_limit(ns, rng):
    """Z^b -> -1e30 removes the b-terms: softmax pooling over the m rows of each block.

    The expected value is built with scipy's softmax (a library routine).
    """
    from scipy.special import softmax
    n, c, m = 20, 3, 5
    Ca, Cb, Za, Zb, Ba, Bb = _rand_compress_inputs(rng, n, c, m)
    Zb = np.full((n, c), -1e30)
    out = ns.compress(Ca, Cb, Za, Zb, Ba, Bb, m)
    for i in range(n // m):
        w = softmax(Za[m * i:m * i + m] + Ba, axis=0)
        np.testing.assert_allclose(out[i], (w * Ca[m * i:m * i + m]).sum(0), rtol=1e-12, atol=1e-12)


def check_compress_brute(ns, brute, rng):
    for (n, c, m) in ((12, 3, 1), (13, 5, 2), (27, 3, 4), (30, 1, 3)):
        args = _rand_compress_inputs(rng, n, c, m, scale=2.0)
        out = ns.compress(*args, m)
        exp = np.array(brute.compress(*[a.tolist() for a in args], m)).reshape(out.shape)
        np.testing.assert_allclose(out, exp, rtol=1e-12, atol=1e-12)


# ---------------------------------------------------------------------------
# lightning indexer (eq 8)
# ---------------------------------------------------------------------------


def check_indexer_golden(ns):
    g = load_golden("indexer_nh2_c2.json")
    nc = g["t"] // g["m"]
    s = ns.index_scores_row(g["qI"], g["wI"], g["KIcomp"], nc)
    np.testing.assert_allclose(s, g["expected_scores"], rtol=0, atol=g["tol"])
    assert list(ns.topk(s, g["k"])) == g["expected_topk"]


def check_indexer_nonneg_linear(ns, rng):
    """ReLU makes each head term >= 0, so w >= 0 gives I >= 0; I is linear in w."""
    qI = rng.standard_normal((6, 8))
    K = rng.standard_normal((50, 8))
    w = np.abs(rng.standard_normal(6))
    s = ns.index_scores_row(qI, w, K, 50)
    assert np.all(s >= 0.0)
    assert np.any(s > 0.0)
    s1 = ns.index_scores_row(qI, np.ones(6) * 1.0, K, 50)
    # one head with w = 1 is max(0, q . K): check against a library dot product
    single = ns.index_scores_row(qI[:1], np.ones(1), K, 50)
    np.testing.assert_allclose(single, np.maximum(0.0, np.dot(K, qI[0])), rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(ns.index_scores_row(qI, -2.5 * w, K, 50), -2.5 * s, rtol=1e-12)
    assert s1.shape == (50,)


def check_indexer_causal(ns, rng):
    """Blocks s >= floor(t/m) must not influence I[t, :] (candidates s < floor(t/m))."""
    m = 4
    qI = rng.standard_normal((3, 5))
    w = rng.standard_normal(3)
    K = rng.standard_normal((20, 5))
    for t in (0, 3, 4, 17, 45, 79):
        nc = t // m
        s = ns.index_scores_row(qI, w, K, nc)
        assert s.shape == (nc,)
        K2 = K.copy()
        K2[nc:] = 1e30 * np.sign(rng.standard_normal((20 - nc, 5)))
        np.testing.assert_array_equal(ns.index_scores_row(qI, w, K2, nc), s)


def check_indexer_brute(ns, brute, rng):
    qI = rng.standard_normal((4, 7))
    w = rng.standard_normal(4)
    K = rng.standard_normal((30, 7))
    s = ns.index_scores_row(qI, w, K, 30)
    exp = [brute.index_score(qI.tolist(), w.tolist(), K.tolist(), j) for j in range(30)]
    np.testing.assert_allclose(s, exp, rtol=1e-12, atol=1e-12)


# ---------------------------------------------------------------------------
# top-k (eq 9)
# ---------------------------------------------------------------------------


def check_topk_golden(ns):
    g = load_golden("topk_ties.json")
    for k, exp in g["cases"].items():
        assert list(ns.topk(g["scores"], int(k))) == exp, (k, list(ns.topk(g["scores"], int(k))))


def check_topk_library(ns, rng):
    """Agrees with heapq.nlargest on (score, -index): many exact ties from small integers."""
    for trial in range(30):
        n = int(rng.integers(1, 200))
        k = int(rng.integers(1, 64))
        s = rng.integers(-4, 5, size=n).astype(np.float64)
        s[s == 0] = np.where(rng.random(np.sum(s == 0)) < 0.5, -0.0, 0.0)
        exp = sorted(j for _, j in heapq.nlargest(k, ((float(v) + 0.0, -j) for j, v in enumerate(s))))
        exp = sorted(-j for j in exp)
        assert list(ns.topk(s, k)) == exp


def check_topk_special(ns, rng):
    s = rng.standard_normal(37)
    assert list(ns.topk(s, 37)) == list(range(37))
    assert list(ns.topk(s, 100)) == list(range(37))
    assert list(ns.topk(np.full(40, 2.5), 9)) == list(range(9))
    base = list(ns.topk(s, 11))
    assert list(ns.topk(s * 4.0, 11)) == base  # positive power-of-2 scale leaves the set unchanged
    assert list(ns.topk(np.zeros(0), 5)) == []


def check_topk_brute(ns, brute, rng):
    for _ in range(20):
        n = int(rng.integers(1, 60))
        k = int(rng.integers(1, 20))
        s = rng.integers(-3, 4, size=n).astype(np.float64)
        assert list(ns.topk(s, k)) == brute.topk(s.tolist(), k)


# ---------------------------------------------------------------------------
# shared-KV MQA (eq 11)
# ---------------------------------------------------------------------------


def check_mqa_golden(ns):
    g = load_golden("mqa_c2.json")
    o, lse = ns.mqa(g["q"], g["C_sel"], g["scale"])
    np.testing.assert_allclose(o, g["expected_o"], rtol=0, atol=g["tol"])
    np.testing.assert_allclose(lse, g["expected_lse"], rtol=0, atol=g["tol"])


def check_mqa_sdpa(ns, rng):
    """Key = value = the selected rows: equals torch's scaled-dot-product attention (fp64, CPU)."""
    import torch
    nh, c, ns_ = 5, 16, 23
    q = rng.standard_normal((nh, c))
    C = rng.standard_normal((ns_, c))
    o, lse = ns.mqa(q, C, 1.0 / math.sqrt(c))
    Ct = torch.from_numpy(C)[None, None]
    ref = torch.nn.functional.scaled_dot_product_attention(torch.from_numpy(q)[None, :, None, :],
                                                           Ct, Ct)[0, :, 0, :].numpy()
    np.testing.assert_allclose(o, ref, rtol=1e-10, atol=1e-12)
    from scipy.special import logsumexp
    np.testing.assert_allclose(lse, logsumexp((q @ C.T) / math.sqrt(c), axis=1), rtol=1e-12)


def check_mqa_special(ns, rng):
    nh, c = 3, 8
    C = rng.standard_normal((9, c))
    o, lse = ns.mqa(np.zeros((nh, c)), C, 0.3)  # q = 0: uniform weights -> mean of the rows
    np.testing.assert_allclose(o, np.broadcast_to(C.mean(0), o.shape), rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, math.log(9.0), rtol=1e-12)
    q = rng.standard_normal((nh, c))
    o1, _ = ns.mqa(q, C[4:5], 0.3)  # one row: output is that row
    np.testing.assert_allclose(o1, np.broadcast_to(C[4], o1.shape), rtol=0, atol=1e-12)
    perm = rng.permutation(9)
    o2, l2 = ns.mqa(q, C[perm], 0.3)
    o3, l3 = ns.mqa(q, C, 0.3)
    np.testing.assert_allclose(o2, o3, rtol=1e-12, atol=1e-12)
    o4, l4 = ns.mqa(q[1:2], C, 0.3)  # heads are independent
    np.testing.assert_allclose(o4[0], o3[1], rtol=1e-12, atol=1e-12)
    oe, le = ns.mqa(q, np.zeros((0, c)), 0.3)
    assert np.all(oe == 0) and np.all(np.isneginf(le))


# ---------------------------------------------------------------------------
# whole layer
# ---------------------------------------------------------------------------


def tiny_params(rng, n, d, c, cI, m, dc, nh, nhI):
    P = {"H": rng.standard_normal((n, d))}
    for name in ("W_aKV", "W_bKV", "W_aZ", "W_bZ"):
        P[name] = rng.standard_normal((d, c)) / math.sqrt(d)
    for name in ("W_aKV_I", "W_bKV_I", "W_aZ_I", "W_bZ_I"):
        P[name] = rng.standard_normal((d, cI)) / math.sqrt(d)
    P["B_a"], P["B_b"] = rng.standard_normal((m, c)) * 0.3, rng.standard_normal((m, c)) * 0.3
    P["B_aI"], P["B_bI"] = rng.standard_normal((m, cI)) * 0.3, rng.standard_normal((m, cI)) * 0.3
    P["W_DQ"] = rng.standard_normal((d, dc)) / math.sqrt(d)
    P["W_UQI"] = rng.standard_normal((dc, cI * nhI)) / math.sqrt(dc)
    P["W_w"] = rng.standard_normal((d, nhI)) / math.sqrt(d)
    P["W_UQ"] = rng.standard_normal((dc, c * nh)) / math.sqrt(dc)
    return P


def check_prefill_brute(ns, brute, rng):
    for (n, d, c, cI, m, dc, nh, nhI, k) in ((17, 6, 3, 2, 1, 4, 2, 3, 5),
                                            (26, 5, 5, 3, 2, 3, 3, 2, 4),
                                            (33, 7, 4, 4, 4, 5, 2, 2, 3)):
        P = tiny_params(rng, n, d, c, cI, m, dc, nh, nhI)
        o1 = ns.prefill(P, m, k, nh, nhI)
        o2 = brute.prefill({key: v.tolist() for key, v in P.items()}, m, k, nh, nhI)
        np.testing.assert_allclose(o1["Ccomp"], o2["Ccomp"], rtol=1e-11, atol=1e-12)
        np.testing.assert_allclose(o1["KIcomp"], o2["KIcomp"], rtol=1e-11, atol=1e-12)
        for t in range(n):
            np.testing.assert_allclose(o1["scores"][t], o2["scores"][t], rtol=1e-10, atol=1e-12)
            assert [int(x) for x in o1["idx"][t] if x >= 0] == o2["idx"][t]
            np.testing.assert_allclose(o1["o"][t], np.array(o2["o"][t]), rtol=1e-10, atol=1e-12)
            np.testing.assert_allclose(o1["lse"][t], o2["lse"][t], rtol=1e-10)


def check_prefill_dense_limit(ns, rng):
    """k >= number of blocks: the selection keeps every causal block, so eq 11 becomes
    dense attention over C^Comp with the mask s < floor(t/m); checked against
    torch's scaled-dot-product attention (fp64, CPU, boolean mask)."""
    import torch
    n, d, c, cI, m, dc, nh, nhI = 40, 8, 6, 3, 4, 5, 3, 2
    P = tiny_params(rng, n, d, c, cI, m, dc, nh, nhI)
    out = ns.prefill(P, m, n, nh, nhI)
    N = n // m
    q = torch.from_numpy(out["q"]).permute(1, 0, 2)[None]  # [1, nh, n, c]
    C = torch.from_numpy(out["Ccomp"])[None, None]
    mask = torch.arange(N)[None, :] < (torch.arange(n) // m)[:, None]
    rows = mask.any(1)
    ref = torch.nn.functional.scaled_dot_product_attention(q[:, :, rows], C, C,
                                                           attn_mask=mask[rows])[0]
    np.testing.assert_allclose(out["o"][rows.numpy()], ref.permute(1, 0, 2).numpy(),
                               rtol=1e-10, atol=1e-12)
    assert np.all(out["o"][~rows.numpy()] == 0)  # tokens t < m have no candidates
    assert np.all(np.isneginf(out["lse"][~rows.numpy()]))


def check_decode_matches_prefill_row(ns, rng):
    """A decode query appended after L tokens sees the same candidates as prefill token t = L."""
    n, d, c, cI, m, dc, nh, nhI, k = 37, 6, 4, 3, 4, 5, 2, 3, 4
    P = tiny_params(rng, n, d, c, cI, m, dc, nh, nhI)
    full = ns.prefill(P, m, k, nh, nhI)
    L = 33
    N = L // m
    dec = ns.decode(full["q"][L:L + 1], full["qI"][L:L + 1], full["wI"][L:L + 1],
                    full["Ccomp"][:N], full["KIcomp"][:N], [L], [0], m, k)
    assert list(dec["idx"][0]) == list(full["idx"][L])
    np.testing.assert_allclose(dec["o"][0], full["o"][L], rtol=1e-12, atol=1e-14)
    # with a cache offset: rows of the sequence start at kv_offset
    pad = rng.standard_normal((5, c))
    padI = rng.standard_normal((5, cI))
    dec2 = ns.decode(full["q"][L:L + 1], full["qI"][L:L + 1], full["wI"][L:L + 1],
                     np.concatenate([pad, full["Ccomp"][:N]]),
                     np.concatenate([padI, full["KIcomp"][:N]]), [L], [5], m, k)
    assert list(dec2["idx"][0]) == list(full["idx"][L])
    np.testing.assert_allclose(dec2["o"][0], full["o"][L], rtol=1e-12, atol=1e-14)


def check_rows_match_brute(ns, brute, rng):
    """The sampled-row form of eqs 1-11 (compression over the prefix the rows need, the query side on the
    chosen rows only) equals the pure-loop evaluation of the whole layer on those rows: compressed entries,
    scores, selections, outputs and lse.  Rows include tokens t < m (no candidates), the last token, rows
    given out of order and a repeated row; m in {1, 2, 4}.  The second case has c = c^I and n_h = n_h^I, so
    a swap of the eq 6 and eq 10 up-projections runs without a shape error and must show in the values."""
    for (n, d, c, cI, m, dc, nh, nhI, k, rows) in (
            (21, 5, 3, 2, 1, 4, 2, 3, 4, [20, 0, 7, 13, 7]),
            (30, 6, 4, 4, 2, 5, 2, 2, 3, [1, 29, 0, 17, 4, 16]),
            (37, 7, 5, 3, 4, 4, 3, 2, 3, [3, 2, 36, 35, 12, 19, 8]),
            (9, 4, 3, 3, 4, 3, 2, 2, 2, [0, 3]),  # every row before the first complete block
            (9, 4, 3, 3, 4, 3, 2, 2, 2, [])):
        P = tiny_params(rng, n, d, c, cI, m, dc, nh, nhI)
        got = ns.prefill_rows(P, m, k, nh, nhI, rows)
        ref = brute.prefill({key: v.tolist() for key, v in P.items()}, m, k, nh, nhI)
        N_used = max(rows) // m if rows else 0
        assert got["Ccomp"].shape == (N_used, c) and got["KIcomp"].shape == (N_used, cI)
        np.testing.assert_allclose(got["Ccomp"], np.array(ref["Ccomp"]).reshape(-1, c)[:N_used],
                                   rtol=1e-11, atol=1e-12)
        np.testing.assert_allclose(got["KIcomp"], np.array(ref["KIcomp"]).reshape(-1, cI)[:N_used],
                                   rtol=1e-11, atol=1e-12)
        assert len(got["scores"]) == len(rows) and got["idx"].shape == (len(rows), k)
        for j, t in enumerate(rows):
            assert got["scores"][j].shape == (t // m,)
            np.testing.assert_allclose(got["scores"][j], ref["scores"][t], rtol=1e-10, atol=1e-12)
            assert [int(x) for x in got["idx"][j] if x >= 0] == ref["idx"][t]
            np.testing.assert_allclose(got["o"][j], np.array(ref["o"][t]), rtol=1e-10, atol=1e-12)
            np.testing.assert_allclose(got["lse"][j], ref["lse"][t], rtol=1e-10)


ALL_CHECKS = [
    ("compress_golden", lambda ns, b, r: check_compress_golden(ns)),
    ("compress_constant_rows", lambda ns, b, r: check_compress_constant_rows(ns, r)),
    ("compress_mean_pool", lambda ns, b, r: check_compress_mean_pool(ns, r)),
    ("compress_weights", lambda ns, b, r: check_compress_weights(ns, r)),
    ("compress_overlap", lambda ns, b, r: check_compress_overlap(ns, r)),
    ("compress_convex", lambda ns, b, r: check_compress_convex(ns, r)),
    ("compress_no_overlap_limit", lambda ns, b, r: check_compress_no_overlap_limit(ns, r)),
    ("compress_brute", lambda ns, b, r: check_compress_brute(ns, b, r)),
    ("indexer_golden", lambda ns, b, r: check_indexer_golden(ns)),
    ("indexer_nonneg_linear", lambda ns, b, r: check_indexer_nonneg_linear(ns, r)),
    ("indexer_causal", lambda ns, b, r: check_indexer_causal(ns, r)),
    ("indexer_brute", lambda ns, b, r: check_indexer_brute(ns, b, r)),
    ("topk_golden", lambda ns, b, r: check_topk_golden(ns)),
    ("topk_library", lambda ns, b, r: check_topk_library(ns, r)),
    ("topk_special", lambda ns, b, r: check_topk_special(ns, r)),
    ("topk_brute", lambda ns, b, r: check_topk_brute(ns, b, r)),
    ("mqa_golden", lambda ns, b, r: check_mqa_golden(ns)),
    ("mqa_sdpa", lambda ns, b, r: check_mqa_sdpa(ns, r)),
    ("mqa_special", lambda ns, b, r: check_mqa_special(ns, r)),
    ("prefill_brute", lambda ns, b, r: check_prefill_brute(ns, b, r)),
    ("prefill_dense_limit", lambda ns, b, r: check_prefill_dense_limit(ns, r)),
    ("decode_matches_prefill_row", lambda ns, b, r: check_decode_matches_prefill_row(ns, r)),
    ("rows_match_brute", lambda ns, b, r: check_rows_match_brute(ns, b, r)),
]
