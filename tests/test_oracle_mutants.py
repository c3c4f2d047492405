"""Plant plausible mistakes in copies of the oracle and show the pins catch each.

Every mutant below is a wrong reading or a slip one could make while writing
the oracle from the page "Compressed Sparse Attention": a dropped term, a
wrong index, a wrong axis, a wrong sign or operand order.  The test passes
only if at least one pin fails for every mutant, i.e. the pins would have
caught that mistake in the real oracle.  Mutants live here, on the CPU.
"""
import zlib
from types import SimpleNamespace

import numpy as np
import pytest

from oracle import brute, csa_oracle as O
from pins import ALL_CHECKS, oracle_ns


def _ns(**over):
    ns = oracle_ns()
    d = dict(vars(ns))
    d.update(over)
    return SimpleNamespace(**d)


def _compress_with(weights_fn, value_shift=1):
    """compress() rebuilt around a (possibly mutated) weight function / b-row shift."""
    def compress(Ca, Cb, Za, Zb, Ba, Bb, m, return_weights=False):
        Ca, Cb = np.asarray(Ca, float), np.asarray(Cb, float)
        n, c = Ca.shape
        N = n // m
        S = weights_fn(Za, Zb, Ba, Bb, m)
        va = Ca[:N * m].reshape(N, m, c)
        vb = np.zeros((N, m, c))
        for i in range(1, N):
            lo = m * (i - value_shift)
            vb[i] = Cb[lo:lo + m] if lo + m <= n else 0.0
        out = (S * np.concatenate([va, vb], 1)).sum(1)
        return (out, S) if return_weights else out
    return compress


def _weights_wrong_axis(Za, Zb, Ba, Bb, m):  # softmax over channels instead of the 2m rows
    S = O.compress_weights(Za, Zb, Ba, Bb, m)
    lam = np.log(np.maximum(S, 1e-300))
    e = np.exp(lam - lam.max(2, keepdims=True))
    return e / e.sum(2, keepdims=True)


def _weights_swapped_bias(Za, Zb, Ba, Bb, m):
    return O.compress_weights(Za, Zb, Bb, Ba, m)


def _weights_reversed_bias(Za, Zb, Ba, Bb, m):  # bias rows applied in reverse position order
    return O.compress_weights(Za, Zb, np.asarray(Ba)[::-1], np.asarray(Bb)[::-1], m)


def _weights_no_b(Za, Zb, Ba, Bb, m):  # b-terms dropped from the softmax
    return O.compress_weights(Za, np.full(np.shape(Zb), -np.inf), Ba, Bb, m)


def _weights_block0_zero_logit(Za, Zb, Ba, Bb, m):  # block 0 padded with logit 0, not -inf
    S = O.compress_weights(Za, Zb, Ba, Bb, m)
    Za, Ba = np.asarray(Za, float), np.asarray(Ba, float)
    la = Za[:m] + Ba
    lam = np.concatenate([la, np.zeros_like(la)], 0)
    e = np.exp(lam - lam.max(0))
    S = S.copy()
    S[0] = e / e.sum(0)
    return S


def _index_relu_after_sum(qI, wI, K, nc):
    q, w, K = np.asarray(qI, float), np.asarray(wI, float), np.asarray(K, float)[:nc]
    return np.maximum(w @ (q @ K.T), 0.0)


def _index_no_weight(qI, wI, K, nc):
    return O.index_scores_row(qI, np.ones(np.shape(wI)), K, nc)


def _index_off_by_one(qI, wI, K, nc):
    return O.index_scores_row(qI, wI, K, nc + 1)


def _index_abs(qI, wI, K, nc):
    q, w, K = np.asarray(qI, float), np.asarray(wI, float), np.asarray(K, float)[:nc]
    return w @ np.abs(q @ K.T)


def _topk_high_index_ties(s, k):
    s = np.asarray(s, float)
    n = s.shape[0]
    order = np.lexsort((-np.arange(n), -s))
    return np.sort(order[:min(k, n)])


def _topk_smallest(s, k):
    s = np.asarray(s, float)
    n = s.shape[0]
    order = np.lexsort((np.arange(n), s))
    return np.sort(order[:min(k, n)])


def _topk_signed_zero(s, k):  # -0.0 ranked below +0.0
    s = np.asarray(s, float)
    n = s.shape[0]
    key = s - np.signbit(s) * (s == 0) * 1e-300
    order = np.lexsort((np.arange(n), -key))
    return np.sort(order[:min(k, n)])


def _mqa_no_scale(q, C, scale):
    return O.mqa(q, C, 1.0)


def _mqa_head_softmax(q, C, scale):  # softmax across heads instead of across keys
    q, C = np.asarray(q, float), np.asarray(C, float)
    if C.shape[0] == 0:
        return O.mqa(q, C, scale)
    lg = scale * (q @ C.T)
    p = np.exp(lg - lg.max(0, keepdims=True))
    p = p / p.sum(0, keepdims=True)
    return p @ C, O.mqa(q, C, scale)[1]


def _mqa_lse_no_max(q, C, scale):
    o, lse = O.mqa(q, C, scale)
    q, C = np.asarray(q, float), np.asarray(C, float)
    if C.shape[0] == 0:
        return o, lse
    lg = scale * (q @ C.T)
    return o, np.log(np.exp(lg - lg.max(1, keepdims=True)).sum(1))


def _rows_variant(prefix_blocks=lambda rows, m: int(max(rows)) // m if len(rows) else 0,
                  swap_uq=False, query_row_shift=0, positions_from_order=False):
    """prefill_rows rebuilt from the oracle's parts with one planted slip (the defaults give the correct
    function): the prefix of blocks compressed, eq 6 / eq 10 up-projections swapped, the query side read
    from the wrong hidden-state rows, or candidate counts taken from the rows' order instead of their
    token positions."""
    def prefill_rows(P, m, k, n_h, n_hI, rows, scale=None):
        H = np.asarray(P["H"], float)
        rows = np.asarray(rows, dtype=np.int64)
        Hc = H[:prefix_blocks(rows, m) * m]
        proj = lambda X, names: [O.project(X, P[nm]) for nm in names]  # noqa: E731
        Ccomp = O.compress(*proj(Hc, ("W_aKV", "W_bKV", "W_aZ", "W_bZ")), P["B_a"], P["B_b"], m)
        KIcomp = O.compress(*proj(Hc, ("W_aKV_I", "W_bKV_I", "W_aZ_I", "W_bZ_I")), P["B_aI"], P["B_bI"], m)
        Hr = H[np.clip(rows + query_row_shift, 0, H.shape[0] - 1)]
        cQ = O.project(Hr, P["W_DQ"])
        cI, c = np.shape(P["B_aI"])[1], np.shape(P["B_a"])[1]
        wUQI, wUQ = (P["W_UQ"], P["W_UQI"]) if swap_uq else (P["W_UQI"], P["W_UQ"])
        qI = O.project(cQ, wUQI).reshape(len(rows), n_hI, cI)
        wI = O.project(Hr, P["W_w"])
        q = O.project(cQ, wUQ).reshape(len(rows), n_h, c)
        ncand = O.n_candidates(np.arange(len(rows)) if positions_from_order else rows, m)
        scores = O.index_scores(qI, wI, KIcomp, ncand)
        idx = O.topk_rows(scores, k)
        o, lse = O._mqa_rows(q, Ccomp, idx, np.zeros(len(rows), np.int64),
                             O.default_scale(c) if scale is None else scale)
        return {"Ccomp": Ccomp, "KIcomp": KIcomp, "qI": qI, "wI": wI, "q": q, "scores": scores,
                "idx": idx, "o": o, "lse": lse}
    return prefill_rows


MUTANTS = {
    "compress_wrong_axis": dict(compress=_compress_with(_weights_wrong_axis),
                                compress_weights=_weights_wrong_axis),
    "compress_swapped_bias": dict(compress=_compress_with(_weights_swapped_bias),
                                  compress_weights=_weights_swapped_bias),
    "compress_reversed_bias": dict(compress=_compress_with(_weights_reversed_bias),
                                   compress_weights=_weights_reversed_bias),
    "compress_no_b_terms": dict(compress=_compress_with(_weights_no_b),
                                compress_weights=_weights_no_b),
    "compress_b_rows_same_block": dict(compress=_compress_with(O.compress_weights, value_shift=0)),
    "compress_block0_zero_logit": dict(compress=_compress_with(_weights_block0_zero_logit),
                                       compress_weights=_weights_block0_zero_logit),
    "index_relu_after_sum": dict(index_scores_row=_index_relu_after_sum),
    "index_no_weight": dict(index_scores_row=_index_no_weight),
    "index_off_by_one": dict(index_scores_row=_index_off_by_one),
    "index_abs": dict(index_scores_row=_index_abs),
    "topk_high_index_ties": dict(topk=_topk_high_index_ties),
    "topk_smallest": dict(topk=_topk_smallest),
    "topk_signed_zero": dict(topk=_topk_signed_zero),
    "mqa_no_scale": dict(mqa=_mqa_no_scale),
    "mqa_head_softmax": dict(mqa=_mqa_head_softmax),
    "mqa_lse_no_max": dict(mqa=_mqa_lse_no_max),
    "rows_prefix_one_block_short": dict(prefill_rows=_rows_variant(
        prefix_blocks=lambda rows, m: max(int(max(rows)) // m - 1, 0) if len(rows) else 0)),
    "rows_prefix_whole_rows": dict(prefill_rows=_rows_variant(
        prefix_blocks=lambda rows, m: (int(max(rows)) + 1) // m if len(rows) else 0)),
    "rows_swapped_up_projections": dict(prefill_rows=_rows_variant(swap_uq=True)),
    "rows_query_from_previous_token": dict(prefill_rows=_rows_variant(query_row_shift=-1)),
    "rows_positions_from_order": dict(prefill_rows=_rows_variant(positions_from_order=True)),
}

# checks that exercise only a single function; the whole-layer checks call
# the real module's composites and so cannot see a mutant of a part
_PART_CHECKS = [(n, c) for n, c in ALL_CHECKS if not n.startswith(("prefill", "decode"))]


def test_rows_variant_without_slip_passes():
    """The rebuilt prefill_rows with no planted slip passes the pin, so the mutants above fail it for
    their slip alone."""
    from pins import check_rows_match_brute
    check_rows_match_brute(_ns(prefill_rows=_rows_variant()), brute, np.random.Generator(np.random.PCG64(5)))


@pytest.mark.parametrize("mutant", sorted(MUTANTS))
def test_pins_catch(mutant):
    ns = _ns(**MUTANTS[mutant])
    caught = []
    for name, check in _PART_CHECKS:
        rng = np.random.Generator(np.random.PCG64(zlib.crc32(name.encode())))
        try:
            check(ns, brute, rng)
        except (AssertionError, ValueError, IndexError):
            caught.append(name)
    assert caught, f"no pin catches mutant {mutant}"
