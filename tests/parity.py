"""Comparison rules shared by the GPU parity tests.

* Floating outputs (compressed entries, projections, attention outputs) are
  compared per row: max_j |gpu - ref| / max_j |ref| <= 2e-2 (fp32
  accumulation, bf16 storage).  Rows whose reference is all zero must be
  within 1e-6 absolutely.
* Gradients that are sums over tokens (weight gradients X^T dY) are
  compared against the size of their terms: max_j |gpu - ref| <= 2e-2 *
  max_j (|X|^T |dY|) per row, since cancellation between tokens can make a
  row's maximum far smaller than the bf16 rounding of the terms it sums.
* dq of the attention backward: the library forms D = dO . o from the
  stored (bf16) forward output, which moves dq by up to
  scale |dO|_2 |o - o_bf16|_2 max|o| <= scale |dO|_2 2^-8 |o|_2 max|o|
  per head; that bound is added to the row tolerance.
* Top-k index sets: with tau the reference's k-th largest score of a row and
  eps = 1e-3 |tau| + 1e-6 max|score|, the GPU set G must hold every
  candidate scoring above tau + eps and nothing scoring below tau - eps;
  |G| = min(k, n_cand), entries distinct and in range, other slots -1.
  Rows with n_cand <= k must hold exactly all candidates.
"""
from __future__ import annotations

import numpy as np
import torch

ROW_TOL = 2e-2
TOPK_REL = 1e-3


def to_np64(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def row_maxrel(gpu: np.ndarray, ref: np.ndarray) -> np.ndarray:
    g = gpu.reshape(-1, gpu.shape[-1])
    r = ref.reshape(-1, ref.shape[-1])
    den = np.abs(r).max(axis=1)
    err = np.abs(g - r).max(axis=1)
    out = np.where(den > 0, err / np.where(den > 0, den, 1.0), err)
    return out


def assert_rows_close(gpu, ref, tol=ROW_TOL, what=""):
    gpu = np.asarray(gpu, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert gpu.shape == ref.shape, (what, gpu.shape, ref.shape)
    assert np.all(np.isfinite(gpu)), f"{what}: non-finite GPU output"
    rel = row_maxrel(gpu, ref)
    zero_rows = np.abs(ref.reshape(-1, ref.shape[-1])).max(axis=1) == 0
    bad = np.where(zero_rows, rel > 1e-6, rel > tol)
    worst = int(np.argmax(rel)) if rel.size else -1
    assert not bad.any(), (f"{what}: {int(bad.sum())} of {bad.size} rows exceed {tol}; "
                           f"worst row {worst} rel {rel[worst]:.3e}")
    return float(rel.max()) if rel.size else 0.0


def assert_sum_rows_close(gpu, ref, term_scale, tol=ROW_TOL, what=""):
    """Rows of a sum over tokens: error within tol of the row's largest |X|^T |dY| entry."""
    gpu = np.asarray(gpu, dtype=np.float64).reshape(-1, np.shape(gpu)[-1])
    ref = np.asarray(ref, dtype=np.float64).reshape(gpu.shape)
    scale = np.asarray(term_scale, dtype=np.float64).reshape(gpu.shape).max(axis=1)
    assert np.all(np.isfinite(gpu)), f"{what}: non-finite GPU output"
    rel = np.abs(gpu - ref).max(axis=1) / np.where(scale > 0, scale, 1.0)
    worst = int(np.argmax(rel))
    assert np.all(rel <= tol), f"{what}: worst row {worst} rel {rel[worst]:.3e} of its term scale"
    return float(rel.max())


def assert_dq_close(gpu, ref, dO, o, scale, tol=ROW_TOL, what="dq"):
    """dq rows [.., heads, c]: row tolerance plus the bound of the stored-output rounding (see above)."""
    gpu = np.asarray(gpu, dtype=np.float64).reshape(-1, np.shape(gpu)[-1])
    ref = np.asarray(ref, dtype=np.float64).reshape(gpu.shape)
    dO = np.asarray(dO, dtype=np.float64).reshape(gpu.shape)
    o = np.asarray(o, dtype=np.float64).reshape(gpu.shape)
    assert np.all(np.isfinite(gpu)), f"{what}: non-finite GPU output"
    extra = scale * np.linalg.norm(dO, axis=1) * 2.0 ** -8 * np.linalg.norm(o, axis=1) * np.abs(o).max(axis=1)
    err = np.abs(gpu - ref).max(axis=1)
    allowed = tol * np.abs(ref).max(axis=1) + extra + 1e-7
    worst = int(np.argmax(err / allowed))
    assert np.all(err <= allowed), f"{what}: row {worst} off by {err[worst]:.3e} (allowed {allowed[worst]:.3e})"
    return float((err / allowed).max())


def check_topk_row(sel_row: np.ndarray, scores: np.ndarray, k: int, rel: float = TOPK_REL):
    """Returns the number of band-exempt differences from the exact reference set."""
    nc = scores.shape[0]
    sel_row = np.asarray(sel_row)
    valid = sel_row[sel_row >= 0]
    want = min(k, nc)
    assert valid.shape[0] == want, f"row holds {valid.shape[0]} indices, expected {want}"
    assert np.all(sel_row[sel_row < 0] == -1)
    assert np.unique(valid).shape[0] == want, "duplicate indices"
    assert valid.min(initial=0) >= 0 and valid.max(initial=-1) < nc, "index out of range"
    if nc <= k:
        assert set(valid.tolist()) == set(range(nc))
        return 0
    tau = np.sort(scores)[::-1][k - 1]
    eps = rel * abs(tau) + 1e-6 * np.abs(scores).max()
    G = set(valid.tolist())
    must = set(np.nonzero(scores > tau + eps)[0].tolist())
    allowed = set(np.nonzero(scores >= tau - eps)[0].tolist())
    assert must <= G, f"missing {sorted(must - G)[:8]} (tau {tau})"
    assert G <= allowed, f"unexpected {sorted(G - allowed)[:8]} (tau {tau})"
    order = np.lexsort((np.arange(nc), -scores))
    exact = set(order[:k].tolist())
    return len(exact - G)


def check_topk(sel: np.ndarray, score_rows, k: int, rel: float = TOPK_REL):
    swaps = 0
    for r, s in enumerate(score_rows):
        try:
            swaps += check_topk_row(sel[r], np.asarray(s, dtype=np.float64), k, rel)
        except AssertionError as e:
            raise AssertionError(f"row {r}: {e}") from None
    return swaps


def exact_sets_equal(sel: np.ndarray, ref_idx: np.ndarray):
    for r in range(sel.shape[0]):
        a = sorted(int(x) for x in sel[r] if x >= 0)
        b = sorted(int(x) for x in ref_idx[r] if x >= 0)
        assert a == b, f"row {r}: {a[:10]} != {b[:10]}"
