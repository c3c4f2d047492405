"""Seeded synthetic inputs for the CSA hot path.

This module is shared by the tests, the benchmark and the oracle-side checks.
It draws random tensors and stores them; it contains none of the CSA
arithmetic (no projection, compression, scoring, selection or attention).

Storage conventions
-------------------
* fp32 tensors are ``numpy.float32`` arrays.
* bf16 tensors are ``numpy.uint16`` arrays holding the bf16 bit patterns,
  obtained from an fp32 draw by round-to-nearest-even.  ``bf16_to_f32`` /
  ``bf16_to_f64`` widen them exactly.

Distributions (the workload descriptions write ``N(0, x)``; the readings
below are the ones the whole project uses):
* weight matrices ``N(0, 1/fan_in)``: variance ``1/fan_in``;
* positional biases ``B^a, B^b ~ N(0, 0.1)``: standard deviation ``0.1``;
* queries ``N(0, 1/sqrt(dim))``: standard deviation ``dim**-0.5``, so
  ``q . K`` has unit variance for unit-variance keys;
* hidden states, caches and indexer head weights ``N(0, 1)``.

Generator: ``numpy.random.Generator(PCG64(seed))``; default seed is the
workload number.  Tensors are drawn in the order the workload lists them,
then the ones it leaves implicit, in equation order.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Dict, Optional

import numpy as np

# ---------------------------------------------------------------------------
# bf16 storage helpers (bit conversion only)
# ---------------------------------------------------------------------------


def f32_to_bf16(x) -> np.ndarray:
    """Round fp32 values to bf16 (round to nearest, ties to even); returns uint16 bits."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    r = (u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_to_f32(b) -> np.ndarray:
    """Widen bf16 bit patterns (uint16) to fp32 exactly."""
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


def bf16_to_f64(b) -> np.ndarray:
    return bf16_to_f32(b).astype(np.float64)


def to_f64(x, dtype: str) -> np.ndarray:
    """Exact widening of a stored tensor (fp32 array or bf16 bits) to float64."""
    if dtype == "bf16":
        return bf16_to_f64(x)
    return np.asarray(x, dtype=np.float32).astype(np.float64)


# ---------------------------------------------------------------------------
# workloads
# ---------------------------------------------------------------------------


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    kind: str  # "prefill" | "decode"
    dtype: str  # "f32" | "bf16"
    m: int
    c: int
    cI: int
    nhI: int
    nh: int
    k: int
    # prefill
    n: int = 0
    d: int = 0
    dc: int = 0
    # decode
    B: int = 0
    L: int = 0  # fixed context length (0 -> ragged)
    Lmin: int = 0
    Lmax: int = 0


WORKLOADS: Dict[int, Workload] = {
    1: Workload("prefill_n512_fp32", "prefill", "f32", m=4, c=64, cI=32, nhI=4, nh=8, k=16,
                n=512, d=256, dc=128),
    2: Workload("decode_b32_ctx8k_bf16", "decode", "bf16", m=4, c=512, cI=128, nhI=64, nh=64,
                k=512, B=32, L=8192),
    3: Workload("prefill_n32768_bf16", "prefill", "bf16", m=4, c=512, cI=128, nhI=64, nh=64,
                k=512, n=32768, d=4096, dc=1536),
    4: Workload("decode_b8_ctx128k_bf16", "decode", "bf16", m=4, c=512, cI=128, nhI=64, nh=64,
                k=1024, B=8, L=131072),
    5: Workload("decode_ragged_b64_ctx1k-64k_bf16", "decode", "bf16", m=8, c=512, cI=128,
                nhI=32, nh=128, k=256, B=64, Lmin=1024, Lmax=65536),
}


def rng_for(seed: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(seed))


def _normal(rng, shape, std, dtype):
    x = rng.standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        x *= np.float32(std)
    if dtype == "bf16":
        return f32_to_bf16(x)
    return x


def normal(rng, shape, std: float = 1.0, dtype: str = "f32") -> np.ndarray:
    """Seeded N(0, std^2) draws: fp32, or bf16 bit patterns (uint16) for dtype "bf16"."""
    return _normal(rng, shape, std, dtype)


# Order in which prefill parameters are drawn (after H).
PREFILL_PARAM_ORDER = (
    "W_aKV", "W_bKV", "W_aZ", "W_bZ", "B_a", "B_b",
    "W_DQ", "W_UQI", "W_w",
    "W_aKV_I", "W_bKV_I", "W_aZ_I", "W_bZ_I", "B_aI", "B_bI",
    "W_UQ",
)


def prefill_shapes(w: Workload) -> Dict[str, tuple]:
    d, c, cI, m, dc = w.d, w.c, w.cI, w.m, w.dc
    return {
        "W_aKV": (d, c), "W_bKV": (d, c), "W_aZ": (d, c), "W_bZ": (d, c),
        "B_a": (m, c), "B_b": (m, c),
        "W_DQ": (d, dc), "W_UQI": (dc, cI * w.nhI), "W_w": (d, w.nhI),
        "W_aKV_I": (d, cI), "W_bKV_I": (d, cI), "W_aZ_I": (d, cI), "W_bZ_I": (d, cI),
        "B_aI": (m, cI), "B_bI": (m, cI),
        "W_UQ": (dc, c * w.nh),
    }


def _fan_in(name: str, w: Workload) -> int:
    return w.dc if name in ("W_UQI", "W_UQ") else w.d


def make_prefill(w: Workload, seed: Optional[int] = None, n: Optional[int] = None) -> Dict[str, np.ndarray]:
    """Hidden states and all parameters of one prefill workload.

    ``n`` overrides the sequence length (the parameters do not depend on it).
    """
    if seed is None:
        seed = next(k for k, v in WORKLOADS.items() if v == w)
    rng = rng_for(seed)
    n = w.n if n is None else n
    out: Dict[str, np.ndarray] = {"H": _normal(rng, (n, w.d), 1.0, w.dtype)}
    shapes = prefill_shapes(w)
    for name in PREFILL_PARAM_ORDER:
        if name.startswith("B_"):
            std = 0.1
        else:
            std = 1.0 / math.sqrt(_fan_in(name, w))
        out[name] = _normal(rng, shapes[name], std, w.dtype)
    return out


def ragged_lengths(rng, B: int, Lmin: int, Lmax: int) -> np.ndarray:
    """Context lengths log-uniform in [Lmin, Lmax], floored and clamped."""
    u = rng.uniform(math.log(Lmin), math.log(Lmax), size=B)
    L = np.floor(np.exp(u)).astype(np.int64)
    return np.clip(L, Lmin, Lmax)


def make_decode(w: Workload, seed: Optional[int] = None, B: Optional[int] = None,
                L: Optional[int] = None, q_std_mult: float = 1.0) -> Dict[str, np.ndarray]:
    """Compressed caches, queries and head weights of one decode batch.

    Sequence b holds ``N_b = floor(L_b / m)`` compressed entries stored from row
    ``kv_offset[b]`` of the shared cache buffers (exclusive prefix sum of N_b).
    ``B``/``L`` override batch size / fixed context length for small cases.
    """
    if seed is None:
        seed = next(k for k, v in WORKLOADS.items() if v == w)
    rng = rng_for(seed)
    B = w.B if B is None else B
    if w.L or L is not None:
        lens = np.full(B, w.L if L is None else L, dtype=np.int64)
    else:
        lens = ragged_lengths(rng, B, w.Lmin, w.Lmax)
    nblk = lens // w.m
    kv_offset = np.zeros(B, dtype=np.int64)
    kv_offset[1:] = np.cumsum(nblk)[:-1]
    rows = int(nblk.sum())
    out = {
        "seq_len": lens,
        "n_blocks": nblk,
        "kv_offset": kv_offset,
        "Ccomp": _normal(rng, (rows, w.c), 1.0, w.dtype),
        "KIcomp": _normal(rng, (rows, w.cI), 1.0, w.dtype),
        "q": _normal(rng, (B, w.nh, w.c), q_std_mult / math.sqrt(w.c), w.dtype),
        "qI": _normal(rng, (B, w.nhI, w.cI), 1.0 / math.sqrt(w.cI), w.dtype),
        "wI": rng.standard_normal(size=(B, w.nhI), dtype=np.float32),
    }
    return out


def random_selection(rng, n_cand: np.ndarray, k: int) -> np.ndarray:
    """A valid index set per query: min(k, n_cand) distinct indices in [0, n_cand), -1 padded.

    Used to drive the attention stage on its own with selections that do not
    come from any implementation of the selector.
    """
    n_cand = np.asarray(n_cand, dtype=np.int64)
    idx = np.full((n_cand.shape[0], k), -1, dtype=np.int32)
    for r, nc in enumerate(n_cand):
        nc = int(nc)
        if nc <= 0:
            continue
        take = min(k, nc)
        if take == nc:
            sel = rng.permutation(nc)
        else:
            sel = rng.choice(nc, size=take, replace=False)
        idx[r, :take] = sel.astype(np.int32)
    return idx
