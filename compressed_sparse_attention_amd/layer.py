"""CSA layer composites on top of the C ABI: ``prefill`` and ``decode``.

Only device-memory plumbing happens here (allocating outputs and taking
views); each step runs in libcsa's kernels through ``api``.

Parameter layout (done once by ``pack_prefill_params``):
  * every weight is stored transposed ([out, in], the way a linear layer
    keeps it), which is the operand layout of ``csa_project``;
  * the nine projections of the hidden states -- W^aKV, W^bKV, W^aZ, W^bZ
    (eqs 1-2), their indexer-key counterparts, and W^DQ (eq 5) -- are
    stacked into one [4c + 4c^I + d_c, d] matrix, so a single GEMM reads H
    once and writes all of them side by side into one [n, 4c + 4c^I + d_c]
    buffer; compression then reads column slices of that buffer;
  * W^w (eq 7) is its own small GEMM with an fp32 output (head weights are
    fp32), W^UQ of eq 6 and of eq 10 are two GEMMs on c^Q.
"""
from __future__ import annotations

import math
from typing import Dict, Optional

import numpy as np
import torch

from . import api
from .synth import bf16_to_f32

_H_SIDE = ("W_aKV", "W_bKV", "W_aZ", "W_bZ", "W_aKV_I", "W_bKV_I", "W_aZ_I", "W_bZ_I", "W_DQ")


def to_device(x: np.ndarray, dtype: str, device) -> torch.Tensor:
    """Stored array (fp32, or bf16 bits as uint16) -> torch tensor on `device`."""
    if dtype == "bf16" and x.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).to(device).view(torch.bfloat16)
    if x.dtype == np.uint16:
        x = bf16_to_f32(x)
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(device)


def pack_prefill_params(P: Dict[str, np.ndarray], dtype: str, device) -> Dict[str, torch.Tensor]:
    """Device copies of the parameters in the layout the prefill path uses."""
    t = {}
    WH = np.concatenate([np.asarray(P[name]) for name in _H_SIDE], axis=1)  # [d, 4c+4cI+dc]
    t["W_H_t"] = to_device(np.ascontiguousarray(WH.T), dtype, device)
    t["W_w_t"] = to_device(np.ascontiguousarray(np.asarray(P["W_w"]).T), dtype, device)
    t["W_UQI_t"] = to_device(np.ascontiguousarray(np.asarray(P["W_UQI"]).T), dtype, device)
    t["W_UQ_t"] = to_device(np.ascontiguousarray(np.asarray(P["W_UQ"]).T), dtype, device)
    for name in ("B_a", "B_b", "B_aI", "B_bI"):
        t[name] = to_device(np.asarray(P[name]), dtype, device)
    t["c"] = int(np.asarray(P["B_a"]).shape[1])
    t["cI"] = int(np.asarray(P["B_aI"]).shape[1])
    t["dc"] = int(np.asarray(P["W_DQ"]).shape[1])
    return t


class PrefillBuffers:
    """Intermediate and output buffers of one prefill shape (reused across calls).  selection = "dense"
    (csa_index_topk: the causal score matrix, then the selector) or "stream" (csa_index_topk_stream: the
    indexer keeps only the scores that can still be selected)."""

    def __init__(self, n: int, m: int, k: int, nh: int, nhI: int, c: int, cI: int, dc: int, dtype, device,
                 selection: str = "dense"):
        if selection not in ("dense", "stream"):
            raise ValueError("selection must be 'dense' or 'stream'")
        self.selection = selection
        width = 4 * c + 4 * cI + dc
        N = n // m
        self.Y_H = torch.empty(n, width, dtype=dtype, device=device)
        self.wI = torch.empty(n, nhI, dtype=torch.float32, device=device)
        self.qI = torch.empty(n, nhI * cI, dtype=dtype, device=device)
        self.q = torch.empty(n, nh * c, dtype=dtype, device=device)
        self.Ccomp = torch.empty(N, c, dtype=dtype, device=device)
        self.KIcomp = torch.empty(N, cI, dtype=dtype, device=device)
        self.idx = torch.empty(n, k, dtype=torch.int32, device=device)
        self.o = torch.empty(n, nh, c, dtype=dtype, device=device)
        self.lse = torch.empty(n, nh, dtype=torch.float32, device=device)
        ws_i = (api.csa_index_topk_workspace(n, N, nhI, k) if selection == "dense"
                else api.csa_index_topk_stream_workspace(n, N))
        ws_m = api.csa_sparse_mqa_workspace(n, nh, c, k)
        self.ws_index = torch.empty(max(ws_i, 1), dtype=torch.uint8, device=device)
        self.ws_mqa = torch.empty(max(ws_m, 1), dtype=torch.uint8, device=device)


def prefill(H: torch.Tensor, W: Dict[str, torch.Tensor], m: int, k: int, nh: int, nhI: int,
            scale: Optional[float] = None, buf: Optional[PrefillBuffers] = None,
            selection: str = "dense") -> PrefillBuffers:
    """Eqs 1-11 for one sequence H [n, d]: every token is a query (causal).  `selection` picks the eqs 8-9
    path when buf is not given (see PrefillBuffers)."""
    n = H.shape[0]
    c, cI, dc = W["c"], W["cI"], W["dc"]
    if buf is None:
        buf = PrefillBuffers(n, m, k, nh, nhI, c, cI, dc, H.dtype, H.device, selection=selection)
    Y = buf.Y_H
    api.csa_project(H, W["W_H_t"], Y)  # eqs 1, 2 (+ indexer copies), 5
    api.csa_project(H, W["W_w_t"], buf.wI)  # eq 7
    cQ = Y[:, 4 * c + 4 * cI:]
    api.csa_project(cQ, W["W_UQI_t"], buf.qI)  # eq 6
    api.csa_compress(Y[:, 0:c], Y[:, c:2 * c], Y[:, 2 * c:3 * c], Y[:, 3 * c:4 * c], W["B_a"], W["B_b"], m,
                     buf.Ccomp)  # eqs 3-4
    o = 4 * c
    api.csa_compress(Y[:, o:o + cI], Y[:, o + cI:o + 2 * cI], Y[:, o + 2 * cI:o + 3 * cI],
                     Y[:, o + 3 * cI:o + 4 * cI], W["B_aI"], W["B_bI"], m, buf.KIcomp)
    if buf.selection == "stream":
        api.csa_index_topk_stream(buf.qI.view(n, nhI, cI), buf.wI, buf.KIcomp, m, k, n // m, buf.idx,
                                  workspace=buf.ws_index)  # eqs 8-9 without the score matrix
    else:
        api.csa_index_topk(buf.qI.view(n, nhI, cI), buf.wI, buf.KIcomp, m, k, n // m, buf.idx,
                           workspace=buf.ws_index)  # eqs 8-9
    # the largest projection runs after the indexer, whose MFMA rate suffers
    # when it follows this GEMM directly
    api.csa_project(cQ, W["W_UQ_t"], buf.q)  # eq 10
    sc = 1.0 / math.sqrt(c) if scale is None else scale
    api.csa_sparse_mqa(buf.q.view(n, nh, c), buf.Ccomp, buf.idx, sc, buf.o, buf.lse,
                       workspace=buf.ws_mqa)  # eq 11
    return buf


class PrefillGrads:
    """Gradient buffers of one prefill shape (reused across calls).  Weight gradients are kept in the
    transposed layout of the weights they belong to (W_H_t, W_UQ_t); bias gradients are fp32."""

    def __init__(self, n: int, m: int, k: int, nh: int, c: int, cI: int, dc: int, d: int, dtype, device,
                 n_seqs: Optional[int] = None, n_blocks: Optional[int] = None):
        """One sequence of n tokens, or (n_seqs and n_blocks given) n tokens of packed sequences."""
        width = 4 * c + 4 * cI + dc
        N = n // m if n_seqs is None else n_blocks
        self.dq = torch.empty(n, nh * c, dtype=dtype, device=device)
        self.dCcomp = torch.empty(max(N, 1), c, dtype=torch.float32, device=device)[:N]
        self.dY_H = torch.zeros(n, width, dtype=dtype, device=device)  # indexer columns stay zero
        self.dH = torch.empty(n, d, dtype=dtype, device=device)
        self.dW_H_t = torch.empty(width, d, dtype=dtype, device=device)
        self.dW_UQ_t = torch.empty(nh * c, dc, dtype=dtype, device=device)
        self.dB_a = torch.empty(m, c, dtype=torch.float32, device=device)
        self.dB_b = torch.empty(m, c, dtype=torch.float32, device=device)
        ws_c = (api.csa_compress_backward_workspace(n, m, c) if n_seqs is None
                else api.csa_compress_backward_varlen_workspace(n_seqs, N, m, c))
        ws = max(api.csa_sparse_mqa_backward_workspace(n, nh, c, k, N), ws_c,
                 api.csa_project_backward_workspace(dtype, n, nh * c, dc, True, True),
                 api.csa_project_backward_workspace(dtype, n, width, d, True, True))
        self.ws = torch.empty(max(ws, 16), dtype=torch.uint8, device=device)


def prefill_backward(H: torch.Tensor, W: Dict[str, torch.Tensor], buf: PrefillBuffers, dO: torch.Tensor, m: int,
                     k: int, nh: int, scale: Optional[float] = None,
                     grads: Optional[PrefillGrads] = None) -> PrefillGrads:
    """Gradients of sum(dO * o) after ``prefill`` filled ``buf``: eq 11, eqs 3-4, eq 10, then eqs 1, 2, 5.

    The selection (eqs 6-9) passes no gradient, so the indexer's columns of dY_H stay zero and its
    weights get none.
    """
    n, d = H.shape
    c, cI, dc = W["c"], W["cI"], W["dc"]
    if grads is None:
        grads = PrefillGrads(n, m, k, nh, c, cI, dc, d, H.dtype, H.device)
    g = grads
    sc = 1.0 / math.sqrt(c) if scale is None else scale
    api.csa_sparse_mqa_backward(buf.q.view(n, nh, c), buf.Ccomp, buf.idx, sc, buf.o, buf.lse, dO,
                                g.dq.view(n, nh, c), g.dCcomp, workspace=g.ws)  # eq 11
    Y, dY = buf.Y_H, g.dY_H
    api.csa_compress_backward(Y[:, 0:c], Y[:, c:2 * c], Y[:, 2 * c:3 * c], Y[:, 3 * c:4 * c], W["B_a"], W["B_b"], m,
                              g.dCcomp, dY[:, 0:c], dY[:, c:2 * c], dY[:, 2 * c:3 * c], dY[:, 3 * c:4 * c],
                              g.dB_a, g.dB_b, workspace=g.ws)  # eqs 3-4
    o = 4 * c + 4 * cI
    api.csa_project_backward(Y[:, o:], W["W_UQ_t"], g.dq, dX=dY[:, o:], dWt=g.dW_UQ_t, workspace=g.ws)  # eq 10
    api.csa_project_backward(H, W["W_H_t"], dY, dX=g.dH, dWt=g.dW_H_t, workspace=g.ws)  # eqs 1, 2, 5
    return g


class VarlenPrefill:
    """Buffers and offsets of a prefill of several packed sequences (token rows of sequence b:
    cu[b] .. cu[b+1]-1; its compressed entries: rows block_offset[b] .. block_offset[b+1]-1)."""

    def __init__(self, lengths, m: int, k: int, nh: int, nhI: int, c: int, cI: int, dc: int, dtype, device):
        cu, bo = [0], [0]
        for L in lengths:
            if L < 0:
                raise ValueError("negative sequence length")
            cu.append(cu[-1] + int(L))
            bo.append(bo[-1] + int(L) // m)
        self.lengths = [int(L) for L in lengths]
        self.n, self.n_blocks = cu[-1], bo[-1]
        self.max_cand = max([(L - 1) // m for L in self.lengths if L > 0], default=0)
        self.cu = torch.tensor(cu, dtype=torch.int64, device=device)
        self.block_offset = torch.tensor(bo, dtype=torch.int64, device=device)
        n = self.n
        width = 4 * c + 4 * cI + dc
        self.Y_H = torch.empty(n, width, dtype=dtype, device=device)
        self.wI = torch.empty(n, nhI, dtype=torch.float32, device=device)
        self.qI = torch.empty(n, nhI * cI, dtype=dtype, device=device)
        self.q = torch.empty(n, nh * c, dtype=dtype, device=device)
        self.Ccomp = torch.empty(max(self.n_blocks, 1), c, dtype=dtype, device=device)
        self.KIcomp = torch.empty(max(self.n_blocks, 1), cI, dtype=dtype, device=device)
        self.idx = torch.empty(n, k, dtype=torch.int32, device=device)
        self.o = torch.empty(n, nh, c, dtype=dtype, device=device)
        self.lse = torch.empty(n, nh, dtype=torch.float32, device=device)
        self.q_seq = torch.empty(max(n, 1), dtype=torch.int32, device=device)
        ws_i = api.csa_index_topk_varlen_workspace(len(lengths), n, self.max_cand, k)
        ws_m = api.csa_sparse_mqa_workspace(n, nh, c, k)
        self.ws_index = torch.empty(max(ws_i, 1), dtype=torch.uint8, device=device)
        self.ws_mqa = torch.empty(max(ws_m, 1), dtype=torch.uint8, device=device)


def prefill_varlen(H: torch.Tensor, lengths, W: Dict[str, torch.Tensor], m: int, k: int, nh: int, nhI: int,
                   scale: Optional[float] = None, buf: Optional[VarlenPrefill] = None) -> VarlenPrefill:
    """Eqs 1-11 for several sequences packed in H [sum(lengths), d]: each sequence is a causal prefill of
    its own (its tokens see only its own compressed entries)."""
    c, cI, dc = W["c"], W["cI"], W["dc"]
    if buf is None:
        buf = VarlenPrefill(lengths, m, k, nh, nhI, c, cI, dc, H.dtype, H.device)
    n = buf.n
    if H.shape[0] != n:
        raise ValueError("H must hold sum(lengths) rows")
    Y = buf.Y_H
    api.csa_project(H, W["W_H_t"], Y)  # eqs 1, 2 (+ indexer copies), 5
    api.csa_project(H, W["W_w_t"], buf.wI)  # eq 7
    cQ = Y[:, 4 * c + 4 * cI:]
    api.csa_project(cQ, W["W_UQI_t"], buf.qI)  # eq 6
    api.csa_compress_varlen(Y[:, 0:c], Y[:, c:2 * c], Y[:, 2 * c:3 * c], Y[:, 3 * c:4 * c], W["B_a"], W["B_b"], m,
                            buf.cu, buf.block_offset, buf.n_blocks, buf.Ccomp)  # eqs 3-4
    o = 4 * c
    api.csa_compress_varlen(Y[:, o:o + cI], Y[:, o + cI:o + 2 * cI], Y[:, o + 2 * cI:o + 3 * cI],
                            Y[:, o + 3 * cI:o + 4 * cI], W["B_aI"], W["B_bI"], m, buf.cu, buf.block_offset,
                            buf.n_blocks, buf.KIcomp)
    api.csa_index_topk_varlen(buf.qI.view(n, nhI, cI), buf.wI, buf.KIcomp, m, k, buf.max_cand, buf.cu,
                              buf.block_offset, buf.idx, q_seq_out=buf.q_seq[:n], workspace=buf.ws_index)  # eqs 8-9
    api.csa_project(cQ, W["W_UQ_t"], buf.q)  # eq 10
    sc = 1.0 / math.sqrt(c) if scale is None else scale
    api.csa_sparse_mqa(buf.q.view(n, nh, c), buf.Ccomp, buf.idx, sc, buf.o, buf.lse, q_seq=buf.q_seq[:n],
                       kv_offset=buf.block_offset, workspace=buf.ws_mqa)  # eq 11
    return buf


def prefill_varlen_backward(H: torch.Tensor, W: Dict[str, torch.Tensor], buf: VarlenPrefill, dO: torch.Tensor,
                            m: int, k: int, nh: int, scale: Optional[float] = None,
                            grads: Optional[PrefillGrads] = None) -> PrefillGrads:
    """Gradients of sum(dO * o) after ``prefill_varlen`` filled ``buf``; the order of ``prefill_backward``.

    Per-token gradients (dq, dH and the projection rows) follow each token's own sequence; the weight and
    bias gradients are shared parameters and sum over every sequence.
    """
    n, d = H.shape
    c, cI, dc = W["c"], W["cI"], W["dc"]
    if n != buf.n:
        raise ValueError("H must hold sum(lengths) rows")
    if grads is None:
        grads = PrefillGrads(n, m, k, nh, c, cI, dc, d, H.dtype, H.device, n_seqs=len(buf.lengths),
                             n_blocks=buf.n_blocks)
    g = grads
    sc = 1.0 / math.sqrt(c) if scale is None else scale
    api.csa_sparse_mqa_backward(buf.q.view(n, nh, c), buf.Ccomp[:buf.n_blocks], buf.idx, sc, buf.o, buf.lse, dO,
                                g.dq.view(n, nh, c), g.dCcomp, q_seq=buf.q_seq[:n], kv_offset=buf.block_offset,
                                workspace=g.ws)  # eq 11
    Y, dY = buf.Y_H, g.dY_H
    api.csa_compress_backward_varlen(Y[:, 0:c], Y[:, c:2 * c], Y[:, 2 * c:3 * c], Y[:, 3 * c:4 * c], W["B_a"],
                                     W["B_b"], m, buf.cu, buf.block_offset, buf.n_blocks, g.dCcomp, dY[:, 0:c],
                                     dY[:, c:2 * c], dY[:, 2 * c:3 * c], dY[:, 3 * c:4 * c], g.dB_a, g.dB_b,
                                     workspace=g.ws)  # eqs 3-4
    o = 4 * c + 4 * cI
    api.csa_project_backward(Y[:, o:], W["W_UQ_t"], g.dq, dX=dY[:, o:], dWt=g.dW_UQ_t, workspace=g.ws)  # eq 10
    api.csa_project_backward(H, W["W_H_t"], dY, dX=g.dH, dWt=g.dW_H_t, workspace=g.ws)  # eqs 1, 2, 5
    return g


class DecodeBuffers:
    """Outputs and the persistent workspace of decode steps of one batch shape."""

    def __init__(self, B: int, k: int, nh: int, c: int, nhI: int, max_cand: int, dtype, device):
        self.idx = torch.empty(B, k, dtype=torch.int32, device=device)
        self.scores = torch.empty(B, k, dtype=torch.float32, device=device)
        self.o = torch.empty(B, nh, c, dtype=dtype, device=device)
        self.lse = torch.empty(B, nh, dtype=torch.float32, device=device)
        self.q_seq = torch.arange(B, dtype=torch.int32, device=device)
        self.shape = (B, max_cand, nhI, nh, c, k)
        ws = api.csa_decode_workspace(*self.shape)
        # zero once: every csa_decode call leaves it ready for the next one
        self.ws = torch.zeros(max(ws, 1), dtype=torch.uint8, device=device)


def decode(q, qI, wI, Ccomp, KIcomp, seq_len, kv_offset, m: int, k: int, max_cand: int,
           scale: Optional[float] = None, buf: Optional[DecodeBuffers] = None) -> DecodeBuffers:
    """One decode step: query b is appended after seq_len[b] tokens of sequence b (eqs 8, 9, 11).

    seq_len, kv_offset: int64 device tensors [B]; max_cand >= max_b floor(seq_len[b]/m).
    """
    B, nh, c = q.shape
    nhI = qI.shape[1]
    if buf is None or buf.shape != (B, max_cand, nhI, nh, c, k):
        buf = DecodeBuffers(B, k, nh, c, nhI, max_cand, q.dtype, q.device)
    sc = 1.0 / math.sqrt(c) if scale is None else scale
    api.csa_decode(qI, wI, KIcomp, q, Ccomp, m, k, max_cand, sc, seq_len, buf.idx, buf.o, buf.ws, lse=buf.lse,
                   score_out=buf.scores, q_seq=buf.q_seq, kv_offset=kv_offset)
    return buf


class DecodeState:
    """Per-sequence decode state of B sequences (the cache maintenance of a decode loop).

    * Ccomp / KIcomp: compressed caches with room for ``capacity`` blocks per
      sequence; sequence b's rows start at kv_offset[b] = b * capacity.
    * ring / ring_I: the projected rows [C^a|C^b|Z^a|Z^b] of each sequence's last
      2m tokens (token t in slot t mod 2m), main and indexer widths.
    * t: position of each sequence's next token (int64, device), mirrored on
      the host in t_host so that a step can be refused before it launches.

    Sequence b may hold tokens 0 .. capacity * m - 1.  Token t belongs to block
    floor(t/m), so token capacity * m would eventually write row capacity of its
    sequence -- the next sequence's first row, or past the end of the buffer --
    and ``decode_step`` raises before any sequence reaches it.
    """

    def __init__(self, B: int, capacity: int, m: int, c: int, cI: int, dtype, device):
        self.B, self.capacity, self.m = B, capacity, m
        self.Ccomp = torch.zeros(B * capacity, c, dtype=dtype, device=device)
        self.KIcomp = torch.zeros(B * capacity, cI, dtype=dtype, device=device)
        self.kv_offset = torch.arange(B, dtype=torch.int64, device=device) * capacity
        self.ring = torch.zeros(B, 2 * m, 4 * c, dtype=dtype, device=device)
        self.ring_I = torch.zeros(B, 2 * m, 4 * cI, dtype=dtype, device=device)
        self.t = torch.zeros(B, dtype=torch.int64, device=device)
        self.t_host = np.zeros(B, dtype=np.int64)

    def check_room(self):
        """Raises if some sequence's next token would not fit in its cache rows."""
        full = np.nonzero(self.t_host >= self.capacity * self.m)[0]
        if full.size:
            b = int(full[0])
            raise ValueError(f"sequence {b} is at token {int(self.t_host[b])}: its cache holds "
                             f"{self.capacity} blocks of {self.m} tokens (tokens 0 .. "
                             f"{self.capacity * self.m - 1})")

    def load_prefill(self, b: int, buf: "PrefillBuffers", c: int, cI: int):
        """Hand sequence b over from a prefill of its first L tokens (copies only)."""
        L = buf.Y_H.shape[0]
        nb = L // self.m
        if nb > self.capacity:
            raise ValueError("prefill longer than the cache capacity")
        o = b * self.capacity
        self.Ccomp[o:o + nb].copy_(buf.Ccomp[:nb])
        self.KIcomp[o:o + nb].copy_(buf.KIcomp[:nb])
        for tok in range(max(0, L - 2 * self.m), L):
            slot = tok % (2 * self.m)
            self.ring[b, slot].copy_(buf.Y_H[tok, :4 * c])
            self.ring_I[b, slot].copy_(buf.Y_H[tok, 4 * c:4 * c + 4 * cI])
        self.t[b] = L
        self.t_host[b] = L


def decode_step(H_new: torch.Tensor, W: Dict[str, torch.Tensor], state: DecodeState, m: int, k: int, nh: int,
                nhI: int, scale: Optional[float] = None, buf: Optional[DecodeBuffers] = None) -> DecodeBuffers:
    """One decode step with cache maintenance: every sequence b appends token state.t[b] with hidden
    state H_new[b].  Eqs 1, 2, 5, 6, 7, 10 for the new tokens (two paired few-row GEMM launches), eqs 3-4
    appended to the compressed caches when a block completes, then eqs 8, 9, 11 for the new tokens; positions
    advance."""
    B = H_new.shape[0]
    if B != state.B:
        raise ValueError("H_new must hold one row per sequence of the state")
    state.check_room()
    c, cI = W["c"], W["cI"]
    width = 4 * c + 4 * cI + W["dc"]
    Y = torch.empty(B, width, dtype=H_new.dtype, device=H_new.device)
    wI = torch.empty(B, nhI, dtype=torch.float32, device=H_new.device)
    qI = torch.empty(B, nhI * cI, dtype=H_new.dtype, device=H_new.device)
    q = torch.empty(B, nh * c, dtype=H_new.dtype, device=H_new.device)
    api.csa_project_pair(H_new, W["W_H_t"], Y, W["W_w_t"], wI)  # eqs 1, 2 (+ indexer copies), 5; eq 7
    cQ = Y[:, 4 * c + 4 * cI:]
    api.csa_project_pair(cQ, W["W_UQ_t"], q, W["W_UQI_t"], qI)  # eq 10; eq 6
    api.csa_compress_append_pair(Y[:, :4 * c], state.ring, W["B_a"], W["B_b"], state.Ccomp,  # eqs 3-4, both caches
                                 Y[:, 4 * c:4 * c + 4 * cI], state.ring_I, W["B_aI"], W["B_bI"], state.KIcomp,
                                 m, state.t, state.kv_offset)
    # the block a token completes is not among its own candidates (s < floor(t/m))
    buf = decode(q.view(B, nh, c), qI.view(B, nhI, cI), wI, state.Ccomp, state.KIcomp, state.t, state.kv_offset,
                 m, k, state.capacity, scale=scale, buf=buf)
    # this step's projected queries (eqs 6, 7, 10), kept for inspection until the next step
    buf.q_in, buf.qI_in, buf.wI_in = q.view(B, nh, c), qI.view(B, nhI, cI), wI
    state.t += 1
    state.t_host += 1
    return buf
