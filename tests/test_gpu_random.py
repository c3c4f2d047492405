"""Seeded random-shape GPU parity: the compression, selection, attention, compression-gradient and projection
calls on shapes drawn at random (sizes, ragged edges, head counts, k, column pitches), each against the oracle
as in the hand-picked cases.  Every case is fixed by its index, so a failure names a reproducible shape."""
import math

import numpy as np
import pytest
import torch

from compressed_sparse_attention_amd import api, synth
from compressed_sparse_attention_amd.layer import to_device
from oracle import csa_oracle as O
from parity import assert_rows_close, check_topk, to_np64

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
TD = {"f32": torch.float32, "bf16": torch.bfloat16}


def _rng(tag, i):
    return synth.rng_for(1000 * tag + i)


def _draw(rng, shape, std, dtype):
    x = rng.standard_normal(size=shape, dtype=np.float32) * np.float32(std)
    return synth.f32_to_bf16(x) if dtype == "bf16" else x


def _f64(x, dtype):
    return synth.to_f64(x, dtype)


@pytest.mark.parametrize("i", range(16))
def test_random_compress(i):
    rng = _rng(1, i)
    dtype = ["f32", "bf16"][i % 2]
    m = int(rng.choice([1, 2, 3, 4, 5, 6, 8, 16]))
    c = 4 * int(rng.integers(1, 161))
    n = int(rng.integers(0, 2500)) if i % 5 else int(rng.integers(0, 3 * m))
    cp = (c + 7) // 8 * 8 + 8 * int(rng.integers(0, 3))  # column pitch of the four slices
    print(f"compress case {i}: {dtype} n={n} m={m} c={c} pitch={cp}", flush=True)
    P = _draw(rng, (n, 4 * cp), 1.0, dtype)
    Pz = _draw(rng, (n, 4 * cp), 2.0, dtype)
    P = np.where((np.arange(4 * cp) // cp)[None, :] >= 2, Pz, P)
    Ba, Bb = _draw(rng, (m, c), 0.5, dtype), _draw(rng, (m, c), 0.5, dtype)
    Pd = to_device(P, dtype, DEV)
    N = n // m
    out = torch.full((max(N, 1), cp), 3.0, dtype=TD[dtype], device=DEV)[:N, :c]  # rows 16-byte aligned
    api.csa_compress(*[Pd[:, j * cp:j * cp + c] for j in range(4)], to_device(Ba, dtype, DEV),
                     to_device(Bb, dtype, DEV), m, out)
    torch.cuda.synchronize()
    if N:
        P64 = _f64(P, dtype)
        ref = O.compress(*[P64[:, j * cp:j * cp + c] for j in range(4)], _f64(Ba, dtype), _f64(Bb, dtype), m)
        assert_rows_close(to_np64(out), ref, what=f"compress case {i}")


@pytest.mark.parametrize("i", range(12))
def test_random_index_topk_decode(i):
    rng = _rng(2, i)
    dtype = "f32" if i % 6 == 5 else "bf16"
    m = int(rng.choice([1, 2, 4, 8]))
    nhI = int(rng.integers(1, 65))
    cI = int(rng.choice([32, 64, 128, 256]))
    k = int(rng.integers(1, 1500))
    B = int(rng.integers(1, 9))
    lens = rng.integers(0, 4 * 8000, size=B).astype(np.int64)
    lens[rng.random(B) < 0.2] = int(rng.integers(0, 4 * m))  # some sequences with no or few blocks
    print(f"index_topk case {i}: {dtype} m={m} nhI={nhI} cI={cI} k={k} lens={lens.tolist()}", flush=True)
    nblk = lens // m
    off = np.zeros_like(nblk)
    off[1:] = np.cumsum(nblk)[:-1]
    K = _draw(rng, (max(int(nblk.sum()), 1), cI), 1.0, dtype)
    qI = _draw(rng, (B, nhI, cI), 1.0 / math.sqrt(cI), dtype)
    wI = rng.standard_normal((B, nhI), dtype=np.float32)
    idx = torch.full((B, k), 123456, dtype=torch.int32, device=DEV)
    max_cand = int(nblk.max())
    api.csa_index_topk(to_device(qI, dtype, DEV), to_device(wI, "f32", DEV), to_device(K, dtype, DEV), m, k,
                       max_cand, idx, q_seq=torch.arange(B, dtype=torch.int32, device=DEV),
                       q_pos=torch.tensor(lens, device=DEV), kv_offset=torch.tensor(off, device=DEV))
    torch.cuda.synchronize()
    K64 = _f64(K, dtype)
    rows = [O.index_scores_row(_f64(qI[b], dtype), wI[b].astype(np.float64), K64[off[b]:off[b] + nblk[b]],
                               int(nblk[b])) for b in range(B)]
    check_topk(idx.cpu().numpy(), rows, k)


@pytest.mark.parametrize("i", range(12))
def test_random_sparse_mqa(i):
    rng = _rng(3, i)
    dtype = "f32" if i % 4 == 3 else "bf16"
    c = int(rng.choice([64, 128, 256, 512]))
    nh = int(rng.integers(1, 131))
    k = int(rng.integers(1, 701))
    nblk = int(rng.integers(1, 801))
    # short batches (split slots) and long ones (one workgroup per query and head group), kept to a size the
    # oracle finishes quickly
    B = int(rng.integers(1, 41)) if i % 3 else int(rng.integers(520, 641))
    while B * nh * min(k, nblk) * c > 3e8 and nh > 1:
        nh = max(1, nh // 2)
    qmult = float(rng.choice([1.0, 4.0, 16.0]))
    print(f"sparse_mqa case {i}: {dtype} B={B} nh={nh} c={c} k={k} nblk={nblk} q x{qmult}", flush=True)
    C = _draw(rng, (B * nblk, c), 1.0, dtype)
    q = _draw(rng, (B, nh, c), qmult / math.sqrt(c), dtype)
    ncand = rng.integers(0, nblk + 1, size=B)
    idx = synth.random_selection(rng, ncand, k)
    if i % 2:
        idx = np.stack([rng.permutation(row) for row in idx])  # -1 slots between valid ones
    off = np.arange(B, dtype=np.int64) * nblk
    o = torch.full((B, nh, c), 5.0, dtype=TD[dtype], device=DEV)
    lse = torch.empty(B, nh, dtype=torch.float32, device=DEV)
    scale = 1.0 / math.sqrt(c)
    api.csa_sparse_mqa(to_device(q, dtype, DEV), to_device(C, dtype, DEV), torch.from_numpy(idx).to(DEV), scale, o,
                       lse, q_seq=torch.arange(B, dtype=torch.int32, device=DEV),
                       kv_offset=torch.from_numpy(off).to(DEV))
    torch.cuda.synchronize()
    C64, q64 = _f64(C, dtype), _f64(q, dtype)
    o_np, lse_np = to_np64(o), lse.cpu().numpy().astype(np.float64)
    for b in range(B):
        sel = idx[b][idx[b] >= 0]
        ro, rl = O.mqa(q64[b], C64[off[b] + sel], scale)
        assert_rows_close(o_np[b], ro, what=f"mqa case {i} o[{b}]")
        if sel.size == 0:
            assert np.all(np.isneginf(lse_np[b]))
        else:
            assert np.allclose(lse_np[b], rl, rtol=1e-3, atol=1e-3)


@pytest.mark.parametrize("i", range(8))
def test_random_compress_backward(i):
    rng = _rng(4, i)
    dtype = ["f32", "bf16"][i % 2]
    m = int(rng.choice([1, 2, 3, 4, 8, 16]))
    c = 4 * int(rng.integers(1, 161))
    n = int(rng.integers(0, 2000))
    cp = (c + 7) // 8 * 8 + 8 * int(rng.integers(0, 3))
    print(f"compress_backward case {i}: {dtype} n={n} m={m} c={c} pitch={cp}", flush=True)
    P = _draw(rng, (n, 4 * cp), 1.0, dtype)
    Pz = _draw(rng, (n, 4 * cp), 2.0, dtype)
    P = np.where((np.arange(4 * cp) // cp)[None, :] >= 2, Pz, P)
    Ba, Bb = _draw(rng, (m, c), 0.5, dtype), _draw(rng, (m, c), 0.5, dtype)
    N = n // m
    dC = rng.standard_normal(size=(N, c)).astype(np.float32)
    Pd = to_device(P, dtype, DEV)
    G = torch.full((n, 4 * cp), 7.0, dtype=TD[dtype], device=DEV)
    gs = [G[:, j * cp:j * cp + c] for j in range(4)]
    dBa = torch.full((m, c), 7.0, device=DEV)
    dBb = torch.full((m, c), 7.0, device=DEV)
    api.csa_compress_backward(*[Pd[:, j * cp:j * cp + c] for j in range(4)], to_device(Ba, dtype, DEV),
                              to_device(Bb, dtype, DEV), m, torch.from_numpy(dC).to(DEV), *gs, dBa, dBb)
    torch.cuda.synchronize()
    P64 = _f64(P, dtype)
    ref = O.compress_backward(*[P64[:, j * cp:j * cp + c] for j in range(4)], _f64(Ba, dtype), _f64(Bb, dtype), m,
                              dC.astype(np.float64))
    if n:
        for w in range(4):
            assert_rows_close(to_np64(gs[w]), ref[w], what=f"compress_backward case {i} grad {w}")
    mag_a = np.abs(ref[2][:N * m]).reshape(N, m, c).sum(0) if N else np.zeros((m, c))
    mag_b = np.abs(ref[3][:(N - 1) * m]).reshape(N - 1, m, c).sum(0) if N > 1 else np.zeros((m, c))
    tol = 1e-5 if dtype == "f32" else 1e-4
    for got, want, mag in ((dBa, ref[4], mag_a), (dBb, ref[5], mag_b)):
        assert np.all(np.abs(to_np64(got) - want) <= tol * mag + 1e-7), f"compress_backward case {i} bias"


@pytest.mark.parametrize("i", range(10))
def test_random_project(i):
    rng = _rng(5, i)
    din, dout = [("bf16", "bf16"), ("bf16", "f32"), ("f32", "f32")][i % 3]
    M = int(rng.integers(1, 1200))
    N = 8 * int(rng.integers(1, 200))
    K = 8 * int(rng.integers(1, 300)) if i % 2 else 64 * int(rng.integers(1, 40))
    print(f"project case {i}: {din}->{dout} M={M} N={N} K={K}", flush=True)
    X = _draw(rng, (M, K), 1.0, din)
    W = _draw(rng, (K, N), 1.0 / math.sqrt(K), din)
    Y = torch.empty(M, N, dtype=TD[dout], device=DEV)
    api.csa_project(to_device(X, din, DEV), to_device(np.ascontiguousarray(W.T), din, DEV), Y)
    torch.cuda.synchronize()
    assert_rows_close(to_np64(Y), O.project(_f64(X, din), _f64(W, din)), what=f"project case {i}")


def _mqa_ref(q64, C64, idx, row_off, scale):
    """Oracle attention of every query over its selected rows (o [B, nh, c])."""
    out = np.zeros_like(q64)
    for b in range(q64.shape[0]):
        sel = idx[b][idx[b] >= 0]
        out[b] = O.mqa(q64[b], C64[row_off[b] + sel], scale)[0]
    return out


@pytest.mark.parametrize("i", range(8))
def test_random_sparse_mqa_backward(i):
    from parity import assert_dq_close
    rng = _rng(6, i)
    c = 512
    nh = int(rng.integers(1, 131))
    k = int(rng.integers(1, 600))
    nblk = int(rng.integers(1, 700))
    qps = int(rng.integers(1, 12))
    B = int(rng.integers(1, 60))
    while B * nh * min(k, nblk) * c > 2e8 and nh > 1:
        nh = max(1, nh // 2)
    qmult = float(rng.choice([1.0, 4.0, 8.0]))
    nseq = (B + qps - 1) // qps
    print(f"sparse_mqa_backward case {i}: B={B} nh={nh} k={k} nblk={nblk} queries/seq={qps} q x{qmult}", flush=True)
    C = _draw(rng, (nseq * nblk, c), 1.0, "bf16")
    q = _draw(rng, (B, nh, c), qmult / math.sqrt(c), "bf16")
    dO = _draw(rng, (B, nh, c), 1.0, "bf16")
    idx = synth.random_selection(rng, rng.integers(0, nblk + 1, size=B), k)
    if i % 2:
        idx = np.stack([rng.permutation(row) for row in idx])
    q_seq = (np.arange(B) // qps).astype(np.int32)
    off = np.arange(nseq, dtype=np.int64) * nblk
    qd, Cd, dOd = to_device(q, "bf16", DEV), to_device(C, "bf16", DEV), to_device(dO, "bf16", DEV)
    idxd = torch.from_numpy(idx).to(DEV)
    qsd, offd = torch.from_numpy(q_seq).to(DEV), torch.from_numpy(off).to(DEV)
    o = torch.empty(B, nh, c, dtype=torch.bfloat16, device=DEV)
    lse = torch.empty(B, nh, dtype=torch.float32, device=DEV)
    scale = 1.0 / math.sqrt(c)
    api.csa_sparse_mqa(qd, Cd, idxd, scale, o, lse, q_seq=qsd, kv_offset=offd)
    dq = torch.full((B, nh, c), 9.0, dtype=torch.bfloat16, device=DEV)
    dC = torch.full((nseq * nblk, c), 9.0, dtype=torch.float32, device=DEV)
    api.csa_sparse_mqa_backward(qd, Cd, idxd, scale, o, lse, dOd, dq, dC, q_seq=qsd, kv_offset=offd)
    torch.cuda.synchronize()
    q64, C64, dO64 = _f64(q, "bf16"), _f64(C, "bf16"), _f64(dO, "bf16")
    ref_dq, ref_dC = O.sparse_mqa_backward(q64, C64, idx, off[q_seq], scale, dO64)
    assert_rows_close(to_np64(dC), ref_dC, what=f"mqa backward case {i} dCcomp")
    assert_dq_close(to_np64(dq), ref_dq, dO64, _mqa_ref(q64, C64, idx, off[q_seq], scale), scale,
                    what=f"mqa backward case {i} dq")


def _packed(lengths, m, lead):
    cu = (np.concatenate([[0], np.cumsum(lengths)]) + lead).astype(np.int64)
    bo = np.concatenate([[0], np.cumsum(np.asarray(lengths, np.int64) // m)]).astype(np.int64)
    return cu, bo


@pytest.mark.parametrize("i", range(6))
def test_random_compress_varlen_forward_and_backward(i):
    rng = _rng(7, i)
    dtype = ["bf16", "f32"][i % 2]
    m = int(rng.choice([1, 2, 4, 8, 16]))
    c = 8 * int(rng.integers(1, 70))
    lengths = [int(x) for x in rng.integers(0, 700, size=int(rng.integers(0, 25)))]
    lead = int(rng.integers(0, 5))
    cu, bo = _packed(lengths, m, lead)
    n = int(cu[-1]) + int(rng.integers(0, 4))
    nb = int(bo[-1])
    cp = c + 8 * int(rng.integers(0, 3))
    print(f"varlen compression case {i}: {dtype} m={m} c={c} lead={lead} lengths={lengths}", flush=True)
    P = _draw(rng, (n, 4 * cp), 1.0, dtype)
    Pz = _draw(rng, (n, 4 * cp), 2.0, dtype)
    P = np.where((np.arange(4 * cp) // cp)[None, :] >= 2, Pz, P)
    Ba, Bb = _draw(rng, (m, c), 0.5, dtype), _draw(rng, (m, c), 0.5, dtype)
    dCc = rng.standard_normal(size=(nb, c)).astype(np.float32)
    Pd = to_device(P, dtype, DEV)
    sl = [Pd[:, j * cp:j * cp + c] for j in range(4)]
    Bad, Bbd = to_device(Ba, dtype, DEV), to_device(Bb, dtype, DEV)
    cud, bod = torch.tensor(cu, device=DEV), torch.tensor(bo, device=DEV)
    out = torch.full((nb + 1, cp), 3.0, dtype=TD[dtype], device=DEV)[:, :c]
    api.csa_compress_varlen(*sl, Bad, Bbd, m, cud, bod, nb, out)
    G = torch.full((n, 4 * cp), 7.0, dtype=TD[dtype], device=DEV)
    gs = [G[:, j * cp:j * cp + c] for j in range(4)]
    dBa = torch.full((m, c), 7.0, device=DEV)
    dBb = torch.full((m, c), 7.0, device=DEV)
    api.csa_compress_backward_varlen(*sl, Bad, Bbd, m, cud, bod, nb, torch.from_numpy(dCc).to(DEV), *gs, dBa, dBb)
    torch.cuda.synchronize()
    P64 = _f64(P, dtype)
    got_out, got_g = to_np64(out), to_np64(G).reshape(n, 4, cp)
    sum_a, sum_b = np.zeros((m, c)), np.zeros((m, c))
    mag_a, mag_b = np.zeros((m, c)), np.zeros((m, c))
    for b in range(len(lengths)):
        seg = P64[cu[b]:cu[b + 1]]
        parts = [seg[:, j * cp:j * cp + c] for j in range(4)]
        N = int(bo[b + 1] - bo[b])
        if N:
            ref = O.compress(*parts, _f64(Ba, dtype), _f64(Bb, dtype), m)
            assert_rows_close(got_out[bo[b]:bo[b + 1]], ref, what=f"varlen case {i} sequence {b}")
        g = O.compress_backward(*parts, _f64(Ba, dtype), _f64(Bb, dtype), m, dCc[bo[b]:bo[b + 1]].astype(np.float64))
        if seg.shape[0]:
            for w in range(4):
                assert_rows_close(got_g[cu[b]:cu[b + 1], w, :c], g[w], what=f"varlen case {i} seq {b} grad {w}")
        sum_a += g[4]
        sum_b += g[5]
        mag_a += np.abs(g[2][:N * m]).reshape(N, m, c).sum(0) if N else 0.0
        mag_b += np.abs(g[3][:(N - 1) * m]).reshape(N - 1, m, c).sum(0) if N > 1 else 0.0
    tol = 1e-5 if dtype == "f32" else 1e-4
    for gpu, want, mag in ((dBa, sum_a, mag_a), (dBb, sum_b, mag_b)):
        assert np.all(np.abs(to_np64(gpu) - want) <= tol * mag + 1e-7), f"varlen case {i} bias gradient"
    assert np.all(got_out[nb:] == 3.0)
    assert np.all(got_g[:lead] == 7.0) and np.all(got_g[int(cu[-1]):] == 7.0)


@pytest.mark.parametrize("i", range(8))
def test_random_project_backward(i):
    rng = _rng(8, i)
    din, dout = [("bf16", "bf16"), ("bf16", "f32"), ("f32", "f32")][i % 3]
    M = int(rng.integers(1, 900))
    N = 8 * int(rng.integers(1, 120))
    K = 8 * int(rng.integers(1, 120))
    print(f"project_backward case {i}: {din}->{dout} M={M} N={N} K={K}", flush=True)
    X = _draw(rng, (M, K), 1.0, din)
    W = _draw(rng, (K, N), 1.0 / math.sqrt(K), din)
    dY = _draw(rng, (M, N), 1.0, din)
    dX = torch.full((M, K), 7.0, dtype=TD[dout], device=DEV)
    dWt = torch.full((N, K), 7.0, dtype=TD[dout], device=DEV)
    api.csa_project_backward(to_device(X, din, DEV), to_device(np.ascontiguousarray(W.T), din, DEV),
                             to_device(dY, din, DEV), dX, dWt)
    torch.cuda.synchronize()
    ref_dX, ref_dW = O.project_backward(_f64(X, din), _f64(W, din), _f64(dY, din))
    assert_rows_close(to_np64(dX), ref_dX, what=f"project_backward case {i} dX")
    assert_rows_close(to_np64(dWt), ref_dW.T, what=f"project_backward case {i} dWt")


@pytest.mark.parametrize("i", range(6))
def test_random_decode(i):
    """csa_decode (eqs 8, 9, 11 in one call): the selection against the oracle's scores, and the output against
    the oracle's attention over the selection the GPU made."""
    from compressed_sparse_attention_amd import layer
    rng = _rng(9, i)
    m = int(rng.choice([2, 4, 8]))
    nhI = int(rng.integers(1, 65))
    cI = int(rng.choice([64, 128]))
    nh = int(rng.integers(1, 129))
    c = int(rng.choice([128, 256, 512]))
    k = int(rng.integers(1, 800))
    B = int(rng.integers(1, 12))
    lens = rng.integers(0, 4 * 6000, size=B).astype(np.int64)
    while B * nh * min(k, int(lens.max()) // m + 1) * c > 2e8 and nh > 1:
        nh = max(1, nh // 2)
    print(f"decode case {i}: B={B} m={m} nhI={nhI} cI={cI} nh={nh} c={c} k={k} lens={lens.tolist()}", flush=True)
    nblk = lens // m
    off = np.zeros_like(nblk)
    off[1:] = np.cumsum(nblk)[:-1]
    rows = max(int(nblk.sum()), 1)
    K = _draw(rng, (rows, cI), 1.0, "bf16")
    C = _draw(rng, (rows, c), 1.0, "bf16")
    qI = _draw(rng, (B, nhI, cI), 1.0 / math.sqrt(cI), "bf16")
    q = _draw(rng, (B, nh, c), 4.0 / math.sqrt(c), "bf16")
    wI = rng.standard_normal((B, nhI), dtype=np.float32)
    max_cand = int(nblk.max())
    buf = layer.decode(to_device(q, "bf16", DEV), to_device(qI, "bf16", DEV), to_device(wI, "f32", DEV),
                       to_device(C, "bf16", DEV), to_device(K, "bf16", DEV), torch.tensor(lens, device=DEV),
                       torch.tensor(off, device=DEV), m, k, max_cand)
    torch.cuda.synchronize()
    idx = buf.idx.cpu().numpy()
    K64 = _f64(K, "bf16")
    score_rows = [O.index_scores_row(_f64(qI[b], "bf16"), wI[b].astype(np.float64), K64[off[b]:off[b] + nblk[b]],
                                     int(nblk[b])) for b in range(B)]
    check_topk(idx, score_rows, k)
    ref_o = _mqa_ref(_f64(q, "bf16"), _f64(C, "bf16"), idx, off, 1.0 / math.sqrt(c))
    assert_rows_close(to_np64(buf.o), ref_o, what=f"decode case {i} o")


@pytest.mark.parametrize("i", range(6))
def test_random_compress_append(i):
    """Decode-time cache maintenance on random shapes: sequences that already hold a random number of tokens
    grow one token per call; the appended compressed rows equal the oracle's compression of the whole
    sequences, and no other cache row is touched."""
    rng = _rng(10, i)
    dtype = ["bf16", "f32"][i % 2]
    m = int(rng.choice([1, 2, 4, 8, 16]))
    c = 4 * int(rng.integers(1, 150))
    B = int(rng.integers(1, 6))
    steps = int(rng.integers(1, 41))
    pre = [int(x) for x in rng.integers(0, 3 * m + 6, size=B)]
    print(f"compress_append case {i}: {dtype} m={m} c={c} B={B} steps={steps} pre={pre}", flush=True)
    cp = (c + 7) // 8 * 8
    seqs = []
    for b in range(B):
        n = pre[b] + steps
        Y = _draw(rng, (n, 4 * c), 1.0, dtype)
        Yz = _draw(rng, (n, 4 * c), 2.0, dtype)
        seqs.append(np.where((np.arange(4 * c) // c)[None, :] >= 2, Yz, Y))
    Ba, Bb = _draw(rng, (m, c), 0.5, dtype), _draw(rng, (m, c), 0.5, dtype)
    cap = max(pre) // m + steps // m + 2
    Cbig = torch.full((B * cap, cp), 3.0, dtype=TD[dtype], device=DEV)
    C = Cbig[:, :c]
    ring = torch.zeros(B, 2 * m, 4 * c, dtype=TD[dtype], device=DEV)
    for b in range(B):
        for tok in range(max(0, pre[b] - 2 * m), pre[b]):
            ring[b, tok % (2 * m)] = to_device(seqs[b][tok], dtype, DEV)
    off = torch.arange(B, dtype=torch.int64, device=DEV) * cap
    t = torch.tensor(pre, dtype=torch.int64, device=DEV)
    Bad, Bbd = to_device(Ba, dtype, DEV), to_device(Bb, dtype, DEV)
    new_rows = torch.zeros(B, 4 * c, dtype=TD[dtype], device=DEV)
    for s in range(steps):
        new_rows.copy_(to_device(np.stack([seqs[b][pre[b] + s] for b in range(B)]), dtype, DEV))
        api.csa_compress_append(new_rows, ring, Bad, Bbd, m, t, off, C)
        t += 1
    torch.cuda.synchronize()
    got = to_np64(C)
    for b in range(B):
        S = _f64(seqs[b], dtype)
        ref = O.compress(S[:, :c], S[:, c:2 * c], S[:, 2 * c:3 * c], S[:, 3 * c:], _f64(Ba, dtype), _f64(Bb, dtype), m)
        lo, hi = pre[b] // m, (pre[b] + steps) // m
        rows = got[b * cap:(b + 1) * cap]
        if hi > lo:
            assert_rows_close(rows[lo:hi], ref[lo:hi], what=f"compress_append case {i} sequence {b}")
        assert np.all(rows[:lo] == 3.0) and np.all(rows[hi:] == 3.0)
    assert torch.all(Cbig[:, c:] == 3.0)


@pytest.mark.parametrize("i", range(5))
def test_random_index_topk_varlen(i):
    rng = _rng(11, i)
    dtype = "f32" if i == 4 else "bf16"
    m = int(rng.choice([1, 2, 4, 8]))
    nhI = int(rng.integers(1, 65))
    cI = int(rng.choice([32, 64, 128, 256]))
    k = int(rng.integers(1, 300))
    lengths = [int(x) for x in rng.integers(0, 600, size=int(rng.integers(1, 6)))]
    print(f"index_topk_varlen case {i}: {dtype} m={m} nhI={nhI} cI={cI} k={k} lengths={lengths}", flush=True)
    cu, bo = _packed(lengths, m, 0)
    n, nb = int(cu[-1]), int(bo[-1])
    if n == 0:
        return
    K = _draw(rng, (max(nb, 1), cI), 1.0, dtype)
    qI = _draw(rng, (n, nhI, cI), 1.0 / math.sqrt(cI), dtype)
    wI = rng.standard_normal((n, nhI), dtype=np.float32)
    max_cand = max([(L - 1) // m for L in lengths if L > 0], default=0)
    idx = torch.full((n, k), 123456, dtype=torch.int32, device=DEV)
    qs = torch.full((n,), -5, dtype=torch.int32, device=DEV)
    api.csa_index_topk_varlen(to_device(qI, dtype, DEV), to_device(wI, "f32", DEV), to_device(K, dtype, DEV), m, k,
                              max_cand, torch.tensor(cu, device=DEV), torch.tensor(bo, device=DEV), idx,
                              q_seq_out=qs)
    torch.cuda.synchronize()
    seq_of = np.repeat(np.arange(len(lengths)), lengths)
    assert np.array_equal(qs.cpu().numpy(), seq_of)
    K64, q64 = _f64(K, dtype), _f64(qI, dtype)
    rows = []
    for t in range(n):
        b = seq_of[t]
        nc = int((t - cu[b]) // m)
        rows.append(O.index_scores_row(q64[t], wI[t].astype(np.float64), K64[bo[b]:bo[b] + nc], nc))
    check_topk(idx.cpu().numpy(), rows, k)
