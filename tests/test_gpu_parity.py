"""GPU parity: each C-ABI entry point against the oracle on the same seeded inputs.

Inputs are drawn by ``synth`` (never by the HIP side); the oracle widens the
stored values exactly to float64.  Sizes span several tiles and a ragged
tail; edge cases cover empty and short inputs.  Tolerances: see parity.py.
"""
import math

import numpy as np
import pytest
import torch

from compressed_sparse_attention_amd import api, synth
from compressed_sparse_attention_amd.layer import to_device
from oracle import csa_oracle as O
from parity import assert_rows_close, check_topk, exact_sets_equal, to_np64

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
TD = {"f32": torch.float32, "bf16": torch.bfloat16}


def draw(rng, shape, std, dtype):
    x = rng.standard_normal(size=shape, dtype=np.float32) * np.float32(std)
    return synth.f32_to_bf16(x) if dtype == "bf16" else x


def f64(x, dtype):
    return synth.to_f64(x, dtype)


# ---------------------------------------------------------------------------
# projections (eqs 1, 2, 5, 6, 7, 10)
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("din,dout,M,N,K", [
    ("f32", "f32", 512, 512, 256),
    ("f32", "f32", 77, 40, 24),
    ("bf16", "bf16", 300, 200, 136),
    ("bf16", "f32", 130, 64, 4096),
    ("bf16", "bf16", 1000, 1536, 4096),
    ("bf16", "bf16", 520, 296, 200),  # large-tile kernel: ragged M and N edges and a K tail
    ("bf16", "f32", 260, 264, 1000),
    # K a multiple of 64: the copy-pipelined large-tile kernel (two stages up to many, ragged edges)
    ("bf16", "bf16", 256, 256, 64),
    ("bf16", "bf16", 520, 296, 192),
    ("bf16", "f32", 260, 260, 1024),
    ("bf16", "bf16", 777, 1032, 1536),
    # the copy-pipelined kernel: four 32-deep stages (one more than its ring holds), twelve with ragged
    # edges, thirty-two on one whole tile
    ("bf16", "bf16", 300, 264, 128),
    ("bf16", "bf16", 513, 520, 384),
    ("bf16", "bf16", 256, 256, 1024),
    ("bf16", "bf16", 8, 4096, 4096),  # few-row (decode token) kernel
    ("bf16", "f32", 3, 64, 200),
    ("bf16", "bf16", 16, 1000, 1536),
    ("bf16", "bf16", 1, 40, 8),
    # few rows, short K, many columns: 64-column workgroups over all of K (a ragged last block, a K tail)
    ("bf16", "bf16", 8, 32768, 1536),
    ("bf16", "f32", 5, 16392, 1000),
])
def test_project(din, dout, M, N, K):
    rng = synth.rng_for(M * 7 + N)
    X = draw(rng, (M, K), 1.0, din)
    W = draw(rng, (K, N), 1.0 / math.sqrt(K), din)
    Xd = to_device(X, din, DEV)
    Wt = to_device(np.ascontiguousarray(W.T), din, DEV)
    Y = torch.empty(M, N, dtype=TD[dout], device=DEV)
    api.csa_project(Xd, Wt, Y)
    torch.cuda.synchronize()
    assert_rows_close(to_np64(Y), O.project(f64(X, din), f64(W, din)), what="project")


@pytest.mark.parametrize("din,d1,d2,M,N1,N2,K", [
    ("bf16", "bf16", "f32", 8, 4096, 64, 4096),    # one launch: a stacked H-side weight with the w^I head weights
    ("bf16", "bf16", "bf16", 8, 1000, 264, 1536),  # one launch, ragged column blocks in both products
    ("bf16", "f32", "bf16", 3, 40, 24, 200),       # one launch, K tail
    # 64-column workgroups over all of K (the decode query side: eq 10 and eq 6 weights, d_c = 1536)
    ("bf16", "bf16", "bf16", 8, 32768, 8192, 1536),
    # the same kernel with ragged column blocks in both products, a K tail inside a super-step, 5 rows
    ("bf16", "bf16", "f32", 5, 12344, 4104, 1000),
    ("bf16", "bf16", "bf16", 16, 16000, 400, 1920),  # 16 rows, the largest K it takes
    # the waves splitting K over d-long rows: 3 rows, a K tail inside a super-step, ragged column blocks
    ("bf16", "bf16", "f32", 3, 296, 40, 2200),
    ("bf16", "bf16", "bf16", 8, 520, 16, 4096),
    ("bf16", "bf16", "f32", 40, 296, 64, 200),     # more than 16 rows: two launches
    ("f32", "f32", "f32", 5, 48, 16, 24),
])
def test_project_pair(din, d1, d2, M, N1, N2, K):
    """Both products of csa_project_pair against the oracle's projection."""
    rng = synth.rng_for(M * 11 + N1 + 3 * N2)
    X = draw(rng, (M, K), 1.0, din)
    W1 = draw(rng, (K, N1), 1.0 / math.sqrt(K), din)
    W2 = draw(rng, (K, N2), 1.0 / math.sqrt(K), din)
    Xd = to_device(X, din, DEV)
    Wt1 = to_device(np.ascontiguousarray(W1.T), din, DEV)
    Wt2 = to_device(np.ascontiguousarray(W2.T), din, DEV)
    Y1 = torch.empty(M, N1, dtype=TD[d1], device=DEV)
    Y2 = torch.empty(M, N2, dtype=TD[d2], device=DEV)
    api.csa_project_pair(Xd, Wt1, Y1, Wt2, Y2)
    torch.cuda.synchronize()
    assert_rows_close(to_np64(Y1), O.project(f64(X, din), f64(W1, din)), what="project_pair Y1")
    assert_rows_close(to_np64(Y2), O.project(f64(X, din), f64(W2, din)), what="project_pair Y2")


@pytest.mark.parametrize("din,dout,M,N,K", [
    ("f32", "f32", 77, 40, 24),          # token count not a multiple of 8 (zero-padded contraction)
    ("bf16", "bf16", 1000, 1536, 4096),  # large-tile kernels for both products
    ("bf16", "f32", 130, 64, 200),
    ("bf16", "bf16", 8, 4096, 4096),     # few-row kernel for dX
    ("bf16", "bf16", 3, 64, 200),
])
def test_project_backward(din, dout, M, N, K):
    """dX = dY W^T and dW^T = dY^T X against the oracle's gradients of Y = X W."""
    rng = synth.rng_for(M * 5 + N + K)
    X = draw(rng, (M, K), 1.0, din)
    W = draw(rng, (K, N), 1.0 / math.sqrt(K), din)
    dY = draw(rng, (M, N), 1.0, din)
    Xd, dYd = to_device(X, din, DEV), to_device(dY, din, DEV)
    Wt = to_device(np.ascontiguousarray(W.T), din, DEV)
    dX = torch.full((M, K), 7.0, dtype=TD[dout], device=DEV)
    dWt = torch.full((N, K), 7.0, dtype=TD[dout], device=DEV)
    api.csa_project_backward(Xd, Wt, dYd, dX, dWt)
    torch.cuda.synchronize()
    ref_dX, ref_dW = O.project_backward(f64(X, din), f64(W, din), f64(dY, din))
    assert_rows_close(to_np64(dX), ref_dX, what="dX")
    assert_rows_close(to_np64(dWt), ref_dW.T, what="dWt")


@pytest.mark.parametrize("M,K,N", [(257, 128, 96), (300, 128, 264)])
def test_project_strided_views(M, K, N):
    """Input column slice (ldx > K) and output column slice of a wider buffer (ldy > N)."""
    rng = synth.rng_for(99 + M)
    X = draw(rng, (M, 3 * K), 1.0, "bf16")
    W = draw(rng, (K, N), 0.1, "bf16")
    Xd = to_device(X, "bf16", DEV)
    Wt = to_device(np.ascontiguousarray(W.T), "bf16", DEV)
    Ybig = torch.full((M, 4 * N), 7.0, dtype=torch.bfloat16, device=DEV)
    api.csa_project(Xd[:, K:2 * K], Wt, Ybig[:, N:2 * N])
    torch.cuda.synchronize()
    ref = O.project(f64(X, "bf16")[:, K:2 * K], f64(W, "bf16"))
    assert_rows_close(to_np64(Ybig[:, N:2 * N]), ref, what="project slice")
    untouched = torch.cat([Ybig[:, :N], Ybig[:, 2 * N:]], 1)
    assert torch.all(untouched == 7.0)


def test_project_output_half_chunk():
    """bf16 output with N % 8 == 4 (possible only with ldy > N): the last 4 columns of each row are a half
    16-byte chunk; the columns between N and ldy keep their sentinel."""
    rng = synth.rng_for(123)
    M, K, N = 300, 128, 260
    X = draw(rng, (M, K), 1.0, "bf16")
    W = draw(rng, (K, N), 0.1, "bf16")
    Ybig = torch.full((M, N + 4), 7.0, dtype=torch.bfloat16, device=DEV)
    api.csa_project(to_device(X, "bf16", DEV), to_device(np.ascontiguousarray(W.T), "bf16", DEV), Ybig[:, :N])
    torch.cuda.synchronize()
    assert_rows_close(to_np64(Ybig[:, :N]), O.project(f64(X, "bf16"), f64(W, "bf16")), what="project")
    assert torch.all(Ybig[:, N:] == 7.0)


# ---------------------------------------------------------------------------
# compression (eqs 3-4)
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("dtype,n,m,c", [
    ("f32", 512, 4, 64), ("f32", 514, 4, 32), ("bf16", 1000, 4, 512), ("bf16", 999, 8, 128),
    ("bf16", 64, 1, 512), ("bf16", 37, 2, 12), ("bf16", 3, 4, 64),
])
def test_compress(dtype, n, m, c):
    """Ca, Cb, Za, Zb are column slices of one projection buffer (slices start on 16-byte boundaries)."""
    rng = synth.rng_for(n + m + c)
    cp = (c + 7) // 8 * 8  # slice spacing keeps every slice 16-byte aligned
    P = draw(rng, (n, 4 * cp), 1.0, dtype)
    Pz = draw(rng, (n, 4 * cp), 2.0, dtype)  # logits with spread so the softmax is not flat
    P = np.where((np.arange(4 * cp) // cp)[None, :] >= 2, Pz, P)
    Ba = draw(rng, (m, c), 0.5, dtype)
    Bb = draw(rng, (m, c), 0.5, dtype)
    Pd = to_device(P, dtype, DEV)
    out = torch.full((n // m, cp), 3.0, dtype=TD[dtype], device=DEV)[:, :c]  # rows padded to 16 bytes
    sl = [Pd[:, i * cp:i * cp + c] for i in range(4)]
    api.csa_compress(*sl, to_device(Ba, dtype, DEV), to_device(Bb, dtype, DEV), m, out)
    torch.cuda.synchronize()
    P64 = f64(P, dtype)
    parts = [P64[:, i * cp:i * cp + c] for i in range(4)]
    ref = O.compress(*parts, f64(Ba, dtype), f64(Bb, dtype), m)
    if n // m:
        assert_rows_close(to_np64(out), ref, what="compress")


def test_compress_mean_pool_exact():
    """Equal logits and B = 0: mean pooling; integer values and m = 4 make fp32 exact."""
    rng = synth.rng_for(5)
    n, m, c = 256, 4, 64
    C = rng.integers(-50, 50, size=(n, 2 * c)).astype(np.float32)
    Z = np.full((n, 2 * c), 0.75, dtype=np.float32)
    P = np.concatenate([C, Z], 1)
    B = np.zeros((m, c), np.float32)
    Pd = to_device(P, "f32", DEV)
    out = torch.empty(n // m, c, dtype=torch.float32, device=DEV)
    Bd = to_device(B, "f32", DEV)
    api.csa_compress(Pd[:, 0:c], Pd[:, c:2 * c], Pd[:, 2 * c:3 * c], Pd[:, 3 * c:], Bd, Bd, m, out)
    torch.cuda.synchronize()
    ref = O.compress(P[:, :c], P[:, c:2 * c], P[:, 2 * c:3 * c], P[:, 3 * c:], B, B, m)
    assert np.array_equal(out.cpu().numpy().astype(np.float64), ref)


@pytest.mark.parametrize("dtype,n,m,c", [
    ("f32", 64, 4, 64), ("bf16", 1030, 4, 512), ("bf16", 37, 8, 12), ("f32", 3, 4, 16), ("bf16", 4, 4, 64),
    ("f32", 2000, 16, 40), ("bf16", 9000, 1, 128), ("bf16", 0, 4, 64), ("bf16", 70001, 4, 512),
])
def test_compress_backward(dtype, n, m, c):
    """Gradients of eqs 3-4: inputs and outputs are column slices of [n, 4c'] buffers (as the forward
    projection lays them out); the output buffer starts full of a sentinel, so every row must be written."""
    rng = synth.rng_for(3 * n + m + c)
    cp = (c + 7) // 8 * 8
    P = draw(rng, (n, 4 * cp), 1.0, dtype)
    Pz = draw(rng, (n, 4 * cp), 2.0, dtype)
    P = np.where((np.arange(4 * cp) // cp)[None, :] >= 2, Pz, P)
    Ba = draw(rng, (m, c), 0.5, dtype)
    Bb = draw(rng, (m, c), 0.5, dtype)
    N = n // m
    dC = rng.standard_normal(size=(N, cp), dtype=np.float32)
    Pd = to_device(P, dtype, DEV)
    sl = [Pd[:, i * cp:i * cp + c] for i in range(4)]
    dCd = torch.from_numpy(dC).to(DEV)[:, :c]
    G = torch.full((n, 4 * cp), 7.0, dtype=TD[dtype], device=DEV)
    gs = [G[:, i * cp:i * cp + c] for i in range(4)]
    dBa = torch.full((m, c), 7.0, device=DEV)
    dBb = torch.full((m, c), 7.0, device=DEV)
    api.csa_compress_backward(*sl, to_device(Ba, dtype, DEV), to_device(Bb, dtype, DEV), m, dCd, *gs, dBa, dBb)
    torch.cuda.synchronize()
    P64 = f64(P, dtype)
    parts = [P64[:, i * cp:i * cp + c] for i in range(4)]
    if n > 20000:  # the oracle on sampled blocks: blocks 0, 1, a middle one and the last two, plus the tail
        blocks = sorted({0, 1, N // 2, N - 2, N - 1})
        for i in blocks:
            lo = max(i - 1, 0) * m
            hi = min((i + 2) * m, n)  # block i's rows, the rows feeding it, and the next block (b-gradients)
            sub = [x[lo:hi] for x in parts]
            j = i - lo // m
            dsub = np.zeros((hi // m - lo // m, c))
            dsub[j] = dC[i, :c]
            ref = O.compress_backward(*sub, f64(Ba, dtype), f64(Bb, dtype), m, dsub)
            # rows of block i: a-gradients from block i alone (dsub is zero for its neighbours)
            a0, a1 = i * m - lo, (i + 1) * m - lo
            for w, gi in ((0, 0), (2, 2)):
                assert_rows_close(to_np64(gs[gi][i * m:(i + 1) * m]), ref[w][a0:a1], what=f"block {i} a-grad {gi}")
            if i > 0:  # block i's b-gradients land on block i-1's rows
                b0, b1 = (i - 1) * m - lo, i * m - lo
                for w, gi in ((1, 1), (3, 3)):
                    got = to_np64(gs[gi][(i - 1) * m:i * m])
                    assert_rows_close(got, ref[w][b0:b1], what=f"block {i} b-grad {gi}")
        tail = to_np64(G[N * m:])
        assert np.all(tail[:, :c] == 0) and np.all(tail[:, 2 * cp:2 * cp + c] == 0)
        assert np.all(to_np64(G[(N - 1) * m:])[:, cp:cp + c] == 0)
        # the bias gradients: the per-position sums of the dZ rows the GPU wrote (a property that holds at any
        # size), recomputed in float64 from the GPU's own per-row gradients
        dZa = to_np64(gs[2])[:N * m].reshape(N, m, c)
        dZb = to_np64(gs[3])[:(N - 1) * m].reshape(N - 1, m, c)
        for got, want, mag in ((dBa, dZa.sum(0), np.abs(dZa).sum(0)), (dBb, dZb.sum(0), np.abs(dZb).sum(0))):
            err = np.abs(to_np64(got) - want)
            assert np.all(err <= 1e-2 * mag + 1e-6), f"bias gradient off by {err.max()}"
        return
    ref = O.compress_backward(*parts, f64(Ba, dtype), f64(Bb, dtype), m, dC[:, :c].astype(np.float64))
    for w in range(4):
        got = to_np64(gs[w])
        if n:
            assert_rows_close(got, ref[w], what=f"grad {w}")
    # bias gradients: error bounded relative to the sum of the magnitudes of the terms they add up
    mag_a = np.abs(ref[2][:N * m]).reshape(N, m, c).sum(0) if N else np.zeros((m, c))
    mag_b = np.abs(ref[3][:(N - 1) * m]).reshape(N - 1, m, c).sum(0) if N > 1 else np.zeros((m, c))
    tol = 1e-5 if dtype == "f32" else 1e-4
    for got, want, mag in ((dBa, ref[4], mag_a), (dBb, ref[5], mag_b)):
        err = np.abs(to_np64(got) - want)
        assert np.all(err <= tol * mag + 1e-7), f"bias gradient off by {err.max()}"
    if n:  # the padding columns between the slices are untouched
        pad = to_np64(G).reshape(n, 4, cp)[:, :, c:]
        assert np.all(pad == 7.0)


# ---------------------------------------------------------------------------
# indexer + top-k (eqs 8-9)
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("dtype,m,c,steps", [
    ("f32", 4, 64, 23), ("bf16", 4, 512, 21), ("bf16", 1, 128, 7), ("bf16", 8, 12, 40), ("f32", 64, 16, 140),
    ("bf16", 2, 2560, 5), ("f32", 4, 1100, 9),
])
def test_compress_append(dtype, m, c, steps):
    """One token per sequence per call: three sequences that already hold 0, 5 and 2m + 3 tokens (ring
    holding their last 2m rows) grow by `steps` tokens; the rows the appends write must equal the oracle's
    compression of each whole sequence, and every other cache row stays untouched."""
    rng = synth.rng_for(m * 1000 + c)
    pre = [0, 5, 2 * m + 3]
    B = len(pre)
    cp = (c + 7) // 8 * 8
    seqs = []
    for b in range(B):
        n = pre[b] + steps
        Y = draw(rng, (n, 4 * c), 1.0, dtype)
        Yz = draw(rng, (n, 4 * c), 2.0, dtype)
        seqs.append(np.where((np.arange(4 * c) // c)[None, :] >= 2, Yz, Y))
    Ba = draw(rng, (m, c), 0.5, dtype)
    Bb = draw(rng, (m, c), 0.5, dtype)
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
    wide = torch.zeros(B, 4 * c + 8, dtype=TD[dtype], device=DEV)  # new rows are a column slice
    for s in range(steps):
        wide[:, :4 * c] = to_device(np.stack([seqs[b][pre[b] + s] for b in range(B)]), dtype, DEV)
        api.csa_compress_append(wide[:, :4 * c], ring, Bad, Bbd, m, t, off, C)
        t += 1
    torch.cuda.synchronize()
    got = to_np64(C)
    for b in range(B):
        S = f64(seqs[b], dtype)
        ref = O.compress(S[:, :c], S[:, c:2 * c], S[:, 2 * c:3 * c], S[:, 3 * c:], f64(Ba, dtype), f64(Bb, dtype), m)
        lo, hi = pre[b] // m, (pre[b] + steps) // m
        rows = got[b * cap:(b + 1) * cap]
        assert_rows_close(rows[lo:hi], ref[lo:hi], what=f"appended rows of sequence {b}")
        assert np.all(rows[:lo] == 3.0) and np.all(rows[hi:] == 3.0)
    assert torch.all(Cbig[:, c:] == 3.0)


@pytest.mark.parametrize("dtype,m,c1,c2", [("bf16", 4, 512, 128), ("f32", 3, 64, 20), ("bf16", 1, 36, 64)])
def test_compress_append_pair_equals_two_calls(dtype, m, c1, c2):
    """csa_compress_append_pair on a main and an indexer cache of the same sequences gives, step after step,
    exactly the caches and rings of two csa_compress_append calls (tokens that complete a block and tokens
    that do not, sequences at different positions)."""
    rng = synth.rng_for(m * 7 + c1 + c2)
    pre = [0, 5, 2 * m + 3, 1]
    B, steps = len(pre), 3 * m + 1
    cap = max(pre) // m + steps // m + 2
    off = torch.arange(B, dtype=torch.int64, device=DEV) * cap
    t1 = torch.tensor(pre, dtype=torch.int64, device=DEV)
    t2 = t1.clone()
    caches = []
    for c in (c1, c2):
        Ba = to_device(draw(rng, (m, c), 0.5, dtype), dtype, DEV)
        Bb = to_device(draw(rng, (m, c), 0.5, dtype), dtype, DEV)
        ring = to_device(draw(rng, (B, 2 * m, 4 * c), 1.0, dtype), dtype, DEV)
        cp = (c + 7) // 8 * 8  # cache rows padded to 16 bytes; the cache is a column slice
        C = torch.full((B * cap, cp), 3.0, dtype=TD[dtype], device=DEV)[:, :c]
        C2 = torch.full((B * cap, cp), 3.0, dtype=TD[dtype], device=DEV)[:, :c]
        caches.append((c, Ba, Bb, ring, C, ring.clone(), C2))
    wide = 4 * c1 + 4 * c2 + 8
    for s in range(steps):
        Y = to_device(draw(rng, (B, wide), 1.5, dtype), dtype, DEV)
        (ca, Baa, Bba, ra, Ca, ra2, Ca2), (cb, Bab, Bbb, rb, Cb, rb2, Cb2) = caches
        api.csa_compress_append_pair(Y[:, :4 * ca], ra, Baa, Bba, Ca, Y[:, 4 * ca:4 * ca + 4 * cb], rb, Bab, Bbb, Cb,
                                     m, t1, off)
        api.csa_compress_append(Y[:, :4 * ca], ra2, Baa, Bba, m, t2, off, Ca2)
        api.csa_compress_append(Y[:, 4 * ca:4 * ca + 4 * cb], rb2, Bab, Bbb, m, t2, off, Cb2)
        t1 += 1
        t2 += 1
        torch.cuda.synchronize()
        for x, (c, _, _, r, C, r2, C2) in enumerate(caches):
            assert torch.equal(r, r2) and torch.equal(C, C2), f"step {s}, cache {x + 1}"


def _run_index_topk(qI, wI, K, m, k, lens, kv_offset, dtype, prefill_mode=False):
    B = qI.shape[0]
    idx = torch.full((B, k), 123456, dtype=torch.int32, device=DEV)
    sc = torch.empty(B, k, dtype=torch.float32, device=DEV)
    if prefill_mode:
        max_cand = B // m
        api.csa_index_topk(to_device(qI, dtype, DEV), to_device(wI, "f32", DEV), to_device(K, dtype, DEV), m, k,
                           max_cand, idx, score_out=sc)
    else:
        max_cand = int(max(lens) // m) if len(lens) else 0
        api.csa_index_topk(to_device(qI, dtype, DEV), to_device(wI, "f32", DEV), to_device(K, dtype, DEV), m, k,
                           max_cand, idx, score_out=sc,
                           q_seq=torch.arange(B, dtype=torch.int32, device=DEV),
                           q_pos=torch.tensor(lens, dtype=torch.int64, device=DEV),
                           kv_offset=torch.tensor(kv_offset, dtype=torch.int64, device=DEV))
    torch.cuda.synchronize()
    return idx.cpu().numpy(), sc.cpu().numpy().astype(np.float64)


def _decode_case(rng, lens, m, nhI, cI, dtype):
    lens = np.asarray(lens, np.int64)
    nblk = lens // m
    off = np.zeros_like(nblk)
    off[1:] = np.cumsum(nblk)[:-1]
    rows = max(int(nblk.sum()), 1)
    K = draw(rng, (rows, cI), 1.0, dtype)
    qI = draw(rng, (len(lens), nhI, cI), 1.0 / math.sqrt(cI), dtype)
    wI = rng.standard_normal((len(lens), nhI), dtype=np.float32)
    return lens, off, K, qI, wI


def _oracle_rows(qI, wI, K, lens, off, m, dtype):
    K64 = f64(K, dtype)
    rows = []
    for b in range(len(lens)):
        nc = int(lens[b] // m)
        rows.append(O.index_scores_row(f64(qI[b], dtype), wI[b].astype(np.float64), K64[off[b]:off[b] + nc], nc))
    return rows


@pytest.mark.parametrize("dtype,lens,m,nhI,cI,k", [
    ("bf16", [0, 7, 100, 2051, 8195, 4096], 4, 64, 128, 64),
    ("bf16", [9000, 1024, 30000], 8, 32, 128, 256),
    ("f32", [512, 3, 64, 200], 4, 4, 32, 16),
    ("bf16", [2048 * 4, 2048 * 4], 4, 64, 128, 512),
    ("bf16", [777, 5000], 4, 20, 64, 33),
    ("bf16", [4 * 20000, 4 * 9000, 4 * 12345, 4 * 32768], 4, 64, 128, 1000),  # indexer-built histogram
    ("bf16", [4 * 40000, 4 * 70000], 4, 64, 128, 2048),  # rows longer than the LDS row cache
    ("bf16", [0, 100, 4 * 9000, 4 * 33000, 4 * 1500], 4, 64, 128, 1024),  # rows of 0..17 chunks
])
def test_index_topk_decode(dtype, lens, m, nhI, cI, k):
    rng = synth.rng_for(sum(lens) + k)
    lens, off, K, qI, wI = _decode_case(rng, lens, m, nhI, cI, dtype)
    idx, sc = _run_index_topk(qI, wI, K, m, k, lens, off, dtype)
    rows = _oracle_rows(qI, wI, K, lens, off, m, dtype)
    check_topk(idx, rows, k)
    for b, s in enumerate(rows):  # returned scores are the selected candidates' scores
        if s.size == 0:
            assert np.all(idx[b] == -1) and np.all(np.isneginf(sc[b]))
            continue
        sel = idx[b][idx[b] >= 0]
        got = sc[b][idx[b] >= 0]
        assert np.allclose(got, s[sel], rtol=1e-3, atol=1e-4 * (np.abs(s).max() + 1e-30))
        assert np.all(np.isneginf(sc[b][idx[b] < 0]))


def test_index_topk_many_long_rows_shared_sequence():
    """520 queries at different positions of one 16384-block sequence: too many rows for the
    per-chunk selector's lists, so each row is selected by one workgroup from the sweep's histogram.
    The same workspace is used twice in a row."""
    rng = synth.rng_for(520)
    cI, nhI, m, k, nb = 32, 2, 4, 300, 16384
    K = draw(rng, (nb, cI), 1.0, "bf16")
    B = 520
    pos = rng.integers(4 * 8200, 4 * nb + 1, size=B).astype(np.int64)
    qI = draw(rng, (B, nhI, cI), 1.0 / math.sqrt(cI), "bf16")
    wI = rng.standard_normal((B, nhI), dtype=np.float32)
    ws = torch.zeros(api.csa_index_topk_workspace(B, nb, nhI, k), dtype=torch.uint8, device=DEV)
    args = dict(q_seq=torch.zeros(B, dtype=torch.int32, device=DEV), q_pos=torch.tensor(pos, device=DEV),
                kv_offset=torch.zeros(1, dtype=torch.int64, device=DEV), workspace=ws)
    qd, wd, Kd = to_device(qI, "bf16", DEV), to_device(wI, "f32", DEV), to_device(K, "bf16", DEV)
    K64 = f64(K, "bf16")
    rows = [O.index_scores_row(f64(qI[b], "bf16"), wI[b].astype(np.float64), K64[:pos[b] // m], int(pos[b] // m))
            for b in range(B)]
    for _ in range(2):
        idx = torch.full((B, k), 123456, dtype=torch.int32, device=DEV)
        api.csa_index_topk(qd, wd, Kd, m, k, nb, idx, **args)
        torch.cuda.synchronize()
        check_topk(idx.cpu().numpy(), rows, k)


@pytest.mark.parametrize("nhI,wset", [(1, (1.0,)), (8, (-1.0, 0.5, 2.0)), (64, (-2.0, -0.5, 0.0, 1.0, 3.0))])
def test_index_topk_exact_ties(nhI, wset):
    """Small-integer inputs make every fp32 score exact: sets must equal the oracle's exactly,
    including the lower-index tie-break and -0.0 == +0.0."""
    rng = synth.rng_for(nhI)
    cI, m, k = 64, 4, 40
    lens = np.array([4 * 600, 4 * 41, 4 * 1000], np.int64)
    nblk = lens // m
    off = np.concatenate([[0], np.cumsum(nblk)[:-1]])
    K = synth.f32_to_bf16(rng.integers(-2, 3, size=(int(nblk.sum()), cI)).astype(np.float32))
    qI = synth.f32_to_bf16(rng.integers(-1, 2, size=(3, nhI, cI)).astype(np.float32))
    wI = rng.choice(np.array(wset, np.float32), size=(3, nhI))
    idx, _ = _run_index_topk(qI, wI, K, m, k, lens, off, "bf16")
    rows = _oracle_rows(qI, wI, K, lens, off, m, "bf16")
    exact_sets_equal(idx, O.topk_rows(rows, k))


@pytest.mark.parametrize("lens,k", [
    ([4 * 20000, 4 * 30000], 15000),  # k-th score is 0: > 4096 candidates share the threshold bin
    ([4 * 40000], 22000),  # same, on a row longer than the LDS row cache
    ([4 * 3000, 4 * 7000], 2500),  # short rows: histogram built by the selector itself
])
def test_index_topk_many_ties_long_rows(lens, k):
    """One head with w = 1 and integer dots: about half the scores are exactly 0, so the
    threshold bin is huge and the lower-index tie-break decides thousands of slots."""
    rng = synth.rng_for(len(lens) * 1000 + k)
    cI, m = 32, 4
    lens = np.array(lens, np.int64)
    nblk = lens // m
    off = np.concatenate([[0], np.cumsum(nblk)[:-1]])
    K = synth.f32_to_bf16(rng.integers(-2, 3, size=(int(nblk.sum()), cI)).astype(np.float32))
    qI = synth.f32_to_bf16(rng.integers(-1, 2, size=(len(lens), 1, cI)).astype(np.float32))
    wI = np.ones((len(lens), 1), np.float32)
    idx, _ = _run_index_topk(qI, wI, K, m, k, lens, off, "bf16")
    rows = _oracle_rows(qI, wI, K, lens, off, m, "bf16")
    exact_sets_equal(idx, O.topk_rows(rows, k))


@pytest.mark.parametrize("dtype,n,m,nhI,cI,k", [
    ("f32", 512, 4, 4, 32, 16), ("bf16", 1000, 4, 64, 128, 64), ("bf16", 333, 2, 16, 64, 8),
])
def test_index_topk_prefill(dtype, n, m, nhI, cI, k):
    rng = synth.rng_for(n + nhI)
    K = draw(rng, (n // m, cI), 1.0, dtype)
    qI = draw(rng, (n, nhI, cI), 1.0 / math.sqrt(cI), dtype)
    wI = rng.standard_normal((n, nhI), dtype=np.float32)
    idx, _ = _run_index_topk(qI, wI, K, m, k, None, None, dtype, prefill_mode=True)
    K64 = f64(K, dtype)
    rows = [O.index_scores_row(f64(qI[t], dtype), wI[t].astype(np.float64), K64, t // m) for t in range(n)]
    check_topk(idx, rows, k)


def _run_stream(qI, wI, K, m, k, dtype, max_cand):
    n = qI.shape[0]
    qd, Kd = to_device(qI, dtype, DEV), to_device(K, dtype, DEV)
    wd = torch.from_numpy(np.ascontiguousarray(wI)).to(DEV)
    idx = torch.full((n, k), 123456, dtype=torch.int32, device=DEV)
    sc = torch.full((n, k), 7.0, dtype=torch.float32, device=DEV)
    api.csa_index_topk_stream(qd, wd, Kd, m, k, max_cand, idx, score_out=sc)
    torch.cuda.synchronize()
    return idx.cpu().numpy(), sc.cpu().numpy()


def _check_stream_rows(idx, sc, rows, k):
    """Each row: a valid selection (the comparison rules), listed in increasing index order, -1 after it,
    and score_out = the oracle's score of each listed index (fp32 rounding)."""
    check_topk(idx, rows, k)
    for t, row in enumerate(rows):
        sel = idx[t][idx[t] >= 0]
        assert np.all(np.diff(sel) > 0), f"row {t}: not in index order"
        assert np.all(idx[t][len(sel):] == -1)
        if sel.size:
            ref = row[sel]
            assert np.allclose(sc[t][:len(sel)], ref, rtol=1e-4, atol=1e-5 * np.abs(row).max()), f"row {t}: scores"
        assert np.all(np.isneginf(sc[t][len(sel):]))


@pytest.mark.parametrize("dtype,n,m,nhI,cI,k", [
    ("f32", 512, 4, 4, 32, 16),      # the fp32 prefill workload's shapes
    ("bf16", 1000, 4, 64, 128, 64),  # the 32768-token layer's widths on 1000 tokens
    ("bf16", 333, 2, 16, 64, 8),
    ("bf16", 4100, 1, 8, 32, 700),   # rows up to 4099 candidates: thresholds rise late
    ("bf16", 9000, 1, 4, 64, 40),    # lists longer than one 8192-entry segment
])
def test_index_topk_stream(dtype, n, m, nhI, cI, k):
    """Streaming selection (no causal score matrix) against the oracle's eq 8 scores: valid selections,
    in index order, with their scores."""
    rng = synth.rng_for(7 * n + nhI)
    K = draw(rng, (n // m, cI), 1.0, dtype)
    qI = draw(rng, (n, nhI, cI), 1.0 / math.sqrt(cI), dtype)
    wI = rng.standard_normal((n, nhI), dtype=np.float32)
    idx, sc = _run_stream(qI, wI, K, m, k, dtype, n // m)
    K64 = f64(K, dtype)
    rows = [O.index_scores_row(f64(qI[t], dtype), wI[t].astype(np.float64), K64, t // m) for t in range(n)]
    _check_stream_rows(idx, sc, rows, k)


@pytest.mark.parametrize("nhI,wset,k", [(1, (1.0,), 40), (8, (-1.0, 0.5, 2.0), 40), (64, (-2.0, 0.0, 1.0, 3.0), 40),
                                        (1, (1.0,), 900)])
def test_index_topk_stream_exact_ties(nhI, wset, k):
    """Small-integer inputs make every fp32 score exact: the streaming selection must equal the oracle's
    set exactly (lower-index tie-break, -0.0 == +0.0), also when most scores tie at the threshold (one head,
    w = 1: half the scores are exactly 0)."""
    rng = synth.rng_for(31 * nhI + k)
    cI, m, n = 64, 4, 4000
    K = synth.f32_to_bf16(rng.integers(-2, 3, size=(n // m, cI)).astype(np.float32))
    qI = synth.f32_to_bf16(rng.integers(-1, 2, size=(n, nhI, cI)).astype(np.float32))
    wI = rng.choice(np.array(wset, np.float32), size=(n, nhI))
    idx, sc = _run_stream(qI, wI, K, m, k, "bf16", n // m)
    K64 = f64(K, "bf16")
    rows = [O.index_scores_row(f64(qI[t], "bf16"), wI[t].astype(np.float64), K64, t // m) for t in range(n)]
    exact_sets_equal(idx, O.topk_rows(rows, k))
    _check_stream_rows(idx, sc, rows, k)


def test_index_topk_stream_same_sets_as_dense():
    """The streaming and the materialised paths select the same sets on the same inputs (integer inputs:
    exact scores, so no band-exempt differences are possible)."""
    rng = synth.rng_for(4242)
    n, m, nhI, cI, k = 3000, 4, 16, 64, 100
    K = synth.f32_to_bf16(rng.integers(-3, 4, size=(n // m, cI)).astype(np.float32))
    qI = synth.f32_to_bf16(rng.integers(-2, 3, size=(n, nhI, cI)).astype(np.float32))
    wI = rng.choice(np.array((-1.0, 0.25, 1.0, 2.0), np.float32), size=(n, nhI))
    idx_s, _ = _run_stream(qI, wI, K, m, k, "bf16", n // m)
    idx_d, _ = _run_index_topk(qI, wI, K, m, k, None, None, "bf16", prefill_mode=True)
    exact_sets_equal(idx_s, idx_d)


# ---------------------------------------------------------------------------
# sparse MQA (eq 11)
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("dtype,B,nh,c,k,nblk,qmult,layout", [
    ("bf16", 4, 64, 512, 512, 3000, 1.0, "prefix"),
    ("bf16", 3, 64, 512, 100, 700, 8.0, "prefix"),
    ("bf16", 2, 128, 512, 256, 400, 32.0, "prefix"),
    ("f32", 5, 8, 64, 16, 128, 1.0, "prefix"),
    ("bf16", 3, 20, 128, 70, 90, 4.0, "prefix"),
    ("bf16", 600, 64, 512, 200, 300, 4.0, "prefix"),
    ("f32", 530, 8, 64, 70, 40, 2.0, "prefix"),
    ("bf16", 64, 64, 512, 1024, 1500, 8.0, "prefix"),  # several 128-row chunks per split
    ("bf16", 520, 128, 256, 130, 500, 2.0, "prefix"),  # long batch, two 64-head groups, c = 256
    ("bf16", 512, 20, 128, 200, 260, 1.0, "prefix"),  # long batch, partial head tile, c = 128
    # long batch, selections of every length 0 .. 700 (trailing chunks of -1 slots are skipped)
    ("bf16", 560, 64, 512, 512, 700, 2.0, "ragged"),
    # -1 slots scattered between valid ones (no prefix: every chunk is walked)
    ("bf16", 560, 64, 512, 512, 700, 2.0, "scatter"),
    ("bf16", 4, 64, 512, 512, 700, 2.0, "scatter"),
    # long batch, c = 512, a partial head group (20 heads) and k not a multiple of the 64-slot chunk
    ("bf16", 600, 20, 512, 96, 120, 2.0, "scatter"),
    ("bf16", 530, 100, 512, 200, 250, 4.0, "ragged"),  # two head groups, the second partial
    ("bf16", 520, 192, 512, 128, 200, 2.0, "ragged"),  # three head groups of one query in different workgroups
    # short batches of many queries (16-head tiles over several rounds), partial head tiles, c = 512, 256, 128
    ("bf16", 200, 20, 512, 300, 400, 2.0, "scatter"),
    ("bf16", 40, 40, 256, 400, 500, 4.0, "ragged"),
    ("bf16", 100, 64, 128, 300, 350, 1.0, "prefix"),
])
def test_sparse_mqa(dtype, B, nh, c, k, nblk, qmult, layout):
    rng = synth.rng_for(B * nh + k)
    C = draw(rng, (B * nblk, c), 1.0, dtype)
    q = draw(rng, (B, nh, c), qmult / math.sqrt(c), dtype)
    ncand = np.full(B, nblk)
    ncand[-1] = 0  # one query with nothing selected
    if B > 2:
        ncand[1] = min(nblk, k // 2 + 1)  # a short selection padded with -1
    if layout != "prefix":
        ncand = rng.integers(0, nblk + 1, size=B)
        ncand[0] = 0
    idx = synth.random_selection(rng, ncand, k)
    if layout == "scatter":
        idx = np.stack([rng.permutation(row) for row in idx])
    off = np.arange(B, dtype=np.int64) * nblk
    o = torch.full((B, nh, c), 5.0, dtype=TD[dtype], device=DEV)
    lse = torch.empty(B, nh, dtype=torch.float32, device=DEV)
    scale = 1.0 / math.sqrt(c)
    api.csa_sparse_mqa(to_device(q, dtype, DEV), to_device(C, dtype, DEV),
                       torch.from_numpy(idx).to(DEV), scale, o, lse,
                       q_seq=torch.arange(B, dtype=torch.int32, device=DEV),
                       kv_offset=torch.from_numpy(off).to(DEV))
    torch.cuda.synchronize()
    C64, q64 = f64(C, dtype), f64(q, dtype)
    for b in range(B):
        sel = idx[b][idx[b] >= 0]
        ro, rl = O.mqa(q64[b], C64[off[b] + sel], scale)
        assert_rows_close(to_np64(o[b]), ro, what=f"mqa o[{b}]")
        got = lse[b].cpu().numpy().astype(np.float64)
        if sel.size == 0:
            assert np.all(np.isneginf(got))
        else:
            assert np.allclose(got, rl, rtol=1e-3, atol=1e-3)


@pytest.mark.parametrize("B,nh,k,nblk,qps,layout", [
    (40, 64, 64, 100, 1, "prefix"),     # one 64-head group, an empty and a short selection
    (37, 20, 100, 150, 3, "scatter"),   # partial head tile, k not a multiple of the chunk, -1 between slots
    (24, 128, 96, 70, 4, "ragged"),     # two head groups summed into one key gradient
    (33, 64, 512, 700, 11, "ragged"),   # long selections; 11 queries share each sequence's rows
    (4200, 16, 512, 600, 700, "prefix"),  # over 2^21 (query, slot) pairs: the shares are summed in two passes
    (40, 16, 64, 500, 1, "scatter"),    # 20000 compressed rows: the sort counts in global memory, not in LDS
])
def test_sparse_mqa_backward(B, nh, k, nblk, qps, layout):
    """Gradients of eq 11 against the oracle: dq per query and head, dCcomp per compressed row (queries of a
    sequence share its rows, so every row collects several queries' shares).  o and lse come from the
    library's own forward, as in training."""
    c = 512
    rng = synth.rng_for(B * nh + k + nblk)
    nseq = (B + qps - 1) // qps
    C = draw(rng, (nseq * nblk, c), 1.0, "bf16")
    q = draw(rng, (B, nh, c), 4.0 / math.sqrt(c), "bf16")
    dO = draw(rng, (B, nh, c), 1.0, "bf16")
    ncand = np.full(B, nblk)
    ncand[-1] = 0
    if B > 2:
        ncand[1] = min(nblk, k // 2 + 1)
    if layout != "prefix":
        ncand = rng.integers(0, nblk + 1, size=B)
        ncand[0] = 0
    idx = synth.random_selection(rng, ncand, k)
    if layout == "scatter":
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
    ref_dq, ref_dC = O.sparse_mqa_backward(f64(q, "bf16"), f64(C, "bf16"), idx, off[q_seq], scale, f64(dO, "bf16"))
    assert_rows_close(to_np64(dq), ref_dq, what="dq")
    assert_rows_close(to_np64(dC), ref_dC, what="dCcomp")


def test_sparse_mqa_backward_run_twice():
    """The key gradient's fp32 sums are not in a fixed order (shares of one compressed row that span several
    sorted segments meet in atomic adds), so two runs on the same inputs may differ in rounding only: per
    row by at most (number of shares + 1) * 2^-23 times the sum of the shares' magnitudes (from the
    oracle's per-query gradients).  dq is summed inside one workgroup per query and must be bit-identical.
    1200 queries share two sequences' 600 rows (about 600 shares per row, several 512-pair segments)."""
    B, nh, k, nblk, qps, c = 1200, 16, 512, 600, 600, 512
    rng = synth.rng_for(4242)
    nseq = B // qps
    C = draw(rng, (nseq * nblk, c), 1.0, "bf16")
    q = draw(rng, (B, nh, c), 4.0 / math.sqrt(c), "bf16")
    dO = draw(rng, (B, nh, c), 1.0, "bf16")
    idx = synth.random_selection(rng, rng.integers(k // 2, nblk + 1, size=B), k)
    q_seq = (np.arange(B) // qps).astype(np.int32)
    off = np.arange(nseq, dtype=np.int64) * nblk
    qd, Cd, dOd = to_device(q, "bf16", DEV), to_device(C, "bf16", DEV), to_device(dO, "bf16", DEV)
    idxd = torch.from_numpy(idx).to(DEV)
    qsd, offd = torch.from_numpy(q_seq).to(DEV), torch.from_numpy(off).to(DEV)
    o = torch.empty(B, nh, c, dtype=torch.bfloat16, device=DEV)
    lse = torch.empty(B, nh, dtype=torch.float32, device=DEV)
    scale = 1.0 / math.sqrt(c)
    api.csa_sparse_mqa(qd, Cd, idxd, scale, o, lse, q_seq=qsd, kv_offset=offd)
    runs = []
    for _ in range(2):
        dq = torch.empty(B, nh, c, dtype=torch.bfloat16, device=DEV)
        dC = torch.empty(nseq * nblk, c, dtype=torch.float32, device=DEV)
        api.csa_sparse_mqa_backward(qd, Cd, idxd, scale, o, lse, dOd, dq, dC, q_seq=qsd, kv_offset=offd)
        runs.append((dq.cpu(), dC.cpu().numpy().astype(np.float64)))
    torch.cuda.synchronize()
    assert torch.equal(runs[0][0].view(torch.int16), runs[1][0].view(torch.int16)), "dq differs between runs"
    q64, C64, dO64 = f64(q, "bf16"), f64(C, "bf16"), f64(dO, "bf16")
    abs_sum = np.zeros((nseq * nblk, c))
    count = np.zeros(nseq * nblk)
    for r in range(B):
        sel = idx[r][idx[r] >= 0]
        rows = off[q_seq[r]] + sel
        _, dc = O.mqa_backward(q64[r], C64[rows], scale, dO64[r])
        np.add.at(abs_sum, rows, np.abs(dc))
        np.add.at(count, rows, 1)
    diff = np.abs(runs[0][1] - runs[1][1])
    bound = (count[:, None] + 1) * 2.0 ** -23 * abs_sum
    worst = np.unravel_index(np.argmax(diff - bound), diff.shape)
    print(f"dCcomp run-to-run: {int((diff > 0).any(axis=1).sum())} of {diff.shape[0]} rows differ, "
          f"max |diff| {diff.max():.3e}; up to {int(count.max())} shares per row")
    assert np.all(diff <= bound), f"row {worst[0]}: runs differ by {diff[worst]:.3e} > {bound[worst]:.3e}"


# ---------------------------------------------------------------------------
# csa_decode: eqs 8, 9 and 11 in one call with a persistent workspace
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("lens,nq_rep,nhI,cI,nh,c,k,keys", [
    # per-chunk selector (long rows), a short row, an empty row
    ([4 * 9000, 4 * 20000, 4 * 33000, 100, 0, 4 * 5000], 1, 8, 64, 16, 128, 512, "random"),
    # 520 long rows of one sequence: one workgroup per row from the sweep's histogram
    ([4 * 9100], 520, 2, 32, 4, 64, 300, "random"),
    # c = 512, short batch: the attention finishes the long rows' selection itself (each split its own
    # slots); short and empty rows beside them
    ([4 * 9000, 4 * 20000, 4 * 33000, 100, 0, 4 * 5000], 1, 8, 64, 16, 512, 512, "random"),
    # the same with a ragged last split (k = 300) and a partly empty second head tile (20 heads)
    ([4 * 9000, 4 * 12000, 4 * 70], 1, 4, 32, 20, 512, 300, "random"),
    # every key one of two rows: each row's scores take two values, so thousands of keys tie at the
    # threshold (more candidates than one LDS segment of the finishing phase holds)
    ([4 * 12000, 4 * 30000], 1, 4, 64, 16, 512, 512, "two"),
    # the longest rows the per-chunk selector takes (64 chunks of 2048 candidates), beside shorter ones
    ([4 * 131000, 4 * 70000, 4 * 9000], 1, 4, 64, 16, 512, 512, "random"),
])
def test_decode_call_equals_two_calls(lens, nq_rep, nhI, cI, nh, c, k, keys):
    """Three back-to-back csa_decode calls on one workspace (zeroed once), each with new queries, give
    exactly the results of csa_index_topk (fresh workspace) followed by csa_sparse_mqa: the calls leave
    the histogram and counters zero for the next one."""
    rng = synth.rng_for(sum(lens) + nq_rep)
    m = 4
    if nq_rep > 1:  # many queries at different positions of one sequence
        nb = lens[0] // m
        pos = rng.integers(4 * 8200, 4 * nb + 1, size=nq_rep).astype(np.int64)
        off = np.zeros(1, np.int64)
        q_seq = torch.zeros(nq_rep, dtype=torch.int32, device=DEV)
        rows = nb
    else:
        pos = np.asarray(lens, np.int64)
        nblk = pos // m
        off = np.zeros_like(nblk)
        off[1:] = np.cumsum(nblk)[:-1]
        q_seq = torch.arange(len(lens), dtype=torch.int32, device=DEV)
        rows = max(int(nblk.sum()), 1)
    B = len(pos)
    max_cand = int(pos.max() // m)
    if keys == "two":
        two = draw(rng, (2, cI), 1.0, "bf16")
        K = to_device(two[np.arange(rows) % 2], "bf16", DEV)
    else:
        K = to_device(draw(rng, (rows, cI), 1.0, "bf16"), "bf16", DEV)
    C = to_device(draw(rng, (rows, c), 1.0, "bf16"), "bf16", DEV)
    q_pos = torch.tensor(pos, device=DEV)
    kv_off = torch.tensor(off, device=DEV)
    ws = torch.zeros(api.csa_decode_workspace(B, max_cand, nhI, nh, c, k), dtype=torch.uint8, device=DEV)
    scale = 1.0 / math.sqrt(c)
    for call in range(3):
        qI = to_device(draw(rng, (B, nhI, cI), 1.0 / math.sqrt(cI), "bf16"), "bf16", DEV)
        wI = to_device(rng.standard_normal((B, nhI), dtype=np.float32), "f32", DEV)
        q = to_device(draw(rng, (B, nh, c), 4.0 / math.sqrt(c), "bf16"), "bf16", DEV)
        idx1 = torch.full((B, k), 7, dtype=torch.int32, device=DEV)
        sc1 = torch.empty(B, k, device=DEV)
        o1 = torch.empty(B, nh, c, dtype=torch.bfloat16, device=DEV)
        lse1 = torch.empty(B, nh, device=DEV)
        api.csa_decode(qI, wI, K, q, C, m, k, max_cand, scale, q_pos, idx1, o1, ws, lse=lse1, score_out=sc1,
                       q_seq=q_seq, kv_offset=kv_off)
        idx2 = torch.full((B, k), 9, dtype=torch.int32, device=DEV)
        sc2 = torch.empty(B, k, device=DEV)
        o2 = torch.empty(B, nh, c, dtype=torch.bfloat16, device=DEV)
        lse2 = torch.empty(B, nh, device=DEV)
        api.csa_index_topk(qI, wI, K, m, k, max_cand, idx2, score_out=sc2, q_seq=q_seq, q_pos=q_pos, kv_offset=kv_off)
        api.csa_sparse_mqa(q, C, idx2, scale, o2, lse2, q_seq=q_seq, kv_offset=kv_off)
        torch.cuda.synchronize()
        assert torch.equal(idx1, idx2), f"call {call}: selections differ"
        assert torch.equal(sc1, sc2) and torch.equal(o1, o2) and torch.equal(lse1, lse2), f"call {call}"
    if nq_rep == 1:  # the selection itself is the oracle's
        Kn = K.view(torch.int16).cpu().numpy().view(np.uint16)
        qn = qI.view(torch.int16).cpu().numpy().view(np.uint16)
        srows = _oracle_rows(qn, wI.cpu().numpy(), Kn, pos, off, m, "bf16")
        check_topk(idx1.cpu().numpy(), srows, k)


# ---------------------------------------------------------------------------
# packed sequences: compression and indexer + top-k per sequence
# ---------------------------------------------------------------------------
def _packed(lengths, m):
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int64)
    bo = np.concatenate([[0], np.cumsum(np.asarray(lengths) // m)]).astype(np.int64)
    return cu, bo


@pytest.mark.parametrize("dtype,lengths,m,c", [
    ("f32", [0, 3, 5, 17, 64, 130], 4, 64), ("bf16", [1000, 1, 257, 4], 4, 512), ("bf16", [9, 31, 2], 8, 12),
    ("bf16", [40, 0, 0, 7], 1, 128),
])
def test_compress_varlen(dtype, lengths, m, c):
    """Each packed sequence is compressed as if alone: its rows equal the oracle's compression of its slice."""
    rng = synth.rng_for(sum(lengths) + m + c)
    cu, bo = _packed(lengths, m)
    n = int(cu[-1])
    cp = (c + 7) // 8 * 8
    P = draw(rng, (n, 4 * cp), 1.0, dtype)
    Pz = draw(rng, (n, 4 * cp), 2.0, dtype)
    P = np.where((np.arange(4 * cp) // cp)[None, :] >= 2, Pz, P)
    Ba = draw(rng, (m, c), 0.5, dtype)
    Bb = draw(rng, (m, c), 0.5, dtype)
    Pd = to_device(P, dtype, DEV)
    nb = int(bo[-1])
    out = torch.full((nb + 2, cp), 3.0, dtype=TD[dtype], device=DEV)[:, :c]
    sl = [Pd[:, i * cp:i * cp + c] for i in range(4)]
    api.csa_compress_varlen(*sl, to_device(Ba, dtype, DEV), to_device(Bb, dtype, DEV), m,
                            torch.tensor(cu, device=DEV), torch.tensor(bo, device=DEV), nb, out)
    torch.cuda.synchronize()
    got = to_np64(out)
    P64 = f64(P, dtype)
    for b in range(len(lengths)):
        seg = P64[cu[b]:cu[b + 1]]
        ref = O.compress(*[seg[:, i * cp:i * cp + c] for i in range(4)], f64(Ba, dtype), f64(Bb, dtype), m)
        if ref.shape[0]:
            assert_rows_close(got[bo[b]:bo[b + 1]], ref, what=f"sequence {b}")
    assert np.all(got[nb:] == 3.0)  # rows past the blocks are untouched


@pytest.mark.parametrize("dtype,lengths,m,c,lead", [
    ("f32", [0, 3, 5, 17, 64, 130], 4, 64, 0), ("bf16", [1000, 1, 257, 4], 4, 512, 3), ("bf16", [9, 31, 2], 8, 12, 0),
    ("bf16", [40, 0, 0, 7], 1, 128, 5), ("bf16", "many", 4, 128, 2), ("f32", [], 4, 16, 0), ("bf16", [2, 3], 4, 64, 1),
])
def test_compress_backward_varlen(dtype, lengths, m, c, lead):
    """Gradients of eqs 3-4 for packed sequences: each sequence's rows get the oracle's gradients of its own slice,
    the bias gradients sum over every sequence, and rows outside the sequences (the first `lead` rows and two rows
    after the last sequence) keep their sentinel."""
    if lengths == "many":  # 300 sequences: several units per workgroup and a deep sequence search
        lengths = [int(x) for x in synth.rng_for(77).integers(0, 40, size=300)]
    rng = synth.rng_for(sum(lengths) + 7 * m + c + lead)
    cu, bo = _packed(lengths, m)
    cu = cu + lead
    n = int(cu[-1]) + 2
    nb = int(bo[-1])
    cp = (c + 7) // 8 * 8
    P = draw(rng, (n, 4 * cp), 1.0, dtype)
    Pz = draw(rng, (n, 4 * cp), 2.0, dtype)
    P = np.where((np.arange(4 * cp) // cp)[None, :] >= 2, Pz, P)
    Ba = draw(rng, (m, c), 0.5, dtype)
    Bb = draw(rng, (m, c), 0.5, dtype)
    dC = rng.standard_normal(size=(nb, cp), dtype=np.float32)
    Pd = to_device(P, dtype, DEV)
    sl = [Pd[:, i * cp:i * cp + c] for i in range(4)]
    G = torch.full((n, 4 * cp), 7.0, dtype=TD[dtype], device=DEV)
    gs = [G[:, i * cp:i * cp + c] for i in range(4)]
    dBa = torch.full((m, c), 7.0, device=DEV)
    dBb = torch.full((m, c), 7.0, device=DEV)
    api.csa_compress_backward_varlen(*sl, to_device(Ba, dtype, DEV), to_device(Bb, dtype, DEV), m,
                                     torch.tensor(cu, device=DEV), torch.tensor(bo, device=DEV), nb,
                                     torch.from_numpy(dC).to(DEV)[:, :c], *gs, dBa, dBb)
    torch.cuda.synchronize()
    got = to_np64(G).reshape(n, 4, cp)
    P64 = f64(P, dtype)
    sum_a, sum_b = np.zeros((m, c)), np.zeros((m, c))
    mag_a, mag_b = np.zeros((m, c)), np.zeros((m, c))
    for b in range(len(lengths)):
        seg = P64[cu[b]:cu[b + 1]]
        ref = O.compress_backward(*[seg[:, i * cp:i * cp + c] for i in range(4)], f64(Ba, dtype), f64(Bb, dtype), m,
                                  dC[bo[b]:bo[b + 1], :c].astype(np.float64))
        if seg.shape[0]:
            for w in range(4):
                assert_rows_close(got[cu[b]:cu[b + 1], w, :c], ref[w], what=f"sequence {b} grad {w}")
        N = bo[b + 1] - bo[b]
        sum_a += ref[4]
        sum_b += ref[5]
        mag_a += np.abs(ref[2][:N * m]).reshape(N, m, c).sum(0) if N else 0.0
        mag_b += np.abs(ref[3][:(N - 1) * m]).reshape(N - 1, m, c).sum(0) if N > 1 else 0.0
    tol = 1e-5 if dtype == "f32" else 1e-4
    for gpu, want, mag in ((dBa, sum_a, mag_a), (dBb, sum_b, mag_b)):
        err = np.abs(to_np64(gpu) - want)
        assert np.all(err <= tol * mag + 1e-7), f"bias gradient off by {err.max()}"
    assert np.all(got[:lead] == 7.0) and np.all(got[int(cu[-1]):] == 7.0)  # rows outside the sequences
    assert np.all(got[:, :, c:] == 7.0)  # the padding columns between the slices


@pytest.mark.parametrize("dtype,lengths,m,nhI,cI,k", [
    ("bf16", [1, 40, 257, 1000, 33], 4, 64, 128, 64),
    ("f32", [130, 0, 77, 512], 4, 4, 32, 16),
    ("bf16", [3000, 70], 2, 20, 64, 300),
])
def test_index_topk_varlen(dtype, lengths, m, nhI, cI, k):
    """Token t of packed sequence b selects among its own sequence's first floor(t/m) blocks."""
    rng = synth.rng_for(sum(lengths) + nhI + k)
    cu, bo = _packed(lengths, m)
    n, nb = int(cu[-1]), int(bo[-1])
    K = draw(rng, (max(nb, 1), cI), 1.0, dtype)
    qI = draw(rng, (n, nhI, cI), 1.0 / math.sqrt(cI), dtype)
    wI = rng.standard_normal((n, nhI), dtype=np.float32)
    max_cand = max((L - 1) // m for L in lengths if L > 0)
    idx = torch.full((n, k), 123456, dtype=torch.int32, device=DEV)
    sc = torch.empty(n, k, dtype=torch.float32, device=DEV)
    qs = torch.full((n,), -5, dtype=torch.int32, device=DEV)
    api.csa_index_topk_varlen(to_device(qI, dtype, DEV), to_device(wI, "f32", DEV), to_device(K, dtype, DEV), m, k,
                              max_cand, torch.tensor(cu, device=DEV), torch.tensor(bo, device=DEV), idx,
                              score_out=sc, q_seq_out=qs)
    torch.cuda.synchronize()
    seq_of = np.repeat(np.arange(len(lengths)), lengths)
    assert np.array_equal(qs.cpu().numpy(), seq_of)
    K64, q64 = f64(K, dtype), f64(qI, dtype)
    rows = []
    for t in range(n):
        b = seq_of[t]
        nc = int((t - cu[b]) // m)
        rows.append(O.index_scores_row(q64[t], wI[t].astype(np.float64), K64[bo[b]:bo[b] + nc], nc))
    check_topk(idx.cpu().numpy(), rows, k)
