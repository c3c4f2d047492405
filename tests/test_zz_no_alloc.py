"""csa_decode_noalloc (the decode call whose scratch is a static per-GPU array, for callers that cannot
allocate) against csa_decode with its own zeroed workspace: results bit-identical, over calls in a row whose
sizes change (so the scratch holds the previous call's layout), and sizes past the scratch refused."""
import math

import pytest
import torch

from compressed_sparse_attention_amd import api

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _batch(seed, B, N, nhI, cI, nh, c, m, short_last):
    """Seeded caches (N blocks per sequence) and one query per sequence, on the GPU."""
    g = torch.Generator(device=DEV)
    g.manual_seed(seed)
    rows = B * N
    d = {
        "KI": torch.randn(rows, cI, generator=g, device=DEV).to(torch.bfloat16),
        "C": torch.randn(rows, c, generator=g, device=DEV).to(torch.bfloat16),
        "qI": (torch.randn(B, nhI, cI, generator=g, device=DEV) / math.sqrt(cI)).to(torch.bfloat16),
        "q": (torch.randn(B, nh, c, generator=g, device=DEV) / math.sqrt(c)).to(torch.bfloat16),
        "wI": torch.randn(B, nhI, generator=g, device=DEV),
    }
    lens = torch.full((B,), N * m, dtype=torch.int64)
    if short_last:
        lens[-1] = N * m // 3 + 1  # fewer candidates than the others
    d["q_pos"] = lens.to(DEV)
    d["kv_offset"] = (torch.arange(B, dtype=torch.int64) * N).to(DEV)
    d["q_seq"] = torch.arange(B, dtype=torch.int32, device=DEV)
    return d


def _run(d, m, k, max_cand, noalloc):
    B, nh, c = d["q"].shape
    idx = torch.full((B, k), -7, dtype=torch.int32, device=DEV)
    o = torch.full((B, nh, c), 7.0, dtype=torch.bfloat16, device=DEV)
    lse = torch.full((B, nh), 7.0, dtype=torch.float32, device=DEV)
    sc = torch.full((B, k), 7.0, dtype=torch.float32, device=DEV)
    args = (d["qI"], d["wI"], d["KI"], d["q"], d["C"], m, k, max_cand, 1.0 / math.sqrt(c), d["q_pos"], idx, o)
    kw = dict(lse=lse, score_out=sc, q_seq=d["q_seq"], kv_offset=d["kv_offset"])
    if noalloc:
        api.csa_decode_noalloc(*args, **kw)
    else:
        ws = torch.zeros(api.csa_decode_workspace(B, max_cand, d["qI"].shape[1], nh, c, k), dtype=torch.uint8,
                         device=DEV)
        api.csa_decode(*args, ws, **kw)
    torch.cuda.synchronize()
    return idx, o, lse, sc


def _same(a, b, what):
    for x, y, nm in zip(a, b, ("idx", "o", "lse", "scores")):
        assert torch.equal(x.view(torch.int16) if x.dtype == torch.bfloat16 else x,
                           y.view(torch.int16) if y.dtype == torch.bfloat16 else y), f"{what}: {nm} differs"


# (B, blocks per sequence, n_hI, c^I, n_h, c, m, k): the 8 x 131072-token batch (multi-workgroup selection,
# split attention), then a smaller batch of another layout, then the first sizes again
CASES = [(8, 32768, 64, 128, 64, 512, 4, 1024, 11),
         (3, 5000, 32, 128, 16, 512, 8, 512, 12),
         (8, 32768, 64, 128, 64, 512, 4, 1024, 13)]


def test_noalloc_equals_decode_over_changing_sizes():
    for B, N, nhI, cI, nh, c, m, k, seed in CASES:
        print(f"decode_noalloc case B={B} blocks={N} nhI={nhI} cI={cI} nh={nh} c={c} m={m} k={k} seed={seed}",
              flush=True)
        d = _batch(seed, B, N, nhI, cI, nh, c, m, short_last=True)
        got = _run(d, m, k, N, noalloc=True)
        ref = _run(d, m, k, N, noalloc=False)
        _same(got, ref, f"B={B} blocks={N}")
        assert int((got[0] >= 0).sum()) > 0
        # a second call on the same inputs right away (the scratch holds this call's own layout)
        _same(_run(d, m, k, N, noalloc=True), ref, f"B={B} blocks={N}, repeated")
        del d


def test_noalloc_refuses_sizes_past_its_scratch():
    """64 queries over 131072-block rows need more scratch than the static array holds: refused with
    CSA_ERR_WORKSPACE, outputs untouched."""
    B, nhI, cI, nh, c, k, N = 64, 64, 128, 64, 512, 1024, 131072
    qI = torch.zeros(B, nhI, cI, dtype=torch.bfloat16, device=DEV)
    q = torch.zeros(B, nh, c, dtype=torch.bfloat16, device=DEV)
    wI = torch.zeros(B, nhI, device=DEV)
    KI = torch.zeros(16, cI, dtype=torch.bfloat16, device=DEV)
    C = torch.zeros(16, c, dtype=torch.bfloat16, device=DEV)
    idx = torch.full((B, k), -7, dtype=torch.int32, device=DEV)
    o = torch.full((B, nh, c), 7.0, dtype=torch.bfloat16, device=DEV)
    q_pos = torch.full((B,), 4 * N, dtype=torch.int64, device=DEV)
    with pytest.raises(api.CSAError) as e:
        api.csa_decode_noalloc(qI, wI, KI, q, C, 4, k, N, 1.0 / math.sqrt(c), q_pos, idx, o)
    assert e.value.status == api.CSA_ERR_WORKSPACE
    torch.cuda.synchronize()
    assert bool((idx == -7).all()) and bool((o == 7.0).all())
