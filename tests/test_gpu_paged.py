"""Paged caches (per-token arrays in a pool of pages, one page table per
sequence) against contiguous caches holding the same tokens: the pool pages of
every sequence are a random permutation, and every result — codes, scales,
value records, means, codebook, idx, attention output, the fused append and the
K-means baseline — must be bit-identical to the contiguous cache's.  The
contiguous path itself is checked against the oracle elsewhere.
"""

import numpy as np
import pytest
import torch

import sikv_synth as S
from gpu_util import SM, dev_bf16, say

pytestmark = pytest.mark.gpu

sk = pytest.importorskip("bit_self_indexed_amd")

P = 256


def _pool_gather(pool, table, B):
    """Pool rows [n_pages, Hkv, P, ...] back to the logical [B, Hkv, pps * P, ...]."""
    pps = table.shape[1]
    out = [torch.cat([pool[table[b, j]] for j in range(pps)], dim=1) for b in range(B)]
    return torch.stack(out)


def _caches(w, d, quant_v, codebook, seed, n_pages=None):
    B, Hkv = w.batch, w.n_kv_heads
    pps = (w.n_tokens + 16 + P - 1) // P
    cap = pps * P
    if n_pages is None:
        n_pages = B * pps + 5
        rng = np.random.default_rng(seed)
        perm = rng.permutation(n_pages)[:B * pps].reshape(B, pps)
    else:  # a large pool: the sequences' pages shuffled among its last ones
        rng = np.random.default_rng(seed)
        perm = (n_pages - 1 - rng.permutation(B * pps)).reshape(B, pps)
    table = torch.tensor(perm, dtype=torch.int32, device="cuda")
    Vc = torch.zeros((B, Hkv, cap, 128), dtype=torch.bfloat16, device="cuda")
    Vc[:, :, :w.n_tokens] = dev_bf16(d["V"])
    pool_v = None
    if not quant_v:
        pool_v = torch.zeros((n_pages, Hkv, P, 128), dtype=torch.bfloat16, device="cuda")
        for b in range(B):
            for j in range(pps):
                pool_v[perm[b, j]] = Vc[b, :, j * P:(j + 1) * P]
    cont = sk.Cache(B, Hkv, cap, v=None if quant_v else Vc, codebook=codebook, quant_v=quant_v)
    paged = sk.Cache.paged(B, Hkv, P, n_pages, table, v=pool_v, codebook=codebook,
                           quant_v=quant_v)
    return cont, paged, perm, Vc


@pytest.mark.parametrize("quant_v,codebook", [(False, False), (True, False), (False, True)],
                         ids=["bf16_v", "2bit_v", "codebook"])
def test_paged_matches_contiguous(quant_v, codebook):
    w = S.custom("paged", 2, 8, 2, 5000, 400, n_planted=8, cfg_id=190)
    say(f"[paged] quant_v={quant_v} codebook={codebook} N={w.n_tokens} page={P}")
    d = S.draw(w)
    N = w.n_tokens
    cont, paged, perm, Vc = _caches(w, d, quant_v, codebook, 191)
    K, q = dev_bf16(d["K"]), dev_bf16(d["q"])
    for c in (cont, paged):
        sk.sikv_encode(c, K[:, :, :N - 1])
        if quant_v:
            sk.sikv_encode_v(c, Vc[:, :, :N - 1])
    torch.cuda.synchronize()
    table = paged.page_table.cpu().numpy()
    for name in ("codes", "alpha") + (("vrec",) if quant_v else ()):
        g = _pool_gather(getattr(paged, name), table, w.batch)[:, :, :N - 1]
        assert torch.equal(g, getattr(cont, name)[:, :, :N - 1]), name
    for name in ("mu", "k_sink") + (("codebook",) if codebook else ()) + \
            (("v_sink",) if quant_v else ()):
        assert torch.equal(getattr(paged, name), getattr(cont, name)), name
    res = []
    for c in (cont, paged):
        idx = torch.empty((w.batch, w.n_kv_heads, w.top_k), dtype=torch.int32, device="cuda")
        c.n_tokens = N - 1
        out1 = sk.sikv_decode_step(c, q, w.top_k, SM, idx_out=idx).clone()
        idx1 = idx.clone()
        out2 = sk.sikv_append_decode_step(c, K[:, :, N - 1:N], q, w.top_k, SM, idx_out=idx,
                                          v_new=Vc[:, :, N - 1:N] if quant_v else None)
        torch.cuda.synchronize()
        res.append((idx1.cpu(), out1.cpu(), idx.cpu(), out2.cpu()))
    for a, b, what in zip(res[0], res[1], ("idx", "out", "idx after append", "out after append")):
        assert torch.equal(a, b), what
    g = _pool_gather(paged.codes, table, w.batch)[:, :, N - 1]
    assert torch.equal(g, cont.codes[:, :, N - 1])


def test_paged_ragged_and_kmeans():
    w = S.custom("paged_rag", 3, 8, 2, 4200, 300, n_planted=8, cfg_id=192)
    lengths = [4200, 2500, 300]
    say(f"[paged] ragged lengths={lengths} + K-means")
    d = S.draw(w)
    cont, paged, perm, Vc = _caches(w, d, False, True, 193)
    K, q = dev_bf16(d["K"]), dev_bf16(d["q"])
    for c in (cont, paged):
        for b, n in enumerate(lengths):
            vb = c.view(b)
            vb.n_tokens = n
            sk.sikv_encode(vb, K[b:b + 1, :, :n])
        c.n_tokens = max(lengths)
        c.seq_lens = torch.tensor(lengths, dtype=torch.int32, device="cuda")
    res = []
    for c in (cont, paged):
        idx = torch.empty((w.batch, w.n_kv_heads, w.top_k), dtype=torch.int32, device="cuda")
        out = sk.sikv_decode_step(c, q, w.top_k, SM, idx_out=idx)
        cb = []
        for b, n in enumerate(lengths[:2]):
            vb = c.view(b)
            vb.n_tokens = n
            sk.sikv_kmeans_codebook(vb, K[b:b + 1, :, :n], 3)
        torch.cuda.synchronize()
        res.append((idx.cpu(), out.cpu(), c.codebook.cpu()))
    for a, b, what in zip(res[0], res[1], ("idx", "out", "K-means codebook")):
        assert torch.equal(a, b), what


@pytest.mark.parametrize("quant_v", [False, True], ids=["bf16_v", "2bit_v"])
def test_pool_beyond_32bit_offsets(quant_v):
    """A pool of more than 2^24 rows (33000 pages of 2 heads x 256 tokens), the
    sequences in its last pages: the attention's 64-bit addressing form, which
    must give the contiguous cache's results bit for bit."""
    w = S.custom("big_pool", 2, 8, 2, 3000, 200, n_planted=8, cfg_id=194)
    n_pages = 33000  # rows 33000 * 2 * 256 > 2^24
    say(f"[paged] pool of {n_pages} pages, quant_v={quant_v}")
    d = S.draw(w)
    N = w.n_tokens
    cont, paged, perm, Vc = _caches(w, d, quant_v, False, 195, n_pages=n_pages)
    assert int(perm.min()) * w.n_kv_heads * P >= 1 << 24
    K, q = dev_bf16(d["K"]), dev_bf16(d["q"])
    res = []
    for c in (cont, paged):
        sk.sikv_encode(c, K[:, :, :N - 1])
        if quant_v:
            sk.sikv_encode_v(c, Vc[:, :, :N - 1])
        idx = torch.empty((w.batch, w.n_kv_heads, w.top_k), dtype=torch.int32, device="cuda")
        c.n_tokens = N - 1
        out = sk.sikv_append_decode_step(c, K[:, :, N - 1:N], q, w.top_k, SM, idx_out=idx,
                                         v_new=Vc[:, :, N - 1:N] if quant_v else None)
        torch.cuda.synchronize()
        res.append((idx.cpu(), out.cpu()))
    del paged
    assert torch.equal(res[0][0], res[1][0]), "idx"
    assert torch.equal(res[0][1], res[1][1]), "out"
