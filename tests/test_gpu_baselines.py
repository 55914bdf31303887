"""GPU parity of the comparators behind the pages' module speed-ups (technical
summary §4, efficiency): the K-means baseline of the sign clustering and the
full dot-product retrieval scores, through the C ABI, against the oracle.

K-means: bit-exact (fixed-order fp32 distances decide the assignments on both
sides; the means are exact fixed-point sums).  Dense scores: |s - s_oracle| <=
1e-5 * sum_c |qbar_c k_c| (one fp32 accumulation of 128 products against fp64).
"""

import numpy as np
import pytest
import torch

import oracle as O
import sikv_synth as S
from gpu_util import dev_bf16, say

pytestmark = pytest.mark.gpu

sk = pytest.importorskip("bit_self_indexed_amd")

KM_CASES = [
    ("km_small", S.custom("km_small", 1, 4, 2, 3001, 100, n_planted=4, cfg_id=170)),
    ("km_multi_block", S.custom("km_multi", 2, 4, 1, 9100, 100, n_planted=8, cfg_id=171)),
]


@pytest.mark.parametrize("name,w", KM_CASES, ids=[c[0] for c in KM_CASES])
def test_kmeans_codebook_parity(name, w):
    say(f"[baseline] case={name} B={w.batch} Hkv={w.n_kv_heads} N={w.n_tokens}")
    d = S.draw(w)
    N = w.n_tokens
    K = dev_bf16(d["K"])
    cache = sk.Cache(w.batch, w.n_kv_heads, N, v=dev_bf16(d["V"]), codebook=True)
    sk.sikv_encode(cache, K)
    torch.cuda.synchronize()
    one_pass = cache.codebook.cpu().numpy().copy()
    enc = O.encode(d["K"], N)
    for n_iter in (1, 3, 20):
        sk.sikv_kmeans_codebook(cache, K, n_iter)
        torch.cuda.synchronize()
        got = cache.codebook.cpu().numpy()
        if n_iter == 1:   # one Lloyd step from the vertices is the one-pass codebook
            assert np.array_equal(got.view(np.uint32), one_pass.view(np.uint32))
        for b in range(w.batch):
            for h in range(w.n_kv_heads):
                ref = O.kmeans_codebook(d["K"][b, h], enc["mu"][b, h], enc["alpha"][b, h], N,
                                        n_iter)
                assert np.array_equal(got[b, h].view(np.uint32), ref.view(np.uint32)), \
                    f"{name} n_iter={n_iter} b={b} h={h}"


@pytest.mark.parametrize("B,Hq,Hkv,N", [(2, 8, 2, 3001), (1, 5, 1, 257), (1, 8, 8, 20000)])
def test_dense_scores_parity(B, Hq, Hkv, N):
    say(f"[baseline] dense scores B={B} Hq={Hq} Hkv={Hkv} N={N}")
    w = S.custom("dscore", B, Hq, Hkv, N, 10, n_planted=2, cfg_id=172 + N % 7)
    d = S.draw(w)
    got = sk.sikv_dense_scores(dev_bf16(d["q"]), dev_bf16(d["K"])).cpu().numpy()
    ref = O.dense_scores(d["q"], d["K"], Hkv, N)
    qbar = O.group_query(d["q"], Hkv)
    kf = S.bf16_bits_to_f32(d["K"]).astype(np.float64)
    bound = 1e-5 * np.einsum("bhc,bhtc->bht", np.abs(qbar), np.abs(kf)) + 1e-30
    assert np.all(np.abs(got - ref) <= bound), float((np.abs(got - ref) / bound).max())
