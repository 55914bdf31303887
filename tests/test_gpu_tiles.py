"""Score tiles of 2, 4 and 8 groups of 64 tokens per wave (the small parity
cases plan one): at B = 4, 8 KV heads and lengths whose plan picks U = 8, 4 and
2 (256*U tokens per tile, the largest U leaving >= 1024 tiles), with ragged
sequence ends inside a tile, a wave's quarter and a 64-token group.

- Paged pools (shuffled pages of 256 and 1024 tokens) against contiguous caches
  holding the same tokens: same plan, so positions and outputs are identical.
- The ragged batch against each sequence run alone (batch-1 views, a smaller U):
  the exact top-k is the same set in the same order whatever the tiling; the
  attention sums in another split order, so it is compared to fp32 rounding.

GPU against GPU: no oracle is needed for either comparison (the oracle pins the
same kernels at the small sizes).  Inputs are seeded Gaussian bf16 drawn on the
device.
"""

import math

import numpy as np
import pytest
import torch

from gpu_util import say

pytestmark = pytest.mark.gpu

sk = pytest.importorskip("bit_self_indexed_amd")

SM = 1.0 / math.sqrt(128)
B, HQ, HKV = 4, 32, 8
# name, longest length N, lengths (ragged ends inside a tile, a quarter, a group), k
SHAPES = [
    ("U8", 66000, [66000, 40001, 65537, 2100], 3000),
    ("U4", 40064, [40064, 33333, 20065, 700], 2000),
    ("U2", 20064, [20064, 17001, 9999, 64 + 512 + 7], 1000),
]


def _plan_u(n_tokens):
    n = n_tokens - 64
    for u in (8, 4, 2):
        if B * HKV * -(-n // (256 * u)) >= 1024:
            return u
    return 1


def _draw(N, seed):
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    K = torch.randn((B, HKV, N, 128), generator=g, device="cuda").to(torch.bfloat16)
    V = torch.randn((B, HKV, N, 128), generator=g, device="cuda").to(torch.bfloat16)
    q = torch.randn((B, HQ, 128), generator=g, device="cuda").to(torch.bfloat16)
    return K, V, q


def _prefill(cache, K, lengths):
    for b, n in enumerate(lengths):
        vb = cache.view(b)
        vb.n_tokens = n
        sk.sikv_encode(vb, K[b:b + 1, :, :n])
    cache.n_tokens = max(lengths)
    cache.seq_lens = torch.tensor(lengths, dtype=torch.int32, device="cuda")


def _step(cache, q, k):
    idx = torch.empty((B, HKV, k), dtype=torch.int32, device="cuda")
    out = sk.sikv_decode_step(cache, q, k, SM, idx_out=idx)
    torch.cuda.synchronize()
    return idx.cpu(), out.cpu()


@pytest.mark.parametrize("name,N,lengths,k", SHAPES, ids=[s[0] for s in SHAPES])
def test_ragged_batch_matches_each_sequence(name, N, lengths, k):
    assert _plan_u(N) == int(name[1:])
    say(f"[tiles] ragged {name} N={N} lengths={lengths} k={k}")
    K, V, q = _draw(N, 400 + N % 97)
    cache = sk.Cache(B, HKV, N, v=V)
    _prefill(cache, K, lengths)
    idx, out = _step(cache, q, k)
    for b, n in enumerate(lengths):
        kb = min(k, n - 64)
        assert torch.all(idx[b, :, kb:] == -1), f"{name} b={b}: tail of the idx row"
        vb = cache.view(b)
        vb.n_tokens = n
        i1 = torch.empty((1, HKV, kb), dtype=torch.int32, device="cuda")
        o1 = sk.sikv_decode_step(vb, q[b:b + 1], kb, SM, idx_out=i1)
        torch.cuda.synchronize()
        assert torch.equal(idx[b, :, :kb], i1[0].cpu()), f"{name} b={b}: top-k"
        ref = o1[0].cpu().double()
        err = ((out[b].double() - ref).abs().amax(dim=1) /
               ref.abs().amax(dim=1).clamp_min(1e-30))
        assert float(err.max()) <= 1e-5, f"{name} b={b}: attention {float(err.max()):.3e}"


@pytest.mark.parametrize("page", [256, 1024])
@pytest.mark.parametrize("name,N,lengths,k", SHAPES[:2], ids=[s[0] for s in SHAPES[:2]])
def test_paged_pool_matches_contiguous(name, N, lengths, k, page):
    say(f"[tiles] paged {name} page={page} N={N} lengths={lengths} k={k}")
    K, V, q = _draw(N, 500 + page)
    pps = -(-N // page)
    cap = pps * page
    n_pages = B * pps + 3
    perm = np.random.default_rng(page + N).permutation(n_pages)[:B * pps].reshape(B, pps)
    table = torch.tensor(perm, dtype=torch.int32, device="cuda")
    Vc = torch.zeros((B, HKV, cap, 128), dtype=torch.bfloat16, device="cuda")
    Vc[:, :, :N] = V
    del V
    pool_v = torch.zeros((n_pages, HKV, page, 128), dtype=torch.bfloat16, device="cuda")
    for b in range(B):
        for j in range(pps):
            pool_v[perm[b, j]] = Vc[b, :, j * page:(j + 1) * page]
    cont = sk.Cache(B, HKV, cap, v=Vc)
    paged = sk.Cache.paged(B, HKV, page, n_pages, table, v=pool_v)
    for c in (cont, paged):
        _prefill(c, K, lengths)
    a, b = _step(cont, q, k), _step(paged, q, k)
    assert torch.equal(a[0], b[0]), f"{name} page={page}: top-k"
    assert torch.equal(a[1], b[1]), f"{name} page={page}: attention"


def test_sixteen_groups_per_wave():
    """Past 2048 tiles of 2048 tokens the plan doubles the tile (U = 16, two
    load steps per wave): one head of 4.2M tokens, the candidate path against
    the select kernel's exact rescan of the whole head."""
    n = 2049 * 2048 + 100            # candidates: 2050 tiles of 2048 would exceed 2048
    N, k = 64 + n, 5000
    say(f"[tiles] U16 N={N} k={k}")
    g = torch.Generator(device="cuda")
    g.manual_seed(16)
    K = torch.randn((1, 1, N, 128), generator=g, device="cuda").to(torch.bfloat16)
    V = torch.randn((1, 1, N, 128), generator=g, device="cuda").to(torch.bfloat16)
    q = torch.randn((1, 4, 128), generator=g, device="cuda").to(torch.bfloat16)
    cache = sk.Cache(1, 1, N, v=V)
    sk.sikv_encode(cache, K)
    del K
    i1 = torch.empty((1, 1, k), dtype=torch.int32, device="cuda")
    o1 = sk.sikv_decode_step(cache, q, k, SM, idx_out=i1).cpu()
    i2 = torch.empty_like(i1)
    o2 = sk.sikv_decode_step(cache, q, k, SM, idx_out=i2, exact_select=True).cpu()
    torch.cuda.synchronize()
    assert torch.equal(i1.cpu(), i2.cpu()), "U16 top-k against the exact rescan"
    assert torch.equal(o1, o2), "U16 attention"
    assert int(i1.min()) >= 64 and int(i1.max()) < N


@pytest.mark.parametrize("page", [256])
def test_paged_quantised_values_match_contiguous(page):
    """2-bit value records at the U = 8 shape: a paged pool against a contiguous
    cache, both with ragged lengths (bit-identical positions and outputs)."""
    name, N, lengths, k = SHAPES[0]
    say(f"[tiles] paged 2-bit {name} page={page} N={N} lengths={lengths} k={k}")
    K, V, q = _draw(N, 700 + page)
    pps = -(-N // page)
    cap = pps * page
    n_pages = B * pps + 3
    perm = np.random.default_rng(page + N + 1).permutation(n_pages)[:B * pps].reshape(B, pps)
    table = torch.tensor(perm, dtype=torch.int32, device="cuda")
    cont = sk.Cache(B, HKV, cap, quant_v=True)
    paged = sk.Cache.paged(B, HKV, page, n_pages, table, quant_v=True)
    for c in (cont, paged):
        for b, n in enumerate(lengths):
            vb = c.view(b)
            vb.n_tokens = n
            sk.sikv_encode(vb, K[b:b + 1, :, :n])
            sk.sikv_encode_v(vb, V[b:b + 1, :, :n])
        c.n_tokens = max(lengths)
        c.seq_lens = torch.tensor(lengths, dtype=torch.int32, device="cuda")
    a, b = _step(cont, q, k), _step(paged, q, k)
    assert torch.equal(a[0], b[0]), f"2-bit page={page}: top-k"
    assert torch.equal(a[1], b[1]), f"2-bit page={page}: attention"
