"""Pins of the CPU oracle against facts that do not come from the oracle itself.

Page: "Self-Indexing KVCache: Predicting Sparse Attention from Compressed Keys"
(web summary, technical part), sections cited as §2.1 item n.  Hand-derived
values live in tests/golden/hand_cases.json.  Each test is built so that a
plausible slip in the oracle (dropped term, wrong sign or index, transposed
operand, wrong bit order, wrong reduction order) makes it fail.
"""

import heapq
import itertools
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle as O
import sikv_synth as S

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "hand_cases.json")))


def _bf16(x):
    return S.f32_to_bf16_bits(np.asarray(x, np.float32))


def _rand_keys(rng, n, mu_scale=2.0, h=1):
    mu = rng.normal(0, mu_scale, (h, 1, 128)).astype(np.float32)
    return _bf16(mu + rng.standard_normal((h, n, 128)).astype(np.float32))


# ----------------------------------------------------------------- tree / mean
def test_tree_order_golden():
    g = GOLD["tree_order"]
    got = O.tree_sum_f32(np.array(g["leaves"], np.float32))
    assert float(got) == g["expected"]
    seq = np.float32(0)
    for v in g["leaves"]:
        seq = np.float32(seq + np.float32(v))
    assert float(seq) == g["sequential_would_give"] != g["expected"]


def test_tree_padding_is_neutral():
    rng = np.random.default_rng(1)
    x = rng.standard_normal(37).astype(np.float32)
    a = O.tree_sum_f32(x)
    b = O.tree_sum_f32(np.concatenate([x, np.zeros(64 - 37, np.float32)]))
    c = O.tree_sum_f32(np.concatenate([x, np.zeros(256 - 37, np.float32)]))
    assert a == b == c
    # integers: exact, so the tree must give the true sum
    xi = rng.integers(-1000, 1000, 1000).astype(np.float32)
    assert float(O.tree_sum_f32(xi)) == float(xi.astype(np.int64).sum())


@pytest.mark.parametrize("n", [65, 100, 1000, 4096, 5003])
def test_channel_mean_vs_fp64(n):
    rng = np.random.default_rng(n)
    k = _rand_keys(rng, n)
    mu = O.channel_mean(k, n)[0]
    x = S.bf16_bits_to_f32(k[0, 64:n]).astype(np.float64)
    ref = x.mean(axis=0)
    levels = math.ceil(math.log2(n)) + 1
    bound = levels * 2.0 ** -24 * np.abs(x).sum(axis=0) / (n - 64) + 2.0 ** -24 * np.abs(ref)
    assert np.all(np.abs(mu - ref) <= bound)


def test_channel_mean_ignores_sinks_and_tail():
    rng = np.random.default_rng(2)
    k = _rand_keys(rng, 600)
    mu = O.channel_mean(k, 500)
    k2 = k.copy()
    k2[:, :64] = _bf16(np.full((1, 64, 128), 1e4))
    k2[:, 500:] = _bf16(np.full((1, 100, 128), -1e4))
    assert np.array_equal(mu, O.channel_mean(k2, 500))


# ----------------------------------------------------------------- codes / scale
def _layout_row():
    g = GOLD["code_layout"]
    row = np.full(128, g["other_value"], np.float32)
    row[g["negative_channels"]] = g["negative_value"]
    bits = _bf16(row)
    bits[g["zero_channels_pos"]] = 0x0000
    bits[g["zero_channels_neg"]] = 0x8000
    return bits[None, :], np.full(128, g["mu"], np.float32)


def test_code_layout_golden():
    g = GOLD["code_layout"]
    k, mu = _layout_row()
    code = O.pack_codes(O.sign_bits(k, mu))[0]
    assert code.tobytes().hex() == g["expected_code_hex"]
    nib = O.code_nibbles(code)
    for j, v in g["expected_nibbles"].items():
        assert nib[int(j)] == v
    assert float(O.token_scale(k, mu)[0]) == g["expected_alpha"]


def test_codes_bruteforce_bits():
    rng = np.random.default_rng(3)
    k = _rand_keys(rng, 70)[0]
    mu = O.channel_mean(k[None], 70)[0]
    codes = O.pack_codes(O.sign_bits(k, mu))
    x = S.bf16_bits_to_f32(k)
    for t in range(0, 70, 7):
        for c in range(128):
            byte = int(codes[t, c // 8])
            assert ((byte >> (c % 8)) & 1) == (1 if float(x[t, c]) < float(mu[c]) else 0)
        for j in range(32):
            pat = sum((1 << i) for i in range(4) if float(x[t, 4 * j + i]) < float(mu[4 * j + i]))
            assert O.code_nibbles(codes[t])[j] == pat


def test_entropy_balance():
    """§2.1 item 1: subtracting the channel mean balances the signs.  With mean
    offsets N(0,2) the raw sign rate of channel c is Phi(-m_c); after centring it
    is close to 1/2 for every channel."""
    rng = np.random.default_rng(4)
    n = 20000
    m = rng.normal(0, math.sqrt(2), 128).astype(np.float32)
    k = _bf16(m[None, :] + rng.standard_normal((n, 128)).astype(np.float32))
    mu = O.channel_mean(k[None], n)[0]
    rate = O.sign_bits(k[64:], mu).mean(axis=0)
    assert np.all(np.abs(rate - 0.5) < 0.02)
    raw = O.sign_bits(k[64:], np.zeros(128, np.float32)).mean(axis=0)
    phi = 0.5 * (1 + np.vectorize(math.erf)(-m / math.sqrt(2)))
    assert np.all(np.abs(raw - phi) < 0.02)
    assert np.abs(raw - 0.5).max() > 0.3


def test_scale_is_least_squares_optimum():
    rng = np.random.default_rng(5)
    k = _rand_keys(rng, 300)[0]
    mu = O.channel_mean(k[None], 300)[0]
    alpha = O.token_scale(k, mu).astype(np.float64)
    kt = S.bf16_bits_to_f32(k).astype(np.float64) - mu.astype(np.float64)
    sgn = np.where(O.sign_bits(k, mu), -1.0, 1.0)
    for eps in (1e-3, -1e-3):
        e0 = ((kt - alpha[:, None] * sgn) ** 2).sum(axis=1)
        e1 = ((kt - (alpha * (1 + eps))[:, None] * sgn) ** 2).sum(axis=1)
        assert np.all(e1 > e0)
    fs = np.array([math.fsum(np.abs(np.float32(S.bf16_bits_to_f32(k[t])) - mu).astype(np.float64))
                   for t in range(300)]) / 128
    assert np.allclose(alpha, fs, rtol=1e-6, atol=0)


def test_round_trip():
    """§2.1 item 1 (dual use): re-encoding the reconstructed keys against the same
    mean gives the same codes, and the scale back to within rounding."""
    rng = np.random.default_rng(6)
    k = _rand_keys(rng, 400)[0]
    mu = O.channel_mean(k[None], 400)[0]
    codes = O.pack_codes(O.sign_bits(k, mu))
    alpha = O.token_scale(k, mu)
    khat = O.dequantize(codes, alpha, mu)
    bits2 = khat < mu[None, :]
    assert np.array_equal(O.pack_codes(bits2), codes)
    alpha2 = np.abs(khat - mu[None, :]).astype(np.float64).mean(axis=1)
    assert np.allclose(alpha2, alpha, rtol=1e-5, atol=0)


def test_dequantize_values():
    k, mu = _layout_row()
    codes = O.pack_codes(O.sign_bits(k, mu))
    khat = O.dequantize(codes, np.array([0.5], np.float32), mu + np.float32(2.0))
    g = GOLD["code_layout"]
    expect = np.full(128, 2.5, np.float32)
    expect[g["negative_channels"]] = 1.5
    assert np.array_equal(khat[0], expect)


def test_encode_layout_and_sinks():
    rng = np.random.default_rng(7)
    k = _rand_keys(rng, 300, h=2)[None]           # [1,2,300,128]
    enc = O.encode(k, 260)
    assert enc["codes"].shape == (1, 2, 260, 16) and enc["alpha"].shape == (1, 2, 260)
    assert np.array_equal(enc["k_sink"], k[:, :, :64])
    app = O.encode_rows(k[:, :, 260:], enc["mu"])
    full = O.encode_rows(k[:, :, :300], enc["mu"])
    assert np.array_equal(app["codes"], full["codes"][:, :, 260:])
    assert np.array_equal(full["codes"][:, :, :260], enc["codes"])


# ----------------------------------------------------------------- LUT / scores
def test_lut_golden_subvector():
    g = GOLD["lut_subvector"]
    q = np.zeros(128)
    q[:4] = g["q_piece"]
    lut = O.query_lut(q)
    for p, v in g["expected"].items():
        assert lut[0, int(p)] == v
    assert np.all(lut[1:] == 0)


def test_lut_enumerates_all_sign_vertices():
    rng = np.random.default_rng(8)
    q = rng.standard_normal(128)
    lut = O.query_lut(q)
    for j in range(32):
        for signs in itertools.product((1.0, -1.0), repeat=4):
            p = sum((1 << i) for i, s in enumerate(signs) if s < 0)
            assert lut[j, p] == pytest.approx(float(np.dot(q[4 * j:4 * j + 4], signs)), abs=1e-12)


def test_lut_score_identity():
    """LUT score plus q.mu equals the plain dot product of the group's queries with
    the reconstructed key (computed without any table) to fp64 rounding."""
    rng = np.random.default_rng(9)
    B, Hq, Hkv, N = 2, 6, 2, 500
    q = _bf16(rng.standard_normal((B, Hq, 128)))
    k = _bf16(rng.normal(0, 1.5, (B, Hkv, 1, 128)) + rng.standard_normal((B, Hkv, N, 128)))
    enc = O.encode(k, N)
    G = Hq // Hkv
    qf = S.bf16_bits_to_f32(q).astype(np.float64)
    for b in range(B):
        for h in range(Hkv):
            s = O.head_scores(q, enc["codes"][b, h], enc["alpha"][b, h], b, h, Hkv, N)
            bits = np.unpackbits(enc["codes"][b, h, 64:N], axis=-1, bitorder="little")
            khat = (enc["mu"][b, h].astype(np.float64)[None, :]
                    + enc["alpha"][b, h, 64:N].astype(np.float64)[:, None] * (1.0 - 2.0 * bits))
            direct = sum(khat @ qf[b, h * G + g] for g in range(G))
            qmu = sum(float(qf[b, h * G + g] @ enc["mu"][b, h].astype(np.float64)) for g in range(G))
            assert np.allclose(s + qmu, direct, rtol=1e-12, atol=1e-10)


def test_group_query_is_contiguous():
    q = np.zeros((1, 8, 128), np.uint16)
    q[0, 5] = _bf16(np.ones(128))
    qb = O.group_query(q, 2)             # G = 4: heads 4..7 -> KV head 1
    assert np.all(qb[0, 0] == 0) and np.all(qb[0, 1] == 1)


# ----------------------------------------------------------------- top-k
def test_topk_golden_ties():
    g = GOLD["topk_ties"]
    got = O.select_topk(np.array(g["scores"]), g["k"], g["first_token"])
    assert got.tolist() == g["expected_idx"]


@pytest.mark.parametrize("seed", range(6))
def test_topk_bruteforce(seed):
    rng = np.random.default_rng(seed)
    m = int(rng.integers(1, 13))
    s = np.round(rng.standard_normal(m), 1)            # rounding forces ties
    for k in range(1, m + 1):
        brute = sorted(range(m), key=lambda i: (-s[i], i))[:k]
        assert O.select_topk(s, k).tolist() == sorted(i + 64 for i in brute)


def test_topk_heapq():
    rng = np.random.default_rng(11)
    s = rng.standard_normal(5000)
    got = O.select_topk(s, 300)
    ref = sorted(i + 64 for i in heapq.nlargest(300, range(5000), key=lambda i: s[i]))
    assert got.tolist() == ref


# ----------------------------------------------------------------- attention
def _small_cache(seed, B=1, Hq=4, Hkv=2, N=300):
    rng = np.random.default_rng(seed)
    q = _bf16(rng.standard_normal((B, Hq, 128)))
    k = _bf16(rng.normal(0, 1.5, (B, Hkv, 1, 128)) + rng.standard_normal((B, Hkv, N, 128)))
    v = _bf16(rng.standard_normal((B, Hkv, N, 128)))
    return q, k, v, O.encode(k, N)


def test_attention_all_tokens_equals_dense_sdpa():
    """With k = N - 64 the sparse path is dense softmax attention over
    [K_sink; K^] (checked through torch's fp64 scaled_dot_product_attention)."""
    q, k, v, enc = _small_cache(12)
    N, G, sm = 300, 2, 1 / math.sqrt(128)
    res = O.decode_step(q, enc, v, N - 64, sm, N)
    for h in range(2):
        kap = np.concatenate([S.bf16_bits_to_f32(enc["k_sink"][0, h]),
                              O.dequantize(enc["codes"][0, h, 64:], enc["alpha"][0, h, 64:],
                                           enc["mu"][0, h])]).astype(np.float64)
        qq = torch.tensor(S.bf16_bits_to_f32(q[0, h * G:(h + 1) * G]), dtype=torch.float64)
        kk = torch.tensor(kap)[None].expand(G, -1, -1)
        vv = torch.tensor(S.bf16_bits_to_f32(v[0, h]).astype(np.float64))[None].expand(G, -1, -1)
        ref = torch.nn.functional.scaled_dot_product_attention(
            qq[:, None, :], kk, vv, scale=sm)[:, 0].numpy()
        assert np.allclose(res["out"][0, h * G:(h + 1) * G], ref, rtol=1e-6, atol=1e-7)
        assert res["idx"][0, h].tolist() == list(range(64, N))


def test_attention_zero_query_is_mean_of_attended_values():
    q, k, v, enc = _small_cache(13)
    q[:] = 0
    res = O.decode_step(q, enc, v, 50, 0.088, 300)
    for h in range(2):
        rows = np.concatenate([np.arange(64), res["idx"][0, h]])
        ref = S.bf16_bits_to_f32(v[0, h, rows]).astype(np.float64).mean(axis=0)
        assert np.allclose(res["out"][0, 2 * h], ref, rtol=1e-6, atol=1e-7)


def test_attention_one_dominant_token():
    q, k, v, enc = _small_cache(14, Hq=1, Hkv=1)
    qf = S.bf16_bits_to_f32(q[0, 0]).astype(np.float64)
    # make candidate 200 equal to a large multiple of q: its reconstructed key
    # points along q's signs with a huge scale
    row = np.sign(qf) * -1e3
    k2 = k.copy()
    k2[0, 0, 200] = _bf16(row)
    enc2 = O.encode(k2, 300)
    # flip: the stored code of token 200 has all signs opposite to q -> tiny score;
    # attend with -q so token 200 dominates
    qn = _bf16(-S.bf16_bits_to_f32(q))
    res = O.decode_step(qn, enc2, v, 5, 1.0, 300)
    assert 200 in res["idx"][0, 0].tolist()
    assert np.allclose(res["out"][0, 0], S.bf16_bits_to_f32(v[0, 0, 200]), rtol=0, atol=1e-6)


def test_planted_recall_tiny():
    """On the tiny workload every planted token scores into the top 256."""
    w = S.WORKLOADS["tiny_4k"]
    d = S.draw(w)
    enc = O.encode(d["K"], w.n_tokens)
    res = O.decode_step(d["q"], enc, d["V"], w.top_k, 1 / math.sqrt(128), w.n_tokens)
    assert set(d["planted"][0, 0].tolist()) <= set(res["idx"][0, 0].tolist())


# ----------------------------------------------------------------- codebook
def _cb_case(rows_f32, mu_f32, alpha=None):
    """Rows (float32 values exactly representable in bf16) -> codebook inputs."""
    kb = _bf16(rows_f32)
    mu = np.asarray(mu_f32, np.float32)
    codes = O.pack_codes(O.sign_bits(kb, mu))
    a = O.token_scale(kb, mu) if alpha is None else np.asarray(alpha, np.float32)
    return kb, mu, codes, a


def test_codebook_identical_members_and_pair_mean():
    """Closed forms: members sharing x = k~/alpha give exactly that centre; two
    members give their mean; the pattern index follows the sign bits."""
    n = 64 + 3
    rows = np.ones((n, 128), np.float32)
    rows[64, :4] = [2.0, -1.0, 0.5, -0.25]           # pattern 0b1010 = 10
    rows[65, :4] = [2.0, -1.0, 0.5, -0.25]
    rows[66, :4] = [4.0, -3.0, 1.5, -0.75]           # same pattern
    alpha = np.ones(n, np.float32)
    alpha[66] = 2.0                                   # x = (2, -1.5, 0.75, -0.375)
    kb, mu, codes, a = _cb_case(rows, np.zeros(128, np.float32), alpha)
    cb = O.codebook(kb, mu, codes, a, n)
    exp = (np.array([2.0, -1.0, 0.5, -0.25]) * 2 + np.array([2.0, -1.5, 0.75, -0.375])) / 3
    assert np.array_equal(cb[0, 10], exp.astype(np.float32))
    # sub-vector 1 of every member is (1,1,1,1) -> pattern 0, centre exactly 1 / alpha mean
    assert np.allclose(cb[1, 0], (1.0 + 1.0 + 0.5) / 3, rtol=0, atol=2 ** -24)
    # all other clusters are empty -> sign vertices
    v = O.centres()
    for p in range(16):
        if p != 10:
            assert np.array_equal(cb[0, p], v[p].astype(np.float32))


def test_codebook_of_pure_sign_data_is_the_vertices():
    """|k_c - mu_c| = alpha for every channel: every member is exactly a sign
    vertex, so every non-empty centre is its vertex."""
    rng = np.random.default_rng(21)
    n = 64 + 500
    mu = rng.integers(-4, 4, 128).astype(np.float32)
    sgn = np.where(rng.random((n, 128)) < 0.5, -1.0, 1.0).astype(np.float32)
    kb, mu, codes, a = _cb_case(mu + 0.5 * sgn, mu)
    assert np.all(a == 0.5)
    cb = O.codebook(kb, mu, codes, a, n)
    assert np.array_equal(cb, np.broadcast_to(O.centres()[None], cb.shape).astype(np.float32))


def test_codebook_is_least_squares_and_sign_consistent():
    """For fixed assignments the mean minimises the squared error of x = k~/alpha
    (perturbation), and every component has the sign its pattern bit implies."""
    rng = np.random.default_rng(22)
    n = 64 + 3000
    kb = _rand_keys(rng, n)[0]
    mu = O.channel_mean(kb, n)
    codes = O.pack_codes(O.sign_bits(kb, mu))
    a = O.token_scale(kb, mu)
    cb = O.codebook(kb, mu, codes, a, n).astype(np.float64)
    x = ((S.bf16_bits_to_f32(kb[64:]) - mu).astype(np.float32) / a[64:, None]).astype(np.float64)
    nib = O.code_nibbles(codes[64:])
    for j in (0, 7, 31):
        for p in range(16):
            m = x[nib[:, j] == p, 4 * j:4 * j + 4]
            if len(m) == 0:
                continue
            f0 = ((m - cb[j, p]) ** 2).sum()
            for i in range(4):
                for eps in (1e-3, -1e-3):
                    c = cb[j, p].copy()
                    c[i] += eps
                    assert ((m - c) ** 2).sum() > f0
            bits = (p >> np.arange(4)) & 1
            assert np.all(np.where(bits == 1, cb[j, p] < 0, cb[j, p] > 0))


def test_codebook_lut_scores_match_bruteforce():
    """LUT scores with data centres equal alpha * sum_c qbar_c * centre component,
    accumulated channel by channel in a plain loop (tiny case)."""
    rng = np.random.default_rng(23)
    n = 64 + 40
    kb = _rand_keys(rng, n)[0]
    enc = O.encode(kb[None, None], n, with_codebook=True)
    cb, codes, a = enc["codebook"][0, 0], enc["codes"][0, 0], enc["alpha"][0, 0]
    qbar = rng.standard_normal(128)
    s = O.lut_scores(O.query_lut(qbar, cb), codes[64:], a[64:])
    for t in range(40):
        acc = 0.0
        for c in range(128):
            byte = int(codes[64 + t, c // 8])
            j = c // 4
            p = (byte >> (4 * (j & 1))) & 0xF
            acc += qbar[c] * float(cb[j, p, c % 4])
        assert abs(s[t] - float(a[64 + t]) * acc) <= 1e-12 * (1 + abs(s[t]))
    # and the dequantised keys reproduce the same dot products
    kh = O.dequantize(codes[64:], a[64:], enc["mu"][0, 0], cb).astype(np.float64)
    direct = (kh - enc["mu"][0, 0].astype(np.float64)) @ qbar
    assert np.allclose(direct, s, rtol=1e-5, atol=1e-5)


def test_codebook_attention_all_tokens_equals_dense_sdpa():
    """With data centres and k = N - 64 the sparse path is dense attention over
    [K_sink; K^(codebook)]."""
    rng = np.random.default_rng(24)
    B, Hq, Hkv, N, G, sm = 1, 2, 1, 200, 2, 1 / math.sqrt(128)
    q = _bf16(rng.standard_normal((B, Hq, 128)))
    k = _bf16(rng.normal(0, 1.5, (B, Hkv, 1, 128)) + rng.standard_normal((B, Hkv, N, 128)))
    v = _bf16(rng.standard_normal((B, Hkv, N, 128)))
    enc = O.encode(k, N, with_codebook=True)
    res = O.decode_step(q, enc, v, N - 64, sm, N)
    kap = np.concatenate([S.bf16_bits_to_f32(enc["k_sink"][0, 0]),
                          O.dequantize(enc["codes"][0, 0, 64:], enc["alpha"][0, 0, 64:],
                                       enc["mu"][0, 0], enc["codebook"][0, 0])]).astype(np.float64)
    qq = torch.tensor(S.bf16_bits_to_f32(q[0]), dtype=torch.float64)
    kk = torch.tensor(kap)[None].expand(G, -1, -1)
    vv = torch.tensor(S.bf16_bits_to_f32(v[0, 0]).astype(np.float64))[None].expand(G, -1, -1)
    ref = torch.nn.functional.scaled_dot_product_attention(qq[:, None, :], kk, vv, scale=sm)[:, 0]
    assert np.allclose(res["out"][0], ref.numpy(), rtol=1e-6, atol=1e-7)


def test_codebook_reconstruction_beats_vertices():
    """The data centres reconstruct the keys with less squared error than the
    scaled sign vertices (they are the per-cluster least-squares fit)."""
    rng = np.random.default_rng(25)
    n = 64 + 2000
    kb = _rand_keys(rng, n)[0]
    enc = O.encode(kb[None, None], n, with_codebook=True)
    x = S.bf16_bits_to_f32(kb[64:]).astype(np.float64)
    c, a, mu = enc["codes"][0, 0, 64:], enc["alpha"][0, 0, 64:], enc["mu"][0, 0]
    e_cb = ((O.dequantize(c, a, mu, enc["codebook"][0, 0]) - x) ** 2).sum()
    e_v = ((O.dequantize(c, a, mu) - x) ** 2).sum()
    assert e_cb < e_v


# ----------------------------------------------------------------- quantised values
def test_value_quantisation_hand_case():
    """Hand-derived case: a group holding exactly z, z+s, z+2s, z+3s (fp16-exact)
    gets codes 0..3, the layout puts channel c at byte c // 4, bits 2*(c % 4)."""
    row = np.zeros(128, np.float32)
    row[:32] = np.tile(np.array([1.0, 1.5, 2.0, 2.5], np.float32), 8)     # z=1, s=0.5
    row[32:64] = -3.0                                                       # constant group
    row[64:96] = np.linspace(-1.0, 2.0, 32).astype(np.float32)
    row[96:] = np.tile(np.array([0.25, 0.0, 0.0, 0.0], np.float32), 8)
    codes, sz = O.quantize_v(_bf16(row)[None])
    assert codes.shape == (1, 32) and sz.shape == (1, 4, 2)
    # group 0: codes 0,1,2,3 repeated -> byte 0b11100100
    assert codes[0, :8].tolist() == [0b11100100] * 8
    assert sz[0, 0].view(np.float16).tolist() == [0.5, 1.0]
    # group 1: constant -> scale 0, zero -3, codes 0
    assert codes[0, 8:16].tolist() == [0] * 8
    assert sz[0, 1].view(np.float16).tolist() == [0.0, -3.0]
    # group 3: one 0.25 then three zeros per 4 channels -> codes 3,0,0,0 -> byte 0b00000011
    assert codes[0, 24:].tolist() == [3] * 8
    rec = O.dequantize_v(codes, sz)[0]
    assert np.array_equal(rec[:32], row[:32].astype(np.float64))
    assert np.array_equal(rec[32:64], row[32:64].astype(np.float64))
    # group 3: scale 0.25 / 3 is not fp16-exact, so the top level is 3 * fp16(0.25 / 3)
    s3 = float(np.float16(np.float32(0.25) / np.float32(3)))
    assert rec[96] == 3 * s3 and abs(rec[96] - 0.25) < 2 ** -12
    assert np.all(rec[97:100] == 0.0)


def test_value_quantisation_error_bound_and_extremes():
    """Every reconstructed value lies within half a step (plus the fp16 rounding of the
    scale and zero point) of the input; codes span 0..3 and the group minimum is
    reconstructed exactly up to the zero point's rounding."""
    rng = np.random.default_rng(31)
    v = _bf16(rng.standard_normal((500, 128)) * rng.uniform(0.1, 5.0, (500, 1)))
    codes, sz = O.quantize_v(v)
    rec = O.dequantize_v(codes, sz)
    x = S.bf16_bits_to_f32(v).astype(np.float64).reshape(500, 4, 32)
    s = sz[..., 0].view(np.float16).astype(np.float64)[..., None]
    z = sz[..., 1].view(np.float16).astype(np.float64)[..., None]
    err = np.abs(rec.reshape(500, 4, 32) - x)
    zerr = np.abs(z - x.min(axis=-1, keepdims=True))
    bound = 0.5 * s + zerr + 3 * np.abs(s - (x.max(-1, keepdims=True) - x.min(-1, keepdims=True)) / 3) + 1e-6
    assert np.all(err <= bound)
    q = np.stack([(codes >> (2 * i)) & 3 for i in range(4)], -1).reshape(500, 4, 32)
    assert q.min() == 0 and q.max() == 3
    assert np.all(q.min(axis=-1) == 0)


def test_quantised_value_attention_equals_dense_sdpa():
    """With k = N - 64 and quantised values the sparse path is dense attention with the
    bf16 sink values and the reconstructed values of every other token."""
    rng = np.random.default_rng(32)
    B, Hq, Hkv, N, G, sm = 1, 2, 1, 180, 2, 1 / math.sqrt(128)
    q = _bf16(rng.standard_normal((B, Hq, 128)))
    k = _bf16(rng.normal(0, 1.5, (B, Hkv, 1, 128)) + rng.standard_normal((B, Hkv, N, 128)))
    v = _bf16(rng.standard_normal((B, Hkv, N, 128)))
    enc = O.encode(k, N)
    vq = O.quantize_v(v)
    res = O.decode_step(q, enc, v, N - 64, sm, N, vq=vq)
    kap = np.concatenate([S.bf16_bits_to_f32(enc["k_sink"][0, 0]),
                          O.dequantize(enc["codes"][0, 0, 64:], enc["alpha"][0, 0, 64:],
                                       enc["mu"][0, 0])]).astype(np.float64)
    vals = np.concatenate([S.bf16_bits_to_f32(v[0, 0, :64]).astype(np.float64),
                           O.dequantize_v(vq[0][0, 0, 64:], vq[1][0, 0, 64:])])
    qq = torch.tensor(S.bf16_bits_to_f32(q[0]), dtype=torch.float64)
    ref = torch.nn.functional.scaled_dot_product_attention(
        qq[:, None, :], torch.tensor(kap)[None].expand(G, -1, -1),
        torch.tensor(vals)[None].expand(G, -1, -1), scale=sm)[:, 0]
    assert np.allclose(res["out"][0], ref.numpy(), rtol=1e-6, atol=1e-7)


# ----------------------------------------------------------------- K-means baseline
def _head_case(seed, n):
    w = S.custom("km", 1, 4, 1, n, 100, n_planted=4, cfg_id=seed)
    K = S.draw(w)["K"][0, 0]
    e = O.encode(K[None, None], n)
    return K, e["mu"][0, 0], e["codes"][0, 0], e["alpha"][0, 0]


@pytest.mark.parametrize("seed,n", [(160, 3000), (161, 5003)])
def test_kmeans_one_iteration_is_the_codebook(seed, n):
    """From the sign vertices, a point's nearest vertex is its sign pattern, so the
    first Lloyd step is exactly the one-pass sign clustering (empty clusters keep
    the vertex in both)."""
    K, mu, codes, alpha = _head_case(seed, n)
    cb = O.codebook(K, mu, codes, alpha, n)
    km = O.kmeans_codebook(K, mu, alpha, n, 1)
    assert np.array_equal(cb.view(np.uint32), km.view(np.uint32))


def test_kmeans_objective_never_increases():
    K, mu, _, alpha = _head_case(162, 4000)
    objs = [O.kmeans_objective(K, mu, alpha, 4000, O.kmeans_codebook(K, mu, alpha, 4000, it))
            for it in (1, 2, 3, 5, 8, 20)]
    assert all(b <= a * (1 + 1e-9) for a, b in zip(objs, objs[1:])), objs
    assert objs[-1] < 0.9 * objs[0]                     # the iterations do move the centres


def test_kmeans_matches_scikit_learn_lloyd():
    """scikit-learn's Lloyd K-means from the same 16 vertices, on points whose
    clusters straddle the orthant borders (so the assignment changes after the
    first step) and are exactly representable (mu = 0, alpha = 1: x = k)."""
    from sklearn.cluster import KMeans
    rng = np.random.default_rng(163)
    v = O.centres()
    n_per, n = 40, 64 + 16 * 40
    rows = np.zeros((n, 128), np.float32)
    for j in range(32):
        true = v * rng.uniform(0.3, 1.6, (16, 4))
        pts = np.repeat(true, n_per, axis=0) + rng.normal(0, 0.45, (16 * n_per, 4))
        rows[64:, 4 * j:4 * j + 4] = pts[rng.permutation(16 * n_per)]
    kb = _bf16(rows)
    x = S.bf16_bits_to_f32(kb).astype(np.float64)
    mu, alpha = np.zeros(128, np.float32), np.ones(n, np.float32)
    ours = O.kmeans_codebook(kb, mu, alpha, n, 20)
    moved = 0
    for j in range(32):
        pts = x[64:, 4 * j:4 * j + 4]
        km = KMeans(n_clusters=16, init=v.copy(), n_init=1, max_iter=20, tol=0.0,
                    algorithm="lloyd").fit(pts)
        assert np.bincount(km.labels_, minlength=16).min() > 0
        np.testing.assert_allclose(ours[j], km.cluster_centers_, rtol=0, atol=1e-5)
        sign_pattern = ((pts < 0) * (1 << np.arange(4))).sum(axis=1)
        moved += int(np.any(km.labels_ != sign_pattern))
    assert moved > 0                                     # the assignment did change


# ----------------------------------------------------------------- dense retrieval scores
def test_dense_scores_closed_form():
    """Keys that are scaled unit vectors: score = s_t * qbar[c_t], with qbar the sum
    of the group's query rows (small integers: every value exact)."""
    rng = np.random.default_rng(164)
    B, Hkv, G, N = 2, 3, 2, 70
    q = rng.integers(-4, 5, (B, Hkv * G, 128)).astype(np.float32)
    K = np.zeros((B, Hkv, N, 128), np.float32)
    c = rng.integers(0, 128, (B, Hkv, N))
    sc = rng.integers(-3, 4, (B, Hkv, N)).astype(np.float32)
    for b in range(B):
        for h in range(Hkv):
            for t in range(N):
                K[b, h, t, c[b, h, t]] = sc[b, h, t]
    got = O.dense_scores(_bf16(q), _bf16(K), Hkv, N)
    for b in range(B):
        for h in range(Hkv):
            qbar = q[b, h * G] + q[b, h * G + 1]
            for t in range(N):
                assert got[b, h, t] == sc[b, h, t] * qbar[c[b, h, t]]


def test_dense_scores_equal_lut_scores_on_exact_reconstructions():
    """Keys k = alpha * v with v a sign vector, in +/- pairs so that the channel
    mean is exactly 0 and every token's scale is alpha: the key is its own
    reconstruction, so the full dot product equals the LUT-GEMV score."""
    rng = np.random.default_rng(165)
    n_pairs = 200
    signs = rng.choice([-1.0, 1.0], (n_pairs, 128))
    scale = 2.0 ** rng.integers(-3, 3, n_pairs)
    half = signs * scale[:, None]
    rows = np.empty((64 + 2 * n_pairs, 128), np.float32)
    rows[:64] = rng.standard_normal((64, 128))
    rows[64::2] = half
    rows[65::2] = -half
    n = rows.shape[0]
    kb = _bf16(rows)
    e = O.encode(kb[None, None], n)
    assert not np.any(e["mu"])
    q = _bf16(rng.standard_normal((1, 3, 128)))
    lut = O.query_lut(O.group_query(q, 1)[0, 0])
    s_lut = O.lut_scores(lut, e["codes"][0, 0, 64:], e["alpha"][0, 0, 64:])
    s_dense = O.dense_scores(q, kb[None, None], 1, n)[0, 0, 64:]
    np.testing.assert_allclose(s_dense, s_lut, rtol=1e-15, atol=1e-12)
