"""GPU parity of the HIP path (through the C ABI) against the CPU oracle, on
seeded inputs that span several tiles with ragged tails, plus edge cases.

Marked `gpu`: needs an MI355X and the built library; there is no fallback.
"""

import math

import numpy as np
import pytest
import torch

import oracle as O
import sikv_synth as S
from gpu_util import (SM, check_rows, check_scores, check_topk, dev_bf16, host_u16, oracle_head,
                      oracle_scores, say)

pytestmark = pytest.mark.gpu

sk = pytest.importorskip("bit_self_indexed_amd")

CASES = [
    # name, B, Hq, Hkv, N, k, capacity extra
    ("tiny_4k", None),
    ("g3_ragged", S.custom("g3_ragged", 2, 6, 2, 5037, 300, n_planted=8, cfg_id=101)),
    ("g8_k1", S.custom("g8_k1", 1, 8, 1, 3001, 1, n_planted=4, cfg_id=102)),
    ("g1_all", S.custom("g1_all", 3, 3, 3, 2100, 2036, n_planted=4, cfg_id=103)),
    ("one_candidate", S.custom("one_candidate", 1, 4, 1, 65, 1, n_planted=1, cfg_id=104)),
    ("g5_multi_tile", S.custom("g5_multi_tile", 2, 10, 2, 20123, 1500, n_planted=16, cfg_id=105)),
    ("llama8b_32k", None),
]


def _workload(name, w):
    return S.WORKLOADS[name] if w is None else w


def _setup(w, extra_capacity=29):
    d = S.draw(w)
    cap = w.n_tokens + extra_capacity
    K = dev_bf16(d["K"])
    V = torch.zeros((w.batch, w.n_kv_heads, cap, 128), dtype=torch.bfloat16, device="cuda")
    V[:, :, :w.n_tokens] = dev_bf16(d["V"])
    q = dev_bf16(d["q"])
    cache = sk.Cache(w.batch, w.n_kv_heads, cap, v=V)
    return d, K, V, q, cache


def _oracle_cache(d, w):
    return [[oracle_head(d["K"][b, h], w.n_tokens) for h in range(w.n_kv_heads)]
            for b in range(w.batch)]


@pytest.mark.parametrize("name,w", CASES, ids=[c[0] for c in CASES])
def test_parity_case(name, w):
    w = _workload(name, w)
    say(f"[parity] case={name} B={w.batch} Hq={w.n_q_heads} Hkv={w.n_kv_heads} "
        f"N={w.n_tokens} k={w.top_k}")
    d, K, V, q, cache = _setup(w)
    oc = _oracle_cache(d, w)

    # encode: bit-exact
    sk.sikv_encode(cache, K)
    torch.cuda.synchronize()
    mu, codes = cache.mu.cpu().numpy(), cache.codes.cpu().numpy()
    alpha, ksink = cache.alpha.cpu().numpy(), host_u16(cache.k_sink)
    for b in range(w.batch):
        for h in range(w.n_kv_heads):
            o = oc[b][h]
            assert np.array_equal(mu[b, h].view(np.uint32), o["mu"].view(np.uint32)), (b, h)
            assert np.array_equal(codes[b, h, :w.n_tokens], o["codes"]), (b, h)
            assert np.array_equal(alpha[b, h, :w.n_tokens].view(np.uint32),
                                  o["alpha"].view(np.uint32)), (b, h)
            assert np.array_equal(ksink[b, h], o["k_sink"]), (b, h)

    # scores and top-k
    scores = torch.full((w.batch, w.n_kv_heads, cache.capacity), float("nan"), device="cuda")
    idx = sk.sikv_score_topk(cache, q, w.top_k, scores=scores)
    torch.cuda.synchronize()
    gs, gi = scores.cpu().numpy(), idx.cpu().numpy()
    qbar = O.group_query(d["q"], w.n_kv_heads)
    oidx = np.zeros((w.batch, w.n_kv_heads, w.top_k), np.int32)
    for b in range(w.batch):
        for h in range(w.n_kv_heads):
            o = oc[b][h]
            s = oracle_scores(d["q"], o["codes"], o["alpha"], b, h, w.n_kv_heads, w.n_tokens)
            check_scores(gs[b, h, 64:w.n_tokens], s, o["alpha"][64:w.n_tokens], qbar[b, h],
                         f"{name} scores b={b} h={h}")
            check_topk(gi[b, h], s, w.top_k, w.n_tokens, f"{name} topk b={b} h={h}")
            oidx[b, h] = O.select_topk(s, w.top_k)

    # exact whole-head selection path gives the identical selection
    idx2 = sk.sikv_score_topk(cache, q, w.top_k, exact_select=True)
    torch.cuda.synchronize()
    assert np.array_equal(idx2.cpu().numpy(), gi)

    # attention on the oracle's selection
    G = w.group
    out = sk.sikv_sparse_attn(cache, q, torch.from_numpy(oidx).cuda(), SM)
    torch.cuda.synchronize()
    go = out.cpu().numpy()
    for b in range(w.batch):
        for h in range(w.n_kv_heads):
            o = oc[b][h]
            ref = O.sparse_attention(d["q"][b, h * G:(h + 1) * G], oidx[b, h], o["k_sink"],
                                     o["codes"], o["alpha"], o["mu"], d["V"][b, h], SM)
            check_rows(go[b, h * G:(h + 1) * G], ref, f"{name} attn b={b} h={h}")

    # decode step end to end: selection by the set rule, output against the
    # oracle's attention over the GPU's own selection
    idx_out = torch.empty((w.batch, w.n_kv_heads, w.top_k), dtype=torch.int32, device="cuda")
    out2 = sk.sikv_decode_step(cache, q, w.top_k, SM, idx_out=idx_out)
    torch.cuda.synchronize()
    di, do = idx_out.cpu().numpy(), out2.cpu().numpy()
    assert np.array_equal(di, gi)
    for b in range(w.batch):
        for h in range(w.n_kv_heads):
            o = oc[b][h]
            ref = O.sparse_attention(d["q"][b, h * G:(h + 1) * G], di[b, h], o["k_sink"],
                                     o["codes"], o["alpha"], o["mu"], d["V"][b, h], SM)
            check_rows(do[b, h * G:(h + 1) * G], ref, f"{name} decode b={b} h={h}")

    # determinism: a second run is bitwise identical
    out3 = sk.sikv_decode_step(cache, q, w.top_k, SM, idx_out=idx_out)
    torch.cuda.synchronize()
    assert np.array_equal(idx_out.cpu().numpy(), di)
    assert np.array_equal(out3.cpu().numpy().view(np.uint32), do.view(np.uint32))


def test_append_and_strided_inputs():
    w = S.custom("append", 2, 8, 2, 6100, 700, n_planted=8, cfg_id=110)
    say(f"[parity] case=append_strided N={w.n_tokens}")
    d = S.draw(w)
    n0 = w.n_tokens - 37
    # keys stored token-major [B, N, Hkv, 128] and passed as a strided view
    Kt = dev_bf16(np.ascontiguousarray(d["K"].transpose(0, 2, 1, 3)))
    Kview = Kt.permute(0, 2, 1, 3)
    Vt = dev_bf16(np.ascontiguousarray(d["V"].transpose(0, 2, 1, 3)))
    Vview = Vt.permute(0, 2, 1, 3)
    q = dev_bf16(d["q"])
    cache = sk.Cache(w.batch, w.n_kv_heads, w.n_tokens + 100, v=Vview)
    sk.sikv_encode(cache, Kview[:, :, :n0])
    sk.sikv_encode(cache, Kview[:, :, n0:], t_begin=n0, recompute_mu=False)
    cache.n_tokens = w.n_tokens
    torch.cuda.synchronize()
    codes, alpha, mu = cache.codes.cpu().numpy(), cache.alpha.cpu().numpy(), cache.mu.cpu().numpy()
    G = w.group
    idx_out = torch.empty((w.batch, w.n_kv_heads, w.top_k), dtype=torch.int32, device="cuda")
    out = sk.sikv_decode_step(cache, q, w.top_k, SM, idx_out=idx_out).cpu().numpy()
    gi = idx_out.cpu().numpy()
    for b in range(w.batch):
        for h in range(w.n_kv_heads):
            pre = oracle_head(d["K"][b, h, :n0], n0)
            app = O.encode_rows(d["K"][b, h, n0:], pre["mu"])
            assert np.array_equal(mu[b, h].view(np.uint32), pre["mu"].view(np.uint32))
            assert np.array_equal(codes[b, h, :n0], pre["codes"])
            assert np.array_equal(codes[b, h, n0:w.n_tokens], app["codes"])
            assert np.array_equal(alpha[b, h, n0:w.n_tokens].view(np.uint32),
                                  app["alpha"].view(np.uint32))
            call = np.concatenate([pre["codes"], app["codes"]])
            aall = np.concatenate([pre["alpha"], app["alpha"]])
            s = oracle_scores(d["q"], call, aall, b, h, w.n_kv_heads, w.n_tokens)
            check_topk(gi[b, h], s, w.top_k, w.n_tokens, f"append b={b} h={h}")
            ref = O.sparse_attention(d["q"][b, h * G:(h + 1) * G], gi[b, h], pre["k_sink"], call,
                                     aall, pre["mu"], d["V"][b, h], SM)
            check_rows(out[b, h * G:(h + 1) * G], ref, f"append attn b={b} h={h}")



def test_value_rows_beyond_32bit_offsets():
    """V rows 16 MB apart (a row stride too wide for the attention's 32-bit
    offsets): the kernels' 64-bit addressing form, against the oracle and
    bit-identical to the same values in a compact layout."""
    w = S.custom("wide_v", 1, 8, 2, 160, 64, n_planted=4, cfg_id=111)
    say(f"[parity] case=wide_value_stride N={w.n_tokens}")
    d = S.draw(w)
    N, G = w.n_tokens, w.group
    vst = (1 << 23) + 128                       # elements: 2 * vst bytes >= 2^24
    buf = torch.empty(N * vst, dtype=torch.bfloat16, device="cuda")  # ~2.7 GB
    Vwide = buf.as_strided((1, w.n_kv_heads, N, 128), (N * vst, 128, vst, 1))
    V = dev_bf16(d["V"])
    Vwide.copy_(V)
    K, q = dev_bf16(d["K"]), dev_bf16(d["q"])
    outs, idxs = [], []
    for vv in (Vwide, V):
        cache = sk.Cache(w.batch, w.n_kv_heads, N, v=vv)
        sk.sikv_encode(cache, K)
        idx_out = torch.empty((w.batch, w.n_kv_heads, w.top_k), dtype=torch.int32, device="cuda")
        outs.append(sk.sikv_decode_step(cache, q, w.top_k, SM, idx_out=idx_out).cpu().numpy())
        idxs.append(idx_out.cpu().numpy())
        torch.cuda.synchronize()
    del buf, Vwide
    assert np.array_equal(idxs[0], idxs[1])
    assert np.array_equal(outs[0].view(np.uint32), outs[1].view(np.uint32))
    for h in range(w.n_kv_heads):
        pre = oracle_head(d["K"][0, h], N)
        s = oracle_scores(d["q"], pre["codes"], pre["alpha"], 0, h, w.n_kv_heads, N)
        check_topk(idxs[0][0, h], s, w.top_k, N, f"wide_v h={h}")
        ref = O.sparse_attention(d["q"][0, h * G:(h + 1) * G], idxs[0][0, h], pre["k_sink"],
                                 pre["codes"], pre["alpha"], pre["mu"], d["V"][0, h], SM)
        check_rows(outs[0][0, h * G:(h + 1) * G], ref, f"wide_v attn h={h}")

CB_CASES = [
    ("cb_tiny_4k", None),
    ("cb_g5_multi_tile", S.custom("cb_g5", 2, 10, 2, 20123, 1500, n_planted=16, cfg_id=130)),
    ("cb_mu_per_head", S.custom("cb_mu", 2, 8, 2, 9000, 600, n_planted=8, cfg_id=131,
                                mu_per_head=True)),
]


@pytest.mark.parametrize("name,w", CB_CASES, ids=[c[0] for c in CB_CASES])
def test_codebook_parity(name, w):
    """Data-derived centres: the codebook is bit-exact, scores / top-k / attention /
    decode step match the oracle with the same centres, appends keep them."""
    w = S.WORKLOADS["tiny_4k"] if w is None else w
    say(f"[parity] case={name} B={w.batch} Hq={w.n_q_heads} Hkv={w.n_kv_heads} "
        f"N={w.n_tokens} k={w.top_k}")
    d = S.draw(w)
    N, G = w.n_tokens, w.group
    n0 = N - 5                                        # prefill, then 5 appended tokens
    K, q = dev_bf16(d["K"]), dev_bf16(d["q"])
    V = dev_bf16(d["V"])
    cache = sk.Cache(w.batch, w.n_kv_heads, N, v=V, codebook=True)
    sk.sikv_encode(cache, K[:, :, :n0])
    sk.sikv_encode(cache, K[:, :, n0:], t_begin=n0, recompute_mu=False)
    torch.cuda.synchronize()
    gcb = cache.codebook.cpu().numpy()
    codes, alpha = cache.codes.cpu().numpy(), cache.alpha.cpu().numpy()
    oc = {}
    for b in range(w.batch):
        for h in range(w.n_kv_heads):
            pre = O.encode(d["K"][b, h, :n0][None, None], n0, with_codebook=True)
            app = O.encode_rows(d["K"][b, h, n0:N], pre["mu"][0, 0])
            cb = pre["codebook"][0, 0]
            assert np.array_equal(gcb[b, h].view(np.uint32), cb.view(np.uint32)), (b, h)
            call = np.concatenate([pre["codes"][0, 0], app["codes"]])
            aall = np.concatenate([pre["alpha"][0, 0], app["alpha"]])
            assert np.array_equal(codes[b, h, :N], call)
            assert np.array_equal(alpha[b, h, :N].view(np.uint32), aall.view(np.uint32))
            oc[b, h] = dict(codes=call, alpha=aall, cb=cb, mu=pre["mu"][0, 0],
                            k_sink=pre["k_sink"][0, 0])

    scores = torch.full((w.batch, w.n_kv_heads, N), float("nan"), device="cuda")
    idx = sk.sikv_score_topk(cache, q, w.top_k, scores=scores)
    torch.cuda.synchronize()
    gs, gi = scores.cpu().numpy(), idx.cpu().numpy()
    qbar = O.group_query(d["q"], w.n_kv_heads)
    oidx = np.zeros((w.batch, w.n_kv_heads, w.top_k), np.int32)
    for (b, h), o in oc.items():
        s = O.head_scores(d["q"], o["codes"], o["alpha"], b, h, w.n_kv_heads, N, o["cb"])
        A = np.abs(O.query_lut(qbar[b, h], o["cb"])).max(axis=1).sum()
        check_scores(gs[b, h, 64:N], s, o["alpha"][64:N], qbar[b, h], f"{name} scores b={b} h={h}",
                     lut_bound=A)
        check_topk(gi[b, h], s, w.top_k, N, f"{name} topk b={b} h={h}")
        oidx[b, h] = O.select_topk(s, w.top_k)

    idx2 = sk.sikv_score_topk(cache, q, w.top_k, exact_select=True)
    torch.cuda.synchronize()
    assert np.array_equal(idx2.cpu().numpy(), gi)

    out = sk.sikv_sparse_attn(cache, q, torch.from_numpy(oidx).cuda(), SM).cpu().numpy()
    idx_out = torch.empty_like(idx)
    out2 = sk.sikv_decode_step(cache, q, w.top_k, SM, idx_out=idx_out).cpu().numpy()
    di = idx_out.cpu().numpy()
    assert np.array_equal(di, gi)
    for (b, h), o in oc.items():
        for sel, res, what in ((oidx[b, h], out, "attn"), (di[b, h], out2, "decode")):
            ref = O.sparse_attention(d["q"][b, h * G:(h + 1) * G], sel, o["k_sink"], o["codes"],
                                     o["alpha"], o["mu"], d["V"][b, h], SM, o["cb"])
            check_rows(res[b, h * G:(h + 1) * G], ref, f"{name} {what} b={b} h={h}")


def test_fused_append_matches_separate_calls():
    """sikv_append_decode_step == sikv_encode (append) + sikv_decode_step, bit for bit
    (new row's code and scale, idx, attention output), at a small and a multi-tile size."""
    for w in (S.custom("fused_small", 1, 4, 1, 3000, 200, n_planted=8, cfg_id=120),
              S.custom("fused_multi", 2, 8, 2, 9000, 700, n_planted=8, cfg_id=121)):
        say(f"[parity] case={w.name} N={w.n_tokens}")
        d = S.draw(w)
        K, V, q = dev_bf16(d["K"]), dev_bf16(d["V"]), dev_bf16(d["q"])
        N = w.n_tokens
        res = []
        for fused in (False, True):
            cache = sk.Cache(w.batch, w.n_kv_heads, N, v=V)
            sk.sikv_encode(cache, K[:, :, :N - 1])
            idx = torch.empty((w.batch, w.n_kv_heads, w.top_k), dtype=torch.int32, device="cuda")
            if fused:
                out = sk.sikv_append_decode_step(cache, K[:, :, N - 1:N], q, w.top_k, SM,
                                                 idx_out=idx)
            else:
                sk.sikv_encode(cache, K[:, :, N - 1:N], t_begin=N - 1, recompute_mu=False)
                out = sk.sikv_decode_step(cache, q, w.top_k, SM, idx_out=idx)
            torch.cuda.synchronize()
            assert cache.n_tokens == N
            res.append((cache.codes[:, :, N - 1].cpu().numpy(),
                        cache.alpha[:, :, N - 1].cpu().numpy().view(np.uint32),
                        idx.cpu().numpy(), out.cpu().numpy().view(np.uint32)))
        for a, b, what in zip(res[0], res[1], ("code", "alpha", "idx", "out")):
            assert np.array_equal(a, b), f"{w.name}: {what} differs"
        # and the fused row matches the oracle's append encoding
        for b in range(w.batch):
            for h in range(w.n_kv_heads):
                pre = oracle_head(d["K"][b, h, :N - 1], N - 1)
                app = O.encode_rows(d["K"][b, h, N - 1:N], pre["mu"])
                assert np.array_equal(res[1][0][b, h], app["codes"][0])
                assert np.array_equal(res[1][1][b, h], app["alpha"].view(np.uint32)[0])


def test_all_scores_tied():
    """Identical key rows: every candidate has the same score, so the top-k is the
    k smallest positions (ties go to the smaller position)."""
    w = S.custom("ties", 1, 4, 2, 9000, 777, n_planted=0, cfg_id=111)
    say("[parity] case=all_tied")
    d = S.draw(w)
    K = d["K"].copy()
    K[:, :, 64:] = K[:, :, 64:65]
    cache = sk.Cache(w.batch, w.n_kv_heads, w.n_tokens, v=dev_bf16(d["V"]))
    sk.sikv_encode(cache, dev_bf16(K))
    q = dev_bf16(d["q"])
    idx = sk.sikv_score_topk(cache, q, w.top_k).cpu().numpy()
    expect = np.arange(64, 64 + w.top_k)
    for h in range(w.n_kv_heads):
        assert np.array_equal(idx[0, h], expect)



def test_select_list_in_workspace():
    """More candidates than the select kernel keeps in LDS (16384): the candidate
    list goes to the workspace.  (a) every score tied at N = 20000 (no usable
    score spread: radix rounds over the whole list); (b) random keys with
    k = 15500 of 65472 candidates (about 18K pass the sampled threshold)."""
    w = S.custom("ties_big", 1, 4, 1, 20000, 777, n_planted=0, cfg_id=112)
    say("[parity] case=ties_big")
    d = S.draw(w)
    K = d["K"].copy()
    K[:, :, 64:] = K[:, :, 64:65]
    cache = sk.Cache(w.batch, w.n_kv_heads, w.n_tokens, v=dev_bf16(d["V"]))
    sk.sikv_encode(cache, dev_bf16(K))
    idx = sk.sikv_score_topk(cache, dev_bf16(d["q"]), w.top_k).cpu().numpy()
    assert np.array_equal(idx[0, 0], np.arange(64, 64 + w.top_k))

    w = S.custom("big_k", 1, 4, 1, 65536, 15500, n_planted=16, cfg_id=113)
    say("[parity] case=big_k")
    d = S.draw(w)
    N, G = w.n_tokens, w.group
    q = dev_bf16(d["q"])
    cache = sk.Cache(w.batch, w.n_kv_heads, N, v=dev_bf16(d["V"]))
    sk.sikv_encode(cache, dev_bf16(d["K"]))
    idx_out = torch.empty((1, 1, w.top_k), dtype=torch.int32, device="cuda")
    out = sk.sikv_decode_step(cache, q, w.top_k, SM, idx_out=idx_out).cpu().numpy()
    di = idx_out.cpu().numpy()
    o = oracle_head(d["K"][0, 0], N)
    s = oracle_scores(d["q"], o["codes"], o["alpha"], 0, 0, 1, N)
    check_topk(di[0, 0], s, w.top_k, N, "big_k topk")
    idx2 = sk.sikv_score_topk(cache, q, w.top_k, exact_select=True).cpu().numpy()
    assert np.array_equal(idx2, di)
    ref = O.sparse_attention(d["q"][0, :G], di[0, 0], o["k_sink"], o["codes"], o["alpha"],
                             o["mu"], d["V"][0, 0], SM)
    check_rows(out[0, :G], ref, "big_k decode")


@pytest.mark.parametrize("B,Hkv,parts", [(2, 32, 3), (10, 8, 2), (1, 16, 4), (11, 8, 1)],
                         ids=["3_parts", "2_parts", "4_parts", "1_part"])
def test_select_parts(B, Hkv, parts):
    """The select kernel splits a head's ordered emit over up to four blocks, as
    many as keep its grid (plus one table block per head) within 256 blocks:
    64 heads take 3 parts, 80 take 2, 16 take 4, 88 take 1.  Every head's
    selection must equal the exact whole-head path's and follow the oracle."""
    w = S.custom(f"parts{parts}", B, Hkv, Hkv, 12000, 1100, n_planted=8, cfg_id=230 + parts)
    say(f"[parity] case=select_parts B={B} Hkv={Hkv} parts={parts}")
    d = S.draw(w)
    q = dev_bf16(d["q"])
    cache = sk.Cache(w.batch, w.n_kv_heads, w.n_tokens, v=dev_bf16(d["V"]))
    sk.sikv_encode(cache, dev_bf16(d["K"]))
    gi = sk.sikv_score_topk(cache, q, w.top_k).cpu().numpy()
    ge = sk.sikv_score_topk(cache, q, w.top_k, exact_select=True).cpu().numpy()
    assert np.array_equal(gi, ge)
    for b, h in [(0, 0), (B - 1, Hkv - 1), (B // 2, Hkv // 2)]:
        o = oracle_head(d["K"][b, h], w.n_tokens)
        s = oracle_scores(d["q"], o["codes"], o["alpha"], b, h, w.n_kv_heads, w.n_tokens)
        check_topk(gi[b, h], s, w.top_k, w.n_tokens, f"parts {parts} topk b={b} h={h}")


@pytest.mark.parametrize("n_tied", [40, 100])
def test_tied_keys_at_the_kth(n_tied):
    """n_tied tokens share the key row of the token whose score is the k-th
    largest, so the k-th's histogram bin holds about n_tied keys (40: ranked by
    one wave; 100: more than its 64 lanes, by radix rounds).  The selection takes
    the tied tokens with the smallest positions first, like the oracle's, and
    equals the exact whole-head path's."""
    w = S.custom(f"tied{n_tied}", 1, 4, 1, 9000, 600, n_planted=0, cfg_id=240 + n_tied)
    say(f"[parity] case=tied_keys_at_the_kth n_tied={n_tied}")
    d = S.draw(w)
    K = d["K"].copy()
    N, k = w.n_tokens, w.top_k
    o = oracle_head(K[0, 0], N)
    s = oracle_scores(d["q"], o["codes"], o["alpha"], 0, 0, 1, N)
    t_k = 64 + int(np.argsort(-s, kind="stable")[k - 1])
    rng = np.random.default_rng(7 + n_tied)
    others = rng.choice(np.setdiff1d(np.arange(64, N), [t_k]), n_tied - 1, replace=False)
    K[0, 0, others] = K[0, 0, t_k]
    o = oracle_head(K[0, 0], N)
    s = oracle_scores(d["q"], o["codes"], o["alpha"], 0, 0, 1, N)
    # (the copies move the channel mean a little: take k so that the tied
    # tokens straddle the k-th rank)
    s_tie = s[t_k - 64]
    tied = np.nonzero(s == s_tie)[0] + 64
    assert len(tied) >= n_tied
    k = int((s > s_tie).sum()) + n_tied // 2
    q = dev_bf16(d["q"])
    cache = sk.Cache(w.batch, w.n_kv_heads, N, v=dev_bf16(d["V"]))
    sk.sikv_encode(cache, dev_bf16(K))
    gi = sk.sikv_score_topk(cache, q, k).cpu().numpy()[0, 0]
    ge = sk.sikv_score_topk(cache, q, k, exact_select=True).cpu().numpy()[0, 0]
    assert np.array_equal(gi, ge)
    check_topk(gi, s, k, N, f"tied {n_tied}")
    # the tie rule: of the tied tokens, exactly the smallest positions are taken
    ref = O.select_topk(s, k)
    assert np.array_equal(np.intersect1d(gi, tied), np.intersect1d(ref, tied))
    taken = np.intersect1d(gi, tied)
    assert len(taken) == n_tied // 2 and np.array_equal(taken, tied[:len(taken)])


@pytest.mark.parametrize("stale", ["high", "neg_inf", "zero"])
def test_stale_threshold_word(stale):
    """A tagged threshold word left in the caller's workspace (a fresh buffer may
    hold anything) must not change the selection.  The words lead the workspace,
    8 bytes per (b, KV head): the tag 0x53494b56 in the upper half, the fp32
    threshold in the lower; the select kernel clears each one after reading it.
    Tiles that take the planted word: high, keep nothing (fewer than k
    candidates: whole-head rescan); neg_inf, keep every token, which the select
    kernel accepts (a list of all 39936 candidates, past the LDS list: the
    workspace path); zero, record a threshold other than the one the leader
    publishes (whole-head rescan).  156 tiles per head, so the select kernel's
    long-context gather runs too."""
    w = S.custom("stale", 2, 8, 2, 40000, 3000, n_planted=8, cfg_id=177)
    say(f"[parity] case=stale_threshold_word {stale}")
    d = S.draw(w)
    q = dev_bf16(d["q"])
    cache = sk.Cache(w.batch, w.n_kv_heads, w.n_tokens, v=dev_bf16(d["V"]))
    sk.sikv_encode(cache, dev_bf16(d["K"]))
    first = sk.sikv_score_topk(cache, q, w.top_k).cpu().numpy()  # (sizes the workspace)
    buf = cache.ws.buf
    off = (-buf.data_ptr()) % 256
    words = buf[off:off + 8 * w.batch * w.n_kv_heads].view(torch.int64)
    assert bool(torch.all(words == 0)), "the previous call left its threshold words set"
    tau = {"high": 3.0e38, "neg_inf": float("-inf"), "zero": 0.0}[stale]
    tau_bits = int(np.array([tau], np.float32).view(np.uint32)[0])
    words.fill_((0x53494B56 << 32) | tau_bits)
    torch.cuda.synchronize()
    gi = sk.sikv_score_topk(cache, q, w.top_k).cpu().numpy()
    assert bool(torch.all(words == 0)), "planted threshold words were not read and cleared"
    for b in range(w.batch):
        for h in range(w.n_kv_heads):
            o = oracle_head(d["K"][b, h], w.n_tokens)
            s = oracle_scores(d["q"], o["codes"], o["alpha"], b, h, w.n_kv_heads, w.n_tokens)
            check_topk(gi[b, h], s, w.top_k, w.n_tokens, f"stale {stale} topk b={b} h={h}")
    assert np.array_equal(gi, first)


def test_dense_comparator():
    w = S.custom("dense", 2, 8, 2, 3000, 100, n_planted=4, cfg_id=112)
    say("[parity] case=dense_comparator")
    d = S.draw(w)
    out = sk.sikv_dense_attn(dev_bf16(d["q"]), dev_bf16(d["K"]), dev_bf16(d["V"]), SM)
    out = out.cpu().numpy()
    G = w.group
    for b in range(w.batch):
        for h in range(w.n_kv_heads):
            qf = S.bf16_bits_to_f32(d["q"][b, h * G:(h + 1) * G]).astype(np.float64)
            kf = S.bf16_bits_to_f32(d["K"][b, h]).astype(np.float64)
            vf = S.bf16_bits_to_f32(d["V"][b, h]).astype(np.float64)
            lg = qf @ kf.T * SM
            p = np.exp(lg - lg.max(axis=1, keepdims=True))
            p /= p.sum(axis=1, keepdims=True)
            check_rows(out[b, h * G:(h + 1) * G], p @ vf, f"dense b={b} h={h}", tol=1e-4)


def test_stream_copy():
    src = torch.randint(0, 255, (1 << 20,), dtype=torch.uint8, device="cuda")
    dst = torch.zeros_like(src)
    sk.sikv_stream_copy(dst, src)
    torch.cuda.synchronize()
    assert torch.equal(dst, src)


def test_caller_owned_timer():
    """A Timer attached to one cache times that cache's calls only: one launch of
    each decode kernel per step, positive durations; an untimed cache's calls
    and a second timer see nothing of it."""
    w = S.WORKLOADS["tiny_4k"]
    say("[timer] tiny_4k, two caches, one timed")
    d = S.draw(w)
    K, V, q = dev_bf16(d["K"]), dev_bf16(d["V"]), dev_bf16(d["q"])
    timed, plain = sk.Cache(1, 1, w.n_tokens, v=V), sk.Cache(1, 1, w.n_tokens, v=V)
    for c in (timed, plain):
        sk.sikv_encode(c, K)
    t1, t2 = sk.Timer(), sk.Timer()
    timed.timer = t1
    for _ in range(3):
        o1 = sk.sikv_decode_step(timed, q, w.top_k, SM)
        o2 = sk.sikv_decode_step(plain, q, w.top_k, SM)
    torch.cuda.synchronize()
    r1, r2 = t1.read(), t2.read()
    for name in ("score", "select", "attn", "combine"):
        assert r1[name][0] == 3 and r1[name][1] > 0.0, (name, r1[name])
    assert all(n == 0 for n, _ in r2.values())
    assert r1["codes"][0] == 0          # the prefill ran before the timer was attached
    assert r1["tables"][0] == 0         # the decode step's score kernel builds the tables
    assert torch.equal(o1, o2)
    t1.reset()
    assert all(n == 0 for n, _ in t1.read().values())
    t1.close()
    t2.close()
