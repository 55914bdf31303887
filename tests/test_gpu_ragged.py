"""Ragged batches (per-sequence lengths in the cache descriptor) against the
oracle run on each sequence at its own length: prefill through batch-1 views,
then the decode step and the fused append step over the whole batch.

A sequence with fewer than k candidates keeps all of them (k_b = n_b - 64) and
the rest of its idx row is -1.  Equal lengths give results bit-identical to no
length array.
"""

import numpy as np
import pytest
import torch

import oracle as O
import sikv_synth as S
from gpu_util import SM, check_rows, check_topk, dev_bf16, oracle_head, oracle_scores, say

pytestmark = pytest.mark.gpu

sk = pytest.importorskip("bit_self_indexed_amd")

LENGTHS = [5037, 3001, 4100, 300]   # the last: 236 candidates < k
K_TOP = 300


def _prefill(w, d, lengths, quant_v):
    B, Hkv = w.batch, w.n_kv_heads
    cap = w.n_tokens
    V = dev_bf16(d["V"])
    cache = sk.Cache(B, Hkv, cap, v=None if quant_v else V, quant_v=quant_v)
    K = dev_bf16(d["K"])
    for b, n in enumerate(lengths):
        vb = cache.view(b)
        vb.n_tokens = n
        sk.sikv_encode(vb, K[b:b + 1, :, :n])
        if quant_v:
            sk.sikv_encode_v(vb, V[b:b + 1, :, :n])
    cache.n_tokens = max(lengths)
    cache.seq_lens = torch.tensor(lengths, dtype=torch.int32, device="cuda")
    torch.cuda.synchronize()
    return cache


def _check_batch(w, d, lengths, idx, out, quant_v, what):
    G = w.group
    for b, n in enumerate(lengths):
        kb = min(K_TOP, n - 64)
        assert np.all(idx[b, :, kb:] == -1), f"{what} b={b}: tail of the idx row"
        vq = O.quantize_v(d["V"][b, :, :n]) if quant_v else None
        for h in range(w.n_kv_heads):
            o = oracle_head(d["K"][b, h, :n], n)
            s = oracle_scores(d["q"], o["codes"], o["alpha"], b, h, w.n_kv_heads, n)
            check_topk(idx[b, h, :kb], s, kb, n, f"{what} topk b={b} h={h}")
            ref = O.sparse_attention(d["q"][b, h * G:(h + 1) * G], idx[b, h, :kb], o["k_sink"],
                                     o["codes"], o["alpha"], o["mu"], d["V"][b, h], SM,
                                     vq=None if vq is None else (vq[0][h], vq[1][h]))
            check_rows(out[b, h * G:(h + 1) * G], ref, f"{what} attn b={b} h={h}")


@pytest.mark.parametrize("quant_v", [False, True], ids=["bf16_v", "2bit_v"])
def test_ragged_decode_step(quant_v):
    w = S.custom("ragged", len(LENGTHS), 8, 2, max(LENGTHS) + 40, K_TOP, n_planted=8,
                 cfg_id=180)
    say(f"[ragged] lengths={LENGTHS} k={K_TOP} quant_v={quant_v}")
    d = S.draw(w)
    cache = _prefill(w, d, LENGTHS, quant_v)
    # the per-sequence prefill is the oracle's encode at each length
    mu, codes = cache.mu.cpu().numpy(), cache.codes.cpu().numpy()
    for b, n in enumerate(LENGTHS):
        for h in range(w.n_kv_heads):
            o = oracle_head(d["K"][b, h, :n], n)
            assert np.array_equal(mu[b, h].view(np.uint32), o["mu"].view(np.uint32))
            assert np.array_equal(codes[b, h, :n], o["codes"])
    q = dev_bf16(d["q"])
    idx = torch.empty((w.batch, w.n_kv_heads, K_TOP), dtype=torch.int32, device="cuda")
    out = sk.sikv_decode_step(cache, q, K_TOP, SM, idx_out=idx)
    torch.cuda.synchronize()
    _check_batch(w, d, LENGTHS, idx.cpu().numpy(), out.cpu().numpy(), quant_v, "decode")


def test_ragged_fused_append():
    """Each sequence appends its own next token at its own position."""
    w = S.custom("ragged_app", len(LENGTHS), 8, 2, max(LENGTHS) + 40, K_TOP, n_planted=8,
                 cfg_id=181)
    say(f"[ragged] fused append lengths={LENGTHS}")
    d = S.draw(w)
    cache = _prefill(w, d, LENGTHS, False)
    knew = np.stack([d["K"][b, :, n] for b, n in enumerate(LENGTHS)])[:, :, None, :]
    q = dev_bf16(d["q"])
    idx = torch.empty((w.batch, w.n_kv_heads, K_TOP), dtype=torch.int32, device="cuda")
    out = sk.sikv_append_decode_step(cache, dev_bf16(knew), q, K_TOP, SM, idx_out=idx)
    torch.cuda.synchronize()
    new_lengths = [n + 1 for n in LENGTHS]
    assert cache.seq_lens.cpu().tolist() == new_lengths
    codes, alpha = cache.codes.cpu().numpy(), cache.alpha.cpu().numpy()
    G = w.group
    gi, go = idx.cpu().numpy(), out.cpu().numpy()
    for b, n in enumerate(LENGTHS):
        kb = min(K_TOP, n + 1 - 64)
        assert np.all(gi[b, :, kb:] == -1)
        for h in range(w.n_kv_heads):
            pre = oracle_head(d["K"][b, h, :n], n)
            app = O.encode_rows(d["K"][b, h, n:n + 1], pre["mu"])
            assert np.array_equal(codes[b, h, n], app["codes"][0])
            assert np.array_equal(alpha[b, h, n:n + 1].view(np.uint32), app["alpha"].view(np.uint32))
            call = np.concatenate([pre["codes"], app["codes"]])
            aall = np.concatenate([pre["alpha"], app["alpha"]])
            s = oracle_scores(d["q"], call, aall, b, h, w.n_kv_heads, n + 1)
            check_topk(gi[b, h, :kb], s, kb, n + 1, f"append topk b={b} h={h}")
            ref = O.sparse_attention(d["q"][b, h * G:(h + 1) * G], gi[b, h, :kb], pre["k_sink"],
                                     call, aall, pre["mu"], d["V"][b, h], SM)
            check_rows(go[b, h * G:(h + 1) * G], ref, f"append attn b={b} h={h}")


def test_equal_lengths_match_no_length_array():
    w = S.custom("ragged_eq", 2, 8, 2, 6000, 500, n_planted=8, cfg_id=182)
    say("[ragged] equal lengths == no lengths")
    d = S.draw(w)
    K, V, q = dev_bf16(d["K"]), dev_bf16(d["V"]), dev_bf16(d["q"])
    res = []
    for with_lens in (False, True):
        cache = sk.Cache(w.batch, w.n_kv_heads, w.n_tokens, v=V)
        sk.sikv_encode(cache, K)
        if with_lens:
            cache.seq_lens = torch.full((w.batch,), w.n_tokens, dtype=torch.int32, device="cuda")
        idx = torch.empty((w.batch, w.n_kv_heads, w.top_k), dtype=torch.int32, device="cuda")
        out = sk.sikv_decode_step(cache, q, w.top_k, SM, idx_out=idx)
        torch.cuda.synchronize()
        res.append((idx.cpu().numpy(), out.cpu().numpy().view(np.uint32)))
    assert np.array_equal(res[0][0], res[1][0])
    assert np.array_equal(res[0][1], res[1][1])
