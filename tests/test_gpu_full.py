"""GPU parity at the full workload sizes, in the launch configuration the
benchmark times (same calls, same shapes).  Encode is compared bit-exactly and
the decode step by the selection set rule and the attention bound on a sample
of (batch, KV head) pairs that the oracle recomputes one by one.
"""

import numpy as np
import pytest
import torch

import oracle as O
import sikv_synth as S
from gpu_util import SM, check_rows, check_topk, dev_bf16, host_u16, oracle_head, oracle_scores, say

pytestmark = pytest.mark.gpu

sk = pytest.importorskip("bit_self_indexed_amd")

FULL = ["long_128k", "encode_heavy_32k", "extreme_512k"]


def _heads(w):
    pairs = [(0, 0), (w.batch - 1, w.n_kv_heads - 1), (w.batch // 2, w.n_kv_heads // 2)]
    return sorted(set(pairs))


@pytest.mark.parametrize("name", FULL)
def test_full_size(name):
    w = S.WORKLOADS[name]
    say(f"[full] case={name} B={w.batch} Hq={w.n_q_heads} Hkv={w.n_kv_heads} N={w.n_tokens} "
        f"k={w.top_k}")
    d = S.draw(w)
    say(f"[full] {name}: inputs drawn")
    K, V, q = dev_bf16(d["K"]), dev_bf16(d["V"]), dev_bf16(d["q"])
    cache = sk.Cache(w.batch, w.n_kv_heads, w.n_tokens, v=V)
    sk.sikv_encode(cache, K)
    idx = torch.empty((w.batch, w.n_kv_heads, w.top_k), dtype=torch.int32, device="cuda")
    out = sk.sikv_decode_step(cache, q, w.top_k, SM, idx_out=idx)
    torch.cuda.synchronize()
    say(f"[full] {name}: GPU done")
    gi, go = idx.cpu().numpy(), out.cpu().numpy()
    G = w.group
    for b, h in _heads(w):
        o = oracle_head(d["K"][b, h], w.n_tokens)
        assert np.array_equal(cache.mu[b, h].cpu().numpy().view(np.uint32), o["mu"].view(np.uint32))
        assert np.array_equal(cache.codes[b, h].cpu().numpy(), o["codes"])
        assert np.array_equal(cache.alpha[b, h].cpu().numpy().view(np.uint32),
                              o["alpha"].view(np.uint32))
        assert np.array_equal(host_u16(cache.k_sink[b, h]), o["k_sink"])
        s = oracle_scores(d["q"], o["codes"], o["alpha"], b, h, w.n_kv_heads, w.n_tokens)
        nd = check_topk(gi[b, h], s, w.top_k, w.n_tokens, f"{name} b={b} h={h}")
        ref = O.sparse_attention(d["q"][b, h * G:(h + 1) * G], gi[b, h], o["k_sink"], o["codes"],
                                 o["alpha"], o["mu"], d["V"][b, h], SM)
        err = check_rows(go[b, h * G:(h + 1) * G], ref, f"{name} attn b={b} h={h}")
        planted = set(d["planted"][b, h].tolist())
        recall = len(planted & set(gi[b, h].tolist())) / max(1, len(planted))
        say(f"[full] {name} b={b} h={h}: set diff {nd}, attn err {err:.2e}, planted recall {recall:.2f}")
    del K, V, q, cache
    torch.cuda.empty_cache()
