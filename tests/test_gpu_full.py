"""GPU parity at the full workload sizes, through the call the benchmark times.

The benchmark's step is: prefill of tokens 0..N-2 with ``sikv_encode`` (the
channel mean is frozen there), then one ``sikv_append_decode_step`` that
encodes token N-1 inside the step and runs the decode step over all N tokens.
These tests run exactly that sequence at the workloads' full sizes, so the
score kernel takes the same tile shape (2048-token tiles) and the attention
the same grid as in the benchmark, and check EVERY (batch, KV head) pair
against the oracle:

  - prefill mean, codes, scales and sink rows bit-exact, and the appended
    row's code and scale bit-exact (oracle ``encode`` then ``encode_rows``
    with the frozen mean);
  - 2-bit value records (codes, scale/zero words, key code copy) bit-exact,
    the appended value row included;
  - the selection by the set rule against the oracle's fp64 scores;
  - attention within 2e-3 per row, on the GPU's selection;
  - a second identical step (the benchmark repeats the same append) gives
    bit-identical idx and output.

Layouts: contiguous with bf16 values, contiguous with 2-bit values, and a
paged pool of 256-token pages in a shuffled order (the benchmark's paged
variant), where the GPU arrays are gathered back through the page table
before the comparison.

Page: "Self-Indexing KVCache: Predicting Sparse Attention from Compressed Keys",
§2.1 items 1-4.
"""

import numpy as np
import pytest
import torch

import oracle as O
import sikv_synth as S
from gpu_util import SM, check_rows, check_topk, dev_bf16, host_u16, say

pytestmark = pytest.mark.gpu

sk = pytest.importorskip("bit_self_indexed_amd")

PAGE = 256
_DRAWS = {}


def _draw(name):
    """One draw per workload for the whole module (drawing 1 GiB of keys and
    values takes seconds); the largest is dropped before another is made."""
    if name not in _DRAWS:
        _DRAWS.clear()
        say(f"[full] drawing {name}")
        _DRAWS[name] = S.draw(S.WORKLOADS[name])
    return _DRAWS[name]


def _from_pool(pool, table):
    """Pool rows [n_pages, Hkv, P, ...] -> the logical [B, Hkv, pps * P, ...] arrays."""
    B, pps = table.shape
    g = pool[table.reshape(-1).long()]                        # [B * pps, Hkv, P, ...]
    g = g.view((B, pps) + tuple(pool.shape[1:]))
    g = g.transpose(1, 2)                                     # [B, Hkv, pps, P, ...]
    return g.reshape((B, pool.shape[1], pps * pool.shape[2]) + tuple(pool.shape[3:]))


def _run_bench_sequence(w, d, layout):
    """The benchmark's step on a fresh cache; returns host copies of everything
    the checks read."""
    B, Hkv, N = w.batch, w.n_kv_heads, w.n_tokens
    K, q = dev_bf16(d["K"]), dev_bf16(d["q"])
    V = dev_bf16(d["V"])
    quant_v = layout == "2bit_v"
    if layout == "paged":
        pps = (N + PAGE - 1) // PAGE
        n_pages = B * pps
        gen = torch.Generator(device="cpu")
        gen.manual_seed(7)
        perm = torch.randperm(n_pages, generator=gen).to(torch.int32)
        table = perm.view(B, pps).cuda()
        Vpad = torch.zeros((B, Hkv, pps * PAGE, 128), dtype=torch.bfloat16, device="cuda")
        Vpad[:, :, :N] = V
        pool = torch.empty((n_pages, Hkv, PAGE, 128), dtype=torch.bfloat16, device="cuda")
        pool[perm.cuda().long()] = Vpad.view(B, Hkv, pps, PAGE, 128).permute(
            0, 2, 1, 3, 4).reshape(n_pages, Hkv, PAGE, 128)
        del Vpad
        cache = sk.Cache.paged(B, Hkv, PAGE, n_pages, table, v=pool)
        cache.n_tokens = N - 1
    else:
        cache = sk.Cache(B, Hkv, N, v=None if quant_v else V, quant_v=quant_v)
    sk.sikv_encode(cache, K[:, :, :N - 1])                     # prefill, mean frozen here
    if quant_v:
        sk.sikv_encode_v(cache, V[:, :, :N - 1])
    idx = torch.empty((B, Hkv, w.top_k), dtype=torch.int32, device="cuda")
    out = torch.empty((B, w.n_q_heads, 128), dtype=torch.float32, device="cuda")
    runs = []
    for _ in range(2):                                         # the benchmark repeats the step
        cache.n_tokens = N - 1
        sk.sikv_append_decode_step(cache, K[:, :, N - 1:N], q, w.top_k, SM, idx_out=idx, out=out,
                                   v_new=V[:, :, N - 1:N] if quant_v else None)
        torch.cuda.synchronize()
        runs.append((idx.cpu().numpy().copy(), out.cpu().numpy().copy()))
    assert np.array_equal(runs[0][0], runs[1][0]), "idx differs between identical steps"
    assert np.array_equal(runs[0][1], runs[1][1]), "output differs between identical steps"
    res = {"idx": runs[0][0], "out": runs[0][1],
           "mu": cache.mu.cpu().numpy(), "k_sink": host_u16(cache.k_sink)}
    if layout == "paged":
        res["codes"] = _from_pool(cache.codes, cache.page_table)[:, :, :N].cpu().numpy()
        res["alpha"] = _from_pool(cache.alpha, cache.page_table)[:, :, :N].cpu().numpy()
    else:
        res["codes"] = cache.codes[:, :, :N].cpu().numpy()
        res["alpha"] = cache.alpha[:, :, :N].cpu().numpy()
    if quant_v:
        rec = cache.vrec[:, :, :N].cpu().numpy()
        res["vq"] = rec[..., :32]
        res["vsz"] = np.ascontiguousarray(rec[..., 32:48]).view(np.uint16).reshape(
            rec.shape[:3] + (4, 2))
        res["keycopy"] = rec[..., 48:64]
        res["v_sink"] = host_u16(cache.v_sink)
    del cache, K, V, q, idx, out
    torch.cuda.empty_cache()
    return res


def _check_pair(w, d, r, b, h, quant_v):
    N, G = w.n_tokens, w.group
    Kh = d["K"][b, h]
    pre = O.encode(Kh[None, None, :N - 1], N - 1)
    mu = pre["mu"][0, 0]
    app = O.encode_rows(Kh[N - 1:N], mu)
    codes = np.concatenate([pre["codes"][0, 0], app["codes"]])
    alpha = np.concatenate([pre["alpha"][0, 0], app["alpha"]])
    what = f"{w.name} b={b} h={h}"
    assert np.array_equal(r["mu"][b, h].view(np.uint32), mu.view(np.uint32)), f"{what}: mu"
    assert np.array_equal(r["k_sink"][b, h], pre["k_sink"][0, 0]), f"{what}: k_sink"
    assert np.array_equal(r["codes"][b, h, :N - 1], codes[:N - 1]), f"{what}: prefill codes"
    assert np.array_equal(r["alpha"][b, h, :N - 1].view(np.uint32),
                          alpha[:N - 1].view(np.uint32)), f"{what}: prefill scales"
    assert np.array_equal(r["codes"][b, h, N - 1], codes[N - 1]), f"{what}: appended code"
    assert r["alpha"][b, h, N - 1].view(np.uint32) == alpha[N - 1].view(np.uint32), \
        f"{what}: appended scale"
    vq = None
    if quant_v:
        oq, osz = O.quantize_v(d["V"][b, h, :N])
        assert np.array_equal(r["vq"][b, h], oq), f"{what}: value codes"
        assert np.array_equal(r["vsz"][b, h], osz), f"{what}: value scale/zero words"
        assert np.array_equal(r["keycopy"][b, h], codes), f"{what}: key code copy"
        assert np.array_equal(r["v_sink"][b, h], d["V"][b, h, :64]), f"{what}: value sinks"
        vq = (oq, osz)
    s = O.head_scores(d["q"], codes, alpha, b, h, w.n_kv_heads, N)
    gi = r["idx"][b, h]
    nd = check_topk(gi, s, w.top_k, N, what)
    ref = O.sparse_attention(d["q"][b, h * G:(h + 1) * G], gi, pre["k_sink"][0, 0], codes, alpha,
                             mu, d["V"][b, h], SM, vq=vq)
    err = check_rows(r["out"][b, h * G:(h + 1) * G], ref, f"{what} attention")
    planted = set(d["planted"][b, h].tolist())
    recall = len(planted & set(gi.tolist())) / max(1, len(planted))
    return nd, err, recall


CASES = [("long_128k", "bf16_v"), ("long_128k", "2bit_v"), ("long_128k", "paged"),
         ("encode_heavy_32k", "bf16_v"), ("extreme_512k", "bf16_v")]


@pytest.mark.parametrize("name,layout", CASES, ids=[f"{n}-{l}" for n, l in CASES])
def test_bench_step_all_pairs(name, layout):
    w = S.WORKLOADS[name]
    say(f"[full] case={name} layout={layout} B={w.batch} Hq={w.n_q_heads} Hkv={w.n_kv_heads} "
        f"N={w.n_tokens} k={w.top_k}: prefill N-1, then sikv_append_decode_step twice")
    d = _draw(name)
    r = _run_bench_sequence(w, d, layout)
    say(f"[full] {name}/{layout}: GPU done, checking {w.batch * w.n_kv_heads} pairs")
    worst, diffs, recalls = 0.0, 0, []
    for b in range(w.batch):
        for h in range(w.n_kv_heads):
            nd, err, rec = _check_pair(w, d, r, b, h, layout == "2bit_v")
            worst, diffs = max(worst, err), diffs + nd
            recalls.append(rec)
    say(f"[full] {name}/{layout}: all {len(recalls)} pairs ok; tie-band set differences {diffs}, "
        f"worst attention row error {worst:.2e}, planted recall min {min(recalls):.2f}")
