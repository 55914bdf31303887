"""GPU parity of the 2-bit value path (quantised values, full-precision sinks)
against the oracle: codes and scale/zero words bit-exact, attention and decode
step within the attention tolerance, the fused append bit-identical to the
separate calls.

Page: "Self-Indexing KVCache: Predicting Sparse Attention from Compressed Keys",
§2.1 item 3 (sinks kept in full precision) and the 2-bit value reading that the
oracle's ``quantize_v`` states.
"""

import numpy as np
import pytest
import torch

import oracle as O
import sikv_synth as S
from gpu_util import SM, check_rows, check_topk, dev_bf16, host_u16, oracle_head, oracle_scores, say

pytestmark = pytest.mark.gpu

sk = pytest.importorskip("bit_self_indexed_amd")


def _edge_rows(V):
    """Plant value rows that hit the degenerate cases of the per-group scheme."""
    V = V.copy()
    one, neg_zero = np.uint16(0x3F80), np.uint16(0x8000)
    V[:, :, 100, :32] = one                       # constant group: scale 0, all codes 0
    V[:, :, 101, 32:64] &= np.uint16(0x7FFF)
    V[:, :, 101, 40] = neg_zero                   # minimum -0: stored zero point +0
    V[:, :, 102, 64:96] = 0                       # all-zero group
    wide = S.bf16_bits_to_f32(V[:, :, 103, 96:]) * np.float32(1024.0)
    V[:, :, 103, 96:] = S.f32_to_bf16_bits(wide)  # wide-range group (|v| up to a few 1000)
    return V


def _with_rows(sel, rows, k):
    """A k-token selection holding `rows` plus the first other tokens of `sel`."""
    rest = [t for t in sel.tolist() if t not in rows][:k - len(rows)]
    return np.array(sorted(rows + rest), np.int32)


def _vq_host(cache, n):
    vq = cache.vq[:, :, :n].cpu().numpy()
    vsz = cache.vsz[:, :, :n].cpu().numpy().view(np.uint16).reshape(vq.shape[:3] + (4, 2))
    return vq, vsz


QV_CASES = [
    ("qv_g4_ragged", S.custom("qv_g4", 1, 4, 1, 3001, 200, n_planted=4, cfg_id=140)),
    ("qv_g5_multi_tile", S.custom("qv_g5", 2, 10, 2, 20123, 1500, n_planted=16, cfg_id=141)),
    ("qv_g8", S.custom("qv_g8", 1, 16, 2, 9100, 777, n_planted=8, cfg_id=142)),
]


@pytest.mark.parametrize("name,w", QV_CASES, ids=[c[0] for c in QV_CASES])
def test_quantised_value_parity(name, w):
    say(f"[qv] case={name} B={w.batch} Hq={w.n_q_heads} Hkv={w.n_kv_heads} N={w.n_tokens} "
        f"k={w.top_k}")
    d = S.draw(w)
    N, G = w.n_tokens, w.group
    Vh = _edge_rows(d["V"])
    K, q = dev_bf16(d["K"]), dev_bf16(d["q"])
    cache = sk.Cache(w.batch, w.n_kv_heads, N + 13, quant_v=True)
    sk.sikv_encode(cache, K)
    n1 = 1000                                     # values written in two calls
    sk.sikv_encode_v(cache, dev_bf16(Vh[:, :, :n1]))
    sk.sikv_encode_v(cache, dev_bf16(Vh[:, :, n1:]), t_begin=n1)
    torch.cuda.synchronize()
    oq, osz = O.quantize_v(Vh)
    gq, gsz = _vq_host(cache, N)
    assert np.array_equal(gq, oq), f"{name}: value codes differ"
    assert np.array_equal(gsz, osz), f"{name}: scale/zero words differ"
    assert np.array_equal(host_u16(cache.v_sink), Vh[:, :, :64])
    # each value record also carries its token's key code
    rec = cache.vrec[:, :, :N].cpu().numpy()
    assert np.array_equal(rec[..., 48:64], cache.codes[:, :, :N].cpu().numpy())

    oc = [[oracle_head(d["K"][b, h], N) for h in range(w.n_kv_heads)] for b in range(w.batch)]
    oidx = np.zeros((w.batch, w.n_kv_heads, w.top_k), np.int32)
    for b in range(w.batch):
        for h in range(w.n_kv_heads):
            s = oracle_scores(d["q"], oc[b][h]["codes"], oc[b][h]["alpha"], b, h, w.n_kv_heads, N)
            # the edge rows are attended
            oidx[b, h] = _with_rows(O.select_topk(s, w.top_k), [100, 101, 102, 103], w.top_k)
    out = sk.sikv_sparse_attn(cache, q, torch.from_numpy(oidx).cuda(), SM).cpu().numpy()
    idx_out = torch.empty((w.batch, w.n_kv_heads, w.top_k), dtype=torch.int32, device="cuda")
    out2 = sk.sikv_decode_step(cache, q, w.top_k, SM, idx_out=idx_out).cpu().numpy()
    di = idx_out.cpu().numpy()
    for b in range(w.batch):
        for h in range(w.n_kv_heads):
            o = oc[b][h]
            s = oracle_scores(d["q"], o["codes"], o["alpha"], b, h, w.n_kv_heads, N)
            check_topk(di[b, h], s, w.top_k, N, f"{name} topk b={b} h={h}")
            for sel, res, what in ((oidx[b, h], out, "attn"), (di[b, h], out2, "decode")):
                ref = O.sparse_attention(d["q"][b, h * G:(h + 1) * G], sel, o["k_sink"],
                                         o["codes"], o["alpha"], o["mu"], Vh[b, h], SM,
                                         vq=(oq[b, h], osz[b, h]))
                check_rows(res[b, h * G:(h + 1) * G], ref, f"{name} {what} b={b} h={h}")


def test_quantised_value_fused_append():
    """sikv_append_decode_step with v_new == sikv_encode + sikv_encode_v of the new
    token + sikv_decode_step, bit for bit, at a small and a multi-tile size."""
    for w in (S.custom("qv_fused_small", 1, 4, 1, 3000, 200, n_planted=8, cfg_id=150),
              S.custom("qv_fused_multi", 2, 8, 2, 9000, 700, n_planted=8, cfg_id=151)):
        say(f"[qv] case={w.name} N={w.n_tokens}")
        d = S.draw(w)
        K, V, q = dev_bf16(d["K"]), dev_bf16(d["V"]), dev_bf16(d["q"])
        N = w.n_tokens
        res = []
        for fused in (False, True):
            cache = sk.Cache(w.batch, w.n_kv_heads, N, quant_v=True)
            sk.sikv_encode(cache, K[:, :, :N - 1])
            sk.sikv_encode_v(cache, V[:, :, :N - 1])
            idx = torch.empty((w.batch, w.n_kv_heads, w.top_k), dtype=torch.int32, device="cuda")
            if fused:
                out = sk.sikv_append_decode_step(cache, K[:, :, N - 1:N], q, w.top_k, SM,
                                                 idx_out=idx, v_new=V[:, :, N - 1:N])
            else:
                sk.sikv_encode(cache, K[:, :, N - 1:N], t_begin=N - 1, recompute_mu=False)
                sk.sikv_encode_v(cache, V[:, :, N - 1:N], t_begin=N - 1)
                out = sk.sikv_decode_step(cache, q, w.top_k, SM, idx_out=idx)
            torch.cuda.synchronize()
            vq, vsz = _vq_host(cache, N)
            rec = cache.vrec[:, :, N - 1].cpu().numpy()
            res.append((vq[:, :, N - 1], vsz[:, :, N - 1], idx.cpu().numpy(),
                        out.cpu().numpy().view(np.uint32), rec))
        assert np.array_equal(res[1][4][..., 48:64], cache.codes[:, :, N - 1].cpu().numpy())
        for a, b, what in zip(res[0], res[1], ("vq", "vsz", "idx", "out", "record")):
            assert np.array_equal(a, b), f"{w.name}: {what} differs"
        oq, osz = O.quantize_v(d["V"][:, :, N - 1:N])
        assert np.array_equal(res[1][0], oq[:, :, 0])
        assert np.array_equal(res[1][1], osz[:, :, 0])
        # and the output matches the oracle over the selection made
        G = w.group
        oqa, osza = O.quantize_v(d["V"])
        for b in range(w.batch):
            for h in range(w.n_kv_heads):
                o = oracle_head(d["K"][b, h, :N - 1], N - 1)
                app = O.encode_rows(d["K"][b, h, N - 1:N], o["mu"])
                call = np.concatenate([o["codes"], app["codes"]])
                aall = np.concatenate([o["alpha"], app["alpha"]])
                ref = O.sparse_attention(d["q"][b, h * G:(h + 1) * G], res[1][2][b, h],
                                         o["k_sink"], call, aall, o["mu"], d["V"][b, h], SM,
                                         vq=(oqa[b, h], osza[b, h]))
                got = res[1][3].view(np.float32)[b, h * G:(h + 1) * G]
                check_rows(got, ref, f"{w.name} out b={b} h={h}")


GROUPS = [(g, qv) for g in range(1, 9) for qv in (False, True)]


@pytest.mark.parametrize("G,quant_v", GROUPS,
                         ids=[f"g{g}_{'2bit' if qv else 'bf16'}" for g, qv in GROUPS])
def test_every_group_size(G, quant_v):
    """Every query-group size the attention kernel is built for (1 to 8 query
    heads per KV head), with either value layout: attention on the oracle's
    selection and the decode step, against the oracle."""
    w = S.custom(f"grp{G}", 2, 2 * G, 2, 2600, 257, n_planted=4, cfg_id=250 + 2 * G + quant_v)
    say(f"[qv] case=group G={G} quant_v={quant_v} B={w.batch} Hq={w.n_q_heads} N={w.n_tokens}")
    d = S.draw(w)
    N = w.n_tokens
    K, V, q = dev_bf16(d["K"]), dev_bf16(d["V"]), dev_bf16(d["q"])
    if quant_v:
        cache = sk.Cache(w.batch, w.n_kv_heads, N, quant_v=True)
        sk.sikv_encode(cache, K)
        sk.sikv_encode_v(cache, V)
        vq = O.quantize_v(d["V"])
    else:
        cache = sk.Cache(w.batch, w.n_kv_heads, N, v=V)
        sk.sikv_encode(cache, K)
    oc = [[oracle_head(d["K"][b, h], N) for h in range(w.n_kv_heads)] for b in range(w.batch)]
    oidx = np.zeros((w.batch, w.n_kv_heads, w.top_k), np.int32)
    for b in range(w.batch):
        for h in range(w.n_kv_heads):
            s = oracle_scores(d["q"], oc[b][h]["codes"], oc[b][h]["alpha"], b, h, w.n_kv_heads, N)
            oidx[b, h] = O.select_topk(s, w.top_k)
    out = sk.sikv_sparse_attn(cache, q, torch.from_numpy(oidx).cuda(), SM).cpu().numpy()
    idx_out = torch.empty((w.batch, w.n_kv_heads, w.top_k), dtype=torch.int32, device="cuda")
    out2 = sk.sikv_decode_step(cache, q, w.top_k, SM, idx_out=idx_out).cpu().numpy()
    di = idx_out.cpu().numpy()
    for b in range(w.batch):
        for h in range(w.n_kv_heads):
            o = oc[b][h]
            s = oracle_scores(d["q"], o["codes"], o["alpha"], b, h, w.n_kv_heads, N)
            check_topk(di[b, h], s, w.top_k, N, f"G={G} topk b={b} h={h}")
            vkw = {"vq": (vq[0][b, h], vq[1][b, h])} if quant_v else {}
            for sel, res, what in ((oidx[b, h], out, "attn"), (di[b, h], out2, "decode")):
                ref = O.sparse_attention(d["q"][b, h * G:(h + 1) * G], sel, o["k_sink"],
                                         o["codes"], o["alpha"], o["mu"], d["V"][b, h], SM, **vkw)
                check_rows(res[b, h * G:(h + 1) * G], ref, f"G={G} {what} b={b} h={h}")


def _midpoint_rows(rng, n_rows):
    """Value rows whose groups put most entries on or beside the rounding
    midpoints z16 + (j + 1/2) s16 of their own group (the bf16 values nearest to
    them and up to two steps either side), over scales from fp16 subnormals to
    a few thousand; a third of the groups have z = 0 and a power-of-two scale,
    where the midpoints are exact bf16 values (ties)."""
    shape = (n_rows, 4)
    e = rng.integers(-26, 12, size=shape).astype(np.float64)
    ties = rng.random(shape) < 1 / 3
    z = np.where(ties, 0.0, rng.normal(size=shape) * 4.0 * 2.0 ** e)
    mx = np.where(ties, 3.0 * 2.0 ** e, z + rng.uniform(0.3, 3.0, size=shape) * 3.0 * 2.0 ** e)
    zb = S.bf16_bits_to_f32(S.f32_to_bf16_bits(z.astype(np.float32)))
    mb = S.bf16_bits_to_f32(S.f32_to_bf16_bits(mx.astype(np.float32)))
    mb = np.maximum(mb, zb)
    # the group's stored zero and scale, as the quantiser defines them
    s = ((mb - zb) / np.float32(3)).astype(np.float32)
    z16 = zb.astype(np.float16).astype(np.float64)
    s16 = s.astype(np.float16).astype(np.float64)
    j = rng.integers(0, 3, size=shape + (30,))
    mid = z16[..., None] + (j + 0.5) * s16[..., None]
    mid = np.where(np.isfinite(mid), mid, zb[..., None])
    b0 = S.f32_to_bf16_bits(mid.astype(np.float32)).astype(np.int32)
    nb = b0 + rng.integers(-2, 3, size=b0.shape)
    # a step that would change the sign or leave the finite values (at +-0 or
    # next to inf) keeps the midpoint itself: the inputs hold no NaN
    keep = ((nb >> 15) == (b0 >> 15)) & (((nb >> 7) & 0xFF) != 0xFF) & (nb >= 0)
    bits = np.where(keep, nb, b0).astype(np.uint16)
    vals = np.clip(S.bf16_bits_to_f32(bits), zb[..., None], mb[..., None])
    g = np.concatenate([zb[..., None], mb[..., None], vals], axis=-1)  # [rows, 4, 32]
    perm = rng.permuted(np.broadcast_to(np.arange(32), g.shape), axis=-1)
    g = np.take_along_axis(g, perm, axis=-1)
    return S.f32_to_bf16_bits(g.reshape(n_rows, 128).astype(np.float32))


def test_value_codes_at_rounding_midpoints():
    """Value codes and (scale, zero) words bit-exact against the oracle where the
    rounding decides: entries on and beside the midpoints between code levels,
    exact ties included, at scales from fp16 subnormals up."""
    B, Hkv, N = 1, 2, 64 + 6000
    rng = np.random.default_rng(np.random.SeedSequence([2024, 12, 3]))
    V = np.stack([_midpoint_rows(rng, N) for _ in range(B * Hkv)]).reshape(B, Hkv, N, 128)
    K = S.f32_to_bf16_bits(rng.normal(size=(B, Hkv, N, 128)).astype(np.float32))
    say(f"[qv] case=midpoints B={B} Hkv={Hkv} N={N}")
    cache = sk.Cache(B, Hkv, N, quant_v=True)
    sk.sikv_encode(cache, dev_bf16(K))
    sk.sikv_encode_v(cache, dev_bf16(V))
    torch.cuda.synchronize()
    oq, osz = O.quantize_v(V)
    gq, gsz = _vq_host(cache, N)
    assert np.array_equal(gsz[:, :, 64:], osz[:, :, 64:]), "scale/zero words differ"
    bad = np.argwhere(gq[:, :, 64:] != oq[:, :, 64:])
    assert bad.size == 0, f"value codes differ at {len(bad)} bytes, first {bad[:4].tolist()}"
