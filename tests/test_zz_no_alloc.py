"""The allocation-free entry point, sikv_append_decode_step_static, against the
workspace entry point it is a variant of, sikv_append_decode_step.

Two calls in a row share the library's static device scratch, the second on a
smaller input (fewer heads, fewer tokens, 2-bit values), so that it also shows
that nothing from the first call's scratch contents leaks into the second.  Each
call runs on its own copy of an identical cache, next to the workspace call on
the other copy; the selections must be identical, the outputs within the
attention bound (normwise 2e-3 per row; in fact the kernels are the same and the
outputs bit-identical), the appended rows identical, and the static call's
selection and output must also meet the oracle's set rule and attention bound.
The binding allocates no torch memory for the static call (out and idx given).

Page: "Self-Indexing KVCache: Predicting Sparse Attention from Compressed Keys",
§2.1 items 1-4.
"""

import numpy as np
import pytest
import torch

import oracle as O
import sikv_synth as S
from gpu_util import SM, check_rows, check_topk, dev_bf16, say

pytestmark = pytest.mark.gpu

sk = pytest.importorskip("bit_self_indexed_amd")

CASES = [
    ("first", S.custom("noalloc_big", 2, 8, 2, 20000, 1500, n_planted=16, cfg_id=210), False),
    ("second_smaller", S.custom("noalloc_small", 1, 4, 1, 3000, 200, n_planted=4, cfg_id=211),
     True),
]


def _cache(w, d, quant_v):
    N = w.n_tokens
    K, V = dev_bf16(d["K"]), dev_bf16(d["V"])
    c = sk.Cache(w.batch, w.n_kv_heads, N, v=None if quant_v else V, quant_v=quant_v)
    sk.sikv_encode(c, K[:, :, :N - 1])
    if quant_v:
        sk.sikv_encode_v(c, V[:, :, :N - 1])
    return c, K, V


def test_static_scratch_matches_workspace_call():
    for label, w, quant_v in CASES:
        N, G = w.n_tokens, w.group
        say(f"[no-alloc] {label}: B={w.batch} Hq={w.n_q_heads} Hkv={w.n_kv_heads} N={N} "
            f"k={w.top_k} quant_v={quant_v}")
        d = S.draw(w)
        q = dev_bf16(d["q"])
        ref_c, K, V = _cache(w, d, quant_v)
        st_c, _, _ = _cache(w, d, quant_v)
        kn, vn = K[:, :, N - 1:N], (V[:, :, N - 1:N] if quant_v else None)
        idx_r = torch.empty((w.batch, w.n_kv_heads, w.top_k), dtype=torch.int32, device="cuda")
        idx_s = torch.empty_like(idx_r)
        out_r = torch.empty((w.batch, w.n_q_heads, 128), dtype=torch.float32, device="cuda")
        out_s = torch.empty_like(out_r)
        sk.sikv_append_decode_step(ref_c, kn, q, w.top_k, SM, idx_out=idx_r, out=out_r, v_new=vn)
        torch.cuda.synchronize()
        before = torch.cuda.memory_stats().get("allocation.all.allocated", 0)
        sk.sikv_append_decode_step_static(st_c, kn, q, w.top_k, SM, idx_out=idx_s, out=out_s,
                                          v_new=vn)
        torch.cuda.synchronize()
        assert torch.cuda.memory_stats().get("allocation.all.allocated", 0) == before, \
            "the static call allocated torch memory"
        gi_r, gi_s = idx_r.cpu().numpy(), idx_s.cpu().numpy()
        go_r, go_s = out_r.cpu().numpy(), out_s.cpu().numpy()
        assert np.array_equal(gi_s, gi_r), f"{label}: selections differ"
        err = check_rows(go_s.reshape(-1, 128), go_r.reshape(-1, 128), f"{label}: static vs ws")
        assert torch.equal(st_c.codes[:, :, N - 1], ref_c.codes[:, :, N - 1])
        assert torch.equal(st_c.alpha[:, :, N - 1], ref_c.alpha[:, :, N - 1])
        if quant_v:
            assert torch.equal(st_c.vrec[:, :, N - 1], ref_c.vrec[:, :, N - 1])
        # the static call's own result against the oracle
        codes = st_c.codes[:, :, :N].cpu().numpy()
        alpha = st_c.alpha[:, :, :N].cpu().numpy()
        vq = None
        for b in range(w.batch):
            for h in range(w.n_kv_heads):
                pre = O.encode(d["K"][b:b + 1, h:h + 1, :N - 1], N - 1)
                app = O.encode_rows(d["K"][b, h, N - 1:N], pre["mu"][0, 0])
                assert np.array_equal(codes[b, h, N - 1], app["codes"][0])
                s = O.head_scores(d["q"], codes[b, h], alpha[b, h], b, h, w.n_kv_heads, N)
                check_topk(gi_s[b, h], s, w.top_k, N, f"{label} b={b} h={h}")
                if quant_v:
                    vq = O.quantize_v(d["V"][b, h, :N])
                ref = O.sparse_attention(d["q"][b, h * G:(h + 1) * G], gi_s[b, h],
                                         pre["k_sink"][0, 0], codes[b, h], alpha[b, h],
                                         pre["mu"][0, 0], d["V"][b, h], SM, vq=vq)
                check_rows(go_s[b, h * G:(h + 1) * G], ref, f"{label} attention b={b} h={h}")
        say(f"[no-alloc] {label}: ok (static vs workspace max row error {err:.1e}, "
            f"max abs diff {np.abs(go_s - go_r).max():.1e})")
        del ref_c, st_c, K, V, q
        torch.cuda.empty_cache()
