"""Seeded synthetic inputs for the self-indexing compressed-key decode path.

This module only *draws* inputs: keys, values and queries shaped like the
decode layers of the models the method was evaluated on (Llama-3.1-8B:
32 query heads / 8 KV heads; Qwen2.5-14B: 40 / 8; head dim 128), stored as
bf16 bit patterns in ``uint16`` arrays.  It contains none of the method's
arithmetic (no channel means, sign codes, scales, lookup tables, scores,
selection or attention) so that both the CPU oracle and the HIP path can
consume it without sharing any of the computation they are compared on.

Recipe (all draws are float32, applied in this order, then rounded to bf16
with round-to-nearest-even):

1. per-channel offset ``m_c ~ N(0, 2)`` (variance 2); one draw shared by
   every (batch, KV head) unless ``mu_per_head`` (then one per head);
2. ``K[t, c] = m_c + z``, ``z ~ N(0, 1)``;
3. planted relevant tokens at distinct uniformly random positions in
   ``[64, N)``: ``K[t] = 3 * sqrt(128) * u_h + z'`` with ``z' ~ N(0, 1)`` and
   ``u_h`` the unit vector of the sum of the KV head's query group;
4. optional recency bias on the last 4096 tokens:
   ``K[t] += 2 * exp(-d / 1024) * sqrt(128) * u_h`` with ``d = N - 1 - t``;
5. four outlier channels (shared by all heads) multiplied by 8 on every row;
6. queries ``q ~ N(0, 1)`` per query head, values ``V ~ N(0, 1)``.

Every array is drawn from ``numpy.random.default_rng(SeedSequence([cfg_id,
tag, ...]))`` with tags 1 (offsets), 2 (outlier channels), 3 (queries),
4 (key noise), 5 (planted positions), 6 (planted noise), 7 (values), so any
(batch, head) slice can be regenerated on its own.
"""

from __future__ import annotations

import dataclasses
import math

import numpy as np

HEAD_DIM = 128
N_SINK = 64


@dataclasses.dataclass(frozen=True)
class Workload:
    """Shape and recipe of one synthetic decode workload."""

    name: str
    cfg_id: int
    batch: int
    n_q_heads: int
    n_kv_heads: int
    n_tokens: int
    top_k: int
    n_planted: int
    mu_per_head: bool = False
    recency: bool = False
    description: str = ""

    @property
    def group(self) -> int:
        return self.n_q_heads // self.n_kv_heads

    @property
    def n_candidates(self) -> int:
        return self.n_tokens - N_SINK

    def with_(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


# The five workloads: a tiny single-head case the oracle finishes instantly,
# a Llama-3-8B-shaped 32K layer, the 128K long-context case (7.5 % of the
# tokens kept), an encode-heavy batch-16 prefill-then-decode case, and a
# 512K Qwen2.5-14B-shaped case with a recency bias.
WORKLOADS = {
    "tiny_4k": Workload(
        "tiny_4k", 0, 1, 1, 1, 4096, 256, 16,
        description="1 query head, 1 KV head, N=4096, top-k 256 + 64 sinks"),
    "llama8b_32k": Workload(
        "llama8b_32k", 1, 1, 32, 8, 32768, 2048, 16,
        description="Llama-3-8B-shaped layer, B=1, 32/8 heads, N=32768, top-k 2048"),
    "long_128k": Workload(
        "long_128k", 2, 4, 32, 8, 131072, 9830, 64,
        description="B=4, 32/8 heads, N=131072, top-k 9830 (7.5 %) + 64 sinks"),
    "encode_heavy_32k": Workload(
        "encode_heavy_32k", 3, 16, 32, 8, 32768, 1024, 16, mu_per_head=True,
        description="B=16, 32/8 heads, N=32768, per-head channel offsets, top-k 1024"),
    "extreme_512k": Workload(
        "extreme_512k", 4, 1, 40, 8, 524288, 4096, 128, recency=True,
        description="Qwen2.5-14B-shaped, B=1, 40/8 heads, N=524288, top-k 4096, recency bias"),
}


def custom(name: str, batch: int, n_q_heads: int, n_kv_heads: int, n_tokens: int,
           top_k: int, n_planted: int = 8, cfg_id: int = 100, **kw) -> Workload:
    """A workload of arbitrary shape (parity and edge-case tests)."""
    return Workload(name, cfg_id, batch, n_q_heads, n_kv_heads, n_tokens, top_k,
                    n_planted, **kw)


def _rng(*key: int) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence([int(k) for k in key]))


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bf16 (nearest, ties to even); returns uint16 bit patterns."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    r = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(u: np.ndarray) -> np.ndarray:
    return (np.asarray(u, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def draw_queries(w: Workload) -> np.ndarray:
    """q as bf16 bits, shape [B, Hq, 128]."""
    out = np.empty((w.batch, w.n_q_heads, HEAD_DIM), np.uint16)
    for b in range(w.batch):
        out[b] = f32_to_bf16_bits(
            _rng(w.cfg_id, 3, b).standard_normal((w.n_q_heads, HEAD_DIM), dtype=np.float32))
    return out


def _offsets(w: Workload, b: int, h: int) -> np.ndarray:
    key = (w.cfg_id, 1, b, h) if w.mu_per_head else (w.cfg_id, 1)
    return (_rng(*key).standard_normal(HEAD_DIM, dtype=np.float32)
            * np.float32(math.sqrt(2.0))).astype(np.float32)


def outlier_channels(w: Workload) -> np.ndarray:
    return np.sort(_rng(w.cfg_id, 2).choice(HEAD_DIM, 4, replace=False))


def planted_positions(w: Workload, b: int, h: int) -> np.ndarray:
    n = min(w.n_planted, w.n_candidates)
    if n <= 0:
        return np.zeros(0, np.int64)
    return np.sort(_rng(w.cfg_id, 5, b, h).choice(w.n_candidates, n, replace=False) + N_SINK)


def _group_direction(q_bits: np.ndarray, w: Workload, b: int, h: int) -> np.ndarray:
    g0 = h * w.group
    s = bf16_bits_to_f32(q_bits[b, g0:g0 + w.group]).sum(axis=0, dtype=np.float32)
    nrm = float(np.linalg.norm(s))
    return (s / np.float32(nrm if nrm > 0 else 1.0)).astype(np.float32)


def draw_keys_head(w: Workload, q_bits: np.ndarray, b: int, h: int,
                   n_rows: int | None = None) -> np.ndarray:
    """K rows [n_rows, 128] (bf16 bits) of one (batch, KV head)."""
    n = w.n_tokens if n_rows is None else n_rows
    k = _rng(w.cfg_id, 4, b, h).standard_normal((n, HEAD_DIM), dtype=np.float32)
    k += _offsets(w, b, h)[None, :]
    u = _group_direction(q_bits, w, b, h)
    scale = np.float32(math.sqrt(HEAD_DIM))
    pos = planted_positions(w, b, h)
    pos = pos[pos < n]
    if pos.size:
        noise = _rng(w.cfg_id, 6, b, h).standard_normal((pos.size, HEAD_DIM), dtype=np.float32)
        k[pos] = np.float32(3.0) * scale * u[None, :] + noise
    if w.recency:
        t0 = max(N_SINK, w.n_tokens - 4096)
        t = np.arange(t0, min(n, w.n_tokens))
        if t.size:
            d = (w.n_tokens - 1 - t).astype(np.float32)
            bias = (np.float32(2.0) * np.exp(-d / np.float32(1024.0)) * scale).astype(np.float32)
            k[t] += bias[:, None] * u[None, :]
    k[:, outlier_channels(w)] *= np.float32(8.0)
    return f32_to_bf16_bits(k)


def draw_values_head(w: Workload, b: int, h: int, n_rows: int | None = None) -> np.ndarray:
    n = w.n_tokens if n_rows is None else n_rows
    return f32_to_bf16_bits(
        _rng(w.cfg_id, 7, b, h).standard_normal((n, HEAD_DIM), dtype=np.float32))


def draw(w: Workload, with_values: bool = True) -> dict:
    """All inputs of a workload: q [B,Hq,D], K and V [B,Hkv,N,D] as bf16 bits."""
    q = draw_queries(w)
    K = np.empty((w.batch, w.n_kv_heads, w.n_tokens, HEAD_DIM), np.uint16)
    V = np.empty_like(K) if with_values else None
    for b in range(w.batch):
        for h in range(w.n_kv_heads):
            K[b, h] = draw_keys_head(w, q, b, h)
            if with_values:
                V[b, h] = draw_values_head(w, b, h)
    planted = np.stack([np.stack([planted_positions(w, b, h) for h in range(w.n_kv_heads)])
                        for b in range(w.batch)])
    return {"q": q, "K": K, "V": V, "planted": planted, "workload": w}
