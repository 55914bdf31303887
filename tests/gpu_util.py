"""Shared helpers of the GPU parity tests (uploading seeded inputs, running the
HIP path through the binding, and the comparison rules).

Comparison rules (page: "Self-Indexing KVCache: Predicting Sparse Attention
from Compressed Keys", §2.1):
  - mean, codes, scales, sink rows: bit-exact;
  - scores: |s_gpu - s_oracle| <= 4e-6 * alpha_t * sum_c |qbar_c| (fp32 look-up
    accumulation of 32 terms, each a 4-term fp32 sum, against fp64);
  - top-k: same size, ascending, distinct, in [64, N); every token in the
    symmetric difference with the oracle's set has |s_t - s_(k)| <= 1e-4 |s_(k)|
    (oracle fp64 scores, s_(k) the k-th largest);
  - attention: per output row, max|o - r| / max|r| <= 2e-3.
"""

from __future__ import annotations

import math
import sys

import numpy as np
import torch

import oracle as O
import sikv_synth as S

SM = 1.0 / math.sqrt(128)
ATTN_TOL = 2e-3
SET_TOL = 1e-4
SCORE_TOL = 4e-6


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def dev_bf16(a_u16: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a_u16).view(np.int16)).cuda().view(torch.bfloat16)


def host_u16(t: torch.Tensor) -> np.ndarray:
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def oracle_head(K_u16_head: np.ndarray, n_tokens: int) -> dict:
    """Oracle encode of one (b, h): K [N, 128] -> mu [128], codes [N,16], alpha [N], k_sink."""
    e = O.encode(K_u16_head[None, None], n_tokens)
    return {k: v[0, 0] for k, v in e.items()}


def oracle_scores(q_u16: np.ndarray, codes, alpha, b: int, h: int, n_kv: int, n_tokens: int):
    return O.head_scores(q_u16, codes, alpha, b, h, n_kv, n_tokens)


def check_topk(gpu_idx: np.ndarray, s: np.ndarray, k: int, n_tokens: int, what: str = ""):
    gi = np.asarray(gpu_idx, np.int64)
    assert gi.shape == (k,), what
    assert np.all(np.diff(gi) > 0), f"{what}: idx not strictly ascending"
    assert gi[0] >= 64 and gi[-1] < n_tokens, what
    ref = O.select_topk(s, k)
    sk_ = np.sort(s)[::-1][k - 1]
    diff = set(gi.tolist()) ^ set(ref.tolist())
    bad = [t for t in diff if abs(s[t - 64] - sk_) > SET_TOL * abs(sk_)]
    assert not bad, f"{what}: {len(bad)} tokens outside the tie band, e.g. {bad[:5]}"
    return len(diff)


def check_rows(out: np.ndarray, ref: np.ndarray, what: str = "", tol: float = ATTN_TOL):
    out = np.asarray(out, np.float64).reshape(-1, 128)
    ref = np.asarray(ref, np.float64).reshape(-1, 128)
    err = np.abs(out - ref).max(axis=1) / np.maximum(np.abs(ref).max(axis=1), 1e-30)
    assert np.all(err <= tol), f"{what}: worst row error {err.max():.3e}"
    return float(err.max())


def check_scores(gpu_s: np.ndarray, s: np.ndarray, alpha: np.ndarray, qbar: np.ndarray, what="",
                 lut_bound=None):
    """lut_bound: bound on |sum_j LUT[j][p_j]| (default sum_c |qbar_c|, exact for the
    sign vertices; with a codebook, sum_j max_p |LUT[j][p]|)."""
    a_bound = np.abs(qbar).sum() if lut_bound is None else lut_bound
    bound = SCORE_TOL * alpha.astype(np.float64) * a_bound + 1e-30
    err = np.abs(gpu_s.astype(np.float64) - s)
    assert np.all(err <= bound), f"{what}: worst score error ratio {(err / bound).max():.3f}"
