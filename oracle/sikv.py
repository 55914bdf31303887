"""Plain, slow CPU oracle of self-indexing compressed-key decode attention.

TEST INFRASTRUCTURE: only the tests, the smoke check and the benchmark's
CPU-baseline leg use this module.  It shares no code with the HIP path.

Source of the method: the web summary of "Self-Indexing KVCache: Predicting
Sparse Attention from Compressed Keys" (arXiv 2603.14224), technical summary.
Citations below name its sections: §1 (problem), §2 (methodology),
§2.1 items 1-4 (core components), §3 (contributions).  The summary prints no
equations, so every formula here is the plainest reading of that prose; each
such reading is marked READING where it is made.

Precision: every score, logit, softmax and weighted sum is fp64.  Two
reductions are fp32 on purpose, because their exact bits decide the sign
codes and are required to match bit for bit: the per-channel mean and the
per-token scale, each summed by an adjacent-pair binary tree (READING: the
summary fixes no summation order; this one is written down here and the GPU
reproduces it).  bf16 inputs are uint16 bit patterns, decoded exactly.

Pins (tests/test_oracle_pins.py checks each function against something other
than itself): tree order (hand-computed leaves), mean (fp64 mean within the
tree error bound), codes (hand-derived layout fixture, brute-force bits,
entropy balance), scale (least-squares optimality, round trip), lookup table
(all 16 sign vertices enumerated, exact identity with the dequantised dot
product), top-k (brute-force sort, heapq), attention (dense softmax attention
through torch's fp64 SDPA when every token is kept, q = 0, one dominant
token), decode step (planted-token recall), codebook (closed-form members,
pure-sign data gives the vertices, least-squares optimality and sign
consistency by perturbation, brute-force channel loop for its scores, dense
SDPA with its reconstructed keys, lower reconstruction error than the
vertices), quantised values (hand-derived layout and codes, exact levels, constant
groups, error bound against the scale, all-tokens attention against SDPA over the
reconstructed values), K-means baseline (one iteration equals the one-pass codebook,
scikit-learn's Lloyd K-means on separated clusters, non-increasing objective), dense
retrieval scores (equal to the LUT scores plus q.mu on keys that are exactly their
own reconstruction).  No function is left unpinned.
"""

from __future__ import annotations

import numpy as np

HEAD_DIM = 128          # D: the only head size of the evaluated models (Llama-3.1-8B, Qwen2.5-14B)
N_SINK = 64             # §2.1 item 3: 64 full-precision sink tokens kept at prefill
SUB_DIM = 4             # §2.1 item 1: keys are split into 4-dimensional sub-vectors
N_SUB = HEAD_DIM // SUB_DIM
N_PATTERNS = 16         # §2.1 item 1: a sub-vector's sign pattern picks one of 16 clusters
CODE_BYTES = HEAD_DIM // 8


# --------------------------------------------------------------------------- #
# bf16 and fixed-order fp32 helpers
# --------------------------------------------------------------------------- #
def bf16_to_f32(bits) -> np.ndarray:
    """Exact decode of bf16 bit patterns (uint16) to float32."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def tree_sum_f32(x, axis: int = -1) -> np.ndarray:
    """Adjacent-pair binary-tree sum in float32 along ``axis``.

    The leaves are padded with +0.0 up to the next power of two P; then, level
    by level, element i of the next level is fl32(x[2i] + x[2i+1]).  Padding to
    any larger power of two gives the same value (the extra subtrees are +0.0
    and are added last).
    """
    x = np.moveaxis(np.asarray(x, dtype=np.float32), axis, -1)
    n = x.shape[-1]
    p = 1
    while p < n:
        p *= 2
    if p != n:
        pad = np.zeros(x.shape[:-1] + (p - n,), np.float32)
        x = np.concatenate([x, pad], axis=-1)
    while x.shape[-1] > 1:
        x = x[..., 0::2] + x[..., 1::2]
    return x[..., 0]


# --------------------------------------------------------------------------- #
# Prefill compression: §2.1 items 1 and 3
# --------------------------------------------------------------------------- #
def channel_mean(k_bits, n_tokens: int) -> np.ndarray:
    """Per-channel mean of the keys that get quantised (§2.1 item 1, entropy-aware
    normalisation: subtract the channel mean so that + and - signs balance).

    READING: the mean runs over the non-sink tokens t in [64, N) of the same
    (batch, KV head); sink rows are stored in full precision (§2.1 item 3) and
    do not enter it.  Sum: ``tree_sum_f32`` over the token axis with the sink
    rows and the rows past N replaced by +0.0; then one correctly rounded fp32
    division by fl32(N - 64).

    k_bits: [..., >=N, 128] bf16 bits.  Returns float32 [..., 128].
    """
    if n_tokens <= N_SINK:
        raise ValueError("need more than 64 tokens")
    x = bf16_to_f32(np.asarray(k_bits)[..., :n_tokens, :]).copy()
    x[..., :N_SINK, :] = np.float32(0.0)
    s = tree_sum_f32(x, axis=-2)
    return (s / np.float32(n_tokens - N_SINK)).astype(np.float32)


def sign_bits(k_bits, mu) -> np.ndarray:
    """Sign of each normalised channel as a bit: 1 iff fp32(k_c) < mu_c (§2.1 item 1,
    sign-based 1-bit VQ).  A tie (k_c == mu_c, also -0 vs +0) gives bit 0, i.e. sign +1.
    Returns bool [..., T, 128]."""
    x = bf16_to_f32(k_bits)
    return x < np.asarray(mu, np.float32)[..., None, :]


def pack_codes(bits) -> np.ndarray:
    """READING (layout): bit c of a token's 16-byte code is channel c, least
    significant bit first: byte c // 8, bit c % 8.  Hence the 4-bit pattern of
    sub-vector j (channels 4j..4j+3) is nibble j, low nibble first, with bit i
    of the pattern = channel 4j + i."""
    return np.packbits(np.asarray(bits, bool), axis=-1, bitorder="little")


def token_scale(k_bits, mu) -> np.ndarray:
    """Per-token scale alpha_t = mean_c |fp32(k_c) - mu_c| (READING: the summary gives
    no scale; 1 bit per dimension plus one per-token scale, with the mean absolute
    deviation, the least-squares optimum for a fixed sign vector).

    Sum: ``tree_sum_f32`` over the 128 channels of |fl32(k_c - mu_c)|; then an
    exact multiplication by 2^-7.  Returns float32 [..., T]."""
    x = bf16_to_f32(k_bits)
    a = np.abs(x - np.asarray(mu, np.float32)[..., None, :]).astype(np.float32)
    return (tree_sum_f32(a, axis=-1) * np.float32(2.0 ** -7)).astype(np.float32)


def encode(k_bits, n_tokens: int, with_codebook: bool = False) -> dict:
    """Prefill compression of one cache (§2.1 items 1 and 3).

    k_bits: [B, H, >=N, 128] bf16 bits.  Returns mu [B,H,128] f32, codes
    [B,H,N,16] u8 (written for every token, sinks included, for a uniform
    layout), alpha [B,H,N] f32 and k_sink [B,H,64,128] (bf16 bits, the first 64
    rows copied unchanged: READING, sinks are the initial positions)."""
    k_bits = np.asarray(k_bits)
    mu = channel_mean(k_bits, n_tokens)
    rows = k_bits[..., :n_tokens, :]
    out = {
        "mu": mu,
        "codes": pack_codes(sign_bits(rows, mu)),
        "alpha": token_scale(rows, mu),
        "k_sink": np.array(k_bits[..., :N_SINK, :], dtype=np.uint16),
    }
    if with_codebook:   # optional data-derived centres (``codebook``), per (b, h)
        lead = k_bits.shape[:-2]
        cb = np.zeros(lead + (N_SUB, N_PATTERNS, SUB_DIM), np.float32)
        for ix in np.ndindex(*lead):
            cb[ix] = codebook(k_bits[ix], mu[ix], out["codes"][ix], out["alpha"][ix], n_tokens)
        out["codebook"] = cb
    return out


def encode_rows(k_bits, mu) -> dict:
    """Codes and scales of rows appended after prefill, with the channel mean
    frozen (READING: the mean is computed once at prefill)."""
    return {"codes": pack_codes(sign_bits(k_bits, mu)), "alpha": token_scale(k_bits, mu)}


def dequantize(codes, alpha, mu, cb=None) -> np.ndarray:
    """Reconstructed key k^_c = fl32(mu_c + alpha * v_c) (§2.1 item 1: the code
    doubles as the quantised key), with v the centre of the token's cluster in
    sub-vector j = c // 4: the sign vertex (v_c = +1 for bit 0, -1 for bit 1)
    or, given a codebook ``cb`` [32,16,4], component c % 4 of cb[j, nibble_j].
    mu + alpha*v is formed in fp64 and rounded once (for sign vertices alpha*v
    is exact and this is the fp32 sum).  Returns float32 [..., T, 128]."""
    a = np.asarray(alpha, np.float64)[..., :, None]
    if cb is None:
        bits = np.unpackbits(np.asarray(codes, np.uint8), axis=-1, bitorder="little")
        v = 1.0 - 2.0 * bits.astype(np.float64)
    else:
        nib = code_nibbles(codes).astype(np.intp)                       # [..., T, 32]
        v = np.asarray(cb, np.float64)[np.arange(N_SUB), nib].reshape(nib.shape[:-1] + (HEAD_DIM,))
    return (np.asarray(mu, np.float64)[..., None, :] + a * v).astype(np.float32)


CB_FRAC_BITS = 24   # fixed-point fraction bits of the codebook accumulators


def codebook(k_bits, mu, codes, alpha, n_tokens: int) -> np.ndarray:
    """Data-derived cluster centres of one (batch, KV head) (§2.1 item 1: the
    sign pattern of a 4-dim sub-vector assigns it to one of 16 clusters in a
    single pass, with no iterations; §2.1 item 2: the query is dotted with the
    16 centre vectors).

    READING: centre C[j, p] (4 components) = mean, over the prefill non-sink
    tokens t in [64, N) whose sub-vector j has pattern p, of the normalised
    sub-vector divided by the token's scale, x = fl32(fl32(k_c - mu_c) / alpha_t)
    (a token with alpha_t = 0 adds 0).  Each x is turned into fixed point,
    rint(x * 2^24) (int64, ties to even), so that the sums are exact and
    order-free; C = fl32((sum * 2^-24) / count) with the division in fp64.  An
    empty cluster keeps its sign vertex.  Frozen for appended tokens, like mu.

    k_bits [>=N, 128] bf16 bits; mu [128]; codes [>=N, 16]; alpha [>=N].
    Returns float32 [32, 16, 4]."""
    rows = slice(N_SINK, n_tokens)
    kt = (bf16_to_f32(np.asarray(k_bits)[rows]) - np.asarray(mu, np.float32)).astype(np.float32)
    a = np.asarray(alpha, np.float32)[rows][:, None]
    with np.errstate(divide="ignore", invalid="ignore"):
        x = np.where(a > 0, kt / np.where(a > 0, a, np.float32(1)), np.float32(0)).astype(np.float32)
    fx = np.rint(x.astype(np.float64) * 2.0 ** CB_FRAC_BITS).astype(np.int64)
    fx = fx.reshape(-1, N_SUB, SUB_DIM)                                   # [T, 32, 4]
    nib = code_nibbles(np.asarray(codes)[rows]).astype(np.intp)           # [T, 32]
    sums = np.zeros((N_SUB, N_PATTERNS, SUB_DIM), np.int64)
    cnt = np.zeros((N_SUB, N_PATTERNS), np.int64)
    for j in range(N_SUB):
        np.add.at(sums[j], nib[:, j], fx[:, j, :])
        np.add.at(cnt[j], nib[:, j], 1)
    mean = (sums.astype(np.float64) * 2.0 ** -CB_FRAC_BITS) / np.maximum(cnt, 1)[..., None]
    out = np.where(cnt[..., None] > 0, mean, centres()[None, :, :])
    return out.astype(np.float32)


def normalised_subvectors(k_bits, mu, alpha, n_tokens: int) -> np.ndarray:
    """The points the clustering works on: x = fl32(fl32(k_c - mu_c) / alpha_t) for the
    prefill non-sink tokens t in [64, N) (0 where alpha_t = 0), grouped into the 32
    4-dim sub-vectors.  Returns float32 [N - 64, 32, 4]."""
    rows = slice(N_SINK, n_tokens)
    kt = (bf16_to_f32(np.asarray(k_bits)[rows]) - np.asarray(mu, np.float32)).astype(np.float32)
    a = np.asarray(alpha, np.float32)[rows][:, None]
    with np.errstate(divide="ignore", invalid="ignore"):
        x = np.where(a > 0, kt / np.where(a > 0, a, np.float32(1)), np.float32(0)).astype(np.float32)
    return x.reshape(-1, N_SUB, SUB_DIM)


def kmeans_codebook(k_bits, mu, alpha, n_tokens: int, n_iter: int = 20) -> np.ndarray:
    """The iterative clustering the one-pass sign clustering replaces (§2.1 item 1)
    and is timed against (§4, module speed-ups: K-means with 20 iterations).

    READING (the pages name only "K-means, 20 iterations"): Lloyd iterations on the
    same points as ``codebook`` (``normalised_subvectors``), 16 clusters per
    sub-vector position j, started from the 16 sign vertices.  Each iteration assigns
    every point to its nearest centre, the squared Euclidean distance taken in fp32 in
    a fixed order, ((d0^2 + d1^2) + d2^2) + d3^2 with d_i = fl32(x_i - c_i) (each
    product and sum rounded to fp32), the lowest index winning ties; then a centre is
    the mean of its points, with the fixed-point sums and fp64 division of
    ``codebook``; an empty cluster keeps its previous centre.  Starting from the
    vertices, the nearest vertex of a point is its sign pattern, so one iteration
    gives exactly ``codebook``.

    k_bits [>=N, 128] bf16 bits; mu [128]; alpha [>=N].  Returns float32 [32, 16, 4]."""
    x = normalised_subvectors(k_bits, mu, alpha, n_tokens)               # [T, 32, 4]
    fx = np.rint(x.astype(np.float64) * 2.0 ** CB_FRAC_BITS)             # exact integers
    c = np.broadcast_to(centres().astype(np.float32), (N_SUB, N_PATTERNS, SUB_DIM)).copy()
    for _ in range(n_iter):
        d = (x[:, :, None, :] - c[None, :, :, :]).astype(np.float32)     # [T, 32, 16, 4]
        sq = (d * d).astype(np.float32)
        dist = (((sq[..., 0] + sq[..., 1]).astype(np.float32) + sq[..., 2]).astype(np.float32)
                + sq[..., 3]).astype(np.float32)                         # [T, 32, 16]
        lab = np.argmin(dist, axis=-1)                                   # first minimum
        new = c.copy()
        for j in range(N_SUB):
            cnt = np.bincount(lab[:, j], minlength=N_PATTERNS)
            for i in range(SUB_DIM):
                sm = np.bincount(lab[:, j], weights=fx[:, j, i], minlength=N_PATTERNS)
                mean = (sm * 2.0 ** -CB_FRAC_BITS) / np.maximum(cnt, 1)
                new[j, :, i] = np.where(cnt > 0, mean, c[j, :, i]).astype(np.float32)
        c = new
    return c


def kmeans_objective(k_bits, mu, alpha, n_tokens: int, cb) -> float:
    """Sum over points of the squared distance to the nearest centre (fp64)."""
    x = normalised_subvectors(k_bits, mu, alpha, n_tokens).astype(np.float64)
    d = ((x[:, :, None, :] - np.asarray(cb, np.float64)[None]) ** 2).sum(-1)
    return float(d.min(axis=-1).sum())


def dense_scores(q_bits, k_bits, n_kv_heads: int, n_tokens: int) -> np.ndarray:
    """Full dot-product retrieval, the comparator of the LUT-GEMV score (§4, module
    speed-ups: retrieval against the full dot product): the selection query of each
    KV head (``group_query``) dotted with every cached bf16 key, t < N, in fp64.
    q_bits [B,Hq,128]; k_bits [B,Hkv,>=N,128] -> fp64 [B,Hkv,N]."""
    qbar = group_query(q_bits, n_kv_heads)                               # [B, Hkv, 128]
    k = bf16_to_f32(np.asarray(k_bits)[..., :n_tokens, :]).astype(np.float64)
    return np.einsum("bhc,bhtc->bht", qbar, k)


# --------------------------------------------------------------------------- #
# Quantised values (2-bit, per token): the memory side of the method
# --------------------------------------------------------------------------- #
V_GROUP = 32          # channels per value group (one scale and one zero point each)
V_LEVELS = 3          # 2 bits: codes 0..3


def quantize_v(v_bits):
    """READING (values): the pages report the KV cache shrinking about 5x with 2-bit
    quantisation at the compression ratio of a 2-bit per-token value scheme, and keep the
    64 sink tokens in full precision (§2.1 item 3).  Read here as: every non-sink value
    row is split into 4 groups of 32 channels; per group, z = min (+0 when it is zero),
    scale s = fl32((max - z) / 3), both stored as fp16 (round to nearest even); code q_c = clamp(rint(fl32(
    fl32(v_c - z16) / s16)), 0, 3) with z16, s16 the stored values (q = 0 when s16 = 0).
    Layout: codes [..., T, 32] u8, channel c at byte c // 4, bits 2*(c % 4) and up;
    scales [..., T, 4, 2] uint16 fp16 bits, (scale, zero) per group.

    v_bits [..., T, 128] bf16 bits.  Returns (codes, sz)."""
    x = bf16_to_f32(v_bits).astype(np.float32)
    g = x.reshape(x.shape[:-1] + (HEAD_DIM // V_GROUP, V_GROUP))
    z = g.min(axis=-1)
    z = np.where(z == 0, np.float32(0), z).astype(np.float32)   # a zero minimum is +0
    s = ((g.max(axis=-1) - z) / np.float32(V_LEVELS)).astype(np.float32)
    z16, s16 = z.astype(np.float16), s.astype(np.float16)
    zf, sf = z16.astype(np.float32)[..., None], s16.astype(np.float32)[..., None]
    with np.errstate(divide="ignore", invalid="ignore"):
        r = ((g - zf).astype(np.float32) / np.where(sf > 0, sf, np.float32(1))).astype(np.float32)
    q = np.where(sf > 0, np.clip(np.rint(r), 0, V_LEVELS), 0).astype(np.uint8)
    q = q.reshape(x.shape)                                       # [..., T, 128]
    q4 = q.reshape(q.shape[:-1] + (HEAD_DIM // 4, 4))
    codes = (q4[..., 0] | (q4[..., 1] << 2) | (q4[..., 2] << 4) | (q4[..., 3] << 6)).astype(np.uint8)
    sz = np.stack([s16.view(np.uint16), z16.view(np.uint16)], axis=-1)
    return codes, sz


def dequantize_v(codes, sz) -> np.ndarray:
    """v^_c = z + q_c * s with the stored fp16 scale and zero point (exact in fp64).
    codes [..., T, 32], sz [..., T, 4, 2] -> fp64 [..., T, 128]."""
    c = np.asarray(codes, np.uint8)
    q = np.stack([(c >> (2 * i)) & 3 for i in range(4)], axis=-1).reshape(c.shape[:-1] + (HEAD_DIM,))
    s = np.asarray(sz, np.uint16)[..., 0].view(np.float16).astype(np.float64)
    z = np.asarray(sz, np.uint16)[..., 1].view(np.float16).astype(np.float64)
    grp = np.arange(HEAD_DIM) // V_GROUP
    return z[..., grp] + q.astype(np.float64) * s[..., grp]


# --------------------------------------------------------------------------- #
# Decode retrieval: §2.1 item 2 (compressed-domain top-k by LUT-GEMV)
# --------------------------------------------------------------------------- #
def centres() -> np.ndarray:
    """The 16 centre vectors of a 4-dim sub-vector (READING: the sign vertices;
    the per-token scale carries the magnitude).  Row p, element i: +1 if bit i
    of p is 0 else -1.  Shape [16, 4], fp64."""
    p = np.arange(N_PATTERNS)[:, None]
    i = np.arange(SUB_DIM)[None, :]
    return np.where((p >> i) & 1, -1.0, 1.0)


def group_query(q_bits, n_kv_heads: int) -> np.ndarray:
    """Selection query of each KV head: the sum of its query group (READING:
    grouped-query attention with contiguous groups, heads h*G..h*G+G-1, selection
    per KV head by the group's summed score).  q_bits [B,Hq,128] -> fp64 [B,Hkv,128]."""
    q = bf16_to_f32(q_bits).astype(np.float64)
    b, hq, d = q.shape
    return q.reshape(b, n_kv_heads, hq // n_kv_heads, d).sum(axis=2)


def query_lut(qbar, cb=None) -> np.ndarray:
    """§2.1 item 2: split the query like the key and dot each 4-dim piece with the
    16 centres (the sign vertices, or the codebook ``cb`` [32,16,4] of the KV
    head).  qbar [..., 128] -> LUT [..., 32, 16] fp64."""
    qs = np.asarray(qbar, np.float64).reshape(qbar.shape[:-1] + (N_SUB, SUB_DIM))
    if cb is None:
        return qs @ centres().T
    return np.einsum("...ji,jpi->...jp", qs, np.asarray(cb, np.float64))


def code_nibbles(codes) -> np.ndarray:
    """Cluster index of every sub-vector: nibble j of the code. [..., 16] -> [..., 32]."""
    c = np.asarray(codes, np.uint8)
    lo = c & 0x0F
    hi = c >> 4
    return np.stack([lo, hi], axis=-1).reshape(c.shape[:-1] + (N_SUB,))


def lut_scores(lut, codes, alpha) -> np.ndarray:
    """§2.1 item 2: score a token by looking up each sub-vector's cluster in the
    query's table and accumulating, all in the quantised domain:
    s_t = alpha_t * sum_j LUT[j, nibble_j(code_t)].  fp64.

    This is q.(k^ - mu) for the dequantised key; the term q.mu is the same for
    every token and does not change the ranking, so it is left out.
    lut [32,16]; codes [T,16]; alpha [T] -> [T]."""
    nib = code_nibbles(codes).astype(np.intp)
    acc = np.asarray(lut)[np.arange(N_SUB)[None, :], nib].sum(axis=-1)
    return np.asarray(alpha, np.float64) * acc


def select_topk(scores, k: int, first_token: int = N_SINK) -> np.ndarray:
    """Top-k tokens by score (§2.1 item 2).  scores[i] belongs to token
    first_token + i.  Order: larger score first, ties to the smaller position
    (READING); the result is returned in ascending token order."""
    s = np.asarray(scores, np.float64)
    if not 1 <= k <= s.size:
        raise ValueError("need 1 <= k <= number of candidates")
    t = np.arange(s.size)
    order = np.lexsort((t, -s))
    return np.sort(order[:k]).astype(np.int64) + first_token


# --------------------------------------------------------------------------- #
# Sparse attention over top-k plus sinks: §2.1 items 3 and 4
# --------------------------------------------------------------------------- #
def sparse_attention(q_bits_group, idx, k_sink_bits, codes, alpha, mu, v_bits,
                     sm_scale: float, cb=None, vq=None) -> np.ndarray:
    """Attention of the G query heads of one KV head over S = {0..63} U idx
    (§2.1 item 3: sinks always kept in full precision; item 4: keys dequantised
    inside the attention).  Keys: bf16 sink rows for t < 64, else k^_t (fp32,
    ``dequantize``).  Values: the bf16 V rows, unmodified (READING).  Logits
    (q_g . kappa_t) * sm_scale; softmax over S; output sum_t p_t V_t.  No mask:
    a decoding query sees every cached token.  fp64, returned as float32 [G,128].

    q_bits_group [G,128]; idx [k] (token positions >= 64); k_sink_bits [64,128];
    codes [N,16], alpha [N], mu [128], v_bits [N,128] of that KV head; cb: its
    codebook or None (sign vertices); vq: None, or its quantised values (codes [N,32],
    sz [N,4,2]) from ``quantize_v``, used for every attended t >= 64 (the sinks keep
    their bf16 rows)."""
    idx = np.asarray(idx, np.int64)
    q = bf16_to_f32(q_bits_group).astype(np.float64)
    kap = np.concatenate([bf16_to_f32(k_sink_bits).astype(np.float64),
                          dequantize(np.asarray(codes)[idx], np.asarray(alpha)[idx],
                                     mu, cb).astype(np.float64)], axis=0)
    rows = np.concatenate([np.arange(N_SINK, dtype=np.int64), idx])
    vals = bf16_to_f32(np.asarray(v_bits)[rows]).astype(np.float64)
    if vq is not None:
        vals[N_SINK:] = dequantize_v(np.asarray(vq[0])[idx], np.asarray(vq[1])[idx])
    logits = (kap @ q.T) * float(sm_scale)                      # [|S|, G]
    logits -= logits.max(axis=0, keepdims=True)
    p = np.exp(logits)
    p /= p.sum(axis=0, keepdims=True)
    return (p.T @ vals).astype(np.float32)


def head_scores(q_bits, codes, alpha, b: int, h: int, n_kv_heads: int,
                n_tokens: int, cb=None) -> np.ndarray:
    """Selection scores of the candidates t in [64, N) of one (batch, KV head)
    (cb: that head's codebook, or None for the sign vertices)."""
    qbar = group_query(q_bits[b:b + 1], n_kv_heads)[0, h]
    return lut_scores(query_lut(qbar, cb), codes[N_SINK:n_tokens], alpha[N_SINK:n_tokens])


def decode_step(q_bits, cache: dict, v_bits, top_k: int, sm_scale: float,
                n_tokens: int, heads=None, vq=None) -> dict:
    """One decode step: LUT scores -> top-k -> sparse attention, per (b, KV head).

    cache: ``encode`` output (codes/alpha indexed by token; the codebook is used
    when present).  v_bits [B,H,>=N,128].
    heads: optional list of (b, h) pairs to compute (others left zero / -1).
    vq: optional quantised values (codes [B,H,N,32], sz [B,H,N,4,2]).
    Returns idx [B,H,k] int64 and out [B,Hq,128] float32."""
    q_bits = np.asarray(q_bits)
    b_n, hq, _ = q_bits.shape
    n_kv = cache["mu"].shape[1]
    g = hq // n_kv
    idx = np.full((b_n, n_kv, top_k), -1, np.int64)
    out = np.zeros((b_n, hq, HEAD_DIM), np.float32)
    pairs = heads if heads is not None else [(b, h) for b in range(b_n) for h in range(n_kv)]
    cbs = cache.get("codebook")
    for b, h in pairs:
        cb = None if cbs is None else cbs[b, h]
        s = head_scores(q_bits, cache["codes"][b, h], cache["alpha"][b, h], b, h, n_kv, n_tokens,
                        cb)
        sel = select_topk(s, top_k)
        idx[b, h] = sel
        out[b, h * g:(h + 1) * g] = sparse_attention(
            q_bits[b, h * g:(h + 1) * g], sel, cache["k_sink"][b, h], cache["codes"][b, h],
            cache["alpha"][b, h], cache["mu"][b, h], v_bits[b, h], sm_scale, cb,
            None if vq is None else (vq[0][b, h], vq[1][b, h]))
    return {"idx": idx, "out": out}
