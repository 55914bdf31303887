// Internal declarations of the gfx950 kernels and their host launchers.
//
// Method: "Self-Indexing KVCache: Predicting Sparse Attention from Compressed
// Keys" (web summary, technical part, §2.1 items 1-4).  Every kernel is written
// for wave64 CDNA4: one lane per token where a token is processed whole (score,
// attention logits), 16 lanes x 16 bytes per 256-byte row where a row is
// streamed (encode, value gathers).
#pragma once

#include <hip/hip_fp16.h>
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

struct sikv_timer;  // the C ABI's opaque, caller-owned kernel timer

namespace sikv {

// Where the kernels of one library call go: the caller's stream, and the
// caller's timer (null: the call is not timed).  Nothing else is shared
// between calls.
struct Launch {
  hipStream_t stream;
  ::sikv_timer* timer;
};

constexpr int kD = 128;          // head dim
constexpr int kSink = 64;        // full-precision sink tokens (§2.1 item 3)
constexpr int kCodeBytes = 16;   // 1 bit per channel
// Quantised values: one 64-byte record per token row: its 2-bit value codes
// (32 B), the (scale, zero) fp16 words of its 4 channel groups (16 B) and a
// copy of its 16-byte key code, so that the attention fetches one record (plus
// the scale) per attended token instead of four scattered pieces.
constexpr int kVRecBytes = 64;
constexpr int kVRecSz = 32;    // offset of the 4 (scale, zero) words
constexpr int kVRecCode = 48;  // offset of the key code copy
constexpr int kSub = 32;         // 4-dim sub-vectors per key (§2.1 item 1)
constexpr int kLut = kSub * 16;  // table entries per query
constexpr int kMaxGroup = 8;

// Kernel ids of the optional caller-owned timer.
enum KernelId {
  KID_MU_PARTIAL = 0,
  KID_MU_FINAL,
  KID_CODES,
  KID_TABLES,
  KID_SCORE,
  KID_SELECT,
  KID_ATTN,
  KID_COMBINE,
  KID_DENSE,
  KID_COPY,
  KID_CB_FINAL,
  KID_VCODES,
  KID_KM_ASSIGN,
  KID_DSCORES,
  KID_COUNT
};

// ---------------------------------------------------------------- device helpers
__device__ __forceinline__ float bf16lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Channel c (0..7) of 8 bf16 values packed in a uint4.
__device__ __forceinline__ float chan(const uint4& w, int c) {
  const uint32_t x = (c >> 1) == 0 ? w.x : (c >> 1) == 1 ? w.y : (c >> 1) == 2 ? w.z : w.w;
  return (c & 1) ? bf16hi(x) : bf16lo(x);
}

// Sign code and scale of one key row held by 16 consecutive lanes (lane cg of
// the group: channels 8cg..8cg+7 in w, their means in m).  Bit c = (k_c < mu_c)
// (§2.1 item 1, entropy-aware normalisation then sign); scale = adjacent-pair
// fp32 tree of |fl(k_c - mu_c)| over the 128 channels, times 2^-7: each lane's 8
// channels are an aligned subtree and the xor butterfly over lanes 1, 2, 4, 8
// forms the top levels, so every lane ends with the same bits.  Returns, in lane
// cg with cg % 4 == 0, the code bytes of channels 8cg..8cg+31 as one word.
struct RowCode {
  uint32_t word;
  float alpha;
  uint32_t byte;  // this lane's code byte (channels 8cg..8cg+7)
};
__device__ __forceinline__ RowCode encode_row16(const uint4& w, const float (&m)[8]) {
  uint32_t byte = 0;
  float a[8];
#pragma unroll
  for (int c = 0; c < 8; ++c) {
    const float x = chan(w, c);
    byte |= (x < m[c] ? 1u : 0u) << c;
    a[c] = fabsf(x - m[c]);
  }
  float s = ((a[0] + a[1]) + (a[2] + a[3])) + ((a[4] + a[5]) + (a[6] + a[7]));
  s += __shfl_xor(s, 1);
  s += __shfl_xor(s, 2);
  s += __shfl_xor(s, 4);
  s += __shfl_xor(s, 8);
  const uint32_t v16 = byte | (__shfl_down(byte, 1, 16) << 8);
  const uint32_t v32 = v16 | (__shfl_down(v16, 2, 16) << 16);
  return RowCode{v32, s * 0.0078125f, byte};
}

// 2-bit values, per group of 32 channels of a bf16 value row: zero point
// z = min, scale s = fl32((max - z) / 3), both rounded to fp16; code
// q_c = clamp(rint(fl32(fl32(v_c - z16) / s16)), 0, 3) (0 unless s16 is positive
// and finite).
//
// The code is found without dividing: with d = fl32(v_c - z16) and s = s16 > 0,
// rint (ties to even) gives q >= 1 iff r = fl32(d / s) > 1/2, q >= 2 iff r >= 3/2
// and q >= 3 iff r > 5/2.  r reaches a float F iff d / s passes the midpoint
// between F and the float below it (at the midpoint itself, iff F is even), so
// the three conditions are d / s > 1/2 + 2^-25, d / s >= 3/2 - 2^-24 and
// d / s > 5/2 + 2^-23.  Each midpoint times s is exact in fp64 (25 by 11
// significant bits); the smallest float that satisfies the condition is the
// group's threshold, and q is the number of thresholds d reaches.  A NaN d
// reaches none, as a NaN quotient clamps to 0; s16 = 0, inf or NaN makes every
// threshold NaN.
__device__ __forceinline__ float vq_next_up(float t) {  // t positive and finite
  return __uint_as_float(__float_as_uint(t) + 1u);
}
__device__ __forceinline__ float vq_least_ge(double p) {  // smallest float >= p > 0
  const float t = (float)p;
  return (double)t < p ? vq_next_up(t) : t;
}
__device__ __forceinline__ float vq_least_gt(double p) {  // smallest float > p > 0
  const float t = (float)p;
  return (double)t <= p ? vq_next_up(t) : t;
}
struct VqRule {
  float zf, t1, t2, t3;
  uint32_t sz;  // the (scale, zero) fp16 bits as one word
};
__device__ __forceinline__ VqRule vq_rule(float lo, float hi) {
  lo = lo == 0.0f ? 0.0f : lo;  // a zero minimum is stored as +0
  const __half z16 = __float2half_rn(lo);
  const __half s16 = __float2half_rn(__fdiv_rn(hi - lo, 3.0f));
  const float sf = __half2float(s16);
  const double s64 = (double)sf;
  const bool ok = sf > 0.0f && sf < INFINITY;
  VqRule r;
  r.zf = __half2float(z16);
  r.t1 = ok ? vq_least_gt((0.5 + 0x1p-25) * s64) : __builtin_nanf("");
  r.t2 = ok ? vq_least_ge((1.5 - 0x1p-24) * s64) : __builtin_nanf("");
  r.t3 = ok ? vq_least_gt((2.5 + 0x1p-23) * s64) : __builtin_nanf("");
  r.sz = (uint32_t)__half_as_ushort(s16) | ((uint32_t)__half_as_ushort(z16) << 16);
  return r;
}
__device__ __forceinline__ uint32_t vq_code(const VqRule& r, float x) {
  const float d = x - r.zf;
  return (uint32_t)(d >= r.t1) + (uint32_t)(d >= r.t2) + (uint32_t)(d >= r.t3);
}

// One value row held by 16 consecutive lanes (lane cg: channels 8cg..8cg+7 in
// w; a group = 4 lanes): the lane's 16 code bits (channel 8cg+i at bits 2i) and
// its group's (scale, zero) word.
struct VRowCode {
  uint32_t bits;
  uint32_t sz;
};
__device__ __forceinline__ VRowCode quantize_vrow16(const uint4& w) {
  float x[8];
  float lo = 0.0f, hi = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    x[i] = chan(w, i);
    lo = i == 0 ? x[i] : fminf(lo, x[i]);
    hi = i == 0 ? x[i] : fmaxf(hi, x[i]);
  }
  lo = fminf(lo, __shfl_xor(lo, 1));
  hi = fmaxf(hi, __shfl_xor(hi, 1));
  lo = fminf(lo, __shfl_xor(lo, 2));
  hi = fmaxf(hi, __shfl_xor(hi, 2));
  const VqRule r = vq_rule(lo, hi);
  uint32_t bits = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) bits |= vq_code(r, x[i]) << (2 * i);
  return VRowCode{bits, r.sz};
}

// One whole group held by one lane (w[u]: channels 8u..8u+7 of the group): its
// 64 code bits (channel j at bits 2j of lo / hi for j < 16 / j >= 16) and its
// (scale, zero) word.
struct VGroupCode {
  uint32_t lo, hi, sz;
};
__device__ __forceinline__ VGroupCode quantize_vgroup32(const uint4 (&w)[4]) {
  float x[32];
#pragma unroll
  for (int u = 0; u < 4; ++u)
#pragma unroll
    for (int i = 0; i < 8; ++i) x[8 * u + i] = chan(w[u], i);
  float lo = x[0], hi = x[0];
#pragma unroll
  for (int j = 1; j < 32; ++j) {
    lo = fminf(lo, x[j]);
    hi = fmaxf(hi, x[j]);
  }
  const VqRule r = vq_rule(lo, hi);
  VGroupCode c{0u, 0u, r.sz};
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    c.lo |= vq_code(r, x[j]) << (2 * j);
    c.hi |= vq_code(r, x[16 + j]) << (2 * j);
  }
  return c;
}

// Where token t of (batch b, KV head h) lives in the per-token arrays (codes,
// alpha, value records and, paged, the bf16 V pool).  Contiguous: row
// (b * Hkv + h) * capacity + t.  Paged: the sequence's page table entry for t
// names a pool page of 2^lg_page tokens holding all KV heads: row
// (page * Hkv + h) * 2^lg_page + t mod 2^lg_page.
struct RowMap {
  int64_t capacity;
  const int32_t* table;  // null: contiguous; else [B][pps] page ids
  int lg_page;
  int pps;
  int Hkv;
  __device__ __forceinline__ int64_t row(int b, int h, int t) const {
    if (table == nullptr) return ((int64_t)b * Hkv + h) * capacity + t;
    const int64_t pg = table[(int64_t)b * pps + (t >> lg_page)];
    return ((pg * Hkv + h) << lg_page) | (int64_t)(t & ((1 << lg_page) - 1));
  }
};

// Ragged batches: the length of sequence b is seq_lens[b] clamped into
// [65, n_max] (n_max, the descriptor's n_tokens, when seq_lens is null), and it
// selects min(k, length - 64) tokens.
__device__ __forceinline__ int seq_len(const int32_t* seq_lens, int b, int n_max) {
  return seq_lens != nullptr ? min(max(seq_lens[b], kSink + 1), n_max) : n_max;
}
__host__ __device__ __forceinline__ int seq_topk(int k, int n) {
  return k < n - kSink ? k : n - kSink;
}

// Order-preserving map of fp32 (no NaN) to uint32.
__device__ __forceinline__ uint32_t score_key(float s) {
  uint32_t u = __float_as_uint(s);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float key_score(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7fffffffu) : ~k);
}

// Look-up table of one query vector x (LDS, 128 floats): lut[j*16 + p] =
// ((+-x0 +- x1) +- x2) +- x3 with x_i = x[4j+i], negative iff bit i of p is set
// (§2.1 item 2: a query piece dotted with the 16 sign vertices).  No barrier.
__device__ __forceinline__ float sign_entry(float x0, float x1, float x2, float x3, int p) {
  float v = (p & 1) ? -x0 : x0;
  v += (p & 2) ? -x1 : x1;
  v += (p & 4) ? -x2 : x2;
  v += (p & 8) ? -x3 : x3;
  return v;
}
__device__ __forceinline__ float lut_entry(const float* x, int e) {
  const int j = e >> 4;
  return sign_entry(x[4 * j], x[4 * j + 1], x[4 * j + 2], x[4 * j + 3], e & 15);
}

// Table entry with data-derived centres: lut[j*16 + p] = x(4j..4j+3) . cb[j*16 + p]
// (cb: the KV head's codebook, 16 centres of 4 components per sub-vector).
__device__ __forceinline__ float cb_lut_entry(const float* x, const float4* cb, int e) {
  const int j = e >> 4;
  const float4 c = cb[e];
  return ((x[4 * j] * c.x + x[4 * j + 1] * c.y) + x[4 * j + 2] * c.z) + x[4 * j + 3] * c.w;
}

// Byte k of x, zero-extended, as one v_perm_b32 (selector byte 0x0c yields 0x00).
__device__ __forceinline__ uint32_t byte_of(uint32_t x, uint32_t k) {
  return __builtin_amdgcn_perm(0u, x, 0x0c0c0c00u | k);
}

// Sum over the 8 sub-vectors of one code word with a nibble table (sub-vectors
// 8w..8w+7, table slice of sub-vector j at byte 64*j).  The nibbles are moved to
// byte lanes already multiplied by 4 (even nibbles from d << 2, odd ones from
// d >> 2), so each look-up needs a single byte extract for its LDS address.
__device__ __forceinline__ float lut_word(const float* __restrict__ lutw, uint32_t d) {
  const uint32_t e = (d << 2) & 0x3c3c3c3cu;
  const uint32_t o = (d >> 2) & 0x3c3c3c3cu;
  const char* L = reinterpret_cast<const char*>(lutw);
  float a = *reinterpret_cast<const float*>(L + 0 * 64 + byte_of(e, 0));
  float c = *reinterpret_cast<const float*>(L + 1 * 64 + byte_of(o, 0));
  a += *reinterpret_cast<const float*>(L + 2 * 64 + byte_of(e, 1));
  c += *reinterpret_cast<const float*>(L + 3 * 64 + byte_of(o, 1));
  a += *reinterpret_cast<const float*>(L + 4 * 64 + byte_of(e, 2));
  c += *reinterpret_cast<const float*>(L + 5 * 64 + byte_of(o, 2));
  a += *reinterpret_cast<const float*>(L + 6 * 64 + byte_of(e, 3));
  c += *reinterpret_cast<const float*>(L + 7 * 64 + byte_of(o, 3));
  return a + c;
}

// q . sigma(code) with a per-query-head nibble table: (w0 + w1) + (w2 + w3).
__device__ __forceinline__ float lut_dot(const float* __restrict__ lut, uint4 c) {
  return (lut_word(lut, c.x) + lut_word(lut + 128, c.y)) +
         (lut_word(lut + 256, c.z) + lut_word(lut + 384, c.w));
}

// Selection table in int32 fixed point: itab[j*16 + p] = rint(lut[j*16 + p] * 2^e)
// with 2^e chosen per KV head so that sum_c |qbar_c| * 2^e < 2^30.  Integer sums
// are exact and order-free, and v_add3 adds two terms per instruction; the
// rounding of the 32 terms costs at most 16 * 2^-e <= 2^-26 * sum_c |qbar_c|.
__device__ __forceinline__ int ilut_word(const int* __restrict__ lutw, uint32_t d) {
  const uint32_t e = (d << 2) & 0x3c3c3c3cu;
  const uint32_t o = (d >> 2) & 0x3c3c3c3cu;
  const char* L = reinterpret_cast<const char*>(lutw);
  const int a0 = *reinterpret_cast<const int*>(L + 0 * 64 + byte_of(e, 0));
  const int a1 = *reinterpret_cast<const int*>(L + 1 * 64 + byte_of(o, 0));
  const int a2 = *reinterpret_cast<const int*>(L + 2 * 64 + byte_of(e, 1));
  const int a3 = *reinterpret_cast<const int*>(L + 3 * 64 + byte_of(o, 1));
  const int a4 = *reinterpret_cast<const int*>(L + 4 * 64 + byte_of(e, 2));
  const int a5 = *reinterpret_cast<const int*>(L + 5 * 64 + byte_of(o, 2));
  const int a6 = *reinterpret_cast<const int*>(L + 6 * 64 + byte_of(e, 3));
  const int a7 = *reinterpret_cast<const int*>(L + 7 * 64 + byte_of(o, 3));
  return (a0 + a1 + a2) + (a3 + a4 + a5) + (a6 + a7);
}

__device__ __forceinline__ int ilut_dot(const int* __restrict__ itab, uint4 c) {
  return ilut_word(itab, c.x) + ilut_word(itab + 128, c.y) + ilut_word(itab + 256, c.z) +
         ilut_word(itab + 384, c.w);
}

// Selection score of one token, as used by every kernel that ranks tokens
// (same table, exact integer sum, then alpha * (sum * 2^-e)); -0 is mapped to
// +0 so that equal scores have equal keys.
__device__ __forceinline__ float selection_score(const int* __restrict__ itab, float inv_scale,
                                                 uint4 c, float a) {
  return a * ((float)ilut_dot(itab, c) * inv_scale) + 0.0f;
}

// ---------------------------------------------------------------- cross-lane (DPP)
// Moves within 16-lane rows (data-parallel primitives) and lane reads: plain
// VALU work, where __shfl_* goes through the LDS crossbar (ds_bpermute) with
// its latency on every step of a reduction or scan.
enum : int {
  kDppRowShr1 = 0x111, kDppRowShr2 = 0x112, kDppRowShr4 = 0x114, kDppRowShr8 = 0x118,
  kDppRowRor1 = 0x121, kDppRowRor2 = 0x122, kDppRowRor4 = 0x124, kDppRowRor8 = 0x128,
  kDppRowBcast15 = 0x142, kDppRowBcast31 = 0x143,
};
// x moved by kCtrl; lanes whose source is outside the row, or whose row is not
// in kRowMask, read 0.
template <int kCtrl, int kRowMask = 0xf>
__device__ __forceinline__ int dpp(int x) {
  return __builtin_amdgcn_update_dpp(0, x, kCtrl, kRowMask, 0xf, true);
}
template <int kCtrl>
__device__ __forceinline__ float dpp(float x) {
  return __int_as_float(dpp<kCtrl>(__float_as_int(x)));
}
__device__ __forceinline__ float readlane(float x, int l) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), l));
}

// Inclusive prefix sum over the 64 lanes (row scans, then rows 0-1 carried
// into rows 1 and 3, then rows 0-1 into rows 2-3).
__device__ __forceinline__ int wave_incl_scan(int x) {
  x += dpp<kDppRowShr1>(x);
  x += dpp<kDppRowShr2>(x);
  x += dpp<kDppRowShr4>(x);
  x += dpp<kDppRowShr8>(x);
  x += dpp<kDppRowBcast15, 0xa>(x);
  x += dpp<kDppRowBcast31, 0xc>(x);
  return x;
}

// op over each 16-lane row, the result in every lane of the row.
template <class T, class Op>
__device__ __forceinline__ T row_allreduce(T x, Op op) {
  x = op(x, dpp<kDppRowRor8>(x));
  x = op(x, dpp<kDppRowRor4>(x));
  x = op(x, dpp<kDppRowRor2>(x));
  x = op(x, dpp<kDppRowRor1>(x));
  return x;
}

// Sum over the 64 lanes, the same value in every lane.  Call it in wave-uniform
// control flow and branch only on its result: lane reads inside a branch would
// let the compiler move the reduction's last step into the branch, where the
// lanes read no longer execute it.
__device__ __forceinline__ float wave_sum(float x) {
  const float v = row_allreduce(x, [](float a, float b) { return a + b; });
  return (readlane(v, 0) + readlane(v, 16)) + (readlane(v, 32) + readlane(v, 48));
}

// Number of set bits of a 64-lane ballot below this lane.
__device__ __forceinline__ int ballot_rank(uint64_t m) {
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32),
                                   __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
}

// ---------------------------------------------------------------- host launchers
// encode.hip
constexpr int kMuTile = 4096;  // tokens per mean partial (an aligned subtree of the token tree)
hipError_t launch_mu_partial(const uint16_t* k, int64_t sb, int64_t sh, int64_t st, int B, int Hkv,
                             int n_tokens, float* partial, int nblk, const Launch& s);
hipError_t launch_mu_final(const float* partial, int BH, int nblk, int n_tokens, float* mu,
                           const Launch& s);
// vrec (may be null): value records, whose key code copy is written too.
hipError_t launch_codes(const uint16_t* k, int64_t sb, int64_t sh, int64_t st, int B, int Hkv,
                        int t_begin, int t_end, const RowMap& rm, const float* mu, uint8_t* codes,
                        float* alpha, uint16_t* k_sink, uint8_t* vrec, const Launch& s);
// 2-bit value codes of rows t_begin..t_end-1 (quantize_vgroup32) into bytes 0..47 of
// their records vrec [B*Hkv][cap][64]; rows below 64 are also copied to v_sink.
hipError_t launch_vcodes(const uint16_t* v, int64_t sb, int64_t sh, int64_t st, int B, int Hkv,
                         int t_begin, int t_end, const RowMap& rm, uint8_t* vrec,
                         uint16_t* v_sink, const Launch& s);
// Prefill codes with the codebook statistics: like launch_codes over [0, n_tokens),
// plus, per block of kCbTiles x 128 tokens, the fixed-point sums of k~/alpha and
// the counts of every (sub-vector, pattern) over the tokens [64, n_tokens),
// written to cb_part [B*Hkv][nblk][kCbStride] (nblk = cb_blocks(n_tokens)).
constexpr int kCbTiles = 32;
constexpr int kCbStride = kSub * 16 * 4 + kSub * 16;  // sums (int64) then counts
constexpr int kCbFracBits = 24;
inline int cb_blocks(int n_tokens) { return (n_tokens + 128 * kCbTiles - 1) / (128 * kCbTiles); }
hipError_t launch_codes_cb(const uint16_t* k, int64_t sb, int64_t sh, int64_t st, int B, int Hkv,
                           int n_tokens, const RowMap& rm, const float* mu, uint8_t* codes,
                           float* alpha, uint16_t* k_sink, uint8_t* vrec, long long* cb_part,
                           const Launch& s);
// Codebook from the block statistics: centre = fl32((sum * 2^-24) / count) in
// fp64; an empty cluster gets the sign vertex (keep = 0) or keeps the centre
// already in codebook (keep = 1).  codebook [B*Hkv][32][16][4].
hipError_t launch_cb_final(const long long* cb_part, int BH, int nblk, float* codebook,
                           const Launch& s, int keep = 0);
// One Lloyd step of the K-means baseline, stage 1: every prefill point x
// (tokens [64, n_tokens), x = fl32(fl32(k - mu) / alpha)) goes to its nearest
// centre of `centres` [B*Hkv][32][16][4] (null: the sign vertices), squared
// distance in fp32 ((d0^2 + d1^2) + d2^2) + d3^2, lowest index on ties; block
// statistics as launch_codes_cb (then launch_cb_final with keep = 1).
hipError_t launch_kmeans_assign(const uint16_t* k, int64_t sb, int64_t sh, int64_t st, int B,
                                int Hkv, int n_tokens, const RowMap& rm, const float* mu,
                                const float* alpha, const float* centres, long long* cb_part,
                                const Launch& s);

// score.hip
// The retrieval of one decode step (§2.1 item 2), per (b, KV head): one score
// kernel launch whose first n_heads blocks are the heads' leaders (selection
// table, sampled threshold) and whose other blocks score 256*U-token tiles
// (U = chunk / 256) and keep the tokens at or above the threshold; then the
// select kernel (exact top-k, ascending positions), whose second n_heads
// blocks make the attention tables (ta: q, mu, k_sink, codebook, att_*).
// seq_lens (may be null): per-sequence lengths of a ragged batch (seq_len /
// seq_topk above); n_tokens is then the longest, which sizes grids.  mode 1:
// sampled threshold; 2: a threshold that forces the select kernel's exact
// whole-head path.  codebook (may be null): the KV heads' centres
// [B*Hkv][32][16][4] (else the sign vertices).  k_new (may be null): bf16 key of
// each sequence's last token (element (b,h,c) at k_new[b*ksb + h*ksh + c]),
// encoded into codes / alpha by the score kernel with the frozen mean
// (bit-identical to launch_codes) and left out of the sample; v_new (may be
// null): that token's bf16 value row, quantised into its value record.  The
// attention tables: att_lut [B*Hq][512], att_qmu [B*Hq] (q_g . mu), att_slog
// [B*Hq][64] (exact sink logits q_g . k_sink[r]).
// Everything the score kernel's two kinds of blocks read and write (the
// kernel takes it by value).
struct ScoreArgs {
  int n_heads;  // B * Hkv: the score kernel's first n_heads blocks are the leaders
  // cache
  uint8_t* codes;
  float* alpha;
  RowMap rm;
  int n_tokens, Hkv;
  const int32_t* seq_lens;
  const float* mu;
  const uint16_t* k_sink;
  const float* codebook;  // [B*Hkv][32][16][4] or null (sign vertices)
  uint8_t* vrec;          // value records or null
  // query and selection
  const uint16_t* q;
  int n_q_heads, G, top_k, mode;
  // appended token (k_new null: none)
  const uint16_t* k_new;
  int64_t ksb, ksh;
  const uint16_t* v_new;
  int64_t vnsb, vnsh;
  // workspace
  unsigned long long* tau_word;  // [B*Hkv]: published threshold (tag << 32 | tau bits)
  float* bin_scale;              // [2][B*Hkv]: the select kernel's bin scale, then tau (untagged)
  int* sel_lut;                  // [B*Hkv][512]
  float* sel_inv;                // [B*Hkv]
  float* att_lut;                // [B*Hq][512]
  float* att_qmu;                // [B*Hq]
  float* att_slog;               // [B*Hq][64]
  uint32_t* app_key;             // [B*Hkv]: an appended token's selection key
  int n_chunks;
  uint32_t* cand_key;
  int32_t* cand_t;
  int2* chunk_count;             // [B*Hkv][n_chunks]: (candidates, tau bits the tile used)
  float* scores_opt;
};

hipError_t launch_score(const ScoreArgs& a, int chunk, const Launch& s);
// The attention tables alone, one block per head (mode, k_new and the
// selection outputs unused).
hipError_t launch_tables(const ScoreArgs& a, const Launch& s);
hipError_t launch_select(int B, int Hkv, const uint8_t* codes, const float* alpha, const RowMap& rm,
                         int n_tokens, const int32_t* seq_lens, const int* sel_lut,
                         const float* sel_inv, int top_k, int chunk, int n_chunks,
                         uint32_t* cand_key, int32_t* cand_t, const int2* chunk_count,
                         unsigned long long* tau_word, const float* bin_scale,
                         const uint32_t* app_key, uint32_t* comp_key, int32_t* comp_t,
                         int32_t* idx, const ScoreArgs& ta, const Launch& s);

// attn.hip
// Attended entries are processed in chunks of kAttnChunk; a block takes
// chunks_per_block consecutive chunks of one (b, KV head) and writes one
// (max, sum, o) partial per query head.
constexpr int kAttnChunk = 32;
constexpr int kAttnMaxCpb = 64;  // chunks per block at most (the block's positions sit in LDS)
// vrec (may be null): quantised values (records as launch_vcodes, key code copy
// included; vsink [B*Hkv][64][128] bf16) replace the bf16 V rows and the codes.
hipError_t launch_attn(int n_q_heads, int B, int Hkv, const uint8_t* codes, const float* alpha,
                       const uint16_t* v, int64_t vsb, int64_t vsh, int64_t vst,
                       const uint8_t* vrec, const uint16_t* vsink, const RowMap& rm,
                       int64_t n_rows, int n_tokens, const int32_t* seq_lens,
                       const int32_t* idx, int top_k, const float* att_lut,
                       const float* att_qmu, const float* att_slog, float sm_scale,
                       int chunks_per_block, int n_splits, float* part_o, float* part_ml,
                       const Launch& s);
hipError_t launch_combine(const float* part_o, const float* part_ml, int BHq, int n_splits,
                          float* out, const Launch& s);

// dense.hip
// Full dot-product retrieval scores: scores[bh * n_tokens + t] = qbar . k_t for
// t < n_tokens, qbar = sum of the G query rows of the KV head (fp32, g order).
hipError_t launch_dense_scores(const uint16_t* q, int n_q_heads, int B, int Hkv, int n_tokens,
                               const uint16_t* k, int64_t ksb, int64_t ksh, int64_t kst,
                               float* scores, const Launch& s);
hipError_t launch_dense(const uint16_t* q, int n_q_heads, int B, int Hkv, int n_tokens,
                        const uint16_t* k, int64_t ksb, int64_t ksh, int64_t kst,
                        const uint16_t* v, int64_t vsb, int64_t vsh, int64_t vst, float sm_scale,
                        int split, int n_splits, float* part_o, float* part_ml, const Launch& s);

// util.hip
hipError_t launch_copy(void* dst, const void* src, size_t bytes, const Launch& s);

// Caller-owned kernel timer (api.cpp; the C ABI's sikv_timer): launch_k asks it
// for a pair of events to bracket a launch with.  Returns null events when the
// timer is null (an untimed call).
void timing_events(::sikv_timer* timer, int kernel_id, hipEvent_t* start, hipEvent_t* stop);

// Helper used by the launchers: launch on the context's stream, bracketed by the
// timer's events when the call is timed.
template <typename... KArgs, typename... Args>
inline hipError_t launch_k(int kid, void (*kern)(KArgs...), dim3 grid, dim3 block, size_t shmem,
                           const Launch& s, Args... args) {
  hipEvent_t e0 = nullptr, e1 = nullptr;
  if (s.timer != nullptr) timing_events(s.timer, kid, &e0, &e1);
  if (e0) {
    hipExtLaunchKernelGGL(kern, grid, block, shmem, s.stream, e0, e1, 0, args...);
  } else {
    hipLaunchKernelGGL(kern, grid, block, shmem, s.stream, args...);
  }
  return hipGetLastError();
}

}  // namespace sikv
