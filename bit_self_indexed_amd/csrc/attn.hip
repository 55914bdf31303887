// Fused dequantise + sparse attention over sinks and top-k (gfx950).
//
// "Self-Indexing KVCache: Predicting Sparse Attention from Compressed Keys",
// technical summary §2.1 item 3 (64 full-precision sink tokens always kept) and
// item 4 (dequantisation fused with sparse attention in one pass).
//
// One block per (split of the attended list, b*h); the block serves the G query
// heads of the KV head, so every gathered code and V row is read once per KV
// head.  Three phases over the split's <= 256 entries:
//   A  one lane per token: logits.  Sinks: exact dot with the bf16 key row.
//      Compressed tokens: q.k^ = q.mu + alpha * sum_j LUT_g[j][nibble_j] with a
//      per-query-head table in LDS (the key is never materialised; the rounding
//      of mu + alpha*v to fp32 is a relative 2^-24 effect, far inside the fp32
//      accumulation error).
//   B  per head: max, exp2, sum over the split (logits pre-scaled by log2 e).
//   C  16 lanes x 16 bytes per gathered V row, fp32 FMAs, 4 rows in flight per
//      lane group; cross-group reduction by shuffles and LDS.
// The combine kernel merges the splits' (max, sum, o) partials.
#include <hip/hip_ext.h>

#include "sikv_internal.h"

namespace sikv {

namespace {

constexpr int kSplitMax = 256;

template <int G>
__global__ __launch_bounds__(256) void attn_kernel(
    const uint16_t* __restrict__ q, int n_q_heads, int Hkv, const uint8_t* __restrict__ codes,
    const float* __restrict__ alpha, const float* __restrict__ mu,
    const uint16_t* __restrict__ k_sink, const uint16_t* __restrict__ v, int64_t vsb, int64_t vsh,
    int64_t vst, int capacity, int n_tokens, const int32_t* __restrict__ idx, int top_k,
    float sm_log2,
    int split, int n_splits, float* __restrict__ part_o, float* __restrict__ part_ml) {
  __shared__ float qf[G][kD];
  __shared__ float lutq[G][kLut];
  __shared__ float mus[kD];
  __shared__ float qmu[G];
  __shared__ int tok[kSplitMax];
  __shared__ float pl[G][kSplitMax];
  __shared__ float red[4][G][kD];
  __shared__ float wm[G], wl[G];

  const int bh = blockIdx.y, b = bh / Hkv, h = bh - b * Hkv;
  const int s = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int L = kSink + top_k;
  const int e0 = s * split;
  const int ne = min(L, e0 + split) - e0;
  const int64_t row0 = (int64_t)bh * capacity;

  // Token of this lane and its code/scale loads, issued before the table build.
  int t = -1;
  if (tid < ne) {
    const int e = e0 + tid;
    t = e < kSink ? e : idx[(int64_t)bh * top_k + (e - kSink)];
    t = min(max(t, 0), n_tokens - 1);  // memory safety only: indices must be valid
    tok[tid] = t;
  }
  uint4 c = make_uint4(0u, 0u, 0u, 0u);
  float a = 0.0f;
  if (t >= kSink) {
    c = *reinterpret_cast<const uint4*>(codes + (row0 + t) * kCodeBytes);
    a = alpha[row0 + t];
  }
  const uint16_t* qb = q + ((int64_t)b * n_q_heads + (int64_t)h * G) * kD;
  for (int i = tid; i < G * kD; i += 256)
    qf[i / kD][i % kD] = __uint_as_float((uint32_t)qb[i] << 16);
  if (tid < kD) mus[tid] = mu[(int64_t)bh * kD + tid];
  __syncthreads();
  for (int i = tid; i < G * kLut; i += 256) {
    const int g = i / kLut, e = i % kLut, j = e >> 4, p = e & 15;
    const float* x = &qf[g][4 * j];
    float val = (p & 1) ? -x[0] : x[0];
    val += (p & 2) ? -x[1] : x[1];
    val += (p & 4) ? -x[2] : x[2];
    val += (p & 8) ? -x[3] : x[3];
    lutq[g][e] = val;
  }
  for (int g = wave; g < G; g += 4) {
    float d = fmaf(qf[g][lane], mus[lane], qf[g][lane + 64] * mus[lane + 64]);
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) d += __shfl_xor(d, o);
    if (lane == 0) qmu[g] = d;
  }
  __syncthreads();

  // Phase A: logits (log2 domain).
  if (tid < ne) {
    float lg[G];
    if (t < kSink) {
      const uint16_t* kr = k_sink + ((int64_t)bh * kSink + t) * kD;
#pragma unroll
      for (int g = 0; g < G; ++g) lg[g] = 0.0f;
      for (int c8 = 0; c8 < kD / 8; ++c8) {
        const uint4 w = *reinterpret_cast<const uint4*>(kr + c8 * 8);
        const float x[8] = {bf16lo(w.x), bf16hi(w.x), bf16lo(w.y), bf16hi(w.y),
                            bf16lo(w.z), bf16hi(w.z), bf16lo(w.w), bf16hi(w.w)};
#pragma unroll
        for (int g = 0; g < G; ++g)
#pragma unroll
          for (int i = 0; i < 8; ++i) lg[g] = fmaf(qf[g][c8 * 8 + i], x[i], lg[g]);
      }
    } else {
#pragma unroll
      for (int g = 0; g < G; ++g) lg[g] = fmaf(a, lut_dot(lutq[g], c), qmu[g]);
    }
#pragma unroll
    for (int g = 0; g < G; ++g) pl[g][tid] = lg[g] * sm_log2;
  }
  __syncthreads();

  // Phase B: per-head max and exp2 over the split.
  for (int g = wave; g < G; g += 4) {
    float mx = -INFINITY;
    for (int i = lane; i < ne; i += 64) mx = fmaxf(mx, pl[g][i]);
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o));
    float sum = 0.0f;
    for (int i = lane; i < ne; i += 64) {
      const float p = exp2f(pl[g][i] - mx);
      pl[g][i] = p;
      sum += p;
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) sum += __shfl_xor(sum, o);
    if (lane == 0) {
      wm[g] = mx;
      wl[g] = sum;
    }
  }
  __syncthreads();

  // Phase C: P.V over gathered rows.
  const int rg = tid >> 4, cg = tid & 15;
  float acc[G][8];
#pragma unroll
  for (int g = 0; g < G; ++g)
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[g][i] = 0.0f;
  const uint16_t* vb = v + (int64_t)b * vsb + (int64_t)h * vsh + cg * 8;
  for (int e = rg; e < ne; e += 64) {
    uint4 w[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int ee = e + 16 * u;
      w[u] = ee < ne ? *reinterpret_cast<const uint4*>(vb + (int64_t)tok[ee] * vst)
                     : make_uint4(0u, 0u, 0u, 0u);
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int ee = e + 16 * u;
      if (ee < ne) {
        const float x[8] = {bf16lo(w[u].x), bf16hi(w[u].x), bf16lo(w[u].y), bf16hi(w[u].y),
                            bf16lo(w[u].z), bf16hi(w[u].z), bf16lo(w[u].w), bf16hi(w[u].w)};
#pragma unroll
        for (int g = 0; g < G; ++g) {
          const float p = pl[g][ee];
#pragma unroll
          for (int i = 0; i < 8; ++i) acc[g][i] = fmaf(p, x[i], acc[g][i]);
        }
      }
    }
  }
#pragma unroll
  for (int g = 0; g < G; ++g)
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      float x = acc[g][i];
      x += __shfl_xor(x, 16);
      x += __shfl_xor(x, 32);
      acc[g][i] = x;
    }
  if (lane < 16) {
#pragma unroll
    for (int g = 0; g < G; ++g)
#pragma unroll
      for (int i = 0; i < 8; ++i) red[wave][g][cg * 8 + i] = acc[g][i];
  }
  __syncthreads();
  const int64_t hq0 = (int64_t)b * n_q_heads + (int64_t)h * G;
  for (int i = tid; i < G * kD; i += 256) {
    const int g = i / kD, ch = i % kD;
    const float o = (red[0][g][ch] + red[1][g][ch]) + (red[2][g][ch] + red[3][g][ch]);
    part_o[((hq0 + g) * n_splits + s) * kD + ch] = o;
  }
  if (tid < G) {
    part_ml[((hq0 + tid) * n_splits + s) * 2 + 0] = wm[tid];
    part_ml[((hq0 + tid) * n_splits + s) * 2 + 1] = wl[tid];
  }
}

// out = sum_s 2^(m_s - m) o_s / sum_s 2^(m_s - m) l_s, one block per query head.
__global__ __launch_bounds__(128) void combine_kernel(const float* __restrict__ part_o,
                                                      const float* __restrict__ part_ml,
                                                      int n_splits, float* __restrict__ out) {
  const int64_t r = blockIdx.x;
  const int ch = threadIdx.x;
  const float* ml = part_ml + r * n_splits * 2;
  float m = -INFINITY;
  for (int s = 0; s < n_splits; ++s) m = fmaxf(m, ml[2 * s]);
  float l = 0.0f, o = 0.0f;
  for (int s = 0; s < n_splits; ++s) {
    const float w = exp2f(ml[2 * s] - m);
    l = fmaf(w, ml[2 * s + 1], l);
    o = fmaf(w, part_o[(r * n_splits + s) * kD + ch], o);
  }
  out[r * kD + ch] = o / l;
}

}  // namespace

hipError_t launch_attn(const uint16_t* q, int n_q_heads, int B, int Hkv, const uint8_t* codes,
                       const float* alpha, const float* mu, const uint16_t* k_sink,
                       const uint16_t* v, int64_t vsb, int64_t vsh, int64_t vst, int capacity,
                       int n_tokens, const int32_t* idx, int top_k, float sm_scale, int split,
                       int n_splits, float* part_o, float* part_ml, hipStream_t s) {
  if (split > kSplitMax) return hipErrorInvalidValue;
  const float sm_log2 = sm_scale * 1.4426950408889634f;
  const dim3 grid(n_splits, B * Hkv), block(256);
#define SIKV_ATTN_CASE(GG)                                                                       \
  case GG:                                                                                       \
    return launch_k(KID_ATTN, attn_kernel<GG>, grid, block, 0, s, q, n_q_heads, Hkv, codes,      \
                    alpha, mu, k_sink, v, vsb, vsh, vst, capacity, n_tokens, idx, top_k, sm_log2,\
                    split, n_splits, part_o, part_ml);
  switch (n_q_heads / Hkv) {
    SIKV_ATTN_CASE(1)
    SIKV_ATTN_CASE(2)
    SIKV_ATTN_CASE(3)
    SIKV_ATTN_CASE(4)
    SIKV_ATTN_CASE(5)
    SIKV_ATTN_CASE(6)
    SIKV_ATTN_CASE(7)
    SIKV_ATTN_CASE(8)
    default:
      return hipErrorInvalidValue;
  }
#undef SIKV_ATTN_CASE
}

hipError_t launch_combine(const float* part_o, const float* part_ml, int BHq, int n_splits,
                          float* out, hipStream_t s) {
  return launch_k(KID_COMBINE, combine_kernel, dim3(BHq), dim3(kD), 0, s, part_o, part_ml,
                  n_splits, out);
}

}  // namespace sikv
