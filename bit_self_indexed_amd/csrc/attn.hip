// Fused dequantise + sparse attention over sinks and top-k (gfx950).
//
// "Self-Indexing KVCache: Predicting Sparse Attention from Compressed Keys",
// technical summary §2.1 item 3 (64 full-precision sink tokens always kept) and
// item 4 (dequantisation fused with sparse attention in one pass).
//
// One block per (split of <= 256 attended entries, b*h); the block serves the G
// query heads of the KV head, so every gathered code and V row is read once per
// KV head.  Order of work inside a block:
//   1  each 16-lane group issues the gathers of its V rows (16 bytes per lane)
//      as soon as the indices are known; they are consumed last;
//   2  one lane per entry loads its code and scale (sinks: the bf16 key row);
//   3  the per-query-head tables LUT_g[j][p] = q_g(4j..4j+3) . (sign vertex p)
//      and q_g . mu, built once per KV head by the prep kernel, are copied to LDS;
//   4  logits: q.k^ = q.mu + alpha * sum_j LUT_g[j][nibble_j] (the key is never
//      materialised; rounding mu + alpha*v to fp32 first is a relative 2^-24
//      effect, far inside the fp32 accumulation error); sinks: exact dot with
//      the bf16 row; pre-scaled by log2(e) * sm_scale;
//   5  per head: max, exp2, sum over the split;
//   6  P.V from the prefetched rows, fp32 FMAs, reduced over the 16 groups,
//      written as this split's (max, sum, o) partial.
// The combine kernel then merges the splits.  (A last-block-merges variant
// needs device-scope fences, which on gfx950 write back and invalidate the
// whole L2 of the XCD in every block: far slower than one more launch.)
#include <hip/hip_ext.h>

#include "sikv_internal.h"

namespace sikv {

namespace {

constexpr int kSplitMax = 256;       // attended-list entries per block
constexpr int kPf = kSplitMax / 16;  // V rows prefetched per 16-lane group

template <int G>
__global__ __launch_bounds__(256) void attn_kernel(
    const uint16_t* __restrict__ q, int n_q_heads, int Hkv, const uint8_t* __restrict__ codes,
    const float* __restrict__ alpha, const uint16_t* __restrict__ k_sink,
    const uint16_t* __restrict__ v, int64_t vsb, int64_t vsh, int64_t vst, int capacity,
    int n_tokens, const int32_t* __restrict__ idx, int top_k, const float* __restrict__ att_lut,
    const float* __restrict__ att_qmu, float sm_log2, int split, int n_splits,
    float* __restrict__ part_o, float* __restrict__ part_ml) {
  __shared__ float qf[G][kD];
  __shared__ float lutq[G][kLut];
  __shared__ float pl[G][kSplitMax];
  __shared__ float red[4][G][kD];
  __shared__ float wm[G], wl[G];

  const int bh = blockIdx.y, b = bh / Hkv, h = bh - b * Hkv;
  const int s = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int rg = tid >> 4, cg = tid & 15;
  const int L = kSink + top_k;
  const int e0 = s * split;
  const int ne = min(L, e0 + split) - e0;
  const int64_t row0 = (int64_t)bh * capacity;
  const int32_t* ib = idx + (int64_t)bh * top_k;
  const int64_t hq0 = (int64_t)b * n_q_heads + (int64_t)h * G;

  // 1. V rows of this lane group's entries.
  const uint16_t* vb = v + (int64_t)b * vsb + (int64_t)h * vsh + cg * 8;
  uint4 vr[kPf];
#pragma unroll
  for (int u = 0; u < kPf; ++u) {
    const int el = rg + 16 * u;
    uint4 w = make_uint4(0u, 0u, 0u, 0u);
    if (el < ne) {
      const int e = e0 + el;
      int t = e < kSink ? e : ib[e - kSink];
      t = min(max(t, 0), n_tokens - 1);  // memory safety only: indices must be valid
      w = *reinterpret_cast<const uint4*>(vb + (int64_t)t * vst);
    }
    vr[u] = w;
  }
  // 2. Logit inputs: one lane per entry.
  int ta = 0;
  uint4 ch = make_uint4(0u, 0u, 0u, 0u);
  float a = 0.0f;
  if (tid < ne) {
    const int e = e0 + tid;
    ta = e < kSink ? e : ib[e - kSink];
    ta = min(max(ta, 0), n_tokens - 1);
    if (ta >= kSink) {
      ch = *reinterpret_cast<const uint4*>(codes + (row0 + ta) * kCodeBytes);
      a = alpha[row0 + ta];
    }
  }
  // 3. Tables of the G query heads (and the queries themselves if this split
  //    holds sink entries).
  {
    const float4* src = reinterpret_cast<const float4*>(att_lut + hq0 * kLut);
    float4* dst = reinterpret_cast<float4*>(&lutq[0][0]);
    for (int i = tid; i < G * kLut / 4; i += 256) dst[i] = src[i];
  }
  if (e0 < kSink) {
    const uint16_t* qb = q + hq0 * kD;
    for (int i = tid; i < G * kD; i += 256)
      qf[i / kD][i % kD] = __uint_as_float((uint32_t)qb[i] << 16);
  }
  float qmu[G];
#pragma unroll
  for (int g = 0; g < G; ++g) qmu[g] = att_qmu[hq0 + g];
  __syncthreads();

  // 4. Logits (log2 domain).
  if (tid < ne) {
    float lg[G];
    if (ta < kSink) {
      const uint16_t* kr = k_sink + ((int64_t)bh * kSink + ta) * kD;
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
      for (int g = 0; g < G; ++g) lg[g] = fmaf(a, lut_dot(lutq[g], ch), qmu[g]);
    }
#pragma unroll
    for (int g = 0; g < G; ++g) pl[g][tid] = lg[g] * sm_log2;
  }
  __syncthreads();

  // 5. Per-head max and exp2 over the split.
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

  // 6. P.V over the prefetched rows.
  float acc[G][8];
#pragma unroll
  for (int g = 0; g < G; ++g)
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[g][i] = 0.0f;
#pragma unroll
  for (int u = 0; u < kPf; ++u) {
    const int el = rg + 16 * u;
    if (el < ne) {
      const uint4 w = vr[u];
      const float x[8] = {bf16lo(w.x), bf16hi(w.x), bf16lo(w.y), bf16hi(w.y),
                          bf16lo(w.z), bf16hi(w.z), bf16lo(w.w), bf16hi(w.w)};
#pragma unroll
      for (int g = 0; g < G; ++g) {
        const float p = pl[g][el];
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[g][i] = fmaf(p, x[i], acc[g][i]);
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
  for (int i = tid; i < G * kD; i += 256) {
    const int g = i / kD, c = i % kD;
    part_o[((hq0 + g) * n_splits + s) * kD + c] =
        (red[0][g][c] + red[1][g][c]) + (red[2][g][c] + red[3][g][c]);
  }
  if (tid < G) {
    part_ml[((hq0 + tid) * n_splits + s) * 2 + 0] = wm[tid];
    part_ml[((hq0 + tid) * n_splits + s) * 2 + 1] = wl[tid];
  }
}

// Split merge, one block per query head:
//   out = sum_s 2^(m_s - M) o_s / sum_s 2^(m_s - M) l_s,  M = max_s m_s.
// Thread (split group sg of 8, channel quad cq of 32) accumulates every 8th
// split with float4 loads, 4 splits in flight; groups are summed in LDS.
__global__ __launch_bounds__(256) void combine_kernel(const float* __restrict__ part_o,
                                                      const float* __restrict__ part_ml,
                                                      int n_splits, float* __restrict__ out) {
  __shared__ float red[8][kD];
  __shared__ float wred[2][4];
  const int64_t r = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int sg = tid >> 5, cq = tid & 31;
  const float* ml = part_ml + r * n_splits * 2;
  float m = -INFINITY;
  for (int s = tid; s < n_splits; s += 256) m = fmaxf(m, ml[2 * s]);
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) m = fmaxf(m, __shfl_xor(m, o));
  if (lane == 0) wred[0][wave] = m;
  __syncthreads();
  m = fmaxf(fmaxf(wred[0][0], wred[0][1]), fmaxf(wred[0][2], wred[0][3]));
  float l = 0.0f;
  for (int s = tid; s < n_splits; s += 256) l = fmaf(exp2f(ml[2 * s] - m), ml[2 * s + 1], l);
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) l += __shfl_xor(l, o);
  if (lane == 0) wred[1][wave] = l;
  const float4* po = reinterpret_cast<const float4*>(part_o + r * n_splits * kD) + cq;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  int s = sg;
  for (; s + 24 < n_splits; s += 32) {
    float wv[4];
    float4 ov[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      wv[u] = ml[2 * (s + 8 * u)];
      ov[u] = po[(int64_t)(s + 8 * u) * (kD / 4)];
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const float w = exp2f(wv[u] - m);
      acc.x = fmaf(w, ov[u].x, acc.x);
      acc.y = fmaf(w, ov[u].y, acc.y);
      acc.z = fmaf(w, ov[u].z, acc.z);
      acc.w = fmaf(w, ov[u].w, acc.w);
    }
  }
  for (; s < n_splits; s += 8) {
    const float w = exp2f(ml[2 * s] - m);
    const float4 ov = po[(int64_t)s * (kD / 4)];
    acc.x = fmaf(w, ov.x, acc.x);
    acc.y = fmaf(w, ov.y, acc.y);
    acc.z = fmaf(w, ov.z, acc.z);
    acc.w = fmaf(w, ov.w, acc.w);
  }
  red[sg][cq * 4 + 0] = acc.x;
  red[sg][cq * 4 + 1] = acc.y;
  red[sg][cq * 4 + 2] = acc.z;
  red[sg][cq * 4 + 3] = acc.w;
  __syncthreads();
  if (tid < kD) {
    const float L = (wred[1][0] + wred[1][1]) + (wred[1][2] + wred[1][3]);
    const float o = ((red[0][tid] + red[1][tid]) + (red[2][tid] + red[3][tid])) +
                    ((red[4][tid] + red[5][tid]) + (red[6][tid] + red[7][tid]));
    out[r * kD + tid] = o / L;
  }
}

}  // namespace

hipError_t launch_attn(const uint16_t* q, int n_q_heads, int B, int Hkv, const uint8_t* codes,
                       const float* alpha, const uint16_t* k_sink, const uint16_t* v, int64_t vsb,
                       int64_t vsh, int64_t vst, int capacity, int n_tokens, const int32_t* idx,
                       int top_k, const float* att_lut, const float* att_qmu, float sm_scale,
                       int split, int n_splits, float* part_o, float* part_ml, hipStream_t s) {
  if (split > kSplitMax) return hipErrorInvalidValue;
  const float sm_log2 = sm_scale * 1.4426950408889634f;
  const dim3 grid(n_splits, B * Hkv), block(256);
#define SIKV_ATTN_CASE(GG)                                                                     \
  case GG:                                                                                     \
    return launch_k(KID_ATTN, attn_kernel<GG>, grid, block, 0, s, q, n_q_heads, Hkv, codes,    \
                    alpha, k_sink, v, vsb, vsh, vst, capacity, n_tokens, idx, top_k, att_lut,  \
                    att_qmu, sm_log2, split, n_splits, part_o, part_ml);
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
  return launch_k(KID_COMBINE, combine_kernel, dim3(BHq), dim3(256), 0, s, part_o, part_ml,
                  n_splits, out);
}

}  // namespace sikv
