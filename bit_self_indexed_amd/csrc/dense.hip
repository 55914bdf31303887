// Dense bf16 decode attention over every cached token (gfx950): the
// comparator the sparse path is measured against (the summary compares with
// full FlashAttention-2 attention, §3 and §4).  Split-K flash decoding: one
// block per (split of the tokens, b*h), serving all G query heads so each K/V
// row is read once per KV head.  Per sub-block of 256 tokens:
//   A  16 lanes x 16 bytes per K row, partial dots for the G heads, xor-butterfly
//      over the 16 lanes; 4 rows in flight per lane group;
//   B  per head: sub-block max, running-max rescale, exp2, running sum;
//   C  16 lanes x 16 bytes per V row, fp32 FMAs into the running accumulators.
// Partials go through the same combine kernel as the sparse path.
#include <hip/hip_ext.h>

#include "sikv_internal.h"

namespace sikv {

namespace {

constexpr int kTile = 256;

template <int G>
__global__ __launch_bounds__(256) void dense_kernel(
    const uint16_t* __restrict__ q, int n_q_heads, int Hkv, int n_tokens,
    const uint16_t* __restrict__ k, int64_t ksb, int64_t ksh, int64_t kst,
    const uint16_t* __restrict__ v, int64_t vsb, int64_t vsh, int64_t vst, float sm_log2, int split,
    int n_splits, float* __restrict__ part_o, float* __restrict__ part_ml) {
  __shared__ float pl[G][kTile];
  __shared__ float red[4][G][kD];
  __shared__ float run_m[G], run_l[G], scale_s[G];
  const int bh = blockIdx.y, b = bh / Hkv, h = bh - b * Hkv;
  const int s = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int rg = tid >> 4, cg = tid & 15;
  const int t_begin = s * split;
  const int t_end = min(n_tokens, t_begin + split);

  float qr[G][8];
  {
    const uint16_t* qb = q + ((int64_t)b * n_q_heads + (int64_t)h * G) * kD + cg * 8;
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const uint4 w = *reinterpret_cast<const uint4*>(qb + g * kD);
      qr[g][0] = bf16lo(w.x) * sm_log2; qr[g][1] = bf16hi(w.x) * sm_log2;
      qr[g][2] = bf16lo(w.y) * sm_log2; qr[g][3] = bf16hi(w.y) * sm_log2;
      qr[g][4] = bf16lo(w.z) * sm_log2; qr[g][5] = bf16hi(w.z) * sm_log2;
      qr[g][6] = bf16lo(w.w) * sm_log2; qr[g][7] = bf16hi(w.w) * sm_log2;
    }
  }
  if (tid < G) {
    run_m[tid] = -INFINITY;
    run_l[tid] = 0.0f;
  }
  float acc[G][8];
#pragma unroll
  for (int g = 0; g < G; ++g)
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[g][i] = 0.0f;
  const uint16_t* kb = k + (int64_t)b * ksb + (int64_t)h * ksh + cg * 8;
  const uint16_t* vb = v + (int64_t)b * vsb + (int64_t)h * vsh + cg * 8;

  for (int sb0 = t_begin; sb0 < t_end; sb0 += kTile) {
    const int ne = min(kTile, t_end - sb0);
    // A: logits
    for (int e = rg; e < ne; e += 64) {
      uint4 w[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int ee = e + 16 * u;
        w[u] = ee < ne ? *reinterpret_cast<const uint4*>(kb + (int64_t)(sb0 + ee) * kst)
                       : make_uint4(0u, 0u, 0u, 0u);
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const float x[8] = {bf16lo(w[u].x), bf16hi(w[u].x), bf16lo(w[u].y), bf16hi(w[u].y),
                            bf16lo(w[u].z), bf16hi(w[u].z), bf16lo(w[u].w), bf16hi(w[u].w)};
        float d[G];
#pragma unroll
        for (int g = 0; g < G; ++g) {
          float t = qr[g][0] * x[0];
#pragma unroll
          for (int i = 1; i < 8; ++i) t = fmaf(qr[g][i], x[i], t);
          t += __shfl_xor(t, 1);
          t += __shfl_xor(t, 2);
          t += __shfl_xor(t, 4);
          t += __shfl_xor(t, 8);
          d[g] = t;
        }
        const int ee = e + 16 * u;
        if (cg == 0 && ee < ne) {
#pragma unroll
          for (int g = 0; g < G; ++g) pl[g][ee] = d[g];
        }
      }
    }
    __syncthreads();
    // B: running softmax state
    for (int g = wave; g < G; g += 4) {
      float mx = -INFINITY;
      for (int i = lane; i < ne; i += 64) mx = fmaxf(mx, pl[g][i]);
#pragma unroll
      for (int o = 32; o > 0; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o));
      const float m_old = run_m[g];
      const float m_new = fmaxf(m_old, mx);
      float sum = 0.0f;
      for (int i = lane; i < ne; i += 64) {
        const float p = exp2f(pl[g][i] - m_new);
        pl[g][i] = p;
        sum += p;
      }
#pragma unroll
      for (int o = 32; o > 0; o >>= 1) sum += __shfl_xor(sum, o);
      if (lane == 0) {
        const float sc = exp2f(m_old - m_new);
        scale_s[g] = sc;
        run_l[g] = fmaf(run_l[g], sc, sum);
        run_m[g] = m_new;
      }
    }
    __syncthreads();
    // C: rescale and accumulate P.V
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const float sc = scale_s[g];
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[g][i] *= sc;
    }
    for (int e = rg; e < ne; e += 64) {
      uint4 w[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int ee = e + 16 * u;
        w[u] = ee < ne ? *reinterpret_cast<const uint4*>(vb + (int64_t)(sb0 + ee) * vst)
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
    __syncthreads();
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
    part_o[((hq0 + g) * n_splits + s) * kD + ch] =
        (red[0][g][ch] + red[1][g][ch]) + (red[2][g][ch] + red[3][g][ch]);
  }
  if (tid < G) {
    part_ml[((hq0 + tid) * n_splits + s) * 2 + 0] = run_m[tid];
    part_ml[((hq0 + tid) * n_splits + s) * 2 + 1] = run_l[tid];
  }
}

// Full dot-product retrieval (the comparator of the LUT-GEMV score): one block
// per (256 tokens, b*h); 16 lanes x 16 bytes per bf16 key row, all 16 rows of
// a thread issued before any is used, partial dots reduced over the 16 lanes.
// The selection query qbar = sum of the G query rows (fp32, g ascending), each
// lane holding its 8 channels.
constexpr int kScoreRows = 16;  // rows per 16-lane group per block
__global__ __launch_bounds__(256) void dense_scores_kernel(
    const uint16_t* __restrict__ q, int n_q_heads, int Hkv, int G, int n_tokens,
    const uint16_t* __restrict__ k, int64_t ksb, int64_t ksh, int64_t kst,
    float* __restrict__ scores) {
  const int bh = blockIdx.y, b = bh / Hkv, h = bh - b * Hkv;
  const int tid = threadIdx.x, rg = tid >> 4, cg = tid & 15;
  float qs[8];
  {
    const uint16_t* qb = q + ((int64_t)b * n_q_heads + (int64_t)h * G) * kD + cg * 8;
    const uint4 w0 = *reinterpret_cast<const uint4*>(qb);
#pragma unroll
    for (int i = 0; i < 8; ++i) qs[i] = chan(w0, i);
    for (int g = 1; g < G; ++g) {
      const uint4 w = *reinterpret_cast<const uint4*>(qb + (int64_t)g * kD);
#pragma unroll
      for (int i = 0; i < 8; ++i) qs[i] += chan(w, i);
    }
  }
  const int t0 = blockIdx.x * 16 * kScoreRows;
  const uint16_t* kb = k + (int64_t)b * ksb + (int64_t)h * ksh + cg * 8;
  uint4 w[kScoreRows];
#pragma unroll
  for (int u = 0; u < kScoreRows; ++u) {
    const int t = t0 + u * 16 + rg;
    w[u] = t < n_tokens ? *reinterpret_cast<const uint4*>(kb + (int64_t)t * kst)
                        : make_uint4(0u, 0u, 0u, 0u);
  }
#pragma unroll
  for (int u = 0; u < kScoreRows; ++u) {
    float d = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) d = fmaf(qs[i], chan(w[u], i), d);
    d += __shfl_xor(d, 8);
    d += __shfl_xor(d, 4);
    d += __shfl_xor(d, 2);
    d += __shfl_xor(d, 1);
    const int t = t0 + u * 16 + rg;
    if (cg == 0 && t < n_tokens) scores[(int64_t)bh * n_tokens + t] = d;
  }
}

}  // namespace

hipError_t launch_dense_scores(const uint16_t* q, int n_q_heads, int B, int Hkv, int n_tokens,
                               const uint16_t* k, int64_t ksb, int64_t ksh, int64_t kst,
                               float* scores, const Launch& s) {
  const int G = n_q_heads / Hkv;
  if (G < 1 || G * Hkv != n_q_heads || n_tokens < 1) return hipErrorInvalidValue;
  const dim3 grid((n_tokens + 16 * kScoreRows - 1) / (16 * kScoreRows), B * Hkv), block(256);
  return launch_k(KID_DSCORES, dense_scores_kernel, grid, block, 0, s, q, n_q_heads, Hkv, G,
                  n_tokens, k, ksb, ksh, kst, scores);
}

hipError_t launch_dense(const uint16_t* q, int n_q_heads, int B, int Hkv, int n_tokens,
                        const uint16_t* k, int64_t ksb, int64_t ksh, int64_t kst,
                        const uint16_t* v, int64_t vsb, int64_t vsh, int64_t vst, float sm_scale,
                        int split, int n_splits, float* part_o, float* part_ml, const Launch& s) {
  const float sm_log2 = sm_scale * 1.4426950408889634f;
  const dim3 grid(n_splits, B * Hkv), block(256);
#define SIKV_DENSE_CASE(GG)                                                                     \
  case GG:                                                                                      \
    return launch_k(KID_DENSE, dense_kernel<GG>, grid, block, 0, s, q, n_q_heads, Hkv, n_tokens, \
                    k, ksb, ksh, kst, v, vsb, vsh, vst, sm_log2, split, n_splits, part_o,       \
                    part_ml);
  switch (n_q_heads / Hkv) {
    SIKV_DENSE_CASE(1)
    SIKV_DENSE_CASE(2)
    SIKV_DENSE_CASE(3)
    SIKV_DENSE_CASE(4)
    SIKV_DENSE_CASE(5)
    SIKV_DENSE_CASE(6)
    SIKV_DENSE_CASE(7)
    SIKV_DENSE_CASE(8)
    default:
      return hipErrorInvalidValue;
  }
#undef SIKV_DENSE_CASE
}

}  // namespace sikv
