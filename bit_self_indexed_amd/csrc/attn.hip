// Fused dequantise + sparse attention over sinks and top-k (gfx950).
//
// "Self-Indexing KVCache: Predicting Sparse Attention from Compressed Keys",
// technical summary §2.1 item 3 (64 full-precision sink tokens always kept) and
// item 4 (dequantisation fused with sparse attention in one pass).
//
// The attended list of one (b, KV head) is entries 0..63 (the sinks) followed
// by the k selected positions.  It is cut into chunks of 32 entries; every wave
// runs its own loop over chunks with an online softmax, so waves never wait for
// each other until the final merge of the block's four waves.  A block serves
// the G query heads of its KV head: each gathered code and V row is read once.
// Per chunk, in one wave:
//   logits   lane (e, half) computes entry e for the heads g = half, half+2, ...:
//            q_g . k^ = q_g . mu + alpha * sum_j LUT_g[j][nibble_j]  (the key is
//            never materialised; rounding mu + alpha*v to fp32 first would be a
//            relative 2^-24 effect, far inside the fp32 accumulation error);
//            sink entries take the exact bf16-key logits made by the prep kernel;
//   softmax  chunk max per head over 32 lanes, running max / sum update,
//            probabilities through a wave-private LDS row;
//   P.V      16-lane group r owns entries r, r+4, ..., r+28: 16 bytes (8 bf16
//            channels) of each V row per lane, fp32 FMAs into G x 8 accumulators.
// The next chunk's codes, scales and V rows are requested before the current
// chunk is computed.  The combine kernel then merges the blocks' partials.
// (A last-block-merges variant needs device-scope fences, which on gfx950 write
// back and invalidate the whole L2 of the XCD in every block: far slower than
// one more launch.)
#include <hip/hip_ext.h>

#include "sikv_internal.h"

namespace sikv {

namespace {

constexpr int kRows = kAttnChunk / 4;  // V rows per 16-lane group per chunk

// Logit inputs of one chunk for one lane.
template <int G>
struct ChunkRegs {
  uint4 code;                   // code of entry (lane & 31)
  float a;                      // its scale (0 for sinks)
  int t;                        // its token position
  float sl[(G + 1) / 2];        // sink logits of this lane's heads (sinks only)
};

__device__ __forceinline__ void wave_sync_lds() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

template <int G>
__device__ __forceinline__ void load_chunk(ChunkRegs<G>& r, int chunk, int L, int lane,
                                           const int32_t* __restrict__ ib,
                                           const uint8_t* __restrict__ crow,
                                           const float* __restrict__ arow, int n_tokens,
                                           const float* __restrict__ slog) {
  const int el = lane & 31, half = lane >> 5;
  const int e = chunk * kAttnChunk + el;
  if (chunk * kAttnChunk < kSink) {  // sink chunk (wave-uniform)
    r.t = e;
    r.code = make_uint4(0u, 0u, 0u, 0u);
    r.a = 0.0f;
#pragma unroll
    for (int i = 0; i < (G + 1) / 2; ++i) r.sl[i] = slog[min(2 * i + half, G - 1) * kSink + e];
  } else {
    // entries past the end re-read the last one; their probabilities are zero
    const int t = min(max(ib[min(e, L - 1) - kSink], 0), n_tokens - 1);  // clamp: memory safety
    r.t = t;
    r.code = *reinterpret_cast<const uint4*>(crow + (int64_t)t * kCodeBytes);
    r.a = arow[t];
#pragma unroll
    for (int i = 0; i < (G + 1) / 2; ++i) r.sl[i] = 0.0f;
  }
}

// Where a lane finds the values of its 8 channels: bf16 rows, or (quantised
// values) 2-bit codes + the group's fp16 (scale, zero) for t >= 64 and the bf16
// sink rows for t < 64.
struct VSource {
  const uint16_t* vb;    // bf16 V at this lane's channels, row stride vst
  int64_t vst;
  const uint8_t* vq;     // this head's value codes, 32 B per token
  const uint32_t* vsz;   // this head's (scale, zero) words, 4 per token
  const uint16_t* vsk;   // this head's bf16 sink rows at this lane's channels
};

// V rows of one chunk for this lane's 16-lane group (t from load_chunk; rows
// past the end of the list are real rows whose probability is zero).  QV and a
// non-sink chunk: .x holds the lane's 16 code bits, .y its group's scale/zero.
template <bool QV>
__device__ __forceinline__ void load_rows(uint4 (&vr)[kRows], int lane, int t, bool sink_chunk,
                                          const VSource& vs) {
  const int grp = lane >> 4, seg = lane & 15;
#pragma unroll
  for (int u = 0; u < kRows; ++u) {
    const int tu = __shfl(t, grp + 4 * u);
    if (!QV) {
      vr[u] = *reinterpret_cast<const uint4*>(vs.vb + (int64_t)tu * vs.vst);
    } else if (sink_chunk) {
      vr[u] = *reinterpret_cast<const uint4*>(vs.vsk + (int64_t)tu * kD);
    } else {
      vr[u].x = *reinterpret_cast<const uint16_t*>(vs.vq + (int64_t)tu * kVCodeBytes + 2 * seg);
      vr[u].y = vs.vsz[(int64_t)tu * 4 + (seg >> 2)];
      vr[u].z = 0u;
      vr[u].w = 0u;
    }
  }
}

template <int G, bool QV>
__global__ __launch_bounds__(256, (G <= 4 && !QV) ? 4 : 2) void attn_kernel(
    int n_q_heads, int Hkv, const uint8_t* __restrict__ codes, const float* __restrict__ alpha,
    const uint16_t* __restrict__ v, int64_t vsb, int64_t vsh, int64_t vst,
    const uint8_t* __restrict__ vq, const uint32_t* __restrict__ vsz,
    const uint16_t* __restrict__ vsink, int capacity,
    int n_tokens, const int32_t* __restrict__ idx, int top_k, const float* __restrict__ att_lut,
    const float* __restrict__ att_qmu, const float* __restrict__ att_slog, float sm_log2,
    int cpb, int n_splits, float* __restrict__ part_o, float* __restrict__ part_ml) {
  constexpr int GH = (G + 1) / 2;
  __shared__ float lutq[G][kLut];
  __shared__ __align__(16) float pb[4][kAttnChunk][G];
  __shared__ float mo[4][G][kD];
  __shared__ float mml[4][G][2];

  const int bh = blockIdx.y, b = bh / Hkv, h = bh - b * Hkv;
  const int s = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int el = lane & 31, half = lane >> 5, seg = lane & 15, grp = lane >> 4;
  const int L = kSink + top_k;
  const int n_chunks = (L + kAttnChunk - 1) / kAttnChunk;
  const int c_end = min(n_chunks, (s + 1) * cpb);
  const int64_t row0 = (int64_t)bh * capacity;
  const int64_t hq0 = (int64_t)b * n_q_heads + (int64_t)h * G;
  const int32_t* ib = idx + (int64_t)bh * top_k;
  const uint8_t* crow = codes + row0 * kCodeBytes;
  const float* arow = alpha + row0;
  VSource vs;
  vs.vb = QV ? nullptr : v + (int64_t)b * vsb + (int64_t)h * vsh + seg * 8;
  vs.vst = vst;
  vs.vq = QV ? vq + row0 * kVCodeBytes : nullptr;
  vs.vsz = QV ? vsz + row0 * 4 : nullptr;
  vs.vsk = QV ? vsink + (int64_t)bh * kSink * kD + seg * 8 : nullptr;
  const float* slog = att_slog + hq0 * kSink;

  int c = s * cpb + wave;
  ChunkRegs<G> nx;
  if (c < c_end) load_chunk<G>(nx, c, L, lane, ib, crow, arow, n_tokens, slog);

  {
    const float4* src = reinterpret_cast<const float4*>(att_lut + hq0 * kLut);
    float4* dst = reinterpret_cast<float4*>(&lutq[0][0]);
    for (int i = tid; i < G * kLut / 4; i += 256) dst[i] = src[i];
  }
  float qmu[GH];
#pragma unroll
  for (int i = 0; i < GH; ++i) qmu[i] = (2 * i + half < G) ? att_qmu[hq0 + 2 * i + half] : 0.0f;
  __syncthreads();

  float m[G], lsum[GH], acc[G][8], zacc[G];  // zacc: sum of p * zero point (QV)
#pragma unroll
  for (int g = 0; g < G; ++g) {
    m[g] = -INFINITY;
    zacc[g] = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[g][i] = 0.0f;
  }
#pragma unroll
  for (int i = 0; i < GH; ++i) lsum[i] = 0.0f;

  for (; c < c_end; c += 4) {
    const ChunkRegs<G> cur = nx;
    if (c + 4 < c_end) load_chunk<G>(nx, c + 4, L, lane, ib, crow, arow, n_tokens, slog);
    const bool live = c * kAttnChunk + el < L;
    // logits (log2 domain) of this lane's heads g = 2i + half
    float lg[GH];
#pragma unroll
    for (int i = 0; i < GH; ++i) {
      const int g = min(2 * i + half, G - 1);
      float dot;
      if (c * kAttnChunk < kSink) {
        dot = cur.sl[i];
      } else {
        dot = fmaf(cur.a, lut_dot(lutq[g], cur.code), qmu[i]);
      }
      lg[i] = (live && 2 * i + half < G) ? dot * sm_log2 : -INFINITY;
    }
    const bool sink_chunk = c * kAttnChunk < kSink;
    uint4 vr[kRows];
    load_rows<QV>(vr, lane, cur.t, sink_chunk, vs);
    // chunk max per head: heads of parity `half` live in this half of the wave
    float cm[GH], co[GH];
#pragma unroll
    for (int i = 0; i < GH; ++i) {
      float x = lg[i];
#pragma unroll
      for (int o = 16; o > 0; o >>= 1) x = fmaxf(x, __shfl_xor(x, o));
      cm[i] = x;
      co[i] = __shfl_xor(x, 32);
    }
    float sc[G];
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const float mx = ((g & 1) == half) ? cm[g >> 1] : co[g >> 1];
      const float mn = fmaxf(m[g], mx);
      sc[g] = exp2f(m[g] - mn);
      m[g] = mn;
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[g][i] *= sc[g];
      if (QV) zacc[g] *= sc[g];
    }
#pragma unroll
    for (int i = 0; i < GH; ++i) {
      const int g1 = min(2 * i + 1, G - 1);
      const float mg = half ? m[g1] : m[2 * i];
      const float sg = half ? sc[g1] : sc[2 * i];
      const float p = exp2f(lg[i] - mg);
      lsum[i] = fmaf(lsum[i], sg, p);
      if (2 * i + half < G) pb[wave][el][2 * i + half] = p;
    }
    wave_sync_lds();
    // P.V
    if (!QV || sink_chunk) {
#pragma unroll
      for (int u = 0; u < kRows; ++u) {
        const int eu = grp + 4 * u;
        const uint4 w = vr[u];
        const float x[8] = {bf16lo(w.x), bf16hi(w.x), bf16lo(w.y), bf16hi(w.y),
                            bf16lo(w.z), bf16hi(w.z), bf16lo(w.w), bf16hi(w.w)};
#pragma unroll
        for (int g = 0; g < G; ++g) {
          const float p = pb[wave][eu][g];
#pragma unroll
          for (int i = 0; i < 8; ++i) acc[g][i] = fmaf(p, x[i], acc[g][i]);
        }
      }
    } else {
      // v = z + q * s: acc += (p * s) * q per channel, p * z once per row
#pragma unroll
      for (int u = 0; u < kRows; ++u) {
        const int eu = grp + 4 * u;
        const uint32_t qb = vr[u].x, sz = vr[u].y;
        const float sv = __half2float(__ushort_as_half((unsigned short)(sz & 0xffffu)));
        const float zv = __half2float(__ushort_as_half((unsigned short)(sz >> 16)));
        float qf[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) qf[i] = (float)((qb >> (2 * i)) & 3u);
#pragma unroll
        for (int g = 0; g < G; ++g) {
          const float p = pb[wave][eu][g];
          const float ps = p * sv;
          zacc[g] = fmaf(p, zv, zacc[g]);
#pragma unroll
          for (int i = 0; i < 8; ++i) acc[g][i] = fmaf(ps, qf[i], acc[g][i]);
        }
      }
    }
    wave_sync_lds();
  }

  // Wave partial: sums over the four 16-lane groups and over the 32 lanes.
#pragma unroll
  for (int g = 0; g < G; ++g)
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      float x = QV ? acc[g][i] + zacc[g] : acc[g][i];
      x += __shfl_xor(x, 16);
      x += __shfl_xor(x, 32);
      acc[g][i] = x;
    }
#pragma unroll
  for (int i = 0; i < GH; ++i) {
    float x = lsum[i];
#pragma unroll
    for (int o = 16; o > 0; o >>= 1) x += __shfl_xor(x, o);
    lsum[i] = x;
  }
  if (lane < 16) {
#pragma unroll
    for (int g = 0; g < G; ++g)
#pragma unroll
      for (int i = 0; i < 8; ++i) mo[wave][g][seg * 8 + i] = acc[g][i];
  }
  if (el == 0) {
#pragma unroll
    for (int i = 0; i < GH; ++i) {
      const int g = 2 * i + half;
      if (g < G) {
        mml[wave][g][0] = half ? m[min(2 * i + 1, G - 1)] : m[2 * i];
        mml[wave][g][1] = lsum[i];
      }
    }
  }
  __syncthreads();
  // Block merge of the four wave partials (waves without a chunk hold -inf, 0).
  for (int i = tid; i < G * kD; i += 256) {
    const int g = i / kD, ch = i % kD;
    const float M = fmaxf(fmaxf(mml[0][g][0], mml[1][g][0]), fmaxf(mml[2][g][0], mml[3][g][0]));
    float o = 0.0f, l = 0.0f;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const float f = exp2f(mml[w][g][0] - M);
      o = fmaf(f, mo[w][g][ch], o);
      l = fmaf(f, mml[w][g][1], l);
    }
    part_o[((hq0 + g) * n_splits + s) * kD + ch] = o;
    if (ch == 0) {
      part_ml[((hq0 + g) * n_splits + s) * 2 + 0] = M;
      part_ml[((hq0 + g) * n_splits + s) * 2 + 1] = l;
    }
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

hipError_t launch_attn(int n_q_heads, int B, int Hkv, const uint8_t* codes, const float* alpha,
                       const uint16_t* v, int64_t vsb, int64_t vsh, int64_t vst,
                       const uint8_t* vq, const uint32_t* vsz, const uint16_t* vsink, int capacity,
                       int n_tokens, const int32_t* idx, int top_k, const float* att_lut,
                       const float* att_qmu, const float* att_slog, float sm_scale,
                       int chunks_per_block, int n_splits, float* part_o, float* part_ml,
                       hipStream_t s) {
  const int n_chunks = (kSink + top_k + kAttnChunk - 1) / kAttnChunk;
  if (chunks_per_block < 1 || (int64_t)n_splits * chunks_per_block < n_chunks ||
      (int64_t)(n_splits - 1) * chunks_per_block >= n_chunks)
    return hipErrorInvalidValue;
  const float sm_log2 = sm_scale * 1.4426950408889634f;
  const dim3 grid(n_splits, B * Hkv), block(256);
#define SIKV_ATTN_CASE(GG)                                                                     \
  case GG:                                                                                     \
    if (vq != nullptr)                                                                         \
      return launch_k(KID_ATTN, attn_kernel<GG, true>, grid, block, 0, s, n_q_heads, Hkv,      \
                      codes, alpha, v, vsb, vsh, vst, vq, vsz, vsink, capacity, n_tokens, idx, \
                      top_k, att_lut, att_qmu, att_slog, sm_log2, chunks_per_block, n_splits,  \
                      part_o, part_ml);                                                        \
    return launch_k(KID_ATTN, attn_kernel<GG, false>, grid, block, 0, s, n_q_heads, Hkv,       \
                    codes, alpha, v, vsb, vsh, vst, vq, vsz, vsink, capacity, n_tokens, idx,   \
                    top_k, att_lut, att_qmu, att_slog, sm_log2, chunks_per_block, n_splits,    \
                    part_o, part_ml);
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
