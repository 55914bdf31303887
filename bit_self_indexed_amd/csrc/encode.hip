// Prefill / append compression of the key cache (gfx950).
//
// "Self-Indexing KVCache: Predicting Sparse Attention from Compressed Keys",
// technical summary §2.1 item 1: keys are centred by their channel mean
// (entropy-aware normalisation), then every channel contributes its sign as one
// bit, so each 4-dim sub-vector lands in one of 16 clusters; §2.1 item 3: the
// format is token-wise and the 64 first tokens stay in full precision.
//
// Bit-exactness: the mean and the per-token scale are sums whose rounding
// decides the codes, so both follow one fixed order, the adjacent-pair binary
// tree in fp32 (mean: over the token axis with sink rows and rows past N as
// +0.0, padded to a power of two; scale: over the 128 channels).  Every
// blocking below is an aligned power-of-two split of that tree.
#include <hip/hip_ext.h>

#include "sikv_internal.h"

namespace sikv {

namespace {

// Pairwise tree over 16 leaves (one aligned 16-leaf subtree).
__device__ __forceinline__ float tree16(const float* l) {
  const float a0 = l[0] + l[1], a1 = l[2] + l[3], a2 = l[4] + l[5], a3 = l[6] + l[7];
  const float a4 = l[8] + l[9], a5 = l[10] + l[11], a6 = l[12] + l[13], a7 = l[14] + l[15];
  const float b0 = a0 + a1, b1 = a2 + a3, b2 = a4 + a5, b3 = a6 + a7;
  return (b0 + b1) + (b2 + b3);
}

// Mean, stage 1: one block per (4096-token tile, b*h), 16 sub-tiles of 256
// tokens in turn.  In a sub-tile, thread (rs, cg) owns the aligned 16-row group
// rs and channels 8cg..8cg+7; its 16-leaf subtree is summed in registers and
// the 16 group sums are combined by the next 4 levels of the tree; the 16
// sub-tile sums then form the 4 levels above.  Leaves outside [64, N) are +0.0
// (never loaded).
__global__ __launch_bounds__(256) void mu_partial_kernel(const uint16_t* __restrict__ k, int64_t sb,
                                                         int64_t sh, int64_t st, int Hkv,
                                                         int n_tokens, float* __restrict__ partial,
                                                         int nblk) {
  __shared__ float red[16][kD + 1];
  __shared__ float subs[16][kD];
  const int bh = blockIdx.y, b = bh / Hkv, h = bh - b * Hkv;
  const int tid = threadIdx.x, cg = tid & 15, rs = tid >> 4;
  const uint16_t* base = k + (int64_t)b * sb + (int64_t)h * sh + cg * 8;
  for (int sub = 0; sub < 16; ++sub) {
    const int t0 = blockIdx.x * kMuTile + sub * 256 + rs * 16;
    uint4 w[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int t = t0 + i;
      w[i] = (t >= kSink && t < n_tokens) ? *reinterpret_cast<const uint4*>(base + (int64_t)t * st)
                                          : make_uint4(0u, 0u, 0u, 0u);
    }
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      float l[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) l[i] = chan(w[i], c);
      red[rs][cg * 8 + c] = tree16(l);
    }
    __syncthreads();
    if (tid < kD) {
      float l[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) l[r] = red[r][tid];
      subs[sub][tid] = tree16(l);
    }
    __syncthreads();
  }
  if (tid < kD) {
    float l[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) l[r] = subs[r][tid];
    partial[((int64_t)bh * nblk + blockIdx.x) * kD + tid] = tree16(l);
  }
}

// Mean, stage 2: one block per b*h, one thread per channel.  The tile sums are
// the leaves of the remaining levels (padded with +0.0 to a power of two) and
// are reduced by a binary counter: leaf i is merged with the pending subtree of
// each level where i has a trailing 1 bit, which is exactly the pairwise tree.
// Leaves are loaded 16 at a time ahead of the merges.
__global__ __launch_bounds__(128) void mu_final_kernel(const float* __restrict__ partial, int nblk,
                                                       int n_tokens, float* __restrict__ mu) {
  __shared__ float stk[32][kD];
  const int bh = blockIdx.x, c = threadIdx.x;
  int n2 = 1, levels = 0;
  while (n2 < nblk) {
    n2 <<= 1;
    ++levels;
  }
  const float* p = partial + (int64_t)bh * nblk * kD + c;
  for (int i0 = 0; i0 < n2; i0 += 16) {
    float leaf[16];
#pragma unroll
    for (int u = 0; u < 16; ++u) leaf[u] = (i0 + u < nblk) ? p[(int64_t)(i0 + u) * kD] : 0.0f;
#pragma unroll
    for (int u = 0; u < 16; ++u) {
      const int i = i0 + u;
      if (i >= n2) break;
      float x = leaf[u];
      int lvl = 0;
      for (unsigned ii = (unsigned)i; ii & 1u; ii >>= 1) {
        x = stk[lvl][c] + x;
        ++lvl;
      }
      stk[lvl][c] = x;
    }
  }
  mu[(int64_t)bh * kD + c] = __fdiv_rn(stk[levels][c], (float)(n_tokens - kSink));
}

// Codes, scales and sink copy: one block per (tpb 128-token tiles, b*h); 16
// lanes per 256-byte key row (encode_row16), 8 channels (one code byte) per lane,
// 8 rows per thread and tile.  CB: also accumulate the codebook statistics of
// the block's tokens in [64, n_tokens) (§2.1 item 1, one-pass clustering: a
// sub-vector's cluster is its sign pattern): x_c = fl32(fl32(k_c - mu_c) /
// alpha), rint(x_c * 2^24) added as int64 (exact, order-free) to the bin of
// (sub-vector, pattern), and the count of that bin; block totals go to cb_part.
template <bool CB>
__global__ __launch_bounds__(256) void codes_kernel(const uint16_t* __restrict__ k, int64_t sb,
                                                    int64_t sh, int64_t st, int Hkv, int t_begin,
                                                    int t_end, RowMap rm, int tpb,
                                                    const float* __restrict__ mu,
                                                    uint8_t* __restrict__ codes,
                                                    float* __restrict__ alpha,
                                                    uint16_t* __restrict__ k_sink,
                                                    uint8_t* __restrict__ vrec,
                                                    long long* __restrict__ cb_part) {
  __shared__ unsigned long long cbs[CB ? kSub * 16 * 4 : 1];
  __shared__ int cbn[CB ? kSub * 16 : 1];
  // Blocks walk the keys backwards (last head and tile first): right after the
  // mean pass, whose last-read rows are the likeliest to still sit in the
  // memory-side cache.
  const int bh = gridDim.y - 1 - blockIdx.y, b = bh / Hkv, h = bh - b * Hkv;
  const int bx = gridDim.x - 1 - blockIdx.x;
  const int tid = threadIdx.x, cg = tid & 15, rs = tid >> 4;
  if (CB) {
    for (int i = tid; i < kSub * 16 * 4; i += 256) cbs[i] = 0ull;
    for (int i = tid; i < kSub * 16; i += 256) cbn[i] = 0;
    __syncthreads();
  }
  float m[8];
  {
    const float4 m0 = *reinterpret_cast<const float4*>(mu + (int64_t)bh * kD + cg * 8);
    const float4 m1 = *reinterpret_cast<const float4*>(mu + (int64_t)bh * kD + cg * 8 + 4);
    m[0] = m0.x; m[1] = m0.y; m[2] = m0.z; m[3] = m0.w;
    m[4] = m1.x; m[5] = m1.y; m[6] = m1.z; m[7] = m1.w;
  }
  const uint16_t* base = k + (int64_t)b * sb + (int64_t)h * sh + cg * 8;
  const int n_tiles = (t_end - t_begin + 127) / 128;
  const int tile_end = min(n_tiles, (int)(bx + 1) * tpb);
  for (int tile = bx * tpb; tile < tile_end; ++tile) {
    const int tb = t_begin + tile * 128;
    uint4 w[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int t = tb + i * 16 + rs;
      w[i] = (t < t_end) ? *reinterpret_cast<const uint4*>(base + (int64_t)(t - t_begin) * st)
                         : make_uint4(0u, 0u, 0u, 0u);
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int t = tb + i * 16 + rs;
      const RowCode rc = encode_row16(w[i], m);
      if (t < t_end) {
        const int64_t row = rm.row(b, h, t);
        if ((cg & 3) == 0) {
          *reinterpret_cast<uint32_t*>(codes + row * kCodeBytes + cg) = rc.word;
          if (vrec != nullptr)
            *reinterpret_cast<uint32_t*>(vrec + row * kVRecBytes + kVRecCode + cg) = rc.word;
        }
        if (cg == 0) alpha[row] = rc.alpha;
        if (t < kSink)
          *reinterpret_cast<uint4*>(k_sink + ((int64_t)bh * kSink + t) * kD + cg * 8) = w[i];
      }
      if (CB && t >= kSink && t < t_end) {
        const int bin0 = (2 * cg) * 16 + (int)(rc.byte & 15u);
        const int bin1 = (2 * cg + 1) * 16 + (int)(rc.byte >> 4);
#pragma unroll
        for (int c = 0; c < 8; ++c) {
          const float d = chan(w[i], c) - m[c];
          const float x = rc.alpha > 0.0f ? __fdiv_rn(d, rc.alpha) : 0.0f;
          const long long fx = __double2ll_rn((double)x * (double)(1 << kCbFracBits));
          atomicAdd(&cbs[(c < 4 ? bin0 : bin1) * 4 + (c & 3)], (unsigned long long)fx);
        }
        atomicAdd(&cbn[bin0], 1);
        atomicAdd(&cbn[bin1], 1);
      }
    }
  }
  if (CB) {
    __syncthreads();
    long long* out = cb_part + ((int64_t)bh * gridDim.x + bx) * kCbStride;
    for (int i = tid; i < kSub * 16 * 4; i += 256) out[i] = (long long)cbs[i];
    for (int i = tid; i < kSub * 16; i += 256) out[kSub * 16 * 4 + i] = cbn[i];
  }
}

// Value codes: one block per (128-row tile, b*h); 4 lanes per row, each with
// one 32-channel group (quantize_vgroup32), so that a group's scale and
// thresholds are made once per lane and no lane exchanges anything; thread
// (rs, g) takes rows rs and rs + 64 of the tile, all of their loads issued
// first.  Each lane writes its group's 8 code bytes and (scale, zero) word;
// rows below 64 are also kept whole in v_sink.
__global__ __launch_bounds__(256) void vcodes_kernel(const uint16_t* __restrict__ v, int64_t sb,
                                                     int64_t sh, int64_t st, int Hkv, int t_begin,
                                                     int t_end, RowMap rm,
                                                     uint8_t* __restrict__ vrec,
                                                     uint16_t* __restrict__ v_sink) {
  const int bh = blockIdx.y, b = bh / Hkv, h = bh - b * Hkv;
  const int tid = threadIdx.x, g = tid & 3, rs = tid >> 2;
  const int tb = t_begin + blockIdx.x * 128;
  const uint16_t* base = v + (int64_t)b * sb + (int64_t)h * sh + g * 32;
  uint4 w[2][4];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int t = tb + i * 64 + rs;
    const uint4* p = reinterpret_cast<const uint4*>(base + (int64_t)(t - t_begin) * st);
#pragma unroll
    for (int u = 0; u < 4; ++u) w[i][u] = (t < t_end) ? p[u] : make_uint4(0u, 0u, 0u, 0u);
  }
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int t = tb + i * 64 + rs;
    const VGroupCode gc = quantize_vgroup32(w[i]);
    if (t < t_end) {
      uint8_t* rec = vrec + rm.row(b, h, t) * kVRecBytes;
      *reinterpret_cast<uint2*>(rec + 8 * g) = make_uint2(gc.lo, gc.hi);
      *reinterpret_cast<uint32_t*>(rec + kVRecSz + 4 * g) = gc.sz;
      if (t < kSink) {
        uint4* dst = reinterpret_cast<uint4*>(v_sink + ((int64_t)bh * kSink + t) * kD + g * 32);
#pragma unroll
        for (int u = 0; u < 4; ++u) dst[u] = w[i][u];
      }
    }
  }
}

// Codebook, stage 2: one block per b*h, thread (j, p).  Block statistics are
// summed in block order (exact integer sums), then centre_i =
// fl32((sum_i * 2^-24) / count) computed in fp64; empty cluster: sign vertex p.
__global__ __launch_bounds__(512) void cb_final_kernel(const long long* __restrict__ part, int nblk,
                                                       float* __restrict__ codebook, int keep) {
  const int bh = blockIdx.x, jp = threadIdx.x, p = jp & 15;
  long long s[4] = {0, 0, 0, 0}, n = 0;
  for (int bk = 0; bk < nblk; ++bk) {
    const long long* q = part + ((int64_t)bh * nblk + bk) * kCbStride;
#pragma unroll
    for (int i = 0; i < 4; ++i) s[i] += q[jp * 4 + i];
    n += q[kSub * 16 * 4 + jp];
  }
  float4* dst = reinterpret_cast<float4*>(codebook) + (int64_t)bh * kSub * 16 + jp;
  const float4 prev = keep ? *dst : make_float4(0.f, 0.f, 0.f, 0.f);
  const float* pv = &prev.x;
  float4 c;
  float* cv = &c.x;
#pragma unroll
  for (int i = 0; i < 4; ++i)
    cv[i] = n > 0 ? (float)(((double)s[i] * (1.0 / (double)(1 << kCbFracBits))) / (double)n)
                  : (keep ? pv[i] : (((p >> i) & 1) ? -1.0f : 1.0f));
  *dst = c;
}

// K-means baseline, assignment step: the points and block statistics of
// codes_kernel<true>, with the cluster of a sub-vector chosen as its nearest
// centre instead of its sign pattern.  Thread (row group rs, channel group cg)
// holds sub-vectors 2cg and 2cg+1 of its tokens, so it keeps their 2 x 16
// centres in registers.
__global__ __launch_bounds__(256, 2) void kmeans_assign_kernel(
    const uint16_t* __restrict__ k, int64_t sb, int64_t sh, int64_t st, int Hkv, int n_tokens,
    RowMap rm, int tpb, const float* __restrict__ mu, const float* __restrict__ alpha,
    const float* __restrict__ centres, long long* __restrict__ cb_part) {
  __shared__ unsigned long long cbs[kSub * 16 * 4];
  __shared__ int cbn[kSub * 16];
  const int bh = blockIdx.y, b = bh / Hkv, h = bh - b * Hkv;
  const int tid = threadIdx.x, cg = tid & 15, rs = tid >> 4;
  float4 cen[2][16];
#pragma unroll
  for (int half = 0; half < 2; ++half)
#pragma unroll
    for (int p = 0; p < 16; ++p)
      cen[half][p] = centres != nullptr
                         ? reinterpret_cast<const float4*>(centres)[((int64_t)bh * kSub + 2 * cg +
                                                                     half) * 16 + p]
                         : make_float4((p & 1) ? -1.f : 1.f, (p & 2) ? -1.f : 1.f,
                                       (p & 4) ? -1.f : 1.f, (p & 8) ? -1.f : 1.f);
  for (int i = tid; i < kSub * 16; i += 256) cbn[i] = 0;
  for (int i = tid; i < kSub * 16 * 4; i += 256) cbs[i] = 0ull;
  __syncthreads();
  float m[8];
  {
    const float4 m0 = *reinterpret_cast<const float4*>(mu + (int64_t)bh * kD + cg * 8);
    const float4 m1 = *reinterpret_cast<const float4*>(mu + (int64_t)bh * kD + cg * 8 + 4);
    m[0] = m0.x; m[1] = m0.y; m[2] = m0.z; m[3] = m0.w;
    m[4] = m1.x; m[5] = m1.y; m[6] = m1.z; m[7] = m1.w;
  }
  const uint16_t* base = k + (int64_t)b * sb + (int64_t)h * sh + cg * 8;
  const int n_tiles = (n_tokens + 127) / 128;
  const int tile_end = min(n_tiles, (int)(blockIdx.x + 1) * tpb);
  for (int tile = blockIdx.x * tpb; tile < tile_end; ++tile) {
    const int tb = tile * 128;
    uint4 w[8];
    float a[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int t = tb + i * 16 + rs;
      const bool ok = t >= kSink && t < n_tokens;
      w[i] = ok ? *reinterpret_cast<const uint4*>(base + (int64_t)t * st) : make_uint4(0u, 0u, 0u, 0u);
      a[i] = ok ? alpha[rm.row(b, h, t)] : 0.0f;
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int t = tb + i * 16 + rs;
      if (t < kSink || t >= n_tokens) continue;
      float x[8];
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        const float d = chan(w[i], c) - m[c];
        x[c] = a[i] > 0.0f ? __fdiv_rn(d, a[i]) : 0.0f;
      }
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        const int j = 2 * cg + half;
        const float* xs = x + 4 * half;
        int best = 0;
        float bd = 0.0f;
#pragma unroll
        for (int p = 0; p < 16; ++p) {
          const float4 c = cen[half][p];
          const float d0 = xs[0] - c.x, d1 = xs[1] - c.y, d2 = xs[2] - c.z, d3 = xs[3] - c.w;
          const float dist = ((d0 * d0 + d1 * d1) + d2 * d2) + d3 * d3;
          if (p == 0 || dist < bd) {
            bd = dist;
            best = p;
          }
        }
        const int bin = j * 16 + best;
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const long long fx = __double2ll_rn((double)xs[c] * (double)(1 << kCbFracBits));
          atomicAdd(&cbs[bin * 4 + c], (unsigned long long)fx);
        }
        atomicAdd(&cbn[bin], 1);
      }
    }
  }
  __syncthreads();
  long long* out = cb_part + ((int64_t)bh * gridDim.x + blockIdx.x) * kCbStride;
  for (int i = tid; i < kSub * 16 * 4; i += 256) out[i] = (long long)cbs[i];
  for (int i = tid; i < kSub * 16; i += 256) out[kSub * 16 * 4 + i] = cbn[i];
}

}  // namespace

hipError_t launch_mu_partial(const uint16_t* k, int64_t sb, int64_t sh, int64_t st, int B, int Hkv,
                             int n_tokens, float* partial, int nblk, const Launch& s) {
  return launch_k(KID_MU_PARTIAL, mu_partial_kernel, dim3(nblk, B * Hkv), dim3(256), 0, s, k, sb,
                  sh, st, Hkv, n_tokens, partial, nblk);
}

hipError_t launch_mu_final(const float* partial, int BH, int nblk, int n_tokens, float* mu,
                           const Launch& s) {
  return launch_k(KID_MU_FINAL, mu_final_kernel, dim3(BH), dim3(kD), 0, s, partial, nblk,
                  n_tokens, mu);
}

hipError_t launch_codes(const uint16_t* k, int64_t sb, int64_t sh, int64_t st, int B, int Hkv,
                        int t_begin, int t_end, const RowMap& rm, const float* mu, uint8_t* codes,
                        float* alpha, uint16_t* k_sink, uint8_t* vrec, const Launch& s) {
  const int tiles = (t_end - t_begin + 127) / 128;
  return launch_k(KID_CODES, codes_kernel<false>, dim3(tiles, B * Hkv), dim3(256), 0, s, k, sb,
                  sh, st, Hkv, t_begin, t_end, rm, 1, mu, codes, alpha, k_sink, vrec,
                  (long long*)nullptr);
}

hipError_t launch_vcodes(const uint16_t* v, int64_t sb, int64_t sh, int64_t st, int B, int Hkv,
                         int t_begin, int t_end, const RowMap& rm, uint8_t* vrec,
                         uint16_t* v_sink, const Launch& s) {
  const int tiles = (t_end - t_begin + 127) / 128;
  return launch_k(KID_VCODES, vcodes_kernel, dim3(tiles, B * Hkv), dim3(256), 0, s, v, sb, sh, st,
                  Hkv, t_begin, t_end, rm, vrec, v_sink);
}

hipError_t launch_codes_cb(const uint16_t* k, int64_t sb, int64_t sh, int64_t st, int B, int Hkv,
                           int n_tokens, const RowMap& rm, const float* mu, uint8_t* codes,
                           float* alpha, uint16_t* k_sink, uint8_t* vrec, long long* cb_part,
                           const Launch& s) {
  return launch_k(KID_CODES, codes_kernel<true>, dim3(cb_blocks(n_tokens), B * Hkv), dim3(256), 0,
                  s, k, sb, sh, st, Hkv, 0, n_tokens, rm, kCbTiles, mu, codes, alpha, k_sink,
                  vrec, cb_part);
}

hipError_t launch_cb_final(const long long* cb_part, int BH, int nblk, float* codebook,
                           const Launch& s, int keep) {
  return launch_k(KID_CB_FINAL, cb_final_kernel, dim3(BH), dim3(kSub * 16), 0, s, cb_part, nblk,
                  codebook, keep);
}

hipError_t launch_kmeans_assign(const uint16_t* k, int64_t sb, int64_t sh, int64_t st, int B,
                                int Hkv, int n_tokens, const RowMap& rm, const float* mu,
                                const float* alpha, const float* centres, long long* cb_part,
                                const Launch& s) {
  return launch_k(KID_KM_ASSIGN, kmeans_assign_kernel, dim3(cb_blocks(n_tokens), B * Hkv),
                  dim3(256), 0, s, k, sb, sh, st, Hkv, n_tokens, rm, kCbTiles, mu, alpha,
                  centres, cb_part);
}

}  // namespace sikv
