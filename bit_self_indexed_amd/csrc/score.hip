// Compressed-domain retrieval (gfx950): LUT-GEMV scoring and exact top-k.
//
// "Self-Indexing KVCache: Predicting Sparse Attention from Compressed Keys",
// technical summary §2.1 item 2: the query is split like the keys, each piece is
// dotted with the 16 cluster centres to form a look-up table, and every cached
// token is scored by looking up its sub-vector codes and accumulating, without
// decoding the keys; the top-k tokens are then selected.
//
// Three kernels per decode step, all exact:
//   sample  - one block per (b, h): scores a fixed, evenly spaced sample of the
//             candidates and takes a conservative threshold tau below the
//             expected k-th score (the whole candidate set when it is small);
//   score   - the HBM stream: 16-byte code + 4-byte scale per token, one lane per
//             token, table in LDS; tokens with score >= tau are written, in token
//             order, to a per-tile slot (no atomics, no global sort);
//   select  - one block per (b, h): radix select of the exact k-th largest over
//             the candidates, then an ordered compaction (ascending positions,
//             ties to the smaller position).  If fewer than k candidates passed
//             (tau too high), the block rescans the whole head and selects over
//             every token, so the result never depends on the sample.
#include <hip/hip_ext.h>

#include "sikv_internal.h"

namespace sikv {

namespace {

constexpr int kSampleMax = 4096;     // sampled candidates per head
constexpr int kSampleRun = 256;      // contiguous tokens per sample stratum
constexpr int kSelectLds = 12288;    // candidates kept in LDS by select
constexpr int kMaxChunks = 4096;

// ------------------------------------------------------------------ block helpers
// Exclusive prefix sum of one int per thread over the block (blockDim multiple
// of 64, at most 1024).  tmp: LDS, >= 17 ints.  Returns the exclusive sum and
// writes the block total to *total.  Contains barriers.
__device__ __forceinline__ int block_excl_scan(int v, int* tmp, int* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int nw = blockDim.x >> 6;
  int x = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(x, o);
    if (lane >= o) x += y;
  }
  if (lane == 63) tmp[wave] = x;
  __syncthreads();
  if (threadIdx.x == 0) {
    int run = 0;
    for (int w = 0; w < nw; ++w) {
      const int c = tmp[w];
      tmp[w] = run;
      run += c;
    }
    tmp[16] = run;
  }
  __syncthreads();
  const int r = tmp[wave] + x - v;
  *total = tmp[16];
  __syncthreads();
  return r;
}

__device__ __forceinline__ uint32_t wave_min_u32(uint32_t x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x = min(x, (uint32_t)__shfl_xor((int)x, o));
  return x;
}
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x = max(x, (uint32_t)__shfl_xor((int)x, o));
  return x;
}

// Block-wide min and max of per-thread values; tmp: LDS >= 32 uint32.
__device__ __forceinline__ void block_minmax(uint32_t lo, uint32_t hi, uint32_t* tmp,
                                             uint32_t* out_lo, uint32_t* out_hi) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nw = blockDim.x >> 6;
  lo = wave_min_u32(lo);
  hi = wave_max_u32(hi);
  if (lane == 0) {
    tmp[wave] = lo;
    tmp[16 + wave] = hi;
  }
  __syncthreads();
  uint32_t a = 0xffffffffu, c = 0u;
  for (int w = 0; w < nw; ++w) {
    a = min(a, tmp[w]);
    c = max(c, tmp[16 + w]);
  }
  *out_lo = a;
  *out_hi = c;
  __syncthreads();
}

struct Kth {
  uint32_t key;  // value of the k-th largest key
  int above;     // keys strictly larger than it
  int need;      // keys equal to it that belong to the top k (>= 1)
};

// k-th largest of n keys (1 <= k <= n) held at `keys` (LDS or global), all in
// [lo, hi].  Radix select on key - lo, 11-bit digits from the highest bit that
// varies, LDS histograms.  hist: LDS >= 2048 uint32; tmp: LDS >= 20 ints.
__device__ Kth block_kth_largest(const uint32_t* keys, int n, int k, uint32_t lo, uint32_t hi,
                                 uint32_t* hist, int* tmp) {
  const uint32_t span = hi - lo;
  int top = span ? 32 - __clz(span) : 0;
  uint32_t prefix = 0;
  int need = k, above = 0;
  while (top > 0) {
    const int width = top < 11 ? top : 11;
    const int shift = top - width;
    const int nb = 1 << width;
    for (int i = threadIdx.x; i < nb; i += blockDim.x) hist[i] = 0u;
    __syncthreads();
    const uint64_t want = (uint64_t)prefix >> top;
    for (int i = threadIdx.x; i < n; i += blockDim.x) {
      const uint32_t r = keys[i] - lo;
      if (((uint64_t)r >> top) == want) atomicAdd(&hist[(r >> shift) & (uint32_t)(nb - 1)], 1u);
    }
    __syncthreads();
    // Bins of this thread: a contiguous run, scanned in ascending digit order.
    const int per = (nb + blockDim.x - 1) / blockDim.x;
    const int d0 = threadIdx.x * per;
    int cnt = 0;
    for (int d = d0; d < d0 + per && d < nb; ++d) cnt += (int)hist[d];
    int total;
    int pre = block_excl_scan(cnt, tmp, &total);
    // The digit holding the element of ascending rank x = total - need.
    const int x = total - need;
    for (int d = d0; d < d0 + per && d < nb; ++d) {
      const int c = (int)hist[d];
      if (pre <= x && x < pre + c) {
        tmp[18] = d;
        tmp[19] = total - (pre + c);  // elements in larger digits
      }
      pre += c;
    }
    __syncthreads();
    const int dsel = tmp[18];
    above += tmp[19];
    need -= tmp[19];
    prefix |= (uint32_t)dsel << shift;
    top = shift;
    __syncthreads();
  }
  return Kth{lo + prefix, above, need};
}

// Writes the selected positions of keys[0..n) (in list order, which is ascending
// position) to out: every key > kth, and the first `need` keys == kth.
__device__ void block_emit_selected(const uint32_t* keys, const int32_t* pos, int n, int k, Kth r,
                                    int32_t* __restrict__ out, int* tmp) {
  int run_gt = 0, run_eq = 0;
  for (int base = 0; base < n; base += blockDim.x) {
    const int i = base + threadIdx.x;
    int gt = 0, eq = 0;
    if (i < n) {
      const uint32_t kk = keys[i];
      gt = kk > r.key;
      eq = kk == r.key;
    }
    int total;
    const int ex = block_excl_scan((gt << 16) | eq, tmp, &total);
    const int gt_before = run_gt + (ex >> 16);
    const int eq_before = run_eq + (ex & 0xffff);
    const int p = gt_before + min(eq_before, r.need);
    if ((gt || (eq && eq_before < r.need)) && p < k) out[p] = pos[i];
    run_gt += total >> 16;
    run_eq += total & 0xffff;
  }
}

// ------------------------------------------------------------------ sample
__global__ __launch_bounds__(1024) void sample_kernel(const uint16_t* __restrict__ q, int n_q_heads,
                                                      int Hkv, int G, const uint8_t* __restrict__ codes,
                                                      const float* __restrict__ alpha, int capacity,
                                                      int n_tokens, int rank, int force_exact,
                                                      float* __restrict__ tau) {
  __shared__ float qbar[kD];
  __shared__ float lut[kLut];
  __shared__ uint32_t keys[kSampleMax];
  __shared__ uint32_t hist[2048];
  __shared__ int tmp[32];
  __shared__ uint32_t mm[32];
  const int bh = blockIdx.x, b = bh / Hkv, h = bh - b * Hkv;
  if (force_exact) {
    if (threadIdx.x == 0) tau[bh] = __uint_as_float(0x7f800000u);  // +inf: nothing passes
    return;
  }
  const int n = n_tokens - kSink;
  const bool full = n <= kSampleMax;
  const int m = full ? n : kSampleMax;
  if (!full && rank > m) {  // threshold would sit below every sample: keep all
    if (threadIdx.x == 0) tau[bh] = __uint_as_float(0xff800000u);
    return;
  }
  build_selection_lut(q, b, h, n_q_heads, G, qbar, lut);
  const int64_t row0 = (int64_t)bh * capacity;
  uint32_t lo = 0xffffffffu, hi = 0u;
  for (int i = threadIdx.x; i < m; i += blockDim.x) {
    int t;
    if (full) {
      t = kSink + i;
    } else {
      const int sidx = i / kSampleRun;
      const int start = (int)(((int64_t)sidx * (n - kSampleRun)) / (kSampleMax / kSampleRun - 1));
      t = kSink + start + (i - sidx * kSampleRun);
    }
    const uint4 c = *reinterpret_cast<const uint4*>(codes + (row0 + t) * kCodeBytes);
    const uint32_t key = score_key(selection_score(lut, c, alpha[row0 + t]));
    keys[i] = key;
    lo = min(lo, key);
    hi = max(hi, key);
  }
  block_minmax(lo, hi, mm, &lo, &hi);
  const Kth kt = block_kth_largest(keys, m, rank, lo, hi, hist, tmp);
  if (threadIdx.x == 0) tau[bh] = key_score(kt.key);
}

// ------------------------------------------------------------------ score
// One block per (tile of 256*U candidates, b*h); lane <-> token.  All code and
// scale loads of the tile are issued before the table is built.
template <int U>
__global__ __launch_bounds__(256) void score_kernel(
    const uint16_t* __restrict__ q, int n_q_heads, int Hkv, int G, const uint8_t* __restrict__ codes,
    const float* __restrict__ alpha, int capacity, int n_tokens, const float* __restrict__ tau,
    int n_chunks, uint32_t* __restrict__ cand_key, int32_t* __restrict__ cand_t,
    int32_t* __restrict__ chunk_count, float* __restrict__ scores_opt) {
  __shared__ float qbar[kD];
  __shared__ float lut[kLut];
  __shared__ int wcnt[U][4];
  constexpr int kChunk = 256 * U;
  const int bh = blockIdx.y, b = bh / Hkv, h = bh - b * Hkv;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int t0 = kSink + blockIdx.x * kChunk;
  const int64_t row0 = (int64_t)bh * capacity;
  uint4 c[U];
  float a[U];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int t = t0 + u * 256 + tid;
    if (t < n_tokens) {
      c[u] = *reinterpret_cast<const uint4*>(codes + (row0 + t) * kCodeBytes);
      a[u] = alpha[row0 + t];
    } else {
      c[u] = make_uint4(0u, 0u, 0u, 0u);
      a[u] = 0.0f;
    }
  }
  build_selection_lut(q, b, h, n_q_heads, G, qbar, lut);
  const float th = tau[bh];
  uint64_t mask[U];
  uint32_t key[U];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int t = t0 + u * 256 + tid;
    const float s = selection_score(lut, c[u], a[u]);
    const bool valid = t < n_tokens;
    if (scores_opt != nullptr && valid) scores_opt[row0 + t] = s;
    key[u] = score_key(s);
    mask[u] = __ballot(valid && s >= th);
    if (lane == 0) wcnt[u][wave] = __popcll(mask[u]);
  }
  __syncthreads();
  int run = 0;
  const int64_t slot = ((int64_t)bh * n_chunks + blockIdx.x) * kChunk;
#pragma unroll
  for (int u = 0; u < U; ++u) {
    int off = run;
    for (int w = 0; w < 4; ++w) {
      const int cw = wcnt[u][w];
      if (w < wave) off += cw;
      run += cw;
    }
    if ((mask[u] >> lane) & 1ull) {
      const int p = off + ballot_rank(mask[u]);
      cand_key[slot + p] = key[u];
      cand_t[slot + p] = t0 + u * 256 + tid;
    }
  }
  if (tid == 0) chunk_count[(int64_t)bh * n_chunks + blockIdx.x] = run;
}

// ------------------------------------------------------------------ select
__global__ __launch_bounds__(1024) void select_kernel(
    const uint16_t* __restrict__ q, int n_q_heads, int Hkv, int G, const uint8_t* __restrict__ codes,
    const float* __restrict__ alpha, int capacity, int n_tokens, int top_k, int chunk, int n_chunks,
    const uint32_t* __restrict__ cand_key, const int32_t* __restrict__ cand_t,
    const int32_t* __restrict__ chunk_count, uint32_t* __restrict__ comp_key,
    int32_t* __restrict__ comp_t, int32_t* __restrict__ idx) {
  __shared__ int off[kMaxChunks + 1];
  __shared__ uint32_t hist[2048];
  __shared__ uint32_t lkey[kSelectLds];
  __shared__ int32_t lpos[kSelectLds];
  __shared__ float qbar[kD];
  __shared__ float lut[kLut];
  __shared__ int tmp[32];
  __shared__ uint32_t mm[32];
  const int bh = blockIdx.x, b = bh / Hkv, h = bh - b * Hkv;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, nw = blockDim.x >> 6;
  const int n = n_tokens - kSink;
  int32_t* out = idx + (int64_t)bh * top_k;
  if (top_k >= n) {  // every candidate is kept
    for (int j = tid; j < top_k; j += blockDim.x) out[j] = kSink + j;
    return;
  }
  // Tile counts -> offsets of each tile's candidates in the ordered list.
  {
    const int per = (n_chunks + blockDim.x - 1) / blockDim.x;
    const int c0 = tid * per;
    int s = 0;
    for (int ci = c0; ci < c0 + per && ci < n_chunks; ++ci)
      s += chunk_count[(int64_t)bh * n_chunks + ci];
    int total;
    int pre = block_excl_scan(s, tmp, &total);
    for (int ci = c0; ci < c0 + per && ci < n_chunks; ++ci) {
      off[ci] = pre;
      pre += chunk_count[(int64_t)bh * n_chunks + ci];
    }
    if (tid == 0) off[n_chunks] = total;
    __syncthreads();
  }
  int C = off[n_chunks];
  const int64_t cbase = (int64_t)bh * n_chunks * chunk;
  const uint32_t* keys;
  const int32_t* pos;
  uint32_t lo = 0xffffffffu, hi = 0u;
  if (C < top_k) {
    // Exact path over the whole head: rescore every candidate, in order.
    build_selection_lut(q, b, h, n_q_heads, G, qbar, lut);
    const int64_t row0 = (int64_t)bh * capacity;
    for (int i = tid; i < n; i += blockDim.x) {
      const int t = kSink + i;
      const uint4 c = *reinterpret_cast<const uint4*>(codes + (row0 + t) * kCodeBytes);
      const uint32_t key = score_key(selection_score(lut, c, alpha[row0 + t]));
      comp_key[cbase + i] = key;
      comp_t[cbase + i] = t;
      lo = min(lo, key);
      hi = max(hi, key);
    }
    C = n;
    keys = comp_key + cbase;
    pos = comp_t + cbase;
  } else {
    const bool in_lds = C <= kSelectLds;
    uint32_t* dk = in_lds ? lkey : comp_key + cbase;
    int32_t* dp = in_lds ? lpos : comp_t + cbase;
    for (int ci = wave; ci < n_chunks; ci += nw) {
      const int o = off[ci], cnt = off[ci + 1] - o;
      const int64_t src = cbase + (int64_t)ci * chunk;
      for (int j = lane; j < cnt; j += 64) {
        const uint32_t key = cand_key[src + j];
        dk[o + j] = key;
        dp[o + j] = cand_t[src + j];
        lo = min(lo, key);
        hi = max(hi, key);
      }
    }
    keys = dk;
    pos = dp;
  }
  block_minmax(lo, hi, mm, &lo, &hi);  // its barriers also publish the copies
  const Kth r = block_kth_largest(keys, C, top_k, lo, hi, hist, tmp);
  block_emit_selected(keys, pos, C, top_k, r, out, tmp);
}

}  // namespace

// rank: how many of the sampled scores lie at or above tau.  For a small head the
// whole candidate set is the sample and rank = k (tau is then the exact k-th
// score).  Otherwise the expected rank of the k-th score in the sample plus five
// standard deviations and a small floor, so that fewer than k tokens pass only
// with negligible probability; the select kernel handles that case exactly anyway.
hipError_t launch_sample(const uint16_t* q, int n_q_heads, int B, int Hkv, const uint8_t* codes,
                         const float* alpha, int capacity, int n_tokens, int top_k, int force_exact,
                         float* tau, hipStream_t s) {
  const int n = n_tokens - kSink;
  int rank;
  if (n <= kSampleMax) {
    rank = top_k;
  } else {
    const double e = (double)top_k * kSampleMax / (double)n;
    double r = e + 5.0 * __builtin_sqrt(e) + 8.0;
    rank = r > kSampleMax ? kSampleMax + 1 : (int)r + 1;
  }
  return launch_k(KID_SAMPLE, sample_kernel, dim3(B * Hkv), dim3(1024), 0, s, q, n_q_heads, Hkv,
                  n_q_heads / Hkv, codes, alpha, capacity, n_tokens, rank, force_exact, tau);
}

hipError_t launch_score(const uint16_t* q, int n_q_heads, int B, int Hkv, const uint8_t* codes,
                        const float* alpha, int capacity, int n_tokens, const float* tau,
                        int chunk, int n_chunks, uint32_t* cand_key, int32_t* cand_t,
                        int32_t* chunk_count, float* scores_opt, hipStream_t s) {
  const dim3 grid(n_chunks, B * Hkv), block(256);
  const int G = n_q_heads / Hkv;
#define SIKV_SCORE_CASE(UU)                                                                     \
  case 256 * UU:                                                                                \
    return launch_k(KID_SCORE, score_kernel<UU>, grid, block, 0, s, q, n_q_heads, Hkv, G, codes, \
                    alpha, capacity, n_tokens, tau, n_chunks, cand_key, cand_t, chunk_count,    \
                    scores_opt);
  switch (chunk) {
    SIKV_SCORE_CASE(1)
    SIKV_SCORE_CASE(2)
    SIKV_SCORE_CASE(4)
    SIKV_SCORE_CASE(8)
    SIKV_SCORE_CASE(16)
    default:
      return hipErrorInvalidValue;
  }
#undef SIKV_SCORE_CASE
}

hipError_t launch_select(const uint16_t* q, int n_q_heads, int B, int Hkv, const uint8_t* codes,
                         const float* alpha, int capacity, int n_tokens, int top_k, int chunk,
                         int n_chunks, uint32_t* cand_key, int32_t* cand_t,
                         const int32_t* chunk_count, uint32_t* comp_key, int32_t* comp_t,
                         int32_t* idx, hipStream_t s) {
  if (n_chunks > kMaxChunks) return hipErrorInvalidValue;
  return launch_k(KID_SELECT, select_kernel, dim3(B * Hkv), dim3(1024), 0, s, q, n_q_heads, Hkv,
                  n_q_heads / Hkv, codes, alpha, capacity, n_tokens, top_k, chunk, n_chunks,
                  cand_key, cand_t, chunk_count, comp_key, comp_t, idx);
}

}  // namespace sikv
