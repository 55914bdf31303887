// Compressed-domain retrieval (gfx950): LUT-GEMV scoring and exact top-k.
//
// "Self-Indexing KVCache: Predicting Sparse Attention from Compressed Keys",
// technical summary §2.1 item 2: the query is split like the keys, each piece is
// dotted with the 16 cluster centres to form a look-up table, and every cached
// token is scored by looking up its sub-vector codes and accumulating, without
// decoding the keys; the top-k tokens are then selected.
//
// Three kernels per decode step, all exact:
//   prep    - one block per (b, h): builds the selection query's table (the
//             16-entry table of each 4-dim sub-vector, in int32 fixed point so
//             that a token's 32 look-ups are summed exactly with 3-input integer
//             adds), the attention tables of the G query heads, their q.mu and
//             the exact logits of the 64 sinks; then scores a stratified sample
//             of 3072 candidates (16 contiguous tokens from the middle of each of
//             192 equal segments) and takes a conservative threshold tau below
//             the expected k-th score (the whole candidate set when it is small);
//   score   - the HBM stream: 16-byte code + 4-byte scale per token, one lane per
//             token, one wave per tile with its loads a step ahead of its
//             look-ups, 2 KB table in LDS (16-entry look-ups never conflict in
//             the LDS banks); tokens with score >= tau are written, in token
//             order, to a per-tile slot (no atomics);
//   select  - one block per (b, h): radix select of the exact k-th largest over
//             the candidates, then an ordered compaction (ascending positions,
//             ties to the smaller position).  If fewer than k candidates passed
//             (tau too high), the block rescans the whole head and selects over
//             every token, so the result never depends on the sample.
#include <hip/hip_ext.h>

#include <type_traits>

#include "sikv_internal.h"

namespace sikv {

namespace {

constexpr int kSampleMax = 3072;   // sampled candidates per head
constexpr int kSampleRun = 16;     // contiguous tokens per stratum (192 strata)
constexpr int kSelectLds = 16384;  // candidates kept in LDS by select
constexpr int kMaxChunks = 2048;
constexpr int kSubMax = 1024;

// ------------------------------------------------------------------ block helpers
// Exclusive prefix sum of one int per thread over the block (blockDim a multiple
// of 64, at most 1024).  tmp: LDS, >= 16 ints.  Returns the exclusive sum and the
// block total.  Two barriers.
__device__ __forceinline__ int block_excl_scan(int v, int* tmp, int* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int nw = blockDim.x >> 6;
  const int x = wave_incl_scan(v);
  if (lane == 63) tmp[wave] = x;
  __syncthreads();
  const int t = lane < nw ? tmp[lane] : 0;  // wave totals in lanes 0..nw-1 (row 0)
  const int ts = wave_incl_scan(t);
  const int wbase = __builtin_amdgcn_readlane(ts, wave) - __builtin_amdgcn_readlane(t, wave);
  *total = __builtin_amdgcn_readlane(ts, nw - 1);
  __syncthreads();  // tmp may be reused as soon as this returns
  return wbase + x - v;
}

__device__ __forceinline__ uint32_t wave_min_u32(uint32_t x) {
  const int r = row_allreduce((int)x, [](int a, int b) { return (int)min((uint32_t)a, (uint32_t)b); });
  const uint32_t a = (uint32_t)__builtin_amdgcn_readlane(r, 0), b = (uint32_t)__builtin_amdgcn_readlane(r, 16);
  const uint32_t c = (uint32_t)__builtin_amdgcn_readlane(r, 32), d = (uint32_t)__builtin_amdgcn_readlane(r, 48);
  return min(min(a, b), min(c, d));
}
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t x) {
  const int r = row_allreduce((int)x, [](int a, int b) { return (int)max((uint32_t)a, (uint32_t)b); });
  const uint32_t a = (uint32_t)__builtin_amdgcn_readlane(r, 0), b = (uint32_t)__builtin_amdgcn_readlane(r, 16);
  const uint32_t c = (uint32_t)__builtin_amdgcn_readlane(r, 32), d = (uint32_t)__builtin_amdgcn_readlane(r, 48);
  return max(max(a, b), max(c, d));
}

// Block-wide min and max of per-thread values; tmp: LDS >= 32 uint32.
__device__ __forceinline__ void block_minmax(uint32_t lo, uint32_t hi, uint32_t* tmp,
                                             uint32_t* out_lo, uint32_t* out_hi,
                                             bool reuse = true) {
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
  if (reuse) __syncthreads();  // before tmp is written again
}

struct Kth {
  uint32_t key;  // value of the k-th largest key
  int above;     // keys strictly larger than it
  int need;      // keys equal to it that belong to the top k (>= 1)
};

// One radix round: among the keys whose bits of (key - lo) above `top` equal
// those of `prefix`, histogram the next digit (<= 11 bits, ending at `shift`)
// and find the digit holding the k-th largest of them.  hist: LDS >= 2048;
// tmp: LDS >= 24 ints.  Returns (digit, count in larger digits, count in it).
struct Round {
  int digit, above, count, shift;
};

// Given a histogram of nb bins (in LDS, published) over keys in ascending bin
// order, the bin holding the k-th largest key: (bin, keys in larger bins, keys
// in it).  tmp: LDS >= 24 ints.  Five barriers.
__device__ __forceinline__ Round hist_pick(const uint32_t* hist, int nb, int k, int* tmp,
                                           int top_fill = -1);

__device__ __forceinline__ Round block_round(const uint32_t* keys, int n, int k, uint32_t lo,
                                             int top, uint32_t prefix, uint32_t* hist, int* tmp) {
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
  Round r = hist_pick(hist, nb, k, tmp);
  r.shift = shift;
  return r;
}

// top_fill >= 0: the top bin (nb - 1) was not counted; its count is top_fill
// minus the other bins' total.
__device__ __forceinline__ Round hist_pick(const uint32_t* hist, int nb, int k, int* tmp,
                                           int top_fill) {
  const int per = (nb + blockDim.x - 1) / blockDim.x;
  const int d0 = threadIdx.x * per;
  const bool implicit_top = top_fill >= 0;
  int cnt = 0;
  for (int d = d0; d < d0 + per && d < nb; ++d)
    cnt += (implicit_top && d == nb - 1) ? 0 : (int)hist[d];
  int total;
  int pre = block_excl_scan(cnt, tmp, &total);
  const int top_count = implicit_top ? top_fill - total : 0;
  if (implicit_top) total = top_fill;
  const int x = total - k;  // ascending rank of the k-th largest among the matched
  for (int d = d0; d < d0 + per && d < nb; ++d) {
    const int c = (implicit_top && d == nb - 1) ? top_count : (int)hist[d];
    if (pre <= x && x < pre + c) {
      tmp[18] = d;
      tmp[19] = total - (pre + c);
      tmp[20] = c;
    }
    pre += c;
  }
  __syncthreads();
  const Round r{tmp[18], tmp[19], tmp[20], 0};
  __syncthreads();
  return r;
}

// need-th largest (1 <= need <= m <= 64) of the keys sub[0..m) by wave 0 alone:
// lane l holds key l and counts the keys above and equal to it, reading the
// others one by one from lane registers (v_readlane, no LDS round trips); the
// lanes with gt < need <= gt + eq hold the answer.  Result in out[0] (key),
// out[1] (number of keys greater than it).  Caller provides the barrier.
__device__ __forceinline__ void wave_kth(const uint32_t* sub, int m, int need, int* out) {
  if (threadIdx.x >= 64) return;
  const int lane = threadIdx.x;
  const uint32_t x = lane < m ? sub[lane] : 0u;
  int gt = 0, eq = 0;
  for (int i = 0; i < m; ++i) {
    const uint32_t y = (uint32_t)__builtin_amdgcn_readlane((int)x, i);
    gt += y > x ? 1 : 0;
    eq += y == x ? 1 : 0;
  }
  const uint64_t hit = __ballot(lane < m && gt < need && need <= gt + eq);
  const int l = (int)__builtin_ctzll(hit);  // hit != 0: the need-th largest exists
  const int key = __builtin_amdgcn_readlane((int)x, l), above = __builtin_amdgcn_readlane(gt, l);
  if (lane == 0) {
    out[0] = key;
    out[1] = above;
  }
}

// Exact k-th largest of n keys in [lo, hi] (1 <= k <= n).  The first round runs
// over all keys; the keys of its boundary digit (usually few) are then copied to
// `sub` (LDS) and resolved by one wave when they are at most 64, else by more
// rounds over them only.
__device__ Kth block_kth(const uint32_t* keys, int n, int k, uint32_t lo, uint32_t hi,
                         uint32_t* hist, int* tmp, uint32_t* sub, int* scount) {
  const uint32_t span = hi - lo;
  int top = span ? 32 - __clz(span) : 0;
  uint32_t prefix = 0;
  int need = k, above = 0;
  const uint32_t* src = keys;
  int ns = n;
  bool first = true;
  while (top > 0) {
    const Round r = block_round(src, ns, need, lo, top, prefix, hist, tmp);
    above += r.above;
    need -= r.above;
    prefix |= (uint32_t)r.digit << r.shift;
    top = r.shift;
    if (first && top > 0 && r.count <= kSubMax) {
      if (threadIdx.x == 0) *scount = 0;
      __syncthreads();
      const uint64_t want = (uint64_t)prefix >> top;
      for (int i = threadIdx.x; i < ns; i += blockDim.x) {
        const uint32_t key = src[i];
        if (((uint64_t)(key - lo) >> top) == want) sub[atomicAdd(scount, 1)] = key;
      }
      __syncthreads();
      src = sub;
      ns = r.count;
      if (ns <= 64) {
        wave_kth(sub, ns, need, tmp + 24);
        __syncthreads();
        const uint32_t key = (uint32_t)tmp[24];
        const int gt = tmp[25];
        __syncthreads();
        return Kth{key, above + gt, need - gt};
      }
    }
    first = false;
  }
  return Kth{lo + prefix, above, need};
}

// Writes the positions of the selected keys (all keys > kth, then the first
// `need` keys == kth in list order) to out, in list order (= ascending
// position).  Each thread owns a contiguous run of the list.
__device__ void block_emit(const uint32_t* keys, const int32_t* pos, int n, int k, Kth r,
                           int32_t* __restrict__ out, int* tmp) {
  const int per = (n + blockDim.x - 1) / blockDim.x;
  const int i0 = threadIdx.x * per, i1 = min(n, i0 + per);
  int gt = 0, eq = 0;
  for (int i = i0; i < i1; ++i) {
    const uint32_t kk = keys[i];
    gt += kk > r.key;
    eq += kk == r.key;
  }
  int gt_before, eq_before;
  if (n < 65536) {
    int tot;
    const int ex = block_excl_scan((gt << 16) | eq, tmp, &tot);
    gt_before = ex >> 16;
    eq_before = ex & 0xffff;
  } else {
    int tg, te;
    gt_before = block_excl_scan(gt, tmp, &tg);
    eq_before = block_excl_scan(eq, tmp, &te);
  }
  int o = gt_before + min(eq_before, r.need);
  for (int i = i0; i < i1; ++i) {
    const uint32_t kk = keys[i];
    bool take = kk > r.key;
    if (kk == r.key) take = eq_before++ < r.need;
    if (take && o < k) out[o++] = pos[i];
  }
}

// The select kernel's LDS list (n <= kSelectLds entries) cut into one run per
// thread, held in registers: an odd run length, so that the runs' strided LDS
// reads never share a bank.
constexpr int kEmitRun = 17;  // longest run: odd and >= kSelectLds / 1024
static_assert(kEmitRun >= ((kSelectLds / 1024) | 1), "runs of a 1024-thread block");
struct Run {
  uint32_t key[kEmitRun];
  int32_t pos[kEmitRun];
  int per, i0, n;
  __device__ __forceinline__ bool valid(int j) const { return j < per && i0 + j < n; }
};

// Loads the runs (blockDim.x = 1024).  No barrier.
__device__ __forceinline__ void run_load(Run& rn, const uint32_t* keys, const int32_t* pos, int n) {
  rn.per = ((n + blockDim.x - 1) / blockDim.x) | 1;
  rn.i0 = threadIdx.x * rn.per;
  rn.n = n;
#pragma unroll
  for (int j = 0; j < kEmitRun; ++j) {
    rn.key[j] = rn.valid(j) ? keys[rn.i0 + j] : 0u;
    rn.pos[j] = rn.valid(j) ? pos[rn.i0 + j] : 0;
  }
}

// block_emit over the runs, with coalesced output: the (gt, eq) counts are
// scanned, every thread writes its taken positions into the key list (stage;
// the caller no longer needs it), and the block copies them out in order,
// consecutive threads storing consecutive entries.  Two barriers beyond the
// scan.
__device__ void run_emit(const Run& rn, int k, Kth r, uint32_t* stage, int32_t* __restrict__ out,
                         int* tmp) {
  int gt = 0, eq = 0;
#pragma unroll
  for (int j = 0; j < kEmitRun; ++j) {
    gt += (rn.valid(j) && rn.key[j] > r.key) ? 1 : 0;
    eq += (rn.valid(j) && rn.key[j] == r.key) ? 1 : 0;
  }
  int tot;
  const int ex = block_excl_scan((gt << 16) | eq, tmp, &tot);  // n <= kSelectLds < 2^16
  int eq_before = ex & 0xffff;
  int o = (ex >> 16) + min(eq_before, r.need);
  __syncthreads();  // no thread reads the list any more
#pragma unroll
  for (int j = 0; j < kEmitRun; ++j) {
    bool take = rn.valid(j) && rn.key[j] > r.key;
    if (rn.valid(j) && rn.key[j] == r.key) take = eq_before++ < r.need;
    if (take && o < k) stage[o++] = (uint32_t)rn.pos[j];
  }
  __syncthreads();
  for (int j = threadIdx.x; j < k; j += blockDim.x) out[j] = (int32_t)stage[j];
}

// Copies the selection table of one head from global memory into LDS (2 KB).
// No barrier.
__device__ __forceinline__ void load_itab(const int* __restrict__ gtab, int* itab) {
  const int4* src = reinterpret_cast<const int4*>(gtab);
  int4* dst = reinterpret_cast<int4*>(itab);
  for (int i = threadIdx.x; i < kLut / 4; i += blockDim.x) dst[i] = src[i];
}

// Two bounds from one 2048-bin equal-width histogram of the n scores sc, all in
// [smin, smax]: *lo at or below the k_lo-th largest (the lower edge of its bin,
// lowered by one more bin so that rounding cannot lift it above), and *hi at or
// above the k_hi-th largest (the upper edge of its bin, raised by one more bin;
// smax if k_hi < 1).  1 <= k_lo <= n.  hist: LDS, 2048 counters already zero
// (and published); tmp: LDS >= 24 ints, which hold the two bins on return (no
// barrier after their last read: the caller does not reuse tmp or hist).
__device__ void block_score_band(const float* sc, int n, int k_lo, int k_hi, float smin,
                                 float smax, uint32_t* hist, int* tmp, float* lo, float* hi) {
  if (!(smax > smin)) {
    *lo = smin;
    *hi = smax;
    return;
  }
  constexpr int kBins = 2048;
  const float w = (smax - smin) * (1.0f / kBins);
  const float inv = (float)kBins / (smax - smin);
  for (int i = threadIdx.x; i < n; i += blockDim.x) {
    const int d = min(max((int)((sc[i] - smin) * inv), 0), kBins - 1);
    atomicAdd(&hist[d], 1u);
  }
  __syncthreads();
  const int per = (kBins + blockDim.x - 1) / blockDim.x;
  const int d0 = threadIdx.x * per;
  int cnt = 0;
  for (int d = d0; d < d0 + per && d < kBins; ++d) cnt += (int)hist[d];
  if (threadIdx.x == 0) tmp[21] = kBins - 1;  // published by the scan's barriers
  int total;
  int pre = block_excl_scan(cnt, tmp, &total);  // uses tmp[0..15]
  const int x_lo = total - k_lo;  // ascending ranks of the k-th largest
  const int x_hi = total - k_hi;
  for (int d = d0; d < d0 + per && d < kBins; ++d) {
    const int c = (int)hist[d];
    if (pre <= x_lo && x_lo < pre + c) tmp[18] = d;
    if (k_hi >= 1 && pre <= x_hi && x_hi < pre + c) tmp[21] = d;
    pre += c;
  }
  __syncthreads();
  const int dl = tmp[18], dh = tmp[21];
  *lo = smin + (float)(dl - 1) * w;
  *hi = k_hi >= 1 ? fminf(smax, smin + (float)(dh + 2) * w) : smax;
}

// rank: how many of the sampled scores lie at or above tau.  For a small head the
// whole candidate set (n <= 3072) is the sample and rank = k (tau is then at most
// the exact k-th score).  Otherwise the expected rank e = k * 3072 / n of the k-th
// score in the sample plus five standard deviations and a small floor, so that
// fewer than k tokens pass only with negligible probability (the select kernel
// handles that case exactly anyway).  rank_hi: the rank of the upper end of the
// select kernel's score bins, e - 5 sqrt(e) - 8 (the k-th score lies below it
// with high probability), or the top of the sample if that is below 1.
__device__ __forceinline__ void sample_ranks(int k, int n, int* rank, int* rank_hi) {
  if (n <= kSampleMax) {
    *rank = k;
    *rank_hi = k;
    return;
  }
  const double e = (double)k * kSampleMax / (double)n;
  const double r = e + 5.0 * sqrt(e) + 8.0;
  *rank = r > kSampleMax ? kSampleMax + 1 : (int)r + 1;
  const double rh = e - 5.0 * sqrt(e) - 8.0;
  *rank_hi = rh < 1.0 ? 0 : (int)rh;
}

// ------------------------------------------------------------------ prep
// mode 0: attention tables only (sel_lut, sel_inv and tau unused); 1: all tables
// + sampled threshold; 2: all tables + tau = +inf (forces the exact whole-head
// selection).  k_new != null: first encode the key of token n_tokens-1 (append);
// the sample then leaves that token out.  Every global load is issued before
// the first barrier.
__global__ __launch_bounds__(1024) void prep_kernel(
    const uint16_t* __restrict__ q, int n_q_heads, int Hkv, int G, const float* __restrict__ mu,
    uint8_t* __restrict__ codes, float* __restrict__ alpha, RowMap rm, int n_tokens,
    const uint16_t* __restrict__ k_sink, const uint16_t* __restrict__ k_new, int64_t ksb,
    int64_t ksh, const uint16_t* __restrict__ v_new, int64_t vnsb, int64_t vnsh,
    uint8_t* __restrict__ vrec,
    const float* __restrict__ codebook, int top_k, int mode, const int32_t* __restrict__ seq_lens,
    int* __restrict__ sel_lut, float* __restrict__ sel_inv, float* __restrict__ att_lut,
    float* __restrict__ att_qmu, float* __restrict__ att_slog, float* __restrict__ tau,
    float* __restrict__ bin_scale) {
  __shared__ float qv[kMaxGroup + 1][kD];  // q_g, then the selection query (sum)
  __shared__ float mus[kD];
  __shared__ int itab[kLut];
  __shared__ float red_a[2];
  __shared__ float4 cbl[kLut];             // codebook centres of this KV head, if any
  __shared__ float jmax[kSub];
  __shared__ float ssc[kSampleMax];
  __shared__ uint32_t hist[2048];
  __shared__ int tmp[32];
  __shared__ uint32_t mm[32];
  const int bh = blockIdx.x, b = bh / Hkv, h = bh - b * Hkv;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int nt = seq_len(seq_lens, b, n_tokens);                   // this sequence's length
  const int n = nt - kSink - (k_new != nullptr ? 1 : 0);  // candidates the sample covers
  int rank = 1, rank_hi = 0;
  if (mode == 1) sample_ranks(seq_topk(top_k, nt), n, &rank, &rank_hi);
  const bool full = n <= kSampleMax;
  const int m = full ? n : kSampleMax;
  const bool sample = mode == 1 && m > 0 && rank <= m;
  const int64_t hq0 = (int64_t)b * n_q_heads + (int64_t)h * G;
  const bool has_cb = codebook != nullptr;
  const float4 cbv = (has_cb && tid < kLut)
                         ? reinterpret_cast<const float4*>(codebook)[(int64_t)bh * kLut + tid]
                         : make_float4(0.f, 0.f, 0.f, 0.f);

  for (int i = tid; i < 2048; i += blockDim.x) hist[i] = 0u;  // the band's counters

  // Appended value row (quantised values): 16 lanes of wave 1, 8 channels each.
  uint4 vw = make_uint4(0u, 0u, 0u, 0u);
  if (v_new != nullptr && tid >= 64 && tid < 80)
    vw = *reinterpret_cast<const uint4*>(v_new + (int64_t)b * vnsb + (int64_t)h * vnsh +
                                         (tid - 64) * 8);
  // Appended key row: 16 lanes x 8 channels, with the matching means.
  uint4 kw = make_uint4(0u, 0u, 0u, 0u);
  float km[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  if (k_new != nullptr && tid < 16) {
    kw = *reinterpret_cast<const uint4*>(k_new + (int64_t)b * ksb + (int64_t)h * ksh + tid * 8);
    const float4 m0 = *reinterpret_cast<const float4*>(mu + (int64_t)bh * kD + tid * 8);
    const float4 m1 = *reinterpret_cast<const float4*>(mu + (int64_t)bh * kD + tid * 8 + 4);
    km[0] = m0.x; km[1] = m0.y; km[2] = m0.z; km[3] = m0.w;
    km[4] = m1.x; km[5] = m1.y; km[6] = m1.z; km[7] = m1.w;
  }

  // The query, mean and sink rows are loaded first: the tables need only them
  // and are built while the sample's loads are still in flight (loads complete
  // in order, so a wait for q never waits for the sample).
  const uint4 ks = *reinterpret_cast<const uint4*>(k_sink + ((int64_t)bh * kSink + (tid >> 4)) * kD +
                                                   (tid & 15) * 8);
  // (unconditional loads at clamped indices: a load in a branch whose value is
  // used inside it would wait there for every load issued before it)
  const uint16_t qraw = q[hq0 * kD + min(tid, G * kD - 1)];
  const float mraw = mu[(int64_t)bh * kD + min(tid, kD - 1)];

  // Sample rows: stratum st = i / 16 of 192 equal segments, 16 tokens centred in
  // it (the whole candidate set when small).  Every lane loads a real row (token
  // 64 for unused slots, never scored), so the wait counts do not depend on
  // which lanes sample; page ids, if paged, are all loaded before any code.
  constexpr int kPer = kSampleMax / 1024;
  int st_t[kPer];
  bool use[kPer];
#pragma unroll
  for (int u = 0; u < kPer; ++u) {
    const int i = tid + u * 1024;
    use[u] = sample && i < m;
    int t = kSink + i;
    if (!full) {
      const int st = i / kSampleRun, ns = kSampleMax / kSampleRun;
      const int64_t seg0 = (int64_t)st * n / ns, seg1 = (int64_t)(st + 1) * n / ns;
      t = kSink + (int)(seg0 + (seg1 - seg0 - kSampleRun) / 2) + (i - st * kSampleRun);
    }
    st_t[u] = use[u] ? t : kSink;
  }
  int64_t rows[kPer];
  if (rm.table != nullptr) {
    int32_t pg[kPer];
#pragma unroll
    for (int u = 0; u < kPer; ++u) pg[u] = rm.table[(int64_t)b * rm.pps + (st_t[u] >> rm.lg_page)];
#pragma unroll
    for (int u = 0; u < kPer; ++u)
      rows[u] = (((int64_t)pg[u] * Hkv + h) << rm.lg_page) |
                (int64_t)(st_t[u] & ((1 << rm.lg_page) - 1));
  } else {
#pragma unroll
    for (int u = 0; u < kPer; ++u) rows[u] = ((int64_t)b * Hkv + h) * rm.capacity + st_t[u];
  }
  uint4 c[kPer];
  float a[kPer];
#pragma unroll
  for (int u = 0; u < kPer; ++u) {
    c[u] = *reinterpret_cast<const uint4*>(codes + rows[u] * kCodeBytes);
    a[u] = alpha[rows[u]];
  }
  if (tid < G * kD) qv[tid / kD][tid % kD] = __uint_as_float((uint32_t)qraw << 16);
  if (tid < kD) mus[tid] = mraw;
  if (has_cb && tid < kLut) cbl[tid] = cbv;
  if (k_new != nullptr && wave == 0) {  // the whole wave runs the 16-lane shuffles
    const RowCode rc = encode_row16(kw, km);
    const int64_t row = rm.row(b, h, nt - 1);
    if (tid < 16 && (tid & 3) == 0) {
      *reinterpret_cast<uint32_t*>(codes + row * kCodeBytes + tid) = rc.word;
      if (vrec != nullptr)
        *reinterpret_cast<uint32_t*>(vrec + row * kVRecBytes + kVRecCode + tid) = rc.word;
    }
    if (tid == 0) alpha[row] = rc.alpha;
  }
  if (v_new != nullptr && wave == 1) {  // the whole wave runs the 4-lane shuffles
    const VRowCode rc = quantize_vrow16(vw);
    const uint32_t pair = rc.bits | (__shfl_down(rc.bits, 1, 16) << 16);
    const int cg = lane;
    uint8_t* rec = vrec + rm.row(b, h, nt - 1) * kVRecBytes;
    if (cg < 16 && (cg & 1) == 0) *reinterpret_cast<uint32_t*>(rec + 2 * cg) = pair;
    if (cg < 16 && (cg & 3) == 0) *reinterpret_cast<uint32_t*>(rec + kVRecSz + cg) = rc.sz;
  }
  __syncthreads();

  // Selection query (fp32 sum, g ascending) and sum |qbar|; q_g . mu; attention
  // tables of the G query heads.
  if (tid < kD) {
    float s = qv[0][tid];
    for (int g = 1; g < G; ++g) s += qv[g][tid];
    qv[kMaxGroup][tid] = s;
    const float v = wave_sum(fabsf(s));
    if (lane == 0) red_a[wave] = v;
  } else if (wave >= 2 && wave < 2 + G) {
    const int g = wave - 2;
    const float d = wave_sum(fmaf(qv[g][lane], mus[lane], qv[g][lane + 64] * mus[lane + 64]));
    if (lane == 0) att_qmu[hq0 + g] = d;
  }
  for (int i = tid; i < G * kLut; i += blockDim.x)
    att_lut[hq0 * kLut + i] = has_cb ? cb_lut_entry(qv[i / kLut], cbl, i % kLut)
                                     : lut_entry(qv[i / kLut], i % kLut);
  // Exact logits of the sinks (full-precision keys): q_g . k_sink[r], fp32.
  {
    const int r = tid >> 4, c0 = (tid & 15) * 8;
    const float x[8] = {bf16lo(ks.x), bf16hi(ks.x), bf16lo(ks.y), bf16hi(ks.y),
                        bf16lo(ks.z), bf16hi(ks.z), bf16lo(ks.w), bf16hi(ks.w)};
    for (int g = 0; g < G; ++g) {
      float d = 0.0f;
#pragma unroll
      for (int i = 0; i < 8; ++i) d = fmaf(qv[g][c0 + i], x[i], d);
      d = row_allreduce(d, [](float a, float b) { return a + b; });  // the row's 16 lanes
      if ((tid & 15) == 0) att_slog[(hq0 + g) * kSink + r] = d;
    }
  }
  if (mode == 0) return;
  __syncthreads();

  // Selection table in fixed point.  A bounds |sum_j LUT[j][p_j]|: sum_c |qbar_c|
  // for the sign vertices, sum_j max_p |LUT[j][p]| for a codebook.  With
  // A = m * 2^x (m in [0.5, 1)) the scale is 2^(30 - x), so any sum of 32
  // entries stays below 2^30 in magnitude.
  const float lv = tid < kLut ? (has_cb ? cb_lut_entry(qv[kMaxGroup], cbl, tid)
                                        : lut_entry(qv[kMaxGroup], tid))
                              : 0.0f;
  float A;
  if (has_cb) {
    const float x = row_allreduce(fabsf(lv), [](float a, float b) { return fmaxf(a, b); });
    if (tid < kLut && (tid & 15) == 0) jmax[tid >> 4] = x;
    __syncthreads();
    A = 0.0f;
    for (int j = 0; j < kSub; ++j) A += jmax[j];
  } else {
    A = red_a[0] + red_a[1];
  }
  int ex = 0;
  if (A > 0.0f) {
    frexpf(A, &ex);
    ex = 30 - ex;
  }
  const float inv = ldexpf(1.0f, -ex);
  if (tid < kLut) {
    const int v = (int)rintf(ldexpf(lv, ex));
    itab[tid] = v;
    sel_lut[(int64_t)bh * kLut + tid] = v;
  }
  if (tid == 0) sel_inv[bh] = inv;
  if (mode == 2 || !sample) {  // +inf: nothing passes; -inf: keep all
    if (tid == 0) {
      tau[bh] = __uint_as_float(mode == 2 ? 0x7f800000u : 0xff800000u);
      bin_scale[bh] = 0.0f;
    }
    return;
  }
  __syncthreads();
  uint32_t lo = 0xffffffffu, hi = 0u;
#pragma unroll
  for (int u = 0; u < kPer; ++u) {
    const int i = tid + u * 1024;
    if (i < m) {
      const float sv = selection_score(itab, inv, c[u], a[u]);
      ssc[i] = sv;
      lo = min(lo, score_key(sv));
      hi = max(hi, score_key(sv));
    }
  }
  block_minmax(lo, hi, mm, &lo, &hi, false);  // its barrier also publishes ssc; mm is not reused
  float th, th_hi;
  block_score_band(ssc, m, rank, rank_hi, key_score(lo), key_score(hi), hist, tmp, &th, &th_hi);
  if (tid == 0) {
    tau[bh] = th;
    // the select kernel bins candidate scores linearly, 2048 bins from tau up
    // to an upper estimate of the k-th score (higher scores share the top bin)
    const float span = th_hi - th;
    bin_scale[bh] = span > 0.0f ? 2048.0f / span : 0.0f;
  }
}

// ------------------------------------------------------------------ score
// One block per tile of 256*U candidates (lane <-> token); wave w scores the
// tile's w-th quarter, U groups of 64 tokens, on its own, and the four waves
// meet once more only to place their candidates.  Small enough (<= 64 VGPRs
// at U = 8) for eight waves per SIMD, so that a 2048-tile grid is resident at
// once.  Each wave issues all its loads before the table barrier; they are
// unconditional, at token indices clamped to the sequence's last token
// (always a valid row), so the compiler counts the loads in flight exactly
// and each group waits only for its own data.  Rows are 32-bit lane offsets
// from a wave-uniform base row: a 64-token group lies within one page of a
// paged cache (groups start at multiples of 64, pages at multiples of
// >= 256), so one page id serves the group.  Candidates (score >= tau) are
// written in token order after the last load.
template <int U, bool kPaged, int S = (U < 8 ? U : 8)>
__global__ __launch_bounds__(256) void score_kernel(
    const uint8_t* __restrict__ codes, const float* __restrict__ alpha, RowMap rm,
    int n_tokens, int Hkv, const int32_t* __restrict__ seq_lens,
    const int* __restrict__ sel_lut, const float* __restrict__ sel_inv,
    const float* __restrict__ tau, int n_chunks, uint32_t* __restrict__ cand_key,
    int32_t* __restrict__ cand_t, int32_t* __restrict__ chunk_count,
    float* __restrict__ scores_opt) {
  constexpr int kChunk = 256 * U;
  constexpr int NS = U / S;  // steps of S groups, all loaded before the table barrier
  static_assert(U % S == 0 && NS <= 2, "tile shape");
  __shared__ int itab[kLut];
  __shared__ int wcnt[4];
  const int bh = blockIdx.y, b = bh / Hkv, h = bh - b * Hkv;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: rows from scalar bases
  const int nt = seq_len(seq_lens, b, n_tokens);
  const int t0 = kSink + blockIdx.x * kChunk;  // the tile's first token
  const int tw = t0 + wave * (64 * U);         // this wave's first token
  const int lim = nt - tw;  // tokens of this wave's quarter in the sequence (<= 0: none)
  const int2 tv = reinterpret_cast<const int2*>(sel_lut + (int64_t)bh * kLut)[tid];
  const int64_t hrow = (int64_t)bh * rm.capacity;  // contiguous: the head's first row
  // Paged: the quarter's tokens (clamped to the sequence) span at most U + 1
  // pages; lane j holds the id of the j-th, read out per group with a lane read
  // (a per-group load would wait behind every code load in flight).
  const int lg = rm.lg_page;
  const int pfirst = min(tw, nt - 1) >> lg;
  int pv = 0;
  if constexpr (kPaged)
    pv = rm.table[(int64_t)b * rm.pps + min(pfirst + lane, (nt - 1) >> lg)];
  // Loads of step st.
  uint4 c[NS][S];
  float a[NS][S];
  auto load_step = [&](int st) {
#pragma unroll
    for (int u = 0; u < S; ++u) {
      const int g0 = tw + (st * S + u) * 64;  // first token of the group
      const int gb = min(g0, nt - 1);         // base row's token (uniform)
      const uint32_t o = (uint32_t)(min(g0 + lane, nt - 1) - gb);
      int64_t r0;
      if constexpr (kPaged) {
        const int64_t pg = __builtin_amdgcn_readlane(pv, (gb >> lg) - pfirst);
        r0 = ((pg * Hkv + h) << lg) | (int64_t)(gb & ((1 << lg) - 1));
      } else {
        r0 = hrow + gb;
      }
      c[st][u] = *reinterpret_cast<const uint4*>(
          reinterpret_cast<const char*>(codes + r0 * kCodeBytes) + (o << 4));
      a[st][u] = *reinterpret_cast<const float*>(
          reinterpret_cast<const char*>(alpha + r0) + (o << 2));
    }
  };
  load_step(0);
  if constexpr (NS > 1) load_step(1);
  int tz;
  asm volatile("v_mov_b32 %0, 0" : "=v"(tz));  // the table is stored after the loads go out
  reinterpret_cast<int2*>(itab)[tid] = make_int2(tv.x ^ tz, tv.y ^ tz);
  const float inv = sel_inv[bh];
  const float th = tau[bh];
  __syncthreads();
  uint32_t key[U];
  uint32_t bits = 0;  // bit g: token g*64 + lane of the quarter passed
  // gate: a zero from an asm placed after the table barrier (then after the
  // previous step's sums); the step's codes and scales are read through it, so
  // their decode stays behind it, in order: without it the compiler hoists
  // most look-ups into one batch (85 VGPRs, fewer waves per SIMD).
  auto score_step = [&](int st, int gate) {
#pragma unroll
    for (int u = 0; u < S; ++u) {
      const int g = st * S + u;
      uint4 cg = c[st][u];
      cg.x ^= gate, cg.y ^= gate, cg.z ^= gate, cg.w ^= gate;
      const float ag = __int_as_float(__float_as_int(a[st][u]) ^ gate);
      const float sv = selection_score(itab, inv, cg, ag);
      key[g] = score_key(sv);
      if (g * 64 + lane < lim && sv >= th) bits |= 1u << g;
    }
  };
  int gate;
  asm volatile("v_mov_b32 %0, 0" : "=v"(gate));
#pragma unroll
  for (int st = 0; st < NS; ++st) {
    score_step(st, gate);
    // after this step's sums (so that the next step's look-ups are not issued
    // before them, nor this step's sums moved past the count exchange)
    asm volatile("v_mov_b32 %0, 0" : "=v"(gate) : "v"(bits));
  }
  int cnt = 0;
#pragma unroll
  for (int g = 0; g < U; ++g) cnt += __popcll(__ballot((bits >> g) & 1u));
  if (lane == 0) wcnt[wave] = cnt;
  __syncthreads();
  int run = 0;  // candidates of the waves before this one
#pragma unroll
  for (int w = 0; w < 3; ++w) run += w < wave ? wcnt[w] : 0;
  const int64_t slot = ((int64_t)bh * n_chunks + blockIdx.x) * kChunk;
  uint32_t* __restrict__ kout = cand_key + slot;
  int32_t* __restrict__ tout = cand_t + slot;
#pragma unroll
  for (int g = 0; g < U; ++g) {
    const bool pass = (bits >> g) & 1u;
    const uint64_t m = __ballot(pass);
    if (pass) {
      const int p = run + ballot_rank(m);
      kout[p] = key[g];
      tout[p] = tw + g * 64 + lane;
    }
    run += __popcll(m);
  }
  if (scores_opt != nullptr) {  // key_score inverts score_key exactly
    float* __restrict__ so = scores_opt + hrow + tw;
#pragma unroll
    for (int g = 0; g < U; ++g)
      if (g * 64 + lane < lim) so[g * 64 + lane] = key_score(key[g]);
  }
  if (tid == 255) chunk_count[(int64_t)bh * n_chunks + blockIdx.x] = run;  // the last wave's run ends the tile
}

// Histogram count of one key per lane (valid lanes only).  Keys above the band
// all land in the top bin, which is not counted here (its count is the list
// length minus the other bins', taken by hist_pick): one LDS atomic each on one
// address would serialise.
__device__ __forceinline__ void count_bin(uint32_t* hist, bool valid, int bin) {
  if (valid && bin != 2047) atomicAdd(&hist[bin], 1u);
}

// ------------------------------------------------------------------ select
// The select kernel's rare paths, kept out of line: inlined, their live values
// pushed the common path past the SGPR budget (54 spilled SGPRs, reloaded by
// lane reads; out of line, 42 around the calls, and the select kernel went from
// 14.26 to 13.63 us at long_128k).

// Fewer than k candidates passed: rescore the whole head with the score
// kernel's table and arithmetic, in order, and select over all of it.
__device__ __noinline__ void select_exact_head(
    const uint8_t* __restrict__ codes, const float* __restrict__ alpha, RowMap rm, int Hkv,
    int bh, int n, int top_k, const int* __restrict__ sel_lut, const float* __restrict__ sel_inv,
    uint32_t* __restrict__ comp_key, int32_t* __restrict__ comp_t, int* itab, uint32_t* hist,
    int* tmp, uint32_t* sub, int* scount, uint32_t* mm, int32_t* __restrict__ out) {
  const int tid = threadIdx.x;
  load_itab(sel_lut + (int64_t)bh * kLut, itab);
  const float inv = sel_inv[bh];
  __syncthreads();
  const int b = bh / Hkv, h = bh - b * Hkv;
  uint32_t lo = 0xffffffffu, hi = 0u;
  for (int i = tid; i < n; i += blockDim.x) {
    const int t = kSink + i;
    const int64_t r = rm.row(b, h, t);
    const uint4 c = *reinterpret_cast<const uint4*>(codes + r * kCodeBytes);
    const uint32_t key = score_key(selection_score(itab, inv, c, alpha[r]));
    comp_key[i] = key;
    comp_t[i] = t;
    lo = min(lo, key);
    hi = max(hi, key);
  }
  block_minmax(lo, hi, mm, &lo, &hi);
  const Kth r = block_kth(comp_key, n, top_k, lo, hi, hist, tmp, sub, scount);
  block_emit(comp_key, comp_t, n, top_k, r, out, tmp);
}

// More candidates than the LDS list holds: the ordered list goes to the
// workspace (tile by tile, wave w taking tiles w, w + 16, ...) and radix rounds
// select over it.
__device__ __noinline__ void select_workspace(
    const uint32_t* __restrict__ cand_key, const int32_t* __restrict__ cand_t, int chunk,
    int n_chunks, const int* off, int C, int top_k, uint32_t* __restrict__ comp_key,
    int32_t* __restrict__ comp_t, uint32_t* hist, int* tmp, uint32_t* sub, int* scount,
    uint32_t* mm, int32_t* __restrict__ out) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nw = blockDim.x >> 6;
  uint32_t lo = 0xffffffffu, hi = 0u;
  for (int ci = wave; ci < n_chunks; ci += nw) {
    const int o = off[ci], cnt = off[ci + 1] - o;
    const int64_t src = (int64_t)ci * chunk;
    for (int j = lane; j < cnt; j += 64) {
      const uint32_t key = cand_key[src + j];
      comp_key[o + j] = key;
      comp_t[o + j] = cand_t[src + j];
      lo = min(lo, key);
      hi = max(hi, key);
    }
  }
  block_minmax(lo, hi, mm, &lo, &hi);  // its barriers also publish the copies
  const Kth r = block_kth(comp_key, C, top_k, lo, hi, hist, tmp, sub, scount);
  block_emit(comp_key, comp_t, C, top_k, r, out, tmp);
}

// The k-th's bin holds too many keys (e.g. no usable bin scale): radix rounds
// over the whole LDS list.
__device__ __noinline__ Kth select_degenerate(const uint32_t* lkey, int C, int top_k,
                                              uint32_t* hist, int* tmp, uint32_t* sub,
                                              int* scount, uint32_t* mm) {
  uint32_t lo = 0xffffffffu, hi = 0u;
  for (int i = threadIdx.x; i < C; i += blockDim.x) {
    lo = min(lo, lkey[i]);
    hi = max(hi, lkey[i]);
  }
  block_minmax(lo, hi, mm, &lo, &hi);
  return block_kth(lkey, C, top_k, lo, hi, hist, tmp, sub, scount);
}

__global__ __launch_bounds__(1024) void select_kernel(
    const uint8_t* __restrict__ codes, const float* __restrict__ alpha, RowMap rm,
    int n_tokens, int Hkv, const int32_t* __restrict__ seq_lens,
    const int* __restrict__ sel_lut, const float* __restrict__ sel_inv, int top_k_max,
    int chunk, int n_chunks,
    const uint32_t* __restrict__ cand_key, const int32_t* __restrict__ cand_t,
    const int32_t* __restrict__ chunk_count, const float* __restrict__ tau,
    const float* __restrict__ bin_scale, uint32_t* __restrict__ comp_key,
    int32_t* __restrict__ comp_t, int32_t* __restrict__ idx) {
  __shared__ int off[kMaxChunks + 1];
  __shared__ uint32_t hist[2048];
  __shared__ uint32_t lkey[kSelectLds];
  __shared__ int32_t lpos[kSelectLds];
  __shared__ uint32_t sub[2 * kSubMax];  // boundary-bin keys, then block_kth's own sub-list
  __shared__ int tmp[32];
  __shared__ uint32_t mm[32];
  __shared__ int scount;
  const int bh = blockIdx.x;
  const int tid = threadIdx.x;
  const int nt = seq_len(seq_lens, bh / Hkv, n_tokens);
  const int n = nt - kSink;
  const int top_k = seq_topk(top_k_max, nt);  // this sequence's k; the rest of its row is -1
  int32_t* out = idx + (int64_t)bh * top_k_max;
  for (int j = top_k + tid; j < top_k_max; j += blockDim.x) out[j] = -1;
  if (top_k >= n) {  // every candidate is kept
    for (int j = tid; j < top_k; j += blockDim.x) out[j] = kSink + j;
    return;
  }
  for (int i = tid; i < 2048; i += blockDim.x) hist[i] = 0u;  // published by the scan's barriers
  // Tile counts -> offsets of each tile's candidates in the ordered list.  The
  // counts are loaded first, then the first 256 slots of each wave's first four
  // tiles, which stay in flight while the counts are scanned (loads complete in
  // order; all of them unconditional at clamped indices, so that no wait sits
  // inside a branch).  A tile's slot region holds chunk >= 256 entries, so every
  // slot load is in bounds; slots past a tile's count are discarded.
  const int64_t cbase = (int64_t)bh * n_chunks * chunk;
  uint32_t pk[4][4];
  int32_t pt[4][4];
  {
    const int per = (n_chunks + blockDim.x - 1) / blockDim.x;  // <= 2
    const int c0 = tid * per;
    int cs[2];
#pragma unroll
    for (int j = 0; j < 2; ++j)
      cs[j] = chunk_count[(int64_t)bh * n_chunks + min(c0 + j, n_chunks - 1)];
    {
      const int lane = tid & 63, wave = tid >> 6, nw = blockDim.x >> 6;
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int64_t src = cbase + (int64_t)min(wave + v * nw, n_chunks - 1) * chunk;
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          pk[v][u] = cand_key[src + lane + 64 * u];
          pt[v][u] = cand_t[src + lane + 64 * u];
        }
      }
    }
#pragma unroll
    for (int j = 0; j < 2; ++j)
      if (!(j < per && c0 + j < n_chunks)) cs[j] = 0;
    int total;
    int pre = block_excl_scan(cs[0] + cs[1], tmp, &total);
#pragma unroll
    for (int j = 0; j < 2; ++j)
      if (j < per && c0 + j < n_chunks) {
        off[c0 + j] = pre;
        pre += cs[j];
      }
    if (tid == 0) off[n_chunks] = total;
    __syncthreads();
  }
  const int C = off[n_chunks];
  uint32_t lo = 0xffffffffu, hi = 0u;
  if (C < top_k) {  // the LDS list is unused: it holds the table
    select_exact_head(codes, alpha, rm, Hkv, bh, n, top_k, sel_lut, sel_inv, comp_key + cbase,
                      comp_t + cbase, reinterpret_cast<int*>(lkey), hist, tmp, sub, &scount, mm,
                      out);
    return;
  }
  // Gather the candidates into one ordered list.  Wave w copies tiles w, w+nw,
  // ...; the first 256 candidates of 4 tiles are loaded before any is stored.
  // Kept in LDS, each candidate's score is also counted in a 2048-bin linear
  // histogram from tau up (bin width set by the prep kernel from its sample).
  const bool in_lds = C <= kSelectLds;
  const float th = tau[bh], bsc = bin_scale[bh];
  auto bin_of = [th, bsc](uint32_t key) {
    const float z = (key_score(key) - th) * bsc;  // NaN (no scale) -> bin 0
    return z >= 2047.0f ? 2047 : (z > 0.0f ? (int)z : 0);
  };
  // Two instances, so that the LDS list is written with LDS stores (a pointer
  // that may address either memory would make every store a flat one, which
  // waits on both memory counters).
  auto gather = [&](auto lds_tag) {
    constexpr bool kLds = decltype(lds_tag)::value;
    uint32_t* __restrict__ dk = kLds ? lkey : comp_key + cbase;
    int32_t* __restrict__ dp = kLds ? lpos : comp_t + cbase;
    const int lane = tid & 63, wave = tid >> 6, nw = blockDim.x >> 6;
    for (int c0 = wave; c0 < n_chunks; c0 += 4 * nw) {
      uint32_t kk[4][4];
      int32_t tt[4][4];
      if (c0 == wave) {
#pragma unroll
        for (int v = 0; v < 4; ++v)
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            kk[v][u] = pk[v][u];
            tt[v][u] = pt[v][u];
          }
      } else {
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const int ci = c0 + v * nw;
          const int o = ci < n_chunks ? off[ci] : 0;
          const int cnt = ci < n_chunks ? off[ci + 1] - o : 0;
          const int64_t src = cbase + (int64_t)ci * chunk;
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            const int j = lane + 64 * u;
            kk[v][u] = j < cnt ? cand_key[src + j] : 0u;
            tt[v][u] = j < cnt ? cand_t[src + j] : 0;
          }
        }
      }
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int ci = c0 + v * nw;
        if (ci >= n_chunks) continue;
        const int o = off[ci], cnt = off[ci + 1] - o;
        const int64_t src = cbase + (int64_t)ci * chunk;
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int j = lane + 64 * u;
          if (j < cnt) {
            dk[o + j] = kk[v][u];
            dp[o + j] = tt[v][u];
            if constexpr (!kLds) {  // the LDS list takes its range only when needed
              lo = min(lo, kk[v][u]);
              hi = max(hi, kk[v][u]);
            }
          }
          if constexpr (kLds) count_bin(hist, j < cnt, bin_of(kk[v][u]));
        }
        for (int j0 = 256; j0 < cnt; j0 += 64) {  // tiles with many candidates
          const int j = j0 + lane;
          const uint32_t key = j < cnt ? cand_key[src + j] : 0u;
          if (j < cnt) {
            dk[o + j] = key;
            dp[o + j] = cand_t[src + j];
            if constexpr (!kLds) {
              lo = min(lo, key);
              hi = max(hi, key);
            }
          }
          if constexpr (kLds) count_bin(hist, j < cnt, bin_of(key));
        }
      }
    }
  };
  if (!in_lds) {
    select_workspace(cand_key + cbase, cand_t + cbase, chunk, n_chunks, off, C, top_k,
                     comp_key + cbase, comp_t + cbase, hist, tmp, sub, &scount, mm, out);
    return;
  }
  gather(std::true_type{});
  if (in_lds) {
    __syncthreads();  // publishes the list and the histogram
    // Each thread's run of the list goes to registers while the histogram is
    // scanned for the boundary bin of the k-th largest; the bin's keys (usually
    // a few dozen) go to a sub-list resolved by one wave, or by radix rounds if
    // more than 64.
    Run rn;
    run_load(rn, lkey, lpos, C);
    const Round rb = hist_pick(hist, 2048, top_k, tmp, C);
    Kth r;
    if (rb.count <= kSubMax) {
      // The keys of the k-th's bin d form one interval [klo, khi] (bin_of never
      // decreases as the key grows; patterns above +inf are taken as the top
      // bin), so that the pass below compares keys instead of recomputing every
      // bin.  Wave 0 finds the first key of a bin >= d, wave 1 of a bin >= d+1:
      // 64 keys around the key of tau + e / bin_scale, or, if the boundary is
      // not among them, 6 bits a round from the top.
      if (tid < 128) {
        const int lane = tid & 63, d = rb.digit;
        const int e = tid < 64 ? d : d + 1;
        auto below = [&](uint32_t k) {  // bin of k < e
          return (k > 0xff800000u ? 2047 : bin_of(k)) < e;
        };
        uint32_t first = 0u;  // e == 0: every key
        if (e > 2047) {
          first = 0xffffffffu;  // none: khi ends at the last key
        } else if (e > 0) {
          const uint32_t x0 = score_key(th + (float)e / bsc);
          const uint32_t base = min(max(x0, 32u), 0xffffffffu - 63u) - 32u;
          const int t = __popcll(__ballot(below(base + (uint32_t)lane)));
          if (t > 0 && t < 64) {
            first = base + (uint32_t)t;
          } else {
            uint32_t a = 0u;  // the last key below e (key 0 is: bin 0 < e)
#pragma unroll
            for (int r = 0; r < 6; ++r) {
              const int sh = r < 5 ? 26 - 6 * r : 0;  // bits 31..26, ..., 7..2, then 1..0
              const bool ok = (r < 5 || lane < 4) && below(a | ((uint32_t)lane << sh));
              a |= (uint32_t)(__popcll(__ballot(ok)) - 1) << sh;
            }
            first = a + 1u;
          }
        }
        if (lane == 0) mm[tid >> 6] = tid < 64 ? first : (e > 2047 ? first : first - 1u);
      }
      if (tid == 0) scount = 0;
      __syncthreads();
      const uint32_t klo = mm[0], khi = mm[1];
#pragma unroll
      for (int j = 0; j < kEmitRun; ++j)
        if (rn.valid(j) && rn.key[j] >= klo && rn.key[j] <= khi)
          sub[atomicAdd(&scount, 1)] = rn.key[j];
      __syncthreads();
      const int ns = scount, need = top_k - rb.above;
      if (ns <= 64) {
        wave_kth(sub, ns, need, tmp + 24);
        __syncthreads();
        r = Kth{(uint32_t)tmp[24], rb.above + tmp[25], need - tmp[25]};
        __syncthreads();
      } else {
        uint32_t slo = 0xffffffffu, shi = 0u;
        for (int i = tid; i < ns; i += blockDim.x) {
          slo = min(slo, sub[i]);
          shi = max(shi, sub[i]);
        }
        block_minmax(slo, shi, mm, &slo, &shi);
        const Kth rs = block_kth(sub, ns, need, slo, shi, hist, tmp, sub + kSubMax, &scount);
        r = Kth{rs.key, rb.above + rs.above, rs.need};
      }
    } else {  // degenerate spread (e.g. no usable bin scale): radix over the whole list
      r = select_degenerate(lkey, C, top_k, hist, tmp, sub, &scount, mm);
    }
    run_emit(rn, top_k, r, lkey, out, tmp);
  }
}

}  // namespace

hipError_t launch_prep(const uint16_t* q, int n_q_heads, int B, int Hkv, const float* mu,
                       uint8_t* codes, float* alpha, const RowMap& rm, int n_tokens,
                       const uint16_t* k_sink, const uint16_t* k_new, int64_t ksb, int64_t ksh,
                       const uint16_t* v_new, int64_t vnsb, int64_t vnsh, uint8_t* vrec,
                       const float* codebook, int top_k, int mode, int* sel_lut,
                       float* sel_inv, float* att_lut, float* att_qmu, float* att_slog,
                       float* tau, float* bin_scale, const int32_t* seq_lens, const Launch& s) {
  return launch_k(KID_PREP, prep_kernel, dim3(B * Hkv), dim3(1024), 0, s, q, n_q_heads, Hkv,
                  n_q_heads / Hkv, mu, codes, alpha, rm, n_tokens, k_sink, k_new, ksb, ksh,
                  v_new, vnsb, vnsh, vrec, codebook, top_k, mode, seq_lens, sel_lut, sel_inv,
                  att_lut, att_qmu, att_slog, tau, bin_scale);
}

hipError_t launch_score(int B, int Hkv, const uint8_t* codes, const float* alpha, const RowMap& rm,
                        int n_tokens, const int32_t* seq_lens, const int* sel_lut,
                        const float* sel_inv, const float* tau, int chunk,
                        int n_chunks, uint32_t* cand_key, int32_t* cand_t, int32_t* chunk_count,
                        float* scores_opt, const Launch& s) {
  const dim3 grid(n_chunks, B * Hkv), block(256);
#define SIKV_SCORE_CASE(UU)                                                                    \
  case 256 * UU:                                                                               \
    return rm.table != nullptr                                                                 \
               ? launch_k(KID_SCORE, score_kernel<UU, true>, grid, block, 0, s, codes, alpha,  \
                          rm, n_tokens, Hkv, seq_lens, sel_lut, sel_inv, tau, n_chunks,        \
                          cand_key, cand_t, chunk_count, scores_opt)                           \
               : launch_k(KID_SCORE, score_kernel<UU, false>, grid, block, 0, s, codes, alpha, \
                          rm, n_tokens, Hkv, seq_lens, sel_lut, sel_inv, tau, n_chunks,        \
                          cand_key, cand_t, chunk_count, scores_opt);
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

hipError_t launch_select(int B, int Hkv, const uint8_t* codes, const float* alpha, const RowMap& rm,
                         int n_tokens, const int32_t* seq_lens, const int* sel_lut,
                         const float* sel_inv, int top_k, int chunk, int n_chunks,
                         uint32_t* cand_key, int32_t* cand_t, const int32_t* chunk_count,
                         const float* tau, const float* bin_scale, uint32_t* comp_key,
                         int32_t* comp_t, int32_t* idx, const Launch& s) {
  if (n_chunks > kMaxChunks) return hipErrorInvalidValue;
  return launch_k(KID_SELECT, select_kernel, dim3(B * Hkv), dim3(1024), 0, s, codes, alpha,
                  rm, n_tokens, Hkv, seq_lens, sel_lut, sel_inv, top_k, chunk, n_chunks,
                  cand_key, cand_t,
                  chunk_count, tau, bin_scale, comp_key, comp_t, idx);
}

}  // namespace sikv
