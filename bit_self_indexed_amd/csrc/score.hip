// Compressed-domain retrieval (gfx950): LUT-GEMV scoring and exact top-k.
//
// "Self-Indexing KVCache: Predicting Sparse Attention from Compressed Keys",
// technical summary §2.1 item 2: the query is split like the keys, each piece is
// dotted with the 16 cluster centres to form a look-up table, and every cached
// token is scored by looking up its sub-vector codes and accumulating, without
// decoding the keys; the top-k tokens are then selected.
//
// Two kernels per decode step, all exact:
//   score   - leader blocks, one per (b, h), first in the grid: build the
//             selection query's table (the 16-entry table of each 4-dim
//             sub-vector, in int32 fixed point so that a token's 32 look-ups
//             are summed exactly with 3-input integer adds), score a stratified
//             sample of 2048 candidates (16 contiguous tokens from the middle of
//             each of 128 equal segments) and publish a conservative threshold
//             tau below the expected k-th score through a tagged word (the
//             whole candidate set when it is small); then each scores its head's
//             last tile.  Tile blocks: the HBM stream, 16-byte code + 4-byte
//             scale per token, one lane per token, the same table built in LDS
//             while the loads are in flight (16-entry look-ups never conflict in
//             the LDS banks); tokens with score >= tau are written, in token
//             order, to a per-tile slot (no atomics) with the tau used;
//   select  - up to four blocks per (b, h) (as many as one block per CU
//             allows), which all check the tiles' thresholds and find the
//             exact k-th largest over the candidates; each then writes its
//             part of the ordered compaction (ascending positions, ties to
//             the smaller position).
//             If fewer than k candidates passed (tau too high), a tile kept its
//             tokens with another threshold, or the k-th is below tau, the block
//             rescans the whole head and selects over every token, so the result
//             never depends on the sample or on timing.  Extra blocks of the
//             same launch build the attention tables (the G query heads'
//             look-up tables, q.mu, the exact logits of the 64 sinks).
#include <hip/hip_ext.h>


#include "sikv_internal.h"

namespace sikv {

namespace {

constexpr int kSampleMax = 2048;   // sampled candidates per head
constexpr int kSampleRun = 16;     // contiguous tokens per stratum (128 strata)
constexpr int kBandBins = 1024;    // equal-width bins of the sample's band
constexpr int kSelectLds = 20480;  // candidates kept in LDS by select (keys + 16-bit offsets)
constexpr int kMaxChunks = 2048;
constexpr int kSubMax = 1024;
constexpr int kSelectBlocks = 256;  // select grid target: one 1024-thread block per CU
constexpr int kGatherRun = 10;  // select: candidates a thread loads together past the first tiles

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

// block_excl_scan and the block-wide OR of one flag per thread, in the same two
// barriers.  tmp: LDS, >= 32 ints.  (__syncthreads_or reads the block's y and z
// sizes with a vector load and waits for every load in flight before it.)
__device__ __forceinline__ int block_excl_scan_or(int v, bool f, int* tmp, int* total, bool* any) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int nw = blockDim.x >> 6;
  const int x = wave_incl_scan(v);
  const bool wf = __ballot(f) != 0ull;
  if (lane == 63) {
    tmp[wave] = x;
    tmp[16 + wave] = wf ? 1 : 0;
  }
  __syncthreads();
  const int t = lane < nw ? tmp[lane] : 0;
  *any = __ballot(lane < nw && tmp[16 + lane] != 0) != 0ull;
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

// Emit from the select kernel's LDS list (n <= kSelectLds entries: keys, and
// positions as 16-bit offsets within their tile): the positions of the
// selected keys (all keys > kth, then the first `need` keys == kth in list
// order) in list order (= ascending position).  Each thread owns a contiguous
// run of the list, of odd length so that the runs' strided LDS reads never
// share a bank; it reads its run's keys and offsets into registers in one
// batch and counts them; the counts are scanned (after which no thread reads
// the list), every thread writes its taken positions into the list's storage
// (stage), and the block copies them out in order, consecutive threads storing
// consecutive words (scattered per-thread stores would cost one memory request
// per lane).  A position is its tile's first token (64 + tile * chunk; the
// tile of list entry i is the last one whose list offset off[tile] <= i) plus
// the offset; entries past the tiles (an appended token) take last_pos.  The
// tile of the run's first entry comes from a binary search of off[], then only
// crossings read it again.  n_parts blocks share a head's list: block `part`
// emits entries [lo, hi) of it, first counting the entries taken before them.
// kEmitRun: the longest run, odd and >= (kSelectLds / n_parts) / 1024.
template <int kEmitRun>
__device__ void list_emit(const uint32_t* keys, const uint16_t* ofs, int n, int part,
                          int n_parts, const int* off, int n_chunks, int chunk, int last_pos,
                          int k, Kth r, int32_t* stage, int32_t* __restrict__ out, int* tmp) {
  const int lo = (int)((int64_t)n * part / n_parts);
  const int hi = (int)((int64_t)n * (part + 1) / n_parts);
  // the entries taken before this part: keys above the k-th, and the first
  // r.need of the keys equal to it
  int gt0 = 0, eq0 = 0;
  if (part > 0) {
    int g = 0, e = 0;
    for (int i = threadIdx.x; i < lo; i += blockDim.x) {
      const uint32_t key = keys[i];
      g += key > r.key ? 1 : 0;
      e += key == r.key ? 1 : 0;
    }
    int t0;
    block_excl_scan((g << 16) | e, tmp, &t0);  // n <= kSelectLds < 2^16
    gt0 = t0 >> 16;
    eq0 = t0 & 0xffff;
  }
  const int nn = hi - lo;
  const int per = ((nn + blockDim.x - 1) / blockDim.x) | 1;
  const int i0 = lo + min(nn, (int)threadIdx.x * per), m = min(hi - i0, per);  // m <= kEmitRun
  uint32_t kk[kEmitRun];
  uint16_t oo[kEmitRun];
#pragma unroll
  for (int j = 0; j < kEmitRun; ++j) {
    kk[j] = j < m ? keys[i0 + j] : 0u;
    oo[j] = j < m ? ofs[i0 + j] : (uint16_t)0;
  }
  int ci = 0;
  for (int step = 1 << 11; step > 0; step >>= 1)
    if (ci + step <= n_chunks && off[ci + step] <= i0) ci += step;
  int next = ci < n_chunks ? off[ci + 1] : 0x7fffffff;  // first entry of the following tile
  int gt = 0, eq = 0;
#pragma unroll
  for (int j = 0; j < kEmitRun; ++j) {
    gt += (j < m && kk[j] > r.key) ? 1 : 0;
    eq += (j < m && kk[j] == r.key) ? 1 : 0;
  }
  int tot;
  const int ex = block_excl_scan((gt << 16) | eq, tmp, &tot);  // n <= kSelectLds < 2^16
  int eq_before = eq0 + (ex & 0xffff);
  int o = gt0 + (ex >> 16) + min(eq_before, r.need);
#pragma unroll
  for (int j = 0; j < kEmitRun; ++j) {
    bool take = j < m && kk[j] > r.key;
    if (j < m && kk[j] == r.key) take = eq_before++ < r.need;
    if (take && o < k) {
      const int i = i0 + j;
      while (i >= next) {  // crossing into a later tile (rare)
        ++ci;
        next = ci < n_chunks ? off[ci + 1] : 0x7fffffff;
      }
      stage[o++] = ci < n_chunks ? kSink + ci * chunk + (int)oo[j] : last_pos;
    }
  }
  __syncthreads();
  // this part's outputs: [taken before it, taken up to its end)
  const int o0 = min(gt0 + min(eq0, r.need), k);
  const int o1 = min(gt0 + (tot >> 16) + min(eq0 + (tot & 0xffff), r.need), k);
  for (int j = o0 + (int)threadIdx.x; j < o1; j += blockDim.x) out[j] = stage[j];
}

// Copies the selection table of one head from global memory into LDS (2 KB).
// No barrier.
__device__ __forceinline__ void load_itab(const int* __restrict__ gtab, int* itab) {
  const int4* src = reinterpret_cast<const int4*>(gtab);
  int4* dst = reinterpret_cast<int4*>(itab);
  for (int i = threadIdx.x; i < kLut / 4; i += blockDim.x) dst[i] = src[i];
}

// Two bounds from one kBandBins-bin equal-width histogram of the m sample
// scores sc[0..m) (LDS; thread tid wrote sc[tid + 256u] and passes the minimum
// and maximum of its valid ones): *lo at or below the k_lo-th largest (the
// lower edge of its bin, lowered by one more bin so that rounding cannot lift
// it above), *hi at or above the k_hi-th largest (the upper edge of its bin,
// raised by one more bin; the maximum if k_hi < 1).  1 <= k_lo <= m.  Two
// barriers; then wave 0 alone scans the bins, and its results are the ones to
// use.  hist: LDS, kBandBins counters already zero (and published); red: LDS
// >= 8 floats.
template <int P>
__device__ void block_score_band(const float* sc, float smin, float smax, int m, int k_lo, int k_hi,
                                 uint32_t* hist, float* red, float* lo, float* hi) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  smin = row_allreduce(smin, [](float x, float y) { return fminf(x, y); });
  smax = row_allreduce(smax, [](float x, float y) { return fmaxf(x, y); });
  smin = fminf(fminf(readlane(smin, 0), readlane(smin, 16)), fminf(readlane(smin, 32), readlane(smin, 48)));
  smax = fmaxf(fmaxf(readlane(smax, 0), readlane(smax, 16)), fmaxf(readlane(smax, 32), readlane(smax, 48)));
  if (lane == 0) {
    red[wave] = smin;
    red[4 + wave] = smax;
  }
  __syncthreads();
  smin = fminf(fminf(red[0], red[1]), fminf(red[2], red[3]));
  smax = fmaxf(fmaxf(red[4], red[5]), fmaxf(red[6], red[7]));
  if (!(smax > smin)) {
    *lo = smin;
    *hi = smax;
    return;
  }
  const float w = (smax - smin) * (1.0f / kBandBins);
  const float inv = (float)kBandBins / (smax - smin);
#pragma unroll
  for (int u = 0; u < P; ++u) {
    const int i = tid + 256 * u;
    if (i < m) atomicAdd(&hist[min(max((int)((sc[i] - smin) * inv), 0), kBandBins - 1)], 1u);
  }
  __syncthreads();
  if (wave != 0) return;
  // lane l owns bins kB*l .. kB*l + kB - 1 (ascending scores)
  constexpr int kB = kBandBins / 64;
  uint32_t cnt[kB];
  int tot = 0;
#pragma unroll
  for (int u = 0; u < kB; ++u) {
    cnt[u] = hist[lane * kB + u];
    tot += (int)cnt[u];
  }
  int pre = wave_incl_scan(tot) - tot;
  const int x_lo = m - k_lo, x_hi = m - k_hi;  // ascending ranks of the k-th largest
  int dl = -1, dh = -1;
#pragma unroll
  for (int u = 0; u < kB; ++u) {
    const int c = (int)cnt[u];
    if (pre <= x_lo && x_lo < pre + c) dl = lane * kB + u;
    if (k_hi >= 1 && pre <= x_hi && x_hi < pre + c) dh = lane * kB + u;
    pre += c;
  }
  const uint64_t ml = __ballot(dl >= 0), mh = __ballot(dh >= 0);  // one lane each
  const int bl = __builtin_amdgcn_readlane(dl, (int)__builtin_ctzll(ml));
  const int bhi = mh ? __builtin_amdgcn_readlane(dh, (int)__builtin_ctzll(mh)) : kBandBins - 1;
  *lo = smin + (float)(bl - 1) * w;
  *hi = k_hi >= 1 ? fminf(smax, smin + (float)(bhi + 2) * w) : smax;
}

// rank: how many of the sampled scores lie at or above tau.  For a small head the
// whole candidate set (n <= 2048) is the sample and rank = k (tau is then at most
// the exact k-th score).  Otherwise the expected rank e = k * 2048 / n of the k-th
// score in the sample plus four standard deviations (of a binomial count; the
// stratified sample varies less) and a small floor, so that fewer than k tokens
// pass only with negligible probability (about 3e-5 per head; the select kernel
// handles that case exactly anyway).  rank_hi: the rank of the upper end of the
// select kernel's score bins, e - 4 sqrt(e) - 8 (the k-th score lies below it
// with high probability), or the top of the sample if that is below 1.
__device__ __forceinline__ void sample_ranks(int k, int n, int* rank, int* rank_hi) {
  if (n <= kSampleMax) {
    *rank = k;
    *rank_hi = k;
    return;
  }
  const double e = (double)k * kSampleMax / (double)n;
  const double r = e + 4.0 * sqrt(e) + 8.0;
  *rank = r > kSampleMax ? kSampleMax + 1 : (int)r + 1;
  const double rh = e - 4.0 * sqrt(e) - 8.0;
  *rank_hi = rh < 1.0 ? 0 : (int)rh;
}

// The threshold word: a head's leader block publishes (kTauTag << 32 | tau bits)
// with one device-scope store; the select kernel clears it after reading it, so
// a word left from an earlier call never carries the tag.
constexpr uint32_t kTauTag = 0x53494b56u;
constexpr int kTauPolls = 4096;  // bounded wait: then the tile keeps every token

// ------------------------------------------------------------------ selection table
// The selection query's int32 table (§2.1 item 2), built by any block of 256
// threads of the head: thread tid makes entries 2tid and 2tid+1 (sub-vector
// j = tid >> 3).  Every block that builds it performs the same operations in the
// same order and gets the same bits, so a token's score is one value in every
// kernel.  qbar_c = sum over g ascending of q_g,c (fp32); A bounds the 32-term
// sums (sum_c |qbar_c| for the sign vertices, as a wave sum of |qbar_2l| +
// |qbar_2l+1| over lanes l; sum_j max_p |LUT[j][p]| in j order for a
// codebook); with A = m * 2^x, m in [0.5, 1), entries are rint(LUT * 2^(30 - x)).
// Per lane: G 4-byte loads of q (channels 2l, 2l+1) and, with a codebook, the
// two centres.  jmax: LDS [32] (codebook only; one extra barrier).
struct SelQ {
  uint32_t qw[kMaxGroup];  // packed bf16 pairs: channels 2l, 2l+1 of q_g
  float4 c0, c1;           // codebook centres of entries 2tid, 2tid+1
};
template <bool kCb>
__device__ __forceinline__ void sel_issue(SelQ& s, const uint16_t* __restrict__ q, int64_t hq0,
                                          int G, const float* __restrict__ cb, int tid) {
  const int lane = tid & 63;
#pragma unroll
  for (int g = 0; g < kMaxGroup; ++g)
    s.qw[g] = g < G ? *reinterpret_cast<const uint32_t*>(q + (hq0 + g) * kD + 2 * lane) : 0u;
  if constexpr (kCb) {
    s.c0 = reinterpret_cast<const float4*>(cb)[2 * tid];
    s.c1 = reinterpret_cast<const float4*>(cb)[2 * tid + 1];
  }
}
// The rest of the table from this lane's two channels of the summed query
// (q0 = qbar_2l, q1 = qbar_2l+1; every wave holds all 128 channels).
template <bool kCb>
__device__ __forceinline__ int2 sel_finish(float q0, float q1, const float4& c0, const float4& c1,
                                           float* jmax, int tid, float* inv_out) {
  const int lane = tid & 63;
  // channels 4j..4j+3 of this thread's sub-vector (j = tid >> 3 <= 31) sit in
  // lanes 2j and 2j+1 of every wave
  const int j = tid >> 3;
  const int src = 2 * j;
  const float x0 = __shfl(q0, src), x1 = __shfl(q1, src);
  const float x2 = __shfl(q0, src + 1), x3 = __shfl(q1, src + 1);
  float v0, v1;
  if constexpr (kCb) {
    v0 = ((x0 * c0.x + x1 * c0.y) + x2 * c0.z) + x3 * c0.w;
    v1 = ((x0 * c1.x + x1 * c1.y) + x2 * c1.z) + x3 * c1.w;
  } else {
    v0 = sign_entry(x0, x1, x2, x3, (2 * tid) & 15);
    v1 = sign_entry(x0, x1, x2, x3, (2 * tid + 1) & 15);
  }
  float A;
  if constexpr (kCb) {
    float mx = fmaxf(fabsf(v0), fabsf(v1));
    mx = fmaxf(mx, __shfl_xor(mx, 1));
    mx = fmaxf(mx, __shfl_xor(mx, 2));
    mx = fmaxf(mx, __shfl_xor(mx, 4));
    if ((lane & 7) == 0) jmax[j] = mx;
    __syncthreads();
    A = 0.0f;
    for (int jj = 0; jj < kSub; ++jj) A += jmax[jj];
  } else {
    A = wave_sum(fabsf(q0) + fabsf(q1));
  }
  int ex = 0;
  if (A > 0.0f) {
    frexpf(A, &ex);
    ex = 30 - ex;
  }
  *inv_out = ldexpf(1.0f, -ex);
  return make_int2((int)rintf(ldexpf(v0, ex)), (int)rintf(ldexpf(v1, ex)));
}

// From the query words in registers (sel_issue).
template <bool kCb>
__device__ __forceinline__ int2 sel_build(const SelQ& s, int G, float* jmax, int tid,
                                          float* inv_out) {
  float q0 = bf16lo(s.qw[0]), q1 = bf16hi(s.qw[0]);
#pragma unroll
  for (int g = 1; g < kMaxGroup; ++g)
    if (g < G) {
      q0 += bf16lo(s.qw[g]);
      q1 += bf16hi(s.qw[g]);
    }
  return sel_finish<kCb>(q0, q1, s.c0, s.c1, jmax, tid, inv_out);
}

// From the G query rows staged in LDS (qs: [G][64] words, channels 2l, 2l+1 in
// word l); the same sums in the same order as sel_build.
template <bool kCb>
__device__ __forceinline__ int2 sel_build_lds(const uint32_t* qs, int G, const float4& c0,
                                              const float4& c1, float* jmax, int tid,
                                              float* inv_out) {
  const int lane = tid & 63;
  float q0 = bf16lo(qs[lane]), q1 = bf16hi(qs[lane]);
  for (int g = 1; g < G; ++g) {
    const uint32_t w = qs[g * 64 + lane];
    q0 += bf16lo(w);
    q1 += bf16hi(w);
  }
  return sel_finish<kCb>(q0, q1, c0, c1, jmax, tid, inv_out);
}

// ------------------------------------------------------------------ attention tables
// Tables of the G query heads for the attention kernel, by one block of 256
// threads: att_lut[g][e] = q_g(4j..4j+3) . c_e (the sign vertex or the centre e,
// j = e >> 4), att_qmu[g] = q_g . mu, and the exact logits of the 64 sinks,
// att_slog[g][r] = q_g . k_sink[r] (full-precision keys, §2.1 item 3), fp32.
__device__ void attention_tables(const ScoreArgs& a, int bh) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int b = bh / a.Hkv, h = bh - b * a.Hkv, G = a.G;
  const int64_t hq0 = (int64_t)b * a.n_q_heads + (int64_t)h * G;
  const float* cb = a.codebook != nullptr ? a.codebook + (int64_t)bh * kLut * 4 : nullptr;
  // table entries 2tid, 2tid+1 (sub-vector j) of every query head
  {
    const int j = tid >> 3;
    float4 c0 = make_float4(0.f, 0.f, 0.f, 0.f), c1 = c0;
    if (cb != nullptr) {
      c0 = reinterpret_cast<const float4*>(cb)[2 * tid];
      c1 = reinterpret_cast<const float4*>(cb)[2 * tid + 1];
    }
    for (int g = 0; g < G; ++g) {
      const uint2 w = *reinterpret_cast<const uint2*>(a.q + (hq0 + g) * kD + 4 * j);
      const float xs[4] = {bf16lo(w.x), bf16hi(w.x), bf16lo(w.y), bf16hi(w.y)};
      float2 v;
      if (cb != nullptr) {
        v.x = ((xs[0] * c0.x + xs[1] * c0.y) + xs[2] * c0.z) + xs[3] * c0.w;
        v.y = ((xs[0] * c1.x + xs[1] * c1.y) + xs[2] * c1.z) + xs[3] * c1.w;
      } else {
        v.x = sign_entry(xs[0], xs[1], xs[2], xs[3], (2 * tid) & 15);
        v.y = sign_entry(xs[0], xs[1], xs[2], xs[3], (2 * tid + 1) & 15);
      }
      reinterpret_cast<float2*>(a.att_lut + (hq0 + g) * kLut)[tid] = v;
    }
  }
  // q_g . mu: wave w takes heads w, w + 4
  for (int g = wave; g < G; g += 4) {
    const float* m = a.mu + (int64_t)bh * kD;
    const uint16_t* qg = a.q + (hq0 + g) * kD;
    const float d = wave_sum(fmaf(__uint_as_float((uint32_t)qg[lane] << 16), m[lane],
                                  __uint_as_float((uint32_t)qg[lane + 64] << 16) * m[lane + 64]));
    if (lane == 0) a.att_qmu[hq0 + g] = d;
  }
  // sink logits: 16 lanes per sink row (8 channels each), 16 rows per pass
  const int c0 = (tid & 15) * 8;
  for (int r0 = 0; r0 < kSink; r0 += 16) {
    const int r = r0 + (tid >> 4);
    const uint4 ks = *reinterpret_cast<const uint4*>(a.k_sink + ((int64_t)bh * kSink + r) * kD + c0);
    const float x[8] = {bf16lo(ks.x), bf16hi(ks.x), bf16lo(ks.y), bf16hi(ks.y),
                        bf16lo(ks.z), bf16hi(ks.z), bf16lo(ks.w), bf16hi(ks.w)};
    for (int g = 0; g < G; ++g) {
      const uint4 qq = *reinterpret_cast<const uint4*>(a.q + (hq0 + g) * kD + c0);
      const float y[8] = {bf16lo(qq.x), bf16hi(qq.x), bf16lo(qq.y), bf16hi(qq.y),
                          bf16lo(qq.z), bf16hi(qq.z), bf16lo(qq.w), bf16hi(qq.w)};
      float d = 0.0f;
#pragma unroll
      for (int i = 0; i < 8; ++i) d = fmaf(y[i], x[i], d);
      d = row_allreduce(d, [](float u, float v) { return u + v; });  // the row's 16 lanes
      if ((tid & 15) == 0) a.att_slog[(hq0 + g) * kSink + r] = d;
    }
  }
}

// Attention tables alone (a standalone sparse attention call): one block of
// 256 threads per (b, KV head).
__global__ __launch_bounds__(256) void tables_kernel(ScoreArgs a) {
  attention_tables(a, blockIdx.x);
}

// The appended token (k_new, the sequence's last): code and scale with the
// frozen mean (bit-identical to the encode kernel), value record, and its
// selection key for the select kernel (one wave; not on the threshold's path).
__device__ __forceinline__ void leader_append(const ScoreArgs& a, int bh, int b, int h, int nt,
                                              const int* itab, float inv) {
  const int tid = threadIdx.x, lane = tid & 63;
  // key row: lanes 0..15, 8 channels each, with their means; value row: lanes
  // 16..31
  uint4 kw = make_uint4(0u, 0u, 0u, 0u), vw = kw;
  float km[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  {
    if (lane < 16) {
      kw = *reinterpret_cast<const uint4*>(a.k_new + (int64_t)b * a.ksb + (int64_t)h * a.ksh +
                                           lane * 8);
      const float4 m0 = *reinterpret_cast<const float4*>(a.mu + (int64_t)bh * kD + lane * 8);
      const float4 m1 = *reinterpret_cast<const float4*>(a.mu + (int64_t)bh * kD + lane * 8 + 4);
      km[0] = m0.x; km[1] = m0.y; km[2] = m0.z; km[3] = m0.w;
      km[4] = m1.x; km[5] = m1.y; km[6] = m1.z; km[7] = m1.w;
    } else if (lane < 32 && a.v_new != nullptr) {
      vw = *reinterpret_cast<const uint4*>(a.v_new + (int64_t)b * a.vnsb + (int64_t)h * a.vnsh +
                                           (lane - 16) * 8);
    }
  }
  uint4 cn = make_uint4(0u, 0u, 0u, 0u);
  float an = 0.0f;
  {  // the whole wave runs the 16-lane shuffles
    const RowCode rc = encode_row16(kw, km);
    const int64_t row = a.rm.row(b, h, nt - 1);
    if (lane < 16 && (lane & 3) == 0) {
      *reinterpret_cast<uint32_t*>(a.codes + row * kCodeBytes + lane) = rc.word;
      if (a.vrec != nullptr)
        *reinterpret_cast<uint32_t*>(a.vrec + row * kVRecBytes + kVRecCode + lane) = rc.word;
    }
    if (lane == 0) a.alpha[row] = rc.alpha;
    if (a.v_new != nullptr) {
      const VRowCode vc = quantize_vrow16(vw);  // lanes 16..31 hold the value row
      const uint32_t pair = vc.bits | (__shfl_down(vc.bits, 1, 16) << 16);
      const int cg = lane - 16;
      uint8_t* rec = a.vrec + row * kVRecBytes;
      if (cg >= 0 && cg < 16 && (cg & 1) == 0) *reinterpret_cast<uint32_t*>(rec + 2 * cg) = pair;
      if (cg >= 0 && cg < 16 && (cg & 3) == 0)
        *reinterpret_cast<uint32_t*>(rec + kVRecSz + cg) = vc.sz;
    }
    cn = make_uint4((uint32_t)__builtin_amdgcn_readlane((int)rc.word, 0),
                    (uint32_t)__builtin_amdgcn_readlane((int)rc.word, 4),
                    (uint32_t)__builtin_amdgcn_readlane((int)rc.word, 8),
                    (uint32_t)__builtin_amdgcn_readlane((int)rc.word, 12));
    an = readlane(rc.alpha, 0);
  }
  if (lane == 0) {
    const float sv = selection_score(itab, inv, cn, an);
    a.app_key[bh] = score_key(sv);
    if (a.scores_opt != nullptr) a.scores_opt[(int64_t)bh * a.rm.capacity + nt - 1] = sv;
  }
}

// ------------------------------------------------------------------ leader
// One block per (b, KV head), dispatched before every tile block of the score
// kernel (lowest block indices): the selection table (kept in the workspace
// for the select kernel's exact path) and the sampled threshold tau, published
// to the head's tiles through the threshold word; the block then scores the
// head's last tile itself (so the grid has one block per tile) (the attention tables are made
// by extra blocks of the select kernel, off this path).
// Sample: stratum st = i / 16 of 128 equal segments of the head's candidates,
// 16 contiguous tokens centred in it (the whole candidate set when it is small;
// an appended token, the last one, is left out).  The leader also encodes an appended token (k_new) into
// the cache and leaves its selection key for the select kernel.  Three rounds
// of 3 sample rows per thread (4 rounds: more rows in flight would take the
// kernel past 64 VGPRs, below eight waves per SIMD).  mode 1: sampled tau;
// mode 2: tau = +inf (nothing passes: the select kernel takes its exact
// whole-head path).  No sample (it would not bound the k-th): tau = -inf.
template <bool kCb>
__device__ float leader(const ScoreArgs& a, int bh, int* itab, uint32_t* hist, uint32_t* qs,
                        float* ssc, float* red, float* jmax) {
  constexpr int kRows = kSampleMax / 256;  // sample rows per thread, all in flight at once
  static_assert(kRows * 256 == kSampleMax, "sample split");
  __builtin_amdgcn_s_setprio(3);  // issue ahead of the tile waves sharing the CU
  const int tid = threadIdx.x, wave = tid >> 6;
  const int b = bh / a.Hkv, h = bh - b * a.Hkv;
  const int nt = seq_len(a.seq_lens, b, a.n_tokens);
  const bool append = a.k_new != nullptr;
  const int n = nt - kSink - (append ? 1 : 0);  // candidates the sample covers
  int rank = 1, rank_hi = 0;
  if (a.mode == 1) sample_ranks(seq_topk(a.top_k, nt), n, &rank, &rank_hi);
  const bool full = n <= kSampleMax;
  const int m = full ? n : kSampleMax;
  const bool sample = a.mode == 1 && m > 0 && rank <= m;
  const int64_t hq0 = (int64_t)b * a.n_q_heads + (int64_t)h * a.G;
  const float* cb = a.codebook != nullptr ? a.codebook + (int64_t)bh * kLut * 4 : nullptr;
  for (int i = tid; i < kBandBins; i += 256) hist[i] = 0u;  // the band's counters
  // The G query rows (8 bytes per thread) and the centres, then the sample: the
  // table's wait does not include the sample rows, and the rows go to LDS first
  // so that only two registers per thread hold them while the sample is in
  // flight.
  const uint2 qv = tid < a.G * 32
                       ? *reinterpret_cast<const uint2*>(a.q + (hq0 + (tid >> 5)) * kD + 4 * (tid & 31))
                       : make_uint2(0u, 0u);
  float4 c0 = make_float4(0.f, 0.f, 0.f, 0.f), c1 = c0;
  if constexpr (kCb) {
    c0 = reinterpret_cast<const float4*>(cb)[2 * tid];
    c1 = reinterpret_cast<const float4*>(cb)[2 * tid + 1];
  }
  // Every lane loads a real sample row (token 64 for unused slots, never
  // scored).
  uint4 c[kRows];
  float al[kRows];
  if (sample) {
    // rows as 32-bit offsets from a uniform base: the head's first row
    // (contiguous) or the pool's (paged: pool rows fit in 32 bits)
    const bool paged = a.rm.table != nullptr;
    const int64_t base = paged ? 0 : (int64_t)bh * a.rm.capacity;
    const char* cbase = reinterpret_cast<const char*>(a.codes + base * kCodeBytes);
    const char* abase = reinterpret_cast<const char*>(a.alpha + base);
    uint32_t r[kRows];
#pragma unroll
    for (int u = 0; u < kRows; ++u) {
      const int i = tid + u * 256;
      int t = kSink + i;
      if (!full) {
        const int st = i / kSampleRun, ns = kSampleMax / kSampleRun;
        const int64_t seg0 = (int64_t)st * n / ns, seg1 = (int64_t)(st + 1) * n / ns;
        t = kSink + (int)(seg0 + (seg1 - seg0 - kSampleRun) / 2) + (i - st * kSampleRun);
      }
      r[u] = (uint32_t)(i < m ? t : kSink);
    }
    if (paged) {  // every row's page id first (one round trip), then the rows
      const int lg = a.rm.lg_page;
      int pg[kRows];
#pragma unroll
      for (int u = 0; u < kRows; ++u) pg[u] = a.rm.table[(int64_t)b * a.rm.pps + (r[u] >> lg)];
#pragma unroll
      for (int u = 0; u < kRows; ++u)
        r[u] = (uint32_t)((((int64_t)pg[u] * a.Hkv + h) << lg) | (int64_t)(r[u] & ((1u << lg) - 1)));
    }
#pragma unroll
    for (int u = 0; u < kRows; ++u) {
      c[u] = *reinterpret_cast<const uint4*>(cbase + (size_t)r[u] * kCodeBytes);
      al[u] = *reinterpret_cast<const float*>(abase + (size_t)r[u] * 4);
    }
  }
  if (tid < a.G * 32) reinterpret_cast<uint2*>(qs)[tid] = qv;
  __syncthreads();  // qs
  float inv;
  const int2 tv = sel_build_lds<kCb>(qs, a.G, c0, c1, jmax, tid, &inv);
  reinterpret_cast<int2*>(itab)[tid] = tv;
  reinterpret_cast<int2*>(a.sel_lut + (int64_t)bh * kLut)[tid] = tv;
  if (tid == 0) a.sel_inv[bh] = inv;
  __syncthreads();  // itab; every read of qs is done
  // no sample: +inf (mode 2: nothing passes) or -inf (keep all)
  float th = a.mode == 2 ? INFINITY : -INFINITY, th_hi = 0.0f;
  if (sample) {
    float smin = INFINITY, smax = -INFINITY;
#pragma unroll
    for (int u = 0; u < kRows; ++u) {  // each row's registers free as soon as it is scored
      const float sv = selection_score(itab, inv, c[u], al[u]);
      ssc[tid + u * 256] = sv;
      if (tid + u * 256 < m) {
        smin = fminf(smin, sv);
        smax = fmaxf(smax, sv);
      }
    }
    block_score_band<kRows>(ssc, smin, smax, m, rank, rank_hi, hist, red, &th, &th_hi);
  }
  if (wave == 1 && append) leader_append(a, bh, b, h, nt, itab, inv);  // beside the publication
  if (tid == 0) {
    // the select kernel bins candidate scores linearly, 2048 bins from tau up
    // to an upper estimate of the k-th score (higher scores share the top bin)
    const float span = th_hi - th;
    a.bin_scale[bh] = sample && span > 0.0f ? 2048.0f / span : 0.0f;
    a.bin_scale[a.n_heads + bh] = th;  // the select kernel's copy, never cleared
    __hip_atomic_store(a.tau_word + bh, ((unsigned long long)kTauTag << 32) | __float_as_uint(th),
                       __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  __builtin_amdgcn_s_setprio(0);  // the block's own tile follows at normal priority
  return inv;
}

// The published threshold of a head: w, lane 0's earlier load of the word,
// if it already carries the tag, else lane 0 polls (device-scope loads, a
// short sleep between them); after kTauPolls polls the wave gives up and
// returns -inf (the tile then keeps every token: a correct, slower
// selection).  Wave-uniform result.
__device__ __forceinline__ float wait_tau(unsigned long long* word, unsigned long long w) {
  if ((threadIdx.x & 63) == 0) {
    for (int i = 0; i < kTauPolls && (uint32_t)(w >> 32) != kTauTag; ++i) {
      __builtin_amdgcn_s_sleep(4);
      w = __hip_atomic_load(word, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
  const uint32_t tag = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(w >> 32));
  const uint32_t tb = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)w);
  return tag == kTauTag ? __uint_as_float(tb) : -INFINITY;
}

// ------------------------------------------------------------------ score
// Grid: B*Hkv leader blocks (above; each also scores its head's last tile),
// then one block per other tile of 256*U candidates of a head, 1-D, head-major:
// one block per tile in all, so that a grid of 2048 tiles is resident at once
// (eight blocks per CU).  In a tile, lane <-> token; wave w
// scores the tile's w-th quarter, U groups of 64 tokens, on its own.  Each wave
// issues all its loads first; they are unconditional, at token indices clamped
// to the sequence's last token (always a valid row), so the compiler counts the
// loads in flight exactly and each group waits only for its own data.  Rows are
// 32-bit lane offsets from a wave-uniform base row: a 64-token group lies
// within one page of a paged cache (groups start at multiples of 64, pages at
// multiples of >= 256), so one page id serves the group.  The block builds the
// selection table itself (the same bits as its leader's) while the loads are
// in flight; once its tokens are scored, each wave waits for the leader's tau
// and the candidates (score >= tau) are written in token order, with the tau
// the tile used.  An appended token (the sequence's last) is left to the
// leader, which encodes and scores it; the select kernel adds it at the end of
// the head's candidates.
// Eight waves per SIMD (64 VGPRs) for tiles of up to 8 groups, so that the
// 2048-tile grid at 128K tokens is resident at once; the leader path and the
// tile path each fit, but the allocator would give the merged kernel a few more
// without the bound (the codebook variant spills 32 bytes per lane).
template <int U, bool kPaged, bool kCb, int S = (U < 8 ? U : 8)>
__global__ __launch_bounds__(256, (U <= 8 ? 8 : 1)) void score_kernel(ScoreArgs a) {
  constexpr int kChunk = 256 * U;
  constexpr int NS = U / S;  // steps of S groups, all loaded before the table barrier
  static_assert(U % S == 0 && NS <= 2, "tile shape");
  __shared__ int itab[kLut];
  __shared__ uint32_t hist[kBandBins];    // leader only
  __shared__ uint32_t qs[kMaxGroup * 64];  // leader only: the query rows
  __shared__ float ssc[kSampleMax];       // leader only: the sample scores
  __shared__ float red[8];                // leader only
  __shared__ float jmax[kSub];
  __shared__ int wcnt[4];
  __shared__ uint32_t wtau[4];
  // Block bh < n_heads: the leader of head bh, which then scores the head's
  // last tile with the table it built; the other blocks score tiles
  // 0 .. n_chunks - 2 of their head.
  const bool lead = (int)blockIdx.x < a.n_heads;
  int bh, cx;
  if (lead) {
    bh = blockIdx.x;
    cx = a.n_chunks - 1;
  } else {
    const int tile = blockIdx.x - a.n_heads, per = a.n_chunks - 1;
    bh = tile / per;
    cx = tile - bh * per;
  }
  float inv = 0.0f;
  if (lead) inv = leader<kCb>(a, bh, itab, hist, qs, ssc, red, jmax);
  const int b = bh / a.Hkv, h = bh - b * a.Hkv;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: rows from scalar bases
  // tokens the tiles score: an appended token (the sequence's last) is the
  // leader's, which writes its row in this same kernel
  const int nt = seq_len(a.seq_lens, b, a.n_tokens) - (a.k_new != nullptr ? 1 : 0);
  const int t0 = kSink + cx * kChunk;  // the tile's first token
  const int tw = t0 + wave * (64 * U);  // this wave's first token
  const int lim = nt - tw;  // tokens of this wave's quarter in the sequence (<= 0: none)
  const int64_t hq0 = (int64_t)b * a.n_q_heads + (int64_t)h * a.G;
  const float* cb = a.codebook != nullptr ? a.codebook + (int64_t)bh * kLut * 4 : nullptr;
  SelQ sq;
  if (!lead) sel_issue<kCb>(sq, a.q, hq0, a.G, cb, tid);
  const int64_t hrow = (int64_t)bh * a.rm.capacity;  // contiguous: the head's first row
  // Paged: the quarter's tokens (clamped to the sequence) span at most U + 1
  // pages; lane j holds the id of the j-th, read out per group with a lane read
  // (a per-group load would wait behind every code load in flight).
  const int lg = a.rm.lg_page;
  const int pfirst = min(tw, nt - 1) >> lg;
  int pv = 0;
  if constexpr (kPaged)
    pv = a.rm.table[(int64_t)b * a.rm.pps + min(pfirst + lane, (nt - 1) >> lg)];
  // Loads of step st.
  uint4 c[NS][S];
  float al[NS][S];
  auto row_base = [&](int gb) {
    if constexpr (kPaged) {
      const int64_t pg = __builtin_amdgcn_readlane(pv, (gb >> lg) - pfirst);
      return ((pg * a.Hkv + h) << lg) | (int64_t)(gb & ((1 << lg) - 1));
    } else {
      return hrow + gb;
    }
  };
  auto load_step = [&](int st) {
#pragma unroll
    for (int u = 0; u < S; ++u) {
      const int g0 = tw + (st * S + u) * 64;  // first token of the group
      const int gb = min(g0, nt - 1);         // base row's token (uniform)
      const uint32_t o = (uint32_t)(min(g0 + lane, nt - 1) - gb);
      const int64_t r0 = row_base(gb);
      c[st][u] = *reinterpret_cast<const uint4*>(
          reinterpret_cast<const char*>(a.codes + r0 * kCodeBytes) + (o << 4));
      al[st][u] = *reinterpret_cast<const float*>(
          reinterpret_cast<const char*>(a.alpha + r0) + (o << 2));
    }
  };
  load_step(0);
  if constexpr (NS > 1) load_step(1);
  if (!lead) {  // (the leader's table is in itab already)
    const int2 tv = sel_build<kCb>(sq, a.G, jmax, tid, &inv);
    int tz;
    asm volatile("v_mov_b32 %0, 0" : "=v"(tz));  // the table is stored after the loads go out
    reinterpret_cast<int2*>(itab)[tid] = make_int2(tv.x ^ tz, tv.y ^ tz);
  }
  __syncthreads();
  uint32_t key[U];
  // gate: a zero from an asm placed after the table barrier (then after the
  // previous step's sums); the step's codes and scales are read through it, so
  // their decode stays behind it, in order: without it the compiler hoists
  // most look-ups into one batch (more VGPRs, fewer waves per SIMD).
  auto score_step = [&](int st, int gate) {
#pragma unroll
    for (int u = 0; u < S; ++u) {
      const int g = st * S + u;
      uint4 cg = c[st][u];
      cg.x ^= gate, cg.y ^= gate, cg.z ^= gate, cg.w ^= gate;
      const float ag = __int_as_float(__float_as_int(al[st][u]) ^ gate);
      key[g] = score_key(selection_score(itab, inv, cg, ag));
    }
  };
  // One device-scope load of the threshold word, issued behind the code loads
  // (it completes after them, so no group waits for it): a tile that finishes
  // after the leader published finds tau without a further round trip.
  unsigned long long tw0 = 0ull;
  if (lane == 0 && lim > 0)
    tw0 = __hip_atomic_load(a.tau_word + bh, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  int gate;
  asm volatile("v_mov_b32 %0, 0" : "=v"(gate));
#pragma unroll
  for (int st = 0; st < NS; ++st) {
    score_step(st, gate);
    uint32_t dep = key[st * S];
#pragma unroll
    for (int u = 1; u < S; ++u) dep ^= key[st * S + u];
    asm volatile("v_mov_b32 %0, 0" : "=v"(gate) : "v"(dep));
  }
  const float th = lim > 0 ? wait_tau(a.tau_word + bh, tw0) : -INFINITY;  // nothing to keep: no wait
  const uint32_t thk = score_key(th + 0.0f);
  uint32_t bits = 0;  // bit g: token g*64 + lane of the quarter passed
#pragma unroll
  for (int g = 0; g < U; ++g)
    if (g * 64 + lane < lim && key[g] >= thk) bits |= 1u << g;
  int cnt = 0;
#pragma unroll
  for (int g = 0; g < U; ++g) cnt += __popcll(__ballot((bits >> g) & 1u));
  if (lane == 0) {
    wcnt[wave] = cnt;
    wtau[wave] = __float_as_uint(th);
  }
  __syncthreads();
  int run = 0;  // candidates of the waves before this one
#pragma unroll
  for (int w = 0; w < 3; ++w) run += w < wave ? wcnt[w] : 0;
  const int64_t slot = ((int64_t)bh * a.n_chunks + cx) * kChunk;
  uint32_t* __restrict__ kout = a.cand_key + slot;
  int32_t* __restrict__ tout = a.cand_t + slot;
#pragma unroll
  for (int g = 0; g < U; ++g) {
    const bool pass = (bits >> g) & 1u;
    const uint64_t mk = __ballot(pass);
    if (pass) {
      const int p = run + ballot_rank(mk);
      kout[p] = key[g];
      tout[p] = tw + g * 64 + lane;
    }
    run += __popcll(mk);
  }
  if (a.scores_opt != nullptr) {  // key_score inverts score_key exactly
    float* __restrict__ so = a.scores_opt + hrow + tw;
#pragma unroll
    for (int g = 0; g < U; ++g)
      if (g * 64 + lane < lim) so[g * 64 + lane] = key_score(key[g]);
  }
  if (tid == 255) {  // the last wave's run ends the tile
    // The threshold the tile kept its tokens with: the published one if any
    // wave saw it (-inf, a wave that gave up waiting, keeps a superset); two
    // different real values (a stale word, then the published one) are
    // recorded as a NaN, which sends the head to the exact path.
    uint32_t rec = 0xff800000u;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const uint32_t x = wtau[w];
      if (x != 0xff800000u) rec = (rec == 0xff800000u || rec == x) ? x : 0x7fc00001u;
    }
    a.chunk_count[(int64_t)bh * a.n_chunks + cx] = make_int2(run, (int)rec);
  }
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
template <int P>  // one copy per select kernel (one shared by several cost them SGPR spills)
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
// workspace (tile by tile, wave w taking tiles w, w + 16, ...; an appended
// token last) and radix rounds select over it.
template <int P>
__device__ __noinline__ bool select_workspace(
    const uint32_t* __restrict__ cand_key, const int32_t* __restrict__ cand_t, int chunk,
    int n_chunks, const int* off, int C, int top_k, bool extra, uint32_t extra_key,
    int32_t extra_pos, uint32_t thk, uint32_t* __restrict__ comp_key,
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
  if (extra && threadIdx.x == 0) {  // the appended token, last in the list
    comp_key[C - 1] = extra_key;
    comp_t[C - 1] = extra_pos;
    lo = min(lo, extra_key);
    hi = max(hi, extra_key);
  }
  block_minmax(lo, hi, mm, &lo, &hi);  // its barriers also publish the copies
  const Kth r = block_kth(comp_key, C, top_k, lo, hi, hist, tmp, sub, scount);
  if (r.key < thk) return false;  // below the threshold: not provably the k-th
  block_emit(comp_key, comp_t, C, top_k, r, out, tmp);
  return true;
}

// The k-th's bin holds too many keys (e.g. no usable bin scale): radix rounds
// over the whole LDS list.
template <int P>
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

template <int kParts>
__global__ __launch_bounds__(1024) void select_kernel(
    const uint8_t* __restrict__ codes, const float* __restrict__ alpha, RowMap rm,
    int n_tokens, int Hkv, const int32_t* __restrict__ seq_lens,
    const int* __restrict__ sel_lut, const float* __restrict__ sel_inv, int top_k_max,
    int chunk, int n_chunks,
    const uint32_t* __restrict__ cand_key, const int32_t* __restrict__ cand_t,
    const int2* __restrict__ chunk_count, unsigned long long* __restrict__ tau_word,
    const float* __restrict__ bin_scale, const uint32_t* __restrict__ app_key,
    uint32_t* __restrict__ comp_key, int32_t* __restrict__ comp_t, int32_t* __restrict__ idx,
    ScoreArgs ta) {
  constexpr int n_parts = kParts;
  __shared__ int off[kMaxChunks + 1];
  __shared__ uint32_t hist[2048];
  __shared__ uint32_t lkey[kSelectLds];
  __shared__ uint16_t lofs[kSelectLds];
  __shared__ uint32_t sub[2 * kSubMax];  // boundary-bin keys, then block_kth's own sub-list
  __shared__ int tmp[32];
  __shared__ uint32_t mm[32];
  __shared__ int scount;
  if ((int)blockIdx.x >= n_parts * ta.n_heads) {  // the grid's tail: attention tables
    if (threadIdx.x < 256) attention_tables(ta, blockIdx.x - n_parts * ta.n_heads);
    return;
  }
  // n_parts (1..4) blocks per head, which build the same list and find the
  // same k-th; each then emits its part of the ordered selection.  The rare
  // paths (the whole-head rescan, the list in the workspace) are the first
  // block's alone.
  const int bh = blockIdx.x / n_parts, part = blockIdx.x % n_parts;
  const int tid = threadIdx.x;
  const int nt = seq_len(seq_lens, bh / Hkv, n_tokens);
  const int n = nt - kSink;
  const int top_k = seq_topk(top_k_max, nt);  // this sequence's k; the rest of its row is -1
  // The threshold the head's leader published, from its untagged copy (never
  // cleared, so all of the head's blocks read the same value); the first block
  // clears the tagged word for the next call's tiles.
  const uint32_t thb = __float_as_uint(bin_scale[ta.n_heads + bh]);
  int32_t* out = idx + (int64_t)bh * top_k_max;
  if (top_k >= n) {  // every candidate is kept
    if (part == 0) {
      if (tid == 0) tau_word[bh] = 0ull;
      for (int j = tid; j < top_k_max; j += blockDim.x) out[j] = j < top_k ? kSink + j : -1;
    }
    return;
  }
  if (part == 0)
    for (int j = top_k + tid; j < top_k_max; j += blockDim.x) out[j] = -1;
  for (int i = tid; i < 2048; i += blockDim.x) hist[i] = 0u;  // published by the scan's barriers
  // Tile counts -> offsets of each tile's candidates in the ordered list.  The
  // counts are loaded first, then the first kPreG * 64 slots of each wave's
  // first four tiles, which stay in flight while the counts are scanned (loads
  // complete in order; all of them unconditional at indices clamped into the
  // tile's slot region, so that no wait sits inside a branch); slots past a
  // tile's count are discarded.
  constexpr int kPreG = 4;  // 256 slots
  const int64_t cbase = (int64_t)bh * n_chunks * chunk;
  uint32_t pk[4][kPreG];
  int32_t pt[4][kPreG];
  int any_bad;
  {
    const int per = (n_chunks + blockDim.x - 1) / blockDim.x;  // <= 2
    const int c0 = tid * per;
    int2 cu[2];
    // the counts go out first (as ordinary loads the compiler issued them after
    // the slot loads, and the scan then waited for every one of those)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const unsigned long long w = __hip_atomic_load(
          reinterpret_cast<const unsigned long long*>(chunk_count) + (int64_t)bh * n_chunks +
              min(c0 + j, n_chunks - 1),
          __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
      cu[j] = make_int2((int)(uint32_t)w, (int)(uint32_t)(w >> 32));
    }
    __builtin_amdgcn_sched_barrier(0);
    {
      const int lane = tid & 63, wave = tid >> 6, nw = blockDim.x >> 6;
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int64_t src = cbase + (int64_t)min(wave + v * nw, n_chunks - 1) * chunk;
#pragma unroll
        for (int u = 0; u < kPreG; ++u) {
          const int j = min(lane + 64 * u, chunk - 1);
          pk[v][u] = cand_key[src + j];
          pt[v][u] = cand_t[src + j];
        }
      }
    }
    // A tile that kept its tokens with another threshold than the published one
    // (not -inf, the tile's own fallback, which keeps every token) may have
    // dropped some of the top k: the head then takes the exact path.
    int cs[2];
    bool bad = false;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const bool real = (j < per) & (c0 + j < n_chunks);  // no branch: the load stays first
      cs[j] = real ? cu[j].x : 0;
      bad |= real && (uint32_t)cu[j].y != thb && (uint32_t)cu[j].y != 0xff800000u;
    }
    int total;
    bool bad_any;
    int pre = block_excl_scan_or(cs[0] + cs[1], bad, tmp, &total, &bad_any);
#pragma unroll
    for (int j = 0; j < 2; ++j)
      if (j < per && c0 + j < n_chunks) {
        off[c0 + j] = pre;
        pre += cs[j];
      }
    if (tid == 0) off[n_chunks] = total;
    any_bad = bad_any ? 1 : 0;
    __syncthreads();  // off
  }
  if (part == 0 && tid == 0) tau_word[bh] = 0ull;  // every tile read it in the score kernel
  // An appended token (scored by the leader; the tiles stop before it) is the
  // head's last position: it follows every tile's candidates in the list.
  const int Ct = off[n_chunks];
  const uint32_t thk = score_key(__uint_as_float(thb) + 0.0f);
  const uint32_t akey = app_key != nullptr ? app_key[bh] : 0u;
  const bool ap = app_key != nullptr && akey >= thk;
  const int C = Ct + (ap ? 1 : 0);
  if (C < top_k || any_bad) {  // the LDS list is unused: it holds the table
    if (part) return;
    select_exact_head<kParts>(codes, alpha, rm, Hkv, bh, n, top_k, sel_lut, sel_inv,
                              comp_key + cbase, comp_t + cbase,
                              reinterpret_cast<int*>(lkey), hist, tmp, sub, &scount, mm,
                              out);
    return;
  }
  // Gather the candidates into one ordered list.  Wave w copies tiles w, w+nw,
  // ...; the first 256 candidates of 4 tiles are loaded before any is stored.
  // Kept in LDS, each candidate's score is also counted in a 2048-bin linear
  // histogram from tau up (bin width set by the leader from its sample).
  const bool in_lds = C <= kSelectLds;
  const float th = __uint_as_float(thb), bsc = bin_scale[bh];
  auto bin_of = [th, bsc](uint32_t key) {
    const float z = (key_score(key) - th) * bsc;  // NaN (no scale) -> bin 0
    return z >= 2047.0f ? 2047 : (z > 0.0f ? (int)z : 0);
  };
  // The list in LDS: each tile's candidates at its offset, positions as offsets
  // within the tile.
  auto gather = [&]() {
    const int lane = tid & 63, wave = tid >> 6, nw = blockDim.x >> 6;
    // Tiles wave + v*nw (v < 4): from the slots loaded before the scan.
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int ci = wave + v * nw;
      if (ci >= n_chunks) continue;
      const int o = off[ci], cnt = off[ci + 1] - o;
      const int64_t src = cbase + (int64_t)ci * chunk;
      const int tb = kSink + ci * chunk;  // the tile's first token
#pragma unroll
      for (int u = 0; u < kPreG; ++u) {
        const int j = lane + 64 * u;
        if (j < cnt) {
          lkey[o + j] = pk[v][u];
          lofs[o + j] = (uint16_t)(pt[v][u] - tb);
        }
        count_bin(hist, j < cnt, bin_of(pk[v][u]));
      }
      for (int j0 = 64 * kPreG; j0 < cnt; j0 += 64) {  // tiles with many candidates
        const int j = j0 + lane;
        const uint32_t key = j < cnt ? cand_key[src + j] : 0u;
        if (j < cnt) {
          lkey[o + j] = key;
          lofs[o + j] = (uint16_t)(cand_t[src + j] - tb);
        }
        count_bin(hist, j < cnt, bin_of(key));
      }
    }
    // Any further tiles (long contexts): their candidates, list entries
    // off[4 nw] .. Ct, as one contiguous run per thread, kGatherRun entries a
    // batch with all of a batch's loads in flight together; a run's tile comes
    // from a binary search of off[], then only crossings read it again.
    const int t4 = 4 * nw;
    if (n_chunks > t4) {
      const int L0 = off[t4], n_rest = Ct - L0;
      const int per = (n_rest + (int)blockDim.x - 1) / (int)blockDim.x;
      const int i0 = L0 + min(n_rest, tid * per), m = min(L0 + n_rest - i0, per);
      int ci = t4;
      for (int step = 1 << 11; step > 0; step >>= 1)
        if (ci + step < n_chunks && off[ci + step] <= i0) ci += step;
      int base = off[ci], next = off[ci + 1];
      for (int b0 = 0; b0 < m; b0 += kGatherRun) {
        uint32_t kk[kGatherRun];
        int32_t tt[kGatherRun];
        int cc[kGatherRun];
#pragma unroll
        for (int j = 0; j < kGatherRun; ++j) {
          const int i = i0 + b0 + j;
          kk[j] = 0u;
          tt[j] = 0;
          cc[j] = ci;
          if (b0 + j < m) {
            while (i >= next) {  // crossing into a later tile
              ++ci;
              base = next;
              next = off[ci + 1];
            }
            const int64_t sl = cbase + (int64_t)ci * chunk + (i - base);
            kk[j] = cand_key[sl];
            tt[j] = cand_t[sl];
            cc[j] = ci;
          }
        }
#pragma unroll
        for (int j = 0; j < kGatherRun; ++j) {
          const int i = i0 + b0 + j;
          if (b0 + j < m) {
            lkey[i] = kk[j];
            lofs[i] = (uint16_t)(tt[j] - (kSink + cc[j] * chunk));
          }
          count_bin(hist, b0 + j < m, bin_of(kk[j]));
        }
      }
    }
  };

  if (!in_lds) {
    if (part) return;
    if (!select_workspace<kParts>(cand_key + cbase, cand_t + cbase, chunk, n_chunks, off, C,
                                  top_k, ap, akey, nt - 1, thk, comp_key + cbase,
                                  comp_t + cbase, hist, tmp, sub, &scount, mm, out)) {
      __syncthreads();
      select_exact_head<kParts>(codes, alpha, rm, Hkv, bh, n, top_k, sel_lut, sel_inv,
                                comp_key + cbase, comp_t + cbase,
                                reinterpret_cast<int*>(lkey), hist, tmp, sub, &scount, mm, out);
    }
    return;
  }
  gather();
  if (ap && tid == 0) {  // its position comes from the emit (past the tiles)
    lkey[Ct] = akey;
    lofs[Ct] = 0;
    count_bin(hist, true, bin_of(akey));
  }
  if (in_lds) {
    __syncthreads();  // publishes the list and the histogram
    // The histogram is scanned for the boundary bin of the k-th largest; the
    // bin's keys (usually a few dozen) go to a sub-list resolved by one wave,
    // or by radix rounds if more than 64.
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
      for (int i = tid; i < C; i += blockDim.x) {
        const uint32_t key = lkey[i];
        if (key >= klo && key <= khi) sub[atomicAdd(&scount, 1)] = key;
      }
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
      r = select_degenerate<kParts>(lkey, C, top_k, hist, tmp, sub, &scount, mm);
    }
    // The list holds every token at or above the published threshold (tiles
    // that gave up waiting kept more); its k-th is the head's k-th only if it
    // is not below that threshold (else some of the top k may be missing).
    if (r.key < thk) {
      if (part) return;
      __syncthreads();  // the LDS list is reused by the exact path
      select_exact_head<kParts>(codes, alpha, rm, Hkv, bh, n, top_k, sel_lut, sel_inv,
                                comp_key + cbase, comp_t + cbase,
                                reinterpret_cast<int*>(lkey), hist, tmp, sub, &scount, mm, out);
      return;
    }
    int32_t* stage = reinterpret_cast<int32_t*>(lkey);
    // runs of at most (kSelectLds / n_parts) / 1024 entries, odd
    constexpr int kRun = (((kSelectLds + n_parts - 1) / n_parts + 1023) / 1024) | 1;
    list_emit<kRun>(lkey, lofs, C, part, n_parts, off, n_chunks, chunk, nt - 1, top_k, r, stage,
                    out, tmp);
  }
}

}  // namespace

hipError_t launch_tables(const ScoreArgs& a, const Launch& s) {
  return launch_k(KID_TABLES, tables_kernel, dim3(a.n_heads), dim3(256), 0, s, a);
}

hipError_t launch_score(const ScoreArgs& a, int chunk, const Launch& s) {
  const dim3 grid((unsigned)a.n_heads * (unsigned)a.n_chunks), block(256);
#define SIKV_SCORE_CASE(UU)                                                                 \
  case 256 * UU:                                                                            \
    if (a.codebook != nullptr)                                                              \
      return a.rm.table != nullptr                                                          \
                 ? launch_k(KID_SCORE, score_kernel<UU, true, true>, grid, block, 0, s, a)  \
                 : launch_k(KID_SCORE, score_kernel<UU, false, true>, grid, block, 0, s, a); \
    return a.rm.table != nullptr                                                            \
               ? launch_k(KID_SCORE, score_kernel<UU, true, false>, grid, block, 0, s, a)   \
               : launch_k(KID_SCORE, score_kernel<UU, false, false>, grid, block, 0, s, a);
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
                         uint32_t* cand_key, int32_t* cand_t, const int2* chunk_count,
                         unsigned long long* tau_word, const float* bin_scale,
                         const uint32_t* app_key, uint32_t* comp_key, int32_t* comp_t,
                         int32_t* idx, const ScoreArgs& ta, const Launch& s) {
  if (n_chunks > kMaxChunks) return hipErrorInvalidValue;
  // Blocks per head: up to four, while the grid (plus one block per head for
  // the attention tables) stays within one 1024-thread block per CU.
  int n_parts = 4;
  while (n_parts > 1 && (int64_t)(n_parts + 1) * B * Hkv > kSelectBlocks) --n_parts;
#define SIKV_SELECT(P)                                                                         \
  launch_k(KID_SELECT, select_kernel<P>, dim3((P + 1) * B * Hkv), dim3(1024), 0, s, codes, alpha, \
           rm, n_tokens, Hkv, seq_lens, sel_lut, sel_inv, top_k, chunk, n_chunks, cand_key,     \
           cand_t, chunk_count, tau_word, bin_scale, app_key, comp_key, comp_t, idx, ta)
  const hipError_t e = n_parts == 4   ? SIKV_SELECT(4)
                       : n_parts == 3 ? SIKV_SELECT(3)
                       : n_parts == 2 ? SIKV_SELECT(2)
                                      : SIKV_SELECT(1);
#undef SIKV_SELECT
  return e;
}

}  // namespace sikv
