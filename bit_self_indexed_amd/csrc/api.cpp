// Host side of the C ABI declared in include/sikv.h: argument validation,
// workspace planning and the launch sequences of each call.  Nothing here
// allocates device memory, synchronises a stream or keeps state between calls:
// each call builds its launch context (stream, optional caller-owned timer)
// from its own arguments.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cmath>
#include <new>
#include <vector>

#include "../../include/sikv.h"
#include "sikv_internal.h"

namespace {

using namespace sikv;

constexpr size_t kAlign = 256;
constexpr int kMaxChunks = 2048;
// Attention grid targets: one block per CU for bf16 values (256-byte rows; fewer
// concurrent gather streams measured faster), two for 2-bit value records
// (64 bytes; more waves to cover the gathers' latency).
constexpr int64_t kAttnBlocksBf16 = 256;
constexpr int64_t kAttnBlocksQv = 512;

inline size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }
inline int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }
inline bool misaligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) != 0; }

// ------------------------------------------------------------------ plans
struct EncodePlan {
  int nblk;          // mean partial tiles per head
  int cb_nblk;       // codebook statistics blocks per head (0: no codebook)
  size_t off_cb, bytes;
};

struct ScorePlan {
  int chunk, n_chunks;
  size_t off_tau, off_bin, off_cnt, off_ckey, off_ct, off_pkey, off_pt, off_tab, off_inv,
      off_lut, off_qmu, off_slog, off_app;
  size_t bytes;
};

struct AttnPlan {
  int cpb, n_splits;
  size_t off_o, off_ml, off_lut, off_qmu, off_slog, bytes;
};

// Attention tables of the query heads, written by the score kernel's leaders
// (or, for a standalone attention call, the tables kernel).
struct AttnTables {
  float* lut;
  float* qmu;
  float* slog;
};

struct DecodePlan {
  ScorePlan sp;
  AttnPlan ap;
  size_t off_idx, off_score, off_attn, bytes;
};

EncodePlan plan_encode(const sikv_cache_desc* c) {
  EncodePlan p;
  const size_t BH = (size_t)c->batch * c->n_kv_heads;
  p.nblk = (int)cdiv(c->n_tokens, kMuTile);
  p.cb_nblk = c->codebook != nullptr ? cb_blocks(c->n_tokens) : 0;
  p.off_cb = align_up(BH * p.nblk * kD * sizeof(float));
  p.bytes = p.off_cb + align_up(BH * p.cb_nblk * kCbStride * sizeof(long long));
  return p;
}

// Tile of the score kernel: 256*U candidates per block, the largest U in
// {8,4,2,1} that still gives >= 1024 blocks (4 per CU), widened if the tile
// count would exceed what the select kernel keeps in LDS.
bool plan_score(const sikv_cache_desc* c, int n_q_heads, ScorePlan* p) {
  const int64_t BH = (int64_t)c->batch * c->n_kv_heads;
  const int64_t n = (int64_t)c->n_tokens - kSink;
  int U = 1;
  for (int u : {8, 4, 2}) {
    if (BH * cdiv(n, 256 * u) >= 1024) {
      U = u;
      break;
    }
  }
  while (cdiv(n, 256 * U) > kMaxChunks && U < 16) U *= 2;
  if (cdiv(n, 256 * U) > kMaxChunks) return false;
  p->chunk = 256 * U;
  p->n_chunks = (int)cdiv(n, p->chunk);
  const size_t cap = (size_t)BH * p->n_chunks * p->chunk;
  size_t o = 0;
  p->off_tau = o;  o += align_up((size_t)BH * sizeof(unsigned long long));
  p->off_bin = o;  o += align_up((size_t)2 * BH * sizeof(float));  // bin scales, then tau
  p->off_cnt = o;  o += align_up((size_t)BH * p->n_chunks * sizeof(int2));
  p->off_ckey = o; o += align_up(cap * sizeof(uint32_t));
  p->off_ct = o;   o += align_up(cap * sizeof(int32_t));
  p->off_pkey = o; o += align_up(cap * sizeof(uint32_t));
  p->off_pt = o;   o += align_up(cap * sizeof(int32_t));
  p->off_tab = o;  o += align_up((size_t)BH * kLut * sizeof(int32_t));
  p->off_inv = o;  o += align_up((size_t)BH * sizeof(float));
  p->off_lut = o;  o += align_up((size_t)c->batch * n_q_heads * kLut * sizeof(float));
  p->off_qmu = o;  o += align_up((size_t)c->batch * n_q_heads * sizeof(float));
  p->off_slog = o; o += align_up((size_t)c->batch * n_q_heads * kSink * sizeof(float));
  p->off_app = o;  o += align_up((size_t)BH * sizeof(uint32_t));
  p->bytes = o;
  return true;
}

// Attention grid: the attended list (64 sinks + k) of each (b, KV head) is cut
// into chunks of kAttnChunk entries; a block of four waves takes chunks_per_block
// consecutive chunks (a multiple of 4, so every wave gets the same count), the
// smallest such that the grid stays within the value format's target (at most
// kAttnMaxCpb, the block's LDS slice of positions): each wave then loops over
// several chunks with its prefetch running ahead, which measured faster than
// more, shorter-lived blocks.  Workspace: the block partials (o, max, sum) and,
// for a standalone call, the query heads' tables.
void plan_attn(const sikv_cache_desc* c, int n_q_heads, int top_k, AttnPlan* p) {
  const int64_t BH = (int64_t)c->batch * c->n_kv_heads;
  const int64_t nch = cdiv((int64_t)kSink + top_k, kAttnChunk);
  const int64_t target = c->vrec != nullptr ? kAttnBlocksQv : kAttnBlocksBf16;
  int64_t cpb = 4;
  while (BH * cdiv(nch, cpb) > target && cpb < kAttnMaxCpb) cpb += 4;
  p->cpb = (int)cpb;
  p->n_splits = (int)cdiv(nch, cpb);
  const size_t rows = (size_t)c->batch * n_q_heads * p->n_splits;
  const size_t hq = (size_t)c->batch * n_q_heads;
  p->off_o = 0;
  p->off_ml = align_up(rows * kD * sizeof(float));
  p->off_lut = p->off_ml + align_up(rows * 2 * sizeof(float));
  p->off_qmu = p->off_lut + align_up(hq * kLut * sizeof(float));
  p->off_slog = p->off_qmu + align_up(hq * sizeof(float));
  p->bytes = p->off_slog + align_up(hq * kSink * sizeof(float));
}

bool plan_decode(const sikv_cache_desc* c, int n_q_heads, int top_k, DecodePlan* p) {
  if (!plan_score(c, n_q_heads, &p->sp)) return false;
  plan_attn(c, n_q_heads, top_k, &p->ap);
  p->off_idx = 0;
  p->off_score = align_up((size_t)c->batch * c->n_kv_heads * top_k * sizeof(int32_t));
  p->off_attn = p->off_score + p->sp.bytes;
  p->bytes = p->off_attn + p->ap.bytes;
  return true;
}

// ------------------------------------------------------------------ validation
// Token-row addressing of the cache's per-token arrays (contiguous or paged).
RowMap rows_of(const sikv_cache_desc* c) {
  RowMap m;
  m.capacity = c->capacity;
  m.table = c->page_table;
  m.lg_page = c->page_table != nullptr ? __builtin_ctz((unsigned)c->page_size) : 0;
  m.pps = c->pages_per_seq;
  m.Hkv = c->n_kv_heads;
  return m;
}

// Rows the attention can address from its per-head bases: a head's capacity
// (contiguous), or the whole pool (paged: its rows are pool rows).
int64_t attn_rows(const sikv_cache_desc* c) {
  return c->page_table != nullptr ? (int64_t)c->n_pages * c->n_kv_heads * c->page_size
                                  : c->capacity;
}

sikv_status check_desc(const sikv_cache_desc* c) {
  if (c == nullptr) return SIKV_ERR_INVALID_ARG;
  if (c->head_dim != kD || c->n_sink != kSink) return SIKV_ERR_UNSUPPORTED;
  if (c->batch < 1 || c->n_kv_heads < 1 || (int64_t)c->batch * c->n_kv_heads > 65535)
    return SIKV_ERR_INVALID_ARG;
  if (c->n_tokens <= kSink || c->capacity < c->n_tokens) return SIKV_ERR_INVALID_ARG;
  if (!c->codes || !c->alpha || !c->mu || !c->k_sink) return SIKV_ERR_INVALID_ARG;
  if (misaligned(c->codes, 16) || misaligned(c->alpha, 4) || misaligned(c->mu, 16) ||
      misaligned(c->k_sink, 16) || misaligned(c->codebook, 16) || misaligned(c->seq_lens, 4))
    return SIKV_ERR_INVALID_ARG;
  if (c->page_table != nullptr) {
    // pages of a power-of-two size >= 256 tokens holding all KV heads; the pool
    // row index fits in int32 (the attention stages rows in LDS as int32)
    const int64_t P = c->page_size;
    if (P < 256 || (P & (P - 1)) != 0 || c->pages_per_seq < 1 || c->n_pages < 1 ||
        misaligned(c->page_table, 4) || (int64_t)c->pages_per_seq * P != c->capacity ||
        (int64_t)c->n_pages * c->n_kv_heads * P > 0x7fffffffLL)
      return SIKV_ERR_INVALID_ARG;
  }
  if ((c->vrec != nullptr || c->v_sink != nullptr) &&
      (!c->vrec || !c->v_sink || misaligned(c->vrec, 64) || misaligned(c->v_sink, 16)))
    return SIKV_ERR_INVALID_ARG;
  if ((c->flags & ~SIKV_FLAG_EXACT_SELECT) != 0) return SIKV_ERR_INVALID_ARG;
  return SIKV_OK;
}

// The launch context of a call on this cache: its stream and the descriptor's
// timer.
Launch ctx(const sikv_cache_desc* c, void* stream) {
  return Launch{static_cast<hipStream_t>(stream), c->timer};
}

bool bad_strides(int64_t sb, int64_t sh, int64_t st) {
  return sb < 0 || sh < 0 || st < 0 || (sb % 8) || (sh % 8) || (st % 8);
}

sikv_status check_v(const sikv_cache_desc* c) {
  if (c->vrec != nullptr) return SIKV_OK;  // quantised values (checked in check_desc)
  if (c->v == nullptr || misaligned(c->v, 16) || bad_strides(c->v_stride_b, c->v_stride_h, c->v_stride_t))
    return SIKV_ERR_INVALID_ARG;
  if (c->page_table != nullptr &&  // paged: the V pool [n_pages][Hkv][page_size][128], dense
      (c->v_stride_t != kD || c->v_stride_h != (int64_t)c->page_size * kD ||
       c->v_stride_b != (int64_t)c->n_kv_heads * c->page_size * kD))
    return SIKV_ERR_INVALID_ARG;
  return SIKV_OK;
}

sikv_status check_query(const sikv_cache_desc* c, const uint16_t* q, int n_q_heads, int top_k) {
  if (q == nullptr || misaligned(q, 16)) return SIKV_ERR_INVALID_ARG;
  if (n_q_heads < 1 || n_q_heads % c->n_kv_heads) return SIKV_ERR_INVALID_ARG;
  if (n_q_heads / c->n_kv_heads > kMaxGroup) return SIKV_ERR_UNSUPPORTED;
  if (top_k < 1 || top_k > c->n_tokens - kSink) return SIKV_ERR_INVALID_ARG;
  return SIKV_OK;
}

sikv_status check_ws(const void* ws, size_t ws_bytes, size_t need) {
  if (need == 0) return SIKV_OK;
  if (ws == nullptr || misaligned(ws, kAlign) || ws_bytes < need) return SIKV_ERR_WORKSPACE;
  return SIKV_OK;
}

#define SIKV_TRY(expr)                               \
  do {                                               \
    if ((expr) != hipSuccess) return SIKV_ERR_HIP;   \
  } while (0)

template <typename T>
T* at(void* ws, size_t off) {
  return reinterpret_cast<T*>(static_cast<char*>(ws) + off);
}

// The score kernel's arguments for this cache and query (workspace pointers
// left null).
ScoreArgs score_args(const sikv_cache_desc* c, const uint16_t* q, int n_q_heads, int top_k) {
  ScoreArgs a{};
  a.n_heads = c->batch * c->n_kv_heads;
  a.codes = c->codes;
  a.alpha = c->alpha;
  a.rm = rows_of(c);
  a.n_tokens = c->n_tokens;
  a.Hkv = c->n_kv_heads;
  a.seq_lens = c->seq_lens;
  a.mu = c->mu;
  a.k_sink = c->k_sink;
  a.codebook = c->codebook;
  a.vrec = c->vrec;
  a.q = q;
  a.n_q_heads = n_q_heads;
  a.G = n_q_heads / c->n_kv_heads;
  a.top_k = top_k;
  a.mode = (c->flags & SIKV_FLAG_EXACT_SELECT) ? 2 : 1;
  return a;
}

// score (leaders: selection table + threshold; tiles: candidates) -> select
// (+ the query heads' attention tables, left in the workspace for a following
// attention).  k_new (may be null): key of each sequence's last token,
// encoded by the score kernel first.
sikv_status run_score_topk(const sikv_cache_desc* c, const uint16_t* q, int n_q_heads, int top_k,
                           int32_t* idx, float* scores_opt, void* ws, const ScorePlan& sp,
                           const uint16_t* k_new, int64_t ksb, int64_t ksh,
                           const uint16_t* v_new, int64_t vnsb, int64_t vnsh, const Launch& s) {
  ScoreArgs a = score_args(c, q, n_q_heads, top_k);
  a.k_new = k_new;
  a.ksb = ksb;
  a.ksh = ksh;
  a.v_new = v_new;
  a.vnsb = vnsb;
  a.vnsh = vnsh;
  a.tau_word = at<unsigned long long>(ws, sp.off_tau);
  a.bin_scale = at<float>(ws, sp.off_bin);
  a.sel_lut = at<int32_t>(ws, sp.off_tab);
  a.sel_inv = at<float>(ws, sp.off_inv);
  a.att_lut = at<float>(ws, sp.off_lut);
  a.att_qmu = at<float>(ws, sp.off_qmu);
  a.att_slog = at<float>(ws, sp.off_slog);
  a.app_key = at<uint32_t>(ws, sp.off_app);
  a.n_chunks = sp.n_chunks;
  a.cand_key = at<uint32_t>(ws, sp.off_ckey);
  a.cand_t = at<int32_t>(ws, sp.off_ct);
  a.chunk_count = at<int2>(ws, sp.off_cnt);
  a.scores_opt = scores_opt;
  SIKV_TRY(launch_score(a, sp.chunk, s));
  SIKV_TRY(launch_select(c->batch, c->n_kv_heads, c->codes, c->alpha, rows_of(c), c->n_tokens,
                         c->seq_lens, a.sel_lut, a.sel_inv, top_k, sp.chunk, sp.n_chunks,
                         a.cand_key, a.cand_t, a.chunk_count, a.tau_word, a.bin_scale,
                         k_new != nullptr ? a.app_key : nullptr, at<uint32_t>(ws, sp.off_pkey),
                         at<int32_t>(ws, sp.off_pt), idx, a, s));
  return SIKV_OK;
}

// Attention (+ split merge).  tab: the query heads' tables; built here by a
// tables launch when the caller has none (standalone call).
sikv_status run_attn(const sikv_cache_desc* c, const uint16_t* q, int n_q_heads,
                     const int32_t* idx, int top_k, float sm_scale, float* out, void* ws,
                     const AttnPlan& ap, const AttnTables* tab, const Launch& s) {
  float* po = at<float>(ws, ap.off_o);
  float* pml = at<float>(ws, ap.off_ml);
  AttnTables own{at<float>(ws, ap.off_lut), at<float>(ws, ap.off_qmu), at<float>(ws, ap.off_slog)};
  if (tab == nullptr) {
    ScoreArgs a = score_args(c, q, n_q_heads, top_k);
    a.att_lut = own.lut;
    a.att_qmu = own.qmu;
    a.att_slog = own.slog;
    SIKV_TRY(launch_tables(a, s));
    tab = &own;
  }
  SIKV_TRY(launch_attn(n_q_heads, c->batch, c->n_kv_heads, c->codes, c->alpha, c->v,
                       c->v_stride_b, c->v_stride_h, c->v_stride_t, c->vrec, c->v_sink,
                       rows_of(c), attn_rows(c), c->n_tokens, c->seq_lens, idx, top_k, tab->lut,
                       tab->qmu, tab->slog, sm_scale, ap.cpb, ap.n_splits, po,
                       pml, s));
  SIKV_TRY(launch_combine(po, pml, c->batch * n_q_heads, ap.n_splits, out, s));
  return SIKV_OK;
}

const char* const g_names[KID_COUNT] = {"mu_partial", "mu_final", "codes", "tables",
                                        "score",      "select",   "attn",  "combine",
                                        "dense",      "copy",     "cb_final", "vcodes",
                                        "kmeans_assign", "dense_scores"};

}  // namespace

// ------------------------------------------------------------------ timer
// The caller-owned kernel timer: event pairs of the launches not yet read, a
// pool of reusable events, and the per-kernel totals.
struct sikv_timer {
  struct Pending {
    int kid;
    hipEvent_t e0, e1;
  };
  std::vector<Pending> pending;
  std::vector<hipEvent_t> pool;
  double ms[KID_COUNT] = {};
  int64_t cnt[KID_COUNT] = {};

  hipEvent_t take() {
    if (!pool.empty()) {
      hipEvent_t e = pool.back();
      pool.pop_back();
      return e;
    }
    hipEvent_t e = nullptr;
    if (hipEventCreate(&e) != hipSuccess) return nullptr;
    return e;
  }
  sikv_status drain() {
    sikv_status st = SIKV_OK;
    for (auto& p : pending) {
      float ms_ = 0.0f;
      if (hipEventSynchronize(p.e1) != hipSuccess ||
          hipEventElapsedTime(&ms_, p.e0, p.e1) != hipSuccess)
        st = SIKV_ERR_HIP;
      else {
        ms[p.kid] += ms_;
        cnt[p.kid] += 1;
      }
      pool.push_back(p.e0);
      pool.push_back(p.e1);
    }
    pending.clear();
    return st;
  }
};

namespace sikv {
void timing_events(::sikv_timer* t, int kernel_id, hipEvent_t* start, hipEvent_t* stop) {
  *start = *stop = nullptr;
  hipEvent_t a = t->take(), b = t->take();
  if (!a || !b) {  // no events: the launch goes untimed
    if (a) t->pool.push_back(a);
    if (b) t->pool.push_back(b);
    return;
  }
  t->pending.push_back({kernel_id, a, b});
  *start = a;
  *stop = b;
}
}  // namespace sikv

namespace {

// ------------------------------------------------------------------ static scratch
// The workspace of the allocation-free entry point: a static array in this
// file's device code, one per GPU (the runtime gives every device its own copy
// when it loads the code object there).  In host code `scratch` names a host
// stand-in, not device memory, so it is never passed to a kernel: its device
// address, per device, comes from hipGetSymbolAddress with that device
// current, once, and is kept in g_scratch.  That per-device address is the
// only state the library keeps; it never changes once set.
constexpr int kMaxDevices = 64;
static __device__ __align__(256) unsigned char scratch[SIKV_STATIC_SCRATCH_BYTES];
std::atomic<void*> g_scratch[kMaxDevices];

// Device address of the scratch of the device `stream` belongs to (the current
// device for the null stream).
sikv_status static_scratch(void* stream, void** out) {
  int dev = 0, cur = 0;
  if (hipGetDevice(&cur) != hipSuccess) return SIKV_ERR_HIP;
  dev = cur;
  if (stream != nullptr && hipStreamGetDevice(static_cast<hipStream_t>(stream), &dev) != hipSuccess)
    return SIKV_ERR_HIP;
  if (dev < 0 || dev >= kMaxDevices) return SIKV_ERR_UNSUPPORTED;
  void* p = g_scratch[dev].load(std::memory_order_acquire);
  if (p == nullptr) {
    if (dev != cur && hipSetDevice(dev) != hipSuccess) return SIKV_ERR_HIP;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (dev != cur && hipSetDevice(cur) != hipSuccess) return SIKV_ERR_HIP;
    if (e != hipSuccess || p == nullptr || misaligned(p, kAlign)) return SIKV_ERR_HIP;
    g_scratch[dev].store(p, std::memory_order_release);  // the same value on any race
  }
  *out = p;
  return SIKV_OK;
}

}  // namespace

// ================================================================== C ABI
extern "C" {

sikv_status sikv_encode(const sikv_cache_desc* c, const uint16_t* k, int64_t k_stride_b,
                        int64_t k_stride_h, int64_t k_stride_t, int32_t t_begin, int32_t t_end,
                        int32_t recompute_mu, void* ws, size_t ws_bytes, void* stream) {
  sikv_status st = check_desc(c);
  if (st != SIKV_OK) return st;
  if (k == nullptr || misaligned(k, 16) || bad_strides(k_stride_b, k_stride_h, k_stride_t))
    return SIKV_ERR_INVALID_ARG;
  if (recompute_mu != 0 && recompute_mu != 1) return SIKV_ERR_INVALID_ARG;
  if (t_begin < 0 || t_end <= t_begin || t_end > c->capacity) return SIKV_ERR_INVALID_ARG;
  const Launch s = ctx(c, stream);
  if (recompute_mu) {
    if (t_begin != 0 || t_end != c->n_tokens) return SIKV_ERR_INVALID_ARG;
    const EncodePlan p = plan_encode(c);
    st = check_ws(ws, ws_bytes, p.bytes);
    if (st != SIKV_OK) return st;
    float* partial = static_cast<float*>(ws);
    SIKV_TRY(launch_mu_partial(k, k_stride_b, k_stride_h, k_stride_t, c->batch, c->n_kv_heads,
                               c->n_tokens, partial, p.nblk, s));
    SIKV_TRY(launch_mu_final(partial, c->batch * c->n_kv_heads, p.nblk, c->n_tokens, c->mu, s));
    if (c->codebook != nullptr) {  // codes + codebook statistics in one pass, then the centres
      long long* part = at<long long>(ws, p.off_cb);
      SIKV_TRY(launch_codes_cb(k, k_stride_b, k_stride_h, k_stride_t, c->batch, c->n_kv_heads,
                               c->n_tokens, rows_of(c), c->mu, c->codes, c->alpha, c->k_sink,
                               c->vrec, part, s));
      SIKV_TRY(launch_cb_final(part, c->batch * c->n_kv_heads, p.cb_nblk, c->codebook, s));
      return SIKV_OK;
    }
  }
  SIKV_TRY(launch_codes(k, k_stride_b, k_stride_h, k_stride_t, c->batch, c->n_kv_heads, t_begin,
                        t_end, rows_of(c), c->mu, c->codes, c->alpha, c->k_sink, c->vrec, s));
  return SIKV_OK;
}

sikv_status sikv_score_topk(const sikv_cache_desc* c, const uint16_t* q, int32_t n_q_heads,
                            int32_t top_k, int32_t* idx, float* scores_opt, void* ws,
                            size_t ws_bytes, void* stream) {
  sikv_status st = check_desc(c);
  if (st != SIKV_OK) return st;
  st = check_query(c, q, n_q_heads, top_k);
  if (st != SIKV_OK) return st;
  if (idx == nullptr || misaligned(idx, 4) || misaligned(scores_opt, 4)) return SIKV_ERR_INVALID_ARG;
  ScorePlan sp;
  if (!plan_score(c, n_q_heads, &sp)) return SIKV_ERR_UNSUPPORTED;
  st = check_ws(ws, ws_bytes, sp.bytes);
  if (st != SIKV_OK) return st;
  return run_score_topk(c, q, n_q_heads, top_k, idx, scores_opt, ws, sp, nullptr, 0, 0, nullptr,
                        0, 0, ctx(c, stream));
}

sikv_status sikv_sparse_attn(const sikv_cache_desc* c, const uint16_t* q, int32_t n_q_heads,
                             const int32_t* idx, int32_t top_k, float sm_scale, float* out,
                             void* ws, size_t ws_bytes, void* stream) {
  sikv_status st = check_desc(c);
  if (st != SIKV_OK) return st;
  st = check_query(c, q, n_q_heads, top_k);
  if (st != SIKV_OK) return st;
  st = check_v(c);
  if (st != SIKV_OK) return st;
  if (idx == nullptr || misaligned(idx, 4) || out == nullptr || misaligned(out, 4))
    return SIKV_ERR_INVALID_ARG;
  if (!std::isfinite(sm_scale)) return SIKV_ERR_INVALID_ARG;
  AttnPlan ap;
  plan_attn(c, n_q_heads, top_k, &ap);
  st = check_ws(ws, ws_bytes, ap.bytes);
  if (st != SIKV_OK) return st;
  return run_attn(c, q, n_q_heads, idx, top_k, sm_scale, out, ws, ap, nullptr, ctx(c, stream));
}

namespace {

// ws == nullptr with use_static: the stream's device's static scratch (after
// every check, so an invalid call touches nothing).
sikv_status decode_step(const sikv_cache_desc* c, const uint16_t* k_new, int64_t ksb, int64_t ksh,
                        const uint16_t* v_new, int64_t vnsb, int64_t vnsh,
                        const uint16_t* q, int32_t n_q_heads, int32_t top_k, float sm_scale,
                        int32_t* idx_out_opt, float* out, void* ws, size_t ws_bytes,
                        void* stream, bool use_static = false) {
  sikv_status st = check_desc(c);
  if (st != SIKV_OK) return st;
  st = check_query(c, q, n_q_heads, top_k);
  if (st != SIKV_OK) return st;
  st = check_v(c);
  if (st != SIKV_OK) return st;
  if (out == nullptr || misaligned(out, 4) || misaligned(idx_out_opt, 4)) return SIKV_ERR_INVALID_ARG;
  if (!std::isfinite(sm_scale)) return SIKV_ERR_INVALID_ARG;
  DecodePlan dp;
  if (!plan_decode(c, n_q_heads, top_k, &dp)) return SIKV_ERR_UNSUPPORTED;
  if (use_static) {
    if (dp.bytes > SIKV_STATIC_SCRATCH_BYTES) return SIKV_ERR_WORKSPACE;
    st = static_scratch(stream, &ws);
    if (st != SIKV_OK) return st;
    ws_bytes = SIKV_STATIC_SCRATCH_BYTES;
  }
  st = check_ws(ws, ws_bytes, dp.bytes);
  if (st != SIKV_OK) return st;
  const Launch s = ctx(c, stream);
  int32_t* idx = idx_out_opt ? idx_out_opt : at<int32_t>(ws, dp.off_idx);
  char* wsc = at<char>(ws, dp.off_score);
  st = run_score_topk(c, q, n_q_heads, top_k, idx, nullptr, wsc, dp.sp, k_new, ksb, ksh, v_new,
                      vnsb, vnsh, s);
  if (st != SIKV_OK) return st;
  const AttnTables tab{at<float>(wsc, dp.sp.off_lut), at<float>(wsc, dp.sp.off_qmu),
                       at<float>(wsc, dp.sp.off_slog)};
  return run_attn(c, q, n_q_heads, idx, top_k, sm_scale, out, at<char>(ws, dp.off_attn), dp.ap,
                  &tab, s);
}
}  // namespace

sikv_status sikv_decode_step(const sikv_cache_desc* c, const uint16_t* q, int32_t n_q_heads,
                             int32_t top_k, float sm_scale, int32_t* idx_out_opt, float* out,
                             void* ws, size_t ws_bytes, void* stream) {
  return decode_step(c, nullptr, 0, 0, nullptr, 0, 0, q, n_q_heads, top_k, sm_scale, idx_out_opt,
                     out, ws, ws_bytes, stream);
}

sikv_status sikv_append_decode_step(const sikv_cache_desc* c, const uint16_t* k_new,
                                    int64_t k_stride_b, int64_t k_stride_h,
                                    const uint16_t* v_new, int64_t v_stride_b,
                                    int64_t v_stride_h, const uint16_t* q, int32_t n_q_heads,
                                    int32_t top_k, float sm_scale, int32_t* idx_out_opt,
                                    float* out, void* ws, size_t ws_bytes, void* stream) {
  if (k_new == nullptr || misaligned(k_new, 16) || bad_strides(k_stride_b, k_stride_h, 0))
    return SIKV_ERR_INVALID_ARG;
  if (v_new != nullptr && (c == nullptr || c->vrec == nullptr || misaligned(v_new, 16) ||
                           bad_strides(v_stride_b, v_stride_h, 0)))
    return SIKV_ERR_INVALID_ARG;
  return decode_step(c, k_new, k_stride_b, k_stride_h, v_new, v_stride_b, v_stride_h, q,
                     n_q_heads, top_k, sm_scale, idx_out_opt, out, ws, ws_bytes, stream);
}

sikv_status sikv_append_decode_step_static(const sikv_cache_desc* c, const uint16_t* k_new,
                                           int64_t k_stride_b, int64_t k_stride_h,
                                           const uint16_t* v_new, int64_t v_stride_b,
                                           int64_t v_stride_h, const uint16_t* q,
                                           int32_t n_q_heads, int32_t top_k, float sm_scale,
                                           int32_t* idx_out_opt, float* out, void* stream) {
  if (k_new == nullptr || misaligned(k_new, 16) || bad_strides(k_stride_b, k_stride_h, 0))
    return SIKV_ERR_INVALID_ARG;
  if (v_new != nullptr && (c == nullptr || c->vrec == nullptr || misaligned(v_new, 16) ||
                           bad_strides(v_stride_b, v_stride_h, 0)))
    return SIKV_ERR_INVALID_ARG;
  return decode_step(c, k_new, k_stride_b, k_stride_h, v_new, v_stride_b, v_stride_h, q,
                     n_q_heads, top_k, sm_scale, idx_out_opt, out, nullptr, 0, stream, true);
}

sikv_status sikv_encode_v(const sikv_cache_desc* c, const uint16_t* v, int64_t v_stride_b,
                          int64_t v_stride_h, int64_t v_stride_t, int32_t t_begin, int32_t t_end,
                          void* stream) {
  const sikv_status st = check_desc(c);
  if (st != SIKV_OK) return st;
  if (c->vrec == nullptr) return SIKV_ERR_INVALID_ARG;
  if (v == nullptr || misaligned(v, 16) || bad_strides(v_stride_b, v_stride_h, v_stride_t))
    return SIKV_ERR_INVALID_ARG;
  if (t_begin < 0 || t_end <= t_begin || t_end > c->capacity) return SIKV_ERR_INVALID_ARG;
  SIKV_TRY(launch_vcodes(v, v_stride_b, v_stride_h, v_stride_t, c->batch, c->n_kv_heads, t_begin,
                         t_end, rows_of(c), c->vrec, c->v_sink, ctx(c, stream)));
  return SIKV_OK;
}

size_t sikv_workspace_bytes(int32_t op, const sikv_cache_desc* c, int32_t n_q_heads,
                            int32_t top_k) {
  if (check_desc(c) != SIKV_OK) return 0;
  switch (op) {
    case SIKV_OP_ENCODE:
      return plan_encode(c).bytes;
    case SIKV_OP_SCORE_TOPK: {
      if (check_query(c, reinterpret_cast<const uint16_t*>(kAlign), n_q_heads, top_k) != SIKV_OK)
        return 0;
      ScorePlan sp;
      return plan_score(c, n_q_heads, &sp) ? sp.bytes : 0;
    }
    case SIKV_OP_SPARSE_ATTN: {
      if (check_query(c, reinterpret_cast<const uint16_t*>(kAlign), n_q_heads, top_k) != SIKV_OK)
        return 0;
      AttnPlan ap;
      plan_attn(c, n_q_heads, top_k, &ap);
      return ap.bytes;
    }
    case SIKV_OP_DECODE_STEP: {
      if (check_query(c, reinterpret_cast<const uint16_t*>(kAlign), n_q_heads, top_k) != SIKV_OK)
        return 0;
      DecodePlan dp;
      return plan_decode(c, n_q_heads, top_k, &dp) ? dp.bytes : 0;
    }
    case SIKV_OP_KMEANS:
      if (c->codebook == nullptr) return 0;
      return align_up((size_t)c->batch * c->n_kv_heads * cb_blocks(c->n_tokens) * kCbStride *
                      sizeof(long long));
    default:
      return 0;
  }
}

const char* sikv_status_str(sikv_status s) {
  switch (s) {
    case SIKV_OK:
      return "ok";
    case SIKV_ERR_INVALID_ARG:
      return "invalid argument (null or misaligned pointer, bad size or range)";
    case SIKV_ERR_UNSUPPORTED:
      return "unsupported (head_dim must be 128, 64 sinks, 1..8 query heads per KV head, "
             "a score tile plan for the context length)";
    case SIKV_ERR_WORKSPACE:
      return "workspace missing, not 256-byte aligned, or smaller than sikv_workspace_bytes";
    case SIKV_ERR_HIP:
      return "HIP kernel launch or runtime call failed";
    default:
      return "unknown status";
  }
}

int32_t sikv_abi_version(void) { return SIKV_ABI_VERSION; }
size_t sikv_desc_size(void) { return sizeof(sikv_cache_desc); }

size_t sikv_dense_workspace_bytes(int32_t batch, int32_t n_kv_heads, int32_t n_q_heads,
                                  int32_t n_tokens) {
  if (batch < 1 || n_kv_heads < 1 || n_q_heads < 1 || n_tokens < 1 || n_q_heads % n_kv_heads)
    return 0;
  const int64_t BH = (int64_t)batch * n_kv_heads;
  const int64_t per_head = cdiv(1024, BH);
  int64_t split = cdiv(cdiv(n_tokens, per_head), 256) * 256;
  if (split < 256) split = 256;
  const int64_t n_splits = cdiv(n_tokens, split);
  const size_t rows = (size_t)batch * n_q_heads * n_splits;
  return align_up(rows * kD * sizeof(float)) + align_up(rows * 2 * sizeof(float));
}

sikv_status sikv_kmeans_codebook(const sikv_cache_desc* c, const uint16_t* k, int64_t k_stride_b,
                                 int64_t k_stride_h, int64_t k_stride_t, int32_t n_iter, void* ws,
                                 size_t ws_bytes, void* stream) {
  sikv_status st = check_desc(c);
  if (st != SIKV_OK) return st;
  if (c->codebook == nullptr || k == nullptr || misaligned(k, 16) ||
      bad_strides(k_stride_b, k_stride_h, k_stride_t) || n_iter < 1 || n_iter > 1000)
    return SIKV_ERR_INVALID_ARG;
  st = check_ws(ws, ws_bytes, sikv_workspace_bytes(SIKV_OP_KMEANS, c, 1, 1));
  if (st != SIKV_OK) return st;
  long long* part = static_cast<long long*>(ws);
  const Launch s = ctx(c, stream);
  const int BH = c->batch * c->n_kv_heads, nblk = cb_blocks(c->n_tokens);
  for (int it = 0; it < n_iter; ++it) {
    SIKV_TRY(launch_kmeans_assign(k, k_stride_b, k_stride_h, k_stride_t, c->batch, c->n_kv_heads,
                                  c->n_tokens, rows_of(c), c->mu, c->alpha,
                                  it == 0 ? nullptr : c->codebook, part, s));
    SIKV_TRY(launch_cb_final(part, BH, nblk, c->codebook, s, it == 0 ? 0 : 1));
  }
  return SIKV_OK;
}

sikv_status sikv_dense_scores(int32_t batch, int32_t n_kv_heads, int32_t n_q_heads,
                              int32_t n_tokens, const uint16_t* q, const uint16_t* k,
                              int64_t k_stride_b, int64_t k_stride_h, int64_t k_stride_t,
                              float* scores, void* stream, sikv_timer* timer) {
  if (batch < 1 || n_kv_heads < 1 || n_q_heads < 1 || n_tokens < 1 || n_q_heads % n_kv_heads ||
      (int64_t)batch * n_kv_heads > 65535)
    return SIKV_ERR_INVALID_ARG;
  if (n_q_heads / n_kv_heads > kMaxGroup) return SIKV_ERR_UNSUPPORTED;
  if (!q || !k || !scores || misaligned(q, 16) || misaligned(k, 16) || misaligned(scores, 4) ||
      bad_strides(k_stride_b, k_stride_h, k_stride_t))
    return SIKV_ERR_INVALID_ARG;
  SIKV_TRY(launch_dense_scores(q, n_q_heads, batch, n_kv_heads, n_tokens, k, k_stride_b,
                               k_stride_h, k_stride_t, scores,
                               Launch{static_cast<hipStream_t>(stream), timer}));
  return SIKV_OK;
}

sikv_status sikv_dense_attn(int32_t batch, int32_t n_kv_heads, int32_t n_q_heads, int32_t n_tokens,
                            const uint16_t* q, const uint16_t* k, int64_t k_stride_b,
                            int64_t k_stride_h, int64_t k_stride_t, const uint16_t* v,
                            int64_t v_stride_b, int64_t v_stride_h, int64_t v_stride_t,
                            float sm_scale, float* out, void* ws, size_t ws_bytes, void* stream,
                            sikv_timer* timer) {
  if (batch < 1 || n_kv_heads < 1 || n_q_heads < 1 || n_tokens < 1 || n_q_heads % n_kv_heads ||
      (int64_t)batch * n_kv_heads > 65535)
    return SIKV_ERR_INVALID_ARG;
  if (n_q_heads / n_kv_heads > kMaxGroup) return SIKV_ERR_UNSUPPORTED;
  if (!q || !k || !v || !out || misaligned(q, 16) || misaligned(k, 16) || misaligned(v, 16) ||
      misaligned(out, 4) || bad_strides(k_stride_b, k_stride_h, k_stride_t) ||
      bad_strides(v_stride_b, v_stride_h, v_stride_t) || !std::isfinite(sm_scale))
    return SIKV_ERR_INVALID_ARG;
  const size_t need = sikv_dense_workspace_bytes(batch, n_kv_heads, n_q_heads, n_tokens);
  sikv_status st = check_ws(ws, ws_bytes, need);
  if (st != SIKV_OK) return st;
  const int64_t BH = (int64_t)batch * n_kv_heads;
  const int64_t per_head = cdiv(1024, BH);
  int64_t split = cdiv(cdiv(n_tokens, per_head), 256) * 256;
  if (split < 256) split = 256;
  const int n_splits = (int)cdiv(n_tokens, split);
  const size_t rows = (size_t)batch * n_q_heads * n_splits;
  float* po = static_cast<float*>(ws);
  float* pml = at<float>(ws, align_up(rows * kD * sizeof(float)));
  const Launch s{static_cast<hipStream_t>(stream), timer};
  SIKV_TRY(launch_dense(q, n_q_heads, batch, n_kv_heads, n_tokens, k, k_stride_b, k_stride_h,
                        k_stride_t, v, v_stride_b, v_stride_h, v_stride_t, sm_scale, (int)split,
                        n_splits, po, pml, s));
  SIKV_TRY(launch_combine(po, pml, batch * n_q_heads, n_splits, out, s));
  return SIKV_OK;
}

sikv_status sikv_stream_copy(void* dst, const void* src, size_t bytes, void* stream,
                             sikv_timer* timer) {
  if (!dst || !src || bytes == 0 || bytes % 16 || misaligned(dst, 16) || misaligned(src, 16))
    return SIKV_ERR_INVALID_ARG;
  SIKV_TRY(launch_copy(dst, src, bytes, Launch{static_cast<hipStream_t>(stream), timer}));
  return SIKV_OK;
}

sikv_status sikv_timer_create(sikv_timer** out) {
  if (out == nullptr) return SIKV_ERR_INVALID_ARG;
  *out = new (std::nothrow) sikv_timer();
  return *out != nullptr ? SIKV_OK : SIKV_ERR_HIP;
}

sikv_status sikv_timer_destroy(sikv_timer* t) {
  if (t == nullptr) return SIKV_OK;
  sikv_status st = t->drain();
  for (hipEvent_t e : t->pool)
    if (hipEventDestroy(e) != hipSuccess) st = SIKV_ERR_HIP;
  delete t;
  return st;
}

sikv_status sikv_timer_reset(sikv_timer* t) {
  if (t == nullptr) return SIKV_ERR_INVALID_ARG;
  const sikv_status st = t->drain();
  for (int i = 0; i < KID_COUNT; ++i) {
    t->ms[i] = 0.0;
    t->cnt[i] = 0;
  }
  return st;
}

int32_t sikv_timer_count(void) { return KID_COUNT; }

const char* sikv_timer_name(int32_t id) {
  return (id >= 0 && id < KID_COUNT) ? g_names[id] : "unknown";
}

sikv_status sikv_timer_read(sikv_timer* t, int32_t id, int64_t* launches, double* total_ms) {
  if (t == nullptr || id < 0 || id >= KID_COUNT || !launches || !total_ms)
    return SIKV_ERR_INVALID_ARG;
  const sikv_status st = t->drain();
  *launches = t->cnt[id];
  *total_ms = t->ms[id];
  return st;
}

}  // extern "C"
