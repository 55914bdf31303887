// Internal declarations of the gfx950 kernels and their host launchers.
//
// Method: "Self-Indexing KVCache: Predicting Sparse Attention from Compressed
// Keys" (web summary, technical part, §2.1 items 1-4).  Every kernel is written
// for wave64 CDNA4: one lane per token where a token is processed whole (score,
// attention logits), 16 lanes x 16 bytes per 256-byte row where a row is
// streamed (encode, value gathers).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace sikv {

constexpr int kD = 128;          // head dim
constexpr int kSink = 64;        // full-precision sink tokens (§2.1 item 3)
constexpr int kCodeBytes = 16;   // 1 bit per channel
constexpr int kSub = 32;         // 4-dim sub-vectors per key (§2.1 item 1)
constexpr int kLut = kSub * 16;  // table entries per query
constexpr int kMaxGroup = 8;

// Kernel ids for the optional timing facility.
enum KernelId {
  KID_MU_PARTIAL = 0,
  KID_MU_FINAL,
  KID_CODES,
  KID_SAMPLE,
  KID_SCORE,
  KID_SELECT,
  KID_ATTN,
  KID_COMBINE,
  KID_DENSE,
  KID_COPY,
  KID_COUNT
};

// ---------------------------------------------------------------- device helpers
__device__ __forceinline__ float bf16lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Order-preserving map of fp32 (no NaN) to uint32.
__device__ __forceinline__ uint32_t score_key(float s) {
  uint32_t u = __float_as_uint(s);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float key_score(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7fffffffu) : ~k);
}

// Selection query (sum of the KV head's G query heads, fp32, g ascending) and its
// look-up table, in LDS: lut[j*16 + p] = ((+-x0 +- x1) +- x2) +- x3 with x_i the
// query's channel 4j+i and the sign of x_i negative iff bit i of p is set
// (§2.1 item 2: a query piece dotted with the 16 sign vertices).  Every thread of
// the block must call it; ends with a barrier.
__device__ __forceinline__ void build_selection_lut(const uint16_t* __restrict__ q, int b, int h,
                                                    int n_q_heads, int G, float* qbar,
                                                    float* lut) {
  const int tid = threadIdx.x;
  if (tid < kD) {
    const uint16_t* qp = q + ((size_t)b * n_q_heads + (size_t)h * G) * kD + tid;
    float s = __uint_as_float((uint32_t)qp[0] << 16);
    for (int g = 1; g < G; ++g) s += __uint_as_float((uint32_t)qp[(size_t)g * kD] << 16);
    qbar[tid] = s;
  }
  __syncthreads();
  for (int e = tid; e < kLut; e += blockDim.x) {
    const int j = e >> 4, p = e & 15;
    const float x0 = qbar[4 * j], x1 = qbar[4 * j + 1], x2 = qbar[4 * j + 2], x3 = qbar[4 * j + 3];
    float v = (p & 1) ? -x0 : x0;
    v += (p & 2) ? -x1 : x1;
    v += (p & 4) ? -x2 : x2;
    v += (p & 8) ? -x3 : x3;
    lut[e] = v;
  }
  __syncthreads();
}

// Sum over the 8 sub-vectors held in one 32-bit word of a code (sub-vectors
// 8w..8w+7).  The nibbles are moved to byte lanes already multiplied by 4 (even
// nibbles from d << 2, odd ones from d >> 2), so each look-up needs a single
// byte extract for its LDS address; the table slice of sub-vector j starts at
// byte 64*j.
__device__ __forceinline__ float lut_word(const float* __restrict__ lutw, uint32_t d) {
  const uint32_t e = (d << 2) & 0x3c3c3c3cu;
  const uint32_t o = (d >> 2) & 0x3c3c3c3cu;
  const char* L = reinterpret_cast<const char*>(lutw);
  float a = *reinterpret_cast<const float*>(L + 0 * 64 + (e & 0xffu));
  float c = *reinterpret_cast<const float*>(L + 1 * 64 + (o & 0xffu));
  a += *reinterpret_cast<const float*>(L + 2 * 64 + ((e >> 8) & 0xffu));
  c += *reinterpret_cast<const float*>(L + 3 * 64 + ((o >> 8) & 0xffu));
  a += *reinterpret_cast<const float*>(L + 4 * 64 + ((e >> 16) & 0xffu));
  c += *reinterpret_cast<const float*>(L + 5 * 64 + ((o >> 16) & 0xffu));
  a += *reinterpret_cast<const float*>(L + 6 * 64 + (e >> 24));
  c += *reinterpret_cast<const float*>(L + 7 * 64 + (o >> 24));
  return a + c;
}

// Compressed-domain score of one token: sum_j LUT[j][nibble_j] (fixed order:
// per word as in lut_word, words combined as (w0 + w1) + (w2 + w3)).  The
// caller multiplies by the token's scale.
__device__ __forceinline__ float lut_dot(const float* __restrict__ lut, uint4 c) {
  const float s0 = lut_word(lut + 0 * 128, c.x);
  const float s1 = lut_word(lut + 1 * 128, c.y);
  const float s2 = lut_word(lut + 2 * 128, c.z);
  const float s3 = lut_word(lut + 3 * 128, c.w);
  return (s0 + s1) + (s2 + s3);
}

// Selection score as used by every kernel that ranks tokens; -0 is mapped to +0
// so that equal scores have equal keys.
__device__ __forceinline__ float selection_score(const float* __restrict__ lut, uint4 c, float a) {
  return a * lut_dot(lut, c) + 0.0f;
}

// Number of set bits of a 64-lane ballot below this lane.
__device__ __forceinline__ int ballot_rank(uint64_t m) {
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32),
                                   __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
}

// ---------------------------------------------------------------- host launchers
// encode.hip
hipError_t launch_mu_partial(const uint16_t* k, int64_t sb, int64_t sh, int64_t st, int B, int Hkv,
                             int n_tokens, float* partial, int nblk, hipStream_t s);
hipError_t launch_mu_final(const float* partial, int BH, int nblk, int n_tokens, float* mu,
                           hipStream_t s);
hipError_t launch_codes(const uint16_t* k, int64_t sb, int64_t sh, int64_t st, int B, int Hkv,
                        int t_begin, int t_end, int capacity, const float* mu, uint8_t* codes,
                        float* alpha, uint16_t* k_sink, hipStream_t s);

// score.hip
hipError_t launch_sample(const uint16_t* q, int n_q_heads, int B, int Hkv, const uint8_t* codes,
                         const float* alpha, int capacity, int n_tokens, int top_k, int force_exact,
                         float* tau, hipStream_t s);
hipError_t launch_score(const uint16_t* q, int n_q_heads, int B, int Hkv, const uint8_t* codes,
                        const float* alpha, int capacity, int n_tokens, const float* tau,
                        int chunk, int n_chunks, uint32_t* cand_key, int32_t* cand_t,
                        int32_t* chunk_count, float* scores_opt, hipStream_t s);
hipError_t launch_select(const uint16_t* q, int n_q_heads, int B, int Hkv, const uint8_t* codes,
                         const float* alpha, int capacity, int n_tokens, int top_k, int chunk,
                         int n_chunks, uint32_t* cand_key, int32_t* cand_t,
                         const int32_t* chunk_count, uint32_t* comp_key, int32_t* comp_t,
                         int32_t* idx, hipStream_t s);

// attn.hip
hipError_t launch_attn(const uint16_t* q, int n_q_heads, int B, int Hkv, const uint8_t* codes,
                       const float* alpha, const float* mu, const uint16_t* k_sink,
                       const uint16_t* v, int64_t vsb, int64_t vsh, int64_t vst, int capacity,
                       int n_tokens, const int32_t* idx, int top_k, float sm_scale, int split,
                       int n_splits, float* part_o, float* part_ml, hipStream_t s);
hipError_t launch_combine(const float* part_o, const float* part_ml, int BHq, int n_splits,
                          float* out, hipStream_t s);

// dense.hip
hipError_t launch_dense(const uint16_t* q, int n_q_heads, int B, int Hkv, int n_tokens,
                        const uint16_t* k, int64_t ksb, int64_t ksh, int64_t kst,
                        const uint16_t* v, int64_t vsb, int64_t vsh, int64_t vst, float sm_scale,
                        int split, int n_splits, float* part_o, float* part_ml, hipStream_t s);

// util.hip
hipError_t launch_copy(void* dst, const void* src, size_t bytes, hipStream_t s);

// Timing facility (api.cpp): launch through these so a timed run can bracket
// every kernel with events.  Returns the events to use (or null ones).
void timing_events(int kernel_id, hipEvent_t* start, hipEvent_t* stop);

// Helper used by the launchers: launch with optional start/stop events.
template <typename... KArgs, typename... Args>
inline hipError_t launch_k(int kid, void (*kern)(KArgs...), dim3 grid, dim3 block, size_t shmem,
                           hipStream_t s, Args... args) {
  hipEvent_t e0 = nullptr, e1 = nullptr;
  timing_events(kid, &e0, &e1);
  if (e0) {
    hipExtLaunchKernelGGL(kern, grid, block, shmem, s, e0, e1, 0, args...);
  } else {
    hipLaunchKernelGGL(kern, grid, block, shmem, s, args...);
  }
  return hipGetLastError();
}

}  // namespace sikv
