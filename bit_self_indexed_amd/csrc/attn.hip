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
//            sink entries take the exact bf16-key logits made beside the
//            selection (the select launch's table blocks);
//   softmax  chunk max per head over 32 lanes, running max / sum update,
//            probabilities through a wave-private LDS row;
//   P.V      16-lane group r owns entries r, r+4, ..., r+28: 16 bytes (8 bf16
//            channels) of each V row per lane, fp32 FMAs into G x 8 accumulators;
//            2-bit values with G <= 4: matrix-core products (below).
// The block first copies its slice of the position list into LDS (one round
// trip), so a wave can issue all loads of its next chunk (codes, scales and V
// rows) right after the current chunk's have arrived, before computing it.
// Measured on the 128K shape (random positions, 8 rotating layers): ~25 us for
// blocks of 10 chunks per wave; contiguous positions take ~8 us less and a
// single resident layer another ~5 us less, so the time is set by the random
// gathers themselves (DRAM pages, translation); without the P.V arithmetic or
// without the logit look-ups (timing-only builds) it is ~1.5 us shorter each,
// and fewer, longer-lived blocks are slower by ~1.7 us per extra chunk per
// wave.  The combine kernel then merges the blocks' partials.
// (A last-block-merges variant needs device-scope fences, which on gfx950 write
// back and invalidate the whole L2 of the XCD in every block: far slower than
// one more launch.)
#include <hip/hip_ext.h>

#include "sikv_internal.h"

namespace sikv {

namespace {

constexpr int kRows = kAttnChunk / 4;  // V rows per 16-lane group per chunk

// P.V of the 2-bit-value path on the matrix cores (G <= 4), per chunk of 32
// entries, as v_mfma_f32_16x16x32_f16 products with K = the chunk's entries
// (K index = entry index e):
//   out[g][c] = sum_e p[g][e] (z[e][c/32] + s[e][c/32] q[e][c])
//             = sum_e A[4 (c/32) + g][e] B[e][c] + sum_e p[g][e] (z - 4 s)[e][c/32],
//   A[4 gc + g][e] = p[g][e] s[e][gc] * 2^10 (fp16, as a high and a low part),
//   B[e][c] = 4 + q[e][c] (exact in fp16: bits 0x4400 | q << 8).
// Row 4 gc + g of A pairs head g with channel group gc, so the 16 rows carry
// all four groups; of each product's output only the rows of the block's own
// channel group are kept.  The offset 4 keeps B away from fp16 subnormals
// (which the matrix cores do not multiply exactly) and 2^10 keeps A's small
// terms normal; a chunk whose value scale exceeds kMfScaleMax (A's high part
// would overflow fp16) takes the FMA path instead.
constexpr bool mf_path(int G, bool QV) { return QV && G <= 4; }
constexpr float kMfScale = 1024.0f;
constexpr float kMfScaleMax = 63.0f;
constexpr int kBtStride = kD + 8;  // halves per staged B row (padded: rows 16 banks apart)
typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float float4v __attribute__((ext_vector_type(4)));
typedef float float8v __attribute__((ext_vector_type(8)));
typedef short short4v __attribute__((ext_vector_type(4)));
typedef short short8v __attribute__((ext_vector_type(8)));

// Per-wave LDS of the matrix-core path: the chunk's probabilities by head, the
// value scales by channel group, and B (entry rows of 128 halves).
struct MfLds {
  float pT[4][kAttnChunk];
  float sg[4][kAttnChunk];
  __attribute__((aligned(16))) _Float16 bt[kAttnChunk][kBtStride];
};

__device__ __forceinline__ void wave_sync_lds() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Logit tables of a pair of query heads (2i, 2i + 1), interleaved: entry e of
// head 2i + par at float 2e + par, so sub-vector j's 16 entries span 128 bytes.
// The two halves of a wave serve the two heads of a pair: a lane's offset into
// the pair table (par * 4 bytes) is set into the nibbles' byte offsets
// (nibble * 8) by the same and-or that masks them, and each look-up's address
// is then one byte extract with the rest an immediate offset.  Same look-ups
// and the same order of additions as lut_word / lut_dot.
__device__ __forceinline__ float lut_word_pair(const float* __restrict__ lutw, uint32_t d,
                                               uint32_t par4) {
  const uint32_t e = ((d << 3) & 0x78787878u) | par4;
  const uint32_t o = ((d >> 1) & 0x78787878u) | par4;
  const char* L = reinterpret_cast<const char*>(lutw);
  float a = *reinterpret_cast<const float*>(L + 0 * 128 + byte_of(e, 0));
  float c = *reinterpret_cast<const float*>(L + 1 * 128 + byte_of(o, 0));
  a += *reinterpret_cast<const float*>(L + 2 * 128 + byte_of(e, 1));
  c += *reinterpret_cast<const float*>(L + 3 * 128 + byte_of(o, 1));
  a += *reinterpret_cast<const float*>(L + 4 * 128 + byte_of(e, 2));
  c += *reinterpret_cast<const float*>(L + 5 * 128 + byte_of(o, 2));
  a += *reinterpret_cast<const float*>(L + 6 * 128 + byte_of(e, 3));
  c += *reinterpret_cast<const float*>(L + 7 * 128 + byte_of(o, 3));
  return a + c;
}
__device__ __forceinline__ float lut_dot_pair(const float* __restrict__ lutp, uint4 c,
                                              uint32_t par4) {
  return (lut_word_pair(lutp, c.x, par4) + lut_word_pair(lutp + 256, c.y, par4)) +
         (lut_word_pair(lutp + 512, c.z, par4) + lut_word_pair(lutp + 768, c.w, par4));
}

// Where a lane finds its inputs: codes / scales of the head, bf16 V at this
// lane's channels (row stride vst), or (quantised values) the head's 2-bit
// codes (32 B per token), (scale, zero) words (4 per token) and bf16 sink rows.
struct Src {
  const uint8_t* codes;
  const float* alpha;
  const float* slog;     // sink logits of the block's G query heads [G][64]
  const uint16_t* vb;
  int64_t vst;
  const uint8_t* vrec;    // quantised values: the head's 64-byte value records
  const uint16_t* vsk;
  const char* vbase;      // bf16 V rows without the lane's column offset
  uint32_t vstb, vlane;   // row stride and the lane's column offset, in bytes
};

// A load at a 32-bit byte offset from a block-uniform base: one scalar base
// plus one VGPR per load, where a 64-bit row times stride product costs four
// multiplies.  Used when every row the kernel can address lies within 2^24
// rows and 4 GiB of its base (checked on the host).
template <typename T>
__device__ __forceinline__ T ld32(const void* base, uint32_t off) {
  return *reinterpret_cast<const T*>(reinterpret_cast<const char*>(base) + off);
}

// Registers of one chunk for one lane: the logit inputs of entry (lane & 31)
// and the V data of the 16-lane group's 8 rows (entries grp, grp+4, ...).
// Quantised values of a non-sink chunk: v[u].x holds the lane's 16 code bits,
// v[u].y its group's scale/zero word.
template <int G>
struct Chunk {
  uint4 code;
  float a;
  float sl[(G + 1) / 2];  // sink logits (sink chunks)
  uint4 v[kRows];
};

// Issues every load of chunk c (block-local lc).  sidx holds the rows of the
// block's entries, relative to the Src bases (entries past the list end repeat
// its last), so every address is a real row.  A sink chunk reads the sink
// logits (and, quantised, the bf16 sink rows) by entry index instead.
template <int G, bool QV, bool kO32>
__device__ __forceinline__ void load_chunk(Chunk<G>& x, int c, int lc, bool sink,
                                           const int* sidx, int lane, const Src& src) {
  const int el = lane & 31, half = lane >> 5, grp = lane >> 4, seg = lane & 15;
  const int t = sidx[lc * kAttnChunk + el];
  if (sink) {
    x.code = make_uint4(0u, 0u, 0u, 0u);
    x.a = 0.0f;
#pragma unroll
    for (int i = 0; i < (G + 1) / 2; ++i)
      x.sl[i] = src.slog[min(2 * i + half, G - 1) * kSink + c * kAttnChunk + el];
  } else {
    // quantised values: the key code copy in the token's value record, which the
    // V loads below fetch anyway
    if constexpr (kO32) {
      const uint32_t ut = (uint32_t)t;
      x.code = QV ? ld32<uint4>(src.vrec, ut * kVRecBytes + kVRecCode)
                  : ld32<uint4>(src.codes, ut * kCodeBytes);
      x.a = ld32<float>(src.alpha, ut * 4u);
    } else {
      x.code = QV ? *reinterpret_cast<const uint4*>(src.vrec + (int64_t)t * kVRecBytes + kVRecCode)
                  : *reinterpret_cast<const uint4*>(src.codes + (int64_t)t * kCodeBytes);
      x.a = src.alpha[t];
    }
#pragma unroll
    for (int i = 0; i < (G + 1) / 2; ++i) x.sl[i] = 0.0f;
  }
#pragma unroll
  for (int u = 0; u < kRows; ++u) {
    const int tu = sidx[lc * kAttnChunk + grp + 4 * u];
    if (!QV) {
      if constexpr (kO32)
        x.v[u] = ld32<uint4>(src.vbase, __umul24((uint32_t)tu, src.vstb) + src.vlane);
      else
        x.v[u] = *reinterpret_cast<const uint4*>(src.vb + (int64_t)tu * src.vst);
    } else if (sink) {
      x.v[u] = *reinterpret_cast<const uint4*>(src.vsk + (int64_t)(c * kAttnChunk + grp + 4 * u) * kD);
    } else {
      if constexpr (kO32) {
        const uint32_t r = (uint32_t)tu * kVRecBytes;
        x.v[u].x = ld32<uint16_t>(src.vrec, r + 2 * seg);
        x.v[u].y = ld32<uint32_t>(src.vrec, r + kVRecSz + 4 * (seg >> 2));
      } else {
        const uint8_t* rec = src.vrec + (int64_t)tu * kVRecBytes;
        x.v[u].x = *reinterpret_cast<const uint16_t*>(rec + 2 * seg);
        x.v[u].y = *reinterpret_cast<const uint32_t*>(rec + kVRecSz + 4 * (seg >> 2));
      }
      x.v[u].z = 0u;
      x.v[u].w = 0u;
    }
  }
}

// Online-softmax state of one wave (heads of parity `half` in this half).
template <int G>
struct Acc {
  float m[G], lsum[(G + 1) / 2], acc[G][8], zacc[G];  // zacc: sum of p * zero point (QV)
  float4v d[8];  // matrix-core path: one 16x16 output block per 16 channels
};

template <int G, bool QV>
__device__ __forceinline__ void process_chunk(Acc<G>& st, const Chunk<G>& x, bool sink, bool live,
                                              const float (*lutp)[2 * kLut], const float* qmu,
                                              float sm_log2, float (*pbw)[G], MfLds* mf,
                                              int lane) {
  constexpr int GH = (G + 1) / 2;
  constexpr bool kMf = mf_path(G, QV);
  const int el = lane & 31, half = lane >> 5, grp = lane >> 4, seg = lane & 15;
  // matrix-core path for this chunk: stage B and the group scales first (they
  // do not depend on the probabilities); a scale above kMfScaleMax anywhere in
  // the chunk sends it to the FMA path
  bool use_mf = false;
  if constexpr (kMf) {
    if (!sink) {
      bool big = false;
#pragma unroll
      for (int u = 0; u < kRows; ++u) {
        const uint32_t sz = x.v[u].y;
        big |= !(fabsf(__half2float(__ushort_as_half((unsigned short)(sz & 0xffffu)))) <= kMfScaleMax);
      }
      use_mf = __ballot(big) == 0ull;
      if (use_mf) {
#pragma unroll
        for (int u = 0; u < kRows; ++u) {
          const int eu = grp + 4 * u;
          const uint32_t y = x.v[u].x & 0xffffu, t = y | (y << 14);
          // dword k: channels 2k, 2k+1 of the lane's eight, each 4 + q as fp16
          uint4 w;
          w.x = ((t << 8) & 0x03000300u) | 0x44004400u;
          w.y = ((t << 4) & 0x03000300u) | 0x44004400u;
          w.z = (t & 0x03000300u) | 0x44004400u;
          w.w = ((t >> 4) & 0x03000300u) | 0x44004400u;
          *reinterpret_cast<uint4*>(&mf->bt[eu][8 * seg]) = w;
          if ((seg & 3) == 0)
            mf->sg[seg >> 2][eu] = __half2float(__ushort_as_half((unsigned short)(x.v[u].y & 0xffffu)));
        }
      }
    }
  }
  // logits (log2 domain) of this lane's heads g = 2i + half (with G odd, the
  // last pair's second slot is a zero table whose logits are masked)
  float lg[GH];
  const uint32_t par4 = half ? 0x04040404u : 0u;
#pragma unroll
  for (int i = 0; i < GH; ++i) {
    const float dot = sink ? x.sl[i] : fmaf(x.a, lut_dot_pair(lutp[i], x.code, par4), qmu[i]);
    lg[i] = (live && 2 * i + half < G) ? dot * sm_log2 : -INFINITY;
  }
  // chunk max per head: heads of parity `half` live in this half of the wave
  // (row maxima by DPP, then the four rows' values read as scalars)
  float cm[GH], co[GH];
#pragma unroll
  for (int i = 0; i < GH; ++i) {
    const float v = row_allreduce(lg[i], [](float a, float b) { return fmaxf(a, b); });
    const float h0 = fmaxf(readlane(v, 0), readlane(v, 16));
    const float h1 = fmaxf(readlane(v, 32), readlane(v, 48));
    cm[i] = half ? h1 : h0;
    co[i] = half ? h0 : h1;
  }
  // The running maxima are the same in every lane (lane reads), so whether a
  // chunk raises any of them is a wave-wide branch; one that raises none keeps
  // the accumulators as they are (its factors would all be exactly 1).
  float sc[G], mn[G];
  bool grow = false;
#pragma unroll
  for (int g = 0; g < G; ++g) {
    const float mx = ((g & 1) == half) ? cm[g >> 1] : co[g >> 1];
    mn[g] = fmaxf(st.m[g], mx);
    grow |= mn[g] != st.m[g];
    sc[g] = 1.0f;
  }
  if (__builtin_amdgcn_ballot_w64(grow) != 0ull) {
#pragma unroll
    for (int g = 0; g < G; ++g) {
      sc[g] = exp2f(st.m[g] - mn[g]);
      st.m[g] = mn[g];
#pragma unroll
      for (int i = 0; i < 8; ++i) st.acc[g][i] *= sc[g];
      if (QV) st.zacc[g] *= sc[g];
    }
    if constexpr (kMf) {  // output rows 4 * (lane / 16) + j are head j of a channel group
#pragma unroll
      for (int nb = 0; nb < 8; ++nb)
#pragma unroll
        for (int j = 0; j < 4; ++j) st.d[nb][j] *= j < G ? sc[j] : 0.0f;
    }
  }
#pragma unroll
  for (int i = 0; i < GH; ++i) {
    const int g1 = min(2 * i + 1, G - 1);
    const float m_odd = st.m[g1], m_even = st.m[2 * i];  // values, not addresses, are selected
    const float s_odd = sc[g1], s_even = sc[2 * i];
    const float mg = half ? m_odd : m_even;
    const float sg = half ? s_odd : s_even;
    const float p = exp2f(lg[i] - mg);
    st.lsum[i] = fmaf(st.lsum[i], sg, p);
    if (2 * i + half < G) {
      pbw[el][2 * i + half] = p;
      if constexpr (kMf) mf->pT[2 * i + half][el] = p;
    }
  }
  wave_sync_lds();
  // P.V
  if constexpr (kMf) {
    if (use_mf) {
      // A (lane: row m = lane % 16 = 4 gc + g, entries 8 (lane / 16) .. + 7)
      const int am = lane & 15, agc = am >> 2, ag = am & 3, k0 = 8 * (lane >> 4);
      float8v af;
#pragma unroll
      for (int j = 0; j < 8; ++j)
        af[j] = ag < G ? mf->pT[ag < G ? ag : 0][k0 + j] * mf->sg[agc][k0 + j] * kMfScale : 0.0f;
      const half8 ahi = __builtin_convertvector(af, half8);
      const half8 alo = __builtin_convertvector(af - __builtin_convertvector(ahi, float8v), half8);
      // B by transposed LDS reads: lane (k4 = lane / 16, r = lane % 16) points at
      // entry k0 + 4 h + r / 4, channels 16 nb + 4 (r % 4) .. + 3, and receives
      // entries k0 + 4 h .. + 3 of channel 16 nb + r
      const int r = lane & 15;
#pragma unroll
      for (int nb = 0; nb < 8; ++nb) {
        short4v t4[2];
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
          const _Float16* src = &mf->bt[k0 + 4 * hh + (r >> 2)][16 * nb + 4 * (r & 3)];
          t4[hh] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (__attribute__((address_space(3))) short4v*)(
                  (__attribute__((address_space(3))) void*)src));
        }
        // whole-vector bit casts: building the fragment element by element from the
        // transposed reads compiles to wrong register moves
        const half8 bv = __builtin_bit_cast(
            half8, __builtin_shufflevector(t4[0], t4[1], 0, 1, 2, 3, 4, 5, 6, 7));
        st.d[nb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ahi, bv, st.d[nb], 0, 0, 0);
        st.d[nb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(alo, bv, st.d[nb], 0, 0, 0);
      }
      // zero points: sum_e p (z - 4 s), per lane for its channel group
#pragma unroll
      for (int u = 0; u < kRows; ++u) {
        const int eu = grp + 4 * u;
        const uint32_t sz = x.v[u].y;
        const float sv = __half2float(__ushort_as_half((unsigned short)(sz & 0xffffu)));
        const float zv = __half2float(__ushort_as_half((unsigned short)(sz >> 16)));
        const float z4 = fmaf(-4.0f, sv, zv);
#pragma unroll
        for (int g = 0; g < G; ++g) st.zacc[g] = fmaf(pbw[eu][g], z4, st.zacc[g]);
      }
      wave_sync_lds();
      return;
    }
  }
  if (!QV || sink) {
#pragma unroll
    for (int u = 0; u < kRows; ++u) {
      const int eu = grp + 4 * u;
      const uint4 w = x.v[u];
      const float v[8] = {bf16lo(w.x), bf16hi(w.x), bf16lo(w.y), bf16hi(w.y),
                          bf16lo(w.z), bf16hi(w.z), bf16lo(w.w), bf16hi(w.w)};
#pragma unroll
      for (int g = 0; g < G; ++g) {
        const float p = pbw[eu][g];
#pragma unroll
        for (int i = 0; i < 8; ++i) st.acc[g][i] = fmaf(p, v[i], st.acc[g][i]);
      }
    }
  } else {
    // v = z + q * s: acc += (p * s) * q per channel, p * z once per row
#pragma unroll
    for (int u = 0; u < kRows; ++u) {
      const int eu = grp + 4 * u;
      const uint32_t qb = x.v[u].x, sz = x.v[u].y;
      const float sv = __half2float(__ushort_as_half((unsigned short)(sz & 0xffffu)));
      const float zv = __half2float(__ushort_as_half((unsigned short)(sz >> 16)));
      float qf[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) qf[i] = (float)((qb >> (2 * i)) & 3u);
#pragma unroll
      for (int g = 0; g < G; ++g) {
        const float p = pbw[eu][g];
        const float ps = p * sv;
        st.zacc[g] = fmaf(p, zv, st.zacc[g]);
#pragma unroll
        for (int i = 0; i < 8; ++i) st.acc[g][i] = fmaf(ps, qf[i], st.acc[g][i]);
      }
    }
  }
  wave_sync_lds();
}

template <int G, bool QV, bool kO32>
__global__ __launch_bounds__(256, 2) void attn_kernel(
    int n_q_heads, int Hkv, const uint8_t* __restrict__ codes, const float* __restrict__ alpha,
    const uint16_t* __restrict__ v, int64_t vsb, int64_t vsh, int64_t vst,
    const uint8_t* __restrict__ vrec,
    const uint16_t* __restrict__ vsink, RowMap rm, int n_tokens,
    const int32_t* __restrict__ seq_lens, const int32_t* __restrict__ idx, int top_k,
    const float* __restrict__ att_lut,
    const float* __restrict__ att_qmu, const float* __restrict__ att_slog, float sm_log2,
    int cpb, int n_splits, float* __restrict__ part_o, float* __restrict__ part_ml) {
  constexpr int GH = (G + 1) / 2;
  __shared__ float lutp[GH][2 * kLut];  // head pairs, interleaved (lut_word_pair)
  __shared__ int sidx[kAttnMaxCpb * kAttnChunk];
  __shared__ __align__(16) float pb[4][kAttnChunk][G];
  __shared__ float mo[4][G][kD];
  __shared__ float mml[4][G][2];
  __shared__ MfLds mfl[mf_path(G, QV) ? 4 : 1];

  const int bh = blockIdx.y, b = bh / Hkv, h = bh - b * Hkv;
  const int s = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: scalar loop control
  const int el = lane & 31, half = lane >> 5, seg = lane & 15;
  const int nt = seq_len(seq_lens, b, n_tokens);          // this sequence's length
  const int L = kSink + seq_topk(top_k, nt);               // its attended entries
  const int n_chunks = (L + kAttnChunk - 1) / kAttnChunk;
  const int c0 = s * cpb, c_end = min(n_chunks, c0 + cpb);  // may be empty (ragged batch)
  // Rows: contiguous, relative to this head's first row (positions); paged,
  // absolute pool rows (the bf16 V pool then has the rows' layout, vst apart).
  const bool paged = rm.table != nullptr;
  const int64_t row0 = paged ? 0 : (int64_t)bh * rm.capacity;
  const int64_t hq0 = (int64_t)b * n_q_heads + (int64_t)h * G;
  const int32_t* ib = idx + (int64_t)bh * top_k;
  Src src;
  src.codes = codes + row0 * kCodeBytes;
  src.alpha = alpha + row0;
  src.slog = att_slog + hq0 * kSink;
  src.vb = QV ? nullptr : (paged ? v : v + (int64_t)b * vsb + (int64_t)h * vsh) + seg * 8;
  src.vst = vst;
  src.vbase = QV ? nullptr
                 : reinterpret_cast<const char*>(paged ? v : v + (int64_t)b * vsb + (int64_t)h * vsh);
  src.vstb = (uint32_t)(vst * 2);
  src.vlane = (uint32_t)seg * 16u;
  src.vrec = QV ? vrec + row0 * kVRecBytes : nullptr;
  src.vsk = QV ? vsink + (int64_t)bh * kSink * kD + seg * 8 : nullptr;

  // The block's positions (clamped into [0, n_tokens): memory safety only) and
  // the G attention tables into LDS.  Every load of a round is issued before
  // the first is used (as a load-store loop, each iteration waited for its
  // load: up to eight round trips before the first chunk): the positions and
  // the tables, then, for a paged cache, the page ids.
  float qmu[GH];
  {
    constexpr int kPer = kAttnMaxCpb * kAttnChunk / 256;  // positions per thread at most
    constexpr int kLutPer = (G * kLut / 4 + 255) / 256;   // table float4s per thread
    const int e0 = c0 * kAttnChunk, ne = (c_end - c0) * kAttnChunk;
    const float4* lsrc = reinterpret_cast<const float4*>(att_lut + hq0 * kLut);
    float4 lv[kLutPer];  // (unconditional loads at clamped indices: no branch, no scratch)
#pragma unroll
    for (int u = 0; u < kLutPer; ++u) lv[u] = lsrc[min(tid + 256 * u, G * kLut / 4 - 1)];
    int tv[kPer];
#pragma unroll
    for (int u = 0; u < kPer; ++u) {
      const int i = tid + 256 * u;
      const int e = min(e0 + i, L - 1);
      tv[u] = (i < ne && e >= kSink) ? ib[e - kSink] : e;
    }
#pragma unroll
    for (int i = 0; i < GH; ++i) qmu[i] = (2 * i + half < G) ? att_qmu[hq0 + 2 * i + half] : 0.0f;
    __builtin_amdgcn_sched_barrier(0);  // all of the round's loads are out
#pragma unroll
    for (int u = 0; u < kLutPer; ++u) {  // (threads past the end rewrite the last entries)
      const int f = min(tid + 256 * u, G * kLut / 4 - 1);  // float4 f: head g, entries 4r..
      const int g = f / (kLut / 4), r = f - g * (kLut / 4);
      float* d = &lutp[g >> 1][8 * r + (g & 1)];
      d[0] = lv[u].x;
      d[2] = lv[u].y;
      d[4] = lv[u].z;
      d[6] = lv[u].w;
    }
    if constexpr (G & 1) {  // the last pair's second slot
#pragma unroll
      for (int e = tid; e < kLut; e += 256) lutp[GH - 1][2 * e + 1] = 0.0f;
    }
#pragma unroll
    for (int u = 0; u < kPer; ++u) {
      const int e = min(e0 + tid + 256 * u, L - 1);
      tv[u] = e < kSink ? e : min(max(tv[u], 0), nt - 1);
    }
    if (paged) {  // the page ids of all positions, then the rows
      int pg[kPer];
#pragma unroll
      for (int u = 0; u < kPer; ++u)
        pg[u] = tid + 256 * u < ne ? rm.table[(int64_t)b * rm.pps + (tv[u] >> rm.lg_page)] : 0;
#pragma unroll
      for (int u = 0; u < kPer; ++u)
        tv[u] = (int)((((int64_t)pg[u] * Hkv + h) << rm.lg_page) |
                      (int64_t)(tv[u] & ((1 << rm.lg_page) - 1)));
    }
#pragma unroll
    for (int u = 0; u < kPer; ++u)
      if (tid + 256 * u < ne) sidx[tid + 256 * u] = tv[u];
  }
  __syncthreads();

  MfLds* mfw = &mfl[mf_path(G, QV) ? wave : 0];
  Acc<G> st;
#pragma unroll
  for (int nb = 0; nb < 8; ++nb) st.d[nb] = float4v{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
  for (int g = 0; g < G; ++g) {
    st.m[g] = -INFINITY;
    st.zacc[g] = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) st.acc[g][i] = 0.0f;
  }
#pragma unroll
  for (int i = 0; i < GH; ++i) st.lsum[i] = 0.0f;

  // Wave w takes the block's chunks w, w+4, ...  A sink chunk (only the first
  // chunk of waves 0 and 1 of split 0) is done on its own; then every chunk's
  // loads are issued one chunk ahead, right after the previous chunk's have
  // been consumed, so the only loads a chunk waits for were issued a whole
  // chunk earlier (the last chunk is peeled: no branch around the prefetch).
  int c = c0 + wave;
  if (c < c_end && c * kAttnChunk < kSink) {
    Chunk<G> sk;
    load_chunk<G, QV, kO32>(sk, c, c - c0, true, sidx, lane, src);
    process_chunk<G, QV>(st, sk, true, true, lutp, qmu, sm_log2, pb[wave], mfw, lane);
    c += 4;
  }
  if (c < c_end) {
    const int c_last = c + ((c_end - 1 - c) & ~3);
    Chunk<G> nx;
    load_chunk<G, QV, kO32>(nx, c, c - c0, false, sidx, lane, src);
    for (; c < c_last; c += 4) {
      const Chunk<G> cur = nx;
      load_chunk<G, QV, kO32>(nx, c + 4, c + 4 - c0, false, sidx, lane, src);
      __builtin_amdgcn_sched_barrier(0);  // keep the prefetch ahead of the chunk's work
      process_chunk<G, QV>(st, cur, false, c * kAttnChunk + el < L, lutp, qmu, sm_log2, pb[wave],
                           mfw, lane);
    }
    process_chunk<G, QV>(st, nx, false, c * kAttnChunk + el < L, lutp, qmu, sm_log2, pb[wave],
                         mfw, lane);
  }

  // Wave partial: sums over the four 16-lane groups and over the 32 lanes.
#pragma unroll
  for (int g = 0; g < G; ++g)
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      float x = QV ? st.acc[g][i] + st.zacc[g] : st.acc[g][i];
      x += __shfl_xor(x, 16);
      x += __shfl_xor(x, 32);
      st.acc[g][i] = x;
    }
#pragma unroll
  for (int i = 0; i < GH; ++i) {
    const float x = row_allreduce(st.lsum[i], [](float a, float b) { return a + b; });
    const float h0 = readlane(x, 0) + readlane(x, 16), h1 = readlane(x, 32) + readlane(x, 48);
    st.lsum[i] = half ? h1 : h0;
  }
  if (lane < 16) {
#pragma unroll
    for (int g = 0; g < G; ++g)
#pragma unroll
      for (int i = 0; i < 8; ++i) mo[wave][g][seg * 8 + i] = st.acc[g][i];
  }
  if constexpr (mf_path(G, QV)) {
    // matrix-core products: lane (r4 = lane / 16, n = lane % 16) holds, for the
    // channel blocks nb = 2 r4 and 2 r4 + 1 (channel group r4), head j's output
    // at channel 16 nb + n
    wave_sync_lds();
    const int r4 = lane >> 4, n = lane & 15;
#pragma unroll
    for (int nb = 0; nb < 8; ++nb) {
      if ((nb >> 1) != r4) continue;
#pragma unroll
      for (int j = 0; j < G; ++j) mo[wave][j][16 * nb + n] += st.d[nb][j] * (1.0f / kMfScale);
    }
  }
  if (el == 0) {
#pragma unroll
    for (int i = 0; i < GH; ++i) {
      const int g = 2 * i + half;
      if (g < G) {
        const float m_odd = st.m[min(2 * i + 1, G - 1)], m_even = st.m[2 * i];
        mml[wave][g][0] = half ? m_odd : m_even;
        mml[wave][g][1] = st.lsum[i];
      }
    }
  }
  __syncthreads();
  // Block merge of the four wave partials (waves without a chunk hold -inf, 0;
  // a block without any, possible in a ragged batch, writes (-inf, 0, 0)).
  for (int i = tid; i < G * kD; i += 256) {
    const int g = i / kD, ch = i % kD;
    const float M = fmaxf(fmaxf(mml[0][g][0], mml[1][g][0]), fmaxf(mml[2][g][0], mml[3][g][0]));
    float o = 0.0f, l = 0.0f;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const float f = M == -INFINITY ? 0.0f : exp2f(mml[w][g][0] - M);
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
  const int sg = tid >> 5, cq = tid & 31;  // split group, 16-byte column slice
  const float2* __restrict__ ml = reinterpret_cast<const float2*>(part_ml + r * n_splits * 2);
  const float4* __restrict__ po = reinterpret_cast<const float4*>(part_o + r * n_splits * kD) + cq;
  // Splits sg, sg + 8, sg + 16, sg + 24 are loaded before the maximum is known
  // (unconditionally, at clamped indices, and masked after), so the partials
  // are fetched in the same round trip as the maxima.
  constexpr int kPre = 4;
  float2 mv[kPre];
  float4 ov[kPre];
#pragma unroll
  for (int u = 0; u < kPre; ++u) {
    const int sc = min(sg + 8 * u, n_splits - 1);
    mv[u] = ml[sc];
    ov[u] = po[(int64_t)sc * (kD / 4)];
  }
  float m = -INFINITY;
#pragma unroll
  for (int u = 0; u < kPre; ++u)
    if (sg + 8 * u < n_splits) m = fmaxf(m, mv[u].x);
  for (int sc = sg + 8 * kPre; sc < n_splits; sc += 8) m = fmaxf(m, ml[sc].x);
  {
    const float v = row_allreduce(m, [](float a, float b) { return fmaxf(a, b); });
    m = fmaxf(fmaxf(readlane(v, 0), readlane(v, 16)), fmaxf(readlane(v, 32), readlane(v, 48)));
  }
  if (lane == 0) wred[0][wave] = m;
  __syncthreads();
  m = fmaxf(fmaxf(wred[0][0], wred[0][1]), fmaxf(wred[0][2], wred[0][3]));
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  float l = 0.0f;  // summed by the cq == 0 lane of each split group only
#pragma unroll
  for (int u = 0; u < kPre; ++u) {
    if (sg + 8 * u < n_splits) {
      const float w = exp2f(mv[u].x - m);
      if (cq == 0) l = fmaf(w, mv[u].y, l);
      acc.x = fmaf(w, ov[u].x, acc.x);
      acc.y = fmaf(w, ov[u].y, acc.y);
      acc.z = fmaf(w, ov[u].z, acc.z);
      acc.w = fmaf(w, ov[u].w, acc.w);
    }
  }
  for (int sc = sg + 8 * kPre; sc < n_splits; sc += 8) {
    const float2 x = ml[sc];
    const float4 o4 = po[(int64_t)sc * (kD / 4)];
    const float w = exp2f(x.x - m);
    if (cq == 0) l = fmaf(w, x.y, l);
    acc.x = fmaf(w, o4.x, acc.x);
    acc.y = fmaf(w, o4.y, acc.y);
    acc.z = fmaf(w, o4.z, acc.z);
    acc.w = fmaf(w, o4.w, acc.w);
  }
  l = wave_sum(l);
  if (lane == 0) wred[1][wave] = l;
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
                       const uint8_t* vrec, const uint16_t* vsink, const RowMap& rm,
                       int64_t n_rows, int n_tokens, const int32_t* seq_lens,
                       const int32_t* idx, int top_k, const float* att_lut,
                       const float* att_qmu, const float* att_slog, float sm_scale,
                       int chunks_per_block, int n_splits, float* part_o, float* part_ml,
                       const Launch& s) {
  const int n_chunks = (kSink + top_k + kAttnChunk - 1) / kAttnChunk;
  if (chunks_per_block < 1 || chunks_per_block > kAttnMaxCpb ||
      (int64_t)n_splits * chunks_per_block < n_chunks ||
      (int64_t)(n_splits - 1) * chunks_per_block >= n_chunks)
    return hipErrorInvalidValue;
  const float sm_log2 = sm_scale * 1.4426950408889634f;
  const dim3 grid(n_splits, B * Hkv), block(256);
  // 32-bit offsets: rows below 2^24 (the 24-bit multiply), and for bf16 values
  // a row stride below 2^24 bytes with the last row's end within 4 GiB
  const int64_t kRowLim = int64_t(1) << 24;
  const bool o32 = n_rows > 0 && n_rows <= kRowLim &&
                   (vrec != nullptr || (vst > 0 && 2 * vst < kRowLim &&
                                        n_rows * 2 * vst <= (int64_t(1) << 32) - 256));
#define SIKV_ATTN_ARGS                                                                         \
  grid, block, 0, s, n_q_heads, Hkv, codes, alpha, v, vsb, vsh, vst, vrec, vsink, rm, n_tokens,  \
      seq_lens, idx, top_k, att_lut, att_qmu, att_slog, sm_log2, chunks_per_block, n_splits,   \
      part_o, part_ml
#define SIKV_ATTN_CASE(GG)                                                                     \
  case GG:                                                                                     \
    if (vrec != nullptr)                                                                       \
      return o32 ? launch_k(KID_ATTN, attn_kernel<GG, true, true>, SIKV_ATTN_ARGS)             \
                 : launch_k(KID_ATTN, attn_kernel<GG, true, false>, SIKV_ATTN_ARGS);           \
    return o32 ? launch_k(KID_ATTN, attn_kernel<GG, false, true>, SIKV_ATTN_ARGS)              \
               : launch_k(KID_ATTN, attn_kernel<GG, false, false>, SIKV_ATTN_ARGS);
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
#undef SIKV_ATTN_ARGS
}

hipError_t launch_combine(const float* part_o, const float* part_ml, int BHq, int n_splits,
                          float* out, const Launch& s) {
  return launch_k(KID_COMBINE, combine_kernel, dim3(BHq), dim3(256), 0, s, part_o, part_ml,
                  n_splits, out);
}

}  // namespace sikv
