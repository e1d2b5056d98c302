// HIP kernels for gfx950 (CDNA4): the per-row forward of greedy block verification.
//
// Every kernel here computes each row (one token position) with arithmetic
// that does not depend on how many rows the launch carries or what the other
// rows hold: the same MFMA instruction shape and k order for every row count,
// a split-K plan fixed per weight matrix, fixed-order reductions, and
// attention whose split plan depends only on the row's own context length.
// That is what makes a verify row bit-identical to a one-token decode of the
// same prefix ("Phase 23: Speculative Verify Parity", section 1: the batched
// verify path drifted from per-token decode at bf16 near-ties; "Shape and
// cache history in Gemma block verification", section "Source evidence and
// competing explanations": reduction orders that change with the number of
// rows are what moved the scores).
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "sv_internal.h"

// No implicit fused multiply-adds: every expression rounds exactly as
// written, so an operation written once and used by two kernels (the GEMM
// epilogues, the attention block step, the split fold) gives the same bits
// in both, whatever code surrounds it.  Fused operations are written out
// (fmaf) where they are meant.
#pragma clang fp contract(off)

namespace sv {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4v __attribute__((ext_vector_type(4)));

// Weight stream load: read once per forward, so marked non-temporal.
__device__ __forceinline__ uint4 ld_stream(const uint4* p) {
  const u32x4v v = __builtin_nontemporal_load(reinterpret_cast<const u32x4v*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}

// ------------------------------------------------------------ scalar helpers
__device__ __forceinline__ float bf2f(uint16_t b) { return __uint_as_float(((uint32_t)b) << 16); }

// fp32 -> bf16, round to nearest even; NaN stays NaN.
__device__ __forceinline__ uint16_t f2bf(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

__device__ __forceinline__ uint32_t pack2(uint16_t lo, uint16_t hi) { return (uint32_t)lo | ((uint32_t)hi << 16); }

// fp32 -> IEEE binary16 bits, round to nearest even (hardware conversion).
__device__ __forceinline__ uint16_t f2h(float f) { return __builtin_bit_cast(uint16_t, (_Float16)f); }
__device__ __forceinline__ float h2f(uint16_t b) { return (float)__builtin_bit_cast(_Float16, b); }

__device__ __forceinline__ f32x4 mfma16x16x32_f16(uint4 a, uint4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), c, 0, 0,
                                                0);
}

__device__ __forceinline__ f32x4 mfma16x16x32(uint4 a, uint4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b),
                                                c, 0, 0, 0);
}

// Every lane ends with the same value: at each butterfly stage a lane adds
// (a + b) while its partner adds (b + a), which is the same float.
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o);
  return v;
}
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}

// Orderable 64-bit key: larger logit wins; among equal logits the lower id
// wins (the low word holds ~id).  -0.0 is folded onto +0.0 so they tie.
__device__ __forceinline__ uint64_t argmax_key(float v, uint32_t id) {
  uint32_t u = __float_as_uint(v);
  if (v == 0.0f) u = 0u;
  u = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  return ((uint64_t)u << 32) | (uint64_t)(0xffffffffu - id);
}
__device__ __forceinline__ uint64_t umax64(uint64_t a, uint64_t b) { return a > b ? a : b; }

// Fixed-order block sum of 256 threads (4 waves): butterfly in each wave,
// then ((w0 + w1) + w2) + w3.  Returns the sum to every thread.
__device__ __forceinline__ float block_sum256(float v, float* lds4) {
  v = wave_sum(v);
  const int w = threadIdx.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) lds4[w] = v;
  __syncthreads();
  float s = lds4[0];
  s = s + lds4[1];
  s = s + lds4[2];
  s = s + lds4[3];
  return s;
}

// ------------------------------------------------------------ packed weights
// bf16 tile chunk: 16 outputs x 32 inputs = 1 KiB, stored in MFMA operand
// order: lane l = g*16 + i holds outputs (tile*16 + i), inputs (chunk*32 +
// 8g .. +7) as one 16-byte vector at byte 16*l.  Chunks are stored
// tile-major ([n_tile][k_chunk]).
//
// int4 tile: 16 outputs x 128 inputs (two scale groups of 64) = 1 KiB of
// codes; lane l's 16 bytes hold 32 nibbles c = 0..31 for input
// 128*kt + 64*(c/16) + 32*((c%16)/8) + 8g + c%8 (nibble 2b low, 2b+1 high of
// byte b).  Scales: per tile 64 B = [group 0..1][16 outputs] bf16.

// ------------------------------------------------------------ skinny GEMM
// Y[r][n] = sum_k B[r][k] * W[n][k] for r < M.  An *item* is one packed
// output tile (16 outputs) over the whole K.  A workgroup of NW waves takes
// items blockIdx.x, blockIdx.x + gridDim.x, ...; its waves split K into NW
// contiguous slices (fixed per matrix).  Each wave runs its chunks in
// ascending order through one MFMA accumulator chain per row tile, the hi
// plane of a chunk before its lo plane; the NW wave partials are added in
// wave order through LDS.  The row count only sets how many row tiles are
// computed, and no value crosses workgroups, so a row's result never depends
// on M.  Weights are requested before anything else and the next item's
// weights are in flight while the current item is reduced and finished.
//
// RMSNorm commutes with the product: W (x * g / rms) = (W (x * g)) / rms, so
// producers hand over planes of x * g and the consumer scales its outputs by
// 1 / rms in the epilogue.  Epilogue per role:
//   QKV      tile = 8 dims + their RoPE partners (+ dh/2): 1/rms, RoPE, K/V
//            into the paged cache (fp16), q (fp32) to the workspace
//   O, down  residual add, per-16-column sum of squares, planes of x * g_next
//   gate/up  tile = 8 gate + 8 up outputs of the same features: 1/rms,
//            act(g) * u as planes
//   LM head  1/rms, per-16-column (max logit, lowest id), optional fp32 logits

// An fp32 vector as the MFMA operand pair hi = bf16(h), lo = bf16(h - hi)
// (the difference is exact in fp32): two MFMAs against the exact bf16
// weights give the products of h to about 16 significant bits.
struct BPair {
  uint4 hi, lo;
};

__device__ __forceinline__ BPair split8(const float (&h)[8]) {
  uint16_t hb[8], lb[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    hb[e] = f2bf(h[e]);
    lb[e] = f2bf(h[e] - bf2f(hb[e]));
  }
  BPair b;
  b.hi = make_uint4(pack2(hb[0], hb[1]), pack2(hb[2], hb[3]), pack2(hb[4], hb[5]), pack2(hb[6], hb[7]));
  b.lo = make_uint4(pack2(lb[0], lb[1]), pack2(lb[2], lb[3]), pack2(lb[4], lb[5]), pack2(lb[6], lb[7]));
  return b;
}

__device__ __forceinline__ void split1(float h, uint16_t& hi, uint16_t& lo) {
  hi = f2bf(h);
  lo = f2bf(h - bf2f(hi));
}

__device__ __forceinline__ BPair bzero() { return BPair{make_uint4(0u, 0u, 0u, 0u), make_uint4(0u, 0u, 0u, 0u)}; }

__device__ __forceinline__ BPair load_planes(const GemmArgs& a, int r, int k0) {
  const size_t off = (size_t)r * a.K + k0;
  return BPair{*reinterpret_cast<const uint4*>(a.bhi + off), *reinterpret_cast<const uint4*>(a.blo + off)};
}

__device__ __forceinline__ f32x4 mfma_pair(uint4 a, const BPair& b, f32x4 c) {
  c = mfma16x16x32(a, b.hi, c);
  return mfma16x16x32(a, b.lo, c);
}

// The same compensated pair in fp16 (hi = fp16(h), lo = fp16(h - hi)), for
// products against the fp16 KV cache.
__device__ __forceinline__ BPair split8_f16(const float (&h)[8]) {
  uint16_t hb[8], lb[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    hb[e] = f2h(h[e]);
    lb[e] = f2h(h[e] - h2f(hb[e]));
  }
  BPair b;
  b.hi = make_uint4(pack2(hb[0], hb[1]), pack2(hb[2], hb[3]), pack2(hb[4], hb[5]), pack2(hb[6], hb[7]));
  b.lo = make_uint4(pack2(lb[0], lb[1]), pack2(lb[2], lb[3]), pack2(lb[4], lb[5]), pack2(lb[6], lb[7]));
  return b;
}

__device__ __forceinline__ f32x4 mfma_pair_f16(uint4 a, const BPair& b, f32x4 c) {
  c = mfma16x16x32_f16(a, b.hi, c);
  return mfma16x16x32_f16(a, b.lo, c);
}

// 8 int4 codes (one 32-bit word, nibble e = code of element e, two's
// complement) -> one MFMA operand of 8 bf16 holding the integers exactly.
// Code e is sign-extended and converted to fp32; an integer of magnitude at
// most 8 has a zero low half in fp32, so its bf16 is the high half, and
// v_perm packs the high halves of two fp32 values into one word.
__device__ __forceinline__ uint32_t code_f32_bits(uint32_t w, int e) {
  return __float_as_uint((float)(((int)(w << (28 - 4 * e))) >> 28));
}
__device__ __forceinline__ uint32_t codes2(uint32_t w, int e) {   // elements e (low half) and e + 1
  return __builtin_amdgcn_perm(code_f32_bits(w, e + 1), code_f32_bits(w, e), 0x07060302u);
}
__device__ __forceinline__ uint4 codes8(uint32_t w) {
  return make_uint4(codes2(w, 0), codes2(w, 2), codes2(w, 4), codes2(w, 6));
}

__device__ __forceinline__ float act_fn(float x, int act) {
  if (act == 0) return x / (1.0f + expf(-x));
  const float c = 0.7978845608028654f;  // sqrt(2/pi)
  return 0.5f * x * (1.0f + tanhf(c * (x + 0.044715f * (x * x * x))));
}

// Kernel span measurement: every workgroup stamps the device's constant-rate
// wall clock when it starts and when it ends; the slot keeps the earliest
// start and the latest end (global atomics, read by the host after the
// stream has synchronised).
__device__ __forceinline__ void prof_start(unsigned long long* prof) {
  if (prof != nullptr && threadIdx.x == 0) atomicMin(prof, (unsigned long long)wall_clock64());
}
// The GEMM kernels read the clock at entry and publish the start once their
// first loads are out: a wave that publishes first waits on the clock read
// (and on the scalar load of the slot pointer) before it can issue them.
__device__ __forceinline__ void prof_publish_start(unsigned long long* prof, unsigned long long t_start) {
  if (prof != nullptr && threadIdx.x == 0) atomicMin(prof, t_start);
}
__device__ __forceinline__ void prof_end(unsigned long long* prof) {
  if (prof != nullptr) {
    __syncthreads();
    if (threadIdx.x == 0) atomicMax(prof + 1, (unsigned long long)wall_clock64());
  }
}

// n / d for n >= 0 and n * d < 2^32, as the high word of n * m with
// m = ceil(2^32 / d) = (2^32 + e) / d, 0 <= e < d: n m / 2^32 = n / d + n e /
// (d 2^32), and n e / (d 2^32) < n / 2^32 < 1 / d, which never carries the
// quotient past the next integer.  d = 1 takes n itself (m would not fit).
inline unsigned div_magic(int d) {
  return d <= 1 ? 0u : (unsigned)((0x100000000ull + (unsigned)d - 1u) / (unsigned)d);
}
__device__ __forceinline__ int div_m(int n, int d, unsigned magic) {
  return d == 1 ? n : (int)__umulhi((unsigned)n, magic);
}

constexpr int kMaxWaves = 16;
constexpr int kStageBytes = kGemmStageBytes;   // LDS for staged activation planes (hi + lo)

struct GemmShared {
  uint4 dummy;                // target of stage stores that carry no data
  f32x4 red[kMaxWaves][64];   // wave partials of one row tile
  float y[kMaxRows][16];      // finished outputs of the item
  float inv[kMaxRows];        // 1 / rms of each row (RMSNorm consumers)
  unsigned long long best[kMaxRows];   // LM head: this workgroup's row argmax keys
};

// Pair index of row i of a QKV tile (the weight packing below): rows i and
// i ^ 4 are a (dim, RoPE partner) pair.
__device__ __forceinline__ int pair_of(int i) { return 4 * (i >> 3) + (i & 3); }

__host__ __device__ __forceinline__ constexpr bool norm_role(int role) {
  return role == kRoleQkv || role == kRoleGateUp || role == kRoleLmHead;
}

// 1 / sqrt(mean(x^2) + eps) of row r from its per-16-column sums of
// squares: each lane adds its slices lane, lane + 64, ... in order, then a
// butterfly over the wave (one wave per row).
__device__ __forceinline__ float row_inv_rms(const GemmArgs& a, int r, int lane) {
  const int nsl = a.K >> 4;
  const float* p = a.ss + (size_t)r * nsl;
  float v = 0.f;
  for (int i = lane; i < nsl; i += 64) v = v + p[i];
  v = wave_sum(v);
  return 1.0f / sqrtf(v / (float)a.K + a.eps);
}
__device__ __forceinline__ void rows_inv_rms(const GemmArgs& a, GemmShared& sh, int wave, int lane, int nw) {
  for (int r = wave; r < a.M; r += nw) {
    const float v = row_inv_rms(a, r, lane);
    if (lane == 0) sh.inv[r] = v;
  }
}

// Global operands of the epilogue element (r, c) = (idx / 16, idx % 16) of
// item T, loaded when the item starts so the epilogue does not wait on them:
// O / down read the residual and the next gain, QKV the RoPE pair and the
// physical page of its row.  Only the element idx = threadIdx.x is
// prefetched (blockDim >= 16 M); any other element loads in the epilogue.
struct EpiPre {
  float x, gain;
  float2 cs;
  int page, pos;          // QKV: physical page and position of the row
  uint16_t* pool;         // QKV: KV pool of the row's sequence
  int n_pages;
};

template <int ROLE>
__device__ __forceinline__ EpiPre epi_load(const GemmArgs& a, int T, int idx) {
  EpiPre e{0.f, 0.f, make_float2(0.f, 0.f), 0, 0, nullptr, 0};
  if (idx >= a.M * 16) return e;
  const int r = idx >> 4, c = idx & 15;
  if (ROLE == kRoleO || ROLE == kRoleDown) {
    const int n = T * 16 + c;
    e.x = a.x[(size_t)r * a.N + n];
    e.gain = bf2f(a.gnext[n]);
  } else if (ROLE == kRoleQkv) {
    const int half = a.dh >> 1, gph = half >> 3;
    const int hh = T / gph, sb = T % gph;
    const int* table = a.page_table;
    e.pool = a.kv_pool;
    e.n_pages = a.n_pages;
    if (a.seqs != nullptr) {   // batched: the row's own sequence
      const SeqDev& sd = a.seqs[a.rowseq[r]];
      e.pos = sd.kv_len + r - sd.row0;
      table = sd.page_table;
      e.pool = sd.kv_pool;
      e.n_pages = sd.n_pages;
    } else {
      e.pos = a.params[0] + r;
    }
    if (hh < a.nq + a.nkv) e.cs = a.rope[(size_t)e.pos * half + 8 * sb + pair_of(c)];
    if (hh >= a.nq) e.page = table[e.pos / kPage];
  }
  return e;
}

// Epilogue of element (r, c) of item (tile) T: yv(cc) is the finished sum of
// column cc of row r, invr the row's 1 / rms (RMSNorm consumers), best_r the
// workgroup's argmax key slot of the row (LM head, in LDS).  Both GEMM
// kernels call this, so an output does not depend on which one produced it.
// The caller runs whole 16-lane groups (the 16 columns of one row) together.
template <int ROLE, class YV>
__device__ __forceinline__ void epi_element(const GemmArgs& a, int T, int r, int c, const EpiPre& e, float invr,
                                            YV yv, unsigned long long* best_r) {
  float y = yv(c);
  if (norm_role(ROLE)) y = y * invr;
  if (ROLE == kRoleO || ROLE == kRoleDown) {
    const int n = T * 16 + c;
    const size_t xi = (size_t)r * a.N + n;
    const float xn = e.x + y;
    a.x[xi] = xn;
    float sq = xn * xn;
#pragma unroll
    for (int o = 8; o >= 1; o >>= 1) sq += __shfl_xor(sq, o);
    if (c == 0) a.ss_out[(size_t)r * (a.N >> 4) + T] = sq;
    split1(xn * e.gain, a.uhi[xi], a.ulo[xi]);
  } else if (ROLE == kRoleGateUp) {               // [gate 8 | up 8] of features 8T..8T+7
    const float up = yv((c & 7) + 8) * invr;
    if (c < 8) {
      const size_t ai = (size_t)r * (a.N >> 1) + T * 8 + c;
      split1(act_fn(y, a.act) * up, a.ahi[ai], a.alo[ai]);
    }
  } else if (ROLE == kRoleQkv) {                  // dim 8s + pair_of(c) at c, its partner at c ^ 4
    const int half = a.dh >> 1;
    const int gph = half >> 3;
    const int hh = T / gph, sb = T % gph;
    const bool lo = (c & 4) == 0;
    const int i = 8 * sb + pair_of(c);
    const int d = lo ? i : half + i;
    const int pos = e.pos;
    float out = y;
    if (hh < a.nq + a.nkv) {
      const float2 cs = e.cs;
      const float partner = yv(c ^ 4) * invr;
      out = lo ? (y * cs.x - partner * cs.y) : (y * cs.x + partner * cs.y);
    }
    if (hh < a.nq) {
      a.q_out[((size_t)r * a.nq + hh) * a.dh + d] = out;
    } else {
      const int kv = hh < a.nq + a.nkv ? 0 : 1;
      const int head = hh - a.nq - kv * a.nkv;
      const int page = e.page;
      const size_t base = ((((size_t)a.layer * e.n_pages + page) * 2 + kv) * a.nkv + head) * kPage * a.dh;
      // K rows are [slot][dh]; V is stored transposed inside the page, [dh][slot]
      const size_t el = kv == 0 ? (size_t)(pos % kPage) * a.dh + d : (size_t)d * kPage + (pos % kPage);
      e.pool[base + el] = f2h(out);
    }
  } else {                                        // kRoleLmHead
    const int n = T * 16 + c;
    if (a.logits != nullptr) a.logits[(size_t)r * a.N + n] = y;
    uint64_t b = argmax_key(y, (uint32_t)n);
#pragma unroll
    for (int o = 8; o >= 1; o >>= 1) b = umax64(b, __shfl_xor(b, o));
    if (c == 0) atomicMax(best_r, (unsigned long long)b);
  }
}

// Epilogue on the finished 16 columns of item (tile) T, or on columns
// [8 hf, 8 hf + 8) only for a half item (hf >= 0: QKV, whose
// column pairs never cross the halves; the other half's columns then hold
// copies of these and are not written).
template <int ROLE>
__device__ __forceinline__ void gemm_epilogue(const GemmArgs& a, GemmShared& sh, int T, const EpiPre& pre, int hf) {
  for (int idx = threadIdx.x; idx < a.M * 16; idx += blockDim.x) {
    const int r = idx >> 4, c = idx & 15;
    if (hf >= 0 && (c >> 3) != hf) continue;
    const EpiPre e = idx == (int)threadIdx.x ? pre : epi_load<ROLE>(a, T, idx);
    epi_element<ROLE>(a, T, r, c, e, sh.inv[r], [&](int cc) { return sh.y[r][cc]; }, &sh.best[r]);
  }
}

// Wave partials of one item -> LDS -> summed in wave order -> sh.y -> epilogue.
template <int TM, int ROLE>
__device__ __forceinline__ void gemm_finish(const GemmArgs& a, GemmShared& sh, f32x4 (&acc)[TM], int T, int wave,
                                            int lane, int nw, const EpiPre& pre, int hf = -1) {
#pragma unroll
  for (int rt = 0; rt < TM; ++rt) {
    sh.red[wave][lane] = acc[rt];
    __syncthreads();
    // 256 threads: thread t sums component t % 4 of lane t / 4 over the
    // waves, all partials loaded first, added in wave order
    const float* red = reinterpret_cast<const float*>(sh.red);
    for (int t = threadIdx.x; t < 256; t += blockDim.x) {
      float v = 0.f;
#pragma unroll
      for (int w0 = 0; w0 < kMaxWaves; w0 += 8) {   // two batches of 8 loads
        float part[8];
#pragma unroll
        for (int w = 0; w < 8; ++w) part[w] = red[(w0 + w) * 256 + t];
#pragma unroll
        for (int w = 0; w < 8; ++w)
          if (w0 + w < nw) v = (w0 + w == 0) ? part[w] : v + part[w];
      }
      // lane l holds Y[r = rt*16 + (l & 15)][column 4 (l >> 4) + component]
      const int l = t >> 2;
      const int r = rt * 16 + (l & 15);
      if (r < a.M) sh.y[r][4 * (l >> 4) + (t & 3)] = v;
    }
    __syncthreads();
  }
  gemm_epilogue<ROLE>(a, sh, T, pre, hf);
  __syncthreads();
}

// LM head: the workgroup's row maxima start at 0 (below every key) and go to
// the global row keys with one atomic max per row at the end.  The key orders
// by logit and then by lowest id, so the maximum does not depend on which
// workgroup or item contributed first.
template <int ROLE>
__device__ __forceinline__ void row_best_init(const GemmArgs& a, GemmShared& sh) {
  if (ROLE == kRoleLmHead)
    for (int r = threadIdx.x; r < a.M; r += blockDim.x) sh.best[r] = 0ull;
}
template <int ROLE>
__device__ __forceinline__ void row_best_publish(const GemmArgs& a, GemmShared& sh) {
  if (ROLE == kRoleLmHead) {
    __syncthreads();
    for (int r = threadIdx.x; r < a.M; r += blockDim.x) atomicMax(a.best + r, sh.best[r]);
  }
}

// Activation planes of chunk range [c_lo, c_lo + n_chunks) of every row,
// staged in LDS as [row][k] with a 16-byte pad per row (bank spread).
// `unit` = inputs per chunk (32 for bf16, 128 for int4).
struct Stage {
  uint16_t* hi;
  uint16_t* lo;
  int stride;   // bf16 elements per LDS row
};

__device__ __forceinline__ void stage_planes(const GemmArgs& a, const Stage& st, int c_lo, int n_chunks, int unit) {
  const int width = n_chunks * unit;            // inputs per row in the stage
  const int vec_per_row = width >> 3;           // 16-byte vectors per row and plane
  const int total = a.M * vec_per_row;
  const size_t k0 = (size_t)c_lo * unit;
  for (int i = threadIdx.x; i < total; i += blockDim.x) {
    const int r = i / vec_per_row, v = i % vec_per_row;
    const size_t src = (size_t)r * a.K + k0 + (size_t)v * 8;
    *reinterpret_cast<uint4*>(st.hi + r * st.stride + v * 8) = *reinterpret_cast<const uint4*>(a.bhi + src);
    *reinterpret_cast<uint4*>(st.lo + r * st.stride + v * 8) = *reinterpret_cast<const uint4*>(a.blo + src);
  }
}

// MFMA column (row slot) r of a row tile reads row min(r, M - 1).  An MFMA
// output column depends only on its own B column, so the duplicated columns
// past M change no kept result; they are dropped at the end.  Clamping keeps
// every MFMA out of divergent control flow: an MFMA in a branch that only
// some lanes take has been seen to overwrite registers that the lanes on the
// other side of the branch still hold live.
__device__ __forceinline__ int row_of(int r, int M) { return r < M ? r : M - 1; }

__device__ __forceinline__ BPair lds_pair(const Stage& st, int r, int k) {
  return BPair{*reinterpret_cast<const uint4*>(st.hi + r * st.stride + k),
               *reinterpret_cast<const uint4*>(st.lo + r * st.stride + k)};
}

// Chunks per LDS stage: the largest multiple of nw * nb dividing the chunk
// count whose activation planes for M rows fit the stage budget (0 if even
// nw * nb chunks do not fit).  It only decides when activations are staged,
// never the order of any sum.
__host__ __device__ __forceinline__ int stage_chunks(int n_chunks, int nw, int M, int unit, int nb) {
  int best = 0;
  const int step = nw * nb;
  for (int cs = step; cs <= n_chunks; cs += step) {
    if (n_chunks % cs) continue;
    if ((size_t)M * (cs * unit + 8) * 4 <= (size_t)kStageBytes) best = cs;
  }
  return best;
}

// Double-buffered stages (bf16): stage = NB chunks per wave (one ring group),
// two LDS buffers; the next stage's planes (at most kStageRegs 16-byte
// vectors per thread) are loaded into registers while the current stage's
// MFMAs run, then written to the other buffer, with one barrier per stage
// and no drain of the weight ring.
constexpr int kStageRegs = 4;
__host__ __device__ __forceinline__ bool stage_double_ok(int n_chunks, int nw, int M, int unit, int nb,
                                                         int nthreads) {
  const int cs = nw * nb;
  if (n_chunks % cs != 0 || cs == n_chunks) return false;
  if (2 * (size_t)M * (cs * unit + 8) * 4 > (size_t)kStageBytes) return false;
  return 2 * M * cs * (unit / 8) <= kStageRegs * nthreads;
}

// Activation planes of chunks [c_lo, c_lo + n_chunks) of every row into
// registers (vector i = threadIdx.x + k * blockDim.x of the hi plane, then
// the lo plane; loads past the end repeat the last vector, so the loads are
// unconditional) and from registers into a stage buffer.
struct StageRegs {
  uint4 v0, v1, v2, v3;   // kStageRegs vectors (plain members: they stay in registers)
};
// nthr = threads of the workgroup, passed in: reading blockDim inside the
// loop is a memory load whose wait would drain the weight ring.
__device__ __forceinline__ const uint16_t* stage_src(const GemmArgs& a, int c_lo, int n_chunks, int unit, int k,
                                                     int nthr) {
  const int vpr = (n_chunks * unit) >> 3;
  const int per_plane = a.M * vpr;
  int i = threadIdx.x + k * nthr;
  i = i < 2 * per_plane ? i : 2 * per_plane - 1;
  const int pl = i >= per_plane, ii = pl ? i - per_plane : i;
  const int r = ii / vpr, v = ii % vpr;
  return (pl ? a.blo : a.bhi) + (size_t)r * a.K + (size_t)c_lo * unit + (size_t)v * 8;
}
__device__ __forceinline__ StageRegs stage_fetch(const GemmArgs& a, int c_lo, int n_chunks, int unit, int nthr) {
  StageRegs s;
  s.v0 = *reinterpret_cast<const uint4*>(stage_src(a, c_lo, n_chunks, unit, 0, nthr));
  s.v1 = *reinterpret_cast<const uint4*>(stage_src(a, c_lo, n_chunks, unit, 1, nthr));
  s.v2 = *reinterpret_cast<const uint4*>(stage_src(a, c_lo, n_chunks, unit, 2, nthr));
  s.v3 = *reinterpret_cast<const uint4*>(stage_src(a, c_lo, n_chunks, unit, 3, nthr));
  return s;
}
// Unconditional LDS stores (a thread without a vector writes the dummy slot):
// a store that may or may not run would make the compiler drain every load
// before reusing its register.
__device__ __forceinline__ void stage_put(const GemmArgs& a, const Stage& st, int n_chunks, int unit, int k,
                                          uint4 val, uint4* dummy, int nthr) {
  const int vpr = (n_chunks * unit) >> 3;
  const int per_plane = a.M * vpr;
  const int i = threadIdx.x + k * nthr;
  const bool ok = i < 2 * per_plane;
  const int ic = ok ? i : 0;
  const int pl = ic >= per_plane, ii = pl ? ic - per_plane : ic;
  const int r = ii / vpr, v = ii % vpr;
  uint4* dst = reinterpret_cast<uint4*>((pl ? st.lo : st.hi) + r * st.stride + v * 8);
  *(ok ? dst : dummy) = val;
}
__device__ __forceinline__ void stage_store(const GemmArgs& a, const Stage& st, int n_chunks, int unit,
                                            const StageRegs& s, uint4* dummy, int nthr) {
  stage_put(a, st, n_chunks, unit, 0, s.v0, dummy, nthr);
  stage_put(a, st, n_chunks, unit, 1, s.v1, dummy, nthr);
  stage_put(a, st, n_chunks, unit, 2, s.v2, dummy, nthr);
  stage_put(a, st, n_chunks, unit, 3, s.v3, dummy, nthr);
}

// Prologue with the loads ordered by need: the first stage's activation
// planes (up to kProRegs vectors per thread) and the RMSNorm sums (one row
// per wave, up to kSsRegs slices per lane) are requested before the weight
// ring, so waiting for them leaves the ring in flight.
constexpr int kProRegs = 8, kSsRegs = 8;
struct ProRegs {   // named members, not arrays: they must stay in registers
  uint4 v0, v1, v2, v3, v4, v5, v6, v7;
  float s0, s1, s2, s3, s4, s5, s6, s7;
};
__host__ __device__ __forceinline__ bool prologue_fast(const GemmArgs& a, int cs, int unit, int nw, bool norm) {
  const int n_vec = 2 * a.M * ((cs * unit) >> 3);
  if (n_vec > kProRegs * nw * 64) return false;
  return !norm || (a.M <= nw && (a.K >> 4) <= 64 * kSsRegs);
}
// Vector k of this thread: index i = threadIdx.x + k * nthr over the hi
// plane's rows, then the lo plane's; q = i / vpr is the plane row (lo plane
// row q - M from q = M on), m = i % vpr the vector in it.  (q, m) step from
// k to k + 1 without a division, so the weight ring, requested after these
// loads, is not held up by per-vector divisions.
struct ProIdx {
  int q, m, dq, dm, vpr;
  __device__ __forceinline__ ProIdx(int vpr_, int nthr) : vpr(vpr_) {
    q = (int)threadIdx.x / vpr;
    m = (int)threadIdx.x - q * vpr;
    dq = nthr / vpr;
    dm = nthr - dq * vpr;
  }
  __device__ __forceinline__ void next() {
    q += dq;
    m += dm;
    if (m >= vpr) { m -= vpr; ++q; }
  }
};
__device__ __forceinline__ uint4 pro_load(const GemmArgs& a, const ProIdx& p) {
  if (p.q >= 2 * a.M) return make_uint4(0u, 0u, 0u, 0u);
  const int pl = p.q >= a.M, r = pl ? p.q - a.M : p.q;
  return *reinterpret_cast<const uint4*>((pl ? a.blo : a.bhi) + (size_t)r * a.K + (size_t)p.m * 8);
}
__device__ __forceinline__ void pro_store(const GemmArgs& a, const Stage& st, const ProIdx& p, uint4 val) {
  if (p.q >= 2 * a.M) return;
  const int pl = p.q >= a.M, r = pl ? p.q - a.M : p.q;
  *reinterpret_cast<uint4*>((pl ? st.lo : st.hi) + r * st.stride + p.m * 8) = val;
}
__device__ __forceinline__ float ss_load(const GemmArgs& a, int wave, int lane, int k) {
  const int nsl = a.K >> 4;
  const int i = lane + 64 * k;
  return i < nsl ? a.ss[(size_t)wave * nsl + i] : 0.f;
}
__device__ __forceinline__ ProRegs prologue_issue(const GemmArgs& a, int cs, int unit, int nthr, int wave, int lane,
                                                  bool norm) {
  ProIdx p((cs * unit) >> 3, nthr);
  ProRegs pr;
  pr.v0 = pro_load(a, p); p.next(); pr.v1 = pro_load(a, p); p.next();
  pr.v2 = pro_load(a, p); p.next(); pr.v3 = pro_load(a, p); p.next();
  pr.v4 = pro_load(a, p); p.next(); pr.v5 = pro_load(a, p); p.next();
  pr.v6 = pro_load(a, p); p.next(); pr.v7 = pro_load(a, p);
  pr.s0 = pr.s1 = pr.s2 = pr.s3 = pr.s4 = pr.s5 = pr.s6 = pr.s7 = 0.f;
  if (norm && wave < a.M) {
    pr.s0 = ss_load(a, wave, lane, 0); pr.s1 = ss_load(a, wave, lane, 1);
    pr.s2 = ss_load(a, wave, lane, 2); pr.s3 = ss_load(a, wave, lane, 3);
    pr.s4 = ss_load(a, wave, lane, 4); pr.s5 = ss_load(a, wave, lane, 5);
    pr.s6 = ss_load(a, wave, lane, 6); pr.s7 = ss_load(a, wave, lane, 7);
  }
  return pr;
}
__device__ __forceinline__ void prologue_finish(const GemmArgs& a, const Stage& st, int cs, int unit, int nthr,
                                                int wave, int lane, bool norm, const ProRegs& pr, GemmShared& sh) {
  if (norm && wave < a.M) {
    // the same order as rows_inv_rms: each lane adds its slices in order (the
    // zeros past the row's slices add exactly nothing), then the butterfly
    float v = 0.f;
    v = v + pr.s0; v = v + pr.s1; v = v + pr.s2; v = v + pr.s3;
    v = v + pr.s4; v = v + pr.s5; v = v + pr.s6; v = v + pr.s7;
    v = wave_sum(v);
    if (lane == 0) sh.inv[wave] = 1.0f / sqrtf(v / (float)a.K + a.eps);
  }
  ProIdx p((cs * unit) >> 3, nthr);
  pro_store(a, st, p, pr.v0); p.next(); pro_store(a, st, p, pr.v1); p.next();
  pro_store(a, st, p, pr.v2); p.next(); pro_store(a, st, p, pr.v3); p.next();
  pro_store(a, st, p, pr.v4); p.next(); pro_store(a, st, p, pr.v5); p.next();
  pro_store(a, st, p, pr.v6); p.next(); pro_store(a, st, p, pr.v7);
}

// Weight loads of one wave run as a ring of NB slots: a slot is refilled with
// the chunk NB positions ahead as soon as its MFMAs are issued, across item
// boundaries, so NB loads stay in flight through the cross-wave reduction of
// each item.  Position (item T, c) of wave w is chunk kc = w + nw * c of T;
// the ring changes only when chunks arrive, never the order of any sum.
struct LoadCursor {
  int T, c;     // item (bf16: this workgroup's item ordinal; int4: the tile) and chunk position
  size_t off;   // chunk (T, c): bf16, this lane's uint4 offset; int4, the chunk index
};

// Items of one workgroup.  Whole items T = b, b + G, ... below n_full; for
// QKV, when the r = n_items % G items of the last round would leave
// workgroups idle (r <= G/2), each of those items is split into its two
// 8-column halves, one half per workgroup, so every workgroup streams the
// same bytes (the 8B shape: 384 items on 256 workgroups).  A half item loads
// only its own rows' weights (lanes of the other half repeat them) and
// writes only its own columns; every output's sums are those of the whole
// item.  launch_gemm sets n_full and n_half (2 r, or 0 without a split).
// Measured on MI355X: the split code path costs a gate/up GEMM more than
// splitting would gain on these shapes, so only QKV takes it.
template <int ROLE>
struct ItemPlan {
  static constexpr bool kSplits = ROLE == kRoleQkv;
  int n_full, n_half, G;
  // item o of this workgroup: tile T and half hf (-1: whole); -1 past its last
  __device__ __forceinline__ int tile(int o, int& hf) const {
    const int b = blockIdx.x;
    const int T = b + o * G;
    hf = -1;
    if (T < n_full) return T;
    if (kSplits && b < n_half && T - G < n_full) {
      hf = b & 1;
      return n_full + (b >> 1);
    }
    return -1;
  }
  // whether item (T, hf) of this workgroup is followed by another
  __device__ __forceinline__ bool has_next(int T, int hf) const {
    return hf < 0 && (T + G < n_full || (kSplits && (int)blockIdx.x < n_half));
  }
};

// bf16: wave w accumulates chunks w, w + NW, w + 2 NW, ... of each item in
// that order (DBL: double-buffered stages of NB chunks per wave).
// Leading (preloaded) arguments, as for the register-operand kernels: the
// weights, activation planes and sums of squares, K, the grid size G and
// three packed words (ring_pack): pA = M | pro_fast << 7 | waves << 8 |
// cpi << 13 | n_stages << 23, pB = cs | cpws << 16, pC = n_full | n_half << 21.
template <int TM, int ROLE, int NB, bool DBL>
__global__ __launch_bounds__(1024) void k_gemm_bf16(const void* W, const uint16_t* bhi, const uint16_t* blo,
                                                    const float* ss, int K, int G, unsigned pA, unsigned pB,
                                                    unsigned pC, GemmArgs args) {
  GemmArgs a = args;
  a.W = W; a.bhi = bhi; a.blo = blo; a.ss = ss; a.K = K;
  a.M = (int)(pA & 127u); a.pro_fast = (int)((pA >> 7) & 1u); a.cpi = (int)((pA >> 13) & 1023u);
  a.n_stages = (int)(pA >> 23); a.cs = (int)(pB & 0xffffu); a.cpws = (int)(pB >> 16);
  a.n_full = (int)(pC & 0x1fffffu); a.n_half = (int)(pC >> 21);
  const unsigned long long t_start = wall_clock64();
  __builtin_amdgcn_sched_barrier(0);       // (the clock read stays at entry)
  __shared__ GemmShared sh;
  __shared__ __align__(16) uint16_t stage_mem[kStageBytes / 2];
  const int nw = (int)((pA >> 8) & 31u);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int j = lane & 15, g = lane >> 4;
  const int KC = a.K >> 5;
  const int cs = a.cs;                          // DBL: nw * NB
  const int n_stages = a.n_stages;
  const int cpws = a.cpws;                      // chunks per wave per stage (multiple of NB; DBL: NB)
  const int cpi = a.cpi;                        // chunks per wave per item (multiple of NB)
  const int stride = cs * 32 + 8;
  const int buf_elems = 2 * a.M * stride;       // one buffer: hi then lo planes
  // stage buffer b (no array of pointers: a runtime index would put it in scratch)
  auto stage_buf = [&](int b) {
    Stage x;
    x.stride = stride;
    x.hi = stage_mem + b * buf_elems;
    x.lo = x.hi + (size_t)a.M * stride;
    return x;
  };
  const ItemPlan<ROLE> ip{a.n_full, a.n_half, G};
  // packed weights are tile-major: chunk kc of tile T is the KiB at (T * KC + kc)
  const uint4* W4 = reinterpret_cast<const uint4*>(a.W);
  // this lane's uint4 inside chunk 0 of item o (a half item's other lanes load its own rows)
  auto item_off = [&](int o) {                 // (past the last item: computed, never loaded)
    int hf;
    const int T = max(ip.tile(o, hf), 0);
    const int ln = hf < 0 ? lane : ((lane & ~8) | (hf << 3));
    return ((size_t)T * KC + wave) * 64 + ln;
  };
  LoadCursor cur{0, 0, item_off(0)};
  // Unconditional: the caller never refills past this workgroup's last item
  // (loads that may or may not be issued would leave the compiler unable to
  // count outstanding loads, and every wait would drain them all).
  auto refill = [&](uint4& slot) {
    slot = ld_stream(W4 + cur.off);
    cur.off += (size_t)nw * 64;
    if (++cur.c == cpi) {
      cur.c = 0;
      cur.T += 1;                               // next item ordinal of this workgroup
      cur.off = item_off(cur.T);
    }
  };
  const bool fast = a.pro_fast != 0;
  ProRegs pr{};
  if (fast) pr = prologue_issue(a, cs, 32, nw * 64, wave, lane, norm_role(ROLE));
  uint4 A[NB];
#pragma unroll
  for (int u = 0; u < NB; ++u) refill(A[u]);     // weights stream from here on (NB <= cpi)
  prof_publish_start(a.prof, t_start);
  row_best_init<ROLE>(a, sh);
  if (fast) {
    prologue_finish(a, stage_buf(0), cs, 32, nw * 64, wave, lane, norm_role(ROLE), pr, sh);
    __syncthreads();
  } else {
    if (norm_role(ROLE)) rows_inv_rms(a, sh, wave, lane, nw);   // read only by the epilogue
    if (n_stages == 1 || DBL) {
      stage_planes(a, stage_buf(0), 0, cs, 32);
      __syncthreads();
    }
  }
  int buf = 0;                                  // DBL: buffer of the current stage

  for (int o = 0;; ++o) {
    int hf;
    const int T = ip.tile(o, hf);
    if (T < 0) break;
    const EpiPre pre = epi_load<ROLE>(a, T, threadIdx.x);
    f32x4 acc[TM];
#pragma unroll
    for (int rt = 0; rt < TM; ++rt) acc[rt] = f32x4{0.f, 0.f, 0.f, 0.f};
    int cl0 = 0, si = 0;                        // position inside the current stage, and its index
    for (int c0 = 0; c0 < cpi; c0 += NB) {
      if (!DBL && n_stages > 1 && cl0 == 0) {
        __syncthreads();
        stage_planes(a, stage_buf(0), si * cs, cs, 32);
        __syncthreads();
      }
      StageRegs sreg{};
      if (DBL) {                                // next stage (cyclically: the next item restarts at 0)
        const int s_next = si + 1;
        sreg = stage_fetch(a, s_next < n_stages ? s_next * cs : 0, cs, 32, nw * 64);
      }
      const Stage st = stage_buf(DBL ? buf : 0);
      // (each of the two copies below ends with its own stage store, so the
      // waits before the store count exactly the loads of that copy)
      auto group = [&](bool refills) {
#pragma unroll
        for (int u = 0; u < NB; ++u) {
          const int kl = (wave + nw * (cl0 + u)) * 32 + g * 8;   // input index inside the stage
#pragma unroll
          for (int rt = 0; rt < TM; ++rt)
            acc[rt] = mfma_pair(A[u], lds_pair(st, row_of(rt * 16 + j, a.M), kl), acc[rt]);
          if (refills) refill(A[u]);
        }
        if (DBL) {
          // the other buffer was last read in the previous stage, before the
          // previous barrier; after this barrier every wave reads the new one
          stage_store(a, stage_buf(buf ^ 1), cs, 32, sreg, &sh.dummy, nw * 64);
          __syncthreads();
        }
      };
      if (ip.has_next(T, hf) || c0 + NB < cpi) group(true);
      else group(false);                        // the last NB chunks of this workgroup
      if (DBL) buf ^= 1;
      cl0 += NB;
      if (cl0 == cpws) { cl0 = 0; ++si; }
    }
    gemm_finish<TM, ROLE>(a, sh, acc, T, wave, lane, nw, pre, hf);
  }
  row_best_publish<ROLE>(a, sh);
  prof_end(a.prof);
}

// bf16, one row tile, each wave's activation operands held in registers:
// wave w only multiplies the input columns of its chain's chunks (w, w + S,
// ...), the same for every item, so it loads those CPW operand pairs once and
// the weight ring streams the workgroup's items through them, with no LDS
// stage and no restaging per item (k_gemm_bf16 restages every item once the
// rows' planes outgrow one stage).  The item plan, the ring, the sums (chain
// w over its chunks in order, hi plane before lo plane, the chain sums met in
// LDS in chain order) and the epilogue are k_gemm_bf16's.  TM = 2 (17..24
// rows of K <= 4096): rows 16.. are staged once into LDS, whole K, and the
// second row tile reads them there.  Leading arguments as k_gemm_bf16's
// (pA, pC of ring_pack).
template <int ROLE, int NB, int CPW, int TM>
__global__ __launch_bounds__(1024) void k_gemm_bf16rb(const void* W, const uint16_t* bhi, const uint16_t* blo,
                                                      const float* ss, int K, int G, unsigned pA, unsigned pC,
                                                      GemmArgs args) {
  static_assert(CPW % NB == 0, "the ring depth divides the chunks per wave");
  static_assert(TM == 1 || TM == 2, "one or two row tiles");
  GemmArgs a = args;
  a.W = W; a.bhi = bhi; a.blo = blo; a.ss = ss; a.K = K;
  a.M = (int)(pA & 127u); a.n_full = (int)(pC & 0x1fffffu); a.n_half = (int)(pC >> 21);
  const unsigned long long t_start = wall_clock64();
  __builtin_amdgcn_sched_barrier(0);       // (the clock read stays at entry)
  __shared__ GemmShared sh;
  __shared__ __align__(16) uint16_t stage_mem[TM == 2 ? kStageBytes / 2 : 8];
  const int nw = (int)((pA >> 8) & 31u);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int j = lane & 15, g = lane >> 4;
  const int KC = a.K >> 5;
  const ItemPlan<ROLE> ip{a.n_full, a.n_half, G};
  // TM = 2: rows 16.. (a2), whole K, one LDS stage
  GemmArgs a2 = a;
  Stage st2{};
  ProRegs pr{};
  if constexpr (TM == 2) {
    a2.bhi = a.bhi + (size_t)16 * a.K;
    a2.blo = a.blo + (size_t)16 * a.K;
    a2.M = a.M - 16;
    st2.stride = KC * 32 + 8;
    st2.hi = stage_mem;
    st2.lo = stage_mem + (size_t)a2.M * st2.stride;
    pr = prologue_issue(a2, KC, 32, nw * 64, wave, lane, false);
  }
  const uint4* W4 = reinterpret_cast<const uint4*>(a.W);
  auto item_off = [&](int o) {                 // (as in k_gemm_bf16)
    int hf;
    const int T = max(ip.tile(o, hf), 0);
    const int ln = hf < 0 ? lane : ((lane & ~8) | (hf << 3));
    return ((size_t)T * KC + wave) * 64 + ln;
  };
  LoadCursor cur{0, 0, item_off(0)};
  auto refill = [&](uint4& slot) {
    slot = ld_stream(W4 + cur.off);
    cur.off += (size_t)nw * 64;
    if (++cur.c == CPW) {
      cur.c = 0;
      cur.T += 1;
      cur.off = item_off(cur.T);
    }
  };
  // this wave's activation operands (row j, clamped), then the row sums of
  // squares (norm roles), then the weights: a wait on the first two never
  // holds the weight ring
  const int r = row_of(j, a.M);
  BPair B[CPW];
#pragma unroll
  for (int c = 0; c < CPW; ++c) B[c] = load_planes(a, r, (wave + nw * c) * 32 + g * 8);
  if constexpr (TM == 2) {
    // the staged rows go to LDS before the weight ring starts (their loads
    // were issued first, so this waits on them alone): held across the ring
    // they would push the registers past the limit
    prologue_finish(a2, st2, KC, 32, nw * 64, wave, lane, false, pr, sh);
  }
  // slices of sums of squares per lane and row: K <= 8192 (two row tiles: K <= 4096)
  constexpr int SSL = TM == 2 ? 4 : 8;
  float s[TM][SSL];
#pragma unroll
  for (int rt = 0; rt < TM; ++rt)
#pragma unroll
    for (int t = 0; t < SSL; ++t) s[rt][t] = 0.f;
  // with 16 waves each wave takes row wave of each row tile, its slices in
  // registers ahead of the ring; fewer waves take rows_inv_rms's loop instead
  const bool ss_regs = norm_role(ROLE) && nw == 16;
  if (ss_regs) {
#pragma unroll
    for (int rt = 0; rt < TM; ++rt)
      if (wave + 16 * rt < a.M) {
#pragma unroll
        for (int t = 0; t < SSL; ++t) s[rt][t] = ss_load(a, wave + 16 * rt, lane, t);
      }
  }
  uint4 A[NB];
#pragma unroll
  for (int u = 0; u < NB; ++u) refill(A[u]);
  prof_publish_start(a.prof, t_start);
  row_best_init<ROLE>(a, sh);
  if (norm_role(ROLE) && !ss_regs) rows_inv_rms(a, sh, wave, lane, nw);
  if (ss_regs) {
#pragma unroll
    for (int rt = 0; rt < TM; ++rt)
      if (wave + 16 * rt < a.M) {
        // the same order as rows_inv_rms: each lane adds its slices in order
        // (the zeros past the row's slices add exactly nothing), then the butterfly
        float v = 0.f;
#pragma unroll
        for (int t = 0; t < SSL; ++t) v = v + s[rt][t];
        v = wave_sum(v);
        if (lane == 0) sh.inv[wave + 16 * rt] = 1.0f / sqrtf(v / (float)a.K + a.eps);
      }
  }
  if constexpr (TM == 2) __syncthreads();
  for (int o = 0;; ++o) {
    int hf;
    const int T = ip.tile(o, hf);
    if (T < 0) break;
    const EpiPre pre = epi_load<ROLE>(a, T, threadIdx.x);
    f32x4 acc[TM];
#pragma unroll
    for (int rt = 0; rt < TM; ++rt) acc[rt] = f32x4{0.f, 0.f, 0.f, 0.f};
    auto group = [&](int c0, bool refills) {
#pragma unroll
      for (int u = 0; u < NB; ++u) {
        acc[0] = mfma_pair(A[u], B[c0 + u], acc[0]);
        if constexpr (TM == 2)
          acc[1] = mfma_pair(A[u], lds_pair(st2, row_of(j, a2.M), (wave + nw * (c0 + u)) * 32 + g * 8), acc[1]);
        if (refills) refill(A[u]);
      }
    };
#pragma unroll
    for (int c0 = 0; c0 + NB < CPW; c0 += NB) group(c0, true);
    if (ip.has_next(T, hf)) group(CPW - NB, true);
    else group(CPW - NB, false);                 // the last NB chunks of this workgroup
    gemm_finish<TM, ROLE>(a, sh, acc, T, wave, lane, nw, pre, hf);
  }
  row_best_publish<ROLE>(a, sh);
  prof_end(a.prof);
}

// int4 weights: wave w takes 128-input tiles w, w + NW, ...; per row tile and
// per scale group, the MFMAs over the group's 64 inputs (hi and lo planes of
// each 32-input chunk) start from zero; the group sum is then scaled by the
// fp32 group scale and added to the running fp32 sum in group order.  The
// weight ring holds each tile's codes and its two groups' scales.
struct Int4Slot {
  uint4 q;
  uint2 s0, s1;
};

template <int TM, int ROLE, int NB>
__global__ __launch_bounds__(1024) void k_gemm_int4(const void* W, const void* Wscale, const uint16_t* bhi,
                                                    const uint16_t* blo, const float* ss, int K, int G, unsigned pA,
                                                    unsigned pB, GemmArgs args) {
  GemmArgs a = args;                    // leading arguments preloaded (ring_pack, as in k_gemm_bf16)
  a.W = W; a.Wscale = Wscale; a.bhi = bhi; a.blo = blo; a.ss = ss; a.K = K;
  a.M = (int)(pA & 127u); a.cpi = (int)((pA >> 13) & 1023u); a.n_stages = (int)(pA >> 23);
  a.cs = (int)(pB & 0xffffu); a.cpws = (int)(pB >> 16);
  const unsigned long long t_start = wall_clock64();
  __builtin_amdgcn_sched_barrier(0);       // (the clock read stays at entry)
  __shared__ GemmShared sh;
  __shared__ __align__(16) uint16_t stage_mem[kStageBytes / 2];
  const int nw = (int)((pA >> 8) & 31u);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int j = lane & 15, g = lane >> 4;
  const int KT = a.K >> 7;                 // 128-input tiles
  const int cs = a.cs;
  const int n_stages = a.n_stages;
  const int cpws = a.cpws;
  const int cpi = a.cpi;
  Stage st;
  st.stride = cs * 128 + 8;
  st.hi = stage_mem;
  st.lo = stage_mem + (size_t)a.M * st.stride;
  const int n_items = a.N >> 4;
  const uint4* Wq = reinterpret_cast<const uint4*>(a.W) + lane;
  const uint2* Ws = reinterpret_cast<const uint2*>(a.Wscale) + g;
  // tile (T, kt): codes at uint4 (T * KT + kt) * 64, scales at uint2 (T * KT + kt) * 8
  LoadCursor cur{(int)blockIdx.x, 0, (size_t)blockIdx.x * KT + wave};
  auto refill = [&](Int4Slot& slot) {   // unconditional, as in the bf16 kernel
    slot.q = ld_stream(Wq + cur.off * 64);
    slot.s0 = Ws[cur.off * 8];
    slot.s1 = Ws[cur.off * 8 + 4];
    cur.off += nw;
    if (++cur.c == cpi) {
      cur.c = 0;
      cur.T += G;
      cur.off = (size_t)cur.T * KT + wave;
    }
  };
  Int4Slot Q[NB];
#pragma unroll
  for (int u = 0; u < NB; ++u) refill(Q[u]);
  prof_publish_start(a.prof, t_start);
  if (norm_role(ROLE)) rows_inv_rms(a, sh, wave, lane, nw);
  if (n_stages == 1) {
    stage_planes(a, st, 0, cs, 128);
    __syncthreads();
  }
  for (int T = blockIdx.x; T < n_items; T += G) {
    const EpiPre pre = epi_load<ROLE>(a, T, threadIdx.x);
    f32x4 acc[TM];
#pragma unroll
    for (int rt = 0; rt < TM; ++rt) acc[rt] = f32x4{0.f, 0.f, 0.f, 0.f};
    int cl0 = 0, si = 0;                    // position inside the current stage, and its index
    for (int c0 = 0; c0 < cpi; c0 += NB) {
      if (n_stages > 1 && cl0 == 0) {
        __syncthreads();
        stage_planes(a, st, si * cs, cs, 128);
        __syncthreads();
      }
      auto group = [&](bool refills) {
#pragma unroll
      for (int u = 0; u < NB; ++u) {
        const int kl = (wave + nw * (cl0 + u)) * 128;      // input index inside the stage
#pragma unroll
        for (int gq = 0; gq < 2; ++gq) {
          const uint2 SC = gq == 0 ? Q[u].s0 : Q[u].s1;
          const uint4 A0 = codes8(gq == 0 ? Q[u].q.x : Q[u].q.z), A1 = codes8(gq == 0 ? Q[u].q.y : Q[u].q.w);
          const float s0 = bf2f((uint16_t)(SC.x & 0xffffu)), s1 = bf2f((uint16_t)(SC.x >> 16));
          const float s2 = bf2f((uint16_t)(SC.y & 0xffffu)), s3 = bf2f((uint16_t)(SC.y >> 16));
#pragma unroll
          for (int rt = 0; rt < TM; ++rt) {
            const int r = row_of(rt * 16 + j, a.M);
            f32x4 p = f32x4{0.f, 0.f, 0.f, 0.f};
            p = mfma_pair(A0, lds_pair(st, r, kl + gq * 64 + g * 8), p);
            p = mfma_pair(A1, lds_pair(st, r, kl + gq * 64 + 32 + g * 8), p);
            acc[rt].x = fmaf(s0, p.x, acc[rt].x);
            acc[rt].y = fmaf(s1, p.y, acc[rt].y);
            acc[rt].z = fmaf(s2, p.z, acc[rt].z);
            acc[rt].w = fmaf(s3, p.w, acc[rt].w);
          }
        }
        if (refills) refill(Q[u]);
      }
      };
      if (T + G < n_items || c0 + NB < cpi) group(true);
      else group(false);
      cl0 += NB;
      if (cl0 == cpws) { cl0 = 0; ++si; }
    }
    gemm_finish<TM, ROLE>(a, sh, acc, T, wave, lane, nw, pre);
  }
  prof_end(a.prof);
}

// int4 weights, one row tile (at most 16 rows), register operands: the
// small int4 matrices are bound by latency, not bytes (a Gemma-shaped layer
// streams 1-10 MB per GEMM), so every load a workgroup needs goes out at
// once -- the codes and scales of all IG items' tiles, then each wave's own
// activation operands (wave w only ever multiplies the input columns of its
// chain's tiles, so nothing is staged in LDS and no barrier comes before
// the MFMAs) -- and the IG items share one reduction.  CPI tiles per wave
// and item; the activation operands of tiles 0 and 1 load up front, those
// of tile c + 2 after tile c's MFMAs.  The sums are k_gemm_int4's: chain w
// runs its tiles in order, per tile the scale groups in order, each group
// summed from zero over its two 32-input chunks (hi plane before lo plane)
// and added to the chain sum scaled by the group scale; the chain sums meet
// in LDS in chain order.
template <int IG, int TM>
struct Int4rShared {
  f32x4 red[IG * TM][kMaxWaves][64];
  float y[IG][16 * TM][16];
  float inv[16 * TM];
};

// The register-operand kernels take the fields they need before their first
// loads as leading scalar arguments (SM packs S | M << 8): the library is
// built so that the hardware loads the first 14 dwords of a kernel's
// arguments (pointers and scalars; a struct is never preloaded) into SGPRs
// before a wave starts, so no wave first waits on a scalar load of its
// argument block.  G is the grid size.  The other fields stay in GemmArgs.
template <int ROLE, int CPI, int IG, int TM>
__global__ __launch_bounds__(768) void k_gemm_int4r(const void* W, const void* Wscale, const uint16_t* bhi,
                                                    const uint16_t* blo, unsigned long long* prof, int N, int K,
                                                    int G, int SM, GemmArgs args) {
  // tiles whose activation operands are held at once (one with two row tiles)
  constexpr int CPA = TM == 2 ? 1 : (CPI < 2 ? CPI : 2);
  GemmArgs a = args;
  a.W = W; a.Wscale = Wscale; a.bhi = bhi; a.blo = blo; a.prof = prof;
  a.N = N; a.K = K; a.S = SM & 0xff; a.M = SM >> 8;
  const unsigned long long t_start = wall_clock64();
  __builtin_amdgcn_sched_barrier(0);       // (the clock read stays at entry)
  __shared__ Int4rShared<IG, TM> sh;
  const int nw = a.S, nthr = 64 * a.S;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int j = lane & 15, g = lane >> 4;
  const int KT = a.K >> 7;
  const int n_items = a.N >> 4;
  int n_my = 1;                            // items of this workgroup, 1..IG (compares, no division)
#pragma unroll
  for (int i = 1; i < IG; ++i) n_my += ((int)blockIdx.x + i * G < n_items) ? 1 : 0;
  int T[IG];
#pragma unroll
  for (int i = 0; i < IG; ++i) T[i] = (int)blockIdx.x + (i < n_my ? i : n_my - 1) * G;
  // codes and scales of every (tile position, item): tile kt = wave + nw c of item T_i
  const uint4* Wq = reinterpret_cast<const uint4*>(a.W) + lane;
  const uint2* Ws = reinterpret_cast<const uint2*>(a.Wscale) + g;
  uint4 q[CPI][IG];
  uint2 s0[CPI][IG], s1[CPI][IG];
#pragma unroll
  for (int c = 0; c < CPI; ++c)
#pragma unroll
    for (int i = 0; i < IG; ++i) {
      const size_t off = (size_t)T[i] * KT + wave + (size_t)nw * c;
      q[c][i] = ld_stream(Wq + off * 64);
      s0[c][i] = Ws[off * 8];
      s1[c][i] = Ws[off * 8 + 4];
    }
  // this lane's activation operands of a tile: row 16 rt + j (clamped), inputs
  // kt*128 + 64 gq + 32 h + 8 g .. +7, hi and lo planes
  auto act = [&](int c, BPair (&B)[TM][2][2]) {
    const int kt = wave + nw * c;
#pragma unroll
    for (int rt = 0; rt < TM; ++rt)
#pragma unroll
      for (int gq = 0; gq < 2; ++gq)
#pragma unroll
        for (int h = 0; h < 2; ++h)
          B[rt][gq][h] = load_planes(a, row_of(rt * 16 + j, a.M), kt * 128 + gq * 64 + h * 32 + g * 8);
  };
  BPair B[CPA][TM][2][2];
#pragma unroll
  for (int c = 0; c < CPA; ++c) act(c, B[c]);
  prof_publish_start(a.prof, t_start);
  if (norm_role(ROLE))
    for (int rr = wave; rr < a.M; rr += nw) {
      const float v = row_inv_rms(a, rr, lane);
      if (lane == 0) sh.inv[rr] = v;
    }
  // epilogue operands of element e of item i, for t = threadIdx.x = i M 16 + e
  const int per_item = a.M * 16;
  const int i_pre = (int)threadIdx.x / per_item;
  const EpiPre pre = epi_load<ROLE>(a, T[i_pre < n_my ? i_pre : 0], (int)threadIdx.x - i_pre * per_item);
  f32x4 acc[IG][TM];
#pragma unroll
  for (int i = 0; i < IG; ++i)
#pragma unroll
    for (int rt = 0; rt < TM; ++rt) acc[i][rt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int c = 0; c < CPI; ++c) {
    BPair (&Bc)[TM][2][2] = B[c % CPA];
#pragma unroll
    for (int i = 0; i < IG; ++i)
#pragma unroll
      for (int gq = 0; gq < 2; ++gq) {
        const uint2 SC = gq == 0 ? s0[c][i] : s1[c][i];
        const uint4 A0 = codes8(gq == 0 ? q[c][i].x : q[c][i].z), A1 = codes8(gq == 0 ? q[c][i].y : q[c][i].w);
        const float f0 = bf2f((uint16_t)(SC.x & 0xffffu)), f1 = bf2f((uint16_t)(SC.x >> 16));
        const float f2 = bf2f((uint16_t)(SC.y & 0xffffu)), f3 = bf2f((uint16_t)(SC.y >> 16));
#pragma unroll
        for (int rt = 0; rt < TM; ++rt) {
          f32x4 p = f32x4{0.f, 0.f, 0.f, 0.f};
          p = mfma_pair(A0, Bc[rt][gq][0], p);
          p = mfma_pair(A1, Bc[rt][gq][1], p);
          acc[i][rt].x = fmaf(f0, p.x, acc[i][rt].x);
          acc[i][rt].y = fmaf(f1, p.y, acc[i][rt].y);
          acc[i][rt].z = fmaf(f2, p.z, acc[i][rt].z);
          acc[i][rt].w = fmaf(f3, p.w, acc[i][rt].w);
        }
      }
    if (c + CPA < CPI) act(c + CPA, Bc);
  }
  // the IG items' chain sums meet in LDS, in chain order (one 16-row tile of
  // one item per 256 threads' pass)
#pragma unroll
  for (int i = 0; i < IG; ++i)
#pragma unroll
    for (int rt = 0; rt < TM; ++rt) sh.red[i * TM + rt][wave][lane] = acc[i][rt];
  __syncthreads();
  for (int t = threadIdx.x; t < IG * TM * 256; t += nthr) {
    const int it = t >> 8, tt = t & 255;
    const int i = it / TM, rt = it - i * TM;
    const float* red = reinterpret_cast<const float*>(sh.red[it]);
    float v = 0.f;
#pragma unroll
    for (int w0 = 0; w0 < kMaxWaves; w0 += 8) {
      float part[8];
#pragma unroll
      for (int w = 0; w < 8; ++w) part[w] = red[(w0 + w) * 256 + tt];
#pragma unroll
      for (int w = 0; w < 8; ++w)
        if (w0 + w < nw) v = (w0 + w == 0) ? part[w] : v + part[w];
    }
    const int l = tt >> 2;
    const int rr = rt * 16 + (l & 15);
    if (rr < a.M) sh.y[i][rr][4 * (l >> 4) + (tt & 3)] = v;
  }
  __syncthreads();
  for (int idx = threadIdx.x; idx < n_my * per_item; idx += nthr) {
    const int i = idx / per_item, e = idx - i * per_item;
    const int rr = e >> 4, cc = e & 15;
    const EpiPre ep = idx == (int)threadIdx.x ? pre : epi_load<ROLE>(a, T[i], e);
    epi_element<ROLE>(a, T[i], rr, cc, ep, sh.inv[rr], [&](int c2) { return sh.y[i][rr][c2]; }, nullptr);
  }
  prof_end(a.prof);
}

// Items per workgroup up to MAXIG (the most whose registers fit without
// spilling at CPI tiles per wave).
template <int ROLE, int CPI, int MAXIG, int TM>
static hipError_t launch_int4r_ig(const GemmArgs& a, int grid, int ig, hipStream_t st) {
  const dim3 block(64 * a.S), g(grid);
  if (ig > MAXIG) return hipErrorNotSupported;
  switch (ig) {
    case 1: hipLaunchKernelGGL((k_gemm_int4r<ROLE, CPI, 1, TM>), g, block, 0, st, a.W, a.Wscale, a.bhi, a.blo, a.prof, a.N, a.K, grid, a.S | (a.M << 8), a); break;
    case 2: hipLaunchKernelGGL((k_gemm_int4r<ROLE, CPI, (MAXIG >= 2 ? 2 : 1), TM>), g, block, 0, st, a.W, a.Wscale, a.bhi, a.blo, a.prof, a.N, a.K, grid, a.S | (a.M << 8), a); break;
    case 3: hipLaunchKernelGGL((k_gemm_int4r<ROLE, CPI, (MAXIG >= 3 ? 3 : 1), TM>), g, block, 0, st, a.W, a.Wscale, a.bhi, a.blo, a.prof, a.N, a.K, grid, a.S | (a.M << 8), a); break;
    case 4: hipLaunchKernelGGL((k_gemm_int4r<ROLE, CPI, (MAXIG >= 4 ? 4 : 1), TM>), g, block, 0, st, a.W, a.Wscale, a.bhi, a.blo, a.prof, a.N, a.K, grid, a.S | (a.M << 8), a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

// The register-operand int4 kernel where it applies (at most 32 rows in one
// or two row tiles, at most 12 waves, 1, 2 or 4 tiles per wave and item, at
// most 4 items per workgroup, 2 at 4 tiles); hipErrorNotSupported otherwise.
template <int ROLE, int TM>
static hipError_t launch_int4r_tm(const GemmArgs& a, int grid, int cpi, int ig, hipStream_t st) {
  switch (cpi) {
    case 1: return launch_int4r_ig<ROLE, 1, 4, TM>(a, grid, ig, st);
    case 2: return launch_int4r_ig<ROLE, 2, (TM == 2 ? 3 : 4), TM>(a, grid, ig, st);   // (4 spill at two tiles)
    case 4: return launch_int4r_ig<ROLE, 4, 2, TM>(a, grid, ig, st);
    default: return hipErrorNotSupported;
  }
}
template <int ROLE>
static hipError_t launch_int4r(const GemmArgs& a, int grid, hipStream_t st) {
  const int cpi = (a.K >> 7) / a.S;
  const int ig = ((a.N >> 4) + grid - 1) / grid;
  if (a.M > 32 || a.S > 12) return hipErrorNotSupported;
  return a.M > 16 ? launch_int4r_tm<ROLE, 2>(a, grid, cpi, ig, st) : launch_int4r_tm<ROLE, 1>(a, grid, cpi, ig, st);
}

// bf16 weights of small K (1, 2 or 4 chunks per wave), one row tile, the
// same register-operand scheme as k_gemm_int4r: the workgroup's IG items'
// chunks and each wave's own activation operands are requested at once, no
// LDS stage, one reduction for the IG items.  The sums are k_gemm_bf16's:
// chain w runs chunks w, w + S, w + 2S, ... in order through one MFMA
// accumulator (hi plane before lo plane), and the S chain sums meet in LDS
// in chain order.  Not for the LM head (its many items per workgroup keep
// the ring kernel).  Measured on MI355X (0.6B shape, K = 4): QKV 7.7 -> 6.0
// us, gate/up 7.8 -> 6.4 us per layer against the ring kernel; at 6 chunks
// per wave (0.6B down) and 8 (8B O) it was no faster, so those keep the ring.
template <int IG>
struct Bf16rShared {
  f32x4 red[IG][kMaxWaves][64];
  float y[IG][16][16];
  float inv[16];
};

template <int ROLE, int CPW, int IG>
__global__ __launch_bounds__(1024) void k_gemm_bf16r(const void* W, const uint16_t* bhi, const uint16_t* blo,
                                                     unsigned long long* prof, int N, int K, int S, int M, int G,
                                                     GemmArgs args) {
  GemmArgs a = args;
  a.W = W; a.bhi = bhi; a.blo = blo; a.prof = prof; a.N = N; a.K = K; a.S = S; a.M = M;
  const unsigned long long t_start = wall_clock64();
  __builtin_amdgcn_sched_barrier(0);       // (the clock read stays at entry)
  __shared__ Bf16rShared<IG> sh;
  const int nw = a.S, nthr = 64 * a.S;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int j = lane & 15, g = lane >> 4;
  const int KC = a.K >> 5;
  const int n_items = a.N >> 4;
  int n_my = 1;                            // items of this workgroup, 1..IG (compares, no division)
#pragma unroll
  for (int i = 1; i < IG; ++i) n_my += ((int)blockIdx.x + i * G < n_items) ? 1 : 0;
  int T[IG];
#pragma unroll
  for (int i = 0; i < IG; ++i) T[i] = (int)blockIdx.x + (i < n_my ? i : n_my - 1) * G;
  const uint4* W4 = reinterpret_cast<const uint4*>(a.W) + lane;
  uint4 A[CPW][IG];
#pragma unroll
  for (int c = 0; c < CPW; ++c)
#pragma unroll
    for (int i = 0; i < IG; ++i) A[c][i] = ld_stream(W4 + ((size_t)T[i] * KC + wave + (size_t)nw * c) * 64);
  const int r = row_of(j, a.M);
  BPair B[CPW];
#pragma unroll
  for (int c = 0; c < CPW; ++c) B[c] = load_planes(a, r, (wave + nw * c) * 32 + g * 8);
  prof_publish_start(a.prof, t_start);
  if (norm_role(ROLE))
    for (int rr = wave; rr < a.M; rr += nw) {
      const float v = row_inv_rms(a, rr, lane);
      if (lane == 0) sh.inv[rr] = v;
    }
  const int per_item = a.M * 16;
  const int i_pre = (int)threadIdx.x / per_item;
  const EpiPre pre = epi_load<ROLE>(a, T[i_pre < n_my ? i_pre : 0], (int)threadIdx.x - i_pre * per_item);
  f32x4 acc[IG];
#pragma unroll
  for (int i = 0; i < IG; ++i) acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int c = 0; c < CPW; ++c)
#pragma unroll
    for (int i = 0; i < IG; ++i) acc[i] = mfma_pair(A[c][i], B[c], acc[i]);
#pragma unroll
  for (int i = 0; i < IG; ++i) sh.red[i][wave][lane] = acc[i];
  __syncthreads();
  for (int t = threadIdx.x; t < IG * 256; t += nthr) {
    const int i = t >> 8, tt = t & 255;
    const float* red = reinterpret_cast<const float*>(sh.red[i]);
    float v = 0.f;
#pragma unroll
    for (int w0 = 0; w0 < kMaxWaves; w0 += 8) {
      float part[8];
#pragma unroll
      for (int w = 0; w < 8; ++w) part[w] = red[(w0 + w) * 256 + tt];
#pragma unroll
      for (int w = 0; w < 8; ++w)
        if (w0 + w < nw) v = (w0 + w == 0) ? part[w] : v + part[w];
    }
    const int l = tt >> 2;
    const int rr = l & 15;
    if (rr < a.M) sh.y[i][rr][4 * (l >> 4) + (tt & 3)] = v;
  }
  __syncthreads();
  for (int idx = threadIdx.x; idx < n_my * per_item; idx += nthr) {
    const int i = idx / per_item, e = idx - i * per_item;
    const int rr = e >> 4, cc = e & 15;
    const EpiPre ep = idx == (int)threadIdx.x ? pre : epi_load<ROLE>(a, T[i], e);
    epi_element<ROLE>(a, T[i], rr, cc, ep, sh.inv[rr], [&](int c2) { return sh.y[i][rr][c2]; }, nullptr);
  }
  prof_end(a.prof);
}

// Items per workgroup up to MAXIG (the most whose registers fit without
// spilling at CPW chunks per wave).
template <int ROLE, int CPW, int MAXIG>
static hipError_t launch_bf16r_ig(const GemmArgs& a, int grid, int ig, hipStream_t st) {
  const dim3 block(64 * a.S), g(grid);
  if (ig > MAXIG) return hipErrorNotSupported;
  switch (ig) {
    case 1: hipLaunchKernelGGL((k_gemm_bf16r<ROLE, CPW, 1>), g, block, 0, st, a.W, a.bhi, a.blo, a.prof, a.N, a.K, a.S, a.M, grid, a); break;
    case 2: hipLaunchKernelGGL((k_gemm_bf16r<ROLE, CPW, (MAXIG >= 2 ? 2 : 1)>), g, block, 0, st, a.W, a.bhi, a.blo, a.prof, a.N, a.K, a.S, a.M, grid, a); break;
    case 3: hipLaunchKernelGGL((k_gemm_bf16r<ROLE, CPW, (MAXIG >= 3 ? 3 : 1)>), g, block, 0, st, a.W, a.bhi, a.blo, a.prof, a.N, a.K, a.S, a.M, grid, a); break;
    default: return hipErrorNotSupported;
  }
  return hipGetLastError();
}

// The register-operand bf16 kernel where it applies (at most 16 rows, 1, 2
// or 4 chunks per wave and item, at most 3 items per workgroup (2 at 4
// chunks), not the LM head); hipErrorNotSupported otherwise.
template <int ROLE>
static hipError_t launch_bf16r(const GemmArgs& a, int grid, hipStream_t st) {
  const int cpw = (a.K >> 5) / a.S;
  const int ig = ((a.N >> 4) + grid - 1) / grid;
  if (ROLE == kRoleLmHead || a.M > 16) return hipErrorNotSupported;
  switch (cpw) {
    case 1: return launch_bf16r_ig<ROLE, 1, 3>(a, grid, ig, st);
    case 2: return launch_bf16r_ig<ROLE, 2, 3>(a, grid, ig, st);
    case 4: return launch_bf16r_ig<ROLE, 4, 2>(a, grid, ig, st);
    default: return hipErrorNotSupported;
  }
}

// bf16 items in groups, stages outermost (17..64 rows whose activation planes
// do not fit one LDS stage): a workgroup takes its items IG at a time and,
// for each stage of one chunk per wave (two LDS buffers; the next stage's
// planes come to registers while this one computes), runs that stage for all
// IG items, so the planes are staged once per group instead of once per
// item, and the weight ring never waits for them.  Wave w still adds chunks
// w, w + NW, w + 2 NW, ... of each item in that order (one per stage) and an
// item's wave partials meet in LDS in wave order: the weight-streaming
// kernel's sums.  Ring slot ig streams item ig of the group; the slots of a
// partial last group re-read the workgroup's last item, and those items are
// not finished.
// Stages of up to 33 rows are double-buffered (the next stage is stored
// while this one is read, one barrier per stage); 34..64 rows fit one buffer,
// so the next stage waits in registers until every wave is done with the
// current one (two barriers per stage).  NREG 16-byte vectors per thread
// carry a stage (M / 8 of them with 16 waves).
struct GrpStageRegs {   // plain members: they stay in registers
  uint4 v0, v1, v2, v3, v4, v5, v6, v7;
};
// 0: the grouped kernel does not apply; 1: double-buffered; 2: single-buffered
__host__ __device__ __forceinline__ int grp_mode(int M, int waves) {
  const size_t one = (size_t)M * (waves * 32 + 8) * 4;
  if (2 * one <= (size_t)kStageBytes && 2 * M * 4 <= 5 * 64) return 1;
  if (one <= (size_t)kStageBytes && 2 * M * 4 <= 8 * 64) return 2;
  return 0;
}

template <int TM, int ROLE, int IG, bool DB>
__global__ __launch_bounds__(1024) void k_gemm_grp(const void* W, const uint16_t* bhi, const uint16_t* blo, int N,
                                                   int K, int M, int S, int G, unsigned g_magic, GemmArgs args) {
  constexpr int NREG = DB ? 5 : 8;
  GemmArgs a = args;                    // leading arguments preloaded (as in k_gemm_bf16)
  a.W = W; a.bhi = bhi; a.blo = blo; a.N = N; a.K = K; a.M = M; a.S = S;
  const unsigned long long t_start = wall_clock64();
  __builtin_amdgcn_sched_barrier(0);       // (the clock read stays at entry)
  __shared__ GemmShared sh;
  __shared__ __align__(16) uint16_t stage_mem[kStageBytes / 2];
  const int nw = a.S, nthr = 64 * a.S;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int j = lane & 15, g = lane >> 4;
  const int KC = a.K >> 5;
  const int n_st = KC / nw;                     // stages of one chunk per wave
  const int stride = nw * 32 + 8;
  const int buf_elems = 2 * a.M * stride;
  auto stage_buf = [&](int b) {
    Stage x;
    x.stride = stride;
    x.hi = stage_mem + b * buf_elems;
    x.lo = x.hi + (size_t)a.M * stride;
    return x;
  };
  auto fetch = [&](int s) {                     // planes of stage s into registers (unconditional loads)
    GrpStageRegs r{};
    r.v0 = *reinterpret_cast<const uint4*>(stage_src(a, s * nw, nw, 32, 0, nthr));
    r.v1 = *reinterpret_cast<const uint4*>(stage_src(a, s * nw, nw, 32, 1, nthr));
    r.v2 = *reinterpret_cast<const uint4*>(stage_src(a, s * nw, nw, 32, 2, nthr));
    r.v3 = *reinterpret_cast<const uint4*>(stage_src(a, s * nw, nw, 32, 3, nthr));
    r.v4 = *reinterpret_cast<const uint4*>(stage_src(a, s * nw, nw, 32, 4, nthr));
    if constexpr (NREG > 5) {
      r.v5 = *reinterpret_cast<const uint4*>(stage_src(a, s * nw, nw, 32, 5, nthr));
      r.v6 = *reinterpret_cast<const uint4*>(stage_src(a, s * nw, nw, 32, 6, nthr));
      r.v7 = *reinterpret_cast<const uint4*>(stage_src(a, s * nw, nw, 32, 7, nthr));
    }
    return r;
  };
  auto store = [&](const Stage& st, const GrpStageRegs& r) {
    stage_put(a, st, nw, 32, 0, r.v0, &sh.dummy, nthr);
    stage_put(a, st, nw, 32, 1, r.v1, &sh.dummy, nthr);
    stage_put(a, st, nw, 32, 2, r.v2, &sh.dummy, nthr);
    stage_put(a, st, nw, 32, 3, r.v3, &sh.dummy, nthr);
    stage_put(a, st, nw, 32, 4, r.v4, &sh.dummy, nthr);
    if constexpr (NREG > 5) {
      stage_put(a, st, nw, 32, 5, r.v5, &sh.dummy, nthr);
      stage_put(a, st, nw, 32, 6, r.v6, &sh.dummy, nthr);
      stage_put(a, st, nw, 32, 7, r.v7, &sh.dummy, nthr);
    }
  };
  const int n_items = a.N >> 4;
  const int n_my = div_m(n_items - 1 - (int)blockIdx.x, G, g_magic) + 1;   // items of this workgroup (>= 1)
  const int n_grp = (n_my + IG - 1) / IG;
  const uint4* W4 = reinterpret_cast<const uint4*>(a.W) + lane;
  auto item_of = [&](int grp, int ig) {
    const int k = grp * IG + ig;
    return (int)blockIdx.x + (k < n_my ? k : n_my - 1) * G;
  };
  auto chunk = [&](int grp, int s, int ig) {   // chunk wave + nw s of slot ig's item
    return ld_stream(W4 + ((size_t)item_of(grp, ig) * KC + wave + (size_t)nw * s) * 64);
  };

  GrpStageRegs sr = fetch(0);
  uint4 A[IG];
#pragma unroll
  for (int ig = 0; ig < IG; ++ig) A[ig] = chunk(0, 0, ig);
  prof_publish_start(a.prof, t_start);
  row_best_init<ROLE>(a, sh);
  if (norm_role(ROLE)) rows_inv_rms(a, sh, wave, lane, nw);   // read only by the epilogue
  store(stage_buf(0), sr);
  __syncthreads();
  int buf = 0;
  for (int grp = 0; grp < n_grp; ++grp) {
    EpiPre pre[IG];
#pragma unroll
    for (int ig = 0; ig < IG; ++ig) pre[ig] = epi_load<ROLE>(a, item_of(grp, ig), threadIdx.x);
    f32x4 acc[IG][TM];
#pragma unroll
    for (int ig = 0; ig < IG; ++ig)
#pragma unroll
      for (int rt = 0; rt < TM; ++rt) acc[ig][rt] = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int s = 0; s < n_st; ++s) {
      // the ring's next round: the next stage of this group, else stage 0 of
      // the next group, else (end of the stream) this round again
      int gn = grp, sn = s + 1;
      if (sn == n_st) {
        sn = 0;
        gn = grp + 1;
        if (gn == n_grp) {
          gn = grp;
          sn = s;
        }
      }
      sr = fetch(s + 1 < n_st ? s + 1 : 0);
      const Stage st = stage_buf(DB ? buf : 0);
      const int kl = wave * 32 + g * 8;         // this wave's chunk inside the stage
#pragma unroll
      for (int ig = 0; ig < IG; ++ig) {
#pragma unroll
        for (int rt = 0; rt < TM; ++rt)
          acc[ig][rt] = mfma_pair(A[ig], lds_pair(st, row_of(rt * 16 + j, a.M), kl), acc[ig][rt]);
        A[ig] = chunk(gn, sn, ig);
      }
      if constexpr (DB) {
        // the other buffer was last read in the previous stage, before the
        // previous barrier; after this barrier every wave reads the new one
        store(stage_buf(buf ^ 1), sr);
        __syncthreads();
        buf ^= 1;
      } else {
        __syncthreads();                        // every wave is done with the stage
        store(stage_buf(0), sr);
        __syncthreads();
      }
    }
#pragma unroll
    for (int ig = 0; ig < IG; ++ig)
      if (grp * IG + ig < n_my) gemm_finish<TM, ROLE>(a, sh, acc[ig], item_of(grp, ig), wave, lane, nw, pre[ig]);
  }
  row_best_publish<ROLE>(a, sh);
  prof_end(a.prof);
}

// Group size: up to the workgroup's item count, capped where the
// accumulators, ring slots and epilogue prefetches still fit 128 VGPRs
// without spilling (4 for one row tile, 2 for two or three; QKV, whose
// epilogue prefetch is largest, one less step).
template <int TM, int ROLE>
constexpr int grp_max_items() {
  return TM == 1 ? (ROLE == kRoleQkv ? 2 : 4) : (TM == 2 ? 2 : (ROLE == kRoleQkv ? 1 : 2));
}
template <int TM, int ROLE, bool DB>
static void launch_grp(const GemmArgs& a, int grid, int per, hipStream_t st) {
  // single-buffered stages hold 8 registers of planes: groups of two fit the LM head's three row tiles only
  constexpr int IGM = DB ? grp_max_items<TM, ROLE>() : (TM == 3 && ROLE == kRoleLmHead ? 2 : 1);
  const dim3 block(64 * a.S), g(grid);
  if (IGM >= 4 && per >= 4) hipLaunchKernelGGL((k_gemm_grp<TM, ROLE, (IGM >= 4 ? 4 : 1), DB>), g, block, 0, st, a.W, a.bhi, a.blo, a.N, a.K, a.M, a.S, grid, div_magic(grid), a);
  else if (IGM >= 2 && per >= 2) hipLaunchKernelGGL((k_gemm_grp<TM, ROLE, (IGM >= 2 ? 2 : 1), DB>), g, block, 0, st, a.W, a.bhi, a.blo, a.N, a.K, a.M, a.S, grid, div_magic(grid), a);
  else hipLaunchKernelGGL((k_gemm_grp<TM, ROLE, 1, DB>), g, block, 0, st, a.W, a.bhi, a.blo, a.N, a.K, a.M, a.S, grid, div_magic(grid), a);
}
// The packed leading arguments of k_gemm_bf16; false if a field does not fit
// its bits (no supported shape comes near: M <= 64, at most 16 waves).
struct RingPack {
  unsigned a = 0, b = 0, c = 0;
};
static bool ring_pack(const GemmArgs& a, RingPack& p) {
  if (a.M < 1 || a.M > 127 || a.S < 1 || a.S > 31 || a.cpi < 0 || a.cpi > 1023 || a.n_stages < 0 ||
      a.n_stages > 511 || a.cs < 0 || a.cs > 0xffff || a.cpws < 0 || a.cpws > 0xffff || a.n_full < 0 ||
      a.n_full > 0x1fffff || a.n_half < 0 || a.n_half > 2047 || (a.pro_fast != 0 && a.pro_fast != 1))
    return false;
  p.a = (unsigned)a.M | ((unsigned)a.pro_fast << 7) | ((unsigned)a.S << 8) | ((unsigned)a.cpi << 13) |
        ((unsigned)a.n_stages << 23);
  p.b = (unsigned)a.cs | ((unsigned)a.cpws << 16);
  p.c = (unsigned)a.n_full | ((unsigned)a.n_half << 21);
  return true;
}

template <int ROLE>
static hipError_t gemm_dispatch_grp(const GemmArgs& a, int grid, hipStream_t st) {
  const int tm = (a.M + 15) / 16;
  const int per = ((a.N >> 4) + grid - 1) / grid;   // most items of one workgroup
  if (grp_mode(a.M, a.S) == 1) {
    if (tm == 2) launch_grp<2, ROLE, true>(a, grid, per, st);
    else if (tm == 3) launch_grp<3, ROLE, true>(a, grid, per, st);
    else return hipErrorInvalidValue;
  } else {
    if (tm == 4) launch_grp<4, ROLE, false>(a, grid, per, st);
    else if (tm == 3) launch_grp<3, ROLE, false>(a, grid, per, st);
    else return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <int ROLE, bool INT4, int NB>
static hipError_t gemm_dispatch_nb(const GemmArgs& a, int grid, hipStream_t st, bool dbl) {
  const dim3 block(64 * a.S);
  const int tm = (a.M + 15) / 16;
  RingPack rp;
  if (!ring_pack(a, rp)) return hipErrorInvalidValue;
  if constexpr (INT4) {
    // only the (rows, ring depth) pairs gemm_ring_depth can pick are built
    switch (tm) {
      case 1: hipLaunchKernelGGL((k_gemm_int4<1, ROLE, NB>), dim3(grid), block, 0, st, a.W, a.Wscale, a.bhi, a.blo, a.ss, a.K, grid, rp.a, rp.b, a); break;
      case 2:
        if constexpr (NB <= 2) hipLaunchKernelGGL((k_gemm_int4<2, ROLE, NB>), dim3(grid), block, 0, st, a.W, a.Wscale, a.bhi, a.blo, a.ss, a.K, grid, rp.a, rp.b, a);
        else return hipErrorInvalidValue;
        break;
      case 3:
        if constexpr (NB == 1) hipLaunchKernelGGL((k_gemm_int4<3, ROLE, NB>), dim3(grid), block, 0, st, a.W, a.Wscale, a.bhi, a.blo, a.ss, a.K, grid, rp.a, rp.b, a);
        else return hipErrorInvalidValue;
        break;
      case 4:
        if constexpr (NB == 1) hipLaunchKernelGGL((k_gemm_int4<4, ROLE, NB>), dim3(grid), block, 0, st, a.W, a.Wscale, a.bhi, a.blo, a.ss, a.K, grid, rp.a, rp.b, a);
        else return hipErrorInvalidValue;
        break;
      default: return hipErrorInvalidValue;
    }
  } else {
    switch (tm) {
      case 1:
        if (dbl) {
          if constexpr (NB == 4 || NB == 8) hipLaunchKernelGGL((k_gemm_bf16<1, ROLE, NB, true>), dim3(grid), block, 0, st, a.W, a.bhi, a.blo, a.ss, a.K, grid, rp.a, rp.b, rp.c, a);
          else return hipErrorInvalidValue;
        } else {
          hipLaunchKernelGGL((k_gemm_bf16<1, ROLE, NB, false>), dim3(grid), block, 0, st, a.W, a.bhi, a.blo, a.ss, a.K, grid, rp.a, rp.b, rp.c, a);
        }
        break;
      case 2:
        if constexpr (NB == 3 || NB == 6) {
          return hipErrorInvalidValue;
        } else {
          if (dbl) return hipErrorInvalidValue;
          hipLaunchKernelGGL((k_gemm_bf16<2, ROLE, NB, false>), dim3(grid), block, 0, st, a.W, a.bhi, a.blo, a.ss, a.K, grid, rp.a, rp.b, rp.c, a);
        }
        break;
      case 3:
        if constexpr (NB <= 4 && NB != 3) {
          if (dbl) return hipErrorInvalidValue;
          hipLaunchKernelGGL((k_gemm_bf16<3, ROLE, NB, false>), dim3(grid), block, 0, st, a.W, a.bhi, a.blo, a.ss, a.K, grid, rp.a, rp.b, rp.c, a);
        } else {
          return hipErrorInvalidValue;
        }
        break;
      case 4:
        if constexpr (NB == 1) {
          if (dbl) return hipErrorInvalidValue;
          hipLaunchKernelGGL((k_gemm_bf16<4, ROLE, NB, false>), dim3(grid), block, 0, st, a.W, a.bhi, a.blo, a.ss, a.K, grid, rp.a, rp.b, rp.c, a);
        } else {
          return hipErrorInvalidValue;
        }
        break;
      default: return hipErrorInvalidValue;
    }
  }
  return hipGetLastError();
}

// Ring depth: the deepest of 8 / 4 / 2 / 1 that divides the chunks each wave
// takes per item and per LDS stage (int4: capped by the row count, so its
// registers fit).  *dbl: double-buffered stages (bf16, one row tile, when K
// does not fit one stage), preferred over single-buffered restaging.
int gemm_ring_depth(int n_chunks, int waves, int M, int unit, bool* dbl) {
  *dbl = false;
  const int nthreads = 64 * waves;
  if (unit == 32 && M <= 16 && stage_chunks(n_chunks, waves, M, unit, 1) < n_chunks) {
    for (int nb : {8, 4}) {
      if ((n_chunks / waves) % nb) continue;
      if (stage_double_ok(n_chunks, waves, M, unit, nb, nthreads)) {
        *dbl = true;
        return nb;
      }
    }
  }
  // register budget: bf16 rings are 8 deep up to 32 rows, 4 up to 48, then
  // 1; int4 ring slots also hold scales: 4 deep up to 16 rows, 2 up to 32,
  // then 1
  const int cap = unit == 128 ? (M <= 16 ? 4 : (M <= 32 ? 2 : 1)) : (M <= 32 ? 8 : (M <= 48 ? 4 : 1));
  // bf16 at one row tile also takes rings of 6 and 3 (chunks per wave that 8
  // and 4 do not divide: 96 chunks over 16 waves, 48 over 16)
  for (int nb : {8, 6, 4, 3, 2, 1}) {
    if (nb > cap || ((nb == 6 || nb == 3) && (unit != 32 || M > 16))) continue;
    if ((n_chunks / waves) % nb) continue;
    const int cs = stage_chunks(n_chunks, waves, M, unit, nb);
    if (cs > 0) return nb;
  }
  return 0;
}

// 0: never, 1: when the planes take more than one stage, 2: at one row tile
constexpr int kRbMode = 1;

template <int ROLE, int TM>
static hipError_t launch_bf16rb(const GemmArgs& a, int grid, int nb, hipStream_t st) {
  RingPack rp;
  if (!ring_pack(a, rp)) return hipErrorInvalidValue;
  const dim3 block(64 * a.S), g(grid);
#define SV_RB(NB_, CPW_) hipLaunchKernelGGL((k_gemm_bf16rb<ROLE, NB_, CPW_, TM>), g, block, 0, st, a.W, a.bhi, a.blo, a.ss, a.K, grid, rp.a, rp.c, a)
  (void)nb;                      // the ring holds a wave's whole item (no stage bounds it)
  switch (a.cpi) {
    case 8:                      // (QKV: a ring of 4, two row tiles: of 2, as deeper ones spill)
      if constexpr (TM == 2) SV_RB(2, 8);
      else if constexpr (ROLE == kRoleQkv) SV_RB(4, 8);
      else SV_RB(8, 8);
      break;
    case 4: SV_RB(4, 4); break;
    case 2: SV_RB(2, 2); break;
    case 1: SV_RB(1, 1); break;
    default: return hipErrorNotSupported;
  }
#undef SV_RB
  return hipGetLastError();
}

template <int ROLE, bool INT4>
static hipError_t gemm_dispatch(const GemmArgs& a_in, int grid, hipStream_t st) {
  bool dbl = false;
  const int unit = INT4 ? 128 : 32, n_chunks = a_in.K / unit, nw = a_in.S;
  const int nb = gemm_ring_depth(n_chunks, nw, a_in.M, unit, &dbl);
  if (nb < 1) return hipErrorInvalidValue;
  GemmArgs a = a_in;
  a.cs = dbl ? nw * nb : stage_chunks(n_chunks, nw, a.M, unit, nb);
  a.n_stages = n_chunks / a.cs;
  a.cpws = a.cs / nw;
  a.cpi = n_chunks / nw;
  a.pro_fast = !INT4 && (a.n_stages == 1 || dbl) && prologue_fast(a, a.cs, unit, nw, norm_role(ROLE));
  if constexpr (!INT4) {
    // one row tile whose planes take more than one stage: the register-operand
    // ring (at most 8 chunks per wave, the sums of squares of K <= 8192 rows)
    if (kRbMode > 0 && a.M <= 16 && a.cpi <= 8 && (a.n_stages > 1 || kRbMode > 1) && a.K <= 8192) {
      const hipError_t e = launch_bf16rb<ROLE, 1>(a, grid, nb, st);
      if (e != hipErrorNotSupported) return e;
    }
  }
  switch (nb) {
    case 8:
      if constexpr (INT4) return hipErrorInvalidValue;
      else return gemm_dispatch_nb<ROLE, INT4, 8>(a, grid, st, dbl);
    case 6:
      if constexpr (INT4) return hipErrorInvalidValue;
      else return gemm_dispatch_nb<ROLE, INT4, 6>(a, grid, st, dbl);
    case 3:
      if constexpr (INT4) return hipErrorInvalidValue;
      else return gemm_dispatch_nb<ROLE, INT4, 3>(a, grid, st, dbl);
    case 4: return gemm_dispatch_nb<ROLE, INT4, 4>(a, grid, st, dbl);
    case 2: return gemm_dispatch_nb<ROLE, INT4, 2>(a, grid, st, dbl);
    case 1: return gemm_dispatch_nb<ROLE, INT4, 1>(a, grid, st, dbl);
    default: return hipErrorInvalidValue;
  }
}

// a.S: waves splitting K inside one workgroup (fixed per matrix, 1..16);
// grid: workgroups (each loops over items); any grid gives the same bits.
hipError_t launch_gemm(const GemmArgs& a, int role, int grid, hipStream_t st) {
  if (a.M < 1 || a.M > kMaxRows || a.S < 1 || a.S > kMaxWaves || a.N % 16 || grid < 1) return hipErrorInvalidValue;
  if (a.fmt == 1 ? (a.K % (128 * a.S)) : (a.K % (32 * a.S))) return hipErrorInvalidValue;
  // the smallest activation stage (one chunk per wave) must fit the LDS budget
  if (a.M > gemm_max_rows(a.fmt == 1 ? 128 : 32, a.S)) return hipErrorInvalidValue;
  grid = grid > (a.N >> 4) ? (a.N >> 4) : grid;
  const bool i4 = a.fmt == 1;
  // item plan of k_gemm_bf16 (QKV splits the last round's items into halves
  // when that spreads them over at most every workgroup)
  GemmArgs b = a;
  const int n_items = a.N >> 4, r = n_items % grid;
  const bool split = role == kRoleQkv && r > 0 && 2 * r <= grid;
  b.n_full = split ? n_items - r : n_items;
  b.n_half = split ? 2 * r : 0;
  // 17..64 rows whose bf16 planes do not fit one stage: items in groups,
  // stages outermost (9..16 rows whose planes take more than one stage run
  // k_gemm_bf16rb).  Measured on the 8B shape, batch of 8 sequences (about
  // 39 rows): the grouped kernel 9.61 against 10.0 ms per step for the
  // restaging ring kernel, whose ring is one chunk deep at 34..48 rows.
  // 17..24 rows: the register-operand ring with rows 16.. in one LDS stage
  // (at most 8 chunks per wave, K <= 4096; the staged rows' planes fit the
  // stage and the fast prologue).  Measured on the 8B shape at 17 rows: O,
  // gate/up, down and the LM head gain (K = 16 step 5.556 -> 5.052 ms), QKV
  // (a ring of 2 and a spill at two tiles) was slower and keeps the grouped
  // kernel.
  if (!i4 && kRbMode > 0 && a.M >= 17 && a.M <= 24 && (a.K >> 5) / a.S <= 8 && a.K <= 4096) {
    GemmArgs c = b;
    c.cpi = (a.K >> 5) / a.S;
    c.cs = c.cpws = c.n_stages = c.pro_fast = 0;
    GemmArgs rest = c;
    rest.M = a.M - 16;
    if ((size_t)rest.M * ((size_t)a.K + 8) * 4 <= (size_t)kStageBytes && prologue_fast(rest, a.K >> 5, 32, a.S, false)) {
      hipError_t e = hipErrorNotSupported;
      switch (role) {
        case kRoleO: e = launch_bf16rb<kRoleO, 2>(c, grid, 0, st); break;
        case kRoleGateUp: e = launch_bf16rb<kRoleGateUp, 2>(c, grid, 0, st); break;
        case kRoleDown: e = launch_bf16rb<kRoleDown, 2>(c, grid, 0, st); break;
        case kRoleLmHead: e = launch_bf16rb<kRoleLmHead, 2>(c, grid, 0, st); break;
        default: break;
      }
      if (e != hipErrorNotSupported) return e;
    }
  }
  const int mode = grp_mode(a.M, a.S);
  const bool grp = mode != 0;
  if (!i4 && a.M >= 17 && grp && stage_chunks(a.K >> 5, a.S, a.M, 32, 1) < (a.K >> 5)) {
    switch (role) {
      case kRoleQkv: return gemm_dispatch_grp<kRoleQkv>(b, grid, st);
      case kRoleO: return gemm_dispatch_grp<kRoleO>(b, grid, st);
      case kRoleGateUp: return gemm_dispatch_grp<kRoleGateUp>(b, grid, st);
      case kRoleDown: return gemm_dispatch_grp<kRoleDown>(b, grid, st);
      case kRoleLmHead: return gemm_dispatch_grp<kRoleLmHead>(b, grid, st);
      default: return hipErrorInvalidValue;
    }
  }
  if (!i4 && a.M <= 16) {
    hipError_t e = hipErrorNotSupported;
    switch (role) {
      case kRoleQkv: e = launch_bf16r<kRoleQkv>(b, grid, st); break;
      case kRoleO: e = launch_bf16r<kRoleO>(b, grid, st); break;
      case kRoleGateUp: e = launch_bf16r<kRoleGateUp>(b, grid, st); break;
      case kRoleDown: e = launch_bf16r<kRoleDown>(b, grid, st); break;
      default: break;
    }
    if (e != hipErrorNotSupported) return e;
  }
  if (i4 && a.M <= 32) {
    hipError_t e = hipErrorNotSupported;
    switch (role) {
      case kRoleQkv: e = launch_int4r<kRoleQkv>(b, grid, st); break;
      case kRoleO: e = launch_int4r<kRoleO>(b, grid, st); break;
      case kRoleGateUp: e = launch_int4r<kRoleGateUp>(b, grid, st); break;
      case kRoleDown: e = launch_int4r<kRoleDown>(b, grid, st); break;
      default: break;
    }
    if (e != hipErrorNotSupported) return e;
  }
  switch (role) {
    case kRoleQkv: return i4 ? gemm_dispatch<kRoleQkv, true>(b, grid, st) : gemm_dispatch<kRoleQkv, false>(b, grid, st);
    case kRoleO: return i4 ? gemm_dispatch<kRoleO, true>(b, grid, st) : gemm_dispatch<kRoleO, false>(b, grid, st);
    case kRoleGateUp:
      return i4 ? gemm_dispatch<kRoleGateUp, true>(b, grid, st) : gemm_dispatch<kRoleGateUp, false>(b, grid, st);
    case kRoleDown: return i4 ? gemm_dispatch<kRoleDown, true>(b, grid, st) : gemm_dispatch<kRoleDown, false>(b, grid, st);
    case kRoleLmHead:
      if (i4) return hipErrorInvalidValue;
      return gemm_dispatch<kRoleLmHead, false>(b, grid, st);
    default: return hipErrorInvalidValue;
  }
}

// ------------------------------------------------------------ tiled GEMM (many rows)
// The same sums as the weight-streaming kernels, for forwards of many rows
// (prefill chunks).  Per output, chain w (w < S) adds chunks w, w + S,
// w + 2S, ... in that order through one MFMA accumulator (hi plane before lo
// plane), and the S chain sums are added in chain order: in the
// weight-streaming kernel chain w is wave w and the chains meet in LDS; here
// every wave runs all S chains in turn for its own output tile, keeping the
// running chain sum in registers.  So all waves of a workgroup walk one
// chunk sequence (chain 0's chunks, then chain 1's, ...) and share each
// chunk's weights and activations through LDS, and each weight tile is read
// from HBM once per row block instead of once per 64 rows.
//
// Workgroup: 4 waves and a tile of 128 rows x 8 items (128 outputs); wave
// (wr, wc) owns rows 64 wr .. +63 and items 4 wc .. +3 (4 x 4 MFMA tiles).
// One chunk per pipeline step: its activation planes (128 rows x 32 inputs,
// stored in MFMA operand order) and its 8 weight tiles (1 KiB each, already
// in operand order) are fetched to registers one step ahead and written to
// the other of two LDS buffers; one barrier per step.  Rows past M read row
// M - 1 (their MFMA columns are dropped) and items past N read the last item
// (their outputs are not stored).
constexpr int kTileRows = 128, kTileItems = 8;
constexpr int kTileActVecs = kTileRows * 4;                       // 16-byte vectors of one plane of one step
constexpr int kTileStepVecs = 2 * kTileActVecs + kTileItems * 64;  // hi, lo, weights: 1536 (24 KiB)

struct TileShared {
  float inv[kTileRows];
  unsigned long long best[kTileRows];
};

// Slot of activation vector (row tile row `row`, 8-input group q) inside its
// 64-vector row tile.  An MFMA operand read has lane l take group l / 16 of
// row l % 16; a staging store has 4 neighbouring lanes take the 4 groups of
// one row.  XORing the row with a per-group constant keeps every aligned run
// of 8 (and of 16) lanes on distinct 16-byte bank groups in both patterns.
__device__ __forceinline__ int act_slot(int q, int row) {
  return q * 16 + (row ^ ((q & 1 ? 10 : 0) ^ (q & 2 ? 4 : 0)));
}

struct TileRegs {   // one step of this thread's loads (plain members: they stay in registers)
  uint4 h0, h1, l0, l1, w0, w1;
};

// Workgroup -> (row block, column block) of the tiled GEMMs.  Workgroups
// are dealt to the 8 XCDs round-robin; each XCD gets a contiguous range of
// the column-major (column block, row block) order, so the row blocks of one
// column block run side by side on one XCD and read its weight tiles through
// one L2.
__device__ __forceinline__ void tiled_block(int M, int n_items, int& r0, int& T0) {
  const int n_rb = (M + kTileRows - 1) / kTileRows;
  const int n_cb = (n_items + kTileItems - 1) / kTileItems;
  const int nblk = n_rb * n_cb;
  const int q8 = nblk >> 3, rem = nblk & 7, xcd = blockIdx.x & 7, loc = blockIdx.x >> 3;
  const int lin = (xcd < rem ? xcd * (q8 + 1) : rem * (q8 + 1) + (xcd - rem) * q8) + loc;
  r0 = (lin % n_rb) * kTileRows;
  T0 = (lin / n_rb) * kTileItems;
}

// Epilogue of a tiled workgroup, two items per wave at a time: the wave's
// finished sums go to its own LDS slice of 64 rows x (2 items x 16 + 4 pad)
// floats (lds: at least 4 x 9 KiB, free once the K loop's last barrier has
// passed; the pad spreads the 16 rows of one MFMA store over distinct
// banks), then 16-lane groups run the shared element epilogue row by row.
template <int ROLE>
__device__ __forceinline__ void tiled_epilogue(const GemmArgs& a, TileShared& sh, float* lds, const f32x4 (&y)[4][4],
                                               int r0, int T0, int wave, int lane) {
  const int wr = wave >> 1, wc = wave & 1;
  const int n_items = a.N >> 4;
  constexpr int kRowF = 2 * 16 + 4;
  float* ys = lds + wave * 64 * kRowF;
#pragma unroll
  for (int p = 0; p < 2; ++p) {
#pragma unroll
    for (int rt = 0; rt < 4; ++rt)
#pragma unroll
      for (int c2 = 0; c2 < 2; ++c2) {
        const f32x4 v = y[rt][2 * p + c2];
        *reinterpret_cast<float4*>(ys + (rt * 16 + (lane & 15)) * kRowF + c2 * 16 + 4 * (lane >> 4)) =
            make_float4(v.x, v.y, v.z, v.w);
      }
    __syncthreads();
    for (int it = 0; it < 32; ++it) {
      const int idx = it * 64 + lane;
      const int c2 = idx >> 10, rl = (idx >> 4) & 63, cc = idx & 15;
      const int r = r0 + wr * 64 + rl, T = T0 + wc * 4 + 2 * p + c2;
      if (r < a.M && T < n_items) {
        const float* yr = ys + rl * kRowF + c2 * 16;
        const int rs = wr * 64 + rl;
        epi_element<ROLE>(a, T, r, cc, epi_load<ROLE>(a, T, r * 16 + cc), sh.inv[rs],
                          [&](int k) { return yr[k]; }, &sh.best[rs]);
      }
    }
    __syncthreads();
  }
  if (ROLE == kRoleLmHead && threadIdx.x < kTileRows && r0 + (int)threadIdx.x < a.M)
    atomicMax(a.best + r0 + threadIdx.x, sh.best[threadIdx.x]);
}

// RMS scales of the tile's rows and the LM head's row keys, before the K loop.
template <int ROLE>
__device__ __forceinline__ void tiled_prologue(const GemmArgs& a, TileShared& sh, int r0, int wave, int lane) {
  if (norm_role(ROLE))
    for (int rl = wave; rl < kTileRows; rl += 4) {
      const float v = r0 + rl < a.M ? row_inv_rms(a, r0 + rl, lane) : 0.f;
      if (lane == 0) sh.inv[rl] = v;
    }
  if (ROLE == kRoleLmHead && threadIdx.x < kTileRows) sh.best[threadIdx.x] = 0ull;
}

template <int ROLE>
__global__ __launch_bounds__(256, 2) void k_gemm_tiled(GemmArgs a) {
  __shared__ TileShared sh;
  __shared__ uint4 lds[2 * kTileStepVecs];
  prof_start(a.prof);
  const int t = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6), lane = t & 63;
  const int wr = wave >> 1, wc = wave & 1;
  const int n_items = a.N >> 4;
  int r0, T0;
  tiled_block(a.M, n_items, r0, T0);
  const int KC = a.K >> 5, S = a.S, cpi = KC / S;

  // this thread's vectors of a step: activation vector v = t + 256 i (row
  // v / 4, inputs 8 (v % 4) ..) of each plane, weight vector t + 256 i
  size_t asrc0, asrc1;
  int adst0, adst1;
  {
    const int v0 = t, v1 = t + 256;
    const int rr0 = v0 >> 2, rr1 = v1 >> 2;
    asrc0 = (size_t)min(r0 + rr0, a.M - 1) * a.K + (v0 & 3) * 8;
    asrc1 = (size_t)min(r0 + rr1, a.M - 1) * a.K + (v1 & 3) * 8;
    adst0 = (rr0 >> 4) * 64 + act_slot(v0 & 3, rr0 & 15);
    adst1 = (rr1 >> 4) * 64 + act_slot(v1 & 3, rr1 & 15);
  }
  const uint4* W4 = reinterpret_cast<const uint4*>(a.W);
  const size_t wsrc0 = (size_t)min(T0 + (t >> 6), n_items - 1) * KC * 64 + (t & 63);
  const size_t wsrc1 = (size_t)min(T0 + ((t + 256) >> 6), n_items - 1) * KC * 64 + (t & 63);
  auto fetch = [&](int kc) {
    TileRegs g;
    const size_t ko = (size_t)kc * 32;
    g.h0 = *reinterpret_cast<const uint4*>(a.bhi + asrc0 + ko);
    g.h1 = *reinterpret_cast<const uint4*>(a.bhi + asrc1 + ko);
    g.l0 = *reinterpret_cast<const uint4*>(a.blo + asrc0 + ko);
    g.l1 = *reinterpret_cast<const uint4*>(a.blo + asrc1 + ko);
    g.w0 = W4[wsrc0 + (size_t)kc * 64];
    g.w1 = W4[wsrc1 + (size_t)kc * 64];
    return g;
  };
  auto put = [&](int b, const TileRegs& g) {
    uint4* B = lds + b * kTileStepVecs;
    B[adst0] = g.h0;
    B[adst1] = g.h1;
    B[kTileActVecs + adst0] = g.l0;
    B[kTileActVecs + adst1] = g.l1;
    B[2 * kTileActVecs + t] = g.w0;
    B[2 * kTileActVecs + 256 + t] = g.w1;
  };

  // step s runs chunk (s / cpi) + S (s % cpi): chain s / cpi, position s % cpi
  // (steps past the end fetch the last chunk again: the loads stay unconditional)
  auto chunk_of = [&](int s) {
    s = min(s, KC - 1);
    return s / cpi + S * (s % cpi);
  };
  put(0, fetch(chunk_of(0)));
  TileRegs g1 = fetch(chunk_of(1));
  tiled_prologue<ROLE>(a, sh, r0, wave, lane);
  __syncthreads();

  f32x4 acc[4][4], y[4][4];
#pragma unroll
  for (int rt = 0; rt < 4; ++rt)
#pragma unroll
    for (int ct = 0; ct < 4; ++ct) {
      acc[rt][ct] = f32x4{0.f, 0.f, 0.f, 0.f};
      y[rt][ct] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
  const int aslot = act_slot(lane >> 4, lane & 15);
  auto compute = [&](int s) {
    const uint4* B = lds + (s & 1) * kTileStepVecs;
    uint4 A[4];
#pragma unroll
    for (int ct = 0; ct < 4; ++ct) A[ct] = B[2 * kTileActVecs + (wc * 4 + ct) * 64 + lane];
#pragma unroll
    for (int rt = 0; rt < 4; ++rt) {
      const BPair bp{B[(wr * 4 + rt) * 64 + aslot], B[kTileActVecs + (wr * 4 + rt) * 64 + aslot]};
#pragma unroll
      for (int ct = 0; ct < 4; ++ct) acc[rt][ct] = mfma_pair(A[ct], bp, acc[rt][ct]);
    }
    if (s % cpi == cpi - 1) {   // chain s / cpi complete: add it to the running sum in chain order
      const bool first = s < cpi;
#pragma unroll
      for (int rt = 0; rt < 4; ++rt)
#pragma unroll
        for (int ct = 0; ct < 4; ++ct) {
          y[rt][ct] = first ? acc[rt][ct] : y[rt][ct] + acc[rt][ct];
          acc[rt][ct] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
    }
  };
  // Two steps in flight: while step s computes from LDS buffer s % 2, the
  // loads of step s + 2 are issued and those of step s + 1 (issued one step
  // earlier) are stored to the other buffer; one barrier per step.
  for (int s = 0; s < KC; s += 2) {
    const TileRegs g0 = fetch(chunk_of(s + 2));
    compute(s);
    put(1, g1);
    __syncthreads();
    if (s + 1 < KC) {
      g1 = fetch(chunk_of(s + 3));
      compute(s + 1);
      put(0, g0);
      __syncthreads();
    }
  }

  tiled_epilogue<ROLE>(a, sh, reinterpret_cast<float*>(lds), y, r0, T0, wave, lane);
  prof_end(a.prof);
}

// The tiled GEMM for int4 weights.  A pipeline step is one scale group (64
// inputs) of one 128-input tile: per output, chain w runs its tiles w,
// w + S, ... and within a tile its groups 0, 1, each group summed from zero
// by MFMA (the hi and lo planes of its two 32-input halves) and added to the
// chain by fmaf with the column's fp32 scale; chains are summed in chain
// order: the arithmetic of the weight-streaming int4 kernel.  Per step the
// workgroup stages the group's activation halves (128 rows x 64 inputs, in
// MFMA operand order), each item's code half-lanes (8 bytes per lane) and
// each item's 16 group scales.
constexpr int kTile4Act = 4 * kTileActVecs;              // hi / lo x two 32-input halves: 2048 vectors
constexpr int kTile4Step = kTile4Act + kTileItems * 32 + kTileItems * 2;   // + codes (as uint4 pairs) + scales: 2320
static_assert(4 * 64 * (2 * 16 + 4) <= 2 * kTileStepVecs * 4, "epilogue slices fit the staging buffers");

struct Tile4Regs {   // one step of this thread's loads
  uint4 a0, a1, a2, a3, a4, a5, a6, a7;
  uint2 c0, c1;
  uint4 s;
};

template <int ROLE>
__global__ __launch_bounds__(256, 1) void k_gemm_tiled_int4(GemmArgs a) {
  __shared__ TileShared sh;
  __shared__ uint4 lds[2 * kTile4Step];
  prof_start(a.prof);
  const int t = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6), lane = t & 63;
  const int wr = wave >> 1, wc = wave & 1, g = lane >> 4;
  const int n_items = a.N >> 4;
  int r0, T0;
  tiled_block(a.M, n_items, r0, T0);
  const int KT = a.K >> 7, S = a.S, cpi = KT / S;   // 128-input tiles; tiles per chain
  const int spc = 2 * cpi;                          // steps per chain (two groups per tile)

  // activation vector v = t + 256 u (u < 8) of the step: plane v / 1024, half
  // (v / 512) % 2, row (v % 512) / 4, 8-input group v % 4
  auto act_off = [&](int u) {   // element offset inside the group's 64 inputs of the row
    const int v = t + 256 * u, rr = (v & 511) >> 2;
    return (size_t)min(r0 + rr, a.M - 1) * a.K + ((v >> 9) & 1) * 32 + (v & 3) * 8;
  };
  auto act_dst = [&](int u) {
    const int v = t + 256 * u, rr = (v & 511) >> 2;
    return (((v >> 9) & 3) * 8 + (rr >> 4)) * 64 + act_slot(v & 3, rr & 15);
  };
  const uint2* W2 = reinterpret_cast<const uint2*>(a.W);
  const uint4* S4 = reinterpret_cast<const uint4*>(a.Wscale);
  const int it0 = t >> 6, it1 = (t + 256) >> 6;                 // code vectors: item, lane t % 64
  const size_t cbase0 = (size_t)min(T0 + it0, n_items - 1) * KT;
  const size_t cbase1 = (size_t)min(T0 + it1, n_items - 1) * KT;
  const size_t sbase = (size_t)min(T0 + ((t & 15) >> 1), n_items - 1) * KT;   // scale vectors: item (t % 16) / 2
  auto fetch = [&](int kt, int gq) {
    Tile4Regs r;
    const size_t k0 = (size_t)kt * 128 + gq * 64;
    r.a0 = *reinterpret_cast<const uint4*>(a.bhi + act_off(0) + k0);
    r.a1 = *reinterpret_cast<const uint4*>(a.bhi + act_off(1) + k0);
    r.a2 = *reinterpret_cast<const uint4*>(a.bhi + act_off(2) + k0);
    r.a3 = *reinterpret_cast<const uint4*>(a.bhi + act_off(3) + k0);
    r.a4 = *reinterpret_cast<const uint4*>(a.blo + act_off(4) + k0);
    r.a5 = *reinterpret_cast<const uint4*>(a.blo + act_off(5) + k0);
    r.a6 = *reinterpret_cast<const uint4*>(a.blo + act_off(6) + k0);
    r.a7 = *reinterpret_cast<const uint4*>(a.blo + act_off(7) + k0);
    r.c0 = W2[((cbase0 + kt) * 64 + (t & 63)) * 2 + gq];
    r.c1 = W2[((cbase1 + kt) * 64 + (t & 63)) * 2 + gq];
    r.s = S4[(sbase + kt) * 4 + gq * 2 + (t & 1)];
    return r;
  };
  auto put = [&](int b, const Tile4Regs& r) {
    uint4* B = lds + b * kTile4Step;
    B[act_dst(0)] = r.a0; B[act_dst(1)] = r.a1; B[act_dst(2)] = r.a2; B[act_dst(3)] = r.a3;
    B[act_dst(4)] = r.a4; B[act_dst(5)] = r.a5; B[act_dst(6)] = r.a6; B[act_dst(7)] = r.a7;
    uint2* C = reinterpret_cast<uint2*>(B + kTile4Act);
    C[t] = r.c0;
    C[t + 256] = r.c1;
    if (t < 16) B[kTile4Act + kTileItems * 32 + t] = r.s;   // LDS store: no load waits on it
  };

  put(0, fetch(0, 0));
  tiled_prologue<ROLE>(a, sh, r0, wave, lane);
  __syncthreads();

  f32x4 acc[4][4], y[4][4];
#pragma unroll
  for (int rt = 0; rt < 4; ++rt)
#pragma unroll
    for (int ct = 0; ct < 4; ++ct) {
      acc[rt][ct] = f32x4{0.f, 0.f, 0.f, 0.f};
      y[rt][ct] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
  const int n_steps = 2 * KT;
  const int aslot = act_slot(lane >> 4, lane & 15);
  int w = 0, c = 0;   // chain and step inside the chain (tile c / 2, group c % 2)
  for (int s = 0; s < n_steps; ++s) {
    const int wn = c + 1 == spc ? w + 1 : w, cn = c + 1 == spc ? 0 : c + 1;
    const Tile4Regs nx = s + 1 < n_steps ? fetch(wn + S * (cn >> 1), cn & 1) : fetch(w + S * (c >> 1), c & 1);
    const uint4* B = lds + (s & 1) * kTile4Step;
    const uint2* C = reinterpret_cast<const uint2*>(B + kTile4Act);
    const uint2* SC = reinterpret_cast<const uint2*>(B + kTile4Act + kTileItems * 32);
#pragma unroll
    for (int rt = 0; rt < 4; ++rt) {
      const int ro = (wr * 4 + rt) * 64 + aslot;
      const BPair b0{B[ro], B[2 * kTileActVecs + ro]};                          // half 0: hi, lo
      const BPair b1{B[kTileActVecs + ro], B[3 * kTileActVecs + ro]};           // half 1: hi, lo
#pragma unroll
      for (int ct = 0; ct < 4; ++ct) {
        const int item = wc * 4 + ct;
        const uint2 q = C[item * 64 + lane];
        const uint2 sc = SC[item * 4 + g];           // the item's 16 group scales: 4 per lane group
        const uint4 A0 = codes8(q.x), A1 = codes8(q.y);
        f32x4 p = f32x4{0.f, 0.f, 0.f, 0.f};
        p = mfma_pair(A0, b0, p);
        p = mfma_pair(A1, b1, p);
        const float s0 = bf2f((uint16_t)(sc.x & 0xffffu)), s1 = bf2f((uint16_t)(sc.x >> 16));
        const float s2 = bf2f((uint16_t)(sc.y & 0xffffu)), s3 = bf2f((uint16_t)(sc.y >> 16));
        acc[rt][ct].x = fmaf(s0, p.x, acc[rt][ct].x);
        acc[rt][ct].y = fmaf(s1, p.y, acc[rt][ct].y);
        acc[rt][ct].z = fmaf(s2, p.z, acc[rt][ct].z);
        acc[rt][ct].w = fmaf(s3, p.w, acc[rt][ct].w);
      }
    }
    if (c + 1 == spc) {   // chain w complete: add it to the running sum in chain order
#pragma unroll
      for (int rt = 0; rt < 4; ++rt)
#pragma unroll
        for (int ct = 0; ct < 4; ++ct) {
          y[rt][ct] = w == 0 ? acc[rt][ct] : y[rt][ct] + acc[rt][ct];
          acc[rt][ct] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
    }
    put((s + 1) & 1, nx);
    __syncthreads();
    w = wn;
    c = cn;
  }
  tiled_epilogue<ROLE>(a, sh, reinterpret_cast<float*>(lds), y, r0, T0, wave, lane);
  prof_end(a.prof);
}

hipError_t launch_gemm_tiled(const GemmArgs& a, int role, hipStream_t st) {
  if (a.M < 1 || a.S < 1 || a.N % 16 || (a.fmt != 0 && a.fmt != 1) || a.K % ((a.fmt ? 128 : 32) * a.S))
    return hipErrorInvalidValue;
  const int n_items = a.N >> 4;
  const int nblk = ((a.M + kTileRows - 1) / kTileRows) * ((n_items + kTileItems - 1) / kTileItems);
  const dim3 grid(nblk), block(256);
  if (a.fmt == 1) {
    switch (role) {
      case kRoleQkv: hipLaunchKernelGGL(k_gemm_tiled_int4<kRoleQkv>, grid, block, 0, st, a); break;
      case kRoleO: hipLaunchKernelGGL(k_gemm_tiled_int4<kRoleO>, grid, block, 0, st, a); break;
      case kRoleGateUp: hipLaunchKernelGGL(k_gemm_tiled_int4<kRoleGateUp>, grid, block, 0, st, a); break;
      case kRoleDown: hipLaunchKernelGGL(k_gemm_tiled_int4<kRoleDown>, grid, block, 0, st, a); break;
      default: return hipErrorInvalidValue;   // the LM head is bf16
    }
    return hipGetLastError();
  }
  switch (role) {
    case kRoleQkv: hipLaunchKernelGGL(k_gemm_tiled<kRoleQkv>, grid, block, 0, st, a); break;
    case kRoleO: hipLaunchKernelGGL(k_gemm_tiled<kRoleO>, grid, block, 0, st, a); break;
    case kRoleGateUp: hipLaunchKernelGGL(k_gemm_tiled<kRoleGateUp>, grid, block, 0, st, a); break;
    case kRoleDown: hipLaunchKernelGGL(k_gemm_tiled<kRoleDown>, grid, block, 0, st, a); break;
    case kRoleLmHead: hipLaunchKernelGGL(k_gemm_tiled<kRoleLmHead>, grid, block, 0, st, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

// ------------------------------------------------------------ attention
// Split plan of one row, a function of its own ctx only: nb = ceil(ctx/64)
// blocks of 64 absolute positions, bps = ceil(nb / 64) blocks per split,
// ns = ceil(nb / bps) splits; split i covers positions
// [64 i bps, min(64 (i+1) bps, ctx)).  Contexts up to 4096 get one block per
// split, longer ones at most 64 splits (a 32K context: 64 splits of 8
// blocks), so a long row still spreads over many waves.  Measured on MI355X
// (8B shape at 32K, K = 4 step): at most 32 / 48 / 64 / 96 / 128 splits
// 5.04 / 4.81 / 4.71 / 4.83 / 4.87 ms; more splits shorten each wave's
// block walk but write and fold more partials.
__host__ __device__ __forceinline__ int attn_bps(int ctx) {
  const int nb = (ctx + kAttnBlock - 1) / kAttnBlock;
  return (nb + kAttnMaxSplits - 1) / kAttnMaxSplits;
}
__host__ __device__ __forceinline__ int attn_ns(int ctx) {
  const int nb = (ctx + kAttnBlock - 1) / kAttnBlock;
  const int bps = attn_bps(ctx);
  return bps == 1 ? nb : (nb + bps - 1) / bps;   // (contexts up to 4096 skip the division)
}

int attn_splits(int ctx) { return attn_ns(ctx); }
int attn_blocks_per_split(int ctx) { return attn_bps(ctx); }
// The split count is not monotone in ctx (ctx 4096: 64 one-block splits;
// ctx 4097: 33 two-block splits), so a launch covers the most splits of any
// of its rows, not those of its longest row.
int attn_splits_max(int kv_len, int M) {
  int n = 1;
  for (int r = 0; r < M; ++r) n = max(n, attn_ns(kv_len + r + 1));
  return n;
}

// Fold of a row's split partials (m_i, l_i, o_i), in split order:
//   (M, L, O) = (m_0, l_0, o_0);  for i >= 1: M' = max(M, m_i),
//   a = 2^(M - M'), b = 2^(m_i - M'), L = L a + l_i b, O = O a + o_i b;
//   output = O / L.
// The same sequence of operations runs in the in-workgroup fold and in the
// combine kernel, so a row's bits do not depend on which one ran.
struct Fold {
  float m, l, o;
  __device__ __forceinline__ void first(float mi, float li, float oi) { m = mi; l = li; o = oi; }
  __device__ __forceinline__ void add(float mi, float li, float oi) {
    const float mn = fmaxf(m, mi);
    const float wa = exp2f(m - mn), wb = exp2f(mi - mn);
    l = l * wa + li * wb;
    o = o * wa + oi * wb;
    m = mn;
  }
};

// A unit of attention work is (KV head h, q tile qt, split sp): 16 q-rows
// (q-row qr = r*G + jj is row r with query head h*G + jj) against the split
// sp of each row's own context ctx_r = kv_len + r + 1.  One wave computes a
// unit, walking the union of its rows' ranges in blocks of 64 absolute
// positions, in increasing order:
//   s_t = (K_t . q) * log2(e)/sqrt(dh)      MFMA chains over d (K rows of
//                                           the paged cache as the A operand)
//   positions outside the row's range -> -inf by select; block max;
//   p_t = 2^(s_t - m_new) (0 when masked);  l = l * 2^(m - m_new) + sum p;
//   o   = o * 2^(m - m_new) + V^T p         MFMA chains over t (V^T rows of
//                                           the page-transposed V cache)
// The KV cache holds fp16; q and p enter the f16 MFMAs as compensated fp16
// pairs (hi + lo).  A block with no valid position for a row leaves its
// (m, l, o) exactly as they were (the rescale factor is 1, p = 0), so extra
// blocks of the union change nothing; every MFMA column is one q-row, so a
// row's result does not depend on the rows beside it.  V elements at
// positions >= kv_len + M (never written) are zeroed before use, so stale or
// poisoned cache never meets p = 0 as 0 * NaN.
//
// Workgroup (x, h): q tile qt = x % n_qt and splits [s_lo, s_lo + spw) with
// s_lo = (x / n_qt) * spw; unit u = split s_lo + u on wave u % wpb.  With
// final_fold (spw covers every split) the partials go to LDS and the
// workgroup folds each row's splits and writes its output planes; otherwise
// they go to the global partial buffer for the combine kernel.
constexpr int kAttnFoldSplits = 3;   // up to this many splits a row is folded in LDS by one workgroup

template <int DH>
struct AttnUnitLds {
  float m[16], l[16];
  float o[16][DH + 4];   // padded rows: the 16 lanes of a wave's stores hit different banks
};

// Physical pages of the 4 logical pages of block b: one 16-byte load of
// consecutive page-table entries (the table is 16-byte aligned); a block
// overhanging max_ctx (its positions are masked) reads clamped entries.
__device__ __forceinline__ int4 attn_block_pages(const AttnArgs& a, int b) {
  int4 q;
  if (4 * b + 4 <= a.n_lpages) {
    q = *reinterpret_cast<const int4*>(a.page_table + 4 * b);
  } else {
    const int last = a.n_lpages - 1;
    q = make_int4(a.page_table[min(4 * b, last)], a.page_table[min(4 * b + 1, last)],
                  a.page_table[min(4 * b + 2, last)], a.page_table[min(4 * b + 3, last)]);
  }
  return q;
}

// MFMA operands of one block of 64 positions for KV head h.
// attn_block_pages through the scalar data cache (b and the table are
// wave-uniform): the entries arrive in SGPRs under lgkmcnt, so waiting for
// them never waits for the K/V loads in flight.  The table is written
// before the launch, never during it.
__device__ __forceinline__ int4 attn_block_pages_s(const AttnArgs& a, int b) {
  typedef const __attribute__((address_space(4))) int* CInt;
  const CInt t = (CInt)a.page_table;
  const int last = a.n_lpages - 1;
  const int e = 4 * b;
  if (e + 4 <= a.n_lpages) return make_int4(t[e], t[e + 1], t[e + 2], t[e + 3]);
  return make_int4(t[min(e, last)], t[min(e + 1, last)], t[min(e + 2, last)], t[min(e + 3, last)]);
}

template <int DH>
struct AttnKV {
  uint4 k[4][DH / 32];          // lane (g, j): K[pos = 64b + 16pt + j][32c + 8g .. +7], one page per pt
  uint2 vlo[DH / 16][2];        // V^T of chunk ks: positions {32ks + 4g .. +3} of d = 16dt + j
  uint2 vhi[DH / 16][2];        //                  positions {32ks + 16 + 4g .. +3}
};

// element offset of (page, w = 0: K / 1: V) of KV head h
__device__ __forceinline__ size_t attn_page_base(const AttnArgs& a, int h, int page, int w, int dh) {
  return ((((size_t)a.layer * a.n_pages + page) * 2 + w) * a.nkv + h) * ((size_t)kPage * dh);
}

template <int DH>
__device__ __forceinline__ void attn_load_k(const AttnArgs& a, int h, int j, int g, int4 pq, AttnKV<DH>& kv) {
  constexpr int DC = DH / 32;
  const int pg[4] = {__builtin_amdgcn_readfirstlane(pq.x), __builtin_amdgcn_readfirstlane(pq.y),
                     __builtin_amdgcn_readfirstlane(pq.z), __builtin_amdgcn_readfirstlane(pq.w)};
#pragma unroll
  for (int pt = 0; pt < 4; ++pt) {
    const uint16_t* kb = a.kv_pool + attn_page_base(a, h, pg[pt], 0, DH) + (size_t)j * DH + g * 8;
#pragma unroll
    for (int c = 0; c < DC; ++c) kv.k[pt][c] = *reinterpret_cast<const uint4*>(kb + c * 32);
  }
}

template <int DH>
__device__ __forceinline__ void attn_load_v(const AttnArgs& a, int h, int j, int g, int4 pq, AttnKV<DH>& kv) {
  constexpr int DT = DH / 16;
  const int pg[4] = {__builtin_amdgcn_readfirstlane(pq.x), __builtin_amdgcn_readfirstlane(pq.y),
                     __builtin_amdgcn_readfirstlane(pq.z), __builtin_amdgcn_readfirstlane(pq.w)};
  auto page_base = [&](int page, int w) { return attn_page_base(a, h, page, w, DH); };
#pragma unroll
  for (int ks = 0; ks < 2; ++ks) {
    const uint16_t* va = a.kv_pool + page_base(pg[2 * ks], 1) + g * 4;
    const uint16_t* vb = a.kv_pool + page_base(pg[2 * ks + 1], 1) + g * 4;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      kv.vlo[dt][ks] = *reinterpret_cast<const uint2*>(va + (size_t)(dt * 16 + j) * kPage);
      kv.vhi[dt][ks] = *reinterpret_cast<const uint2*>(vb + (size_t)(dt * 16 + j) * kPage);
    }
  }
}

template <int DH>
__device__ __forceinline__ void attn_load_kv(const AttnArgs& a, int h, int j, int g, int4 pq, AttnKV<DH>& kv) {
  attn_load_k<DH>(a, h, j, g, pq, kv);
  attn_load_v<DH>(a, h, j, g, pq, kv);
}

// One block b of a unit: scores (attn_block_scores, from K only), mask to
// the lane's row range [lo, hi), online-softmax update of (m, l, o)
// (attn_block_update, from V).  Every attention kernel runs exactly this
// sequence of operations (attn_block_step, or the two halves with loads
// between them).
template <int DH>
__device__ __forceinline__ void attn_block_scores(const AttnKV<DH>& kv, const BPair (&qop)[DH / 32], f32x4 (&sc)[4]) {
  constexpr int DC = DH / 32;
#pragma unroll
  for (int pt = 0; pt < 4; ++pt) {
    f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < DC; ++c) acc = mfma_pair_f16(kv.k[pt][c], qop[c], acc);
    sc[pt] = acc;
  }
}

template <int DH>
__device__ __forceinline__ void attn_block_update(const AttnArgs& a, const AttnKV<DH>& kv, const f32x4 (&sc)[4], int b,
                                                  int g, int lo, int hi, int ctx_max, float& m, float& l,
                                                  f32x4 (&o)[DH / 16]) {
  constexpr int DT = DH / 16;
  // lane (g, j) holds scores of q-row j at positions 64b + 16pt + 4g + v
  float s[16];
  float bmax = -INFINITY;
#pragma unroll
  for (int pt = 0; pt < 4; ++pt)
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int tpos = b * kAttnBlock + pt * 16 + 4 * g + v;
      const float sv = sc[pt][v] * a.scale_log2;
      s[pt * 4 + v] = (tpos >= lo && tpos < hi) ? sv : -INFINITY;
      bmax = fmaxf(bmax, s[pt * 4 + v]);
    }
  bmax = fmaxf(bmax, __shfl_xor(bmax, 16));
  bmax = fmaxf(bmax, __shfl_xor(bmax, 32));
  const float mn = fmaxf(m, bmax);
  const float alpha = (mn == -INFINITY) ? 1.0f : exp2f(m - mn);
  uint16_t pb[16], pl[16];
  float psum = 0.f;
#pragma unroll
  for (int e = 0; e < 16; ++e) {
    const float pv = (s[e] == -INFINITY) ? 0.f : exp2f(s[e] - mn);
    pb[e] = f2h(pv);
    pl[e] = f2h(pv - h2f(pb[e]));
    psum = psum + pv;
  }
  psum = psum + __shfl_xor(psum, 16);
  psum = psum + __shfl_xor(psum, 32);
  l = l * alpha + psum;
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) {
    o[dt].x = o[dt].x * alpha; o[dt].y = o[dt].y * alpha;
    o[dt].z = o[dt].z * alpha; o[dt].w = o[dt].w * alpha;
  }
  // zero V elements at positions >= kv_len + M (never written in this cache)
  auto vmask = [&](uint2 v, int pos0) {
    const int n_ok = ctx_max - pos0;               // valid elements among pos0 .. pos0 + 3
    if (n_ok >= 4) return v;
    if (n_ok <= 0) return make_uint2(0u, 0u);
    const uint32_t m0 = n_ok >= 2 ? 0xffffffffu : 0x0000ffffu;
    const uint32_t m1 = n_ok >= 4 ? 0xffffffffu : (n_ok == 3 ? 0x0000ffffu : 0u);
    return make_uint2(v.x & m0, v.y & m1);
  };
#pragma unroll
  for (int ks = 0; ks < 2; ++ks) {
    const int pa = 2 * ks, pbt = 2 * ks + 1;
    BPair Bp;
    Bp.hi = make_uint4(pack2(pb[pa * 4 + 0], pb[pa * 4 + 1]), pack2(pb[pa * 4 + 2], pb[pa * 4 + 3]),
                       pack2(pb[pbt * 4 + 0], pb[pbt * 4 + 1]), pack2(pb[pbt * 4 + 2], pb[pbt * 4 + 3]));
    Bp.lo = make_uint4(pack2(pl[pa * 4 + 0], pl[pa * 4 + 1]), pack2(pl[pa * 4 + 2], pl[pa * 4 + 3]),
                       pack2(pl[pbt * 4 + 0], pl[pbt * 4 + 1]), pack2(pl[pbt * 4 + 2], pl[pbt * 4 + 3]));
    const int p0 = b * kAttnBlock + pa * 16 + 4 * g, p1 = b * kAttnBlock + pbt * 16 + 4 * g;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      const uint2 v0 = vmask(kv.vlo[dt][ks], p0), v1 = vmask(kv.vhi[dt][ks], p1);
      o[dt] = mfma_pair_f16(make_uint4(v0.x, v0.y, v1.x, v1.y), Bp, o[dt]);
    }
  }
  m = mn;
}

template <int DH>
__device__ __forceinline__ void attn_block_step(const AttnArgs& a, const AttnKV<DH>& kv, const BPair (&qop)[DH / 32],
                                                int b, int g, int lo, int hi, int ctx_max, float& m, float& l,
                                                f32x4 (&o)[DH / 16]) {
  f32x4 sc[4];
  attn_block_scores<DH>(kv, qop, sc);
  attn_block_update<DH>(a, kv, sc, b, g, lo, hi, ctx_max, m, l, o);
}

// Rows of the q tile starting at q-row qbase (of a sequence of M rows) whose
// ranges make up a unit: r0 .. r1.
__device__ __forceinline__ void attn_tile_rows(int qbase, int G, unsigned gm, int M, int& r0, int& r1) {
  r0 = div_m(qbase, G, gm);
  r1 = min(div_m(qbase + 15, G, gm), M - 1);
}

// The view of one q tile: its sequence's pool, page table and length, the
// q-row the tile starts at and the sequence's rows [row0, row0 + m).  A
// single-sequence forward is one sequence of all M rows.
struct AttnView {
  AttnArgs av;   // the arguments with the sequence's pool and page table
  int qbase, row0, m;
};
__device__ __forceinline__ AttnView attn_view(const AttnArgs& a, int qt) {
  AttnView v{a, qt * 16, 0, a.M};
  if (a.seqs != nullptr) {
    const int2 tl = a.tiles[qt];
    const SeqDev& sd = a.seqs[tl.x];
    v.av.kv_pool = sd.kv_pool;
    v.av.page_table = sd.page_table;
    v.av.n_pages = sd.n_pages;
    v.av.n_lpages = sd.n_lpages;
    v.qbase = tl.y;
    v.row0 = sd.row0;
    v.m = sd.m;
  }
  return v;
}
__device__ __forceinline__ int attn_kv_len(const AttnArgs& a, int qt) {
  return a.seqs != nullptr ? a.seqs[a.tiles[qt].x].kv_len : a.params[0];
}
__device__ __forceinline__ int attn_n_tiles(const AttnArgs& a) { return a.n_qt; }

// Union of the tile rows' ranges of split sp, in whole blocks [b_lo, b_hi)
// (wave-uniform; empty when no row of the tile has that split).
__device__ __forceinline__ void attn_split_union(int kv_len, int r0, int r1, int sp, int& b_lo, int& b_hi) {
  b_lo = 0x7fffffff;
  b_hi = 0;
  for (int rr = r0; rr <= r1; ++rr) {
    const int c = kv_len + rr + 1;
    if (sp >= attn_ns(c)) continue;
    const int bps = attn_bps(c);
    b_lo = min(b_lo, sp * bps);
    b_hi = max(b_hi, (min((sp + 1) * bps * kAttnBlock, c) + kAttnBlock - 1) / kAttnBlock);
  }
}

// Instances: FOLD, at most kAttnFoldSplits splits folded in LDS by one
// 8-wave workgroup per (q tile, KV head); otherwise one single-wave
// workgroup per (q tile, split, KV head) writing global partials, with
// EARLY (every row one block per split: the unit's block requested before
// q) or, for several blocks per split, a block walk whose first block is
// requested at the caller's guess bps_g of the blocks per split (PIPE: the
// pipelined walk at one wave per SIMD).  BATCH: the launch has a sequence
// table.
template <int DH, bool FOLD, bool EARLY, bool BATCH, bool PIPE = false>
__global__ __launch_bounds__((FOLD || EARLY || !PIPE) ? 512 : 64) void k_attn_mfma(const float* q, const int* page_table, const int* params,
                                                   const SeqDev* seqs, unsigned pk1, unsigned pk2, unsigned qt_magic,
                                                   unsigned sg_magic, unsigned g_magic, int bps_g, AttnArgs args) {
  constexpr int DC = DH / 32;            // d chunks of the score MFMA
  constexpr int DT = DH / 16;            // d tiles of the P.V MFMA
  __shared__ AttnUnitLds<DH> ul[FOLD ? kAttnFoldSplits : 1];
  // preloaded leading arguments (attn_pack): everything the first loads need
  AttnArgs a = args;
  a.q = q; a.page_table = page_table; a.params = params; a.seqs = seqs;
  a.n_qt = (int)(pk1 & 255u); a.n_sg = (int)((pk1 >> 8) & 255u); a.G = (int)((pk1 >> 16) & 31u);
  a.spw = (int)((pk1 >> 21) & 7u); a.nkv = (int)(pk1 >> 24); a.nq = a.G * a.nkv;
  a.M = (int)(pk2 & 127u); a.n_split = (int)((pk2 >> 7) & 255u); a.n_lpages = (int)(pk2 >> 15);
  a.qt_magic = qt_magic; a.sg_magic = sg_magic; a.g_magic = g_magic;
  const unsigned long long t_start = wall_clock64();
  __builtin_amdgcn_sched_barrier(0);     // (the clock read stays at entry)
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int j = lane & 15, g = lane >> 4;
  const int G = a.G;
  const int n_qt = a.n_qt;
  // Workgroup -> (q tile, split group, KV head).  Workgroups are dealt to the
  // 8 XCDs round-robin in launch order; when the (split group, head) units
  // come in multiples of 8, the q tiles of one unit are placed 8 apart so
  // they run on the same XCD and read the unit's K/V through one L2.
  const int n_sg = a.n_sg;
  const int n_units = n_sg * a.nkv;
  const int lid = blockIdx.x + n_qt * n_sg * blockIdx.y;
  int qt, sg, h;
  if (n_qt > 1 && (n_units & 7) == 0) {
    const int l8 = lid >> 3;
    const int qd = div_m(l8, n_qt, a.qt_magic);   // lid / (8 n_qt)
    qt = l8 - qd * n_qt;
    const int u = qd * 8 + (lid & 7);
    h = div_m(u, n_sg, a.sg_magic);
    sg = u - h * n_sg;
  } else {
    sg = div_m(blockIdx.x, n_qt, a.qt_magic);
    qt = blockIdx.x - sg * n_qt;
    h = blockIdx.y;
  }
  const int s_lo = sg * a.spw;
  const int s_hi = min(s_lo + a.spw, a.n_split);
  // (BATCH: the launch has a sequence table; a single sequence takes no
  // branch on it, so nothing waits on the table fields before the q loads)
  const AttnView V = BATCH ? attn_view(a, qt) : AttnView{a, qt * 16, 0, a.M};
  const AttnArgs& av = V.av;
  const int n_qr = V.m * G;
  // this lane's q-row (independent of kv_len: its q loads go out first);
  // r is the row inside the tile's sequence
  const int qr = V.qbase + j;
  const bool have = qr < n_qr;
  const int rq = div_m(qr, G, a.g_magic);
  const int r = have ? rq : 0;
  const int head = h * G + (have ? qr - rq * G : 0);
  auto block_pages = [&](int b) { return attn_block_pages(av, b); };
  // the first unit's first block is its split index times the blocks per
  // split, which the caller guesses from the first row (every row of a
  // context up to 8192 has one block per split): fetch its pages before the
  // context length is known
  const int b_guess = EARLY ? s_lo + wave : (s_lo + wave) * bps_g;
  int4 pq_guess = (FOLD || EARLY) ? block_pages(b_guess) : attn_block_pages_s(av, b_guess);
  const int kv_len = BATCH ? attn_kv_len(a, qt) : a.params[0];
  // EARLY (the launcher's choice for the split kernel of at most
  // kAttnMaxSplits / 2 splits): every row then has one block per split (a
  // row of two or more blocks per split has more than kAttnMaxSplits / 2
  // splits), so a unit is block b_guess or nothing.
  // Its K/V go out as soon as the page numbers arrive, ahead of q, which the
  // previous kernel has just written and which arrives no sooner: loads
  // complete in issue order, so q issued first would hold the K/V back by
  // its whole latency.  The pages are clamped into the pool for this load
  // (a unit past its rows' context never uses it); a used block lies inside
  // the context, whose pages are valid, so the clamp leaves them unchanged.
  // The split kernel of more splits (rows of two or more blocks per split:
  // one unit per workgroup) requests the guessed first block the same way;
  // its block loop starts from it when the guess holds.
  constexpr bool kHoist = EARLY || !FOLD;
  AttnKV<DH> kv_first;
  if (kHoist && (!EARLY || b_guess < s_hi)) {             // wave-uniform
    const int np = av.n_pages - 1;
    const int4 pc = make_int4(min(max(pq_guess.x, 0), np), min(max(pq_guess.y, 0), np),
                              min(max(pq_guess.z, 0), np), min(max(pq_guess.w, 0), np));
    attn_load_kv<DH>(av, h, j, g, pc, kv_first);
  }
  float4 qraw[DC][2];
  {
    const float4* qp = reinterpret_cast<const float4*>(a.q + ((size_t)(V.row0 + r) * a.nq + head) * DH + g * 8);
#pragma unroll
    for (int c = 0; c < DC; ++c) { qraw[c][0] = qp[c * 8]; qraw[c][1] = qp[c * 8 + 1]; }
  }
  prof_publish_start(a.prof, t_start);
  const int ctx_max = kv_len + V.m;
  const int ctx = kv_len + r + 1;
  BPair qop[DC];
#pragma unroll
  for (int c = 0; c < DC; ++c) {
    const float4 q0 = qraw[c][0], q1 = qraw[c][1];
    const float qv[8] = {q0.x, q0.y, q0.z, q0.w, q1.x, q1.y, q1.z, q1.w};
    qop[c] = have ? split8_f16(qv) : bzero();
  }

  // a wave runs at most one split: spw <= wpb (the fold takes at most
  // kAttnFoldSplits <= 8 splits on 8 waves, the split kernel one on one)
  static_assert(kAttnFoldSplits <= 8, "one split per wave");
  const int sp = s_lo + wave;
  if (sp < s_hi) {     // wave-uniform
    int lo = 0, hi = 0;
    if (have && sp < attn_ns(ctx)) {
      const int bps = attn_bps(ctx);
      lo = sp * bps * kAttnBlock;
      hi = min((sp + 1) * bps * kAttnBlock, ctx);
    }
    // union of the tile's rows' ranges (wave-uniform), in whole blocks
    int b_lo, b_hi;
    {
      int r0, r1;
      attn_tile_rows(V.qbase, G, a.g_magic, V.m, r0, r1);
      attn_split_union(kv_len, r0, r1, sp, b_lo, b_hi);
    }
    f32x4 o[DT];
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) o[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
    float m = -INFINITY, l = 0.f;

    if constexpr (EARLY) {
      if (b_lo < b_hi) attn_block_step<DH>(av, kv_first, qop, b_guess, g, lo, hi, ctx_max, m, l, o);
    } else if constexpr (!FOLD) {
      if (b_lo < b_hi) {                                   // wave-uniform
        // (a missed guess reloads: the rows span a change of blocks per split)
        if (b_lo != b_guess) attn_load_kv<DH>(av, h, j, g, attn_block_pages_s(av, b_lo), kv_first);
        if constexpr (PIPE) {
          // (one wave per SIMD: registers for a second block's K)  Block
          // b + 1's K goes out once block b's scores have read K, and its V
          // once block b's update has read V, so each load runs under the
          // other half's arithmetic.  The loads are unconditional (the last
          // block reloads itself), so every wait counts exactly; the page
          // numbers come through scalar loads, whose waits leave them alone.
          int4 pn = attn_block_pages_s(av, min(b_lo + 1, b_hi - 1));   // pages of block b + 1
          for (int b = b_lo; b < b_hi; ++b) {
            const int4 pn2 = attn_block_pages_s(av, min(b + 2, b_hi - 1));
            f32x4 sc[4];
            attn_block_scores<DH>(kv_first, qop, sc);
            attn_load_k<DH>(av, h, j, g, pn, kv_first);
            attn_block_update<DH>(av, kv_first, sc, b, g, lo, hi, ctx_max, m, l, o);
            attn_load_v<DH>(av, h, j, g, pn, kv_first);
            pn = pn2;
          }
        } else {
          for (int b = b_lo;;) {
            const int4 pq = attn_block_pages_s(av, b + 1 < b_hi ? b + 1 : b);   // in flight during this block
            attn_block_step<DH>(av, kv_first, qop, b, g, lo, hi, ctx_max, m, l, o);
            if (++b >= b_hi) break;
            attn_load_kv<DH>(av, h, j, g, pq, kv_first);
          }
        }
      }
    } else {
      int4 pq = (b_lo == b_guess) ? pq_guess : block_pages(b_lo < b_hi ? b_lo : 0);
      for (int b = b_lo; b < b_hi; ++b) {
        AttnKV<DH> kv;
        attn_load_kv<DH>(av, h, j, g, pq, kv);
        pq = block_pages(b + 1 < b_hi ? b + 1 : b);   // next block's pages, in flight during this block
        attn_block_step<DH>(av, kv, qop, b, g, lo, hi, ctx_max, m, l, o);
      }
    }

    // lane (g, j) holds o of q-row j for d = 16dt + 4g + v
    if constexpr (FOLD) {
      AttnUnitLds<DH>& U = ul[sp];
      if (g == 0) { U.m[j] = m; U.l[j] = l; }
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
        *reinterpret_cast<float4*>(&U.o[j][dt * 16 + 4 * g]) = make_float4(o[dt].x, o[dt].y, o[dt].z, o[dt].w);
    } else if (have && hi > lo) {
      float* part = a.part + (((size_t)(V.row0 + r) * a.nq + head) * a.part_splits + sp) * (DH + 4);
      if (g == 0) { part[0] = m; part[1] = l; }
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
        *reinterpret_cast<float4*>(part + 4 + dt * 16 + 4 * g) = make_float4(o[dt].x, o[dt].y, o[dt].z, o[dt].w);
    }
  }

  if constexpr (FOLD) {
    __syncthreads();
    // every split of this tile is here: thread (jj, d0) folds 4 outputs of q-row jj in split order
    constexpr int TPR = DH / 4;              // threads per q-row
    for (int t = threadIdx.x; t < 16 * TPR; t += blockDim.x) {
      const int jj = t / TPR, d0 = (t % TPR) * 4;
      const int q2 = V.qbase + jj;
      if (q2 >= n_qr) continue;
      const int r2 = div_m(q2, G, a.g_magic), head2 = h * G + (q2 - r2 * G);
      const int ns = attn_ns(kv_len + r2 + 1);
      // the Fold arithmetic, with the weights of a split shared by the 4 outputs
      float fm = ul[0].m[jj], fl = ul[0].l[jj];
      float4 fo = *reinterpret_cast<const float4*>(&ul[0].o[jj][d0]);
      for (int sp = 1; sp < ns; ++sp) {
        const float mi = ul[sp].m[jj], li = ul[sp].l[jj];
        const float4 oi = *reinterpret_cast<const float4*>(&ul[sp].o[jj][d0]);
        const float mn = fmaxf(fm, mi);
        const float wa = exp2f(fm - mn), wb = exp2f(mi - mn);
        fl = fl * wa + li * wb;
        fo.x = fo.x * wa + oi.x * wb; fo.y = fo.y * wa + oi.y * wb;
        fo.z = fo.z * wa + oi.z * wb; fo.w = fo.w * wa + oi.w * wb;
        fm = mn;
      }
      const float ov[4] = {fo.x, fo.y, fo.z, fo.w};
      uint16_t hb[4], lb[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) split1(ov[e] / fl, hb[e], lb[e]);
      const size_t oi = ((size_t)(V.row0 + r2) * a.nq + head2) * DH + d0;
      *reinterpret_cast<uint2*>(a.ohi + oi) = make_uint2(pack2(hb[0], hb[1]), pack2(hb[2], hb[3]));
      *reinterpret_cast<uint2*>(a.olo + oi) = make_uint2(pack2(lb[0], lb[1]), pack2(lb[2], lb[3]));
    }
    prof_end(a.prof);
  }
}

// Attention for forwards of many rows (prefill chunks): one wave per
// (q tile, KV head) runs every split of its rows in split order.  Each
// split's (m, l, o) comes from the same block steps as in k_attn_mfma and is
// folded into the row's running result as soon as it is done, with the fold
// arithmetic of the split kernels (split 0 first; then M' = max(M, m_i),
// L = L 2^(M - M') + l_i 2^(m_i - M'), O likewise), so a row's bits equal
// those the split kernels give it, with no partial buffer and no combine
// pass.  Parallelism comes from the many q tiles instead of the splits.
template <int DH>
__global__ __launch_bounds__(256) void k_attn_rows(AttnArgs a) {
  constexpr int DC = DH / 32, DT = DH / 16;
  prof_start(a.prof);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int j = lane & 15, g = lane >> 4;
  const int G = a.G;
  const int n_qt = attn_n_tiles(a);
  // Workgroups are dealt to the 8 XCDs round-robin in launch order; with the
  // KV head varying fastest, each XCD runs one head's q tiles (with 8 KV
  // heads), which walk that head's K/V in step and share it through the
  // XCD's L2 instead of each reading it from the memory-side cache.
  const int h = blockIdx.x % a.nkv;
  const int qt = (blockIdx.x / a.nkv) * 4 + wave;
  if (qt < n_qt) {   // wave-uniform
    const AttnView V = attn_view(a, qt);
    const AttnArgs& av = V.av;
    const int n_qr = V.m * G;
    const int qr = V.qbase + j;
    const bool have = qr < n_qr;
    const int rq = div_m(qr, G, a.g_magic);
    const int r = have ? rq : 0;
    const int head = h * G + (have ? qr - rq * G : 0);
    BPair qop[DC];
    {
      const float4* qp = reinterpret_cast<const float4*>(a.q + ((size_t)(V.row0 + r) * a.nq + head) * DH + g * 8);
#pragma unroll
      for (int c = 0; c < DC; ++c) {
        const float4 q0 = qp[c * 8], q1 = qp[c * 8 + 1];
        const float qv[8] = {q0.x, q0.y, q0.z, q0.w, q1.x, q1.y, q1.z, q1.w};
        qop[c] = have ? split8_f16(qv) : bzero();
      }
    }
    const int kv_len = attn_kv_len(a, qt);
    const int ctx_max = kv_len + V.m;
    const int ctx = kv_len + r + 1;
    const int ns_row = attn_ns(ctx);
    int r0, r1;
    attn_tile_rows(V.qbase, G, a.g_magic, V.m, r0, r1);
    int ns_max = 1;
    for (int rr = r0; rr <= r1; ++rr) ns_max = max(ns_max, attn_ns(kv_len + rr + 1));

    float fm = 0.f, fl = 0.f;
    f32x4 fo[DT];
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) fo[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int sp = 0; sp < ns_max; ++sp) {
      int lo = 0, hi = 0;
      if (have && sp < ns_row) {
        const int bps = attn_bps(ctx);
        lo = sp * bps * kAttnBlock;
        hi = min((sp + 1) * bps * kAttnBlock, ctx);
      }
      int b_lo, b_hi;
      attn_split_union(kv_len, r0, r1, sp, b_lo, b_hi);
      f32x4 o[DT];
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) o[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
      float m = -INFINITY, l = 0.f;
      int4 pq = attn_block_pages(av, b_lo < b_hi ? b_lo : 0);
      for (int b = b_lo; b < b_hi; ++b) {
        AttnKV<DH> kv;
        attn_load_kv<DH>(av, h, j, g, pq, kv);
        pq = attn_block_pages(av, b + 1 < b_hi ? b + 1 : b);
        attn_block_step<DH>(av, kv, qop, b, g, lo, hi, ctx_max, m, l, o);
      }
      if (sp == 0) {
        fm = m;
        fl = l;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) fo[dt] = o[dt];
      } else if (sp < ns_row) {
        const float mn = fmaxf(fm, m);
        const float wa = exp2f(fm - mn), wb = exp2f(m - mn);
        fl = fl * wa + l * wb;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
          fo[dt].x = fo[dt].x * wa + o[dt].x * wb; fo[dt].y = fo[dt].y * wa + o[dt].y * wb;
          fo[dt].z = fo[dt].z * wa + o[dt].z * wb; fo[dt].w = fo[dt].w * wa + o[dt].w * wb;
        }
        fm = mn;
      }
    }
    if (have) {
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        const float ov[4] = {fo[dt].x, fo[dt].y, fo[dt].z, fo[dt].w};
        uint16_t hb[4], lb[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) split1(ov[e] / fl, hb[e], lb[e]);
        const size_t oi = ((size_t)(V.row0 + r) * a.nq + head) * DH + dt * 16 + 4 * g;
        *reinterpret_cast<uint2*>(a.ohi + oi) = make_uint2(pack2(hb[0], hb[1]), pack2(hb[2], hb[3]));
        *reinterpret_cast<uint2*>(a.olo + oi) = make_uint2(pack2(lb[0], lb[1]), pack2(lb[2], lb[3]));
      }
    }
  }
  prof_end(a.prof);
}

// Two q tiles per wave (single-sequence forwards, whose
// adjacent tiles share one page table): each block's K/V operands are loaded
// once and used for every tile of the wave, halving the load bytes per
// q-row; the block range of a split is the union over the wave's tiles, and
// blocks outside a row's own range are exact no-ops for it, so every row
// keeps the arithmetic of the split kernels.
template <int DH>
__global__ __launch_bounds__(256) void k_attn_rows2(AttnArgs a) {
  constexpr int TPW = 2;
  // the running fold of each tile's rows, per lane: [wave][tile][dt][lane]
  __shared__ f32x4 fo_lds[4 * TPW * (DH / 16) * 64];
  constexpr int DC = DH / 32, DT = DH / 16;
  prof_start(a.prof);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int j = lane & 15, g = lane >> 4;
  const int G = a.G;
  const int n_qt = attn_n_tiles(a);
  // Workgroups are dealt to the 8 XCDs round-robin in launch order; with the
  // KV head varying fastest, each XCD runs one head's q tiles (with 8 KV
  // heads), which walk that head's K/V in step and share it through the
  // XCD's L2 instead of each reading it from the memory-side cache.
  const int h = blockIdx.x % a.nkv;
  const int qt0 = ((blockIdx.x / a.nkv) * 4 + wave) * TPW;
  if (qt0 < n_qt) {   // wave-uniform
    const AttnView V = attn_view(a, qt0);
    const AttnArgs& av = V.av;
    const int n_qr = V.m * G;
    const int kv_len = attn_kv_len(a, qt0);
    const int ctx_max = kv_len + V.m;
    bool have[TPW];
    int r[TPW], head[TPW], ctx[TPW], ns_row[TPW];
    BPair qop[TPW][DC];
    int rlo = V.m, rhi = 0;   // rows of the wave's tiles
#pragma unroll
    for (int u = 0; u < TPW; ++u) {
      const int qbase = V.qbase + 16 * u;
      const int qr = qbase + j;
      have[u] = qt0 + u < n_qt && qr < n_qr;
      const int rq = div_m(qr, G, a.g_magic);
      r[u] = have[u] ? rq : 0;
      head[u] = h * G + (have[u] ? qr - rq * G : 0);
      const float4* qp = reinterpret_cast<const float4*>(a.q + ((size_t)(V.row0 + r[u]) * a.nq + head[u]) * DH + g * 8);
#pragma unroll
      for (int c = 0; c < DC; ++c) {
        const float4 q0 = qp[c * 8], q1 = qp[c * 8 + 1];
        const float qv[8] = {q0.x, q0.y, q0.z, q0.w, q1.x, q1.y, q1.z, q1.w};
        qop[u][c] = have[u] ? split8_f16(qv) : bzero();
      }
      ctx[u] = kv_len + r[u] + 1;
      ns_row[u] = attn_ns(ctx[u]);
      if (qt0 + u < n_qt && qbase < n_qr) {
        int r0, r1;
        attn_tile_rows(qbase, G, a.g_magic, V.m, r0, r1);
        rlo = min(rlo, r0);
        rhi = max(rhi, r1);
      }
    }
    int ns_max = 1;
    for (int rr = rlo; rr <= rhi; ++rr) ns_max = max(ns_max, attn_ns(kv_len + rr + 1));

    float fm[TPW], fl[TPW];
    auto fo = [&](int u, int dt) -> f32x4& { return fo_lds[((wave * TPW + u) * DT + dt) * 64 + lane]; };
#pragma unroll
    for (int u = 0; u < TPW; ++u) {
      fm[u] = 0.f;
      fl[u] = 0.f;
    }
    // One block stream across the splits: block b + 1's K goes out once both
    // tiles' scores of block b have read K, and its V once both updates have
    // read V, so each load runs under the other half's arithmetic (one wave
    // per SIMD: nothing else hides the latency); the block after a split's
    // last is the next split's first (every split of the union has a block:
    // sp < ns_max is a split of one of the rows), the very last reloads
    // itself.  The loads are unconditional and the page numbers come through
    // scalar loads, so every wait counts exactly.  Each tile runs
    // attn_block_step's operations in its order.
    int b_lo, b_hi;
    attn_split_union(kv_len, rlo, rhi, 0, b_lo, b_hi);
    AttnKV<DH> kv;
    attn_load_kv<DH>(av, h, j, g, attn_block_pages_s(av, b_lo), kv);
    for (int sp = 0; sp < ns_max; ++sp) {
      int lo[TPW], hi[TPW];
#pragma unroll
      for (int u = 0; u < TPW; ++u) {
        lo[u] = 0;
        hi[u] = 0;
        if (have[u] && sp < ns_row[u]) {
          const int bps = attn_bps(ctx[u]);
          lo[u] = sp * bps * kAttnBlock;
          hi[u] = min((sp + 1) * bps * kAttnBlock, ctx[u]);
        }
      }
      int nb_lo = b_hi - 1, nb_hi = b_hi;               // (past the last split: reload its last block)
      if (sp + 1 < ns_max) attn_split_union(kv_len, rlo, rhi, sp + 1, nb_lo, nb_hi);
      f32x4 o[TPW][DT];
      float m[TPW], l[TPW];
#pragma unroll
      for (int u = 0; u < TPW; ++u) {
        m[u] = -INFINITY;
        l[u] = 0.f;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) o[u][dt] = f32x4{0.f, 0.f, 0.f, 0.f};
      }
      for (int b = b_lo; b < b_hi; ++b) {
        const int4 pn = attn_block_pages_s(av, b + 1 < b_hi ? b + 1 : nb_lo);   // the next block's pages
        f32x4 sc[TPW][4];
#pragma unroll
        for (int u = 0; u < TPW; ++u) attn_block_scores<DH>(kv, qop[u], sc[u]);
        attn_load_k<DH>(av, h, j, g, pn, kv);
#pragma unroll
        for (int u = 0; u < TPW; ++u)
          attn_block_update<DH>(av, kv, sc[u], b, g, lo[u], hi[u], ctx_max, m[u], l[u], o[u]);
        attn_load_v<DH>(av, h, j, g, pn, kv);
      }
      b_lo = nb_lo;
      b_hi = nb_hi;
#pragma unroll
      for (int u = 0; u < TPW; ++u) {
        if (sp == 0) {
          fm[u] = m[u];
          fl[u] = l[u];
#pragma unroll
          for (int dt = 0; dt < DT; ++dt) fo(u, dt) = o[u][dt];
        } else if (sp < ns_row[u]) {
          const float mn = fmaxf(fm[u], m[u]);
          const float wa = exp2f(fm[u] - mn), wb = exp2f(m[u] - mn);
          fl[u] = fl[u] * wa + l[u] * wb;
#pragma unroll
          for (int dt = 0; dt < DT; ++dt) {
            f32x4 f = fo(u, dt);
            f.x = f.x * wa + o[u][dt].x * wb; f.y = f.y * wa + o[u][dt].y * wb;
            f.z = f.z * wa + o[u][dt].z * wb; f.w = f.w * wa + o[u][dt].w * wb;
            fo(u, dt) = f;
          }
          fm[u] = mn;
        }
      }
    }
#pragma unroll
    for (int u = 0; u < TPW; ++u) {
      if (have[u]) {
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
          const f32x4 f = fo(u, dt);
          const float ov[4] = {f.x, f.y, f.z, f.w};
          uint16_t hb[4], lb[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) split1(ov[e] / fl[u], hb[e], lb[e]);
          const size_t oi = ((size_t)(V.row0 + r[u]) * a.nq + head[u]) * DH + dt * 16 + 4 * g;
          *reinterpret_cast<uint2*>(a.ohi + oi) = make_uint2(pack2(hb[0], hb[1]), pack2(hb[2], hb[3]));
          *reinterpret_cast<uint2*>(a.olo + oi) = make_uint2(pack2(lb[0], lb[1]), pack2(lb[2], lb[3]));
        }
      }
    }
  }
  prof_end(a.prof);
}

// Fold of the global partials of row r, query head j (record [m, l, -, -, o[dh]]):
// the row's records are staged in LDS with coalesced 16-byte loads (a long
// context has up to kAttnMaxSplits of them), then thread d folds output d in split order.
// Launched with 256 threads.  The loads cover the launch's most splits
// (n_split, at most part_splits) and go out with the context length's, not
// after it; records past the row's own split count are dropped.
template <int DH>
__global__ __launch_bounds__(256) void k_attn_combine(float* part, const int* params, const SeqDev* seqs,
                                                      const int* rowseq, int nq, int part_splits, int n_split,
                                                      AttnArgs args) {
  AttnArgs a = args;                     // leading arguments preloaded (as in k_attn_mfma)
  a.part = part; a.params = params; a.seqs = seqs; a.rowseq = rowseq; a.nq = nq; a.part_splits = part_splits;
  __shared__ float4 rec[kAttnMaxSplits * (DH + 4) / 4];
  const int j = blockIdx.x, r = blockIdx.y;
  int ctx = a.params[0] + r + 1;
  if (a.seqs != nullptr) {
    const SeqDev& sd = a.seqs[a.rowseq[r]];
    ctx = sd.kv_len + r - sd.row0 + 1;
  }
  const float4* base = reinterpret_cast<const float4*>(a.part + ((size_t)r * a.nq + j) * a.part_splits * (DH + 4));
  const int n4_max = n_split * ((DH + 4) / 4);
  // every record of the row in one round of loads (at most 9 per thread)
  constexpr int U = (kAttnMaxSplits * (DH + 4) / 4 + 255) / 256;
  float4 v[U];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int i = threadIdx.x + u * 256;
    v[u] = base[i < n4_max ? i : 0];
  }
  const int ns = attn_ns(ctx);
  const int n4 = ns * ((DH + 4) / 4);
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int i = threadIdx.x + u * 256;
    if (i < n4) rec[i] = v[u];
  }
  __syncthreads();
  const float* p = reinterpret_cast<const float*>(rec);
  // The fold's running maximum is a prefix maximum of the m_i (fmaxf is
  // exact), so every step's weights 2^(M_{i-1} - M_i) and 2^(m_i - M_i) can
  // be formed at once from a scan; only the (l, o) updates stay sequential,
  // two dependent operations per split instead of the whole step.  The
  // values are those of Fold::add, operation for operation.
  __shared__ float wab[2][kAttnMaxSplits];
  if (threadIdx.x < 64) {
    const int i0 = threadIdx.x, i1 = threadIdx.x + 64;
    const float m0 = i0 < ns ? p[i0 * (DH + 4)] : -INFINITY;
    const float m1 = i1 < ns ? p[i1 * (DH + 4)] : -INFINITY;
    float s0 = m0, s1 = m1;                      // inclusive prefix maxima of splits i0, i1
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const float t0 = __shfl_up(s0, o), t1 = __shfl_up(s1, o);
      if (i0 >= o) { s0 = fmaxf(s0, t0); s1 = fmaxf(s1, t1); }
    }
    const float all0 = __shfl(s0, 63);           // M_63
    s1 = fmaxf(s1, all0);
    float q0 = __shfl_up(s0, 1), q1 = __shfl_up(s1, 1);   // M_{i-1}
    if (i0 == 0) q1 = all0;
    if (i0 >= 1 && i0 < ns) { wab[0][i0] = exp2f(q0 - s0); wab[1][i0] = exp2f(m0 - s0); }
    if (i1 < ns) { wab[0][i1] = exp2f(q1 - s1); wab[1][i1] = exp2f(m1 - s1); }
  }
  __syncthreads();
  const int d = threadIdx.x;
  if (d < DH) {
    float l = p[1], o = p[4 + d];
#pragma unroll 8
    for (int i = 1; i < ns; ++i) {
      const float wa = wab[0][i], wb = wab[1][i];
      l = l * wa + p[i * (DH + 4) + 1] * wb;
      o = o * wa + p[i * (DH + 4) + 4 + d] * wb;
    }
    const size_t oi = (size_t)r * a.nq * DH + (size_t)j * DH + d;
    split1(o / l, a.ohi[oi], a.olo[oi]);
  }
  prof_end(a.prof);
}

// The packed leading arguments of k_attn_mfma: pk1 = n_qt | n_sg << 8 |
// G << 16 | spw << 21 | nkv << 24, pk2 = M | n_split << 7 | n_lpages << 15;
// false if a field does not fit its bits.
static bool attn_pack(const AttnArgs& a, unsigned& pk1, unsigned& pk2) {
  if (a.n_qt < 1 || a.n_qt > 255 || a.n_sg < 1 || a.n_sg > 255 || a.G < 1 || a.G > 31 || a.spw < 1 ||
      a.spw > 7 || a.nkv < 1 || a.nkv > 255 || a.nq != a.G * a.nkv || a.M < 1 || a.M > 127 || a.n_split < 1 ||
      a.n_split > 255 || a.n_lpages < 1 || a.n_lpages > 0x1ffff)
    return false;
  pk1 = (unsigned)a.n_qt | ((unsigned)a.n_sg << 8) | ((unsigned)a.G << 16) | ((unsigned)a.spw << 21) |
        ((unsigned)a.nkv << 24);
  pk2 = (unsigned)a.M | ((unsigned)a.n_split << 7) | ((unsigned)a.n_lpages << 15);
  return true;
}

// The split kernel (LDS fold, early-K/V split or plain split; single sequence
// or sequence table) and, without the fold, the combine pass.
template <int DH>
static bool launch_attn_split(const AttnArgs& a, dim3 grid, dim3 block, bool early, bool pipe, unsigned pk1,
                              unsigned pk2, hipStream_t st) {
  const bool batch = a.seqs != nullptr;
#define SV_ATTN_LEAD a.q, a.page_table, a.params, a.seqs, pk1, pk2, a.qt_magic, a.sg_magic, a.g_magic, \
                     a.bps_guess > 1 ? a.bps_guess : 1, a
  if (a.final_fold) {
    if (batch) hipLaunchKernelGGL((k_attn_mfma<DH, true, false, true>), grid, block, 0, st, SV_ATTN_LEAD);
    else hipLaunchKernelGGL((k_attn_mfma<DH, true, false, false>), grid, block, 0, st, SV_ATTN_LEAD);
  } else if (early) {
    if (batch) hipLaunchKernelGGL((k_attn_mfma<DH, false, true, true>), grid, block, 0, st, SV_ATTN_LEAD);
    else hipLaunchKernelGGL((k_attn_mfma<DH, false, true, false>), grid, block, 0, st, SV_ATTN_LEAD);
  } else if (pipe) {
    if (batch) hipLaunchKernelGGL((k_attn_mfma<DH, false, false, true, true>), grid, block, 0, st, SV_ATTN_LEAD);
    else hipLaunchKernelGGL((k_attn_mfma<DH, false, false, false, true>), grid, block, 0, st, SV_ATTN_LEAD);
  } else {
    if (batch) hipLaunchKernelGGL((k_attn_mfma<DH, false, false, true>), grid, block, 0, st, SV_ATTN_LEAD);
    else hipLaunchKernelGGL((k_attn_mfma<DH, false, false, false>), grid, block, 0, st, SV_ATTN_LEAD);
  }
#undef SV_ATTN_LEAD
  if (!a.final_fold)
    hipLaunchKernelGGL(k_attn_combine<DH>, dim3(a.nq, a.M), dim3(256), 0, st, a.part, a.params, a.seqs, a.rowseq,
                       a.nq, a.part_splits, a.n_split, a);
  return true;
}

hipError_t launch_attention(const AttnArgs& a_in, hipStream_t st) {
  AttnArgs a = a_in;
  const int G = a.nq / a.nkv;
  if ((a.seqs == nullptr && a.M * G > kAttnQRows) || a.n_split < 1 || a.n_split > kAttnMaxSplits || a.n_lpages < 1 ||
      (a.seqs != nullptr && (a.n_tiles < 1 || a.rowseq == nullptr)) ||
      (a.n_split > kAttnFoldSplits && a.n_split > a.part_splits))
    return hipErrorInvalidValue;
  const int n_qt = a.seqs != nullptr ? a.n_tiles : (a.M * G + 15) / 16;
  // up to kAttnFoldSplits splits: one workgroup of 8 waves per (q tile, KV
  // head) runs them and folds them in LDS; more: one single-wave workgroup
  // per (q tile, split, KV head), then the combine pass.  Measured on MI355X
  // (8 KV heads, 1-5 rows): the LDS fold is 0.6 us faster at 2 splits, even
  // at 3, and falls behind from 5 (15.6 against 10.3 us at 10 splits), as
  // its few workgroups leave most of the chip idle; single-wave split
  // workgroups match or beat 2- and 4-wave ones at every context up to 32K.
  a.final_fold = a.n_split <= kAttnFoldSplits ? 1 : 0;
  a.spw = a.final_fold ? a.n_split : 1;
  a.wpb = a.final_fold ? 8 : 1;
  a.G = G;
  a.n_qt = n_qt;
  a.n_sg = (a.n_split + a.spw - 1) / a.spw;
  a.g_magic = div_magic(G);
  a.qt_magic = div_magic(n_qt);
  a.sg_magic = div_magic(a.n_sg);
  const int n_wg = n_qt * a.n_sg;
  const dim3 grid(n_wg, a.nkv), block(64 * a.wpb);
  // split kernel of at most kAttnMaxSplits / 2 splits: one block per split
  // for every row, so the unit's K/V can go out ahead of q.  Measured on
  // MI355X: 0.6B shape at 512-640 positions (10 splits) attention 250.3 ->
  // 246.7 us per K = 4 step; the LDS-fold kernel (2-3 splits) was slower
  // with it (8B 271.5 -> 275.7, Gemma 239.7 -> 246.1 us), so it keeps its
  // loads in the old order.
  const bool early = a.n_split <= kAttnMaxSplits / 2;
  // the split kernel of several blocks per split, when its waves fit one per
  // SIMD: the instance that keeps a second block's K in flight (more
  // registers, one wave per SIMD).  Measured on MI355X, 8B shape at 32K (64
  // splits of 8 blocks, 2 q tiles = 1024 waves): K = 4 step 4.72 -> 4.65 ms;
  // at K = 16 / 32 (5 / 9 q tiles) it lost 0.8 / 2.5 % to the two-waves-per-
  // SIMD kernel, so those keep it.  Both run the same operations on every row.
  const bool pipe = !a.final_fold && !early && a.n_simd > 0 && n_wg * a.nkv <= a.n_simd;
  unsigned pk1, pk2;
  if (!attn_pack(a, pk1, pk2)) return hipErrorInvalidValue;
  if (a.dh == 128) {
    if (!launch_attn_split<128>(a, grid, block, early, pipe, pk1, pk2, st)) return hipErrorInvalidValue;
  } else if (a.dh == 64) {
    if (!launch_attn_split<64>(a, grid, block, early, pipe, pk1, pk2, st)) return hipErrorInvalidValue;
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_attention_rows(const AttnArgs& a_in, hipStream_t st) {
  if (a_in.M < 1 || a_in.n_lpages < 1 || a_in.nkv < 1 || a_in.nq % a_in.nkv) return hipErrorInvalidValue;
  AttnArgs a = a_in;
  const int n_qt = a.seqs != nullptr ? a.n_tiles : (a.M * (a.nq / a.nkv) + 15) / 16;
  a.G = a.nq / a.nkv;
  a.n_qt = n_qt;
  a.n_sg = 1;
  a.g_magic = div_magic(a.G);
  a.qt_magic = div_magic(n_qt);
  a.sg_magic = 0u;
  // two q tiles per wave where the tiles share one sequence
  const int tpw = a.seqs == nullptr ? 2 : 1;
  const dim3 grid(((n_qt + 4 * tpw - 1) / (4 * tpw)) * a.nkv), block(256);
  if (a.dh == 128) {
    if (tpw == 2) hipLaunchKernelGGL(k_attn_rows2<128>, grid, block, 0, st, a);
    else hipLaunchKernelGGL(k_attn_rows<128>, grid, block, 0, st, a);
  } else if (a.dh == 64) {
    if (tpw == 2) hipLaunchKernelGGL(k_attn_rows2<64>, grid, block, 0, st, a);
    else hipLaunchKernelGGL(k_attn_rows<64>, grid, block, 0, st, a);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

// ------------------------------------------------------------ embedding gather
// x[r] = E[id_r] widened to fp32, the per-16-column sums of squares the
// first RMSNorm reads (16-lane butterfly, like the residual epilogue), and
// the planes of x * g_attn of layer 0.
// One thread per (row, feature): x = E[id] (exact bf16 -> fp32), the row's
// per-16-column sums of squares (16 consecutive lanes), planes of x * g0.
// Block (r, 0) also clears row r's argmax key for the LM head.  The forward's
// parameters [kv_len, M, ids] come straight from the caller's pinned host
// buffer (hparams, read over the bus); block (r, 0) stores id r, and block
// (0, 0) kv_len and M, into the device copy (params) the later kernels read.
__global__ __launch_bounds__(256) void k_embed(const int* __restrict__ hparams, int* __restrict__ params,
                                               const uint16_t* __restrict__ E, int d, float* __restrict__ x,
                                               float* __restrict__ ss, const uint16_t* __restrict__ g0,
                                               uint16_t* __restrict__ uhi, uint16_t* __restrict__ ulo,
                                               unsigned long long* __restrict__ best) {
  const int r = blockIdx.y;
  const int k = blockIdx.x * 256 + threadIdx.x;
  const int id = hparams[2 + r];
  if (blockIdx.x == 0 && threadIdx.x == 0) {
    best[r] = 0ull;
    params[2 + r] = id;
    if (r == 0) { params[0] = hparams[0]; params[1] = hparams[1]; }
  }
  if (k >= d) return;   // d is a multiple of 16, so whole 16-lane groups exit together
  // the embedding is packed like a bf16 weight matrix: 16-row tiles of 32-input chunks
  const size_t off = ((size_t)(id >> 4) * (d >> 5) + (k >> 5)) * 512 + (size_t)(((k & 31) >> 3) * 16 + (id & 15)) * 8 + (k & 7);
  const float v = bf2f(E[off]);
  x[(size_t)r * d + k] = v;
  float sq = v * v;
#pragma unroll
  for (int o = 8; o >= 1; o >>= 1) sq += __shfl_xor(sq, o);
  if ((k & 15) == 0) ss[(size_t)r * (d >> 4) + (k >> 4)] = sq;
  split1(v * bf2f(g0[k]), uhi[(size_t)r * d + k], ulo[(size_t)r * d + k]);
}

hipError_t launch_embed(const int* hparams, int* params, int M, const void* embed, int vocab, int d, float* x,
                        float* ss, const uint16_t* g0, uint16_t* uhi, uint16_t* ulo, unsigned long long* best,
                        hipStream_t st) {
  (void)vocab;
  hipLaunchKernelGGL(k_embed, dim3((d + 255) / 256, M), dim3(256), 0, st, hparams, params, (const uint16_t*)embed, d,
                     x, ss, g0, uhi, ulo, best);
  return hipGetLastError();
}

// ------------------------------------------------------------ argmax + acceptance
// Row argmax over the LM head's per-16-column bests (max of packed keys,
// order-free), then the greedy acceptance: n = number of leading drafts equal
// to the argmax of the row before them; next = argmax of row n.
// result: [0] n, [1] next, [2 + r] argmax of row r.
// Row argmax a_r from the LM head's row keys; verify rows accept the longest
// prefix of drafts d_i = a_i (row i+1 holds d_i); result = [n, next, a_0..].
__global__ __launch_bounds__(64) void k_accept(const int* params, int M, int verify, const unsigned long long* best,
                                               int* result) {
  const int lane = threadIdx.x;
  auto id_of = [&](int r) { return (int)(0xffffffffu - (uint32_t)(best[r] & 0xffffffffu)); };
  const int a_r = lane < M ? id_of(lane) : 0;
  if (lane < M) result[2 + lane] = a_r;
  for (int r = 64 + lane; r < M; r += 64) result[2 + r] = id_of(r);   // rows past 64 (prefill forwards)
  int n;
  if (verify) {   // M <= 64
    const int k = M - 1;
    const bool miss = lane < k && params[2 + lane + 1] != a_r;
    const unsigned long long mask = __ballot(miss);
    n = mask ? (__ffsll((long long)mask) - 1) : k;
  } else {
    n = M - 1;
  }
  const int next = n < 64 ? __shfl(a_r, n) : id_of(n);
  if (lane == 0) { result[0] = n; result[1] = next; }
}

hipError_t launch_accept(const int* params, int M, int verify, const unsigned long long* best, int* result,
                         hipStream_t st) {
  if (M < 1 || (verify && M > 64)) return hipErrorInvalidValue;
  hipLaunchKernelGGL(k_accept, dim3(1), dim3(64), 0, st, params, M, verify, best, result);
  return hipGetLastError();
}

// Batched verify: every row's argmax, then per sequence (one lane each) the
// same acceptance rule over its own rows.
__global__ __launch_bounds__(64) void k_accept_batch(const int* params, int M, const SeqDev* seqs, int n_seq,
                                                     const unsigned long long* best, int* result) {
  const int lane = threadIdx.x;
  auto id_of = [&](int r) { return (int)(0xffffffffu - (uint32_t)(best[r] & 0xffffffffu)); };
  for (int r = lane; r < M; r += 64) result[2 + r] = id_of(r);
  if (lane < n_seq) {
    const SeqDev& sd = seqs[lane];
    int n = 0;
    while (n < sd.m - 1 && params[2 + sd.row0 + n + 1] == id_of(sd.row0 + n)) ++n;
    result[2 + M + 2 * lane] = n;
    result[2 + M + 2 * lane + 1] = id_of(sd.row0 + n);
  }
}

hipError_t launch_accept_batch(const int* params, int M, const SeqDev* seqs, int n_seq,
                               const unsigned long long* best, int* result, hipStream_t st) {
  if (M < 1 || n_seq < 1 || n_seq > 64) return hipErrorInvalidValue;
  hipLaunchKernelGGL(k_accept_batch, dim3(1), dim3(64), 0, st, params, M, seqs, n_seq, best, result);
  return hipGetLastError();
}

// ------------------------------------------------------------ audit mode
// Top-k of one fp32 logits row by the argmax key order (larger logit first,
// the lower id among equal logits): every block takes k rounds of a block
// max over its slice (the winner is removed each round), then one block
// does the same over the blocks' candidates.  k <= kTopkMax.
__device__ __forceinline__ unsigned long long block_max_key(unsigned long long v, unsigned long long* lds16) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = umax64(v, __shfl_xor(v, o));
  const int w = threadIdx.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) lds16[w] = v;
  __syncthreads();
  unsigned long long m = 0ull;
  for (int i = 0; i < (int)(blockDim.x >> 6); ++i) m = umax64(m, lds16[i]);
  return m;
}

__global__ __launch_bounds__(256) void k_topk_blocks(const float* __restrict__ row, int V, int k,
                                                     unsigned long long* __restrict__ cand) {
  __shared__ unsigned long long keys[kTopkSlice];
  __shared__ unsigned long long red[16];
  const int per = (V + gridDim.x - 1) / gridDim.x;
  const int lo = blockIdx.x * per, n = min(per, V - lo);
  for (int i = threadIdx.x; i < kTopkSlice; i += blockDim.x)
    keys[i] = i < n ? argmax_key(row[lo + i], (uint32_t)(lo + i)) : 0ull;
  __syncthreads();
  for (int r = 0; r < k; ++r) {
    unsigned long long v = 0ull;
    for (int i = threadIdx.x; i < kTopkSlice; i += blockDim.x) v = umax64(v, keys[i]);
    const unsigned long long m = block_max_key(v, red);
    if (threadIdx.x == 0) cand[(size_t)blockIdx.x * k + r] = m;
    for (int i = threadIdx.x; i < kTopkSlice; i += blockDim.x)
      if (keys[i] == m && m != 0ull) keys[i] = 0ull;
    __syncthreads();
  }
}

__global__ __launch_bounds__(256) void k_topk_merge(unsigned long long* __restrict__ cand, int n, int k,
                                                    unsigned long long* __restrict__ out) {
  __shared__ unsigned long long red[16];
  for (int r = 0; r < k; ++r) {
    unsigned long long v = 0ull;
    for (int i = threadIdx.x; i < n; i += blockDim.x) v = umax64(v, cand[i]);
    const unsigned long long m = block_max_key(v, red);
    if (threadIdx.x == 0) out[r] = m;
    for (int i = threadIdx.x; i < n; i += blockDim.x)
      if (cand[i] == m && m != 0ull) cand[i] = 0ull;
    __syncthreads();
  }
}

hipError_t launch_topk(const float* row, int V, int k, unsigned long long* cand, unsigned long long* out,
                       hipStream_t st) {
  const int blocks = (V + kTopkSlice - 1) / kTopkSlice;
  if (k < 1 || k > kTopkMax || blocks > kTopkBlocks) return hipErrorInvalidValue;
  hipLaunchKernelGGL(k_topk_blocks, dim3(blocks), dim3(256), 0, st, row, V, k, cand);
  hipLaunchKernelGGL(k_topk_merge, dim3(1), dim3(256), 0, st, cand, blocks * k, k, out);
  return hipGetLastError();
}

// Selected logits: out[i] = row[ids[i]].
__global__ __launch_bounds__(256) void k_gather(const float* __restrict__ row, const int* __restrict__ ids, int n,
                                                float* __restrict__ out) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) out[i] = row[ids[i]];
}
hipError_t launch_gather(const float* row, const int* ids, int n, float* out, hipStream_t st) {
  if (n < 1) return hipErrorInvalidValue;
  hipLaunchKernelGGL(k_gather, dim3((n + 255) / 256), dim3(256), 0, st, row, ids, n, out);
  return hipGetLastError();
}

// Copy the committed KV of one context into another's pool: logical pages
// [0, n_lp) of every layer, through each context's page table (a page is
// 2 * n_kv * 16 * dh contiguous fp16 values per layer).
__global__ __launch_bounds__(256) void k_copy_pages(const uint4* __restrict__ src, const int* __restrict__ src_pt,
                                                    int src_pages, uint4* __restrict__ dst,
                                                    const int* __restrict__ dst_pt, int dst_pages, int page_vecs) {
  const int lp = blockIdx.x, layer = blockIdx.y;
  const uint4* s = src + ((size_t)layer * src_pages + src_pt[lp]) * page_vecs;
  uint4* d = dst + ((size_t)layer * dst_pages + dst_pt[lp]) * page_vecs;
  for (int i = threadIdx.x; i < page_vecs; i += blockDim.x) d[i] = s[i];
}
hipError_t launch_copy_pages(const void* src, const int* src_pt, int src_pages, void* dst, const int* dst_pt,
                             int dst_pages, int n_lp, int n_layers, int page_bytes, hipStream_t st) {
  if (n_lp < 1 || page_bytes % 16) return hipErrorInvalidValue;
  hipLaunchKernelGGL(k_copy_pages, dim3(n_lp, n_layers), dim3(256), 0, st, (const uint4*)src, src_pt, src_pages,
                     (uint4*)dst, dst_pt, dst_pages, page_bytes / 16);
  return hipGetLastError();
}

// ------------------------------------------------------------ weight packing
// Pure permutation into the tile layouts above.  Row i (0..15) of output
// tile T comes from:
//   layout 0: src0 row 16T + i
//   layout 1 (gate/up): i < 8: src0 (gate) row 8T + i; else src1 (up) row 8T + i - 8
//   layout 2 (QKV, per head of head_dim rows, gph = head_dim/16 tiles per
//            head): tile (head h, s) holds, for f = pair_of(i), dim 8s + f
//            in row i when i & 4 == 0 and its RoPE partner dh/2 + 8s + f in
//            row i ^ 4, so either 8-row half of the tile holds whole pairs
__device__ __forceinline__ int pack_src_row(int layout, int T, int i, int dh, int& which) {
  which = 0;
  if (layout == 1) {
    which = i >= 8;
    return 8 * T + (i & 7);
  }
  if (layout == 2) {
    const int half = dh >> 1, gph = half >> 3;
    const int hh = T / gph, sb = T % gph;
    return hh * dh + ((i & 4) ? half : 0) + 8 * sb + pair_of(i);
  }
  return T * 16 + i;
}

// bf16 tiles are stored tile-major: chunk kc of tile T is KiB (T * KC + kc),
// so one workgroup streams one contiguous run per item.
__global__ void k_pack_bf16(int layout, const uint16_t* s0, const uint16_t* s1, int n_out, int k, int dh, uint4* dst) {
  const int KC = k >> 5;
  const int n_tiles = n_out >> 4;
  const size_t total = (size_t)n_tiles * KC * 64;
  for (size_t idx = (size_t)blockIdx.x * blockDim.x + threadIdx.x; idx < total; idx += (size_t)gridDim.x * blockDim.x) {
    const int lane = (int)(idx & 63);
    const size_t tk = idx >> 6;
    const int kc = (int)(tk % KC);
    const int T = (int)(tk / KC);
    int which;
    const int row = pack_src_row(layout, T, lane & 15, dh, which);
    const uint16_t* src = which ? s1 : s0;
    const int col = kc * 32 + (lane >> 4) * 8;
    dst[idx] = *reinterpret_cast<const uint4*>(src + (size_t)row * k + col);
  }
}

__global__ void k_pack_int4(int layout, const int8_t* s0, const uint16_t* s0s, const int8_t* s1, const uint16_t* s1s,
                            int n_out, int k, int dh, uint4* dst, uint16_t* dst_s) {
  const int KT = k >> 7;
  const size_t total = (size_t)(n_out >> 4) * KT * 64;
  for (size_t idx = (size_t)blockIdx.x * blockDim.x + threadIdx.x; idx < total; idx += (size_t)gridDim.x * blockDim.x) {
    const int lane = (int)(idx & 63);
    const size_t tk = idx >> 6;
    const int kt = (int)(tk % KT);
    const int T = (int)(tk / KT);
    int which;
    const int i = lane & 15, g = lane >> 4;
    const int row = pack_src_row(layout, T, i, dh, which);
    const int8_t* src = which ? s1 : s0;
    uint32_t w[4] = {0u, 0u, 0u, 0u};
    for (int c = 0; c < 32; ++c) {
      const int col = kt * 128 + (c >> 4) * 64 + ((c & 15) >> 3) * 32 + g * 8 + (c & 7);
      const uint32_t nib = (uint32_t)(src[(size_t)row * k + col]) & 15u;
      w[c >> 3] |= nib << ((c & 7) * 4);
    }
    dst[idx] = make_uint4(w[0], w[1], w[2], w[3]);
    // scales: tile (T, kt) holds [group 0..1][16 outputs]; lanes 0..31 write one each
    if (lane < 32) {
      const int gq = lane >> 4, ii = lane & 15;
      int w2;
      const int srow = pack_src_row(layout, T, ii, dh, w2);
      dst_s[tk * 32 + lane] = (w2 ? s1s : s0s)[(size_t)srow * (k >> 6) + kt * 2 + gq];
    }
  }
}

__global__ void k_prof_reset(unsigned long long* slots, int n_pairs) {
  for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < n_pairs; i += gridDim.x * blockDim.x) {
    slots[2 * i] = ~0ull;
    slots[2 * i + 1] = 0ull;
  }
}

hipError_t launch_prof_reset(unsigned long long* slots, int n_pairs, hipStream_t st) {
  hipLaunchKernelGGL(k_prof_reset, dim3(1), dim3(256), 0, st, slots, n_pairs);
  return hipGetLastError();
}

hipError_t launch_pack(int fmt, int layout, const void* src0, const void* src0_scales, const void* src1,
                       const void* src1_scales, int n, int k, int dh, void* dst, void* dst_scales, hipStream_t st) {
  const int blocks = 2048;
  const int n_out = layout == 1 ? 2 * n : n;
  if (fmt == 0) {
    hipLaunchKernelGGL(k_pack_bf16, dim3(blocks), dim3(256), 0, st, layout, (const uint16_t*)src0,
                       (const uint16_t*)src1, n_out, k, dh, (uint4*)dst);
  } else {
    hipLaunchKernelGGL(k_pack_int4, dim3(blocks), dim3(256), 0, st, layout, (const int8_t*)src0,
                       (const uint16_t*)src0_scales, (const int8_t*)src1, (const uint16_t*)src1_scales, n_out, k, dh,
                       (uint4*)dst, (uint16_t*)dst_scales);
  }
  return hipGetLastError();
}

}  // namespace sv
