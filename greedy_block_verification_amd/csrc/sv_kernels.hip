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

namespace sv {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
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
// bf16 tile: 16 outputs x 32 inputs = 1 KiB, stored in MFMA operand order:
// lane l = g*16 + i holds outputs (tile*16 + i), inputs (chunk*32 + 8g .. +7)
// as one 16-byte vector at byte 16*l.  Tiles are [n_tile][k_chunk], so one
// wave streaming a tile row reads contiguous KiBs.
//
// int4 tile: 16 outputs x 128 inputs (two scale groups of 64) = 1 KiB of
// codes; lane l's 16 bytes hold 32 nibbles c = 0..31 for input
// 128*kt + 64*(c/16) + 32*((c%16)/8) + 8g + c%8 (nibble 2b low, 2b+1 high of
// byte b).  Scales: per tile 64 B = [group 0..1][16 outputs] bf16.

// ------------------------------------------------------------ skinny GEMM
// Y[r][n] = sum_k B[r][k] * W[n][k] for r < M.  Workgroup = 4 waves on one
// 64-output group (4 tiles); the S*4 (split, wave) slices of K are fixed per
// matrix.  Each wave runs its chunks in ascending order through one MFMA
// accumulator chain per (row tile, output tile); the 4 wave partials are added
// in wave order; split partials are added in split order by the epilogue.
// The row count only sets how many row tiles are computed.

template <int BM>
__device__ __forceinline__ uint4 load_b(const GemmArgs& a, int r, int k0, float inv) {
  if (BM == kBBf16) {
    return *reinterpret_cast<const uint4*>(a.xb + (size_t)r * a.K + k0);
  } else {
    const float4* xp = reinterpret_cast<const float4*>(a.xf + (size_t)r * a.K + k0);
    const float4 x0 = xp[0], x1 = xp[1];
    const uint4 gb = *reinterpret_cast<const uint4*>(a.gain + k0);
    const float xs[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
    const uint32_t gw[4] = {gb.x, gb.y, gb.z, gb.w};
    uint16_t h[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float g = bf2f((uint16_t)((gw[e >> 1] >> ((e & 1) * 16)) & 0xffffu));
      h[e] = f2bf((xs[e] * inv) * g);
    }
    return make_uint4(pack2(h[0], h[1]), pack2(h[2], h[3]), pack2(h[4], h[5]), pack2(h[6], h[7]));
  }
}

// int4 nibble -> bf16 bits of the integer code (exact).
__device__ __forceinline__ uint16_t code_bf16(uint32_t nib) {
  const int q = (int)(nib ^ 8u) - 8;
  return f2bf((float)q);
}

// 8 nibbles (one 32-bit word) -> one MFMA operand of 8 bf16.
__device__ __forceinline__ uint4 codes8(uint32_t w) {
  return make_uint4(pack2(code_bf16(w & 15u), code_bf16((w >> 4) & 15u)),
                    pack2(code_bf16((w >> 8) & 15u), code_bf16((w >> 12) & 15u)),
                    pack2(code_bf16((w >> 16) & 15u), code_bf16((w >> 20) & 15u)),
                    pack2(code_bf16((w >> 24) & 15u), code_bf16((w >> 28) & 15u)));
}

template <int TM, int BM, int OUT, int TAG>
__global__ __launch_bounds__(256) void k_gemm_bf16(GemmArgs a) {
  __shared__ f32x4 red[4][4][64];
  __shared__ uint64_t bestw[4][16];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int ng = blockIdx.x, s = blockIdx.y;
  const int KC = a.K >> 5;
  const int cpw = KC / (a.S * 4);
  const int kc0 = (s * 4 + wave) * cpw;
  const int j = lane & 15, g = lane >> 4;

  float inv[TM];
#pragma unroll
  for (int rt = 0; rt < TM; ++rt) {
    inv[rt] = 0.f;
    if (BM == kBNorm) {
      const int r = rt * 16 + j;
      if (r < a.M) {
        const int nsl = a.K >> 8;
        float sum = a.ss[(size_t)r * nsl];
        for (int c = 1; c < nsl; ++c) sum = sum + a.ss[(size_t)r * nsl + c];
        inv[rt] = 1.0f / sqrtf(sum / (float)a.K + a.eps);
      }
    }
  }

  f32x4 acc[TM][4];
#pragma unroll
  for (int rt = 0; rt < TM; ++rt)
#pragma unroll
    for (int t = 0; t < 4; ++t) acc[rt][t] = f32x4{0.f, 0.f, 0.f, 0.f};

  const uint4* Wt = reinterpret_cast<const uint4*>(a.W) + (size_t)(ng * 4) * KC * 64 + lane;
#pragma unroll 2
  for (int c = 0; c < cpw; ++c) {
    const int kc = kc0 + c;
    uint4 A[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) A[t] = ld_stream(Wt + ((size_t)t * KC + kc) * 64);
#pragma unroll
    for (int rt = 0; rt < TM; ++rt) {
      const int r = rt * 16 + j;
      uint4 B = make_uint4(0u, 0u, 0u, 0u);
      if (r < a.M) B = load_b<BM>(a, r, kc * 32 + g * 8, inv[rt]);
#pragma unroll
      for (int t = 0; t < 4; ++t) acc[rt][t] = mfma16x16x32(A[t], B, acc[rt][t]);
    }
  }

#pragma unroll
  for (int rt = 0; rt < TM; ++rt) {
#pragma unroll
    for (int t = 0; t < 4; ++t) red[wave][t][lane] = acc[rt][t];
    __syncthreads();
    // Thread (wave w, lane) finishes output tile w: wave partials in order.
    f32x4 v = red[0][wave][lane];
    const f32x4 v1 = red[1][wave][lane], v2 = red[2][wave][lane], v3 = red[3][wave][lane];
    v.x = v.x + v1.x; v.y = v.y + v1.y; v.z = v.z + v1.z; v.w = v.w + v1.w;
    v.x = v.x + v2.x; v.y = v.y + v2.y; v.z = v.z + v2.z; v.w = v.w + v2.w;
    v.x = v.x + v3.x; v.y = v.y + v3.y; v.z = v.z + v3.z; v.w = v.w + v3.w;
    // v[i] = Y[r = rt*16 + j][n = (ng*4 + wave)*16 + 4g + i]
    const int r = rt * 16 + j;
    const int n0 = (ng * 4 + wave) * 16 + 4 * g;
    if (OUT == kOutPartial) {
      if (r < a.M)
        *reinterpret_cast<float4*>(a.partial + ((size_t)s * a.M + r) * a.N + n0) = make_float4(v.x, v.y, v.z, v.w);
    } else {
      if (a.logits != nullptr && r < a.M)
        *reinterpret_cast<float4*>(a.logits + (size_t)r * a.N + n0) = make_float4(v.x, v.y, v.z, v.w);
      uint64_t b = argmax_key(v.x, n0);
      b = umax64(b, argmax_key(v.y, n0 + 1));
      b = umax64(b, argmax_key(v.z, n0 + 2));
      b = umax64(b, argmax_key(v.w, n0 + 3));
      b = umax64(b, __shfl_xor(b, 16));
      b = umax64(b, __shfl_xor(b, 32));
      if (g == 0) bestw[wave][j] = b;
      __syncthreads();
      if (threadIdx.x < 16) {
        const int rr = rt * 16 + threadIdx.x;
        const uint64_t bb = umax64(umax64(bestw[0][threadIdx.x], bestw[1][threadIdx.x]),
                                   umax64(bestw[2][threadIdx.x], bestw[3][threadIdx.x]));
        if (rr < a.M) a.best[(size_t)rr * (a.N >> 6) + ng] = bb;
      }
    }
    __syncthreads();
  }
}

// int4 weights: per (row tile, output tile) and per scale group, two MFMAs
// over the group's 64 inputs start from zero; the group sum is then scaled
// by the fp32 group scale and added to the running fp32 sum in group order.
template <int TM, int BM, int OUT, int TAG>
__global__ __launch_bounds__(256) void k_gemm_int4(GemmArgs a) {
  __shared__ f32x4 red[4][4][64];
  __shared__ uint64_t bestw[4][16];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int ng = blockIdx.x, s = blockIdx.y;
  const int KT = a.K >> 7;                 // 128-input tiles
  const int tpw = KT / (a.S * 4);
  const int kt0 = (s * 4 + wave) * tpw;
  const int j = lane & 15, g = lane >> 4;

  float inv[TM];
#pragma unroll
  for (int rt = 0; rt < TM; ++rt) {
    inv[rt] = 0.f;
    if (BM == kBNorm) {
      const int r = rt * 16 + j;
      if (r < a.M) {
        const int nsl = a.K >> 8;
        float sum = a.ss[(size_t)r * nsl];
        for (int c = 1; c < nsl; ++c) sum = sum + a.ss[(size_t)r * nsl + c];
        inv[rt] = 1.0f / sqrtf(sum / (float)a.K + a.eps);
      }
    }
  }

  f32x4 acc[TM][4];
#pragma unroll
  for (int rt = 0; rt < TM; ++rt)
#pragma unroll
    for (int t = 0; t < 4; ++t) acc[rt][t] = f32x4{0.f, 0.f, 0.f, 0.f};

  const uint4* Wt = reinterpret_cast<const uint4*>(a.W) + (size_t)(ng * 4) * KT * 64 + lane;
  const uint2* St = reinterpret_cast<const uint2*>(a.Wscale) + (size_t)(ng * 4) * KT * 8 + g;
  for (int c = 0; c < tpw; ++c) {
    const int kt = kt0 + c;
    uint4 Q[4];
    uint2 SC[4][2];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      Q[t] = ld_stream(Wt + ((size_t)t * KT + kt) * 64);
      const uint2* sp = St + ((size_t)t * KT + kt) * 8;
      SC[t][0] = sp[0];
      SC[t][1] = sp[4];
    }
#pragma unroll
    for (int gq = 0; gq < 2; ++gq) {
      uint4 Bv[TM][2];
#pragma unroll
      for (int rt = 0; rt < TM; ++rt) {
        const int r = rt * 16 + j;
#pragma unroll
        for (int ch = 0; ch < 2; ++ch) {
          Bv[rt][ch] = make_uint4(0u, 0u, 0u, 0u);
          if (r < a.M) Bv[rt][ch] = load_b<BM>(a, r, kt * 128 + gq * 64 + ch * 32 + g * 8, inv[rt]);
        }
      }
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const uint32_t w0 = gq == 0 ? Q[t].x : Q[t].z;
        const uint32_t w1 = gq == 0 ? Q[t].y : Q[t].w;
        const uint4 A0 = codes8(w0), A1 = codes8(w1);
        const float s0 = bf2f((uint16_t)(SC[t][gq].x & 0xffffu)), s1 = bf2f((uint16_t)(SC[t][gq].x >> 16));
        const float s2 = bf2f((uint16_t)(SC[t][gq].y & 0xffffu)), s3 = bf2f((uint16_t)(SC[t][gq].y >> 16));
#pragma unroll
        for (int rt = 0; rt < TM; ++rt) {
          f32x4 p = f32x4{0.f, 0.f, 0.f, 0.f};
          p = mfma16x16x32(A0, Bv[rt][0], p);
          p = mfma16x16x32(A1, Bv[rt][1], p);
          acc[rt][t].x = fmaf(s0, p.x, acc[rt][t].x);
          acc[rt][t].y = fmaf(s1, p.y, acc[rt][t].y);
          acc[rt][t].z = fmaf(s2, p.z, acc[rt][t].z);
          acc[rt][t].w = fmaf(s3, p.w, acc[rt][t].w);
        }
      }
    }
  }

#pragma unroll
  for (int rt = 0; rt < TM; ++rt) {
#pragma unroll
    for (int t = 0; t < 4; ++t) red[wave][t][lane] = acc[rt][t];
    __syncthreads();
    f32x4 v = red[0][wave][lane];
    const f32x4 v1 = red[1][wave][lane], v2 = red[2][wave][lane], v3 = red[3][wave][lane];
    v.x = v.x + v1.x; v.y = v.y + v1.y; v.z = v.z + v1.z; v.w = v.w + v1.w;
    v.x = v.x + v2.x; v.y = v.y + v2.y; v.z = v.z + v2.z; v.w = v.w + v2.w;
    v.x = v.x + v3.x; v.y = v.y + v3.y; v.z = v.z + v3.z; v.w = v.w + v3.w;
    const int r = rt * 16 + j;
    const int n0 = (ng * 4 + wave) * 16 + 4 * g;
    if (OUT == kOutPartial) {
      if (r < a.M)
        *reinterpret_cast<float4*>(a.partial + ((size_t)s * a.M + r) * a.N + n0) = make_float4(v.x, v.y, v.z, v.w);
    }
    __syncthreads();
  }
}

// TAG only names the weight matrix (qkv, o, gate/up, down, LM head) so each
// role is a separate kernel symbol in profiles; the code is the same.
template <int BM, int OUT, int TAG>
static hipError_t gemm_dispatch(const GemmArgs& a, hipStream_t st) {
  const dim3 grid(a.N / kColGroup, a.S), block(256);
  const int tm = (a.M + 15) / 16;
  if (a.fmt == 1) {
    if (OUT != kOutPartial) return hipErrorInvalidValue;
    switch (tm) {
      case 1: hipLaunchKernelGGL((k_gemm_int4<1, BM, OUT, TAG>), grid, block, 0, st, a); break;
      case 2: hipLaunchKernelGGL((k_gemm_int4<2, BM, OUT, TAG>), grid, block, 0, st, a); break;
      case 3: hipLaunchKernelGGL((k_gemm_int4<3, BM, OUT, TAG>), grid, block, 0, st, a); break;
      case 4: hipLaunchKernelGGL((k_gemm_int4<4, BM, OUT, TAG>), grid, block, 0, st, a); break;
      default: return hipErrorInvalidValue;
    }
  } else {
    switch (tm) {
      case 1: hipLaunchKernelGGL((k_gemm_bf16<1, BM, OUT, TAG>), grid, block, 0, st, a); break;
      case 2: hipLaunchKernelGGL((k_gemm_bf16<2, BM, OUT, TAG>), grid, block, 0, st, a); break;
      case 3: hipLaunchKernelGGL((k_gemm_bf16<3, BM, OUT, TAG>), grid, block, 0, st, a); break;
      case 4: hipLaunchKernelGGL((k_gemm_bf16<4, BM, OUT, TAG>), grid, block, 0, st, a); break;
      default: return hipErrorInvalidValue;
    }
  }
  return hipGetLastError();
}

hipError_t launch_gemm(const GemmArgs& a, int role, hipStream_t st) {
  if (a.M < 1 || a.M > kMaxRows || a.N % kColGroup != 0) return hipErrorInvalidValue;
  switch (role) {
    case kRoleQkv: return gemm_dispatch<kBNorm, kOutPartial, kRoleQkv>(a, st);
    case kRoleO: return gemm_dispatch<kBBf16, kOutPartial, kRoleO>(a, st);
    case kRoleGateUp: return gemm_dispatch<kBNorm, kOutPartial, kRoleGateUp>(a, st);
    case kRoleDown: return gemm_dispatch<kBBf16, kOutPartial, kRoleDown>(a, st);
    case kRoleLmHead: return gemm_dispatch<kBNorm, kOutArgmax, kRoleLmHead>(a, st);
    default: return hipErrorInvalidValue;
  }
}

// ------------------------------------------------------------ split-K epilogues
// One workgroup owns 256 consecutive outputs (whole heads; whole gate/up tile
// pairs) and walks the rows.  Split partials are summed in split order.
__device__ __forceinline__ float act_fn(float x, int act) {
  if (act == 0) return x / (1.0f + expf(-x));
  const float c = 0.7978845608028654f;  // sqrt(2/pi)
  return 0.5f * x * (1.0f + tanhf(c * (x + 0.044715f * (x * x * x))));
}

__global__ __launch_bounds__(256) void k_epilogue(EpiArgs a) {
  __shared__ float y[kEpiCols];
  __shared__ float red4[4];
  const int t = threadIdx.x;
  const int n = blockIdx.x * kEpiCols + t;
  const bool live = n < a.N;
  const int kv_len = a.params[0];
  for (int r = 0; r < a.M; ++r) {
    float v = 0.f;
    if (live) {
      v = a.partial[(size_t)r * a.N + n];
      for (int s = 1; s < a.S; ++s) v = v + a.partial[((size_t)s * a.M + r) * a.N + n];
    }
    if (a.kind == kEpiResid) {
      float xn = 0.f;
      if (live) {
        xn = a.x[(size_t)r * a.N + n] + v;
        a.x[(size_t)r * a.N + n] = xn;
      }
      const float sq = block_sum256(xn * xn, red4);
      if (t == 0) a.ss[(size_t)r * (a.N >> 8) + blockIdx.x] = sq;
    } else if (a.kind == kEpiGlu) {
      y[t] = v;
      __syncthreads();
      if (t < kEpiCols / 2) {
        const int b = t >> 4, i = t & 15;
        const int f = blockIdx.x * (kEpiCols / 2) + t;
        if (f < (a.N >> 1)) {
          const float gate = y[32 * b + i], up = y[32 * b + 16 + i];
          a.act_out[(size_t)r * (a.N >> 1) + f] = f2bf(act_fn(gate, a.act) * up);
        }
      }
      __syncthreads();
    } else {  // kEpiQkv
      y[t] = v;
      __syncthreads();
      if (live) {
        const int qd = a.nq * a.dh, kd = a.nkv * a.dh;
        const int half = a.dh >> 1;
        const int pos = kv_len + r;
        const int d = n % a.dh;
        const int i = d % half;
        float out = v;
        if (n < qd + kd) {
          const float2 cs = a.rope[(size_t)pos * half + i];
          const float partner = (d < half) ? y[t + half] : y[t - half];
          out = (d < half) ? (v * cs.x - partner * cs.y) : (v * cs.x + partner * cs.y);
        }
        if (n < qd) {
          a.q_out[(size_t)r * qd + n] = out;
        } else {
          const int kv = (n < qd + kd) ? 0 : 1;
          const int h = (n - qd - kv * kd) / a.dh;
          const int page = a.page_table[pos / kPage];
          const size_t off = ((((size_t)a.layer * a.n_pages + page) * 2 + kv) * a.nkv + h) * kPage + (pos % kPage);
          a.kv_pool[off * a.dh + d] = f2bf(out);
        }
      }
      __syncthreads();
    }
  }
}

hipError_t launch_epilogue(const EpiArgs& a, hipStream_t st) {
  const int blocks = (a.N + kEpiCols - 1) / kEpiCols;
  hipLaunchKernelGGL(k_epilogue, dim3(blocks), dim3(256), 0, st, a);
  return hipGetLastError();
}

// ------------------------------------------------------------ attention
// One wave per (split, q head, row).  Row r attends to ctx = kv_len + r + 1
// positions; split i covers [512 i, min(512 (i+1), ctx)), walked in blocks of
// 64 absolute positions (one per lane).  Scores are sequential fp32 dot
// products; masked lanes take -inf by select and are skipped in P.V, so a
// position past ctx (stale or poisoned KV) never enters the arithmetic.
template <int DH>
__global__ __launch_bounds__(64) void k_attn_split(AttnArgs a) {
  constexpr int PER = DH / 64;
  __shared__ float qs[DH];
  const int split = blockIdx.x, j = blockIdx.y, r = blockIdx.z;
  const int lane = threadIdx.x;
  const int kv_len = a.params[0];
  const int ctx = kv_len + r + 1;
  const int t0 = split * kAttnSplit;
  if (t0 >= ctx) return;
  const int t1 = min(ctx, t0 + kAttnSplit);
  const int h = j / (a.nq / a.nkv);
  for (int d = lane; d < DH; d += 64) qs[d] = a.q[((size_t)r * a.nq + j) * DH + d];
  __syncthreads();

  const size_t layer_base = (size_t)a.layer * a.n_pages;
  auto kv_row = [&](int pos, int kv) -> const uint16_t* {
    const int page = a.page_table[pos / kPage];
    const size_t off = (((layer_base + page) * 2 + kv) * a.nkv + h) * kPage + (pos % kPage);
    return a.kv_pool + off * DH;
  };

  float m = -INFINITY, l = 0.f;
  float o[PER];
#pragma unroll
  for (int e = 0; e < PER; ++e) o[e] = 0.f;

  for (int b = t0; b < t1; b += 64) {
    const int t = b + lane;
    const bool valid = t < t1;
    float s = -INFINITY;
    if (valid) {
      const uint4* kp = reinterpret_cast<const uint4*>(kv_row(t, 0));
      float dot = 0.f;
#pragma unroll 4
      for (int d8 = 0; d8 < DH / 8; ++d8) {
        const uint4 kk = kp[d8];
        const uint32_t w[4] = {kk.x, kk.y, kk.z, kk.w};
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float kf = bf2f((uint16_t)((w[e >> 1] >> ((e & 1) * 16)) & 0xffffu));
          dot = fmaf(qs[d8 * 8 + e], kf, dot);
        }
      }
      s = dot * a.scale_log2;
    }
    const float mn = fmaxf(m, wave_max(s));
    const float alpha = exp2f(m - mn);
    const float p = valid ? exp2f(s - mn) : 0.f;
    l = l * alpha + wave_sum(p);
    const int nt = min(64, t1 - b);
    float accv[PER];
#pragma unroll
    for (int e = 0; e < PER; ++e) accv[e] = 0.f;
    for (int tt = 0; tt < nt; ++tt) {
      const float pt = __shfl(p, tt);
      const uint16_t* vp = kv_row(b + tt, 1) + lane * PER;
#pragma unroll
      for (int e = 0; e < PER; ++e) accv[e] = fmaf(pt, bf2f(vp[e]), accv[e]);
    }
#pragma unroll
    for (int e = 0; e < PER; ++e) o[e] = o[e] * alpha + accv[e];
    m = mn;
  }
  float* part = a.part + (((size_t)r * a.nq + j) * a.n_split + split) * (DH + 2);
  if (lane == 0) { part[0] = m; part[1] = l; }
#pragma unroll
  for (int e = 0; e < PER; ++e) part[2 + lane * PER + e] = o[e];
}

// Combine the row's splits in split order: o = sum_i w_i o_i / sum_i w_i l_i
// with w_i = 2^(m_i - max m).
template <int DH>
__global__ __launch_bounds__(64) void k_attn_combine(AttnArgs a) {
  constexpr int PER = DH / 64;
  const int j = blockIdx.x, r = blockIdx.y, lane = threadIdx.x;
  const int ctx = a.params[0] + r + 1;
  const int ns = (ctx + kAttnSplit - 1) / kAttnSplit;
  const float* base = a.part + ((size_t)r * a.nq + j) * a.n_split * (DH + 2);
  float mx = base[0];
  for (int i = 1; i < ns; ++i) mx = fmaxf(mx, base[(size_t)i * (DH + 2)]);
  float L = 0.f, O[PER];
#pragma unroll
  for (int e = 0; e < PER; ++e) O[e] = 0.f;
  for (int i = 0; i < ns; ++i) {
    const float* p = base + (size_t)i * (DH + 2);
    const float w = exp2f(p[0] - mx);
    L = L + p[1] * w;
#pragma unroll
    for (int e = 0; e < PER; ++e) O[e] = O[e] + p[2 + lane * PER + e] * w;
  }
#pragma unroll
  for (int e = 0; e < PER; ++e)
    a.out[(size_t)r * a.nq * DH + (size_t)j * DH + lane * PER + e] = f2bf(O[e] / L);
}

hipError_t launch_attention(const AttnArgs& a, hipStream_t st) {
  if (a.dh == 128) {
    hipLaunchKernelGGL(k_attn_split<128>, dim3(a.n_split, a.nq, a.M), dim3(64), 0, st, a);
    hipLaunchKernelGGL(k_attn_combine<128>, dim3(a.nq, a.M), dim3(64), 0, st, a);
  } else if (a.dh == 64) {
    hipLaunchKernelGGL(k_attn_split<64>, dim3(a.n_split, a.nq, a.M), dim3(64), 0, st, a);
    hipLaunchKernelGGL(k_attn_combine<64>, dim3(a.nq, a.M), dim3(64), 0, st, a);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

// ------------------------------------------------------------ embedding gather
// x[r] = E[id_r] widened to fp32, plus the per-256-column sums of squares the
// first RMSNorm reads (same slicing and order as the residual epilogue).
__global__ __launch_bounds__(256) void k_embed(const int* params, const uint16_t* E, int d, float* x, float* ss) {
  __shared__ float red4[4];
  const int r = blockIdx.x, t = threadIdx.x;
  const int id = params[2 + r];
  const int KC = d >> 5;
  for (int c = 0; c < (d >> 8); ++c) {
    const int k = c * 256 + t;
    const size_t off = ((size_t)(id >> 4) * KC + (k >> 5)) * 512 + (size_t)(((k & 31) >> 3) * 16 + (id & 15)) * 8 + (k & 7);
    const float v = bf2f(E[off]);
    x[(size_t)r * d + k] = v;
    const float sq = block_sum256(v * v, red4);
    if (t == 0) ss[(size_t)r * (d >> 8) + c] = sq;
  }
}

hipError_t launch_embed(const int* params, int M, const void* embed, int vocab, int d, float* x, float* ss,
                        hipStream_t st) {
  (void)vocab;
  hipLaunchKernelGGL(k_embed, dim3(M), dim3(256), 0, st, params, (const uint16_t*)embed, d, x, ss);
  return hipGetLastError();
}

// ------------------------------------------------------------ argmax + acceptance
// Row argmax over the LM head's per-64-column bests (max of packed keys,
// order-free), then the greedy acceptance: n = number of leading drafts equal
// to the argmax of the row before them; next = argmax of row n.
// result: [0] n, [1] next, [2 + r] argmax of row r.
__global__ __launch_bounds__(1024) void k_accept(const int* params, int M, int verify, const uint64_t* best,
                                                 int n_groups, int* result) {
  __shared__ int am[kMaxRows];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  for (int r = wave; r < M; r += 16) {
    uint64_t b = 0;
    for (int i = lane; i < n_groups; i += 64) b = umax64(b, best[(size_t)r * n_groups + i]);
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) b = umax64(b, __shfl_xor(b, o));
    if (lane == 0) am[r] = (int)(0xffffffffu - (uint32_t)(b & 0xffffffffu));
  }
  __syncthreads();
  if (wave == 0) {
    const int a_r = lane < M ? am[lane] : 0;
    if (lane < M) result[2 + lane] = a_r;
    int n;
    if (verify) {
      const int k = M - 1;
      const bool miss = lane < k && params[2 + lane + 1] != a_r;
      const unsigned long long mask = __ballot(miss);
      n = mask ? (__ffsll((long long)mask) - 1) : k;
    } else {
      n = M - 1;
    }
    const int next = __shfl(a_r, n);
    if (lane == 0) { result[0] = n; result[1] = next; }
  }
}

hipError_t launch_accept(const int* params, int M, int verify, const uint64_t* best, int n_groups, int* result,
                         hipStream_t st) {
  hipLaunchKernelGGL(k_accept, dim3(1), dim3(1024), 0, st, params, M, verify, best, n_groups, result);
  return hipGetLastError();
}

// ------------------------------------------------------------ weight packing
// Pure permutation into the tile layouts above.  Output tile T takes source
// tile T (no interleave) or, when src1 is given, tile T/2 of src0 (T even)
// or src1 (T odd): gate and up outputs of the same 16 features share a
// 32-output pair of tiles.
__global__ void k_pack_bf16(const uint16_t* s0, const uint16_t* s1, int n, int k, uint4* dst) {
  const int KC = k >> 5;
  const int n_tiles_out = (s1 ? 2 * n : n) >> 4;
  const size_t total = (size_t)n_tiles_out * KC * 64;
  for (size_t idx = (size_t)blockIdx.x * blockDim.x + threadIdx.x; idx < total; idx += (size_t)gridDim.x * blockDim.x) {
    const int lane = (int)(idx & 63);
    const size_t tk = idx >> 6;
    const int kc = (int)(tk % KC);
    const int T = (int)(tk / KC);
    const uint16_t* src = s0;
    int st = T;
    if (s1) { src = (T & 1) ? s1 : s0; st = T >> 1; }
    const int row = st * 16 + (lane & 15);
    const int col = kc * 32 + (lane >> 4) * 8;
    dst[idx] = *reinterpret_cast<const uint4*>(src + (size_t)row * k + col);
  }
}

__global__ void k_pack_int4(const int8_t* s0, const uint16_t* s0s, const int8_t* s1, const uint16_t* s1s, int n,
                            int k, uint4* dst, uint16_t* dst_s) {
  const int KT = k >> 7;
  const int n_tiles_out = (s1 ? 2 * n : n) >> 4;
  const size_t total = (size_t)n_tiles_out * KT * 64;
  for (size_t idx = (size_t)blockIdx.x * blockDim.x + threadIdx.x; idx < total; idx += (size_t)gridDim.x * blockDim.x) {
    const int lane = (int)(idx & 63);
    const size_t tk = idx >> 6;
    const int kt = (int)(tk % KT);
    const int T = (int)(tk / KT);
    const int8_t* src = s0;
    const uint16_t* srcs = s0s;
    int st = T;
    if (s1) { src = (T & 1) ? s1 : s0; srcs = (T & 1) ? s1s : s0s; st = T >> 1; }
    const int i = lane & 15, g = lane >> 4;
    const int row = st * 16 + i;
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
      dst_s[tk * 32 + lane] = srcs[(size_t)(st * 16 + ii) * (k >> 6) + kt * 2 + gq];
    }
  }
}

hipError_t launch_pack(int fmt, const void* src0, const void* src0_scales, const void* src1, const void* src1_scales,
                       int n, int k, void* dst, void* dst_scales, hipStream_t st) {
  const int blocks = 2048;
  if (fmt == 0) {
    hipLaunchKernelGGL(k_pack_bf16, dim3(blocks), dim3(256), 0, st, (const uint16_t*)src0, (const uint16_t*)src1, n, k,
                       (uint4*)dst);
  } else {
    hipLaunchKernelGGL(k_pack_int4, dim3(blocks), dim3(256), 0, st, (const int8_t*)src0, (const uint16_t*)src0_scales,
                       (const int8_t*)src1, (const uint16_t*)src1_scales, n, k, (uint4*)dst, (uint16_t*)dst_scales);
  }
  return hipGetLastError();
}

}  // namespace sv
