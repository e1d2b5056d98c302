// Internal declarations shared by the HIP kernels (sv_kernels.hip) and the
// host runtime (sv_runtime.cpp).  Not part of the public ABI.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sv {

constexpr int kMaxRows = 64;        // rows of one forward (verify: k+1; prefill chunk)
constexpr int kPage = 16;           // positions per KV page
constexpr int kAttnSplit = 512;     // positions per attention split (fixed: the split plan depends only on ctx)
constexpr int kColGroup = 64;       // output columns one GEMM workgroup owns (4 MFMA tiles of 16)
constexpr int kEpiCols = 256;       // columns one epilogue workgroup owns (whole heads, 8 gate/up tiles)

// Parameters of one forward, staged host -> device before the launches.
// Layout in device memory: int32 [0] kv_len, [1] rows, [2..2+64) row ids.
constexpr int kParamInts = 2 + kMaxRows;

enum BMode { kBBf16 = 0, kBNorm = 1 };
enum OutMode { kOutPartial = 0, kOutArgmax = 1 };
enum EpiKind { kEpiQkv = 0, kEpiResid = 1, kEpiGlu = 2 };
// Weight-matrix roles of the skinny GEMM (fix B operand mode and output mode).
enum GemmRole { kRoleQkv = 0, kRoleO = 1, kRoleGateUp = 2, kRoleDown = 3, kRoleLmHead = 4 };

struct GemmArgs {
  const void* W;         // packed weight tiles
  const void* Wscale;    // packed int4 group scales (int4 only)
  int N, K, S, M;        // outputs, inputs, fixed split-K count, rows
  int fmt;               // 0 bf16, 1 int4
  // B operand (activations)
  const uint16_t* xb;    // kBBf16: [M][K] bf16
  const float* xf;       // kBNorm: [M][K] fp32 residual
  const float* ss;       // kBNorm: [M][K/256] partial sums of squares
  const uint16_t* gain;  // kBNorm: [K] bf16
  float eps;
  // outputs
  float* partial;        // kOutPartial: [S][M][N] fp32
  uint64_t* best;        // kOutArgmax: [M][N/64] packed (orderable logit, ~id)
  float* logits;         // kOutArgmax, optional: [M][N] fp32
};

struct EpiArgs {
  const float* partial;  // [S][M][N]
  int S, M, N;
  int kind;
  const int* params;     // device forward parameters (kv_len)
  // qkv
  float* q_out;          // [M][nq*dh] fp32, after RoPE
  uint16_t* kv_pool;
  const int* page_table;
  int n_pages, layer, nq, nkv, dh;
  const float2* rope;    // [max_ctx][dh/2] (cos, sin)
  // resid
  float* x;              // [M][N] fp32 residual, updated in place
  float* ss;             // [M][N/256] partial sums of squares of the new x
  // glu
  uint16_t* act_out;     // [M][N/2] bf16
  int act;               // 0 SiLU, 1 tanh-GELU
};

struct AttnArgs {
  const int* params;
  const float* q;        // [M][nq][dh]
  const uint16_t* kv_pool;
  const int* page_table;
  int n_pages, layer, nq, nkv, dh, M, n_split;
  float scale_log2;      // log2(e) / sqrt(dh)
  float* part;           // [M][nq][n_split][dh + 2]  (m, l, o[dh])
  uint16_t* out;         // [M][nq*dh] bf16
};

hipError_t launch_gemm(const GemmArgs& a, int role, hipStream_t st);
hipError_t launch_epilogue(const EpiArgs& a, hipStream_t st);
hipError_t launch_attention(const AttnArgs& a, hipStream_t st);
hipError_t launch_embed(const int* params, int M, const void* embed, int vocab, int d,
                        float* x, float* ss, hipStream_t st);
hipError_t launch_accept(const int* params, int M, int verify, const uint64_t* best, int n_groups,
                         int* result, hipStream_t st);
hipError_t launch_pack(int fmt, const void* src0, const void* src0_scales, const void* src1,
                       const void* src1_scales, int n, int k, void* dst, void* dst_scales,
                       hipStream_t st);

}  // namespace sv
