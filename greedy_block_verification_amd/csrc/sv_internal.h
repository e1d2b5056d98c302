// Internal declarations shared by the HIP kernels (sv_kernels.hip) and the
// host runtime (sv_runtime.cpp).  Not part of the public ABI.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sv {

constexpr int kMaxRows = 64;        // rows of one forward (verify: k+1; prefill chunk)
constexpr int kPage = 16;           // positions per KV page
constexpr int kAttnBlock = 64;      // positions per online-softmax block
constexpr int kAttnMaxSplits = 32;  // most KV splits of one row (the split plan depends only on its ctx)
constexpr int kAttnQRows = 256;     // most (row, q head) pairs one attention workgroup holds (16 MFMA tiles)
constexpr int kColGroup = 64;       // LM-head columns per argmax record (4 MFMA tiles of 16)
constexpr int kEpiCols = 256;       // columns one epilogue workgroup owns (whole heads, 8 gate/up tiles)

// Parameters of one forward, staged host -> device before the launches.
// Layout in device memory: int32 [0] kv_len, [1] rows, [2..2+64) row ids.
constexpr int kParamInts = 2 + kMaxRows;

enum BMode { kBBf16 = 0, kBNorm = 1 };
enum OutMode { kOutPartial = 0, kOutArgmax = 1 };
// Weight-matrix roles of the skinny GEMM (fix B operand mode and output mode).
enum GemmRole { kRoleQkv = 0, kRoleO = 1, kRoleGateUp = 2, kRoleDown = 3, kRoleLmHead = 4 };

struct GemmArgs {
  const void* W;         // packed weight tiles
  const void* Wscale;    // packed int4 group scales (int4 only)
  int N, K, S, M;        // outputs, inputs, waves splitting K per workgroup (fixed per matrix), rows
  int fmt;               // 0 bf16, 1 int4
  // B operand (activations)
  const uint16_t* xb;    // kBBf16: [M][K] bf16
  const float* xf;       // kBNorm: [M][K] fp32 residual
  const float* ss;       // kBNorm: [M][K/16] partial sums of squares
  const uint16_t* gain;  // kBNorm: [K] bf16
  float eps;
  // epilogues
  const int* params;     // device forward parameters (kv_len)
  float* x;              // O / down: [M][N] fp32 residual, updated in place
  float* ss_out;         // O / down: [M][N/16] sums of squares of the new x
  uint16_t* act_out;     // gate/up: [M][N/2] bf16
  int act;               // 0 SiLU, 1 tanh-GELU
  uint16_t* q_out;       // QKV: [M][nq][dh] bf16 after RoPE
  uint16_t* kv_pool;
  const int* page_table;
  int n_pages, layer, nq, nkv, dh;
  const float2* rope;    // [max_ctx][dh/2] (cos, sin)
  uint64_t* best;        // LM head: [M][N/16] packed (orderable logit, ~id)
  float* logits;         // LM head, optional: [M][N] fp32
};

struct AttnArgs {
  const int* params;
  const uint16_t* q;     // [M][nq][dh] bf16, after RoPE
  const uint16_t* kv_pool;
  const int* page_table;
  int n_pages, layer, nq, nkv, dh, M, n_split;   // n_split: splits of the longest row (grid x)
  float scale_log2;      // log2(e) / sqrt(dh)
  float* part;           // [M][nq][kAttnMaxSplits][dh + 4]  (m, l, -, -, o[dh])
  uint16_t* out;         // [M][nq*dh] bf16
};

hipError_t launch_gemm(const GemmArgs& a, int role, int grid, hipStream_t st);
hipError_t launch_attention(const AttnArgs& a, hipStream_t st);
// Number of KV splits of a row attending to ctx positions.
int attn_splits(int ctx);
hipError_t launch_embed(const int* params, int M, const void* embed, int vocab, int d,
                        float* x, float* ss, hipStream_t st);
hipError_t launch_accept(const int* params, int M, int verify, const uint64_t* best, int n_groups,
                         int* result, hipStream_t st);
hipError_t launch_pack(int fmt, int layout, const void* src0, const void* src0_scales, const void* src1,
                       const void* src1_scales, int n, int k, int dh, void* dst, void* dst_scales,
                       hipStream_t st);

}  // namespace sv
