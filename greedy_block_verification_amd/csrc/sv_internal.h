// Internal declarations shared by the HIP kernels (sv_kernels.hip) and the
// host runtime (sv_runtime.cpp).  Not part of the public ABI.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sv {

constexpr int kMaxRows = 64;        // rows of a weight-streaming forward (verify: k+1; short prefill chunks)
constexpr int kMaxPrefillRows = 16384;   // most rows of one row-tiled (prefill) forward
constexpr int kPage = 16;           // positions per KV page
constexpr int kGemmStageBytes = 136 * 1024;   // LDS a GEMM workgroup stages activation planes in
constexpr int kAttnBlock = 64;      // positions per online-softmax block (4 pages)
constexpr int kAttnMaxSplits = 64;  // most KV splits of one row (the split plan depends only on its ctx)
constexpr int kAttnQRows = 256;     // most (row, q head) pairs one attention workgroup holds (16 MFMA tiles)
constexpr int kColGroup = 64;       // LM-head columns per argmax record (4 MFMA tiles of 16)
constexpr int kEpiCols = 256;       // columns one epilogue workgroup owns (whole heads, 8 gate/up tiles)

// Parameters of one forward, staged host -> device before the launches.
// Layout in device memory: int32 [0] kv_len, [1] rows, [2..2+rows) row ids.

// One sequence of a batched forward (several contexts' windows in one pass):
// its KV pool and page table, its committed length and its rows [row0, row0 + m).
struct SeqDev {
  uint16_t* kv_pool;
  const int* page_table;
  int n_pages, n_lpages;   // physical pages of its pool, logical pages (max_ctx / 16)
  int kv_len, row0, m, pad;
};
constexpr int kMaxBatch = 64;       // most sequences of one batched forward

// Weight-matrix roles of the skinny GEMM (each has its own epilogue).
enum GemmRole { kRoleQkv = 0, kRoleO = 1, kRoleGateUp = 2, kRoleDown = 3, kRoleLmHead = 4 };

// Activations cross kernels as two bf16 planes hi, lo ([rows][width], the
// value is hi + lo to about 16 significant bits): they are the GEMMs' MFMA
// operands as they are.
struct GemmArgs {
  const void* W;         // packed weight tiles
  const void* Wscale;    // packed int4 group scales (int4 only)
  int N, K, S, M;        // outputs, inputs, waves splitting K per workgroup (fixed per matrix), rows
  int fmt;               // 0 bf16, 1 int4
  const uint16_t* bhi;   // activation planes [M][K]
  const uint16_t* blo;
  // RMSNorm consumers (QKV, gate/up, LM head): the planes hold x * g; the
  // epilogue scales by 1 / sqrt(mean(x^2) + eps) from the residual's sums of squares
  const float* ss;       // [M][K/16]
  float eps;
  const int* params;     // device forward parameters (kv_len)
  // residual roles (O, down): x += y, sums of squares, planes of x * g_next
  float* x;              // [M][N] fp32
  float* ss_out;         // [M][N/16]
  const uint16_t* gnext; // bf16 [N] gain of the next RMSNorm
  uint16_t* uhi;         // [M][N]
  uint16_t* ulo;
  // gate/up: planes of act(gate) * up
  uint16_t* ahi;         // [M][N/2]
  uint16_t* alo;
  int act;               // 0 SiLU, 1 tanh-GELU
  // QKV: RoPE, q to the workspace, K/V (fp16) into the paged cache
  float* q_out;          // [M][nq][dh] fp32
  uint16_t* kv_pool;
  const int* page_table;
  int n_pages, layer, nq, nkv, dh;
  const float2* rope;    // [max_ctx][dh/2] (cos, sin)
  // batched forward (else null): row r belongs to sequence rowseq[r]; its
  // position, pool and page table come from seqs[] instead of the fields above
  const SeqDev* seqs;
  const int* rowseq;
  // LM head
  unsigned long long* best;   // [M] row argmax keys (orderable logit, ~id), zeroed by the embed kernel
  float* logits;         // optional [M][N] fp32
  unsigned long long* prof;   // optional [2]: (min start, max end) device wall clock
  // item plan of the one-workgroup-per-CU bf16 kernel (set by launch_gemm):
  // whole items below n_full, and half items for workgroups below n_half
  int n_full, n_half;
  // launch constants of the skinny kernels (set by the host dispatch, so no
  // division runs before the weight ring starts): chunks per LDS stage,
  // stages per item, chunks per wave per stage and per item, and whether the
  // bf16 kernel stages its activations through the register prologue
  int cs, n_stages, cpws, cpi, pro_fast;
};

struct AttnArgs {
  const int* params;
  const float* q;        // [M][nq][dh] fp32, after RoPE
  const uint16_t* kv_pool;
  const int* page_table;
  int n_pages, layer, nq, nkv, dh, M, n_split;   // n_split: splits of the longest row
  int n_lpages;          // logical pages (page_table entries) = max_ctx / 16
  float scale_log2;      // log2(e) / sqrt(dh)
  float* part;           // [M][nq][part_splits][dh + 4]  (m, l, -, -, o[dh])
  int part_splits;       // split slots per (row, q head) in `part` (most splits any row of this context can have)
  uint16_t* ohi;         // output planes [M][nq*dh]
  uint16_t* olo;
  unsigned long long* prof;   // optional [2]: start stamped by the split kernel, end by the last kernel
  // batched forward (else null): q tile t covers q-rows tiles[t].y .. +15 of
  // sequence tiles[t].x (a tile never mixes sequences)
  const SeqDev* seqs;
  const int* rowseq;
  const int2* tiles;
  int n_tiles;
  // set by launch_attention
  int spw;               // splits per workgroup
  int wpb;               // waves per workgroup
  int final_fold;        // 1: one workgroup per KV head folds its splits in LDS and writes the output
  // set by the launchers: q heads per KV head, q tiles and split groups, and
  // for each the multiplier that divides by it (n / d as the high word of
  // n * magic), so the kernels run no integer division before their loads
  int G, n_qt, n_sg;
  unsigned g_magic, qt_magic, sg_magic;
  // set by the caller: blocks per split of the first row, the split
  // kernel's guess of where a unit starts (checked: speed only; 0 = 1), and
  // the device's SIMDs (4 per CU; 0: unknown)
  int bps_guess;
  int n_simd;
};

hipError_t launch_gemm(const GemmArgs& a, int role, int grid, hipStream_t st);
// Rows a GEMM with `waves` waves and `unit` inputs per chunk can stage (one
// chunk per wave: rows x (waves x unit + 8 pad) x 4 bytes of hi + lo planes).
inline int gemm_max_rows(int unit, int waves) {
  return kGemmStageBytes / ((waves * unit + 8) * 4);
}
hipError_t launch_attention(const AttnArgs& a, hipStream_t st);
// Forwards of many rows (prefill chunks): the same per-row arithmetic as
// launch_gemm / launch_attention, tiled for rows instead of streamed for
// weights.  M is any row count; bf16 weights only.
hipError_t launch_gemm_tiled(const GemmArgs& a, int role, hipStream_t st);
hipError_t launch_attention_rows(const AttnArgs& a, hipStream_t st);
// Number of KV splits of a row attending to ctx positions.
int attn_splits(int ctx);
// Blocks of 64 positions per split for a row of context ctx.
int attn_blocks_per_split(int ctx);
// Most splits of any row of a forward of M rows after kv_len positions (the
// rows attend to kv_len + 1 .. kv_len + M positions).
int attn_splits_max(int kv_len, int M);
// Embedding rows of the forward's ids; also clears the M row-argmax keys.
// hparams: the forward's [kv_len, M, ids] in pinned host memory (device
// address); params: their device copy, which k_embed writes for the later kernels
hipError_t launch_embed(const int* hparams, int* params, int M, const void* embed, int vocab, int d, float* x,
                        float* ss, const uint16_t* g0, uint16_t* uhi, uint16_t* ulo, unsigned long long* best,
                        hipStream_t st);
hipError_t launch_accept(const int* params, int M, int verify, const unsigned long long* best, int* result,
                         hipStream_t st);
// Batched verify: per sequence s, n_s leading matches among its rows and
// next_s = argmax of row row0_s + n_s, at result[2 + M + 2 s], [2 + M + 2 s + 1].
hipError_t launch_accept_batch(const int* params, int M, const SeqDev* seqs, int n_seq,
                               const unsigned long long* best, int* result, hipStream_t st);
// Audit mode.  Top-k of an fp32 row in argmax-key order (cand: kTopkBlocks *
// kTopkMax scratch keys, out: k keys), selected-logit gather, and the copy of
// one context's committed KV pages into another's pool.
constexpr int kTopkMax = 64, kTopkSlice = 1024, kTopkBlocks = 1024;
hipError_t launch_topk(const float* row, int V, int k, unsigned long long* cand, unsigned long long* out,
                       hipStream_t st);
hipError_t launch_gather(const float* row, const int* ids, int n, float* out, hipStream_t st);
hipError_t launch_copy_pages(const void* src, const int* src_pt, int src_pages, void* dst, const int* dst_pt,
                             int dst_pages, int n_lp, int n_layers, int page_bytes, hipStream_t st);
// Profiling slots: (start, end) pairs set to (max, 0) before a forward.
hipError_t launch_prof_reset(unsigned long long* slots, int n_pairs, hipStream_t st);
hipError_t launch_pack(int fmt, int layout, const void* src0, const void* src0_scales, const void* src1,
                       const void* src1_scales, int n, int k, int dh, void* dst, void* dst_scales,
                       hipStream_t st);

}  // namespace sv
