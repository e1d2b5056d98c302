// Host runtime behind the sv_* C ABI: argument checks, context state
// (kv_len, next_id, per-position greedy history), workspace layout, and the
// launch sequence of one forward.  All arithmetic runs in sv_kernels.hip.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <array>
#include <cstdlib>
#include <map>
#include <cmath>
#include <cstring>
#include <mutex>
#include <new>
#include <vector>

#include "../../include/sv.h"
#include "sv_internal.h"

using namespace sv;

namespace {

struct GemmPlan {
  int N = 0, K = 0, S = 1, fmt = 0;   // S: waves splitting K in one workgroup
  int grid = 1;                       // persistent workgroups (each loops over 16-output items)
};

struct Layout {
  int rows = 0;   // most rows of one forward: 64, or max_prefill_rows when larger
  int max_tiles = 0;   // attention q tiles of a batched forward
  size_t batch = 0, batch_bytes = 0;   // batched-forward tables: rowseq [rows], seqs [kMaxBatch], tiles
  size_t topk = 0, sel = 0;   // audit mode: top-k scratch keys and results, selected-logit ids and values
  size_t params = 0, x = 0, ss = 0, q = 0, attn_part = 0, uplanes = 0, oplanes = 0, aplanes = 0, best = 0,
         logits = 0, rope = 0, prof = 0, total = 0;
  int max_split = 1;
};

size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

// Waves that split K inside one GEMM workgroup.  It depends only on the
// matrix shape, never on the number of rows, so every row count shares one
// summation order.
int choose_waves(int K, int unit, int max_waves) {
  const int chunks = K / unit;
  for (int w : {16, 12, 8, 6, 4, 3, 2, 1})
    if (w <= max_waves && chunks % w == 0) return w;
  return 0;
}

bool valid_config(const sv_config& c) {
  if (c.n_layers < 1 || c.d_model < 256 || c.n_q_heads < 1 || c.n_kv_heads < 1 || c.d_ff < 256 || c.vocab < 64)
    return false;
  if (c.head_dim != 64 && c.head_dim != 128) return false;
  if (c.n_q_heads % c.n_kv_heads != 0) return false;
  if (c.d_model % 256 || (c.n_q_heads * c.head_dim) % 256 || c.d_ff % 256 || c.vocab % kColGroup) return false;
  if ((c.n_kv_heads * c.head_dim) % 64) return false;
  if (c.act != 0 && c.act != 1) return false;
  if (c.weight_fmt != 0 && c.weight_fmt != 1) return false;
  if (c.weight_fmt == 1 && (c.d_model % 512 || (c.n_q_heads * c.head_dim) % 512 || c.d_ff % 512)) return false;
  if (c.page_size != kPage || c.max_ctx < kPage || c.max_ctx % kPage) return false;
  if (c.max_k < 0 || c.max_k > kMaxRows - 1) return false;
  if (c.max_prefill_rows != 0 && (c.max_prefill_rows <= kMaxRows || c.max_prefill_rows > kMaxPrefillRows)) return false;
  if (!(c.rms_eps > 0.f) || !(c.rope_theta > 1.f)) return false;
  return true;
}

struct Plans {
  GemmPlan qkv, o, gu, d, lm;
};

// Persistent workgroups per GEMM: per_cu per compute unit, never more than
// there are 16-output items.  A GEMM workgroup holds a whole CU's worth of
// waves and LDS, so the layer GEMMs take one per CU; the LM head's many
// items take two.  Any grid gives the same bits.
int grid_for(int N, int per_cu, int n_cu) { return std::max(1, std::min(N / 16, per_cu * n_cu)); }

Plans make_plans(const sv_config& c, int n_cu) {
  const int qd = c.n_q_heads * c.head_dim, kd = c.n_kv_heads * c.head_dim;
  const bool i4 = c.weight_fmt == 1;
  const int unit = i4 ? 128 : 32;
  // int4 chunks are 128 inputs wide: at most 12 waves keeps a one-chunk-per-wave
  // activation stage small enough for 22 rows
  const int maxw = i4 ? 12 : 16;
  Plans p;
  p.qkv = {qd + 2 * kd, c.d_model, choose_waves(c.d_model, unit, maxw), c.weight_fmt};
  p.o = {c.d_model, qd, choose_waves(qd, unit, maxw), c.weight_fmt};
  p.gu = {2 * c.d_ff, c.d_model, choose_waves(c.d_model, unit, maxw), c.weight_fmt};
  p.d = {c.d_model, c.d_ff, choose_waves(c.d_ff, unit, maxw), c.weight_fmt};
  p.lm = {c.vocab, c.d_model, choose_waves(c.d_model, 32, 16), 0};
  for (GemmPlan* g : {&p.qkv, &p.o, &p.gu, &p.d}) g->grid = grid_for(g->N, 1, n_cu);
  p.lm.grid = grid_for(p.lm.N, 2, n_cu);
  return p;
}

// Rows one forward may carry: at most 64, at most kAttnQRows (row, q head)
// pairs of one KV head in the attention workgroup, and no more than every
// GEMM can stage in LDS.
int max_rows(const sv_config& c, const Plans& p) {
  int m = std::min(kMaxRows, kAttnQRows / (c.n_q_heads / c.n_kv_heads));
  for (const GemmPlan* g : {&p.qkv, &p.o, &p.gu, &p.d, &p.lm})
    if (g->S > 0) m = std::min(m, gemm_max_rows(g->fmt == 1 ? 128 : 32, g->S));
  return m;
}

bool plans_ok(const sv_config& c, const Plans& p) {
  for (const GemmPlan* g : {&p.qkv, &p.o, &p.gu, &p.d, &p.lm})
    if (g->S < 1) return false;
  return c.max_k + 1 <= max_rows(c, p);
}

constexpr int kMaxSelected = 4096;   // ids of one selected-logit read

// Kernel roles the profiler can time (sv_set_profile).
constexpr int kProfRoles = 6;
constexpr int kRoleAttn = 5;
// One (start, end) slot per profiled launch of a forward: role r of layer l
// (the LM head uses layer 0).
int prof_pairs(const sv_config& c) { return kProfRoles * c.n_layers; }

Layout make_layout(const sv_config& c, const Plans& p) {
  Layout L;
  L.rows = std::max(kMaxRows, (int)c.max_prefill_rows);
  const size_t R = L.rows;
  const int qd = c.n_q_heads * c.head_dim;
  // most splits any row of this context can have: one block per split up to
  // kAttnMaxSplits blocks, never more than kAttnMaxSplits
  L.max_split = std::min((c.max_ctx + kAttnBlock - 1) / kAttnBlock, kAttnMaxSplits);
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off = align_up(off + bytes, 256);
    return o;
  };
  L.params = take(sizeof(int) * (2 + R));
  // batched forward tables (one host-to-device copy with the params)
  const int G = c.n_q_heads / c.n_kv_heads;
  L.max_tiles = (int)((R * G + 15) / 16) + kMaxBatch;
  L.batch_bytes = R * 4 + kMaxBatch * sizeof(SeqDev) + (size_t)L.max_tiles * 8;
  L.batch = take(L.batch_bytes);
  L.x = take(R * c.d_model * 4);
  L.ss = take(R * (c.d_model / 16) * 4);
  L.q = take(R * qd * 4);
  // split partials: only forwards of at most 64 rows use the split kernels
  L.attn_part = take((size_t)kMaxRows * c.n_q_heads * (size_t)L.max_split * (c.head_dim + 4) * 4);
  L.uplanes = take(2 * R * c.d_model * 2);   // hi, lo planes of x * g (RMSNorm consumers' input)
  L.oplanes = take(2 * R * qd * 2);          // attention output
  L.aplanes = take(2 * R * c.d_ff * 2);      // act(gate) * up
  L.best = take(R * 8);
  L.logits = take(R * (size_t)c.vocab * 4);
  L.rope = take((size_t)c.max_ctx * (c.head_dim / 2) * 8);
  L.prof = take(prof_pairs(c) * 16);
  L.topk = take((size_t)(kTopkBlocks + 1) * kTopkMax * 8);
  L.sel = take((size_t)kMaxSelected * 8);
  L.total = off;
  return L;
}

size_t kv_pool_bytes_for(const sv_config& c, int n_pages) {
  return (size_t)c.n_layers * n_pages * 2 * c.n_kv_heads * kPage * c.head_dim * 2;
}

}  // namespace

// Intermediates of sv_verify_noalloc: one array per GPU, held until the
// process ends.  In host code `scratch` names a host-side stand-in, not
// device memory: its device address on each GPU comes from
// hipGetSymbolAddress (scratch_address below), and only that address is
// ever handed to a kernel.  Every sv_verify_noalloc call on a GPU uses that
// GPU's one copy, so calls that overlap in time on one GPU race.
constexpr size_t kScratchBytes = size_t(32) << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_addr[kMaxDevices] = {};

// Device address of `scratch` on GPU `dev`, which must be the current
// device; looked up once per device and kept.
sv_status scratch_address(int dev, void** out) {
  if (dev < 0 || dev >= kMaxDevices) return SV_EDEVICE;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_addr[dev] == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return SV_EDEVICE;
    g_scratch_addr[dev] = p;
  }
  *out = g_scratch_addr[dev];
  return SV_OK;
}
}  // namespace

struct sv_ctx {
  sv_config cfg{};
  sv_weights w{};
  std::vector<sv_layer_weights> layers;
  sv_buffers buf{};
  hipStream_t stream = nullptr;
  Plans plans;
  Layout lay;
  char* ws = nullptr;
  int* h_params = nullptr;   // pinned, coherent: k_embed reads it over the bus (device address hd_params)
  int* h_result = nullptr;   // pinned, coherent: k_accept writes it over the bus (device address hd_result)
  int* hd_params = nullptr;
  int* hd_result = nullptr;
  void* scratch = nullptr;   // device address of this GPU's copy of `scratch` (sv_verify_noalloc)
  char* h_batch = nullptr;   // pinned staging of the batched-forward tables
  unsigned long long* h_prof = nullptr;   // pinned copy of the profiling slots
  int kv_len = 0;
  int next_id = -1;
  std::vector<int> hist;     // hist[p] = greedy id after positions 0..p
  int store_logits = 0;
  int last_rows = 0;
  int last_stored_logits = 0;
  std::vector<int> last_argmax;   // [lay.rows]
  // profiling: wall-clock spans of the enabled kernel roles
  int prof_mask = 0;
  double wall_khz = 0.0;               // device wall-clock rate
  int n_cu = 0;                        // compute units of the device
  double prof_ms[kProfRoles] = {};
  int64_t prof_n[kProfRoles] = {};

  // HIP graphs of whole forwards, keyed by (rows, attention splits, mode,
  // logits, profile mask, batch sequences, batch q tiles, the split
  // kernel's blocks-per-split guess)
  hipStream_t cap_stream = nullptr;
  bool use_graphs = true;
  std::map<std::array<int, 8>, hipGraphExec_t> graphs;

  template <class T>
  T* at(size_t off) { return reinterpret_cast<T*>(ws + off); }
};

namespace {

// Device buffers one forward computes in: the per-forward intermediates
// (params copy, residual, sums of squares, q, attention partials, activation
// planes, row argmax keys), the optional logits output, the profiling slots
// and the RoPE table.  R is the row stride of the plane buffers (lo plane =
// hi plane + R rows).
struct FwdBufs {
  int R = 0;
  int* params = nullptr;
  float *x = nullptr, *ss = nullptr, *q = nullptr, *part = nullptr, *logits = nullptr;
  int part_splits = 0;
  uint16_t *uplanes = nullptr, *oplanes = nullptr, *aplanes = nullptr;
  unsigned long long *best = nullptr, *prof = nullptr;
  const float2* rope = nullptr;
};

// The context's workspace (every forward of sv_prefill, sv_decode_step,
// sv_verify and sv_verify_batch).
FwdBufs ws_bufs(sv_ctx* c) {
  FwdBufs b;
  b.R = c->lay.rows;
  b.params = c->at<int>(c->lay.params);
  b.x = c->at<float>(c->lay.x);
  b.ss = c->at<float>(c->lay.ss);
  b.q = c->at<float>(c->lay.q);
  b.part = c->at<float>(c->lay.attn_part);
  b.part_splits = c->lay.max_split;
  b.uplanes = c->at<uint16_t>(c->lay.uplanes);
  b.oplanes = c->at<uint16_t>(c->lay.oplanes);
  b.aplanes = c->at<uint16_t>(c->lay.aplanes);
  b.best = c->at<unsigned long long>(c->lay.best);
  b.logits = c->at<float>(c->lay.logits);
  b.prof = c->at<unsigned long long>(c->lay.prof);
  b.rope = c->at<const float2>(c->lay.rope);
  return b;
}

// sv_verify_noalloc: the per-forward intermediates of M rows whose attention
// runs n_split splits, carved from `base` (this GPU's scratch address; null
// only sizes them); the observer logits (an output) and the RoPE table (an
// input built by sv_create) stay in the context's workspace, and nothing is
// profiled.  Returns the bytes the intermediates take.
size_t scratch_bufs(sv_ctx* c, char* base, int M, int n_split, FwdBufs* out) {
  const sv_config& cfg = c->cfg;
  const size_t qd = (size_t)cfg.n_q_heads * cfg.head_dim;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    char* p = base == nullptr ? nullptr : base + off;
    off = align_up(off + bytes, 256);
    return p;
  };
  FwdBufs b;
  b.R = M;
  b.params = reinterpret_cast<int*>(take(sizeof(int) * (2 + (size_t)M)));
  b.x = reinterpret_cast<float*>(take((size_t)M * cfg.d_model * 4));
  b.ss = reinterpret_cast<float*>(take((size_t)M * (cfg.d_model / 16) * 4));
  b.q = reinterpret_cast<float*>(take((size_t)M * qd * 4));
  b.part_splits = std::max(n_split, 1);
  b.part = reinterpret_cast<float*>(take((size_t)M * cfg.n_q_heads * b.part_splits * (cfg.head_dim + 4) * 4));
  b.uplanes = reinterpret_cast<uint16_t*>(take(2 * (size_t)M * cfg.d_model * 2));
  b.oplanes = reinterpret_cast<uint16_t*>(take(2 * (size_t)M * qd * 2));
  b.aplanes = reinterpret_cast<uint16_t*>(take(2 * (size_t)M * cfg.d_ff * 2));
  b.best = reinterpret_cast<unsigned long long*>(take((size_t)M * 8));
  b.logits = c->at<float>(c->lay.logits);
  b.prof = nullptr;
  b.rope = c->at<const float2>(c->lay.rope);
  if (out) *out = b;
  return off;
}

// Profiling slot of (role, layer) when that role is enabled, else null.
unsigned long long* prof_slot(sv_ctx* c, const FwdBufs& fb, int role, int layer) {
  if (fb.prof == nullptr || !(c->prof_mask & (1 << role))) return nullptr;
  return fb.prof + 2 * ((size_t)role * c->cfg.n_layers + layer);
}

// Add the spans of the last forward's timed launches (slots copied to host).
void prof_accumulate(sv_ctx* c) {
  const int L = c->cfg.n_layers;
  for (int role = 0; role < kProfRoles; ++role) {
    if (!(c->prof_mask & (1 << role))) continue;
    for (int l = 0; l < L; ++l) {
      const unsigned long long s = c->h_prof[2 * (role * L + l)], e = c->h_prof[2 * (role * L + l) + 1];
      if (e == 0 || e < s) continue;   // launch not in this forward
      c->prof_ms[role] += (double)(e - s) / c->wall_khz;
      c->prof_n[role] += 1;
    }
  }
}

// tiled: forwards of more than 64 rows run the row-tiled kernels (the same
// per-row arithmetic as the weight-streaming ones).
hipError_t gemm_timed(sv_ctx* c, const FwdBufs& fb, GemmArgs& g, int role, int grid, hipStream_t st, bool tiled) {
  g.prof = prof_slot(c, fb, role, g.layer);
  const hipError_t e = tiled ? launch_gemm_tiled(g, role, st) : launch_gemm(g, role, grid, st);
  g.prof = nullptr;
  return e;
}

// Queue one whole forward of M rows (kernels only) on `st`.
// Device tables of a batched forward (all null / 0 for one sequence).
struct BatchDev {
  const SeqDev* seqs = nullptr;
  const int* rowseq = nullptr;
  const int2* tiles = nullptr;
  int n_seq = 0, n_tiles = 0;
};

BatchDev batch_dev(sv_ctx* c, int n_seq, int n_tiles) {
  BatchDev b;
  if (n_seq == 0) return b;
  char* base = c->at<char>(c->lay.batch);
  b.rowseq = reinterpret_cast<const int*>(base);
  b.seqs = reinterpret_cast<const SeqDev*>(base + (size_t)c->lay.rows * 4);
  b.tiles = reinterpret_cast<const int2*>(base + (size_t)c->lay.rows * 4 + kMaxBatch * sizeof(SeqDev));
  b.n_seq = n_seq;
  b.n_tiles = n_tiles;
  return b;
}

hipError_t enqueue_forward(sv_ctx* c, const FwdBufs& fb, int M, int verify, int n_split, int logits,
                           const BatchDev& bd, hipStream_t st) {
  const sv_config& cfg = c->cfg;
  const bool tiled = M > kMaxRows;
  const int R = fb.R;
  const int qd = cfg.n_q_heads * cfg.head_dim;
  int* d_params = fb.params;
  float* x = fb.x;
  float* ss = fb.ss;
  float* q = fb.q;
  uint16_t* uhi = fb.uplanes;
  uint16_t* ulo = uhi + (size_t)R * cfg.d_model;
  uint16_t* ohi = fb.oplanes;
  uint16_t* olo = ohi + (size_t)R * qd;
  uint16_t* ahi = fb.aplanes;
  uint16_t* alo = ahi + (size_t)R * cfg.d_ff;
  uint16_t* kv = static_cast<uint16_t*>(c->buf.kv_pool);
  auto gain = [](const void* p) { return static_cast<const uint16_t*>(p); };

  hipError_t e = hipSuccess;
  if (c->prof_mask != 0 && fb.prof != nullptr &&
      (e = launch_prof_reset(fb.prof, prof_pairs(cfg), st)) != hipSuccess)
    return e;
  unsigned long long* best = fb.best;
  e = launch_embed(c->hd_params, d_params, M, c->w.embed, cfg.vocab, cfg.d_model, x, ss, gain(c->layers[0].g_attn), uhi,
                   ulo, best, st);
  if (e != hipSuccess) return e;

  GemmArgs g{};
  g.M = M;
  g.eps = cfg.rms_eps;
  g.params = d_params;
  g.ss = ss;
  g.x = x;
  g.ss_out = ss;
  g.uhi = uhi;
  g.ulo = ulo;
  g.ahi = ahi;
  g.alo = alo;
  g.act = cfg.act;
  g.q_out = q;
  g.kv_pool = kv;
  g.page_table = c->buf.page_table;
  g.n_pages = c->buf.n_pages;
  g.nq = cfg.n_q_heads;
  g.nkv = cfg.n_kv_heads;
  g.dh = cfg.head_dim;
  g.rope = fb.rope;
  g.seqs = bd.seqs;
  g.rowseq = bd.rowseq;
  auto plan = [&](const GemmPlan& p, const void* W, const void* Ws, const uint16_t* bhi, const uint16_t* blo) {
    g.W = W; g.Wscale = Ws; g.N = p.N; g.K = p.K; g.S = p.S; g.fmt = p.fmt; g.bhi = bhi; g.blo = blo;
  };

  for (int l = 0; l < cfg.n_layers; ++l) {
    const sv_layer_weights& L = c->layers[l];
    g.layer = l;
    // attention block: (norm) QKV + RoPE + KV append, attention, O + residual
    plan(c->plans.qkv, L.wqkv, L.wqkv_scales, uhi, ulo);
    if ((e = gemm_timed(c, fb, g, kRoleQkv, c->plans.qkv.grid, st, tiled)) != hipSuccess) return e;
    AttnArgs at{};
    at.params = d_params; at.q = q; at.kv_pool = kv; at.page_table = c->buf.page_table; at.n_pages = c->buf.n_pages;
    at.layer = l; at.nq = cfg.n_q_heads; at.nkv = cfg.n_kv_heads; at.dh = cfg.head_dim; at.M = M;
    at.n_split = n_split; at.n_lpages = cfg.max_ctx / kPage; at.scale_log2 = (float)(1.4426950408889634 / std::sqrt((double)cfg.head_dim));
    at.part = fb.part; at.part_splits = fb.part_splits; at.ohi = ohi; at.olo = olo;
    at.prof = prof_slot(c, fb, kRoleAttn, l);
    at.seqs = bd.seqs; at.rowseq = bd.rowseq; at.tiles = bd.tiles; at.n_tiles = bd.n_tiles;
    at.bps_guess = bd.seqs != nullptr ? 1 : attn_blocks_per_split(c->kv_len + 1);
    at.n_simd = 4 * c->n_cu;
    if ((e = tiled ? launch_attention_rows(at, st) : launch_attention(at, st)) != hipSuccess) return e;
    plan(c->plans.o, L.wo, L.wo_scales, ohi, olo);
    g.gnext = gain(L.g_mlp);
    if ((e = gemm_timed(c, fb, g, kRoleO, c->plans.o.grid, st, tiled)) != hipSuccess) return e;
    // MLP block: (norm) gate/up + activation, down + residual
    plan(c->plans.gu, L.wgu, L.wgu_scales, uhi, ulo);
    if ((e = gemm_timed(c, fb, g, kRoleGateUp, c->plans.gu.grid, st, tiled)) != hipSuccess) return e;
    plan(c->plans.d, L.wd, L.wd_scales, ahi, alo);
    g.gnext = l + 1 < cfg.n_layers ? gain(c->layers[l + 1].g_attn) : gain(c->w.g_final);
    if ((e = gemm_timed(c, fb, g, kRoleDown, c->plans.d.grid, st, tiled)) != hipSuccess) return e;
  }

  // (final norm) LM head + per-16-column argmax, then acceptance
  plan(c->plans.lm, c->w.lm_head, nullptr, uhi, ulo);
  g.layer = 0;
  g.best = best;
  g.logits = logits ? fb.logits : nullptr;
  if ((e = gemm_timed(c, fb, g, kRoleLmHead, c->plans.lm.grid, st, tiled)) != hipSuccess) return e;
  if (bd.seqs != nullptr) return launch_accept_batch(d_params, M, bd.seqs, bd.n_seq, best, c->hd_result, st);
  return launch_accept(d_params, M, verify, best, c->hd_result, st);
}

// One forward of M rows on c's stream: the params go into the pinned buffer
// the first kernel reads (and, for a batched forward of n_seq > 0 sequences,
// the tables the caller staged in h_batch go up), the kernels run (a cached
// HIP graph for up to 64 rows) and write the result [n, next, a_0 .. a_{M-1},
// (n_s, next_s) per sequence] into pinned memory, and the profiling slots
// come back.  No copy kernel runs for the params or the result.  kv_len: the
// params' length (one sequence).  The buffers are rewritten only after the
// previous forward's synchronisation, so no forward reads another's params.
sv_status run_forward(sv_ctx* c, int M, const int* ids, int verify, int n_split, int n_seq, int n_tiles, int logits) {
  hipStream_t st = c->stream;
  c->h_params[0] = c->kv_len;
  c->h_params[1] = M;
  std::memcpy(c->h_params + 2, ids, sizeof(int) * M);
  if (n_seq > 0 && hipMemcpyAsync(c->at<char>(c->lay.batch), c->h_batch, c->lay.batch_bytes, hipMemcpyHostToDevice,
                                  st) != hipSuccess)
    return SV_EDEVICE;
  const BatchDev bd = batch_dev(c, n_seq, n_tiles);

  const FwdBufs fb = ws_bufs(c);
  if (c->use_graphs && M <= kMaxRows) {   // forwards of many rows take milliseconds: launched directly
    // (the guess is a kernel argument: a graph captured at one blocks-per-split
    // would otherwise replay it at another, correct but reloading every unit)
    const int bps_guess = n_seq > 0 ? 1 : attn_blocks_per_split(c->kv_len + 1);
    const std::array<int, 8> key = {M, n_split, verify, logits, c->prof_mask, n_seq, n_tiles, bps_guess};
    auto it = c->graphs.find(key);
    if (it == c->graphs.end()) {
      hipGraph_t graph = nullptr;
      hipGraphExec_t exec = nullptr;
      if (hipStreamBeginCapture(c->cap_stream, hipStreamCaptureModeThreadLocal) != hipSuccess) return SV_EDEVICE;
      const hipError_t e = enqueue_forward(c, fb, M, verify, n_split, logits, bd, c->cap_stream);
      const hipError_t e2 = hipStreamEndCapture(c->cap_stream, &graph);
      hipError_t e3 = hipErrorUnknown;
      if (e == hipSuccess && e2 == hipSuccess && graph != nullptr) e3 = hipGraphInstantiate(&exec, graph, nullptr, nullptr, 0);
      if (graph) (void)hipGraphDestroy(graph);
      if (e3 != hipSuccess) return SV_EDEVICE;
      it = c->graphs.emplace(key, exec).first;
    }
    if (hipGraphLaunch(it->second, st) != hipSuccess) return SV_EDEVICE;
  } else {
    if (enqueue_forward(c, fb, M, verify, n_split, logits, bd, st) != hipSuccess) return SV_EDEVICE;
  }
  if (c->prof_mask != 0 && hipMemcpyAsync(c->h_prof, c->at<unsigned long long>(c->lay.prof),
                                          16 * (size_t)prof_pairs(c->cfg), hipMemcpyDeviceToHost, st) != hipSuccess)
    return SV_EDEVICE;
  if (hipStreamSynchronize(st) != hipSuccess) return SV_EDEVICE;
  if (c->prof_mask != 0) prof_accumulate(c);
  return SV_OK;
}

// sv_verify_noalloc's forward: the same kernels, launched directly (no HIP
// graph is instantiated) with the intermediates in this GPU's scratch array
// (the caller has checked that they fit).  The row argmax keys there are
// cleared by the first kernel; every other intermediate is written before
// it is read, so nothing a previous call left behind is used.
sv_status run_forward_noalloc(sv_ctx* c, int M, const int* ids, int n_split, int logits) {
  hipStream_t st = c->stream;
  c->h_params[0] = c->kv_len;
  c->h_params[1] = M;
  std::memcpy(c->h_params + 2, ids, sizeof(int) * M);
  FwdBufs fb;
  scratch_bufs(c, static_cast<char*>(c->scratch), M, n_split, &fb);
  if (enqueue_forward(c, fb, M, 1, n_split, logits, BatchDev{}, st) != hipSuccess) return SV_EDEVICE;
  if (hipStreamSynchronize(st) != hipSuccess) return SV_EDEVICE;
  return SV_OK;
}

sv_status forward(sv_ctx* c, int M, const int* ids, int verify, bool noalloc = false) {
  const int n_split = attn_splits_max(c->kv_len, M);
  const sv_status s = noalloc ? run_forward_noalloc(c, M, ids, n_split, c->store_logits)
                              : run_forward(c, M, ids, verify, n_split, 0, 0, c->store_logits);
  if (s != SV_OK) return s;
  c->last_rows = M;
  c->last_stored_logits = c->store_logits;
  for (int r = 0; r < M; ++r) c->last_argmax[r] = c->h_result[2 + r];
  return SV_OK;
}

bool ids_ok(const sv_ctx* c, const int32_t* ids, int n) {
  for (int i = 0; i < n; ++i)
    if (ids[i] < 0 || ids[i] >= c->cfg.vocab) return false;
  return true;
}

sv_status verify_impl(sv_ctx* c, int32_t prefix_len, const int32_t* draft_ids, int32_t k, int32_t* n_accepted,
                      int32_t* next_id, bool noalloc) {
  if (!c) return SV_EINVAL;
  if (k < 0 || k > c->cfg.max_k || (k > 0 && !draft_ids)) return SV_EINVAL;
  if (prefix_len != c->kv_len || c->next_id < 0) return SV_ESTATE;
  if (k > 0 && !ids_ok(c, draft_ids, k)) return SV_EINVAL;
  if ((int64_t)c->kv_len + k + 1 > c->cfg.max_ctx) return SV_ENOSPACE;
  if (noalloc) {
    if (c->scratch == nullptr) return SV_EDEVICE;
    if (scratch_bufs(c, nullptr, k + 1, attn_splits_max(c->kv_len, k + 1), nullptr) > kScratchBytes)
      return SV_ESCRATCH;
  }
  int rows[kMaxRows];
  rows[0] = c->next_id;
  for (int i = 0; i < k; ++i) rows[1 + i] = draft_ids[i];
  const sv_status s = forward(c, k + 1, rows, 1, noalloc);
  if (s != SV_OK) return s;
  const int n = c->h_result[0];
  for (int r = 0; r <= n; ++r) c->hist[c->kv_len + r] = c->h_result[2 + r];
  c->kv_len += n + 1;
  c->next_id = c->h_result[1];
  if (n_accepted) *n_accepted = n;
  if (next_id) *next_id = c->next_id;
  return SV_OK;
}


}  // namespace

extern "C" {

const char* sv_status_str(sv_status s) {
  switch (s) {
    case SV_OK: return "ok";
    case SV_EINVAL: return "invalid argument";
    case SV_ESTATE: return "call does not match context state";
    case SV_ENOSPACE: return "KV capacity exceeded";
    case SV_EDEVICE: return "HIP device error";
    case SV_EUNSUPPORTED: return "unsupported configuration";
    case SV_ESCRATCH: return "intermediates exceed the library's static scratch array";
  }
  return "unknown status";
}

sv_status sv_query_sizes(const sv_config* cfg, int64_t* kv_pool_bytes, int64_t* workspace_bytes) {
  if (!cfg || !valid_config(*cfg)) return SV_EINVAL;
  const Plans p = make_plans(*cfg, 256);
  if (!plans_ok(*cfg, p)) return SV_EUNSUPPORTED;
  const Layout L = make_layout(*cfg, p);
  if (kv_pool_bytes) *kv_pool_bytes = (int64_t)kv_pool_bytes_for(*cfg, cfg->max_ctx / kPage);
  if (workspace_bytes) *workspace_bytes = (int64_t)L.total;
  return SV_OK;
}

sv_status sv_packed_linear_bytes(int32_t fmt, int32_t n, int32_t k, int64_t* bytes, int64_t* scale_bytes) {
  if (n <= 0 || k <= 0 || n % 16) return SV_EINVAL;
  if (fmt == 0) {
    if (k % 32) return SV_EINVAL;
    if (bytes) *bytes = (int64_t)n * k * 2;
    if (scale_bytes) *scale_bytes = 0;
    return SV_OK;
  }
  if (fmt == 1) {
    if (k % 128) return SV_EINVAL;
    if (bytes) *bytes = (int64_t)n * k / 2;
    if (scale_bytes) *scale_bytes = (int64_t)n * (k / 64) * 2;
    return SV_OK;
  }
  return SV_EINVAL;
}

sv_status sv_pack_linear(int32_t fmt, int32_t layout, const void* src0, const void* src0_scales, const void* src1,
                         const void* src1_scales, int32_t n, int32_t k, int32_t head_dim, void* dst, void* dst_scales,
                         void* stream) {
  if (!src0 || !dst) return SV_EINVAL;
  if (sv_packed_linear_bytes(fmt, n, k, nullptr, nullptr) != SV_OK) return SV_EINVAL;
  if (fmt == 1 && (!src0_scales || !dst_scales || (src1 && !src1_scales))) return SV_EINVAL;
  if (layout < 0 || layout > 2) return SV_EINVAL;
  if ((layout == 1) != (src1 != nullptr)) return SV_EINVAL;
  if (layout == 2 && ((head_dim != 64 && head_dim != 128) || n % head_dim)) return SV_EINVAL;
  if (launch_pack(fmt, layout, src0, src0_scales, src1, src1_scales, n, k, head_dim, dst, dst_scales,
                  (hipStream_t)stream) != hipSuccess)
    return SV_EDEVICE;
  return SV_OK;
}

sv_status sv_create(const sv_config* cfg, const sv_weights* w, const sv_buffers* buf, void* stream, sv_ctx** out) {
  if (!out) return SV_EINVAL;
  *out = nullptr;
  if (!cfg || !w || !buf || !valid_config(*cfg)) return SV_EINVAL;
  if (!w->embed || !w->lm_head || !w->g_final || !w->layers) return SV_EINVAL;
  for (int l = 0; l < cfg->n_layers; ++l) {
    const sv_layer_weights& L = w->layers[l];
    if (!L.wqkv || !L.wo || !L.wgu || !L.wd || !L.g_attn || !L.g_mlp) return SV_EINVAL;
    if (cfg->weight_fmt == 1 && (!L.wqkv_scales || !L.wo_scales || !L.wgu_scales || !L.wd_scales)) return SV_EINVAL;
  }
  int dev = 0, n_cu = 0, wall_khz = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&n_cu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n_cu < 1 ||
      hipDeviceGetAttribute(&wall_khz, hipDeviceAttributeWallClockRate, dev) != hipSuccess || wall_khz < 1)
    return SV_EDEVICE;
  const Plans p = make_plans(*cfg, n_cu);
  if (!plans_ok(*cfg, p)) return SV_EUNSUPPORTED;
  const Layout lay = make_layout(*cfg, p);
  void* scratch_addr = nullptr;
  if (scratch_address(dev, &scratch_addr) != SV_OK) return SV_EDEVICE;
  if (!buf->kv_pool || !buf->page_table || !buf->workspace) return SV_EINVAL;
  if (reinterpret_cast<uintptr_t>(buf->page_table) % 16 != 0) return SV_EINVAL;   // read 4 entries at a time
  if (buf->n_pages < 1 || buf->kv_pool_bytes < (int64_t)kv_pool_bytes_for(*cfg, buf->n_pages)) return SV_EINVAL;
  if (buf->workspace_bytes < (int64_t)lay.total) return SV_EINVAL;
  // Every logical page must map into the pool: a bad entry would address
  // memory outside it.
  const int n_logical = cfg->max_ctx / kPage;
  std::vector<int32_t> pt(n_logical);
  if (hipMemcpy(pt.data(), buf->page_table, sizeof(int32_t) * n_logical, hipMemcpyDeviceToHost) != hipSuccess)
    return SV_EDEVICE;
  for (int32_t v : pt)
    if (v < 0 || v >= buf->n_pages) return SV_EINVAL;

  sv_ctx* c = new (std::nothrow) sv_ctx();
  if (!c) return SV_EDEVICE;
  c->cfg = *cfg;
  c->layers.assign(w->layers, w->layers + cfg->n_layers);
  c->w = *w;
  c->w.layers = c->layers.data();
  c->buf = *buf;
  c->stream = (hipStream_t)stream;
  c->plans = p;
  c->lay = lay;
  c->wall_khz = wall_khz;
  c->n_cu = n_cu;
  c->ws = static_cast<char*>(buf->workspace);
  c->scratch = scratch_addr;
  c->hist.assign(cfg->max_ctx, -1);
  c->last_argmax.assign(lay.rows, 0);
  const unsigned mapped = hipHostMallocMapped | hipHostMallocCoherent;
  if (hipHostMalloc((void**)&c->h_params, sizeof(int) * (2 + lay.rows), mapped) != hipSuccess ||
      hipHostMalloc((void**)&c->h_result, sizeof(int) * (2 + lay.rows + 2 * kMaxBatch), mapped) != hipSuccess ||
      hipHostGetDevicePointer((void**)&c->hd_params, c->h_params, 0) != hipSuccess ||
      hipHostGetDevicePointer((void**)&c->hd_result, c->h_result, 0) != hipSuccess ||
      hipHostMalloc((void**)&c->h_batch, lay.batch_bytes, hipHostMallocDefault) != hipSuccess ||
      hipHostMalloc((void**)&c->h_prof, 16 * (size_t)prof_pairs(*cfg), hipHostMallocDefault) != hipSuccess) {
    sv_destroy(c);
    return SV_EDEVICE;
  }
  // RoPE table: angle pos * theta^(-2i/dh) in double, cos/sin rounded once to float.
  const int half = cfg->head_dim / 2;
  std::vector<float> tab((size_t)cfg->max_ctx * half * 2);
  for (int pos = 0; pos < cfg->max_ctx; ++pos)
    for (int i = 0; i < half; ++i) {
      const double ang = (double)pos * std::pow((double)cfg->rope_theta, -2.0 * i / cfg->head_dim);
      tab[((size_t)pos * half + i) * 2 + 0] = (float)std::cos(ang);
      tab[((size_t)pos * half + i) * 2 + 1] = (float)std::sin(ang);
    }
  const char* ng = std::getenv("SV_NO_GRAPH");
  c->use_graphs = !(ng && ng[0] == '1');
  if (hipStreamCreateWithFlags(&c->cap_stream, hipStreamNonBlocking) != hipSuccess) {
    c->cap_stream = nullptr;
    sv_destroy(c);
    return SV_EDEVICE;
  }
  if (hipMemcpyAsync(c->ws + lay.rope, tab.data(), tab.size() * 4, hipMemcpyHostToDevice, c->stream) != hipSuccess ||
      hipStreamSynchronize(c->stream) != hipSuccess) {
    sv_destroy(c);
    return SV_EDEVICE;
  }
  *out = c;
  return SV_OK;
}

void sv_destroy(sv_ctx* c) {
  if (!c) return;
  for (auto& kv : c->graphs) (void)hipGraphExecDestroy(kv.second);
  if (c->cap_stream) (void)hipStreamDestroy(c->cap_stream);
  if (c->h_params) (void)hipHostFree(c->h_params);
  if (c->h_result) (void)hipHostFree(c->h_result);
  if (c->h_batch) (void)hipHostFree(c->h_batch);
  if (c->h_prof) (void)hipHostFree(c->h_prof);
  delete c;
}

int32_t sv_kv_len(const sv_ctx* c) { return c ? c->kv_len : -1; }
int32_t sv_next_id(const sv_ctx* c) { return c ? c->next_id : -1; }

sv_status sv_prefill(sv_ctx* c, const int32_t* ids, int32_t n, int32_t* next_id) {
  if (!c || !ids || n < 1) return SV_EINVAL;
  if (!ids_ok(c, ids, n)) return SV_EINVAL;
  if ((int64_t)c->kv_len + n > c->cfg.max_ctx) return SV_ENOSPACE;
  // forwards of up to max_prefill_rows rows (row-tiled kernels) while more
  // than 64 ids remain, then of up to 64 (weight-streaming kernels); every
  // row's bits are the same either way
  const int small = max_rows(c->cfg, c->plans);
  for (int off = 0; off < n;) {
    const int left = n - off;
    const int m = (c->cfg.max_prefill_rows > 0 && left > small) ? std::min(left, (int)c->cfg.max_prefill_rows)
                                                                : std::min(left, small);
    const sv_status s = forward(c, m, ids + off, 0);
    if (s != SV_OK) return s;
    for (int r = 0; r < m; ++r) c->hist[c->kv_len + r] = c->h_result[2 + r];
    c->kv_len += m;
    c->next_id = c->h_result[1];
    off += m;
  }
  if (next_id) *next_id = c->next_id;
  return SV_OK;
}

sv_status sv_decode_step(sv_ctx* c, int32_t token, int32_t* next_id) {
  if (!c) return SV_EINVAL;
  if (!ids_ok(c, &token, 1)) return SV_EINVAL;
  if (c->kv_len + 1 > c->cfg.max_ctx) return SV_ENOSPACE;
  const sv_status s = forward(c, 1, &token, 1);
  if (s != SV_OK) return s;
  c->hist[c->kv_len] = c->h_result[2];
  c->kv_len += 1;
  c->next_id = c->h_result[1];
  if (next_id) *next_id = c->next_id;
  return SV_OK;
}

sv_status sv_verify(sv_ctx* c, int32_t prefix_len, const int32_t* draft_ids, int32_t k, int32_t* n_accepted,
                    int32_t* next_id) {
  return verify_impl(c, prefix_len, draft_ids, k, n_accepted, next_id, false);
}

sv_status sv_verify_noalloc(sv_ctx* c, int32_t prefix_len, const int32_t* draft_ids, int32_t k,
                            int32_t* n_accepted, int32_t* next_id) {
  return verify_impl(c, prefix_len, draft_ids, k, n_accepted, next_id, true);
}

sv_status sv_verify_batch(sv_ctx* const* ctxs, int32_t n, const int32_t* prefix_lens, const int32_t* ks,
                          const int32_t* draft_ids, int32_t* n_accepted, int32_t* next_ids) {
  if (!ctxs || n < 1 || n > kMaxBatch || !prefix_lens || !ks) return SV_EINVAL;
  sv_ctx* c0 = ctxs[0];
  if (!c0) return SV_EINVAL;
  // every argument is checked before anything runs
  int M = 0, n_drafts = 0;
  for (int i = 0; i < n; ++i) {
    const sv_ctx* c = ctxs[i];
    if (!c) return SV_EINVAL;
    for (int j = 0; j < i; ++j)
      if (ctxs[j] == c) return SV_EINVAL;
    sv_config a = c->cfg, b = c0->cfg;
    a.max_prefill_rows = b.max_prefill_rows = 0;
    if (std::memcmp(&a, &b, sizeof(sv_config)) != 0) return SV_EINVAL;
    if (c->w.embed != c0->w.embed || c->w.lm_head != c0->w.lm_head || c->w.g_final != c0->w.g_final ||
        std::memcmp(c->layers.data(), c0->layers.data(), sizeof(sv_layer_weights) * c0->layers.size()) != 0)
      return SV_EINVAL;
    if (ks[i] < 0 || ks[i] > c->cfg.max_k || (ks[i] > 0 && !draft_ids)) return SV_EINVAL;
    if (ks[i] > 0 && !ids_ok(c, draft_ids + n_drafts, ks[i])) return SV_EINVAL;
    if (prefix_lens[i] != c->kv_len || c->next_id < 0) return SV_ESTATE;
    if ((int64_t)c->kv_len + ks[i] + 1 > c->cfg.max_ctx) return SV_ENOSPACE;
    M += ks[i] + 1;
    n_drafts += ks[i];
  }
  if (M > c0->lay.rows) return SV_EINVAL;

  // rows, their sequences, the sequence table and the attention q tiles
  std::vector<int> rows(M);
  int* rowseq = reinterpret_cast<int*>(c0->h_batch);
  SeqDev* seqs = reinterpret_cast<SeqDev*>(c0->h_batch + (size_t)c0->lay.rows * 4);
  int2* tiles = reinterpret_cast<int2*>(c0->h_batch + (size_t)c0->lay.rows * 4 + kMaxBatch * sizeof(SeqDev));
  const int G = c0->cfg.n_q_heads / c0->cfg.n_kv_heads;
  int row = 0, d = 0, n_tiles = 0, n_split = 1, logits = 0;
  for (int i = 0; i < n; ++i) {
    sv_ctx* c = ctxs[i];
    const int m = ks[i] + 1;
    SeqDev sd{};
    sd.kv_pool = static_cast<uint16_t*>(c->buf.kv_pool);
    sd.page_table = c->buf.page_table;
    sd.n_pages = c->buf.n_pages;
    sd.n_lpages = c->cfg.max_ctx / kPage;
    sd.kv_len = c->kv_len;
    sd.row0 = row;
    sd.m = m;
    seqs[i] = sd;
    rows[row] = c->next_id;
    for (int j = 0; j < ks[i]; ++j) rows[row + 1 + j] = draft_ids[d + j];
    for (int j = 0; j < m; ++j) rowseq[row + j] = i;
    for (int q = 0; q < m * G; q += 16) tiles[n_tiles++] = make_int2(i, q);
    n_split = std::max(n_split, attn_splits_max(c->kv_len, m));
    logits |= c->store_logits;
    row += m;
    d += ks[i];
  }
  const sv_status s = run_forward(c0, M, rows.data(), 1, n_split, n, n_tiles, logits);
  if (s != SV_OK) return s;
  // commit each sequence as its own verify would; observer-mode contexts get
  // their rows' logits in their own workspace
  for (int i = 0; i < n; ++i) {
    sv_ctx* c = ctxs[i];
    const int r0 = seqs[i].row0, m = seqs[i].m;
    const int na = c0->h_result[2 + M + 2 * i], nx = c0->h_result[2 + M + 2 * i + 1];
    if (c->store_logits && c != c0 &&
        hipMemcpyAsync(c->at<float>(c->lay.logits), c0->at<float>(c0->lay.logits) + (size_t)r0 * c0->cfg.vocab,
                       sizeof(float) * (size_t)m * c0->cfg.vocab, hipMemcpyDeviceToDevice, c0->stream) != hipSuccess)
      return SV_EDEVICE;
    for (int r = 0; r < m; ++r) c->last_argmax[r] = c0->h_result[2 + r0 + r];
    for (int r = 0; r <= na; ++r) c->hist[c->kv_len + r] = c0->h_result[2 + r0 + r];
    c->kv_len += na + 1;
    c->next_id = nx;
    c->last_rows = m;
    c->last_stored_logits = c->store_logits;
    if (n_accepted) n_accepted[i] = na;
    if (next_ids) next_ids[i] = nx;
  }
  if (hipStreamSynchronize(c0->stream) != hipSuccess) return SV_EDEVICE;
  return SV_OK;
}

// ---- audit mode
sv_status sv_topk(sv_ctx* c, int32_t row, int32_t k, int32_t* ids, float* vals) {
  if (!c || !ids || k < 1 || k > kTopkMax || k > c->cfg.vocab) return SV_EINVAL;
  if (!c->last_stored_logits || c->last_rows == 0) return SV_ESTATE;
  if (row < 0 || row >= c->last_rows) return SV_EINVAL;
  const float* src = c->at<float>(c->lay.logits) + (size_t)row * c->cfg.vocab;
  unsigned long long* cand = c->at<unsigned long long>(c->lay.topk);
  unsigned long long* out = cand + (size_t)kTopkBlocks * kTopkMax;
  std::vector<unsigned long long> h(k);
  if (launch_topk(src, c->cfg.vocab, k, cand, out, c->stream) != hipSuccess ||
      hipMemcpyAsync(h.data(), out, sizeof(unsigned long long) * k, hipMemcpyDeviceToHost, c->stream) != hipSuccess ||
      hipStreamSynchronize(c->stream) != hipSuccess)
    return SV_EDEVICE;
  for (int i = 0; i < k; ++i) {
    // key = (orderable logit bits, ~id): undo both maps
    const uint32_t lo = (uint32_t)(h[i] & 0xffffffffu), hi = (uint32_t)(h[i] >> 32);
    ids[i] = (int32_t)(0xffffffffu - lo);
    const uint32_t u = (hi & 0x80000000u) ? (hi & 0x7fffffffu) : ~hi;
    float f;
    std::memcpy(&f, &u, 4);
    if (vals) vals[i] = f;
  }
  return SV_OK;
}

sv_status sv_selected_logits(sv_ctx* c, int32_t row, const int32_t* ids, int32_t n, float* vals) {
  if (!c || !ids || !vals || n < 1 || n > kMaxSelected) return SV_EINVAL;
  if (!c->last_stored_logits || c->last_rows == 0) return SV_ESTATE;
  if (row < 0 || row >= c->last_rows) return SV_EINVAL;
  if (!ids_ok(c, ids, n)) return SV_EINVAL;
  int* d_ids = c->at<int>(c->lay.sel);
  float* d_out = reinterpret_cast<float*>(d_ids + kMaxSelected);
  const float* src = c->at<float>(c->lay.logits) + (size_t)row * c->cfg.vocab;
  if (hipMemcpyAsync(d_ids, ids, sizeof(int) * n, hipMemcpyHostToDevice, c->stream) != hipSuccess ||
      launch_gather(src, d_ids, n, d_out, c->stream) != hipSuccess ||
      hipMemcpyAsync(vals, d_out, sizeof(float) * n, hipMemcpyDeviceToHost, c->stream) != hipSuccess ||
      hipStreamSynchronize(c->stream) != hipSuccess)
    return SV_EDEVICE;
  return SV_OK;
}

sv_status sv_clone_state(sv_ctx* dst, const sv_ctx* src) {
  if (!dst || !src || dst == src) return SV_EINVAL;
  sv_config a = dst->cfg, b = src->cfg;
  a.max_prefill_rows = b.max_prefill_rows = 0;
  if (std::memcmp(&a, &b, sizeof(sv_config)) != 0) return SV_EINVAL;
  if (src->kv_len > 0) {
    const sv_config& cfg = src->cfg;
    const int n_lp = (src->kv_len + kPage - 1) / kPage;
    const int page_bytes = 2 * cfg.n_kv_heads * kPage * cfg.head_dim * 2;
    if (hipStreamSynchronize(src->stream) != hipSuccess ||
        launch_copy_pages(src->buf.kv_pool, src->buf.page_table, src->buf.n_pages, dst->buf.kv_pool,
                          dst->buf.page_table, dst->buf.n_pages, n_lp, cfg.n_layers, page_bytes,
                          dst->stream) != hipSuccess ||
        hipStreamSynchronize(dst->stream) != hipSuccess)
      return SV_EDEVICE;
  }
  dst->kv_len = src->kv_len;
  dst->next_id = src->next_id;
  dst->hist = src->hist;
  dst->last_rows = 0;
  dst->last_stored_logits = 0;
  return SV_OK;
}

sv_status sv_kv_truncate(sv_ctx* c, int32_t new_len) {
  if (!c) return SV_EINVAL;
  if (new_len < 1 || new_len > c->kv_len) return SV_EINVAL;
  c->kv_len = new_len;
  c->next_id = c->hist[new_len - 1];
  return SV_OK;
}

sv_status sv_history(const sv_ctx* c, int32_t* host_dst, int32_t n) {
  if (!c || !host_dst || n < 0 || n > c->kv_len) return SV_EINVAL;
  for (int i = 0; i < n; ++i) host_dst[i] = c->hist[i];
  return SV_OK;
}

sv_status sv_restore(sv_ctx* c, int32_t kv_len, const int32_t* greedy_hist) {
  if (!c || !greedy_hist || kv_len < 1 || kv_len > c->cfg.max_ctx) return SV_EINVAL;
  if (!ids_ok(c, greedy_hist, kv_len)) return SV_EINVAL;
  for (int i = 0; i < kv_len; ++i) c->hist[i] = greedy_hist[i];
  c->kv_len = kv_len;
  c->next_id = greedy_hist[kv_len - 1];
  return SV_OK;
}

sv_status sv_set_debug(sv_ctx* c, int32_t store_logits) {
  if (!c || (store_logits != 0 && store_logits != 1)) return SV_EINVAL;
  c->store_logits = store_logits;
  return SV_OK;
}

sv_status sv_get_logits(sv_ctx* c, int32_t row, float* host_dst, int32_t vocab) {
  if (!c || !host_dst || vocab != c->cfg.vocab) return SV_EINVAL;
  if (!c->last_stored_logits || c->last_rows == 0) return SV_ESTATE;
  if (row < 0 || row >= c->last_rows) return SV_EINVAL;
  const float* src = c->at<float>(c->lay.logits) + (size_t)row * vocab;
  if (hipMemcpyAsync(host_dst, src, sizeof(float) * vocab, hipMemcpyDeviceToHost, c->stream) != hipSuccess ||
      hipStreamSynchronize(c->stream) != hipSuccess)
    return SV_EDEVICE;
  return SV_OK;
}

sv_status sv_set_profile(sv_ctx* c, int32_t mask) {
  if (!c || mask < 0 || mask >= (1 << kProfRoles)) return SV_EINVAL;
  c->prof_mask = mask;
  return SV_OK;
}

sv_status sv_profile_read(const sv_ctx* c, int32_t role, double* total_ms, int64_t* launches) {
  if (!c || role < 0 || role >= kProfRoles) return SV_EINVAL;
  if (total_ms) *total_ms = c->prof_ms[role];
  if (launches) *launches = c->prof_n[role];
  return SV_OK;
}

sv_status sv_profile_reset(sv_ctx* c) {
  if (!c) return SV_EINVAL;
  for (int r = 0; r < kProfRoles; ++r) { c->prof_ms[r] = 0.0; c->prof_n[r] = 0; }
  return SV_OK;
}

sv_status sv_last_argmax(const sv_ctx* c, int32_t* dst, int32_t* m) {
  if (!c || !dst || !m) return SV_EINVAL;
  if (c->last_rows == 0) return SV_ESTATE;
  *m = c->last_rows;
  for (int r = 0; r < c->last_rows; ++r) dst[r] = c->last_argmax[r];
  return SV_OK;
}

}  // extern "C"
