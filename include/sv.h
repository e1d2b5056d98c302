/* sv.h -- C ABI of libsv.so: greedy block verification on one MI355X (gfx950).
 *
 * The library runs the target model's forward for speculative decoding with
 * greedy acceptance.  One verify forward scores the pending greedy token plus
 * K draft tokens (M = K + 1 rows) in one pass, takes one argmax per row, keeps
 * the longest prefix of drafts that matches, and rolls the paged KV cache back
 * to it.  Every row's arithmetic is independent of M and of the other rows, so
 * a verify row is bit-identical to a one-token decode of the same prefix, and
 * the KV bits of a prefix do not depend on how the cache was built.
 *
 * Conventions for every entry point
 *   - Return value: sv_status (0 = SV_OK, negative = error).  No C++
 *     exception crosses the ABI.  Every argument is checked before any device
 *     work is queued, so an error leaves the context exactly as it was.
 *   - Pointers documented as "device" are HIP device addresses; "host" are CPU
 *     addresses.  Device memory (weights, KV pool, page table, workspace) is
 *     allocated and owned by the caller and must outlive the context.
 *   - A context is one sequence, and is not thread-safe.  All device work of
 *     a context runs on the hip stream given to sv_create; calls that return
 *     results (prefill, decode, verify) synchronise that stream before
 *     returning.
 *   - bf16 is IEEE binary32 truncated to its upper 16 bits (raw uint16).
 */
#ifndef SV_H
#define SV_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  SV_OK = 0,
  SV_EINVAL = -1,        /* bad argument (shape, id out of range, null pointer) */
  SV_ESTATE = -2,        /* call does not match the context state (prefix_len != kv_len, ...) */
  SV_ENOSPACE = -3,      /* KV capacity (max_ctx or pages) would be exceeded */
  SV_EDEVICE = -4,       /* a HIP call failed */
  SV_EUNSUPPORTED = -5,  /* configuration this build does not implement */
  SV_ESCRATCH = -6       /* sv_verify_noalloc: the call's intermediates exceed the library's static array */
} sv_status;

/* Model and capacity description.  Shapes: d_model, n_q_heads*head_dim and
 * d_ff multiples of 256 (int4: of 128 as well); head_dim 64 or 128;
 * n_q_heads a multiple of n_kv_heads; vocab a multiple of 64. */
typedef struct {
  int32_t n_layers, d_model, n_q_heads, n_kv_heads, head_dim, d_ff, vocab;
  int32_t act;          /* 0: SwiGLU (SiLU gate), 1: GeGLU (tanh-GELU gate) */
  int32_t weight_fmt;   /* linears: 0 bf16, 1 int4 symmetric group-64 with bf16 scales */
  int32_t tied;         /* 1: LM head is the embedding table (lm_head may equal embed) */
  float rms_eps, rope_theta;
  int32_t page_size;    /* must be 16 */
  int32_t max_ctx;      /* KV capacity in positions, multiple of page_size */
  int32_t max_k;        /* most drafts per verify, 0..63 */
  int32_t max_prefill_rows; /* 0: sv_prefill runs forwards of at most 64 rows
                               (the weight-streaming kernels of decode and verify);
                               65..16384: while more than 64 ids remain, forwards
                               of up to this many rows through row-tiled kernels
                               (bf16 and int4) with the same per-row arithmetic.
                               The workspace grows with it. */
} sv_config;

/* One layer's weights, all device pointers in the packed layouts that
 * sv_pack_linear produces:
 *   wqkv  [q | k | v] rows (n_q*dh + 2*n_kv*dh outputs) x d_model inputs, layout 2
 *   wo    d_model outputs x n_q*dh inputs
 *   wgu   gate and up, interleaved by sv_pack_linear layout 1, 2*d_ff outputs x d_model
 *   wd    d_model outputs x d_ff inputs
 *   *_scales: packed bf16 group scales (int4 only, else NULL)
 *   g_attn, g_mlp: bf16 RMSNorm gains [d_model] (plain, unpacked). */
typedef struct {
  const void *wqkv, *wqkv_scales, *wo, *wo_scales, *wgu, *wgu_scales, *wd, *wd_scales;
  const void *g_attn, *g_mlp;
} sv_layer_weights;

/* embed: packed bf16 [vocab x d_model] (sv_pack_linear of the row-major
 * table); lm_head: packed bf16 [vocab x d_model] (== embed when tied);
 * g_final: bf16 [d_model]; layers: host array of n_layers entries (copied). */
typedef struct {
  const void *embed, *lm_head, *g_final;
  const sv_layer_weights *layers;
} sv_weights;

/* Caller-owned device buffers.
 *   kv_pool: IEEE fp16, n_pages pages.  The block of page p, layer l, kv
 *            (0 = K, 1 = V), head h starts at element
 *            B = (((l*n_pages + p)*2 + kv)*n_kv + h)*16*head_dim; inside it,
 *            K of slot s, element e is at B + s*head_dim + e, and V is stored
 *            transposed, element e of slot s at B + e*16 + s.
 *   page_table: int32 [max_ctx/16], 16-byte aligned (SV_EINVAL otherwise),
 *            logical page -> physical page in [0, n_pages); read by the
 *            kernels, never written.
 *   workspace: at least the size sv_query_sizes reports; its contents are
 *            the library's between calls. */
typedef struct {
  void *kv_pool; int64_t kv_pool_bytes;
  const int32_t *page_table; int32_t n_pages;
  void *workspace; int64_t workspace_bytes;
} sv_buffers;

typedef struct sv_ctx sv_ctx;

/* Sizes the caller must allocate for cfg: KV pool bytes for max_ctx positions
 * (one page per 16 positions) and workspace bytes.  Host-only; no device call. */
sv_status sv_query_sizes(const sv_config *cfg, int64_t *kv_pool_bytes, int64_t *workspace_bytes);

/* Bytes of the packed form of an [n x k] linear (outputs x inputs) in format
 * fmt (0 bf16, 1 int4); *scale_bytes is 0 for bf16.  Host-only. */
sv_status sv_packed_linear_bytes(int32_t fmt, int32_t n, int32_t k, int64_t *bytes, int64_t *scale_bytes);

/* Repack a row-major linear into the tiled layout the kernels stream
 * (a pure permutation, bit-exact).  src0: device [n x k] (bf16, or int8 codes
 * in [-8, 7] for fmt 1) with src0_scales device bf16 [n x k/64] (fmt 1).
 * layout 0: plain (O, down, embedding / LM head).
 * layout 1: gate/up; src1 is the up matrix [n x k] (+ scales), and the packed
 *           output holds 2n outputs, 16-output blocks of src0 and src1
 *           interleaved.
 * layout 2: fused QKV ([q heads | k heads | v heads] x head_dim rows); rows
 *           are reordered inside each head so every 64-output group holds
 *           RoPE pairs (i, i + head_dim/2).  head_dim is 64 or 128.
 * dst / dst_scales: device, sizes from sv_packed_linear_bytes (for 2n outputs
 * with layout 1).  Runs on `stream` (hipStream_t, NULL = default). */
sv_status sv_pack_linear(int32_t fmt, int32_t layout, const void *src0, const void *src0_scales,
                         const void *src1, const void *src1_scales, int32_t n, int32_t k,
                         int32_t head_dim, void *dst, void *dst_scales, void *stream);

/* Create a context at kv_len = 0.  Validates cfg and buffer sizes, uploads the
 * RoPE table (angle pos * theta^(-2i/head_dim), cos/sin evaluated in double and
 * rounded once to float) into the workspace.  `stream` is a hipStream_t.  The
 * context owns a few small pinned, device-mapped host buffers (the forward's
 * params, which its first kernel reads over the bus, and the result its last
 * kernel writes there), freed by sv_destroy.  Errors: SV_EINVAL (bad cfg or
 * buffer sizes), SV_EUNSUPPORTED, SV_EDEVICE (a HIP allocation or copy). */
sv_status sv_create(const sv_config *cfg, const sv_weights *w, const sv_buffers *buf,
                    void *stream, sv_ctx **out);
void sv_destroy(sv_ctx *ctx);

/* Commit n ids at positions kv_len..kv_len+n-1 (a fresh prefill when kv_len
 * is 0, a block commit otherwise; the whole committed prefix of the cache
 * histories compared in "Shape and cache history in Gemma block
 * verification", section "Same-prefix controls").  Runs in forwards of at
 * most 64 rows with the kernels of decode and verify, or, with
 * max_prefill_rows set, of up to that many rows with row-tiled kernels (the
 * compute-bound prefill: each weight tile is read once per 128 rows); each
 * row's logits, argmax and KV bits are those a one-token decode gives it
 * either way.  On return
 * kv_len += n and *next_id (host) is the greedy id after the last row.
 * ids: host int32 [n], each in [0, vocab).  Errors: SV_EINVAL (n < 1, bad id),
 * SV_ENOSPACE (kv_len + n > max_ctx). */
sv_status sv_prefill(sv_ctx *ctx, const int32_t *ids, int32_t n, int32_t *next_id);

/* One-token decode: commit `token` at position kv_len and return the greedy
 * id after it (the per-token decode path that "Phase 23: Speculative Verify
 * Parity" makes authoritative, section 1).  Bit-identical to row 0 of any
 * verify at the same prefix.  Errors as sv_prefill with n = 1. */
sv_status sv_decode_step(sv_ctx *ctx, int32_t token, int32_t *next_id);

/* Greedy block verify ("Phase 23: Speculative Verify Parity", section 2,
 * steps 1-5; acceptance rule of "Shape and cache history in Gemma block
 * verification", section "Mechanism and failure").
 * Rows [next_id, draft_ids[0..k-1]] at positions kv_len..kv_len+k are
 * forwarded in one pass (KV of all rows written first, row r attends to
 * kv_len + r + 1 positions).  With a_r the argmax of row r (ties to the lowest
 * id), n = the number of leading i with draft_ids[i] == a_i.  The cache keeps
 * positions < kv_len + n + 1; kv_len becomes prefix_len + n + 1 and next_id
 * becomes a_n.  k = 0 is exactly sv_decode_step(sv_next_id(ctx)).
 * prefix_len must equal kv_len (SV_ESTATE); 0 <= k <= max_k; ids in
 * [0, vocab); kv_len + k + 1 <= max_ctx (SV_ENOSPACE).  Outputs are host. */
sv_status sv_verify(sv_ctx *ctx, int32_t prefix_len, const int32_t *draft_ids, int32_t k,
                    int32_t *n_accepted, int32_t *next_id);

/* sv_verify for callers that cannot allocate (a serving loop or harness in
 * which no call may reach hipMalloc, hipFree or any other allocating
 * routine).  Arguments, checks, kernels and results are sv_verify's, bit for
 * bit: the same (n_accepted, next_id), KV bits, history and observer logits.
 * What differs: the forward's intermediates (the params copy, residual rows,
 * sums of squares, q, attention split partials, activation planes and row
 * argmax keys) live in one static device array of the library instead of the
 * context's workspace, and the kernels are launched directly, so no HIP graph
 * is instantiated.  The observer logits still go to the workspace (an
 * output), the RoPE table is read from it (an input sv_create wrote), and no
 * profiling stamps are taken.
 *
 * The array holds 32 MiB on every GPU the library runs on, for the life of
 * the process.  A call needs about (k+1) x [d_model x 8.25 + n_q x head_dim x
 * 8 + d_ff x 4 + n_q x splits x (head_dim + 4) x 4 + 12] bytes (nine buffers,
 * each rounded up to 256 B), where splits is the most attention splits of
 * any row of the window (a row at context c has ceil(c / 64) of them up to
 * 64 and never more than 64); above 32 MiB the call returns SV_ESCRATCH
 * before any launch (for example the 8B shape at a 32K context with k above
 * 27).  Every call on one GPU shares that GPU's array: calls whose execution
 * overlaps on one GPU (other threads, other streams) race and their results
 * are undefined.  Nothing a previous call left in the
 * array is read: the row keys are cleared by the first kernel and every
 * other intermediate is written before it is read.
 * Errors: as sv_verify, plus SV_ESCRATCH; SV_EDEVICE if the array's device
 * address could not be obtained at sv_create. */
sv_status sv_verify_noalloc(sv_ctx *ctx, int32_t prefix_len, const int32_t *draft_ids, int32_t k,
                            int32_t *n_accepted, int32_t *next_id);

/* Batched greedy block verify: n contexts of one model (identical sv_config
 * apart from max_prefill_rows, identical weight pointers) each verify their
 * own window -- rows [next_id_i, draft_ids of i] at positions kv_len_i ..
 * kv_len_i + k_i -- in ONE forward of M = sum(k_i + 1) rows.  Rows of
 * different sequences meet only in the weight GEMMs, whose per-row
 * arithmetic does not depend on the other rows, and attention reads each
 * row's own sequence's KV pool and page table; so every context ends in
 * exactly the state (KV bits, history, next_id, observer logits) that
 * sv_verify on it alone gives, whatever the batch holds or its order.
 * ks: host int32 [n], 0 <= k_i <= max_k; draft_ids: host int32 [sum k_i],
 * sequence i's drafts after sequence i-1's; prefix_lens: host int32 [n],
 * each equal to that context's kv_len (SV_ESTATE otherwise).  n_accepted,
 * next_ids: host int32 [n] outputs (may be NULL).  1 <= n <= 64; M at most
 * the rows of ctxs[0] (64, or its max_prefill_rows when larger): the forward
 * runs in ctxs[0]'s workspace on its stream.  Contexts must be distinct.
 * Errors: SV_EINVAL (shapes, ids, mismatched contexts, too many rows),
 * SV_ESTATE, SV_ENOSPACE; all checked before any launch. */
sv_status sv_verify_batch(sv_ctx *const *ctxs, int32_t n, const int32_t *prefix_lens, const int32_t *ks,
                          const int32_t *draft_ids, int32_t *n_accepted, int32_t *next_ids);

/* Roll back to the first new_len committed positions in O(1) ("Phase 23:
 * Speculative Verify Parity", section 2, step 5): kv_len = new_len and
 * next_id = the greedy id recorded after position new_len - 1.  KV past
 * new_len is left in place and never read again.  1 <= new_len <= kv_len. */
sv_status sv_kv_truncate(sv_ctx *ctx, int32_t new_len);

/* Checkpoint / resume of a sequence.  sv_history copies the greedy id
 * recorded after each of the first n committed positions (n <= kv_len) to
 * host_dst.  sv_restore declares that positions [0, kv_len) of this
 * context's KV pool (through its page table) hold a committed prefix -- for
 * instance a copy of another context's pool -- with greedy history
 * greedy_hist (host int32 [kv_len], ids in [0, vocab)); afterwards kv_len is
 * that value and next_id = greedy_hist[kv_len - 1].  The library does not
 * read the pool here: the caller vouches for its contents.  Errors:
 * SV_EINVAL (kv_len outside [1, max_ctx], bad id, null pointer). */
sv_status sv_history(const sv_ctx *ctx, int32_t *host_dst, int32_t n);
sv_status sv_restore(sv_ctx *ctx, int32_t kv_len, const int32_t *greedy_hist);

int32_t sv_kv_len(const sv_ctx *ctx);
int32_t sv_next_id(const sv_ctx *ctx);

/* Observer mode ("Shape and cache history in Gemma block verification",
 * section "Same-prefix controls": inspecting logits must not change the
 * argmax array).  store_logits = 1 makes every later forward also store its
 * fp32 logits; the argmax computation is untouched. */
sv_status sv_set_debug(sv_ctx *ctx, int32_t store_logits);

/* Copy the fp32 logits of row `row` of the last forward (observer mode on)
 * to host_dst [vocab].  SV_ESTATE if no forward stored logits; SV_EINVAL for a
 * row outside the last forward. */
sv_status sv_get_logits(sv_ctx *ctx, int32_t row, float *host_dst, int32_t vocab);

/* Argmax a_0..a_{M-1} of every row of the last forward (host int32 [M]);
 * *m receives M.  dst must hold max(64, max_prefill_rows) entries. */
sv_status sv_last_argmax(const sv_ctx *ctx, int32_t *dst, int32_t *m);

/* Audit mode (the diagnostics of "Phase 23: Speculative Verify Parity",
 * section 4 -- dump the top candidates where verify and decode disagree,
 * audit sampled steps against one-token decode -- and the selected-logit
 * reads of "Shape and cache history in Gemma block verification", section
 * "Next discriminating tests", which must leave the argmax bits alone: they
 * only read the logits observer mode stored, on the device).
 *
 * sv_topk: the k largest logits of row `row` of the last forward, in the
 * argmax order (larger logit first, the lower id first among equal logits;
 * -0.0 counts as +0.0), so ids[0] is that row's argmax.  ids: host int32 [k],
 * vals: host float [k] or NULL; 1 <= k <= 64.  SV_ESTATE if the last forward
 * stored no logits (sv_set_debug), SV_EINVAL for a bad row or k. */
sv_status sv_topk(sv_ctx *ctx, int32_t row, int32_t k, int32_t *ids, float *vals);

/* sv_selected_logits: vals[i] = logit of ids[i] in row `row` of the last
 * forward, gathered on the device.  ids: host int32 [n], each in
 * [0, vocab); vals: host float [n]; 1 <= n <= 4096.  Errors as sv_topk. */
sv_status sv_selected_logits(sv_ctx *ctx, int32_t row, const int32_t *ids, int32_t n, float *vals);

/* sv_clone_state: make dst hold src's committed state -- the KV of positions
 * [0, kv_len) (whole pages, copied on the device through both page tables),
 * the greedy history, kv_len and next_id -- so a decode audit can replay a
 * step of src on dst.  Both contexts must have the same sv_config apart from
 * max_prefill_rows (SV_EINVAL otherwise, or if dst == src).  dst's observer
 * logits are dropped. */
sv_status sv_clone_state(sv_ctx *dst, const sv_ctx *src);

/* Measurement (the per-kernel timing a roofline figure needs): every launch
 * of an enabled kernel role stamps the device's constant-rate wall clock
 * (hipDeviceAttributeWallClockRate) when its first workgroup starts and when
 * its last one ends; the spans are summed on the host after each forward's
 * synchronisation.  A profiled forward runs the same kernels (in the same
 * HIP graph) as an unprofiled one, plus one small kernel that clears the
 * stamp slots and a copy of the slots to host.
 * Roles: 0 QKV GEMM, 1 O-projection GEMM, 2 gate/up GEMM, 3 down GEMM,
 * 4 LM-head GEMM, 5 attention (split + combine).  Bit r of `mask` enables
 * role r; mask 0 stops recording and keeps the totals. */
sv_status sv_set_profile(sv_ctx *ctx, int32_t mask);
sv_status sv_profile_read(const sv_ctx *ctx, int32_t role, double *total_ms, int64_t *launches);
sv_status sv_profile_reset(sv_ctx *ctx);

const char *sv_status_str(sv_status s);

#ifdef __cplusplus
}
#endif
#endif /* SV_H */
