// Host-only build of the library: the HIP calls of the host runtime on host
// memory, and the kernel launchers replaced by a toy model that runs on the
// CPU, so the runtime's argument checks, context state and commit logic can
// be tested without a GPU.  Test infrastructure only.
//
// Toy model: the greedy id after any row is (its id + 1) mod vocab.  The
// embed launcher copies the forward's parameters as the embed kernel does;
// the acceptance launchers apply the acceptance rule to the toy argmax; the
// page-copy launcher copies pages through both page tables; every other
// launcher does nothing.
#include <hip/hip_runtime.h>

#include <cstdlib>
#include <cstring>
#include <vector>

#include "../../greedy_block_verification_amd/csrc/sv_internal.h"

static int g_vocab = 1;
static int g_launches = 0;   // launchers called since load (no-op kernels included)

extern "C" int stub_launches() { return g_launches; }

hipError_t hipGetDevice(int* dev) { *dev = 0; return hipSuccess; }
hipError_t hipDeviceGetAttribute(int* v, hipDeviceAttribute_t attr, int) {
  *v = attr == hipDeviceAttributeMultiprocessorCount ? 256 : 100000;
  return hipSuccess;
}
hipError_t hipGetSymbolAddress(void** p, const void* symbol) { *p = const_cast<void*>(symbol); return hipSuccess; }
hipError_t hipHostMalloc(void** p, size_t bytes, unsigned) {
  *p = std::calloc(1, bytes ? bytes : 1);
  return *p ? hipSuccess : hipErrorUnknown;
}
hipError_t hipHostFree(void* p) { std::free(p); return hipSuccess; }
hipError_t hipHostGetDevicePointer(void** dev, void* host, unsigned) { *dev = host; return hipSuccess; }
hipError_t hipMemcpy(void* dst, const void* src, size_t bytes, hipMemcpyKind) {
  std::memmove(dst, src, bytes);
  return hipSuccess;
}
hipError_t hipMemcpyAsync(void* dst, const void* src, size_t bytes, hipMemcpyKind k, hipStream_t) {
  return hipMemcpy(dst, src, bytes, k);
}
hipError_t hipStreamCreateWithFlags(hipStream_t* st, unsigned) {
  *st = reinterpret_cast<hipStream_t>(std::malloc(1));
  return hipSuccess;
}
hipError_t hipStreamDestroy(hipStream_t st) { std::free(st); return hipSuccess; }
hipError_t hipStreamSynchronize(hipStream_t) { return hipSuccess; }
// Graph capture cannot record host calls: the runtime is run with SV_NO_GRAPH=1
hipError_t hipStreamBeginCapture(hipStream_t, hipStreamCaptureMode) { return hipErrorNotSupported; }
hipError_t hipStreamEndCapture(hipStream_t, hipGraph_t* g) { *g = nullptr; return hipErrorNotSupported; }
hipError_t hipGraphInstantiate(hipGraphExec_t*, hipGraph_t, hipGraphNode_t*, char*, size_t) { return hipErrorNotSupported; }
hipError_t hipGraphLaunch(hipGraphExec_t, hipStream_t) { return hipErrorNotSupported; }
hipError_t hipGraphDestroy(hipGraph_t) { return hipSuccess; }
hipError_t hipGraphExecDestroy(hipGraphExec_t) { return hipSuccess; }

namespace sv {

static int ceil_div(int a, int b) { return (a + b - 1) / b; }
// The split plan (a function of the row's own context): 64-position blocks,
// at most kAttnMaxSplits splits.
static int ns_of(int ctx) {
  const int nb = ceil_div(ctx, kAttnBlock), bps = ceil_div(nb, kAttnMaxSplits);
  return ceil_div(nb, bps);
}
int attn_splits(int ctx) { return ns_of(ctx); }
int attn_blocks_per_split(int ctx) { return ceil_div(ceil_div(ctx, kAttnBlock), kAttnMaxSplits); }
int attn_splits_max(int kv_len, int M) {
  int m = 1;
  for (int r = 0; r < M; ++r) m = ns_of(kv_len + r + 1) > m ? ns_of(kv_len + r + 1) : m;
  return m;
}

static int toy_next(int id) { return (id + 1) % g_vocab; }

hipError_t launch_gemm(const GemmArgs&, int, int, hipStream_t) { ++g_launches; return hipSuccess; }
hipError_t launch_gemm_tiled(const GemmArgs&, int, hipStream_t) { ++g_launches; return hipSuccess; }
hipError_t launch_attention(const AttnArgs&, hipStream_t) { ++g_launches; return hipSuccess; }
hipError_t launch_attention_rows(const AttnArgs&, hipStream_t) { ++g_launches; return hipSuccess; }
hipError_t launch_prof_reset(unsigned long long*, int, hipStream_t) { ++g_launches; return hipSuccess; }
hipError_t launch_topk(const float*, int, int, unsigned long long*, unsigned long long*, hipStream_t) {
  ++g_launches;
  return hipSuccess;
}
hipError_t launch_gather(const float*, const int*, int, float*, hipStream_t) { ++g_launches; return hipSuccess; }
hipError_t launch_pack(int, int, const void*, const void*, const void*, const void*, int, int, int, void*, void*,
                       hipStream_t) {
  ++g_launches;
  return hipSuccess;
}

hipError_t launch_embed(const int* hparams, int* params, int M, const void*, int vocab, int, float*, float*,
                        const uint16_t*, uint16_t*, uint16_t*, unsigned long long* best, hipStream_t) {
  ++g_launches;
  g_vocab = vocab;
  std::memcpy(params, hparams, sizeof(int) * (2 + (size_t)M));
  for (int r = 0; r < M; ++r) best[r] = 0ull;
  return hipSuccess;
}

hipError_t launch_accept(const int* params, int M, int verify, const unsigned long long*, int* result, hipStream_t) {
  ++g_launches;
  if (M < 1 || (verify && M > 64)) return hipErrorInvalidValue;
  for (int r = 0; r < M; ++r) result[2 + r] = toy_next(params[2 + r]);
  int n = M - 1;
  if (verify) {
    n = 0;
    while (n < M - 1 && params[2 + n + 1] == result[2 + n]) ++n;
  }
  result[0] = n;
  result[1] = result[2 + n];
  return hipSuccess;
}

hipError_t launch_accept_batch(const int* params, int M, const SeqDev* seqs, int n_seq, const unsigned long long*,
                               int* result, hipStream_t) {
  ++g_launches;
  if (M < 1 || n_seq < 1 || n_seq > 64) return hipErrorInvalidValue;
  for (int r = 0; r < M; ++r) result[2 + r] = toy_next(params[2 + r]);
  for (int s = 0; s < n_seq; ++s) {
    int n = 0;
    while (n < seqs[s].m - 1 && params[2 + seqs[s].row0 + n + 1] == result[2 + seqs[s].row0 + n]) ++n;
    result[2 + M + 2 * s] = n;
    result[2 + M + 2 * s + 1] = result[2 + seqs[s].row0 + n];
  }
  return hipSuccess;
}

hipError_t launch_copy_pages(const void* src, const int* src_pt, int src_pages, void* dst, const int* dst_pt,
                             int dst_pages, int n_lp, int n_layers, int page_bytes, hipStream_t) {
  ++g_launches;
  if (n_lp < 1 || page_bytes % 16) return hipErrorInvalidValue;
  for (int l = 0; l < n_layers; ++l)
    for (int lp = 0; lp < n_lp; ++lp)
      std::memcpy(static_cast<char*>(dst) + ((size_t)l * dst_pages + dst_pt[lp]) * page_bytes,
                  static_cast<const char*>(src) + ((size_t)l * src_pages + src_pt[lp]) * page_bytes, page_bytes);
  return hipSuccess;
}

}  // namespace sv
