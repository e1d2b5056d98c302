// Host logic of libsv (argument checks, context state, commit, rollback,
// batched verify bookkeeping, the no-allocation path's size check) built
// against host_stubs.cpp: no GPU, the toy model "greedy id after a row =
// its id + 1 mod vocab".  Built with g++ (optionally with the address and
// undefined-behaviour sanitizers) and run by tests/test_host_runtime_cpu.py.
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <vector>

#include "sv.h"

extern "C" int stub_launches();

static int g_fail = 0;
#define CHECK(c)                                                           \
  do {                                                                     \
    if (!(c)) {                                                            \
      std::fprintf(stderr, "FAIL %s:%d: %s\n", __FILE__, __LINE__, #c);  \
      ++g_fail;                                                            \
    }                                                                      \
  } while (0)

static sv_config tiny_cfg() {
  sv_config c{};
  c.n_layers = 2; c.d_model = 256; c.n_q_heads = 4; c.n_kv_heads = 2; c.head_dim = 64; c.d_ff = 1024;
  c.vocab = 2048; c.act = 0; c.weight_fmt = 0; c.tied = 1; c.rms_eps = 1e-6f; c.rope_theta = 1e4f;
  c.page_size = 16; c.max_ctx = 256; c.max_k = 8; c.max_prefill_rows = 0;
  return c;
}

static char g_dummy[64];   // weight pointers: never dereferenced by the host runtime

struct Ctx {
  sv_config cfg{};
  std::vector<sv_layer_weights> layers;
  sv_weights w{};
  std::vector<char> kv, ws;
  std::vector<int32_t> pt;
  sv_buffers buf{};
  sv_ctx* c = nullptr;
  int status = 0;
  explicit Ctx(const sv_config& cf, int pt_shift = 0) : cfg(cf) {
    int64_t kvb = 0, wsb = 0;
    status = sv_query_sizes(&cfg, &kvb, &wsb);
    if (status != SV_OK) return;
    layers.resize(cfg.n_layers);
    for (auto& L : layers) {
      L.wqkv = L.wo = L.wgu = L.wd = L.g_attn = L.g_mlp = g_dummy;
      if (cfg.weight_fmt == 1) L.wqkv_scales = L.wo_scales = L.wgu_scales = L.wd_scales = g_dummy;
    }
    w.embed = w.lm_head = w.g_final = g_dummy;
    w.layers = layers.data();
    kv.assign((size_t)kvb, 0);
    ws.assign((size_t)wsb, 0);
    const int n_pages = cfg.max_ctx / cfg.page_size;
    pt.resize(n_pages + 4);
    for (int i = 0; i < n_pages; ++i) pt[i] = (i + pt_shift) % n_pages;
    buf = sv_buffers{kv.data(), kvb, pt.data(), n_pages, ws.data(), wsb};
    status = sv_create(&cfg, &w, &buf, nullptr, &c);
  }
  ~Ctx() { sv_destroy(c); }
};

static int nxt(int id, int V) { return (id + 1) % V; }

static void test_config_checks() {
  sv_config c = tiny_cfg();
  int64_t a = 0, b = 0;
  CHECK(sv_query_sizes(&c, &a, &b) == SV_OK && a == 2LL * 16 * 2 * 2 * 16 * 64 * 2 && b > 0);
  sv_config bad = c; bad.page_size = 32; CHECK(sv_query_sizes(&bad, &a, &b) == SV_EINVAL);
  bad = c; bad.head_dim = 96; CHECK(sv_query_sizes(&bad, &a, &b) == SV_EINVAL);
  bad = c; bad.n_q_heads = 3; CHECK(sv_query_sizes(&bad, &a, &b) == SV_EINVAL);
  bad = c; bad.max_k = 64; CHECK(sv_query_sizes(&bad, &a, &b) == SV_EINVAL);
  bad = c; bad.weight_fmt = 1; CHECK(sv_query_sizes(&bad, &a, &b) == SV_EINVAL);   // d_model 256: not a multiple of 512
  bad = c; bad.max_prefill_rows = 64; CHECK(sv_query_sizes(&bad, &a, &b) == SV_EINVAL);
  bad = c; bad.max_ctx = 100; CHECK(sv_query_sizes(&bad, &a, &b) == SV_EINVAL);
  CHECK(sv_query_sizes(nullptr, &a, &b) == SV_EINVAL);
  int64_t pb = 0, ps = 0;
  CHECK(sv_packed_linear_bytes(1, 32, 256, &pb, &ps) == SV_OK && pb == 32 * 256 / 2 && ps == 32 * 4 * 2);
  CHECK(sv_packed_linear_bytes(0, 20, 256, &pb, &ps) == SV_EINVAL);
  const char* seen[7];
  int k = 0;
  for (sv_status s : {SV_OK, SV_EINVAL, SV_ESTATE, SV_ENOSPACE, SV_EDEVICE, SV_EUNSUPPORTED, SV_ESCRATCH}) {
    seen[k] = sv_status_str(s);
    CHECK(seen[k] && std::strlen(seen[k]) > 0);
    for (int i = 0; i < k; ++i) CHECK(std::strcmp(seen[i], seen[k]) != 0);
    ++k;
  }
}

static void test_create_checks() {
  sv_config c = tiny_cfg();
  Ctx ok(c);
  CHECK(ok.status == SV_OK && ok.c && sv_kv_len(ok.c) == 0 && sv_next_id(ok.c) == -1);
  sv_ctx* out = reinterpret_cast<sv_ctx*>(&g_dummy);
  CHECK(sv_create(&c, &ok.w, &ok.buf, nullptr, &out) == SV_OK);   // the same buffers: allowed (caller's memory)
  sv_destroy(out);
  CHECK(sv_create(&c, nullptr, &ok.buf, nullptr, &out) == SV_EINVAL && out == nullptr);
  sv_buffers small = ok.buf; small.workspace_bytes -= 1;
  CHECK(sv_create(&c, &ok.w, &small, nullptr, &out) == SV_EINVAL);
  sv_buffers badpt = ok.buf; badpt.n_pages = 3;   // entries >= 3 point outside the pool
  CHECK(sv_create(&c, &ok.w, &badpt, nullptr, &out) == SV_EINVAL);
  sv_buffers mis = ok.buf; mis.page_table = ok.pt.data() + 1;   // not 16-byte aligned
  CHECK(sv_create(&c, &ok.w, &mis, nullptr, &out) == SV_EINVAL);
  std::vector<sv_layer_weights> holes(ok.layers);
  holes[1].wd = nullptr;
  sv_weights wh = ok.w; wh.layers = holes.data();
  CHECK(sv_create(&c, &wh, &ok.buf, nullptr, &out) == SV_EINVAL);
  sv_destroy(nullptr);
}

static void test_prefill_decode_verify_truncate() {
  sv_config c = tiny_cfg();
  const int V = c.vocab;
  Ctx t(c);
  CHECK(t.status == SV_OK);
  sv_ctx* x = t.c;
  int32_t nx = -7;
  std::vector<int32_t> ids = {5, 17, 2047, 0, 33, 100, 7, 8, 9, 10};
  CHECK(sv_prefill(x, ids.data(), 0, &nx) == SV_EINVAL);
  std::vector<int32_t> bad = ids; bad[3] = V;
  CHECK(sv_prefill(x, bad.data(), 10, &nx) == SV_EINVAL && sv_kv_len(x) == 0);
  std::vector<int32_t> big(c.max_ctx + 1, 1);
  CHECK(sv_prefill(x, big.data(), (int)big.size(), &nx) == SV_ENOSPACE && sv_kv_len(x) == 0);
  const int l0 = stub_launches();
  CHECK(sv_prefill(x, ids.data(), 10, &nx) == SV_OK);
  CHECK(stub_launches() - l0 == 2 + 5 * c.n_layers + 1);   // embed, 5 per layer, LM head, accept
  CHECK(sv_kv_len(x) == 10 && nx == nxt(10, V) && sv_next_id(x) == nx);
  std::vector<int32_t> hist(10);
  CHECK(sv_history(x, hist.data(), 10) == SV_OK);
  for (int i = 0; i < 10; ++i) CHECK(hist[i] == nxt(ids[i], V));
  CHECK(sv_history(x, hist.data(), 11) == SV_EINVAL);
  // decode
  int32_t d = 0;
  CHECK(sv_decode_step(x, 2047, &d) == SV_OK && d == 0 && sv_kv_len(x) == 11);
  CHECK(sv_decode_step(x, -1, &d) == SV_EINVAL && sv_kv_len(x) == 11);
  // verify: state and argument errors leave the context alone
  int32_t n = -1, nv = -1;
  const int32_t cur = sv_next_id(x);   // 0 + 1
  int32_t dr[9] = {nxt(cur, V), nxt(nxt(cur, V), V), 999, 4, 5, 6, 7, 8, 9};
  CHECK(sv_verify(x, 10, dr, 3, &n, &nv) == SV_ESTATE);
  CHECK(sv_verify(x, 11, dr, 9, &n, &nv) == SV_EINVAL);
  CHECK(sv_verify(x, 11, nullptr, 2, &n, &nv) == SV_EINVAL);
  int32_t drbad[2] = {1, V};
  CHECK(sv_verify(x, 11, drbad, 2, &n, &nv) == SV_EINVAL && sv_kv_len(x) == 11);
  // mismatch at index 2: n = 2, next = the correction (the toy greedy id after d_1)
  CHECK(sv_verify(x, 11, dr, 3, &n, &nv) == SV_OK);
  CHECK(n == 2 && nv == nxt(dr[1], V) && sv_kv_len(x) == 14 && sv_next_id(x) == nv);
  std::vector<int32_t> h(14);
  CHECK(sv_history(x, h.data(), 14) == SV_OK);
  CHECK(h[11] == nxt(cur, V) && h[12] == nxt(dr[0], V) && h[13] == nxt(dr[1], V));
  // every draft accepted: the bonus id is the toy greedy id after the last draft
  const int32_t c2 = sv_next_id(x);
  int32_t all[4] = {nxt(c2, V), nxt(nxt(c2, V), V), nxt(nxt(nxt(c2, V), V), V), nxt(nxt(nxt(nxt(c2, V), V), V), V)};
  CHECK(sv_verify(x, 14, all, 4, &n, &nv) == SV_OK && n == 4 && nv == nxt(all[3], V) && sv_kv_len(x) == 19);
  // k = 0 is a decode of the pending id
  const int32_t c3 = sv_next_id(x);
  CHECK(sv_verify(x, 19, nullptr, 0, &n, &nv) == SV_OK && n == 0 && nv == nxt(c3, V) && sv_kv_len(x) == 20);
  // rollback restores next_id from the history
  CHECK(sv_kv_truncate(x, 0) == SV_EINVAL && sv_kv_truncate(x, 21) == SV_EINVAL);
  CHECK(sv_kv_truncate(x, 12) == SV_OK && sv_kv_len(x) == 12 && sv_next_id(x) == h[11]);
  CHECK(sv_kv_truncate(x, 12) == SV_OK && sv_kv_len(x) == 12);
  // capacity: a window past max_ctx is refused before anything runs
  std::vector<int32_t> fill(c.max_ctx - 12 - 2, 3);
  CHECK(sv_prefill(x, fill.data(), (int)fill.size(), &nx) == SV_OK && sv_kv_len(x) == c.max_ctx - 2);
  int32_t two[2] = {1, 2};
  CHECK(sv_verify(x, c.max_ctx - 2, two, 2, &n, &nv) == SV_ENOSPACE && sv_kv_len(x) == c.max_ctx - 2);
  CHECK(sv_verify(x, c.max_ctx - 2, two, 1, &n, &nv) == SV_OK && sv_kv_len(x) >= c.max_ctx - 1);
}

static void test_restore_observer_audit() {
  sv_config c = tiny_cfg();
  Ctx t(c), u(c, 3);   // u: a different page-table permutation
  CHECK(t.status == SV_OK && u.status == SV_OK);
  std::vector<int32_t> hist(40);
  for (int i = 0; i < 40; ++i) hist[i] = (i * 37) % c.vocab;
  CHECK(sv_restore(t.c, 0, hist.data()) == SV_EINVAL);
  CHECK(sv_restore(t.c, c.max_ctx + 1, hist.data()) == SV_EINVAL);
  std::vector<int32_t> hb = hist; hb[5] = -3;
  CHECK(sv_restore(t.c, 40, hb.data()) == SV_EINVAL && sv_kv_len(t.c) == 0);
  CHECK(sv_restore(t.c, 40, hist.data()) == SV_OK && sv_kv_len(t.c) == 40 && sv_next_id(t.c) == hist[39]);
  // observer mode: no logits before a forward that stored them
  float row[2048];
  CHECK(sv_get_logits(t.c, 0, row, c.vocab) == SV_ESTATE);
  int32_t ids[4];
  CHECK(sv_topk(t.c, 0, 4, ids, nullptr) == SV_ESTATE);
  CHECK(sv_set_debug(t.c, 1) == SV_OK);
  int32_t d = 0, m = 0, arg[64];
  CHECK(sv_decode_step(t.c, hist[39], &d) == SV_OK);
  CHECK(sv_get_logits(t.c, 0, row, c.vocab) == SV_OK);
  CHECK(sv_get_logits(t.c, 1, row, c.vocab) == SV_EINVAL);
  CHECK(sv_get_logits(t.c, 0, row, c.vocab - 1) == SV_EINVAL);
  CHECK(sv_topk(t.c, 0, 0, ids, nullptr) == SV_EINVAL && sv_topk(t.c, 0, 65, ids, nullptr) == SV_EINVAL);
  CHECK(sv_last_argmax(t.c, arg, &m) == SV_OK && m == 1 && arg[0] == d);
  // clone the committed state into a context with another page table
  CHECK(sv_clone_state(t.c, t.c) == SV_EINVAL);
  for (size_t i = 0; i < t.kv.size(); ++i) t.kv[i] = (char)(i * 131 + 7);
  CHECK(sv_clone_state(u.c, t.c) == SV_OK);
  CHECK(sv_kv_len(u.c) == 41 && sv_next_id(u.c) == sv_next_id(t.c));
  std::vector<int32_t> ht(41), hu(41);
  CHECK(sv_history(t.c, ht.data(), 41) == SV_OK && sv_history(u.c, hu.data(), 41) == SV_OK && ht == hu);
  const int n_pages = c.max_ctx / 16;
  const size_t page_bytes = t.kv.size() / ((size_t)c.n_layers * n_pages);
  for (int l = 0; l < c.n_layers; ++l)
    for (int lp = 0; lp < 3; ++lp)   // the committed 41 positions fill 3 logical pages
      CHECK(std::memcmp(&u.kv[((size_t)l * n_pages + u.pt[lp]) * page_bytes],
                        &t.kv[((size_t)l * n_pages + t.pt[lp]) * page_bytes], page_bytes) == 0);
  sv_config other = c; other.max_ctx = 512;
  Ctx o(other);
  CHECK(sv_clone_state(o.c, t.c) == SV_EINVAL);
  CHECK(sv_set_profile(t.c, 1 << 6) == SV_EINVAL && sv_set_profile(t.c, -1) == SV_EINVAL);
  CHECK(sv_set_profile(t.c, (1 << 6) - 1) == SV_OK && sv_set_profile(t.c, 0) == SV_OK);
  double ms = 0; int64_t launches = 0;
  CHECK(sv_profile_read(t.c, 6, &ms, &launches) == SV_EINVAL);
  CHECK(sv_profile_read(t.c, 0, &ms, &launches) == SV_OK);
}

static void test_batch() {
  sv_config c = tiny_cfg();
  const int V = c.vocab;
  Ctx a(c), b(c), m1(c), m2(c);
  std::vector<int32_t> pa = {1, 2, 3}, pb = {400, 401, 402, 403, 404, 405, 406};
  int32_t nx;
  CHECK(sv_prefill(a.c, pa.data(), 3, &nx) == SV_OK && sv_prefill(m1.c, pa.data(), 3, &nx) == SV_OK);
  CHECK(sv_prefill(b.c, pb.data(), 7, &nx) == SV_OK && sv_prefill(m2.c, pb.data(), 7, &nx) == SV_OK);
  sv_ctx* ctxs[2] = {a.c, b.c};
  int32_t pl[2] = {3, 7}, ks[2] = {3, 2};
  const int ca = sv_next_id(a.c), cb = sv_next_id(b.c);
  int32_t drafts[5] = {nxt(ca, V), 7, 9, nxt(cb, V), nxt(nxt(cb, V), V)};
  int32_t na[2], nn[2];
  // errors first: nothing changes
  sv_ctx* dup[2] = {a.c, a.c};
  CHECK(sv_verify_batch(dup, 2, pl, ks, drafts, na, nn) == SV_EINVAL);
  int32_t plbad[2] = {3, 6};
  CHECK(sv_verify_batch(ctxs, 2, plbad, ks, drafts, na, nn) == SV_ESTATE);
  int32_t ksbad[2] = {3, 9};
  CHECK(sv_verify_batch(ctxs, 2, pl, ksbad, drafts, na, nn) == SV_EINVAL);
  CHECK(sv_verify_batch(ctxs, 0, pl, ks, drafts, na, nn) == SV_EINVAL);
  CHECK(sv_kv_len(a.c) == 3 && sv_kv_len(b.c) == 7);
  CHECK(sv_verify_batch(ctxs, 2, pl, ks, drafts, na, nn) == SV_OK);
  int32_t n1, x1, n2, x2;
  CHECK(sv_verify(m1.c, 3, drafts, 3, &n1, &x1) == SV_OK && sv_verify(m2.c, 7, drafts + 3, 2, &n2, &x2) == SV_OK);
  CHECK(na[0] == n1 && nn[0] == x1 && na[1] == n2 && nn[1] == x2);
  CHECK(n1 == 1 && n2 == 2);
  CHECK(sv_kv_len(a.c) == sv_kv_len(m1.c) && sv_kv_len(b.c) == sv_kv_len(m2.c));
  std::vector<int32_t> h1(sv_kv_len(a.c)), h2(sv_kv_len(a.c));
  CHECK(sv_history(a.c, h1.data(), (int)h1.size()) == SV_OK && sv_history(m1.c, h2.data(), (int)h2.size()) == SV_OK);
  CHECK(h1 == h2);
  sv_config other = c; other.vocab = 1024;
  Ctx o(other);
  int32_t po[1] = {5};
  CHECK(sv_prefill(o.c, po, 1, &nx) == SV_OK);
  sv_ctx* mixed[2] = {a.c, o.c};
  int32_t plm[2] = {sv_kv_len(a.c), 1}, km[2] = {0, 0};
  CHECK(sv_verify_batch(mixed, 2, plm, km, nullptr, na, nn) == SV_EINVAL);
}

static void test_noalloc() {
  sv_config c = tiny_cfg();
  const int V = c.vocab;
  Ctx a(c), b(c);
  std::vector<int32_t> p = {10, 11, 12, 13, 14};
  int32_t nx, n1, x1, n2, x2;
  CHECK(sv_prefill(a.c, p.data(), 5, &nx) == SV_OK && sv_prefill(b.c, p.data(), 5, &nx) == SV_OK);
  int32_t dr[3] = {nxt(nx, V), 77, 3};
  CHECK(sv_verify(a.c, 5, dr, 3, &n1, &x1) == SV_OK && sv_verify_noalloc(b.c, 5, dr, 3, &n2, &x2) == SV_OK);
  CHECK(n1 == n2 && x1 == x2 && n1 == 1 && sv_kv_len(a.c) == sv_kv_len(b.c));
  CHECK(sv_verify_noalloc(b.c, 4, dr, 3, &n2, &x2) == SV_ESTATE);
  // the 8B shape at a 32K context: 33 rows of 64 splits need more than 32 MiB, 28 rows fit
  sv_config s{};
  s.n_layers = 1; s.d_model = 4096; s.n_q_heads = 32; s.n_kv_heads = 8; s.head_dim = 128; s.d_ff = 12288;
  s.vocab = 2048; s.tied = 1; s.rms_eps = 1e-6f; s.rope_theta = 1e4f; s.page_size = 16; s.max_ctx = 32768;
  s.max_k = 32;
  Ctx big(s);
  CHECK(big.status == SV_OK);
  std::vector<int32_t> hist(32704, 1);
  CHECK(sv_restore(big.c, 32704, hist.data()) == SV_OK);
  std::vector<int32_t> d32(32, 5);
  CHECK(sv_verify_noalloc(big.c, 32704, d32.data(), 32, &n2, &x2) == SV_ESCRATCH && sv_kv_len(big.c) == 32704);
  CHECK(sv_verify_noalloc(big.c, 32704, d32.data(), 28, &n2, &x2) == SV_ESCRATCH && sv_kv_len(big.c) == 32704);
  CHECK(sv_verify_noalloc(big.c, 32704, d32.data(), 27, &n2, &x2) == SV_OK && sv_kv_len(big.c) == 32705 + n2);
}

int main() {
  setenv("SV_NO_GRAPH", "1", 1);
  test_config_checks();
  test_create_checks();
  test_prefill_decode_verify_truncate();
  test_restore_observer_audit();
  test_batch();
  test_noalloc();
  if (g_fail) {
    std::fprintf(stderr, "%d check(s) failed\n", g_fail);
    return 1;
  }
  std::printf("host logic ok\n");
  return 0;
}
