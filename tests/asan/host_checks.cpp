// Host-side checks of libfa's C ABI, built with AddressSanitizer and
// UndefinedBehaviorSanitizer on the host code and run without a GPU.
//
// Every entry point checks its arguments on the host before anything is
// enqueued. This program drives those checks, the size and split functions
// and fa_check_cu_seqlens over many cases: arrays sit in heap blocks of
// exactly their size, so a read or write past one is a sanitizer report, and
// each status is compared with the one the header documents. With no device
// present, a call whose arguments pass reaches the HIP runtime and must come
// back as FA_ERR_HIP (in an FA_DEBUG build, already at the cu_seqlens copy).
// Prints "host checks ok: <n> cases" and exits 0 when every case holds.
#include <climits>
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <initializer_list>
#include <random>
#include <vector>

#include "fa.h"

namespace {

int g_cases = 0, g_fail = 0;

void expect(bool ok, const char* what, int line, long long got = 0) {
  ++g_cases;
  if (!ok) {
    ++g_fail;
    std::fprintf(stderr, "FAIL line %d: %s (got %lld)\n", line, what, got);
  }
}
#define EXPECT_ST(call, want) \
  do { const int st_ = (call); expect(st_ == (want), #call " == " #want, __LINE__, st_); } while (0)
#define EXPECT(cond) expect((cond), #cond, __LINE__)

// fa_check_cu_seqlens on a copy of `v` in a heap block of exactly v.size() entries
int cu_check(const std::vector<int32_t>& v, int B, int N) {
  int32_t* p = static_cast<int32_t*>(std::malloc(sizeof(int32_t) * (v.empty() ? 1 : v.size())));
  if (!v.empty()) std::memcpy(p, v.data(), sizeof(int32_t) * v.size());
  const int st = fa_check_cu_seqlens(p, B, N);
  std::free(p);
  return st;
}

// The condition written out on its own: entry 0 is 0, every length in [0, N].
bool cu_valid(const std::vector<int32_t>& v, int N) {
  if (v.empty() || v[0] != 0) return false;
  for (size_t s = 1; s < v.size(); ++s) {
    const long long len = (long long)v[s] - v[s - 1];
    if (len < 0 || len > N) return false;
  }
  return true;
}

void cu_seqlens_cases() {
  EXPECT_ST(cu_check({0}, 0, 0), FA_OK);
  EXPECT_ST(cu_check({0, 5}, 1, 5), FA_OK);
  EXPECT_ST(cu_check({0, 5}, 1, 4), FA_ERR_INVALID_ARG);          // longer than N
  EXPECT_ST(cu_check({1, 5}, 1, 8), FA_ERR_INVALID_ARG);          // first entry not 0
  EXPECT_ST(cu_check({0, 5, 3}, 2, 8), FA_ERR_INVALID_ARG);       // decreasing
  EXPECT_ST(cu_check({0, 0, 0, 7}, 3, 7), FA_OK);                 // empty sequences
  EXPECT_ST(cu_check({0, INT_MAX}, 1, INT_MAX), FA_OK);
  EXPECT_ST(cu_check({0, INT_MAX, INT_MIN}, 2, INT_MAX), FA_ERR_INVALID_ARG);  // no wrap-around
  EXPECT_ST(cu_check({0, -1}, 1, 4), FA_ERR_INVALID_ARG);
  EXPECT_ST(fa_check_cu_seqlens(nullptr, 1, 4), FA_ERR_INVALID_ARG);
  EXPECT_ST(cu_check({0, 1}, -1, 4), FA_ERR_INVALID_ARG);
  EXPECT_ST(cu_check({0, 1}, 1, -1), FA_ERR_INVALID_ARG);
  // random arrays, about half of them valid, against the condition above
  std::mt19937 rng(12345);
  for (int it = 0; it < 4000; ++it) {
    const int B = (int)(rng() % 40);
    const int N = (int)(rng() % 300);
    std::vector<int32_t> v(B + 1, 0);
    for (int s = 0; s < B; ++s) v[s + 1] = v[s] + (N ? (int32_t)(rng() % (N + 1)) : 0);
    if (rng() % 2 && B > 0) {   // one corrupted entry
      const int i = (int)(rng() % (B + 1));
      v[i] += (int32_t)(rng() % 7) - 3;
    }
    EXPECT_ST(cu_check(v, B, N), cu_valid(v, N) ? FA_OK : FA_ERR_INVALID_ARG);
  }
}

// 16-byte aligned host blocks standing in for device tensors: the argument
// checks only look at the addresses, and no launch gets past the runtime.
struct Buffers {
  std::vector<void*> all;
  void* get(size_t bytes) {
    void* p = std::aligned_alloc(256, (bytes + 255) / 256 * 256);
    all.push_back(p);
    return p;
  }
  ~Buffers() {
    for (void* p : all) std::free(p);
  }
};

void forward_cases(Buffers& m) {
  const int B = 2, H = 4, N = 64, d = 128;
  const size_t t = (size_t)B * N * H * d * 2;
  void *q = m.get(t), *k = m.get(t), *v = m.get(t), *o = m.get(t);
  float* lse = static_cast<float*>(m.get((size_t)H * B * N * 4));
  const float sc = 0.125f;
  EXPECT_ST(fa_fwd(q, k, v, o, lse, B, H, H, N, d, sc, 1, nullptr, (fa_dtype)7, nullptr),
            FA_ERR_INVALID_ARG);
  EXPECT_ST(fa_fwd(q, k, v, o, lse, B, H, H, N, 96, sc, 1, nullptr, FA_BF16, nullptr),
            FA_ERR_UNSUPPORTED);
  EXPECT_ST(fa_fwd(q, k, v, o, lse, B, 6, 4, N, d, sc, 1, nullptr, FA_BF16, nullptr),
            FA_ERR_INVALID_ARG);                                   // Hq % Hkv != 0
  EXPECT_ST(fa_fwd(q, k, v, o, lse, B, H, H, N, d, NAN, 1, nullptr, FA_BF16, nullptr),
            FA_ERR_INVALID_ARG);
  EXPECT_ST(fa_fwd(q, k, v, o, lse, B, H, H, N, d, -sc, 1, nullptr, FA_BF16, nullptr),
            FA_ERR_INVALID_ARG);
  EXPECT_ST(fa_fwd(q, k, v, o, lse, B, H, H, N, d, sc, 2, nullptr, FA_BF16, nullptr),
            FA_ERR_INVALID_ARG);
  EXPECT_ST(fa_fwd(q, k, v, o, lse, -1, H, H, N, d, sc, 1, nullptr, FA_BF16, nullptr),
            FA_ERR_INVALID_ARG);
  EXPECT_ST(fa_fwd(static_cast<char*>(q) + 2, k, v, o, lse, B, H, H, N, d, sc, 1, nullptr,
                   FA_BF16, nullptr), FA_ERR_INVALID_ARG);        // misaligned
  EXPECT_ST(fa_fwd(nullptr, k, v, o, lse, B, H, H, N, d, sc, 1, nullptr, FA_BF16, nullptr),
            FA_ERR_INVALID_ARG);
  EXPECT_ST(fa_fwd(nullptr, nullptr, nullptr, nullptr, nullptr, 0, H, H, N, d, sc, 1, nullptr,
                   FA_BF16, nullptr), FA_OK);                     // B = 0: nothing to do
  EXPECT_ST(fa_fwd(q, k, v, o, lse, B, H, H, 0, d, sc, 0, nullptr, FA_FP16, nullptr), FA_OK);
  // past the argument checks: no device, so the runtime refuses
  EXPECT_ST(fa_fwd(q, k, v, o, lse, B, H, H, N, d, sc, 1, nullptr, FA_BF16, nullptr), FA_ERR_HIP);
  int32_t* cu = static_cast<int32_t*>(m.get(3 * sizeof(int32_t)));
  cu[0] = 0; cu[1] = 40; cu[2] = 100;
  EXPECT_ST(fa_fwd(q, k, v, o, lse, B, H, H, N, d, sc, 1, cu, FA_BF16, nullptr), FA_ERR_HIP);

  EXPECT_ST(fa_fwd_window(q, k, v, o, lse, B, H, H, N, d, sc, -2, 0, nullptr, FA_BF16, nullptr),
            FA_ERR_INVALID_ARG);
  EXPECT_ST(fa_fwd_window(q, k, v, o, lse, B, H, H, N, d, sc, 3, -3, nullptr, FA_BF16, nullptr),
            FA_ERR_INVALID_ARG);
  EXPECT_ST(fa_fwd_softcap(q, k, v, o, lse, B, H, H, N, d, sc, 1, -1.f, nullptr, FA_BF16, nullptr),
            FA_ERR_INVALID_ARG);
  EXPECT_ST(fa_fwd_softcap(q, k, v, o, lse, B, H, H, N, d, sc, 1, INFINITY, nullptr, FA_BF16,
                           nullptr), FA_ERR_INVALID_ARG);
  EXPECT_ST(fa_fwd_dropout(q, k, v, o, lse, B, H, H, N, d, sc, 1, 1.f, 7, nullptr, FA_BF16,
                           nullptr), FA_ERR_INVALID_ARG);
  EXPECT_ST(fa_fwd_dropout(q, k, v, o, lse, B, H, H, N, d, sc, 1, NAN, 7, nullptr, FA_BF16,
                           nullptr), FA_ERR_INVALID_ARG);
  EXPECT_ST(fa_fwd_window_softcap(q, k, v, o, lse, B, H, H, N, d, sc, 8, 8, -2.f, nullptr,
                                  FA_BF16, nullptr), FA_ERR_INVALID_ARG);
  // kvlen: exactly one cu_seqlens given
  EXPECT_ST(fa_fwd_kvlen(q, k, v, o, lse, B, H, H, N, N, d, sc, 1, cu, nullptr, FA_BF16, nullptr),
            FA_ERR_INVALID_ARG);
  EXPECT_ST(fa_fwd_kvlen(q, k, v, o, lse, B, H, H, N, N, d, sc, 1, nullptr, cu, FA_BF16, nullptr),
            FA_ERR_INVALID_ARG);
  // fp8: descales must be finite and > 0
  EXPECT_ST(fa_fwd_fp8(q, k, v, o, lse, B, H, H, N, d, sc, 1, nullptr, 0.f, 1.f, 1.f, FA_BF16,
                       nullptr), FA_ERR_INVALID_ARG);
  EXPECT_ST(fa_fwd_fp8(q, k, v, o, lse, B, H, H, N, d, sc, 1, nullptr, 1.f, NAN, 1.f, FA_BF16,
                       nullptr), FA_ERR_INVALID_ARG);
}

// fa_fwd_ex / fa_bwd_ex: the options struct sits in a heap block of exactly its size, so
// a read past it is reported
void options_cases(Buffers& m) {
  const int B = 2, H = 4, N = 64, d = 128;
  const size_t t = (size_t)B * N * H * d * 2;
  void *q = m.get(t), *k = m.get(t), *v = m.get(t), *o = m.get(t), *dout = m.get(t);
  void *dq = m.get(t), *dk = m.get(t), *dv = m.get(t);
  float* lse = static_cast<float*>(m.get((size_t)H * B * N * 4));
  const size_t wsb = fa_bwd_workspace_size(B, H, H, N, d);
  void* ws = m.get(wsb);
  const float sc = 0.125f;
  fa_attn_options* op = static_cast<fa_attn_options*>(m.get(sizeof(fa_attn_options)));
  auto set = [&](int mask, int wl, int wr, float cap, float p) {
    op->struct_size = sizeof(fa_attn_options);
    op->mask = (fa_mask)mask;
    op->window_left = wl;
    op->window_right = wr;
    op->softcap = cap;
    op->dropout_p = p;
    op->dropout_seed = 11;
  };
  auto fwd = [&](const fa_attn_options* x) {
    return fa_fwd_ex(q, k, v, o, lse, B, H, H, N, d, sc, x, nullptr, FA_BF16, nullptr);
  };
  auto bwd = [&](const fa_attn_options* x) {
    return fa_bwd_ex(q, k, v, o, dout, lse, dq, dk, dv, B, H, H, N, d, sc, x, nullptr, FA_BF16,
                     ws, wsb, nullptr);
  };
  EXPECT_ST(fwd(nullptr), FA_ERR_INVALID_ARG);
  EXPECT_ST(bwd(nullptr), FA_ERR_INVALID_ARG);
  set(FA_MASK_CAUSAL, -1, -1, 0.f, 0.f);
  op->struct_size = sizeof(fa_attn_options) - 8;
  EXPECT_ST(fwd(op), FA_ERR_INVALID_ARG);                        // struct too small
  set(3, -1, -1, 0.f, 0.f);
  EXPECT_ST(fwd(op), FA_ERR_INVALID_ARG);                        // no such mask
  EXPECT_ST(bwd(op), FA_ERR_INVALID_ARG);
  set(FA_MASK_WINDOW, 8, 0, 0.f, 0.2f);
  EXPECT_ST(fwd(op), FA_ERR_UNSUPPORTED);                        // dropout with a window
  set(FA_MASK_CAUSAL, -1, -1, 5.f, 0.2f);
  EXPECT_ST(bwd(op), FA_ERR_UNSUPPORTED);                        // dropout with a soft cap
  set(FA_MASK_WINDOW, -2, 0, 0.f, 0.f);
  EXPECT_ST(fwd(op), FA_ERR_INVALID_ARG);                        // the window entry's check
  set(FA_MASK_NONE, -1, -1, -1.f, 0.f);
  EXPECT_ST(fwd(op), FA_ERR_INVALID_ARG);                        // the soft-cap entry's check
  set(FA_MASK_CAUSAL, -1, -1, 0.f, 0.f);
  EXPECT_ST(bwd(op), FA_ERR_HIP);                                 // past the checks
  const int routes[5][5] = {{FA_MASK_NONE, -1, -1, 0, 0}, {FA_MASK_WINDOW, 16, 0, 0, 0},
                            {FA_MASK_CAUSAL, -1, -1, 1, 0}, {FA_MASK_WINDOW, 8, 8, 1, 0},
                            {FA_MASK_CAUSAL, -1, -1, 0, 1}};
  for (const auto& r : routes) {
    set(r[0], r[1], r[2], r[3] ? 30.f : 0.f, r[4] ? 0.1f : 0.f);
    EXPECT_ST(fwd(op), FA_ERR_HIP);
    EXPECT_ST(bwd(op), FA_ERR_HIP);
  }
}

void backward_cases(Buffers& m) {
  const int B = 2, H = 4, N = 64, d = 128;
  const size_t t = (size_t)B * N * H * d * 2;
  void *q = m.get(t), *k = m.get(t), *v = m.get(t), *o = m.get(t), *dout = m.get(t);
  void *dq = m.get(t), *dk = m.get(t), *dv = m.get(t);
  float* lse = static_cast<float*>(m.get((size_t)H * B * N * 4));
  const float sc = 0.125f;
  const size_t ws_bytes = fa_bwd_workspace_size(B, H, H, N, d);
  EXPECT(ws_bytes > 0);
  void* ws = m.get(ws_bytes);
  EXPECT_ST(fa_bwd(q, k, v, o, dout, lse, dq, dk, dv, B, H, H, N, d, sc, 1, nullptr, FA_BF16,
                   ws, ws_bytes - 1, nullptr), FA_ERR_WORKSPACE);
  EXPECT_ST(fa_bwd(q, k, v, o, dout, lse, dq, dk, dv, B, H, H, N, d, sc, 1, nullptr, FA_BF16,
                   nullptr, ws_bytes, nullptr), FA_ERR_WORKSPACE);
  EXPECT_ST(fa_bwd(q, k, v, o, dout, lse, dq, dk, dv, B, H, H, N, 80, sc, 1, nullptr, FA_BF16,
                   ws, ws_bytes, nullptr), FA_ERR_UNSUPPORTED);
  EXPECT_ST(fa_bwd(q, k, v, o, dout, lse, nullptr, dk, dv, B, H, H, N, d, sc, 1, nullptr,
                   FA_BF16, ws, ws_bytes, nullptr), FA_ERR_INVALID_ARG);
  const int ns = fa_bwd_num_stages();
  EXPECT(ns >= 1);
  EXPECT_ST(fa_bwd_stage(ns, q, k, v, o, dout, lse, dq, dk, dv, B, H, H, N, d, sc, 1, nullptr,
                         FA_BF16, ws, ws_bytes, nullptr), FA_ERR_INVALID_ARG);
  EXPECT_ST(fa_bwd_stage(-2, q, k, v, o, dout, lse, dq, dk, dv, B, H, H, N, d, sc, 1, nullptr,
                         FA_BF16, ws, ws_bytes, nullptr), FA_ERR_INVALID_ARG);
  EXPECT_ST(fa_bwd(q, k, v, o, dout, lse, dq, dk, dv, B, H, H, N, d, sc, 1, nullptr, FA_BF16,
                   ws, ws_bytes, nullptr), FA_ERR_HIP);
  // allocation-free variant: Hq·(B·N + 64) beyond 4,194,304 before any HIP call
  EXPECT_ST(fa_bwd_noalloc(q, k, v, o, dout, lse, dq, dk, dv, 1, 64, 64, 65536, d, sc, 1,
                           nullptr, FA_BF16, nullptr), FA_ERR_WORKSPACE);
  EXPECT_ST(fa_bwd_noalloc(q, k, v, o, dout, lse, dq, dk, dv, B, H, H, N, d, sc, 1, nullptr,
                           FA_BF16, nullptr), FA_ERR_HIP);
  EXPECT_ST(fa_bwd_dropout(q, k, v, o, dout, lse, dq, dk, dv, B, H, H, N, d, sc, 1, -0.5f, 1,
                           nullptr, FA_BF16, ws, ws_bytes, nullptr), FA_ERR_INVALID_ARG);
  EXPECT_ST(fa_bwd_window(q, k, v, o, dout, lse, dq, dk, dv, B, H, H, N, d, sc, -5, 0, nullptr,
                          FA_BF16, ws, ws_bytes, nullptr), FA_ERR_INVALID_ARG);
  int32_t* cu = static_cast<int32_t*>(m.get(3 * sizeof(int32_t)));
  cu[0] = 0; cu[1] = 10; cu[2] = 20;
  EXPECT_ST(fa_bwd_kvlen(q, k, v, o, dout, lse, dq, dk, dv, B, H, H, N, N, d, sc, 1, cu, nullptr,
                         FA_BF16, ws, ws_bytes, nullptr), FA_ERR_INVALID_ARG);
}

void size_cases() {
  // the workspace bound grows with every size and is 0 on bad ones
  EXPECT(fa_bwd_workspace_size(-1, 4, 4, 64, 128) == 0);
  EXPECT(fa_bwd_workspace_size(1, 4, 3, 64, 128) == 0);
  size_t prev = 0;
  for (int n = 1; n <= 1 << 16; n *= 2) {   // 256-byte granules: equal for small n
    const size_t s = fa_bwd_workspace_size(2, 8, 2, n, 128);
    EXPECT(s >= prev && s % 256 == 0 && s >= 2 * 8 * (2 * (size_t)n + 64) * sizeof(float));
    prev = s;
  }
  for (int d : {64, 128, 256})
    for (int nk : {1, 100, 4096, 65536}) {
      const int s = fa_kvcache_num_splits(4, 32, 8, 1, nk, d);
      EXPECT(s >= 1 && s <= 256);
      const int s8 = fa_kvcache_fp8_num_splits(4, 32, 8, 1, nk, d);
      EXPECT(s8 >= 1 && s8 <= 256);
      EXPECT(fa_fwd_kvcache_workspace_size(4, 32, 8, 1, nk, d, 0) > 0);
      EXPECT(fa_fwd_kvcache_workspace_size(4, 32, 8, 1, nk, d, -1) == 0);
      EXPECT(fa_fwd_kvcache_workspace_size(4, 32, 8, 1, nk, d, 300) >=
             fa_fwd_kvcache_workspace_size(4, 32, 8, 1, nk, d, 0));
    }
  for (int st = -8; st <= 8; ++st) {
    const char* s = fa_status_string(st);
    EXPECT(s != nullptr && std::strlen(s) > 0);
  }
}

void decode_cases(Buffers& m) {
  const int B = 2, Hq = 8, Hkv = 2, Nq = 1, Nk = 256, d = 128;
  void* q = m.get((size_t)B * Nq * Hq * d * 2);
  void* kc = m.get((size_t)B * Nk * Hkv * d * 2);
  void* vc = m.get((size_t)B * Nk * Hkv * d * 2);
  int32_t* lens = static_cast<int32_t*>(m.get(B * sizeof(int32_t)));
  lens[0] = 100; lens[1] = 256;
  void* o = m.get((size_t)B * Nq * Hq * d * 2);
  float* lse = static_cast<float*>(m.get((size_t)Hq * B * Nq * 4));
  const size_t wsb = fa_fwd_kvcache_workspace_size(B, Hq, Hkv, Nq, Nk, d, 0);
  void* ws = m.get(wsb);
  EXPECT_ST(fa_fwd_kvcache(q, kc, vc, nullptr, o, lse, B, Hq, Hkv, Nq, Nk, d, 0.1f, 1, 0, FA_BF16,
                           ws, wsb, nullptr), FA_ERR_INVALID_ARG);
  EXPECT_ST(fa_fwd_kvcache(q, kc, vc, lens, o, lse, B, Hq, Hkv, Nq, Nk, d, 0.1f, 1, 0, FA_BF16,
                           ws, 16, nullptr), FA_ERR_WORKSPACE);
  EXPECT_ST(fa_fwd_kvcache_stage(5, q, kc, vc, lens, o, lse, B, Hq, Hkv, Nq, Nk, d, 0.1f, 1, 0,
                                 FA_BF16, ws, wsb, nullptr), FA_ERR_INVALID_ARG);
  EXPECT_ST(fa_fwd_kvcache_local(q, kc, vc, lens, o, lse, B, Hq, Hkv, Nq, Nk, d, 0.1f, 1, -3,
                                 0.f, 0, FA_BF16, ws, wsb, nullptr), FA_ERR_INVALID_ARG);
  EXPECT_ST(fa_fwd_kvcache(q, kc, vc, lens, o, lse, B, Hq, Hkv, Nq, Nk, d, 0.1f, 1, 0, FA_BF16,
                           ws, wsb, nullptr), FA_ERR_HIP);
}

}  // namespace

int main() {
  Buffers m;
  cu_seqlens_cases();
  forward_cases(m);
  options_cases(m);
  backward_cases(m);
  size_cases();
  decode_cases(m);
  if (g_fail) {
    std::fprintf(stderr, "%d of %d host checks failed\n", g_fail, g_cases);
    return 1;
  }
  std::printf("host checks ok: %d cases\n", g_cases);
  return 0;
}
