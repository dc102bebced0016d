// C ABI of libfa.so (declared in include/fa.h): argument checks, then the
// kernel launches. Nothing here allocates device memory. The global state is
// the cache of the decode kernel's occupancy figures (decode_residency),
// filled once per process with values that are the same for every caller,
// and fa_bwd_noalloc's fixed device array `scratch` with its per-device
// addresses. Built with FA_DEBUG defined, every cu_seqlens argument is
// copied to the host and checked before the launch, and every launch is
// followed by a synchronisation that reports a failed kernel.
#include <algorithm>
#include <atomic>
#include <mutex>
#include <cmath>
#include <cstddef>
#include <cstdint>

#include "fa.h"
#include "fa_kernels.h"

#ifdef FA_DEBUG
#include <vector>
#endif

namespace {

// The status of a call whose launches returned `e`. Debug builds also wait for
// the work and report a kernel that failed.
int launched(hipError_t e, hipStream_t stream) {
  if (e != hipSuccess) return FA_ERR_HIP;
#ifdef FA_DEBUG
  if (hipStreamSynchronize(stream) != hipSuccess || hipGetLastError() != hipSuccess)
    return FA_ERR_HIP;
#else
  (void)stream;
#endif
  return FA_OK;
}

// Debug builds: fa_check_cu_seqlens on a host copy of the device array `cu`
// (B+1 entries, lengths at most N). Release builds: FA_OK without reading it.
int debug_cu_seqlens(const int32_t* cu, int B, int N, hipStream_t stream) {
#ifdef FA_DEBUG
  if (cu == nullptr || B <= 0) return FA_OK;
  std::vector<int32_t> h((size_t)B + 1);
  if (hipMemcpyAsync(h.data(), cu, h.size() * sizeof(int32_t), hipMemcpyDeviceToHost, stream) !=
          hipSuccess ||
      hipStreamSynchronize(stream) != hipSuccess)
    return FA_ERR_HIP;
  return fa_check_cu_seqlens(h.data(), B, N);
#else
  (void)cu;
  (void)B;
  (void)N;
  (void)stream;
  return FA_OK;
#endif
}

constexpr float kLog2e = 1.4426950408889634f;

// Checks shared by fa_fwd and fa_bwd that need no pointer. Returns FA_OK or
// the status to report; *noop is set when there is nothing to compute.
int check_sizes(int B, int Hq, int Hkv, int N, int d, float scale, int causal, int dtype,
                bool* noop, int max_d = 128) {
  *noop = false;
  if (dtype != FA_FP16 && dtype != FA_BF16) return FA_ERR_INVALID_ARG;
  if (B < 0 || N < 0 || Hq <= 0 || Hkv <= 0 || d <= 0) return FA_ERR_INVALID_ARG;
  if (Hq % Hkv != 0) return FA_ERR_INVALID_ARG;
  if (causal != 0 && causal != 1) return FA_ERR_INVALID_ARG;
  if (!std::isfinite(scale) || !(scale > 0.f)) return FA_ERR_INVALID_ARG;
  if (d != 64 && d != 128 && !(d == 256 && max_d >= 256)) return FA_ERR_UNSUPPORTED;
  // token and grid indices are 32-bit inside the kernels
  const int64_t T = (int64_t)B * N;
  if (T >= (int64_t)1 << 31 || T * Hq >= (int64_t)1 << 31) return FA_ERR_UNSUPPORTED;
  if (B == 0 || N == 0) *noop = true;
  return FA_OK;
}

// The kernels move 16-byte vectors; device pointers must be 16-byte aligned.
bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// A sliding window (left, right), −1 = unbounded, as a mask mode and bounds
// clamped to N. Returns FA_OK, or the status to report for a bad pair.
int window_mode(int left, int right, int N, int* mask, int* wl, int* wr) {
  if (left < -1 || right < -1) return FA_ERR_INVALID_ARG;
  *wl = *wr = 0;
  if (left < 0 && right < 0) {
    *mask = fa::kMaskNone;
  } else if (left < 0 && right == 0) {
    *mask = fa::kMaskCausal;       // the causal kernels, tuned for this band
  } else {
    *mask = fa::kMaskWindow;
    // q0 + 128 + wr must stay inside int: keep N and the bounds below 2^30
    if (N >= (1 << 30)) return FA_ERR_UNSUPPORTED;
    *wl = left < 0 ? N : std::min(left, N);
    *wr = right < 0 ? N : std::min(right, N);
  }
  return FA_OK;
}

// A soft cap c: 0 = none; otherwise finite and > 0, with scale / c finite
// (any mask, any supported head dimension). Sets the kernels' two
// constants (scale / c and c·log2 e). Returns FA_OK or the status to report.
int cap_constants(float softcap, float scale, int mask, int d, float* cap_in, float* cap_out) {
  *cap_in = *cap_out = 0.f;
  if (softcap == 0.f) return FA_OK;
  if (!std::isfinite(softcap) || !(softcap > 0.f)) return FA_ERR_INVALID_ARG;
  *cap_in = scale / softcap;
  *cap_out = softcap * kLog2e;
  if (!std::isfinite(*cap_in) || !std::isfinite(*cap_out)) return FA_ERR_INVALID_ARG;
  (void)mask;   // every mask, a window included
  (void)d;      // every supported head dimension, 256 included
  return FA_OK;
}

// Dropout probability p: 0 = none; otherwise 0 < p < 1 with keep threshold
// t = floor(256·(1 − p) + 1/2) >= 1, only with the unmasked or causal mask
// (any supported head dimension). Returns FA_OK or the status to report.
int drop_constants(float p, int mask, int d, uint32_t* t) {
  *t = 256;
  if (p == 0.f) return FA_OK;
  if (!std::isfinite(p) || !(p > 0.f) || !(p < 1.f)) return FA_ERR_INVALID_ARG;
  const double x = std::floor(256.0 * (1.0 - (double)p) + 0.5);
  if (x < 1.0) return FA_ERR_INVALID_ARG;
  *t = (uint32_t)std::min(x, 256.0);
  (void)d;   // every supported head dimension, 256 included
  if (mask == fa::kMaskWindow) return FA_ERR_UNSUPPORTED;
  return FA_OK;
}

int fwd_common(const void* q, const void* k, const void* v, void* o, float* lse, int B, int Hq,
               int Hkv, int N, int d, float scale, int mask, int wl, int wr,
               const int32_t* cu_seqlens, int dtype, hipStream_t stream, float softcap = 0.f,
               float dropout_p = 0.f, uint64_t seed = 0) {
  bool noop;
  int st = check_sizes(B, Hq, Hkv, N, d, scale, 0, dtype, &noop, 256);
  if (st != FA_OK) return st;
  float cap_in, cap_out;
  st = cap_constants(softcap, scale, mask, d, &cap_in, &cap_out);
  if (st != FA_OK) return st;
  uint32_t keep_t;
  st = drop_constants(dropout_p, mask, d, &keep_t);
  if (st != FA_OK || noop) return st;
  if (!q || !k || !v || !o || !lse) return FA_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(lse))
    return FA_ERR_INVALID_ARG;
  fa::FwdArgs a;
  a.q = q;
  a.k = k;
  a.v = v;
  a.o = o;
  a.lse = lse;
  a.cu_seqlens = cu_seqlens;
  a.B = B;
  a.Hq = Hq;
  a.Hkv = Hkv;
  a.N = N;
  a.group = Hq / Hkv;
  const int br = fa::fwd_query_tile();
  a.n_qtiles = (N + br - 1) / br;
  a.scale_log2 = scale * kLog2e;
  a.wl = wl;
  a.wr = wr;
  a.cap_in = cap_in;
  a.cap_out = cap_out;
  a.seed_lo = (uint32_t)seed;
  a.seed_hi = (uint32_t)(seed >> 32);
  a.keep_t = keep_t;
  a.drop_scale = 256.f / (float)keep_t;
  if ((int64_t)a.n_qtiles * Hq * B >= (int64_t)1 << 31) return FA_ERR_UNSUPPORTED;
  st = debug_cu_seqlens(cu_seqlens, B, N, stream);
  if (st != FA_OK) return st;
  hipError_t e = fa::launch_fwd(a, dtype == FA_BF16, d, mask, cu_seqlens != nullptr,
                                softcap != 0.f, dropout_p != 0.f, stream);
  return launched(e, stream);
}

}  // namespace

extern "C" {

int fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int B, int Hq,
           int Hkv, int N, int d, float scale, int causal, const int32_t* cu_seqlens, fa_dtype dtype,
           hipStream_t stream) {
  if (causal != 0 && causal != 1) return FA_ERR_INVALID_ARG;
  return fwd_common(q, k, v, o, lse, B, Hq, Hkv, N, d, scale,
                    causal ? fa::kMaskCausal : fa::kMaskNone, 0, 0, cu_seqlens, dtype, stream);
}

int fa_fwd_kvlen(const void* q, const void* k, const void* v, void* o, float* lse, int B, int Hq,
                 int Hkv, int Nq, int Nk, int d, float scale, int causal,
                 const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k, fa_dtype dtype,
                 hipStream_t stream) {
  const bool varlen = cu_seqlens_q != nullptr;
  if (varlen != (cu_seqlens_k != nullptr)) return FA_ERR_INVALID_ARG;
  bool noop;
  int st = check_sizes(B, Hq, Hkv, Nq, d, scale, causal, dtype, &noop, 256);
  if (st != FA_OK) return st;
  if (Nk < 0) return FA_ERR_INVALID_ARG;
  if ((int64_t)B * Nk >= (int64_t)1 << 31) return FA_ERR_UNSUPPORTED;
  if (noop) return FA_OK;   // no query
  if (!q || !o || !lse) return FA_ERR_INVALID_ARG;
  if (Nk > 0 && (!k || !v)) return FA_ERR_INVALID_ARG;   // with Nk = 0 no key is read
  const void* ptrs[] = {q, k, v, o, lse};
  for (const void* p : ptrs)
    if (p && !aligned16(p)) return FA_ERR_INVALID_ARG;
  fa::FwdArgs a;
  a.q = q;
  a.k = k;
  a.v = v;
  a.o = o;
  a.lse = lse;
  a.cu_seqlens = cu_seqlens_q;
  a.cu_seqlens_k = cu_seqlens_k;
  a.B = B;
  a.Hq = Hq;
  a.Hkv = Hkv;
  a.N = Nq;
  a.Nk = Nk;
  a.group = Hq / Hkv;
  const int br = fa::fwd_query_tile();
  a.n_qtiles = (Nq + br - 1) / br;
  a.scale_log2 = scale * kLog2e;
  a.wl = a.wr = 0;
  a.cap_in = a.cap_out = 0.f;
  a.seed_lo = a.seed_hi = 0;
  a.keep_t = 256;
  a.drop_scale = 1.f;
  if ((int64_t)a.n_qtiles * Hq * B >= (int64_t)1 << 31) return FA_ERR_UNSUPPORTED;
  if (varlen) {
    int st = debug_cu_seqlens(cu_seqlens_q, B, Nq, stream);
    if (st == FA_OK) st = debug_cu_seqlens(cu_seqlens_k, B, Nk, stream);
    if (st != FA_OK) return st;
  }
  hipError_t e = fa::launch_fwd_kvlen(a, dtype == FA_BF16, d, causal != 0, varlen, stream);
  return launched(e, stream);
}

int fa_fwd_softcap(const void* q, const void* k, const void* v, void* o, float* lse, int B,
                   int Hq, int Hkv, int N, int d, float scale, int causal, float softcap,
                   const int32_t* cu_seqlens, fa_dtype dtype, hipStream_t stream) {
  if (causal != 0 && causal != 1) return FA_ERR_INVALID_ARG;
  return fwd_common(q, k, v, o, lse, B, Hq, Hkv, N, d, scale,
                    causal ? fa::kMaskCausal : fa::kMaskNone, 0, 0, cu_seqlens, dtype, stream,
                    softcap);
}

int fa_fwd_dropout(const void* q, const void* k, const void* v, void* o, float* lse, int B,
                   int Hq, int Hkv, int N, int d, float scale, int causal, float dropout_p,
                   uint64_t seed, const int32_t* cu_seqlens, fa_dtype dtype, hipStream_t stream) {
  if (causal != 0 && causal != 1) return FA_ERR_INVALID_ARG;
  return fwd_common(q, k, v, o, lse, B, Hq, Hkv, N, d, scale,
                    causal ? fa::kMaskCausal : fa::kMaskNone, 0, 0, cu_seqlens, dtype, stream, 0.f,
                    dropout_p, seed);
}

int fa_fwd_window_softcap(const void* q, const void* k, const void* v, void* o, float* lse,
                          int B, int Hq, int Hkv, int N, int d, float scale, int window_left,
                          int window_right, float softcap, const int32_t* cu_seqlens, fa_dtype dtype,
                          hipStream_t stream) {
  int mask, wl, wr;
  const int st = window_mode(window_left, window_right, N, &mask, &wl, &wr);
  if (st != FA_OK) return st;
  return fwd_common(q, k, v, o, lse, B, Hq, Hkv, N, d, scale, mask, wl, wr, cu_seqlens, dtype,
                    stream, softcap);
}

int fa_fwd_window(const void* q, const void* k, const void* v, void* o, float* lse, int B,
                  int Hq, int Hkv, int N, int d, float scale, int window_left, int window_right,
                  const int32_t* cu_seqlens, fa_dtype dtype, hipStream_t stream) {
  int mask, wl, wr;
  const int st = window_mode(window_left, window_right, N, &mask, &wl, &wr);
  if (st != FA_OK) return st;
  return fwd_common(q, k, v, o, lse, B, Hq, Hkv, N, d, scale, mask, wl, wr, cu_seqlens, dtype,
                    stream);
}

int fa_fwd_fp8(const void* q, const void* k, const void* v, void* o, float* lse, int B, int Hq,
               int Hkv, int N, int d, float scale, int causal, const int32_t* cu_seqlens,
               float descale_q, float descale_k, float descale_v, fa_dtype out_dtype,
               hipStream_t stream) {
  bool noop;
  int st = check_sizes(B, Hq, Hkv, N, d, scale, causal, out_dtype, &noop, 256);
  if (st != FA_OK) return st;
  for (float x : {descale_q, descale_k, descale_v})
    if (!std::isfinite(x) || !(x > 0.f)) return FA_ERR_INVALID_ARG;
  const float c = scale * descale_q * descale_k * kLog2e;
  if (!std::isfinite(c) || !(c > 0.f)) return FA_ERR_INVALID_ARG;
  if (noop) return FA_OK;
  if (!q || !k || !v || !o || !lse) return FA_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(lse))
    return FA_ERR_INVALID_ARG;
  fa::Fp8FwdArgs a;
  a.q = q;
  a.k = k;
  a.v = v;
  a.o = o;
  a.lse = lse;
  a.cu_seqlens = cu_seqlens;
  a.B = B;
  a.Hq = Hq;
  a.Hkv = Hkv;
  a.N = N;
  a.group = Hq / Hkv;
  const int br = fa::fwd_fp8_query_tile();
  a.n_qtiles = (N + br - 1) / br;
  a.scale_log2 = c;
  a.wl = a.wr = 0;
  a.o_scale = descale_v;
  if ((int64_t)a.n_qtiles * Hq * B >= (int64_t)1 << 31) return FA_ERR_UNSUPPORTED;
  st = debug_cu_seqlens(cu_seqlens, B, N, stream);
  if (st != FA_OK) return st;
  hipError_t e = fa::launch_fwd_fp8(a, out_dtype == FA_BF16, d, causal != 0,
                                    cu_seqlens != nullptr, stream);
  return launched(e, stream);
}

size_t fa_bwd_workspace_size(int B, int Hq, int Hkv, int N, int d) {
  bool noop;
  if (check_sizes(B, Hq, Hkv, N, d, 1.f, 0, FA_FP16, &noop, 256) != FA_OK) return 0;
  // D = rowsum(dO∘O) and LSE·log2(e): two float32 [Hq][B·N + 64] arrays
  // (tiles may read up to 63 rows past a sequence end); 256-byte granule
  const size_t bytes = 2 * (size_t)Hq * ((size_t)B * N + 64) * sizeof(float);
  return (bytes + 255) / 256 * 256;
}

namespace {

int bwd_common(int stage, const void* q, const void* k, const void* v, const void* o,
               const void* dout, const float* lse, void* dq, void* dk, void* dv, int B, int Hq,
               int Hkv, int N, int d, float scale, int mask, int wl, int wr,
               const int32_t* cu_seqlens, int dtype, void* workspace, size_t workspace_bytes,
               hipStream_t stream, float softcap = 0.f, float dropout_p = 0.f,
               uint64_t seed = 0) {
  bool noop;
  int st = check_sizes(B, Hq, Hkv, N, d, scale, 0, dtype, &noop, 256);
  if (st != FA_OK) return st;
  float cap_in, cap_out;
  st = cap_constants(softcap, scale, mask, d, &cap_in, &cap_out);
  if (st != FA_OK) return st;
  uint32_t keep_t;
  st = drop_constants(dropout_p, mask, d, &keep_t);
  if (st != FA_OK || noop) return st;
  if (!q || !k || !v || !o || !dout || !lse || !dq || !dk || !dv) return FA_ERR_INVALID_ARG;
  const void* ptrs[] = {q, k, v, o, dout, lse, dq, dk, dv, workspace};
  for (const void* p : ptrs)
    if (p && !aligned16(p)) return FA_ERR_INVALID_ARG;
  if (!workspace || workspace_bytes < fa_bwd_workspace_size(B, Hq, Hkv, N, d))
    return FA_ERR_WORKSPACE;
  fa::BwdArgs a;
  a.q = q;
  a.k = k;
  a.v = v;
  a.o = o;
  a.dout = dout;
  a.lse = lse;
  a.dq = dq;
  a.dk = dk;
  a.dv = dv;
  a.ws_stride = B * N + 64;
  a.delta = static_cast<float*>(workspace);
  a.lse2 = a.delta + (size_t)Hq * a.ws_stride;
  a.cu_seqlens = cu_seqlens;
  a.B = B;
  a.Hq = Hq;
  a.Hkv = Hkv;
  a.N = N;
  a.group = Hq / Hkv;
  a.scale = scale;
  a.scale_log2 = scale * kLog2e;
  a.wl = wl;
  a.wr = wr;
  a.cap_in = cap_in;
  a.cap_out = cap_out;
  a.seed_lo = (uint32_t)seed;
  a.seed_hi = (uint32_t)(seed >> 32);
  a.keep_t = keep_t;
  a.drop_scale = 256.f / (float)keep_t;
  st = debug_cu_seqlens(cu_seqlens, B, N, stream);
  if (st != FA_OK) return st;
  hipError_t e = fa::launch_bwd(a, dtype == FA_BF16, d, mask, cu_seqlens != nullptr,
                                softcap != 0.f, dropout_p != 0.f, stage, stream);
  return launched(e, stream);
}

}  // namespace

int fa_bwd(const void* q, const void* k, const void* v, const void* o, const void* dout,
           const float* lse, void* dq, void* dk, void* dv, int B, int Hq, int Hkv, int N, int d,
           float scale, int causal, const int32_t* cu_seqlens, fa_dtype dtype, void* workspace,
           size_t workspace_bytes, hipStream_t stream) {
  if (causal != 0 && causal != 1) return FA_ERR_INVALID_ARG;
  return bwd_common(-1, q, k, v, o, dout, lse, dq, dk, dv, B, Hq, Hkv, N, d, scale,
                    causal ? fa::kMaskCausal : fa::kMaskNone, 0, 0, cu_seqlens, dtype, workspace,
                    workspace_bytes, stream);
}

}  // extern "C"

// Scratch of fa_bwd_noalloc: the backward's workspace (D and LSE·log2 e) in a
// fixed device array, so that a call needs no allocation. Every GPU the library
// runs on holds its own copy from module load until the process ends. In host
// code `scratch` names a host-side stand-in, not the device array: the device
// address comes from hipGetSymbolAddress, once per device.
static __device__ __align__(256) unsigned char scratch[FA_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr size_t kScratchBytes = FA_NOALLOC_SCRATCH_BYTES;
constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch_ptr[kMaxDevices];
std::mutex g_scratch_mu;

// The current device's address of `scratch`, or nullptr (no device, or the
// runtime refused the lookup).
void* scratch_ptr() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  void* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (p) return p;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  p = g_scratch_ptr[dev].load(std::memory_order_relaxed);
  if (!p) {
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess) p = nullptr;
    if (p) g_scratch_ptr[dev].store(p, std::memory_order_release);
  }
  return p;
}

}  // namespace

extern "C" {

int fa_bwd_noalloc(const void* q, const void* k, const void* v, const void* o, const void* dout,
                   const float* lse, void* dq, void* dk, void* dv, int B, int Hq, int Hkv, int N,
                   int d, float scale, int causal, const int32_t* cu_seqlens, fa_dtype dtype,
                   hipStream_t stream) {
  if (causal != 0 && causal != 1) return FA_ERR_INVALID_ARG;
  bool noop;
  int st = check_sizes(B, Hq, Hkv, N, d, scale, causal, dtype, &noop, 256);
  if (st != FA_OK || noop) return st;
  if (fa_bwd_workspace_size(B, Hq, Hkv, N, d) > kScratchBytes) return FA_ERR_WORKSPACE;
  void* ws = scratch_ptr();
  if (!ws) {
    (void)hipGetLastError();
    return FA_ERR_HIP;
  }
  return bwd_common(-1, q, k, v, o, dout, lse, dq, dk, dv, B, Hq, Hkv, N, d, scale,
                    causal ? fa::kMaskCausal : fa::kMaskNone, 0, 0, cu_seqlens, dtype, ws,
                    kScratchBytes, stream);
}

int fa_bwd_window(const void* q, const void* k, const void* v, const void* o, const void* dout,
                  const float* lse, void* dq, void* dk, void* dv, int B, int Hq, int Hkv, int N,
                  int d, float scale, int window_left, int window_right,
                  const int32_t* cu_seqlens, fa_dtype dtype, void* workspace, size_t workspace_bytes,
                  hipStream_t stream) {
  return fa_bwd_window_stage(-1, q, k, v, o, dout, lse, dq, dk, dv, B, Hq, Hkv, N, d, scale,
                             window_left, window_right, cu_seqlens, dtype, workspace,
                             workspace_bytes, stream);
}

int fa_bwd_window_stage(int stage, const void* q, const void* k, const void* v, const void* o,
                        const void* dout, const float* lse, void* dq, void* dk, void* dv, int B,
                        int Hq, int Hkv, int N, int d, float scale, int window_left,
                        int window_right, const int32_t* cu_seqlens, fa_dtype dtype, void* workspace,
                        size_t workspace_bytes, hipStream_t stream) {
  if (stage < -1 || stage >= fa::bwd_num_stages()) return FA_ERR_INVALID_ARG;
  int mask, wl, wr;
  const int st = window_mode(window_left, window_right, N, &mask, &wl, &wr);
  if (st != FA_OK) return st;
  return bwd_common(stage, q, k, v, o, dout, lse, dq, dk, dv, B, Hq, Hkv, N, d, scale, mask, wl,
                    wr, cu_seqlens, dtype, workspace, workspace_bytes, stream);
}

int fa_bwd_window_softcap_stage(int stage, const void* q, const void* k, const void* v,
                                const void* o, const void* dout, const float* lse, void* dq,
                                void* dk, void* dv, int B, int Hq, int Hkv, int N, int d,
                                float scale, int window_left, int window_right, float softcap,
                                const int32_t* cu_seqlens, fa_dtype dtype, void* workspace,
                                size_t workspace_bytes, hipStream_t stream) {
  if (stage < -1 || stage >= fa::bwd_num_stages()) return FA_ERR_INVALID_ARG;
  int mask, wl, wr;
  const int st = window_mode(window_left, window_right, N, &mask, &wl, &wr);
  if (st != FA_OK) return st;
  return bwd_common(stage, q, k, v, o, dout, lse, dq, dk, dv, B, Hq, Hkv, N, d, scale, mask, wl,
                    wr, cu_seqlens, dtype, workspace, workspace_bytes, stream, softcap);
}

int fa_bwd_window_softcap(const void* q, const void* k, const void* v, const void* o,
                          const void* dout, const float* lse, void* dq, void* dk, void* dv,
                          int B, int Hq, int Hkv, int N, int d, float scale, int window_left,
                          int window_right, float softcap, const int32_t* cu_seqlens, fa_dtype dtype,
                          void* workspace, size_t workspace_bytes, hipStream_t stream) {
  return fa_bwd_window_softcap_stage(-1, q, k, v, o, dout, lse, dq, dk, dv, B, Hq, Hkv, N, d,
                                     scale, window_left, window_right, softcap, cu_seqlens, dtype,
                                     workspace, workspace_bytes, stream);
}

int fa_bwd_softcap(const void* q, const void* k, const void* v, const void* o, const void* dout,
                   const float* lse, void* dq, void* dk, void* dv, int B, int Hq, int Hkv, int N,
                   int d, float scale, int causal, float softcap, const int32_t* cu_seqlens,
                   fa_dtype dtype, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  return fa_bwd_softcap_stage(-1, q, k, v, o, dout, lse, dq, dk, dv, B, Hq, Hkv, N, d, scale,
                              causal, softcap, cu_seqlens, dtype, workspace, workspace_bytes,
                              stream);
}

int fa_bwd_softcap_stage(int stage, const void* q, const void* k, const void* v, const void* o,
                         const void* dout, const float* lse, void* dq, void* dk, void* dv, int B,
                         int Hq, int Hkv, int N, int d, float scale, int causal, float softcap,
                         const int32_t* cu_seqlens, fa_dtype dtype, void* workspace,
                         size_t workspace_bytes, hipStream_t stream) {
  if (stage < -1 || stage >= fa::bwd_num_stages()) return FA_ERR_INVALID_ARG;
  if (causal != 0 && causal != 1) return FA_ERR_INVALID_ARG;
  return bwd_common(stage, q, k, v, o, dout, lse, dq, dk, dv, B, Hq, Hkv, N, d, scale,
                    causal ? fa::kMaskCausal : fa::kMaskNone, 0, 0, cu_seqlens, dtype, workspace,
                    workspace_bytes, stream, softcap);
}

int fa_bwd_dropout(const void* q, const void* k, const void* v, const void* o, const void* dout,
                   const float* lse, void* dq, void* dk, void* dv, int B, int Hq, int Hkv, int N,
                   int d, float scale, int causal, float dropout_p, uint64_t seed,
                   const int32_t* cu_seqlens, fa_dtype dtype, void* workspace, size_t workspace_bytes,
                   hipStream_t stream) {
  return fa_bwd_dropout_stage(-1, q, k, v, o, dout, lse, dq, dk, dv, B, Hq, Hkv, N, d, scale,
                              causal, dropout_p, seed, cu_seqlens, dtype, workspace,
                              workspace_bytes, stream);
}

int fa_bwd_dropout_stage(int stage, const void* q, const void* k, const void* v, const void* o,
                         const void* dout, const float* lse, void* dq, void* dk, void* dv, int B,
                         int Hq, int Hkv, int N, int d, float scale, int causal, float dropout_p,
                         uint64_t seed, const int32_t* cu_seqlens, fa_dtype dtype, void* workspace,
                         size_t workspace_bytes, hipStream_t stream) {
  if (stage < -1 || stage >= fa::bwd_num_stages()) return FA_ERR_INVALID_ARG;
  if (causal != 0 && causal != 1) return FA_ERR_INVALID_ARG;
  return bwd_common(stage, q, k, v, o, dout, lse, dq, dk, dv, B, Hq, Hkv, N, d, scale,
                    causal ? fa::kMaskCausal : fa::kMaskNone, 0, 0, cu_seqlens, dtype, workspace,
                    workspace_bytes, stream, 0.f, dropout_p, seed);
}

int fa_bwd_num_stages(void) { return fa::bwd_num_stages(); }

// fa_attn_options as the binding mirrors it (ctypes lays it out by the same C rules)
static_assert(sizeof(fa_attn_options) == 40 && offsetof(fa_attn_options, mask) == 8 &&
                  offsetof(fa_attn_options, softcap) == 20 &&
                  offsetof(fa_attn_options, dropout_seed) == 32,
              "fa_attn_options layout");

// The options of fa_fwd_ex / fa_bwd_ex, checked; which entry point they select.
enum class ExRoute { kPlain, kWindow, kSoftcap, kWindowSoftcap, kDropout };

static int ex_route(const fa_attn_options* opts, ExRoute* route) {
  if (opts == nullptr || opts->struct_size < sizeof(fa_attn_options)) return FA_ERR_INVALID_ARG;
  const int mask = static_cast<int>(opts->mask);
  if (mask != FA_MASK_NONE && mask != FA_MASK_CAUSAL && mask != FA_MASK_WINDOW)
    return FA_ERR_INVALID_ARG;
  const bool window = mask == FA_MASK_WINDOW;
  const bool cap = opts->softcap != 0.f, drop = opts->dropout_p != 0.f;
  if (drop && (window || cap)) return FA_ERR_UNSUPPORTED;
  *route = drop ? ExRoute::kDropout
         : window ? (cap ? ExRoute::kWindowSoftcap : ExRoute::kWindow)
         : cap ? ExRoute::kSoftcap : ExRoute::kPlain;
  return FA_OK;
}

int fa_fwd_ex(const void* q, const void* k, const void* v, void* o, float* lse, int B, int Hq,
              int Hkv, int N, int d, float scale, const fa_attn_options* opts,
              const int32_t* cu_seqlens, fa_dtype dtype, hipStream_t stream) {
  ExRoute r;
  const int st = ex_route(opts, &r);
  if (st != FA_OK) return st;
  const int causal = opts->mask == FA_MASK_CAUSAL;
  switch (r) {
    case ExRoute::kWindow:
      return fa_fwd_window(q, k, v, o, lse, B, Hq, Hkv, N, d, scale, opts->window_left,
                           opts->window_right, cu_seqlens, dtype, stream);
    case ExRoute::kSoftcap:
      return fa_fwd_softcap(q, k, v, o, lse, B, Hq, Hkv, N, d, scale, causal, opts->softcap,
                            cu_seqlens, dtype, stream);
    case ExRoute::kWindowSoftcap:
      return fa_fwd_window_softcap(q, k, v, o, lse, B, Hq, Hkv, N, d, scale, opts->window_left,
                                   opts->window_right, opts->softcap, cu_seqlens, dtype, stream);
    case ExRoute::kDropout:
      return fa_fwd_dropout(q, k, v, o, lse, B, Hq, Hkv, N, d, scale, causal, opts->dropout_p,
                            opts->dropout_seed, cu_seqlens, dtype, stream);
    default:
      return fa_fwd(q, k, v, o, lse, B, Hq, Hkv, N, d, scale, causal, cu_seqlens, dtype, stream);
  }
}

int fa_bwd_ex(const void* q, const void* k, const void* v, const void* o, const void* dout,
              const float* lse, void* dq, void* dk, void* dv, int B, int Hq, int Hkv, int N,
              int d, float scale, const fa_attn_options* opts, const int32_t* cu_seqlens,
              fa_dtype dtype, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  ExRoute r;
  const int st = ex_route(opts, &r);
  if (st != FA_OK) return st;
  const int causal = opts->mask == FA_MASK_CAUSAL;
  switch (r) {
    case ExRoute::kWindow:
      return fa_bwd_window(q, k, v, o, dout, lse, dq, dk, dv, B, Hq, Hkv, N, d, scale,
                           opts->window_left, opts->window_right, cu_seqlens, dtype, workspace,
                           workspace_bytes, stream);
    case ExRoute::kSoftcap:
      return fa_bwd_softcap(q, k, v, o, dout, lse, dq, dk, dv, B, Hq, Hkv, N, d, scale, causal,
                            opts->softcap, cu_seqlens, dtype, workspace, workspace_bytes, stream);
    case ExRoute::kWindowSoftcap:
      return fa_bwd_window_softcap(q, k, v, o, dout, lse, dq, dk, dv, B, Hq, Hkv, N, d, scale,
                                   opts->window_left, opts->window_right, opts->softcap,
                                   cu_seqlens, dtype, workspace, workspace_bytes, stream);
    case ExRoute::kDropout:
      return fa_bwd_dropout(q, k, v, o, dout, lse, dq, dk, dv, B, Hq, Hkv, N, d, scale, causal,
                            opts->dropout_p, opts->dropout_seed, cu_seqlens, dtype, workspace,
                            workspace_bytes, stream);
    default:
      return fa_bwd(q, k, v, o, dout, lse, dq, dk, dv, B, Hq, Hkv, N, d, scale, causal,
                    cu_seqlens, dtype, workspace, workspace_bytes, stream);
  }
}

}  // extern "C"

namespace {

// The backward of fa_fwd_kvlen; stage < 0 runs every stage.
int bwd_kvlen_common(int stage, const void* q, const void* k, const void* v, const void* o,
                     const void* dout, const float* lse, void* dq, void* dk, void* dv, int B,
                     int Hq, int Hkv, int Nq, int Nk, int d, float scale, int causal,
                     const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k, int dtype,
                     void* workspace, size_t workspace_bytes, hipStream_t stream) {
  const bool varlen = cu_seqlens_q != nullptr;
  if (varlen != (cu_seqlens_k != nullptr)) return FA_ERR_INVALID_ARG;
  bool noop;
  int st = check_sizes(B, Hq, Hkv, Nq, d, scale, causal, dtype, &noop, 128);
  if (st != FA_OK) return st;
  if (Nk < 0) return FA_ERR_INVALID_ARG;
  if ((int64_t)B * Nk >= (int64_t)1 << 31 || (int64_t)B * Nk * Hkv >= (int64_t)1 << 31)
    return FA_ERR_UNSUPPORTED;
  // no query: dk, dv are zero (still written); no key either: nothing to do
  if (B == 0 || (Nq == 0 && Nk == 0)) return FA_OK;
  if (Nq > 0 && (!q || !o || !dout || !lse || !dq)) return FA_ERR_INVALID_ARG;
  if (Nk > 0 && (!k || !v || !dk || !dv)) return FA_ERR_INVALID_ARG;
  const void* ptrs[] = {q, k, v, o, dout, lse, dq, dk, dv, workspace};
  for (const void* p : ptrs)
    if (p && !aligned16(p)) return FA_ERR_INVALID_ARG;
  if (!workspace || workspace_bytes < fa_bwd_workspace_size(B, Hq, Hkv, Nq, d))
    return FA_ERR_WORKSPACE;
  fa::BwdArgs a;
  a.q = q;
  a.k = k;
  a.v = v;
  a.o = o;
  a.dout = dout;
  a.lse = lse;
  a.dq = dq;
  a.dk = dk;
  a.dv = dv;
  a.ws_stride = B * Nq + 64;
  a.delta = static_cast<float*>(workspace);
  a.lse2 = a.delta + (size_t)Hq * a.ws_stride;
  a.cu_seqlens = cu_seqlens_q;
  a.cu_seqlens_k = cu_seqlens_k;
  a.B = B;
  a.Hq = Hq;
  a.Hkv = Hkv;
  a.N = Nq;
  a.Nk = Nk;
  a.group = Hq / Hkv;
  a.scale = scale;
  a.scale_log2 = scale * kLog2e;
  a.wl = a.wr = 0;
  a.cap_in = a.cap_out = 0.f;
  a.seed_lo = a.seed_hi = 0;
  a.keep_t = 256;
  a.drop_scale = 1.f;
  if (varlen) {
    int st = debug_cu_seqlens(cu_seqlens_q, B, Nq, stream);
    if (st == FA_OK) st = debug_cu_seqlens(cu_seqlens_k, B, Nk, stream);
    if (st != FA_OK) return st;
  }
  hipError_t e = fa::launch_bwd_kvlen(a, dtype == FA_BF16, d, causal != 0, varlen, stage, stream);
  return launched(e, stream);
}

}  // namespace

extern "C" {

int fa_bwd_kvlen(const void* q, const void* k, const void* v, const void* o, const void* dout,
                 const float* lse, void* dq, void* dk, void* dv, int B, int Hq, int Hkv, int Nq,
                 int Nk, int d, float scale, int causal, const int32_t* cu_seqlens_q,
                 const int32_t* cu_seqlens_k, fa_dtype dtype, void* workspace,
                 size_t workspace_bytes, hipStream_t stream) {
  return bwd_kvlen_common(-1, q, k, v, o, dout, lse, dq, dk, dv, B, Hq, Hkv, Nq, Nk, d, scale,
                          causal, cu_seqlens_q, cu_seqlens_k, dtype, workspace, workspace_bytes,
                          stream);
}

int fa_bwd_kvlen_stage(int stage, const void* q, const void* k, const void* v, const void* o,
                       const void* dout, const float* lse, void* dq, void* dk, void* dv, int B,
                       int Hq, int Hkv, int Nq, int Nk, int d, float scale, int causal,
                       const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k, fa_dtype dtype,
                       void* workspace, size_t workspace_bytes, hipStream_t stream) {
  if (stage < 0 || stage >= fa::bwd_num_stages()) return FA_ERR_INVALID_ARG;
  return bwd_kvlen_common(stage, q, k, v, o, dout, lse, dq, dk, dv, B, Hq, Hkv, Nq, Nk, d, scale,
                          causal, cu_seqlens_q, cu_seqlens_k, dtype, workspace, workspace_bytes,
                          stream);
}

int fa_bwd_stage(int stage, const void* q, const void* k, const void* v, const void* o,
                 const void* dout, const float* lse, void* dq, void* dk, void* dv, int B, int Hq,
                 int Hkv, int N, int d, float scale, int causal, const int32_t* cu_seqlens,
                 fa_dtype dtype, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  if (stage < 0 || stage >= fa::bwd_num_stages()) return FA_ERR_INVALID_ARG;
  if (causal != 0 && causal != 1) return FA_ERR_INVALID_ARG;
  return bwd_common(stage, q, k, v, o, dout, lse, dq, dk, dv, B, Hq, Hkv, N, d, scale,
                    causal ? fa::kMaskCausal : fa::kMaskNone, 0, 0, cu_seqlens, dtype, workspace,
                    workspace_bytes, stream);
}

namespace {

// Sizes of fa_fwd_kvcache; *noop when there is nothing to compute.
int check_kvcache(int B, int Hq, int Hkv, int Nq, int Nk, int d, float scale, int causal,
                  int num_splits, int dtype, bool* noop) {
  *noop = false;
  if (dtype != FA_FP16 && dtype != FA_BF16) return FA_ERR_INVALID_ARG;
  if (B < 0 || Nq < 0 || Nk < 0 || Hq <= 0 || Hkv <= 0 || d <= 0 || num_splits < 0)
    return FA_ERR_INVALID_ARG;
  if (Hq % Hkv != 0) return FA_ERR_INVALID_ARG;
  if (causal != 0 && causal != 1) return FA_ERR_INVALID_ARG;
  if (!std::isfinite(scale) || !(scale > 0.f)) return FA_ERR_INVALID_ARG;
  if (d != 64 && d != 128 && d != 256) return FA_ERR_UNSUPPORTED;
  // cache and row indices are formed in 64 bits, grid and query counts in 32
  if ((int64_t)B * Nq * Hq >= (int64_t)1 << 31 || (int64_t)Nk * Hkv * d >= (int64_t)1 << 31)
    return FA_ERR_UNSUPPORTED;
  if (B == 0 || Nq == 0) *noop = true;
  return FA_OK;
}

// decode_kernel workgroups resident per CU and CUs per device: the runtime's
// occupancy figure for the exact instantiation when a device is present
// (cached per configuration: one GPU type per process), else the same bound
// from LDS (160 KiB per CU) and registers (two-wave workgroups; the waves per
// SIMD the register counts of this build allow: 4 at d = 64, 2 at d = 128 (3
// for an e4m3 cache), 1 at d = 256).
struct Residency {
  int per_cu, cus;
};
Residency decode_residency(int d, bool kv8, int dtype, int causal) {
  static std::atomic<int> cache[2][3][2][2][2];   // [bf16][d][causal][kv8][per_cu, cus]
  const int di = d == 64 ? 0 : d == 128 ? 1 : 2;
  const int bi = dtype == FA_BF16 ? 1 : 0, ci = causal ? 1 : 0, ki = kv8 ? 1 : 0;
  std::atomic<int>* c = cache[bi][di][ci][ki];
  int per_cu = c[0].load(std::memory_order_relaxed);
  int cus = c[1].load(std::memory_order_relaxed);
  if (per_cu > 0 && cus > 0) return {per_cu, cus};
  int dev = 0;
  per_cu = 0;
  cus = 0;
  if (hipGetDevice(&dev) == hipSuccess &&
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess &&
      cus > 0)
    per_cu = fa::decode_resident_per_cu(dtype == FA_BF16, d, causal != 0, kv8);
  (void)hipGetLastError();
  if (per_cu > 0) {
    c[0].store(per_cu, std::memory_order_relaxed);
    c[1].store(cus, std::memory_order_relaxed);
    return {per_cu, cus};
  }
  const int by_lds = (160 * 1024) / fa::decode_lds_bytes(d, kv8);
  const int by_regs = 2 * (d == 256 ? 1 : d == 128 ? (kv8 ? 3 : 2) : 4);
  return {std::max(1, std::min(by_lds, by_regs)), 256};
}

// Key ranges per (entry, KV head): as many as keep every decode_kernel
// workgroup resident at once (one round of waves over the GPU). Measured on
// 8192-token caches, the call is fastest at exactly one full round and a
// second, partly filled round costs up to 40 %. Each range holds at least
// eight key tiles (256 keys: on 4096-token caches shorter ranges measured
// slower, their merge and fixed costs outweighing the extra parallelism), and
// there are at most 256 ranges.
// An e4m3 cache at d <= 128 takes half that many workgroups, rounded up (so up
// to a full round when the half is not whole): measured on six shapes at
// d = 128 (2048- to 32768-token caches, 1 and 4 queries, 8 and 64 query heads)
// and one at d = 64, half the resident count was fastest in every one, by
// 9-18 % over a full round (decode_llama's shape over an e4m3 cache: 47.5
// against 54.7 µs). At d = 256, where only two workgroups fit per CU, half
// measured 30 % slower than the full round, which is kept there.
// The count depends on the head dimension and the cache type only: the
// residency taken is the smallest over query dtype and mask, so the query
// functions below, which take neither, report exactly what a call uses.
int kv_splits(int B, int Hq, int Hkv, int Nq, int Nk, int d, bool kv8) {
  const int tk = fa::decode_tile_keys();
  Residency r = decode_residency(d, kv8, FA_FP16, 0);
  for (int dt : {FA_FP16, FA_BF16})
    for (int c : {0, 1}) {
      const Residency x = decode_residency(d, kv8, dt, c);
      r.per_cu = std::min(r.per_cu, x.per_cu);
      r.cus = std::min(r.cus, x.cus);
    }
  const int64_t rows = (int64_t)(Hq / Hkv) * Nq;
  const int64_t base = (int64_t)B * Hkv * ((rows + 31) / 32);
  const int64_t slots = (int64_t)r.per_cu * r.cus, b = base > 0 ? base : 1;
  const int64_t want = kv8 && d <= 128 ? (slots + 2 * b - 1) / (2 * b) : slots / b;
  const int64_t most = std::max<int64_t>(1, (Nk + 8 * tk - 1) / (8 * tk));
  return (int)std::max<int64_t>(1, std::min<int64_t>(want, std::min<int64_t>(most, 256)));
}

}  // namespace

int fa_kvcache_num_splits(int B, int Hq, int Hkv, int Nq, int Nk, int d) {
  bool noop;
  if (check_kvcache(B, Hq, Hkv, Nq, Nk, d, 1.f, 0, 0, FA_FP16, &noop) != FA_OK) return 0;
  return kv_splits(B, Hq, Hkv, Nq, Nk, d, false);
}

int fa_kvcache_fp8_num_splits(int B, int Hq, int Hkv, int Nq, int Nk, int d) {
  bool noop;
  if (check_kvcache(B, Hq, Hkv, Nq, Nk, d, 1.f, 0, 0, FA_FP16, &noop) != FA_OK) return 0;
  return kv_splits(B, Hq, Hkv, Nq, Nk, d, true);
}

size_t fa_fwd_kvcache_workspace_size(int B, int Hq, int Hkv, int Nq, int Nk, int d,
                                     int num_splits) {
  bool noop;
  if (check_kvcache(B, Hq, Hkv, Nq, Nk, d, 1.f, 0, num_splits, FA_FP16, &noop) != FA_OK) return 0;
  // num_splits = 0: enough for either cache type's automatic count
  const int sp = num_splits > 0
                     ? num_splits
                     : std::max(kv_splits(B, Hq, Hkv, Nq, Nk, d, false),
                                kv_splits(B, Hq, Hkv, Nq, Nk, d, true));
  const size_t bytes = (size_t)sp * B * Hq * Nq * (size_t)(d + 1) * sizeof(float);
  return (bytes + 255) / 256 * 256;
}

namespace {

// kv8: e4m3fn caches with descales descale_k, descale_v (ignored otherwise).
int kvcache_common(int stage, const void* q, const void* k_cache, const void* v_cache,
                   const int32_t* cache_seqlens, void* o, float* lse, int B, int Hq, int Hkv,
                   int Nq, int Nk, int d, float scale, int causal, int num_splits, int dtype,
                   void* workspace, size_t workspace_bytes, hipStream_t stream, bool kv8 = false,
                   float descale_k = 1.f, float descale_v = 1.f) {
  bool noop;
  int st = check_kvcache(B, Hq, Hkv, Nq, Nk, d, scale, causal, num_splits, dtype, &noop);
  if (st != FA_OK) return st;
  if (kv8 && !(std::isfinite(descale_k) && descale_k > 0.f && std::isfinite(descale_v) &&
               descale_v > 0.f))
    return FA_ERR_INVALID_ARG;
  if (noop) return st;
  if (!q || !k_cache || !v_cache || !cache_seqlens || !o || !lse) return FA_ERR_INVALID_ARG;
  const void* ptrs[] = {q, k_cache, v_cache, o, lse, workspace};
  for (const void* p : ptrs)
    if (p && !aligned16(p)) return FA_ERR_INVALID_ARG;
  if ((reinterpret_cast<uintptr_t>(cache_seqlens) & 3u) != 0) return FA_ERR_INVALID_ARG;
  const int sp = num_splits > 0 ? num_splits : kv_splits(B, Hq, Hkv, Nq, Nk, d, kv8);
  if (!workspace || workspace_bytes < fa_fwd_kvcache_workspace_size(B, Hq, Hkv, Nq, Nk, d, sp))
    return FA_ERR_WORKSPACE;
  fa::DecodeArgs a;
  a.q = q;
  a.k = k_cache;
  a.v = v_cache;
  a.seqlens = cache_seqlens;
  a.o = o;
  a.lse = lse;
  const size_t units = (size_t)B * Hq * Nq;
  a.part_o = static_cast<float*>(workspace);
  a.part_lse = a.part_o + (size_t)sp * units * d;
  a.B = B;
  a.Hq = Hq;
  a.Hkv = Hkv;
  a.Nq = Nq;
  a.Nk = Nk;
  a.group = Hq / Hkv;
  a.rows = a.group * Nq;
  a.n_rb = (a.rows + 31) / 32;
  a.splits = sp;
  const int tk = fa::decode_tile_keys();
  const int per = (Nk + sp - 1) / sp;
  a.chunk = std::max(tk, (per + tk - 1) / tk * tk);
  a.scale_log2 = scale * kLog2e * (kv8 ? descale_k : 1.f);
  a.o_scale = kv8 ? descale_v : 1.f;
  if (!std::isfinite(a.scale_log2) || !(a.scale_log2 > 0.f)) return FA_ERR_INVALID_ARG;
  if ((int64_t)a.n_rb * sp * Hkv * B >= (int64_t)1 << 31) return FA_ERR_UNSUPPORTED;
  hipError_t e = fa::launch_decode(a, dtype == FA_BF16, d, causal != 0, kv8, stage, stream);
  return launched(e, stream);
}

}  // namespace

int fa_fwd_kvcache(const void* q, const void* k_cache, const void* v_cache,
                   const int32_t* cache_seqlens, void* o, float* lse, int B, int Hq, int Hkv,
                   int Nq, int Nk, int d, float scale, int causal, int num_splits, fa_dtype dtype,
                   void* workspace, size_t workspace_bytes, hipStream_t stream) {
  return kvcache_common(-1, q, k_cache, v_cache, cache_seqlens, o, lse, B, Hq, Hkv, Nq, Nk, d,
                        scale, causal, num_splits, dtype, workspace, workspace_bytes, stream);
}

int fa_fwd_kvcache_num_stages(void) { return fa::decode_num_stages(); }

int fa_fwd_kvcache_stage(int stage, const void* q, const void* k_cache, const void* v_cache,
                         const int32_t* cache_seqlens, void* o, float* lse, int B, int Hq,
                         int Hkv, int Nq, int Nk, int d, float scale, int causal, int num_splits,
                         fa_dtype dtype, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  if (stage < 0 || stage >= fa::decode_num_stages()) return FA_ERR_INVALID_ARG;
  return kvcache_common(stage, q, k_cache, v_cache, cache_seqlens, o, lse, B, Hq, Hkv, Nq, Nk, d,
                        scale, causal, num_splits, dtype, workspace, workspace_bytes, stream);
}

int fa_fwd_kvcache_local(const void* q, const void* k_cache, const void* v_cache,
                         const int32_t* cache_seqlens, void* o, float* lse, int B, int Hq,
                         int Hkv, int Nq, int Nk, int d, float scale, int causal,
                         int window_left, float softcap, int num_splits, fa_dtype dtype,
                         void* workspace, size_t workspace_bytes, hipStream_t stream) {
  bool noop;
  int st = check_kvcache(B, Hq, Hkv, Nq, Nk, d, scale, causal, num_splits, dtype, &noop);
  if (st != FA_OK) return st;
  if (window_left < -1) return FA_ERR_INVALID_ARG;
  float cap_in = 0.f, cap_out = 0.f;
  if (softcap != 0.f) {
    if (!std::isfinite(softcap) || !(softcap > 0.f)) return FA_ERR_INVALID_ARG;
    cap_in = scale / softcap;
    cap_out = softcap * kLog2e;
    if (!std::isfinite(cap_in) || !std::isfinite(cap_out)) return FA_ERR_INVALID_ARG;
  }
  if (noop) return FA_OK;
  if (!q || !k_cache || !v_cache || !cache_seqlens || !o || !lse) return FA_ERR_INVALID_ARG;
  const void* ptrs[] = {q, k_cache, v_cache, o, lse, workspace};
  for (const void* p : ptrs)
    if (p && !aligned16(p)) return FA_ERR_INVALID_ARG;
  if ((reinterpret_cast<uintptr_t>(cache_seqlens) & 3u) != 0) return FA_ERR_INVALID_ARG;
  // the keys any query of an entry can see: the last Nq + window_left positions
  const int wl = window_left < 0 ? Nk : std::min(window_left, Nk);
  const int span = (int)std::min<int64_t>(Nk, (int64_t)Nq + wl);
  const int sp = num_splits > 0 ? num_splits : kv_splits(B, Hq, Hkv, Nq, span, d, false);
  if (!workspace || workspace_bytes < fa_fwd_kvcache_workspace_size(B, Hq, Hkv, Nq, Nk, d, sp))
    return FA_ERR_WORKSPACE;
  fa::DecodeArgs a;
  a.q = q;
  a.k = k_cache;
  a.v = v_cache;
  a.seqlens = cache_seqlens;
  a.o = o;
  a.lse = lse;
  const size_t units = (size_t)B * Hq * Nq;
  a.part_o = static_cast<float*>(workspace);
  a.part_lse = a.part_o + (size_t)sp * units * d;
  a.B = B;
  a.Hq = Hq;
  a.Hkv = Hkv;
  a.Nq = Nq;
  a.Nk = Nk;
  a.group = Hq / Hkv;
  a.rows = a.group * Nq;
  a.n_rb = (a.rows + 31) / 32;
  a.splits = sp;
  const int tk = fa::decode_tile_keys();
  const int per = (std::max(span, 1) + sp - 1) / sp;
  a.chunk = std::max(tk, (per + tk - 1) / tk * tk);
  a.scale_log2 = softcap != 0.f ? 1.f : scale * kLog2e;   // capped logits are in log2 units
  a.o_scale = 1.f;
  a.wl = wl;
  a.cap_on = softcap != 0.f;
  a.cap_in = cap_in;
  a.cap_out = cap_out;
  if ((int64_t)a.n_rb * sp * Hkv * B >= (int64_t)1 << 31) return FA_ERR_UNSUPPORTED;
  hipError_t e = fa::launch_decode_ext(a, dtype == FA_BF16, d, causal != 0, -1, stream);
  return launched(e, stream);
}

int fa_fwd_kvcache_fp8(const void* q, const void* k_cache, const void* v_cache,
                       const int32_t* cache_seqlens, void* o, float* lse, int B, int Hq, int Hkv,
                       int Nq, int Nk, int d, float scale, int causal, float descale_k,
                       float descale_v, int num_splits, fa_dtype dtype, void* workspace,
                       size_t workspace_bytes, hipStream_t stream) {
  return kvcache_common(-1, q, k_cache, v_cache, cache_seqlens, o, lse, B, Hq, Hkv, Nq, Nk, d,
                        scale, causal, num_splits, dtype, workspace, workspace_bytes, stream, true,
                        descale_k, descale_v);
}

int fa_fwd_kvcache_fp8_stage(int stage, const void* q, const void* k_cache, const void* v_cache,
                             const int32_t* cache_seqlens, void* o, float* lse, int B, int Hq,
                             int Hkv, int Nq, int Nk, int d, float scale, int causal,
                             float descale_k, float descale_v, int num_splits, fa_dtype dtype,
                             void* workspace, size_t workspace_bytes, hipStream_t stream) {
  if (stage < 0 || stage >= fa::decode_num_stages()) return FA_ERR_INVALID_ARG;
  return kvcache_common(stage, q, k_cache, v_cache, cache_seqlens, o, lse, B, Hq, Hkv, Nq, Nk, d,
                        scale, causal, num_splits, dtype, workspace, workspace_bytes, stream, true,
                        descale_k, descale_v);
}

int fa_check_cu_seqlens(const int32_t* cu_seqlens_host, int B, int N) {
  if (cu_seqlens_host == nullptr || B < 0 || N < 0) return FA_ERR_INVALID_ARG;
  if (cu_seqlens_host[0] != 0) return FA_ERR_INVALID_ARG;
  for (int s = 0; s < B; ++s) {
    const int64_t len = (int64_t)cu_seqlens_host[s + 1] - cu_seqlens_host[s];
    if (len < 0 || len > N) return FA_ERR_INVALID_ARG;
  }
  return FA_OK;
}

const char* fa_status_string(int status) {
  switch (status) {
    case FA_OK: return "FA_OK: success";
    case FA_ERR_INVALID_ARG: return "FA_ERR_INVALID_ARG: invalid argument";
    case FA_ERR_UNSUPPORTED: return "FA_ERR_UNSUPPORTED: outside the supported envelope";
    case FA_ERR_HIP: return "FA_ERR_HIP: the HIP runtime refused the launch";
    case FA_ERR_WORKSPACE: return "FA_ERR_WORKSPACE: workspace missing or too small";
    default: return "unknown fa status";
  }
}

}  // extern "C"
