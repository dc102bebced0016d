// Launch interface between the C-ABI layer (fa_api.hip) and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

// Which keys a query sees (positions local to its sequence): all, keys j ≤ i
// (causal), or keys i − wl ≤ j ≤ i + wr (sliding window; wl, wr ≤ N).
constexpr int kMaskNone = 0, kMaskCausal = 1, kMaskWindow = 2;

struct FwdArgs {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  const int32_t* cu_seqlens;  // null for fixed length
  int B, Hq, Hkv, N;
  int group;                  // Hq / Hkv
  int n_qtiles;               // ceil(N / query tile)
  float scale_log2;           // scale · log2(e)
  int wl, wr;                 // window bounds (kMaskWindow only)
  float cap_in, cap_out;      // soft cap c: scale / c and c · log2(e) (softcap kernels only)
  uint32_t seed_lo, seed_hi;  // dropout: Philox key
  uint32_t keep_t;            // dropout: keep iff byte < keep_t
  float drop_scale;           // dropout: 256 / keep_t
  // separate key lengths (launch_fwd_kvlen only): keys [B·Nk] or cu_seqlens_k
  const int32_t* cu_seqlens_k = nullptr;
  int Nk = 0;
};

// FP8 forward: q, k, v hold e4m3fn codes; scale_log2 already includes both
// input descales (scale · descale_q · descale_k · log2 e) and O is multiplied
// by o_scale (the descale of V) before it is rounded to the output type.
struct Fp8FwdArgs : FwdArgs {
  float o_scale;
};

struct BwdArgs {
  const void* q;
  const void* k;
  const void* v;
  const void* o;
  const void* dout;
  const float* lse;
  void* dq;
  void* dk;
  void* dv;
  float* delta;               // workspace: rowsum(dO∘O), [Hq][ws_stride] float32
  float* lse2;                // workspace: LSE·log2(e), [Hq][ws_stride] float32
  int ws_stride;              // B·N + 64: rows may be read up to 63 past a sequence end
  const int32_t* cu_seqlens;
  int B, Hq, Hkv, N;
  int group;
  float scale;
  float scale_log2;
  int wl, wr;                 // window bounds (kMaskWindow only)
  float cap_in, cap_out;      // soft cap c: scale / c and c · log2(e) (softcap kernels only)
  uint32_t seed_lo, seed_hi;  // dropout: Philox key
  uint32_t keep_t;            // dropout: keep iff byte < keep_t
  float drop_scale;           // dropout: 256 / keep_t
  // separate key lengths (launch_bwd_kvlen only): keys [B·Nk] or cu_seqlens_k;
  // the queries of a sequence are its last positions, as in the forward
  const int32_t* cu_seqlens_k = nullptr;
  int Nk = 0;
};

struct DecodeArgs {
  const void* q;              // [B, Nq, Hq, d]
  const void* k;              // [B, Nk, Hkv, d]
  const void* v;
  const int32_t* seqlens;     // [B] valid cache positions (device)
  void* o;                    // [B, Nq, Hq, d]
  float* lse;                 // [Hq, B·Nq]
  float* part_o;              // workspace [splits][B·Hq·Nq][d] float32
  float* part_lse;            // workspace [splits][B·Hq·Nq] float32
  int B, Hq, Hkv, Nq, Nk;
  int group;                  // Hq / Hkv
  int rows;                   // group · Nq rows per (entry, KV head)
  int n_rb;                   // ceil(rows / 32)
  int splits;                 // key ranges per (entry, KV head)
  int chunk;                  // keys per range, a multiple of the key tile
  float scale_log2;           // scale · log2(e) (· descale of K for an e4m3 cache)
  float o_scale;              // O factor: 1, or the descale of V for an e4m3 cache
  // launch_decode_ext only: window of wl keys behind each query, soft cap
  int wl = 0;
  int cap_on = 0;
  float cap_in = 0.f, cap_out = 0.f;   // scale / c and c·log2 e (scale_log2 = 1 then)
};

int fwd_query_tile();
// softcap: logits c·tanh(scale·q·k / c); dropout: keep decisions from the
// Philox stream of the seed (each: mask kMaskNone or kMaskCausal, d <= 128,
// not both)
hipError_t launch_fwd(const FwdArgs& a, bool bf16_in, int d, int mask, bool varlen, bool softcap,
                      bool dropout, hipStream_t s);
// Queries and keys of different lengths per sequence (a.N / a.cu_seqlens for the
// queries, a.Nk / a.cu_seqlens_k for the keys), the queries being the last
// positions: mask none or causal, no window, soft cap or dropout.
hipError_t launch_fwd_kvlen(const FwdArgs& a, bool bf16_in, int d, bool causal, bool varlen,
                            hipStream_t s);
int fwd_fp8_query_tile();
hipError_t launch_fwd_fp8(const Fp8FwdArgs& a, bool bf16_out, int d, bool causal, bool varlen,
                          hipStream_t s);
// stage < 0: every stage in order; otherwise only stage 0 (D = rowsum(dO∘O)),
// 1 (dK, dV) or 2 (dQ).
int bwd_num_stages();
hipError_t launch_bwd(const BwdArgs& a, bool bf16_in, int d, int mask, bool varlen, bool softcap,
                      bool dropout, int stage, hipStream_t s);
// The backward of launch_fwd_kvlen (a.N / a.cu_seqlens for the queries, a.Nk /
// a.cu_seqlens_k for the keys): mask none or causal, d = 64 or 128.
hipError_t launch_bwd_kvlen(const BwdArgs& a, bool bf16_in, int d, bool causal, bool varlen,
                            int stage, hipStream_t s);
int decode_tile_keys();
// stage < 0: both stages; 0: per-range partial results; 1: merge into o, lse.
// kv8: k and v hold e4m3fn codes (q and o stay 16-bit).
int decode_num_stages();
// decode_kernel workgroups (two waves each) resident per CU for this instantiation,
// from the runtime's occupancy calculation; 0 when no device is available.
int decode_resident_per_cu(bool bf16_in, int d, bool causal, bool kv8);
int decode_lds_bytes(int d, bool kv8);   // LDS per decode_kernel workgroup
// 16-bit caches with a sliding window (a.wl) and/or a soft cap (a.cap_on)
hipError_t launch_decode_ext(const DecodeArgs& a, bool bf16_in, int d, bool causal, int stage,
                             hipStream_t s);
hipError_t launch_decode(const DecodeArgs& a, bool bf16_in, int d, bool causal, bool kv8,
                         int stage, hipStream_t s);

}  // namespace fa
