// Attention of a few new queries over a key/value cache (decode), gfx950.
//
// Per batch entry b the cache holds L_b valid positions; the Nq new queries
// are its newest Nq positions (query i at L_b − Nq + i) and, when causal, see
// the keys at or before their position. The cache is split along the keys
// into `splits` ranges; one workgroup per (32-row block, split, KV head,
// entry) streams its range of K and V through LDS once and computes, for the
// rows of that block, a partial O over its keys and the matching log-sum-exp.
// The rows are the Hq/Hkv query heads of the KV head times the Nq queries,
// so the cache is read once per KV head, not once per query head. A second
// kernel merges the partials exactly by their log-sum-exp (one exchange step:
// LSE = ln Σ_s e^{LSE_s}, O = Σ_s e^{LSE_s − LSE}·O_s), the identity that also
// merges results computed on different GPUs.
//
// The tile step is the forward's: Sᵀ = K·Qᵀ on MFMA (a lane per row), masking,
// online softmax with a lazily raised reference max, Oᵀ += Vᵀ·Pᵀ with Vᵀ read
// transposed from the row-major LDS tile. The work per byte is small (d FLOP
// per loaded K or V element per row), so the kernel is bound by HBM: K/V tiles
// of 32 keys are copied global -> LDS three stages deep. A workgroup has two
// waves: one only issues the copies and waits for them, the other only
// computes, with one LDS barrier per tile between them. In one wave doing
// both, the copies of the next tile and the arithmetic of the current one
// overlapped poorly (issuing a tile's copies held the wave back), and even a
// few hundred VALU operations per tile cost a large part of the bandwidth; with
// the roles split, the arithmetic hides under the copies. Every
// cache byte is read exactly once, so the copies carry the non-temporal cache
// policy: on MI355X that alone moved a copy-only pass of this access pattern
// from 5.9 to 6.7 TB/s.
//
// An e4m3 cache (the FP8 KV cache of the FlashAttention-2 全解析 page,
// blog.gitcode.com, section 4.3) takes the same path at half the cache bytes: tiles are copied as raw
// codes and each operand is widened to the query's 16-bit type in registers
// (every e4m3 value is exact in bf16 and in fp16), so the products are those
// of the 16-bit kernel on the decoded cache; the per-tensor descales enter
// the score scale (K) and the output normalisation (V).
#include <type_traits>

#include "fa_device.h"
#include "fa_kernels.h"

namespace fa {

namespace {

constexpr int kTK = 32;       // keys per tile
constexpr int kStages = 3;    // K/V tiles in flight or in use
constexpr float kRescaleHeadroom = 8.f;

// s_waitcnt with vmcnt = N (0..63), other counters not waited for
template <int N>
__device__ __forceinline__ void wait_vmem_le() {
  static_assert(N >= 0 && N < 64, "vmcnt holds 0..63");
  __builtin_amdgcn_s_waitcnt(0x0f70 | (N & 15) | ((N >> 4) << 14));
}

// Wait until at most min(newer, MAXN) tiles of PER_TILE copies each are outstanding.
template <int PER_TILE, int MAXN>
__device__ __forceinline__ void wait_tiles(int newer) {
  if constexpr (MAXN <= 0) {
    wait_vmem_le<0>();
  } else {
    if (newer >= MAXN)
      wait_vmem_le<MAXN * PER_TILE>();
    else
      wait_tiles<PER_TILE, MAXN - 1>(newer);
  }
}

// ---- e4m3 cache tiles -------------------------------------------------------
// kTK x D-byte tiles; the 16-byte chunks of row r are stored in the order
// chunk ^ kv8_swz(r). Rows of D bytes put 256 / D rows on one 256-byte sweep
// of the 64 banks; the permutation makes both reads below conflict free:
// 16 lanes reading one chunk of 16 consecutive rows (K), and 32 lanes
// reading 8 consecutive rows x 2 adjacent chunks with the transposing read (V).
template <int D>
__device__ __forceinline__ constexpr int kv8_swz(int r) {
  constexpr int s = D == 64 ? 2 : D == 128 ? 1 : 0;
  return (((r >> s) & (D / 32 - 1)) << 1) | ((r >> 3) & 1);
}

// Copy rows r0 .. r0+kTK-1 of an e4m3 matrix (row stride `rstride` bytes)
// into an LDS tile, 16 bytes per lane and 1 KiB per instruction; rows at or
// past L repeat row L-1 (L >= 1), and the kernel masks those keys.
template <int D>
__device__ __forceinline__ void tile_dma_kv8(uint8_t* lds, const uint8_t* src, int64_t rstride,
                                             int r0, int L, int lane) {
  constexpr int CPR = D / 16;   // chunks per row
  constexpr int RPI = 64 / CPR; // rows per instruction
#pragma unroll
  for (int u = 0; u < kTK / RPI; ++u) {
    const int row = u * RPI + lane / CPR;
    const int c = (lane % CPR) ^ kv8_swz<D>(row);
    const uint8_t* g = src + (int64_t)min(r0 + row, L - 1) * rstride + c * 16;
#if defined(__HIP_DEVICE_COMPILE__)  // the host pass cannot type-check this device builtin
    __builtin_amdgcn_global_load_lds(g, (__attribute__((address_space(3))) void*)(lds + u * 1024),
                                     16, 0, kCpolStream);
#else
    (void)g;
#endif
  }
}

// Per-lane byte offsets of tile_dma_kv8's copies relative to the tile's first
// row, and the buffer-form copy of a tile whose kTK rows all lie inside the
// range (faster to issue than the flat-address form beside other waves' MFMAs).
template <int D>
struct Kv8Plan {
  static constexpr int CPR = D / 16;
  static constexpr int RPI = 64 / CPR;
  static constexpr int PER = kTK / RPI;   // copy instructions per tile
  uint32_t off[PER];
  __device__ __forceinline__ Kv8Plan(int64_t rstride, int lane) {
#pragma unroll
    for (int u = 0; u < PER; ++u) {
      const int row = u * RPI + lane / CPR;
      const int c = (lane % CPR) ^ kv8_swz<D>(row);
      off[u] = (uint32_t)(row * rstride + c * 16);
    }
  }
};
template <int D>
__device__ __forceinline__ void tile_dma_kv8_in(uint8_t* lds, const uint8_t* src_r0,
                                                const Kv8Plan<D>& p) {
#if defined(__HIP_DEVICE_COMPILE__)
  const __amdgpu_buffer_rsrc_t rsrc =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(src_r0), 0, 0x7fffffff, kBufferDword3);
#pragma unroll
  for (int u = 0; u < Kv8Plan<D>::PER; ++u)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        rsrc, (__attribute__((address_space(3))) void*)(lds + u * 1024), 16, p.off[u], 0, 0,
        kCpolStream);
#else
  (void)lds;
  (void)src_r0;
  (void)p;
#endif
}

// Eight e4m3 codes (bytes of w0 then w1, in order) as eight values of T,
// two per dword, lower element first. Exact: e4m3 has 3 mantissa bits and
// exponents 2^-9 .. 2^8, all inside both 16-bit types.
template <typename T>
__device__ __forceinline__ u32x4 widen8(uint32_t w0, uint32_t w1) {
  if constexpr (__is_same(T, bf16)) {
    return u32x4{__builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, 1.f, false)),
                 __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, 1.f, true)),
                 __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, 1.f, false)),
                 __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, 1.f, true))};
  } else {
    return u32x4{__builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w0, 1.f, false)),
                 __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w0, 1.f, true)),
                 __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w1, 1.f, false)),
                 __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w1, 1.f, true))};
  }
}

// Logical chunk c (bytes 16c .. 16c+15) of row r of an e4m3 tile.
template <int D>
__device__ __forceinline__ u32x4 kv8_chunk(const uint8_t* t, int r, int c) {
  return *reinterpret_cast<const u32x4*>(t + r * D + 16 * (c ^ kv8_swz<D>(r)));
}

// Vᵀ operand bytes for columns 32·cb .. +31 and keys k0 .. k0+7: in each
// 16-lane group lanes 2m, 2m+1 address key k0 + m, bytes 0-7 and 8-15 of the
// group's 16-column chunk, and the transposing read hands lane i column i of
// the 8 keys, one byte per key in key order.
template <int D>
__device__ __forceinline__ u32x2 kv8_tr(const uint8_t* t, int k0, int cb, int lane) {
  typedef int i32x2 __attribute__((ext_vector_type(2)));
  typedef __attribute__((address_space(3))) i32x2 lds_i32x2;
  const int j = lane & 15;
  const int row = k0 + (j >> 1), c = 2 * cb + ((lane >> 4) & 1);
  const i32x2 x = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
      (lds_i32x2*)(t + row * D + 16 * (c ^ kv8_swz<D>(row)) + 8 * (j & 1)));
  return __builtin_bit_cast(u32x2, x);
}

// With an e4m3 cache, MFMA row ρ of Sᵀ reads key kv8_key(ρ) of the tile (bits
// 2 and 3 swapped): the accumulator elements that form the P operand of key
// step kk in lane half h then hold keys 16kk + 8h + 0..7 in order, the eight
// consecutive keys one transposing byte read delivers for Vᵀ.
__device__ __forceinline__ constexpr int kv8_key(int rho) {
  return (rho & ~12) | ((rho & 4) << 1) | ((rho & 8) >> 1);
}

template <typename T, bool KV8>
struct CacheElem {
  using type = T;
};
template <typename T>
struct CacheElem<T, true> {
  using type = uint8_t;
};

// EXT: a sliding window of a.wl keys behind each query (keys j >= p − wl stay
// visible; the key ranges then start at the entry's floor L − Nq − wl) and,
// when a.cap_on, soft-capped logits a.cap_out·tanh(z·a.cap_in) (scale_log2 = 1).
template <typename T, int D, bool CAUSAL, bool KV8, bool EXT = false>
__global__ __launch_bounds__(128, D <= 128 ? 2 : 1) void decode_kernel(DecodeArgs a) {
  using C = typename CacheElem<T, KV8>::type;   // cache element: T or an e4m3 code
  constexpr int NKB = D / 16;
  constexpr int NCB = D / 32;
  constexpr int TILE = kTK * D;
  // copy instructions per K or V tile: 16 bytes per lane
  constexpr int PER = kTK * D * (int)sizeof(C) / 1024;
  __shared__ __attribute__((aligned(1024))) C k_lds[kStages][TILE];
  __shared__ __attribute__((aligned(1024))) C v_lds[kStages][TILE];

  // wave 0 copies, wave 1 computes; the wave index is the same on every lane
  // (readfirstlane lets the compiler see that, so branches on it are scalar)
  const int lane = threadIdx.x & 63, col = lane & 31, half = lane >> 5;
  const bool copier = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6) == 0;
  int idx = blockIdx.x;
  const int rb = idx % a.n_rb;
  idx /= a.n_rb;
  const int sp = idx % a.splits;
  idx /= a.splits;
  const int g = idx % a.Hkv, b = idx / a.Hkv;

  const int L = min(max(a.seqlens[b], 0), a.Nk);   // valid cache positions
  // keys before the window of the entry's first query are never visible
  const int k_floor = EXT ? max(0, L - a.Nq - a.wl) : 0;
  const int k_begin = k_floor + sp * a.chunk;
  const int k_end = min(L, k_begin + a.chunk);

  // this lane's row: query head g·group + hg, query i
  const int r = rb * 32 + col;
  const bool row_ok = r < a.rows;
  const int hg = row_ok ? r / a.Nq : 0, qi = row_ok ? r % a.Nq : 0;
  const int h = g * a.group + hg;
  const int qpos = L - a.Nq + qi;                     // the query's position in the sequence
  const int64_t unit = ((int64_t)b * a.Hq + h) * a.Nq + qi;
  const int64_t units = (int64_t)a.B * a.Hq * a.Nq;
  float* po = a.part_o + ((int64_t)sp * units + unit) * D;
  float* pl = a.part_lse + (int64_t)sp * units + unit;

  f32x16 o[NCB];
#pragma unroll
  for (int cb = 0; cb < NCB; ++cb) o[cb] = f32x16{};
  float mc = -INFINITY, l = 0.f, lr = 0.f;   // lr: row sum of P as rounded to T

  if (k_begin < k_end) {
    const int64_t kvs = (int64_t)a.Hkv * D;
    const C* kp = static_cast<const C*>(a.k) + (int64_t)b * a.Nk * kvs + (int64_t)g * D;
    const C* vp = static_cast<const C*>(a.v) + (int64_t)b * a.Nk * kvs + (int64_t)g * D;
    const int ntiles = (k_end - k_begin + kTK - 1) / kTK;
    // copies of tile t into its stage: a tile inside the range from its first
    // row's address with the buffer form; the range's ragged last tile with the
    // flat form, whose rows past k_end repeat row k_end-1 (masked below)
    auto issue = [&](int t, const auto& plan) __attribute__((always_inline)) {
      C* kd = k_lds[t % kStages];
      C* vd = v_lds[t % kStages];
      const int r0 = k_begin + t * kTK;
      if (r0 + kTK <= k_end) {
        if constexpr (KV8) {
          tile_dma_kv8_in<D>(kd, kp + (int64_t)r0 * kvs, plan);
          tile_dma_kv8_in<D>(vd, vp + (int64_t)r0 * kvs, plan);
        } else {
          tile_dma_in<T, kTK, D, 1, kCpolStream>(kd, kp + (int64_t)r0 * kvs, plan, 0);
          tile_dma_in<T, kTK, D, 1, kCpolStream>(vd, vp + (int64_t)r0 * kvs, plan, 0);
        }
      } else if constexpr (KV8) {
        tile_dma_kv8<D>(kd, kp, kvs, r0, k_end, lane);
        tile_dma_kv8<D>(vd, vp, kvs, r0, k_end, lane);
      } else {
        tile_dma<T, kTK, D, 1, kCpolStream>(kd, kp, kvs, r0, k_end, 0, lane);
        tile_dma<T, kTK, D, 1, kCpolStream>(vd, vp, kvs, r0, k_end, 0, lane);
      }
    };
    if (copier) {
      // Each role runs its own loop (one barrier per tile in each, the same
      // count), so neither role's loop state takes registers from the other.
      // Iteration t: start tile t+kStages-1 into the stage tile t-1 left (the
      // computing wave is done with it, by the previous barrier), then wait
      // until tile t+1 has landed (at most kStages-2 newer tiles outstanding).
      using Plan = std::conditional_t<KV8, Kv8Plan<D>, DmaPlan<T, kTK, D, 1>>;
      const Plan plan = [&] {
        if constexpr (KV8) return Kv8Plan<D>(kvs, lane);
        else return DmaPlan<T, kTK, D, 1>(kvs, 0, lane);
      }();
#pragma unroll
      for (int p = 0; p < kStages - 1; ++p)
        if (p < ntiles) issue(p, plan);
      wait_tiles<2 * PER, kStages - 2>(ntiles - 1);
      lds_barrier();   // tile 0 is in LDS
      for (int t = 0; t < ntiles; ++t) {
        if (t + kStages - 1 < ntiles) issue(t + kStages - 1, plan);
        wait_tiles<2 * PER, kStages - 2>(ntiles - 2 - t);
        lds_barrier();   // tile t+1 is in LDS; tile t is no longer read
      }
      return;
    }
    u32x4 qf[NKB];
    {
      const T* qp = static_cast<const T*>(a.q) + (((int64_t)b * a.Nq + qi) * a.Hq + h) * D;
      // k step kb covers head columns 16kb + 8h .. +7 in lane half h; with an
      // e4m3 cache one 16-byte K read serves two steps, so step 2m + u covers
      // columns 32m + 16h + 8u .. +7 instead (the same columns for both operands)
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
        const int col0 = KV8 ? 32 * (kb >> 1) + 16 * half + 8 * (kb & 1) : kb * 16 + half * 8;
        qf[kb] = row_ok ? ldg16(qp + col0) : u32x4{0, 0, 0, 0};
      }
    }
    const float c = a.scale_log2;
    const int krow = KV8 ? kv8_key(col) : col;   // the tile row MFMA row `col` reads

    // the computing wave's step: consume tile t from the stage (kt, vt)
    auto step = [&](const C* kt, const C* vt, int t) __attribute__((always_inline)) {
      const int kbase = k_begin + t * kTK;

      f32x16 s = f32x16{};
      if constexpr (KV8) {
#pragma unroll
        for (int m = 0; m < NKB / 2; ++m) {
          const u32x4 raw = kv8_chunk<D>(kt, krow, 2 * m + half);
          s = mfma32<T>(widen8<T>(raw[0], raw[1]), qf[2 * m], s);
          s = mfma32<T>(widen8<T>(raw[2], raw[3]), qf[2 * m + 1], s);
        }
      } else {
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
          s = mfma32<T>(lds_row16<T, D>(kt, krow, 2 * kb + half), qf[kb], s);
      }

      if constexpr (EXT) {
        if (a.cap_on) {   // uniform
#pragma unroll
          for (int i = 0; i < 16; ++i) s[i] = a.cap_out * tanh_fast(s[i] * a.cap_in);
        }
      }
      // mask keys past the range and, causally, keys after the query
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int rho = 8 * (i >> 2) + 4 * half + (i & 3);   // accumulator row of s[i]
        const int kj = kbase + (KV8 ? kv8_key(rho) : rho);
        bool vis = kj < k_end && !(CAUSAL && kj > qpos);
        if constexpr (EXT) vis = vis && kj >= qpos - a.wl;
        s[i] = vis ? s[i] : -INFINITY;
      }
      float mx = s[0];
#pragma unroll
      for (int i = 1; i < 16; ++i) mx = fmaxf(mx, s[i]);
      const float mxc = wave_max_halves(mx) * c;
      if (__builtin_amdgcn_ballot_w64(mxc > mc + kRescaleHeadroom) != 0) {
        const float mc_new = fmaxf(mc, mxc);
        // a row that has seen no key yet keeps mc = −inf and nothing to scale
        const float alpha = mc_new == -INFINITY ? 1.f : fast_exp2(mc - mc_new);
        l *= alpha;
        lr *= alpha;
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb) o[cb] *= alpha;
        mc = mc_new;
      }
      const float mcs = mc == -INFINITY ? 0.f : mc;   // all of such a row's scores are −inf
      float ls[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        s[i] = fast_exp2(fmaf(s[i], c, -mcs));
        if constexpr (kLseFromUnrounded<T>) ls[i & 3] += s[i];
      }
      if constexpr (kLseFromUnrounded<T>) l += (ls[0] + ls[1]) + (ls[2] + ls[3]);
#pragma unroll
      for (int kk = 0; kk < kTK / 16; ++kk) {
        const u32x4 pf = acc_operand<T>(s, kk * 2);
        lr = dot2_sum<T>(pf, lr);   // the same sum over P as rounded for the MFMAs
        if constexpr (KV8) {
#pragma unroll
          for (int cb = 0; cb < NCB; ++cb) {
            const u32x2 vb = kv8_tr<D>(vt, kk * 16 + 8 * half, cb, lane);
            o[cb] = mfma32<T>(widen8<T>(vb[0], vb[1]), pf, o[cb]);
          }
        } else {
          const int k0 = kk * 16 + 4 * half;
#pragma unroll
          for (int cb = 0; cb < NCB; ++cb)
            o[cb] = mfma32<T>(lds_tr8<T, D>(vt, k0, k0 + 8, cb * 32, lane), pf, o[cb]);
        }
      }
    };

    lds_barrier();   // tile 0 is in LDS
    for (int t = 0; t < ntiles; ++t) {
      step(k_lds[t % kStages], v_lds[t % kStages], t);
      lds_barrier();   // done with tile t; tile t+1 is in LDS
    }
  }

  // partial result of this split: normalised O and its LSE (−inf, O = 0 if no key)
  // O is normalised by the sum of the rounded P that the MFMAs consumed;
  // the LSE as in kLseFromUnrounded
  if (copier) return;   // (a workgroup with an empty key range)
  const float lr_tot = wave_sum_halves(lr);
  const float l_tot = kLseFromUnrounded<T> ? wave_sum_halves(l) : lr_tot;
  if (row_ok) {
    const bool any = l_tot > 0.f;
    const float inv = any ? a.o_scale / lr_tot : 0.f;   // o_scale: descale of V (1 for T)
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        float4 w;
        w.x = o[cb][4 * rr + 0] * inv;
        w.y = o[cb][4 * rr + 1] * inv;
        w.z = o[cb][4 * rr + 2] * inv;
        w.w = o[cb][4 * rr + 3] * inv;
        *reinterpret_cast<float4*>(po + cb * 32 + 8 * rr + 4 * half) = w;
      }
    if (half == 0) *pl = any ? (mc + log2f(l_tot)) * kLn2 : -INFINITY;
  }
}

// Merge of the splits for one (entry, query head, query) row per wave:
// LSE = m + ln Σ_s e^{LSE_s − m}, O = Σ_s e^{LSE_s − LSE}·O_s (m = max_s LSE_s).
// The lanes load the splits' LSEs in parallel (64 at a time); each split's
// weight is then broadcast and its partial O rows accumulated, so the loads
// of different splits are independent of each other.
template <typename T, int D>
__global__ __launch_bounds__(256) void decode_combine_kernel(DecodeArgs a) {
  constexpr int PER_LANE = D / 64;
  constexpr int BLK = 16;   // splits whose partial rows are loaded together
  const int64_t units = (int64_t)a.B * a.Hq * a.Nq;
  const int64_t unit = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (unit >= units) return;   // whole waves leave together (unit is wave-uniform)
  const float* pl = a.part_lse + unit;
  const float* po = a.part_o + unit * D + PER_LANE * lane;
  const int64_t ostride = units * D;   // between the partial rows of consecutive splits
  // The first 64 splits' LSEs (one per lane) and the first BLK splits'
  // partial rows are loaded before anything waits for them: with at most BLK
  // splits the merge takes one memory round trip.
  const float ls0 = lane < a.splits ? pl[(int64_t)lane * units] : -INFINITY;
  float vals[BLK][PER_LANE];
#pragma unroll
  for (int u = 0; u < BLK; ++u)
#pragma unroll
    for (int e = 0; e < PER_LANE; ++e) vals[u][e] = u < a.splits ? po[u * ostride + e] : 0.f;
  float m = ls0;
  for (int sp = lane + 64; sp < a.splits; sp += 64) m = fmaxf(m, pl[(int64_t)sp * units]);
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) m = fmaxf(m, __shfl_xor(m, off));
  float acc[PER_LANE] = {};
  float wsum = 0.f;
  if (m != -INFINITY) {
    for (int base = 0; base < a.splits; base += 64) {
      const int sp = base + lane;
      const float ls = base == 0 ? ls0 : sp < a.splits ? pl[(int64_t)sp * units] : -INFINITY;
      const float w = ls == -INFINITY ? 0.f : expf(ls - m);   // a split with no key weighs 0
      const int cnt = min(64, a.splits - base);   // uniform
      for (int j0 = 0; j0 < cnt; j0 += BLK) {
        if (base > 0 || j0 > 0) {   // later blocks: loaded together, then accumulated
#pragma unroll
          for (int u = 0; u < BLK; ++u)
#pragma unroll
            for (int e = 0; e < PER_LANE; ++e)
              vals[u][e] = j0 + u < cnt ? po[(int64_t)(base + j0 + u) * ostride + e] : 0.f;
        }
#pragma unroll
        for (int u = 0; u < BLK; ++u) {
          const float wj = j0 + u < cnt ? __shfl(w, j0 + u) : 0.f;
          wsum += wj;
#pragma unroll
          for (int e = 0; e < PER_LANE; ++e) acc[e] = fmaf(wj, vals[u][e], acc[e]);
        }
      }
    }
  }
  const int qi = (int)(unit % a.Nq);
  const int64_t bh = unit / a.Nq;
  const int h = (int)(bh % a.Hq), b = (int)(bh / a.Hq);
  T* op = static_cast<T*>(a.o) + (((int64_t)b * a.Nq + qi) * a.Hq + h) * D;
  const float inv = wsum > 0.f ? 1.f / wsum : 0.f;
  if constexpr (PER_LANE == 4) {
    u32x2 w;
    w[0] = pack2<T>(acc[0] * inv, acc[1] * inv);
    w[1] = pack2<T>(acc[2] * inv, acc[3] * inv);
    *reinterpret_cast<u32x2*>(op + 4 * lane) = w;
  } else if constexpr (PER_LANE == 2) {
    *reinterpret_cast<uint32_t*>(op + 2 * lane) = pack2<T>(acc[0] * inv, acc[1] * inv);
  } else {
    op[lane] = static_cast<T>(acc[0] * inv);
  }
  if (lane == 0)
    a.lse[(int64_t)h * a.B * a.Nq + (int64_t)b * a.Nq + qi] =
        wsum > 0.f ? m + logf(wsum) : -INFINITY;
}

template <typename T, int D, bool CAUSAL, bool KV8, bool EXT = false>
hipError_t launch(const DecodeArgs& a, int stage, hipStream_t s) {
  (void)hipGetLastError();  // drop an error left pending by earlier, unrelated HIP calls
  if (stage < 0 || stage == 0) {
    const int64_t g1 = (int64_t)a.n_rb * a.splits * a.Hkv * a.B;
    hipLaunchKernelGGL((decode_kernel<T, D, CAUSAL, KV8, EXT>), dim3((unsigned)g1), dim3(128), 0,
                       s, a);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (stage < 0 || stage == 1) {
    const int64_t units = (int64_t)a.B * a.Hq * a.Nq;
    hipLaunchKernelGGL((decode_combine_kernel<T, D>), dim3((unsigned)((units + 3) / 4)),
                       dim3(256), 0, s, a);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

// Resident two-wave workgroups of one decode_kernel instantiation per CU, as
// the runtime computes them from its LDS and register allocation; 0 if the
// runtime cannot tell (no device).
template <typename T, int D, bool CAUSAL, bool KV8>
int occupancy() {
  int n = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(
          &n, reinterpret_cast<const void*>(&decode_kernel<T, D, CAUSAL, KV8>), 128, 0) !=
      hipSuccess) {
    (void)hipGetLastError();
    return 0;
  }
  return n;
}

template <typename T, bool KV8>
int occupancy_of(int d, bool causal) {
  if (d == 64) return causal ? occupancy<T, 64, true, KV8>() : occupancy<T, 64, false, KV8>();
  if (d == 128) return causal ? occupancy<T, 128, true, KV8>() : occupancy<T, 128, false, KV8>();
  return causal ? occupancy<T, 256, true, KV8>() : occupancy<T, 256, false, KV8>();
}

template <typename T, bool KV8>
hipError_t dispatch(const DecodeArgs& a, int d, bool causal, int stage, hipStream_t s) {
  if (d == 64)
    return causal ? launch<T, 64, true, KV8>(a, stage, s) : launch<T, 64, false, KV8>(a, stage, s);
  if (d == 128)
    return causal ? launch<T, 128, true, KV8>(a, stage, s) : launch<T, 128, false, KV8>(a, stage, s);
  return causal ? launch<T, 256, true, KV8>(a, stage, s) : launch<T, 256, false, KV8>(a, stage, s);
}

}  // namespace

int decode_tile_keys() { return kTK; }
int decode_num_stages() { return 2; }

int decode_resident_per_cu(bool bf16_in, int d, bool causal, bool kv8) {
  if (bf16_in)
    return kv8 ? occupancy_of<bf16, true>(d, causal) : occupancy_of<bf16, false>(d, causal);
  return kv8 ? occupancy_of<f16, true>(d, causal) : occupancy_of<f16, false>(d, causal);
}

int decode_lds_bytes(int d, bool kv8) { return kStages * 2 * kTK * d * (kv8 ? 1 : 2); }

template <typename T>
static hipError_t dispatch_ext(const DecodeArgs& a, int d, bool causal, int stage, hipStream_t s) {
  if (d == 64)
    return causal ? launch<T, 64, true, false, true>(a, stage, s)
                  : launch<T, 64, false, false, true>(a, stage, s);
  if (d == 128)
    return causal ? launch<T, 128, true, false, true>(a, stage, s)
                  : launch<T, 128, false, false, true>(a, stage, s);
  return causal ? launch<T, 256, true, false, true>(a, stage, s)
                : launch<T, 256, false, false, true>(a, stage, s);
}

hipError_t launch_decode_ext(const DecodeArgs& a, bool bf16_in, int d, bool causal, int stage,
                             hipStream_t s) {
  return bf16_in ? dispatch_ext<bf16>(a, d, causal, stage, s)
                 : dispatch_ext<f16>(a, d, causal, stage, s);
}

hipError_t launch_decode(const DecodeArgs& a, bool bf16_in, int d, bool causal, bool kv8,
                         int stage, hipStream_t s) {
  if (bf16_in)
    return kv8 ? dispatch<bf16, true>(a, d, causal, stage, s)
               : dispatch<bf16, false>(a, d, causal, stage, s);
  return kv8 ? dispatch<f16, true>(a, d, causal, stage, s)
             : dispatch<f16, false>(a, d, causal, stage, s);
}

}  // namespace fa
