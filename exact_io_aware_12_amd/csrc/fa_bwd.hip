// Fused attention backward for gfx950.
//
// The probabilities are never stored: each kernel recomputes S from Q and K
// tiles and P = exp(S·scale − LSE) from the forward's row log-sum-exp
// (recomputation in the backward pass, FlashAttention guide, cxbdf.cn,
// part 2, item 3). With dP = dO·Vᵀ and D_i = rowsum(dO∘O) (equal to
// Σ_j P_ij·dP_ij because O_i = Σ_j P_ij·V_j):
//   dS = P∘(dP − D),  dV = Pᵀ·dO,  dK = scale·dSᵀ·Q,  dQ = scale·dS·K.
//
// Three kernels (stages 0, 1, 2) on one stream, all deterministic (fixed
// summation order); stages 1 and 2 both depend on stage 0 only:
//   delta_kernel  D = rowsum(dO∘O) and LSE·log2 e, float32      (HBM bound)
//   dkdv_kernel   one workgroup per 128-key tile of one KV head; loops over
//                 the query heads of its group and the visible 64-query
//                 tiles; dKᵀ and dVᵀ accumulate in registers
//   dq_kernel     one workgroup per 128-query tile of one query head; loops
//                 over the visible 64-key tiles; dQᵀ accumulates in registers
// Q/dO (stage 1) and K/V (stage 2) tiles are copied global -> LDS directly,
// double-buffered, one barrier per tile. The transposed operands (Qᵀ, dOᵀ,
// Kᵀ) are read from the same row-major tiles with the transposing LDS read.
#include <type_traits>

#include "fa_device.h"
#include "fa_kernels.h"

namespace fa {

namespace {

constexpr int kThreads = 256;
constexpr int kWaves = 4;

// A sequence's queries (first token, count, tokens of the batch) and keys
// (first token, count); off = Lk − L is the key position of query 0 (0 unless
// KVLEN: the queries are the last L of the Lk positions).
struct SeqInfo {
  int seq0, L, T;
  int seq0k, Lk, off;
};

template <bool VARLEN, bool KVLEN = false>
__device__ __forceinline__ SeqInfo seq_info(const BwdArgs& a, int b) {
  SeqInfo r;
  if constexpr (VARLEN) {
    r.seq0 = a.cu_seqlens[b];
    r.L = a.cu_seqlens[b + 1] - r.seq0;
    r.T = a.cu_seqlens[a.B];
  } else {
    r.seq0 = b * a.N;
    r.L = a.N;
    r.T = a.B * a.N;
  }
  if constexpr (KVLEN) {
    if constexpr (VARLEN) {
      r.seq0k = a.cu_seqlens_k[b];
      r.Lk = a.cu_seqlens_k[b + 1] - r.seq0k;
    } else {
      r.seq0k = b * a.Nk;
      r.Lk = a.Nk;
    }
  } else {
    r.seq0k = r.seq0;
    r.Lk = r.L;
  }
  r.off = r.Lk - r.L;
  return r;
}

template <typename T>
__device__ __forceinline__ float lo_f(uint32_t w) {
  if constexpr (__is_same(T, bf16)) return __uint_as_float(w << 16);
  else return (float)__builtin_bit_cast(f16, (uint16_t)(w & 0xffffu));
}
template <typename T>
__device__ __forceinline__ float hi_f(uint32_t w) {
  if constexpr (__is_same(T, bf16)) return __uint_as_float(w & 0xffff0000u);
  else return (float)__builtin_bit_cast(f16, (uint16_t)(w >> 16));
}

// ---------------------------------------------------------------------------
// D_i = Σ_c dO[i,c]·O[i,c] and LSE_i·log2 e; D/8 consecutive threads share one
// (head, token) row.
template <typename T, int D, bool VARLEN>
__global__ __launch_bounds__(kThreads) void delta_kernel(BwdArgs a) {
  constexpr int TPR = D / 8;
  const int T_total = VARLEN ? a.cu_seqlens[a.B] : a.B * a.N;
  const int64_t rows = (int64_t)T_total * a.Hq;
  const int64_t row = (int64_t)blockIdx.x * (kThreads / TPR) + threadIdx.x / TPR;
  const int part = threadIdx.x % TPR;
  float acc = 0.f;
  // rows are ordered head-major (row = h·T + t) so that consecutive groups
  // write consecutive entries of the [head][token] workspace
  const int h = (int)(row / T_total), t = (int)(row - (int64_t)h * T_total);
  const int64_t src = ((int64_t)t * a.Hq + h) * D + part * 8;
  if (row < rows) {
    const u32x4 x = ldg16(static_cast<const T*>(a.dout) + src);
    const u32x4 y = ldg16(static_cast<const T*>(a.o) + src);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      acc = fmaf(lo_f<T>(x[i]), lo_f<T>(y[i]), acc);
      acc = fmaf(hi_f<T>(x[i]), hi_f<T>(y[i]), acc);
    }
  }
#pragma unroll
  for (int off = TPR / 2; off > 0; off >>= 1) acc += __shfl_xor(acc, off);
  if (row < rows && part == 0) {
    a.delta[(int64_t)h * a.ws_stride + t] = acc;
    a.lse2[(int64_t)h * a.ws_stride + t] = a.lse[(int64_t)h * T_total + t] * kLog2e;
  }
}

// Copy R floats of LSE·log2 e and of D (rows q0 .. q0+R-1 of one head) into
// lds[0..R-1] and lds[R..2R-1]: one instruction, lanes 0 .. R/2-1 of one wave.
// Rows past the sequence end read neighbouring workspace entries; the callers
// mask those rows.
// Buffer-form copies (one per array, on that array's lanes): they issue far
// faster than flat-address copies beside the MFMA work of other waves.
template <int R>
__device__ __forceinline__ void rows_dma(float* lds, const float* lse2, const float* delta,
                                         int lane) {
  constexpr int LN = R / 4;   // lanes per array
#if defined(__HIP_DEVICE_COMPILE__)
  typedef __attribute__((address_space(3))) void lds_void;
  if (lane < LN) {
    const __amdgpu_buffer_rsrc_t r =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(lse2), 0, 0x7fffffff, kBufferDword3);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)lds, 16, 16 * lane, 0, 0, 0);
  } else if (lane < 2 * LN) {
    const __amdgpu_buffer_rsrc_t r =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(delta), 0, 0x7fffffff, kBufferDword3);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)lds, 16, 16 * (lane - LN), 0, 0, 0);
  }
#else
  (void)lds;
  (void)lse2;
  (void)delta;
  (void)lane;
#endif
}

// ---------------------------------------------------------------------------
// dK, dV. Orientation S = Q·Kᵀ with 32 keys as MFMA columns, so the
// accumulators of P and dS hold one key per lane and 16 queries in
// registers, which is exactly the B-operand layout dVᵀ = dOᵀ·P and
// dKᵀ = Qᵀ·dS need.
//
// A workgroup owns 128 keys of one KV head and runs 8 waves, two per SIMD:
// waves w and w+4 share keys k0+32w .. k0+32w+31. Wave w (producer) keeps K
// and V of those keys in registers and turns a 64-query tile into P and dS
// (S and dP by MFMA, then the softmax gradient on the VALU); wave w+4
// (consumer) keeps dKᵀ and dVᵀ in registers and runs the dVᵀ += dOᵀ·P and
// dKᵀ += Qᵀ·dS products. P and dS pass through LDS in operand layout. The
// consumer works one tile behind the producer, so one wave's VALU work
// overlaps the other's MFMAs on the same SIMD.
//
// Per iteration j (j = -1 .. ntile-1), after one workgroup barrier A (tile
// j+1's Q, dO, LSE and D have landed; the copy of tile j+2 starts into the
// stage that tile j-1 used and has until the next A to land):
//   consumer: P, dS of tile j from LDS into registers, then releases its
//      pair's exchange buffer (an LDS flag) and runs the dK/dV products;
//   producer: waits for its own consumer's release only (not for the whole
//      workgroup), then S, dP, P and dS of tile j+1 into the buffer.
// Q/dO tiles take 3 stages: j (consumer), j+1 (producer), j+2 (in flight).
constexpr int kDkvKeys = 128;     // keys per workgroup (32 per wave pair)
constexpr int kDkvQ = 64;         // queries per tile
constexpr int kDkvWaves = 8;      // 4 producers, 4 consumers
constexpr int kDkvThreads = 64 * kDkvWaves;
constexpr int kDkvStages = 3;
constexpr int kDkvKK = kDkvQ / 16;   // 16-query MFMA k-steps per tile

// Hand-over of a pair's P/dS buffer. The consumer of a pair releases
// iteration j once its reads of the buffer (tile j's P and dS) have returned;
// the producer acquires iteration j just before it overwrites the buffer with
// tile j+1. The consumer never waits for the producer inside an iteration, so
// every release happens; the spin is bounded all the same.
constexpr int kHandSpinLimit = 1 << 20;

typedef volatile __attribute__((address_space(3))) int lds_flag_t;

__device__ __forceinline__ void pair_release(const int* flag, int j) {
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");   // the buffer reads have returned
  *(lds_flag_t*)(uintptr_t)lds_addr(flag) = j;
}

__device__ __forceinline__ void pair_acquire(const int* flag, int j) {
  lds_flag_t* f = (lds_flag_t*)(uintptr_t)lds_addr(flag);
  for (int spin = 0; spin < kHandSpinLimit; ++spin) {
    if (__builtin_amdgcn_readfirstlane(*f) >= j) break;
    __builtin_amdgcn_s_sleep(1);
  }
  asm volatile("" ::: "memory");   // the buffer writes stay after the wait
}

// Producer: P and dS of one 64-query tile for 32 keys, written to `xp`
// (P) and `xs` (dS) as MFMA B operands, [k-step][lane]. EDGE tiles zero P
// and dS for queries past the end and, causally, for keys after the query.
// CAP: soft-capped logits, s = cap_out·tanh(z·cap_in) in log2 units; dS then
// carries the derivative factor 1 − tanh² (the scale is applied at the end).
// DROP: dropout; the P handed to dV is P∘Z and dS = P∘(Z∘dP − D), with
// Z = 256/t where the weight is kept and 0 where it is dropped.
template <typename T, int D, bool CAUSAL, bool EDGE, bool WIN, bool CAP = false, bool DROP = false>
__device__ __forceinline__ void dkdv_produce(const T* qt_, const T* dot_, const float* ld,
                                             const u32x4 (&kf)[D / 16],
                                             const u32x4 (&vf)[D / 16], u32x4* xp, u32x4* xs,
                                             float c, int q0, int L, int key, int wl, int wr,
                                             int lane, float cap_in = 0.f, float cap_out = 0.f,
                                             const DropKey* dk = nullptr, int seq = 0,
                                             int head = 0, float zs = 0.f, int off = 0,
                                             const int* hand = nullptr, int hand_j = 0) {
  constexpr int NKB = D / 16;
  constexpr int NQB = kDkvQ / 32;
  const int col = lane & 31, half = lane >> 5;
  constexpr uint32_t QBLK = 32 * D * sizeof(T);   // 32 rows
  // Per 32-query block: S and dP by MFMA, with the Q and dO operands read
  // two k-steps ahead of their MFMAs across the whole tile (so the next
  // block's first operands are in flight during this block's arithmetic).
  constexpr int AHEAD = 2, NSTEP = NQB * NKB;
  // The buffer is written below, so the consumer must have read it first.
  // The wait sits right before the first write, where the consumer has
  // finished long since; with a soft cap or dropout, whose tiles need more
  // registers, it sits before the tile instead, since a wait inside the tile
  // splits its code and makes the compiler spill (measured on train_16k: the
  // late wait made dK/dV 3.7 % faster than the early one).
  constexpr bool kLateWait = !CAP && !DROP;
  if constexpr (!kLateWait) pair_acquire(hand, hand_j);
  u32x4 qa[AHEAD + 1], da[AHEAD + 1];
  auto fetch = [&](int step) __attribute__((always_inline)) {
    const int qb = step / NKB, kb = step % NKB;
    const uint32_t off = row16_off<D>(col, 2 * kb + half) + qb * QBLK;
    qa[step % (AHEAD + 1)] = lds_at16<T>(qt_, off);
    da[step % (AHEAD + 1)] = lds_at16<T>(dot_, off);
  };
#pragma unroll
  for (int st = 0; st < AHEAD; ++st) fetch(st);
#pragma unroll
  for (int qb = 0; qb < NQB; ++qb) {
    f32x16 s = f32x16{}, dp = f32x16{};
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
      const int st = qb * NKB + kb;
      if (st + AHEAD < NSTEP) fetch(st + AHEAD);
      s = mfma32<T>(qa[st % (AHEAD + 1)], kf[kb], s);
      dp = mfma32<T>(da[st % (AHEAD + 1)], vf[kb], dp);
    }
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) {
      const int qoff = qb * 32 + 8 * rr + 4 * half;
      const float4 lv = *reinterpret_cast<const float4*>(ld + qoff);
      const float4 dv4 = *reinterpret_cast<const float4*>(ld + kDkvQ + qoff);
      const float lsev[4] = {lv.x, lv.y, lv.z, lv.w};
      const float dlv[4] = {dv4.x, dv4.y, dv4.z, dv4.w};
      // queries q0 + qoff + 0..3 of this lane's key; one generator call per run
      // (sharing calls across the key quad, as the forward does, measured slower here)
      uint32_t dbytes = 0;
      if constexpr (DROP) dbytes = drop_col_bytes(*dk, seq, head, q0 + qoff, key);
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const int i4 = 4 * rr + t;
        float p, ds;
        if constexpr (CAP) {
          const float th = tanh_fast(s[i4] * cap_in);
          p = fast_exp2(fmaf(th, cap_out, -lsev[t]));
          ds = p * (dp[i4] - dlv[t]) * fmaf(-th, th, 1.f);
        } else if constexpr (DROP) {
          p = fast_exp2(fmaf(s[i4], c, -lsev[t]));
          const float z = drop_keep(dbytes, t, dk->t) ? zs : 0.f;
          ds = p * fmaf(dp[i4], z, -dlv[t]);
          p *= z;
        } else {
          p = fast_exp2(fmaf(s[i4], c, -lsev[t]));
          ds = p * (dp[i4] - dlv[t]);
        }
        if constexpr (EDGE) {
          const int q = q0 + qoff + t;
          bool keep = q < L && !(CAUSAL && key > q + off);
          if constexpr (WIN) keep = keep && q >= key - wr && q <= key + wl;
          p = keep ? p : 0.f;
          ds = keep ? ds : 0.f;
        }
        s[i4] = p;
        dp[i4] = ds;
      }
    }
    if (kLateWait && qb == 0) pair_acquire(hand, hand_j);
#pragma unroll
    for (int h2 = 0; h2 < 2; ++h2) {
      xp[(2 * qb + h2) * 64 + lane] = acc_operand<T>(s, h2 * 2);
      xs[(2 * qb + h2) * 64 + lane] = acc_operand<T>(dp, h2 * 2);
    }
  }
}

// WIN: sliding window (see fwd_kernel); CAUSAL is false then
// KVLEN: keys of their own length (see seq_info); no window, cap or dropout
template <typename T, int D, bool CAUSAL, bool VARLEN, bool WIN, bool CAP = false,
          bool DROP = false, bool KVLEN = false>
__global__ __launch_bounds__(kDkvThreads, 1) void dkdv_kernel(BwdArgs a, int n_ktiles) {
  constexpr int NKB = D / 16;
  constexpr int NCB = D / 32;
  constexpr int TILE = kDkvQ * D;
  __shared__ __attribute__((aligned(1024))) T qd_lds[kDkvStages][2][TILE];   // [stage][Q, dO]
  __shared__ __attribute__((aligned(16))) float ld_lds[kDkvStages][2 * kDkvQ];  // LSE·log2 e, D
  __shared__ __attribute__((aligned(16))) u32x4 xch[4][2][kDkvKK * 64];   // [pair][P, dS]
  __shared__ int hand[4];   // per pair: the last iteration whose P/dS the consumer has read

  // the wave index is the same on every lane: readfirstlane lets the compiler
  // see that, so branches on it are scalar rather than divergent
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int pair = wave & 3;
  const bool producer = wave < 4;
  const int col = lane & 31, half = lane >> 5;
  if (tid < 4) hand[tid] = -2;   // ordered before any use by the first barrier A

  const int G = gridDim.x;
  const int logical = xcd_remap(blockIdx.x, G);
  const int kt = logical % n_ktiles;           // ascending = heaviest first when causal
  const int gb = logical / n_ktiles;
  const int b = gb % a.B, g = gb / a.B;   // sequence fastest: XCD ranges balanced for varlen
  const SeqInfo si = seq_info<VARLEN, KVLEN>(a, b);
  const int k0 = kt * kDkvKeys;
  if (k0 >= si.Lk) return;
  const int L = si.L, Lk = si.Lk, off = si.off;   // queries, keys, key position of query 0

  const int64_t qs = (int64_t)a.Hq * D, kvs = (int64_t)a.Hkv * D;
  const int key = k0 + pair * 32 + col;
  const int pk_first = k0 + pair * 32;   // first key of this wave pair

  // Query tiles of one head: [qt_lo, qt_hi) hold every query that sees a key
  // of the block; [qi_lo, qi_hi) need no masking (each of their queries sees
  // every key of the block). The rest are edge tiles: the causal diagonal or
  // the window's two ends, and a ragged last tile. The edge tiles of every
  // head of the group come first, then the interior ones.
  int qt_lo, qi_lo, qi_hi, qt_hi;
  const int wl = WIN ? a.wl : 0, wr = WIN ? a.wr : 0;
  if constexpr (WIN) {
    qt_lo = max(0, k0 - wr) / kDkvQ;
    qt_hi = (min(L, k0 + kDkvKeys + wl) + kDkvQ - 1) / kDkvQ;
    const int first_all = min(k0 + kDkvKeys, L) - 1 - wr;   // first query seeing every key
    qi_lo = min(max(qt_lo, first_all <= 0 ? 0 : (first_all + kDkvQ - 1) / kDkvQ), qt_hi);
    const int last_all = k0 + wl - (kDkvQ - 1);   // a tile starting here ends at k0 + wl
    qi_hi = min(min(last_all < 0 ? 0 : last_all / kDkvQ + 1, L / kDkvQ), qt_hi);
    if (qi_hi < qi_lo) qi_hi = qi_lo;
  } else if constexpr (KVLEN) {
    // causal: query i sees key j iff j <= i + off. Tiles from the one holding
    // the first query that sees key k0; interior from the first query that
    // sees every key of the block (keys past Lk never reach dK, dV)
    qt_hi = (L + kDkvQ - 1) / kDkvQ;
    qt_lo = CAUSAL ? min(max(0, k0 - off) / kDkvQ, qt_hi) : 0;
    const int first_all = CAUSAL ? min(k0 + kDkvKeys, Lk) - 1 - off : 0;
    qi_lo = min(max(qt_lo, first_all <= 0 ? 0 : (first_all + kDkvQ - 1) / kDkvQ), qt_hi);
    qi_hi = max(qi_lo, qt_hi - (L % kDkvQ != 0 ? 1 : 0));
  } else {
    qt_lo = CAUSAL ? k0 / kDkvQ : 0;
    qt_hi = (L + kDkvQ - 1) / kDkvQ;
    const int nd = CAUSAL ? min(kDkvKeys / kDkvQ, qt_hi - qt_lo) : 0;
    qi_lo = qt_lo + nd;
    qi_hi = max(qi_lo, qt_hi - ((L % kDkvQ != 0 && qt_hi - qt_lo > nd) ? 1 : 0));
  }
  const int ne_lo = qi_lo - qt_lo, ne = ne_lo + (qt_hi - qi_hi), ni = qi_hi - qi_lo;
  const int n_edge = a.group * ne, ntile = a.group * (qt_hi - qt_lo);
  auto tile_of = [&](int i, int& r) -> int {   // tile i -> (head r, query tile)
    if (i < n_edge) {
      r = i / ne;
      const int e = i - r * ne;
      return e < ne_lo ? qt_lo + e : qi_hi + (e - ne_lo);
    }
    const int j = i - n_edge;
    r = j / ni;
    return qi_lo + (j - r * ni);
  };
  // whether a query tile holds no query that sees any key of this wave pair
  auto pair_idle = [&](int q0) -> bool {
    if (CAUSAL && q0 + kDkvQ - 1 + off < pk_first) return true;
    if (WIN && (q0 + kDkvQ - 1 < pk_first - wr || q0 > pk_first + 31 + wl)) return true;
    return false;
  };
  const DmaPlan<T, kDkvQ, D, kDkvWaves> plan(qs, wave, lane);
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);
  // start copying tile i into a stage: Q at qdn, dO at qdn + TILE, the rows at
  // ldn; qg, dog, l2g, dg are a.q, a.dout, a.lse2 and a.delta
  auto issue = [&](int i, T* qdn, float* ldn, const T* qg, const T* dog, const float* l2g,
                   const float* dg) __attribute__((always_inline)) {
    int r;
    const int q0 = tile_of(i, r) * kDkvQ;
    const int h = g * a.group + r;
    const T* qp = qg + (int64_t)si.seq0 * qs + (int64_t)h * D;
    const T* dop = dog + (int64_t)si.seq0 * qs + (int64_t)h * D;
    if (q0 + kDkvQ <= L) {
      tile_dma_in<T, kDkvQ, D, kDkvWaves>(qdn, qp + (int64_t)q0 * qs, plan, wave_u);
      tile_dma_in<T, kDkvQ, D, kDkvWaves>(qdn + TILE, dop + (int64_t)q0 * qs, plan, wave_u);
    } else {
      tile_dma<T, kDkvQ, D, kDkvWaves>(qdn, qp, qs, q0, L, wave, lane);
      tile_dma<T, kDkvQ, D, kDkvWaves>(qdn + TILE, dop, qs, q0, L, wave, lane);
    }
    if (wave == 0) {
      const int64_t w0 = (int64_t)h * a.ws_stride + si.seq0 + q0;
      rows_dma<kDkvQ>(ldn, l2g + w0, dg + w0, lane);
    }
  };
  const T* q_g = static_cast<const T*>(a.q);
  const T* do_g = static_cast<const T*>(a.dout);
  // tile i sits in stage i % 3; iteration j copies tile j+2, so the first
  // iteration (j = -1) copies tile 1
  if (ntile > 0) issue(0, qd_lds[0][0], ld_lds[0], q_g, do_g, a.lse2, a.delta);

  u32x4* xp = xch[pair][0];
  u32x4* xs = xch[pair][1];
  const float c = a.scale_log2;

  // In iteration j the copies of tile j+2 run while the producers read tile
  // j+1 and the consumers tile j: three distinct stages. The bodies below
  // take the stages as restrict-qualified pointers, which tells the compiler
  // so; otherwise the reads of tiles j and j+1 would wait for the copies of
  // tile j+2 and leave them nothing to overlap. The copies' global sources
  // come in restrict-qualified too: with every pointer a copy uses being a
  // restrict parameter, the compiler can tell the copies apart from the reads
  // without proving that no pointer escaped. The pair hand-over waits only
  // for LDS operations for the same reason: the copies of tile j+2 need to
  // have landed only at the next iteration's barrier A.
  if (producer) {
    // K and V fragments of this pair's 32 keys (B operands), kept in registers
    u32x4 kf[NKB], vf[NKB];
    const T* kp = static_cast<const T*>(a.k) + (int64_t)(si.seq0k + key) * kvs + (int64_t)g * D;
    const T* vp = static_cast<const T*>(a.v) + (int64_t)(si.seq0k + key) * kvs + (int64_t)g * D;
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
      kf[kb] = key < Lk ? ldg16(kp + kb * 16 + half * 8) : u32x4{0, 0, 0, 0};
      vf[kb] = key < Lk ? ldg16(vp + kb * 16 + half * 8) : u32x4{0, 0, 0, 0};
    }
    // iteration j: copy tile j+2 into the stage (qdn, ldn); P and dS of tile
    // t = j+1 from the stage (qdt, ldt)
    auto body = [&](int j, const T* __restrict__ qdt, const float* __restrict__ ldt,
                    T* __restrict__ qdn, float* __restrict__ ldn, const T* __restrict__ qg,
                    const T* __restrict__ dog, const float* __restrict__ l2g,
                    const float* __restrict__ dg) __attribute__((always_inline)) {
      if (j + 2 < ntile) issue(j + 2, qdn, ldn, qg, dog, l2g, dg);
      const int t = j + 1;
      if (t < ntile) {
        int r;
        const int q0 = tile_of(t, r) * kDkvQ;
        if (!pair_idle(q0)) {
          const DropKey dk{a.seed_lo, a.seed_hi, a.keep_t};
          const int h = g * a.group + r;
          if (t < n_edge)
            dkdv_produce<T, D, CAUSAL, true, WIN, CAP, DROP>(
                qdt, qdt + TILE, ldt, kf, vf, xp, xs, c, q0, L, key, wl, wr, lane, a.cap_in,
                a.cap_out, &dk, b, h, a.drop_scale, off, &hand[pair], j);
          else
            dkdv_produce<T, D, CAUSAL, false, WIN, CAP, DROP>(
                qdt, qdt + TILE, ldt, kf, vf, xp, xs, c, q0, L, key, wl, wr, lane, a.cap_in,
                a.cap_out, &dk, b, h, a.drop_scale, off, &hand[pair], j);
        }
      }
    };
    for (int j = -1; j < ntile; ++j) {
      wait_vmem_all();   // this wave's copies of tile j+1 (and K, V) have landed
      __syncthreads();   // A
      const int st = (j + 1) % kDkvStages, sn = (j + 2) % kDkvStages;
      body(j, qd_lds[st][0], ld_lds[st], qd_lds[sn][0], ld_lds[sn], q_g, do_g, a.lse2, a.delta);
    }
  } else {
    f32x16 dkt[NCB], dvt[NCB];
    uint32_t tro[NCB][2];   // byte offsets of the transposing reads (rows 4h.., 4h+8..)
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) {
      dkt[cb] = f32x16{};
      dvt[cb] = f32x16{};
      // below 2^18: with a constant added the sum cannot wrap, so the k-step
      // constants fold into the reads' offset fields
      tro[cb][0] = tr8_off<D>(4 * half, cb * 32, lane) & kLdsAddrMask;
      tro[cb][1] = tr8_off<D>(4 * half + 8, cb * 32, lane) & kLdsAddrMask;
    }
    // iteration j: copy tile j+2 into the stage (qdn, ldn); dK, dV products of
    // tile j from the stage qdt
    auto body = [&](int j, const T* __restrict__ qdt, T* __restrict__ qdn,
                    float* __restrict__ ldn, const T* __restrict__ qg, const T* __restrict__ dog,
                    const float* __restrict__ l2g, const float* __restrict__ dg)
                    __attribute__((always_inline)) {
      if (j + 2 < ntile) issue(j + 2, qdn, ldn, qg, dog, l2g, dg);
      bool active = false;
      u32x4 pb[kDkvKK], sb[kDkvKK];
      if (j >= 0) {
        int r;
        const int q0 = tile_of(j, r) * kDkvQ;
        active = !pair_idle(q0);
        if (active) {
#pragma unroll
          for (int kk = 0; kk < kDkvKK; ++kk) {
            pb[kk] = xp[kk * 64 + lane];
            sb[kk] = xs[kk * 64 + lane];
          }
        }
      }
      pair_release(&hand[pair], j);   // tile j's P and dS are in registers
      if (active) {
        constexpr uint32_t KSTEP = 16 * D * sizeof(T);   // 16 rows
        constexpr uint32_t DO = TILE * sizeof(T);        // the dO tile follows the Q tile
#pragma unroll
        for (int kk = 0; kk < kDkvKK; ++kk) {
#pragma unroll
          for (int cb = 0; cb < NCB; ++cb) {
            const uint32_t oa = tro[cb][0] + kk * KSTEP, ob = tro[cb][1] + kk * KSTEP;
            dvt[cb] = mfma32<T>(lds_tr8_at<T>(qdt, oa + DO, ob + DO), pb[kk], dvt[cb]);
            dkt[cb] = mfma32<T>(lds_tr8_at<T>(qdt, oa, ob), sb[kk], dkt[cb]);
          }
        }
        // operand reads run one k-step (2·NCB products) ahead of the products
        constexpr int kSgMFMA = 0x008, kSgDSRead = 0x100;
        constexpr int kPer = 2 * NCB;   // products per k-step, 2 reads each
        __builtin_amdgcn_sched_group_barrier(kSgDSRead, 2 * kPer, 0);
#pragma unroll
        for (int i = 0; i < (kDkvKK - 1) * kPer; ++i) {
          __builtin_amdgcn_sched_group_barrier(kSgMFMA, 1, 0);
          __builtin_amdgcn_sched_group_barrier(kSgDSRead, 2, 0);
        }
        __builtin_amdgcn_sched_group_barrier(kSgMFMA, kPer, 0);
      }
    };
    for (int j = -1; j < ntile; ++j) {
      wait_vmem_all();
      __syncthreads();   // A: tile j's P and dS are in LDS
      const int st = (j + kDkvStages) % kDkvStages, sn = (j + 2) % kDkvStages;
      body(j, qd_lds[st][0], qd_lds[sn][0], ld_lds[sn], q_g, do_g, a.lse2, a.delta);
    }
    if (key < Lk) {
      const int64_t ko = (int64_t)(si.seq0k + key) * kvs + (int64_t)g * D;
      T* dkp = static_cast<T*>(a.dk) + ko;
      T* dvp = static_cast<T*>(a.dv) + ko;
      const float sc = a.scale;
#pragma unroll
      for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
          const int d0 = cb * 32 + 8 * rr + 4 * half;
          u32x2 w;
          w[0] = pack2<T>(dkt[cb][4 * rr + 0] * sc, dkt[cb][4 * rr + 1] * sc);
          w[1] = pack2<T>(dkt[cb][4 * rr + 2] * sc, dkt[cb][4 * rr + 3] * sc);
          *reinterpret_cast<u32x2*>(dkp + d0) = w;
          w[0] = pack2<T>(dvt[cb][4 * rr + 0], dvt[cb][4 * rr + 1]);
          w[1] = pack2<T>(dvt[cb][4 * rr + 2], dvt[cb][4 * rr + 3]);
          *reinterpret_cast<u32x2*>(dvp + d0) = w;
        }
    }
  }
}

// ---------------------------------------------------------------------------
// dK, dV at d = 256. The two-role kernel above cannot hold 32 keys' dKᵀ and
// dVᵀ (256 accumulator registers) with two waves per SIMD, and one wave
// holding both with K and V fragments does not fit 512 registers either. So
// two passes over the same tiles, one wave per SIMD owning 32 keys: PASS 0
// computes S (K fragments in registers), P and dVᵀ += dOᵀ·P; PASS 1 computes
// S and dP (K and V fragments), dS and dKᵀ += Qᵀ·dS. S is computed twice (one
// more GEMM on top of the four). Keys are MFMA columns, so P and dS come out
// in the B-operand layout of the dV/dK products, whose Qᵀ, dOᵀ operands are
// transposing LDS reads. Q/dO tiles of 64 queries are double-buffered in LDS
// (128 KiB at d = 256). Masks none, causal or a sliding window (WIN, as in
// fwd_kernel; CAUSAL is false then), varlen, GQA; CAP and DROP as in
// dkdv_produce (soft-capped logits, dS times 1 − tanh²; dropout: dV takes
// P∘Z, dS = P∘(Z∘dP − D)).
constexpr int kWideKeys = 128;   // keys per workgroup (32 per wave)
constexpr int kWideQ = 64;       // queries per tile

template <typename T, int D, bool CAUSAL, bool EDGE, int PASS, bool CAP, bool WIN, bool DROP>
__device__ __forceinline__ void dkdv_wide_tile(const T* qt_, const T* dot_, const float* ld,
                                               const u32x4 (&kf)[D / 16],
                                               const u32x4 (&vf)[D / 16], f32x16 (&acc)[D / 32],
                                               float c, int q0, int L, int key, int lane,
                                               float cap_in, float cap_out, int wl, int wr,
                                               const DropKey& dk, int seq, int head, float zs) {
  constexpr int NKB = D / 16;
  constexpr int NCB = D / 32;
  const int col = lane & 31, half = lane >> 5;
#pragma unroll
  for (int qb = 0; qb < kWideQ / 32; ++qb) {
    f32x16 s = f32x16{}, dp = f32x16{};
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
      s = mfma32<T>(lds_row16<T, D>(qt_, qb * 32 + col, 2 * kb + half), kf[kb], s);
      if constexpr (PASS == 1)
        dp = mfma32<T>(lds_row16<T, D>(dot_, qb * 32 + col, 2 * kb + half), vf[kb], dp);
    }
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) {
      const int qoff = qb * 32 + 8 * rr + 4 * half;
      const float4 lv = *reinterpret_cast<const float4*>(ld + qoff);
      const float4 dv4 = *reinterpret_cast<const float4*>(ld + kWideQ + qoff);
      const float lsev[4] = {lv.x, lv.y, lv.z, lv.w};
      const float dlv[4] = {dv4.x, dv4.y, dv4.z, dv4.w};
      uint32_t dbytes = 0;   // dropout: queries q0 + qoff + 0..3 of this lane's key
      if constexpr (DROP) dbytes = drop_col_bytes(dk, seq, head, q0 + qoff, key);
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const int i4 = 4 * rr + t;
        float p, ds;
        if constexpr (CAP) {
          const float th = tanh_fast(s[i4] * cap_in);
          p = fast_exp2(fmaf(th, cap_out, -lsev[t]));
          ds = p * (dp[i4] - dlv[t]) * fmaf(-th, th, 1.f);
        } else if constexpr (DROP) {
          p = fast_exp2(fmaf(s[i4], c, -lsev[t]));
          const float z = drop_keep(dbytes, t, dk.t) ? zs : 0.f;
          ds = p * fmaf(dp[i4], z, -dlv[t]);
          p *= z;
        } else {
          p = fast_exp2(fmaf(s[i4], c, -lsev[t]));
          ds = p * (dp[i4] - dlv[t]);
        }
        if constexpr (EDGE) {
          const int q = q0 + qoff + t;
          bool keep = q < L && !(CAUSAL && key > q);
          if constexpr (WIN) keep = keep && q >= key - wr && q <= key + wl;
          p = keep ? p : 0.f;
          ds = keep ? ds : 0.f;
        }
        s[i4] = p;
        dp[i4] = ds;
      }
    }
#pragma unroll
    for (int h2 = 0; h2 < 2; ++h2) {
      // PASS 0: dVᵀ += dOᵀ·P; PASS 1: dKᵀ += Qᵀ·dS
      const u32x4 b = acc_operand<T>(PASS == 0 ? s : dp, h2 * 2);
      const int kq = qb * 32 + h2 * 16 + 4 * half;
#pragma unroll
      for (int cb = 0; cb < NCB; ++cb)
        acc[cb] = mfma32<T>(lds_tr8<T, D>(PASS == 0 ? dot_ : qt_, kq, kq + 8, cb * 32, lane), b,
                            acc[cb]);
    }
  }
}

template <typename T, int D, bool CAUSAL, bool VARLEN, int PASS, bool CAP, bool WIN, bool DROP>
__global__ __launch_bounds__(kThreads, 1) void dkdv_wide_kernel(BwdArgs a, int n_ktiles) {
  constexpr int NKB = D / 16;
  constexpr int NCB = D / 32;
  constexpr int TILE = kWideQ * D;
  __shared__ __attribute__((aligned(1024))) T q_lds[2][TILE];
  __shared__ __attribute__((aligned(1024))) T do_lds[2][TILE];
  __shared__ __attribute__((aligned(16))) float ld_lds[2][2 * kWideQ];   // LSE·log2 e, D

  // the wave index is the same on every lane: readfirstlane lets the compiler
  // see that, so branches on it are scalar rather than divergent
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = lane & 31, half = lane >> 5;

  const int G = gridDim.x;
  const int logical = xcd_remap(blockIdx.x, G);
  const int kt = logical % n_ktiles;           // ascending = heaviest first when causal
  const int gb = logical / n_ktiles;
  const int b = gb % a.B, g = gb / a.B;   // sequence fastest, as in the other kernels
  const SeqInfo si = seq_info<VARLEN>(a, b);
  const int k0 = kt * kWideKeys;
  if (k0 >= si.L) return;
  const int L = si.L;

  const int64_t qs = (int64_t)a.Hq * D, kvs = (int64_t)a.Hkv * D;
  const int key = k0 + wave * 32 + col;
  // Query tiles of one head: [qt_begin, qt_end), of which [ia, ib) are
  // interior (every query sees every key of the block: no mask). The front
  // edge tiles (the causal diagonal below k0 + 128, a window's leading edge)
  // and back edge tiles (a window's trailing edge, a ragged last tile) of every
  // head of the group come first, then the interior tiles.
  const int wl = WIN ? a.wl : 0, wr = WIN ? a.wr : 0;
  int qt_begin, qt_end, ia, ib;
  if constexpr (WIN) {
    // query i sees key j iff j − wr <= i <= j + wl
    const int lo = max(0, k0 - wr), hi = min(L, k0 + kWideKeys + wl);
    qt_begin = lo / kWideQ;
    qt_end = hi > lo ? (hi + kWideQ - 1) / kWideQ : qt_begin;
    const int first = k0 + kWideKeys - 1 - wr;   // interior queries: [first, k0 + wl]
    ia = max(qt_begin, first <= 0 ? 0 : (first + kWideQ - 1) / kWideQ);
    const int last = k0 + wl - (kWideQ - 1);      // a tile starting here ends at k0 + wl
    ib = min(min(last < 0 ? 0 : last / kWideQ + 1, L / kWideQ), qt_end);
    if (ib < ia) ib = ia;
    ia = min(ia, qt_end);
    ib = min(max(ib, ia), qt_end);
  } else {
    qt_begin = CAUSAL ? k0 / kWideQ : 0;
    qt_end = (L + kWideQ - 1) / kWideQ;
    const int nq0 = qt_end - qt_begin;
    const int nd = CAUSAL ? min(kWideKeys / kWideQ, nq0) : 0;
    ia = qt_begin + nd;
    ib = qt_end - ((L % kWideQ != 0 && nq0 > nd) ? 1 : 0);
  }
  const int nq = qt_end - qt_begin, nf = ia - qt_begin, ni = ib - ia;
  const int ne = nq - ni;
  const int n_edge = a.group * ne, ntile = a.group * nq;
  auto tile_of = [&](int i, int& r) -> int {   // tile i -> (head r, query tile)
    if (i < n_edge) {
      r = i / ne;
      const int e = i - r * ne;
      return e < nf ? qt_begin + e : ib + (e - nf);
    }
    const int j = i - n_edge;
    r = j / ni;
    return ia + (j - r * ni);
  };
  auto issue = [&](int i, int buf) {
    int r;
    const int q0 = tile_of(i, r) * kWideQ;
    const int h = g * a.group + r;
    const T* qp = static_cast<const T*>(a.q) + (int64_t)si.seq0 * qs + (int64_t)h * D;
    const T* dop = static_cast<const T*>(a.dout) + (int64_t)si.seq0 * qs + (int64_t)h * D;
    tile_dma<T, kWideQ, D, kWaves>(q_lds[buf], qp, qs, q0, L, wave, lane);
    tile_dma<T, kWideQ, D, kWaves>(do_lds[buf], dop, qs, q0, L, wave, lane);
    if (wave == 0) {
      const int64_t w0 = (int64_t)h * a.ws_stride + si.seq0 + q0;
      rows_dma<kWideQ>(ld_lds[buf], a.lse2 + w0, a.delta + w0, lane);
    }
  };
  if (ntile > 0) issue(0, 0);

  // K and V fragments of this wave's 32 keys (B operands), kept in registers
  u32x4 kf[NKB], vf[NKB];
  {
    const T* kp = static_cast<const T*>(a.k) + (int64_t)(si.seq0 + key) * kvs + (int64_t)g * D;
    const T* vp = static_cast<const T*>(a.v) + (int64_t)(si.seq0 + key) * kvs + (int64_t)g * D;
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
      kf[kb] = key < L ? ldg16(kp + kb * 16 + half * 8) : u32x4{0, 0, 0, 0};
      vf[kb] = (PASS == 1 && key < L) ? ldg16(vp + kb * 16 + half * 8) : u32x4{0, 0, 0, 0};
    }
  }
  f32x16 acc[NCB];   // dVᵀ (PASS 0) or dKᵀ (PASS 1)
#pragma unroll
  for (int cb = 0; cb < NCB; ++cb) acc[cb] = f32x16{};
  const float c = CAP ? 1.f : a.scale_log2;   // capped logits are already in log2 units
  const float cap_in = CAP ? a.cap_in : 0.f, cap_out = CAP ? a.cap_out : 0.f;
  const DropKey dk{a.seed_lo, a.seed_hi, a.keep_t};
  const int wk_first = k0 + wave * 32;

  auto step = [&](auto edge_tag, int i) {
    constexpr bool EDGE = decltype(edge_tag)::value;
    const int buf = i & 1;
    wait_vmem_all();   // this thread's copies of tile i have landed
    __syncthreads();   // everyone's have; tile i-1 is no longer read
    if (i + 1 < ntile) issue(i + 1, buf ^ 1);
    int r;
    const int q0 = tile_of(i, r) * kWideQ;
    // a diagonal tile can lie entirely before this wave's keys
    if (EDGE && CAUSAL && q0 + kWideQ - 1 < wk_first) return;
    // or an edge tile of a window outside the windows of all this wave's keys
    if (EDGE && WIN && (q0 + kWideQ - 1 < wk_first - wr || q0 > wk_first + 31 + wl)) return;
    dkdv_wide_tile<T, D, CAUSAL, EDGE, PASS, CAP, WIN, DROP>(
        q_lds[buf], do_lds[buf], ld_lds[buf], kf, vf, acc, c, q0, L, key, lane, cap_in, cap_out,
        wl, wr, dk, b, g * a.group + r, a.drop_scale);
  };
  for (int i = 0; i < n_edge; ++i) step(std::true_type{}, i);
  for (int i = n_edge; i < ntile; ++i) step(std::false_type{}, i);

  if (key < L) {
    const int64_t off = (int64_t)(si.seq0 + key) * kvs + (int64_t)g * D;
    T* outp = static_cast<T*>(PASS == 0 ? a.dv : a.dk) + off;
    const float sc = PASS == 0 ? 1.f : a.scale;   // dK = scale · Σ dSᵀ Q
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        const int d0 = cb * 32 + 8 * rr + 4 * half;
        u32x2 w;
        w[0] = pack2<T>(acc[cb][4 * rr + 0] * sc, acc[cb][4 * rr + 1] * sc);
        w[1] = pack2<T>(acc[cb][4 * rr + 2] * sc, acc[cb][4 * rr + 3] * sc);
        *reinterpret_cast<u32x2*>(outp + d0) = w;
      }
  }
}

// ---------------------------------------------------------------------------
// dQ. Orientation Sᵀ = K·Qᵀ as in the forward: one query per lane, so LSE and
// D are per-lane scalars and the dSᵀ accumulator is the B operand of
// dQᵀ = Kᵀ·dSᵀ (Kᵀ read transposed from the row-major K tile).
constexpr int kDqQ = 128;   // queries per workgroup (32 per wave)
constexpr int kDqK = 64;    // keys per tile
#ifndef FA_DQ_AHEAD
#define FA_DQ_AHEAD 1
#endif

// One 64-key tile for one wave's 32 queries: Sᵀ and dPᵀ, then
// dSᵀ = P∘(dP − D) with P = exp2(S·c − LSE·log2 e), then dQᵀ += Kᵀ·dSᵀ.
// EDGE tiles zero P for keys past the end and, causally, for keys after the
// query.
// CAP as in dkdv_produce
// CAP and DROP as in dkdv_produce
template <typename T, int D, bool CAUSAL, bool EDGE, bool WIN, bool CAP = false, bool DROP = false>
__device__ __forceinline__ void dq_tile(const T* kt, const T* vt, const u32x4 (&qf)[D / 16],
                                        const u32x4 (&df)[D / 16], f32x16 (&dqt)[D / 32], float c,
                                        float lse2, float dl, int kv0, int L, int qrow, int wl,
                                        int wr, int lane, float cap_in = 0.f,
                                        float cap_out = 0.f, const DropKey* dk = nullptr,
                                        int seq = 0, int head = 0, float zs = 0.f) {
  constexpr int NKB = D / 16;
  constexpr int NCB = D / 32;
  constexpr int NJB = kDqK / 32;
  constexpr int A = FA_DQ_AHEAD;   // K/V row reads in flight ahead of their MFMAs
  const int col = lane & 31, half = lane >> 5;
  // the K and V rows of Sᵀ and dPᵀ are read A MFMA steps ahead, and the
  // next 32-key block's first rows during this block's dQ products
  u32x4 ka[A + 1], va[A + 1];
  auto fetch_s = [&](int jb, int kb) __attribute__((always_inline)) {
    ka[kb % (A + 1)] = lds_row16<T, D>(kt, jb * 32 + col, 2 * kb + half);
    va[kb % (A + 1)] = lds_row16<T, D>(vt, jb * 32 + col, 2 * kb + half);
  };
#pragma unroll
  for (int kb = 0; kb < A; ++kb) fetch_s(0, kb);
#pragma unroll
  for (int jb = 0; jb < NJB; ++jb) {   // 32-key blocks
    f32x16 s = f32x16{}, dp = f32x16{};
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
      if (kb + A < NKB) fetch_s(jb, kb + A);
      s = mfma32<T>(ka[kb % (A + 1)], qf[kb], s);
      dp = mfma32<T>(va[kb % (A + 1)], df[kb], dp);
    }
    uint32_t dbytes[4] = {0, 0, 0, 0};   // keys kv0 + 32·jb + 8·r + 4·half + 0..3
    if constexpr (DROP) {
      const int jr[4] = {kv0 + jb * 32 + 4 * half, kv0 + jb * 32 + 8 + 4 * half,
                         kv0 + jb * 32 + 16 + 4 * half, kv0 + jb * 32 + 24 + 4 * half};
      drop_row_bytes_quad(*dk, seq, head, qrow, jr, dbytes);
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      float p, g = 1.f;
      if constexpr (CAP) {
        const float th = tanh_fast(s[i] * cap_in);
        p = fast_exp2(fmaf(th, cap_out, -lse2));
        g = fmaf(-th, th, 1.f);
      } else {
        p = fast_exp2(fmaf(s[i], c, -lse2));
      }
      if constexpr (EDGE) {
        const int kj = kv0 + jb * 32 + 8 * (i >> 2) + 4 * half + (i & 3);
        bool vis = kj < L && !(CAUSAL && kj > qrow);
        if constexpr (WIN) vis = vis && kj >= qrow - wl && kj <= qrow + wr;
        p = vis ? p : 0.f;
      }
      if constexpr (CAP) dp[i] = p * (dp[i] - dl) * g;
      else if constexpr (DROP)
        dp[i] = p * fmaf(dp[i], drop_keep(dbytes[i >> 2], i & 3, dk->t) ? zs : 0.f, -dl);
      else dp[i] = p * (dp[i] - dl);
    }
    if (jb + 1 < NJB) {
#pragma unroll
      for (int kb = 0; kb < A; ++kb) fetch_s(jb + 1, kb);
    }
#pragma unroll
    for (int h2 = 0; h2 < 2; ++h2) {
      const u32x4 sb = acc_operand<T>(dp, h2 * 2);
      const int kq = jb * 32 + h2 * 16 + 4 * half;
#pragma unroll
      for (int cb = 0; cb < NCB; ++cb)
        dqt[cb] = mfma32<T>(lds_tr8<T, D>(kt, kq, kq + 8, cb * 32, lane), sb, dqt[cb]);
    }
  }
}

// two workgroups per CU up to d = 128; at d = 256 the dQ accumulators and the
// Q and dO fragments take 256 registers and the kernel runs one per CU
// KVLEN: keys of their own length (see seq_info); no window, cap or dropout
template <typename T, int D, bool CAUSAL, bool VARLEN, bool WIN, bool CAP = false,
          bool DROP = false, bool KVLEN = false>
__global__ __launch_bounds__(kThreads, D <= 128 ? 2 : 1) void dq_kernel(BwdArgs a, int n_qtiles) {
  constexpr int NKB = D / 16;
  constexpr int NCB = D / 32;
  constexpr int TILE = kDqK * D;
  __shared__ __attribute__((aligned(1024))) T lds[2][2][TILE];   // [buffer][K, V]

  // the wave index is the same on every lane: readfirstlane lets the compiler
  // see that, so branches on it are scalar rather than divergent
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = lane & 31, half = lane >> 5;

  const int G = gridDim.x;
  const int logical = xcd_remap(blockIdx.x, G);
  const int qt_ord = logical % n_qtiles;
  const int hb = logical / n_qtiles;
  const int b = hb % a.B, h = hb / a.B;   // sequence fastest: XCD ranges balanced for varlen
  const int qt = CAUSAL ? n_qtiles - 1 - qt_ord : qt_ord;
  const SeqInfo si = seq_info<VARLEN, KVLEN>(a, b);
  const int q0 = qt * kDqQ;
  if (q0 >= si.L) return;
  const int L = si.L, Lk = si.Lk, off = si.off;   // queries, keys, key position of query 0
  const int g = h / a.group;

  const int64_t qs = (int64_t)a.Hq * D, kvs = (int64_t)a.Hkv * D;
  const T* kp = static_cast<const T*>(a.k) + (int64_t)si.seq0k * kvs + (int64_t)g * D;
  const T* vp = static_cast<const T*>(a.v) + (int64_t)si.seq0k * kvs + (int64_t)g * D;
  // key tiles [j_lo, j_hi) visible to some query; [ja, jb) need no masking
  // (the same split as in fwd_kernel)
  int j_lo, ja, jb, j_hi;
  const int wl = WIN ? a.wl : 0, wr = WIN ? a.wr : 0;
  if constexpr (WIN) {
    j_lo = max(0, q0 - wl) / kDqK;
    j_hi = (min(L, q0 + kDqQ + wr) + kDqK - 1) / kDqK;
    const int first_all = q0 + kDqQ - 1 - wl;
    ja = max(j_lo, first_all <= 0 ? 0 : (first_all + kDqK - 1) / kDqK);
    const int last_all = q0 + wr - (kDqK - 1);
    jb = min(min(last_all < 0 ? 0 : last_all / kDqK + 1, L / kDqK), j_hi);
    if (jb < ja) jb = ja;
  } else {
    // causal: query i sees keys j <= i + off; the end may be <= 0 with KVLEN
    // (no key for any query of the tile: dQ = 0)
    const int kv_end = CAUSAL ? min(Lk, q0 + kDqQ + off) : Lk;
    j_lo = ja = 0;
    j_hi = kv_end > 0 ? (kv_end + kDqK - 1) / kDqK : 0;
    jb = min(CAUSAL ? min(max(q0 + off + 1, 0) / kDqK, Lk / kDqK) : Lk / kDqK, j_hi);
  }
  const int ntiles = j_hi;
  if (ntiles > j_lo) {
    tile_dma<T, kDqK, D, kWaves>(lds[0][0], kp, kvs, j_lo * kDqK, Lk, wave, lane);
    tile_dma<T, kDqK, D, kWaves>(lds[0][1], vp, kvs, j_lo * kDqK, Lk, wave, lane);
  }

  const int qrow = q0 + wave * 32 + col;
  u32x4 qf[NKB], df[NKB];
  float lse2 = 0.f, dl = 0.f;
  {
    const int64_t off = (int64_t)(si.seq0 + qrow) * qs + (int64_t)h * D;
    const T* qp = static_cast<const T*>(a.q) + off;
    const T* dop = static_cast<const T*>(a.dout) + off;
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
      qf[kb] = qrow < L ? ldg16(qp + kb * 16 + half * 8) : u32x4{0, 0, 0, 0};
      df[kb] = qrow < L ? ldg16(dop + kb * 16 + half * 8) : u32x4{0, 0, 0, 0};
    }
    if (qrow < L) {
      lse2 = a.lse2[(int64_t)h * a.ws_stride + si.seq0 + qrow];
      dl = a.delta[(int64_t)h * a.ws_stride + si.seq0 + qrow];
    }
  }
  f32x16 dqt[NCB];
#pragma unroll
  for (int cb = 0; cb < NCB; ++cb) dqt[cb] = f32x16{};
  const DropKey dk{a.seed_lo, a.seed_hi, a.keep_t};
  const float c = a.scale_log2;
  const int wq_first = q0 + wave * 32, wq_last = wq_first + 31;
  const DmaPlan<T, kDqK, D, kWaves> plan(kvs, wave, lane);
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);
  // buf_tag fixes the tile's LDS buffer at compile time in the unrolled
  // interior pairs, so every LDS read is a per-lane register plus an immediate
  auto step = [&](auto edge_tag, auto buf_tag, int j) __attribute__((always_inline)) {
    constexpr bool EDGE = decltype(edge_tag)::value;
    constexpr int FIXED = decltype(buf_tag)::value;   // 0, 1, or -1 for (j − j_lo) & 1
    const int BUF = FIXED >= 0 ? FIXED : ((j - j_lo) & 1);
    const int kv0 = j * kDqK;
    const T* kt = lds[BUF][0];
    const T* vt = lds[BUF][1];
    wait_vmem_all();
    __syncthreads();
    if (j + 1 < ntiles) {
      const int n0 = kv0 + kDqK;
      if (n0 + kDqK <= Lk) {
        tile_dma_in<T, kDqK, D, kWaves>(lds[BUF ^ 1][0], kp + (int64_t)n0 * kvs, plan, wave_u);
        tile_dma_in<T, kDqK, D, kWaves>(lds[BUF ^ 1][1], vp + (int64_t)n0 * kvs, plan, wave_u);
      } else {
        tile_dma<T, kDqK, D, kWaves>(lds[BUF ^ 1][0], kp, kvs, n0, Lk, wave, lane);
        tile_dma<T, kDqK, D, kWaves>(lds[BUF ^ 1][1], vp, kvs, n0, Lk, wave, lane);
      }
    }
    if (EDGE && CAUSAL && kv0 > wq_last + off) return;   // every key after this wave's queries
    if (EDGE && WIN && (kv0 > wq_last + wr || kv0 + kDqK - 1 < wq_first - wl))
      return;   // the tile lies outside the windows of all this wave's queries
    // keys are compared with the query's position qrow + off
    dq_tile<T, D, CAUSAL, EDGE, WIN, CAP, DROP>(kt, vt, qf, df, dqt, c, lse2, dl, kv0, Lk,
                                                qrow + off, wl, wr, lane, a.cap_in, a.cap_out,
                                                &dk, b, h, a.drop_scale);
  };
  using B0 = std::integral_constant<int, 0>;
  using B1 = std::integral_constant<int, 1>;
  using BR = std::integral_constant<int, -1>;
  int j = j_lo;
  if constexpr (WIN)
    for (; j < ja; ++j) step(std::true_type{}, BR{}, j);   // the window's left edge tiles
  // the unrolled pairs need registers that d = 256 and the window variants lack
  if constexpr (D <= 128 && !WIN) {
    if (j < jb && ((j - j_lo) & 1)) step(std::false_type{}, BR{}, j++);
    for (; j + 1 < jb; j += 2) {   // tile j in buffer 0, tile j+1 in buffer 1
      step(std::false_type{}, B0{}, j);
      step(std::false_type{}, B1{}, j + 1);
    }
    if (j < jb) step(std::false_type{}, BR{}, j++);
  } else {
    for (; j < jb; ++j) step(std::false_type{}, BR{}, j);
  }
  for (; j < ntiles; ++j) step(std::true_type{}, BR{}, j);

  if (qrow < L) {
    T* dqp = static_cast<T*>(a.dq) + (int64_t)(si.seq0 + qrow) * qs + (int64_t)h * D;
    const float sc = a.scale;
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        u32x2 w;
        w[0] = pack2<T>(dqt[cb][4 * rr + 0] * sc, dqt[cb][4 * rr + 1] * sc);
        w[1] = pack2<T>(dqt[cb][4 * rr + 2] * sc, dqt[cb][4 * rr + 3] * sc);
        *reinterpret_cast<u32x2*>(dqp + cb * 32 + 8 * rr + 4 * half) = w;
      }
  }
}

template <typename T, int D, bool CAUSAL, bool VARLEN, bool WIN, bool CAP = false,
          bool DROP = false, bool KVLEN = false>
hipError_t launch(const BwdArgs& a, int stage, hipStream_t s) {
  static_assert(!KVLEN || D <= 128, "separate key lengths: d = 64 or 128");
  (void)hipGetLastError();  // drop an error left pending by earlier, unrelated HIP calls
  if (stage < 0 || stage == 0) {
    const int64_t rows = (int64_t)a.B * a.N * a.Hq;   // upper bound on T·Hq
    const int rows_per_block = kThreads / (D / 8);
    const int g0 = (int)((rows + rows_per_block - 1) / rows_per_block);
    if (g0 > 0)
      hipLaunchKernelGGL((delta_kernel<T, D, VARLEN>), dim3(g0), dim3(kThreads), 0, s, a);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (stage < 0 || stage == 1) {
    if constexpr (D == 256) {
      const int nkt = (a.N + kWideKeys - 1) / kWideKeys;
      hipLaunchKernelGGL((dkdv_wide_kernel<T, D, CAUSAL, VARLEN, 0, CAP, WIN, DROP>),
                         dim3(nkt * a.Hkv * a.B), dim3(kThreads), 0, s, a, nkt);
      const hipError_t e0 = hipGetLastError();
      if (e0 != hipSuccess) return e0;
      hipLaunchKernelGGL((dkdv_wide_kernel<T, D, CAUSAL, VARLEN, 1, CAP, WIN, DROP>),
                         dim3(nkt * a.Hkv * a.B), dim3(kThreads), 0, s, a, nkt);
    } else {
      const int nkt = ((KVLEN ? a.Nk : a.N) + kDkvKeys - 1) / kDkvKeys;
      if (nkt > 0)
        hipLaunchKernelGGL((dkdv_kernel<T, D, CAUSAL, VARLEN, WIN, CAP, DROP, KVLEN>),
                           dim3(nkt * a.Hkv * a.B), dim3(kDkvThreads), 0, s, a, nkt);
    }
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (stage < 0 || stage == 2) {
    const int nqt = (a.N + kDqQ - 1) / kDqQ;
    if (nqt > 0)
      hipLaunchKernelGGL((dq_kernel<T, D, CAUSAL, VARLEN, WIN, CAP, DROP, KVLEN>),
                         dim3(nqt * a.Hq * a.B), dim3(kThreads), 0, s, a, nqt);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

template <typename T, int D>
hipError_t dispatch_mask(const BwdArgs& a, int mask, bool varlen, bool cap, bool drop, int stage,
                         hipStream_t s) {
  if (drop) {   // dropout: no window (checked by the caller)
    if (mask == kMaskCausal)
      return varlen ? launch<T, D, true, true, false, false, true>(a, stage, s)
                    : launch<T, D, true, false, false, false, true>(a, stage, s);
    return varlen ? launch<T, D, false, true, false, false, true>(a, stage, s)
                  : launch<T, D, false, false, false, false, true>(a, stage, s);
  }
  if (cap) {
    if (mask == kMaskWindow)
      return varlen ? launch<T, D, false, true, true, true>(a, stage, s)
                    : launch<T, D, false, false, true, true>(a, stage, s);
    if (mask == kMaskCausal)
      return varlen ? launch<T, D, true, true, false, true>(a, stage, s)
                    : launch<T, D, true, false, false, true>(a, stage, s);
    return varlen ? launch<T, D, false, true, false, true>(a, stage, s)
                  : launch<T, D, false, false, false, true>(a, stage, s);
  }
  if (mask == kMaskWindow)
    return varlen ? launch<T, D, false, true, true>(a, stage, s)
                  : launch<T, D, false, false, true>(a, stage, s);
  if (mask == kMaskCausal)
    return varlen ? launch<T, D, true, true, false>(a, stage, s)
                  : launch<T, D, true, false, false>(a, stage, s);
  return varlen ? launch<T, D, false, true, false>(a, stage, s)
                : launch<T, D, false, false, false>(a, stage, s);
}

}  // namespace

int bwd_num_stages() { return 3; }

// d = 256: unmasked, causal or a window, each with or without a soft cap;
// dropout with the first two (the caller rejects the rest)
template <typename T>
hipError_t dispatch_256(const BwdArgs& a, int mask, bool varlen, bool cap, bool drop, int stage,
                        hipStream_t s) {
  if (drop) {
    if (mask == kMaskCausal)
      return varlen ? launch<T, 256, true, true, false, false, true>(a, stage, s)
                    : launch<T, 256, true, false, false, false, true>(a, stage, s);
    return varlen ? launch<T, 256, false, true, false, false, true>(a, stage, s)
                  : launch<T, 256, false, false, false, false, true>(a, stage, s);
  }
  if (cap) {
    if (mask == kMaskWindow)
      return varlen ? launch<T, 256, false, true, true, true>(a, stage, s)
                    : launch<T, 256, false, false, true, true>(a, stage, s);
    if (mask == kMaskCausal)
      return varlen ? launch<T, 256, true, true, false, true>(a, stage, s)
                    : launch<T, 256, true, false, false, true>(a, stage, s);
    return varlen ? launch<T, 256, false, true, false, true>(a, stage, s)
                  : launch<T, 256, false, false, false, true>(a, stage, s);
  }
  if (mask == kMaskWindow)
    return varlen ? launch<T, 256, false, true, true>(a, stage, s)
                  : launch<T, 256, false, false, true>(a, stage, s);
  if (mask == kMaskCausal)
    return varlen ? launch<T, 256, true, true, false>(a, stage, s)
                  : launch<T, 256, true, false, false>(a, stage, s);
  return varlen ? launch<T, 256, false, true, false>(a, stage, s)
                : launch<T, 256, false, false, false>(a, stage, s);
}

hipError_t launch_bwd_kvlen(const BwdArgs& a, bool bf16_in, int d, bool causal, bool varlen,
                            int stage, hipStream_t s) {
  // <T, D, CAUSAL, VARLEN, WIN, CAP, DROP, KVLEN>
#define FA_KVLEN_BWD(T, D)                                                                   \
  (causal ? (varlen ? launch<T, D, true, true, false, false, false, true>(a, stage, s)       \
                    : launch<T, D, true, false, false, false, false, true>(a, stage, s))     \
          : (varlen ? launch<T, D, false, true, false, false, false, true>(a, stage, s)      \
                    : launch<T, D, false, false, false, false, false, true>(a, stage, s)))
  if (bf16_in) return d == 64 ? FA_KVLEN_BWD(bf16, 64) : FA_KVLEN_BWD(bf16, 128);
  return d == 64 ? FA_KVLEN_BWD(f16, 64) : FA_KVLEN_BWD(f16, 128);
#undef FA_KVLEN_BWD
}

hipError_t launch_bwd(const BwdArgs& a, bool bf16_in, int d, int mask, bool varlen, bool cap,
                      bool drop, int stage, hipStream_t s) {
  if (d == 256) return bf16_in ? dispatch_256<bf16>(a, mask, varlen, cap, drop, stage, s)
                               : dispatch_256<f16>(a, mask, varlen, cap, drop, stage, s);
  if (bf16_in)
    return d == 64 ? dispatch_mask<bf16, 64>(a, mask, varlen, cap, drop, stage, s)
                   : dispatch_mask<bf16, 128>(a, mask, varlen, cap, drop, stage, s);
  return d == 64 ? dispatch_mask<f16, 64>(a, mask, varlen, cap, drop, stage, s)
                 : dispatch_mask<f16, 128>(a, mask, varlen, cap, drop, stage, s);
}

}  // namespace fa
