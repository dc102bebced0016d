// Fused attention forward for gfx950.
//
// One workgroup = 4 wavefronts = a tile of 128 query rows of one (sequence,
// query head); each wavefront owns 32 rows. The workgroup streams the visible
// 64-key tiles (128 at d = 64) of K and V through LDS (tiling and fusion as in the
// FlashAttention guide, cxbdf.cn, part 2; K/V blocks in fast on-chip memory
// with a loop over Q blocks, Flash Attention 是什麼, adersaytech.com, section
// 分塊計算), so S and P live only in registers.
//
// Per key tile and wavefront:
//   Sᵀ = K·Qᵀ        32 MFMA columns = the wave's 32 queries, so every lane
//                    owns one query row and the row statistics are lane-local
//                    (plus one exchange between the two lane halves)
//   online softmax   base-2 exponentials with the scale folded in
//                    (c = scale·log2 e); the reference max is raised only when
//                    a row's max exceeds it by more than 2^8, so P ≤ 256 and O
//                    is rarely rescaled
//   Oᵀ += Vᵀ·Pᵀ      P comes from the Sᵀ accumulator registers; the Vᵀ operand
//                    is read transposed from the row-major V tile
// K and V tiles are copied global -> LDS directly and double-buffered: the
// next tile is in flight while the current one is computed.
// Epilogue: O = Oᵀ/lr rounded to the input type, with lr the row sum of P as
// rounded for the MFMAs; LSE = (m·c + log2 l)·ln 2, with l the fp32 row sum
// of the unrounded P for bf16 and lr for fp16.
#include <type_traits>

#include "fa_device.h"
#include "fa_kernels.h"

namespace fa {

namespace {

constexpr int kBR = 128;  // query rows per workgroup
// Keys per tile: 128 at d = 64, where a wave's tile state is small enough to
// take twice the keys per step (more independent MFMA chains per step, half
// the steps on the longest causal tile's critical path), 64 otherwise (and
// with dropout, whose generator calls are laid out for 64-key tiles).
template <int D, bool DROP>
constexpr int keys_per_tile() { return D == 64 && !DROP ? 128 : 64; }
constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr float kRescaleHeadroom = 8.f;  // log2 of the largest P before the max is raised

// One tile of BC keys for one wave's 32 query rows: Sᵀ = K·Qᵀ, online softmax
// with a lazily raised reference max, Oᵀ += Vᵀ·Pᵀ. EDGE tiles mask keys past
// the sequence end and, causally, keys after the query. CAP: the logits
// are soft-capped, s = c_out·tanh(z·c_in) in log2 units (then c is 1).
// DROP: dropout on the weights; the row sum lr still takes every weight, the
// P·V product only the kept ones (scaled by 256/t in the epilogue).
template <typename T, int D, bool CAUSAL, bool EDGE, bool WIN, bool CAP = false, bool DROP = false>
__device__ __forceinline__ void fwd_tile(const T* kt, const T* vt, const u32x4 (&qf)[D / 16],
                                         f32x16 (&o)[D / 32], float& mc, float& l, float& lr,
                                         float c, int kv0, int L, int qrow, int wl, int wr,
                                         int lane, float cap_in = 0.f, float cap_out = 0.f,
                                         const DropKey* dk = nullptr, int seq = 0, int head = 0,
                                         bool empty_rows = false) {
  constexpr int NKB = D / 16;
  constexpr int NCB = D / 32;
  constexpr int BC = keys_per_tile<D, DROP>();
  constexpr int NJB = BC / 32;   // 32-key blocks of Sᵀ
  const int col = lane & 31, half = lane >> 5;
  // ---- Sᵀ = K·Qᵀ ----------------------------------------------------------
  f32x16 s[NJB];
#pragma unroll
  for (int jb = 0; jb < NJB; ++jb) s[jb] = f32x16{};
#pragma unroll
  for (int kb = 0; kb < NKB; ++kb) {
#pragma unroll
    for (int jb = 0; jb < NJB; ++jb)
      s[jb] = mfma32<T>(lds_row16<T, D>(kt, jb * 32 + col, 2 * kb + half), qf[kb], s[jb]);
  }
  if constexpr (CAP) {
#pragma unroll
    for (int jb = 0; jb < NJB; ++jb)
#pragma unroll
      for (int i = 0; i < 16; ++i) s[jb][i] = cap_out * tanh_fast(s[jb][i] * cap_in);
  }

  // ---- mask: keys past the sequence end, keys after the query (causal) ---
  if constexpr (EDGE) {
#pragma unroll
    for (int jb = 0; jb < NJB; ++jb)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int key = kv0 + jb * 32 + 8 * (i >> 2) + 4 * half + (i & 3);
        bool vis = key < L && !(CAUSAL && key > qrow);
        if constexpr (WIN) vis = vis && key >= qrow - wl && key <= qrow + wr;
        s[jb][i] = vis ? s[jb][i] : -INFINITY;
      }
  }

  // ---- online softmax with a lazily raised reference max -----------------
  float mx = s[0][0];
#pragma unroll
  for (int i = 1; i < 16; ++i) mx = fmaxf(mx, s[0][i]);
#pragma unroll
  for (int jb = 1; jb < NJB; ++jb)
#pragma unroll
    for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s[jb][i]);
  const float mxc = wave_max_halves(mx) * c;
  // a window's edge tile can hold no visible key for a row that has seen none
  // yet either: such a row keeps mc = −inf, scales nothing and adds P = 0
  // (so can a row placed before every key when the key and query lengths differ)
  const bool guard = (WIN || empty_rows) && EDGE;
  if (__builtin_amdgcn_ballot_w64(mxc > mc + kRescaleHeadroom) != 0) {   // wave-uniform
    const float mc_new = fmaxf(mc, mxc);     // finite otherwise: key 0 is in tile 0
    const float alpha = (guard && mc_new == -INFINITY) ? 1.f : fast_exp2(mc - mc_new);
    l *= alpha;
    lr *= alpha;
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) o[cb] *= alpha;
    mc = mc_new;
  }
  // bf16 also sums the unrounded P in fp32 for the LSE (kLseFromUnrounded)
  float ls[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int jb = 0; jb < NJB; ++jb)
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      s[jb][i] = fast_exp2(fmaf(s[jb][i], c, guard && mc == -INFINITY ? 0.f : -mc));
      if constexpr (kLseFromUnrounded<T>) ls[i & 3] += s[jb][i];
    }
  if constexpr (kLseFromUnrounded<T>) l += (ls[0] + ls[1]) + (ls[2] + ls[3]);

  // ---- Oᵀ += Vᵀ·Pᵀ ---------------------------------------------------------
  // lr sums P as rounded to T for the MFMAs; O is normalised by it, so that
  // the rounding of a dominant P cancels in O instead of scaling it
  float r[BC / 16];   // independent partial sums: short dependency chains
  // dropout: the row bytes of key runs kv0 + 16·kk + 4·half (+ 8), kk = 0..3
  uint32_t drb[2][4] = {{0, 0, 0, 0}, {0, 0, 0, 0}};
  if constexpr (DROP) {
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const int jr[4] = {kv0 + 4 * half + 8 * e, kv0 + 16 + 4 * half + 8 * e,
                         kv0 + 32 + 4 * half + 8 * e, kv0 + 48 + 4 * half + 8 * e};
      drop_row_bytes_quad(*dk, seq, head, qrow, jr, drb[e]);
    }
  }
#pragma unroll
  for (int kk = 0; kk < BC / 16; ++kk) {
    u32x4 pf = acc_operand<T>(s[kk >> 1], (kk & 1) * 2);
    r[kk] = dot2_sum<T>(pf, 0.f);
    const int k0 = kk * 16 + 4 * half;
    if constexpr (DROP) {   // keys kv0 + k0 + 0..3 (dwords 0, 1) and + 8..11 (dwords 2, 3)
      const uint32_t b0 = drb[0][kk], b1 = drb[1][kk];
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const uint32_t by = w < 2 ? b0 : b1;
        const int n = 2 * (w & 1);
        const uint32_t m = (drop_keep(by, n, dk->t) ? 0x0000ffffu : 0u) |
                           (drop_keep(by, n + 1, dk->t) ? 0xffff0000u : 0u);
        pf[w] &= m;
      }
    }
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb)
      o[cb] = mfma32<T>(lds_tr8<T, D>(vt, k0, k0 + 8, cb * 32, lane), pf, o[cb]);
  }
  float rs = (r[0] + r[1]) + (r[2] + r[3]);
#pragma unroll
  for (int kk = 4; kk < BC / 16; kk += 4) rs += (r[kk] + r[kk + 1]) + (r[kk + 2] + r[kk + 3]);
  lr += rs;
}

// WIN: sliding window, key j visible from query i iff i − a.wl ≤ j ≤ i + a.wr
// (bounds clamped to N by the caller; CAUSAL is false then)
// KVLEN: the keys of a sequence have their own length Lk (a.Nk, or
// a.cu_seqlens_k) and the Lq queries are its last Lq positions: query i sits
// at position i + Lk − Lq and, when causal, sees keys j ≤ i + Lk − Lq (no
// window, soft cap or dropout). A query that sees no key gets O = 0, LSE = −inf.
template <typename T, int D, bool CAUSAL, bool VARLEN, bool WIN, bool CAP = false,
          bool DROP = false, bool KVLEN = false>
// two workgroups per CU up to d = 128; at d = 256 the O accumulators alone
// take 128 registers and the kernel runs one workgroup per CU
__global__ __launch_bounds__(kThreads, D <= 128 ? 2 : 1) void fwd_kernel(FwdArgs a) {
  constexpr int kBC = keys_per_tile<D, DROP>();   // keys per tile
  constexpr int NKB = D / 16;    // k steps of K·Qᵀ
  constexpr int NCB = D / 32;    // 32-row blocks of Oᵀ
  constexpr int TILE = kBC * D;  // elements per K or V tile
  __shared__ __attribute__((aligned(1024))) T lds[2][2][TILE];   // [buffer][K, V]

  // the wave index is the same on every lane: readfirstlane lets the compiler
  // see that, so branches on it are scalar rather than divergent
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = lane & 31, half = lane >> 5;

  // ---- work decomposition: (q tile, sequence, head), heavy tiles first -----
  const int G = gridDim.x;
  const int logical = xcd_remap(blockIdx.x, G);
  const int qt_ord = logical % a.n_qtiles;
  // sequence index fastest: each XCD's contiguous range holds the same heads
  // of every sequence (balanced when lengths differ), and the q tiles of one
  // (sequence, head) stay adjacent so they share K and V in that XCD's L2
  const int hb = logical / a.n_qtiles;
  const int b = hb % a.B, h = hb / a.B;
  const int qt = CAUSAL ? a.n_qtiles - 1 - qt_ord : qt_ord;

  int seq0, L, T_total;   // the sequence's queries: first token, count, tokens of the batch
  if constexpr (VARLEN) {
    seq0 = a.cu_seqlens[b];
    L = a.cu_seqlens[b + 1] - seq0;
    T_total = a.cu_seqlens[a.B];
  } else {
    seq0 = b * a.N;
    L = a.N;
    T_total = a.B * a.N;
  }
  int seq0k = seq0, Lk = L;   // its keys
  if constexpr (KVLEN) {
    if constexpr (VARLEN) {
      seq0k = a.cu_seqlens_k[b];
      Lk = a.cu_seqlens_k[b + 1] - seq0k;
    } else {
      seq0k = b * a.Nk;
      Lk = a.Nk;
    }
  }
  const int off = KVLEN ? Lk - L : 0;   // key position of query 0
  const int q0 = qt * kBR;
  if (q0 >= L) return;
  const int g = h / a.group;

  const int64_t qs = (int64_t)a.Hq * D, kvs = (int64_t)a.Hkv * D;
  const T* qp = static_cast<const T*>(a.q) + (int64_t)seq0 * qs + (int64_t)h * D;
  const T* kp = static_cast<const T*>(a.k) + (int64_t)seq0k * kvs + (int64_t)g * D;
  const T* vp = static_cast<const T*>(a.v) + (int64_t)seq0k * kvs + (int64_t)g * D;

  // Key tiles [j_lo, j_hi) are visible to some row of the workgroup; within
  // them [ja, jb) need no masking (every key inside the sequence and visible
  // to every row). The rest (causal diagonal, window edges, a ragged end) run
  // with masking.
  int j_lo, ja, jb, j_hi;
  if constexpr (WIN) {
    const int k_lo = max(0, q0 - a.wl);
    const int k_hi = min(Lk, q0 + kBR + a.wr);   // one past the last visible key
    j_lo = k_lo / kBC;
    j_hi = (k_hi + kBC - 1) / kBC;
    const int first_all = q0 + kBR - 1 - a.wl;  // first key every row sees
    ja = max(j_lo, first_all <= 0 ? 0 : (first_all + kBC - 1) / kBC);
    const int last_all = q0 + a.wr - (kBC - 1);   // a tile starting here ends at q0 + wr
    jb = min(min(last_all < 0 ? 0 : last_all / kBC + 1, Lk / kBC), j_hi);
    if (jb < ja) jb = ja;
  } else {
    j_lo = ja = 0;
    if constexpr (KVLEN) {
      // the end may be <= 0 here (no key for any row of the tile, or Lk = 0)
      const int kv_end = CAUSAL ? min(Lk, q0 + kBR + off) : Lk;
      j_hi = kv_end > 0 ? (kv_end + kBC - 1) / kBC : 0;
      jb = min(CAUSAL ? min(max(q0 + off + 1, 0) / kBC, Lk / kBC) : Lk / kBC, j_hi);
    } else {
      const int kv_end = CAUSAL ? min(L, q0 + kBR) : L;
      j_hi = (kv_end + kBC - 1) / kBC;
      jb = min(CAUSAL ? min((q0 + 1) / kBC, L / kBC) : L / kBC, j_hi);
    }
  }
  const int ntiles = j_hi;

  // first tile in flight before anything else (there is none only with KVLEN)
  if (!KVLEN || ntiles > j_lo) {
    tile_dma<T, kBC, D, kWaves>(lds[0][0], kp, kvs, j_lo * kBC, Lk, wave, lane);
    tile_dma<T, kBC, D, kWaves>(lds[0][1], vp, kvs, j_lo * kBC, Lk, wave, lane);
  }

  // ---- Q fragments (B operand of Sᵀ = K·Qᵀ), kept in registers -------------
  const int qrow = q0 + wave * 32 + col;
  u32x4 qf[NKB];
  if (qrow < L) {
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) qf[kb] = ldg16(qp + qrow * qs + kb * 16 + half * 8);
  } else {
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) qf[kb] = u32x4{0, 0, 0, 0};
  }

  f32x16 o[NCB];
#pragma unroll
  for (int cb = 0; cb < NCB; ++cb) o[cb] = f32x16{};
  const float c = CAP ? 1.f : a.scale_log2;   // capped logits are already in log2 units
  const float cap_in = CAP ? a.cap_in : 0.f, cap_out = CAP ? a.cap_out : 0.f;
  const DropKey dk{a.seed_lo, a.seed_hi, a.keep_t};
  float mc = -INFINITY;   // reference max of S·c for this row
  float l = 0.f;          // Σ P over this lane half's keys (fp32), for the LSE (bf16)
  float lr = 0.f;         // the same sum of P rounded to T, for normalising O
  const int wq_first = q0 + wave * 32, wq_last = wq_first + 31;
  const int wl = WIN ? a.wl : 0, wr = WIN ? a.wr : 0;

  const DmaPlan<T, kBC, D, kWaves> plan(kvs, wave, lane);
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);
  // One tile: the copies of tile j+1 go into one LDS buffer (kn, vn) while
  // tile j is read from the other (kt, vt). Restrict-qualified, the two
  // buffers are known to be distinct, so the compiler does not make the reads
  // of tile j wait for the copies in flight (without it the transposing reads
  // of V waited for them, and the next tile's copy overlapped only the first
  // half of a tile). One body serves every call site: called with different
  // buffers, its pointer arguments stay arguments until it is inlined, which
  // is where the compiler turns the qualifiers into alias information.
  auto body = [&](auto edge_tag, int j, const T* __restrict__ kt, const T* __restrict__ vt,
                  T* __restrict__ kn, T* __restrict__ vn) __attribute__((always_inline)) {
    constexpr bool EDGE = decltype(edge_tag)::value;
    const int kv0 = j * kBC;
    if (j + 1 < ntiles) {
      const int n0 = kv0 + kBC;
      if (n0 + kBC <= Lk) {
        tile_dma_in<T, kBC, D, kWaves>(kn, kp + (int64_t)n0 * kvs, plan, wave_u);
        tile_dma_in<T, kBC, D, kWaves>(vn, vp + (int64_t)n0 * kvs, plan, wave_u);
      } else {
        tile_dma<T, kBC, D, kWaves>(kn, kp, kvs, n0, Lk, wave, lane);
        tile_dma<T, kBC, D, kWaves>(vn, vp, kvs, n0, Lk, wave, lane);
      }
    }
    // every key of the tile is after this wave's rows
    if (EDGE && CAUSAL && kv0 > wq_last + off) return;
    if (EDGE && WIN && (kv0 > wq_last + wr || kv0 + kBC - 1 < wq_first - wl))
      return;   // the tile lies outside the windows of all this wave's rows
    fwd_tile<T, D, CAUSAL, EDGE, WIN, CAP, DROP>(kt, vt, qf, o, mc, l, lr, c, kv0, Lk,
                                                 qrow + off, wl, wr, lane, cap_in, cap_out, &dk,
                                                 b, h, KVLEN);
  };
  // tile j sits in LDS buffer (j − j_lo) & 1; buf_tag fixes the tile's LDS
  // buffer at compile time where it is known (the unrolled interior pairs), so
  // that every LDS address is a per-lane register plus an immediate offset
  auto step = [&](auto edge_tag, auto buf_tag, int j) __attribute__((always_inline)) {
    constexpr int FIXED = decltype(buf_tag)::value;   // 0, 1, or -1 for (j − j_lo) & 1
    const int BUF = FIXED >= 0 ? FIXED : ((j - j_lo) & 1);
    wait_vmem_all();   // this thread's copies of tile j have landed
    __syncthreads();   // everyone's have, and tile j-1 is no longer read
    body(edge_tag, j, lds[BUF][0], lds[BUF][1], lds[BUF ^ 1][0], lds[BUF ^ 1][1]);
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
    for (; j + 1 < jb; j += 2) {   // tile j is in buffer 0, tile j+1 in buffer 1
      step(std::false_type{}, B0{}, j);
      step(std::false_type{}, B1{}, j + 1);
    }
    if (j < jb) step(std::false_type{}, BR{}, j++);
  } else {
    for (; j < jb; ++j) step(std::false_type{}, BR{}, j);
  }
  for (; j < ntiles; ++j) step(std::true_type{}, BR{}, j);

  // ---- epilogue -------------------------------------------------------------
  const float lr_tot = wave_sum_halves(lr);
  const float l_tot = kLseFromUnrounded<T> ? wave_sum_halves(l) : lr_tot;
  if (qrow < L) {
    // a row that saw no key (KVLEN only): O = 0, LSE = −inf
    const bool any = !KVLEN || l_tot > 0.f;
    const float inv = any ? (DROP ? a.drop_scale : 1.f) / lr_tot : 0.f;
    T* op = static_cast<T*>(a.o) + (int64_t)seq0 * qs + (int64_t)h * D + qrow * qs;
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        u32x2 w;
        w[0] = pack2<T>(o[cb][4 * r + 0] * inv, o[cb][4 * r + 1] * inv);
        w[1] = pack2<T>(o[cb][4 * r + 2] * inv, o[cb][4 * r + 3] * inv);
        *reinterpret_cast<u32x2*>(op + cb * 32 + 8 * r + 4 * half) = w;
      }
    if (half == 0)
      a.lse[(int64_t)h * T_total + seq0 + qrow] = any ? (mc + log2f(l_tot)) * kLn2 : -INFINITY;
  }
}

template <typename T, int D, bool CAUSAL, bool VARLEN, bool WIN, bool CAP = false,
          bool DROP = false, bool KVLEN = false>
hipError_t launch(const FwdArgs& a, hipStream_t stream) {
  const int grid = a.n_qtiles * a.Hq * a.B;
  (void)hipGetLastError();  // drop an error left pending by earlier, unrelated HIP calls
  hipLaunchKernelGGL((fwd_kernel<T, D, CAUSAL, VARLEN, WIN, CAP, DROP, KVLEN>), dim3(grid),
                     dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

template <typename T, int D>
hipError_t dispatch_kvlen(const FwdArgs& a, bool causal, bool varlen, hipStream_t s) {
  if (causal)
    return varlen ? launch<T, D, true, true, false, false, false, true>(a, s)
                  : launch<T, D, true, false, false, false, false, true>(a, s);
  return varlen ? launch<T, D, false, true, false, false, false, true>(a, s)
                : launch<T, D, false, false, false, false, false, true>(a, s);
}

template <typename T, int D>
hipError_t dispatch_mask(const FwdArgs& a, int mask, bool varlen, bool cap, bool drop,
                         hipStream_t s) {
  // dropout: no window; soft cap: any mask (checked by the caller)
  if (drop) {
    if (mask == kMaskCausal)
      return varlen ? launch<T, D, true, true, false, false, true>(a, s)
                    : launch<T, D, true, false, false, false, true>(a, s);
    return varlen ? launch<T, D, false, true, false, false, true>(a, s)
                  : launch<T, D, false, false, false, false, true>(a, s);
  }
  if (cap) {
    if (mask == kMaskWindow)
      return varlen ? launch<T, D, false, true, true, true>(a, s)
                    : launch<T, D, false, false, true, true>(a, s);
    if (mask == kMaskCausal)
      return varlen ? launch<T, D, true, true, false, true>(a, s)
                    : launch<T, D, true, false, false, true>(a, s);
    return varlen ? launch<T, D, false, true, false, true>(a, s)
                  : launch<T, D, false, false, false, true>(a, s);
  }
  if (mask == kMaskWindow)
    return varlen ? launch<T, D, false, true, true>(a, s) : launch<T, D, false, false, true>(a, s);
  if (mask == kMaskCausal)
    return varlen ? launch<T, D, true, true, false>(a, s) : launch<T, D, true, false, false>(a, s);
  return varlen ? launch<T, D, false, true, false>(a, s) : launch<T, D, false, false, false>(a, s);
}

}  // namespace

int fwd_query_tile() { return kBR; }

hipError_t launch_fwd(const FwdArgs& a, bool bf16_in, int d, int mask, bool varlen, bool cap,
                      bool drop, hipStream_t s) {
  if (bf16_in) {
    if (d == 64) return dispatch_mask<bf16, 64>(a, mask, varlen, cap, drop, s);
    if (d == 128) return dispatch_mask<bf16, 128>(a, mask, varlen, cap, drop, s);
    return dispatch_mask<bf16, 256>(a, mask, varlen, cap, drop, s);
  }
  if (d == 64) return dispatch_mask<f16, 64>(a, mask, varlen, cap, drop, s);
  if (d == 128) return dispatch_mask<f16, 128>(a, mask, varlen, cap, drop, s);
  return dispatch_mask<f16, 256>(a, mask, varlen, cap, drop, s);
}

hipError_t launch_fwd_kvlen(const FwdArgs& a, bool bf16_in, int d, bool causal, bool varlen,
                            hipStream_t s) {
  if (bf16_in) {
    if (d == 64) return dispatch_kvlen<bf16, 64>(a, causal, varlen, s);
    if (d == 128) return dispatch_kvlen<bf16, 128>(a, causal, varlen, s);
    return dispatch_kvlen<bf16, 256>(a, causal, varlen, s);
  }
  if (d == 64) return dispatch_kvlen<f16, 64>(a, causal, varlen, s);
  if (d == 128) return dispatch_kvlen<f16, 128>(a, causal, varlen, s);
  return dispatch_kvlen<f16, 256>(a, causal, varlen, s);
}

}  // namespace fa
