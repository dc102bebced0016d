// FP8 (e4m3) attention forward for gfx950.
//
// Q, K and V are e4m3fn codes, each tensor with one descale factor (a code's
// value times the descale is the real input); O is written as bf16 or fp16
// and LSE as fp32, as in the 16-bit forward. The pages name e4m3 as the
// 8-bit attention format and credit FlashAttention-3 with an FP8 forward
// (Flash Attention 是什麼, adersaytech.com, FA-1 to FA-4 table; FlashAttention-2
// 全解析, blog.gitcode.com, section 4.3); the scaling recipe is not given there and
// per-tensor descales are the plain reading.
//
// Same tiling as the 16-bit forward (128 query rows per workgroup, 32 per
// wave, 64-key tiles streamed through LDS, double-buffered), with the gfx950
// FP8 matrix instruction v_mfma_scale_f32_32x32x64_f8f6f4 (64-deep k step,
// unit block scales):
//   Sᵀ = K·Qᵀ      A = K rows, B = Q rows (32 bytes of one row per lane).
//                  The 32 rows of each MFMA block are a permutation of the
//                  tile's keys chosen so that lane half g's accumulators
//                  hold keys 32g .. 32g+31 in order (element r of block jb
//                  is key 32g + 16·jb + r).
//   softmax        as in the 16-bit kernel: base-2, scale folded into c;
//                  the reference sits 8 (log2 units) below the running max,
//                  so P ≤ 2^8 < 448 (the largest e4m3 value), the row's
//                  largest weight is exactly 2^8 and few weights are small
//                  enough for e4m3's subnormal range.
//   Oᵀ += Vᵀ·Pᵀ    P rounded to e4m3 (nearest even) packs straight into the
//                  B operand (slot e of half g = key 32g + e); the Vᵀ operand
//                  comes from 8-bit transposing LDS reads, 8 keys per read.
//   Σ P (rounded)  one more MFMA with an all-ones A operand: every element of
//                  its accumulator is the column sum of the rounded P, so O
//                  is normalised by exactly the weights it was built from.
// The LSE uses the fp32 sum of the unrounded P: one e4m3 rounding can move a
// weight by 6 %, far more than an LSE tolerance allows.
#include <type_traits>

#include "fa_device.h"
#include "fa_kernels.h"

namespace fa {

namespace {

typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef uint8_t u8;
typedef int i32x2 __attribute__((ext_vector_type(2)));

constexpr int kBR = 128;  // query rows per workgroup
constexpr int kBC = 64;   // keys per tile
constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr float kRescaleHeadroom = 8.f;
constexpr int kScaleOne = 127;           // E8M0 block scale code of 2^0
constexpr uint32_t kOnes = 0x38383838u;  // four e4m3 1.0

__device__ __forceinline__ f32x16 mfma_fp8(i32x8 a, i32x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, kScaleOne, 0,
                                                          kScaleOne);
}

// LDS tile: D-byte rows, 16-byte chunks stored in the order chunk ^ swz8<D>(row).
// The permutation spreads over all banks (a) the 16 rows {16jb + 0..7,
// 32 + 16jb + 0..7} that 16 lanes read one chunk of for Sᵀ, and (b) the 8
// consecutive rows x 2 chunks that 32 lanes read with the transposing read
// for Vᵀ. Where a row lands in the 256 bytes of one pass over the banks
// depends on the row's low bits when rows are shorter than 256 bytes, so
// the chunk permutation needs only the row bits that do not already do so:
//   d = 64  (four rows per pass):  bits 2 and 5 of the row;
//   d = 128 (two rows per pass):   bits 1, 2 and 5;
//   d = 256 (one row per pass):    bits 0, 1, 2 and 5.
template <int D>
__device__ __forceinline__ constexpr int swz8(int r) {
  if constexpr (D == 64) return (((r >> 2) & 1) << 1) | ((r >> 5) & 1);
  else if constexpr (D == 128) return (((r >> 1) & 3) << 1) | ((r >> 5) & 1);
  else return ((r & 7) << 1) | ((r >> 5) & 1);
}

// The tile row (key) that MFMA row i of key block jb reads for Sᵀ: rows with
// (i >> 2) & 1 == g land in lane half g's accumulators, in order.
__device__ __forceinline__ constexpr int s_key(int jb, int i) {
  return 32 * ((i >> 2) & 1) + 16 * jb + 4 * (i >> 3) + (i & 3);
}

// Copy a 64-row x D-byte tile global -> LDS (16 bytes per lane, 1 KiB per
// wave instruction, lane l's bytes land in slot l). Rows at or past L repeat
// row L-1 (L >= 1); the kernel masks those keys.
template <int D>
__device__ __forceinline__ void tile_dma8(u8* lds, const u8* src, int64_t rstride, int r0, int L,
                                          int wave, int lane) {
  constexpr int CPR = D / 16;            // chunks per row
  constexpr int RPI = 64 / CPR;          // rows per instruction
  constexpr int PER = kBC / RPI / kWaves;
#pragma unroll
  for (int u = 0; u < PER; ++u) {
    const int inst = wave * PER + u;
    const int row = inst * RPI + lane / CPR;
    const int c = (lane % CPR) ^ swz8<D>(row);
    const u8* g = src + (int64_t)min(r0 + row, L - 1) * rstride + c * 16;
#if defined(__HIP_DEVICE_COMPILE__)
    __builtin_amdgcn_global_load_lds(g, (__attribute__((address_space(3))) void*)(lds + inst * 1024),
                                     16, 0, 0);
#else
    (void)g;
#endif
  }
}

// Per-lane byte offsets of the pieces tile_dma8 copies, for tiles that lie
// wholly inside the sequence (copied from a uniform base through a buffer
// resource).
template <int D>
struct DmaPlan8 {
  static constexpr int CPR = D / 16;
  static constexpr int RPI = 64 / CPR;
  static constexpr int PER = kBC / RPI / kWaves;
  uint32_t off[PER];
  __device__ __forceinline__ DmaPlan8(int64_t rstride, int wave, int lane) {
#pragma unroll
    for (int u = 0; u < PER; ++u) {
      const int row = (wave * PER + u) * RPI + lane / CPR;
      off[u] = (uint32_t)(row * rstride + ((lane % CPR) ^ swz8<D>(row)) * 16);
    }
  }
};

template <int D>
__device__ __forceinline__ void tile_dma8_in(u8* lds, const u8* src_r0, const DmaPlan8<D>& p,
                                             int wave) {
#if defined(__HIP_DEVICE_COMPILE__)
  const __amdgpu_buffer_rsrc_t rsrc =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<u8*>(src_r0), 0, 0x7fffffff, kBufferDword3);
#pragma unroll
  for (int u = 0; u < DmaPlan8<D>::PER; ++u)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        rsrc, (__attribute__((address_space(3))) void*)(lds + (wave * DmaPlan8<D>::PER + u) * 1024),
        16, p.off[u], 0, 0, 0);
#else
  (void)lds;
  (void)src_r0;
  (void)p;
  (void)wave;
#endif
}

__device__ __forceinline__ u32x4 lds16_at(const u8* t, int byte) {
  return *reinterpret_cast<const u32x4*>(t + byte);
}

// A operand of Sᵀ: row s_key(jb, lane % 32), bytes 64·ks + 32·g .. +31.
template <int D>
__device__ __forceinline__ i32x8 k_operand(const u8* kt, int jb, int ks, int lane) {
  const int row = s_key(jb, lane & 31);
  const int c0 = 4 * ks + 2 * (lane >> 5);
  const u32x4 a = lds16_at(kt, row * D + 16 * (c0 ^ swz8<D>(row)));
  const u32x4 b = lds16_at(kt, row * D + 16 * ((c0 + 1) ^ swz8<D>(row)));
  return i32x8{(int)a[0], (int)a[1], (int)a[2], (int)a[3], (int)b[0], (int)b[1], (int)b[2],
               (int)b[3]};
}

// A operand of Oᵀ for columns 32·cb .. +31: lane l gets column 32·cb + l%32
// of keys 32g .. 32g+31 (g = l/32), 8 keys per transposing read. In each
// 16-lane group lanes 2m, 2m+1 address key 32g + 8r + m, bytes 0-7 and 8-15
// of the group's 16-column span; the read hands lane i column i of the 8 rows.
template <int D>
__device__ __forceinline__ i32x8 v_operand(const u8* vt, int cb, int lane) {
  typedef __attribute__((address_space(3))) i32x2 lds_i32x2;
  const int j = lane & 15, grp = (lane >> 4) & 1, g = lane >> 5;
  const int c = 2 * cb + grp;
  i32x8 r;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int row = 32 * g + 8 * q + (j >> 1);
    const i32x2 t = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
        (lds_i32x2*)(vt + row * D + 16 * (c ^ swz8<D>(row)) + 8 * (j & 1)));
    r[2 * q] = t[0];
    r[2 * q + 1] = t[1];
  }
  return r;
}

// P (two accumulators, key 32g + 16·jb + r in element r of s[jb]) rounded to
// e4m3, four keys per dword in key order: the B operand of Oᵀ += Vᵀ·Pᵀ.
__device__ __forceinline__ i32x8 p_operand(const f32x16 (&s)[2]) {
  i32x8 p;
#pragma unroll
  for (int w = 0; w < 8; ++w) {
    const int jb = w >> 2, r = 4 * (w & 3);
    // the first convert fills bytes 0-1 and keeps bytes 2-3 of its third
    // operand, which the second convert overwrites: any register will do
    const int lo = __builtin_amdgcn_cvt_pk_fp8_f32(s[jb][r], s[jb][r + 1],
                                                   __builtin_bit_cast(int, s[jb][r + 2]), false);
    p[w] = __builtin_amdgcn_cvt_pk_fp8_f32(s[jb][r + 2], s[jb][r + 3], lo, true);
  }
  return p;
}

// Where the next tile's copies go and come from (NONE: no next tile).
enum class NextCopy { NONE, INSIDE, CLAMPED };

// One 64-key tile. The copies of the next tile into the other LDS buffer are
// issued first; with every LDS pointer declared __restrict__ in this one
// inlined function the compiler knows those copies do not overlap the
// current tile's reads and does not make the reads wait for them.
template <int D, bool CAUSAL, bool EDGE>
__device__ __forceinline__ void fwd8_tile(const u8* __restrict__ kt, const u8* __restrict__ vt,
                                          u8* __restrict__ nk, u8* __restrict__ nv, NextCopy next,
                                          const u8* kp, const u8* vp, int64_t kvs, int n0,
                                          const DmaPlan8<D>& plan, int wave_u, int wave,
                                          bool skip, const i32x8 (&qf)[D / 64],
                                          f32x16 (&o)[D / 32], f32x16& lsum, float& mc, float& l,
                                          float c, int kv0, int L, int qrow, int lane) {
  constexpr int NKS = D / 64;
  constexpr int NCB = D / 32;
  if (next == NextCopy::INSIDE) {
    tile_dma8_in<D>(nk, kp + (int64_t)n0 * kvs, plan, wave_u);
    tile_dma8_in<D>(nv, vp + (int64_t)n0 * kvs, plan, wave_u);
  } else if (next == NextCopy::CLAMPED) {
    tile_dma8<D>(nk, kp, kvs, n0, L, wave, lane);
    tile_dma8<D>(nv, vp, kvs, n0, L, wave, lane);
  }
  if (skip) return;
  const int half = lane >> 5;
  // ---- Sᵀ = K·Qᵀ ----------------------------------------------------------
  f32x16 s[2] = {f32x16{}, f32x16{}};
#pragma unroll
  for (int ks = 0; ks < NKS; ++ks)
#pragma unroll
    for (int jb = 0; jb < 2; ++jb) s[jb] = mfma_fp8(k_operand<D>(kt, jb, ks, lane), qf[ks], s[jb]);

  if constexpr (EDGE) {
#pragma unroll
    for (int jb = 0; jb < 2; ++jb)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int key = kv0 + 32 * half + 16 * jb + i;
        const bool vis = key < L && !(CAUSAL && key > qrow);
        s[jb][i] = vis ? s[jb][i] : -INFINITY;
      }
  }

  // ---- online softmax (lazily raised reference max) -----------------------
  float mx = s[0][0];
#pragma unroll
  for (int i = 1; i < 16; ++i) mx = fmaxf(mx, s[0][i]);
#pragma unroll
  for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s[1][i]);
  const float mxc = wave_max_halves(mx) * c;
  // The reference is kept exactly kRescaleHeadroom below the row's running max
  // (raised when a tile's max passes the running max, decided per wave): every
  // weight is at most 2^8 = 256 < 448, the row's largest weight is exactly 256,
  // an e4m3 value, and small weights sit 2^8 further above e4m3's coarse
  // subnormal range than with weights ≤ 1.
  if (__builtin_amdgcn_ballot_w64(mxc > mc + kRescaleHeadroom) != 0) {   // wave-uniform
    // finite: key 0 is visible to every row
    const float mc_new = fmaxf(mc, mxc - kRescaleHeadroom);
    const float alpha = fast_exp2(mc - mc_new);
    l *= alpha;
    lsum[0] *= alpha;
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) o[cb] *= alpha;
    mc = mc_new;
  }
  float ls[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int jb = 0; jb < 2; ++jb)
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      s[jb][i] = fast_exp2(fmaf(s[jb][i], c, -mc));
      ls[i & 3] += s[jb][i];
    }
  l += (ls[0] + ls[1]) + (ls[2] + ls[3]);

  // ---- Oᵀ += Vᵀ·Pᵀ and the rounded row sum ---------------------------------
  const i32x8 pf = p_operand(s);
  const int ones = (int)kOnes;
  lsum = mfma_fp8(i32x8{ones, ones, ones, ones, ones, ones, ones, ones}, pf, lsum);
#pragma unroll
  for (int cb = 0; cb < NCB; ++cb) o[cb] = mfma_fp8(v_operand<D>(vt, cb, lane), pf, o[cb]);
}

// two workgroups per CU up to d = 128; at d = 256 the O accumulators alone take
// 128 registers and the kernel runs one per CU
template <typename TO, int D, bool CAUSAL, bool VARLEN>
__global__ __launch_bounds__(kThreads, D <= 128 ? 2 : 1) void fwd8_kernel(Fp8FwdArgs a) {
  constexpr int NKS = D / 64;
  constexpr int NCB = D / 32;
  constexpr int TILE = kBC * D;   // bytes per K or V tile
  __shared__ __attribute__((aligned(1024))) u8 lds[2][2][TILE];   // [buffer][K, V]

  // the wave index is the same on every lane: readfirstlane lets the compiler
  // see that, so branches on it are scalar rather than divergent
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = lane & 31, half = lane >> 5;

  // ---- work decomposition as in the 16-bit forward -------------------------
  const int G = gridDim.x;
  const int logical = xcd_remap(blockIdx.x, G);
  const int qt_ord = logical % a.n_qtiles;
  const int hb = logical / a.n_qtiles;
  const int b = hb % a.B, h = hb / a.B;
  const int qt = CAUSAL ? a.n_qtiles - 1 - qt_ord : qt_ord;

  int seq0, L, T_total;
  if constexpr (VARLEN) {
    seq0 = a.cu_seqlens[b];
    L = a.cu_seqlens[b + 1] - seq0;
    T_total = a.cu_seqlens[a.B];
  } else {
    seq0 = b * a.N;
    L = a.N;
    T_total = a.B * a.N;
  }
  const int q0 = qt * kBR;
  if (q0 >= L) return;
  const int g = h / a.group;

  const int64_t qs = (int64_t)a.Hq * D, kvs = (int64_t)a.Hkv * D;
  const u8* qp = static_cast<const u8*>(a.q) + (int64_t)seq0 * qs + (int64_t)h * D;
  const u8* kp = static_cast<const u8*>(a.k) + (int64_t)seq0 * kvs + (int64_t)g * D;
  const u8* vp = static_cast<const u8*>(a.v) + (int64_t)seq0 * kvs + (int64_t)g * D;

  // tiles [0, jb) need no mask; [jb, ntiles) hold the causal diagonal or the
  // ragged end of the sequence
  const int kv_end = CAUSAL ? min(L, q0 + kBR) : L;
  const int ntiles = (kv_end + kBC - 1) / kBC;
  const int jb = min(CAUSAL ? min((q0 + 1) / kBC, L / kBC) : L / kBC, ntiles);

  tile_dma8<D>(lds[0][0], kp, kvs, 0, L, wave, lane);
  tile_dma8<D>(lds[0][1], vp, kvs, 0, L, wave, lane);

  // ---- Q fragments: lane (query col, half g) holds bytes 64·ks + 32·g .. +31
  const int qrow = q0 + wave * 32 + col;
  i32x8 qf[NKS];
#pragma unroll
  for (int ks = 0; ks < NKS; ++ks) {
    u32x4 x = u32x4{0, 0, 0, 0}, y = u32x4{0, 0, 0, 0};
    if (qrow < L) {
      const u8* p = qp + qrow * qs + 64 * ks + 32 * half;
      x = *reinterpret_cast<const u32x4*>(p);
      y = *reinterpret_cast<const u32x4*>(p + 16);
    }
    qf[ks] = i32x8{(int)x[0], (int)x[1], (int)x[2], (int)x[3],
                   (int)y[0], (int)y[1], (int)y[2], (int)y[3]};
  }

  f32x16 o[NCB];
#pragma unroll
  for (int cb = 0; cb < NCB; ++cb) o[cb] = f32x16{};
  f32x16 lsum = f32x16{};     // every element: Σ of the rounded P of this row
  const float c = a.scale_log2;
  float mc = -INFINITY;
  float l = 0.f;              // Σ of the unrounded P over this lane half's keys
  const int wq_last = q0 + wave * 32 + 31;

  const DmaPlan8<D> plan(kvs, wave, lane);
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);
  // tile j sits in LDS buffer j & 1; buf_tag fixes it at compile time where
  // it is known (the unrolled interior pairs), so that every LDS address is a
  // per-lane register plus an immediate offset
  auto step = [&](auto edge_tag, auto buf_tag, int j) __attribute__((always_inline)) {
    constexpr bool EDGE = decltype(edge_tag)::value;
    constexpr int FIXED = decltype(buf_tag)::value;   // 0, 1, or -1 for j & 1
    const int BUF = FIXED >= 0 ? FIXED : (j & 1);
    const int kv0 = j * kBC;
    wait_vmem_all();   // this thread's copies of tile j have landed
    __syncthreads();   // everyone's have, and tile j-1 is no longer read
    const int n0 = kv0 + kBC;
    const NextCopy next = j + 1 >= ntiles ? NextCopy::NONE
                          : n0 + kBC <= L ? NextCopy::INSIDE : NextCopy::CLAMPED;
    // an edge tile wholly after this wave's rows is only copied, not computed
    const bool skip = EDGE && CAUSAL && kv0 > wq_last;
    fwd8_tile<D, CAUSAL, EDGE>(lds[BUF][0], lds[BUF][1], lds[BUF ^ 1][0], lds[BUF ^ 1][1], next,
                               kp, vp, kvs, n0, plan, wave_u, wave, skip, qf, o, lsum, mc, l, c,
                               kv0, L, qrow, lane);
  };
  using B0 = std::integral_constant<int, 0>;
  using B1 = std::integral_constant<int, 1>;
  using BR = std::integral_constant<int, -1>;
  int j = 0;
  for (; j + 1 < jb; j += 2) {   // tile j is in buffer 0, tile j+1 in buffer 1
    step(std::false_type{}, B0{}, j);
    step(std::false_type{}, B1{}, j + 1);
  }
  if (j < jb) step(std::false_type{}, BR{}, j++);
  for (; j < ntiles; ++j) step(std::true_type{}, BR{}, j);

  // ---- epilogue -------------------------------------------------------------
  const float l_tot = wave_sum_halves(l);
  if (qrow < L) {
    const float inv = a.o_scale / lsum[0];
    TO* op = static_cast<TO*>(a.o) + (int64_t)seq0 * qs + (int64_t)h * D + (int64_t)qrow * qs;
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        u32x2 w;
        w[0] = pack2<TO>(o[cb][4 * r + 0] * inv, o[cb][4 * r + 1] * inv);
        w[1] = pack2<TO>(o[cb][4 * r + 2] * inv, o[cb][4 * r + 3] * inv);
        *reinterpret_cast<u32x2*>(op + cb * 32 + 8 * r + 4 * half) = w;
      }
    if (half == 0) a.lse[(int64_t)h * T_total + seq0 + qrow] = (mc + log2f(l_tot)) * kLn2;
  }
}

template <typename TO, int D, bool CAUSAL, bool VARLEN>
hipError_t launch8(const Fp8FwdArgs& a, hipStream_t stream) {
  const int grid = a.n_qtiles * a.Hq * a.B;
  (void)hipGetLastError();
  hipLaunchKernelGGL((fwd8_kernel<TO, D, CAUSAL, VARLEN>), dim3(grid), dim3(kThreads), 0, stream,
                     a);
  return hipGetLastError();
}

template <typename TO, int D>
hipError_t dispatch8(const Fp8FwdArgs& a, bool causal, bool varlen, hipStream_t s) {
  if (causal) return varlen ? launch8<TO, D, true, true>(a, s) : launch8<TO, D, true, false>(a, s);
  return varlen ? launch8<TO, D, false, true>(a, s) : launch8<TO, D, false, false>(a, s);
}

}  // namespace

int fwd_fp8_query_tile() { return kBR; }

hipError_t launch_fwd_fp8(const Fp8FwdArgs& a, bool bf16_out, int d, bool causal, bool varlen,
                          hipStream_t s) {
  // d is 64, 128 or 256 (checked by the caller)
  if (d == 64)
    return bf16_out ? dispatch8<bf16, 64>(a, causal, varlen, s)
                    : dispatch8<f16, 64>(a, causal, varlen, s);
  if (d == 256)
    return bf16_out ? dispatch8<bf16, 256>(a, causal, varlen, s)
                    : dispatch8<f16, 256>(a, causal, varlen, s);
  return bf16_out ? dispatch8<bf16, 128>(a, causal, varlen, s)
                  : dispatch8<f16, 128>(a, causal, varlen, s);
}

}  // namespace fa
