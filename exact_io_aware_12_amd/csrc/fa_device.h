// Device helpers shared by the forward and backward kernels (gfx950 only).
//
// MFMA 32x32x16 (bf16 / fp16 in, fp32 accumulate), one wavefront of 64 lanes:
//   A operand: lane l holds row  l%32, k-slots 8·(l/32) + e, e = 0..7
//   B operand: lane l holds col  l%32, k-slots 8·(l/32) + e
//   C/D      : lane l holds col  l%32, rows 8·r + 4·(l/32) + t in element 4·r + t
// The contraction pairs A's slot (l/32, e) with B's slot (l/32, e), so any
// consistent assignment of the k index to slots is a valid product. The
// kernels use that freedom to feed an accumulator straight back in as an
// operand: an accumulator column holds, in lane half h, the k values
// {4h..4h+3, 8+4h..8+4h+3} of each 16-wide k step, and the matching operand
// from LDS is stored with the same permutation (see perm16()).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

typedef __bf16 bf16;
typedef _Float16 f16;
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef f16 f16x8 __attribute__((ext_vector_type(8)));
typedef bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef f16 f16x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

template <typename T>
__device__ __forceinline__ f32x16 mfma32(u32x4 a, u32x4 b, f32x16 c) {
  if constexpr (__is_same(T, bf16)) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
  } else {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                  __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
  }
}

// Two floats -> two 16-bit values of T packed in one dword, round to nearest even.
template <typename T>
__device__ __forceinline__ uint32_t pack2(float lo, float hi) {
  f32x2 x = {lo, hi};
  if constexpr (__is_same(T, bf16)) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(x, bf16x2));
  } else {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(x, f16x2));
  }
}

// Elements 4·r .. 4·r+7 of an accumulator (rows 8r+4h+t and 8(r+1)+4h+t for
// even r) as one 8-element operand, i.e. the 16-wide k step r/2 of the
// accumulator's row dimension in the permuted slot order.
template <typename T>
__device__ __forceinline__ u32x4 acc_operand(const f32x16& a, int r) {
  u32x4 p;
  p[0] = pack2<T>(a[4 * r + 0], a[4 * r + 1]);
  p[1] = pack2<T>(a[4 * r + 2], a[4 * r + 3]);
  p[2] = pack2<T>(a[4 * r + 4], a[4 * r + 5]);
  p[3] = pack2<T>(a[4 * r + 6], a[4 * r + 7]);
  return p;
}

// Position, inside a 16-wide k step, where operand data for index x (0..15)
// is stored so that lane half h reads slots e = 0..7 contiguously as the
// indices {4h..4h+3, 8+4h..8+4h+3}: the middle two groups of 4 swap places.
__device__ __forceinline__ constexpr int perm16(int x) {
  return (x & ~15) | (((x >> 2) & 1) << 3) | (((x >> 3) & 1) << 2) | (x & 3);
}

// 4 rows x 8 columns of 16-bit values (one 16-byte chunk per row) ->
// column w as 4 values (rows 0..3) in two dwords.
__device__ __forceinline__ u32x2 transpose_col(const u32x4 (&in)[4], int w) {
  const int dw = w >> 1;
  u32x2 r;
  if (w & 1) {
    r[0] = (in[0][dw] >> 16) | (in[1][dw] & 0xffff0000u);
    r[1] = (in[2][dw] >> 16) | (in[3][dw] & 0xffff0000u);
  } else {
    r[0] = (in[0][dw] & 0xffffu) | (in[1][dw] << 16);
    r[1] = (in[2][dw] & 0xffffu) | (in[3][dw] << 16);
  }
  return r;
}

// Lanes l and l^32 hold the two halves of one column. v_permlane32_swap
// (gfx950) exchanges the upper half of its first operand with the lower half
// of its second, so swapping x with itself leaves, in every lane, x of lanes
// l and l^32 in the two results (in the same order on both halves: the sum
// is bitwise identical across the pair). A VALU exchange, no LDS round trip.
__device__ __forceinline__ float wave_max_halves(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

__device__ __forceinline__ float wave_sum_halves(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// ---------------------------------------------------------------------------
// Dropout keep decisions. Philox4x32-10, the counter-based generator of
// Salmon, Moraes, Dror and Shaw ("Parallel Random Numbers: As Easy as 1, 2,
// 3", SC '11): per round two 32 x 32 -> 64-bit products,
// c <- (hi1 ^ c1 ^ k0, lo1, hi0 ^ c3 ^ k1, lo0), the key advanced by the Weyl
// constants between rounds. One call covers a 4 x 4 block of (query i, key j)
// of one query head and sequence: counter (j/4, i/4, head, seq), key = seed;
// word i % 4, byte j % 4 is the element's byte, kept iff byte < t.
__device__ __forceinline__ u32x4 philox4x32_10(uint32_t c0, uint32_t c1, uint32_t c2,
                                               uint32_t c3, uint32_t k0, uint32_t k1) {
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    if (r) {
      k0 += 0x9E3779B9u;
      k1 += 0xBB67AE85u;
    }
    const uint64_t p0 = (uint64_t)0xD2511F53u * c0;
    const uint64_t p1 = (uint64_t)0xCD9E8D57u * c2;
    const uint32_t n0 = (uint32_t)(p1 >> 32) ^ c1 ^ k0;
    const uint32_t n2 = (uint32_t)(p0 >> 32) ^ c3 ^ k1;
    c1 = (uint32_t)p1;
    c3 = (uint32_t)p0;
    c0 = n0;
    c2 = n2;
  }
  return u32x4{c0, c1, c2, c3};
}

struct DropKey {
  uint32_t k0, k1;   // the seed
  uint32_t t;        // keep iff byte < t (1 ≤ t ≤ 256)
};

// The bytes of query i for keys j0 .. j0+3 (j0 % 4 == 0): byte n is key j0 + n.
__device__ __forceinline__ uint32_t drop_row_bytes(const DropKey& dk, int seq, int head, int i,
                                                   int j0) {
  const u32x4 w = philox4x32_10((uint32_t)j0 >> 2, (uint32_t)i >> 2, (uint32_t)head,
                                (uint32_t)seq, dk.k0, dk.k1);
  const int r = i & 3;
  return r == 0 ? w[0] : r == 1 ? w[1] : r == 2 ? w[2] : w[3];
}

// The bytes of key j for queries i0 .. i0+3 (i0 % 4 == 0): byte n is query i0 + n.
__device__ __forceinline__ uint32_t drop_col_bytes(const DropKey& dk, int seq, int head, int i0,
                                                   int j) {
  const u32x4 w = philox4x32_10((uint32_t)j >> 2, (uint32_t)i0 >> 2, (uint32_t)head,
                                (uint32_t)seq, dk.k0, dk.k1);
  const int sh = 8 * (j & 3);
  return ((w[0] >> sh) & 0xffu) | (((w[1] >> sh) & 0xffu) << 8) |
         (((w[2] >> sh) & 0xffu) << 16) | (((w[3] >> sh) & 0xffu) << 24);
}

__device__ __forceinline__ uint32_t pick4(const u32x4& w, int n) {
  return n == 0 ? w[0] : n == 1 ? w[1] : n == 2 ? w[2] : w[3];
}

// drop_row_bytes for four key runs j[0..3] at once, shared by the four lanes of
// a quad that hold the four queries of one 4 x 4 block row (query i, lane quad
// index i % 4; j[] the same on all four lanes). Each lane runs the generator
// for run j[i % 4] only; three exchanges inside the quad hand every lane its
// word of the other three calls. out[m] is the row bytes for run j[m].
__device__ __forceinline__ void drop_row_bytes_quad(const DropKey& dk, int seq, int head, int i,
                                                    const int (&j)[4], uint32_t (&out)[4]) {
  const int s = i & 3;
  const int js = s == 0 ? j[0] : s == 1 ? j[1] : s == 2 ? j[2] : j[3];
  const u32x4 w = philox4x32_10((uint32_t)js >> 2, (uint32_t)i >> 2, (uint32_t)head,
                                (uint32_t)seq, dk.k0, dk.k1);
  uint32_t got[4];   // got[r]: from lane s ^ r, i.e. run j[s ^ r]
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const uint32_t send = pick4(w, s ^ r);   // lane s ^ r wants word s ^ r
    got[r] = r == 0 ? send : (uint32_t)__shfl_xor((int)send, r);
  }
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    const int r = s ^ m;
    out[m] = r == 0 ? got[0] : r == 1 ? got[1] : r == 2 ? got[2] : got[3];
  }
}

__device__ __forceinline__ bool drop_keep(uint32_t bytes, int n, uint32_t t) {
  return ((bytes >> (8 * n)) & 0xffu) < t;
}

// tanh(x) = 1 − 2 / (1 + e^(2x)) from the exponential and reciprocal units:
// exactly ±1 once e^(2x) overflows or vanishes, absolute error ≈1e-7 near 0.
__device__ __forceinline__ float tanh_fast(float x) {
  return 1.f - 2.f * __builtin_amdgcn_rcpf(1.f + fast_exp2(x * (2.f * kLog2e)));
}

// Hardware places workgroup w on XCD w % 8 (8 XCDs, each with its own L2).
// Return a logical id so that each XCD receives one contiguous range of
// logical ids; consecutive logical ids then share K/V tiles within one L2.
__device__ __forceinline__ int xcd_remap(int w, int G) {
  const int per = G >> 3, rem = G & 7, x = w & 7;
  return x * per + (x < rem ? x : rem) + (w >> 3);
}

template <typename T>
__device__ __forceinline__ u32x4 ldg16(const T* p) {
  return *reinterpret_cast<const u32x4*>(p);
}

template <typename T>
__device__ __forceinline__ u32x4 lds16(const T* p) {
  return *reinterpret_cast<const u32x4*>(p);
}

// Row-major tile: rows r0 .. r0+R-1 of a sequence with L rows, D columns,
// into lds[r·LS + c]; rows at or past L are zero. Consecutive threads read
// consecutive 16-byte chunks of a row.
template <typename T, int R, int D, int LS, int NT>
__device__ __forceinline__ void tile_to_lds(T* lds, const T* src, int64_t rstride, int r0, int L,
                                            int tid) {
  constexpr int CH = R * D / 8;
#pragma unroll
  for (int u = 0; u < (CH + NT - 1) / NT; ++u) {
    const int ci = tid + NT * u;
    if (CH % NT == 0 || ci < CH) {
      const int r = ci / (D / 8), dc = ci % (D / 8);
      u32x4 val = u32x4{0, 0, 0, 0};
      if (r0 + r < L) val = ldg16(src + (int64_t)(r0 + r) * rstride + dc * 8);
      *reinterpret_cast<u32x4*>(lds + r * LS + dc * 8) = val;
    }
  }
}

// Transposed tile: lds_t[c·LS_T + perm16(r)] = src[r0 + r][c], rows at or past
// L are zero. A thread reads a 4-row x 8-column block and writes 8 rows of
// the transpose (4 values each). When ROWS_TOO is set the same block is also
// stored row-major into lds[r·LS + c].
template <typename T, int R, int D, int LS_T, int NT, bool ROWS_TOO = false, int LS = D + 8>
__device__ __forceinline__ void tile_to_lds_t(T* lds_t, T* lds, const T* src, int64_t rstride,
                                              int r0, int L, int tid) {
  constexpr int BL = (R / 4) * (D / 8);
#pragma unroll
  for (int u = 0; u < (BL + NT - 1) / NT; ++u) {
    const int bi = tid + NT * u;
    if (BL % NT == 0 || bi < BL) {
      const int rq = bi % (R / 4), dc = bi / (R / 4);
      u32x4 in[4];
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        const int row = r0 + 4 * rq + rr;
        in[rr] = row < L ? ldg16(src + (int64_t)row * rstride + dc * 8) : u32x4{0, 0, 0, 0};
      }
      const int pos = perm16(4 * rq);
#pragma unroll
      for (int w = 0; w < 8; ++w)
        *reinterpret_cast<u32x2*>(lds_t + (dc * 8 + w) * LS_T + pos) = transpose_col(in, w);
      if constexpr (ROWS_TOO) {
#pragma unroll
        for (int rr = 0; rr < 4; ++rr)
          *reinterpret_cast<u32x4*>(lds + (4 * rq + rr) * LS + dc * 8) = in[rr];
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Direct global -> LDS staging (gfx950 global_load_lds, 16 bytes per lane).
// A wave instruction writes 1 KiB of LDS: lane l's 16 bytes land in slot l.
// Tiles are row-major with D·2-byte rows; the 16-byte chunks of row r are
// stored in the order chunk ^ swz(r), chosen per lane on the global side.
// The permutation makes both read patterns below bank-conflict free (64
// banks x 4 bytes): 16 lanes reading one chunk of 16 consecutive rows, and
// 32 lanes reading 4 consecutive rows x 32 columns with the transposing read.
// Rows of 256 and 512 bytes (d = 128, 256) start on the same bank, so the
// bank of a chunk depends only on its index mod 16 and one 4-bit
// permutation serves both; 128-byte rows (d = 64) need their own.
template <int D>
__device__ __forceinline__ constexpr int swz(int r) {
  return D >= 128 ? (((r & 3) << 2) | ((r >> 2) & 3)) : ((((r >> 1) & 1) << 2) | ((r >> 2) & 3));
}

// Cache-policy operand of a global load: 0 keeps the lines for reuse; kCpolStream
// marks them non-temporal (the gfx940-family NT bit), for data read exactly once.
constexpr int kCpolStream = 2;

// Stage rows r0 .. r0+R-1 (row stride `rstride` elements) of a D-column tile.
// Rows at or past L are replaced by row L-1 (L >= 1): callers mask them.
// The tile is split evenly over the NW waves of the workgroup; CPOL is the
// copies' cache policy.
template <typename T, int R, int D, int NW, int CPOL = 0>
__device__ __forceinline__ void tile_dma(T* lds, const T* src, int64_t rstride, int r0, int L,
                                         int wave, int lane) {
  constexpr int CPR = D / 8;                  // 16-byte chunks per row
  constexpr int RPI = 64 / CPR;               // rows per wave instruction
  constexpr int INSTS = R / RPI;
  static_assert(INSTS % NW == 0, "tile rows must split evenly over the waves");
#pragma unroll
  for (int u = 0; u < INSTS / NW; ++u) {
    const int inst = wave * (INSTS / NW) + u;
    const int row = inst * RPI + lane / CPR;
    const int c = (lane % CPR) ^ swz<D>(row);
    const int srow = min(r0 + row, L - 1);
    const T* g = src + (int64_t)srow * rstride + c * 8;
#if defined(__HIP_DEVICE_COMPILE__)  // the host pass cannot type-check this device builtin
    __builtin_amdgcn_global_load_lds(g, (__attribute__((address_space(3))) void*)(lds + inst * 512),
                                     16, 0, CPOL);
#else
    (void)g;
#endif
  }
}

// Fourth dword of a raw buffer resource on gfx9-family parts: 32-bit data
// format, no swizzle; with stride 0 the range check is on byte offsets.
constexpr int kBufferDword3 = 0x00020000;

// Per-lane byte offsets, relative to the tile's first row, of the pieces a
// wave copies in tile_dma. They are the same for every tile of a matrix, so
// a tile that lies wholly inside the sequence is copied from a uniform base
// pointer plus these offsets, with no per-tile vector address arithmetic.
template <typename T, int R, int D, int NW>
struct DmaPlan {
  static constexpr int CPR = D / 8;
  static constexpr int RPI = 64 / CPR;
  static constexpr int PER = R / RPI / NW;   // copy instructions per wave
  static_assert((R / RPI) % NW == 0, "tile rows must split evenly over the waves");
  uint32_t off[PER];
  __device__ __forceinline__ DmaPlan(int64_t rstride, int wave, int lane) {
#pragma unroll
    for (int u = 0; u < PER; ++u) {
      const int row = (wave * PER + u) * RPI + lane / CPR;
      const int c = (lane % CPR) ^ swz<D>(row);
      off[u] = (uint32_t)((row * rstride + c * 8) * (int64_t)sizeof(T));
    }
  }
};

// tile_dma for a tile whose R rows all lie inside the sequence; `src_r0`
// points at the tile's first row and `wave` is the same on all lanes. A
// buffer load with a 32-bit per-lane offset keeps the base in scalar
// registers; the resource covers 2 GiB from the tile's first row and the
// offsets stay far below that. The buffer form also issues far faster than
// the flat-address form (global_load_lds) while another wave on the same SIMD
// runs MFMAs: measured on MI355X, 8 copies took 149 cycles against 1925.
// CPOL is the copies' cache policy.
template <typename T, int R, int D, int NW, int CPOL = 0>
__device__ __forceinline__ void tile_dma_in(T* lds, const T* src_r0, const DmaPlan<T, R, D, NW>& p,
                                            int wave) {
#if defined(__HIP_DEVICE_COMPILE__)  // the host pass cannot type-check these device builtins
  const __amdgpu_buffer_rsrc_t rsrc =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<T*>(src_r0), 0, 0x7fffffff, kBufferDword3);
#pragma unroll
  for (int u = 0; u < DmaPlan<T, R, D, NW>::PER; ++u)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        rsrc,
        (__attribute__((address_space(3))) void*)(lds + (wave * DmaPlan<T, R, D, NW>::PER + u) * 512),
        16, p.off[u], 0, 0, CPOL);
#else
  (void)lds;
  (void)src_r0;
  (void)p;
  (void)wave;
#endif
}

// 16-byte operand read: row r, logical chunk c (8 elements from column 8c).
template <typename T, int D>
__device__ __forceinline__ u32x4 lds_row16(const T* lds, int r, int c) {
  return *reinterpret_cast<const u32x4*>(lds + r * D + 8 * (c ^ swz<D>(r)));
}

typedef short i16x4 __attribute__((ext_vector_type(4)));

// Transposed operand from a row-major tile (rows = k, columns = n): lane l
// receives, for MFMA slots 0..7, tile[k][n] with n = n0 + l%32 and
// k = k0 + {0..3} (slots 0-3) and k1 + {0..3} (slots 4-7). With lane j of a
// 16-lane group reading row k+(j>>2), columns n+4(j&3)..+3, the transposing
// read hands lane i of the group the 4 rows of column n+i.
template <typename T, int D>
__device__ __forceinline__ u32x4 lds_tr8(const T* lds, int k0, int k1, int n0, int lane) {
  const int j = lane & 15;
  const int n = n0 + 16 * ((lane >> 4) & 1) + 4 * (j & 3);
  const int c = n >> 3, off = n & 7;
  const int ka = k0 + (j >> 2), kb = k1 + (j >> 2);
  typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
  const i16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (lds_i16x4*)(lds + ka * D + 8 * (c ^ swz<D>(ka)) + off));
  const i16x4 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (lds_i16x4*)(lds + kb * D + 8 * (c ^ swz<D>(kb)) + off));
  const u32x2 ua = __builtin_bit_cast(u32x2, a), ub = __builtin_bit_cast(u32x2, b);
  return u32x4{ua[0], ua[1], ub[0], ub[1]};
}

// The same two reads with the per-lane byte offsets precomputed. The offsets
// depend only on the lane and on the row and column blocks mod 16, so a loop
// computes them once and adds a uniform tile base (and constant k steps)
// instead of redoing the swizzle arithmetic for every read.
template <int D>
__device__ __forceinline__ uint32_t row16_off(int r, int c) {
  return (uint32_t)(r * D + 8 * (c ^ swz<D>(r))) * 2u;
}
template <int D>
__device__ __forceinline__ uint32_t tr8_off(int k, int n0, int lane) {
  const int j = lane & 15;
  const int n = n0 + 16 * ((lane >> 4) & 1) + 4 * (j & 3);
  const int kr = k + (j >> 2);
  return (uint32_t)(kr * D + 8 * ((n >> 3) ^ swz<D>(kr)) + (n & 7)) * 2u;
}
template <typename T>
__device__ __forceinline__ u32x4 lds_at16(const T* base, uint32_t off) {
  return *reinterpret_cast<const u32x4*>(reinterpret_cast<const char*>(base) + off);
}
template <typename T>
__device__ __forceinline__ u32x4 lds_tr8_at(const T* base, uint32_t off_a, uint32_t off_b) {
  typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
  const char* b = reinterpret_cast<const char*>(base);
  const i16x4 x = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(b + off_a));
  const i16x4 y = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(b + off_b));
  const u32x2 ux = __builtin_bit_cast(u32x2, x), uy = __builtin_bit_cast(u32x2, y);
  return u32x4{ux[0], ux[1], uy[0], uy[1]};
}

// LDS byte address of a __shared__ object (32 bits) and reads at such an
// address: an address of the form (uniform base + per-lane offset) + constant
// lets the constant go into the instruction's offset field.
constexpr uint32_t kLdsAddrMask = (1u << 18) - 1;   // every LDS byte address is below this

template <typename P>
__device__ __forceinline__ uint32_t lds_addr(const P* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) char*)(const char*)p;
}
__device__ __forceinline__ u32x4 lds_read16(uint32_t addr) {
  return *(const __attribute__((address_space(3))) u32x4*)(uintptr_t)addr;
}
__device__ __forceinline__ u32x4 lds_read_tr8(uint32_t addr_a, uint32_t addr_b) {
  typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
  const i16x4 x = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(uintptr_t)addr_a);
  const i16x4 y = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(uintptr_t)addr_b);
  const u32x2 ux = __builtin_bit_cast(u32x2, x), uy = __builtin_bit_cast(u32x2, y);
  return u32x4{ux[0], ux[1], uy[0], uy[1]};
}

// Sum of the 8 values of a packed operand (4 dwords of 2 x T), fp32 accumulate.
template <typename T>
__device__ __forceinline__ float dot2_sum(u32x4 p, float acc) {
  if constexpr (__is_same(T, bf16)) {
    const bf16x2 one = __builtin_bit_cast(bf16x2, 0x3f803f80u);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t w = p[i];  // bit_cast straight from p[i] would ignore the index
      acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w), one, acc, false);
    }
  } else {
    const f16x2 one = __builtin_bit_cast(f16x2, 0x3c003c00u);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t w = p[i];
      acc = __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, w), one, acc, false);
    }
  }
  return acc;
}

__device__ __forceinline__ void wait_vmem_all() { __builtin_amdgcn_s_waitcnt(0x0f70); }

// Workgroup barrier for LDS traffic only: this wave's LDS reads and writes
// have completed (lgkmcnt 0) when it arrives. Unlike __syncthreads it does not
// wait for global loads or for global -> LDS copies still in flight (a
// workgroup release fence does, since the copies write LDS); the caller orders
// those copies itself. The memory clobber keeps the compiler from moving
// memory accesses across it.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// The forward kernels normalise O by the row sum of P as rounded to T for the
// MFMAs (the rounding of a dominant P then cancels in O). The LSE takes that
// same sum for fp16, whose rounding (2^-11 relative at most) stays inside the
// LSE tolerance, but needs its own fp32 sum of the unrounded P for bf16, where
// one rounding (up to 2^-8) could move a dominated row's LSE by 4e-3.
template <typename T>
constexpr bool kLseFromUnrounded = __is_same(T, bf16);

}  // namespace fa
