// Device-side building blocks shared by the RLA-2 kernels (forward, state build, decode,
// feature map, backward): element helpers, cross-lane sums, the MFMA fragment layout, the
// feature map of a token pair and the segment table. Everything sits in an anonymous
// namespace, so each translation unit that includes this header has its own copy.
//
// MFMA operand layout. For v_mfma_f32_16x16x32_bf16 (and 16x16x4 f32) the A operand of
// lane l carries row l%16, the B operand carries column l%16, and the D tile of lane l
// holds rows 4*(l/16)+i, i<4, of column l%16. The contraction index is free to permute as
// long as A and B agree, so every k-block of 32 here uses the order
//   slot (g = l/16, j < 4) -> index 4g + j,  slot (g, j >= 4) -> index 16 + 4g + (j - 4),
// which is exactly the set of rows a lane holds in two vertically stacked D tiles. A
// running state kept in accumulators therefore becomes a B operand with no data movement,
// and so does the attention tile A^T = K' Q'^T (rows = keys) as the A operand of A V.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "rla2_internal.h"

namespace rla2 {
namespace {

typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float float2v __attribute__((ext_vector_type(2)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef short i16x2 __attribute__((ext_vector_type(2)));
constexpr int kBufFlags = 0x00020000;  // gfx9 buffer resource word 3 (32-bit raw data)
// Cache policy of the streaming input loads and output stores (the slc bit: each byte is
// touched once per kernel). Measured on the long-context forward: it keeps the segment
// records and the reused small tables resident and speeds up every forward kernel.
constexpr int kLoadStream = 2;

constexpr int NT = 256;  // threads per workgroup of the chunk kernels

// ----------------------------------------------------------------------------------------
// element helpers

__device__ __forceinline__ float bf2f(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

__device__ __forceinline__ uint16_t f2bf(float f) {  // round to nearest even
  return __builtin_bit_cast(uint16_t, static_cast<__bf16>(f));
}

// bf16 pair, round to nearest even
__device__ __forceinline__ uint32_t pack_bf2(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(float2v{a, b}, bf16x2));
}
// the two bf16 halves of a packed word as floats
__device__ __forceinline__ float bf_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

template <bool BF>
struct Elem;
template <>
struct Elem<true> {
  using St = uint16_t;
  __device__ static float to_f(St x) { return bf2f(x); }
  __device__ static St from_f(float x) { return f2bf(x); }
};
template <>
struct Elem<false> {
  using St = float;
  __device__ static float to_f(St x) { return x; }
  __device__ static St from_f(float x) { return x; }
};

// Copy N bytes between 4-byte-aligned locations with the widest vector moves that fit.
template <int N>
__device__ __forceinline__ void copy_bytes(void* dst, const void* src) {
  static_assert(N % 4 == 0, "");
  if constexpr (N % 16 == 0) {
#pragma unroll
    for (int i = 0; i < N / 16; ++i)
      reinterpret_cast<uint4*>(dst)[i] = reinterpret_cast<const uint4*>(src)[i];
  } else if constexpr (N == 8) {
    *reinterpret_cast<uint2*>(dst) = *reinterpret_cast<const uint2*>(src);
  } else {
#pragma unroll
    for (int i = 0; i < N / 4; ++i)
      reinterpret_cast<uint32_t*>(dst)[i] = reinterpret_cast<const uint32_t*>(src)[i];
  }
}

// ----------------------------------------------------------------------------------------
// cross-lane sums on the VALU (DPP and the gfx950 lane-swap instructions), no LDS traffic

// Sum over each aligned group of 8 lanes, returned in all 8: quad_perm [1,0,3,2] and
// [2,3,0,1] add the lanes of a quad, row_half_mirror (lane i <- 7 - i) adds the other quad.
__device__ __forceinline__ float sum8(float x) {
  x += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0xB1, 0xF, 0xF, false));
  x += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x4E, 0xF, 0xF, false));
  x += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x141, 0xF, 0xF, false));
  return x;
}

// Sum of lanes l, l ^ 16, l ^ 32, l ^ 48 (the four 16-lane rows), returned in all of them.
// Swapping row pairs of a value with itself yields one copy of each row of the pair in the
// two results, so their sum is the pair sum in every lane; rows 16 apart first, then halves.
__device__ __forceinline__ float sum_rows4(float x) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_int(x), __float_as_int(x), false, false);
  x = __int_as_float(a[0]) + __int_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_int(x), __float_as_int(x), false, false);
  return __int_as_float(b[0]) + __int_as_float(b[1]);
}

// ----------------------------------------------------------------------------------------
// geometry of the chunk kernels for head dim D and element type

template <bool BF, int D>
struct Geo {
  using St = typename Elem<BF>::St;
  static constexpr int ES = sizeof(St);
  static constexpr int HALF = D / 2;
  static constexpr int E = D / 16;     // dims per lane in each RoPE half (8 lanes per token)
  static constexpr int ROWP = D + (BF ? 8 : 4);   // pitch (elements) of row-major [token][dim]
  static constexpr int COLP = kChunk + (BF ? 8 : 4);  // pitch of transposed [dim][token]
  static constexpr int NW = (D / 16 < 4) ? D / 16 : 4;  // waves that own state columns
  static constexpr int DVW = D / NW;   // value columns per such wave
  static constexpr int CT = DVW / 16;  // 16-wide column tiles per wave
  static constexpr int RT = D / 16;    // 16-high row tiles of the state
  static constexpr int KB = D / 32;    // 32-wide k-blocks over the head dim
  static_assert(E >= 2 && E % 2 == 0 && (E * ES) % 4 == 0, "");
};

// One MFMA k-block of 32 contraction indices, in the slot order described at the top.
template <bool BF>
struct Frag;
template <>
struct Frag<true> {
  bf16x8 v;
};
template <>
struct alignas(16) Frag<false> {
  float v[8];
};

__device__ __forceinline__ floatx4 mma(const Frag<true>& a, const Frag<true>& b, floatx4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a.v, b.v, c, 0, 0, 0);
}
__device__ __forceinline__ floatx4 mma(const Frag<false>& a, const Frag<false>& b, floatx4 c) {
#pragma unroll
  for (int j = 0; j < 8; ++j) c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.v[j], b.v[j], c, 0, 0, 0);
  return c;
}

// Fragment of row `row` of an LDS array with element pitch `pitch`, k-block `kb`:
// elements kb*32 + 4g + {0..3} and kb*32 + 16 + 4g + {0..3}.
template <bool BF>
__device__ __forceinline__ Frag<BF> lds_frag(const typename Elem<BF>::St* base, int pitch, int row,
                                             int kb, int g) {
  using St = typename Elem<BF>::St;
  Frag<BF> f;
  const St* p = base + row * pitch + kb * 32 + 4 * g;
  copy_bytes<4 * sizeof(St)>(&f.v, p);
  copy_bytes<4 * sizeof(St)>(reinterpret_cast<char*>(&f.v) + 4 * sizeof(St), p + 16);
  return f;
}

// The same slot order with the contraction running down the rows of a row-major bf16 LDS
// array [k][n] (pitch in elements): lane (c16, g) gets elements [k0 + 4g + j][n0 + c16] and
// [k0 + 16 + 4g + j][n0 + c16], j < 4. gfx950's transposing LDS read (ds_read_b64_tr_b16)
// hands destination lane l of each 16-lane group element j of the 8 bytes read by source
// lane 4j + l/4 at position l%4; so source lane s of group g points at row k0 + 4g + s/4,
// columns n0 + 4(s%4) .. +3, and one read per half gives the whole fragment.
__device__ __forceinline__ Frag<true> lds_frag_tr(const uint16_t* base, int pitch, int k0, int n0, int lane) {
  typedef short v4i16 __attribute__((ext_vector_type(4)));
  typedef __attribute__((address_space(3))) v4i16 lds_v4i16;
  const int c16 = lane & 15, g = lane >> 4;
  const uint16_t* p = base + (k0 + 4 * g + (c16 >> 2)) * pitch + n0 + 4 * (c16 & 3);
  const v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(p));
  const v4i16 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(p + 16 * pitch));
  Frag<true> f;
  typedef short v8i16 __attribute__((ext_vector_type(8)));
  const v8i16 w = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  f.v = __builtin_bit_cast(bf16x8, w);
  return f;
}

// Row fragment in the contiguous slot order: lane (c16, g) gets elements [row][32 kb + 8g + j],
// j < 8, in one 16-byte read. Both operands of a contraction must use the same slot order;
// for accumulator-born operands this is arranged by the tile-to-dim map of the accumulators.
__device__ __forceinline__ Frag<true> lds_frag_c(const uint16_t* base, int pitch, int row, int kb, int g) {
  Frag<true> f;
  copy_bytes<16>(&f.v, base + row * pitch + kb * 32 + 8 * g);
  return f;
}

// lds_frag_tr for the contiguous slot order: the 16 operand rows are columns c0 + 8a + b
// (row 4a + b, a, b < 4) of the row-major array, so an accumulator tile built from it holds,
// in lane (c, g), the columns c0 + 8g + i. Tiles c0 = 32 kb and c0 = 32 kb + 4 then pair up
// (acc_frag) into a contiguous-order operand over columns 32 kb .. 32 kb + 31.
__device__ __forceinline__ Frag<true> lds_frag_tr_s8(const uint16_t* base, int pitch, int k0, int c0, int lane) {
  typedef short v4i16 __attribute__((ext_vector_type(4)));
  typedef __attribute__((address_space(3))) v4i16 lds_v4i16;
  const int c16 = lane & 15, g = lane >> 4;
  const uint16_t* p = base + (k0 + 4 * g + (c16 >> 2)) * pitch + c0 + 8 * (c16 & 3);
  const v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(p));
  const v4i16 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(p + 16 * pitch));
  Frag<true> f;
  typedef short v8i16 __attribute__((ext_vector_type(8)));
  const v8i16 w = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  f.v = __builtin_bit_cast(bf16x8, w);
  return f;
}

// Operand whose every element is 1 (against it, K'^T gives the column sums of K').
template <bool BF>
__device__ __forceinline__ Frag<BF> ones_frag() {
  Frag<BF> f;
  if constexpr (BF) {
#pragma unroll
    for (int j = 0; j < 8; ++j) f.v[j] = static_cast<__bf16>(1.0f);
  } else {
#pragma unroll
    for (int j = 0; j < 8; ++j) f.v[j] = 1.0f;
  }
  return f;
}

// Fragment from two vertically stacked accumulator tiles (rows 0..15 and 16..31 of a block).
__device__ __forceinline__ Frag<true> acc_frag_bf(floatx4 lo, floatx4 hi) {
  Frag<true> f;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    f.v[j] = static_cast<__bf16>(lo[j]);
    f.v[4 + j] = static_cast<__bf16>(hi[j]);
  }
  return f;
}
__device__ __forceinline__ Frag<false> acc_frag_f(floatx4 lo, floatx4 hi) {
  Frag<false> f;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    f.v[j] = lo[j];
    f.v[4 + j] = hi[j];
  }
  return f;
}
template <bool BF>
__device__ __forceinline__ Frag<BF> acc_frag(floatx4 lo, floatx4 hi) {
  if constexpr (BF) return acc_frag_bf(lo, hi);
  else return acc_frag_f(lo, hi);
}

// ----------------------------------------------------------------------------------------
// feature map of a token pair in the chunk kernels
//
// Lane mapping (256 threads, 64 tokens): lane l owns tokens t0 = 2*(l/8), t0 + 1 and, in each
// RoPE half h, the E dims [h*D/2 + (l%8)*E, +E). Rotate-half RoPE pairs dim j with j + D/2,
// so both partners of every pair sit in the same lane; the RMS statistic is a sum over the 8
// lanes of a token (xor-shuffles 1, 2, 4).

template <bool BF, int D>
struct Raw {  // one tensor's elements for the lane's two tokens, packed in 32-bit words
  static constexpr int W = Geo<BF, D>::E * Geo<BF, D>::ES / 4;  // words per (token, half)
  alignas(16) uint32_t w[2][2][W];
  __device__ __forceinline__ float get(int tok, int h, int e) const {
    if constexpr (BF) return __uint_as_float(e & 1 ? (w[tok][h][e >> 1] & 0xffff0000u) : (w[tok][h][e >> 1] << 16));
    else return __uint_as_float(w[tok][h][e]);
  }
  __device__ __forceinline__ uint32_t bits(int tok, int h, int e) const {  // raw element bits
    if constexpr (BF) return e & 1 ? (w[tok][h][e >> 1] >> 16) : (w[tok][h][e >> 1] & 0xffffu);
    else return w[tok][h][e];
  }
};

template <bool BF, int D>
__device__ __forceinline__ void load_raw(Raw<BF, D>& r, const typename Elem<BF>::St* chunk_base,
                                         int t0, int m, int nvalid) {
  using G = Geo<BF, D>;
#pragma unroll
  for (int tok = 0; tok < 2; ++tok) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      if (t0 + tok < nvalid) {
        copy_bytes<G::E * G::ES>(r.w[tok][h], chunk_base + (size_t)(t0 + tok) * D + h * G::HALF + m * G::E);
      } else {
#pragma unroll
        for (int i = 0; i < Raw<BF, D>::W; ++i) r.w[tok][h][i] = 0u;
      }
    }
  }
}

// Feature-map arithmetic shared by every chunk kernel, so q' and k' are bitwise the same
// wherever they are formed.
//
// 1/sqrt(mean(x^2) + rms_eps) of token `tok`: the lane's 2E elements plus the other 7 lanes
// of the token (xor-shuffles 1, 2, 4).
template <bool BF, int D>
__device__ __forceinline__ float rms_inv(const Raw<BF, D>& r, int tok, float rms_eps) {
  using G = Geo<BF, D>;
  float ss = 0.f;
  if constexpr (BF) {  // bf16 products are exact in fp32: two squares per dot instruction
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int i = 0; i < Raw<BF, D>::W; ++i) {
        const bf16x2 x = __builtin_bit_cast(bf16x2, r.w[tok][h][i]);
        ss = __builtin_amdgcn_fdot2_f32_bf16(x, x, ss, false);
      }
  } else {
#pragma unroll
    for (int e = 0; e < G::E; ++e) {
      const float a = r.get(tok, 0, e), b = r.get(tok, 1, e);
      ss += a * a;
      ss += b * b;
    }
  }
  ss = sum8(ss);
  return rsqrtf(__builtin_fmaf(ss, 1.0f / D, rms_eps));
}

// The feature-map arithmetic below is written with explicit fused multiply-adds and no
// implicit contraction, so every kernel that forms q' or k' rounds identically.
//
// (cos, sin) of A + B from (cos A, sin A) and (cos B, sin B).
__device__ __forceinline__ float2 angle_sum(float2 a, float2 b) {
#pragma clang fp contract(off)
  return make_float2(__builtin_fmaf(a.x, b.x, -(a.y * b.y)), __builtin_fmaf(a.y, b.x, a.x * b.y));
}

// One rotate-half pair (x1 = dim j, x2 = dim j + D/2): y = x * inv * gamma, rotated by the
// angle with (cos, sin) = cs. The ReLU follows in put_pairs.
__device__ __forceinline__ void rope_pair(float x1, float x2, float inv, float g1, float g2, float2 cs,
                                          float& u1, float& u2) {
#pragma clang fp contract(off)
  const float y1 = (x1 * inv) * g1;
  const float y2 = (x2 * inv) * g2;
  u1 = __builtin_fmaf(y1, cs.x, -(y2 * cs.y));
  u2 = __builtin_fmaf(y2, cs.x, y1 * cs.y);
}

// ReLU of elements e, e + 1 of both halves of token `tok` (u?[0] at e, u?[1] at e + 1),
// rounded to the element type, into `o`. bf16: two values per RNE conversion, then the ReLU
// on the packed pair as a 16-bit signed max with 0 (a bf16 value is negative exactly when
// its sign bit is set, and rounding never changes a sign, so this equals rounding max(u, 0)).
template <bool BF, int D>
__device__ __forceinline__ void put_pairs(Raw<BF, D>& o, int tok, int e, const float (&u1)[2],
                                          const float (&u2)[2]) {
  if constexpr (BF) {
    const i16x2 zero = i16x2{0, 0};
    o.w[tok][0][e >> 1] = __builtin_bit_cast(
        uint32_t, __builtin_elementwise_max(__builtin_bit_cast(i16x2, __builtin_convertvector(float2v{u1[0], u1[1]}, bf16x2)), zero));
    o.w[tok][1][e >> 1] = __builtin_bit_cast(
        uint32_t, __builtin_elementwise_max(__builtin_bit_cast(i16x2, __builtin_convertvector(float2v{u2[0], u2[1]}, bf16x2)), zero));
  } else {
    o.w[tok][0][e] = __float_as_uint(fmaxf(u1[0], 0.f));
    o.w[tok][0][e + 1] = __float_as_uint(fmaxf(u1[1], 0.f));
    o.w[tok][1][e] = __float_as_uint(fmaxf(u2[0], 0.f));
    o.w[tok][1][e + 1] = __float_as_uint(fmaxf(u2[1], 0.f));
  }
}

// x' = ReLU(RoPE(RMSNorm(x))) rounded to the element type (result in `o`, same layout as raw).
// rope_lo: [64][D/2] float2 (cos, sin) of t*theta_j; rope_hi_row: the [D/2] row of 64*a*theta_j
// for the chunk's first position 64*a. The rotation angle of token t is 64*a*theta + t*theta.
template <bool BF, int D>
__device__ __forceinline__ void feature_map_pair(const Raw<BF, D>& r, Raw<BF, D>& o, const float* gamma,
                                                 const float2* rope_lo, const float2* rope_hi_row,
                                                 int t0, int m, float rms_eps) {
  using G = Geo<BF, D>;
#pragma unroll
  for (int tok = 0; tok < 2; ++tok) {
    const float inv = rms_inv<BF, D>(r, tok, rms_eps);
    const float2* lo = rope_lo + (t0 + tok) * G::HALF;
#pragma unroll
    for (int e = 0; e < G::E; e += 2) {
      float u1[2], u2[2];
#pragma unroll
      for (int x = 0; x < 2; ++x) {
        const int j = m * G::E + e + x;
        rope_pair(r.get(tok, 0, e + x), r.get(tok, 1, e + x), inv, gamma[j], gamma[j + G::HALF],
                  angle_sum(rope_hi_row[j], lo[j]), u1[x], u2[x]);
      }
      put_pairs<BF, D>(o, tok, e, u1, u2);
    }
  }
}

// load_raw through a buffer resource covering exactly the segment's tokens: reads past the
// segment's end return zeros without touching memory, so the load is issued
// unconditionally (a fixed number of loads per chunk keeps the wait counts exact).
// ONLY >= 0: that token of the pair alone.
template <bool BF, int D, int ONLY = -1>
__device__ __forceinline__ void load_raw_buf(Raw<BF, D>& r, __amdgpu_buffer_rsrc_t rs, int tok, int m) {
  using G = Geo<BF, D>;
  constexpr int NB = G::E * G::ES;  // bytes per (token, half) of this lane
#pragma unroll
  for (int t = 0; t < 2; ++t)
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      if (ONLY >= 0 && t != ONLY) continue;
      const int off = ((tok + t) * D + hh * G::HALF + m * G::E) * G::ES;
      if constexpr (NB >= 16) {
#pragma unroll
        for (int p = 0; p < NB / 16; ++p) {
          const u32x4 x = __builtin_amdgcn_raw_buffer_load_b128(rs, off + 16 * p, 0, kLoadStream);
#pragma unroll
          for (int i = 0; i < 4; ++i) r.w[t][hh][4 * p + i] = x[i];
        }
      } else if constexpr (NB == 8) {
        const u32x2 x = __builtin_amdgcn_raw_buffer_load_b64(rs, off, 0, kLoadStream);
        r.w[t][hh][0] = x[0];
        r.w[t][hh][1] = x[1];
      } else {
        r.w[t][hh][0] = __builtin_amdgcn_raw_buffer_load_b32(rs, off, 0, kLoadStream);
      }
    }
}

// Per-segment state record: d*d + d floats. S is stored fragment-native: the 4 accumulator
// values lane l of state wave w holds in tile (rt, ct) are contiguous, at
//   rec_frag(w, rt, ct, l) = (((w * RT + rt) * CT + ct) * 64 + l) * 4,
// which is S[16 rt + 4 (l / 16) + i][w * DVW + 16 ct + l % 16], i < 4; z follows at d*d.
// Writers and readers move 16 bytes per lane; only the final-state export permutes.
template <bool BF, int D>
__device__ __forceinline__ int rec_frag(int w, int rt, int ct, int l) {
  using G = Geo<BF, D>;
  return (((w * G::RT + rt) * G::CT + ct) * 64 + l) * 4;
}

// The record read into the contiguous-order tile map (lds_frag_tr_s8): in tile pt, lane (c, g)
// row i holds dim 32 (pt / 2) + 8g + 4 (pt % 2) + i, which the record keeps in tile
// 2 (pt / 2) + g / 2 at lane (c, 2 (g % 2) + pt % 2), row i.
template <int D>
__device__ __forceinline__ int rec_frag_c(int w, int pt, int ct, int lane) {
  const int c16 = lane & 15, g = lane >> 4;
  return rec_frag<true, D>(w, 2 * (pt / 2) + g / 2, ct, 16 * (2 * (g % 2) + pt % 2) + c16);
}

// The same map with every per-lane constant in registers: g1[e], g2[e] = gamma of dims
// j, j + D/2 (j = m*E + e); lo[tok][e] = (cos, sin) of (t0 + tok)*theta_j; hi[e] = (cos, sin)
// of 64*a*theta_j for the chunk's first position 64*a.
template <bool BF, int D, int ONLY = -1>  // ONLY >= 0: that token of the pair alone
__device__ __forceinline__ void feature_map_lane(const Raw<BF, D>& r, Raw<BF, D>& o, const float (&g1)[Geo<BF, D>::E],
                                                 const float (&g2)[Geo<BF, D>::E],
                                                 const float2 (&lo)[2][Geo<BF, D>::E],
                                                 const float2 (&hi)[Geo<BF, D>::E], float rms_eps) {
  using G = Geo<BF, D>;
#pragma unroll
  for (int tok = 0; tok < 2; ++tok) {
    if (ONLY >= 0 && tok != ONLY) continue;
    const float inv = rms_inv<BF, D>(r, tok, rms_eps);
#pragma unroll
    for (int e = 0; e < G::E; e += 2) {
      float u1[2], u2[2];
#pragma unroll
      for (int x = 0; x < 2; ++x)
        rope_pair(r.get(tok, 0, e + x), r.get(tok, 1, e + x), inv, g1[e + x], g2[e + x],
                  angle_sum(hi[e + x], lo[tok][e + x]), u1[x], u2[x]);
      put_pairs<BF, D>(o, tok, e, u1, u2);
    }
  }
}

// q' and k' of the same two tokens: one angle per (token, pair) serves both.
template <bool BF, int D>
__device__ __forceinline__ void feature_map_qk(const Raw<BF, D>& rq, const Raw<BF, D>& rk, Raw<BF, D>& oq,
                                               Raw<BF, D>& ok, const float* gq, const float* gk,
                                               const float2* rope_lo, const float2* rope_hi_row, int t0, int m,
                                               float rms_eps) {
  using G = Geo<BF, D>;
#pragma unroll
  for (int tok = 0; tok < 2; ++tok) {
    const float invq = rms_inv<BF, D>(rq, tok, rms_eps);
    const float invk = rms_inv<BF, D>(rk, tok, rms_eps);
    const float2* lo = rope_lo + (t0 + tok) * G::HALF;
#pragma unroll
    for (int e = 0; e < G::E; e += 2) {
      float q1[2], q2[2], k1[2], k2[2];
#pragma unroll
      for (int x = 0; x < 2; ++x) {
        const int j = m * G::E + e + x;
        const float2 cs = angle_sum(rope_hi_row[j], lo[j]);
        rope_pair(rq.get(tok, 0, e + x), rq.get(tok, 1, e + x), invq, gq[j], gq[j + G::HALF], cs, q1[x], q2[x]);
        rope_pair(rk.get(tok, 0, e + x), rk.get(tok, 1, e + x), invk, gk[j], gk[j + G::HALF], cs, k1[x], k2[x]);
      }
      put_pairs<BF, D>(oq, tok, e, q1, q2);
      put_pairs<BF, D>(ok, tok, e, k1, k2);
    }
  }
}

// Store a lane's pair tokens row-major into [64][ROWP].
template <bool BF, int D, int ONLY = -1>
__device__ __forceinline__ void store_rows(typename Elem<BF>::St* dst, const Raw<BF, D>& o, int t0, int m,
                                           int pitch = Geo<BF, D>::ROWP) {
  using G = Geo<BF, D>;
#pragma unroll
  for (int tok = 0; tok < 2; ++tok)
#pragma unroll
    for (int h = 0; h < 2; ++h)
      if (ONLY < 0 || tok == ONLY) copy_bytes<G::E * G::ES>(dst + (t0 + tok) * pitch + h * G::HALF + m * G::E, o.w[tok][h]);
}

// Store a lane's pair tokens transposed into [D][COLP]: one 2-token word per dim.
template <bool BF, int D>
__device__ __forceinline__ void store_cols(typename Elem<BF>::St* dst, const Raw<BF, D>& o, int t0, int m) {
  using G = Geo<BF, D>;
#pragma unroll
  for (int h = 0; h < 2; ++h)
#pragma unroll
    for (int e = 0; e < G::E; ++e) {
      const int dim = h * G::HALF + m * G::E + e;
      if constexpr (BF) {
        const uint32_t w = o.bits(0, h, e) | (o.bits(1, h, e) << 16);
        *reinterpret_cast<uint32_t*>(dst + dim * G::COLP + t0) = w;
      } else {
        *reinterpret_cast<uint2*>(dst + dim * G::COLP + t0) = make_uint2(o.bits(0, h, e), o.bits(1, h, e));
      }
    }
}

// Arrival counter of the four MMA waves of a warp-specialised kernel: each wave adds 1 with
// release semantics (its LDS writes land first), then polls with acquire semantics until the
// count reaches `target` (all four have arrived at this meeting: the count only grows, so the
// n-th meeting waits for 4 n). The poll is bounded (`polls` rounds, tens of milliseconds at
// the default) so that a wave can never spin forever; a wave that gives up records it in the
// workspace header (HDR_WAIT, a plain vector store from lane 0) and goes on, so the kernel
// still ends normally and the host can tell that the call's outputs are not valid.
__device__ __forceinline__ void mma_wave_sync(unsigned* cnt, unsigned target, int lane, uint32_t polls,
                                              uint32_t* hdr) {
  if (lane == 0) __hip_atomic_fetch_add(cnt, 1u, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);
  for (uint32_t spin = 0; spin < polls; ++spin) {
    if (__hip_atomic_load(cnt, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_WORKGROUP) >= target) return;
    __builtin_amdgcn_s_sleep(1);
  }
  if (__hip_atomic_load(cnt, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_WORKGROUP) >= target) return;
  if (lane == 0) hdr[HDR_WAIT] = 1u;
}

// The other side of a hand-over counter: a wave that only waits (it does not arrive) until the
// count reaches `target`, with the same bounded poll and the same record in the header when
// the bound runs out. The waves that hand over add to the counter with release semantics after
// their last access to the memory being handed over.
__device__ __forceinline__ void wait_count(unsigned* cnt, unsigned target, int lane, uint32_t polls, uint32_t* hdr) {
  for (uint32_t spin = 0; spin < polls; ++spin) {
    if (__hip_atomic_load(cnt, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_WORKGROUP) >= target) return;
    __builtin_amdgcn_s_sleep(1);
  }
  if (__hip_atomic_load(cnt, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_WORKGROUP) >= target) return;
  if (lane == 0) hdr[HDR_WAIT] = 1u;
}

// Checksum of cu_seqlens[0 .. n_docs] (0 without cu_seqlens) for the plan stamp: a wrapping
// sum of one mixed word per entry, so every thread order gives the same value. Called by all
// threads of a 1024-thread workgroup; every thread gets the result.
__device__ __forceinline__ uint32_t cu_mix(uint32_t j, uint32_t x) {
  uint32_t h = x * 0x9E3779B1u + j * 0x85EBCA77u + 0x165667B1u;
  h ^= h >> 15;
  h *= 0x2C1B3C6Du;
  h ^= h >> 12;
  return h;
}

__device__ __forceinline__ uint32_t cu_checksum_block(const int32_t* __restrict__ cu, int n_docs) {
  __shared__ uint32_t red[1024];
  const int tid = threadIdx.x;
  uint32_t acc = 0u;
  if (cu != nullptr)
    for (int j = tid; j <= n_docs; j += 1024) acc += cu_mix((uint32_t)j, (uint32_t)cu[j]);
  red[tid] = acc;
  __syncthreads();
  for (int off = 512; off > 0; off >>= 1) {
    if (tid < off) red[tid] += red[tid + off];
    __syncthreads();
  }
  const uint32_t total = red[0];
  __syncthreads();
  return total;
}

// The backward kernels' entry check: run only when the set-up launch of the call cleared them
// to (HDR_GO of the backward's own workspace).
__device__ __forceinline__ bool bwd_go(const uint32_t* hdr) { return hdr[HDR_GO] != 0u; }

struct SegInfo {
  int row, start, len, pos0;
  int hirow;  // RoPE chunk row of the segment's first chunk
};

__device__ __forceinline__ SegInfo read_seg(const int32_t* tab, int seg) {
  const int4 a = *reinterpret_cast<const int4*>(tab + (size_t)seg * kTabInts);
  return SegInfo{a.x, a.y, a.z, a.w, tab[(size_t)seg * kTabInts + TAB_HIROW]};
}

// read_seg for a table that another call wrote (the backward reading a forward's workspace):
// every field is clamped into the plan's ranges (row < rows, start + len <= L, len <= seg_len,
// the segment's RoPE rows within the n_rope rows of the table), so even a corrupted table can
// only give wrong numbers, never an access outside the tensors or the tables.
struct TabLimits {
  int rows;     // batch rows of the tensors (1 when packed)
  int seg_len;  // tokens per segment at most
  int n_rope;   // rows of the coarse RoPE table
};

__device__ __forceinline__ SegInfo read_seg_clamped(const int32_t* tab, int seg, int L, TabLimits lim) {
  SegInfo si = read_seg(tab, seg);
  si.row = min(max(si.row, 0), lim.rows - 1);
  si.start = min(max(si.start, 0), L);
  si.len = min(max(si.len, 0), min(lim.seg_len, L - si.start));
  si.pos0 = max(si.pos0, 0);
  const int nch = (si.len + kChunk - 1) / kChunk;
  si.hirow = min(max(si.hirow, 0), max(lim.n_rope - nch, 0));
  return si;
}

template <bool BF, int D, int ONLY = -1>  // ONLY >= 0: that token of the pair alone
__device__ __forceinline__ void store_raw_buf(const Raw<BF, D>& r, __amdgpu_buffer_rsrc_t rs, int tok, int m) {
  using G = Geo<BF, D>;
  constexpr int NB = G::E * G::ES;  // bytes per (token, half) of this lane
#pragma unroll
  for (int t = 0; t < 2; ++t)
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      if (ONLY >= 0 && t != ONLY) continue;
      const int off = ((tok + t) * D + hh * G::HALF + m * G::E) * G::ES;
      if constexpr (NB >= 16) {
#pragma unroll
        for (int p = 0; p < NB / 16; ++p)
          __builtin_amdgcn_raw_buffer_store_b128(
              u32x4{r.w[t][hh][4 * p], r.w[t][hh][4 * p + 1], r.w[t][hh][4 * p + 2], r.w[t][hh][4 * p + 3]}, rs,
              off + 16 * p, 0, kLoadStream);
      } else if constexpr (NB == 8) {
        __builtin_amdgcn_raw_buffer_store_b64(u32x2{r.w[t][hh][0], r.w[t][hh][1]}, rs, off, 0, kLoadStream);
      } else {
        __builtin_amdgcn_raw_buffer_store_b32(r.w[t][hh][0], rs, off, 0, kLoadStream);
      }
    }
}

// ----------------------------------------------------------------------------------------
// Token-split tiles for kernels in which a token's result depends only on its own rows and on
// document states that do not change along the sweep (here the bidirectional read-out with the
// L2 denominator). A wave takes 16 tokens; lane (t = l % 16, g = l / 16) holds
// token t's dims 32 kb + 8g + j, j < 8, of every k-block kb < d/32. That set is at once
//  - the B-operand slots of the token's row in k-block kb (slot j = contraction index 8g + j),
//  - the rows the lane receives in the output tiles 2p, 2p + 1 of a product whose tile 2p + h,
//    row 4g + i stands for dim 32 p + 8g + 4h + i (so output dims 32 p + 8g .. + 7 are one
//    16-byte piece of the token's row),
//  - closed under the rotate-half pairing for d >= 64 (dims a and a + d/2 sit in k-blocks kb and
//    kb + d/64 of the same lane),
// so a token goes from its raw row to its stored result in the lane's registers; a per-token
// reduction is a sum over the four lanes t + 16g (sum_rows4). The constant states enter as
// A-operand fragments in LDS, built once per workgroup from the record (ql_operands).

template <int D>
struct QL {
  static_assert(D >= 64 && D % 64 == 0, "rotate-half pairs must stay in the lane");
  static constexpr int KB = D / 32;  // k-blocks: 16-byte pieces of a lane's part of a row
  static constexpr int NP = KB / 2;  // k-blocks of the first RoPE half
  static constexpr int R = D / 16;   // 16-dim output tiles
};

// Raw row piece of token `tok` (segment-relative) through a range-checked buffer resource:
// tokens past the segment read zeros.
template <int D>
__device__ __forceinline__ void ql_load(u32x4 (&x)[D / 32], __amdgpu_buffer_rsrc_t rs, int tok, int g) {
#pragma unroll
  for (int kb = 0; kb < D / 32; ++kb)
    x[kb] = __builtin_amdgcn_raw_buffer_load_b128(rs, (tok * D + 32 * kb + 8 * g) * 2, 0, kLoadStream);
}

// element j < 8 of a 16-byte bf16 piece
__device__ __forceinline__ float ql_elem(const u32x4& x, int j) {
  return __uint_as_float(j & 1 ? (x[j >> 1] & 0xffff0000u) : (x[j >> 1] << 16));
}

// 1/rms of the token (the four lanes of the token together)
template <int D>
__device__ __forceinline__ float ql_rms_inv(const u32x4 (&x)[D / 32], float rms_eps) {
  float part[4] = {0.f, 0.f, 0.f, 0.f};  // four independent chains
#pragma unroll
  for (int kb = 0; kb < D / 32; ++kb)
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      // through a scalar: a bit cast applied to the vector element itself compiled to element
      // 0 for every w (hipcc 7.2)
      const uint32_t word = x[kb][w];
      const bf16x2 p = __builtin_bit_cast(bf16x2, word);
      part[w] = __builtin_amdgcn_fdot2_f32_bf16(p, p, part[w], false);
    }
  float ss = (part[0] + part[1]) + (part[2] + part[3]);
  ss = sum_rows4(ss);
  return rsqrtf(__builtin_fmaf(ss, 1.0f / D, rms_eps));
}

// x' = ReLU(RoPE(RMSNorm(x))) of the lane's dims, rounded to bf16, as B-operand fragments;
// gam[kb][j] = gamma of dim 32 kb + 8g + j, cs[kb][j] (kb < d/64) = (cos, sin) of the token's
// angle for the pair (32 kb + 8g + j, + d/2). The arithmetic is the chunk kernels' (rope_pair,
// then ReLU of the RNE rounding as a 16-bit signed max).
template <int D>
__device__ __forceinline__ void ql_map(const u32x4 (&x)[D / 32], float inv, const float (&gam)[D / 32][8],
                                       const float2 (&cs)[D / 64][8], Frag<true> (&xf)[D / 32]) {
  constexpr int NP = D / 64;
  const i16x2 zero = i16x2{0, 0};
#pragma unroll
  for (int kb = 0; kb < NP; ++kb) {
    u32x4 w1, w2;
#pragma unroll
    for (int j = 0; j < 8; j += 2) {
      float u1[2], u2[2];
#pragma unroll
      for (int y = 0; y < 2; ++y)
        rope_pair(ql_elem(x[kb], j + y), ql_elem(x[kb + NP], j + y), inv, gam[kb][j + y], gam[kb + NP][j + y],
                  cs[kb][j + y], u1[y], u2[y]);
      w1[j >> 1] = __builtin_bit_cast(
          uint32_t, __builtin_elementwise_max(__builtin_bit_cast(i16x2, __builtin_convertvector(float2v{u1[0], u1[1]}, bf16x2)), zero));
      w2[j >> 1] = __builtin_bit_cast(
          uint32_t, __builtin_elementwise_max(__builtin_bit_cast(i16x2, __builtin_convertvector(float2v{u2[0], u2[1]}, bf16x2)), zero));
    }
    xf[kb].v = __builtin_bit_cast(bf16x8, w1);
    xf[kb + NP].v = __builtin_bit_cast(bf16x8, w2);
  }
}

// A-operand fragments of a d x d record state M (fragment-native, rec_frag) for products
// over token-split tiles, written to LDS as [tile T][k-block kb][lane] 16-byte fragments
// (8 bf16 each). TRANS: the operand is M^T (its rows are M's columns, the contraction runs
// over M's rows), else M. Each element is rounded to bf16 into `hi` and, when `lo` is given,
// the rest (element - hi) rounded to bf16 into `lo`, so hi + lo carries ~16 significant bits.
// Operand row r lands in tile 2 (r / 32) + (r / 4) % 2, row 4 ((r % 32) / 8) + r % 4 (the output
// dims of the tiles above); contraction index c in k-block c / 32, slot 8 ((c % 32) / 8) + c % 8.
template <int D, bool TRANS>
__device__ __forceinline__ void ql_operands(uint16_t* hi, uint16_t* lo, const float* rec, int tid, int nthr) {
  using G = Geo<true, D>;
  constexpr int KB = D / 32;
  for (int e = tid; e < D * D; e += nthr) {
    const int i = e & 3, l = (e >> 2) & 63;
    int rest = e >> 8;
    const int ct = rest % G::CT;
    rest /= G::CT;
    const int rt = rest % G::RT, w = rest / G::RT;
    const int a = 16 * rt + 4 * (l >> 4) + i, v = w * G::DVW + 16 * ct + (l & 15);
    const int r = TRANS ? v : a, c = TRANS ? a : v;
    const int T = 2 * (r >> 5) + ((r >> 2) & 1), m = 4 * ((r & 31) >> 3) + (r & 3);
    const int idx = ((T * KB + (c >> 5)) * 64 + 16 * ((c & 31) >> 3) + m) * 8 + (c & 7);
    const float x = rec[e];
    const uint16_t hb = f2bf(x);
    hi[idx] = hb;
    if (lo != nullptr) lo[idx] = f2bf(x - bf2f(hb));
  }
}

}  // namespace
}  // namespace rla2
