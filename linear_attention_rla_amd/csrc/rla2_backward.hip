// HIP kernels of the RLA-2 causal backward on gfx950 (bf16 activations, fp32 states).
//
// Method: neuralnet.cpp development page "线性注意力家族：RLA / RAPT / RLA-2 与 GPU 落地"
// (the RLA page), §4.2 backward of the layer. With g_t = dL/dout_t, den_t = q'_t . z_t + eps,
// num_t = S_t^T q'_t and the page's gnum_t = g_t / den_t, scale_t = gd_t = -(g_t . num_t) / den_t^2:
//   dq'_t = S_t gnum_t + gd_t z_t                                  (forward states S_t, z_t)
//   dk'_i = P_i v_i + p_i,   dv_i = P_i^T k'_i                     (reverse states, same document)
//   P_i = sum_{t >= i} q'_t gnum_t^T = sum_{t >= i} (q'_t / den_t) g_t^T
//   p_i = sum_{t >= i} gd_t q'_t     = sum_{t >= i} (q'_t / den_t) (gd_t den_t)
// then through the ReLU (gate q' > 0), the inverse RoPE rotation and the RMSNorm backward
// to dq, dk and the RMSNorm weight gradients; dv needs no map.
//
// Numerics. g_t . num_t is formed in fp32 from the states and the chunk's scores (no rounded
// forward output is read). The weight of a query on its own key, B_tt = g_t . v_t / den_t +
// gd_t, is formed as (g_t . v_t (den_t - s_tt) - (g_t . num_t - s_tt g_t . v_t)) / den_t^2
// with both brackets summed without the self term, so a token that sees only itself (the
// first token of a document without an initial state, den - s_tt = eps) keeps its eps-sized
// gradient instead of the rounding noise of two cancelling O(1) terms. The running states
// enter the MFMA as a pair of bf16 operands (the rounded value and the rounded remainder);
// the reverse states are built from Q^ = bf16(q'/den) against the exact bf16 g and the fp32
// gd den, so P v_i and p_i share one rounding of each query.
//
// Chunked like the forward (C = 64 tokens, documents cut into segments of whole chunks):
//   (forward state pass)  prefix records of S, z per (segment, head)
//   bwd_dq_ws    per (segment, head), 32-token steps in order, S and z running (warp-
//                specialised: mappers for q', k' and for the map backward, MMA waves between):
//                  A^T = mask(K' Q'^T), Bv^T = V G^T (keys x queries), den, g . num, gd, B_tt
//                  dQ'^T = (S G^T) / den + z gd^T + K'^T B^T,  B^T = mask(Bv^T / den + gd) (B_tt on
//                  the diagonal); the map backward of q; den, gd and B_tt per token to memory
//   bwd_pstate   per (segment, head): sums of Q^^T G and Q^^T (gd den) over the segment
//   (suffix scan) exclusive sums over the later segments of each document
//   bwd_dkv_ws   per (segment, head), 32-token steps in reverse order, P and p running (warp-
//                specialised as bwd_dq_ws):
//                  A = mask(Q' K'^T), B = mask(G V^T / den + gd) (queries x keys, B_tt on the diagonal)
//                  dK'^T = P V^T + Q'^T B + p 1^T,  dV^T = P^T K'^T + G^T (A / den)
//                then the map backward of k
//   bwd_dgamma   sums the per-segment RMSNorm-weight partials
// Operand layout conventions are those of rla2_device.h. The running states live only in MFMA
// accumulators: an accumulator tile is at once an A operand whose rows are its columns and a
// B operand whose columns are its columns, both contracting over its rows, so a state held
// with the right orientation serves its products directly (the dk, dv sweep keeps P in both
// orientations, one per product); as operands they enter as a bf16 pair (value + remainder).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "rla2_device.h"
#include "rla2_internal.h"

namespace rla2 {
namespace {

// q'/den per token, rounded to bf16 (the query operand of the reverse states); inv = 1/den.
template <int D, int ONLY = -1>  // ONLY >= 0: that token of the pair alone
__device__ __forceinline__ void scale_raw(const Raw<true, D>& x, Raw<true, D>& o, const float (&inv)[2]) {
  constexpr int E = Geo<true, D>::E;
#pragma unroll
  for (int tok = 0; tok < 2; ++tok)
    if (ONLY < 0 || tok == ONLY)
#pragma unroll
    for (int hh = 0; hh < 2; ++hh)
#pragma unroll
      for (int e = 0; e < E; e += 2)
        o.w[tok][hh][e >> 1] = pack_bf2(x.get(tok, hh, e) * inv[tok], x.get(tok, hh, e + 1) * inv[tok]);
}

// Operand whose every column holds the per-token values w[32 kb + slot] (slot order of
// rla2_device.h), as a bf16 pair: hi = the rounded values, lo = the rounded remainders.
__device__ __forceinline__ void token_col_frags(const float* w, int kb, int g, Frag<true>& fhi, Frag<true>& flo) {
  const float* a = w + 32 * kb + 4 * g;
  const float* b = a + 16;
  const uint32_t h0 = pack_bf2(a[0], a[1]), h1 = pack_bf2(a[2], a[3]);
  const uint32_t h2 = pack_bf2(b[0], b[1]), h3 = pack_bf2(b[2], b[3]);
  fhi.v = __builtin_bit_cast(bf16x8, u32x4{h0, h1, h2, h3});
  flo.v = __builtin_bit_cast(bf16x8, u32x4{pack_bf2(a[0] - bf_lo(h0), a[1] - bf_hi(h0)),
                                           pack_bf2(a[2] - bf_lo(h1), a[3] - bf_hi(h1)),
                                           pack_bf2(b[0] - bf_lo(h2), b[1] - bf_hi(h2)),
                                           pack_bf2(b[2] - bf_lo(h3), b[3] - bf_hi(h3))});
}

// The lane's pair of tokens back from row-major [32][ROWP] LDS rows (the inverse of store_rows).
template <int D>
__device__ __forceinline__ void load_rows(const uint16_t* src, int t0, int m, Raw<true, D>& r) {
  using G = Geo<true, D>;
#pragma unroll
  for (int tok = 0; tok < 2; ++tok)
#pragma unroll
    for (int hh = 0; hh < 2; ++hh)
      copy_bytes<G::E * 2>(r.w[tok][hh], src + (t0 + tok) * G::ROWP + hh * G::HALF + m * G::E);
}

// one fp32 value per token from a [rows, H, L] plane (0 past the segment)
__device__ __forceinline__ float load_tok(__amdgpu_buffer_rsrc_t r, int tok) {
  return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, tok * 4, 0, 0));
}

// Map backward of the lane's two tokens (RMSNorm -> rotate-half RoPE -> ReLU, reversed):
// dx' from fp32 rows `dxp` ([64][FP]); the pre-activation is formed again exactly as the
// forward forms it, so the ReLU gate u > 0 matches the forward's q' > 0. Accumulates the
// RMSNorm-weight gradient of the lane's dims in dg1 (dims m E + e) and dg2 (+ D/2), and
// returns dx rounded to bf16 in the lane's raw layout.
template <int D>
__device__ __forceinline__ void map_backward(const Raw<true, D>& r, Raw<true, D>& dx, const float* dxp, int fp,
                                             const float (&g1)[Geo<true, D>::E], const float (&g2)[Geo<true, D>::E],
                                             const float2 (&lo)[2][Geo<true, D>::E],
                                             const float2 (&hi)[Geo<true, D>::E], float rms_eps, int t0, int m,
                                             float (&dg1)[Geo<true, D>::E], float (&dg2)[Geo<true, D>::E]) {
  using G = Geo<true, D>;
  constexpr int E = G::E;
#pragma unroll
  for (int tok = 0; tok < 2; ++tok) {
    // the lane's dx' values of both halves, read whole and gated below (a read behind the gate
    // compiles to one masked 4-byte read per value)
    float dp1[E], dp2[E];
    copy_bytes<E * 4>(dp1, dxp + (t0 + tok) * fp + m * E);
    copy_bytes<E * 4>(dp2, dxp + (t0 + tok) * fp + G::HALF + m * E);
    const float inv = rms_inv<true, D>(r, tok, rms_eps);
    float dy1[E], dy2[E];
    float T = 0.f;
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const float2 cs = angle_sum(hi[e], lo[tok][e]);
      const float x1 = r.get(tok, 0, e), x2 = r.get(tok, 1, e);
      float u1, u2;
      rope_pair(x1, x2, inv, g1[e], g2[e], cs, u1, u2);
      const float d1 = u1 > 0.f ? dp1[e] : 0.f;
      const float d2 = u2 > 0.f ? dp2[e] : 0.f;
      dy1[e] = __builtin_fmaf(d1, cs.x, d2 * cs.y);     // inverse rotation
      dy2[e] = __builtin_fmaf(d2, cs.x, -(d1 * cs.y));
      T = __builtin_fmaf(g1[e] * dy1[e], x1, T);
      T = __builtin_fmaf(g2[e] * dy2[e], x2, T);
      dg1[e] = __builtin_fmaf(dy1[e], x1 * inv, dg1[e]);
      dg2[e] = __builtin_fmaf(dy2[e], x2 * inv, dg2[e]);
    }
    T = sum8(T);
    const float coef = inv * inv * inv * T * (1.0f / D);
#pragma unroll
    for (int e = 0; e < E; e += 2) {
      const float a0 = __builtin_fmaf(inv * g1[e], dy1[e], -(coef * r.get(tok, 0, e)));
      const float a1 = __builtin_fmaf(inv * g1[e + 1], dy1[e + 1], -(coef * r.get(tok, 0, e + 1)));
      const float b0 = __builtin_fmaf(inv * g2[e], dy2[e], -(coef * r.get(tok, 1, e)));
      const float b1 = __builtin_fmaf(inv * g2[e + 1], dy2[e + 1], -(coef * r.get(tok, 1, e + 1)));
      dx.w[tok][0][e >> 1] = pack_bf2(a0, a1);
      dx.w[tok][1][e >> 1] = pack_bf2(b0, b1);
    }
  }
}


// map_backward with the forward mapper's results handed over: the ReLU gates of the lane's
// elements (gate[tok] bit 2e: dim m E + e, bit 2e + 1: its partner + D/2) and 1/rms of each
// token, as the forward mapper formed them for the same rows, so the pre-activation is not
// formed again; the arithmetic from the inverse rotation on is map_backward's, and so are the
// results, bit for bit.
template <int D>
__device__ __forceinline__ void map_backward_gated(const Raw<true, D>& r, Raw<true, D>& dx, const float* dxp, int fp,
                                                   const float (&g1)[Geo<true, D>::E], const float (&g2)[Geo<true, D>::E],
                                                   const float2 (&lo)[2][Geo<true, D>::E],
                                                   const float2 (&hi)[Geo<true, D>::E], const float (&invs)[2],
                                                   const uint32_t (&gate)[2], int t0, int m,
                                                   float (&dg1)[Geo<true, D>::E], float (&dg2)[Geo<true, D>::E]) {
  using G = Geo<true, D>;
  constexpr int E = G::E;
#pragma unroll
  for (int tok = 0; tok < 2; ++tok) {
    float dp1[E], dp2[E];
    copy_bytes<E * 4>(dp1, dxp + (t0 + tok) * fp + m * E);
    copy_bytes<E * 4>(dp2, dxp + (t0 + tok) * fp + G::HALF + m * E);
    const float inv = invs[tok];
    float dy1[E], dy2[E];
    float T = 0.f;
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const float2 cs = angle_sum(hi[e], lo[tok][e]);
      const float x1 = r.get(tok, 0, e), x2 = r.get(tok, 1, e);
      const float d1 = (gate[tok] >> (2 * e)) & 1u ? dp1[e] : 0.f;
      const float d2 = (gate[tok] >> (2 * e + 1)) & 1u ? dp2[e] : 0.f;
      dy1[e] = __builtin_fmaf(d1, cs.x, d2 * cs.y);     // inverse rotation
      dy2[e] = __builtin_fmaf(d2, cs.x, -(d1 * cs.y));
      T = __builtin_fmaf(g1[e] * dy1[e], x1, T);
      T = __builtin_fmaf(g2[e] * dy2[e], x2, T);
      dg1[e] = __builtin_fmaf(dy1[e], x1 * inv, dg1[e]);
      dg2[e] = __builtin_fmaf(dy2[e], x2 * inv, dg2[e]);
    }
    T = sum8(T);
    const float coef = inv * inv * inv * T * (1.0f / D);
#pragma unroll
    for (int e = 0; e < E; e += 2) {
      const float a0 = __builtin_fmaf(inv * g1[e], dy1[e], -(coef * r.get(tok, 0, e)));
      const float a1 = __builtin_fmaf(inv * g1[e + 1], dy1[e + 1], -(coef * r.get(tok, 0, e + 1)));
      const float b0 = __builtin_fmaf(inv * g2[e], dy2[e], -(coef * r.get(tok, 1, e)));
      const float b1 = __builtin_fmaf(inv * g2[e + 1], dy2[e + 1], -(coef * r.get(tok, 1, e + 1)));
      dx.w[tok][0][e >> 1] = pack_bf2(a0, a1);
      dx.w[tok][1][e >> 1] = pack_bf2(b0, b1);
    }
  }
}

// ----------------------------------------------------------------------------------------
// bwd_pstate: per (segment, head), the segment's totals of the reverse states,
// sum_t Q^_t g_t^T (d x d, fragment-native like the forward records) and sum_t Q^_t gd_t den_t
// (where the z of a forward record sits); Q^_t = bf16(q'_t / den_t), den and gd from bwd_dq.

template <int D, bool ALL>
__global__ __launch_bounds__(256, 2) void bwd_pstate_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ dout, const float* __restrict__ gamma_q,
    const int32_t* __restrict__ tab, const int32_t* __restrict__ nseg, const float2* __restrict__ rope_lo,
    const float2* __restrict__ rope_hi, const float* __restrict__ den, const float* __restrict__ gd,
    float* __restrict__ pstates, int H, int L, float rms_eps, const uint32_t* __restrict__ hdr, TabLimits lim,
    int first_too) {
  using G = Geo<true, D>;
  using R = Raw<true, D>;
  constexpr int BUF = kChunk * G::ROWP;
  constexpr int RT = G::RT, CT = G::CT, E = G::E;
  constexpr int ZR = RT >= 4 ? RT / 4 : 1;  // row tiles of p per wave
  __shared__ __attribute__((aligned(16))) uint16_t sH[BUF];  // Q^ rows
  __shared__ __attribute__((aligned(16))) uint16_t sG[BUF];  // dout rows
  __shared__ float sW[kChunk];                                // gd den
  __shared__ __attribute__((aligned(16))) float2 sHi[kMaxSegChunks * G::HALF];  // RoPE rows of the chunks

  const int seg = blockIdx.x, h = blockIdx.y;
  if (!bwd_go(hdr) || seg >= *nseg) return;
  const SegInfo si = read_seg_clamped(tab, seg, L, lim);
  if (si.len == 0) return;  // only a corrupted table has empty segments
  // causal: a document's first segment is skipped (no earlier segment reads its total) unless
  // first_too asks for the whole-document totals of the documents that start from the initial
  // state (each row's segment at token 0); bidirectional (ALL): every segment's total goes into
  // the document's
  if (!ALL && si.pos0 == 0 && !(first_too && si.start == 0)) return;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int nch = __builtin_amdgcn_readfirstlane((si.len + kChunk - 1) / kChunk);
  const int t0 = 2 * (tid >> 3), m = tid & 7;
  const int c16 = lane & 15, g = lane >> 4;
  const size_t tok0 = ((size_t)si.row * H + h) * (size_t)L + si.start;
  const int seg_bytes = si.len * D * 2;
  const __amdgpu_buffer_rsrc_t rq = __builtin_amdgcn_make_buffer_rsrc((void*)(q + tok0 * D), 0, seg_bytes, kBufFlags);
  const __amdgpu_buffer_rsrc_t rg = __builtin_amdgcn_make_buffer_rsrc((void*)(dout + tok0 * D), 0, seg_bytes, kBufFlags);
  const __amdgpu_buffer_rsrc_t rd = __builtin_amdgcn_make_buffer_rsrc((void*)(den + tok0), 0, si.len * 4, kBufFlags);
  const __amdgpu_buffer_rsrc_t rw = __builtin_amdgcn_make_buffer_rsrc((void*)(gd + tok0), 0, si.len * 4, kBufFlags);
  float g1[E], g2[E];
  float2 lo[2][E];
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const int j = m * E + e;
    g1[e] = gamma_q[(size_t)h * D + j];
    g2[e] = gamma_q[(size_t)h * D + j + G::HALF];
    lo[0][e] = rope_lo[t0 * G::HALF + j];
    lo[1][e] = rope_lo[(t0 + 1) * G::HALF + j];
  }
  {
    const float2* hi0 = rope_hi + (size_t)si.hirow * G::HALF;
    for (int i = tid; i < min(nch, kMaxSegChunks) * G::HALF; i += 256) sHi[i] = hi0[i];
  }
  floatx4 P[RT][CT], pz[ZR];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt)
#pragma unroll
    for (int ct = 0; ct < CT; ++ct) P[rt][ct] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int z = 0; z < ZR; ++z) pz[z] = floatx4{0.f, 0.f, 0.f, 0.f};
  const bool zwave = wave * ZR < RT;

  // two chunks of inputs in flight: register set c % 2 holds chunk c and is refilled with
  // chunk c + 2 as it frees up (dout first, then q one token at a time)
  struct In {
    R xq, xg;
    float dn[2], w[2];
  };
  auto issue = [&](In& in, int c) {  // chunk c's inputs; tokens past the segment read 0 and weigh nothing
    load_raw_buf<true, D>(in.xg, rg, c * kChunk + t0, m);
#pragma unroll
    for (int tok = 0; tok < 2; ++tok) {
      in.dn[tok] = load_tok(rd, c * kChunk + t0 + tok);
      in.w[tok] = load_tok(rw, c * kChunk + t0 + tok);
    }
    load_raw_buf<true, D>(in.xq, rq, c * kChunk + t0, m);
  };
  In set0, set1;
  issue(set0, 0);
  issue(set1, 1);
  auto step = [&](int c, In& in) {
    __syncthreads();  // the previous chunk's operands are consumed (the first time: sHi is written)
    float2 hi[E];
    copy_bytes<E * 8>(hi, sHi + c * G::HALF + m * E);
    store_rows<true, D>(sG, in.xg, t0, m);
    load_raw_buf<true, D>(in.xg, rg, (c + 2) * kChunk + t0, m);
    const float inv[2] = {in.dn[0] > 0.f ? 1.0f / in.dn[0] : 0.f, in.dn[1] > 0.f ? 1.0f / in.dn[1] : 0.f};
    if (m == 0) {
      sW[t0] = in.w[0] * in.dn[0];
      sW[t0 + 1] = in.w[1] * in.dn[1];
    }
#pragma unroll
    for (int tok = 0; tok < 2; ++tok) {
      in.dn[tok] = load_tok(rd, (c + 2) * kChunk + t0 + tok);
      in.w[tok] = load_tok(rw, (c + 2) * kChunk + t0 + tok);
    }
    auto map_tok = [&](auto tok_c) {
      constexpr int tok = decltype(tok_c)::value;
      R oq, oh;
      feature_map_lane<true, D, tok>(in.xq, oq, g1, g2, lo, hi, rms_eps);
      scale_raw<D, tok>(oq, oh, inv);
      store_rows<true, D, tok>(sH, oh, t0, m);
      load_raw_buf<true, D, tok>(in.xq, rq, (c + 2) * kChunk + t0, m);
    };
    map_tok(std::integral_constant<int, 0>{});
    map_tok(std::integral_constant<int, 1>{});
    __syncthreads();
    if (wave < G::NW) {
      Frag<true> Nf[CT][2];
#pragma unroll
      for (int ct = 0; ct < CT; ++ct) {
        Nf[ct][0] = lds_frag_tr(sG, G::ROWP, 0, wave * G::DVW + ct * 16, lane);
        Nf[ct][1] = lds_frag_tr(sG, G::ROWP, 32, wave * G::DVW + ct * 16, lane);
      }
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
          const Frag<true> a = lds_frag_tr(sH, G::ROWP, 32 * kb, 16 * rt, lane);
#pragma unroll
          for (int ct = 0; ct < CT; ++ct) P[rt][ct] = mma(a, Nf[ct][kb], P[rt][ct]);
        }
    }
    if (zwave) {  // p += Q^^T (gd den) against an operand holding it in every column
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        Frag<true> w_hi, w_lo;
        token_col_frags(sW, kb, g, w_hi, w_lo);
#pragma unroll
        for (int z = 0; z < ZR; ++z) {
          const Frag<true> a = lds_frag_tr(sH, G::ROWP, 32 * kb, 16 * (wave * ZR + z), lane);
          pz[z] = mma(a, w_hi, pz[z]);
          pz[z] = mma(a, w_lo, pz[z]);
        }
      }
    }
  };
  for (int c = 0; c < nch; c += 2) {
    step(c, set0);
    if (c + 1 < nch) step(c + 1, set1);
  }
  float* rec = pstates + ((size_t)seg * H + h) * (size_t)(D * D + D);
  if (wave < G::NW) {
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
      for (int ct = 0; ct < CT; ++ct)
        __builtin_nontemporal_store(P[rt][ct], reinterpret_cast<floatx4*>(rec + rec_frag<true, D>(wave, rt, ct, lane)));
  }
  if (zwave && c16 < 4) {  // every column of pz holds the sums of rows 16 rt + 4g + i
#pragma unroll
    for (int z = 0; z < ZR; ++z) rec[D * D + (wave * ZR + z) * 16 + 4 * g + c16] = pz[z][c16];
  }
}

// ----------------------------------------------------------------------------------------
// bwd_dq_ws: the dq sweep, warp-specialised, 8 waves, one workgroup per CU, steps of 32 tokens (half
// a chunk; the RoPE row of the chunk serves both halves, the in-chunk angles are rows 0..31 or
// 32..63 of the small table).
//   waves 4, 5 ("forward mappers"): q', k' and the raw v rows of sub-chunk st into buffer st % 2,
//          its raw q into a ring of three (raw q, k, v of two sub-chunks in flight);
//   waves 0..3 ("MMA waves"): sub-chunk st - 1 from the other buffer. The running state lives
//          only in accumulators, as S^T (rows = value dims, columns = key dims a; wave w holds
//          the key dims of the forward's value-column split): an accumulator tile is at once an
//          A operand whose rows are its columns and a B operand whose columns are its columns,
//          both with the contraction over its rows, so (S g)[a] = sum_v S^T[v][a] g[v] and
//          S^T += V^T K' need no transposed copy. Per step: the wave's rows of (S G^T) (the
//          state as a bf16 pair) and its part of q' . (S g) for all 32 queries; waves 0, 1 also
//          the score tiles of query tile w (A^T, V G^T, q' . z); meeting; waves 0, 1: den, g.num,
//          gd, B_tt and B^T (to LDS and to the per-token planes); meeting; every wave: its rows
//          of dQ'^T = (S G^T)/den + z gd^T + K'^T B^T as fp32 rows of the dq' buffer of the
//          sub-chunk and S^T += V^T K'; waves 2, 3 form z for the next sub-chunk during the scores;
//   waves 6, 7 ("backward mappers"): the raw dout rows of sub-chunk st into buffer st % 2
//          (two sub-chunks in flight), then the map backward of sub-chunk st - 2 from its dq'
//          rows and the raw q in the ring.
// One workgroup barrier per step; the MMA waves also meet twice among themselves.

template <int D>
__device__ __forceinline__ void split_frag(floatx4 a, floatx4 b, Frag<true>& hi, Frag<true>& lo) {
  // the accumulator pair (rows 0..15, 16..31 of a k-block) as bf16 operands: value + remainder
  const uint32_t h0 = pack_bf2(a[0], a[1]), h1 = pack_bf2(a[2], a[3]);
  const uint32_t h2 = pack_bf2(b[0], b[1]), h3 = pack_bf2(b[2], b[3]);
  hi.v = __builtin_bit_cast(bf16x8, u32x4{h0, h1, h2, h3});
  lo.v = __builtin_bit_cast(bf16x8, u32x4{pack_bf2(a[0] - bf_lo(h0), a[1] - bf_hi(h0)),
                                          pack_bf2(a[2] - bf_lo(h1), a[3] - bf_hi(h1)),
                                          pack_bf2(b[0] - bf_lo(h2), b[1] - bf_hi(h2)),
                                          pack_bf2(b[2] - bf_lo(h3), b[3] - bf_hi(h3))});
}

template <int D, bool BIDIR>
__global__ __launch_bounds__(512, 1) void bwd_dq_ws_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    const uint16_t* __restrict__ dout, const float* __restrict__ gamma_q, const float* __restrict__ gamma_k,
    const int32_t* __restrict__ tab, const int32_t* __restrict__ nseg, const float2* __restrict__ rope_lo,
    const float2* __restrict__ rope_hi, const float* __restrict__ states, uint16_t* __restrict__ dq,
    float* __restrict__ den_out, float* __restrict__ gd_out, float* __restrict__ bd_out, float* __restrict__ dg_part,
    int H, int L, float rms_eps, float eps, uint32_t* __restrict__ hdr, uint32_t polls, TabLimits lim) {
  using G = Geo<true, D>;
  using R = Raw<true, D>;
  constexpr int C2 = 32;                 // tokens per step
  constexpr int BUF = C2 * G::ROWP;      // elements of one raw-q ring buffer
  // operand rows (q', k', v, dout) at a pitch of D + 16: the 16-byte row-fragment reads
  // (lds_frag_c) and the transposing reads are then free of bank conflicts
  constexpr int QP = D + 16, BUFQ = C2 * QP;
  constexpr int FP = D + 4;              // pitch of the fp32 dq' rows
  constexpr int RT = G::RT, CT = G::CT, KB = G::KB, E = G::E, NW = G::NW;
  __shared__ __attribute__((aligned(16))) uint16_t sQ[2 * BUFQ];
  __shared__ __attribute__((aligned(16))) uint16_t sK[2 * BUFQ];
  __shared__ __attribute__((aligned(16))) uint16_t sV[2 * BUFQ];
  __shared__ __attribute__((aligned(16))) uint16_t sG[2 * BUFQ];
  __shared__ __attribute__((aligned(16))) uint16_t sRq[3 * BUF];  // raw q rows, ring of three
  // bidirectional: the forward mapper's ReLU gates (a word per lane and token) and 1/rms per
  // token, beside the raw rows in the ring, for the backward mappers
  __shared__ uint32_t sGate[BIDIR ? 3 * C2 * 8 : 1];
  __shared__ float sRinv[BIDIR ? 3 * C2 : 1];
  __shared__ __attribute__((aligned(16))) float sdQ[2 * C2 * FP];
  __shared__ Frag<true> sB[2 * 64];                    // B^T operands of query tiles 0, 1
  __shared__ __attribute__((aligned(16))) float sZ[2 * D];  // z before the sub-chunk, by parity
  // z as an MFMA A operand, by parity: row 0 = bf16(z), row 1 = bf16(z - bf16(z)), other rows 0,
  // so Z Q'^T gives q'.z (to ~2^-17 relative) in rows 0 + 1 of each query column
  __shared__ Frag<true> sZf[2 * KB * 64];
  __shared__ float sIdot[4 * C2];                      // each MMA wave's part of q' . (S g)
  __shared__ float sInv[C2], sGd[C2];
  __shared__ unsigned sArrive;

  const int seg = blockIdx.x, h = blockIdx.y;
  if (!bwd_go(hdr) || seg >= *nseg) return;  // the whole workgroup leaves together
  const SegInfo si = read_seg_clamped(tab, seg, L, lim);
  if (si.len == 0) return;  // only a corrupted table has empty segments
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int ns = __builtin_amdgcn_readfirstlane((si.len + C2 - 1) / C2);  // sub-chunks
  const int nsteps = (ns + 3) & ~1;  // >= ns + 2, even for the mappers' two-step turns
  const int c16 = lane & 15, g = lane >> 4;
  const size_t tok0 = ((size_t)si.row * H + h) * (size_t)L + si.start;
  const int seg_bytes = si.len * D * 2;
  auto rsrc = [&](const uint16_t* base) {
    return __builtin_amdgcn_make_buffer_rsrc((void*)(base + tok0 * D), 0, seg_bytes, kBufFlags);
  };
  const float* rec = states + ((size_t)seg * H + h) * (size_t)(D * D + D);
  if (tid < D) sZ[tid] = rec[D * D + tid];
  if (tid == 0) sArrive = 0u;
  for (int i = tid; i < 2 * KB * 64; i += 512) sZf[i] = Frag<true>{};
  __syncthreads();
  // the two data lanes of each z fragment (contiguous slot order): slot (g, j) of fragment kb
  // holds dim kb 32 + 8g + j; lane 16g holds bf16(z), lane 16g + 1 the remainder.
  // Called by one wave: lane l converts dims 2l, 2l + 1.
  auto put_zf = [&](Frag<true>* zf, const float* zsrc) {
    uint16_t* zf16 = reinterpret_cast<uint16_t*>(zf);
#pragma unroll
    for (int x = 0; x < 2; ++x) {
      const int dim = 2 * lane + x;
      if (dim < D) {
        const int kb2 = dim / 32, r = dim % 32;
        const int gg = r >> 3, jj = r & 7;
        const float zv = zsrc[dim];
        const uint32_t hw = pack_bf2(zv, 0.f);
        zf16[(kb2 * 64 + 16 * gg) * 8 + jj] = static_cast<uint16_t>(hw & 0xffffu);
        zf16[(kb2 * 64 + 16 * gg + 1) * 8 + jj] = static_cast<uint16_t>(pack_bf2(zv - bf_lo(hw), 0.f) & 0xffffu);
      }
    }
  };
  float dg1[E], dg2[E];  // RMSNorm-weight partials (backward mappers)
#pragma unroll
  for (int e = 0; e < E; ++e) dg1[e] = dg2[e] = 0.f;

  // in-chunk RoPE angles of a mapper lane's tokens for even (rows t0, t0 + 1) and odd
  // (rows 32 + t0, 33 + t0) sub-chunks; the mapper loops take two steps per turn, so the
  // parity, and with it the array, is known at compile time
  auto load_lo2 = [&](float2 (&lo)[2][E], int row, int m) {
#pragma unroll
    for (int e = 0; e < E; ++e) {
      lo[0][e] = rope_lo[(size_t)row * G::HALF + m * E + e];
      lo[1][e] = rope_lo[(size_t)(row + 1) * G::HALF + m * E + e];
    }
  };
  auto hi_row = [&](float2 (&hr)[E], int c, int m) {  // RoPE row of sub-chunk c's chunk
    copy_bytes<E * 8>(hr, rope_hi + (size_t)(si.hirow + (min(c, ns - 1) >> 1)) * G::HALF + m * E);
  };

  if (wave >= 6) {
    // ======== backward mappers: the raw v and dout rows of sub-chunk st (two sub-chunks in
    // flight), then the map backward of sub-chunk st - 2 with its raw q from the ring
    const int mt = tid & 127, t0 = 2 * (mt >> 3), m = mt & 7;
    const __amdgpu_buffer_rsrc_t rg = rsrc(dout), rdq = rsrc(dq);
    float gq1[E], gq2[E];
#pragma unroll
    for (int e = 0; e < E; ++e) {
      gq1[e] = gamma_q[(size_t)h * D + m * E + e];
      gq2[e] = gamma_q[(size_t)h * D + G::HALF + m * E + e];
    }
    float2 lo[2][E], hr[E];  // angles of the sub-chunk mapped back next, loaded a step ahead
    R va, vb;  // raw dout of an even / odd sub-chunk
    auto issue = [&](R& x, int c) { load_raw_buf<true, D>(x, rg, c * C2 + t0, m); };
    auto bstep = [&](int st, R& x) {
      if (st < ns) store_rows<true, D>(sG + (st & 1) * BUFQ, x, t0, m, QP);
      issue(x, st + 2);  // into the registers just consumed
      const int c = st - 2;  // same parity as st
      if (c >= 0 && c < ns) {
        R xq, dx;
        load_rows<D>(sRq + (c % 3) * BUF, t0, m, xq);
        if constexpr (BIDIR) {
          const float invs[2] = {sRinv[(c % 3) * C2 + t0], sRinv[(c % 3) * C2 + t0 + 1]};
          const uint32_t gates[2] = {sGate[((c % 3) * C2 + t0) * 8 + m], sGate[((c % 3) * C2 + t0 + 1) * 8 + m]};
          map_backward_gated<D>(xq, dx, sdQ + (c & 1) * C2 * FP, FP, gq1, gq2, lo, hr, invs, gates, t0, m, dg1, dg2);
        } else {
          map_backward<D>(xq, dx, sdQ + (c & 1) * C2 * FP, FP, gq1, gq2, lo, hr, rms_eps, t0, m, dg1, dg2);
        }
        store_raw_buf<true, D>(dx, rdq, c * C2 + t0, m);  // rows past the segment are dropped
      }
      hi_row(hr, st - 1, m);  // the angles of sub-chunk st - 1, mapped back in the next step
      load_lo2(lo, ((st - 1) & 1) * C2 + t0, m);
      __syncthreads();  // Y
    };
    issue(va, 0);
    issue(vb, 1);
    for (int st = 0; st < nsteps; st += 2) {
      bstep(st, va);
      bstep(st + 1, vb);
    }
  } else if (wave >= 4) {
    // ======== forward mappers: q', k' of sub-chunk st into buffer st % 2 and its raw q into
    // the ring (two sub-chunks of raw q, k in flight)
    const int mt = tid & 127, t0 = 2 * (mt >> 3), m = mt & 7;
    const __amdgpu_buffer_rsrc_t rq = rsrc(q), rk = rsrc(k), rv = rsrc(v);
    float gq1[E], gq2[E], gk1[E], gk2[E];
#pragma unroll
    for (int e = 0; e < E; ++e) {
      gq1[e] = gamma_q[(size_t)h * D + m * E + e];
      gq2[e] = gamma_q[(size_t)h * D + G::HALF + m * E + e];
      gk1[e] = gamma_k[(size_t)h * D + m * E + e];
      gk2[e] = gamma_k[(size_t)h * D + G::HALF + m * E + e];
    }
    float2 lo[2][E], hia[E], hib[E];  // lo: angles of the sub-chunk mapped next
    load_lo2(lo, t0, m);
    R qa[3], qb[3];  // raw q, k, v of an even / odd sub-chunk
    auto issue = [&](R (&x)[3], float2 (&hr)[E], int c) {
      hi_row(hr, c, m);
      load_raw_buf<true, D>(x[0], rq, c * C2 + t0, m);
      if constexpr (!BIDIR) {  // the bidirectional dq needs no k or v (no scores, no state update)
        load_raw_buf<true, D>(x[1], rk, c * C2 + t0, m);
        load_raw_buf<true, D>(x[2], rv, c * C2 + t0, m);
      }
    };
    auto fstep = [&](int st, R (&x)[3], float2 (&hr)[E]) {
      if (st < ns) {
        const int b = (st & 1) * BUFQ;
        R oq, ok;
#pragma unroll
        for (int tok = 0; tok < 2; ++tok) {
          const float invq = rms_inv<true, D>(x[0], tok, rms_eps);
          const float invk = BIDIR ? 0.f : rms_inv<true, D>(x[1], tok, rms_eps);
          uint32_t gm = 0u;  // bidirectional: the gates of the lane's elements
#pragma unroll
          for (int e = 0; e < E; e += 2) {
            float q1[2], q2[2], k1[2], k2[2];
#pragma unroll
            for (int y = 0; y < 2; ++y) {
              const float2 cs = angle_sum(hr[e + y], lo[tok][e + y]);
              rope_pair(x[0].get(tok, 0, e + y), x[0].get(tok, 1, e + y), invq, gq1[e + y], gq2[e + y], cs, q1[y], q2[y]);
              if constexpr (!BIDIR)
                rope_pair(x[1].get(tok, 0, e + y), x[1].get(tok, 1, e + y), invk, gk1[e + y], gk2[e + y], cs, k1[y], k2[y]);
              if constexpr (BIDIR)
                gm |= (q1[y] > 0.f ? 1u : 0u) << (2 * (e + y)) | (q2[y] > 0.f ? 2u : 0u) << (2 * (e + y));
            }
            put_pairs<true, D>(oq, tok, e, q1, q2);
            if constexpr (!BIDIR) put_pairs<true, D>(ok, tok, e, k1, k2);
          }
          if constexpr (BIDIR) {
            sGate[((st % 3) * C2 + t0 + tok) * 8 + m] = gm;
            if (m == 0) sRinv[(st % 3) * C2 + t0 + tok] = invq;
          }
        }
        store_rows<true, D>(sQ + b, oq, t0, m, QP);
        if constexpr (!BIDIR) {
          store_rows<true, D>(sK + b, ok, t0, m, QP);
          store_rows<true, D>(sV + b, x[2], t0, m, QP);
        }
        store_rows<true, D>(sRq + (st % 3) * BUF, x[0], t0, m);
      }
      issue(x, hr, st + 2);  // into the registers just consumed
      load_lo2(lo, ((st + 1) & 1) * C2 + t0, m);
      __syncthreads();  // Y
    };
    issue(qa, hia, 0);
    issue(qb, hib, 1);
    for (int st = 0; st < nsteps; st += 2) {
      fstep(st, qa, hia);
      fstep(st + 1, qb, hib);
    }
  } else {
  // ======== MMA waves: step st processes sub-chunk c = st - 1
  // S^T in the contiguous-order tile map: tile rt, lane (c, g), row i is v = 32 (rt / 2) + 8g +
  // 4 (rt % 2) + i; columns a = wave DVW + 16 ct + c. Tiles 2kb, 2kb + 1 pair up into operands
  // whose slots match the 16-byte dout fragments.
  floatx4 ST[RT][CT];
  {
    const int wv = wave < NW ? wave : 0;
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
      for (int ct = 0; ct < CT; ++ct) {
        const int a = wv * G::DVW + 16 * ct + c16;  // record: S[a][v] at its fragment-native place
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int vv = 32 * (rt / 2) + 8 * g + 4 * (rt % 2) + i;
          const int w2 = vv / G::DVW, ct2 = (vv % G::DVW) / 16, l2 = 16 * ((a % 16) / 4) + vv % 16;
          ST[rt][ct][i] = rec[rec_frag<true, D>(w2, a / 16, ct2, l2) + a % 4];
        }
      }
  }
  if (wave == 0) put_zf(sZf, sZ);  // parity 0: z before the first sub-chunk
  // waves 2, 3 form the column sums of K' (row tiles 4 (w - 2) .. + 3) while waves 0, 1 do the
  // score tiles; their lanes (i, g), i < 4, hold z of dims 16 tile + 4g + i in registers and
  // write z and its operand form for the next sub-chunk straight into the other parity
  constexpr int ZT = RT / 2;  // column-sum tiles per wave
  float zreg[ZT];
#pragma unroll
  for (int z = 0; z < ZT; ++z) zreg[z] = rec[D * D + min(16 * ((wave & 1) * ZT + z) + 4 * g + (c16 & 3), D - 1)];
  unsigned meet = 0;
  for (int st = 0; st < nsteps; ++st) {
    const int c = st - 1;
    if (c >= 0 && c < ns) {  // uniform over the MMA waves
      const int nv = min(C2, si.len - c * C2);
      const uint16_t* cQ = sQ + (c & 1) * BUFQ;
      const uint16_t* cK = sK + (c & 1) * BUFQ;
      const uint16_t* cV = sV + (c & 1) * BUFQ;
      const uint16_t* cG = sG + (c & 1) * BUFQ;
      const float* zc = sZ + (BIDIR ? 0 : (c & 1) * D);  // bidirectional: the document's z throughout
      // ---- phase A: this wave's rows of S G^T (state as a bf16 pair) and its part of q'.(S g)
      floatx4 Y[CT][2];
      Frag<true> Gf[2][KB];
#pragma unroll
      for (int tt = 0; tt < 2; ++tt)
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) Gf[tt][kb] = lds_frag_c(cG, QP, tt * 16 + c16, kb, g);
      if (wave < NW) {
#pragma unroll
        for (int ct = 0; ct < CT; ++ct) {
          Y[ct][0] = Y[ct][1] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int kb = 0; kb < KB; ++kb) {
            Frag<true> sh, sl;
            split_frag<D>(ST[2 * kb][ct], ST[2 * kb + 1][ct], sh, sl);
#pragma unroll
            for (int tt = 0; tt < 2; ++tt) {
              Y[ct][tt] = mma(sh, Gf[tt][kb], Y[ct][tt]);
              Y[ct][tt] = mma(sl, Gf[tt][kb], Y[ct][tt]);
            }
          }
        }
#pragma unroll
        for (int tt = 0; tt < 2; ++tt) {
          float part = 0.f;
#pragma unroll
          for (int ct = 0; ct < CT; ++ct) {
            const uint2 qa = *reinterpret_cast<const uint2*>(cQ + (tt * 16 + c16) * QP + wave * G::DVW + 16 * ct + 4 * g);
            part = __builtin_fmaf(bf_lo(qa.x), Y[ct][tt][0], part);
            part = __builtin_fmaf(bf_hi(qa.x), Y[ct][tt][1], part);
            part = __builtin_fmaf(bf_lo(qa.y), Y[ct][tt][2], part);
            part = __builtin_fmaf(bf_hi(qa.y), Y[ct][tt][3], part);
          }
          part = sum_rows4(part);
          if (g == 0) sIdot[wave * C2 + tt * 16 + c16] = part;
        }
      }
      if (!BIDIR && wave >= 2) {  // z after this sub-chunk, into the other parity
        const Frag<true> ones = ones_frag<true>();
        float* zn = sZ + ((c + 1) & 1) * D;
        uint16_t* zf16 = reinterpret_cast<uint16_t*>(sZf + ((c + 1) & 1) * KB * 64);
#pragma unroll
        for (int z = 0; z < ZT; ++z) {
          const int T = (wave & 1) * ZT + z;
          const floatx4 zs = mma(lds_frag_tr(cK, QP, 0, 16 * T, lane), ones, floatx4{0.f, 0.f, 0.f, 0.f});
          if (c16 < 4) {
            // dim 16 T + 4g + i: fragment T / 2, slot 4 (g % 2) + i of lane 16 (2 (T % 2) + g / 2)
            // (bf16 of z) and of the lane after it (the remainder)
            zreg[z] += c16 == 0 ? zs[0] : c16 == 1 ? zs[1] : c16 == 2 ? zs[2] : zs[3];
            zn[16 * T + 4 * g + c16] = zreg[z];
            const uint32_t hw = pack_bf2(zreg[z], 0.f);
            uint16_t* dst = zf16 + ((T / 2) * 64 + 16 * (2 * (T % 2) + g / 2)) * 8 + 4 * (g % 2) + c16;
            dst[0] = static_cast<uint16_t>(hw & 0xffffu);
            dst[8] = static_cast<uint16_t>(pack_bf2(zreg[z] - bf_lo(hw), 0.f) & 0xffffu);
          }
        }
      }
      // score tiles of query tile tt = wave (waves 0, 1)
      const int tt = wave & 1;
      const int t = tt * 16 + c16;  // this lane's query
      floatx4 At[2], Bt[2];
      float rs_o = 0.f, dot_o = 0.f, sself = 0.f, bself = 0.f, qz = 0.f;
      if (wave < 2) {
        Frag<true> Qf[KB], Gt[KB];  // the query tile's rows (read again: no runtime register index)
        floatx4 zq = floatx4{0.f, 0.f, 0.f, 0.f};
        const Frag<true>* zf = sZf + (BIDIR ? 0 : (c & 1) * KB * 64);
        Frag<true> Zf[KB];
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) {
          Qf[kb] = lds_frag_c(cQ, QP, t, kb, g);
          Gt[kb] = lds_frag_c(cG, QP, t, kb, g);
          Zf[kb] = zf[kb * 64 + lane];
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) zq = mma(Zf[kb], Qf[kb], zq);
        if (g == 0) qz = zq[0] + zq[1];  // q'_t . z (rows 0, 1 of Z Q'^T)
#pragma unroll
        for (int kt = 0; kt < 2; ++kt) {
          At[kt] = Bt[kt] = floatx4{0.f, 0.f, 0.f, 0.f};
          if (!BIDIR && kt <= tt) {  // bidirectional: the block's keys are inside the document's states
            Frag<true> Kt[KB], Vt[KB];  // key tile kt's rows, requested before its MFMAs
#pragma unroll
            for (int kb = 0; kb < KB; ++kb) {
              Kt[kb] = lds_frag_c(cK, QP, kt * 16 + c16, kb, g);
              Vt[kb] = lds_frag_c(cV, QP, kt * 16 + c16, kb, g);
            }
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int kb = 0; kb < KB; ++kb) {
              At[kt] = mma(Kt[kb], Qf[kb], At[kt]);
              Bt[kt] = mma(Vt[kb], Gt[kb], Bt[kt]);
            }
          }
        }
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const float sc = At[kt][i];
            const bool before = kt < tt || (kt == tt && 4 * g + i < c16);
            const bool self = kt == tt && 4 * g + i == c16;
            rs_o += before ? sc : 0.f;
            dot_o = __builtin_fmaf(before ? sc : 0.f, Bt[kt][i], dot_o);
            sself += self ? sc : 0.f;
            bself += self ? Bt[kt][i] : 0.f;
          }
        rs_o = sum_rows4(rs_o);
        dot_o = sum_rows4(dot_o);
        sself = sum_rows4(sself);
        bself = sum_rows4(bself);
        qz = sum_rows4(qz);
      }
      meet += 4;
      mma_wave_sync(&sArrive, meet, lane, polls, hdr);
      // ---- phase B (waves 0, 1): den, g.num, gd, B_tt, the B^T operand of query tile tt
      if (wave < 2) {
        float idot = 0.f;
#pragma unroll
        for (int w = 0; w < NW; ++w) idot += sIdot[w * C2 + t];
        dot_o += idot;  // g . num without the self term
        const float den_o = rs_o + qz + eps;
        const float den = den_o + sself;
        const float inv = 1.0f / den;
        const float inv2 = inv * inv;
        const float gdv = -__builtin_fmaf(sself, bself, dot_o) * inv2;
        const float bdv = __builtin_fmaf(bself, den_o, -dot_o) * inv2;
        if (g == 0) {
          sInv[t] = inv;
          sGd[t] = gdv;
          if (t < nv) {
            const size_t ix = tok0 + (size_t)c * C2 + t;
            den_out[ix] = den;
            gd_out[ix] = gdv;
            bd_out[ix] = bdv;
          }
        }
        floatx4 x[2];
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const bool before = kt < tt || (kt == tt && 4 * g + i < c16);
            const bool self = kt == tt && 4 * g + i == c16;
            x[kt][i] = before ? __builtin_fmaf(Bt[kt][i], inv, gdv) : (self ? bdv : 0.f);
          }
        if constexpr (!BIDIR) sB[tt * 64 + lane] = acc_frag<true>(x[0], x[1]);
      }
      // the K' column fragments (for dQ' and the state update) and this wave's z values do not
      // depend on phase B: requested before the meeting
      Frag<true> Kc[CT];
      float4 zv[CT];
#pragma unroll
      for (int ct = 0; ct < CT; ++ct) {
        if constexpr (!BIDIR) Kc[ct] = lds_frag_tr(cK, QP, 0, (wave & 3) * G::DVW + 16 * ct, lane);
        zv[ct] = *reinterpret_cast<const float4*>(zc + (wave & 3) * G::DVW + 16 * ct + 4 * g);
      }
      meet += 4;
      mma_wave_sync(&sArrive, meet, lane, polls, hdr);
      // ---- phase C: this wave's rows of dQ'^T, then the state
      if (wave < NW) {
        float* dqb = sdQ + (c & 1) * C2 * FP;
        float invs[2], gds[2];
        Frag<true> bfs[2];
#pragma unroll
        for (int tq = 0; tq < 2; ++tq) {
          invs[tq] = sInv[tq * 16 + c16];
          gds[tq] = sGd[tq * 16 + c16];
          if constexpr (!BIDIR) bfs[tq] = sB[tq * 64 + lane];
        }
        Frag<true> avn[2];  // the state update's row fragments, one tile ahead
        if constexpr (!BIDIR) avn[0] = lds_frag_tr_s8(cV, QP, 0, 0, lane);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int tq = 0; tq < 2; ++tq) {
          const int tc = tq * 16 + c16;  // query column of the tiles
          const float inv = invs[tq], gdv = gds[tq];
#pragma unroll
          for (int ct = 0; ct < CT; ++ct) {
            const int a0 = wave * G::DVW + 16 * ct + 4 * g;
            floatx4 acc = Y[ct][tq];
#pragma unroll
            for (int i = 0; i < 4; ++i) acc[i] = __builtin_fmaf(acc[i], inv, gdv * zv[ct][i]);
            if constexpr (!BIDIR) acc = mma(Kc[ct], bfs[tq], acc);
            *reinterpret_cast<floatx4*>(dqb + tc * FP + a0) = acc;
          }
        }
        // S^T += V^T K' (the 32 tokens are one k-block); bidirectional: the state is the document's
        if constexpr (!BIDIR) {
#pragma unroll
          for (int rt = 0; rt < RT; ++rt) {
            const int cur = rt & 1, nxt = cur ^ 1;
            if (rt + 1 < RT) avn[nxt] = lds_frag_tr_s8(cV, QP, 0, 32 * ((rt + 1) / 2) + 4 * ((rt + 1) % 2), lane);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int ct = 0; ct < CT; ++ct) ST[rt][ct] = mma(avn[cur], Kc[ct], ST[rt][ct]);
          }
        }
      }
    }
    __syncthreads();  // Y
  }
  }
  // RMSNorm-weight partials of the two backward-mapper waves: lanes sharing m, then the waves
  __syncthreads();  // every wave is done with LDS
  if (wave >= 6) {
    const int m = tid & 7;
#pragma unroll
    for (int e = 0; e < E; ++e) {
#pragma unroll
      for (int o = 8; o < 64; o <<= 1) {
        dg1[e] += __shfl_xor(dg1[e], o);
        dg2[e] += __shfl_xor(dg2[e], o);
      }
    }
    if (lane < 8) {
#pragma unroll
      for (int e = 0; e < E; ++e) {
        sdQ[(wave - 6) * D + m * E + e] = dg1[e];
        sdQ[(wave - 6) * D + G::HALF + m * E + e] = dg2[e];
      }
    }
  }
  __syncthreads();
  float* dst = dg_part + ((size_t)seg * H + h) * 2 * D;
  for (int i = tid; i < D; i += 512) dst[i] = sdQ[i] + sdQ[D + i];
}

// ----------------------------------------------------------------------------------------
// bwd_dkv_ws: the dk, dv sweep, warp-specialised like bwd_dq_ws (8 waves, one workgroup per CU,
// 32-token steps), sub-chunks in reverse order.
//   waves 4, 5 ("forward mappers"): q', k', the raw v rows and Q^ = bf16(q'/den) of sub-chunk
//          j (the j-th from the end) into buffer j % 2, with 1/den, gd, B_tt and gd den per token
//          (from the planes bwd_dq wrote); its raw k into a ring of three;
//   waves 0..3 ("MMA waves"): sub-chunk j - 1. The reverse state lives only in accumulators,
//          twice: P^T (rows = value dims v, columns = the wave's slice of the query dims a) for
//          dK'^T = P V^T, and P (rows a, columns = the wave's slice of v) for dV^T = P^T K'^T, so
//          each product contracts over the rows of its accumulator tiles and no transposed copy
//          is needed. Per step: waves 0, 1, key tile w: A = mask(Q' K'^T) and B = mask(G V^T /
//          den + gd) (B_tt on the diagonal) as the B operands A/den and B (queries x keys);
//          meeting; every wave: its rows of dK'^T = P V^T + Q'^T B + p (fp32 rows of the dk'
//          buffer) and of dV^T = P^T K'^T + G^T (A/den) (stored), then P^T += G^T Q^,
//          P += Q^^T G, and (wave 0) p for the next sub-chunk, all states as bf16 operand pairs;
//   waves 6, 7 ("backward mappers"): the raw dout rows of sub-chunk j into buffer j % 2, then
//          the map backward of k for sub-chunk j - 2 from its dk' rows and the ring.
// One workgroup barrier per step; the MMA waves also meet once among themselves.

template <int D, bool BIDIR>
__global__ __launch_bounds__(512, 1) void bwd_dkv_ws_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    const uint16_t* __restrict__ dout, const float* __restrict__ gamma_q, const float* __restrict__ gamma_k,
    const int32_t* __restrict__ tab, const int32_t* __restrict__ nseg, const float2* __restrict__ rope_lo,
    const float2* __restrict__ rope_hi, const float* __restrict__ pstates, const float* __restrict__ den,
    const float* __restrict__ gd, const float* __restrict__ bd, uint16_t* __restrict__ dk, uint16_t* __restrict__ dv,
    float* __restrict__ dg_part, int H, int L, float rms_eps, uint32_t* __restrict__ hdr, uint32_t polls,
    TabLimits lim) {
  using G = Geo<true, D>;
  using R = Raw<true, D>;
  constexpr int C2 = 32;
  constexpr int BUF = C2 * G::ROWP;  // raw-k ring buffer
  // operand rows (q', k', v, dout, Q^) at a pitch of D + 16 (conflict-free 16-byte row-fragment
  // and transposing reads)
  constexpr int QP = D + 16, BUFQ = C2 * QP;
  constexpr int FP = D + 4;
  constexpr int RT = G::RT, CT = G::CT, KB = G::KB, E = G::E, NW = G::NW;
  __shared__ __attribute__((aligned(16))) uint16_t sQ[2 * BUFQ];
  __shared__ __attribute__((aligned(16))) uint16_t sK[2 * BUFQ];
  __shared__ __attribute__((aligned(16))) uint16_t sV[2 * BUFQ];
  __shared__ __attribute__((aligned(16))) uint16_t sG[2 * BUFQ];
  __shared__ __attribute__((aligned(16))) uint16_t sH[2 * BUFQ];  // Q^ rows
  __shared__ __attribute__((aligned(16))) uint16_t sRk[3 * BUF];  // raw k rows, ring of three
  __shared__ __attribute__((aligned(16))) float sdK[2 * C2 * FP];
  __shared__ Frag<true> sAp[2 * 64], sBp[2 * 64];  // per key tile: A/den and B (queries x keys)
  __shared__ __attribute__((aligned(16))) float sP[2 * D];   // p after the sub-chunk, by parity
  __shared__ __attribute__((aligned(16))) float sI[2 * C2];
  __shared__ __attribute__((aligned(16))) float sGd[2 * C2];
  __shared__ __attribute__((aligned(16))) float sBd[2 * C2];
  __shared__ __attribute__((aligned(16))) float sW[2 * C2];
  __shared__ unsigned sArrive;

  const int seg = blockIdx.x, h = blockIdx.y;
  if (!bwd_go(hdr) || seg >= *nseg) return;  // the whole workgroup leaves together
  const SegInfo si = read_seg_clamped(tab, seg, L, lim);
  if (si.len == 0) return;  // only a corrupted table has empty segments
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int ns = __builtin_amdgcn_readfirstlane((si.len + C2 - 1) / C2);  // sub-chunks
  const int nsteps = (ns + 3) & ~1;
  const int c16 = lane & 15, g = lane >> 4;
  const size_t tok0 = ((size_t)si.row * H + h) * (size_t)L + si.start;
  const int seg_bytes = si.len * D * 2;
  auto rsrc = [&](const uint16_t* base) {
    return __builtin_amdgcn_make_buffer_rsrc((void*)(base + tok0 * D), 0, seg_bytes, kBufFlags);
  };
  auto rsrc_tok = [&](const float* base) {
    return __builtin_amdgcn_make_buffer_rsrc((void*)(base + tok0), 0, si.len * 4, kBufFlags);
  };
  const float* rec = pstates + ((size_t)seg * H + h) * (size_t)(D * D + D);
  if (tid < D) sP[tid] = rec[D * D + tid];
  if (tid == 0) sArrive = 0u;
  __syncthreads();
  float dg1[E], dg2[E];  // RMSNorm-weight partials of k (backward mappers)
#pragma unroll
  for (int e = 0; e < E; ++e) dg1[e] = dg2[e] = 0.f;
  auto sub = [&](int j) { return ns - 1 - j; };  // the j-th sub-chunk from the end
  // the same for loads: j past the last step gives the sub-chunk just past the segment, which
  // the buffer range check turns into zeros
  auto sub_ld = [&](int j) { return j < ns ? ns - 1 - j : ns; };
  auto load_lo2 = [&](float2 (&lo)[2][E], int row, int m) {
#pragma unroll
    for (int e = 0; e < E; ++e) {
      lo[0][e] = rope_lo[(size_t)row * G::HALF + m * E + e];
      lo[1][e] = rope_lo[(size_t)(row + 1) * G::HALF + m * E + e];
    }
  };
  auto hi_row = [&](float2 (&hr)[E], int c, int m) {  // RoPE row of sub-chunk c's chunk
    copy_bytes<E * 8>(hr, rope_hi + (size_t)(si.hirow + (min(max(c, 0), ns - 1) >> 1)) * G::HALF + m * E);
  };

  if (wave >= 6) {
    // ======== backward mappers: dout rows of sub-chunk j, map backward of k for j - 2
    const int mt = tid & 127, t0 = 2 * (mt >> 3), m = mt & 7;
    const __amdgpu_buffer_rsrc_t rg = rsrc(dout), rdk = rsrc(dk);
    float gk1[E], gk2[E];
#pragma unroll
    for (int e = 0; e < E; ++e) {
      gk1[e] = gamma_k[(size_t)h * D + m * E + e];
      gk2[e] = gamma_k[(size_t)h * D + G::HALF + m * E + e];
    }
    float2 lo[2][E], hr[E];  // angles of the sub-chunk mapped back next, loaded a step ahead
    R ga, gb;  // raw dout of an even / odd step
    // (the bidirectional dk, dv need no dout: P and p are the document's totals)
    auto issue = [&](R& x, int j) {
      if constexpr (!BIDIR) load_raw_buf<true, D>(x, rg, sub_ld(j) * C2 + t0, m);
    };
    auto bstep = [&](int st, R& x) {
      if (!BIDIR && st < ns) store_rows<true, D>(sG + (st & 1) * BUFQ, x, t0, m, QP);
      issue(x, st + 2);
      const int j = st - 2;
      if (j >= 0 && j < ns) {
        R xk, dx;
        load_rows<D>(sRk + (j % 3) * BUF, t0, m, xk);
        map_backward<D>(xk, dx, sdK + (j & 1) * C2 * FP, FP, gk1, gk2, lo, hr, rms_eps, t0, m, dg1, dg2);
        store_raw_buf<true, D>(dx, rdk, sub(j) * C2 + t0, m);  // rows past the segment are dropped
      }
      hi_row(hr, sub(st - 1), m);  // the angles of step st - 1's sub-chunk, mapped back next step
      load_lo2(lo, (sub(st - 1) & 1) * C2 + t0, m);
      __syncthreads();  // Y
    };
    issue(ga, 0);
    issue(gb, 1);
    for (int st = 0; st < nsteps; st += 2) {
      bstep(st, ga);
      bstep(st + 1, gb);
    }
  } else if (wave >= 4) {
    // ======== forward mappers: q', k', v, Q^ rows and per-token values of sub-chunk j
    const int mt = tid & 127, t0 = 2 * (mt >> 3), m = mt & 7;
    const __amdgpu_buffer_rsrc_t rq = rsrc(q), rk = rsrc(k), rv = rsrc(v);
    const __amdgpu_buffer_rsrc_t rd = rsrc_tok(den), rw = rsrc_tok(gd), rb = rsrc_tok(bd);
    float gq1[E], gq2[E], gk1[E], gk2[E];
#pragma unroll
    for (int e = 0; e < E; ++e) {
      gq1[e] = gamma_q[(size_t)h * D + m * E + e];
      gq2[e] = gamma_q[(size_t)h * D + G::HALF + m * E + e];
      gk1[e] = gamma_k[(size_t)h * D + m * E + e];
      gk2[e] = gamma_k[(size_t)h * D + G::HALF + m * E + e];
    }
    float2 lo[2][E], hia[E], hib[E];
    load_lo2(lo, (sub(0) & 1) * C2 + t0, m);
    R xa[3], xb[3];  // raw q, k, v of an even / odd step
    auto issue = [&](R (&x)[3], float2 (&hr)[E], float (&tv)[3][2], int j) {
      hi_row(hr, sub(j), m);
      if constexpr (!BIDIR) load_raw_buf<true, D>(x[0], rq, sub_ld(j) * C2 + t0, m);
      load_raw_buf<true, D>(x[1], rk, sub_ld(j) * C2 + t0, m);
      load_raw_buf<true, D>(x[2], rv, sub_ld(j) * C2 + t0, m);
      if constexpr (!BIDIR) {
#pragma unroll
        for (int tok = 0; tok < 2; ++tok) {  // den, gd, bd (tokens past the segment read 0 and weigh nothing)
          tv[0][tok] = load_tok(rd, sub_ld(j) * C2 + t0 + tok);
          tv[1][tok] = load_tok(rw, sub_ld(j) * C2 + t0 + tok);
          tv[2][tok] = load_tok(rb, sub_ld(j) * C2 + t0 + tok);
        }
      }
    };
    auto fstep = [&](int st, R (&x)[3], float2 (&hr)[E], float (&tv)[3][2]) {
      if (st < ns) {
        const int b = (st & 1) * BUFQ;
        R oq, ok, oh;
#pragma unroll
        for (int tok = 0; tok < 2; ++tok) {
          const float invq = BIDIR ? 0.f : rms_inv<true, D>(x[0], tok, rms_eps);
          const float invk = rms_inv<true, D>(x[1], tok, rms_eps);
#pragma unroll
          for (int e = 0; e < E; e += 2) {
            float q1[2], q2[2], k1[2], k2[2];
#pragma unroll
            for (int y = 0; y < 2; ++y) {
              const float2 cs = angle_sum(hr[e + y], lo[tok][e + y]);
              if constexpr (!BIDIR)
                rope_pair(x[0].get(tok, 0, e + y), x[0].get(tok, 1, e + y), invq, gq1[e + y], gq2[e + y], cs, q1[y], q2[y]);
              rope_pair(x[1].get(tok, 0, e + y), x[1].get(tok, 1, e + y), invk, gk1[e + y], gk2[e + y], cs, k1[y], k2[y]);
            }
            if constexpr (!BIDIR) put_pairs<true, D>(oq, tok, e, q1, q2);
            put_pairs<true, D>(ok, tok, e, k1, k2);
          }
        }
        const float dn[2] = {tv[0][0], tv[0][1]}, gdl[2] = {tv[1][0], tv[1][1]}, bdl[2] = {tv[2][0], tv[2][1]};
        const float inv[2] = {dn[0] > 0.f ? 1.0f / dn[0] : 0.f, dn[1] > 0.f ? 1.0f / dn[1] : 0.f};
        if constexpr (!BIDIR) {
          scale_raw<D>(oq, oh, inv);
          store_rows<true, D>(sQ + b, oq, t0, m, QP);
          store_rows<true, D>(sH + b, oh, t0, m, QP);
        }
        store_rows<true, D>(sK + b, ok, t0, m, QP);
        store_rows<true, D>(sV + b, x[2], t0, m, QP);
        store_rows<true, D>(sRk + (st % 3) * BUF, x[1], t0, m);
        if (!BIDIR && m == 0) {
#pragma unroll
          for (int tok = 0; tok < 2; ++tok) {
            const int ix = (st & 1) * C2 + t0 + tok;
            sI[ix] = inv[tok];
            sGd[ix] = gdl[tok];
            sBd[ix] = bdl[tok];
            sW[ix] = gdl[tok] * dn[tok];
          }
        }
      }
      issue(x, hr, tv, st + 2);  // into the registers just consumed
      load_lo2(lo, (sub(st + 1) & 1) * C2 + t0, m);
      __syncthreads();  // Y
    };
    float ta[3][2], tb[3][2];
    issue(xa, hia, ta, 0);
    issue(xb, hib, tb, 1);
    for (int st = 0; st < nsteps; st += 2) {
      fstep(st, xa, hia, ta);
      fstep(st + 1, xb, hib, tb);
    }
  } else {
    // ======== MMA waves: step st processes sub-chunk sub(st - 1)
    // both in the contiguous-order tile map: in tile rt, lane (c, g), row i is dim
    // 32 (rt / 2) + 8g + 4 (rt % 2) + i, so tiles 2kb, 2kb + 1 pair up into operands whose
    // slots match the 16-byte row fragments
    floatx4 PT[RT][CT];  // P^T: rows v, columns a = wave DVW + 16 ct + c16
    floatx4 PM[RT][CT];  // P: rows a, columns v = wave DVW + 16 ct + c16
    {
      const int wv = wave < NW ? wave : 0;
#pragma unroll
      for (int rt = 0; rt < RT; ++rt)
#pragma unroll
        for (int ct = 0; ct < CT; ++ct) {
          PM[rt][ct] = *reinterpret_cast<const floatx4*>(rec + rec_frag_c<D>(wv, rt, ct, lane));
          const int a = wv * G::DVW + 16 * ct + c16;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int vv = 32 * (rt / 2) + 8 * g + 4 * (rt % 2) + i;
            const int w2 = vv / G::DVW, ct2 = (vv % G::DVW) / 16, l2 = 16 * ((a % 16) / 4) + vv % 16;
            PT[rt][ct][i] = rec[rec_frag<true, D>(w2, a / 16, ct2, l2) + a % 4];
          }
        }
    }
    const __amdgpu_buffer_rsrc_t rdv = rsrc(dv);
    unsigned meet = 0;
    for (int st = 0; st < nsteps; ++st) {
      const int j = st - 1;
      if (j >= 0 && j < ns) {  // uniform over the MMA waves
        const int c = sub(j), nv = min(C2, si.len - c * C2);
        const int pb = (j & 1);
        const uint16_t* cQ = sQ + pb * BUFQ;
        const uint16_t* cK = sK + pb * BUFQ;
        const uint16_t* cV = sV + pb * BUFQ;
        const uint16_t* cG = sG + pb * BUFQ;
        const uint16_t* cH = sH + pb * BUFQ;
        const float* cI = sI + pb * C2;
        const float* pc = sP + (BIDIR ? 0 : pb * D);  // bidirectional: the document's p throughout
        // ---- phase A (waves 0, 1): key tile kt = wave (the bidirectional sweep has no
        // in-block terms: every query's contribution is in the document's P and p)
        if (!BIDIR && wave < 2) {
          const int kt = wave;
          const int key = kt * 16 + c16;
          Frag<true> Kf[KB], Vf[KB];
#pragma unroll
          for (int kb = 0; kb < KB; ++kb) {
            Kf[kb] = lds_frag_c(cK, QP, key, kb, g);
            Vf[kb] = lds_frag_c(cV, QP, key, kb, g);
          }
          // 1/den, gd and B_tt of the lane's four query rows of each query tile: one 16-byte
          // read per tile and value, requested with the fragments, used through selects
          float4 ri4[2], gd4[2], bd4[2];
#pragma unroll
          for (int tt = 0; tt < 2; ++tt) {
            ri4[tt] = *reinterpret_cast<const float4*>(cI + tt * 16 + 4 * g);
            gd4[tt] = *reinterpret_cast<const float4*>(sGd + pb * C2 + tt * 16 + 4 * g);
            bd4[tt] = *reinterpret_cast<const float4*>(sBd + pb * C2 + tt * 16 + 4 * g);
          }
          __builtin_amdgcn_sched_barrier(0);
          floatx4 Aq[2], Bq[2];  // rows = queries of tile tt, column = this lane's key
#pragma unroll
          for (int tt = 0; tt < 2; ++tt) {
            Aq[tt] = Bq[tt] = floatx4{0.f, 0.f, 0.f, 0.f};
            if (tt >= kt) {
#pragma unroll
              for (int kb = 0; kb < KB; ++kb) {
                Aq[tt] = mma(lds_frag_c(cQ, QP, tt * 16 + c16, kb, g), Kf[kb], Aq[tt]);
                Bq[tt] = mma(lds_frag_c(cG, QP, tt * 16 + c16, kb, g), Vf[kb], Bq[tt]);
              }
            }
          }
          floatx4 xa[2], xb[2];
#pragma unroll
          for (int tt = 0; tt < 2; ++tt)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const bool after = tt > kt || (tt == kt && 4 * g + i > c16);
              const bool self = tt == kt && 4 * g + i == c16;
              const float ri = ri4[tt][i];
              xa[tt][i] = (after || self) ? Aq[tt][i] * ri : 0.f;
              xb[tt][i] = after ? __builtin_fmaf(Bq[tt][i], ri, gd4[tt][i]) : (self ? bd4[tt][i] : 0.f);
            }
          sAp[kt * 64 + lane] = acc_frag<true>(xa[0], xa[1]);
          sBp[kt * 64 + lane] = acc_frag<true>(xb[0], xb[1]);
        }
        if constexpr (!BIDIR) {
          meet += 4;
          mma_wave_sync(&sArrive, meet, lane, polls, hdr);
        }
        // ---- phase B: this wave's rows of dK'^T and dV^T, then the states. The k-blocks are the
        // outer loop, so every V and K' fragment is read once for both column tiles, and each
        // k-block's fragments are requested one k-block ahead (the last k-block requests the
        // operands of the closing terms); the per-accumulator MFMA order is that of the plain
        // loops (k-blocks in order, then the closing term).
        if (wave < NW) {
          float* dkb = sdK + pb * C2 * FP;
          floatx4 y[CT][2], z[CT][2];  // dK'^T and dV^T tiles (column tile ct, key tile kt)
#pragma unroll
          for (int ct = 0; ct < CT; ++ct)
#pragma unroll
            for (int kt = 0; kt < 2; ++kt) y[ct][kt] = z[ct][kt] = floatx4{0.f, 0.f, 0.f, 0.f};
          Frag<true> fv[2][2], fk[2][2];  // V and K' fragments of a k-block, by k-block parity
#pragma unroll
          for (int kt = 0; kt < 2; ++kt) {
            fv[0][kt] = lds_frag_c(cV, QP, kt * 16 + c16, 0, g);
            fk[0][kt] = lds_frag_c(cK, QP, kt * 16 + c16, 0, g);
          }
          Frag<true> qt[CT], gt[CT], bq[2], aq[2];  // operands of the closing terms
#pragma unroll
          for (int kb = 0; kb < KB; ++kb) {
            const int cur = kb & 1, nxt = cur ^ 1;
            if (kb + 1 < KB) {
#pragma unroll
              for (int kt = 0; kt < 2; ++kt) {
                fv[nxt][kt] = lds_frag_c(cV, QP, kt * 16 + c16, kb + 1, g);
                fk[nxt][kt] = lds_frag_c(cK, QP, kt * 16 + c16, kb + 1, g);
              }
            } else if constexpr (!BIDIR) {
#pragma unroll
              for (int ct = 0; ct < CT; ++ct) {
                qt[ct] = lds_frag_tr(cQ, QP, 0, wave * G::DVW + 16 * ct, lane);
                gt[ct] = lds_frag_tr(cG, QP, 0, wave * G::DVW + 16 * ct, lane);
              }
#pragma unroll
              for (int kt = 0; kt < 2; ++kt) {
                bq[kt] = sBp[kt * 64 + lane];
                aq[kt] = sAp[kt * 64 + lane];
              }
            }
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int ct = 0; ct < CT; ++ct) {
              Frag<true> ph, pl;
              split_frag<D>(PT[2 * kb][ct], PT[2 * kb + 1][ct], ph, pl);
              // the value gradient has no cancelling terms: P rounded to bf16 once is enough there
              const Frag<true> pm = acc_frag<true>(PM[2 * kb][ct], PM[2 * kb + 1][ct]);
#pragma unroll
              for (int kt = 0; kt < 2; ++kt) {
                y[ct][kt] = mma(ph, fv[cur][kt], y[ct][kt]);
                y[ct][kt] = mma(pl, fv[cur][kt], y[ct][kt]);
                z[ct][kt] = mma(pm, fk[cur][kt], z[ct][kt]);
              }
            }
          }
          // the reverse-state update's row fragments, requested while the closing terms run
          Frag<true> Hc[CT], Gc[CT], grn[2], hrn[2];
          if constexpr (!BIDIR) {
#pragma unroll
            for (int ct = 0; ct < CT; ++ct) {
              Hc[ct] = lds_frag_tr(cH, QP, 0, wave * G::DVW + 16 * ct, lane);
              Gc[ct] = lds_frag_tr(cG, QP, 0, wave * G::DVW + 16 * ct, lane);
            }
            grn[0] = lds_frag_tr_s8(cG, QP, 0, 0, lane);
            hrn[0] = lds_frag_tr_s8(cH, QP, 0, 0, lane);
          }
          __builtin_amdgcn_sched_barrier(0);
#pragma unroll
          for (int ct = 0; ct < CT; ++ct) {
            const int a0 = wave * G::DVW + 16 * ct + 4 * g;
#pragma unroll
            for (int kt = 0; kt < 2; ++kt) {
              if constexpr (!BIDIR) y[ct][kt] = mma(qt[ct], bq[kt], y[ct][kt]);
#pragma unroll
              for (int i = 0; i < 4; ++i) y[ct][kt][i] += pc[a0 + i];
              *reinterpret_cast<floatx4*>(dkb + (kt * 16 + c16) * FP + a0) = y[ct][kt];
              if constexpr (!BIDIR) z[ct][kt] = mma(gt[ct], aq[kt], z[ct][kt]);
              const int key = kt * 16 + c16;
              // keys past the segment are dropped; these 8-byte pieces of a row come from four
              // waves, so they carry the default cache policy and meet in L2 as whole lines (with
              // the streaming policy the partial lines went to memory: 1174 -> 1058 us per call
              // measured on the 16K-token backward)
              const int off = ((c * C2 + key) * D + a0) * 2;
              __builtin_amdgcn_raw_buffer_store_b64(
                  u32x2{pack_bf2(z[ct][kt][0], z[ct][kt][1]), pack_bf2(z[ct][kt][2], z[ct][kt][3])}, rdv,
                  key < nv ? off : seg_bytes, 0, 0);
            }
          }
          // P^T += G^T Q^ and P += Q^^T G (the 32 tokens are one k-block); each row tile's two
          // fragments are requested one tile ahead. Bidirectional: the states are the document's.
#pragma unroll
          for (int rt = 0; rt < (BIDIR ? 0 : RT); ++rt) {
            const int cur = rt & 1, nxt = cur ^ 1;
            if (rt + 1 < RT) {
              grn[nxt] = lds_frag_tr_s8(cG, QP, 0, 32 * ((rt + 1) / 2) + 4 * ((rt + 1) % 2), lane);
              hrn[nxt] = lds_frag_tr_s8(cH, QP, 0, 32 * ((rt + 1) / 2) + 4 * ((rt + 1) % 2), lane);
            }
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int ct = 0; ct < CT; ++ct) {
              PT[rt][ct] = mma(grn[cur], Hc[ct], PT[rt][ct]);
              PM[rt][ct] = mma(hrn[cur], Gc[ct], PM[rt][ct]);
            }
          }
        }
        if (!BIDIR && wave == 0) {  // p after this sub-chunk, into the other parity: p += Q^^T (gd den)
          Frag<true> w_hi, w_lo;
          token_col_frags(sW + pb * C2, 0, g, w_hi, w_lo);
          float* pn = sP + ((j + 1) & 1) * D;
          // every row tile's fragment and old p value requested together
          Frag<true> hrs[RT];
          float pold[RT];
#pragma unroll
          for (int rt = 0; rt < RT; ++rt) {
            hrs[rt] = lds_frag_tr(cH, QP, 0, 16 * rt, lane);
            pold[rt] = pc[rt * 16 + 4 * g + (c16 & 3)];
          }
          __builtin_amdgcn_sched_barrier(0);
#pragma unroll
          for (int rt = 0; rt < RT; ++rt) {
            floatx4 pv = mma(hrs[rt], w_hi, floatx4{0.f, 0.f, 0.f, 0.f});
            pv = mma(hrs[rt], w_lo, pv);
            if (c16 < 4) pn[rt * 16 + 4 * g + c16] = pold[rt] + pv[c16];
          }
        }
      }
      __syncthreads();  // Y
    }
  }
  // RMSNorm-weight partials of k from the two backward-mapper waves
  __syncthreads();  // every wave is done with LDS
  if (wave >= 6) {
    const int m = tid & 7;
#pragma unroll
    for (int e = 0; e < E; ++e) {
#pragma unroll
      for (int o = 8; o < 64; o <<= 1) {
        dg1[e] += __shfl_xor(dg1[e], o);
        dg2[e] += __shfl_xor(dg2[e], o);
      }
    }
    if (lane < 8) {
#pragma unroll
      for (int e = 0; e < E; ++e) {
        sdK[(wave - 6) * D + m * E + e] = dg1[e];
        sdK[(wave - 6) * D + G::HALF + m * E + e] = dg2[e];
      }
    }
  }
  __syncthreads();
  float* dst = dg_part + ((size_t)seg * H + h) * 2 * D + D;
  for (int i = tid; i < D; i += 512) dst[i] = sdK[i] + sdK[D + i];
}

// ----------------------------------------------------------------------------------------
// bwd_dgamma: RMSNorm-weight gradients, the per-segment partials summed in segment order
// (deterministic): part[(seg H + h) 2D + j] (q: j < D, k: D + j).

__global__ void bwd_dgamma_kernel(const float* __restrict__ part, const int32_t* __restrict__ nseg, int n_seg_max,
                                  int H, int D, float* __restrict__ dgq, float* __restrict__ dgk,
                                  const uint32_t* __restrict__ hdr) {
  const int h = blockIdx.x, j = threadIdx.x;
  if (j >= 2 * D || !bwd_go(hdr)) return;
  const int n = min(*nseg, n_seg_max);
  float acc = 0.f;
  for (int s = 0; s < n; ++s) acc += part[((size_t)s * H + h) * 2 * D + j];
  if (j < D) {
    if (dgq != nullptr) dgq[(size_t)h * D + j] = acc;
  } else if (dgk != nullptr) {
    dgk[(size_t)h * D + j - D] = acc;
  }
}

// ----------------------------------------------------------------------------------------
// Generic backward: fp32 activations in both modes (bf16 runs the warp-specialised sweeps
// above, causal and bidirectional). Same formulas as the sweeps
// (RLA page §4.2): with g = dL/dout, per query t the forward quantities are formed again,
//   causal:         den_t = q'_t . z_prev + sum_{i<=t} a_ti + eps,
//                   g . num_t = q'_t . (S_prev g_t) + sum_{i<=t} a_ti (g_t . v_i)
//   bidirectional:  den_t = q'_t . z_doc + eps,  g . num_t = q'_t . (S_doc g_t)
// (a_ti = the score rounded to the element type, as the forward uses it), gd_t = -(g . num_t) /
// den_t^2, and
//   dq'_t = (S g_t) / den_t + gd_t z + [causal] sum_{i<=t} k'_i B_ti,  B_ti = (g_t . v_i) / den_t
//           + gd_t, with the self weight B_tt formed without its cancelling O(1) terms
//   dk'_i = P v_i + p + [causal] sum_{t>=i} q'_t B_ti,  dv_i = P^T k'_i + [causal] sum_{t>=i}
//           (a_ti / den_t) g_t
// where P = sum_t Q^_t g_t^T, p = sum_t Q^_t (gd den)_t, Q^ = q'/den rounded to the element
// type, summed over the later tokens of the document (causal: per segment in the dq kernel,
// over the later segments by the suffix scan, over the later blocks in the dk/dv kernel) or
// over the whole document (bidirectional: the total scan). 4 waves, blocks of 32 tokens,
// lanes 0..127 map the query side (q, dout), lanes 128..255 the key side (k, v); states in
// accumulators (the dq kernel holds S^T, whose tiles serve S g directly; the dk/dv kernel P
// and P^T); bf16 states enter the products that can cancel (S g, P v) as value + remainder.

constexpr int kTB = 32;  // tokens per block of the generic backward

// Fragment of the transposed view of a row-major LDS array [k][n] (pitch in elements): lane
// (c16, g) gets [k0 + 4g + j][n0 + c16] and [k0 + 16 + 4g + j][n0 + c16], j < 4 (the slot
// order of lds_frag): the transposing LDS read for bf16, eight reads for fp32.
template <bool BF>
__device__ __forceinline__ Frag<BF> lds_frag_t(const typename Elem<BF>::St* base, int pitch, int k0, int n0,
                                               int lane) {
  if constexpr (BF) {
    return lds_frag_tr(base, pitch, k0, n0, lane);
  } else {
    const int c16 = lane & 15, g = lane >> 4;
    Frag<false> f;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      f.v[j] = base[(k0 + 4 * g + j) * pitch + n0 + c16];
      f.v[4 + j] = base[(k0 + 16 + 4 * g + j) * pitch + n0 + c16];
    }
    return f;
  }
}

// The same slots scaled per token (slot token k0 + 4g + j, k0 + 16 + 4g + j) by w[token] and
// rounded to the element type: the Q^ = q'/den operand from the q' rows.
template <bool BF>
__device__ __forceinline__ Frag<BF> scale_slots(Frag<BF> f, const float* w, int k0, int lane) {
  const int g = lane >> 4;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const float s = w[k0 + (j >> 2) * 16 + 4 * g + (j & 3)];
    if constexpr (BF) f.v[j] = static_cast<__bf16>(static_cast<float>(f.v[j]) * s);
    else f.v[j] = f.v[j] * s;
  }
  return f;
}

// An fp32 accumulator pair (rows 0..15 and 16..31 of a k-block) as an MFMA operand: bf16 value
// and remainder (two products), fp32 exact (one).
template <bool BF>
struct OpPair {
  Frag<BF> hi, lo;
};
template <bool BF, int D>
__device__ __forceinline__ OpPair<BF> op_pair(floatx4 a, floatx4 b) {
  OpPair<BF> r;
  if constexpr (BF) split_frag<D>(a, b, r.hi, r.lo);
  else r.hi = acc_frag_f(a, b);
  return r;
}
template <bool BF>
__device__ __forceinline__ floatx4 mma_pair(const OpPair<BF>& a, const Frag<BF>& b, floatx4 c) {
  c = mma(a.hi, b, c);
  if constexpr (BF) c = mma(a.lo, b, c);
  return c;
}

// Operand whose every column holds w[token] (slot order), as an exact pair for fp32 or a bf16
// value + remainder pair.
template <bool BF>
__device__ __forceinline__ OpPair<BF> token_cols(const float* w, int lane) {
  OpPair<BF> r;
  const int g = lane >> 4;
  if constexpr (BF) {
    token_col_frags(w, 0, g, r.hi, r.lo);
  } else {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      r.hi.v[j] = w[4 * g + j];
      r.hi.v[4 + j] = w[16 + 4 * g + j];
    }
  }
  return r;
}

// Map backward of the lane's two tokens for either element type (see map_backward): dx' from
// fp32 rows `dxp`, the pre-activation formed again exactly as the forward forms it (gamma,
// in-chunk angle rows lo_base[t0 + tok], chunk row hi_row), the weight gradient accumulated
// in dg1 / dg2, dx rounded to the element type in the lane's raw layout.
template <bool BF, int D>
__device__ __forceinline__ void map_backward_g(const Raw<BF, D>& r, Raw<BF, D>& dx, const float* dxp, int fp,
                                               const float* gamma, const float2* lo_base, const float2* hi_row,
                                               float rms_eps, int t0, int m, float (&dg1)[Geo<BF, D>::E],
                                               float (&dg2)[Geo<BF, D>::E]) {
  using G = Geo<BF, D>;
  constexpr int E = G::E;
#pragma unroll
  for (int tok = 0; tok < 2; ++tok) {
    const float inv = rms_inv<BF, D>(r, tok, rms_eps);
    const float2* lo = lo_base + (t0 + tok) * G::HALF;
    float dy1[E], dy2[E];
    float T = 0.f;
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const int j = m * E + e;
      const float2 cs = angle_sum(hi_row[j], lo[j]);
      const float x1 = r.get(tok, 0, e), x2 = r.get(tok, 1, e);
      float u1, u2;
      rope_pair(x1, x2, inv, gamma[j], gamma[j + G::HALF], cs, u1, u2);
      const float d1 = u1 > 0.f ? dxp[(t0 + tok) * fp + j] : 0.f;
      const float d2 = u2 > 0.f ? dxp[(t0 + tok) * fp + G::HALF + j] : 0.f;
      dy1[e] = __builtin_fmaf(d1, cs.x, d2 * cs.y);  // inverse rotation
      dy2[e] = __builtin_fmaf(d2, cs.x, -(d1 * cs.y));
      T = __builtin_fmaf(gamma[j] * dy1[e], x1, T);
      T = __builtin_fmaf(gamma[j + G::HALF] * dy2[e], x2, T);
      dg1[e] = __builtin_fmaf(dy1[e], x1 * inv, dg1[e]);
      dg2[e] = __builtin_fmaf(dy2[e], x2 * inv, dg2[e]);
    }
    T = sum8(T);
    const float coef = inv * inv * inv * T * (1.0f / D);
#pragma unroll
    for (int e = 0; e < E; e += 2) {
      const int j = m * E + e;
      const float a0 = __builtin_fmaf(inv * gamma[j], dy1[e], -(coef * r.get(tok, 0, e)));
      const float a1 = __builtin_fmaf(inv * gamma[j + 1], dy1[e + 1], -(coef * r.get(tok, 0, e + 1)));
      const float b0 = __builtin_fmaf(inv * gamma[j + G::HALF], dy2[e], -(coef * r.get(tok, 1, e)));
      const float b1 = __builtin_fmaf(inv * gamma[j + G::HALF + 1], dy2[e + 1], -(coef * r.get(tok, 1, e + 1)));
      if constexpr (BF) {
        dx.w[tok][0][e >> 1] = pack_bf2(a0, a1);
        dx.w[tok][1][e >> 1] = pack_bf2(b0, b1);
      } else {
        dx.w[tok][0][e] = __float_as_uint(a0);
        dx.w[tok][0][e + 1] = __float_as_uint(a1);
        dx.w[tok][1][e] = __float_as_uint(b0);
        dx.w[tok][1][e + 1] = __float_as_uint(b1);
      }
    }
  }
}

// The lane's two tokens (rows t0, t0 + 1, first nv rows valid) to global memory.
template <bool BF, int D>
__device__ __forceinline__ void store_raw(const Raw<BF, D>& x, typename Elem<BF>::St* base, int t0, int m, int nv) {
  using G = Geo<BF, D>;
#pragma unroll
  for (int tok = 0; tok < 2; ++tok)
    if (t0 + tok < nv)
#pragma unroll
      for (int hh = 0; hh < 2; ++hh)
        copy_bytes<G::E * G::ES>(base + (size_t)(t0 + tok) * D + hh * G::HALF + m * G::E, x.w[tok][hh]);
}

// The segment record's S (or P) as transposed tiles: tile (rt, ct) of wave w, lane (c16, g),
// row i holds M[a][c] with a = w DVW + 16 ct + c16 and c = 16 rt + 4g + i, gathered from the
// fragment-native record.
template <bool BF, int D>
__device__ __forceinline__ void load_rec_transposed(const float* rec, int w, int lane,
                                                    floatx4 (&T)[Geo<BF, D>::RT][Geo<BF, D>::CT]) {
  using G = Geo<BF, D>;
  const int c16 = lane & 15, g = lane >> 4;
#pragma unroll
  for (int rt = 0; rt < G::RT; ++rt)
#pragma unroll
    for (int ct = 0; ct < G::CT; ++ct) {
      const int a = w * G::DVW + 16 * ct + c16;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int c = 16 * rt + 4 * g + i;
        const int w2 = c / G::DVW, ct2 = (c % G::DVW) / 16, l2 = 16 * ((a % 16) / 4) + c % 16;
        T[rt][ct][i] = rec[rec_frag<BF, D>(w2, a / 16, ct2, l2) + a % 4];
      }
    }
}

// RMSNorm-weight partials of the 128 lanes of one side (two waves): lanes sharing m, then the
// waves, into dst[0 .. D). `red` holds 2 D floats of LDS; every thread calls it.
template <int D, int E>
__device__ __forceinline__ void write_dgamma(float (&dg1)[E], float (&dg2)[E], int side_wave, bool mine, int lane,
                                             float* red, float* dst) {
  const int m = lane & 7;
  if (mine) {
#pragma unroll
    for (int e = 0; e < E; ++e) {
#pragma unroll
      for (int o = 8; o < 64; o <<= 1) {
        dg1[e] += __shfl_xor(dg1[e], o);
        dg2[e] += __shfl_xor(dg2[e], o);
      }
    }
    if (lane < 8) {
#pragma unroll
      for (int e = 0; e < E; ++e) {
        red[side_wave * D + m * E + e] = dg1[e];
        red[side_wave * D + D / 2 + m * E + e] = dg2[e];
      }
    }
  }
  __syncthreads();
  for (int i = threadIdx.x; i < D; i += NT) dst[i] = red[i] + red[D + i];
}

template <bool BF, int D, bool CAUSAL>
__global__ __launch_bounds__(NT, 1) void gbwd_dq_kernel(
    const typename Elem<BF>::St* __restrict__ q, const typename Elem<BF>::St* __restrict__ k,
    const typename Elem<BF>::St* __restrict__ v, const typename Elem<BF>::St* __restrict__ dout,
    const float* __restrict__ gamma_q, const float* __restrict__ gamma_k, const int32_t* __restrict__ tab,
    const int32_t* __restrict__ nseg, const float2* __restrict__ rope_lo, const float2* __restrict__ rope_hi,
    const float* __restrict__ states, typename Elem<BF>::St* __restrict__ dq, float* __restrict__ den_out,
    float* __restrict__ gd_out, float* __restrict__ bd_out, float* __restrict__ pstates,
    float* __restrict__ dg_part, int H, int L, float rms_eps, float eps, const uint32_t* __restrict__ hdr,
    TabLimits lim) {
  using G = Geo<BF, D>;
  using St = typename G::St;
  using EL = Elem<BF>;
  constexpr int RT = G::RT, CT = G::CT, KB = G::KB, E = G::E, NW = G::NW, P = G::ROWP, FP = D + 4;
  constexpr int ZR = RT >= 4 ? RT / 4 : 1;  // row tiles of p per wave
  __shared__ __attribute__((aligned(16))) St sQ[kTB * P];  // q'
  __shared__ __attribute__((aligned(16))) St sG[kTB * P];  // dout
  __shared__ __attribute__((aligned(16))) St sK[CAUSAL ? kTB * P : 8];
  __shared__ __attribute__((aligned(16))) St sV[CAUSAL ? kTB * P : 8];
  __shared__ __attribute__((aligned(16))) float sdQ[kTB * FP];  // dq' rows; also the weight partials
  __shared__ float sZ[2 * D];  // z before the block, by block parity
  __shared__ float sQz[kTB], sGs[4 * kTB], sInv[kTB], sGd[kTB], sBtt[kTB], sW[kTB];
  __shared__ float sRx[kTB], sGx[kTB], sAtt[kTB], sGvt[kTB];
  __shared__ floatx4 sGV[3 * 64];  // causal: g.v tiles (query tile, key tile) (0,0), (1,0), (1,1)

  const int seg = blockIdx.x, h = blockIdx.y;
  if (!bwd_go(hdr) || seg >= *nseg) return;
  const SegInfo si = read_seg_clamped(tab, seg, L, lim);
  if (si.len == 0) return;  // only a corrupted table has empty segments
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int c16 = lane & 15, g = lane >> 4;
  const int side = tid >> 7, t0 = 2 * ((tid & 127) >> 3), m = tid & 7;
  const size_t tok0 = ((size_t)si.row * H + h) * (size_t)L + si.start;
  const float* gq = gamma_q + (size_t)h * D;
  const float* gk = gamma_k + (size_t)h * D;
  const int wv = wave < NW ? wave : 0;  // waves without state columns keep a harmless copy
  const float* rec = states + ((size_t)seg * H + h) * (size_t)(D * D + D);

  floatx4 ST[RT][CT];  // S^T: rows = value dims, columns = this wave's key dims
  load_rec_transposed<BF, D>(rec, wv, lane, ST);
  if (tid < D) sZ[tid] = rec[D * D + tid];
  floatx4 Pt[RT][CT];  // sum_t Q^_t g_t^T: rows = query dims a, columns = this wave's value dims
  floatx4 pc[ZR];      // sum_t Q^_t (gd den)_t: row tiles wave ZR + z, every column
#pragma unroll
  for (int rt = 0; rt < RT; ++rt)
#pragma unroll
    for (int ct = 0; ct < CT; ++ct) Pt[rt][ct] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int z = 0; z < ZR; ++z) pc[z] = floatx4{0.f, 0.f, 0.f, 0.f};
  float dg1[E], dg2[E];
#pragma unroll
  for (int e = 0; e < E; ++e) dg1[e] = dg2[e] = 0.f;
  Raw<BF, D> rq;  // query-side lanes: raw q of their tokens (for the map backward)

  const int nblk = (si.len + kTB - 1) / kTB;
  for (int blk = 0; blk < nblk; ++blk) {
    const int nv = min(kTB, si.len - blk * kTB);
    const int par = blk & 1;
    const size_t row0 = tok0 + (size_t)blk * kTB;  // first token row of the block
    const float2* hr = rope_hi + (size_t)(si.hirow + (blk >> 1)) * G::HALF;
    const float2* lob = rope_lo + (size_t)par * kTB * G::HALF;
    const float* zc = sZ + (CAUSAL ? par * D : 0);  // bidirectional: the document's z throughout
    __syncthreads();  // the previous block's LDS reads are done

    // ---- map: query side q', dout rows, q'.z; key side (causal) k', v rows
    if (side == 0) {
      Raw<BF, D> rg, oq;
      load_raw<BF, D>(rq, q + row0 * D, t0, m, nv);
      load_raw<BF, D>(rg, dout + row0 * D, t0, m, nv);
      feature_map_pair<BF, D>(rq, oq, gq, lob, hr, t0, m, rms_eps);
      store_rows<BF, D>(sQ, oq, t0, m);
      store_rows<BF, D>(sG, rg, t0, m);
#pragma unroll
      for (int tok = 0; tok < 2; ++tok) {
        float pz = 0.f;
#pragma unroll
        for (int e = 0; e < E; ++e) {
          const int j = m * E + e;
          pz = __builtin_fmaf(oq.get(tok, 0, e), zc[j], pz);
          pz = __builtin_fmaf(oq.get(tok, 1, e), zc[j + G::HALF], pz);
        }
        pz = sum8(pz);
        if (m == 0) sQz[t0 + tok] = pz;
      }
    } else if constexpr (CAUSAL) {
      Raw<BF, D> rk, rv, ok;
      load_raw<BF, D>(rk, k + row0 * D, t0, m, nv);
      load_raw<BF, D>(rv, v + row0 * D, t0, m, nv);
      feature_map_pair<BF, D>(rk, ok, gk, lob, hr, t0, m, rms_eps);
      store_rows<BF, D>(sK, ok, t0, m);
      store_rows<BF, D>(sV, rv, t0, m);
    }
    __syncthreads();

    // ---- A: Y = S G^T for this wave's key dims and its part of q'.(S g); causal score tiles
    floatx4 Y[CT][2];
    if (wave < NW) {
#pragma unroll
      for (int ct = 0; ct < CT; ++ct) {
        OpPair<BF> Sa[KB];
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) Sa[kb] = op_pair<BF, D>(ST[2 * kb][ct], ST[2 * kb + 1][ct]);
#pragma unroll
        for (int tt = 0; tt < 2; ++tt) {
          floatx4 y = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int kb = 0; kb < KB; ++kb) y = mma_pair<BF>(Sa[kb], lds_frag<BF>(sG, P, 16 * tt + c16, kb, g), y);
          Y[ct][tt] = y;  // lane (t, g): rows a = wave DVW + 16 ct + 4g + i of query 16 tt + t
        }
      }
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) {
        float part = 0.f;
#pragma unroll
        for (int ct = 0; ct < CT; ++ct)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            part = __builtin_fmaf(EL::to_f(sQ[(16 * tt + c16) * P + wave * G::DVW + 16 * ct + 4 * g + i]),
                                  Y[ct][tt][i], part);
        part = sum_rows4(part);
        if (g == 0) sGs[wave * kTB + 16 * tt + c16] = part;
      }
    }
    if constexpr (CAUSAL) {
      if (wave < 2) {  // query tile tt = wave against key tiles kt <= tt
        const int tt = wave;
        Frag<BF> Qf[KB], Gf[KB];
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) {
          Qf[kb] = lds_frag<BF>(sQ, P, 16 * tt + c16, kb, g);
          Gf[kb] = lds_frag<BF>(sG, P, 16 * tt + c16, kb, g);
        }
        float rx = 0.f, gx = 0.f, aself = 0.f, gvself = 0.f;
#pragma unroll
        for (int kt = 0; kt < 2; ++kt) {
          if (kt > tt) continue;
          floatx4 s = floatx4{0.f, 0.f, 0.f, 0.f}, gv = s;
#pragma unroll
          for (int kb = 0; kb < KB; ++kb) {
            s = mma(lds_frag<BF>(sK, P, 16 * kt + c16, kb, g), Qf[kb], s);
            gv = mma(lds_frag<BF>(sV, P, 16 * kt + c16, kb, g), Gf[kb], gv);
          }
          // lane (t, g): query 16 tt + t, keys 16 kt + 4g + i
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int key = 4 * g + i;
            if (kt == tt && key > c16) {  // a key after the query
              gv[i] = 0.f;
              continue;
            }
            const float a = EL::to_f(EL::from_f(s[i]));  // the weight the forward uses
            if (kt == tt && key == c16) {
              aself = a;
              gvself = gv[i];
            } else {
              rx += a;
              gx = __builtin_fmaf(a, gv[i], gx);
            }
          }
          sGV[(tt == 0 ? 0 : 1 + kt) * 64 + lane] = gv;
        }
        rx = sum_rows4(rx);
        gx = sum_rows4(gx);
        aself = sum_rows4(aself);
        gvself = sum_rows4(gvself);
        if (g == 0) {
          const int t = 16 * tt + c16;
          sRx[t] = rx;
          sGx[t] = gx;
          sAtt[t] = aself;
          sGvt[t] = gvself;
        }
      }
    }
    __syncthreads();

    // ---- B: per token den, gd, the self weight B_tt (sums without the self term first), and the
    // planes the dk/dv kernel reads
    if (tid < kTB) {
      const int t = tid;
      float gs = 0.f;
#pragma unroll
      for (int w = 0; w < NW; ++w) gs += sGs[w * kTB + t];
      float den, gd, btt = 0.f;
      if constexpr (CAUSAL) {
        const float denx = sQz[t] + sRx[t] + eps;  // without the self term
        den = denx + sAtt[t];
        const float gnx = gs + sGx[t];
        const float gn = __builtin_fmaf(sAtt[t], sGvt[t], gnx);
        const float inv = 1.0f / den;
        gd = -gn * inv * inv;
        btt = __builtin_fmaf(sGvt[t], denx, -gnx) * inv * inv;
        if (t < nv) {
          den_out[row0 + t] = den;
          gd_out[row0 + t] = gd;
          bd_out[row0 + t] = btt;
        }
      } else {
        den = sQz[t] + eps;
        const float inv = 1.0f / den;
        gd = -gs * inv * inv;
      }
      sInv[t] = 1.0f / den;
      sGd[t] = gd;
      sBtt[t] = btt;
      sW[t] = t < nv ? gd * den : 0.f;
    }
    __syncthreads();

    // ---- C: dq' tiles; then the reverse-state totals and (causal) the state update
    floatx4 dQ[CT][2];
    if (wave < NW) {
      Frag<BF> Kt[CT];  // K'^T rows a, keys of the block (causal)
      if constexpr (CAUSAL) {
#pragma unroll
        for (int ct = 0; ct < CT; ++ct) Kt[ct] = lds_frag_t<BF>(sK, P, 0, wave * G::DVW + 16 * ct, lane);
      }
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) {
        const int t = 16 * tt + c16;
        const float inv = sInv[t], gd = sGd[t];
        Frag<BF> bf;  // B^T operand (keys x this lane's query t), causal
        if constexpr (CAUSAL) {
          floatx4 bt[2];
#pragma unroll
          for (int kt = 0; kt < 2; ++kt) {
            bt[kt] = floatx4{0.f, 0.f, 0.f, 0.f};
            if (kt <= tt) {
              const floatx4 gv = sGV[(tt == 0 ? 0 : 1 + kt) * 64 + lane];
#pragma unroll
              for (int i = 0; i < 4; ++i) {
                const int key = 4 * g + i;
                float b = __builtin_fmaf(gv[i], inv, gd);
                if (kt == tt && key == c16) b = sBtt[t];
                if (kt == tt && key > c16) b = 0.f;
                bt[kt][i] = b;
              }
            }
          }
          bf = acc_frag<BF>(bt[0], bt[1]);
        }
#pragma unroll
        for (int ct = 0; ct < CT; ++ct) {
          const int a0 = wave * G::DVW + 16 * ct + 4 * g;
          floatx4 o;
#pragma unroll
          for (int i = 0; i < 4; ++i) o[i] = __builtin_fmaf(Y[ct][tt][i], inv, zc[a0 + i] * gd);
          if constexpr (CAUSAL) o = mma(Kt[ct], bf, o);
          dQ[ct][tt] = o;
        }
      }
      // P += Q^^T G and p += Q^^T (gd den) over the block's queries
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) {
        const Frag<BF> qh = scale_slots<BF>(lds_frag_t<BF>(sQ, P, 0, 16 * rt, lane), sInv, 0, lane);
#pragma unroll
        for (int ct = 0; ct < CT; ++ct)
          Pt[rt][ct] = mma(qh, lds_frag_t<BF>(sG, P, 0, wave * G::DVW + 16 * ct, lane), Pt[rt][ct]);
      }
      if (wave * ZR < RT) {
        const OpPair<BF> wcol = token_cols<BF>(sW, lane);
#pragma unroll
        for (int z = 0; z < ZR; ++z) {
          const Frag<BF> qh = scale_slots<BF>(lds_frag_t<BF>(sQ, P, 0, 16 * (wave * ZR + z), lane), sInv, 0, lane);
          pc[z] = mma(qh, wcol.hi, pc[z]);
          if constexpr (BF) pc[z] = mma(qh, wcol.lo, pc[z]);
        }
      }
      if constexpr (CAUSAL) {  // S^T += V^T K'
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
          const Frag<BF> vt = lds_frag_t<BF>(sV, P, 0, 16 * rt, lane);
#pragma unroll
          for (int ct = 0; ct < CT; ++ct)
            ST[rt][ct] = mma(vt, lds_frag_t<BF>(sK, P, 0, wave * G::DVW + 16 * ct, lane), ST[rt][ct]);
        }
      }
    }
    if constexpr (CAUSAL) {  // z for the next block (the other parity): z + the column sums of K'
      for (int a = tid; a < D; a += NT) {
        float cs = 0.f;
        for (int i = 0; i < kTB; ++i) cs += EL::to_f(sK[i * P + a]);
        sZ[(par ^ 1) * D + a] = zc[a] + cs;
      }
    }
    if (wave < NW) {
#pragma unroll
      for (int ct = 0; ct < CT; ++ct)
#pragma unroll
        for (int tt = 0; tt < 2; ++tt)
          *reinterpret_cast<floatx4*>(&sdQ[(16 * tt + c16) * FP + wave * G::DVW + 16 * ct + 4 * g]) = dQ[ct][tt];
    }
    __syncthreads();

    // ---- D: map backward of q
    if (side == 0) {
      Raw<BF, D> dx;
      map_backward_g<BF, D>(rq, dx, sdQ, FP, gq, lob, hr, rms_eps, t0, m, dg1, dg2);
      store_raw<BF, D>(dx, dq + row0 * D, t0, m, nv);
    }
  }
  __syncthreads();

  // the segment's reverse-state totals (fragment-native records; p where a record keeps z)
  float* prec = pstates + ((size_t)seg * H + h) * (size_t)(D * D + D);
  if (wave < NW) {
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
      for (int ct = 0; ct < CT; ++ct)
        *reinterpret_cast<floatx4*>(prec + rec_frag<BF, D>(wave, rt, ct, lane)) = Pt[rt][ct];
  }
  if (wave * ZR < RT && c16 < 4) {  // every column of pc holds the sums of rows 16 tile + 4g + i
#pragma unroll
    for (int z = 0; z < ZR; ++z) prec[D * D + (wave * ZR + z) * 16 + 4 * g + c16] = pc[z][c16];
  }
  write_dgamma<D, E>(dg1, dg2, wave, side == 0, lane, sdQ, dg_part + ((size_t)seg * H + h) * 2 * D);
}

template <bool BF, int D, bool CAUSAL>
__global__ __launch_bounds__(NT, 1) void gbwd_dkv_kernel(
    const typename Elem<BF>::St* __restrict__ q, const typename Elem<BF>::St* __restrict__ k,
    const typename Elem<BF>::St* __restrict__ v, const typename Elem<BF>::St* __restrict__ dout,
    const float* __restrict__ gamma_q, const float* __restrict__ gamma_k, const int32_t* __restrict__ tab,
    const int32_t* __restrict__ nseg, const float2* __restrict__ rope_lo, const float2* __restrict__ rope_hi,
    const float* __restrict__ pstates, const float* __restrict__ den, const float* __restrict__ gdp,
    const float* __restrict__ bdp, typename Elem<BF>::St* __restrict__ dk, typename Elem<BF>::St* __restrict__ dv,
    float* __restrict__ dg_part, int H, int L, float rms_eps, const uint32_t* __restrict__ hdr, TabLimits lim) {
  using G = Geo<BF, D>;
  using St = typename G::St;
  using EL = Elem<BF>;
  constexpr int RT = G::RT, CT = G::CT, KB = G::KB, E = G::E, NW = G::NW, P = G::ROWP, FP = D + 4;
  __shared__ __attribute__((aligned(16))) St sK[kTB * P];  // k'
  __shared__ __attribute__((aligned(16))) St sV[kTB * P];  // v
  __shared__ __attribute__((aligned(16))) St sQ[CAUSAL ? kTB * P : 8];  // q'
  __shared__ __attribute__((aligned(16))) St sG[CAUSAL ? kTB * P : 8];  // dout
  __shared__ __attribute__((aligned(16))) float sdK[kTB * FP];  // dk' rows; also the weight partials
  __shared__ float sP[2 * D];  // p after the block (causal: over the later tokens), by block parity
  __shared__ float sI[kTB], sGd[kTB], sBd[kTB], sW[kTB];
  __shared__ Frag<BF> sAop[2 * 64], sBop[2 * 64];  // causal, per key tile: A/den and B (queries x keys)

  const int seg = blockIdx.x, h = blockIdx.y;
  if (!bwd_go(hdr) || seg >= *nseg) return;
  const SegInfo si = read_seg_clamped(tab, seg, L, lim);
  if (si.len == 0) return;  // only a corrupted table has empty segments
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int c16 = lane & 15, g = lane >> 4;
  const int side = tid >> 7, t0 = 2 * ((tid & 127) >> 3), m = tid & 7;
  const size_t tok0 = ((size_t)si.row * H + h) * (size_t)L + si.start;
  const float* gq = gamma_q + (size_t)h * D;
  const float* gk = gamma_k + (size_t)h * D;
  const int wv = wave < NW ? wave : 0;
  const float* rec = pstates + ((size_t)seg * H + h) * (size_t)(D * D + D);

  floatx4 Pm[RT][CT];  // P: rows = query dims a, columns = this wave's value dims (the record's map)
  floatx4 PT[RT][CT];  // P^T: rows = value dims, columns = this wave's query dims
#pragma unroll
  for (int rt = 0; rt < RT; ++rt)
#pragma unroll
    for (int ct = 0; ct < CT; ++ct)
      Pm[rt][ct] = *reinterpret_cast<const floatx4*>(rec + rec_frag<BF, D>(wv, rt, ct, lane));
  load_rec_transposed<BF, D>(rec, wv, lane, PT);
  if (tid < D) sP[tid] = rec[D * D + tid];
  float dg1[E], dg2[E];
#pragma unroll
  for (int e = 0; e < E; ++e) dg1[e] = dg2[e] = 0.f;
  Raw<BF, D> rk;  // key-side lanes: raw k of their tokens (for the map backward)

  const int nblk = (si.len + kTB - 1) / kTB;
  for (int j = 0; j < nblk; ++j) {
    const int blk = CAUSAL ? nblk - 1 - j : j;  // causal: from the last block back
    const int nv = min(kTB, si.len - blk * kTB);
    const int par = j & 1;
    const size_t row0 = tok0 + (size_t)blk * kTB;
    const float2* hr = rope_hi + (size_t)(si.hirow + (blk >> 1)) * G::HALF;
    const float2* lob = rope_lo + (size_t)(blk & 1) * kTB * G::HALF;
    const float* pcur = sP + par * D;
    __syncthreads();  // the previous block's LDS reads are done

    // ---- map: key side k', v rows; query side (causal) q', dout rows and the per-token values
    if (side == 1) {
      Raw<BF, D> rv, ok;
      load_raw<BF, D>(rk, k + row0 * D, t0, m, nv);
      load_raw<BF, D>(rv, v + row0 * D, t0, m, nv);
      feature_map_pair<BF, D>(rk, ok, gk, lob, hr, t0, m, rms_eps);
      store_rows<BF, D>(sK, ok, t0, m);
      store_rows<BF, D>(sV, rv, t0, m);
    } else if constexpr (CAUSAL) {
      Raw<BF, D> rq, rg, oq;
      load_raw<BF, D>(rq, q + row0 * D, t0, m, nv);
      load_raw<BF, D>(rg, dout + row0 * D, t0, m, nv);
      feature_map_pair<BF, D>(rq, oq, gq, lob, hr, t0, m, rms_eps);
      store_rows<BF, D>(sQ, oq, t0, m);
      store_rows<BF, D>(sG, rg, t0, m);
      if (m < 2) {
        const int t = t0 + m;
        const bool in = t < nv;
        const float dn = in ? den[row0 + t] : 1.f, gd = in ? gdp[row0 + t] : 0.f;
        sI[t] = 1.0f / dn;
        sGd[t] = gd;
        sBd[t] = in ? bdp[row0 + t] : 0.f;
        sW[t] = gd * dn;
      }
    }
    __syncthreads();

    // ---- A (causal): per key tile kt = wave, the operands A/den and B over the block's queries
    if constexpr (CAUSAL) {
      if (wave < 2) {
        const int kt = wave;
        Frag<BF> Kf[KB], Vf[KB];
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) {
          Kf[kb] = lds_frag<BF>(sK, P, 16 * kt + c16, kb, g);
          Vf[kb] = lds_frag<BF>(sV, P, 16 * kt + c16, kb, g);
        }
        floatx4 ad[2], bd[2];
#pragma unroll
        for (int tt = 0; tt < 2; ++tt) {
          ad[tt] = bd[tt] = floatx4{0.f, 0.f, 0.f, 0.f};
          if (tt < kt) continue;  // queries before the keys
          floatx4 s = floatx4{0.f, 0.f, 0.f, 0.f}, gv = s;
#pragma unroll
          for (int kb = 0; kb < KB; ++kb) {
            s = mma(lds_frag<BF>(sQ, P, 16 * tt + c16, kb, g), Kf[kb], s);
            gv = mma(lds_frag<BF>(sG, P, 16 * tt + c16, kb, g), Vf[kb], gv);
          }
          // lane (i, g): key 16 kt + i, queries t = 16 tt + 4g + r
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int t = 16 * tt + 4 * g + r;
            if (tt == kt && 4 * g + r < c16) continue;  // a query before the key
            const float a = EL::to_f(EL::from_f(s[r]));  // the weight the forward uses
            ad[tt][r] = a * sI[t];
            bd[tt][r] = (tt == kt && 4 * g + r == c16) ? sBd[t] : __builtin_fmaf(gv[r], sI[t], sGd[t]);
          }
        }
        sAop[kt * 64 + lane] = acc_frag<BF>(ad[0], ad[1]);
        sBop[kt * 64 + lane] = acc_frag<BF>(bd[0], bd[1]);
      }
      __syncthreads();
    }

    // ---- B: dk' tiles (to LDS) and dv tiles (to memory); then (causal) P, P^T and p advance
    if (wave < NW) {
#pragma unroll
      for (int ct = 0; ct < CT; ++ct) {
        const int a0 = wave * G::DVW + 16 * ct;
        OpPair<BF> PTa[KB];  // P^T pairs: rows = this wave's query dims, contraction over value dims
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) PTa[kb] = op_pair<BF, D>(PT[2 * kb][ct], PT[2 * kb + 1][ct]);
        Frag<BF> Qt;
        if constexpr (CAUSAL) Qt = lds_frag_t<BF>(sQ, P, 0, a0, lane);
#pragma unroll
        for (int kt = 0; kt < 2; ++kt) {
          floatx4 o = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int kb = 0; kb < KB; ++kb) o = mma_pair<BF>(PTa[kb], lds_frag<BF>(sV, P, 16 * kt + c16, kb, g), o);
          if constexpr (CAUSAL) o = mma(Qt, sBop[kt * 64 + lane], o);
#pragma unroll
          for (int i = 0; i < 4; ++i) o[i] += pcur[a0 + 4 * g + i];
          *reinterpret_cast<floatx4*>(&sdK[(16 * kt + c16) * FP + a0 + 4 * g]) = o;
        }
      }
#pragma unroll
      for (int ct = 0; ct < CT; ++ct) {
        const int c0 = wave * G::DVW + 16 * ct;
        Frag<BF> Pa[KB];  // P (value rows of this wave, contraction over query dims), rounded once
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) Pa[kb] = acc_frag<BF>(Pm[2 * kb][ct], Pm[2 * kb + 1][ct]);
        Frag<BF> Gt;
        if constexpr (CAUSAL) Gt = lds_frag_t<BF>(sG, P, 0, c0, lane);
#pragma unroll
        for (int kt = 0; kt < 2; ++kt) {
          floatx4 o = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int kb = 0; kb < KB; ++kb) o = mma(Pa[kb], lds_frag<BF>(sK, P, 16 * kt + c16, kb, g), o);
          if constexpr (CAUSAL) o = mma(Gt, sAop[kt * 64 + lane], o);
          const int i = 16 * kt + c16;  // key row; value columns c0 + 4g .. + 3
          if (i < nv) {
            St* dst = dv + (row0 + i) * D + c0 + 4 * g;
            if constexpr (BF) {
              *reinterpret_cast<uint2*>(dst) = make_uint2(pack_bf2(o[0], o[1]), pack_bf2(o[2], o[3]));
            } else {
              *reinterpret_cast<float4*>(dst) = make_float4(o[0], o[1], o[2], o[3]);
            }
          }
        }
      }
      if constexpr (CAUSAL) {  // P += Q^^T G and P^T += G^T Q^ over the block's queries
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
          const Frag<BF> qh = scale_slots<BF>(lds_frag_t<BF>(sQ, P, 0, 16 * rt, lane), sI, 0, lane);
          const Frag<BF> gt = lds_frag_t<BF>(sG, P, 0, 16 * rt, lane);
#pragma unroll
          for (int ct = 0; ct < CT; ++ct) {
            Pm[rt][ct] = mma(qh, lds_frag_t<BF>(sG, P, 0, wave * G::DVW + 16 * ct, lane), Pm[rt][ct]);
            PT[rt][ct] = mma(gt, scale_slots<BF>(lds_frag_t<BF>(sQ, P, 0, wave * G::DVW + 16 * ct, lane), sI, 0, lane),
                             PT[rt][ct]);
          }
        }
      }
    }
    if constexpr (CAUSAL) {  // p for the next block (the other parity): p + sum_t Q^_t (gd den)_t
      for (int a = tid; a < D; a += NT) {
        float acc = 0.f;
        for (int t = 0; t < kTB; ++t) acc = __builtin_fmaf(EL::to_f(EL::from_f(EL::to_f(sQ[t * P + a]) * sI[t])), sW[t], acc);
        sP[(par ^ 1) * D + a] = pcur[a] + acc;
      }
    } else {
      if (tid < D) sP[(par ^ 1) * D + tid] = pcur[tid];
    }
    __syncthreads();

    // ---- C: map backward of k
    if (side == 1) {
      Raw<BF, D> dx;
      map_backward_g<BF, D>(rk, dx, sdK, FP, gk, lob, hr, rms_eps, t0, m, dg1, dg2);
      store_raw<BF, D>(dx, dk + row0 * D, t0, m, nv);
    }
  }
  __syncthreads();
  write_dgamma<D, E>(dg1, dg2, wave - 2, side == 1, lane, sdK, dg_part + ((size_t)seg * H + h) * 2 * D + D);
}

template <bool BF, int D, bool CAUSAL>
hipError_t run_backward_generic(const Plan& p, const FwdArgs& a, const BwdArgs& b, hipStream_t s, hipEvent_t* ev) {
  using St = typename Elem<BF>::St;
  auto mark = [&](int i) {
    if (ev != nullptr) (void)hipEventRecord(ev[i], s);
  };
  const int fmode = CAUSAL ? SCAN_PREFIX : SCAN_TOTAL;  // what the forward's records hold
  hipError_t e = hipSuccess;
  if (b.saved == nullptr) {
    e = launch_fwd_states(p, a, s, ev, fmode);
    if (e != hipSuccess) return e;
  } else {
    mark(0);
    e = launch_saved_check(p, b.saved, a.ws, a.cu, fmode, s);
    if (e != hipSuccess) return e;
    for (int i = 1; i < 3; ++i) mark(i);
  }
  const char* fw = b.saved != nullptr ? b.saved : a.ws;
  // the whole-document reverse totals of the documents that start from the initial state
  float* ginit = b.ginit_S != nullptr || b.ginit_z != nullptr ? reinterpret_cast<float*>(a.ws + p.off_ginit) : nullptr;
  if (p.n_seg_max == 0) {
    for (int i = 3; i <= kNumBwdKernels; ++i) mark(i);
    if (ginit != nullptr) return launch_initial_grad(p, ginit, b, reinterpret_cast<const uint32_t*>(a.ws), s);
    return hipGetLastError();
  }
  uint32_t* hdr = reinterpret_cast<uint32_t*>(a.ws);
  const TabLimits lim{p.packed ? 1 : p.B, p.seg_len, p.n_hi + p.hi_off};
  const int32_t* tab = reinterpret_cast<const int32_t*>(fw + p.off_tab);
  const int32_t* nseg = reinterpret_cast<const int32_t*>(fw + p.off_nseg);
  const float2* rlo = reinterpret_cast<const float2*>(fw + p.off_rope_lo);
  const float2* rhi = reinterpret_cast<const float2*>(fw + p.off_rope_hi);
  const float* states = reinterpret_cast<const float*>(fw + p.off_states);
  float* pstates = reinterpret_cast<float*>(a.ws + p.off_pstates);
  float* den = reinterpret_cast<float*>(a.ws + p.off_den);
  float* gd = reinterpret_cast<float*>(a.ws + p.off_gd);
  float* bd = reinterpret_cast<float*>(a.ws + p.off_bd);
  float* dgp = reinterpret_cast<float*>(a.ws + p.off_dgpart);
  const St* q = static_cast<const St*>(a.q);
  const St* k = static_cast<const St*>(a.k);
  const St* v = static_cast<const St*>(a.v);
  const St* g = static_cast<const St*>(b.dout);
  const dim3 grid(p.n_seg_max, p.H);
  mark(3);
  hipLaunchKernelGGL((gbwd_dq_kernel<BF, D, CAUSAL>), grid, dim3(NT), 0, s, q, k, v, g, a.gq, a.gk, tab, nseg, rlo,
                     rhi, states, static_cast<St*>(b.dq), den, gd, bd, pstates, dgp, p.H, p.L, a.rms_eps, a.eps,
                     static_cast<const uint32_t*>(hdr), lim);
  mark(4);  // the reverse-state totals come from the dq kernel
  mark(5);
  e = launch_scan_records(p, fw, pstates, CAUSAL ? SCAN_SUFFIX : SCAN_TOTAL, hdr, s, ginit);
  if (e != hipSuccess) return e;
  if (ginit != nullptr) {
    e = launch_initial_grad(p, ginit, b, hdr, s);
    if (e != hipSuccess) return e;
  }
  mark(6);
  hipLaunchKernelGGL((gbwd_dkv_kernel<BF, D, CAUSAL>), grid, dim3(NT), 0, s, q, k, v, g, a.gq, a.gk, tab, nseg, rlo,
                     rhi, static_cast<const float*>(pstates), static_cast<const float*>(den),
                     static_cast<const float*>(gd), static_cast<const float*>(bd), static_cast<St*>(b.dk),
                     static_cast<St*>(b.dv), dgp, p.H, p.L, a.rms_eps, static_cast<const uint32_t*>(hdr), lim);
  mark(7);
  if (b.dgamma_q != nullptr || b.dgamma_k != nullptr)
    hipLaunchKernelGGL(bwd_dgamma_kernel, dim3(p.H), dim3(2 * D), 0, s, dgp, nseg, p.n_seg_max, p.H, D, b.dgamma_q,
                       b.dgamma_k, static_cast<const uint32_t*>(hdr));
  mark(8);
  return hipGetLastError();
}

template <int D, bool BIDIR>
hipError_t run_backward(const Plan& p, const FwdArgs& a, const BwdArgs& b, hipStream_t s, hipEvent_t* ev) {
  auto mark = [&](int i) {
    if (ev != nullptr) (void)hipEventRecord(ev[i], s);
  };
  // the forward's segment table, RoPE tables and state records (causal: the prefix before each
  // segment; bidirectional: the document's totals): formed again, or read from the workspace of
  // the matching forward (same plan, so the same offsets)
  const int fmode = BIDIR ? SCAN_TOTAL : SCAN_PREFIX;
  hipError_t e = hipSuccess;
  if (b.saved == nullptr) {
    e = launch_fwd_states(p, a, s, ev, fmode);
    if (e != hipSuccess) return e;
  } else {
    // the forward's plan stamp against this plan: the backward kernels run only on a match
    mark(0);
    e = launch_saved_check(p, b.saved, a.ws, a.cu, fmode, s);
    if (e != hipSuccess) return e;
    for (int i = 1; i < 3; ++i) mark(i);
  }
  uint32_t* hdr = reinterpret_cast<uint32_t*>(a.ws);
  const TabLimits lim{p.packed ? 1 : p.B, p.seg_len, p.n_hi + p.hi_off};
  const char* fw = b.saved != nullptr ? b.saved : a.ws;
  // the whole-document reverse totals of the documents that start from the initial state
  float* ginit = b.ginit_S != nullptr || b.ginit_z != nullptr ? reinterpret_cast<float*>(a.ws + p.off_ginit) : nullptr;
  if (p.n_seg_max == 0) {
    for (int i = 3; i <= kNumBwdKernels; ++i) mark(i);
    if (ginit != nullptr) return launch_initial_grad(p, ginit, b, reinterpret_cast<const uint32_t*>(a.ws), s);
    return hipGetLastError();
  }
  const int32_t* tab = reinterpret_cast<const int32_t*>(fw + p.off_tab);
  const int32_t* nseg = reinterpret_cast<const int32_t*>(fw + p.off_nseg);
  const float2* rlo = reinterpret_cast<const float2*>(fw + p.off_rope_lo);
  const float2* rhi = reinterpret_cast<const float2*>(fw + p.off_rope_hi);
  const float* states = reinterpret_cast<const float*>(fw + p.off_states);
  float* pstates = reinterpret_cast<float*>(a.ws + p.off_pstates);
  float* den = reinterpret_cast<float*>(a.ws + p.off_den);
  float* gd = reinterpret_cast<float*>(a.ws + p.off_gd);
  float* bd = reinterpret_cast<float*>(a.ws + p.off_bd);
  float* dgp = reinterpret_cast<float*>(a.ws + p.off_dgpart);
  const auto* q = static_cast<const uint16_t*>(a.q);
  const auto* k = static_cast<const uint16_t*>(a.k);
  const auto* v = static_cast<const uint16_t*>(a.v);
  const auto* g = static_cast<const uint16_t*>(b.dout);
  const dim3 grid(p.n_seg_max, p.H);
  mark(3);
  hipLaunchKernelGGL((bwd_dq_ws_kernel<D, BIDIR>), grid, dim3(512), 0, s, q, k, v, g, a.gq, a.gk, tab, nseg, rlo, rhi,
                     states, static_cast<uint16_t*>(b.dq), den, gd, bd, dgp, p.H, p.L, a.rms_eps, a.eps, hdr,
                     p.wait_polls, lim);
  mark(4);
  hipLaunchKernelGGL((bwd_pstate_kernel<D, BIDIR>), grid, dim3(256), 0, s, q, g, a.gq, tab, nseg, rlo, rhi, den, gd,
                     pstates, p.H, p.L, a.rms_eps, hdr, lim, ginit != nullptr ? 1 : 0);
  mark(5);
  e = launch_scan_records(p, fw, pstates, BIDIR ? SCAN_TOTAL : SCAN_SUFFIX, hdr, s, ginit);
  if (e != hipSuccess) return e;
  if (ginit != nullptr) {
    e = launch_initial_grad(p, ginit, b, hdr, s);
    if (e != hipSuccess) return e;
  }
  mark(6);
  hipLaunchKernelGGL((bwd_dkv_ws_kernel<D, BIDIR>), grid, dim3(512), 0, s, q, k, v, g, a.gq, a.gk, tab, nseg, rlo, rhi,
                     pstates, den, gd, bd, static_cast<uint16_t*>(b.dk), static_cast<uint16_t*>(b.dv), dgp, p.H, p.L,
                     a.rms_eps, hdr, p.wait_polls, lim);
  mark(7);
  if (b.dgamma_q != nullptr || b.dgamma_k != nullptr)
    hipLaunchKernelGGL(bwd_dgamma_kernel, dim3(p.H), dim3(2 * D), 0, s, dgp, nseg, p.n_seg_max, p.H, D, b.dgamma_q,
                       b.dgamma_k, static_cast<const uint32_t*>(hdr));
  mark(8);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_backward(const Plan& p, const FwdArgs& a, const BwdArgs& b, hipStream_t s, hipEvent_t* ev) {
  const bool bf = p.dtype == 1, causal = !p.bidirectional;
#define RLA2_BWD(DD)                                                                                  \
  if (bf) return causal ? run_backward<DD, false>(p, a, b, s, ev) : run_backward<DD, true>(p, a, b, s, ev); \
  return causal ? run_backward_generic<false, DD, true>(p, a, b, s, ev)                             \
                : run_backward_generic<false, DD, false>(p, a, b, s, ev)
  switch (p.d) {
    case 32: RLA2_BWD(32);
    case 64: RLA2_BWD(64);
    case 128: RLA2_BWD(128);
  }
#undef RLA2_BWD
  return hipErrorInvalidValue;
}

}  // namespace rla2
