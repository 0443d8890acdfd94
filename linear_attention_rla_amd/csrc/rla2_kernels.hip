// HIP kernels for RLA-2 causal ReLU linear attention on gfx950 (CDNA4, wave64).
//
// Method: neuralnet.cpp development page "线性注意力家族：RLA / RAPT / RLA-2 与 GPU 落地"
// (the RLA page). §3 gives q' = ReLU(RoPE(RMSNorm(q))), k' likewise, the state
// S_t = S_{t-1} + k'_t (x) v_t, z_t = z_{t-1} + k'_t and out_t = q'_t S_t / (q'_t . z_t + eps);
// §1 notes that the fixed-size state lets training accumulate it chunk-parallel; §2.2/§4.1
// clear the state at document starts.
//
// Chunked evaluation used here (C = 64 tokens per chunk, documents split into segments of
// whole chunks):
//   prep         cu_seqlens -> table of (row, first token, length, first position) segments,
//                and cos/sin of p*theta_j for p < 64 and for p = 64*a (angle addition rebuilds
//                any position from the two, so no per-token transcendental is needed)
//   chunk_state  per (segment, head): Sum over the segment of K'^T V and of K' (MFMA); the
//                last segment of a document is skipped unless final states are exported
//   state_scan   per (document, head): exclusive prefix of segment totals in fp32;
//                the inclusive end is the document's final state
//   chunk_out    per (segment, head): sweep the segment's chunks in order with the running
//                state S in MFMA accumulators:
//                  A   = causal_mask(Q'_c K'_c^T)                       (within the chunk)
//                  num = A V_c + Q'_c S,  den = A 1 + Q'_c z + eps,  out = num / den
//                  S  += K'_c^T V_c,      z  += sum of the rows of K'_c
//   decode       one token per sequence: feature map, S += k' (x) v, z += k', read-out
//
// The feature map (RMSNorm -> rotate-half RoPE -> ReLU) runs inside chunk_state,
// chunk_out and decode on the data just loaded, so q', k' never travel through HBM.
//
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <cmath>

#include <type_traits>

#include "rla2_device.h"
#include "rla2_internal.h"

namespace rla2 {
namespace {

// ----------------------------------------------------------------------------------------
// seg_map: documents -> segments of at most seg_len tokens (whole chunks), one workgroup.

__device__ __forceinline__ void seg_map_block(const int32_t* __restrict__ cu, int n_docs, int L, int seg_len,
                                              int n_seg_max, int hi_off, int32_t* __restrict__ tab,
                                              int32_t* __restrict__ docoff, int32_t* __restrict__ nseg) {
  __shared__ int scan[1024];
  __shared__ int carry_s;
  const int tid = threadIdx.x;
  if (tid == 0) carry_s = 0;
  __syncthreads();
  for (int base = 0; base < n_docs; base += 1024) {
    const int j = base + tid;
    int start = 0, end = 0, row = 0, cnt = 0;
    if (j < n_docs) {
      if (cu != nullptr) {
        start = min(max(cu[j], 0), L);
        end = min(max(cu[j + 1], start), L);
      } else {
        row = j;
        end = L;
      }
      cnt = (end - start + seg_len - 1) / seg_len;
    }
    scan[tid] = cnt;
    __syncthreads();
    for (int off = 1; off < 1024; off <<= 1) {
      const int add = tid >= off ? scan[tid - off] : 0;
      __syncthreads();
      scan[tid] += add;
      __syncthreads();
    }
    const int carry = carry_s;
    const int first = carry + scan[tid] - cnt;
    if (j < n_docs) {
      docoff[j] = min(first, n_seg_max);
      for (int s = 0; s < cnt; ++s) {
        const int idx = first + s;
        if (idx >= n_seg_max) break;
        int4 e;
        e.x = row;
        e.y = start + s * seg_len;
        e.z = min(seg_len, end - start - s * seg_len);
        e.w = s * seg_len;
        *reinterpret_cast<int4*>(tab + (size_t)idx * kTabInts) = e;
        tab[(size_t)idx * kTabInts + TAB_DOC] = j;
        tab[(size_t)idx * kTabInts + TAB_LAST] = s == cnt - 1;
        // the first document of each row (every row when unpacked) reads the offset rows
        const bool first = cu == nullptr || j == 0;
        tab[(size_t)idx * kTabInts + TAB_HIROW] = (first ? hi_off : 0) + e.w / kChunk;
      }
    }
    __syncthreads();
    if (tid == 1023) carry_s = carry + scan[1023];
    __syncthreads();
  }
  if (tid == 0) {
    const int total = min(carry_s, n_seg_max);
    docoff[n_docs] = total;
    *nseg = total;
  }
}

// ----------------------------------------------------------------------------------------
// rope_table: (cos, sin) of p * theta_j, theta_j = base^(-2j/D), in fp64, rounded to fp32.
// lo rows 0..63 hold p = row; hi rows a < n_hi hold p = 64 a, and rows n_hi + a (present
// when the first documents start at an offset) hold p = pos_off + 64 a.

__device__ __forceinline__ void rope_entry(int idx, float2* __restrict__ lo, float2* __restrict__ hi, int half, int D,
                                           int n_hi, int hi_off, int pos_off, float base) {
  const int rows = kChunk + n_hi + hi_off;
  if (idx >= rows * half) return;
  const int row = idx / half, j = idx % half;
  const double theta = pow((double)base, -2.0 * (double)j / (double)D);
  double p;
  if (row < kChunk) p = (double)row;
  else if (row < kChunk + n_hi) p = (double)kChunk * (double)(row - kChunk);
  else p = (double)pos_off + (double)kChunk * (double)(row - kChunk - n_hi);
  double s, c;
  sincos(p * theta, &s, &c);
  const float2 v = make_float2((float)c, (float)s);
  if (row < kChunk) lo[row * half + j] = v;
  else hi[(row - kChunk) * half + j] = v;
}

// prep: block 0 builds the segment table and the workspace's status header (flags cleared,
// the backward's go word set, the plan stamp with the cu_seqlens checksum), blocks 1.. the
// RoPE tables (one launch for all).
__global__ __launch_bounds__(1024) void prep_kernel(const int32_t* __restrict__ cu, int n_docs, int L, int seg_len,
                                                    int n_seg_max, int32_t* __restrict__ tab,
                                                    int32_t* __restrict__ docoff, int32_t* __restrict__ nseg,
                                                    float2* __restrict__ lo, float2* __restrict__ hi, int half, int D,
                                                    int n_hi, int hi_off, int pos_off, float base,
                                                    uint32_t* __restrict__ hdr, Stamp stamp) {
  if (blockIdx.x == 0) {
    seg_map_block(cu, n_docs, L, seg_len, n_seg_max, hi_off, tab, docoff, nseg);
    const uint32_t sum = cu_checksum_block(cu, n_docs);
    if (threadIdx.x < kStampWords)
      hdr[HDR_STAMP + threadIdx.x] = threadIdx.x == kStampWords - 1 ? sum : stamp.w[threadIdx.x];
    if (threadIdx.x == 0) {
      hdr[HDR_WAIT] = 0u;
      hdr[HDR_MISMATCH] = 0u;
      hdr[HDR_GO] = 1u;
    }
  } else {
    rope_entry((blockIdx.x - 1) * 1024 + threadIdx.x, lo, hi, half, D, n_hi, hi_off, pos_off, base);
  }
}

// The saved backward's set-up: compare the plan stamp in the forward's workspace header with
// this call's plan (and the checksum of this call's cu_seqlens), then clear the backward
// workspace's flags and let its kernels run (HDR_GO) only on a match.
__global__ __launch_bounds__(1024) void saved_check_kernel(const uint32_t* __restrict__ fwd_hdr,
                                                           uint32_t* __restrict__ hdr, Stamp stamp,
                                                           const int32_t* __restrict__ cu, int n_docs) {
  const uint32_t sum = cu_checksum_block(cu, n_docs);
  __shared__ int bad;
  if (threadIdx.x == 0) bad = 0;
  __syncthreads();
  if (threadIdx.x < kStampWords) {
    const uint32_t want = threadIdx.x == kStampWords - 1 ? sum : stamp.w[threadIdx.x];
    if (fwd_hdr[HDR_STAMP + threadIdx.x] != want) atomicOr(&bad, 1);
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    hdr[HDR_WAIT] = 0u;
    hdr[HDR_MISMATCH] = bad ? 1u : 0u;
    hdr[HDR_GO] = bad ? 0u : 1u;
  }
}

// ----------------------------------------------------------------------------------------
// chunk_state: per (segment, head), T = Sum_chunks K'^T V and Sum K' over the segment.
//
// Per chunk: every lane maps two tokens of k and stores K' and V in LDS (bf16 row-major,
// read back through the transposing LDS read; fp32 transposed), then the state waves add
// K'^T V to their accumulators and K'^T 1 (the column sums of K', ZR row tiles per wave).
// Raw k, v of the next two chunks are in flight in registers throughout (range-checked
// buffer loads, issued unconditionally so the wait counts stay exact); the RoPE rows of
// the segment sit in LDS and the per-lane RMSNorm weights and in-chunk angles in
// registers, so no other vector-memory load is ever waited on inside the sweep.

// With L2 (the original RLA's denominator) the kernel also accumulates the second state
// A = sum K'^T K' for the same value-column split, K' standing in for V, into `astates`
// (same record layout; the z slot is zero).
template <bool BF, int D, bool L2 = false>
__global__ __launch_bounds__(NT, L2 ? 1 : 2) void chunk_state_kernel(
    const typename Elem<BF>::St* __restrict__ k, const typename Elem<BF>::St* __restrict__ v,
    const float* __restrict__ gamma_k, const int32_t* __restrict__ tab, const int32_t* __restrict__ nseg,
    const float2* __restrict__ rope_lo, const float2* __restrict__ rope_hi, float* __restrict__ states,
    float* __restrict__ astates, int H, int L, float rms_eps, int skip_last) {
  using G = Geo<BF, D>;
  using St = typename G::St;
  using R = Raw<BF, D>;
  constexpr int KR = BF ? kChunk : D;           // rows of the K' and V arrays (row-major / transposed)
  constexpr int KP = BF ? G::ROWP : G::COLP;    // their pitch
  constexpr int ZR = G::RT >= 4 ? G::RT / 4 : 1;  // row tiles of the column sums per wave
  __shared__ __attribute__((aligned(16))) St sKx[KR * KP];
  __shared__ __attribute__((aligned(16))) St sVx[KR * KP];
  __shared__ __attribute__((aligned(16))) float2 sHi[kMaxSegChunks * G::HALF];  // RoPE rows of the chunks

  const int seg = blockIdx.x, h = blockIdx.y;
  if (seg >= *nseg || (skip_last && tab[(size_t)seg * kTabInts + TAB_LAST])) return;
  const SegInfo si = read_seg(tab, seg);
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int nch = __builtin_amdgcn_readfirstlane((si.len + kChunk - 1) / kChunk);
  const int t0 = 2 * (tid >> 3), m = tid & 7;
  const int c16 = lane & 15, g = lane >> 4;
  const size_t tok0 = ((size_t)si.row * H + h) * (size_t)L + si.start;
  const int seg_bytes = si.len * D * G::ES;
  const __amdgpu_buffer_rsrc_t rk = __builtin_amdgcn_make_buffer_rsrc((void*)(k + tok0 * D), 0, seg_bytes, kBufFlags);
  const __amdgpu_buffer_rsrc_t rv = __builtin_amdgcn_make_buffer_rsrc((void*)(v + tok0 * D), 0, seg_bytes, kBufFlags);
  {
    const float2* hi0 = rope_hi + (size_t)si.hirow * G::HALF;
    for (int i = tid; i < min(nch, kMaxSegChunks) * G::HALF; i += NT) sHi[i] = hi0[i];
  }
  float g1[G::E], g2[G::E];
  float2 lo[2][G::E];
#pragma unroll
  for (int e = 0; e < G::E; ++e) {
    const int j = m * G::E + e;
    g1[e] = gamma_k[(size_t)h * D + j];
    g2[e] = gamma_k[(size_t)h * D + j + G::HALF];
    lo[0][e] = rope_lo[t0 * G::HALF + j];
    lo[1][e] = rope_lo[(t0 + 1) * G::HALF + j];
  }

  auto kt_frag = [&](int rt, int kb2) -> Frag<BF> {  // K'^T rows [16 rt, +16), tokens of block kb2
    if constexpr (BF) return lds_frag_tr(sKx, KP, 32 * kb2, 16 * rt, lane);
    else return lds_frag<BF>(sKx, KP, rt * 16 + c16, kb2, g);
  };
  auto v_frag = [&](int n0, int kb2) -> Frag<BF> {  // V columns [n0, n0 + 16), tokens of block kb2
    if constexpr (BF) return lds_frag_tr(sVx, KP, 32 * kb2, n0, lane);
    else return lds_frag<BF>(sVx, KP, n0 + c16, kb2, g);
  };

  floatx4 acc[G::RT][G::CT];
  floatx4 accA[L2 ? G::RT : 1][G::CT];
  floatx4 zc[ZR];
#pragma unroll
  for (int rt = 0; rt < G::RT; ++rt)
#pragma unroll
    for (int ct = 0; ct < G::CT; ++ct) acc[rt][ct] = floatx4{0.f, 0.f, 0.f, 0.f};
  if constexpr (L2) {
#pragma unroll
    for (int rt = 0; rt < G::RT; ++rt)
#pragma unroll
      for (int ct = 0; ct < G::CT; ++ct) accA[rt][ct] = floatx4{0.f, 0.f, 0.f, 0.f};
  }
#pragma unroll
  for (int zr = 0; zr < ZR; ++zr) zc[zr] = floatx4{0.f, 0.f, 0.f, 0.f};
  const bool zwave = wave * ZR < G::RT;

  auto issue = [&](R (&r)[2], int c) {  // bf16: in the order step refills
    load_raw_buf<BF, D>(r[1], rv, c * kChunk + t0, m);
    load_raw_buf<BF, D>(r[0], rk, c * kChunk + t0, m);
  };
  auto step = [&](int c, R (&r)[2]) {
    __syncthreads();  // the previous chunk's LDS reads are done (the first time: sHi is written)
    if constexpr (BF) {
      // the registers of chunk c are refilled with chunk c + 2 as they free up: v first, then k
      // one token at a time
      if (c < nch) store_rows<BF, D>(sVx, r[1], t0, m);
      load_raw_buf<BF, D>(r[1], rv, (c + 2) * kChunk + t0, m);
      float2 hi[G::E];
      if (c < nch) copy_bytes<G::E * 8>(hi, sHi + c * G::HALF + m * G::E);
      auto map_tok = [&](auto tok_c) {
        constexpr int tok = decltype(tok_c)::value;
        if (c < nch) {
          R o;
          feature_map_lane<BF, D, tok>(r[0], o, g1, g2, lo, hi, rms_eps);
          store_rows<BF, D, tok>(sKx, o, t0, m);
        }
        load_raw_buf<BF, D, tok>(r[0], rk, (c + 2) * kChunk + t0, m);
      };
      map_tok(std::integral_constant<int, 0>{});
      map_tok(std::integral_constant<int, 1>{});
    } else {
      if (c < nch) {
        float2 hi[G::E];
        copy_bytes<G::E * 8>(hi, sHi + c * G::HALF + m * G::E);
        R o;
        feature_map_lane<BF, D>(r[0], o, g1, g2, lo, hi, rms_eps);
        store_cols<BF, D>(sKx, o, t0, m);
        store_cols<BF, D>(sVx, r[1], t0, m);
      }
      issue(r, c + 2);  // into the registers just consumed
    }
    __syncthreads();
    if (c < nch && wave < G::NW) {
      Frag<BF> Vf[G::CT][2];
#pragma unroll
      for (int ct = 0; ct < G::CT; ++ct) {
        Vf[ct][0] = v_frag(wave * G::DVW + ct * 16, 0);
        Vf[ct][1] = v_frag(wave * G::DVW + ct * 16, 1);
      }
#pragma unroll
      for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
        for (int rt = 0; rt < G::RT; ++rt) {
          const Frag<BF> a = kt_frag(rt, kb2);
#pragma unroll
          for (int ct = 0; ct < G::CT; ++ct) acc[rt][ct] = mma(a, Vf[ct][kb2], acc[rt][ct]);
        }
      if constexpr (L2) {  // A += K'^T K' for this wave's columns (K' columns as the value operand)
#pragma unroll
        for (int kb2 = 0; kb2 < 2; ++kb2) {
          Frag<BF> Kc[G::CT];
#pragma unroll
          for (int ct = 0; ct < G::CT; ++ct) Kc[ct] = kt_frag(wave * G::CT + ct, kb2);
#pragma unroll
          for (int rt = 0; rt < G::RT; ++rt) {
            const Frag<BF> a = kt_frag(rt, kb2);
#pragma unroll
            for (int ct = 0; ct < G::CT; ++ct) accA[rt][ct] = mma(a, Kc[ct], accA[rt][ct]);
          }
        }
      }
      if (zwave) {
        const Frag<BF> ones = ones_frag<BF>();
#pragma unroll
        for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
          for (int zr = 0; zr < ZR; ++zr) zc[zr] = mma(kt_frag(wave * ZR + zr, kb2), ones, zc[zr]);
      }
    }
  };
  R set0[2], set1[2];
  issue(set0, 0);
  issue(set1, 1);
  for (int c = 0; c < nch; c += 2) {
    step(c, set0);
    step(c + 1, set1);
  }

  float* rec = states + ((size_t)seg * H + h) * (size_t)(D * D + D);
  if (wave < G::NW) {
#pragma unroll
    for (int rt = 0; rt < G::RT; ++rt)
#pragma unroll
      for (int ct = 0; ct < G::CT; ++ct)
        __builtin_nontemporal_store(acc[rt][ct], reinterpret_cast<floatx4*>(rec + rec_frag<BF, D>(wave, rt, ct, lane)));
  }
  if (zwave && c16 < 4) {  // every column of zc holds the sums of rows 16 rt + 4g + i
#pragma unroll
    for (int zr = 0; zr < ZR; ++zr) rec[D * D + (wave * ZR + zr) * 16 + 4 * g + c16] = zc[zr][c16];
  }
  if constexpr (L2) {
    float* arec = astates + ((size_t)seg * H + h) * (size_t)(D * D + D);
    if (wave < G::NW) {
#pragma unroll
      for (int rt = 0; rt < G::RT; ++rt)
#pragma unroll
        for (int ct = 0; ct < G::CT; ++ct)
          __builtin_nontemporal_store(accA[rt][ct],
                                      reinterpret_cast<floatx4*>(arec + rec_frag<BF, D>(wave, rt, ct, lane)));
    }
    if (tid < D) arec[D * D + tid] = 0.f;
  }
}

// chunk_state with the L2 denominator's second state, bf16: 8 waves, one workgroup per CU.
// Waves 0..3 accumulate S = sum K'^T V and the column sums of K' (the value-column split of S),
// waves 4..7 accumulate A = sum K'^T K' (the same split of A's columns), so each wave carries one
// state (the 4-wave kernel carrying both ran at one wave per SIMD). Every wave also maps one
// token per 8 lanes: step st maps chunk st into buffer st % 2 while the MFMAs run on chunk
// st - 1 from the other buffer; one barrier per step. Two chunks of raw k, v are in flight per
// lane, refilled as they free up.
template <int D>
__global__ __launch_bounds__(512, 1) void chunk_state_l2_kernel(
    const uint16_t* __restrict__ k, const uint16_t* __restrict__ v, const float* __restrict__ gamma_k,
    const int32_t* __restrict__ tab, const int32_t* __restrict__ nseg, const float2* __restrict__ rope_lo,
    const float2* __restrict__ rope_hi, float* __restrict__ states, float* __restrict__ astates, int H, int L,
    float rms_eps, int skip_last) {
  using G = Geo<true, D>;
  using R = Raw<true, D>;
  constexpr int BUF = kChunk * G::ROWP;
  constexpr int ZR = G::RT >= 4 ? G::RT / 4 : 1;  // row tiles of the column sums per S wave
  __shared__ __attribute__((aligned(16))) uint16_t sK[2 * BUF];
  __shared__ __attribute__((aligned(16))) uint16_t sV[2 * BUF];
  __shared__ __attribute__((aligned(16))) float2 sHi[kMaxSegChunks * G::HALF];  // RoPE rows of the chunks

  const int seg = blockIdx.x, h = blockIdx.y;
  if (seg >= *nseg || (skip_last && tab[(size_t)seg * kTabInts + TAB_LAST])) return;
  const SegInfo si = read_seg(tab, seg);
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int nch = __builtin_amdgcn_readfirstlane((si.len + kChunk - 1) / kChunk);
  const int tg = tid >> 3, m = tid & 7;  // this lane group's token of the chunk (0..63)
  const int c16 = lane & 15, g = lane >> 4;
  const size_t tok0 = ((size_t)si.row * H + h) * (size_t)L + si.start;
  const int seg_bytes = si.len * D * 2;
  const __amdgpu_buffer_rsrc_t rk = __builtin_amdgcn_make_buffer_rsrc((void*)(k + tok0 * D), 0, seg_bytes, kBufFlags);
  const __amdgpu_buffer_rsrc_t rv = __builtin_amdgcn_make_buffer_rsrc((void*)(v + tok0 * D), 0, seg_bytes, kBufFlags);
  {
    const float2* hi0 = rope_hi + (size_t)si.hirow * G::HALF;
    for (int i = tid; i < min(nch, kMaxSegChunks) * G::HALF; i += 512) sHi[i] = hi0[i];
  }
  float g1[G::E], g2[G::E];
  float2 lo[2][G::E];  // slot 0: the in-chunk angles of token tg (the lane maps token slot 0 only)
#pragma unroll
  for (int e = 0; e < G::E; ++e) {
    const int j = m * G::E + e;
    g1[e] = gamma_k[(size_t)h * D + j];
    g2[e] = gamma_k[(size_t)h * D + j + G::HALF];
    lo[0][e] = rope_lo[tg * G::HALF + j];
    lo[1][e] = lo[0][e];
  }
  const bool swave = wave < 4;                        // S (and z) or A
  const int cw = swave ? wave : wave - 4;             // the wave's column block
  const bool owns = cw < G::NW;
  const bool zwave = swave && cw * ZR < G::RT;
  floatx4 acc[G::RT][G::CT];
  floatx4 zc[ZR];
#pragma unroll
  for (int rt = 0; rt < G::RT; ++rt)
#pragma unroll
    for (int ct = 0; ct < G::CT; ++ct) acc[rt][ct] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int zr = 0; zr < ZR; ++zr) zc[zr] = floatx4{0.f, 0.f, 0.f, 0.f};

  struct In {
    R xk, xv;
  };
  auto issue = [&](In& in, int c) {  // in the order step refills
    load_raw_buf<true, D, 0>(in.xv, rv, c * kChunk + tg, m);
    load_raw_buf<true, D, 0>(in.xk, rk, c * kChunk + tg, m);
  };
  auto step = [&](int st, In& in) {
    if (st < nch) {  // chunk st into buffer st % 2
      uint16_t* bK = sK + (st & 1) * BUF;
      uint16_t* bV = sV + (st & 1) * BUF;
      store_rows<true, D, 0>(bV, in.xv, tg, m);
      load_raw_buf<true, D, 0>(in.xv, rv, (st + 2) * kChunk + tg, m);
      float2 hi[G::E];
      copy_bytes<G::E * 8>(hi, sHi + st * G::HALF + m * G::E);
      R o;
      feature_map_lane<true, D, 0>(in.xk, o, g1, g2, lo, hi, rms_eps);
      store_rows<true, D, 0>(bK, o, tg, m);
      load_raw_buf<true, D, 0>(in.xk, rk, (st + 2) * kChunk + tg, m);
    }
    if (st >= 1 && owns) {  // chunk st - 1 from the other buffer
      const uint16_t* cK = sK + ((st + 1) & 1) * BUF;
      const uint16_t* cV = sV + ((st + 1) & 1) * BUF;
#pragma unroll
      for (int kb2 = 0; kb2 < 2; ++kb2) {
        Frag<true> B[G::CT];  // V columns (S waves) or K' columns (A waves) of this wave
#pragma unroll
        for (int ct = 0; ct < G::CT; ++ct)
          B[ct] = lds_frag_tr(swave ? cV : cK, G::ROWP, 32 * kb2, cw * G::DVW + ct * 16, lane);
#pragma unroll
        for (int rt = 0; rt < G::RT; ++rt) {
          const Frag<true> a = lds_frag_tr(cK, G::ROWP, 32 * kb2, 16 * rt, lane);
#pragma unroll
          for (int ct = 0; ct < G::CT; ++ct) acc[rt][ct] = mma(a, B[ct], acc[rt][ct]);
        }
      }
      if (zwave) {
        const Frag<true> ones = ones_frag<true>();
#pragma unroll
        for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
          for (int zr = 0; zr < ZR; ++zr)
            zc[zr] = mma(lds_frag_tr(cK, G::ROWP, 32 * kb2, 16 * (cw * ZR + zr), lane), ones, zc[zr]);
      }
    }
    __syncthreads();
  };
  In set0, set1;
  issue(set0, 0);
  issue(set1, 1);
  __syncthreads();  // sHi
  for (int st = 0; st <= nch; st += 2) {
    step(st, set0);
    if (st + 1 <= nch) step(st + 1, set1);
  }

  float* rec = (swave ? states : astates) + ((size_t)seg * H + h) * (size_t)(D * D + D);
  if (owns) {
#pragma unroll
    for (int rt = 0; rt < G::RT; ++rt)
#pragma unroll
      for (int ct = 0; ct < G::CT; ++ct)
        __builtin_nontemporal_store(acc[rt][ct], reinterpret_cast<floatx4*>(rec + rec_frag<true, D>(cw, rt, ct, lane)));
  }
  if (zwave && c16 < 4) {  // every column of zc holds the sums of rows 16 rt + 4g + i
#pragma unroll
    for (int zr = 0; zr < ZR; ++zr) rec[D * D + (cw * ZR + zr) * 16 + 4 * g + c16] = zc[zr][c16];
  }
  if (!swave && tid - 256 < D) rec[D * D + tid - 256] = 0.f;
}

// ----------------------------------------------------------------------------------------
// state_scan: per (document, head, 1024-float tile of the state record), walk the document's
// segments in order, starting from the initial state for the first document of each row
// (every document when unpacked, document 0 when packed) and from zero otherwise. Mode
// SCAN_PREFIX replaces each segment total by its exclusive prefix (the causal forward),
// SCAN_TOTAL writes the document's total into every one of its segment records (the
// bidirectional forward), SCAN_NONE leaves the records alone (the state build). The
// inclusive end is the document's final state. SCAN_SUFFIX walks the segments from the
// last to the first and replaces each total by the sum over the later segments of its
// document (the reverse states of the backward; no initial state). The export of the
// inclusive end goes to every document's own slot of final_S / final_z, or, with
// export_first, only for the documents that start from the initial state, one slot per row
// (the backward's gradient with respect to the initial state: the whole document's reverse
// state).

__global__ __launch_bounds__(256) void state_scan_kernel(float* __restrict__ states, const int32_t* __restrict__ docoff,
                                                         int H, int D, int n_tiles, int mode,
                                                         float* __restrict__ final_S, float* __restrict__ final_z,
                                                         const float* __restrict__ init_S,
                                                         const float* __restrict__ init_z, int init_all,
                                                         int export_first, const uint32_t* __restrict__ go_hdr) {
  if (go_hdr != nullptr && !bwd_go(go_hdr)) return;  // the backward's reverse scan after a failed check
  const int doc = blockIdx.x / n_tiles, tile = blockIdx.x % n_tiles, h = blockIdx.y;
  const int R4 = (D * D + D) / 4;
  const int e4 = tile * 256 + threadIdx.x;
  if (e4 >= R4) return;
  const int e = 4 * e4;
  // S part of the record: the 4 floats at e4 are S[row + i][col], i < 4 (fragment-native)
  int row = 0, col = 0;
  if (e < D * D) {
    const int RT = D / 16, NW = D / 16 < 4 ? D / 16 : 4, CT = D / NW / 16;
    const int ln = e4 % 64, t = e4 / 64;
    const int ct = t % CT, rt = (t / CT) % RT, w = t / CT / RT;
    row = 16 * rt + 4 * (ln / 16);
    col = w * (D / NW) + 16 * ct + ln % 16;
  }
  const int s0 = docoff[doc], s1 = docoff[doc + 1];
  const bool exp = (final_S != nullptr || final_z != nullptr) && (!export_first || init_all || doc == 0);
  const int xdoc = export_first && !init_all ? 0 : doc;  // the export slot
  auto put_end = [&](float4 r) {
    if (final_S != nullptr && e < D * D) {  // fragment-native record -> row-major [d][d]
      float* dst = final_S + ((size_t)xdoc * H + h) * D * D + (size_t)row * D + col;
      dst[0] = r.x;
      dst[D] = r.y;
      dst[2 * D] = r.z;
      dst[3 * D] = r.w;
    }
    if (final_z != nullptr && e >= D * D)
      *reinterpret_cast<float4*>(final_z + ((size_t)xdoc * H + h) * D + (e - D * D)) = r;
  };
  float4* st = reinterpret_cast<float4*>(states);
  float4 run = make_float4(0.f, 0.f, 0.f, 0.f);
  if (init_S != nullptr && (init_all || doc == 0)) {
    if (e < D * D) {
      const float* src = init_S + (size_t)h * D * D + (size_t)row * D + col;
      run = make_float4(src[0], src[D], src[2 * D], src[3 * D]);
    } else if (init_z != nullptr) {  // (the L2 mode's A records have no z: it stays zero)
      run = *reinterpret_cast<const float4*>(init_z + (size_t)h * D + (e - D * D));
    }
  }
  constexpr int kBatch = 16;  // records in flight per thread
  if (mode == SCAN_SUFFIX) {
    for (int s = s1 - 1; s >= s0; s -= kBatch) {
      const int cnt = min(kBatch, s - s0 + 1);
      float4 val[kBatch];
#pragma unroll
      for (int j = 0; j < kBatch; ++j) {  // the first record's total is needed for the export only
        val[j] = make_float4(0.f, 0.f, 0.f, 0.f);
        if (j < cnt && (s - j > s0 || exp)) val[j] = st[((size_t)(s - j) * H + h) * R4 + e4];
      }
#pragma unroll
      for (int j = 0; j < kBatch; ++j) {
        if (j < cnt) {
          st[((size_t)(s - j) * H + h) * R4 + e4] = run;
          run.x += val[j].x;
          run.y += val[j].y;
          run.z += val[j].z;
          run.w += val[j].w;
        }
      }
    }
    if (exp) put_end(run);
    return;
  }
  // the prefix mode without an export never needs the last record's total (it may be unset)
  const int s_read = mode == SCAN_PREFIX && final_S == nullptr && final_z == nullptr ? s1 - 1 : s1;
  for (int s = s0; s < s1; s += kBatch) {
    const int cnt = min(kBatch, s1 - s);
    float4 val[kBatch];
#pragma unroll
    for (int j = 0; j < kBatch; ++j) {
      val[j] = make_float4(0.f, 0.f, 0.f, 0.f);
      if (j < cnt && s + j < s_read) val[j] = st[((size_t)(s + j) * H + h) * R4 + e4];
    }
#pragma unroll
    for (int j = 0; j < kBatch; ++j) {
      if (j < cnt) {
        if (mode == SCAN_PREFIX) st[((size_t)(s + j) * H + h) * R4 + e4] = run;
        run.x += val[j].x;
        run.y += val[j].y;
        run.z += val[j].z;
        run.w += val[j].w;
      }
    }
  }
  if (mode == SCAN_TOTAL)
    for (int s = s0; s < s1; ++s) st[((size_t)s * H + h) * R4 + e4] = run;
  if (exp) put_end(run);
}

// The gradient with respect to the initial state: per element of [H][d][d] and [H][d], the
// sum over the rows (in row order) of the totals the scan exported with export_first.
__global__ __launch_bounds__(256) void initial_grad_kernel(const float* __restrict__ totals, int rows, int H, int D,
                                                           float* __restrict__ gS, float* __restrict__ gz,
                                                           const uint32_t* __restrict__ go_hdr) {
  if (go_hdr != nullptr && !bwd_go(go_hdr)) return;
  const size_t nS = (size_t)H * D * D, nz = (size_t)H * D;
  const size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
  float acc = 0.f;
  if (i < nS) {
    for (int r = 0; r < rows; ++r) acc += totals[(size_t)r * nS + i];
    if (gS != nullptr) gS[i] = acc;
  } else if (i < nS + nz) {
    const float* tz = totals + (size_t)rows * nS;
    for (int r = 0; r < rows; ++r) acc += tz[(size_t)r * nz + (i - nS)];
    if (gz != nullptr) gz[i - nS] = acc;
  }
}

// ----------------------------------------------------------------------------------------
// chunk_out: per (segment, head), sweep the chunks of C tokens (C in {16, 32, 64, 128}) with the
// running state in accumulators: every query reads the state at the start of its chunk and
// the keys of its chunk up to itself directly (RLA page §3 formula, split by the associativity
// of §1). LDS holds one 64-token block of Q', K', V at a time:
//   C <= 64  one pass per block; the block holds 64 / C chunks, and inside it the state
//            advances chunk by chunk in the output phase (S += K'_j^T V_j over the tokens of
//            chunk j only); q'.z of a later chunk adds the fp32 scores of the block's earlier
//            chunks (their keys are part of that chunk's z) to q'.z of the block start
//   C = 128  a chunk is two blocks: pass (0, 0) gives the first block's queries from its own
//            keys; passes (1, 0) and (1, 1) give the second block's queries from the keys of
//            both blocks (the first block's k, v are loaded and mapped again), and advance the
//            state with both blocks' keys
// Per pass, three phases separated by workgroup barriers:
//   map   all 256 lanes: q' (first pass of a query block, with q'.z per token) and k' of two
//         tokens each, Q', K', V rows into LDS (bf16: the K'^T and V operands are read back
//         with the transposing LDS read; fp32: K'^T and V^T are also stored transposed); then
//         the next pass's loads are issued
//   score wave w: the score tile of query tile w against the pass's keys, masked to the keys of
//         the query's chunk up to itself, rounded to the element type and stored in LDS as
//         the B operand of A V; row sums accumulate over the query block's passes, the last
//         one gives 1/(rowsum + q'.z + eps)
//   out   wave w < NW (value columns [w*DVW, (w+1)*DVW)): O^T = S^T Q'^T (first pass of the
//         query block) + V^T A^T accumulated in registers over the passes, so each lane holds
//         4 consecutive output columns of one row, written after the last pass; S += K'^T V in
//         the accumulators; wave 0 also forms the column sums of K' against a ones operand and
//         adds them to z.
// Below d = 128 registers stay under 256 and LDS under 80 KB (bf16), so two workgroups share
// a CU; at d = 128 one workgroup per CU holds the state in registers.
//
// L2 (the original RLA's denominator, sqrt(sum_i s_ti^2) + eps): the waves also carry the
// second state A = sum k'k'^T (same column split), the score phase keeps the sum of the
// squared weights (and, for the earlier chunks of a block, of the squared fp32 scores), and
// a phase between score and out (first pass of a query block) forms q'_t^T A q'_t as
// A^T Q'^T (the shape of the S^T Q'^T term) dotted with q'_t, summed over the waves in LDS
// (one more barrier); A advances with K' as the value operand. One workgroup per CU.
//
// The bf16 path runs chunk_out_ws_kernel below instead (C = 16, 32, 64, and 128 with the Sum
// denominator); this kernel serves fp32 and the L2 denominator at C = 128.

template <bool BF, int D, bool L2, int C>
__global__ __launch_bounds__(NT, (L2 || D == 128) ? 1 : 2) void chunk_out_kernel(
    const typename Elem<BF>::St* __restrict__ q, const typename Elem<BF>::St* __restrict__ k,
    const typename Elem<BF>::St* __restrict__ v, const float* __restrict__ gamma_q,
    const float* __restrict__ gamma_k, const int32_t* __restrict__ tab, const int32_t* __restrict__ nseg,
    const float2* __restrict__ rope_lo, const float2* __restrict__ rope_hi, const float* __restrict__ states,
    const float* __restrict__ astates, typename Elem<BF>::St* __restrict__ out, int H, int L, float rms_eps,
    float eps) {
  using G = Geo<BF, D>;
  using St = typename G::St;
  using EL = Elem<BF>;
  static_assert(C == 16 || C == 32 || C == 64 || C == 128, "chunk");
  constexpr int NB = C > kChunk ? C / kChunk : 1;  // 64-token blocks per chunk
  constexpr int TPC = (C < kChunk ? C : kChunk) / 16;  // 16-row tiles per chunk inside a block
  constexpr int NSUB = 4 / TPC;                    // chunks per block
  constexpr int NP = NB * (NB + 1) / 2;            // passes per chunk
  constexpr int TD = BF ? 1 : D;  // rows of the transposed copies (fp32 only)
  __shared__ __attribute__((aligned(16))) St sQ[kChunk * G::ROWP];
  __shared__ __attribute__((aligned(16))) St sK[kChunk * G::ROWP];
  __shared__ __attribute__((aligned(16))) St sV[BF ? kChunk * G::ROWP : 8];
  __shared__ __attribute__((aligned(16))) St sKT[TD * G::COLP];
  __shared__ __attribute__((aligned(16))) St sVT[TD * G::COLP];
  __shared__ Frag<BF> sA[4 * 2 * 64];  // [query tile][key block][lane]: B operands of V^T A^T
  __shared__ float sZ[D];
  __shared__ float sQz[kChunk];
  __shared__ float sInv[kChunk];
  __shared__ float sQuad[L2 ? 4 * kChunk : 1];  // L2: each state wave's part of q'^T A q'
  __shared__ float sRs2[L2 ? kChunk : 1];       // L2: sum of the squared weights

  const int seg = blockIdx.x, h = blockIdx.y;
  if (seg >= *nseg) return;
  const SegInfo si = read_seg(tab, seg);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int t0 = 2 * (tid >> 3), m = tid & 7;
  const int c16 = lane & 15, g = lane >> 4;
  const size_t tok0 = ((size_t)si.row * H + h) * (size_t)L + si.start;
  const St* qb = q + tok0 * D;
  const St* kb = k + tok0 * D;
  const St* vb = v + tok0 * D;
  St* ob = out + tok0 * D;
  const float* gq = gamma_q + (size_t)h * D;
  const float* gk = gamma_k + (size_t)h * D;

  // K'^T rows [16 rt, +16) x tokens of k-block kb2; V (as V^T rows or as the B operand of
  // the state update, the same fragment) for value columns [n0, n0 + 16) x k-block kb2
  auto kt_frag = [&](int rt, int kb2) -> Frag<BF> {
    if constexpr (BF) return lds_frag_tr(sK, G::ROWP, 32 * kb2, 16 * rt, lane);
    else return lds_frag<BF>(sKT, G::COLP, rt * 16 + c16, kb2, g);
  };
  auto v_frag = [&](int n0, int kb2) -> Frag<BF> {
    if constexpr (BF) return lds_frag_tr(sV, G::ROWP, 32 * kb2, n0, lane);
    else return lds_frag<BF>(sVT, G::COLP, n0 + c16, kb2, g);
  };
  // Only the tokens [16 half, 16 half + 16) of a 32-token k-block: the slot order puts tokens
  // 4g + i in slots 0..3 and 16 + 4g + i in slots 4..7 (rla2_device.h), so the other half's
  // slots are cleared (a chunk of 16 tokens inside a k-block).
  auto keep_half = [&](Frag<BF> f, int half) -> Frag<BF> {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      if ((j >> 2) != half) {
        if constexpr (BF) f.v[j] = static_cast<__bf16>(0.0f);
        else f.v[j] = 0.0f;
      }
    }
    return f;
  };

  // running state S (this wave's value columns) and z, from the exclusive prefix
  const float* rec = states + ((size_t)seg * H + h) * (size_t)(D * D + D);
  floatx4 S[G::RT][G::CT];
  {
    const int wv = wave < G::NW ? wave : 0;  // waves without state columns keep a harmless copy
#pragma unroll
    for (int rt = 0; rt < G::RT; ++rt)
#pragma unroll
      for (int ct = 0; ct < G::CT; ++ct)
        S[rt][ct] = *reinterpret_cast<const floatx4*>(rec + rec_frag<BF, D>(wv, rt, ct, lane));
  }
  if (tid < D) sZ[tid] = rec[D * D + tid];
  floatx4 Ak[L2 ? G::RT : 1][G::CT];  // L2: A, this wave's columns
  if constexpr (L2) {
    const float* arec = astates + ((size_t)seg * H + h) * (size_t)(D * D + D);
    const int wv = wave < G::NW ? wave : 0;
#pragma unroll
    for (int rt = 0; rt < G::RT; ++rt)
#pragma unroll
      for (int ct = 0; ct < G::CT; ++ct)
        Ak[rt][ct] = *reinterpret_cast<const floatx4*>(arec + rec_frag<BF, D>(wv, rt, ct, lane));
  }

  // passes: chunk ch = p / NP; r = p % NP gives (query block qi, key block ki), ki <= qi
  const int nblk = (si.len + kChunk - 1) / kChunk;
  const int npass = (si.len + C - 1) / C * NP;
  auto pass_blocks = [&](int p, int& qblk, int& kblk, int& qi, int& ki) {
    const int ch = p / NP, r = p % NP;
    qi = r == 0 ? 0 : (r <= 2 ? 1 : 2);  // NB <= 2
    ki = r - qi * (qi + 1) / 2;
    qblk = ch * NB + qi;
    kblk = ch * NB + ki;
  };
  Raw<BF, D> rq, rk, rv;
  auto issue = [&](int p) {  // raw q (first pass of its query block), k, v of pass p
    int qblk, kblk, qi, ki;
    pass_blocks(p, qblk, kblk, qi, ki);
    if (p >= npass || qblk >= nblk) return;
    if (ki == 0) load_raw<BF, D>(rq, qb + (size_t)qblk * kChunk * D, t0, m, si.len - qblk * kChunk);
    load_raw<BF, D>(rk, kb + (size_t)kblk * kChunk * D, t0, m, si.len - kblk * kChunk);
    load_raw<BF, D>(rv, vb + (size_t)kblk * kChunk * D, t0, m, si.len - kblk * kChunk);
  };
  issue(0);

  floatx4 O[NB > 1 ? G::CT : 1][4];  // C = 128: O^T tiles of the query block, summed over its passes
  float rs_acc = 0.f, rs2_acc = 0.f, zrs = 0.f, zrs2 = 0.f;  // score waves: row sums of their tile

  for (int p = 0; p < npass; ++p) {
    int qblk, kblk, qi, ki;
    pass_blocks(p, qblk, kblk, qi, ki);
    if (qblk >= nblk) continue;  // the last chunk of the segment ends before this block
    const bool first = ki == 0, last = ki == qi, upd = qi == NB - 1;
    const int nvq = min(kChunk, si.len - qblk * kChunk);  // valid query rows of the block
    __syncthreads();  // B1: the previous pass's LDS reads are done; its z update is visible

    // ---- map
    {
      const float2* hq = rope_hi + (size_t)(si.hirow + qblk) * G::HALF;
      const float2* hk = rope_hi + (size_t)(si.hirow + kblk) * G::HALF;
      // The RMSNorm weights and the in-chunk RoPE table are the same for every block; hiding
      // their addresses from the optimiser keeps it from holding ~64 loaded values in
      // registers across the whole sweep (they are re-read from cache each pass instead).
      const float* gqi = gq;
      const float* gki = gk;
      const float2* loi = rope_lo;
      asm volatile("" : "+s"(gqi), "+s"(gki), "+s"(loi));
      Raw<BF, D> oq, ok;
      if (first && qblk == kblk) {
        feature_map_qk<BF, D>(rq, rk, oq, ok, gqi, gki, loi, hq, t0, m, rms_eps);
      } else {
        if (first) feature_map_pair<BF, D>(rq, oq, gqi, loi, hq, t0, m, rms_eps);
        feature_map_pair<BF, D>(rk, ok, gki, loi, hk, t0, m, rms_eps);
      }
      if (first) {
        store_rows<BF, D>(sQ, oq, t0, m);
        // q'_t . z of the two tokens (z at the start of the block), from the rounded q'
#pragma unroll
        for (int tok = 0; tok < 2; ++tok) {
          float pz = 0.f;
#pragma unroll
          for (int e = 0; e < G::E; ++e) {
            const int j = m * G::E + e;
            pz += oq.get(tok, 0, e) * sZ[j];
            pz += oq.get(tok, 1, e) * sZ[j + G::HALF];
          }
          pz = sum8(pz);
          if (m == 0) sQz[t0 + tok] = pz;
        }
      }
      store_rows<BF, D>(sK, ok, t0, m);
      if constexpr (!BF) store_cols<BF, D>(sKT, ok, t0, m);
    }
    if constexpr (BF) store_rows<BF, D>(sV, rv, t0, m);
    else store_cols<BF, D>(sVT, rv, t0, m);
    issue(p + 1);
    __syncthreads();  // B2: the pass's operands in LDS

    // ---- score: wave w owns query tile w
    {
      const int tt = wave;
      Frag<BF> Qf[G::KB];
#pragma unroll
      for (int kb2 = 0; kb2 < G::KB; ++kb2) Qf[kb2] = lds_frag<BF>(sQ, G::ROWP, tt * 16 + c16, kb2, g);
      if (first) rs_acc = rs2_acc = zrs = zrs2 = 0.f;
      // A^T tiles (rows = keys of tile kt, cols = queries of tile tt)
      floatx4 At[4];
      float rs = 0.f, rs2 = 0.f, zs = 0.f, zs2 = 0.f;
#pragma unroll
      for (int kt = 0; kt < 4; ++kt) {
        At[kt] = floatx4{0.f, 0.f, 0.f, 0.f};
        // keys of an earlier block of the chunk: all weighted; same block: up to the query,
        // weighted inside the query's chunk, through z (fp32 scores) in an earlier chunk
        const bool earlier_blk = ki < qi;
        const bool same_chunk = kt / TPC == tt / TPC;
        if (earlier_blk || kt <= tt) {
#pragma unroll
          for (int kb2 = 0; kb2 < G::KB; ++kb2)
            At[kt] = mma(lds_frag<BF>(sK, G::ROWP, kt * 16 + c16, kb2, g), Qf[kb2], At[kt]);
          if (earlier_blk || same_chunk) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              float a = At[kt][i];
              if (!earlier_blk && kt == tt && 4 * g + i > c16) a = 0.f;  // key after the query token
              a = EL::to_f(EL::from_f(a));                              // the weight the MFMA will use
              At[kt][i] = a;
              rs += a;
              if constexpr (L2) rs2 = __builtin_fmaf(a, a, rs2);
            }
          } else {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              zs += At[kt][i];
              if constexpr (L2) zs2 = __builtin_fmaf(At[kt][i], At[kt][i], zs2);
            }
            At[kt] = floatx4{0.f, 0.f, 0.f, 0.f};
          }
        }
      }
      rs_acc += sum_rows4(rs);  // every lane with c16 == t holds the row sum of query 16*tt + t
      if constexpr (TPC < 4) zrs += sum_rows4(zs);
      if constexpr (L2) {
        rs2_acc += sum_rows4(rs2);
        if constexpr (TPC < 4) zrs2 += sum_rows4(zs2);
      }
      sA[(tt * 2) * 64 + lane] = acc_frag<BF>(At[0], At[1]);
      sA[(tt * 2 + 1) * 64 + lane] = acc_frag<BF>(At[2], At[3]);
      if (last && g == 0) {
        if constexpr (L2) sRs2[tt * 16 + c16] = rs2_acc + zrs2;
        else sInv[tt * 16 + c16] = 1.0f / (rs_acc + zrs + sQz[tt * 16 + c16] + eps);
      }
    }
    __syncthreads();  // B3: score tiles and row reciprocals in LDS

    if constexpr (L2) {  // ---- q'_t^T A q'_t: this wave's columns a, all 64 queries
      if (first) {
        if (wave < G::NW) {
          float part[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int ct = 0; ct < G::CT; ++ct) {
            Frag<BF> Aa[G::KB];  // A^T (= A) rounded to the element type as the A operand
#pragma unroll
            for (int kb2 = 0; kb2 < G::KB; ++kb2) Aa[kb2] = acc_frag<BF>(Ak[2 * kb2][ct], Ak[2 * kb2 + 1][ct]);
            const int col = wave * G::DVW + ct * 16 + 4 * g;
#pragma unroll
            for (int tt = 0; tt < 4; ++tt) {
              floatx4 y = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
              for (int kb2 = 0; kb2 < G::KB; ++kb2) y = mma(Aa[kb2], lds_frag<BF>(sQ, G::ROWP, tt * 16 + c16, kb2, g), y);
              const St* qrow = sQ + (tt * 16 + c16) * G::ROWP + col;  // q'_t at dims col .. col + 3
#pragma unroll
              for (int i = 0; i < 4; ++i) part[tt] = __builtin_fmaf(EL::to_f(qrow[i]), y[i], part[tt]);
            }
          }
#pragma unroll
          for (int tt = 0; tt < 4; ++tt) {
            const float pp = sum_rows4(part[tt]);
            if (g == 0) sQuad[wave * kChunk + tt * 16 + c16] = pp;
          }
        }
        __syncthreads();  // B4: every wave's part of the quadratic form in LDS
      }
    }
    auto row_scale = [&](int t) -> float {  // 1 / den of query row t
      if constexpr (L2) {
        float quad = sRs2[t];
#pragma unroll
        for (int w = 0; w < G::NW; ++w) quad += sQuad[w * kChunk + t];
        return 1.0f / (__builtin_sqrtf(quad) + eps);
      } else {
        return sInv[t];
      }
    };

    // ---- out, then the state update
    if (wave < G::NW) {
      Frag<BF> Vf[G::CT][2];
#pragma unroll
      for (int ct = 0; ct < G::CT; ++ct) {
        Vf[ct][0] = v_frag(wave * G::DVW + ct * 16, 0);
        Vf[ct][1] = v_frag(wave * G::DVW + ct * 16, 1);
      }
      // S += K'^T V over the key tokens [16 * 4 j / NSUB, ...) of chunk j of the block (NSUB
      // chunks per block), or over the whole block
      auto advance = [&](int j) {
        constexpr int NKB = NSUB == 1 ? 2 : 1;  // 32-token k-blocks of the update
#pragma unroll
        for (int x = 0; x < NKB; ++x) {
          const int kb2 = NSUB == 1 ? x : (NSUB == 2 ? j : j / 2);
#pragma unroll
          for (int rt = 0; rt < G::RT; ++rt) {
            const Frag<BF> a = kt_frag(rt, kb2);
#pragma unroll
            for (int ct = 0; ct < G::CT; ++ct) {
              const Frag<BF> b = NSUB == 4 ? keep_half(Vf[ct][kb2], j & 1) : Vf[ct][kb2];
              S[rt][ct] = mma(a, b, S[rt][ct]);
            }
            if constexpr (L2) {  // A += K'^T K' (K' columns of this wave as the value operand)
#pragma unroll
              for (int ct = 0; ct < G::CT; ++ct) {
                const Frag<BF> kc = kt_frag(wave * G::CT + ct, kb2);
                Ak[rt][ct] = mma(a, NSUB == 4 ? keep_half(kc, j & 1) : kc, Ak[rt][ct]);
              }
            }
          }
        }
      };
      // this lane's 4 output columns col .. col + 3 of query row 16 tt + c16, scaled by 1/den
      auto store_tile = [&](floatx4 o, int tt, int ct) {
        const int col = wave * G::DVW + ct * 16 + 4 * g;
        const int t = tt * 16 + c16;
        const float r = row_scale(t);
        if (t < nvq) {
          St* dst = ob + ((size_t)qblk * kChunk + t) * D + col;
          if constexpr (BF) {
            const uint32_t w0 = __builtin_bit_cast(uint32_t, __builtin_convertvector(float2v{o[0] * r, o[1] * r}, bf16x2));
            const uint32_t w1 = __builtin_bit_cast(uint32_t, __builtin_convertvector(float2v{o[2] * r, o[3] * r}, bf16x2));
            *reinterpret_cast<uint2*>(dst) = make_uint2(w0, w1);
          } else {
            *reinterpret_cast<float4*>(dst) = make_float4(o[0] * r, o[1] * r, o[2] * r, o[3] * r);
          }
        }
      };
#pragma unroll
      for (int j = 0; j < NSUB; ++j) {
#pragma unroll
        for (int ct = 0; ct < G::CT; ++ct) {
          Frag<BF> Sa[G::KB];  // S^T rounded to the element type as the A operand
          if (first) {
#pragma unroll
            for (int kb2 = 0; kb2 < G::KB; ++kb2) Sa[kb2] = acc_frag<BF>(S[2 * kb2][ct], S[2 * kb2 + 1][ct]);
          }
#pragma unroll 1
          for (int x = 0; x < TPC; ++x) {
            const int tt = j * TPC + x;
            floatx4 o = floatx4{0.f, 0.f, 0.f, 0.f};
            if constexpr (NB > 1) {
              if (!first) o = O[ct][tt];
            }
            if (first) {
#pragma unroll
              for (int kb2 = 0; kb2 < G::KB; ++kb2) o = mma(Sa[kb2], lds_frag<BF>(sQ, G::ROWP, tt * 16 + c16, kb2, g), o);
            }
            o = mma(Vf[ct][0], sA[(tt * 2) * 64 + lane], o);
            o = mma(Vf[ct][1], sA[(tt * 2 + 1) * 64 + lane], o);
            if constexpr (NB == 1) store_tile(o, tt, ct);  // one pass per query block
            else O[ct][tt] = o;
          }
        }
        if constexpr (NSUB > 1) advance(j);  // the next chunk of the block reads the advanced state
      }
      if constexpr (NSUB == 1) {
        if (upd) advance(0);
      }
      if constexpr (NB > 1) {
        if (last) {
#pragma unroll
          for (int ct = 0; ct < G::CT; ++ct)
#pragma unroll
            for (int tt = 0; tt < 4; ++tt) store_tile(O[ct][tt], tt, ct);
        }
      }
      // z += the column sums of the pass's K' (read again after B1), with the state update
      if (wave == 0 && (NSUB > 1 || upd)) {
        const Frag<BF> ones = ones_frag<BF>();
#pragma unroll
        for (int rt = 0; rt < G::RT; ++rt) {
          floatx4 zc = mma(kt_frag(rt, 0), ones, floatx4{0.f, 0.f, 0.f, 0.f});
          zc = mma(kt_frag(rt, 1), ones, zc);  // every column holds the sums of rows 16 rt + 4g + i
          if (c16 < 4) sZ[rt * 16 + 4 * g + c16] += zc[c16];
        }
      }
    }
  }
}

// chunk_out for bf16, warp-specialised: 8 waves, one workgroup per CU.
//
// Waves 4..7 ("mappers") turn raw q, k, v into the chunk operands: the feature map of q
// and k (VALU work; both share the rotation angles) and the Q', K', V rows in LDS. They keep
// two chunks of raw input in flight in registers. Waves 0..3 ("MMA waves") run the score and
// output phases on the previous chunk from the other half of a double-buffered LDS and stage
// the output rows; the rows of the chunk before leave for memory at the end of the step, half
// from each role (L2: from the mappers). Each SIMD holds one wave of each kind, so the
// mappers' VALU work overlaps the MMA waves' matrix and LDS work, and the input loads overlap
// both.
//
// Step s (s = 0 .. nsteps-1): mappers map chunk s into buffer s % 2; MMA waves process chunk
// s - 1 from buffer (s - 1) % 2. One workgroup barrier per step (Y, at its end: buffer s % 2
// is complete, buffer (s - 1) % 2 is free again, the z operand for chunk s, written in the
// score phase of chunk s - 1, is visible).
// Inside the step the MMA waves also meet among themselves (score tiles and row reciprocals
// of every query tile are complete before anyone forms outputs) on an LDS arrival counter,
// which the mappers never wait on.
// Chunks of 128 tokens (Sum denominator) are two consecutive 64-token blocks: every query of
// the second block reads all 64 keys of the first block directly (RLA page §3 formula inside
// the chunk), and the state and z advance once per chunk, after its second block. While the
// MMA waves process a second block they read the first block's K' and V from the other
// parity's buffers and put the cross-block weights in that parity's Q' buffer; in that step
// the mappers map the next block into registers and store it only after all four MMA waves
// have released those buffers (sRelease, a bounded wait like the MMA waves' meeting).

// Score phase of MMA wave TT (query tile TT of the chunk): the causal tiles K'_kt Q'_TT^T
// (kt <= TT) and Z Q'_TT^T, the diagonal tile masked, every weight rounded to bf16 once
// (pairs of tiles packed as the B operands of V^T A^T); the row sums are taken from the
// packed weights with a bf16 dot against ones, so numerator and denominator use the same
// weights. The wave also forms the column sums of K' for row tiles [Z0, Z1): lane (i, g),
// i < 4, keeps z of dim 16 tile + 4g + i in zreg, adds the chunk's column sum and writes the
// result as the next chunk's z operand (zf_next, the other buffer of the pair). Every LDS
// operand is requested before the first MFMA.
// L2: no q'.z and no column sums; the row's sum of squared weights goes to sInv instead.
// Chunks of C < 64 tokens (C / 16 query tiles each): only the key tiles of the query tile's own
// chunk become weights; the keys of the step's earlier chunks reach the query through the state,
// which the MMA waves advance between the chunks, so the denominator takes their scores, unrounded
// (Sum: the scores; L2: their squares), in place of q'.(z they added).
// Chunks of C = 128 tokens (two 64-token blocks; Sum only): on the second block (CROSS) the
// query tile also scores all 64 keys of the chunk's first block (cKx) without a mask, packs
// those weights the same way into sAx and adds them to its row sum; z stays at the chunk's
// start for both blocks, so on the first block (ZADV false) the lanes that keep z add the
// block's column sums to zreg but write the unchanged z as the next block's operand.
template <int D, int TT, int Z0, int Z1, int NZR, bool L2 = false, int C = 64, bool CROSS = false, bool ZADV = true>
__device__ __forceinline__ void ws_score(const uint16_t* cQ, const uint16_t* cK, int qp, const Frag<true>* sZf,
                                         Frag<true>* zf_next, float (&zreg)[NZR], Frag<true>* sA, float* sInv,
                                         float eps, int lane, const uint16_t* cKx = nullptr,
                                         Frag<true>* sAx = nullptr) {
  using G = Geo<true, D>;
  constexpr int KB = G::KB, NZ = Z1 - Z0, NP = TT / 2 + 1;
  constexpr int KT0 = C >= 64 ? 0 : (TT / (C / 16)) * (C / 16);  // first key tile of the query tile's chunk
  static_assert(!L2 || NZ == 0, "");
  static_assert(NZ <= NZR, "");
  static_assert(!CROSS || (C == 128 && !L2), "cross-block weights: chunks of 128 tokens, Sum denominator");
  const int c16 = lane & 15, g = lane >> 4;
  Frag<true> Qf[KB], Kf[TT + 1][KB], Zf[KB], Ct[NZ > 0 ? NZ : 1][2];
#pragma unroll
  for (int kb2 = 0; kb2 < KB; ++kb2) Qf[kb2] = lds_frag_c(cQ, qp, TT * 16 + c16, kb2, g);
#pragma unroll
  for (int kt = 0; kt <= TT; ++kt)
#pragma unroll
    for (int kb2 = 0; kb2 < KB; ++kb2) Kf[kt][kb2] = lds_frag_c(cK, qp, kt * 16 + c16, kb2, g);
  if constexpr (!L2) {
#pragma unroll
    for (int kb2 = 0; kb2 < KB; ++kb2) Zf[kb2] = sZf[kb2 * 64 + lane];
  }
#pragma unroll
  for (int z = 0; z < NZ; ++z) {
    Ct[z][0] = lds_frag_tr(cK, qp, 0, 16 * (Z0 + z), lane);
    Ct[z][1] = lds_frag_tr(cK, qp, 32, 16 * (Z0 + z), lane);
  }
  floatx4 At[TT + 1];
#pragma unroll
  for (int kt = 0; kt <= TT; ++kt) At[kt] = floatx4{0.f, 0.f, 0.f, 0.f};
  floatx4 zq = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int kb2 = 0; kb2 < KB; ++kb2) {
#pragma unroll
    for (int kt = 0; kt <= TT; ++kt) At[kt] = mma(Kf[kt][kb2], Qf[kb2], At[kt]);
    if constexpr (!L2) zq = mma(Zf[kb2], Qf[kb2], zq);
  }
#pragma unroll
  for (int i = 0; i < 4; ++i)
    if (4 * g + i > c16) At[TT][i] = 0.f;  // key after the query token
  // packed bf16 weights, word i of pair b: rows 2i, 2i + 1 of tile 2b (i < 2) or of tile
  // 2b + 1 (i >= 2), the slot order of acc_frag
  uint32_t pw[NP][4];
#pragma unroll
  for (int b = 0; b < NP; ++b)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int kt = 2 * b + (i >> 1), r = 2 * (i & 1);
      pw[b][i] = kt <= TT && kt >= KT0
                     ? __builtin_bit_cast(uint32_t, __builtin_convertvector(float2v{At[kt % (TT + 1)][r], At[kt % (TT + 1)][r + 1]}, bf16x2))
                     : 0u;
    }
  float rs = 0.f;
  const bf16x2 ones2 = bf16x2{static_cast<__bf16>(1.0f), static_cast<__bf16>(1.0f)};
#pragma unroll
  for (int b = 0; b < NP; ++b)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const bf16x2 w2 = __builtin_bit_cast(bf16x2, pw[b][i]);
      // Sum: the weights against ones; L2: the weights against themselves (sum of squares)
      rs = __builtin_amdgcn_fdot2_f32_bf16(w2, L2 ? w2 : ones2, rs, false);
    }
#pragma unroll
  for (int kt = 0; kt < KT0; ++kt)  // the step's earlier chunks (C < 64)
#pragma unroll
    for (int i = 0; i < 4; ++i) rs = L2 ? __builtin_fmaf(At[kt][i], At[kt][i], rs) : rs + At[kt][i];
  if constexpr (CROSS) {  // the chunk's first block: all four key tiles, packed as pairs 0, 1
    floatx4 Ax[4];
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) Ax[kt] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kb2 = 0; kb2 < KB; ++kb2) {
      Frag<true> Kx[4];
#pragma unroll
      for (int kt = 0; kt < 4; ++kt) Kx[kt] = lds_frag_c(cKx, qp, kt * 16 + c16, kb2, g);
#pragma unroll
      for (int kt = 0; kt < 4; ++kt) Ax[kt] = mma(Kx[kt], Qf[kb2], Ax[kt]);
    }
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      uint32_t px[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int kt = 2 * b + (i >> 1), r = 2 * (i & 1);
        px[i] = __builtin_bit_cast(uint32_t, __builtin_convertvector(float2v{Ax[kt][r], Ax[kt][r + 1]}, bf16x2));
        rs = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, px[i]), ones2, rs, false);
      }
      *reinterpret_cast<u32x4*>(&sAx[(TT * 2 + b) * 64 + lane]) = u32x4{px[0], px[1], px[2], px[3]};
    }
  }
  if constexpr (!L2) {
    if (g == 0) rs += zq[0] + zq[1];  // q'.z of query 16 TT + c16 (rows 0, 1 of Z Q'^T)
  }
  rs = sum_rows4(rs);  // lanes with c16 == t: row sum + q'.z of query 16 TT + t
#pragma unroll
  for (int b = 0; b < NP; ++b)
    *reinterpret_cast<u32x4*>(&sA[(TT * 2 + b) * 64 + lane]) = u32x4{pw[b][0], pw[b][1], pw[b][2], pw[b][3]};
  if (g == 0) sInv[TT * 16 + c16] = L2 ? rs : 1.0f / (rs + eps);
  if constexpr (NZ > 0) {
    const Frag<true> ones = ones_frag<true>();
#pragma unroll
    for (int z = 0; z < NZ; ++z) {
      floatx4 zc = mma(Ct[z][0], ones, floatx4{0.f, 0.f, 0.f, 0.f});
      zc = mma(Ct[z][1], ones, zc);  // every column holds the sums of rows 16 (Z0 + z) + 4g + i
      if (c16 < 4) {
        // dim 16 T + 4g + i (T = Z0 + z) sits in fragment T / 2, slot 4 (g % 2) + i of lane
        // 16 (2 (T % 2) + g / 2) (bf16 of z) and of the lane after it (the remainder)
        const int T = Z0 + z;
        const float zold = zreg[z];
        zreg[z] += c16 == 0 ? zc[0] : c16 == 1 ? zc[1] : c16 == 2 ? zc[2] : zc[3];
        const float zw = ZADV ? zreg[z] : zold;  // the next block's z operand
        const __bf16 hi = static_cast<__bf16>(zw);
        const __bf16 lo = static_cast<__bf16>(zw - static_cast<float>(hi));
        uint16_t* zf16 = reinterpret_cast<uint16_t*>(zf_next + (T / 2) * 64 + 16 * (2 * (T % 2) + g / 2));
        zf16[4 * (g % 2) + c16] = __builtin_bit_cast(uint16_t, hi);
        zf16[8 + 4 * (g % 2) + c16] = __builtin_bit_cast(uint16_t, lo);
      }
    }
  }
}

// L2 (the original RLA's denominator sqrt(sum_i s_ti^2) + eps): the MMA waves also hold the
// second state A = sum k'k'^T (the same value-column split and tile map as S). After the
// state update of chunk c they form its q'^T A_prev q' as A_prev^T Q'^T dotted with q' (their
// parts go to LDS) and advance A with its K'; the chunk's numerators are staged unnormalised
// with the rows' sums of squared weights, and one step later each output row is scaled by
// 1 / (sqrt(sum) + eps) as it leaves for memory. Nothing new waits inside a step.
template <int D, bool L2 = false, int C = 64>
__global__ __launch_bounds__(512, 1) void chunk_out_ws_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    const float* __restrict__ gamma_q, const float* __restrict__ gamma_k, const int32_t* __restrict__ tab,
    const int32_t* __restrict__ nseg, const float2* __restrict__ rope_lo, const float2* __restrict__ rope_hi,
    const float* __restrict__ states, const float* __restrict__ astates, uint16_t* __restrict__ out, int H, int L,
    float rms_eps, float eps, uint32_t* __restrict__ hdr, uint32_t polls) {
  static_assert(!(L2 && C == 128), "chunks of 128 tokens with the L2 denominator run the generic kernel");
  using G = Geo<true, D>;
  using St = uint16_t;
  using R = Raw<true, D>;
  constexpr int BUF = kChunk * G::ROWP;  // elements of one V or output buffer
  // Q' and K' rows at a pitch of D + 16: the 16-byte row-fragment reads (lds_frag_c) and the
  // transposing reads of K' are then free of bank conflicts
  constexpr int QP = D + 16, BUFQ = kChunk * QP;
  __shared__ __attribute__((aligned(16))) St sQ[2 * BUFQ];
  __shared__ __attribute__((aligned(16))) St sK[2 * BUFQ];
  __shared__ __attribute__((aligned(16))) St sV[2 * BUF];
  __shared__ __attribute__((aligned(16))) St sO[2 * BUF];  // output rows of chunk c in buffer c % 2
  __shared__ Frag<true> sA[4 * 2 * 64];  // [query tile][key block][lane]: B operands of V^T A^T
  __shared__ float sInv[kChunk];
  // z as an MFMA A operand: row 0 = bf16(z), row 1 = bf16(z - bf16(z)), rows 2..15 = 0, so
  // Z Q'^T gives q'.z (to ~2^-17 relative) in rows 0 + 1 of each query column; z before
  // chunk c in buffer c % 2
  __shared__ Frag<true> sZf[2 * G::KB * 64];
  __shared__ unsigned sArrive;  // MMA-wave arrivals (mma_wave_sync)
  __shared__ unsigned sRelease;  // C = 128: the MMA waves' releases of the first block's buffers
  // C = 128: the cross-block weights of a chunk's second block go into the first block's Q'
  // buffer, which nothing reads in that step; at d = 32 that buffer is too small for them
  constexpr bool XOWN = C == 128 && BUFQ * 2 < 4 * 2 * 64 * 16;
  __shared__ Frag<true> sXown[XOWN ? 4 * 2 * 64 : 1];
  // L2, by step parity: rows' sums of squared weights (MMA waves) and the mappers' parts of
  // q'^T A_prev q', for the chunk the MMA waves processed in that step
  __shared__ float sRs2[L2 ? 2 * kChunk : 1];
  __shared__ float sQuad[L2 ? 2 * 4 * kChunk : 1];

  const int seg = blockIdx.x, h = blockIdx.y;
  if (seg >= *nseg) return;  // the whole workgroup leaves together
  const SegInfo si = read_seg(tab, seg);
  const int tid = threadIdx.x, lane = tid & 63;
  // wave index and chunk count in scalar registers: the role branches below are uniform
  // per wave, so every wave executes exactly its own role's barriers
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int nch = __builtin_amdgcn_readfirstlane((si.len + kChunk - 1) / kChunk);
  // steps 0 .. nch do work (the last one forms the last chunk's output); rounded up to even
  // for the mappers' two-step loop
  const int nsteps = (nch + 3) & ~1;
  const int c16 = lane & 15, g = lane >> 4;
  const size_t tok0 = ((size_t)si.row * H + h) * (size_t)L + si.start;
  const int seg_bytes = si.len * D * 2;
  const float* rec = states + ((size_t)seg * H + h) * (size_t)(D * D + D);
  if (tid == 0) sArrive = 0u;
  if constexpr (C == 128) {
    if (tid == 0) sRelease = 0u;
  }
  // z operand fragments (contiguous slot order): slot (g, j) of fragment kb holds dim
  // kb*32 + 8g + j; lane 16g holds bf16(z) there, lane 16g + 1 the residual, every other lane
  // zeros (written once). The initial z goes to buffer 0 (lane l converts dims 2l, 2l + 1);
  // later buffers are written by the column-sum lanes in the score phase.
  auto put_zf = [&](const float* zsrc) {
    uint16_t* zf16 = reinterpret_cast<uint16_t*>(sZf);
#pragma unroll
    for (int x = 0; x < 2 && 2 * lane + x < D; ++x) {
      const int dim = 2 * lane + x, kb2 = dim / 32, r = dim % 32;
      const int gg = r >> 3, j = r & 7;
      const float zv = zsrc[dim];
      const __bf16 hi = static_cast<__bf16>(zv);
      const __bf16 lo = static_cast<__bf16>(zv - static_cast<float>(hi));
      zf16[(kb2 * 64 + 16 * gg) * 8 + j] = __builtin_bit_cast(uint16_t, hi);
      zf16[(kb2 * 64 + 16 * gg + 1) * 8 + j] = __builtin_bit_cast(uint16_t, lo);
    }
  };
  for (int i = tid; i < 2 * G::KB * 64; i += 512) sZf[i] = Frag<true>{};
  __syncthreads();
  if (wave == 0) put_zf(rec + D * D);
  __syncthreads();

  const __amdgpu_buffer_rsrc_t ro = __builtin_amdgcn_make_buffer_rsrc((void*)(out + tok0 * D), 0, seg_bytes, kBufFlags);
  // Chunk st - 2's output rows, staged in sO[st % 2] in the previous step, leave as whole rows,
  // issued by NWAY waves (w = 0 .. NWAY - 1). In the sum mode all eight waves share them at
  // the end of the step (each role has some slack there, neither enough for all the stores;
  // at d = 32 one wave instruction covers 16 rows and the four MMA waves issue them);
  // with the L2 denominator the four mappers issue them (the MMA waves also carry the A
  // state). The same stores are issued every step: rows past the segment (and every row when
  // there is no such chunk) fall outside the buffer range and are dropped.
  constexpr int NWS = D >= 64 ? 8 : 4;  // waves sharing the stores in the sum mode
  auto store_rows_out = [&](int st, int w, auto nway_c) {
    constexpr int NWAY = decltype(nway_c)::value;
    constexpr int PPR = D / 8;     // 16-byte pieces per row
    constexpr int RPI = 64 / PPR;  // rows per wave instruction
    static_assert(kChunk % (NWAY * RPI) == 0, "whole rows per wave");
    const int cw = st - 2;
    const bool any = cw >= 0 && cw < nch;
    const St* so = sO + (st & 1) * BUF;
#pragma unroll
    for (int i = 0; i < kChunk / (NWAY * RPI); ++i) {
      const int rr = (i * NWAY + w) * RPI + lane / PPR, pc = lane % PPR;
      const int off = any ? ((cw * kChunk + rr) * D + pc * 8) * 2 : seg_bytes;
      u32x4 piece = *reinterpret_cast<const u32x4*>(so + rr * G::ROWP + pc * 8);
      if constexpr (L2) {  // the row's 1 / (sqrt(sum of squared scores) + eps), from step st - 1
        const int par = (st + 1) & 1;
        float quad = sRs2[par * kChunk + rr];
#pragma unroll
        for (int wv = 0; wv < G::NW; ++wv) quad += sQuad[(par * 4 + wv) * kChunk + rr];
        const float rsc = 1.0f / (__builtin_sqrtf(quad) + eps);
#pragma unroll
        for (int j = 0; j < 4; ++j)
          piece[j] = __builtin_bit_cast(uint32_t, __builtin_convertvector(
              float2v{__uint_as_float(piece[j] << 16) * rsc, __uint_as_float(piece[j] & 0xffff0000u) * rsc}, bf16x2));
      }
      __builtin_amdgcn_raw_buffer_store_b128(piece, ro, off, 0, kLoadStream);
    }
  };
  if (wave >= 4) {
    // ======== mappers: nsteps steps, one barrier each
    const int mt = tid & 255;  // two tokens per 8 lanes
    const int t0 = 2 * (mt >> 3), m = mt & 7;
    const __amdgpu_buffer_rsrc_t rq = __builtin_amdgcn_make_buffer_rsrc((void*)(q + tok0 * D), 0, seg_bytes, kBufFlags);
    const __amdgpu_buffer_rsrc_t rk = __builtin_amdgcn_make_buffer_rsrc((void*)(k + tok0 * D), 0, seg_bytes, kBufFlags);
    const __amdgpu_buffer_rsrc_t rv = __builtin_amdgcn_make_buffer_rsrc((void*)(v + tok0 * D), 0, seg_bytes, kBufFlags);
    // per-lane constants: RMSNorm weights of this lane's dims, in-chunk RoPE angles of its tokens
    float gq1[G::E], gq2[G::E], gk1[G::E], gk2[G::E];
    float2 lo[2][G::E];
#pragma unroll
    for (int e = 0; e < G::E; ++e) {
      const int j = m * G::E + e;
      gq1[e] = gamma_q[(size_t)h * D + j];
      gq2[e] = gamma_q[(size_t)h * D + j + G::HALF];
      gk1[e] = gamma_k[(size_t)h * D + j];
      gk2[e] = gamma_k[(size_t)h * D + j + G::HALF];
      lo[0][e] = rope_lo[t0 * G::HALF + j];
      lo[1][e] = rope_lo[(t0 + 1) * G::HALF + j];
    }
    // Every step issues the same loads (chunks past the end read zeros from the buffer
    // range check), so the compiler's wait counts let chunk st + 1 stay in flight while
    // chunk st is mapped.
    const float2* hi0 = rope_hi + (size_t)si.hirow * G::HALF + m * G::E;
    auto issue = [&](R (&r)[3], float2 (&hi)[G::E], int c) {  // in the order mstep refills
      load_raw_buf<true, D>(r[2], rv, c * kChunk + t0, m);
      load_raw_buf<true, D, 0>(r[0], rq, c * kChunk + t0, m);
      load_raw_buf<true, D, 0>(r[1], rk, c * kChunk + t0, m);
      load_raw_buf<true, D, 1>(r[0], rq, c * kChunk + t0, m);
      load_raw_buf<true, D, 1>(r[1], rk, c * kChunk + t0, m);
      copy_bytes<G::E * 8>(hi, hi0 + (size_t)min(c, nch - 1) * G::HALF);  // RoPE row of the chunk's start
    };
    auto mstep = [&](int st, R (&r)[3], float2 (&hi)[G::E]) {
      const int bm = (st & 1) * BUF;
      // The registers of chunk st are refilled with chunk cn as they free up: v (no mapping)
      // first, then q and k one token at a time, then the RoPE row, so the loads leave early.
      const int cn = st + 2;
      // C = 128: while the MMA waves process the second block of a chunk they still read the
      // first block's K' and V, and use the first block's Q' buffer for the cross-block weights,
      // all in the buffers of this step's parity; so in those steps (st even, the MMA waves on
      // block st - 1) every row of block st is held in registers and stored only once the MMA
      // waves have released the buffers (4 releases per such step on sRelease)
      const bool defer = C == 128 && (st & 1) == 0 && st >= 2 && st < nch;
      if (!defer) {
        if (st < nch) store_rows<true, D>(sV + bm, r[2], t0, m);
        load_raw_buf<true, D>(r[2], rv, cn * kChunk + t0, m);
      }
      R oq, ok;  // both tokens when deferred, else token by token
      auto map_tok = [&](auto tok_c) {
        constexpr int tok = decltype(tok_c)::value;
        if (st < nch) {
          const float invq = rms_inv<true, D>(r[0], tok, rms_eps);
          const float invk = rms_inv<true, D>(r[1], tok, rms_eps);
#pragma unroll
          for (int e = 0; e < G::E; e += 2) {
            float q1[2], q2[2], k1[2], k2[2];
#pragma unroll
            for (int x = 0; x < 2; ++x) {
              const float2 cs = angle_sum(hi[e + x], lo[tok][e + x]);
              rope_pair(r[0].get(tok, 0, e + x), r[0].get(tok, 1, e + x), invq, gq1[e + x], gq2[e + x], cs,
                        q1[x], q2[x]);
              rope_pair(r[1].get(tok, 0, e + x), r[1].get(tok, 1, e + x), invk, gk1[e + x], gk2[e + x], cs,
                        k1[x], k2[x]);
            }
            put_pairs<true, D>(oq, tok, e, q1, q2);
            put_pairs<true, D>(ok, tok, e, k1, k2);
          }
          if (!defer) {
            store_rows<true, D, tok>(sQ + (st & 1) * BUFQ, oq, t0, m, QP);
            store_rows<true, D, tok>(sK + (st & 1) * BUFQ, ok, t0, m, QP);
          }
        }
        load_raw_buf<true, D, tok>(r[0], rq, cn * kChunk + t0, m);
        load_raw_buf<true, D, tok>(r[1], rk, cn * kChunk + t0, m);
      };
      map_tok(std::integral_constant<int, 0>{});
      map_tok(std::integral_constant<int, 1>{});
      if constexpr (C == 128) {
        if (defer) {
          wait_count(&sRelease, 4u * (unsigned)(st / 2), lane, polls, hdr);
          store_rows<true, D>(sV + bm, r[2], t0, m);
          store_rows<true, D>(sQ + (st & 1) * BUFQ, oq, t0, m, QP);
          store_rows<true, D>(sK + (st & 1) * BUFQ, ok, t0, m, QP);
          load_raw_buf<true, D>(r[2], rv, cn * kChunk + t0, m);
        }
      }
      copy_bytes<G::E * 8>(hi, hi0 + (size_t)min(cn, nch - 1) * G::HALF);
      if constexpr (L2) store_rows_out(st, wave - 4, std::integral_constant<int, 4>{});
      else if constexpr (NWS == 8) store_rows_out(st, wave, std::integral_constant<int, 8>{});
      __syncthreads();  // Y
    };
    R set0[3], set1[3];
    float2 hi0r[G::E], hi1r[G::E];
    issue(set0, hi0r, 0);
    issue(set1, hi1r, 1);
    for (int st = 0; st < nsteps; st += 2) {
      mstep(st, set0, hi0r);
      mstep(st + 1, set1, hi1r);
    }
    return;
  }

  // ======== MMA waves: nsteps steps, one workgroup barrier each; step st processes chunk st - 1
  // running state, value columns of this wave, in the contiguous-order tile map: tiles 2kb and
  // 2kb + 1 pair up (acc_frag) into S^T operands whose slots match the 16-byte Q' fragments
  floatx4 S[G::RT][G::CT];
  floatx4 Am[L2 ? G::RT : 1][G::CT];  // L2: A = sum k'k'^T, the same columns and tile map as S
  {
    const int wv = wave < G::NW ? wave : 0;
    const float* arec = L2 ? astates + ((size_t)seg * H + h) * (size_t)(D * D + D) : nullptr;
#pragma unroll
    for (int rt = 0; rt < G::RT; ++rt)
#pragma unroll
      for (int ct = 0; ct < G::CT; ++ct) {
        S[rt][ct] = *reinterpret_cast<const floatx4*>(rec + rec_frag_c<D>(wv, rt, ct, lane));
        if constexpr (L2) Am[rt][ct] = *reinterpret_cast<const floatx4*>(arec + rec_frag_c<D>(wv, rt, ct, lane));
      }
  }
  // Accumulation order everywhere below: the contraction block is the outer loop and the
  // independent accumulators the inner one, so consecutive MFMAs never wait on each other.
  // column sums of K': row tiles [Z_w, Z_w+1) on wave w, more on the waves with fewer score
  // tiles (measured: a column-sum tile costs about 2.5 key tiles); their lanes (i, g), i < 4,
  // hold z of dims 16 tile + 4g + i
  constexpr int Z1 = G::RT == 8 ? 3 : G::RT / 2, Z2 = G::RT == 8 ? 5 : G::RT == 4 ? 3 : 2;
  constexpr int Z3 = G::RT == 8 ? 7 : G::RT;
  constexpr int NZR = G::RT == 8 ? 3 : G::RT / 2;
  float zreg[NZR];
  {
    const int z0 = wave == 0 ? 0 : wave == 1 ? Z1 : wave == 2 ? Z2 : Z3;
#pragma unroll
    for (int z = 0; z < NZR; ++z) {
      const int dim = min(16 * (z0 + z) + 4 * g + (c16 & 3), D - 1);
      zreg[z] = L2 ? 0.f : rec[D * D + dim];
    }
  }
  for (int st = 0; st < nsteps; ++st) {
    const St* cQ = sQ + ((st + 1) & 1) * BUFQ;  // buffers holding chunk st - 1
    const St* cK = sK + ((st + 1) & 1) * BUFQ;
    const St* cV = sV + ((st + 1) & 1) * BUF;
    const int c = st - 1;
    const bool work = st >= 1 && st <= nch;  // uniform over the MMA waves
    if (work) {  // ---- score: wave w owns query tile w
      if constexpr (L2) {
        float* rs2 = sRs2 + (st & 1) * kChunk;
        switch (wave) {
          case 0: ws_score<D, 0, 0, 0, NZR, true, C>(cQ, cK, QP, sZf, sZf, zreg, sA, rs2, eps, lane); break;
          case 1: ws_score<D, 1, 0, 0, NZR, true, C>(cQ, cK, QP, sZf, sZf, zreg, sA, rs2, eps, lane); break;
          case 2: ws_score<D, 2, 0, 0, NZR, true, C>(cQ, cK, QP, sZf, sZf, zreg, sA, rs2, eps, lane); break;
          default: ws_score<D, 3, 0, 0, NZR, true, C>(cQ, cK, QP, sZf, sZf, zreg, sA, rs2, eps, lane); break;
        }
      } else if constexpr (C == 128) {
        // block c of its chunk: the first (c even) or the second (c odd, with the first block's
        // keys in the other parity's K' buffer, its cross-block weights into the other parity's
        // Q' buffer, which no one reads in this step)
        const Frag<true>* zf = sZf + (c & 1) * G::KB * 64;  // z at the chunk's start
        Frag<true>* zn = sZf + ((c + 1) & 1) * G::KB * 64;
        const St* cKx = sK + (st & 1) * BUFQ;
        Frag<true>* sAx = XOWN ? sXown : reinterpret_cast<Frag<true>*>(sQ + (st & 1) * BUFQ);
        if (c & 1) {
          switch (wave) {
            case 0: ws_score<D, 0, 0, Z1, NZR, false, C, true, true>(cQ, cK, QP, zf, zn, zreg, sA, sInv, eps, lane, cKx, sAx); break;
            case 1: ws_score<D, 1, Z1, Z2, NZR, false, C, true, true>(cQ, cK, QP, zf, zn, zreg, sA, sInv, eps, lane, cKx, sAx); break;
            case 2: ws_score<D, 2, Z2, Z3, NZR, false, C, true, true>(cQ, cK, QP, zf, zn, zreg, sA, sInv, eps, lane, cKx, sAx); break;
            default: ws_score<D, 3, Z3, G::RT, NZR, false, C, true, true>(cQ, cK, QP, zf, zn, zreg, sA, sInv, eps, lane, cKx, sAx); break;
          }
        } else {
          switch (wave) {
            case 0: ws_score<D, 0, 0, Z1, NZR, false, C, false, false>(cQ, cK, QP, zf, zn, zreg, sA, sInv, eps, lane); break;
            case 1: ws_score<D, 1, Z1, Z2, NZR, false, C, false, false>(cQ, cK, QP, zf, zn, zreg, sA, sInv, eps, lane); break;
            case 2: ws_score<D, 2, Z2, Z3, NZR, false, C, false, false>(cQ, cK, QP, zf, zn, zreg, sA, sInv, eps, lane); break;
            default: ws_score<D, 3, Z3, G::RT, NZR, false, C, false, false>(cQ, cK, QP, zf, zn, zreg, sA, sInv, eps, lane); break;
          }
        }
      } else {
        const Frag<true>* zf = sZf + (c & 1) * G::KB * 64;  // z before chunk c
        Frag<true>* zn = sZf + ((c + 1) & 1) * G::KB * 64;  // z before chunk c + 1
        switch (wave) {
          case 0: ws_score<D, 0, 0, Z1, NZR, false, C>(cQ, cK, QP, zf, zn, zreg, sA, sInv, eps, lane); break;
          case 1: ws_score<D, 1, Z1, Z2, NZR, false, C>(cQ, cK, QP, zf, zn, zreg, sA, sInv, eps, lane); break;
          case 2: ws_score<D, 2, Z2, Z3, NZR, false, C>(cQ, cK, QP, zf, zn, zreg, sA, sInv, eps, lane); break;
          default: ws_score<D, 3, Z3, G::RT, NZR, false, C>(cQ, cK, QP, zf, zn, zreg, sA, sInv, eps, lane); break;
        }
      }
    }
    mma_wave_sync(&sArrive, 4u * (unsigned)(st + 1), lane, polls, hdr);
    if constexpr (C == 128) {
      if (work && wave < G::NW) {  // ---- output, then (second block) the chunk's state update
        const bool second = (c & 1) != 0;
        Frag<true> Vf[G::CT][2];
#pragma unroll
        for (int ct = 0; ct < G::CT; ++ct) {
          Vf[ct][0] = lds_frag_tr(cV, G::ROWP, 0, wave * G::DVW + ct * 16, lane);
          Vf[ct][1] = lds_frag_tr(cV, G::ROWP, 32, wave * G::DVW + ct * 16, lane);
        }
        floatx4 o[G::CT][4];
#pragma unroll
        for (int ct = 0; ct < G::CT; ++ct)
#pragma unroll
          for (int tt = 0; tt < 4; ++tt) o[ct][tt] = floatx4{0.f, 0.f, 0.f, 0.f};
        // S^T Q'^T with the state at the chunk's start (it advances only after the second block)
#pragma unroll
        for (int kb2 = 0; kb2 < G::KB; ++kb2) {
          Frag<true> sa[G::CT];
#pragma unroll
          for (int ct = 0; ct < G::CT; ++ct) sa[ct] = acc_frag<true>(S[2 * kb2][ct], S[2 * kb2 + 1][ct]);
#pragma unroll
          for (int tt = 0; tt < 4; ++tt) {
            const Frag<true> qf = lds_frag_c(cQ, QP, tt * 16 + c16, kb2, g);
#pragma unroll
            for (int ct = 0; ct < G::CT; ++ct) o[ct][tt] = mma(sa[ct], qf, o[ct][tt]);
          }
        }
        // the block's own keys (key-tile pairs up to the query tile's)
#pragma unroll
        for (int tt = 0; tt < 4; ++tt)
#pragma unroll
          for (int b = 0; b <= tt / 2; ++b) {
            const Frag<true> ab = sA[(tt * 2 + b) * 64 + lane];
#pragma unroll
            for (int ct = 0; ct < G::CT; ++ct) o[ct][tt] = mma(Vf[ct][b], ab, o[ct][tt]);
          }
        const St* pK = sK + (st & 1) * BUFQ;  // the chunk's first block (second block only)
        const St* pV = sV + (st & 1) * BUF;
        const Frag<true>* sAx = XOWN ? sXown : reinterpret_cast<const Frag<true>*>(sQ + (st & 1) * BUFQ);
        Frag<true> Vp[G::CT][2];
        if (second) {  // the first block's keys: every key-tile pair, for every query tile
#pragma unroll
          for (int ct = 0; ct < G::CT; ++ct) {
            Vp[ct][0] = lds_frag_tr(pV, G::ROWP, 0, wave * G::DVW + ct * 16, lane);
            Vp[ct][1] = lds_frag_tr(pV, G::ROWP, 32, wave * G::DVW + ct * 16, lane);
          }
#pragma unroll
          for (int tt = 0; tt < 4; ++tt)
#pragma unroll
            for (int b = 0; b < 2; ++b) {
              const Frag<true> ab = sAx[(tt * 2 + b) * 64 + lane];
#pragma unroll
              for (int ct = 0; ct < G::CT; ++ct) o[ct][tt] = mma(Vp[ct][b], ab, o[ct][tt]);
            }
        }
#pragma unroll
        for (int tt = 0; tt < 4; ++tt) {
          const int t = tt * 16 + c16;
          const float rr = sInv[t];
#pragma unroll
          for (int ct = 0; ct < G::CT; ++ct) {
            const int col = wave * G::DVW + ct * 16 + 4 * g;
            const uint32_t w0 = __builtin_bit_cast(uint32_t, __builtin_convertvector(float2v{o[ct][tt][0] * rr, o[ct][tt][1] * rr}, bf16x2));
            const uint32_t w1 = __builtin_bit_cast(uint32_t, __builtin_convertvector(float2v{o[ct][tt][2] * rr, o[ct][tt][3] * rr}, bf16x2));
            *reinterpret_cast<uint2*>(sO + (c & 1) * BUF + t * G::ROWP + col) = make_uint2(w0, w1);
          }
        }
        if (second) {  // S += K'^T V over both blocks of the chunk
#pragma unroll
          for (int blk = 0; blk < 2; ++blk) {
            const St* kb = blk == 0 ? pK : cK;
#pragma unroll
            for (int kb2 = 0; kb2 < 2; ++kb2) {
#pragma unroll
              for (int rt = 0; rt < G::RT; ++rt) {
                const Frag<true> a = lds_frag_tr_s8(kb, QP, 32 * kb2, 32 * (rt / 2) + 4 * (rt % 2), lane);
#pragma unroll
                for (int ct = 0; ct < G::CT; ++ct) S[rt][ct] = mma(a, blk == 0 ? Vp[ct][kb2] : Vf[ct][kb2], S[rt][ct]);
              }
            }
          }
        }
      }
      // every MMA wave hands the first block's buffers back to the mappers after the second
      // block (its last reads of them are above; the release orders them before the count)
      if (work && (c & 1) && lane == 0)
        __hip_atomic_fetch_add(&sRelease, 1u, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);
    } else if (work && wave < G::NW) {  // ---- output, then the state update
      Frag<true> Vf[G::CT][2];
#pragma unroll
      for (int ct = 0; ct < G::CT; ++ct) {
        Vf[ct][0] = lds_frag_tr(cV, G::ROWP, 0, wave * G::DVW + ct * 16, lane);
        Vf[ct][1] = lds_frag_tr(cV, G::ROWP, 32, wave * G::DVW + ct * 16, lane);
      }
      // S += K'^T V over the step's chunk u (C = 64: the whole step; C = 32: k-block u; C = 16:
      // half of k-block u / 2, the other half's slots of the V operand zeroed)
      constexpr int TPS = C / 16, NSUB = kChunk / C;  // query tiles per chunk, chunks per step
      auto advance = [&](int u) {
#pragma unroll
        for (int kb2 = 0; kb2 < 2; ++kb2) {
          if (C == 32 && kb2 != u) continue;
          if (C == 16 && kb2 != u / 2) continue;
          Frag<true> vb[G::CT];
#pragma unroll
          for (int ct = 0; ct < G::CT; ++ct) {
            vb[ct] = Vf[ct][kb2];
            if constexpr (C == 16) {  // slots j < 4: tokens 32 kb2 + 4g + j; j >= 4: 16 further
#pragma unroll
              for (int j = 0; j < 4; ++j) vb[ct].v[(u & 1) ? j : 4 + j] = static_cast<__bf16>(0.f);
            }
          }
#pragma unroll
          for (int rt = 0; rt < G::RT; ++rt) {
            const Frag<true> a = lds_frag_tr_s8(cK, QP, 32 * kb2, 32 * (rt / 2) + 4 * (rt % 2), lane);
#pragma unroll
            for (int ct = 0; ct < G::CT; ++ct) S[rt][ct] = mma(a, vb[ct], S[rt][ct]);
          }
        }
      };
      // O^T for the 64 rows and this wave's columns, chunk by chunk: the query tiles of chunk u
      // read the state before chunk u (advanced past the step's earlier chunks) and the weights
      // of chunk u's own keys; each Q' fragment is read once and serves every column tile
      floatx4 o[G::CT][4];
#pragma unroll
      for (int ct = 0; ct < G::CT; ++ct)
#pragma unroll
        for (int tt = 0; tt < 4; ++tt) o[ct][tt] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int u = 0; u < NSUB; ++u) {
        if (u > 0) advance(u - 1);
#pragma unroll
        for (int kb2 = 0; kb2 < G::KB; ++kb2) {
          Frag<true> sa[G::CT];  // S^T rounded to bf16 as the A operand
#pragma unroll
          for (int ct = 0; ct < G::CT; ++ct) sa[ct] = acc_frag<true>(S[2 * kb2][ct], S[2 * kb2 + 1][ct]);
#pragma unroll
          for (int tt = u * TPS; tt < (u + 1) * TPS; ++tt) {
            const Frag<true> qf = lds_frag_c(cQ, QP, tt * 16 + c16, kb2, g);
#pragma unroll
            for (int ct = 0; ct < G::CT; ++ct) o[ct][tt] = mma(sa[ct], qf, o[ct][tt]);
          }
        }
        // the weights of the chunk's keys: key-tile pairs b (tiles 2b, 2b + 1) from the
        // chunk's first pair up to the query tile's
#pragma unroll
        for (int tt = u * TPS; tt < (u + 1) * TPS; ++tt)
#pragma unroll
          for (int b = (u * TPS) / 2; b <= tt / 2; ++b) {
            const Frag<true> ab = sA[(tt * 2 + b) * 64 + lane];
#pragma unroll
            for (int ct = 0; ct < G::CT; ++ct) o[ct][tt] = mma(Vf[ct][b], ab, o[ct][tt]);
          }
      }
      // each lane holds 4 consecutive columns of one row: 8-byte range-checked stores (rows
      // past the segment fall outside the buffer range and are dropped)
#pragma unroll
      for (int tt = 0; tt < 4; ++tt) {
        const int t = tt * 16 + c16;  // this lane's query row
        const float rr = L2 ? 1.0f : sInv[t];  // L2: normalised when the row leaves, a step later
#pragma unroll
        for (int ct = 0; ct < G::CT; ++ct) {  // columns col .. col + 3
          const int col = wave * G::DVW + ct * 16 + 4 * g;
          const uint32_t w0 = __builtin_bit_cast(uint32_t, __builtin_convertvector(float2v{o[ct][tt][0] * rr, o[ct][tt][1] * rr}, bf16x2));
          const uint32_t w1 = __builtin_bit_cast(uint32_t, __builtin_convertvector(float2v{o[ct][tt][2] * rr, o[ct][tt][3] * rr}, bf16x2));
          *reinterpret_cast<uint2*>(sO + (c & 1) * BUF + t * G::ROWP + col) = make_uint2(w0, w1);
        }
      }
      advance(NSUB - 1);  // the step's last chunk (C = 64: the whole step)
      if constexpr (L2) {  // q'^T A_prev q' of chunk c (this wave's columns, to LDS), then A += K'^T K'
        Frag<true> aa[G::KB][G::CT];  // A_prev (symmetric) rounded to bf16 as the A operand
#pragma unroll
        for (int kb2 = 0; kb2 < G::KB; ++kb2)
#pragma unroll
          for (int ct = 0; ct < G::CT; ++ct) aa[kb2][ct] = acc_frag<true>(Am[2 * kb2][ct], Am[2 * kb2 + 1][ct]);
#pragma unroll
        for (int tt = 0; tt < 4; ++tt) {
          float part = 0.f;
#pragma unroll
          for (int ct = 0; ct < G::CT; ++ct) {
            floatx4 y = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kb2 = 0; kb2 < G::KB; ++kb2) y = mma(aa[kb2][ct], lds_frag_c(cQ, QP, tt * 16 + c16, kb2, g), y);
            const int col = wave * G::DVW + ct * 16 + 4 * g;
            const uint2 qa = *reinterpret_cast<const uint2*>(cQ + (tt * 16 + c16) * QP + col);
            part = __builtin_fmaf(__uint_as_float(qa.x << 16), y[0], part);
            part = __builtin_fmaf(__uint_as_float(qa.x & 0xffff0000u), y[1], part);
            part = __builtin_fmaf(__uint_as_float(qa.y << 16), y[2], part);
            part = __builtin_fmaf(__uint_as_float(qa.y & 0xffff0000u), y[3], part);
          }
          part = sum_rows4(part);
          if (g == 0) sQuad[((st & 1) * 4 + wave) * kChunk + tt * 16 + c16] = part;
        }
#pragma unroll
        for (int kb2 = 0; kb2 < 2; ++kb2) {
          Frag<true> Kc[G::CT];
#pragma unroll
          for (int ct = 0; ct < G::CT; ++ct) Kc[ct] = lds_frag_tr(cK, QP, 32 * kb2, wave * G::DVW + ct * 16, lane);
#pragma unroll
          for (int rt = 0; rt < G::RT; ++rt) {
            const Frag<true> a = lds_frag_tr_s8(cK, QP, 32 * kb2, 32 * (rt / 2) + 4 * (rt % 2), lane);
#pragma unroll
            for (int ct = 0; ct < G::CT; ++ct) Am[rt][ct] = mma(a, Kc[ct], Am[rt][ct]);
          }
        }
      }
    }
    if constexpr (!L2) store_rows_out(st, wave, std::integral_constant<int, NWS>{});
    __syncthreads();  // Y
  }
}

// ----------------------------------------------------------------------------------------
// readout (bidirectional forward): per (segment, head), every token reads its document's
// whole state, out_t = q'_t S_doc / (q'_t . z_doc + eps). The document state arrives in the
// segment's record (fragment-native S, then z); the state waves round it once to the MFMA
// operand type and keep it in registers. Software-pipelined over the chunks with one barrier
// per step: step c maps q of chunk c + 1 (every lane, two tokens per 8 lanes) into one half of
// a double-buffered LDS, the state waves form O^T = S^T Q'^T of chunk c from the other half,
// scale each row by 1/(q'.z + eps) and stage it, and every lane writes the staged rows of
// chunk c - 1 as whole rows (range-checked buffer stores). Raw q and the RoPE row of the next
// two chunks are in flight in registers. q'.z: bf16, one more MFMA tile per state wave, z as
// the bf16 pair hi + lo (rows 4i hold hi, rows 4i + 1 lo, so every lane's accumulator has
// both for its token; products exact, fp32 sums); fp32, a dot product in the map step.
// L2 (the original RLA's denominator over the whole document, RLA page §2.1, §4.1 causal=false):
// out_t = q'_t S_doc / (sqrt(q'_t^T A_doc q'_t) + eps). The second document state A arrives in
// its own records; the state waves also hold it as MFMA operands, form A Q'^T beside S^T Q'^T and
// dot it with q' for their part of each row's quadratic form (LDS, by chunk parity). The rows are
// staged unnormalised and scaled by 1/(sqrt(q'^T A q') + eps) as they leave in the next step,
// after the barrier that completes the quadratic forms (bf16: rounded twice, <= 2 2^-9 relative).

template <bool BF, int D, bool L2>
__global__ __launch_bounds__(NT, (L2 && D == 128) ? 1 : 2) void readout_kernel(
    const typename Elem<BF>::St* __restrict__ q, const float* __restrict__ gamma_q, const int32_t* __restrict__ tab,
    const int32_t* __restrict__ nseg, const float2* __restrict__ rope_lo, const float2* __restrict__ rope_hi,
    const float* __restrict__ states, const float* __restrict__ astates, typename Elem<BF>::St* __restrict__ out,
    int H, int L, float rms_eps, float eps) {
  using G = Geo<BF, D>;
  using St = typename G::St;
  using R = Raw<BF, D>;
  constexpr int BUF = kChunk * G::ROWP;     // elements of one output row buffer
  constexpr int EPP = 16 / G::ES;           // elements per 16-byte piece
  constexpr int PPR = D / EPP;              // 16-byte pieces per row
  // bf16: Q' rows at a pitch of D + 16 for conflict-free 16-byte row-fragment reads
  constexpr int QP = BF ? D + 16 : G::ROWP, BUFQ = kChunk * QP;
  __shared__ __attribute__((aligned(16))) St sQ[2 * BUFQ];
  __shared__ __attribute__((aligned(16))) St sO[2 * BUF];
  __shared__ __attribute__((aligned(16))) float sZ[D];
  __shared__ float sInv[2 * kChunk];
  __shared__ float sQuad[L2 ? 2 * 4 * kChunk : 1];  // L2: each state wave's part of q'^T A q', by chunk parity

  const int seg = blockIdx.x, h = blockIdx.y;
  if (seg >= *nseg) return;  // the whole workgroup leaves together
  const SegInfo si = read_seg(tab, seg);
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int nch = __builtin_amdgcn_readfirstlane((si.len + kChunk - 1) / kChunk);
  const int t0 = 2 * (tid >> 3), m = tid & 7;
  const int c16 = lane & 15, g = lane >> 4;
  const size_t tok0 = ((size_t)si.row * H + h) * (size_t)L + si.start;
  const int seg_bytes = si.len * D * G::ES;
  const __amdgpu_buffer_rsrc_t rq = __builtin_amdgcn_make_buffer_rsrc((void*)(q + tok0 * D), 0, seg_bytes, kBufFlags);
  const __amdgpu_buffer_rsrc_t ro = __builtin_amdgcn_make_buffer_rsrc((void*)(out + tok0 * D), 0, seg_bytes, kBufFlags);
  const float* rec = states + ((size_t)seg * H + h) * (size_t)(D * D + D);
  if (tid < D) sZ[tid] = rec[D * D + tid];
  float g1[G::E], g2[G::E];
  float2 lo[2][G::E];
#pragma unroll
  for (int e = 0; e < G::E; ++e) {
    const int j = m * G::E + e;
    g1[e] = gamma_q[(size_t)h * D + j];
    g2[e] = gamma_q[(size_t)h * D + j + G::HALF];
    lo[0][e] = rope_lo[t0 * G::HALF + j];
    lo[1][e] = rope_lo[(t0 + 1) * G::HALF + j];
  }
  // S^T as the A operand of O^T = S^T Q'^T, value columns of this wave (bf16: read into the
  // contiguous-order tile map, whose slots match the 16-byte Q' fragments)
  Frag<BF> sa[G::KB][G::CT];
  Frag<BF> aa[L2 ? G::KB : 1][G::CT];  // L2: A (symmetric, so A^T) in the same tile map
  {
    const int wv = wave < G::NW ? wave : 0;
    auto tile = [&](const float* r, int rt, int ct) {
      if constexpr (BF) return *reinterpret_cast<const floatx4*>(r + rec_frag_c<D>(wv, rt, ct, lane));
      else return *reinterpret_cast<const floatx4*>(r + rec_frag<BF, D>(wv, rt, ct, lane));
    };
    const float* arec = L2 ? astates + ((size_t)seg * H + h) * (size_t)(D * D + D) : nullptr;
#pragma unroll
    for (int kb2 = 0; kb2 < G::KB; ++kb2)
#pragma unroll
      for (int ct = 0; ct < G::CT; ++ct) {
        sa[kb2][ct] = acc_frag<BF>(tile(rec, 2 * kb2, ct), tile(rec, 2 * kb2 + 1, ct));
        if constexpr (L2) aa[kb2][ct] = acc_frag<BF>(tile(arec, 2 * kb2, ct), tile(arec, 2 * kb2 + 1, ct));
      }
  }
  // bf16: z as the A operand of the q'.z tile, contiguous slot order (slot (g, j) of k-block kb
  // is dim 32 kb + 8g + j): rows 4i hold bf16(z), rows 4i + 1 the residual, the rest zeros
  Frag<true> zfr[BF ? G::KB : 1];
  if constexpr (BF && !L2) {
#pragma unroll
    for (int kb2 = 0; kb2 < G::KB; ++kb2)
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const float zv = rec[D * D + 32 * kb2 + 8 * g + j];
        const __bf16 zh = static_cast<__bf16>(zv);
        const __bf16 zl = static_cast<__bf16>(zv - static_cast<float>(zh));
        zfr[kb2].v[j] = (c16 & 3) == 0 ? zh : (c16 & 3) == 1 ? zl : static_cast<__bf16>(0.f);
      }
  }
  const float2* hi0 = rope_hi + (size_t)si.hirow * G::HALF + m * G::E;
  auto issue = [&](R& r, float2 (&hi)[G::E], int c) {  // in the order map_chunk refills
    load_raw_buf<BF, D>(r, rq, c * kChunk + t0, m);
    copy_bytes<G::E * 8>(hi, hi0 + (size_t)min(c, nch - 1) * G::HALF);  // RoPE row of the chunk's start
  };
  // q' of chunk c into sQ[c % 2] (fp32: with its row reciprocals); the registers are refilled with
  // chunk c + 2 one token at a time as they free up, then the RoPE row
  auto map_chunk = [&](int c, R& r, float2 (&hi)[G::E]) {
    auto map_tok = [&](auto tok_c) {
      constexpr int tok = decltype(tok_c)::value;
      R o;
      feature_map_lane<BF, D, tok>(r, o, g1, g2, lo, hi, rms_eps);
      store_rows<BF, D, tok>(sQ + (c & 1) * BUFQ, o, t0, m, QP);
      if constexpr (!BF && !L2) {  // fp32: q'.z here, against z in LDS
        float p = 0.f;
#pragma unroll
        for (int e = 0; e < G::E; ++e) {
          p = __builtin_fmaf(o.get(tok, 0, e), sZ[m * G::E + e], p);
          p = __builtin_fmaf(o.get(tok, 1, e), sZ[G::HALF + m * G::E + e], p);
        }
        p = sum8(p);
        if (m == 0) sInv[(c & 1) * kChunk + t0 + tok] = 1.0f / (p + eps);
      }
      load_raw_buf<BF, D, tok>(r, rq, (c + 2) * kChunk + t0, m);
    };
    map_tok(std::integral_constant<int, 0>{});
    map_tok(std::integral_constant<int, 1>{});
    copy_bytes<G::E * 8>(hi, hi0 + (size_t)min(c + 2, nch - 1) * G::HALF);
  };
  // O^T of chunk c for this wave's value columns, all 64 rows, staged in sO[c % 2]
  auto mma_chunk = [&](int c) {
    const St* cQ = sQ + (c & 1) * BUFQ;
    St* cO = sO + (c & 1) * BUF;
    floatx4 o4[G::CT][4], dn[4], y4[L2 ? G::CT : 1][4];
#pragma unroll
    for (int t4 = 0; t4 < 4; ++t4) {
      dn[t4] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ct = 0; ct < G::CT; ++ct) o4[ct][t4] = floatx4{0.f, 0.f, 0.f, 0.f};
      if constexpr (L2) {
#pragma unroll
        for (int ct = 0; ct < G::CT; ++ct) y4[ct][t4] = floatx4{0.f, 0.f, 0.f, 0.f};
      }
    }
#pragma unroll
    for (int kb2 = 0; kb2 < G::KB; ++kb2)
#pragma unroll
      for (int t4 = 0; t4 < 4; ++t4) {
        Frag<BF> qf;
        if constexpr (BF) qf = lds_frag_c(cQ, QP, t4 * 16 + c16, kb2, g);
        else qf = lds_frag<BF>(cQ, QP, t4 * 16 + c16, kb2, g);
#pragma unroll
        for (int ct = 0; ct < G::CT; ++ct) {
          o4[ct][t4] = mma(sa[kb2][ct], qf, o4[ct][t4]);
          if constexpr (L2) y4[ct][t4] = mma(aa[kb2][ct], qf, y4[ct][t4]);
        }
        if constexpr (BF && !L2) dn[t4] = mma(zfr[kb2], qf, dn[t4]);
      }
    if constexpr (L2) {  // this wave's part of q'^T A q' for every row of the chunk
#pragma unroll
      for (int t4 = 0; t4 < 4; ++t4) {
        float part = 0.f;
#pragma unroll
        for (int ct = 0; ct < G::CT; ++ct) {
          const St* qrow = cQ + (t4 * 16 + c16) * QP + wave * G::DVW + ct * 16 + 4 * g;  // q' at the columns
#pragma unroll
          for (int i = 0; i < 4; ++i) part = __builtin_fmaf(Elem<BF>::to_f(qrow[i]), y4[ct][t4][i], part);
        }
        part = sum_rows4(part);
        if (g == 0) sQuad[((c & 1) * 4 + wave) * kChunk + t4 * 16 + c16] = part;
      }
    }
#pragma unroll
    for (int t4 = 0; t4 < 4; ++t4) {
      const int t = t4 * 16 + c16;  // this lane's row; columns col .. col + 3
      float rr;
      if constexpr (L2) rr = 1.f;  // scaled as the row leaves
      else if constexpr (BF) rr = 1.0f / (dn[t4][0] + dn[t4][1] + eps);
      else rr = sInv[(c & 1) * kChunk + t];
#pragma unroll
      for (int ct = 0; ct < G::CT; ++ct) {
        const int col = wave * G::DVW + ct * 16 + 4 * g;
        if constexpr (BF) {
          const uint32_t w0 = __builtin_bit_cast(uint32_t, __builtin_convertvector(float2v{o4[ct][t4][0] * rr, o4[ct][t4][1] * rr}, bf16x2));
          const uint32_t w1 = __builtin_bit_cast(uint32_t, __builtin_convertvector(float2v{o4[ct][t4][2] * rr, o4[ct][t4][3] * rr}, bf16x2));
          *reinterpret_cast<uint2*>(cO + t * G::ROWP + col) = make_uint2(w0, w1);
        } else {
          *reinterpret_cast<float4*>(cO + t * G::ROWP + col) =
              make_float4(o4[ct][t4][0] * rr, o4[ct][t4][1] * rr, o4[ct][t4][2] * rr, o4[ct][t4][3] * rr);
        }
      }
    }
  };
  // the staged rows of chunk c (rows past the segment are dropped by the range check)
  auto store_chunk = [&](int c) {
    const St* cO = sO + (c & 1) * BUF;
#pragma unroll
    for (int i = tid; i < kChunk * PPR; i += NT) {
      const int rr = i / PPR, pc = i % PPR;
      u32x4 piece = *reinterpret_cast<const u32x4*>(cO + rr * G::ROWP + pc * EPP);
      if constexpr (L2) {  // 1/(sqrt(q'^T A q') + eps) of the row, from the state waves' parts
        float quad = 0.f;
#pragma unroll
        for (int w = 0; w < G::NW; ++w) quad += sQuad[((c & 1) * 4 + w) * kChunk + rr];
        const float sc = 1.0f / (__builtin_sqrtf(quad) + eps);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          if constexpr (BF) {
            piece[j] = __builtin_bit_cast(uint32_t, __builtin_convertvector(
                float2v{__uint_as_float(piece[j] << 16) * sc, __uint_as_float(piece[j] & 0xffff0000u) * sc}, bf16x2));
          } else {
            piece[j] = __float_as_uint(__uint_as_float(piece[j]) * sc);
          }
        }
      }
      __builtin_amdgcn_raw_buffer_store_b128(piece, ro, ((c * kChunk + rr) * D + pc * EPP) * G::ES, 0, kLoadStream);
    }
  };
  R set0, set1;
  float2 hs0[G::E], hs1[G::E];
  issue(set0, hs0, 0);
  issue(set1, hs1, 1);
  __syncthreads();  // z in LDS
  map_chunk(0, set0, hs0);
  __syncthreads();
  // steps s = 0 .. nch: map chunk s + 1, MMA of chunk s, store of chunk s - 1. Every
  // condition below is uniform over the workgroup, so all waves meet every barrier.
  for (int c = 0; c <= nch; c += 2) {
    if (c + 1 < nch) map_chunk(c + 1, set1, hs1);
    if (c < nch && wave < G::NW) mma_chunk(c);
    if (c >= 1) store_chunk(c - 1);
    __syncthreads();
    if (c + 1 > nch) break;
    if (c + 2 < nch) map_chunk(c + 2, set0, hs0);
    if (c + 1 < nch && wave < G::NW) mma_chunk(c + 1);
    store_chunk(c);
    __syncthreads();
  }
}

// ----------------------------------------------------------------------------------------
// readout_l2_ql (bidirectional forward with the L2 denominator, bf16, d = 64 or 128): the
// read-out on token-split tiles. Every output row needs only its own q and the document's
// states, so each wave carries whole 16-token tiles from the raw q to the stored row in
// registers (the lane layout of QL above): RMS statistic over the token's four lanes, RoPE
// and ReLU in the lane, O^T = S^T Q'^T and A Q'^T on the MFMA with S^T and A (A is symmetric;
// both rounded once to bf16) as A operands that the workgroup builds in LDS from the segment's
// records, q'^T A q' in the lane and over its four lanes, and the row stored as 16-byte
// pieces. The loop has no barrier and no LDS traffic besides those operand reads and the
// segment's RoPE and gamma rows. 8 waves, one workgroup per CU; wave w takes the 16-token tile
// w % 4 of chunks w / 4, w / 4 + 2, ..., two tiles per pass, so a lane's in-chunk position,
// and with it its row of the fine RoPE table, is fixed for the whole loop.

template <int D>
__global__ __launch_bounds__(512, 2) void readout_l2_ql_kernel(
    const uint16_t* __restrict__ q, const float* __restrict__ gamma_q, const int32_t* __restrict__ tab,
    const int32_t* __restrict__ nseg, const float2* __restrict__ rope_lo, const float2* __restrict__ rope_hi,
    const float* __restrict__ states, const float* __restrict__ astates, uint16_t* __restrict__ out, int H, int L,
    float rms_eps, float eps) {
  using Q = QL<D>;
  constexpr int KB = Q::KB, NP = Q::NP, R = Q::R, HALF = D / 2;
  __shared__ Frag<true> sS[R * KB * 64];  // S^T operands [tile][k-block][lane]
  __shared__ Frag<true> sA[R * KB * 64];  // A operands
  __shared__ __attribute__((aligned(16))) float2 sHi[kMaxSegChunks * HALF];  // the segment's RoPE chunk rows
  __shared__ __attribute__((aligned(16))) float sGam[D];  // gamma_q of the head

  const int seg = blockIdx.x, h = blockIdx.y;
  if (seg >= *nseg) return;  // the whole workgroup leaves together
  const SegInfo si = read_seg(tab, seg);
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int nch = __builtin_amdgcn_readfirstlane((si.len + kChunk - 1) / kChunk);
  const int c16 = lane & 15, g = lane >> 4;
  const size_t tok0 = ((size_t)si.row * H + h) * (size_t)L + si.start;
  const int seg_bytes = si.len * D * 2;
  const __amdgpu_buffer_rsrc_t rq = __builtin_amdgcn_make_buffer_rsrc((void*)(q + tok0 * D), 0, seg_bytes, kBufFlags);
  const __amdgpu_buffer_rsrc_t ro = __builtin_amdgcn_make_buffer_rsrc((void*)(out + tok0 * D), 0, seg_bytes, kBufFlags);
  const float* rec = states + ((size_t)seg * H + h) * (size_t)(D * D + D);
  ql_operands<D, true>(reinterpret_cast<uint16_t*>(sS), nullptr, rec, tid, 512);
  ql_operands<D, true>(reinterpret_cast<uint16_t*>(sA), nullptr, astates + ((size_t)seg * H + h) * (size_t)(D * D + D),
                       tid, 512);
  for (int i = tid; i < min(nch, kMaxSegChunks) * HALF; i += 512) sHi[i] = rope_hi[(size_t)si.hirow * HALF + i];
  if (tid < D) sGam[tid] = gamma_q[(size_t)h * D + tid];
  const int pos = (wave & 3) * 16 + c16;  // the lane's in-chunk position
  float2 lo[NP][8];
#pragma unroll
  for (int kb = 0; kb < NP; ++kb)
#pragma unroll
    for (int j = 0; j < 8; ++j) lo[kb][j] = rope_lo[pos * HALF + 32 * kb + 8 * g + j];
  __syncthreads();  // operands, gamma and RoPE rows in LDS

  // two tiles per pass, tile u of chunk c + 2u (chunks past the segment read zeros and are never
  // stored), so that every operand fragment read from LDS serves both
  // each tile's registers are refilled with its tile of the next pass as soon as the tile is
  // mapped, so the raw q of the next pass is in flight during this pass's products and stores
  auto pass = [&](int c, u32x4 (&x0)[KB], u32x4 (&x1)[KB]) {
    // the operands are read from LDS per pass: kept in registers across the loop (the
    // compiler's choice, as the LDS does not change) they would take 128 VGPRs at d = 128
    asm volatile("" ::: "memory");
    Frag<true> qf[2][KB];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      u32x4(&x)[KB] = u ? x1 : x0;
      const int cu = min(c + 2 * u, nch - 1);  // the RoPE row (a chunk past the segment maps zeros)
      const float inv = ql_rms_inv<D>(x, rms_eps);
      float2 cs[NP][8];
#pragma unroll
      for (int kb = 0; kb < NP; ++kb)
#pragma unroll
        for (int j = 0; j < 8; ++j) cs[kb][j] = angle_sum(sHi[cu * HALF + 32 * kb + 8 * g + j], lo[kb][j]);
      float gam[KB][8];  // gamma at the lane's dims (LDS broadcast reads)
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) copy_bytes<32>(gam[kb], sGam + 32 * kb + 8 * g);
      ql_map<D>(x, inv, gam, cs, qf[u]);
      ql_load<D>(x, rq, (c + 4 + 2 * u) * kChunk + pos, g);
    }
    floatx4 o[2][R];
    float quad[2][2] = {{0.f, 0.f}, {0.f, 0.f}};  // two chains per tile
#pragma unroll
    for (int t = 0; t < R; ++t) {
      o[0][t] = o[1][t] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
        const Frag<true> f = sS[(t * KB + kb) * 64 + lane];
        o[0][t] = mma(f, qf[0][kb], o[0][t]);
        o[1][t] = mma(f, qf[1][kb], o[1][t]);
      }
      // q'^T A q' from A Q'^T: tile 2p + h row 4g + i is dim 32 p + 8g + 4h + i
      floatx4 y[2] = {floatx4{0.f, 0.f, 0.f, 0.f}, floatx4{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
        const Frag<true> f = sA[(t * KB + kb) * 64 + lane];
        y[0] = mma(f, qf[0][kb], y[0]);
        y[1] = mma(f, qf[1][kb], y[1]);
      }
#pragma unroll
      for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          quad[u][t & 1] = __builtin_fmaf(static_cast<float>(qf[u][t >> 1].v[4 * (t & 1) + i]), y[u][i], quad[u][t & 1]);
    }
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const float rr = 1.0f / (__builtin_sqrtf(sum_rows4(quad[u][0] + quad[u][1])) + eps);
      const int tok = (c + 2 * u) * kChunk + pos;
#pragma unroll
      for (int p = 0; p < KB; ++p) {
        u32x4 w;
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
          w[2 * hh] = pack_bf2(o[u][2 * p + hh][0] * rr, o[u][2 * p + hh][1] * rr);
          w[2 * hh + 1] = pack_bf2(o[u][2 * p + hh][2] * rr, o[u][2 * p + hh][3] * rr);
        }
        __builtin_amdgcn_raw_buffer_store_b128(w, ro, (tok * D + 32 * p + 8 * g) * 2, 0, 0);  // past the segment: dropped
      }
    }
  };
  // chunks c0, c0 + 2, ... in passes of two
  const int c0 = wave >> 2;
  u32x4 xa[KB], xb[KB];
  ql_load<D>(xa, rq, c0 * kChunk + pos, g);
  ql_load<D>(xb, rq, (c0 + 2) * kChunk + pos, g);
  for (int c = c0; c < nch; c += 4) pass(c, xa, xb);
}

// ----------------------------------------------------------------------------------------
// feature_map: the preamble alone, x' = ReLU(RoPE(RMSNorm(x))) materialised. Per (segment,
// head, tensor): the same lane mapping and device functions as the chunk kernels (two
// tokens per 8 lanes), so x' is bitwise what the forward forms internally; raw x and the
// RoPE row of the next two chunks in flight in registers; each lane writes its elements back
// with range-checked buffer stores (tokens past the segment are dropped).

template <bool BF, int D>
__global__ __launch_bounds__(NT, 2) void feature_map_kernel(
    const typename Elem<BF>::St* __restrict__ q, const typename Elem<BF>::St* __restrict__ k,
    const float* __restrict__ gamma_q, const float* __restrict__ gamma_k, const int32_t* __restrict__ tab,
    const int32_t* __restrict__ nseg, const float2* __restrict__ rope_lo, const float2* __restrict__ rope_hi,
    typename Elem<BF>::St* __restrict__ q_out, typename Elem<BF>::St* __restrict__ k_out, int H, int L,
    float rms_eps) {
  using G = Geo<BF, D>;
  using R = Raw<BF, D>;
  const int seg = blockIdx.x, h = blockIdx.y;
  const auto* x = blockIdx.z == 0 ? q : k;
  auto* y = blockIdx.z == 0 ? q_out : k_out;
  const float* gamma = blockIdx.z == 0 ? gamma_q : gamma_k;
  if (seg >= *nseg || x == nullptr) return;  // the whole workgroup leaves together
  const SegInfo si = read_seg(tab, seg);
  const int tid = threadIdx.x;
  const int nch = __builtin_amdgcn_readfirstlane((si.len + kChunk - 1) / kChunk);
  const int t0 = 2 * (tid >> 3), m = tid & 7;
  const size_t tok0 = ((size_t)si.row * H + h) * (size_t)L + si.start;
  const int seg_bytes = si.len * D * G::ES;
  const __amdgpu_buffer_rsrc_t rx = __builtin_amdgcn_make_buffer_rsrc((void*)(x + tok0 * D), 0, seg_bytes, kBufFlags);
  const __amdgpu_buffer_rsrc_t ry = __builtin_amdgcn_make_buffer_rsrc((void*)(y + tok0 * D), 0, seg_bytes, kBufFlags);
  float g1[G::E], g2[G::E];
  float2 lo[2][G::E];
#pragma unroll
  for (int e = 0; e < G::E; ++e) {
    const int j = m * G::E + e;
    g1[e] = gamma[(size_t)h * D + j];
    g2[e] = gamma[(size_t)h * D + j + G::HALF];
    lo[0][e] = rope_lo[t0 * G::HALF + j];
    lo[1][e] = rope_lo[(t0 + 1) * G::HALF + j];
  }
  const float2* hi0 = rope_hi + (size_t)si.hirow * G::HALF + m * G::E;
  auto issue = [&](R& r, float2 (&hi)[G::E], int c) {  // in the order step refills
    load_raw_buf<BF, D>(r, rx, c * kChunk + t0, m);
    copy_bytes<G::E * 8>(hi, hi0 + (size_t)min(c, nch - 1) * G::HALF);  // RoPE row of the chunk's start
  };
  auto step = [&](int c, R& r, float2 (&hi)[G::E]) {
    // the registers of chunk c are refilled with chunk c + 2 one token at a time, then the
    // RoPE row, so the loads leave while the other token is still being mapped
    auto map_tok = [&](auto tok_c) {
      constexpr int tok = decltype(tok_c)::value;
      R o;
      feature_map_lane<BF, D, tok>(r, o, g1, g2, lo, hi, rms_eps);
      store_raw_buf<BF, D, tok>(o, ry, c * kChunk + t0, m);
      load_raw_buf<BF, D, tok>(r, rx, (c + 2) * kChunk + t0, m);
    };
    map_tok(std::integral_constant<int, 0>{});
    map_tok(std::integral_constant<int, 1>{});
    copy_bytes<G::E * 8>(hi, hi0 + (size_t)min(c + 2, nch - 1) * G::HALF);
  };
  R set0, set1;
  float2 hs0[G::E], hs1[G::E];
  issue(set0, hs0, 0);
  issue(set1, hs1, 1);
  for (int c = 0; c < nch; c += 2) {
    step(c, set0, hs0);
    if (c + 1 < nch) step(c + 1, set1, hs1);
  }
}

// ----------------------------------------------------------------------------------------
// decode: one workgroup per (sequence, head). Every global load is issued first (the fp32
// state rows of each thread, then z, v and the new token's q, k), so the state traffic is in
// flight while wave 0 maps q and wave 1 maps k (lane j holds the RoPE pair j, j + D/2; the
// frequencies come from the host in fp64 and the angle is formed in fp64). Then every
// thread updates D/RG rows of a 4-column strip of S in place and accumulates its share of
// q'S; the partial read-outs meet in LDS.
// L2: the same thread also holds its rows of the second state A (RLA page §4.1: A = sum
// k' k'^T), updates them with k' (x) k' and accumulates its share of q'^T A q' (RLA page
// §2.1: the squared scores summed, read from the updated state); the denominator is the
// square root of the workgroup's sum plus eps. z is then optional (updated when given).

struct Theta {
  double t[64];  // base^(-2j/d), j < d/2, computed on the host in fp64
};

template <bool BF, int D, bool L2>
constexpr int decode_threads() {  // L2 (d >= 64): twice the threads, each with half the rows of S and A
  return (L2 && D >= 64) ? 512 : 256;
}

template <bool BF, int D, bool L2>
__global__ __launch_bounds__((decode_threads<BF, D, L2>())) void decode_kernel(const typename Elem<BF>::St* __restrict__ q,
                                                     const typename Elem<BF>::St* __restrict__ k,
                                                     const typename Elem<BF>::St* __restrict__ v,
                                                     const int32_t* __restrict__ positions,
                                                     const float* __restrict__ gamma_q,
                                                     const float* __restrict__ gamma_k, float rms_eps, Theta th,
                                                     float eps, float* __restrict__ S, float* __restrict__ z,
                                                     float* __restrict__ A,
                                                     typename Elem<BF>::St* __restrict__ out, int H) {
  using EL = Elem<BF>;
  constexpr int NT = decode_threads<BF, D, L2>();
  constexpr int HALF = D / 2;
  constexpr int C4 = D / 4;           // 4-column strips
  constexpr int RG = NT / C4;         // row groups
  constexpr int RPT = D / RG;         // rows per thread
  static_assert(RPT >= 1 && RG * RPT == D && HALF <= 64, "decode tiling");
  __shared__ float sq[D], sk[D], sv[D];
  __shared__ float part[RG][D];
  __shared__ float sden[NT / 64];

  const int nh = blockIdx.x;          // n * H + h
  const int n = nh / H, h = nh % H;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const size_t base = (size_t)nh * D;
  float* Sp = S + (size_t)nh * D * D;

  // every global load first: the state dominates the traffic. Plain loads with streaming
  // (nontemporal) stores measured fastest for this in-place read-modify-write.
  const int c4 = tid % C4, rg = tid / C4;
  floatx4 st[RPT];
#pragma unroll
  for (int r = 0; r < RPT; ++r)
    st[r] = *(reinterpret_cast<const floatx4*>(Sp + (size_t)(rg + r * RG) * D) + c4);
  floatx4 sa[L2 ? RPT : 1];
  float* Ap = L2 ? A + (size_t)nh * D * D : nullptr;
  if constexpr (L2) {
#pragma unroll
    for (int r = 0; r < RPT; ++r)
      sa[r] = *(reinterpret_cast<const floatx4*>(Ap + (size_t)(rg + r * RG) * D) + c4);
  }
  const bool has_z = !L2 || z != nullptr;
  float zold = 0.f, vv = 0.f;
  if (tid < D) {
    if (has_z) zold = z[base + tid];
    vv = EL::to_f(v[base + tid]);
  }
  float x1 = 0.f, x2 = 0.f, gm1 = 0.f, gm2 = 0.f;
  int p = 0;
  if (wave < 2 && lane < HALF) {
    const typename EL::St* x = (wave == 0 ? q : k) + base;
    const float* gm = (wave == 0 ? gamma_q : gamma_k) + (size_t)h * D;
    x1 = EL::to_f(x[lane]);
    x2 = EL::to_f(x[lane + HALF]);
    gm1 = gm[lane];
    gm2 = gm[lane + HALF];
    p = max(positions[n], 0);
  }

  if (wave < 2 && lane < HALF) {
    float ss = x1 * x1 + x2 * x2;
#pragma unroll
    for (int o = 1; o < HALF; o <<= 1) ss += __shfl_xor(ss, o);
    const float inv = 1.0f / sqrtf(ss * (1.0f / D) + rms_eps);
    const float y1 = x1 * inv * gm1, y2 = x2 * inv * gm2;
    double sd, cd;
    sincos((double)p * th.t[lane], &sd, &cd);
    const float c = (float)cd, s = (float)sd;
    float* dst = wave == 0 ? sq : sk;
    dst[lane] = EL::to_f(EL::from_f(fmaxf(y1 * c - y2 * s, 0.f)));
    dst[lane + HALF] = EL::to_f(EL::from_f(fmaxf(y2 * c + y1 * s, 0.f)));
  }
  if (tid < D) sv[tid] = vv;
  __syncthreads();

  const float v0 = sv[4 * c4], v1 = sv[4 * c4 + 1], v2 = sv[4 * c4 + 2], v3 = sv[4 * c4 + 3];
  float a0 = 0.f, a1 = 0.f, a2 = 0.f, a3 = 0.f;
  float quad = 0.f;  // L2: this thread's share of q'^T A q'
#pragma unroll
  for (int r = 0; r < RPT; ++r) {
    const int row = rg + r * RG;
    const float kr = sk[row], qr = sq[row];
    floatx4 x = st[r];
    x[0] += kr * v0;
    x[1] += kr * v1;
    x[2] += kr * v2;
    x[3] += kr * v3;
    __builtin_nontemporal_store(x, reinterpret_cast<floatx4*>(Sp + (size_t)row * D) + c4);
    a0 += qr * x[0];
    a1 += qr * x[1];
    a2 += qr * x[2];
    a3 += qr * x[3];
  }
  if constexpr (L2) {  // A after S: one store stream at a time (401 -> 391 us on the 256 x 32 workload)
    const float k0 = sk[4 * c4], k1 = sk[4 * c4 + 1], k2 = sk[4 * c4 + 2], k3 = sk[4 * c4 + 3];
    const float q0 = sq[4 * c4], q1 = sq[4 * c4 + 1], q2 = sq[4 * c4 + 2], q3 = sq[4 * c4 + 3];
#pragma unroll
    for (int r = 0; r < RPT; ++r) {
      const int row = rg + r * RG;
      const float kr = sk[row], qr = sq[row];
      floatx4 y = sa[r];
      y[0] += kr * k0;
      y[1] += kr * k1;
      y[2] += kr * k2;
      y[3] += kr * k3;
      __builtin_nontemporal_store(y, reinterpret_cast<floatx4*>(Ap + (size_t)row * D) + c4);
      quad += qr * (y[0] * q0 + y[1] * q1 + y[2] * q2 + y[3] * q3);
    }
  }
  part[rg][4 * c4] = a0;
  part[rg][4 * c4 + 1] = a1;
  part[rg][4 * c4 + 2] = a2;
  part[rg][4 * c4 + 3] = a3;

  // z += k'; Sum: den = q' . z_new; L2: den = sqrt(q'^T A_new q') + eps
  float dz = 0.f;
  if (tid < D && has_z) {
    const float zn = zold + sk[tid];
    z[base + tid] = zn;
    if constexpr (!L2) dz = sq[tid] * zn;
  }
  if constexpr (L2) dz = quad;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) dz += __shfl_xor(dz, o);
  if (lane == 0) sden[wave] = dz;
  __syncthreads();
  if (tid < D) {
    float num = 0.f;
#pragma unroll
    for (int r = 0; r < RG; ++r) num += part[r][tid];
    float red = 0.f;
#pragma unroll
    for (int w = 0; w < NT / 64; ++w) red += sden[w];
    const float den = L2 ? sqrtf(red) + eps : red + eps;
    out[base + tid] = EL::from_f(num / den);
  }
}

// ----------------------------------------------------------------------------------------
// launchers

// prep, chunk state and the scan of the segment records (mode: ScanMode); events 0..2
template <bool BF, int D>
hipError_t run_states(const Plan& p, const FwdArgs& a, hipStream_t s, hipEvent_t* ev, int mode) {
  using St = typename Elem<BF>::St;
  int32_t* tab = reinterpret_cast<int32_t*>(a.ws + p.off_tab);
  int32_t* docoff = reinterpret_cast<int32_t*>(a.ws + p.off_docoff);
  int32_t* nseg = reinterpret_cast<int32_t*>(a.ws + p.off_nseg);
  float2* rlo = reinterpret_cast<float2*>(a.ws + p.off_rope_lo);
  float2* rhi = reinterpret_cast<float2*>(a.ws + p.off_rope_hi);
  float* states = reinterpret_cast<float*>(a.ws + p.off_states);
  const int half = D / 2;
  auto mark = [&](int i) {
    if (ev != nullptr) (void)hipEventRecord(ev[i], s);
  };

  mark(0);
  const int rope_entries = (kChunk + p.n_hi + p.hi_off) * half;
  hipLaunchKernelGGL(prep_kernel, dim3(1 + (rope_entries + 1023) / 1024), dim3(1024), 0, s, a.cu, p.n_docs, p.L,
                     p.seg_len, p.n_seg_max, tab, docoff, nseg, rlo, rhi, half, D, p.n_hi, p.hi_off, p.initial_pos,
                     a.rope_base, reinterpret_cast<uint32_t*>(a.ws), make_stamp(p, mode));
  mark(1);
  // the L2 forward (and the export of its final A) also needs the records of A = sum k'k'^T
  const bool l2 = p.l2 && (a.out != nullptr || a.final_A != nullptr);
  float* astates = reinterpret_cast<float*>(a.ws + p.off_astates);
  // The exclusive prefixes never read the total of a document's last segment: unless the
  // final states are exported, that segment's state is not formed.
  const bool want_final = a.final_S != nullptr || a.final_z != nullptr || a.final_A != nullptr;
  const int skip_last = mode == SCAN_PREFIX && !want_final;
  if (p.n_seg_max > 0) {
    if (l2 && BF) {
      hipLaunchKernelGGL((chunk_state_l2_kernel<D>), dim3(p.n_seg_max, p.H), dim3(512), 0, s,
                         static_cast<const uint16_t*>(a.k), static_cast<const uint16_t*>(a.v), a.gk, tab, nseg, rlo,
                         rhi, states, astates, p.H, p.L, a.rms_eps, skip_last);
    } else if (l2) {
      hipLaunchKernelGGL((chunk_state_kernel<BF, D, true>), dim3(p.n_seg_max, p.H), dim3(NT), 0, s,
                         static_cast<const St*>(a.k), static_cast<const St*>(a.v), a.gk, tab, nseg, rlo, rhi,
                         states, astates, p.H, p.L, a.rms_eps, skip_last);
    } else {
      hipLaunchKernelGGL((chunk_state_kernel<BF, D>), dim3(p.n_seg_max, p.H), dim3(NT), 0, s,
                         static_cast<const St*>(a.k), static_cast<const St*>(a.v), a.gk, tab, nseg, rlo, rhi,
                         states, static_cast<float*>(nullptr), p.H, p.L, a.rms_eps, skip_last);
    }
  }
  mark(2);
  const int n_tiles = ((D * D + D) / 4 + 255) / 256;
  if (want_final || (mode != SCAN_NONE && p.n_seg_max > 0)) {
    hipLaunchKernelGGL(state_scan_kernel, dim3(p.n_docs * n_tiles, p.H), dim3(256), 0, s, states, docoff, p.H, D,
                       n_tiles, mode, a.final_S, a.final_z, a.init_S, a.init_z, p.packed ? 0 : 1, 0,
                       static_cast<const uint32_t*>(nullptr));
  }
  if (l2 && (a.final_A != nullptr || (mode != SCAN_NONE && p.n_seg_max > 0))) {  // A the same way, from A0
    hipLaunchKernelGGL(state_scan_kernel, dim3(p.n_docs * n_tiles, p.H), dim3(256), 0, s, astates, docoff, p.H, D,
                       n_tiles, mode, a.final_A, (float*)nullptr, a.init_A, (const float*)nullptr,
                       p.packed ? 0 : 1, 0, static_cast<const uint32_t*>(nullptr));
  }
  return hipGetLastError();
}

template <bool BF, int D>
hipError_t run_chunked(const Plan& p, const FwdArgs& a, hipStream_t s, hipEvent_t* ev) {
  using St = typename Elem<BF>::St;
  int32_t* tab = reinterpret_cast<int32_t*>(a.ws + p.off_tab);
  int32_t* nseg = reinterpret_cast<int32_t*>(a.ws + p.off_nseg);
  float2* rlo = reinterpret_cast<float2*>(a.ws + p.off_rope_lo);
  float2* rhi = reinterpret_cast<float2*>(a.ws + p.off_rope_hi);
  float* states = reinterpret_cast<float*>(a.ws + p.off_states);
  auto mark = [&](int i) {
    if (ev != nullptr) (void)hipEventRecord(ev[i], s);
  };
  const bool fwd = a.out != nullptr;
  const int mode = !fwd ? SCAN_NONE : (p.bidirectional ? SCAN_TOTAL : SCAN_PREFIX);
  hipError_t e = run_states<BF, D>(p, a, s, ev, mode);
  if (e != hipSuccess) return e;
  mark(3);
  if (fwd && p.n_seg_max > 0 && p.bidirectional && p.l2 && BF && D >= 64) {
    // the token-split read-out: 344 -> 267 us on the long-context workload (the column-split
    // one runs one wave per SIMD there); with the Sum denominator the column-split read-out is
    // the faster (207 against 240 us), so it keeps that mode
    hipLaunchKernelGGL((readout_l2_ql_kernel<(D >= 64 ? D : 64)>), dim3(p.n_seg_max, p.H), dim3(512), 0, s,
                       static_cast<const uint16_t*>(a.q), a.gq, tab, nseg, rlo, rhi, states,
                       reinterpret_cast<const float*>(a.ws + p.off_astates), static_cast<uint16_t*>(a.out), p.H, p.L,
                       a.rms_eps, a.eps);
  } else if (fwd && p.n_seg_max > 0 && p.bidirectional && p.l2) {
    hipLaunchKernelGGL((readout_kernel<BF, D, true>), dim3(p.n_seg_max, p.H), dim3(NT), 0, s,
                       static_cast<const St*>(a.q), a.gq, tab, nseg, rlo, rhi, states,
                       reinterpret_cast<const float*>(a.ws + p.off_astates), static_cast<St*>(a.out), p.H, p.L,
                       a.rms_eps, a.eps);
  } else if (fwd && p.n_seg_max > 0 && p.bidirectional) {
    hipLaunchKernelGGL((readout_kernel<BF, D, false>), dim3(p.n_seg_max, p.H), dim3(NT), 0, s,
                       static_cast<const St*>(a.q), a.gq, tab, nseg, rlo, rhi, states, nullptr,
                       static_cast<St*>(a.out), p.H, p.L, a.rms_eps, a.eps);
  } else if (fwd && p.n_seg_max > 0) {
    const float* astates = p.l2 ? reinterpret_cast<const float*>(a.ws + p.off_astates) : nullptr;
    if (BF && (p.chunk <= kChunk || !p.l2)) {  // C = 16, 32, 64 (and 128 with the Sum denominator): warp-specialised
      auto pick = [&](auto c_const) {
        constexpr int CC = decltype(c_const)::value;
        return p.l2 ? chunk_out_ws_kernel<D, true, CC> : chunk_out_ws_kernel<D, false, CC>;
      };
      auto kern = p.chunk == 16 ? pick(std::integral_constant<int, 16>{})
                : p.chunk == 32 ? pick(std::integral_constant<int, 32>{})
                : p.chunk == 128 ? chunk_out_ws_kernel<D, false, 128>
                                 : pick(std::integral_constant<int, 64>{});
      hipLaunchKernelGGL(kern, dim3(p.n_seg_max, p.H), dim3(512), 0, s, static_cast<const uint16_t*>(a.q),
                         static_cast<const uint16_t*>(a.k), static_cast<const uint16_t*>(a.v), a.gq, a.gk, tab, nseg,
                         rlo, rhi, states, astates, static_cast<uint16_t*>(a.out), p.H, p.L, a.rms_eps, a.eps,
                         reinterpret_cast<uint32_t*>(a.ws), p.wait_polls);
    } else {
      auto pick = [&](auto c_const) {
        constexpr int CC = decltype(c_const)::value;
        return p.l2 ? chunk_out_kernel<BF, D, true, CC> : chunk_out_kernel<BF, D, false, CC>;
      };
      auto kern = p.chunk == 16 ? pick(std::integral_constant<int, 16>{})
                : p.chunk == 32 ? pick(std::integral_constant<int, 32>{})
                : p.chunk == 128 ? pick(std::integral_constant<int, 128>{})
                                 : pick(std::integral_constant<int, 64>{});
      hipLaunchKernelGGL(kern, dim3(p.n_seg_max, p.H), dim3(NT), 0, s, static_cast<const St*>(a.q),
                         static_cast<const St*>(a.k), static_cast<const St*>(a.v), a.gq, a.gk, tab, nseg, rlo, rhi,
                         states, astates, static_cast<St*>(a.out), p.H, p.L, a.rms_eps, a.eps);
    }
  }
  mark(4);
  return hipGetLastError();
}

template <bool BF, int D>
hipError_t run_feature_map(const Plan& p, const FwdArgs& a, void* q_out, void* k_out, hipStream_t s) {
  using St = typename Elem<BF>::St;
  int32_t* tab = reinterpret_cast<int32_t*>(a.ws + p.off_tab);
  int32_t* docoff = reinterpret_cast<int32_t*>(a.ws + p.off_docoff);
  int32_t* nseg = reinterpret_cast<int32_t*>(a.ws + p.off_nseg);
  float2* rlo = reinterpret_cast<float2*>(a.ws + p.off_rope_lo);
  float2* rhi = reinterpret_cast<float2*>(a.ws + p.off_rope_hi);
  const int half = D / 2;
  const int rope_entries = (kChunk + p.n_hi + p.hi_off) * half;
  hipLaunchKernelGGL(prep_kernel, dim3(1 + (rope_entries + 1023) / 1024), dim3(1024), 0, s, a.cu, p.n_docs, p.L,
                     p.seg_len, p.n_seg_max, tab, docoff, nseg, rlo, rhi, half, D, p.n_hi, p.hi_off, p.initial_pos,
                     a.rope_base, reinterpret_cast<uint32_t*>(a.ws), make_stamp(p, SCAN_TABLES));
  if (p.n_seg_max > 0) {
    hipLaunchKernelGGL((feature_map_kernel<BF, D>), dim3(p.n_seg_max, p.H, 2), dim3(NT), 0, s,
                       static_cast<const St*>(a.q), static_cast<const St*>(a.k), a.gq, a.gk, tab, nseg, rlo, rhi,
                       static_cast<St*>(q_out), static_cast<St*>(k_out), p.H, p.L, a.rms_eps);
  }
  return hipGetLastError();
}

template <bool BF, int D>
hipError_t run_decode(int N, int H, const void* q, const void* k, const void* v, const int32_t* pos,
                      const float* gq, const float* gk, float rms_eps, float rope_base, float eps, float* S,
                      float* z, float* A, void* out, hipStream_t s) {
  using St = typename Elem<BF>::St;
  Theta th{};
  for (int j = 0; j < D / 2; ++j) th.t[j] = std::pow((double)rope_base, -2.0 * (double)j / (double)D);
  if (A != nullptr)
    hipLaunchKernelGGL((decode_kernel<BF, D, true>), dim3(N * H), dim3(decode_threads<BF, D, true>()), 0, s,
                       static_cast<const St*>(q),
                       static_cast<const St*>(k), static_cast<const St*>(v), pos, gq, gk, rms_eps, th, eps, S, z,
                       A, static_cast<St*>(out), H);
  else
    hipLaunchKernelGGL((decode_kernel<BF, D, false>), dim3(N * H), dim3(decode_threads<BF, D, false>()), 0, s,
                       static_cast<const St*>(q),
                       static_cast<const St*>(k), static_cast<const St*>(v), pos, gq, gk, rms_eps, th, eps, S, z,
                       nullptr, static_cast<St*>(out), H);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_chunked(const Plan& p, const FwdArgs& a, hipStream_t s, hipEvent_t* ev) {
  const bool bf = p.dtype == 1;
  switch (p.d) {
    case 32: return bf ? run_chunked<true, 32>(p, a, s, ev) : run_chunked<false, 32>(p, a, s, ev);
    case 64: return bf ? run_chunked<true, 64>(p, a, s, ev) : run_chunked<false, 64>(p, a, s, ev);
    case 128: return bf ? run_chunked<true, 128>(p, a, s, ev) : run_chunked<false, 128>(p, a, s, ev);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_fwd_states(const Plan& p, const FwdArgs& a, hipStream_t s, hipEvent_t* ev, int mode) {
  const bool bf = p.dtype == 1;
  switch (p.d) {
    case 32: return bf ? run_states<true, 32>(p, a, s, ev, mode) : run_states<false, 32>(p, a, s, ev, mode);
    case 64: return bf ? run_states<true, 64>(p, a, s, ev, mode) : run_states<false, 64>(p, a, s, ev, mode);
    case 128: return bf ? run_states<true, 128>(p, a, s, ev, mode) : run_states<false, 128>(p, a, s, ev, mode);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_scan_records(const Plan& p, const char* ws, float* states, int mode, const uint32_t* go_hdr,
                               hipStream_t s, float* totals) {
  const int32_t* docoff = reinterpret_cast<const int32_t*>(ws + p.off_docoff);
  const int D = p.d;
  const int n_tiles = ((D * D + D) / 4 + 255) / 256;
  const int rows = p.packed ? 1 : p.B;
  float* tz = totals != nullptr ? totals + (size_t)rows * p.H * D * D : nullptr;
  hipLaunchKernelGGL(state_scan_kernel, dim3(p.n_docs * n_tiles, p.H), dim3(256), 0, s, states, docoff, p.H, D,
                     n_tiles, mode, totals, tz, (const float*)nullptr, (const float*)nullptr, p.packed ? 0 : 1,
                     totals != nullptr ? 1 : 0, go_hdr);
  return hipGetLastError();
}

hipError_t launch_initial_grad(const Plan& p, const float* totals, const BwdArgs& b, const uint32_t* go_hdr,
                               hipStream_t s) {
  const size_t n = (size_t)p.H * p.d * (p.d + 1);
  const int rows = p.n_seg_max > 0 ? (p.packed ? 1 : p.B) : 0;  // no segments: no token reads the state
  hipLaunchKernelGGL(initial_grad_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, totals, rows, p.H, p.d,
                     b.ginit_S, b.ginit_z, go_hdr);
  return hipGetLastError();
}

hipError_t launch_saved_check(const Plan& p, const char* fwd_ws, char* ws, const int32_t* cu, int mode,
                              hipStream_t s) {
  hipLaunchKernelGGL(saved_check_kernel, dim3(1), dim3(1024), 0, s, reinterpret_cast<const uint32_t*>(fwd_ws),
                     reinterpret_cast<uint32_t*>(ws), make_stamp(p, mode), cu, p.n_docs);
  return hipGetLastError();
}

hipError_t launch_feature_map(const Plan& p, const FwdArgs& a, void* q_out, void* k_out, hipStream_t s) {
  const bool bf = p.dtype == 1;
  switch (p.d) {
    case 32: return bf ? run_feature_map<true, 32>(p, a, q_out, k_out, s) : run_feature_map<false, 32>(p, a, q_out, k_out, s);
    case 64: return bf ? run_feature_map<true, 64>(p, a, q_out, k_out, s) : run_feature_map<false, 64>(p, a, q_out, k_out, s);
    case 128: return bf ? run_feature_map<true, 128>(p, a, q_out, k_out, s) : run_feature_map<false, 128>(p, a, q_out, k_out, s);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_decode(int N, int H, int d, int dtype, const void* q, const void* k, const void* v,
                         const int32_t* pos, const float* gq, const float* gk, float rms_eps, float rope_base,
                         float eps, float* S, float* z, float* A, void* out, hipStream_t s) {
  const bool bf = dtype == 1;
#define RLA2_DEC(DD)                                                                                           \
  return bf ? run_decode<true, DD>(N, H, q, k, v, pos, gq, gk, rms_eps, rope_base, eps, S, z, A, out, s)      \
            : run_decode<false, DD>(N, H, q, k, v, pos, gq, gk, rms_eps, rope_base, eps, S, z, A, out, s)
  switch (d) {
    case 32: RLA2_DEC(32);
    case 64: RLA2_DEC(64);
    case 128: RLA2_DEC(128);
  }
#undef RLA2_DEC
  return hipErrorInvalidValue;
}

}  // namespace rla2
