// Host side of librla2.so: argument validation, workspace planning and the
// extern "C" entry points declared in include/rla2.h. Every check runs before
// any HIP call, so every error path can be exercised on a machine with no GPU.
#include "rla2.h"

#include <atomic>
#include <cmath>
#include <cstdlib>
#include <cstring>
#include <initializer_list>
#include <vector>

#include "rla2_internal.h"

namespace {

using rla2::Plan;

constexpr int32_t kAbiVersion = 7;

// Poll bound of the MMA waves' meetings inside the warp-specialised kernels (a debug hook
// lets tests lower it; see rla2_debug_set_wait_polls).
std::atomic<uint32_t> g_wait_polls{rla2::kDefaultWaitPolls};

// HIP's dispatch takes the grid size in work-items per dimension as a 32-bit count.
constexpr unsigned long long kMaxGridItems = 0xFFFFFFFFull;
static_assert(RLA2_FWD_KERNELS == rla2::kNumFwdKernels, "kernel count of the profiled forward");
static_assert(RLA2_BWD_KERNELS == rla2::kNumBwdKernels, "kernel count of the profiled backward");

bool supported_d(int d) { return d == 32 || d == 64 || d == 128; }
bool finite_pos(float x) { return std::isfinite(x) && x > 0.0f; }
size_t align_up(size_t x) { return (x + rla2::kAlign - 1) / rla2::kAlign * rla2::kAlign; }
size_t elem_bytes(int dtype) { return dtype == RLA2_F32 ? 4 : 2; }

// RLA2_VALIDATE: unset or "0" = off, "1" = on, anything else is an error
// (the convention of the ruDNN README §11 environment flags). Read once.
int validate_mode() {
  static const int mode = [] {
    const char* s = std::getenv("RLA2_VALIDATE");
    if (s == nullptr || std::strcmp(s, "0") == 0) return 0;
    if (std::strcmp(s, "1") == 0) return 1;
    return -1;
  }();
  return mode;
}

struct Range {
  const void* p;
  size_t n;
};

bool misaligned(std::initializer_list<const void*> ps) {
  for (const void* p : ps)
    if (p != nullptr && (reinterpret_cast<uintptr_t>(p) % 16) != 0) return true;
  return false;
}

bool overlap(Range a, Range b) {
  if (a.p == nullptr || b.p == nullptr || a.n == 0 || b.n == 0) return false;
  auto x = reinterpret_cast<uintptr_t>(a.p), y = reinterpret_cast<uintptr_t>(b.p);
  return x < y + b.n && y < x + a.n;
}

// Automatic segment length for the bf16 path. The output kernel runs one workgroup per
// (segment, head), 256 of them resident at once at d >= 64 (LDS and registers allow one per
// CU) and 512 at d = 32; a segment of n 64-token blocks costs it about n + 4 steps (n, plus
// the pipeline's fill and drain and the first loads' latency). The state pass runs two
// workgroups per CU over every segment but each document's last, at about half a step per
// block. The modelled time is the sum of rounds of resident workgroups times the steps of
// one, for both. Dense input has rows * ceil(L / seg) segments per head; for packed input
// each document's last segment is partial, so the count is taken as ceil(T / seg) plus half
// a segment per document. Ties go to the longer segment (fewer records through the scan).
// Measured against the segment lengths it replaces: [4, 8, 2048, 64] 42.5 -> 31.8 us (256
// instead of 128 tokens), the packed [1, 16, 16384, 128] workload 147 -> 115 us (640 instead
// of 512); the long-context workload keeps 4096.
int auto_seg_len(long long rows, long long L, long long H, long long n_docs, bool packed, int d, int seg_min) {
  const long long slots = d == 32 ? 512 : 256;
  long long best_cost = -1;
  int best = seg_min;
  for (int seg = seg_min; seg <= rla2::kMaxSegChunks * rla2::kChunk; seg += seg_min) {
    const long long per = (L + seg - 1) / seg;
    const long long nseg2 = packed ? 2 * per + n_docs : 2 * rows * per;  // twice the segments per head
    const long long out_wg = nseg2 * H / 2;
    const long long state_wg = nseg2 > 2 * n_docs ? (nseg2 - 2 * n_docs) * H / 2 : 0;
    const long long blocks = seg / rla2::kChunk;
    const long long cost2 = 2 * ((out_wg + slots - 1) / slots) * (blocks + 4) +  // twice the modelled time
                            ((state_wg + 511) / 512) * blocks;
    if (best_cost < 0 || cost2 <= best_cost) {
      best_cost = cost2;
      best = seg;
    }
  }
  return best;
}

// Shared checks of a forward / state-build descriptor. Fills the plan on success. The state
// build (no output kernel: every segment's total goes through the scan) keeps the
// 512-workgroup rule for its automatic segment length, which gives it the fewest records.
rla2_status plan_desc(const rla2_fwd_desc* d, Plan* p, bool state_build = false) {
  if (d == nullptr) return RLA2_ERR_NULL_POINTER;
  if (d->B < 0 || d->H < 0 || d->L < 0 || d->d < 0) return RLA2_ERR_BAD_SHAPE;
  if (d->cu_seqlens != nullptr && (d->B != 1 || d->n_docs < 0)) return RLA2_ERR_BAD_SHAPE;
  if (!supported_d(d->d)) return RLA2_ERR_UNSUPPORTED;
  if (d->dtype != RLA2_F32 && d->dtype != RLA2_BF16) return RLA2_ERR_UNSUPPORTED;
  if (d->chunk != 16 && d->chunk != 32 && d->chunk != 64 && d->chunk != 128) return RLA2_ERR_UNSUPPORTED;
  // a segment is a whole number of chunks and of 64-token blocks, at most 64 blocks long
  const long long seg_req = (long long)d->seg_chunks * d->chunk;
  if (d->seg_chunks < 0 || seg_req > (long long)rla2::kMaxSegChunks * rla2::kChunk || seg_req % rla2::kChunk != 0)
    return RLA2_ERR_BAD_VALUE;
  if (!finite_pos(d->eps) || !finite_pos(d->rms_eps) || !finite_pos(d->rope_base))
    return RLA2_ERR_BAD_VALUE;
  if (validate_mode() < 0) return RLA2_ERR_BAD_VALUE;
  if (d->bidirectional != 0 && d->bidirectional != 1) return RLA2_ERR_BAD_VALUE;
  if (d->initial_pos < 0 || (long long)d->initial_pos + d->L > INT32_MAX) return RLA2_ERR_BAD_VALUE;
  if ((d->initial_S == nullptr) != (d->initial_z == nullptr)) return RLA2_ERR_NULL_POINTER;
  if (d->denominator != RLA2_DEN_SUM && d->denominator != RLA2_DEN_L2) return RLA2_ERR_BAD_VALUE;
  // the second state exists in the L2 mode only, and there starts with the first state
  if (d->denominator != RLA2_DEN_L2 && (d->initial_A != nullptr || d->final_A != nullptr)) return RLA2_ERR_BAD_VALUE;
  if (d->denominator == RLA2_DEN_L2 && (d->initial_S == nullptr) != (d->initial_A == nullptr))
    return RLA2_ERR_NULL_POINTER;
  // every token index and every segment index must stay within int32 on device
  const long long tokens = (long long)d->B * d->L;
  if (tokens > INT32_MAX || (long long)d->B * d->H > INT32_MAX) return RLA2_ERR_BAD_SHAPE;
  if (d->H > 65535) return RLA2_ERR_BAD_SHAPE;  // heads are the grid's y dimension

  p->B = d->B;
  p->chunk = d->chunk;
  p->H = d->H;
  p->L = d->L;
  p->d = d->d;
  p->dtype = d->dtype;
  p->bidirectional = d->bidirectional == 1;
  p->l2 = d->denominator == RLA2_DEN_L2;
  p->initial_pos = d->initial_pos;
  p->packed = d->cu_seqlens != nullptr;
  p->n_docs = p->packed ? d->n_docs : d->B;
  const int rows = p->packed ? 1 : p->B;
  const long long L = p->L;
  // Segment length: the sweep kernels run one workgroup per (segment, head). The bf16 path
  // takes the modelled best (auto_seg_len); otherwise the longest segment that still gives 512
  // workgroups, two per CU of the 256-CU part (fewer segments mean less fp32 state traffic
  // through the inter-segment scan and fewer pipeline fills; measured on the long-context
  // forward: 64-chunk segments 651 us, 32-chunk 693 us, 16-chunk 754 us).
  const int seg_min = d->chunk > rla2::kChunk ? d->chunk : rla2::kChunk;
  int seg = 0;
  if (d->seg_chunks > 0) {
    seg = (int)seg_req;
  } else if (d->dtype == RLA2_BF16 && !state_build) {
    seg = auto_seg_len(rows, L, d->H, p->n_docs, p->packed, d->d, seg_min);
  } else {
    seg = seg_min;
    for (int cand = rla2::kMaxSegChunks * rla2::kChunk; cand >= seg_min; cand /= 2) {
      long long wg = (long long)rows * ((L + cand - 1) / cand) * (p->H > 0 ? p->H : 1);
      if (wg >= 512) { seg = cand; break; }
    }
  }
  p->seg_len = seg;
  long long nseg = p->packed ? (L + seg - 1) / seg + p->n_docs : (long long)rows * ((L + seg - 1) / seg);
  if (p->n_docs == 0 || p->H == 0) nseg = 0;
  if (nseg > INT32_MAX / 8) return RLA2_ERR_BAD_SHAPE;
  p->n_seg_max = (int)nseg;
  p->n_hi = (int)((L + rla2::kChunk - 1) / rla2::kChunk);
  if (p->n_hi < 1) p->n_hi = 1;
  // with a position offset the first documents read a second set of chunk rows,
  // (initial_pos + 64 a) * theta, right after the plain set
  p->hi_off = p->initial_pos != 0 ? p->n_hi : 0;
  // every launch's grid must fit the dispatch: the sweeps run up to 512 work-items per
  // (segment, head), the state scan 256 per (document, 1024-float tile of a record), the
  // set-up launch 1024 per 1024 RoPE entries (indexed in int32)
  {
    const unsigned long long tiles = ((unsigned long long)p->d * p->d + p->d + 1023) / 1024;
    const unsigned long long rope = (unsigned long long)(rla2::kChunk + 2LL * p->n_hi) * (p->d / 2);
    if ((unsigned long long)p->n_seg_max * 512 > kMaxGridItems ||
        (unsigned long long)p->n_docs * tiles * 256 > kMaxGridItems || (rope / 1024 + 2) * 1024 > (unsigned long long)INT32_MAX)
      return RLA2_ERR_BAD_SHAPE;
  }
  p->wait_polls = g_wait_polls.load(std::memory_order_relaxed);

  const size_t half = (size_t)p->d / 2;
  const size_t rec = (size_t)p->d * p->d + p->d;
  size_t off = rla2::kHdrBytes;  // the status header comes first
  p->off_tab = off;
  off = align_up(off + (size_t)p->n_seg_max * rla2::kTabInts * 4);
  p->off_docoff = off;
  off = align_up(off + ((size_t)p->n_docs + 1) * 4);
  p->off_nseg = off;
  off = align_up(off + 4);
  p->off_rope_lo = off;
  off = align_up(off + (size_t)rla2::kChunk * half * 8);
  p->off_rope_hi = off;
  off = align_up(off + (size_t)(p->n_hi + p->hi_off) * half * 8);
  p->off_states = off;
  p->bytes_tables = (p->n_docs == 0 || p->H == 0) ? 0 : off;
  off = align_up(off + (size_t)p->n_seg_max * p->H * rec * 4);
  p->off_astates = off;  // the L2 mode's second record set (A = sum k'k'^T), same layout
  if (p->l2) off = align_up(off + (size_t)p->n_seg_max * p->H * rec * 4);
  p->bytes = (p->n_docs == 0 || p->H == 0) ? 0 : off;  // no documents or heads: nothing to run
  const size_t tokh = (size_t)rows * p->H * (size_t)p->L;
  p->off_pstates = off;
  off = align_up(off + (size_t)p->n_seg_max * p->H * rec * 4);
  p->off_den = off;
  off = align_up(off + tokh * 4);
  p->off_gd = off;
  off = align_up(off + tokh * 4);
  p->off_bd = off;
  off = align_up(off + tokh * 4);
  p->off_dgpart = off;
  off = align_up(off + (size_t)p->n_seg_max * p->H * p->d * 2 * 4);
  p->off_ginit = off;  // only when the backward is asked for the initial state's gradient
  if (d->grad_initial_S != nullptr || d->grad_initial_z != nullptr)
    off = align_up(off + (size_t)(p->packed ? 1 : p->B) * p->H * rec * 4);
  p->bytes_bwd = (p->n_docs == 0 || p->H == 0) ? 0 : off;
  return RLA2_OK;
}

// Synchronous check of the cu_seqlens contract (only with RLA2_VALIDATE=1).
rla2_status check_seqlens(const Plan& p, const int32_t* cu, hipStream_t stream) {
  std::vector<int32_t> h((size_t)p.n_docs + 1);
  if (hipStreamSynchronize(stream) != hipSuccess) return RLA2_ERR_HIP;
  if (hipMemcpy(h.data(), cu, h.size() * 4, hipMemcpyDeviceToHost) != hipSuccess)
    return RLA2_ERR_HIP;
  if (h[0] != 0 || h.back() != p.L) return RLA2_ERR_BAD_SEQLENS;
  for (size_t j = 1; j < h.size(); ++j)
    if (h[j] < h[j - 1]) return RLA2_ERR_BAD_SEQLENS;
  return RLA2_OK;
}

rla2_status finish(hipError_t e) {
  if (e != hipSuccess) return RLA2_ERR_HIP;
  return hipGetLastError() == hipSuccess ? RLA2_OK : RLA2_ERR_HIP;
}

}  // namespace

namespace rla2 {

Stamp make_stamp(const Plan& p, int mode) {
  Stamp st{};
  const uint32_t f[] = {kStampMagic, (uint32_t)kAbiVersion, (uint32_t)p.B, (uint32_t)p.H, (uint32_t)p.L,
                        (uint32_t)p.d, (uint32_t)p.dtype, (uint32_t)p.n_docs, (uint32_t)p.packed,
                        (uint32_t)p.seg_len, (uint32_t)p.n_seg_max, (uint32_t)p.n_hi, (uint32_t)p.hi_off,
                        (uint32_t)p.initial_pos, (uint32_t)mode | ((uint32_t)p.l2 << 8)};
  static_assert(sizeof(f) / sizeof(f[0]) == kStampWords - 1, "the last stamp word is the checksum");
  for (int i = 0; i < kStampWords - 1; ++i) st.w[i] = f[i];
  return st;
}

}  // namespace rla2

namespace {

// The backward's supported modes: bf16 or fp32 activations, causal or bidirectional, the Sum
// denominator.
bool bwd_supported(const Plan& p) { return !p.l2; }

// The backward entry points; `saved` (with `saved_bytes`) is the matching forward's workspace,
// or null.
rla2_status bwd_impl(const rla2_fwd_desc* desc, const void* q, const void* k, const void* v, const float* gamma_q,
                     const float* gamma_k, const void* dout, void* dq, void* dk, void* dv, float* dgamma_q,
                     float* dgamma_k, void* workspace, size_t workspace_bytes, const void* saved,
                     size_t saved_bytes, hipStream_t stream, hipEvent_t* events) {
  Plan p;
  rla2_status st = plan_desc(desc, &p);
  if (st != RLA2_OK) return st;
  if (!bwd_supported(p)) return RLA2_ERR_UNSUPPORTED;
  const size_t act = (size_t)p.B * p.H * p.L * p.d * elem_bytes(p.dtype);
  const size_t gam = (size_t)p.H * p.d * 4;
  if (act > 0 && (q == nullptr || k == nullptr || v == nullptr || dout == nullptr ||
                  dq == nullptr || dk == nullptr || dv == nullptr || gamma_q == nullptr || gamma_k == nullptr))
    return RLA2_ERR_NULL_POINTER;
  if (p.packed && desc->cu_seqlens == nullptr) return RLA2_ERR_NULL_POINTER;
  if (p.bytes_bwd > 0 && (workspace == nullptr || workspace_bytes < p.bytes_bwd)) return RLA2_ERR_WORKSPACE;
  if (workspace != nullptr && (reinterpret_cast<uintptr_t>(workspace) % rla2::kAlign) != 0)
    return RLA2_ERR_WORKSPACE;
  // the forward's workspace holds its records up to p.bytes (the Sum mode has no second set)
  if (saved != nullptr && (saved_bytes < p.bytes || (reinterpret_cast<uintptr_t>(saved) % rla2::kAlign) != 0))
    return RLA2_ERR_WORKSPACE;
  if (misaligned({q, k, v, dout, dq, dk, dv, gamma_q, gamma_k, dgamma_q, dgamma_k, desc->initial_S,
                  desc->initial_z, desc->grad_initial_S, desc->grad_initial_z}))
    return RLA2_ERR_MISALIGNED;
  const Range outs[] = {{dq, act}, {dk, act}, {dv, act}, {dgamma_q, gam}, {dgamma_k, gam},
                        {desc->grad_initial_S, (size_t)p.H * p.d * p.d * 4}, {desc->grad_initial_z, gam}};
  constexpr size_t n_outs = sizeof(outs) / sizeof(outs[0]);
  const Range ws{workspace, p.bytes_bwd};
  const Range ins[] = {{q, act}, {k, act}, {v, act}, {dout, act}, {gamma_q, gam}, {gamma_k, gam},
                       {desc->cu_seqlens, ((size_t)p.n_docs + 1) * 4},
                       {desc->initial_S, (size_t)p.H * p.d * p.d * 4}, {desc->initial_z, (size_t)p.H * p.d * 4},
                       {saved, saved != nullptr ? p.bytes : 0}};
  for (const Range& r : ins) {
    if (overlap(ws, r)) return RLA2_ERR_ALIAS;
    for (const Range& o : outs)
      if (overlap(o, r)) return RLA2_ERR_ALIAS;
  }
  for (size_t i = 0; i < n_outs; ++i) {
    if (overlap(outs[i], ws)) return RLA2_ERR_ALIAS;
    for (size_t j = i + 1; j < n_outs; ++j)
      if (overlap(outs[i], outs[j])) return RLA2_ERR_ALIAS;
  }
  if (p.packed && validate_mode() == 1) {
    st = check_seqlens(p, desc->cu_seqlens, stream);
    if (st != RLA2_OK) return st;
  }
  if (p.n_docs == 0 || p.H == 0) return RLA2_OK;
  rla2::FwdArgs a{desc->cu_seqlens, q, k, v, gamma_q, gamma_k, nullptr, nullptr, nullptr,
                  desc->initial_S, desc->initial_z, desc->eps, desc->rms_eps, desc->rope_base,
                  static_cast<char*>(workspace)};
  rla2::BwdArgs b{dout, dq, dk, dv, dgamma_q, dgamma_k, static_cast<const char*>(saved), desc->grad_initial_S,
                  desc->grad_initial_z};
  return finish(rla2::launch_backward(p, a, b, stream, events));
}

}  // namespace

extern "C" {

const char* rla2_status_string(rla2_status s) {
  switch (s) {
    case RLA2_OK: return "RLA2_OK";
    case RLA2_ERR_NULL_POINTER: return "RLA2_ERR_NULL_POINTER: a required pointer is NULL";
    case RLA2_ERR_BAD_SHAPE: return "RLA2_ERR_BAD_SHAPE: negative size or inconsistent shape";
    case RLA2_ERR_UNSUPPORTED: return "RLA2_ERR_UNSUPPORTED: head dim, dtype or chunk not supported";
    case RLA2_ERR_BAD_VALUE: return "RLA2_ERR_BAD_VALUE: eps, rms_eps, rope_base or option out of range";
    case RLA2_ERR_WORKSPACE: return "RLA2_ERR_WORKSPACE: workspace missing or too small";
    case RLA2_ERR_ALIAS: return "RLA2_ERR_ALIAS: an output overlaps another buffer";
    case RLA2_ERR_HIP: return "RLA2_ERR_HIP: a HIP runtime call failed";
    case RLA2_ERR_BAD_SEQLENS: return "RLA2_ERR_BAD_SEQLENS: cu_seqlens breaks its contract";
    case RLA2_ERR_MISALIGNED: return "RLA2_ERR_MISALIGNED: a tensor pointer is not 16-byte aligned";
  }
  return "RLA2_ERR_UNKNOWN";
}

int32_t rla2_abi_version(void) { return kAbiVersion; }

uint32_t rla2_debug_set_wait_polls(uint32_t polls) {
  return g_wait_polls.exchange(polls, std::memory_order_relaxed);
}

rla2_status rla2_workspace_flags(const void* workspace, size_t workspace_bytes, hipStream_t stream,
                                 uint32_t* flags) {
  if (workspace == nullptr || flags == nullptr) return RLA2_ERR_NULL_POINTER;
  if (workspace_bytes < rla2::kHdrBytes || (reinterpret_cast<uintptr_t>(workspace) % rla2::kAlign) != 0)
    return RLA2_ERR_WORKSPACE;
  uint32_t w[2] = {0u, 0u};
  if (hipStreamSynchronize(stream) != hipSuccess) return RLA2_ERR_HIP;
  if (hipMemcpy(w, workspace, sizeof(w), hipMemcpyDeviceToHost) != hipSuccess) return RLA2_ERR_HIP;
  *flags = (w[rla2::HDR_WAIT] != 0u ? RLA2_FLAG_WAIT_EXHAUSTED : 0u) |
           (w[rla2::HDR_MISMATCH] != 0u ? RLA2_FLAG_PLAN_MISMATCH : 0u);
  return RLA2_OK;
}

rla2_status rla2_fwd_workspace_size(const rla2_fwd_desc* desc, size_t* bytes) {
  if (bytes == nullptr) return RLA2_ERR_NULL_POINTER;
  Plan p;
  rla2_status st = plan_desc(desc, &p);
  if (st != RLA2_OK) return st;
  *bytes = p.bytes;
  return RLA2_OK;
}

rla2_status rla2_state_from_prefix_workspace_size(const rla2_fwd_desc* desc, size_t* bytes) {
  if (bytes == nullptr) return RLA2_ERR_NULL_POINTER;
  Plan p;
  rla2_status st = plan_desc(desc, &p, true);
  if (st != RLA2_OK) return st;
  *bytes = p.bytes;
  return RLA2_OK;
}

rla2_status rla2_fwd_chunked(const rla2_fwd_desc* desc, const void* q, const void* k,
                             const void* v, const float* gamma_q, const float* gamma_k,
                             void* out, float* final_S, float* final_z, void* workspace,
                             size_t workspace_bytes, hipStream_t stream) {
  return rla2_fwd_chunked_profiled(desc, q, k, v, gamma_q, gamma_k, out, final_S, final_z, workspace,
                                   workspace_bytes, stream, nullptr);
}

rla2_status rla2_fwd_chunked_profiled(const rla2_fwd_desc* desc, const void* q, const void* k,
                                      const void* v, const float* gamma_q, const float* gamma_k,
                                      void* out, float* final_S, float* final_z, void* workspace,
                                      size_t workspace_bytes, hipStream_t stream, hipEvent_t* events) {
  Plan p;
  rla2_status st = plan_desc(desc, &p);
  if (st != RLA2_OK) return st;
  const size_t act = (size_t)p.B * p.H * p.L * p.d * elem_bytes(p.dtype);
  const size_t gam = (size_t)p.H * p.d * 4;
  const size_t fsb = (size_t)p.n_docs * p.H * p.d * p.d * 4;
  const size_t fzb = (size_t)p.n_docs * p.H * p.d * 4;
  if (act > 0 && (q == nullptr || k == nullptr || v == nullptr || out == nullptr))
    return RLA2_ERR_NULL_POINTER;
  if (gam > 0 && act > 0 && (gamma_q == nullptr || gamma_k == nullptr)) return RLA2_ERR_NULL_POINTER;
  if (p.packed && desc->cu_seqlens == nullptr) return RLA2_ERR_NULL_POINTER;
  if (p.bytes > 0 && (workspace == nullptr || workspace_bytes < p.bytes)) return RLA2_ERR_WORKSPACE;
  if (workspace != nullptr && (reinterpret_cast<uintptr_t>(workspace) % rla2::kAlign) != 0)
    return RLA2_ERR_WORKSPACE;
  if (misaligned({q, k, v, out, gamma_q, gamma_k, final_S, final_z, desc->initial_S, desc->initial_z,
                  desc->initial_A, desc->final_A}))
    return RLA2_ERR_MISALIGNED;
  const Range o{out, act}, fs{final_S, fsb}, fz{final_z, fzb}, fa{desc->final_A, fsb}, ws{workspace, p.bytes};
  const Range ins[] = {{q, act}, {k, act}, {v, act}, {gamma_q, gam}, {gamma_k, gam},
                       {desc->cu_seqlens, ((size_t)p.n_docs + 1) * 4},
                       {desc->initial_S, (size_t)p.H * p.d * p.d * 4}, {desc->initial_z, (size_t)p.H * p.d * 4},
                       {desc->initial_A, (size_t)p.H * p.d * p.d * 4}};
  const Range outs[] = {o, fs, fz, fa, ws};
  for (const Range& r : ins)
    for (const Range& x : outs)
      if (overlap(x, r)) return RLA2_ERR_ALIAS;
  for (size_t i = 0; i < 5; ++i)
    for (size_t j = i + 1; j < 5; ++j)
      if (overlap(outs[i], outs[j])) return RLA2_ERR_ALIAS;
  if (p.packed && validate_mode() == 1) {
    st = check_seqlens(p, desc->cu_seqlens, stream);
    if (st != RLA2_OK) return st;
  }
  if (p.n_docs == 0 || p.H == 0) return RLA2_OK;
  rla2::FwdArgs a{desc->cu_seqlens, q, k, v, gamma_q, gamma_k, out, final_S, final_z,
                  desc->initial_S, desc->initial_z, desc->eps, desc->rms_eps, desc->rope_base,
                  static_cast<char*>(workspace), desc->initial_A, desc->final_A};
  return finish(rla2::launch_chunked(p, a, stream, events));
}

rla2_status rla2_state_from_prefix(const rla2_fwd_desc* desc, const void* k, const void* v,
                                   const float* gamma_k, float* S, float* z, void* workspace,
                                   size_t workspace_bytes, hipStream_t stream) {
  Plan p;
  rla2_status st = plan_desc(desc, &p, true);
  if (st != RLA2_OK) return st;
  const size_t act = (size_t)p.B * p.H * p.L * p.d * elem_bytes(p.dtype);
  const size_t gam = (size_t)p.H * p.d * 4;
  const size_t sb = (size_t)p.n_docs * p.H * p.d * p.d * 4;
  const size_t zb = (size_t)p.n_docs * p.H * p.d * 4;
  if (act > 0 && (k == nullptr || v == nullptr || gamma_k == nullptr)) return RLA2_ERR_NULL_POINTER;
  if (sb > 0 && (S == nullptr || z == nullptr)) return RLA2_ERR_NULL_POINTER;
  if (p.packed && desc->cu_seqlens == nullptr) return RLA2_ERR_NULL_POINTER;
  if (p.bytes > 0 && (workspace == nullptr || workspace_bytes < p.bytes)) return RLA2_ERR_WORKSPACE;
  if (workspace != nullptr && (reinterpret_cast<uintptr_t>(workspace) % rla2::kAlign) != 0)
    return RLA2_ERR_WORKSPACE;
  if (misaligned({k, v, gamma_k, S, z, desc->initial_S, desc->initial_z, desc->initial_A, desc->final_A}))
    return RLA2_ERR_MISALIGNED;
  const Range rs{S, sb}, rz{z, zb}, ra{desc->final_A, sb}, ws{workspace, p.bytes};
  const Range ins[] = {{k, act}, {v, act}, {gamma_k, gam}, {desc->cu_seqlens, ((size_t)p.n_docs + 1) * 4},
                       {desc->initial_S, (size_t)p.H * p.d * p.d * 4}, {desc->initial_z, (size_t)p.H * p.d * 4},
                       {desc->initial_A, (size_t)p.H * p.d * p.d * 4}};
  const Range outs[] = {rs, rz, ra, ws};
  for (const Range& r : ins)
    for (const Range& x : outs)
      if (overlap(x, r)) return RLA2_ERR_ALIAS;
  for (size_t i = 0; i < 4; ++i)
    for (size_t j = i + 1; j < 4; ++j)
      if (overlap(outs[i], outs[j])) return RLA2_ERR_ALIAS;
  if (p.packed && validate_mode() == 1) {
    st = check_seqlens(p, desc->cu_seqlens, stream);
    if (st != RLA2_OK) return st;
  }
  if (p.n_docs == 0 || p.H == 0) return RLA2_OK;
  rla2::FwdArgs a{desc->cu_seqlens, nullptr, k, v, nullptr, gamma_k, nullptr, S, z,
                  desc->initial_S, desc->initial_z, desc->eps, desc->rms_eps, desc->rope_base,
                  static_cast<char*>(workspace), desc->initial_A, desc->final_A};
  return finish(rla2::launch_chunked(p, a, stream));
}

rla2_status rla2_bwd_workspace_size(const rla2_fwd_desc* desc, size_t* bytes) {
  if (bytes == nullptr) return RLA2_ERR_NULL_POINTER;
  Plan p;
  rla2_status st = plan_desc(desc, &p);
  if (st != RLA2_OK) return st;
  if (!bwd_supported(p)) return RLA2_ERR_UNSUPPORTED;
  *bytes = p.bytes_bwd;
  return RLA2_OK;
}

rla2_status rla2_bwd_chunked(const rla2_fwd_desc* desc, const void* q, const void* k, const void* v,
                             const float* gamma_q, const float* gamma_k, const void* dout,
                             void* dq, void* dk, void* dv, float* dgamma_q, float* dgamma_k, void* workspace,
                             size_t workspace_bytes, hipStream_t stream) {
  return bwd_impl(desc, q, k, v, gamma_q, gamma_k, dout, dq, dk, dv, dgamma_q, dgamma_k, workspace,
                  workspace_bytes, nullptr, 0, stream, nullptr);
}

rla2_status rla2_bwd_chunked_profiled(const rla2_fwd_desc* desc, const void* q, const void* k, const void* v,
                                      const float* gamma_q, const float* gamma_k, const void* dout, void* dq,
                                      void* dk, void* dv, float* dgamma_q, float* dgamma_k, void* workspace,
                                      size_t workspace_bytes, hipStream_t stream, hipEvent_t* events) {
  return bwd_impl(desc, q, k, v, gamma_q, gamma_k, dout, dq, dk, dv, dgamma_q, dgamma_k, workspace,
                  workspace_bytes, nullptr, 0, stream, events);
}

rla2_status rla2_bwd_chunked_saved(const rla2_fwd_desc* desc, const void* q, const void* k, const void* v,
                                   const float* gamma_q, const float* gamma_k, const void* dout, void* dq,
                                   void* dk, void* dv, float* dgamma_q, float* dgamma_k, void* workspace,
                                   size_t workspace_bytes, const void* fwd_workspace,
                                   size_t fwd_workspace_bytes, hipStream_t stream, hipEvent_t* events) {
  Plan p;
  rla2_status st = plan_desc(desc, &p);
  if (st != RLA2_OK) return st;
  if (!bwd_supported(p)) return RLA2_ERR_UNSUPPORTED;
  if (p.bytes > 0 && fwd_workspace == nullptr) return RLA2_ERR_NULL_POINTER;
  return bwd_impl(desc, q, k, v, gamma_q, gamma_k, dout, dq, dk, dv, dgamma_q, dgamma_k, workspace,
                  workspace_bytes, p.bytes > 0 ? fwd_workspace : nullptr, fwd_workspace_bytes, stream, events);
}

rla2_status rla2_feature_map_workspace_size(const rla2_fwd_desc* desc, size_t* bytes) {
  if (bytes == nullptr) return RLA2_ERR_NULL_POINTER;
  Plan p;
  rla2_status st = plan_desc(desc, &p);
  if (st != RLA2_OK) return st;
  *bytes = p.bytes_tables;
  return RLA2_OK;
}

rla2_status rla2_feature_map(const rla2_fwd_desc* desc, const void* q, const void* k, const float* gamma_q,
                             const float* gamma_k, void* q_out, void* k_out, void* workspace,
                             size_t workspace_bytes, hipStream_t stream) {
  Plan p;
  rla2_status st = plan_desc(desc, &p);
  if (st != RLA2_OK) return st;
  const size_t act = (size_t)p.B * p.H * p.L * p.d * elem_bytes(p.dtype);
  const size_t gam = (size_t)p.H * p.d * 4;
  if (q == nullptr && k == nullptr) return RLA2_ERR_NULL_POINTER;
  if (act > 0 && q != nullptr && (q_out == nullptr || gamma_q == nullptr)) return RLA2_ERR_NULL_POINTER;
  if (act > 0 && k != nullptr && (k_out == nullptr || gamma_k == nullptr)) return RLA2_ERR_NULL_POINTER;
  if (q == nullptr) q_out = nullptr;
  if (k == nullptr) k_out = nullptr;
  if (p.packed && desc->cu_seqlens == nullptr) return RLA2_ERR_NULL_POINTER;
  if (p.bytes_tables > 0 && (workspace == nullptr || workspace_bytes < p.bytes_tables)) return RLA2_ERR_WORKSPACE;
  if (workspace != nullptr && (reinterpret_cast<uintptr_t>(workspace) % rla2::kAlign) != 0)
    return RLA2_ERR_WORKSPACE;
  if (misaligned({q, k, gamma_q, gamma_k, q_out, k_out})) return RLA2_ERR_MISALIGNED;
  const Range oq{q_out, act}, ok{k_out, act}, ws{workspace, p.bytes_tables};
  const Range ins[] = {{q, act}, {k, act}, {gamma_q, gam}, {gamma_k, gam},
                       {desc->cu_seqlens, ((size_t)p.n_docs + 1) * 4}};
  for (const Range& r : ins)
    if (overlap(oq, r) || overlap(ok, r) || overlap(ws, r)) return RLA2_ERR_ALIAS;
  if (overlap(oq, ok) || overlap(oq, ws) || overlap(ok, ws)) return RLA2_ERR_ALIAS;
  if (p.packed && validate_mode() == 1) {
    st = check_seqlens(p, desc->cu_seqlens, stream);
    if (st != RLA2_OK) return st;
  }
  if (p.n_docs == 0 || p.H == 0 || act == 0) return RLA2_OK;
  rla2::FwdArgs a{desc->cu_seqlens, q, k, nullptr, gamma_q, gamma_k, nullptr, nullptr, nullptr, nullptr, nullptr,
                  desc->eps, desc->rms_eps, desc->rope_base, static_cast<char*>(workspace)};
  return finish(rla2::launch_feature_map(p, a, q_out, k_out, stream));
}

rla2_status rla2_decode_step(int32_t N, int32_t H, int32_t d, int32_t dtype, const void* q,
                             const void* k, const void* v, const int32_t* positions,
                             const float* gamma_q, const float* gamma_k, float rms_eps,
                             float rope_base, float eps, float* S, float* z, void* out,
                             hipStream_t stream) {
  if (N < 0 || H < 0 || d < 0) return RLA2_ERR_BAD_SHAPE;
  if (!supported_d(d)) return RLA2_ERR_UNSUPPORTED;
  if (dtype != RLA2_F32 && dtype != RLA2_BF16) return RLA2_ERR_UNSUPPORTED;
  if (!finite_pos(eps) || !finite_pos(rms_eps) || !finite_pos(rope_base)) return RLA2_ERR_BAD_VALUE;
  // one 256-thread workgroup per (sequence, head)
  if ((unsigned long long)N * H * 256 > kMaxGridItems) return RLA2_ERR_BAD_SHAPE;
  const size_t act = (size_t)N * H * d * elem_bytes(dtype);
  if (act == 0) return RLA2_OK;
  if (q == nullptr || k == nullptr || v == nullptr || positions == nullptr || gamma_q == nullptr ||
      gamma_k == nullptr || S == nullptr || z == nullptr || out == nullptr)
    return RLA2_ERR_NULL_POINTER;
  if (misaligned({q, k, v, out, gamma_q, gamma_k, S, z})) return RLA2_ERR_MISALIGNED;
  const size_t sb = (size_t)N * H * d * d * 4, zb = (size_t)N * H * d * 4, gam = (size_t)H * d * 4;
  const Range o{out, act}, rs{S, sb}, rz{z, zb};
  const Range ins[] = {{q, act}, {k, act}, {v, act}, {positions, (size_t)N * 4}, {gamma_q, gam},
                       {gamma_k, gam}};
  for (const Range& r : ins)
    if (overlap(o, r) || overlap(rs, r) || overlap(rz, r)) return RLA2_ERR_ALIAS;
  if (overlap(o, rs) || overlap(o, rz) || overlap(rs, rz)) return RLA2_ERR_ALIAS;
  return finish(rla2::launch_decode(N, H, d, dtype, q, k, v, positions, gamma_q, gamma_k, rms_eps,
                                    rope_base, eps, S, z, nullptr, out, stream));
}

rla2_status rla2_decode_step_l2(int32_t N, int32_t H, int32_t d, int32_t dtype, const void* q,
                                const void* k, const void* v, const int32_t* positions,
                                const float* gamma_q, const float* gamma_k, float rms_eps,
                                float rope_base, float eps, float* S, float* A, float* z, void* out,
                                hipStream_t stream) {
  if (N < 0 || H < 0 || d < 0) return RLA2_ERR_BAD_SHAPE;
  if (!supported_d(d)) return RLA2_ERR_UNSUPPORTED;
  if (dtype != RLA2_F32 && dtype != RLA2_BF16) return RLA2_ERR_UNSUPPORTED;
  if (!finite_pos(eps) || !finite_pos(rms_eps) || !finite_pos(rope_base)) return RLA2_ERR_BAD_VALUE;
  if ((unsigned long long)N * H * 256 > kMaxGridItems) return RLA2_ERR_BAD_SHAPE;
  const size_t act = (size_t)N * H * d * elem_bytes(dtype);
  if (act == 0) return RLA2_OK;
  if (q == nullptr || k == nullptr || v == nullptr || positions == nullptr || gamma_q == nullptr ||
      gamma_k == nullptr || S == nullptr || A == nullptr || out == nullptr)
    return RLA2_ERR_NULL_POINTER;
  if (misaligned({q, k, v, out, gamma_q, gamma_k, S, A, z})) return RLA2_ERR_MISALIGNED;
  const size_t sb = (size_t)N * H * d * d * 4, zb = (size_t)N * H * d * 4, gam = (size_t)H * d * 4;
  const Range o{out, act}, rs{S, sb}, ra{A, sb}, rz{z, z != nullptr ? zb : 0};
  const Range ins[] = {{q, act}, {k, act}, {v, act}, {positions, (size_t)N * 4}, {gamma_q, gam},
                       {gamma_k, gam}};
  for (const Range& r : ins)
    if (overlap(o, r) || overlap(rs, r) || overlap(ra, r) || overlap(rz, r)) return RLA2_ERR_ALIAS;
  if (overlap(o, rs) || overlap(o, ra) || overlap(o, rz) || overlap(rs, ra) || overlap(rs, rz) || overlap(ra, rz))
    return RLA2_ERR_ALIAS;
  return finish(rla2::launch_decode(N, H, d, dtype, q, k, v, positions, gamma_q, gamma_k, rms_eps,
                                    rope_base, eps, S, z, A, out, stream));
}

}  // extern "C"
