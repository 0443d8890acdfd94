// Internal interface between the host entry points (rla2_api.cpp) and the
// kernel launchers (rla2_kernels.hip). Not part of the public ABI.
#pragma once

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

namespace rla2 {

constexpr int kChunk = 64;          // tokens per block: the LDS tile of the chunk kernels, the unit of
                                    // the segment table and of the coarse RoPE table (the chunk of
                                    // the output sweep, Plan::chunk, may be 16, 32, 64 or 128)
constexpr int kMaxSegChunks = 64;   // chunks per segment at most (the state kernel keeps a
                                    // segment's RoPE rows in LDS)
constexpr int kTabInts = 8;         // int32 fields per segment-table entry
constexpr size_t kAlign = 256;

// Every workspace starts with a status header of kHdrBytes (uint32 words):
//   HDR_WAIT      1 after a bounded in-kernel wait of the call ran out (outputs undefined)
//   HDR_MISMATCH  1 when a backward was handed a forward workspace whose plan stamp does not
//                 match its own plan (nothing was computed)
//   HDR_GO        1 when the backward kernels may run (set by the set-up launch)
//   HDR_STAMP..   the plan stamp the set-up launch writes: kStampWords words, the last one a
//                 checksum of cu_seqlens
// The set-up launch of every call clears the flag words first.
constexpr size_t kHdrBytes = 256;
enum HdrWord { HDR_WAIT = 0, HDR_MISMATCH = 1, HDR_GO = 2, HDR_STAMP = 16 };
constexpr int kStampWords = 16;
constexpr uint32_t kStampMagic = 0x32414C52u;  // "RLA2"
constexpr uint32_t kDefaultWaitPolls = 1u << 21;

// Plan stamp: the fields a backward needs to match between its plan and the forward that
// wrote a workspace it reads (word kStampWords - 1 is the cu_seqlens checksum, formed on the
// device).
struct Stamp {
  uint32_t w[kStampWords];
};

// Segment-table entry fields (int32 each).
// TAB_LAST: 1 for the last segment of its document.
enum TabField { TAB_ROW = 0, TAB_START = 1, TAB_LEN = 2, TAB_POS0 = 3, TAB_DOC = 4, TAB_HIROW = 5, TAB_LAST = 6 };

// Everything a launch needs about the problem and the workspace carve-up.
struct Plan {
  int B, H, L, d, dtype;
  int chunk;           // tokens per chunk of the output sweep (16, 32, 64 or 128)
  bool bidirectional;  // every token reads its whole document's state
  int initial_pos;     // first position of the first document of each row
  int n_docs;          // documents (B when not packed)
  bool packed;         // cu_seqlens given
  int seg_len;         // tokens per segment, multiple of kChunk and of chunk
  int n_seg_max;       // upper bound on segments (grid size of the sweep kernels)
  int n_hi;            // rows of the coarse RoPE table (positions / 64)
  int hi_off;          // 0, or n_hi when the first documents use the offset rows
  bool l2;             // the original RLA's L2 denominator (second state A = sum k'k'^T)
  size_t off_tab, off_docoff, off_nseg, off_rope_lo, off_rope_hi, off_states;
  size_t off_astates;  // L2 mode: records of A, after those of S
  size_t bytes;        // total workspace bytes
  size_t bytes_tables; // bytes up to the state records (what the feature map alone needs)
  // backward: a second set of segment records (reverse states); den, gd and the query's
  // weight on its own key per token-head; per-(segment, head) partial RMSNorm-weight
  // gradients of q and k
  size_t off_pstates, off_den, off_gd, off_bd, off_dgpart;
  // backward: the reverse-state totals of the documents that start from the initial state
  // (one per row; packed: one), row-major [rows][H][d][d] then [rows][H][d]
  size_t off_ginit;
  size_t bytes_bwd;    // total backward workspace bytes
  uint32_t wait_polls; // poll bound of the MMA waves' meetings (rla2_debug_set_wait_polls)
};

// What the state scan leaves in the segment records: SCAN_NONE segment totals (the state
// build), SCAN_PREFIX each segment's exclusive prefix (the causal forward), SCAN_TOTAL the
// document total in every record (the bidirectional forward), SCAN_SUFFIX the sum over the
// later segments of the document (the backward's reverse states). SCAN_TABLES: a workspace
// with the tables only (the feature map).
enum ScanMode { SCAN_NONE = 0, SCAN_PREFIX = 1, SCAN_TOTAL = 2, SCAN_SUFFIX = 3, SCAN_TABLES = 4 };

// The stamp of plan p for a workspace whose records hold scan mode `mode`.
Stamp make_stamp(const Plan& p, int mode);

struct FwdArgs {
  const int32_t* cu;   // device or null
  const void *q, *k, *v;
  const float *gq, *gk;
  void* out;           // null for the state build
  float *final_S, *final_z;
  const float *init_S, *init_z;  // optional initial state, [H, d, d] and [H, d]
  float eps, rms_eps, rope_base;
  char* ws;
  const float* init_A = nullptr;  // L2 mode: optional initial second state, [H, d, d]
  float* final_A = nullptr;       // L2 mode: optional export of the second state, [N, H, d, d]
};

// Launch the whole chunked forward (out != null) or the state build (out == null).
// `ev` (optional) gets kNumFwdKernels + 1 events recorded around the kernels.
constexpr int kNumFwdKernels = 4;
hipError_t launch_chunked(const Plan& p, const FwdArgs& a, hipStream_t s, hipEvent_t* ev = nullptr);

// Backward arguments (bf16 activations).
struct BwdArgs {
  const void* dout;            // cotangent of the forward output, [B, H, L, d]
  void *dq, *dk, *dv;          // written, [B, H, L, d]
  float *dgamma_q, *dgamma_k;  // written, [H, d] (null: not formed)
  const char* saved;           // the matching causal forward's workspace (segment table, RoPE
                               // tables, prefix records), or null: the state pass runs again
  float *ginit_S, *ginit_z;    // written, [H, d, d] and [H, d]: the gradient with respect to the
                               // initial state (null: not formed)
};

// prep + chunk state + a scan of the records in mode `mode` (what the backward needs of the
// forward's state pass: SCAN_PREFIX causal, SCAN_TOTAL bidirectional; `ev`, optional, gets
// events 0..2 before the three launches).
hipError_t launch_fwd_states(const Plan& p, const FwdArgs& a, hipStream_t s, hipEvent_t* ev, int mode);
// A scan of a record set over the segments of each document (mode SCAN_SUFFIX or SCAN_TOTAL;
// no initial state); go_hdr: null, or the header whose HDR_GO must be set for the scan to run.
// `totals` (null: none) receives the whole-document totals of the documents that start from
// the initial state, row-major, laid out as at Plan::off_ginit.
hipError_t launch_scan_records(const Plan& p, const char* ws, float* states, int mode, const uint32_t* go_hdr,
                               hipStream_t s, float* totals = nullptr);
// The gradient with respect to the initial state: the row sums (in row order) of the totals
// launch_scan_records exported, into b.ginit_S / b.ginit_z.
hipError_t launch_initial_grad(const Plan& p, const float* totals, const struct BwdArgs& b, const uint32_t* go_hdr,
                               hipStream_t s);
// The saved backward's set-up launch: compares the stamp in fwd_ws's header with
// make_stamp(p, mode) and the checksum of cu, and writes ws's header (flags, HDR_GO).
hipError_t launch_saved_check(const Plan& p, const char* fwd_ws, char* ws, const int32_t* cu, int mode,
                              hipStream_t s);
// the whole chunked backward (rla2_backward.hip); `ev` (optional) gets kNumBwdKernels + 1
// events recorded around the kernels
constexpr int kNumBwdKernels = 8;
hipError_t launch_backward(const Plan& p, const FwdArgs& a, const BwdArgs& b, hipStream_t s,
                           hipEvent_t* ev = nullptr);

// The feature map alone: prep, then q' and k' (either input may be null).
hipError_t launch_feature_map(const Plan& p, const FwdArgs& a, void* q_out, void* k_out, hipStream_t s);

// One decode step: the Sum denominator when A is null (z required), the L2 denominator with
// the second state A otherwise (z optional).
hipError_t launch_decode(int N, int H, int d, int dtype, const void* q, const void* k,
                         const void* v, const int32_t* pos, const float* gq, const float* gk,
                         float rms_eps, float rope_base, float eps, float* S, float* z, float* A,
                         void* out, hipStream_t s);

}  // namespace rla2
