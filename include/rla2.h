/*
 * rla2.h -- C ABI of librla2.so: RLA-2 causal ReLU linear attention on gfx950.
 *
 * The method (neuralnet.cpp development page "线性注意力家族：RLA / RAPT / RLA-2 与
 * GPU 落地", called the RLA page below):
 *   q' = ReLU(RoPE(RMSNorm(q))), k' = ReLU(RoPE(RMSNorm(k)))   (RLA page §3; §1: no
 *        1/sqrt(d) scaling, per-head RMSNorm, RoPE before the ReLU; v is untouched)
 *   S_t = S_{t-1} + k'_t (x) v_t   (d x d),   z_t = z_{t-1} + k'_t   (RLA page §3)
 *   out_t = q'_t S_t / (q'_t . z_t + eps)                             (RLA page §3)
 * with S and z cleared at every document start (RLA page §2.2 and §4.1).
 * RMSNorm: x * gamma / sqrt(mean(x^2) + rms_eps), fp32 statistics, F32 weight
 * (ruDNN README §7; candle "常用层" page, RmsNorm). RoPE: rotate-half pairing of
 * dimension j with j + d/2, angle p * base^(-2j/d) (candle "常用层" page,
 * rotary_emb). Positions restart at 0 at each document start.
 *
 * Conventions shared by every entry point:
 *  - Tensor pointers are DEVICE pointers, dense row-major (C order), no strides,
 *    16-byte aligned (RLA2_ERR_MISALIGNED otherwise; cu_seqlens and positions
 *    need only 4-byte alignment). Descriptors, sizes and scalars are host values.
 *  - Activations q, k, v, out use the element type given by rla2_dtype; RMSNorm
 *    weights and states are always fp32. Every reduction accumulates in fp32.
 *  - Every call validates all host-visible arguments first. On any error nothing
 *    is enqueued and no output is touched. On RLA2_OK the work is enqueued on
 *    `stream` (asynchronous; no host synchronisation) except where noted.
 *  - The library never allocates device memory and keeps no per-call state.
 *    The caller owns every buffer, including the workspace, and must keep them
 *    alive until the stream has executed the call.
 *  - `out` must not overlap any input, state or workspace (RLA2_ERR_ALIAS).
 *    q, k and v may overlap each other (they are only read).
 *  - NaN/Inf inputs are not checked; they propagate to the outputs.
 *  - RLA2_ERR_HIP means a HIP launch failed; outputs are then undefined.
 *  - Supported head dimensions: 32, 64, 128. Supported chunks: 16, 32, 64, 128.
 *  - Sizes whose kernel grids would not fit one dispatch (more than 2^32 work-items in a
 *    grid dimension: roughly 8 million segments, or about a million documents at d = 128)
 *    return RLA2_ERR_BAD_SHAPE.
 */
#ifndef RLA2_H_
#define RLA2_H_

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum rla2_status {
  RLA2_OK = 0,
  RLA2_ERR_NULL_POINTER = 1, /* a required pointer is NULL                        */
  RLA2_ERR_BAD_SHAPE = 2,    /* negative size, or a shape rule below is broken     */
  RLA2_ERR_UNSUPPORTED = 3,  /* head dim, dtype or chunk outside the supported set */
  RLA2_ERR_BAD_VALUE = 4,    /* eps/rms_eps/rope_base not finite and > 0, bad env  */
  RLA2_ERR_WORKSPACE = 5,    /* workspace NULL or smaller than the queried size    */
  RLA2_ERR_ALIAS = 6,        /* an output overlaps an input or another output      */
  RLA2_ERR_HIP = 7,          /* a HIP runtime call failed                          */
  RLA2_ERR_BAD_SEQLENS = 8,  /* RLA2_VALIDATE=1 found a cu_seqlens contract breach */
  RLA2_ERR_MISALIGNED = 9    /* a tensor pointer is not 16-byte aligned             */
} rla2_status;

typedef enum rla2_dtype { RLA2_F32 = 0, RLA2_BF16 = 1 } rla2_dtype;

/*
 * Shape and options of a chunked forward or a state build.
 *  B, H, L, d   logical [B, H, L, d] of q, k, v (and out). With cu_seqlens the
 *               input is packed: B must be 1 and L is the total token count T.
 *  dtype        element type of q, k, v, out (rla2_dtype).
 *  chunk        C, tokens per chunk of the chunked evaluation: 16, 32, 64 or 128
 *               (RLA2_ERR_UNSUPPORTED otherwise). Every query reads the state at the
 *               start of its chunk and the keys of its chunk up to itself directly
 *               (the associativity of RLA page §1 applied per chunk); C changes only
 *               the rounding, not the result. In bf16 every size runs the
 *               warp-specialised output kernel (except 128 with the L2 denominator);
 *               fp32 runs a generic kernel. The backward always works in 32-token
 *               steps of its own, whatever C.
 *  seg_chunks   chunks per sequential segment of the sweep (a tuning knob that only
 *               changes fp32 summation order); 0 selects it automatically (bf16: the
 *               length a model of the sweeps' rounds of resident workgroups times
 *               their steps rates fastest; fp32 and the state build: the longest that
 *               still gives 512 workgroups). A segment
 *               of seg_chunks * chunk tokens must be a multiple of 64 tokens and at
 *               most 4096 (RLA2_ERR_BAD_VALUE otherwise): 0..64 for C = 64, multiples
 *               of 4 up to 256 for C = 16, of 2 up to 128 for C = 32, 0..32 for
 *               C = 128.
 *  eps          denominator offset, RLA page §3 uses 1e-4. Finite, > 0.
 *  rms_eps      RMSNorm epsilon (inside the square root). Finite, > 0.
 *  rope_base    RoPE base (10000 on the RLA-2 workloads). Finite, > 0.
 *  cu_seqlens   NULL: each of the B rows is one document [0, L).
 *               Otherwise DEVICE int32[n_docs + 1] prefix sums of document lengths:
 *               cu[0] == 0, non-decreasing, cu[n_docs] == L (the contract of the
 *               CANN ops-transformer page, Compressor constraints). Contents are a
 *               caller contract, checked (with a host synchronisation) only when
 *               the environment variable RLA2_VALIDATE=1; out-of-range values are
 *               clamped to [0, L] so they can never cause an out-of-bounds access.
 *               Zero-length documents are allowed.
 *  n_docs       number of documents when cu_seqlens != NULL (>= 0); ignored
 *               (treated as B) when cu_seqlens == NULL.
 *  bidirectional  0: causal, out_t reads the state after token t (RLA page §3).
 *               1: every token reads its whole document's state, out_t =
 *               q'_t S_doc / (q'_t . z_doc + eps) (RLA page §4.1, the scan's
 *               causal=false mode: one constant state per document). Other
 *               values return RLA2_ERR_BAD_VALUE.
 *  initial_S, initial_z  optional DEVICE fp32 [H, d, d] and [H, d] (both or
 *               neither; one of them NULL returns RLA2_ERR_NULL_POINTER): a state
 *               that starts the first document of each row -- every row when
 *               cu_seqlens == NULL, document 0 when packed -- as the prefix scan's
 *               A0/B0 inputs of RLA page §4.1 do (one per head, shared by the
 *               batch rows, first document only). Layout as final_S:
 *               initial_S[h][a][c] pairs key dim a with value dim c. Read only;
 *               outputs must not overlap them (RLA2_ERR_ALIAS).
 *  initial_pos  position of the first token of the first document of each row
 *               (>= 0; a continuation passes the length of the context its
 *               initial state summarises). Other documents start at 0.
 *               initial_pos + L must fit in int32 (RLA2_ERR_BAD_VALUE otherwise).
 *  denominator  RLA2_DEN_SUM (0): the RLA-2 denominator q'_t . z_t + eps (RLA page
 *               §3). RLA2_DEN_L2 (1): the original RLA's L2 denominator (RLA page
 *               §2.1), out_t = sum_i s_ti v_i / (sqrt(sum_i s_ti^2) + eps),
 *               s_ti = q'_t . k'_i over the same key range (causal or the whole
 *               document), formed from the second state A = sum_i k'_i k'_i^T (RLA
 *               page §4.1): sum_i s_ti^2 = q'_t^T A q'_t; the page's eps for it is
 *               1e-6. The backward of the L2 mode is not built (RLA2_ERR_UNSUPPORTED).
 *               Other values return RLA2_ERR_BAD_VALUE.
 *  initial_A    L2 mode only (RLA2_ERR_BAD_VALUE otherwise): optional DEVICE fp32
 *               [H, d, d], the second state A0 that starts the first document of each
 *               row with initial_S (RLA page §4.1: A0 and B0 together; with an initial
 *               state in the L2 mode it is required, RLA2_ERR_NULL_POINTER otherwise).
 *               Read only; symmetric in exact arithmetic (A0[a][b] = sum k'[a] k'[b]).
 *  final_A      L2 mode only (RLA2_ERR_BAD_VALUE otherwise): optional DEVICE fp32
 *               [N, H, d, d] output, each document's second state after its last token
 *               (plus initial_A for the first document of each row): written by
 *               rla2_fwd_chunked and by rla2_state_from_prefix; NULL = not exported.
 *  grad_initial_S, grad_initial_z  read by the backward calls only (the other calls
 *               ignore them): optional DEVICE fp32 [H, d, d] and [H, d] outputs, the
 *               gradients of the loss with respect to initial_S and initial_z (each may be
 *               NULL = not formed; the state is taken as zero where initial_S is NULL, which
 *               is the same forward). The initial state enters the first document of each
 *               row (RLA page §4.1), so with g = dL/dout, den_t = q'_t . z_t + eps:
 *               grad_initial_S[h] = sum_t q'_t g_t^T / den_t and grad_initial_z[h] =
 *               -sum_t (g_t . out_t) / den_t q'_t over the tokens of those documents, summed
 *               over the rows in row order (deterministic) -- the backward's reverse state
 *               at each such document's first token. Written, not accumulated; 16-byte
 *               aligned (RLA2_ERR_MISALIGNED) and overlapping no other buffer
 *               (RLA2_ERR_ALIAS).
 * The number of documents N is n_docs with cu_seqlens, B without.
 * A zero-initialised descriptor tail (bidirectional = initial_pos = 0, NULL
 * initial state, denominator = RLA2_DEN_SUM, NULL initial_A and final_A, NULL
 * gradient outputs) is the plain causal forward.
 */
typedef struct rla2_fwd_desc {
  int32_t B, H, L, d;
  int32_t dtype;
  int32_t chunk;
  int32_t seg_chunks;
  float eps, rms_eps, rope_base;
  const int32_t* cu_seqlens;
  int32_t n_docs;
  int32_t bidirectional;
  int32_t initial_pos;
  const float* initial_S;
  const float* initial_z;
  int32_t denominator;
  const float* initial_A;
  float* final_A;
  float* grad_initial_S;
  float* grad_initial_z;
} rla2_fwd_desc;

#define RLA2_DEN_SUM 0
#define RLA2_DEN_L2 1

/* Human-readable name of a status code (static storage; never NULL). */
const char* rla2_status_string(rla2_status status);

/* ABI version of this header (bumped on any layout or signature change). */
int32_t rla2_abi_version(void);

/*
 * Device-side checks. Every workspace starts with a small status header that the first
 * launch of each call clears; the call's kernels raise these flags in it:
 *  RLA2_FLAG_WAIT_EXHAUSTED  a bounded wait inside a kernel ran out (the four matrix waves of
 *                            a workgroup meet on an LDS arrival counter in the bf16 forward
 *                            and backward sweeps; every wait is bounded so that no wave can
 *                            spin forever). The call's outputs are undefined.
 *  RLA2_FLAG_PLAN_MISMATCH   rla2_bwd_chunked_saved: fwd_workspace was not last written by a
 *                            forward whose plan matches desc (shape, segmentation, position
 *                            offset, cu_seqlens contents, causal or bidirectional records).
 *                            The backward then computed nothing; dq, dk, dv and the weight
 *                            gradients are left unwritten.
 * rla2_workspace_flags synchronises `stream`, then reads the flags of the last call that used
 * `workspace` (workspace_bytes: its size, at least 256). RLA2_ERR_NULL_POINTER for a NULL
 * workspace or flags, RLA2_ERR_WORKSPACE when it is misaligned or too small, RLA2_ERR_HIP
 * when the stream or the copy fails.
 */
#define RLA2_FLAG_WAIT_EXHAUSTED 1u
#define RLA2_FLAG_PLAN_MISMATCH 2u
rla2_status rla2_workspace_flags(const void* workspace, size_t workspace_bytes, hipStream_t stream,
                                 uint32_t* flags);

/*
 * Test hook for the bounded waits above: the number of polls a matrix wave makes before it
 * gives up at a meeting, for calls that start after this one (process-wide; the default is
 * about 2 million polls, tens of milliseconds). 0 makes every meeting give up at once: the
 * kernels still run to their normal end and raise RLA2_FLAG_WAIT_EXHAUSTED, and their
 * outputs are garbage. Returns the previous value.
 */
uint32_t rla2_debug_set_wait_polls(uint32_t polls);

/*
 * Workspace bytes rla2_fwd_chunked needs for `desc` (host call, no GPU work).
 * Writes *bytes; returns the same validation status the forward would.
 */
rla2_status rla2_fwd_workspace_size(const rla2_fwd_desc* desc, size_t* bytes);

/*
 * Chunked RLA-2 forward (RLA page §3 formula; the chunking is the
 * associativity of §1: a d x d state carried across chunks, each chunk's own
 * causal part formed directly). Causal, or bidirectional per desc->bidirectional;
 * an optional initial state per desc->initial_S/initial_z.
 *  q, k, v      [B, H, L, d] dtype, read only.
 *  gamma_q/k    [H, d] fp32 RMSNorm weights of q and k.
 *  out          [B, H, L, d] dtype, written (every row of every document).
 *  final_S      optional [N, H, d, d] fp32: each document's state after its last
 *               token, S[a][c] = sum_i k'_i[a] v_i[c] (plus the initial state for
 *               the first document of each row); NULL = not exported.
 *  final_z      optional [N, H, d] fp32, z = sum_i k'_i; NULL = not exported.
 *  workspace    device scratch of at least rla2_fwd_workspace_size() bytes,
 *               256-byte aligned; contents on entry are ignored. After a causal
 *               forward with the Sum denominator it holds the status header (plan
 *               stamp and flags, see rla2_workspace_flags), the segment table, the
 *               RoPE tables and every segment's prefix state, which
 *               rla2_bwd_chunked_saved reads in place of forming them again.
 * L == 0 or N == 0 is a valid no-op (final states of empty documents are 0).
 */
rla2_status rla2_fwd_chunked(const rla2_fwd_desc* desc, const void* q, const void* k,
                             const void* v, const float* gamma_q, const float* gamma_k,
                             void* out, float* final_S, float* final_z, void* workspace,
                             size_t workspace_bytes, hipStream_t stream);

/* Number of kernels one forward launches (see rla2_fwd_chunked_profiled). */
#define RLA2_FWD_KERNELS 4

/*
 * rla2_fwd_chunked for measurement tools. `events` holds RLA2_FWD_KERNELS + 1
 * events created by the caller (hipEventCreate). events[i] is recorded on
 * `stream` right before kernel i of the forward -- 0 set-up (segment map and
 * RoPE tables), 1 chunk state, 2 state scan, 3 chunk output -- and events[RLA2_FWD_KERNELS]
 * after the last, so hipEventElapsedTime(events[i], events[i + 1]) is kernel i's
 * duration (0 when the kernel is not needed). NULL `events` behaves exactly like
 * rla2_fwd_chunked. Same arguments, ownership and errors otherwise.
 */
rla2_status rla2_fwd_chunked_profiled(const rla2_fwd_desc* desc, const void* q, const void* k,
                                      const void* v, const float* gamma_q, const float* gamma_k,
                                      void* out, float* final_S, float* final_z, void* workspace,
                                      size_t workspace_bytes, hipStream_t stream,
                                      hipEvent_t* events);

/*
 * rla2_fwd_chunked for callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation): the same forward with no
 * workspace argument. Its workspace is a file-scope device array of
 * RLA2_NOALLOC_SCRATCH_BYTES (64 MiB) that each GPU the library runs on holds until the
 * process ends; the call allocates nothing (its first call on a device only looks up the
 * array's address there). Problems whose rla2_fwd_workspace_size exceeds that size return
 * RLA2_ERR_WORKSPACE before anything is enqueued (the long-context forward of 32 heads x
 * 65536 tokens at d = 128 needs about 35 MB). Every call on a GPU shares that GPU's array:
 * calls that overlap on one GPU (on other streams or threads) race and must be serialised
 * by the caller. The call's device-side flags (rla2_workspace_flags) stay in that array and
 * cannot be read back. Arguments, outputs and other errors as for rla2_fwd_chunked.
 */
#define RLA2_NOALLOC_SCRATCH_BYTES (64u << 20)
rla2_status rla2_fwd_chunked_noalloc(const rla2_fwd_desc* desc, const void* q, const void* k,
                                     const void* v, const float* gamma_q, const float* gamma_k,
                                     void* out, float* final_S, float* final_z, hipStream_t stream);

/* Workspace bytes rla2_state_from_prefix needs for `desc`. */
rla2_status rla2_state_from_prefix_workspace_size(const rla2_fwd_desc* desc, size_t* bytes);

/*
 * State of every document after its last token, from its keys and values:
 * S = sum_i k'_i (x) v_i, z = sum_i k'_i (RLA page §3 state; §4.2 forward_step
 * keeps exactly this pair as its cache). q is not needed. The first document of
 * each row starts from desc->initial_S/initial_z at desc->initial_pos, as in the
 * forward; desc->bidirectional is validated but does not change the result. In the L2
 * mode a non-NULL desc->final_A also receives each document's second state
 * A = sum_i k'_i k'_i^T (starting from desc->initial_A): the cache of an L2 continuation.
 *  k, v     [B, H, L, d] dtype (packed [1, H, T, d] with cu_seqlens).
 *  gamma_k  [H, d] fp32.
 *  S        [N, H, d, d] fp32, written.   z  [N, H, d] fp32, written.
 * desc->eps is validated but unused.
 */
rla2_status rla2_state_from_prefix(const rla2_fwd_desc* desc, const void* k, const void* v,
                                   const float* gamma_k, float* S, float* z, void* workspace,
                                   size_t workspace_bytes, hipStream_t stream);

/* Workspace bytes rla2_bwd_chunked needs for `desc` (more when desc->grad_initial_S or
 * grad_initial_z is set: one whole-document reverse total per row). */
rla2_status rla2_bwd_workspace_size(const rla2_fwd_desc* desc, size_t* bytes);

/*
 * Chunked backward of the forward (RLA page §4.2 backward of the layer): with g = dL/dout,
 * gnum_t = g_t / (q'_t . z_t + eps), scale_t = -(g_t . num_t) / (q'_t . z_t + eps)^2,
 * dq'_t = S_t gnum_t + scale_t z_t and, with the suffix sums P_i = sum_{t >= i} q'_t gnum_t^T
 * and p_i = sum_{t >= i} scale_t q'_t (same document), dk'_i = P_i v_i + p_i,
 * dv_i = P_i^T k'_i; then through the ReLU (gate q' > 0), RoPE and RMSNorm to dq, dk and the
 * RMSNorm weights. desc->bidirectional = 1 differentiates the bidirectional forward (the
 * page's bidirectional branch: S_t, z_t are the document's totals for every query, P_i, p_i
 * the document's totals for every key). The forward's states and g . num are recomputed from
 * q, k, v (the forward output is not an input). bf16 or fp32 activations; the Sum
 * denominator only (RLA2_ERR_UNSUPPORTED for the L2 denominator). An initial state and
 * position offset in desc are taken into account; the gradient with respect to the initial
 * state goes to desc->grad_initial_S / grad_initial_z when they are set (the reverse states
 * P, p at each first document's first token: the suffix scan's whole-document totals, summed
 * over the rows by one more small launch). desc->chunk does not change the arithmetic of the
 * backward.
 *  q, k, v       [B, H, L, d] dtype, the forward's inputs.
 *  gamma_q/k     [H, d] fp32.
 *  dout          [B, H, L, d] dtype, dL/dout (read).
 *  dq, dk, dv    [B, H, L, d] dtype, written.
 *  dgamma_q/k    optional [H, d] fp32, written (NULL = not formed).
 *  workspace     at least rla2_bwd_workspace_size() bytes, 256-byte aligned.
 * Outputs must not overlap any input, each other or the workspace (RLA2_ERR_ALIAS).
 */
rla2_status rla2_bwd_chunked(const rla2_fwd_desc* desc, const void* q, const void* k, const void* v,
                             const float* gamma_q, const float* gamma_k, const void* dout,
                             void* dq, void* dk, void* dv, float* dgamma_q,
                             float* dgamma_k, void* workspace, size_t workspace_bytes,
                             hipStream_t stream);

#define RLA2_BWD_KERNELS 8

/*
 * rla2_bwd_chunked with hipEvent_t markers, for measurement tools. `events` holds
 * RLA2_BWD_KERNELS + 1 events created by the caller; event i is recorded on `stream`
 * right before kernel i -- 0 set-up, 1 chunk state, 2 prefix scan of the states, 3 dq,
 * 4 reverse-state totals, 5 suffix scan, 6 dk and dv, 7 RMSNorm-weight sums -- and
 * events[RLA2_BWD_KERNELS] after the last (a kernel that is not needed takes no time).
 * NULL `events` behaves exactly like rla2_bwd_chunked. Same arguments, ownership and
 * errors otherwise.
 */
rla2_status rla2_bwd_chunked_profiled(const rla2_fwd_desc* desc, const void* q, const void* k,
                                      const void* v, const float* gamma_q, const float* gamma_k,
                                      const void* dout, void* dq, void* dk, void* dv,
                                      float* dgamma_q, float* dgamma_k, void* workspace,
                                      size_t workspace_bytes, hipStream_t stream,
                                      hipEvent_t* events);

/*
 * rla2_bwd_chunked without its state pass: the forward's states S_t, z_t (RLA page §4.2,
 * the states the backward of the layer reads) are taken from `fwd_workspace`, the
 * workspace of an rla2_fwd_chunked call with the same desc (causal or bidirectional, Sum
 * denominator) and the same k, v, gamma_k and initial state, not written since. The plan stamp that forward
 * left in the workspace header (shape, segmentation, position offset, scan mode and a
 * checksum of the cu_seqlens contents) is compared on the device with this call's plan
 * first: on a mismatch no backward kernel touches memory and the backward's own workspace
 * reports RLA2_FLAG_PLAN_MISMATCH (rla2_workspace_flags); the tensors k, v, gamma_k and the
 * initial state cannot be checked and remain the caller's contract. fwd_workspace is only
 * read, so one forward's workspace serves any number of backward calls. Results are bitwise
 * those of rla2_bwd_chunked.
 *  fwd_workspace        device pointer, 256-byte aligned, at least
 *                       rla2_fwd_workspace_size() bytes (fwd_workspace_bytes); it may
 *                       not overlap the outputs or `workspace` (RLA2_ERR_ALIAS).
 *  events               NULL, or RLA2_BWD_KERNELS + 1 events as for
 *                       rla2_bwd_chunked_profiled (kernels 0..2 are not run).
 * Other arguments, ownership and errors as for rla2_bwd_chunked; RLA2_ERR_WORKSPACE when
 * fwd_workspace is too small or misaligned, RLA2_ERR_NULL_POINTER when it is NULL and
 * the problem is not empty.
 */
rla2_status rla2_bwd_chunked_saved(const rla2_fwd_desc* desc, const void* q, const void* k,
                                   const void* v, const float* gamma_q, const float* gamma_k,
                                   const void* dout, void* dq, void* dk, void* dv,
                                   float* dgamma_q, float* dgamma_k, void* workspace,
                                   size_t workspace_bytes, const void* fwd_workspace,
                                   size_t fwd_workspace_bytes, hipStream_t stream,
                                   hipEvent_t* events);

/* Workspace bytes rla2_feature_map needs for `desc` (segment table and RoPE tables). */
rla2_status rla2_feature_map_workspace_size(const rla2_fwd_desc* desc, size_t* bytes);

/*
 * The shared preamble of the layer on its own (RLA page §4.2: Q/K -> RMSNorm ->
 * RoPE -> ReLU; §3: q' = ReLU(RoPE(RMSNorm(q))), k' likewise), materialised:
 *  q, k          [B, H, L, d] dtype, read; either may be NULL (then its gamma
 *                and output are ignored), not both.
 *  gamma_q/k     [H, d] fp32.
 *  q_out, k_out  [B, H, L, d] dtype, written with q' and k', rounded once to the
 *                element type. Bitwise the values the forward forms internally.
 * Positions follow desc exactly as in the forward (restart at each document
 * start; the first document of each row starts at desc->initial_pos);
 * desc->eps, bidirectional and the initial state are validated but unused.
 * Outputs must not overlap any input, each other or the workspace.
 */
rla2_status rla2_feature_map(const rla2_fwd_desc* desc, const void* q, const void* k,
                             const float* gamma_q, const float* gamma_k, void* q_out, void* k_out,
                             void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * One decode step for N sequences (RLA page §4.2 forward_step): the feature map
 * of the new token at its position, then the state update first
 * (S += k' (x) v, z += k'), then the read-out out = q' S / (q' . z + eps).
 *  q, k, v     [N, H, d] dtype, the new token of each sequence.
 *  positions   DEVICE int32[N]: position of the new token (its prefix length),
 *              >= 0 (negative values are treated as 0).
 *  gamma_q/k   [H, d] fp32.
 *  S, z        [N, H, d, d], [N, H, d] fp32, updated IN PLACE.
 *  out         [N, H, d] dtype, written.
 * N == 0 is a valid no-op.
 */
rla2_status rla2_decode_step(int32_t N, int32_t H, int32_t d, int32_t dtype, const void* q,
                             const void* k, const void* v, const int32_t* positions,
                             const float* gamma_q, const float* gamma_k, float rms_eps,
                             float rope_base, float eps, float* S, float* z, void* out,
                             hipStream_t stream);

/*
 * One decode step with the original RLA's L2 denominator (RLA page §4.2 forward_step
 * with the §2.1 closed form; the second state is the A of the §4.1 scan): the feature
 * map of the new token at its position, then the state update first (S += k' (x) v,
 * A += k' (x) k', z += k' when z is given), then the read-out
 * out = q' S / (sqrt(q'^T A q') + eps), eps the L2 constant (1e-6 on the page).
 *  q, k, v, positions, gamma_q/k, out   as in rla2_decode_step.
 *  S, A        [N, H, d, d] fp32, updated IN PLACE (A: the states of
 *              rla2_state_from_prefix's final_A in the L2 mode).
 *  z           [N, H, d] fp32, updated in place, or NULL (the L2 read-out does not
 *              use it).
 * Errors as rla2_decode_step; A must not be NULL (RLA2_ERR_NULL_POINTER), and S, A,
 * z and out must not overlap each other or an input (RLA2_ERR_ALIAS). N == 0 is a
 * valid no-op.
 */
rla2_status rla2_decode_step_l2(int32_t N, int32_t H, int32_t d, int32_t dtype, const void* q,
                                const void* k, const void* v, const int32_t* positions,
                                const float* gamma_q, const float* gamma_k, float rms_eps,
                                float rope_base, float eps, float* S, float* A, float* z,
                                void* out, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* RLA2_H_ */
