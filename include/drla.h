/*
 * drla -- chunked prefill of delta-rule linear attention on MI355X (gfx950).
 *
 * C ABI.  Plain pointers and sizes; no framework types.  Device pointers are
 * HIP device memory; host pointers are ordinary host memory.
 *
 * What is computed.  For every sequence and value head, the token-by-token
 * gated delta rule that "Empowering Hybrid Attention Models on NPUs"
 * describes in Section 2.1 (the state S_{t-1} is updated with K_t and V_t,
 * then the output is read from the updated state S_t with Q_t), with the
 * state stored key-major, S in R^{dk x dv}:
 *
 *   GDN (scalar gate per token and head, Section 1 and Section 2.1):
 *     S_t = exp(g_t) (I - beta_t k_t k_t^T) S_{t-1} + beta_t k_t v_t^T
 *   KDA (per-channel gate, Section 1; its cumulative gate is per key
 *        channel, Section 7.5):
 *     S_t = (I - beta_t k_t k_t^T) Diag(exp(g_t)) S_{t-1} + beta_t k_t v_t^T
 *   both: o_t = S_t^T q_t
 *
 * evaluated chunkwise (64 tokens) in the Map-Reduce-Map form of Section 2.1:
 * a chunk-parallel prep kernel (operators #1-#3 Gate, KKT, Solve, and the
 * factor T diag(beta) that operator #4 W/U is built from, kept unexpanded
 * as in Section 5's operator rewriting), then the state scan (#5 H) fused
 * with the output (#6 O) chunk by chunk, state first-read, then output,
 * then in-place update (Section 5, "cross-chunk reordering").  Sequences
 * can be scanned as segments at once, stitched by the segments' affine
 * state maps (Section 4, Chunk-Seg-Seg mapping).  Results equal the
 * recurrence up to rounding.
 *
 * Layouts (row-major, token-major, sequences packed back to back):
 *   q, k        [T, h_qk, dk]    io dtype
 *   v           [T, h_v,  dv]    io dtype
 *   beta        [T, h_v]         fp32, used as given (typically in (0,1))
 *   g           GDN: [T, h_v]; KDA: [T, h_v, dk]   fp32 log-decay (<= 0)
 *   h0, ht      [N, h_v, dk, dv] fp32 (key-major state per sequence, head)
 *   o           [T, h_v, dv]     io dtype
 *   cu_seqlens  [N+1] int32, cu[0] = 0, non-decreasing, cu[N] = T.
 * io dtype: bf16, fp16 (the precision of the experiment setup, Section 7.1:
 * FP16 q/k/v with fp32 gates and states) or fp32;
 * arithmetic accumulates in fp32 and chunk intermediates are stored in the
 * io dtype.
 * v-head h reads q/k head h / (h_v / h_qk) (contiguous groups).  Without
 * cu_seqlens the T tokens are N equal-length sequences (a dense batch).
 * Chunks start at every sequence start; a sequence's last chunk may be short.
 *
 * Ownership.  The caller owns every buffer, including the workspace (size
 * from drla_workspace_bytes).  The library allocates no device memory, keeps
 * no state between calls except the thread-local last-error text, and never
 * synchronises: a call enqueues its kernels on `stream` (a hipStream_t; NULL
 * = the default stream) and returns.  The workspace must not be used by
 * another call until this call's kernels have finished on `stream`.
 *
 * Errors.  Every argument check happens before anything is enqueued; on an
 * error nothing is launched and nothing is written.  A launch failure returns
 * DRLA_ERR_HIP.  drla_last_error() gives a message for the last failing call
 * on this host thread.  Device faults surface at the caller's next
 * synchronisation, as for any kernel.
 */
#ifndef DRLA_H
#define DRLA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define DRLA_CHUNK 64

typedef enum {
  DRLA_OK = 0,
  DRLA_ERR_NULL = 1,        /* a required pointer is NULL                     */
  DRLA_ERR_SHAPE = 2,       /* negative/zero sizes, h_v % h_qk != 0, T % N    */
  DRLA_ERR_UNSUPPORTED = 3, /* dk or dv not in {64, 128}; unknown io dtype    */
  DRLA_ERR_ALIGN = 4,       /* a device pointer is not 16-byte aligned        */
  DRLA_ERR_SEQLENS = 5,     /* cu_seqlens malformed, or only one of the pair  */
  DRLA_ERR_WORKSPACE = 6,   /* workspace NULL or smaller than required        */
  DRLA_ERR_ALIAS = 7,       /* an output overlaps an input (ht == h0 allowed) */
  DRLA_ERR_HIP = 8          /* a HIP launch or runtime call failed            */
} drla_status;

typedef enum { DRLA_BF16 = 0, DRLA_F32 = 1, DRLA_F16 = 2 } drla_dtype;

typedef struct {
  int32_t n_seqs;       /* N >= 1                                          */
  int32_t h_qk;         /* query/key heads                                  */
  int32_t h_v;          /* value heads; multiple of h_qk                    */
  int32_t dk;           /* key dim, 64 or 128                               */
  int32_t dv;           /* value dim, 64 or 128                             */
  int32_t io_dtype;     /* drla_dtype of q, k, v and o                      */
  int64_t total_tokens; /* T >= 0                                           */
} drla_problem;

/* Workspace bytes a gdn_prefill or kda_prefill call on `p` needs (the
 * larger of the two; a GDN call uses less).  `cu_seqlens_host` is the host
 * copy of cu_seqlens (NULL for a dense batch).  Returns 0 if `p` or the
 * lengths are invalid (the prefill call then reports why). */
size_t drla_workspace_bytes(const drla_problem* p,
                            const int32_t* cu_seqlens_host);

/* Gated DeltaNet chunked prefill (scalar gate g [T, h_v]).
 *   q, k, v, beta, g      device inputs, layouts above
 *   h0                    device [N,h_v,dk,dv] fp32 initial state, or NULL (zeros)
 *   cu_seqlens_dev/_host  the same [N+1] array on device and host, or both NULL
 *                         (with N = 1 the call is run, and its workspace laid
 *                         out, as the dense call; the arrays are not read).
 *                         The host copy is validated here and sizes the
 *                         launch and the workspace; the kernels take the
 *                         lengths from the device copy, which the first
 *                         kernel checks against the host copy (cu[0] = 0,
 *                         non-decreasing, cu[N] = T, chunk counts, and a
 *                         64-bit fingerprint of all N+1 entries).  If the
 *                         two differ the call runs as N empty sequences: no
 *                         token is read, o is left unwritten, ht = h0 (zeros
 *                         without h0), and drla_prefill_status reports
 *                         DRLA_ERR_SEQLENS; the call itself, asynchronous,
 *                         has already returned DRLA_OK.
 *   o                     device output [T,h_v,dv] in io dtype
 *   ht                    device output [N,h_v,dk,dv] fp32 final state, or NULL;
 *                         may be exactly h0 (in-place state update)
 *   workspace, ws_bytes   device scratch of at least drla_workspace_bytes(p, cu_host)
 *   stream                hipStream_t
 * All device pointers must be 16-byte aligned. */
drla_status gdn_prefill(const drla_problem* p, const void* q, const void* k,
                        const void* v, const float* beta, const float* g,
                        const float* h0, const int32_t* cu_seqlens_dev,
                        const int32_t* cu_seqlens_host, void* o, float* ht,
                        void* workspace, size_t workspace_bytes, void* stream);

/* Kimi Delta Attention chunked prefill: identical to gdn_prefill except that
 * g is per key channel, [T, h_v, dk] fp32.
 * Gate range: any g <= 0 whose magnitude, summed over the tokens between
 * any row of a 16-token tile of a chunk and the tile's ninth row, stays
 * below 88 per key channel (|g| < 11 per token suffices, a per-token decay
 * above e^{-11}).  The in-chunk products weigh each key channel by
 * e^{B_r - B_i} (B the in-chunk cumulative gate, r >= i): tiles below the
 * diagonal factor it about their row tile's first row (both factors at most
 * 1, any gate), the diagonal tiles about their ninth row in fp32 (factors
 * within e^{+-8 max|g|}).  gdn_prefill takes exponentials of gate
 * differences directly and accepts any g <= 0.  The same range holds for
 * decay_prefill with per_channel. */
drla_status kda_prefill(const drla_problem* p, const void* q, const void* k,
                        const void* v, const float* beta, const float* g,
                        const float* h0, const int32_t* cu_seqlens_dev,
                        const int32_t* cu_seqlens_host, void* o, float* ht,
                        void* workspace, size_t workspace_bytes, void* stream);

/* One decode step of Gated DeltaNet: one token per sequence continuing
 * from the state h0 -- the per-token recurrence of "Empowering Hybrid
 * Attention Models on NPUs", Section 2.1, that the chunked prefill also
 * computes (decay the state, x = S^T k, S += beta k (v - x)^T, o = S^T q).
 *   p                     total_tokens must equal n_seqs (row n is sequence
 *                         n's token); dk, dv, heads and io dtype as prefill
 *   q, k                  device [N, h_qk, dk] in io dtype
 *   v                     device [N, h_v, dv] in io dtype
 *   beta, g               device [N, h_v] fp32 (g: log-decay)
 *   h0                    device [N, h_v, dk, dv] fp32 state, or NULL (zeros)
 *   o                     device output [N, h_v, dv] in io dtype
 *   ht                    device output [N, h_v, dk, dv] fp32, or NULL; may
 *                         be exactly h0 (the usual in-place step)
 *   stream                hipStream_t
 * No workspace; all device pointers 16-byte aligned; errors as prefill
 * (checked before anything is enqueued). */
drla_status gdn_decode(const drla_problem* p, const void* q, const void* k,
                       const void* v, const float* beta, const float* g,
                       const float* h0, void* o, float* ht, void* stream);

/* Kimi Delta Attention decode step: as gdn_decode with g per key channel,
 * [N, h_v, dk] fp32 (the state's key rows decay by e^{g}). */
drla_status kda_decode(const drla_problem* p, const void* q, const void* k,
                       const void* v, const float* beta, const float* g,
                       const float* h0, void* o, float* ht, void* stream);

/* Decay-only linear attention, the temporal-decay form of RetNet and GLA
 * ("Empowering Hybrid Attention Models on NPUs", Section 8, Related Work):
 * no delta rule and no beta,
 *   S_t = Diag(exp(g_t)) S_{t-1} + k_t v_t^T,   o_t = S_t^T q_t,
 * with a scalar gate g [T, h_v] (per_channel == 0) or a per-key-channel gate
 * g [T, h_v, dk] (per_channel != 0).  Same kernels, layouts, workspace,
 * ownership and errors as gdn_prefill / kda_prefill (beta is not passed);
 * chunkwise this is the delta-rule form with T = I and no state read in V'. */
drla_status decay_prefill(int per_channel, const drla_problem* p, const void* q,
                          const void* k, const void* v, const float* g,
                          const float* h0, const int32_t* cu_seqlens_dev,
                          const int32_t* cu_seqlens_host, void* o, float* ht,
                          void* workspace, size_t workspace_bytes, void* stream);

/* Decode step of decay-only linear attention: as gdn_decode / kda_decode
 * without beta (S = Diag(exp(g)) S + k v^T, o = S^T q). */
drla_status decay_decode(int per_channel, const drla_problem* p, const void* q,
                         const void* k, const void* v, const float* g,
                         const float* h0, void* o, float* ht, void* stream);

/* Flags of drla_prefill_ex. */
#define DRLA_KEEP_INTERMEDIATES 1 /* also write V' and the per-chunk state (tests) */
#define DRLA_DECAY_ONLY 2         /* decay-only linear attention (decay_prefill); beta unused */
#define DRLA_SERIAL 4             /* scan every sequence in one pass (no segment split) */
#define DRLA_HEAD_SCAN 8          /* scalar gate, 16-bit io: the head-resident scan */
#define DRLA_COLUMN_SCAN 16       /* the per-16-column scan, its segment split as usual */

/* gdn_prefill (kda == 0) or kda_prefill (kda != 0) with options.
 *   flags         any combination of DRLA_KEEP_INTERMEDIATES, DRLA_DECAY_ONLY,
 *                 DRLA_SERIAL and one of DRLA_HEAD_SCAN, DRLA_COLUMN_SCAN,
 *                 or 0 (both scan flags: DRLA_ERR_UNSUPPORTED).
 *                 The state scan runs one workgroup per (sequence, head,
 *                 16 state columns).  Calls with dk == dv whose
 *                 U = n_seqs * h_v * dv/16 column blocks
 *                 leave most of the device idle split every sequence's
 *                 chunks into np segments that are scanned at once: np the
 *                 most up to 16 for which (2 np - 1) U is at most the
 *                 device's compute units (and at most 256) and the longest
 *                 sequence has at least 4 np chunks; the later segments
 *                 take floor(n / np) chunks each, segment 0 the rest.
 *                 Scalar-gate calls with 16-bit inputs may instead run a
 *                 later segment's two chains in one workgroup (np U at most
 *                 the compute units) where that split cannot run or leaves
 *                 at least 96 chunks per segment; segment 0 is then longer
 *                 than the others, which take floor(256 n / (w + 256 (np -
 *                 1))) chunks each, w = 352 for two segments, else 307.
 *                 DRLA_HEAD_SCAN (scalar gate, 16-bit inputs, not with
 *                 DRLA_KEEP_INTERMEDIATES) runs the head-resident scan
 *                 instead: one workgroup per (sequence, head) unit holds all
 *                 dv state columns; when the units leave compute units idle
 *                 and dk == dv, each sequence's n chunks are split into np
 *                 segments scanned at once and stitched by their affine
 *                 state maps (Section 4, Chunk-Seg-Seg mapping): np the most
 *                 with n_seqs h_v np at most the compute units (at most
 *                 256), np^2 <= 9 n_max, at least two chunks per segment of
 *                 the longest sequence (n_max chunks) and np <= 128; fewer
 *                 than three segments run one pass.  Without flags,
 *                 scalar-gate calls with 16-bit inputs and dk = dv = 128
 *                 take the head-resident scan where its measured timing
 *                 model predicts it at least 10% faster (8 to 16 heads and
 *                 long sequences, or many more (head, 16-column) chains
 *                 than compute units; the rule is the one in the library's
 *                 launch header, drla_auto_head_scan, at 256 compute units).
 *                 DRLA_COLUMN_SCAN keeps the per-16-column scan, segments
 *                 included.  DRLA_SERIAL runs either scan in one pass (same
 *                 results up to rounding); alone it selects the
 *                 per-16-column scan.
 *                 DRLA_DECAY_ONLY runs decay_prefill (kda selects the
 *                 per-channel gate; beta is ignored and may be NULL).
 *                 With DRLA_KEEP_INTERMEDIATES the kernels
 *                 also store, per (value head, chunk), V' = U - W S (the
 *                 "v_c" intermediate of Section 5) and the state entering the
 *                 chunk, at the offsets drla_workspace_layout reports for the
 *                 same flags; the workspace must then be that layout's total.
 *   stage_events  NULL, or three caller-created hipEvent_t (passed as void*)
 *                 recorded on `stream`: [0] before the first kernel, [1]
 *                 after the prep kernel (operators #1-#4 of Section 2.1), [2]
 *                 after the scan/output kernel (#5, #6), so that a benchmark
 *                 can time each kernel on the stream it runs on.  A failing
 *                 event record returns DRLA_ERR_HIP.
 * Other arguments and errors as for gdn_prefill. */
drla_status drla_prefill_ex(int kda, int flags, const drla_problem* p, const void* q,
                            const void* k, const void* v, const float* beta,
                            const float* g, const float* h0,
                            const int32_t* cu_seqlens_dev,
                            const int32_t* cu_seqlens_host, void* o, float* ht,
                            void* workspace, size_t workspace_bytes, void* stream,
                            void* const* stage_events);

/* Byte offsets of the regions of the workspace of a call of drla_prefill_ex
 * with the same kda, problem, lengths and flags, for inspection by tests.
 * Each is stored per (value head, chunk), chunk index fastest, as MFMA
 * operand fragments: a fragment covers 16 "outer" x 32 "inner" indices and
 * is 64 lanes x 8 contiguous elements; lane l = 16 g + c (g < 4, c < 16)
 * holds outer index c at inner indices 4g + j (j < 4) and 12 + 4g + j
 * (4 <= j < 8).
 *   tb:  T diag(beta), T = (I + A)^{-1}; 8 fragments (outer token tile 0..3,
 *        inner token block 0..1, index tile*2 + block); fragments 1 and 3
 *        lie above the diagonal (zero) and are not stored, here and in pm
 *   pm:  P = lower_incl(Q K^T (.) D) (the intra-chunk output weights), 8
 *        fragments in the same order
 *   kt:  K~^T, K~ = e^{b_n - b} (.) K; dk/8 fragments (outer key-channel
 *        tile, inner token block, index tile*2 + block); only for KDA and
 *        fp32 inputs (else 0: that scan transposes K on chip)
 *   kw, qw (KDA only): K (.) e^{B}, Q (.) e^{B}; dk/8 fragments (outer token
 *        tile, inner key block, index tile*(dk/32) + block)
 *   gam: decay factors, fp32: GDN e^{b_r} for the 64 token rows (row 63 is
 *        e^{b_n}) then e^{b_n - b_r}, 128 floats; KDA e^{b_n} per key
 *        channel, dk floats
 *   vp, h (only with DRLA_KEEP_INTERMEDIATES, else 0): V' (outer value tile,
 *        inner token block, index tile*2 + block) and the state entering the
 *        chunk (outer value tile, inner key block, index tile*(dk/32) + block)
 *   seg (calls with dk == dv that the segment split takes on a 256-CU
 *        device, else 0):
 *        for np segments, the fp32 state after the first segment, np - 1
 *        zero-start final states and np - 1 maps of the entering state
 *        (fp32, per (sequence, head)), np - 1 entering states as io-type
 *        fragments, then the maps' contribution to o per token, laid out as o
 *   hs (head-resident scan calls that split into np > 1 segments on a
 *        256-CU device, else 0): np - 1 fp32 state sets of dk x dv per (sequence, head) unit
 *        (the segments' zero-start final states, replaced in place by the
 *        states entering segments 1 .. np - 1), then np - 2 segment maps of
 *        dk x dk per unit in io type
 * head_scan records which scan the call takes: 1 for the head-resident scan
 * (DRLA_HEAD_SCAN, or chosen by its timing model), 0 for the per-16-column
 * scan.
 * Elements are io dtype except gam and the seg and hs states (fp32).
 * n_chunks is the total chunk count over all sequences.  Returns DRLA_OK or
 * a validation error. */
typedef struct {
  int64_t n_chunks;
  size_t sched, tb, pm, kt, kw, qw, gam, vp, h, seg, hs, total;
  size_t head_scan; /* 1: the call takes the head-resident scan, 0: the per-16-column one */
} drla_layout;
drla_status drla_workspace_layout(int kda, const drla_problem* p,
                                  const int32_t* cu_seqlens_host, int flags,
                                  drla_layout* out);

/* Bytes of the library's own scratch array (per GPU) that
 * drla_prefill_noalloc uses in place of a workspace: 64 MiB. */
#define DRLA_NOALLOC_SCRATCH_BYTES (64ull << 20)

/* drla_prefill_ex without a workspace, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc).  The call allocates nothing: its
 * kernels use a fixed scratch array of DRLA_NOALLOC_SCRATCH_BYTES that the
 * library holds on each GPU it runs on until the process ends (its device
 * address is looked up once per device, at the first call there).
 *   kda, flags, p, q ... ht, stream   as drla_prefill_ex (no stage events)
 * Errors as drla_prefill_ex; a call whose workspace (drla_workspace_layout
 * for the same kda, problem, lengths and flags) exceeds the scratch array
 * returns DRLA_ERR_WORKSPACE before touching the device.  Every call on a
 * GPU shares that GPU's array: calls that overlap in time on one GPU (on
 * different streams, or from different host threads without ordering)
 * race and give wrong results.  Calls ordered on one stream are safe; no
 * call relies on what an earlier one left in the array. */
drla_status drla_prefill_noalloc(int kda, int flags, const drla_problem* p,
                                 const void* q, const void* k, const void* v,
                                 const float* beta, const float* g,
                                 const float* h0, const int32_t* cu_seqlens_dev,
                                 const int32_t* cu_seqlens_host, void* o,
                                 float* ht, void* stream);

/* Whether the device and host cu_seqlens of the last packed prefill call
 * that used `workspace` agreed (see cu_seqlens_dev/_host at gdn_prefill).
 * p and cu_seqlens_host: that call's; workspace: its workspace, or NULL for
 * this GPU's drla_prefill_noalloc scratch (the current device's).  Waits
 * for `stream` (the call's stream), then reads the status word the call's
 * first kernel wrote into the workspace's schedule region.  Returns DRLA_OK
 * if they agreed or the call was not packed (N = 1 or no cu_seqlens: no
 * device lengths are read), DRLA_ERR_SEQLENS if they differed (or the word
 * holds no status), DRLA_ERR_HIP if the read failed, and the validation
 * errors of drla_workspace_bytes for a malformed p or cu_seqlens_host.
 * Costs a device-to-host copy and a stream synchronisation: a debugging or
 * checking aid, not part of the prefill. */
drla_status drla_prefill_status(const drla_problem* p, const int32_t* cu_seqlens_host,
                                const void* workspace, void* stream);

const char* drla_status_str(drla_status s);
const char* drla_last_error(void);
int drla_version(void);

#ifdef __cplusplus
}
#endif
#endif /* DRLA_H */
