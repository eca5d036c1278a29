// Internal interface between the C ABI layer (drla_api.cpp) and the kernel
// launcher (drla_launch.hip).  Not part of the public ABI.
#ifndef DRLA_LAUNCH_H
#define DRLA_LAUNCH_H
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#define DRLA_CHUNK_TOKENS 64

// Segment count of the segment-split scan of a dense call (1: no split):
// the most P <= 16 for which the scan's workgroups all fit on `cus` compute
// units at once (one per CU; K = sequences x heads x dv/16 chains) and
// the longest sequence has at least 4 P chunks (cps).  The scan takes
// (2P - 1) K workgroups, or P K with `paired` chains (a later segment's
// zero-start and transition chains in one workgroup: the LDS-fed GDN scan).
static inline int32_t drla_seg_count(int64_t K, int64_t cps, int64_t cus, bool paired) {
  int32_t np = 1;
  for (int32_t p = 2; p <= 16; ++p)
    if (K > 0 && (paired ? p : 2 * p - 1) * K <= cus && cps >= 4 * p) np = p;
  return np;
}

// Segment plan of a dense call: np segments, and whether a later segment's
// two chains share a workgroup (`paired`, only where `can_pair`: the LDS-fed
// GDN scan).  Pairing fits twice the segments on the chip but runs the
// paired workgroups about 1.3x slower per chunk, and every segment past the
// second adds a serial compose step (2-3 us), so it is taken only where the
// unpaired split cannot run (its 3 K workgroups exceed the compute units) or
// leaves at least 96 chunks per segment.  Measured on MI355X (GDN bf16, one
// sequence; call us, unpaired -> paired): H16 d128 T4096 one pass 68.5 ->
// 63.7 (2 segments), H2 T65536 172 -> 160 (8 -> 16 segments); H4 T16384 98
// -> 97, H8 T8192 85 -> 84 (equal); H4 T4096 44 -> 56, H8 T4096 52 -> 59,
// H4 d64 T8192 38 -> 53, H1 T65536 125 -> 140 (16 segments either way).
static inline int32_t drla_seg_plan(int64_t K, int64_t cps, int64_t cus, bool can_pair, bool* paired) {
  const int32_t nu = drla_seg_count(K, cps, cus, false);
  const int32_t npp = can_pair ? drla_seg_count(K, cps, cus, true) : 1;
  const bool pair = npp > nu && (nu == 1 || cps / nu >= 96);
  if (paired) *paired = pair;
  return pair ? npp : nu;
}

// Weight of segment 0 against each later segment with paired chains, x 256
// (seg_span): about the period per chunk of a paired workgroup over that of
// a one-chain workgroup, so that all segments end together.  Measured best
// on MI355X (GDN, d = 128): 352 at two segments (16 heads; 307 and 400 are
// 2-4 % slower), 307 from four (2 to 8 heads, 4 to 16 segments).
static inline int32_t drla_seg_pair_w0(int32_t np) { return np == 2 ? 352 : 307; }

// Segments per sequence of the head-resident scan: as many as give every
// (sequence, head) unit's segments one compute unit each (units x np <=
// cus), at most about sqrt(9 n) for n chunks of the longest sequence (the
// serial compose step grows with np while the segment scans shrink with
// n / np), at least two chunks per segment, at most 128.  Fewer than three
// segments gain nothing over one pass: 1.
static inline int32_t drla_hs_count(int64_t units, int64_t max_cps, int64_t cus) {
  if (units <= 0 || max_cps <= 0) return 1;
  int64_t np = cus / units;
  int64_t cap = 1;
  while ((cap + 1) * (cap + 1) <= 9 * max_cps) ++cap;
  if (np > cap) np = cap;
  if (np > max_cps / 2) np = max_cps / 2;
  if (np > 128) np = 128;
  return np < 3 ? 1 : (int32_t)np;
}

// Whether a call without DRLA_HEAD_SCAN or DRLA_SERIAL takes the
// head-resident scan: GDN or decay-only, 16-bit inputs, dk = dv = 128 (the
// shapes its timing model was measured on), when the model predicts it at
// least 10 % faster than the per-16-column scan.  Scan-stage models from
// MI355X measurements (microseconds; n chunks of the longest sequence,
// unit_chunks the chunks of all (sequence, head) units together):
//   head-resident, np_hs >= 3 segments: 36 + 8.5 ceil(n / np_hs);
//   head-resident, one pass: 4.07 max(n, unit_chunks / cus) -- with every
//     compute unit busy, each pulling all of its unit's operands from HBM;
//   per-16-column, chains (units x dv/16) <= cus: 0.9 ceil(n / np_seg) plus
//     12 for the compose and fix-up when it splits (its chains run at once);
//   per-16-column, more chains than compute units: 1.06 max(n, unit_chunks
//     dv/16 / cus) -- bound by the chunks each compute unit is dealt.
// The last two are from one 8-sequence, 32-head packed batch (scan 545
// against 460 us); with fewer busy compute units the head-resident scan
// runs faster per chunk than 4.07, so the rule errs towards the
// per-16-column scan.  np_seg is the unpaired count: where drla_seg_plan
// pairs chains instead (16 heads of d = 128), the paired split's stage took
// 48.9, 84.3 and about 197 us at 4,096, 8,192 and 16,384 tokens against
// this estimate's 57.6, 115 and 230, and the choice (per-16-column, then
// head-resident from 16,384 tokens, 168 us) is the faster one either way.
static inline bool drla_auto_head_scan(int64_t units, int64_t max_cps, int64_t unit_chunks, int32_t dk,
                                       int32_t dv, int64_t cus) {
  if (dk != 128 || dv != 128 || units <= 0 || max_cps <= 0 || cus <= 0) return false;
  const int64_t chains = units * (dv / 16);
  const double n = (double)max_cps;
  const int32_t nh = drla_hs_count(units, max_cps, cus);
  double t_head, t_col;
  if (nh >= 3) {
    t_head = 36.0 + 8.5 * (double)((max_cps + nh - 1) / nh);
  } else {
    const double per_cu = (double)unit_chunks / (double)cus;
    t_head = 4.07 * (n > per_cu ? n : per_cu);
  }
  if (chains > cus) {
    const double per_cu = (double)unit_chunks * (double)(dv / 16) / (double)cus;
    t_col = 1.06 * (n > per_cu ? n : per_cu);
  } else {
    const int32_t ns = drla_seg_count(chains, max_cps, cus, false);
    t_col = 0.9 * (double)((max_cps + ns - 1) / ns) + (ns > 1 ? 12.0 : 0.0);
  }
  return t_head < 0.9 * t_col;
}

// Bytes of the head-resident scan's region for `units` units, np segments,
// dk x dv states and io elements of `es` bytes: np - 1 fp32 state sets, then
// np - 2 segment maps (dk x dk, io type).
static inline size_t drla_hs_bytes(int64_t units, int64_t dk, int64_t dv, int32_t np, size_t es) {
  if (np <= 1) return 0;
  return (size_t)(np - 1) * units * dk * dv * 4 + (size_t)(np > 2 ? np - 2 : 0) * units * dk * dk * es;
}

// Layout of the seg region (byte offsets from its start) for `units`
// (sequence, head) pairs of a d x d state, T tokens in all, h_v heads, np
// segments and io elements of `es` bytes: the state after segment 0, then
// np - 1 zero-start final states N, np - 1 transition maps M (all fp32),
// np - 1 entering states as io-type MFMA fragments, then G [T, h_v, d].
typedef struct {
  size_t mid, n, m, f, g, total;
} drla_seg_layout;
static inline drla_seg_layout drla_seg_offsets(int64_t units, int64_t d, int64_t T, int64_t h_v, int32_t np,
                                               size_t es) {
  const size_t us = (size_t)units * d * d;
  drla_seg_layout L;
  L.mid = 0;
  L.n = L.mid + us * 4;
  L.m = L.n + (size_t)(np - 1) * us * 4;
  L.f = L.m + (size_t)(np - 1) * us * 4;
  L.g = L.f + (size_t)(np - 1) * us * es;
  L.total = L.g + (size_t)T * h_v * d * es;
  return L;
}

// Fingerprint of a cu_seqlens array: the sum over its entries i of a
// 64-bit mix (the splitmix64 finaliser, Steele, Lea and Flood 2014) of
// (i, cu[i]).  The host takes it over cu_seqlens_host, the schedule kernel
// over the device copy; a sum is order-free, so the kernel's threads add
// their entries in any order.
__host__ __device__ static inline uint64_t drla_cu_mix(uint64_t i, uint32_t v) {
  uint64_t z = ((i << 32) | v) + 0x9E3779B97F4A7C15ull;
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

// The schedule region of a packed call, in int32 words from its start:
// chunk_seq [nc], chunk_start [nc], seq_chunk0 [n + 1], seq_order [n],
// the checked lengths cu [n + 1], the status word [1].
static inline int64_t drla_sched_words(int64_t nc, int64_t n) { return 2 * nc + 3 * n + 3; }
static inline int64_t drla_sched_cu(int64_t nc, int64_t n) { return 2 * nc + 2 * n + 1; }
static inline int64_t drla_sched_status(int64_t nc, int64_t n) { return 2 * nc + 3 * n + 2; }

typedef struct {
  const void* q;
  const void* k;
  const void* v;
  const float* beta;
  const float* g;
  const float* h0;
  const int32_t* cu_dev;  // NULL for a dense batch
  uint64_t cu_hash;       // drla_cu_mix summed over cu_seqlens_host
  void* o;
  float* ht;
  void* workspace;
  // byte offsets into the workspace; vp/h only used when inspect != 0
  size_t off_sched, off_tb, off_pm, off_kt, off_kw, off_qw, off_gam, off_vp, off_h;
  size_t off_seg;  // 0, or the segment-mode scan's states and G (dense calls)
  size_t off_hs;   // 0, or the head-resident scan's segment states and maps
  int32_t hs_np;   // segments the hs region holds (drla_hs_count at 256 CUs)
  int32_t seg_np;  // segments the seg region holds (drla_seg_count at 256 CUs)
  int64_t max_cps; // chunks of the longest sequence
  int64_t total_tokens;
  int64_t n_chunks;
  int32_t n_seqs, h_qk, h_v, dk, dv;
  int32_t kda, f32, f16, inspect;  // f32 / f16: io dtype (neither: bf16)
  int32_t decay_only;              // decay-only linear attention (no delta rule)
  int32_t serial;                  // scan every sequence in one pass (no segment split)
  int32_t head_scan;               // GDN 16-bit: the head-resident scan (DRLA_HEAD_SCAN)
  void* stream;
  void* const* stage_events;  // NULL, or 3 hipEvent_t recorded at kernel boundaries
} drla_launch_args;

hipError_t drla_launch(const drla_launch_args* a);

typedef struct {
  const void* q;
  const void* k;
  const void* v;
  const float* beta;
  const float* g;
  const float* h0;
  void* o;
  float* ht;
  int32_t n_seqs, h_qk, h_v, dk, dv;
  int32_t kda, f32, f16;
  int32_t decay_only;
  void* stream;
} drla_decode_args;

hipError_t drla_launch_decode(const drla_decode_args* a);

#endif
