// Kernel parameter blocks and per-variant launchers (internal).
#ifndef DRLA_KERNELS_H
#define DRLA_KERNELS_H

#include "drla_common.h"

namespace drla {

struct PrepParams {
  const void* q;
  const void* k;
  const float* beta;
  const float* g;
  void* tb;    // Tb = T diag(beta): 8 fragments per (head, chunk)
  void* pm;    // P: 8 fragments per (head, chunk)
  void* kt;    // K~^T: dk/8 fragments per (head, chunk), or null (not needed)
  void* kw;    // KDA: K e^{B}, dk/8 fragments
  void* qw;    // KDA: Q e^{B}, dk/8 fragments
  float* gam;  // GDN: e^{b_r} then e^{b_n - b_r}, 128 floats; KDA: e^{b_n} per key channel
  Sched s;
  int32_t h_qk, h_v, grp;
  int64_t nc;
  int32_t decay_only;  // no delta rule: beta = 1, A = 0 (T = I); beta may be null
};

// Segment-parallel scan (dk = dv): every sequence's n chunks are split into
// np segments (seg_span: segment 0 weighted w0 / 256 against each later
// one).  Segment 0 is scanned from h0 (final state into mid).  Every later
// segment s is scanned both from a zero state (its local outputs into o,
// final state into n[s-1]) and from the identity with V = 0 (the
// "transition": outputs G into g, final state M into m[s-1]); with `pair`
// one workgroup runs both chains over one copy of the chunk operands, else
// each has its own workgroups.  With E_1 = mid and E_{s+1} = N_s + M_s E_s
// (seg_compose), segment s's true outputs are o += G E_s (seg_fix) and
// ht = E_np.
struct SegParams {
  int32_t s1;   // > 0: segment mode
  int32_t np;   // segments
  int32_t w0;   // weight of segment 0 against a later segment, x 256
  int32_t pair; // 1: a later segment's two chains share a workgroup
  int64_t us;   // elements of one state set: sequences x heads x dk x dv
  void* g;      // [T, h_v, dk] in the io type, like o
  float* mid;   // [N, h_v, dk, dv]
  float* n;     // [np - 1][N, h_v, dk, dv]
  float* m;     // [np - 1][N, h_v, dk, dk]
  void* midf;   // [np - 1] E_s in the io type as A fragments: per (sequence,
                // head), dv/16 column tiles x dk/32 key blocks x 64 lanes x 8
};

struct ScanParams {
  const void* q;
  const void* k;
  const void* v;
  const float* g;
  const float* h0;
  void* o;
  float* ht;
  const void* tb;
  const void* pm;
  const void* kt;
  const void* kw;
  const void* qw;
  const float* gam;
  void* insp_vp;  // optional: V' per (head, chunk), fragments (dv tile, token block)
  void* insp_h;   // optional: state entering each chunk, fragments (dv tile, dk block)
  Sched s;
  int32_t h_qk, h_v, grp;
  int64_t nc;
  int32_t decay_only;  // no delta rule: R = V (no X term)
  SegParams seg;       // segment mode (both per-16-column scans)
};

// Head-resident scan (drla_hscan.hip): GDN and decay-only linear attention
// with a scalar gate and 16-bit inputs.  One workgroup per (unit, segment),
// all dv state columns; np segments per sequence (n / np chunks each, the
// last takes the rest), stitched by the segments' affine state maps.
struct HScanParams {
  const void* q;
  const void* k;
  const void* v;
  const float* h0;
  void* o;
  float* ht;
  const void* tb;    // prep: diag(e^{b_n - b}) Tb, 8 fragments per (head, chunk)
  const void* pm;    // prep: P Tb, 8 fragments per (head, chunk)
  const float* gam;  // prep: e^{b_r} then e^{b_n - b_r}, 128 floats per (head, chunk)
  float* en;         // np - 1 state sets (N_s, then E_{s+1}), tile order, fp32
  void* phi;         // np - 2 segment maps Phi_1 .. Phi_{np-2}, A fragments, io type
  Sched s;
  int32_t h_qk, h_v, grp;
  int64_t nc;
  int32_t np;     // segments per sequence (1: one pass)
  int32_t units;  // (sequence, head) units; indexed by rank (longest first when packed)
  int32_t decay_only;
};

template <int DK, int DV, typename T>
hipError_t launch_hscan(const HScanParams& P, hipStream_t st);

// One decode step: every input row is one sequence's token.
struct DecodeParams {
  const void* q;   // [N, h_qk, dk]
  const void* k;   // [N, h_qk, dk]
  const void* v;   // [N, h_v, dv]
  const float* beta;  // [N, h_v]
  const float* g;     // [N, h_v] (KDA: [N, h_v, dk])
  const float* h0;    // [N, h_v, dk, dv] or null
  void* o;            // [N, h_v, dv]
  float* ht;          // [N, h_v, dk, dv] or null; may be h0
  int32_t h_qk, h_v;
  int32_t decay_only;  // no delta rule: S = a S + k v^T; beta unused
};

hipError_t launch_schedule(const int32_t* cu, int n_seqs, int64_t nc, int64_t T, int64_t max_cps,
                           uint64_t hash, int32_t* sched, hipStream_t st);

template <int DK, bool KDA, typename ET>
hipError_t launch_prep(const PrepParams& P, int64_t nblk, hipStream_t st);

template <int DK, int DV, bool KDA, typename ET>
hipError_t launch_scan(const ScanParams& P, int64_t nblk, bool inspect, hipStream_t st);

// GDN with 16-bit inputs (T = bf16 or f16): the LDS-fed scan (drla_scan_lds.hip)
template <int DK, int DV, typename T>
hipError_t launch_scan_lds(const ScanParams& P, int64_t nblk, bool inspect, hipStream_t st);
// KDA with 16-bit inputs: the same LDS-fed scan on prep's K e^B, K~^T and
// Q e^B fragments
template <int DK, int DV, typename T>
hipError_t launch_scan_lds_kda(const ScanParams& P, int64_t nblk, bool inspect, hipStream_t st);

// After a segment-mode scan: o += G mid over segment 1, ht = n + M mid.
template <int DK, typename T>
hipError_t launch_seg_compose(const ScanParams& P, int64_t n_units, hipStream_t st);
template <int DK, typename T>
hipError_t launch_seg_fix(const ScanParams& P, int64_t n_units, int32_t cps, hipStream_t st);

}  // namespace drla

#endif
