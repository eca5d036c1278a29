// Kernel launcher: picks the (dk, dv, gate, dtype) variant and enqueues
// schedule (packed input only) -> prep -> scan on the caller's stream.
#include "drla_common.h"
#include "drla_kernels.h"

#include <atomic>

namespace drla {

// KDA operand bytes from which the LDS-fed scan takes KDA calls (launch_all).
constexpr int64_t kKdaLdsScanBytes = 112ll << 20;

// Compute units of the current device (cached per device).
static int device_cus() {
  static std::atomic<int> cached[16];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 16) return 0;
  int n = cached[dev].load(std::memory_order_relaxed);
  if (n == 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n < 1) return 0;
    cached[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}

template <int DK, int DV, bool KDA, typename ET>
static hipError_t launch_all(const drla_launch_args* a, const Sched& s) {
  hipStream_t st = (hipStream_t)a->stream;
  void* const* ev = a->stage_events;
  char* ws = (char*)a->workspace;
  hipError_t e = hipSuccess;
  auto mark = [&](int i) {
    if (ev && e == hipSuccess) e = hipEventRecord((hipEvent_t)ev[i], st);
  };
  const int grp = a->h_v / a->h_qk;
  const int64_t nc = a->n_chunks;

  PrepParams pp = {};
  pp.q = a->q;
  pp.k = a->k;
  pp.beta = a->beta;
  pp.g = a->g;
  pp.tb = ws + a->off_tb;
  pp.pm = ws + a->off_pm;
  // the LDS-fed scan (GDN, 16-bit inputs) transposes K itself and needs no K~^T
  constexpr bool kLdsScan = !KDA && sizeof(ET) == 2;
  pp.kt = kLdsScan ? nullptr : ws + a->off_kt;
  pp.kw = KDA ? ws + a->off_kw : nullptr;
  pp.qw = KDA ? ws + a->off_qw : nullptr;
  pp.gam = (float*)(ws + a->off_gam);
  pp.s = s;
  pp.h_qk = a->h_qk;
  pp.h_v = a->h_v;
  pp.grp = grp;
  pp.nc = nc;
  pp.decay_only = a->decay_only;

  ScanParams sp = {};
  sp.q = a->q;
  sp.k = a->k;
  sp.v = a->v;
  sp.g = a->g;
  sp.h0 = a->h0;
  sp.o = a->o;
  sp.ht = a->ht;
  sp.tb = pp.tb;
  sp.pm = pp.pm;
  sp.kt = pp.kt;
  sp.kw = pp.kw;
  sp.qw = pp.qw;
  sp.gam = pp.gam;
  sp.insp_vp = a->inspect ? ws + a->off_vp : nullptr;
  sp.insp_h = a->inspect ? ws + a->off_h : nullptr;
  sp.s = s;
  sp.h_qk = a->h_qk;
  sp.h_v = a->h_v;
  sp.grp = grp;
  sp.nc = nc;
  sp.decay_only = a->decay_only;

  mark(0);
  if (e == hipSuccess && s.chunk_seq && a->n_seqs > 0)
    e = launch_schedule(a->cu_dev, a->n_seqs, nc, a->total_tokens, a->max_cps, a->cu_hash,
                        (int32_t*)(ws + a->off_sched), st);
  if (e == hipSuccess) e = launch_prep<DK, KDA, ET>(pp, nc * a->h_v, st);
  mark(1);
  // Head-resident scan (DRLA_HEAD_SCAN; scalar gate, 16-bit inputs): one
  // workgroup per (sequence, head) unit and segment
  if constexpr (kLdsScan) {
    if (a->head_scan && !a->inspect) {
      HScanParams hp = {};
      hp.q = a->q;
      hp.k = a->k;
      hp.v = a->v;
      hp.h0 = a->h0;
      hp.o = a->o;
      hp.ht = a->ht;
      hp.tb = pp.tb;
      hp.pm = pp.pm;
      hp.gam = pp.gam;
      hp.s = s;
      hp.h_qk = a->h_qk;
      hp.h_v = a->h_v;
      hp.grp = grp;
      hp.nc = nc;
      hp.units = (int32_t)((int64_t)a->n_seqs * a->h_v);
      hp.decay_only = a->decay_only;
      int32_t np = 1;
      if (a->off_hs && DK == DV && !a->serial) {
        const int cus = device_cus();
        np = cus > 0 ? drla_hs_count(hp.units, a->max_cps, cus) : 1;
        if (np > a->hs_np) np = a->hs_np;  // what the workspace holds
      }
      hp.np = np;
      if (np > 1) {
        char* hs = ws + a->off_hs;
        hp.en = (float*)hs;
        hp.phi = hs + (size_t)(a->hs_np - 1) * hp.units * DK * DV * 4;
      }
      if (e == hipSuccess) e = launch_hscan<DK, DV, ET>(hp, st);
      mark(2);
      return e;
    }
  }
  // packed input: the scan deals (sequence, head) units in groups of eight
  // (scan_item); the grid covers whole groups
  const int64_t units = (int64_t)a->n_seqs * a->h_v;
  int64_t nscan = (s.seq_order ? (units + 7) / 8 * 8 : units) * (DV / 16);
  // Segment mode (SegParams): a call whose scan leaves most of the chip
  // idle takes np segments, as many as let all its scan workgroups (one per
  // compute unit) run at once: (2 np - 1) K, or np K with the LDS-fed GDN
  // scan's paired chains, whose segment 0 is made longer by the paired
  // workgroups' longer period (drla_seg_pair_w0); drla_seg_plan picks the
  // form.  (With more workgroups than compute units the scan's period per
  // chunk grows with the occupancy more than the shorter segments save.)
  // The KDA and fp32 scans take the unpaired form.
  bool seg = false;
  if constexpr (DK == DV) {
    const int64_t K = units * (DV / 16);
    const int cus = device_cus();
    bool pair = false;
    int32_t np = cus > 0 ? drla_seg_plan(K, a->max_cps, cus, kLdsScan, &pair) : 1;
    if (np > a->seg_np) np = a->seg_np;  // what the workspace holds
    if (a->off_seg && !a->inspect && !a->serial && np > 1) {
      seg = true;
      const drla_seg_layout L = drla_seg_offsets(units, DK, a->total_tokens, a->h_v, a->seg_np, sizeof(ET));
      char* sg = ws + a->off_seg;
      sp.seg.s1 = 1;
      sp.seg.np = np;
      sp.seg.pair = pair ? 1 : 0;
      sp.seg.w0 = pair ? drla_seg_pair_w0(np) : 256;
      sp.seg.us = units * DK * DV;
      sp.seg.mid = (float*)(sg + L.mid);
      sp.seg.n = (float*)(sg + L.n);
      sp.seg.m = (float*)(sg + L.m);
      sp.seg.midf = sg + L.f;
      sp.seg.g = sg + L.g;
      nscan = (pair ? np : 2 * np - 1) * K;
    }
  }
  if (e == hipSuccess) {
    if constexpr (kLdsScan)
      e = launch_scan_lds<DK, DV, ET>(sp, nscan, a->inspect != 0, st);
    else if constexpr (KDA && sizeof(ET) == 2) {
      // KDA with 16-bit inputs: the LDS-fed scan once prep's operands
      // (K e^B, K~^T and Q e^B, 3 C dk elements per head and chunk) crowd
      // the 256 MiB last-level cache, the register-fed scan below that
      // (measured: the LDS-fed one 5-15% faster from 120 MiB, 3-8% slower
      // at 96 MiB and below)
      const int64_t opnd = nc * a->h_v * 3 * C * DK * (int64_t)sizeof(ET);
      if (opnd >= kKdaLdsScanBytes)
        e = launch_scan_lds_kda<DK, DV, ET>(sp, nscan, a->inspect != 0, st);
      else
        e = launch_scan<DK, DV, KDA, ET>(sp, nscan, a->inspect != 0, st);
    } else {
      e = launch_scan<DK, DV, KDA, ET>(sp, nscan, a->inspect != 0, st);
    }
  }
  if constexpr (DK == DV) {
    // (two segments: the fix-up launch forms ht itself)
    if (seg && sp.seg.np > 2 && e == hipSuccess) e = launch_seg_compose<DK, ET>(sp, units, st);
    if (seg && e == hipSuccess) e = launch_seg_fix<DK, ET>(sp, units, (int32_t)a->max_cps, st);
  }
  mark(2);
  return e;
}

}  // namespace drla

hipError_t drla_launch(const drla_launch_args* a) {
  using namespace drla;
  Sched s = {};
  int32_t* sched = (int32_t*)((char*)a->workspace + a->off_sched);
  if (a->cu_dev) {
    s.chunk_seq = sched;
    s.chunk_start = sched + a->n_chunks;
    s.seq_chunk0 = sched + 2 * a->n_chunks;
    s.seq_order = sched + 2 * a->n_chunks + a->n_seqs + 1;
    s.cu = sched + drla_sched_cu(a->n_chunks, a->n_seqs);  // the checked copy
  } else {
    s.seq_len = a->n_seqs > 0 ? a->total_tokens / a->n_seqs : 0;
    s.cps = (int32_t)((s.seq_len + C - 1) / C);
  }
  s.n_seqs = a->n_seqs;
  const int io = a->f32 ? 1 : a->f16 ? 2 : 0;
  const int key = (a->dk == 128 ? 1 : 0) | (a->dv == 128 ? 2 : 0) | (a->kda ? 4 : 0) | (io << 3);
#define DRLA_CASE(K, DK_, DV_, KDA_, ET_) \
  case K:                                 \
    return launch_all<DK_, DV_, KDA_, ET_>(a, s);
  switch (key) {
    DRLA_CASE(0, 64, 64, false, bf16)
    DRLA_CASE(1, 128, 64, false, bf16)
    DRLA_CASE(2, 64, 128, false, bf16)
    DRLA_CASE(3, 128, 128, false, bf16)
    DRLA_CASE(4, 64, 64, true, bf16)
    DRLA_CASE(5, 128, 64, true, bf16)
    DRLA_CASE(6, 64, 128, true, bf16)
    DRLA_CASE(7, 128, 128, true, bf16)
    DRLA_CASE(8, 64, 64, false, float)
    DRLA_CASE(9, 128, 64, false, float)
    DRLA_CASE(10, 64, 128, false, float)
    DRLA_CASE(11, 128, 128, false, float)
    DRLA_CASE(12, 64, 64, true, float)
    DRLA_CASE(13, 128, 64, true, float)
    DRLA_CASE(14, 64, 128, true, float)
    DRLA_CASE(15, 128, 128, true, float)
    DRLA_CASE(16, 64, 64, false, f16)
    DRLA_CASE(17, 128, 64, false, f16)
    DRLA_CASE(18, 64, 128, false, f16)
    DRLA_CASE(19, 128, 128, false, f16)
    DRLA_CASE(20, 64, 64, true, f16)
    DRLA_CASE(21, 128, 64, true, f16)
    DRLA_CASE(22, 64, 128, true, f16)
    DRLA_CASE(23, 128, 128, true, f16)
    default:
      return hipErrorInvalidValue;
  }
#undef DRLA_CASE
}
