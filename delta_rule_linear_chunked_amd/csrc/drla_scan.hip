// Sequential state scan fused with the output Map (gfx950).
//
// Operator #5 (H) of the Map-Reduce-Map split in "Empowering Hybrid
// Attention Models on NPUs", Section 2.1, is the only sequence-dependent
// step; operator #6 (O) needs only the state entering the chunk and the
// intermediate v_c (Section 5).  Following Section 5's chunk-first order
// (read the state, produce the output, then update the state in place), one
// workgroup walks the chunks of one (sequence, value head, 16 state columns)
// with the state in registers and produces the chunk's output on the way:
//
//   X   = diag(e^b) K S                    (KDA: (K e^{B}) S)
//   V'  = Tb (V - X)                       (= U - W S of Section 5's rewriting)
//   O   = diag(e^b) Q S + P V'             (KDA: (Q e^{B}) S + P V')
//   S  <- e^{b_n} S + K~^T V'              (KDA: Diag(e^{b_n}) S + K~^T V')
//
// Tb, P and K~^T come from the prep kernel.  The state columns are
// independent (the column split of Section 4, "Computation Splitting"), so
// workgroups for different column blocks never communicate; the 16 columns
// are the width of one MFMA tile.
//
// Inside the workgroup wave w owns token tile w (16 tokens) for X, V', O,
// and rows [16 (dk/64) w, ...) of the state for its update.  Per chunk the
// waves exchange the state (as 16-bit/fp32 fragments) and R = V - X through
// LDS, with two barriers.  Every wave needs all six Tb fragments; each loads
// at most two of them and the set is shared through LDS, so the chunk's
// operands cross the CU's load path once.
//
// KDA with 16-bit inputs (RING): the operand stream into registers bounds the
// kernel, so only each wave's own token tile of K e^B and Q e^B goes to
// registers; K~^T, Tb, P, V and e^{b_n} come through a three-slot LDS ring
// that two more waves fill with LDS-direct loads two chunks ahead.
#include "drla_common.h"
#include "drla_kernels.h"

namespace drla {

// Operands of one chunk for wave w.  Every load is unconditional: the
// chunk's rows of q, k, v and g are read through buffer resources limited to
// its valid tokens, so rows past the end of a short chunk read as zero, and
// no load sits behind a branch (a branch would make the compiler wait for
// all outstanding loads, including the next chunk's).
template <int DK, bool KDA, typename ET>
struct ScanOps {
  typedef typename VT<ET>::v4 V4;
  typedef typename VT<ET>::v8 V8;
  static constexpr int KB = DK / 32;
  static constexpr int MT = DK / 64;  // state row tiles per wave
  V8 kr[KB];       // K rows of token tile w, key channels 32p + 8g + j (KDA: K e^{B})
  V8 qr[KB];       // Q rows, same order (KDA: Q e^{B})
  V8 kt[MT][2];    // K~^T fragments of this wave's state rows
  V8 tb[2];        // this wave's share of the Tb fragments (see tb_frag)
  V8 pb[2];        // P fragments (w, 0), (w, 1)
  V4 vv;           // V at token 16w + c, columns 16 nb + 4g + e
  floatx4 gm[MT];  // KDA: e^{b_n} of this lane's state rows
  float eb;        // GDN: e^{b} of token 16w + c
  float gam;       // GDN: e^{b_n}
  rsrc_t orsrc;    // this chunk's rows of o
};

struct ScanCtx {
  int64_t ts;    // first token of the sequence (of the segment, in segment mode)
  int64_t te;    // one past the sequence's last token
  int64_t c0;    // workspace index of its first chunk
  int h, hk, nb, w, lane;
  bool vzero;    // V read as zero (segment transition blocks)
  void* obase;   // o, or G for segment transition blocks
};

// The six nonzero Tb fragments (0,0) (1,0) (2,0) (2,1) (3,0) (3,1) sit at
// these indices of the eight in the workspace; wave w loads shares 2w, 2w+1
// (wave 3 repeats the last one, so no load depends on the wave).
__device__ __forceinline__ int tb_frag(int j) { return j < 2 ? 2 * j : j + 2; }
__device__ __forceinline__ int tb_share(int w, int s) { return min(2 * w + s, 5); }

// One slot of the RING variant's operand ring (16-bit ET).
template <int DK, typename ET>
struct RingSlot {
  typedef typename VT<ET>::v8 V8;
  V8 kt[DK / 8][64];                             // K~^T fragments, index tile*2 + block
  V8 tb[6][64];                                  // Tb fragments, tb_frag order
  V8 pm[6][64];                                  // P fragments, same order
  __attribute__((aligned(16))) ET v[C][16];      // V, this block's 16 columns
  __attribute__((aligned(16))) float gam[256];   // e^{b_n} per key channel (dk used)
};

template <bool KDA, typename ET>
constexpr bool ring_variant() { return KDA && sizeof(ET) == 2; }

template <int DK, int DV, bool KDA, typename ET>
__device__ __forceinline__ void scan_load(ScanOps<DK, KDA, ET>& o, const ScanParams& P, const ScanCtx& x,
                                          int i) {
  constexpr bool RING = ring_variant<KDA, ET>();
  typedef typename VT<ET>::v4 V4;
  typedef typename VT<ET>::v8 V8;
  constexpr int KB = DK / 32, MT = DK / 64, es = sizeof(ET);
  const int lane = x.lane, w = x.w, g4 = lane >> 4, c16 = lane & 15;
  const int64_t t0 = x.ts + (int64_t)C * i;
  const int64_t left = x.te - t0;
  const uint32_t len = (uint32_t)(left < C ? left : C);
  const int64_t ch = (int64_t)x.h * P.nc + x.c0 + i;
  const int rw = 16 * w + c16;  // this lane's token in the chunk
  const uint32_t loff = (uint32_t)lane * sizeof(V8);  // lane's slot in a fragment
  if (KDA) {
    const rsrc_t kw = make_rsrc((const V8*)P.kw + ch * (C * DK / 8), C * DK * es);
    const rsrc_t qw = make_rsrc((const V8*)P.qw + ch * (C * DK / 8), C * DK * es);
#pragma unroll
    for (int p = 0; p < KB; ++p) {
      o.kr[p] = fload<V8>(kw, loff, w * KB + p);
      o.qr[p] = fload<V8>(qw, loff, w * KB + p);
    }
    if constexpr (!RING) {
      const rsrc_t gr = make_rsrc(P.gam + ch * DK, DK * 4);
#pragma unroll
      for (int m = 0; m < MT; ++m) o.gm[m] = bload<floatx4>(gr, state_row(w * MT + m, 4 * g4) * 4);
    }
  } else {
    const size_t qrow = (size_t)P.h_qk * DK;
    const rsrc_t kr = make_rsrc((const ET*)P.k + t0 * qrow, len * qrow * es);
    const rsrc_t qr = make_rsrc((const ET*)P.q + t0 * qrow, len * qrow * es);
    const uint32_t off = (uint32_t)(((size_t)rw * P.h_qk + x.hk) * DK + 8 * g4) * es;
#pragma unroll
    for (int p = 0; p < KB; ++p) {
      o.kr[p] = bload<V8>(kr, off + 32 * p * es);
      o.qr[p] = bload<V8>(qr, off + 32 * p * es);
    }
    const rsrc_t gr = make_rsrc(P.gam + ch * (2 * C), C * 4);
    // e^{b_n} is the same for every lane; an opaque per-lane offset keeps
    // it a vector value, so no scalar copy has to wait for the load
    uint32_t last = (C - 1) * 4;
    asm("" : "+v"(last));
    o.eb = bload<float>(gr, rw * 4);
    o.gam = bload<float>(gr, last);
  }
  const size_t vrow = (size_t)P.h_v * DV;
  o.orsrc = make_rsrc((ET*)x.obase + t0 * vrow, len * vrow * es);
  if constexpr (RING) return;
  const rsrc_t ktr = make_rsrc((const V8*)P.kt + ch * (C * DK / 8), C * DK * es);
#pragma unroll
  for (int m = 0; m < MT; ++m)
#pragma unroll
    for (int p = 0; p < 2; ++p) o.kt[m][p] = fload<V8>(ktr, loff, (w * MT + m) * 2 + p);
  const rsrc_t tbr = make_rsrc((const V8*)P.tb + ch * (8 * 64), 8 * 64 * sizeof(V8));
  o.tb[0] = fload<V8>(tbr, loff, tb_frag(tb_share(w, 0)));
  o.tb[1] = fload<V8>(tbr, loff, tb_frag(tb_share(w, 1)));
  const rsrc_t pmr = make_rsrc((const V8*)P.pm + ch * (8 * 64), 8 * 64 * sizeof(V8));
  o.pb[0] = fload<V8>(pmr, loff, 2 * w);
  o.pb[1] = fload<V8>(pmr, loff, 2 * w + 1);  // zero for w < 2
  const rsrc_t vr = make_rsrc((const ET*)P.v + t0 * vrow, x.vzero ? 0u : (uint32_t)(len * vrow * es));
  o.vv = bload<V4>(vr, (uint32_t)(((size_t)rw * P.h_v + x.h) * DV + 16 * x.nb + 4 * g4) * es);
}

template <int DK, int DV, bool KDA, typename ET, bool INSPECT>
__global__ __launch_bounds__((ring_variant<KDA, ET>() ? 384 : 256)) void scan_kernel(ScanParams P) {
  typedef typename VT<ET>::v4 V4;
  typedef typename VT<ET>::v8 V8;
  constexpr int KB = DK / 32, MT = DK / 64, NB = DV / 16, es = sizeof(ET);
  constexpr bool RING = ring_variant<KDA, ET>();
  constexpr int NS = 3;                          // RING: slots
  __shared__ V8 Sf[KB][64];                      // state entering the chunk, as fragments (inner = key channel)
  __shared__ V8 Rf[2][64];                       // R = V - X, as B fragments (inner = token)
  __shared__ V8 Tbs[RING ? 1 : 2][6][64];        // Tb fragments of chunk i (slot i % 2)
  __shared__ __attribute__((aligned(16))) unsigned char ring_raw[RING ? NS * sizeof(RingSlot<DK, ET>) : 16];
  RingSlot<DK, ET>* const ring = (RingSlot<DK, ET>*)ring_raw;

  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave index, uniform
  const int g4 = lane >> 4, c16 = lane & 15;
  int seq, h, nb;
  int kind = 0, sg = 0;  // 0: whole sequence; segment mode: 1, 2, 3 and the segment (seg_item)
  if (P.seg.s1 > 0) {
    int unit;
    seg_item(P.s.n_seqs * P.h_v, NB, P.seg.np, false, unit, nb, kind, sg);
    seq = unit / P.h_v;
    h = unit - seq * P.h_v;
  } else if (!scan_item(P.s, P.h_v, NB, seq, h, nb)) {
    return;  // the whole workgroup: past the last unit
  }

  ScanCtx x;
  x.h = h;
  x.hk = h / P.grp;
  x.nb = nb;
  x.w = w;
  x.lane = lane;
  int64_t n;  // chunks of this sequence
  if (P.s.chunk_seq) {
    x.ts = P.s.cu[seq];
    x.te = P.s.cu[seq + 1];
    int64_t c1;
    seq_chunks(P.s, seq, P.nc, x.c0, c1);
    n = x.te > x.ts ? (x.te - x.ts + C - 1) / C : 0;
    if (n > c1 - x.c0) n = c1 - x.c0;  // device lengths disagree with the table
  } else {
    x.ts = (int64_t)seq * P.s.seq_len;
    x.te = x.ts + P.s.seq_len;
    x.c0 = (int64_t)seq * P.s.cps;
    n = P.s.cps;
  }
  if (kind > 0) {
    // segment sg of this sequence (seg_span)
    int64_t first, len;
    seg_span(n, P.seg.np, P.seg.w0, sg, first, len);
    x.ts += (int64_t)C * first;
    x.c0 += first;
    n = len;
  }
  // segment transition blocks (kind 3) scan V = 0 from the identity and
  // write G in place of o; the final state goes to ht, or to the segment
  // mode's state sets
  x.vzero = kind == 3;
  x.obase = kind == 3 ? P.seg.g : P.o;
  float* const sout = kind == 0   ? P.ht
                      : kind == 1 ? P.seg.mid
                                  : (kind == 2 ? P.seg.n : P.seg.m) + (int64_t)(sg - 1) * P.seg.us;
  const int col = 16 * nb + c16;
  const int64_t sbase = ((int64_t)seq * P.h_v + h) * DK * DV;

  if constexpr (RING) {
    if (w >= 4) {
      // ---------------- loader waves (RING) ----------------
      // wave 4: K~^T and e^{b_n}; wave 5: Tb, P and this block's 16
      // columns of V.  Chunk i goes to slot i % NS two chunks ahead; every
      // copy reads through a descriptor that ends at the chunk's data (V:
      // at its last valid token, so rows past it read zero).
      constexpr int K4 = DK / 8 + 1, K5 = 6 + 6 + 2;  // copies per chunk
      const int nn = __builtin_amdgcn_readfirstlane((int)n);
      const uint32_t vstride = (uint32_t)(P.h_v * DV * es);
      const uint32_t voff = (uint32_t)(lane >> 1) * vstride + 16u * (uint32_t)(lane & 1);
      const uint32_t lo = 16u * (uint32_t)lane;
      auto issue = [&](int i) {
        RingSlot<DK, ET>& sl = ring[i % NS];
        const int64_t ch = (int64_t)h * P.nc + x.c0 + i;
        if (w == 4) {
          const rsrc_t kr = make_rsrc((const V8*)P.kt + ch * (C * DK / 8), C * DK * es);
#pragma unroll
          for (int f = 0; f < DK / 8; ++f) lds_dma16(kr, lo + 1024u * f, 0, &sl.kt[f][0]);
          lds_dma16(make_rsrc(P.gam + ch * DK, DK * 4), lo, 0, sl.gam);
        } else {
          const rsrc_t tr = make_rsrc((const V8*)P.tb + ch * (8 * 64), 8 * 64 * sizeof(V8));
          const rsrc_t pr = make_rsrc((const V8*)P.pm + ch * (8 * 64), 8 * 64 * sizeof(V8));
#pragma unroll
          for (int j = 0; j < 6; ++j) lds_dma16(tr, lo + 1024u * tb_frag(j), 0, &sl.tb[j][0]);
#pragma unroll
          for (int j = 0; j < 6; ++j) lds_dma16(pr, lo + 1024u * tb_frag(j), 0, &sl.pm[j][0]);
          const int64_t t0 = x.ts + (int64_t)C * i;
          const int64_t left = x.te - t0;
          const uint32_t len = (uint32_t)(left < C ? left : C);
          const rsrc_t vr = make_rsrc((const ET*)P.v + (t0 * P.h_v + h) * DV + 16 * nb,
                                      x.vzero ? 0u : (len - 1) * vstride + 16 * es);
          lds_dma16(vr, voff, 0, &sl.v[0][0]);
          lds_dma16(vr, voff + 32 * vstride, 0, &sl.v[32][0]);
        }
      };
      // wait until at most one chunk's copies (issued after the one
      // waited for) are in flight, or none
      auto wait_all_but_one = [&](bool one) {
        if (!one)
          __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
        else if (w == 4)
          __builtin_amdgcn_s_waitcnt(vmcnt_imm(K4));
        else
          __builtin_amdgcn_s_waitcnt(vmcnt_imm(K5));
      };
      if (nn > 0) {
        issue(0);
        if (nn > 1) issue(1);
        wait_all_but_one(nn > 1);  // chunk 0 has landed
      }
      // as many barriers as the compute waves: two per chunk
      for (int t = 0; t < nn; ++t) {
        lds_barrier();  // chunk t under way; slot (t + 2) % NS was last read in chunk t - 1
        const bool more = t + 2 < nn;
        if (more) issue(t + 2);
        lds_barrier();
        wait_all_but_one(more);  // chunk t + 1 has landed before the next chunk starts
      }
      __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
      return;
    }
  }

  // this wave's state rows: tiles w*MT + m, element e is key channel
  // state_row(mt, 4g + e), column col
  floatx4 S[MT];
#pragma unroll
  for (int m = 0; m < MT; ++m)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int row = state_row(w * MT + m, 4 * g4 + e);
      S[m][e] = kind == 3                 ? (row == col ? 1.f : 0.f)
                : kind != 2 && P.h0 ? P.h0[sbase + (int64_t)row * DV + col]
                                    : 0.f;
    }
  auto put_state = [&]() {
#pragma unroll
    for (int m = 0; m < MT; ++m) {
      const int mt = w * MT + m;
      ((V4*)&Sf[mt >> 1][lane])[mt & 1] = pack4<ET>(S[m]);
    }
  };
  put_state();

  // R element (token 16w + c, column 4g + e) belongs to fragment w/2, lane
  // 16 (c/4) + 4g + e, slot 4 (w%2) + c%4
  ET* const rdst = (ET*)&Rf[w >> 1][16 * (c16 >> 2) + 4 * g4] + 4 * (w & 1) + (c16 & 3);
  const uint32_t ooff = (uint32_t)(((size_t)(16 * w + c16) * P.h_v + h) * DV + 16 * nb + 4 * g4) * es;

  // this wave's Tb fragments of chunk i into the shared set; slot i % 2 was
  // last read in chunk i - 2, which every wave has finished once it is past
  // the first barrier of chunk i - 1
  auto put_tb = [&](const ScanOps<DK, KDA, ET>& op, int i) {
    if constexpr (!RING) {
      Tbs[i & 1][tb_share(w, 0)][lane] = op.tb[0];
      Tbs[i & 1][tb_share(w, 1)][lane] = op.tb[1];
    }
  };

  auto step = [&](const ScanOps<DK, KDA, ET>& op, int i) {
    // GDN decay factors (from prep): e^{b} of this lane's token, e^{b_n}
    const float eb = KDA ? 1.f : op.eb, gam = KDA ? 1.f : op.gam;
    lds_barrier();  // the state entering this chunk is in Sf, its Tb in Tbs (RING: chunk i in its slot)
    V8 sf[KB];
#pragma unroll
    for (int p = 0; p < KB; ++p) sf[p] = Sf[p][lane];
    // operands shared through LDS (RING: all but K e^B and Q e^B).  RING
    // reads V first and the operands of the second half (Tb, K~^T, P, the
    // decay) only once the products of X and O are issued: one wave issues
    // an LDS read every ~23 cycles, so reading them all up front would hold
    // the products back.
    V8 tb[6], kt[MT][2], pb[2];
    V4 vv;
    floatx4 gm[MT];
    const RingSlot<DK, ET>& sl = ring[RING ? i % NS : 0];
    if constexpr (RING) {
      vv = *(const V4*)&sl.v[16 * w + c16][4 * g4];
    } else {
#pragma unroll
      for (int f = 0; f < 6; ++f) tb[f] = Tbs[i & 1][f][lane];
      vv = op.vv;
#pragma unroll
      for (int m = 0; m < MT; ++m) {
        kt[m][0] = op.kt[m][0];
        kt[m][1] = op.kt[m][1];
        gm[m] = op.gm[m];
      }
      pb[0] = op.pb[0];
      pb[1] = op.pb[1];
    }
    if (INSPECT && w == 0) {
      V8* hp = (V8*)P.insp_h + ((int64_t)h * P.nc + x.c0 + i) * (int64_t)(DK * DV / 8);
#pragma unroll
      for (int p = 0; p < KB; ++p) hp[(nb * KB + p) * 64 + lane] = sf[p];
    }
    // X^T and the state part of O^T for token tile w: lane holds
    // [column 4g + e][token 16w + c]
    floatx4 xt = zero4(), o = zero4();
#pragma unroll
    for (int p = 0; p < KB; ++p) {
      xt = mma(sf[p], op.kr[p], xt);
      o = mma(sf[p], op.qr[p], o);
    }
    if constexpr (RING) {
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int f = 0; f < 6; ++f) tb[f] = sl.tb[f][lane];
#pragma unroll
      for (int m = 0; m < MT; ++m) {
        kt[m][0] = sl.kt[(w * MT + m) * 2][lane];
        kt[m][1] = sl.kt[(w * MT + m) * 2 + 1][lane];
        gm[m] = *(const floatx4*)&sl.gam[state_row(w * MT + m, 4 * g4)];
      }
      // P fragments (w, 0) and (w, 1) in tb_frag order; (w, 1) is zero and
      // unused for w < 2
      pb[0] = sl.pm[w < 2 ? w : 2 * w - 2][lane];
      pb[1] = sl.pm[w < 2 ? 0 : 2 * w - 1][lane];
      __builtin_amdgcn_sched_barrier(0);
    }
    const float ex = P.decay_only ? 0.f : eb;  // decay-only: R = V
#pragma unroll
    for (int e = 0; e < 4; ++e) rdst[8 * e] = (ET)(to_f(vv[e]) - ex * xt[e]);
    lds_barrier();  // R of all token tiles is in Rf
    const V8 rf0 = Rf[0][lane], rf1 = Rf[1][lane];
    floatx4 vt[4];
    vt[0] = mma(tb[0], rf0, zero4());
    vt[1] = mma(tb[1], rf0, zero4());
    vt[2] = mma(tb[3], rf1, mma(tb[2], rf0, zero4()));
    vt[3] = mma(tb[5], rf1, mma(tb[4], rf0, zero4()));
    // V' as the A operand of O^T and the B operand of the update (K~ already
    // carries e^{b_n - b})
    V8 vf[2];
#pragma unroll
    for (int p = 0; p < 2; ++p) vf[p] = pack<ET>(vt[2 * p], vt[2 * p + 1]);
    if (INSPECT && w == 0) {
      V8* vp = (V8*)P.insp_vp + ((int64_t)h * P.nc + x.c0 + i) * (int64_t)(C * DV / 8);
      vp[(nb * 2 + 0) * 64 + lane] = vf[0];
      vp[(nb * 2 + 1) * 64 + lane] = vf[1];
    }
    // S <- gamma S + K~^T V'
#pragma unroll
    for (int m = 0; m < MT; ++m) {
      if (KDA)
        S[m] *= gm[m];
      else
        S[m] *= gam;
      S[m] = mma(kt[m][0], vf[0], S[m]);
      S[m] = mma(kt[m][1], vf[1], S[m]);
    }
    put_state();
    // O^T tile: columns are tokens 16w + c; rows past the end are dropped
    o *= eb;
    o = mma(vf[0], pb[0], o);
    if (w >= 2) o = mma(vf[1], pb[1], o);
    bstore(op.orsrc, ooff, pack4<ET>(o));
  };

  // Two operand sets: the next chunk's operands load while this chunk
  // computes.  The fp32 variant's operands are twice as large; it loads one
  // chunk at a time.
  if (n > 0) {
    constexpr bool kPingPong = sizeof(ET) == 2;
    if (kPingPong) {
      // The scheduling barriers keep the memory operations in program order
      // -- next chunk's loads, this chunk's products, this chunk's store --
      // so that waiting for this chunk's operands never waits for the loads
      // just issued (loads and stores share one in-order counter).
      // Chunk counters are 32-bit and wave-uniform so that the loop control
      // stays on the scalar unit.
      const int nn = __builtin_amdgcn_readfirstlane((int)n);
      if constexpr (RING) {
        // only K e^B and Q e^B go to registers: three sets, loaded two
        // chunks ahead, cover the load latency
        ScanOps<DK, KDA, ET> bufa, bufb, bufc;
        scan_load<DK, DV, KDA, ET>(bufa, P, x, 0);
        scan_load<DK, DV, KDA, ET>(bufb, P, x, min(1, nn - 1));
        for (int i = 0; i < nn; i += 3) {
          __builtin_amdgcn_sched_barrier(0);
          scan_load<DK, DV, KDA, ET>(bufc, P, x, min(i + 2, nn - 1));
          __builtin_amdgcn_sched_barrier(0);
          step(bufa, i);
          __builtin_amdgcn_sched_barrier(0);
          if (i + 1 >= nn) break;
          scan_load<DK, DV, KDA, ET>(bufa, P, x, min(i + 3, nn - 1));
          __builtin_amdgcn_sched_barrier(0);
          step(bufb, i + 1);
          __builtin_amdgcn_sched_barrier(0);
          if (i + 2 >= nn) break;
          scan_load<DK, DV, KDA, ET>(bufb, P, x, min(i + 4, nn - 1));
          __builtin_amdgcn_sched_barrier(0);
          step(bufc, i + 2);
        }
      } else {
      ScanOps<DK, KDA, ET> bufa, bufb;
      scan_load<DK, DV, KDA, ET>(bufa, P, x, 0);
      put_tb(bufa, 0);
      for (int i = 0; i < nn; i += 2) {
        __builtin_amdgcn_sched_barrier(0);
        scan_load<DK, DV, KDA, ET>(bufb, P, x, min(i + 1, nn - 1));
        __builtin_amdgcn_sched_barrier(0);
        step(bufa, i);
        __builtin_amdgcn_sched_barrier(0);
        if (i + 1 >= nn) break;
        put_tb(bufb, i + 1);
        scan_load<DK, DV, KDA, ET>(bufa, P, x, min(i + 2, nn - 1));
        __builtin_amdgcn_sched_barrier(0);
        step(bufb, i + 1);
        __builtin_amdgcn_sched_barrier(0);
        put_tb(bufa, i + 2);
      }
      }
    } else {
      const int nn = __builtin_amdgcn_readfirstlane((int)n);
      ScanOps<DK, KDA, ET> buf;
      for (int i = 0; i < nn; ++i) {
        scan_load<DK, DV, KDA, ET>(buf, P, x, i);
        put_tb(buf, i);
        step(buf, i);
      }
    }
  }
  if (sout) {
#pragma unroll
    for (int m = 0; m < MT; ++m)
#pragma unroll
      for (int e = 0; e < 4; ++e)
        sout[sbase + (int64_t)state_row(w * MT + m, 4 * g4 + e) * DV + col] = S[m][e];
  }
  if (kind == 1) {
    // the same state as the fix-up's A fragments (outer = column, inner =
    // key channels 32p + 8g + j) in the io type, each wave its own tiles
    // (half a fragment each, as put_state packs them)
    V8* mf = (V8*)P.seg.midf + (((int64_t)seq * P.h_v + h) * NB + nb) * (KB * 64);
#pragma unroll
    for (int m = 0; m < MT; ++m) {
      const int mt = w * MT + m;
      ((V4*)&mf[(mt >> 1) * 64 + lane])[mt & 1] = pack4<ET>(S[m]);
    }
  }
}

template <int DK, int DV, bool KDA, typename ET>
hipError_t launch_scan(const ScanParams& P, int64_t nblk, bool inspect, hipStream_t st) {
  if (nblk > 0) {
    constexpr unsigned threads = ring_variant<KDA, ET>() ? 384 : 256;
    if (inspect)
      hipLaunchKernelGGL((scan_kernel<DK, DV, KDA, ET, true>), dim3((unsigned)nblk), dim3(threads), 0, st, P);
    else
      hipLaunchKernelGGL((scan_kernel<DK, DV, KDA, ET, false>), dim3((unsigned)nblk), dim3(threads), 0, st, P);
  }
  return hipGetLastError();
}

}  // namespace drla

namespace drla {
#define DRLA_SCAN_INST(DK_, DV_, KDA_, ET_) \
  template hipError_t launch_scan<DK_, DV_, KDA_, ET_>(const ScanParams&, int64_t, bool, hipStream_t);
DRLA_SCAN_INST(64, 64, false, bf16)
DRLA_SCAN_INST(128, 64, false, bf16)
DRLA_SCAN_INST(64, 128, false, bf16)
DRLA_SCAN_INST(128, 128, false, bf16)
DRLA_SCAN_INST(64, 64, true, bf16)
DRLA_SCAN_INST(128, 64, true, bf16)
DRLA_SCAN_INST(64, 128, true, bf16)
DRLA_SCAN_INST(128, 128, true, bf16)
DRLA_SCAN_INST(64, 64, true, f16)
DRLA_SCAN_INST(128, 64, true, f16)
DRLA_SCAN_INST(64, 128, true, f16)
DRLA_SCAN_INST(128, 128, true, f16)
DRLA_SCAN_INST(64, 64, false, float)
DRLA_SCAN_INST(128, 64, false, float)
DRLA_SCAN_INST(64, 128, false, float)
DRLA_SCAN_INST(128, 128, false, float)
DRLA_SCAN_INST(64, 64, true, float)
DRLA_SCAN_INST(128, 64, true, float)
DRLA_SCAN_INST(64, 128, true, float)
DRLA_SCAN_INST(128, 128, true, float)
#undef DRLA_SCAN_INST
}  // namespace drla
