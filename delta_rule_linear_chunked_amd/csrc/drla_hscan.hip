// Head-resident, segment-parallel state scan fused with the output Map
// (GDN and decay-only linear attention with a scalar gate; 16-bit inputs).
//
// Operators #5 (H) and #6 (O) of the Map-Reduce-Map split in "Empowering
// Hybrid Attention Models on NPUs", Section 2.1, organised after its
// Section 4: one workgroup holds a whole (sequence, value head) unit -- all
// dv state columns, split column-wise across its waves with no reduction
// between them ("Computation Splitting") -- and a long sequence is cut into
// segments that are scanned at once and stitched afterwards, the idea that
// section's "Chunk-Seg-Seg Mapping" applies to a head's chain.  Per chunk
// (GEMM-first, Section 5's rewriting, with Tv = diag(e^{b_n - b}) Tb and
// P Tb from the prep kernel):
//
//   R   = V - diag(e^b) K S            (decay-only: R = V)
//   V~  = Tv R                          (= diag(e^{b_n - b}) V')
//   S  <- e^{b_n} S + K^T V~
//   O   = diag(e^b) Q S_in + (P Tb) R   (S_in: the state entering the chunk)
//
// A chunk maps the state affinely, S -> M S + N.  With np segments per
// sequence three kernels run:
//
//   transition   per (unit, segment s < np - 1): the segment's map.  Half the
//                waves scan the identity with V = 0 (their final state is
//                Phi_s, the product of the segment's M), half scan from zero
//                with V (N_s); segment 0's value waves start from h0, so
//                that N_0 is already the state E_1 entering segment 1.
//   compose      per (unit, 16 columns): E_{s+1} = Phi_s E_s + N_s, s = 1 ..
//                np - 2, in place over the N sets.
//   value        per (unit, segment): the chunk recurrence from E_s (E_0 =
//                h0) with the outputs; the last segment writes ht.
//
// With np = 1 only the value kernel runs (one pass per unit).  The same chunk
// operands cross a CU's load path once per chunk for all dv columns: every
// wave copies its share of the next chunk's K and Q rows, V rows, Tv, P Tb
// and decay factors into a ring of LDS slots with LDS-direct buffer loads,
// and touches a later chunk's lines so that those copies hit L2.  One
// workgroup barrier per chunk.
#include "drla_common.h"
#include "drla_kernels.h"

namespace drla {

typedef short hs_shortx4 __attribute__((ext_vector_type(4)));

// Transposing LDS read of 16-bit elements (ds_read_b64_tr_b16): within a
// 16-lane group, lane i receives element i % 4 of the four-element segments
// addressed by lanes 4j + i / 4, j = 0..3.  `p` must be 8-byte aligned.
template <typename T>
__device__ __forceinline__ typename VT<T>::v4 hs_tr(const void* p) {
  const hs_shortx4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) hs_shortx4*)(p));
  return __builtin_bit_cast(typename VT<T>::v4, v);
}

// Byte offset of 16-byte chunk j of row r of a K or Q tile (rows of DK
// 16-bit elements): the chunk index is XORed with the row, so a fragment's
// 16 rows fall on different banks.
template <int DK>
__device__ __forceinline__ int hs_kswz(int r, int j) {
  constexpr int NCH = DK / 8;
  return r * (DK * 2) + ((j ^ (r & (NCH - 1))) << 4);
}
// The same for V rows (DV elements), XORed with twice the row: the four
// rows and two chunks that one transposing read touches land on eight
// different 16-byte positions.
template <int DV>
__device__ __forceinline__ int hs_vswz(int r, int j) {
  constexpr int NVC = DV / 8;
  return r * (DV * 2) + ((j ^ ((2 * r) & (NVC - 1))) << 4);
}

// One ring slot: a chunk's operands.  WQ: with Q rows and P Tb (value
// kernel); without them for the transition kernel.
template <int DK, int DV, typename T, bool WQ>
struct HSlot {
  typedef typename VT<T>::v8 H8;
  __attribute__((aligned(16))) unsigned char k[C * DK * 2];
  __attribute__((aligned(16))) unsigned char v[C * DV * 2];
  __attribute__((aligned(16))) unsigned char q[WQ ? C * DK * 2 : 16];
  H8 tb[6][64];            // Tv fragments (0,0)(1,0)(2,0)(2,1)(3,0)(3,1)
  H8 pm[WQ ? 6 : 1][64];   // P Tb fragments, same order
  __attribute__((aligned(16))) float eb[C];   // e^{b_r}
  __attribute__((aligned(16))) float ebn[C];  // e^{b_n - b_r}
};

// Work item of a scan workgroup: (sequence, head, segment) and the
// segment's chunks.  Dense batch: units in order; packed input: longest
// sequence first.  The np segments of a unit take consecutive indices.
struct HItem {
  int seq, h, sg;
  int64_t ts, te;  // the sequence's tokens
  int64_t c0;      // its first chunk in the chunk numbering of the workspace
  int64_t cs;      // the segment's first chunk within the sequence
  int n;           // the segment's chunks
};

__device__ __forceinline__ bool hs_item(const HScanParams& P, int nseg, HItem& it, bool pairs = false) {
  const int b = blockIdx.x;
  int r = b / nseg;
  it.sg = b - r * nseg;
  // One pass (`pairs`: the value kernel with np = 1, whose outputs are
  // indexed by unit, not by workgroup) with grouped heads: the value heads
  // of one query/key head read
  // the same K and Q rows, so they go to one XCD (workgroups are dealt to
  // the eight XCDs in turn) and share its L2: workgroup b takes member
  // (b / 8) % grp of query/key group ((b / 8) / grp) * 8 + b % 8, so each run
  // of 8 grp workgroups still covers 8 grp consecutive units (longest
  // first when packed).
  if (pairs && nseg == 1 && P.grp > 1 && (P.units / P.grp) % 8 == 0) {
    const int y = b / 8;
    r = ((y / P.grp) * 8 + b % 8) * P.grp + y % P.grp;
  }
  if (r >= P.units) return false;
  if (P.s.seq_order) {
    it.seq = P.s.seq_order[r / P.h_v];
    if (it.seq < 0 || it.seq >= P.s.n_seqs) return false;
  } else {
    it.seq = r / P.h_v;
  }
  it.h = r % P.h_v;
  int64_t nch;
  if (P.s.chunk_seq) {
    it.ts = P.s.cu[it.seq];
    it.te = P.s.cu[it.seq + 1];
    int64_t c1;
    seq_chunks(P.s, it.seq, P.nc, it.c0, c1);
    nch = it.te > it.ts ? (it.te - it.ts + C - 1) / C : 0;
    if (nch > c1 - it.c0) nch = c1 - it.c0;  // device lengths disagree with the table
  } else {
    it.ts = (int64_t)it.seq * P.s.seq_len;
    it.te = it.ts + P.s.seq_len;
    it.c0 = (int64_t)it.seq * P.s.cps;
    nch = P.s.cps;
  }
  // segment sg: chunks [sg s1, (sg + 1) s1), the last one to the end
  const int64_t s1 = nch / P.np;
  it.cs = s1 * it.sg;
  it.n = (int)(it.sg == P.np - 1 ? nch - it.cs : s1);
  return true;
}

// The chunk copies and L2 touches of one kernel.  NW waves share a
// chunk's copies (1-KiB LDS-direct loads; the decay factors as two 256-byte
// loads): every wave copies the same number of K, Q and V row blocks, and
// one or more of the fragment and decay-factor items (waves past the last
// item repeat it: the same bytes to the same place).  Likewise for the
// touches (one 4-byte load per 128-byte line, into a sink).  So every wave
// issues NCPW copies and NTPW touches per chunk and its wait counts are
// compile-time constants.
template <int DK, int DV, typename T, bool WQ, int NW>
struct HCopy {
  static constexpr int NKB = C * DK * 2 / 1024;  // 1-KiB blocks of K (and Q) rows
  static constexpr int NVB = C * DV * 2 / 1024;  // of V rows
  static_assert(NKB % NW == 0 && NVB % NW == 0, "row blocks shared evenly");
  static constexpr int KPW = NKB / NW, VPW = NVB / NW;  // blocks per wave
  static constexpr int NF = (WQ ? 12 : 6) + 2;          // fragment and decay-factor items
  static constexpr int FPW = (NF + NW - 1) / NW;
  static constexpr int NCPW = KPW * (WQ ? 2 : 1) + VPW + FPW;
  static constexpr int KL = DK * 2 / 128, VL = DV * 2 / 128;  // lines per K (Q), V row
  static constexpr int NT = KL * (WQ ? 2 : 1) + VL + (WQ ? 2 : 1) + 1;
  static constexpr int NTPW = (NT + NW - 1) / NW;
};

template <int DK, int DV, typename T, bool WQ, int NW>
struct HChunkIO {
  typedef HCopy<DK, DV, T, WQ, NW> CP;
  typedef typename VT<T>::v8 H8;
  const HScanParams* P;
  const HItem* it;
  int w, lane, hk;
  uint32_t kstride, vstride;
  uint32_t koff[CP::KPW], voff[CP::VPW];  // per-lane source offsets of this wave's row blocks

  __device__ __forceinline__ void init() {
    constexpr int NCH = DK / 8, RPI = 1024 / (DK * 2);
    constexpr int NVC = DV / 8, RPV = 1024 / (DV * 2);
#pragma unroll
    for (int m = 0; m < CP::KPW; ++m) {
      const int r = (w * CP::KPW + m) * RPI + lane / NCH;
      koff[m] = (uint32_t)r * kstride + 16u * (uint32_t)((lane % NCH) ^ (r & (NCH - 1)));
    }
#pragma unroll
    for (int m = 0; m < CP::VPW; ++m) {
      const int r = (w * CP::VPW + m) * RPV + lane / NVC;
      voff[m] = (uint32_t)r * vstride + 16u * (uint32_t)((lane % NVC) ^ ((2 * r) & (NVC - 1)));
    }
  }
  __device__ __forceinline__ uint32_t len(int i) const {
    const int64_t left = it->te - (it->ts + (int64_t)C * (it->cs + i));
    return (uint32_t)(left < C ? (left < 0 ? 0 : left) : C);
  }
  __device__ __forceinline__ int64_t tok(int i) const { return it->ts + (int64_t)C * (it->cs + i); }
  __device__ __forceinline__ int64_t chunk(int i) const { return (int64_t)it->h * P->nc + it->c0 + it->cs + i; }

  // copy chunk i of the segment into slot `sl`
  __device__ __forceinline__ void copy(int i, HSlot<DK, DV, T, WQ>& sl) const {
    const uint32_t L = len(i);
    const int64_t t0 = tok(i);
    const int64_t ch = chunk(i);
    const rsrc_t kr = make_rsrc((const T*)P->k + (t0 * P->h_qk + hk) * DK, L ? (L - 1) * kstride + DK * 2 : 0);
#pragma unroll
    for (int m = 0; m < CP::KPW; ++m) lds_dma16(kr, koff[m], 0, sl.k + (w * CP::KPW + m) * 1024);
    if constexpr (WQ) {
      const rsrc_t qr = make_rsrc((const T*)P->q + (t0 * P->h_qk + hk) * DK, L ? (L - 1) * kstride + DK * 2 : 0);
#pragma unroll
      for (int m = 0; m < CP::KPW; ++m) lds_dma16(qr, koff[m], 0, sl.q + (w * CP::KPW + m) * 1024);
    }
    const rsrc_t vr = make_rsrc((const T*)P->v + (t0 * P->h_v + it->h) * DV, L ? (L - 1) * vstride + DV * 2 : 0);
#pragma unroll
    for (int m = 0; m < CP::VPW; ++m) lds_dma16(vr, voff[m], 0, sl.v + (w * CP::VPW + m) * 1024);
    // fragment items f = w + NW m: Tv 0..5, (P Tb 6..11), then e^{b}, e^{b_n - b}
#pragma unroll
    for (int m = 0; m < CP::FPW; ++m) {
      int f = w + NW * m;
      f = f < CP::NF ? f : CP::NF - 1;
      if (f < CP::NF - 2) {
        // fragments 0, 2, 4, 5, 6, 7 of 8 (the ones below the diagonal)
        const bool pmf = f >= 6;
        const int ff = pmf ? f - 6 : f;
        const int src_f = ff == 0 ? 0 : (ff == 1 ? 2 : ff + 2);
        const rsrc_t fr = make_rsrc((const H8*)(pmf ? P->pm : P->tb) + ch * (8 * 64), 8 * 1024);
        H8* dst = pmf ? &sl.pm[WQ ? ff : 0][0] : &sl.tb[ff][0];
        lds_dma16(fr, 16u * lane + (uint32_t)src_f * 1024u, 0, dst);
      } else {
        const rsrc_t gr = make_rsrc(P->gam + ch * (2 * C), 2 * C * 4);
        const bool second = f == CP::NF - 1;
        lds_dma4(gr, 4u * lane + (second ? 4u * C : 0u), 0, second ? sl.ebn : sl.eb);
      }
    }
  }

  // touch the 128-byte lines of chunk i (L2 prefetch)
  __device__ __forceinline__ void touch(int i, float* sink) const {
    const uint32_t L = len(i);
    const int64_t t0 = tok(i);
    const int64_t ch = chunk(i);
#pragma unroll
    for (int m = 0; m < CP::NTPW; ++m) {
      int gi = w + NW * m;
      gi = gi < CP::NT ? gi : CP::NT - 1;
      if (gi < CP::KL * (WQ ? 2 : 1)) {
        const bool isq = gi >= CP::KL;
        const T* src = (const T*)(isq ? P->q : P->k) + (t0 * P->h_qk + hk) * DK;
        lds_dma4(make_rsrc(src, L ? (L - 1) * kstride + DK * 2 : 0),
                 (uint32_t)lane * kstride + 128u * (uint32_t)(isq ? gi - CP::KL : gi), 0, sink);
      } else if (gi < CP::KL * (WQ ? 2 : 1) + CP::VL) {
        const T* src = (const T*)P->v + (t0 * P->h_v + it->h) * DV;
        lds_dma4(make_rsrc(src, L ? (L - 1) * vstride + DV * 2 : 0),
                 (uint32_t)lane * vstride + 128u * (uint32_t)(gi - CP::KL * (WQ ? 2 : 1)), 0, sink);
      } else if (gi < CP::NT - 1) {
        const bool pmf = gi == CP::NT - 2 && WQ;
        lds_dma4(make_rsrc((const H8*)(pmf ? P->pm : P->tb) + ch * (8 * 64), 8 * 1024), 128u * (uint32_t)frag_line(lane),
                 0, sink);
      } else {
        lds_dma4(make_rsrc(P->gam + ch * (2 * C), 2 * C * 4), 128u * (lane & 3), 0, sink);
      }
    }
  }
};

// The chunk recurrence for CT column tiles of one wave (global column tiles
// ct0 .. ct0 + CT - 1).  State tile (ct, mt), element e of lane (g, c) is
// S[state_row(mt, 4g + e)][16 (ct0 + ct) + c]; sf holds it as 16-bit B
// fragments (inner = key channel).  DECAY: R = V.  vscale multiplies V (0
// on the transition waves, which scan V = 0).  WO: also the outputs (O^T tiles, lane (g, c) = [column 4g + e]
// [token 16 nt + c]).
// The value kernel (WQ) keeps the 16-bit fragments of the state entering
// the chunk (its output multiplies them too); the transition kernel, with
// twice the columns per wave, packs them from S when a product needs them.
template <int DK, int DV, typename T, bool WQ, int CT, bool DECAY>
struct HWave {
  typedef typename VT<T>::v8 H8;
  typedef typename VT<T>::v4 H4;
  static constexpr int KB = DK / 32, KT = DK / 16;
  floatx4 S[CT][KT];
  H8 sf[WQ ? CT : 1][WQ ? KB : 1];

  __device__ __forceinline__ void pack_state() {
    if constexpr (WQ) {
#pragma unroll
      for (int ct = 0; ct < CT; ++ct)
#pragma unroll
        for (int p = 0; p < KB; ++p) sf[ct][p] = pack<T>(S[ct][2 * p], S[ct][2 * p + 1]);
    }
  }
  __device__ __forceinline__ H8 sfrag(int ct, int p) const {
    if constexpr (WQ)
      return sf[ct][p];
    else
      return pack<T>(S[ct][2 * p], S[ct][2 * p + 1]);
  }

  // One chunk.  Returns R (as A fragments, outer = column, inner = token)
  // for the output's P Tb term when WO.
  template <bool WO>
  __device__ __forceinline__ void step(const HSlot<DK, DV, T, WQ>& sl, int ct0, int lane, floatx4 (*o)[4],
                                       float vscale) {
    const int g4 = lane >> 4, c16 = lane & 15;
    // Four phases separated by scheduling barriers (each phase's operand
    // reads are not hoisted above the previous one: register pressure); in
    // phases 3 and 4 an independent stream of products (the output's) fills
    // the matrix pipe while the chain's short dependent products wait.
    auto phase = [] { __builtin_amdgcn_sched_barrier(0); };
    // 1: X = K S, one inner block (32 key channels) at a time
    floatx4 x[CT][4];
#pragma unroll
    for (int ct = 0; ct < CT; ++ct)
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) x[ct][nt] = zero4();
    if constexpr (!DECAY) {
#pragma unroll
      for (int p = 0; p < KB; ++p) {
        H8 kr[4];
#pragma unroll
        for (int nt = 0; nt < 4; ++nt) kr[nt] = *(const H8*)(sl.k + hs_kswz<DK>(16 * nt + c16, 4 * p + g4));
#pragma unroll
        for (int ct = 0; ct < CT; ++ct) {
          const H8 sfp = sfrag(ct, p);
#pragma unroll
          for (int nt = 0; nt < 4; ++nt) x[ct][nt] = mma(kr[nt], sfp, x[ct][nt]);
        }
      }
    }
    phase();
    // 2: R = V - diag(e^b) X, as B fragments (inner = token)
    floatx4 ebv[4];
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) ebv[nt] = *(const floatx4*)&sl.eb[16 * nt + 4 * g4];
    H8 rf[CT][2];
#pragma unroll
    for (int ct = 0; ct < CT; ++ct) {
      H4 vv[4];
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) {
        const int r = 16 * nt + 4 * g4 + (c16 >> 2);
        const int col = 16 * (ct0 + ct) + 4 * (c16 & 3);
        vv[nt] = hs_tr<T>(sl.v + hs_vswz<DV>(r, col >> 3) + 2 * (col & 7));
      }
      floatx4 rr[4];
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float vf = to_f(vv[nt][e]) * vscale;
          rr[nt][e] = DECAY ? vf : vf - ebv[nt][e] * x[ct][nt][e];
        }
      }
      rf[ct][0] = pack<T>(rr[0], rr[1]);
      rf[ct][1] = pack<T>(rr[2], rr[3]);
    }
    phase();
    // 3: V~ = Tv R, and the output's state part O^T = S_in^T Q^T (S_in is
    // still in sf; the state moves on in phase 4)
    H8 tbf[6];
#pragma unroll
    for (int f = 0; f < 6; ++f) tbf[f] = sl.tb[f][lane];
    floatx4 vt[CT][4];
#pragma unroll
    for (int ct = 0; ct < CT; ++ct) {
      vt[ct][0] = mma(tbf[0], rf[ct][0], zero4());
      vt[ct][1] = mma(tbf[1], rf[ct][0], zero4());
      vt[ct][2] = mma(tbf[2], rf[ct][0], zero4());
      vt[ct][3] = mma(tbf[4], rf[ct][0], zero4());
    }
#pragma unroll
    for (int ct = 0; ct < CT; ++ct) {
      vt[ct][2] = mma(tbf[3], rf[ct][1], vt[ct][2]);
      vt[ct][3] = mma(tbf[5], rf[ct][1], vt[ct][3]);
    }
    if constexpr (WO) {
#pragma unroll
      for (int ct = 0; ct < CT; ++ct)
#pragma unroll
        for (int nt = 0; nt < 4; ++nt) o[ct][nt] = zero4();
#pragma unroll
      for (int p = 0; p < KB; ++p) {
        H8 qr[4];
#pragma unroll
        for (int nt = 0; nt < 4; ++nt) qr[nt] = *(const H8*)(sl.q + hs_kswz<DK>(16 * nt + c16, 4 * p + g4));
#pragma unroll
        for (int ct = 0; ct < CT; ++ct)
#pragma unroll
          for (int nt = 0; nt < 4; ++nt) o[ct][nt] = mma(sf[ct][p], qr[nt], o[ct][nt]);
      }
    }
    H8 vs[CT][2];
#pragma unroll
    for (int ct = 0; ct < CT; ++ct) {
      vs[ct][0] = pack<T>(vt[ct][0], vt[ct][1]);
      vs[ct][1] = pack<T>(vt[ct][2], vt[ct][3]);
    }
    phase();
    // 4: S <- e^{b_n} S + K^T V~ (K^T fragments, outer = key channel
    // state_row(mt, c), inner = token, by transposing reads of the K rows),
    // and the output's intra-chunk part (P Tb R)^T = R^T (P Tb)^T after
    // scaling the state part by e^{b} of its token
    const float gam = sl.eb[C - 1];  // e^{b_n}
#pragma unroll
    for (int ct = 0; ct < CT; ++ct)
#pragma unroll
      for (int mt = 0; mt < KT; ++mt) S[ct][mt] *= gam;
#pragma unroll
    for (int p = 0; p < 2; ++p)
#pragma unroll
      for (int mt = 0; mt < KT; ++mt) {
        H4 kt[2];
#pragma unroll
        for (int hf = 0; hf < 2; ++hf) {
          const int r0 = 32 * p + 4 * g4 + (c16 >> 2) + 16 * hf;
          const int d = state_row(mt, 4 * (c16 & 3));
          kt[hf] = hs_tr<T>(sl.k + hs_kswz<DK>(r0, d >> 3) + 2 * (d & 7));
        }
        const H8 ktf = cat<T>(kt[0], kt[1]);
#pragma unroll
        for (int ct = 0; ct < CT; ++ct) S[ct][mt] = mma(ktf, vs[ct][p], S[ct][mt]);
      }
    if constexpr (WO) {
      H8 pmf[6];
#pragma unroll
      for (int f = 0; f < 6; ++f) pmf[f] = sl.pm[WQ ? f : 0][lane];
      float ebt[4];
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) ebt[nt] = sl.eb[16 * nt + c16];
#pragma unroll
      for (int ct = 0; ct < CT; ++ct) {
#pragma unroll
        for (int nt = 0; nt < 4; ++nt) o[ct][nt] *= ebt[nt];
        o[ct][0] = mma(rf[ct][0], pmf[0], o[ct][0]);
        o[ct][1] = mma(rf[ct][0], pmf[1], o[ct][1]);
        o[ct][2] = mma(rf[ct][0], pmf[2], o[ct][2]);
        o[ct][3] = mma(rf[ct][0], pmf[4], o[ct][3]);
        o[ct][2] = mma(rf[ct][1], pmf[3], o[ct][2]);
        o[ct][3] = mma(rf[ct][1], pmf[5], o[ct][3]);
      }
    }
    pack_state();
  }
};

// Initial state of a wave's columns from a key-major [dk, dv] fp32 array
// (h0 of the unit), or zero.
template <int DK, int DV, typename T, bool WQ, int CT, bool DECAY>
__device__ __forceinline__ void hs_load_user(HWave<DK, DV, T, WQ, CT, DECAY>& W, const float* src, int ct0, int lane) {
  const int g4 = lane >> 4, c16 = lane & 15;
#pragma unroll
  for (int ct = 0; ct < CT; ++ct)
#pragma unroll
    for (int mt = 0; mt < DK / 16; ++mt)
#pragma unroll
      for (int e = 0; e < 4; ++e)
        W.S[ct][mt][e] = src[(int64_t)state_row(mt, 4 * g4 + e) * DV + 16 * (ct0 + ct) + c16];
}
template <int DK, int DV, typename T, bool WQ, int CT, bool DECAY>
__device__ __forceinline__ void hs_zero(HWave<DK, DV, T, WQ, CT, DECAY>& W) {
#pragma unroll
  for (int ct = 0; ct < CT; ++ct)
#pragma unroll
    for (int mt = 0; mt < DK / 16; ++mt) W.S[ct][mt] = zero4();
}

// State sets in the workspace are kept in tile order: per (unit), column
// tile ct (dv/16), row tile mt (dk/16), 64 lanes x 4 floats -- each lane's
// accumulator tile as one 16-byte access.
__device__ __forceinline__ int64_t hs_tile_off(int ctg, int mt, int kt, int lane) {
  return (((int64_t)ctg * kt + mt) * 64 + lane) * 4;
}

// ---- value kernel ------------------------------------------------------------
// Waves 0..3 compute, DV/4 columns each, and store O; they never wait on
// vector memory.  Waves 4, 5 copy the next chunk into the other slot of a
// two-slot ring and wait for their copies before each barrier; wave 6 only
// touches the lines of chunk t + PF, so that those copies hit L2.  Every
// wave keeps its own vector-memory counter, so a copy never waits behind a
// touch that misses L2 or behind a store.
template <int DK, int DV, typename T, bool DECAY>
__global__ __launch_bounds__(448) void hscan_value_kernel(HScanParams P) {
  constexpr int NCW = 4, CT = DV / 64, NS = 2, PF = 4, KT = DK / 16;
  typedef HCopy<DK, DV, T, true, 1> TP;   // one touch wave
  __shared__ HSlot<DK, DV, T, true> slot[NS];
  __shared__ __attribute__((aligned(16))) float sink[64];

  HItem it;
  if (!hs_item(P, P.np, it, P.np == 1)) return;  // the whole workgroup: past the last unit
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g4 = lane >> 4, c16 = lane & 15;
  const int n = __builtin_amdgcn_readfirstlane(it.n);
  const int64_t unit = (int64_t)it.seq * P.h_v + it.h;

  if (w >= NCW) {
    // ---- copy waves (4, 5) and the touch wave (6)
    if (w < NCW + 2) {
      HChunkIO<DK, DV, T, true, 2> io;
      io.P = &P;
      io.it = &it;
      io.w = w - NCW;
      io.lane = lane;
      io.hk = it.h / P.grp;
      io.kstride = (uint32_t)P.h_qk * DK * 2;
      io.vstride = (uint32_t)P.h_v * DV * 2;
      io.init();
      if (n > 0) io.copy(0, slot[0]);
      __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
      lds_barrier();
      for (int t = 0; t < n; ++t) {
        io.copy(t + 1 < n ? t + 1 : n - 1, slot[(t + 1) % NS]);
        __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));  // chunk t + 1 has landed
        lds_barrier();
      }
    } else {
      HChunkIO<DK, DV, T, true, 1> io;
      io.P = &P;
      io.it = &it;
      io.w = 0;
      io.lane = lane;
      io.hk = it.h / P.grp;
      io.kstride = (uint32_t)P.h_qk * DK * 2;
      io.vstride = (uint32_t)P.h_v * DV * 2;
      if (n > 0) {
#pragma unroll
        for (int i = 1; i < PF; ++i) io.touch(i < n ? i : n - 1, sink);
      }
      lds_barrier();
      for (int t = 0; t < n; ++t) {
        // at most about three chunks of touches in flight
        __builtin_amdgcn_s_waitcnt(vmcnt_imm(2 * TP::NTPW));
        io.touch(t + PF < n ? t + PF : n - 1, sink);
        lds_barrier();
      }
    }
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
    return;
  }

  // ---- compute waves
  const int ct0 = CT * w;
  HWave<DK, DV, T, true, CT, DECAY> W;
  if (it.sg == 0) {
    if (P.h0)
      hs_load_user(W, P.h0 + unit * DK * DV, ct0, lane);
    else
      hs_zero(W);
  } else {
    const float* e = P.en + ((int64_t)(it.sg - 1) * P.units + blockIdx.x / P.np) * DK * DV;
#pragma unroll
    for (int ct = 0; ct < CT; ++ct)
#pragma unroll
      for (int mt = 0; mt < KT; ++mt) W.S[ct][mt] = *(const floatx4*)(e + hs_tile_off(ct0 + ct, mt, KT, lane));
  }
  W.pack_state();
  lds_barrier();  // chunk 0 has landed

  const uint32_t orow = (uint32_t)(((size_t)c16 * P.h_v + it.h) * DV + 16 * ct0 + 4 * g4) * 2;
  const uint32_t ostep = (uint32_t)(16 * P.h_v * DV * 2);  // 16 tokens
  const uint32_t tstride = (uint32_t)(P.h_v * DV * 2);     // bytes per token of o
  floatx4 o[CT][4];
  for (int t = 0; t < n; ++t) {
    W.template step<true>(slot[t % NS], ct0, lane, o, 1.f);
    lds_barrier();  // slot t % NS free; chunk t + 1 has landed
    // store O (rows past the end of the sequence are dropped)
    const int64_t left = it.te - (it.ts + (int64_t)C * (it.cs + t));
    const uint32_t len = (uint32_t)(left < C ? left : C);
    const rsrc_t orr = make_rsrc((T*)P.o + (it.ts + (int64_t)C * (it.cs + t)) * P.h_v * DV, len * tstride);
#pragma unroll
    for (int ct = 0; ct < CT; ++ct)
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) bstore(orr, orow + nt * ostep + 32u * ct, pack4<T>(o[ct][nt]));
  }
  if (it.sg == P.np - 1 && P.ht) {
    float* dst = P.ht + unit * DK * DV;
#pragma unroll
    for (int ct = 0; ct < CT; ++ct)
#pragma unroll
      for (int mt = 0; mt < KT; ++mt)
#pragma unroll
        for (int e = 0; e < 4; ++e) dst[(int64_t)state_row(mt, 4 * g4 + e) * DV + 16 * (ct0 + ct) + c16] = W.S[ct][mt][e];
  }
}

// ---- transition kernel ---------------------------------------------------------
// Segment s < np - 1 of a unit: waves 0..3 scan the identity with V = 0
// (Phi_s), waves 4..7 scan from zero with V (N_s; from h0 for s = 0, which
// then gives E_1), dk/4 columns each; two waves share each SIMD, so one
// wave's products fill the matrix pipe while the other waits on LDS or on a
// dependent product.  dk = dv; a three-slot ring.
template <int DK, typename T, bool DECAY>
__global__ __launch_bounds__(512) void hscan_trans_kernel(HScanParams P) {
  constexpr int DV = DK, NW = 8, CT = DK / 64, NS = 3, KT = DK / 16, KB = DK / 32;
  typedef HCopy<DK, DV, T, false, NW> CP;
  typedef typename VT<T>::v8 H8;
  typedef typename VT<T>::v4 H4;
  __shared__ HSlot<DK, DV, T, false> slot[NS];
  static_assert(sizeof(HSlot<DK, DV, T, false>) * NS >= DK * DK * 2, "Phi transpose fits in the ring");

  HItem it;
  if (!hs_item(P, P.np - 1, it)) return;
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g4 = lane >> 4, c16 = lane & 15;
  const int n = __builtin_amdgcn_readfirstlane(it.n);
  const int64_t unit = (int64_t)it.seq * P.h_v + it.h;
  const int64_t urank = blockIdx.x / (P.np - 1);
  const bool phi = w < 4;               // transition waves
  const bool idle = phi && it.sg == 0;  // segment 0 needs no map
  const int ct0 = CT * (w & 3);

  HChunkIO<DK, DV, T, false, NW> io;
  io.P = &P;
  io.it = &it;
  io.w = w;
  io.lane = lane;
  io.hk = it.h / P.grp;
  io.kstride = (uint32_t)P.h_qk * DK * 2;
  io.vstride = (uint32_t)P.h_v * DV * 2;
  io.init();

  HWave<DK, DV, T, false, CT, DECAY> W;
  if (phi) {
#pragma unroll
    for (int ct = 0; ct < CT; ++ct)
#pragma unroll
      for (int mt = 0; mt < KT; ++mt)
#pragma unroll
        for (int e = 0; e < 4; ++e) W.S[ct][mt][e] = state_row(mt, 4 * g4 + e) == 16 * (ct0 + ct) + c16 ? 1.f : 0.f;
  } else {
    if (it.sg == 0 && P.h0)
      hs_load_user(W, P.h0 + unit * DK * DV, ct0, lane);
    else
      hs_zero(W);
  }
  W.pack_state();

  // The copies run two chunks ahead (the workgroups of this kernel read
  // the chunks once each; no L2 touches: a touch that misses would hold up
  // the copies issued after it on this wave's in-order counter).
  if (n > 0) {
    io.copy(0, slot[0]);
    io.copy(n > 1 ? 1 : 0, slot[1]);
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(CP::NCPW));  // chunk 0 has landed
  }
  lds_barrier();
  for (int t = 0; t < n; ++t) {
    io.copy(t + 2 < n ? t + 2 : n - 1, slot[(t + 2) % NS]);
    if (!idle) W.template step<false>(slot[t % NS], ct0, lane, nullptr, phi ? 0.f : 1.f);
    // chunk t + 1 has landed once at most chunk t + 2's copies are pending
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(CP::NCPW));
    lds_barrier();
  }
  __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
  lds_barrier();  // every wave is done with the ring

  // Value waves: N_s (E_1 for segment 0) in tile order.  Transition waves:
  // Phi as A fragments for the compose kernel (outer = row key channel
  // state_row(mt, c), inner = column key channel 32p + 8g + j), through LDS:
  // stored transposed (row j = column j of Phi, contiguous rows of Phi),
  // then read back with transposing reads.  All eight waves pass the barrier
  // between the two steps.
  unsigned char* M = (unsigned char*)&slot[0];
  if (!phi) {
    float* e = P.en + ((int64_t)it.sg * P.units + urank) * DK * DV;
#pragma unroll
    for (int ct = 0; ct < CT; ++ct)
#pragma unroll
      for (int mt = 0; mt < KT; ++mt) *(floatx4*)(e + hs_tile_off(ct0 + ct, mt, KT, lane)) = W.S[ct][mt];
  } else if (!idle) {
#pragma unroll
    for (int ct = 0; ct < CT; ++ct)
#pragma unroll
      for (int mt = 0; mt < KT; ++mt) {
        const int j = 16 * (ct0 + ct) + c16;
        const int i0 = state_row(mt, 4 * g4);
        *(H4*)(M + hs_kswz<DK>(j, i0 >> 3) + 2 * (i0 & 7)) = pack4<T>(W.S[ct][mt]);
      }
  }
  lds_barrier();
  if (phi && !idle) {
    H8* dst = (H8*)P.phi + ((int64_t)(it.sg - 1) * P.units + urank) * (KT * KB * 64);
    for (int f = w; f < KT * KB; f += 2) {
      const int mt = f / KB, p = f - mt * KB;
      H4 hv[2];
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
        const int jr = 32 * p + 8 * g4 + 4 * hf + (c16 >> 2);
        const int i0 = 32 * (mt >> 1) + 8 * (c16 & 3) + 4 * (mt & 1);
        hv[hf] = hs_tr<T>(M + hs_kswz<DK>(jr, i0 >> 3) + 2 * (i0 & 7));
      }
      dst[f * 64 + lane] = cat<T>(hv[0], hv[1]);
    }
  }
}

// ---- compose kernel ------------------------------------------------------------
// One workgroup per (unit, 16 state columns): E_{s+1} = Phi_s E_s + N_s for
// s = 1 .. np - 2, over the N sets in place (set 0 holds E_1).  Waves 0..3
// each own two row tiles of E (rows of Phi) and copy their rows of Phi_s and
// their tiles of N_s three steps ahead into a private three-slot LDS ring;
// per step they multiply, publish their part of E_{s+1} as a 16-bit
// fragment (the next step's B operand) and as fp32 tiles, and pass one
// barrier.  Wave 4 stores the fp32 tiles to the workspace one step later
// and touches Phi a few steps ahead of the copies.  Only the copy waves
// wait on their vector-memory counter.
template <int DK, typename T>
struct HCompLds {
  typedef typename VT<T>::v8 H8;
  static constexpr int KB = DK / 32;
  struct Ring {
    H8 phi[2][KB][64];   // rows 2w, 2w + 1 of Phi (A fragments)
    floatx4 nt[2][64];   // N tiles of those rows
  };
  Ring ring[3][4];       // [slot][wave]
  H8 ef[2][4][64];       // E as B fragments (fragment p from wave p), two steps
  floatx4 out[2][DK / 16][64];  // fp32 E tiles for the store wave, two steps
};

template <int DK, typename T>
__global__ __launch_bounds__(320) void hscan_compose_kernel(HScanParams P) {
  constexpr int KT = DK / 16, KB = DK / 32, DV = DK, PF = 6;
  typedef typename VT<T>::v8 H8;
  static_assert(KT == 8 || KT == 4, "dk 64 or 128");
  __shared__ HCompLds<DK, T> L;
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int nbk = DV / 16;
  const int urank = blockIdx.x / nbk, ctg = blockIdx.x - urank * nbk;
  if (urank >= P.units) return;
  const int64_t us = (int64_t)P.units * DK * DV;
  const int64_t ps = (int64_t)P.units * (KT * KB * 64);  // fragments per Phi set
  float* const e0 = P.en + (int64_t)urank * DK * DV;
  const int last = P.np - 2;  // steps s = 1 .. last
  // A sequence of fewer chunks than segments has only its last segment
  // non-empty: the state entering it is E_1 (its initial state) itself,
  // copied in fp32 (no product with the identity maps).
  int64_t nch;
  if (P.s.seq_order) {
    const int seq = P.s.seq_order[urank / P.h_v];
    const int64_t L = seq >= 0 && seq < P.s.n_seqs ? (int64_t)P.s.cu[seq + 1] - P.s.cu[seq] : 0;
    nch = L > 0 ? (L + C - 1) / C : 0;
  } else {
    nch = P.s.cps;
  }
  if (nch / P.np == 0) {
    if (w == 0) {
#pragma unroll
      for (int mt = 0; mt < KT; ++mt) {
        const floatx4 e = *(const floatx4*)(e0 + hs_tile_off(ctg, mt, KT, lane));
        for (int s = 1; s <= last; ++s) *(floatx4*)(e0 + s * us + hs_tile_off(ctg, mt, KT, lane)) = e;
      }
    }
    return;
  }
  constexpr int MPW = KT / 4;  // row tiles per compute wave (2 at dk 128, 1 at 64)

  if (w < 4) {
    // copies of step s (1 <= s <= last) into ring slot s % 3
    const H8* phi = (const H8*)P.phi + (int64_t)urank * (KT * KB * 64);
    auto copy = [&](int s) {
      typename HCompLds<DK, T>::Ring& r = L.ring[s % 3][w];
      const rsrc_t pr = make_rsrc(phi + (int64_t)(s - 1) * ps, KT * KB * 64 * 16);
      const rsrc_t nr = make_rsrc(e0 + s * us, DK * DV * 4);
#pragma unroll
      for (int m = 0; m < MPW; ++m) {
        const int mt = MPW * w + m;
#pragma unroll
        for (int p = 0; p < KB; ++p) lds_dma16(pr, (uint32_t)(((mt * KB + p) * 64 + lane) * 16), 0, &r.phi[m][p][0]);
        lds_dma16(nr, (uint32_t)(hs_tile_off(ctg, mt, KT, lane) * 4), 0, &r.nt[m][0]);
      }
    };
    constexpr int NCP = MPW * (KB + 1);  // copies per step
    // E_1 (set 0) in registers, published as fragment w
    floatx4 E[MPW];
#pragma unroll
    for (int m = 0; m < MPW; ++m) E[m] = *(const floatx4*)(e0 + hs_tile_off(ctg, MPW * w + m, KT, lane));
    if (KT == 8) {
      L.ef[0][w][lane] = pack<T>(E[0], E[MPW - 1]);
    } else {
      // dk 64: wave w holds one row tile; fragment p = (tiles 2p, 2p+1) is
      // assembled from two waves through the fp32 tiles
      L.out[0][w][lane] = E[0];
    }
    for (int s = 1; s <= last && s <= 3; ++s) copy(s);
    lds_barrier();
    if (KT == 4 && w < 2) L.ef[0][w][lane] = pack<T>(L.out[0][2 * w][lane], L.out[0][2 * w + 1][lane]);
    if (KT == 4) lds_barrier();
    for (int s = 1; s <= last; ++s) {
      // step s's copies have landed once at most those of s + 1, s + 2 are pending
      const int ahead = (last - s) < 2 ? (last - s) : 2;
      if (ahead == 2)
        __builtin_amdgcn_s_waitcnt(vmcnt_imm(2 * NCP));
      else if (ahead == 1)
        __builtin_amdgcn_s_waitcnt(vmcnt_imm(NCP));
      else
        __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
      const typename HCompLds<DK, T>::Ring& r = L.ring[s % 3][w];
      H8 ef[KB];
#pragma unroll
      for (int p = 0; p < KB; ++p) ef[p] = L.ef[(s - 1) & 1][p][lane];
      floatx4 X[MPW];
#pragma unroll
      for (int m = 0; m < MPW; ++m) {
        X[m] = r.nt[m][lane];
#pragma unroll
        for (int p = 0; p < KB; ++p) X[m] = mma(r.phi[m][p][lane], ef[p], X[m]);
      }
#pragma unroll
      for (int m = 0; m < MPW; ++m) L.out[s & 1][MPW * w + m][lane] = X[m];
      if (KT == 8) L.ef[s & 1][w][lane] = pack<T>(X[0], X[MPW - 1]);
      lds_barrier();  // E_{s+1} published; ring slot s % 3 free
      if (KT == 4) {
        if (w < 2) L.ef[s & 1][w][lane] = pack<T>(L.out[s & 1][2 * w][lane], L.out[s & 1][2 * w + 1][lane]);
        lds_barrier();
      }
      if (s + 3 <= last) copy(s + 3);
    }
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
  } else {
    // store wave: E_{s+1} into set s, one step behind; touches of Phi
    const char* phib = (const char*)P.phi + (int64_t)urank * (KT * KB * 64 * 16);
    __shared__ __attribute__((aligned(16))) float sink[64];
    auto touch = [&](int s) {
      if (s > last) return;
      const rsrc_t pr = make_rsrc(phib + (int64_t)(s - 1) * ps * 16, KT * KB * 64 * 16);
      // 32 KiB (dk 128): 256 lines, 64 per load
#pragma unroll
      for (int j = 0; j < KT * KB * 64 * 16 / 8192; ++j) lds_dma4(pr, (uint32_t)(j * 8192 + lane * 128), 0, sink);
    };
    for (int s = 4; s < 4 + PF; ++s) touch(s);
    lds_barrier();
    if (KT == 4) lds_barrier();
    for (int s = 1; s <= last; ++s) {
      __builtin_amdgcn_s_waitcnt(vmcnt_imm(40));
      touch(s + 3 + PF);
      lds_barrier();
      if (KT == 4) lds_barrier();
      float* es = e0 + s * us;
#pragma unroll
      for (int mt = 0; mt < KT; ++mt) *(floatx4*)(es + hs_tile_off(ctg, mt, KT, lane)) = L.out[s & 1][mt][lane];
    }
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
  }
}

// ---- launchers -------------------------------------------------------------------

template <int DK, int DV, typename T>
hipError_t launch_hscan(const HScanParams& P, hipStream_t st) {
  if (P.units <= 0) return hipGetLastError();
  if constexpr (DK == DV) {
    if (P.np > 1) {
      const dim3 g1((unsigned)(P.units * (P.np - 1)));
      if (P.decay_only)
        hipLaunchKernelGGL((hscan_trans_kernel<DK, T, true>), g1, dim3(512), 0, st, P);
      else
        hipLaunchKernelGGL((hscan_trans_kernel<DK, T, false>), g1, dim3(512), 0, st, P);
      hipError_t e = hipGetLastError();
      if (e != hipSuccess) return e;
      if (P.np > 2) {
        hipLaunchKernelGGL((hscan_compose_kernel<DK, T>), dim3((unsigned)(P.units * (DV / 16))), dim3(320), 0, st, P);
        e = hipGetLastError();
        if (e != hipSuccess) return e;
      }
    }
  }
  const dim3 g3((unsigned)(P.units * P.np));
  if (P.decay_only)
    hipLaunchKernelGGL((hscan_value_kernel<DK, DV, T, true>), g3, dim3(448), 0, st, P);
  else
    hipLaunchKernelGGL((hscan_value_kernel<DK, DV, T, false>), g3, dim3(448), 0, st, P);
  return hipGetLastError();
}

#define DRLA_HSCAN_INST(DK_, DV_, T_) template hipError_t launch_hscan<DK_, DV_, T_>(const HScanParams&, hipStream_t);
DRLA_HSCAN_INST(64, 64, bf16)
DRLA_HSCAN_INST(128, 64, bf16)
DRLA_HSCAN_INST(64, 128, bf16)
DRLA_HSCAN_INST(128, 128, bf16)
DRLA_HSCAN_INST(64, 64, f16)
DRLA_HSCAN_INST(128, 64, f16)
DRLA_HSCAN_INST(64, 128, f16)
DRLA_HSCAN_INST(128, 128, f16)
#undef DRLA_HSCAN_INST

}  // namespace drla
