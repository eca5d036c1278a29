// Sequential state scan fused with the output Map, LDS-fed (GDN, 16-bit
// inputs: bf16 or fp16).
//
// Same computation as drla_scan.hip -- operators #5 (H) and #6 (O) of the
// Map-Reduce-Map split in "Empowering Hybrid Attention Models on NPUs",
// Section 2.1, in the chunk-first order of its Section 5 -- organised so
// that every byte a workgroup needs crosses the CU's load path once:
//
//   wave 0    (state)   the state recurrence of the chunk, with the 16 state
//                       columns in registers:
//                         R   = V - diag(e^b) K S
//                         V~  = Tv R        = diag(e^{b_n - b}) V'
//                         S  <- e^{b_n} S + K^T V~
//                       where Tv = diag(e^{b_n - b}) Tb and V' = Tb R
//   waves 1,2 (loaders) copy the operands of chunk t+2 (K and Q rows, Tv,
//                       P Tb, this block's 16 columns of V, the decay factors)
//                       into a three-slot LDS ring with LDS-direct loads;
//                       wave 1 also touches this block's share of chunk
//                       t+PF so that it sits in L2 when its copy is issued
//   wave 3    (output)  O = diag(e^b) Q S + (P Tb) R for the chunk (= P V'),
//                       and its store
//
// K^T is never stored: the state wave reads K rows from LDS with the
// transposing ds_read_b64_tr_b16 (within a 16-lane group, lane i receives
// element i%4 of the four-element segments addressed by lanes 4j + i/4,
// j = 0..3).  One workgroup barrier per chunk (next state and R published,
// ring slot released, next chunk's operands landed); the output wave adds
// the (P Tb) R term of a chunk one chunk later, keeping P Tb in registers.
// Folding the row decay into Tv and Tb into P removes the decay factors of
// V' and the scaling of V' from the state wave's serial chain; all three
// factors have entries of magnitude at most those of Tb and P.
//
// KDA (per-channel gate, 16-bit inputs) runs the same kernel on prep's
// operands: the ring holds K e^{B} and K~^T = (K (.) e^{B_n - B})^T as MFMA
// fragments (so the state wave's K^T reads are plain 16-byte reads), Tb, P,
// V and e^{B_n} per key channel; the state wave forms R = V - (K e^B) S,
// V' = Tb R and S <- Diag(e^{B_n}) S + K~^T V' and hands V' to the output
// wave, which forms O = (Q e^B) S + P V' with its Q e^B fragments loaded
// into registers one chunk ahead (they do not fit the ring).
//
// Segment mode with paired chains (GDN; SegParams::pair): a later segment's
// workgroup scans it both from a zero state (waves 0 and 3, as above) and
// from the identity with V = 0, the transition, on a fifth wave that also
// forms the transition's outputs G = diag(e^b) Q M + (P Tb) R from its own
// registers (there is no LDS left for a second state and R exchange), so
// both chains share one copy of the chunk operands and a unit's segments
// take np workgroups per column block instead of 2 np - 1.
//
// Only the loader waves issue loads into LDS, so their wait counts are
// exact: every chunk each issues exactly kIssued copies, and wave 1
// kTouched touches.
#include "drla_common.h"
#include "drla_kernels.h"

namespace drla {

typedef short shortx4 __attribute__((ext_vector_type(4)));

// Transposing LDS read (see above) of 16-bit elements of type T; `p` must
// be 8-byte aligned.
template <typename T>
__device__ __forceinline__ typename VT<T>::v4 ds_read_tr(const void* p) {
  const shortx4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) shortx4*)(p));
  return __builtin_bit_cast(typename VT<T>::v4, v);
}


template <int DK, typename T>
struct LdsSlot {
  typedef typename VT<T>::v8 H8;
  static constexpr int RB = DK * 2;                       // bytes per K/Q row
  __attribute__((aligned(16))) unsigned char k[C * RB];  // K rows, 16-byte chunks swizzled (KDA: K e^B fragments)
  __attribute__((aligned(16))) unsigned char q[C * RB];  // Q rows, same (KDA: K~^T fragments)
  H8 tb[6][64];                                       // Tv fragments (0,0)(1,0)(2,0)(2,1)(3,0)(3,1) (KDA: Tb)
  H8 pm[6][64];                                       // P Tb fragments, same order (KDA: P)
  __attribute__((aligned(16))) T v[C][16];             // V, this block's 16 columns
  __attribute__((aligned(16))) float dec[2 * C];          // e^{b_r}, then e^{b_n - b_r} (KDA: e^{B_n} per key channel)
};

// Byte offset of 16-byte chunk j of row r in a swizzled K/Q tile (the chunk
// index is XORed with the row so that a fragment's 16 rows hit 16 banks).
template <int DK>
__device__ __forceinline__ int swz(int r, int j) {
  constexpr int NCH = DK / 8;
  return r * (DK * 2) + ((j ^ (r & (NCH - 1))) << 4);
}

// DECAY: decay-only linear attention (no delta rule): R = V, so the state
// wave reads no K rows and runs no X products.  KDA: the per-channel gate.
// PAIR: segment mode with paired chains (five waves).
template <int DK, int DV, bool INSPECT, typename T, bool DECAY, bool KDA, bool PAIR = false>
__global__ __launch_bounds__(PAIR ? 320 : 256) void scan_lds_kernel(ScanParams P) {
  typedef typename VT<T>::v8 H8;
  typedef typename VT<T>::v4 H4;
  constexpr int KB = DK / 32, KT = DK / 16, NB = DV / 16;
  constexpr int NS = 3;                       // ring slots
  constexpr int PF = 6;                       // L2 touch distance, chunks
  constexpr int NCH = DK / 8;                 // 16-byte chunks per row
  constexpr int RPI = 1024 / (DK * 2);        // rows per 1 KiB copy
  constexpr int kIssued = C / RPI + 6 + 2;    // copies per loader wave and chunk
  static_assert(!KDA || DK <= 2 * C, "KDA: e^{B_n} fits the slot's two decay rows");
  // L2 touches: line groups of a chunk (see touch_group), NTC touch loads
  // per column block and chunk, issued by loader wave 1
  constexpr int KL = DK * 2 / 128, VL = DV * 2 / 128;  // lines per K/Q row, per V row
  constexpr int FL = (DK * C * 2 / 128 + 63) / 64;     // KDA: groups per 16-bit fragment array
  constexpr int NG = KDA ? 3 * FL + 2 + VL + 1 : 2 * KL + 2 + VL + 1;
  constexpr int NTC = (NG + NB - 1) / NB;
  constexpr int kTouched = NTC;               // touches per chunk (loader wave 1)
  __shared__ LdsSlot<DK, T> slot[NS];
  __shared__ H8 sbuf[2][KB][64];  // state entering a chunk, B fragments (inner = key channel)
  __shared__ H8 vbuf[2][2][64];   // R (KDA: V') of the last two chunks, A fragments (inner = token)
  __shared__ __attribute__((aligned(16))) float touch[64];  // sink of the L2 touches, never read

  static_assert(!PAIR || (!KDA && !INSPECT && DK == DV), "paired chains: GDN segment mode");
  const int tid = threadIdx.x, lane = tid & 63;
  // w: the wave's role -- 0 state, 1 and 2 loaders, 3 output, 4 (PAIR) the
  // transition chain.  With PAIR the hardware waves 0..4 take the roles 0,
  // 4, 3, 1, 2, so that the two chains' waves sit on different SIMDs
  // (wave i on SIMD i % 4) and the busy SIMD 0 shares with a loader.
  const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int w = PAIR ? (wid == 0 ? 0 : wid == 1 ? 4 : wid == 2 ? 3 : wid - 2) : wid;
  const int g4 = lane >> 4, c16 = lane & 15;
  int seq, h, nb;
  int kind = 0, sg = 0;  // 0: whole sequence; segment mode: 1 .. 4 and the segment (seg_item)
  if (P.seg.s1 > 0) {
    int unit;
    seg_item(P.s.n_seqs * P.h_v, NB, P.seg.np, PAIR, unit, nb, kind, sg);
    seq = unit / P.h_v;
    h = unit - seq * P.h_v;
  } else if (!scan_item(P.s, P.h_v, NB, seq, h, nb)) {
    return;  // the whole workgroup: past the last unit
  }
  const int hk = h / P.grp;

  int64_t ts, te, c0, nch;
  if (P.s.chunk_seq) {
    ts = P.s.cu[seq];
    te = P.s.cu[seq + 1];
    int64_t c1;
    seq_chunks(P.s, seq, P.nc, c0, c1);
    nch = te > ts ? (te - ts + C - 1) / C : 0;
    if (nch > c1 - c0) nch = c1 - c0;  // device lengths disagree with the table
  } else {
    ts = (int64_t)seq * P.s.seq_len;
    te = ts + P.s.seq_len;
    c0 = (int64_t)seq * P.s.cps;
    nch = P.s.cps;
  }
  if (kind > 0) {
    // segment sg of this sequence (seg_span)
    int64_t first, len;
    seg_span(nch, P.seg.np, P.seg.w0, sg, first, len);
    ts += (int64_t)C * first;
    c0 += first;
    nch = len;
  }
  const int n = __builtin_amdgcn_readfirstlane((int)nch);
  // the chain this wave scans: kind 4 is kind 2 on the state and output
  // waves and kind 3 on the transition wave
  const int ck = kind == 4 ? (w == 4 ? 3 : 2) : kind;
  T* const obase = (T*)(ck == 3 ? P.seg.g : P.o);
  float* const sout = ck == 0   ? P.ht
                      : ck == 1 ? P.seg.mid
                                : (ck == 2 ? P.seg.n : P.seg.m) + (int64_t)(sg - 1) * P.seg.us;
  const int64_t sbase = ((int64_t)seq * P.h_v + h) * DK * DV;
  const int col = 16 * nb + c16;
  const T* kg = (const T*)P.k;
  const T* qg = (const T*)P.q;
  const T* vg = (const T*)P.v;

  // ---- loaders: copy chunk i into ring slot i % NS ------------------------
  // wave 1: K rows, Tb, decay factors; wave 2: Q rows, P, V.  Each copy goes
  // through a buffer descriptor that starts at the chunk and ends at its last
  // valid token, so rows past the end of a short chunk read zero (their Tb
  // rows and columns are zero as well: beta = 0 there).  The per-lane byte
  // offsets are the same for every chunk.
  constexpr int NP = NCH > RPI ? NCH / RPI : 1;  // swizzle patterns of the row copies
  const uint32_t kstride = (uint32_t)P.h_qk * DK * 2;  // bytes between tokens of q, k
  const uint32_t vstride = (uint32_t)P.h_v * DV * 2;   // bytes between tokens of v
  uint32_t roff[NP];
#pragma unroll
  for (int v = 0; v < NP; ++v) {
    const int r = v * RPI + lane / NCH;
    roff[v] = (uint32_t)r * kstride + 16u * (uint32_t)((lane % NCH) ^ (r & (NCH - 1)));
  }
  const uint32_t voff = (uint32_t)(lane >> 1) * vstride + 16u * (uint32_t)(lane & 1);
  auto chunk_len = [&](int i) -> uint32_t {
    const int64_t left = te - (ts + (int64_t)C * i);
    return (uint32_t)(left < C ? left : C);
  };
  auto row_rsrc = [&](int i) -> rsrc_t {
    const T* src = (w == 1 ? kg : qg) + ((ts + (int64_t)C * i) * P.h_qk + hk) * DK;
    return make_rsrc(src, (chunk_len(i) - 1) * kstride + DK * 2);
  };
  auto v_rsrc = [&](int i) -> rsrc_t {
    const T* src = vg + ((ts + (int64_t)C * i) * P.h_v + h) * DV + 16 * nb;
    // segment 1 transition blocks scan V = 0 from the identity: an empty
    // range makes every V copy write zeros
    return make_rsrc(src, kind == 3 ? 0u : (chunk_len(i) - 1) * vstride + 32);
  };
  auto frag_rsrc = [&](int i) -> rsrc_t {
    const int64_t ch = (int64_t)h * P.nc + c0 + i;
    return make_rsrc((const H8*)(w == 1 ? P.tb : P.pm) + ch * (8 * 64), 8 * 1024);
  };
  auto gam_rsrc = [&](int i) -> rsrc_t {
    const int64_t ch = (int64_t)h * P.nc + c0 + i;
    // KDA: e^{B_n} per key channel; else e^{b_r}, then e^{b_n - b_r}
    return KDA ? make_rsrc(P.gam + ch * DK, DK * 4) : make_rsrc(P.gam + ch * (2 * C), 2 * C * 4);
  };
  // KDA: the chunk's K e^B (wave 1) or K~^T (wave 2) fragments, or Q e^B
  auto kda_rsrc = [&](const void* base, int i) -> rsrc_t {
    const int64_t ch = (int64_t)h * P.nc + c0 + i;
    return make_rsrc((const H8*)base + ch * (C * DK / 8), C * DK * 2);
  };
  auto issue = [&](int i) {
    LdsSlot<DK, T>& sl = slot[i % NS];
    unsigned char* dst = w == 1 ? sl.k : sl.q;
    if constexpr (KDA) {
      const rsrc_t fa = kda_rsrc(w == 1 ? P.kw : P.kt, i);
#pragma unroll
      for (int u = 0; u < C / RPI; ++u) lds_dma16(fa, 16u * lane + u * 1024, 0, dst + u * 1024);
    } else {
      const rsrc_t rr = row_rsrc(i);
#pragma unroll
      for (int u = 0; u < C / RPI; ++u)
        lds_dma16(rr, roff[u % NP] + (uint32_t)(u / NP) * (NP * RPI) * kstride, 0, dst + u * 1024);
    }
    const rsrc_t fr = frag_rsrc(i);
    H8(*fdst)[64] = w == 1 ? sl.tb : sl.pm;
    const uint32_t lo = 16u * lane;
    lds_dma16(fr, lo + 0 * 1024, 0, &fdst[0][0]);
    lds_dma16(fr, lo + 2 * 1024, 0, &fdst[1][0]);
    lds_dma16(fr, lo + 4 * 1024, 0, &fdst[2][0]);
    lds_dma16(fr, lo + 5 * 1024, 0, &fdst[3][0]);
    lds_dma16(fr, lo + 6 * 1024, 0, &fdst[4][0]);
    lds_dma16(fr, lo + 7 * 1024, 0, &fdst[5][0]);
    if (w == 1) {
      const rsrc_t gr = gam_rsrc(i);
      lds_dma4(gr, 4u * lane, 0, sl.dec);
      lds_dma4(gr, 4u * lane + 4 * C, 0, sl.dec + C);
    } else {
      const rsrc_t vr = v_rsrc(i);
      lds_dma16(vr, voff, 0, &sl.v[0][0]);
      lds_dma16(vr, voff + 32 * vstride, 0, &sl.v[32][0]);
    }
  };
  // L2 touches: the eight (four) column blocks of a head share their
  // XCD's L2, so each touches its own share of a chunk's 128-byte lines --
  // K rows, Q rows, Tb, P, the head's V rows, the decay factors (KDA: the
  // K e^B, K~^T and Q e^B fragments in place of the rows) -- NTC touch
  // loads per chunk, issued by loader wave 1 only.
  auto touch_group = [&](int gi, int i) {
    const int64_t tc = ts + (int64_t)C * i;
    const uint32_t lrow = (chunk_len(i) - 1);
    if (KDA && gi < 3 * FL) {  // K e^B, K~^T or Q e^B fragments, lines 64 (gi % FL) ..
      const void* base = gi < FL ? P.kw : gi < 2 * FL ? P.kt : P.qw;
      lds_dma4(kda_rsrc(base, i), 128u * (uint32_t)(lane + 64 * (gi % FL)), 0, touch);
      return;
    }
    if (KDA) gi += 2 * KL - 3 * FL;  // the groups below, past the rows
    if (gi < 2 * KL) {  // K or Q rows, line gi % KL
      const T* src = (gi < KL ? kg : qg) + (tc * P.h_qk + hk) * DK;
      lds_dma4(make_rsrc(src, lrow * kstride + DK * 2), (uint32_t)lane * kstride + 128u * (uint32_t)(gi % KL), 0, touch);
    } else if (gi < 2 * KL + 2) {  // Tb or P fragments
      const int64_t ch = (int64_t)h * P.nc + c0 + i;
      const H8* fr = (const H8*)(gi == 2 * KL ? P.tb : P.pm) + ch * (8 * 64);
      lds_dma4(make_rsrc(fr, 8 * 1024), 128u * (uint32_t)frag_line(lane), 0, touch);
    } else if (gi < 2 * KL + 2 + VL) {  // the head's V rows, line gi - 2 KL - 2
      const T* src = vg + (tc * P.h_v + h) * DV;
      lds_dma4(make_rsrc(src, lrow * vstride + DV * 2), (uint32_t)lane * vstride + 128u * (uint32_t)(gi - 2 * KL - 2), 0,
               touch);
    } else {  // decay factors
      lds_dma4(gam_rsrc(i), 128u * (lane & 3), 0, touch);
    }
  };
  auto prefetch = [&](int i) {
#pragma unroll
    for (int j = 0; j < NTC; ++j) touch_group(nb + j * NB < NG ? nb + j * NB : NG - 1, i);
  };

  // ---- prologue ------------------------------------------------------------
  floatx4 S[KT];  // state wave: tile mt, element e is key channel state_row(mt, 4g + e)
  H8 sf[KB];   // state wave: S as 16-bit B fragments (inner = key channel)
  if (w == 0) {
#pragma unroll
    for (int mt = 0; mt < KT; ++mt)
#pragma unroll
      for (int e = 0; e < 4; ++e)
        S[mt][e] = ck == 3   ? (state_row(mt, 4 * g4 + e) == col ? 1.f : 0.f)
                   : ck < 2 && P.h0 ? P.h0[sbase + (int64_t)state_row(mt, 4 * g4 + e) * DV + col]
                                    : 0.f;
#pragma unroll
    for (int p = 0; p < KB; ++p) {
      sf[p] = pack<T>(S[2 * p], S[2 * p + 1]);
      sbuf[0][p][lane] = sf[p];
    }
  } else if (w < 3 && n > 0) {
    issue(0);
    issue(n > 1 ? 1 : 0);
    if (w == 1) {
      // touches for chunks 2..5 (the loop touches chunk t + PF)
#pragma unroll
      for (int i = 2; i < PF; ++i) prefetch(i < n ? i : n - 1);
      // chunk 0 has landed once at most the later copies and touches are pending
      __builtin_amdgcn_s_waitcnt(vmcnt_imm(kIssued + (PF - 2) * kTouched));
    } else {
      __builtin_amdgcn_s_waitcnt(vmcnt_imm(kIssued));
    }
  }
  lds_barrier();

  const uint32_t orow = (uint32_t)(((size_t)c16 * P.h_v + h) * DV + 16 * nb + 4 * g4) * 2;
  const uint32_t ostep = (uint32_t)(16 * P.h_v * DV * 2);  // 16 tokens
  // output wave: add (P Tb) R of chunk i (first token t0i) to the partial O^T
  // and store it; rows past the end of the sequence are dropped
  floatx4 o[4];
  H8 pmf[6];
  auto finish_output = [&](int64_t t0i, int i) {
    const H8 vf0 = vbuf[i & 1][0][lane], vf1 = vbuf[i & 1][1][lane];
    o[0] = mma(vf0, pmf[0], o[0]);
    o[1] = mma(vf0, pmf[1], o[1]);
    o[2] = mma(vf0, pmf[2], o[2]);
    o[3] = mma(vf0, pmf[4], o[3]);
    o[2] = mma(vf1, pmf[3], o[2]);
    o[3] = mma(vf1, pmf[5], o[3]);
    const int64_t left = te - t0i;
    const uint32_t len = (uint32_t)(left < C ? left : C);
    const rsrc_t orr = make_rsrc(obase + t0i * P.h_v * DV, len * (uint32_t)(P.h_v * DV * 2));
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) bstore(orr, orow + nt * ostep, pack4<T>(o[nt]));
  };

  int64_t t0prev = 0;  // output wave: first token of the chunk in o

  // Each role runs its own loop (one barrier per chunk in each), so that
  // the registers one role keeps across chunks are free in the others.
  if (w == 0) {
    for (int t = 0; t < n; ++t) {
      const LdsSlot<DK, T>& sl = slot[t % NS];
      const int64_t ch = (int64_t)h * P.nc + c0 + t;
      // ---------------- state wave ----------------
      // Nothing of this wave is in flight here; saying so lets the compiler
      // count the LDS reads below exactly (it cannot see through the
      // loaders' LDS-direct loads on the other branch).
      __builtin_amdgcn_s_waitcnt(0);
      // LDS reads in the order they are consumed: the operands of R and V'
      // and the K rows of X first, then (while X runs) the K^T fragments of
      // the update.  `sf` holds the state entering the chunk (packed at the
      // end of the last chunk).
      if (INSPECT) {
        H8* hp = (H8*)P.insp_h + ch * (int64_t)(DK * DV / 8);
#pragma unroll
        for (int p = 0; p < KB; ++p) hp[(nb * KB + p) * 64 + lane] = sf[p];
      }
      H8 tbf[6];
#pragma unroll
      for (int f = 0; f < 6; ++f) tbf[f] = sl.tb[f][lane];
      // V[16 nt + 4g + e][c] via the transposing read: lane 4e' + q of the
      // group addresses row 16 nt + 4g + e', columns 4q..4q+3
      H4 vv[4];
      floatx4 ebv[4];  // e^{b} of this lane's rows (GDN)
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) {
        vv[nt] = ds_read_tr<T>(&sl.v[16 * nt + 4 * g4 + (c16 >> 2)][4 * (c16 & 3)]);
        if constexpr (!KDA) ebv[nt] = *(const floatx4*)&sl.dec[16 * nt + 4 * g4];
      }
      // the state's decay: e^{b_n} (GDN), e^{B_n} of each state row (KDA)
      float gam = 1.f;
      floatx4 gmv[KDA ? KT : 1];
      if constexpr (KDA) {
#pragma unroll
        for (int mt = 0; mt < KT; ++mt) gmv[mt] = *(const floatx4*)&sl.dec[state_row(mt, 4 * g4)];
      } else {
        gam = sl.dec[C - 1];
      }
      // K rows of X's products (KDA: the K e^B fragments, token tile nt,
      // inner block p)
      H8 kr[KB][4];
      if constexpr (!DECAY) {
#pragma unroll
        for (int p = 0; p < KB; ++p)
#pragma unroll
          for (int nt = 0; nt < 4; ++nt)
            kr[p][nt] = KDA ? ((const H8*)sl.k)[(nt * KB + p) * 64 + lane]
                            : *(const H8*)(sl.k + swz<DK>(16 * nt + c16, 4 * p + g4));
      }
      __builtin_amdgcn_sched_barrier(0);
      // X = K S for the four token tiles (lane holds [16 nt + 4g + e][c]),
      // interleaved with work that does not depend on it: the K^T reads of
      // the update (outer = key channel state_row(mt, c), inner = token;
      // lane 4e' + q of group g addresses token 32p + 4g + e' (+16 for the
      // upper half), channels state_row(mt, 4q) .. +3), V to floats and the
      // decay of the state.  Step i issues one product, two reads (KDA: one
      // read of a K~^T fragment, (mt, p) = (i / 2, i % 2)) and NV vector
      // operations.
      floatx4 x[4];
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) x[nt] = zero4();
      H4 kt[2][KT][2];
      H8 ktf[KDA ? 2 : 1][KDA ? KT : 1];
      floatx4 vfl[4];
      static_assert(2 * 2 * KT == 2 * 4 * KB, "two K^T reads per product");
      constexpr int NV = (4 * KT + 16 + 4 * KB - 1) / (4 * KB);  // vector operations per product
#pragma unroll
      for (int i = 0; i < 4 * KB; ++i) {
        if constexpr (!DECAY) x[i % 4] = mma(kr[i / 4][i % 4], sf[i / 4], x[i % 4]);
        if constexpr (KDA) {
          ktf[i % 2][i / 2] = ((const H8*)sl.q)[i * 64 + lane];
        } else {
#pragma unroll
          for (int jj = 0; jj < 2; ++jj) {
            const int j = 2 * i + jj, p = j / (2 * KT), mt = (j / 2) % KT, hf = j % 2;
            const int r0 = 32 * p + 4 * g4 + (c16 >> 2) + 16 * hf;
            const int d = state_row(mt, 4 * (c16 & 3));
            kt[p][mt][hf] = ds_read_tr<T>(sl.k + swz<DK>(r0, d >> 3) + 2 * (d & 7));
          }
        }
#pragma unroll
        for (int jj = 0; jj < NV; ++jj) {
          const int j = NV * i + jj;
          if (j < 4 * KT) {
            S[j / 4][j % 4] *= KDA ? gmv[KDA ? j / 4 : 0][j % 4] : gam;
          } else if (j < 4 * KT + 16) {
            const int q2 = j - 4 * KT;
            vfl[q2 / 4][q2 % 4] = to_f(vv[q2 / 4][q2 % 4]);
          }
        }
        __builtin_amdgcn_sched_barrier(0);
      }
      // R = V - diag(e^b) X (KDA: V - X), as B fragments (inner = token);
      // decay-only: R = V
      floatx4 rr[4];
#pragma unroll
      for (int nt = 0; nt < 4; ++nt)
#pragma unroll
        for (int e = 0; e < 4; ++e)
          rr[nt][e] = DECAY ? vfl[nt][e] : KDA ? vfl[nt][e] - x[nt][e] : vfl[nt][e] - ebv[nt][e] * x[nt][e];
      const H8 rf0 = pack<T>(rr[0], rr[1]), rf1 = pack<T>(rr[2], rr[3]);
      // GDN: R goes to the output wave, which multiplies it with P Tb
      if constexpr (!KDA) {
        vbuf[t & 1][0][lane] = rf0;
        vbuf[t & 1][1][lane] = rf1;
      }
      // diag(e^{b_n - b}) V' = (diag(e^{b_n - b}) Tb) R (KDA: V' = Tb R)
      floatx4 vt[4];
      vt[0] = mma(tbf[0], rf0, zero4());
      vt[1] = mma(tbf[1], rf0, zero4());
      vt[2] = mma(tbf[2], rf0, zero4());
      vt[3] = mma(tbf[4], rf0, zero4());
      vt[2] = mma(tbf[3], rf1, vt[2]);
      vt[3] = mma(tbf[5], rf1, vt[3]);
      const H8 vs0 = pack<T>(vt[0], vt[1]), vs1 = pack<T>(vt[2], vt[3]);
      // KDA: V' goes to the output wave, which multiplies it with P
      if constexpr (KDA) {
        vbuf[t & 1][0][lane] = vs0;
        vbuf[t & 1][1][lane] = vs1;
      }
      if (INSPECT) {
        // V' itself, for the intermediate checks
        floatx4 vq[4];
#pragma unroll
        for (int nt = 0; nt < 4; ++nt) {
          const floatx4 env = KDA ? floatx4{1.f, 1.f, 1.f, 1.f} : *(const floatx4*)&sl.dec[C + 16 * nt + 4 * g4];
#pragma unroll
          for (int e = 0; e < 4; ++e) vq[nt][e] = KDA ? vt[nt][e] : vt[nt][e] / env[e];
        }
        H8* vp = (H8*)P.insp_vp + ch * (int64_t)(C * DV / 8);
        vp[(nb * 2 + 0) * 64 + lane] = pack<T>(vq[0], vq[1]);
        vp[(nb * 2 + 1) * 64 + lane] = pack<T>(vq[2], vq[3]);
      }
      // S <- e^{b_n} S + K^T (diag(e^{b_n - b}) V') (KDA: Diag(e^{B_n}) S + K~^T V')
#pragma unroll
      for (int p = 0; p < 2; ++p)
#pragma unroll
        for (int mt = 0; mt < KT; ++mt)
          S[mt] = mma(KDA ? ktf[KDA ? p : 0][KDA ? mt : 0] : cat<T>(kt[p][mt][0], kt[p][mt][1]), p == 0 ? vs0 : vs1,
                      S[mt]);
#pragma unroll
      for (int p = 0; p < KB; ++p) {
        sf[p] = pack<T>(S[2 * p], S[2 * p + 1]);
        sbuf[(t + 1) & 1][p][lane] = sf[p];
      }
      lds_barrier();  // next state and this R published, slot t % NS free, chunk t+1 landed
    }
    if (sout) {
#pragma unroll
      for (int mt = 0; mt < KT; ++mt)
#pragma unroll
        for (int e = 0; e < 4; ++e)
          sout[sbase + (int64_t)state_row(mt, 4 * g4 + e) * DV + col] = S[mt][e];
    }
    if (kind == 1) {
      // the same state, packed as it entered the last product: the A
      // fragments (outer = column, inner = key channel) of the fix-up
      H8* mf = (H8*)P.seg.midf + (((int64_t)seq * P.h_v + h) * NB + nb) * (KB * 64);
#pragma unroll
      for (int p = 0; p < KB; ++p) mf[p * 64 + lane] = sf[p];
    }
  } else if (w == 3) {
    // KDA: the Q e^B fragments (token tile nt, inner block p) of the next
    // chunk, loaded from the workspace one chunk ahead (unconditionally:
    // past the last chunk the last one again)
    H8 qn[KDA ? 4 : 1][KDA ? KB : 1];
    auto load_q = [&](int i) {
      const rsrc_t qrs = kda_rsrc(P.qw, i);
#pragma unroll
      for (int nt = 0; nt < 4; ++nt)
#pragma unroll
        for (int p = 0; p < KB; ++p) qn[nt][p] = fload<H8>(qrs, 16u * lane, nt * KB + p);
    };
    if constexpr (KDA) {
      if (n > 0) load_q(0);
    }
    for (int t = 0; t < n; ++t) {
      const LdsSlot<DK, T>& sl = slot[t % NS];
      const int64_t t0 = ts + (int64_t)C * t;
      // ---------------- output wave ----------------
      // finish the previous chunk: its R (KDA: V') was published at the last barrier
      if (t > 0) finish_output(t0prev, t - 1);
      // state part of this chunk's O^T: lane holds [column 4g + e][token 16 nt + c]
      H8 so[KB];
#pragma unroll
      for (int p = 0; p < KB; ++p) so[p] = sbuf[t & 1][p][lane];
      H8 qr[4][KB];
      if constexpr (KDA) {
#pragma unroll
        for (int nt = 0; nt < 4; ++nt)
#pragma unroll
          for (int p = 0; p < KB; ++p) qr[nt][p] = qn[nt][p];
        load_q(t + 1 < n ? t + 1 : n - 1);
      } else {
#pragma unroll
        for (int nt = 0; nt < 4; ++nt)
#pragma unroll
          for (int p = 0; p < KB; ++p) qr[nt][p] = *(const H8*)(sl.q + swz<DK>(16 * nt + c16, 4 * p + g4));
      }
      float ebt[4];
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) ebt[nt] = KDA ? 1.f : sl.dec[16 * nt + c16];
#pragma unroll
      for (int f = 0; f < 6; ++f) pmf[f] = sl.pm[f][lane];  // kept for the next step
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) o[nt] = zero4();
#pragma unroll
      for (int p = 0; p < KB; ++p)
#pragma unroll
        for (int nt = 0; nt < 4; ++nt) o[nt] = mma(so[p], qr[nt][p], o[nt]);
      if constexpr (!KDA) {
#pragma unroll
        for (int nt = 0; nt < 4; ++nt) o[nt] *= ebt[nt];
      }
      t0prev = t0;
      lds_barrier();  // next state and this R published, slot t % NS free, chunk t+1 landed
    }
    if (n > 0) finish_output(t0prev, n - 1);
  } else if (PAIR && w == 4) {
    // ---------------- transition wave (PAIR) ----------------
    // Segment-0 workgroups leave it idle; it keeps the barrier count.
    if (kind != 4) {
      for (int t = 0; t < n; ++t) lds_barrier();
      return;
    }
    // M from the identity, R = -diag(e^b) K M (V = 0), M <- e^{b_n} M +
    // K^T (Tv R), as the state wave's chain; the outputs G = diag(e^b) Q M +
    // (P Tb) R as the output wave forms O, from this wave's M fragments and
    // R.  This wave copies nothing into LDS: after this wait nothing of it is
    // in flight but its own stores of G.
    __builtin_amdgcn_s_waitcnt(0);
    floatx4 M[KT];
    H8 mf[KB];  // M entering the chunk, B fragments (inner = key channel)
#pragma unroll
    for (int mt = 0; mt < KT; ++mt)
#pragma unroll
      for (int e = 0; e < 4; ++e) M[mt][e] = state_row(mt, 4 * g4 + e) == col ? 1.f : 0.f;
#pragma unroll
    for (int p = 0; p < KB; ++p) mf[p] = pack<T>(M[2 * p], M[2 * p + 1]);
    for (int t = 0; t < n; ++t) {
      const LdsSlot<DK, T>& sl = slot[t % NS];
      const int64_t t0 = ts + (int64_t)C * t;
      // G's state part diag(e^b) Q M; lane: [column 4g + e][token 16 nt + c]
      floatx4 gq[4];
      {
        H8 qr[4][KB];
#pragma unroll
        for (int nt = 0; nt < 4; ++nt)
#pragma unroll
          for (int p = 0; p < KB; ++p) qr[nt][p] = *(const H8*)(sl.q + swz<DK>(16 * nt + c16, 4 * p + g4));
#pragma unroll
        for (int nt = 0; nt < 4; ++nt) gq[nt] = zero4();
#pragma unroll
        for (int p = 0; p < KB; ++p)
#pragma unroll
          for (int nt = 0; nt < 4; ++nt) gq[nt] = mma(mf[p], qr[nt][p], gq[nt]);
      }
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) gq[nt] *= sl.dec[16 * nt + c16];
      // (phases fenced so that at most one phase's fragments are live: the
      // wave has at most 256 registers)
      __builtin_amdgcn_sched_barrier(0);
      const float gam = sl.dec[C - 1];
      if constexpr (DECAY) {
        // R = V = 0: M <- e^{b_n} M, and G has no (P Tb) R part
#pragma unroll
        for (int mt = 0; mt < KT; ++mt) M[mt] *= gam;
      } else {
        H8 tbf[6];
#pragma unroll
        for (int f = 0; f < 6; ++f) tbf[f] = sl.tb[f][lane];
        floatx4 ebv[4];
#pragma unroll
        for (int nt = 0; nt < 4; ++nt) ebv[nt] = *(const floatx4*)&sl.dec[16 * nt + 4 * g4];
        H8 kr[KB][4];
#pragma unroll
        for (int p = 0; p < KB; ++p)
#pragma unroll
          for (int nt = 0; nt < 4; ++nt) kr[p][nt] = *(const H8*)(sl.k + swz<DK>(16 * nt + c16, 4 * p + g4));
        __builtin_amdgcn_sched_barrier(0);
        // X = K M, interleaved with the K^T reads and the decay of M (the
        // state wave's order)
        floatx4 x[4];
#pragma unroll
        for (int nt = 0; nt < 4; ++nt) x[nt] = zero4();
        H4 kt[2][KT][2];
        constexpr int NVM = (4 * KT + 4 * KB - 1) / (4 * KB);
#pragma unroll
        for (int i = 0; i < 4 * KB; ++i) {
          x[i % 4] = mma(kr[i / 4][i % 4], mf[i / 4], x[i % 4]);
#pragma unroll
          for (int jj = 0; jj < 2; ++jj) {
            const int j = 2 * i + jj, p = j / (2 * KT), mt = (j / 2) % KT, hf = j % 2;
            const int r0 = 32 * p + 4 * g4 + (c16 >> 2) + 16 * hf;
            const int d = state_row(mt, 4 * (c16 & 3));
            kt[p][mt][hf] = ds_read_tr<T>(sl.k + swz<DK>(r0, d >> 3) + 2 * (d & 7));
          }
#pragma unroll
          for (int jj = 0; jj < NVM; ++jj) {
            const int j = NVM * i + jj;
            if (j < 4 * KT) M[j / 4][j % 4] *= gam;
          }
          __builtin_amdgcn_sched_barrier(0);
        }
        floatx4 rr[4];
#pragma unroll
        for (int nt = 0; nt < 4; ++nt)
#pragma unroll
          for (int e = 0; e < 4; ++e) rr[nt][e] = 0.f - ebv[nt][e] * x[nt][e];
        const H8 rf0 = pack<T>(rr[0], rr[1]), rf1 = pack<T>(rr[2], rr[3]);
        floatx4 vt[4];
        vt[0] = mma(tbf[0], rf0, zero4());
        vt[1] = mma(tbf[1], rf0, zero4());
        vt[2] = mma(tbf[2], rf0, zero4());
        vt[3] = mma(tbf[4], rf0, zero4());
        vt[2] = mma(tbf[3], rf1, vt[2]);
        vt[3] = mma(tbf[5], rf1, vt[3]);
        const H8 vs0 = pack<T>(vt[0], vt[1]), vs1 = pack<T>(vt[2], vt[3]);
        __builtin_amdgcn_sched_barrier(0);
        H8 ptb[6];  // P Tb, read while the update runs
#pragma unroll
        for (int f = 0; f < 6; ++f) ptb[f] = sl.pm[f][lane];
#pragma unroll
        for (int p = 0; p < 2; ++p)
#pragma unroll
          for (int mt = 0; mt < KT; ++mt) M[mt] = mma(cat<T>(kt[p][mt][0], kt[p][mt][1]), p == 0 ? vs0 : vs1, M[mt]);
        // G's (P Tb) R part (R as A fragments: outer = column, inner = token)
        gq[0] = mma(rf0, ptb[0], gq[0]);
        gq[1] = mma(rf0, ptb[1], gq[1]);
        gq[2] = mma(rf0, ptb[2], gq[2]);
        gq[3] = mma(rf0, ptb[4], gq[3]);
        gq[2] = mma(rf1, ptb[3], gq[2]);
        gq[3] = mma(rf1, ptb[5], gq[3]);
      }
      const int64_t left = te - t0;
      const uint32_t len = (uint32_t)(left < C ? left : C);
      const rsrc_t orr = make_rsrc(obase + t0 * P.h_v * DV, len * (uint32_t)(P.h_v * DV * 2));
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) bstore(orr, orow + nt * ostep, pack4<T>(gq[nt]));
#pragma unroll
      for (int p = 0; p < KB; ++p) mf[p] = pack<T>(M[2 * p], M[2 * p + 1]);
      lds_barrier();  // slot t % NS free, chunk t+1 landed
    }
#pragma unroll
    for (int mt = 0; mt < KT; ++mt)
#pragma unroll
      for (int e = 0; e < 4; ++e) sout[sbase + (int64_t)state_row(mt, 4 * g4 + e) * DV + col] = M[mt][e];
  } else {
    for (int t = 0; t < n; ++t) {
      // ---------------- loader waves ----------------
      issue(t + 2 < n ? t + 2 : n - 1);
      // chunk t+1's copy has landed; chunk t+2's copy and the touches issued
      // after t+1's copy (chunks t+5 and t+6, often HBM misses) may be pending
      if (w == 1) {
        prefetch(t + PF < n ? t + PF : n - 1);
        __builtin_amdgcn_s_waitcnt(vmcnt_imm(kIssued + 2 * kTouched));
      } else {
        __builtin_amdgcn_s_waitcnt(vmcnt_imm(kIssued));
      }
      lds_barrier();  // next state and this R published, slot t % NS free, chunk t+1 landed
    }
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
  }
}

// Segment mode, second step (see SegParams): one workgroup per (unit, 16
// state columns) chains the entering states in fp32, E_1 = mid, E_{s+1} =
// N_s + M_s E_s, writes E_2 .. E_{np-1} as the fix-up's A fragments (E_1's
// come from the segment-0 scan) and ht = E_np.  The product runs on fp32
// MFMA (16x16x4): dk/16 waves, wave w takes row tile w of M_s, the
// B operand (E_s, k = 16 (kk / 4) + 4g + kk % 4 in step kk) sits in
// registers, the A operand comes from M_s staged in LDS (rows padded by 4
// floats, so a 16-lane phase of the 16-byte reads hits distinct banks).
// M_{s+1} and N_{s+1} are loaded while step s computes.
template <int DK, typename T>
__global__ __launch_bounds__(DK * 4) void seg_compose_kernel(ScanParams P, int32_t units) {
  typedef typename VT<T>::v8 H8;
  constexpr int DV = DK, KB = DK / 32, CT = DV / 16;
  constexpr int LD = DK + 4;             // padded row of M in LDS
  constexpr int LE = 20;                 // padded row of E in LDS
  constexpr int NT = DK * 4;             // threads: one wave per row tile
  constexpr int NM = DK * DK / 4 / NT;   // floatx4 loads of M per thread
  constexpr int RW = 1;                  // row tiles per wave
  constexpr int KS = DK / 4;             // MFMA steps over k
  __shared__ __attribute__((aligned(16))) float mb[2][DK * LD];  // M_s, double-buffered
  __shared__ __attribute__((aligned(16))) float eb[DK * LE];     // E_s, this block's 16 columns
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int g4 = lane >> 4, c16 = lane & 15;
  const int u = blockIdx.x / CT, cb = blockIdx.x - u * CT;
  const int64_t base = (int64_t)u * DK * DV;
  floatx4 mr[NM], nr[RW], nc[RW];
  auto load = [&](int s) {  // M_s (coalesced) and this lane's N_s entries into registers
    const int64_t so = (int64_t)(s - 1) * P.seg.us + base;
    const floatx4* m4 = (const floatx4*)(P.seg.m + so);
#pragma unroll
    for (int f = 0; f < NM; ++f) mr[f] = m4[f * NT + tid];
#pragma unroll
    for (int i = 0; i < RW; ++i)
#pragma unroll
      for (int e = 0; e < 4; ++e)
        nr[i][e] = P.seg.n[so + (int64_t)(16 * (RW * w + i) + 4 * g4 + e) * DV + 16 * cb + c16];
  };
  auto stage = [&](int buf) {  // registers -> LDS rows
#pragma unroll
    for (int f = 0; f < NM; ++f) {
      const int e = 4 * (f * NT + tid);
      *(floatx4*)&mb[buf][(e / DK) * LD + e % DK] = mr[f];
    }
  };
  for (int i = tid; i < DK * 16; i += NT) eb[(i / 16) * LE + i % 16] = P.seg.mid[base + (int64_t)(i / 16) * DV + 16 * cb + i % 16];
  load(1);
  stage(0);
#pragma unroll
  for (int i = 0; i < RW; ++i) nc[i] = nr[i];
  __syncthreads();
  for (int s = 1; s < P.seg.np; ++s) {
    const bool more = s + 1 < P.seg.np;
    if (more) load(s + 1);  // in flight during this step
    if (s >= 2) {
      // E_s as fragments: lane 16g + c of key block p holds column 16 cb + c
      // at key channels 32p + 8g + j
      H8* mf = (H8*)P.seg.midf + (int64_t)(s - 1) * (P.seg.us / 8) + ((int64_t)u * CT + cb) * (KB * 64);
      for (int f = tid; f < KB * 64; f += NT) {
        const int p = f / 64, l = f % 64, g = l >> 4, c = l & 15;
        H8 x;
#pragma unroll
        for (int j = 0; j < 8; ++j) x[j] = (T)eb[(32 * p + 8 * g + j) * LE + c];
        mf[f] = x;
      }
    }
    float bf[KS];  // B: E_s[k][c16], k = 16 (kk / 4) + 4 g + kk % 4
#pragma unroll
    for (int kk = 0; kk < KS; ++kk) bf[kk] = eb[(16 * (kk >> 2) + 4 * g4 + (kk & 3)) * LE + c16];
    floatx4 acc[RW];
    const float* mbuf = mb[(s - 1) & 1];
#pragma unroll
    for (int i = 0; i < RW; ++i) {
      acc[i] = nc[i];
      const float* arow = mbuf + (16 * (RW * w + i) + c16) * LD + 4 * g4;
#pragma unroll
      for (int kq = 0; kq < KS / 4; ++kq) {
        const floatx4 a4 = *(const floatx4*)(arow + 16 * kq);  // M[row c][16 kq + 4g + j]
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i] = __builtin_amdgcn_mfma_f32_16x16x4f32(a4[j], bf[4 * kq + j], acc[i], 0, 0, 0);
      }
    }
    __syncthreads();  // every read of E_s and of M_s's buffer is done
    // lane: rows 16 rt + 4g + e, column c16
#pragma unroll
    for (int i = 0; i < RW; ++i)
#pragma unroll
      for (int e = 0; e < 4; ++e) eb[(16 * (RW * w + i) + 4 * g4 + e) * LE + c16] = acc[i][e];
    if (more) {
      stage(s & 1);
#pragma unroll
      for (int i = 0; i < RW; ++i) nc[i] = nr[i];
    }
    __syncthreads();
  }
  if (P.ht) {
    for (int i = tid; i < DK * 16; i += NT)
      P.ht[base + (int64_t)(i / 16) * DV + 16 * cb + i % 16] = eb[(i / 16) * LE + i % 16];
  }
}

// Two segments: ht = N_1 + M_1 E_1 for 16 state columns (column tile ct)
// of unit u, on a fix-up workgroup's four waves (wave w takes row tiles
// RT w .. RT w + RT - 1), in fp32 on 16x16x4 MFMA.  Step 4q + j contracts
// key channel k = 16q + 4g + j on lanes 16g + c, so that four lanes read 64
// consecutive bytes of an M row at once.  Every load is issued before the
// first product.
template <int DK>
__device__ __forceinline__ void seg_final2(const ScanParams& P, int u, int ct) {
  constexpr int RT = DK / 64, KS = DK / 4;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int g4 = lane >> 4, c16 = lane & 15;
  const int64_t base = (int64_t)u * DK * DK;
  float bf[KS];  // B: E_1[16q + 4g + j][16 ct + c] in step 4q + j
#pragma unroll
  for (int kk = 0; kk < KS; ++kk)
    bf[kk] = P.seg.mid[base + (int64_t)(16 * (kk >> 2) + 4 * g4 + (kk & 3)) * DK + 16 * ct + c16];
  floatx4 acc[RT], a4[RT][KS / 4];  // acc lane: rows 16 rt + 4g + e, column 16 ct + c
#pragma unroll
  for (int i = 0; i < RT; ++i) {
    const int rt = RT * w + i;
#pragma unroll
    for (int e = 0; e < 4; ++e) acc[i][e] = P.seg.n[base + (int64_t)(16 * rt + 4 * g4 + e) * DK + 16 * ct + c16];
    const float* arow = P.seg.m + base + (int64_t)(16 * rt + c16) * DK + 4 * g4;
#pragma unroll
    for (int q = 0; q < KS / 4; ++q) a4[i][q] = *(const floatx4*)(arow + 16 * q);  // M_1[row][16q + 4g + j]
  }
#pragma unroll
  for (int q = 0; q < KS / 4; ++q)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int i = 0; i < RT; ++i) acc[i] = __builtin_amdgcn_mfma_f32_16x16x4f32(a4[i][q][j], bf[4 * q + j], acc[i], 0, 0, 0);
#pragma unroll
  for (int i = 0; i < RT; ++i)
#pragma unroll
    for (int e = 0; e < 4; ++e)
      P.ht[base + (int64_t)(16 * (RT * w + i) + 4 * g4 + e) * DK + 16 * ct + c16] = acc[i][e];
}

// Segment mode, last step: one workgroup per (unit, segment s >= 1, cpb
// consecutive chunks of it), O^T += E_s^T G^T for the chunks' tokens.  E_s's
// A fragments (outer = state column, inner = key channels 32p + 8g + j) are
// staged in LDS once; G is read as row fragments (outer = token, the same
// channels); wave w takes tokens 16w .. 16w + 15 of each chunk and updates o
// 8 bytes per lane.  ng workgroups per segment cover the longest.  With two
// segments (no compose step) the first nfin workgroups, units x dv/16 of
// them, form ht (seg_final2) while the others fix o.  When the unit count is
// a multiple of 8, both kinds are dealt as seg_item deals the scan's (a
// unit's work in one XCD's share of the indices), so that each reads G, o,
// M, N and the entering states on the XCD whose L2 the scan wrote them
// through.
template <int DK, typename T>
__global__ __launch_bounds__(256) void seg_fix_kernel(ScanParams P, int32_t ng, int32_t cpb, int32_t nfin) {
  typedef typename VT<T>::v8 H8;
  typedef typename VT<T>::v4 H4;
  constexpr int DV = DK, KB = DK / 32, CT = DV / 16;
  __shared__ H8 af[CT * KB * 64];  // E_s as A fragments
  const int units = P.s.n_seqs * P.h_v, nsg = P.seg.np - 1;
  const int nfix = units * nsg * ng;
  const bool xcd = units % 8 == 0;  // then nfin and nfix are multiples of 8 too
  if ((int)blockIdx.x < nfin) {
    const int b = (int)blockIdx.x;
    const int l = xcd ? (b % 8) * (nfin / 8) + b / 8 : b;
    seg_final2<DK>(P, l / CT, l % CT);
    return;
  }
  const int b = (int)blockIdx.x - nfin;
  const int bid = xcd ? (b % 8) * (nfix / 8) + b / 8 : b;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int g4 = lane >> 4, c16 = lane & 15;
  const int u = bid / (nsg * ng), rem = bid - u * (nsg * ng);
  const int s = 1 + rem / ng, cg = rem - (s - 1) * ng;
  const int seq = u / P.h_v, h = u - seq * P.h_v;
  // the sequence's tokens and chunks, as the scan takes them
  int64_t ts, te, n_i;
  if (P.s.chunk_seq) {
    ts = P.s.cu[seq];
    te = P.s.cu[seq + 1];
    int64_t c0, c1;
    seq_chunks(P.s, seq, P.nc, c0, c1);
    n_i = te > ts ? (te - ts + C - 1) / C : 0;
    if (n_i > c1 - c0) n_i = c1 - c0;
  } else {
    ts = (int64_t)seq * P.s.seq_len;
    te = ts + P.s.seq_len;
    n_i = P.s.cps;
  }
  int64_t first, len;
  seg_span(n_i, P.seg.np, P.seg.w0, s, first, len);
  const int cs = (int)first, ce = (int)(first + len);
  const int cb = cs + cg * cpb, cend = cb + cpb < ce ? cb + cpb : ce;
  if (cb >= cend) return;  // the whole workgroup: past its segment's end
  constexpr uint32_t es = sizeof(T);
  const uint32_t kstride = (uint32_t)P.h_v * DK * es;  // G has o's layout
  // lane: columns 16 ct + 4g + e of token 16 w + c
  const uint32_t off0 = (uint32_t)(((16 * w + c16) * P.h_v + h) * DV + 4 * g4) * es;
  const uint32_t goff = (uint32_t)(16 * w + c16) * kstride + (uint32_t)(8 * g4) * es;
  auto rsrcs = [&](int c, rsrc_t& gr, rsrc_t& orr) {
    const int64_t t0 = ts + (int64_t)c * C;
    const int64_t left = te - t0;
    const uint32_t len = (uint32_t)(left < C ? left : C);
    gr = make_rsrc((const T*)P.seg.g + (t0 * P.h_v + h) * DK, (len - 1) * kstride + DK * es);
    orr = make_rsrc((T*)P.o + t0 * P.h_v * DV, len * (uint32_t)(P.h_v * DV * es));
  };
  // the next chunk's G and o are loaded while this one is multiplied and stored
  rsrc_t gr, orr;
  rsrcs(cb, gr, orr);
  H8 gf[KB];
  H4 ov[CT];
#pragma unroll
  for (int p = 0; p < KB; ++p) gf[p] = bload<H8>(gr, goff + 32 * es * p);
#pragma unroll
  for (int ct = 0; ct < CT; ++ct) ov[ct] = bload<H4>(orr, off0 + 16 * es * ct);
  // E_s's fragments into LDS while the first chunk's G and o are in flight
  const H8* mf = (const H8*)P.seg.midf + (int64_t)(s - 1) * (P.seg.us / 8) + (int64_t)u * (CT * KB * 64);
#pragma unroll
  for (int f = 0; f < CT * KB * 64 / 256; ++f) af[f * 256 + tid] = mf[f * 256 + tid];
  __syncthreads();
  for (int c = cb; c < cend; ++c) {
    rsrc_t grn = gr, orn = orr;
    H8 gn[KB];
    H4 on[CT];
    if (c + 1 < cend) {
      rsrcs(c + 1, grn, orn);
#pragma unroll
      for (int p = 0; p < KB; ++p) gn[p] = bload<H8>(grn, goff + 32 * es * p);
#pragma unroll
      for (int ct = 0; ct < CT; ++ct) on[ct] = bload<H4>(orn, off0 + 16 * es * ct);
    }
#pragma unroll
    for (int ct = 0; ct < CT; ++ct) {
      floatx4 acc = zero4();
#pragma unroll
      for (int p = 0; p < KB; ++p) acc = mma(af[(ct * KB + p) * 64 + lane], gf[p], acc);
      floatx4 sum;
#pragma unroll
      for (int e = 0; e < 4; ++e) sum[e] = to_f(ov[ct][e]) + acc[e];
      bstore(orr, off0 + 16 * es * ct, pack4<T>(sum));
    }
    gr = grn;
    orr = orn;
#pragma unroll
    for (int p = 0; p < KB; ++p) gf[p] = gn[p];
#pragma unroll
    for (int ct = 0; ct < CT; ++ct) ov[ct] = on[ct];
  }
}

template <int DK, typename T>
hipError_t launch_seg_compose(const ScanParams& P, int64_t n_units, hipStream_t st) {
  hipLaunchKernelGGL((seg_compose_kernel<DK, T>), dim3((unsigned)(n_units * (DK / 16))), dim3(DK * 4), 0, st, P,
                     (int32_t)n_units);
  return hipGetLastError();
}

template <int DK, typename T>
hipError_t launch_seg_fix(const ScanParams& P, int64_t n_units, int32_t cps, hipStream_t st) {
  // cps: chunks of the longest sequence, whose later segments are the
  // longest (seg_span)
  const int32_t last = (int32_t)((256 * (int64_t)cps) / (P.seg.w0 + 256 * (P.seg.np - 1)));
  // chunks per workgroup: one while that leaves at most a workgroup per
  // compute unit (256), at most four (each workgroup loads E_s once)
  const int64_t per = n_units * (P.seg.np - 1) * (int64_t)last / 256;
  const int32_t cpb = per < 1 ? 1 : per > 4 ? 4 : (int32_t)per;
  const int32_t ng = (last + cpb - 1) / cpb;
  const int64_t nfix = n_units * (P.seg.np - 1) * ng;
  // two segments: ht = N_1 + M_1 E_1 in the same launch (no compose step)
  const int64_t nfin = P.seg.np == 2 && P.ht ? n_units * (DK / 16) : 0;
  if (nfix + nfin <= 0) return hipSuccess;
  hipLaunchKernelGGL((seg_fix_kernel<DK, T>), dim3((unsigned)(nfix + nfin)), dim3(256), 0, st, P, ng, cpb,
                     (int32_t)nfin);
  return hipGetLastError();
}

#define DRLA_SEG_INST(DK_, T_)                                                                      \
  template hipError_t launch_seg_compose<DK_, T_>(const ScanParams&, int64_t, hipStream_t);         \
  template hipError_t launch_seg_fix<DK_, T_>(const ScanParams&, int64_t, int32_t, hipStream_t);
DRLA_SEG_INST(64, bf16)
DRLA_SEG_INST(128, bf16)
DRLA_SEG_INST(64, f16)
DRLA_SEG_INST(128, f16)
DRLA_SEG_INST(64, float)
DRLA_SEG_INST(128, float)
#undef DRLA_SEG_INST

template <int DK, int DV, typename T, bool KDA>
static void launch_scan_lds_v(const ScanParams& P, int64_t nblk, bool inspect, hipStream_t st) {
  if constexpr (!KDA && DK == DV) {
    if (P.seg.s1 > 0 && P.seg.pair && !inspect) {
      if (P.decay_only)
        hipLaunchKernelGGL((scan_lds_kernel<DK, DV, false, T, true, false, true>), dim3((unsigned)nblk), dim3(320), 0,
                           st, P);
      else
        hipLaunchKernelGGL((scan_lds_kernel<DK, DV, false, T, false, false, true>), dim3((unsigned)nblk), dim3(320),
                           0, st, P);
      return;
    }
  }
  if (P.decay_only && inspect)
    hipLaunchKernelGGL((scan_lds_kernel<DK, DV, true, T, true, KDA>), dim3((unsigned)nblk), dim3(256), 0, st, P);
  else if (P.decay_only)
    hipLaunchKernelGGL((scan_lds_kernel<DK, DV, false, T, true, KDA>), dim3((unsigned)nblk), dim3(256), 0, st, P);
  else if (inspect)
    hipLaunchKernelGGL((scan_lds_kernel<DK, DV, true, T, false, KDA>), dim3((unsigned)nblk), dim3(256), 0, st, P);
  else
    hipLaunchKernelGGL((scan_lds_kernel<DK, DV, false, T, false, KDA>), dim3((unsigned)nblk), dim3(256), 0, st, P);
}

template <int DK, int DV, typename T>
hipError_t launch_scan_lds(const ScanParams& P, int64_t nblk, bool inspect, hipStream_t st) {
  if (nblk > 0) launch_scan_lds_v<DK, DV, T, false>(P, nblk, inspect, st);
  return hipGetLastError();
}

template <int DK, int DV, typename T>
hipError_t launch_scan_lds_kda(const ScanParams& P, int64_t nblk, bool inspect, hipStream_t st) {
  if (nblk > 0) launch_scan_lds_v<DK, DV, T, true>(P, nblk, inspect, st);
  return hipGetLastError();
}

#define DRLA_SCAN_LDS_INST(DK_, DV_, T_)                                                             \
  template hipError_t launch_scan_lds<DK_, DV_, T_>(const ScanParams&, int64_t, bool, hipStream_t); \
  template hipError_t launch_scan_lds_kda<DK_, DV_, T_>(const ScanParams&, int64_t, bool, hipStream_t);
DRLA_SCAN_LDS_INST(64, 64, bf16)
DRLA_SCAN_LDS_INST(128, 64, bf16)
DRLA_SCAN_LDS_INST(64, 128, bf16)
DRLA_SCAN_LDS_INST(128, 128, bf16)
DRLA_SCAN_LDS_INST(64, 64, f16)
DRLA_SCAN_LDS_INST(128, 64, f16)
DRLA_SCAN_LDS_INST(64, 128, f16)
DRLA_SCAN_LDS_INST(128, 128, f16)
#undef DRLA_SCAN_LDS_INST

}  // namespace drla
