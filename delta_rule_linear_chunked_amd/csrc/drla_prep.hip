// Chunk-parallel preparation for delta-rule chunked prefill (gfx950).
//
// "Empowering Hybrid Attention Models on NPUs", Section 2.1 splits chunked
// prefill into chunk-independent Map operators (#1 Gate, #2 KKT, #3 Solve,
// #4 W/U), a sequence-dependent Reduce (#5 H) and a chunk-independent output
// Map (#6 O); Section 5 factors the inverse out of W ("operator rewriting")
// so that the products with K, S and Q no longer wait for the inversion.
// This kernel does the chunk-independent part once per (chunk, value head):
//
//   #1 Gate   b_r = sum_{i<=r} g_i in the chunk (per key channel for KDA)
//   #2 KKT    A = strict_lower(diag(beta) (K K^T (.) D)),  D_ri = e^{b_r-b_i}
//             (KDA: (K e^{B}) (K e^{-B})^T, the decay per key channel)
//   #3 Solve  T = (I + A)^{-1}: 16x16 diagonal blocks by forward
//             substitution, the rest by two rounds of blocked products
//   #4 factor Tb = T diag(beta): W = Tb diag(e^b) K and U = Tb V are never
//             formed; the scan applies Tb to V - diag(e^b) K S instead
//             (Section 5's rewriting: V' = U - W S = Tb (V - diag(e^b) K S)).
//
// It also emits the chunk-local operands of the output Map, so that the
// sequential kernel only multiplies:
//   P   = lower_incl(Q K^T (.) D)                 (KDA: (Q e^{B})(K e^{-B})^T)
//   K~^T with K~ = diag(e^{b_n - b}) K            (KDA: K (.) e^{b_n - B});
//        not needed (null) when the scan transposes K itself
//   the decay factors: GDN e^{b_r} and e^{b_n - b_r} per token row;
//   KDA e^{b_n} per key channel, and K e^{B}, Q e^{B}.
// All are written in MFMA fragment order (drla_common.h).
#include <atomic>

#include <type_traits>

#include "drla_common.h"
#include "drla_kernels.h"

namespace drla {

// Batches of at most this many sequences: the schedule kernel keeps their
// lengths and first chunks in LDS, writes the chunk table with every thread
// and ranks the sequences itself.
constexpr int kScheduleLdsSeqs = 1024;

// Chunk table of packed input, built from a checked copy of the device
// cu_seqlens (the kernels after this one read only the copy).  The device
// array must equal the host copy the call was sized and validated with:
// cu[0] = 0, non-decreasing, cu[n] = T, at most max_cps chunks in a
// sequence, nc chunks in all, and the fingerprint of its n + 1 entries equal
// to the host's.  A call that passes runs on the device lengths (now bounded
// by T and by the workspace).  One that fails runs as n empty sequences:
// every chunk entry empty, the copy all zero, so no kernel reads a token,
// o is not written and each final state is the initial one; the status
// word is then 1 (else 0).
__global__ __launch_bounds__(256) void schedule_kernel(const int32_t* cu, int n_seqs, int64_t nc,
                                                        int64_t T, int64_t max_cps, uint64_t hash,
                                                        int32_t* chunk_seq, int32_t* chunk_start,
                                                        int32_t* seq_chunk0, int32_t* cu_ok,
                                                        int32_t* seq_order, int32_t* status) {
  constexpr int kLds = kScheduleLdsSeqs;
  __shared__ int32_t sc[256];
  __shared__ int32_t cul[kLds + 1];  // the lengths (n <= kLds)
  __shared__ int32_t sc0[kLds + 1];  // first chunk of each sequence (n <= kLds)
  __shared__ unsigned long long red[3][4];  // per wave: fingerprint, chunks, failed checks
  const int t = threadIdx.x;
  const bool small = n_seqs <= kLds;
  uint64_t h = 0, cs = 0;
  int b = 0;
  for (int s = t; s <= n_seqs; s += 256) {
    const int32_t a = cu[s];
    if (small) cul[s] = a;
    h += drla_cu_mix((uint64_t)s, (uint32_t)a);
    if ((s == 0 && a != 0) || (s == n_seqs && (int64_t)a != T)) b = 1;
    if (s < n_seqs) {
      const int64_t L = (int64_t)cu[s + 1] - a;
      const int64_t c = L > 0 ? (L + C - 1) / C : 0;
      if (L < 0 || c > max_cps) b = 1;
      cs += (uint64_t)c;
    }
  }
  // sums over the workgroup: within each wave by shuffles, then the four
  // waves' partial sums through LDS (no atomics)
  uint64_t bb = (uint64_t)b;
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    h += __shfl_xor(h, off);
    cs += __shfl_xor(cs, off);
    bb |= __shfl_xor(bb, off);
  }
  if ((t & 63) == 0) {
    red[0][t >> 6] = h;
    red[1][t >> 6] = cs;
    red[2][t >> 6] = bb;
  }
  __syncthreads();
  const uint64_t h_sum = red[0][0] + red[0][1] + red[0][2] + red[0][3];
  const uint64_t c_sum = red[1][0] + red[1][1] + red[1][2] + red[1][3];
  const bool ok = (red[2][0] | red[2][1] | red[2][2] | red[2][3]) == 0 && h_sum == hash &&
                  c_sum == (uint64_t)nc;
  if (!ok) {
    for (int64_t c = t; c < nc; c += 256) {
      chunk_seq[c] = -1;
      chunk_start[c] = 0;
    }
    for (int s = t; s <= n_seqs; s += 256) {
      seq_chunk0[s] = 0;
      cu_ok[s] = 0;
      if (small && s < n_seqs) seq_order[s] = s;  // all empty: ranked by index
    }
    if (t == 0) status[0] = 1;
    return;
  }
  for (int s = t; s <= n_seqs; s += 256) cu_ok[s] = small ? cul[s] : cu[s];
  int64_t carry = 0;
  for (int base = 0; base < n_seqs; base += 256) {
    const int s = base + t;
    int cnt = 0;
    int64_t st = 0;
    if (s < n_seqs) {
      st = small ? cul[s] : cu[s];
      const int64_t L = (int64_t)(small ? cul[s + 1] : cu[s + 1]) - st;
      cnt = L > 0 ? (int)((L + C - 1) / C) : 0;
    }
    sc[t] = cnt;
    __syncthreads();
    for (int off = 1; off < 256; off <<= 1) {
      const int add = t >= off ? sc[t - off] : 0;
      __syncthreads();
      sc[t] += add;
      __syncthreads();
    }
    const int64_t excl = carry + sc[t] - cnt;
    if (s < n_seqs) {
      seq_chunk0[s] = (int32_t)excl;
      if (small) {
        sc0[s] = (int32_t)excl;
      } else {
        for (int j = 0; j < cnt; ++j) {
          const int64_t idx = excl + j;
          if (idx < nc) {
            chunk_seq[idx] = s;
            chunk_start[idx] = (int32_t)(st + (int64_t)C * j);
          }
        }
      }
    }
    carry += sc[255];
    __syncthreads();
  }
  if (t == 0) {
    seq_chunk0[n_seqs] = (int32_t)carry;
    status[0] = 0;
  }
  if (small) {
    // the sequences ranked longest first (ties by index) for the scan's
    // dealing order, from the lengths in LDS (larger batches: rank_kernel)
    for (int s = t; s < n_seqs; s += 256) {
      const int32_t mine = cul[s + 1] - cul[s];
      int rank = 0;
      for (int j = 0; j < n_seqs; ++j) {
        const int32_t l = cul[j + 1] - cul[j];
        rank += (l > mine || (l == mine && j < s)) ? 1 : 0;
      }
      seq_order[rank] = s;
    }
    // every thread a run of chunks: the sequence holding chunk c is the last
    // s with sc0[s] <= c (sc0[0] = 0 <= c < nc = sc0[n]), found by bisection
    if (t == 0) sc0[n_seqs] = (int32_t)carry;
    __syncthreads();
    for (int64_t c = t; c < nc; c += 256) {
      int lo = 0, hi = n_seqs;
      while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (sc0[mid] <= c) lo = mid;
        else hi = mid;
      }
      chunk_seq[c] = lo;
      chunk_start[c] = cul[lo] + (int32_t)(C * (c - sc0[lo]));
    }
  }
}

// Sequences ranked longest first (ties by index) for the scan's dealing
// order: one thread per sequence counts the longer ones, the lengths staged
// through LDS 256 at a time.  seq_order[rank] = sequence.
__global__ __launch_bounds__(256) void rank_kernel(const int32_t* cu, int n_seqs, int32_t* seq_order) {
  __shared__ int32_t lens[256];
  const int s = blockIdx.x * 256 + threadIdx.x;
  const int32_t mine = s < n_seqs ? cu[s + 1] - cu[s] : 0;
  int rank = 0;
  for (int base = 0; base < n_seqs; base += 256) {
    const int o = base + threadIdx.x;
    lens[threadIdx.x] = o < n_seqs ? cu[o + 1] - cu[o] : -1;
    __syncthreads();
    const int m = n_seqs - base < 256 ? n_seqs - base : 256;
    for (int i = 0; i < m; ++i) {
      const int32_t l = lens[i];
      rank += (l > mine || (l == mine && base + i < s)) ? 1 : 0;
    }
    __syncthreads();
  }
  if (s < n_seqs) seq_order[rank] = s;
}

// Position of element e (0..31) of a 32-element block in fragment order:
// element kmap(g, j) at 8g + j.
__device__ __forceinline__ int kpos(int e) { return 8 * ((e & 15) >> 2) + 4 * (e >> 4) + (e & 3); }

// A persistent grid of 256-thread workgroups walks the (chunk, value head)
// units.  PF: while a workgroup computes one unit, the loads of its next
// unit are in flight (K, Q, beta, g into registers).  KT: write K~^T (the
// register-fed scans need it; the LDS-fed one transposes K itself).
//
// KDA: every thread owns eight adjacent key channels and a run of GR rows of
// the chunk; it forms the cumulative gate B of its rows in registers (the
// runs' offsets come from one exclusive scan over the runs per channel) and
// writes B log2(e) to a table in LDS beside the raw K and Q rows.  The
// products A and P weigh every key channel by e^{B_r - B_i} (r >= i, so the
// exponent is never positive); each operand fragment is scaled as it is
// loaded, about a reference row chosen per 16-row tile so that no factor
// can overflow:
//   off-diagonal tiles (row tile I > column tile J): the first row of row
//     tile I, m = 16 I; X_r e^{B_r - B_m} and K_i e^{B_m - B_i} are both
//     at most |X_r|, |K_i| (any gate), and go to the 16-bit products;
//   diagonal tiles: the tile's row 16 I + 8; the factors lie within
//     e^{+-8 max|g|}, which bf16 and fp32 operands hold (fp16 ones go to
//     fp32 products, 16x16x4 fp32 MFMA), so the gate need only satisfy
//     8 |g| < 88 per token and channel.
// The scan's operands K e^{B}, Q e^{B}, (K e^{B_n - B})^T and e^{B_n}
// take non-positive exponents only.
//
// KDA's Q rows never go to LDS: each wave reads the row fragments of the Q
// tiles it multiplies straight into registers (and writes those tiles'
// Q e^{B}).  LDS is reused across phases: K (and KDA's B table) live until
// the chunk operands are written, T from the solve on, in the same bytes;
// KDA's A and the runs' totals take the bytes of the B table.
template <int DK, bool KDA, typename ET, bool KT, bool PF, bool G2>
__global__ __launch_bounds__(256, sizeof(ET) == 2 ? 2 : 1) void prep_kernel(PrepParams P, int64_t nunits) {
  static_assert(!(KDA && PF), "KDA: one unit per workgroup (its Q fragments stay in registers)");
  typedef typename VT<ET>::v8 V8;
  typedef typename VT<ET>::v16b V16;
  constexpr int PE = VT<ET>::per16;
  constexpr int KB = DK / 32;
  constexpr int KP = DK + 16 / (int)sizeof(ET);  // padded row: 16-byte aligned, 4-bank skew
  constexpr int TP = C + 4;
  constexpr int CG = DK / 8;                     // KDA gate: groups of 8 channels
  constexpr int GP = 256 / CG;                   // KDA gate: runs of rows per channel
  constexpr int GR = C / GP;                     // KDA gate: rows per run
  constexpr bool LF = !KDA && !KT;               // operands for the LDS-fed scan
  static_assert(!LF || sizeof(ET) == 2, "the LDS-fed scans take 16-bit inputs");
  static_assert(!G2 || LF, "value heads in pairs: the LDS-fed scans' operands only");
  constexpr int NG = G2 ? 2 : 1;                 // value heads per unit (G2: a pair sharing K, Q)
  constexpr int KV = DK / PE;                    // 16-byte pieces per K row
  constexpr int NKV = C * KV / 256;              // K pieces per thread
  constexpr int KS_BYTES = C * KP * (int)sizeof(ET);
  constexpr int TS_BYTES = C * TP * 4;
  constexpr int BP = DK + 4;                     // KDA: padded row of the B table (floats)
  constexpr int BL_BYTES = KDA ? C * BP * 4 : 0;
  static_assert(!KDA || (BL_BYTES >= C * TP * 4 && BL_BYTES >= 256 / (DK / 8) * DK * 4),
                "KDA: A and the runs' totals fit in the bytes of the B table");
  // KDA: the B table (then A) after the larger of the K rows and T, so that
  // the solve's A and T never share bytes
  constexpr int BL_OFF = KS_BYTES > TS_BYTES ? KS_BYTES : TS_BYTES;
  constexpr int U_BYTES = KDA ? BL_OFF + BL_BYTES : (KS_BYTES > TS_BYTES ? KS_BYTES : TS_BYTES);
  __shared__ __attribute__((aligned(16))) unsigned char un[U_BYTES];
  __shared__ __attribute__((aligned(16))) float As_st[KDA ? 1 : C][TP];  // A (GDN)
  __shared__ __attribute__((aligned(16))) float bs[NG][C];     // per value head of the unit
  __shared__ __attribute__((aligned(16))) float betas[NG][C];
  __shared__ floatx4 pxch[KDA ? 64 : 1];  // KDA: one P^T tile passed between waves
  ET(*Ks)[KP] = (ET(*)[KP])un;                   // K rows (phases 0-1)
  float(*Bl)[BP] = (float(*)[BP])(un + BL_OFF);  // KDA: B log2(e) (phases 0-1)
  float(*As)[TP] = KDA ? (float(*)[TP])(un + BL_OFF) : As_st;  // A (KDA: in the B table's bytes)
  float(*Ts)[TP] = (float(*)[TP])un;             // T (phase 2 on)

  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int g4 = lane >> 4, c16 = lane & 15;
  const ET* kg = (const ET*)P.k;
  const ET* qg = (const ET*)P.q;
  const int pr = 3 - wv;  // this wave's row tile of P
  const int rq = 16 * pr + c16;

  struct Unit {
    int h, hk, len;
    int64_t t0, ch;
  };
  auto unit_of = [&](int64_t u) {
    Unit U;
    const int64_t hu = u / P.nc;
    const int64_t c = u - hu * P.nc;
    U.h = (int)hu * NG;  // G2: the pair's first value head
    int seq;
    chunk_of(P.s, c, seq, U.t0, U.len);
    U.hk = U.h / P.grp;
    U.ch = (int64_t)U.h * P.nc + c;
    return U;
  };
  // a unit's inputs in registers; tokens past the sequence end read as zero
  // (beta = g = 0: they write nothing and do not decay)
  V16 kpre[NKV];
  // KDA: Q row fragments (key channels 32p + 8g .. +7 of row 16 t + c) of
  // row tile qt_a = (w + 3) mod 4, whose P^T tiles and Q e^{B} this wave
  // forms, and of qt_b, the other row tile it multiplies (waves 1 and 3)
  V8 qa[KDA ? KB : 1], qb[KDA ? KB : 1];
  const int qt_a = (wv + 3) & 3, qt_b = wv == 1 ? 2 : wv == 3 ? 3 : qt_a;
  V8 qpre[KDA ? 1 : KB];     // GDN: Q fragments of this wave's P tile
  float bpre = 0.f, gpre = 0.f;
  floatx4 gvpre[KDA ? GR : 1][2];  // KDA: gates of this thread's rows and 8 channels
  auto load = [&](const Unit& U) {
#pragma unroll
    for (int i = 0; i < NKV; ++i) {
      const int idx = tid + 256 * i, r = idx / KV, cv = idx - r * KV;
      V16 x = {};
      if (r < U.len) x = *(const V16*)(kg + ((U.t0 + r) * P.h_qk + U.hk) * DK + cv * PE);
      kpre[i] = x;
    }
    if (KDA) {
      const int ra = 16 * qt_a + c16, rb = 16 * qt_b + c16;
#pragma unroll
      for (int p = 0; p < KB; ++p) {
        V8 x = {}, y = {};
        if (ra < U.len) x = *(const V8*)(qg + ((U.t0 + ra) * P.h_qk + U.hk) * DK + 32 * p + 8 * g4);
        if (rb < U.len) y = *(const V8*)(qg + ((U.t0 + rb) * P.h_qk + U.hk) * DK + 32 * p + 8 * g4);
        qa[p] = x;
        qb[p] = y;
      }
    } else {
#pragma unroll
      for (int p = 0; p < KB; ++p) {
        V8 x = {};
        if (rq < U.len) x = row_slots<ET>(qg + ((U.t0 + rq) * P.h_qk + U.hk) * DK + 32 * p, g4);
        qpre[p] = x;
      }
    }
    // wave m < NG: row `lane` of value head U.h + m
    if (tid < NG * C) {
      bpre = lane < U.len ? (P.decay_only ? 1.f : P.beta[(U.t0 + lane) * P.h_v + U.h + wv]) : 0.f;
      if (!KDA) gpre = lane < U.len ? P.g[(U.t0 + lane) * P.h_v + U.h + wv] : 0.f;
    }
    if (KDA) {
      const int d0 = 8 * (tid % CG), part = tid / CG;
#pragma unroll
      for (int i = 0; i < GR; ++i) {
        const int r = part * GR + i;
        gvpre[i][0] = gvpre[i][1] = zero4();
        if (r < U.len) {
          const floatx4* gp = (const floatx4*)(P.g + ((U.t0 + r) * P.h_v + U.h) * DK + d0);
          gvpre[i][0] = gp[0];
          gvpre[i][1] = gp[1];
        }
      }
    }
  };

  // PF: a persistent grid; otherwise one unit per workgroup, dealt in
  // reverse chunk-major order: the units written last are the first chunks
  // of every head, which the scans read first (the last-level cache keeps
  // the most recent writes)
  int64_t u = blockIdx.x;
  if constexpr (!PF) {
    const int64_t hus = nunits / P.nc, r = nunits - 1 - u;
    u = (r % hus) * P.nc + r / hus;
  }
  Unit U = unit_of(u);
  load(U);
  for (;;) {
    [[maybe_unused]] const int len = U.len;
    [[maybe_unused]] const int64_t t0 = U.t0;
    const int64_t ch = U.ch;

    // ---- phase 0: stage the unit, start loading the next one -------------------
    V8 qf[KB];
    if (!KDA) {
#pragma unroll
      for (int p = 0; p < KB; ++p) qf[p] = qpre[KDA ? 0 : p];
    }
#pragma unroll
    for (int i = 0; i < NKV; ++i) {
      const int idx = tid + 256 * i, r = idx / KV, cv = idx - r * KV;
      if (LF) {
        // fragment order within each 32-element block: the 8 elements one
        // lane of group g takes (4g..4g+3, 16+4g..16+4g+3) sit at 8g..8g+7
        const int e0 = (cv * PE) & 31, base = (cv * PE) - e0;
        typedef typename VT<ET>::v4 V4;
        const V16 x = kpre[i];
        const V4 lo = {x[0], x[1], x[2], x[3]}, hi = {x[4], x[5], x[6], x[7]};
        *(V4*)&Ks[r][base + kpos(e0)] = lo;
        *(V4*)&Ks[r][base + kpos(e0 + 4)] = hi;
      } else {
        *(V16*)&Ks[r][cv * PE] = kpre[i];
      }
    }
    // #1 Gate: in-chunk prefix sums of the log-decay
    if (tid < NG * C) {
      betas[wv][lane] = bpre;
      if (!KDA) {
        float x = gpre;
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
          const float y = __shfl_up(x, off);
          if (lane >= off) x += y;
        }
        bs[wv][lane] = x;
      }
    }
    // KDA: per key channel, GP runs of GR rows; prefix sums in registers,
    // the runs' totals to LDS (in the bytes A takes later)
    floatx4 bv[KDA ? GR : 1][2];
    float* const Bt = &As[0][0];  // [GP][DK] run totals, then their exclusive prefix
    if (KDA) {
      const int d0 = 8 * (tid % CG), part = tid / CG;
      floatx4 run0 = zero4(), run1 = zero4();
#pragma unroll
      for (int i = 0; i < GR; ++i) {
        run0 += gvpre[i][0];
        run1 += gvpre[i][1];
        bv[i][0] = run0;
        bv[i][1] = run1;
      }
      *(floatx4*)&Bt[part * DK + d0] = run0;
      *(floatx4*)&Bt[part * DK + d0 + 4] = run1;
    }
    const int64_t unext = u + gridDim.x;
    Unit Un = U;
    if (unext < nunits) {
      Un = unit_of(unext);
      if (PF) load(Un);
    }
    __syncthreads();
    if (KDA) {
      // one thread per key channel: the runs' exclusive prefix (in place)
      // and e^{B_n} (rows past the end of the chunk carry the last B)
      if (tid < DK) {
        float acc = 0.f;
#pragma unroll
        for (int q2 = 0; q2 < GP; ++q2) {
          const float tq = Bt[q2 * DK + tid];
          Bt[q2 * DK + tid] = acc;
          acc += tq;
        }
        P.gam[ch * DK + tid] = __expf(acc);
      }
      __syncthreads();
      const int d0 = 8 * (tid % CG), part = tid / CG;
      const floatx4 o0 = *(const floatx4*)&Bt[part * DK + d0];
      const floatx4 o1 = *(const floatx4*)&Bt[part * DK + d0 + 4];
      __syncthreads();  // the runs' totals are read; the B table takes their bytes
      constexpr float kLog2e = 1.4426950408889634f;
#pragma unroll
      for (int i = 0; i < GR; ++i) {
        const int r = part * GR + i;
        *(floatx4*)&Bl[r][d0] = (bv[i][0] + o0) * kLog2e;
        *(floatx4*)&Bl[r][d0 + 4] = (bv[i][1] + o1) * kLog2e;
      }
      __syncthreads();
    }

    // the value head being finished (G2: each of the pair in turn) and its
    // gate and beta tables
    const float* bsv = &bs[0][0];
    const float* betv = &betas[0][0];
    int64_t chm = ch;

    // ---- phase 1: products and the chunk operands --------------------------------
    // GDN: K row fragment of token tile t, inner block p
    auto kfrag = [&](int t, int p) -> V8 {
      const int r = 16 * t + c16;
      if (LF) return *(const V8*)&Ks[r][32 * p + 8 * g4];
      return row_slots<ET>(&Ks[r][32 * p], g4);
    };
    // KDA: fragment of row `xrow` (K or Q) at the eight contiguous key
    // channels d .. d + 7, each weighted by 2^{x}, x = brow - bref (right:
    // bref - brow) in the B table's units; the caller picks bref so that
    // x <= 0
    typedef typename VT<ET>::v4 V4;
    auto kda_frag = [&](const ET* xrow, const float* brow, const float* bref, int d, bool right) -> V8 {
      const V4 x0 = *(const V4*)(xrow + d), x1 = *(const V4*)(xrow + d + 4);
      const floatx4 b0 = *(const floatx4*)(brow + d), b1 = *(const floatx4*)(brow + d + 4);
      const floatx4 r0 = *(const floatx4*)(bref + d), r1 = *(const floatx4*)(bref + d + 4);
      V8 y;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        y[j] = (ET)(to_f(x0[j]) * __builtin_amdgcn_exp2f(right ? r0[j] - b0[j] : b0[j] - r0[j]));
        y[j + 4] = (ET)(to_f(x1[j]) * __builtin_amdgcn_exp2f(right ? r1[j] - b1[j] : b1[j] - r1[j]));
      }
      return y;
    };

    // P of this wave's row tile as B fragments of P^T (kept for the LDS-fed
    // scan's form, which stores P Tb instead of P)
    V8 pfr[2];
    // #2 KKT (row tile w of A) and the output Map's P (row tile 3 - w)
    const int rt = wv;
    floatx4 acc[4], pt[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      acc[t] = zero4();
      pt[t] = zero4();
    }
    if constexpr (KDA) {
      // Tiles of A (row tile I, column tile J <= I) and of P^T (J, I), each
      // factored about a reference row of its own so that no factor
      // overflows:
      //   J < I: the row tile's first row m = 16 I; rows (K and Q of tile I)
      //     X_r e^{B_r - B_m}, columns K_i e^{B_m - B_i}, every factor at
      //     most 1 for any gate; 16-bit products;
      //   J = I: the tile's row c = 16 I + 8; factors within e^{+-8 max|g|},
      //     products in the operand type (bf16 and fp32 hold them; fp32
      //     products for fp16 operands).
      // A tile and its P^T tile share their column operand and the K and Q
      // rows of a tile share their factors, so a wave takes whole row tiles
      // and diagonals, balanced by their exponentials (per lane and inner
      // block: 8 per row tile, 8 per column tile, 16 per diagonal):
      //   wave 0: row tile 3 against column tiles 0, 1, 2;
      //   wave 1: row tile 2 against 0, 1, and diagonal 0;
      //   wave 2: row tile 1 against 0, and diagonal 1;
      //   wave 3: diagonals 2 and 3.
      // acc[] and pt[] hold the wave's A and P^T tiles in that order.
      constexpr bool kF32Diag = std::is_same<ET, f16>::value;
      typedef typename std::conditional<kF32Diag, floatx8, V8>::type DV8;
      // 2^{+-(Bl[r] - Bl[m])} at channels d .. d + 7
      auto factors = [&](int r, int m, int d, bool right) -> floatx8 {
        const floatx4 b0 = *(const floatx4*)&Bl[r][d], b1 = *(const floatx4*)&Bl[r][d + 4];
        const floatx4 m0 = *(const floatx4*)&Bl[m][d], m1 = *(const floatx4*)&Bl[m][d + 4];
        floatx8 f;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          f[j] = __builtin_amdgcn_exp2f(right ? m0[j] - b0[j] : b0[j] - m0[j]);
          f[j + 4] = __builtin_amdgcn_exp2f(right ? m1[j] - b1[j] : b1[j] - m1[j]);
        }
        return f;
      };
      auto scaled = [&](const ET* xrow, int d, const floatx8& f) -> V8 {
        const V4 x0 = *(const V4*)(xrow + d), x1 = *(const V4*)(xrow + d + 4);
        V8 y;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          y[j] = (ET)(to_f(x0[j]) * f[j]);
          y[j + 4] = (ET)(to_f(x1[j]) * f[j + 4]);
        }
        return y;
      };
      // the same for a fragment held in registers (KDA's Q rows)
      auto scaled_v = [&](const V8& x, const floatx8& f) -> V8 {
        V8 y;
#pragma unroll
        for (int j = 0; j < 8; ++j) y[j] = (ET)(to_f(x[j]) * f[j]);
        return y;
      };
      auto scaled_vd = [&](const V8& x, const floatx8& f) -> DV8 {
        if constexpr (kF32Diag) {
          floatx8 y;
#pragma unroll
          for (int j = 0; j < 8; ++j) y[j] = to_f(x[j]) * f[j];
          return y;
        } else {
          return scaled_v(x, f);
        }
      };
      auto scaled_d = [&](const ET* xrow, int d, const floatx8& f) -> DV8 {
        if constexpr (kF32Diag) {
          const V4 x0 = *(const V4*)(xrow + d), x1 = *(const V4*)(xrow + d + 4);
          floatx8 y;
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            y[j] = to_f(x0[j]) * f[j];
            y[j + 4] = to_f(x1[j]) * f[j + 4];
          }
          return y;
        } else {
          return scaled(xrow, d, f);
        }
      };
      // row tile I (its Q fragment q) against column tiles 0 .. nj-1, into
      // acc[0 .. nj), pt[0 .. nj)
      auto offdiag = [&](int I, int nj, int d, const V8& q) {
        const int r = 16 * I + c16, m = 16 * I;
        const floatx8 f = factors(r, m, d, false);
        const V8 kr = scaled(&Ks[r][0], d, f), qr = scaled_v(q, f);
#pragma unroll
        for (int t = 0; t < 3; ++t) {
          if (t < nj) {
            const V8 kc = kda_frag(&Ks[16 * t + c16][0], &Bl[16 * t + c16][0], &Bl[m][0], d, true);
            acc[t] = mma(kr, kc, acc[t]);
            pt[t] = mma(kc, qr, pt[t]);
          }
        }
      };
      // diagonal tile I (its Q fragment q), into acc[sl], pt[sl]
      auto diag = [&](int I, int sl, int d, const V8& q) {
        const int r = 16 * I + c16, c = 16 * I + 8;
        const floatx8 f = factors(r, c, d, false), gi = factors(r, c, d, true);
        const DV8 kg = scaled_d(&Ks[r][0], d, gi);
        acc[sl] = mma(scaled_d(&Ks[r][0], d, f), kg, acc[sl]);
        pt[sl] = mma(kg, scaled_vd(q, f), pt[sl]);
      };
#pragma unroll
      for (int p = 0; p < KB; ++p) {
        const int d = 32 * p + 8 * g4;
        if (wv == 0) {
          offdiag(3, 3, d, qa[p]);
        } else if (wv == 1) {
          offdiag(2, 2, d, qb[p]);
          diag(0, 2, d, qa[p]);
        } else if (wv == 2) {
          offdiag(1, 1, d, qa[p]);
          diag(1, 1, d, qa[p]);
        } else {
          diag(2, 0, d, qa[p]);
          diag(3, 1, d, qb[p]);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
      if (wv == 0) pxch[lane] = pt[2];  // P^T tile (2, 3), packed by wave 3
    } else {
      // Every wave multiplies its row tile with all four column tiles (the
      // products past the diagonal are dropped), so all K fragments are read
      // from LDS at once and no branch splits the reads from the products.
      V8 ar[KB], kc[4][KB];
#pragma unroll
      for (int p = 0; p < KB; ++p) ar[p] = kfrag(rt, p);
#pragma unroll
      for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int p = 0; p < KB; ++p) kc[t][p] = kfrag(t, p);
#pragma unroll
      for (int p = 0; p < KB; ++p)
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          acc[t] = mma(ar[p], kc[t][p], acc[t]);  // A tile (rt, t)
          pt[t] = mma(kc[t][p], qf[p], pt[t]);    // P^T tile (t, pr) = K_t Q_pr^T
        }
    }
    // A and P from the products: A to LDS for the solve, P to the workspace
    // (KDA: after the chunk operands below, whose reads of the B table must
    // end before A takes its bytes)
    auto store_ap = [&]() {
      // A: strictly lower part, scaled by beta_r (and e^{b_r - b_i} for GDN);
      // tiles past the diagonal are never read.  The gate values come from
      // LDS once per lane: this lane's four rows as one vector, one column
      // per tile.
      const floatx4 betr = *(const floatx4*)&betv[16 * rt + 4 * g4];
      const floatx4 bsr = *(const floatx4*)&bsv[16 * rt + 4 * g4];
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        if (t > rt) continue;
        const float bsi = bsv[16 * t + c16];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int r = 16 * rt + 4 * g4 + e, i = 16 * t + c16;
          float x = 0.f;
          if (i < r && !P.decay_only) {
            x = betr[e] * acc[t][e];
            if (!KDA) x *= __expf(bsr[e] - bsi);
          }
          As[r][i] = x;
        }
      }
      // P: tiles jt = 2p, 2p+1 of P^T form fragment (pr, p) of P (outer =
      // query token, inner = key token); inclusive lower part only
      const float bsq = bsv[rq];
      // (the raw products stay: G2 gates them again for the second head)
      floatx4 pg4[4];
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const floatx4 bsj = *(const floatx4*)&bsv[16 * t + 4 * g4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int j = 16 * t + 4 * g4 + e;
          float x = 0.f;
          if (j <= rq) x = KDA ? pt[t][e] : pt[t][e] * __expf(bsq - bsj[e]);
          pg4[t][e] = x;
        }
      }
      pfr[0] = pack<ET>(pg4[0], pg4[1]);
      pfr[1] = pack<ET>(pg4[2], pg4[3]);
      if (!LF) {
        V8* pg = (V8*)P.pm + chm * (8 * 64);
        pg[(pr * 2 + 0) * 64 + lane] = pfr[0];
        if (pr >= 2) pg[(pr * 2 + 1) * 64 + lane] = pfr[1];  // (0, 1), (1, 1): zero, never read
      }
    };
    // KDA: the tiles of the wave's assignment above
    auto store_ap_kda = [&]() {
      auto put_a = [&](int I, int J, const floatx4& v) {
        const floatx4 betr = *(const floatx4*)&betv[16 * I + 4 * g4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int r = 16 * I + 4 * g4 + e, i = 16 * J + c16;
          As[r][i] = (i < r && !P.decay_only) ? betr[e] * v[e] : 0.f;
        }
      };
      // diagonal P^T tile (I, I): keys j <= query r
      auto mask_p = [&](floatx4 v) -> floatx4 {
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (4 * g4 + e > c16) v[e] = 0.f;
        return v;
      };
      V8* pg = (V8*)P.pm + ch * (8 * 64);
      const floatx4 z = zero4();
      // fragment (I, p) of P: P^T tiles J = 2p, 2p + 1 of row tile I
      if (wv == 0) {
        put_a(3, 0, acc[0]);
        put_a(3, 1, acc[1]);
        put_a(3, 2, acc[2]);
        pg[6 * 64 + lane] = pack<ET>(pt[0], pt[1]);
      } else if (wv == 1) {
        put_a(2, 0, acc[0]);
        put_a(2, 1, acc[1]);
        put_a(0, 0, acc[2]);
        pg[4 * 64 + lane] = pack<ET>(pt[0], pt[1]);
        pg[0 * 64 + lane] = pack<ET>(mask_p(pt[2]), z);
      } else if (wv == 2) {
        put_a(1, 0, acc[0]);
        put_a(1, 1, acc[1]);
        pg[2 * 64 + lane] = pack<ET>(pt[0], mask_p(pt[1]));
      } else {
        put_a(2, 2, acc[0]);
        put_a(3, 3, acc[1]);
        pg[5 * 64 + lane] = pack<ET>(mask_p(pt[0]), z);
        pg[7 * 64 + lane] = pack<ET>(pxch[lane], mask_p(pt[1]));
      }
    };
    // G2: the pair's two value heads share the K and Q rows and the raw
    // products; each is gated, solved and written in turn
    for (int mj = 0; mj < NG; ++mj) {
      if (mj > 0) {
        __syncthreads();  // the first head's T and staged Tb are read
        bsv = &bs[mj][0];
        betv = &betas[mj][0];
        chm = ch + (int64_t)mj * P.nc;
      }
      if (!KDA) store_ap();
      // K~^T = (e^{b_n - b} (.) K)^T in fragments (outer = the 16 key channels
      // of state tile mt in the scan's row order, inner = token block p);
      // KDA: K (.) e^{B_n - B}
      if (KT) {
        constexpr int NF = (DK / 16) * 2;
        V8* ktg = (V8*)P.kt + ch * (int64_t)(C * DK / 8);
        for (int f = wv; f < NF; f += 4) {
          const int mt = f >> 1, p = f & 1;
          const int d = state_row(mt, c16);
          V8 x;
  #pragma unroll
          for (int j = 0; j < 8; ++j) {
            const int i = 32 * p + kmap(g4, j);
            x[j] = KDA ? (ET)(to_f(Ks[i][d]) * __builtin_amdgcn_exp2f(Bl[C - 1][d] - Bl[i][d]))
                       : (ET)(to_f(Ks[i][d]) * __expf(bsv[C - 1] - bsv[i]));
          }
          ktg[f * 64 + lane] = x;
        }
      }
      if (KDA) {
        // K e^{B} and Q e^{B} as row fragments (token tile nt, inner block p)
        // with contiguous key channels 32p + 8g + j, the scan's state order;
        // each wave writes token tile qt_a, whose Q rows it holds
        V8* kwg = (V8*)P.kw + ch * (int64_t)(C * DK / 8);
        V8* qwg = (V8*)P.qw + ch * (int64_t)(C * DK / 8);
  #pragma unroll
        for (int p = 0; p < KB; ++p) {
          const int f = qt_a * KB + p;
          const int r = 16 * qt_a + c16, d = 32 * p + 8 * g4;
          const V4 k0 = *(const V4*)&Ks[r][d], k1 = *(const V4*)&Ks[r][d + 4];
          const floatx4 b0 = *(const floatx4*)&Bl[r][d], b1 = *(const floatx4*)&Bl[r][d + 4];
          V8 xk, xq;
  #pragma unroll
          for (int j = 0; j < 4; ++j) {
            const float e0 = __builtin_amdgcn_exp2f(b0[j]), e1 = __builtin_amdgcn_exp2f(b1[j]);
            xk[j] = (ET)(to_f(k0[j]) * e0);
            xq[j] = (ET)(to_f(qa[p][j]) * e0);
            xk[j + 4] = (ET)(to_f(k1[j]) * e1);
            xq[j + 4] = (ET)(to_f(qa[p][j + 4]) * e1);
          }
          kwg[f * 64 + lane] = xk;
          qwg[f * 64 + lane] = xq;
        }
        __syncthreads();  // the B table is read; A takes its bytes
        store_ap_kda();
      } else if (tid < C) {
        // GDN: e^{b_r} and e^{b_n - b_r} of every row; row 63 of the first
        // holds e^{b_n} (rows past the end carry the last b)
        P.gam[chm * (2 * C) + tid] = __expf(bsv[tid]);
        P.gam[chm * (2 * C) + C + tid] = __expf(bsv[C - 1] - bsv[tid]);
      }
      __syncthreads();  // K and the gate table are dead from here; T takes their bytes

      // ---- phase 2: #3 Solve --------------------------------------------------------
      if (wv == 0) {
        // level 0: the four 16x16 diagonal blocks of T by forward substitution,
        // one column per lane (block lane/16, column lane%16).  Rows of A are
        // read four entries at a time, LA rows ahead of the row being solved,
        // so that the 16-step chain does not wait on each row's reads; four
        // partial sums per row.
        constexpr int LA = 3;
        const int bb = lane >> 4, cc = lane & 15, o = 16 * bb;
        floatx4 ar[16][4];
        auto read_row = [&](int r) {
  #pragma unroll
          for (int i4 = 0; i4 < (r + 3) / 4; ++i4) ar[r][i4] = *(const floatx4*)&As[o + r][o + 4 * i4];
        };
  #pragma unroll
        for (int r = 1; r <= LA; ++r) read_row(r);
        float t[16];
  #pragma unroll
        for (int r = 0; r < 16; ++r) {
          if (r >= 1 && r + LA < 16) read_row(r + LA);
          float acc[4] = {(r == cc) ? 1.f : 0.f, 0.f, 0.f, 0.f};
  #pragma unroll
          for (int i4 = 0; i4 < (r + 3) / 4; ++i4) {
  #pragma unroll
            for (int e = 0; e < 4; ++e)
              if (4 * i4 + e < r) acc[e] -= ar[r][i4][e] * t[4 * i4 + e];
          }
          t[r] = (acc[0] + acc[1]) + (acc[2] + acc[3]);
        }
  #pragma unroll
        for (int r = 0; r < 16; ++r) Ts[o + r][o + cc] = t[r];
      } else {
        // the upper off-diagonal 16x16 blocks of T are zero
        for (int idx = tid - 64; idx < 6 * 256; idx += 192) {
          const int blk = idx >> 8, e = idx & 255;
          const int bi = blk < 3 ? 0 : (blk < 5 ? 1 : 2);
          const int bj = blk < 3 ? blk + 1 : (blk < 5 ? blk - 1 : 3);
          Ts[16 * bi + (e >> 4)][16 * bj + (e & 15)] = 0.f;
        }
      }
      __syncthreads();

      // level 1: T_10 = -T_11 A_10 T_00 and T_32 = -T_33 A_32 T_22 (16-wide
      // contractions, zero-padded to the 32-wide fragment)
      if (wv < 2) {
        const int b0 = 16 * (2 * wv), b1 = b0 + 16;
        V8 a = {}, tb = {}, tl = {};
  #pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int k = 4 * g4 + j;
          a[j] = (ET)As[b1 + c16][b0 + k];
          tb[j] = (ET)Ts[b0 + k][b0 + c16];
          tl[j] = (ET)Ts[b1 + c16][b1 + k];
        }
        const floatx4 y = mma(a, tb, zero4());  // Y = A_10 T_00
        V8 yb = {};
  #pragma unroll
        for (int j = 0; j < 4; ++j) yb[j] = (ET)y[j];
        const floatx4 t = mma(tl, yb, zero4());  // T_11 Y
  #pragma unroll
        for (int e = 0; e < 4; ++e) Ts[b1 + 4 * g4 + e][b0 + c16] = -t[e];
      }
      __syncthreads();

      // level 2: rows 32..63 x columns 32jt..32jt+15 = -T2 (A21 T1), where T1
      // and T2 are the finished 32x32 diagonal halves
      if (wv < 2) {
        const int jt = wv;
        floatx4 z[2];
  #pragma unroll
        for (int m = 0; m < 2; ++m) {
          const int r = 32 + 16 * m + c16;
          V8 a, tb;
  #pragma unroll
          for (int j = 0; j < 8; ++j) {
            const int k = kmap(g4, j);
            a[j] = (ET)As[r][k];
            tb[j] = (ET)Ts[k][16 * jt + c16];
          }
          z[m] = mma(a, tb, zero4());
        }
        const V8 zb = pack<ET>(z[0], z[1]);
  #pragma unroll
        for (int m = 0; m < 2; ++m) {
          const int r = 32 + 16 * m + c16;
          V8 tl;
  #pragma unroll
          for (int j = 0; j < 8; ++j) tl[j] = (ET)Ts[r][32 + kmap(g4, j)];
          const floatx4 t = mma(tl, zb, zero4());
  #pragma unroll
          for (int e = 0; e < 4; ++e) Ts[32 + 16 * m + 4 * g4 + e][16 * jt + c16] = -t[e];
        }
      }
      __syncthreads();

      // #4: Tb = T diag(beta) as fragments (outer = token tile nt, inner = token
      // block p), eight per (chunk, head); the ones above the diagonal are zero.
      // LF: diag(e^{b_n - b}) Tb instead (the scan then forms e^{b_n - b} (.) V'
      // directly), and Tb itself staged in the io type, row-major, in the bytes
      // of A for P Tb below.  A lane's eight entries of a fragment are two runs
      // of four columns (kmap), read as two vectors of T and of beta.
      constexpr int TBP = C + 8;  // LF: padded row of the staged Tb (io type)
      ET(*TbL)[TBP] = (ET(*)[TBP])&As[0][0];
      static_assert(!LF || C * TBP * sizeof(ET) <= sizeof(float) * C * TP, "staged Tb fits in the bytes of A");
      {
        const int nt = wv, r = 16 * nt + c16;
        const float en = LF ? __expf(bsv[C - 1] - bsv[r]) : 1.f;
        V8* tg = (V8*)P.tb + chm * (8 * 64);
  #pragma unroll
        for (int p = 0; p < 2; ++p) {
          const int c0 = 32 * p + 4 * g4, c1 = c0 + 16;
          const floatx4 t0 = *(const floatx4*)&Ts[r][c0], t1 = *(const floatx4*)&Ts[r][c1];
          const floatx4 b0 = *(const floatx4*)&betv[c0], b1 = *(const floatx4*)&betv[c1];
          V8 x;
          V4 y0, y1;
  #pragma unroll
          for (int j = 0; j < 4; ++j) {
            const float u0 = t0[j] * b0[j], u1 = t1[j] * b1[j];
            x[j] = (ET)(u0 * en);
            x[j + 4] = (ET)(u1 * en);
            y0[j] = (ET)u0;
            y1[j] = (ET)u1;
          }
          if constexpr (LF) {
            *(V4*)&TbL[r][c0] = y0;
            *(V4*)&TbL[r][c1] = y1;
          }
          // fragments (0, 1) and (1, 1) lie above the diagonal: zero, and no
          // scan reads them, so they are not stored
          if (2 * p <= nt) tg[(nt * 2 + p) * 64 + lane] = x;
        }
      }
      if constexpr (LF) {
        // P Tb for the output Map (the scan multiplies it with R = V - e^b X):
        // tiles (it, pr) of (P Tb)^T = Tb^T P^T, packed in pairs into fragment
        // (pr, p) with P's layout (outer = query token, inner = token).  The
        // Tb^T fragments come from the staged rows by transposing reads: lane
        // (c, g) gets Tb[32p + 4g + j][16 it + c] (and rows + 16), j = 0..3.
        __syncthreads();
        floatx4 ptt[4];
  #pragma unroll
        for (int it = 0; it < 4; ++it) {
          ptt[it] = zero4();
  #pragma unroll
          for (int p = 0; p < 2; ++p) {
            const int rr = 32 * p + 4 * g4 + (c16 >> 2), cc = 16 * it + 4 * (c16 & 3);
            const V4 lo = lds_read_tr16<ET>(&TbL[rr][cc]), hi = lds_read_tr16<ET>(&TbL[rr + 16][cc]);
            ptt[it] = mma(cat<ET>(lo, hi), pfr[p], ptt[it]);
          }
        }
        V8* pg = (V8*)P.pm + chm * (8 * 64);
        pg[(pr * 2 + 0) * 64 + lane] = pack<ET>(ptt[0], ptt[1]);
        if (pr >= 2) pg[(pr * 2 + 1) * 64 + lane] = pack<ET>(ptt[2], ptt[3]);
      }
    }
    if (!PF) break;
    u += gridDim.x;
    if (u >= nunits) break;
    __syncthreads();  // T is read; the next unit's K takes its bytes
    U = Un;
  }
}

// Workgroups of one prep kernel variant that fit on the chip at once (cached
// per variant and device: the variants differ in registers and LDS).  Host
// threads may race to fill an entry; they all compute the same value.
template <int DK, bool KDA, typename ET, bool KT, bool PF, bool G2>
static int64_t resident_groups() {
  auto kern = prep_kernel<DK, KDA, ET, KT, PF, G2>;
  static std::atomic<int64_t> cached[16];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 16) dev = 0;
  int64_t fit = cached[dev].load(std::memory_order_relaxed);
  if (fit == 0) {
    int per_cu = 0, cus = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kern, 256, 0) != hipSuccess || per_cu < 1)
      per_cu = 1;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 1)
      cus = 256;
    fit = (int64_t)per_cu * cus;
    cached[dev].store(fit, std::memory_order_relaxed);
  }
  return fit;
}

// One-unit workgroups hold no next unit's loads in registers, so where
// registers set the occupancy (GDN) about twice as many fit per CU as in the
// persistent grid, and they win at every size; the persistent grid, which
// loads a workgroup's next unit while it computes the current one, is taken
// only where it fits as many per CU and the units do not all fit at once.
// KDA always takes one unit per workgroup: its Q fragments stay in
// registers, and without Q rows in LDS three workgroups fit per CU at
// dk = 128 (16-bit inputs) against two in the persistent grid.
template <int DK, bool KDA, typename ET, bool KT, bool G2 = false>
static hipError_t launch_prep_v(const PrepParams& P, int64_t nblk, hipStream_t st) {
  if constexpr (!KDA) {
    const int64_t fit1 = resident_groups<DK, KDA, ET, KT, false, G2>();
    const int64_t fit = resident_groups<DK, KDA, ET, KT, true, G2>();
    if (nblk > fit1 && fit1 <= fit) {
      const dim3 grid((unsigned)(nblk < fit ? nblk : fit));
      hipLaunchKernelGGL((prep_kernel<DK, KDA, ET, KT, true, G2>), grid, dim3(256), 0, st, P, nblk);
      return hipGetLastError();
    }
  }
  if (nblk > 0x7fffffff) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL((prep_kernel<DK, KDA, ET, KT, false, G2>), dim3((unsigned)nblk), dim3(256), 0, st, P, nblk);
  return hipGetLastError();
}

template <int DK, bool KDA, typename ET>
hipError_t launch_prep(const PrepParams& P, int64_t nblk, hipStream_t st) {
  if (nblk <= 0) return hipGetLastError();
  // fp32 inputs always take the register-fed scan, which needs K~^T
  if constexpr (KDA || sizeof(ET) == 4)
    return launch_prep_v<DK, KDA, ET, true>(P, nblk, st);
  else if (P.kt)
    return launch_prep_v<DK, false, ET, true>(P, nblk, st);
  else if (P.grp % 2 == 0)  // grouped heads: value heads in pairs sharing K, Q
    return launch_prep_v<DK, false, ET, false, true>(P, nblk / 2, st);
  else
    return launch_prep_v<DK, false, ET, false>(P, nblk, st);
}

hipError_t launch_schedule(const int32_t* cu, int n_seqs, int64_t nc, int64_t T, int64_t max_cps,
                           uint64_t hash, int32_t* sched, hipStream_t st) {
  int32_t* cu_ok = sched + drla_sched_cu(nc, n_seqs);
  int32_t* order = sched + 2 * nc + n_seqs + 1;
  hipLaunchKernelGGL(schedule_kernel, dim3(1), dim3(256), 0, st, cu, n_seqs, nc, T, max_cps, hash, sched,
                     sched + nc, sched + 2 * nc, cu_ok, order, sched + drla_sched_status(nc, n_seqs));
  // batches the schedule kernel keeps in LDS are ranked there
  if (n_seqs > kScheduleLdsSeqs)
    hipLaunchKernelGGL(rank_kernel, dim3((unsigned)((n_seqs + 255) / 256)), dim3(256), 0, st, cu_ok, n_seqs,
                       order);
  return hipGetLastError();
}

#define DRLA_PREP_INST(DK_, KDA_, ET_) \
  template hipError_t launch_prep<DK_, KDA_, ET_>(const PrepParams&, int64_t, hipStream_t);
DRLA_PREP_INST(64, false, bf16)
DRLA_PREP_INST(128, false, bf16)
DRLA_PREP_INST(64, true, bf16)
DRLA_PREP_INST(128, true, bf16)
DRLA_PREP_INST(64, false, f16)
DRLA_PREP_INST(128, false, f16)
DRLA_PREP_INST(64, true, f16)
DRLA_PREP_INST(128, true, f16)
DRLA_PREP_INST(64, false, float)
DRLA_PREP_INST(128, false, float)
DRLA_PREP_INST(64, true, float)
DRLA_PREP_INST(128, true, float)
#undef DRLA_PREP_INST

}  // namespace drla
