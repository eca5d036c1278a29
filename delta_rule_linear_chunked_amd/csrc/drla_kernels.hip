// Chunked prefill of delta-rule linear attention for gfx950 (CDNA4).
//
// The Map-Reduce-Map evaluation of "Empowering Hybrid Attention Models on
// NPUs", Section 2.1 ("Chunkwise Map-Reduce-Map Execution"), as three HIP
// kernels:
//   prep    (Map, chunk-parallel)   #1 Gate, #2 KKT, #3 Solve, #4 W/U
//   scan    (Reduce, per sequence)  #5 H: V' = U - W S, S <- e^{b_n} S + K~^T V'
//   output  (Map, chunk-parallel)   #6 O: O = (e^b Q) S + lower(Q K^T (.) D) V'
// The page names the operators but prints no formulas; the chunk identities
// used here follow from the token recurrence of its Section 2.1 (state
// updated with K_t, V_t, then output read with Q_t):
//   b_r = sum_{i<=r} g_i (in-chunk),  D_ri = e^{b_r - b_i} (i <= r)
//   A = strict_lower(diag(beta) (K K^T (.) D)),  T = (I + A)^{-1}
//   W = T diag(beta e^b) K,  U = T diag(beta) V
//   V' = U - W S (Section 5 calls this intermediate v_c),
//   O = diag(e^b) Q S + lower_incl(Q K^T (.) D) V'
//   S_next = e^{b_n} S + (diag(e^{b_n - b}) K)^T V'
// For KDA the decay is per key channel: the K K^T and Q K^T products become
// (K e^{B})(K e^{-B})^T and (Q e^{B})(K e^{-B})^T, e^{b} K becomes K e^{B},
// and the state decays as Diag(e^{b_n}) S.
//
// Matrix products run on MFMA (v_mfma_f32_16x16x32_bf16 for bf16 inputs,
// v_mfma_f32_16x16x4_f32 x8 for fp32 inputs), fp32 accumulation.
//
// Fragment order.  A 16x16 MFMA accumulator tile holds, in lane l
// (g = l/16, c = l%16), element [4g + i][c] for i = 0..3.  An operand block
// covers 16 rows ("outer" index) x 32 contraction indices ("inner"); lane l
// holds 8 elements of row c at inner positions
//   kmap(g, j) = 4g + j          for j < 4
//              = 16 + 4g + j - 4 for j >= 4,
// the same map for the A and the B operand (the sum over the contraction
// does not depend on which slot carries which index).  With this map the
// two accumulator tiles of rows [32p, 32p+16) and [32p+16, 32p+32) of a
// product are, lane by lane, exactly the operand block for inner block p:
// a result becomes the next product's operand without leaving registers.
// Intermediates in the workspace are stored as such blocks, 64 lanes x 8
// elements contiguous (1 KiB bf16), so every access is one coalesced 16-byte
// (bf16) or 32-byte (fp32) load or store per lane:
//   W  (outer token tile nt 0..3, inner dk block p)   index (nt*DK/32 + p)
//   K~ (outer dk tile mt, inner token block p 0..1)   index (mt*2 + p)
//   U, V' (outer dv tile nt, inner token block p)     index (nt*2 + p)
//   h  (outer dv tile nt, inner dk block p)           index (nt*DK/32 + p)
// per (v-head, chunk), chunk index fastest.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "drla_launch.h"

namespace drla {

typedef __bf16 bf16;
typedef bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef float floatx8 __attribute__((ext_vector_type(8)));

constexpr int C = DRLA_CHUNK_TOKENS;

template <typename ET> struct VT;
template <> struct VT<bf16> {
  typedef bf16x4 v4;   // 4 elements (8 bytes)
  typedef bf16x8 v8;   // one operand slot set (16 bytes)
  typedef bf16x8 v16b; // one 16-byte vector
  static constexpr int per16 = 8;
};
template <> struct VT<float> {
  typedef floatx4 v4;
  typedef floatx8 v8;
  typedef floatx4 v16b;
  static constexpr int per16 = 4;
};

__device__ __forceinline__ floatx4 mma(const bf16x8& a, const bf16x8& b, floatx4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ floatx4 mma(const floatx8& a, const floatx8& b, floatx4 c) {
#pragma unroll
  for (int j = 0; j < 8; ++j) c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[j], b[j], c, 0, 0, 0);
  return c;
}

__device__ __forceinline__ int kmap(int g, int j) { return j < 4 ? 4 * g + j : 12 + 4 * g + j; }

template <typename ET>
__device__ __forceinline__ typename VT<ET>::v8 cat(typename VT<ET>::v4 lo, typename VT<ET>::v4 hi) {
  return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}

// Two accumulator tiles -> one operand slot set, rounded to ET.
template <typename ET>
__device__ __forceinline__ typename VT<ET>::v8 pack(const floatx4& a, const floatx4& b) {
  typename VT<ET>::v8 r;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    r[j] = (ET)a[j];
    r[j + 4] = (ET)b[j];
  }
  return r;
}

// Operand slots of one row of a row-major array: row points at inner index 0
// of the 32-wide block.
template <typename ET>
__device__ __forceinline__ typename VT<ET>::v8 row_slots(const ET* row, int g) {
  typedef typename VT<ET>::v4 V4;
  return cat<ET>(*(const V4*)(row + 4 * g), *(const V4*)(row + 16 + 4 * g));
}

template <typename ET>
__device__ __forceinline__ float to_f(ET x) { return (float)x; }

struct Sched {
  const int32_t* chunk_seq;   // [nc] sequence of each chunk (packed input), else null
  const int32_t* chunk_start; // [nc] first token of each chunk
  const int32_t* seq_chunk0;  // [N+1] first chunk of each sequence
  const int32_t* cu;          // [N+1] device cu_seqlens (packed input)
  int64_t seq_len;            // dense batch: tokens per sequence
  int32_t cps;                // dense batch: chunks per sequence
  int32_t n_seqs;
};

struct Params {
  const void* q;
  const void* k;
  const void* v;
  const float* beta;
  const float* g;
  const float* h0;
  void* o;
  float* ht;
  void* w;
  void* kt;
  void* u;
  void* vp;
  void* h;
  float* gamma;
  Sched s;
  int32_t h_qk, h_v, grp;
  int64_t nc;
};

__device__ __forceinline__ void chunk_of(const Sched& s, int64_t c, int& seq, int64_t& t0, int& len) {
  if (s.chunk_seq) {
    seq = s.chunk_seq[c];
    if (seq < 0 || seq >= s.n_seqs) {  // inconsistent device/host lengths: do nothing
      seq = 0;
      t0 = 0;
      len = 0;
      return;
    }
    t0 = s.chunk_start[c];
    const int64_t end = s.cu[seq + 1];
    const int64_t n = end - t0;
    len = (int)(n < 0 ? 0 : (n > C ? C : n));
  } else {
    seq = (int)(c / s.cps);
    const int64_t local = c - (int64_t)seq * s.cps;
    t0 = (int64_t)seq * s.seq_len + local * C;
    const int64_t n = s.seq_len - local * C;
    len = (int)(n > C ? C : n);
  }
}

__device__ __forceinline__ void seq_chunks(const Sched& s, int seq, int64_t nc, int64_t& c0, int64_t& c1) {
  if (s.chunk_seq) {
    c0 = s.seq_chunk0[seq];
    c1 = s.seq_chunk0[seq + 1];
    c0 = c0 < 0 ? 0 : (c0 > nc ? nc : c0);
    c1 = c1 < c0 ? c0 : (c1 > nc ? nc : c1);
  } else {
    c0 = (int64_t)seq * s.cps;
    c1 = c0 + s.cps;
  }
}

// ---------------------------------------------------------------------------
// Chunk table for packed (varlen) input: one workgroup, prefix sum of the
// per-sequence chunk counts.  Entries past `nc` are never written.
__global__ __launch_bounds__(256) void schedule_kernel(const int32_t* cu, int n_seqs, int64_t nc,
                                                        int32_t* chunk_seq, int32_t* chunk_start,
                                                        int32_t* seq_chunk0) {
  __shared__ int32_t sc[256];
  const int t = threadIdx.x;
  int64_t carry = 0;
  for (int base = 0; base < n_seqs; base += 256) {
    const int s = base + t;
    int cnt = 0;
    int64_t st = 0;
    if (s < n_seqs) {
      st = cu[s];
      const int64_t L = (int64_t)cu[s + 1] - st;
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
      for (int j = 0; j < cnt; ++j) {
        const int64_t idx = excl + j;
        if (idx < nc) {
          chunk_seq[idx] = s;
          chunk_start[idx] = (int32_t)(st + (int64_t)C * j);
        }
      }
    }
    carry += sc[255];
    __syncthreads();
  }
  if (t == 0) seq_chunk0[n_seqs] = (int32_t)carry;
}

// ---------------------------------------------------------------------------
// prep: one workgroup (4 waves) per (chunk, v-head).
//   #1 Gate: in-chunk cumulative log-decay b (scalar per token for GDN, per
//            key channel for KDA)
//   #2 KKT:  A = strict_lower(diag(beta) (K K^T (.) D))
//   #3 Solve: T = (I + A)^{-1} by forward substitution in LDS, one column
//            of T per lane, fp32
//   #4 W/U:  W = T diag(beta e^b) K, U = T diag(beta) V (MFMA), plus
//            K~ = e^{b_n - b} (.) K and gamma = e^{b_n} for the scan.
template <int DK, int DV, bool KDA, typename ET>
__global__ __launch_bounds__(256) void prep_kernel(Params P) {
  typedef typename VT<ET>::v4 V4;
  typedef typename VT<ET>::v8 V8;
  typedef typename VT<ET>::v16b V16;
  constexpr int PE = VT<ET>::per16;
  constexpr int TP = C + 4;  // padded row of the transposed tiles (keeps 8/16-byte alignment)
  __shared__ __attribute__((aligned(16))) ET Kts[DK][TP];  // K^T: [channel][token]
  __shared__ __attribute__((aligned(16))) ET Vts[DV][TP];  // V^T
  __shared__ __attribute__((aligned(16))) float As[C][C + 4];  // A, then T in place
  __shared__ float bs[C];
  __shared__ float betas[C];
  __shared__ float Bs[KDA ? C : 1][KDA ? DK + 4 : 1];

  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int g4 = lane >> 4, c16 = lane & 15;
  const int64_t bid = blockIdx.x;
  const int h = (int)(bid / P.nc);
  const int64_t c = bid - (int64_t)h * P.nc;
  int seq, len;
  int64_t t0;
  chunk_of(P.s, c, seq, t0, len);
  const int hk = h / P.grp;
  const int64_t ch = (int64_t)h * P.nc + c;
  const ET* kg = (const ET*)P.k;
  const ET* vg = (const ET*)P.v;

  // #1 Gate (and beta).  Tokens past the sequence end get beta = g = 0, so
  // they write nothing and do not decay.
  if (tid < C) {
    float be = 0.f, gg = 0.f;
    if (tid < len) {
      be = P.beta[(t0 + tid) * P.h_v + h];
      if (!KDA) gg = P.g[(t0 + tid) * P.h_v + h];
    }
    betas[tid] = be;
    if (!KDA) {
      float x = gg;
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const float y = __shfl_up(x, off);
        if (lane >= off) x += y;
      }
      bs[tid] = x;
    }
  }
  if (KDA) {
    for (int d = tid; d < DK; d += 256) {
      float run = 0.f;
#pragma unroll 8
      for (int r = 0; r < C; ++r) {
        const float gv = r < len ? P.g[((t0 + r) * P.h_v + h) * DK + d] : 0.f;
        run += gv;
        Bs[r][d] = run;
      }
    }
  }
  // K and V of the chunk, transposed into LDS (zero rows past the end).
  {
    constexpr int KV = DK / PE;
    for (int idx = tid; idx < C * KV; idx += 256) {
      const int r = idx / KV, cv = idx - r * KV;
      V16 x = {};
      if (r < len) x = *(const V16*)(kg + ((t0 + r) * P.h_qk + hk) * DK + cv * PE);
#pragma unroll
      for (int e = 0; e < PE; ++e) Kts[cv * PE + e][r] = x[e];
    }
    constexpr int VV = DV / PE;
    for (int idx = tid; idx < C * VV; idx += 256) {
      const int r = idx / VV, cv = idx - r * VV;
      V16 x = {};
      if (r < len) x = *(const V16*)(vg + ((t0 + r) * P.h_v + h) * DV + cv * PE);
#pragma unroll
      for (int e = 0; e < PE; ++e) Vts[cv * PE + e][r] = x[e];
    }
  }
  __syncthreads();

  // #2 KKT: wave wv computes row tile ti = wv of A (tiles tj <= ti).
  {
    const int ti = wv;
    const int rr = 16 * ti + c16;
    V8 af[DK / 32];
#pragma unroll
    for (int p = 0; p < DK / 32; ++p) {
      V8 x = {};
      if (rr < len) x = row_slots<ET>(kg + ((t0 + rr) * P.h_qk + hk) * DK + 32 * p, g4);
      if (KDA) {
#pragma unroll
        for (int j = 0; j < 8; ++j) x[j] = (ET)(to_f(x[j]) * __expf(Bs[rr][32 * p + kmap(g4, j)]));
      }
      af[p] = x;
    }
    for (int tj = 0; tj <= ti; ++tj) {
      const int ii0 = 16 * tj + c16;
      floatx4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int p = 0; p < DK / 32; ++p) {
        V8 y = {};
        if (ii0 < len) y = row_slots<ET>(kg + ((t0 + ii0) * P.h_qk + hk) * DK + 32 * p, g4);
        if (KDA) {
#pragma unroll
          for (int j = 0; j < 8; ++j) y[j] = (ET)(to_f(y[j]) * __expf(-Bs[ii0][32 * p + kmap(g4, j)]));
        }
        acc = mma(af[p], y, acc);
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int r = 16 * ti + 4 * g4 + e, i = 16 * tj + c16;
        float a = 0.f;
        if (i < r) {
          a = betas[r] * acc[e];
          if (!KDA) a *= __expf(bs[r] - bs[i]);
        }
        As[r][i] = a;
      }
    }
  }
  __syncthreads();

  if (wv == 0) {
    // #3 Solve: (I + A) T = I, column `lane` of T, rows in order.  T[i][lane]
    // is zero for i < lane, so no masking is needed.
    float t[C];
#pragma unroll
    for (int r = 0; r < C; ++r) {
      float acc = (r == lane) ? 1.f : 0.f;
#pragma unroll
      for (int i = 0; i < r; ++i) acc -= As[r][i] * t[i];
      t[r] = acc;
    }
    // every read of A by this wave precedes these writes
#pragma unroll
    for (int r = 0; r < C; ++r) As[r][lane] = t[r];
  } else {
    // K~ = e^{b_n - b} (.) K in operand order (outer dk tile, inner token
    // block), and gamma = e^{b_n}.  b_n = b at the last token (padding has
    // g = 0).
    constexpr int NF = (DK / 16) * 2;
    ET* ktg = (ET*)P.kt + ch * (int64_t)(C * DK);
    for (int f = wv - 1; f < NF; f += 3) {
      const int mt = f >> 1, p = f & 1;
      const int d = 16 * mt + c16;
      V8 x = row_slots<ET>(&Kts[d][32 * p], g4);
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int i = 32 * p + kmap(g4, j);
        const float sc = KDA ? __expf(Bs[C - 1][d] - Bs[i][d]) : __expf(bs[C - 1] - bs[i]);
        x[j] = (ET)(to_f(x[j]) * sc);
      }
      *(V8*)(ktg + ((int64_t)f * 64 + lane) * 8) = x;
    }
    if (KDA) {
      for (int d = tid - 64; d < DK; d += 192) P.gamma[ch * DK + d] = __expf(Bs[C - 1][d]);
    } else if (tid == 64) {
      P.gamma[ch] = __expf(bs[C - 1]);
    }
  }
  __syncthreads();

  // #4 W/U.  W^T = K^T (T diag(beta e^b))^T; tiles (2p, nt) and (2p+1, nt)
  // of W^T form W's operand block (nt, p).  T is lower triangular, so token
  // block kb only contributes to row tiles nt >= 2 kb.
  {
    ET* wg = (ET*)P.w + ch * (int64_t)(C * DK);
    for (int f = wv; f < 4 * (DK / 32); f += 4) {
      const int nt = f & 3, p = f >> 2;
      floatx4 acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = acc0;
      const int r = 16 * nt + c16;
      for (int kb = 0; kb <= (nt >> 1); ++kb) {
        V8 bfr;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const int i = 32 * kb + kmap(g4, j);
          float x = As[r][i] * betas[i];
          if (!KDA) x *= __expf(bs[i]);
          bfr[j] = (ET)x;
        }
#pragma unroll
        for (int mm = 0; mm < 2; ++mm) {
          const int d = 16 * (2 * p + mm) + c16;
          V8 afr = row_slots<ET>(&Kts[d][32 * kb], g4);
          if (KDA) {
#pragma unroll
            for (int j = 0; j < 8; ++j) afr[j] = (ET)(to_f(afr[j]) * __expf(Bs[32 * kb + kmap(g4, j)][d]));
          }
          if (mm == 0)
            acc0 = mma(afr, bfr, acc0);
          else
            acc1 = mma(afr, bfr, acc1);
        }
      }
      *(V8*)(wg + ((int64_t)(nt * (DK / 32) + p) * 64 + lane) * 8) = pack<ET>(acc0, acc1);
    }
    // U = (T diag(beta)) V; tiles (2p, nt), (2p+1, nt) form block (nt, p).
    ET* ug = (ET*)P.u + ch * (int64_t)(C * DV);
    for (int f = wv; f < (DV / 16) * 2; f += 4) {
      const int nt = f >> 1, p = f & 1;
      floatx4 acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = acc0;
      for (int kb = 0; kb <= p; ++kb) {
        const V8 bfr = row_slots<ET>(&Vts[16 * nt + c16][32 * kb], g4);
#pragma unroll
        for (int mm = 0; mm < 2; ++mm) {
          const int r = 16 * (2 * p + mm) + c16;
          V8 afr;
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            const int i = 32 * kb + kmap(g4, j);
            afr[j] = (ET)(As[r][i] * betas[i]);
          }
          if (mm == 0)
            acc0 = mma(afr, bfr, acc0);
          else
            acc1 = mma(afr, bfr, acc1);
        }
      }
      *(V8*)(ug + ((int64_t)(nt * 2 + p) * 64 + lane) * 8) = pack<ET>(acc0, acc1);
    }
  }
}

// ---------------------------------------------------------------------------
// scan: one wave per (sequence, v-head, 16-column block of dv).  The state
// columns are independent (the column split of Section 4, "Computation
// Splitting"), so a wave owns S[:, 16 cols] in registers, fp32, for the
// whole sequence and never synchronises with another wave.  Per chunk:
//   h[c] = S  (stored for the output kernel, io dtype)
//   V'   = U - W S
//   S    = gamma S + K~^T V'
// The next chunk's operands are loaded before the current chunk's products.
template <int DK, int DV, bool KDA, typename ET>
struct ScanOps {
  typedef typename VT<ET>::v8 V8;
  V8 w[4][DK / 32];
  V8 kt[DK / 16][2];
  V8 u[2];
  floatx4 gam[KDA ? DK / 16 : 1];
};

template <int DK, int DV, bool KDA, typename ET>
__device__ __forceinline__ void scan_load(ScanOps<DK, DV, KDA, ET>& o, const Params& P, int64_t ch, int nb,
                                          int lane) {
  typedef typename VT<ET>::v8 V8;
  const V8* wp = (const V8*)P.w + ch * (int64_t)(C * DK / 8);
  const V8* kp = (const V8*)P.kt + ch * (int64_t)(C * DK / 8);
  const V8* up = (const V8*)P.u + ch * (int64_t)(C * DV / 8);
#pragma unroll
  for (int nt = 0; nt < 4; ++nt)
#pragma unroll
    for (int p = 0; p < DK / 32; ++p) o.w[nt][p] = wp[(nt * (DK / 32) + p) * 64 + lane];
#pragma unroll
  for (int mt = 0; mt < DK / 16; ++mt)
#pragma unroll
    for (int p = 0; p < 2; ++p) o.kt[mt][p] = kp[(mt * 2 + p) * 64 + lane];
#pragma unroll
  for (int p = 0; p < 2; ++p) o.u[p] = up[(nb * 2 + p) * 64 + lane];
  if (KDA) {
    const int g4 = lane >> 4;
#pragma unroll
    for (int mt = 0; mt < (KDA ? DK / 16 : 1); ++mt)
      o.gam[mt] = *(const floatx4*)(P.gamma + ch * DK + 16 * mt + 4 * g4);
  } else {
    const float gsc = P.gamma[ch];
    o.gam[0] = floatx4{gsc, gsc, gsc, gsc};
  }
}

template <int DK, int DV, bool KDA, typename ET>
__device__ __forceinline__ void scan_step(const ScanOps<DK, DV, KDA, ET>& cur, floatx4 (&S)[DK / 16],
                                          const Params& P, int64_t ch, int nb, int lane) {
  typedef typename VT<ET>::v8 V8;
  constexpr int KT = DK / 16, KB = DK / 32;
  // state entering the chunk, as operand blocks (outer: these 16 columns,
  // inner: dk block p) -- stored for the output kernel, and the B operand
  // of W S
  V8 sf[KB];
  V8* hp = (V8*)P.h + ch * (int64_t)(DK * DV / 8);
#pragma unroll
  for (int p = 0; p < KB; ++p) {
    sf[p] = pack<ET>(S[2 * p], S[2 * p + 1]);
    hp[(nb * KB + p) * 64 + lane] = sf[p];
  }
  // V' = U - W S   (4 token tiles)
  floatx4 vt[4];
#pragma unroll
  for (int nt = 0; nt < 4; ++nt) {
    floatx4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int p = 0; p < KB; ++p) acc = mma(cur.w[nt][p], sf[p], acc);
#pragma unroll
    for (int e = 0; e < 4; ++e) vt[nt][e] = to_f(cur.u[nt >> 1][(nt & 1) * 4 + e]) - acc[e];
  }
  V8 vf[2];
  V8* vpp = (V8*)P.vp + ch * (int64_t)(C * DV / 8);
#pragma unroll
  for (int p = 0; p < 2; ++p) {
    vf[p] = pack<ET>(vt[2 * p], vt[2 * p + 1]);
    vpp[(nb * 2 + p) * 64 + lane] = vf[p];
  }
  // S = gamma S + K~^T V'
#pragma unroll
  for (int mt = 0; mt < KT; ++mt) {
    const floatx4 gm = cur.gam[KDA ? mt : 0];
#pragma unroll
    for (int e = 0; e < 4; ++e) S[mt][e] *= gm[e];
#pragma unroll
    for (int p = 0; p < 2; ++p) S[mt] = mma(cur.kt[mt][p], vf[p], S[mt]);
  }
}

template <int DK, int DV, bool KDA, typename ET>
__global__ __launch_bounds__(64) void scan_kernel(Params P) {
  typedef typename VT<ET>::v8 V8;
  constexpr int NB = DV / 16, KT = DK / 16, KB = DK / 32;
  const int lane = threadIdx.x, g4 = lane >> 4, c16 = lane & 15;
  // XCD-aware order: consecutive workgroups go to different XCDs; remap so
  // that the NB column blocks of one (sequence, head), which read the same
  // W and K~, run on one XCD and share its L2.
  int b = blockIdx.x;
  const int G = gridDim.x;
  if (G % 8 == 0) b = (b % 8) * (G / 8) + b / 8;
  const int unit = b / NB, nb = b - unit * NB;
  const int seq = unit / P.h_v, h = unit - seq * P.h_v;
  int64_t c0, c1;
  seq_chunks(P.s, seq, P.nc, c0, c1);
  const int col = 16 * nb + c16;
  const int64_t sbase = ((int64_t)seq * P.h_v + h) * DK * DV;

  floatx4 S[KT];
#pragma unroll
  for (int mt = 0; mt < KT; ++mt)
#pragma unroll
    for (int e = 0; e < 4; ++e) S[mt][e] = P.h0 ? P.h0[sbase + (int64_t)(16 * mt + 4 * g4 + e) * DV + col] : 0.f;

  // Two operand sets (ping-pong: the next chunk's operands load while this
  // chunk computes) need 2 x 136 registers for bf16; fp32 operands at
  // dk = 128 are twice as large and would not fit in the 512 registers of a
  // wave, so that variant loads one chunk at a time.
  constexpr bool kPingPong = sizeof(ET) == 2 || DK == 64;
  if (kPingPong) {
    ScanOps<DK, DV, KDA, ET> bufa, bufb;
    if (c0 < c1) scan_load(bufa, P, (int64_t)h * P.nc + c0, nb, lane);
    for (int64_t c = c0; c < c1; c += 2) {
      const int64_t ch = (int64_t)h * P.nc + c;
      if (c + 1 < c1) scan_load(bufb, P, ch + 1, nb, lane);
      scan_step<DK, DV, KDA, ET>(bufa, S, P, ch, nb, lane);
      if (c + 1 >= c1) break;
      if (c + 2 < c1) scan_load(bufa, P, ch + 2, nb, lane);
      scan_step<DK, DV, KDA, ET>(bufb, S, P, ch + 1, nb, lane);
    }
  } else {
    ScanOps<DK, DV, KDA, ET> buf;
    for (int64_t c = c0; c < c1; ++c) {
      const int64_t ch = (int64_t)h * P.nc + c;
      scan_load(buf, P, ch, nb, lane);
      scan_step<DK, DV, KDA, ET>(buf, S, P, ch, nb, lane);
    }
  }
  if (P.ht) {
#pragma unroll
    for (int mt = 0; mt < KT; ++mt)
#pragma unroll
      for (int e = 0; e < 4; ++e) P.ht[sbase + (int64_t)(16 * mt + 4 * g4 + e) * DV + col] = S[mt][e];
  }
}

// ---------------------------------------------------------------------------
// output: one workgroup (4 waves) per (chunk, v-head); wave w produces the 16
// tokens [16w, 16w+16) of the chunk for all dv, as O^T tiles:
//   O^T = S^T (e^b Q)^T + V'^T P^T,  P = lower_incl(Q K^T (.) D)
// P^T is computed as K Q^T so that its accumulator tiles are already the B
// operand of V'^T P^T.
template <int DK, int DV, bool KDA, typename ET>
__global__ __launch_bounds__(256) void output_kernel(Params P) {
  typedef typename VT<ET>::v4 V4;
  typedef typename VT<ET>::v8 V8;
  constexpr int KB = DK / 32, NT = DV / 16;
  __shared__ float Bs[KDA ? C : 1][KDA ? DK + 4 : 1];
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int g4 = lane >> 4, c16 = lane & 15;
  const int64_t bid = blockIdx.x;
  const int h = (int)(bid / P.nc);
  const int64_t c = bid - (int64_t)h * P.nc;
  int seq, len;
  int64_t t0;
  chunk_of(P.s, c, seq, t0, len);
  const int hk = h / P.grp;
  const int64_t ch = (int64_t)h * P.nc + c;
  const ET* qg = (const ET*)P.q;
  const ET* kg = (const ET*)P.k;

  float bl = 0.f;  // GDN: cumulative log-decay of token `lane`
  if (!KDA) {
    float x = lane < len ? P.g[(t0 + lane) * P.h_v + h] : 0.f;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const float y = __shfl_up(x, off);
      if (lane >= off) x += y;
    }
    bl = x;
  } else {
    for (int d = tid; d < DK; d += 256) {
      float run = 0.f;
#pragma unroll 8
      for (int r = 0; r < C; ++r) {
        run += r < len ? P.g[((t0 + r) * P.h_v + h) * DK + d] : 0.f;
        Bs[r][d] = run;
      }
    }
    __syncthreads();
  }

  const int w = wv;
  const int rl = 16 * w + c16;  // this lane's token (column of the O^T tiles)
  const float br = KDA ? 0.f : __shfl(bl, rl);
  // (e^B (.) Q) rows as the B operand (inner = dk)
  V8 qf[KB];
#pragma unroll
  for (int p = 0; p < KB; ++p) {
    V8 x = {};
    if (rl < len) x = row_slots<ET>(qg + ((t0 + rl) * P.h_qk + hk) * DK + 32 * p, g4);
    if (KDA) {
#pragma unroll
      for (int j = 0; j < 8; ++j) x[j] = (ET)(to_f(x[j]) * __expf(Bs[rl][32 * p + kmap(g4, j)]));
    }
    qf[p] = x;
  }
  // P^T tiles (it, w) for it <= w
  floatx4 pt[4];
#pragma unroll
  for (int it = 0; it < 4; ++it) {
    pt[it] = floatx4{0.f, 0.f, 0.f, 0.f};
    if (it <= w) {
      const int ir = 16 * it + c16;
      floatx4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int p = 0; p < KB; ++p) {
        V8 x = {};
        if (ir < len) x = row_slots<ET>(kg + ((t0 + ir) * P.h_qk + hk) * DK + 32 * p, g4);
        if (KDA) {
#pragma unroll
          for (int j = 0; j < 8; ++j) x[j] = (ET)(to_f(x[j]) * __expf(-Bs[ir][32 * p + kmap(g4, j)]));
        }
        acc = mma(x, qf[p], acc);
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int i = 16 * it + 4 * g4 + e;
        const float bi = KDA ? 0.f : __shfl(bl, i);
        pt[it][e] = (i <= rl) ? (KDA ? acc[e] : acc[e] * __expf(br - bi)) : 0.f;
      }
    }
  }
  V8 pf[2];
  pf[0] = pack<ET>(pt[0], pt[1]);
  pf[1] = pack<ET>(pt[2], pt[3]);
  const float eb = KDA ? 1.f : __expf(br);

  const V8* hp = (const V8*)P.h + ch * (int64_t)(DK * DV / 8);
  const V8* vpp = (const V8*)P.vp + ch * (int64_t)(C * DV / 8);
  ET* og = (ET*)P.o;
#pragma unroll 2
  for (int mt = 0; mt < NT; ++mt) {
    floatx4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int p = 0; p < KB; ++p) acc = mma(hp[(mt * KB + p) * 64 + lane], qf[p], acc);
    acc *= eb;
    acc = mma(vpp[(mt * 2 + 0) * 64 + lane], pf[0], acc);
    if (w >= 2) acc = mma(vpp[(mt * 2 + 1) * 64 + lane], pf[1], acc);
    if (rl < len) {
      V4 out;
#pragma unroll
      for (int e = 0; e < 4; ++e) out[e] = (ET)acc[e];
      *(V4*)(og + ((t0 + rl) * P.h_v + h) * DV + 16 * mt + 4 * g4) = out;
    }
  }
}

// ---------------------------------------------------------------------------
template <int DK, int DV, bool KDA, typename ET>
static hipError_t launch_all(const Params& P, int n_seqs, const int32_t* cu_dev, int32_t* sched,
                             hipStream_t st, void* const* ev) {
  hipError_t e = hipSuccess;
  auto mark = [&](int i) {
    if (ev && e == hipSuccess) e = hipEventRecord((hipEvent_t)ev[i], st);
  };
  mark(0);
  if (P.s.chunk_seq && n_seqs > 0) {
    hipLaunchKernelGGL(schedule_kernel, dim3(1), dim3(256), 0, st, cu_dev, n_seqs, P.nc, sched,
                       sched + P.nc, sched + 2 * P.nc);
  }
  const int64_t nblk = P.nc * P.h_v;
  if (nblk > 0) hipLaunchKernelGGL((prep_kernel<DK, DV, KDA, ET>), dim3((unsigned)nblk), dim3(256), 0, st, P);
  mark(1);
  const int64_t nscan = (int64_t)n_seqs * P.h_v * (DV / 16);
  if (nscan > 0) hipLaunchKernelGGL((scan_kernel<DK, DV, KDA, ET>), dim3((unsigned)nscan), dim3(64), 0, st, P);
  mark(2);
  if (nblk > 0) hipLaunchKernelGGL((output_kernel<DK, DV, KDA, ET>), dim3((unsigned)nblk), dim3(256), 0, st, P);
  mark(3);
  const hipError_t le = hipGetLastError();
  return e != hipSuccess ? e : le;
}

}  // namespace drla

// Launch entry used by the C ABI layer.
hipError_t drla_launch(const drla_launch_args* a) {
  using namespace drla;
  Params P = {};
  P.q = a->q;
  P.k = a->k;
  P.v = a->v;
  P.beta = a->beta;
  P.g = a->g;
  P.h0 = a->h0;
  P.o = a->o;
  P.ht = a->ht;
  char* ws = (char*)a->workspace;
  P.w = ws + a->off_w;
  P.kt = ws + a->off_kt;
  P.u = ws + a->off_u;
  P.vp = ws + a->off_vp;
  P.h = ws + a->off_h;
  P.gamma = (float*)(ws + a->off_gamma);
  int32_t* sched = (int32_t*)(ws + a->off_sched);
  if (a->cu_dev) {
    P.s.chunk_seq = sched;
    P.s.chunk_start = sched + a->n_chunks;
    P.s.seq_chunk0 = sched + 2 * a->n_chunks;
    P.s.cu = a->cu_dev;
  } else {
    P.s.seq_len = a->n_seqs > 0 ? a->total_tokens / a->n_seqs : 0;
    P.s.cps = (int32_t)((P.s.seq_len + C - 1) / C);
  }
  P.s.n_seqs = a->n_seqs;
  P.h_qk = a->h_qk;
  P.h_v = a->h_v;
  P.grp = a->h_v / a->h_qk;
  P.nc = a->n_chunks;
  hipStream_t st = (hipStream_t)a->stream;
  const int key = (a->dk == 128 ? 1 : 0) | (a->dv == 128 ? 2 : 0) | (a->kda ? 4 : 0) | (a->f32 ? 8 : 0);
#define DRLA_CASE(K, DK_, DV_, KDA_, ET_) \
  case K:                                 \
    return launch_all<DK_, DV_, KDA_, ET_>(P, a->n_seqs, a->cu_dev, sched, st, a->stage_events);
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
    default:
      return hipErrorInvalidValue;
  }
#undef DRLA_CASE
}
