// Single-token decode step: one token of the gated delta rule per sequence,
// the per-token recurrence of "Empowering Hybrid Attention Models on NPUs",
// Section 2.1, with the state stored key-major (S is dk x dv):
//
//   GDN:  S <- e^{g} S                      KDA:  S <- Diag(e^{g}) S
//         x  = S^T k
//         S <- S + beta k (v - x)^T
//         o  = S^T q
//
// Nothing here is a contraction worth a matrix core: per (sequence, value
// head) the step reads and writes the 64 KiB fp32 state once and does 4
// multiply-adds per state element, so it is bound by HBM.  One 256-thread
// workgroup per (sequence, value head); thread t owns state column
// j = t % dv and a contiguous run of RPT rows, so every row of the state is
// read and written as one coalesced line per wave.  The two column sums
// (x, o) combine the row groups' partial sums through LDS.  Each state
// element is read and written by the same thread, so ht may be h0.  The
// state streams through once, so its loads and stores are non-temporal.
#include "drla_common.h"
#include "drla_kernels.h"

namespace drla {

template <int DK, int DV, bool KDA, typename ET>
__global__ __launch_bounds__(256) void decode_kernel(DecodeParams P) {
  constexpr int RG = 256 / DV;  // row groups
  constexpr int RPT = DK / RG;  // rows per thread
  __shared__ float kq[2][DK];   // k, q of this token (fp32)
  __shared__ float al[KDA ? DK : 1];
  __shared__ float vs[DV];
  __shared__ float part[2][RG][DV];

  const int tid = threadIdx.x;
  const int j = tid % DV, rg = tid / DV;
  const int unit = blockIdx.x;  // sequence * h_v + head
  const int n = unit / P.h_v, h = unit - n * P.h_v;
  const int hk = h / (P.h_v / P.h_qk);
  const int64_t sbase = (int64_t)unit * DK * DV;

  // the state block first: its loads are the long ones
  float s[RPT];
#pragma unroll
  for (int r = 0; r < RPT; ++r)
    s[r] = P.h0 ? __builtin_nontemporal_load(&P.h0[sbase + (int64_t)(rg * RPT + r) * DV + j]) : 0.f;

  const ET* qg = (const ET*)P.q + ((int64_t)n * P.h_qk + hk) * DK;
  const ET* kg = (const ET*)P.k + ((int64_t)n * P.h_qk + hk) * DK;
  const ET* vg = (const ET*)P.v + ((int64_t)n * P.h_v + h) * DV;
  if (tid < DK) {
    kq[0][tid] = to_f(kg[tid]);
    kq[1][tid] = to_f(qg[tid]);
    if (KDA) al[tid] = __expf(P.g[((int64_t)n * P.h_v + h) * DK + tid]);
  }
  if (tid < DV) vs[tid] = to_f(vg[tid]);
  const float beta = P.decay_only ? 1.f : P.beta[(int64_t)n * P.h_v + h];
  const float ag = KDA ? 1.f : __expf(P.g[(int64_t)n * P.h_v + h]);
  __syncthreads();

  // decay, then this row group's share of x = S^T k
  float px = 0.f;
#pragma unroll
  for (int r = 0; r < RPT; ++r) {
    const int i = rg * RPT + r;
    s[r] *= KDA ? al[i] : ag;
    px += s[r] * kq[0][i];
  }
  part[0][rg][j] = px;
  __syncthreads();
  float x = 0.f;
#pragma unroll
  for (int q = 0; q < RG; ++q) x += part[0][q][j];
  if (P.decay_only) x = 0.f;  // no delta rule: S += k v^T
  const float u = beta * (vs[j] - x);

  // rank-one update, its store, and this row group's share of o = S^T q
  float po = 0.f;
#pragma unroll
  for (int r = 0; r < RPT; ++r) {
    const int i = rg * RPT + r;
    s[r] += kq[0][i] * u;
    po += s[r] * kq[1][i];
  }
  if (P.ht) {
#pragma unroll
    for (int r = 0; r < RPT; ++r) __builtin_nontemporal_store(s[r], &P.ht[sbase + (int64_t)(rg * RPT + r) * DV + j]);
  }
  part[1][rg][j] = po;
  __syncthreads();
  if (rg == 0) {
    float o = 0.f;
#pragma unroll
    for (int q = 0; q < RG; ++q) o += part[1][q][j];
    ((ET*)P.o)[((int64_t)n * P.h_v + h) * DV + j] = (ET)o;
  }
}

template <int DK, int DV, bool KDA, typename ET>
static hipError_t launch_decode_v(const DecodeParams& P, int64_t units, hipStream_t st) {
  hipLaunchKernelGGL((decode_kernel<DK, DV, KDA, ET>), dim3((unsigned)units), dim3(256), 0, st, P);
  return hipGetLastError();
}

}  // namespace drla

hipError_t drla_launch_decode(const drla_decode_args* a) {
  using namespace drla;
  DecodeParams P;
  P.q = a->q;
  P.k = a->k;
  P.v = a->v;
  P.beta = a->beta;
  P.g = a->g;
  P.h0 = a->h0;
  P.o = a->o;
  P.ht = a->ht;
  P.h_qk = a->h_qk;
  P.h_v = a->h_v;
  P.decay_only = a->decay_only;
  const int64_t units = (int64_t)a->n_seqs * a->h_v;
  if (units == 0) return hipSuccess;
  hipStream_t st = (hipStream_t)a->stream;
  const int io = a->f32 ? 1 : a->f16 ? 2 : 0;
  const int key = (a->dk == 128 ? 1 : 0) | (a->dv == 128 ? 2 : 0) | (a->kda ? 4 : 0) | (io << 3);
#define DRLA_DEC_CASE(K, DK_, DV_, KDA_, ET_) \
  case K:                                   \
    return launch_decode_v<DK_, DV_, KDA_, ET_>(P, units, st);
  switch (key) {
    DRLA_DEC_CASE(0, 64, 64, false, bf16)
    DRLA_DEC_CASE(1, 128, 64, false, bf16)
    DRLA_DEC_CASE(2, 64, 128, false, bf16)
    DRLA_DEC_CASE(3, 128, 128, false, bf16)
    DRLA_DEC_CASE(4, 64, 64, true, bf16)
    DRLA_DEC_CASE(5, 128, 64, true, bf16)
    DRLA_DEC_CASE(6, 64, 128, true, bf16)
    DRLA_DEC_CASE(7, 128, 128, true, bf16)
    DRLA_DEC_CASE(8, 64, 64, false, float)
    DRLA_DEC_CASE(9, 128, 64, false, float)
    DRLA_DEC_CASE(10, 64, 128, false, float)
    DRLA_DEC_CASE(11, 128, 128, false, float)
    DRLA_DEC_CASE(12, 64, 64, true, float)
    DRLA_DEC_CASE(13, 128, 64, true, float)
    DRLA_DEC_CASE(14, 64, 128, true, float)
    DRLA_DEC_CASE(15, 128, 128, true, float)
    DRLA_DEC_CASE(16, 64, 64, false, f16)
    DRLA_DEC_CASE(17, 128, 64, false, f16)
    DRLA_DEC_CASE(18, 64, 128, false, f16)
    DRLA_DEC_CASE(19, 128, 128, false, f16)
    DRLA_DEC_CASE(20, 64, 64, true, f16)
    DRLA_DEC_CASE(21, 128, 64, true, f16)
    DRLA_DEC_CASE(22, 64, 128, true, f16)
    DRLA_DEC_CASE(23, 128, 128, true, f16)
  }
#undef DRLA_DEC_CASE
  return hipErrorInvalidValue;
}
