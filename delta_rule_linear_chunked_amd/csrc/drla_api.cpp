// C ABI of drla: argument checks, chunk count and workspace layout, then
// one call into the kernel launcher.  Every check runs before anything is
// enqueued; on error nothing is launched or written.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <mutex>
#include <string>

#include "../../include/drla.h"
#include "drla_launch.h"

static_assert(DRLA_CHUNK == DRLA_CHUNK_TOKENS, "chunk size mismatch");

// Scratch memory of drla_prefill_noalloc: a fixed array in this library's
// device code object, one copy per GPU, held until the process ends.  In
// host code `scratch` is only a stand-in symbol; its device address comes
// from hipGetSymbolAddress (scratch_address below) and only that address
// is ever passed to a kernel.
static __device__ __align__(256) unsigned char scratch[DRLA_NOALLOC_SCRATCH_BYTES];

namespace {

thread_local std::string g_last_error;

drla_status fail(drla_status s, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
drla_status fail(drla_status s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return s;
}

// Device address of `scratch` on the current device, resolved once per
// device (each GPU holds its own copy of the array at its own address).
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];

drla_status scratch_address(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(DRLA_ERR_HIP, "hipGetDevice failed: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices) return fail(DRLA_ERR_HIP, "device index %d out of range", dev);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !ptr)
      return fail(DRLA_ERR_HIP, "hipGetSymbolAddress(scratch) failed: %s", hipGetErrorString(e));
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return DRLA_OK;
}

size_t align_up(size_t x) { return (x + 255) & ~(size_t)255; }

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

bool overlap(const void* a, size_t na, const void* b, size_t nb) {
  if (!a || !b || na == 0 || nb == 0) return false;
  const uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
  return x < y + nb && y < x + na;
}

// Checks the problem description and host lengths; computes the chunk count.
drla_status check_problem(const drla_problem* p, const int32_t* cu_host, int64_t* n_chunks) {
  if (!p) return fail(DRLA_ERR_NULL, "problem is NULL");
  if (p->n_seqs < 1) return fail(DRLA_ERR_SHAPE, "n_seqs must be >= 1 (got %d)", p->n_seqs);
  if (p->h_qk < 1 || p->h_v < 1) return fail(DRLA_ERR_SHAPE, "head counts must be >= 1");
  if (p->h_v % p->h_qk != 0)
    return fail(DRLA_ERR_SHAPE, "h_v (%d) must be a multiple of h_qk (%d)", p->h_v, p->h_qk);
  if (p->total_tokens < 0) return fail(DRLA_ERR_SHAPE, "total_tokens must be >= 0");
  if (p->total_tokens > INT32_MAX) return fail(DRLA_ERR_SHAPE, "total_tokens must fit in int32");
  if ((p->dk != 64 && p->dk != 128) || (p->dv != 64 && p->dv != 128))
    return fail(DRLA_ERR_UNSUPPORTED, "dk, dv must be 64 or 128 (got %d, %d)", p->dk, p->dv);
  if (p->io_dtype != DRLA_BF16 && p->io_dtype != DRLA_F32 && p->io_dtype != DRLA_F16)
    return fail(DRLA_ERR_UNSUPPORTED, "unknown io dtype %d", p->io_dtype);
  int64_t nc = 0;
  if (cu_host) {
    if (cu_host[0] != 0) return fail(DRLA_ERR_SEQLENS, "cu_seqlens[0] must be 0");
    for (int s = 0; s < p->n_seqs; ++s) {
      const int64_t L = (int64_t)cu_host[s + 1] - cu_host[s];
      if (L < 0) return fail(DRLA_ERR_SEQLENS, "cu_seqlens decreases at %d", s);
      nc += (L + DRLA_CHUNK - 1) / DRLA_CHUNK;
    }
    if (cu_host[p->n_seqs] != p->total_tokens)
      return fail(DRLA_ERR_SEQLENS, "cu_seqlens[N] = %d != total_tokens %lld", cu_host[p->n_seqs],
                  (long long)p->total_tokens);
  } else {
    if (p->total_tokens % p->n_seqs != 0)
      return fail(DRLA_ERR_SHAPE, "dense batch: total_tokens %% n_seqs != 0");
    const int64_t L = p->total_tokens / p->n_seqs;
    nc = (int64_t)p->n_seqs * ((L + DRLA_CHUNK - 1) / DRLA_CHUNK);
  }
  if (nc * p->h_v > INT32_MAX) return fail(DRLA_ERR_SHAPE, "too many (chunk, head) pairs");
  if (((int64_t)p->n_seqs * p->h_v + 7) * (p->dv / 16) > INT32_MAX) return fail(DRLA_ERR_SHAPE, "too many sequences");
  *n_chunks = nc;
  return DRLA_OK;
}

// Chunks of the longest sequence (cu_host: a checked packed layout, or NULL
// for a dense batch).
static int64_t max_chunks(const drla_problem* p, const int32_t* cu_host) {
  if (p->n_seqs < 1) return 0;
  if (!cu_host) return (p->total_tokens / p->n_seqs + DRLA_CHUNK - 1) / DRLA_CHUNK;
  int64_t m = 0;
  for (int s = 0; s < p->n_seqs; ++s) {
    const int64_t c = ((int64_t)cu_host[s + 1] - cu_host[s] + DRLA_CHUNK - 1) / DRLA_CHUNK;
    m = c > m ? c : m;
  }
  return m;
}

constexpr int kKnownFlags = DRLA_KEEP_INTERMEDIATES | DRLA_DECAY_ONLY | DRLA_SERIAL | DRLA_HEAD_SCAN | DRLA_COLUMN_SCAN;

// Unknown flags and the two scan choices together are rejected.
static drla_status check_flags(int flags) {
  if (flags & ~kKnownFlags) return fail(DRLA_ERR_UNSUPPORTED, "unknown flags 0x%x", flags);
  if ((flags & DRLA_HEAD_SCAN) && (flags & DRLA_COLUMN_SCAN))
    return fail(DRLA_ERR_UNSUPPORTED, "DRLA_HEAD_SCAN and DRLA_COLUMN_SCAN exclude each other");
  return DRLA_OK;
}

// The head-resident scan serves scalar-gate calls with 16-bit inputs (GDN,
// decay-only) that keep no intermediates: always with DRLA_HEAD_SCAN, and
// without flags where its timing model predicts it faster
// (drla_auto_head_scan, at 256 compute units like the workspace); with
// DRLA_COLUMN_SCAN, or DRLA_SERIAL alone, the per-16-column scan runs.
static bool uses_hs(const drla_problem* p, int64_t nc, int64_t max_cps, bool kda, int flags) {
  if (kda || p->io_dtype == DRLA_F32 || (flags & DRLA_KEEP_INTERMEDIATES)) return false;
  if (flags & DRLA_HEAD_SCAN) return true;
  if (flags & (DRLA_SERIAL | DRLA_COLUMN_SCAN)) return false;
  return p->n_seqs >= 1 && drla_auto_head_scan((int64_t)p->n_seqs * p->h_v, max_cps, nc * p->h_v, p->dk, p->dv, 256);
}

// Segments per sequence the hs region provides for (drla_hs_count at 256
// compute units; one pass when dk != dv or with DRLA_SERIAL).
static int32_t hs_count(const drla_problem* p, int64_t nc, int64_t max_cps, bool kda, int flags) {
  if (!uses_hs(p, nc, max_cps, kda, flags) || p->dk != p->dv || (flags & DRLA_SERIAL) || p->n_seqs < 1) return 1;
  return drla_hs_count((int64_t)p->n_seqs * p->h_v, max_cps, 256);
}

// Segments the per-16-column scan's seg region provides for (drla_seg_plan
// at 256 compute units, over the longest sequence; paired chains possible in
// the LDS-fed scan of scalar-gate 16-bit calls); 1 for calls the split does
// not take.
static int32_t seg_count(const drla_problem* p, int64_t nc, int64_t max_cps, bool kda, int flags) {
  if (uses_hs(p, nc, max_cps, kda, flags) || (flags & (DRLA_KEEP_INTERMEDIATES | DRLA_SERIAL))) return 1;
  if (p->dk != p->dv || p->n_seqs < 1) return 1;
  const bool can_pair = !kda && p->io_dtype != DRLA_F32;
  return drla_seg_plan((int64_t)p->n_seqs * p->h_v * (p->dv / 16), max_cps, 256, can_pair, nullptr);
}

void layout_of(const drla_problem* p, int64_t nc, bool varlen, int64_t max_cps, bool kda, int flags,
               drla_layout* L) {
  const size_t es = p->io_dtype == DRLA_F32 ? 4 : 2;
  const size_t ncH = (size_t)nc * p->h_v;
  const size_t frag = 64 * 8 * es;  // one operand fragment
  const bool keep = (flags & DRLA_KEEP_INTERMEDIATES) != 0;
  size_t off = 0;
  L->n_chunks = nc;
  L->sched = off;
  // packed input: chunk -> sequence, chunk -> first token, sequence -> first
  // chunk, the sequences longest first, the checked lengths, a status word
  off = align_up(off + (varlen ? (size_t)drla_sched_words(nc, p->n_seqs) * 4 : 0));
  L->tb = off;
  off = align_up(off + ncH * 8 * frag);
  L->pm = off;
  off = align_up(off + ncH * 8 * frag);
  // K~^T is only needed by the register-fed scan (KDA, fp32 inputs); the
  // LDS-fed GDN scan transposes K itself
  const bool need_kt = kda || p->io_dtype == DRLA_F32;
  L->kt = need_kt ? off : 0;
  if (need_kt) off = align_up(off + ncH * DRLA_CHUNK * p->dk * es);
  L->kw = kda ? off : 0;
  if (kda) off = align_up(off + ncH * DRLA_CHUNK * p->dk * es);
  L->qw = kda ? off : 0;
  if (kda) off = align_up(off + ncH * DRLA_CHUNK * p->dk * es);
  L->gam = off;
  off = align_up(off + ncH * (kda ? p->dk : 2 * DRLA_CHUNK) * 4);
  L->vp = keep ? off : 0;
  if (keep) off = align_up(off + ncH * DRLA_CHUNK * p->dv * es);
  L->h = keep ? off : 0;
  if (keep) off = align_up(off + ncH * (size_t)p->dk * p->dv * es);
  // Segment-split per-16-column scan (calls with dk = dv that leave most of
  // a 256-CU chip idle): its states and G
  const int32_t np = seg_count(p, nc, max_cps, kda, flags);
  L->seg = np > 1 ? off : 0;
  if (np > 1)
    off = align_up(off + drla_seg_offsets((int64_t)p->n_seqs * p->h_v, p->dk, p->total_tokens, p->h_v, np, es).total);
  // Head-resident scan (DRLA_HEAD_SCAN) with segments: the segments' states
  // and maps
  const int32_t hnp = hs_count(p, nc, max_cps, kda, flags);
  L->hs = hnp > 1 ? off : 0;
  if (hnp > 1) off = align_up(off + drla_hs_bytes((int64_t)p->n_seqs * p->h_v, p->dk, p->dv, hnp, es));
  L->total = off;
  L->head_scan = uses_hs(p, nc, max_cps, kda, flags) ? 1 : 0;
}

// Packed input that the kernels take as such: more than one sequence.
static bool packed(const drla_problem* p, const int32_t* cu_host) { return cu_host != nullptr && p->n_seqs > 1; }

drla_status run(bool kda, int flags, const drla_problem* p, const void* q, const void* k, const void* v,
                const float* beta, const float* g, const float* h0, const int32_t* cu_dev,
                const int32_t* cu_host, void* o, float* ht, void* ws, size_t ws_bytes, void* stream,
                void* const* stage_events) {
  int64_t nc = 0;
  if (!p) return fail(DRLA_ERR_NULL, "problem is NULL");
  if ((cu_dev == nullptr) != (cu_host == nullptr))
    return fail(DRLA_ERR_SEQLENS, "cu_seqlens_dev and cu_seqlens_host must both be set or both NULL");
  drla_status st = check_problem(p, cu_host, &nc);
  if (st != DRLA_OK) return st;
  if ((st = check_flags(flags)) != DRLA_OK) return st;
  // one packed sequence (cu_seqlens = {0, T}, checked above) is a dense call
  if (cu_host && !packed(p, cu_host)) cu_dev = cu_host = nullptr;
  const bool decay = (flags & DRLA_DECAY_ONLY) != 0;
  if (decay) beta = nullptr;  // unused without the delta rule
  const int64_t T = p->total_tokens;
  if (T > 0 && (!q || !k || !v || (!beta && !decay) || !g || !o))
    return fail(DRLA_ERR_NULL, decay ? "q, k, v, g and o must be non-NULL" : "q, k, v, beta, g and o must be non-NULL");
  const void* ptrs[] = {q, k, v, beta, g, h0, cu_dev, o, ht, ws};
  for (const void* x : ptrs)
    if (x && !aligned16(x)) return fail(DRLA_ERR_ALIGN, "device pointers must be 16-byte aligned");
  drla_layout L;
  const int64_t max_cps = max_chunks(p, cu_host);
  layout_of(p, nc, cu_dev != nullptr, max_cps, kda, flags, &L);
  if (L.total > 0 && (!ws || ws_bytes < L.total))
    return fail(DRLA_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", L.total, ws ? ws_bytes : 0);
  const size_t es = p->io_dtype == DRLA_F32 ? 4 : 2;
  const size_t nq = (size_t)T * p->h_qk * p->dk * es, nv = (size_t)T * p->h_v * p->dv * es;
  const size_t nb = (size_t)T * p->h_v * 4, ng = kda ? nb * p->dk : nb;
  const size_t ns = (size_t)p->n_seqs * p->h_v * p->dk * p->dv * 4;
  const size_t ncu = (size_t)(p->n_seqs + 1) * 4;
  struct Buf {
    const void* p;
    size_t n;
  };
  const Buf ins[] = {{q, nq}, {k, nq}, {v, nv}, {beta, nb}, {g, ng}, {h0, ns}, {cu_dev, ncu}};
  const Buf outs[] = {{o, nv}, {ht, ns}, {ws, L.total}};
  for (int i = 0; i < 3; ++i) {
    for (const Buf& b : ins) {
      if (i == 1 && b.p == h0 && ht == h0) continue;  // in-place state update
      if (overlap(outs[i].p, outs[i].n, b.p, b.n))
        return fail(DRLA_ERR_ALIAS, "an output buffer overlaps an input buffer");
    }
    for (int j = i + 1; j < 3; ++j)
      if (overlap(outs[i].p, outs[i].n, outs[j].p, outs[j].n))
        return fail(DRLA_ERR_ALIAS, "output buffers overlap");
  }

  drla_launch_args a;
  memset(&a, 0, sizeof a);
  a.q = q;
  a.k = k;
  a.v = v;
  a.beta = beta;
  a.g = g;
  a.h0 = h0;
  a.cu_dev = cu_dev;
  if (cu_host)
    for (int i = 0; i <= p->n_seqs; ++i) a.cu_hash += drla_cu_mix((uint64_t)i, (uint32_t)cu_host[i]);
  a.o = o;
  a.ht = ht;
  a.workspace = ws;
  a.off_sched = L.sched;
  a.off_tb = L.tb;
  a.off_pm = L.pm;
  a.off_kt = L.kt;
  a.off_kw = L.kw;
  a.off_qw = L.qw;
  a.off_gam = L.gam;
  a.off_vp = L.vp;
  a.off_h = L.h;
  a.off_seg = L.seg;
  a.seg_np = L.seg ? seg_count(p, nc, max_cps, kda, flags) : 1;
  a.off_hs = L.hs;
  a.hs_np = L.hs ? hs_count(p, nc, max_cps, kda, flags) : 1;
  a.max_cps = max_cps;
  a.total_tokens = T;
  a.n_chunks = nc;
  a.n_seqs = p->n_seqs;
  a.h_qk = p->h_qk;
  a.h_v = p->h_v;
  a.dk = p->dk;
  a.dv = p->dv;
  a.kda = kda ? 1 : 0;
  a.f32 = p->io_dtype == DRLA_F32 ? 1 : 0;
  a.f16 = p->io_dtype == DRLA_F16 ? 1 : 0;
  a.inspect = (flags & DRLA_KEEP_INTERMEDIATES) ? 1 : 0;
  a.decay_only = decay ? 1 : 0;
  a.serial = (flags & DRLA_SERIAL) ? 1 : 0;
  a.head_scan = uses_hs(p, nc, max_cps, kda, flags) ? 1 : 0;
  a.stream = stream;
  a.stage_events = stage_events;
  const hipError_t e = drla_launch(&a);
  if (e != hipSuccess) return fail(DRLA_ERR_HIP, "HIP launch failed: %s", hipGetErrorString(e));
  g_last_error.clear();
  return DRLA_OK;
}

drla_status run_decode(bool kda, bool decay, const drla_problem* p, const void* q, const void* k, const void* v,
                       const float* beta, const float* g, const float* h0, void* o, float* ht, void* stream) {
  if (decay) beta = nullptr;  // unused without the delta rule
  int64_t nc = 0;
  drla_status st = check_problem(p, nullptr, &nc);
  if (st != DRLA_OK) return st;
  if (p->total_tokens != p->n_seqs)
    return fail(DRLA_ERR_SHAPE, "decode: total_tokens (%lld) must equal n_seqs (%d), one token each",
                (long long)p->total_tokens, p->n_seqs);
  if (!q || !k || !v || (!beta && !decay) || !g || !o)
    return fail(DRLA_ERR_NULL, decay ? "q, k, v, g and o must be non-NULL" : "q, k, v, beta, g and o must be non-NULL");
  const void* ptrs[] = {q, k, v, beta, g, h0, o, ht};
  for (const void* x : ptrs)
    if (x && !aligned16(x)) return fail(DRLA_ERR_ALIGN, "device pointers must be 16-byte aligned");
  const int64_t N = p->n_seqs;
  const size_t es = p->io_dtype == DRLA_F32 ? 4 : 2;
  const size_t nq = (size_t)N * p->h_qk * p->dk * es, nv = (size_t)N * p->h_v * p->dv * es;
  const size_t nb = (size_t)N * p->h_v * 4, ng = kda ? nb * p->dk : nb;
  const size_t ns = (size_t)N * p->h_v * p->dk * p->dv * 4;
  struct Buf {
    const void* p;
    size_t n;
  };
  const Buf ins[] = {{q, nq}, {k, nq}, {v, nv}, {beta, nb}, {g, ng}, {h0, ns}};
  const Buf outs[] = {{o, nv}, {ht, ns}};
  for (int i = 0; i < 2; ++i)
    for (const Buf& b : ins) {
      if (i == 1 && b.p == h0 && ht == h0) continue;  // in-place state update
      if (overlap(outs[i].p, outs[i].n, b.p, b.n))
        return fail(DRLA_ERR_ALIAS, "an output buffer overlaps an input buffer");
    }
  if (overlap(o, nv, ht, ns)) return fail(DRLA_ERR_ALIAS, "output buffers overlap");
  drla_decode_args a;
  memset(&a, 0, sizeof a);
  a.q = q;
  a.k = k;
  a.v = v;
  a.beta = beta;
  a.g = g;
  a.h0 = h0;
  a.o = o;
  a.ht = ht;
  a.n_seqs = p->n_seqs;
  a.h_qk = p->h_qk;
  a.h_v = p->h_v;
  a.dk = p->dk;
  a.dv = p->dv;
  a.kda = kda ? 1 : 0;
  a.f32 = p->io_dtype == DRLA_F32 ? 1 : 0;
  a.f16 = p->io_dtype == DRLA_F16 ? 1 : 0;
  a.decay_only = decay ? 1 : 0;
  a.stream = stream;
  const hipError_t e = drla_launch_decode(&a);
  if (e != hipSuccess) return fail(DRLA_ERR_HIP, "HIP launch failed: %s", hipGetErrorString(e));
  g_last_error.clear();
  return DRLA_OK;
}

}  // namespace

extern "C" {

drla_status gdn_decode(const drla_problem* p, const void* q, const void* k, const void* v, const float* beta,
                       const float* g, const float* h0, void* o, float* ht, void* stream) {
  return run_decode(false, false, p, q, k, v, beta, g, h0, o, ht, stream);
}

drla_status kda_decode(const drla_problem* p, const void* q, const void* k, const void* v, const float* beta,
                       const float* g, const float* h0, void* o, float* ht, void* stream) {
  return run_decode(true, false, p, q, k, v, beta, g, h0, o, ht, stream);
}

drla_status decay_prefill(int per_channel, const drla_problem* p, const void* q, const void* k, const void* v,
                          const float* g, const float* h0, const int32_t* cu_seqlens_dev,
                          const int32_t* cu_seqlens_host, void* o, float* ht, void* workspace,
                          size_t workspace_bytes, void* stream) {
  return run(per_channel != 0, DRLA_DECAY_ONLY, p, q, k, v, nullptr, g, h0, cu_seqlens_dev, cu_seqlens_host, o,
             ht, workspace, workspace_bytes, stream, nullptr);
}

drla_status decay_decode(int per_channel, const drla_problem* p, const void* q, const void* k, const void* v,
                         const float* g, const float* h0, void* o, float* ht, void* stream) {
  return run_decode(per_channel != 0, true, p, q, k, v, nullptr, g, h0, o, ht, stream);
}

size_t drla_workspace_bytes(const drla_problem* p, const int32_t* cu_seqlens_host) {
  // Enough for either gate kind: the larger of the two layouts.
  int64_t nc = 0;
  if (check_problem(p, cu_seqlens_host, &nc) != DRLA_OK) return 0;
  drla_layout L, G;
  const bool pk = packed(p, cu_seqlens_host);
  const int64_t mc = max_chunks(p, pk ? cu_seqlens_host : nullptr);
  layout_of(p, nc, pk, mc, true, 0, &L);
  layout_of(p, nc, pk, mc, false, 0, &G);
  return L.total > G.total ? L.total : G.total;
}

drla_status drla_workspace_layout(int kda, const drla_problem* p, const int32_t* cu_seqlens_host, int flags,
                                  drla_layout* out) {
  int64_t nc = 0;
  if (!out) return fail(DRLA_ERR_NULL, "layout output is NULL");
  drla_status st = check_problem(p, cu_seqlens_host, &nc);
  if (st != DRLA_OK) return st;
  if ((st = check_flags(flags)) != DRLA_OK) return st;
  const bool pk = packed(p, cu_seqlens_host);
  layout_of(p, nc, pk, max_chunks(p, pk ? cu_seqlens_host : nullptr), kda != 0, flags, out);
  return DRLA_OK;
}

drla_status gdn_prefill(const drla_problem* p, const void* q, const void* k, const void* v, const float* beta,
                        const float* g, const float* h0, const int32_t* cu_seqlens_dev,
                        const int32_t* cu_seqlens_host, void* o, float* ht, void* workspace,
                        size_t workspace_bytes, void* stream) {
  return run(false, 0, p, q, k, v, beta, g, h0, cu_seqlens_dev, cu_seqlens_host, o, ht, workspace,
             workspace_bytes, stream, nullptr);
}

drla_status kda_prefill(const drla_problem* p, const void* q, const void* k, const void* v, const float* beta,
                        const float* g, const float* h0, const int32_t* cu_seqlens_dev,
                        const int32_t* cu_seqlens_host, void* o, float* ht, void* workspace,
                        size_t workspace_bytes, void* stream) {
  return run(true, 0, p, q, k, v, beta, g, h0, cu_seqlens_dev, cu_seqlens_host, o, ht, workspace,
             workspace_bytes, stream, nullptr);
}

drla_status drla_prefill_ex(int kda, int flags, const drla_problem* p, const void* q, const void* k,
                            const void* v, const float* beta, const float* g, const float* h0,
                            const int32_t* cu_seqlens_dev, const int32_t* cu_seqlens_host, void* o,
                            float* ht, void* workspace, size_t workspace_bytes, void* stream,
                            void* const* stage_events) {
  return run(kda != 0, flags, p, q, k, v, beta, g, h0, cu_seqlens_dev, cu_seqlens_host, o, ht, workspace,
             workspace_bytes, stream, stage_events);
}

drla_status drla_prefill_noalloc(int kda, int flags, const drla_problem* p, const void* q, const void* k,
                                 const void* v, const float* beta, const float* g, const float* h0,
                                 const int32_t* cu_seqlens_dev, const int32_t* cu_seqlens_host, void* o,
                                 float* ht, void* stream) {
  // the workspace this call needs, checked against the scratch array before
  // anything touches the device
  drla_layout L;
  const drla_status st = drla_workspace_layout(kda, p, cu_seqlens_host, flags, &L);
  if (st != DRLA_OK) return st;
  if (L.total > DRLA_NOALLOC_SCRATCH_BYTES)
    return fail(DRLA_ERR_WORKSPACE,
                "drla_prefill_noalloc: this call needs %zu bytes of scratch, more than the %llu bytes the "
                "library holds; call gdn_prefill / kda_prefill with a workspace instead",
                L.total, (unsigned long long)DRLA_NOALLOC_SCRATCH_BYTES);
  void* ws = nullptr;
  if (L.total > 0) {
    const drla_status sa = scratch_address(&ws);
    if (sa != DRLA_OK) return sa;
  }
  return run(kda != 0, flags, p, q, k, v, beta, g, h0, cu_seqlens_dev, cu_seqlens_host, o, ht, ws,
             ws ? (size_t)DRLA_NOALLOC_SCRATCH_BYTES : 0, stream, nullptr);
}

drla_status drla_prefill_status(const drla_problem* p, const int32_t* cu_seqlens_host, const void* workspace,
                                void* stream) {
  int64_t nc = 0;
  const drla_status st = check_problem(p, cu_seqlens_host, &nc);
  if (st != DRLA_OK) return st;
  if (!packed(p, cu_seqlens_host) || p->n_seqs < 1) return DRLA_OK;  // no device lengths read
  drla_layout L;
  layout_of(p, nc, true, max_chunks(p, cu_seqlens_host), false, 0, &L);
  const void* ws = workspace;
  if (!ws) {
    void* sp = nullptr;
    const drla_status sa = scratch_address(&sp);
    if (sa != DRLA_OK) return sa;
    ws = sp;
  }
  if (!aligned16(ws)) return fail(DRLA_ERR_ALIGN, "device pointers must be 16-byte aligned");
  const char* word = (const char*)ws + L.sched + (size_t)drla_sched_status(nc, p->n_seqs) * 4;
  int32_t v = -1;
  hipStream_t s = (hipStream_t)stream;
  hipError_t e = hipMemcpyAsync(&v, word, sizeof v, hipMemcpyDeviceToHost, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  if (e != hipSuccess) return fail(DRLA_ERR_HIP, "reading the status word failed: %s", hipGetErrorString(e));
  if (v == 0) {
    g_last_error.clear();
    return DRLA_OK;
  }
  if (v == 1)
    return fail(DRLA_ERR_SEQLENS,
                "cu_seqlens_dev differed from cu_seqlens_host: the call ran as empty sequences "
                "(o not written, final states = initial states)");
  return fail(DRLA_ERR_SEQLENS, "no status word (%d): no packed call has run on this workspace", (int)v);
}

const char* drla_status_str(drla_status s) {
  switch (s) {
    case DRLA_OK: return "ok";
    case DRLA_ERR_NULL: return "null pointer";
    case DRLA_ERR_SHAPE: return "bad shape";
    case DRLA_ERR_UNSUPPORTED: return "unsupported size or dtype";
    case DRLA_ERR_ALIGN: return "misaligned pointer";
    case DRLA_ERR_SEQLENS: return "bad cu_seqlens";
    case DRLA_ERR_WORKSPACE: return "workspace too small";
    case DRLA_ERR_ALIAS: return "overlapping buffers";
    case DRLA_ERR_HIP: return "HIP error";
  }
  return "unknown status";
}

const char* drla_last_error(void) { return g_last_error.c_str(); }

int drla_version(void) { return 7; }

}  // extern "C"
