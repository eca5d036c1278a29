// Internal interface between the C ABI layer (drla_api.cpp) and the kernel
// launcher (drla_launch.hip).  Not part of the public ABI.
#ifndef DRLA_LAUNCH_H
#define DRLA_LAUNCH_H
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#define DRLA_CHUNK_TOKENS 64

typedef struct {
  const void* q;
  const void* k;
  const void* v;
  const float* beta;
  const float* g;
  const float* h0;
  const int32_t* cu_dev;  // NULL for a dense batch
  void* o;
  float* ht;
  void* workspace;
  // byte offsets into the workspace; vp/h only used when inspect != 0
  size_t off_sched, off_tb, off_pm, off_kt, off_kw, off_qw, off_gam, off_vp, off_h;
  size_t off_seg;  // 0, or the segment-mode scan's G and states (dense calls)
  int64_t total_tokens;
  int64_t n_chunks;
  int32_t n_seqs, h_qk, h_v, dk, dv;
  int32_t kda, f32, f16, inspect;  // f32 / f16: io dtype (neither: bf16)
  int32_t decay_only;              // decay-only linear attention (no delta rule)
  int32_t serial;                  // scan every sequence in one pass (no segment split)
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
