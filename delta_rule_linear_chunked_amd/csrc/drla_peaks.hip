// Attainable-peak microbenchmarks for gfx950 (libdrla_peaks.so): a
// streaming copy and independent chains of dependent MFMAs.  They price the
// prefill kernels' roofline against what the chip sustains; nothing of the
// prefill path calls them.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "drla_peaks.h"

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

int cu_count() {
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
  return cus;
}

// One 16-byte vector per thread, non-temporal both ways, one workgroup per
// 4 KiB: of the forms measured on the MI355X (grid-stride loops with 2 to 8
// vectors per thread, block tiles of 2 to 8 vectors, plain or non-temporal
// accesses, hipMemcpy) the fastest.
__global__ __launch_bounds__(256) void copy_kernel(const u32x4* __restrict__ src,
                                                   u32x4* __restrict__ dst, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i < n) __builtin_nontemporal_store(__builtin_nontemporal_load(&src[i]), &dst[i]);
}

// Eight accumulator chains per wave; every MFMA of a chain waits for the
// previous one, the eight chains keep the matrix core's pipeline full.
template <int KIND>
__global__ __launch_bounds__(256) void mfma_kernel(float* __restrict__ out, int iters) {
  const int lane = threadIdx.x & 63;
  floatx4 acc[8];
#pragma unroll
  for (int c = 0; c < 8; ++c) acc[c] = floatx4{0.f, 0.f, 0.f, 0.f};
  const float s = 1.0f / 1024.0f * (float)(lane + 1);
  if constexpr (KIND == 0) {
    bf16x8 a, b;
#pragma unroll
    for (int j = 0; j < 8; ++j) { a[j] = (__bf16)(s * (float)(j + 1)); b[j] = (__bf16)(s - 0.01f * (float)j); }
    for (int it = 0; it < iters; ++it) {
#pragma unroll
      for (int c = 0; c < 8; ++c) acc[c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc[c], 0, 0, 0);
    }
  } else if constexpr (KIND == 1) {
    f16x8 a, b;
#pragma unroll
    for (int j = 0; j < 8; ++j) { a[j] = (_Float16)(s * (float)(j + 1)); b[j] = (_Float16)(s - 0.01f * (float)j); }
    for (int it = 0; it < iters; ++it) {
#pragma unroll
      for (int c = 0; c < 8; ++c) acc[c] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, acc[c], 0, 0, 0);
    }
  } else {
    const float a = s, b = 1.0f - s;
    for (int it = 0; it < iters; ++it) {
#pragma unroll
      for (int c = 0; c < 8; ++c) acc[c] = __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, acc[c], 0, 0, 0);
    }
  }
  float t = 0.f;
#pragma unroll
  for (int c = 0; c < 8; ++c) t += acc[c][0] + acc[c][1] + acc[c][2] + acc[c][3];
  out[(int64_t)blockIdx.x * 256 + threadIdx.x] = t;
}

}  // namespace

extern "C" int drla_peak_copy(const void* src, void* dst, size_t bytes, void* stream) {
  if (!src || !dst || bytes == 0 || bytes % 16 != 0) return 1;
  if (((uintptr_t)src | (uintptr_t)dst) % 16 != 0) return 1;
  const char* s = (const char*)src;
  const char* d = (const char*)dst;
  if (s < d + bytes && d < s + bytes) return 1;
  const int64_t n = (int64_t)(bytes / 16);
  const int64_t blocks = (n + 255) / 256;
  if (blocks > 0x7fffffff) return 1;
  copy_kernel<<<(unsigned)blocks, 256, 0, (hipStream_t)stream>>>((const u32x4*)src, (u32x4*)dst, n);
  return hipGetLastError() == hipSuccess ? 0 : 2;
}

extern "C" int drla_peak_mfma_grid(int blocks) {
  if (blocks > 0) return blocks;
  const int cus = cu_count();
  return cus > 0 ? 8 * cus : 0;
}

extern "C" int drla_peak_mfma(float* out, int kind, int iters, int blocks, void* stream,
                              double* flops, int* grid) {
  if (!out || iters <= 0 || kind < 0 || kind > 2) return 1;
  const int g = drla_peak_mfma_grid(blocks);
  if (g <= 0) return 2;
  hipStream_t st = (hipStream_t)stream;
  if (kind == 0) mfma_kernel<0><<<g, 256, 0, st>>>(out, iters);
  else if (kind == 1) mfma_kernel<1><<<g, 256, 0, st>>>(out, iters);
  else mfma_kernel<2><<<g, 256, 0, st>>>(out, iters);
  if (hipGetLastError() != hipSuccess) return 2;
  const double per = kind == 2 ? 2.0 * 16 * 16 * 4 : 2.0 * 16 * 16 * 32;
  if (flops) *flops = per * 8.0 * (double)iters * 4.0 * (double)g;
  if (grid) *grid = g;
  return 0;
}
