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

// Each thread moves four 16-byte vectors per trip, all four loads issued
// before the first store.  n4 counts groups of four vectors (64 bytes).
__global__ __launch_bounds__(256) void copy_kernel(const u32x4* __restrict__ src,
                                                   u32x4* __restrict__ dst, int64_t n4) {
  const int64_t stride = (int64_t)gridDim.x * 256;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n4; i += stride) {
    const int64_t base = (i / 256) * 1024 + (i % 256);  // 256-thread groups of 4 x 256 vectors
    u32x4 x[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) x[j] = __builtin_nontemporal_load(&src[base + 256 * j]);
#pragma unroll
    for (int j = 0; j < 4; ++j) __builtin_nontemporal_store(x[j], &dst[base + 256 * j]);
  }
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

extern "C" int drla_peak_copy(const void* src, void* dst, size_t bytes, int blocks, void* stream) {
  if (!src || !dst || bytes == 0 || bytes % 64 != 0) return 1;
  if (((uintptr_t)src | (uintptr_t)dst) % 16 != 0) return 1;
  const char* s = (const char*)src;
  const char* d = (const char*)dst;
  if (s < d + bytes && d < s + bytes) return 1;
  const int64_t n4 = (int64_t)(bytes / 64);
  // the index map moves whole groups of 1024 vectors; a tail that is not a
  // whole group goes through a second launch with its own base
  const int64_t whole = (n4 / 256) * 256;
  if (blocks <= 0) {
    const int cus = cu_count();
    if (cus <= 0) return 2;
    blocks = 16 * cus;
  }
  hipStream_t st = (hipStream_t)stream;
  if (whole > 0) {
    const int64_t need = whole / 256;
    const int grid = (int)(need < blocks ? need : blocks);
    copy_kernel<<<grid, 256, 0, st>>>((const u32x4*)src, (u32x4*)dst, whole);
    if (hipGetLastError() != hipSuccess) return 2;
  }
  const int64_t rest = n4 - whole;  // < 256 groups of 64 bytes
  if (rest > 0) {
    const size_t off = (size_t)whole * 64;
    // rest groups of four vectors laid out with stride 256 vectors would
    // overrun; copy the tail as plain bytes
    if (hipMemcpyAsync((char*)dst + off, (const char*)src + off, (size_t)rest * 64,
                       hipMemcpyDeviceToDevice, st) != hipSuccess)
      return 2;
  }
  return 0;
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
