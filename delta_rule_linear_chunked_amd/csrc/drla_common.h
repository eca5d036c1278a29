// Device helpers shared by the prep and scan kernels (gfx950 / CDNA4).
//
// Fragment order.  A 16x16 MFMA accumulator tile holds, in lane l
// (g = l/16, c = l%16), element [4g + e][c] for e = 0..3.  An operand
// fragment covers 16 "outer" indices x 32 contraction ("inner") indices;
// lane l holds 8 elements of outer index c at inner positions
//   kmap(g, j) = 4g + j           (j < 4)
//              = 16 + 4g + j - 4  (j >= 4).
// The A and the B operand use the same map, so every product sums over the
// same index pairs whatever the map is.  With this map the two accumulator
// tiles of rows [32p, 32p+16) and [32p+16, 32p+32) of a product are, lane by
// lane, the operand fragment of inner block p (rows become the contraction
// index, columns the outer index): a result feeds the next product without
// leaving registers.  Intermediates in the workspace are stored as such
// fragments, 64 lanes x 8 elements contiguous (1 KiB in bf16, 2 KiB in
// fp32), so every access is one coalesced 16- or 32-byte access per lane.
#ifndef DRLA_COMMON_H
#define DRLA_COMMON_H

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "drla_launch.h"

namespace drla {

typedef __bf16 bf16;
typedef bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16;
typedef f16 f16x4 __attribute__((ext_vector_type(4)));
typedef f16 f16x8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef float floatx8 __attribute__((ext_vector_type(8)));

constexpr int C = DRLA_CHUNK_TOKENS;  // tokens per chunk

template <typename ET> struct VT;
template <> struct VT<bf16> {
  typedef bf16x4 v4;    // 4 elements (8 bytes)
  typedef bf16x8 v8;    // one fragment slot set (16 bytes)
  typedef bf16x8 v16b;  // one 16-byte vector
  static constexpr int per16 = 8;
};
template <> struct VT<f16> {
  typedef f16x4 v4;
  typedef f16x8 v8;
  typedef f16x8 v16b;
  static constexpr int per16 = 8;
};
template <> struct VT<float> {
  typedef floatx4 v4;
  typedef floatx8 v8;
  typedef floatx4 v16b;
  static constexpr int per16 = 4;
};

// D += A B over one 32-wide inner block (bf16, fp16: one
// v_mfma_f32_16x16x32_bf16 / _f16; fp32: eight v_mfma_f32_16x16x4_f32, slot
// j of every lane in step j).
__device__ __forceinline__ floatx4 mma(const bf16x8& a, const bf16x8& b, floatx4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ floatx4 mma(const f16x8& a, const f16x8& b, floatx4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ floatx4 mma(const floatx8& a, const floatx8& b, floatx4 c) {
#pragma unroll
  for (int j = 0; j < 8; ++j) c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[j], b[j], c, 0, 0, 0);
  return c;
}

// Workgroup barrier for LDS traffic only: waits for this wave's LDS
// operations, not for its outstanding global loads (__syncthreads() would
// drain those too and so defeat loads issued ahead of use).
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

__device__ __forceinline__ int kmap(int g, int j) { return j < 4 ? 4 * g + j : 12 + 4 * g + j; }

// Transposing LDS read of 16-bit elements (ds_read_b64_tr_b16): within a
// 16-lane group, lane i receives element i % 4 of the four-element 8-byte
// segments addressed by lanes 4j + i / 4, j = 0..3.  `p` must be 8-byte
// aligned.
template <typename ET>
__device__ __forceinline__ typename VT<ET>::v4 lds_read_tr16(const void* p) {
  typedef short s4 __attribute__((ext_vector_type(4)));
  const s4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s4*)(p));
  return __builtin_bit_cast(typename VT<ET>::v4, v);
}

// The 48 of the 64 128-byte lines of a (head, chunk)'s eight 16x32
// fragments that hold fragments 0, 2, 4, 5, 6 and 7 (1 and 3 lie above the
// diagonal and are never stored): lane l's line for an L2 touch of the six;
// lanes 48..63 repeat lines 48..63.
__device__ __forceinline__ int frag_line(int l) { return l < 8 ? l : l < 16 ? l + 8 : l < 48 ? l + 16 : l; }

__device__ __forceinline__ floatx4 zero4() { return floatx4{0.f, 0.f, 0.f, 0.f}; }

template <typename ET>
__device__ __forceinline__ typename VT<ET>::v8 cat(typename VT<ET>::v4 lo, typename VT<ET>::v4 hi) {
  return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}

// Two accumulator tiles -> one fragment, rounded to ET (round to nearest even).
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

template <typename ET>
__device__ __forceinline__ typename VT<ET>::v4 pack4(const floatx4& a) {
  typename VT<ET>::v4 r;
#pragma unroll
  for (int j = 0; j < 4; ++j) r[j] = (ET)a[j];
  return r;
}

// Fragment slots of one row of a row-major array; `row` points at inner
// index 0 of the 32-wide block.
template <typename ET>
__device__ __forceinline__ typename VT<ET>::v8 row_slots(const ET* row, int g) {
  typedef typename VT<ET>::v4 V4;
  return cat<ET>(*(const V4*)(row + 4 * g), *(const V4*)(row + 16 + 4 * g));
}

template <typename ET>
__device__ __forceinline__ float to_f(ET x) { return (float)x; }

// Raw buffer access (bounds-checked by the hardware: a load past
// `num_records` bytes returns zero, a store there is dropped).
typedef __amdgpu_buffer_rsrc_t rsrc_t;
__device__ __forceinline__ rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
template <typename V> __device__ __forceinline__ V bload(rsrc_t r, uint32_t off);
template <> __device__ __forceinline__ float bload<float>(rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0));
}
template <> __device__ __forceinline__ bf16x4 bload<bf16x4>(rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(bf16x4, __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0));
}
template <> __device__ __forceinline__ bf16x8 bload<bf16x8>(rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}
template <> __device__ __forceinline__ f16x4 bload<f16x4>(rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(f16x4, __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0));
}
template <> __device__ __forceinline__ f16x8 bload<f16x8>(rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(f16x8, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}
template <> __device__ __forceinline__ floatx4 bload<floatx4>(rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(floatx4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}
template <> __device__ __forceinline__ floatx8 bload<floatx8>(rsrc_t r, uint32_t off) {
  const floatx4 lo = bload<floatx4>(r, off), hi = bload<floatx4>(r, off + 16);
  return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}
// Fragment `f` (64 lanes x 16 or 32 bytes) of a fragment array through a
// buffer resource: the per-lane offset is loop-invariant and the fragment
// offset is a scalar, so no per-load address arithmetic lands in VGPRs.
template <typename V>
__device__ __forceinline__ V fload(rsrc_t r, uint32_t lane_off, int f) {
  if constexpr (sizeof(V) == 16) {
    return __builtin_bit_cast(V, __builtin_amdgcn_raw_buffer_load_b128(r, lane_off, f * 64 * 16, 0));
  } else {
    const floatx4 lo = __builtin_bit_cast(floatx4, __builtin_amdgcn_raw_buffer_load_b128(r, lane_off, f * 64 * 32, 0));
    const floatx4 hi = __builtin_bit_cast(floatx4, __builtin_amdgcn_raw_buffer_load_b128(r, lane_off + 16, f * 64 * 32, 0));
    return __builtin_bit_cast(V, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
  }
}

// LDS-direct buffer loads: lane l's 16 (4) bytes at byte offset voff + soff
// of the buffer land at lds + 16 l (4 l).  Callers keep soff = 0 and put the
// whole offset in voff, which the hardware range check covers: a read past
// the buffer's size returns zero.  The instruction offset stays 0 (it would
// move the LDS side too).  They count in vmcnt only.
typedef __attribute__((address_space(3))) void lds_void;
__device__ __forceinline__ void lds_dma16(rsrc_t r, uint32_t voff, uint32_t soff, void* lds) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)lds, 16, voff, soff, 0, 0);
}
__device__ __forceinline__ void lds_dma4(rsrc_t r, uint32_t voff, uint32_t soff, void* lds) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)lds, 4, voff, soff, 0, 0);
}

// s_waitcnt immediate that waits for at most n outstanding vector memory
// operations (gfx9 encoding: vmcnt bits [3:0] and [15:14]) and nothing else.
constexpr int vmcnt_imm(int n) { return 0x0F70 | (n & 0xF) | ((n >> 4) << 14); }

__device__ __forceinline__ void bstore(rsrc_t r, uint32_t off, f16x4 v) {
  __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2, v), r, off, 0, 0);
}
__device__ __forceinline__ void bstore(rsrc_t r, uint32_t off, bf16x4 v) {
  __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2, v), r, off, 0, 0);
}
__device__ __forceinline__ void bstore(rsrc_t r, uint32_t off, floatx4 v) {
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), r, off, 0, 0);
}

// Key-channel order of the scan's state rows.  State tile mt (16 rows), row
// 4g + e holds key channel 32 (mt/2) + 8g + 4 (mt%2) + e, so that the state
// fragment of inner block p has contiguous channels 32p + 8g + j in slot j:
// the K and Q row fragments it multiplies are single 16-byte loads.
__device__ __forceinline__ int state_row(int mt, int rho) {
  return 32 * (mt >> 1) + 8 * (rho >> 2) + 4 * (mt & 1) + (rho & 3);
}

// Chunk schedule.  Packed input (cu_seqlens): a device table built by
// schedule_kernel.  Dense batch: N sequences of seq_len tokens.
struct Sched {
  const int32_t* chunk_seq;    // [nc] sequence of each chunk (packed input), else null
  const int32_t* chunk_start;  // [nc] first token of each chunk
  const int32_t* seq_chunk0;   // [N+1] first chunk of each sequence
  const int32_t* seq_order;    // [N] sequences, longest first (packed input), else null
  const int32_t* cu;           // [N+1] cu_seqlens as checked by schedule_kernel (packed input)
  int64_t seq_len;             // dense batch: tokens per sequence
  int32_t cps;                 // dense batch: chunks per sequence
  int32_t n_seqs;
};

// Chunk c -> (sequence, first token, valid length).  An entry that is
// inconsistent with the device lengths yields an empty chunk.
__device__ __forceinline__ void chunk_of(const Sched& s, int64_t c, int& seq, int64_t& t0, int& len) {
  if (s.chunk_seq) {
    seq = s.chunk_seq[c];
    if (seq < 0 || seq >= s.n_seqs) {
      seq = 0;
      t0 = 0;
      len = 0;
      return;
    }
    t0 = s.chunk_start[c];
    const int64_t n = (int64_t)s.cu[seq + 1] - t0;
    len = (int)(n < 0 ? 0 : (n > C ? C : n));
  } else {
    seq = (int)(c / s.cps);
    const int64_t local = c - (int64_t)seq * s.cps;
    t0 = (int64_t)seq * s.seq_len + local * C;
    const int64_t n = s.seq_len - local * C;
    len = (int)(n > C ? C : n);
  }
}

// Scan workgroup -> (sequence, value head, column block).  The hardware
// deals workgroups to the eight XCDs round-robin by index, so the column
// blocks of one (sequence, head) unit, which read the same K, Q and prep
// operands, are given indices that land on one XCD and share its L2.  Dense
// batch: units in order.  Packed input: units are dealt longest sequence
// first, unit rank r to XCD r % 8, so that the longest chains start first
// on every XCD; the grid then covers a multiple of eight units and the
// workgroups past the last unit have nothing to do (returns false).
__device__ __forceinline__ bool scan_item(const Sched& s, int h_v, int nbk, int& seq, int& h, int& nb) {
  const int bid = blockIdx.x, G = gridDim.x;
  if (s.seq_order) {
    const int y = bid / 8;
    const int r = (y / nbk) * 8 + bid % 8;
    nb = y % nbk;
    if (r >= s.n_seqs * h_v) return false;
    seq = s.seq_order[r / h_v];
    h = r % h_v;
    return seq >= 0 && seq < s.n_seqs;
  }
  const int b = G % 8 == 0 ? (bid % 8) * (G / 8) + bid / 8 : bid;
  const int unit = b / nbk;
  nb = b - unit * nbk;
  seq = unit / h_v;
  h = unit - seq * h_v;
  return true;
}

// Segment-mode scan workgroup -> (unit, column block, kind, segment):
// kind 1 = segment 0; for segments 1 .. np - 1, kind 2 = from zero, 3 =
// transition, or with `pair` kind 4 = both chains in one workgroup.
// (2 np - 1) K workgroups (pair: np K) for K = units x nbk, all resident at
// once.  A unit's workgroups take consecutive places in one XCD's share of
// the indices (when the count is a multiple of 8), so that its segments,
// and a segment's value and transition blocks, mostly share an L2.
__device__ __forceinline__ void seg_item(int units, int nbk, int np, bool pair, int& unit, int& nb, int& kind,
                                         int& sg) {
  const int bid = blockIdx.x, per = (pair ? np : 2 * np - 1) * nbk, W = units * per;
  const int l = W % 8 == 0 ? (bid % 8) * (W / 8) + bid / 8 : bid;
  unit = l / per;
  int r = l - unit * per;
  if (r < nbk) {
    kind = 1;
    sg = 0;
    nb = r;
  } else if (pair) {
    r -= nbk;
    sg = 1 + r / nbk;
    kind = 4;
    nb = r % nbk;
  } else {
    r -= nbk;
    sg = 1 + r / (2 * nbk);
    r -= (sg - 1) * 2 * nbk;
    kind = 2 + r / nbk;
    nb = r % nbk;
  }
}

// Chunks [first, first + len) of segment sg of a sequence of n chunks cut
// into np segments, segment 0 weighted w0 / 256 against each later one:
// the later segments take ls = floor(256 n / (w0 + 256 (np - 1))) chunks
// each, segment 0 the rest (all of them when n is below np).
__device__ __forceinline__ void seg_span(int64_t n, int np, int w0, int sg, int64_t& first, int64_t& len) {
  const int64_t ls = (256 * n) / (w0 + 256 * (np - 1));
  const int64_t n0 = n - (np - 1) * ls;
  first = sg == 0 ? 0 : n0 + (sg - 1) * ls;
  len = sg == 0 ? n0 : ls;
}

// Chunks [c0, c1) of sequence `seq`, clamped to [0, nc).
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

}  // namespace drla

#endif
