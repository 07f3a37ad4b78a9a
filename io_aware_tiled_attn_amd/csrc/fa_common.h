// Device-side helpers shared by the attention kernels (gfx950 / CDNA4).
//
// Register layouts used throughout (wave64, v_mfma_f32_32x32x16_bf16):
//   A operand  (32 x 16, row-major in the math): lane l holds row l % 32,
//              k = 8 * (l / 32) + 0..7 as 8 consecutive bf16.
//   B operand  (16 x 32): lane l holds column l % 32, k = 8 * (l / 32) + 0..7.
//   C/D        (32 x 32 fp32): lane l, register r holds row
//              8 * (r / 4) + 4 * (l / 32) + (r % 4), column l % 32.
// A product whose output feeds the next product as an operand therefore keeps
// the "column" dimension in the lane index; the kernels arrange their
// products so each lane owns one query (forward) or one key (backward).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fa_layout.h"

namespace fa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ f32x16 mfma32h(f16x8 a, f16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}

// Both halves of the wave exchange values with the lane 32 away and return
// the pair (own, partner) in some order; callers only combine symmetrically.
__device__ __forceinline__ float max_with_lane_xor32(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

__device__ __forceinline__ float sum_with_lane_xor32(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// fp32 -> bf16 pair, round to nearest even (v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  bf16x2 v = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, v);
}

// fp32 -> fp16 pair, round to nearest even (v_cvt_pk_f16_f32).
__device__ __forceinline__ uint32_t pack_f16x2(float lo, float hi) {
  f16x2 v = {(_Float16)lo, (_Float16)hi};
  return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Low halves of a and b as one word (a in the low 16 bits).
__device__ __forceinline__ uint32_t pack_lo16(uint32_t a, uint32_t b) {
  return __builtin_amdgcn_perm(b, a, 0x05040100u);
}
// High halves of a and b as one word (a's high half in the low 16 bits).
__device__ __forceinline__ uint32_t pack_hi16(uint32_t a, uint32_t b) {
  return __builtin_amdgcn_perm(b, a, 0x07060302u);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

// Transposed operand reads from a row-major LDS matrix M with ds_read_b64_tr_b16.
// That instruction hands lane j of each 16-lane group element j % 4 of the
// 8-byte word read by lane 4 e + j / 4 of the group, for e = 0..3; so when
// lane s of a group reads row s / 4 at column 4 (s % 4) of a 4 x 16 block,
// lane j receives the 4 rows of column j.  Two such reads give the 8 k-values
// of an MFMA A or B operand whose k-dimension runs down M's rows.
//
// tr_lane_off is the lane-dependent part of the element offset: lane l reads
// column l % 32 of its block; lane half g = l / 32 starts `half_rows` rows
// further down.  Callers add compile-time row/column offsets.
__device__ __forceinline__ int tr_lane_off(int lane, int pitch, int half_rows) {
  const int s = lane & 15, G = (lane >> 4) & 1, g = lane >> 5;
  return (half_rows * g + (s >> 2)) * pitch + 16 * G + 4 * (s & 3);
}

// p already includes tr_lane_off; lo and hi are element offsets of the two
// 4-row groups (slots 0..3 and 4..7 of the result).
__device__ __forceinline__ bf16x8 lds_tr_pair(const __bf16* p, int lo, int hi) {
  s16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p + lo));
  s16x4 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p + hi));
  typedef short s16x8 __attribute__((ext_vector_type(8)));
  s16x8 r = {a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
  return __builtin_bit_cast(bf16x8, r);
}

// The same two transposed reads as an fp16 operand.
__device__ __forceinline__ f16x8 lds_tr_pair_h(const _Float16* p, int lo, int hi) {
  s16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p + lo));
  s16x4 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p + hi));
  typedef short s16x8 __attribute__((ext_vector_type(8)));
  s16x8 r = {a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
  return __builtin_bit_cast(f16x8, r);
}

// Power-of-two factor 2^e that brings the largest magnitude `amax` of a
// tensor into [1, 2) (1 when amax is 0 or not finite); e is kept within
// +-126 so the factor and its inverse are normal fp32 numbers.
__device__ __forceinline__ float pow2_scale_for(float amax) {
  if (!(amax > 0.f) || !(amax <= 3.0e38f)) return 1.f;
  int E;
  (void)frexpf(amax, &E);   // amax = m 2^E, m in [0.5, 1)
  const int e = min(126, max(-126, 1 - E));
  return ldexpf(1.f, e);
}

// Buffer descriptor over `bytes` bytes at p (raw, 32-bit data format):
// loads at offsets >= bytes return 0 and atomics there are dropped.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ u32x4 bload128(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}
__device__ __forceinline__ u32x2 bload64(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0));
}
__device__ __forceinline__ float bload32f(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0));
}
__device__ __forceinline__ void batomic_add(__amdgpu_buffer_rsrc_t r, uint32_t off, float v) {
  __builtin_amdgcn_raw_ptr_buffer_atomic_fadd_f32(v, r, (int)off, 0, 0);
}

// One buffer_load_dwordx4 ... lds: each lane's 16 bytes at byte offset goff
// of the buffer go to LDS address lds_addr + 16 * lane (lds_addr is uniform
// and travels in M0).  Written as inline assembly so that the compiler does
// not guard every later LDS read of this wave with a wait for the copy (it
// cannot tell which LDS bytes the copy writes); the kernel orders the copy
// itself, with an explicit vmcnt wait and a barrier before any read of the
// bytes it fills.
__device__ __forceinline__ void lds_copy16(__amdgpu_buffer_rsrc_t r, uint32_t goff, uint32_t lds_addr) {
  asm volatile("s_nop 0\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds" ::"v"(goff), "s"(r), "{m0}"(lds_addr)
               : "memory");
}

// s_waitcnt vmcnt(0), leaving the other counters alone.
__device__ __forceinline__ void wait_vmem_all() { __builtin_amdgcn_s_waitcnt(0x0F70); }
// s_waitcnt vmcnt(N): all but the N most recent vector memory loads have
// completed (they complete in issue order); the other counters untouched.
template <int N>
__device__ __forceinline__ void wait_vmem_keep() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt(0x0F70 | (N & 15) | ((N >> 4) << 14));
}

// s_waitcnt vmcnt(N) that the compiler must place before any use of `addr`
// (passed through the asm): an LDS read at an address derived from it cannot
// move above the wait.  For reading bytes this wave's own global -> LDS
// copies wrote, with no workgroup barrier in between.
template <int N>
__device__ __forceinline__ void wait_vmem_keep_before(int& addr) {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%1)" : "+v"(addr) : "n"(N));
}

// Work order for a launch of num_tiles x BH workgroups (tile-major work
// items of BH heads).  The dispatcher hands workgroup i to XCD i % 8, and
// each XCD has its own L2.  When BH is a multiple of 8, XCD x takes heads
// x, x + 8, ... one after another, all tiles of a head before the next
// head, tile 0 first: the tiles running together on an XCD then share one
// or two heads' K/V (forward) or dQ accumulator (backward) in its L2.
// Otherwise workgroups take tiles in order with the head index varying
// fastest.
__device__ __forceinline__ void xcd_head_major(int bid, int BH, int num_tiles, int& bh, int& tile) {
  if ((BH & 7) == 0) {
    layout::xcd_head_major_item(bid & 7, bid >> 3, num_tiles, bh, tile);
  } else {
    tile = bid / BH;
    bh = bid % BH;
  }
}

// Row-wise output of a 32 x D tile held as transposed-product accumulators
// (lane l: row l % 32; register r of 32-column block dm: columns
// 32 dm + 8 (r / 4) + 4 (l / 32) + r % 4), rounded to bf16 after a multiply
// by `fac`, through LDS, so that each global store instruction writes 1 KB
// of whole row segments (instead of 16 bytes in each of 32 rows).
// stage_rows puts the W columns of blocks dm0 .. dm0 + W / 32 - 1 into the
// 64 W bytes at `stage` (layout::fwd_ostage_off for a W-column tile);
// write_staged_rows reads them back 1 KB at a time and stores the rows
// q0 .. q0 + 31 below N at out + row * pitch (W columns each).  A wave's own
// LDS writes and reads stay in order, so a wave that stages and writes its
// own tile needs no barrier in between.  The lane index passes through an
// asm so the address arithmetic is done here, after the caller's main loop,
// instead of being hoisted above it and held in registers throughout.
template <int D, int W = D>
__device__ __forceinline__ void stage_rows(const f32x16 (&acc)[D / 32], float fac, __bf16* stage, int lane_in,
                                           int dm0 = 0) {
  static_assert(W % 32 == 0 && W <= D, "staged width");
  int lane = lane_in;
  asm volatile("" : "+v"(lane));
  const int lc = lane & 31, lg = lane >> 5;
#pragma unroll
  for (int b = 0; b < W / 32; ++b)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const f32x16& a = acc[dm0 + b];
      const u32x2 w = {pack_bf16x2(a[4 * i + 0] * fac, a[4 * i + 1] * fac),
                       pack_bf16x2(a[4 * i + 2] * fac, a[4 * i + 3] * fac)};
      *(u32x2*)(stage + layout::fwd_ostage_off<W>(lc, lg, b, i)) = w;
    }
}

template <int W>
__device__ __forceinline__ void write_staged_rows(const __bf16* stage, __bf16* out, int pitch, int q0, int N,
                                                  int lane_in) {
  int lane = lane_in;
  asm volatile("" : "+v"(lane));
  // All the reads first (they overlap), then the stores of rows below N.
  constexpr int kInst = 32 * W * 2 / 1024;
  u32x4 v[kInst];
#pragma unroll
  for (int j = 0; j < kInst; ++j) v[j] = *(const u32x4*)(stage + j * 512 + 8 * lane);
#pragma unroll
  for (int j = 0; j < kInst; ++j) {
    int row, chunk;
    layout::copy_slot(2 * W, j, lane, layout::FwdSwizzle<W>::k, row, chunk);
    if (q0 + row < N) *(u32x4*)(out + (size_t)(q0 + row) * pitch + 8 * chunk) = v[j];
  }
}

// A wave's whole tile: stage all its blocks into its own LDS, then write.
template <int D>
__device__ __forceinline__ void store_o_rows(const f32x16 (&acc)[D / 32], float fac, __bf16* stage, __bf16* out,
                                             int q0, int N, int lane) {
  stage_rows<D>(acc, fac, stage, lane);
  write_staged_rows<D>(stage, out, D, q0, N, lane);
}

}  // namespace fa
