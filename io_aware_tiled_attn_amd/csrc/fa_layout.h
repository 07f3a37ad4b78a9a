// Index math of the kernels' LDS tiles: which global row and 16-byte chunk
// each lane of a global -> LDS copy fetches, and where each lane's MFMA
// operand reads land; and the forward kernels' workgroup order.  Plain
// integer functions, compiled into the kernels and, on the host, into the
// checker that proves the copies and the reads agree for every tile shape
// the kernels accept, and that the order visits every (head, query tile)
// once (tests/layout_check.hip).
//
// All tiles hold rows of `row_bytes` bytes, unpadded, as 16-byte chunks;
// chunk c of row r is stored at chunk c ^ f(r) for a per-kernel
// permutation f, so that the rows a read instruction touches together fall
// into distinct LDS banks.  A copy instruction (buffer_load ... lds) fills
// 1 KB of a tile in lane order: lane i writes bytes 16 i .. 16 i + 15 of
// the instruction's kilobyte, so it must fetch the global chunk that the
// permutation stores there.
#pragma once

#include <hip/hip_runtime.h>

namespace fa {
namespace layout {

// Row and logical chunk that lane `lane` of copy instruction `inst` fetches
// into a tile of rows `row_bytes` wide, for the permutation f.
template <typename F>
__host__ __device__ inline void copy_slot(int row_bytes, int inst, int lane, F f, int& row, int& chunk) {
  const unsigned byte = (unsigned)inst * 1024u + 16u * (unsigned)lane;   // both are non-negative
  row = (int)(byte / (unsigned)row_bytes);
  chunk = (int)((byte % (unsigned)row_bytes) / 16u) ^ f(row);
}

// ---------------------------------------------------------------------------
// bf16 forward: K and V tiles of BN keys x D bf16 (row_bytes = 2 D).
//   K is read as the A operand of S^T = K Q^T: 16 lanes = 16 consecutive
//   rows at one chunk.  kf spreads 16 consecutive rows over all chunks.
//   V is read with ds_read_b64_tr_b16 (a half-wave covers 4 consecutive
//   rows x 4 consecutive chunks): vf moves each of 4 consecutive rows to a
//   different group of 4 chunks.  Rows per 256-byte bank sweep: 128 / D.
// ---------------------------------------------------------------------------
template <int D>
struct FwdSwizzle {
  static constexpr int kCpr = D / 8;     // chunks per row
  static constexpr int kRpb = 128 / D;   // rows per bank sweep
  __host__ __device__ static int k(int r) { return (r / kRpb) % kCpr; }
  __host__ __device__ static int v(int r) { return 4 * ((r / kRpb) % (kCpr / 4)); }
};

// Element offset of lane (lc, lg)'s K operand for k-step ks (row lc, chunk
// 2 ks + lg); the 32-row blocks of a tile add 32 D.
template <int D>
__host__ __device__ inline int fwd_koff(int lc, int lg, int ks) {
  return lc * D + 8 * ((2 * ks + lg) ^ FwdSwizzle<D>::k(lc));
}

// Element offset of lane's V^T operand read for 32-feature block dm: lane
// (s = lane % 16, G = bit 4, g = bit 5) reads row 4 g + s / 4 of each
// 8-row group at column 32 dm + 16 G + 4 (s % 4); 16-key steps add 16 D and
// the second half of a step 8 D.
template <int D>
__host__ __device__ inline int fwd_voff(int lane, int dm) {
  const int sl = lane & 15, G = (lane >> 4) & 1, g = lane >> 5;
  const int row = 4 * g + (sl >> 2);
  return row * D + 8 * ((4 * dm + 2 * G + ((sl & 3) >> 1)) ^ FwdSwizzle<D>::v(row)) + 4 * (sl & 1);
}

// Q staging of the forward prologue: each wave copies its 32 query rows
// (32 x D bf16, K's chunk permutation, so the B operand reads are the K
// tile's row reads) into a slot of the bytes the prologue leaves unused:
// the third K buffer, then the third V buffer (BN / 32 slots each), then
// slots past the six tile buffers.  Element offsets, with the LDS laid out
// as K buffers 0..2 | V buffers 0..2 of BN x D elements each.
template <int D, int BN>
__host__ __device__ inline int fwd_qslot(int wave) {
  constexpr int kTile = BN * D, kSlot = 32 * D, kPerBuf = BN / 32;
  if (wave < kPerBuf) return 2 * kTile + wave * kSlot;
  if (wave < 2 * kPerBuf) return 5 * kTile + (wave - kPerBuf) * kSlot;
  return 6 * kTile + (wave - 2 * kPerBuf) * kSlot;
}

// Elements past the six tile buffers that the Q slots of 8 waves need.
template <int D, int BN>
__host__ __device__ constexpr int fwd_qslot_extra() {
  return (8 - 2 * (BN / 32) > 0 ? 8 - 2 * (BN / 32) : 0) * 32 * D;
}

// Output staging of the forward epilogue: a wave's 32 x D tile of O (bf16,
// row = query) in LDS with K's chunk permutation.  Lane (lc, lg) writes the
// 4 features 32 dm + 8 i + 4 lg .. + 3 of query lc (element offset below);
// the tile is then read back 1 KB per instruction in lane order, lane i
// taking the row and logical chunk that copy_slot(2 D, inst, i,
// FwdSwizzle<D>::k) names, so each instruction's global stores cover
// consecutive whole rows.
template <int D>
__host__ __device__ inline int fwd_ostage_off(int lc, int lg, int dm, int i) {
  return lc * D + 8 * ((4 * dm + i) ^ FwdSwizzle<D>::k(lc)) + 4 * lg;
}

// ---------------------------------------------------------------------------
// FP8 forward: K and V tiles of BN keys x D bytes (E4M3).
//   K rows are read as A operands of v_mfma_f32_32x32x64_f8f6f4, two
//   chunks per lane; row rho of each 32-key block of S^T holds key
//   fp8_kperm(rho).  V^T is read with ds_read_b64_tr_b8.
// ---------------------------------------------------------------------------
template <int D>
struct Fp8Swizzle {
  static constexpr int kCpr = D / 16;
  static constexpr int kRps = 256 / D;
  // K: the 16 rows one 16-lane read covers differ in (r % kRps, k(r)).
  __host__ __device__ static int k(int r) { return ((r / kRps) & (kCpr / 2 - 1)) | (((r >> 4) & 1) * (kCpr / 2)); }
  // V: 8 consecutive rows differ in (r % kRps, v(r)), and v(r) is even so
  // the two adjacent chunks a 32-lane read covers stay apart.
  __host__ __device__ static int v(int r) { return 2 * ((r / kRps) % (8 / kRps)); }
};

__host__ __device__ inline int fp8_kperm(int rho) {
  return (((rho >> 2) & 1) << 4) | (((rho >> 3) & 3) << 2) | (rho & 3);
}

// Byte offset of lane (lc, lg)'s K operand chunk p (0, 1) of k-step ks.
template <int D>
__host__ __device__ inline int fp8_koff(int lc, int lg, int ks, int p) {
  const int kr = fp8_kperm(lc);
  return kr * D + 16 * ((4 * ks + 2 * lg + p) ^ Fp8Swizzle<D>::k(kr));
}

// Byte offset of lane's first V^T read for 32-feature block dm: 16-lane
// group G reads rows 16 g + 0..7 of chunk 2 dm + G, lane s = lane % 16
// addressing row s / 2, bytes 8 (s % 2); the operand's other reads sit 8,
// 32 and 40 rows further down, and 64-key steps add 64 D.
template <int D>
__host__ __device__ inline int fp8_voff(int lane, int dm) {
  const int sl = lane & 15, G = (lane >> 4) & 1, g = lane >> 5;
  const int row = 16 * g + (sl >> 1);
  return row * D + 16 * ((2 * dm + G) ^ Fp8Swizzle<D>::v(row)) + 8 * (sl & 1);
}

// ---------------------------------------------------------------------------
// Backward: fp16 tiles of D columns (row_bytes = 2 D), read both as rows
// (ds_read_b128; 16 lanes = 16 consecutive rows at one chunk) and as
// columns (ds_read_b64_tr_b16; 32 lanes = 4 consecutive rows x 4
// consecutive chunks, half a chunk each).  With t = r / (128 / D) (the rows
// of one 256-byte bank sweep share t) and L = D / 32,
// f = 4 (t % L) + (t / L) % 4: a bijection on the rows of each 16-row group
// that also puts each of 4 consecutive rows into a different aligned group
// of 4 chunks.
// ---------------------------------------------------------------------------
template <int D>
__host__ __device__ inline int bwd_swz(int r) {
  constexpr int kRpb = 128 / D, kL = D / 32;
  const int t = r / kRpb;
  return ((t % kL) << 2) | ((t / kL) & 3);
}

// Element offset of chunk c (8 fp16 elements) of row r.
template <int D>
__host__ __device__ inline int bwd_chunk_off(int r, int c) {
  return r * D + 8 * (c ^ bwd_swz<D>(r));
}

// This lane's element offset for the transposing read of rows r0 .. r0 + 3
// (lanes 0-31; lanes 32-63: rows r0 + 4 .. r0 + 7) at columns
// 32 dm .. 32 dm + 31: lane s = l % 16, G = bit 4, g = bit 5 reads half a
// chunk of row r0 + 4 g + s / 4 at column 32 dm + 16 G + 4 (s % 4).
template <int D>
__host__ __device__ inline int bwd_tr_off(int lane, int r0, int dm) {
  const int s = lane & 15, G = (lane >> 4) & 1, g = lane >> 5;
  return bwd_chunk_off<D>(r0 + 4 * g + (s >> 2), 4 * dm + 2 * G + ((s & 3) >> 1)) + 4 * (s & 1);
}

// Q and dO staging of the dQ kernel's prologue: slot w (byte offset) holds
// the 32 x D fp16 rows that wave w copies (waves 0-3 Q, waves 4-7 dO of
// query block w % 4), in the bwd_swz layout.  The LDS holds each group's
// three block buffers of S = 128 D bytes (K rows, then V rows) at
// g 3 S + b S; slots 0-3 fill the third buffers of both groups, slots 4-7
// follow the six buffers.
template <int D>
__host__ __device__ constexpr int bwd_dq_qslot(int w) {
  return w < 4 ? (w >> 1) * 3 * (128 * D) + 2 * (128 * D) + (w & 1) * (64 * D) : 6 * (128 * D) + (w - 4) * (64 * D);
}

// ---------------------------------------------------------------------------
// Forward workgroup order over num_qt query tiles x BH heads, the last query
// tile (the heaviest under the causal mask) first.  The dispatcher hands
// workgroup i to XCD i % 8, and each XCD has its own L2.  With hg > 0 (BH a
// multiple of 8 hg), XCD x takes its heads x, x + 8, ... in groups of hg,
// each group's query tiles heaviest first with the group's heads
// interleaved.  hg is chosen (head_group_size) so that one group's tiles
// fill what an XCD runs at once: they start together, walk the same K/V
// tiles in step and find most of them in the XCD's L2.  With hg = 0, tiles
// heaviest first with the head index varying fastest.
// ---------------------------------------------------------------------------
// Item k of XCD x's list (hg > 0): the (head, query tile) that xcd_head_groups
// gives the k-th workgroup placed on that XCD.
__host__ __device__ inline void xcd_item(int x, int k, int num_qt, int hg, int& bh, int& qt) {
  const int per = hg * num_qt;
  const int grp = k / per, r = k % per;
  qt = num_qt - 1 - r / hg;
  bh = x + 8 * (hg * grp + r % hg);
}

__host__ __device__ inline void xcd_head_groups(int bid, int BH, int num_qt, int hg, int& bh, int& qt) {
  if (hg > 0) {
    xcd_item(bid & 7, bid >> 3, num_qt, hg, bh, qt);
  } else {
    qt = num_qt - 1 - bid / BH;
    bh = bid % BH;
  }
}

// Item k of XCD x in the backward kernels' head-major order: the XCD's heads
// x, x + 8, ... one after another, all num_tiles tiles of a head before the
// next, tile 0 first.
__host__ __device__ inline void xcd_head_major_item(int x, int k, int num_tiles, int& bh, int& tile) {
  tile = k % num_tiles;
  bh = (k / num_tiles) * 8 + x;
}

// Persistent launch: W workgroups per XCD, each working through a fixed
// list of its XCD's items (BH / 8 x num_qt of them, in xcd_item order).  In
// round r workgroup j takes item r W + j (r even) or r W + W - 1 - j (r
// odd), so a workgroup that drew one of a round's heavy tiles draws one of
// the next round's light ones.  Returns -1 past the end of the list.
__host__ __device__ inline int persistent_item(int j, int r, int W, int n_items) {
  const int k = r * W + ((r & 1) ? W - 1 - j : j);
  return k < n_items ? k : -1;
}

// The largest power of two g such that g heads' num_qt tiles fit in the
// `resident` workgroups one XCD runs at once and BH is a multiple of 8 g;
// 0 when BH is not a multiple of 8.
__host__ __device__ inline int head_group_size(int resident, int BH, int num_qt) {
  if (BH % 8 != 0) return 0;
  int g = 1;
  while (2 * g * num_qt <= resident && BH % (16 * g) == 0) g *= 2;
  return g;
}

}  // namespace layout
}  // namespace fa
