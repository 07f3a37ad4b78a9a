// Forward attention kernels for gfx950.
//
// Method: exact attention computed tile by tile with the online-softmax
// update (vibeengines.com "FlashAttention, explained", sections "Tiling and
// the online softmax" and "The math, worked with real numbers"): for each
// query row keep a running max m, a running sum l and an output accumulator
// O; for each new key tile rescale l and O by e^(m_old - m_new) and add the
// tile's e^(s - m) and e^(s - m) V; finish with O / l.  The N x N scores
// never leave registers.
//
// bf16 kernel layout (one workgroup = 8 waves = 256 query rows):
//   * each wave owns 32 consecutive queries; its Q slice lives in registers
//     as the B operand of S^T = K Q^T (v_mfma_f32_32x32x16_bf16), so the
//     32x32 accumulator puts one query per lane column: the row max and row
//     sum are in-lane reductions plus one permlane32 swap.
//   * K and V tiles of BN keys are copied into LDS (three buffers each,
//     three tiles ahead) straight from global memory (buffer_load ... lds:
//     no registers and no LDS write instructions) and shared by the 8 waves.  Each key-tile step has two barrier-separated
//     phases: a matrix phase (O += P(t) V(t) and S(t+1) = K(t+1) Q^T) and a
//     vector phase (the online softmax of S(t+1)).  Waves 4-7 run one phase
//     behind waves 0-3, so the two waves sharing a SIMD alternate between the
//     matrix cores and the vector ALU.  Waves 0-3 copy the K tiles and waves
//     4-7 the V tiles.
//   * K and V are stored row-major, rows unpadded, with the 16-byte chunks
//     of each row XOR-permuted so both products read conflict-free.  The A
//     operand of O^T += V^T P^T (V transposed) is read with
//     ds_read_b64_tr_b16, which hands each lane four consecutive keys of one
//     feature column; the two reads per operand take the key order the S^T
//     accumulator leaves in each lane.
//   * P is rounded to bf16 (RNE) and fed back as the B operand directly from
//     the accumulator registers; O^T accumulates in fp32.
//   * The running reference m is the first tile's max and is raised only
//     when a tile's exponentials against it would sum past kPSumLimit in some
//     lane (so every P stays <= kPSumLimit).  Any reference works in exact
//     arithmetic (it cancels in O / l); a lazy one removes the per-tile max
//     reduction and makes the output rescale rare.
//   * Global reads use buffer descriptors sized to the head: reads past the
//     last row return zeros, so ragged tails need no branches.
//   * Workgroups are issued heaviest first (causal), all query tiles of a
//     head on the same XCD, that XCD's heads taken in groups just large
//     enough to fill it (xcd_head_groups): a group's tiles start together
//     and walk the same K/V tiles in step, so most tile copies are served by
//     the XCD's L2.
#include "fa_common.h"
#include "fa_internal.h"
#include "fa_layout.h"

namespace fa {

constexpr float kPSumLimit = 256.0f;
constexpr int kSparseBlock = FA_SPARSE_BLOCK;   // block-mask granularity (queries and keys)
#ifndef FWD_LOOKAHEAD
#define FWD_LOOKAHEAD 7
#endif

template <int D, int BN>
struct FwdCfg {
  static constexpr int kWaves = 8;
  static constexpr int kThreads = kWaves * 64;
  static constexpr int BM = kWaves * 32;
  static constexpr int kTile = BN * D;     // bf16 elements per K or V tile (unpadded rows)
  static constexpr int kBufs = 3;          // LDS buffers per tensor
  // LDS: K buffers 0..2 | V buffers 0..2 | the Q staging slots that do not
  // fit in the third buffers (layout::fwd_qslot) | the sparse list.  After
  // the loop the same bytes stage the output rows (32 x D bf16 per wave).
  static constexpr int kTileBytes = 2 * kBufs * kTile * 2;
  static constexpr int kListOff = 2 * kBufs * kTile + layout::fwd_qslot_extra<D, BN>();   // elements
  static constexpr int kStageBytes = kWaves * 32 * D * 2;
  static constexpr int kLdsBytes = kListOff * 2 > kStageBytes ? kListOff * 2 : kStageBytes;
  // Each group of four waves copies one tensor; 1 KB per copy instruction.
  static constexpr int kDmaPerWave = kTile * 2 / 1024 / 4;
  static_assert(BN % 32 == 0 && D % 32 == 0, "tile shape");
  static_assert(kDmaPerWave >= 1 && kTile * 2 % 4096 == 0, "tile must split into 1 KB copies per wave");
  static_assert(kThreads == 512, "kernel launch bounds assume 512 threads");
};

// Tiles sit in LDS with unpadded rows whose 16-byte chunks are permuted
// (layout::FwdSwizzle: K by its row-read permutation, V by its
// transposing-read permutation), so that the reads of both products hit 64
// distinct banks.
template <int D>
using Swizzle = layout::FwdSwizzle<D>;

// Global -> LDS without registers (buffer_load ... lds): this wave's share
// of a BN x D tile starting at key j0.  Each instruction fills 1 KB of LDS
// in lane order (lane i writes bytes 16i..16i+15); lane i therefore loads
// the global chunk that the swizzle stores at that position.  Rows past the
// head's end read as zero through the buffer descriptor.  Completion is
// tracked by this wave's vmcnt.
template <int D, int BN, bool IS_K>
__device__ __forceinline__ void dma_tile(__amdgpu_buffer_rsrc_t r, __bf16* tile, int j0, int wq, int lane) {
  using C = FwdCfg<D, BN>;
#pragma unroll
  for (int i = 0; i < C::kDmaPerWave; ++i) {
    const int inst = wq * C::kDmaPerWave + i;
    int row, chunk;
    if constexpr (IS_K) layout::copy_slot(2 * D, inst, lane, Swizzle<D>::k, row, chunk);
    else layout::copy_slot(2 * D, inst, lane, Swizzle<D>::v, row, chunk);
    const uint32_t goff = (uint32_t)((j0 + row) * D + 8 * chunk) * 2u;
    lds_copy16(r, goff, (uint32_t)(uintptr_t)(tile + inst * 512));
  }
}

// This wave's 32 query rows (zeros past the head's end, through the buffer
// descriptor) into its LDS staging slot, 1 KB of consecutive rows per
// instruction, chunks permuted as in a K tile.
template <int D>
__device__ __forceinline__ void dma_q(__amdgpu_buffer_rsrc_t r, __bf16* slot, int q0, int lane) {
#pragma unroll
  for (int i = 0; i < 32 * D * 2 / 1024; ++i) {
    int row, chunk;
    layout::copy_slot(2 * D, i, lane, Swizzle<D>::k, row, chunk);
    lds_copy16(r, (uint32_t)((q0 + row) * D + 8 * chunk) * 2u, (uint32_t)(uintptr_t)(slot + i * 512));
  }
}

// S^T = K Q^T for one tile: BN keys x this wave's 32 queries.  The k-steps
// run outermost so the BN/32 accumulator chains interleave, and each
// operand is read L products ahead of its MFMA (as in the matrix phase)
// instead of just before it.  koff[ks] is this lane's element offset of
// its A operand for k-step ks (row lc, chunk 2 ks + lg, swizzled); 32-row
// blocks add 32 D.
template <int D, int BN, int L>
__device__ __forceinline__ void score_tile(f32x16 (&s)[BN / 32], const __bf16* Ks, const int (&koff)[D / 16],
                                          const bf16x8 (&qb)[D / 16]) {
  constexpr int kAll = D / 16 * (BN / 32);
  constexpr int kL = L < kAll ? L : kAll;
  auto load = [&](int i) { return *(const bf16x8*)(Ks + koff[i / (BN / 32)] + 32 * (i % (BN / 32)) * D); };
#pragma unroll
  for (int mb = 0; mb < BN / 32; ++mb) s[mb] = (f32x16){};
  bf16x8 ring[kL];
#pragma unroll
  for (int i = 0; i < kL; ++i) ring[i] = load(i);
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int i = 0; i < kAll; ++i) {
    const bf16x8 a = ring[i % kL];
    s[i % (BN / 32)] = mfma32(a, qb[i / (BN / 32)], s[i % (BN / 32)]);
    if (i + kL < kAll) ring[i % kL] = load(i + kL);
    __builtin_amdgcn_sched_barrier(0);
  }
}

// Keys past the end, and on the diagonal keys after the query, to -inf.
template <int BN>
__device__ __forceinline__ void mask_tile(f32x16 (&s)[BN / 32], int j0, int qlim, int lg) {
#pragma unroll
  for (int mb = 0; mb < BN / 32; ++mb)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int key = j0 + 32 * mb + 8 * (r >> 2) + 4 * lg + (r & 3);
      if (key > qlim) s[mb][r] = -INFINITY;
    }
}

// P = exp2(s * scale * log2 e - m) for one tile, rounded to bf16 and packed
// as the B operands of the P V product.  Returns this lane's sum of P,
// taken in fp32 before rounding so that l, and with it the saved
// logsumexp, is not perturbed by the bf16 rounding of P.
template <int BN>
__device__ __forceinline__ float tile_exp(const f32x16 (&s)[BN / 32], bf16x8 (&pb)[BN / 16], float m,
                                          float scale_log2) {
  float rowsum = 0.f;
#pragma unroll
  for (int mb = 0; mb < BN / 32; ++mb)
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      // Eight independent exponentials at a time, so the transcendental unit
      // is not waiting on one score's argument after another.
      float p[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) p[j] = __builtin_fmaf(s[mb][8 * h + j], scale_log2, -m);
#pragma unroll
      for (int j = 0; j < 8; ++j) p[j] = fast_exp2(p[j]);
      uint32_t w[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        w[e] = pack_bf16x2(p[2 * e], p[2 * e + 1]);
        // Pack here: left to itself the compiler moves the packs past the
        // rescale test (they are redone when it fires) and keeps all the
        // fp32 exponentials live until then.
        asm volatile("" : "+v"(w[e]));
      }
      rowsum += ((p[0] + p[1]) + (p[2] + p[3])) + ((p[4] + p[5]) + (p[6] + p[7]));
      pb[2 * mb + h] = __builtin_bit_cast(bf16x8, ((u32x4){w[0], w[1], w[2], w[3]}));
    }
  return rowsum;
}

// The first tile of a row: the reference m is the tile's max (-inf when
// every score is masked) and l is the tile's sum.  The same values as
// softmax_step from m = -inf, l = 0, O = 0, without the exponentials taken
// against m = -inf first.
template <int BN>
__device__ __forceinline__ void softmax_first(const f32x16 (&s)[BN / 32], bf16x8 (&pb)[BN / 16], float& m_run,
                                              float& l_run, float scale_log2) {
  float mx = -INFINITY;
#pragma unroll
  for (int mb = 0; mb < BN / 32; ++mb)
#pragma unroll
    for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[mb][r]);
  m_run = max_with_lane_xor32(mx) * scale_log2;
  l_run = tile_exp<BN>(s, pb, m_run == -INFINITY ? 0.f : m_run, scale_log2);
}

// Online-softmax step for one tile of scores (this lane's query column).
// The exponentials are taken against the running reference m first.  If
// every lane's sum of this tile's P stays within kPSumLimit, every P does
// too and the tile is done: m, O and l are unchanged.  Otherwise (the first
// tile, where m = -inf, or a tile whose scores climb well above m) m is
// raised to the tile's max, O and l are rescaled by 2^(m_old - m_new), and
// the exponentials are taken again.
template <int D, int BN>
__device__ __forceinline__ void softmax_step(const f32x16 (&s)[BN / 32], bf16x8 (&pb)[BN / 16], float& m_run,
                                             float& l_run, f32x16 (&oacc)[D / 32], float scale_log2) {
  float rs = tile_exp<BN>(s, pb, m_run, scale_log2);
  if (__ballot(!(rs <= kPSumLimit))) {
    float mx = -INFINITY;
#pragma unroll
    for (int mb = 0; mb < BN / 32; ++mb)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[mb][r]);
    mx = max_with_lane_xor32(mx) * scale_log2;
    const float m_new = fmaxf(m_run, mx);
    // 0 on the first tile that sees a key; 1 while no key has been seen
    // (block-sparse rows can start with dropped tiles), where O and l are 0.
    const float alpha = m_new == -INFINITY ? 1.f : fast_exp2(m_run - m_new);
    m_run = m_new;
    l_run *= alpha;
#pragma unroll
    for (int i = 0; i < D / 32; ++i) oacc[i] *= alpha;
    // A query whose keys are all masked so far keeps m = -inf; 0 is used
    // instead so exp2 gives 0 rather than NaN.
    rs = tile_exp<BN>(s, pb, m_run == -INFINITY ? 0.f : m_run, scale_log2);
  }
  l_run += rs;
}

// Both products of a matrix phase, O += P(t) V(t) then S(t+1) = K(t+1) Q^T,
// as one stream of MFMAs whose LDS operands are read L products ahead, so
// the read latency hides behind the preceding MFMAs instead of stalling
// each one.  Scheduling barriers keep the stream in this order.  voff[dm]
// is this lane's element offset of its V^T operand reads for feature block
// dm (swizzled); 16-key steps add 16 D.
//
// The operands of the first L products (P V products: V(t) only) are read
// by matrix_preload.  For d = 128 the kernel issues those reads at the end
// of the wave's vector phase, before the barrier that opens the matrix
// phase (V(t) was published a barrier earlier; K(t+1) only by that
// barrier), so the phase does not open on a full LDS latency.  For d = 64
// the vector phase is the longer one and the reads stay in the phase.
template <int D, int BN>
__device__ __forceinline__ bf16x8 matrix_load(int i, const __bf16* Vs, const int (&voff)[D / 32], const __bf16* Ks,
                                              const int (&koff)[D / 16]) {
  constexpr int kPv = BN / 16 * (D / 32);
  if (i < kPv) {
    const int c = i / (D / 32), dm = i % (D / 32);
    return lds_tr_pair(Vs + voff[dm], (16 * c) * D, (16 * c + 8) * D);
  }
  const int j = i - kPv, ks = j / (BN / 32), mb = j % (BN / 32);
  return *(const bf16x8*)(Ks + koff[ks] + 32 * mb * D);
}

template <int D, int BN, int L>
__device__ __forceinline__ void matrix_preload(bf16x8 (&ring)[L], const __bf16* Vs, const int (&voff)[D / 32],
                                               const __bf16* Ks, const int (&koff)[D / 16]) {
#pragma unroll
  for (int i = 0; i < L; ++i) ring[i] = matrix_load<D, BN>(i, Vs, voff, Ks, koff);
}

// SCORES = false (the last step of an item): the P V products only (when
// the ring is deeper than they are, its in-phase preload also reads score
// operands of a stale K buffer, which go unused).
template <int D, int BN, int L, bool PRELOADED, bool SCORES = true>
__device__ __forceinline__ void matrix_phase(bf16x8 (&ring)[L], f32x16 (&oacc)[D / 32], const bf16x8 (&pb)[BN / 16],
                                             const __bf16* Vs, const int (&voff)[D / 32], f32x16 (&s)[BN / 32],
                                             const __bf16* Ks, const int (&koff)[D / 16],
                                             const bf16x8 (&qb)[D / 16]) {
  constexpr int kPv = BN / 16 * (D / 32);   // O += P V products
  constexpr int kS = D / 16 * (BN / 32);    // S = K Q^T products
  constexpr int kAll = kPv + (SCORES ? kS : 0);
  if constexpr (SCORES) {
#pragma unroll
    for (int mb = 0; mb < BN / 32; ++mb) s[mb] = (f32x16){};
  }
  // The matrix wave takes issue priority over the SIMD's other wave (in its
  // vector phase), so MFMAs are not held back behind its exponentials.
  __builtin_amdgcn_s_setprio(1);
  if constexpr (!PRELOADED) matrix_preload<D, BN, L>(ring, Vs, voff, Ks, koff);
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int i = 0; i < kAll; ++i) {
    const bf16x8 a = ring[i % L];
    if (i < kPv) {
      const int c = i / (D / 32), dm = i % (D / 32);
      oacc[dm] = mfma32(a, pb[c], oacc[dm]);
    } else {
      const int j = i - kPv, ks = j / (BN / 32), mb = j % (BN / 32);
      s[mb] = mfma32(a, qb[ks], s[mb]);
    }
    if (i + L < kAll) ring[i % L] = matrix_load<D, BN>(i + L, Vs, voff, Ks, koff);
    __builtin_amdgcn_sched_barrier(0);
  }
  __builtin_amdgcn_s_setprio(0);
}

// SPARSE: block-sparse attention.  bmask holds, per head, an nb x nb byte
// matrix over (128-query block, 128-key block) pairs; pairs whose byte is 0
// are masked.  The workgroup (two query blocks) visits only the key tiles
// that at least one of its query blocks keeps, in order, from a list built
// in LDS; a wave whose own query block drops a visited tile treats all of
// that tile's scores as masked.
template <int D, int BN, bool CAUSAL, bool SPARSE>
__global__ void __launch_bounds__(512)
fa_fwd_bf16_kernel(const __bf16* __restrict__ Q, const __bf16* __restrict__ K,
                   const __bf16* __restrict__ V, __bf16* __restrict__ O, float* __restrict__ LSE,
                   const uint8_t* __restrict__ bmask, int N, int BH, int num_qt, int hg, int wpx,
                   float scale_log2) {
  using C = FwdCfg<D, BN>;
  static_assert(!SPARSE || (C::BM == 2 * kSparseBlock && kSparseBlock % BN == 0), "sparse blocks vs tiles");
  extern __shared__ __attribute__((aligned(16))) __bf16 smem[];

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform per wave
  const int group = wave >> 2;   // 0: waves 0-3 (one per SIMD), 1: waves 4-7
  const int wq = wave & 3;       // wave within its group

  // One (head, 256-query tile) item per pass.  wpx = 0: this workgroup's
  // single item, heaviest query tiles first with heads grouped per XCD.
  // wpx > 0 (persistent launch, wpx workgroups per XCD): the workgroup works
  // through its share of its XCD's list of items.
  const int xcd_items = BH / 8 * num_qt;
  for (int pass = 0;; ++pass) {
  // The lane index enters each pass as a fresh value, so the per-lane
  // address arithmetic of the pass is done inside it rather than hoisted out
  // of the item loop and held in registers through every step.
  int lane_v = tid & 63;
  asm volatile("" : "+v"(lane_v));
  const int lane = lane_v;
  const int lc = lane & 31;      // lane column: query within the wave
  const int lg = lane >> 5;      // lane half

  // This lane's swizzled LDS offsets.  K (A operand of S^T = K Q^T): row lc,
  // chunk 2 ks + lg.  V (A operand of O^T += V^T P^T via the transposing
  // read): lane (s = lane % 16, G = bit 4, g = bit 5) reads row 4 g + s / 4
  // of each 8-row group at column 32 dm + 16 G + 4 (s % 4); f(row) depends
  // only on s / 4 because the group offsets are multiples of 8 rows.
  int koff[D / 16], voff[D / 32];
#pragma unroll
  for (int ks = 0; ks < D / 16; ++ks) koff[ks] = layout::fwd_koff<D>(lc, lg, ks);
#pragma unroll
  for (int dm = 0; dm < D / 32; ++dm) voff[dm] = layout::fwd_voff<D>(lane, dm);

  int qt, bh;
  if (wpx > 0) {
    const int k = layout::persistent_item(blockIdx.x >> 3, pass, wpx, xcd_items);
    if (k < 0) break;
    layout::xcd_item(blockIdx.x & 7, k, num_qt, hg, bh, qt);
  } else {
    if (pass > 0) break;
    layout::xcd_head_groups(blockIdx.x, BH, num_qt, hg, bh, qt);
  }
  const size_t head_off = (size_t)bh * N * D;
  const uint32_t head_bytes = (uint32_t)N * D * 2u;
  const __amdgpu_buffer_rsrc_t rq = make_rsrc(Q + head_off, head_bytes);
  // Group 0 copies the K tiles into LDS, group 1 the V tiles.
  const __amdgpu_buffer_rsrc_t rmine = make_rsrc((group == 0 ? K : V) + head_off, head_bytes);
  auto kbuf = [&](int i) { return smem + i * C::kTile; };
  auto vbuf = [&](int i) { return smem + (C::kBufs + i) * C::kTile; };
  auto copy_tile = [&](int tile, int buf) {
    if (group == 0) dma_tile<D, BN, true>(rmine, kbuf(buf), tile * BN, wq, lane);
    else dma_tile<D, BN, false>(rmine, vbuf(buf), tile * BN, wq, lane);
  };

  const int q_wave0 = qt * C::BM + wave * 32;
  const int q_idx = q_wave0 + lc;

  // Q first: this wave's rows into its staging slot (read back below as the
  // MFMA B operand once the copy is in).
  const int qslot = layout::fwd_qslot<D, BN>(wave);
  dma_q<D>(rq, smem + qslot, q_wave0, lane);

  f32x16 oacc[D / 32];
#pragma unroll
  for (int i = 0; i < D / 32; ++i) oacc[i] = (f32x16){};
  float m_run = -INFINITY;   // running reference max of scale*log2(e)*s
  float l_run = 0.f;         // this lane's share of the running sum

  const int q_tile_end = min(N, (qt + 1) * C::BM);
  const int key_end = CAUSAL ? q_tile_end : N;
  int num_kt = (key_end + BN - 1) / BN;
  auto masked = [&](int t) { return (t * BN + BN > N) || (CAUSAL && t * BN + BN - 1 > q_wave0); };

  // Sparse: list of visited key tiles, entry = tile | keep(block 0) << 24 |
  // keep(block 1) << 25, built by wave 0 with a ballot compaction.
  int* tlist = (int*)(smem + C::kListOff);   // [0] = count, then entries
  if constexpr (SPARSE) {
    const int nb = (N + kSparseBlock - 1) / kSparseBlock;
    const uint8_t* row0 = bmask + ((size_t)bh * nb + 2 * qt) * nb;
    const bool has1 = 2 * qt + 1 < nb;
    if (wave == 0) {
      int cnt = 0;
      for (int base = 0; base < num_kt; base += 64) {
        const int t = base + lane;
        const int kb = t * BN / kSparseBlock;
        const bool in = t < num_kt;
        const int k0 = in ? (row0[kb] != 0) : 0;
        const int k1 = (in && has1) ? (row0[nb + kb] != 0) : 0;
        const bool live = (k0 | k1) != 0;
        const uint64_t bal = __ballot(live);
        const int pos = cnt + __builtin_amdgcn_mbcnt_hi((uint32_t)(bal >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)bal, 0));
        if (live) tlist[1 + pos] = t | (k0 << 24) | (k1 << 25);
        cnt += __popcll(bal);
      }
      if (lane == 0) tlist[0] = cnt;
    }
    __syncthreads();
    num_kt = __builtin_amdgcn_readfirstlane(tlist[0]);
  }
  auto tile_at = [&](int j) { return SPARSE ? (tlist[1 + j] & 0xFFFFFF) : j; };
  // Sparse: this wave's query block drops visited tile j.
  auto dropped = [&](int j) { return SPARSE && !((tlist[1 + j] >> (24 + group)) & 1); };

  // The first two visited tiles of each tensor.  Visited tile j lives in
  // buffer j % 3.
  if (num_kt > 0) copy_tile(tile_at(0), 0);
  if (num_kt > 1) copy_tile(tile_at(1), 1);
  // Q's copies are older than the tiles': wait for them alone, then read
  // Q^T as the MFMA B operand (lane: Q[q][16 ks + 8 lg .. +7]) with the K
  // tile's row reads.
  int qaddr = qslot;
  if (num_kt > 1) wait_vmem_keep_before<2 * C::kDmaPerWave>(qaddr);
  else if (num_kt == 1) wait_vmem_keep_before<C::kDmaPerWave>(qaddr);
  else wait_vmem_keep_before<0>(qaddr);
  bf16x8 qb[D / 16];
#pragma unroll
  for (int ks = 0; ks < D / 16; ++ks) qb[ks] = *(const bf16x8*)(smem + qaddr + layout::fwd_koff<D>(lc, lg, ks));
  wait_vmem_all();
  // The Q reads are complete (the compiler waits for them at this asm)
  // before any wave passes the barrier and starts tile 2's copy into the
  // third buffers, which hold some of the slots.
#pragma unroll
  for (int ks = 0; ks < D / 16; ++ks) asm volatile("" : "+v"(qb[ks]));
  __syncthreads();
  // The third, into the still unused buffer 2; waited for at the end of the
  // first vector phase.
  if (num_kt > 2) copy_tile(tile_at(2), 2);

  f32x16 s[BN / 32];
  bf16x8 pb[BN / 16];
  // Scores of visited tile j to -inf where masked: all of them when this
  // wave's query block drops the tile (sparse), else keys past N and, under
  // the causal mask, keys after the query.
  auto mask_visit = [&](int j) {
    const int t = tile_at(j);
    if (dropped(j)) {
#pragma unroll
      for (int mb = 0; mb < BN / 32; ++mb)
#pragma unroll
        for (int r = 0; r < 16; ++r) s[mb][r] = -INFINITY;
    } else if (masked(t)) {
      // The lane's last key is rebuilt here, from a lane index the compiler
      // cannot hoist, rather than held in a register through the loop:
      // only the tiles on the causal diagonal and the last one get here.
      int l = lane;
      asm volatile("" : "+v"(l));
      const int lim = CAUSAL ? min(q_wave0 + (l & 31), N - 1) : N - 1;
      mask_tile<BN>(s, t * BN, lim, l >> 5);
    }
  };

  // S and P of the first visited tile.
  if (num_kt > 0) {
    score_tile<D, BN, FWD_LOOKAHEAD>(s, kbuf(0), koff, qb);
    mask_visit(0);
    softmax_first<BN>(s, pb, m_run, l_run, scale_log2);
  }

  // The two waves on each SIMD (waves w and w + 4) alternate: group 1 runs
  // one barrier interval behind group 0, so while one issues the step's
  // MFMAs the other is in its exponentials.  Every wave passes the same
  // number of barriers (group 1 one extra here, group 0 one extra at the
  // end).  Step t works on visited tiles t and t+1 (all key tiles in
  // order, dense).  At the start of its vector phase of step t each group
  // starts the copy of visited tile t+3 of its tensor into buffer t % 3, and
  // at the end of that phase waits for all its copies but that one.  Tile
  // t's last reads (K(t) by both groups' score products of step t-1, V(t)
  // by the P V products of step t, group 1's being the later) end at least
  // one barrier before the copy starts.  Tile t+3 is first read in step
  // t+2 (K(t+3) by group 0's score product, V(t+3) by the operand reads
  // that end the vector phase before it), at least one barrier after the
  // wait of step t+1 that completes it; the copy has three barrier
  // intervals to land, which covers the latency of a tile read that the
  // L2 does not hold.
  constexpr bool kPreload = D == 128;
  static_assert(!kPreload || FWD_LOOKAHEAD <= BN / 16 * (D / 32), "preloaded products must all be P V products");
  bf16x8 ring[FWD_LOOKAHEAD];
  if constexpr (kPreload) matrix_preload<D, BN, FWD_LOOKAHEAD>(ring, vbuf(0), voff, kbuf(1), koff);
  if (group == 1) __syncthreads();

  // Causal (dense, or block-sparse at d = 128, where the 64-key build has
  // the registers for it): visited tiles from n_live on hold only keys
  // after every query of this wave, so their P is zero.  The wave then runs the P V
  // products of tile n_live - 1 alone and, on the steps after it, only the
  // copies, waits and barriers every wave takes part in (skipping exactly
  // zero terms: the result is the same bit for bit).
  constexpr bool kDeadTail = CAUSAL && (!SPARSE || D == 128);
  int n_live = num_kt;
  if constexpr (kDeadTail) {
    // The last key tile holding a key of this wave's queries; visited tiles
    // come in increasing order, so the dead ones are the list's last few.
    const int last = (q_wave0 + 31) / BN;
    if constexpr (SPARSE) {
      while (n_live > 0 && __builtin_amdgcn_readfirstlane(tile_at(n_live - 1)) > last) --n_live;
    } else {
      n_live = min(num_kt, last + 1);
    }
  }
  int b_cur = 0;   // t % 3
  int t = 0;
  for (; t + 1 < n_live; ++t) {
    const int b_next = b_cur == 2 ? 0 : b_cur + 1;    // (t + 1) % 3
    const int b_after = b_cur == 0 ? 2 : b_cur - 1;   // (t + 2) % 3
    // Phase 1 (matrix cores): O += P(t) V(t); S(t+1) = K(t+1) Q^T.  Every
    // wave runs the same instruction stream on every step of this loop: on
    // causal tiles partly above a wave's queries the masked scores give
    // P = 0 (the tiles wholly above them are the tail after the loop).
    matrix_phase<D, BN, FWD_LOOKAHEAD, kPreload>(ring, oacc, pb, vbuf(b_cur), voff, s, kbuf(b_next), koff, qb);
    __syncthreads();
    // Phase 2 (vector ALU): P(t+1).
    const bool copy_next = t + 3 < num_kt;
    if (copy_next) copy_tile(tile_at(t + 3), b_cur);
    mask_visit(t + 1);
    softmax_step<D, BN>(s, pb, m_run, l_run, oacc, scale_log2);
    // V(t+1)'s copy was waited for at the end of the previous step, so the
    // barrier before this phase published it.
    if constexpr (kPreload) matrix_preload<D, BN, FWD_LOOKAHEAD>(ring, vbuf(b_next), voff, kbuf(b_after), koff);
    if (copy_next) wait_vmem_keep<C::kDmaPerWave>();
    else wait_vmem_all();
    __syncthreads();
    b_cur = b_next;
  }
  if constexpr (!kDeadTail) {
    // The last step (outside the loop, so the loop's code stays one
    // stream): O += P V only, there being no next tile; the same two
    // barriers.
    if (num_kt > 0) {
      matrix_phase<D, BN, FWD_LOOKAHEAD, kPreload, false>(ring, oacc, pb, vbuf(b_cur), voff, s, kbuf(b_cur), koff, qb);
      __syncthreads();
      wait_vmem_all();
      __syncthreads();
    }
  } else {
  // The copies and waits of step t's vector phase, for the steps with no
  // softmax.
  auto copies_only = [&]() {
    const bool copy_next = t + 3 < num_kt;
    if (copy_next) copy_tile(tile_at(t + 3), b_cur);
    if (copy_next) wait_vmem_keep<C::kDmaPerWave>();
    else wait_vmem_all();
  };
  // The last live step (outside the loop, so the loop's code stays one
  // stream): O += P V only, there being no next tile this wave sees; the
  // same two barriers.
  if (num_kt > 0) {
    matrix_phase<D, BN, FWD_LOOKAHEAD, kPreload, false>(ring, oacc, pb, vbuf(b_cur), voff, s, kbuf(b_cur), koff, qb);
    __syncthreads();
    copies_only();
    __syncthreads();
    b_cur = b_cur == 2 ? 0 : b_cur + 1;
    ++t;
  }
  // The steps of tiles this wave does not see.
  for (; t < num_kt; ++t) {
    __syncthreads();
    copies_only();
    __syncthreads();
    b_cur = b_cur == 2 ? 0 : b_cur + 1;
  }
  }
  if (group == 0) __syncthreads();

  // Epilogue: O / l rounded to bf16, and LSE = m + ln l (natural log).  The
  // last barrier above follows every wave's last tile read, so the tile
  // buffers are free to stage the output rows.
  const float l_tot = sum_with_lane_xor32(l_run);
  const float inv_l = l_tot > 0.f ? 1.f / l_tot : 0.f;
  store_o_rows<D>(oacc, inv_l, smem + wave * 32 * D, O + head_off, q_wave0, N, lane);
  if (LSE != nullptr && lg == 0 && q_idx < N)
    LSE[(size_t)bh * N + q_idx] = l_tot > 0.f ? m_run * kLn2 + __logf(l_tot) : -INFINITY;
  // Every wave's staged output rows are read back before the next item's
  // first copies (and sparse list) overwrite the LDS.
  if (wpx > 0) __syncthreads();
  }
}

// ---------------------------------------------------------------------------
// fp32 forward: float32 storage and arithmetic throughout (no bf16 rounding
// anywhere).  VALU kernel: TPQ = D/64 lanes per query row, each lane holding
// 64 features of q and of the output accumulator; 32-key tiles of K and V
// are staged in LDS and broadcast to every lane.
// ---------------------------------------------------------------------------
template <int D, bool CAUSAL>
__global__ void __launch_bounds__(256)
fa_fwd_f32_kernel(const float* __restrict__ Q, const float* __restrict__ K, const float* __restrict__ V,
                  float* __restrict__ O, float* __restrict__ LSE, int N, int BH, int num_qt, float scale) {
  constexpr int TPQ = D / 64;
  constexpr int QPB = 256 / TPQ;   // queries per workgroup
  constexpr int BK = 32;
  __shared__ float Ks[BK][D];
  __shared__ float Vs[BK][D];

  const int tid = threadIdx.x;
  const int part = tid % TPQ;
  const int bid = blockIdx.x;
  const int qt = num_qt - 1 - bid / BH;   // heaviest query tiles first
  const int bh = bid % BH;
  const int q_idx = qt * QPB + tid / TPQ;
  const size_t head_off = (size_t)bh * N * D;

  float q[64], acc[64];
  const bool q_ok = q_idx < N;
#pragma unroll
  for (int c = 0; c < 64; ++c) {
    q[c] = q_ok ? Q[head_off + (size_t)q_idx * D + part * 64 + c] : 0.f;
    acc[c] = 0.f;
  }
  float m_run = -INFINITY, l_run = 0.f;
  const int q_last = min(N, (qt + 1) * QPB) - 1;
  const int key_end = CAUSAL ? q_last + 1 : N;
  for (int j0 = 0; j0 < key_end; j0 += BK) {
    __syncthreads();
    for (int e = tid; e < BK * D; e += 256) {
      const int r = e / D, c = e % D;
      const int key = j0 + r;
      Ks[r][c] = key < N ? K[head_off + (size_t)key * D + c] : 0.f;
      Vs[r][c] = key < N ? V[head_off + (size_t)key * D + c] : 0.f;
    }
    __syncthreads();
    float s[BK];
    float mx = -INFINITY;
#pragma unroll
    for (int j = 0; j < BK; ++j) {
      float dot = 0.f;
#pragma unroll
      for (int c = 0; c < 64; ++c) dot = __builtin_fmaf(q[c], Ks[j][part * 64 + c], dot);
      if (TPQ == 2) dot += __shfl_xor(dot, 1);
      const int key = j0 + j;
      const bool masked = key >= N || (CAUSAL && key > q_idx);
      s[j] = masked ? -INFINITY : dot * scale;
      mx = fmaxf(mx, s[j]);
    }
    const float m_new = fmaxf(m_run, mx);
    const float m_use = m_new == -INFINITY ? 0.f : m_new;
    const float alpha = expf(m_run - m_use);
    float psum = 0.f;
#pragma unroll
    for (int c = 0; c < 64; ++c) acc[c] *= alpha;
#pragma unroll
    for (int j = 0; j < BK; ++j) {
      const float p = expf(s[j] - m_use);
      psum += p;
#pragma unroll
      for (int c = 0; c < 64; ++c) acc[c] = __builtin_fmaf(p, Vs[j][part * 64 + c], acc[c]);
    }
    l_run = l_run * alpha + psum;
    m_run = m_new;
  }
  if (q_ok) {
    const float inv = l_run > 0.f ? 1.f / l_run : 0.f;
#pragma unroll
    for (int c = 0; c < 64; ++c) O[head_off + (size_t)q_idx * D + part * 64 + c] = acc[c] * inv;
    if (LSE != nullptr && part == 0)
      LSE[(size_t)bh * N + q_idx] = l_run > 0.f ? m_run + logf(l_run) : -INFINITY;
  }
}

// ---------------------------------------------------------------------------
// Launchers.
// ---------------------------------------------------------------------------
template <int D, int BN, bool CAUSAL, bool SPARSE>
static hipError_t launch_bf16(const FwdArgs& a) {
  using C = FwdCfg<D, BN>;
  const int BH = a.B * a.H;
  const int num_qt = (a.N + C::BM - 1) / C::BM;
  auto kern = fa_fwd_bf16_kernel<D, BN, CAUSAL, SPARSE>;
  // The sparse kernel keeps its list of visited key tiles (count first)
  // after the tile buffers.
  const int list_bytes = SPARSE ? ((4 * ((a.N + BN - 1) / BN + 1) + 15) & ~15) : 0;
  const int lds = C::kListOff * 2 + list_bytes > C::kLdsBytes ? C::kListOff * 2 + list_bytes : C::kLdsBytes;
  // Dynamic LDS above 64 KB must be allowed explicitly; setting the same
  // value from several threads is harmless.
  hipError_t e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, lds);
  if (e != hipSuccess) return e;
  int hg = 0, wpx = 0;
  e = forward_work_layout((const void*)kern, C::kThreads, lds, BH, num_qt, &hg, &wpx);
  if (e != hipSuccess) return e;
  // A block mask can give the items any mix of costs, which the fixed
  // persistent lists would not balance: sparse launches keep one workgroup
  // per item and the hardware's dispatch.
  if (SPARSE) wpx = 0;
  const int grid = wpx > 0 ? 8 * wpx : num_qt * BH;
  hipLaunchKernelGGL(kern, dim3(grid), dim3(C::kThreads), lds, a.stream, (const __bf16*)a.q, (const __bf16*)a.k,
                     (const __bf16*)a.v, (__bf16*)a.o, a.lse, (const uint8_t*)a.bmask, a.N, BH, num_qt, hg, wpx,
                     a.scale * kLog2e);
  return hipGetLastError();
}

template <int D, bool CAUSAL>
static hipError_t launch_f32(const FwdArgs& a) {
  constexpr int QPB = 256 / (D / 64);
  const int BH = a.B * a.H;
  const int num_qt = (a.N + QPB - 1) / QPB;
  hipLaunchKernelGGL((fa_fwd_f32_kernel<D, CAUSAL>), dim3(num_qt * BH), dim3(256), 0, a.stream,
                     (const float*)a.q, (const float*)a.k, (const float*)a.v, (float*)a.o, a.lse, a.N, BH, num_qt,
                     a.scale);
  return hipGetLastError();
}

template <int D, int BN>
static hipError_t launch_bf16_bn(const FwdArgs& a) {
  if (a.bmask) return a.causal ? launch_bf16<D, BN, true, true>(a) : launch_bf16<D, BN, false, true>(a);
  return a.causal ? launch_bf16<D, BN, true, false>(a) : launch_bf16<D, BN, false, false>(a);
}

hipError_t launch_fwd(const FwdArgs& a) {
  if (a.dtype == FA_DTYPE_FP32) {
    if (a.d == 64) return a.causal ? launch_f32<64, true>(a) : launch_f32<64, false>(a);
    return a.causal ? launch_f32<128, true>(a) : launch_f32<128, false>(a);
  }
  // Dense d = 128 by default uses 96-key tiles: each step's fixed cost (two
  // barriers and the skew between the groups) is spread over 1.5x the work
  // of a 64-key step, and 3 x 2 buffers of 24 KB still fit in LDS.  Block
  // masks are laid out over 128-key blocks and keep 64-key tiles.
  if (a.block_n == 0 && a.d == 128 && a.bmask == nullptr)
    return a.causal ? launch_bf16<128, 96, true, false>(a) : launch_bf16<128, 96, false, false>(a);
  const int bn = a.block_n == 0 ? 64 : a.block_n;
  if (a.d == 64) return bn == 32 ? launch_bf16_bn<64, 32>(a) : launch_bf16_bn<64, 64>(a);
  return bn == 32 ? launch_bf16_bn<128, 32>(a) : launch_bf16_bn<128, 64>(a);
}

}  // namespace fa
