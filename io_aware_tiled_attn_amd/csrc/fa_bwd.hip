// Backward attention kernels for gfx950.
//
// The backward pass recomputes each score tile from Q, K and the saved
// per-row log-sum-exp instead of reading a stored probability matrix
// (chorfi.xyz study guide, "Study objectives" and "Main concepts";
// modelfieldguide.com, "An IO-aware rewrite").  The gradient formulas are the
// calculus of O = softmax(scale Q K^T) V for an upstream gradient dO:
//     P = exp(scale S - LSE),  dV = P^T dO,  dP = dO V^T,
//     D_i = sum_c dO_ic O_ic,  dS = P * (dP - D),
//     dQ = scale dS K,         dK = scale dS^T Q.
//
// The products run on v_mfma_f32_32x32x16_f16 with fp32 accumulation.
// Their operands are fp16 copies of Q, dO, K and V, each scaled by a power
// of two per head that brings its largest magnitude into [1, 2): a bf16
// value times a power of two is exact in fp16 down to 2^-14 of that
// magnitude (fp16 keeps 11 significant bits, bf16 8), so S and dP are the
// products of the exact inputs, and P (in [0, 1]) and dS (below 2^10 in these
// units) enter the other products with fp16's rounding, a relative 2^-12.
// The factors are undone in fp32: in the exponent's multiplier, in D's
// units and in the epilogues.
//
// dK and dV are sums over queries and dQ a sum over keys.  Instead of one
// pass that adds every workgroup's dQ share to memory with atomics (float
// atomics on MI355X resolve at the memory side, and at N = 4096 they took
// about 40 % of such a pass), two passes each own their output:
//   1. bwd_prep: per 256-row chunk of a head, D_i = <dO_i, O_i> in fp32 from
//      the bf16 O, and the chunk's largest |Q|, |dO|, |K|, |V|.
//   2. bwd_convert: the head's factors, the scaled fp16 copies of Q and dO,
//      and per row the start values of the S and dP accumulators,
//      -LSE log2 e / c2 and -D in the scaled units.
//   3. bwd_dkdv: key-major, one workgroup per 128-key tile; writes dK, dV,
//      and the scaled fp16 copies of its K and V rows.
//   4. bwd_dq: query-major, one workgroup per 128-query tile; writes dQ.
// The two passes recompute S and dP each: seven products per (query,
// key) pair instead of five, and no atomics.  The main kernels copy their
// fp16 tiles global -> LDS with buffer_load ... lds (no registers, no
// vector instructions), so their vector ALU time goes to P and dS alone.
#include <mutex>

#include "fa_common.h"
#include "fa_internal.h"
#include "fa_layout.h"

namespace fa {

// Device-resident scratch for flash_attn_bwd_noalloc: the backward's
// workspace (bwd_workspace_layout) for callers that cannot allocate.
// Every GPU the library runs on holds its own copy from module load until
// the process ends.  Host code never passes `bwd_scratch` itself to a
// kernel (on the host that name is a stand-in, not a device address); it
// uses the per-device address from hipGetSymbolAddress below.
static __device__ __align__(256) unsigned char bwd_scratch[FA_BWD_NOALLOC_MAX_BYTES];

hipError_t bwd_scratch_address(void** ptr) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static void* addr[kMaxDevices] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (addr[dev] == nullptr) {
    // First use on this device, with the device current: look up where its
    // copy of the array lives.
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(bwd_scratch));
    if (e != hipSuccess) return e;
    addr[dev] = p;
  }
  *ptr = addr[dev];
  return hipSuccess;
}

// ---------------------------------------------------------------------------
// Helpers.
// ---------------------------------------------------------------------------
__device__ __forceinline__ float abs_max_bf16x2(float m, uint32_t w) {
  return fmaxf(m, fmaxf(fabsf(bf16_lo(w)), fabsf(bf16_hi(w))));
}

// bf16 pair times f, rounded to an fp16 pair.
__device__ __forceinline__ uint32_t bf16x2_to_f16x2(uint32_t w, float f) {
  return pack_f16x2(bf16_lo(w) * f, bf16_hi(w) * f);
}
__device__ __forceinline__ u32x4 bf16x8_to_f16x8(u32x4 x, float f) {
  return (u32x4){bf16x2_to_f16x2(x[0], f), bf16x2_to_f16x2(x[1], f), bf16x2_to_f16x2(x[2], f),
                 bf16x2_to_f16x2(x[3], f)};
}

// Largest value of each of m[0..3] over the workgroup (NW waves), in place
// for every thread.  red: NW float4s of LDS.
template <int NW>
__device__ __forceinline__ void block_max4(float (&m)[4], f32x4* red) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1)
#pragma unroll
    for (int t = 0; t < 4; ++t) m[t] = fmaxf(m[t], __shfl_xor(m[t], off));
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = (f32x4){m[0], m[1], m[2], m[3]};
  __syncthreads();
#pragma unroll
  for (int i = 0; i < NW; ++i) {
    const f32x4 r = red[i];
#pragma unroll
    for (int t = 0; t < 4; ++t) m[t] = fmaxf(m[t], r[t]);
  }
}

// ---------------------------------------------------------------------------
// 1. Per 256-row chunk of a head: D_i = sum_c dO_ic O_ic, the largest |Q|,
//    |dO|, |K|, |V| of the chunk, and the chunk's rows of Q and dO as fp16
//    times the chunk's own factors (held in registers from the one read of
//    them; kernel 2 redoes the chunks whose factor is not the head's).
// ---------------------------------------------------------------------------
constexpr int kPrepThreads = 512;
template <int D>
__global__ void __launch_bounds__(kPrepThreads)
fa_bwd_prep_kernel(const __bf16* __restrict__ O, const __bf16* __restrict__ dO, const __bf16* __restrict__ Q,
                   const __bf16* __restrict__ K, const __bf16* __restrict__ V, float* __restrict__ delta,
                   float* __restrict__ part, _Float16* __restrict__ Q16, _Float16* __restrict__ dO16, int N,
                   int nch) {
  constexpr int TPR = D / 8;                   // threads per row, 8 elements each
  constexpr int RPI = kPrepThreads / TPR;      // rows per pass
  constexpr int NP = kBwdChunkRows / RPI;      // passes per chunk
  constexpr int NW = kPrepThreads / 64;
  __shared__ f32x4 red[NW];
  const int bh = blockIdx.x / nch, ch = blockIdx.x % nch;
  const int tid = threadIdx.x, col = (tid % TPR) * 8;
  const int row0 = ch * kBwdChunkRows;
  const int rows = min(kBwdChunkRows, N - row0);
  // Buffer loads over the head: rows past N read as zero, so the passes
  // need no bounds test and all of their loads can be in flight at once.
  const size_t head_off = (size_t)bh * N * D;
  const uint32_t head_bytes = (uint32_t)N * D * 2u;
  const __amdgpu_buffer_rsrc_t ro = make_rsrc(O + head_off, head_bytes), rg = make_rsrc(dO + head_off, head_bytes);
  const __amdgpu_buffer_rsrc_t rq = make_rsrc(Q + head_off, head_bytes), rk = make_rsrc(K + head_off, head_bytes);
  const __amdgpu_buffer_rsrc_t rv = make_rsrc(V + head_off, head_bytes);
  float m[4] = {0.f, 0.f, 0.f, 0.f};
  float acc[NP];
  u32x4 qk[NP], gk[NP];   // this thread's Q and dO chunks of the chunk
#pragma unroll
  for (int p = 0; p < NP; ++p) {
    const int r = tid / TPR + p * RPI;
    // (Rows past the chunk take the first offset past the head, so no
    // offset wraps around 2^32.)
    const uint32_t off = r < rows ? (uint32_t)((row0 + r) * D + col) * 2u : head_bytes;
    const u32x4 o = bload128(ro, off), g = bload128(rg, off), qv = bload128(rq, off);
    const u32x4 kv = bload128(rk, off), vv = bload128(rv, off);
    acc[p] = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      acc[p] += bf16_lo(o[i]) * bf16_lo(g[i]) + bf16_hi(o[i]) * bf16_hi(g[i]);
      m[0] = abs_max_bf16x2(m[0], qv[i]);
      m[1] = abs_max_bf16x2(m[1], g[i]);
      m[2] = abs_max_bf16x2(m[2], kv[i]);
      m[3] = abs_max_bf16x2(m[3], vv[i]);
    }
    qk[p] = qv;
    gk[p] = g;
  }
  // D of each row: the TPR threads of a row hold its partial sums.
#pragma unroll
  for (int p = 0; p < NP; ++p) {
#pragma unroll
    for (int o2 = TPR / 2; o2 > 0; o2 >>= 1) acc[p] += __shfl_xor(acc[p], o2);
  }
#pragma unroll
  for (int p = 0; p < NP; ++p) {
    const int r = tid / TPR + p * RPI;
    if (tid % TPR == 0 && r < rows) delta[(size_t)bh * N + row0 + r] = acc[p];
  }
  block_max4<NW>(m, red);
  if (tid < 4) part[((size_t)bh * nch + ch) * 4 + tid] = m[tid];
  const float fq = pow2_scale_for(m[0]), fg = pow2_scale_for(m[1]);
#pragma unroll
  for (int p = 0; p < NP; ++p) {
    const int r = tid / TPR + p * RPI;
    if (r < rows) {
      const size_t off = ((size_t)bh * N + row0 + r) * D + col;
      *(u32x4*)(Q16 + off) = bf16x8_to_f16x8(qk[p], fq);
      *(u32x4*)(dO16 + off) = bf16x8_to_f16x8(gk[p], fg);
    }
  }
}

// ---------------------------------------------------------------------------
// 2. Per 256-row chunk of a head: the head's factors (from all its chunk
//    maxima); where the chunk's own factor for Q or dO (the one kernel 1
//    converted it with) is not the head's, the chunk's rows of that tensor
//    again from the bf16 source, times the head's factor (so every fp16 copy
//    is the bf16 value times the head's factor, rounded once); and its row
//    terms, in two planes of N floats per head: the start value
//    of the row's S accumulator, -LSE log2 e / c2 with c2 the exponent's
//    multiplier of the scaled S (-inf for a row that saw no key, so that
//    P = exp2(c2 S) = 0 there), and of its dP accumulator, -D times the dO
//    and V factors (so that dS = P dP).  The chunk-0 workgroup of each head
//    records the factors.
// ---------------------------------------------------------------------------
template <int D>
__global__ void __launch_bounds__(256)
fa_bwd_convert_kernel(const __bf16* __restrict__ Q, const __bf16* __restrict__ dO, const float* __restrict__ LSE,
                      const float* __restrict__ delta, const float* __restrict__ part, float* __restrict__ scales,
                      float* __restrict__ rowterm, _Float16* __restrict__ Q16, _Float16* __restrict__ dO16, int N,
                      int nch, float scale_log2) {
  const int bh = blockIdx.x / nch, ch = blockIdx.x % nch;
  const int tid = threadIdx.x;
  // Every wave takes the head's maxima over its chunks by itself (a few
  // dozen floats), with no barrier.
  float f[4];
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    float m = 0.f;
    for (int i = tid & 63; i < nch; i += 64) m = fmaxf(m, part[((size_t)bh * nch + i) * 4 + t]);
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) m = fmaxf(m, __shfl_xor(m, off));
    f[t] = pow2_scale_for(m);
  }
  if (ch == 0 && tid == 0) {
#pragma unroll
    for (int t = 0; t < 4; ++t) scales[bh * 4 + t] = f[t];
  }
  const int row0 = ch * kBwdChunkRows;
  const int rows = min(kBwdChunkRows, N - row0);
  const size_t rbase = (size_t)bh * N + row0;
  if (tid < rows) {
    const float l = LSE[rbase + tid];
    const float c2 = scale_log2 / (f[0] * f[2]);
    float* plane = rowterm + (size_t)2 * bh * N;
    plane[row0 + tid] = l == -INFINITY ? -INFINITY : -(l * kLog2e) / c2;
    plane[N + row0 + tid] = -(delta[rbase + tid] * (f[1] * f[3]));
  }
  const __bf16* src[2] = {Q, dO};
  _Float16* dst[2] = {Q16, dO16};
  const int n8 = rows * (D / 8);
  // All of a thread's loads are issued before its first store, so a chunk
  // costs one memory round trip rather than one per 16-byte piece.
  constexpr int kIter = kBwdChunkRows * (D / 8) / 256;
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    // The same float kernel 1 computed, so the same factor.
    const float own = pow2_scale_for(part[((size_t)bh * nch + ch) * 4 + t]);
    if (own == f[t]) continue;
    u32x4 x[kIter];
#pragma unroll
    for (int j = 0; j < kIter; ++j) {
      const int i = tid + 256 * j;
      if (i < n8) x[j] = *(const u32x4*)(src[t] + rbase * D + 8 * (size_t)i);
    }
#pragma unroll
    for (int j = 0; j < kIter; ++j) {
      const int i = tid + 256 * j;
      if (i < n8) *(u32x4*)(dst[t] + rbase * D + 8 * (size_t)i) = bf16x8_to_f16x8(x[j], f[t]);
    }
  }
}

// ---------------------------------------------------------------------------
// Shared by the two main kernels: 8 waves in two groups of four (waves 0-3,
// waves 4-7; one wave of each group per SIMD).  128 rows are resident (keys
// for dK/dV, queries for dQ); the other side is walked in 32-row blocks, the
// group g taking blocks g, g + 2, g + 4, ... of the list of visited blocks
// into two LDS buffers of its own.  A group's step alternates a matrix
// phase (the gradient products of its previous block and the two
// score-side products of its current block) and a vector phase (P and dS
// of the current block, while its next block is copied into LDS); group 1
// runs one phase behind group 0, so the two waves of a SIMD alternate
// between the matrix cores and the vector ALU.
//
// Tiles sit in LDS as fp16 with unpadded rows whose 16-byte chunks are
// permuted: chunk c of row r is stored at chunk c ^ f(r).  Both ways a tile
// is read then hit 64 distinct banks per 256 bytes served:
//   * rows as MFMA operands (ds_read_b128; 16 lanes = 16 consecutive rows
//     at one chunk): f is a bijection on the rows of each 16-row group;
//   * columns with ds_read_b64_tr_b16 (32 lanes = 4 consecutive rows x 4
//     consecutive chunks, half a chunk each): f puts each of 4 consecutive
//     rows into a different aligned group of 4 chunks.
// With t = r / (128 / D) (the rows of one 256-byte bank sweep share t) and
// L = D / 32: f = 4 (t % L) + (t / L) % 4.
// ---------------------------------------------------------------------------
using layout::bwd_chunk_off;
using layout::bwd_swz;
using layout::bwd_tr_off;

// The reads below address LDS in bytes from a lane constant and an XOR with
// a compile-time constant: chunk 2 ks + lg of row r is at byte
// 2 bwd_chunk_off(r, lg) ^ 32 ks (f only permutes, and 2 ks + lg =
// 2 ks ^ lg), and the transposing read of rows 16 c + 8 h .. at columns
// 32 dm .. is at byte (2 bwd_tr_off(lane, 8 h, 0) ^ 64 dm) + 32 c D (the
// rows' permutation depends on the row only modulo 16, and 32 dm
// columns are 4 dm chunks, which f's upper bits XOR).  The XOR'd bits are
// zero in every row's and buffer's base address.
__device__ __forceinline__ f16x8 lds_row(const _Float16* base, uint32_t byte_off) {
  return *(const f16x8*)((const char*)base + byte_off);
}
__device__ __forceinline__ f16x8 lds_tr_pair_b(const _Float16* base, uint32_t lo_bytes, uint32_t hi_bytes) {
  return lds_tr_pair_h((const _Float16*)((const char*)base + lo_bytes), 0, (int)(hi_bytes - lo_bytes) / 2);
}
// This lane's element offset for the transposing read of rows r0 .. r0 + 3
// (lanes 0-31; lanes 32-63: rows r0 + 4 .. r0 + 7) at feature columns
// 32 dm .. 32 dm + 31: lane s = l % 16, G = bit 4, g = bit 5 reads half a
// chunk of row r0 + 4 g + s / 4 at column 32 dm + 16 G + 4 (s % 4).
template <int D>
__device__ __forceinline__ int bwd_tr_off(int lane, int r0, int dm) {
  const int s = lane & 15, G = (lane >> 4) & 1, g = lane >> 5;
  return bwd_chunk_off<D>(r0 + 4 * g + (s >> 2), 4 * dm + 2 * G + ((s & 3) >> 1)) + 4 * (s & 1);
}

template <int D>
struct BwdCfg {
  static constexpr int kThreads = 512;
  static constexpr int RES = 128;                  // resident rows per workgroup (4 blocks of 32)
  static constexpr int BLK = 32;                   // rows of a walked block
  static constexpr int kResTile = RES * D;         // one resident tensor (dK/dV kernel), fp16 elements
  static constexpr int kBlkTile = BLK * D;
  static constexpr int kResBytes = 2 * kResTile * 2;
  // A staged block: two fp16 tensors, then (dK/dV kernel) the row terms.
  static constexpr int kStageBytes = 2 * kBlkTile * 2 + BLK * 8;
  static constexpr int kStagesBytes = 4 * kStageBytes;            // 2 groups x 2 buffers
  static constexpr int kLdsBytes = kResBytes + kStagesBytes;
  // Closing sum of the two groups' accumulators: per lane of one group,
  // the dK/dV kernel's D floats (dK^T and dV^T halves), the dQ kernel's D / 2.
  static constexpr int kRedBytes = D * 4 * 64 * 4;
  static constexpr int kLdsTotal = kLdsBytes > kRedBytes ? kLdsBytes : kRedBytes;
  // The dQ kernel's blocks are K and V only, three buffers per group.
  static constexpr int kDqStageBytes = 2 * kBlkTile * 2;
  // Six block buffers and (prologue) the Q/dO slots past them
  // (layout::bwd_dq_qslot), or the closing sum.
  static constexpr int kDqLdsTotal = 8 * kDqStageBytes > kRedBytes / 2 ? 8 * kDqStageBytes : kRedBytes / 2;
  static_assert(kDqLdsTotal + 4 * (65536 / BLK + 1) <= 160 * 1024, "dQ LDS budget (with a sparse block list)");
  static_assert(kLdsTotal + 4 * (65536 / BLK + 1) <= 160 * 1024, "LDS budget (with a sparse block list)");
  static_assert(kResBytes % 1024 == 0 && kStageBytes % 256 == 0 && kBlkTile * 2 % 1024 == 0, "tile alignment");
};

// Per-head buffer descriptors over the fp16 copies and the two row-term
// planes (rt0: S start values, rt1: dP start values): rows past N read as
// zero.
struct BwdHead {
  __amdgpu_buffer_rsrc_t q, k, v, g, rt0, rt1;
};

template <int D>
__device__ __forceinline__ BwdHead bwd_head(const _Float16* Q16, const _Float16* K16, const _Float16* V16,
                                            const _Float16* dO16, const float* rowterm, int bh, int N) {
  const size_t head_off = (size_t)bh * N * D;
  const uint32_t head_bytes = (uint32_t)N * D * 2u;
  BwdHead h;
  h.q = make_rsrc(Q16 + head_off, head_bytes);
  h.k = make_rsrc(K16 + head_off, head_bytes);
  h.v = make_rsrc(V16 + head_off, head_bytes);
  h.g = make_rsrc(dO16 + head_off, head_bytes);
  h.rt0 = make_rsrc(rowterm + (size_t)2 * bh * N, (uint32_t)N * 4u);
  h.rt1 = make_rsrc(rowterm + (size_t)2 * bh * N + N, (uint32_t)N * 4u);
  return h;
}

// Rows row0 .. row0 + ROWS of an fp16 [., D] head into a permuted LDS tile,
// copied by NW waves (w = 0 .. NW - 1) with buffer_load ... lds: each
// instruction fills 1 KB of the tile in lane order, lane i fetching the
// global chunk that the permutation stores at byte 16 i.  Completion is
// tracked by the issuing wave's vmcnt.
template <int D, int ROWS, int NW>
__device__ __forceinline__ void dma_rows(__amdgpu_buffer_rsrc_t r, _Float16* tile, int row0, int w, int lane) {
  constexpr int kInst = ROWS * D * 2 / 1024;
  static_assert(kInst % NW == 0, "copy split");
#pragma unroll
  for (int i = 0; i < kInst / NW; ++i) {
    const int inst = w * (kInst / NW) + i;
    int row, c;
    layout::copy_slot(2 * D, inst, lane, bwd_swz<D>, row, c);
    lds_copy16(r, (uint32_t)((row0 + row) * D + 8 * c) * 2u, (uint32_t)(uintptr_t)((char*)tile + inst * 1024));
  }
}

// Wave 0 lists the visited 32-row blocks whose 128-block entry `keep(e)`
// is nonzero among candidates 0 .. n - 1 into list[1 ..] (count in list[0]),
// then every wave reads the count.
template <typename Keep>
__device__ __forceinline__ int build_block_list(int* list, int n, int wave, int lane, Keep keep) {
  if (wave == 0) {
    int cnt = 0;
    for (int base = 0; base < n; base += 64) {
      const int e = base + lane;
      const bool live = e < n && keep(e);
      const uint64_t bal = __ballot(live);
      const int pos = cnt + __builtin_amdgcn_mbcnt_hi((uint32_t)(bal >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)bal, 0));
      if (live) list[1 + pos] = e;
      cnt += __popcll(bal);
    }
    if (lane == 0) list[0] = cnt;
  }
  __syncthreads();
  return __builtin_amdgcn_readfirstlane(list[0]);
}

// The matrix phase of a step as one stream of MFMAs whose LDS operands are
// read kLookahead operands ahead of their product, so the read latency
// hides behind the preceding products.  The stream is the gradient
// products of the group's previous block, then the two score-side products
// of its current block.  Scheduling barriers keep it in this order.  Either
// half can run alone (GRADS / SCORES): a wave's first step has no previous
// block, and the round after its last step no current one.
constexpr int kLookahead = 8;

// dK/dV kernel.  Operands: per (c, dm) of the gradient products dO^T then
// Q^T (transposing reads of the previous block, rows 16 c .. 16 c + 15),
// then per k-step Q, K, dO, V rows (Q, dO of the current block; K, V
// resident, already offset to this wave's key block).  GRADS / SCORES
// false: the stream without the gradient / the score-side products.
template <int D, bool GRADS = true, bool SCORES = true>
__device__ __forceinline__ void dkdv_matrix_phase(f32x16 (&dk_acc)[D / 32], f32x16 (&dv_acc)[D / 32],
                                                  const uint32_t (&pw)[8], const uint32_t (&dsw)[8], f32x16& sc,
                                                  f32x16& dpc, const _Float16* Qp, const _Float16* Gp,
                                                  const _Float16* Qc, const _Float16* Gc, const _Float16* Kr,
                                                  const _Float16* Vr, const float* Lc, int lg, uint32_t rowx,
                                                  uint32_t trx0, uint32_t trx1) {
  constexpr int DM = D / 32, KS = D / 16, L = kLookahead;
  constexpr int NG = GRADS ? 4 * DM : 0;   // gradient products (one operand read each)
  constexpr int NS = SCORES ? 2 * KS : 0;  // score products (two operand reads each)
  constexpr int NL = NG + 2 * NS;          // operand reads
  auto load = [&](int j) -> f16x8 {
    if (j < NG) {
      const int c = (j / 2) / DM, dm = (j / 2) % DM;
      return lds_tr_pair_b(j % 2 == 0 ? Gp : Qp, (trx0 ^ (64u * dm)) + 32u * c * D, (trx1 ^ (64u * dm)) + 32u * c * D);
    }
    const int i = j - NG, t = i % 4;
    const _Float16* base = t == 0 ? Qc : t == 1 ? Kr : t == 2 ? Gc : Vr;
    return lds_row(base, rowx ^ (32u * (i / 4)));
  };
  f16x8 ring[L];
#pragma unroll
  for (int j = 0; j < L && j < NL; ++j) ring[j] = load(j);
  // S and dP start at their rows' start values (register i: row
  // 8 (i / 4) + 4 lg + i % 4 of the block), -LSE log2 e / c2 and -D, so the
  // vector phase takes P = exp2(c2 S) and dS = P dP.  They are read a few
  // gradient products before the score products (early enough to complete
  // behind them, late enough not to be held through all of them).
  constexpr int kStartAt = NG > 8 ? NG - 8 : 0;
  auto load_start = [&]() {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const f32x4 a = *(const f32x4*)(Lc + 8 * i + 4 * lg);
      const f32x4 b = *(const f32x4*)(Lc + 32 + 8 * i + 4 * lg);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        sc[4 * i + j] = a[j];
        dpc[4 * i + j] = b[j];
      }
    }
  };
  __builtin_amdgcn_s_setprio(1);
  __builtin_amdgcn_sched_barrier(0);
  int next = L;   // next operand to read
#pragma unroll
  for (int k = 0; k < NG + NS; ++k) {
    if (SCORES && k == kStartAt) load_start();
    int used;   // operands consumed through this product
    if (k < NG) {
      const int c = (k / 2) / DM, dm = (k / 2) % DM;
      const uint32_t* w = k % 2 == 0 ? pw : dsw;
      const f16x8 b = __builtin_bit_cast(f16x8, ((u32x4){w[4 * c], w[4 * c + 1], w[4 * c + 2], w[4 * c + 3]}));
      if (k % 2 == 0) dv_acc[dm] = mfma32h(ring[k % L], b, dv_acc[dm]);
      else dk_acc[dm] = mfma32h(ring[k % L], b, dk_acc[dm]);
      used = k + 1;
    } else {
      const int i = k - NG, j = NG + 4 * (i / 2) + 2 * (i % 2);
      if (i % 2 == 0) sc = mfma32h(ring[j % L], ring[(j + 1) % L], sc);
      else dpc = mfma32h(ring[j % L], ring[(j + 1) % L], dpc);
      used = j + 2;
    }
#pragma unroll
    for (int j = next; j < used + L && j < NL; ++j) ring[j % L] = load(j);
    next = used + L < NL ? used + L : NL;
    __builtin_amdgcn_sched_barrier(0);
  }
  __builtin_amdgcn_s_setprio(0);
}

// dQ kernel.  Operands: per (c, dm) K^T (transposing read of the previous
// block), then (SCORES) per k-step K and V rows of the current block; Q and
// dO are the register B operands.  The score accumulators start at st0 and
// dpt0 (the lane's query's -LSE log2 e / c2 and -D) instead of zero.
template <int D, bool SCORES = true>
__device__ __forceinline__ void dq_matrix_phase(f32x16 (&dq_acc)[D / 32], const uint32_t (&dsw)[8], f32x16& st,
                                                f32x16& dpt, const f16x8 (&qbf)[D / 16], const f16x8 (&gbf)[D / 16],
                                                const _Float16* Kp, const _Float16* Kc, const _Float16* Vc,
                                                uint32_t rowx, uint32_t trx0, uint32_t trx1, float st0, float dpt0) {
  constexpr int DM = D / 32, KS = D / 16, L = kLookahead;
  constexpr int NG = 2 * DM;
  constexpr int NS = SCORES ? 2 * KS : 0;
  constexpr int NL = NG + NS;              // one operand read per product
  auto load = [&](int j) -> f16x8 {
    if (j < NG) {
      const int c = j / DM, dm = j % DM;
      return lds_tr_pair_b(Kp, (trx0 ^ (64u * dm)) + 32u * c * D, (trx1 ^ (64u * dm)) + 32u * c * D);
    }
    const int i = j - NG;
    return lds_row(i % 2 == 0 ? Kc : Vc, rowx ^ (32u * (i / 2)));
  };
  f16x8 ring[L];
#pragma unroll
  for (int j = 0; j < L && j < NL; ++j) ring[j] = load(j);
  // (An empty asm per phase keeps the compiler from holding splatted copies
  // of the start values across the loop.)
  if constexpr (SCORES) {
    asm volatile("" : "+v"(st0), "+v"(dpt0));
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      st[i] = st0;
      dpt[i] = dpt0;
    }
  }
  __builtin_amdgcn_s_setprio(1);
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int k = 0; k < NL; ++k) {
    if (k < NG) {
      const int c = k / DM, dm = k % DM;
      const f16x8 b = __builtin_bit_cast(f16x8, ((u32x4){dsw[4 * c], dsw[4 * c + 1], dsw[4 * c + 2], dsw[4 * c + 3]}));
      dq_acc[dm] = mfma32h(ring[k % L], b, dq_acc[dm]);
    } else {
      const int i = k - NG;
      if (i % 2 == 0) st = mfma32h(ring[k % L], qbf[i / 2], st);
      else dpt = mfma32h(ring[k % L], gbf[i / 2], dpt);
    }
    if (k + L < NL) ring[k % L] = load(k + L);
    __builtin_amdgcn_sched_barrier(0);
  }
  __builtin_amdgcn_s_setprio(0);
}

// ---------------------------------------------------------------------------
// 3. dK and dV: one workgroup per 128-key tile of one head.  Wave w owns key
//    block kb = w % 4 (32 keys); group g = w / 4 walks every other visited
//    32-query block.  K and V of the tile sit in LDS (their rows are the B
//    operands of S = Q K^T and dP = dO V^T, one key per lane); Q and dO of a
//    block are staged; dV^T += dO^T P and dK^T += Q^T dS take their A
//    operands with ds_read_b64_tr_b16 and P, dS straight from registers.
// SPARSE: block-sparse attention.  bmask holds, per head, an nb x nb byte
// matrix over (128-query block, 128-key block) pairs (a workgroup's keys are
// one key block); the workgroup visits only the query blocks its mask
// column keeps.
// ---------------------------------------------------------------------------
template <int D, bool CAUSAL, bool SPARSE>
__global__ void __launch_bounds__(512)
fa_bwd_dkdv_kernel(const _Float16* __restrict__ Q16, const __bf16* __restrict__ K, const __bf16* __restrict__ V,
                   const _Float16* __restrict__ dO16, _Float16* __restrict__ K16, _Float16* __restrict__ V16,
                   const float* __restrict__ rowterm, const float* __restrict__ scales, __bf16* __restrict__ dK,
                   __bf16* __restrict__ dV, const uint8_t* __restrict__ bmask, int N, int BH, int wpx, float scale,
                   float scale_log2) {
  using C = BwdCfg<D>;
  static_assert(C::RES == FA_SPARSE_BLOCK && FA_SPARSE_BLOCK % C::BLK == 0, "sparse blocks vs tiles");
  constexpr int DM = D / 32;                 // 32-feature blocks
  extern __shared__ __attribute__((aligned(16))) char smem_raw[];
  _Float16* Ks = (_Float16*)smem_raw;                              // [RES][D], permuted chunks
  _Float16* Vs = Ks + C::kResTile;

  const int wave = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);   // uniform per wave
  const int kb = wave & 3;                   // key block of this wave
  const int g = wave >> 2;                   // group

  // One (128-key tile, head) item per pass: this workgroup's own (wpx = 0),
  // or (persistent launch, wpx workgroups per XCD) its share of its XCD's
  // head-major list.
  const int num_tiles = (N + C::RES - 1) / C::RES;
  const int xcd_items = BH / 8 * num_tiles;
  for (int pass = 0;; ++pass) {
  // The thread index enters each pass through an asm, so per-lane address
  // arithmetic stays inside the pass rather than held across all of them.
  int tid_v = threadIdx.x;
  asm volatile("" : "+v"(tid_v));
  const int tid = tid_v;
  const int gt = tid & 255;                  // thread within the group
  const int lane = tid & 63;
  const int lc = lane & 31, lg = lane >> 5;
  int kt, bh;   // key tile (small kt = most query blocks) and head
  if (wpx > 0) {
    const int k = layout::persistent_item(blockIdx.x >> 3, pass, wpx, xcd_items);
    if (k < 0) break;
    layout::xcd_head_major_item(blockIdx.x & 7, k, num_tiles, bh, kt);
  } else {
    if (pass > 0) break;
    xcd_head_major(blockIdx.x, BH, num_tiles, bh, kt);
  }
  const BwdHead h = bwd_head<D>(Q16, K16, V16, dO16, rowterm, bh, N);
  const size_t head_off = (size_t)bh * N * D;

  const int k0 = kt * C::RES;                 // first key of the workgroup
  const int kw0 = k0 + kb * 32;               // first key of this wave
  const int key = kw0 + lc;                   // this lane's key column
  const bool key_ok = key < N;

  // In the fp16 operands' units: the exponent's multiplier for the scaled
  // S and the epilogue factors.
  const float sq = scales[bh * 4 + 0], sg = scales[bh * 4 + 1];
  const float sk = scales[bh * 4 + 2], sv = scales[bh * 4 + 3];
  const float c2 = scale_log2 / (sq * sk);
  const float dk_fac = scale / (sg * sv * sq);
  const float dv_fac = 1.f / sg;

  // Visited 32-query blocks: all from jb on (under the causal mask, blocks
  // before the tile's first key see none of its keys), or those the mask
  // column keeps; the list sits after the other buffers.
  const int jb = CAUSAL ? k0 / C::BLK : 0;
  int n_blk = (N + C::BLK - 1) / C::BLK - jb;
  int* slist = (int*)(smem_raw + C::kLdsTotal);
  if constexpr (SPARSE) {
    const int nb = (N + FA_SPARSE_BLOCK - 1) / FA_SPARSE_BLOCK;
    const uint8_t* col = bmask + (size_t)bh * nb * nb + kt;   // entry of query block i at col[i * nb]
    n_blk = build_block_list(slist, n_blk, wave, lane, [&](int e) {
      return col[(size_t)((jb + e) * C::BLK / FA_SPARSE_BLOCK) * nb] != 0;
    });
  }
  auto blk_at = [&](int e) { return jb + (SPARSE ? slist[1 + e] : e); };
  const int R = (n_blk + 1) / 2;                 // steps of group 0; group 1 has n_blk / 2
  auto valid = [&](int r) { return 2 * r + g < n_blk; };

  char* gstage = smem_raw + C::kResBytes + g * 2 * C::kStageBytes;
  auto Qb = [&](int b) { return (_Float16*)(gstage + b * C::kStageBytes); };
  auto Gb = [&](int b) { return Qb(b) + C::kBlkTile; };
  auto Lb = [&](int b) { return (float*)(Gb(b) + C::kBlkTile); };   // 32 S, then 32 dP start values
  // The group's step r into buffer b: Q and dO rows and the row terms (rows
  // past N read as zeros: their Q and dO rows are zero, so they add nothing).
  auto stage = [&](int r, int b) {
    const int q0 = blk_at(2 * r + g) * C::BLK;
    dma_rows<D, C::BLK, 4>(h.q, Qb(b), q0, kb, lane);
    dma_rows<D, C::BLK, 4>(h.g, Gb(b), q0, kb, lane);
    // The block's 32 S start values (lanes 0-7) and 32 dP start values
    // (lanes 8-15, landing 128 bytes further on).
    if (kb == 0 && lane < C::BLK / 4)
      lds_copy16(h.rt0, (uint32_t)(q0 * 4 + 16 * lane), (uint32_t)(uintptr_t)Lb(b));
    if (kb == 0 && lane >= C::BLK / 4 && lane < C::BLK / 2)
      lds_copy16(h.rt1, (uint32_t)(q0 * 4 + 16 * (lane - C::BLK / 4)), (uint32_t)(uintptr_t)Lb(b));
  };

  // This wave's K / V rows (B operands; row 32 kb + lc has the same chunk
  // permutation as row lc) and the lane's byte constants of its reads.
  const int krow_base = 32 * kb * D;
  const uint32_t rowx = 2u * bwd_chunk_off<D>(lc, lg);
  const uint32_t trx0 = 2u * bwd_tr_off<D>(lane, 0, 0), trx1 = 2u * bwd_tr_off<D>(lane, 8, 0);

  f32x16 dk_acc[DM], dv_acc[DM];
#pragma unroll
  for (int i = 0; i < DM; ++i) {
    dk_acc[i] = (f32x16){};
    dv_acc[i] = (f32x16){};
  }
  f32x16 sc, dpc;             // S and dP of the current block
  uint32_t pw[8], dsw[8];     // P and dS of the previous block, fp16 pairs
#pragma unroll
  for (int i = 0; i < 8; ++i) pw[i] = dsw[i] = 0u;

  // The group's first block into buffer 0 and zeros into the buffers no
  // block is copied to before the loop (no product reads a buffer before a
  // block lands in it: the fill only keeps every stage buffer finite, and
  // without it the loop's register allocation measured about 1 % slower).
  // Then the resident K, V times their factors as fp16, into LDS (the
  // kernel copies them on to the workspace for the dQ kernel at its end,
  // so no wait here covers those stores).
  if (valid(0)) stage(0, 0);
  for (int b = valid(0) ? 1 : 0; b < 2; ++b)
    for (int i = gt; i < C::kStageBytes / 16; i += 256)
      ((u32x4*)(gstage + b * C::kStageBytes))[i] = (u32x4){0u, 0u, 0u, 0u};
  {
    constexpr int kChunks = C::RES * D / 8 / C::kThreads;
    const __amdgpu_buffer_rsrc_t rk = make_rsrc(K + head_off, (uint32_t)N * D * 2u);
    const __amdgpu_buffer_rsrc_t rv = make_rsrc(V + head_off, (uint32_t)N * D * 2u);
    u32x4 kx[kChunks], vx[kChunks];
#pragma unroll
    for (int i = 0; i < kChunks; ++i) {
      const int c = tid + i * C::kThreads;
      const uint32_t off = (uint32_t)((k0 + c / (D / 8)) * D + (c % (D / 8)) * 8) * 2u;
      kx[i] = bload128(rk, off);
      vx[i] = bload128(rv, off);
    }
#pragma unroll
    for (int i = 0; i < kChunks; ++i) {
      const int c = tid + i * C::kThreads, row = c / (D / 8), ch = c % (D / 8);
      const int lo = bwd_chunk_off<D>(row, ch);
      *(u32x4*)(Ks + lo) = bf16x8_to_f16x8(kx[i], sk);
      *(u32x4*)(Vs + lo) = bf16x8_to_f16x8(vx[i], sv);
    }
  }
  wait_vmem_all();
  __syncthreads();
  if (g == 1) __syncthreads();
  // P = exp2(c2 S) and dS = P dP of step r (S and dP started at their rows'
  // start values) as fp16 pairs.
  auto scores_to_p = [&](int r) {
    // Keys past N and (causal) keys after the query: P = 0.  The query
    // offset of register i is 8 (i / 4) + 4 lg + i % 4.
    const int qw0 = blk_at(2 * r + g) * C::BLK;
    if ((kw0 + 31 >= N) || (CAUSAL && qw0 < kw0 + 31)) {
      const int tl = !key_ok ? 64 : (CAUSAL ? key - qw0 - 4 * lg : -64);
#pragma unroll
      for (int i = 0; i < 16; ++i) sc[i] = 8 * (i >> 2) + (i & 3) >= tl ? sc[i] : -INFINITY;
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float p[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) p[j] = fast_exp2(sc[4 * i + j] * c2);
      pw[2 * i] = pack_f16x2(p[0], p[1]);
      pw[2 * i + 1] = pack_f16x2(p[2], p[3]);
      dsw[2 * i] = pack_f16x2(p[0] * dpc[4 * i], p[1] * dpc[4 * i + 1]);
      dsw[2 * i + 1] = pack_f16x2(p[2] * dpc[4 * i + 2], p[3] * dpc[4 * i + 3]);
    }
  };
  // The copy of step r + 1 into the buffer step r - 1 used (its last reader
  // was the matrix phase just ended).
  auto stage_next = [&](int r) {
    if (valid(r + 1)) stage(r + 1, (r + 1) & 1);
  };
  // The group's steps are r < n_valid; round r runs the gradient products
  // of step r - 1 and the score-side products of step r, so the first round
  // has no gradient products and round n_valid no score products.  Under
  // the causal mask (dense) the first d0 steps of this wave are query
  // blocks that end before its first key (P = dS = 0): it runs only its
  // share of the copies, the waits and the barriers on those rounds, and
  // its first live round has no gradient products either (skipping exact
  // zeros: the result is the same bit for bit).  Rounds past n_valid only
  // keep the barriers.
  const int n_valid = (n_blk - g + 1) / 2;
  int d0 = 0;
  if constexpr (CAUSAL && !SPARSE) d0 = min(n_valid, kb > g ? (kb - g + 1) / 2 : 0);
  int r = 0;
  for (; r < d0; ++r) {
    __syncthreads();
    stage_next(r);
    wait_vmem_all();
    __syncthreads();
  }
  if (r < n_valid) {
    dkdv_matrix_phase<D, false, true>(dk_acc, dv_acc, pw, dsw, sc, dpc, Qb(0), Gb(0), Qb(r & 1), Gb(r & 1),
                                      Ks + krow_base, Vs + krow_base, Lb(r & 1), lg, rowx, trx0, trx1);
    __syncthreads();
    stage_next(r);
    scores_to_p(r);
    wait_vmem_all();
    __syncthreads();
    ++r;
  }
  for (; r < n_valid; ++r) {
    // Matrix phase: dV and dK of step r - 1; S and dP of step r.
    {
      const int cb = r & 1, pbuf = cb ^ 1;
      dkdv_matrix_phase<D>(dk_acc, dv_acc, pw, dsw, sc, dpc, Qb(pbuf), Gb(pbuf), Qb(cb), Gb(cb), Ks + krow_base,
                           Vs + krow_base, Lb(cb), lg, rowx, trx0, trx1);
    }
    __syncthreads();
    // Vector phase: the next copy, P and dS of step r, the wait.
    stage_next(r);
    scores_to_p(r);
    wait_vmem_all();
    __syncthreads();
  }
  // Round n_valid: the gradient products of the last step.
  if (r <= R) {
    if (n_valid > d0) {
      const int pbuf = (r & 1) ^ 1;
      dkdv_matrix_phase<D, true, false>(dk_acc, dv_acc, pw, dsw, sc, dpc, Qb(pbuf), Gb(pbuf), Qb(0), Gb(0),
                                        Ks + krow_base, Vs + krow_base, Lb(0), lg, rowx, trx0, trx1);
    }
    __syncthreads();
    wait_vmem_all();
    __syncthreads();
    ++r;
  }
  for (; r <= R; ++r) {
    __syncthreads();
    __syncthreads();
  }
  if (g == 0) __syncthreads();

  // The fp16 K, V rows of the tile (rows below N) on to the workspace for
  // the dQ kernel; the closing sum below reuses this LDS.
  {
    // All the LDS reads first (they overlap), then the stores.
    constexpr int kChunks = C::RES * D / 8 / C::kThreads;
    u32x4 kv[kChunks], vv[kChunks];
#pragma unroll
    for (int i = 0; i < kChunks; ++i) {
      const int c = tid + i * C::kThreads, row = c / (D / 8), ch = c % (D / 8);
      const int lo = bwd_chunk_off<D>(row, ch);
      kv[i] = *(const u32x4*)(Ks + lo);
      vv[i] = *(const u32x4*)(Vs + lo);
    }
#pragma unroll
    for (int i = 0; i < kChunks; ++i) {
      const int c = tid + i * C::kThreads, row = c / (D / 8), ch = c % (D / 8);
      if (k0 + row < N) {
        const size_t go = head_off + (size_t)(k0 + row) * D + 8 * ch;
        *(u32x4*)(K16 + go) = kv[i];
        *(u32x4*)(V16 + go) = vv[i];
      }
    }
  }
  __syncthreads();

  // Close: the two groups' partial dK^T and dV^T are summed through LDS.
  // Group 0 finishes dK and group 1 dV: each writes the other's partial,
  // 16 bytes per lane and instruction with consecutive lanes on consecutive
  // chunks, then adds the one it finishes.  Stored as dK = scale dK^T and
  // dV = dV^T in the inputs' units, bf16 rows of this lane's key.
  // red_at(t, c): chunk c (accumulator registers 4 (c % 4) .. + 3 of
  // feature block c / 4) of tensor t (0 dK, 1 dV) of key block kb.
  f32x4* red = (f32x4*)smem_raw;
  auto red_at = [&](int t, int c) { return red + (((size_t)t * (D / 8) + c) * 4 + kb) * 64 + lane; };
  // (The branches on g keep every register index a constant.)
  auto put = [&](const f32x16 (&a)[DM], int t) {
#pragma unroll
    for (int c = 0; c < D / 8; ++c)
      *red_at(t, c) = (f32x4){a[c / 4][4 * (c % 4)], a[c / 4][4 * (c % 4) + 1], a[c / 4][4 * (c % 4) + 2],
                              a[c / 4][4 * (c % 4) + 3]};
  };
  auto add_partner = [&](f32x16 (&a)[DM], int t) {
#pragma unroll
    for (int c = 0; c < D / 8; ++c) {
      const f32x4 b = *red_at(t, c);
      const int dm = c / 4, r0 = 4 * (c % 4);
#pragma unroll
      for (int e = 0; e < 4; ++e) a[dm][r0 + e] += b[e];
    }
  };
  if (g == 0) put(dv_acc, 1);
  else put(dk_acc, 0);
  __syncthreads();
  if (g == 0) add_partner(dk_acc, 0);
  else add_partner(dv_acc, 1);
  // Every partial is read before the LDS stages the finished rows: this
  // wave's 32 keys (rows kw0 .. kw0 + 31) of its tensor, written as whole
  // rows.
  __syncthreads();
  {
    __bf16* stage = (__bf16*)smem_raw + wave * 32 * D;
    if (g == 0) store_o_rows<D>(dk_acc, dk_fac, stage, dK + head_off, kw0, N, lane);
    else store_o_rows<D>(dv_acc, dv_fac, stage, dV + head_off, kw0, N, lane);
  }
  // The closing sum's LDS is read by every wave before the next item's
  // copies and conversions overwrite it.
  if (wpx > 0) __syncthreads();
  }
}

// ---------------------------------------------------------------------------
// 4. dQ: one workgroup per 128-query tile of one head.  Wave w owns query
//    block qb = w % 4; group g = w / 4 walks every other visited 32-key
//    block.  With the scores transposed (S^T = K Q^T, one query per lane),
//    Q and dO are the B operands (registers), the staged K and V rows the A
//    operands, and dS^T feeds dQ^T += K^T dS^T straight from registers with
//    K^T read transposed in the key order the accumulator leaves.
// SPARSE: the workgroup's 128 queries are one mask row; it visits only the
// key blocks that row keeps.
// ---------------------------------------------------------------------------
template <int D, bool CAUSAL, bool SPARSE>
__global__ void __launch_bounds__(512)
fa_bwd_dq_kernel(const _Float16* __restrict__ Q16, const _Float16* __restrict__ K16,
                 const _Float16* __restrict__ V16, const _Float16* __restrict__ dO16,
                 const float* __restrict__ rowterm, const float* __restrict__ scales, __bf16* __restrict__ dQ,
                 const uint8_t* __restrict__ bmask, int N, int BH, int wpx, float scale, float scale_log2) {
  using C = BwdCfg<D>;
  static_assert(C::RES == FA_SPARSE_BLOCK && FA_SPARSE_BLOCK % C::BLK == 0, "sparse blocks vs tiles");
  constexpr int KS = D / 16;
  constexpr int DM = D / 32;
  extern __shared__ __attribute__((aligned(16))) char smem_raw[];

  const int wave = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
  const int qb = wave & 3;                   // query block of this wave
  const int g = wave >> 2;                   // group
  const int num_qt = (N + C::RES - 1) / C::RES;

  // One (128-query tile, head) item per pass, as in the dK/dV kernel.
  const int xcd_items = BH / 8 * num_qt;
  for (int pass = 0;; ++pass) {
  int tid_v = threadIdx.x;
  asm volatile("" : "+v"(tid_v));
  const int tid = tid_v;
  const int gt = tid & 255;
  const int lane = tid & 63;
  const int lc = lane & 31, lg = lane >> 5;
  int tile, bh;
  if (wpx > 0) {
    const int k = layout::persistent_item(blockIdx.x >> 3, pass, wpx, xcd_items);
    if (k < 0) break;
    layout::xcd_head_major_item(blockIdx.x & 7, k, num_qt, bh, tile);
  } else {
    if (pass > 0) break;
    xcd_head_major(blockIdx.x, BH, num_qt, bh, tile);
  }
  const int qt = num_qt - 1 - tile;          // heaviest query tiles first (causal)
  const BwdHead h = bwd_head<D>(Q16, K16, V16, dO16, rowterm, bh, N);

  const int qw0 = qt * C::RES + qb * 32;     // first query of this wave
  const int q = qw0 + lc;                    // this lane's query
  const float sq = scales[bh * 4 + 0], sg = scales[bh * 4 + 1];
  const float sk = scales[bh * 4 + 2], sv = scales[bh * 4 + 3];
  const float c2 = scale_log2 / (sq * sk);
  const float dq_fac = scale / (sk * sg * sv);

  // Q (waves 0-3) or dO (waves 4-7) rows of this wave's query block into
  // its LDS slot, 1 KB of consecutive rows per copy (zeros past N); read
  // back below as the B operands.
  dma_rows<D, C::BLK, 1>(g == 0 ? h.q : h.g, (_Float16*)(smem_raw + layout::bwd_dq_qslot<D>(wave)), qw0, 0, lane);
  // Start values of this lane's S^T and dP^T accumulators (the row terms
  // the preprocessing wrote): -LSE log2 e / c2 (-inf past N, so P = 0 there)
  // and -D in the scaled dP's units; then P^T = exp2(c2 S^T) and
  // dS^T = P^T dP^T.
  float st0 = -INFINITY, dpt0 = 0.f;
  if (q < N) {
    st0 = bload32f(h.rt0, (uint32_t)q * 4u);
    dpt0 = bload32f(h.rt1, (uint32_t)q * 4u);
  }

  f32x16 dq_acc[DM];
#pragma unroll
  for (int i = 0; i < DM; ++i) dq_acc[i] = (f32x16){};

  // Visited 32-key blocks: all up to the tile's last query (causal) or N,
  // or those the mask row keeps.
  const int q_tile_end = min(N, (qt + 1) * C::RES);
  int n_blk = ((CAUSAL ? q_tile_end : N) + C::BLK - 1) / C::BLK;
  int* slist = (int*)(smem_raw + C::kDqLdsTotal);
  if constexpr (SPARSE) {
    const int nb = (N + FA_SPARSE_BLOCK - 1) / FA_SPARSE_BLOCK;
    const uint8_t* mrow = bmask + ((size_t)bh * nb + qt) * nb;   // this query block's mask row
    n_blk = build_block_list(slist, n_blk, wave, lane,
                             [&](int e) { return mrow[e * C::BLK / FA_SPARSE_BLOCK] != 0; });
  }
  auto blk_at = [&](int e) { return SPARSE ? slist[1 + e] : e; };
  const int R = (n_blk + 1) / 2;
  auto valid = [&](int r) { return 2 * r + g < n_blk; };

  // Three buffers per group: step r in buffer r % 3, copied two steps ahead.
  char* gstage = smem_raw + g * 3 * C::kDqStageBytes;
  auto Kb = [&](int b) { return (_Float16*)(gstage + b * C::kDqStageBytes); };
  auto Vb = [&](int b) { return Kb(b) + C::kBlkTile; };
  constexpr int kCopies = 2 * (C::BLK * D * 2 / 1024) / 4;   // copy instructions per wave and step
  auto stage = [&](int r, int b) {
    const int k0 = blk_at(2 * r + g) * C::BLK;
    dma_rows<D, C::BLK, 4>(h.k, Kb(b), k0, qb, lane);
    dma_rows<D, C::BLK, 4>(h.v, Vb(b), k0, qb, lane);
  };
  const uint32_t rowx = 2u * bwd_chunk_off<D>(lc, lg);
  const uint32_t trx0 = 2u * bwd_tr_off<D>(lane, 0, 0), trx1 = 2u * bwd_tr_off<D>(lane, 8, 0);

  f32x16 st_acc, dpt;         // S^T and dP^T of the current block
  uint32_t dsw[8];            // dS^T of the previous block, fp16 pairs
#pragma unroll
  for (int i = 0; i < 8; ++i) dsw[i] = 0u;

  // The group's first two blocks into buffers 0 and 1, zeros into those of
  // them the group has no block for (no product reads those).  Round 0's
  // gradient products, whose dS is zero, read buffer 2, which then holds
  // the Q slots: finite operands.
  if (valid(0)) stage(0, 0);
  if (valid(1)) stage(1, 1);
  for (int b = 0; b < 2; ++b)
    if (!valid(b))
      for (int i = gt; i < C::kDqStageBytes / 16; i += 256)
        ((u32x4*)(gstage + b * C::kDqStageBytes))[i] = (u32x4){0u, 0u, 0u, 0u};
  wait_vmem_all();
  __syncthreads();
  // Q^T and dO^T as B operands: lane holds 8 features of its query's row.
  // The reads complete here (the asm uses them), before any wave passes a
  // barrier after which block 2's copy may land on the slots in buffer 2.
  f16x8 qbf[KS], gbf[KS];
  {
    const _Float16* qs = (const _Float16*)(smem_raw + layout::bwd_dq_qslot<D>(qb));
    const _Float16* gs = (const _Float16*)(smem_raw + layout::bwd_dq_qslot<D>(4 + qb));
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      qbf[ks] = *(const f16x8*)(qs + bwd_chunk_off<D>(lc, 2 * ks + lg));
      gbf[ks] = *(const f16x8*)(gs + bwd_chunk_off<D>(lc, 2 * ks + lg));
    }
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) asm volatile("" : "+v"(qbf[ks]), "+v"(gbf[ks]));
  }
  if (g == 1) __syncthreads();
  int cb = 0;   // r % 3
  // P^T and dS^T of step r (the vector phase's arithmetic).
  auto scores_to_ds = [&](int r) {
    // A group without a step r masks all its scores (P = dS = 0).
    // Otherwise keys past N and (causal) keys after the query: P = 0.
    // The key offset of register i is 8 (i / 4) + 4 lg + i % 4.
    const bool has = valid(r);
    const int kw0 = has ? blk_at(2 * r + g) * C::BLK : 0;
    if (!has || (kw0 + 31 >= N) || (CAUSAL && kw0 + 31 > qw0)) {
      const int tl = has ? min(N - 1, CAUSAL ? q : N - 1) - kw0 - 4 * lg : -64;
#pragma unroll
      for (int i = 0; i < 16; ++i) st_acc[i] = 8 * (i >> 2) + (i & 3) <= tl ? st_acc[i] : -INFINITY;
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float p0 = fast_exp2(st_acc[2 * i] * c2);
      const float p1 = fast_exp2(st_acc[2 * i + 1] * c2);
      dsw[i] = pack_f16x2(p0 * dpt[2 * i], p1 * dpt[2 * i + 1]);
    }
  };
  // The copy of step r + 2 into the buffer step r - 1 used (its last reader
  // was the matrix phase just ended), then the wait: step r + 1's copy
  // (issued a step ago) has landed; step r + 2's may still be in flight
  // (the loop issues no other memory loads).
  auto copy_and_wait = [&](int r, int pbuf) {
    const bool copy = valid(r + 2);
    if (copy) stage(r + 2, pbuf);
    return copy;
  };
  auto wait_copies = [&](bool copy) {
    if (copy) wait_vmem_keep<kCopies>();
    else wait_vmem_all();
  };
  // Round r runs the dQ products of step r - 1 and the score-side products
  // of step r.  The wave's steps are r < n_live: the group's steps (blocks
  // 2 r + g up to the last visited one) and, under the causal mask (dense),
  // only those up to its last query's key block; the later blocks hold no
  // key it sees (P = dS = 0).  Round n_live runs the dQ products of step
  // n_live - 1 alone, the rounds after it only the copies, waits and
  // barriers every wave takes part in (skipping exact zeros: the result is
  // the same bit for bit).
  int lb = n_blk - 1;   // last visited block with a key the wave sees
  if constexpr (CAUSAL && !SPARSE) lb = min(lb, (qw0 + 31) / C::BLK);
  const int n_live = lb >= g ? (lb - g) / 2 + 1 : 0;
  int r = 0;
  for (; r < n_live; ++r) {
    const int pbuf = cb == 0 ? 2 : cb - 1, nbuf = cb == 2 ? 0 : cb + 1;   // (r - 1) % 3, (r + 1) % 3
    // Matrix phase: dQ^T of step r - 1; S^T and dP^T of step r.
    dq_matrix_phase<D>(dq_acc, dsw, st_acc, dpt, qbf, gbf, Kb(pbuf), Kb(cb), Vb(cb), rowx, trx0, trx1, st0, dpt0);
    __syncthreads();
    // Vector phase: the next copy, P^T = exp2(c2 S^T) and dS^T = P^T dP^T
    // of step r as fp16 pairs, the wait.
    const bool copy = copy_and_wait(r, pbuf);
    scores_to_ds(r);
    wait_copies(copy);
    __syncthreads();
    cb = nbuf;
  }
  if (r <= R) {
    const int pbuf = cb == 0 ? 2 : cb - 1, nbuf = cb == 2 ? 0 : cb + 1;
    if (n_live > 0)
      dq_matrix_phase<D, false>(dq_acc, dsw, st_acc, dpt, qbf, gbf, Kb(pbuf), Kb(cb), Vb(cb), rowx, trx0, trx1,
                                st0, dpt0);
    __syncthreads();
    wait_copies(copy_and_wait(r, pbuf));
    __syncthreads();
    cb = nbuf;
    ++r;
  }
  for (; r <= R; ++r) {
    const int pbuf = cb == 0 ? 2 : cb - 1, nbuf = cb == 2 ? 0 : cb + 1;
    __syncthreads();
    wait_copies(copy_and_wait(r, pbuf));
    __syncthreads();
    cb = nbuf;
  }
  if (g == 0) __syncthreads();

  // Close: the two groups' partial dQ^T are summed through LDS, group 0
  // finishing feature blocks 0 .. DM / 2 - 1 and group 1 the rest: each
  // writes its partial of the other's half (16 bytes per lane and
  // instruction, consecutive lanes on consecutive chunks), then adds the
  // other's partial of its own half and stores dQ = scale dQ^T in the
  // inputs' units as bf16 of this lane's query row.  red_at(c): chunk c
  // (accumulator registers 4 (c % 4) .. + 3 of feature block c / 4) of
  // query block qb.
  f32x4* red = (f32x4*)smem_raw;
  auto red_at = [&](int c) { return red + ((size_t)c * 4 + qb) * 64 + lane; };
  constexpr int kHalf = D / 16;   // chunks per half
  // (The branches on g keep every register index a constant.)
  auto put = [&](int c0) {
#pragma unroll
    for (int j = 0; j < kHalf; ++j) {
      const int c = c0 + j;
      *red_at(c) = (f32x4){dq_acc[c / 4][4 * (c % 4)], dq_acc[c / 4][4 * (c % 4) + 1], dq_acc[c / 4][4 * (c % 4) + 2],
                           dq_acc[c / 4][4 * (c % 4) + 3]};
    }
  };
  auto add_partner = [&](int c0) {
#pragma unroll
    for (int j = 0; j < kHalf; ++j) {
      const int c = c0 + j, dm = c / 4, r0 = 4 * (c % 4);
      const f32x4 b = *red_at(c);
#pragma unroll
      for (int e = 0; e < 4; ++e) dq_acc[dm][r0 + e] += b[e];
    }
  };
  if (g == 0) put(kHalf);
  else put(0);
  __syncthreads();
  if (g == 0) add_partner(0);
  else add_partner(kHalf);
  // Every partial is read before the LDS stages the finished rows: this
  // wave's half (D / 2 columns) of its 32 query rows, staged in its own
  // LDS and written as whole half rows.
  __syncthreads();
  {
    __bf16* stage = (__bf16*)smem_raw + wave * 32 * (D / 2);
    __bf16* out = dQ + (size_t)bh * N * D + g * (D / 2);
    if (g == 0) stage_rows<D, D / 2>(dq_acc, dq_fac, stage, lane, 0);
    else stage_rows<D, D / 2>(dq_acc, dq_fac, stage, lane, DM / 2);
    write_staged_rows<D / 2>(stage, out, D, qw0, N, lane);
  }
  // The closing sum's LDS is read by every wave before the next item's
  // copies overwrite it.
  if (wpx > 0) __syncthreads();
  }
}

// ---------------------------------------------------------------------------
// Launchers.
// ---------------------------------------------------------------------------
template <int D, bool CAUSAL, bool SPARSE>
static hipError_t launch_bwd_d(const BwdArgs& a) {
  using C = BwdCfg<D>;
  const int BH = a.B * a.H;
  const int nch = (a.N + kBwdChunkRows - 1) / kBwdChunkRows;
  hipError_t e = hipSuccess;
  // The sparse kernels keep their list of visited blocks (count first) after
  // the other buffers.
  const int list_bytes = SPARSE ? ((4 * ((a.N + C::BLK - 1) / C::BLK + 1) + 15) & ~15) : 0;
  const int lds = C::kLdsTotal + list_bytes;
  const int dq_lds = C::kDqLdsTotal + list_bytes;   // the list sits after the buffers
  const int num_tiles = (a.N + C::RES - 1) / C::RES;
  const _Float16* q16 = (const _Float16*)a.q16;
  const _Float16* k16 = (const _Float16*)a.k16;   // written by the dK/dV kernel
  const _Float16* v16 = (const _Float16*)a.v16;
  const _Float16* do16 = (const _Float16*)a.do16;
  if (a.phases & FA_BWD_PREPROCESS) {
    hipLaunchKernelGGL(fa_bwd_prep_kernel<D>, dim3((unsigned)(BH * nch)), dim3(kPrepThreads), 0, a.stream,
                       (const __bf16*)a.o, (const __bf16*)a.dout, (const __bf16*)a.q, (const __bf16*)a.k,
                       (const __bf16*)a.v, a.delta, a.part, (_Float16*)a.q16, (_Float16*)a.do16, a.N, nch);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    hipLaunchKernelGGL(fa_bwd_convert_kernel<D>, dim3((unsigned)(BH * nch)), dim3(256), 0, a.stream,
                       (const __bf16*)a.q, (const __bf16*)a.dout, a.lse, (const float*)a.delta,
                       (const float*)a.part, a.scales, a.rowterm, (_Float16*)a.q16, (_Float16*)a.do16, a.N, nch,
                       a.scale * kLog2e);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  if (a.phases & FA_BWD_MAIN) {
    auto kern = fa_bwd_dkdv_kernel<D, CAUSAL, SPARSE>;
    if ((e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, lds)) != hipSuccess)
      return e;
    // Persistent for dense masks; a block mask can give its tiles any mix of
    // costs (a global column's tile visits every query block), which the
    // fixed lists would not balance, so sparse launches keep one workgroup
    // per tile and the hardware's dispatch.
    int wpx = 0;
    if (!SPARSE && (e = persistent_width((const void*)kern, C::kThreads, lds, BH, num_tiles, &wpx)) != hipSuccess)
      return e;
    const int grid = wpx > 0 ? 8 * wpx : num_tiles * BH;
    hipLaunchKernelGGL(kern, dim3(grid), dim3(C::kThreads), lds, a.stream, q16, (const __bf16*)a.k,
                       (const __bf16*)a.v, do16, (_Float16*)a.k16, (_Float16*)a.v16,
                       (const float*)a.rowterm, (const float*)a.scales, (__bf16*)a.dk, (__bf16*)a.dv,
                       (const uint8_t*)a.bmask, a.N, BH, wpx, a.scale, a.scale * kLog2e);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  if (a.phases & FA_BWD_FINALIZE) {
    auto kern = fa_bwd_dq_kernel<D, CAUSAL, SPARSE>;
    if ((e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, dq_lds)) !=
        hipSuccess)
      return e;
    int wpx = 0;   // persistent for dense masks only, as above
    if (!SPARSE && (e = persistent_width((const void*)kern, C::kThreads, dq_lds, BH, num_tiles, &wpx)) != hipSuccess)
      return e;
    const int grid = wpx > 0 ? 8 * wpx : num_tiles * BH;
    hipLaunchKernelGGL(kern, dim3(grid), dim3(C::kThreads), dq_lds, a.stream, q16, k16, v16, do16,
                       (const float*)a.rowterm, (const float*)a.scales, (__bf16*)a.dq, (const uint8_t*)a.bmask,
                       a.N, BH, wpx, a.scale, a.scale * kLog2e);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  return e;
}

template <int D, bool SPARSE>
static hipError_t launch_bwd_c(const BwdArgs& a) {
  return a.causal ? launch_bwd_d<D, true, SPARSE>(a) : launch_bwd_d<D, false, SPARSE>(a);
}

hipError_t launch_bwd(const BwdArgs& a) {
  if (a.bmask) return a.d == 64 ? launch_bwd_c<64, true>(a) : launch_bwd_c<128, true>(a);
  return a.d == 64 ? launch_bwd_c<64, false>(a) : launch_bwd_c<128, false>(a);
}

}  // namespace fa
