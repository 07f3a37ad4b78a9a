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
// Three kernels on one stream:
//   1. bwd_prep: D_i = <dO_i, O_i> in fp32 from the bf16 O, and zero the fp32
//      dQ accumulator.
//   2. bwd_main: one workgroup of 4 waves per 128-key tile of one head.  Each
//      wave keeps its 32 keys' K and V rows in registers (the B operands of
//      S = Q K^T and dP = dO V^T, so each lane owns one key column of the
//      32x32 accumulators) and accumulates dK^T and dV^T for them in fp32.
//      The workgroup walks 64-row query tiles (Q, dO, LSE, D staged through
//      LDS, double buffered), two 32-row blocks per wave and step; dV^T += dO^T P and dK^T += Q^T dS take their
//      transposed A operands with ds_read_b64_tr_b16.  dS goes through LDS
//      once (as dS^T) so that dQ = dS K can be formed for the tile, and each
//      wave adds its 32 x 32 blocks of dQ to the fp32 accumulator with
//      hardware float atomics.  P and dS enter the dV, dK and dQ products as
//      two bf16 terms each (rounded value + residual): one bf16 term alone
//      leaves a relative error of up to 2^-9 per element, which at N = 4096
//      costs up to ~8e-3 absolute in the gradients.
//   3. bwd_dq_finalize: dQ = scale * accumulator, rounded to bf16.
#include <mutex>

#include "fa_common.h"
#include "fa_internal.h"

namespace fa {

// Device-resident scratch for flash_attn_bwd_noalloc: the backward's
// workspace (fp32 dQ accumulator and D) for callers that cannot allocate.
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
// 1. D_i = sum_c dO_ic O_ic; zero the dQ accumulator.
// ---------------------------------------------------------------------------
template <int D>
__global__ void __launch_bounds__(256)
fa_bwd_prep_kernel(const __bf16* __restrict__ O, const __bf16* __restrict__ dO, float* __restrict__ delta,
                   float* __restrict__ dq_acc, long rows) {
  constexpr int TPR = D / 8;          // threads per row, 8 elements each
  constexpr int RPB = 256 / TPR;      // rows per block
  const long row = (long)blockIdx.x * RPB + threadIdx.x / TPR;
  const int part = threadIdx.x % TPR;
  float acc = 0.f;
  if (row < rows) {
    const u32x4 o = *(const u32x4*)(O + row * D + part * 8);
    const u32x4 g = *(const u32x4*)(dO + row * D + part * 8);
#pragma unroll
    for (int i = 0; i < 4; ++i)
      acc += bf16_lo(o[i]) * bf16_lo(g[i]) + bf16_hi(o[i]) * bf16_hi(g[i]);
    float* z = dq_acc + row * D + part * 8;
    *(f32x4*)z = (f32x4){0.f, 0.f, 0.f, 0.f};
    *(f32x4*)(z + 4) = (f32x4){0.f, 0.f, 0.f, 0.f};
  }
#pragma unroll
  for (int off = TPR / 2; off > 0; off >>= 1) acc += __shfl_xor(acc, off);
  if (row < rows && part == 0) delta[row] = acc;
}

// ---------------------------------------------------------------------------
// 2. Main backward kernel.
// ---------------------------------------------------------------------------
template <int D>
struct BwdCfg {
  static constexpr int kWaves = 4;
  static constexpr int kThreads = 256;
  static constexpr int BN = 128;                 // keys per workgroup (32 per wave)
  static constexpr int BM = 64;                  // queries per step
  static constexpr int QB = BM / 32;             // 32-query blocks per step
  static constexpr int kRowPitch = D + 8;        // Q / dO tile rows in LDS
  static constexpr int kKtPitch = BN + 8;        // K^T rows in LDS
  static constexpr int kDsPitch = BM + 8;        // dS^T rows in LDS
  static constexpr int kTile = BM * kRowPitch;   // elements of one Q or dO tile
  // LDS layout (bytes): K^T | stage 0 (Q, dO, lse, delta) | stage 1 | dS^T hi | dS^T lo
  static constexpr int kKtBytes = D * kKtPitch * 2;
  static constexpr int kStageBytes = 2 * kTile * 2 + 2 * BM * 4;
  static constexpr int kDsBytes = 2 * BN * kDsPitch * 2;   // hi and lo terms
  static constexpr int kLdsBytes = kKtBytes + 2 * kStageBytes + kDsBytes;
  static constexpr int kChunks = BM * D / 8;     // 16-byte chunks per Q tile
  static constexpr int kChunksPerThread = kChunks / kThreads;
  // dQ blocks (32 queries x 32 features) per step, shared out over the waves.
  static constexpr int kDqBlocks = QB * (D / 32);
  static constexpr int kDqPerWave = kDqBlocks / kWaves;
  static_assert(kChunks % kThreads == 0, "tile staging");
  static_assert(kDqBlocks % kWaves == 0, "dQ work split");
  static_assert(kThreads == 256, "kernel launch bounds assume 256 threads");
  static_assert(kLdsBytes <= 160 * 1024, "LDS budget");
};

template <int D>
struct BwdStage {
  u32x4 q[BwdCfg<D>::kChunksPerThread];
  u32x4 g[BwdCfg<D>::kChunksPerThread];
  float lse;    // LSE of one row as loaded (threads 0..BM-1), +inf past N
  float dlt;    // D for one row (threads BM..2BM-1)
};

// Per-head buffer descriptors: rows past N read as zero; dQ atomics past N
// are dropped.
struct BwdHead {
  __amdgpu_buffer_rsrc_t q, k, v, g, lse, dlt, dq;
};

template <int D>
__device__ __forceinline__ void bwd_load_stage(BwdStage<D>& st, const BwdHead& h, int q0, int N, int tid) {
  using C = BwdCfg<D>;
#pragma unroll
  for (int i = 0; i < C::kChunksPerThread; ++i) {
    const int c = tid + i * C::kThreads;
    const int row = c / (D / 8), col = (c % (D / 8)) * 8;
    const uint32_t off = (uint32_t)((q0 + row) * D + col) * 2u;
    st.q[i] = bload128(h.q, off);
    st.g[i] = bload128(h.g, off);
  }
  // LSE (+inf past N) and D (0 past N), kept as loaded: nothing here
  // waits for the loads, which complete behind the step's computation and
  // are first used in bwd_store_stage.
  if (tid < C::BM) {
    const int q = q0 + tid;
    st.lse = q < N ? bload32f(h.lse, (uint32_t)q * 4u) : INFINITY;
  } else if (tid < 2 * C::BM) {
    st.dlt = bload32f(h.dlt, (uint32_t)(q0 + tid - C::BM) * 4u);
  }
}

template <int D>
__device__ __forceinline__ void bwd_store_stage(const BwdStage<D>& st, char* stage, int tid) {
  using C = BwdCfg<D>;
  __bf16* Qs = (__bf16*)stage;
  __bf16* Gs = Qs + C::kTile;
  float* Ls = (float*)(Gs + C::kTile);
  float* Ds = Ls + C::BM;
#pragma unroll
  for (int i = 0; i < C::kChunksPerThread; ++i) {
    const int c = tid + i * C::kThreads;
    const int row = c / (D / 8), col = (c % (D / 8)) * 8;
    *(u32x4*)(Qs + row * C::kRowPitch + col) = st.q[i];
    *(u32x4*)(Gs + row * C::kRowPitch + col) = st.g[i];
  }
  // LSE * log2(e); rows that saw no key at all (LSE = -inf) get +inf, so
  // P = 0 there.
  if (tid < C::BM) Ls[tid] = st.lse == -INFINITY ? INFINITY : st.lse * kLog2e;
  else if (tid < 2 * C::BM) Ds[tid - C::BM] = st.dlt;
}

// SPARSE: block-sparse attention.  bmask holds, per head, an nb x nb byte
// matrix over (128-query block, 128-key block) pairs (a workgroup's keys are
// one key block); the workgroup visits only the 64-query steps whose query
// block its mask column keeps, from a list built in LDS.
template <int D, bool CAUSAL, bool SPARSE>
__global__ void __launch_bounds__(256)
fa_bwd_main_kernel(const __bf16* __restrict__ Q, const __bf16* __restrict__ K, const __bf16* __restrict__ V,
                   const __bf16* __restrict__ dO, const float* __restrict__ LSE, const float* __restrict__ delta,
                   float* __restrict__ dq_acc, __bf16* __restrict__ dK, __bf16* __restrict__ dV,
                   const uint8_t* __restrict__ bmask, int N, int BH, float scale, float scale_log2) {
  using C = BwdCfg<D>;
  static_assert(C::BN == FA_SPARSE_BLOCK && FA_SPARSE_BLOCK % C::BM == 0, "sparse blocks vs tiles");
  constexpr int QB = C::QB;
  extern __shared__ __attribute__((aligned(16))) char smem_raw[];
  __bf16* Kt = (__bf16*)smem_raw;                                  // [D][kKtPitch]
  char* stages = smem_raw + C::kKtBytes;
  __bf16* dSt = (__bf16*)(stages + 2 * C::kStageBytes);            // [BN][kDsPitch], hi term
  __bf16* dSt_lo = dSt + C::BN * C::kDsPitch;                      // lo term

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);       // uniform per wave
  const int lane = tid & 63;
  const int lc = lane & 31, lg = lane >> 5;
  int kt, bh;   // key tile (small kt = most query tiles) and head
  xcd_head_major(blockIdx.x, BH, (N + C::BN - 1) / C::BN, bh, kt);
  const size_t head_off = (size_t)bh * N * D;
  const uint32_t head_bytes = (uint32_t)N * D * 2u;
  BwdHead h;
  h.q = make_rsrc(Q + head_off, head_bytes);
  h.k = make_rsrc(K + head_off, head_bytes);
  h.v = make_rsrc(V + head_off, head_bytes);
  h.g = make_rsrc(dO + head_off, head_bytes);
  h.lse = make_rsrc(LSE + (size_t)bh * N, (uint32_t)N * 4u);
  h.dlt = make_rsrc(delta + (size_t)bh * N, (uint32_t)N * 4u);
  h.dq = make_rsrc(dq_acc + head_off, head_bytes * 2u);

  const int k0 = kt * C::BN;                  // first key of the workgroup
  const int kw0 = k0 + wave * 32;             // first key of this wave
  const int key = kw0 + lc;                   // this lane's key column
  const bool key_ok = key < N;
  // Lane parts of the LDS offsets (the rest are compile-time constants).
  const int row_lane_off = lc * C::kRowPitch + 8 * lg;          // Q / dO rows as A operands
  const int tr_off_p = tr_lane_off(lane, C::kRowPitch, 4);      // Q^T / dO^T, accumulator key order
  const int tr_off_n = tr_lane_off(lane, C::kDsPitch, 8);       // dS from dS^T, natural key order
  const int kt_lane_off = lc * C::kKtPitch + 8 * lg;            // K (from K^T) as B operand

  // K and V rows of this lane's key as B operands (k = feature).
  bf16x8 kb[D / 16], vb[D / 16];
#pragma unroll
  for (int ks = 0; ks < D / 16; ++ks) {
    const uint32_t off = (uint32_t)(key * D + 16 * ks + 8 * lg) * 2u;
    kb[ks] = __builtin_bit_cast(bf16x8, bload128(h.k, off));
    vb[ks] = __builtin_bit_cast(bf16x8, bload128(h.v, off));
  }
  // K^T of the workgroup's keys in LDS for dQ = dS K.
  for (int e = tid; e < C::BN * (D / 4); e += C::kThreads) {
    const int r = e / (D / 4), c4 = (e % (D / 4)) * 4;
    const u32x2 val = bload64(h.k, (uint32_t)((k0 + r) * D + c4) * 2u);
    __bf16 tmp[4];
    *(u32x2*)tmp = val;
#pragma unroll
    for (int j = 0; j < 4; ++j) Kt[(c4 + j) * C::kKtPitch + r] = tmp[j];
  }

  f32x16 dk_acc[D / 32], dv_acc[D / 32];
#pragma unroll
  for (int i = 0; i < D / 32; ++i) {
    dk_acc[i] = (f32x16){};
    dv_acc[i] = (f32x16){};
  }

  // Query steps (BM queries each) that can see these keys: qt_begin.. all
  // of them (dense), or the ones the mask column keeps, listed in LDS after
  // the other buffers (count first).
  const int qt_begin = CAUSAL ? k0 / C::BM : 0;
  int n_steps = (N + C::BM - 1) / C::BM - qt_begin;
  int* slist = (int*)(smem_raw + C::kLdsBytes);
  if constexpr (SPARSE) {
    const int nb = (N + FA_SPARSE_BLOCK - 1) / FA_SPARSE_BLOCK;
    const uint8_t* col = bmask + (size_t)bh * nb * nb + kt;   // entry of query block i at col[i * nb]
    if (wave == 0) {
      int cnt = 0;
      for (int base = 0; base < n_steps; base += 64) {
        const int qs = qt_begin + base + lane;
        const bool live = base + lane < n_steps && col[(size_t)(qs * C::BM / FA_SPARSE_BLOCK) * nb] != 0;
        const uint64_t bal = __ballot(live);
        const int pos = cnt + __builtin_amdgcn_mbcnt_hi((uint32_t)(bal >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)bal, 0));
        if (live) slist[1 + pos] = qs;
        cnt += __popcll(bal);
      }
      if (lane == 0) slist[0] = cnt;
    }
    __syncthreads();
    n_steps = __builtin_amdgcn_readfirstlane(slist[0]);
  }
  auto step_at = [&](int j) { return SPARSE ? slist[1 + j] : qt_begin + j; };
  // dQ partials of the previous step, added to the accumulator with atomics
  // spread over the next step's matrix and vector work (four at a time) so
  // that their issue overlaps computation instead of stalling the wave.
  f32x16 dq_pend[C::kDqPerWave];
  int q0_pend = -1;
  int qbk[C::kDqPerWave], dmk[C::kDqPerWave];
#pragma unroll
  for (int j = 0; j < C::kDqPerWave; ++j) {
    const int blk = wave * C::kDqPerWave + j;
    qbk[j] = blk / (D / 32);
    dmk[j] = blk % (D / 32);
  }
  constexpr int kPendParts = 8;
  constexpr int kPendPerPart = C::kDqPerWave * 16 / kPendParts;
  static_assert(C::kDqPerWave * 16 % kPendParts == 0, "atomic spreading");
  auto flush_pending = [&](int part) {
    if (q0_pend >= 0) {
#pragma unroll
      for (int t = 0; t < kPendPerPart; ++t) {
        const int idx = part * kPendPerPart + t, j = idx / 16, r = idx % 16;
        const int q = q0_pend + 32 * qbk[j] + 8 * (r >> 2) + 4 * lg + (r & 3);
        batomic_add(h.dq, (uint32_t)(q * D + 32 * dmk[j] + lc) * 4u, dq_pend[j][r]);
      }
    }
  };
  BwdStage<D> st;
  if (n_steps > 0) {
    bwd_load_stage<D>(st, h, step_at(0) * C::BM, N, tid);
    bwd_store_stage<D>(st, stages, tid);
  }

  for (int it = 0; it < n_steps; ++it) {
    const int q0 = step_at(it) * C::BM;
    const bool more = it + 1 < n_steps;
    if (more) bwd_load_stage<D>(st, h, step_at(it + 1) * C::BM, N, tid);
    __syncthreads();   // stage `it` visible; previous dS^T reads finished
    char* stage = stages + (it & 1) * C::kStageBytes;
    const __bf16* Qs = (const __bf16*)stage;
    const __bf16* Gs = Qs + C::kTile;
    const float* Ls = (const float*)(Gs + C::kTile);
    const float* Ds = Ls + C::BM;

    // Two 32-query blocks per step.  For block b:
    //   S = Q K^T and dP = dO V^T (32 queries x this wave's 32 keys);
    //   P = exp2(s * scale * log2 e - LSE * log2 e), dS = P (dP - D), each
    //   kept as a bf16 pair (rounded value, rounded residual), with causal
    //   masking (key > query) and keys past N giving P = 0 (scores set to
    //   -inf, on the steps that need it); dS^T to LDS;
    //   dV^T += dO^T P and dK^T += Q^T dS, the A operands read down the
    //   columns in the key order P's accumulator layout leaves in each lane.
    // With one wave per SIMD, the matrix and vector work of the two blocks
    // are interleaved by hand: block 1's score MFMAs run in four chunks,
    // each beside a quarter of block 0's vector work, and block 0's dV/dK
    // MFMAs beside block 1's vector work; scheduling barriers keep the
    // chunks in order.
    static_assert(QB == 2, "the step interleaves exactly two query blocks");
    // Masking is needed only where this wave's keys run past N or (causal)
    // past the step's first query; elsewhere every P is kept.
    const bool step_mask = (kw0 + 31 >= N) || (CAUSAL && q0 < kw0 + 31);
    const __bf16* qrow = Qs + row_lane_off;
    const __bf16* grow = Gs + row_lane_off;
    const __bf16* gtr = Gs + tr_off_p;
    const __bf16* qtr = Qs + tr_off_p;
    constexpr int KS = D / 16;                 // k-steps of the score products
    constexpr int KSC = (KS + 3) / 4;          // k-steps per chunk
    constexpr int DM = D / 32;
    constexpr int UPC = (2 * DM + 3) / 4;      // (c, dm) dV/dK pairs per chunk

    f32x16 sc[QB], dpc[QB];
    // Scores of masked (key, query) pairs to -inf, so P and dS are 0 there.
    auto mask_scores = [&](int b) {
      if (step_mask) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int q = q0 + 32 * b + 8 * (r >> 2) + 4 * lg + (r & 3);
          const bool keep = key_ok & (!CAUSAL | (q >= key));
          sc[b][r] = keep ? sc[b][r] : -INFINITY;
        }
      }
    };
    auto score_steps = [&](int b, int ks0, int ks1) {
#pragma unroll
      for (int ks = ks0; ks < ks1; ++ks) {
        const int off = 32 * b * C::kRowPitch + 16 * ks;
        const bf16x8 qa = *(const bf16x8*)(qrow + off);
        const bf16x8 ga = *(const bf16x8*)(grow + off);
        sc[b] = mfma32(qa, kb[ks], sc[b]);
        dpc[b] = mfma32(ga, vb[ks], dpc[b]);
      }
    };
    uint32_t pw[QB][8], pl[QB][8], dsw[QB][8], dsl[QB][8];
    auto vector_group = [&](int b, int i) {
      const f32x4 l4 = *(const f32x4*)(Ls + 32 * b + 8 * i + 4 * lg);
      const f32x4 d4 = *(const f32x4*)(Ds + 32 * b + 8 * i + 4 * lg);
      float p[4], ds[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int r = 4 * i + j;
        const float pe = fast_exp2(__builtin_fmaf(sc[b][r], scale_log2, -l4[j]));
        const float pv = pe;
        p[j] = pv;
        ds[j] = pv * (dpc[b][r] - d4[j]);
      }
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        const uint32_t ph = pack_bf16x2(p[2 * hh], p[2 * hh + 1]);
        const uint32_t dh = pack_bf16x2(ds[2 * hh], ds[2 * hh + 1]);
        pw[b][2 * i + hh] = ph;
        pl[b][2 * i + hh] = pack_bf16x2(p[2 * hh] - bf16_lo(ph), p[2 * hh + 1] - bf16_hi(ph));
        dsw[b][2 * i + hh] = dh;
        dsl[b][2 * i + hh] = pack_bf16x2(ds[2 * hh] - bf16_lo(dh), ds[2 * hh + 1] - bf16_hi(dh));
      }
      // dS^T[key][q .. q+3] (both terms) for the dQ product.
      const int off = (wave * 32 + lc) * C::kDsPitch + 32 * b + 8 * i + 4 * lg;
      *(u32x2*)(dSt + off) = (u32x2){dsw[b][2 * i], dsw[b][2 * i + 1]};
      *(u32x2*)(dSt_lo + off) = (u32x2){dsl[b][2 * i], dsl[b][2 * i + 1]};
    };
    auto operand = [&](const uint32_t (&w)[8], int c) {
      return __builtin_bit_cast(bf16x8, ((u32x4){w[4 * c], w[4 * c + 1], w[4 * c + 2], w[4 * c + 3]}));
    };
    auto update_pairs = [&](int b, int u0, int u1) {
#pragma unroll
      for (int u = u0; u < u1; ++u) {
        const int c = u / DM, dm = u % DM;
        const int r0 = 32 * b + 16 * c;
        const int lo = r0 * C::kRowPitch + 32 * dm, hi = (r0 + 8) * C::kRowPitch + 32 * dm;
        const bf16x8 ga = lds_tr_pair(gtr, lo, hi);
        const bf16x8 qa = lds_tr_pair(qtr, lo, hi);
        dv_acc[dm] = mfma32(ga, operand(pw[b], c), dv_acc[dm]);
        dk_acc[dm] = mfma32(qa, operand(dsw[b], c), dk_acc[dm]);
        dv_acc[dm] = mfma32(ga, operand(pl[b], c), dv_acc[dm]);
        dk_acc[dm] = mfma32(qa, operand(dsl[b], c), dk_acc[dm]);
      }
    };

#pragma unroll
    for (int b = 0; b < QB; ++b) {
      sc[b] = (f32x16){};
      dpc[b] = (f32x16){};
    }
    score_steps(0, 0, KS);
    mask_scores(0);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      score_steps(1, min(KS, j * KSC), min(KS, (j + 1) * KSC));
      vector_group(0, j);
      flush_pending(j);
      __builtin_amdgcn_sched_barrier(0);
    }
    mask_scores(1);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      update_pairs(0, min(2 * DM, j * UPC), min(2 * DM, (j + 1) * UPC));
      vector_group(1, j);
      flush_pending(4 + j);
      __builtin_amdgcn_sched_barrier(0);
    }
    update_pairs(1, 0, 2 * DM);
    if (more) bwd_store_stage<D>(st, stages + ((it + 1) & 1) * C::kStageBytes, tid);
    __syncthreads();   // dS^T complete

    // dQ (BM x D) for this query tile from the workgroup's 128 keys: the
    // (query block, feature block) pairs are dealt out to the waves, each
    // summing over all keys; independent blocks of a wave interleave.
    {
      f32x16 acc[C::kDqPerWave];
#pragma unroll
      for (int j = 0; j < C::kDqPerWave; ++j) acc[j] = (f32x16){};
      const __bf16* dsp = dSt + tr_off_n;
      const __bf16* dslp = dSt_lo + tr_off_n;
      const __bf16* ktp = Kt + kt_lane_off;
#pragma unroll
      for (int ks = 0; ks < C::BN / 16; ++ks) {
        const int kk = 16 * ks;
#pragma unroll
        for (int j = 0; j < C::kDqPerWave; ++j) {
          const int lo = kk * C::kDsPitch + 32 * qbk[j], hi = (kk + 4) * C::kDsPitch + 32 * qbk[j];
          const bf16x8 a = lds_tr_pair(dsp, lo, hi);
          const bf16x8 al = lds_tr_pair(dslp, lo, hi);
          const bf16x8 b = *(const bf16x8*)(ktp + 32 * dmk[j] * C::kKtPitch + kk);
          acc[j] = mfma32(a, b, acc[j]);
          acc[j] = mfma32(al, b, acc[j]);
        }
      }
#pragma unroll
      for (int j = 0; j < C::kDqPerWave; ++j) dq_pend[j] = acc[j];
      q0_pend = q0;
    }
  }
#pragma unroll
  for (int part = 0; part < kPendParts; ++part) flush_pending(part);

  // dK = scale dK^T, dV = dV^T, stored as bf16 rows of this lane's key.
  if (key < N) {
    __bf16* dkr = dK + head_off + (size_t)key * D;
    __bf16* dvr = dV + head_off + (size_t)key * D;
#pragma unroll
    for (int dm = 0; dm < D / 32; ++dm)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        u32x2 wk = {pack_bf16x2(dk_acc[dm][4 * i] * scale, dk_acc[dm][4 * i + 1] * scale),
                    pack_bf16x2(dk_acc[dm][4 * i + 2] * scale, dk_acc[dm][4 * i + 3] * scale)};
        u32x2 wv = {pack_bf16x2(dv_acc[dm][4 * i], dv_acc[dm][4 * i + 1]),
                    pack_bf16x2(dv_acc[dm][4 * i + 2], dv_acc[dm][4 * i + 3])};
        *(u32x2*)(dkr + 32 * dm + 8 * i + 4 * lg) = wk;
        *(u32x2*)(dvr + 32 * dm + 8 * i + 4 * lg) = wv;
      }
  }
}

// ---------------------------------------------------------------------------
// 3. dQ = scale * accumulator -> bf16.
// ---------------------------------------------------------------------------
__global__ void __launch_bounds__(256)
fa_bwd_dq_finalize_kernel(const float* __restrict__ acc, __bf16* __restrict__ dq, long n8, float scale) {
  const long i = (long)blockIdx.x * 256 + threadIdx.x;
  if (i >= n8) return;
  const f32x4 a = *(const f32x4*)(acc + 8 * i);
  const f32x4 b = *(const f32x4*)(acc + 8 * i + 4);
  u32x4 w = {pack_bf16x2(a[0] * scale, a[1] * scale), pack_bf16x2(a[2] * scale, a[3] * scale),
             pack_bf16x2(b[0] * scale, b[1] * scale), pack_bf16x2(b[2] * scale, b[3] * scale)};
  *(u32x4*)(dq + 8 * i) = w;
}

template <int D, bool CAUSAL, bool SPARSE>
static hipError_t launch_bwd_d(const BwdArgs& a) {
  using C = BwdCfg<D>;
  const int BH = a.B * a.H;
  const long rows = (long)BH * a.N;
  hipError_t e = hipSuccess;
  if (a.phases & FA_BWD_PREPROCESS) {
    constexpr int RPB = 256 / (D / 8);
    hipLaunchKernelGGL(fa_bwd_prep_kernel<D>, dim3((unsigned)((rows + RPB - 1) / RPB)), dim3(256), 0, a.stream,
                       (const __bf16*)a.o, (const __bf16*)a.dout, a.delta, a.dq_acc, rows);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  if (a.phases & FA_BWD_MAIN) {
    auto kern = fa_bwd_main_kernel<D, CAUSAL, SPARSE>;
    // The sparse kernel keeps its list of visited query steps (count first)
    // after the other buffers.
    const int list_bytes = SPARSE ? ((4 * ((a.N + C::BM - 1) / C::BM + 1) + 15) & ~15) : 0;
    const int lds = C::kLdsBytes + list_bytes;
    if ((e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, lds)) != hipSuccess)
      return e;
    const int num_kt = (a.N + C::BN - 1) / C::BN;
    hipLaunchKernelGGL(kern, dim3(num_kt * BH), dim3(C::kThreads), lds, a.stream, (const __bf16*)a.q,
                       (const __bf16*)a.k, (const __bf16*)a.v, (const __bf16*)a.dout, a.lse, a.delta, a.dq_acc,
                       (__bf16*)a.dk, (__bf16*)a.dv, (const uint8_t*)a.bmask, a.N, BH, a.scale,
                       a.scale * kLog2e);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  if (a.phases & FA_BWD_FINALIZE) {
    const long n8 = rows * D / 8;
    hipLaunchKernelGGL(fa_bwd_dq_finalize_kernel, dim3((unsigned)((n8 + 255) / 256)), dim3(256), 0, a.stream,
                       a.dq_acc, (__bf16*)a.dq, n8, a.scale);
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
