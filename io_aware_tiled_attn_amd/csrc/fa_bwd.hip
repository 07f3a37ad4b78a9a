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
//      The workgroup walks 32-row query tiles (Q, dO, LSE, D staged through
//      LDS, double buffered); dV^T += dO^T P and dK^T += Q^T dS take their
//      transposed A operands with ds_read_b64_tr_b16.  dS goes through LDS
//      once (as dS^T) so that dQ = dS K can be formed for the tile, and each
//      wave adds its 32 x 32 block of dQ to the fp32 accumulator with
//      hardware float atomics.  P and dS enter the dV, dK and dQ products as
//      two bf16 terms each (rounded value + residual): one bf16 term alone
//      leaves a relative error of up to 2^-9 per element, which at N = 4096
//      costs up to ~8e-3 absolute in the gradients.
//   3. bwd_dq_finalize: dQ = scale * accumulator, rounded to bf16.
#include "fa_common.h"
#include "fa_internal.h"

namespace fa {

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

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
  static constexpr int BN = 128;                 // keys per workgroup
  static constexpr int BM = 32;                  // queries per step
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
  static_assert(kChunks % kThreads == 0, "tile staging");
  static_assert(kThreads == 256, "kernel launch bounds assume 256 threads");
};

// 8 bf16 taken down the rows of a row-major LDS matrix: lane l receives
// M[r_lo + 0..3][col0 + l % 32] as slots 0..3 and M[r_hi + 0..3][col0 + l % 32]
// as slots 4..7 (r_lo, r_hi may differ between the two lane halves).
// ds_read_b64_tr_b16 hands lane j of each 16-lane group element j % 4 of the
// 8-byte word read by lane 4 e + j / 4 of that group, for e = 0..3; so lane s
// of the group reads row (s / 4) at column 4 (s % 4) of its 4 x 16 block.
__device__ __forceinline__ bf16x8 lds_read_down(const __bf16* M, int pitch, int col0, int r_lo, int r_hi,
                                                int lane) {
  const int s = lane & 15, G = lane >> 4;
  const int col = col0 + 16 * (G & 1) + 4 * (s & 3);
  const __bf16* p0 = M + (r_lo + (s >> 2)) * pitch + col;
  const __bf16* p1 = M + (r_hi + (s >> 2)) * pitch + col;
  s16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)p0);
  s16x4 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)p1);
  typedef short s16x8 __attribute__((ext_vector_type(8)));
  s16x8 r = {a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
  return __builtin_bit_cast(bf16x8, r);
}

template <int D>
struct BwdStage {
  u32x4 q[BwdCfg<D>::kChunksPerThread];
  u32x4 g[BwdCfg<D>::kChunksPerThread];
  float lse2;   // LSE * log2(e) for one row (threads 0..BM-1), +inf past N
  float dlt;    // D for one row (threads BM..2BM-1)
};

template <int D>
__device__ __forceinline__ void bwd_load_stage(BwdStage<D>& st, const __bf16* Qh, const __bf16* dOh,
                                               const float* lse_h, const float* dlt_h, int q0, int N, int tid) {
  using C = BwdCfg<D>;
#pragma unroll
  for (int i = 0; i < C::kChunksPerThread; ++i) {
    const int c = tid + i * C::kThreads;
    const int row = c / (D / 8), col = (c % (D / 8)) * 8;
    const int q = q0 + row;
    u32x4 a = {0u, 0u, 0u, 0u}, b = {0u, 0u, 0u, 0u};
    if (q < N) {
      a = *(const u32x4*)(Qh + (size_t)q * D + col);
      b = *(const u32x4*)(dOh + (size_t)q * D + col);
    }
    st.q[i] = a;
    st.g[i] = b;
  }
  if (tid < C::BM) {
    const int q = q0 + tid;
    st.lse2 = q < N ? lse_h[q] * kLog2e : INFINITY;
  } else if (tid < 2 * C::BM) {
    const int q = q0 + tid - C::BM;
    st.dlt = q < N ? dlt_h[q] : 0.f;
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
  if (tid < C::BM) Ls[tid] = st.lse2;
  else if (tid < 2 * C::BM) Ds[tid - C::BM] = st.dlt;
}

template <int D, bool CAUSAL>
__global__ void __launch_bounds__(256)
fa_bwd_main_kernel(const __bf16* __restrict__ Q, const __bf16* __restrict__ K, const __bf16* __restrict__ V,
                   const __bf16* __restrict__ dO, const float* __restrict__ LSE, const float* __restrict__ delta,
                   float* __restrict__ dq_acc, __bf16* __restrict__ dK, __bf16* __restrict__ dV, int N, int BH,
                   float scale, float scale_log2) {
  using C = BwdCfg<D>;
  extern __shared__ __attribute__((aligned(16))) char smem_raw[];
  __bf16* Kt = (__bf16*)smem_raw;                                  // [D][kKtPitch]
  char* stages = smem_raw + C::kKtBytes;
  __bf16* dSt = (__bf16*)(stages + 2 * C::kStageBytes);            // [BN][kDsPitch], hi term
  __bf16* dSt_lo = dSt + C::BN * C::kDsPitch;                      // lo term

  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int lc = lane & 31, lg = lane >> 5;
  const int kt = blockIdx.x / BH;       // key tile; small kt = most query tiles
  const int bh = blockIdx.x % BH;
  const size_t head_off = (size_t)bh * N * D;
  const __bf16* Qh = Q + head_off;
  const __bf16* Kh = K + head_off;
  const __bf16* Vh = V + head_off;
  const __bf16* dOh = dO + head_off;
  const float* lse_h = LSE + (size_t)bh * N;
  const float* dlt_h = delta + (size_t)bh * N;
  float* dqh = dq_acc + head_off;

  const int k0 = kt * C::BN;                  // first key of the workgroup
  const int key = k0 + wave * 32 + lc;        // this lane's key column

  // K and V rows of this lane's key as B operands (k = feature).
  bf16x8 kb[D / 16], vb[D / 16];
#pragma unroll
  for (int ks = 0; ks < D / 16; ++ks) {
    u32x4 a = {0u, 0u, 0u, 0u}, b = {0u, 0u, 0u, 0u};
    if (key < N) {
      a = *(const u32x4*)(Kh + (size_t)key * D + 16 * ks + 8 * lg);
      b = *(const u32x4*)(Vh + (size_t)key * D + 16 * ks + 8 * lg);
    }
    kb[ks] = __builtin_bit_cast(bf16x8, a);
    vb[ks] = __builtin_bit_cast(bf16x8, b);
  }
  // K^T of the workgroup's keys in LDS for dQ = dS K.
  for (int e = tid; e < C::BN * (D / 4); e += C::kThreads) {
    const int r = e / (D / 4), c4 = (e % (D / 4)) * 4;
    const int kk = k0 + r;
    u32x2 val = {0u, 0u};
    if (kk < N) val = *(const u32x2*)(Kh + (size_t)kk * D + c4);
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

  // Query tiles that can see these keys.
  const int qt_begin = CAUSAL ? k0 / C::BM : 0;
  const int qt_end = (N + C::BM - 1) / C::BM;
  BwdStage<D> st;
  if (qt_begin < qt_end) {
    bwd_load_stage<D>(st, Qh, dOh, lse_h, dlt_h, qt_begin * C::BM, N, tid);
    bwd_store_stage<D>(st, stages, tid);
  }

  for (int qt = qt_begin; qt < qt_end; ++qt) {
    const int it = qt - qt_begin;
    const int q0 = qt * C::BM;
    if (qt + 1 < qt_end) bwd_load_stage<D>(st, Qh, dOh, lse_h, dlt_h, q0 + C::BM, N, tid);
    __syncthreads();   // stage `it` visible; previous dS^T reads finished
    char* stage = stages + (it & 1) * C::kStageBytes;
    const __bf16* Qs = (const __bf16*)stage;
    const __bf16* Gs = Qs + C::kTile;
    const float* Ls = (const float*)(Gs + C::kTile);
    const float* Ds = Ls + C::BM;

    // S = Q K^T and dP = dO V^T: 32 queries x this wave's 32 keys.
    f32x16 s = (f32x16){}, dp = (f32x16){};
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) {
      const bf16x8 qa = *(const bf16x8*)(Qs + lc * C::kRowPitch + 16 * ks + 8 * lg);
      const bf16x8 ga = *(const bf16x8*)(Gs + lc * C::kRowPitch + 16 * ks + 8 * lg);
      s = mfma32(qa, kb[ks], s);
      dp = mfma32(ga, vb[ks], dp);
    }
    // P = exp2(s * scale * log2 e - LSE * log2 e); dS = P (dP - D).  Each is
    // kept as a bf16 pair (rounded value, rounded residual).
    const bool diag = CAUSAL && (q0 < k0 + wave * 32 + 31);
    uint32_t pw[8], pl[8], dsw[8], dsl[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const f32x4 l4 = *(const f32x4*)(Ls + 8 * i + 4 * lg);
      const f32x4 d4 = *(const f32x4*)(Ds + 8 * i + 4 * lg);
      float p[4], ds[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int r = 4 * i + j;
        float pv = fast_exp2(__builtin_fmaf(s[r], scale_log2, -l4[j]));
        const int q = q0 + 8 * i + 4 * lg + j;
        if ((diag && key > q) || key >= N) pv = 0.f;
        p[j] = pv;
        ds[j] = pv * (dp[r] - d4[j]);
      }
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const uint32_t ph = pack_bf16x2(p[2 * h], p[2 * h + 1]);
        const uint32_t dh = pack_bf16x2(ds[2 * h], ds[2 * h + 1]);
        pw[2 * i + h] = ph;
        pl[2 * i + h] = pack_bf16x2(p[2 * h] - bf16_lo(ph), p[2 * h + 1] - bf16_hi(ph));
        dsw[2 * i + h] = dh;
        dsl[2 * i + h] = pack_bf16x2(ds[2 * h] - bf16_lo(dh), ds[2 * h + 1] - bf16_hi(dh));
      }
      // dS^T[key][q .. q+3] (both terms) for the dQ product.
      const int off = (wave * 32 + lc) * C::kDsPitch + 8 * i + 4 * lg;
      *(u32x2*)(dSt + off) = (u32x2){dsw[2 * i], dsw[2 * i + 1]};
      *(u32x2*)(dSt_lo + off) = (u32x2){dsl[2 * i], dsl[2 * i + 1]};
    }
    // B operands (k = query, in the accumulator's lane order).
    bf16x8 pB[2], pBl[2], dsB[2], dsBl[2];
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      pB[c] = __builtin_bit_cast(bf16x8, ((u32x4){pw[4 * c], pw[4 * c + 1], pw[4 * c + 2], pw[4 * c + 3]}));
      pBl[c] = __builtin_bit_cast(bf16x8, ((u32x4){pl[4 * c], pl[4 * c + 1], pl[4 * c + 2], pl[4 * c + 3]}));
      dsB[c] = __builtin_bit_cast(bf16x8, ((u32x4){dsw[4 * c], dsw[4 * c + 1], dsw[4 * c + 2], dsw[4 * c + 3]}));
      dsBl[c] = __builtin_bit_cast(bf16x8, ((u32x4){dsl[4 * c], dsl[4 * c + 1], dsl[4 * c + 2], dsl[4 * c + 3]}));
    }
    // dV^T += dO^T P and dK^T += Q^T dS (A operands read down the columns).
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      const int r_lo = 16 * c + 4 * lg, r_hi = 16 * c + 8 + 4 * lg;
#pragma unroll
      for (int dm = 0; dm < D / 32; ++dm) {
        const bf16x8 ga = lds_read_down(Gs, C::kRowPitch, 32 * dm, r_lo, r_hi, lane);
        const bf16x8 qa = lds_read_down(Qs, C::kRowPitch, 32 * dm, r_lo, r_hi, lane);
        dv_acc[dm] = mfma32(ga, pB[c], dv_acc[dm]);
        dv_acc[dm] = mfma32(ga, pBl[c], dv_acc[dm]);
        dk_acc[dm] = mfma32(qa, dsB[c], dk_acc[dm]);
        dk_acc[dm] = mfma32(qa, dsBl[c], dk_acc[dm]);
      }
    }
    if (qt + 1 < qt_end) bwd_store_stage<D>(st, stages + ((it + 1) & 1) * C::kStageBytes, tid);
    __syncthreads();   // dS^T complete

    // dQ(32 x D) for this query tile from the workgroup's 128 keys.  D = 128:
    // wave w forms feature block w over all keys; D = 64: feature block
    // w % 2 over key half w / 2.
    {
      constexpr int kBlocks = D / 32;
      constexpr int kSplit = C::kWaves / kBlocks;           // key groups
      constexpr int kSteps = C::BN / 16 / kSplit;
      const int dm = wave % kBlocks;
      const int kgrp = wave / kBlocks;
      f32x16 acc = (f32x16){};
#pragma unroll
      for (int j = 0; j < kSteps; ++j) {
        const int kk = (kgrp * kSteps + j) * 16;
        const bf16x8 a = lds_read_down(dSt, C::kDsPitch, 0, kk + 8 * lg, kk + 8 * lg + 4, lane);
        const bf16x8 al = lds_read_down(dSt_lo, C::kDsPitch, 0, kk + 8 * lg, kk + 8 * lg + 4, lane);
        const bf16x8 b = *(const bf16x8*)(Kt + (32 * dm + lc) * C::kKtPitch + kk + 8 * lg);
        acc = mfma32(a, b, acc);
        acc = mfma32(al, b, acc);
      }
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int q = q0 + 8 * (r >> 2) + 4 * lg + (r & 3);
        if (q < N) unsafeAtomicAdd(dqh + (size_t)q * D + 32 * dm + lc, acc[r]);
      }
    }
  }

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

template <int D, bool CAUSAL>
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
    auto kern = fa_bwd_main_kernel<D, CAUSAL>;
    (void)hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, C::kLdsBytes);
    const int num_kt = (a.N + C::BN - 1) / C::BN;
    hipLaunchKernelGGL(kern, dim3(num_kt * BH), dim3(C::kThreads), C::kLdsBytes, a.stream, (const __bf16*)a.q,
                       (const __bf16*)a.k, (const __bf16*)a.v, (const __bf16*)a.dout, a.lse, a.delta, a.dq_acc,
                       (__bf16*)a.dk, (__bf16*)a.dv, a.N, BH, a.scale, a.scale * kLog2e);
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

hipError_t launch_bwd(const BwdArgs& a) {
  if (a.d == 64) return a.causal ? launch_bwd_d<64, true>(a) : launch_bwd_d<64, false>(a);
  return a.causal ? launch_bwd_d<128, true>(a) : launch_bwd_d<128, false>(a);
}

}  // namespace fa
