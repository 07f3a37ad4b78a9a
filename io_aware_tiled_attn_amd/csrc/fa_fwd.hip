// Forward attention kernels for gfx950.
//
// Method: exact attention computed tile by tile with the online-softmax
// update (vibeengines.com "FlashAttention, explained", sections "Tiling and
// the online softmax" and "The math, worked with real numbers"): for each
// query row keep a running max m, a running sum l and an output accumulator
// O; for each new key tile, m_new = max(m, tile max), rescale l and O by
// e^(m - m_new), add the tile's e^(s - m_new) and e^(s - m_new) V; finish
// with O / l.  The N x N scores never leave registers.
//
// bf16 kernel layout (one workgroup = 8 waves = 256 query rows):
//   * each wave owns 32 consecutive queries; its Q slice lives in registers
//     as the B operand of S^T = K Q^T (v_mfma_f32_32x32x16_bf16), so the
//     32x32 accumulator puts one query per lane column: the row max and row
//     sum are in-lane reductions plus one permlane32 swap.
//   * K and V tiles of BN keys are staged in LDS, double buffered, shared by
//     the 8 waves.  K is stored row-major with padding; V is stored
//     transposed (V^T[d][key]) with the keys of each 16-key group reordered
//     so the A operand of O^T += V^T P^T is one 16-byte LDS read per lane
//     and matches the key order the S^T accumulator leaves in each lane.
//   * P is rounded to bf16 (RNE) and fed back as the B operand directly from
//     the accumulator registers; O^T accumulates in fp32.
//   * workgroups are issued heaviest first (causal), with all query tiles of
//     one head on the same XCD (dispatch is round-robin over 8 XCDs and the
//     head index is the fast-varying part of the workgroup id).
#include "fa_common.h"
#include "fa_internal.h"

namespace fa {

template <int D, int BN>
struct FwdCfg {
  static constexpr int kWaves = 8;
  static constexpr int kThreads = kWaves * 64;
  static constexpr int BM = kWaves * 32;
  static constexpr int kKPitch = D + 8;    // bf16 elements per K row in LDS
  static constexpr int kVPitch = BN + 8;   // bf16 elements per V^T row in LDS
  static constexpr int kKTile = BN * kKPitch;
  static constexpr int kVTile = D * kVPitch;
  static constexpr int kStage = kKTile + kVTile;
  static constexpr int kLdsBytes = 2 * kStage * 2;
  static constexpr int kKChunks = BN * D / 8;             // 16-byte K chunks
  static constexpr int kKPerThread = (kKChunks + kThreads - 1) / kThreads;
  static constexpr int kVBlocks = (BN / 4) * (D / 4);     // 4x4 V blocks
  static constexpr int kVPerThread = (kVBlocks + kThreads - 1) / kThreads;
  static_assert(BN % 32 == 0 && D % 32 == 0, "tile shape");
  static_assert(kThreads == 512, "kernel launch bounds assume 512 threads");
};

// Position of key k (0 <= k < BN) inside its LDS row of V^T: bits 2 and 3
// swapped, so keys {4g..4g+3, 8+4g..8+4g+3} of each 16-key group are
// adjacent for lane half g.
__device__ __forceinline__ int vt_key_slot(int k) {
  return (k & ~0xC) | ((k & 4) << 1) | ((k & 8) >> 1);
}

template <int D, int BN>
struct FwdStage {
  u32x4 k[FwdCfg<D, BN>::kKPerThread];
  u32x2 v[FwdCfg<D, BN>::kVPerThread][4];
};

template <int D, int BN>
__device__ __forceinline__ void fwd_load_tile(FwdStage<D, BN>& st, const __bf16* __restrict__ Kh,
                                              const __bf16* __restrict__ Vh, int j0, int N, int tid) {
  using C = FwdCfg<D, BN>;
#pragma unroll
  for (int i = 0; i < C::kKPerThread; ++i) {
    const int c = tid + i * C::kThreads;
    const int row = c / (D / 8), col = (c % (D / 8)) * 8;
    const int key = j0 + row;
    u32x4 val = {0u, 0u, 0u, 0u};
    if (c < C::kKChunks && key < N) val = *(const u32x4*)(Kh + (size_t)key * D + col);
    st.k[i] = val;
  }
#pragma unroll
  for (int i = 0; i < C::kVPerThread; ++i) {
    const int b = tid + i * C::kThreads;
    const int kb = b / (D / 4), db = b % (D / 4);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int key = j0 + 4 * kb + r;
      u32x2 val = {0u, 0u};
      if (b < C::kVBlocks && key < N) val = *(const u32x2*)(Vh + (size_t)key * D + 4 * db);
      st.v[i][r] = val;
    }
  }
}

template <int D, int BN>
__device__ __forceinline__ void fwd_store_tile(const FwdStage<D, BN>& st, __bf16* Ks, __bf16* Vts, int tid) {
  using C = FwdCfg<D, BN>;
#pragma unroll
  for (int i = 0; i < C::kKPerThread; ++i) {
    const int c = tid + i * C::kThreads;
    if (c < C::kKChunks) {
      const int row = c / (D / 8), col = (c % (D / 8)) * 8;
      *(u32x4*)(Ks + row * C::kKPitch + col) = st.k[i];
    }
  }
#pragma unroll
  for (int i = 0; i < C::kVPerThread; ++i) {
    const int b = tid + i * C::kThreads;
    if (b < C::kVBlocks) {
      const int kb = b / (D / 4), db = b % (D / 4);
      const int slot = vt_key_slot(4 * kb);
      // 4 keys x 4 features in, 4 features x 4 keys out.
      const u32x2* r = st.v[i];
      u32x2 o0 = {pack_lo16(r[0][0], r[1][0]), pack_lo16(r[2][0], r[3][0])};
      u32x2 o1 = {pack_hi16(r[0][0], r[1][0]), pack_hi16(r[2][0], r[3][0])};
      u32x2 o2 = {pack_lo16(r[0][1], r[1][1]), pack_lo16(r[2][1], r[3][1])};
      u32x2 o3 = {pack_hi16(r[0][1], r[1][1]), pack_hi16(r[2][1], r[3][1])};
      __bf16* base = Vts + (4 * db) * C::kVPitch + slot;
      *(u32x2*)(base + 0 * C::kVPitch) = o0;
      *(u32x2*)(base + 1 * C::kVPitch) = o1;
      *(u32x2*)(base + 2 * C::kVPitch) = o2;
      *(u32x2*)(base + 3 * C::kVPitch) = o3;
    }
  }
}

template <int D, int BN, bool CAUSAL>
__global__ void __launch_bounds__(512)
fa_fwd_bf16_kernel(const __bf16* __restrict__ Q, const __bf16* __restrict__ K,
                   const __bf16* __restrict__ V, __bf16* __restrict__ O, float* __restrict__ LSE,
                   int N, int BH, int num_qt, float scale_log2) {
  using C = FwdCfg<D, BN>;
  extern __shared__ __attribute__((aligned(16))) __bf16 smem[];

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int lc = lane & 31;     // lane column: query within the wave
  const int lg = lane >> 5;     // lane half

  const int bid = blockIdx.x;
  const int qt = num_qt - 1 - bid / BH;   // heaviest query tiles first
  const int bh = bid % BH;
  const size_t head_off = (size_t)bh * N * D;
  const __bf16* Qh = Q + head_off;
  const __bf16* Kh = K + head_off;
  const __bf16* Vh = V + head_off;

  const int q_wave0 = qt * C::BM + wave * 32;
  const int q_idx = q_wave0 + lc;

  // Q^T as MFMA B operand: lane holds Q[q][16 ks + 8 lg .. +7].
  bf16x8 qb[D / 16];
#pragma unroll
  for (int ks = 0; ks < D / 16; ++ks) {
    u32x4 val = {0u, 0u, 0u, 0u};
    if (q_idx < N) val = *(const u32x4*)(Qh + (size_t)q_idx * D + 16 * ks + 8 * lg);
    qb[ks] = __builtin_bit_cast(bf16x8, val);
  }

  f32x16 oacc[D / 32];
#pragma unroll
  for (int i = 0; i < D / 32; ++i) oacc[i] = (f32x16){};
  float m_run = -INFINITY;   // running max of scale*log2(e)*s
  float l_run = 0.f;         // this lane's share of the running sum

  const int q_tile_end = min(N, (qt + 1) * C::BM);
  const int key_end = CAUSAL ? q_tile_end : N;
  const int num_kt = (key_end + BN - 1) / BN;

  FwdStage<D, BN> st;
  fwd_load_tile<D, BN>(st, Kh, Vh, 0, N, tid);
  fwd_store_tile<D, BN>(st, smem, smem + C::kKTile, tid);

  for (int t = 0; t < num_kt; ++t) {
    const int j0 = t * BN;
    if (t + 1 < num_kt) fwd_load_tile<D, BN>(st, Kh, Vh, j0 + BN, N, tid);
    __syncthreads();
    const __bf16* Ks = smem + (t & 1) * C::kStage;
    const __bf16* Vts = Ks + C::kKTile;

    const bool wave_live = !CAUSAL || j0 <= q_wave0 + 31;
    if (wave_live) {
      // S^T = K Q^T for this tile: BN keys x 32 queries.
      f32x16 s[BN / 32];
#pragma unroll
      for (int mb = 0; mb < BN / 32; ++mb) {
        f32x16 acc = (f32x16){};
        const __bf16* krow = Ks + (32 * mb + lc) * C::kKPitch + 8 * lg;
#pragma unroll
        for (int ks = 0; ks < D / 16; ++ks) {
          bf16x8 a = *(const bf16x8*)(krow + 16 * ks);
          acc = mfma32(a, qb[ks], acc);
        }
        s[mb] = acc;
      }
      // Mask keys past the end and, on the diagonal, keys after the query.
      const bool need_mask = (j0 + BN > N) || (CAUSAL && j0 + BN - 1 > q_wave0);
      if (need_mask) {
        const int qlim = CAUSAL ? min(q_idx, N - 1) : N - 1;
#pragma unroll
        for (int mb = 0; mb < BN / 32; ++mb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int key = j0 + 32 * mb + 8 * (r >> 2) + 4 * lg + (r & 3);
            if (key > qlim) s[mb][r] = -INFINITY;
          }
      }
      float mx = -INFINITY;
#pragma unroll
      for (int mb = 0; mb < BN / 32; ++mb)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[mb][r]);
      mx = max_with_lane_xor32(mx);
      const float m_new = fmaxf(m_run, mx * scale_log2);
      const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
      const float alpha = fast_exp2(m_run - m_use);
      m_run = m_new;

      // P = exp2(s * scale * log2(e) - m), packed to bf16 as the B operand.
      bf16x8 pb[BN / 16];
      float rowsum = 0.f;
#pragma unroll
      for (int mb = 0; mb < BN / 32; ++mb) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          uint32_t w[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float p0 = fast_exp2(__builtin_fmaf(s[mb][8 * h + 2 * e], scale_log2, -m_use));
            const float p1 = fast_exp2(__builtin_fmaf(s[mb][8 * h + 2 * e + 1], scale_log2, -m_use));
            rowsum += p0 + p1;
            w[e] = pack_bf16x2(p0, p1);
          }
          u32x4 wv = {w[0], w[1], w[2], w[3]};
          pb[2 * mb + h] = __builtin_bit_cast(bf16x8, wv);
        }
      }
      l_run = l_run * alpha + rowsum;
      if (__ballot(alpha != 1.f)) {
#pragma unroll
        for (int i = 0; i < D / 32; ++i) oacc[i] *= alpha;
      }
      // O^T += V^T P^T.
#pragma unroll
      for (int c = 0; c < BN / 16; ++c) {
#pragma unroll
        for (int dm = 0; dm < D / 32; ++dm) {
          bf16x8 a = *(const bf16x8*)(Vts + (32 * dm + lc) * C::kVPitch + 16 * c + 8 * lg);
          oacc[dm] = mfma32(a, pb[c], oacc[dm]);
        }
      }
    }
    if (t + 1 < num_kt) {
      __bf16* Kn = smem + ((t + 1) & 1) * C::kStage;
      fwd_store_tile<D, BN>(st, Kn, Kn + C::kKTile, tid);
    }
  }

  // Epilogue: O / l rounded to bf16, and LSE = m + ln l (natural log).
  const float l_tot = sum_with_lane_xor32(l_run);
  const float inv_l = l_tot > 0.f ? 1.f / l_tot : 0.f;
  if (q_idx < N) {
    __bf16* orow = O + head_off + (size_t)q_idx * D;
#pragma unroll
    for (int dm = 0; dm < D / 32; ++dm)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        u32x2 w = {pack_bf16x2(oacc[dm][4 * i + 0] * inv_l, oacc[dm][4 * i + 1] * inv_l),
                   pack_bf16x2(oacc[dm][4 * i + 2] * inv_l, oacc[dm][4 * i + 3] * inv_l)};
        *(u32x2*)(orow + 32 * dm + 8 * i + 4 * lg) = w;
      }
    if (LSE != nullptr && lg == 0)
      LSE[(size_t)bh * N + q_idx] = l_tot > 0.f ? m_run * kLn2 + __logf(l_tot) : -INFINITY;
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
  const int qt = num_qt - 1 - bid / BH;
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
template <int D, int BN, bool CAUSAL>
static hipError_t launch_bf16(const FwdArgs& a) {
  using C = FwdCfg<D, BN>;
  const int BH = a.B * a.H;
  const int num_qt = (a.N + C::BM - 1) / C::BM;
  auto kern = fa_fwd_bf16_kernel<D, BN, CAUSAL>;
  // Dynamic LDS above 64 KB must be allowed explicitly; setting the same
  // value from several threads is harmless.
  (void)hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, C::kLdsBytes);
  hipLaunchKernelGGL(kern, dim3(num_qt * BH), dim3(C::kThreads), C::kLdsBytes, a.stream,
                     (const __bf16*)a.q, (const __bf16*)a.k, (const __bf16*)a.v, (__bf16*)a.o, a.lse, a.N, BH,
                     num_qt, a.scale * kLog2e);
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
  return a.causal ? launch_bf16<D, BN, true>(a) : launch_bf16<D, BN, false>(a);
}

hipError_t launch_fwd(const FwdArgs& a) {
  if (a.dtype == FA_DTYPE_FP32) {
    if (a.d == 64) return a.causal ? launch_f32<64, true>(a) : launch_f32<64, false>(a);
    return a.causal ? launch_f32<128, true>(a) : launch_f32<128, false>(a);
  }
  const int bn = a.block_n == 0 ? 64 : a.block_n;
  if (a.d == 64) {
    if (bn == 32) return launch_bf16_bn<64, 32>(a);
    if (bn == 64) return launch_bf16_bn<64, 64>(a);
    return launch_bf16_bn<64, 128>(a);
  }
  if (bn == 32) return launch_bf16_bn<128, 32>(a);
  if (bn == 64) return launch_bf16_bn<128, 64>(a);
  return launch_bf16_bn<128, 128>(a);
}

}  // namespace fa
