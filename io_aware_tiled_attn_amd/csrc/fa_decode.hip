// Decoding with a key/value cache: Nq <= 16 new queries per head attend to
// an Nk-entry cache, split over the keys (split-KV).
//
// The pages ask which parts of FlashAttention's speed-up carry over to
// autoregressive decoding with a KV cache (chorfi.xyz study guide,
// "Discussion prompts").  With a handful of queries per head the work is
// one read of K and V, so the path is bound by HBM bandwidth, not by the
// matrix cores: the tiling that keeps the score matrix on chip still
// applies, the MFMA utilisation argument does not.
//
// Method: the same online-softmax rule as the forward pass
// (vibeengines.com, "Tiling and the online softmax": running max m, running
// sum l, rescaled accumulator O), applied first within each split of the
// keys and then once more to merge the splits, each split's result entering
// as a block with its own (m, l, O) (carried as O/l and its log-sum-exp).
//
// Layout: one wave per (head, split).  Queries are padded to 16, the width
// of v_mfma_f32_16x16x32_bf16:
//   S^T (16 keys x 16 queries) = K Q^T: K rows straight from global memory
//     as A operands (lane l: key l % 16, features 8 (l / 16) + 0..7 of each
//     32-feature step), Q^T in registers as B operands;
//   the accumulator leaves each lane one query (l % 16) and keys
//     4 (l / 16) + 0..3 of the 16-key block, so a query's max and sum span
//     the four lanes l % 16 + 16 g;
//   O^T (16 features x 16 queries per block) += V^T P^T over 32-key steps:
//     P^T is the B operand built from two score blocks (keys 4 g + 0..3 and
//     16 + 4 g + 0..3 in lane group g); V^T is read from this wave's LDS
//     copy of the V tile with ds_read_b64_tr_b16 in the same key order.
// Each split writes O/l (fp32) and LSE; a second kernel merges the splits.
#include "fa_common.h"
#include "fa_internal.h"

namespace fa {

typedef float f32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f32x4_t mfma16(bf16x8 a, bf16x8 b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

template <int D>
struct DecCfg {
  static constexpr int kWaves = 4;            // independent waves per workgroup
  static constexpr int KT = 32;               // keys per tile
  static constexpr int kPitch = D + 16;       // bf16 elements per V row in LDS
  static constexpr int kTileElems = KT * kPitch;
  static constexpr int kLdsBytes = kWaves * kTileElems * 2;
  static constexpr int kVChunks = KT * D / 8 / 64;   // 16-byte V chunks per lane per tile
};

// Splits of the keys per head: enough waves to fill the GPU (about 4 per
// SIMD), each split at least one tile.  The workspace size uses the same
// formula.
__host__ __device__ inline int decode_splits(int BH, int Nk) {
  const int tiles = (Nk + 31) / 32;
  int s = (4096 + BH - 1) / BH;
  if (s > tiles) s = tiles;
  if (s > 256) s = 256;
  return s < 1 ? 1 : s;
}

// Four waves per SIMD (at most 128 registers each): decode_splits sizes the
// launch for exactly that many waves, so they all run in one round.
template <int D, bool CAUSAL>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(4)))
fa_decode_split_kernel(const __bf16* __restrict__ Q, const __bf16* __restrict__ K, const __bf16* __restrict__ V,
                       float* __restrict__ part_o, float* __restrict__ part_lse, int BH, int Nq, int Nk,
                       int n_split, float scale_log2) {
  using C = DecCfg<D>;
  extern __shared__ __attribute__((aligned(16))) __bf16 smem[];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int unit = blockIdx.x * C::kWaves + wave;   // (head, split) pair of this wave
  if (unit >= BH * n_split) return;                 // wave-uniform; no barriers in this kernel
  const int bh = unit / n_split, split = unit % n_split;
  const int qi = lane & 15;    // query of this lane's accumulator column
  const int g = lane >> 4;     // lane group
  __bf16* vt = smem + wave * C::kTileElems;

  // Keys of this split, whole tiles.
  const int tiles = (Nk + C::KT - 1) / C::KT;
  const int t0 = (int)((long)tiles * split / n_split), t1 = (int)((long)tiles * (split + 1) / n_split);

  const __amdgpu_buffer_rsrc_t rq = make_rsrc(Q + (size_t)bh * Nq * D, (uint32_t)Nq * D * 2u);
  const __amdgpu_buffer_rsrc_t rk = make_rsrc(K + (size_t)bh * Nk * D, (uint32_t)Nk * D * 2u);
  const __amdgpu_buffer_rsrc_t rv = make_rsrc(V + (size_t)bh * Nk * D, (uint32_t)Nk * D * 2u);

  // Q^T as B operands (queries past Nq read as zero).
  bf16x8 qb[D / 32];
#pragma unroll
  for (int ks = 0; ks < D / 32; ++ks)
    qb[ks] = __builtin_bit_cast(bf16x8, bload128(rq, (uint32_t)(qi * D + 32 * ks + 8 * g) * 2u));

  f32x4_t oacc[D / 16];
#pragma unroll
  for (int i = 0; i < D / 16; ++i) oacc[i] = (f32x4_t){};
  float m_run = -INFINITY, l_run = 0.f;   // per query (same in the 4 lanes of a query)
  // Keys a query may see: all, or (causal) up to Nk - Nq + query.
  const int key_lim = CAUSAL ? Nk - Nq + qi : Nk - 1;
  // Transposing-read offset: group g reads rows 4 g + s / 4 at column 4 (s % 4).
  const int s16 = lane & 15;
  const int tr_off = (4 * g + (s16 >> 2)) * C::kPitch + 4 * (s16 & 3);

  for (int t = t0; t < t1; ++t) {
    const int k0 = t * C::KT;
    // K rows as A operands, straight from global memory.
    bf16x8 ka[2][D / 32];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int ks = 0; ks < D / 32; ++ks)
        ka[kb][ks] = __builtin_bit_cast(
            bf16x8, bload128(rk, (uint32_t)((k0 + 16 * kb + (lane & 15)) * D + 32 * ks + 8 * g) * 2u));
    // V tile rows into this wave's LDS buffer (row-major, padded).
    u32x4 vr[C::kVChunks];
#pragma unroll
    for (int i = 0; i < C::kVChunks; ++i) {
      const int c = lane + 64 * i, row = c / (D / 8), col = (c % (D / 8)) * 8;
      vr[i] = bload128(rv, (uint32_t)((k0 + row) * D + col) * 2u);
    }
#pragma unroll
    for (int i = 0; i < C::kVChunks; ++i) {
      const int c = lane + 64 * i, row = c / (D / 8), col = (c % (D / 8)) * 8;
      *(u32x4*)(vt + row * C::kPitch + col) = vr[i];
    }
    // Scores: two 16-key blocks.
    f32x4_t s[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      s[kb] = (f32x4_t){};
#pragma unroll
      for (int ks = 0; ks < D / 32; ++ks) s[kb] = mfma16(ka[kb][ks], qb[ks], s[kb]);
    }
    // Mask keys past the cache (and, causal, past the query's position).
    if (k0 + C::KT > Nk || (CAUSAL && k0 + C::KT - 1 > Nk - Nq)) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int key = k0 + 16 * kb + 4 * g + r;
          if (key > key_lim || key >= Nk) s[kb][r] = -INFINITY;
        }
    }
    // Online softmax for this tile (eager max).
    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 4; ++r) mx = fmaxf(mx, s[kb][r]);
    mx = fmaxf(mx, __shfl_xor(mx, 16));
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float m_new = fmaxf(m_run, mx * scale_log2);
    const float m_use = m_new == -INFINITY ? 0.f : m_new;
    const float alpha = m_new == -INFINITY ? 1.f : fast_exp2(m_run - m_new);
    float p[8], rs = 0.f;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        p[4 * kb + r] = fast_exp2(__builtin_fmaf(s[kb][r], scale_log2, -m_use));
        rs += p[4 * kb + r];
      }
    m_run = m_new;
    l_run = l_run * alpha + rs;   // this lane's partial; the four lanes of a query are summed at the end
    const bf16x8 pb = __builtin_bit_cast(
        bf16x8, ((u32x4){pack_bf16x2(p[0], p[1]), pack_bf16x2(p[2], p[3]), pack_bf16x2(p[4], p[5]),
                         pack_bf16x2(p[6], p[7])}));
    // O^T += V^T P^T, 16 features per block; V^T read from LDS, keys in the
    // order of pb: rows 4 g + 0..3 then 16 + 4 g + 0..3.
#pragma unroll
    for (int dm = 0; dm < D / 16; ++dm) {
      const bf16x8 a = lds_tr_pair(vt + tr_off, 16 * dm, 16 * C::kPitch + 16 * dm);
      oacc[dm] = mfma16(a, pb, oacc[dm] * alpha);
    }
  }

  // This split's O / l and LSE per query (queries past Nq are not written).
  float l_tot = l_run + __shfl_xor(l_run, 16);
  l_tot += __shfl_xor(l_tot, 32);
  if (qi < Nq) {
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
    float* po = part_o + ((size_t)unit * 16 + qi) * D;
#pragma unroll
    for (int dm = 0; dm < D / 16; ++dm)
      *(f32x4_t*)(po + 16 * dm + 4 * g) = oacc[dm] * inv;
    if (g == 0) part_lse[(size_t)unit * 16 + qi] = l_tot > 0.f ? m_run * kLn2 + __logf(l_tot) : -INFINITY;
  }
}

// Merge of the splits for one (head, query): LSE = log sum_s e^(lse_s),
// O = sum_s e^(lse_s - LSE) O_s (the online-softmax rule applied to whole
// splits).  One 64-lane wave per (head, query); lane c covers features
// c, c + 64, ... .
template <int D>
__global__ void __launch_bounds__(256)
fa_decode_merge_kernel(const float* __restrict__ part_o, const float* __restrict__ part_lse,
                       __bf16* __restrict__ O, float* __restrict__ LSE, int BH, int Nq, int n_split) {
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);   // (head, query)
  if (row >= BH * Nq) return;
  const int bh = row / Nq, qi = row % Nq;
  float m = -INFINITY;
  for (int s = 0; s < n_split; ++s) m = fmaxf(m, part_lse[((size_t)bh * n_split + s) * 16 + qi]);
  float acc[D / 64] = {};
  float tot = 0.f;
  if (m != -INFINITY) {
    for (int s = 0; s < n_split; ++s) {
      const size_t u = (size_t)bh * n_split + s;
      const float w = __expf(part_lse[u * 16 + qi] - m);
      tot += w;
#pragma unroll
      for (int j = 0; j < D / 64; ++j) acc[j] = __builtin_fmaf(w, part_o[(u * 16 + qi) * D + lane + 64 * j], acc[j]);
    }
  }
  const float inv = tot > 0.f ? 1.f / tot : 0.f;
  __bf16* orow = O + ((size_t)bh * Nq + qi) * D;
#pragma unroll
  for (int j = 0; j < D / 64; ++j) orow[lane + 64 * j] = (__bf16)(acc[j] * inv);
  if (LSE != nullptr && lane == 0) LSE[(size_t)bh * Nq + qi] = tot > 0.f ? m + __logf(tot) : -INFINITY;
}

template <int D, bool CAUSAL>
static hipError_t launch_decode_d(const DecodeArgs& a) {
  using C = DecCfg<D>;
  const int BH = a.B * a.H;
  const int n_split = decode_splits(BH, a.Nk);
  const int units = BH * n_split;
  hipLaunchKernelGGL((fa_decode_split_kernel<D, CAUSAL>), dim3((units + C::kWaves - 1) / C::kWaves), dim3(256),
                     C::kLdsBytes, a.stream, (const __bf16*)a.q, (const __bf16*)a.k, (const __bf16*)a.v, a.part_o,
                     a.part_lse, BH, a.Nq, a.Nk, n_split, a.scale * kLog2e);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int rows = BH * a.Nq;
  hipLaunchKernelGGL((fa_decode_merge_kernel<D>), dim3((rows + 3) / 4), dim3(256), 0, a.stream, a.part_o,
                     a.part_lse, (__bf16*)a.o, a.lse, BH, a.Nq, n_split);
  return hipGetLastError();
}

hipError_t launch_decode(const DecodeArgs& a) {
  if (a.d == 64) return a.causal ? launch_decode_d<64, true>(a) : launch_decode_d<64, false>(a);
  return a.causal ? launch_decode_d<128, true>(a) : launch_decode_d<128, false>(a);
}

// Workspace: partial O [units][16][d] fp32 (padded to 256 bytes), then
// partial LSE [units][16] fp32; units = B*H*splits.
static size_t decode_o_bytes(int B, int H, int Nk, int d) {
  const size_t units = (size_t)B * H * decode_splits(B * H, Nk);
  return (units * 16 * (size_t)d * 4 + 255) & ~(size_t)255;
}

size_t decode_workspace_bytes(int B, int H, int Nk, int d) {
  const size_t units = (size_t)B * H * decode_splits(B * H, Nk);
  return (decode_o_bytes(B, H, Nk, d) + units * 16 * 4 + 255) & ~(size_t)255;
}

float* decode_part_lse(float* part_o, int B, int H, int Nk, int d) {
  return reinterpret_cast<float*>(reinterpret_cast<char*>(part_o) + decode_o_bytes(B, H, Nk, d));
}

}  // namespace fa
