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
// Their operands are fp16 copies of Q, dO, K and V, made as the tiles are
// staged, each scaled by a power of two per head that brings its largest
// magnitude into [1, 2): a bf16
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
//   2. bwd_scales: each head's four factors from its chunk maxima.
//   3. bwd_dkdv: key-major.  One workgroup of 8 waves per 128-key tile: wave
//      w owns key block w % 4 and the query half w / 4 of every 64-query
//      step, recomputes S, dP, P and dS for its 32 x 32 block and
//      accumulates partial dK^T and dV^T; the halves are summed through LDS.
//   4. bwd_dq: query-major.  One workgroup of 8 waves per 128-query tile:
//      wave w owns query block w % 4 and the key half w / 4 of every
//      64-key step, recomputes S^T, dP^T, P^T and dS^T (one query per lane)
//      and accumulates partial dQ^T; the halves are summed through LDS and
//      dQ is written once.
// The two passes recompute S and dP each: seven products per (query,
// key) tile pair instead of five, and no atomics.
#include <mutex>

#include "fa_common.h"
#include "fa_internal.h"

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

// Largest value of x over the workgroup (NW waves), returned to every
// thread.  red: NW floats of LDS.
template <int NW>
__device__ __forceinline__ float block_max(float x, float* red) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) x = fmaxf(x, __shfl_xor(x, off));
  __syncthreads();   // red may still be read by a previous call
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = x;
  __syncthreads();
  float m = red[0];
#pragma unroll
  for (int i = 1; i < NW; ++i) m = fmaxf(m, red[i]);
  return m;
}

// ---------------------------------------------------------------------------
// 1. Per 256-row chunk of a head: D_i = sum_c dO_ic O_ic and the largest
//    |Q|, |dO|, |K|, |V| of the chunk.
// ---------------------------------------------------------------------------
template <int D>
__global__ void __launch_bounds__(256)
fa_bwd_prep_kernel(const __bf16* __restrict__ O, const __bf16* __restrict__ dO, const __bf16* __restrict__ Q,
                   const __bf16* __restrict__ K, const __bf16* __restrict__ V, float* __restrict__ delta,
                   float* __restrict__ part, int N, int nch) {
  constexpr int TPR = D / 8;          // threads per row, 8 elements each
  constexpr int RPI = 256 / TPR;      // rows per pass
  __shared__ float red[4];
  const int bh = blockIdx.x / nch, ch = blockIdx.x % nch;
  const int tid = threadIdx.x, col = (tid % TPR) * 8;
  const int row0 = ch * kBwdChunkRows;
  const int rows = min(kBwdChunkRows, N - row0);
  float m[4] = {0.f, 0.f, 0.f, 0.f};
  for (int r = tid / TPR; r < rows; r += RPI) {
    const size_t off = ((size_t)bh * N + row0 + r) * D + col;
    const u32x4 o = *(const u32x4*)(O + off);
    const u32x4 g = *(const u32x4*)(dO + off);
    const u32x4 qv = *(const u32x4*)(Q + off);
    const u32x4 kv = *(const u32x4*)(K + off);
    const u32x4 vv = *(const u32x4*)(V + off);
    float acc = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      acc += bf16_lo(o[i]) * bf16_lo(g[i]) + bf16_hi(o[i]) * bf16_hi(g[i]);
      m[0] = abs_max_bf16x2(m[0], qv[i]);
      m[1] = abs_max_bf16x2(m[1], g[i]);
      m[2] = abs_max_bf16x2(m[2], kv[i]);
      m[3] = abs_max_bf16x2(m[3], vv[i]);
    }
    // The TPR threads of a row share r, so they run this together.
#pragma unroll
    for (int o2 = TPR / 2; o2 > 0; o2 >>= 1) acc += __shfl_xor(acc, o2);
    if (tid % TPR == 0) delta[(size_t)bh * N + row0 + r] = acc;
  }
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    m[t] = block_max<4>(m[t], red);
    if (tid == 0) part[((size_t)bh * nch + ch) * 4 + t] = m[t];
  }
}

// ---------------------------------------------------------------------------
// 2. One thread per (head, tensor): the power-of-two factor that brings the
//    head's largest |Q|, |dO|, |K| or |V| into [1, 2).
// ---------------------------------------------------------------------------
__global__ void __launch_bounds__(256)
fa_bwd_scales_kernel(const float* __restrict__ part, float* __restrict__ scales, int n, int nch) {
  const int t = blockIdx.x * 256 + threadIdx.x;   // head t / 4, tensor t % 4
  if (t >= n) return;
  const float* p = part + (size_t)(t >> 2) * nch * 4 + (t & 3);
  float m = 0.f;
  for (int i = 0; i < nch; ++i) m = fmaxf(m, p[4 * i]);
  scales[t] = pow2_scale_for(m);
}

// bf16 pair times f, rounded to an fp16 pair.
__device__ __forceinline__ uint32_t bf16x2_to_f16x2(uint32_t w, float f) {
  return pack_f16x2(bf16_lo(w) * f, bf16_hi(w) * f);
}
__device__ __forceinline__ u32x4 bf16x8_to_f16x8(u32x4 x, float f) {
  return (u32x4){bf16x2_to_f16x2(x[0], f), bf16x2_to_f16x2(x[1], f), bf16x2_to_f16x2(x[2], f),
                 bf16x2_to_f16x2(x[3], f)};
}

// ---------------------------------------------------------------------------
// Shared by the two main kernels: 8 waves, 128 rows resident in LDS (keys
// for dK/dV, queries for dQ) and 64 rows of the other side staged per step
// through registers into a double-buffered LDS stage.  Rows are padded to
// D + 8 fp16 elements.
// ---------------------------------------------------------------------------
template <int D>
struct BwdCfg {
  static constexpr int kThreads = 512;
  static constexpr int RES = 128;                // resident rows per workgroup (4 blocks of 32)
  static constexpr int STEP = 64;                // staged rows per step (2 halves of 32)
  static constexpr int kPitch = D + 8;           // LDS row pitch (fp16 elements)
  static constexpr int kResTile = RES * kPitch;  // one resident tensor
  static constexpr int kStepTile = STEP * kPitch;
  static constexpr int kResBytes = 2 * kResTile * 2;                  // two resident tensors
  static constexpr int kStageBytes = 2 * kStepTile * 2 + 2 * STEP * 4; // two staged tensors + two row terms
  static constexpr int kLdsBytes = kResBytes + 2 * kStageBytes;
  static constexpr int kStageChunks = STEP * D / 8 / kThreads;       // 16-byte chunks per thread and tensor
  static constexpr int kResChunks = RES * D / 8 / kThreads;
  // Closing sum of the two halves' accumulators: D floats per lane of four
  // waves, feature-major.
  static constexpr int kRedBytes = D * 4 * 64 * 4;
  static constexpr int kLdsTotal = kLdsBytes > kRedBytes ? kLdsBytes : kRedBytes;
  // The dQ kernel keeps its resident rows in registers: two stages, or its
  // closing sum (D / 2 floats per lane of four waves).
  static constexpr int kDqLdsTotal = 2 * kStageBytes > kRedBytes / 2 ? 2 * kStageBytes : kRedBytes / 2;
  static_assert(STEP * D / 8 % kThreads == 0 && RES * D / 8 % kThreads == 0, "tile staging");
  static_assert(kLdsTotal + 4 * (65536 / STEP + 1) <= 160 * 1024, "LDS budget (with a sparse step list)");
};

// Per-head buffer descriptors: rows past N read as zero.
struct BwdHead {
  __amdgpu_buffer_rsrc_t q, k, v, g, lse, dlt;
};

template <int D>
__device__ __forceinline__ BwdHead bwd_head(const __bf16* Q, const __bf16* K, const __bf16* V, const __bf16* dO,
                                            const float* LSE, const float* delta, int bh, int N) {
  const size_t head_off = (size_t)bh * N * D;
  const uint32_t head_bytes = (uint32_t)N * D * 2u;
  BwdHead h;
  h.q = make_rsrc(Q + head_off, head_bytes);
  h.k = make_rsrc(K + head_off, head_bytes);
  h.v = make_rsrc(V + head_off, head_bytes);
  h.g = make_rsrc(dO + head_off, head_bytes);
  h.lse = make_rsrc(LSE + (size_t)bh * N, (uint32_t)N * 4u);
  h.dlt = make_rsrc(delta + (size_t)bh * N, (uint32_t)N * 4u);
  return h;
}

// Rows r0 .. r0 + ROWS of two bf16 tensors (a, b) into padded fp16 LDS
// tiles, through registers: load issues the loads, store scales the values
// by the tensors' factors, rounds them to fp16 and writes them.
template <int D, int ROWS>
struct RowPair {
  static constexpr int kChunks = ROWS * D / 8 / 512;
  u32x4 a[kChunks], b[kChunks];
  __device__ __forceinline__ void load(__amdgpu_buffer_rsrc_t ra, __amdgpu_buffer_rsrc_t rb, int r0, int tid) {
#pragma unroll
    for (int i = 0; i < kChunks; ++i) {
      const int c = tid + i * 512;
      const uint32_t off = (uint32_t)((r0 + c / (D / 8)) * D + (c % (D / 8)) * 8) * 2u;
      a[i] = bload128(ra, off);
      b[i] = bload128(rb, off);
    }
  }
  __device__ __forceinline__ void store(_Float16* ta, _Float16* tb, float fa, float fb, int tid) const {
#pragma unroll
    for (int i = 0; i < kChunks; ++i) {
      const int c = tid + i * 512;
      const int off = (c / (D / 8)) * (D + 8) + (c % (D / 8)) * 8;
      *(u32x4*)(ta + off) = bf16x8_to_f16x8(a[i], fa);
      *(u32x4*)(tb + off) = bf16x8_to_f16x8(b[i], fb);
    }
  }
};

// ---------------------------------------------------------------------------
// 3. dK and dV: one workgroup of 8 waves per 128-key tile of one head, two
//    waves per SIMD.  Wave w owns key block kb = w % 4 (32 keys) and query
//    half qh = w / 4 of each 64-query step.  K and V of the tile sit in LDS
//    (their rows are the B operands of S = Q K^T and dP = dO V^T, one key
//    per lane); Q and dO of the step are staged; dV^T += dO^T P and
//    dK^T += Q^T dS take their A operands with ds_read_b64_tr_b16.
// SPARSE: block-sparse attention.  bmask holds, per head, an nb x nb byte
// matrix over (128-query block, 128-key block) pairs (a workgroup's keys are
// one key block); the workgroup visits only the 64-query steps whose query
// block its mask column keeps, from a list built in LDS.
// ---------------------------------------------------------------------------
template <int D, bool CAUSAL, bool SPARSE>
__global__ void __launch_bounds__(512)
fa_bwd_dkdv_kernel(const __bf16* __restrict__ Q, const __bf16* __restrict__ K, const __bf16* __restrict__ V,
                   const __bf16* __restrict__ dO, const float* __restrict__ LSE,
                   const float* __restrict__ delta, const float* __restrict__ scales, __bf16* __restrict__ dK,
                   __bf16* __restrict__ dV, const uint8_t* __restrict__ bmask, int N, int BH, float scale,
                   float scale_log2) {
  using C = BwdCfg<D>;
  static_assert(C::RES == FA_SPARSE_BLOCK && FA_SPARSE_BLOCK % C::STEP == 0, "sparse blocks vs tiles");
  constexpr int KS = D / 16;                 // k-steps of the score products
  constexpr int DM = D / 32;                 // 32-feature blocks
  extern __shared__ __attribute__((aligned(16))) char smem_raw[];
  _Float16* Ks = (_Float16*)smem_raw;                              // [RES][kPitch]
  _Float16* Vs = Ks + C::kResTile;
  char* stages = smem_raw + C::kResBytes;

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);       // uniform per wave
  const int kb = wave & 3;                   // key block of this wave
  const int qh = wave >> 2;                  // query half of each step
  const int lane = tid & 63;
  const int lc = lane & 31, lg = lane >> 5;
  int kt, bh;   // key tile (small kt = most query steps) and head
  xcd_head_major(blockIdx.x, BH, (N + C::RES - 1) / C::RES, bh, kt);
  const BwdHead h = bwd_head<D>(Q, K, V, dO, LSE, delta, bh, N);

  const int k0 = kt * C::RES;                 // first key of the workgroup
  const int kw0 = k0 + kb * 32;               // first key of this wave
  const int key = kw0 + lc;                   // this lane's key column
  const bool key_ok = key < N;

  // In the copies' units: the exponent's multiplier for the scaled S, D's
  // factor into the scaled dP's units, the epilogue factors of dK and dV.
  const float sq = scales[bh * 4 + 0], sg = scales[bh * 4 + 1];
  const float sk = scales[bh * 4 + 2], sv = scales[bh * 4 + 3];
  const float c2 = scale_log2 / (sq * sk);
  const float dsc = sg * sv;
  const float dk_fac = scale / (sg * sv * sq);
  const float dv_fac = 1.f / sg;

  {
    RowPair<D, C::RES> kv;
    kv.load(h.k, h.v, k0, tid);
    kv.store(Ks, Vs, sk, sv, tid);
  }

  const int qrow_off = (32 * qh + lc) * C::kPitch + 8 * lg;             // Q / dO rows, A operands
  const int krow_off = (32 * kb + lc) * C::kPitch + 8 * lg;             // K / V rows, B operands
  const int tr_off = tr_lane_off(lane, C::kPitch, 4) + 32 * qh * C::kPitch;   // Q^T / dO^T

  f32x16 dk_acc[DM], dv_acc[DM];
#pragma unroll
  for (int i = 0; i < DM; ++i) {
    dk_acc[i] = (f32x16){};
    dv_acc[i] = (f32x16){};
  }

  // Query steps (STEP queries each) that can see these keys: all from
  // qt_begin (dense), or the ones the mask column keeps, listed in LDS after
  // the other buffers (count first).
  const int qt_begin = CAUSAL ? k0 / C::STEP : 0;
  int n_steps = (N + C::STEP - 1) / C::STEP - qt_begin;
  int* slist = (int*)(smem_raw + C::kLdsTotal);
  if constexpr (SPARSE) {
    const int nb = (N + FA_SPARSE_BLOCK - 1) / FA_SPARSE_BLOCK;
    const uint8_t* col = bmask + (size_t)bh * nb * nb + kt;   // entry of query block i at col[i * nb]
    if (wave == 0) {
      int cnt = 0;
      for (int base = 0; base < n_steps; base += 64) {
        const int qs = qt_begin + base + lane;
        const bool live = base + lane < n_steps && col[(size_t)(qs * C::STEP / FA_SPARSE_BLOCK) * nb] != 0;
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

  // Stage: Q and dO rows, LSE * log2 e (+inf past N and for rows that saw
  // no key, so P = 0 there) and D in the scaled dP's units.
  RowPair<D, C::STEP> qg;
  float lse_raw = 0.f, dlt_raw = 0.f;
  auto load_stage = [&](int q0) {
    qg.load(h.q, h.g, q0, tid);
    if (tid < C::STEP) lse_raw = q0 + tid < N ? bload32f(h.lse, (uint32_t)(q0 + tid) * 4u) : INFINITY;
    else if (tid < 2 * C::STEP) dlt_raw = bload32f(h.dlt, (uint32_t)(q0 + tid - C::STEP) * 4u);
  };
  auto store_stage = [&](int buf) {
    _Float16* Qs = (_Float16*)(stages + buf * C::kStageBytes);
    _Float16* Gs = Qs + C::kStepTile;
    float* Ls = (float*)(Gs + C::kStepTile);
    qg.store(Qs, Gs, sq, sg, tid);
    if (tid < C::STEP) Ls[tid] = lse_raw == -INFINITY ? INFINITY : lse_raw * kLog2e;
    else if (tid < 2 * C::STEP) Ls[tid] = dlt_raw * dsc;
  };
  if (n_steps > 0) {
    load_stage(step_at(0) * C::STEP);
    store_stage(0);
  }

  for (int it = 0; it < n_steps; ++it) {
    const int q0 = step_at(it) * C::STEP;
    const bool more = it + 1 < n_steps;
    if (more) load_stage(step_at(it + 1) * C::STEP);
    __syncthreads();   // stage `it` (and K, V) visible; the other buffer's last reads done
    const _Float16* Qs = (const _Float16*)(stages + (it & 1) * C::kStageBytes);
    const _Float16* Gs = Qs + C::kStepTile;
    const float* Ls = (const float*)(Gs + C::kStepTile);
    const float* Ds = Ls + C::STEP;
    const int qw0 = q0 + 32 * qh;              // first query of this wave's half

    // S = Q K^T and dP = dO V^T, 32 queries x this wave's 32 keys (a wave
    // whose queries all precede its keys under the causal mask computes a
    // block of zeros: a branch around it costs more registers than the 2 %
    // of matrix work it would save).
    f32x16 sc = (f32x16){}, dpc = (f32x16){};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const f16x8 qa = *(const f16x8*)(Qs + qrow_off + 16 * ks);
      const f16x8 ka = *(const f16x8*)(Ks + krow_off + 16 * ks);
      const f16x8 ga = *(const f16x8*)(Gs + qrow_off + 16 * ks);
      const f16x8 va = *(const f16x8*)(Vs + krow_off + 16 * ks);
      sc = mfma32h(qa, ka, sc);
      dpc = mfma32h(ga, va, dpc);
    }
    // Keys past N and (causal) keys after the query: P = 0.  The query
    // offset of register r is 8 (r / 4) + 4 lg + r % 4.
    if ((kw0 + 31 >= N) || (CAUSAL && qw0 < kw0 + 31)) {
      const int tl = key_ok ? (CAUSAL ? key - qw0 - 4 * lg : -64) : 64;
#pragma unroll
      for (int r = 0; r < 16; ++r) sc[r] = 8 * (r >> 2) + (r & 3) >= tl ? sc[r] : -INFINITY;
    }
    // P = exp2(s c2 - LSE log2 e), dS = P (dP - D), packed as fp16.
    uint32_t pw[8], dsw[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const f32x4 l4 = *(const f32x4*)(Ls + 32 * qh + 8 * i + 4 * lg);
      const f32x4 d4 = *(const f32x4*)(Ds + 32 * qh + 8 * i + 4 * lg);
      float p[4], ds[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int r = 4 * i + j;
        p[j] = fast_exp2(__builtin_fmaf(sc[r], c2, -l4[j]));
        ds[j] = p[j] * (dpc[r] - d4[j]);
      }
      pw[2 * i] = pack_f16x2(p[0], p[1]);
      pw[2 * i + 1] = pack_f16x2(p[2], p[3]);
      dsw[2 * i] = pack_f16x2(ds[0], ds[1]);
      dsw[2 * i + 1] = pack_f16x2(ds[2], ds[3]);
    }
    // dV^T += dO^T P and dK^T += Q^T dS: the A operands read down the
    // columns in the query order P's accumulator layout leaves in each lane.
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      const f16x8 pb = __builtin_bit_cast(f16x8, ((u32x4){pw[4 * c], pw[4 * c + 1], pw[4 * c + 2], pw[4 * c + 3]}));
      const f16x8 db = __builtin_bit_cast(f16x8, ((u32x4){dsw[4 * c], dsw[4 * c + 1], dsw[4 * c + 2], dsw[4 * c + 3]}));
#pragma unroll
      for (int dm = 0; dm < DM; ++dm) {
        const int lo = (16 * c) * C::kPitch + 32 * dm, hi = (16 * c + 8) * C::kPitch + 32 * dm;
        const f16x8 ga = lds_tr_pair_h(Gs + tr_off, lo, hi);
        const f16x8 qa = lds_tr_pair_h(Qs + tr_off, lo, hi);
        dv_acc[dm] = mfma32h(ga, pb, dv_acc[dm]);
        dk_acc[dm] = mfma32h(qa, db, dk_acc[dm]);
      }
    }
    if (more) store_stage((it + 1) & 1);
  }

  // Sum the two query halves' dK^T and dV^T through LDS (feature-major, so
  // consecutive lanes touch consecutive words), then store dK = scale dK^T
  // and dV = dV^T in the inputs' units as bf16 rows of this lane's key.
  __syncthreads();   // every read of the tile buffers is done
  float* red = (float*)smem_raw;
  auto red_at = [&](int j) { return red + ((size_t)j * 4 + kb) * 64 + lane; };
  if (qh == 1) {
#pragma unroll
    for (int dm = 0; dm < DM; ++dm)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        *red_at(16 * dm + r) = dk_acc[dm][r];
        *red_at(D / 2 + 16 * dm + r) = dv_acc[dm][r];
      }
  }
  __syncthreads();
  if (qh == 0 && key_ok) {
#pragma unroll
    for (int dm = 0; dm < DM; ++dm)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        dk_acc[dm][r] += *red_at(16 * dm + r);
        dv_acc[dm][r] += *red_at(D / 2 + 16 * dm + r);
      }
    const size_t row = ((size_t)bh * N + key) * D;
#pragma unroll
    for (int dm = 0; dm < DM; ++dm)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        u32x2 wk = {pack_bf16x2(dk_acc[dm][4 * i] * dk_fac, dk_acc[dm][4 * i + 1] * dk_fac),
                    pack_bf16x2(dk_acc[dm][4 * i + 2] * dk_fac, dk_acc[dm][4 * i + 3] * dk_fac)};
        u32x2 wv = {pack_bf16x2(dv_acc[dm][4 * i] * dv_fac, dv_acc[dm][4 * i + 1] * dv_fac),
                    pack_bf16x2(dv_acc[dm][4 * i + 2] * dv_fac, dv_acc[dm][4 * i + 3] * dv_fac)};
        *(u32x2*)(dK + row + 32 * dm + 8 * i + 4 * lg) = wk;
        *(u32x2*)(dV + row + 32 * dm + 8 * i + 4 * lg) = wv;
      }
  }
}

// ---------------------------------------------------------------------------
// 4. dQ: one workgroup of 8 waves per 128-query tile of one head.  Wave w
//    owns query block qb = w % 4 and key half kh = w / 4 of each 64-key
//    step.  With the scores transposed (S^T = K Q^T, one query per lane),
//    Q and dO are the B operands (registers), the staged K and V rows the A
//    operands, and dS^T feeds dQ^T += K^T dS^T straight from registers with
//    K^T read transposed in the key order the accumulator leaves.
// SPARSE: the workgroup's 128 queries are one mask row; it visits only the
// 64-key steps whose key block that row keeps.
// ---------------------------------------------------------------------------
template <int D, bool CAUSAL, bool SPARSE>
__global__ void __launch_bounds__(512)
fa_bwd_dq_kernel(const __bf16* __restrict__ Q, const __bf16* __restrict__ K, const __bf16* __restrict__ V,
                 const __bf16* __restrict__ dO, const float* __restrict__ LSE,
                 const float* __restrict__ delta, const float* __restrict__ scales, __bf16* __restrict__ dQ,
                 const uint8_t* __restrict__ bmask, int N, int BH, float scale, float scale_log2) {
  using C = BwdCfg<D>;
  static_assert(C::RES == FA_SPARSE_BLOCK && FA_SPARSE_BLOCK % C::STEP == 0, "sparse blocks vs tiles");
  constexpr int KS = D / 16;
  constexpr int DM = D / 32;
  extern __shared__ __attribute__((aligned(16))) char smem_raw[];
  char* stages = smem_raw;   // the resident rows (Q, dO) live in registers here

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int qb = wave & 3;                   // query block of this wave
  const int kh = wave >> 2;                  // key half of each step
  const int lane = tid & 63;
  const int lc = lane & 31, lg = lane >> 5;
  const int num_qt = (N + C::RES - 1) / C::RES;
  int tile, bh;
  xcd_head_major(blockIdx.x, BH, num_qt, bh, tile);
  const int qt = num_qt - 1 - tile;          // heaviest query tiles first (causal)
  const BwdHead h = bwd_head<D>(Q, K, V, dO, LSE, delta, bh, N);

  const int qw0 = qt * C::RES + qb * 32;     // first query of this wave
  const int q = qw0 + lc;                    // this lane's query
  const float sq = scales[bh * 4 + 0], sg = scales[bh * 4 + 1];
  const float sk = scales[bh * 4 + 2], sv = scales[bh * 4 + 3];
  const float c2 = scale_log2 / (sq * sk);
  const float dq_fac = scale / (sk * sg * sv);

  // Q^T and dO^T as B operands: lane holds 8 features of its query's row.
  f16x8 qbf[KS], gbf[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    const uint32_t off = (uint32_t)(q * D + 16 * ks + 8 * lg) * 2u;
    qbf[ks] = __builtin_bit_cast(f16x8, bf16x8_to_f16x8(bload128(h.q, off), sq));
    gbf[ks] = __builtin_bit_cast(f16x8, bf16x8_to_f16x8(bload128(h.g, off), sg));
  }
  // This lane's LSE * log2 e (+inf past N or for a row that saw no key, so
  // P = 0) and D in the scaled dP's units.
  float lq = INFINITY, dq_d = 0.f;
  if (q < N) {
    const float l = bload32f(h.lse, (uint32_t)q * 4u);
    lq = l == -INFINITY ? INFINITY : l * kLog2e;
    dq_d = bload32f(h.dlt, (uint32_t)q * 4u) * (sg * sv);
  }

  f32x16 dq_acc[DM];
#pragma unroll
  for (int i = 0; i < DM; ++i) dq_acc[i] = (f32x16){};

  const int q_tile_end = min(N, (qt + 1) * C::RES);
  int n_steps = ((CAUSAL ? q_tile_end : N) + C::STEP - 1) / C::STEP;
  int* slist = (int*)(smem_raw + C::kDqLdsTotal);
  if constexpr (SPARSE) {
    const int nb = (N + FA_SPARSE_BLOCK - 1) / FA_SPARSE_BLOCK;
    const uint8_t* row = bmask + ((size_t)bh * nb + qt) * nb;   // this query block's mask row
    if (wave == 0) {
      int cnt = 0;
      for (int base = 0; base < n_steps; base += 64) {
        const int ks_ = base + lane;
        const bool live = ks_ < n_steps && row[ks_ * C::STEP / FA_SPARSE_BLOCK] != 0;
        const uint64_t bal = __ballot(live);
        const int pos = cnt + __builtin_amdgcn_mbcnt_hi((uint32_t)(bal >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)bal, 0));
        if (live) slist[1 + pos] = ks_;
        cnt += __popcll(bal);
      }
      if (lane == 0) slist[0] = cnt;
    }
    __syncthreads();
    n_steps = __builtin_amdgcn_readfirstlane(slist[0]);
  }
  auto step_at = [&](int j) { return SPARSE ? slist[1 + j] : j; };

  const int krow_off = (32 * kh + lc) * C::kPitch + 8 * lg;                 // K / V rows, A operands
  const int tr_off = tr_lane_off(lane, C::kPitch, 4) + 32 * kh * C::kPitch;  // K^T, accumulator key order

  RowPair<D, C::STEP> kv;
  auto stage_k = [&](int buf) { return (_Float16*)(stages + buf * C::kStageBytes); };
  if (n_steps > 0) {
    kv.load(h.k, h.v, step_at(0) * C::STEP, tid);
    kv.store(stage_k(0), stage_k(0) + C::kStepTile, sk, sv, tid);
  }

  for (int it = 0; it < n_steps; ++it) {
    const int kst0 = step_at(it) * C::STEP;
    const bool more = it + 1 < n_steps;
    if (more) kv.load(h.k, h.v, step_at(it + 1) * C::STEP, tid);
    __syncthreads();   // stage `it` visible; the other buffer's last reads done
    const _Float16* Ks = stage_k(it & 1);
    const _Float16* Vs = Ks + C::kStepTile;
    const int kw0 = kst0 + 32 * kh;            // first key of this wave's half

    // S^T = K Q^T and dP^T = V dO^T: this wave's 32 keys x 32 queries.
    f32x16 st = (f32x16){}, dpt = (f32x16){};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const f16x8 ka = *(const f16x8*)(Ks + krow_off + 16 * ks);
      const f16x8 va = *(const f16x8*)(Vs + krow_off + 16 * ks);
      st = mfma32h(ka, qbf[ks], st);
      dpt = mfma32h(va, gbf[ks], dpt);
    }
    // Keys past N and (causal) keys after the query: P = 0.  The key offset
    // of register r is 8 (r / 4) + 4 lg + r % 4.
    if ((kw0 + 31 >= N) || (CAUSAL && kw0 + 31 > qw0)) {
      const int tl = min(N - 1, CAUSAL ? q : N - 1) - kw0 - 4 * lg;
#pragma unroll
      for (int r = 0; r < 16; ++r) st[r] = 8 * (r >> 2) + (r & 3) <= tl ? st[r] : -INFINITY;
    }
    // P^T = exp2(s c2 - LSE log2 e), dS^T = P^T (dP^T - D), packed as fp16
    // (the B operands of dQ^T += K^T dS^T).
    uint32_t dsw[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float p0 = fast_exp2(__builtin_fmaf(st[2 * i], c2, -lq));
      const float p1 = fast_exp2(__builtin_fmaf(st[2 * i + 1], c2, -lq));
      dsw[i] = pack_f16x2(p0 * (dpt[2 * i] - dq_d), p1 * (dpt[2 * i + 1] - dq_d));
    }
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      const f16x8 db = __builtin_bit_cast(f16x8, ((u32x4){dsw[4 * c], dsw[4 * c + 1], dsw[4 * c + 2], dsw[4 * c + 3]}));
#pragma unroll
      for (int dm = 0; dm < DM; ++dm) {
        const int lo = (16 * c) * C::kPitch + 32 * dm, hi = (16 * c + 8) * C::kPitch + 32 * dm;
        const f16x8 ka = lds_tr_pair_h(Ks + tr_off, lo, hi);
        dq_acc[dm] = mfma32h(ka, db, dq_acc[dm]);
      }
    }
    if (more) kv.store(stage_k((it + 1) & 1), stage_k((it + 1) & 1) + C::kStepTile, sk, sv, tid);
  }

  // Sum the two key halves' dQ^T through LDS and store dQ = scale dQ^T in
  // the inputs' units as bf16 rows of this lane's query.
  __syncthreads();
  float* red = (float*)smem_raw;
  auto red_at = [&](int j) { return red + ((size_t)j * 4 + qb) * 64 + lane; };
  if (kh == 1) {
#pragma unroll
    for (int dm = 0; dm < DM; ++dm)
#pragma unroll
      for (int r = 0; r < 16; ++r) *red_at(16 * dm + r) = dq_acc[dm][r];
  }
  __syncthreads();
  if (kh == 0 && q < N) {
    const size_t row = ((size_t)bh * N + q) * D;
#pragma unroll
    for (int dm = 0; dm < DM; ++dm)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float v4[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) v4[j] = (dq_acc[dm][4 * i + j] + *red_at(16 * dm + 4 * i + j)) * dq_fac;
        *(u32x2*)(dQ + row + 32 * dm + 8 * i + 4 * lg) = (u32x2){pack_bf16x2(v4[0], v4[1]), pack_bf16x2(v4[2], v4[3])};
      }
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
  // The sparse kernels keep their list of visited steps (count first) after
  // the other buffers.
  const int list_bytes = SPARSE ? ((4 * ((a.N + C::STEP - 1) / C::STEP + 1) + 15) & ~15) : 0;
  const int lds = C::kLdsTotal + list_bytes;
  const int dq_lds = C::kDqLdsTotal + list_bytes;
  const int num_tiles = (a.N + C::RES - 1) / C::RES;
  if (a.phases & FA_BWD_PREPROCESS) {
    hipLaunchKernelGGL(fa_bwd_prep_kernel<D>, dim3((unsigned)(BH * nch)), dim3(256), 0, a.stream,
                       (const __bf16*)a.o, (const __bf16*)a.dout, (const __bf16*)a.q, (const __bf16*)a.k,
                       (const __bf16*)a.v, a.delta, a.part, a.N, nch);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    hipLaunchKernelGGL(fa_bwd_scales_kernel, dim3((unsigned)((4 * BH + 255) / 256)), dim3(256), 0, a.stream,
                       (const float*)a.part, a.scales, 4 * BH, nch);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  if (a.phases & FA_BWD_MAIN) {
    auto kern = fa_bwd_dkdv_kernel<D, CAUSAL, SPARSE>;
    if ((e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, lds)) != hipSuccess)
      return e;
    hipLaunchKernelGGL(kern, dim3(num_tiles * BH), dim3(C::kThreads), lds, a.stream, (const __bf16*)a.q,
                       (const __bf16*)a.k, (const __bf16*)a.v, (const __bf16*)a.dout, a.lse, a.delta,
                       a.scales, (__bf16*)a.dk, (__bf16*)a.dv, (const uint8_t*)a.bmask, a.N, BH, a.scale,
                       a.scale * kLog2e);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  if (a.phases & FA_BWD_FINALIZE) {
    auto kern = fa_bwd_dq_kernel<D, CAUSAL, SPARSE>;
    if ((e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, dq_lds)) !=
        hipSuccess)
      return e;
    hipLaunchKernelGGL(kern, dim3(num_tiles * BH), dim3(C::kThreads), dq_lds, a.stream, (const __bf16*)a.q,
                       (const __bf16*)a.k, (const __bf16*)a.v, (const __bf16*)a.dout, a.lse, a.delta,
                       a.scales, (__bf16*)a.dq, (const uint8_t*)a.bmask, a.N, BH, a.scale, a.scale * kLog2e);
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
