// Merge of two partial attention results over disjoint sets of keys.
//
// The online-softmax update rule (vibeengines.com "FlashAttention, explained",
// section "Tiling and the online softmax") folds a new block of keys into a
// running (m, l, O); applied to whole blocks whose results are carried as
// (O = normalised output, LSE = m + ln l), it reads
//     L = ln(e^La + e^Lb),   O = e^(La - L) Oa + e^(Lb - L) Ob.
// This is the step a sequence-parallel ring repeats as key/value chunks
// visit a device holding some query rows (the long-context use the same page
// draws from linear memory, section "Worth knowing"): each visiting chunk's
// forward result is folded into the running one.  The running O is kept in
// fp32; each partial O comes from the bf16 forward.
//
// One thread per 8 features of a row (d / 8 threads per row, all in one
// wave, so every lane of a row reads the row's LSE before one lane writes it).
#include "fa_common.h"
#include "fa_internal.h"

namespace fa {

template <int D>
__global__ void __launch_bounds__(256)
fa_merge_kernel(float* __restrict__ o_acc, float* __restrict__ lse_acc, const __bf16* __restrict__ o_part,
                const float* __restrict__ lse_part, __bf16* __restrict__ o_out, long rows) {
  constexpr int TPR = D / 8;          // threads per row
  constexpr int RPB = 256 / TPR;      // rows per block
  static_assert(64 % TPR == 0, "a row's threads share one wave");
  const long row = (long)blockIdx.x * RPB + threadIdx.x / TPR;
  const int part = threadIdx.x % TPR;
  if (row >= rows) return;
  const float la = lse_acc[row], lb = lse_part[row];
  const float m = fmaxf(la, lb);
  float wa = 1.f, wb = 0.f, L = -INFINITY;   // no key on either side: keep the zeros
  if (m != -INFINITY) {
    wa = __expf(la - m);
    wb = __expf(lb - m);
    const float s = wa + wb;
    L = m + __logf(s);
    wa /= s;
    wb /= s;
  }
  float* oa = o_acc + row * D + part * 8;
  const u32x4 ob = *(const u32x4*)(o_part + row * D + part * 8);
  f32x4 a0 = *(const f32x4*)oa, a1 = *(const f32x4*)(oa + 4);
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    a0[2 * i] = wa * a0[2 * i] + wb * bf16_lo(ob[i]);
    a0[2 * i + 1] = wa * a0[2 * i + 1] + wb * bf16_hi(ob[i]);
    a1[2 * i] = wa * a1[2 * i] + wb * bf16_lo(ob[2 + i]);
    a1[2 * i + 1] = wa * a1[2 * i + 1] + wb * bf16_hi(ob[2 + i]);
  }
  *(f32x4*)oa = a0;
  *(f32x4*)(oa + 4) = a1;
  if (o_out != nullptr) {
    const u32x4 w = {pack_bf16x2(a0[0], a0[1]), pack_bf16x2(a0[2], a0[3]), pack_bf16x2(a1[0], a1[1]),
                     pack_bf16x2(a1[2], a1[3])};
    *(u32x4*)(o_out + row * D + part * 8) = w;
  }
  if (part == 0) lse_acc[row] = L;
}

hipError_t launch_merge(const MergeArgs& a) {
  const int tpr = a.d / 8;
  const long rpb = 256 / tpr;
  const dim3 grid((unsigned)((a.rows + rpb - 1) / rpb));
  if (a.d == 64)
    hipLaunchKernelGGL(fa_merge_kernel<64>, grid, dim3(256), 0, a.stream, a.o_acc, a.lse_acc,
                       (const __bf16*)a.o_part, a.lse_part, (__bf16*)a.o_out, a.rows);
  else
    hipLaunchKernelGGL(fa_merge_kernel<128>, grid, dim3(256), 0, a.stream, a.o_acc, a.lse_acc,
                       (const __bf16*)a.o_part, a.lse_part, (__bf16*)a.o_out, a.rows);
  return hipGetLastError();
}

}  // namespace fa
