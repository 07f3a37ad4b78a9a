// Internal interface between the C-ABI entry points (fa_api.cpp) and the
// kernel launchers.  Arguments reaching these functions are validated.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>

#include "../../include/flash_attn.h"
#include "fa_layout.h"

namespace fa {

struct FwdArgs {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  int B, H, N, d;
  float scale;
  int causal;
  int dtype;
  int block_n;   // 0 = default
  hipStream_t stream;
  const unsigned char* bmask;   // block-sparse mask [B, H, nb, nb], or null (dense)
};

struct FwdFp8Args {
  const void* q;   // E4M3 codes [B, H, N, d]
  const void* k;
  const void* v;
  float q_descale, k_descale, v_descale;
  void* o;         // bf16 [B, H, N, d]
  float* lse;      // [B, H, N] or null
  int B, H, N, d;
  float scale;
  int causal;
  hipStream_t stream;
};

// Work layout of a forward launch of `kern` over num_qt query tiles x BH
// heads, from the workgroups one XCD runs at once (occupancy x compute
// units / 8 XCDs): hg, the heads per XCD group (layout::xcd_head_groups;
// 0 when BH is not a multiple of 8), and wpx, the workgroups per XCD of a
// persistent launch (layout::persistent_item; 0 for one workgroup per item,
// the launch used when hg is 0).
inline hipError_t forward_work_layout(const void* kern, int threads, int lds, int BH, int num_qt, int* hg,
                                      int* wpx) {
  *hg = 0;
  *wpx = 0;
  if (BH % 8 != 0) return hipSuccess;
  int occ = 0, dev = 0, cus = 0;
  hipError_t e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, kern, threads, (size_t)lds);
  if (e == hipSuccess) e = hipGetDevice(&dev);
  if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return e;
  const int resident = occ * cus / 8;
  *hg = layout::head_group_size(resident, BH, num_qt);
  const int items = BH / 8 * num_qt;
  *wpx = resident < 1 ? 0 : (resident < items ? resident : items);
  return hipSuccess;
}

// Workgroups per XCD of a persistent launch of `kern` over BH heads x
// tiles_per_head items (layout::persistent_item over each XCD's
// head-major list): as many as one XCD runs at once, at most its items; 0
// (one workgroup per item) when BH is not a multiple of 8.
inline hipError_t persistent_width(const void* kern, int threads, int lds, int BH, int tiles_per_head, int* wpx) {
  *wpx = 0;
  if (BH % 8 != 0) return hipSuccess;
  int occ = 0, dev = 0, cus = 0;
  hipError_t e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, kern, threads, (size_t)lds);
  if (e == hipSuccess) e = hipGetDevice(&dev);
  if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return e;
  const int resident = occ * cus / 8, items = BH / 8 * tiles_per_head;
  *wpx = resident < 1 ? 0 : (resident < items ? resident : items);
  return hipSuccess;
}

// Rows of one head that one preprocessing workgroup covers.
constexpr int kBwdChunkRows = 256;

// The backward workspace, in this order, each part 256-byte aligned:
//   delta   fp32 [B, H, N]       D_i = sum_c dO_ic O_ic
//   part    fp32 [B, H, nch, 4]  largest |Q|, |dO|, |K|, |V| of each 256-row chunk
//   scales  fp32 [B, H, 4]       per-head power-of-two factors of Q, dO, K, V
//   rowterm fp32 [B, H, 2, N]    per head two planes of per-row start values
//                                of the main kernels' accumulators: S at
//                                -LSE log2 e / c2 (-inf for a row that saw no
//                                key), dP at -D times the dO and V factors
//   q16, do16, k16, v16          fp16 [B, H, N, d] each: the inputs times their factors
struct BwdWorkspace {
  size_t delta, part, scales, rowterm, q16, do16, k16, v16, total;
};
inline BwdWorkspace bwd_workspace_layout(int B, int H, int N, int d) {
  auto al = [](size_t x) { return (x + 255) & ~(size_t)255; };
  const size_t bh = (size_t)B * H, rows = bh * N;
  const size_t nch = ((size_t)N + kBwdChunkRows - 1) / kBwdChunkRows;
  BwdWorkspace w;
  size_t o = 0;
  w.delta = o;   o += al(rows * 4);
  w.part = o;    o += al(bh * nch * 4 * 4);
  w.scales = o;  o += al(bh * 4 * 4);
  w.rowterm = o; o += al(rows * 8);
  w.q16 = o;     o += al(rows * d * 2);
  w.do16 = o;    o += al(rows * d * 2);
  w.k16 = o;     o += al(rows * d * 2);
  w.v16 = o;     o += al(rows * d * 2);
  w.total = o;
  return w;
}

struct BwdArgs {
  const void* q;
  const void* k;
  const void* v;
  const void* o;
  const void* dout;
  const float* lse;
  void* dq;
  void* dk;
  void* dv;
  float* delta;    // workspace parts (bwd_workspace_layout)
  float* part;
  float* scales;
  float* rowterm;
  void* q16;
  void* do16;
  void* k16;
  void* v16;
  int B, H, N, d;
  float scale;
  int causal;
  int phases;     // FA_BWD_* mask
  hipStream_t stream;
  const unsigned char* bmask;   // block-sparse mask [B, H, nb, nb], or null (dense)
};

struct DecodeArgs {
  const void* q;   // [B, H, Nq, d]
  const void* k;   // [B, H, Nk, d]
  const void* v;
  void* o;         // [B, H, Nq, d]
  float* lse;      // [B, H, Nq] or null
  float* part_o;   // workspace: fp32 [B*H*splits, 16, d]
  float* part_lse; // workspace: fp32 [B*H*splits, 16]
  int B, H, Nq, Nk, d;
  float scale;
  int causal;
  hipStream_t stream;
};

struct MergeArgs {
  float* o_acc;          // fp32 [rows, d], in/out
  float* lse_acc;        // fp32 [rows], in/out
  const void* o_part;    // bf16 [rows, d]
  const float* lse_part; // fp32 [rows]
  void* o_out;           // bf16 [rows, d] or null
  long rows;
  int d;
  hipStream_t stream;
};

hipError_t launch_fwd(const FwdArgs& a);
hipError_t launch_merge(const MergeArgs& a);
hipError_t launch_fwd_fp8(const FwdFp8Args& a);
hipError_t launch_bwd(const BwdArgs& a);
// This device's address of the static backward scratch
// (FA_BWD_NOALLOC_MAX_BYTES bytes, 256-byte aligned).
hipError_t bwd_scratch_address(void** ptr);
hipError_t launch_decode(const DecodeArgs& a);
size_t decode_workspace_bytes(int B, int H, int Nk, int d);   // valid sizes only
float* decode_part_lse(float* part_o, int B, int H, int Nk, int d);   // LSE part of the workspace

}  // namespace fa
