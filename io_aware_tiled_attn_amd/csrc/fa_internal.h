// Internal interface between the C-ABI entry points (fa_api.cpp) and the
// kernel launchers.  Arguments reaching these functions are validated.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>

#include "../../include/flash_attn.h"

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
  float* dq_acc;   // workspace: fp32 [B, H, N, d]
  float* delta;    // workspace: fp32 [B, H, N]
  int B, H, N, d;
  float scale;
  int causal;
  int phases;     // FA_BWD_* mask
  hipStream_t stream;
  const unsigned char* bmask;   // block-sparse mask [B, H, nb, nb], or null (dense)
};

hipError_t launch_fwd(const FwdArgs& a);
hipError_t launch_bwd(const BwdArgs& a);

}  // namespace fa
