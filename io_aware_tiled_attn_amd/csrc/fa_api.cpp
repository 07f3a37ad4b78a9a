// C-ABI entry points of libflash_attn.so: argument validation (no HIP call
// before it passes), dispatch to the kernel launchers, status reporting.
#include <cmath>
#include <cstdint>
#include <cstring>

#include "fa_internal.h"

namespace {

thread_local char g_last_hip_error[256] = "";

int hip_status(hipError_t e) {
  if (e == hipSuccess) return FA_OK;
  const char* s = hipGetErrorString(e);
  std::strncpy(g_last_hip_error, s ? s : "unknown HIP error", sizeof(g_last_hip_error) - 1);
  g_last_hip_error[sizeof(g_last_hip_error) - 1] = '\0';
  return FA_ERR_HIP;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Largest element count of one [B, H, N, d] tensor the kernels index with
// 32-bit row arithmetic inside a head and 64-bit offsets across heads.
constexpr long long kMaxElems = (1LL << 31) - 1;
// Inside one head the kernels use 32-bit byte offsets and buffer-descriptor
// sizes; the widest is a float32 tensor's head, 4 N d bytes, so one head's
// N d must stay below 2^30 (which also keeps a tile read past the
// head's end, (N + 256) d bf16 elements, inside 32 bits).
constexpr long long kMaxHeadElems = (1LL << 30) - 1;

int check_sizes(int B, int H, int N, int d, float scale, int causal) {
  if (B < 1 || H < 1 || N < 1 || d < 1) return FA_ERR_INVALID_ARG;
  if (!std::isfinite(scale) || !(scale > 0.f)) return FA_ERR_INVALID_ARG;
  if (causal != 0 && causal != 1) return FA_ERR_INVALID_ARG;
  if ((long long)B * H * N * d > kMaxElems) return FA_ERR_INVALID_ARG;
  if (d != 64 && d != 128) return FA_ERR_UNSUPPORTED;
  if ((long long)N * d > kMaxHeadElems) return FA_ERR_UNSUPPORTED;
  return FA_OK;
}

int fwd_impl(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int N, int d,
             float scale, int causal, int dtype, void* stream, int block_n,
             const unsigned char* bmask = nullptr) {
  if (!q || !k || !v || !o) return FA_ERR_INVALID_ARG;
  int st = check_sizes(B, H, N, d, scale, causal);
  if (st != FA_OK) return st;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || (lse && !aligned16(lse)))
    return FA_ERR_INVALID_ARG;
  if (dtype != FA_DTYPE_BF16 && dtype != FA_DTYPE_FP32) return FA_ERR_UNSUPPORTED;
  if (dtype == FA_DTYPE_BF16 && block_n != 0 && block_n != 32 && block_n != 64)
    return FA_ERR_UNSUPPORTED;
  if (dtype == FA_DTYPE_FP32 && block_n != 0 && block_n != 32) return FA_ERR_UNSUPPORTED;
  fa::FwdArgs a{q, k, v, o, lse, B, H, N, d, scale, causal, dtype, block_n, (hipStream_t)stream, bmask};
  return hip_status(fa::launch_fwd(a));
}

int bwd_impl(const void* q, const void* k, const void* v, const void* o, const void* dout, const float* lse,
             void* dq, void* dk, void* dv, void* workspace, size_t workspace_bytes, int B, int H, int N, int d,
             float scale, int causal, int dtype, void* stream, int phases, const unsigned char* bmask) {
  if (!q || !k || !v || !o || !dout || !lse || !dq || !dk || !dv || !workspace) return FA_ERR_INVALID_ARG;
  if (phases <= 0 || (phases & ~FA_BWD_ALL) != 0) return FA_ERR_INVALID_ARG;
  int st = check_sizes(B, H, N, d, scale, causal);
  if (st != FA_OK) return st;
  const void* ptrs[] = {q, k, v, o, dout, lse, dq, dk, dv};
  for (const void* p : ptrs)
    if (!aligned16(p)) return FA_ERR_INVALID_ARG;
  if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0) return FA_ERR_INVALID_ARG;
  if (dtype != FA_DTYPE_BF16) return FA_ERR_UNSUPPORTED;
  const size_t need = flash_attn_bwd_workspace_size(B, H, N, d);
  if (workspace_bytes < need) return FA_ERR_INVALID_ARG;
  const fa::BwdWorkspace w = fa::bwd_workspace_layout(B, H, N, d);
  char* ws = static_cast<char*>(workspace);
  fa::BwdArgs a{q, k, v, o, dout, lse, dq, dk, dv,
                reinterpret_cast<float*>(ws + w.delta), reinterpret_cast<float*>(ws + w.part),
                reinterpret_cast<float*>(ws + w.scales), reinterpret_cast<float*>(ws + w.rowterm),
                ws + w.q16, ws + w.do16, ws + w.k16, ws + w.v16,
                B, H, N, d, scale, causal, phases, (hipStream_t)stream, bmask};
  return hip_status(fa::launch_bwd(a));
}

// The block-sparse entry points: the dense checks plus the mask pointer,
// bf16 and the length limit of the LDS tile lists.
int sparse_checks(const unsigned char* bmask, int N, int d, int dtype) {
  if (!bmask) return FA_ERR_INVALID_ARG;
  if (N < 1 || d < 1) return FA_ERR_INVALID_ARG;
  if (dtype != FA_DTYPE_BF16) return FA_ERR_UNSUPPORTED;
  if (N > FA_SPARSE_MAX_N) return FA_ERR_UNSUPPORTED;
  return FA_OK;
}

}  // namespace

extern "C" {

int flash_attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int N, int d,
                   float scale, int causal, int dtype, void* stream) {
  return fwd_impl(q, k, v, o, lse, B, H, N, d, scale, causal, dtype, stream, 0);
}

int flash_attn_fwd_ex(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int N,
                      int d, float scale, int causal, int dtype, void* stream, int block_n) {
  return fwd_impl(q, k, v, o, lse, B, H, N, d, scale, causal, dtype, stream, block_n);
}

int flash_attn_fwd_fp8(const void* q, const void* k, const void* v, float q_descale, float k_descale,
                       float v_descale, void* o, float* lse, int B, int H, int N, int d, float scale, int causal,
                       void* stream) {
  if (!q || !k || !v || !o) return FA_ERR_INVALID_ARG;
  const float ds[] = {q_descale, k_descale, v_descale};
  for (float x : ds)
    if (!std::isfinite(x) || !(x > 0.f)) return FA_ERR_INVALID_ARG;
  int st = check_sizes(B, H, N, d, scale, causal);
  if (st != FA_OK) return st;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || (lse && !aligned16(lse)))
    return FA_ERR_INVALID_ARG;
  fa::FwdFp8Args a{q, k, v, q_descale, k_descale, v_descale, o, lse, B, H, N, d, scale, causal,
                   (hipStream_t)stream};
  return hip_status(fa::launch_fwd_fp8(a));
}

int flash_attn_merge(float* o_acc, float* lse_acc, const void* o_part, const float* lse_part, void* o_out,
                     long long rows, int d, void* stream) {
  if (!o_acc || !lse_acc || !o_part || !lse_part) return FA_ERR_INVALID_ARG;
  if (rows < 1 || d < 1 || rows * d > kMaxElems) return FA_ERR_INVALID_ARG;
  if (d != 64 && d != 128) return FA_ERR_UNSUPPORTED;
  if (!aligned16(o_acc) || !aligned16(o_part) || (o_out && !aligned16(o_out))) return FA_ERR_INVALID_ARG;
  fa::MergeArgs a{o_acc, lse_acc, o_part, lse_part, o_out, (long)rows, d, (hipStream_t)stream};
  return hip_status(fa::launch_merge(a));
}

int flash_attn_device_info(int device, int* cu_count, int* clock_khz) {
  if (!cu_count || !clock_khz || device < 0) return FA_ERR_INVALID_ARG;
  hipError_t e = hipDeviceGetAttribute(cu_count, hipDeviceAttributeMultiprocessorCount, device);
  if (e == hipSuccess) e = hipDeviceGetAttribute(clock_khz, hipDeviceAttributeClockRate, device);
  return hip_status(e);
}

size_t flash_attn_bwd_workspace_size(int B, int H, int N, int d) {
  if (B < 1 || H < 1 || N < 1 || d < 1) return 0;
  if ((long long)B * H * N * d > kMaxElems) return 0;
  return fa::bwd_workspace_layout(B, H, N, d).total;
}

int flash_attn_bwd_ex(const void* q, const void* k, const void* v, const void* o, const void* dout,
                      const float* lse, void* dq, void* dk, void* dv, void* workspace, size_t workspace_bytes, int B,
                      int H, int N, int d, float scale, int causal, int dtype, void* stream, int phases) {
  return bwd_impl(q, k, v, o, dout, lse, dq, dk, dv, workspace, workspace_bytes, B, H, N, d, scale, causal, dtype,
                  stream, phases, nullptr);
}

int flash_attn_bwd(const void* q, const void* k, const void* v, const void* o, const void* dout, const float* lse,
                   void* dq, void* dk, void* dv, void* workspace, size_t workspace_bytes, int B, int H, int N, int d,
                   float scale, int causal, int dtype, void* stream) {
  return flash_attn_bwd_ex(q, k, v, o, dout, lse, dq, dk, dv, workspace, workspace_bytes, B, H, N, d, scale, causal,
                           dtype, stream, FA_BWD_ALL);
}

int flash_attn_bwd_noalloc(const void* q, const void* k, const void* v, const void* o, const void* dout,
                           const float* lse, void* dq, void* dk, void* dv, int B, int H, int N, int d, float scale,
                           int causal, int dtype, void* stream) {
  // The same checks as flash_attn_bwd (a stand-in workspace pointer passes
  // the workspace checks), before any HIP call.
  const void* ws_check = reinterpret_cast<const void*>(uintptr_t{256});
  if (!q || !k || !v || !o || !dout || !lse || !dq || !dk || !dv) return FA_ERR_INVALID_ARG;
  int st = check_sizes(B, H, N, d, scale, causal);
  if (st != FA_OK) return st;
  const void* ptrs[] = {q, k, v, o, dout, lse, dq, dk, dv, ws_check};
  for (const void* p : ptrs)
    if (!aligned16(p)) return FA_ERR_INVALID_ARG;
  if (dtype != FA_DTYPE_BF16) return FA_ERR_UNSUPPORTED;
  if (flash_attn_bwd_workspace_size(B, H, N, d) > FA_BWD_NOALLOC_MAX_BYTES) return FA_ERR_UNSUPPORTED;
  void* scratch = nullptr;
  const hipError_t e = fa::bwd_scratch_address(&scratch);
  if (e != hipSuccess) return hip_status(e);
  return bwd_impl(q, k, v, o, dout, lse, dq, dk, dv, scratch, FA_BWD_NOALLOC_MAX_BYTES, B, H, N, d, scale, causal,
                  dtype, stream, FA_BWD_ALL, nullptr);
}

int flash_attn_fwd_blocksparse(const void* q, const void* k, const void* v, void* o, float* lse,
                               const unsigned char* block_mask, int B, int H, int N, int d, float scale, int causal,
                               int dtype, void* stream) {
  if (!q || !k || !v || !o) return FA_ERR_INVALID_ARG;
  int st = check_sizes(B, H, N, d, scale, causal);
  if (st == FA_OK) st = sparse_checks(block_mask, N, d, dtype);
  if (st != FA_OK) return st;
  return fwd_impl(q, k, v, o, lse, B, H, N, d, scale, causal, dtype, stream, 0, block_mask);
}

int flash_attn_bwd_blocksparse(const void* q, const void* k, const void* v, const void* o, const void* dout,
                               const float* lse, const unsigned char* block_mask, void* dq, void* dk, void* dv,
                               void* workspace, size_t workspace_bytes, int B, int H, int N, int d, float scale,
                               int causal, int dtype, void* stream) {
  if (!q || !k || !v || !o || !dout || !lse || !dq || !dk || !dv || !workspace) return FA_ERR_INVALID_ARG;
  int st = check_sizes(B, H, N, d, scale, causal);
  if (st == FA_OK) st = sparse_checks(block_mask, N, d, dtype);
  if (st != FA_OK) return st;
  return bwd_impl(q, k, v, o, dout, lse, dq, dk, dv, workspace, workspace_bytes, B, H, N, d, scale, causal, dtype,
                  stream, FA_BWD_ALL, block_mask);
}

size_t flash_attn_decode_workspace_size(int B, int H, int Nk, int d) {
  if (B < 1 || H < 1 || Nk < 1 || (d != 64 && d != 128)) return 0;
  if ((long long)B * H * Nk * d > kMaxElems) return 0;
  return fa::decode_workspace_bytes(B, H, Nk, d);
}

int flash_attn_decode(const void* q, const void* k, const void* v, void* o, float* lse, void* workspace,
                      size_t workspace_bytes, int B, int H, int Nq, int Nk, int d, float scale, int causal, int dtype,
                      void* stream) {
  if (!q || !k || !v || !o || !workspace) return FA_ERR_INVALID_ARG;
  if (B < 1 || H < 1 || Nq < 1 || Nk < 1 || d < 1) return FA_ERR_INVALID_ARG;
  if (!std::isfinite(scale) || !(scale > 0.f)) return FA_ERR_INVALID_ARG;
  if (causal != 0 && causal != 1) return FA_ERR_INVALID_ARG;
  if ((long long)B * H * Nk * d > kMaxElems) return FA_ERR_INVALID_ARG;
  if (Nq > Nk) return FA_ERR_INVALID_ARG;
  if (d != 64 && d != 128) return FA_ERR_UNSUPPORTED;
  if ((long long)Nk * d > kMaxHeadElems) return FA_ERR_UNSUPPORTED;
  if (Nq > FA_DECODE_MAX_Q) return FA_ERR_UNSUPPORTED;
  if (dtype != FA_DTYPE_BF16) return FA_ERR_UNSUPPORTED;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || (lse && !aligned16(lse)))
    return FA_ERR_INVALID_ARG;
  if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0) return FA_ERR_INVALID_ARG;
  const size_t need = fa::decode_workspace_bytes(B, H, Nk, d);
  if (workspace_bytes < need) return FA_ERR_INVALID_ARG;
  // Layout: partial O (256-byte aligned), then partial LSE.
  float* part_o = static_cast<float*>(workspace);
  fa::DecodeArgs a{q, k, v, o, lse, part_o, nullptr, B, H, Nq, Nk, d, scale, causal, (hipStream_t)stream};
  a.part_lse = fa::decode_part_lse(part_o, B, H, Nk, d);
  return hip_status(fa::launch_decode(a));
}

const char* flash_attn_status_string(int status) {
  switch (status) {
    case FA_OK: return "ok";
    case FA_ERR_INVALID_ARG: return "invalid argument";
    case FA_ERR_UNSUPPORTED: return "unsupported configuration";
    case FA_ERR_HIP: return "HIP runtime error";
    default: return "unknown status";
  }
}

const char* flash_attn_last_hip_error(void) { return g_last_hip_error; }

}  // extern "C"
