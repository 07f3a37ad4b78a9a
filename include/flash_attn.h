/*
 * flash_attn.h - exact tiled attention (FlashAttention) on AMD Instinct
 * MI355X (gfx950): the C ABI of libflash_attn.so.
 *
 * What is computed.  For every batch b and head h, with Q, K, V the
 * [N, d] slices of that head,
 *     S = scale * Q K^T          (causal: S_ij = -inf where key j > query i)
 *     P = softmax(S) row by row  (safe softmax: subtract the row max m_i,
 *                                 exponentiate, divide by the row sum l_i)
 *     O = P V,   LSE_i = m_i + ln(l_i)
 * This is the standard attention of "FlashAttention, explained"
 * (vibeengines.com), sections "The math, worked with real numbers" and
 * "Solve it yourself", which divides the scores by sqrt(d); here the factor
 * is the explicit argument `scale`.  The forward kernel walks the keys tile
 * by tile and keeps a running max, a running sum and a rescaled output
 * accumulator per query row (same page, section "Tiling and the online
 * softmax"), so the N x N matrix S is never written to memory; the extra
 * memory is O and LSE only (chorfi.xyz study guide, "Guarantees versus
 * empirical results": extra memory linear in N).  The backward pass
 * recomputes the score tiles from LSE instead of storing P (chorfi.xyz,
 * "Study objectives"; modelfieldguide.com, "An IO-aware rewrite").
 *
 * Conventions shared by every entry point.
 *   - Pointers are device pointers (hipMalloc'd or torch CUDA tensors) owned
 *     by the caller.  The library never allocates or frees device memory.
 *   - Q, K, V, O, dO, dQ, dK, dV are contiguous row-major [B, H, N, d]
 *     (the element of (b, h, n, c) sits at ((b*H + h)*N + n)*d + c) in the
 *     element type `dtype`.  LSE is contiguous [B, H, N] float32.
 *     Base pointers must be 16-byte aligned.  Outputs must not alias inputs.
 *   - Supported: B >= 1, H >= 1, N >= 1 (any N; the tail tile is masked),
 *     d in {64, 128}, finite scale > 0, causal in {0, 1}.  Causal masks key
 *     j > query i, with queries and keys aligned at index 0.
 *   - dtype FA_DTYPE_BF16: bfloat16 storage, fp32 accumulation inside the
 *     kernels, round-to-nearest-even on every narrowing.  FA_DTYPE_FP32:
 *     float32 storage and float32 arithmetic throughout (forward only).
 *   - B*H*N*d must stay below 2^31 elements per tensor
 *     (FA_ERR_INVALID_ARG otherwise), and one head's N*d below 2^30
 *     (FA_ERR_UNSUPPORTED otherwise: inside a head the kernels address
 *     memory with 32-bit byte offsets, the widest being a float32 head of
 *     4*N*d bytes).
 *   - stream is a hipStream_t; NULL means the default stream.  Every call is
 *     asynchronous: it validates its arguments, enqueues kernels on `stream`
 *     and returns.  Faults during execution surface at the caller's next
 *     synchronisation of that stream.
 *   - Errors: arguments are checked before any HIP call; a bad argument
 *     returns FA_ERR_INVALID_ARG or FA_ERR_UNSUPPORTED with nothing enqueued.
 *     A failed launch returns FA_ERR_HIP.  No exception crosses the ABI.
 *   - The functions keep no state between calls and may be called from
 *     several host threads.
 */
#ifndef FLASH_ATTN_H
#define FLASH_ATTN_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

enum fa_status {
    FA_OK = 0,
    FA_ERR_INVALID_ARG = 1,  /* null pointer, non-positive size, bad flag  */
    FA_ERR_UNSUPPORTED = 2,  /* valid request this library does not serve */
    FA_ERR_HIP = 3           /* the HIP runtime rejected a launch          */
};

enum fa_dtype {
    FA_DTYPE_BF16 = 0,
    FA_DTYPE_FP32 = 1
};

/*
 * Forward pass: O = softmax(scale * Q K^T [causal mask]) V and the per-row
 * natural-log LSE, the definition above evaluated by the online-softmax
 * update rule of vibeengines.com "The math, worked with real numbers":
 * m_new = max(m_old, block max); l_new = l_old e^(m_old - m_new) + sum of
 * e^(s - m_new); O_new = O_old e^(m_old - m_new) + sum of e^(s - m_new) V;
 * result O / l.
 *   q, k, v : [B, H, N, d] dtype, read only.
 *   o       : [B, H, N, d] dtype, written.
 *   lse     : [B, H, N] float32, written (may be NULL to skip it).
 * Returns FA_OK, FA_ERR_INVALID_ARG (null q/k/v/o, B/H/N < 1, scale not
 * finite and > 0, causal not 0/1, misaligned pointer, too many elements),
 * FA_ERR_UNSUPPORTED (d not 64/128, unknown dtype) or FA_ERR_HIP.
 */
int flash_attn_fwd(const void* q, const void* k, const void* v,
                   void* o, float* lse,
                   int B, int H, int N, int d,
                   float scale, int causal, int dtype, void* stream);

/*
 * Same as flash_attn_fwd with the key-tile width forced: block_n = 0 picks
 * the default (96 keys per tile for bf16 at d = 128 without a block mask,
 * 64 otherwise), else 32 or 64 keys per tile (bf16 only; the fp32 path
 * accepts 0 or 32).  The result must not depend on it (vibeengines.com,
 * "Solve it yourself": the block size never changes the answer); tests use
 * it to check that.  Other values return FA_ERR_UNSUPPORTED.
 */
int flash_attn_fwd_ex(const void* q, const void* k, const void* v,
                      void* o, float* lse,
                      int B, int H, int N, int d,
                      float scale, int causal, int dtype, void* stream,
                      int block_n);

/*
 * Bytes of device workspace flash_attn_bwd needs, each part rounded up to
 * 256 bytes: D_i = sum_c dO_ic O_ic (fp32 [B, H, N]); the largest |Q|,
 * |dO|, |K|, |V| of every 256-row chunk (fp32 [B, H, ceil(N/256), 4]); four
 * fp32 factors per head; two fp32 row terms per row (LSE log2 e and D in the
 * scaled units); and the scaled fp16 copies of Q, dO, K and V
 * ([B, H, N, d] each): about B*H*N*(8*d + 12) bytes, linear in N.  Returns
 * 0 for invalid sizes.
 */
size_t flash_attn_bwd_workspace_size(int B, int H, int N, int d);

/*
 * Backward pass: gradients of O with respect to Q, K and V for the
 * upstream gradient dO, recomputing each score tile from Q, K and the saved
 * LSE (P = exp(scale * q.k - LSE)) instead of reading a stored P.  The
 * gradient formulas are the calculus of the forward definition:
 *     dV = P^T dO,  dP = dO V^T,  D_i = sum_c dO_ic O_ic,
 *     dS = P * (dP - D),  dQ = scale dS K,  dK = scale dS^T Q.
 * The products run in fp16 with fp32 accumulation.  Q, dO, K and V enter
 * them as fp16 copies (in the workspace) times a power of two per head and
 * tensor that brings the head's largest magnitude into [1, 2); that copy is
 * exact for every value
 * down to 2^-14 of the largest, so S and dP are exact products of the bf16
 * inputs, and P and dS enter dV, dK and dQ rounded to fp16 (11 significant
 * bits).  The factors are divided out in fp32.  Each gradient element is
 * written once, by one workgroup, in a fixed order: results are
 * bit-reproducible.
 *   q, k, v, o, dout : [B, H, N, d] bf16, read only (o, lse from the
 *                      forward pass with the same scale and causal flag;
 *                      D is formed from this bf16 o).
 *   lse              : [B, H, N] float32.
 *   dq, dk, dv       : [B, H, N, d] bf16, written.
 *   workspace        : device buffer of at least
 *                      flash_attn_bwd_workspace_size(B, H, N, d) bytes,
 *                      256-byte aligned, owned by the caller; its contents
 *                      on entry do not matter and are clobbered.
 * dtype must be FA_DTYPE_BF16 (FA_DTYPE_FP32 returns FA_ERR_UNSUPPORTED).
 * Other errors as for flash_attn_fwd, plus FA_ERR_INVALID_ARG for a null
 * or short workspace.
 */
int flash_attn_bwd(const void* q, const void* k, const void* v,
                   const void* o, const void* dout, const float* lse,
                   void* dq, void* dk, void* dv,
                   void* workspace, size_t workspace_bytes,
                   int B, int H, int N, int d,
                   float scale, int causal, int dtype, void* stream);

/*
 * flash_attn_bwd split into its phases, for callers that time or schedule
 * them separately.  `phases` is a bit mask:
 *   FA_BWD_PREPROCESS (1): D_i = sum_c dO_ic O_ic and the chunk maxima,
 *                          then the per-head factors, the row terms and
 *                          the scaled fp16 copies of Q and dO, into the
 *                          workspace (two kernels);
 *   FA_BWD_MAIN       (2): one workgroup per 128-key tile recomputes P and
 *                          dS tile by tile and writes dK and dV, and the
 *                          scaled fp16 copies of K and V into the workspace;
 *   FA_BWD_FINALIZE   (4): one workgroup per 128-query tile recomputes P
 *                          and dS tile by tile and writes dQ.
 * Each phase reads what the phases before it wrote to the workspace.
 * Running the phases in that order, on one stream, with the same arguments
 * and workspace, equals one flash_attn_bwd call (phases = 7).  A mask of 0
 * or with other bits returns FA_ERR_INVALID_ARG.  Other arguments and errors
 * as for flash_attn_bwd.
 */
enum fa_bwd_phase {
    FA_BWD_PREPROCESS = 1,
    FA_BWD_MAIN = 2,
    FA_BWD_FINALIZE = 4,
    FA_BWD_ALL = 7
};

int flash_attn_bwd_ex(const void* q, const void* k, const void* v,
                      const void* o, const void* dout, const float* lse,
                      void* dq, void* dk, void* dv,
                      void* workspace, size_t workspace_bytes,
                      int B, int H, int N, int d,
                      float scale, int causal, int dtype, void* stream,
                      int phases);

/*
 * flash_attn_bwd without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc).  The workspace lives in a static
 * device array of FA_BWD_NOALLOC_MAX_BYTES bytes that the library holds on
 * every GPU it runs on until the process ends; the call allocates nothing
 * and calls no allocating routine.  Shapes whose workspace
 * (flash_attn_bwd_workspace_size) exceeds that size return
 * FA_ERR_UNSUPPORTED; e.g. B*H*N*(8*d + 12) bytes up to 64 MiB, as
 * B2 H16 N2048 d64.  Every call on one GPU uses that GPU's one array, and
 * each call overwrites it: calls that overlap on one GPU (on different
 * streams, or from several host threads, without ordering) race and give
 * wrong gradients; calls ordered on one stream are safe.  Arguments,
 * results and errors as for flash_attn_bwd (all three kernels run).
 */
#define FA_BWD_NOALLOC_MAX_BYTES ((size_t)64 << 20)

int flash_attn_bwd_noalloc(const void* q, const void* k, const void* v,
                           const void* o, const void* dout, const float* lse,
                           void* dq, void* dk, void* dv,
                           int B, int H, int N, int d,
                           float scale, int causal, int dtype, void* stream);

/*
 * Block-sparse attention.  The pages name block-sparse FlashAttention as an
 * approximate extension of the method (chorfi.xyz study guide, "Main
 * concepts to understand"; vibeengines.com lists its Path-256 result among
 * the headline numbers) without defining it.  Here: a block mask over
 * (query block, key block) pairs of FA_SPARSE_BLOCK x FA_SPARSE_BLOCK
 * elements; the scores of every pair whose mask entry is 0 are -inf (weight
 * 0), and the rest is the attention defined above (with the causal mask on
 * top when causal = 1).  A query row left with no key gets O = 0,
 * LSE = -inf, and zero gradients.
 *   block_mask : device pointer to unsigned char [B, H, nb, nb],
 *                nb = ceil(N / FA_SPARSE_BLOCK); entry [b][h][i][j] != 0
 *                keeps the pair (query block i, key block j).  Read only;
 *                the backward call must see the mask the forward saw.
 * Work follows the mask: the forward loads and multiplies only the key
 * tiles that one of a workgroup's two query blocks keeps, the backward only
 * the (key block, 64-query step) pairs the mask keeps.
 * bf16 only (FA_DTYPE_FP32 returns FA_ERR_UNSUPPORTED); N <= 65536 (the
 * per-workgroup list of visited tiles lives in LDS), else
 * FA_ERR_UNSUPPORTED.  Other arguments, errors and conventions as for
 * flash_attn_fwd / flash_attn_bwd; a null block_mask is FA_ERR_INVALID_ARG.
 */
#define FA_SPARSE_BLOCK 128
#define FA_SPARSE_MAX_N 65536

int flash_attn_fwd_blocksparse(const void* q, const void* k, const void* v,
                               void* o, float* lse, const unsigned char* block_mask,
                               int B, int H, int N, int d,
                               float scale, int causal, int dtype, void* stream);

int flash_attn_bwd_blocksparse(const void* q, const void* k, const void* v,
                               const void* o, const void* dout, const float* lse,
                               const unsigned char* block_mask,
                               void* dq, void* dk, void* dv,
                               void* workspace, size_t workspace_bytes,
                               int B, int H, int N, int d,
                               float scale, int causal, int dtype, void* stream);

/*
 * Decoding with a key/value cache (split-KV).  The pages ask which parts of
 * the speed-up carry over to autoregressive decoding with a KV cache
 * (chorfi.xyz study guide, "Discussion prompts").  Here: Nq new queries per
 * head (1 <= Nq <= FA_DECODE_MAX_Q) attend to an Nk-entry cache
 * (Nq <= Nk); they are the cache's last Nq positions, so with causal = 1
 * query i sees keys j <= Nk - Nq + i, and with causal = 0 every key.  The
 * keys are split across waves; each split runs the online-softmax rule of
 * the forward pass and the splits are merged with the same rule.
 *   q        : [B, H, Nq, d] bf16.   k, v : [B, H, Nk, d] bf16 (the cache).
 *   o        : [B, H, Nq, d] bf16, written.   lse : [B, H, Nq] fp32 or NULL.
 *   workspace: at least flash_attn_decode_workspace_size(B, H, Nk, d) bytes,
 *              256-byte aligned (per-split partial results), clobbered.
 * bf16 only; d in {64, 128}; B*H*Nk*d below 2^31 and Nk*d below 2^30.  Errors as for
 * flash_attn_fwd, plus FA_ERR_UNSUPPORTED for Nq > FA_DECODE_MAX_Q and
 * FA_ERR_INVALID_ARG for Nq > Nk or a null or short workspace.
 */
#define FA_DECODE_MAX_Q 16

size_t flash_attn_decode_workspace_size(int B, int H, int Nk, int d);

int flash_attn_decode(const void* q, const void* k, const void* v,
                      void* o, float* lse,
                      void* workspace, size_t workspace_bytes,
                      int B, int H, int Nq, int Nk, int d,
                      float scale, int causal, int dtype, void* stream);

/*
 * FP8 forward.  The pages list FP8 support as part of FlashAttention-3's
 * rebuild for newer hardware (vibeengines.com, "FlashAttention, explained",
 * section "Why it still matters") without defining it.  Here: Q, K and V are
 * stored as 8-bit E4M3 codes (OCP 8-bit floating point, E4M3 variant: sign,
 * 4 exponent bits with bias 7, 3 mantissa bits, no infinities, codes 0x7F
 * and 0xFF are NaN, largest finite value 448), one byte per element in the
 * [B, H, N, d] layout, each tensor with one float descale factor: the value
 * of a Q element is e4m3(code) * q_descale, likewise for K and V.  The
 * result is the attention defined above of those values, O in bf16 and LSE
 * in fp32.  Both products run on the FP8 matrix cores; the probabilities
 * enter the second product rounded to E4M3, so O carries that rounding (a
 * relative error of up to 2^-4 per probability); LSE does not.
 *   q, k, v      : [B, H, N, d] E4M3 codes, read only.
 *   *_descale    : finite and > 0.
 *   o            : [B, H, N, d] bf16, written.   lse : [B, H, N] fp32 or NULL.
 * Errors as for flash_attn_fwd (a descale that is not finite and > 0 is
 * FA_ERR_INVALID_ARG); d in {64, 128}.
 */
int flash_attn_fwd_fp8(const void* q, const void* k, const void* v,
                       float q_descale, float k_descale, float v_descale,
                       void* o, float* lse,
                       int B, int H, int N, int d,
                       float scale, int causal, void* stream);

/*
 * Merge of two partial attention results over disjoint sets of keys, the
 * online-softmax update rule of vibeengines.com "FlashAttention, explained"
 * ("Tiling and the online softmax") applied to whole blocks in LSE form:
 *     L = ln(e^La + e^Lb),   O = e^(La - L) Oa + e^(Lb - L) Ob,
 * row by row.  It is the step a sequence-parallel (ring) schedule repeats
 * as key/value chunks visit the device that holds some query rows: each
 * chunk's forward result (O, LSE from flash_attn_fwd) is folded into a
 * running result.  Start the running result at o_acc = 0, lse_acc = -inf.
 * A row with LSE = -inf on both sides (no key yet) stays 0 / -inf.
 *   o_acc    : float32 [rows, d], read and written (the running output).
 *   lse_acc  : float32 [rows], read and written.
 *   o_part   : bf16 [rows, d], read.   lse_part : float32 [rows], read.
 *   o_out    : bf16 [rows, d], written with the merged output (may be NULL).
 *   rows     : number of rows (B * H * N for [B, H, N, d] tensors).
 * d in {64, 128} (else FA_ERR_UNSUPPORTED); null inputs, rows < 1,
 * rows * d >= 2^31 or a misaligned o_acc / o_part / o_out give
 * FA_ERR_INVALID_ARG.  o_out must not alias the inputs.
 */
int flash_attn_merge(float* o_acc, float* lse_acc, const void* o_part, const float* lse_part,
                     void* o_out, long long rows, int d, void* stream);

/*
 * Compute units and peak clock (kHz) of HIP device `device`, for reporting
 * peaks (dense bf16 MFMA: units x clock x 4096 FLOP per cycle on gfx950).
 * A HIP call; FA_ERR_INVALID_ARG for null outputs or a negative device,
 * FA_ERR_HIP if the runtime refuses.
 */
int flash_attn_device_info(int device, int* cu_count, int* clock_khz);

/* Static, never-NULL description of a status code (unknown codes included). */
const char* flash_attn_status_string(int status);

/* Text of the last HIP error seen by a call on this host thread ("" if none). */
const char* flash_attn_last_hip_error(void);

#ifdef __cplusplus
}
#endif

#endif /* FLASH_ATTN_H */
