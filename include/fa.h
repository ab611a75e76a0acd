/*
 * fa.h — C ABI of the MI355X (gfx950) exact-attention library, libfa.so: the forward pass
 * (fa_fwd) and its gradients (fa_bwd).
 *
 * The operation (FlashAttention forward) is the standard scaled-dot-product
 * attention the pages start from — "PyTorch Transformer Flash Attention机制：
 * 内存访问优化与CUDA Kernel融合的底层实现" (zyxy.net), section 1, and
 * "FlashAttention算法原理与性能优化实战" (intelliparadigm), section 1.1 —
 * computed tile by tile with the online-softmax recurrence ("Flash Attention
 * 是怎么做到又快又省显存的？", cnblogs, section 时间复杂度) in the FA2 loop order
 * and grid (Triton FA2 walkthrough, xrbh.cn), so the N x N score matrix never
 * reaches device memory. For every batch b, query head hq and query row i:
 *
 *   S_ij   = scale * sum_c Q[b,hq,i,c] * K[b,hkv,j,c],   hkv = hq / (Hq / Hkv)
 *   keys j visible to row i: all j < N, or only j <= i when causal
 *   O[b,hq,i,:] = sum_j softmax_j(S_i.) * V[b,hkv,j,:]
 *   lse[b,hq,i] = ln sum_j exp(S_ij)          (natural log, over visible j)
 *
 * The per-row log-sum-exp is the statistic a backward pass recomputes the
 * probabilities from (intelliparadigm page, section 1.2.3; the FA2
 * walkthrough's logsumexp L). Grouped-query attention follows the
 * intelliparadigm page, section 1.3: query heads are grouped consecutively,
 * G = Hq / Hkv query heads per K/V head.
 *
 * Layout: every tensor is dense and row-major in the [batch, head, seq, dim]
 * order of the zyxy.net page's section 1 (B, H, L, D):
 *   q  [B][Hq ][N][d]   in_dtype
 *   k  [B][Hkv][N][d]   in_dtype
 *   v  [B][Hkv][N][d]   in_dtype
 *   o  [B][Hq ][N][d]   out_dtype
 *   lse[B][Hq ][N]      float32
 *
 * Ownership: all five pointers are device pointers owned by the caller (for
 * example from PyTorch). The library allocates no device memory, takes no
 * workspace and keeps no per-call state beyond a thread-local copy of the
 * last HIP error. o and lse must not overlap q, k, v or each other.
 *
 * Execution: calls are asynchronous on `stream` (a hipStream_t; NULL means
 * the default stream) and return once the kernel is enqueued. A device-side
 * fault surfaces at the caller's next synchronisation, as usual for HIP.
 * Results are deterministic: no atomics, a fixed reduction order.
 *
 * Errors: arguments are checked on the host before any HIP call; on any
 * error nothing is launched and the outputs are left untouched.
 */
#ifndef FA_H_
#define FA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Element types. Inputs: FA_F16 or FA_BF16. Output O: FA_F32, or the input type. */
typedef enum {
  FA_F16 = 0,
  FA_BF16 = 1,
  FA_F32 = 2
} fa_dtype;

typedef enum {
  FA_OK = 0,
  FA_ERR_NULLPTR = 1,     /* a pointer argument is NULL */
  FA_ERR_SHAPE = 2,       /* B, Hq, Hkv, N or d < 1; Hq not a multiple of Hkv; non-finite
                             or non-positive scale; sizes beyond the 32-bit index range */
  FA_ERR_UNSUPPORTED = 3, /* d not a multiple of 16 from 32 to 128; in_dtype not
                             F16/BF16; out_dtype not F32 or in_dtype */
  FA_ERR_ALIGN = 4,       /* a pointer not 16-byte aligned */
  FA_ERR_HIP = 5,         /* the HIP runtime reported an error; see fa_last_hip_error() */
  FA_ERR_SCRATCH = 6      /* fa_fwd_split_noalloc: the problem needs more scratch than the
                             library's static array holds (FA_NOALLOC_SCRATCH_BYTES) */
} fa_status;

/*
 * fa_fwd — exact attention forward (O and the natural-log LSE), see above.
 *
 *   q, k, v   device pointers, layouts above, element type in_dtype
 *   o         device pointer, [B][Hq][N][d] of out_dtype
 *   lse       device pointer, [B][Hq][N] float32
 *   B, Hq, Hkv, N, d   sizes; Hq % Hkv == 0; d a multiple of 16 from 32 to
 *             128: 32, 48, 64, 80, 96, 112 or 128 (the intelliparadigm page,
 *             section 1.3, asks for head dimensions that are not powers of
 *             two); N >= 1 (any N,
 *             tails are masked); B*Hq*ceil(N/128) below 2^31; N*d at most
 *             2^30 - 2^16 (a K/V head plane under 2 GiB)
 *   scale     multiplies Q.K^T (commonly 1/sqrt(d)); finite and > 0
 *   causal    0: every key visible; 1: key j visible to query i iff j <= i
 *   in_dtype  FA_F16 or FA_BF16
 *   out_dtype FA_F32 (recommended: keeps O within fp32 rounding) or in_dtype
 *   stream    hipStream_t to enqueue on, or NULL
 *
 * Returns FA_OK after enqueueing, or an error status with nothing launched.
 */
fa_status fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
                 int64_t B, int64_t Hq, int64_t Hkv, int64_t N, int64_t d,
                 float scale, int causal, fa_dtype in_dtype, fa_dtype out_dtype,
                 void* stream);

/*
 * fa_fwd_ex — fa_fwd with separate query and key lengths and a sliding-window
 * band. The intelliparadigm page's operator bounds a window with pre_tokens
 * and next_tokens (section 2.2) and tiles with separate query and key
 * lengths (section 2.3). Query row i sits at key position i + (Nk - Nq), so
 * its diagonal is aligned with the end of the key sequence, and it sees key j
 * iff
 *
 *   i + (Nk - Nq) - window_left  <=  j  <=  i + (Nk - Nq) + window_right
 *
 * A negative edge is unlimited. fa_fwd(causal = 1) is Nq = Nk with
 * window_left = -1 and window_right = 0; fa_fwd(causal = 0) has both edges
 * unlimited. A row that sees no key gets O = 0 and lse = -inf.
 *
 *   q, o      [B][Hq][Nq][d];  lse [B][Hq][Nq];  k, v [B][Hkv][Nk][d]
 *   Nq, Nk    >= 1, each with N*d at most 2^30 - 2^16
 * Other arguments, errors and execution as fa_fwd.
 */
fa_status fa_fwd_ex(const void* q, const void* k, const void* v, void* o, float* lse,
                    int64_t B, int64_t Hq, int64_t Hkv, int64_t Nq, int64_t Nk, int64_t d,
                    float scale, int64_t window_left, int64_t window_right,
                    fa_dtype in_dtype, fa_dtype out_dtype, void* stream);

/*
 * fa_fwd_split — fa_fwd_ex with the keys of every Q-tile cut into chunks that
 * separate work-groups process, for problems whose batch x heads x Q-tiles
 * leaves the GPU under-filled (the FA2 walkthrough: parallelism along the
 * sequence when batch and heads are small; the intelliparadigm page's
 * hierarchical tiling of long sequences, section 6.1). Each chunk's
 * normalised O and LSE go to the workspace, and a merge kernel combines them
 * with the online-softmax rule: LSE = ln sum_s exp(LSE_s) and
 * O = sum_s exp(LSE_s - LSE) O_s.
 *
 *   n_splits   0: automatic: no split when batch x heads x Q-tiles reaches 512
 *              work-groups, else about 512 / that count chunks, but no chunk
 *              shorter than 512 keys (grids up to 32 work-groups), 1024 keys
 *              (up to 255) or 4096 keys (256..511); otherwise the number of
 *              chunks wanted, at most 16. Chunks are whole 64-key tiles, at
 *              least two, so fewer may be used.
 *   workspace  device pointer to fa_fwd_split_workspace_bytes(...) bytes,
 *              16-byte aligned, owned by the caller. It may be NULL when that
 *              size is 0, which means no split: the call is then fa_fwd_ex.
 * Other arguments, errors and execution as fa_fwd_ex. The result equals
 * fa_fwd_ex's up to rounding order. Calls that share a workspace must not
 * run concurrently.
 */
fa_status fa_fwd_split(const void* q, const void* k, const void* v, void* o, float* lse,
                       float* workspace, int64_t B, int64_t Hq, int64_t Hkv, int64_t Nq,
                       int64_t Nk, int64_t d, float scale, int64_t window_left,
                       int64_t window_right, int n_splits, fa_dtype in_dtype,
                       fa_dtype out_dtype, void* stream);

/*
 * fa_fwd_split_noalloc — fa_fwd_split for callers that cannot allocate device
 * memory: code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc. The split partials go to a static scratch array inside the
 * library, FA_NOALLOC_SCRATCH_BYTES (64 MiB) on each GPU the library runs on,
 * held until the process ends; the call allocates nothing and takes no
 * workspace. The caller still passes the inputs and outputs.
 *   The array used is the current device's; stream must belong to that device
 *   (or be NULL), else FA_ERR_UNSUPPORTED. The first call on a device looks up
 *   its array's address (hipGetSymbolAddress); make one call before capturing.
 *   A problem whose partials (fa_fwd_split_workspace_bytes) exceed the array
 *   returns FA_ERR_SCRATCH with nothing launched; a problem that does not split
 *   needs no scratch and runs as fa_fwd_ex.
 *   Every call on a GPU shares that GPU's array, which keeps the last call's
 *   partials (each call writes every partial it reads, so nothing needs to
 *   start at zero): calls that overlap on one GPU (several streams or threads)
 *   race, and the caller must serialise them.
 * Other arguments, errors and execution as fa_fwd_split.
 */
#define FA_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
fa_status fa_fwd_split_noalloc(const void* q, const void* k, const void* v, void* o, float* lse,
                               int64_t B, int64_t Hq, int64_t Hkv, int64_t Nq, int64_t Nk,
                               int64_t d, float scale, int64_t window_left,
                               int64_t window_right, int n_splits, fa_dtype in_dtype,
                               fa_dtype out_dtype, void* stream);

/*
 * fa_fwd_fp8 — fa_fwd_ex for fp8 inputs. The zyxy lecture (section 5) lists fp8
 * among the input types of the FA2 generation of kernels. q, k and v hold OCP
 * e4m3 bytes (sign, 4 exponent bits with bias 7, 3 mantissa bits; 0x7F and 0xFF
 * are NaN), laid out as fa_fwd's q, k and v with one byte per element; the value
 * of an element is its e4m3 value times the tensor's descale. Scores are
 * scale * (descale_q q) . (descale_k k); both products run on gfx950's fp8
 * matrix cores with fp32 accumulation; the probabilities are rounded to e4m3
 * for the P V product (relative 2^-4, or 2^-10 of the row's running maximum in
 * e4m3's subnormal range), and O is divided by the sum of those rounded values.
 *
 *   o          device pointer, [B][Hq][Nq][d] float32
 *   lse        device pointer, [B][Hq][Nq] float32, natural log of the sum of exp(score)
 *   descale_q, descale_k, descale_v   finite and > 0 (FA_ERR_SHAPE otherwise)
 *   window_left, window_right         the band of fa_fwd_ex (causal: -1, 0)
 * Sizes, alignment (16 bytes), errors and execution as fa_fwd_ex. No split keys
 * and no mask input.
 */
fa_status fa_fwd_fp8(const void* q, const void* k, const void* v, float* o, float* lse,
                     float descale_q, float descale_k, float descale_v, int64_t B, int64_t Hq,
                     int64_t Hkv, int64_t Nq, int64_t Nk, int64_t d, float scale,
                     int64_t window_left, int64_t window_right, void* stream);

/*
 * fa_fwd_dropout — fa_fwd_ex with dropout on the probabilities: the Ascend
 * operator's keep_prob attribute (the intelliparadigm page, section 2.2, and its
 * call in section 4.1), the Dropout step of FlashAttention-1's Algorithm 2 that
 * the cnblogs page points to. Each (query, key) pair is kept independently and
 * kept probabilities are scaled by the inverse of the keep probability:
 *
 *   O_i = sum_j (Z_ij / keep) P_ij V_j,   lse as without dropout (the undropped
 *   softmax's statistic, which a backward recomputes P from).
 *
 * Z comes from Philox4x32-10 (Salmon et al., "Parallel random numbers: as easy
 * as 1, 2, 3", SC 2011) so that it can be drawn again: for head plane
 * h = b * Hq + hq, query row i and key j, the call with counter
 * (j / 4, i / 4, h, offset) and key (seed & 0xffffffff, seed >> 32) gives four
 * 32-bit words; byte j % 4 (bits 8 (j % 4) ..) of word i % 4 is the pair's random
 * byte, and the pair is kept iff that byte is below T = round(256 keep_prob),
 * clamped to [1, 256]. keep is therefore T / 256 and the scale applied 256 / T.
 *
 *   keep_prob  in (0, 1] (FA_ERR_SHAPE otherwise); 1 keeps every pair
 *   seed       64-bit Philox key; offset: counter word 3, so that calls with one
 *              seed can draw independent masks (e.g. one offset per layer)
 * The probabilities are normalised by the sum of their rounded 16-bit values as
 * in fa_fwd, with every pair in the sum (dropped or not). Inputs FA_F16 or
 * FA_BF16; no split keys and no mask input. Other arguments, errors and
 * execution as fa_fwd_ex.
 */
fa_status fa_fwd_dropout(const void* q, const void* k, const void* v, void* o, float* lse,
                         int64_t B, int64_t Hq, int64_t Hkv, int64_t Nq, int64_t Nk, int64_t d,
                         float scale, int64_t window_left, int64_t window_right,
                         float keep_prob, uint64_t seed, uint32_t offset, fa_dtype in_dtype,
                         fa_dtype out_dtype, void* stream);

/*
 * fa_fwd_mask — fa_fwd_split with a mask input: the Ascend operator's optional
 * boolean attn_mask (the intelliparadigm page, section 2.2), which is the Mask
 * step of FlashAttention-1's Algorithm 2 that the cnblogs page points to. Key
 * j is hidden from query i of head (b, h) when the byte
 *   mask[b * mask_b_stride + h * mask_h_stride + i * mask_row_stride + j]
 * is nonzero (the operator's convention: 1 means masked out), on top of the
 * band. A row that sees no key gets O = 0 and lse = -inf.
 *
 *   mask            device pointer to bytes, 4-byte aligned, owned by the
 *                   caller; read only
 *   mask_b_stride, mask_h_stride   bytes between batch elements and between
 *                   query heads; 0 shares one plane across them. Multiples of 4
 *   mask_row_stride bytes between query rows: >= Nk, a multiple of 4, with
 *                   Nq * mask_row_stride at most 2^31 - 2^16
 *   workspace       device pointer to fa_fwd_mask_workspace_bytes(..., mask_b_stride,
 *                   mask_h_stride) bytes,
 *                   16-byte aligned, owned by the caller; never NULL (the
 *                   split partials, if any, then the mask's key hull)
 *   n_splits        as fa_fwd_split (1: no split)
 * Before the attention kernel a pre-pass reads the mask once, packs it into one
 * bit per key in the workspace (the attention kernel reads those bits), and
 * records, for each Q-tile of 128 rows and chunk of 1024 keys, the first and
 * last key some row of the tile may see; the attention kernel then visits only
 * the key tiles between them, so the keys a mask hides from a whole Q-tile
 * cost no work.
 * Other arguments, errors and execution as fa_fwd_split; a NULL mask or
 * workspace is FA_ERR_NULLPTR, a misaligned one FA_ERR_ALIGN. Calls that share
 * a workspace must not run concurrently.
 */
fa_status fa_fwd_mask(const void* q, const void* k, const void* v, void* o, float* lse,
                      const void* mask, int64_t mask_b_stride, int64_t mask_h_stride,
                      int64_t mask_row_stride, float* workspace, int64_t B, int64_t Hq,
                      int64_t Hkv, int64_t Nq, int64_t Nk, int64_t d, float scale,
                      int64_t window_left, int64_t window_right, int n_splits,
                      fa_dtype in_dtype, fa_dtype out_dtype, void* stream);

/*
 * fa_fwd_float_mask — fa_fwd_ex with a float attn_mask: the Ascend operator's
 * optional attn_mask in its fp16 and fp32 forms (the intelliparadigm page,
 * section 2.2). The pages give those forms no meaning; the reading taken is
 * an additive mask (PyTorch's convention for a float attention mask): score
 * (i, j) of head (b, h) becomes
 *   scale * q_i . k_j + mask[b * mask_b_stride + h * mask_h_stride + i * mask_row_stride + j]
 * (strides in elements) before the softmax, on top of the band. -inf hides the
 * key; a row whose visible keys are all hidden gets O = 0 and lse = -inf. The
 * lse is the logsumexp of the masked scores. Entries must be finite or -inf.
 *
 *   mask            device pointer, 16-byte aligned, owned by the caller; read only
 *   mask_dtype      FA_F16 or FA_F32 (FA_ERR_UNSUPPORTED otherwise)
 *   mask_b_stride, mask_h_stride   elements between batch elements and between
 *                   query heads; 0 shares one plane across them. Multiples of 4
 *   mask_row_stride elements between query rows: >= Nk, a multiple of 4, with
 *                   (Nq + 32) * mask_row_stride * (element bytes) at most 2^31 - 2^16
 * Inputs FA_F16 or FA_BF16; no split keys. The attention kernel reads the mask
 * values of the tiles it visits (the band still skips whole tiles). Other
 * arguments, errors and execution as fa_fwd_ex; a NULL mask is FA_ERR_NULLPTR,
 * a misaligned one FA_ERR_ALIGN.
 */
fa_status fa_fwd_float_mask(const void* q, const void* k, const void* v, void* o, float* lse,
                            const void* mask, fa_dtype mask_dtype, int64_t mask_b_stride,
                            int64_t mask_h_stride, int64_t mask_row_stride, int64_t B,
                            int64_t Hq, int64_t Hkv, int64_t Nq, int64_t Nk, int64_t d,
                            float scale, int64_t window_left, int64_t window_right,
                            fa_dtype in_dtype, fa_dtype out_dtype, void* stream);

/*
 * fa_fwd_mask_workspace_bytes — bytes of workspace fa_fwd_mask needs for a mask
 * with these batch and head strides (0: shared along that axis), each part
 * starting at a 256-byte boundary: the split partials of
 * fa_fwd_split_workspace_bytes, then P x ceil(Nq / 128) x ceil(Nk / 1024)
 * pairs of int32 (the mask's key hull), then P x Nq x ceil(Nk / 32) words of
 * 32 bits (the mask packed to one bit per key), where P, the number of mask
 * planes, is (B if mask_b_stride else 1) x (Hq if mask_h_stride else 1).
 * 0 when the arguments are invalid. Makes no HIP call.
 */
size_t fa_fwd_mask_workspace_bytes(int64_t B, int64_t Hq, int64_t Nq, int64_t Nk, int64_t d,
                                   int n_splits, int64_t mask_b_stride, int64_t mask_h_stride);

/*
 * fa_fwd_split_workspace_bytes — bytes of workspace fa_fwd_split needs
 * (chunks x rows x (d + 1) floats), 0 when it would not split (or the
 * arguments are invalid). Makes no HIP call.
 */
size_t fa_fwd_split_workspace_bytes(int64_t B, int64_t Hq, int64_t Nq, int64_t Nk, int64_t d,
                                    int n_splits);

/* Static, NUL-terminated description of a status code (never NULL). */
const char* fa_status_str(fa_status s);

/* The hipError_t value behind the most recent FA_ERR_HIP on the calling thread (0 if none). */
int fa_last_hip_error(void);

/*
 * fa_fwd_tile — the work decomposition fa_fwd uses for a problem, so a
 * caller can reason about the launch (for example to count the K/V bytes
 * each work-group reads). Writes the query rows per work-group (*block_m),
 * the keys per inner tile (*block_n) and the work-group count (*grid).
 * Validates like fa_fwd (pointers to outputs must be non-NULL) and makes no
 * HIP call.
 */
fa_status fa_fwd_tile(int64_t B, int64_t Hq, int64_t Hkv, int64_t N, int64_t d, int causal,
                      fa_dtype in_dtype, int* block_m, int* block_n, int64_t* grid);

/*
 * fa_bwd — gradients of the attention fa_fwd computes, with respect to q, k
 * and v, given dout, the gradient arriving at its output o. The backward
 * pass recomputes the probabilities from q, k and the forward's lse rather
 * than storing them (intelliparadigm page, section 1.2.3, recomputation;
 * cnblogs page, summary; the Triton FA2 walkthrough keeps logsumexp L for
 * the backward pass). Per (batch, query head), with P the probabilities fa_fwd
 * applied and s = scale:
 *
 *   dV = P^T dO    dP = dO V^T    D_i = sum_c dO[i,c] O[i,c]
 *   dS = P o (dP - D)    (o: elementwise, D subtracted from row i)
 *   dQ = s dS K    dK = s dS^T Q
 *
 * and each K/V head's dK and dV are the sums over its G query heads.
 *
 *   q, k, v   as given to fa_fwd
 *   o, lse    as fa_fwd produced them; o of o_dtype (FA_F32 or in_dtype)
 *   dout      device pointer, [B][Hq][N][d] of in_dtype: the gradient at o
 *   dq        device pointer, [B][Hq][N][d] float32, written
 *   dk, dv    device pointers, [B][Hkv][N][d] float32, written
 *   workspace device pointer to fa_bwd_workspace_bytes(B, Hq, N, d) bytes
 *             of scratch, owned by the caller. Its contents on entry do not
 *             matter; afterwards it holds per-row statistics. Calls that
 *             share a workspace must not run concurrently.
 *   sizes, scale, causal, in_dtype, stream: as for fa_fwd
 *
 * The outputs must not overlap any input, the workspace or each other. The
 * call enqueues three kernels on `stream` (row statistics, dK/dV, dQ) and
 * allocates nothing. Results are deterministic (no atomics). Errors are
 * reported as for fa_fwd, and every argument is checked before any HIP call.
 */
fa_status fa_bwd(const void* q, const void* k, const void* v, const void* o, const float* lse,
                 const void* dout, float* dq, float* dk, float* dv, float* workspace,
                 int64_t B, int64_t Hq, int64_t Hkv, int64_t N, int64_t d,
                 float scale, int causal, fa_dtype in_dtype, fa_dtype o_dtype,
                 void* stream);

/*
 * fa_bwd_ex — fa_bwd for fa_fwd_ex: separate query and key lengths and the
 * same band. q, o, dout and dq are [B][Hq][Nq][d], lse [B][Hq][Nq], k, v, dk
 * and dv [B][Hkv][Nk][d]; the workspace is fa_bwd_workspace_bytes(B, Hq, Nq,
 * d) bytes. Rows that see no key contribute nothing and get dq = 0; keys no
 * row sees get dk = dv = 0. Other arguments, errors and execution as fa_bwd.
 */
fa_status fa_bwd_ex(const void* q, const void* k, const void* v, const void* o, const float* lse,
                    const void* dout, float* dq, float* dk, float* dv, float* workspace,
                    int64_t B, int64_t Hq, int64_t Hkv, int64_t Nq, int64_t Nk, int64_t d,
                    float scale, int64_t window_left, int64_t window_right,
                    fa_dtype in_dtype, fa_dtype o_dtype, void* stream);

/*
 * fa_bwd_dropout — fa_bwd_ex for a forward run with fa_fwd_dropout: the same
 * keep_prob, seed and offset draw the same keep mask Z (the Philox bytes of
 * fa_fwd_dropout), which is held fixed, and the chain rule through the scaled,
 * masked probabilities gives
 *   dV = (Z o P / keep)^T dO,  dP = (dO V^T) o Z / keep,  D_i = dO_i . O_i,
 *   dS = P o (dP - D),  dQ = s dS K,  dK = s dS^T Q
 * with P the undropped softmax (recomputed from the forward's LSE) and O the
 * forward's (dropped) output. keep_prob in (0, 1] (FA_ERR_SHAPE otherwise).
 * Other arguments, workspace, errors and execution as fa_bwd_ex.
 */
fa_status fa_bwd_dropout(const void* q, const void* k, const void* v, const void* o,
                         const float* lse, const void* dout, float* dq, float* dk, float* dv,
                         float* workspace, int64_t B, int64_t Hq, int64_t Hkv, int64_t Nq,
                         int64_t Nk, int64_t d, float scale, int64_t window_left,
                         int64_t window_right, float keep_prob, uint64_t seed, uint32_t offset,
                         fa_dtype in_dtype, fa_dtype o_dtype, void* stream);

/*
 * fa_bwd_float_mask — fa_bwd_ex for a forward run with fa_fwd_float_mask: the
 * same additive mask (arguments and layout as fa_fwd_float_mask) enters the
 * recomputed scores, so P and dS are those of the masked softmax; the mask
 * takes no gradient. The LSE must come from the masked forward.
 * Other arguments, workspace, errors and execution as fa_bwd_ex; a NULL mask is
 * FA_ERR_NULLPTR, a misaligned one FA_ERR_ALIGN.
 */
fa_status fa_bwd_float_mask(const void* q, const void* k, const void* v, const void* o,
                            const float* lse, const void* dout, float* dq, float* dk, float* dv,
                            float* workspace, const void* mask, fa_dtype mask_dtype,
                            int64_t mask_b_stride, int64_t mask_h_stride,
                            int64_t mask_row_stride, int64_t B, int64_t Hq, int64_t Hkv,
                            int64_t Nq, int64_t Nk, int64_t d, float scale,
                            int64_t window_left, int64_t window_right, fa_dtype in_dtype,
                            fa_dtype o_dtype, void* stream);

/*
 * fa_bwd_mask — fa_bwd_ex for a forward run with fa_fwd_mask: the same mask
 * (arguments and layout as fa_fwd_mask) hides the same scores, so P and dS
 * are zero there. The LSE must come from the masked forward.
 *   workspace  device pointer to fa_bwd_mask_workspace_bytes(..., mask_b_stride,
 *              mask_h_stride) bytes (the row statistics, then the mask packed
 *              to bits and its summaries), 16-byte aligned, owned by the caller
 * A pre-pass reads the mask once, as in fa_fwd_mask, and also writes it by key
 * columns; the dQ kernel then visits only the key tiles inside each Q-tile's
 * hull, and the dK/dV kernel only the Q-tiles whose block with its key tile has
 * a visible pair, reading one column word per key and 32-query block.
 * Other arguments, errors and execution as fa_bwd_ex; a NULL mask is
 * FA_ERR_NULLPTR, a misaligned one FA_ERR_ALIGN.
 */
fa_status fa_bwd_mask(const void* q, const void* k, const void* v, const void* o,
                      const float* lse, const void* dout, float* dq, float* dk, float* dv,
                      float* workspace, const void* mask, int64_t mask_b_stride,
                      int64_t mask_h_stride, int64_t mask_row_stride, int64_t B, int64_t Hq,
                      int64_t Hkv, int64_t Nq, int64_t Nk, int64_t d, float scale,
                      int64_t window_left, int64_t window_right, fa_dtype in_dtype,
                      fa_dtype o_dtype, void* stream);

/*
 * fa_bwd_mask_workspace_bytes — bytes of workspace fa_bwd_mask needs for a mask
 * with these batch and head strides (0: shared along that axis): the row
 * statistics of fa_bwd_workspace_bytes(B, Hq, Nq, d), then, each at a 256-byte
 * boundary, the key hull and the packed mask as for fa_fwd_mask_workspace_bytes,
 * then P x ceil(Nk / 128) x ceil(Nq / 128) flag bytes, then P x Nk x ceil(Nq / 32)
 * words of 32 bits (the mask by key columns) (P mask planes).
 * 0 when the arguments are invalid. Makes no HIP call.
 */
size_t fa_bwd_mask_workspace_bytes(int64_t B, int64_t Hq, int64_t Nq, int64_t Nk, int64_t d,
                                   int64_t mask_b_stride, int64_t mask_h_stride);

/*
 * fa_bwd_workspace_bytes — size in bytes of the workspace fa_bwd (or
 * fa_bwd_ex, with N = Nq) needs for these sizes (two floats per query row,
 * rows padded to a multiple of 128), or 0 when the sizes are invalid for
 * fa_bwd. Makes no HIP call.
 */
size_t fa_bwd_workspace_bytes(int64_t B, int64_t Hq, int64_t N, int64_t d);

#ifdef __cplusplus
}
#endif

#endif /* FA_H_ */
