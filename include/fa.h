/*
 * libfa — exact tiled attention (FlashAttention-2 forward and recomputation
 * backward) for AMD Instinct MI355X (gfx950).
 *
 * What is computed (per batch b and head h, rows q_i, k_j, v_j of Q, K, V):
 *
 *   S_ij = scale * <q_i, k_j>, then S_ij = -inf where the key is masked;
 *   P    = row-wise softmax(S);   O = P V;   LSE_i = ln sum_j exp(S_ij).
 *
 * This is plain softmax attention, computed exactly (FlashAttention-2 wiki
 * pages, opening paragraph: same result as standard attention, no loss of
 * precision) but in one fused pass that keeps the N x N score matrix on chip
 * (FlashAttention-NeurIPS22 digest, section "核心方法": tiling with an online
 * softmax, kernel fusion of matmul + mask + softmax + matmul).  The forward
 * saves only O and one softmax statistic per row, LSE; the backward
 * recomputes S and P from Q, K and LSE instead of reading them from memory
 * (same section, "Backward recomputation").
 *
 * Conventions shared by every call
 * --------------------------------
 * - Tensors are BHND: element (b, h, n, k) of a [B, H, N, d] tensor sits at
 *   ((b * H + h) * N + n) * d + k, densely packed, no strides.
 * - Q, K, V, O, dO, dQ, dK, dV hold IEEE bfloat16 bit patterns (uint16).
 *   LSE and the workspace are float32.  All tensor pointers are DEVICE
 *   pointers owned by the caller; the library never allocates or frees
 *   memory and keeps no pointer after a call returns.
 * - Masks.  causal != 0 masks key j for query i when j > i.  blockmask, if
 *   not NULL, is a DEVICE pointer to nb x nb uint8 values (nb =
 *   ceil(N / mask_block)), row-major, shared by every batch and head; key j
 *   is masked for query i when blockmask[(i / mask_block) * nb +
 *   j / mask_block] == 0 (block-sparse attention, digest section "核心方法",
 *   Block-sparse 扩展: zero blocks are skipped).  Both masks may be combined.
 * - A query row whose keys are all masked gets O = 0 and LSE = -inf, and
 *   contributes nothing to dK or dV; its dQ row is 0.
 * - Outputs are rounded to bfloat16 with round-to-nearest-even.
 * - Work is enqueued on `stream` (NULL = the null stream) and the call
 *   returns without synchronising.  Results are bitwise reproducible from
 *   run to run: no atomics are used anywhere (FlashAttention-2 wiki,
 *   "性能与效率": the algorithm is exact and deterministic).
 * - Outputs must not overlap inputs or each other.
 *
 * Supported domain (anything else returns FA_ERR_UNSUPPORTED):
 *   d in {64, 128}; N >= 0 (any length; a partial last tile is masked);
 *   scale finite and > 0; mask_block a positive multiple of 128 when
 *   blockmask != NULL (ignored otherwise); N * d < 2^31 and
 *   ceil(N / 128) * B * H < 2^31; bf16 tensor pointers 16-byte aligned,
 *   float32 pointers 4-byte aligned.
 *   B, H or N equal to 0 is a valid empty problem: nothing is launched.
 *
 * Errors.  Every argument check happens before any HIP call, and on error
 * nothing is launched.  A launch failure is reported as FA_ERR_HIP (from
 * hipGetLastError).  No C++ exception crosses this interface.
 */
#ifndef LIBFA_FA_H
#define LIBFA_FA_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  FA_OK = 0,
  FA_ERR_NULL = 1,        /* a required pointer is NULL                         */
  FA_ERR_SHAPE = 2,       /* a negative dimension                               */
  FA_ERR_UNSUPPORTED = 3, /* outside the supported domain listed above          */
  FA_ERR_WORKSPACE = 4,   /* workspace NULL or smaller than fa_bwd_workspace_bytes */
  FA_ERR_HIP = 5,         /* the HIP runtime reported an error at launch        */
  FA_ERR_SCRATCH = 6      /* fa_bwd_noalloc: B*H*N above FA_NOALLOC_MAX_ROWS     */
} fa_status;

/*
 * Forward pass: O = softmax(scale * Q K^T + mask) V and LSE.
 *
 * The running row maximum and row sum of the online softmax (digest section
 * "核心方法", Tiling 与 online softmax) are merged tile by tile; the division
 * by the row sum is applied once at the end (FlashAttention-2 wiki,
 * "技术架构与工作原理", item 1: fewer non-matmul operations).
 *
 *   Q, K, V    [B, H, N, d] bf16, read only.
 *   O          [B, H, N, d] bf16, written.
 *   LSE        [B, H, N] float32, written: natural-log log-sum-exp of the
 *              scaled, masked scores of each row (-inf for an empty row).
 *   scale      multiplies Q K^T before masking.
 *   blockmask  NULL (no block mask) or device uint8 [nb, nb], see above.
 *
 * Returns FA_OK, or FA_ERR_NULL / FA_ERR_SHAPE / FA_ERR_UNSUPPORTED /
 * FA_ERR_HIP.
 */
int fa_fwd(const void* Q, const void* K, const void* V,
           int B, int H, int N, int d, float scale, int causal,
           const uint8_t* blockmask, int mask_block,
           void* O, float* LSE, hipStream_t stream);

/*
 * Bytes of device workspace fa_bwd needs: one float32 per query row for
 * D_i = sum_k dO_ik * O_ik, i.e. 4 * B * H * N (0 for invalid or empty
 * arguments).
 */
size_t fa_bwd_workspace_bytes(int B, int H, int N, int d);

/*
 * Backward pass: gradients of L = sum(dO * O) with respect to Q, K and V,
 * recomputing S and P from Q, K and the saved LSE (digest section "核心方法",
 * Backward recomputation).  Two stream-ordered launches:
 *   1. per block of queries: D_i = sum_k dO_ik * O_ik for the block's rows,
 *      stored in the workspace, then dQ = scale * dS K with dP = dO V^T and
 *      dS = P * (dP - D) recomputed tile by tile; dQ is written once, so no
 *      atomics are needed;
 *   2. per block of keys: dV = P^T dO, dP = dO V^T, dS = P * (dP - D),
 *      dK = scale * dS^T Q, reading D from the workspace.
 * fa_bwd_dq_dsum followed by fa_bwd_dkdv (below) are exactly these two
 * launches; the three-stage order fa_bwd_dsum, fa_bwd_dkdv, fa_bwd_dq gives
 * the same bits.
 *
 *   Q, K, V, O, dO   [B, H, N, d] bf16, read only.  O and LSE must be the
 *                    outputs of fa_fwd for the same Q, K, V, scale and
 *                    masks.
 *   LSE              [B, H, N] float32, read only.
 *   dQ, dK, dV       [B, H, N, d] bf16, written.
 *   workspace        device memory of at least fa_bwd_workspace_bytes(),
 *                    4-byte aligned; contents on entry are ignored.
 *
 * Returns FA_OK, or FA_ERR_NULL / FA_ERR_SHAPE / FA_ERR_UNSUPPORTED /
 * FA_ERR_WORKSPACE / FA_ERR_HIP.
 */
int fa_bwd(const void* Q, const void* K, const void* V, const void* O,
           const void* dO, const float* LSE,
           int B, int H, int N, int d, float scale, int causal,
           const uint8_t* blockmask, int mask_block,
           void* dQ, void* dK, void* dV,
           void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * fa_bwd without a workspace argument, for callers that cannot allocate
 * device memory: code under HIP graph capture, tight serving loops, and
 * harnesses that forbid allocation.  The call itself allocates nothing (no
 * hipMalloc, hipFree or allocating library routine); D lives in a static
 * device array of FA_NOALLOC_MAX_ROWS floats (16 MiB) inside the library,
 * which every GPU the library runs on holds until the process ends.  Same
 * kernels and launch order as fa_bwd, so the results are the same bits.
 *
 *   Arguments as fa_bwd, minus workspace and workspace_bytes.
 *   B * H * N must not exceed FA_NOALLOC_MAX_ROWS, else FA_ERR_SCRATCH is
 *   returned and nothing is launched.
 *
 * All calls on one GPU share that GPU's scratch array, which keeps the last
 * call's D: calls that overlap on one GPU (issued on different streams
 * without ordering between them) race and give undefined results.  The first
 * call on a device looks up the array's address there (FA_ERR_HIP if that
 * fails).  Other errors as fa_bwd.
 */
#define FA_NOALLOC_MAX_ROWS 4194304
int fa_bwd_noalloc(const void* Q, const void* K, const void* V, const void* O,
                   const void* dO, const float* LSE,
                   int B, int H, int N, int d, float scale, int causal,
                   const uint8_t* blockmask, int mask_block,
                   void* dQ, void* dK, void* dV, hipStream_t stream);

/*
 * The three stages of fa_bwd as separate calls, for callers that schedule
 * them themselves (for example fa_bwd_dkdv and fa_bwd_dq on two streams once
 * fa_bwd_dsum has finished: they read the same inputs and write disjoint
 * outputs).  fa_bwd_dsum, then fa_bwd_dkdv, then fa_bwd_dq on one stream
 * give the same bits as fa_bwd.  Arguments mean what they mean for fa_bwd; Dsum is the
 * float32 [B, H, N] buffer of D_i = sum_k dO_ik * O_ik (the workspace of
 * fa_bwd), written by fa_bwd_dsum and read by the other two.  Same errors
 * as fa_bwd, with FA_ERR_NULL for a NULL Dsum.
 */
int fa_bwd_dsum(const void* O, const void* dO, int B, int H, int N, int d,
                float* Dsum, hipStream_t stream);

int fa_bwd_dkdv(const void* Q, const void* K, const void* V, const void* dO,
                const float* LSE, const float* Dsum,
                int B, int H, int N, int d, float scale, int causal,
                const uint8_t* blockmask, int mask_block,
                void* dK, void* dV, hipStream_t stream);

int fa_bwd_dq(const void* Q, const void* K, const void* V, const void* dO,
              const float* LSE, const float* Dsum,
              int B, int H, int N, int d, float scale, int causal,
              const uint8_t* blockmask, int mask_block,
              void* dQ, hipStream_t stream);

/*
 * fa_bwd_dq and fa_bwd_dsum in one launch: dQ as fa_bwd_dq gives it, and D
 * written to Dsum with the same bits fa_bwd_dsum writes (the workgroup
 * forms D for its own rows before its main loop, summing in the same
 * order).  fa_bwd is exactly this call, then fa_bwd_dkdv, on one stream.
 * O is read only for D.  Errors as fa_bwd_dq, with FA_ERR_NULL for a NULL
 * O and FA_ERR_UNSUPPORTED for a misaligned one.
 */
int fa_bwd_dq_dsum(const void* Q, const void* K, const void* V, const void* O,
                   const void* dO, const float* LSE,
                   int B, int H, int N, int d, float scale, int causal,
                   const uint8_t* blockmask, int mask_block,
                   float* Dsum, void* dQ, hipStream_t stream);

/*
 * Attention with N_q query rows and N_k key rows (cross attention, and the
 * decoding case with a KV cache, which the pages leave untreated:
 * FlashAttention-NeurIPS22 digest, "设计取舍" (boundary conditions) and
 * "Critical Analysis" (假设压力测试) note that the decode phase with a growing
 * KV cache is not characterised).  Q, O, dO, dQ are
 * [B, H, Nq, d], K, V, dK, dV are [B, H, Nk, d], LSE [B, H, Nq]; a block mask
 * is ceil(Nq / mask_block) x ceil(Nk / mask_block).  The causal mask is
 * aligned bottom-right: query i sees key j iff j <= i + (Nk - Nq), i.e. the
 * queries are the last Nq positions of the key sequence; rows with
 * i + Nk - Nq < 0 see no key (O = 0, LSE = -inf, dQ = 0).  With Nq = Nk these
 * are exactly fa_fwd and fa_bwd.  Nk = 0 is allowed (every row empty; K, V,
 * dK, dV may then be NULL); with Nq = 0 and Nk > 0 fa_bwd_nqk writes dK = dV
 * = 0.  The workspace is fa_bwd_workspace_bytes(B, H, Nq, d).  Errors as for
 * fa_fwd and fa_bwd.
 */
int fa_fwd_nqk(const void* Q, const void* K, const void* V,
               int B, int H, int Nq, int Nk, int d, float scale, int causal,
               const uint8_t* blockmask, int mask_block,
               void* O, float* LSE, hipStream_t stream);

int fa_bwd_nqk(const void* Q, const void* K, const void* V, const void* O,
               const void* dO, const float* LSE,
               int B, int H, int Nq, int Nk, int d, float scale, int causal,
               const uint8_t* blockmask, int mask_block,
               void* dQ, void* dK, void* dV,
               void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * Forward with the key axis split across workgroups (split-KV), for shapes with
 * few query rows and a long key sequence (decoding against a KV cache), where
 * one workgroup per 128 query rows and head would leave most of the GPU idle.
 * The key tiles of each query block are cut into num_splits ranges; each range
 * produces a normalised partial O_s and its LSE_s in the workspace, and a
 * second launch merges them: LSE = log sum_s exp(LSE_s), O = sum_s
 * exp(LSE_s - LSE) O_s, which is the softmax over all keys (the same
 * rescaling identity the online softmax applies tile by tile, digest "核心方法",
 * Tiling 与 online softmax).  Arguments and results are those of fa_fwd_nqk.
 *   num_splits  <= 0: chosen by fa_fwd_splitkv_num_splits; 1: no split (then
 *               exactly fa_fwd_nqk, workspace unused).  Counts beyond the
 *               number of 64-key tiles are reduced.
 *   workspace   DEVICE, 16-byte aligned, at least
 *               fa_fwd_splitkv_workspace_bytes(B, H, Nq, Nk, d, num_splits)
 *               bytes (0 when no split results); else FA_ERR_WORKSPACE.
 * Results agree with fa_fwd_nqk to rounding (the merge adds up to num_splits
 * fp32 terms per element); not bitwise.
 */
int fa_fwd_splitkv(const void* Q, const void* K, const void* V,
                   int B, int H, int Nq, int Nk, int d, float scale, int causal,
                   const uint8_t* blockmask, int mask_block, int num_splits,
                   void* workspace, size_t workspace_bytes,
                   void* O, float* LSE, hipStream_t stream);

/* The split count fa_fwd_splitkv uses for num_splits <= 0 (at least 1): about
 * one workgroup per compute unit (256 in flight) with 4 to 256 64-key tiles
 * per range; 0 for invalid shapes. */
int fa_fwd_splitkv_num_splits(int B, int H, int Nq, int Nk, int d);

/* Workspace bytes fa_fwd_splitkv needs for that num_splits (0: no split, or
 * invalid shapes): splits * B * H * Nq * (d + 1) * 4. */
size_t fa_fwd_splitkv_workspace_bytes(int B, int H, int Nq, int Nk, int d, int num_splits);

/*
 * Dropout on the attention probabilities.  The pages list dropout among the
 * steps fused into the single attention kernel, between the softmax and the
 * second product (FlashAttention-NeurIPS22 digest, "核心方法", Kernel
 * fusion), and have the backward rebuild what it needs on chip ("核心方法",
 * Backward recomputation); the mask is therefore drawn from a counter-based
 * generator and regenerated by the backward, never stored.
 *
 *   P = softmax(scale * Q K^T + mask) as in fa_fwd; LSE is P's (no dropout);
 *   O = (P * keep / (1 - p_drop)) V.
 *
 * One draw of Philox4x32-10 (Salmon et al., "Parallel random numbers: as easy
 * as 1, 2, 3", SC 2011) on the counter (j / 4, i / 2, b * H + h, offset) under
 * the key (seed mod 2^32, seed / 2^32) decides the two queries i and four keys
 * j that share those quotients: element (b, h, i, j) takes the 16-bit half
 * e mod 2 (low half first) of output word e / 2, e = 4 (i mod 2) + (j mod 4),
 * and is kept iff that value is >= floor(p_drop * 2^16).  The same
 * (p_drop, seed, offset) must be passed to
 * fa_bwd_dropout; a caller takes a fresh offset (or seed) per call to get a
 * fresh mask.  p_drop must satisfy 0 <= p_drop < 1 (else FA_ERR_UNSUPPORTED);
 * p_drop = 0 gives exactly fa_fwd / fa_bwd.  Other arguments and errors are
 * those of fa_fwd / fa_bwd.  fa_bwd_dropout returns the gradients of
 * sum(dO * O) for that O: dV = Pd^T dO with Pd = P * keep / (1 - p_drop), and
 * dS = P * (dP * keep / (1 - p_drop) - D), D_i = sum_k dO_ik O_ik.
 */
int fa_fwd_dropout(const void* Q, const void* K, const void* V,
                   int B, int H, int N, int d, float scale, int causal,
                   const uint8_t* blockmask, int mask_block,
                   float p_drop, uint64_t seed, uint32_t offset,
                   void* O, float* LSE, hipStream_t stream);

int fa_bwd_dropout(const void* Q, const void* K, const void* V, const void* O,
                   const void* dO, const float* LSE,
                   int B, int H, int N, int d, float scale, int causal,
                   const uint8_t* blockmask, int mask_block,
                   float p_drop, uint64_t seed, uint32_t offset,
                   void* dQ, void* dK, void* dV,
                   void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * The keep decisions of that dropout stream as bytes: keep[((b * H + h) * N
 * + i) * N + j] = 1 if element (b, h, i, j) is kept, else 0 (DEVICE pointer,
 * B * H * N * N bytes, caller-owned; for inspection and tests).  Ignores
 * masking (a masked element's probability is 0 whatever its keep bit).
 * FA_ERR_SHAPE for negative sizes, FA_ERR_UNSUPPORTED for a bad p_drop or
 * more than 2^40 bytes, FA_ERR_NULL for a NULL keep with a non-empty shape.
 */
int fa_dropout_keep_mask(int B, int H, int N, float p_drop, uint64_t seed,
                         uint32_t offset, uint8_t* keep, hipStream_t stream);

/*
 * FP8 forward.  The FlashAttention-2 wiki ("与后续版本的比较",
 * FlashAttention-3) names 8-bit floating point as the following generation's
 * route to more speed; it fixes no format or scaling.  Here Q, K and V are
 * [B,H,N,d] arrays of one-byte E4M3 codes (OCP 8-bit floating point, the
 * variant without infinities: sign, 4 exponent bits with bias 7, 3 mantissa
 * bits; max 448), DEVICE pointers, 16-byte aligned.  Element x of Q stands for
 * value(x) * q_descale, and likewise for K and V with their own fp32 factor.
 *
 *   O   = softmax(scale * Q K^T + mask) V of those values, bf16 [B,H,N,d];
 *   LSE = natural-log row log-sum-exp of the scaled, masked scores, fp32.
 *
 * Both products run on the 8-bit matrix cores with fp32 accumulation; P is
 * rounded to E4M3 (nearest even) before the P V product, which moves each
 * element of O by at most 2^-4 sum_j P_ij |v_j| + 2^-14 sum_j |v_j| (visible
 * j) plus bf16 output rounding; LSE is formed from the unrounded fp32 P.
 * Masks, N (any N >= 0), d (64 or 128) and errors as fa_fwd; the three
 * descales must be finite and > 0, and scale * q_descale * k_descale * log2(e)
 * between 1e-30 and 1e30 (else FA_ERR_UNSUPPORTED).  Codes 0x7F / 0xFF (NaN)
 * give undefined results.
 */
int fa_fwd_fp8(const void* Q, const void* K, const void* V,
               int B, int H, int N, int d, float scale,
               float q_descale, float k_descale, float v_descale, int causal,
               const uint8_t* blockmask, int mask_block,
               void* O, float* LSE, hipStream_t stream);

/* Static, human-readable text for a status code (never NULL). */
const char* fa_strerror(int status);

#ifdef __cplusplus
}
#endif

#endif /* LIBFA_FA_H */
