/*
 * mshard.h - C ABI of libmshard.so: one tensor-parallel rank's shard of the
 * transformer MLP block (forward and backward) and of the vocab-parallel output
 * layer fused with cross-entropy, as hand-written HIP kernels for gfx950.
 *
 * The operations are those of the Megatron-LM intra-layer split:
 *   - Megatron-LM explainer (azimuth.plus/paper/megatron-lm), "core idea:
 *     slicing the feed-forward network": Y = GeLU(XA), Z = Dropout(YB); A is
 *     split by columns so each rank applies GeLU to X A_i with no
 *     synchronisation, B by rows so Y_i B_i is this rank's partial of YB.
 *   - same page, "the f and g operators": f (before the block) is the identity
 *     forward and all-reduces the input gradient backward; g (after the block)
 *     all-reduces the partial outputs forward and is the identity backward.
 *     This library computes everything between f and g for one rank: it emits
 *     the partials Z_i and dX_i that g and f would sum.
 *   - Megatron-LM paper notes (notes.yuuk.io), "vocab-embedding parallelism":
 *     E_{H x v} is split along the vocabulary, each rank computes its partial
 *     GEMM X E_i, and the output GEMM is fused with the cross-entropy so only
 *     b*s values per quantity leave the rank instead of b*s*v logits.
 *   - Megatron Core bitwise-determinism news item (news.hamidun.com): every
 *     reduction here runs in a fixed order with private per-writer workspace,
 *     and no floating-point atomics are used, so repeated calls with the same
 *     inputs give bitwise-identical outputs.
 *
 * Conventions shared by every entry point
 *   - Matrices are row-major in the pages' math layout: X[T x h], A_i[h x f_i],
 *     B_i[f_i x h], E_i[h x v_i], dZ[T x h]; T = b*s tokens (the order of b and
 *     s does not matter: every operation is per token row).
 *   - bf16 values are passed as raw 16-bit patterns (ms_bf16).  Every GEMM
 *     multiplies bf16 inputs with fp32 accumulation; bf16 outputs are rounded
 *     once, to nearest even.
 *   - All pointers are DEVICE pointers on the current HIP device, except where
 *     stated.  The caller owns every buffer and the stream; the library never
 *     allocates, frees or synchronises.
 *   - Work is enqueued on `stream` (a hipStream_t; NULL = default stream).
 *     MS_OK means "validated and enqueued"; device faults surface at the
 *     caller's next synchronisation, as with any HIP launch.
 *   - Validation runs first, on the host, without touching device memory.  On
 *     any error nothing is enqueued, the status is returned, and
 *     ms_last_error() gives a message.  Checks: required pointers non-NULL;
 *     T >= 1 and h, f_i, v_i >= 8, multiples of 8 and below 2^22; every buffer and the
 *     workspace 16-byte aligned; every buffer smaller than 2^31 bytes; no output
 *     overlapping an input, another output or the workspace; workspace at least
 *     the size the matching *_workspace_bytes function returns.
 *   - Preconditions that are not checked: device pointers are valid for the
 *     sizes given; 0 <= target < v_global; inputs are finite (NaN/Inf simply
 *     propagate).  Calls that share a workspace must not overlap in time.
 *   - Determinism: identical inputs, shapes, device model and library build give
 *     bitwise-identical outputs, whatever the stream, buffer addresses or prior
 *     workspace contents.
 */
#ifndef MSHARD_H
#define MSHARD_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef uint16_t ms_bf16; /* raw bf16 bit pattern */

typedef enum {
  MS_OK = 0,
  MS_ERR_NULL = 1,      /* a required pointer is NULL */
  MS_ERR_SHAPE = 2,     /* a size is out of range or not a multiple of 8 */
  MS_ERR_ALIGN = 3,     /* a buffer is not 16-byte aligned */
  MS_ERR_ALIAS = 4,     /* an output overlaps an input, another output or the workspace */
  MS_ERR_WORKSPACE = 5, /* workspace missing or too small */
  MS_ERR_ENUM = 6,      /* unknown enum value */
  MS_ERR_HIP = 7        /* a HIP call failed (no gfx950 device, launch failure, ...) */
} ms_status;

/* GeLU form.  The pages name GeLU without a formula: MS_GELU_ERF is the
 * definition x * Phi(x); MS_GELU_TANH is the tanh approximation from the GELU
 * paper (Hendrycks & Gimpel). */
typedef enum { MS_GELU_ERF = 0, MS_GELU_TANH = 1 } ms_gelu;

/* Bytes of device workspace that mlp_shard_fwd and mlp_shard_bwd need for these
 * sizes (one number covers both).  Returns 0 for invalid sizes. */
size_t mlp_shard_workspace_bytes(int64_t T, int64_t h, int64_t f_i);

/* Bytes of workspace mlp_shard_fwd itself needs: 0 when its launch plan uses
 * none (then its workspace may be NULL), else mlp_shard_workspace_bytes.  The
 * forward uses a workspace when the tiles of X A_i or of Y_i B_i leave the
 * GPU's last round of workgroups mostly idle: it then splits the contraction
 * of that GEMM's last tile columns into slices there, summed in slice order.
 * Returns 0 for invalid sizes. */
size_t mlp_shard_fwd_workspace_bytes(int64_t T, int64_t h, int64_t f_i);

/* Forward of one rank's MLP shard (explainer, "core idea"; paper notes, "MLP
 * block split"):
 *     H_i = X A_i (+ b1_i),   Y_i = GeLU(H_i),   Z_i = Y_i B_i.
 * Inputs : X[T x h], A_i[h x f_i], B_i[f_i x h] bf16; b1_i[f_i] bf16 or NULL
 *          (column-sharded bias added before GeLU).
 * Outputs: H_i[T x f_i] and Y_i[T x f_i] bf16 (saved for the backward; Y_i is
 *          GeLU of the fp32 pre-activation, then rounded); Z_i[T x h] fp32,
 *          this rank's partial of YB (g would sum it over ranks; the second
 *          bias and dropout act after that sum and are not applied here).
 * Workspace: mlp_shard_fwd_workspace_bytes(T, h, f_i) bytes, or NULL when that
 *          is 0; too small or NULL when needed -> MS_ERR_WORKSPACE. */
ms_status mlp_shard_fwd(const ms_bf16* X, const ms_bf16* A_i, const ms_bf16* b1_i, const ms_bf16* B_i,
                        int64_t T, int64_t h, int64_t f_i, ms_gelu gelu,
                        ms_bf16* H_i, ms_bf16* Y_i, float* Z_i,
                        void* workspace, size_t workspace_bytes, void* stream);

/* Backward of one rank's MLP shard, by the chain rule with dZ arriving
 * unchanged through g's backward (explainer, "the f and g operators"):
 *     dH_i = (dZ B_i^T) * GeLU'(H_i),   dB_i = Y_i^T dZ,   dA_i = X^T dH_i,
 *     db1_i = sum over tokens of dH_i,  dX_i = dH_i A_i^T.
 * Inputs : X[T x h], A_i[h x f_i], B_i[f_i x h], H_i and Y_i[T x f_i] (from the
 *          forward), dZ[T x h], all bf16.
 * Outputs: dX_i[T x h] fp32 (this rank's partial; f would all-reduce it);
 *          dA_i[h x f_i], dB_i[f_i x h] bf16; db1_i[f_i] bf16 or NULL (skip).
 * Weight-gradient GEMMs may split the token contraction; their partial sums go
 * to private workspace slices and are added in ascending slice order. */
ms_status mlp_shard_bwd(const ms_bf16* X, const ms_bf16* A_i, const ms_bf16* B_i,
                        const ms_bf16* H_i, const ms_bf16* Y_i, const ms_bf16* dZ,
                        int64_t T, int64_t h, int64_t f_i, ms_gelu gelu,
                        float* dX_i, ms_bf16* dA_i, ms_bf16* dB_i, ms_bf16* db1_i,
                        void* workspace, size_t workspace_bytes, void* stream);

/* Bytes of device workspace vocab_ce_shard_fwd needs.  Returns 0 for invalid sizes. */
size_t vocab_ce_workspace_bytes(int64_t T, int64_t h, int64_t v_i);

/* Vocab-parallel logits GEMM fused with the cross-entropy partials (paper
 * notes, "vocab-embedding parallelism").  The logits L = X E_i (fp32) are
 * never written to memory.  Per token t:
 *     m_i[t] = max_j L[t,j],   s_i[t] = sum_j exp(L[t,j] - m_i[t]),
 *     z_i[t] = L[t, target[t] - vocab_start] if vocab_start <= target[t] <
 *              vocab_start + v_i (this rank owns the target), else 0.
 * Inputs : X[T x h], E_i[h x v_i] bf16; target[T] int64 global vocabulary ids;
 *          vocab_start = first global id of this shard (>= 0).
 * Outputs: m_i, s_i, z_i [T] fp32.  Every column of E_i, padded ones included,
 *          takes part in the softmax. */
ms_status vocab_ce_shard_fwd(const ms_bf16* X, const ms_bf16* E_i, const int64_t* target,
                             int64_t T, int64_t h, int64_t v_i, int64_t vocab_start,
                             float* m_i, float* s_i, float* z_i,
                             void* workspace, size_t workspace_bytes, void* stream);

/* vocab_ce_shard_fwd without a workspace argument, for callers that cannot
 * allocate device memory (code under stream capture, tight serving loops,
 * harnesses that forbid allocation).  The per-tile partials live in a static
 * device array of 32 MiB, one per GPU, held until the process ends; its device
 * address is looked up once per GPU on the first call there.  Sizes whose
 * partials need more (vocab_ce_workspace_bytes(T, h, v_i) > 32 MiB, i.e.
 * 12 * T * ceil(v_i / 256) bytes rounded up) are refused with MS_ERR_WORKSPACE
 * before anything is enqueued.  Every call on a GPU uses that GPU's array and
 * leaves its own partials in it: calls that overlap in time on one GPU (other
 * streams, other threads) race and must not be made.  Each call writes every
 * partial it reads, so nothing needs clearing between calls.  Arguments,
 * outputs, validation and results are those of vocab_ce_shard_fwd; the same
 * kernels run, so the outputs are bitwise those of vocab_ce_shard_fwd. */
ms_status vocab_ce_shard_fwd_noalloc(const ms_bf16* X, const ms_bf16* E_i, const int64_t* target,
                                     int64_t T, int64_t h, int64_t v_i, int64_t vocab_start,
                                     float* m_i, float* s_i, float* z_i, void* stream);

/* Bytes of device workspace ce_combine needs (currently 0 for valid sizes). */
size_t ce_combine_workspace_bytes(int32_t t, int64_t T);

/* Merge the t vocab shards' partials into the loss, in ascending rank order:
 *     M = max_r m[r][t],  S = sum_r s[r][t] exp(m[r][t] - M),
 *     loss[t] = ln S + M - sum_r z[r][t],
 *     loss_mean = (fixed-order pairwise sum of loss) / T.
 * Inputs : m, s, z fp32, each [t x T] row-major (rank r's vector at offset r*T).
 * Outputs: loss[T] fp32; loss_mean[1] fp32 or NULL (skip).  t >= 1. */
ms_status ce_combine(const float* m, const float* s, const float* z, int32_t t, int64_t T,
                     float* loss, float* loss_mean,
                     void* workspace, size_t workspace_bytes, void* stream);

/* Bytes of device workspace attn_shard_bwd needs: dO, the per-row delta,
 * dQKV and, when a token contraction is split, fp32 slices of the weight
 * gradients.  attn_shard_fwd needs none.  Returns 0 for invalid sizes. */
size_t attn_shard_workspace_bytes(int64_t b, int64_t s, int64_t h, int64_t n, int64_t d);

/* Forward of one rank's self-attention shard (explainer, "attention"; paper
 * notes, "self-attention block split": the Q, K, V projections are split by
 * columns so each rank computes its own heads with no exchange, the output
 * projection is split by rows so this rank's heads give a partial that g
 * sums):
 *     [Q | K | V] = X Wqkv_i,
 *     O_i[:, head j] = softmax(Q_j K_j^T / sqrt(d) + mask) V_j   per sequence,
 *     Z_i = O_i Wo_i.
 * The per-head formula is the textbook scaled dot-product attention (the
 * pages name heads only); mask: causal (a token sees itself and earlier
 * tokens of its sequence) when `causal` is 1, none when 0.
 * Sizes  : b sequences of s tokens (T = b*s rows, sequence-major), hidden h,
 *          n heads of size d on this rank (d a multiple of 16, 16..128);
 *          n*b < 2^31 and s <= 4194240 (65535 blocks of 64 rows), else
 *          MS_ERR_SHAPE.
 * Inputs : X[T x h]; Wqkv_i[h x 3nd] = [W_Q,i | W_K,i | W_V,i], head j at
 *          columns j*d of each block; Wo_i[nd x h] (the matching rows of W_O);
 *          all bf16.
 * Outputs: QKV[T x 3nd] and O[T x nd] bf16, lse[n x T] fp32 (natural log of
 *          each softmax row's normaliser), all saved for the backward;
 *          Z_i[T x h] fp32 (this rank's partial). */
ms_status attn_shard_fwd(const ms_bf16* X, const ms_bf16* Wqkv_i, const ms_bf16* Wo_i,
                         int64_t b, int64_t s, int64_t h, int64_t n, int64_t d, int32_t causal,
                         ms_bf16* QKV, ms_bf16* O, float* lse, float* Z_i,
                         void* workspace, size_t workspace_bytes, void* stream);

/* Backward of attn_shard_fwd by the chain rule, dZ arriving unchanged through
 * g's backward:
 *     dO = dZ Wo_i^T,  dWo_i = O^T dZ;  per sequence and head, with P the
 *     softmax and delta = rowsum(dO * O):  dV = P^T dO,
 *     dS = P * (dO V^T - delta),  dQ = dS K / sqrt(d),  dK = dS^T Q / sqrt(d);
 *     dWqkv_i = X^T [dQ | dK | dV],  dX_i = [dQ | dK | dV] Wqkv_i^T.
 * The attention core recomputes P from QKV and lse; dO and dQKV are rounded
 * to bf16 in the workspace.  Two kernels (one over query blocks for dQ, which
 * also forms delta, then one over key blocks for dK and dV) keep every sum in
 * a fixed order.
 * Inputs : X, Wqkv_i, Wo_i, dZ[T x h] bf16; QKV, O, lse from the forward.
 * Outputs: dX_i[T x h] fp32 (this rank's partial; f sums it); dWqkv_i[h x 3nd],
 *          dWo_i[nd x h] bf16. */
ms_status attn_shard_bwd(const ms_bf16* X, const ms_bf16* Wqkv_i, const ms_bf16* Wo_i,
                         const ms_bf16* QKV, const ms_bf16* O, const float* lse, const ms_bf16* dZ,
                         int64_t b, int64_t s, int64_t h, int64_t n, int64_t d, int32_t causal,
                         float* dX_i, ms_bf16* dWqkv_i, ms_bf16* dWo_i,
                         void* workspace, size_t workspace_bytes, void* stream);

/* Bytes of device workspace vocab_ce_shard_bwd needs: the per-token records,
 * the bf16 logit gradient [T x v_i] and, when the token contraction of dE_i
 * is split, its fp32 slices.  Returns 0 for invalid sizes. */
size_t vocab_ce_bwd_workspace_bytes(int64_t T, int64_t h, int64_t v_i);

/* Backward of the vocab-parallel logits GEMM fused with cross-entropy (paper
 * notes, "vocab-embedding parallelism", which gives the forward; the backward
 * is the derivative of softmax cross-entropy through L = X E_i).  For the
 * objective sum_t coef[t] loss[t], with coef[t] = grad_scale * dloss[t]
 * (grad_scale alone when dloss is NULL; grad_scale = 1/T gives the mean):
 *     M, S   = the token's statistics over the whole vocabulary, merged from
 *              the ranks' partials in ascending rank order as ce_combine does,
 *     dL[t,j] = coef[t] (exp(L[t,j] - M[t]) / S[t] - [vocab_start + j == target[t]]),
 *     dX_i   = dL E_i^T,   dE_i = X^T dL.
 * L is recomputed (same GEMM as vocab_ce_shard_fwd); dL is rounded to bf16 in
 * the workspace between the GEMMs.
 * Inputs : X[T x h], E_i[h x v_i] bf16; target[T] int64 global ids;
 *          m, s fp32 [t x T] row-major: every rank's vocab_ce_shard_fwd
 *          outputs m_i, s_i, rank r's at offset r*T (the same buffers
 *          ce_combine takes); dloss[T] fp32 or NULL; vocab_start >= 0; t >= 1.
 * Outputs: dX_i[T x h] fp32 (this rank's partial over its vocab columns; the
 *          ranks' partials sum to dX); dE_i[h x v_i] bf16 (this rank's slice).
 * Errors : as the other entry points; MS_ERR_SHAPE also when the workspace
 *          would reach 2^31 bytes (T * v_i * 2 plus records and slices). */
ms_status vocab_ce_shard_bwd(const ms_bf16* X, const ms_bf16* E_i, const int64_t* target,
                             const float* m, const float* s, int32_t t,
                             const float* dloss, float grad_scale,
                             int64_t T, int64_t h, int64_t v_i, int64_t vocab_start,
                             float* dX_i, ms_bf16* dE_i,
                             void* workspace, size_t workspace_bytes, void* stream);

/* Kernels that ms_arm_kernel_events can bracket (one GEMM launch each, or the
 * attention core's launches as one; the split-K reductions and CE
 * tile-combine kernels are not included). */
typedef enum {
  MS_K_CE_GEMM = 0, /* vocab_ce_shard_fwd: X E_i with the fused CE epilogue     */
  MS_K_FWD_H = 1,   /* mlp_shard_fwd:  X A_i (+ b1) with the GeLU epilogue      */
  MS_K_FWD_Z = 2,   /* mlp_shard_fwd:  Y_i B_i -> Z_i                           */
  MS_K_BWD_DH = 3,  /* mlp_shard_bwd:  dZ B_i^T with the GeLU' epilogue -> dH   */
  MS_K_BWD_DB = 4,  /* mlp_shard_bwd:  Y_i^T dZ                                 */
  MS_K_BWD_DA = 5,  /* mlp_shard_bwd:  X^T dH                                   */
  MS_K_BWD_DX = 6,  /* mlp_shard_bwd:  dH A_i^T -> dX_i                         */
  MS_K_CE_BWD_L = 7,  /* vocab_ce_shard_bwd: X E_i recomputed -> dL             */
  MS_K_CE_BWD_DX = 8, /* vocab_ce_shard_bwd: dL E_i^T -> dX_i                   */
  MS_K_CE_BWD_DE = 9, /* vocab_ce_shard_bwd: X^T dL -> dE_i                     */
  MS_K_ATTN_QKV = 10,       /* attn_shard_fwd: X Wqkv_i -> QKV                    */
  MS_K_ATTN_CORE_FWD = 11,  /* attn_shard_fwd: the attention core                 */
  MS_K_ATTN_OUT = 12,       /* attn_shard_fwd: O Wo_i -> Z_i                      */
  MS_K_ATTN_BWD_DO = 13,    /* attn_shard_bwd: dZ Wo_i^T -> dO                    */
  MS_K_ATTN_BWD_DWO = 14,   /* attn_shard_bwd: O^T dZ -> dWo_i                    */
  MS_K_ATTN_CORE_BWD = 15,  /* attn_shard_bwd: delta and the core's dQ, dK, dV    */
  MS_K_ATTN_BWD_DWQKV = 16, /* attn_shard_bwd: X^T dQKV -> dWqkv_i                */
  MS_K_ATTN_BWD_DX = 17,    /* attn_shard_bwd: dQKV Wqkv_i^T -> dX_i              */
  MS_K_COUNT = 18
} ms_kernel;

/* Measurement hook, no effect on results.  Arms two caller-created HIP events
 * (hipEvent_t passed as void*, created with timing enabled) for kernel k: the
 * next call on this host thread of the entry point that launches k records
 * `before` on its stream immediately before that launch and `after`
 * immediately after it, so hipEventElapsedTime(before, after) is that one
 * kernel's device time.  mlp_shard_bwd may run two independent GEMMs, (dB, dH)
 * or (dA, dX), as one paired launch, and vocab_ce_shard_bwd likewise (dE, dX);
 * both ids then bracket that one launch and time it together.  The entry point disarms k when it returns (also on
 * error).  before == after == NULL disarms k.  Errors: MS_ERR_ENUM for an
 * unknown k, MS_ERR_NULL if exactly one event is NULL. */
ms_status ms_arm_kernel_events(ms_kernel k, void* before, void* after);

/* Number of 64-bit words ms_fingerprint writes for a buffer of `bytes` bytes
 * in chunks of `chunk_bytes`: 1 + ceil(bytes / chunk_bytes), or 2 when bytes
 * is 0.  Returns 0 when chunk_bytes is not a positive multiple of 8 (at most
 * 2^40), bytes >= 2^48, or there would be 2^31 chunks or more. */
size_t ms_fingerprint_words(size_t bytes, size_t chunk_bytes);

/* Fingerprint of a device buffer, for finding the first call whose outputs
 * differ between two runs (determinism news item, "debugging methodology":
 * tensors fingerprinted on the GPU, chunk-wise where the order of the data
 * matters).  The hash is XXH64 with seed 0 (xxHash's published
 * specification).  The buffer is split into chunks of chunk_bytes (the last
 * one shorter; one empty chunk when bytes is 0).
 * Output : out[1 + k] = XXH64 of chunk k; out[0] = XXH64 of out[1 ..] as
 *          little-endian 64-bit words, in chunk order.  out is a DEVICE array
 *          of ms_fingerprint_words(bytes, chunk_bytes) uint64.
 * Inputs : buf, a DEVICE pointer, 8-byte aligned; it may hold any bytes.
 * Errors : MS_ERR_SHAPE for sizes ms_fingerprint_words rejects, MS_ERR_NULL,
 *          MS_ERR_ALIGN (8 bytes for buf and out), MS_ERR_ALIAS if out
 *          overlaps buf.  One thread hashes each chunk: a debugging aid, not
 *          a fast path. */
ms_status ms_fingerprint(const void* buf, size_t bytes, size_t chunk_bytes, uint64_t* out, void* stream);

/* Text for the last non-OK status returned on the calling thread ("" if none).
 * The pointer stays valid until the next library call on this thread. */
const char* ms_last_error(void);

/* Library version string (host pointer, static storage). */
const char* ms_version(void);

/* Compute units and peak shader clock of HIP device `device`, as the runtime
 * reports them (hipDeviceAttributeMultiprocessorCount and
 * hipDeviceAttributeClockRate), so that a caller can state the dense bf16 MFMA
 * peak of the card it measures on: compute_units x 4096 flop per clock x clock
 * (gfx950: 4 matrix cores per compute unit, 1024 bf16 flop per clock each).
 * Outputs are HOST pointers.  Errors: MS_ERR_NULL for a NULL output,
 * MS_ERR_HIP if the runtime query fails (no device, bad index). */
ms_status ms_device_info(int32_t device, int32_t* compute_units, int32_t* clock_khz);

#ifdef __cplusplus
}
#endif

#endif /* MSHARD_H */
