/*
 * tiled_attn.h -- C ABI of the fused softmax-attention library for MI355X (gfx950).
 *
 * What is computed. For every (batch b, head h) slice, with S = scale * Q K^T:
 *   O   = softmax(S) V                       (row softmax over the keys)
 *   LSE = ln sum_j exp(S_ij)                 (natural log, one value per query row)
 * as defined by the Lecture 17 page "Tensor Core, HBM, SRAM and FlashAttention"
 * §8.1 (scaled dot-product attention) and computed the way its §8.2-§8.3
 * describe: Q, K and V are tiled, each score tile is formed on chip, a running
 * row maximum and sum are rescaled online, and the full N x N score and
 * probability matrices never reach device memory. The backward entry point
 * returns the exact gradients of sum(O * dO) and, as the CS336 Lecture 5
 * notes §7.2 ("Recomputation") describe, recomputes the score tiles from the
 * saved LSE instead of storing them.
 *
 * Layout. Q, K, V, O, dO, dQ, dK, dV are dense row-major [B, H, N, d] arrays
 * (d innermost, no strides); LSE is a dense [B, H, N] float array. Every
 * pointer is a device pointer. attn_fwd and attn_bwd take Q, K and V of one
 * length N; attn_fwd_ex takes N_q queries against N_k keys (Q, O: [B,H,N_q,d];
 * K, V: [B,H,N_k,d]; LSE: [B,H,N_q]).
 *
 * Causal mask (attn_fwd_ex with ATTN_MASK_CAUSAL). The Lecture 17 page names
 * masks and causal attention (end of §8.3) as part of a real attention
 * kernel without defining them; here query i sees key j iff
 * j <= i + (N_k - N_q), i.e. the N_q queries are the last N_q positions of the
 * key sequence (for N_q = N_k: j <= i). A query that sees no key (only when
 * N_q > N_k) gets O = 0 and LSE = -inf.
 *
 * Supported: d in {64, 128}; 1 <= N with N * d * 4 < 2^31 (one head is
 * addressed with 32-bit byte offsets; any N, a ragged last tile is masked);
 * element type bfloat16 (ATTN_BF16; inputs and outputs bf16, all softmax
 * arithmetic and accumulation in fp32) or float (ATTN_FP32; fp32 everywhere,
 * forward only); scale finite and >= 0. A call with B*H*N == 0 does nothing
 * and returns ATTN_OK.
 *
 * Ownership. The caller owns every buffer, including the backward workspace.
 * The library allocates and frees nothing and keeps no per-call state.
 *
 * Execution. Work is enqueued on `stream` (a hipStream_t; NULL = the null
 * stream) and the call returns without waiting: results are valid once the
 * stream has been synchronised. Calls on different streams that write the
 * same buffers race.
 *
 * Errors. Every argument is validated on the host before anything is
 * enqueued: on a failed check the call returns ATTN_ERR_INVALID_ARGUMENT or
 * ATTN_ERR_UNSUPPORTED, launches nothing, leaves all outputs untouched, and
 * attn_last_error() (per host thread) describes the problem. A failed kernel
 * launch returns ATTN_ERR_HIP with the HIP error text. No C++ exception
 * crosses this interface.
 */
#ifndef TILED_ATTN_H_
#define TILED_ATTN_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  ATTN_OK = 0,
  ATTN_ERR_INVALID_ARGUMENT = 1, /* null/misaligned pointer, negative size, aliasing, bad scale ... */
  ATTN_ERR_UNSUPPORTED = 2,      /* a valid request this library does not implement (e.g. d = 96) */
  ATTN_ERR_HIP = 3               /* the HIP runtime reported an error while enqueuing */
} attn_status;

typedef enum {
  ATTN_BF16 = 0, /* bfloat16 storage, fp32 arithmetic */
  ATTN_FP32 = 1  /* float storage and arithmetic */
} attn_dtype;

typedef enum {
  ATTN_MASK_NONE = 0,   /* every query sees every key */
  ATTN_MASK_CAUSAL = 1  /* query i sees key j iff j <= i + N_k - N_q */
} attn_mask;

/* Library interface version (increments on any ABI change). */
int attn_version(void);

/* Static, human-readable name of a status code. Never NULL. */
const char* attn_status_string(attn_status status);

/* Detail of the last failed call on this host thread ("" if none). The
 * returned string stays valid until the next library call on this thread. */
const char* attn_last_error(void);

/*
 * Forward pass: O = softmax(scale * Q K^T) V and LSE, per (b, h).
 *   q, k, v  [B,H,N,d] inputs of type `dtype`, 16-byte aligned.
 *   o        [B,H,N,d] output of type `dtype`, 16-byte aligned; must not
 *            overlap any input.
 *   lse      [B,H,N] float output, 16-byte aligned; LSE_i = ln sum_j
 *            exp(scale * q_i . k_j) (the log of the softmax denominator, as
 *            the online statistics m + ln l of the Lecture 17 page §8.3).
 * Source: Lecture 17 page §8.1 (definition), §8.2 (tiled, IO-aware flow),
 * §8.3 (online softmax update m' = max(m, max s), alpha = e^(m - m'),
 * l' = alpha l + sum p, o' = alpha o + p V, O = o / l).
 * The library picks the workgroup shape of the kernels from the grid
 * size; two environment variables override that choice (for tests and
 * experiments; results agree within the stated tolerance either way):
 * TILED_ATTN_FWD_WAVES = 2, 4 or 8 waves per workgroup of the bf16 kernels,
 * and TILED_ATTN_FWD_KSPLIT = 1 (never) or 2 (where the launch allows it)
 * for splitting a workgroup's keys between its waves (bf16: two wave groups
 * of an unmasked launch; fp32: the four waves of a 32-query workgroup);
 * TILED_ATTN_FWD_DECODE = 1 keeps bf16 launches with one query per head on
 * the tiled kernels instead of the one-query kernel; TILED_ATTN_FWD_F32_BM =
 * 16 or 32 fixes the query tile of the fp32 key-split kernel at d = 64,
 * and TILED_ATTN_FWD_KSPLIT_BN = 64 or 128 the key tile of the bf16
 * key-split kernel at d = 64.
 */
attn_status attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
                     int64_t B, int64_t H, int64_t N, int64_t d, float scale,
                     attn_dtype dtype, void* stream);

/* Bytes of device workspace attn_fwd_ex needs for `num_splits` key splits:
 * 0 for num_splits = 1, else num_splits * B*H*N_q * (d + 1) * 4 (the fp32
 * partial O and LSE of every split); for num_splits = 0, what the library's
 * own choice needs on the current device (0 if that cannot be queried). 0
 * also for invalid sizes. */
size_t attn_fwd_ex_workspace_bytes(int64_t B, int64_t H, int64_t Nq, int64_t Nk, int64_t d,
                                   int64_t num_splits, attn_dtype dtype);

/* Number of key splits attn_fwd_ex picks with num_splits = 0 on the current
 * device: 1 when the query tiles alone give every compute unit work; else,
 * for bf16 with at least 128 queries, enough splits of the 256-query tiles
 * to fill the chip once if each split keeps at least 2048 keys, otherwise
 * splits of the smaller tiles for about two workgroups per compute unit
 * (each at least 256 keys); with one query per head about one workgroup per
 * compute unit (each split at least 512 keys); at most 128. 0 on invalid
 * sizes or a HIP error. */
int64_t attn_fwd_ex_auto_splits(int64_t B, int64_t H, int64_t Nq, int64_t Nk, int64_t d,
                                attn_dtype dtype);

/*
 * Forward pass with N_q queries against N_k keys, an optional causal mask,
 * and an optional split of the key range.
 *   q         [B,H,Nq,d] input of type `dtype`, 16-byte aligned.
 *   k, v      [B,H,Nk,d] inputs of type `dtype`, 16-byte aligned (may be
 *             NULL when Nk = 0: then every row gets O = 0, LSE = -inf).
 *   o, lse    [B,H,Nq,d] and [B,H,Nq] outputs as in attn_fwd.
 *   mask      ATTN_MASK_NONE or ATTN_MASK_CAUSAL (see the header comment).
 *   num_splits
 *             1: one pass over all keys per query tile (workspace unused,
 *             may be NULL); 2 .. 128: the keys are cut into that many ranges
 *             of whole 128-key tiles (fewer when N_k is short), each range's
 *             attention is computed by its own workgroups into `workspace`
 *             as an fp32 (O_r, LSE_r) pair, and a second kernel merges them
 *             (attn_merge's rule); 0: the library's choice: the
 *             split count attn_fwd_ex_auto_splits reports, or, for bf16
 *             without a mask when the grid of 256-query tiles would end in
 *             a last round of workgroups at most half full, the heads of
 *             the whole rounds unsplit and the remaining heads split over
 *             the keys (wave quantization, CS336 Lecture 5 notes §6.2).
 *             Results agree with the one-pass ones within rounding.
 *   workspace device scratch of at least attn_fwd_ex_workspace_bytes() for
 *             the split count used, 16-byte aligned, owned by the caller,
 *             contents on entry ignored; must not overlap anything else.
 * Source: Lecture 17 page §8.1-§8.3 (the computation), end of §8.3 (masks
 * and causal attention), §9.2 (prefill and decode: few queries against a
 * long key sequence); the split follows the partial results written back to
 * global memory and continued from in the CS336 Lecture 5 transcript
 * (FlashAttention passage). attn_fwd(q,k,v,o,lse,B,H,N,d,...) equals
 * attn_fwd_ex with Nq = Nk = N, ATTN_MASK_NONE, num_splits = 1.
 * Errors as for attn_fwd; also an unknown mask, num_splits outside 0 .. 128,
 * or a missing or too small workspace (ATTN_ERR_INVALID_ARGUMENT).
 */
attn_status attn_fwd_ex(const void* q, const void* k, const void* v, void* o, float* lse,
                        int64_t B, int64_t H, int64_t Nq, int64_t Nk, int64_t d, float scale,
                        attn_mask mask, int64_t num_splits, void* workspace,
                        size_t workspace_bytes, attn_dtype dtype, void* stream);

/*
 * attn_fwd_ex that also records how long its attention kernel ran, into two
 * events of the caller: the timing of GPU work with events on its stream
 * (Lecture 17 page §10.2), here without event commands of their own between
 * back-to-back launches, which would add their gaps to the measured time.
 *   start_event, stop_event
 *             hipEvent_t handles (passed as void*) that the caller created
 *             with timing enabled, or NULL. The library binds them to the
 *             start and the end of the call's attention kernel (its launch
 *             over the query tiles; the merge of key splits, when there is
 *             one, runs after stop_event), so that hipEventElapsedTime of the
 *             two gives that kernel's execution time (with the library's
 *             split of a partial last round, num_splits = 0, from the start
 *             of the first of its two attention launches to the end of the
 *             second). A NULL event is not touched.
 * A call that launches nothing (B*H*Nq == 0) or fails its checks leaves both
 * events as they were. Arguments, results and errors otherwise as for
 * attn_fwd_ex; a non-NULL event must be a live hipEvent_t of the current
 * device (the library cannot check a handle: anything else is undefined),
 * and a launch error the runtime reports returns ATTN_ERR_HIP.
 */
attn_status attn_fwd_ex_timed(const void* q, const void* k, const void* v, void* o, float* lse,
                              int64_t B, int64_t H, int64_t Nq, int64_t Nk, int64_t d, float scale,
                              attn_mask mask, int64_t num_splits, void* workspace,
                              size_t workspace_bytes, attn_dtype dtype, void* stream,
                              void* start_event, void* stop_event);

/*
 * Merge of attention results over disjoint key sets into the result over
 * their union (the rescaling of the online update, Lecture 17 page §8.3,
 * applied to partial results written back to memory, CS336 Lecture 5
 * transcript, FlashAttention passage):
 *   LSE = ln sum_r exp(LSE_r),   O = sum_r exp(LSE_r - LSE) O_r,
 * with parts of LSE_r = -inf weighing nothing (all parts empty: O = 0,
 * LSE = -inf). The same step combines the per-device results of a sequence
 * split across devices.
 *   o_parts    [P,B,H,N,d] float (each part normalised, O_r = o_r / l_r),
 *              16-byte aligned.
 *   lse_parts  [P,B,H,N] float, natural log, 4-byte aligned.
 *   o          [B,H,N,d] output of type `dtype` (bf16: rounded once, RNE),
 *              16-byte aligned; lse [B,H,N] float output, 4-byte aligned.
 *              Outputs must not overlap the inputs or each other.
 * 1 <= P <= 2^20; d in {64, 128}.
 */
attn_status attn_merge(const float* o_parts, const float* lse_parts, int64_t num_parts, int64_t B,
                       int64_t H, int64_t N, int64_t d, void* o, float* lse, attn_dtype dtype,
                       void* stream);

/*
 * Matrix product C = A B^T (the tiled GEMM of the Lecture 17 page §2.1 and
 * §5.2-§5.3; B given as [N, K], both operands contiguous along k).
 *   a  [M, K] bf16, b [N, K] bf16, c [M, N] bf16 output (fp32 accumulation,
 *      rounded once, RNE); dense row-major, 16-byte aligned; c must not
 *      overlap a or b. M*K*2 and N*K*2 < 2^31; K a multiple of 8.
 * One workgroup computes one 128 x 128 tile of C, so the work comes in
 * ceil(M/128) * ceil(N/128) tiles: the unit whose count against the compute
 * units sets wave quantization (CS336 Lecture 5 notes §6.2). K = 0 gives
 * C = 0; M*N = 0 does nothing. bf16 only (ATTN_FP32: ATTN_ERR_UNSUPPORTED).
 */
attn_status attn_matmul_nt(const void* a, const void* b, void* c, int64_t M, int64_t N, int64_t K,
                           attn_dtype dtype, void* stream);

/*
 * MXFP8 quantization (CS336 Lecture 5 transcript, low-precision formats:
 * E4M3 elements, 4 exponent and 3 mantissa bits, with one power-of-two scale
 * stored in 8 bits for every 32 consecutive elements).
 *   x       [batch, rows, cols] bf16 input, 16-byte aligned.
 *   transpose = 0: q [batch, rows, cols] E4M3 bytes, scales [batch, rows,
 *           cols/32]: blocks of 32 along cols (cols % 32 == 0). This is the
 *           layout of Q and K (blocks along d).
 *   transpose = 1: q [batch, cols, rows], the transpose, and scales
 *           [batch, cols, rows/32]: blocks of 32 along the original rows
 *           (rows % 32 == 0). This is the copy V^T [d, N] that O = P V needs
 *           (its reduction runs over the keys).
 * Element codes: OCP E4M3 (bias 7, largest finite 448, no infinities), round
 * to nearest even. A block's scale byte is e + 127 for the smallest e with
 * max|x| <= 448 * 2^e (clamped to 0..254, 0 for an all-zero block), so no
 * element saturates. q is 16-byte aligned; outputs must not overlap x.
 * bf16 input only; finite inputs only.
 */
attn_status attn_quantize_mxfp8(const void* x, int64_t batch, int64_t rows, int64_t cols, int transpose,
                                void* q, void* scales, attn_dtype dtype, void* stream);

/*
 * MXFP8 attention forward: O and LSE of softmax attention on the MXFP8
 * inputs (attn_quantize_mxfp8 layouts), computed with gfx950's MX-scaled
 * matrix instructions; P is rounded to MXFP8 in blocks of 32 keys before
 * O = P V (the softmax statistics stay fp32).
 *   q8, k8       [B,H,N,d] E4M3, 16-byte aligned; q_scales, k_scales
 *                [B,H,N,d/32], 4-byte aligned.
 *   vt8          [B,H,d,N] E4M3 (V transposed), 16-byte aligned; vt_scales
 *                [B,H,d,N/32], 4-byte aligned.
 *   o            [B,H,N,d] bf16 output; lse [B,H,N] float output (as attn_fwd).
 * N a multiple of 32; d in {64, 128}. Error bound against attention on the
 * dequantized inputs: |O - O_ref| <= 2^-4 (P |V|) + rounding of O to bf16.
 */
attn_status attn_fwd_mxfp8(const void* q8, const void* q_scales, const void* k8, const void* k_scales,
                           const void* vt8, const void* vt_scales, void* o, float* lse, int64_t B,
                           int64_t H, int64_t N, int64_t d, float scale, void* stream);

/* Bytes of device workspace attn_bwd needs for these sizes (the per-row
 * term D_i = sum_k dO_ik O_ik, one float per query row). */
size_t attn_bwd_workspace_bytes(int64_t B, int64_t H, int64_t N, int64_t d, attn_dtype dtype);

/*
 * Backward pass: the gradients of sum(O * dO) with respect to Q, K, V.
 *   q, k, v, o, dout   [B,H,N,d] inputs (o and lse as returned by attn_fwd
 *                      for the same q, k, v, scale), 16-byte aligned.
 *   lse                [B,H,N] float input.
 *   dq, dk, dv         [B,H,N,d] outputs of type `dtype` (fp32 accumulation,
 *                      rounded once); must not overlap any input or each other.
 *   workspace          device scratch of at least attn_bwd_workspace_bytes()
 *                      bytes, 16-byte aligned, owned by the caller; its
 *                      contents on entry are ignored.
 * The score and probability tiles are recomputed from q, k and lse; no
 * N x N matrix is stored (CS336 Lecture 5 notes §7.2 "Recomputation"; the
 * CS336 2026 Lecture 05 note, "FlashAttention 解析" ②). Gradient formulas are
 * the exact derivative of the forward definition:
 *   dV = P^T dO, dP = dO V^T, D_i = dO_i . O_i, dS = P * (dP - D),
 *   dQ = scale dS K, dK = scale dS^T Q.
 * bf16 only (ATTN_FP32 returns ATTN_ERR_UNSUPPORTED).
 * The library picks the workgroup shapes of its two sweeps from the grid
 * size; TILED_ATTN_BWD_DKDV_WAVES = 4 or 8 (128 or 256 keys per dK/dV
 * workgroup) and TILED_ATTN_BWD_DQ_WAVES = 4 or 8 (128 or 256 queries per
 * dQ workgroup) override that choice, for tests and experiments; the
 * results are bit-identical either way.
 */
attn_status attn_bwd(const void* q, const void* k, const void* v, const void* o,
                     const void* dout, const float* lse, void* dq, void* dk, void* dv,
                     void* workspace, size_t workspace_bytes,
                     int64_t B, int64_t H, int64_t N, int64_t d, float scale,
                     attn_dtype dtype, void* stream);

/*
 * Backward pass with N_q queries against N_k keys and an optional causal
 * mask: the gradients of sum(O * dO) for O = attn_fwd_ex(q, k, v, mask).
 *   q, o, dout     [B,H,Nq,d] bf16 inputs; lse [B,H,Nq] float (as returned by
 *                  attn_fwd_ex for the same q, k, v, scale, mask; rows with no
 *                  visible key carry LSE = -inf and get dQ = 0).
 *   k, v           [B,H,Nk,d] bf16 inputs.
 *   dq             [B,H,Nq,d] output; dk, dv [B,H,Nk,d] outputs (bf16, fp32
 *                  accumulation, rounded once); no overlaps.
 *   workspace      at least attn_bwd_workspace_bytes(B, H, Nq, d, dtype)
 *                  bytes (one float per query row).
 * A masked (query, key) pair has P = 0 and contributes to no gradient; with
 * Nq = 0 the call writes dK = dV = 0, with Nk = 0 it writes dQ = 0. Tensors
 * with zero rows may be NULL. Sources as for attn_bwd, the mask as for
 * attn_fwd_ex. attn_bwd equals attn_bwd_ex with Nq = Nk = N, ATTN_MASK_NONE.
 */
attn_status attn_bwd_ex(const void* q, const void* k, const void* v, const void* o,
                        const void* dout, const float* lse, void* dq, void* dk, void* dv,
                        void* workspace, size_t workspace_bytes, int64_t B, int64_t H, int64_t Nq,
                        int64_t Nk, int64_t d, float scale, attn_mask mask, attn_dtype dtype,
                        void* stream);

/* Largest B * H * Nq that attn_bwd_ex_noalloc accepts (its fixed scratch). */
#define ATTN_NOALLOC_MAX_ROWS (1 << 22)

/*
 * attn_bwd_ex without a workspace, for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc). Arguments, results and errors are those of attn_bwd_ex
 * minus the workspace; the caller still provides every input and output.
 * The per-row terms D_i go to a fixed array of ATTN_NOALLOC_MAX_ROWS floats
 * (16 MiB) that the library holds on each device it runs on until the
 * process ends; B * H * Nq above ATTN_NOALLOC_MAX_ROWS returns
 * ATTN_ERR_UNSUPPORTED. Nothing is allocated, freed or cleared: every D_i a
 * call reads is written earlier in the same call. All calls on one device
 * share that array, so calls that overlap in time on one device (different
 * streams, or host threads) race; serialise them.
 */
attn_status attn_bwd_ex_noalloc(const void* q, const void* k, const void* v, const void* o,
                                const void* dout, const float* lse, void* dq, void* dk, void* dv,
                                int64_t B, int64_t H, int64_t Nq, int64_t Nk, int64_t d, float scale,
                                attn_mask mask, attn_dtype dtype, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* TILED_ATTN_H_ */
