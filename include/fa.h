/*
 * fa.h -- C ABI of the MI355X (gfx950) exact-attention library libfa.so.
 *
 * What the library computes
 * -------------------------
 * Exact softmax attention, O = softmax(scale * Q K^T) V, evaluated tile by
 * tile with a running (online) row maximum and row sum so that the N x N
 * score matrix never reaches HBM, and the gradients of that attention,
 * recomputing the probabilities from Q, K and the saved per-row
 * log-sum-exp instead of storing them.  The pages this follows:
 *   - "Flash Attention Explained: How IO-Aware Computing Made Long Context
 *     Practical" (institutepm.com), section "How Flash Attention Fixes It:
 *     Tiling and Recomputation": tile the input, fuse into one kernel,
 *     compute softmax incrementally, recompute during the backward pass;
 *   - "What Is Flash Attention? The Real Speed and Memory Gains, Explained"
 *     (bestllmfor.com), section "How Flash Attention works" (tiling and
 *     recomputation; the result is exact up to floating-point rounding);
 *   - the interface shape (Q, K, V as [batch, seq_len, num_heads, head_dim],
 *     a softmax scale defaulting to 1/sqrt(head_dim), a causal flag) is the
 *     one in the holysheep.ai review, "Implementing Flash Attention in Your
 *     Architecture", and its shape checks in "Common Errors and Fixes",
 *     Error 4;
 *   - grouped-query attention (fewer key / value heads than query heads)
 *     and sliding-window attention (each token sees only nearby tokens) are
 *     named as techniques used together with it in "Flash Attention
 *     Explained", section "Flash Attention vs. Related Techniques"; the _ex
 *     entry points take both.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Tensors are caller-owned DEVICE memory.  bf16 tensors are contiguous
 *    [B, N, H, d] (BSHD) with element (b, n, h, c) at ((b*N + n)*H + h)*d + c,
 *    where N is N_q and H the query heads for Q, O, dO, dQ, and N is N_k and
 *    H is H_kv for K, V, dK, dV (N_q = N_k = N and H_kv = H for fa_fwd and
 *    fa_bwd; H_kv = H for the _qk entry points).  Query head h reads key /
 *    value head h / (H / H_kv).  The log-sum-exp is contiguous float32
 *    [B, H, N_q].
 *  - Base pointers must be 16-byte aligned.  Outputs must not alias inputs.
 *  - d must be 64 or 128.  B, H, H_kv, N_q, N_k >= 1 (any length: the
 *    kernels mask ragged tiles), H a multiple of H_kv, and each tensor must
 *    have fewer than 2^31 elements; so must (N_q + 128) * H * d and
 *    (N_k + 128) * H_kv * d (one batch's rows plus the zero-filled rows a
 *    tile copy may run past the end), else FA_ERR_SHAPE.
 *  - scale is any finite float (0 allowed; negative allowed).
 *  - causal: 0 = every key visible; 1 = key j visible to query i iff
 *    j <= i + (N_k - N_q), i.e. the keys are aligned to the end of the
 *    queries (for N_q = N_k: j <= i).  When N_q > N_k the first N_q - N_k
 *    query rows see no key: their output row is 0, their log-sum-exp is
 *    -inf, and their dQ row is 0.
 *  - window (the _ex entry points; 0 = none): with W > 0 query i also sees
 *    only keys j with |i + (N_k - N_q) - j| < W, i.e. with causal = 1 the W
 *    keys ending at its own position (itself and the W - 1 before it).
 *  - stream is a hipStream_t (NULL = the legacy default stream).  Calls only
 *    enqueue work and return; results are valid once the stream is
 *    synchronised.  The library allocates no memory; besides its loaded
 *    kernels, its only state is the fixed scratch array of fa_bwd_noalloc
 *    (one per GPU, below) and that array's address per device.
 *  - Every argument is validated before any HIP call.  On a bad argument
 *    nothing is launched and a negative FA_ERR_* code is returned.  A failed
 *    launch returns FA_ERR_LAUNCH.
 */
#ifndef FA_MI355X_H
#define FA_MI355X_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  FA_OK = 0,
  FA_ERR_NULL = -1,       /* a required pointer is NULL                      */
  FA_ERR_SHAPE = -2,      /* a size not positive, H % H_kv != 0, or overflow */
  FA_ERR_HEADDIM = -3,    /* d is not 64 or 128                              */
  FA_ERR_SEQLEN = -4,     /* reserved: every length >= 1 is accepted          */
  FA_ERR_ALIGN = -5,      /* a base pointer is not 16-byte aligned           */
  FA_ERR_WORKSPACE = -6,  /* workspace NULL or smaller than required         */
  FA_ERR_SCALE = -7,      /* scale is NaN or infinite                        */
  FA_ERR_LAUNCH = -8,     /* the HIP launch reported an error                */
  FA_ERR_ARG = -9,        /* causal not 0/1, window or num_splits < 0, an    */
                          /* output aliases an input or another output, or   */
                          /* (fa_bwd_noalloc) a stream of another device     */
  FA_ERR_SCRATCH = -10    /* fa_bwd_noalloc: B * H * N_q above 2^21 rows     */
} fa_status;

/*
 * Forward pass.
 *   q, k, v : bf16 [B, N, H, d] inputs.
 *   o       : bf16 [B, N, H, d] output, O = softmax(scale * Q K^T) V, rows
 *             normalised, rounded to bf16 (round to nearest even).
 *   lse     : float32 [B, H, N] output, lse[b,h,i] = ln sum_j exp(s_ij) over
 *             the visible keys of row i, where s_ij = scale * q_i . k_j (the
 *             natural-log log-sum-exp of the scaled scores).  The backward
 *             pass consumes it.
 * Accumulation is float32; QK^T and PV run on bf16 matrix cores with the
 * probabilities rounded to bf16 before the PV product.
 * Returns FA_OK or an FA_ERR_* code (see the conventions above).
 */
fa_status fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
                 int B, int H, int N, int d, float scale, int causal, void* stream);

/*
 * Forward pass with N_q query rows and N_k key / value rows (cross attention
 * when they differ; the causal mask is aligned to the end, see above).
 * q, o: [B, N_q, H, d]; k, v: [B, N_k, H, d]; lse: [B, H, N_q].  Otherwise
 * as fa_fwd, which is fa_fwd_qk with N_q = N_k = N.
 */
fa_status fa_fwd_qk(const void* q, const void* k, const void* v, void* o, float* lse,
                    int B, int H, int Nq, int Nk, int d, float scale, int causal, void* stream);

/*
 * Forward pass, general form: H query heads over H_kv key / value heads
 * (grouped-query attention; H_kv = 1 is multi-query attention), N_q query
 * and N_k key rows, and an optional sliding window of W = window keys (see
 * the conventions above).  q, o: [B, N_q, H, d]; k, v: [B, N_k, H_kv, d];
 * lse: [B, H, N_q].  fa_fwd_qk is fa_fwd_ex with H_kv = H, window = 0.
 */
fa_status fa_fwd_ex(const void* q, const void* k, const void* v, void* o, float* lse,
                    int B, int H, int H_kv, int Nq, int Nk, int d, float scale, int causal, int window,
                    void* stream);

/*
 * Forward pass for decoding: few query rows against a long key sequence.
 * Decoding is bound by reading the key / value cache ("What Is Flash
 * Attention? The Real Speed and Memory Gains, Explained", bestllmfor.com,
 * "What you actually gain on a local machine"), so this entry point splits
 * the keys over several workgroups, packs the H / H_kv query heads that
 * share a key / value head into one tile (each key and value is read once
 * per group), and merges the splits by their log-sum-exp.  Arguments and
 * results are those of fa_fwd_ex, plus:
 *   num_splits : key splits per (batch, key head); 0 lets the library
 *                choose (enough workgroups to fill the GPU).
 *   workspace  : device memory of at least fa_decode_workspace_size(...)
 *                bytes (same shape arguments and num_splits), 256-byte
 *                aligned, caller-owned, overwritten; may be NULL when that
 *                size is 0 (a single split).
 * When (H / H_kv) * N_q exceeds 32 rows the tile cannot be packed and the
 * call runs fa_fwd_ex instead (the workspace size is then 0).
 */
size_t fa_decode_workspace_size(int B, int H, int H_kv, int Nq, int Nk, int d, int causal, int window,
                                int num_splits);
fa_status fa_fwd_decode(const void* q, const void* k, const void* v, void* o, float* lse,
                        int B, int H, int H_kv, int Nq, int Nk, int d, float scale, int causal, int window,
                        int num_splits, void* workspace, size_t workspace_bytes, void* stream);

/*
 * Bytes of device workspace fa_bwd needs for this shape: two float32
 * [B, H, N] row terms, -D_i = -sum_c dO_ic * O_ic and -lse_i * log2(e),
 * rounded up to a multiple of 256 bytes.  For fa_bwd_qk and fa_bwd_ex pass
 * N = N_q and H = the number of query heads.
 * Returns 0 for an invalid shape.
 */
size_t fa_bwd_workspace_size(int B, int H, int N, int d);

/*
 * Backward pass by recomputation.
 *   q, k, v, o : bf16 [B, N, H, d], the forward's inputs and its output O.
 *   lse        : float32 [B, H, N] from fa_fwd with the same arguments.
 *   dO         : bf16 [B, N, H, d], gradient of the loss with respect to O.
 *   dq, dk, dv : bf16 [B, N, H, d] outputs, gradients of the loss with
 *                respect to q, k and v (float32 accumulation, rounded to
 *                bf16 at the end).
 *   workspace  : device memory of at least fa_bwd_workspace_size(B,H,N,d)
 *                bytes, 256-byte aligned, caller-owned; its contents on
 *                entry do not matter and are overwritten.
 * The probabilities are recomputed tile by tile as exp(s_ij - lse_i); the
 * score and probability matrices are never stored.  Every output element is
 * summed in a fixed order, so results are identical from run to run.
 * Returns FA_OK or an FA_ERR_* code.
 */
fa_status fa_bwd(const void* q, const void* k, const void* v, const void* o,
                 const float* lse, const void* dO, void* dq, void* dk, void* dv,
                 int B, int H, int N, int d, float scale, int causal,
                 void* workspace, size_t workspace_bytes, void* stream);

/*
 * Backward pass with N_q query rows and N_k key / value rows.  q, o, dO, dq:
 * [B, N_q, H, d]; k, v, dk, dv: [B, N_k, H, d]; lse: [B, H, N_q] from
 * fa_fwd_qk with the same arguments; workspace of at least
 * fa_bwd_workspace_size(B, H, N_q, d) bytes.  Keys that no query sees get
 * dK = dV = 0.  Otherwise as fa_bwd, which is fa_bwd_qk with N_q = N_k = N.
 */
fa_status fa_bwd_qk(const void* q, const void* k, const void* v, const void* o,
                    const float* lse, const void* dO, void* dq, void* dk, void* dv,
                    int B, int H, int Nq, int Nk, int d, float scale, int causal,
                    void* workspace, size_t workspace_bytes, void* stream);

/*
 * Backward pass, general form (the arguments of fa_fwd_ex).  q, o, dO, dq:
 * [B, N_q, H, d]; k, v, dk, dv: [B, N_k, H_kv, d]; lse: [B, H, N_q] from
 * fa_fwd_ex with the same arguments; workspace of at least
 * fa_bwd_workspace_size(B, H, N_q, d) bytes.  dk and dv of a key / value
 * head sum the contributions of every query head that reads it.  Keys that
 * no query sees get dK = dV = 0.  fa_bwd_qk is fa_bwd_ex with H_kv = H,
 * window = 0.
 */
fa_status fa_bwd_ex(const void* q, const void* k, const void* v, const void* o,
                    const float* lse, const void* dO, void* dq, void* dk, void* dv,
                    int B, int H, int H_kv, int Nq, int Nk, int d, float scale, int causal, int window,
                    void* workspace, size_t workspace_bytes, void* stream);

/*
 * Backward pass that allocates nothing and takes no workspace, for callers
 * that cannot allocate device memory (code under HIP graph capture, tight
 * serving loops, harnesses that forbid allocation).  Arguments and results
 * are those of fa_bwd_ex without the workspace: the row terms go to a
 * static scratch array of 16 MiB inside the library, one per GPU, held
 * until the process ends.
 *  - Limit: B * H * N_q <= 2^21 query rows (8 bytes of scratch per row);
 *    larger problems return FA_ERR_SCRATCH and launch nothing.
 *  - stream must belong to the current device (else FA_ERR_ARG).  The first
 *    call on a device looks up that device's scratch address.
 *  - Calls that overlap on one GPU (concurrent streams, or threads) share
 *    the array and race; serialise them.  Nothing in it needs to start at
 *    zero: each call writes every row term before reading it.
 */
fa_status fa_bwd_noalloc(const void* q, const void* k, const void* v, const void* o,
                         const float* lse, const void* dO, void* dq, void* dk, void* dv,
                         int B, int H, int H_kv, int Nq, int Nk, int d, float scale, int causal, int window,
                         void* stream);

/* Static, human-readable text for a status code (never NULL). */
const char* fa_status_string(fa_status s);

/* Library version, major * 10000 + minor * 100 + patch. */
int fa_version(void);

#ifdef __cplusplus
}
#endif

#endif /* FA_MI355X_H */
