/*
 * fa.h -- C ABI of the exact-attention library for AMD Instinct MI355X (gfx950).
 *
 * What is computed (the definitions this library implements):
 *
 *   O = softmax(scale * Q K^T [+ M]) V,  row by row over the keys,
 *
 * the scaled dot-product attention of "Attention Mechanism: Revolusi
 * Representasi Sequence", section 3 ("Scaled Dot-Product Attention: Formula
 * Inti"): Q is (n_q, d), K is (n_k, d), V is (n_k, d) (value width equal to
 * the key width).  With causal = 1 the mask M of section 4.4 ("Causal /
 * Masked Attention") hides key j from query i exactly when j > i, counted
 * from the first row and first key (top-left alignment when n_q != n_k), so
 * every query sees at least key 0.
 *
 * The forward pass streams key/value blocks through on-chip memory with an
 * online softmax (running row maximum and running row sum, "Attention
 * Mechanism" section 13, with the exp(m_old - m_new) factor on the old output
 * that the printed update leaves out), so the n_q x n_k score matrix is never
 * written to device memory ("Apa itu FlashAttention", section "Cara kerja
 * teknik Tiling dan Recomputation"; "Flash Attention Nedir?", sections
 * "Tiling" and "Online Softmax").  It returns O and the per-row natural-log
 * log-sum-exp LSE_i = ln sum_j exp(scale * q_i . k_j) over visible keys.
 *
 * The backward pass recomputes the probabilities block by block from Q, K and
 * the saved LSE instead of storing them ("Apa itu FlashAttention" and "Flash
 * Attention Nedir?", sections on recomputation), and applies the chain rule
 * through O = P V and P = softmax(S):
 *   D_i = sum_c dO_ic O_ic,  P_ij = exp(scale q_i . k_j - LSE_i),
 *   dV = P^T dO,  dP = dO V^T,  dS = P o (dP - D),
 *   dQ = scale dS K,  dK = scale dS^T Q.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * Layout   q, o, dO, dq: contiguous (B, H, n_q, d); k, v, dk, dv: contiguous
 *          (B, H, n_k, d); lse: contiguous (B, H, n_q) float32.
 *          Rows are row-major with d innermost.
 * dtype    FA_DTYPE_BF16: q, k, v, o, dO, dq, dk, dv hold bfloat16 and all
 *          accumulation is float32; results are rounded to nearest-even.
 *          FA_DTYPE_FP32: those tensors hold float32 and every product runs
 *          on float32 matrix cores.  lse is always float32.
 * Pointers All tensor pointers are device pointers.  q, k, v, o, dO, dq, dk,
 *          dv must be 16-byte aligned, lse 4-byte aligned, the backward
 *          workspace 256-byte aligned.
 * Ownership The caller owns every buffer.  The library allocates and frees
 *          nothing, never synchronises, and does not modify inputs.  Outputs
 *          are fully overwritten (never accumulated into) and must not alias
 *          any input; aliasing is undefined.
 * Stream   Work is enqueued on `stream` (a hipStream_t; NULL = the null
 *          stream) and the call returns once it is enqueued; results are
 *          valid after the caller synchronises that stream.  The calls keep
 *          no state and are safe to make from several threads.  They put
 *          nothing on the stream but kernel launches (no allocation, memset,
 *          copy or synchronisation), so a caller may record them into a HIP
 *          graph by stream capture and replay it.
 * Sizes    B, H, n_q, n_k >= 1; d is 32, 64 or 128; B*H and each of n_q, n_k
 *          at most 2^31 - 1; scale finite and >= 0; causal 0 or 1.
 * Errors   Every argument is validated on the host before anything is
 *          launched; on failure the call returns a nonzero fa_status and
 *          leaves all outputs untouched.  A failed launch is reported as
 *          FA_ERR_LAUNCH.  Faults inside a kernel surface as HIP errors at the
 *          caller's next synchronisation.  Non-finite input values are not
 *          checked and propagate into the outputs.  No C++ exception crosses
 *          this interface and nothing is printed.
 */
#ifndef EXACT_ATTENTION_FA_H
#define EXACT_ATTENTION_FA_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum fa_status {
  FA_OK = 0,
  FA_ERR_INVALID_ARG = 1,   /* NULL pointer, size < 1, bad causal, non-finite or negative scale */
  FA_ERR_UNSUPPORTED = 2,   /* head width d or dtype the library does not provide */
  FA_ERR_WORKSPACE = 3,     /* backward workspace missing or smaller than required */
  FA_ERR_LAUNCH = 4,        /* the HIP runtime refused a kernel launch */
  FA_ERR_ALIGNMENT = 5,     /* a tensor pointer is not aligned as required */
  FA_ERR_TOO_LARGE = 6      /* sizes beyond the fixed scratch of fa_backward_noalloc */
} fa_status;

typedef enum fa_dtype {
  FA_DTYPE_FP32 = 0,
  FA_DTYPE_BF16 = 1
} fa_dtype;

/* Forward pass.  Writes o (B,H,n_q,d; dtype) and lse (B,H,n_q; float32).
 * One kernel launch on `stream`.  bf16 shapes with few query rows per key
 * (n_k >= 1024 and B*H*ceil(n_q/256) <= 32, or <= 64 for d <= 64) run on the
 * split-key kernel of fa_decode with one chunk, which spreads each row
 * block's keys over several waves (no workspace); all others on the forward
 * kernel.  Both compute the same function and agree within rounding. */
int fa_forward(const void* q, const void* k, const void* v, void* o, float* lse,
               int B, int H, int n_q, int n_k, int d, float scale, int causal,
               int dtype, void* stream);

/* Bytes of device workspace the backward pass needs for these sizes: two
 * float32 (B,H,n_q) row vectors (the row sums D and LSE * log2(e)), each
 * padded to a multiple of 256 bytes with at least 16 bytes of slack.
 * Returns 0 for invalid or unsupported sizes. */
size_t fa_backward_workspace_size(int B, int H, int n_q, int n_k, int d, int dtype);

/* Backward pass from the saved o and lse of fa_forward (same q, k, v, scale,
 * causal).  Writes dq, dk, dv in dtype.  `workspace` is caller-owned device
 * memory of at least fa_backward_workspace_size(...) bytes, 256-byte aligned;
 * its contents on entry do not matter.  Runs the three stages below in order
 * on `stream`; it is deterministic (no atomics; bitwise repeatable). */
int fa_backward(const void* q, const void* k, const void* v, const void* o,
                const void* dO, const float* lse, void* dq, void* dk, void* dv,
                void* workspace, size_t workspace_bytes,
                int B, int H, int n_q, int n_k, int d, float scale, int causal,
                int dtype, void* stream);

/* fa_backward without a workspace argument and without allocating anything,
 * for callers that cannot allocate device memory: code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation.  The
 * workspace is a fixed scratch array of 16 MiB that the library holds on
 * each GPU it runs on until the process ends, so B*H*n_q may be at most
 * about 2 million rows (2 * round_up(4 B*H*n_q + 16, 256) <= 16 MiB);
 * larger sizes return FA_ERR_TOO_LARGE before anything is launched.  The
 * first call on each device is its set-up: the library looks up the
 * scratch's device address (hipGetSymbolAddress), and the HIP runtime may
 * map the array on that device then -- make one call before a graph capture
 * or an allocation-free region.  Later calls touch no allocator.  One K/V
 * head per query head.  Results are bit for bit those of fa_backward.
 * `stream` must belong to the calling thread's current device (else
 * FA_ERR_INVALID_ARG).  All calls on one GPU share its scratch: two calls
 * that overlap in time on one GPU (different streams, or threads) race and
 * must be ordered by the caller.  The scratch needs no clearing: each call
 * writes the row vectors before it reads them, and the few entries read past
 * their end (rows past n_q, masked) never reach a result.  Other arguments
 * and errors as fa_backward. */
int fa_backward_noalloc(const void* q, const void* k, const void* v, const void* o,
                        const void* dO, const float* lse, void* dq, void* dk, void* dv,
                        int B, int H, int n_q, int n_k, int d, float scale, int causal,
                        int dtype, void* stream);

/* Backward stage 1: writes into `workspace` the float32 row sums
 * D_i = sum_c dO_ic * o_ic (the row term of the softmax gradient, from the
 * saved output) and LSE_i * log2(e).  Workspace as for fa_backward. */
int fa_backward_preprocess(const void* o, const void* dO, const float* lse,
                           void* workspace, size_t workspace_bytes,
                           int B, int H, int n_q, int d, int dtype, void* stream);

/* Backward stage 2: dk and dv, from the workspace of stage 1.  One pass over
 * the query blocks for every key block, recomputing P from the saved LSE,
 * with dV = P^T dO and dK = scale dS^T Q. */
int fa_backward_dkdv(const void* q, const void* k, const void* v, const void* dO,
                     const void* workspace, size_t workspace_bytes, void* dk, void* dv,
                     int B, int H, int n_q, int n_k, int d, float scale, int causal,
                     int dtype, void* stream);

/* Backward stage 3: dq = scale dS K, from the workspace of stage 1.  One
 * pass over the key blocks for every query block, recomputing P and dP. */
int fa_backward_dq(const void* q, const void* k, const void* v, const void* dO,
                   const void* workspace, size_t workspace_bytes, void* dq,
                   int B, int H, int n_q, int n_k, int d, float scale, int causal,
                   int dtype, void* stream);

/* Grouped-query and multi-query attention ("Attention Mechanism: Revolusi
 * Representasi Sequence", section 12 "GQA vs MQA -- KV Cache Optimization"):
 * k and v hold H_kv heads, (B,H_kv,n_k,d), and query heads
 * h = j*(H/H_kv) .. (j+1)*(H/H_kv) - 1 all attend to K/V head j -- the same
 * result as repeating every K/V head H/H_kv times along the head axis.
 * H_kv = H is fa_forward; H_kv = 1 is multi-query attention.  H_kv must
 * divide H (otherwise FA_ERR_INVALID_ARG); everything else as fa_forward. */
int fa_forward_gqa(const void* q, const void* k, const void* v, void* o, float* lse,
                   int B, int H, int H_kv, int n_q, int n_k, int d, float scale,
                   int causal, int dtype, void* stream);

/* Backward pass of fa_forward_gqa.  dk and dv are (B,H_kv,n_k,d): the
 * gradient of a shared K/V head is the sum over the query heads of its
 * group (the adjoint of the repetition).  So that few K/V heads still give
 * enough parallel work, a group's query heads may be split into runs whose
 * float32 partial sums the workspace holds and a final pass adds up in a
 * fixed order (results are repeatable bit for bit).  The workspace must
 * hold fa_backward_gqa_workspace_size(B, H, H_kv, n_q, n_k, d, dtype) bytes
 * (equal to fa_backward_workspace_size when H_kv = H), else
 * FA_ERR_WORKSPACE; dq and other errors as for fa_backward. */
size_t fa_backward_gqa_workspace_size(int B, int H, int H_kv, int n_q, int n_k, int d, int dtype);

int fa_backward_gqa(const void* q, const void* k, const void* v, const void* o,
                    const void* dO, const float* lse, void* dq, void* dk, void* dv,
                    void* workspace, size_t workspace_bytes,
                    int B, int H, int H_kv, int n_q, int n_k, int d, float scale,
                    int causal, int dtype, void* stream);

/* Extended forward pass: shared K/V heads as fa_forward_gqa, plus where each
 * query row sits on the key axis and a sliding window.  Query row i is at
 * absolute position p = i + q_offset; key j is hidden when causal and j > p
 * ("Attention Mechanism", section 4.4, with the rows shifted by q_offset:
 * q_offset = n_k - n_q aligns the last query with the last key, as when new
 * queries attend to a longer cache) and, when window >= 0, when
 * |p - j| > window (section 4.5 "Sparse Attention": only the +-w
 * neighbours).  q_offset = 0, window = -1 is fa_forward_gqa.  A row that sees
 * no key gets o = 0 and lse = -inf.  |q_offset| <= 2^29,
 * -1 <= window <= 2^29 and, when either is in use, n_q, n_k <= 2^29;
 * otherwise FA_ERR_INVALID_ARG. */
int fa_forward_ext(const void* q, const void* k, const void* v, void* o, float* lse,
                   int B, int H, int H_kv, int n_q, int n_k, int d, float scale,
                   int causal, int q_offset, int window, int dtype, void* stream);

/* Forward pass merged into a prior result: one step of attention whose keys
 * arrive in chunks ("Attention Mechanism", section 16 "Ring Attention": each
 * worker holds a slice of the keys and the query rows visit every slice),
 * with the online softmax's rescaling ("Attention Mechanism", section 13:
 * the old output is weighted by the exponential of the change of the running
 * maximum) applied to whole results in the kernel's epilogue, so a step needs
 * no separate merge pass.
 *   o_prior, lse_prior  the rows' result over the keys seen so far:
 *                       (B,H,n_q,d) in prior_dtype and (B,H,n_q) float32
 *                       natural-log LSE; a row with lse_prior = -inf has no
 *                       prior (its o_prior is never read and may hold anything)
 *   o, lse              receive the result over those keys and this call's
 *                       k, v: (B,H,n_q,d) in out_dtype and (B,H,n_q) float32
 * With this call's own result (O_n, LSE_n) -- what fa_forward_ext would
 * return for the same arguments -- lse = ln(exp(lse_prior) + exp(LSE_n)) and
 * o = exp(lse_prior - lse) o_prior + exp(LSE_n - lse) O_n; a row without keys
 * on either side gets o = 0, lse = -inf.  Chaining calls over key chunks
 * [a, b) with query offset q_offset - a, starting from lse_prior = -inf,
 * gives the result over all keys.  prior_dtype and out_dtype are each
 * FA_DTYPE_FP32 or dtype (bf16 inputs may keep a float32 running result);
 * else FA_ERR_UNSUPPORTED.  o may be o_prior itself when the two dtypes
 * match and lse may be lse_prior (in-place accumulation); any other overlap
 * between them is FA_ERR_INVALID_ARG.  The other arguments, alignment and
 * errors as fa_forward_ext; always the forward kernel (never the split-key
 * route), one launch on `stream`. */
int fa_forward_merge(const void* q, const void* k, const void* v, const void* o_prior,
                     const float* lse_prior, int prior_dtype, void* o, float* lse, int out_dtype,
                     int B, int H, int H_kv, int n_q, int n_k, int d, float scale, int causal,
                     int q_offset, int window, int dtype, void* stream);

/* Backward pass of fa_forward_ext (same q_offset and window); workspace as
 * for fa_backward_gqa.  For attention over key chunks (fa_forward_merge),
 * the call for one chunk with the final o and lse over all keys gives that
 * chunk's exact dk, dv and its share of dq: the full dq is the sum over the
 * chunks. */
int fa_backward_ext(const void* q, const void* k, const void* v, const void* o,
                    const void* dO, const float* lse, void* dq, void* dk, void* dv,
                    void* workspace, size_t workspace_bytes,
                    int B, int H, int H_kv, int n_q, int n_k, int d, float scale,
                    int causal, int q_offset, int window, int dtype, void* stream);

/* Merge of attention results over disjoint key sets into the result over
 * their union ("Attention Mechanism", section 13: the online softmax's
 * rescaling applied to whole parts; section 16 "Ring Attention": attention
 * over keys spread across workers).  Part p holds o_p (normalised over its
 * own keys) and lse_p; the result is lse = ln sum_p exp(lse_p) and
 * o = sum_p exp(lse_p - lse) o_p.  Parts with lse_p = -inf (no visible key)
 * contribute nothing; a row with -inf in every part gets o = 0, lse = -inf.
 *   o_parts    (n_parts, rows, d), parts_dtype (FA_DTYPE_FP32 or _BF16)
 *   lse_parts  (n_parts, rows) float32
 *   o          (rows, d), out_dtype;  lse (rows) float32
 * The parts of fa_forward_ext calls over key chunks [a, b) with query offset
 * q_offset - a (rows = B*H*n_q) merge into the call over all keys.  n_parts,
 * rows >= 1; d in {32, 64, 128}; o_parts, o 16-byte aligned; outputs must not
 * alias the parts.  Asynchronous on `stream`. */
int fa_lse_merge(const void* o_parts, const float* lse_parts, void* o, float* lse,
                 int n_parts, long long rows, int d, int parts_dtype, int out_dtype,
                 void* stream);

/* Split-KV decoding ("Attention Mechanism", section 8, "Key-Value (KV)
 * Cache"): a few query rows (q: (B,H,n_q,d)) against a long cache (k, v:
 * (B,H_kv,n_k,d)), with the masks of fa_forward_ext -- for new tokens at the
 * end of the cache pass causal = 1, q_offset = n_k - n_q.  The key axis is
 * cut into n_splits chunks of whole 128-key blocks; each chunk's result goes
 * to the workspace and fa_lse_merge's rule combines them into o (B,H,n_q,d)
 * and lse (B,H,n_q).  bf16 only (FA_ERR_UNSUPPORTED otherwise); other
 * arguments and errors as fa_forward_ext.  n_splits >= 1 (fa_decode_splits
 * gives the library's choice); with more than one chunk the workspace must
 * hold fa_decode_workspace_size(B, H, n_q, d, n_splits) bytes, 256-byte
 * aligned (else FA_ERR_WORKSPACE / FA_ERR_ALIGNMENT); with one chunk it may
 * be NULL. */
int fa_decode(const void* q, const void* k, const void* v, void* o, float* lse,
              void* workspace, size_t workspace_bytes,
              int B, int H, int H_kv, int n_q, int n_k, int d, float scale,
              int causal, int q_offset, int window, int n_splits, int dtype, void* stream);

/* Workspace bytes fa_decode needs for n_splits chunks (0 for one chunk;
 * 0 for invalid sizes). */
size_t fa_decode_workspace_size(int B, int H, int n_q, int d, int n_splits);

/* The number of chunks fa_decode uses by default for a shape: enough
 * workgroups to fill the GPU, chunks of at least 256 keys (>= 1; 0 for
 * invalid sizes). */
int fa_decode_splits(int B, int H, int H_kv, int n_q, int n_k);

/* Static text for a status code ("unknown status" for other values). */
const char* fa_status_string(int status);

/* Library interface version (major * 10000 + minor * 100 + patch). */
int fa_version(void);

#ifdef __cplusplus
}
#endif

#endif /* EXACT_ATTENTION_FA_H */
