/*
 * Exact scaled-dot-product attention for AMD Instinct MI355X (gfx950).
 *
 * C ABI of libattn.so.  Plain pointers and sizes only; every pointer argument
 * except those named "host" is a device address.  The library never
 * allocates or frees memory, never synchronises, and keeps no state between
 * calls: it is re-entrant, and calls on different streams may overlap.  Work
 * is enqueued on `stream` (a hipStream_t; NULL means the default stream) and
 * the function returns once it is launched.  Inputs must stay unchanged and
 * outputs untouched until the stream reaches the call.
 *
 * Layouts are contiguous, row-major, with the head dimension innermost.
 *
 * Error convention: 0 on success, a negative ATTN_ERR_* code otherwise.
 * Every check except ATTN_ERR_HIP runs on the host before any HIP call, so a
 * rejected call has no side effect.  attn_strerror() names a code.
 */
#ifndef EXACT_ATTN_H
#define EXACT_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Element types of Q, K, V and O. */
#define ATTN_F32 0  /* IEEE fp32 */
#define ATTN_BF16 1 /* bfloat16; accumulation is always fp32 */

#define ATTN_OK 0
#define ATTN_ERR_INVALID_ARG (-1) /* null or misaligned pointer, bad size, bad scale */
#define ATTN_ERR_UNSUPPORTED (-2) /* head dim not 64/128, dtype, verify query packing */
#define ATTN_ERR_WORKSPACE (-3)   /* verify workspace smaller than required */
#define ATTN_ERR_HIP (-4)         /* the kernel launch failed */
#define ATTN_ERR_TOO_LARGE (-5)   /* attn_verify_noalloc: sizes beyond its static scratch */

/*
 * attn_fwd -- O = softmax(scale * Q K^T + mask) V, and per-row LSE.
 *
 * Definition: "Warmup Guide -- Inference Optimization at Depth", Ch.1
 * (S = QK^T, P = softmax(S), O = PV) with Ch.4's 1/sqrt(d) scale and causal
 * mask; computed as in its Ch.4 / Ch.3 (tiles of Q, K/V streamed on chip,
 * online softmax with running max and denominator, one normalised write per
 * row block; the score matrix is never stored) and as the Mechanics section
 * of "FlashAttention, speculative decoding, quantisation and parallelism"
 * sketches it.  The result equals the plain definition up to floating-point
 * rounding.
 *
 *   q    [B, H,   Sq, d]  dtype           (read)
 *   k, v [B, Hkv, Sk, d]  dtype           (read)
 *   o    [B, H,   Sq, d]  dtype           (written)
 *   lse  [B, H,   Sq]     fp32            (written; may be NULL to skip)
 *
 * Query head h reads KV head h / (H / Hkv) (grouped-query attention).
 * causal != 0: key j is visible to query i iff j <= i + Sk - Sq (the mask is
 * aligned to the bottom-right corner; for Sq == Sk this is j <= i).
 * scale must be finite and > 0 (normally 1/sqrt(d)).
 * lse = ln(sum_j exp(scale * q_i.k_j)) over the visible keys, natural log of
 * the scaled logits.  A row with no visible key gets O = 0 and lse = -inf.
 * Rounding: O is rounded to nearest-even from fp32.  In the bf16 path the
 * probabilities are rounded to bf16 before the P.V product; O is divided by
 * the sum of those rounded probabilities (its weights sum to one), and lse
 * uses the sum of the unrounded fp32 probabilities.
 *
 * Sizes: B, Sq, Sk >= 0 (zero sizes are allowed; B*Sq == 0 is a no-op and a
 * pointer whose tensor is empty may be NULL); Sq, Sk <= 2^30 and
 * d in {64, 128} (else ATTN_ERR_UNSUPPORTED); H, Hkv >= 1 with H % Hkv == 0.
 * Pointers must be 16-byte aligned (lse: 4-byte).
 *
 * Work order: in a bf16 causal call with at least 32 blocks of 256 query
 * rows per head (a multiple of 8) and B*H a multiple of 16, the lightest
 * quarter of every head's blocks is handed out at run time through a counter
 * in a small static device array of the library (64 counters per GPU, taken
 * in turn; a call waits, on the GPU, for the previous call that used its
 * counter, so calls on different streams never share one).  A call made
 * while its stream is being captured into a graph uses a fixed order
 * instead.  O and lse are bit-for-bit the same either way.  The stream must
 * belong to the current device.
 */
int attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
             int B, int H, int Hkv, int Sq, int Sk, int d,
             int causal, float scale, int dtype, void* stream);

/*
 * attn_verify_workspace_bytes -- bytes of device workspace attn_verify needs
 * for these sizes: fp32 partial outputs and LSEs for every (sequence, query
 * head, new token, piece slot), where a segment (sequence, KV head) is cut
 * into at most ceil(256 / Hkv) + 2 pieces, plus one int32 piece count per
 * segment.  Independent of the cache lengths.  Returns 0 for invalid sizes.
 */
size_t attn_verify_workspace_bytes(int B, int H, int Hkv, int kq, int d);

/*
 * attn_verify -- attention of kq new query tokens per sequence against a
 * ragged KV cache: the verify step of speculative decoding, where the target
 * model scores all drafted positions in one pass ("FlashAttention,
 * speculative decoding, quantisation and parallelism", Mechanics /
 * Speculative decoding).  Computed as Flash-Decoding ("Making Decode Fast",
 * §5: split the keys across compute units, then a small final combine): the
 * keys of all (sequence, KV head) segments are cut into 256 equal slices, a
 * split kernel writes a partial (O_p, LSE_p) per piece of segment in a slice,
 * and a merge kernel combines the pieces with the two-block update of
 * "Warmup Guide", Ch.3.
 *
 *   q                 [B, H, kq, d]                 bf16 (read)
 *   k_cache, v_cache  [B, Hkv, cache_stride, d]     bf16 (read; only the first
 *                                                   seqlens_k[b] rows of each
 *                                                   (b, head) are read)
 *   seqlens_k         [B] int32 (device): valid keys of sequence b, which
 *                     include the kq new tokens' keys as the last kq rows
 *   o                 [B, H, kq, d]                 bf16 (written)
 *   lse               [B, H, kq]                    fp32 (written; may be NULL)
 *   workspace         attn_verify_workspace_bytes(...) bytes, caller-owned,
 *                     16-byte aligned, contents ignored
 *
 * Query i of sequence b sees keys [0, seqlens_k[b] - kq + i] (causal among
 * the new tokens, bottom-right aligned).  max_seqlen_k is a host-side bound
 * with max_seqlen_k >= every seqlens_k[b] and max_seqlen_k <= cache_stride;
 * device values above it are clamped to it, negative values to 0.  Rows with
 * no visible key get O = 0 and lse = -inf.  dtype must be ATTN_BF16;
 * d in {64, 128}; (H / Hkv) * kq <= 64, else ATTN_ERR_UNSUPPORTED (the query
 * rows that share one KV head are packed into one or two 32-row matrix
 * tiles, so each cache byte is read once).
 */
int attn_verify(const void* q, const void* k_cache, const void* v_cache,
                const int32_t* seqlens_k, int max_seqlen_k, int cache_stride,
                void* o, float* lse, int B, int H, int Hkv, int kq, int d,
                float scale, int dtype, void* workspace, size_t workspace_bytes,
                void* stream);

/*
 * attn_verify_noalloc -- attn_verify without a workspace, for callers that
 * cannot allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid allocation).  Same arguments (minus the
 * workspace), kernels, semantics and bitwise results as attn_verify.  The
 * partials live in a static device array of 32 MiB that each GPU holds from
 * the library's load until the process ends; its address on the current
 * device is looked up on the first call on that device.  The stream must
 * belong to the current device.  Sizes whose
 * attn_verify_workspace_bytes(B, H, Hkv, kq, d) exceed 32 MiB are rejected
 * with ATTN_ERR_TOO_LARGE before any HIP call (the verify workload of 8
 * sequences, 32 query heads over 8 KV heads, kq = 5, d = 128 needs 22.5 MB).
 * The call allocates and frees nothing.  Every call on one GPU shares that
 * GPU's array and overwrites it: calls that overlap on one device (on
 * different streams, or from different host threads without ordering) race
 * and give wrong results; order them.  Nothing needs clearing between calls
 * (each call writes every slot it reads).
 */
int attn_verify_noalloc(const void* q, const void* k_cache, const void* v_cache,
                        const int32_t* seqlens_k, int max_seqlen_k, int cache_stride,
                        void* o, float* lse, int B, int H, int Hkv, int kq, int d,
                        float scale, int dtype, void* stream);

/*
 * attn_verify_tree -- attn_verify for a draft *tree* instead of a chain
 * ("Making Decode Fast", §3: proposing a tree of candidates and verifying it
 * with tree attention in one pass raises the acceptance length).  The kq new
 * tokens of sequence b are tree nodes whose keys are the last kq of its
 * seqlens_k[b] keys (node t at position seqlens_k[b] - kq + t).  Node i sees
 * every earlier cache key and new key t iff bit t of tree_mask[b][i] is set
 * (normally its ancestors and itself).  The causal chain is
 * tree_mask[b][i] = 2^(i+1) - 1, for which the result equals attn_verify's
 * bit for bit.  A row that sees no key gets O = 0, lse = -inf.
 *
 *   tree_mask   [B, kq] uint32 (device); kq <= 32 (ATTN_ERR_UNSUPPORTED
 *               above), besides the packing limit (H / Hkv) * kq <= 64
 *
 * All other arguments, the workspace and the errors are those of
 * attn_verify, plus ATTN_ERR_INVALID_ARG for a null or misaligned tree_mask
 * when B > 0.
 */
int attn_verify_tree(const void* q, const void* k_cache, const void* v_cache,
                     const int32_t* seqlens_k, int max_seqlen_k, int cache_stride,
                     const uint32_t* tree_mask, void* o, float* lse, int B, int H, int Hkv,
                     int kq, int d, float scale, int dtype, void* workspace,
                     size_t workspace_bytes, void* stream);

/*
 * attn_verify_paged -- attn_verify on a paged KV cache ("Warmup Guide --
 * Inference Optimization at Depth", Ch.8: the cache is stored in fixed-size
 * blocks of tokens and each sequence owns a block table mapping its logical
 * blocks to physical ones; the attention kernel gathers K/V through the table,
 * once per tile, as the guide's interview answer on FlashAttention and
 * PagedAttention describes).  Same queries, outputs, masking, workspace and
 * semantics as attn_verify; only the cache addressing differs:
 *
 *   k_pages, v_pages  [num_pages, Hkv, page_size, d]  bf16 (read)
 *   block_table       [B, max_blocks_per_seq] int32 (device): logical block i
 *                     of sequence b (its keys i*page_size .. +page_size-1) is
 *                     physical page block_table[b][i].  Pages may be shared
 *                     between sequences (prefix sharing).  Only the entries
 *                     covering seqlens_k[b] keys are read.  An entry outside
 *                     [0, num_pages) maps its block to no storage: its keys
 *                     do not exist and no query attends to them (a row left
 *                     with no key gets O = 0 and lse = -inf).
 *   page_size         keys per page: a power of two in [16, 4096] (each
 *                     16-key half of the kernel's 32-key step reads one
 *                     page)
 *   max_seqlen_k      host bound, <= max_blocks_per_seq * page_size
 *
 * Workspace: attn_verify_workspace_bytes(B, H, Hkv, kq, d) bytes.  Errors as
 * for attn_verify, plus ATTN_ERR_INVALID_ARG for a page size outside the
 * supported set or a null block table when max_seqlen_k > 0.
 */
int attn_verify_paged(const void* q, const void* k_pages, const void* v_pages,
                      const int32_t* block_table, int max_blocks_per_seq, int num_pages,
                      int page_size, const int32_t* seqlens_k, int max_seqlen_k,
                      void* o, float* lse, int B, int H, int Hkv, int kq, int d,
                      float scale, int dtype, void* workspace, size_t workspace_bytes,
                      void* stream);

/*
 * attn_bwd_workspace_bytes -- bytes of device workspace attn_bwd needs: two
 * fp32 values per query row (rowsum(dO * O) and the base-2 LSE), each array
 * aligned to 256 bytes.  Returns 0 for invalid sizes.
 */
size_t attn_bwd_workspace_bytes(int B, int H, int Sq);

/*
 * attn_bwd -- gradients of exact attention with respect to Q, K and V for an
 * upstream gradient dO of its output ("Warmup Guide -- Inference
 * Optimization at Depth", Ch.4, backward pass: P is recomputed from Q, K and
 * the forward pass's per-row statistics instead of being stored).  With
 * S = scale Q K^T (masked as in attn_fwd), P = softmax(S), O = P V:
 *   dV = P^T dO, dP = dO V^T, dS = P * (dP - rowsum(dO * O)),
 *   dQ = scale dS K, dK = scale dS^T Q;
 * grouped-query heads sum into the dK, dV of their KV head.
 *
 *   q, o, dout   [B, H, Sq, d]     bf16 (read; o and lse as written by attn_fwd)
 *   k, v         [B, Hkv, Sk, d]   bf16 (read)
 *   lse          [B, H, Sq]        fp32 (read; natural log, -inf for empty rows)
 *   dq           [B, H, Sq, d]     bf16 (written)
 *   dk, dv       [B, Hkv, Sk, d]   bf16 (written)
 *   workspace    attn_bwd_workspace_bytes(B, H, Sq) bytes, 16-byte aligned
 *
 * Accumulation is fp32; the outputs are rounded to bf16 (nearest even).
 * Rows that see no key get dQ = 0 and contribute nothing to dK, dV.  Keys no
 * query sees get dK = dV = 0.  No atomics: results are deterministic.
 * dtype must be ATTN_BF16; d in {64, 128}; Sq, Sk <= 2^30; causal is
 * bottom-right aligned.  Errors as for attn_fwd, plus ATTN_ERR_WORKSPACE.
 * Work order: in a causal call with at least 32 blocks of 256 query rows (a
 * multiple of 4) and B*H a multiple of 8, or at least 16 blocks of 256 keys
 * (a multiple of 4) and B*Hkv a multiple of 8, the lightest quarter of those
 * blocks is claimed at run time through counters in a static device array,
 * as in attn_fwd (one counter slot per call, taken in turn, ordered after the
 * slot's previous call; the fixed order under stream capture).  The
 * gradients are bit-for-bit the same either way.
 */
int attn_bwd(const void* q, const void* k, const void* v, const void* o, const void* dout,
             const float* lse, void* dq, void* dk, void* dv, int B, int H, int Hkv, int Sq,
             int Sk, int d, int causal, float scale, int dtype, void* workspace,
             size_t workspace_bytes, void* stream);

/*
 * attn_spec_accept_workspace_bytes -- bytes of device workspace
 * attn_spec_accept needs: two int64 sums per (sequence, 4096-entry chunk of
 * the vocabulary), then one int32 per sequence (its first rejected
 * position, passed from the first kernel to the second).  Returns 0 for
 * invalid sizes.
 */
size_t attn_spec_accept_workspace_bytes(int B, int V);

/*
 * attn_spec_accept -- the acceptance rule of speculative decoding, applied to
 * B sequences after one verify pass ("Warmup Guide -- Inference Optimization
 * at Depth", Ch.6: accept drafted token x with probability min(1, p(x)/q(x));
 * at the first rejection resample from norm(max(0, p - q)) and discard the
 * rest of the draft; "FlashAttention, speculative decoding, quantisation and
 * parallelism", Mechanics / Speculative decoding: if all k drafts survive, one
 * more token is sampled from the target's distribution at position k).  The
 * output is then distributed exactly as sampling the target alone.
 *
 *   draft_tokens  [B, k]       int32  drafted tokens (device)
 *   draft_probs   [B, k, V]    fp32   draft distributions q_i (device)
 *   target_probs  [B, k+1, V]  fp32   target distributions p_i (device)
 *   u_accept      [B, k]       fp32   uniforms in [0, 1): draft i of
 *                                     sequence b is accepted iff
 *                                     u_accept[b][i] < min(1, p_i(x)/q_i(x))
 *                                     (fp32, correctly rounded division); a
 *                                     token with q_i(x) = 0 is accepted iff
 *                                     p_i(x) > 0; a token outside [0, V) is
 *                                     rejected
 *   u_sample      [B]          fp32   uniform in [0, 1) that picks the extra
 *                                     token by inverse CDF
 *   n_accepted    [B]          int32  written: accepted drafts j (0..k)
 *   out_tokens    [B, k+1]     int32  written: the j accepted drafts, the
 *                                     sampled token, then -1
 *
 * Sampling: weights w (the residual max(0, p_j - q_j) after a rejection at
 * j, else p_k), each clamped to [0, 1] (NaN as 0), are put on a fixed-point
 * grid W = floor(w * 2^40); with T = floor(u_sample * sum W) (clamped to
 * [0, sum W - 1]) the token is the first index whose running sum of W exceeds
 * T.  A residual with no mass falls back to p_j; a distribution with no mass
 * at all gives token -1.  The random numbers are the caller's; the library
 * draws none.
 *
 * Sizes: B, k >= 0; 1 <= V <= 2^22 (ATTN_ERR_UNSUPPORTED above).  Pointers
 * must be 4-byte aligned (workspace: 8-byte), non-null unless their tensor is
 * empty.  Errors: ATTN_ERR_INVALID_ARG, ATTN_ERR_UNSUPPORTED,
 * ATTN_ERR_WORKSPACE, ATTN_ERR_HIP.  Work is enqueued on `stream`.
 */
int attn_spec_accept(const int32_t* draft_tokens, const float* draft_probs,
                     const float* target_probs, const float* u_accept,
                     const float* u_sample, int32_t* n_accepted, int32_t* out_tokens,
                     int B, int k, int V, void* workspace, size_t workspace_bytes,
                     void* stream);

/* Static, human-readable name of an ATTN_* return code. */
const char* attn_strerror(int code);

#ifdef __cplusplus
}
#endif

#endif /* EXACT_ATTN_H */
