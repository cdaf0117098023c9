/*
 * lsh_attn.h -- C ABI of the MI355X (gfx950) LSH-attention forward pass.
 *
 * The method is the LSH attention of "Reformer: The Efficient Transformer"
 * (ICLR 2020) as the following pages describe it:
 *   - ultralytics.com glossary entry "Reformer", section "Atenção LSH":
 *     angular LSH (bucket = index of the largest entry of [xR, -xR] for a
 *     random matrix R of shape [rounds, d, n_buckets/2]), sort by bucket,
 *     equal blocks, attention within the own block and the previous block,
 *     several hash rounds in parallel;
 *   - twgreatdaily.com walkthrough, section "1 LSH Attention": shared
 *     queries and keys (Q = K), attention restricted to the query's bucket by
 *     masking a larger candidate set, sort by bucket then position, chunks
 *     of m sorted items that look back one chunk, multi-round hashing whose
 *     attended set is the union of the rounds' sets;
 *   - ai-scholar.tech summary, section "Transformerの問題点とは": scaled
 *     dot-product attention, softmax(q k^T / sqrt(d_k)) v.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Every pointer argument is caller-owned DEVICE memory (hipMalloc'd or a
 *    torch CUDA tensor), except `shape` and `stage`, which are host values,
 *    and the host outputs of lsh_attention_fwd_timed. The library
 *    never allocates or frees device memory and keeps no pointer after a call.
 *  - `stream` is a hipStream_t passed as void* (NULL = the default stream).
 *    Work is enqueued asynchronously on it; inputs must stay valid and
 *    unmodified until that work completes. Only lsh_attention_fwd_timed waits.
 *  - Tensors are dense row-major with these shapes (T = B*H):
 *      qk, v, out      [B, H, L, d]            dtype = shape->dtype
 *      R               [n_hashes, d, n_buckets/2]   float32, shared by all
 *                                              batches and heads; with
 *                                              LSH_PER_HEAD_R [H, n_hashes,
 *                                              d, n_buckets/2]
 *      buckets         [B, H, n_hashes, L]     int32, by original position
 *      perm            [B, H, n_hashes, L]     int32, perm[s] = position in
 *                                              sorted slot s of that round
 *      inv             [B, H, n_hashes, L]     int32, inv[i] = slot of position i
 *      lse_sorted      [B, H, n_hashes, L]     float32, by sorted slot
 *      o_sorted        [B, H, n_hashes, L, d]  float32, by sorted slot
 *  - Every tensor pointer and the workspace must be 16-byte aligned (the
 *    kernels move rows in 16-byte pieces); a misaligned pointer is rejected
 *    with LSH_ERR_ARG.
 *  - Inputs must be finite.
 *  - Return value: LSH_OK (0) or a negative LSH_ERR_* code. Argument checks
 *    run on the host before anything is enqueued; on any error nothing has
 *    been enqueued unless the code is LSH_ERR_HIP, and lsh_last_error()
 *    describes the failure. Output contents are unspecified after an error.
 *  - An empty problem (B, H or L equal to 0) is valid and enqueues nothing.
 *  - Calls on different streams that share a workspace race; give each
 *    concurrent call its own workspace.
 */
#ifndef LSH_ATTN_H
#define LSH_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum { LSH_F32 = 0, LSH_BF16 = 1 };

/* Bits of lsh_shape_t.flags. */
enum {
    /* The key side of every attention score uses the unit vector x_j / |x_j|
     * (walkthrough "1 LSH Attention": its stripped formula is where the
     * method normalises keys); queries keep their length and the hash is
     * unchanged. A zero vector gives a zero key. The backward differentiates
     * through the norm. */
    LSH_KEY_NORM = 1,
    /* R is [H, n_hashes, d, n_buckets/2]: head h hashes with its own
     * rotations R[h] in every batch, instead of one R shared by all heads (the
     * glossary's R has no head axis; this is the alternative of giving each
     * head independent random rotations). Only the hash reads R. */
    LSH_PER_HEAD_R = 2
};

enum {
    LSH_OK = 0,
    LSH_ERR_ARG = -1,         /* an argument breaks a constraint listed below   */
    LSH_ERR_WORKSPACE = -2,   /* workspace pointer NULL or smaller than needed  */
    LSH_ERR_HIP = -3          /* a HIP launch or runtime call failed            */
};

/* Problem description (host struct, read during the call only). Every
 * constraint below is checked on the host; a shape that breaks one is
 * rejected with LSH_ERR_ARG.
 *   B, H, L, d   batch, heads, sequence length, head dimension; B, H, L >= 0
 *                and d in {64, 128} (the head sizes the kernels are built for).
 *   n_buckets    even, 2 <= n_buckets <= 4096.
 *   n_hashes     hash rounds, 1 <= n_hashes <= 4096.
 *   chunk_len    m >= 1 with L % m == 0 (the pages cut the sorted sequence
 *                into equal chunks).
 *   causal       0 or 1: key position must not exceed the query position.
 *   dtype        LSH_F32 or LSH_BF16 for qk, v and out.
 *   flags        0, or LSH_KEY_NORM and/or LSH_PER_HEAD_R (other bits:
 *                LSH_ERR_ARG).
 * Also required: B*H*n_hashes*L < 2^31 (every per-slot array is indexed
 * with 32-bit integers; this replaces a bound on a packed 32-bit
 * (round, bucket, position) sort key, which the sort does not use). */
typedef struct lsh_shape {
    int32_t B, H, L, d;
    int32_t n_buckets, n_hashes, chunk_len, causal;
    int32_t dtype;
    int32_t flags;
} lsh_shape_t;

/* Bytes of workspace needed by `stage` ("hash", "sort", "fwd", "fwd_qk",
 * "fwd_x", "state" or "bwd") for `shape`. "state" is the size of the buffer
 * lsh_attention_fwd_train fills for lsh_attention_bwd. LSH_KEY_NORM adds
 * 4 bytes per token (B*H*L) to "fwd", "fwd_x" and "bwd".
 * Errors: an unknown or NULL stage, or an invalid shape, returns 0 and sets
 * lsh_last_error(); after a successful call lsh_last_error() is "" (a valid
 * empty problem may need 0 bytes, so test the message, not the size). */
size_t lsh_workspace_size(const char *stage, const lsh_shape_t *shape);

/* Step 1 -- angular LSH over n_hashes rounds (glossary "Atenção LSH";
 * walkthrough "1 LSH Attention" for one hash function per round).
 * buckets[b,h,r,i] = first index of the maximum of [x R_r, -x R_r] where
 * x = qk[b,h,i,:], evaluated as if in exact arithmetic: a fast pass on the
 * matrix cores bounds its own rounding error, and every token-round whose
 * decision that bound cannot certify is recomputed in double precision, so
 * the result matches an exact evaluation except where two entries differ by
 * less than about 1e-12 relative. Deterministic.
 *   qk       [B,H,L,d] shape->dtype      R   [n_hashes, d, n_buckets/2] f32
 *   buckets  [B,H,n_hashes,L] int32 (out)
 *   ws       device workspace of at least lsh_workspace_size("hash") bytes.
 *            After the work completes, the first int32 of ws holds the number
 *            of token-rounds that were re-decided in double precision. */
int lsh_hash(const void *qk, const float *R, const lsh_shape_t *shape, int32_t *buckets,
             void *ws, size_t ws_bytes, void *stream);

/* Step 2 -- stable sort of each (b,h,round) by (bucket, position)
 * (walkthrough "1 LSH Attention": sort by bucket, then by position inside the
 * bucket). Bit-exact and deterministic.
 *   buckets  [B,H,n_hashes,L] int32, values in [0, n_buckets)
 *   perm     [B,H,n_hashes,L] int32 (out)   inv [B,H,n_hashes,L] int32 (out)
 *   ws       at least lsh_workspace_size("sort") bytes. */
int lsh_sort(const int32_t *buckets, const lsh_shape_t *shape, int32_t *perm, int32_t *inv,
             void *ws, size_t ws_bytes, void *stream);

/* lsh_sort without a workspace argument, for callers that cannot allocate
 * device memory (code under HIP graph capture, serving loops, harnesses that
 * forbid allocation). Same kernels and result as lsh_sort; the sort's
 * per-tile counts live in a static device array of 16 MiB that the library
 * holds on each GPU it runs on until the process ends (its address is looked
 * up on the first call on a device). It calls no allocating routine.
 *   buckets, perm, inv   as for lsh_sort
 *   stream               must belong to the current device (else LSH_ERR_ARG)
 * Errors: LSH_ERR_WORKSPACE when lsh_workspace_size("sort") exceeds 16 MiB
 * (e.g. B*H*n_hashes * ceil(L/4096) * n_buckets * 4 bytes past it); the
 * other checks as for lsh_sort. Calls that overlap on one GPU (several
 * streams or host threads) share the array and race: serialise them. */
int lsh_sort_noalloc(const int32_t *buckets, const lsh_shape_t *shape, int32_t *perm,
                     int32_t *inv, void *stream);

/* Steps 3+4 -- gather into sorted order and chunked attention (walkthrough
 * "1 LSH Attention"; glossary "Atenção LSH"). For sorted slot s of a round,
 * with chunk c = s / m, the candidate keys are the slots of chunks c-1 and c
 * of the same round (chunk 0 has no look-back). Key position j is valid for
 * query position i when bucket(j) == bucket(i) and, if causal, j <= i. The
 * score is (x_i . x_j) / sqrt(d) (with LSH_KEY_NORM, also divided by |x_j|),
 * lowered by 1e5 when j == i, so a query attends to itself only when no
 * other key is valid. Softmax in float32.
 *   qk, v     [B,H,L,d] shape->dtype
 *   buckets   [B,H,n_hashes,L] int32     perm [B,H,n_hashes,L] int32
 *   o_sorted  [B,H,n_hashes,L,d] f32 (out)
 *   lse_sorted[B,H,n_hashes,L] f32 (out), natural-log partition function. */
int lsh_chunk_attend(const void *qk, const void *v, const int32_t *buckets, const int32_t *perm,
                     const lsh_shape_t *shape, float *o_sorted, float *lse_sorted, void *stream);

/* Steps 3+4 with separate queries and keys (an ablation). The walkthrough's
 * "1 LSH Attention" shows the bucket-sorted attention matrix before it sets
 * Q = K: queries and keys each hashed and sorted by bucket, so a bucket's
 * query and key counts need not match and a bucket may hold queries but no
 * keys. Here query slot s (chunk c = s / m of the queries' order perm_q)
 * sees the key slots of chunks c-1 and c of the keys' order perm_k; key
 * position j counts for query position i when buckets_k(j) == buckets_q(i)
 * and, if causal, j <= i; the score is (q_i . k_j) / sqrt(d) with no self
 * penalty. A query with no key that counts gets a zero row and lse -inf.
 *   q, k, v                [B,H,L,d] shape->dtype
 *   buckets_q, buckets_k   [B,H,n_hashes,L] int32 (lsh_hash of q and of k)
 *   perm_q, perm_k         [B,H,n_hashes,L] int32 (lsh_sort of each)
 *   o_sorted, lse_sorted   by query slot, as for lsh_chunk_attend
 * LSH_KEY_NORM is refused (LSH_ERR_ARG): it belongs to shared vectors. */
int lsh_chunk_attend_qk(const void *q, const void *k, const void *v, const int32_t *buckets_q,
                        const int32_t *buckets_k, const int32_t *perm_q, const int32_t *perm_k,
                        const lsh_shape_t *shape, float *o_sorted, float *lse_sorted,
                        void *stream);

/* Step 5 -- un-sort and combine the rounds (walkthrough "1 LSH Attention":
 * multi-round hashing attends to the union of the rounds' sets). For each
 * position i: l_r = lse_sorted[r, inv_r[i]], Z = logsumexp_r l_r,
 * out_i = sum_r exp(l_r - Z) * o_sorted[r, inv_r[i]].
 *   o_sorted [B,H,n_hashes,L,d] f32   lse_sorted [B,H,n_hashes,L] f32
 *   inv      [B,H,n_hashes,L] int32   out [B,H,L,d] shape->dtype (out)
 * A round whose lse is -inf (no key, separate queries and keys only) takes
 * weight 0; a position with no other round gets a zero row. */
int lsh_unsort_combine(const float *o_sorted, const float *lse_sorted, const int32_t *inv,
                       const lsh_shape_t *shape, void *out, void *stream);

/* Whole forward: steps 1-5 on `stream`, intermediates in `ws`
 * (at least lsh_workspace_size("fwd") bytes; the first int32 of ws is the
 * hash stage's re-decided count, as in lsh_hash). The launches depend on the
 * shape: with bf16 I/O, chunk 64 and one hash round the chunk pass writes
 * out itself (the combine's weight is 1) and no combine kernel runs; a
 * segment of at most 4096 positions is sorted by one kernel instead of
 * three, and one of two to four tiles (4096 < L <= 16384, n_buckets <=
 * 2048) by two; with n_buckets <= 64 the hash's full scans store their
 * buckets themselves and no finishing kernel runs. */
int lsh_attention_fwd(const void *qk, const void *v, const float *R, const lsh_shape_t *shape,
                      void *out, void *ws, size_t ws_bytes, void *stream);

/* Whole forward with separate queries and keys (the ablation of
 * lsh_chunk_attend_qk): q and k are hashed with the same R and sorted on
 * their own, then attended and combined through the queries' order. out
 * rows of queries that find no key in any round are zero.
 *   q, k, v [B,H,L,d] shape->dtype; R as for lsh_hash; out [B,H,L,d]
 *   ws      at least lsh_workspace_size("fwd_qk") bytes
 * LSH_KEY_NORM is refused (LSH_ERR_ARG). */
int lsh_attention_fwd_qk(const void *q, const void *k, const void *v, const float *R,
                         const lsh_shape_t *shape, void *out, void *ws, size_t ws_bytes,
                         void *stream);

/* Diagnostic twin of lsh_attention_fwd: the same launches, with a HIP event
 * recorded after each kernel. It waits for the stream, then writes each
 * kernel's duration in milliseconds to kernel_ms[k] and its static name to
 * kernel_names[k] (both host arrays of max_kernels entries; names may be
 * NULL) and the number of kernels to *n_kernels. */
int lsh_attention_fwd_timed(const void *qk, const void *v, const float *R,
                            const lsh_shape_t *shape, void *out, void *ws, size_t ws_bytes,
                            void *stream, float *kernel_ms, const char **kernel_names,
                            int32_t max_kernels, int32_t *n_kernels);

/* Input projections ahead of step 1 (glossary "Atenção LSH": queries and
 * keys come from one shared projection; ai-scholar.tech summary, section
 * "Reformerを用いた結果": model width 1024 split over 8 heads). Two bias-free
 * linear maps of the token vectors, each with H*d outputs; head h takes
 * outputs h*d .. h*d + d - 1:
 *   qk[b,h,l,e] = sum_k x[b,l,k] * w_qk[h*d + e, k]     (v likewise, w_v)
 *   x         [B, L, d_model]       shape->dtype
 *   w_qk, w_v [H*d, d_model]        shape->dtype (a linear layer's weight:
 *                                   row = output, column = input)
 *   qk, v     [B, H, L, d]          shape->dtype (out)
 * Accumulation in float32 (bf16: matrix cores), outputs rounded to nearest
 * even. d_model must be a positive multiple of 8 (else LSH_ERR_ARG). Only
 * B, H, L, d and dtype of `shape` are used, but the whole shape must be
 * valid. No workspace. */
int lsh_qkv_project(const void *x, const void *w_qk, const void *w_v, const lsh_shape_t *shape,
                    int32_t d_model, void *qk, void *v, void *stream);

/* lsh_qkv_project followed by lsh_attention_fwd, with qk and v kept in the
 * workspace (at least lsh_workspace_size("fwd_x") bytes; its first int32 is
 * the hash stage's re-decided count, as in lsh_hash).
 *   x [B, L, d_model], w_qk, w_v [H*d, d_model], R as for lsh_hash,
 *   out [B, H, L, d]. */
int lsh_attention_fwd_x(const void *x, const void *w_qk, const void *w_v, const float *R,
                        const lsh_shape_t *shape, int32_t d_model, void *out, void *ws,
                        size_t ws_bytes, void *stream);

/* Forward for training: lsh_attention_fwd, and the sort it used plus the
 * log of each position's total partition function are written to `state`
 * (device memory of at least lsh_workspace_size("state") bytes, owned by
 * the caller, read by lsh_attention_bwd; its layout is internal to the
 * library). `ws` is as for lsh_attention_fwd. */
int lsh_attention_fwd_train(const void *qk, const void *v, const float *R,
                            const lsh_shape_t *shape, void *out, void *state,
                            size_t state_bytes, void *ws, size_t ws_bytes, void *stream);

/* Backward of lsh_attention_fwd_train. The hash and the sort are piecewise
 * constant and carry no gradient; the attention of each position is one
 * softmax over every (round, key) hit of its rounds' windows (walkthrough
 * "1 LSH Attention": the union of the rounds' sets), so with P the weight of
 * a hit, D_i = dout_i . out_i and s = x_i . x_j / sqrt(d):
 *   dv_j += P dout_i,  dS = P (dout_i . v_j - D_i),
 *   dqk_i += dS x_j / sqrt(d),  dqk_j += dS x_i / sqrt(d)
 * (queries and keys are the same vectors, so both terms land in dqk).
 *   qk, v, out, dout [B,H,L,d] shape->dtype (out as returned by the training
 *                    forward, dout the gradient of the loss with respect to it)
 *   state            as filled by lsh_attention_fwd_train for these inputs
 *   dqk, dv          [B,H,L,d] shape->dtype (out)
 *   ws               at least lsh_workspace_size("bwd") bytes
 * Accumulation in float32; deterministic (no atomics). */
int lsh_attention_bwd(const void *qk, const void *v, const void *out, const void *dout,
                      const void *state, size_t state_bytes, const lsh_shape_t *shape, void *dqk,
                      void *dv, void *ws, size_t ws_bytes, void *stream);

/* Chunked feed-forward (walkthrough "3 分塊": positions are independent, so
 * the rows are processed a chunk at a time to bound the wide intermediate;
 * scholar "Reformerを用いた結果" for d_model 1024, d_ff 4096). For every row m:
 *     out[m] = relu(x[m] W1^T + b1) W2^T + b2
 * (the Transformer's position-wise feed-forward; the pages name neither the
 * activation nor the biases, so a NULL bias is zero).
 *   x, out   [rows, d_model] dtype             d_model, d_ff: multiples of 8
 *   w1       [d_ff, d_model] dtype (output-major, as a linear layer stores it)
 *   b1       [d_ff] dtype or NULL
 *   w2       [d_model, d_ff] dtype             b2 [d_model] dtype or NULL
 *   ws       lsh_ffn_workspace_size bytes: one chunk's intermediate,
 *            min(chunk_rows, rows) * d_ff elements of dtype, caller-owned;
 *            lsh_ffn_workspace_size returns 0 and sets lsh_last_error() for
 *            invalid sizes (rows = 0 validly needs 0 bytes)
 * The result does not depend on chunk_rows (rows are independent; bit-equal
 * across chunk sizes). bf16: matrix cores, fp32 accumulation, the
 * intermediate rounded to bf16 after bias and ReLU; fp32: fp32 throughout.
 * Errors: LSH_ERR_ARG for sizes, dtype, NULL or misaligned tensors;
 * LSH_ERR_WORKSPACE for a missing or small workspace. */
size_t lsh_ffn_workspace_size(int64_t rows, int32_t d_ff, int32_t chunk_rows, int32_t dtype);
int lsh_ffn_chunked(const void *x, const void *w1, const void *b1, const void *w2,
                    const void *b2, int64_t rows, int32_t d_model, int32_t d_ff,
                    int32_t chunk_rows, int32_t dtype, void *out, void *ws, size_t ws_bytes,
                    void *stream);

/* Message for the last error on the calling thread ("" if none). */
const char *lsh_last_error(void);

/* Test hook for the LSH_ERR_HIP path. After lsh_debug_fail_launch(n) with
 * n >= 1, the n-th launcher status checked by the forward entry points
 * (lsh_attention_fwd, _fwd_x, _fwd_train, _fwd_qk; counted from 1, on the
 * calling thread) is reported as a HIP launch failure: the call returns
 * LSH_ERR_HIP naming the step, as if the runtime had refused that launch.
 * The kernels themselves run normally and nothing on the device fails; the
 * outputs of that call are unspecified, as after any error. n = 0 turns the
 * hook off (it is off by default and after it has fired); n < 0 is
 * LSH_ERR_ARG. */
int lsh_debug_fail_launch(int32_t n);

#ifdef __cplusplus
}
#endif

#endif /* LSH_ATTN_H */
