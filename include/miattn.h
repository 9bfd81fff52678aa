/* libmiattn -- exact attention for one AMD Instinct MI355X (gfx950) GPU.
 *
 * C ABI only: plain pointers, ints and floats. Device pointers are HIP
 * device memory; `stream` is a hipStream_t passed as void* (NULL = the
 * default stream). Every call only enqueues work on `stream` and returns; no
 * call synchronises the host. Kernel faults surface at the caller's next
 * synchronisation, not as a return code.
 *
 * Operation (all entry points): exact attention
 *     O = softmax(scale * Q K^T  [+ causal mask]) V
 * as written out on the DistFlashAttn reviews page (review 1 summary) and
 * called exact, not approximate, on the FlashAttention abstract page; the
 * saved per-row statistic is the logsumexp (FlashAttention-2 reviews page,
 * reviewer 2, point 2).
 *
 * Tensor layouts (all contiguous, row-major):
 *   q, o, dout, dq : [B, N, H,   d]   element type `dtype`
 *   k, v, dk, dv   : [B, N, Hkv, d]   element type `dtype`
 *   lse            : [B, H, N]        float32, natural-log logsumexp of the
 *                                     scaled, masked scores of each row
 * Query head h reads K/V head h / (H / Hkv) (grouped-query attention; the
 * FlashAttention-2 reviews page, reviewer 1, MQA/GQA paragraph of the
 * backward section). Under `causal`, key j is visible to query i iff j <= i.
 *
 * Status codes: every entry point returns MIATTN_OK or an error code and
 * leaves a message for attn_last_error() (per host thread). Arguments are
 * validated before anything is enqueued; on error nothing is enqueued.
 *   MIATTN_EINVAL       null pointer, B/H/Hkv/N < 1, H % Hkv != 0, causal not
 *                       0/1, non-finite scale, pointer not 16-byte aligned,
 *                       nchunks not a positive divisor of N (chunked calls),
 *                       outputs aliasing inputs where forbidden.
 *   MIATTN_EUNSUPPORTED d not 64 or 128, unknown dtype, or a size that does
 *                       not fit 32-bit indexing: B*H*N >= 2^31 or
 *                       (N + 64)*H*d >= 2^31.
 *   MIATTN_ELAUNCH      the HIP runtime reported an error at launch.
 *   MIATTN_ENOMEM       a stream-ordered scratch allocation failed.
 *
 * Ownership: the caller allocates and owns every buffer passed in. The
 * library keeps no pointer to them after a call returns beyond the work
 * enqueued on `stream`. Scratch that a call needs comes from one device
 * buffer that the library keeps per (device, stream) and uses only in that
 * stream's order. A call that needs more takes the rest with hipMallocAsync
 * on `stream`, then replaces the buffer with one of its full size (the old
 * one freed with hipFreeAsync on `stream`): after the largest call, calls
 * allocate nothing. Calls made while `stream` is being captured into a graph
 * use stream-ordered allocations only, which the graph then owns. The buffer
 * lives until attn_release_scratch(stream); call that before destroying a
 * stream the library was used on.
 */
#ifndef MIATTN_H
#define MIATTN_H

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MIATTN_OK = 0,
  MIATTN_EINVAL = 1,
  MIATTN_EUNSUPPORTED = 2,
  MIATTN_ELAUNCH = 3,
  MIATTN_ENOMEM = 4
} miattn_status;

typedef enum {
  MIATTN_F32 = 0,   /* float32 in and out; float32 arithmetic */
  MIATTN_BF16 = 1   /* bfloat16 in and out; bf16 matrix products with float32 accumulation */
} miattn_dtype;

/* Forward pass: writes o and lse.
 * A tiled pass with online-softmax rescaling (FlashAttention abstract page:
 * tiling between HBM and on-chip memory; FlashAttention-2 reviews page,
 * reviewer 2, points 1-3: deferred rescaling, logsumexp saved, parallelism
 * over the sequence). Key tiles entirely above the diagonal are skipped
 * under `causal` (FlashAttention-2 reviews page, reviewer 4, section 3.1).
 * o and lse must not alias q, k or v. */
int attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
             int B, int H, int Hkv, int N, int d, int causal, float scale,
             void* stream, int dtype);

/* Forward pass of Nq new query rows against a key/value cache: decoding
 * (Nq = 1) and chunked prefill (Nq > 1) at inference time, which the
 * FlashAttention-2 reviews page names as a use of the method (reviewer 2,
 * strengths; reviewer 3, point 3). The cache's key range is cut into nsplit
 * chunks processed in parallel, and their partial results are combined with
 * the logsumexp merge of attn_merge (DistFlashAttn reviews page, reviews 1
 * and 4: partial results over key chunks are combined). Writes o and lse.
 *   q, o          : [B, Nq, H, d] bf16 (o is overwritten)
 *   k_cache, v_cache: [B, Nk, Hkv, d] bf16, Nk = cache capacity in rows
 *   k_lens        : device int32 [B], the number of valid cache rows of each
 *                   batch entry (values are clamped to [0, Nk]), or NULL for
 *                   Nk everywhere. Rows at or past k_lens[b] may hold
 *                   anything (stale or unwritten values, NaN included): the
 *                   kernels read them as zeros and they never enter the
 *                   result.
 *   lse           : [B, H, Nq] float32
 *   causal        : 0 = every query row sees all valid cache rows; 1 = query
 *                   row i of batch b sits at position k_lens[b] - Nq + i and
 *                   sees cache rows j <= that position (the new rows are the
 *                   last Nq positions of the sequence). A row that sees no
 *                   key gets o = 0 and lse = -inf.
 *   nsplit        : 1..1024, or 0 to let the library choose. With at most
 *                   32 query rows per K/V head group (Nq * H / Hkv <= 32,
 *                   decoding) it is the number of equal key ranges that the
 *                   valid keys of all batch entries, taken in order, are cut
 *                   into per K/V head, so that the work is the same for every
 *                   range whatever the length mix (default: four ranges per
 *                   compute unit over the K/V heads, each >= 256 keys).
 *                   Otherwise it is the number of equal chunks of every
 *                   entry's cache (default: about 2048 single-wave workgroups
 *                   in all, each chunk >= 256 keys, rounded up to a multiple
 *                   of 32 keys, which can lower the count). The result does
 *                   not depend on it beyond float32 rounding.
 *   dtype         : MIATTN_BF16 only (MIATTN_EUNSUPPORTED otherwise).
 * Scratch: float32 partials of (nsplit + B) [ranges] or nsplit * B [chunks]
 * slots of Nq * H * (d + 1) values.
 * o and lse must not alias q, k_cache or v_cache. */
int attn_fwd_kvcache(const void* q, const void* k_cache, const void* v_cache, const int* k_lens,
                     void* o, float* lse, int B, int H, int Hkv, int Nq, int Nk, int d, int causal,
                     float scale, int nsplit, void* stream, int dtype);

/* Causal sliding-window (local) attention, forward: the same operation as
 * attn_fwd with causal = 1 and a banded mask -- query row i sees key rows j
 * with i - window < j <= i (window keys including its own). FlashAttention-2
 * reviews page, the authors' general response: the method with local
 * (sliding-window) attention trained Mistral-7B; BurstAttention rebuttal
 * page: sparse attention only changes the attention mask. Key tiles wholly
 * outside every row's window are skipped. window >= 1 (MIATTN_EINVAL
 * otherwise); window >= N gives plain causal attention. All other arguments,
 * layouts and errors as attn_fwd. */
int attn_fwd_window(const void* q, const void* k, const void* v, void* o, float* lse,
                    int B, int H, int Hkv, int N, int d, int window, float scale,
                    void* stream, int dtype);

/* Packed variable-length batch, forward: nseq sequences of different
 * lengths stored back to back (FlashAttention-2 reviews page, reviewer 2's
 * questions: batches whose tokens carry no explicit sequence dimension; here
 * the boundaries are given as offsets). Sequence s owns rows
 * [cu_seqlens[s], cu_seqlens[s + 1]) of q, k, v, o and attends only within
 * itself, with the causal mask (and, if window > 0, the sliding window of
 * attn_fwd_window) applied at positions relative to its first row.
 *   q, o      : [total, H, d];  k, v: [total, Hkv, d];  lse: [H, total]
 *   cu_seqlens: device int32 [nseq + 1], 0 = cu_seqlens[0] <= ... <=
 *               cu_seqlens[nseq] = total, each length <= max_len. The host
 *               cannot read them; a kernel clamps every offset to [0, total],
 *               so malformed offsets give wrong rows but no access outside
 *               the tensors.
 *   max_len   : the longest sequence (sizes the grid), 1 <= max_len <= total.
 *   window    : 0, or >= 1 with causal = 1.
 * Errors as attn_fwd, plus MIATTN_EINVAL for nseq outside [1, 65535],
 * max_len outside [1, total], or a null or misaligned cu_seqlens. */
int attn_fwd_varlen(const void* q, const void* k, const void* v, void* o, float* lse,
                    const int* cu_seqlens, int nseq, int max_len, int total, int H, int Hkv, int d,
                    int causal, int window, float scale, void* stream, int dtype);

/* Backward of attn_fwd_varlen: dq [total, H, d], dk, dv [total, Hkv, d]
 * (dtype, or float32 added into under accumulate = 1) from that forward's o
 * and lse. Scratch: float32 [H, total]. Arguments and errors as
 * attn_fwd_varlen and attn_bwd. */
int attn_bwd_varlen(const void* q, const void* k, const void* v, const void* o, const float* lse,
                    const int* cu_seqlens, int nseq, int max_len, int total, int H, int Hkv, int d,
                    int causal, int window, float scale, void* stream, const void* dout, void* dq,
                    void* dk, void* dv, int dtype, int accumulate);

/* Block-sparse attention, forward (FlashAttention abstract page: the
 * extension to block-sparse attention; FlashAttention-2 reviews page,
 * reviewer 3's question on sparse block masks): attn_fwd where only the
 * blocks a block mask keeps are computed. Exact attention under that mask;
 * an approximation of dense attention.
 *   block_mask: device uint8 [ceil(N / 256)][ceil(N / 128)], shared by every
 *               batch and head: entry (r, c) != 0 keeps query rows
 *               [256 r, 256 r + 256) x keys [128 c, 128 c + 128); applied on
 *               top of the causal mask when causal = 1. Read on the stream;
 *               the caller keeps it alive until the call's work completes.
 * A query row left with no key gets o = 0 and lse = -inf (the merge
 * identity). Other arguments, layouts and errors as attn_fwd, plus
 * MIATTN_EINVAL for a null block_mask or outputs overlapping it.
 * bf16 scratch: int32 tile lists of about (N / 256 + N / 128) * N / 64
 * entries (stream-ordered allocation). */
int attn_fwd_blocksparse(const void* q, const void* k, const void* v, void* o, float* lse,
                         const unsigned char* block_mask, int B, int H, int Hkv, int N, int d,
                         int causal, float scale, void* stream, int dtype);

/* Backward of attn_fwd_blocksparse from its o and lse, with the same
 * block_mask: dq, dk, dv as attn_bwd (rows with no key get zero
 * gradients). Arguments, scratch and errors as attn_bwd and
 * attn_fwd_blocksparse. */
int attn_bwd_blocksparse(const void* q, const void* k, const void* v, const void* o, const float* lse,
                         const unsigned char* block_mask, int B, int H, int Hkv, int N, int d,
                         int causal, float scale, void* stream, const void* dout, void* dq, void* dk,
                         void* dv, int dtype, int accumulate);

/* Backward pass: from q, k, v, the forward's o and lse, and dout = dL/dO,
 * produces dq, dk, dv without forming the N x N matrix. The forward is not
 * re-run: P is rebuilt tile by tile from the saved lse (DistFlashAttn
 * reviews page, review 1 point 3: the backward needs no recomputation of the
 * forward). dk and dv of a K/V head are summed over the query heads that
 * read it.
 *   accumulate = 0: dq, dk, dv have element type `dtype` and are overwritten.
 *   accumulate = 1: dq, dk, dv are float32 buffers and the gradients are
 *                   added to their contents.
 * Scratch: one float32 [B, H, N] vector (rowsum(dout * o)).
 * Outputs must not alias any input or each other. */
int attn_bwd(const void* q, const void* k, const void* v, const void* o, const float* lse,
             int B, int H, int Hkv, int N, int d, int causal, float scale,
             void* stream, const void* dout, void* dq, void* dk, void* dv,
             int dtype, int accumulate);

/* Backward of attn_fwd_window: dq, dk, dv of causal sliding-window attention
 * (query row i sees key rows j with i - window < j <= i), from that forward's
 * o and lse. window >= 1; all other arguments, layouts, scratch and errors as
 * attn_bwd. */
int attn_bwd_window(const void* q, const void* k, const void* v, const void* o, const float* lse,
                    int B, int H, int Hkv, int N, int d, int window, float scale,
                    void* stream, const void* dout, void* dq, void* dk, void* dv,
                    int dtype, int accumulate);

/* attn_bwd for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc): the
 * same arguments, layouts, results and errors as attn_bwd, but the one
 * scratch buffer of the backward, the float32 [B, H, N] rowsum vector
 * D = rowsum(dout * o), lives in a fixed device array of 4194304 floats
 * (16 MiB) that the library holds on every device it runs on until the
 * process ends. The call allocates and frees nothing. Its address is looked
 * up once per device, at the first call with that device current.
 * Errors: MIATTN_EINVAL if B * H * N exceeds 4194304 (the message gives both
 * numbers), before anything is enqueued; MIATTN_ELAUNCH if the array's
 * address cannot be obtained. Every call on one device shares that device's
 * array, and D is written in full by each call before it is read, so
 * consecutive calls need no clearing; calls that overlap in time on one
 * device (concurrent streams, several host threads) race on it and must be
 * ordered by the caller. */
int attn_bwd_noalloc(const void* q, const void* k, const void* v, const void* o, const float* lse,
                     int B, int H, int Hkv, int N, int d, int causal, float scale,
                     void* stream, const void* dout, void* dq, void* dk, void* dv,
                     int dtype, int accumulate);

/* attn_bwd with per-kernel timing marks, for measurement tools: the same
 * arguments, results and errors as attn_bwd, and additionally
 *   marks[0] is recorded on `stream` after the backward's first kernel,
 *   marks[1] after its second,
 * where marks[0], marks[1] are hipEvent_t handles (passed as void*) that the
 * caller created and owns. marks == NULL records nothing. For dtype
 * MIATTN_BF16 the first kernel is the dQ kernel (which also forms the
 * rowsum D = rowsum(dout * o) of its rows) and the second the dK/dV kernel:
 * the intervals between an event the caller records before the call,
 * marks[0] and marks[1] are their durations, and an event recorded after the
 * call adds an empty interval. For MIATTN_F32 the first kernel is the rowsum
 * kernel and the second the float32 backward block.
 * MIATTN_ELAUNCH also covers a failed hipEventRecord. */
int attn_bwd_timed(const void* q, const void* k, const void* v, const void* o, const float* lse,
                   int B, int H, int Hkv, int N, int d, int causal, float scale,
                   void* stream, const void* dout, void* dq, void* dk, void* dv,
                   int dtype, int accumulate, void* const* marks);

/* Merge of two partial results of the same query rows over disjoint key
 * sets a and b into the result over a u b (DistFlashAttn reviews page,
 * reviews 1 and 4: partial chunk results are combined; BurstAttention
 * rebuttal page: partial softmax results are combined across devices):
 *     lse = ln(e^lse_a + e^lse_b)  (computed with the max factored out)
 *     o   = e^(lse_a - lse) o_a + e^(lse_b - lse) o_b
 * A partial whose lse is -inf (an empty key set) contributes nothing,
 * whatever its o holds; rows where both lse are -inf give o = 0, lse = -inf.
 * o_a, o_b, o: [B, N, H, d] of `dtype`; lse_a, lse_b, lse: [B, H, N] float32.
 * In-place use is allowed: o may equal o_a or o_b, lse may equal lse_a or
 * lse_b (each element is read before it is written by the same thread).
 * Errors: MIATTN_EINVAL for an output that overlaps an input at any other
 * offset, overlaps an input of the other kind, or overlaps the other output;
 * the size, pointer and dtype errors of attn_fwd. */
int attn_merge(const void* o_a, const float* lse_a, const void* o_b, const float* lse_b,
               void* o, float* lse, int B, int H, int N, int d, int dtype, void* stream);

/* Forward pass of causal attention computed as nchunks x nchunks chunk
 * pairs: the sequence is cut into nchunks chunks of N / nchunks rows; pair
 * (i, j), j <= i, is attention of query chunk i over key chunk j (masked
 * only when i == j), and the partials of a query chunk are combined with the
 * merge above. Pairs are processed in balanced rounds: one round holds the
 * diagonal pairs and the pairs at chunk distance nchunks/2, and round t
 * (t = 1 .. nchunks/2 - 1) holds the pairs at distances t and nchunks - t,
 * so every round carries the same amount of work (the DistFlashAttn reviews
 * page, review 1 point 1 and review 3: redistributing causal work from later
 * to earlier workers). nchunks must be even (or 1) and divide N.
 * Same arguments and outputs as attn_fwd with causal = 1. For MIATTN_BF16 the
 * forward kernel of each pair merges its rows into the query chunk's running
 * float32 result as it stores them (the last pair writes o and lse); for
 * MIATTN_F32 each pair's float32 partial is merged by the merge kernel.
 * Scratch: the float32 running output and LSE, [B, N, H, d] and [B, H, N]
 * (MIATTN_F32: twice that, for the partials). */
int attn_fwd_chunked(const void* q, const void* k, const void* v, void* o, float* lse,
                     int B, int H, int Hkv, int N, int d, float scale,
                     void* stream, int dtype, int nchunks);

/* Backward pass over the same chunk pairs and rounds as attn_fwd_chunked:
 * every pair's gradients are taken with the final o and lse of its query
 * chunk and summed in float32 (MIATTN_BF16: the first pair of a chunk stores
 * its float32 sums, later pairs add to them and the last one adds and writes
 * the bf16 result; MIATTN_F32: zeroed accumulators, converted at the end).
 * Same arguments and outputs as attn_bwd with causal = 1 and accumulate = 0.
 * Scratch: float32 dq, dk, dv sums and the [B, H, N] rowsum vector. */
int attn_bwd_chunked(const void* q, const void* k, const void* v, const void* o, const float* lse,
                     int B, int H, int Hkv, int N, int d, float scale,
                     void* stream, const void* dout, void* dq, void* dk, void* dv,
                     int dtype, int nchunks);

/* The pair order used by the chunked entry points, for inspection (host
 * only, no GPU work). Writes up to `capacity` entries: pair p belongs to
 * round round_of[p] and is query chunk q_chunk[p] over key chunk k_chunk[p].
 * Returns the number of pairs, nchunks * (nchunks + 1) / 2, or -1 if
 * nchunks is not 1 or a positive even number or capacity is too small. */
int attn_chunk_schedule(int nchunks, int* round_of, int* q_chunk, int* k_chunk, int capacity);

/* Message of the last error on this host thread ("" after success). The
 * pointer stays valid until the next call on this thread. */
const char* attn_last_error(void);

/* Library version string. */
const char* attn_version(void);

/* Frees the scratch buffer kept for `stream` on the current device, in
 * stream order (hipFreeAsync on `stream`); the next call on the stream
 * allocates again. Nothing to free is not an error. Errors: MIATTN_ELAUNCH
 * if the HIP runtime reports one. */
int attn_release_scratch(void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MIATTN_H */
