/*
 * swa.h -- C ABI of libswa: sliding-window grouped-query attention on
 * AMD Instinct MI355X (gfx950).
 *
 * Pages cited (title; section):
 *   [SPYRE]  "Enable compact sliding-window attention for Gemma 3 and Gemma 4
 *            variants" (torch-spyre/hf-adapters pull request 496)
 *   [BONSAI] "Gemma3 Local Attention Cache" (jax-ml/bonsai issue 124)
 *   [SDPA]   "Add SDPA attention implementation" (ServiceNow/Fast-LLM pull
 *            request 512)
 *
 * Conventions shared by every entry point
 *   - All tensor arguments are DEVICE pointers on the current HIP device,
 *     row-major and contiguous, 16-byte aligned.  The caller allocates and
 *     owns every buffer (inputs, outputs, rings, ring_meta, workspace);
 *     the library allocates nothing and keeps no state between calls
 *     (swa_decode_step_noalloc alone uses a static device array of the
 *     library as its workspace).
 *   - dtype selects the element type of every floating-point tensor of the
 *     call: SWA_BF16 (bfloat16) or SWA_F32 (float32).  Arithmetic is fp32
 *     (matrix-core products accumulate in fp32; bf16 outputs are rounded to
 *     nearest even).
 *   - head dimension d must be a multiple of 64 from 64 to 512 (64, 128,
 *     192, 256, 320, 384, 448, 512; [SDPA] Test plan exercises the
 *     non-power-of-two size 320), else SWA_EUNSUPPORTED; hq must be a multiple
 *     of hkv; query head h reads key/value head h / (hq / hkv), the head
 *     map of repeat_interleave ([SDPA] Summary) without materialising it.
 *   - stream is a hipStream_t (NULL = the null stream).  Every call only
 *     enqueues work on it and returns; results are ready when the stream
 *     reaches that point.
 *   - Return value: SWA_OK, or a negative SWA_E* code.  Every argument check
 *     runs on the host before anything is enqueued, so an error return
 *     means nothing was launched.  Conditions only the device can see (a
 *     ring overflow, malformed device-resident lengths) are reported
 *     through the sticky flag SWA_META_ERR in ring_meta (see below); device
 *     code clamps every index it derives from device data to the buffer
 *     sizes given here, so malformed device data cannot cause an
 *     out-of-bounds access.
 *   - Calls that overlap on one stream are ordered; calls on different
 *     streams that share a buffer race, as for any HIP kernel.
 */
#ifndef SWA_H
#define SWA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SWA_API __attribute__((visibility("default")))

/* return codes */
#define SWA_OK 0
#define SWA_EINVAL (-1)       /* null pointer, bad size, misaligned pointer  */
#define SWA_EUNSUPPORTED (-2) /* d, dtype, mode or size outside the range    */
#define SWA_ELAUNCH (-3)      /* the HIP runtime refused a kernel launch     */
#define SWA_EWORKSPACE (-4)   /* workspace missing or smaller than required  */
#define SWA_ESCRATCH (-5)     /* sizes need more than the static scratch     */

/* element types */
#define SWA_BF16 0
#define SWA_F32 1

/* prefill masks */
#define SWA_CAUSAL 0
#define SWA_BLOCKWISE 1

/* ring_meta: int32 [batch, 4] per sequence, device memory */
#define SWA_META_POS 0    /* position of the newest cached token            */
#define SWA_META_ANCHOR 1 /* position held by logical ring row 0            */
#define SWA_META_START 2  /* physical ring row holding the anchor position  */
#define SWA_META_LO 3     /* left padding: positions < lo are never read    */
#define SWA_META_ERR ((int32_t)0x80000000) /* sticky error bit, in field LO */

/* largest ring supported by swa_cache_roll / swa_decode */
#define SWA_MAX_RING_ROWS 65536

/*
 * swa_prefill -- attention over packed variable-length documents.
 *
 * [SDPA] Summary: documents are packed back to back and delimited by
 * cu_seqlens; no query attends across a document boundary.  [SPYRE]
 * Summary: global layers are causal, sliding layers apply a window, and for
 * vision-language prompts the sliding mask is the window AND (causal OR
 * same image block).  For query token i and key token j of one document:
 *
 *   allowed(i, j) = (window <= 0 || i - j < window)
 *                   && (j <= i || (causal_mode == SWA_BLOCKWISE
 *                                  && ids[i] >= 0 && i, j in one image block))
 *
 *   out[i, h, :] = sum_j softmax_j(scale * <q[i,h], k[j,h/g]>) v[j, h/g, :]
 *
 * over the allowed j; a row with no allowed key is 0 (cannot happen: the
 * query itself is always allowed).  The window is one-sided: keys after the
 * query (only admitted inside an image block) never fail it.  An image
 * block is a maximal run of consecutive tokens of one document carrying the
 * same non-negative id; id -1 marks text.
 *
 *   q [total_tokens, hq, d], k and v [total_tokens, hkv, d], out like q.
 *   cu_seqlens int32 [num_docs + 1]: 0 = cu[0] <= cu[1] <= ... =
 *     cu[num_docs] = total_tokens (device).  Rows outside any document are
 *     treated as one-token documents.
 *   doc_or_block_ids int32 [total_tokens] (device): required for
 *     SWA_BLOCKWISE, ignored (may be NULL) for SWA_CAUSAL.
 *   window <= 0 means unlimited.  scale <= 0 means 1 / sqrt(d).
 * Masked key tiles are skipped: the work done is proportional to the
 * allowed pairs, not to total_tokens^2.
 */
SWA_API int swa_prefill(const void* q, const void* k, const void* v,
                        const int32_t* cu_seqlens,
                        const int32_t* doc_or_block_ids, int32_t window,
                        int32_t causal_mode, void* out, int32_t total_tokens,
                        int32_t num_docs, int32_t hq, int32_t hkv, int32_t d,
                        int32_t dtype, float scale, void* stream);

/*
 * swa_prefill_chunk -- prefill of one chunk of each document against the
 * document's cache so far.
 *
 * [SPYRE] Summary: chunked prefill is preserved: a prompt is prefilled in
 * chunks, each attending to the keys already cached plus its own.  For
 * document b the keys are its first len_k = cu_seqlens_k[b+1] -
 * cu_seqlens_k[b] positions and the queries are the LAST len_q =
 * cu_seqlens_q[b+1] - cu_seqlens_q[b] of them (0 <= len_q <= len_k), so
 * query row i of b sits at position len_k - len_q + i.  The mask is
 * swa_prefill's over positions 0 .. len_k - 1 of the document: a chunk's
 * rows equal those rows of swa_prefill over the document cut at len_k
 * (for SWA_CAUSAL, the rows of the whole document: later keys are never
 * allowed); an image block is cut at len_k too (its later tokens are not
 * cached yet).  swa_prefill is the case cu_seqlens_q == cu_seqlens_k.
 *
 *   q [total_q, hq, d], out like q; k and v [total_k, hkv, d];
 *   cu_seqlens_q, cu_seqlens_k int32 [num_docs + 1] (device), each
 *   non-decreasing from 0 to total_q / total_k, with len_q <= len_k per
 *   document (malformed offsets give unspecified values, never an
 *   out-of-bounds access);
 *   doc_or_block_ids int32 [total_k] (device), indexed by key row:
 *   required for SWA_BLOCKWISE, ignored for SWA_CAUSAL.
 *   window, causal_mode, scale, dtype, stream as for swa_prefill.
 */
SWA_API int swa_prefill_chunk(const void* q, const void* k, const void* v,
                              const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                              const int32_t* doc_or_block_ids, int32_t window,
                              int32_t causal_mode, void* out, int32_t total_q,
                              int32_t total_k, int32_t num_docs, int32_t hq, int32_t hkv,
                              int32_t d, int32_t dtype, float scale, void* stream);

/*
 * swa_prefill_backward -- gradients of swa_prefill (whole prompts).
 *
 * [SDPA] Benchmarks time the attention implementations forward and
 * backward in training at head sizes up to 512.  For the loss
 * sum(dout * out), where out = swa_prefill(q, k, v, ...) with the same
 * cu_seqlens, ids, window, mode and scale, this writes
 *   dq = d loss / d q  [total_tokens, hq, d]
 *   dk = d loss / d k  [total_tokens, hkv, d]   (summed over the hq / hkv
 *   dv = d loss / d v  [total_tokens, hkv, d]    query heads of each group)
 * in the element type of the inputs (bf16 rounded to nearest even).  out is
 * the forward's output (read only for delta_i = <dout_i, out_i>, the term
 * of the softmax's Jacobian); dout is the gradient arriving at out, laid
 * out like q.  lse: the rows' log-sum-exp as swa_prefill_lse stores it
 * (float32 [hq, total_tokens], 4-byte aligned), or NULL, in which case the
 * backward recomputes it with one more pass over the keys.  Every output element is written exactly once,
 * without atomics: the result is deterministic.
 *   d: a multiple of 64 from 64 to 512, as everywhere.
 *   workspace: device memory of at least
 *   swa_prefill_backward_workspace_bytes(total_tokens, hq) bytes, 16-byte
 *   aligned, owned by the caller, contents on entry ignored (per-row
 *   statistics and key intervals are written there); SWA_EWORKSPACE if
 *   missing or too small.
 *   Other arguments as for swa_prefill.  Calls sharing a workspace race
 *   unless ordered on one stream.
 */
SWA_API size_t swa_prefill_backward_workspace_bytes(int32_t total_tokens, int32_t hq);
SWA_API int swa_prefill_backward(const void* q, const void* k, const void* v, const void* out,
                                 const void* dout, const int32_t* cu_seqlens,
                                 const int32_t* doc_or_block_ids, int32_t window,
                                 int32_t causal_mode, const float* lse, void* dq, void* dk,
                                 void* dv, int32_t total_tokens, int32_t num_docs, int32_t hq,
                                 int32_t hkv, int32_t d, int32_t dtype, float scale,
                                 void* workspace, size_t workspace_bytes, void* stream);

/*
 * swa_prefill_lse -- swa_prefill that also stores each row's log-sum-exp,
 * the softmax statistic a backward pass needs: for query row i and head h,
 *   lse[h * total_tokens + i] = log(sum over allowed keys j of
 *                                   exp(scale * <q[i, h], k[j, h / g]>))
 * (natural log; -inf for a row with no allowed key).  lse: float32
 * [hq, total_tokens] (device, 4-byte aligned, caller-owned), required when
 * total_tokens > 0.  Every other argument and the output as for
 * swa_prefill; out is bitwise the same as swa_prefill's.  Passing this lse
 * to swa_prefill_backward spares the backward its pass over the keys that
 * recomputes it.
 */
SWA_API int swa_prefill_lse(const void* q, const void* k, const void* v,
                            const int32_t* cu_seqlens, const int32_t* doc_or_block_ids,
                            int32_t window, int32_t causal_mode, void* out, float* lse,
                            int32_t total_tokens, int32_t num_docs, int32_t hq, int32_t hkv,
                            int32_t d, int32_t dtype, float scale, void* stream);

/*
 * Bytes of workspace swa_decode needs for these sizes: split counters plus
 * fp32 split-K partials.  Depends only on the sizes, never on positions.
 */
SWA_API size_t swa_decode_workspace_bytes(int32_t batch, int32_t hq,
                                          int32_t hkv, int32_t d,
                                          int32_t ring_rows);

/*
 * swa_decode -- one query token per sequence against its compact ring.
 *
 * [SPYRE] Summary and Compilation behavior: decode reads a compact cache of
 * window + slack rows; decode position, buffer origin, unwritten rows, left
 * padding and window placement are tensor data, so one fixed-shape launch
 * serves every step.  [BONSAI] Steps 2-3: the cache is written with modulo
 * wrap-around and the mask follows the wrap.  Here the per-sequence state
 * is ring_meta[b] = {pos, anchor, start, lo}; physical row r holds position
 * a = anchor + ((r - start) mod ring_rows), and the query (the token at
 * position pos, already appended) reads exactly the rows with
 *   max(lo, pos - window + 1, 0) <= a <= pos.
 *
 *   q [batch, hq, d]; k_ring, v_ring [batch, hkv, ring_rows, d];
 *   ring_meta int32 [batch, 4] (device); out [batch, hq, d].
 *   window >= 1; ring_rows > window.  scale <= 0 means 1 / sqrt(d).
 *   workspace: device buffer of at least swa_decode_workspace_bytes(...)
 *   bytes, zero-filled before its first use.  Its leading words are split
 *   counters that every call returns to zero (in stream order), so later
 *   calls with the SAME sizes can reuse it as is; zero it again before a
 *   call with different sizes (the counter region moves with the sizes).
 *   Calls that overlap (different streams) must not share a workspace.
 * The launch grid depends only on (batch, hq, hkv, d, ring_rows).
 */
SWA_API int swa_decode(const void* q, const void* k_ring, const void* v_ring,
                       const int32_t* ring_meta, int32_t window, void* out,
                       int32_t batch, int32_t ring_rows, int32_t hq,
                       int32_t hkv, int32_t d, int32_t dtype, float scale,
                       void* workspace, size_t workspace_bytes, void* stream);

/*
 * swa_decode_step -- one whole decode step of every sequence in one launch:
 * the periodic roll (by metadata), the append of the new token and the
 * decode of its query.
 *
 * [SPYRE] Summary: the compact cache holds window + slack anchored rows,
 * receives each new token through the compact cache index and is rolled
 * every slack-count tokens; Compilation behavior: every position-dependent
 * value is tensor data, one fixed-shape launch per step.  [BONSAI] Steps
 * 2-3: writes wrap with a modulo and the mask follows the wrap.  For each
 * sequence b, from ring_meta[b] = {pos, anchor, start, lo}: p = pos + 1;
 * if p - anchor >= ring_rows, anchor += A and start = (start + A) mod
 * ring_rows with A = ring_rows - window (every position keeps its physical
 * row; the A oldest rows, all outside the window, become free: the same
 * state as swa_cache_roll reaches by copying, without moving bytes).  Then,
 * as swa_cache_append, row slot(p) of every kv head receives k_new[b] /
 * v_new[b] and pos = p (if the ring is still full, nothing is written, pos
 * is kept and SWA_META_ERR is set).  Then, as swa_decode, out[b] is the
 * attention of q[b] over the rows of positions max(lo, pos - window + 1, 0)
 * .. pos.  ring_meta is updated in place.
 *
 *   q [batch, hq, d]; k_new, v_new [batch, hkv, d];
 *   k_ring, v_ring [batch, hkv, ring_rows, d]; ring_meta int32 [batch, 4];
 *   out [batch, hq, d]; window >= 1, ring_rows > window; scale <= 0 means
 *   1 / sqrt(d); workspace as for swa_decode (same size, same reuse rule).
 * Rings advanced only by this call never need swa_cache_roll.  A ring rolled
 * by copy (swa_cache_roll) and one rolled here hold the same positions in
 * different physical rows; both are valid states for every entry point.
 */
SWA_API int swa_decode_step(const void* q, const void* k_new, const void* v_new,
                            void* k_ring, void* v_ring, int32_t* ring_meta, int32_t window,
                            void* out, int32_t batch, int32_t ring_rows, int32_t hq,
                            int32_t hkv, int32_t d, int32_t dtype, float scale,
                            void* workspace, size_t workspace_bytes, void* stream);

/*
 * swa_decode_step_noalloc -- swa_decode_step without a workspace argument,
 * for callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation).
 *
 * Same arguments (minus the workspace), same kernels and bitwise the same
 * results as swa_decode_step.  The split counters and fp32 partials live
 * in a static device array of SWA_NOALLOC_SCRATCH_BYTES inside the
 * library (one per GPU, held until the process ends); the call allocates
 * nothing and calls no allocating routine.  Sizes whose partials and
 * counters do not fit it (counters: batch * (kv heads x head blocks + 1)
 * words within 64 KiB; partials: about batch * hq * splits * (d + 2) * 4
 * bytes within the rest) return SWA_ESCRATCH before anything is launched.
 * The first call on a device resolves the array's address and clears its
 * counter region with a small kernel on `stream`; every call leaves the
 * counters at zero again.  All calls on one GPU share the array: calls
 * that overlap (different streams, or different host threads without
 * ordering) race and must not be issued.
 */
#define SWA_NOALLOC_SCRATCH_BYTES (8u << 20)
SWA_API int swa_decode_step_noalloc(const void* q, const void* k_new, const void* v_new,
                                    void* k_ring, void* v_ring, int32_t* ring_meta,
                                    int32_t window, void* out, int32_t batch, int32_t ring_rows,
                                    int32_t hq, int32_t hkv, int32_t d, int32_t dtype,
                                    float scale, void* stream);

/*
 * swa_cache_append -- write one new token per sequence into its ring.
 *
 * [SPYRE] Summary: decode writes go through the compact cache index;
 * [BONSAI] Step 2: the write position wraps with a modulo.  For each
 * sequence b: p = pos + 1; if p - anchor >= ring_rows the ring is full (a
 * roll is due): nothing is written, pos is kept and SWA_META_ERR is set in
 * ring_meta[b][SWA_META_LO].  Otherwise row slot(p) = (start + p - anchor)
 * mod ring_rows of every kv head receives k_new[b] / v_new[b] and pos = p.
 *
 *   k_new, v_new [batch, hkv, d]; k_ring, v_ring [batch, hkv, ring_rows, d];
 *   ring_meta int32 [batch, 4] (device, updated in place).
 * Bytes are copied unchanged.
 */
SWA_API int swa_cache_append(const void* k_new, const void* v_new,
                             void* k_ring, void* v_ring, int32_t* ring_meta,
                             int32_t batch, int32_t ring_rows, int32_t hkv,
                             int32_t d, int32_t dtype, void* stream);

/*
 * swa_cache_compact -- build each sequence's ring from its prompt cache.
 *
 * [SPYRE] Summary: the prompt-sized sliding cache is compacted at the first
 * decode into a bounded buffer of window + slack anchored rows, and short
 * prompts (shorter than the window) are handled.  For sequence b with
 * prompt length L (prompt_lens[b], or n_b = cu[b+1] - cu[b] when
 * prompt_lens is NULL) and left padding lo (left_pad[b], or 0):
 *   anchor = L - window (negative for short prompts), start = anchor mod
 *   ring_rows (in [0, ring_rows)), pos = L - 1;
 *   positions max(anchor, 0, L - n_b) .. L - 1 are copied from the packed
 *   source (sequence b's rows are the LAST n_b positions of its prompt:
 *   position p is source row cu[b] + p - (L - n_b)) to row slot(p); every
 *   other ring row is zero-filled.
 * The source must cover every position the first decode reads:
 * L - n_b <= max(lo, L - window + 1, 0); 1 <= L, 0 <= lo < L, n_b <= L.
 * A sequence violating this (device data) gets a zero ring and
 * SWA_META_ERR.
 *
 *   k_src, v_src [src_rows, hkv, d]; cu_seqlens int32 [batch + 1] (device);
 *   prompt_lens, left_pad int32 [batch] (device) or NULL;
 *   k_ring, v_ring [batch, hkv, ring_rows, d]; ring_meta int32 [batch, 4]
 *   (device, fully initialised here).  window >= 1, ring_rows > window.
 */
SWA_API int swa_cache_compact(const void* k_src, const void* v_src,
                              const int32_t* cu_seqlens,
                              const int32_t* prompt_lens,
                              const int32_t* left_pad, int32_t src_rows,
                              void* k_ring, void* v_ring, int32_t* ring_meta,
                              int32_t window, int32_t batch, int32_t ring_rows,
                              int32_t hkv, int32_t d, int32_t dtype,
                              void* stream);

/*
 * swa_cache_roll -- the periodic roll of full rings.
 *
 * [SPYRE] Summary: every slack-count (64 for a window + 64 ring) decode
 * tokens the compact caches are rolled with offset-aware device-to-device
 * copies.  For each sequence whose ring is full (pos + 1 - anchor >=
 * ring_rows): rows rotate left by A = ring_rows - window in place
 * (new row r = old row (r + A) mod ring_rows, for every kv head of K and
 * V) and anchor += A; start is unchanged, so the A freed rows are the next
 * A append targets.  Other sequences are untouched, so the call is safe at
 * any cadence; the decision is made on the device from ring_meta.
 *
 *   k_ring, v_ring [batch, hkv, ring_rows, d]; ring_meta int32 [batch, 4].
 */
SWA_API int swa_cache_roll(void* k_ring, void* v_ring, int32_t* ring_meta,
                           int32_t window, int32_t batch, int32_t ring_rows,
                           int32_t hkv, int32_t d, int32_t dtype, void* stream);

/* Static message for a return code. */
SWA_API const char* swa_strerror(int code);

#ifdef __cplusplus
}
#endif

#endif /* SWA_H */
