/*
 * ss_verify.h -- C ABI of libssverify, multi-query verification attention for
 * long-context speculative decoding on AMD Instinct MI355X (gfx950).
 *
 * What the library computes (SpecStream, "Resource-Efficient Speculative
 * Decoding for Long-Context LLM Serving", section 4.2):
 *   All q queries of a verification round share one committed KV history.
 *   The history is consumed chunk by chunk; every chunk yields a partial
 *   online-softmax state (m, l, acc) per query and head (Eq. 7). States are
 *   merged onto a common maximum (Eq. 8) and the output is O = acc / l
 *   (Eq. 9), which equals one softmax over every visible key (Eq. 6). The
 *   GPU-resident candidate rows are attended under a causal or tree mask.
 *
 * Conventions (apply to every call):
 *   - Status: every call returns SS_OK (0) or a negative SS_ERR_* code; the
 *     message of the last failure on the calling thread is ss_last_error().
 *     Nothing throws across this boundary.
 *   - Validation is synchronous and complete before anything is enqueued,
 *     and every resource a call needs (events of the streaming pipeline) is
 *     created before its first enqueue: a call that returns SS_ERR_INVALID_ARG
 *     or SS_ERR_UNSUPPORTED has enqueued no work. SS_ERR_HIP means the HIP
 *     runtime refused an enqueue; a call that enqueues several operations
 *     (ss_verify_history, ss_verify_round, ss_stream_history, the tiering
 *     copies) may then have enqueued the ones before it, which the caller
 *     drains by synchronising its streams (a streaming ring is then reset, so
 *     the next ss_stream_history call must not pass SS_STREAM_CONTINUE).
 *   - Ownership: the caller owns every buffer. The library never allocates
 *     or frees a caller buffer, and allocates no device memory. Buffers must
 *     stay valid until the caller has synchronised the streams it passed.
 *   - Asynchrony: device work is enqueued on the stream(s) passed in (a
 *     hipStream_t handle given as ss_stream_t; NULL = the default stream).
 *     Faults inside kernels surface at the caller's next synchronisation.
 *   - Element types: SS_F32 (float) or SS_BF16 (bfloat16 bit patterns).
 *     Q, K and V share the problem's dtype. States, O and lse are float32.
 *   - Heads: G = n_q_heads / n_kv_heads; query head h reads KV head h / G
 *     (grouped-query attention, contiguous groups).
 *   - Rows: for one request and KV head the "rows" are the R = n_queries * G
 *     pairs (query i, head-in-group hh), row r = i * G + hh.
 *   - Scores are scale * <q, k>; lse is the natural-log softmax denominator
 *     over scaled scores, lse = m + ln(l).
 *   - Supported head_dim: 64 and 128.
 */
#ifndef SS_VERIFY_H
#define SS_VERIFY_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#if defined(__GNUC__)
#define SS_API __attribute__((visibility("default")))
#else
#define SS_API
#endif

#define SS_ABI_VERSION 18

/* status codes */
#define SS_OK 0
#define SS_ERR_INVALID_ARG (-1) /* null pointer, bad size, inconsistent shape   */
#define SS_ERR_UNSUPPORTED (-2) /* valid request this build does not implement */
#define SS_ERR_HIP (-3)         /* the HIP runtime reported an error           */

/* element types */
#define SS_F32 0
#define SS_BF16 1

/* ss_stream_history flags */
#define SS_STREAM_TIMINGS 1  /* record per-chunk events for ss_stream_timings     */
#define SS_STREAM_CONTINUE 2 /* continue the previous call's staging ring          */
/* Ordering checks of the pipeline (diagnostic; the result must not change): */
#define SS_STREAM_POISON 4   /* fill each staging buffer with NaN once it is free, */
                             /* just before its copy                             */
#define SS_STREAM_DELAY 8    /* hold the copy stream about 2 ms before each copy  */

/* chunk-kernel engines (ss_problem_t.engine) */
#define SS_ENGINE_AUTO 0 /* measured choice, see ss_verify_chunk                 */
#define SS_ENGINE_VALU 1 /* vector ALU only (keeps the matrix cores free)      */
#define SS_ENGINE_MFMA 2 /* matrix cores; bf16 (head_dim 64: up to 32 rows)   */

/* A hipStream_t handle (NULL = default stream). */
typedef void* ss_stream_t;

/* Shape of one verification round. */
typedef struct ss_problem {
    int32_t batch;      /* B requests of the round (a Cohort, section 4.2)    */
    int32_t n_q_heads;  /* Hq                                                 */
    int32_t n_kv_heads; /* Hkv, divides Hq                                    */
    int32_t head_dim;   /* d: 64 or 128                                       */
    int32_t n_queries;  /* q queries per request (k drafts + 1, or tree nodes)*/
    int32_t dtype;      /* SS_F32 or SS_BF16                                  */
    float scale;        /* score scale, normally 1/sqrt(d); must be > 0       */
    int32_t engine;     /* SS_ENGINE_*: which units run the chunk kernel       */
} ss_problem_t;

/*
 * A view of device-resident keys and values. Element (b, h, t, x) -- request
 * b, KV head h, token t, feature x -- sits at
 *     base + off_b + h * stride_h + t * stride_t + x
 * (in elements), where off_b = req_offset[b] if req_offset is not NULL and
 * b * stride_b otherwise. The feature axis is contiguous. K and V share the
 * strides. Request b holds len_b tokens: req_len[b] (device array) if not
 * NULL, else max_len. A len_b above max_len is read as max_len.
 * Alignment: k and v 16-byte aligned; strides and offsets multiples of
 * 16 bytes' worth of elements. Offsets and stride_b, stride_h are 64-bit
 * throughout; stride_t may be at most 2^24 elements (SS_ERR_UNSUPPORTED
 * above: keys inside a tile are addressed by 32-bit offsets).
 * Covers head-major [B][Hkv][N][d], token-major ragged [sum N_b][Hkv][d]
 * and staging-chunk layouts.
 */
typedef struct ss_kv_view {
    const void* k;
    const void* v;
    int64_t stride_b;
    int64_t stride_h;
    int64_t stride_t;
    const int64_t* req_offset; /* device [B] or NULL */
    const int32_t* req_len;    /* device [B] or NULL */
    int32_t max_len;           /* uniform length, or upper bound of req_len */
} ss_kv_view_t;

/*
 * Online-softmax state slots (Eq. 7-8), float32, caller-allocated:
 *     acc [n_slots][B][n_queries][Hq][d]
 *     m   [n_slots][B][n_queries][Hq]   running maximum of scaled scores
 *     l   [n_slots][B][n_queries][Hq]   sum of exp(score - m)
 * A slot that saw no key is empty: m = -inf, l = 0, acc = 0 (the initial
 * state of section 4.2).
 */
typedef struct ss_state {
    float* acc;
    float* m;
    float* l;
    int32_t n_slots;
} ss_state_t;

/*
 * Block statistics recorded by ss_verify_history as a by-product of full
 * verification: for every row and block j of block_len history tokens, the
 * online-softmax state (m, l) of the block's keys (in parts whose Eq. 8 fold
 * is the block's state). buf holds ss_block_stats_bytes(problem, n_blocks)
 * bytes (caller-owned, device; layout internal, read by
 * ss_block_importance_stats; needs no initialisation); blocks past n_blocks
 * are not recorded, nor blocks past a request's end.
 */
typedef struct ss_block_stats {
    void* buf;
    int32_t block_len; /* a positive multiple of 128 */
    int32_t n_blocks;
} ss_block_stats_t;

/* ABI version this library implements (SS_ABI_VERSION). */
SS_API int32_t ss_abi_version(void);

/* Message of the last failed call on this thread ("" if none). The pointer
 * stays valid until the next call on this thread. */
SS_API const char* ss_last_error(void);

/* Bytes of acc + m + l for n_slots state slots of this problem, or a
 * negative status if the problem is invalid. Host only. */
SS_API int64_t ss_state_bytes(const ss_problem_t* problem, int32_t n_slots);

/*
 * ss_verify_chunk -- partial states of history chunks (section 4.2: the
 * chunk scores S_j = Q K_j^T / sqrt(d_h) for the whole query group, then the
 * chunk-local state of Eq. 7; consecutive chunks merged by Eq. 8).
 *
 *   q          device [B][n_queries][Hq][d], problem dtype
 *   hist       committed history (every key visible to every query)
 *   chunk_len  C > 0; chunk j of request b covers tokens
 *              [j*C, min((j+1)*C, len_b))
 *   chunk_begin, n_chunks   the chunks [chunk_begin, chunk_begin+n_chunks)
 *              are processed (n_chunks == 0: nothing is enqueued)
 *   chunks_per_slot  cps >= 1: slot slot_begin + s receives the state over
 *              chunks [chunk_begin + s*cps, chunk_begin + (s+1)*cps) clipped
 *              to the range; a slot with no token of a request is written
 *              empty for that request
 *   out        slots [slot_begin, slot_begin + ceil(n_chunks/cps)) must lie
 *              in [0, out->n_slots); they are overwritten
 * Engines (problem->engine). SS_ENGINE_AUTO (the same as SS_ENGINE_MFMA)
 * runs every shape on the matrix cores: for bf16 one MFMA kernel for up to
 * 32 rows per KV head (R = n_queries * G, padded to a 16-row tile) and one
 * for more rows; for fp32 one MFMA kernel (one work-group per 32 rows beyond
 * 32); all for head_dim 128 and 64. On gfx950 the padded MFMA kernel stays
 * bound by HBM down to a single row, ahead of the VALU kernels.
 * SS_ENGINE_VALU forces the VALU kernels (a small-row kernel below 16 rows
 * of bf16 / head_dim 128).
 * Errors: SS_ERR_INVALID_ARG for null pointers, non-positive sizes, slots
 * out of range, bad alignment; SS_ERR_UNSUPPORTED for head_dim outside
 * {64, 128}; SS_ERR_HIP if the launch fails.
 */
SS_API int32_t ss_verify_chunk(const ss_problem_t* problem, const void* q, const ss_kv_view_t* hist,
                               int32_t chunk_len, int32_t chunk_begin, int32_t n_chunks,
                               int32_t chunks_per_slot, const ss_state_t* out, int32_t slot_begin,
                               ss_stream_t stream);

/*
 * ss_verify_history -- the state of every request's whole resident history
 * [0, len_b), cut where the load balances best (section 4.2: the history
 * serves the whole query group, and by Eq. 9 the merged result does not
 * depend on where it is cut), optionally together with the candidate region.
 *
 *   q, hist     as ss_verify_chunk; len_b = req_len[b] (or max_len),
 *               clamped to [0, max_len]
 *   cand        NULL, or the candidate keys/values as in
 *               ss_verify_candidates (cand->max_len == n_queries <= 64);
 *               then the call's slots hold history and candidates together
 *   parents, mask_out  as ss_verify_candidates (used only with cand)
 *   n_slots     slots per (request, KV head) the call may use, >= 1 (>= 2
 *               with cand on the fp32 and VALU engines); the call writes
 *               exactly slots [slot_begin, slot_begin + n_slots) of every
 *               row, the ones it does not need as empty states
 * With the narrow MFMA kernel (AUTO or MFMA engine, bf16, head_dim 128 or
 * 64, R <= 32), and for ragged lengths also with the fp32 MFMA kernel (fp32,
 * R <= 32), where "slots" below are the history's (n_slots, or n_slots - 1
 * after the candidate slot):
 *   - ragged lengths (hist->req_len given) and at least 2 slots: the streams
 *     (request, KV head) are laid end to end, each padded to a multiple of
 *     128 tokens, and cut into equal ranges, one per work-group of a single
 *     full wave of the device; a stream is cut into at most as many pieces
 *     as there are slots (the ranges grow when there are too few slots for
 *     an even cut);
 *   - uniform lengths (req_len NULL): every stream is cut into
 *     P = min(n_slots, max(1, W / (B * Hkv))) equal chunks, W the
 *     work-groups of one full wave, i.e. n_slots = W / (B * Hkv) gives one
 *     chunk per work-group (narrow kernel only).
 * Other engines, and ragged lengths with one slot, cut every request
 * into as many chunks as there are slots, of ceil(max_len / slots)
 * tokens. Chunks are rounded up to a multiple of 128 tokens and run as
 * ss_verify_chunk with chunks_per_slot 1; chunks past a request's end are
 * empty slots.
 * Candidates: the MFMA kernels (narrow and wide-row) attend them as masked
 * key tiles after the history, in the work-groups that hold a stream's
 * first piece (no extra launch, no extra slot); the fp32 and VALU engines
 * run ss_verify_candidates into slot_begin and cut the history into the
 * remaining n_slots - 1 slots.
 * stats: NULL, or record block statistics (narrow MFMA kernel only,
 *   SS_ERR_UNSUPPORTED otherwise): the cut is aligned to block_len (no block
 *   is split between two pieces) and every piece records the (m, l) of its
 *   blocks; which entries exist follows from the lengths alone, so
 *   ss_block_importance_stats takes the same lengths.
 * Errors: as ss_verify_chunk and ss_verify_candidates.
 */
SS_API int32_t ss_verify_history(const ss_problem_t* problem, const void* q, const ss_kv_view_t* hist,
                                 const ss_kv_view_t* cand, const int32_t* parents, uint64_t* mask_out,
                                 const ss_block_stats_t* stats, int32_t n_slots, const ss_state_t* out,
                                 int32_t slot_begin, ss_stream_t stream);

/*
 * ss_verify_candidates -- the state of the GPU-resident candidate region
 * (section 4.2: the GPU region attended under a mask by each query's
 * position), written to one slot.
 *
 *   q        device [B][n_queries][Hq][d]
 *   cand     candidate keys/values; row i of request b is candidate i.
 *            n_cand = n_queries rows per request (cand->req_len is ignored,
 *            cand->max_len must equal n_queries); n_queries <= 64
 *   parents  device int32 [B][n_queries], or NULL for the causal mask
 *            (query i sees candidates j <= i). With parents, query i sees
 *            the ancestors of node i and itself: bits are built as
 *            anc[i] = anc[parents[i]] | (1 << i). parents[i] must satisfy
 *            0 <= parents[i] < i, or be -1 for a root; any other value is
 *            read as -1.
 *   mask_out optional device uint64 [B][n_queries]: receives the visibility
 *            bits (bit j of word i set iff query i sees candidate j)
 *   out, slot  the slot written, 0 <= slot < out->n_slots
 * Errors: as ss_verify_chunk; n_queries > 64 is SS_ERR_UNSUPPORTED.
 */
SS_API int32_t ss_verify_candidates(const ss_problem_t* problem, const void* q, const ss_kv_view_t* cand,
                                    const int32_t* parents, uint64_t* mask_out, const ss_state_t* out,
                                    int32_t slot, ss_stream_t stream);

/*
 * ss_merge_states -- fold slots with Eq. 8 and finalise (O = acc / l,
 * lse = m + ln l; section 4.2 and Eq. 9).
 *
 *   in             slots [0, in->n_slots)
 *   slots_per_req  device int32 [B] or NULL: request b folds its first
 *                  min(slots_per_req[b], n_slots) slots (NULL = all)
 *   o              device float [B][n_queries][Hq][d]
 *   lse            device float [B][n_queries][Hq]
 * A row whose slots are all empty gets O = 0 and lse = -inf.
 */
SS_API int32_t ss_merge_states(const ss_problem_t* problem, const ss_state_t* in, const int32_t* slots_per_req,
                               float* o, float* lse, ss_stream_t stream);

/*
 * ss_verify_round -- one whole verification round on resident KV (section
 * 4.2: the committed history and the masked candidate region in partial
 * states, Eq. 7, folded by Eq. 8 into O = acc / l and lse, Eq. 9):
 * ss_verify_history with the candidate region into slots [0, n_slots) of
 * `work`, then ss_merge_states over those slots into o and lse. With one
 * slot on the MFMA engines the history launch writes o and lse itself
 * (the merge of a single state, with the merge's arithmetic) and no merge
 * launch follows; `work` is then not written.
 *
 *   q, hist, cand, parents, mask_out   as ss_verify_history (cand required)
 *   n_slots   slots per (request, KV head) for the history cut, or 0: the
 *             library's choice (one piece per work-group of one full launch
 *             where the lengths are known on the host; for ragged lengths
 *             on the narrow MFMA kernel 1 -- a work-group per stream -- when
 *             hist->max_len <= 4096 with at least one stream per compute
 *             unit or <= 2048 with three per four units, else 8 for the
 *             balanced cut, on the fp32 MFMA kernel 8 (beyond 32 rows
 *             about two work-groups per compute unit); +1 for the
 *             candidate slot on the fp32 and VALU engines),
 *             limited to work->n_slots
 *   work      caller-allocated state slots (workspace); slots [0, n_slots)
 *             are overwritten, their contents afterwards are not part of
 *             the result
 *   o, lse    as ss_merge_states
 * Errors: as ss_verify_history and ss_merge_states; SS_ERR_INVALID_ARG if
 * n_slots exceeds work->n_slots.
 */
SS_API int32_t ss_verify_round(const ss_problem_t* problem, const void* q, const ss_kv_view_t* hist,
                               const ss_kv_view_t* cand, const int32_t* parents, uint64_t* mask_out,
                               int32_t n_slots, const ss_state_t* work, float* o, float* lse, ss_stream_t stream);

/*
 * ss_verify_round_noalloc -- ss_verify_round for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc): no workspace argument, and the call
 * allocates nothing (no hipMalloc, hipFree or allocating library routine).
 * The state slots live in a static device array of 64 MiB that every GPU
 * the library runs on holds until the process ends; the slot count is the
 * one ss_verify_round picks with n_slots = 0, cut down to what fits in the
 * array. Every slot the call uses is written before it is read, so stale
 * contents of an earlier call never reach the result. All calls on one GPU
 * share that GPU's array: calls that overlap in time on one GPU (on
 * different streams, or from several threads without ordering) race and
 * give undefined results.
 *   Arguments as ss_verify_round, without n_slots and work.
 * Errors: as ss_verify_round; SS_ERR_UNSUPPORTED if not even one state slot
 * (two on the VALU engines) of B * n_queries * Hq * (head_dim + 2) floats
 * fits in the 64 MiB; SS_ERR_HIP if the array's device address cannot be
 * obtained (looked up once per GPU on the first call there).
 */
SS_API int32_t ss_verify_round_noalloc(const ss_problem_t* problem, const void* q, const ss_kv_view_t* hist,
                                       const ss_kv_view_t* cand, const int32_t* parents, uint64_t* mask_out,
                                       float* o, float* lse, ss_stream_t stream);

/*
 * ss_stream_history -- streamed verification over a history held in pinned
 * host memory (section 4.2, pipelined KV transfers: staging buffers, a
 * transfer stream and a compute stream; each chunk is attended as soon as it
 * has landed; adjacent chunks grouped into one transfer; the next layer's
 * history fetched while the current layer finishes).
 *
 *   host_kv      pinned host, chunk-major [n_chunks][2][B][Hkv][C][d]
 *                (K block then V block of each chunk)
 *   req_len      device int32 [B] or NULL: request b's history is its first
 *                req_len[b] tokens (chunk j then holds
 *                clamp(req_len[b] - j*C, 0, C) of them; the rest of the
 *                chunk is copied but not attended); NULL: every request
 *                holds n_chunks * C tokens
 *   chunks_per_copy  adjacent chunks moved by one copy (>= 1): a staging
 *                buffer holds that many chunks
 *   staging      device buffer of n_buf staging buffers (n_buf >= 1, each
 *                chunks_per_copy * 2*B*Hkv*C*d elements)
 *   out          chunk j's state goes to slot slot_begin + j
 *   copy_stream, compute_stream  must differ; the copies run on the first,
 *                the chunk kernels on the second
 *   flags        SS_STREAM_TIMINGS: record per-chunk events (ss_stream_timings).
 *                SS_STREAM_POISON, SS_STREAM_DELAY: diagnostics of the ordering
 *                below. POISON overwrites every staging buffer with NaN on the
 *                copy stream after its wait for the buffer's last reader and
 *                before its copy; DELAY makes the copy stream sleep on the
 *                host (a host function) about 2 ms before every copy. With
 *                correct ordering neither changes any result.
 *                SS_STREAM_CONTINUE: the staging ring (same staging pointer,
 *                n_buf and buffer size) continues from the previous call on
 *                this device: each copy waits only until the last kernel that
 *                read its buffer is done, not for the compute stream's earlier
 *                work, so it may run while the compute stream still finishes
 *                the previous layer (cross-layer prefetch). The caller must
 *                not touch the staging buffers between such calls.
 * Per copy group: the copy stream waits until the chunks that last used the
 * staging buffer have been attended, copies the group, marks it arrived; the
 * compute stream waits for that mark, runs ss_verify_chunk on each of its
 * chunks and marks the buffer free. Without SS_STREAM_CONTINUE the first
 * copy also waits for all work already enqueued on the compute stream. The
 * call returns without synchronising; candidates and merge may follow on
 * the compute stream. Calls on one device may overlap in time on different
 * stream pairs when each has its own staging buffers: they share the
 * device's event objects, but every wait a call enqueues refers to a mark
 * that call recorded (events are recorded and waited under a lock, and a
 * wait takes the event as it was recorded when the wait was enqueued).
 * SS_STREAM_CONTINUE continues the device's most recent call.
 * Errors: as ss_verify_chunk; SS_ERR_INVALID_ARG if the streams are equal,
 * on unknown flags, or on SS_STREAM_CONTINUE with a different ring.
 */
SS_API int32_t ss_stream_history(const ss_problem_t* problem, const void* q, const void* host_kv,
                                 const int32_t* req_len, int32_t chunk_len, int32_t n_chunks,
                                 int32_t chunks_per_copy, void* staging, int32_t n_buf, const ss_state_t* out,
                                 int32_t slot_begin, ss_stream_t copy_stream, ss_stream_t compute_stream,
                                 int32_t flags);

/*
 * ss_stream_timings -- per-chunk event times of a timed ss_stream_history
 * call on this device: back = 0 the latest, 1 the one before, ... (the last
 * 64 are kept). Milliseconds from the compute stream's frontier when that
 * call was made (negative when a continued ring fetched the chunk before
 * the compute stream got there). Call after synchronising both streams.
 * n_chunks must equal that call's n_chunks; chunks of one copy group share
 * its copy times. Any output pointer may be NULL. The exposed wait of the
 * call is max(0, copy_end[0]) + sum over j >= 1 of
 * max(0, copy_end[j] - compute_end[j-1]).
 */
SS_API int32_t ss_stream_timings(int32_t back, int32_t n_chunks, float* copy_begin, float* copy_end,
                                 float* compute_begin, float* compute_end);

/*
 * Block statistics and block-sparse verification: the per-block softmax
 * statistics of a full verification round recycled as a per-head importance
 * signal (the SparseSpec-L abstract on the pages), and verification of the
 * history blocks that signal selects (the Dustin abstract). A block is a
 * chunk of block_len tokens; with one state slot per block (ss_verify_chunk,
 * chunks_per_slot 1) the mass that row r puts on block j is
 * l_j(r) * exp(m_j(r) - lse(r)).
 *
 * ss_verify_chunk_gathered: as ss_verify_chunk over listed chunks: the
 *   list of (request b, KV head g) is chunk_idx[(b * Hkv + g) * n_sel + e],
 *   e < n_sel (device int32 [B][Hkv][n_sel]; an entry < 0 or past the
 *   request's end stands for no keys), and slot slot_begin + s holds entries
 *   [s * chunks_per_slot, (s + 1) * chunks_per_slot) merged, so
 *   ceil(n_sel / chunks_per_slot) slots are written. The selection may differ
 *   per KV head. chunks_per_slot > 1 needs the narrow MFMA engine and at
 *   most 64 chunks per slot (SS_ERR_UNSUPPORTED otherwise), and chunk_len a
 *   multiple of 32.
 * ss_block_importance: importance[b][g][j] = max over the rows r of KV head
 *   g of l_j(r) * exp(m_j(r) - lse(r)), block j's state in slot
 *   slot_begin + j of `states`, lse [B][q][Hq] the round's final lse
 *   (ss_merge_states). Rows with l = 0 or lse = -inf contribute 0. Device
 *   arrays; float32.
 * ss_select_blocks: out[b][g][0..k) = the k blocks of largest importance
 *   among request b's ceil(len_b / block_len) blocks (len_b = req_len[b], or
 *   max_len when req_len is NULL; clamped to [0, max_len]), ties to the lower
 *   index, listed in increasing order, padded with -1. n_blocks <= 8192
 *   (SS_ERR_UNSUPPORTED above). Device arrays.
 */
SS_API int32_t ss_verify_chunk_gathered(const ss_problem_t* problem, const void* q, const ss_kv_view_t* hist,
                                        int32_t chunk_len, const int32_t* chunk_idx, int32_t n_sel,
                                        int32_t chunks_per_slot, const ss_state_t* out, int32_t slot_begin,
                                        ss_stream_t stream);
SS_API int32_t ss_block_importance(const ss_problem_t* problem, const ss_state_t* states, int32_t slot_begin,
                                   int32_t n_blocks, const float* lse, float* importance, ss_stream_t stream);
/* Bytes of a block-statistics buffer for n_blocks blocks, or a negative status. */
SS_API int64_t ss_block_stats_bytes(const ss_problem_t* problem, int32_t n_blocks);
/* As ss_block_importance, from block statistics recorded by ss_verify_history
 * (importance [B][Hkv][stats->n_blocks]); req_len (device int32 [B], or NULL:
 * every request max_len long) and max_len as in that call's history view.
 * Blocks past a request's end get importance 0. */
SS_API int32_t ss_block_importance_stats(const ss_problem_t* problem, const ss_block_stats_t* stats,
                                         const int32_t* req_len, int32_t max_len, const float* lse,
                                         float* importance, ss_stream_t stream);
SS_API int32_t ss_select_blocks(const ss_problem_t* problem, const float* importance, int32_t n_blocks,
                                const int32_t* req_len, int32_t max_len, int32_t block_len, int32_t k, int32_t* out,
                                ss_stream_t stream);

/*
 * Commit-aware KV tiering (SpecStream section 4.1). A request's target KV is
 * split at 0 <= H <= C <= L (Eq. 4): Sealed History [0, H) in a pinned host
 * store (chunk-major, as ss_stream_history reads it), Active Tail [H, C) and
 * Speculative Frontier [C, L) on the GPU. Committed KV migrates to the host
 * in blocks of g tokens once more than T committed tokens sit on the GPU;
 * rejected candidates are reclaimed on the GPU only, since [C', L) never
 * meets [0, H).
 *
 * ss_tier_migration_end: Eq. (5), E = max(H, g * floor(max(0, C - T) / g)).
 *   Host only. SS_ERR_INVALID_ARG unless 0 <= H <= C, g > 0, T >= 0.
 *
 * ss_tier_migrate: enqueue on `stream` the device-to-host copies of the
 *   committed rows [begin[b], end[b]) of every request from the GPU tail
 *   into the host store. tail: device view whose row 0 of request b is token
 *   tail_first[b] (req_offset must be NULL, rows contiguous: stride_t =
 *   head_dim); host_kv: pinned [n_chunks][2][B][Hkv][chunk_len][d]; token t
 *   lands in chunk t / chunk_len, row t % chunk_len. begin, end, tail_first
 *   are host arrays [B]. The caller moves H to end[b] only after the stream
 *   has passed the copies (an event), as section 4.1 requires.
 *   SS_ERR_INVALID_ARG if a range leaves the tail view or the store.
 *
 * ss_kv_copy_rows: enqueue on `stream` the device copies of rows
 *   [src_row[b], src_row[b] + n_rows[b]) of src into rows [dst_row[b], ...)
 *   of dst, K and V, every KV head (host arrays [B]; views with req_offset
 *   NULL and contiguous rows). Moves accepted candidates into the tail and
 *   compacts the tail after a migration (into a second buffer: source and
 *   destination must not overlap).
 */
SS_API int32_t ss_tier_migration_end(int64_t h, int64_t c, int64_t tail, int64_t gran, int64_t* e);
SS_API int32_t ss_tier_migrate(const ss_problem_t* problem, const ss_kv_view_t* tail, const int64_t* tail_first,
                               const int64_t* begin, const int64_t* end, void* host_kv, int32_t chunk_len,
                               int32_t n_chunks, ss_stream_t stream);
SS_API int32_t ss_kv_copy_rows(const ss_problem_t* problem, const ss_kv_view_t* src, const int64_t* src_row,
                               const ss_kv_view_t* dst, const int64_t* dst_row, const int64_t* n_rows,
                               ss_stream_t stream);

/*
 * ss_read_probe -- measurement reference, not part of the method: a kernel
 * that reads bytes (a multiple of 16) from the device buffer src with the
 * history kernels' load shape (16-byte loads, eight in flight per lane), each
 * of n_work_groups work-groups streaming one contiguous span. sink: device
 * uint32 [256], written only for one particular data value. The benchmark
 * reports the history kernels' bandwidth against this one.
 */
SS_API int32_t ss_read_probe(const void* src, int64_t bytes, int32_t n_work_groups, uint32_t* sink,
                             ss_stream_t stream);

/*
 * ss_mfma_probe -- measurement reference, not part of the method: the bf16
 * matrix-core rate the device sustains on given operand values. n_work_groups
 * work-groups of four waves; each wave loads 16 operand fragments (8 bf16 per
 * lane each: 8192 bf16, a window of operands chosen by the wave's index) once
 * and then runs iters x 8 independent v_mfma_f32_16x16x32_bf16 products on
 * them, nothing else in its loop. One launch performs
 * n_work_groups * 4 * iters * 8 * 16384 floating-point operations.
 * operands: device bf16, 16-byte aligned, n_operands >= 8192 (more gives the
 * waves different windows). sink: device float [256], written only for one
 * particular result value. The clock a launch holds depends on the operand
 * values (the chip's power draw does), so the benchmark fills operands like
 * the attention inputs (N(0,1) bf16) and reports the MFMA-bound kernel against
 * this rate as well as against the published peak.
 */
SS_API int32_t ss_mfma_probe(const void* operands, int64_t n_operands, int32_t iters, int32_t n_work_groups,
                             float* sink, ss_stream_t stream);

/*
 * Host-side helpers that expose the integer rules the kernels apply. They run
 * on the CPU, touch no device, and are the same code the kernels compile.
 *
 * ss_tree_mask_host: visibility bits of a candidate tree (n <= 64):
 *   out[i] = (1 << i) | out[parents[i]] when 0 <= parents[i] < i, else
 *   (1 << i). parents and out are host arrays of n entries.
 * ss_slot_tokens_host: the token range [*t0, *t1) that slot s of a chunk call
 *   covers for a request of len tokens.
 * ss_history_plan_host: the balanced cut of ss_verify_history for host
 *   lengths lens[batch] (clamped to [0, max_len]) over n_wg work-groups and
 *   n_slots >= 2 slots (streams laid end to end, each padded to 128 tokens
 *   and followed by a gap of 512 line positions that charges the start of a
 *   piece; each work-group an even share of that line). For every slot (b, g, k) of
 *   plan[batch][n_kv_heads][n_slots][4] it stores {work-group, t0, t1,
 *   writes}: the work-group that writes it, the token range it covers
 *   (t0 = t1 = -1 for a slot filled with the empty state) and how many
 *   times the cut writes it (1 in a correct cut; slots start at
 *   {-1, -1, -1, 0}). *piece_len receives the tokens per work-group.
 */
SS_API int32_t ss_tree_mask_host(const int32_t* parents, int32_t n, uint64_t* out);
SS_API int32_t ss_slot_tokens_host(int32_t len, int32_t chunk_len, int32_t chunk_begin, int32_t n_chunks,
                                   int32_t chunks_per_slot, int32_t s, int64_t* t0, int64_t* t1);
SS_API int32_t ss_history_plan_host(const int32_t* lens, int32_t batch, int32_t n_kv_heads, int32_t max_len,
                                    int32_t n_wg, int32_t n_slots, int64_t* plan, int64_t* piece_len);

#ifdef __cplusplus
}
#endif

#endif /* SS_VERIFY_H */
