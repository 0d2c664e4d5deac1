// Internal definitions shared by the kernels and the host layer of libssverify.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "ss_verify.h"

namespace ssv {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// ---------------------------------------------------------------------------
// Integer rules shared by host and device (the host exports them for tests).
// ---------------------------------------------------------------------------

// Token range of slot s of a chunk call (SpecStream section 4.2: contiguous
// chunks along token positions; cps consecutive chunks per slot).
__host__ __device__ inline void slot_tokens(int32_t len, int32_t chunk_len, int32_t chunk_begin, int32_t n_chunks,
                                            int32_t cps, int32_t s, int64_t* t0, int64_t* t1) {
    const int64_t c0 = (int64_t)chunk_begin + (int64_t)s * cps;
    int64_t c1 = c0 + cps;
    const int64_t c_end = (int64_t)chunk_begin + n_chunks;
    if (c1 > c_end) c1 = c_end;
    int64_t a = c0 * chunk_len, b = c1 * chunk_len;
    if (a > len) a = len;
    if (b > len) b = len;
    if (b < a) b = a;
    *t0 = a;
    *t1 = b;
}

// Balanced split of the resident history (ss_verify_history). Eq. (9) of
// SpecStream section 4.2 makes the merged result independent of where the
// history is cut, so the cuts are placed for an even load: the streams
// (request b, KV head g) are laid end to end on one line, b-major, each
// padded to a multiple of kPlanAlign tokens and followed by a gap of
// plan_charge positions that stands for the cost of starting a piece, and
// work-group w of n_wg takes the line positions [w*L, (w+1)*L). L is the
// larger of total/n_wg (total counting the gaps) and pad_max/(n_slots-1),
// rounded up to kPlanAlign, so that no stream is cut into more than n_slots
// pieces. Piece k of a stream whose tokens sit at line positions [o, o+pad)
// is their part inside work-group floor(o/L)+k's range; it goes to slot k;
// the slots after a stream's last piece hold empty states. A stream of
// length 0 has no pieces: the work-group whose range holds its position o
// owns its empty slots (and the candidate region when it is folded in). The
// kernels leave empty slots to a fill before the launch; fill_end records
// them for the host.
constexpr int kPlanAlign = 128;
// Line positions charged per stream: a work-group pays about 6 us per piece
// (the walk step, Q and the first loads, the merge across waves and the slot
// write, the pipeline drained), the time it streams about 370 tokens in, so
// ranges that hold more stream starts get fewer tokens. Measured on MI355X,
// rounds of 8K-16K-token ragged histories run 6-8% faster with any charge
// from 256 to 512; 512 leaves the 64K-token rounds as they were.
constexpr int kPlanCharge = 512;

__host__ __device__ inline int32_t clamp_len(int32_t len, int32_t max_len) {
    return len < 0 ? 0 : (len > max_len ? max_len : len);
}

__host__ __device__ inline int64_t plan_pad(int32_t len, int32_t align = kPlanAlign) {
    return ((int64_t)len + align - 1) / align * align;
}

// The gap after each stream on the line, a multiple of align so that every
// stream starts at an aligned position.
__host__ __device__ inline int64_t plan_charge(int32_t align = kPlanAlign) {
    return ((int64_t)kPlanCharge + align - 1) / align * align;
}

// Line positions of one stream: its padded tokens and the gap after them.
__host__ __device__ inline int64_t plan_span(int32_t len, int32_t align = kPlanAlign) {
    return plan_pad(len, align) + plan_charge(align);
}

// Tokens per work-group; n_slots >= 2, n_wg >= 1.
// (align: a multiple of kPlanAlign; block statistics align the cut to their
// blocks so that no block is shared by two pieces.)
__host__ __device__ inline int64_t plan_piece_len(int64_t total, int64_t pad_max, int32_t n_wg, int32_t n_slots,
                                                  int32_t align = kPlanAlign) {
    const int64_t even = (total + n_wg - 1) / n_wg;
    const int64_t cap = (pad_max + n_slots - 2) / (n_slots - 1);
    int64_t len = even > cap ? even : cap;
    if (len < align) len = align;
    return (len + align - 1) / align * align;
}

// Last work-group with a non-empty range (0 when the line is empty).
__host__ __device__ inline int64_t plan_last_wg(int64_t total, int64_t piece_len) {
    return total > 0 ? (total - 1) / piece_len : 0;
}

// Where a work-group is in its walk over the line: request b, KV head g of
// that request, and the line position of the request's first stream.
struct PlanCursor {
    int32_t b;
    int32_t g;
    int64_t line;
};

// One piece: compute the state of tokens [t0, t1) of stream (b, g) into
// slot k (k = -1: nothing to compute), then store empty states in slots
// k+1 .. fill_end-1.
struct PlanPiece {
    int32_t b, g, k, fill_end;
    int64_t t0, t1;
};

// Next piece of work-group w after cursor c; false when w owns no more. The
// walk starts at the first request whose streams end after w*L, or that
// starts at or after it, with c = {that request, 0, its line position}.
template <class LenFn>
__host__ __device__ inline bool plan_next(const LenFn& len_of, int32_t batch, int32_t n_kv_heads, int64_t piece_len,
                                          int64_t total, int32_t n_slots, int64_t w, PlanCursor& c, PlanPiece& out,
                                          int32_t align = kPlanAlign) {
    const int64_t lo = w * piece_len, hi = lo + piece_len;
    const int64_t w_last = plan_last_wg(total, piece_len);
    if (w > w_last) return false;
    while (c.b < batch) {
        // streams only start later from here on: none reaches w's range
        if (c.line >= hi) return false;
        const int32_t len = len_of(c.b);
        const int64_t pad = plan_pad(len, align), span = pad + plan_charge(align);
        while (c.g < n_kv_heads) {
            const int64_t o = c.line + (int64_t)c.g * span;
            if (o >= hi) return false;
            const int32_t g = c.g++;
            if (pad == 0) {
                // no tokens: the range that holds o owns the stream
                if (o < lo) continue;
                out = PlanPiece{c.b, g, -1, n_slots, 0, 0};
                return true;
            }
            if (o + pad <= lo) continue;
            const int32_t k = (int32_t)(w - o / piece_len);
            const int32_t n_pieces = (int32_t)((o + pad - 1) / piece_len - o / piece_len + 1);
            int64_t t0 = lo - o, t1 = hi - o;
            if (t0 < 0) t0 = 0;
            if (t1 > pad) t1 = pad;
            if (t0 > len) t0 = len;
            if (t1 > len) t1 = len;
            out = PlanPiece{c.b, g, k, k == n_pieces - 1 ? n_slots : k + 1, t0, t1};
            return true;
        }
        c.line += (int64_t)n_kv_heads * span;
        ++c.b;
        c.g = 0;
    }
    return false;
}

// Ancestor visibility bits of a candidate tree (node i sees itself and its
// ancestors). Parent pointers that do not point strictly backwards are read
// as roots, so the walk is always in bounds.
__host__ __device__ inline uint64_t tree_bits_step(const uint64_t* done, int32_t i, int32_t parent) {
    uint64_t bits = (uint64_t)1 << i;
    if (parent >= 0 && parent < i) bits |= done[parent];
    return bits;
}

__host__ __device__ inline uint64_t chain_bits(int32_t i) {
    return i >= 63 ? ~(uint64_t)0 : (((uint64_t)1 << (i + 1)) - 1);
}

// The same tree bits for node `lane` of one wave (n <= 64 nodes, all lanes
// active), by pointer jumping instead of a walk in node order: after round k
// a lane holds its own bit and those of its ancestors less than 2^k links
// up, and points at the ancestor 2^k links up (or at none), so six rounds
// reach the root of any tree of 64 nodes. The parents are read with one
// coalesced load; lanes >= n return bits of no meaning.
__device__ inline uint64_t wave_tree_bits(const int32_t* parents, int32_t n, int32_t lane) {
    int32_t up = -1;
    if (lane < n) {
        up = parents[lane];
        if (up < 0 || up >= lane) up = -1;
    }
    uint64_t bits = (uint64_t)1 << lane;
#pragma unroll
    for (int k = 0; k < 6; ++k) {
        const int src = up < 0 ? lane : up;
        const uint32_t lo = __shfl((uint32_t)bits, src), hi = __shfl((uint32_t)(bits >> 32), src);
        const int32_t up2 = __shfl(up, src);
        if (up >= 0) {
            bits |= ((uint64_t)hi << 32) | lo;
            up = up2;
        }
    }
    return bits;
}

// Reductions over the four 16-lane groups of a wave (lanes l, l^16, l^32,
// l^48), every lane receiving the result, with the gfx950 lane-swap
// instructions (plain VALU work) instead of shuffles routed through the LDS
// crossbar. The sums associate as (x0 + x16) + (x32 + x48) in every lane.
__device__ __forceinline__ float group4_max(float x) {
    const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
    const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

__device__ __forceinline__ float group4_sum(float x) {
    const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
    const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// ---------------------------------------------------------------------------
// Kernel parameter blocks (passed by value).
// ---------------------------------------------------------------------------

struct ChunkParams {
    const void* q;
    const void* k;
    const void* v;
    int64_t stride_b, stride_h, stride_t;
    const int64_t* req_offset;
    const int32_t* req_len;
    int32_t max_len;
    int32_t batch, n_q_heads, n_kv_heads, group, n_queries, rows;
    float scale;
    int32_t chunk_len, chunk_begin, n_chunks, cps, n_items;
    float* acc;
    float* m;
    float* l;
    int32_t slot_begin;
    int32_t row_blocks;  // VALU kernels: rows are split into blocks of kValuRows
    int32_t plan_slots;  // balanced history split: slots per stream (>= 2)
    // Tokens of each request that lie before the view's first row (a staging
    // chunk of a longer history): the chunk kernels see request b as
    // clamp(req_len[b] - len_offset, 0, max_len) tokens long.
    int64_t len_offset;
    // Gathered chunks: slot s of (request b, KV head g) holds chunk
    // chunk_idx[(b * n_kv_heads + g) * n_sel + s] (< 0: an empty slot);
    // NULL: the contiguous chunk range of slot_tokens.
    const int32_t* chunk_idx;
    int32_t n_sel;
    // Candidate region folded into each stream's first piece (narrow MFMA
    // kernels, ss_verify_history only): with_cand != 0.
    int32_t with_cand;
    const void* ck;
    const void* cv;
    int64_t c_stride_b, c_stride_h, c_stride_t;
    const int64_t* c_req_offset;
    const int32_t* parents;
    uint64_t* mask_out;
    // Block statistics (history kernels of the narrow MFMA engine): per wave
    // quarter w, row r of KV head g (r = i * group + h % group) and block j
    // of stats_block tokens, the state (m, l) of the keys of block j that
    // wave w attended; stats[(((((w * B + b) * Hkv + g) * stats_blocks + j)
    // * rows + r) * 2 + {0: m, 1: l}]. NULL: none.
    float* stats;
    int32_t stats_block, stats_blocks;
    int32_t plan_align;  // balanced cut: stream padding and piece alignment
    // Tokens of every request's whole history when req_len is NULL (the view
    // may show only a part of it, as a staging chunk does).
    int64_t full_len;
    // Whole-round calls with one slot per stream (MFMA chunk kernels):
    // fin_o [B][n_queries][Hq][d] and fin_lse [B][n_queries][Hq] receive the
    // finished rows instead of the slot states. NULL: write the slots.
    float* fin_o;
    float* fin_lse;
};

struct CandParams {
    const void* q;
    const void* k;
    const void* v;
    int64_t stride_b, stride_h, stride_t;
    const int64_t* req_offset;
    int32_t batch, n_q_heads, n_kv_heads, group, n_queries, rows;
    float scale;
    const int32_t* parents;
    uint64_t* mask_out;
    float* acc;
    float* m;
    float* l;
    int32_t slot;
    int32_t row_blocks;
};

struct MergeParams {
    const float* acc;
    const float* m;
    const float* l;
    int32_t n_slots;
    const int32_t* slots_per_req;
    int32_t batch, n_queries, n_q_heads, head_dim;
    float* o;
    float* lse;
};

// Length of request b as the chunk kernels see it (see len_offset).
__host__ __device__ inline int32_t chunk_view_len(const ChunkParams& p, int32_t b) {
    const int64_t n = (p.req_len ? (int64_t)p.req_len[b] : (int64_t)p.max_len) - p.len_offset;
    return (int32_t)(n < 0 ? 0 : (n > p.max_len ? p.max_len : n));
}

// Softmax weights enter the P V products as bf16. Rounding a weight moves it
// by up to 2^-8 relative, so a row that a few keys dominate moves by up to
// that fraction of the spread of their values; over many keys the rounding
// errors average out (N(0,1) data, 128 features: largest error about 4e-3 at
// 2-8 keys, 1.3e-3 at 128, 3.3e-4 at 2048) unless the scores are peaked. The
// wide-row kernel, whose matrix work is the bound, carries each weight's
// rounding remainder as a second bf16 operand for requests with fewer
// history keys than this; for longer ones it checks each piece afterwards
// and attends it again with the remainders where a few keys dominate a row.
constexpr int64_t kSplitBelow = 2048;

// History keys a row of request b meets over the whole call: the request's
// length, or for a gathered call the most keys its list can name.
__host__ __device__ inline int64_t row_history_keys(const ChunkParams& p, int32_t b) {
    if (p.chunk_idx) return (int64_t)p.n_sel * p.chunk_len;
    return p.req_len ? (int64_t)p.req_len[b] : p.full_len;
}

// Token range of slot s of (request b, KV head g) in a chunk call: the
// contiguous chunk range, or the listed chunk of a gathered call.
__host__ __device__ inline void piece_tokens(const ChunkParams& p, int32_t len, int32_t b, int32_t g, int32_t s,
                                             int64_t* t0, int64_t* t1) {
    if (!p.chunk_idx) {
        slot_tokens(len, p.chunk_len, p.chunk_begin, p.n_chunks, p.cps, s, t0, t1);
        return;
    }
    const int32_t c = p.chunk_idx[((int64_t)b * p.n_kv_heads + g) * p.n_sel + s];
    int64_t a = c < 0 ? (int64_t)len : (int64_t)c * p.chunk_len;
    int64_t e = a + p.chunk_len;
    if (a > len) a = len;
    if (e > len) e = len;
    *t0 = a;
    *t1 = e;
}

// ---------------------------------------------------------------------------
// The walk of a history launch over the balanced cut (device side).
// ---------------------------------------------------------------------------

// x of lane 0 in every lane, held in scalar registers.
__device__ __forceinline__ int64_t uniform64(int64_t x) {
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)(uint64_t)x);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)((uint64_t)x >> 32));
    return (int64_t)(((uint64_t)hi << 32) | lo);
}

// Where work-group w of a history launch of gridDim.x work-groups starts:
// the line's length and the piece length of the cut, and a cursor at the
// first request whose streams end after w*L, or that starts at or after it.
// Every wave computes the same (64-lane scans over the requests). False
// when w owns no range.
struct PlanStart {
    int64_t total, piece_len;
    PlanCursor cursor;
};

__device__ __forceinline__ bool plan_start(const ChunkParams& p, int64_t w, PlanStart& st) {
    const int lane = threadIdx.x & 63;
    auto len_of = [&](int32_t b) { return clamp_len(p.req_len ? p.req_len[b] : p.max_len, p.max_len); };

    // Line length and longest padded stream.
    int64_t total = 0, pad_max = 0;
    for (int b0 = 0; b0 < p.batch; b0 += 64) {
        const int b = b0 + lane;
        int64_t mx = b < p.batch ? plan_pad(len_of(b), p.plan_align) : 0;
        int64_t sum = b < p.batch ? mx + plan_charge(p.plan_align) : 0;
#pragma unroll
        for (int off = 32; off > 0; off >>= 1) {
            sum += __shfl_xor(sum, off);
            mx = max(mx, (int64_t)__shfl_xor(mx, off));
        }
        total += sum;
        pad_max = max(pad_max, mx);
    }
    total = uniform64(total * p.n_kv_heads);
    pad_max = uniform64(pad_max);
    const int64_t piece_len = plan_piece_len(total, pad_max, (int32_t)gridDim.x, p.plan_slots, p.plan_align);
    if (w > plan_last_wg(total, piece_len)) return false;
    const int64_t lo = w * piece_len;

    // First request whose streams end after lo, or that starts at or after it.
    int32_t b_first = p.batch;
    int64_t line = 0, carry = 0;
    for (int b0 = 0; b0 < p.batch; b0 += 64) {
        const int b = b0 + lane;
        const int64_t span = b < p.batch ? (int64_t)p.n_kv_heads * plan_span(len_of(b), p.plan_align) : 0;
        int64_t incl = span;
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
            const int64_t t = __shfl_up(incl, off);
            if (lane >= off) incl += t;
        }
        const int64_t start = carry + incl - span;
        const uint64_t hit = __ballot(b < p.batch && (start + span > lo || start >= lo));
        if (hit) {
            const int first = __ffsll((unsigned long long)hit) - 1;
            b_first = b0 + first;
            line = __shfl(start, first);
            break;
        }
        carry += __shfl(incl, 63);
    }
    st.total = total;
    st.piece_len = piece_len;
    st.cursor = PlanCursor{__builtin_amdgcn_readfirstlane(b_first), 0, uniform64(line)};
    return true;
}

// One step of the walk, kept out of line (inline: one definition across
// translation units; noinline: it runs on one lane between pieces, and
// inlined its 64-bit arithmetic would hold registers that the key loop
// needs).
__device__ inline __noinline__ int32_t plan_step(const int32_t* req_len, int32_t max_len, int32_t batch,
                                                 int32_t n_kv_heads, int64_t piece_len, int64_t total,
                                                 int32_t n_slots, int64_t w, PlanCursor* cursor, PlanPiece* out,
                                                 int32_t align) {
    auto len_of = [&](int32_t b) { return clamp_len(req_len ? req_len[b] : max_len, max_len); };
    PlanCursor c = *cursor;
    PlanPiece pc;
    const bool more = plan_next(len_of, batch, n_kv_heads, piece_len, total, n_slots, w, c, pc, align);
    *cursor = c;
    if (more) *out = pc;
    return more ? 1 : 0;
}

struct ImportanceParams {
    const float* m;
    const float* l;
    int32_t slot_begin;  // block j's state is in slot slot_begin + j
    int32_t batch, n_q_heads, n_kv_heads, n_queries, n_blocks;
    const float* lse;    // [B][q][Hq]
    float* importance;   // [B][Hkv][n_blocks]
};

struct SelectParams {
    const float* importance;  // [B][Hkv][n_blocks]
    int32_t batch, n_kv_heads, n_blocks, k, block_len, max_len;
    const int32_t* req_len;
    int32_t* out;             // [B][Hkv][k]
};

struct StatsImportanceParams {
    const float2* ml;   // block statistics, four wave quarters (ChunkParams::stats layout)
    int32_t batch, n_q_heads, n_kv_heads, n_queries, n_blocks, block_len;
    const int32_t* req_len;  // [B] or NULL: every request max_len long
    int32_t max_len;
    const float* lse;   // [B][q][Hq]
    float* importance;  // [B][Hkv][n_blocks]
};

// Wave quarters of the block statistics (the narrow MFMA kernels' waves).
constexpr int kStatsQuarters = 4;

// Blocks the selection kernel holds in LDS.
constexpr int kMaxSelectBlocks = 8192;
// Listed chunks merged into one slot of a gathered call (narrow MFMA kernel).
constexpr int kMaxGatherPerSlot = 64;

// Rows per work-group in the VALU kernels.
constexpr int kValuRows = 32;

// Launchers (defined in the kernel translation units).
hipError_t launch_chunk_valu(const ChunkParams& p, int dtype, int head_dim, hipStream_t stream);
hipError_t launch_chunk_mfma(const ChunkParams& p, int head_dim, hipStream_t stream);
hipError_t launch_chunk_mfma_f32(const ChunkParams& p, int head_dim, hipStream_t stream);
// Balanced split of the whole resident history over one work-group per CU
// (narrow MFMA kernel); p.plan_slots slots from p.slot_begin.
hipError_t launch_history_mfma(const ChunkParams& p, int head_dim, hipStream_t stream);
// The same cut on the fp32 MFMA kernel (no statistics, no candidate region).
hipError_t launch_history_mfma_f32(const ChunkParams& p, int head_dim, hipStream_t stream);
// Work-groups of one launch of the narrow MFMA kernels that covers the
// current device: one per CU.
hipError_t mfma_wave_work_groups(int rows, int* n);
hipError_t launch_chunk_mfma_wide(const ChunkParams& p, int head_dim, hipStream_t stream);
hipError_t launch_chunk_valu_small(const ChunkParams& p, int head_dim, hipStream_t stream);
hipError_t launch_candidates(const CandParams& p, int dtype, int head_dim, hipStream_t stream);
// Row blocks of the candidate kernel for `rows` rows per KV head.
int cand_row_blocks(int rows);
hipError_t launch_merge(const MergeParams& p, hipStream_t stream);
hipError_t launch_importance(const ImportanceParams& p, hipStream_t stream);
hipError_t launch_read_probe(const void* src, int64_t bytes, int32_t n_wg, uint32_t* sink, hipStream_t stream);
// bf16 elements one wave of the matrix-core probe loads (its operand window).
int64_t mfma_probe_wave_elems();
hipError_t launch_mfma_probe(const void* ops, int64_t n_ops, int32_t iters, int32_t n_wg, float* sink,
                             hipStream_t stream);
hipError_t launch_select(const SelectParams& p, hipStream_t stream);
// Empty states (m = -inf, l = 0, acc = 0) in rows [row_begin, row_begin +
// n_rows) of a state buffer (a row: head_dim accumulators, one m, one l).
hipError_t launch_state_fill(float* acc, float* m, float* l, int64_t row_begin, int64_t n_rows, int head_dim,
                             hipStream_t stream);
hipError_t launch_importance_stats(const StatsImportanceParams& p, hipStream_t stream);
// The 32-bit word `word` repeated over bytes (a multiple of 16) at dst.
hipError_t launch_word_fill(void* dst, int64_t bytes, uint32_t word, hipStream_t stream);

}  // namespace ssv
