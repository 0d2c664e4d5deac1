// C ABI of libssverify: argument validation, kernel dispatch and the
// streamed-history pipeline (SpecStream section 4.2, "pipelined KV transfers":
// staging buffers, a transfer stream and a compute stream, per-chunk events).

#include <math.h>
#include <time.h>
#include <stdarg.h>
#include <stdio.h>

#include <mutex>
#include <string>
#include <vector>

#include "ss_common.h"

using namespace ssv;

namespace {

thread_local std::string g_err;

int32_t fail(int32_t code, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof(buf), fmt, ap);
    va_end(ap);
    g_err = buf;
    return code;
}

int32_t ok() {
    g_err.clear();
    return SS_OK;
}

int64_t elem_size(const ss_problem_t* p) { return p->dtype == SS_F32 ? 4 : 2; }

bool aligned16(const void* ptr) { return (reinterpret_cast<uintptr_t>(ptr) & 15u) == 0; }

int32_t check_problem(const ss_problem_t* p) {
    if (!p) return fail(SS_ERR_INVALID_ARG, "problem is NULL");
    if (p->batch <= 0 || p->n_q_heads <= 0 || p->n_kv_heads <= 0 || p->n_queries <= 0 || p->head_dim <= 0)
        return fail(SS_ERR_INVALID_ARG, "batch, heads, head_dim and n_queries must be positive");
    if (p->n_q_heads % p->n_kv_heads != 0)
        return fail(SS_ERR_INVALID_ARG, "n_q_heads (%d) is not a multiple of n_kv_heads (%d)", p->n_q_heads,
                    p->n_kv_heads);
    if (p->dtype != SS_F32 && p->dtype != SS_BF16) return fail(SS_ERR_INVALID_ARG, "unknown dtype %d", p->dtype);
    if (!isfinite(p->scale) || !(p->scale > 0.f)) return fail(SS_ERR_INVALID_ARG, "scale must be finite and positive");
    if (p->engine != SS_ENGINE_AUTO && p->engine != SS_ENGINE_VALU && p->engine != SS_ENGINE_MFMA)
        return fail(SS_ERR_INVALID_ARG, "unknown engine %d", p->engine);
    if (p->head_dim != 64 && p->head_dim != 128)
        return fail(SS_ERR_UNSUPPORTED, "head_dim %d is not supported (64 or 128)", p->head_dim);
    if (p->batch > 65535) return fail(SS_ERR_UNSUPPORTED, "batch above 65535");
    const int64_t rows = (int64_t)p->n_queries * (p->n_q_heads / p->n_kv_heads);
    const int64_t row_blocks = (rows + kValuRows - 1) / kValuRows;
    if ((int64_t)p->n_kv_heads * row_blocks > 65535 || (int64_t)p->n_kv_heads * cand_row_blocks((int)rows) > 65535)
        return fail(SS_ERR_UNSUPPORTED, "too many rows per request");
    return SS_OK;
}

int32_t check_view(const ss_problem_t* p, const ss_kv_view_t* v, const char* name) {
    if (!v) return fail(SS_ERR_INVALID_ARG, "%s view is NULL", name);
    if (!v->k || !v->v) return fail(SS_ERR_INVALID_ARG, "%s keys or values pointer is NULL", name);
    if (!aligned16(v->k) || !aligned16(v->v))
        return fail(SS_ERR_INVALID_ARG, "%s keys and values must be 16-byte aligned", name);
    if (v->max_len < 0) return fail(SS_ERR_INVALID_ARG, "%s max_len is negative", name);
    if (v->stride_b < 0 || v->stride_h < 0 || v->stride_t < 0)
        return fail(SS_ERR_INVALID_ARG, "%s strides must be non-negative", name);
    const int64_t es = elem_size(p);
    if ((v->stride_b * es) % 16 || (v->stride_h * es) % 16 || (v->stride_t * es) % 16)
        return fail(SS_ERR_INVALID_ARG, "%s strides must be multiples of 16 bytes", name);
    if (v->max_len > 1 && v->stride_t < p->head_dim)
        return fail(SS_ERR_INVALID_ARG, "%s stride_t is smaller than head_dim", name);
    // The kernels address a key inside a tile of at most 64 keys by a 32-bit
    // offset from the tile's first key (64-bit): keys * stride_t stays below
    // 2^31 for any stride_t up to 2^24 elements.
    if (v->stride_t > ((int64_t)1 << 24))
        return fail(SS_ERR_UNSUPPORTED, "%s stride_t above 2^24 elements", name);
    return SS_OK;
}

int32_t check_state(const ss_state_t* s, const char* name) {
    if (!s) return fail(SS_ERR_INVALID_ARG, "%s state is NULL", name);
    if (!s->acc || !s->m || !s->l) return fail(SS_ERR_INVALID_ARG, "%s state has a NULL array", name);
    if (s->n_slots <= 0) return fail(SS_ERR_INVALID_ARG, "%s state has no slots", name);
    return SS_OK;
}

// Which chunk kernel serves a problem. AUTO (and MFMA): every shape runs on
// the matrix cores: bf16 with up to 32 rows on the MFMA kernel (padded to a
// 16-row tile), more rows on the wide-row MFMA kernel, fp32 on the fp32 MFMA
// kernel (row groups of 32 beyond 32 rows); head_dim 128 or 64 on all.
// Measured on gfx950, the padded MFMA kernels stay far ahead of the VALU
// kernels, which are bound by vector and LDS issue. VALU forces the vector
// kernels (the small-row kernel below 16 rows of bf16 / head_dim 128); they
// also serve fp32 chunk lists (gathered verification).
enum class ChunkEngine { kValu, kValuSmall, kMfma, kMfmaWide, kMfmaF32 };

ChunkEngine chunk_engine(const ss_problem_t* p) {
    const int rows = p->n_queries * (p->n_q_heads / p->n_kv_heads);
    const bool bf16_128 = p->dtype == SS_BF16 && p->head_dim == 128;
    // every MFMA kernel takes head_dim 128 and 64 (the only ones check_problem admits)
    if (p->engine == SS_ENGINE_VALU) return (bf16_128 && rows < 16) ? ChunkEngine::kValuSmall : ChunkEngine::kValu;
    if (p->dtype == SS_F32) return ChunkEngine::kMfmaF32;
    return rows <= 32 ? ChunkEngine::kMfma : ChunkEngine::kMfmaWide;
}

int32_t validate_chunk(const ss_problem_t* problem, const void* q, const ss_kv_view_t* hist, int32_t chunk_len,
                       int32_t chunk_begin, int32_t n_chunks, int32_t cps, const ss_state_t* out,
                       int32_t slot_begin) {
    int32_t rc = check_problem(problem);
    if (rc) return rc;
    if (!q) return fail(SS_ERR_INVALID_ARG, "q is NULL");
    if (!aligned16(q)) return fail(SS_ERR_INVALID_ARG, "q must be 16-byte aligned");
    if ((rc = check_view(problem, hist, "history"))) return rc;
    if ((rc = check_state(out, "output"))) return rc;
    if (chunk_len <= 0) return fail(SS_ERR_INVALID_ARG, "chunk_len must be positive");
    if (chunk_begin < 0 || n_chunks < 0) return fail(SS_ERR_INVALID_ARG, "negative chunk range");
    if (cps <= 0) return fail(SS_ERR_INVALID_ARG, "chunks_per_slot must be positive");
    if (slot_begin < 0) return fail(SS_ERR_INVALID_ARG, "slot_begin is negative");
    const int64_t items = ((int64_t)n_chunks + cps - 1) / cps;
    if ((int64_t)slot_begin + items > out->n_slots)
        return fail(SS_ERR_INVALID_ARG, "slots [%d, %lld) exceed n_slots %d", slot_begin,
                    (long long)(slot_begin + items), out->n_slots);
    if (items > 0x7fffffff) return fail(SS_ERR_UNSUPPORTED, "too many slots in one call");
    return SS_OK;
}

ChunkParams make_chunk_params(const ss_problem_t* p, const void* q, const ss_kv_view_t* h, int32_t chunk_len,
                              int32_t chunk_begin, int32_t n_chunks, int32_t cps, const ss_state_t* out,
                              int32_t slot_begin) {
    ChunkParams c{};
    c.q = q;
    c.k = h->k;
    c.v = h->v;
    c.stride_b = h->stride_b;
    c.stride_h = h->stride_h;
    c.stride_t = h->stride_t;
    c.req_offset = h->req_offset;
    c.req_len = h->req_len;
    c.max_len = h->max_len;
    c.batch = p->batch;
    c.n_q_heads = p->n_q_heads;
    c.n_kv_heads = p->n_kv_heads;
    c.group = p->n_q_heads / p->n_kv_heads;
    c.n_queries = p->n_queries;
    c.rows = c.n_queries * c.group;
    c.scale = p->scale;
    c.chunk_len = chunk_len;
    c.chunk_begin = chunk_begin;
    c.n_chunks = n_chunks;
    c.cps = cps;
    c.n_items = (int32_t)(((int64_t)n_chunks + cps - 1) / cps);
    c.acc = out->acc;
    c.m = out->m;
    c.l = out->l;
    c.slot_begin = slot_begin;
    c.row_blocks = (c.rows + kValuRows - 1) / kValuRows;
    c.plan_align = kPlanAlign;
    c.full_len = h->max_len;
    return c;
}

hipError_t enqueue_chunk(const ss_problem_t* p, const ChunkParams& c, hipStream_t stream) {
    switch (chunk_engine(p)) {
        case ChunkEngine::kMfma: return launch_chunk_mfma(c, p->head_dim, stream);
        case ChunkEngine::kMfmaWide: return launch_chunk_mfma_wide(c, p->head_dim, stream);
        case ChunkEngine::kValuSmall: return launch_chunk_valu_small(c, p->head_dim, stream);
        case ChunkEngine::kMfmaF32:
            // contiguous pieces only: gathered chunk lists run on the VALU kernel
            if (!c.chunk_idx) return launch_chunk_mfma_f32(c, p->head_dim, stream);
            return launch_chunk_valu(c, p->dtype, p->head_dim, stream);
        default: return launch_chunk_valu(c, p->dtype, p->head_dim, stream);
    }
}

// ---------------------------------------------------------------------------
// Event pool of the streaming pipeline (one per device, reused across calls).
// ---------------------------------------------------------------------------

// Timing events of one streaming call; times are read relative to `start`,
// the compute stream's frontier when the call was made.
struct TimingSet {
    hipEvent_t start = nullptr;
    std::vector<hipEvent_t> copy0, copy1;  // per copy group
    std::vector<hipEvent_t> comp0, comp1;  // per chunk
    int32_t n_chunks = -1, group = 1;
};

constexpr int kTimingRing = 64;  // timed calls kept per device

struct StreamEvents {
    int device = -1;
    std::vector<hipEvent_t> arrived, freed;  // per staging buffer, no timing
    hipEvent_t start = nullptr;              // compute-stream frontier at call start
    // Staging ring as the last call left it, for SS_STREAM_CONTINUE.
    const void* staging = nullptr;
    int64_t buf_bytes = 0;
    int32_t n_buf = 0, next_buf = 0;
    std::vector<char> used;                  // buffer has a recorded `freed`
    TimingSet timing[kTimingRing];
    int64_t timed_calls = 0;
};

std::mutex g_ev_mutex;
std::vector<StreamEvents> g_events;

// SS_STREAM_DELAY: a host function on the copy stream that holds it.
void copy_delay(void*) {
    const struct timespec ts = {0, 2000000};
    nanosleep(&ts, nullptr);
}

hipError_t grow(std::vector<hipEvent_t>& v, size_t n, unsigned flags) {
    while (v.size() < n) {
        hipEvent_t e;
        hipError_t err = hipEventCreateWithFlags(&e, flags);
        if (err != hipSuccess) return err;
        v.push_back(e);
    }
    return hipSuccess;
}

}  // namespace

// ===========================================================================
// exported calls
// ===========================================================================

extern "C" SS_API int32_t ss_abi_version(void) { return SS_ABI_VERSION; }

extern "C" SS_API const char* ss_last_error(void) { return g_err.c_str(); }

extern "C" SS_API int64_t ss_state_bytes(const ss_problem_t* problem, int32_t n_slots) {
    int32_t rc = check_problem(problem);
    if (rc) return rc;
    if (n_slots <= 0) return fail(SS_ERR_INVALID_ARG, "n_slots must be positive");
    const int64_t rows = (int64_t)n_slots * problem->batch * problem->n_queries * problem->n_q_heads;
    ok();
    return rows * (problem->head_dim + 2) * 4;
}

extern "C" SS_API int32_t ss_verify_chunk(const ss_problem_t* problem, const void* q, const ss_kv_view_t* hist,
                                          int32_t chunk_len, int32_t chunk_begin, int32_t n_chunks,
                                          int32_t chunks_per_slot, const ss_state_t* out, int32_t slot_begin,
                                          ss_stream_t stream) {
    int32_t rc = validate_chunk(problem, q, hist, chunk_len, chunk_begin, n_chunks, chunks_per_slot, out, slot_begin);
    if (rc) return rc;
    if (n_chunks == 0) return ok();
    ChunkParams c = make_chunk_params(problem, q, hist, chunk_len, chunk_begin, n_chunks, chunks_per_slot, out,
                                      slot_begin);
    hipError_t e = enqueue_chunk(problem, c, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return fail(SS_ERR_HIP, "chunk kernel launch failed: %s", hipGetErrorString(e));
    return ok();
}

namespace {

// Validation of a candidate view for a problem (shared by the two calls
// that take one).
int32_t check_cand(const ss_problem_t* problem, const ss_kv_view_t* cand) {
    int32_t rc = check_view(problem, cand, "candidate");
    if (rc) return rc;
    if (problem->n_queries > 64) return fail(SS_ERR_UNSUPPORTED, "more than 64 candidates per request");
    if (cand->max_len != problem->n_queries)
        return fail(SS_ERR_INVALID_ARG, "candidate max_len (%d) must equal n_queries (%d)", cand->max_len,
                    problem->n_queries);
    return SS_OK;
}

CandParams make_cand_params(const ss_problem_t* problem, const void* q, const ss_kv_view_t* cand,
                            const int32_t* parents, uint64_t* mask_out, const ss_state_t* out, int32_t slot) {
    CandParams c{};
    c.q = q;
    c.k = cand->k;
    c.v = cand->v;
    c.stride_b = cand->stride_b;
    c.stride_h = cand->stride_h;
    c.stride_t = cand->stride_t;
    c.req_offset = cand->req_offset;
    c.batch = problem->batch;
    c.n_q_heads = problem->n_q_heads;
    c.n_kv_heads = problem->n_kv_heads;
    c.group = problem->n_q_heads / problem->n_kv_heads;
    c.n_queries = problem->n_queries;
    c.rows = c.n_queries * c.group;
    c.scale = problem->scale;
    c.parents = parents;
    c.mask_out = mask_out;
    c.acc = out->acc;
    c.m = out->m;
    c.l = out->l;
    c.slot = slot;
    c.row_blocks = cand_row_blocks(c.rows);
    return c;
}

}  // namespace

namespace {

// Where a whole-round call wants O and lse (see finish in verify_history).
struct FinishOut {
    float* o;
    float* lse;
};

// ss_verify_history without the status bookkeeping of the export (shared
// with the whole-round calls). With `fin` (whole-round calls), a round of
// one slot per stream on the MFMA kernels (narrow and wide-row) writes the finished rows
// into fin->o / fin->lse instead of the slots, and *merged is set: the
// caller then launches no merge.
int32_t verify_history(const ss_problem_t* problem, const void* q, const ss_kv_view_t* hist,
                       const ss_kv_view_t* cand, const int32_t* parents, uint64_t* mask_out,
                       const ss_block_stats_t* stats, int32_t n_slots, const ss_state_t* out, int32_t slot_begin,
                       ss_stream_t stream, const FinishOut* fin = nullptr, bool* merged = nullptr) {
    if (merged) *merged = false;
    if (!hist) return fail(SS_ERR_INVALID_ARG, "history view is NULL");
    if (n_slots < 1) return fail(SS_ERR_INVALID_ARG, "n_slots must be at least 1");
    // validation first (the chunk length does not change its outcome)
    int32_t rc = validate_chunk(problem, q, hist, kPlanAlign, 0, n_slots, 1, out, slot_begin);
    if (rc) return rc;
    if (cand && (rc = check_cand(problem, cand))) return rc;
    const ChunkEngine engine = chunk_engine(problem);
    const bool narrow = engine == ChunkEngine::kMfma;
    // the MFMA kernels attend the candidates inside the history launch
    const bool fuse = cand && (narrow || engine == ChunkEngine::kMfmaWide);
    if (cand && !fuse && n_slots < 2)
        return fail(SS_ERR_INVALID_ARG, "with candidates this engine needs n_slots >= 2");
    if (stats) {
        if (!narrow) return fail(SS_ERR_UNSUPPORTED, "block statistics need the narrow MFMA kernel");
        if (!stats->buf || stats->block_len <= 0 || stats->block_len % kPlanAlign || stats->n_blocks <= 0)
            return fail(SS_ERR_INVALID_ARG, "block statistics: buffer, a positive multiple of %d tokens, blocks",
                        kPlanAlign);
    }
    // Slots of the history (the VALU engines give the first slot to the
    // candidate region).
    const int32_t hist_slots = (cand && !fuse) ? n_slots - 1 : n_slots;
    const int32_t hist_begin = (cand && !fuse) ? slot_begin + 1 : slot_begin;
    const int64_t streams = (int64_t)problem->batch * problem->n_kv_heads;
    // Pieces per stream of a cut by fixed chunks: hist_slots, or for uniform
    // lengths on the narrow kernel one work-group per CU.
    int64_t pieces = hist_slots;
    if (narrow && !hist->req_len) {
        int wgs = 0;
        hipError_t e = mfma_wave_work_groups(problem->n_queries * (problem->n_q_heads / problem->n_kv_heads), &wgs);
        if (e != hipSuccess) return fail(SS_ERR_HIP, "device query failed: %s", hipGetErrorString(e));
        pieces = wgs / streams;
        if (pieces < 1) pieces = 1;
        if (pieces > hist_slots) pieces = hist_slots;
    }
    int64_t chunk = ((int64_t)hist->max_len + pieces - 1) / pieces;
    const int64_t align = stats ? stats->block_len : kPlanAlign;  // blocks never straddle two pieces
    chunk = (chunk + align - 1) / align * align;
    if (chunk < align) chunk = align;
    if (chunk > 0x7fffffff) return fail(SS_ERR_UNSUPPORTED, "history too long for %d slots", hist_slots);
    ChunkParams c = make_chunk_params(problem, q, hist, (int32_t)chunk, 0, hist_slots, 1, out, hist_begin);
    c.plan_align = (int32_t)align;
    hipStream_t s = static_cast<hipStream_t>(stream);
    hipError_t e = hipSuccess;
    if (stats) {
        c.stats = static_cast<float*>(stats->buf);
        c.stats_block = stats->block_len;
        c.stats_blocks = stats->n_blocks;
    }
    if (fuse) {
        c.with_cand = 1;
        c.ck = cand->k;
        c.cv = cand->v;
        c.c_stride_b = cand->stride_b;
        c.c_stride_h = cand->stride_h;
        c.c_stride_t = cand->stride_t;
        c.c_req_offset = cand->req_offset;
        c.parents = parents;
        c.mask_out = mask_out;
    } else if (cand) {
        e = launch_candidates(make_cand_params(problem, q, cand, parents, mask_out, out, slot_begin), problem->dtype,
                              problem->head_dim, s);
        if (e != hipSuccess) return fail(SS_ERR_HIP, "candidate kernel launch failed: %s", hipGetErrorString(e));
    }
    // one slot per stream, every stream's candidates in it: the slot is the result
    const bool finish =
        fin && (narrow || engine == ChunkEngine::kMfmaWide) && !stats && hist_slots == 1 && (fuse || !cand);
    if (finish) {
        c.fin_o = fin->o;
        c.fin_lse = fin->lse;
    }
    // ragged lengths on the narrow and the fp32 MFMA kernels (up to 32 rows,
    // one work-group per piece): the balanced cut
    const bool f32_cut = engine == ChunkEngine::kMfmaF32 && c.rows <= 32;
    if ((narrow || f32_cut) && hist->req_len && hist_slots >= 2) {
        c.plan_slots = hist_slots;
        // every slot starts empty; pieces overwrite theirs
        const int64_t rows = (int64_t)problem->batch * problem->n_queries * problem->n_q_heads;
        e = launch_state_fill(out->acc, out->m, out->l, (int64_t)hist_begin * rows, (int64_t)hist_slots * rows,
                              problem->head_dim, s);
        if (e != hipSuccess) return fail(SS_ERR_HIP, "state fill failed: %s", hipGetErrorString(e));
        e = narrow ? launch_history_mfma(c, problem->head_dim, s) : launch_history_mfma_f32(c, problem->head_dim, s);
    } else {
        e = enqueue_chunk(problem, c, s);
    }
    if (e != hipSuccess) return fail(SS_ERR_HIP, "history kernel launch failed: %s", hipGetErrorString(e));
    if (merged) *merged = finish;
    return SS_OK;
}

}  // namespace

extern "C" SS_API int32_t ss_verify_history(const ss_problem_t* problem, const void* q, const ss_kv_view_t* hist,
                                            const ss_kv_view_t* cand, const int32_t* parents, uint64_t* mask_out,
                                            const ss_block_stats_t* stats, int32_t n_slots, const ss_state_t* out,
                                            int32_t slot_begin, ss_stream_t stream) {
    const int32_t rc = verify_history(problem, q, hist, cand, parents, mask_out, stats, n_slots, out, slot_begin,
                                      stream);
    return rc ? rc : ok();
}

extern "C" SS_API int32_t ss_verify_candidates(const ss_problem_t* problem, const void* q, const ss_kv_view_t* cand,
                                               const int32_t* parents, uint64_t* mask_out, const ss_state_t* out,
                                               int32_t slot, ss_stream_t stream) {
    int32_t rc = check_problem(problem);
    if (rc) return rc;
    if (!q) return fail(SS_ERR_INVALID_ARG, "q is NULL");
    if (!aligned16(q)) return fail(SS_ERR_INVALID_ARG, "q must be 16-byte aligned");
    if ((rc = check_cand(problem, cand))) return rc;
    if ((rc = check_state(out, "output"))) return rc;
    if (slot < 0 || slot >= out->n_slots) return fail(SS_ERR_INVALID_ARG, "slot %d outside [0, %d)", slot, out->n_slots);
    hipError_t e = launch_candidates(make_cand_params(problem, q, cand, parents, mask_out, out, slot), problem->dtype,
                                     problem->head_dim, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return fail(SS_ERR_HIP, "candidate kernel launch failed: %s", hipGetErrorString(e));
    return ok();
}

namespace {

int32_t check_merge_out(const ss_problem_t* problem, const float* o, const float* lse) {
    if (!o || !lse) return fail(SS_ERR_INVALID_ARG, "o or lse is NULL");
    const int64_t n = (int64_t)problem->batch * problem->n_queries * problem->n_q_heads * problem->head_dim;
    if ((n + 255) / 256 > 0x7fffffff) return fail(SS_ERR_UNSUPPORTED, "output too large");
    return SS_OK;
}

int32_t merge_states(const ss_problem_t* problem, const ss_state_t* in, const int32_t* slots_per_req, float* o,
                     float* lse, ss_stream_t stream) {
    int32_t rc = check_problem(problem);
    if (rc) return rc;
    if ((rc = check_state(in, "input"))) return rc;
    if ((rc = check_merge_out(problem, o, lse))) return rc;
    MergeParams m{};
    m.acc = in->acc;
    m.m = in->m;
    m.l = in->l;
    m.n_slots = in->n_slots;
    m.slots_per_req = slots_per_req;
    m.batch = problem->batch;
    m.n_queries = problem->n_queries;
    m.n_q_heads = problem->n_q_heads;
    m.head_dim = problem->head_dim;
    m.o = o;
    m.lse = lse;
    hipError_t e = launch_merge(m, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return fail(SS_ERR_HIP, "merge kernel launch failed: %s", hipGetErrorString(e));
    return SS_OK;
}

// Ragged histories on the narrow MFMA kernel whose whole-round call runs
// faster as one piece per stream (a work-group per (request, KV head), all
// in parallel, finishing O and lse in the same launch) than under the
// balanced cut, whose work-groups run two or three short pieces one after
// another, each paying its start and its merge, and then a merge launch.
// Measured on MI355X (256 CUs), whole-round calls, lengths uniform in
// [n/8, n]: with at least one stream per CU 1.25-1.35x faster at n = 2048,
// 1.03-1.06x at 4096, slower from 5120; with 192 streams 1.23x at 2048, even
// at 3072; fewer streams leave CUs idle.
bool one_piece_per_stream(int64_t max_len, int64_t streams, int64_t cus) {
    return (max_len <= 4096 && streams >= cus) || (max_len <= 2048 && 4 * streams >= 3 * cus);
}

// Slots per (request, KV head) of a whole-round call for this problem and
// history view, before any capacity limit: one piece per work-group of one
// full launch where the lengths are known on the host (uniform lengths on
// the narrow MFMA kernel; the wide-row kernel's fixed chunks); for ragged
// lengths on the narrow kernel one (one_piece_per_stream, judged by the
// view's max_len) or 8 (the balanced cut grows its ranges when the longest
// stream needs more), on the fp32 MFMA kernel 8; and one more for the
// candidate region on the fp32 and VALU engines.
int32_t round_slots(const ss_problem_t* p, const ss_kv_view_t* hist, int32_t* n_slots) {
    const int32_t group = p->n_q_heads / p->n_kv_heads;
    const int32_t rows = p->n_queries * group;
    const int64_t streams = (int64_t)p->batch * p->n_kv_heads;
    int cus = 0;
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return fail(SS_ERR_HIP, "device query failed: %s", hipGetErrorString(e));
    if (cus < 1) cus = 1;
    int64_t s = 1;
    switch (chunk_engine(p)) {
        case ChunkEngine::kMfma:
            if (!hist->req_len)
                s = cus / streams;
            else
                s = one_piece_per_stream(hist->max_len, streams, cus) ? 1 : 8;
            break;
        case ChunkEngine::kMfmaWide: {
            // 8-wave groups of 256 rows, one per CU; 4-wave groups of 128
            // rows, two per CU
            const int64_t per_group = rows > 128 ? 256 : 128, per_cu = rows > 128 ? 1 : 2;
            s = per_cu * cus / (streams * ((rows + per_group - 1) / per_group));
            break;
        }
        case ChunkEngine::kMfmaF32:
            // the candidate slot, plus: uniform lengths one work-group per CU
            // (measured: 2 slots 381 us, 4 slots 404 us on a c2-shaped fp32
            // round); ragged lengths 8 for the balanced cut; beyond 32 rows
            // (fixed chunks, a work-group per row group of 32) about two
            // work-groups per CU
            if (rows > 32)
                s = 1 + 2 * (int64_t)cus / (streams * ((rows + 31) / 32));
            else
                s = hist->req_len ? 9 : 1 + (int64_t)cus / streams;
            if (s > 9) s = 9;
            break;
        default:
            s = 1 + 2 * (int64_t)cus / streams;
            if (s > 9) s = 9;
            break;
    }
    if (s < 1) s = 1;
    if (chunk_engine(p) != ChunkEngine::kMfma && chunk_engine(p) != ChunkEngine::kMfmaWide && s < 2) s = 2;
    if (s > 64) s = 64;
    *n_slots = (int32_t)s;
    return SS_OK;
}

// Everything a whole-round call checks before it enqueues anything (the
// slot storage aside).
int32_t validate_round(const ss_problem_t* problem, const void* q, const ss_kv_view_t* hist,
                       const ss_kv_view_t* cand, const float* o, const float* lse) {
    int32_t rc = check_problem(problem);
    if (rc) return rc;
    if (!q) return fail(SS_ERR_INVALID_ARG, "q is NULL");
    if (!aligned16(q)) return fail(SS_ERR_INVALID_ARG, "q must be 16-byte aligned");
    if ((rc = check_view(problem, hist, "history"))) return rc;
    if (!cand) return fail(SS_ERR_INVALID_ARG, "candidate view is NULL");
    if ((rc = check_cand(problem, cand))) return rc;
    return check_merge_out(problem, o, lse);
}

// The round (history and candidates into slots [0, n_slots), then the
// merge) on given slot storage.
int32_t verify_round(const ss_problem_t* problem, const void* q, const ss_kv_view_t* hist,
                     const ss_kv_view_t* cand, const int32_t* parents, uint64_t* mask_out, int32_t n_slots,
                     const ss_state_t* st, float* o, float* lse, ss_stream_t stream) {
    const FinishOut fin{o, lse};
    bool merged = false;
    int32_t rc = verify_history(problem, q, hist, cand, parents, mask_out, nullptr, n_slots, st, 0, stream, &fin,
                                &merged);
    if (rc || merged) return rc;
    ss_state_t used = *st;  // the merge folds the slots this round wrote, not the whole storage
    used.n_slots = n_slots;
    return merge_states(problem, &used, nullptr, o, lse, stream);
}

}  // namespace

extern "C" SS_API int32_t ss_merge_states(const ss_problem_t* problem, const ss_state_t* in,
                                          const int32_t* slots_per_req, float* o, float* lse, ss_stream_t stream) {
    const int32_t rc = merge_states(problem, in, slots_per_req, o, lse, stream);
    return rc ? rc : ok();
}

extern "C" SS_API int32_t ss_verify_round(const ss_problem_t* problem, const void* q, const ss_kv_view_t* hist,
                                          const ss_kv_view_t* cand, const int32_t* parents, uint64_t* mask_out,
                                          int32_t n_slots, const ss_state_t* work, float* o, float* lse,
                                          ss_stream_t stream) {
    int32_t rc = validate_round(problem, q, hist, cand, o, lse);
    if (rc) return rc;
    if ((rc = check_state(work, "workspace"))) return rc;
    if (n_slots < 0) return fail(SS_ERR_INVALID_ARG, "n_slots is negative");
    if (n_slots == 0) {
        if ((rc = round_slots(problem, hist, &n_slots))) return rc;
        if (n_slots > work->n_slots) n_slots = work->n_slots;
    }
    if (n_slots > work->n_slots)
        return fail(SS_ERR_INVALID_ARG, "n_slots %d exceeds the workspace's %d slots", n_slots, work->n_slots);
    rc = verify_round(problem, q, hist, cand, parents, mask_out, n_slots, work, o, lse, stream);
    return rc ? rc : ok();
}

// ---------------------------------------------------------------------------
// The whole round without a workspace argument, for callers that cannot
// allocate: the state slots live in a static device array of every GPU the
// library runs on.
// ---------------------------------------------------------------------------

namespace {

constexpr int64_t kRoundScratchBytes = (int64_t)64 << 20;

// The slot storage of ss_verify_round_noalloc. Host code never uses this
// name as an address: it is a host-side stand-in for the device array, whose
// device address comes from hipGetSymbolAddress (one per GPU, kept below).
__device__ __attribute__((aligned(256))) unsigned char scratch[kRoundScratchBytes];

constexpr int kScratchDevices = 64;
std::mutex g_scratch_mutex;
void* g_scratch_ptr[kScratchDevices];

// Device address of the current GPU's scratch array, looked up once per
// device with that device current.
int32_t scratch_ptr(void** out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return fail(SS_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
    if (dev < 0 || dev >= kScratchDevices) return fail(SS_ERR_UNSUPPORTED, "device %d beyond %d", dev, kScratchDevices);
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    if (!g_scratch_ptr[dev]) {
        void* ptr = nullptr;
        e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !ptr)
            return fail(SS_ERR_HIP, "hipGetSymbolAddress(scratch): %s", hipGetErrorString(e));
        g_scratch_ptr[dev] = ptr;
    }
    *out = g_scratch_ptr[dev];
    return SS_OK;
}

}  // namespace

extern "C" SS_API int32_t ss_verify_round_noalloc(const ss_problem_t* problem, const void* q,
                                                  const ss_kv_view_t* hist, const ss_kv_view_t* cand,
                                                  const int32_t* parents, uint64_t* mask_out, float* o, float* lse,
                                                  ss_stream_t stream) {
    int32_t rc = validate_round(problem, q, hist, cand, o, lse);
    if (rc) return rc;
    int32_t n_slots = 0;
    if ((rc = round_slots(problem, hist, &n_slots))) return rc;
    // slots that fit: acc [S][rows][d] + m [S][rows] + l [S][rows], fp32
    const int64_t rows = (int64_t)problem->batch * problem->n_queries * problem->n_q_heads;
    const int64_t slot_bytes = rows * (problem->head_dim + 2) * 4;
    const bool valu = chunk_engine(problem) != ChunkEngine::kMfma && chunk_engine(problem) != ChunkEngine::kMfmaWide;
    const int64_t fit = kRoundScratchBytes / slot_bytes;
    if (fit < (valu ? 2 : 1))
        return fail(SS_ERR_UNSUPPORTED, "the round needs %lld bytes of state per slot; the static scratch holds %lld",
                    (long long)slot_bytes, (long long)kRoundScratchBytes);
    if (n_slots > fit) n_slots = (int32_t)fit;
    void* base = nullptr;
    if ((rc = scratch_ptr(&base))) return rc;
    float* f = static_cast<float*>(base);
    ss_state_t st{};
    st.acc = f;
    st.m = f + (int64_t)n_slots * rows * problem->head_dim;
    st.l = st.m + (int64_t)n_slots * rows;
    st.n_slots = n_slots;
    rc = verify_round(problem, q, hist, cand, parents, mask_out, n_slots, &st, o, lse, stream);
    return rc ? rc : ok();
}

extern "C" SS_API int32_t ss_stream_history(const ss_problem_t* problem, const void* q, const void* host_kv,
                                            const int32_t* req_len, int32_t chunk_len, int32_t n_chunks,
                                            int32_t chunks_per_copy, void* staging, int32_t n_buf,
                                            const ss_state_t* out, int32_t slot_begin, ss_stream_t copy_stream,
                                            ss_stream_t compute_stream, int32_t flags) {
    int32_t rc = check_problem(problem);
    if (rc) return rc;
    if (!q || !host_kv || !staging) return fail(SS_ERR_INVALID_ARG, "q, host_kv or staging is NULL");
    if (!aligned16(q) || !aligned16(staging)) return fail(SS_ERR_INVALID_ARG, "q and staging must be 16-byte aligned");
    if ((rc = check_state(out, "output"))) return rc;
    if (chunk_len <= 0 || n_chunks < 0 || n_buf <= 0 || chunks_per_copy <= 0)
        return fail(SS_ERR_INVALID_ARG, "chunk_len, chunks_per_copy and n_buf must be positive, n_chunks non-negative");
    if (slot_begin < 0 || (int64_t)slot_begin + n_chunks > out->n_slots)
        return fail(SS_ERR_INVALID_ARG, "slots [%d, %d) exceed n_slots %d", slot_begin, slot_begin + n_chunks,
                    out->n_slots);
    if (copy_stream == compute_stream) return fail(SS_ERR_INVALID_ARG, "copy and compute streams must differ");
    if (flags & ~(SS_STREAM_TIMINGS | SS_STREAM_CONTINUE | SS_STREAM_POISON | SS_STREAM_DELAY))
        return fail(SS_ERR_INVALID_ARG, "unknown flags %d", flags);
    const bool timed = flags & SS_STREAM_TIMINGS;
    const bool cont = flags & SS_STREAM_CONTINUE;
    const bool poison = flags & SS_STREAM_POISON;
    const bool delay = flags & SS_STREAM_DELAY;

    const int64_t es = elem_size(problem);
    const int64_t half = (int64_t)problem->batch * problem->n_kv_heads * chunk_len * problem->head_dim;
    const int64_t chunk_bytes = 2 * half * es;
    const int64_t buf_bytes = chunk_bytes * chunks_per_copy;
    hipStream_t cs = static_cast<hipStream_t>(copy_stream);
    hipStream_t ks = static_cast<hipStream_t>(compute_stream);

    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return fail(SS_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));

    std::lock_guard<std::mutex> lock(g_ev_mutex);
    if ((int)g_events.size() <= dev) g_events.resize(dev + 1);
    StreamEvents& ev = g_events[dev];
    if (cont && !(ev.staging == staging && ev.n_buf == n_buf && ev.buf_bytes == buf_bytes))
        return fail(SS_ERR_INVALID_ARG, "SS_STREAM_CONTINUE needs the previous call's staging ring");
    if (n_chunks == 0) return ok();
    ev.device = dev;
    const unsigned sync_flags = hipEventDisableTiming;
    if ((e = grow(ev.arrived, n_buf, sync_flags)) != hipSuccess || (e = grow(ev.freed, n_buf, sync_flags)) != hipSuccess)
        return fail(SS_ERR_HIP, "event creation failed: %s", hipGetErrorString(e));
    if (!ev.start && (e = hipEventCreateWithFlags(&ev.start, sync_flags)) != hipSuccess)
        return fail(SS_ERR_HIP, "event creation failed: %s", hipGetErrorString(e));
    const int64_t n_groups = (n_chunks + chunks_per_copy - 1) / chunks_per_copy;
    TimingSet* ts = nullptr;
    if (timed) {
        ts = &ev.timing[ev.timed_calls % kTimingRing];
        if (!ts->start && (e = hipEventCreateWithFlags(&ts->start, hipEventDefault)) != hipSuccess)
            return fail(SS_ERR_HIP, "event creation failed: %s", hipGetErrorString(e));
        if ((e = grow(ts->copy0, n_groups, hipEventDefault)) != hipSuccess ||
            (e = grow(ts->copy1, n_groups, hipEventDefault)) != hipSuccess ||
            (e = grow(ts->comp0, n_chunks, hipEventDefault)) != hipSuccess ||
            (e = grow(ts->comp1, n_chunks, hipEventDefault)) != hipSuccess)
            return fail(SS_ERR_HIP, "event creation failed: %s", hipGetErrorString(e));
    }
    if (!cont) {
        // A fresh ring: the first copies may overwrite staging buffers that
        // earlier compute work still reads, so they wait for everything
        // already on the compute stream.
        ev.staging = staging;
        ev.n_buf = n_buf;
        ev.buf_bytes = buf_bytes;
        ev.next_buf = 0;
        ev.used.assign(n_buf, 0);
    }

    ss_kv_view_t view{};
    view.stride_b = (int64_t)problem->n_kv_heads * chunk_len * problem->head_dim;
    view.stride_h = (int64_t)chunk_len * problem->head_dim;
    view.stride_t = problem->head_dim;
    view.max_len = chunk_len;
    view.req_len = req_len;  // request b holds clamp(req_len[b] - j*C, 0, C) tokens of chunk j

    // A HIP error part-way leaves the earlier operations enqueued; the ring
    // bookkeeping no longer matches what the streams will do, so it is reset
    // (a following SS_STREAM_CONTINUE call is refused).
#define SS_TRY(call)                                                            \
    do {                                                                        \
        hipError_t err_ = (call);                                               \
        if (err_ != hipSuccess) {                                               \
            ev.staging = nullptr;                                               \
            ev.n_buf = 0;                                                       \
            return fail(SS_ERR_HIP, "%s: %s", #call, hipGetErrorString(err_)); \
        }                                                                       \
    } while (0)

    SS_TRY(hipEventRecord(ev.start, ks));
    if (timed) SS_TRY(hipEventRecord(ts->start, ks));
    // Continuing a ring: every buffer waits only for its own last reader
    // (its `freed` mark), so the copies run ahead of whatever else the
    // compute stream does in between: the next layer's history is fetched
    // while the current layer finishes.
    if (!cont) SS_TRY(hipStreamWaitEvent(cs, ev.start, 0));
    for (int64_t gi = 0; gi < n_groups; ++gi) {
        const int32_t bi = (int32_t)((ev.next_buf + gi) % n_buf);
        const int64_t j0 = gi * chunks_per_copy;
        const int64_t nj = (n_chunks - j0) < chunks_per_copy ? (n_chunks - j0) : chunks_per_copy;
        char* buf = static_cast<char*>(staging) + (int64_t)bi * buf_bytes;
        const char* src = static_cast<const char*>(host_kv) + j0 * chunk_bytes;
        if (ev.used[bi]) SS_TRY(hipStreamWaitEvent(cs, ev.freed[bi], 0));
        if (poison) SS_TRY(launch_word_fill(buf, buf_bytes, 0xffffffffu, cs));  // NaN in bf16 and fp32
        if (delay) SS_TRY(hipLaunchHostFunc(cs, copy_delay, nullptr));
        if (timed) SS_TRY(hipEventRecord(ts->copy0[gi], cs));
        SS_TRY(hipMemcpyAsync(buf, src, nj * chunk_bytes, hipMemcpyHostToDevice, cs));
        if (timed) SS_TRY(hipEventRecord(ts->copy1[gi], cs));
        SS_TRY(hipEventRecord(ev.arrived[bi], cs));

        SS_TRY(hipStreamWaitEvent(ks, ev.arrived[bi], 0));
        for (int64_t c = 0; c < nj; ++c) {
            const int64_t j = j0 + c;
            if (timed) SS_TRY(hipEventRecord(ts->comp0[j], ks));
            view.k = buf + c * chunk_bytes;
            view.v = buf + c * chunk_bytes + half * es;
            ChunkParams p = make_chunk_params(problem, q, &view, chunk_len, 0, 1, 1, out, slot_begin + (int32_t)j);
            if (req_len) p.len_offset = j * chunk_len;
            p.full_len = (int64_t)n_chunks * chunk_len;
            SS_TRY(enqueue_chunk(problem, p, ks));
            if (timed) SS_TRY(hipEventRecord(ts->comp1[j], ks));
        }
        SS_TRY(hipEventRecord(ev.freed[bi], ks));
        ev.used[bi] = 1;
    }
#undef SS_TRY
    ev.next_buf = (int32_t)((ev.next_buf + n_groups) % n_buf);
    if (timed) {
        ts->n_chunks = n_chunks;
        ts->group = chunks_per_copy;
        ++ev.timed_calls;
    }
    return ok();
}

extern "C" SS_API int32_t ss_stream_timings(int32_t back, int32_t n_chunks, float* copy_begin, float* copy_end,
                                            float* compute_begin, float* compute_end) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return fail(SS_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
    std::lock_guard<std::mutex> lock(g_ev_mutex);
    if ((int)g_events.size() <= dev) return fail(SS_ERR_INVALID_ARG, "no timed streaming call on this device");
    StreamEvents& ev = g_events[dev];
    if (back < 0 || back >= kTimingRing || back >= ev.timed_calls)
        return fail(SS_ERR_INVALID_ARG, "no timed streaming call %d calls back", back);
    const TimingSet& ts = ev.timing[(ev.timed_calls - 1 - back) % kTimingRing];
    if (n_chunks != ts.n_chunks)
        return fail(SS_ERR_INVALID_ARG, "n_chunks %d differs from the timed call's %d", n_chunks, ts.n_chunks);
    for (int32_t j = 0; j < n_chunks; ++j) {
        const int32_t gi = j / ts.group;
        struct {
            float* out;
            hipEvent_t ev;
        } items[4] = {{copy_begin, ts.copy0[gi]}, {copy_end, ts.copy1[gi]}, {compute_begin, ts.comp0[j]},
                      {compute_end, ts.comp1[j]}};
        for (auto& it : items) {
            if (!it.out) continue;
            float t;
            e = hipEventElapsedTime(&t, ts.start, it.ev);
            if (e != hipSuccess) return fail(SS_ERR_HIP, "hipEventElapsedTime: %s", hipGetErrorString(e));
            it.out[j] = t;
        }
    }
    return ok();
}

// ---------------------------------------------------------------------------
// Block statistics and block-sparse verification (SparseSpec-L's recycled
// attention statistics, Dustin's sparse verification).
// ---------------------------------------------------------------------------

extern "C" SS_API int32_t ss_verify_chunk_gathered(const ss_problem_t* problem, const void* q, const ss_kv_view_t* hist,
                                                   int32_t chunk_len, const int32_t* chunk_idx, int32_t n_sel,
                                                   int32_t chunks_per_slot, const ss_state_t* out, int32_t slot_begin,
                                                   ss_stream_t stream) {
    int32_t rc = validate_chunk(problem, q, hist, chunk_len, 0, n_sel, chunks_per_slot, out, slot_begin);
    if (rc) return rc;
    if (!chunk_idx) return fail(SS_ERR_INVALID_ARG, "chunk_idx is NULL");
    if (chunks_per_slot > 1) {
        if (chunk_engine(problem) != ChunkEngine::kMfma)
            return fail(SS_ERR_UNSUPPORTED, "several gathered chunks per slot need the narrow MFMA engine");
        if (chunk_len % 32) return fail(SS_ERR_INVALID_ARG, "several gathered chunks per slot need chunk_len %% 32 == 0");
        if (chunks_per_slot > kMaxGatherPerSlot)
            return fail(SS_ERR_UNSUPPORTED, "at most %d gathered chunks per slot", kMaxGatherPerSlot);
    }
    if (n_sel == 0) return ok();
    ChunkParams c = make_chunk_params(problem, q, hist, chunk_len, 0, n_sel, chunks_per_slot, out, slot_begin);
    c.chunk_idx = chunk_idx;
    c.n_sel = n_sel;
    hipError_t e = enqueue_chunk(problem, c, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return fail(SS_ERR_HIP, "chunk kernel launch failed: %s", hipGetErrorString(e));
    return ok();
}

extern "C" SS_API int32_t ss_block_importance(const ss_problem_t* problem, const ss_state_t* states, int32_t slot_begin,
                                              int32_t n_blocks, const float* lse, float* importance,
                                              ss_stream_t stream) {
    int32_t rc = check_problem(problem);
    if (rc) return rc;
    if ((rc = check_state(states, "block"))) return rc;
    if (!lse || !importance) return fail(SS_ERR_INVALID_ARG, "lse or importance is NULL");
    if (n_blocks < 0 || slot_begin < 0 || (int64_t)slot_begin + n_blocks > states->n_slots)
        return fail(SS_ERR_INVALID_ARG, "blocks [%d, %d) outside the %d slots", slot_begin, slot_begin + n_blocks,
                    states->n_slots);
    ImportanceParams p{};
    p.m = states->m;
    p.l = states->l;
    p.slot_begin = slot_begin;
    p.batch = problem->batch;
    p.n_q_heads = problem->n_q_heads;
    p.n_kv_heads = problem->n_kv_heads;
    p.n_queries = problem->n_queries;
    p.n_blocks = n_blocks;
    p.lse = lse;
    p.importance = importance;
    hipError_t e = launch_importance(p, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return fail(SS_ERR_HIP, "importance kernel launch failed: %s", hipGetErrorString(e));
    return ok();
}

extern "C" SS_API int64_t ss_block_stats_bytes(const ss_problem_t* problem, int32_t n_blocks) {
    int32_t rc = check_problem(problem);
    if (rc) return rc;
    if (n_blocks <= 0) return fail(SS_ERR_INVALID_ARG, "n_blocks must be positive");
    ok();
    return (int64_t)kStatsQuarters * problem->batch * problem->n_queries * problem->n_q_heads * n_blocks * 2 *
           (int64_t)sizeof(float);
}

extern "C" SS_API int32_t ss_block_importance_stats(const ss_problem_t* problem, const ss_block_stats_t* stats,
                                                    const int32_t* req_len, int32_t max_len, const float* lse,
                                                    float* importance, ss_stream_t stream) {
    int32_t rc = check_problem(problem);
    if (rc) return rc;
    if (!stats || !stats->buf || stats->n_blocks <= 0 || !lse || !importance)
        return fail(SS_ERR_INVALID_ARG, "statistics, lse or importance missing");
    if (stats->block_len <= 0 || stats->block_len % kPlanAlign || max_len < 0)
        return fail(SS_ERR_INVALID_ARG, "block_len must be a positive multiple of %d, max_len >= 0", kPlanAlign);
    StatsImportanceParams p{};
    p.ml = static_cast<const float2*>(stats->buf);
    p.batch = problem->batch;
    p.n_q_heads = problem->n_q_heads;
    p.n_kv_heads = problem->n_kv_heads;
    p.n_queries = problem->n_queries;
    p.n_blocks = stats->n_blocks;
    p.block_len = stats->block_len;
    p.req_len = req_len;
    p.max_len = max_len;
    p.lse = lse;
    p.importance = importance;
    hipError_t e = launch_importance_stats(p, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return fail(SS_ERR_HIP, "importance kernel launch failed: %s", hipGetErrorString(e));
    return ok();
}

extern "C" SS_API int32_t ss_select_blocks(const ss_problem_t* problem, const float* importance, int32_t n_blocks,
                                           const int32_t* req_len, int32_t max_len, int32_t block_len, int32_t k,
                                           int32_t* out, ss_stream_t stream) {
    int32_t rc = check_problem(problem);
    if (rc) return rc;
    if (!importance || !out) return fail(SS_ERR_INVALID_ARG, "importance or out is NULL");
    if (n_blocks < 1 || k < 1 || block_len < 1 || max_len < 0)
        return fail(SS_ERR_INVALID_ARG, "n_blocks, k and block_len must be positive, max_len non-negative");
    if (n_blocks > kMaxSelectBlocks) return fail(SS_ERR_UNSUPPORTED, "more than %d blocks", kMaxSelectBlocks);
    SelectParams p{};
    p.importance = importance;
    p.batch = problem->batch;
    p.n_kv_heads = problem->n_kv_heads;
    p.n_blocks = n_blocks;
    p.k = k;
    p.block_len = block_len;
    p.max_len = max_len;
    p.req_len = req_len;
    p.out = out;
    hipError_t e = launch_select(p, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return fail(SS_ERR_HIP, "selection kernel launch failed: %s", hipGetErrorString(e));
    return ok();
}

// ---------------------------------------------------------------------------
// Commit-aware KV tiering (section 4.1): the migration endpoint rule and the
// row copies that move committed KV between the GPU tail and the host store.
// ---------------------------------------------------------------------------

namespace {

// A per-request row range of a view whose addresses the host can compute:
// no device offsets, contiguous feature rows.
int32_t check_row_view(const ss_problem_t* p, const ss_kv_view_t* v, const char* name) {
    int32_t rc = check_view(p, v, name);
    if (rc) return rc;
    if (v->req_offset) return fail(SS_ERR_INVALID_ARG, "%s view: row copies need req_offset NULL", name);
    if (v->stride_t != p->head_dim) return fail(SS_ERR_INVALID_ARG, "%s view: rows must be contiguous", name);
    return SS_OK;
}

}  // namespace

extern "C" SS_API int32_t ss_tier_migration_end(int64_t h, int64_t c, int64_t tail, int64_t gran, int64_t* e) {
    if (!e) return fail(SS_ERR_INVALID_ARG, "e is NULL");
    if (gran <= 0 || tail < 0) return fail(SS_ERR_INVALID_ARG, "granularity must be positive, tail non-negative");
    if (h < 0 || h > c) return fail(SS_ERR_INVALID_ARG, "need 0 <= H <= C (H=%lld, C=%lld)", (long long)h, (long long)c);
    const int64_t old = c - tail > 0 ? c - tail : 0;
    const int64_t end = gran * (old / gran);
    *e = end > h ? end : h;
    return ok();
}

extern "C" SS_API int32_t ss_kv_copy_rows(const ss_problem_t* problem, const ss_kv_view_t* src, const int64_t* src_row,
                                          const ss_kv_view_t* dst, const int64_t* dst_row, const int64_t* n_rows,
                                          ss_stream_t stream) {
    int32_t rc = check_problem(problem);
    if (rc) return rc;
    if ((rc = check_row_view(problem, src, "source")) || (rc = check_row_view(problem, dst, "destination"))) return rc;
    if (!src_row || !dst_row || !n_rows) return fail(SS_ERR_INVALID_ARG, "row arrays must not be NULL");
    for (int32_t b = 0; b < problem->batch; ++b) {
        if (n_rows[b] < 0 || src_row[b] < 0 || dst_row[b] < 0 || src_row[b] + n_rows[b] > src->max_len ||
            dst_row[b] + n_rows[b] > dst->max_len)
            return fail(SS_ERR_INVALID_ARG, "request %d: rows outside the views", b);
    }
    const int64_t es = elem_size(problem), d = problem->head_dim;
    hipStream_t st = static_cast<hipStream_t>(stream);
    for (int32_t b = 0; b < problem->batch; ++b) {
        if (n_rows[b] == 0) continue;
        for (int kv = 0; kv < 2; ++kv) {
            const char* s0 = static_cast<const char*>(kv ? src->v : src->k) +
                             (b * src->stride_b + src_row[b] * src->stride_t) * es;
            char* d0 = static_cast<char*>(const_cast<void*>(kv ? dst->v : dst->k)) +
                       (b * dst->stride_b + dst_row[b] * dst->stride_t) * es;
            hipError_t e = hipMemcpy2DAsync(d0, dst->stride_h * es, s0, src->stride_h * es, n_rows[b] * d * es,
                                            problem->n_kv_heads, hipMemcpyDeviceToDevice, st);
            if (e != hipSuccess) return fail(SS_ERR_HIP, "row copy failed: %s", hipGetErrorString(e));
        }
    }
    return ok();
}

extern "C" SS_API int32_t ss_tier_migrate(const ss_problem_t* problem, const ss_kv_view_t* tail,
                                          const int64_t* tail_first, const int64_t* begin, const int64_t* end,
                                          void* host_kv, int32_t chunk_len, int32_t n_chunks, ss_stream_t stream) {
    int32_t rc = check_problem(problem);
    if (rc) return rc;
    if ((rc = check_row_view(problem, tail, "tail"))) return rc;
    if (!tail_first || !begin || !end || !host_kv) return fail(SS_ERR_INVALID_ARG, "NULL argument");
    if (chunk_len <= 0 || n_chunks < 0) return fail(SS_ERR_INVALID_ARG, "invalid chunk geometry");
    const int64_t cap = (int64_t)chunk_len * n_chunks;
    for (int32_t b = 0; b < problem->batch; ++b) {
        if (begin[b] < tail_first[b] || end[b] < begin[b] || end[b] > cap ||
            end[b] - tail_first[b] > tail->max_len)
            return fail(SS_ERR_INVALID_ARG, "request %d: range [%lld, %lld) outside the tail or the host store", b,
                        (long long)begin[b], (long long)end[b]);
    }
    const int64_t es = elem_size(problem), d = problem->head_dim, hkv = problem->n_kv_heads;
    const int64_t B = problem->batch, C = chunk_len;
    hipStream_t st = static_cast<hipStream_t>(stream);
    for (int32_t b = 0; b < problem->batch; ++b) {
        for (int64_t t = begin[b]; t < end[b];) {
            const int64_t j = t / C, r = t % C;
            const int64_t n = (end[b] - t) < (C - r) ? (end[b] - t) : (C - r);  // rows within chunk j
            for (int kv = 0; kv < 2; ++kv) {
                const char* s0 = static_cast<const char*>(kv ? tail->v : tail->k) +
                                 (b * tail->stride_b + (t - tail_first[b]) * tail->stride_t) * es;
                // chunk-major host store [J][2][B][Hkv][C][d]
                char* d0 = static_cast<char*>(host_kv) + ((((j * 2 + kv) * B + b) * hkv) * C + r) * d * es;
                hipError_t e = hipMemcpy2DAsync(d0, C * d * es, s0, tail->stride_h * es, n * d * es, hkv,
                                                hipMemcpyDeviceToHost, st);
                if (e != hipSuccess) return fail(SS_ERR_HIP, "migration copy failed: %s", hipGetErrorString(e));
            }
            t += n;
        }
    }
    return ok();
}

extern "C" SS_API int32_t ss_read_probe(const void* src, int64_t bytes, int32_t n_work_groups, uint32_t* sink,
                                        ss_stream_t stream) {
    if (!src || !sink) return fail(SS_ERR_INVALID_ARG, "src or sink is NULL");
    if (!aligned16(src) || bytes < 16 || n_work_groups <= 0)
        return fail(SS_ERR_INVALID_ARG, "src must be 16-byte aligned, bytes >= 16, n_work_groups > 0");
    hipError_t e = launch_read_probe(src, bytes, n_work_groups, sink, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return fail(SS_ERR_HIP, "read probe launch failed: %s", hipGetErrorString(e));
    return ok();
}

extern "C" SS_API int32_t ss_mfma_probe(const void* operands, int64_t n_operands, int32_t iters,
                                        int32_t n_work_groups, float* sink, ss_stream_t stream) {
    if (!operands || !sink) return fail(SS_ERR_INVALID_ARG, "operands or sink is NULL");
    if (!aligned16(operands) || n_operands < mfma_probe_wave_elems() || iters <= 0 || n_work_groups <= 0)
        return fail(SS_ERR_INVALID_ARG, "operands must be 16-byte aligned with n_operands >= %lld, iters > 0, "
                    "n_work_groups > 0", (long long)mfma_probe_wave_elems());
    hipError_t e = launch_mfma_probe(operands, n_operands, iters, n_work_groups, sink, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return fail(SS_ERR_HIP, "matrix-core probe launch failed: %s", hipGetErrorString(e));
    return ok();
}

extern "C" SS_API int32_t ss_tree_mask_host(const int32_t* parents, int32_t n, uint64_t* out) {
    if (!parents || !out) return fail(SS_ERR_INVALID_ARG, "parents or out is NULL");
    if (n < 0 || n > 64) return fail(SS_ERR_INVALID_ARG, "n must be in [0, 64]");
    for (int32_t i = 0; i < n; ++i) out[i] = tree_bits_step(out, i, parents[i]);
    return ok();
}

extern "C" SS_API int32_t ss_slot_tokens_host(int32_t len, int32_t chunk_len, int32_t chunk_begin, int32_t n_chunks,
                                              int32_t chunks_per_slot, int32_t s, int64_t* t0, int64_t* t1) {
    if (!t0 || !t1) return fail(SS_ERR_INVALID_ARG, "t0 or t1 is NULL");
    if (len < 0 || chunk_len <= 0 || chunk_begin < 0 || n_chunks < 0 || chunks_per_slot <= 0 || s < 0)
        return fail(SS_ERR_INVALID_ARG, "invalid chunk arguments");
    slot_tokens(len, chunk_len, chunk_begin, n_chunks, chunks_per_slot, s, t0, t1);
    return ok();
}

extern "C" SS_API int32_t ss_history_plan_host(const int32_t* lens, int32_t batch, int32_t n_kv_heads, int32_t max_len,
                                               int32_t n_wg, int32_t n_slots, int64_t* plan, int64_t* piece_len) {
    if (!lens || !plan || !piece_len) return fail(SS_ERR_INVALID_ARG, "lens, plan or piece_len is NULL");
    if (batch <= 0 || n_kv_heads <= 0 || max_len < 0 || n_wg <= 0 || n_slots < 2)
        return fail(SS_ERR_INVALID_ARG, "invalid plan arguments");
    auto len_of = [&](int32_t b) { return clamp_len(lens[b], max_len); };
    int64_t total = 0, pad_max = 0;
    for (int32_t b = 0; b < batch; ++b) {
        const int64_t pad = plan_pad(len_of(b));
        total += plan_span(len_of(b));
        if (pad > pad_max) pad_max = pad;
    }
    total *= n_kv_heads;
    const int64_t L = plan_piece_len(total, pad_max, n_wg, n_slots);
    *piece_len = L;
    const int64_t n_entries = (int64_t)batch * n_kv_heads * n_slots;
    for (int64_t i = 0; i < n_entries; ++i) {
        plan[4 * i + 0] = plan[4 * i + 1] = plan[4 * i + 2] = -1;
        plan[4 * i + 3] = 0;
    }
    for (int64_t w = 0; w < n_wg; ++w) {
        // The same start rule as the kernel's wave scan, as a plain loop.
        const int64_t lo = w * L;
        int32_t b_first = batch;
        int64_t line = 0, start = 0;
        for (int32_t b = 0; b < batch; ++b) {
            const int64_t span = (int64_t)n_kv_heads * plan_span(len_of(b));
            if (start + span > lo || start >= lo) {
                b_first = b;
                line = start;
                break;
            }
            start += span;
        }
        PlanCursor cur{b_first, 0, line};
        PlanPiece pc;
        while (plan_next(len_of, batch, n_kv_heads, L, total, n_slots, w, cur, pc)) {
            int64_t* e = plan + 4 * (((int64_t)pc.b * n_kv_heads + pc.g) * n_slots);
            if (pc.k >= n_slots) {
                e[4 * (n_slots - 1) + 3] += 1000;  // a piece beyond the slots: flagged
                continue;
            }
            if (pc.k >= 0) {
                e[4 * pc.k + 0] = w;
                e[4 * pc.k + 1] = pc.t0;
                e[4 * pc.k + 2] = pc.t1;
                e[4 * pc.k + 3] += 1;
            }
            for (int32_t j = pc.k + 1; j < pc.fill_end; ++j) {
                e[4 * j + 0] = w;
                e[4 * j + 1] = e[4 * j + 2] = -1;
                e[4 * j + 3] += 1;
            }
        }
    }
    return ok();
}
