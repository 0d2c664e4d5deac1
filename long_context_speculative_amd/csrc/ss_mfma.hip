// MFMA bf16 chunk kernels of libssverify, for up to 32 rows per KV head
// (padded to a 16-row tile) and head_dim 128 or 64.
//
// SpecStream ("Resource-Efficient Speculative Decoding for Long-Context LLM
// Serving"), section 4.2: a history chunk serves the whole verification query
// group. For one (slot, KV head, request) a work-group of 4 waves walks the
// slot's keys in tiles of 32; wave w takes tiles w, w+4, ... Every wave holds
// all R = n_queries * G rows of the KV head (padded to 16 or 32), so each K
// and V byte is read from HBM exactly once and feeds every query and every
// head of the GQA group inside one MFMA.
//
// Per tile, with v_mfma_f32_16x16x32_bf16 (16x16 output tiles):
//   S^T[key][row] = K Q^T            A = K straight from global memory (a
//                                    lane holds 8 consecutive features of one
//                                    key: one 16-byte load), B = Q^T held in
//                                    registers for the whole kernel
//   online softmax (Eq. 7-8)         base-2 exponent on scale*log2(e)-scaled
//                                    scores; the row max needs one exchange
//                                    across the 4 lane groups; the
//                                    accumulator is rescaled only when some
//                                    row's maximum grows
//   O^T[x][row] += V^T P^T           B = P in registers straight from the S^T
//                                    output, as two bf16 operands (the
//                                    rounded weight and its rounding
//                                    remainder), A = V^T read from a per-wave
//                                    LDS tile that holds V transposed
//                                    (key-contiguous rows)
// The 4 waves' states are merged with Eq. (8) through LDS at the end and
// written as the slot's state (m in natural-log units).

#include <type_traits>

#include "ss_common.h"

namespace ssv {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kWaves = 4;
static_assert(kWaves == kStatsQuarters, "block statistics keep one quarter per wave");
constexpr int kThreads = 64 * kWaves;
constexpr int kTile = 32;      // keys per wave iteration
static_assert(kPlanAlign % (kTile * kWaves) == 0, "a block holds a whole step of every wave");
constexpr int kVtRow = 36;     // bf16 per transposed-V row: 32 keys + 4 pad (72 bytes)

template <int D, int NRT>
struct MfmaSmem {
    // Accumulator floats per lane of the feature tiles one wave owns in the
    // final merge (wave w owns the 16-feature tiles xt with xt % kWaves == w).
    static constexpr int kOwnRegs = (D / 16 / kWaves) * NRT * 4;
    uint64_t cbits[32];  // candidate visibility bits (at most 32 candidates here)
    int32_t gidx[kMaxGatherPerSlot];  // a gathered slot's chunk list
    // 16-byte aligned whatever precedes it: at a lesser alignment every 8-
    // and 16-byte LDS access to it is split in two, and the key loop issues
    // twice the LDS instructions (measured: 46% slower launches)
    union alignas(16) {
        uint16_t vt[kWaves][D][kVtRow];
        struct {
            // [owner wave][contributing wave, owner skipped][owned float][lane]
            float acc[kWaves][kWaves - 1][kOwnRegs][64];
            float m[kWaves][16 * NRT];
            float l[kWaves][16 * NRT];
        } mg;
    } u;
};

__device__ __forceinline__ float exp2_hw(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ void wave_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

// Key tiles of a piece. ContigTiles: tokens [t0, t1) in tiles of kTile.
// GatherTiles: the listed chunks of a gathered slot one after the other,
// chunk_len / kTile tiles each (chunk_len a multiple of kTile); a tile of an
// entry < 0 or past the request's end has no keys and is skipped.
struct ContigTiles {
    int64_t t0, t1;
    __device__ int n_tiles() const { return (int)((t1 - t0 + kTile - 1) / kTile); }
    __device__ int64_t tk(int tau) const { return t0 + (int64_t)kTile * tau; }
    __device__ int valid(int tau) const { return (int)min((int64_t)kTile, t1 - tk(tau)); }
};

struct GatherTiles {
    const int32_t* idx;  // the slot's entries, staged in LDS by the kernel
    int32_t n_entries, chunk_len, len;
    __device__ int per_chunk() const { return chunk_len / kTile; }
    __device__ int n_tiles() const { return n_entries * per_chunk(); }
    // First token of tile tau and its keys (0: an entry < 0 or past the end).
    __device__ void tile(int tau, int64_t* tk, int* valid) const {
        const int j = tau / per_chunk();
        const int32_t c = __builtin_amdgcn_readfirstlane(idx[j]);
        const int64_t t = (int64_t)c * chunk_len + (int64_t)kTile * (tau - j * per_chunk());
        const int64_t left = (int64_t)len - t;
        *valid = c < 0 ? 0 : (int)(left < 0 ? 0 : (left > kTile ? kTile : left));
        *tk = *valid > 0 ? t : 0;
    }
};

// State of the key tiles `tl` of stream (at.b(), at.g()) for every row of the
// KV head, and with `cand` also of the request's candidate rows under their
// mask, written to slot at.slot(). `at` is asked again at each use, so
// that a caller can keep these indices out of registers during the key loop.
// Uses the work-group's LDS; callers that run several pieces in a row
// separate them with a barrier.
template <int D, int NRT, bool STATS, class At, class Tiles>
__device__ __forceinline__ void mfma_piece(const ChunkParams& p, MfmaSmem<D, NRT>& sm, const At& at, const Tiles& tl,
                                           bool cand) {
    constexpr bool kGather = std::is_same<Tiles, GatherTiles>::value;
    static_assert(!(kGather && STATS), "block statistics cover contiguous pieces only");
    constexpr int NS = D / 32;   // feature steps of 32 for S = K Q^T
    constexpr int NXT = D / 16;  // 16-feature output tiles for O^T = V^T P^T
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int l16 = lane & 15, q4 = lane >> 4;

    const int64_t base = (p.req_offset ? p.req_offset[at.b()] : (int64_t)at.b() * p.stride_b) +
                         (int64_t)at.g() * p.stride_h;
    const uint16_t* __restrict__ kp = static_cast<const uint16_t*>(p.k) + base;
    const uint16_t* __restrict__ vp = static_cast<const uint16_t*>(p.v) + base;
    const int64_t st = p.stride_t;

    // Q^T fragments: row r = l16 + 16*rt, features 32*k + 8*q4 .. +7.
    bf16x8 qf[NRT][NS];
#pragma unroll
    for (int rt = 0; rt < NRT; ++rt) {
        const int r = l16 + 16 * rt;
        if (r < p.rows) {
            const int i = r / p.group, h = at.g() * p.group + r % p.group;
            const uint16_t* qrow =
                static_cast<const uint16_t*>(p.q) + ((int64_t)(at.b() * p.n_queries + i) * p.n_q_heads + h) * D;
#pragma unroll
            for (int k = 0; k < NS; ++k) qf[rt][k] = as_bf16x8(*reinterpret_cast<const u32x4*>(qrow + 32 * k + 8 * q4));
        } else {
#pragma unroll
            for (int k = 0; k < NS; ++k) qf[rt][k] = as_bf16x8(u32x4{0u, 0u, 0u, 0u});
        }
    }

    floatx4 o[NXT][NRT];
#pragma unroll
    for (int xt = 0; xt < NXT; ++xt)
#pragma unroll
        for (int rt = 0; rt < NRT; ++rt) o[xt][rt] = floatx4{0.f, 0.f, 0.f, 0.f};
    float m_run[NRT], l_run[NRT];  // log2-domain running max; per-lane partial sums
#pragma unroll
    for (int rt = 0; rt < NRT; ++rt) {
        m_run[rt] = -INFINITY;
        l_run[rt] = 0.f;
    }
    const float c = p.scale * kLog2e;

    const int n_tiles = tl.n_tiles();
    uint16_t(*vt)[kVtRow] = sm.u.vt[w];
    static_assert(D == 64 || D == 128, "head_dim 64 or 128");
    constexpr int VH = D / 64;  // V key groups per lane (see load_v_at)
    const int vx = D == 128 ? 8 * l16 : 8 * (l16 & 7);
    auto v_kg = [&](int h) { return D == 128 ? q4 + 4 * h : q4 + 4 * (l16 >> 3); };

    // Loads address a tile as a uniform base (scalar registers) plus a 32-bit
    // per-lane offset. Keys past the range are clamped to its last key so
    // every load stays in bounds; their scores are masked below. K and V are
    // read once per round (the whole GQA group of a KV head shares one
    // work-group), so the loads are non-temporal: streamed past the caches'
    // normal retention, which reads HBM measurably faster on this device.
    // K fragment: keys 16*kt + l16 of the tile, features 32*k + 8*q4 .. +7.
    auto load_k_at = [&](const uint16_t* tb, int stride, int last, u32x4(&dst)[2][NS]) {
#pragma unroll
        for (int kt = 0; kt < 2; ++kt) {
            const int off = min(16 * kt + l16, last) * stride + 8 * q4;
#pragma unroll
            for (int k = 0; k < NS; ++k) dst[kt][k] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(tb + off + 32 * k));
        }
    };
    // V rows 4*kg + e, features vx .. vx+7: with D = 128, key groups
    // kg = q4 + 4*h (h = 0, 1) at vx = 8*l16; with D = 64 the upper half of
    // each 16-lane group takes the other 16 keys, kg = q4 + 4*(l16 >> 3) at
    // vx = 8*(l16 & 7), one key group per lane.
    auto load_v_at = [&](const uint16_t* tb, int stride, int last, u32x4(&dst)[VH][4]) {
#pragma unroll
        for (int h = 0; h < VH; ++h)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int off = min(4 * v_kg(h) + e, last) * stride + vx;
                dst[h][e] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(tb + off));
            }
    };
    const int sti = (int)st;
    // Tile tau's loads (tk: its first token, valid > 0: its keys).
    auto load_k = [&](int64_t tk, int valid, u32x4(&dst)[2][NS]) { load_k_at(kp + tk * st, sti, valid - 1, dst); };
    auto load_v = [&](int64_t tk, int valid, u32x4(&dst)[VH][4]) { load_v_at(vp + tk * st, sti, valid - 1, dst); };

    // Block statistics: the running state of the keys of the current block
    // (stats_block tokens) that this wave attends, written out when the
    // wave moves to the next block: reference maximum m_run, and this
    // lane's share bl of the sum of the (bf16) weights. Entry layout
    // [wave][request][KV head][block][row of the head], so that one store
    // (lane group q4 writes row tile q4) covers consecutive rows.
    float bl[NRT];
#pragma unroll
    for (int rt = 0; rt < NRT; ++rt) bl[rt] = 0.f;
    int64_t blk_cur = -1, blk_end = -1;  // current block and the token that ends it
    auto flush_block = [&](int64_t blk) {
        float mv = -INFINITY, lv = 0.f;
#pragma unroll
        for (int rt = 0; rt < NRT; ++rt) {
            float lsum = bl[rt];
            lsum = group4_sum(lsum);
            if (q4 == rt) {
                mv = m_run[rt];
                lv = lsum;
            }
        }
        const int r = l16 + 16 * q4;
        if (q4 < NRT && r < p.rows && blk < p.stats_blocks) {
            const int64_t e =
                ((((int64_t)w * p.batch + at.b()) * p.n_kv_heads + at.g()) * p.stats_blocks + blk) * p.rows + r;
            *reinterpret_cast<float2*>(p.stats + 2 * e) = make_float2(mv == -INFINITY ? -INFINITY : mv * kLn2, lv);
        }
    };

    // One tile: the first `valid` keys, and of those only the ones whose bit
    // is set in vis[rt] (per lane row) when `masked`. after_stage runs once
    // V is in LDS (its registers are free), after_s once S^T has read K.
    auto consume = [&](u32x4(&kf)[2][NS], u32x4(&vr)[VH][4], int valid, bool masked, const uint32_t(&vis)[NRT],
                       auto after_stage, auto after_s) {
        // Stage V transposed: vt[x][key] holds 4 keys per 8-byte word.
#pragma unroll
        for (int h = 0; h < VH; ++h) {
            const int kg = v_kg(h);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const uint32_t d0 = vr[h][0][i], d1 = vr[h][1][i], d2 = vr[h][2][i], d3 = vr[h][3][i];
                const u32x2 lo{(d0 & 0xffffu) | (d1 << 16), (d2 & 0xffffu) | (d3 << 16)};
                const u32x2 hi{(d0 >> 16) | (d1 & 0xffff0000u), (d2 >> 16) | (d3 & 0xffff0000u)};
                const int x = vx + 2 * i;
                *reinterpret_cast<u32x2*>(&vt[x][4 * kg]) = lo;
                *reinterpret_cast<u32x2*>(&vt[x + 1][4 * kg]) = hi;
            }
        }
        after_stage();

        // S^T = K Q^T
        floatx4 sc[2][NRT];
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
            for (int rt = 0; rt < NRT; ++rt) {
                floatx4 a = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int k = 0; k < NS; ++k)
                    a = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(kf[kt][k]), qf[rt][k], a, 0, 0, 0);
                sc[kt][rt] = a;
            }
        after_s();

        // Scale to base 2, mask keys past the range (and hidden candidates),
        // tile max per row.
        bool grow = false;
        float alpha[NRT];
#pragma unroll
        for (int rt = 0; rt < NRT; ++rt) {
            float mx = -INFINITY;
#pragma unroll
            for (int kt = 0; kt < 2; ++kt)
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int key = 16 * kt + 4 * q4 + j;
                    const bool seen = key < valid && (!masked || ((vis[rt] >> key) & 1u));
                    const float v = seen ? sc[kt][rt][j] * c : -INFINITY;
                    sc[kt][rt][j] = v;
                    mx = fmaxf(mx, v);
                }
            mx = group4_max(mx);
            const float m_new = fmaxf(m_run[rt], mx);
            alpha[rt] = (m_run[rt] == -INFINITY) ? 0.f : exp2_hw(m_run[rt] - m_new);
            grow |= m_new > m_run[rt];
            m_run[rt] = m_new;
        }
        if (__ballot(grow)) {
#pragma unroll
            for (int rt = 0; rt < NRT; ++rt) {
                l_run[rt] *= alpha[rt];
                if constexpr (STATS) bl[rt] *= alpha[rt];
#pragma unroll
                for (int xt = 0; xt < NXT; ++xt) o[xt][rt] *= alpha[rt];
            }
        }

        // P = 2^(S - m) as two bf16 operands of the P V product, the rounded
        // weight and its rounding remainder: with the weight alone a row that
        // a few keys dominate (a short history, the candidate tile) would
        // feel the 2^-8 rounding at full strength. The matrix cores are
        // mostly idle in this HBM-bound kernel, so the second product costs
        // no time. l sums the same two parts.
        bf16x8 pf[NRT], pr[NRT];
#pragma unroll
        for (int rt = 0; rt < NRT; ++rt) {
            float ls = 0.f;
#pragma unroll
            for (int kt = 0; kt < 2; ++kt)
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const float pv = exp2_hw(sc[kt][rt][j] - m_run[rt]);
                    const __bf16 pb = (__bf16)pv;
                    const __bf16 rb = (__bf16)(pv - (float)pb);
                    pf[rt][4 * kt + j] = pb;
                    pr[rt][4 * kt + j] = rb;
                    ls += (float)pb + (float)rb;
                }
            l_run[rt] += ls;
            if constexpr (STATS) bl[rt] += masked ? 0.f : ls;
        }

        wave_sync();
        // O^T += V^T P^T: lane reads keys 4*q4..+3 and 16+4*q4..+3 of row x.
#pragma unroll
        for (int xt = 0; xt < NXT; ++xt) {
            const uint16_t* row = vt[16 * xt + l16];
            const u32x2 lo = *reinterpret_cast<const u32x2*>(row + 4 * q4);
            const u32x2 hi = *reinterpret_cast<const u32x2*>(row + 16 + 4 * q4);
            const bf16x8 a = as_bf16x8(u32x4{lo.x, lo.y, hi.x, hi.y});
#pragma unroll
            for (int rt = 0; rt < NRT; ++rt) {
                o[xt][rt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, pf[rt], o[xt][rt], 0, 0, 0);
                o[xt][rt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, pr[rt], o[xt][rt], 0, 0, 0);
            }
        }
        wave_sync();
    };

    const uint32_t no_vis[NRT] = {};
    u32x4 kf[2][NS], vr[VH][4];
    int tau = w;
    if constexpr (!kGather) {
        const int64_t t0 = tl.t0;
        if (tau < n_tiles) {
            load_k(tl.tk(tau), tl.valid(tau), kf);
            load_v(tl.tk(tau), tl.valid(tau), vr);
        }
        for (; tau < n_tiles; tau += kWaves) {
            const int64_t tk = t0 + (int64_t)kTile * tau;
            // Prefetch the wave's next tile into the registers just consumed:
            // V right away (staged), K once the S^T products have read it.
            const int nxt = tau + kWaves;
            const bool more = nxt < n_tiles;
            // Block statistics: a wave steps kTile * kWaves tokens, so at most
            // one block ends per step; the finished one is written out once V
            // is staged (bl and m_run still hold it), before the V prefetch.
            int64_t done_blk = -1;
            if constexpr (STATS) {
                if (tk >= blk_end) {
                    if (blk_cur >= 0) {
                        done_blk = blk_cur;
                        ++blk_cur;
                    } else {
                        blk_cur = tk / p.stats_block;
                    }
                    blk_end = (blk_cur + 1) * p.stats_block;
                }
            }
            consume(kf, vr, tl.valid(tau), false, no_vis,
                    [&] {
                        if constexpr (STATS) {
                            if (done_blk >= 0) {
                                flush_block(done_blk);
#pragma unroll
                                for (int rt = 0; rt < NRT; ++rt) bl[rt] = 0.f;
                            }
                        }
                        if (more) load_v(tl.tk(nxt), tl.valid(nxt), vr);
                    },
                    [&] { if (more) load_k(tl.tk(nxt), tl.valid(nxt), kf); });
        }
    } else {
        // Gathered chunks: tiles without keys are neither loaded nor
        // attended (nothing is read outside the listed chunks).
        int v_cur = 0;
        int64_t tk_cur = 0;
        if (tau < n_tiles) tl.tile(tau, &tk_cur, &v_cur);
        if (v_cur > 0) {
            load_k(tk_cur, v_cur, kf);
            load_v(tk_cur, v_cur, vr);
        }
        for (; tau < n_tiles; tau += kWaves) {
            const int nxt = tau + kWaves;
            int v_nxt = 0;
            int64_t tk_nxt = 0;
            if (nxt < n_tiles) tl.tile(nxt, &tk_nxt, &v_nxt);
            if (v_cur > 0) {
                consume(kf, vr, v_cur, false, no_vis, [&] { if (v_nxt > 0) load_v(tk_nxt, v_nxt, vr); },
                        [&] { if (v_nxt > 0) load_k(tk_nxt, v_nxt, kf); });
            } else if (v_nxt > 0) {
                load_v(tk_nxt, v_nxt, vr);
                load_k(tk_nxt, v_nxt, kf);
            }
            v_cur = v_nxt;
        }
    }

    if constexpr (STATS) {
        if (blk_cur >= 0) flush_block(blk_cur);
    }

    // The candidate region (section 4.2: the GPU-resident rows under each
    // query's mask) as one more masked tile of wave 0: n_queries <= 32 keys.
    if (cand && w == 0) {
        const int n = p.n_queries;
        const uint64_t bits = p.parents ? wave_tree_bits(p.parents + (int64_t)at.b() * n, n, lane) : chain_bits(lane);
        if (lane < n) sm.cbits[lane] = bits;
        wave_sync();
        if (p.mask_out && at.g() == 0 && lane < n) p.mask_out[(int64_t)at.b() * n + lane] = bits;
        uint32_t vis[NRT];
#pragma unroll
        for (int rt = 0; rt < NRT; ++rt) {
            const int r = l16 + 16 * rt;
            vis[rt] = r < p.rows ? (uint32_t)sm.cbits[r / p.group] : ~0u;  // padded rows see all (discarded)
        }
        const int64_t cbase = (p.c_req_offset ? p.c_req_offset[at.b()] : (int64_t)at.b() * p.c_stride_b) +
                              (int64_t)at.g() * p.c_stride_h;
        load_k_at(static_cast<const uint16_t*>(p.ck) + cbase, (int)p.c_stride_t, n - 1, kf);
        load_v_at(static_cast<const uint16_t*>(p.cv) + cbase, (int)p.c_stride_t, n - 1, vr);
        consume(kf, vr, n, true, vis, [] {}, [] {});
    }

    // Full row sums: the 4 lane groups hold disjoint keys of the same rows.
#pragma unroll
    for (int rt = 0; rt < NRT; ++rt) {
        l_run[rt] = group4_sum(l_run[rt]);
    }

    // Merge the waves' states (Eq. 8) through LDS, the work split by feature
    // tiles: every wave publishes its (m, l) and the accumulator tiles that
    // other waves own, then folds the four partial states of its own tiles
    // and writes them; wave 0 also writes m and l.
    static_assert(NXT % kWaves == 0, "feature tiles split evenly over the waves");
    constexpr int kOwnTile = NRT * 4;  // floats per lane of one owned feature tile
    __syncthreads();  // every wave is done with the V staging area
    if (q4 == 0) {
#pragma unroll
        for (int rt = 0; rt < NRT; ++rt) {
            sm.u.mg.m[w][l16 + 16 * rt] = m_run[rt];
            sm.u.mg.l[w][l16 + 16 * rt] = l_run[rt];
        }
    }
#pragma unroll
    for (int xt = 0; xt < NXT; ++xt) {
        const int owner = xt % kWaves;
        if (owner == w) continue;
        const int slot = w < owner ? w : w - 1;
#pragma unroll
        for (int rt = 0; rt < NRT; ++rt)
#pragma unroll
            for (int j = 0; j < 4; ++j) sm.u.mg.acc[owner][slot][(xt / kWaves) * kOwnTile + rt * 4 + j][lane] = o[xt][rt][j];
    }
    __syncthreads();
    float a[kWaves][NRT];  // weight of each wave's partial state in the merged one
#pragma unroll
    for (int rt = 0; rt < NRT; ++rt) {
        float mw[kWaves], m_tot = -INFINITY;
#pragma unroll
        for (int ww = 0; ww < kWaves; ++ww) {
            mw[ww] = sm.u.mg.m[ww][l16 + 16 * rt];
            m_tot = fmaxf(m_tot, mw[ww]);
        }
        float l_tot = 0.f;
#pragma unroll
        for (int ww = 0; ww < kWaves; ++ww) {
            a[ww][rt] = (mw[ww] == -INFINITY) ? 0.f : exp2_hw(mw[ww] - m_tot);
            l_tot += a[ww][rt] * sm.u.mg.l[ww][l16 + 16 * rt];
        }
        m_run[rt] = m_tot;
        l_run[rt] = l_tot;
    }
#pragma unroll
    for (int rt = 0; rt < NRT; ++rt) {
        const int r = l16 + 16 * rt;
        if (r >= p.rows) continue;
        const int i = r / p.group, h = at.g() * p.group + r % p.group;
        const int64_t row = (((int64_t)at.slot() * p.batch + at.b()) * p.n_queries + i) * p.n_q_heads + h;
        // One slot per stream in a whole-round call (fin_o): the merge of a
        // single state is O = acc / l, lse = m + ln l, written here with the
        // merge kernel's arithmetic instead of the slot.
        const int64_t orow = ((int64_t)at.b() * p.n_queries + i) * p.n_q_heads + h;
        const float m_nat = (m_run[rt] == -INFINITY) ? -INFINITY : m_run[rt] * kLn2;
        const bool seen = m_nat != -INFINITY && l_run[rt] > 0.f;
        if (w == 0 && q4 == 0) {
            if (p.fin_o) {
                p.fin_lse[orow] = seen ? m_nat + __builtin_amdgcn_logf(l_run[rt]) * kLn2 : -INFINITY;
            } else {
                p.m[row] = m_nat;
                p.l[row] = l_run[rt];
            }
        }
#pragma unroll
        for (int xt = 0; xt < NXT; ++xt) {
            if (xt % kWaves != w) continue;
            floatx4 v;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                float x = 0.f;
#pragma unroll
                for (int ww = 0; ww < kWaves; ++ww) {
                    const float part = ww == w ? o[xt][rt][j]
                                               : sm.u.mg.acc[w][ww < w ? ww : ww - 1][(xt / kWaves) * kOwnTile + rt * 4 + j][lane];
                    x += a[ww][rt] * part;
                }
                v[j] = x;
            }
            if (p.fin_o) {
#pragma unroll
                for (int j = 0; j < 4; ++j) v[j] = seen ? v[j] / l_run[rt] : 0.f;
                *reinterpret_cast<floatx4*>(p.fin_o + orow * D + 16 * xt + 4 * q4) = v;
            } else {
                *reinterpret_cast<floatx4*>(p.acc + row * D + 16 * xt + 4 * q4) = v;
            }
        }
    }
}

// Piece indices of the chunk kernel: from the work-group's position.
struct GridAt {
    const ChunkParams& p;
    // KV head fastest: the heads of one (slot, request) are dispatched
    // together, so with token-major layouts they stream the same rows.
    __device__ int g() const { return blockIdx.x % p.n_kv_heads; }
    __device__ int b() const { return blockIdx.z; }
    __device__ int slot() const { return p.slot_begin + (int)(blockIdx.x / p.n_kv_heads); }
};

// Piece indices of the history kernel: re-read from the LDS copy of the
// current piece at every use.
struct LdsAt {
    const ChunkParams& p;
    const volatile PlanPiece* pc;
    __device__ int g() const { return __builtin_amdgcn_readfirstlane(pc->g); }
    __device__ int b() const { return __builtin_amdgcn_readfirstlane(pc->b); }
    __device__ int slot() const { return p.slot_begin + max(__builtin_amdgcn_readfirstlane(pc->k), 0); }
};

template <int D, int NRT, bool STATS, bool GATHER>
__global__ __launch_bounds__(kThreads, 2) void chunk_mfma_kernel(ChunkParams p) {
    __shared__ MfmaSmem<D, NRT> sm;
    const int s = blockIdx.x / p.n_kv_heads;
    const int g = blockIdx.x % p.n_kv_heads;
    const int b = blockIdx.z;
    const int32_t len = chunk_view_len(p, b);
    if constexpr (GATHER) {
        // slot s: entries [s * cps, s * cps + cps) of (b, g)'s list, staged in
        // LDS (cps <= kMaxGatherPerSlot) so that reading them never waits on
        // the key loop's outstanding loads
        const int e0 = s * p.cps;
        const int ne = min(p.cps, p.n_sel - e0);
        if ((int)threadIdx.x < ne) sm.gidx[threadIdx.x] = p.chunk_idx[((int64_t)b * p.n_kv_heads + g) * p.n_sel + e0 + threadIdx.x];
        __syncthreads();
        const GatherTiles tl{sm.gidx, ne, p.chunk_len, len};
        mfma_piece<D, NRT, STATS>(p, sm, GridAt{p}, tl, p.with_cand && s == 0);
    } else {
        int64_t t0, t1;
        piece_tokens(p, len, b, g, s, &t0, &t1);
        mfma_piece<D, NRT, STATS>(p, sm, GridAt{p}, ContigTiles{t0, t1}, p.with_cand && s == 0);
    }
}

// The whole resident history of every request, cut into balanced pieces
// (the line split of plan_next) over gridDim.x work-groups.
template <int D, int NRT, bool STATS>
__global__ __launch_bounds__(kThreads, 2) void history_mfma_kernel(ChunkParams p) {
    __shared__ MfmaSmem<D, NRT> sm;
    const int64_t w = blockIdx.x;
    PlanStart st;
    if (!plan_start(p, w, st)) return;
    const int64_t total = st.total, piece_len = st.piece_len;

    // The walk runs on one lane with its cursor in LDS, so nothing of it is
    // held in registers across a piece.
    __shared__ PlanCursor cursor;
    __shared__ PlanPiece piece;
    __shared__ int32_t has_piece;
    if (threadIdx.x == 0) cursor = st.cursor;
    for (;;) {
        __syncthreads();  // the previous piece is done with LDS; the cursor is visible
        if (threadIdx.x == 0)
            has_piece = plan_step(p.req_len, p.max_len, p.batch, p.n_kv_heads, piece_len, total, p.plan_slots, w,
                                  &cursor, const_cast<PlanPiece*>(&piece), p.plan_align);
        __syncthreads();
        if (!__builtin_amdgcn_readfirstlane(has_piece)) break;
        // Re-read the arguments for every piece: held across the loop they
        // would take scalar registers the key loop needs. (The host pass
        // only checks this body; the kernarg segment exists on the device.)
#if defined(__HIP_DEVICE_COMPILE__)
        const __attribute__((address_space(4))) ChunkParams* args =
            (const __attribute__((address_space(4))) ChunkParams*)__builtin_amdgcn_kernarg_segment_ptr();
        asm volatile("" : "+s"(args));
        const ChunkParams pa = *args;
#else
        const ChunkParams& pa = p;
#endif
        const volatile PlanPiece* pc = &piece;
        const int32_t k = __builtin_amdgcn_readfirstlane(pc->k);
        if (k >= pa.plan_slots) break;  // cannot happen with plan_piece_len; never write past the slots
        // The candidate region joins each stream's first piece; a stream
        // without history gets it alone in slot 0 (t0 = t1 = 0).
        const bool cand = pa.with_cand && k <= 0;
        // Slots without a piece keep the empty states written before the
        // launch (a separate fill: stores here, behind the key loop's reads,
        // cost several times their bytes).
        if (k >= 0 || cand)
            mfma_piece<D, NRT, STATS>(pa, sm, LdsAt{pa, pc}, ContigTiles{uniform64(pc->t0), uniform64(pc->t1)}, cand);
    }
}

template <int D, int NRT>
hipError_t launch_t(const ChunkParams& p, hipStream_t stream) {
    const int64_t gx = (int64_t)p.n_items * p.n_kv_heads;
    if (gx > 0x7fffffff) return hipErrorInvalidValue;
    dim3 grid((unsigned)gx, 1, p.batch);
    if (p.stats)
        hipLaunchKernelGGL((chunk_mfma_kernel<D, NRT, true, false>), grid, dim3(kThreads), 0, stream, p);
    else if (p.chunk_idx && p.cps > 1)
        hipLaunchKernelGGL((chunk_mfma_kernel<D, NRT, false, true>), grid, dim3(kThreads), 0, stream, p);
    else
        hipLaunchKernelGGL((chunk_mfma_kernel<D, NRT, false, false>), grid, dim3(kThreads), 0, stream, p);
    return hipGetLastError();
}

// Work-groups of one history launch: one per CU, queried once per device.
// A CU could hold two of these 4-wave work-groups, but the SIMD arbiter
// favours the older one: it finishes its range early and leaves the other
// streaming alone, so the launch ends later than with one work-group (one
// wave per SIMD) per CU over twice the range.
constexpr int kMaxDevices = 64;

template <int D, int NRT>
hipError_t wave_wgs_t(int* out) {
    static int wave_wgs[kMaxDevices];
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    int n = __atomic_load_n(&wave_wgs[dev], __ATOMIC_RELAXED);
    if (n <= 0) {
        int cus = 0;
        e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
        if (e != hipSuccess) return e;
        n = cus > 0 ? cus : 1;
        __atomic_store_n(&wave_wgs[dev], n, __ATOMIC_RELAXED);
    }
    *out = n;
    return hipSuccess;
}

template <int D, int NRT>
hipError_t launch_hist_t(const ChunkParams& p, hipStream_t stream) {
    int n = 0;
    hipError_t e = wave_wgs_t<D, NRT>(&n);
    if (e != hipSuccess) return e;
    if (p.stats)
        hipLaunchKernelGGL((history_mfma_kernel<D, NRT, true>), dim3(n), dim3(kThreads), 0, stream, p);
    else
        hipLaunchKernelGGL((history_mfma_kernel<D, NRT, false>), dim3(n), dim3(kThreads), 0, stream, p);
    return hipGetLastError();
}

}  // namespace

// head_dim 128 or 64 (the V staging map gives each lane 8 features of one
// or two key groups), up to 32 rows.
hipError_t launch_chunk_mfma(const ChunkParams& p, int head_dim, hipStream_t stream) {
    if ((head_dim != 128 && head_dim != 64) || p.rows > 32) return hipErrorInvalidValue;
    if (head_dim == 64) return p.rows > 16 ? launch_t<64, 2>(p, stream) : launch_t<64, 1>(p, stream);
    return p.rows > 16 ? launch_t<128, 2>(p, stream) : launch_t<128, 1>(p, stream);
}

hipError_t mfma_wave_work_groups(int rows, int* n) {
    if (rows > 32) return hipErrorInvalidValue;
    return rows > 16 ? wave_wgs_t<128, 2>(n) : wave_wgs_t<128, 1>(n);
}

hipError_t launch_history_mfma(const ChunkParams& p, int head_dim, hipStream_t stream) {
    if ((head_dim != 128 && head_dim != 64) || p.rows > 32 || p.plan_slots < 2) return hipErrorInvalidValue;
    if (head_dim == 64) return p.rows > 16 ? launch_hist_t<64, 2>(p, stream) : launch_hist_t<64, 1>(p, stream);
    return p.rows > 16 ? launch_hist_t<128, 2>(p, stream) : launch_hist_t<128, 1>(p, stream);
}

}  // namespace ssv
