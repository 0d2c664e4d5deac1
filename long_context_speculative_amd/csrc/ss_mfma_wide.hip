// MFMA bf16 chunk kernel of libssverify for wide row groups (more than 32
// rows per KV head, e.g. a 64-node candidate tree under 8-way GQA: 512 rows),
// head_dim 128 or 64.
//
// SpecStream ("Resource-Efficient Speculative Decoding for Long-Context LLM
// Serving"), section 4.2: one history chunk serves the whole query group; its
// local state (Eq. 7) is merged tile by tile (Eq. 8).
//
// With hundreds of rows per KV head the work is bound by the matrix cores and
// the softmax arithmetic, not by HBM: every key feeds 512 rows. Layout:
//   - a work-group of NW waves owns 32*NW rows; each wave holds 32 rows (two
//     16-row MFMA tiles) with its Q^T fragments and O^T accumulator in
//     registers, small enough for two waves per SIMD, so one wave's softmax
//     overlaps the other's matrix work;
//   - key tiles of KT (32, or 64 for groups of eight waves) are copied once
//     per work-group into LDS, K and V both in their natural [key][feature]
//     layout (rows padded; see kRow and kVRow), in a ring
//     of three buffers, loads issued three tiles ahead; a 64-key tile halves
//     the barriers and row-maximum reductions per key (about 5% on a 512-row
//     group) at 105 KB of LDS, which one eight-wave group per CU affords;
//   - the loop is software-pipelined: the S products of tile t+1 are issued
//     next to the softmax and P V of tile t, so matrix and vector work of one
//     wave overlap, on top of the two waves per SIMD;
//   - S^T = K Q^T reads K fragments with 16-byte LDS reads; O^T = V^T P^T
//     reads V^T fragments with the transposing LDS read ds_read_b64_tr_b16;
//   - l (the softmax denominator) comes out of the same MFMA as O^T through
//     an all-ones A operand, so it sums exactly the bf16 weights that enter
//     the numerator; for a request with a short history, and for the
//     candidate tiles, a second pass adds each weight's bf16 rounding
//     remainder to both, so rows that a few keys dominate stay exact to
//     about 2^-16;
//   - the score scale is folded into the exponent (one FMA per score), and the
//     running maximum is moved only when a row's maximum grows by more than
//     2^8 over it (weights then stay <= 256; the rescale is rare);
//   - row groups beyond the first re-read the chunk; all row groups of one
//     (slot, KV head, request) are placed on the same XCD (work-group ids 8
//     apart, dispatched back to back) so the re-read hits that XCD's L2, and
//     eight consecutive (slot, KV head) units spread over the eight XCDs.

#include <type_traits>

#include "ss_common.h"

namespace ssv {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef short s16x4 __attribute__((ext_vector_type(4)));

constexpr int kTile = 32;       // keys per MFMA sub-tile (KT keys per iteration)
constexpr float kGrowLog2 = 8.f;  // rescale threshold (log2 units)
// A piece attended without the weights' rounding remainders is attended again
// with them when some row's largest weight exceeds this share of its sum.
constexpr float kShareMax = 1.f / 32.f;

// Row pitches of the staged tiles (head_dim D = 128 or 64). At D = 128 the
// transposing V reads are free of bank conflicts at a 32-byte pad, and so
// are the 16-byte K fragment reads; at the 16-byte K pad used here those
// spend about a third of their LDS cycles in conflicts, yet the
// conflict-free pitch is slower on MI355X: the launch is held by the chip's
// power limit, and with the stall cycles gone it runs at a lower clock
// (fewer cycles, longer time).
template <int D>
struct WideDims {
    static constexpr int kRow = D + 8;     // bf16 per staged K row (16-byte pad)
    static constexpr int kVRow = D + 16;   // bf16 per staged V row (32-byte pad)
    static constexpr int kNS = D / 32;     // 32-feature steps of S = K Q^T
    static constexpr int kNXT = D / 16;    // 16-feature tiles of O^T
    static constexpr int kRowPieces = D / 8;  // 16-byte pieces per key row
};

// 16-byte aligned so that the 16-byte staging stores and K reads are single
// ds_write_b128 / ds_read_b128 (with only the 8-byte alignment of the
// member types the compiler splits them into pairs of 8-byte accesses).
template <int D, int KT>
struct alignas(16) WideSmem {
    uint16_t k[3][KT][WideDims<D>::kRow];
    uint16_t v[3][KT][WideDims<D>::kVRow];
    uint64_t cbits[64];  // candidate visibility bits (n_queries <= 64)
    int32_t again;       // some wave needs the piece attended again
};

__device__ __forceinline__ float exp2_hw(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

__device__ __forceinline__ s16x4 lds_read_tr(const uint16_t* p) {
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) s16x4*)(reinterpret_cast<uintptr_t>(p)));
}

// FIN: one slot per stream in a whole-round call, the rows finished into
// p.fin_o / p.fin_lse instead of the slot (a variant of its own: at 256
// registers the plain kernel has no room for the other epilogue).
template <int D, int NW, int kRT, int KT, bool FIN>
__global__ __launch_bounds__(64 * NW, (kRT == 2 && KT == 32) ? 2 : 1) void chunk_mfma_wide_kernel(ChunkParams p, int row_groups) {
    constexpr int kVRow = WideDims<D>::kVRow;
    constexpr int kNS = WideDims<D>::kNS, kNXT = WideDims<D>::kNXT, kRP = WideDims<D>::kRowPieces;
    static_assert(D == 64 || D == 128, "head_dim 64 or 128");
    static_assert(KT % kTile == 0, "an iteration is whole sub-tiles");
    constexpr int kSub = KT / kTile;           // 32-key sub-tiles per iteration
    constexpr int kKB = 2 * kSub;              // 16-key blocks per iteration
    constexpr int T = 64 * NW;
    constexpr int kPieces = KT * (D / 8);      // 16-byte pieces per K (or V) tile
    constexpr int kPer = kPieces / T;          // pieces of K and of V per thread
    static_assert(kPieces % T == 0, "tile pieces must divide evenly");
    __shared__ WideSmem<D, KT> sm;

    // Work-group -> (unit u = (slot, KV head), row group): eight consecutive
    // units go to the eight XCDs (dispatch is round-robin over them), and the
    // row groups of one unit are 8 ids apart, so they share that XCD's L2.
    const int x = blockIdx.x;
    const int x_hi = x / (8 * row_groups), rem = x % (8 * row_groups);
    const int rg = rem / 8;
    const int u = x_hi * 8 + rem % 8;
    if (u >= p.n_items * p.n_kv_heads) return;
    const int s = u % p.n_items;
    const int g = u / p.n_items;
    const int b = blockIdx.z;
    const int tid = threadIdx.x;
    const int lane = tid & 63, w = tid >> 6;
    const int l16 = lane & 15, q4 = lane >> 4;

    const int32_t len = chunk_view_len(p, b);
    int64_t t0, t1;
    piece_tokens(p, len, b, g, s, &t0, &t1);

    const int64_t base = (p.req_offset ? p.req_offset[b] : (int64_t)b * p.stride_b) + (int64_t)g * p.stride_h;
    const uint16_t* __restrict__ kp = static_cast<const uint16_t*>(p.k) + base;
    const uint16_t* __restrict__ vp = static_cast<const uint16_t*>(p.v) + base;
    const int64_t st = p.stride_t;
    const int sti = (int)st;

    constexpr int kWaveRows = 16 * kRT;
    const int row0 = rg * kWaveRows * NW + kWaveRows * w;  // first row of this wave
    const bool active = row0 < p.rows;

    bf16x8 qf[kRT][kNS];
#pragma unroll
    for (int rt = 0; rt < kRT; ++rt) {
        const int r = row0 + 16 * rt + l16;
        if (r < p.rows) {
            const int i = r / p.group, h = g * p.group + r % p.group;
            const uint16_t* qrow = static_cast<const uint16_t*>(p.q) + ((int64_t)(b * p.n_queries + i) * p.n_q_heads + h) * D;
#pragma unroll
            for (int k = 0; k < kNS; ++k) qf[rt][k] = as_bf16x8(*reinterpret_cast<const u32x4*>(qrow + 32 * k + 8 * q4));
        } else {
#pragma unroll
            for (int k = 0; k < kNS; ++k) qf[rt][k] = as_bf16x8(u32x4{0u, 0u, 0u, 0u});
        }
    }

    floatx4 o[kNXT][kRT], ol[kRT];  // O^T accumulators and the row-sum tile
#pragma unroll
    for (int rt = 0; rt < kRT; ++rt) {
        ol[rt] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int xt = 0; xt < kNXT; ++xt) o[xt][rt] = floatx4{0.f, 0.f, 0.f, 0.f};
    }
    float m_run[kRT];  // reference maximum of c-scaled (log2) scores per row
#pragma unroll
    for (int rt = 0; rt < kRT; ++rt) m_run[rt] = -INFINITY;
    const float c = p.scale * kLog2e;
    const bf16x8 ones = as_bf16x8(u32x4{0x3f803f80u, 0x3f803f80u, 0x3f803f80u, 0x3f803f80u});
    const int n_tiles = (int)((t1 - t0 + KT - 1) / KT);

    // Staging: thread tid copies K and V pieces u = tid + j*T (key u / kRP,
    // features 8*(u % kRP) .. +7). Keys past the range are clamped to its last
    // key (finite values; their scores are masked).
    u32x4 pa[2][kPer], pb[2][kPer];
    auto fetch = [&](int64_t tk, u32x4(&pre)[2][kPer]) __attribute__((always_inline)) {
        const int last = (int)min((int64_t)KT, t1 - tk) - 1;
        const uint16_t* kb = kp + tk * st;
        const uint16_t* vb = vp + tk * st;
#pragma unroll
        for (int j = 0; j < kPer; ++j) {
            const int u = tid + j * T;
            const int off = min(u / kRP, last) * sti + 8 * (u % kRP);
            pre[0][j] = *reinterpret_cast<const u32x4*>(kb + off);
            pre[1][j] = *reinterpret_cast<const u32x4*>(vb + off);
        }
    };
    auto stage = [&](int buf, const u32x4(&pre)[2][kPer]) __attribute__((always_inline)) {
#pragma unroll
        for (int j = 0; j < kPer; ++j) {
            const int u = tid + j * T;
            *reinterpret_cast<u32x4*>(&sm.k[buf][u / kRP][8 * (u % kRP)]) = pre[0][j];
            *reinterpret_cast<u32x4*>(&sm.v[buf][u / kRP][8 * (u % kRP)]) = pre[1][j];
        }
    };

    // S^T = K Q^T (raw dot products) of the tile in LDS buffer buf.
    auto qk = [&](const int buf, const int /*t*/, floatx4(&sc)[kKB][kRT]) __attribute__((always_inline)) {
#pragma unroll
        for (int kt = 0; kt < kKB; ++kt)
#pragma unroll
            for (int rt = 0; rt < kRT; ++rt) sc[kt][rt] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int k = 0; k < kNS; ++k)
#pragma unroll
            for (int kt = 0; kt < kKB; ++kt) {
                const bf16x8 a = as_bf16x8(*reinterpret_cast<const u32x4*>(&sm.k[buf][16 * kt + l16][32 * k + 8 * q4]));
#pragma unroll
                for (int rt = 0; rt < kRT; ++rt)
                    sc[kt][rt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, qf[rt][k], sc[kt][rt], 0, 0, 0);
            }
    };
    // Row maxima of a tile, in c-scaled log2 units (c > 0, so the max of raw
    // scores picks the max of scaled ones).
    auto row_max = [&](const floatx4(&sc)[kKB][kRT], float(&mc)[kRT]) __attribute__((always_inline)) {
#pragma unroll
        for (int rt = 0; rt < kRT; ++rt) {
            float mx = -INFINITY;
#pragma unroll
            for (int kt = 0; kt < kKB; kt += 2)
                mx = fmaxf(mx, fmaxf(fmaxf(fmaxf(sc[kt][rt][0], sc[kt][rt][1]), fmaxf(sc[kt][rt][2], sc[kt][rt][3])),
                                     fmaxf(fmaxf(sc[kt + 1][rt][0], sc[kt + 1][rt][1]),
                                           fmaxf(sc[kt + 1][rt][2], sc[kt + 1][rt][3]))));
            mx = group4_max(mx);
            mc[rt] = mx * c;
        }
    };
    // Moves the reference maximum when some row's tile maximum exceeds it by
    // more than 2^8, rescaling the accumulated state (Eq. 8).
    auto rescale = [&](const float(&mc)[kRT]) __attribute__((always_inline)) {
        bool grow = false;
#pragma unroll
        for (int rt = 0; rt < kRT; ++rt) grow |= mc[rt] > m_run[rt] + kGrowLog2;
        if (__ballot(grow)) {
#pragma unroll
            for (int rt = 0; rt < kRT; ++rt) {
                const float m_new = fmaxf(m_run[rt], mc[rt]);
                const float alpha = (m_run[rt] == -INFINITY) ? 0.f : exp2_hw(m_run[rt] - m_new);
                m_run[rt] = m_new;
                ol[rt] *= alpha;
#pragma unroll
                for (int xt = 0; xt < kNXT; ++xt) o[xt][rt] *= alpha;
            }
        }
    };
    // Per 32-key sub-tile su: P = 2^(c*S - m) in bf16 (slot j of a lane =
    // key 32*su + 4*q4 + j, slot 4 + j = key 32*su + 16 + 4*q4 + j), then
    // O^T += V^T P^T and l += 1^T P^T from LDS buffer buf. For the
    // transposing read, lane (group q4, index l16) points at features
    // 16*xt + 4*(l16 % 4) .. +3 of key 32*su + 4*q4 + l16 / 4 (and of key
    // 32*su + 16 + ...); it receives feature 16*xt + l16 of keys
    // 32*su + 4*q4 .. +3 (and 32*su + 16 + 4*q4 .. +3): the keys of the P
    // slots it holds.
    // kLo: the same products with each weight's bf16 rounding remainder
    // (the weights are recomputed, so the split path needs no more registers
    // than the plain one).
    auto pv_pass = [&](auto lo, const int buf, const floatx4(&sc)[kKB][kRT]) __attribute__((always_inline)) {
        constexpr bool kLo = decltype(lo)::value;
#pragma unroll
        for (int su = 0; su < kSub; ++su) {  // 32-key sub-tiles
            bf16x8 pf[kRT];
#pragma unroll
            for (int rt = 0; rt < kRT; ++rt) {
                const float nm = -m_run[rt];
#pragma unroll
                for (int kt = 0; kt < 2; ++kt)
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        float x = sc[2 * su + kt][rt][j];
                        // the second pass recomputes its weights instead of
                        // keeping the first pass's alive across its products
                        if constexpr (kLo) asm volatile("" : "+v"(x));
                        const float pv = exp2_hw(fmaf(x, c, nm));
                        if constexpr (kLo)
                            pf[rt][4 * kt + j] = (__bf16)(pv - (float)(__bf16)pv);
                        else
                            pf[rt][4 * kt + j] = (__bf16)pv;
                    }
            }
            const uint16_t* vrow0 = &sm.v[buf][kTile * su + 4 * q4 + (l16 >> 2)][4 * (l16 & 3)];
            const uint16_t* vrow1 = vrow0 + 16 * kVRow;
#pragma unroll
            for (int rt = 0; rt < kRT; ++rt)
                ol[rt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ones, pf[rt], ol[rt], 0, 0, 0);
#pragma unroll
            for (int xt = 0; xt < kNXT; ++xt) {
                const s16x4 lo = lds_read_tr(vrow0 + 16 * xt);
                const s16x4 hi = lds_read_tr(vrow1 + 16 * xt);
                const bf16x8 a = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
#pragma unroll
                for (int rt = 0; rt < kRT; ++rt)
                    o[xt][rt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, pf[rt], o[xt][rt], 0, 0, 0);
            }
        }
    };
    auto softmax_pv = [&](auto split, const int buf, const floatx4(&sc)[kKB][kRT]) __attribute__((always_inline)) {
        pv_pass(std::false_type{}, buf, sc);
        if constexpr (decltype(split)::value) pv_pass(std::true_type{}, buf, sc);
    };

    // Software pipeline over the key tiles. Tiles 0 .. n_full-1 hold KT keys;
    // a last partial tile (the tail) is handled after the loop, so the loop
    // body needs no masking and has no branch: the scheduler can interleave
    // the S(t+1) products with the softmax of tile t.
    //
    // At the top of iteration t: LDS buffers t%3 and (t+1)%3 hold tiles t and
    // t+1, sc_cur holds S(t) with the reference maximum already covering it,
    // and one register set holds tile t+2 (loads in flight). Iteration t loads
    // tile t+3 into the other set, forms S(t+1), the softmax and P V of tile
    // t, the maxima of S(t+1), stages tile t+2, then (after the branch-free
    // part) moves the reference maximum for tile t+1. Tile indices past the
    // last tile are clamped to it: their loads and staging are harmless
    // (the buffer they land in is not read again).
    const int n_full = (int)((t1 - t0) / KT);
    const bool has_tail = (t1 - t0) % KT != 0;
    auto tile_start = [&](int t) { return t0 + (int64_t)KT * min(t, n_tiles - 1); };
    auto next_buf = [](int bi) { return bi == 2 ? 0 : bi + 1; };

    floatx4 sc_a[kKB][kRT], sc_b[kKB][kRT];
    float mc[kRT];
    // Masks the keys at or past `valid` of a tile's scores.
    auto mask_tail = [&](floatx4(&sc)[kKB][kRT], int valid) __attribute__((always_inline)) {
#pragma unroll
        for (int kt = 0; kt < kKB; ++kt)
#pragma unroll
            for (int rt = 0; rt < kRT; ++rt)
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    if (16 * kt + 4 * q4 + j >= valid) sc[kt][rt][j] = -INFINITY;
    };

    // The piece tile by tile without the pipeline, each weight's bf16
    // rounding remainder carried as a second operand (a second P V pass; a
    // second pipelined loop would not fit the registers).
    auto careful_pass = [&]() __attribute__((always_inline)) {
        for (int t = 0; t < n_tiles; ++t) {
            fetch(t0 + (int64_t)KT * t, pa);
            if (t > 0) __syncthreads();  // the previous tile is consumed
            stage(0, pa);
            __syncthreads();
            if (active) {
                qk(0, t, sc_a);
                mask_tail(sc_a, (int)min((int64_t)KT, t1 - t0 - (int64_t)KT * t));
                row_max(sc_a, mc);
                rescale(mc);
                softmax_pv(std::true_type{}, 0, sc_a);
            }
        }
    };

    // A request with a short history (row_history_keys below kSplitBelow)
    // takes the careful pass. A longer one takes the pipelined loop without
    // the remainders: a weight's rounding moves a row's result by up to
    // 2^-8 of that weight's share of the row's sum, and over many keys the
    // errors average out, unless a few keys dominate the row. So the loop
    // tracks each row's largest score, and where some row's largest weight
    // is more than kShareMax of its sum (the rounding error's spread is then
    // up to sqrt(kShareMax) of the single-weight one), the work-group attends
    // the piece again with the careful pass. The candidate tiles always
    // carry the remainders.
    if (row_history_keys(p, b) < kSplitBelow) {
        careful_pass();
    } else {
        float m_top[kRT];  // largest c-scaled score of each row so far
#pragma unroll
        for (int rt = 0; rt < kRT; ++rt) m_top[rt] = -INFINITY;
        auto track = [&]() __attribute__((always_inline)) {
#pragma unroll
            for (int rt = 0; rt < kRT; ++rt) m_top[rt] = fmaxf(m_top[rt], mc[rt]);
        };
        if (tid == 0) sm.again = 0;
        if (n_tiles > 0) {
            fetch(tile_start(0), pa);
            stage(0, pa);
            fetch(tile_start(1), pb);
            stage(1, pb);
            fetch(tile_start(2), pa);
        }
        __syncthreads();
        if (active && n_full > 0) {
            qk(0, 0, sc_a);
            row_max(sc_a, mc);
            track();
            rescale(mc);
        }

        // Main loop: iterations t = 0 .. n_full - 2, unrolled by two (register
        // sets pa / pb, score sets sc_a / sc_b alternate roles).
        auto step = [&](auto compute, int t, int b_cur, floatx4(&sc_cur)[kKB][kRT], floatx4(&sc_next)[kKB][kRT],
                        u32x4(&stage_set)[2][kPer], u32x4(&fetch_set)[2][kPer]) __attribute__((always_inline)) {
            const int b1 = next_buf(b_cur), b2 = next_buf(b1);
            fetch(tile_start(t + 3), fetch_set);
            if constexpr (decltype(compute)::value) {
                qk(b1, t + 1, sc_next);
                softmax_pv(std::false_type{}, b_cur, sc_cur);
                row_max(sc_next, mc);
                track();
            }
            stage(b2, stage_set);
            if constexpr (decltype(compute)::value) rescale(mc);
            __syncthreads();
        };
        auto main_loop = [&](auto compute) __attribute__((always_inline)) {
            int bi = 0;
            for (int t = 0; t + 1 < n_full; t += 2) {
                step(compute, t, bi, sc_a, sc_b, pa, pb);
                bi = next_buf(bi);
                if (t + 2 >= n_full) break;
                step(compute, t + 1, bi, sc_b, sc_a, pb, pa);
                bi = next_buf(bi);
            }
        };
        if (active)
            main_loop(std::true_type{});
        else
            main_loop(std::false_type{});

        if (active) {
            // Last full tile: S is in sc_a if n_full is odd, else in sc_b.
            if (n_full > 0) softmax_pv(std::false_type{}, (n_full - 1) % 3, (n_full & 1) ? sc_a : sc_b);
            // The tail tile (staged by the loop or the prologue), with masking.
            if (has_tail) {
                const int bt = n_full % 3;
                qk(bt, n_full, sc_a);
                mask_tail(sc_a, (int)(t1 - t0 - (int64_t)KT * n_full));
                row_max(sc_a, mc);
                track();
                rescale(mc);
                softmax_pv(std::false_type{}, bt, sc_a);
            }
        }
        bool big = false;
        if (active) {
#pragma unroll
            for (int rt = 0; rt < kRT; ++rt) big |= exp2_hw(m_top[rt] - m_run[rt]) > kShareMax * ol[rt][0];
        }
        if (__ballot(big) && lane == 0) atomicOr(&sm.again, 1);
        __syncthreads();  // every wave's verdict is in; the ring buffers are free
        if (__builtin_amdgcn_readfirstlane(sm.again)) {
#pragma unroll
            for (int rt = 0; rt < kRT; ++rt) {
                m_run[rt] = -INFINITY;
                ol[rt] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int xt = 0; xt < kNXT; ++xt) o[xt][rt] = floatx4{0.f, 0.f, 0.f, 0.f};
            }
            careful_pass();
        }
    }

    // The candidate region (section 4.2: the GPU-resident rows under each
    // query's mask), attended after the history by the work-groups of each
    // stream's first piece as masked key tiles (n_queries <= 64 keys). Every
    // wave stages; the uniform condition keeps the barriers uniform.
    if (p.with_cand && s == 0) {
        const int n = p.n_queries;
        if (w == 0) {
            const uint64_t bits = p.parents ? wave_tree_bits(p.parents + (int64_t)b * n, n, lane) : chain_bits(lane);
            if (lane < n) sm.cbits[lane] = bits;
            if (p.mask_out && g == 0 && rg == 0 && lane < n) p.mask_out[(int64_t)b * n + lane] = bits;
        }
        __syncthreads();  // every wave is done with the ring buffers
        const int64_t cbase =
            (p.c_req_offset ? p.c_req_offset[b] : (int64_t)b * p.c_stride_b) + (int64_t)g * p.c_stride_h;
        const uint16_t* ckp = static_cast<const uint16_t*>(p.ck) + cbase;
        const uint16_t* cvp = static_cast<const uint16_t*>(p.cv) + cbase;
        const int cst = (int)p.c_stride_t;
        for (int c0 = 0; c0 < n; c0 += KT) {
            const int last = min(KT, n - c0) - 1;  // rows past the region repeat its last one
#pragma unroll
            for (int j = 0; j < kPer; ++j) {
                const int u = tid + j * T;
                const int off = (c0 + min(u / kRP, last)) * cst + 8 * (u % kRP);
                pa[0][j] = *reinterpret_cast<const u32x4*>(ckp + off);
                pa[1][j] = *reinterpret_cast<const u32x4*>(cvp + off);
            }
            if (c0 > 0) __syncthreads();  // the previous candidate tile is consumed
            stage(0, pa);
            __syncthreads();  // the tile and the visibility bits are in LDS
            if (active) {
                qk(0, 0, sc_a);
#pragma unroll
                for (int rt = 0; rt < kRT; ++rt) {
                    const int r = row0 + 16 * rt + l16;
                    const uint64_t vis = r < p.rows ? sm.cbits[r / p.group] : ~(uint64_t)0;  // padded rows: discarded
#pragma unroll
                    for (int kt = 0; kt < kKB; ++kt)
#pragma unroll
                        for (int j = 0; j < 4; ++j) {
                            const int key = c0 + 16 * kt + 4 * q4 + j;
                            if (key >= n || !((vis >> key) & 1)) sc_a[kt][rt][j] = -INFINITY;
                        }
                }
                row_max(sc_a, mc);
                rescale(mc);
                // A row that has seen no key yet and sees none here keeps
                // the empty state: its weights are 0 against any reference,
                // so take 0 for this tile and restore -inf afterwards.
                bool none[kRT];
#pragma unroll
                for (int rt = 0; rt < kRT; ++rt) {
                    none[rt] = m_run[rt] == -INFINITY;
                    if (none[rt]) m_run[rt] = 0.f;
                }
                softmax_pv(std::true_type{}, 0, sc_a);
#pragma unroll
                for (int rt = 0; rt < kRT; ++rt)
                    if (none[rt]) m_run[rt] = -INFINITY;
            }
        }
    }

    if (!active) return;
#pragma unroll
    for (int rt = 0; rt < kRT; ++rt) {
        const int r = row0 + 16 * rt + l16;
        if (r >= p.rows) continue;
        const int i = r / p.group, h = g * p.group + r % p.group;
        const int64_t row = (((int64_t)(p.slot_begin + s) * p.batch + b) * p.n_queries + i) * p.n_q_heads + h;
        const float m_nat = (m_run[rt] == -INFINITY) ? -INFINITY : m_run[rt] * kLn2;
        const float lr = ol[rt][0];  // every lane holds its row's l
        // One slot per stream in a whole-round call (fin_o): the merge of a
        // single state, O = acc / l and lse = m + ln l, with the merge
        // kernel's arithmetic, written instead of the slot.
        constexpr bool fin = FIN;
        const int64_t orow = ((int64_t)b * p.n_queries + i) * p.n_q_heads + h;
        const bool seen = m_nat != -INFINITY && lr > 0.f;
        if (q4 == 0) {
            if constexpr (fin) {
                p.fin_lse[orow] = seen ? m_nat + __builtin_amdgcn_logf(lr) * kLn2 : -INFINITY;
            } else {
                p.m[row] = m_nat;
                p.l[row] = lr;
            }
        }
        float* dst = (fin ? p.fin_o + orow * D : p.acc + row * D) + 4 * q4;
#pragma unroll
        for (int xt = 0; xt < kNXT; ++xt) {
            floatx4 v = o[xt][rt];
            if constexpr (fin) {
#pragma unroll
                for (int j = 0; j < 4; ++j) v[j] = seen ? v[j] / lr : 0.f;
            }
            *reinterpret_cast<floatx4*>(dst + 16 * xt) = v;
        }
    }
}

template <int D, int NW, int kRT, int KT>
hipError_t launch_wide_t(const ChunkParams& p, hipStream_t stream) {
    const int row_groups = (p.rows + 16 * kRT * NW - 1) / (16 * kRT * NW);
    const int64_t units = (int64_t)p.n_items * p.n_kv_heads;
    const int64_t gx = (units + 7) / 8 * 8 * row_groups;
    if (gx > 0x7fffffff) return hipErrorInvalidValue;
    dim3 grid((unsigned)gx, 1, p.batch);
    if (p.fin_o)
        hipLaunchKernelGGL((chunk_mfma_wide_kernel<D, NW, kRT, KT, true>), grid, dim3(64 * NW), 0, stream, p, row_groups);
    else
        hipLaunchKernelGGL((chunk_mfma_wide_kernel<D, NW, kRT, KT, false>), grid, dim3(64 * NW), 0, stream, p, row_groups);
    return hipGetLastError();
}

template <int D>
hipError_t launch_wide_d(const ChunkParams& p, hipStream_t stream) {
    // 32 rows per wave: up to 128 rows in one group of four waves (32-key
    // tiles, two groups per CU), more rows in groups of eight waves (two per
    // SIMD, 64-key tiles, one group per CU).
    if (p.rows <= 128) return launch_wide_t<D, 4, 2, 32>(p, stream);
    return launch_wide_t<D, 8, 2, 64>(p, stream);
}

}  // namespace

hipError_t launch_chunk_mfma_wide(const ChunkParams& p, int head_dim, hipStream_t stream) {
    if (p.rows <= 32) return hipErrorInvalidValue;
    if (head_dim == 128) return launch_wide_d<128>(p, stream);
    if (head_dim == 64) return launch_wide_d<64>(p, stream);
    return hipErrorInvalidValue;
}

}  // namespace ssv
