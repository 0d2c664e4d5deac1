// fp32 MFMA chunk kernel of libssverify: fp32 inputs, head_dim 128 or 64; up
// to 32 rows per KV head in one work-group, more rows in row groups of 32.
//
// SpecStream ("Resource-Efficient Speculative Decoding for Long-Context LLM
// Serving"), section 4.2: a history chunk serves the whole verification query
// group. For one (slot, KV head, request) a work-group of 4 waves walks the
// slot's keys in tiles of 16; wave w takes tiles w, w+4, ... Every wave holds
// all R = n_queries * G rows of the KV head (padded to 16 or 32), so each K
// and V byte is read from HBM once and feeds every query and every head of
// the GQA group. Beyond 32 rows the fixed-chunk kernel runs one work-group
// per row group of 32 rows; the row groups of one piece sit 8 work-group ids
// apart, which the round-robin dispatch places on the same XCD, so all but
// the first read the piece from that XCD's L2.
//
// Per tile, with v_mfma_f32_16x16x4_f32 (A 16x4: lane l holds A[l%16][l/16];
// B 4x16: B[l/16][l%16]; C 16x16: lane l holds C[4*(l/16)+i][l%16]):
//   S^T[key][row] = K Q^T     the contraction runs over the features in a
//                             permuted order: at step (u, c) lane group j
//                             supplies feature 16u + 4j + c, so one 16-byte
//                             load per lane and u (features 16u + 4j .. +3 of
//                             its key) has the 4 lane groups reading 64
//                             adjacent bytes of each key row; the query rows
//                             are held in the same order
//   online softmax (Eq. 7-8)  base 2, fp32 weights; the row max needs one
//                             exchange across the 4 lane groups
//   O^T[x][row] += V^T P^T    B = P straight from the S^T output (step i:
//                             lane group j gives key 4j+i), A = V^T read from
//                             a per-wave LDS tile of V in [key][feature]
//                             order
// The 4 waves' states are merged with Eq. (8) through LDS at the end and
// written as the slot's state (m in natural-log units).

#include "ss_common.h"

namespace ssv {
namespace {

typedef float floatx4 __attribute__((ext_vector_type(4)));

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kTile = 16;  // keys per wave iteration

template <int D, int NRT>
struct F32Smem {
    // V rows padded by 4 floats: the P V reads of the 4 lane groups (keys
    // 4j+i, 16 consecutive features each) then fall into distinct banks.
    static constexpr int kVPitch = D + 4;
    // Accumulator floats per lane of the feature tiles one wave owns in the
    // final merge (wave w owns the 16-feature tiles xt with xt % kWaves == w).
    static constexpr int kOwnRegs = (D / 16 / kWaves) * NRT * 4;
    union alignas(16) {
        float vt[kWaves][kTile][kVPitch];
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

// State of tokens [t0, t1) of stream (b, g) for rows r0 .. r0 + 16*NRT - 1
// of the KV head (those below p.rows), written to slot `slot` of the state
// buffer.
template <int D, int NRT>
__device__ __forceinline__ void f32_piece(const ChunkParams& p, F32Smem<D, NRT>& sm, int b, int g, int slot,
                                          int64_t t0, int64_t t1, int r0) {
    constexpr int NF = D / 4;    // features per lane group (the contraction's steps for S)
    constexpr int NXT = D / 16;  // 16-feature output tiles for O^T
    static_assert(NXT % kWaves == 0, "feature tiles split evenly over the waves");
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int l16 = lane & 15, q4 = lane >> 4;

    const int64_t base = (p.req_offset ? p.req_offset[b] : (int64_t)b * p.stride_b) + (int64_t)g * p.stride_h;
    const float* __restrict__ kp = static_cast<const float*>(p.k) + base;
    const float* __restrict__ vp = static_cast<const float*>(p.v) + base;
    const int64_t st = p.stride_t;

    // Q^T operand: row r = r0 + l16 + 16*rt, features 16u + 4*q4 .. +3 for u < NF/4.
    float qf[NRT][NF];
#pragma unroll
    for (int rt = 0; rt < NRT; ++rt) {
        const int r = r0 + l16 + 16 * rt;
        if (r < p.rows) {
            const int i = r / p.group, h = g * p.group + r % p.group;
            const float* qrow = static_cast<const float*>(p.q) + ((int64_t)(b * p.n_queries + i) * p.n_q_heads + h) * D +
                                4 * q4;
#pragma unroll
            for (int u = 0; u < NF / 4; ++u) {
                const float4 v = *reinterpret_cast<const float4*>(qrow + 16 * u);
                qf[rt][4 * u] = v.x;
                qf[rt][4 * u + 1] = v.y;
                qf[rt][4 * u + 2] = v.z;
                qf[rt][4 * u + 3] = v.w;
            }
        } else {
#pragma unroll
            for (int u = 0; u < NF; ++u) qf[rt][u] = 0.f;
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
    constexpr int kVP = F32Smem<D, NRT>::kVPitch;
    float(*vt)[kVP] = sm.u.vt[w];

    // Key l16 of the tile (clamped to its last valid key, so every load stays
    // in bounds; the clamped keys' scores are masked), features 16u + 4*q4 ..
    // +3. Read once per round: non-temporal loads.
    auto load_rows = [&](const float* src, int64_t tk, int valid, floatx4(&dst)[NF / 4]) {
        const float* row = src + (tk + min(l16, valid - 1)) * st + 4 * q4;
#pragma unroll
        for (int u = 0; u < NF / 4; ++u) dst[u] = __builtin_nontemporal_load(reinterpret_cast<const floatx4*>(row + 16 * u));
    };

    const int n_tiles = (int)((t1 - t0 + kTile - 1) / kTile);
    floatx4 kf[NF / 4], vr[NF / 4];
    int tau = w;
    if (tau < n_tiles) {
        const int64_t tk = t0 + (int64_t)kTile * tau;
        const int valid = (int)min((int64_t)kTile, t1 - tk);
        load_rows(kp, tk, valid, kf);
        load_rows(vp, tk, valid, vr);
    }
    for (; tau < n_tiles; tau += kWaves) {
        const int valid = (int)min((int64_t)kTile, t1 - (t0 + (int64_t)kTile * tau));
        const int nxt = tau + kWaves;
        const int64_t tk_n = t0 + (int64_t)kTile * nxt;
        const int valid_n = nxt < n_tiles ? (int)min((int64_t)kTile, t1 - tk_n) : 0;

        // Stage V ([key][feature]); its registers then take the next tile's V.
#pragma unroll
        for (int u = 0; u < NF / 4; ++u) *reinterpret_cast<floatx4*>(&vt[l16][16 * u + 4 * q4]) = vr[u];
        if (valid_n > 0) load_rows(vp, tk_n, valid_n, vr);

        // S^T = K Q^T over the permuted features.
        floatx4 sc[NRT];
#pragma unroll
        for (int rt = 0; rt < NRT; ++rt) {
            floatx4 a = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int u = 0; u < NF / 4; ++u) {
                a = __builtin_amdgcn_mfma_f32_16x16x4f32(kf[u].x, qf[rt][4 * u], a, 0, 0, 0);
                a = __builtin_amdgcn_mfma_f32_16x16x4f32(kf[u].y, qf[rt][4 * u + 1], a, 0, 0, 0);
                a = __builtin_amdgcn_mfma_f32_16x16x4f32(kf[u].z, qf[rt][4 * u + 2], a, 0, 0, 0);
                a = __builtin_amdgcn_mfma_f32_16x16x4f32(kf[u].w, qf[rt][4 * u + 3], a, 0, 0, 0);
            }
            sc[rt] = a;
        }
        if (valid_n > 0) load_rows(kp, tk_n, valid_n, kf);

        // Scale to base 2, mask keys past the range, tile max per row (keys
        // 4*q4 + i of the lane, the other lane groups hold the rest).
        bool grow = false;
        float alpha[NRT];
#pragma unroll
        for (int rt = 0; rt < NRT; ++rt) {
            float mx = -INFINITY;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float v = 4 * q4 + i < valid ? sc[rt][i] * c : -INFINITY;
                sc[rt][i] = v;
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
#pragma unroll
                for (int xt = 0; xt < NXT; ++xt) o[xt][rt] *= alpha[rt];
            }
        }
        // P = 2^(S - m), fp32.
#pragma unroll
        for (int rt = 0; rt < NRT; ++rt) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float pv = sc[rt][i] == -INFINITY ? 0.f : exp2_hw(sc[rt][i] - m_run[rt]);
                sc[rt][i] = pv;
                l_run[rt] += pv;
            }
        }

        wave_sync();
        // O^T += V^T P^T: step i takes keys 4j+i (lane group j); lane reads
        // V[4*q4 + i][16*xt + l16].
#pragma unroll
        for (int i = 0; i < 4; ++i) {
#pragma unroll
            for (int xt = 0; xt < NXT; ++xt) {
                const float a = vt[4 * q4 + i][16 * xt + l16];
#pragma unroll
                for (int rt = 0; rt < NRT; ++rt)
                    o[xt][rt] = __builtin_amdgcn_mfma_f32_16x16x4f32(a, sc[rt][i], o[xt][rt], 0, 0, 0);
            }
        }
        wave_sync();
    }

    // Full row sums: the 4 lane groups hold disjoint keys of the same rows.
#pragma unroll
    for (int rt = 0; rt < NRT; ++rt) l_run[rt] = group4_sum(l_run[rt]);

    // Merge the waves' states (Eq. 8) through LDS, the work split by feature
    // tiles: every wave publishes its (m, l) and the accumulator tiles that
    // other waves own, then folds the four partial states of its own tiles
    // and writes them; wave 0 also writes m and l.
    constexpr int kOwnTile = NRT * 4;  // floats per lane of one owned feature tile
    __syncthreads();                   // every wave is done with the V staging area
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
        const int r = r0 + l16 + 16 * rt;
        if (r >= p.rows) continue;
        const int i = r / p.group, h = g * p.group + r % p.group;
        const int64_t row = (((int64_t)slot * p.batch + b) * p.n_queries + i) * p.n_q_heads + h;
        if (w == 0 && q4 == 0) {
            p.m[row] = (m_run[rt] == -INFINITY) ? -INFINITY : m_run[rt] * kLn2;
            p.l[row] = l_run[rt];
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
            *reinterpret_cast<floatx4*>(p.acc + row * D + 16 * xt + 4 * q4) = v;
        }
    }
}

// Slot s of the launch (p.slot_begin + s) of stream (blockIdx.z, g): its
// piece by fixed chunks, for the rows of row group rg (32 rows each). Unit
// u = s * n_kv_heads + g; with one row group the work-group id is u, with
// more, eight consecutive units go to the eight XCDs and the row groups of a
// unit are 8 ids apart (same XCD, so they share its L2).
template <int D, int NRT>
__global__ __launch_bounds__(kThreads, 2) void chunk_mfma_f32_kernel(ChunkParams p, int row_groups) {
    __shared__ F32Smem<D, NRT> sm;
    const int x = blockIdx.x;
    const int x_hi = x / (8 * row_groups), rem = x % (8 * row_groups);
    const int rg = row_groups == 1 ? 0 : rem / 8;
    const int u = row_groups == 1 ? x : x_hi * 8 + rem % 8;
    if (u >= p.n_items * p.n_kv_heads) return;
    const int s = u / p.n_kv_heads;
    const int g = u % p.n_kv_heads;
    const int b = blockIdx.z;
    int64_t t0, t1;
    piece_tokens(p, chunk_view_len(p, b), b, g, s, &t0, &t1);
    f32_piece<D, NRT>(p, sm, b, g, p.slot_begin + s, t0, t1, 32 * rg);
}

// The whole resident history of every request, cut into balanced pieces
// (the line split of plan_next) over gridDim.x work-groups, one per CU;
// work-group w computes the pieces of its range one after another, each
// into its slot (p.plan_slots slots from p.slot_begin; slots without a
// piece keep the empty states written before the launch).
template <int D, int NRT>
__global__ __launch_bounds__(kThreads, 2) void history_mfma_f32_kernel(ChunkParams p) {
    __shared__ F32Smem<D, NRT> sm;
    const int64_t w = blockIdx.x;
    PlanStart st;
    if (!plan_start(p, w, st)) return;
    const int64_t total = st.total, piece_len = st.piece_len;

    // The walk runs on one lane with its cursor in LDS.
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
        if (k < 0) continue;
        f32_piece<D, NRT>(pa, sm, __builtin_amdgcn_readfirstlane(pc->b), __builtin_amdgcn_readfirstlane(pc->g),
                          pa.slot_begin + k, uniform64(pc->t0), uniform64(pc->t1), 0);
    }
}

template <int D, int NRT>
hipError_t launch_f32_t(const ChunkParams& p, hipStream_t stream) {
    const int row_groups = (p.rows + 31) / 32;
    const int64_t units = (int64_t)p.n_items * p.n_kv_heads;
    const int64_t gx = row_groups == 1 ? units : (units + 7) / 8 * 8 * row_groups;
    if (gx > 0x7fffffff) return hipErrorInvalidValue;
    hipLaunchKernelGGL((chunk_mfma_f32_kernel<D, NRT>), dim3((unsigned)gx, 1, p.batch), dim3(kThreads), 0, stream, p,
                       row_groups);
    return hipGetLastError();
}

// Work-groups of one history launch: one per CU (one wave per SIMD, as the
// narrow bf16 kernel's history launch), queried once per device.
constexpr int kMaxDevices = 64;

hipError_t history_wgs(int* out) {
    static int wgs[kMaxDevices];
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    int n = __atomic_load_n(&wgs[dev], __ATOMIC_RELAXED);
    if (n <= 0) {
        int cus = 0;
        e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
        if (e != hipSuccess) return e;
        n = cus > 0 ? cus : 1;
        __atomic_store_n(&wgs[dev], n, __ATOMIC_RELAXED);
    }
    *out = n;
    return hipSuccess;
}

template <int D, int NRT>
hipError_t launch_hist_f32_t(const ChunkParams& p, hipStream_t stream) {
    int n = 0;
    hipError_t e = history_wgs(&n);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((history_mfma_f32_kernel<D, NRT>), dim3(n), dim3(kThreads), 0, stream, p);
    return hipGetLastError();
}

}  // namespace

// fp32, head_dim 128 or 64, any row count (row groups of 32 beyond 32 rows);
// contiguous pieces only (no chunk lists, no block statistics, no candidate
// region).
hipError_t launch_chunk_mfma_f32(const ChunkParams& p, int head_dim, hipStream_t stream) {
    if ((head_dim != 128 && head_dim != 64) || p.rows <= 0 || p.chunk_idx || p.stats || p.with_cand)
        return hipErrorInvalidValue;
    if (head_dim == 64) return p.rows > 16 ? launch_f32_t<64, 2>(p, stream) : launch_f32_t<64, 1>(p, stream);
    return p.rows > 16 ? launch_f32_t<128, 2>(p, stream) : launch_f32_t<128, 1>(p, stream);
}

// The balanced cut on the fp32 kernel: fp32, head_dim 128 or 64, up to 32
// rows, p.plan_slots >= 2, no block statistics, no candidate region.
hipError_t launch_history_mfma_f32(const ChunkParams& p, int head_dim, hipStream_t stream) {
    if ((head_dim != 128 && head_dim != 64) || p.rows > 32 || p.plan_slots < 2 || p.stats || p.with_cand ||
        p.chunk_idx)
        return hipErrorInvalidValue;
    if (head_dim == 64) return p.rows > 16 ? launch_hist_f32_t<64, 2>(p, stream) : launch_hist_f32_t<64, 1>(p, stream);
    return p.rows > 16 ? launch_hist_f32_t<128, 2>(p, stream) : launch_hist_f32_t<128, 1>(p, stream);
}

}  // namespace ssv
