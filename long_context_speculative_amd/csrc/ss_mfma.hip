// MFMA bf16 chunk kernel of libssverify, for 16..32 rows per KV head.
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
//                                    output (bf16), A = V^T read from a
//                                    per-wave LDS tile that holds V transposed
//                                    (key-contiguous rows)
// The 4 waves' states are merged with Eq. (8) through LDS at the end and
// written as the slot's state (m in natural-log units).

#include "ss_common.h"

namespace ssv {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kTile = 32;      // keys per wave iteration
constexpr int kVtRow = 36;     // bf16 per transposed-V row: 32 keys + 4 pad (72 bytes)

template <int D, int NRT>
struct MfmaSmem {
    static constexpr int kAccRegs = (D / 16) * NRT * 4;  // accumulator floats per lane
    union {
        uint16_t vt[kWaves][D][kVtRow];
        struct {
            float acc[kWaves - 1][kAccRegs][64];
            float m[kWaves - 1][16 * NRT];
            float l[kWaves - 1][16 * NRT];
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

template <int D, int NRT>
__global__ __launch_bounds__(kThreads, 2) void chunk_mfma_kernel(ChunkParams p) {
    constexpr int NS = D / 32;   // feature steps of 32 for S = K Q^T
    constexpr int NXT = D / 16;  // 16-feature output tiles for O^T = V^T P^T
    __shared__ MfmaSmem<D, NRT> sm;

    // KV head fastest: the heads of one (slot, request) are dispatched
    // together, so with token-major layouts they stream the same rows.
    const int g = blockIdx.x % p.n_kv_heads;
    const int s = blockIdx.x / p.n_kv_heads;
    const int b = blockIdx.z;
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int l16 = lane & 15, q4 = lane >> 4;

    int32_t len = p.req_len ? p.req_len[b] : p.max_len;
    len = min(max(len, 0), p.max_len);
    int64_t t0, t1;
    slot_tokens(len, p.chunk_len, p.chunk_begin, p.n_chunks, p.cps, s, &t0, &t1);

    const int64_t base = (p.req_offset ? p.req_offset[b] : (int64_t)b * p.stride_b) + (int64_t)g * p.stride_h;
    const uint16_t* __restrict__ kp = static_cast<const uint16_t*>(p.k) + base;
    const uint16_t* __restrict__ vp = static_cast<const uint16_t*>(p.v) + base;
    const int64_t st = p.stride_t;

    // Q^T fragments: row r = l16 + 16*rt, features 32*k + 8*q4 .. +7.
    bf16x8 qf[NRT][NS];
#pragma unroll
    for (int rt = 0; rt < NRT; ++rt) {
        const int r = l16 + 16 * rt;
        if (r < p.rows) {
            const int i = r / p.group, h = g * p.group + r % p.group;
            const uint16_t* qrow = static_cast<const uint16_t*>(p.q) + ((int64_t)(b * p.n_queries + i) * p.n_q_heads + h) * D;
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

    const int64_t n_keys = t1 - t0;
    const int n_tiles = (int)((n_keys + kTile - 1) / kTile);
    uint16_t(*vt)[kVtRow] = sm.u.vt[w];

    // Loads address a tile as a uniform base (scalar registers) plus a 32-bit
    // per-lane offset. Keys past the range are clamped to its last key so
    // every load stays in bounds; their scores are masked below.
    const int sti = (int)st;
    // K fragment: keys 16*kt + l16 of the tile, features 32*k + 8*q4 .. +7.
    auto load_k = [&](int64_t tk, u32x4(&dst)[2][NS]) {
        const uint16_t* tb = kp + tk * st;
        const int last = (int)min((int64_t)kTile, t1 - tk) - 1;
#pragma unroll
        for (int kt = 0; kt < 2; ++kt) {
            const int off = min(16 * kt + l16, last) * sti + 8 * q4;
#pragma unroll
            for (int k = 0; k < NS; ++k) dst[kt][k] = *reinterpret_cast<const u32x4*>(tb + off + 32 * k);
        }
    };
    // V rows 4*kg + e (kg = q4 + 4*h), features 8*l16 .. +7.
    auto load_v = [&](int64_t tk, u32x4(&dst)[2][4]) {
        const uint16_t* tb = vp + tk * st;
        const int last = (int)min((int64_t)kTile, t1 - tk) - 1;
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int off = min(4 * (q4 + 4 * h) + e, last) * sti + 8 * l16;
                dst[h][e] = *reinterpret_cast<const u32x4*>(tb + off);
            }
    };

    u32x4 kf[2][NS], vr[2][4];
    int tau = w;
    if (tau < n_tiles) {
        load_k(t0 + (int64_t)kTile * tau, kf);
        load_v(t0 + (int64_t)kTile * tau, vr);
    }
    for (; tau < n_tiles; tau += kWaves) {
        const int64_t tk = t0 + (int64_t)kTile * tau;

        // Stage V(tau) transposed: vt[x][key] holds 4 keys per 8-byte word.
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int kg = q4 + 4 * h;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const uint32_t d0 = vr[h][0][i], d1 = vr[h][1][i], d2 = vr[h][2][i], d3 = vr[h][3][i];
                const u32x2 lo{(d0 & 0xffffu) | (d1 << 16), (d2 & 0xffffu) | (d3 << 16)};
                const u32x2 hi{(d0 >> 16) | (d1 & 0xffff0000u), (d2 >> 16) | (d3 & 0xffff0000u)};
                const int x = 8 * l16 + 2 * i;
                *reinterpret_cast<u32x2*>(&vt[x][4 * kg]) = lo;
                *reinterpret_cast<u32x2*>(&vt[x + 1][4 * kg]) = hi;
            }
        }

        // Prefetch the wave's next tile into the registers just consumed:
        // V right away (staged above), K once the S^T products have read it.
        const bool more = tau + kWaves < n_tiles;
        if (more) load_v(tk + kTile * kWaves, vr);

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
        if (more) load_k(tk + kTile * kWaves, kf);

        // Scale to base 2, mask keys past the range, tile max per row.
        const int valid = (int)min((int64_t)kTile, t1 - tk);
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
                    const float v = key < valid ? sc[kt][rt][j] * c : -INFINITY;
                    sc[kt][rt][j] = v;
                    mx = fmaxf(mx, v);
                }
            mx = fmaxf(mx, __shfl_xor(mx, 16));
            mx = fmaxf(mx, __shfl_xor(mx, 32));
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

        // P = 2^(S - m) in bf16 (B operand of the PV product); l sums the
        // rounded weights so numerator and denominator use the same values.
        bf16x8 pf[NRT];
#pragma unroll
        for (int rt = 0; rt < NRT; ++rt) {
            float ls = 0.f;
#pragma unroll
            for (int kt = 0; kt < 2; ++kt)
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const __bf16 pb = (__bf16)exp2_hw(sc[kt][rt][j] - m_run[rt]);
                    pf[rt][4 * kt + j] = pb;
                    ls += (float)pb;
                }
            l_run[rt] += ls;
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
            for (int rt = 0; rt < NRT; ++rt) o[xt][rt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, pf[rt], o[xt][rt], 0, 0, 0);
        }
        wave_sync();
    }

    // Full row sums: the 4 lane groups hold disjoint keys of the same rows.
#pragma unroll
    for (int rt = 0; rt < NRT; ++rt) {
        l_run[rt] += __shfl_xor(l_run[rt], 16);
        l_run[rt] += __shfl_xor(l_run[rt], 32);
    }

    // Merge the waves' states (Eq. 8) through LDS; wave 0 writes the slot.
    __syncthreads();
    if (w > 0) {
        int idx = 0;
#pragma unroll
        for (int xt = 0; xt < NXT; ++xt)
#pragma unroll
            for (int rt = 0; rt < NRT; ++rt)
#pragma unroll
                for (int j = 0; j < 4; ++j) sm.u.mg.acc[w - 1][idx++][lane] = o[xt][rt][j];
        if (q4 == 0) {
#pragma unroll
            for (int rt = 0; rt < NRT; ++rt) {
                sm.u.mg.m[w - 1][l16 + 16 * rt] = m_run[rt];
                sm.u.mg.l[w - 1][l16 + 16 * rt] = l_run[rt];
            }
        }
    }
    __syncthreads();
    if (w != 0) return;

    for (int ww = 0; ww < kWaves - 1; ++ww) {
        float a0[NRT], a1[NRT];
#pragma unroll
        for (int rt = 0; rt < NRT; ++rt) {
            const float mw = sm.u.mg.m[ww][l16 + 16 * rt];
            const float lw = sm.u.mg.l[ww][l16 + 16 * rt];
            const float m_new = fmaxf(m_run[rt], mw);
            a0[rt] = (m_run[rt] == -INFINITY) ? 0.f : exp2_hw(m_run[rt] - m_new);
            a1[rt] = (mw == -INFINITY) ? 0.f : exp2_hw(mw - m_new);
            l_run[rt] = a0[rt] * l_run[rt] + a1[rt] * lw;
            m_run[rt] = m_new;
        }
        int idx = 0;
#pragma unroll
        for (int xt = 0; xt < NXT; ++xt)
#pragma unroll
            for (int rt = 0; rt < NRT; ++rt)
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    o[xt][rt][j] = a0[rt] * o[xt][rt][j] + a1[rt] * sm.u.mg.acc[ww][idx++][lane];
                }
    }

#pragma unroll
    for (int rt = 0; rt < NRT; ++rt) {
        const int r = l16 + 16 * rt;
        if (r >= p.rows) continue;
        const int i = r / p.group, h = g * p.group + r % p.group;
        const int64_t row = (((int64_t)(p.slot_begin + s) * p.batch + b) * p.n_queries + i) * p.n_q_heads + h;
        if (q4 == 0) {
            p.m[row] = (m_run[rt] == -INFINITY) ? -INFINITY : m_run[rt] * kLn2;
            p.l[row] = l_run[rt];
        }
#pragma unroll
        for (int xt = 0; xt < NXT; ++xt)
            *reinterpret_cast<floatx4*>(p.acc + row * D + 16 * xt + 4 * q4) = o[xt][rt];
    }
}

template <int D, int NRT>
hipError_t launch_t(const ChunkParams& p, hipStream_t stream) {
    const int64_t gx = (int64_t)p.n_items * p.n_kv_heads;
    if (gx > 0x7fffffff) return hipErrorInvalidValue;
    dim3 grid((unsigned)gx, 1, p.batch);
    hipLaunchKernelGGL((chunk_mfma_kernel<D, NRT>), grid, dim3(kThreads), 0, stream, p);
    return hipGetLastError();
}

}  // namespace

// The V staging map gives each of 16 lanes 8 features of a key: head_dim 128.
hipError_t launch_chunk_mfma(const ChunkParams& p, int head_dim, hipStream_t stream) {
    if (head_dim != 128 || p.rows > 32) return hipErrorInvalidValue;
    return p.rows > 16 ? launch_t<128, 2>(p, stream) : launch_t<128, 1>(p, stream);
}

}  // namespace ssv
