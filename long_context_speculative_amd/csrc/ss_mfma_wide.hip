// MFMA bf16 chunk kernel of libssverify for wide row groups (more than 32
// rows per KV head, e.g. a 64-node candidate tree under 8-way GQA: 512 rows).
//
// SpecStream ("Resource-Efficient Speculative Decoding for Long-Context LLM
// Serving"), section 4.2: one history chunk serves the whole query group; its
// local state (Eq. 7) is merged tile by tile (Eq. 8).
//
// With hundreds of rows per KV head the work is bound by the matrix cores,
// not by HBM: every key feeds 512 rows. A work-group of NW waves owns 64*NW
// rows (each wave 64 rows = four 16-row MFMA tiles, with its Q^T fragments
// and its O^T accumulator in registers). Key tiles of 32 are staged once in
// LDS per work-group, double-buffered, and read by every wave: K row-major
// (A operand of S^T = K Q^T), V transposed to key-contiguous rows (A operand
// of O^T = V^T P^T). Row groups beyond the first re-read the chunk; the
// launch places all row groups of one (slot, KV head, request) on the same
// XCD one after another (work-group ids 8 apart), so the re-read is served by
// that XCD's L2.

#include "ss_common.h"

namespace ssv {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int D = 128;
constexpr int kTile = 32;       // keys per iteration
constexpr int kKRow = D + 8;    // bf16 per staged K row (16-byte pad)
constexpr int kVtRow = 36;      // bf16 per transposed V row (32 keys + 4 pad)
constexpr int kRT = 4;          // 16-row tiles per wave (64 rows)
constexpr int kNS = D / 32;     // 32-feature steps of S = K Q^T
constexpr int kNXT = D / 16;    // 16-feature tiles of O^T

struct WideSmem {
    uint16_t k[2][kTile][kKRow];
    uint16_t vt[2][D][kVtRow];
};

__device__ __forceinline__ float exp2_hw(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

template <int NW>
__global__ __launch_bounds__(64 * NW, 1) void chunk_mfma_wide_kernel(ChunkParams p, int row_groups) {
    constexpr int T = 64 * NW;
    constexpr int kUnits = 256 / T;  // cooperative load units per thread (4 loads of 16 bytes each)
    __shared__ WideSmem sm;

    // Work-group -> (slot, row group): row groups of one slot are 8 ids apart.
    const int x = blockIdx.x;
    const int x_hi = x / (8 * row_groups), rem = x % (8 * row_groups);
    const int rg = rem / 8;
    const int s = x_hi * 8 + rem % 8;
    if (s >= p.n_items) return;
    const int g = blockIdx.y;
    const int b = blockIdx.z;
    const int tid = threadIdx.x;
    const int lane = tid & 63, w = tid >> 6;
    const int l16 = lane & 15, q4 = lane >> 4;

    int32_t len = p.req_len ? p.req_len[b] : p.max_len;
    len = min(max(len, 0), p.max_len);
    int64_t t0, t1;
    slot_tokens(len, p.chunk_len, p.chunk_begin, p.n_chunks, p.cps, s, &t0, &t1);

    const int64_t base = (p.req_offset ? p.req_offset[b] : (int64_t)b * p.stride_b) + (int64_t)g * p.stride_h;
    const uint16_t* __restrict__ kp = static_cast<const uint16_t*>(p.k) + base;
    const uint16_t* __restrict__ vp = static_cast<const uint16_t*>(p.v) + base;
    const int64_t st = p.stride_t;
    const int sti = (int)st;

    const int row0 = rg * 64 * NW + 64 * w;  // first row of this wave
    const bool active = row0 < p.rows;

    // Q^T fragments of the wave's 64 rows.
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

    floatx4 o[kNXT][kRT];
#pragma unroll
    for (int xt = 0; xt < kNXT; ++xt)
#pragma unroll
        for (int rt = 0; rt < kRT; ++rt) o[xt][rt] = floatx4{0.f, 0.f, 0.f, 0.f};
    float m_run[kRT], l_run[kRT];
#pragma unroll
    for (int rt = 0; rt < kRT; ++rt) {
        m_run[rt] = -INFINITY;
        l_run[rt] = 0.f;
    }
    const float c = p.scale * kLog2e;
    const int n_tiles = (int)((t1 - t0 + kTile - 1) / kTile);

    // Cooperative staging. Unit u < 128: V keys 4*(u/16)..+3, features
    // 8*(u%16)..+7; unit u >= 128: the same for K. Keys past the range are
    // clamped to its last key (finite values; their scores are masked).
    u32x4 pre_a[kUnits][4], pre_b[kUnits][4];
    auto fetch = [&](int64_t tk, u32x4(&pre)[kUnits][4]) {
        const int last = (int)min((int64_t)kTile, t1 - tk) - 1;
#pragma unroll
        for (int j = 0; j < kUnits; ++j) {
            const int u = tid + j * T;
            const int uu = u & 127;
            const int kg = uu >> 4, piece = uu & 15;
            const uint16_t* src = (u < 128 ? vp : kp) + tk * st + 8 * piece;
#pragma unroll
            for (int e = 0; e < 4; ++e) pre[j][e] = *reinterpret_cast<const u32x4*>(src + min(4 * kg + e, last) * sti);
        }
    };
    auto stage = [&](int buf, const u32x4(&pre)[kUnits][4]) {
#pragma unroll
        for (int j = 0; j < kUnits; ++j) {
            const int u = tid + j * T;
            const int uu = u & 127;
            const int kg = uu >> 4, piece = uu & 15;
            if (u < 128) {
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const uint32_t d0 = pre[j][0][i], d1 = pre[j][1][i], d2 = pre[j][2][i], d3 = pre[j][3][i];
                    const u32x2 lo{(d0 & 0xffffu) | (d1 << 16), (d2 & 0xffffu) | (d3 << 16)};
                    const u32x2 hi{(d0 >> 16) | (d1 & 0xffff0000u), (d2 >> 16) | (d3 & 0xffff0000u)};
                    const int xx = 8 * piece + 2 * i;
                    *reinterpret_cast<u32x2*>(&sm.vt[buf][xx][4 * kg]) = lo;
                    *reinterpret_cast<u32x2*>(&sm.vt[buf][xx + 1][4 * kg]) = hi;
                }
            } else {
#pragma unroll
                for (int e = 0; e < 4; ++e) *reinterpret_cast<u32x4*>(&sm.k[buf][4 * kg + e][8 * piece]) = pre[j][e];
            }
        }
    };

    // Key tiles go HBM -> registers two tiles ahead, registers -> LDS one
    // tile ahead (double-buffered LDS, two register sets), so a tile's loads
    // have two iterations to land.
    auto process = [&](const int cur, const int64_t tk) {
        if (!active) return;
        // S^T = K Q^T over the tile's 32 keys and the wave's 64 rows.
        floatx4 sc[2][kRT];
#pragma unroll
        for (int kt = 0; kt < 2; ++kt) {
#pragma unroll
            for (int rt = 0; rt < kRT; ++rt) sc[kt][rt] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int k = 0; k < kNS; ++k) {
                const bf16x8 a = as_bf16x8(*reinterpret_cast<const u32x4*>(&sm.k[cur][16 * kt + l16][32 * k + 8 * q4]));
#pragma unroll
                for (int rt = 0; rt < kRT; ++rt)
                    sc[kt][rt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, qf[rt][k], sc[kt][rt], 0, 0, 0);
            }
        }

        // Online softmax in base 2 (Eq. 7-8); rescale only when a max grows.
        const int valid = (int)min((int64_t)kTile, t1 - tk);
        bool grow = false;
        float alpha[kRT];
#pragma unroll
        for (int rt = 0; rt < kRT; ++rt) {
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
            for (int rt = 0; rt < kRT; ++rt) {
                l_run[rt] *= alpha[rt];
#pragma unroll
                for (int xt = 0; xt < kNXT; ++xt) o[xt][rt] *= alpha[rt];
            }
        }
        bf16x8 pf[kRT];
#pragma unroll
        for (int rt = 0; rt < kRT; ++rt) {
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

        // O^T += V^T P^T
#pragma unroll
        for (int xt = 0; xt < kNXT; ++xt) {
            const uint16_t* row = sm.vt[cur][16 * xt + l16];
            const u32x2 lo = *reinterpret_cast<const u32x2*>(row + 4 * q4);
            const u32x2 hi = *reinterpret_cast<const u32x2*>(row + 16 + 4 * q4);
            const bf16x8 a = as_bf16x8(u32x4{lo.x, lo.y, hi.x, hi.y});
#pragma unroll
            for (int rt = 0; rt < kRT; ++rt)
                o[xt][rt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, pf[rt], o[xt][rt], 0, 0, 0);
        }
    };

    if (n_tiles > 0) {
        fetch(t0, pre_a);
        stage(0, pre_a);
    }
    if (n_tiles > 1) fetch(t0 + kTile, pre_b);
    __syncthreads();
    for (int t = 0; t < n_tiles; t += 2) {
        const int64_t tk = t0 + (int64_t)kTile * t;
        if (t + 2 < n_tiles) fetch(tk + 2 * kTile, pre_a);
        process(0, tk);
        if (t + 1 < n_tiles) stage(1, pre_b);
        __syncthreads();
        if (t + 1 >= n_tiles) break;
        if (t + 3 < n_tiles) fetch(tk + 3 * kTile, pre_b);
        process(1, tk + kTile);
        if (t + 2 < n_tiles) stage(0, pre_a);
        __syncthreads();
    }

    if (!active) return;
#pragma unroll
    for (int rt = 0; rt < kRT; ++rt) {
        l_run[rt] += __shfl_xor(l_run[rt], 16);
        l_run[rt] += __shfl_xor(l_run[rt], 32);
    }
#pragma unroll
    for (int rt = 0; rt < kRT; ++rt) {
        const int r = row0 + 16 * rt + l16;
        if (r >= p.rows) continue;
        const int i = r / p.group, h = g * p.group + r % p.group;
        const int64_t row = (((int64_t)(p.slot_begin + s) * p.batch + b) * p.n_queries + i) * p.n_q_heads + h;
        if (q4 == 0) {
            p.m[row] = (m_run[rt] == -INFINITY) ? -INFINITY : m_run[rt] * kLn2;
            p.l[row] = l_run[rt];
        }
#pragma unroll
        for (int xt = 0; xt < kNXT; ++xt)
            *reinterpret_cast<floatx4*>(p.acc + row * D + 16 * xt + 4 * q4) = o[xt][rt];
    }
}

template <int NW>
hipError_t launch_wide_t(const ChunkParams& p, hipStream_t stream) {
    const int row_groups = (p.rows + 64 * NW - 1) / (64 * NW);
    const int64_t gx = (int64_t)((p.n_items + 7) / 8) * 8 * row_groups;
    if (gx > 0x7fffffff) return hipErrorInvalidValue;
    dim3 grid((unsigned)gx, p.n_kv_heads, p.batch);
    hipLaunchKernelGGL((chunk_mfma_wide_kernel<NW>), grid, dim3(64 * NW), 0, stream, p, row_groups);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_chunk_mfma_wide(const ChunkParams& p, int head_dim, hipStream_t stream) {
    if (head_dim != D || p.rows <= 32) return hipErrorInvalidValue;
    const int waves = (p.rows + 63) / 64;
    // Up to 128 rows: two waves (for 33..64 rows the second wave only helps
    // stage tiles); more rows: four waves per row group.
    if (waves >= 3) return launch_wide_t<4>(p, stream);
    return launch_wide_t<2>(p, stream);
}

}  // namespace ssv
