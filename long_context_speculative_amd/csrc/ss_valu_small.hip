// VALU bf16 chunk kernel of libssverify for small row groups: fewer than 16
// rows per KV head (queries x heads of the GQA group do not fill a 16-row
// MFMA tile, e.g. 2 queries under 4-way GQA), head_dim 128.
//
// SpecStream ("Resource-Efficient Speculative Decoding for Long-Context LLM
// Serving"), section 4.2: one history chunk serves the whole query group; the
// chunk-local state (Eq. 7) is merged tile by tile and across waves (Eq. 8).
//
// One work-group of 4 waves per (slot, KV head, request); wave w takes key
// tiles w, w+4, ... of 32 keys. Per tile:
//   scores   lane l holds key l/2 and half l%2 of its 128 features (one
//            16-byte load per 8 features straight from HBM: a wave reads the
//            tile's 8 KB of K contiguously); every row's partial dot product
//            is 32 v_dot2_f32_bf16 against the query row in LDS (a broadcast
//            read), the two halves are joined with one lane exchange;
//   softmax  base 2, scale folded into one FMA, a reference maximum per row
//            that moves only when a score exceeds it by 2^8 (one ballot per
//            row and tile in the common case);
//   P V      V goes to a per-wave LDS tile; lane l then owns output features
//            2l, 2l+1 and accumulates p[row][key] * V[key][2l..2l+1] over the
//            tile's keys, two keys per v_dot2_f32_bf16 (the bf16 weights are
//            read from LDS as a broadcast; l sums the same rounded weights;
//            each weight's rounding remainder follows as a second pair of
//            dot products).
// The 4 waves' states are merged through LDS at the end.

#include "ss_common.h"

namespace ssv {
namespace {

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int D = 128;
constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kTile = 32;
constexpr int kVRow = D + 8;       // bf16 per staged V row
constexpr float kGrowLog2 = 8.f;   // reference-maximum threshold (log2 units)

template <int RMAX>
struct SmallSmem {
    uint16_t q[RMAX][D];                  // query rows of the KV head (zero past R)
    union {
        struct {
            uint16_t v[kWaves][kTile][kVRow];  // per-wave V tile
            uint32_t p[kWaves][RMAX][kTile / 2];  // per-wave bf16 weight pairs (keys 2j, 2j+1)
            uint32_t pr[kWaves][RMAX][kTile / 2]; // their rounding remainders (short histories)
        } t;
        struct {
            float o[kWaves - 1][RMAX][D];
            float m[kWaves - 1][RMAX];
            float l[kWaves - 1][RMAX];
        } mg;
    } u;
};

__device__ __forceinline__ float exp2_hw(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ void wave_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a), __builtin_bit_cast(bf16x2, b), c, false);
}

template <int RMAX>
__global__ __launch_bounds__(kThreads, 2) void chunk_valu_small_kernel(ChunkParams p) {
    __shared__ SmallSmem<RMAX> sm;
    const int g = blockIdx.x % p.n_kv_heads;
    const int s = blockIdx.x / p.n_kv_heads;
    const int b = blockIdx.z;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int kk = lane >> 1, half = lane & 1;
    const int R = p.rows;

    const int32_t len = chunk_view_len(p, b);
    int64_t t0, t1;
    piece_tokens(p, len, b, g, s, &t0, &t1);

    // Query rows of this KV head into LDS (rows past R are zero).
    for (int e = tid; e < RMAX * (D / 8); e += kThreads) {
        const int r = e / (D / 8), x = 8 * (e % (D / 8));
        u32x4 val = {0u, 0u, 0u, 0u};
        if (r < R) {
            const int i = r / p.group, h = g * p.group + r % p.group;
            val = *reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(p.q) +
                                                  ((int64_t)(b * p.n_queries + i) * p.n_q_heads + h) * D + x);
        }
        *reinterpret_cast<u32x4*>(&sm.q[r][x]) = val;
    }
    __syncthreads();

    const int64_t base = (p.req_offset ? p.req_offset[b] : (int64_t)b * p.stride_b) + (int64_t)g * p.stride_h;
    const uint16_t* __restrict__ kp = static_cast<const uint16_t*>(p.k) + base;
    const uint16_t* __restrict__ vp = static_cast<const uint16_t*>(p.v) + base;
    const int64_t st = p.stride_t;
    const int sti = (int)st;
    const float c = p.scale * kLog2e;

    float m_ref[RMAX], l_part[RMAX], o0[RMAX], o1[RMAX];
#pragma unroll
    for (int r = 0; r < RMAX; ++r) {
        m_ref[r] = -INFINITY;
        l_part[r] = 0.f;
        o0[r] = 0.f;
        o1[r] = 0.f;
    }

    const int n_tiles = (int)((t1 - t0 + kTile - 1) / kTile);
    // The weights' bf16 rounding remainders are carried too: where a few
    // keys dominate a row (a short history, or peaked scores over a long
    // one) the rounding does not average out.
    const bool split = true;
    u32x4 kr[8], vr[8];
    // Lane's key of the tile (clamped into the range; masked below) and its
    // 64 features: 8 loads of 16 bytes.
    auto load = [&](int64_t tk) {
        const int last = (int)min((int64_t)kTile, t1 - tk) - 1;
        const int off = min(kk, last) * sti + 64 * half;
        const uint16_t* kb = kp + tk * st + off;
        const uint16_t* vb = vp + tk * st + off;
#pragma unroll
        for (int j = 0; j < 8; ++j) kr[j] = *reinterpret_cast<const u32x4*>(kb + 8 * j);
#pragma unroll
        for (int j = 0; j < 8; ++j) vr[j] = *reinterpret_cast<const u32x4*>(vb + 8 * j);
    };

    int tau = w;
    if (tau < n_tiles) load(t0 + (int64_t)kTile * tau);
    for (; tau < n_tiles; tau += kWaves) {
        const int64_t tk = t0 + (int64_t)kTile * tau;
        const bool valid = kk < (int)min((int64_t)kTile, t1 - tk);

        // V tile to this wave's LDS (natural [key][feature] layout).
#pragma unroll
        for (int j = 0; j < 8; ++j) *reinterpret_cast<u32x4*>(&sm.u.t.v[w][kk][64 * half + 8 * j]) = vr[j];

        // Scores of the lane's key against every row.
        float sc[RMAX];
#pragma unroll
        for (int r = 0; r < RMAX; ++r) {
            const uint16_t* qrow = &sm.q[r][64 * half];
            float a = 0.f;
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const u32x4 qv = *reinterpret_cast<const u32x4*>(qrow + 8 * j);
                a = dot2(kr[j].x, qv.x, a);
                a = dot2(kr[j].y, qv.y, a);
                a = dot2(kr[j].z, qv.z, a);
                a = dot2(kr[j].w, qv.w, a);
            }
            a += __shfl_xor(a, 1);
            sc[r] = valid ? a : -INFINITY;
        }

        // The next tile's loads go out once this tile's K and V are consumed.
        if (tau + kWaves < n_tiles) load(tk + kTile * kWaves);

        // Softmax weights against the reference maxima.
#pragma unroll
        for (int r = 0; r < RMAX; ++r) {
            if (r >= R) continue;
            const float cand = sc[r] * c;
            if (__ballot(cand > m_ref[r] + kGrowLog2)) {
                float mx = cand;
#pragma unroll
                for (int o = 32; o > 1; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o));
                const float m_new = fmaxf(m_ref[r], mx);
                const float alpha = (m_ref[r] == -INFINITY) ? 0.f : exp2_hw(m_ref[r] - m_new);
                m_ref[r] = m_new;
                l_part[r] *= alpha;
                o0[r] *= alpha;
                o1[r] *= alpha;
            }
            // bf16 weight; the pair (p[key], p[key + 1]) is packed by the lane
            // of the even key and stored for the P V products.
            const float pv = exp2_hw(fmaf(sc[r], c, -m_ref[r]));
            const __bf16 pb = (__bf16)pv;
            const uint32_t pbits = __builtin_bit_cast(uint16_t, pb);
            const uint32_t pnext = __shfl_down(pbits, 2);
            if (half == 0) {
                l_part[r] += (float)pb;
                if ((kk & 1) == 0) sm.u.t.p[w][r][kk >> 1] = pbits | (pnext << 16);
            }
            if (split) {
                const __bf16 rb = (__bf16)(pv - (float)pb);
                const uint32_t rbits = __builtin_bit_cast(uint16_t, rb);
                const uint32_t rnext = __shfl_down(rbits, 2);
                if (half == 0) {
                    l_part[r] += (float)rb;
                    if ((kk & 1) == 0) sm.u.t.pr[w][r][kk >> 1] = rbits | (rnext << 16);
                }
            }
        }
        wave_sync();

        // P V: lane owns features 2*lane, 2*lane + 1; two keys per v_dot2.
#pragma unroll 2
        for (int k = 0; k < kTile; k += 8) {
            uint32_t va[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) va[j] = *reinterpret_cast<const uint32_t*>(&sm.u.t.v[w][k + j][2 * lane]);
            uint32_t x0[4], x1[4];  // (V[k][2l], V[k+1][2l]) and (V[k][2l+1], V[k+1][2l+1]) per key pair
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const uint32_t a = va[2 * j], bb = va[2 * j + 1];
                x0[j] = (a & 0xffffu) | (bb << 16);
                x1[j] = (a >> 16) | (bb & 0xffff0000u);
            }
#pragma unroll
            for (int r = 0; r < RMAX; ++r) {
                if (r >= R) continue;
                const u32x4 pp = *reinterpret_cast<const u32x4*>(&sm.u.t.p[w][r][k >> 1]);
                const uint32_t pw[4] = {pp.x, pp.y, pp.z, pp.w};
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    o0[r] = dot2(pw[j], x0[j], o0[r]);
                    o1[r] = dot2(pw[j], x1[j], o1[r]);
                }
                if (split) {
                    const u32x4 rr = *reinterpret_cast<const u32x4*>(&sm.u.t.pr[w][r][k >> 1]);
                    const uint32_t rw[4] = {rr.x, rr.y, rr.z, rr.w};
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        o0[r] = dot2(rw[j], x0[j], o0[r]);
                        o1[r] = dot2(rw[j], x1[j], o1[r]);
                    }
                }
            }
        }
        wave_sync();
    }

    // Row sums over the wave's keys.
#pragma unroll
    for (int r = 0; r < RMAX; ++r) {
        float l = l_part[r];
#pragma unroll
        for (int o = 32; o > 0; o >>= 1) l += __shfl_xor(l, o);
        l_part[r] = l;
    }

    // Merge the 4 waves (Eq. 8) through LDS; wave 0 writes the slot.
    __syncthreads();
    if (w > 0) {
#pragma unroll
        for (int r = 0; r < RMAX; ++r) {
            sm.u.mg.o[w - 1][r][2 * lane] = o0[r];
            sm.u.mg.o[w - 1][r][2 * lane + 1] = o1[r];
            if (lane == 0) {
                sm.u.mg.m[w - 1][r] = m_ref[r];
                sm.u.mg.l[w - 1][r] = l_part[r];
            }
        }
    }
    __syncthreads();
    if (w != 0) return;
#pragma unroll
    for (int r = 0; r < RMAX; ++r) {
        if (r >= R) continue;
        for (int ww = 0; ww < kWaves - 1; ++ww) {
            const float mw = sm.u.mg.m[ww][r];
            const float m_new = fmaxf(m_ref[r], mw);
            const float a0 = (m_ref[r] == -INFINITY) ? 0.f : exp2_hw(m_ref[r] - m_new);
            const float a1 = (mw == -INFINITY) ? 0.f : exp2_hw(mw - m_new);
            l_part[r] = a0 * l_part[r] + a1 * sm.u.mg.l[ww][r];
            o0[r] = a0 * o0[r] + a1 * sm.u.mg.o[ww][r][2 * lane];
            o1[r] = a0 * o1[r] + a1 * sm.u.mg.o[ww][r][2 * lane + 1];
            m_ref[r] = m_new;
        }
        const int i = r / p.group, h = g * p.group + r % p.group;
        const int64_t row = (((int64_t)(p.slot_begin + s) * p.batch + b) * p.n_queries + i) * p.n_q_heads + h;
        if (lane == 0) {
            p.m[row] = (m_ref[r] == -INFINITY) ? -INFINITY : m_ref[r] * kLn2;
            p.l[row] = l_part[r];
        }
        *reinterpret_cast<float2*>(p.acc + row * D + 2 * lane) = float2{o0[r], o1[r]};
    }
}

template <int RMAX>
hipError_t launch_t(const ChunkParams& p, hipStream_t stream) {
    const int64_t gx = (int64_t)p.n_items * p.n_kv_heads;
    if (gx > 0x7fffffff) return hipErrorInvalidValue;
    hipLaunchKernelGGL((chunk_valu_small_kernel<RMAX>), dim3((unsigned)gx, 1, p.batch), dim3(kThreads), 0, stream, p);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_chunk_valu_small(const ChunkParams& p, int head_dim, hipStream_t stream) {
    if (head_dim != D || p.rows >= 16 || p.rows < 1) return hipErrorInvalidValue;
    if (p.rows <= 4) return launch_t<4>(p, stream);
    if (p.rows <= 8) return launch_t<8>(p, stream);
    return launch_t<15>(p, stream);
}

}  // namespace ssv
