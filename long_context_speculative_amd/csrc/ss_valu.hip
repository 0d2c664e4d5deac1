// VALU chunk kernel of libssverify: fp32 inputs, and bf16 shapes whose rows
// do not fill a 16-row MFMA tile.
//
// SpecStream ("Resource-Efficient Speculative Decoding for Long-Context LLM
// Serving"), section 4.2: per chunk, scores of the whole query group against
// the chunk's keys and the chunk-local state of Eq. (7), merged across key
// tiles by Eq. (8).
//
// Layout of work: one work-group per (slot, KV head x row block, request).
// A tile of 64 keys is staged in LDS once and read by every row of the block
// (all queries and all heads of the GQA group). Each wave owns rows; lane k
// scores key k of the tile, row max and sum use cross-lane reductions.

#include "ss_common.h"

namespace ssv {
namespace {

constexpr int kTileKeys = 64;
constexpr int kWaves = 4;
constexpr int kThreads = kWaves * 64;
constexpr int kRowsPerWave = kValuRows / kWaves;

__device__ __forceinline__ float load_elem(const float* p, int64_t i) { return p[i]; }
__device__ __forceinline__ float load_elem(const uint16_t* p, int64_t i) {
    return __uint_as_float(static_cast<uint32_t>(p[i]) << 16);
}

__device__ __forceinline__ float exp2_hw(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
    return v;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
    return v;
}

// Orders this wave's LDS writes before its later LDS reads by other lanes.
__device__ __forceinline__ void wave_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

template <int D>
struct ValuSmem {
    float k[kTileKeys][D + 1];
    float v[kTileKeys][D];
    float q[kValuRows][D];
    float p[kWaves][kTileKeys];
};

// Loads the block's query rows (row r = i * G + hh of KV head g) into LDS.
template <typename T, int D>
__device__ __forceinline__ void load_rows(float (*qs)[D], const T* q, int b, int g, int r0, int nr, int n_queries,
                                          int n_q_heads, int group) {
    for (int idx = threadIdx.x; idx < nr * D; idx += kThreads) {
        const int rr = idx / D, x = idx % D;
        const int r = r0 + rr;
        const int i = r / group, hh = r % group;
        const int h = g * group + hh;
        qs[rr][x] = load_elem(q, ((int64_t)(b * n_queries + i) * n_q_heads + h) * D + x);
    }
}

// Stages keys/values [t, t + nv) in LDS (rows past nv are zero).
template <typename T, int D>
__device__ __forceinline__ void load_tile(ValuSmem<D>& sm, const T* kp, const T* vp, int64_t stride_t, int64_t t,
                                          int nv) {
    for (int idx = threadIdx.x; idx < kTileKeys * D; idx += kThreads) {
        const int key = idx / D, x = idx % D;
        float kv = 0.f, vv = 0.f;
        if (key < nv) {
            const int64_t off = (t + key) * stride_t + x;
            kv = load_elem(kp, off);
            vv = load_elem(vp, off);
        }
        sm.k[key][x] = kv;
        sm.v[key][x] = vv;
    }
}

// One key tile for one row: Eq. (7) on the tile merged into (m, l, acc) by
// Eq. (8). l is kept as per-lane partial sums (all lanes share m).
template <int D>
__device__ __forceinline__ void row_tile_update(ValuSmem<D>& sm, int rr, int lane, int w, bool visible, float scale,
                                                int nv, float& m_run, float& l_run, float (&acc)[D / 64]) {
    float sc = -INFINITY;
    if (visible) {
        float dot = 0.f;
#pragma unroll 16
        for (int x = 0; x < D; ++x) dot = fmaf(sm.q[rr][x], sm.k[lane][x], dot);
        sc = dot * scale;
    }
    const float tmax = wave_max(sc);
    const float m_new = fmaxf(m_run, tmax);
    const float alpha = (m_run == -INFINITY) ? 0.f : exp2_hw((m_run - m_new) * kLog2e);
    const float pr = visible ? exp2_hw((sc - m_new) * kLog2e) : 0.f;
    l_run = l_run * alpha + pr;
    sm.p[w][lane] = pr;
    wave_sync();
#pragma unroll
    for (int j = 0; j < D / 64; ++j) {
        float a = acc[j] * alpha;
        for (int k = 0; k < nv; ++k) a = fmaf(sm.p[w][k], sm.v[k][lane + 64 * j], a);
        acc[j] = a;
    }
    m_run = m_new;
    wave_sync();
}

template <int D>
__device__ __forceinline__ void write_row_state(float* m_out, float* l_out, float* acc_out, int64_t row, int lane,
                                                float m_run, float l_lane, const float (&acc)[D / 64]) {
    const float l_tot = wave_sum(l_lane);
    if (lane == 0) {
        m_out[row] = m_run;
        l_out[row] = l_tot;
    }
#pragma unroll
    for (int j = 0; j < D / 64; ++j) acc_out[row * D + lane + 64 * j] = acc[j];
}

template <typename T, int D>
__global__ __launch_bounds__(kThreads) void chunk_valu_kernel(ChunkParams p) {
    extern __shared__ __align__(16) unsigned char smem_raw[];
    ValuSmem<D>& sm = *reinterpret_cast<ValuSmem<D>*>(smem_raw);

    const int s = blockIdx.x;
    const int g = blockIdx.y / p.row_blocks;
    const int rb = blockIdx.y % p.row_blocks;
    const int b = blockIdx.z;
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int r0 = rb * kValuRows;
    const int nr = min(kValuRows, p.rows - r0);

    const int32_t len = chunk_view_len(p, b);
    int64_t t0, t1;
    piece_tokens(p, len, b, g, s, &t0, &t1);

    load_rows<T, D>(sm.q, static_cast<const T*>(p.q), b, g, r0, nr, p.n_queries, p.n_q_heads, p.group);
    const int64_t base = (p.req_offset ? p.req_offset[b] : (int64_t)b * p.stride_b) + (int64_t)g * p.stride_h;
    const T* kp = static_cast<const T*>(p.k) + base;
    const T* vp = static_cast<const T*>(p.v) + base;

    float m_run[kRowsPerWave], l_run[kRowsPerWave], acc[kRowsPerWave][D / 64];
#pragma unroll
    for (int ri = 0; ri < kRowsPerWave; ++ri) {
        m_run[ri] = -INFINITY;
        l_run[ri] = 0.f;
#pragma unroll
        for (int j = 0; j < D / 64; ++j) acc[ri][j] = 0.f;
    }

    for (int64_t t = t0; t < t1; t += kTileKeys) {
        const int nv = (int)min((int64_t)kTileKeys, t1 - t);
        __syncthreads();
        load_tile<T, D>(sm, kp, vp, p.stride_t, t, nv);
        __syncthreads();
#pragma unroll
        for (int ri = 0; ri < kRowsPerWave; ++ri) {
            const int rr = w + kWaves * ri;
            if (rr < nr) row_tile_update<D>(sm, rr, lane, w, lane < nv, p.scale, nv, m_run[ri], l_run[ri], acc[ri]);
        }
    }

#pragma unroll
    for (int ri = 0; ri < kRowsPerWave; ++ri) {
        const int rr = w + kWaves * ri;
        if (rr < nr) {
            const int r = r0 + rr;
            const int i = r / p.group, h = g * p.group + r % p.group;
            const int64_t row = (((int64_t)(p.slot_begin + s) * p.batch + b) * p.n_queries + i) * p.n_q_heads + h;
            write_row_state<D>(p.m, p.l, p.acc, row, lane, m_run[ri], l_run[ri], acc[ri]);
        }
    }
}

template <typename T, int D>
hipError_t launch_chunk_valu_t(const ChunkParams& p, hipStream_t stream) {
    dim3 grid(p.n_items, p.n_kv_heads * p.row_blocks, p.batch);
    hipLaunchKernelGGL((chunk_valu_kernel<T, D>), grid, dim3(kThreads), sizeof(ValuSmem<D>), stream, p);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_chunk_valu(const ChunkParams& p, int dtype, int head_dim, hipStream_t stream) {
    if (dtype == SS_F32) {
        if (head_dim == 64) return launch_chunk_valu_t<float, 64>(p, stream);
        return launch_chunk_valu_t<float, 128>(p, stream);
    }
    if (head_dim == 64) return launch_chunk_valu_t<uint16_t, 64>(p, stream);
    return launch_chunk_valu_t<uint16_t, 128>(p, stream);
}

}  // namespace ssv
