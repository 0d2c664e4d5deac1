// Candidate-region kernel and state merge of libssverify.
//
// SpecStream ("Resource-Efficient Speculative Decoding for Long-Context LLM
// Serving"), section 4.2: after the history, the GPU-resident region is
// attended under a mask by each query's position; its state joins the
// history states by Eq. (8), and O = a / l once every visible key is in
// (Eq. 9). The tree mask is the ancestor rule of single-pass tree verification
// (Speculative Streaming post, section 3).
//
// candidates_kernel: one work-group per (request, KV head, block of 16 rows).
// The block's query rows and the request's candidate keys and values are
// staged in LDS as fp32; every (row, candidate) score is one thread's dot
// product, every row's softmax one wave's reduction, and every (row, 4
// features) output one thread's sum over candidates. n_cand <= 64.
//
// merge_kernel: one thread per (output row, 4 features), D/4 threads per
// row; each finds the row's common maximum over its slots' m, then folds
// the slots in slot order (Eq. 8: l and its 4 accumulator features, one
// 16-byte load per slot) and divides by l. No lane exchanges, and every
// slot's loads are independent of the others'.

#include "ss_common.h"

namespace ssv {
namespace {

constexpr int kRowsPerBlock = 16;
constexpr int kThreads = 256;

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

// One 16-byte load of consecutive elements, widened to fp32 in LDS.
template <typename T>
__device__ __forceinline__ void load16_f32(const T* src, float* dst);
template <>
__device__ __forceinline__ void load16_f32<float>(const float* src, float* dst) {
    *reinterpret_cast<float4*>(dst) = *reinterpret_cast<const float4*>(src);
}
template <>
__device__ __forceinline__ void load16_f32<uint16_t>(const uint16_t* src, float* dst) {
    const uint4 v = *reinterpret_cast<const uint4*>(src);
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        dst[2 * j] = __uint_as_float(w[j] << 16);
        dst[2 * j + 1] = __uint_as_float(w[j] & 0xffff0000u);
    }
}

// LDS carve-up (floats): K [n][D + 4] | V [n][D] | Q [16][D] | P [16][64] | m, l [16]
template <int D>
__host__ __device__ constexpr int cand_k_stride() { return D + 4; }

template <int D>
__host__ __device__ inline size_t cand_smem_bytes(int n) {
    return sizeof(float) * ((size_t)n * cand_k_stride<D>() + (size_t)n * D + kRowsPerBlock * D +
                            kRowsPerBlock * 64 + 2 * kRowsPerBlock);
}

template <typename T, int D>
__global__ __launch_bounds__(kThreads) void candidates_kernel(CandParams p) {
    extern __shared__ __align__(16) float smem[];
    __shared__ uint64_t bits[64];
    __shared__ int32_t par[64];
    constexpr int KS = cand_k_stride<D>();

    const int n = p.n_queries;
    const int g = blockIdx.y / p.row_blocks;
    const int rb = blockIdx.y % p.row_blocks;
    const int b = blockIdx.z;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int r0 = rb * kRowsPerBlock;
    const int nr = min(kRowsPerBlock, p.rows - r0);

    float* ks = smem;
    float* vs = ks + n * KS;
    float* qs = vs + n * D;
    float* ps = qs + kRowsPerBlock * D;
    float* ms = ps + kRowsPerBlock * 64;
    float* ls = ms + kRowsPerBlock;

    // Visibility bits: causal, or tree ancestors built in node order.
    if (p.parents) {
        if (tid < n) par[tid] = p.parents[(int64_t)b * n + tid];
        __syncthreads();
        if (tid == 0)
            for (int i = 0; i < n; ++i) bits[i] = tree_bits_step(bits, i, par[i]);
    } else if (tid < n) {
        bits[tid] = chain_bits(tid);
    }

    // Stage Q rows, candidate keys and values as fp32, 16 bytes per load
    // (rows are contiguous and 16-byte aligned).
    constexpr int E = 16 / sizeof(T);  // elements per 16-byte load
    const T* q = static_cast<const T*>(p.q);
    for (int e = tid; e < nr * (D / E); e += kThreads) {
        const int rr = e / (D / E), x = E * (e % (D / E));
        const int r = r0 + rr;
        const int i = r / p.group, h = g * p.group + r % p.group;
        load16_f32<T>(q + ((int64_t)(b * p.n_queries + i) * p.n_q_heads + h) * D + x, qs + rr * D + x);
    }
    const int64_t base = (p.req_offset ? p.req_offset[b] : (int64_t)b * p.stride_b) + (int64_t)g * p.stride_h;
    const T* kp = static_cast<const T*>(p.k) + base;
    const T* vp = static_cast<const T*>(p.v) + base;
    for (int e = tid; e < n * (D / E); e += kThreads) {
        const int k = e / (D / E), x = E * (e % (D / E));
        load16_f32<T>(kp + (int64_t)k * p.stride_t + x, ks + k * KS + x);
        load16_f32<T>(vp + (int64_t)k * p.stride_t + x, vs + k * D + x);
    }
    __syncthreads();
    if (p.mask_out && g == 0 && rb == 0 && tid < n) p.mask_out[(int64_t)b * n + tid] = bits[tid];

    // Scores of visible (row, candidate) pairs; -inf elsewhere.
    for (int e = tid; e < nr * n; e += kThreads) {
        const int rr = e / n, k = e % n;
        const int i = (r0 + rr) / p.group;
        float sc = -INFINITY;
        if ((bits[i] >> k) & 1) {
            const float4* qa = reinterpret_cast<const float4*>(qs + rr * D);
            const float4* ka = reinterpret_cast<const float4*>(ks + k * KS);
            float dot = 0.f;
#pragma unroll 8
            for (int x = 0; x < D / 4; ++x) {
                const float4 a = qa[x], c = ka[x];
                dot = fmaf(a.x, c.x, dot);
                dot = fmaf(a.y, c.y, dot);
                dot = fmaf(a.z, c.z, dot);
                dot = fmaf(a.w, c.w, dot);
            }
            sc = dot * p.scale;
        }
        ps[rr * 64 + k] = sc;
    }
    __syncthreads();

    // Row softmax (Eq. 7 over the visible candidates): one wave per row.
    for (int rr = w; rr < nr; rr += kThreads / 64) {
        const float sc = lane < n ? ps[rr * 64 + lane] : -INFINITY;
        const float mx = wave_max(sc);
        const float pr = (sc == -INFINITY) ? 0.f : exp2_hw((sc - mx) * kLog2e);
        const float l = wave_sum(pr);
        if (lane < n) ps[rr * 64 + lane] = pr;
        if (lane == 0) {
            ms[rr] = mx;
            ls[rr] = l;
        }
    }
    __syncthreads();

    // acc = P V, 4 features per thread.
    for (int e = tid; e < nr * (D / 4); e += kThreads) {
        const int rr = e / (D / 4), x = 4 * (e % (D / 4));
        float4 a = {0.f, 0.f, 0.f, 0.f};
        for (int k = 0; k < n; ++k) {
            const float pk = ps[rr * 64 + k];
            const float4 v = *reinterpret_cast<const float4*>(vs + k * D + x);
            a.x = fmaf(pk, v.x, a.x);
            a.y = fmaf(pk, v.y, a.y);
            a.z = fmaf(pk, v.z, a.z);
            a.w = fmaf(pk, v.w, a.w);
        }
        const int r = r0 + rr;
        const int i = r / p.group, h = g * p.group + r % p.group;
        const int64_t row = (((int64_t)p.slot * p.batch + b) * p.n_queries + i) * p.n_q_heads + h;
        *reinterpret_cast<float4*>(p.acc + row * D + x) = a;
        if (x == 0) {
            p.m[row] = ms[rr];
            p.l[row] = ls[rr];
        }
    }
}

// Eq. (8) over the slots of one row, then O = a / l and lse = m + ln l.
template <int D>
__global__ __launch_bounds__(kThreads) void merge_kernel(MergeParams p) {
    constexpr int TPR = D / 4;  // threads per row
    const int64_t n_rows = (int64_t)p.batch * p.n_queries * p.n_q_heads;
    const int64_t t = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    const int64_t row = t / TPR;
    const int x = (int)(t % TPR) * 4;  // first of the thread's 4 features
    if (row >= n_rows) return;
    const int b = (int)(row / ((int64_t)p.n_queries * p.n_q_heads));
    int ns = p.n_slots;
    if (p.slots_per_req) ns = min(max(p.slots_per_req[b], 0), p.n_slots);

    float mx = -INFINITY;
    for (int s = 0; s < ns; ++s) mx = fmaxf(mx, p.m[s * n_rows + row]);
    float lsum = 0.f;
    float4 a = make_float4(0.f, 0.f, 0.f, 0.f);
    if (mx != -INFINITY) {
        // four slots' loads at a time, then their folds in slot order
        for (int s0 = 0; s0 < ns; s0 += 4) {
            float ms[4], ls[4];
            float4 vs[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int s = min(s0 + u, ns - 1);
                ms[u] = p.m[s * n_rows + row];
                ls[u] = p.l[s * n_rows + row];
                vs[u] = *reinterpret_cast<const float4*>(p.acc + (s * n_rows + row) * D + x);
            }
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                if (s0 + u >= ns) break;
                const float f = (ms[u] == -INFINITY) ? 0.f : exp2_hw((ms[u] - mx) * kLog2e);
                lsum = fmaf(f, ls[u], lsum);
                a.x = fmaf(f, vs[u].x, a.x);
                a.y = fmaf(f, vs[u].y, a.y);
                a.z = fmaf(f, vs[u].z, a.z);
                a.w = fmaf(f, vs[u].w, a.w);
            }
        }
    }
    const bool seen = lsum > 0.f;
    const float4 o = seen ? make_float4(a.x / lsum, a.y / lsum, a.z / lsum, a.w / lsum) : make_float4(0.f, 0.f, 0.f, 0.f);
    *reinterpret_cast<float4*>(p.o + row * D + x) = o;
    if (x == 0) p.lse[row] = seen ? mx + __builtin_amdgcn_logf(lsum) * kLn2 : -INFINITY;
}

template <typename T, int D>
hipError_t launch_cand_t(const CandParams& p, hipStream_t stream) {
    dim3 grid(1, p.n_kv_heads * p.row_blocks, p.batch);
    hipLaunchKernelGGL((candidates_kernel<T, D>), grid, dim3(kThreads), cand_smem_bytes<D>(p.n_queries), stream, p);
    return hipGetLastError();
}

// Empty states over a contiguous range of rows: the slots that the balanced
// cut leaves without a piece keep them.
__global__ __launch_bounds__(kThreads) void state_fill_kernel(float4* __restrict__ acc, int64_t n_vec,
                                                              float* __restrict__ m, float* __restrict__ l,
                                                              int64_t n_rows) {
    const int64_t step = (int64_t)gridDim.x * kThreads;
    for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < n_vec; i += step)
        acc[i] = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < n_rows; i += step) {
        m[i] = -INFINITY;
        l[i] = 0.f;
    }
}

// A byte pattern over a buffer (a multiple of 16 bytes, 16-byte aligned).
__global__ __launch_bounds__(kThreads) void word_fill_kernel(uint4* __restrict__ dst, int64_t n_vec, uint32_t word) {
    const int64_t step = (int64_t)gridDim.x * kThreads;
    for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < n_vec; i += step)
        dst[i] = make_uint4(word, word, word, word);
}

}  // namespace

hipError_t launch_word_fill(void* dst, int64_t bytes, uint32_t word, hipStream_t stream) {
    const int64_t n_vec = bytes / 16;
    if (n_vec <= 0) return hipSuccess;
    int64_t blocks = (n_vec + kThreads - 1) / kThreads;
    if (blocks > 8192) blocks = 8192;
    hipLaunchKernelGGL(word_fill_kernel, dim3((unsigned)blocks), dim3(kThreads), 0, stream,
                       static_cast<uint4*>(dst), n_vec, word);
    return hipGetLastError();
}

int cand_row_blocks(int rows) { return (rows + kRowsPerBlock - 1) / kRowsPerBlock; }

hipError_t launch_candidates(const CandParams& p, int dtype, int head_dim, hipStream_t stream) {
    if (dtype == SS_F32) {
        if (head_dim == 64) return launch_cand_t<float, 64>(p, stream);
        return launch_cand_t<float, 128>(p, stream);
    }
    if (head_dim == 64) return launch_cand_t<uint16_t, 64>(p, stream);
    return launch_cand_t<uint16_t, 128>(p, stream);
}

hipError_t launch_state_fill(float* acc, float* m, float* l, int64_t row_begin, int64_t n_rows, int head_dim,
                             hipStream_t stream) {
    if (n_rows <= 0) return hipSuccess;
    const int64_t n_vec = n_rows * head_dim / 4;
    int64_t blocks = (n_vec + kThreads - 1) / kThreads;
    if (blocks > 8192) blocks = 8192;
    hipLaunchKernelGGL(state_fill_kernel, dim3((unsigned)blocks), dim3(kThreads), 0, stream,
                       reinterpret_cast<float4*>(acc + row_begin * head_dim), n_vec, m + row_begin, l + row_begin,
                       n_rows);
    return hipGetLastError();
}

hipError_t launch_merge(const MergeParams& p, hipStream_t stream) {
    const int64_t rows = (int64_t)p.batch * p.n_queries * p.n_q_heads;
    const int64_t threads = rows * (p.head_dim / 4);
    const int64_t blocks = (threads + kThreads - 1) / kThreads;
    if (blocks > 0x7fffffff) return hipErrorInvalidValue;
    if (p.head_dim == 64)
        hipLaunchKernelGGL(merge_kernel<64>, dim3((unsigned)blocks), dim3(kThreads), 0, stream, p);
    else
        hipLaunchKernelGGL(merge_kernel<128>, dim3((unsigned)blocks), dim3(kThreads), 0, stream, p);
    return hipGetLastError();
}

}  // namespace ssv
