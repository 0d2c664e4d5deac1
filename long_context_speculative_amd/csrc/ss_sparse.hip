// Block statistics and block selection of libssverify.
//
// SparseSpec-L (abstract on the pages): the per-head attention statistics of
// full verification are an importance signal for the history; Dustin:
// verification restricted to the critical history blocks. With the history
// verified in blocks of C tokens (one state slot per block, SpecStream
// section 4.2, Eq. 7), the softmax mass that row r of the round puts on block
// j is l_j(r) * exp(m_j(r) - lse(r)), lse the row's final log-normaliser
// (Eq. 8-9); the importance of block j for KV head g is the largest such mass
// over the head's rows.
//
// importance_kernel: one thread per (request, KV head, block); the rows of
// the head are read from the block's slot and the final lse.
// importance_stats_kernel: the same mass from the block statistics the
// history kernels record as a by-product (four wave quarters per block,
// entries [quarter][request][KV head][block][row of the head]).
// select_kernel: one work-group per (request, KV head); every block's rank
// (more important first, ties to the lower index) is counted against all
// others in LDS, the k best are written in increasing index order, padded
// with -1.

#include "ss_common.h"

namespace ssv {
namespace {

constexpr int kThreads = 256;

__global__ __launch_bounds__(kThreads) void importance_kernel(ImportanceParams p) {
    const int64_t id = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    const int64_t total = (int64_t)p.batch * p.n_kv_heads * p.n_blocks;
    if (id >= total) return;
    const int j = (int)(id % p.n_blocks);
    const int g = (int)((id / p.n_blocks) % p.n_kv_heads);
    const int b = (int)(id / ((int64_t)p.n_blocks * p.n_kv_heads));
    const int group = p.n_q_heads / p.n_kv_heads;
    const int rows = p.n_queries * group;
    float best = 0.f;
    for (int r = 0; r < rows; ++r) {
        const int i = r / group, h = g * group + r % group;
        const int64_t out_row = ((int64_t)b * p.n_queries + i) * p.n_q_heads + h;
        const int64_t row = ((int64_t)(p.slot_begin + j) * p.batch + b) * p.n_queries * p.n_q_heads +
                            (int64_t)i * p.n_q_heads + h;
        const float l = p.l[row];
        const float lse = p.lse[out_row];
        if (!(l > 0.f) || !(lse > -INFINITY)) continue;
        // mass = l * e^(m - lse), computed as 2^((m - lse) * log2 e) * l
        const float mass = l * __builtin_amdgcn_exp2f((p.m[row] - lse) * kLog2e);
        best = fmaxf(best, mass);
    }
    p.importance[id] = best;
}

__global__ __launch_bounds__(kThreads) void select_kernel(SelectParams p) {
    extern __shared__ float imp[];
    int32_t* chosen = reinterpret_cast<int32_t*>(imp + p.n_blocks);
    const int g = blockIdx.x % p.n_kv_heads;
    const int b = blockIdx.x / p.n_kv_heads;
    const int64_t base = ((int64_t)b * p.n_kv_heads + g) * p.n_blocks;
    int32_t len = p.req_len ? p.req_len[b] : p.max_len;
    len = len < 0 ? 0 : (len > p.max_len ? p.max_len : len);
    const int valid = (int)min((int64_t)p.n_blocks, ((int64_t)len + p.block_len - 1) / p.block_len);
    for (int i = threadIdx.x; i < p.n_blocks; i += kThreads) imp[i] = p.importance[base + i];
    __syncthreads();
    for (int i = threadIdx.x; i < p.n_blocks; i += kThreads) {
        int rank = 0;
        const float v = imp[i];
        for (int j = 0; j < valid; ++j) {
            const float u = imp[j];
            rank += (u > v || (u == v && j < i)) ? 1 : 0;
        }
        chosen[i] = (i < valid && rank < p.k) ? 1 : 0;
    }
    __syncthreads();
    // position of each kept block among the kept ones (increasing index)
    for (int i = threadIdx.x; i < p.n_blocks; i += kThreads) {
        if (!chosen[i]) continue;
        int pos = 0;
        for (int j = 0; j < i; ++j) pos += chosen[j];
        p.out[((int64_t)b * p.n_kv_heads + g) * p.k + pos] = i;
    }
    const int kept = valid < p.k ? valid : p.k;
    for (int s = kept + threadIdx.x; s < p.k; s += kThreads) p.out[((int64_t)b * p.n_kv_heads + g) * p.k + s] = -1;
}

// Importance from block statistics: the four wave quarters of a block fold
// into its mass l * exp(m - lse) per row, maximised over the KV head's rows.
// One wave per (request, KV head, block): lane r + 32 * half takes row r
// (and rows r + 32, ...) of quarters half and half + 2; entries of
// consecutive rows are adjacent.
__global__ __launch_bounds__(kThreads) void importance_stats_kernel(StatsImportanceParams p) {
    const int lane = threadIdx.x % 64;
    const int64_t unit = (int64_t)blockIdx.x * (kThreads / 64) + threadIdx.x / 64;  // (request, KV head, block)
    const int64_t total = (int64_t)p.batch * p.n_kv_heads * p.n_blocks;
    if (unit >= total) return;  // whole waves
    const int64_t bg = unit / p.n_blocks;
    const int g = (int)(bg % p.n_kv_heads), b = (int)(bg / p.n_kv_heads);
    const int group = p.n_q_heads / p.n_kv_heads;
    const int rows = p.n_queries * group;
    const int half = lane / 32;
    const int64_t quarter = total * rows;
    // The entries that exist: the pieces are block-aligned and a wave takes
    // every fourth tile of a piece, so wave w attended block j iff the block
    // holds more than w tiles of the request's keys.
    const int32_t len = clamp_len(p.req_len ? p.req_len[b] : p.max_len, p.max_len);
    const int j = (int)(unit % p.n_blocks);
    const int64_t keys = (int64_t)len - (int64_t)j * p.block_len;
    const int tiles = keys <= 0 ? 0 : (int)min((int64_t)kStatsQuarters, (min(keys, (int64_t)p.block_len) + 31) / 32);
    float best = 0.f;
    for (int r = lane % 32; r < rows; r += 32) {  // same trip count in both halves
        const int i = r / group, h = g * group + r % group;
        const float lse = p.lse[((int64_t)b * p.n_queries + i) * p.n_q_heads + h];
        float mass = 0.f;
        if (lse > -INFINITY) {
            for (int w = half; w < tiles; w += 2) {
                const float2 ml = p.ml[w * quarter + unit * rows + r];
                if (ml.y > 0.f) mass += ml.y * __builtin_amdgcn_exp2f((ml.x - lse) * kLog2e);
            }
        }
        mass += __shfl_xor(mass, 32);
        best = fmaxf(best, mass);
    }
    for (int off = 16; off >= 1; off >>= 1) best = fmaxf(best, __shfl_xor(best, off));
    if (lane == 0) p.importance[unit] = best;
}

}  // namespace

hipError_t launch_importance_stats(const StatsImportanceParams& p, hipStream_t stream) {
    const int64_t units = (int64_t)p.batch * p.n_kv_heads * p.n_blocks;
    const int64_t wgs = (units + kThreads / 64 - 1) / (kThreads / 64);
    if (wgs == 0) return hipSuccess;
    if (wgs > 0x7fffffff) return hipErrorInvalidValue;
    hipLaunchKernelGGL(importance_stats_kernel, dim3((unsigned)wgs), dim3(kThreads), 0, stream, p);
    return hipGetLastError();
}

hipError_t launch_importance(const ImportanceParams& p, hipStream_t stream) {
    const int64_t total = (int64_t)p.batch * p.n_kv_heads * p.n_blocks;
    const int64_t blocks = (total + kThreads - 1) / kThreads;
    if (blocks == 0) return hipSuccess;
    if (blocks > 0x7fffffff) return hipErrorInvalidValue;
    hipLaunchKernelGGL(importance_kernel, dim3((unsigned)blocks), dim3(kThreads), 0, stream, p);
    return hipGetLastError();
}

hipError_t launch_select(const SelectParams& p, hipStream_t stream) {
    const int64_t wgs = (int64_t)p.batch * p.n_kv_heads;
    if (wgs == 0) return hipSuccess;
    const size_t smem = (size_t)p.n_blocks * (sizeof(float) + sizeof(int32_t));
    hipLaunchKernelGGL(select_kernel, dim3((unsigned)wgs), dim3(kThreads), smem, stream, p);
    return hipGetLastError();
}

}  // namespace ssv
