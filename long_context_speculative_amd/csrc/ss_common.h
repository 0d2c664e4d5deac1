// Internal definitions shared by the kernels and the host layer of libssverify.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "ss_verify.h"

namespace ssv {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// ---------------------------------------------------------------------------
// Integer rules shared by host and device (the host exports them for tests).
// ---------------------------------------------------------------------------

// Token range of slot s of a chunk call (SpecStream section 4.2: contiguous
// chunks along token positions; cps consecutive chunks per slot).
__host__ __device__ inline void slot_tokens(int32_t len, int32_t chunk_len, int32_t chunk_begin, int32_t n_chunks,
                                            int32_t cps, int32_t s, int64_t* t0, int64_t* t1) {
    const int64_t c0 = (int64_t)chunk_begin + (int64_t)s * cps;
    int64_t c1 = c0 + cps;
    const int64_t c_end = (int64_t)chunk_begin + n_chunks;
    if (c1 > c_end) c1 = c_end;
    int64_t a = c0 * chunk_len, b = c1 * chunk_len;
    if (a > len) a = len;
    if (b > len) b = len;
    if (b < a) b = a;
    *t0 = a;
    *t1 = b;
}

// Ancestor visibility bits of a candidate tree (node i sees itself and its
// ancestors). Parent pointers that do not point strictly backwards are read
// as roots, so the walk is always in bounds.
__host__ __device__ inline uint64_t tree_bits_step(const uint64_t* done, int32_t i, int32_t parent) {
    uint64_t bits = (uint64_t)1 << i;
    if (parent >= 0 && parent < i) bits |= done[parent];
    return bits;
}

__host__ __device__ inline uint64_t chain_bits(int32_t i) {
    return i >= 63 ? ~(uint64_t)0 : (((uint64_t)1 << (i + 1)) - 1);
}

// ---------------------------------------------------------------------------
// Kernel parameter blocks (passed by value).
// ---------------------------------------------------------------------------

struct ChunkParams {
    const void* q;
    const void* k;
    const void* v;
    int64_t stride_b, stride_h, stride_t;
    const int64_t* req_offset;
    const int32_t* req_len;
    int32_t max_len;
    int32_t batch, n_q_heads, n_kv_heads, group, n_queries, rows;
    float scale;
    int32_t chunk_len, chunk_begin, n_chunks, cps, n_items;
    float* acc;
    float* m;
    float* l;
    int32_t slot_begin;
    int32_t row_blocks;  // VALU kernels: rows are split into blocks of kValuRows
};

struct CandParams {
    const void* q;
    const void* k;
    const void* v;
    int64_t stride_b, stride_h, stride_t;
    const int64_t* req_offset;
    int32_t batch, n_q_heads, n_kv_heads, group, n_queries, rows;
    float scale;
    const int32_t* parents;
    uint64_t* mask_out;
    float* acc;
    float* m;
    float* l;
    int32_t slot;
    int32_t row_blocks;
};

struct MergeParams {
    const float* acc;
    const float* m;
    const float* l;
    int32_t n_slots;
    const int32_t* slots_per_req;
    int32_t batch, n_queries, n_q_heads, head_dim;
    float* o;
    float* lse;
};

// Rows per work-group in the VALU kernels.
constexpr int kValuRows = 32;

// Launchers (defined in the kernel translation units).
hipError_t launch_chunk_valu(const ChunkParams& p, int dtype, int head_dim, hipStream_t stream);
hipError_t launch_chunk_mfma(const ChunkParams& p, int head_dim, hipStream_t stream);
hipError_t launch_chunk_mfma_wide(const ChunkParams& p, int head_dim, hipStream_t stream);
hipError_t launch_chunk_valu_small(const ChunkParams& p, int head_dim, hipStream_t stream);
hipError_t launch_candidates(const CandParams& p, int dtype, int head_dim, hipStream_t stream);
// Row blocks of the candidate kernel for `rows` rows per KV head.
int cand_row_blocks(int rows);
hipError_t launch_merge(const MergeParams& p, hipStream_t stream);

}  // namespace ssv
