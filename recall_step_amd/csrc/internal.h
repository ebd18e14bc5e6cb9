// Internal declarations shared by the library's HIP sources (not installed).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace avsg {

// Stage One runs one 1024-thread workgroup (16 wave64s) per request.
constexpr int kStage1Threads = 1024;
constexpr int kStage1Waves = kStage1Threads / 64;
// Largest number of selected ids one Stage-One thread holds (K <= 8192).
constexpr int kMaxIdsPerThread = 8;

// Stage Two: 256-thread workgroups, rows resolved in passes of this size.
constexpr int kGatherThreads = 256;
constexpr int kGatherRowsPerPass = 64;
// Largest B * N_q the gather prologue scans in LDS.
constexpr int kMaxTokens = 16384;

__host__ __device__ inline int next_pow2(int v) {
    int p = 1;
    while (p < v) p <<= 1;
    return p;
}

__host__ __device__ inline size_t round16(size_t v) { return (v + 15) & ~size_t(15); }

// LDS layout of the Stage-One workgroup, in bytes from the base.
struct Stage1Layout {
    size_t q, c, f, key, vict, hist, scr, total;
};

__host__ __device__ inline Stage1Layout stage1_layout(int S, int K, int L) {
    Stage1Layout o;
    o.q = 0;                                   // int32 [S] bucket words
    o.c = o.q + size_t(S) * 4;                 // int32 [S] cached ids
    o.f = o.c + size_t(S) * 4;                 // int8  [S] lifetimes
    o.key = round16(o.f + size_t(S));          // uint64 [next_pow2(K)] miss keys
    o.vict = o.key + size_t(next_pow2(K)) * 8; // int32 [K] victim slots
    o.hist = round16(o.vict + size_t(K) * 4);  // int32 [L+2] lifetime histogram
    o.scr = round16(o.hist + size_t(L + 2) * 4);  // int32 [3][32] scan scratch
    o.total = o.scr + 3 * 32 * 4;
    return o;
}

struct Stage1Args {
    int32_t* __restrict__ Q;
    int32_t* __restrict__ C;
    int32_t* __restrict__ F;
    int32_t* __restrict__ CNT;
    const int32_t* __restrict__ topk;
    const int32_t* __restrict__ ctx_len;
    const int64_t* __restrict__ row_base;
    const int32_t* __restrict__ host_rows;
    int32_t* __restrict__ slot_table;
    int8_t* __restrict__ hit_mask;
    int32_t* __restrict__ n_miss;
    int32_t* __restrict__ pairs;
    int64_t host_rows_total;
    int32_t B, Nq, K, S, L, R;
    uint32_t a1, a2, afp;
};

struct GatherArgs {
    const int32_t* __restrict__ n_miss;
    const int32_t* __restrict__ pairs;
    const int64_t* __restrict__ row_base;
    const int32_t* __restrict__ host_rows;
    const uint8_t* __restrict__ host;  // device alias of the pinned pool
    uint8_t* __restrict__ dev;
    int64_t host_rows_total;
    int32_t B, Nq, K, S, row_bytes;
};

struct InitArgs {
    int32_t* Q;
    int32_t* C;
    int32_t* F;
    int32_t* CNT;
    const int32_t* row_mask;
    int32_t B, S;
};

hipError_t stage1_prepare(size_t lds_bytes);
hipError_t launch_stage1(const Stage1Args& a, size_t lds_bytes, hipStream_t s);
hipError_t launch_gather(const GatherArgs& a, int blocks, hipStream_t s);
hipError_t launch_state_init(const InitArgs& a, hipStream_t s);

}  // namespace avsg
