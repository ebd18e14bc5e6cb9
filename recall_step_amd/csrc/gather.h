// Declarations of Stage Two, the gather of missed rows (not installed).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace avsg {

// Stage Two: 256-thread workgroups, rows resolved in passes of this size.
constexpr int kGatherThreads = 256;
constexpr int kGatherRowsPerPass = 256;
// Largest B * N_q the gather prologue scans in LDS.
constexpr int kMaxTokens = 16384;

enum GatherMode { kGatherByRow = 0, kGatherByRequest = 1, kGatherByTopk = 2 };

struct GatherArgs {
    const int32_t* __restrict__ n_miss;
    const int32_t* __restrict__ pairs;
    const int32_t* __restrict__ topk;        // by-top-K mode only
    const int8_t* __restrict__ hit_mask;     // by-top-K mode only
    const int32_t* __restrict__ slot_table;  // by-top-K mode only
    const int64_t* __restrict__ row_base;
    const int32_t* __restrict__ host_rows;
    const uint8_t* __restrict__ host;  // device alias of the pinned pool
    uint8_t* __restrict__ dev;
    int64_t host_rows_total;
    int32_t B, Nq, K, S, row_bytes, mode;
};

hipError_t launch_gather(const GatherArgs& a, int blocks, hipStream_t s);

}  // namespace avsg
