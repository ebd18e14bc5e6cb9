// Internal declarations shared by the library's HIP sources (not installed).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "avsg.h"
#include "gather.h"

namespace avsg {

// Stage One runs one workgroup per request of 256, 512 or 1024 threads (by
// default two ids per thread, 1024 threads from K = 2048); each thread holds
// up to kMaxIdsPerThread ids of a token.
constexpr int kMaxWaves = 16;
constexpr int kMaxIdsPerThread = 8;
// LDS one Stage-One workgroup may use (gfx950: 160 KiB per workgroup).
constexpr size_t kStage1LdsBudget = 160 * 1024;
// The miss-rank bitmap covers at most this many consecutive ids.
constexpr int kMaxBitmapIds = 1 << 18;
// Copies of the lifetime histogram (lane % kHistCopies picks one).
constexpr int kHistCopies = 16;


__host__ __device__ inline int next_pow2(int v) {
    int p = 1;
    while (p < v) p <<= 1;
    return p;
}

__host__ __device__ inline size_t round16(size_t v) { return (v + 15) & ~size_t(15); }

// LDS layout of the Stage-One workgroup, in bytes from the base.
//   q, c    int32 [S]  bucket words, cached ids
//   f       uint8 [S]  lifetimes as G = F + 1 (0 = dead)
//   vict    int32 [K]  victim slots (aliased by the uint16 rank-by-position
//                      table of the sorting fallback)
//   region  the larger of: uint64 [next_pow2(K)] sort keys; int2 [K] miss
//           list; the miss-rank bitmap (bitmap_words uint32) followed by
//           its per-word prefix counts (bitmap_words uint16)
//   hist    int32 [kHistCopies][L+2] lifetime histogram copies
//   scr     int32 [96]  reduction scratch, flags and counters
// total is 0 when even the smallest region does not fit the budget.
struct Stage1Layout {
    size_t q, c, f, vict, region, hist, scr, total;
    int bitmap_words;
};

__host__ __device__ inline Stage1Layout stage1_layout(int S, int K, int L) {
    Stage1Layout o;
    o.q = 0;
    o.c = o.q + size_t(S) * 4;
    o.f = o.c + size_t(S) * 4;
    o.vict = round16(o.f + size_t(S));
    o.region = round16(o.vict + size_t(K) * 4);
    const size_t tail = round16(size_t(kHistCopies) * (L + 2) * 4) + 96 * 4;
    const size_t keys = size_t(next_pow2(K)) * 8;
    size_t avail = o.region + tail < kStage1LdsBudget ? kStage1LdsBudget - o.region - tail : 0;
    size_t words = avail / 6;  // 4 bytes of bits + 2 bytes of prefix per word
    if (words > size_t(kMaxBitmapIds / 32)) words = kMaxBitmapIds / 32;
    words &= ~size_t(7);
    o.bitmap_words = int(words);
    const size_t region = keys > words * 6 ? keys : words * 6;
    o.hist = round16(o.region + region);
    o.scr = round16(o.hist + size_t(kHistCopies) * (L + 2) * 4);
    o.total = o.scr + 96 * 4;
    if (o.total > kStage1LdsBudget) o.total = 0;
    return o;
}

// Sort-merge comparison matcher: one 1024-thread workgroup per request.
constexpr int kSortMergeThreads = 1024;

// LDS layout of the sort-merge workgroup, in bytes from the base.
//   c     int32  [S]              cached ids
//   ref   uint8  [S]              row referenced in this step
//   ckey  uint64 [next_pow2(S)]   sorted (id << 16 | row) keys of the cache
//   xkey  uint64 [next_pow2(K)]   sorted (id << 16 | position) keys
//   flag  int8   [K]              miss flag per sorted id
//   free  int32  [K]              free rows, ascending
//   scr   int32  [64]             scan scratch and counters
// total is 0 when the layout does not fit the LDS budget.
struct SortMergeLayout {
    size_t c, ref, ckey, xkey, flag, free, scr, total;
};

__host__ __device__ inline SortMergeLayout sort_merge_layout(int S, int K) {
    SortMergeLayout o;
    o.c = 0;
    o.ref = size_t(S) * 4;
    o.ckey = round16(o.ref + size_t(S));
    o.xkey = o.ckey + size_t(next_pow2(S)) * 8;
    o.flag = o.xkey + size_t(next_pow2(K)) * 8;
    o.free = round16(o.flag + size_t(K));
    o.scr = round16(o.free + size_t(K) * 4);
    o.total = o.scr + 64 * 4;
    if (o.total > kStage1LdsBudget) o.total = 0;
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
    int32_t predecay;  // 1: apply the once-per-step lifetime decay first
    uint32_t a1, a2, afp;
    int32_t* __restrict__ map;  // dense matcher only: int32 [B][map_len]
    int64_t map_len;
};

struct OffloadArgs {
    int32_t* __restrict__ CNT;
    const int32_t* __restrict__ topk;
    const int64_t* __restrict__ row_base;
    const int32_t* __restrict__ host_rows;
    int32_t* __restrict__ slot_table;
    int8_t* __restrict__ hit_mask;
    int32_t* __restrict__ n_miss;
    int32_t* __restrict__ pairs;
    int64_t host_rows_total;
    int32_t B, Nq, K;
};

struct InitArgs {
    int32_t* Q;
    int32_t* C;
    int32_t* F;
    int32_t* CNT;
    const int32_t* row_mask;
    int32_t B, S;
    int32_t* map;  // NULL unless the dense matcher is configured
    int64_t map_len;
};

// Stage-One workgroup size: `requested` if nonzero, else chosen from K.
int stage1_threads(int K, int requested);
hipError_t stage1_prepare(size_t lds_bytes);
// dense: match through the id -> slot map instead of the hash table.
// grid: the most workgroups to launch (one per CU); with more requests than
// that, the hash matcher's workgroups each take several in turn.
hipError_t launch_stage1(const Stage1Args& a, int threads, int grid, size_t lds_bytes,
                         bool dense, hipStream_t s);
struct PrefetchArgs {
    const float* __restrict__ scores;  // [B][row_len]
    int64_t row_len;
    const int32_t* __restrict__ ctx_len;
    const float* __restrict__ theta;
    const int32_t* __restrict__ cap;
    int32_t* __restrict__ cand;        // [B][K]
    int32_t B, K;
};

struct EmaArgs {
    const float* __restrict__ kth;
    float* __restrict__ theta;
    float alpha;
    int32_t B;
};

hipError_t launch_offload(const OffloadArgs& a, hipStream_t s);
hipError_t launch_prefetch_select(const PrefetchArgs& a, hipStream_t s);
hipError_t launch_ema_threshold(const EmaArgs& a, hipStream_t s);
hipError_t sort_merge_prepare(size_t lds_bytes);
hipError_t launch_sort_merge(const Stage1Args& a, size_t lds_bytes, hipStream_t s);
hipError_t launch_state_init(const InitArgs& a, hipStream_t s);

// Everything a step needs besides its io: what a handle holds, or what the
// allocation-free entry point fills in per call.
struct StepContext {
    avsg_config cfg;
    avsg_buffers bufs;        // map / map_len cleared unless the dense matcher is on
    const uint8_t* host_dev;  // device alias of bufs.host_kv (NULL without a pool)
    size_t lds_bytes;         // Stage-One dynamic LDS of cfg
    int gather_blocks;
    int stage1_threads;
    int stage1_grid;          // most Stage-One workgroups: one per CU
    int32_t* ws_pairs;        // miss list [B][N_q][K][2] used when io->miss_pairs is NULL
};

// Records e as the thread's last HIP error and returns AVSG_EHIP.
int hip_fail(hipError_t e);
// Lets every Stage-One and sort-merge kernel instance use up to lds_bytes of
// dynamic LDS on the current device.
hipError_t prepare_kernels(size_t lds_bytes);
// AVSG_OK if bufs suits cfg (cfg already validated), else an AVSG_E* code.
int check_buffers(const avsg_config* cfg, const avsg_buffers* bufs);
// Fills *out for cfg and bufs on a device with `multiprocessors` CUs and
// `lds_limit` bytes of LDS per workgroup; resolves the host pool's device
// alias (a lookup, no allocation).
int fill_context(const avsg_config* cfg, const avsg_buffers* bufs, int multiprocessors,
                 size_t lds_limit, int32_t* ws_pairs, StepContext* out);
// Enqueue Stage One (predecay: the once-per-step decay first), Stage Two, or
// both; each checks the io fields it reads and returns an AVSG_E* code.
int run_match(const StepContext& x, const avsg_step_io* io, hipStream_t stream, bool predecay);
int run_gather(const StepContext& x, const avsg_step_io* io, hipStream_t stream);
int run_step(const StepContext& x, const avsg_step_io* io, hipStream_t stream);

}  // namespace avsg
