// Stage Two of the recall step: copy every missed KV row from pinned host
// memory into its device slot.
//
// Method: AVSG page, section 3.4 (each miss x_i moves from host position x_i
// to device slot o_i, read directly from host memory with no staging copy)
// and sections 1 / 4.3 (the missed rows are divided evenly across cores, not
// by request or by top-K position).
//
// gfx950 mapping.  A fixed grid of workgroups reads the host pool through its
// device-mapped address (zero-copy loads over the host link).  Every
// workgroup scans the per-token miss counts itself, so the total M never
// leaves the device and the grid needs no host decision; workgroup w then
// copies flat misses [w*M/G, (w+1)*M/G).  Rows are resolved 256 at a time into
// LDS (source and destination byte offsets), after which consecutive lanes
// move consecutive 16-byte chunks of a row: one wave reads 1 KiB of a row's
// contiguous host bytes per instruction.  One workgroup per CU and one
// 16-byte load per lane (about 1 MiB in flight) measured best on gfx950: the
// host link is saturated well before that, and more requests in flight (two,
// four or eight loads per lane, or twice the grid) made the same copy 1-15 %
// slower.
//
// The two partitions the page compares against share the copy loop: by
// request (workgroup w copies all misses of requests w, w+G, ...) and by
// top-K position (each token's K positions are cut into equal ranges, one per
// workgroup, and each range's misses are copied).  Results are identical;
// only the balance of work across workgroups differs.
#include "gather.h"

namespace avsg {
namespace {

constexpr int T = kGatherThreads;
constexpr int kUnroll = 1;

__device__ inline int wave_incl_scan(int v) {
    const int lane = __lane_id();
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        int u = __shfl_up(v, d, 64);
        if (lane >= d) v += u;
    }
    return v;
}

// Exclusive scan of one int per thread over a T-thread workgroup.
__device__ inline int block_excl_scan(int v, int32_t* sWave, int* total) {
    const int tid = threadIdx.x, lane = __lane_id(), w = tid >> 6;
    const int incl = wave_incl_scan(v);
    if (lane == 63) sWave[w] = incl;
    __syncthreads();
    if (w == 0) {
        const int t = lane < T / 64 ? sWave[lane] : 0;
        const int ti = wave_incl_scan(t);
        if (lane < T / 64) sWave[lane] = ti - t;
        if (lane == T / 64 - 1) sWave[T / 64] = ti;
    }
    __syncthreads();
    *total = sWave[T / 64];
    const int r = incl - v + sWave[w];
    __syncthreads();
    return r;
}

// Byte offsets of one miss (host id x of request bq into slot v), or a
// negative source for a row that must not be copied.
__device__ inline void row_offsets(const GatherArgs& a, int bq, int32_t x, int32_t v,
                                   int64_t* src, int64_t* dst) {
    const int64_t rb = a.row_base[bq];
    const int32_t hr = a.host_rows[bq];
    const bool ok = x >= 0 && x < hr && v >= 0 && v < a.S && rb >= 0 &&
                    rb + hr <= a.host_rows_total;
    *src = ok ? (rb + x) * int64_t(a.row_bytes) : int64_t(-1);
    *dst = (int64_t(bq) * a.S + v) * int64_t(a.row_bytes);
}

// A native 16-byte vector: an array of HIP's int4 (a struct around a union)
// can be left in scratch memory, where each load is waited for on its own.
typedef int i32x4 __attribute__((ext_vector_type(4)));

// Copy nrows rows whose byte offsets are in LDS, kUnroll 16-byte chunks per
// lane and pass.  The loads of a pass are unconditional (a rejected row
// reads row 0 of the pool, always in bounds) so all of them are in flight
// at once; only the stores are predicated.  No barrier at the end (a workgroup's last pass then retires
// without waiting for its stores): a caller that rewrites the offsets
// afterwards puts a barrier first.
__device__ inline void copy_rows(const GatherArgs& a, const int64_t* sSrc, const int64_t* sDst,
                                 int nrows) {
    const int cpr = a.row_bytes >> 4;  // 16-byte chunks per row
    const int items = nrows * cpr;
    for (int it0 = threadIdx.x; it0 < items; it0 += T * kUnroll) {
        i32x4 v[kUnroll];
        int64_t d[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const int it = it0 + u * T;
            const int itc = min(it, items - 1);
            const int row = itc / cpr;
            const int c = itc - row * cpr;
            const int64_t src = sSrc[row];
            v[u] = *reinterpret_cast<const i32x4*>(a.host + max(src, int64_t(0)) +
                                                   int64_t(c) * 16);
            d[u] = (it < items && src >= 0) ? sDst[row] + int64_t(c) * 16 : int64_t(-1);
        }
#pragma unroll
        for (int u = 0; u < kUnroll; ++u)
            if (d[u] >= 0) *reinterpret_cast<i32x4*>(a.dev + d[u]) = v[u];
    }
}

__global__ __launch_bounds__(T) void gather_kernel(GatherArgs a) {
    extern __shared__ int32_t sOff[];  // [ntok + 1] exclusive prefix of n
    __shared__ int64_t sSrc[kGatherRowsPerPass];
    __shared__ int64_t sDst[kGatherRowsPerPass];
    __shared__ int32_t sWave[T / 64 + 1];

    // An empty pool has no row to read (every miss is then out of range).
    if (a.host_rows_total <= 0) return;

    const int tid = threadIdx.x;
    const int ntok = a.B * a.Nq;

    // Exclusive scan of the miss counts, in chunks of T tokens.
    int carry = 0;
    for (int base = 0; base < ntok; base += T) {
        const int k = base + tid;
        const int v = k < ntok ? min(max(a.n_miss[k], 0), a.K) : 0;
        int tot;
        const int off = block_excl_scan(v, sWave, &tot);
        if (k < ntok) sOff[k] = carry + off;
        carry += tot;
    }
    if (tid == 0) sOff[ntok] = carry;
    __syncthreads();

    const int64_t M = carry;
    const int64_t lo = M * blockIdx.x / gridDim.x;
    const int64_t hi = M * (blockIdx.x + 1) / gridDim.x;

    for (int64_t base = lo; base < hi; base += kGatherRowsPerPass) {
        const int nrows = int(min<int64_t>(kGatherRowsPerPass, hi - base));
        for (int i = tid; i < nrows; i += T) {
            const int32_t m = int32_t(base + i);
            // Token of flat miss m: last k with sOff[k] <= m.
            int l = 0, h = ntok - 1;
            while (l < h) {
                const int mid = (l + h + 1) >> 1;
                if (sOff[mid] <= m) l = mid; else h = mid - 1;
            }
            const int tok = l;
            const int r = m - sOff[tok];
            const int2 pr = reinterpret_cast<const int2*>(a.pairs)[size_t(tok) * a.K + r];
            row_offsets(a, tok / a.Nq, pr.x, pr.y, &sSrc[i], &sDst[i]);
        }
        __syncthreads();
        copy_rows(a, sSrc, sDst, nrows);
        if (base + kGatherRowsPerPass < hi) __syncthreads();  // offsets rewritten next
    }
}

// Request-level assignment: workgroup w copies every miss of requests
// w, w + G, w + 2G, ...
__global__ __launch_bounds__(T) void gather_by_request_kernel(GatherArgs a) {
    __shared__ int64_t sSrc[kGatherRowsPerPass];
    __shared__ int64_t sDst[kGatherRowsPerPass];
    if (a.host_rows_total <= 0) return;
    for (int bq = blockIdx.x; bq < a.B; bq += gridDim.x) {
        for (int g = 0; g < a.Nq; ++g) {
            const size_t tok = size_t(bq) * a.Nq + g;
            const int n = min(max(a.n_miss[tok], 0), a.K);
            for (int base = 0; base < n; base += kGatherRowsPerPass) {
                const int nrows = min(kGatherRowsPerPass, n - base);
                for (int i = threadIdx.x; i < nrows; i += T) {
                    const int2 pr = reinterpret_cast<const int2*>(a.pairs)[tok * a.K + base + i];
                    row_offsets(a, bq, pr.x, pr.y, &sSrc[i], &sDst[i]);
                }
                __syncthreads();
                copy_rows(a, sSrc, sDst, nrows);
                __syncthreads();
            }
        }
    }
}

// Equal top-K partitioning: each token's K positions are cut into P ranges
// of equal length (P chosen so that B * N_q * P covers the grid); unit
// (token, range) goes to workgroup unit mod G, which copies the misses
// (hit_mask 0) found in its range from the top-K ids and the slot table.
__global__ __launch_bounds__(T) void gather_by_topk_kernel(GatherArgs a) {
    __shared__ int64_t sSrc[kGatherRowsPerPass];
    __shared__ int64_t sDst[kGatherRowsPerPass];
    __shared__ int32_t sWave[T / 64 + 1];
    if (a.host_rows_total <= 0) return;
    const int ntok = a.B * a.Nq;
    const int P = max(1, (int(gridDim.x) + ntok - 1) / ntok);
    const int len = (a.K + P - 1) / P;
    const int units = ntok * P;
    for (int u = blockIdx.x; u < units; u += gridDim.x) {
        const int tok = u / P;
        const int bq = tok / a.Nq;
        const int lo = (u - tok * P) * len;
        const int hi = min(a.K, lo + len);
        // Positions are taken T at a time (one per thread), misses
        // compacted into LDS, then copied.
        for (int base = lo; base < hi; base += T) {
            const int i = base + threadIdx.x;
            const size_t e = size_t(tok) * a.K + i;
            const bool miss = i < hi && a.hit_mask[e] == 0;
            int tot;
            const int off = block_excl_scan(miss ? 1 : 0, sWave, &tot);
            if (miss) row_offsets(a, bq, a.topk[e], a.slot_table[e], &sSrc[off], &sDst[off]);
            __syncthreads();
            // The next range's scan starts with a barrier, so its offsets
            // are written only after this copy has read them.
            if (tot > 0) copy_rows(a, sSrc, sDst, tot);
        }
    }
}

}  // namespace

hipError_t launch_gather(const GatherArgs& a, int blocks, hipStream_t s) {
    if (a.mode == kGatherByRequest) {
        hipLaunchKernelGGL(gather_by_request_kernel, dim3(blocks), dim3(T), 0, s, a);
    } else if (a.mode == kGatherByTopk) {
        hipLaunchKernelGGL(gather_by_topk_kernel, dim3(blocks), dim3(T), 0, s, a);
    } else {
        const size_t lds = size_t(a.B * a.Nq + 1) * sizeof(int32_t);
        hipLaunchKernelGGL(gather_kernel, dim3(blocks), dim3(T), lds, s, a);
    }
    return hipGetLastError();
}

}  // namespace avsg
