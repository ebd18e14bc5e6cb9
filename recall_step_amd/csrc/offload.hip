// The "KV Offload" comparison point: no buffer reuse, every selected row is
// copied every step.
//
// Method: AVSG page, section 4.1 (KV Offload keeps the whole KV cache in
// host memory and transfers every activated entry at each decode step, with
// no reuse) and section 4.5 (it shares AVSG's device pool and host layout).
// The entry at position i of query token g lands in the request's slot
// g*K + i; every valid id is a miss, listed in position order, and the same
// Stage-Two kernels copy the rows.  The reuse state (Q, C, F) is untouched.
//
// gfx950 mapping.  One 256-thread workgroup per request; each thread owns a
// contiguous run of positions of a token so the miss list comes out in
// position order from one workgroup scan.
#include "internal.h"

namespace avsg {
namespace {

constexpr int T = 256;

__device__ inline int wave_incl_scan(int v) {
    const int lane = __lane_id();
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        int u = __shfl_up(v, d, 64);
        if (lane >= d) v += u;
    }
    return v;
}

__global__ __launch_bounds__(T) void offload_kernel(OffloadArgs a) {
    __shared__ int32_t sWave[T / 64 + 1];
    __shared__ int32_t sSum[2];
    const int b = blockIdx.x, tid = threadIdx.x, lane = __lane_id(), w = tid >> 6;
    const int64_t rb = a.row_base[b];
    const int32_t hr = a.host_rows[b];
    const bool row_ok = rb >= 0 && hr >= 0 && rb + hr <= a.host_rows_total;
    const int per = (a.K + T - 1) / T;
    const int i0 = min(tid * per, a.K), i1 = min(i0 + per, a.K);
    int looked = 0;
    uint32_t err = 0;
    for (int g = 0; g < a.Nq; ++g) {
        const size_t tok = size_t(b) * a.Nq + g;
        const int32_t* X = a.topk + tok * a.K;
        int cnt = 0;
        for (int i = i0; i < i1; ++i) {
            const int32_t x = X[i];
            const bool ok = x != -1 && row_ok && x >= 0 && x < hr;
            if (x != -1 && !ok) err |= 1u;
            cnt += ok;
        }
        const int incl = wave_incl_scan(cnt);
        if (lane == 63) sWave[w] = incl;
        __syncthreads();
        if (w == 0) {
            const int t = lane < T / 64 ? sWave[lane] : 0;
            const int ti = wave_incl_scan(t);
            if (lane < T / 64) sWave[lane] = ti - t;
            if (lane == T / 64 - 1) sWave[T / 64] = ti;
        }
        __syncthreads();
        int off = incl - cnt + sWave[w];
        const int total = sWave[T / 64];
        int2* P = reinterpret_cast<int2*>(a.pairs) + tok * a.K;
        for (int i = i0; i < i1; ++i) {
            const int32_t x = X[i];
            const bool ok = x != -1 && row_ok && x >= 0 && x < hr;
            const int32_t slot = g * a.K + i;
            a.slot_table[tok * a.K + i] = ok ? slot : -1;
            a.hit_mask[tok * a.K + i] = ok ? int8_t(0) : int8_t(-1);
            if (ok) P[off++] = make_int2(x, slot);
        }
        if (tid == 0) a.n_miss[tok] = total;
        looked += total;
        __syncthreads();
    }
    const uint64_t e = __ballot(err != 0u);
    if (tid == 0) sSum[0] = 0;
    __syncthreads();
    if (lane == 0 && e) atomicOr(&sSum[0], 1);
    __syncthreads();
    if (tid == 0) {
        int32_t* cnt = a.CNT + size_t(b) * 8;
        cnt[1] = int32_t(uint32_t(cnt[1]) + uint32_t(looked));
        cnt[2] = int32_t(uint32_t(cnt[2]) + uint32_t(looked));
        cnt[6] |= sSum[0];
    }
}

}  // namespace

hipError_t launch_offload(const OffloadArgs& a, hipStream_t s) {
    hipLaunchKernelGGL(offload_kernel, dim3(a.B), dim3(T), 0, s, a);
    return hipGetLastError();
}

}  // namespace avsg
