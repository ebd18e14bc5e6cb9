// The sort-merge matcher the AVSG page compares its hash matching against:
// exact reuse of cached token ids, no lifetimes and no hash table
// (GatherSelection, AVSG page section 2; the dual-pointer baseline of
// section 4.2).
//
// Per request and query token, in order: a valid selected id that some row
// caches is a hit and keeps that row (the lowest such row); rows not yet
// referenced in the step are free, and the token's misses in ascending
// (id, position) order take the free rows in ascending order.  At the end of
// the step rows caching an id >= N are emptied.  Q and F are not used.
//
// gfx950 mapping.  One 1024-thread workgroup per request.  The dual-pointer
// walk over two sorted lists becomes its parallel equivalent: the cached ids
// and the token's ids are each sorted as (id << 16 | index) keys with a
// bitonic network in LDS, and every selected id finds its cached row with a
// binary search of the sorted cache.  Free rows and miss ranks come from
// workgroup scans, so the result is independent of scheduling.
#include "internal.h"

namespace avsg {
namespace {

constexpr int T = kSortMergeThreads;
constexpr int W = T / 64;
constexpr uint64_t kNone = ~uint64_t(0);

__device__ inline int wave_incl_scan(int v) {
    const int lane = __lane_id();
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        int u = __shfl_up(v, d, 64);
        if (lane >= d) v += u;
    }
    return v;
}

// Exclusive scan over the workgroup; scr holds W + 1 ints.  Ends with a
// barrier, so scr may be reused at once.
__device__ inline int block_excl_scan(int v, int32_t* scr, int* total) {
    const int lane = __lane_id(), w = threadIdx.x >> 6;
    const int incl = wave_incl_scan(v);
    if (lane == 63) scr[w] = incl;
    __syncthreads();
    if (w == 0) {
        const int t = lane < W ? scr[lane] : 0;
        const int ti = wave_incl_scan(t);
        if (lane < W) scr[lane] = ti - t;
        if (lane == W - 1) scr[W] = ti;
    }
    __syncthreads();
    *total = scr[W];
    const int r = incl - v + scr[w];
    __syncthreads();
    return r;
}

__device__ void bitonic_sort(uint64_t* key, int P) {
    for (int k = 2; k <= P; k <<= 1) {
        for (int j = k >> 1; j > 0; j >>= 1) {
            for (int q = threadIdx.x; q < (P >> 1); q += T) {
                const int lo = 2 * q - (q & (j - 1));
                const int hi = lo + j;
                const bool up = (lo & k) == 0;
                const uint64_t a = key[lo];
                const uint64_t b = key[hi];
                if ((a > b) == up) {
                    key[lo] = b;
                    key[hi] = a;
                }
            }
            __syncthreads();
        }
    }
}

__global__ __launch_bounds__(T) void sort_merge_kernel(Stage1Args a) {
    extern __shared__ __align__(16) unsigned char smem[];
    const int S = a.S, K = a.K;
    const SortMergeLayout lay = sort_merge_layout(S, K);
    int32_t* sC = reinterpret_cast<int32_t*>(smem + lay.c);
    uint8_t* sRef = smem + lay.ref;
    uint64_t* sCk = reinterpret_cast<uint64_t*>(smem + lay.ckey);
    uint64_t* sXk = reinterpret_cast<uint64_t*>(smem + lay.xkey);
    int8_t* sMiss = reinterpret_cast<int8_t*>(smem + lay.flag);
    int32_t* sFree = reinterpret_cast<int32_t*>(smem + lay.free);
    int32_t* sScr = reinterpret_cast<int32_t*>(smem + lay.scr);

    const int b = blockIdx.x, tid = threadIdx.x;
    int32_t* gC = a.C + size_t(b) * S;
    const int64_t rb = a.row_base[b];
    const int32_t hr = a.host_rows[b];
    const bool row_ok = rb >= 0 && hr >= 0 && rb + hr <= a.host_rows_total;
    const int32_t N = a.ctx_len[b];
    const int PS = next_pow2(S), PK = next_pow2(K);

    for (int j = tid; j < S; j += T) {
        sC[j] = gC[j];
        sRef[j] = 0;
    }
    uint32_t c_hits = 0, c_look = 0, c_miss = 0, c_live = 0, c_err = 0;
    __syncthreads();

    for (int g = 0; g < a.Nq; ++g) {
        const size_t tok = size_t(b) * a.Nq + g;
        const int32_t* X = a.topk + tok * K;
        int32_t* O = a.slot_table + tok * K;
        int8_t* H = a.hit_mask + tok * K;

        // Sorted keys of the cached ids (as they stand before this token's
        // installs) and of the token's valid ids; invalid positions report
        // slot -1 / mask -1 now.
        for (int j = tid; j < PS; j += T)
            sCk[j] = (j < S && sC[j] >= 0) ? (uint64_t(uint32_t(sC[j])) << 16) | uint64_t(j)
                                            : kNone;
        int nv = 0;
        for (int i = tid; i < PK; i += T) {
            uint64_t key = kNone;
            if (i < K) {
                const int32_t x = X[i];
                const bool ok = x != -1 && row_ok && x >= 0 && x < hr;
                if (x != -1 && !ok) c_err |= 1u;
                if (ok) {
                    key = (uint64_t(uint32_t(x)) << 16) | uint64_t(i);
                    ++nv;
                } else {
                    O[i] = -1;
                    H[i] = -1;
                }
            }
            sXk[i] = key;
        }
        int nvalid;
        block_excl_scan(nv, sScr, &nvalid);
        c_look += uint32_t(nv);
        bitonic_sort(sCk, PS);
        bitonic_sort(sXk, PK);

        // Each sorted id looks itself up in the sorted cache.  Contiguous
        // ranges per thread keep the misses in ascending (id, position).
        const int per = (nvalid + T - 1) / T;
        const int r0 = min(tid * per, nvalid), r1 = min(r0 + per, nvalid);
        int nm = 0;
        for (int r = r0; r < r1; ++r) {
            const uint64_t key = sXk[r];
            const uint64_t want = key >> 16;
            int lo = 0, hi = PS;  // first cache key with id >= want
            while (lo < hi) {
                const int mid = (lo + hi) >> 1;
                if ((sCk[mid] >> 16) < want) lo = mid + 1; else hi = mid;
            }
            const int i = int(key & 0xFFFFu);
            if (lo < PS && sCk[lo] != kNone && (sCk[lo] >> 16) == want) {
                const int row = int(sCk[lo] & 0xFFFFu);
                O[i] = row;
                H[i] = 1;
                sRef[row] = 1;
                sMiss[r] = 0;
                ++c_hits;
            } else {
                sMiss[r] = 1;
                ++nm;
                if (r + 1 < nvalid && (sXk[r + 1] >> 16) == want) c_err |= 2u;
            }
        }
        int ng;
        int moff = block_excl_scan(nm, sScr, &ng);
        c_miss += uint32_t(nm);

        // Free rows (not referenced in this step so far), ascending.
        const int E = (S + T - 1) / T;
        const int j0 = min(tid * E, S), j1 = min(j0 + E, S);
        int nf = 0;
        for (int j = j0; j < j1; ++j) nf += sRef[j] == 0;
        int nfree;
        int foff = block_excl_scan(nf, sScr, &nfree);
        for (int j = j0; j < j1 && foff < ng; ++j)
            if (sRef[j] == 0) sFree[foff++] = j;
        __syncthreads();

        // Install the r-th smallest miss into the r-th free row.
        int2* P = reinterpret_cast<int2*>(a.pairs) + tok * K;
        for (int r = r0; r < r1; ++r) {
            if (!sMiss[r]) continue;
            const uint64_t key = sXk[r];
            const int32_t x = int32_t(key >> 16);
            const int i = int(key & 0xFFFFu);
            const int32_t row = moff < nfree ? sFree[moff] : 0;
            if (sC[row] >= 0) ++c_live;
            sC[row] = x;
            sRef[row] = 1;
            O[i] = row;
            H[i] = 0;
            P[moff] = make_int2(x, row);
            ++moff;
        }
        if (tid == 0) a.n_miss[tok] = ng;
        __syncthreads();
    }

    // End of step: empty rows caching a speculative id, write back.
    for (int j = tid; j < S; j += T) gC[j] = sC[j] >= N ? -1 : sC[j];

    // Counters: one LDS atomic per wave and counter.
    int32_t* sCnt = sScr + W + 1;
    if (tid < 8) sCnt[tid] = 0;
    __syncthreads();
    const uint32_t vals[4] = {c_hits, c_look, c_miss, c_live};
    const int idx[4] = {0, 1, 2, 5};
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        int s = int(vals[k]);
#pragma unroll
        for (int d = 32; d > 0; d >>= 1) s += __shfl_xor(s, d, 64);
        if (__lane_id() == 0 && s) atomicAdd(&sCnt[idx[k]], s);
    }
    const uint64_t e1 = __ballot(c_err & 1u), e2 = __ballot(c_err & 2u);
    if (__lane_id() == 0 && (e1 || e2)) atomicOr(&sCnt[6], (e1 ? 1 : 0) | (e2 ? 2 : 0));
    __syncthreads();
    if (tid < 8 && tid != 3 && tid != 4 && tid != 7) {
        int32_t* cnt = a.CNT + size_t(b) * 8;
        if (tid == 6)
            cnt[6] |= sCnt[6];
        else
            cnt[tid] = int32_t(uint32_t(cnt[tid]) + uint32_t(sCnt[tid]));
    }
}

}  // namespace

hipError_t sort_merge_prepare(size_t lds) {
    return hipFuncSetAttribute(reinterpret_cast<const void*>(&sort_merge_kernel),
                               hipFuncAttributeMaxDynamicSharedMemorySize, int(lds));
}

hipError_t launch_sort_merge(const Stage1Args& a, size_t lds, hipStream_t s) {
    hipLaunchKernelGGL(sort_merge_kernel, dim3(a.B), dim3(T), lds, s, a);
    return hipGetLastError();
}

}  // namespace avsg
