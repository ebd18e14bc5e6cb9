// Stage One of the recall step: hash matching, aging and slot assignment.
//
// Method: AVSG page ("AVSG: Accelerated Vectorized Sparse Gather for
// Efficient KV Cache Offload in Sparse-Attention LLM Serving"), section 3.3
// (three passes: refresh with pre-decay, classify, allocate; the Probe
// primitive), section 3.5 (per-slot lifetimes), section 3.6 (MTP tokens in
// sequence through one buffer) and Appendix B (single packed-word scatter,
// exhausted probes, slot preservation, speculative invalidation).
//
// gfx950 mapping.  One 1024-thread workgroup owns one request for the whole
// step.  Its bucket words and cached ids (int32) and its lifetimes (int8) are
// staged in LDS once, every query token runs against the LDS copy, and the
// state is written back once.  Each thread holds up to IPT consecutive ids of
// a token.  Block-wide steps use wave64 shuffles and ballots plus a 16-entry
// LDS carry: ordered miss compaction is an exclusive scan, the victim list is
// an exclusive scan of dead flags in slot order, and the lifetime histogram
// uses wave-aggregated LDS atomics.  Misses are sorted only when the token's
// ids do not already arrive ascending.  Contested buckets are resolved with an
// LDS atomicMax on the miss rank, so the result does not depend on wave
// scheduling.
#include "internal.h"

namespace avsg {
namespace {

constexpr int T = kStage1Threads;
constexpr int W = kStage1Waves;
constexpr int32_t kEmpty = -1;
constexpr int32_t kClaimBase = INT32_MIN;

__device__ inline int wave_incl_scan(int v) {
    const int lane = __lane_id();
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        int u = __shfl_up(v, d, 64);
        if (lane >= d) v += u;
    }
    return v;
}

// Exclusive scan of one int per thread over the workgroup; *total gets the
// sum.  scr needs W+1 ints and must not be in use by a scan still being read.
__device__ inline int block_excl_scan(int v, int32_t* scr, int* total) {
    const int lane = __lane_id();
    const int w = threadIdx.x >> 6;
    int incl = wave_incl_scan(v);
    if (lane == 63) scr[w] = incl;
    __syncthreads();
    if (w == 0) {
        int t = lane < W ? scr[lane] : 0;
        int ti = wave_incl_scan(t);
        if (lane < W) scr[lane] = ti - t;
        if (lane == W - 1) scr[W] = ti;
    }
    __syncthreads();
    *total = scr[W];
    return incl - v + scr[w];
}

__device__ inline int wave_sum(int v) {
#pragma unroll
    for (int d = 32; d > 0; d >>= 1) v += __shfl_xor(v, d, 64);
    return v;
}

__device__ inline uint32_t home_bucket(uint32_t x, uint32_t a1, uint32_t smask) {
    return (a1 * x) & smask;
}

__device__ inline uint32_t stride_of(uint32_t x, uint32_t a2, uint32_t smask) {
    return ((a2 * x) & smask) | 1u;
}

__device__ inline int32_t fp_of(uint32_t x, uint32_t afp) {
    return int32_t((x * afp) >> 17);
}

// Ascending bitonic sort of P (a power of two) 64-bit keys in LDS.
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

template <int IPT>
__global__ __launch_bounds__(T) void stage1_kernel(Stage1Args a) {
    extern __shared__ __align__(16) unsigned char smem[];
    const int S = a.S, K = a.K, L = a.L, R = a.R;
    const uint32_t smask = uint32_t(S) - 1u;
    const Stage1Layout lay = stage1_layout(S, K, L);
    int32_t* sQ = reinterpret_cast<int32_t*>(smem + lay.q);
    int32_t* sC = reinterpret_cast<int32_t*>(smem + lay.c);
    int8_t* sF = reinterpret_cast<int8_t*>(smem + lay.f);
    uint64_t* sKey = reinterpret_cast<uint64_t*>(smem + lay.key);
    int32_t* sVict = reinterpret_cast<int32_t*>(smem + lay.vict);
    int32_t* sHist = reinterpret_cast<int32_t*>(smem + lay.hist);
    int32_t* sScrA = reinterpret_cast<int32_t*>(smem + lay.scr);
    int32_t* sScrB = sScrA + 32;
    int32_t* sMisc = sScrA + 64;

    const int b = blockIdx.x;
    const int tid = threadIdx.x;
    const int lane = __lane_id();
    int32_t* gQ = a.Q + size_t(b) * S;
    int32_t* gC = a.C + size_t(b) * S;
    int32_t* gF = a.F + size_t(b) * S;

    // Stage the request's state; the once-per-step lifetime decay of the
    // first token is fused into the load (lifetimes of a valid state are in
    // [-1, L]; the clamp keeps histogram bins in range for any input).
    for (int j = tid; j < (S >> 2); j += T) {
        reinterpret_cast<int4*>(sQ)[j] = reinterpret_cast<const int4*>(gQ)[j];
        reinterpret_cast<int4*>(sC)[j] = reinterpret_cast<const int4*>(gC)[j];
        const int4 f = reinterpret_cast<const int4*>(gF)[j];
        char4 f8;
        f8.x = int8_t(min(max(f.x - 1, -1), L));
        f8.y = int8_t(min(max(f.y - 1, -1), L));
        f8.z = int8_t(min(max(f.z - 1, -1), L));
        f8.w = int8_t(min(max(f.w - 1, -1), L));
        reinterpret_cast<char4*>(sF)[j] = f8;
    }

    const int64_t rb = a.row_base[b];
    const int32_t hr = a.host_rows[b];
    const bool row_ok = rb >= 0 && hr >= 0 && rb + hr <= a.host_rows_total;
    const int32_t N = a.ctx_len[b];

    // This thread's contiguous slot range for S-wide passes.
    const int E = S >= T ? S / T : 1;
    const int j0 = tid * E;
    const bool has_slots = j0 < S;

    uint32_t c_hits = 0, c_look = 0, c_lcol = 0, c_lexh = 0, c_live = 0, c_visit = 0;
    uint32_t c_err = 0, c_miss = 0;

    if (tid == 0) sMisc[0] = 0;
    __syncthreads();

    for (int g = 0; g < a.Nq; ++g) {
        const size_t tok = size_t(b) * a.Nq + g;
        const int32_t* X = a.topk + tok * K;
        int32_t* O = a.slot_table + tok * K;
        int8_t* H = a.hit_mask + tok * K;
        const int i0 = tid * IPT;

        for (int k = tid; k < L + 2; k += T) sHist[k] = 0;

        // --- Pass 1/2: probe, refresh hits, classify -----------------------
        int32_t x[IPT];
        int32_t slot[IPT];
        uint32_t pos[IPT], dst[IPT];
        bool open[IPT], valid[IPT];
        bool any_open = false;
#pragma unroll
        for (int e = 0; e < IPT; ++e) {
            const int i = i0 + e;
            int32_t v = i < K ? X[i] : -1;
            const bool ok = v != -1 && row_ok && v >= 0 && v < hr;
            if (v != -1 && !ok) c_err |= 1u;
            x[e] = v;
            valid[e] = ok;
            open[e] = ok;
            slot[e] = -1;
            pos[e] = home_bucket(uint32_t(v), a.a1, smask);
            dst[e] = stride_of(uint32_t(v), a.a2, smask);
            any_open |= ok;
        }
        for (int t = 0; t <= R && any_open; ++t) {
            any_open = false;
#pragma unroll
            for (int e = 0; e < IPT; ++e) {
                if (open[e]) {
                    const int32_t wd = sQ[pos[e]];
                    const int32_t s = wd & int32_t(smask);
                    if (wd != kEmpty && sC[s] == x[e]) {
                        slot[e] = s;
                        open[e] = false;
                        c_visit += uint32_t(t + 1);
                    } else {
                        pos[e] = (pos[e] + dst[e]) & smask;
                        any_open = true;
                    }
                }
            }
        }
        int m_local = 0;
#pragma unroll
        for (int e = 0; e < IPT; ++e) {
            const int i = i0 + e;
            if (valid[e]) {
                ++c_look;
                if (slot[e] >= 0) {
                    sF[slot[e]] = int8_t(L);
                    O[i] = slot[e];
                    H[i] = 1;
                    ++c_hits;
                } else {
                    ++m_local;
                    c_visit += uint32_t(R + 1);
                }
            } else if (i < K) {
                O[i] = -1;
                H[i] = -1;
            }
        }

        // Ordered compaction of the misses into (id << 16 | position) keys.
        int ng = 0;
        int off = block_excl_scan(m_local, sScrA, &ng);
#pragma unroll
        for (int e = 0; e < IPT; ++e)
            if (valid[e] && slot[e] < 0)
                sKey[off++] = (uint64_t(uint32_t(x[e])) << 16) | uint64_t(i0 + e);
        if (tid == 0) a.n_miss[tok] = ng;
        c_miss += uint32_t(ng);
        __syncthreads();
        if (ng == 0) continue;

        // --- Misses in ascending id (sort only if not already ascending) ---
        int unsorted = 0;
        for (int r = tid; r + 1 < ng; r += T) unsorted |= sKey[r] > sKey[r + 1];
        {
            const uint64_t bal = __ballot(unsorted);
            if (lane == 0 && bal) sMisc[0] = 1;  // cleared below after use
        }
        __syncthreads();
        const bool need_sort = sMisc[0] != 0;
        if (need_sort) {
            const int P = next_pow2(ng);
            for (int r = ng + tid; r < P; r += T) sKey[r] = ~uint64_t(0);
            __syncthreads();
            if (tid == 0) sMisc[0] = 0;
            bitonic_sort(sKey, P);
        }
        for (int r = tid; r + 1 < ng; r += T)
            if ((sKey[r] >> 16) == (sKey[r + 1] >> 16)) c_err |= 2u;

        // --- Pass 3: least extra decay k* leaving ng dead slots ------------
        // Histogram of lifetimes over bins F+1 in [0, L+1], one wave-
        // aggregated LDS atomic per distinct bin per wave.
        for (int e = 0; e < E; ++e) {
            const int v = has_slots ? int(sF[j0 + e]) + 1 : -1;
            uint64_t active = __ballot(v >= 0);
            while (active) {
                const int leader = __ffsll((unsigned long long)active) - 1;
                const int bin = __shfl(v, leader, 64);
                const uint64_t m = __ballot(v == bin) & active;
                if (lane == leader) atomicAdd(&sHist[bin], __popcll(m));
                active &= ~m;
            }
        }
        __syncthreads();
        if (tid < 64) {
            // k* = least k with #{F < k} = sum(hist[0..k]) >= ng.
            int carry = 0, kstar = -1;
            for (int base = 0; base < L + 2 && kstar < 0; base += 64) {
                const int k = base + lane;
                const int hv = k < L + 2 ? sHist[k] : 0;
                const int cum = wave_incl_scan(hv) + carry;
                const uint64_t reach = __ballot(k < L + 2 && cum >= ng);
                if (reach) kstar = base + __ffsll((unsigned long long)reach) - 1;
                carry = __shfl(cum, 63, 64);
            }
            if (lane == 0) sMisc[1] = kstar < 0 ? L + 1 : kstar;
        }
        __syncthreads();
        const int kstar = sMisc[1];

        // Decay by k*, then CollectDead: the ng lowest-index dead slots.
        int dead_local = 0;
        if (has_slots) {
            for (int e = 0; e < E; ++e) {
                int f = sF[j0 + e];
                if (kstar) {
                    f = max(f - kstar, -1);
                    sF[j0 + e] = int8_t(f);
                }
                dead_local += f == -1;
            }
        }
        int dead_total = 0;
        int doff = block_excl_scan(dead_local, sScrB, &dead_total);
        if (has_slots && doff < ng) {
            for (int e = 0; e < E && doff < ng; ++e)
                if (sF[j0 + e] == -1) sVict[doff++] = j0 + e;
        }
        __syncthreads();

        // Install the r-th smallest miss into the r-th victim.
        for (int r = tid; r < ng; r += T) {
            const uint64_t key = sKey[r];
            const int32_t xv = int32_t(key >> 16);
            const int i = int(key & 0xFFFFu);
            const int32_t v = sVict[r];
            if (sC[v] >= 0) ++c_live;
            sC[v] = xv;
            sF[v] = int8_t(L);
            O[i] = v;
            H[i] = 0;
            reinterpret_cast<int2*>(a.pairs)[tok * K + r] = make_int2(xv, v);
        }
        __syncthreads();

        // Link: first reusable bucket in R+1 rounds, judged on the bucket
        // words before this token's writes and the slots after its installs.
        int32_t tgt[IPT];
#pragma unroll
        for (int k = 0; k < IPT; ++k) {
            const int r = tid + k * T;
            tgt[k] = -1;
            if (r < ng) {
                const uint32_t xv = uint32_t(sKey[r] >> 16);
                uint32_t p = home_bucket(xv, a.a1, smask);
                const uint32_t d = stride_of(xv, a.a2, smask);
                for (int t = 0; t <= R; ++t) {
                    const int32_t wd = sQ[p];
                    bool reusable = wd == kEmpty;
                    if (!reusable) {
                        const int32_t cached = sC[wd & int32_t(smask)];
                        reusable = cached == -1 || fp_of(uint32_t(cached), a.afp) != (wd >> 16);
                    }
                    if (reusable) {
                        tgt[k] = int32_t(p);
                        break;
                    }
                    p = (p + d) & smask;
                }
                if (tgt[k] < 0) ++c_lexh;
            }
        }
        __syncthreads();
#pragma unroll
        for (int k = 0; k < IPT; ++k)
            if (tgt[k] >= 0) sQ[tgt[k]] = kClaimBase;
        __syncthreads();
#pragma unroll
        for (int k = 0; k < IPT; ++k)
            if (tgt[k] >= 0) atomicMax(&sQ[tgt[k]], kClaimBase + 1 + tid + k * T);
        __syncthreads();
#pragma unroll
        for (int k = 0; k < IPT; ++k) {
            if (tgt[k] >= 0) {
                const int r = tid + k * T;
                if (sQ[tgt[k]] == kClaimBase + 1 + r) {
                    const uint32_t xv = uint32_t(sKey[r] >> 16);
                    sQ[tgt[k]] = (fp_of(xv, a.afp) << 16) | sVict[r];
                } else {
                    ++c_lcol;
                }
            }
        }
        __syncthreads();
    }

    // End of step: empty every slot caching a speculative id (>= N), then
    // write the state back (lifetimes widened to int32).
    for (int j = tid; j < (S >> 2); j += T) {
        int4 c = reinterpret_cast<const int4*>(sC)[j];
        if (c.x >= N) c.x = -1;
        if (c.y >= N) c.y = -1;
        if (c.z >= N) c.z = -1;
        if (c.w >= N) c.w = -1;
        reinterpret_cast<int4*>(gC)[j] = c;
        reinterpret_cast<int4*>(gQ)[j] = reinterpret_cast<const int4*>(sQ)[j];
        const char4 f8 = reinterpret_cast<const char4*>(sF)[j];
        reinterpret_cast<int4*>(gF)[j] = make_int4(f8.x, f8.y, f8.z, f8.w);
    }

    // Counters: wave sums, then one LDS atomic per wave and counter.
    int32_t* sCnt = sScrA + 64;  // sMisc area, 8 ints
    __syncthreads();
    if (tid < 8) sCnt[tid] = 0;
    __syncthreads();
    const uint32_t vals[6] = {c_hits, c_look, c_lcol, c_lexh, c_live, c_visit};
    const int idx[6] = {0, 1, 3, 4, 5, 7};
#pragma unroll
    for (int k = 0; k < 6; ++k) {
        const int s = wave_sum(int(vals[k]));
        if (lane == 0 && s) atomicAdd(&sCnt[idx[k]], s);
    }
    const uint64_t e1 = __ballot(c_err & 1u), e2 = __ballot(c_err & 2u);
    if (lane == 0 && (e1 || e2)) atomicOr(&sCnt[6], (e1 ? 1 : 0) | (e2 ? 2 : 0));
    __syncthreads();
    if (tid < 8) {
        int32_t* cnt = a.CNT + size_t(b) * 8;
        const uint32_t add = tid == 2 ? c_miss : uint32_t(sCnt[tid]);
        if (tid == 6)
            cnt[6] = cnt[6] | int32_t(add);
        else
            cnt[tid] = int32_t(uint32_t(cnt[tid]) + add);
    }
}

template <int IPT>
hipError_t launch_ipt(const Stage1Args& a, size_t lds, hipStream_t s) {
    hipLaunchKernelGGL(stage1_kernel<IPT>, dim3(a.B), dim3(T), lds, s, a);
    return hipGetLastError();
}

}  // namespace

hipError_t stage1_prepare(size_t lds_bytes) {
    hipError_t e;
    e = hipFuncSetAttribute(reinterpret_cast<const void*>(&stage1_kernel<1>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, int(lds_bytes));
    if (e != hipSuccess) return e;
    e = hipFuncSetAttribute(reinterpret_cast<const void*>(&stage1_kernel<2>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, int(lds_bytes));
    if (e != hipSuccess) return e;
    e = hipFuncSetAttribute(reinterpret_cast<const void*>(&stage1_kernel<4>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, int(lds_bytes));
    if (e != hipSuccess) return e;
    return hipFuncSetAttribute(reinterpret_cast<const void*>(&stage1_kernel<8>),
                               hipFuncAttributeMaxDynamicSharedMemorySize, int(lds_bytes));
}

hipError_t launch_stage1(const Stage1Args& a, size_t lds, hipStream_t s) {
    const int ipt = (a.K + T - 1) / T;
    if (ipt <= 1) return launch_ipt<1>(a, lds, s);
    if (ipt <= 2) return launch_ipt<2>(a, lds, s);
    if (ipt <= 4) return launch_ipt<4>(a, lds, s);
    return launch_ipt<8>(a, lds, s);
}

}  // namespace avsg
