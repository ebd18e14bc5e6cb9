// Stage One of the recall step: hash matching, aging and slot assignment.
//
// Method: AVSG page ("AVSG: Accelerated Vectorized Sparse Gather for
// Efficient KV Cache Offload in Sparse-Attention LLM Serving"), section 3.3
// (three passes: refresh with pre-decay, classify, allocate; the Probe
// primitive), section 3.5 (per-slot lifetimes), section 3.6 (MTP tokens in
// sequence through one buffer) and Appendix B (single packed-word scatter,
// exhausted probes, slot preservation, speculative invalidation).
//
// gfx950 mapping.  One workgroup owns one request for the whole step (with
// more requests than CUs, one workgroup per CU takes several in turn, the
// next one's state loaded into registers while it works on the current).
// Its bucket words and cached ids (int32) and its lifetimes are staged in
// LDS once and every query token runs against the LDS copy.  Installs and links
// write their C and Q entries through to global memory as they happen, so
// the end of the step writes back only the lifetimes and the slots it
// empties.  Lifetimes are held as one byte per slot, G = F + 1 (0 = dead,
// L + 1 = just refreshed), so dead slots are zero bytes.
//
// A workgroup has 256 to 1024 threads, two ids per thread by default (up to
// eight).  The probe and link rounds wait on LDS, which more waves hide, but
// with four waves per SIMD every per-thread instruction is issued four times
// over, so the code keeps instruction counts low: branch-free rounds (every
// read from an always-valid index, results masked afterwards), DPP scans,
// one-barrier workgroup reductions, counters from ballots.
//
// Each thread owns IPT consecutive positions of a token's top-K list and
// carries their ids through the token: it probes them, refreshes its hits
// and, once it knows the rank of each of its misses among the token's misses
// (ascending id), installs them into the victim of that rank and writes its
// slot-table and hit-mask entries with vector stores.  The install leaves the
// misses in rank order in LDS, and the link runs over that list, one miss per
// lane (more only where a token has more misses than threads), so only as
// many waves as there are misses walk its rounds, each over just the ids its
// lanes hold: a round lasts one wave's chain of dependent instructions.  The rank
// comes from a bitmap held in LDS over [0, host rows) of the request (or, if
// those do not fit it, over [min id, max id] of the token's misses): one
// atomicOr per miss, then prefix popcounts over the words, so rank(x) =
// (misses below x's word) + popc(word bits below x); the same scan counts
// the misses.  When the ids span more than the bitmap or a missing id
// repeats, the token falls back to a bitonic sort of (id, position) keys.
//
// Victims: the dead-slot count is an exclusive scan over slots in index
// order; only when it is short of the miss count does the workgroup build a
// lifetime histogram (16 LDS copies to spread atomics) to find the least
// extra decay.  Contested buckets are resolved with an LDS atomicMin on
// claims encoded below every bucket word (the largest miss rank wins), so no
// result depends on wave scheduling.  Wave scans use DPP row shifts and row
// broadcasts; a workgroup scan needs one barrier.
#include "internal.h"

namespace avsg {
namespace {

constexpr int32_t kEmpty = -1;
constexpr int32_t kClaimBase = INT32_MIN;

// DPP controls (GFX9 encoding): row_shr:n = 0x110 + n, row_bcast:15 / :31.
#define AVSG_DPP_SCAN(x, OP, ID)                                                  \
    do {                                                                          \
        x = OP(x, __builtin_amdgcn_update_dpp(ID, x, 0x111, 0xf, 0xf, false));    \
        x = OP(x, __builtin_amdgcn_update_dpp(ID, x, 0x112, 0xf, 0xf, false));    \
        x = OP(x, __builtin_amdgcn_update_dpp(ID, x, 0x114, 0xf, 0xf, false));    \
        x = OP(x, __builtin_amdgcn_update_dpp(ID, x, 0x118, 0xf, 0xf, false));    \
        x = OP(x, __builtin_amdgcn_update_dpp(ID, x, 0x142, 0xa, 0xf, false));    \
        x = OP(x, __builtin_amdgcn_update_dpp(ID, x, 0x143, 0xc, 0xf, false));    \
    } while (0)

__device__ inline int op_add(int a, int b) { return a + b; }
__device__ inline int op_min(int a, int b) { return min(a, b); }
__device__ inline int op_max(int a, int b) { return max(a, b); }

// Inclusive wave64 scans.
__device__ inline int wave_scan_add(int x) { AVSG_DPP_SCAN(x, op_add, 0); return x; }
__device__ inline int wave_scan_min(int x) { AVSG_DPP_SCAN(x, op_min, INT32_MAX); return x; }
__device__ inline int wave_scan_max(int x) { AVSG_DPP_SCAN(x, op_max, INT32_MIN); return x; }
__device__ inline int lane63(int x) { return __builtin_amdgcn_readlane(x, 63); }

// Inclusive scans within each row of 16 lanes.
#define AVSG_DPP_ROW_SCAN(x, OP, ID)                                              \
    do {                                                                          \
        x = OP(x, __builtin_amdgcn_update_dpp(ID, x, 0x111, 0xf, 0xf, false));    \
        x = OP(x, __builtin_amdgcn_update_dpp(ID, x, 0x112, 0xf, 0xf, false));    \
        x = OP(x, __builtin_amdgcn_update_dpp(ID, x, 0x114, 0xf, 0xf, false));    \
        x = OP(x, __builtin_amdgcn_update_dpp(ID, x, 0x118, 0xf, 0xf, false));    \
    } while (0)
__device__ inline int row_scan_add(int x) { AVSG_DPP_ROW_SCAN(x, op_add, 0); return x; }
__device__ inline int row_scan_min(int x) { AVSG_DPP_ROW_SCAN(x, op_min, INT32_MAX); return x; }
__device__ inline int row_scan_max(int x) { AVSG_DPP_ROW_SCAN(x, op_max, INT32_MIN); return x; }

// Workgroup reductions below take the caller's lane index (0..63).

// Exclusive scan of one int per thread over the workgroup; *total gets the
// sum.  One barrier.  scr holds kMaxWaves ints; two consecutive workgroup
// operations must use different scratch buffers.
template <int T>
__device__ inline int block_excl_scan(int v, int32_t* scr, int* total, int lane) {
    constexpr int NW = T / 64;
    const int w = threadIdx.x >> 6;
    const int incl = wave_scan_add(v);
    if (lane == 63) scr[w] = incl;
    __syncthreads();
    // Lanes 0..NW-1 (NW <= 16: one DPP row) scan the wave totals; each wave
    // reads its prefix with one readlane.
    const int s = row_scan_add(lane < NW ? scr[lane] : 0);
    const int wu = __builtin_amdgcn_readfirstlane(w);
    const int pre = wu > 0 ? __builtin_amdgcn_readlane(s, wu - 1) : 0;
    *total = __builtin_amdgcn_readlane(s, NW - 1);
    return incl - v + pre;
}

// Workgroup sum of v.  One barrier; scr holds kMaxWaves ints.
template <int T>
__device__ inline int block_sum(int v, int32_t* scr, int lane) {
    constexpr int NW = T / 64;
    const int w = threadIdx.x >> 6;
    v = lane63(wave_scan_add(v));
    if (lane == 0) scr[w] = v;
    __syncthreads();
    return __builtin_amdgcn_readlane(row_scan_add(lane < NW ? scr[lane] : 0), NW - 1);
}

// Workgroup sum of v, min of lo and max of hi.  One barrier; scr holds
// 3 * kMaxWaves ints.
template <int T>
__device__ inline void block_sum_min_max(int v, int lo, int hi, int32_t* scr, int* sum,
                                         int* mn, int* mx, int lane) {
    constexpr int NW = T / 64;
    const int w = threadIdx.x >> 6;
    v = lane63(wave_scan_add(v));
    lo = lane63(wave_scan_min(lo));
    hi = lane63(wave_scan_max(hi));
    if (lane == 0) {
        scr[w] = v;
        scr[kMaxWaves + w] = lo;
        scr[2 * kMaxWaves + w] = hi;
    }
    __syncthreads();
    const int l = lane;
    const bool in = l < NW;
    *sum = __builtin_amdgcn_readlane(row_scan_add(in ? scr[l] : 0), NW - 1);
    *mn = __builtin_amdgcn_readlane(row_scan_min(in ? scr[kMaxWaves + l] : INT32_MAX), NW - 1);
    *mx = __builtin_amdgcn_readlane(row_scan_max(in ? scr[2 * kMaxWaves + l] : INT32_MIN), NW - 1);
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

// Dense-map entries are read and written at L2 (agent scope): the map lives
// in global memory and its maxima are taken with L2 atomics, so no access may
// be served from a stale L1 line.
__device__ inline int32_t map_load(const int32_t* p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ inline void map_store(int32_t* p, int32_t v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// Drop the entry of id if it still points at slot j.
__device__ inline void map_clear_if(int32_t* mrow, int64_t map_len, int32_t id, int32_t j) {
    if (id >= 0 && id < map_len && map_load(mrow + id) == j) map_store(mrow + id, -1);
}

// Probe rounds issued between two early-exit checks.
constexpr int kProbeUnroll = 4;

// 0x80 in every byte of x that is zero, 0 elsewhere (exact for all values).
__device__ inline uint32_t zero_bytes(uint32_t x) {
    return ~(((x & 0x7F7F7F7Fu) + 0x7F7F7F7Fu) | x) & 0x80808080u;
}

// Zero n LDS words (n a multiple of 4), one 16-byte store per thread and pass.
template <int T>
__device__ inline void clear_words(uint32_t* w, int n, int tid) {
    for (int k = tid; k < (n >> 2); k += T) reinterpret_cast<uint4*>(w)[k] = make_uint4(0, 0, 0, 0);
}

// Ascending bitonic sort of P (a power of two) 64-bit keys in LDS.
template <int T>
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

// IPT consecutive ids of one token starting at X[i0].  The loads are
// unconditional, from positions clamped to K - 1, and nothing selects or
// moves their results here, so the wait for them falls at the ids' first
// use; positions at or past K are masked to -1 there.
template <int IPT>
__device__ inline void load_ids(const int32_t* __restrict__ X, int i0, int K,
                                int32_t (&x)[IPT]) {
#pragma unroll
    for (int e = 0; e < IPT; ++e) x[e] = X[min(i0 + e, K - 1)];
}

template <int IPT>
__device__ inline void store_outputs(int32_t* __restrict__ O, int8_t* __restrict__ H, int i0,
                                     int K, bool vec, const int32_t (&o)[IPT],
                                     const int8_t (&h)[IPT]) {
    if (vec && i0 + IPT <= K) {
        if constexpr (IPT == 1) {
            O[i0] = o[0];
            H[i0] = h[0];
        } else if constexpr (IPT == 2) {
            *reinterpret_cast<int2*>(O + i0) = make_int2(o[0], o[1]);
            *reinterpret_cast<char2*>(H + i0) = make_char2(h[0], h[1]);
        } else {
#pragma unroll
            for (int q = 0; q < IPT / 4; ++q) {
                *reinterpret_cast<int4*>(O + i0 + 4 * q) =
                    make_int4(o[4 * q], o[4 * q + 1], o[4 * q + 2], o[4 * q + 3]);
                *reinterpret_cast<char4*>(H + i0 + 4 * q) =
                    make_char4(h[4 * q], h[4 * q + 1], h[4 * q + 2], h[4 * q + 3]);
            }
        }
    } else {
#pragma unroll
        for (int e = 0; e < IPT; ++e) {
            if (i0 + e < K) {
                O[i0 + e] = o[e];
                H[i0 + e] = h[e];
            }
        }
    }
}

// Set the bit of each miss x - base in the rank bitmap; a bit found set
// already (a missing id that repeats) raises the flag at flag[0].
template <int IPT>
__device__ inline void mark_misses(uint32_t* bits, int32_t* flag, const int32_t* x,
                                   uint32_t missm, int base, int lane) {
    bool dup = false;
#pragma unroll
    for (int e = 0; e < IPT; ++e) {
        if (missm & (1u << e)) {
            const uint32_t bit = uint32_t(x[e] - base);
            const uint32_t m = 1u << (bit & 31u);
            dup |= (atomicOr(&bits[bit >> 5], m) & m) != 0u;
        }
    }
    if (__ballot(dup) != 0ull && lane == 0) flag[0] = 1;
}

// Ranks of the token's misses (ascending id) from their marks in the
// bitmap over [idlo, idlo + 32 * nw4), nw4 a multiple of 4.  One exclusive
// scan of the words' bit counts, which also carries the dead-slot counts of
// the thread's lifetime words (refreshes done, installs not begun) packed
// above them: both totals stay below 2^16 (misses <= K <= 8192, S <= 16384),
// so the low half never carries.  If there are misses, prefix counts per
// word (uint16, four words per step), a barrier, and one lookup per miss.
// Returns the number of misses; every thread gets the same value.
template <int T, int IPT>
__device__ inline int rank_by_bitmap(const uint32_t* sBits, uint16_t* sPre, const uint32_t* sGw,
                                     int32_t* scr, int nw4, const int32_t* x, uint32_t missm,
                                     int idlo, int dw0, int dwn, int tid, int lane,
                                     int32_t* rank, int* dead_pre, int* dead_all) {
    const int wpt = ((nw4 >> 2) + T - 1) / T * 4;
    const int w0 = min(tid * wpt, nw4), w1 = min(w0 + wpt, nw4);
    int cnt = 0;
    for (int k = w0; k < w1; k += 4) {
        const uint4 q = *reinterpret_cast<const uint4*>(sBits + k);
        cnt += __popc(q.x) + __popc(q.y) + __popc(q.z) + __popc(q.w);
    }
    int dead_local = 0;
    for (int q = 0; q < dwn; ++q) dead_local += __popc(zero_bytes(sGw[dw0 + q]));
    int tot;
    int run = block_excl_scan<T>(cnt | (dead_local << 16), scr, &tot, lane);
    *dead_pre = run >> 16;
    *dead_all = tot >> 16;
    const int ng = tot & 0xFFFF;
    if (ng == 0) return 0;
    run &= 0xFFFF;
    for (int k = w0; k < w1; k += 4) {
        const uint4 q = *reinterpret_cast<const uint4*>(sBits + k);
        const uint32_t p0 = uint32_t(run);
        const uint32_t p1 = p0 + __popc(q.x);
        const uint32_t p2 = p1 + __popc(q.y);
        const uint32_t p3 = p2 + __popc(q.z);
        run = int(p3 + __popc(q.w));
        *reinterpret_cast<uint2*>(sPre + k) = make_uint2(p0 | (p1 << 16), p2 | (p3 << 16));
    }
    __syncthreads();
#pragma unroll
    for (int e = 0; e < IPT; ++e) {
        if (missm & (1u << e)) {
            const uint32_t bit = uint32_t(x[e] - idlo);
            const uint32_t wd = sBits[bit >> 5];
            rank[e] = int(sPre[bit >> 5]) + __popc(wd & ((1u << (bit & 31u)) - 1u));
        }
    }
    return ng;
}

// Four lifetimes F as G = F + gadd clamped to [0, L + 1], one byte each.
__device__ inline uint32_t lifetime_word(int4 f, int gadd, int L) {
    const uint32_t g0 = uint32_t(min(max(f.x + gadd, 0), L + 1));
    const uint32_t g1 = uint32_t(min(max(f.y + gadd, 0), L + 1));
    const uint32_t g2 = uint32_t(min(max(f.z + gadd, 0), L + 1));
    const uint32_t g3 = uint32_t(min(max(f.w + gadd, 0), L + 1));
    return g0 | (g1 << 8) | (g2 << 16) | (g3 << 24);
}

// Link rounds over the first NE of a thread's IPT misses: the first
// reusable bucket (empty, its slot empty, or its fingerprint not the slot's
// id's) in R+1 rounds, judged on the bucket words before this token's link
// writes.  Branch-free within a round; a wave leaves once none of its
// misses still searches.  A round's time is one wave's chain of dependent
// instructions, so a wave whose lanes search with their first NE ids only
// (ranks tid + e*T, e < NE; with at most T misses in a token, NE = 1 in
// every wave) walks the rounds over those, keeping the other ids' reads and
// tests out of the chain.
template <int NE, int IPT>
__device__ inline void link_rounds(const int32_t* sQ, const int32_t* sC, uint32_t (&lp)[IPT],
                                   const uint32_t (&ld)[IPT], int32_t (&tgt)[IPT],
                                   uint32_t& search, int R, uint32_t smask, uint32_t afp) {
    for (int t = 0; t <= R; ++t) {
        if (__ballot(search != 0u) == 0ull) break;
        int32_t wd[NE], cc[NE];
#pragma unroll
        for (int e = 0; e < NE; ++e) wd[e] = sQ[((search >> e) & 1u) ? lp[e] : 0u];
#pragma unroll
        for (int e = 0; e < NE; ++e) cc[e] = sC[wd[e] & int32_t(smask)];
        uint32_t takem = 0;
#pragma unroll
        for (int e = 0; e < NE; ++e)
            takem |= uint32_t((wd[e] == kEmpty) | (cc[e] == -1) |
                              (fp_of(uint32_t(cc[e]), afp) != (wd[e] >> 16)))
                     << e;
        takem &= search;
#pragma unroll
        for (int e = 0; e < NE; ++e) {
            tgt[e] = ((takem >> e) & 1u) ? int32_t(lp[e]) : tgt[e];
            lp[e] = (lp[e] + ld[e]) & smask;
        }
        search &= ~takem;
    }
}

// The kernel's arguments as the several-requests form reads its per-request
// ones (state bases, row tables, counters, B): through a pointer to the
// argument segment that the compiler cannot follow from one read to the
// next, so that those values are loaded where a request starts or is loaded
// ahead instead of being held in scalar registers across the token loop.
typedef __attribute__((address_space(4))) const Stage1Args ConstArgs;

template <bool MULTI>
struct RequestArgs {
    __device__ static const Stage1Args& get(const Stage1Args& a) { return a; }
};

template <>
struct RequestArgs<true> {
    __device__ static ConstArgs& get(const Stage1Args&) {
        ConstArgs* p = (ConstArgs*)__builtin_amdgcn_kernarg_segment_ptr();
        asm volatile("" : "+s"(p));
        return *p;
    }
};

// One staging pass: int4 words j0 + u*T (u < U) of Q, C and F into LDS.
// Branch-free so that all loads of a pass are in flight together: indices
// past the end are clamped to the last word, and the threads that clamp
// store that word's own value again.
template <int T, int U, bool DENSE>
__device__ inline void stage_pass(const int32_t* gQ, const int32_t* gC, const int32_t* gF,
                                  int32_t* sQ, int32_t* sC, uint32_t* sGw, int j0, int nq,
                                  int gadd, int L) {
    int4 q[U], c[U], f[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const int j = min(j0 + u * T, nq - 1);
        if constexpr (!DENSE) q[u] = reinterpret_cast<const int4*>(gQ)[j];
        c[u] = reinterpret_cast<const int4*>(gC)[j];
        f[u] = reinterpret_cast<const int4*>(gF)[j];
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const int j = min(j0 + u * T, nq - 1);
        if constexpr (!DENSE) reinterpret_cast<int4*>(sQ)[j] = q[u];
        reinterpret_cast<int4*>(sC)[j] = c[u];
        sGw[j] = lifetime_word(f[u], gadd, L);
    }
}

// DENSE: the dense id -> slot matcher.  A valid id (also below map_len) is
// a hit iff its map entry m is a slot in [0, S) that caches it; installs
// drop the victim's old entry if it still points at the victim, clear every
// missing id's entry, and after a barrier set it with an atomic maximum of
// the slot (repeated ids: the largest rank, whose victim is the largest
// slot, keeps it); invalidated slots drop their entries.  Q is neither read
// nor written and no bucket is linked.
template <int T, int IPT, bool DENSE, bool MULTI>
__global__ __launch_bounds__(T) void stage1_kernel(Stage1Args a) {
    extern __shared__ __align__(16) unsigned char smem[];
    const int S = a.S, K = a.K, L = a.L, R = a.R;
    const uint32_t smask = uint32_t(S) - 1u;
    const Stage1Layout lay = stage1_layout(S, K, L);
    int32_t* sQ = reinterpret_cast<int32_t*>(smem + lay.q);
    int32_t* sC = reinterpret_cast<int32_t*>(smem + lay.c);
    uint8_t* sG = smem + lay.f;
    uint32_t* sGw = reinterpret_cast<uint32_t*>(smem + lay.f);
    int32_t* sVict = reinterpret_cast<int32_t*>(smem + lay.vict);
    uint16_t* sRank = reinterpret_cast<uint16_t*>(smem + lay.vict);  // aliases sVict
    uint64_t* sKey = reinterpret_cast<uint64_t*>(smem + lay.region);
    uint32_t* sBits = reinterpret_cast<uint32_t*>(smem + lay.region);  // aliases sKey
    uint16_t* sPre = reinterpret_cast<uint16_t*>(smem + lay.region + size_t(lay.bitmap_words) * 4);
    int2* sPair = reinterpret_cast<int2*>(smem + lay.region);          // aliases sKey
    int32_t* sHist = reinterpret_cast<int32_t*>(smem + lay.hist);       // [16][L + 2]
    int32_t* sMM = reinterpret_cast<int32_t*>(smem + lay.scr);          // 3 * kMaxWaves
    int32_t* sS0 = sMM + 3 * kMaxWaves;                                  // kMaxWaves
    int32_t* sS1 = sS0 + kMaxWaves;                                      // kMaxWaves
    int32_t* sMisc = sS1 + kMaxWaves;                                    // flags, counters

    const int tid = threadIdx.x;
    const int lane = __lane_id();
    const int HB = L + 2;  // histogram bins: G in [0, L + 1]
    // Vector stores of a thread's IPT output positions need K % IPT == 0 and
    // base pointers aligned to the vector size.
    const bool vec = (K % IPT) == 0 &&
                     (reinterpret_cast<uintptr_t>(a.slot_table) % (4 * IPT)) == 0 &&
                     (reinterpret_cast<uintptr_t>(a.hit_mask) % IPT) == 0;
    const int i0 = tid * IPT;
    const int gadd = a.predecay ? 0 : 1;
    const int nq = S >> 2;  // int4 words per array

    // MULTI: a workgroup takes requests blockIdx.x, + gridDim.x, ... (the
    // grid is one workgroup per CU, fewer than the requests).  While it
    // works on one request, the next one's state (up to two int4 words per
    // array per thread), its first token's ids, counters and scalars are
    // loaded into registers, so that staging it is LDS stores only.  The
    // hash matcher only: the dense matcher's map loads would wait behind
    // them.  Otherwise a workgroup takes request blockIdx.x alone.
    constexpr bool kPrefetch = MULTI && !DENSE;
    int4 pq0 = make_int4(0, 0, 0, 0), pq1 = pq0, pc0 = pq0, pc1 = pq0, pf0 = pq0, pf1 = pq0;
    int64_t p_rb = 0;
    int32_t p_hr = 0, p_N = 0, p_cnt = 0;
    bool have_pre = false;  // uniform: this request's state is in the registers above
    int32_t xn[IPT];
    for (int b = blockIdx.x;;) {
        const int bn = b + int(gridDim.x);  // this workgroup's next request
        auto& A = RequestArgs<MULTI>::get(a);
        int32_t* gQ = A.Q + size_t(b) * S;
        int32_t* gC = A.C + size_t(b) * S;
        int32_t* gF = A.F + size_t(b) * S;
        int32_t* const mrow = DENSE ? a.map + size_t(b) * size_t(a.map_len) : nullptr;

        int64_t rb;
        int32_t hr, N, cnt_old;
        if (have_pre) {
            // The previous request's end and counters read LDS until here.
            __syncthreads();
            rb = int64_t(__builtin_amdgcn_readfirstlane(int32_t(uint64_t(p_rb)))) & 0xFFFFFFFFll;
            rb |= int64_t(__builtin_amdgcn_readfirstlane(int32_t(uint64_t(p_rb) >> 32))) << 32;
            hr = __builtin_amdgcn_readfirstlane(p_hr);
            N = __builtin_amdgcn_readfirstlane(p_N);
            cnt_old = p_cnt;
            const int ja = min(tid, nq - 1), jb = min(tid + T, nq - 1);
            reinterpret_cast<int4*>(sQ)[ja] = pq0;
            reinterpret_cast<int4*>(sC)[ja] = pc0;
            sGw[ja] = lifetime_word(pf0, gadd, L);
            if (nq > T) {
                reinterpret_cast<int4*>(sQ)[jb] = pq1;
                reinterpret_cast<int4*>(sC)[jb] = pc1;
                sGw[jb] = lifetime_word(pf1, gadd, L);
            }
        } else {
            // The request's scalars are read before anything else so that their
            // latency overlaps the staging loads.
            rb = A.row_base[b];
            hr = A.host_rows[b];
            N = A.ctx_len[b];

            // Stage the request's state.  The once-per-step decay before the
            // first token is fused into the load: G = max(F - 1, -1) + 1,
            // clamped to [0, L + 1] for any input.  A continuation of the step
            // (more query tokens after an earlier call) stages G = F + 1 without
            // the decay.  The first token's ids and the counters are loaded
            // first, so that their latency overlaps the state's loads: up to two
            // passes of staging are straight-line code, with no loop head that
            // would wait for them.
            load_ids<IPT>(a.topk + size_t(b) * a.Nq * K, i0, K, xn);
            cnt_old = A.CNT[size_t(b) * 8 + min(tid, 7)];  // used by tid < 8
            if (nq <= T) {
                stage_pass<T, 1, DENSE>(gQ, gC, gF, sQ, sC, sGw, tid, nq, gadd, L);
            } else if (nq <= 2 * T) {
                stage_pass<T, 2, DENSE>(gQ, gC, gF, sQ, sC, sGw, tid, nq, gadd, L);
            } else {
                for (int j0 = tid; j0 < nq; j0 += 2 * T)
                    stage_pass<T, 2, DENSE>(gQ, gC, gF, sQ, sC, sGw, j0, nq, gadd, L);
            }
        }
        // Whether the next request's state is loaded ahead, during this one.
        const bool prefetch_next = kPrefetch && bn < A.B && nq <= 2 * T;

        const bool row_ok = rb >= 0 && hr >= 0 && rb + hr <= A.host_rows_total;
        // The rank bitmap can cover all of the request's ids.
        const bool narrow_rows = row_ok && hr > 0 && hr <= lay.bitmap_words * 32;

        // Each thread's contiguous run of D lifetime words (4 slots each) for the
        // S-wide passes starts at word tid * D (taken per token below).
        const int nd = S >> 2;
        const int D = nd >= T ? nd / T : 1;  // <= 16: S <= 16384 fits LDS, T >= 256

        // Counters: c_miss is a workgroup total (the same in every thread);
        // c_lcol, c_lexh and c_live are wave totals (from ballots); c_look and
        // c_visit are per thread.  Hits are lookups less misses.
        uint32_t c_look = 0, c_miss = 0;
        uint32_t c_lcol = 0, c_lexh = 0, c_live = 0;
        uint32_t c_visit = 0, c_err = 0;

        // The staging waits have returned every load issued before them.  Using
        // the first token's ids and the old counters here tells the compiler so;
        // otherwise the token loop's head waits for them on every token, and on
        // later tokens that wait also drains the previous token's stores.
    #pragma unroll
        for (int e = 0; e < IPT; ++e) asm volatile("" ::"v"(xn[e]));
        asm volatile("" ::"v"(cnt_old));

        // The rank bitmap starts every token clear: it is cleared here, while
        // the staging loads are in flight, and again after each token that used
        // it, so the rank pass needs no clear and barrier of its own.
        clear_words<T>(sBits, lay.bitmap_words, tid);
        if (tid == 0) sMisc[0] = 0;      // repeated-id flag
        if (tid < 8) sMisc[2 + tid] = 0;  // the counters' workgroup sums, taken at the end
        __syncthreads();

        // N_q >= 1: a do-while leaves no path on which the loop body is skipped,
        // so no load issued before it can still be pending after it.
        bool region_dirty = false;  // dense matcher: the last token used the bitmap region
        int g = 0;
        do {
            // The thread's indices are taken through an opaque copy in each
            // token, so that conditions on them (tid == 0, lane == 63, i0 + e <
            // K, ...) are evaluated where they are used instead of being hoisted
            // out of the loop as 64-bit lane masks, which would take the scalar
            // registers the loop needs and spill them.
            int tid_t = tid;
            asm volatile("" : "+v"(tid_t));
            const int lane_t = tid_t & 63;
            const int i0_t = tid_t * IPT;
            const int dw0_t = tid_t * D;
            const int dwn_t = dw0_t < nd ? D : 0;
            const size_t tok = size_t(b) * a.Nq + g;
            int32_t* O = a.slot_table + tok * K;
            int8_t* H = a.hit_mask + tok * K;

            // The dense matcher reads the pairs until the previous token's last
            // barrier, so it clears the bitmap here instead.
            if constexpr (DENSE)
                if (region_dirty) clear_words<T>(sBits, lay.bitmap_words, tid_t);

            int32_t x[IPT];
    #pragma unroll
            for (int e = 0; e < IPT; ++e) x[e] = i0_t + e < K ? xn[e] : -1;
            // The next token's ids: on the last token, the first token's of the
            // next request when it is loaded ahead, else its own again, unused.
            load_ids<IPT>(a.topk + (g + 1 < a.Nq      ? tok + 1
                                    : prefetch_next ? size_t(bn) * a.Nq
                                                    : tok) * K,
                          i0_t, K, xn);

            for (int k = tid_t; k < kHistCopies * HB; k += T) sHist[k] = 0;

            // --- Pass 1/2: probe, refresh hits, classify -----------------------
            int32_t slot[IPT];
            uint32_t pos[IPT], dst[IPT];
            uint32_t valid = 0;
    #pragma unroll
            for (int e = 0; e < IPT; ++e) {
                const int32_t v = x[e];
                const bool ok = v != -1 && row_ok && v >= 0 && v < hr && (!DENSE || v < a.map_len);
                if (v != -1 && !ok) c_err |= 1u;
                valid |= uint32_t(ok) << e;
                slot[e] = -1;
                pos[e] = home_bucket(uint32_t(v), a.a1, smask);
                dst[e] = stride_of(uint32_t(v), a.a2, smask);
            }
            // Rounds in lock step over the thread's ids, every bucket word of a
            // round loaded before any cached id, so the LDS round trips of all
            // IPT ids overlap.  Every read is issued for every id (bucket and
            // slot indices are always in [0, S)) and the open mask selects the
            // results afterwards: branch-free rounds cost fewer instructions than
            // masking each read.
            uint32_t open = valid;
            if constexpr (DENSE) {
                int32_t m[IPT], cc[IPT];
    #pragma unroll
                for (int e = 0; e < IPT; ++e)
                    m[e] = ((valid >> e) & 1u) ? map_load(mrow + x[e]) : -1;
    #pragma unroll
                for (int e = 0; e < IPT; ++e) cc[e] = (m[e] >= 0 && m[e] < S) ? sC[m[e]] : -2;
    #pragma unroll
                for (int e = 0; e < IPT; ++e) {
                    const bool hit = ((valid >> e) & 1u) && cc[e] == x[e];
                    slot[e] = hit ? m[e] : slot[e];
                    open &= ~(uint32_t(hit) << e);
                }
                c_visit += uint32_t(__popc(valid));
            }
            // The wave leaves the loop once none of its ids is open, checked
            // every kProbeUnroll rounds so that the reads of those rounds can be
            // in flight together (bucket positions do not depend on results).
            for (int t0 = 0; t0 <= (DENSE ? -1 : R); t0 += kProbeUnroll) {
                if (__ballot(open != 0u) == 0ull) break;
    #pragma unroll
                for (int u = 0; u < kProbeUnroll; ++u) {
                    if (t0 + u > R) break;
                    c_visit += uint32_t(__popc(open));
                    // Closed ids read bucket 0 (and so the slot its word names):
                    // one address shared by many lanes is a broadcast, not a
                    // bank conflict, and the round stays branch-free.
                    int32_t wd[IPT], cc[IPT];
    #pragma unroll
                    for (int e = 0; e < IPT; ++e) wd[e] = sQ[((open >> e) & 1u) ? pos[e] : 0u];
    #pragma unroll
                    for (int e = 0; e < IPT; ++e) cc[e] = sC[wd[e] & int32_t(smask)];
                    // Hit bits of every id first, masked by the open ids after,
                    // so that no read is moved under a branch.
                    uint32_t hitm = 0;
    #pragma unroll
                    for (int e = 0; e < IPT; ++e)
                        hitm |= uint32_t((wd[e] != kEmpty) & (cc[e] == x[e])) << e;
                    hitm &= open;
    #pragma unroll
                    for (int e = 0; e < IPT; ++e) {
                        slot[e] = ((hitm >> e) & 1u) ? (wd[e] & int32_t(smask)) : slot[e];
                        pos[e] = (pos[e] + dst[e]) & smask;
                    }
                    open &= ~hitm;
                }
            }
            // The next token's ids are consumed here, before this token issues
            // any store: waiting for a load still in flight at the token's end
            // would also wait for all of the token's stores.
    #pragma unroll
            for (int e = 0; e < IPT; ++e) asm volatile("" ::"v"(xn[e]));
            // The next request's state, scalars and counters, loaded now that
            // no wait in this token is left behind them: they are first needed
            // when this request is done.
            if (g == 0 && prefetch_next) {
                const int ja = min(tid_t, nq - 1), jb = min(tid_t + T, nq - 1);
                auto& An = RequestArgs<MULTI>::get(a);
                const int4* nQ = reinterpret_cast<const int4*>(An.Q + size_t(bn) * S);
                const int4* nC = reinterpret_cast<const int4*>(An.C + size_t(bn) * S);
                const int4* nF = reinterpret_cast<const int4*>(An.F + size_t(bn) * S);
                pq0 = nQ[ja];
                pc0 = nC[ja];
                pf0 = nF[ja];
                if (nq > T) {
                    pq1 = nQ[jb];
                    pc1 = nC[jb];
                    pf1 = nF[jb];
                }
                p_rb = An.row_base[bn];
                p_hr = An.host_rows[bn];
                p_N = An.ctx_len[bn];
                p_cnt = An.CNT[size_t(bn) * 8 + min(tid_t, 7)];
            }
            // open now holds exactly the valid misses.
            const uint32_t missm = open;
            int lo_local = INT32_MAX, hi_local = INT32_MIN;
    #pragma unroll
            for (int e = 0; e < IPT; ++e) {
                if (missm & (1u << e)) {
                    lo_local = min(lo_local, x[e]);
                    hi_local = max(hi_local, x[e]);
                } else if (valid & (1u << e)) {
                    sG[slot[e]] = uint8_t(L + 1);
                }
            }
            const int m_local = __popc(missm);

            c_look += uint32_t(__popc(valid));

            // --- Rank of each miss among the token's misses, ascending id ------
            int32_t rank[IPT];
    #pragma unroll
            for (int e = 0; e < IPT; ++e) rank[e] = -1;
            // Dead-slot prefix and total, when the rank scan counted them (-1:
            // not counted).
            int dead_pre = -1, dead_all = -1;
            int ng = 0;
            bool sorted_rank = false;  // the general-order sort ranks the misses
            if (!DENSE && narrow_rows) {
                // The bitmap spans [0, host_rows), which holds every valid id:
                // the misses are marked at once, and after one barrier the rank
                // scan also yields their count.  (The dense matcher clears the
                // bitmap at the token's start with no barrier before this point,
                // so it takes the other branch.)
                mark_misses<IPT>(sBits, sMisc, x, missm, 0, lane_t);
                __syncthreads();
                if (sMisc[0] == 0) {
                    const int nw4 = int(((uint32_t(hr) + 31u) >> 5) + 3) & ~3;
                    ng = rank_by_bitmap<T, IPT>(sBits, sPre, sGw, sS0, nw4, x, missm, 0, dw0_t,
                                                dwn_t, tid_t, lane_t, rank, &dead_pre, &dead_all);
                } else {
                    sorted_rank = true;  // a missing id repeats
                }
            } else {
                // Miss count (at most K < 2^16) and, unless the bitmap spans the
                // request's rows, the id range of the misses.
                int idlo = 0, idhi = hr - 1;
                if (narrow_rows)
                    ng = block_sum<T>(m_local, sMM, lane_t);
                else
                    block_sum_min_max<T>(m_local, lo_local, hi_local, sMM, &ng, &idlo, &idhi,
                                         lane_t);
                if (ng > 0) {
                    const uint32_t span = uint32_t(idhi) - uint32_t(idlo) + 1u;  // ids >= 0
                    sorted_rank = span > uint32_t(lay.bitmap_words) * 32u;
                    if (!sorted_rank) {
                        mark_misses<IPT>(sBits, sMisc, x, missm, idlo, lane_t);
                        __syncthreads();
                        sorted_rank = sMisc[0] != 0;
                        if (!sorted_rank) {
                            const int nw4 = int(((span + 31u) >> 5) + 3) & ~3;
                            rank_by_bitmap<T, IPT>(sBits, sPre, sGw, sS0, nw4, x, missm, idlo,
                                                   dw0_t, dwn_t, tid_t, lane_t, rank,
                                                   &dead_pre, &dead_all);
                        }
                    }
                }
            }
            if (sorted_rank) {
                // General order: bitonic sort of (id << 16 | position) keys.  The
                // scan that places the keys also counts the misses.
                int off = block_excl_scan<T>(m_local, sS1, &ng, lane_t);
    #pragma unroll
                for (int e = 0; e < IPT; ++e)
                    if (missm & (1u << e))
                        sKey[off++] = (uint64_t(uint32_t(x[e])) << 16) | uint64_t(i0_t + e);
                const int P = next_pow2(ng);
                for (int r = ng + tid_t; r < P; r += T) sKey[r] = ~uint64_t(0);
                __syncthreads();
                bitonic_sort<T>(sKey, P);
                for (int r = tid_t; r < ng; r += T) {
                    const uint64_t k = sKey[r];
                    sRank[int(k & 0xFFFFu)] = uint16_t(r);
                    if (r + 1 < ng && (k >> 16) == (sKey[r + 1] >> 16)) c_err |= 2u;
                }
                __syncthreads();
    #pragma unroll
                for (int e = 0; e < IPT; ++e)
                    if (missm & (1u << e)) rank[e] = int(sRank[i0_t + e]);
            }
            c_miss += uint32_t(ng);

            if (ng > 0) {
                // --- Pass 3: victims ---------------------------------------------
                // Dead slots now; if fewer than ng, the least extra decay k* with
                // #{F < k*} >= ng, applied to every slot.
                // Each thread reads its own lifetime words from LDS in every pass
                // (loops bounded by its word count; no register copy).
                int dead_local = 0;
                int dead_total = dead_all;
                int doff = dead_pre;
                if (dead_all < 0) {
                    for (int q = 0; q < dwn_t; ++q)
                        dead_local += __popc(zero_bytes(sGw[dw0_t + q]));
                    doff = block_excl_scan<T>(dead_local, sS0, &dead_total, lane_t);
                }
                if (dead_total < ng) {
                    // Histogram of G over 16 LDS copies (lane_t % 16 picks one).
                    int32_t* hc = sHist + (lane_t & (kHistCopies - 1)) * HB;
                    for (int q = 0; q < dwn_t; ++q) {
                        const uint32_t gq = sGw[dw0_t + q];
                        atomicAdd(&hc[gq & 0xFFu], 1);
                        atomicAdd(&hc[(gq >> 8) & 0xFFu], 1);
                        atomicAdd(&hc[(gq >> 16) & 0xFFu], 1);
                        atomicAdd(&hc[gq >> 24], 1);
                    }
                    __syncthreads();
                    if (tid_t < 64) {
                        // k* = least k with #{F < k} = #{G <= k} >= ng.
                        int carry = 0, kstar = -1;
                        for (int base = 0; base < HB && kstar < 0; base += 64) {
                            const int k = base + lane_t;
                            int hv = 0;
                            if (k < HB)
                                for (int c = 0; c < kHistCopies; ++c) hv += sHist[c * HB + k];
                            const int cum = wave_scan_add(hv) + carry;
                            const uint64_t reach = __ballot(k < HB && cum >= ng);
                            if (reach) kstar = base + __ffsll((unsigned long long)reach) - 1;
                            carry = lane63(cum);
                        }
                        if (lane_t == 0) sMisc[1] = kstar < 0 ? L + 1 : kstar;
                    }
                    __syncthreads();
                    const uint32_t kstar = uint32_t(sMisc[1]);
                    dead_local = 0;
                    for (int q = 0; q < dwn_t; ++q) {
                        const uint32_t gq = sGw[dw0_t + q];
                        uint32_t r = 0;
    #pragma unroll
                        for (int j = 0; j < 4; ++j) {
                            const uint32_t v = (gq >> (8 * j)) & 0xFFu;
                            r |= (v > kstar ? v - kstar : 0u) << (8 * j);
                        }
                        sGw[dw0_t + q] = r;
                        dead_local += __popc(zero_bytes(r));
                    }
                    doff = block_excl_scan<T>(dead_local, sS1, &dead_total, lane_t);
                }
                // CollectDead: the ng lowest-index dead slots, in slot order.
                for (int q = 0; q < dwn_t && doff < ng; ++q) {
                    uint32_t z = zero_bytes(sGw[dw0_t + q]);
                    while (z && doff < ng) {
                        const int j = (__ffs(int(z)) - 1) >> 3;
                        sVict[doff++] = (dw0_t + q) * 4 + j;
                        z &= z - 1u;
                    }
                }
                // Besides publishing the victims, this barrier keeps the install's
                // pairs (sPair aliases the rank bitmap and its prefix counts) from
                // overwriting words that a slower thread still reads for a rank.
                __syncthreads();

                // --- Install the r-th smallest miss into the r-th victim ---------
                uint32_t livem = 0;
    #pragma unroll
                for (int e = 0; e < IPT; ++e) {
                    if (missm & (1u << e)) {
                        const int r = min(max(rank[e], 0), ng - 1);
                        const int32_t v = sVict[r];
                        const int32_t old = sC[v];
                        livem |= uint32_t(old >= 0) << e;
                        if constexpr (DENSE) {
                            map_clear_if(mrow, a.map_len, old, v);
                            map_store(mrow + x[e], -1);
                        }
                        sC[v] = x[e];
                        gC[v] = x[e];  // written through: C is not written back in full
                        sG[v] = uint8_t(L + 1);
                        slot[e] = v;
                        sPair[r] = make_int2(x[e], v);
                    }
                }
    #pragma unroll
                for (int e = 0; e < IPT; ++e)
                    c_live += uint32_t(__popcll(__ballot((livem >> e) & 1u)));
                __syncthreads();

                if constexpr (DENSE) {
    #pragma unroll
                    for (int e = 0; e < IPT; ++e)
                        if (missm & (1u << e))
                            __hip_atomic_fetch_max(mrow + x[e], slot[e], __ATOMIC_RELAXED,
                                                   __HIP_MEMORY_SCOPE_AGENT);
                    // Miss list (id, slot) in rank order.
                    int2* P = reinterpret_cast<int2*>(a.pairs) + tok * K;
                    for (int r = tid_t; r < ng; r += T) P[r] = sPair[r];
                } else {
                    // --- Link: first reusable bucket in R+1 rounds, judged on the
                    // bucket words before this token's writes and the slots after its
                    // installs; one scatter, the largest rank keeps a contested bucket.
                    // Thread tid_t links the misses of rank tid_t + e*T, read from the
                    // rank-ordered pairs: the ng misses fill the first waves one per
                    // lane_t and the other waves leave at the first round, where a
                    // link by the owning thread keeps every wave walking the rounds.
                    int32_t lx[IPT], ls[IPT], tgt[IPT];
                    uint32_t lp[IPT], ld[IPT];
                    uint32_t search = 0;
    #pragma unroll
                    for (int e = 0; e < IPT; ++e) {
                        const int r = tid_t + e * T;
                        const int2 pr = r < ng ? sPair[r] : make_int2(0, 0);
                        lx[e] = pr.x;
                        ls[e] = pr.y;
                        search |= uint32_t(r < ng) << e;
                        tgt[e] = -1;
                        lp[e] = home_bucket(uint32_t(lx[e]), a.a1, smask);
                        ld[e] = stride_of(uint32_t(lx[e]), a.a2, smask);
                    }
                    // Miss list (id, slot) in rank order, from the same registers.
                    int2* P = reinterpret_cast<int2*>(a.pairs) + tok * K;
    #pragma unroll
                    for (int e = 0; e < IPT; ++e)
                        if ((search >> e) & 1u) P[tid_t + e * T] = make_int2(lx[e], ls[e]);
                    // Checked every round: most links succeed in the first.  The
                    // wave walks the rounds over as many ids per lane as its
                    // lanes' highest searching id needs (1, 2, 4 or IPT).
                    uint32_t wave_ids = 0;
    #pragma unroll
                    for (int e = 1; e < IPT; ++e)
                        wave_ids |= uint32_t(__ballot((search >> e) & 1u) != 0ull) << e;
                    if (wave_ids == 0u)
                        link_rounds<1, IPT>(sQ, sC, lp, ld, tgt, search, R, smask, a.afp);
                    else if (IPT >= 4 && wave_ids < 4u)
                        link_rounds<(IPT >= 4 ? 2 : 1), IPT>(sQ, sC, lp, ld, tgt, search, R,
                                                            smask, a.afp);
                    else if (IPT >= 8 && wave_ids < 16u)
                        link_rounds<(IPT >= 8 ? 4 : 1), IPT>(sQ, sC, lp, ld, tgt, search, R,
                                                            smask, a.afp);
                    else
                        link_rounds<IPT, IPT>(sQ, sC, lp, ld, tgt, search, R, smask, a.afp);
    #pragma unroll
                    for (int e = 0; e < IPT; ++e)
                        c_lexh += uint32_t(__popcll(__ballot((search >> e) & 1u)));
                    // Claims are kClaimBase + (K - 1 - rank): below every bucket
                    // word (>= -1), so the minimum over a bucket's claimants is
                    // the largest rank's, with no reset of the bucket first.
                    __syncthreads();
    #pragma unroll
                    for (int e = 0; e < IPT; ++e)
                        if (tgt[e] >= 0)
                            atomicMin(&sQ[tgt[e]], kClaimBase + (K - 1 - (tid_t + e * T)));
                    __syncthreads();
                    // Every read of the pairs and of the bitmap is done: clear it
                    // for the next token.
                    if (g + 1 < a.Nq) clear_words<T>(sBits, lay.bitmap_words, tid_t);
                    uint32_t lostm = 0;
    #pragma unroll
                    for (int e = 0; e < IPT; ++e) {
                        if (tgt[e] >= 0) {
                            if (sQ[tgt[e]] == kClaimBase + (K - 1 - (tid_t + e * T))) {
                                const int32_t word = (fp_of(uint32_t(lx[e]), a.afp) << 16) | ls[e];
                                sQ[tgt[e]] = word;
                                gQ[tgt[e]] = word;  // written through, like C
                            } else {
                                lostm |= 1u << e;
                            }
                        }
                    }
    #pragma unroll
                    for (int e = 0; e < IPT; ++e)
                        c_lcol += uint32_t(__popcll(__ballot((lostm >> e) & 1u)));
                }
            }

            // Slot table and hit mask of this thread's positions.
            int32_t o[IPT];
            int8_t hm[IPT];
    #pragma unroll
            for (int e = 0; e < IPT; ++e) {
                const bool ok = (valid >> e) & 1u;
                o[e] = ok ? slot[e] : -1;
                hm[e] = ok ? int8_t(((missm >> e) & 1u) ? 0 : 1) : int8_t(-1);
            }
            store_outputs<IPT>(O, H, i0_t, K, vec, o, hm);
            if (tid_t == 0) a.n_miss[tok] = ng;
            if (ng > 0 && tid_t == 0) sMisc[0] = 0;  // read before two barriers at least
            if constexpr (DENSE) region_dirty = ng > 0;
            // The end of the step reads C and the lifetimes, whose last writes
            // (refreshes, decay, installs) came before a barrier of this token,
            // so only a following token (or the dense matcher's map updates)
            // needs this one.
            if (DENSE || g + 1 < a.Nq) __syncthreads();
        } while (++g < a.Nq);

        // End of step: empty every slot caching a speculative id (>= N) and
        // write the lifetimes back (F = G - 1).  Installs and links wrote C and Q
        // through to global memory as they happened, so only the emptied slots
        // are written here.
        for (int j = tid; j < (S >> 2); j += T) {
            const int4 c = reinterpret_cast<const int4*>(sC)[j];
            const int32_t cv[4] = {c.x, c.y, c.z, c.w};
    #pragma unroll
            for (int u = 0; u < 4; ++u) {
                if (cv[u] >= N) {
                    if constexpr (DENSE) map_clear_if(mrow, a.map_len, cv[u], 4 * j + u);
                    gC[4 * j + u] = -1;
                }
            }
            const uint32_t w = sGw[j];
            reinterpret_cast<int4*>(gF)[j] =
                make_int4(int(w & 0xFFu) - 1, int((w >> 8) & 0xFFu) - 1,
                          int((w >> 16) & 0xFFu) - 1, int(w >> 24) - 1);
        }

        // Counters: one wave sum (visits), then one LDS atomic per wave for
        // each counter kept per wave, into sums zeroed before the first token.
        int32_t* sCnt = sMisc + 2;
        const int visits = lane63(wave_scan_add(int(c_visit)));
        const int looks = lane63(wave_scan_add(int(c_look)));
        const uint64_t e1 = __ballot(c_err & 1u), e2 = __ballot(c_err & 2u);
        if (lane == 0) {
            if (looks) atomicAdd(&sCnt[1], looks);
            if (c_lcol) atomicAdd(&sCnt[3], int(c_lcol));
            if (c_lexh) atomicAdd(&sCnt[4], int(c_lexh));
            if (c_live) atomicAdd(&sCnt[5], int(c_live));
            if (visits) atomicAdd(&sCnt[7], visits);
            if (e1 || e2) atomicOr(&sCnt[6], (e1 ? 1 : 0) | (e2 ? 2 : 0));
        }
        __syncthreads();
        if (tid < 8) {
            int32_t* cnt = RequestArgs<MULTI>::get(a).CNT + size_t(b) * 8;
            const uint32_t add = tid == 0   ? uint32_t(sCnt[1]) - c_miss
                                 : tid == 2 ? c_miss
                                            : uint32_t(sCnt[tid]);
            if (tid == 6)
                cnt[6] = cnt_old | int32_t(add);
            else
                cnt[tid] = int32_t(uint32_t(cnt_old) + add);
        }
        if constexpr (!MULTI) break;
        have_pre = prefetch_next;
        b = bn;
        if (b >= RequestArgs<MULTI>::get(a).B) break;
    }
}

// More requests than workgroups (grid < B): the hash matcher's workgroups
// each take several requests, with the next one's state loaded ahead; the
// forms with up to four ids per thread only (eight would spill VGPRs).
template <int T, int IPT>
hipError_t launch_one(const Stage1Args& a, int grid, size_t lds, bool dense, hipStream_t s) {
    if (dense)
        hipLaunchKernelGGL((stage1_kernel<T, IPT, true, false>), dim3(a.B), dim3(T), lds, s, a);
    else if (IPT <= 4 && grid < a.B)
        hipLaunchKernelGGL((stage1_kernel<T, (IPT <= 4 ? IPT : 4), false, true>), dim3(grid),
                           dim3(T), lds, s, a);
    else
        hipLaunchKernelGGL((stage1_kernel<T, IPT, false, false>), dim3(a.B), dim3(T), lds, s, a);
    return hipGetLastError();
}

template <int T, int IPT, bool DENSE, bool MULTI>
hipError_t set_lds(size_t lds) {
    return hipFuncSetAttribute(reinterpret_cast<const void*>(&stage1_kernel<T, IPT, DENSE, MULTI>),
                               hipFuncAttributeMaxDynamicSharedMemorySize, int(lds));
}

template <int T, int IPT>
hipError_t prepare_one(size_t lds) {
    hipError_t e;
    if ((e = set_lds<T, IPT, false, false>(lds)) != hipSuccess) return e;
    if ((e = set_lds<T, IPT, true, false>(lds)) != hipSuccess) return e;
    if constexpr (IPT <= 4) return set_lds<T, IPT, false, true>(lds);
    return hipSuccess;
}

}  // namespace

int stage1_threads(int K, int requested) {
    if (requested) return requested;
    // Two ids per thread up to 1024 threads: the probe and link rounds are
    // LDS-latency bound, and more waves hide more of it (measured on the
    // matching and residency shapes: 1024 threads beat 512 and 256).
    const int half = next_pow2(K) / 2;
    return half <= 256 ? 256 : half >= 1024 ? 1024 : half;
}

template <int T>
hipError_t prepare_t(size_t lds) {
    hipError_t e;
    if ((e = prepare_one<T, 1>(lds)) != hipSuccess) return e;
    if ((e = prepare_one<T, 2>(lds)) != hipSuccess) return e;
    if ((e = prepare_one<T, 4>(lds)) != hipSuccess) return e;
    return prepare_one<T, 8>(lds);
}

hipError_t stage1_prepare(size_t lds) {
    hipError_t e;
    if ((e = prepare_t<256>(lds)) != hipSuccess) return e;
    if ((e = prepare_t<512>(lds)) != hipSuccess) return e;
    return prepare_t<1024>(lds);
}

template <int T>
hipError_t launch_t(const Stage1Args& a, int grid, size_t lds, bool dense, hipStream_t s) {
    const int ipt = (a.K + T - 1) / T;
    if (ipt <= 1) return launch_one<T, 1>(a, grid, lds, dense, s);
    if (ipt <= 2) return launch_one<T, 2>(a, grid, lds, dense, s);
    if (ipt <= 4) return launch_one<T, 4>(a, grid, lds, dense, s);
    return launch_one<T, 8>(a, grid, lds, dense, s);
}

hipError_t launch_stage1(const Stage1Args& a, int threads, int grid, size_t lds, bool dense,
                         hipStream_t s) {
    if (threads == 256) return launch_t<256>(a, grid, lds, dense, s);
    if (threads == 512) return launch_t<512>(a, grid, lds, dense, s);
    return launch_t<1024>(a, grid, lds, dense, s);
}

}  // namespace avsg
