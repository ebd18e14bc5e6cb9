// Lossless threshold prefetch ahead of the recall step.
//
// Method: ECHO ("Efficient KV Cache Offloading with Lossless Prefetching for
// Serving Native Sparse Attention LLMs", decode prefetch): while the indexer
// scores every earlier token, any token whose score exceeds a predicted
// threshold is fetched at once, up to a cap proportional to the context; the
// threshold predicts the K-th highest score of the step with an exponential
// moving average (alpha 0.5 on the page) of the observed K-th scores.  The
// exact top-K selection is unchanged: the guaranteed recall afterwards
// fetches whatever the prefetch missed, and prefetched tokens are hits.
//
// Readings taken: the candidates are the first cap positions in ascending
// order whose float32 score is strictly above the threshold, among positions
// below the verified length N; the moving average starts from the first
// observed K-th score (a threshold of +inf means "no prediction yet").
//
// gfx950 mapping.  One 1024-thread workgroup per request.  Each wave owns a
// contiguous segment of the score row: it counts passing positions with
// ballots, a workgroup scan of the 16 counts gives each wave its output
// offset, and a second pass writes positions in order.
#include "internal.h"

namespace avsg {
namespace {

constexpr int T = 1024;
constexpr int W = T / 64;

__global__ __launch_bounds__(T) void prefetch_select_kernel(PrefetchArgs a) {
    __shared__ int32_t sCount[W + 1];
    const int b = blockIdx.x, tid = threadIdx.x, lane = __lane_id(), w = tid >> 6;
    const int64_t N = min<int64_t>(max(a.ctx_len[b], 0), a.row_len);
    const float theta = a.theta[b];
    const int cap = min(max(a.cap[b], 0), a.K);
    const float* sc = a.scores + size_t(b) * a.row_len;
    int32_t* out = a.cand + size_t(b) * a.K;

    const int64_t seg = (N + W - 1) / W;
    const int64_t s0 = min<int64_t>(int64_t(w) * seg, N), s1 = min<int64_t>(s0 + seg, N);
    int cnt = 0;
    for (int64_t j0 = s0; j0 < s1; j0 += 64) {
        const int64_t j = j0 + lane;
        const bool pass = j < s1 && sc[j] > theta;
        cnt += __popcll(__ballot(pass));
    }
    if (lane == 0) sCount[w] = cnt;
    __syncthreads();
    if (tid == 0) {
        int run = 0;
        for (int u = 0; u < W; ++u) {
            const int c = sCount[u];
            sCount[u] = run;
            run += c;
        }
        sCount[W] = run;
    }
    __syncthreads();
    int off = sCount[w];
    const int total = min(sCount[W], cap);
    for (int64_t j0 = s0; j0 < s1 && off < cap; j0 += 64) {
        const int64_t j = j0 + lane;
        const bool pass = j < s1 && sc[j] > theta;
        const uint64_t m = __ballot(pass);
        const int r = off + __popcll(m & ((1ull << lane) - 1ull));
        if (pass && r < cap) out[r] = int32_t(j);
        off += __popcll(m);
    }
    for (int i = total + tid; i < a.K; i += T) out[i] = -1;
}

__global__ __launch_bounds__(256) void ema_threshold_kernel(EmaArgs a) {
    // Products and sum rounded one at a time (no fused multiply-add), so the
    // update is the same in any float32 implementation.
#pragma clang fp contract(off)
    const int b = blockIdx.x * blockDim.x + threadIdx.x;
    if (b >= a.B) return;
    const float s = a.kth[b];
    const float t = a.theta[b];
    const float p = a.alpha * s;
    const float q = (1.0f - a.alpha) * t;
    a.theta[b] = isinf(t) ? s : p + q;
}

}  // namespace

hipError_t launch_prefetch_select(const PrefetchArgs& a, hipStream_t s) {
    hipLaunchKernelGGL(prefetch_select_kernel, dim3(a.B), dim3(T), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_ema_threshold(const EmaArgs& a, hipStream_t s) {
    hipLaunchKernelGGL(ema_threshold_kernel, dim3((a.B + 255) / 256), dim3(256), 0, s, a);
    return hipGetLastError();
}

}  // namespace avsg
