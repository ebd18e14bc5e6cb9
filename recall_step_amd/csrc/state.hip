// Reset of request rows to the empty state (every slot empty and dead, every
// bucket empty, counters zero; with the dense matcher every map entry absent).
// Plain kernels, so a reset may sit in a captured graph.
#include "internal.h"

namespace avsg {
namespace {

__global__ __launch_bounds__(256) void state_init_kernel(InitArgs a) {
    const int b = blockIdx.x;
    if (a.row_mask && a.row_mask[b] == 0) return;
    int32_t* q = a.Q + size_t(b) * a.S;
    int32_t* c = a.C + size_t(b) * a.S;
    int32_t* f = a.F + size_t(b) * a.S;
    const int4 neg = make_int4(-1, -1, -1, -1);
    for (int j = threadIdx.x; j < (a.S >> 2); j += blockDim.x) {
        reinterpret_cast<int4*>(q)[j] = neg;
        reinterpret_cast<int4*>(c)[j] = neg;
        reinterpret_cast<int4*>(f)[j] = neg;
    }
    if (threadIdx.x < 8) a.CNT[size_t(b) * 8 + threadIdx.x] = 0;
}

// Map rows: grid (chunks, B); each workgroup fills its share of one row.
__global__ __launch_bounds__(256) void map_reset_kernel(InitArgs a) {
    const int b = blockIdx.y;
    if (a.row_mask && a.row_mask[b] == 0) return;
    int32_t* m = a.map + size_t(b) * size_t(a.map_len);
    const int64_t step = int64_t(gridDim.x) * blockDim.x;
    for (int64_t j = int64_t(blockIdx.x) * blockDim.x + threadIdx.x; j < a.map_len; j += step)
        m[j] = -1;
}

}  // namespace

hipError_t launch_state_init(const InitArgs& a, hipStream_t s) {
    hipLaunchKernelGGL(state_init_kernel, dim3(a.B), dim3(256), 0, s, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || !a.map) return e;
    const int64_t chunks = (a.map_len + 256 * 16 - 1) / (256 * 16);
    const int gx = int(chunks < 1024 ? chunks : 1024);
    hipLaunchKernelGGL(map_reset_kernel, dim3(gx, a.B), dim3(256), 0, s, a);
    return hipGetLastError();
}

}  // namespace avsg
