// Allocation-free recall step (avsg_step_noalloc): avsg_step's launches with
// no handle, the miss list kept in a static device array when the caller
// passes none.  For callers that cannot allocate device memory: code under
// HIP graph capture, serving loops that forbid hipMalloc.
#include <mutex>

#include "internal.h"

namespace avsg {
namespace {

// The miss list, (id, slot) int32 pairs [B][N_q][K][2] packed as Stage One
// writes them.  Each device holds its own copy until the process ends.  In
// host code this name is only a handle for hipGetSymbolAddress: kernels get
// the device address resolved below, never the name.
__device__ __align__(256) int32_t scratch[2 * AVSG_NOALLOC_MAX_PAIRS];

constexpr int kMaxDevices = 64;

struct DeviceSetup {
    bool ready;
    int32_t* scratch;      // device address of `scratch` on this device
    int multiprocessors;
    size_t lds_limit;      // LDS per workgroup the Stage-One kernels may use
};

DeviceSetup g_setup[kMaxDevices];
std::mutex g_setup_mutex;

// Once per device, with that device current: resolve the array's address
// and set the kernels' LDS limit.  Queries and attributes only.
int setup_device(int dev, DeviceSetup* out) {
    std::lock_guard<std::mutex> lock(g_setup_mutex);
    DeviceSetup& d = g_setup[dev];
    if (!d.ready) {
        void* ptr = nullptr;
        hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return hip_fail(e);
        if (ptr == nullptr) return AVSG_EHIP;
        hipDeviceProp_t prop;
        e = hipGetDeviceProperties(&prop, dev);
        if (e != hipSuccess) return hip_fail(e);
        const size_t lds = kStage1LdsBudget < size_t(prop.sharedMemPerBlock)
                               ? kStage1LdsBudget
                               : size_t(prop.sharedMemPerBlock);
        e = prepare_kernels(lds);
        if (e != hipSuccess) return hip_fail(e);
        d.scratch = static_cast<int32_t*>(ptr);
        d.multiprocessors = prop.multiProcessorCount;
        d.lds_limit = lds;
        d.ready = true;
    }
    *out = d;
    return AVSG_OK;
}

}  // namespace
}  // namespace avsg

extern "C" int avsg_step_noalloc(const avsg_config* cfg, const avsg_buffers* bufs,
                                 const avsg_step_io* io, void* stream) {
    int rc = avsg_validate_config(cfg);
    if (rc != AVSG_OK) return rc;
    rc = avsg::check_buffers(cfg, bufs);
    if (rc != AVSG_OK) return rc;
    if (!io) return AVSG_EINVAL;
    if (!io->miss_pairs && int64_t(cfg->B) * cfg->N_q * cfg->K > AVSG_NOALLOC_MAX_PAIRS)
        return AVSG_ESCRATCH;
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return avsg::hip_fail(e);
    if (dev < 0 || dev >= avsg::kMaxDevices) return AVSG_EUNSUPPORTED;
    avsg::DeviceSetup d;
    rc = avsg::setup_device(dev, &d);
    if (rc != AVSG_OK) return rc;
    avsg::StepContext ctx;
    rc = avsg::fill_context(cfg, bufs, d.multiprocessors, d.lds_limit, d.scratch, &ctx);
    if (rc != AVSG_OK) return rc;
    return avsg::run_step(ctx, io, static_cast<hipStream_t>(stream));
}
