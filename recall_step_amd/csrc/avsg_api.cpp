// Host side of the C ABI declared in include/avsg.h: validation, handle and
// workspace management, and the launch sequence of a recall step.
#include "avsg.h"

#include <hip/hip_runtime.h>

#include <new>

#include "internal.h"

struct avsg_handle {
    avsg::StepContext ctx;    // ctx.ws_pairs: [B][N_q][K][2] miss list when io gives none
    int device;
    int64_t step_tokens;      // query tokens enqueued since the last avsg_match
};

namespace avsg {

namespace {
thread_local int g_last_hip = 0;
}  // namespace

int hip_fail(hipError_t e) {
    g_last_hip = int(e);
    return AVSG_EHIP;
}

hipError_t prepare_kernels(size_t lds_bytes) {
    hipError_t e = stage1_prepare(lds_bytes);
    return e == hipSuccess ? sort_merge_prepare(lds_bytes) : e;
}

namespace {

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Fields Stage One reads or writes.
bool match_io_ok(const avsg_step_io* io) {
    return io && io->topk && io->ctx_len && io->row_base && io->host_rows &&
           io->slot_table && io->hit_mask && io->n_miss &&
           (io->miss_pairs == nullptr || aligned16(io->miss_pairs));
}

// Fields Stage Two reads (the by-top-K partition reads the top-K ids, hit
// mask and slot table instead of the miss list).
bool gather_io_ok(const avsg_step_io* io, uint32_t flags) {
    if (!io || !io->row_base || !io->host_rows) return false;
    if (flags & AVSG_FLAG_GATHER_BY_TOPK) return io->topk && io->hit_mask && io->slot_table;
    return io->n_miss && (io->miss_pairs == nullptr || aligned16(io->miss_pairs));
}

}  // namespace

int check_buffers(const avsg_config* cfg, const avsg_buffers* bufs) {
    if (!bufs || !bufs->Q || !bufs->C || !bufs->F || !bufs->CNT || !bufs->dev_kv)
        return AVSG_EINVAL;
    if (!aligned16(bufs->Q) || !aligned16(bufs->C) || !aligned16(bufs->F) ||
        !aligned16(bufs->CNT) || !aligned16(bufs->dev_kv))
        return AVSG_EINVAL;
    const bool skip = (cfg->flags & AVSG_FLAG_SKIP_GATHER) != 0;
    if (!skip && (!bufs->host_kv || !aligned16(bufs->host_kv))) return AVSG_EINVAL;
    if (bufs->host_rows_total < 0) return AVSG_EINVAL;
    const bool dense = (cfg->flags & AVSG_FLAG_DENSE_MAP) != 0;
    if (dense && (!bufs->map || bufs->map_len < 1 ||
                  (reinterpret_cast<uintptr_t>(bufs->map) & 3u) != 0))
        return AVSG_EINVAL;
    if (int64_t(cfg->B) * cfg->N_q > kMaxTokens) return AVSG_EUNSUPPORTED;
    return AVSG_OK;
}

int fill_context(const avsg_config* cfg, const avsg_buffers* bufs, int multiprocessors,
                 size_t lds_limit, int32_t* ws_pairs, StepContext* out) {
    const size_t lds = avsg_stage1_lds_bytes(cfg);
    if (lds == 0 || lds > lds_limit) return AVSG_EUNSUPPORTED;
    const uint8_t* host_dev = nullptr;
    if (bufs->host_kv) {
        void* dptr = nullptr;
        hipError_t e = hipHostGetDevicePointer(&dptr, const_cast<void*>(bufs->host_kv), 0);
        if (e != hipSuccess) return hip_fail(e);
        host_dev = static_cast<const uint8_t*>(dptr);
    }
    out->cfg = *cfg;
    out->bufs = *bufs;
    if (!(cfg->flags & AVSG_FLAG_DENSE_MAP)) {
        out->bufs.map = nullptr;
        out->bufs.map_len = 0;
    }
    out->host_dev = host_dev;
    out->lds_bytes = lds;
    out->gather_blocks = cfg->gather_blocks > 0 ? cfg->gather_blocks : multiprocessors;
    out->stage1_threads = stage1_threads(cfg->K, cfg->stage1_threads);
    out->stage1_grid = multiprocessors > 0 ? multiprocessors : 1;
    out->ws_pairs = ws_pairs;
    return AVSG_OK;
}

int run_match(const StepContext& x, const avsg_step_io* io, hipStream_t stream,
              bool predecay) {
    if (!match_io_ok(io)) return AVSG_EINVAL;
    const avsg_config& c = x.cfg;
    int32_t* pairs = io->miss_pairs ? io->miss_pairs : x.ws_pairs;
    if (c.flags & AVSG_FLAG_NO_REUSE) {
        OffloadArgs o;
        o.CNT = x.bufs.CNT;
        o.topk = io->topk;
        o.row_base = io->row_base;
        o.host_rows = io->host_rows;
        o.slot_table = io->slot_table;
        o.hit_mask = io->hit_mask;
        o.n_miss = io->n_miss;
        o.pairs = pairs;
        o.host_rows_total = x.bufs.host_rows_total;
        o.B = c.B;
        o.Nq = c.N_q;
        o.K = c.K;
        hipError_t e = launch_offload(o, stream);
        return e == hipSuccess ? AVSG_OK : hip_fail(e);
    }
    Stage1Args a;
    a.Q = x.bufs.Q;
    a.C = x.bufs.C;
    a.F = x.bufs.F;
    a.CNT = x.bufs.CNT;
    a.topk = io->topk;
    a.ctx_len = io->ctx_len;
    a.row_base = io->row_base;
    a.host_rows = io->host_rows;
    a.slot_table = io->slot_table;
    a.hit_mask = io->hit_mask;
    a.n_miss = io->n_miss;
    a.pairs = pairs;
    a.host_rows_total = x.bufs.host_rows_total;
    a.B = c.B;
    a.Nq = c.N_q;
    a.K = c.K;
    a.S = c.S;
    a.L = c.L;
    a.R = c.R;
    a.predecay = predecay ? 1 : 0;
    a.a1 = c.a1;
    a.a2 = c.a2;
    a.afp = c.a_fp;
    a.map = x.bufs.map;
    a.map_len = x.bufs.map_len;
    hipError_t e = (c.flags & AVSG_FLAG_SORT_MERGE)
                       ? launch_sort_merge(a, x.lds_bytes, stream)
                       : launch_stage1(a, x.stage1_threads, x.stage1_grid, x.lds_bytes,
                                       (c.flags & AVSG_FLAG_DENSE_MAP) != 0, stream);
    return e == hipSuccess ? AVSG_OK : hip_fail(e);
}

int run_gather(const StepContext& x, const avsg_step_io* io, hipStream_t stream) {
    if (!gather_io_ok(io, x.cfg.flags)) return AVSG_EINVAL;
    if (!x.host_dev) return AVSG_EINVAL;
    const avsg_config& c = x.cfg;
    GatherArgs a;
    a.n_miss = io->n_miss;
    a.pairs = io->miss_pairs ? io->miss_pairs : x.ws_pairs;
    a.topk = io->topk;
    a.hit_mask = io->hit_mask;
    a.slot_table = io->slot_table;
    a.row_base = io->row_base;
    a.host_rows = io->host_rows;
    a.host = x.host_dev;
    a.dev = static_cast<uint8_t*>(x.bufs.dev_kv);
    a.host_rows_total = x.bufs.host_rows_total;
    a.B = c.B;
    a.Nq = c.N_q;
    a.K = c.K;
    a.S = c.S;
    a.row_bytes = c.row_bytes;
    a.mode = (c.flags & AVSG_FLAG_GATHER_BY_REQUEST) ? kGatherByRequest
             : (c.flags & AVSG_FLAG_GATHER_BY_TOPK)  ? kGatherByTopk
                                                     : kGatherByRow;
    hipError_t e = launch_gather(a, x.gather_blocks, stream);
    return e == hipSuccess ? AVSG_OK : hip_fail(e);
}

int run_step(const StepContext& x, const avsg_step_io* io, hipStream_t stream) {
    // Both stages' arguments are checked before the first launch, so an
    // error leaves nothing half enqueued.
    if (!match_io_ok(io)) return AVSG_EINVAL;
    const bool gather = !(x.cfg.flags & AVSG_FLAG_SKIP_GATHER);
    if (gather && (!gather_io_ok(io, x.cfg.flags) || !x.host_dev)) return AVSG_EINVAL;
    int rc = run_match(x, io, stream, true);
    if (rc != AVSG_OK || !gather) return rc;
    return run_gather(x, io, stream);
}

}  // namespace avsg

namespace {

int check_device(const avsg_handle* h) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return avsg::hip_fail(e);
    return dev == h->device ? AVSG_OK : AVSG_EINVAL;
}

}  // namespace

extern "C" {

int avsg_version(void) { return AVSG_VERSION; }

const char* avsg_strerror(int code) {
    switch (code) {
        case AVSG_OK: return "ok";
        case AVSG_EINVAL: return "invalid argument or configuration";
        case AVSG_ENOMEM: return "device memory allocation failed";
        case AVSG_EHIP: return "HIP runtime call failed (see avsg_last_hip_error)";
        case AVSG_EUNSUPPORTED: return "configuration beyond this build's limits";
        case AVSG_ESCRATCH:
            return "miss list larger than the static scratch of avsg_step_noalloc "
                   "(B*N_q*K above AVSG_NOALLOC_MAX_PAIRS); pass io->miss_pairs or use "
                   "avsg_step";
        default: return "unknown error code";
    }
}

int avsg_last_hip_error(void) { return avsg::g_last_hip; }

void avsg_config_default(avsg_config* cfg, int32_t B, int32_t N_q, int32_t K,
                         int32_t S, int32_t row_bytes) {
    if (!cfg) return;
    cfg->B = B;
    cfg->N_q = N_q;
    cfg->K = K;
    cfg->S = S;
    cfg->L = 15;
    cfg->R = 7;
    cfg->a1 = 0x9E3779B1u;
    cfg->a2 = 0x85EBCA77u;
    cfg->a_fp = 0xC2B2AE3Du;
    cfg->row_bytes = row_bytes;
    cfg->flags = 0;
    cfg->gather_blocks = 0;
    cfg->stage1_threads = 0;
}

int avsg_validate_config(const avsg_config* c) {
    if (!c) return AVSG_EINVAL;
    if (c->B < 1 || c->N_q < 1 || c->K < 1 || c->K > 8192) return AVSG_EINVAL;
    if (c->S < 16 || c->S > 65536 || (c->S & (c->S - 1)) != 0) return AVSG_EINVAL;
    if (int64_t(c->N_q) * c->K > c->S) return AVSG_EINVAL;
    // Rounds past S - 1 would only revisit buckets (odd stride, S a power
    // of two), and the bound keeps every probe and link loop short.
    if (c->L < 1 || c->L > 127 || c->R < 0 || c->R > c->S - 1) return AVSG_EINVAL;
    if ((c->a1 & 1u) == 0 || (c->a2 & 1u) == 0 || (c->a_fp & 1u) == 0) return AVSG_EINVAL;
    if (c->row_bytes < 16 || (c->row_bytes & 15) != 0) return AVSG_EINVAL;
    if (c->gather_blocks < 0) return AVSG_EINVAL;
    if (c->stage1_threads != 0 && c->stage1_threads != 256 && c->stage1_threads != 512 &&
        c->stage1_threads != 1024)
        return AVSG_EINVAL;
    if (c->stage1_threads != 0 && c->K > c->stage1_threads * avsg::kMaxIdsPerThread)
        return AVSG_EINVAL;
    const uint32_t known = AVSG_FLAG_SKIP_GATHER | AVSG_FLAG_GATHER_BY_REQUEST |
                           AVSG_FLAG_GATHER_BY_TOPK | AVSG_FLAG_NO_REUSE |
                           AVSG_FLAG_SORT_MERGE | AVSG_FLAG_DENSE_MAP;
    if (c->flags & ~known) return AVSG_EINVAL;
    // At most one matcher other than the hash table.
    const uint32_t matchers = c->flags & (AVSG_FLAG_NO_REUSE | AVSG_FLAG_SORT_MERGE |
                                          AVSG_FLAG_DENSE_MAP);
    if (matchers & (matchers - 1u)) return AVSG_EINVAL;
    if ((c->flags & AVSG_FLAG_GATHER_BY_REQUEST) && (c->flags & AVSG_FLAG_GATHER_BY_TOPK))
        return AVSG_EINVAL;
    return AVSG_OK;
}

size_t avsg_stage1_lds_bytes(const avsg_config* c) {
    if (!c) return 0;
    if (c->flags & AVSG_FLAG_SORT_MERGE) return avsg::sort_merge_layout(c->S, c->K).total;
    return avsg::stage1_layout(c->S, c->K, c->L).total;
}

size_t avsg_workspace_bytes(const avsg_config* c) {
    if (!c) return 0;
    return size_t(c->B) * c->N_q * c->K * 2 * sizeof(int32_t);
}

int avsg_create(const avsg_config* cfg, const avsg_buffers* bufs, avsg_handle** out) {
    if (!out) return AVSG_EINVAL;
    *out = nullptr;
    int rc = avsg_validate_config(cfg);
    if (rc != AVSG_OK) return rc;
    rc = avsg::check_buffers(cfg, bufs);
    if (rc != AVSG_OK) return rc;

    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return avsg::hip_fail(e);
    hipDeviceProp_t prop;
    e = hipGetDeviceProperties(&prop, dev);
    if (e != hipSuccess) return avsg::hip_fail(e);
    avsg::StepContext ctx;
    rc = avsg::fill_context(cfg, bufs, prop.multiProcessorCount,
                            size_t(prop.sharedMemPerBlock), nullptr, &ctx);
    if (rc != AVSG_OK) return rc;
    // The limit is the device's, not this config's: handles of other
    // configs and the allocation-free entry point share these kernels.
    e = avsg::prepare_kernels(size_t(prop.sharedMemPerBlock) < avsg::kStage1LdsBudget
                                  ? size_t(prop.sharedMemPerBlock)
                                  : avsg::kStage1LdsBudget);
    if (e != hipSuccess) return avsg::hip_fail(e);

    avsg_handle* h = new (std::nothrow) avsg_handle();
    if (!h) return AVSG_ENOMEM;
    h->ctx = ctx;
    h->device = dev;
    e = hipMalloc(reinterpret_cast<void**>(&h->ctx.ws_pairs), avsg_workspace_bytes(cfg));
    if (e != hipSuccess) {
        avsg::g_last_hip = int(e);
        delete h;
        return AVSG_ENOMEM;
    }
    *out = h;
    return AVSG_OK;
}

int avsg_destroy(avsg_handle* h) {
    if (!h) return AVSG_OK;
    hipError_t e = hipSuccess;
    if (h->ctx.ws_pairs) e = hipFree(h->ctx.ws_pairs);
    delete h;
    return e == hipSuccess ? AVSG_OK : avsg::hip_fail(e);
}

int avsg_state_init(avsg_handle* h, const int32_t* row_mask, void* stream) {
    if (!h) return AVSG_EINVAL;
    int rc = check_device(h);
    if (rc != AVSG_OK) return rc;
    const avsg_buffers& b = h->ctx.bufs;
    avsg::InitArgs a{b.Q, b.C, b.F, b.CNT, row_mask, h->ctx.cfg.B, h->ctx.cfg.S, b.map,
                     b.map_len};
    hipError_t e = avsg::launch_state_init(a, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? AVSG_OK : avsg::hip_fail(e);
}

int avsg_match(avsg_handle* h, const avsg_step_io* io, void* stream) {
    if (!h) return AVSG_EINVAL;
    int rc = check_device(h);
    if (rc != AVSG_OK) return rc;
    rc = avsg::run_match(h->ctx, io, static_cast<hipStream_t>(stream), true);
    if (rc == AVSG_OK) h->step_tokens = h->ctx.cfg.N_q;
    return rc;
}

int avsg_match_continue(avsg_handle* h, const avsg_step_io* io, void* stream) {
    if (!h || (h->ctx.cfg.flags & AVSG_FLAG_SORT_MERGE)) return AVSG_EINVAL;
    // The capacity bound holds for the step as a whole: every query token
    // since the step's avsg_match counts against N_q * K <= S.
    const avsg_config& c = h->ctx.cfg;
    const int64_t tokens = h->step_tokens + c.N_q;
    if (tokens * c.K > c.S) return AVSG_EINVAL;
    int rc = check_device(h);
    if (rc != AVSG_OK) return rc;
    rc = avsg::run_match(h->ctx, io, static_cast<hipStream_t>(stream), false);
    if (rc == AVSG_OK) h->step_tokens = tokens;
    return rc;
}

int avsg_gather(avsg_handle* h, const avsg_step_io* io, void* stream) {
    if (!h) return AVSG_EINVAL;
    int rc = check_device(h);
    if (rc != AVSG_OK) return rc;
    return avsg::run_gather(h->ctx, io, static_cast<hipStream_t>(stream));
}

int avsg_step(avsg_handle* h, const avsg_step_io* io, void* stream) {
    if (!h) return AVSG_EINVAL;
    int rc = check_device(h);
    if (rc != AVSG_OK) return rc;
    rc = avsg::run_step(h->ctx, io, static_cast<hipStream_t>(stream));
    if (rc == AVSG_OK) h->step_tokens = h->ctx.cfg.N_q;
    return rc;
}

int avsg_prefetch_select(avsg_handle* h, const float* scores, int64_t row_len,
                         const int32_t* ctx_len, const float* theta, const int32_t* cap,
                         int32_t* cand, void* stream) {
    if (!h || !scores || row_len < 0 || !ctx_len || !theta || !cap || !cand)
        return AVSG_EINVAL;
    int rc = check_device(h);
    if (rc != AVSG_OK) return rc;
    avsg::PrefetchArgs a{scores, row_len, ctx_len, theta, cap, cand, h->ctx.cfg.B,
                         h->ctx.cfg.K};
    hipError_t e = avsg::launch_prefetch_select(a, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? AVSG_OK : avsg::hip_fail(e);
}

int avsg_ema_threshold(avsg_handle* h, const float* kth, float* theta, float alpha,
                       void* stream) {
    if (!h || !kth || !theta || !(alpha > 0.0f && alpha <= 1.0f)) return AVSG_EINVAL;
    int rc = check_device(h);
    if (rc != AVSG_OK) return rc;
    avsg::EmaArgs a{kth, theta, alpha, h->ctx.cfg.B};
    hipError_t e = avsg::launch_ema_threshold(a, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? AVSG_OK : avsg::hip_fail(e);
}

int avsg_host_alloc(size_t bytes, void** out) {
    if (!out || bytes == 0) return AVSG_EINVAL;
    *out = nullptr;
    hipError_t e = hipHostMalloc(out, bytes, hipHostMallocMapped);
    if (e != hipSuccess) {
        *out = nullptr;
        return avsg::hip_fail(e);
    }
    return AVSG_OK;
}

int avsg_host_free(void* p) {
    if (!p) return AVSG_OK;
    hipError_t e = hipHostFree(p);
    return e == hipSuccess ? AVSG_OK : avsg::hip_fail(e);
}

}  // extern "C"
