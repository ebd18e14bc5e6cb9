/*
 * avsg.h - C ABI of the per-decode-step KV recall library for MI355X (gfx950).
 *
 * The library makes the KV rows that a sparse-attention step selected
 * resident in device memory.  For every request it matches the top-K
 * selected token ids of each query token against a fixed-capacity slot
 * buffer with an open-addressing hash probe, assigns the misses slots by
 * per-slot aging with hit-triggered lifetime refresh, copies the missed rows
 * from pinned host memory into their slots, and emits the slot table that
 * attention reads.  The method is the one described on the page "AVSG:
 * Accelerated Vectorized Sparse Gather for Efficient KV Cache Offload in
 * Sparse-Attention LLM Serving" (cited below as AVSG with its section).
 *
 * Conventions
 *  - Every function returns AVSG_OK (0) or a negative AVSG_E* code.  On
 *    AVSG_EHIP, avsg_last_hip_error() returns the HIP error of the failing
 *    call on this thread.
 *  - "device" pointers are HIP device allocations on the device that was
 *    current when avsg_create ran; "host" pointers are host memory.
 *  - All buffers are caller-owned and must outlive the handle.  The library
 *    owns only the handle and a workspace it allocates in avsg_create.
 *  - avsg_match / avsg_gather / avsg_step only enqueue kernels on `stream`
 *    (a hipStream_t; NULL = the null stream).  They never synchronise, never
 *    allocate and never call hipMemset, so a step can be captured in a HIP
 *    graph and replayed; each replay reads the io buffers at the addresses
 *    given at capture time.
 *  - Bad device data never faults: an id outside a request's host rows is
 *    treated as padding and sets AVSG_ERR_OUT_OF_RANGE in that request's
 *    error counter.  The state buffers (Q, C, F, and the map) must hold what
 *    avsg_state_init and earlier steps wrote; other contents give
 *    unspecified results, with every access still in bounds.
 */
#ifndef AVSG_H
#define AVSG_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define AVSG_VERSION 1

/* Return codes. */
#define AVSG_OK 0
#define AVSG_EINVAL (-1)       /* bad argument or configuration */
#define AVSG_ENOMEM (-2)       /* workspace allocation failed */
#define AVSG_EHIP (-3)         /* a HIP runtime call failed */
#define AVSG_EUNSUPPORTED (-4) /* valid for the method, beyond this build's
                                  limits (e.g. state does not fit in LDS) */
#define AVSG_ESCRATCH (-5)     /* avsg_step_noalloc: the miss list would not
                                  fit its static scratch */

/* Per-request counters, CNT[b][0..7]; they accumulate over steps and wrap
 * modulo 2^32.  Rates are derived from them by the caller (hit rate =
 * HITS / LOOKUPS, AVSG s4.4). */
#define AVSG_CNT_HITS 0            /* valid ids found in the buffer */
#define AVSG_CNT_LOOKUPS 1         /* valid ids looked up */
#define AVSG_CNT_MISSES 2          /* ids given a new slot (one copy each) */
#define AVSG_CNT_LOST_COLLISION 3  /* links overwritten in the same scatter */
#define AVSG_CNT_LOST_EXHAUSTED 4  /* links with no reusable bucket in R+1 */
#define AVSG_CNT_LIVE_EVICTIONS 5  /* victim slots that still cached an id */
#define AVSG_CNT_ERRORS 6          /* sticky AVSG_ERR_* bits */
#define AVSG_CNT_PROBE_VISITS 7    /* buckets examined: t+1 per hit found in
                                      round t, R+1 per miss */

#define AVSG_ERR_OUT_OF_RANGE 1u   /* id not -1 and outside [0, host_rows[b]),
                                      or the request's rows leave the pool */
#define AVSG_ERR_DUPLICATE 2u      /* one token missed the same id twice */

/* Config flags. */
#define AVSG_FLAG_SKIP_GATHER 1u   /* avsg_step runs Stage One only (no host
                                      pool needed) */
/* Comparison points the AVSG page measures against (results are unchanged
 * by the two partition flags; they exist to time the alternatives). */
#define AVSG_FLAG_GATHER_BY_REQUEST 2u /* Stage Two gives each request's
                                      misses to one workgroup (request-level
                                      core assignment, AVSG s4.3) */
#define AVSG_FLAG_GATHER_BY_TOPK 4u /* Stage Two splits each token's top-K
                                      positions into equal ranges, one per
                                      workgroup, and copies the misses found
                                      in each (equal top-K partitioning,
                                      AVSG s4.3); needs topk, hit_mask and
                                      slot_table in the io */
#define AVSG_FLAG_NO_REUSE 8u      /* "KV Offload" (AVSG s4.1): no buffer
                                      reuse; avsg_match makes every valid id a
                                      miss placed at slot g*K + i (position i
                                      of query token g), in position order,
                                      and leaves Q, C, F untouched */
#define AVSG_FLAG_SORT_MERGE 16u   /* the sort-merge matcher the page
                                      compares against (GatherSelection
                                      style, AVSG s2 and s4.2): a valid id
                                      cached in some row is a hit and keeps
                                      that row (the lowest); rows not yet
                                      referenced in the step are free and the
                                      misses in ascending (id, position) take
                                      them in ascending order; no lifetimes,
                                      no hash table; C as the cached ids, Q
                                      and F untouched; end-of-step
                                      invalidation as usual */
#define AVSG_FLAG_DENSE_MAP 32u    /* match through a dense id -> slot map
                                      (avsg_buffers.map) instead of the hash
                                      table: the fixed-size integer map
                                      tensors of the GPU cache manager on the
                                      page "ECHO: Efficient KV Cache
                                      Offloading with Lossless Prefetching for
                                      Serving Native Sparse Attention LLMs".
                                      Aging, victims and invalidation are
                                      AVSG's; a valid id below map_len is a
                                      hit iff its entry m is a slot in [0, S)
                                      that caches it; installs drop the
                                      victim's old entry if it points at the
                                      victim and set the new id's entry (the
                                      largest slot among repeated ids);
                                      invalidated slots drop their entries.
                                      No mapping is ever lost; Q is untouched;
                                      PROBE_VISITS counts one per lookup.
                                      Ids at or beyond map_len are out of
                                      range (AVSG_ERR_OUT_OF_RANGE) */

typedef struct avsg_config {
    int32_t B;         /* requests (batch rows), >= 1 */
    int32_t N_q;       /* query tokens per request and step: 1 initial plus
                          N_mtp speculative ones, processed in order through
                          one shared buffer (AVSG s3.6), >= 1 */
    int32_t K;         /* selected ids per query token, 1..8192 */
    int32_t S;         /* slots (and hash buckets) per request: a power of
                          two, 16..65536, with N_q*K <= S (capacity bound,
                          AVSG App. B "Slot preservation") */
    int32_t L;         /* lifetime given on refresh or install, 1..127
                          (AVSG s3.5) */
    int32_t R;         /* probe rounds beyond the first: a lookup examines up
                          to R+1 buckets (AVSG s3.3 "Probe primitive"),
                          0..S-1 (the odd stride has visited every bucket
                          after S rounds; larger R is AVSG_EINVAL) */
    uint32_t a1;       /* odd multiplier of the home bucket (a1*x) mod S */
    uint32_t a2;       /* odd multiplier of the stride ((a2*x) mod S) | 1 */
    uint32_t a_fp;     /* odd multiplier of the 15-bit fingerprint
                          (x*a_fp mod 2^32) >> 17 kept in bucket words */
    int32_t row_bytes; /* bytes per KV row (e.g. 576 bf16 latent + 128 fp8
                          indexer key = 1280), a positive multiple of 16 */
    uint32_t flags;    /* AVSG_FLAG_* */
    int32_t gather_blocks; /* Stage-Two workgroups; 0 = chosen from the CU
                              count */
    int32_t stage1_threads; /* Stage-One workgroup size: 256, 512 or 1024
                              with K <= 8 * stage1_threads; 0 = chosen from K
                              (a tuning knob: results do not depend on it) */
} avsg_config;

/* Caller-owned buffers bound at create time. */
typedef struct avsg_buffers {
    int32_t* Q;        /* device int32 [B][S]: bucket words fp<<16 | slot,
                          -1 = empty */
    int32_t* C;        /* device int32 [B][S]: cached token id per slot,
                          -1 = empty */
    int32_t* F;        /* device int32 [B][S]: lifetime per slot, -1 = dead,
                          else 0..L */
    int32_t* CNT;      /* device int32 [B][8]: AVSG_CNT_* counters */
    void* dev_kv;      /* device bytes [B][S][row_bytes]: the slot buffer
                          attention reads; slot s of request b is row b*S+s */
    const void* host_kv; /* pinned host bytes [host_rows_total][row_bytes]
                          (from avsg_host_alloc or any pinned, device-mapped
                          allocation); may be NULL with AVSG_FLAG_SKIP_GATHER */
    int64_t host_rows_total; /* rows in host_kv */
    int32_t* map;      /* device int32 [B][map_len], AVSG_FLAG_DENSE_MAP
                          only (else ignored, may be NULL): map[b][x] = slot
                          caching id x of request b, -1 = absent */
    int64_t map_len;   /* ids per map row, >= 1 with AVSG_FLAG_DENSE_MAP */
} avsg_buffers;

/* Per-step inputs and outputs: device pointers. */
typedef struct avsg_step_io {
    const int32_t* topk;      /* int32 [B][N_q][K]: selected ids, any order,
                                 -1 = padding; ids of one token are expected
                                 distinct (AVSG_ERR_DUPLICATE otherwise) */
    const int32_t* ctx_len;   /* int32 [B]: verified context length N; ids
                                 >= N are speculative and their slots are
                                 emptied at the end of the step (AVSG App. B,
                                 "Speculative Invalidation") */
    const int64_t* row_base;  /* int64 [B]: host row of token 0 of request b */
    const int32_t* host_rows; /* int32 [B]: valid host rows of request b */
    int32_t* slot_table;      /* out int32 [B][N_q][K]: slot in [0, S) of each
                                 valid id, -1 for padding (AVSG s3.3: device
                                 positions for attention) */
    int8_t* hit_mask;         /* out int8 [B][N_q][K]: 1 hit, 0 miss,
                                 -1 padding */
    int32_t* n_miss;          /* out int32 [B][N_q]: misses of each token
                                 (the vector n of AVSG s3.3/s3.4) */
    int32_t* miss_pairs;      /* out int32 [B][N_q][K][2] or NULL: entry r of
                                 token (b,g) holds (id, slot) of its r-th
                                 smallest missing id for r < n_miss; NULL uses
                                 the library's workspace */
} avsg_step_io;

typedef struct avsg_handle avsg_handle;

int avsg_version(void);

/* Static text for a return code. */
const char* avsg_strerror(int code);

/* HIP error code (hipError_t value) of the last failing HIP call made by
 * this library on the calling thread; 0 if none. */
int avsg_last_hip_error(void);

/* Fill cfg with the given shape and the defaults L = 15, R = 7,
 * a1 = 0x9E3779B1, a2 = 0x85EBCA77, a_fp = 0xC2B2AE3D, flags = 0,
 * gather_blocks = 0, stage1_threads = 0. */
void avsg_config_default(avsg_config* cfg, int32_t B, int32_t N_q, int32_t K,
                         int32_t S, int32_t row_bytes);

/* AVSG_OK if cfg satisfies every constraint documented in avsg_config,
 * AVSG_EINVAL otherwise.  Needs no GPU. */
int avsg_validate_config(const avsg_config* cfg);

/* LDS bytes the Stage-One kernel needs for cfg (one workgroup holds one
 * request's bucket words, ids and lifetimes, 9 bytes per slot, plus per-token
 * work space; with AVSG_FLAG_SORT_MERGE the sort-merge matcher's cached ids
 * and sort keys), or 0 if cfg does not fit in 160 KiB (gfx950's
 * per-workgroup LDS); avsg_create then returns AVSG_EUNSUPPORTED.  Needs no
 * GPU. */
size_t avsg_stage1_lds_bytes(const avsg_config* cfg);

/* Device bytes avsg_create allocates for its workspace.  Needs no GPU. */
size_t avsg_workspace_bytes(const avsg_config* cfg);

/* Validate cfg and bufs, resolve the device alias of host_kv, allocate the
 * workspace and return a handle in *out.  The handle binds, per request, the
 * device buffer of S slots carried across decode steps (AVSG s3.1, Figure
 * 2) and its metadata table of bucket words, cached ids and lifetimes (AVSG
 * s3.2, the Hash-State table).  Enqueues
 * no work; the state buffers must be initialised with avsg_state_init
 * before the first step.  On failure *out is NULL and nothing is leaked. */
int avsg_create(const avsg_config* cfg, const avsg_buffers* bufs,
                avsg_handle** out);

/* Release what avsg_create allocated: the handle and its workspace (not the
 * caller's buffers, which hold the slot buffer of AVSG s3.1).  NULL is
 * accepted.  Work already enqueued must have finished. */
int avsg_destroy(avsg_handle* h);

/* Enqueue a reset of request rows to the empty state: no bucket word, no
 * cached id and every slot dead (AVSG s3.5: a dead slot is reclaimable; App.
 * B: bucket words pack a fingerprint and a slot), i.e. Q = C = F = -1,
 * CNT = 0 (and, with AVSG_FLAG_DENSE_MAP, every map entry -1).  This is the
 * empty buffer that the first MTP iteration starts from (AVSG s4.4).
 * row_mask: device int32 [B], nonzero = reset that row; NULL = all rows.
 * Uses a kernel (no hipMemset), so it may be captured in a graph. */
int avsg_state_init(avsg_handle* h, const int32_t* row_mask, void* stream);

/* Stage One (AVSG s3.3, s3.5, s3.6 and App. B): for every request, pre-decay
 * lifetimes, then for each query token in order probe, refresh hits, classify,
 * choose victims, install misses and link bucket words; finally empty the
 * slots of speculative ids.  Writes slot_table, hit_mask, n_miss, the miss
 * list, and updates Q, C, F, CNT. */
int avsg_match(avsg_handle* h, const avsg_step_io* io, void* stream);

/* Stage Two (AVSG s3.4): copy the host row of every miss listed by the last
 * avsg_match on this io into its slot of dev_kv, with the missed rows split
 * evenly across workgroups by flat miss index (not by request).  Reads
 * n_miss, the miss list, row_base and host_rows (topk, ctx_len, slot_table
 * and hit_mask may be NULL).  With AVSG_FLAG_GATHER_BY_REQUEST or
 * AVSG_FLAG_GATHER_BY_TOPK the same rows are copied under the other
 * partition; the by-top-K one reads topk, hit_mask and slot_table instead
 * of the miss list.  AVSG_EINVAL if host_kv is NULL. */
int avsg_gather(avsg_handle* h, const avsg_step_io* io, void* stream);

/* One recall step: avsg_match followed by avsg_gather (the gather is skipped
 * under AVSG_FLAG_SKIP_GATHER).  This is the operator of AVSG s3.1 (Figure
 * 2): Stage One (s3.3) resolves every selected id against the buffer as hit
 * or miss and gives each miss a slot, then Stage Two (s3.4) fetches exactly
 * the misses; attention then reads slot_table. */
int avsg_step(avsg_handle* h, const avsg_step_io* io, void* stream);

/* avsg_match for further query tokens of the step already begun by an
 * avsg_match call on the same handle: the same Stage One without the
 * once-per-step lifetime decay.  An avsg_match on tokens A followed by
 * avsg_match_continue on tokens B equals one avsg_match on the tokens
 * (A, B) in order whenever no cached or selected id is at or beyond the
 * verified length N (invalidation runs at the end of each call).  Used to
 * put prefetched candidates ahead of the exact selection.  The capacity
 * bound holds for the whole step: the handle counts the query tokens
 * enqueued since the last avsg_match (or avsg_step), and a continuation
 * that would bring that count times K above S returns AVSG_EINVAL without
 * enqueuing anything (AVSG App. B, "Slot preservation": a slot referenced
 * earlier in the step is only safe from eviction under that bound).
 * AVSG_EINVAL with AVSG_FLAG_SORT_MERGE (its step-local bookkeeping does not
 * span calls). */
int avsg_match_continue(avsg_handle* h, const avsg_step_io* io, void* stream);

/* Prefetch candidates (ECHO, decode prefetch: fetch during the indexer pass
 * every token scoring above a predicted K-th-highest score, at most a cap
 * proportional to context).  For each request b writes cand[b][0..K): the
 * first min(cap[b], K) positions j < min(ctx_len[b], row_len), ascending,
 * whose score scores[b*row_len + j] is strictly above theta[b] (float32
 * compare), then -1.  cand is meant as the topk of an avsg_match ahead of
 * the exact selection's avsg_match_continue.  Device pointers: scores float
 * [B][row_len], ctx_len int32 [B], theta float [B], cap int32 [B], cand
 * int32 [B][K].  Enqueues one kernel. */
int avsg_prefetch_select(avsg_handle* h, const float* scores, int64_t row_len,
                         const int32_t* ctx_len, const float* theta, const int32_t* cap,
                         int32_t* cand, void* stream);

/* Moving-average threshold for the next step (ECHO: alpha 0.5): for each
 * request, theta[b] = kth[b] if theta[b] is infinite (no prediction yet),
 * else alpha*kth[b] + (1 - alpha)*theta[b], each product and the sum rounded
 * to float32 separately.  kth[b] is the K-th highest score of the step just
 * selected.  Device pointers float [B]; 0 < alpha <= 1. */
int avsg_ema_threshold(avsg_handle* h, const float* kth, float* theta, float alpha,
                       void* stream);

/* Miss-list entries (id, slot pairs) the static scratch of
 * avsg_step_noalloc holds on each device: 2 MiB. */
#define AVSG_NOALLOC_MAX_PAIRS (1 << 18)

/* avsg_step for callers that cannot allocate: code under HIP graph capture,
 * serving loops that forbid hipMalloc, harnesses that own all memory.  One
 * recall step (avsg_step's semantics and results) on the current device,
 * with no handle: cfg and bufs are read on each call (same meaning and
 * checks as avsg_create), io and stream as in avsg_step.  It allocates
 * nothing, on the device or the host: when io->miss_pairs is NULL the miss
 * list lives in a static device array of AVSG_NOALLOC_MAX_PAIRS entries that
 * each device holds until the process ends, and a config whose
 * B * N_q * K exceeds that returns AVSG_ESCRATCH before anything is
 * enqueued.  The first call on a device also resolves that array's address
 * and sets the Stage-One kernels' LDS limit there (no allocation).
 * Every call on one device shares its array, and nothing in it needs to
 * start cleared (each step writes the entries it reads); calls that overlap
 * on one device, on different streams or threads, race on it, so order
 * them, or pass io->miss_pairs.  Errors as avsg_create and avsg_step. */
int avsg_step_noalloc(const avsg_config* cfg, const avsg_buffers* bufs,
                      const avsg_step_io* io, void* stream);

/* Allocate `bytes` of pinned host memory mapped into the device's address
 * space, suitable as host_kv; *out = host address.  Free with
 * avsg_host_free. */
int avsg_host_alloc(size_t bytes, void** out);
int avsg_host_free(void* p);

#ifdef __cplusplus
}
#endif

#endif /* AVSG_H */
