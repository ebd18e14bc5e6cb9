/*
 * CPU oracle for the per-decode-step KV recall path.
 *
 * TEST INFRASTRUCTURE ONLY.  Only tests, the smoke check and the benchmark's
 * CPU-baseline leg may load this file's library.  It shares no code, header,
 * table or constant with the GPU library: it is written from the pages alone,
 * as plain sequential C, one request and one query token at a time, in the
 * order the method states its steps.  It is slow on purpose.
 *
 * Sources (titles of the pages; sections as they number them):
 *   [AVSG] "AVSG: Accelerated Vectorized Sparse Gather for Efficient KV Cache
 *          Offload in Sparse-Attention LLM Serving"
 *     s3.1  hit = previously reserved reusable slot; miss = new slot + copy
 *     s3.3  Stage One: pre-decay (first token only), Probe, refresh to L,
 *           classify (slots o_i, miss count n_g), allocate (collect dead
 *           slots, decay all records until enough die, install, link a
 *           bucket); the Probe primitive (h, odd stride d, R+1 buckets,
 *           full cached-id compare)
 *     s3.4  Stage Two: copy host row x_i into device slot o_i for misses
 *     s3.5  per-slot lifetime counter 0..L, reclaimable after more than L
 *           unit decays
 *     s3.6  MTP tokens share one buffer and run in sequence; speculative
 *           entries are invalidated
 *     App. B "Collision and probe-budget semantics" (one packed-word
 *           scatter, exhausted probes write nothing, losers keep their slot
 *           and are copied, no false hits), "Slot preservation under
 *           sequential token processing" (capacity N_q*K <= S), and
 *           "Speculative Invalidation" (every c_j >= N becomes empty)
 *
 * Readings taken where the pages are silent (each one is listed with its
 * reason in the design notes of the repository):
 *   - S is a power of two; h = (a1*x) mod S, d = ((a2*x) mod S) | 1 in
 *     32-bit unsigned arithmetic; bucket t = (h + t*d) mod S, t = 0..R.
 *   - A bucket word packs fp(x) << 16 | slot with fp(x) = (x*afp mod 2^32)
 *     >> 17 (15 bits); EMPTY = -1.  Lookup compares only the cached id.
 *   - Lifetimes live per slot in {-1 (dead)} U [0, L]; every decay clamps
 *     at -1.
 *   - Extra decay k* is the least k >= 0 with #{j : F[j] < k} >= n_g; all
 *     slots are decayed by k*; victims are the n_g lowest-index dead slots;
 *     the r-th smallest missing id takes the r-th victim.
 *   - A bucket is reusable if EMPTY, if its slot is empty (C = -1) or if
 *     its fingerprint differs from fp(C[slot]).  Reusability is judged on Q
 *     before this token's link writes and on C after this token's installs;
 *     when several misses claim one bucket the largest rank wins.
 *   - Ids equal to -1 are padding; any other id outside [0, host_rows[b]),
 *     or any id of a request whose host-row range lies outside the pool, is
 *     treated as padding and sets bit 0 of the request's error word.
 *     Duplicate missing ids within a token set bit 1 and are kept as
 *     separate misses, ordered by (id, position).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORC_EMPTY (-1)

/* Counter layout per request (8 x int32, accumulating across steps). */
enum {
    ORC_HITS = 0, ORC_LOOKUPS = 1, ORC_MISSES = 2, ORC_LOST_COLLISION = 3,
    ORC_LOST_EXHAUSTED = 4, ORC_LIVE_EVICTIONS = 5, ORC_ERRORS = 6,
    ORC_PROBE_VISITS = 7
};

/* Return codes: 0 ok; negative = the oracle caught a broken invariant. */
#define ORC_OK 0
#define ORC_EARG (-1)
#define ORC_EREVICT (-2)    /* a slot referenced earlier in the step was evicted */
#define ORC_ELIFE (-3)      /* a lifetime left [-1, L] */
#define ORC_ENOMEM (-4)

typedef struct {
    int32_t B, Nq, K, S, L, R;
    uint32_t a1, a2, afp;
    int64_t row_bytes;
    int64_t host_rows_total;
} orc_cfg;

typedef struct { int32_t id; int32_t pos; } orc_miss;

int orc_version(void) { return 1; }

/* ---- hash layer (AVSG s3.3, "Probe primitive"; App. B packed words) ---- */

static uint32_t home_bucket(const orc_cfg* c, int32_t x) {
    return (c->a1 * (uint32_t)x) % (uint32_t)c->S;
}

static uint32_t probe_stride(const orc_cfg* c, int32_t x) {
    return ((c->a2 * (uint32_t)x) % (uint32_t)c->S) | 1u;
}

static uint32_t bucket_at(const orc_cfg* c, int32_t x, int32_t t) {
    uint64_t h = home_bucket(c, x), d = probe_stride(c, x);
    return (uint32_t)((h + (uint64_t)t * d) % (uint64_t)c->S);
}

static int32_t fingerprint(const orc_cfg* c, int32_t x) {
    return (int32_t)(((uint32_t)x * c->afp) >> 17);
}

static int32_t pack_word(int32_t fp, int32_t slot) {
    return (int32_t)(((uint32_t)fp << 16) | (uint32_t)slot);
}

static int32_t word_slot(int32_t w) { return (int32_t)((uint32_t)w & 0xFFFFu); }
static int32_t word_fp(int32_t w) { return (int32_t)((uint32_t)w >> 16); }

/* Lookup of one id: first t in 0..R whose bucket word leads to a slot that
 * caches x.  Returns the slot or -1; *visits = buckets examined. */
static int32_t lookup(const orc_cfg* c, const int32_t* Q, const int32_t* C,
                      int32_t x, int32_t* visits) {
    for (int32_t t = 0; t <= c->R; ++t) {
        int32_t w = Q[bucket_at(c, x, t)];
        if (w != ORC_EMPTY && C[word_slot(w)] == x) {
            *visits = t + 1;
            return word_slot(w);
        }
    }
    *visits = c->R + 1;
    return -1;
}

static int bucket_reusable(const orc_cfg* c, const int32_t* C, int32_t w) {
    if (w == ORC_EMPTY) return 1;
    int32_t cached = C[word_slot(w)];
    if (cached == -1) return 1;
    return fingerprint(c, cached) != word_fp(w);
}

static int cmp_miss(const void* a, const void* b) {
    const orc_miss* p = (const orc_miss*)a;
    const orc_miss* q = (const orc_miss*)b;
    if (p->id != q->id) return p->id < q->id ? -1 : 1;
    if (p->pos != q->pos) return p->pos < q->pos ? -1 : 1;
    return 0;
}

static int32_t max32(int32_t a, int32_t b) { return a > b ? a : b; }

/* Counters wrap modulo 2^32, like any 32-bit event counter. */
static void bump(int32_t* c, int64_t v) {
    *c = (int32_t)((uint32_t)*c + (uint32_t)v);
}

/*
 * One recall step for every request.
 *
 * State (in/out, row-major):  Q, C, F  int32 [B][S];  CNT int32 [B][8].
 * Inputs:  topk int32 [B][Nq][K]; ctx_len int32 [B]; row_base int64 [B];
 *          host_rows int32 [B]; host_kv uint8 [host_rows_total][row_bytes]
 *          (may be NULL together with dev_shadow to skip the copy).
 * Outputs: slot_table int32 [B][Nq][K]; hit_mask int8 [B][Nq][K];
 *          n_miss int32 [B][Nq]; miss_pairs int32 [B][Nq][K][2] holding
 *          (id, slot) of the r-th miss at r (entries beyond n_g untouched);
 *          dev_shadow uint8 [B][S][row_bytes], the device slot buffer.
 */
int orc_step(const orc_cfg* cfg, int32_t* Qall, int32_t* Call, int32_t* Fall,
             int32_t* CNTall, const int32_t* topk, const int32_t* ctx_len,
             const int64_t* row_base, const int32_t* host_rows,
             const uint8_t* host_kv, uint8_t* dev_shadow,
             int32_t* slot_table, int8_t* hit_mask, int32_t* n_miss,
             int32_t* miss_pairs)
{
    const int32_t B = cfg->B, Nq = cfg->Nq, K = cfg->K, S = cfg->S, L = cfg->L;
    /* R <= S - 1: an odd stride modulo a power of two has visited every
     * bucket after S rounds, so further rounds would only revisit them. */
    if (B < 0 || Nq < 1 || K < 1 || S < 1 || (S & (S - 1)) != 0 || S > 65536 ||
        (int64_t)Nq * K > S || L < 1 || L > 127 || cfg->R < 0 || cfg->R > S - 1)
        return ORC_EARG;

    orc_miss* misses = (orc_miss*)malloc(sizeof(orc_miss) * (size_t)K);
    int32_t* miss_slot_of = (int32_t*)malloc(sizeof(int32_t) * (size_t)K);
    int32_t* victims = (int32_t*)malloc(sizeof(int32_t) * (size_t)K);
    int32_t* target = (int32_t*)malloc(sizeof(int32_t) * (size_t)K);
    uint8_t* referenced = (uint8_t*)malloc((size_t)S);
    int32_t* found = (int32_t*)malloc(sizeof(int32_t) * (size_t)K);
    if (!misses || !miss_slot_of || !victims || !target || !referenced || !found) {
        free(misses); free(miss_slot_of); free(victims); free(target);
        free(referenced); free(found);
        return ORC_ENOMEM;
    }
    int rc = ORC_OK;

    for (int32_t b = 0; b < B && rc == ORC_OK; ++b) {
        int32_t* Q = Qall + (int64_t)b * S;
        int32_t* C = Call + (int64_t)b * S;
        int32_t* F = Fall + (int64_t)b * S;
        int32_t* cnt = CNTall + (int64_t)b * 8;
        const int row_ok = row_base[b] >= 0 && host_rows[b] >= 0 &&
                           row_base[b] + host_rows[b] <= cfg->host_rows_total;
        memset(referenced, 0, (size_t)S);

        /* Pass 1 prologue: one unit decay of every lifetime, once per request
         * per step, before its first token (AVSG s3.3; App. B). */
        for (int32_t j = 0; j < S; ++j) F[j] = max32(F[j] - 1, -1);

        /* MTP tokens one after another on the same table (AVSG s3.6). */
        for (int32_t g = 0; g < Nq; ++g) {
            const int64_t tok = (int64_t)b * Nq + g;
            const int32_t* X = topk + tok * K;
            int32_t* O = slot_table + tok * K;
            int8_t* H = hit_mask + tok * K;
            int32_t n_valid = 0, n_hit = 0, n_g = 0;

            /* Valid set, Probe, refresh, classify (AVSG s3.3). */
            for (int32_t i = 0; i < K; ++i) {
                int32_t x = X[i];
                found[i] = -1;
                if (x == -1) { O[i] = -1; H[i] = -1; continue; }
                if (!row_ok || x < 0 || x >= host_rows[b]) {
                    cnt[ORC_ERRORS] |= 1;
                    O[i] = -1; H[i] = -1; continue;
                }
                int32_t visits = 0;
                found[i] = lookup(cfg, Q, C, x, &visits);
                bump(&cnt[ORC_PROBE_VISITS], visits);
                ++n_valid;
                if (found[i] < 0) {
                    misses[n_g].id = x;
                    misses[n_g].pos = i;
                    ++n_g;
                }
            }
            /* Refresh every matched slot to L, then record hit slots. */
            for (int32_t i = 0; i < K; ++i) {
                if (found[i] >= 0) {
                    F[found[i]] = L;
                    O[i] = found[i];
                    H[i] = 1;
                    referenced[found[i]] = 1;
                    ++n_hit;
                }
            }
            n_miss[tok] = n_g;

            /* Misses in ascending token id. */
            qsort(misses, (size_t)n_g, sizeof(orc_miss), cmp_miss);
            for (int32_t r = 1; r < n_g; ++r)
                if (misses[r].id == misses[r - 1].id) cnt[ORC_ERRORS] |= 2;

            int32_t lost_exh = 0, lost_col = 0, live_ev = 0;
            if (n_g > 0) {
                /* Pass 3 (a)-(b): decay all records further, by the least
                 * amount that leaves at least n_g dead slots. */
                int32_t kstar = 0;
                for (;;) {
                    int32_t below = 0;
                    for (int32_t j = 0; j < S; ++j) below += (F[j] < kstar);
                    if (below >= n_g) break;
                    ++kstar;
                }
                for (int32_t j = 0; j < S; ++j) F[j] = max32(F[j] - kstar, -1);

                /* CollectDead: the n_g lowest-index dead slots. */
                int32_t nv = 0;
                for (int32_t j = 0; j < S && nv < n_g; ++j)
                    if (F[j] == -1) victims[nv++] = j;

                /* Pass 3 (c): install the r-th miss into the r-th victim. */
                for (int32_t r = 0; r < n_g; ++r) {
                    int32_t v = victims[r];
                    if (referenced[v]) rc = ORC_EREVICT;
                    if (C[v] >= 0) ++live_ev;
                    C[v] = misses[r].id;
                    F[v] = L;
                    O[misses[r].pos] = v;
                    H[misses[r].pos] = 0;
                    referenced[v] = 1;
                    miss_slot_of[r] = v;
                    if (miss_pairs) {
                        int32_t* mp = miss_pairs + (tok * K + r) * 2;
                        mp[0] = misses[r].id;
                        mp[1] = v;
                    }
                }

                /* Pass 3 (d): each miss claims the first reusable bucket of
                 * its probe sequence, judged before any link write of this
                 * token; then one scatter in rank order, so the largest rank
                 * survives on a contested bucket. */
                for (int32_t r = 0; r < n_g; ++r) {
                    target[r] = -1;
                    for (int32_t t = 0; t <= cfg->R; ++t) {
                        uint32_t p = bucket_at(cfg, misses[r].id, t);
                        if (bucket_reusable(cfg, C, Q[p])) { target[r] = (int32_t)p; break; }
                    }
                    if (target[r] < 0) ++lost_exh;
                }
                for (int32_t r = 0; r < n_g; ++r)
                    if (target[r] >= 0)
                        Q[target[r]] = pack_word(fingerprint(cfg, misses[r].id), miss_slot_of[r]);
                for (int32_t r = 0; r < n_g; ++r)
                    if (target[r] >= 0 &&
                        Q[target[r]] != pack_word(fingerprint(cfg, misses[r].id), miss_slot_of[r]))
                        ++lost_col;
            }

            bump(&cnt[ORC_HITS], n_hit);
            bump(&cnt[ORC_LOOKUPS], n_valid);
            bump(&cnt[ORC_MISSES], n_g);
            bump(&cnt[ORC_LOST_COLLISION], lost_col);
            bump(&cnt[ORC_LOST_EXHAUSTED], lost_exh);
            bump(&cnt[ORC_LIVE_EVICTIONS], live_ev);
        }

        /* End of step: every slot caching a position at or beyond the
         * verified length becomes empty (AVSG App. B, Speculative
         * Invalidation).  Lifetimes and bucket words stay. */
        for (int32_t j = 0; j < S; ++j)
            if (C[j] >= ctx_len[b]) C[j] = -1;

        for (int32_t j = 0; j < S; ++j)
            if (F[j] < -1 || F[j] > L) rc = ORC_ELIFE;
    }

    /* Stage Two: copy each missed row from the host pool into its slot, in
     * (request, token, rank) order (AVSG s3.4). */
    if (rc == ORC_OK && host_kv && dev_shadow && miss_pairs) {
        const int64_t rb = cfg->row_bytes;
        for (int32_t b = 0; b < B; ++b)
            for (int32_t g = 0; g < Nq; ++g) {
                const int64_t tok = (int64_t)b * Nq + g;
                for (int32_t r = 0; r < n_miss[tok]; ++r) {
                    const int32_t* mp = miss_pairs + (tok * K + r) * 2;
                    memcpy(dev_shadow + ((int64_t)b * S + mp[1]) * rb,
                           host_kv + (row_base[b] + mp[0]) * rb, (size_t)rb);
                }
            }
    }

    free(misses); free(miss_slot_of); free(victims); free(target);
    free(referenced); free(found);
    return rc;
}

/*
 * AVSG's slot management with a dense id -> slot map in place of the hash
 * table: the fixed-size integer map tensors of ECHO's GPU cache manager
 * (host-slot -> GPU-slot map).  Everything but the lookup and the link is
 * orc_step: pre-decay, refresh to L, ascending misses, least extra decay,
 * lowest-index dead victims, end-of-step invalidation.  Readings taken:
 *   - a valid id x (also x < map_len) is a hit iff m = map[x] is a slot in
 *     [0, S) that caches x (C[m] == x); its slot is m.  Entries only ever
 *     point at slots caching their id, so the check never rejects a map this
 *     step built; it keeps a stale or foreign map harmless.  No mapping is
 *     lost, so there is no collision or exhaustion;
 *   - installing x into slot v first clears the entry of v's old id if it
 *     still points at v, then sets map[x] = v (so among repeated missing ids
 *     the larger rank keeps the entry);
 *   - invalidating slot j clears its id's entry if it points at j.
 * Q is not used.  Counters as orc_step, with one probe visit per lookup.
 */
int orc_step_dense(const orc_cfg* cfg, int32_t* Call, int32_t* Fall, int32_t* CNTall,
                   int32_t* map_all, int64_t map_len, const int32_t* topk,
                   const int32_t* ctx_len, const int64_t* row_base,
                   const int32_t* host_rows, const uint8_t* host_kv, uint8_t* dev_shadow,
                   int32_t* slot_table, int8_t* hit_mask, int32_t* n_miss,
                   int32_t* miss_pairs)
{
    const int32_t B = cfg->B, Nq = cfg->Nq, K = cfg->K, S = cfg->S, L = cfg->L;
    if (B < 0 || Nq < 1 || K < 1 || S < 1 || (int64_t)Nq * K > S || L < 1 || L > 127 ||
        map_len < 1)
        return ORC_EARG;
    orc_miss* misses = (orc_miss*)malloc(sizeof(orc_miss) * (size_t)K);
    int32_t* victims = (int32_t*)malloc(sizeof(int32_t) * (size_t)K);
    if (!misses || !victims) { free(misses); free(victims); return ORC_ENOMEM; }
    int rc = ORC_OK;
    for (int32_t b = 0; b < B && rc == ORC_OK; ++b) {
        int32_t* C = Call + (int64_t)b * S;
        int32_t* F = Fall + (int64_t)b * S;
        int32_t* map = map_all + (int64_t)b * map_len;
        int32_t* cnt = CNTall + (int64_t)b * 8;
        const int row_ok = row_base[b] >= 0 && host_rows[b] >= 0 &&
                           row_base[b] + host_rows[b] <= cfg->host_rows_total;
        for (int32_t j = 0; j < S; ++j) F[j] = max32(F[j] - 1, -1);
        for (int32_t g = 0; g < Nq; ++g) {
            const int64_t tok = (int64_t)b * Nq + g;
            const int32_t* X = topk + tok * K;
            int32_t* O = slot_table + tok * K;
            int8_t* H = hit_mask + tok * K;
            int32_t n_valid = 0, n_hit = 0, n_g = 0, live = 0;
            for (int32_t i = 0; i < K; ++i) {
                int32_t x = X[i];
                O[i] = -1; H[i] = -1;
                if (x == -1) continue;
                if (!row_ok || x < 0 || x >= host_rows[b] || x >= map_len) {
                    cnt[ORC_ERRORS] |= 1;
                    continue;
                }
                ++n_valid;
                const int32_t m = map[x];
                if (m >= 0 && m < S && C[m] == x) {
                    O[i] = m; H[i] = 1; ++n_hit;
                } else {
                    misses[n_g].id = x; misses[n_g].pos = i; ++n_g;
                }
            }
            for (int32_t i = 0; i < K; ++i)
                if (H[i] == 1) F[O[i]] = L;
            n_miss[tok] = n_g;
            qsort(misses, (size_t)n_g, sizeof(orc_miss), cmp_miss);
            for (int32_t r = 1; r < n_g; ++r)
                if (misses[r].id == misses[r - 1].id) cnt[ORC_ERRORS] |= 2;
            if (n_g > 0) {
                int32_t kstar = 0;
                for (;;) {
                    int32_t below = 0;
                    for (int32_t j = 0; j < S; ++j) below += (F[j] < kstar);
                    if (below >= n_g) break;
                    ++kstar;
                }
                for (int32_t j = 0; j < S; ++j) F[j] = max32(F[j] - kstar, -1);
                int32_t nv = 0;
                for (int32_t j = 0; j < S && nv < n_g; ++j)
                    if (F[j] == -1) victims[nv++] = j;
                for (int32_t r = 0; r < n_g; ++r) {
                    const int32_t v = victims[r], x = misses[r].id;
                    if (C[v] >= 0) {
                        ++live;
                        if (C[v] < map_len && map[C[v]] == v) map[C[v]] = -1;
                    }
                    C[v] = x;
                    F[v] = L;
                    map[x] = v;
                    O[misses[r].pos] = v;
                    H[misses[r].pos] = 0;
                    if (miss_pairs) {
                        int32_t* mp = miss_pairs + (tok * K + r) * 2;
                        mp[0] = x;
                        mp[1] = v;
                    }
                }
            }
            bump(&cnt[ORC_HITS], n_hit);
            bump(&cnt[ORC_LOOKUPS], n_valid);
            bump(&cnt[ORC_MISSES], n_g);
            bump(&cnt[ORC_LIVE_EVICTIONS], live);
            bump(&cnt[ORC_PROBE_VISITS], n_valid);
        }
        for (int32_t j = 0; j < S; ++j) {
            if (C[j] >= ctx_len[b]) {
                if (C[j] >= 0 && C[j] < map_len && map[C[j]] == j) map[C[j]] = -1;
                C[j] = -1;
            }
        }
    }
    free(misses);
    free(victims);
    if (rc == ORC_OK && host_kv && dev_shadow && miss_pairs) {
        const int64_t rb = cfg->row_bytes;
        for (int32_t b = 0; b < B; ++b)
            for (int32_t g = 0; g < Nq; ++g) {
                const int64_t tok = (int64_t)b * Nq + g;
                for (int32_t r = 0; r < n_miss[tok]; ++r) {
                    const int32_t* mp = miss_pairs + (tok * K + r) * 2;
                    memcpy(dev_shadow + ((int64_t)b * S + mp[1]) * rb,
                           host_kv + (row_base[b] + mp[0]) * rb, (size_t)rb);
                }
            }
    }
    return rc;
}

/*
 * The "KV Offload" configuration the AVSG page compares against (section
 * 4.1): the whole KV cache stays in host memory and every selected entry is
 * transferred at every decode step, with no reuse.  Reading taken: the entry
 * at position i of query token g of a request lands in that request's slot
 * g*K + i (a fixed, position-indexed destination; N_q*K <= S).  Every valid
 * id is a miss; the miss list holds (id, slot) in position order.  Padding
 * and out-of-range ids are treated as in orc_step.  Q, C and F are not used;
 * the LOOKUPS and MISSES counters grow by the valid ids, ERRORS as usual.
 */
int orc_step_no_reuse(const orc_cfg* cfg, int32_t* CNTall, const int32_t* topk,
                      const int64_t* row_base, const int32_t* host_rows,
                      const uint8_t* host_kv, uint8_t* dev_shadow,
                      int32_t* slot_table, int8_t* hit_mask, int32_t* n_miss,
                      int32_t* miss_pairs)
{
    const int32_t B = cfg->B, Nq = cfg->Nq, K = cfg->K, S = cfg->S;
    if (B < 0 || Nq < 1 || K < 1 || S < 1 || (int64_t)Nq * K > S) return ORC_EARG;
    for (int32_t b = 0; b < B; ++b) {
        int32_t* cnt = CNTall + (int64_t)b * 8;
        const int row_ok = row_base[b] >= 0 && host_rows[b] >= 0 &&
                           row_base[b] + host_rows[b] <= cfg->host_rows_total;
        for (int32_t g = 0; g < Nq; ++g) {
            const int64_t tok = (int64_t)b * Nq + g;
            const int32_t* X = topk + tok * K;
            int32_t* O = slot_table + tok * K;
            int8_t* H = hit_mask + tok * K;
            int32_t n = 0;
            for (int32_t i = 0; i < K; ++i) {
                int32_t x = X[i];
                if (x == -1) { O[i] = -1; H[i] = -1; continue; }
                if (!row_ok || x < 0 || x >= host_rows[b]) {
                    cnt[ORC_ERRORS] |= 1;
                    O[i] = -1; H[i] = -1; continue;
                }
                O[i] = g * K + i;
                H[i] = 0;
                if (miss_pairs) {
                    int32_t* mp = miss_pairs + (tok * K + n) * 2;
                    mp[0] = x;
                    mp[1] = g * K + i;
                }
                ++n;
            }
            n_miss[tok] = n;
            bump(&cnt[ORC_LOOKUPS], n);
            bump(&cnt[ORC_MISSES], n);
        }
    }
    if (host_kv && dev_shadow && miss_pairs) {
        const int64_t rb = cfg->row_bytes;
        for (int32_t b = 0; b < B; ++b)
            for (int32_t g = 0; g < Nq; ++g) {
                const int64_t tok = (int64_t)b * Nq + g;
                for (int32_t r = 0; r < n_miss[tok]; ++r) {
                    const int32_t* mp = miss_pairs + (tok * K + r) * 2;
                    memcpy(dev_shadow + ((int64_t)b * S + mp[1]) * rb,
                           host_kv + (row_base[b] + mp[0]) * rb, (size_t)rb);
                }
            }
    }
    return ORC_OK;
}

/*
 * The sort-merge matcher the AVSG page compares its hash matching against
 * (GatherSelection, section 2; the scalar dual-pointer baseline of section
 * 4.2): exact reuse of cached token ids with no lifetimes and no hash table.
 * Readings taken, per request and query token in order, on the cached ids C:
 *   - a valid id x is a hit iff some row caches it; the hit keeps its row
 *     (the lowest such row);
 *   - rows not referenced by this step's tokens so far are free; the
 *     token's misses in ascending (id, position) order take the free rows in
 *     ascending order, which now cache them;
 *   - at the end of the step every row caching an id >= N is emptied, as in
 *     orc_step.
 * Padding and out-of-range ids are treated as in orc_step.  Q and F are not
 * used.  Counters: HITS, LOOKUPS, MISSES, LIVE_EVICTIONS, ERRORS.
 */
int orc_step_sort_merge(const orc_cfg* cfg, int32_t* Call, int32_t* CNTall,
                        const int32_t* topk, const int32_t* ctx_len,
                        const int64_t* row_base, const int32_t* host_rows,
                        const uint8_t* host_kv, uint8_t* dev_shadow,
                        int32_t* slot_table, int8_t* hit_mask, int32_t* n_miss,
                        int32_t* miss_pairs)
{
    const int32_t B = cfg->B, Nq = cfg->Nq, K = cfg->K, S = cfg->S;
    if (B < 0 || Nq < 1 || K < 1 || S < 1 || (int64_t)Nq * K > S) return ORC_EARG;
    orc_miss* misses = (orc_miss*)malloc(sizeof(orc_miss) * (size_t)K);
    uint8_t* referenced = (uint8_t*)malloc((size_t)S);
    if (!misses || !referenced) { free(misses); free(referenced); return ORC_ENOMEM; }
    for (int32_t b = 0; b < B; ++b) {
        int32_t* C = Call + (int64_t)b * S;
        int32_t* cnt = CNTall + (int64_t)b * 8;
        const int row_ok = row_base[b] >= 0 && host_rows[b] >= 0 &&
                           row_base[b] + host_rows[b] <= cfg->host_rows_total;
        memset(referenced, 0, (size_t)S);
        for (int32_t g = 0; g < Nq; ++g) {
            const int64_t tok = (int64_t)b * Nq + g;
            const int32_t* X = topk + tok * K;
            int32_t* O = slot_table + tok * K;
            int8_t* H = hit_mask + tok * K;
            int32_t n_valid = 0, n_hit = 0, n_g = 0, live = 0;
            /* Hits against the rows as they stand before this token's
             * installs. */
            for (int32_t i = 0; i < K; ++i) {
                int32_t x = X[i];
                O[i] = -1; H[i] = -1;
                if (x == -1) continue;
                if (!row_ok || x < 0 || x >= host_rows[b]) { cnt[ORC_ERRORS] |= 1; continue; }
                ++n_valid;
                int32_t row = -1;
                for (int32_t j = 0; j < S; ++j)
                    if (C[j] == x) { row = j; break; }
                if (row >= 0) {
                    O[i] = row; H[i] = 1; ++n_hit;
                } else {
                    misses[n_g].id = x; misses[n_g].pos = i; ++n_g;
                }
            }
            for (int32_t i = 0; i < K; ++i)
                if (H[i] == 1) referenced[O[i]] = 1;
            qsort(misses, (size_t)n_g, sizeof(orc_miss), cmp_miss);
            for (int32_t r = 1; r < n_g; ++r)
                if (misses[r].id == misses[r - 1].id) cnt[ORC_ERRORS] |= 2;
            int32_t j = 0;
            for (int32_t r = 0; r < n_g; ++r) {
                while (j < S && referenced[j]) ++j;
                if (j >= S) { free(misses); free(referenced); return ORC_EREVICT; }
                if (C[j] >= 0) ++live;
                C[j] = misses[r].id;
                referenced[j] = 1;
                O[misses[r].pos] = j;
                H[misses[r].pos] = 0;
                if (miss_pairs) {
                    int32_t* mp = miss_pairs + (tok * K + r) * 2;
                    mp[0] = misses[r].id;
                    mp[1] = j;
                }
            }
            n_miss[tok] = n_g;
            bump(&cnt[ORC_HITS], n_hit);
            bump(&cnt[ORC_LOOKUPS], n_valid);
            bump(&cnt[ORC_MISSES], n_g);
            bump(&cnt[ORC_LIVE_EVICTIONS], live);
        }
        for (int32_t j = 0; j < S; ++j)
            if (C[j] >= ctx_len[b]) C[j] = -1;
    }
    free(misses);
    free(referenced);
    if (host_kv && dev_shadow && miss_pairs) {
        const int64_t rb = cfg->row_bytes;
        for (int32_t b = 0; b < B; ++b)
            for (int32_t g = 0; g < Nq; ++g) {
                const int64_t tok = (int64_t)b * Nq + g;
                for (int32_t r = 0; r < n_miss[tok]; ++r) {
                    const int32_t* mp = miss_pairs + (tok * K + r) * 2;
                    memcpy(dev_shadow + ((int64_t)b * S + mp[1]) * rb,
                           host_kv + (row_base[b] + mp[0]) * rb, (size_t)rb);
                }
            }
    }
    return ORC_OK;
}

/*
 * Threshold prefetch ahead of the recall (ECHO page, decode prefetch): while
 * the indexer scores every earlier token, tokens scoring above a predicted
 * threshold are fetched at once, at most a capped number; the threshold is
 * a moving average (alpha) of the observed K-th highest scores.
 * Readings taken: candidates are the first min(cap, K) positions j below
 * min(N, row_len), in ascending order, with score strictly above theta
 * (float32); the rest of the row is -1.  The average starts from the first
 * observed score when theta is infinite.
 */
void orc_prefetch_select(const orc_cfg* cfg, const float* scores, int64_t row_len,
                         const int32_t* ctx_len, const float* theta, const int32_t* cap,
                         int32_t* cand)
{
    for (int32_t b = 0; b < cfg->B; ++b) {
        int64_t n = ctx_len[b] < 0 ? 0 : ctx_len[b];
        if (n > row_len) n = row_len;
        int32_t c = cap[b] < 0 ? 0 : cap[b];
        if (c > cfg->K) c = cfg->K;
        int32_t* out = cand + (int64_t)b * cfg->K;
        int32_t m = 0;
        for (int64_t j = 0; j < n && m < c; ++j)
            if (scores[(int64_t)b * row_len + j] > theta[b]) out[m++] = (int32_t)j;
        for (int32_t i = m; i < cfg->K; ++i) out[i] = -1;
    }
}

void orc_ema_threshold(int32_t B, const float* kth, float* theta, float alpha)
{
    for (int32_t b = 0; b < B; ++b) {
        if (isinf(theta[b])) {
            theta[b] = kth[b];
        } else {
            const float p = alpha * kth[b];
            const float q = (1.0f - alpha) * theta[b];
            theta[b] = p + q;
        }
    }
}

/* Empty state: no bucket words, no cached ids, all slots dead, counters 0. */
void orc_state_reset(const orc_cfg* cfg, int32_t* Q, int32_t* C, int32_t* F,
                     int32_t* CNT)
{
    const int64_t n = (int64_t)cfg->B * cfg->S;
    for (int64_t j = 0; j < n; ++j) { Q[j] = ORC_EMPTY; C[j] = -1; F[j] = -1; }
    for (int64_t j = 0; j < (int64_t)cfg->B * 8; ++j) CNT[j] = 0;
}

/* The R+1 buckets a lookup of x examines, in order (for tests). */
void orc_probe_buckets(const orc_cfg* cfg, int32_t x, int32_t* out)
{
    for (int32_t t = 0; t <= cfg->R; ++t) out[t] = (int32_t)bucket_at(cfg, x, t);
}

/* The fingerprint and packed word the link step would store (for tests). */
int32_t orc_word(const orc_cfg* cfg, int32_t x, int32_t slot)
{
    return pack_word(fingerprint(cfg, x), slot);
}
