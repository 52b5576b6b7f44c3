/*
 * rr.h — C ABI of librr.so: RouteRelay event-triggered cross-layer routing on MI355X (gfx950).
 *
 * Source of the operations: "RouteRelay: Event-Triggered Cross-Layer Route Reuse for
 * Efficient Dynamic Sparse Attention" (arXiv 2609.07306).
 *
 *   anchor layer  (Section 4.1; Eq. 1, Eq. 2; Section 3.1 items 1-2):
 *       S = Q K^T for every query row, route R = top-k, near-miss sentinels = the next m,
 *       mandatory sink / recent sentinels (Section 3.1 item 3: chunks 0 .. sink-1 and the
 *       row's last `recent` allowed chunks, those not already in R or the near-miss set),
 *       r random sentinels drawn from the remaining allowed chunks; ledger (Eq. 4) written.
 *   relay layer   (Sections 3.2, 4.1, 4.2; Eq. 5-8):
 *       rescore each row's ledger candidates, alpha = min over R, beta = max over sentinels,
 *       reuse iff alpha > beta + gamma; flagged rows are compacted (ascending h*nq+i) and only
 *       they are routed in full and get new ledger entries (anchor layer := this layer).
 *   hysteresis    (Section 3.2, after Eq. 8), off by default: a row refreshed at relay layer a
 *       is reused untested at layers a+1 .. a+min_reuse, then tested with gamma + gamma_extra
 *       until the first layer at which it passes; rows routed at an anchor layer use gamma.
 *
 * Conventions shared by every entry point
 *   - Q is [heads, nq, d], K is [heads, nk, d], row-major and contiguous, fp32 or bf16
 *     (raw IEEE bfloat16 bits) as set by rr_config.dtype.  d must be 64.
 *   - Scores are raw dot products accumulated in fp32 (no 1/sqrt(d): that factor belongs to
 *     attention, Eq. 3).  Ties are broken by the lower chunk index.
 *   - Causal mode (rr_config.causal = 1, needs nq == nk): query chunk i may use key chunks
 *     j <= i only; rows with fewer than k + m allowed chunks keep all of them.
 *   - Random sentinels: for t = 0, 1, ...: u_t = word (t mod 4) of
 *     Philox4x32-10(counter = (t div 4, i, layer, h), key = (seed lo32, seed hi32))
 *     (Salmon et al., SC'11), j_t = (u_t * n_i) >> 32, accepted if j_t is allowed, not in the
 *     route, near-miss or mandatory set and not accepted before; stop at r accepted.  If at most r chunks
 *     remain they are all taken; after 65536 draws the lowest-index remaining chunks fill up.
 *   - Ledger layout returned by rr_ledger_get: route [heads, nq, k]; sentinels
 *     [heads, nq, m + sink + recent + r] = near-miss segment (m), mandatory segment
 *     (sink + recent), random segment (r); anchor layer [heads, nq].  Each segment ascending,
 *     padded with -1.
 *   - Device pointers are plain HIP device addresses; `stream` is a hipStream_t (NULL = the
 *     null stream).  Compute calls are asynchronous on `stream`; the caller keeps every buffer
 *     alive until that stream's work is done.  Calls on one ledger must be serialised by the
 *     caller (one stream, or explicit ordering).
 *   - Every call validates its arguments on the host before it enqueues anything.  On any
 *     error it returns a negative rr_status, leaves the ledger unchanged, and
 *     rr_last_error() describes the failure (thread-local, valid until the next call).
 *   - A failed kernel launch returns RR_EDEVICE and poisons the ledger: every call but
 *     rr_anchor_route, rr_ledger_set and rr_ledger_destroy then returns RR_ESTATE.
 */
#ifndef RR_H
#define RR_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define RR_ABI_VERSION 5

typedef enum {
    RR_OK = 0,
    RR_EINVAL = -1,        /* bad argument: null pointer, negative size, k < 1, ...         */
    RR_EUNSUPPORTED = -2,  /* valid request outside what the kernels implement (d != 64 ...) */
    RR_ENOMEM = -3,        /* device allocation failed (only rr_ledger_create allocates)     */
    RR_EDEVICE = -4,       /* a HIP runtime call or kernel launch failed                     */
    RR_ESTATE = -5         /* call not allowed in the ledger's state (see each entry point)  */
} rr_status;

typedef enum { RR_F32 = 0, RR_BF16 = 1 } rr_dtype;

typedef struct {
    int32_t heads;    /* H >= 1                                                        */
    int32_t nq;       /* query chunks per head, >= 1                                   */
    int32_t nk;       /* key chunks per head, >= 1 (== nq when causal)                 */
    int32_t d;        /* routing representation width; must be 64                     */
    int32_t k;        /* route width, >= 1                                             */
    int32_t m;        /* near-miss sentinels, >= 0                                     */
    int32_t r;        /* random sentinels, >= 0                                        */
    float gamma;      /* guard margin of Eq. 8, finite and >= 0                        */
    int32_t causal;   /* 0 or 1                                                        */
    int32_t dtype;    /* rr_dtype of Q and K                                           */
    uint64_t seed;    /* random-sentinel key                                           */
    int32_t sink;     /* mandatory sink sentinels (chunks 0 .. sink-1), >= 0           */
    int32_t recent;   /* mandatory recent sentinels (last `recent` allowed chunks), >= 0 */
    int32_t min_reuse;  /* hysteresis: layers a relay-refreshed row is reused untested, >= 0 */
    float gamma_extra;  /* hysteresis: added to gamma for a relay-refreshed row until it     *
                         * passes once; finite and >= 0 (0 and min_reuse 0: plain Eq. 8)      */
} rr_config;
/* c = k + m + sink + recent + r ledger IDs per row.  Limits (RR_EUNSUPPORTED beyond them):
 * d == 64, k + m <= 64 (k + m > 32 only with nk <= 1024), r <= 32, sink + recent <= 32,
 * (hence c <= 128), nk <= 16384 (2M tokens in 128-token chunks) with the route kernel's
 * per-block LDS within 160 KB (64 rows of nk-bit sentinel bitmaps and c-ID staging rows:
 * c <= 86 at nk = 16384, any c up to nk = 8192), nq <= 65536;
 * heads * nq < 2^31 (RR_EINVAL).  A row with fewer allowed chunks than c gets shorter
 * segments, padded with -1. */

typedef struct rr_ledger rr_ledger;   /* opaque; owns the ledger and all scratch device memory */

/* Optional outputs of rr_relay_layer: caller-owned device buffers, each may be NULL. */
typedef struct {
    uint8_t* flags;        /* [heads*nq]  1 = row failed Eq. 8 and was rerouted                  */
    int32_t* rows;         /* [heads*nq]  ascending h*nq+i of flagged rows; first n_rows valid   */
    int32_t* head_counts;  /* [heads]     flagged rows per head                                  */
    int32_t* n_rows;       /* [1]         total flagged rows (rho_l * heads * nq)                */
    float* alpha;          /* [heads*nq]  Eq. 6 at this layer                                    */
    float* beta;           /* [heads*nq]  Eq. 7 at this layer (-inf if the row has no sentinels)  */
    float* cand_scores;    /* [heads*nq*c] score of each ledger ID entering the layer, in ledger *
                            * order (route, near-miss, mandatory, random); NaN where the ID is -1 */
} rr_relay_out;

/* Check a configuration without touching the GPU. */
rr_status rr_config_check(const rr_config* cfg);

/* Allocate a ledger and its scratch memory on the current HIP device (the only allocating
 * call).  The ledger is the routing state of Section 4.1 (three row-major tensors: the route
 * IDs, the sentinel IDs and the anchor layer of each query row, Eq. 4), held in device memory
 * owned by the library until rr_ledger_destroy.  It starts empty: the first compute call on it
 * must be rr_anchor_route.  Errors: RR_EINVAL / RR_EUNSUPPORTED for a bad or unsupported
 * configuration (see rr_config_check), RR_ENOMEM if an allocation fails, RR_EDEVICE if
 * initialising it fails; *out is then NULL. */
rr_status rr_ledger_create(const rr_config* cfg, rr_ledger** out);

/* Width bucket (Section 4.4: ledgers are bucketed by route width; Section 4.3: the ledger
 * stores whichever width the routing policy asks for): a ledger over cfg->nq of the query
 * rows only, with the bucket's own k, m, r.  q_rows (host memory, copied; cfg->nq entries,
 * strictly ascending, each in [0, nq_q)) names the query row of each ledger row; the Q handed
 * to rr_anchor_route / rr_relay_layer is then [heads, nq_q, d] (all query rows), K as usual.
 * Each ledger row is routed exactly as that query row would be in a ledger over all rows
 * with the same configuration (causal limit and sentinel draws follow the query row).
 * Ledger contents, flags, alpha, beta and the compacted list are indexed by ledger row
 * (h * cfg->nq + r).  Causal buckets need nq_q == nk.  Errors as rr_ledger_create, plus
 * RR_EINVAL for a NULL or malformed q_rows. */
rr_status rr_ledger_create_rows(const rr_config* cfg, const int32_t* q_rows, int32_t nq_q,
                                rr_ledger** out);

/* Free the ledger (synchronises the device first).  NULL is ignored. */
void rr_ledger_destroy(rr_ledger* ledger);

/* Anchor layer (Section 4.1): full routing of every row at `layer` (>= 0); rebuilds the whole
 * ledger with anchor layer = `layer`.  Allowed in any state; clears a poisoned ledger. */
rr_status rr_anchor_route(rr_ledger* ledger, const void* q, const void* k, int32_t layer,
                          void* stream);

/* Relay layer (Sections 3.2, 4.1, 4.2) at `layer`: RR_ESTATE unless the ledger has been
 * anchored and `layer` is greater than the last layer it saw.  `out` may be NULL. */
rr_status rr_relay_layer(rr_ledger* ledger, const void* q, const void* k, int32_t layer,
                         void* stream, const rr_relay_out* out);

/* Width buckets (Section 4.4: rows bucketed by route width, each bucket a ledger of its own;
 * Section 4.3: the ledger holds whatever width the policy assigns) advanced together: the
 * anchor layer / relay layer of `n` ledgers (1 <= n <= RR_GROUP_MAX, host array of distinct
 * ledgers) over the same Q and K, in one kernel launch where the kernels allow it instead of
 * one launch per bucket (each of which alone would leave part of the GPU idle).  The ledgers
 * must share heads, nk, dtype, causal, the query rows per head (nq_q) and the device; their
 * k, m, r, sink, recent, gamma and hysteresis settings may differ.  Results are those of
 * calling rr_anchor_route / rr_relay_layer on each ledger in turn, which is also what runs
 * when one launch is not possible: an anchor group with a ledger of k + m > 32, a relay group
 * in which a ledger does not fit the fused kernel or asks for RR_RELAY_COMPACTED, or, with
 * every ledger on RR_RELAY_AUTO, a group outside 128 <= sum of heads * ceil(nq / 128) <= 512.
 * outs: NULL, or a host array of n pointers to optional outputs (each may be NULL), indexed as
 * the ledgers.  The relay group checks every ledger's state (as rr_relay_layer) before
 * launching anything.  Errors: RR_EINVAL for a NULL or repeated ledger, n out of range,
 * ledgers that differ in the shared settings, NULL q / k or layer < 0; RR_ESTATE as
 * rr_relay_layer; RR_EDEVICE if a launch fails (every ledger of the group is then poisoned;
 * in the one-by-one path, the failing ledger and those after it are not advanced). */
#define RR_GROUP_MAX 4
rr_status rr_anchor_route_group(rr_ledger* const* ledgers, int32_t n, const void* q, const void* k,
                                int32_t layer, void* stream);
rr_status rr_relay_layer_group(rr_ledger* const* ledgers, int32_t n, const void* q, const void* k,
                               int32_t layer, void* stream, const rr_relay_out* const* outs);

/* Allocation-free relay layer, for callers that cannot allocate (code under HIP graph capture,
 * tight serving loops, harnesses that forbid device allocation): the relay layer of
 * rr_relay_layer (same kernels and schedule as RR_RELAY_AUTO, same results) on ledger state in
 * caller-owned device memory, updated in place for the rerouted rows:
 *   ids          [heads, nq, c]  each row's route (k) then its sentinels laid out as in
 *                                rr_ledger_get (route and sent concatenated per row)
 *   anchor_layer [heads, nq]     layer of each row's last full routing
 *   refreshed    [heads, nq]     hysteresis state (see rr_ledger_get_refreshed)
 * The layer's working memory (refresh flags, reroute thresholds, per-block flagged-row lists and
 * counts) is one fixed device array of the library, 2375680 bytes per GPU, held until the
 * process ends: heads * ceil(nq / 64) * 64 must not exceed 262144 (RR_EUNSUPPORTED otherwise).
 * Nothing is allocated on the device or the host at call time.  Every call on a GPU uses that
 * GPU's array, and each call rewrites every entry it reads: calls that overlap on one GPU
 * (unordered streams) race and must not be issued.  The state is trusted to be an anchored ledger
 * of this configuration; the layer order is the caller's.  Width buckets are not served.
 * Errors: RR_EINVAL / RR_EUNSUPPORTED for the configuration (as rr_config_check), NULL pointers,
 * layer < 0 or the size limit; RR_EDEVICE if a launch fails. */
rr_status rr_relay_layer_noalloc(const rr_config* cfg, int32_t* ids, int32_t* anchor_layer, uint8_t* refreshed,
                                 const void* q, const void* k, int32_t layer, void* stream,
                                 const rr_relay_out* out);

/* How a relay layer is launched (the result is the same; only the schedule differs):
 *   RR_RELAY_FUSED      one kernel: each block takes 128 ledger rows of one head, stages the
 *                       head's keys in LDS, rescores its rows (Eq. 5-8) from there, gathers its
 *                       flagged rows into its first row slots (the compaction of Sections
 *                       4.1-4.2, within the block) and routes only those in full, as two 64-row
 *                       slices.  Needs k + m <= 32, c <= 32 and nk * d * (2 for bf16, 4 for fp32)
 *                       <= 128 KiB (nk <= 1024 in bf16).  Layers that fill the GPU with
 *                       latency-bound blocks take this path.
 *   RR_RELAY_COMPACTED  the two kernels of Section 4.2: rescoring of every row, then a reroute
 *                       grid over the layer's compacted flagged rows, 64 per block, so that the
 *                       reroute's work scales with the flagged fraction.  Large layers.
 *   RR_RELAY_AUTO       (default) fused when it fits and 128 <= heads * ceil(nq / 128) <= 512,
 *                       else compacted.
 * Errors: RR_EINVAL for a NULL ledger or an unknown mode; RR_EUNSUPPORTED for RR_RELAY_FUSED
 * outside its limits. */
typedef enum { RR_RELAY_AUTO = 0, RR_RELAY_FUSED = 1, RR_RELAY_COMPACTED = 2 } rr_relay_mode;
rr_status rr_ledger_set_relay_mode(rr_ledger* ledger, int32_t mode);

/* Copy the ledger out as the three tensors of Section 4.1 (layout above: route
 * [heads, nq, k], sentinels [heads, nq, m + sink + recent + r], anchor layer [heads, nq], all
 * int32, row-major; the caller owns the destination buffers, sized exactly so).  Any pointer may
 * be NULL to skip that tensor.  dst_is_host = 1: host memory, the call waits for `stream`;
 * 0: device memory, asynchronous.  Errors: RR_EINVAL for a NULL ledger, RR_ESTATE if the ledger
 * is poisoned, RR_EDEVICE if a copy fails. */
rr_status rr_ledger_get(const rr_ledger* ledger, int32_t* route, int32_t* sent,
                        int32_t* anchor_layer, int32_t dst_is_host, void* stream);

/* Check ledger tensors in host memory (layout of rr_ledger_get; the three tensors of Section
 * 4.1) against the rules every routing call leaves them in, without touching the GPU: per row,
 * each segment ascending with -1 padding only at its end; IDs inside the row's allowed chunks
 * [0, n_i) (n_i = query row + 1 under the causal mask, else nk) and distinct across the row's
 * segments; a full route of min(k, n_i) IDs and near-miss segment of min(m, n_i - k_i); mandatory
 * IDs among the sink chunks or the row's last `recent` allowed chunks; min(r, pool) random IDs
 * (Section 3.1); anchor layers within [0, last_layer].  q_rows / nq_q: NULL / ignored, or a
 * width bucket's query rows as in rr_ledger_create_rows.  Returns RR_OK, or RR_EINVAL naming
 * the first offending row (also for NULL tensors or a bad q_rows), RR_EINVAL /
 * RR_EUNSUPPORTED for the configuration as rr_config_check. */
rr_status rr_ledger_validate(const rr_config* cfg, const int32_t* q_rows, int32_t nq_q,
                             const int32_t* route, const int32_t* sent,
                             const int32_t* anchor_layer, int32_t last_layer);

/* Replace the whole ledger (snapshot restore / replay) with the three tensors of Section 4.1:
 * route, sent and anchor_layer are required, same layout as rr_ledger_get, caller-owned and
 * only read; `last_layer` becomes the last layer seen, so the next relay call must use a
 * greater layer.  From host memory (src_is_host = 1) the tensors are first checked as by
 * rr_ledger_validate and refused with RR_EINVAL, the ledger unchanged, if they break a rule;
 * from device memory they are trusted (IDs outside [0, nk) then count as padding in the relay
 * rescoring; a causal-violating or repeated ID is not detected).  The hysteresis state is
 * cleared (see rr_ledger_set_refreshed).  src_is_host as in rr_ledger_get.  Errors: RR_EINVAL
 * for NULL arguments, last_layer < 0 or host tensors that fail the check; RR_EDEVICE if a copy
 * fails (the ledger is then poisoned). */
rr_status rr_ledger_set(rr_ledger* ledger, const int32_t* route, const int32_t* sent,
                        const int32_t* anchor_layer, int32_t last_layer, int32_t src_is_host,
                        void* stream);

/* Hysteresis state, one byte per row [heads, nq]: 1 when the row was last routed by a
 * relay-layer refresh, 0 when by an anchor layer; with hysteresis on (min_reuse > 0 or
 * gamma_extra > 0) a relay test that a refreshed row passes under gamma + gamma_extra also
 * resets it to 0.  rr_ledger_set clears it; rr_ledger_set_refreshed restores a saved copy
 * (values 0 or 1).  Host or device memory as in rr_ledger_get / rr_ledger_set. */
rr_status rr_ledger_get_refreshed(const rr_ledger* ledger, uint8_t* refreshed, int32_t dst_is_host,
                                  void* stream);
rr_status rr_ledger_set_refreshed(rr_ledger* ledger, const uint8_t* refreshed, int32_t src_is_host,
                                  void* stream);

/* Sparse attention over routed chunks, the routes' consumer (Section 2.1: the selected chunks
 * are expanded into token indices for a sparse online-softmax kernel; Section 2.2, Eq. 3):
 * for every query token t of query chunk i, out[t] = softmax(q_t K_R^T / sqrt(64)) V_R, where
 * R is the set of tokens of the chunks listed in routes[h][i] (chunk j = tokens j*64 ..
 * j*64+63; entries outside [0, nk) are padding; in causal mode only key tokens s <= t, and
 * chunks j > i contribute nothing).  A token with no routed key gets 0.
 *   q      [heads, nq*64, 64] bf16 (raw bits), row-major
 *   k      [heads, nk*64, 64] bf16
 *   vt     [heads, nk, 64 (d), 64 (token)] bf16: V of each chunk transposed
 *   routes [heads, nq, kr] int32, e.g. the route tensor of rr_ledger_get (kr = k)
 *   out    [heads, nq*64, 64] fp32, written completely
 * All device memory owned by the caller; asynchronous on `stream`.  Scores and the softmax
 * are fp32; the probabilities enter the value product rounded to bf16.  Stateless (no
 * ledger).  Errors: RR_EINVAL for NULL pointers, sizes < 1, causal with nq != nk;
 * RR_EUNSUPPORTED for chunk_tokens != 64 or kr > 64; RR_EDEVICE if the launch fails. */
rr_status rr_sparse_attention(const void* q, const void* k, const void* vt, const int32_t* routes,
                              int32_t heads, int32_t nq, int32_t nk, int32_t kr, int32_t chunk_tokens,
                              int32_t causal, float* out, void* stream);

/* Per-kernel timing, for measurement.  While profiling is on, every kernel the ledger
 * launches is bracketed by HIP events recorded on its stream (no synchronisation, no device
 * allocation; the events are created on the host as needed, without the system-scope fence
 * that would write back the caches at every record).  rr_ledger_kernel_times waits
 * for the recorded events, writes per kernel kind the number of launches and their summed
 * duration in milliseconds (arrays of RR_KERNEL_KINDS entries, indexed by rr_kernel_kind),
 * and clears the record.  rr_ledger_profile(ledger, 1) also clears it; 0 stops recording. */
typedef enum {
    RR_KERNEL_ROUTE = 0,    /* full routing of every row (rr_anchor_route)                      */
    RR_KERNEL_RESCORE = 1,  /* candidate rescoring + flags (first kernel of a compacted relay)   */
    RR_KERNEL_REROUTE = 2,  /* full routing of the flagged rows (second kernel of a compacted relay) */
    RR_KERNEL_RELAY = 3,    /* fused relay layer: rescoring, compaction and reroute in one kernel */
    RR_KERNEL_LIST = 4,     /* compacted-list output of a fused relay (only when asked for)       */
    RR_KERNEL_KINDS = 5
} rr_kernel_kind;
rr_status rr_ledger_profile(rr_ledger* ledger, int32_t enable);
rr_status rr_ledger_kernel_times(rr_ledger* ledger, int32_t* launches, double* total_ms);

/* Configuration the ledger was created with. */
rr_status rr_ledger_config(const rr_ledger* ledger, rr_config* out);

/* Message for the last failure on this thread ("" if none). */
const char* rr_last_error(void);

int32_t rr_abi_version(void);

#ifdef __cplusplus
}
#endif
#endif /* RR_H */
