/*
 * moonep.h -- C-ABI of the MI355X (gfx950) balanced expert-parallel hot path.
 *
 * What is computed follows these pages:
 *   [NCIJ]  "Moonshot AI Open-Sources MoonEP: A Perfectly Balanced Expert
 *           Parallelism Library for MoE Training" (ncijnetwork.com), sections
 *           "The problem MoonEP targets" and "The core idea: dynamic redundant
 *           experts", the three-property list, and the interactive explainer
 *           (panels "invariant", "memory", "maxvio", "pillars").
 *   [AIPDB] "Moonshot AI open-sources MoonEP for distributed MoE
 *           communication" (aipricedb.com), the README excerpt on zero copy.
 *
 * Model.  R ranks hold E experts, L = E/R each; expert e lives on rank
 * home(e) = e div L.  Each rank has S tokens and each token is routed to K
 * experts, so rank r's routed entries are n = (r*S + t)*K + k.  Every rank
 * receives exactly C = S*K rows whatever the routing skew [NCIJ "The core
 * idea"]: overfull ranks hand whole-expert amounts (lowest expert id first)
 * to redundant copies ("replicas") of those experts hosted on underfull ranks,
 * matched two-pointer in expert order against the deficits in rank order.
 * The R ranks are logical: rank r's [C, H] bf16 buffer is rows [r*C, (r+1)*C)
 * of one device allocation.
 *
 * A step.  Forward: moonep_route_stats, moonep_plan, moonep_weight_slots and
 * moonep_prefetch_weights (the replicas' weights), moonep_dispatch, the expert
 * computation over the buffer (moonep_expert_gemm per projection, with the
 * caller's activation between projections), moonep_combine.  Backward:
 * moonep_combine_bwd, the expert's backward (the caller's), moonep_dispatch_bwd,
 * and moonep_replica_grad_reduce for the replicas' weight-gradients.
 *
 * Conventions shared by every call:
 *  - All array arguments are DEVICE pointers owned by the caller; the library
 *    allocates nothing.  Between calls it keeps only the CU's LDS size (read
 *    once per process) and, per device, whether one kernel's dynamic-LDS limit
 *    has been raised for large E and R.
 *  - `stream` is a hipStream_t passed as void* (NULL = the null stream).  Every
 *    call only enqueues work; none waits for the device, except
 *    moonep_read_error.  Output sizes depend on the shape alone, so no call
 *    needs to read device results on the host [NCIJ explainer "invariant"
 *    panel: static shapes, no per-layer host synchronisation].
 *  - Return value: MOONEP_OK, or a negative MOONEP_ERR_* found on the host
 *    before anything is enqueued (or MOONEP_ERR_HIP if a launch fails).
 *  - Device-side faults in the data (an expert id outside [0, E)) set a sticky
 *    error word in the workspace; read it with moonep_read_error.  Outputs of a
 *    call that saw bad data are unspecified, but every access stays in bounds.
 *  - bf16 arrays are raw 16-bit patterns (uint16_t) and must be 16-byte aligned;
 *    int32/fp32 arrays must be 4-byte aligned.
 */
#ifndef MOONEP_H
#define MOONEP_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct moonep_shape {
    int32_t R; /* ranks (logical), >= 1 */
    int32_t E; /* experts, E % R == 0 [NCIJ explainer warns otherwise], E <= 1024 */
    int32_t S; /* tokens per rank, >= 0 */
    int32_t K; /* experts per token, 1 <= K <= E */
    int32_t H; /* hidden size; H % 8 == 0, H >= 8 */
} moonep_shape;

enum {
    MOONEP_OK = 0,
    MOONEP_ERR_INVALID_SHAPE = -1, /* a shape rule above, or R*S*K >= 2^31 */
    MOONEP_ERR_NULL_PTR = -2,      /* a required pointer is NULL */
    MOONEP_ERR_MISALIGNED = -3,    /* alignment rule above */
    MOONEP_ERR_WORKSPACE = -4,     /* workspace smaller than moonep_workspace_bytes */
    MOONEP_ERR_HIP = -5,           /* a HIP launch or copy failed */
    MOONEP_ERR_ALIAS = -6,         /* forbidden aliasing between arguments */
    MOONEP_ERR_ARG = -7            /* other invalid argument (e.g. G < 0) */
};

/* Device error word values (moonep_read_error). */
enum { MOONEP_DEV_OK = 0, MOONEP_DEV_BAD_EXPERT_ID = 1 };

/* Returns MOONEP_OK if the shape satisfies every rule above. */
int moonep_check_shape(const moonep_shape *shape);

/*
 * Bytes of scratch the caller provides to moonep_route_stats and moonep_plan
 * (the same buffer to both, in that order).  It holds per-segment expert counts
 * and the device error word.  Zero it once when it is allocated; the calls
 * keep it consistent afterwards.  One workspace serves one route_stats ->
 * plan sequence at a time: sequences that may overlap (on different streams)
 * need workspaces of their own, since they would share its counts.  Returns 0
 * for an invalid shape.
 */
size_t moonep_workspace_bytes(const moonep_shape *shape);

/*
 * The replica plan: a fixed-capacity int32 table, cap = E + R replicas (the
 * greedy never needs more than E - L).  Word offsets of its fields:
 */
typedef struct moonep_plan_layout {
    int32_t words;          /* total int32 words of the plan */
    int32_t cap;            /* replica capacity, E + R */
    int32_t header;         /* [16]: see MOONEP_PLAN_H_* */
    int32_t rep_expert;     /* [cap] expert of replica j (plan order) */
    int32_t rep_host;       /* [cap] rank that hosts replica j */
    int32_t rep_count;      /* [cap] rows replica j receives (> 0 for j < n_rep) */
    int32_t rep_spill_off;  /* [cap] offset of j's first entry among its expert's spilled ones */
    int32_t rep_row_off;    /* [cap] first row of replica j in its host's buffer */
    int32_t spill;          /* [E] entries expert e hands to replicas */
    int32_t keep;           /* [E] entries expert e keeps at home = T_e - spill_e */
    int32_t home_row_off;   /* [E] first row of expert e in its home rank's buffer */
    int32_t rep_first;      /* [E] first replica id of expert e (0 if none) */
    int32_t rep_cnt;        /* [E] number of replicas of expert e */
    int32_t exp_rep_list;   /* [E] experts with replicas, ascending (first header[N_SPILL]) */
    int32_t load;           /* [R] rows routed to rank r's home experts before balancing */
    int32_t rank_rep_first; /* [R] first replica id hosted by rank r (0 if none) */
    int32_t rank_rep_cnt;   /* [R] replicas hosted by rank r */
} moonep_plan_layout;

enum {
    MOONEP_PLAN_H_N_REP = 0,     /* replicas in this plan */
    MOONEP_PLAN_H_N_SPILL = 1,   /* experts with replicas */
    MOONEP_PLAN_H_N_DEFICIT = 2, /* ranks below C before balancing */
    MOONEP_PLAN_H_MAX_REP_RANK = 3, /* most replicas hosted by one rank */
    MOONEP_PLAN_H_TMAX = 4,      /* largest expert count */
    MOONEP_PLAN_H_C = 5,         /* rows per rank, S*K */
    MOONEP_PLAN_H_L = 6,         /* experts per rank, E/R */
    MOONEP_PLAN_H_CAP = 7        /* E + R */
};

int moonep_plan_layout_of(const moonep_shape *shape, moonep_plan_layout *layout);
size_t moonep_plan_bytes(const moonep_shape *shape); /* layout.words * 4, 0 if invalid */

/*
 * Route statistics [NCIJ "The problem MoonEP targets"; explainer "maxvio"
 * panel].  topk_idx: int32 [R*S*K], entry n = (r*S + t)*K + k, each in [0, E).
 * Writes expert_counts[e] = T_e (int32 [E]) and maxvio[0] =
 * fp32((Tmax*E)/(R*S*K) - 1) computed in IEEE double (0 when R*S*K == 0), and
 * per-segment counts into the workspace for moonep_plan.
 */
int moonep_route_stats(const moonep_shape *shape, const int32_t *topk_idx, int32_t *expert_counts,
                       float *maxvio, void *workspace, size_t workspace_bytes, void *stream);

/*
 * The replica plan and the slot maps [NCIJ "The core idea" and the
 * three-property list: exactly S*K rows per rank, tokens written straight
 * into expert-grouped rows; explainer "memory" panel: home rows precede
 * prefetch rows].  Must follow moonep_route_stats on the same topk_idx,
 * expert_counts and workspace (stream order).  Writes:
 *   plan        int32 [moonep_plan_bytes/4], layout above; unused replica
 *               entries are 0;
 *   slot_of     int32 [R*S*K]: destination row of entry n, rank*C + row.
 *               Within an expert, entries keep (src rank, token, k) order: the
 *               first keep_e rows stay home, the rest fill its replicas in plan
 *               order.  Rank d's buffer holds its home experts ascending (each
 *               keep_e rows), then the replicas it hosts in plan order;
 *   src_of_slot int32 [R*S*K]: the inverse map, entry placed at each row.
 * With a bad expert id (see the workspace error word) affected entries get
 * slot_of = -1.
 */
int moonep_plan(const moonep_shape *shape, const int32_t *topk_idx, const int32_t *expert_counts,
                void *workspace, size_t workspace_bytes, int32_t *plan, int32_t *slot_of,
                int32_t *src_of_slot, void *stream);

/*
 * The same plan and slot maps with fewer replicas [NCIJ three-property list:
 * a "near-optimal" planning kernel; the pages give no algorithm].  Identical
 * to moonep_plan (arguments, layouts, errors, and the route_stats call that
 * must precede it) except for which entries an overfull rank gives up: it
 * takes whole-expert amounts starting at its LARGEST expert count (ties to the
 * lower expert id) rather than its lowest id, which sheds the excess through
 * the fewest experts.  Each spilling expert is one entry of the spill list
 * that the two-pointer walk matches, so the plan needs fewer replicas: 32
 * instead of 61 on a DeepSeek-V3-like routing (R = 32, E = 256, Zipf 1.2),
 * each replica being one expert's weights to prefetch and one gradient to
 * reduce.  Entry order is as in moonep_plan: an expert's first keep_e
 * entries stay home, the rest fill its replicas in plan order.
 */
int moonep_plan_largest_first(const moonep_shape *shape, const int32_t *topk_idx,
                              const int32_t *expert_counts, void *workspace,
                              size_t workspace_bytes, int32_t *plan, int32_t *slot_of,
                              int32_t *src_of_slot, void *stream);

/*
 * For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the work of
 * moonep_route_stats followed by moonep_plan, with the workspace replaced by a
 * scratch array inside the library, MOONEP_NOALLOC_SCRATCH_BYTES per device
 * (enough for every valid shape), held until the process ends.  Allocates
 * nothing.  Writes expert_counts, maxvio, plan, slot_of and src_of_slot
 * exactly as those two calls do.  Every call on one device shares that
 * device's scratch and leaves its contents behind (nothing in it must start
 * at zero between calls), so calls that overlap on one device -- other
 * streams, other host threads -- race and must be ordered by the caller.  An
 * expert id outside [0, E) gives its entries slot_of = -1 as in moonep_plan;
 * the scratch's error word cannot be read with moonep_read_error.  Returns
 * MOONEP_ERR_WORKSPACE if a shape needed more scratch than the array holds,
 * MOONEP_ERR_HIP if the scratch's device address cannot be obtained.
 */
enum { MOONEP_NOALLOC_SCRATCH_BYTES = 256 + 4 * 1024 * 2048 };
int moonep_plan_noalloc(const moonep_shape *shape, const int32_t *topk_idx, int32_t *expert_counts,
                        float *maxvio, int32_t *plan, int32_t *slot_of, int32_t *src_of_slot,
                        void *stream);

/*
 * Dispatch, the fused permute [NCIJ three-property list, zero copy; AIPDB].
 * x: bf16 [R*S, H] token rows.  buf: bf16 [R*S*K, H], the R static [S*K, H]
 * per-rank buffers [NCIJ explainer "invariant" panel] back to back.
 * buf[slot_of[n]] = x[n div K], a bit copy.  Rows whose slot_of is outside
 * [0, R*S*K) are skipped.  buf must not overlap x.
 */
int moonep_dispatch(const moonep_shape *shape, const uint16_t *x, const int32_t *slot_of,
                    uint16_t *buf, void *stream);

/*
 * Combine, the fused weighted unpermute [NCIJ three-property list and
 * explainer "pillars" panel].  expert_out: bf16 [R*S*K, H] rows in buffer
 * order (may be the dispatch buffer itself); gates: fp32 [R*S*K].
 * y[t] = bf16(sum over k ascending of gates[t*K+k] * expert_out[slot_of[t*K+k]]).
 * Each fp32 x bf16 product is exact in fp64; the products are summed in fp64
 * in ascending k from +0 and the sum is rounded once to bf16 (to nearest
 * even), for terms of any sign.  Out-of-range slots contribute nothing.
 * y: bf16 [R*S, H], must not overlap expert_out.
 */
int moonep_combine(const moonep_shape *shape, const uint16_t *expert_out, const float *gates,
                   const int32_t *slot_of, uint16_t *y, void *stream);

/*
 * Combine backward (the training backward of combine; [NCIJ "The core idea"]).
 * dy: bf16 [R*S, H].  Writes
 *   d_out[slot_of[n]] = bf16(gates[n] * dy[n div K])  (one correct rounding of
 *                       the exact product), bf16 [R*S*K, H];
 *   d_gates[n] = sum_h dy[n div K, h] * expert_out[slot_of[n], h]  (fp32
 *                       accumulation), fp32 [R*S*K].
 * d_out must not overlap dy or expert_out.
 */
int moonep_combine_bwd(const moonep_shape *shape, const uint16_t *dy, const uint16_t *expert_out,
                       const float *gates, const int32_t *slot_of, uint16_t *d_out,
                       float *d_gates, void *stream);

/*
 * Dispatch backward (the training backward of dispatch; [NCIJ "The core
 * idea"]).  d_buf: bf16 [R*S*K, H], the gradient of the dispatch buffer rows.
 * dx[t] = bf16(sum over k ascending of d_buf[slot_of[t*K+k]]), the sum taken in
 * fp64 and rounded once (to nearest even).  dx: bf16 [R*S, H], must not overlap
 * d_buf.  Out-of-range slots contribute nothing.
 */
int moonep_dispatch_bwd(const moonep_shape *shape, const uint16_t *d_buf, const int32_t *slot_of,
                        uint16_t *dx, void *stream);

/*
 * Replica-gradient reduction [NCIJ "The core idea": replica gradients return
 * to their home experts; explainer "memory" panel: they sit in an fp32 reduce
 * buffer that is pulled home and then zeroed for the next microbatch].
 * home_grads: fp32 [E, G]; replica_grads: fp32 [E + R, G], row j = replica j of
 * `plan` (plan order).  For every expert e with replicas:
 *   home[e] = fp32(home[e] + rep[j1] + rep[j2] + ...)  (fp64 sum, plan order),
 * then rep[j] = +0 for every j < n_rep.  Other rows are not touched.  G >= 0;
 * the two arrays must not overlap.
 */
int moonep_replica_grad_reduce(const moonep_shape *shape, const int32_t *plan, int64_t G,
                               float *home_grads, float *replica_grads, void *stream);

/*
 * Replica weight slots [NCIJ "The core idea": redundant experts are
 * prefetched before expert compute; explainer "memory" panel: each rank owns B
 * prefetch slots, the rows that follow the expert rows of its weight tensor;
 * training needs B = E/R, inference may use fewer (3-4 suggested), and a rank
 * that hosts more than B replicas reads the extra ones from their home rank].
 * Writes wslot: int32 [E + R], for replica j < n_rep of `plan` hosted on rank
 * d as its b-th in plan order: wslot[j] = d*B + b when b < B, else -1
 * (overflow: that replica's weights are read at the home expert's row).
 * Entries j >= n_rep are -1.  The plan is not changed.  B >= 0 and
 * R*B < 2^31, else MOONEP_ERR_ARG.
 */
int moonep_weight_slots(const moonep_shape *shape, const int32_t *plan, int32_t B, int32_t *wslot,
                        void *stream);

/*
 * Replica weight prefetch [same passages].  w_home: [E, wbytes] bytes, row e =
 * every weight of expert e (e.g. its gate, up and down projections, in any
 * layout the caller chooses); pool: [R*B, wbytes] bytes, row d*B + b = slot b
 * of rank d.  For every j < n_rep with 0 <= wslot[j] < R*B:
 *   pool[wslot[j]] = w_home[rep_expert[j]]  (a bit copy).
 * Other pool rows are not touched.  wbytes % 16 == 0 (MOONEP_ERR_ARG);
 * w_home and pool 16-byte aligned; they must not overlap.  wslot normally
 * comes from moonep_weight_slots with the same B; slots that two replicas
 * share would race.
 */
int moonep_prefetch_weights(const moonep_shape *shape, const int32_t *plan, const int32_t *wslot,
                            int32_t B, int64_t wbytes, const void *w_home, void *pool,
                            void *stream);

/*
 * Expert compute over the expert-grouped buffer: one projection, a grouped
 * GEMM [NCIJ three-property list: buffer views go straight to the
 * computation, each rank's rows grouped by expert; explainer "memory" panel:
 * replicas read their prefetch slot, or the home expert past B slots].
 * x: bf16 [R*S*K, in_dim], the buffer rows (e.g. the dispatch buffer);
 * y: bf16 [R*S*K, out_dim].  For buffer row r of rank d = r div (S*K):
 *   y[r, n] = bf16( sum_k x[r, k] * W[n, k] )  (fp32 accumulation on the
 *             matrix cores, one rounding to nearest even),
 * where W is the [out_dim, in_dim] row-major matrix starting at element
 * w_offset of the weight row of r's segment: w_home + e*w_stride for a home
 * expert e; for replica j, pool + wslot[j]*w_stride when 0 <= wslot[j] < R*B,
 * else w_home + rep_expert[j]*w_stride.  w_home holds E weight rows, pool R*B
 * (the layouts of moonep_prefetch_weights, counted in bf16 elements here).
 * Limits (else MOONEP_ERR_ARG): in_dim % 64 == 0, in_dim <= 2^22, out_dim % 128 == 0,
 * w_stride and w_offset multiples of 8, w_offset + out_dim*in_dim <= w_stride.
 * x, y, w_home, pool 16-byte aligned; y must not overlap x, w_home or pool.
 */
int moonep_expert_gemm(const moonep_shape *shape, const int32_t *plan, const int32_t *wslot,
                       int32_t B, int32_t in_dim, int32_t out_dim, const uint16_t *x,
                       const uint16_t *w_home, const uint16_t *pool, int64_t w_stride,
                       int64_t w_offset, uint16_t *y, void *stream);

/*
 * Reads the sticky device error word of a workspace into *host_code, then
 * clears it.  Synchronises `stream`.  The only call that waits for the device.
 */
int moonep_read_error(void *workspace, size_t workspace_bytes, int32_t *host_code, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* MOONEP_H */
