/*
 * oracle.c -- TEST INFRASTRUCTURE ONLY.  A plain, slow, single-threaded CPU
 * statement of what the balanced expert-parallel hot path computes.  Only the
 * test suite, the smoke check and the benchmark's CPU-baseline leg may load
 * it.  It shares no code with the GPU library.
 *
 * Pages cited (the text of each is the authority on what is computed):
 *   [NCIJ]  "Moonshot AI Open-Sources MoonEP: A Perfectly Balanced Expert
 *           Parallelism Library for MoE Training" (ncijnetwork.com):
 *           section "The problem MoonEP targets", section "The core idea:
 *           dynamic redundant experts", the three-property list, and the
 *           interactive explainer with its "invariant", "memory", "maxvio"
 *           and "pillars" panels.
 *   [AIPDB] "Moonshot AI open-sources MoonEP for distributed MoE
 *           communication" (aipricedb.com), the README excerpt on zero copy.
 *   [AGIH]  "Moonshot Open-Sources MoonEP for MoE Distributed Communication
 *           and Load Balancing" (agihunt.info), "Core Technical Approach".
 *
 * Notation: R ranks, E experts, L = E/R experts per rank, home(e) = e div L,
 * S tokens per rank, K experts per token, H hidden size, C = S*K rows per
 * rank, N = R*S tokens, NK = N*K routed entries, entry n = token*K + k with
 * token = src_rank*S + t.  T_e = number of entries routed to expert e.
 *
 * The pages give no planner algorithm beyond: redundant experts are planned
 * from the current router output so that every rank receives exactly S*K
 * entries.  The plan below is the plainest greedy that meets it: ranks whose
 * load exceeds C give up whole-expert amounts starting from their lowest
 * expert id until the excess is gone; the given-up amounts, in expert order,
 * are matched two-pointer against the deficits of the ranks below C, in rank
 * order; every match is one replica.
 *
 * Floating point: fp64 wherever the pages do not fix a precision; bf16 and
 * fp32 only where the pages fix the storage type (bf16 dispatch buffer, fp32
 * reduce buffer).  Every rounding to bf16 is one correct rounding
 * (nearest, ties to even) of the fp64 value.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORC_OK 0
#define ORC_ERR_SHAPE (-1)
#define ORC_ERR_EXPERT_ID (-2)
#define ORC_ERR_INTERNAL (-3)

/* ------------------------------------------------------------------------ */
/* bf16 helpers (independent of the GPU library's own)                        */
/* ------------------------------------------------------------------------ */

double orc_bf16_to_double(uint16_t b)
{
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, 4);
    return (double)f;
}

/*
 * Correct rounding of a double to bf16 (8 significant bits, exponent range of
 * fp32, subnormal quantum 2^-133), to nearest with ties to even: scale so the
 * bf16 quantum is 1, round to an integer with rint (the default rounding mode
 * is nearest-even), scale back.  Powers of two scale exactly.
 */
uint16_t orc_bf16_from_double(double d)
{
    if (isnan(d))
        return signbit(d) ? 0xFFC0u : 0x7FC0u;
    if (d == 0.0)
        return signbit(d) ? 0x8000u : 0x0000u;
    int ex;
    (void)frexp(d, &ex);           /* d = m * 2^ex, 0.5 <= |m| < 1 */
    int qexp = (ex < -125 ? -125 : ex) - 8; /* bf16 quantum 2^qexp */
    double r = rint(ldexp(d, -qexp));
    double v = ldexp(r, qexp);
    uint16_t sign = signbit(d) ? 0x8000u : 0u;
    if (fabs(v) >= 0x1p128)
        return (uint16_t)(sign | 0x7F80u);
    float f = (float)v;            /* exact: v has <= 8 significant bits */
    uint32_t u;
    memcpy(&u, &f, 4);
    return (uint16_t)(u >> 16);
}

/* ------------------------------------------------------------------------ */
/* Shape                                                                      */
/* ------------------------------------------------------------------------ */

static int shape_ok(int32_t R, int32_t E, int32_t S, int32_t K)
{
    /* [NCIJ] explainer: the expert count must divide evenly over the ranks. */
    if (R < 1 || E < 1 || S < 0 || K < 1 || K > E || E % R != 0)
        return 0;
    if ((int64_t)R * S * K >= ((int64_t)1 << 31))
        return 0;
    return 1;
}

/* ------------------------------------------------------------------------ */
/* Step 1: route statistics.                                                  */
/* [NCIJ] "The problem MoonEP targets": maxvio = max_e (T_e / Tbar) - 1, where */
/* Tbar is the count of a perfectly balanced routing; the explainer's maxvio  */
/* panel fixes Tbar = S*K*R / E.                                              */
/* ------------------------------------------------------------------------ */

int orc_route_stats(int32_t R, int32_t E, int32_t S, int32_t K, const int32_t *topk,
                    int32_t *T, float *maxvio)
{
    if (!shape_ok(R, E, S, K))
        return ORC_ERR_SHAPE;
    const int64_t NK = (int64_t)R * S * K;
    for (int32_t e = 0; e < E; ++e)
        T[e] = 0;
    for (int64_t n = 0; n < NK; ++n) {
        const int32_t e = topk[n];
        if (e < 0 || e >= E)
            return ORC_ERR_EXPERT_ID;
        T[e] += 1;
    }
    int32_t tmax = 0;
    for (int32_t e = 0; e < E; ++e)
        if (T[e] > tmax)
            tmax = T[e];
    if (NK == 0) {
        *maxvio = 0.0f; /* no tokens: trivially balanced */
    } else {
        /* Tmax / (NK / E) - 1, with one division: (Tmax * E) / NK - 1. */
        const double ratio = (double)((int64_t)tmax * E) / (double)NK;
        *maxvio = (float)(ratio - 1.0);
    }
    return ORC_OK;
}

/* ------------------------------------------------------------------------ */
/* Step 2: the replica plan.                                                  */
/* [NCIJ] "The core idea": every rank receives exactly S*K entries, by        */
/* planning a few redundant experts from the current router output.           */
/* [NCIJ] explainer "memory" panel: prefetch rows follow the home rows, so a  */
/* rank's buffer holds its home experts first and its replicas after.         */
/* ------------------------------------------------------------------------ */

typedef struct {
    int32_t n_rep;        /* replicas emitted */
    int32_t n_spill;      /* experts that give up tokens */
    int32_t n_deficit;    /* ranks below C */
    int32_t max_rep_rank; /* most replicas hosted by one rank */
    /* per replica, in plan order (capacity E + R) */
    int32_t *rep_expert, *rep_host, *rep_count, *rep_spill_off, *rep_row_off;
    /* per expert */
    int32_t *spill, *keep, *home_row_off, *rep_first, *rep_cnt;
    /* per rank */
    int32_t *load, *rank_rep_first, *rank_rep_cnt;
} orc_plan_t;

/*
 * policy 0 (the plain reading of "spill in expert order"): an overfull rank
 * gives up whole-expert amounts starting at its lowest expert id.
 * policy 1 (the "near-optimal" planner of the three-property list, in the
 * plainest form that needs fewer replicas): it gives them up starting at its
 * largest expert count, ties to the lower id.  Taking the largest counts
 * first sheds the excess through the fewest experts, and every spilling
 * expert adds one entry to the spill list that the two-pointer walk matches.
 * Everything after the spill amounts is the same for both.
 */
int orc_plan_policy(int32_t R, int32_t E, int32_t S, int32_t K, const int32_t *T, int32_t policy,
                    orc_plan_t *p)
{
    if (policy != 0 && policy != 1)
        return ORC_ERR_SHAPE;
    if (!shape_ok(R, E, S, K))
        return ORC_ERR_SHAPE;
    const int32_t L = E / R;
    const int32_t C = S * K;
    const int32_t cap = E + R;

    for (int32_t j = 0; j < cap; ++j) {
        p->rep_expert[j] = 0;
        p->rep_host[j] = 0;
        p->rep_count[j] = 0;
        p->rep_spill_off[j] = 0;
        p->rep_row_off[j] = 0;
    }

    /* Rank loads before balancing. */
    for (int32_t r = 0; r < R; ++r) {
        int64_t s = 0;
        for (int32_t e = r * L; e < (r + 1) * L; ++e)
            s += T[e];
        p->load[r] = (int32_t)s;
    }

    /* Overfull ranks give up whole-expert amounts, lowest expert id first
       (policy 0) or largest count first (policy 1). */
    for (int32_t r = 0; r < R; ++r) {
        int32_t excess = p->load[r] > C ? p->load[r] - C : 0;
        if (policy == 0) {
            for (int32_t e = r * L; e < (r + 1) * L; ++e) {
                const int32_t give = T[e] < excess ? T[e] : excess;
                p->spill[e] = give;
                excess -= give;
            }
        } else {
            for (int32_t e = r * L; e < (r + 1) * L; ++e)
                p->spill[e] = 0;
            while (excess > 0) {
                /* the largest count not yet taken; the ascending scan keeps
                   the lowest id among equal counts */
                int32_t best = -1;
                for (int32_t e = r * L; e < (r + 1) * L; ++e)
                    if (p->spill[e] == 0 && T[e] > 0 && (best < 0 || T[e] > T[best]))
                        best = e;
                if (best < 0)
                    return ORC_ERR_INTERNAL;
                const int32_t give = T[best] < excess ? T[best] : excess;
                p->spill[best] = give;
                excess -= give;
            }
        }
    }
    for (int32_t e = 0; e < E; ++e)
        p->keep[e] = T[e] - p->spill[e];

    /* Spill list (ascending expert) and deficit list (ascending rank). */
    int32_t *sp_e = (int32_t *)malloc(sizeof(int32_t) * (size_t)E);
    int32_t *sp_amt = (int32_t *)malloc(sizeof(int32_t) * (size_t)E);
    int32_t *df_r = (int32_t *)malloc(sizeof(int32_t) * (size_t)R);
    int32_t *df_amt = (int32_t *)malloc(sizeof(int32_t) * (size_t)R);
    int32_t ns = 0, nd = 0;
    for (int32_t e = 0; e < E; ++e)
        if (p->spill[e] > 0) {
            sp_e[ns] = e;
            sp_amt[ns] = p->spill[e];
            ++ns;
        }
    for (int32_t r = 0; r < R; ++r)
        if (p->load[r] < C) {
            df_r[nd] = r;
            df_amt[nd] = C - p->load[r];
            ++nd;
        }
    p->n_spill = ns;
    p->n_deficit = nd;

    /* Two-pointer match: each match of a spill amount with a deficit is one
       replica of that expert hosted on that rank. */
    int32_t i = 0, j = 0, nrep = 0;
    int32_t rem_s = ns ? sp_amt[0] : 0;
    int32_t rem_d = nd ? df_amt[0] : 0;
    while (i < ns && j < nd) {
        const int32_t m = rem_s < rem_d ? rem_s : rem_d;
        p->rep_expert[nrep] = sp_e[i];
        p->rep_host[nrep] = df_r[j];
        p->rep_count[nrep] = m;
        p->rep_spill_off[nrep] = sp_amt[i] - rem_s;
        ++nrep;
        rem_s -= m;
        rem_d -= m;
        if (rem_s == 0) {
            ++i;
            rem_s = i < ns ? sp_amt[i] : 0;
        }
        if (rem_d == 0) {
            ++j;
            rem_d = j < nd ? df_amt[j] : 0;
        }
    }
    free(sp_e);
    free(sp_amt);
    free(df_r);
    free(df_amt);
    if (i != ns || j != nd)
        return ORC_ERR_INTERNAL; /* totals of spill and deficit must agree */
    p->n_rep = nrep;

    /* Buffer layout of each rank: home experts ascending (zero-length ones
       included), then the replicas it hosts in plan order. */
    for (int32_t r = 0; r < R; ++r) {
        int32_t row = 0;
        for (int32_t e = r * L; e < (r + 1) * L; ++e) {
            p->home_row_off[e] = row;
            row += p->keep[e];
        }
        p->rank_rep_first[r] = 0;
        p->rank_rep_cnt[r] = 0;
        for (int32_t q = 0; q < nrep; ++q)
            if (p->rep_host[q] == r) {
                if (p->rank_rep_cnt[r] == 0)
                    p->rank_rep_first[r] = q;
                p->rank_rep_cnt[r] += 1;
                p->rep_row_off[q] = row;
                row += p->rep_count[q];
            }
        if (row != C)
            return ORC_ERR_INTERNAL; /* the S*K invariant */
    }
    p->max_rep_rank = 0;
    for (int32_t r = 0; r < R; ++r)
        if (p->rank_rep_cnt[r] > p->max_rep_rank)
            p->max_rep_rank = p->rank_rep_cnt[r];

    for (int32_t e = 0; e < E; ++e) {
        p->rep_first[e] = 0;
        p->rep_cnt[e] = 0;
    }
    for (int32_t q = 0; q < nrep; ++q) {
        const int32_t e = p->rep_expert[q];
        if (p->rep_cnt[e] == 0)
            p->rep_first[e] = q;
        p->rep_cnt[e] += 1;
    }
    return ORC_OK;
}

int orc_plan(int32_t R, int32_t E, int32_t S, int32_t K, const int32_t *T, orc_plan_t *p)
{
    return orc_plan_policy(R, E, S, K, T, 0, p);
}

/* ------------------------------------------------------------------------ */
/* Step 3: slot assignment.  [NCIJ] three-property list, zero copy: each      */
/* token is written straight into its expert-grouped position.  Within an    */
/* expert, entries keep their (src rank, token, k) order: the first keep_e of */
/* them stay home, the rest fill that expert's replicas in plan order.        */
/* slot = dst_rank * C + dst_row.                                             */
/* ------------------------------------------------------------------------ */

int orc_slots(int32_t R, int32_t E, int32_t S, int32_t K, const int32_t *topk,
              const orc_plan_t *p, int32_t *slot_of, int32_t *src_of_slot)
{
    if (!shape_ok(R, E, S, K))
        return ORC_ERR_SHAPE;
    const int32_t L = E / R;
    const int32_t C = S * K;
    const int64_t NK = (int64_t)R * S * K;
    int32_t *seen = (int32_t *)calloc((size_t)E, sizeof(int32_t));
    for (int64_t n = 0; n < NK; ++n) {
        const int32_t e = topk[n];
        if (e < 0 || e >= E) {
            free(seen);
            return ORC_ERR_EXPERT_ID;
        }
        const int32_t pos = seen[e]++; /* entries of e before n */
        int32_t rank, row;
        if (pos < p->keep[e]) {
            rank = e / L;
            row = p->home_row_off[e] + pos;
        } else {
            const int32_t q = pos - p->keep[e];
            int32_t found = -1;
            for (int32_t jj = 0; jj < p->n_rep; ++jj)
                if (p->rep_expert[jj] == e && p->rep_spill_off[jj] <= q &&
                    q < p->rep_spill_off[jj] + p->rep_count[jj])
                    found = jj;
            if (found < 0) {
                free(seen);
                return ORC_ERR_INTERNAL;
            }
            rank = p->rep_host[found];
            row = p->rep_row_off[found] + (q - p->rep_spill_off[found]);
        }
        const int32_t slot = rank * C + row;
        slot_of[n] = slot;
        src_of_slot[slot] = (int32_t)n;
    }
    free(seen);
    return ORC_OK;
}

/* ------------------------------------------------------------------------ */
/* Step 4: dispatch.  Row slot_of[n] of the static [R, S*K, H] bf16 buffer    */
/* receives token n div K's row ([NCIJ] explainer "invariant" panel fixes the */
/* per-rank buffer at S*K*H bf16).  A bit copy.                               */
/* ------------------------------------------------------------------------ */

void orc_dispatch(int64_t NK, int32_t K, int32_t H, const uint16_t *x, const int32_t *slot_of,
                  uint16_t *buf)
{
    for (int64_t n = 0; n < NK; ++n) {
        const int64_t tok = n / K;
        for (int32_t h = 0; h < H; ++h)
            buf[(int64_t)slot_of[n] * H + h] = x[tok * H + h];
    }
}

/* Rows of the dispatch buffer, one by one: buf[row] = x[src_of_slot[row] div K]. */
void orc_dispatch_rows(int32_t K, int32_t H, const uint16_t *x, const int32_t *src_of_slot,
                       int64_t nrows, const int64_t *rows, uint16_t *out)
{
    for (int64_t i = 0; i < nrows; ++i) {
        const int64_t tok = src_of_slot[rows[i]] / K;
        for (int32_t h = 0; h < H; ++h)
            out[i * H + h] = x[tok * H + h];
    }
}

/* ------------------------------------------------------------------------ */
/* Stand-in expert (harness, not part of the path): row r of expert e becomes */
/* bf16(fp32(buf[r]) * scale[e]), one fp32 multiply then one rounding.        */
/* The expert of a row is the expert of the entry placed there.               */
/* ------------------------------------------------------------------------ */

void orc_expert(int64_t rows, int32_t H, const uint16_t *buf, const int32_t *row_expert,
                const float *scale, uint16_t *out)
{
    for (int64_t r = 0; r < rows; ++r) {
        const float s = scale[row_expert[r]];
        for (int32_t h = 0; h < H; ++h) {
            const float v = (float)orc_bf16_to_double(buf[r * H + h]) * s;
            out[r * H + h] = orc_bf16_from_double((double)v);
        }
    }
}

/* ------------------------------------------------------------------------ */
/* Step 5: combine.  [NCIJ] three-property list (fused unpermute) and the     */
/* "pillars" panel: the K expert outputs of a token are gathered back from    */
/* their expert-grouped rows.  y[tok] = sum_k gate[n] * out[slot_of[n]],      */
/* summed in fp64 in ascending k, rounded once to bf16.                       */
/* ------------------------------------------------------------------------ */

void orc_combine(int64_t N, int32_t K, int32_t H, const uint16_t *out, const float *gates,
                 const int32_t *slot_of, uint16_t *y)
{
    for (int64_t t = 0; t < N; ++t)
        for (int32_t h = 0; h < H; ++h) {
            double acc = 0.0;
            for (int32_t k = 0; k < K; ++k) {
                const int64_t n = t * K + k;
                acc += (double)gates[n] * orc_bf16_to_double(out[(int64_t)slot_of[n] * H + h]);
            }
            y[t * H + h] = orc_bf16_from_double(acc);
        }
}

/*
 * The forward of chosen tokens, one by one, without materialising the
 * buffers: for each k, the row at slot_of[n] holds x[src_of_slot[slot] div K];
 * the stand-in expert of the entry's expert scales it; combine sums.  Used at
 * sizes where whole buffers do not fit the host.
 */
void orc_forward_tokens(int32_t K, int32_t H, const uint16_t *x, const int32_t *topk,
                        const float *gates, const int32_t *slot_of, const int32_t *src_of_slot,
                        const float *scale, int64_t ntok, const int64_t *toks, uint16_t *y)
{
    double *acc = (double *)malloc(sizeof(double) * (size_t)H);
    for (int64_t i = 0; i < ntok; ++i) {
        const int64_t t = toks[i];
        for (int32_t h = 0; h < H; ++h)
            acc[h] = 0.0;
        for (int32_t k = 0; k < K; ++k) {
            const int64_t n = t * K + k;
            const int64_t src = src_of_slot[slot_of[n]];
            const float s = scale[topk[src]];
            const int64_t st = src / K;
            for (int32_t h = 0; h < H; ++h) {
                const float v = (float)orc_bf16_to_double(x[st * H + h]) * s;
                const double o = orc_bf16_to_double(orc_bf16_from_double((double)v));
                acc[h] += (double)gates[n] * o;
            }
        }
        for (int32_t h = 0; h < H; ++h)
            y[i * H + h] = orc_bf16_from_double(acc[h]);
    }
    free(acc);
}

/* ------------------------------------------------------------------------ */
/* Step 6: combine backward (training use: [NCIJ] "The core idea" and the     */
/* "memory" panel's backward pass).  y = sum_k g_k out_k, so                  */
/*   d_out[slot_of[n]] = g_n * dy[tok]        (rounded once to bf16)          */
/*   d_gate[n]        = sum_h dy[tok,h] * out[slot_of[n],h]  (fp64, h asc.)   */
/* ------------------------------------------------------------------------ */

void orc_combine_bwd(int64_t N, int32_t K, int32_t H, const uint16_t *dy, const uint16_t *out,
                     const float *gates, const int32_t *slot_of, uint16_t *d_out,
                     float *d_gates)
{
    for (int64_t t = 0; t < N; ++t)
        for (int32_t k = 0; k < K; ++k) {
            const int64_t n = t * K + k;
            const int64_t row = slot_of[n];
            double dot = 0.0;
            for (int32_t h = 0; h < H; ++h) {
                const double g = orc_bf16_to_double(dy[t * H + h]);
                d_out[row * H + h] = orc_bf16_from_double((double)gates[n] * g);
                dot += g * orc_bf16_to_double(out[row * H + h]);
            }
            d_gates[n] = (float)dot;
        }
}

/* ------------------------------------------------------------------------ */
/* Step 6b: dispatch backward (training use, [NCIJ] "The core idea").        */
/* buf[slot_of[n]] = x[n div K], so the gradient of x gathers the K rows of   */
/* the buffer gradient:  dx[tok] = sum_k d_buf[slot_of[tok*K + k]],           */
/* summed in fp64 in ascending k, rounded once to bf16.                       */
/* ------------------------------------------------------------------------ */

void orc_dispatch_bwd(int64_t N, int32_t K, int32_t H, const uint16_t *d_buf,
                      const int32_t *slot_of, uint16_t *dx)
{
    for (int64_t t = 0; t < N; ++t)
        for (int32_t h = 0; h < H; ++h) {
            double acc = 0.0;
            for (int32_t k = 0; k < K; ++k)
                acc += orc_bf16_to_double(d_buf[(int64_t)slot_of[t * K + k] * H + h]);
            dx[t * H + h] = orc_bf16_from_double(acc);
        }
}

/* ------------------------------------------------------------------------ */
/* Step 7: replica-gradient reduction.  [NCIJ] "The core idea": gradients of  */
/* the duplicated experts go back to their home ranks; the "memory" panel:    */
/* they sit in an fp32 reduce buffer, which the reduction pulls home and then */
/* zeroes for the next microbatch.                                            */
/*   home[e] = fp32( home[e] + sum over replicas j of e, plan order, of rep[j]) */
/* summed in fp64 in that order; then rep[j] = +0 for every j < n_rep.        */
/* home rows of experts without replicas are untouched.                       */
/* ------------------------------------------------------------------------ */

void orc_replica_grad_reduce(int32_t E, const orc_plan_t *p, int64_t G, float *home, float *rep)
{
    for (int32_t e = 0; e < E; ++e) {
        if (p->rep_cnt[e] == 0)
            continue;
        for (int64_t i = 0; i < G; ++i) {
            double acc = (double)home[(int64_t)e * G + i];
            for (int32_t q = p->rep_first[e]; q < p->rep_first[e] + p->rep_cnt[e]; ++q)
                acc += (double)rep[(int64_t)q * G + i];
            home[(int64_t)e * G + i] = (float)acc;
        }
    }
    for (int32_t q = 0; q < p->n_rep; ++q)
        for (int64_t i = 0; i < G; ++i)
            rep[(int64_t)q * G + i] = 0.0f;
}

/* The same reduction at chosen element positions only (all experts). */
void orc_replica_grad_reduce_at(int32_t E, const orc_plan_t *p, int64_t G, const float *home_at,
                                const float *rep_at, int64_t nidx, float *home_out)
{
    /* home_at: [E, nidx], rep_at: [n_rep, nidx] values at the chosen positions. */
    for (int32_t e = 0; e < E; ++e)
        for (int64_t i = 0; i < nidx; ++i) {
            double acc = (double)home_at[(int64_t)e * nidx + i];
            for (int32_t q = p->rep_first[e]; q < p->rep_first[e] + p->rep_cnt[e]; ++q)
                acc += (double)rep_at[(int64_t)q * nidx + i];
            home_out[(int64_t)e * nidx + i] = p->rep_cnt[e] ? (float)acc : home_at[(int64_t)e * nidx + i];
        }
    (void)G;
}

/* ------------------------------------------------------------------------ */
/* Step 8: replica weight slots and prefetch.  [NCIJ] explainer, "memory"    */
/* panel: every rank owns B prefetch slots, rows [E, E+B) of one contiguous  */
/* weight tensor that follow the expert rows; training needs B = E/R,        */
/* inference may use fewer (3-4); a rank needing more distinct remote        */
/* experts than B reads the extra ones from their home rank ("overflow").    */
/* "The core idea": the redundant experts are prefetched before expert       */
/* compute.                                                                  */
/*                                                                          */
/* Slots: rank d's replicas, in plan order, take d's slots 0, 1, ..., B-1;   */
/* wslot[j] = d*B + b for the b-th replica hosted on d when b < B, else -1   */
/* (overflow).  Entries j >= n_rep are -1.  The plan itself is unchanged.    */
/* ------------------------------------------------------------------------ */

void orc_weight_slots(int32_t R, int32_t E, int32_t B, const orc_plan_t *p, int32_t *wslot)
{
    for (int32_t j = 0; j < E + R; ++j)
        wslot[j] = -1;
    for (int32_t d = 0; d < R; ++d) {
        int32_t b = 0;  /* replicas of rank d seen so far, in plan order */
        for (int32_t j = 0; j < p->n_rep; ++j) {
            if (p->rep_host[j] != d)
                continue;
            if (b < B)
                wslot[j] = d * B + b;
            ++b;
        }
    }
}

/* Prefetch: the weight bytes of a replica's expert go to its slot.
 *   pool[wslot[j]] = w_home[rep_expert[j]]   (wbytes bytes, a bit copy)
 * for every j < n_rep with wslot[j] >= 0; other pool rows are untouched. */
void orc_prefetch_weights(int64_t wbytes, const orc_plan_t *p, const int32_t *wslot,
                          const uint8_t *w_home, uint8_t *pool)
{
    for (int32_t j = 0; j < p->n_rep; ++j)
        if (wslot[j] >= 0)
            memcpy(pool + (int64_t)wslot[j] * wbytes, w_home + (int64_t)p->rep_expert[j] * wbytes,
                   (size_t)wbytes);
}

/* ------------------------------------------------------------------------ */
/* Step 9: expert compute over the expert-grouped buffer.  [NCIJ] three-     */
/* property list: views of the buffer go straight to the computation, which  */
/* reads each rank's rows grouped by expert; "memory" panel: a replica's     */
/* weights are in its prefetch slot, or, past B slots, at the home expert.   */
/* One projection (a grouped GEMM):                                          */
/*   y[r, n] = bf16( sum_k x[r, k] * W(r)[n, k] )   (fp64 sum, k ascending)  */
/* for buffer row r = d*C + local, where W(r) is the [out_dim, in_dim]       */
/* matrix at element w_offset of the weight row of r's segment:              */
/*   home expert e of rank d holding local  -> w_home row e;                 */
/*   replica j hosted on d holding local    -> pool row wslot[j] if >= 0,    */
/*                                             else w_home row rep_expert[j].*/
/* Weight rows are w_stride bf16 elements apart.  Only the listed rows are   */
/* computed (the full product is too slow for a plain CPU loop at scale);    */
/* with x_compact, x holds just those rows, in the order listed.             */
/* ------------------------------------------------------------------------ */

void orc_expert_gemm_rows(int32_t R, int32_t E, int32_t S, int32_t K, const orc_plan_t *p,
                          const int32_t *wslot, int32_t in_dim, int32_t out_dim, const uint16_t *x,
                          const uint16_t *w_home, const uint16_t *pool, int64_t w_stride,
                          int64_t w_offset, int64_t nrows, const int64_t *rows, int32_t x_compact,
                          uint16_t *y)
{
    const int32_t L = E / R;
    const int64_t C = (int64_t)S * K;
    for (int64_t i = 0; i < nrows; ++i) {
        const int64_t r = rows[i];
        const int32_t d = (int32_t)(r / C);
        const int64_t local = r - (int64_t)d * C;
        const uint16_t *w = NULL;
        for (int32_t e = d * L; e < (d + 1) * L && !w; ++e)
            if (local >= p->home_row_off[e] && local < p->home_row_off[e] + p->keep[e])
                w = w_home + (int64_t)e * w_stride;
        for (int32_t j = 0; j < p->n_rep && !w; ++j)
            if (p->rep_host[j] == d && local >= p->rep_row_off[j] &&
                local < p->rep_row_off[j] + p->rep_count[j])
                w = wslot[j] >= 0 ? pool + (int64_t)wslot[j] * w_stride
                                  : w_home + (int64_t)p->rep_expert[j] * w_stride;
        const uint16_t *xr = x + (x_compact ? i : r) * in_dim;
        for (int32_t n = 0; n < out_dim; ++n) {
            double acc = 0.0;
            if (w) {
                const uint16_t *wn = w + w_offset + (int64_t)n * in_dim;
                for (int32_t k = 0; k < in_dim; ++k)
                    acc += orc_bf16_to_double(xr[k]) * orc_bf16_to_double(wn[k]);
            }
            y[i * out_dim + n] = orc_bf16_from_double(acc);
        }
    }
}
