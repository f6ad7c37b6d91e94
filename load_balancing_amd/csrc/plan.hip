// plan.hip -- the replica plan and the slot maps, in one launch.
//
// What is planned: the MoonEP article (ncijnetwork.com), section "The core
// idea: dynamic redundant experts", requires that every rank receives exactly
// S*K routed entries, by adding a few redundant experts planned from the
// current router output; its three-property list asks that tokens land
// directly in their expert-grouped rows; the explainer's "memory" panel puts
// prefetch (replica) rows after the home rows.  The pages give no planner, so
// this one is the plainest greedy that meets the invariant: ranks above C
// give up whole-expert amounts starting at their lowest expert id (or, in the
// second policy, at their largest expert count, which sheds the excess
// through the fewest experts and so needs fewer replicas); these amounts (in
// expert order) meet the deficits of the ranks below C (in rank order)
// two-pointer; every meeting is one replica.
//
// Parallel form of the two-pointer walk: with A the running totals of the
// spill list and B those of the deficit list, the replicas are exactly the
// gaps between consecutive values of the union of A and B; each value's
// place in the union comes from a binary search in the other list.
//
// The plan is O(E + R) work.  Every workgroup computes it redundantly in LDS
// (no grid-wide barrier, no second launch), with wave 0 alone doing the work
// (see wave_plan: lane l owns experts and ranks l, l + 64, ... in registers,
// scans run on DPP) and no workgroup barrier until the plan is done, while
// the other waves load keys and segment bases.  Five workgroups store it.
// Then each wave assigns the entries of one segment:
//   pos = (entries of the same expert in earlier segments)  -- from rs_scan
//       + (entries of the same expert earlier in this segment) -- a running
//         per-wave LDS counter plus the lane's rank among equal keys of its
//         64-entry chunk (ballot per key bit);
//   pos < keep_e -> home row, else the replica whose spill range holds
//   pos - keep_e (binary search of fixed depth).  Every lane computes both
//   and selects, so the time does not depend on how much of the routing
//   spills.  A wave takes its 64-entry chunks 4 or 8 at a time through each
//   of these steps, so that the LDS round trips of a group overlap.
#include "moonep_internal.hpp"

namespace moonep {

namespace {

// LDS tables of the plan (int32).  E1 = E + 1, R1 = R + 1, CAP = E + R words.
struct PlanLds {
    // per expert
    int32_t *T, *P, *spill, *Sp, *keep, *home_dst, *rep_first, *rep_cnt;
    // spill list (A), index i < nA
    int32_t *Aval, *Aexp, *Aexcl, *posA;
    // per rank / deficit list (B), index j < nB
    int32_t *load, *Bval, *Brank, *Brow, *NC, *posB;  // Brow: first replica row base (load - Dp)
    // per replica (plan order)
    int32_t *U, *rai, *rbj, *rexp, *rhost, *rcnt, *rso, *rrow, *rdst;
    int32_t *misc;  // [16]: scalars of the plan header
    int32_t *run;   // [kWaves][E]: per-wave running counts
    int32_t *keys0; // [kChunkBatch * 64]: wave 0's first keys, staged by wave 1
};

constexpr int kEArrays = 12, kRArrays = 6, kCArrays = 9;

__host__ __device__ inline size_t plan_lds_words(int32_t E, int32_t R)
{
    const size_t e1 = (size_t)E + 1, r1 = (size_t)R + 1, cap = (size_t)E + R;
    return kEArrays * e1 + kRArrays * r1 + kCArrays * cap + 16 + (size_t)kWaves * E +
           (size_t)kChunkBatch * 64;
}

__device__ inline PlanLds carve(int32_t *base, int32_t E, int32_t R)
{
    PlanLds L;
    const int32_t e1 = E + 1, r1 = R + 1, cap = E + R;
    int32_t *p = base;
    int32_t **e_arrays[kEArrays] = {&L.T,         &L.P,         &L.spill,   &L.Sp,
                                    &L.keep,      &L.home_dst,  &L.rep_first, &L.rep_cnt,
                                    &L.Aval,      &L.Aexp,      &L.Aexcl,   &L.posA};
    for (int32_t **a : e_arrays) {
        *a = p;
        p += e1;
    }
    int32_t **r_arrays[kRArrays] = {&L.load, &L.Bval, &L.Brank, &L.Brow, &L.NC, &L.posB};
    for (int32_t **a : r_arrays) {
        *a = p;
        p += r1;
    }
    int32_t **c_arrays[kCArrays] = {&L.U, &L.rai, &L.rbj, &L.rexp, &L.rhost, &L.rcnt, &L.rso,
                                    &L.rrow, &L.rdst};
    for (int32_t **a : c_arrays) {
        *a = p;
        p += cap;
    }
    L.misc = p;
    p += 16;
    L.run = p;
    p += (size_t)kWaves * E;
    L.keys0 = p;
    return L;
}

// Exclusive scans of A arrays held in registers: value i of lane l sits at
// position l + 64 i of its array.  ex[a][i] = sum of array a's values at
// earlier positions; tot[a] = the sum of all of them.  The A x N chains are
// independent of one another, so they interleave.
template <int A, int N>
__device__ inline void strided_scan(const int32_t (&v)[A][N], int32_t (&ex)[A][N], int32_t (&tot)[A])
{
    int32_t inc[A][N];
#pragma unroll
    for (int a = 0; a < A; ++a)
#pragma unroll
        for (int i = 0; i < N; ++i)
            inc[a][i] = wave_incl_sum(v[a][i]);
#pragma unroll
    for (int a = 0; a < A; ++a) {
        int32_t base = 0;
#pragma unroll
        for (int i = 0; i < N; ++i) {
            ex[a][i] = base + inc[a][i] - v[a][i];
            base += __builtin_amdgcn_readlane(inc[a][i], 63);
        }
        tot[a] = base;
    }
}

// For each x1[i]: the number of values of the strictly increasing
// s1[0..n1) below it, and likewise for x2 in s2, in a fixed number of steps
// (2^steps > n1 and n2) so that the time does not depend on n1 and n2.  All
// the searches advance together, one LDS read each per step.
template <int N>
__device__ inline void count_below_sorted2(const int32_t *s1, int n1, const int32_t (&x1)[N],
                                           int32_t (&c1)[N], const int32_t *s2, int n2,
                                           const int32_t (&x2)[N], int32_t (&c2)[N], int steps)
{
#pragma unroll
    for (int i = 0; i < N; ++i) {
        c1[i] = 0;
        c2[i] = 0;
    }
    for (int st = steps; st >= 0; --st) {
#pragma unroll
        for (int i = 0; i < N; ++i) {
            const int t1 = c1[i] + (1 << st), t2 = c2[i] + (1 << st);
            const bool in1 = t1 <= n1, in2 = t2 <= n2;
            const int32_t v1 = s1[(in1 ? t1 : 1) - 1];
            const int32_t v2 = s2[(in2 ? t2 : 1) - 1];
            c1[i] = (in1 & (v1 < x1[i])) ? t1 : c1[i];  // '&': the reads stay unconditional
            c2[i] = (in2 & (v2 < x2[i])) ? t2 : c2[i];
        }
    }
}

__host__ __device__ inline int ceil_log2(int v)
{
    int b = 0;
    while ((1 << b) < v)
        ++b;
    return b;
}

// The whole plan, computed by one wave into the LDS tables.  policy 0: an
// overfull rank spills from its lowest expert id; policy 1: from its largest
// count, ties to the lower id.
//
// Lane l owns experts l, l + 64, ..., and ranks (and list entries) l, l + 64,
// ...: PE of each, PE >= E / 64 >= R / 64.  Each step first reads what it
// needs for all of the lane's items, then computes, then stores, so a
// step's LDS reads are in flight together instead of one round trip per
// item; the scans run on registers.  Everything does the same work whatever
// the data: reads use clamped indices, and a lane with nothing to store
// writes a spare slot that no plan uses (index E of an expert array: at
// least one rank is not overfull, so at most E - 1 experts spill; index R of
// a rank array: when C > 0 at least one rank is not underfull; index cap - 1
// of a replica array: n_rep <= nA + nB - 1 <= cap - 2).  So the plan takes
// the same time with or without replicas.
template <int PE>
__device__ void wave_plan(const PlanLds &S, int32_t (&t)[PE], int32_t R, int32_t E, int32_t C,
                          int32_t policy)
{
    const int lane = lane_id();
    const int32_t Lx = E / R;
    const int32_t cap = E + R;

    // ---- expert counts (t[i]: expert lane + 64 i) and their prefix P -------
    int tmax = 0;
#pragma unroll
    for (int i = 0; i < PE; ++i) {
        t[i] = lane + 64 * i < E ? t[i] : 0;
        tmax = t[i] > tmax ? t[i] : tmax;
    }
    int32_t p[1][PE], ptot[1];
    {
        int32_t tt[1][PE];
#pragma unroll
        for (int i = 0; i < PE; ++i)
            tt[0][i] = t[i];
        strided_scan<1, PE>(tt, p, ptot);
    }
#pragma unroll
    for (int i = 0; i < PE; ++i) {
        const int e = lane + 64 * i;
        if (e < E) {
            S.T[e] = t[i];
            S.P[e] = p[0][i];
        }
    }
    if (lane == 0)
        S.P[E] = ptot[0];
    wave_sync();

    // ---- rank loads, deficits, and the whole-expert spill -----------------
    // P at the first expert of each owned rank and of each owned expert's rank
    int32_t ra[PE], rb[PE], prs[PE], pre[PE];
#pragma unroll
    for (int j = 0; j < PE; ++j) {
        const int r = lane + 64 * j;
        const int rc = r < R ? r : R - 1;
        ra[j] = S.P[rc * Lx];
        rb[j] = S.P[(rc + 1) * Lx];
    }
#pragma unroll
    for (int i = 0; i < PE; ++i) {
        const int e = lane + 64 * i;
        const int r = (e < E ? e : E - 1) / Lx;
        prs[i] = S.P[r * Lx];
        pre[i] = S.P[(r + 1) * Lx];
    }
    int32_t sc[4][PE];  // spill, spill flag (per expert); deficit, deficit flag (per rank)
    int32_t ld[PE];     // rank loads
#pragma unroll
    for (int j = 0; j < PE; ++j) {
        const int r = lane + 64 * j;
        ld[j] = rb[j] - ra[j];
        if (r < R)
            S.load[r] = ld[j];
        sc[2][j] = r < R && ld[j] < C ? C - ld[j] : 0;
        sc[3][j] = r < R && ld[j] < C ? 1 : 0;
    }
    // what the experts taken before e hold: the prefix of the rank's counts
    // (lowest id first), or the sum of the rank's counts ordered before e by
    // (count descending, id ascending), read kLW of the rank's counts at a
    // time for all of the lane's experts together
    int32_t before[PE];
#pragma unroll
    for (int i = 0; i < PE; ++i)
        before[i] = p[0][i] - prs[i];
    if (policy == 1) {
        constexpr int kLW = PE <= 4 ? 8 : 32 / PE;
#pragma unroll
        for (int i = 0; i < PE; ++i)
            before[i] = 0;
        for (int32_t k0 = 0; k0 < Lx; k0 += kLW) {
            int32_t tk[PE][kLW];
#pragma unroll
            for (int i = 0; i < PE; ++i) {
                const int32_t k1 = (lane + 64 * i < E ? lane + 64 * i : E - 1) / Lx * Lx;
#pragma unroll
                for (int u = 0; u < kLW; ++u)
                    tk[i][u] = S.T[k1 + (k0 + u < Lx ? k0 + u : Lx - 1)];
            }
#pragma unroll
            for (int i = 0; i < PE; ++i) {
                const int e = lane + 64 * i;
                const int32_t k1 = (e < E ? e : E - 1) / Lx * Lx;
#pragma unroll
                for (int u = 0; u < kLW; ++u) {
                    const int32_t k = k1 + k0 + u;
                    const bool first = tk[i][u] > t[i] || (tk[i][u] == t[i] && k < e);
                    before[i] += k0 + u < Lx && first ? tk[i][u] : 0;
                }
            }
        }
    }
#pragma unroll
    for (int i = 0; i < PE; ++i) {
        const int e = lane + 64 * i;
        const int32_t excess = (pre[i] - prs[i]) - C;
        int32_t give = excess - before[i];
        give = give < 0 ? 0 : (give > t[i] ? t[i] : give);
        give = excess > 0 && e < E ? give : 0;
        sc[0][i] = give;
        sc[1][i] = give > 0 ? 1 : 0;
        if (e < E) {
            S.spill[e] = give;
            S.keep[e] = t[i] - give;
        }
    }
    int32_t sx[4][PE], stot[4];
    strided_scan<4, PE>(sc, sx, stot);
    const int nA = stot[1], nB = stot[3];
#pragma unroll
    for (int i = 0; i < PE; ++i) {
        const int e = lane + 64 * i;
        if (e < E)
            S.Sp[e] = sx[0][i];
    }
    wave_sync();

    // ---- the spill (A) and deficit (B) lists, compacted; home rows -------
    int32_t sprs[PE];
#pragma unroll
    for (int i = 0; i < PE; ++i) {
        const int e = lane + 64 * i;
        sprs[i] = S.Sp[(e < E ? e : E - 1) / Lx * Lx];
    }
#pragma unroll
    for (int i = 0; i < PE; ++i) {
        const int e = lane + 64 * i;
        const int a = e < E && sc[0][i] > 0 ? sx[1][i] : E;
        S.Aval[a] = sx[0][i] + sc[0][i];
        S.Aexp[a] = e;
        S.Aexcl[a] = sx[0][i];
        if (e < E) {
            const int32_t r = e / Lx;
            // first destination row of expert e at home: rank base + earlier keeps
            S.home_dst[e] = r * C + (p[0][i] - prs[i]) - (sx[0][i] - sprs[i]);
            S.rep_first[e] = 0;
            S.rep_cnt[e] = 0;
        }
    }
#pragma unroll
    for (int j = 0; j < PE; ++j) {
        const int r = lane + 64 * j;
        const int b = r < R && sc[2][j] > 0 ? sx[3][j] : R;
        S.Bval[b] = sx[2][j] + sc[2][j];
        S.Brank[b] = r;
        // a replica that starts at union value lo on this rank starts at row
        // load + (lo - the deficits before this rank) of its buffer
        S.Brow[b] = ld[j] - sx[2][j];
    }
    wave_sync();

    // ---- the union of both lists' running totals -------------------------
    // Two searches of fixed depth, run side by side: each deficit total's
    // place among the spill totals (bca) and each spill total's among the
    // deficit totals (cb).  Both lists hold fewer than E entries (nA <= E - 1,
    // nB <= R - 1), so 2^ea >= E covers both; the extra steps of the shorter
    // list's search change nothing.
    const int ea = ceil_log2(E);
    int32_t bv[PE], bca[PE], avi[PE], cb[PE], ncv[1][PE];
#pragma unroll
    for (int k = 0; k < PE; ++k) {
        const int kk = lane + 64 * k;
        bv[k] = S.Bval[kk < R ? kk : R];
        avi[k] = S.Aval[kk < E ? kk : E];
    }
    {
        int32_t xb[PE], xa[PE];
#pragma unroll
        for (int k = 0; k < PE; ++k) {
            xb[k] = lane + 64 * k < nB ? bv[k] : 0;
            xa[k] = lane + 64 * k < nA ? avi[k] : 0;
        }
        count_below_sorted2<PE>(S.Aval, nA, xb, bca, S.Bval, nB, xa, cb, ea);
    }
    // deficit totals that coincide with a spill total
#pragma unroll
    for (int j = 0; j < PE; ++j) {
        const int jj = lane + 64 * j;
        const int32_t av = S.Aval[bca[j] < E ? bca[j] : E];
        ncv[0][j] = jj < nB && !(bca[j] < nA && av == bv[j]) ? 1 : 0;  // 1 = not shared with A
    }
    int32_t ncx[1][PE], nctot[1];
    strided_scan<1, PE>(ncv, ncx, nctot);
    const int n_rep = nA + nctot[0];
#pragma unroll
    for (int j = 0; j < PE; ++j) {
        const int jj = lane + 64 * j;
        if (jj < R)
            S.NC[jj] = ncx[0][j];
    }
    if (lane == 0)
        S.NC[R] = nctot[0];
    wave_sync();

    // place every spill boundary of the union
    {
        int32_t ncb[PE];
#pragma unroll
        for (int i = 0; i < PE; ++i)
            ncb[i] = S.NC[cb[i]];
#pragma unroll
        for (int i = 0; i < PE; ++i) {
            const int ii = lane + 64 * i;
            const bool live = ii < nA;
            const int pos = live ? ii + ncb[i] : cap - 1;
            S.U[pos] = avi[i];
            S.rai[pos] = ii;
            S.rbj[pos] = cb[i];
            S.posA[live ? ii : E] = pos;
        }
    }
    wave_sync();
    // and every deficit boundary no spill boundary shares
    {
        int32_t pa[PE];
#pragma unroll
        for (int j = 0; j < PE; ++j)
            pa[j] = S.posA[bca[j] < E ? bca[j] : E];
#pragma unroll
        for (int j = 0; j < PE; ++j) {
            const int jj = lane + 64 * j;
            const bool live = jj < nB;
            const bool own = live && ncv[0][j];
            const int pos = own ? bca[j] + ncx[0][j] : pa[j];
            const int w = own ? pos : cap - 1;
            S.U[w] = bv[j];
            S.rai[w] = bca[j];
            S.rbj[w] = jj;
            S.posB[live ? jj : R] = pos;
        }
    }
    wave_sync();

    // ---- replicas, per-expert replica ranges, replicas per rank -----------
    // The range reads do not depend on the replica stores, so they go first
    // and their round trip overlaps the replicas'.
    int32_t ex[PE], pprev[PE], pcur[PE], qprev[PE], qcur[PE];
#pragma unroll
    for (int k = 0; k < PE; ++k) {
        const int kk = lane + 64 * k;
        const int ic = kk < E ? kk : E, jc = kk < R ? kk : R;
        ex[k] = S.Aexp[ic];
        pprev[k] = S.posA[ic > 0 ? ic - 1 : 0];
        pcur[k] = S.posA[ic];
        qprev[k] = S.posB[jc > 0 ? jc - 1 : 0];
        qcur[k] = S.posB[jc];
    }
    constexpr int kJ = 2 * PE < 8 ? 2 * PE : 8;  // replica slots per lane and round: cap <= 128 PE
    for (int m0 = 0; m0 < cap; m0 += 64 * kJ) {
        int32_t lo[kJ], hi[kJ], ri[kJ], rj[kJ];
#pragma unroll
        for (int k = 0; k < kJ; ++k) {
            const int m = m0 + lane + 64 * k;
            const int mc = m < cap ? m : cap - 1;
            lo[k] = S.U[mc > 0 ? mc - 1 : 0];
            hi[k] = S.U[mc];
            ri[k] = S.rai[mc];
            rj[k] = S.rbj[mc];
        }
        int32_t host[kJ], aex[kJ], aexp[kJ], brow[kJ];
#pragma unroll
        for (int k = 0; k < kJ; ++k) {
            const int m = m0 + lane + 64 * k;
            lo[k] = m ? lo[k] : 0;
            // stale past n_rep: clamp to keep reads in bounds
            ri[k] = ri[k] < 0 ? 0 : (ri[k] > E ? E : ri[k]);
            rj[k] = rj[k] < 0 ? 0 : (rj[k] > R ? R : rj[k]);
            host[k] = S.Brank[rj[k]];
            aex[k] = S.Aexcl[ri[k]];
            aexp[k] = S.Aexp[ri[k]];
            brow[k] = S.Brow[rj[k]];
        }
#pragma unroll
        for (int k = 0; k < kJ; ++k) {
            const int m = m0 + lane + 64 * k;
            if (m < cap) {
                const bool live = m < n_rep;
                host[k] = host[k] < 0 ? 0 : (host[k] >= R ? R - 1 : host[k]);
                const int32_t rso = lo[k] - aex[k];
                const int32_t rrow = brow[k] + lo[k];
                S.rexp[m] = live ? aexp[k] : 0;
                S.rhost[m] = live ? host[k] : 0;
                S.rcnt[m] = live ? hi[k] - lo[k] : 0;
                S.rso[m] = live ? rso : 0;
                S.rrow[m] = live ? rrow : 0;
                S.rdst[m] = live ? host[k] * C + rrow - rso : 0;
            }
        }
    }
    int most = 0;
#pragma unroll
    for (int k = 0; k < PE; ++k) {
        const int kk = lane + 64 * k;
        const int e = kk < nA && ex[k] >= 0 && ex[k] < E ? ex[k] : E;
        const int f = kk ? pprev[k] + 1 : 0;
        S.rep_first[e] = f;
        S.rep_cnt[e] = pcur[k] - f + 1;
        const int g = kk ? qprev[k] + 1 : 0;
        const int c = qcur[k] - g + 1;  // replicas hosted by deficit rank kk
        most = kk < nB && c > most ? c : most;
    }
    most = wave_max_nonneg(most);
    tmax = wave_max_nonneg(tmax);
    if (lane == 0) {
        S.misc[MOONEP_PLAN_H_N_REP] = n_rep;
        S.misc[MOONEP_PLAN_H_N_SPILL] = nA;
        S.misc[MOONEP_PLAN_H_N_DEFICIT] = nB;
        S.misc[MOONEP_PLAN_H_MAX_REP_RANK] = most;
        S.misc[MOONEP_PLAN_H_TMAX] = tmax;
        S.misc[MOONEP_PLAN_H_C] = C;
        S.misc[MOONEP_PLAN_H_L] = Lx;
        S.misc[MOONEP_PLAN_H_CAP] = cap;
        for (int h = 8; h < 16; ++h)
            S.misc[h] = 0;
    }
}

}  // namespace

template <int PE, int kSlotGroup>
__global__ __launch_bounds__(kBlock) void plan_slots_kernel(
    const int32_t *__restrict__ topk, const int32_t *__restrict__ counts,
    const int32_t *__restrict__ seg_base, int64_t nk, int32_t R, int32_t E, int32_t C,
    int32_t segw, int32_t nseg, int32_t nbits, int32_t search_steps, int32_t policy,
    int32_t *__restrict__ plan, int32_t *__restrict__ slot_of, int32_t *__restrict__ src_of_slot)
{
    extern __shared__ int32_t lds[];
    const PlanLds S = carve(lds, E, R);
    const int tid = (int)threadIdx.x;
    const int wid = tid >> 6;
    const int lane = lane_id();
    const int32_t seg = (int32_t)blockIdx.x * kWaves + wid;
    const int32_t cap = E + R;

    // Wave 0 loads the expert counts the plan starts from, and the workgroup
    // waits for them before anything else is loaded, so they do not queue
    // behind other loads.  Wave 0 then issues no further global loads until
    // the plan is done; waves 1-3 load, ahead of the plan, the first batch of
    // keys (the chunks that hold entries) of their own segments and, for
    // wave 0, into LDS, and the segment bases of the workgroup's four
    // segments, which sit side by side in each expert's column: one 16-byte
    // load per expert when the segment count is a multiple of 4.
    int32_t t[PE];
    if (wid == 0) {
#pragma unroll
        for (int i = 0; i < PE; ++i) {
            const int e = lane + 64 * i;
            t[i] = counts[e < E ? e : E - 1];
        }
        __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): the counts are in
    }
    __syncthreads();
    const int64_t beg = (int64_t)seg * segw;
    const int64_t end = beg + segw < nk ? beg + segw : nk;
    const int32_t seg0 = (int32_t)blockIdx.x * kWaves;  // the workgroup's first segment (wave 0's)
    const int64_t beg0 = (int64_t)seg0 * segw;
    const int64_t end0 = beg0 + segw < nk ? beg0 + segw : nk;
    int32_t keys[kChunkBatch], keys0[kChunkBatch];
    if (wid != 0 && seg < nseg) {
#pragma unroll
        for (int c = 0; c < kChunkBatch; ++c) {
            const int64_t n = beg + c * 64 + lane;
            keys[c] = -1;
            if (beg + c * 64 < end)
                keys[c] = topk[n < end ? n : end - 1];
        }
    }
    if (wid == 1 && seg0 < nseg) {
#pragma unroll
        for (int c = 0; c < kChunkBatch; ++c) {
            const int64_t n = beg0 + c * 64 + lane;
            keys0[c] = -1;
            if (beg0 + c * 64 < end0)
                keys0[c] = topk[n < end0 ? n : end0 - 1];
        }
    }
    constexpr int kBE = (PE + 2) / 3;  // experts per thread of waves 1-3: E <= 64 PE <= 192 kBE
    int4 bq[kBE];
    if (wid != 0 && seg0 < nseg) {
        const bool vec = (nseg & 3) == 0;  // then seg0 + 3 < nseg and the group is 16-byte aligned
#pragma unroll
        for (int k = 0; k < kBE; ++k) {
            const int e = tid - 64 + (kBlock - 64) * k;
            const int32_t *col = seg_base + (int64_t)(e < E ? e : E - 1) * nseg;
            if (vec) {
                bq[k] = *(const int4 *)(col + seg0);
            } else {
                bq[k].x = col[seg0];
                bq[k].y = col[seg0 + 1 < nseg ? seg0 + 1 : seg0];
                bq[k].z = col[seg0 + 2 < nseg ? seg0 + 2 : seg0];
                bq[k].w = col[seg0 + 3 < nseg ? seg0 + 3 : seg0];
            }
        }
    }
    if (wid == 0) {
        wave_plan<PE>(S, t, R, E, C, policy);
    } else if (seg0 < nseg) {
#pragma unroll
        for (int k = 0; k < kBE; ++k) {
            const int e = tid - 64 + (kBlock - 64) * k;
            if (e < E) {
                S.run[e] = bq[k].x;  // segment seg0 always exists
                if (seg0 + 1 < nseg)
                    S.run[E + e] = bq[k].y;
                if (seg0 + 2 < nseg)
                    S.run[2 * E + e] = bq[k].z;
                if (seg0 + 3 < nseg)
                    S.run[3 * E + e] = bq[k].w;
            }
        }
        if (wid == 1) {
#pragma unroll
            for (int c = 0; c < kChunkBatch; ++c)
                S.keys0[c * 64 + lane] = keys0[c];
        }
    }
    int32_t *run = S.run + wid * E;
    __syncthreads();
    if (wid == 0 && seg < nseg) {
#pragma unroll
        for (int c = 0; c < kChunkBatch; ++c)
            keys[c] = S.keys0[c * 64 + lane];
    }

    // ---- the plan goes out in five parts, from up to five workgroups -------
    const int last_wg = (int)gridDim.x - 1;
    const PlanLayout pl = plan_layout(E, R);
    auto stores_part = [&](int part) { return (int)blockIdx.x == (part < last_wg ? part : last_wg); };
    if (stores_part(0)) {
        if (tid < 16)
            plan[pl.header + tid] = S.misc[tid];
        for (int m = tid; m < cap; m += kBlock) {
            plan[pl.rep_expert + m] = S.rexp[m];
            plan[pl.rep_host + m] = S.rhost[m];
        }
    }
    if (stores_part(3)) {
        for (int m = tid; m < cap; m += kBlock) {
            plan[pl.rep_count + m] = S.rcnt[m];
            plan[pl.rep_spill_off + m] = S.rso[m];
            plan[pl.rep_row_off + m] = S.rrow[m];
        }
    }
    if (stores_part(1)) {
        for (int e = tid; e < E; e += kBlock) {
            const int32_t r = e / (E / R);
            plan[pl.spill + e] = S.spill[e];
            plan[pl.keep + e] = S.keep[e];
            plan[pl.home_row_off + e] = S.home_dst[e] - r * C;
        }
    }
    if (stores_part(4)) {
        const int nA = S.misc[MOONEP_PLAN_H_N_SPILL];
        for (int e = tid; e < E; e += kBlock) {
            plan[pl.rep_first + e] = S.rep_first[e];
            plan[pl.rep_cnt + e] = S.rep_cnt[e];
            plan[pl.exp_rep_list + e] = e < nA ? S.Aexp[e] : 0;
        }
    }
    if (stores_part(2)) {
        // every rank's replica range: empty unless the rank hosts replicas
        const int nB = S.misc[MOONEP_PLAN_H_N_DEFICIT];
        for (int r = tid; r < R; r += kBlock) {
            plan[pl.load + r] = S.load[r];
            plan[pl.rank_rep_first + r] = 0;
            plan[pl.rank_rep_cnt + r] = 0;
        }
        __syncthreads();
        for (int j = tid; j < nB; j += kBlock) {
            const int f = j ? S.posB[j - 1] + 1 : 0;
            plan[pl.rank_rep_first + S.Brank[j]] = f;
            plan[pl.rank_rep_cnt + S.Brank[j]] = S.posB[j] - f + 1;
        }
    }

    // ---- slot assignment: one wave per segment -----------------------------
    // Chunks of 64 entries go kSlotGroup at a time through each step (4 or 8:
    // a segment's chunks, up to 8), so the LDS round trips of a group's
    // chunks overlap.
    if (seg >= nseg)
        return;
    for (int64_t b0 = beg; b0 < end; b0 += 64 * kChunkBatch) {
        if (b0 != beg) {
#pragma unroll
            for (int c = 0; c < kChunkBatch; ++c) {
                const int64_t n = b0 + c * 64 + lane;
                keys[c] = topk[n < end ? n : end - 1];
            }
        }
#pragma unroll
        for (int g = 0; g < kChunkBatch; g += kSlotGroup) {
            if (b0 + (int64_t)g * 64 >= end)
                break;  // no later chunk of the batch holds entries
            int32_t ee[kSlotGroup], got[kSlotGroup], pos[kSlotGroup];
            uint64_t same[kSlotGroup];
            bool ok[kSlotGroup];
            int leader[kSlotGroup];
#pragma unroll
            for (int u = 0; u < kSlotGroup; ++u) {
                const int64_t n = b0 + (g + u) * 64 + lane;
                const int32_t e = keys[g + u];
                ok[u] = n < end && e >= 0 && e < E;
                same[u] = ballot(ok[u]);
                ee[u] = ok[u] ? e : 0;
            }
            match_lanes(ee, nbits, same);  // lanes with an equal key
#pragma unroll
            for (int u = 0; u < kSlotGroup; ++u)
                leader[u] = 63 - __builtin_clzll(same[u] | 1ull);
            // The highest lane of each group of equal keys claims the group's
            // positions with one LDS atomic add, which returns the expert's
            // running count; the other lanes of the group read it from that
            // lane.  LDS executes one wave's atomics in issue order, so the
            // chunks need no barrier between them.
#pragma unroll
            for (int u = 0; u < kSlotGroup; ++u) {
                got[u] = 0;
                if (ok[u] && leader[u] == lane)
                    got[u] = atomicAdd(&run[ee[u]], __popcll(same[u]));
            }
#pragma unroll
            for (int u = 0; u < kSlotGroup; ++u)
                pos[u] = __shfl(got[u], leader[u], 64) + count_below(same[u]);
            // home destination and replica destination, both computed
            int32_t kp[kSlotGroup], home[kSlotGroup], q[kSlotGroup], last[kSlotGroup], j[kSlotGroup];
#pragma unroll
            for (int u = 0; u < kSlotGroup; ++u) {
                kp[u] = S.keep[ee[u]];
                home[u] = S.home_dst[ee[u]];
                j[u] = S.rep_first[ee[u]];
                last[u] = S.rep_cnt[ee[u]];
            }
#pragma unroll
            for (int u = 0; u < kSlotGroup; ++u) {
                home[u] += pos[u];
                q[u] = pos[u] - kp[u];
                last[u] += j[u] - 1;
            }
            // the table reads happen whether or not the entry has a replica, so
            // the search costs the same with and without replicas
            for (int st = search_steps; st >= 0; --st) {
#pragma unroll
                for (int u = 0; u < kSlotGroup; ++u) {
                    const int32_t t = j[u] + (1 << st);
                    const int32_t tt = t <= last[u] ? t : last[u];  // keep the read in the table
                    const int32_t so = S.rso[tt < 0 ? 0 : tt];
                    // '&', not '&&': the read stays unconditional, so the
                    // group's reads are issued together
                    j[u] = ((t <= last[u]) & (so <= q[u])) ? t : j[u];
                }
            }
            int32_t rd[kSlotGroup];
#pragma unroll
            for (int u = 0; u < kSlotGroup; ++u)
                rd[u] = S.rdst[j[u] < 0 ? 0 : j[u]];
#pragma unroll
            for (int u = 0; u < kSlotGroup; ++u) {
                const int64_t n = b0 + (g + u) * 64 + lane;
                const int32_t dst = pos[u] < kp[u] ? home[u] : rd[u] + q[u];
                // dst is in range whenever counts match topk; the check keeps a
                // mismatched call from writing outside src_of_slot.
                if (ok[u] && (uint64_t)(uint32_t)dst < (uint64_t)nk) {
                    slot_of[n] = dst;
                    src_of_slot[dst] = (int32_t)n;
                } else if (n < end) {
                    slot_of[n] = -1;
                }
            }
        }
    }
}

size_t plan_lds_bytes(int32_t E, int32_t R) { return plan_lds_words(E, R) * sizeof(int32_t); }

namespace {

// Large E and R need more than the default 64 KiB of dynamic LDS: raise the
// kernel's limit once per device, to what the largest allowed shape needs,
// so later calls with other shapes fit as well.
template <int PE, int G>
int raise_plan_lds()
{
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess)
        return MOONEP_ERR_HIP;
    static bool raised[64] = {};
    if (dev < 0 || dev >= 64 || !raised[dev]) {
        if (hipFuncSetAttribute((const void *)plan_slots_kernel<PE, G>,
                                hipFuncAttributeMaxDynamicSharedMemorySize,
                                (int)plan_lds_bytes(kMaxExperts, kMaxRanks)) != hipSuccess)
            return MOONEP_ERR_HIP;
        if (dev >= 0 && dev < 64)
            raised[dev] = true;
    }
    return MOONEP_OK;
}

template <int PE, int G>
int run_plan_g(const moonep_shape &s, const WsLayout &w, const int32_t *topk, const int32_t *counts,
               const int32_t *base, int steps, int32_t policy, int32_t *plan, int32_t *slot_of,
               int32_t *src_of_slot, hipStream_t st)
{
    const size_t lds = plan_lds_bytes(s.E, s.R);
    if (lds > 65536) {
        const int rc = raise_plan_lds<PE, G>();
        if (rc != MOONEP_OK)
            return rc;
    }
    const int blocks = w.nseg > 0 ? (w.nseg + kWaves - 1) / kWaves : 1;
    hipLaunchKernelGGL((plan_slots_kernel<PE, G>), dim3(blocks), dim3(kBlock), lds, st, topk, counts,
                       base, w.nk, s.R, s.E, s.S * s.K, w.segw, w.nseg, expert_bits(s.E), steps,
                       policy, plan, slot_of, src_of_slot);
    return hipGetLastError() == hipSuccess ? MOONEP_OK : MOONEP_ERR_HIP;
}

// Chunks per slot group: a segment of up to 256 entries is 4 chunks, a longer
// one is taken 8 at a time.
template <int PE>
int run_plan(const moonep_shape &s, const WsLayout &w, const int32_t *topk, const int32_t *counts,
             const int32_t *base, int steps, int32_t policy, int32_t *plan, int32_t *slot_of,
             int32_t *src_of_slot, hipStream_t st)
{
    if (w.segw <= 256)
        return run_plan_g<PE, 4>(s, w, topk, counts, base, steps, policy, plan, slot_of, src_of_slot, st);
    return run_plan_g<PE, 8>(s, w, topk, counts, base, steps, policy, plan, slot_of, src_of_slot, st);
}

}  // namespace

int launch_plan(const moonep_shape &s, const int32_t *topk, const int32_t *counts, void *ws,
                int32_t *plan, int32_t *slot_of, int32_t *src_of_slot, hipStream_t st,
                int32_t policy)
{
    const WsLayout w = ws_layout(s);
    const int32_t *base = (const int32_t *)((const char *)ws + w.hist_off);
    // Depth of the slot loop's replica search: an expert's replicas sit on
    // distinct deficit ranks, at most R - 1 of them, so the search covers
    // offsets 0 .. R - 2 from its first replica: 2^(steps + 1) >= R - 1.
    int steps = -1;
    while ((1 << (steps + 1)) < s.R - 1)
        ++steps;
    // experts per lane of the planning wave, rounded up to a power of two
    const int per = (s.E + 63) / 64;
    if (per <= 1)
        return run_plan<1>(s, w, topk, counts, base, steps, policy, plan, slot_of, src_of_slot, st);
    if (per <= 2)
        return run_plan<2>(s, w, topk, counts, base, steps, policy, plan, slot_of, src_of_slot, st);
    if (per <= 4)
        return run_plan<4>(s, w, topk, counts, base, steps, policy, plan, slot_of, src_of_slot, st);
    if (per <= 8)
        return run_plan<8>(s, w, topk, counts, base, steps, policy, plan, slot_of, src_of_slot, st);
    static_assert(kMaxExperts <= 64 * 16, "experts per lane of the planning wave");
    return run_plan<16>(s, w, topk, counts, base, steps, policy, plan, slot_of, src_of_slot, st);
}

}  // namespace moonep
