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
// through wave-level scans -- 64 lanes, each owning a contiguous run of
// experts or ranks, with no workgroup barrier until the plan is done.
// Workgroup 0 stores it.  Then each wave assigns the entries of one segment:
//   pos = (entries of the same expert in earlier segments)  -- from rs_scan
//       + (entries of the same expert earlier in this segment) -- a running
//         per-wave LDS counter plus the lane's rank among equal keys of its
//         64-entry chunk (ballot per key bit);
//   pos < keep_e -> home row, else the replica whose spill range holds
//   pos - keep_e (binary search of fixed depth).  Every lane computes both
//   and selects, so the time does not depend on how much of the routing
//   spills.
#include "moonep_internal.hpp"

namespace moonep {

namespace {

// LDS tables of the plan (int32).  E1 = E + 1, R1 = R + 1, CAP = E + R words.
struct PlanLds {
    // per expert
    int32_t *T, *P, *spill, *Sp, *sflag, *sidx, *keep, *home_dst, *rep_first, *rep_cnt;
    // spill list (A), index i < nA
    int32_t *Aval, *Aexp, *Aexcl, *posA;
    // per rank / deficit list (B), index j < nB
    int32_t *load, *D, *dflag, *Dp, *didx, *Bval, *Brank, *Bexcl, *Bca, *nc, *NC, *posB;
    // per replica (plan order)
    int32_t *U, *rai, *rbj, *rexp, *rhost, *rcnt, *rso, *rrow, *rdst;
    int32_t *misc;  // [16]: scalars of the plan header
    int32_t *run;   // [kWaves][E]: per-wave running counts
};

constexpr int kEArrays = 14, kRArrays = 12, kCArrays = 9;

__host__ __device__ inline size_t plan_lds_words(int32_t E, int32_t R)
{
    const size_t e1 = (size_t)E + 1, r1 = (size_t)R + 1, cap = (size_t)E + R;
    return kEArrays * e1 + kRArrays * r1 + kCArrays * cap + 16 + (size_t)kWaves * E;
}

__device__ inline PlanLds carve(int32_t *base, int32_t E, int32_t R)
{
    PlanLds L;
    const int32_t e1 = E + 1, r1 = R + 1, cap = E + R;
    int32_t *p = base;
    int32_t **e_arrays[kEArrays] = {&L.T, &L.P, &L.spill, &L.Sp, &L.sflag, &L.sidx, &L.keep,
                                    &L.home_dst, &L.rep_first, &L.rep_cnt, &L.Aval, &L.Aexp,
                                    &L.Aexcl, &L.posA};
    for (int32_t **a : e_arrays) {
        *a = p;
        p += e1;
    }
    int32_t **r_arrays[kRArrays] = {&L.load, &L.D, &L.dflag, &L.Dp, &L.didx, &L.Bval,
                                    &L.Brank, &L.Bexcl, &L.Bca, &L.nc, &L.NC, &L.posB};
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
    return L;
}

// Exclusive scan across the 64 lanes of a wave; *total = sum of all lanes.
__device__ inline int wave_excl_scan(int v, int *total)
{
    const int lane = lane_id();
    int incl = v;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        const int o = __shfl_up(incl, d, 64);
        if (lane >= d)
            incl += o;
    }
    *total = __shfl(incl, 63, 64);
    return incl - v;
}

__device__ inline int wave_max(int v)
{
#pragma unroll
    for (int d = 32; d > 0; d >>= 1) {
        const int o = __shfl_xor(v, d, 64);
        v = o > v ? o : v;
    }
    return v;
}

// One wave: exclusive scan of in[0..n) into out[0..n], out[n] = total.  Lane
// l owns the contiguous run [l*per, (l+1)*per).  Returns the total.
__device__ int wave_scan_array(const int32_t *in, int32_t *out, int n)
{
    const int lane = lane_id();
    const int per = (n + 63) / 64;
    const int first = lane * per;
    int sum = 0;
    for (int i = 0; i < per; ++i)
        if (first + i < n)
            sum += in[first + i];
    int total = 0;
    int run = wave_excl_scan(sum, &total);
    for (int i = 0; i < per; ++i)
        if (first + i < n) {
            const int v = in[first + i];
            out[first + i] = run;
            run += v;
        }
    if (lane == 0)
        out[n] = total;
    wave_sync();
    return total;
}

// Four independent exclusive scans in one pass, so that their shuffle chains
// interleave: in0/in1 over n01 entries, in2/in3 over n23 entries, each laid
// out as in wave_scan_array (out[n] = total).  Returns the totals of in1 and
// in3 (the list lengths when those are 0/1 flags).
__device__ void wave_scan_arrays4(const int32_t *in0, int32_t *out0, const int32_t *in1,
                                  int32_t *out1, int n01, const int32_t *in2, int32_t *out2,
                                  const int32_t *in3, int32_t *out3, int n23, int *tot1, int *tot3)
{
    const int lane = lane_id();
    const int pa = (n01 + 63) / 64, pb = (n23 + 63) / 64;
    const int fa = lane * pa, fb = lane * pb;
    int s0 = 0, s1 = 0, s2 = 0, s3 = 0;
    for (int i = 0; i < pa; ++i)
        if (fa + i < n01) {
            s0 += in0[fa + i];
            s1 += in1[fa + i];
        }
    for (int i = 0; i < pb; ++i)
        if (fb + i < n23) {
            s2 += in2[fb + i];
            s3 += in3[fb + i];
        }
    int c0 = s0, c1 = s1, c2 = s2, c3 = s3;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        const int o0 = __shfl_up(c0, d, 64), o1 = __shfl_up(c1, d, 64);
        const int o2 = __shfl_up(c2, d, 64), o3 = __shfl_up(c3, d, 64);
        if (lane >= d) {
            c0 += o0;
            c1 += o1;
            c2 += o2;
            c3 += o3;
        }
    }
    const int t0 = __shfl(c0, 63, 64), t1 = __shfl(c1, 63, 64);
    const int t2 = __shfl(c2, 63, 64), t3 = __shfl(c3, 63, 64);
    int r0 = c0 - s0, r1 = c1 - s1, r2 = c2 - s2, r3 = c3 - s3;
    for (int i = 0; i < pa; ++i)
        if (fa + i < n01) {
            const int v0 = in0[fa + i], v1 = in1[fa + i];
            out0[fa + i] = r0;
            out1[fa + i] = r1;
            r0 += v0;
            r1 += v1;
        }
    for (int i = 0; i < pb; ++i)
        if (fb + i < n23) {
            const int v2 = in2[fb + i], v3 = in3[fb + i];
            out2[fb + i] = r2;
            out3[fb + i] = r3;
            r2 += v2;
            r3 += v3;
        }
    if (lane == 0) {
        out0[n01] = t0;
        out1[n01] = t1;
        out2[n23] = t2;
        out3[n23] = t3;
    }
    wave_sync();
    *tot1 = t1;
    *tot3 = t3;
}

// Number of values of the strictly increasing a[0..n) below x, with a fixed
// number of steps (2^steps > every n this is called with), so that the time
// does not depend on n.
__device__ inline int count_below_sorted(const int32_t *a, int n, int32_t x, int steps)
{
    int c = 0;  // a[0..c) < x
    for (int st = steps; st >= 0; --st) {
        const int t = c + (1 << st);
        const bool in = t <= n;
        const bool below = in && a[(in ? t : 1) - 1] < x;
        c = below ? t : c;
    }
    return c;
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
__device__ void wave_plan(const PlanLds &S, const int32_t *__restrict__ counts, int32_t R,
                          int32_t E, int32_t C, int32_t policy)
{
    const int lane = lane_id();
    const int32_t Lx = E / R;
    const int32_t cap = E + R;

    // rank loads before balancing
    for (int e = lane; e < E; e += 64)
        S.T[e] = counts[e];
    wave_sync();
    wave_scan_array(S.T, S.P, E);
    for (int r = lane; r < R; r += 64) {
        const int32_t ld = S.P[(r + 1) * Lx] - S.P[r * Lx];
        S.load[r] = ld;
        S.D[r] = ld < C ? C - ld : 0;
        S.dflag[r] = ld < C ? 1 : 0;
    }
    wave_sync();
    // Everything below does the same work whatever the data: loads use
    // clamped indices, and a lane with nothing to store writes a spare slot
    // that no plan uses (index E of an expert array: at least one rank is not
    // overfull, so at most E - 1 experts spill; index R of a rank array: when
    // C > 0 at least one rank is not underfull; index cap - 1 of a replica
    // array: n_rep <= nA + nB - 1 <= cap - 2).  So the plan takes the same
    // time with or without replicas.

    // whole-expert spill of overfull ranks: what the experts taken before e
    // hold is the prefix of the rank's counts (lowest id first), or the sum of
    // the rank's counts ordered before e by (count descending, id ascending)
    // -- L steps for every expert, whatever the counts
    for (int e = lane; e < E; e += 64) {
        const int32_t r = e / Lx;
        const int32_t excess = S.load[r] - C;
        int32_t before = S.P[e] - S.P[r * Lx];
        if (policy == 1) {
            const int32_t te = S.T[e];
            before = 0;
            for (int32_t k = r * Lx; k < (r + 1) * Lx; ++k) {
                const int32_t tk = S.T[k];
                before += tk > te || (tk == te && k < e) ? tk : 0;
            }
        }
        int32_t give = excess - before;
        give = give < 0 ? 0 : (give > S.T[e] ? S.T[e] : give);
        give = excess > 0 ? give : 0;
        S.spill[e] = give;
        S.keep[e] = S.T[e] - give;
        S.sflag[e] = give > 0 ? 1 : 0;
    }
    wave_sync();
    int nA = 0, nB = 0;
    wave_scan_arrays4(S.spill, S.Sp, S.sflag, S.sidx, E, S.D, S.Dp, S.dflag, S.didx, R, &nA, &nB);

    // compact the spill (A) and deficit (B) lists
    for (int e = lane; e < E; e += 64) {
        const int32_t r = e / Lx;
        const int i = S.spill[e] > 0 ? S.sidx[e] : E;
        S.Aval[i] = S.Sp[e] + S.spill[e];
        S.Aexp[i] = e;
        S.Aexcl[i] = S.Sp[e];
        // first destination row of expert e at home: rank base + earlier keeps
        S.home_dst[e] = r * C + (S.P[e] - S.P[r * Lx]) - (S.Sp[e] - S.Sp[r * Lx]);
        S.rep_first[e] = 0;
        S.rep_cnt[e] = 0;
    }
    for (int r = lane; r < R; r += 64) {
        const int j = S.D[r] > 0 ? S.didx[r] : R;
        S.Bval[j] = S.Dp[r] + S.D[r];
        S.Brank[j] = r;
        S.Bexcl[j] = S.Dp[r];
    }
    wave_sync();

    // The loops below run over all E (or R) slots with the list length as a
    // predicate, and the searches have fixed depth.
    const int ea = ceil_log2(E + 1), rb = ceil_log2(R + 1);

    // deficit totals that coincide with a spill total
    for (int j = lane; j < R; j += 64) {
        const bool live = j < nB;
        const int a = count_below_sorted(S.Aval, nA, live ? S.Bval[j] : 0, ea);
        S.Bca[j] = a;
        S.nc[j] = live && !(a < nA && S.Aval[a] == S.Bval[j]) ? 1 : 0;  // 1 = not shared with A
    }
    wave_sync();
    const int n_rep = nA + wave_scan_array(S.nc, S.NC, R);

    // place every boundary of the union
    for (int i = lane; i < E; i += 64) {
        const bool live = i < nA;
        const int cb = count_below_sorted(S.Bval, nB, live ? S.Aval[i] : 0, rb);
        const int pos = live ? i + S.NC[cb] : cap - 1;
        S.U[pos] = S.Aval[i];
        S.rai[pos] = i;
        S.rbj[pos] = cb;
        S.posA[live ? i : E] = pos;
    }
    wave_sync();
    for (int j = lane; j < R; j += 64) {
        const bool live = j < nB;
        const int ca = S.Bca[j];
        const bool own = live && S.nc[j];  // a deficit boundary no spill boundary shares
        const int pos = own ? ca + S.NC[j] : S.posA[ca < E ? ca : E];
        const int w = own ? pos : cap - 1;
        S.U[w] = S.Bval[j];
        S.rai[w] = ca;
        S.rbj[w] = j;
        S.posB[live ? j : R] = pos;
    }
    wave_sync();

    // replicas, per-expert ranges, header scalars
    for (int m = lane; m < cap; m += 64) {
        const bool live = m < n_rep;
        const int32_t lo = m ? S.U[m - 1] : 0;
        int i = S.rai[m], j = S.rbj[m];  // stale past n_rep: clamp to keep reads in bounds
        i = i < 0 ? 0 : (i > E ? E : i);
        j = j < 0 ? 0 : (j > R ? R : j);
        int32_t host = S.Brank[j];
        host = host < 0 ? 0 : (host >= R ? R - 1 : host);
        const int32_t rso = lo - S.Aexcl[i];
        const int32_t rrow = S.load[host] + (lo - S.Bexcl[j]);
        S.rexp[m] = live ? S.Aexp[i] : 0;
        S.rhost[m] = live ? host : 0;
        S.rcnt[m] = live ? S.U[m] - lo : 0;
        S.rso[m] = live ? rso : 0;
        S.rrow[m] = live ? rrow : 0;
        S.rdst[m] = live ? host * C + rrow - rso : 0;
    }
    for (int i = lane; i < E; i += 64) {
        int e = S.Aexp[i];
        e = i < nA && e >= 0 && e < E ? e : E;
        const int f = i ? S.posA[i - 1] + 1 : 0;
        S.rep_first[e] = f;
        S.rep_cnt[e] = S.posA[i] - f + 1;
    }
    int most = 0;
    for (int j = lane; j < R; j += 64) {
        const int f = j ? S.posB[j - 1] + 1 : 0;
        const int c = S.posB[j] - f + 1;  // replicas hosted by this rank
        most = j < nB && c > most ? c : most;
    }
    int tmax = 0;
    for (int e = lane; e < E; e += 64)
        tmax = S.T[e] > tmax ? S.T[e] : tmax;
    most = wave_max(most);
    tmax = wave_max(tmax);
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

    // Waves other than 0 fetch their segment's bases while wave 0 plans.
    int32_t *run = S.run + wid * E;
    if (seg < nseg)
        for (int e = lane; e < E; e += 64)
            run[e] = seg_base[(int64_t)e * nseg + seg];
    if (wid == 0)
        wave_plan(S, counts, R, E, C, policy);
    __syncthreads();

    // ---- workgroup 0 stores the plan --------------------------------------
    if (blockIdx.x == 0) {
        const PlanLayout pl = plan_layout(E, R);
        if (tid < 16)
            plan[pl.header + tid] = S.misc[tid];
        const int nA = S.misc[MOONEP_PLAN_H_N_SPILL];
        const int nB = S.misc[MOONEP_PLAN_H_N_DEFICIT];
        for (int m = tid; m < cap; m += kBlock) {
            plan[pl.rep_expert + m] = S.rexp[m];
            plan[pl.rep_host + m] = S.rhost[m];
            plan[pl.rep_count + m] = S.rcnt[m];
            plan[pl.rep_spill_off + m] = S.rso[m];
            plan[pl.rep_row_off + m] = S.rrow[m];
        }
        for (int e = tid; e < E; e += kBlock) {
            const int32_t r = e / (E / R);
            plan[pl.spill + e] = S.spill[e];
            plan[pl.keep + e] = S.keep[e];
            plan[pl.home_row_off + e] = S.home_dst[e] - r * C;
            plan[pl.rep_first + e] = S.rep_first[e];
            plan[pl.rep_cnt + e] = S.rep_cnt[e];
            plan[pl.exp_rep_list + e] = e < nA ? S.Aexp[e] : 0;
        }
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
    if (seg >= nseg)
        return;
    const int64_t beg = (int64_t)seg * segw;
    const int64_t end = beg + segw < nk ? beg + segw : nk;
    for (int64_t b0 = beg; b0 < end; b0 += 64 * kChunkBatch) {
        int32_t keys[kChunkBatch];
#pragma unroll
        for (int c = 0; c < kChunkBatch; ++c) {
            const int64_t n = b0 + c * 64 + lane;
            keys[c] = n < end ? topk[n] : -1;
        }
#pragma unroll
        for (int c = 0; c < kChunkBatch; ++c) {
            const int64_t n = b0 + c * 64 + lane;
            const int32_t e = keys[c];
            const bool in = n < end;
            const bool ok = in && e >= 0 && e < E;
            const uint64_t active = ballot(ok);
            if (active == 0) {
                if (in)
                    slot_of[n] = -1;
                continue;
            }
            const uint64_t same = match_lanes(e, active, nbits);
            const int ee = ok ? e : 0;
            // The highest lane of each group of equal keys claims the group's
            // positions with one LDS atomic add, which returns the expert's
            // running count; the other lanes of the group read it from that
            // lane.  LDS executes one wave's atomics in issue order, so the
            // chunks need no barrier between them.
            const int leader = 63 - __builtin_clzll(same | 1ull);
            int32_t got = 0;
            if (ok && leader == lane)
                got = atomicAdd(&run[ee], __popcll(same));
            const int32_t pos = __shfl(got, leader, 64) + count_below(same);
            // home destination and replica destination, both computed
            const int32_t kp = S.keep[ee];
            const int32_t home = S.home_dst[ee] + pos;
            const int32_t q = pos - kp;
            const int32_t f = S.rep_first[ee];
            const int32_t last = f + S.rep_cnt[ee] - 1;
            int32_t j = f;
            // the table reads happen whether or not the entry has a replica, so
            // the loop costs the same with and without replicas
            for (int st = search_steps; st >= 0; --st) {
                const int32_t t = j + (1 << st);
                const int32_t tt = t <= last ? t : last;  // keep the read in the table
                const int32_t so = S.rso[tt < 0 ? 0 : tt];
                j = t <= last && so <= q ? t : j;
            }
            const int32_t rd = S.rdst[j < 0 ? 0 : j];
            const int32_t dst = pos < kp ? home : rd + q;
            // dst is in range whenever counts match topk; the check keeps a
            // mismatched call from writing outside src_of_slot.
            if (ok && (uint64_t)(uint32_t)dst < (uint64_t)nk) {
                slot_of[n] = dst;
                src_of_slot[dst] = (int32_t)n;
            } else if (in) {
                slot_of[n] = -1;
            }
        }
    }
}

size_t plan_lds_bytes(int32_t E, int32_t R) { return plan_lds_words(E, R) * sizeof(int32_t); }

int launch_plan(const moonep_shape &s, const int32_t *topk, const int32_t *counts, void *ws,
                int32_t *plan, int32_t *slot_of, int32_t *src_of_slot, hipStream_t st,
                int32_t policy)
{
    const WsLayout w = ws_layout(s);
    const int32_t *base = (const int32_t *)((const char *)ws + w.hist_off);
    const int blocks = w.nseg > 0 ? (w.nseg + kWaves - 1) / kWaves : 1;
    int steps = 0;
    while ((1 << (steps + 1)) <= s.R)
        ++steps;
    const size_t lds = plan_lds_bytes(s.E, s.R);
    if (lds > 65536) {
        // Large E and R need more than the default 64 KiB of dynamic LDS: raise
        // the kernel's limit once per device, to what the largest allowed shape
        // needs, so later calls with other shapes fit as well.
        int dev = 0;
        if (hipGetDevice(&dev) != hipSuccess)
            return MOONEP_ERR_HIP;
        static bool raised[64] = {};
        if (dev < 0 || dev >= 64 || !raised[dev]) {
            if (hipFuncSetAttribute((const void *)plan_slots_kernel,
                                    hipFuncAttributeMaxDynamicSharedMemorySize,
                                    (int)plan_lds_bytes(kMaxExperts, kMaxRanks)) != hipSuccess)
                return MOONEP_ERR_HIP;
            if (dev >= 0 && dev < 64)
                raised[dev] = true;
        }
    }
    hipLaunchKernelGGL(plan_slots_kernel, dim3(blocks), dim3(kBlock), lds, st, topk, counts, base,
                       w.nk, s.R, s.E, s.S * s.K, w.segw, w.nseg, expert_bits(s.E), steps, policy,
                       plan, slot_of, src_of_slot);
    return hipGetLastError() == hipSuccess ? MOONEP_OK : MOONEP_ERR_HIP;
}

}  // namespace moonep
