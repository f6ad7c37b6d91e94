// plan.hip -- the replica plan and the slot maps, in one launch.
//
// What is planned: the MoonEP article (ncijnetwork.com), section "The core
// idea: dynamic redundant experts", requires that every rank receives exactly
// S*K routed entries, by adding a few redundant experts planned from the
// current router output; its three-property list asks that tokens land
// directly in their expert-grouped rows; the explainer's "memory" panel puts
// prefetch (replica) rows after the home rows.  The pages give no planner, so
// this one is the plainest greedy that meets the invariant: ranks above C
// give up whole-expert amounts starting at their lowest expert id; these
// amounts (in expert order) meet the deficits of the ranks below C (in rank
// order) two-pointer; every meeting is one replica.
//
// Parallel form of the two-pointer walk: with A the running totals of the
// spill list and B those of the deficit list, the replicas are exactly the
// gaps between consecutive values of the union of A and B; each value's
// place in the union comes from a binary search in the other list.  The plan
// is O(E + R) work, so every workgroup computes it redundantly in LDS (no
// grid-wide barrier, no second launch), workgroup 0 stores it, and then each
// wave assigns the entries of one segment:
//   pos = (entries of the same expert in earlier segments)  -- from rs_scan
//       + (entries of the same expert earlier in this segment) -- a running
//         per-wave LDS counter plus the lane's rank among equal keys of its
//         64-entry chunk (ballot per key bit, so time is skew-independent);
//   pos < keep_e -> home row, else the replica whose spill range holds
//   pos - keep_e (fixed-depth binary search).
#include "moonep_internal.hpp"

namespace moonep {

namespace {

// LDS tables of the plan (int32).  E-sized, R-sized and cap-sized arrays.
struct PlanLds {
    int32_t *T, *P, *spill, *Sp, *sidx, *keep, *home_dst, *rep_first, *rep_cnt;
    int32_t *Aval, *Aexp, *Aexcl, *posA;
    int32_t *load, *D, *Dp, *didx, *Bval, *Brank, *Bexcl, *Bca, *NC, *posB;
    int32_t *U, *rai, *rbj, *rexp, *rhost, *rcnt, *rso, *rrow, *rdst;
    int32_t *misc;  // [8]: scan scratch (kWaves) + scalars
    int32_t *run;   // [kWaves][E]
};

__host__ __device__ inline size_t plan_lds_words(int32_t E, int32_t R)
{
    const size_t e1 = (size_t)E + 1, r1 = (size_t)R + 1, cap = (size_t)E + R;
    return 13 * e1 + 10 * r1 + 9 * cap + 16 + (size_t)kWaves * E;
}

__device__ inline PlanLds carve(int32_t *base, int32_t E, int32_t R)
{
    PlanLds L;
    const int32_t e1 = E + 1, r1 = R + 1, cap = E + R;
    int32_t *p = base;
    int32_t **e_arrays[] = {&L.T, &L.P, &L.spill, &L.Sp, &L.sidx, &L.keep, &L.home_dst,
                            &L.rep_first, &L.rep_cnt, &L.Aval, &L.Aexp, &L.Aexcl, &L.posA};
    for (int32_t **a : e_arrays) {
        *a = p;
        p += e1;
    }
    int32_t **r_arrays[] = {&L.load, &L.D, &L.Dp, &L.didx, &L.Bval, &L.Brank, &L.Bexcl, &L.Bca,
                            &L.NC, &L.posB};
    for (int32_t **a : r_arrays) {
        *a = p;
        p += r1;
    }
    int32_t **c_arrays[] = {&L.U, &L.rai, &L.rbj, &L.rexp, &L.rhost, &L.rcnt, &L.rso, &L.rrow,
                            &L.rdst};
    for (int32_t **a : c_arrays) {
        *a = p;
        p += cap;
    }
    L.misc = p;
    p += 16;
    L.run = p;
    return L;
}

// Exclusive scan of in[0..n) into out[0..n] (out[n] = total), whole block.
__device__ void scan_array(const int32_t *in, int32_t *out, int n, int32_t *scratch)
{
    const int per = (n + kBlock - 1) / kBlock;
    const int first = (int)threadIdx.x * per;
    int sum = 0;
    for (int i = 0; i < per; ++i)
        if (first + i < n)
            sum += in[first + i];
    int total = 0;
    int run = block_exclusive_scan(sum, scratch, &total);
    for (int i = 0; i < per; ++i)
        if (first + i < n) {
            const int v = in[first + i];
            out[first + i] = run;
            run += v;
        }
    if (threadIdx.x == 0)
        out[n] = total;
    __syncthreads();
}

// Number of values of the strictly increasing a[0..n) below x.
__device__ inline int count_below_sorted(const int32_t *a, int n, int32_t x)
{
    int lo = 0, hi = n;
    while (lo < hi) {
        const int mid = (lo + hi) >> 1;
        if (a[mid] < x)
            lo = mid + 1;
        else
            hi = mid;
    }
    return lo;
}

}  // namespace

__global__ __launch_bounds__(kBlock) void plan_slots_kernel(
    const int32_t *__restrict__ topk, const int32_t *__restrict__ counts,
    const int32_t *__restrict__ seg_base, int64_t nk, int32_t R, int32_t E, int32_t C,
    int32_t segw, int32_t nseg, int32_t nbits, int32_t search_steps, int32_t *__restrict__ plan,
    int32_t *__restrict__ slot_of, int32_t *__restrict__ src_of_slot)
{
    extern __shared__ int32_t lds[];
    const PlanLds S = carve(lds, E, R);
    const int tid = (int)threadIdx.x;
    const int32_t Lx = E / R;
    const int32_t cap = E + R;

    // ---- loads and whole-expert spill -----------------------------------
    for (int e = tid; e < E; e += kBlock)
        S.T[e] = counts[e];
    __syncthreads();
    scan_array(S.T, S.P, E, S.misc);
    for (int r = tid; r < R; r += kBlock) {
        const int32_t ld = S.P[(r + 1) * Lx] - S.P[r * Lx];
        S.load[r] = ld;
        S.D[r] = ld < C ? C - ld : 0;
        S.Bca[r] = ld < C ? 1 : 0;  // deficit flag, reused below
    }
    __syncthreads();
    for (int e = tid; e < E; e += kBlock) {
        const int32_t r = e / Lx;
        const int32_t excess = S.load[r] - C;
        int32_t give = 0;
        if (excess > 0) {
            const int32_t before = S.P[e] - S.P[r * Lx];
            give = excess - before;
            give = give < 0 ? 0 : (give > S.T[e] ? S.T[e] : give);
        }
        S.spill[e] = give;
        S.keep[e] = S.T[e] - give;
        S.posA[e] = give > 0 ? 1 : 0;  // spill flag, overwritten later
    }
    __syncthreads();
    scan_array(S.spill, S.Sp, E, S.misc);
    scan_array(S.posA, S.sidx, E, S.misc);
    scan_array(S.D, S.Dp, R, S.misc);
    scan_array(S.Bca, S.didx, R, S.misc);
    const int nA = S.sidx[E];
    const int nB = S.didx[R];

    // ---- compact the spill (A) and deficit (B) lists --------------------
    for (int e = tid; e < E; e += kBlock) {
        const int32_t r = e / Lx;
        if (S.spill[e] > 0) {
            const int i = S.sidx[e];
            S.Aval[i] = S.Sp[e] + S.spill[e];
            S.Aexp[i] = e;
            S.Aexcl[i] = S.Sp[e];
        }
        // first destination row of expert e at home: rank base + earlier keeps
        S.home_dst[e] = r * C + (S.P[e] - S.P[r * Lx]) - (S.Sp[e] - S.Sp[r * Lx]);
        S.rep_first[e] = 0;
        S.rep_cnt[e] = 0;
    }
    for (int r = tid; r < R; r += kBlock)
        if (S.D[r] > 0) {
            const int j = S.didx[r];
            S.Bval[j] = S.Dp[r] + S.D[r];
            S.Brank[j] = r;
            S.Bexcl[j] = S.Dp[r];
        }
    __syncthreads();

    // ---- deficit totals that coincide with a spill total ------------------
    for (int j = tid; j < nB; j += kBlock) {
        const int a = count_below_sorted(S.Aval, nA, S.Bval[j]);
        S.Bca[j] = a;
        S.D[j] = (a < nA && S.Aval[a] == S.Bval[j]) ? 0 : 1;  // 1 = not shared with A
    }
    __syncthreads();
    scan_array(S.D, S.NC, nB, S.misc);
    const int n_rep = nA + S.NC[nB];

    // ---- place every boundary of the union ------------------------------
    for (int i = tid; i < nA; i += kBlock) {
        const int cb = count_below_sorted(S.Bval, nB, S.Aval[i]);
        const int pos = i + S.NC[cb];
        S.U[pos] = S.Aval[i];
        S.rai[pos] = i;
        S.rbj[pos] = cb;
        S.posA[i] = pos;
    }
    __syncthreads();
    for (int j = tid; j < nB; j += kBlock) {
        int pos;
        if (S.D[j]) {
            pos = S.Bca[j] + S.NC[j];
            S.U[pos] = S.Bval[j];
            S.rai[pos] = S.Bca[j];
            S.rbj[pos] = j;
        } else {
            pos = S.posA[S.Bca[j]];
        }
        S.posB[j] = pos;
    }
    __syncthreads();

    // ---- replicas, per-expert and per-rank ranges ------------------------
    for (int m = tid; m < cap; m += kBlock) {
        if (m < n_rep) {
            const int32_t lo = m ? S.U[m - 1] : 0;
            const int i = S.rai[m], j = S.rbj[m];
            const int32_t host = S.Brank[j];
            S.rexp[m] = S.Aexp[i];
            S.rhost[m] = host;
            S.rcnt[m] = S.U[m] - lo;
            S.rso[m] = lo - S.Aexcl[i];
            S.rrow[m] = S.load[host] + (lo - S.Bexcl[j]);
            S.rdst[m] = host * C + S.rrow[m] - S.rso[m];
        } else {
            S.rexp[m] = 0;
            S.rhost[m] = 0;
            S.rcnt[m] = 0;
            S.rso[m] = 0;
            S.rrow[m] = 0;
            S.rdst[m] = 0;
        }
    }
    for (int i = tid; i < nA; i += kBlock) {
        const int e = S.Aexp[i];
        const int f = i ? S.posA[i - 1] + 1 : 0;
        S.rep_first[e] = f;
        S.rep_cnt[e] = S.posA[i] - f + 1;
    }
    if (tid < 8)
        S.misc[8 + tid] = 0;
    __syncthreads();
    for (int j = tid; j < nB; j += kBlock) {
        const int f = j ? S.posB[j - 1] + 1 : 0;
        atomicMax(&S.misc[8], S.posB[j] - f + 1);  // most replicas on one rank
    }
    for (int e = tid; e < E; e += kBlock)
        atomicMax(&S.misc[9], S.T[e]);
    __syncthreads();

    // ---- workgroup 0 stores the plan --------------------------------------
    if (blockIdx.x == 0) {
        const PlanLayout pl = plan_layout(E, R);
        if (tid < 16) {
            int32_t v = 0;
            switch (tid) {
            case MOONEP_PLAN_H_N_REP: v = n_rep; break;
            case MOONEP_PLAN_H_N_SPILL: v = nA; break;
            case MOONEP_PLAN_H_N_DEFICIT: v = nB; break;
            case MOONEP_PLAN_H_MAX_REP_RANK: v = S.misc[8]; break;
            case MOONEP_PLAN_H_TMAX: v = S.misc[9]; break;
            case MOONEP_PLAN_H_C: v = C; break;
            case MOONEP_PLAN_H_L: v = Lx; break;
            case MOONEP_PLAN_H_CAP: v = cap; break;
            default: v = 0;
            }
            plan[pl.header + tid] = v;
        }
        for (int m = tid; m < cap; m += kBlock) {
            plan[pl.rep_expert + m] = S.rexp[m];
            plan[pl.rep_host + m] = S.rhost[m];
            plan[pl.rep_count + m] = S.rcnt[m];
            plan[pl.rep_spill_off + m] = S.rso[m];
            plan[pl.rep_row_off + m] = S.rrow[m];
        }
        for (int e = tid; e < E; e += kBlock) {
            const int32_t r = e / Lx;
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
    const int wid = tid >> 6;
    const int lane = lane_id();
    const int32_t seg = (int32_t)blockIdx.x * kWaves + wid;
    if (seg >= nseg)
        return;
    int32_t *run = S.run + wid * E;
    for (int e = lane; e < E; e += 64)
        run[e] = seg_base[(int64_t)e * nseg + seg];
    wave_sync();
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
            const int32_t pos = run[ee] + count_below(same);
            wave_sync();
            if (ok && (same >> lane) == 1ull)
                run[ee] = pos + 1;  // the highest lane of a group holds its last position
            wave_sync();
            int32_t dst;
            const int32_t kp = S.keep[ee];
            if (pos < kp) {
                dst = S.home_dst[ee] + pos;
            } else {
                const int32_t q = pos - kp;
                const int32_t f = S.rep_first[ee];
                const int32_t last = f + S.rep_cnt[ee] - 1;
                int32_t j = f;
                for (int st = search_steps; st >= 0; --st) {
                    const int32_t t = j + (1 << st);
                    if (t <= last && S.rso[t] <= q)
                        j = t;
                }
                dst = S.rdst[j] + q;
            }
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
                int32_t *plan, int32_t *slot_of, int32_t *src_of_slot, hipStream_t st)
{
    const WsLayout w = ws_layout(s);
    const int32_t *base = (const int32_t *)((const char *)ws + w.hist_off);
    const int blocks = w.nseg > 0 ? (w.nseg + kWaves - 1) / kWaves : 1;
    int steps = 0;
    while ((1 << (steps + 1)) <= s.R)
        ++steps;
    const size_t lds = plan_lds_bytes(s.E, s.R);
    if (lds > 65536) {
        // Large E and R need more than the default 64 KiB of dynamic LDS.
        static bool raised = false;
        if (!raised) {
            if (hipFuncSetAttribute((const void *)plan_slots_kernel,
                                    hipFuncAttributeMaxDynamicSharedMemorySize,
                                    (int)lds) != hipSuccess)
                return MOONEP_ERR_HIP;
            raised = true;
        }
    }
    hipLaunchKernelGGL(plan_slots_kernel, dim3(blocks), dim3(kBlock), lds, st, topk, counts, base,
                       w.nk, s.R, s.E, s.S * s.K, w.segw, w.nseg, expert_bits(s.E), steps, plan,
                       slot_of, src_of_slot);
    return hipGetLastError() == hipSuccess ? MOONEP_OK : MOONEP_ERR_HIP;
}

}  // namespace moonep
