// route_stats.hip -- expert counts T_e and maxvio for one routing step.
//
// maxvio = max_e T_e / Tbar - 1 with Tbar = S*K*R/E: the skew measure of the
// MoonEP article (ncijnetwork.com), section "The problem MoonEP targets", with
// Tbar as the explainer's "maxvio" panel computes it.
//
// Two launches:
//   rs_hist: one wave per contiguous segment of routed entries counts its
//            experts into a private LDS histogram (one ballot per key bit
//            finds the lanes sharing an expert, so the last lane of each
//            group adds the group size: no atomics, time independent of how
//            skewed the routing is) and stores it column-wise, [E][nseg].
//   rs_scan: one workgroup per expert turns its column into exclusive
//            per-segment bases (the stable start of each segment within the
//            expert, used by the slot assignment) and the total T_e.  The last
//            workgroup to finish computes Tmax and maxvio.
#include "moonep_internal.hpp"

namespace moonep {

__global__ __launch_bounds__(kBlock) void rs_hist_kernel(const int32_t *__restrict__ topk, int64_t nk,
                                                         int32_t E, int32_t segw, int32_t nseg,
                                                         int32_t nbits, int32_t *__restrict__ hist,
                                                         int32_t *__restrict__ ctl)
{
    extern __shared__ int32_t lds[];
    const int wid = (int)threadIdx.x >> 6;
    const int lane = lane_id();
    int32_t *h = lds + wid * E;
    for (int e = lane; e < E; e += 64)
        h[e] = 0;
    if (blockIdx.x == 0 && threadIdx.x == 0)
        ctl[kCtlTicket] = 0;  // rs_scan runs after this launch completes
    __syncthreads();

    const int32_t seg = (int32_t)blockIdx.x * kWaves + wid;
    if (seg >= nseg)
        return;
    const int64_t beg = (int64_t)seg * segw;
    const int64_t end = beg + segw < nk ? beg + segw : nk;
    bool bad = false;
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
            bad |= in && !ok;
            const uint64_t active = ballot(ok);
            if (active == 0)
                continue;
            const uint64_t same = match_lanes(e, active, nbits);
            if (ok && (same >> lane) == 1ull)  // highest lane of its group
                h[e] += __popcll(same);
            wave_sync();
        }
    }
    if (ballot(bad) != 0 && lane == 0)
        atomicCAS(&ctl[kCtlError], 0, (int32_t)MOONEP_DEV_BAD_EXPERT_ID);
    wave_sync();
    for (int e = lane; e < E; e += 64)
        hist[(int64_t)e * nseg + seg] = h[e];
}

__global__ __launch_bounds__(kBlock) void rs_scan_kernel(int32_t *__restrict__ hist, int32_t nseg,
                                                         int32_t E, int64_t nk,
                                                         int32_t *__restrict__ counts,
                                                         float *__restrict__ maxvio,
                                                         int32_t *__restrict__ ctl)
{
    __shared__ int tmp[kWaves];
    __shared__ int is_last;
    __shared__ int red[kWaves];
    const int e = (int)blockIdx.x;
    int32_t *col = hist + (int64_t)e * nseg;
    constexpr int kPer = kMaxSegments / kBlock;    // entries per thread, at most
    const int per = (nseg + kBlock - 1) / kBlock;  // <= kPer
    const int first = (int)threadIdx.x * per;
    int local[kPer] = {};
    // 16-byte groups when each thread's run is whole groups (per and nseg
    // multiples of 4: a group then lies wholly inside or outside the column,
    // and col is 16-byte aligned); single counts otherwise
    const bool vec = (per & 3) == 0 && (nseg & 3) == 0;
    if (vec) {
#pragma unroll
        for (int c = 0; c < kPer / 4; ++c) {
            const int s = first + 4 * c;
            if (4 * c < per && s < nseg) {
                const int4 v = *(const int4 *)(col + s);
                local[4 * c] = v.x;
                local[4 * c + 1] = v.y;
                local[4 * c + 2] = v.z;
                local[4 * c + 3] = v.w;
            }
        }
    } else {
        for (int i = 0; i < per && i < kPer; ++i) {
            const int s = first + i;
            local[i] = s < nseg ? col[s] : 0;
        }
    }
    int sum = 0;
#pragma unroll
    for (int i = 0; i < kPer; ++i)
        sum += local[i];
    int total = 0;
    int run = block_exclusive_scan(sum, tmp, &total);
    int ex[kPer];
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
        ex[i] = run;
        run += local[i];
    }
    if (vec) {
#pragma unroll
        for (int c = 0; c < kPer / 4; ++c) {
            const int s = first + 4 * c;
            if (4 * c < per && s < nseg)
                *(int4 *)(col + s) = make_int4(ex[4 * c], ex[4 * c + 1], ex[4 * c + 2], ex[4 * c + 3]);
        }
    } else {
        for (int i = 0; i < per && i < kPer; ++i) {
            const int s = first + i;
            if (s < nseg)
                col[s] = ex[i];
        }
    }
    if (threadIdx.x == 0) {
        counts[e] = total;
        __threadfence();
        const int ticket = atomicAdd(&ctl[kCtlTicket], 1);
        is_last = ticket == E - 1;
    }
    __syncthreads();
    if (!is_last)
        return;
    __threadfence();
    int m = 0;
    for (int i = (int)threadIdx.x; i < E; i += kBlock) {
        const int c = __hip_atomic_load(&counts[i], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        m = c > m ? c : m;
    }
    for (int d = 32; d > 0; d >>= 1) {
        const int o = __shfl_xor(m, d, 64);
        m = o > m ? o : m;
    }
    if (lane_id() == 0)
        red[threadIdx.x >> 6] = m;
    __syncthreads();
    if (threadIdx.x == 0) {
        int tmax = 0;
        for (int w = 0; w < kWaves; ++w)
            tmax = red[w] > tmax ? red[w] : tmax;
        if (nk == 0) {
            maxvio[0] = 0.0f;
        } else {
            const double ratio = (double)((int64_t)tmax * E) / (double)nk;
            maxvio[0] = (float)(ratio - 1.0);
        }
        ctl[kCtlTicket] = 0;  // ready for the next call even if rs_hist is skipped
    }
}

int launch_route_stats(const moonep_shape &s, const int32_t *topk, int32_t *counts, float *maxvio,
                       void *ws, hipStream_t st)
{
    const WsLayout w = ws_layout(s);
    int32_t *ctl = (int32_t *)ws;
    int32_t *hist = (int32_t *)((char *)ws + w.hist_off);
    if (w.nseg > 0) {
        const int blocks = (w.nseg + kWaves - 1) / kWaves;
        const size_t lds = (size_t)kWaves * s.E * sizeof(int32_t);
        hipLaunchKernelGGL(rs_hist_kernel, dim3(blocks), dim3(kBlock), lds, st, topk, w.nk, s.E,
                           w.segw, w.nseg, expert_bits(s.E), hist, ctl);
    }
    hipLaunchKernelGGL(rs_scan_kernel, dim3(s.E), dim3(kBlock), 0, st, hist, w.nseg, s.E, w.nk,
                       counts, maxvio, ctl);
    return hipGetLastError() == hipSuccess ? MOONEP_OK : MOONEP_ERR_HIP;
}

}  // namespace moonep
