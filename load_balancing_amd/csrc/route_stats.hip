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
//            group adds the group size with one LDS atomic: time independent
//            of how skewed the routing is); the workgroup then stores its
//            four segments' counts column-wise, [E][nseg], four side by side
//            per expert.
//   rs_scan: one workgroup per expert turns its column into exclusive
//            per-segment bases (the stable start of each segment within the
//            expert, used by the slot assignment) and the total T_e.  maxvio
//            is an atomic max over the experts (see rs_scan_kernel), so no
//            workgroup waits for the others.
#include "moonep_internal.hpp"

namespace moonep {

// Waves (segments) per rs_hist workgroup.  Its counts go out as 16-byte
// column runs, one per expert and four segments; rs_hist on gfx950, us
// (sweep / DeepSeek-V3-like / adversarial): 4.3 / 7.8 / 6.6 at 4 waves, 4.5 /
// 7.5 / 6.4 at 8, 5.5 / 8.9 / 7.7 at 16, against 4.4 / 9.7 / 7.3 for one
// 4-byte store per expert and segment.
constexpr int kHistWaves = 4;
constexpr int kGroup = 4;  // 64-entry chunks matched side by side

template <int HW>
__global__ __launch_bounds__(HW * 64) void rs_hist_kernel(const int32_t *__restrict__ topk, int64_t nk,
                                                         int32_t E, int32_t segw, int32_t nseg,
                                                         int32_t nbits, int32_t *__restrict__ hist,
                                                         int32_t *__restrict__ ctl,
                                                         float *__restrict__ maxvio)
{
    extern __shared__ int32_t lds[];
    const int wid = (int)threadIdx.x >> 6;
    const int lane = lane_id();
    int32_t *h = lds + wid * E;  // this wave's own histogram: no workgroup barrier until the stores
    for (int e = lane; e < E; e += 64)
        h[e] = 0;
    if (blockIdx.x == 0 && threadIdx.x == 0)
        maxvio[0] = 0.0f;  // the start of rs_scan's atomic max, which runs after this launch
    wave_sync();

    const int32_t seg0 = (int32_t)blockIdx.x * HW;  // the workgroup's first segment
    const int32_t seg = seg0 + wid;
    const int64_t beg = (int64_t)seg * segw;
    const int64_t end = seg < nseg ? (beg + segw < nk ? beg + segw : nk) : beg;  // none past nseg
    bool bad = false;
    for (int64_t b0 = beg; b0 < end; b0 += 64 * kChunkBatch) {
        int32_t keys[kChunkBatch];
#pragma unroll
        for (int c = 0; c < kChunkBatch; ++c) {
            const int64_t n = b0 + c * 64 + lane;
            keys[c] = n < end ? topk[n] : -1;
        }
        // chunks kGroup at a time, their key matching side by side
#pragma unroll
        for (int g = 0; g < kChunkBatch; g += kGroup) {
            if (b0 + (int64_t)g * 64 >= end)
                break;  // no later chunk of the batch holds entries
            int32_t ee[kGroup];
            bool ok[kGroup];
            uint64_t same[kGroup];
#pragma unroll
            for (int u = 0; u < kGroup; ++u) {
                const int64_t n = b0 + (g + u) * 64 + lane;
                const int32_t e = keys[g + u];
                const bool in = n < end;
                ok[u] = in && e >= 0 && e < E;
                bad |= in && !ok[u];
                ee[u] = ok[u] ? e : 0;
                same[u] = ballot(ok[u]);
            }
            match_lanes(ee, nbits, same);  // lanes with an equal key
#pragma unroll
            for (int u = 0; u < kGroup; ++u)
                if (ok[u] && (same[u] >> lane) == 1ull)  // highest lane of its group
                    atomicAdd(&h[ee[u]], __popcll(same[u]));  // LDS; no barrier between chunks
        }
    }
    if (ballot(bad) != 0 && lane == 0)
        atomicCAS(&ctl[kCtlError], 0, (int32_t)MOONEP_DEV_BAD_EXPERT_ID);
    __syncthreads();
    // The workgroup's HW segments sit side by side in each expert's column:
    // 16-byte stores, HW / 4 per expert, when the segment count is a multiple
    // of HW (then all of them exist and the run is 16-byte aligned).
    const bool vec = nseg % HW == 0;
    for (int e = (int)threadIdx.x; e < E; e += HW * 64) {
        int32_t *col = hist + (int64_t)e * nseg + seg0;
        if (vec) {
#pragma unroll
            for (int q = 0; q < HW / 4; ++q)
                *(int4 *)(col + 4 * q) = make_int4(lds[(4 * q) * E + e], lds[(4 * q + 1) * E + e],
                                                   lds[(4 * q + 2) * E + e], lds[(4 * q + 3) * E + e]);
        } else {
#pragma unroll
            for (int w = 0; w < HW; ++w)
                if (seg0 + w < nseg)
                    col[w] = lds[w * E + e];
        }
    }
}

// maxvio = fp32((Tmax*E)/nk - 1) is the largest of the experts' fp32((T_e*E)/nk
// - 1): division by nk, the subtraction and the rounding are all monotonic.
// That largest value is >= +0 (Tmax is at least the mean), so an integer max
// of the fp32 bit patterns, started at +0 by rs_hist, finds it: a negative
// value's pattern is a negative integer and never wins.
__global__ __launch_bounds__(kBlock) void rs_scan_kernel(int32_t *__restrict__ hist, int32_t nseg,
                                                         int32_t E, int64_t nk,
                                                         int32_t *__restrict__ counts,
                                                         float *__restrict__ maxvio)
{
    __shared__ int tmp[kWaves];
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
        if (nk == 0) {
            if (e == 0)
                maxvio[0] = 0.0f;  // rs_hist does not run without entries
        } else {
            const double ratio = (double)((int64_t)total * E) / (double)nk;
            atomicMax((int *)maxvio, __float_as_int((float)(ratio - 1.0)));
        }
    }
}

int launch_route_stats(const moonep_shape &s, const int32_t *topk, int32_t *counts, float *maxvio,
                       void *ws, hipStream_t st)
{
    const WsLayout w = ws_layout(s);
    int32_t *ctl = (int32_t *)ws;
    int32_t *hist = (int32_t *)((char *)ws + w.hist_off);
    if (w.nseg > 0) {
        const int blocks = (w.nseg + kHistWaves - 1) / kHistWaves;
        const size_t lds = (size_t)kHistWaves * s.E * sizeof(int32_t);
        hipLaunchKernelGGL(rs_hist_kernel<kHistWaves>, dim3(blocks), dim3(kHistWaves * 64), lds, st, topk,
                           w.nk, s.E, w.segw, w.nseg, expert_bits(s.E), hist, ctl, maxvio);
    }
    hipLaunchKernelGGL(rs_scan_kernel, dim3(s.E), dim3(kBlock), 0, st, hist, w.nseg, s.E, w.nk,
                       counts, maxvio);
    return hipGetLastError() == hipSuccess ? MOONEP_OK : MOONEP_ERR_HIP;
}

}  // namespace moonep
