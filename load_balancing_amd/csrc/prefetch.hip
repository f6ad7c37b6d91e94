// prefetch.hip -- replica weight slots and the weight prefetch.
//
// The MoonEP article (ncijnetwork.com), section "The core idea: dynamic
// redundant experts": the redundant experts are prefetched before expert
// compute.  Its explainer "memory" panel: each rank has B prefetch slots that
// follow the expert rows of one contiguous weight tensor; training needs
// B = E/R, inference may use fewer; a rank that needs more distinct remote
// experts than B reads the extra weights from their home rank instead.
//
// Slots: the replicas a rank hosts have consecutive plan ids starting at
// rank_rep_first (deficits are matched in rank order), so replica j is its
// host's b = j - rank_rep_first[host]-th and takes slot host*B + b when b < B;
// otherwise it overflows (-1).  One thread per replica id.
//
// Prefetch: pool[wslot[j]] = w_home[rep_expert[j]], a bit copy of wbytes per
// slotted replica.  Every workgroup of a persistent grid first gathers the
// slotted replicas into LDS (n_rep is only known on the device), then walks
// (replica, 16 KiB chunk) items with 16-byte non-temporal loads and stores.
#include "moonep_internal.hpp"

namespace moonep {

__global__ __launch_bounds__(kBlock) void weight_slots_kernel(const int32_t *__restrict__ plan,
                                                              PlanLayout pl, int32_t R, int32_t B,
                                                              int32_t *__restrict__ wslot)
{
    const int32_t j = (int32_t)(blockIdx.x * blockDim.x + threadIdx.x);
    if (j >= pl.cap)
        return;
    const int32_t n_rep = plan[pl.header + MOONEP_PLAN_H_N_REP];
    int32_t slot = -1;
    const int32_t host = j < n_rep ? plan[pl.rep_host + j] : -1;
    if (host >= 0 && host < R) {
        const int32_t b = j - plan[pl.rank_rep_first + host];
        slot = b >= 0 && b < B ? host * B + b : -1;
    }
    wslot[j] = slot;
}

constexpr int kPrefetchUnroll = 4;  // 16-byte vectors per thread per item
constexpr int kMaxCap = kMaxExperts + kMaxRanks;

__global__ __launch_bounds__(kBlock) void prefetch_kernel(const int32_t *__restrict__ plan,
                                                          PlanLayout pl, const int32_t *__restrict__ wslot,
                                                          int32_t E, int32_t nslots, int64_t nvec,
                                                          int64_t nchunk,
                                                          const u32x4 *__restrict__ w_home,
                                                          u32x4 *__restrict__ pool)
{
    __shared__ int32_t src[kMaxCap], dst[kMaxCap];
    __shared__ int32_t wave_tot[kWaves];
    __shared__ int32_t n_pref_s;
    const int32_t n_rep_raw = plan[pl.header + MOONEP_PLAN_H_N_REP];
    const int32_t n_rep = n_rep_raw < 0 ? 0 : (n_rep_raw < pl.cap ? n_rep_raw : pl.cap);
    const int lane = lane_id(), wave = threadIdx.x / 64;
    // compact the slotted replicas, in plan order
    int32_t base = 0;
    for (int32_t j0 = 0; j0 < n_rep; j0 += kBlock) {
        const int32_t j = j0 + (int32_t)threadIdx.x;
        const int32_t s = j < n_rep ? wslot[j] : -1;
        const int32_t e = j < n_rep ? plan[pl.rep_expert + j] : -1;
        const bool take = s >= 0 && s < nslots && e >= 0 && e < E;  // in bounds even on a bad table
        const uint64_t m = ballot(take);
        if (lane == 0)
            wave_tot[wave] = __popcll(m);
        __syncthreads();
        int32_t off = base;
        for (int w = 0; w < wave; ++w)
            off += wave_tot[w];
        if (take) {
            const int32_t at = off + count_below(m);
            src[at] = e;
            dst[at] = s;
        }
        for (int w = 0; w < kWaves; ++w)
            base += wave_tot[w];
        __syncthreads();
    }
    if (threadIdx.x == 0)
        n_pref_s = base;
    __syncthreads();
    const int64_t items = (int64_t)n_pref_s * nchunk;
    constexpr int64_t kChunk = (int64_t)kBlock * kPrefetchUnroll;
    for (int64_t it = blockIdx.x; it < items; it += gridDim.x) {
        const int32_t q = (int32_t)(it / nchunk);
        const int64_t c = it - (int64_t)q * nchunk;
        const u32x4 *from = w_home + (int64_t)src[q] * nvec;
        u32x4 *to = pool + (int64_t)dst[q] * nvec;
        const int64_t v0 = c * kChunk + threadIdx.x;
        u32x4 r[kPrefetchUnroll];
#pragma unroll
        for (int u = 0; u < kPrefetchUnroll; ++u) {
            const int64_t v = v0 + (int64_t)u * kBlock;
            r[u] = load_nt(from + (v < nvec ? v : 0));
        }
#pragma unroll
        for (int u = 0; u < kPrefetchUnroll; ++u) {
            const int64_t v = v0 + (int64_t)u * kBlock;
            if (v < nvec)
                store_nt(to + v, r[u]);
        }
    }
}

int launch_weight_slots(const moonep_shape &s, const int32_t *plan, int32_t B, int32_t *wslot,
                        hipStream_t st)
{
    const PlanLayout pl = plan_layout(s.E, s.R);
    hipLaunchKernelGGL(weight_slots_kernel, dim3((pl.cap + kBlock - 1) / kBlock), dim3(kBlock), 0,
                       st, plan, pl, s.R, B, wslot);
    return hipGetLastError() == hipSuccess ? MOONEP_OK : MOONEP_ERR_HIP;
}

int launch_prefetch(const moonep_shape &s, const int32_t *plan, const int32_t *wslot, int32_t B,
                    int64_t wbytes, const void *w_home, void *pool, int grid, hipStream_t st)
{
    if (B == 0 || wbytes == 0)
        return MOONEP_OK;
    const PlanLayout pl = plan_layout(s.E, s.R);
    const int64_t nvec = wbytes / 16;
    const int64_t chunk = (int64_t)kBlock * kPrefetchUnroll;
    const int64_t nchunk = (nvec + chunk - 1) / chunk;
    hipLaunchKernelGGL(prefetch_kernel, dim3(grid), dim3(kBlock), 0, st, plan, pl, wslot,
                       s.E, s.R * B, nvec, nchunk, (const u32x4 *)w_home, (u32x4 *)pool);
    return hipGetLastError() == hipSuccess ? MOONEP_OK : MOONEP_ERR_HIP;
}

}  // namespace moonep
