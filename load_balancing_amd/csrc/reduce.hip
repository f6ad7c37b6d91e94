// reduce.hip -- replica weight-gradients back to their home experts.
//
// The MoonEP article (ncijnetwork.com), section "The core idea: dynamic
// redundant experts": gradients of the duplicated experts are reduced back to
// their home ranks in the backward pass.  Its explainer "memory" panel: those
// gradients sit in an fp32 reduce buffer (not the parameter gradients), and
// the reduction pulls each rank's slots home and then zeroes them for the next
// microbatch.
//
// home[e] = fp32(home[e] + rep[j1] + rep[j2] + ...) summed in fp64 in plan
// order, then rep[j] = 0.  A persistent grid walks (expert-with-replicas,
// chunk) items; the item count lives in the plan on the device, so the launch
// needs no host read.  Pure HBM stream: each replica element is read once and
// overwritten with zero, each home element read once and written once.
#include "moonep_internal.hpp"

namespace moonep {

template <bool kVec>
__global__ __launch_bounds__(kBlock) void replica_reduce_kernel(const int32_t *__restrict__ plan,
                                                                int32_t h_nspill, int32_t o_list,
                                                                int32_t o_first, int32_t o_cnt,
                                                                int64_t G, int64_t nchunk,
                                                                float *__restrict__ home,
                                                                float *__restrict__ rep)
{
    constexpr int64_t kPerThread = 8;  // floats per thread per item
    constexpr int64_t kChunk = kBlock * kPerThread;
    const int32_t n_exp = plan[h_nspill];
    const int64_t items = (int64_t)n_exp * nchunk;
    for (int64_t it = blockIdx.x; it < items; it += gridDim.x) {
        const int32_t ei = (int32_t)(it / nchunk);
        const int64_t c = it - (int64_t)ei * nchunk;
        const int32_t e = plan[o_list + ei];
        const int32_t j0 = plan[o_first + e];
        const int32_t nr = plan[o_cnt + e];
        float *hrow = home + (int64_t)e * G;
        if (kVec) {
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                const int64_t idx = c * kChunk + (int64_t)u * kBlock * 4 + threadIdx.x * 4;
                if (idx >= G)
                    continue;
                const f32x4 h = *(const f32x4 *)(hrow + idx);
                double a0 = h[0], a1 = h[1], a2 = h[2], a3 = h[3];
                for (int32_t j = 0; j < nr; ++j) {
                    u32x4 *rp = (u32x4 *)(rep + (int64_t)(j0 + j) * G + idx);
                    const u32x4 r = load_nt(rp);
                    a0 += (double)__uint_as_float(r[0]);
                    a1 += (double)__uint_as_float(r[1]);
                    a2 += (double)__uint_as_float(r[2]);
                    a3 += (double)__uint_as_float(r[3]);
                    store_nt(rp, u32x4{0, 0, 0, 0});
                }
                f32x4 o = {(float)a0, (float)a1, (float)a2, (float)a3};
                *(f32x4 *)(hrow + idx) = o;
            }
        } else {
            for (int u = 0; u < (int)kPerThread; ++u) {
                const int64_t idx = c * kChunk + (int64_t)u * kBlock + threadIdx.x;
                if (idx >= G)
                    continue;
                double a = hrow[idx];
                for (int32_t j = 0; j < nr; ++j) {
                    float *rp = rep + (int64_t)(j0 + j) * G + idx;
                    a += (double)*rp;
                    *rp = 0.0f;
                }
                hrow[idx] = (float)a;
            }
        }
    }
}

int launch_replica_reduce(const moonep_shape &s, const int32_t *plan, int64_t G, float *home,
                          float *rep, int grid, hipStream_t st)
{
    if (G == 0)
        return MOONEP_OK;
    const PlanLayout pl = plan_layout(s.E, s.R);
    const int64_t chunk = (int64_t)kBlock * 8;
    const int64_t nchunk = (G + chunk - 1) / chunk;
    const bool vec = (G % 4) == 0 && ((uintptr_t)home % 16) == 0 && ((uintptr_t)rep % 16) == 0;
    if (vec)
        hipLaunchKernelGGL(replica_reduce_kernel<true>, dim3(grid), dim3(kBlock), 0, st, plan,
                           pl.header + MOONEP_PLAN_H_N_SPILL, pl.exp_rep_list, pl.rep_first,
                           pl.rep_cnt, G, nchunk, home, rep);
    else
        hipLaunchKernelGGL(replica_reduce_kernel<false>, dim3(grid), dim3(kBlock), 0, st, plan,
                           pl.header + MOONEP_PLAN_H_N_SPILL, pl.exp_rep_list, pl.rep_first,
                           pl.rep_cnt, G, nchunk, home, rep);
    return hipGetLastError() == hipSuccess ? MOONEP_OK : MOONEP_ERR_HIP;
}

}  // namespace moonep
