// movers.hip -- dispatch (fused permute), combine (fused weighted
// unpermute) and combine backward over the static expert-grouped buffer.
//
// The MoonEP article (ncijnetwork.com), three-property list and explainer
// "pillars" panel: tokens are written straight into their expert-grouped
// rows of a fixed S*K-row buffer per rank, and the expert outputs are
// gathered back from there, with no separate permute or copy-out.  The
// aipricedb.com README excerpt adds that the copy from the communication
// buffer into a user buffer is what this removes.
//
// All three are HBM-bound streams of 16-byte bf16 vectors (8 per lane).  Token
// rows are read once; each of a token's K rows of the buffer is one contiguous
// 2H-byte run, so every store and load is fully coalesced.  Write-once
// streams use non-temporal stores.
#include "moonep_internal.hpp"

namespace moonep {

// buf[slot_of[n]] = x[n div K].  One thread per (token, 16-byte vector).
__global__ __launch_bounds__(kBlock) void dispatch_kernel(const u32x4 *__restrict__ x,
                                                          const int32_t *__restrict__ slot_of,
                                                          u32x4 *__restrict__ buf, int64_t total,
                                                          int32_t V, int32_t K, uint32_t nrows)
{
    const int64_t i = (int64_t)blockIdx.x * kBlock + threadIdx.x;
    if (i >= total)
        return;
    const int64_t tok = i / V;
    const int64_t v = i - tok * V;
    const u32x4 val = load_nt(x + i);
    const int32_t *so = slot_of + tok * K;
    for (int k = 0; k < K; ++k) {
        const uint32_t s = (uint32_t)so[k];
        if (s < nrows)
            store_nt(buf + (int64_t)s * V + v, val);
    }
}

// y[t] = bf16(sum_k g * out[slot]) with an fp32 fused multiply-add chain in
// ascending k, starting from +0.
__global__ __launch_bounds__(kBlock) void combine_kernel(const u32x4 *__restrict__ out,
                                                         const float *__restrict__ gates,
                                                         const int32_t *__restrict__ slot_of,
                                                         u32x4 *__restrict__ y, int64_t total,
                                                         int32_t V, int32_t K, uint32_t nrows)
{
    constexpr int KC = 8;
    const int64_t i = (int64_t)blockIdx.x * kBlock + threadIdx.x;
    if (i >= total)
        return;
    const int64_t tok = i / V;
    const int64_t v = i - tok * V;
    float acc[8];
#pragma unroll
    for (int j = 0; j < 8; ++j)
        acc[j] = 0.0f;
    for (int k0 = 0; k0 < K; k0 += KC) {
        u32x4 vals[KC];
        float g[KC];
        bool use[KC];
#pragma unroll
        for (int c = 0; c < KC; ++c) {
            const int k = k0 + c;
            use[c] = false;
            g[c] = 0.0f;
            vals[c] = u32x4{0, 0, 0, 0};
            if (k < K) {
                const uint32_t s = (uint32_t)slot_of[tok * K + k];
                g[c] = gates[tok * K + k];
                use[c] = s < nrows;
                if (use[c])
                    vals[c] = load_nt(out + (int64_t)s * V + v);
            }
        }
#pragma unroll
        for (int c = 0; c < KC; ++c) {
            if (!use[c])
                continue;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                acc[2 * j] = __builtin_fmaf(g[c], bf16_lo(vals[c][j]), acc[2 * j]);
                acc[2 * j + 1] = __builtin_fmaf(g[c], bf16_hi(vals[c][j]), acc[2 * j + 1]);
            }
        }
    }
    u32x4 r;
#pragma unroll
    for (int j = 0; j < 4; ++j)
        r[j] = pack_bf16(acc[2 * j], acc[2 * j + 1]);
    store_nt(y + i, r);
}

// d_out[slot_of[n]] = bf16(g_n * dy[tok]) (exact product, one rounding);
// d_gates[n] = <dy[tok], out[slot_of[n]]> in fp32.  One wave per token; each
// lane walks the row in 16-byte steps, then the wave reduces the K dots.
__global__ __launch_bounds__(kBlock) void combine_bwd_kernel(
    const u32x4 *__restrict__ dy, const u32x4 *__restrict__ out, const float *__restrict__ gates,
    const int32_t *__restrict__ slot_of, u32x4 *__restrict__ d_out, float *__restrict__ d_gates,
    int64_t N, int32_t V, int32_t K, uint32_t nrows)
{
    constexpr int KC = 8;
    const int64_t tok = (int64_t)blockIdx.x * kWaves + (threadIdx.x >> 6);
    if (tok >= N)
        return;
    const int lane = lane_id();
    for (int k0 = 0; k0 < K; k0 += KC) {
        uint32_t s[KC];
        float g[KC], dot[KC];
        bool use[KC];
#pragma unroll
        for (int c = 0; c < KC; ++c) {
            const int k = k0 + c;
            s[c] = 0;
            g[c] = 0.0f;
            dot[c] = 0.0f;
            use[c] = false;
            if (k < K) {
                s[c] = (uint32_t)slot_of[tok * K + k];
                g[c] = gates[tok * K + k];
                use[c] = s[c] < nrows;
            }
        }
        for (int64_t v = lane; v < V; v += 64) {
            const u32x4 d = load_nt(dy + tok * V + v);
            float df[8];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                df[2 * j] = bf16_lo(d[j]);
                df[2 * j + 1] = bf16_hi(d[j]);
            }
#pragma unroll
            for (int c = 0; c < KC; ++c) {
                if (!use[c])
                    continue;
                const int64_t row = (int64_t)s[c] * V + v;
                const u32x4 o = load_nt(out + row);
                u32x4 r;
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    dot[c] = __builtin_fmaf(df[2 * j], bf16_lo(o[j]), dot[c]);
                    dot[c] = __builtin_fmaf(df[2 * j + 1], bf16_hi(o[j]), dot[c]);
                    r[j] = bf16_of_exact_product(g[c], df[2 * j]) |
                           (bf16_of_exact_product(g[c], df[2 * j + 1]) << 16);
                }
                store_nt(d_out + row, r);
            }
        }
#pragma unroll
        for (int c = 0; c < KC; ++c) {
            float t = dot[c];
#pragma unroll
            for (int m = 32; m > 0; m >>= 1)
                t += __shfl_xor(t, m, 64);
            if (lane == 0 && k0 + c < K)
                d_gates[tok * K + k0 + c] = t;
        }
    }
}

int launch_dispatch(const moonep_shape &s, const uint16_t *x, const int32_t *slot_of, uint16_t *buf,
                    hipStream_t st)
{
    const int64_t N = (int64_t)s.R * s.S;
    const int32_t V = s.H / 8;
    const int64_t total = N * V;
    if (total == 0)
        return MOONEP_OK;
    const uint32_t nrows = (uint32_t)(N * s.K);
    const int64_t blocks = (total + kBlock - 1) / kBlock;
    hipLaunchKernelGGL(dispatch_kernel, dim3((uint32_t)blocks), dim3(kBlock), 0, st,
                       (const u32x4 *)x, slot_of, (u32x4 *)buf, total, V, s.K, nrows);
    return hipGetLastError() == hipSuccess ? MOONEP_OK : MOONEP_ERR_HIP;
}

int launch_combine(const moonep_shape &s, const uint16_t *out, const float *gates,
                   const int32_t *slot_of, uint16_t *y, hipStream_t st)
{
    const int64_t N = (int64_t)s.R * s.S;
    const int32_t V = s.H / 8;
    const int64_t total = N * V;
    if (total == 0)
        return MOONEP_OK;
    const uint32_t nrows = (uint32_t)(N * s.K);
    const int64_t blocks = (total + kBlock - 1) / kBlock;
    hipLaunchKernelGGL(combine_kernel, dim3((uint32_t)blocks), dim3(kBlock), 0, st,
                       (const u32x4 *)out, gates, slot_of, (u32x4 *)y, total, V, s.K, nrows);
    return hipGetLastError() == hipSuccess ? MOONEP_OK : MOONEP_ERR_HIP;
}

int launch_combine_bwd(const moonep_shape &s, const uint16_t *dy, const uint16_t *out,
                       const float *gates, const int32_t *slot_of, uint16_t *d_out, float *d_gates,
                       hipStream_t st)
{
    const int64_t N = (int64_t)s.R * s.S;
    if (N == 0)
        return MOONEP_OK;
    const int32_t V = s.H / 8;
    const uint32_t nrows = (uint32_t)(N * s.K);
    const int64_t blocks = (N + kWaves - 1) / kWaves;
    hipLaunchKernelGGL(combine_bwd_kernel, dim3((uint32_t)blocks), dim3(kBlock), 0, st,
                       (const u32x4 *)dy, (const u32x4 *)out, gates, slot_of, (u32x4 *)d_out,
                       d_gates, N, V, s.K, nrows);
    return hipGetLastError() == hipSuccess ? MOONEP_OK : MOONEP_ERR_HIP;
}

}  // namespace moonep
