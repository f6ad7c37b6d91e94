// movers.hip -- dispatch (fused permute), combine (fused weighted
// unpermute), combine backward and dispatch backward over the static
// expert-grouped buffer.
//
// The MoonEP article (ncijnetwork.com), three-property list and explainer
// "pillars" panel: tokens are written straight into their expert-grouped
// rows of a fixed S*K-row buffer per rank, and the expert outputs are
// gathered back from there, with no separate permute or copy-out.  The
// aipricedb.com README excerpt adds that the copy from the communication
// buffer into a user buffer is what this removes.
//
// All four are HBM-bound streams of 16-byte bf16 vectors (8 per lane); each
// of a token's K rows of the buffer is one contiguous 2H-byte run, so every
// access is fully coalesced, and token rows are read once.  Combine and the
// two backwards give one workgroup to one token: its K destination rows and gates
// are uniform (scalar) loads and all K row loads of a thread are issued before
// any use (out-of-range slots read row 0 and are masked afterwards, so no
// branch splits the loads).  Dispatch paces its stores instead (see there).
// Loads are non-temporal, which measured faster on gfx950 than cached ones
// for every mover.  Stores are non-temporal too: write-back or device-scope
// stores made a call itself up to 12% shorter, but they left dirty lines in
// the MALL that the next HBM traffic had to write back.  A call plus the
// 512 MiB read after it took as long as with non-temporal stores (dispatch
// 384 us either way, combine 349), so each call's time here includes its own
// writes to HBM.
#include "moonep_internal.hpp"

namespace moonep {

namespace {

constexpr int KC = 8;  // experts per token handled per pass (registers)

// Largest grid a mover launches, in workgroups; larger problems loop over the
// grid (or, for combine_bwd, take several launches).  A dispatch carries its
// size in work-items as a 32-bit number, and 2^22 workgroups of up to 256
// threads stay well inside it.
constexpr int64_t kMaxGrid = (int64_t)1 << 22;

// Largest workgroup size in {256, 128, 64} that divides V (64 if none).
inline int block_for(int32_t V)
{
    if (V % 256 == 0)
        return 256;
    if (V % 128 == 0)
        return 128;
    return 64;
}

// Resident waves per CU that measured best on gfx950 for each mover in the
// full step on the expert-grouped access pattern, each call starting with
// the MALL and L2 evicted (HBM efficiency falls when more scattered row
// requests are in flight; too few leave it idle): dispatch 12, combine 16,
// combine_bwd 16, dispatch_bwd 12 -- 3, 4, 4 and 3 workgroups of 256 threads.
// On the 1.2 GB sweep step: dispatch 225 us at 12 against 231-235 at 8, 16
// and 20; combine (fp64 sums, 118 VGPRs) 198-203 us at 16 against 205-207 at
// 12 and 225 at 8 (with the earlier fp32 chain, 198 at 12 and 209 at 16); combine_bwd
// 431 us at 16 against 445 at 12; dispatch_bwd, whose fp64 sums need 154
// VGPRs, 228 us at 8 and 203 at 12-20.  Dispatch of rows longer than one
// 256-thread workgroup (H = 4096 and 7168) runs one 64-thread workgroup per
// 1 KiB column block at 24: 3077 us on the DeepSeek-V3-like shape and 1591
// on the adversarial one, against 3180 and 1613 with 128- and 256-thread
// blocks at 16, the best of those (64 threads at 16: 3365 and 1552; at 32:
// 3600 and 1910).  Rows of one block (H = 2048) stay one 256-thread
// workgroup: 228-234 us against 239-249 for 64- or 128-thread blocks.
// combine_bwd of rows longer than one workgroup (each thread looping over
// several vectors) does better at 12: 3252-3294 us against 3388 at 16 on the
// adversarial shape (H = 4096), no change on the DeepSeek-V3-like one.
constexpr int kDispatchWaves = 12, kDispatchBlocksWaves = 24, kCombineWaves = 16,
              kCombineBlocksWaves = 12, kCombineBwdWaves = 16, kCombineBwdLongWaves = 12,
              kDispatchBwdWaves = 12;

// Dynamic LDS a workgroup of `threads` requests so that only
// waves_per_cu / (threads / 64) of them fit in one CU's LDS; the kernels do not
// use it, it only caps residency.
size_t residency_lds(int waves_per_cu, int threads)
{
    static int lds_per_cu = 0;
    if (lds_per_cu == 0) {
        int dev = 0, v = 0;
        if (hipGetDevice(&dev) == hipSuccess &&
            hipDeviceGetAttribute(&v, hipDeviceAttributeMaxSharedMemoryPerMultiprocessor, dev) ==
                hipSuccess && v > 0)
            lds_per_cu = v;
        else
            lds_per_cu = 160 * 1024;
    }
    int per_cu = waves_per_cu / (threads / 64);
    per_cu = per_cu < 2 ? 2 : per_cu;
    // between lds/(per_cu+1) and lds/per_cu, away from both (and under the
    // 64 KiB default dynamic limit), in 256-byte units
    const size_t b = (size_t)((double)lds_per_cu / (per_cu + 0.6));
    return b & ~(size_t)255;
}

}  // namespace

// Expert ids of one token, as uniform loads.  KT > 0: K = KT is known at
// compile time (one wide scalar load); KT == 0: runtime K, read in chunks of
// KC with clamped indices and masked afterwards.
template <int KT>
struct Slots {
    static constexpr int kN = KT > 0 ? KT : KC;
    uint32_t s[kN];
    float g[kN];

    __device__ __forceinline__ void load(const int32_t *so, const float *gt, int32_t K, int32_t k0,
                                         uint32_t nrows, bool with_gates)
    {
#pragma unroll
        for (int c = 0; c < kN; ++c) {
            const bool in = KT > 0 ? true : k0 + c < K;
            const int32_t k = KT > 0 ? c : (in ? k0 + c : K - 1);
            const uint32_t sk = (uint32_t)so[k];
            const float gk = with_gates ? gt[k] : 0.0f;
            s[c] = in && sk < nrows ? sk : 0xFFFFFFFFu;  // all-ones = skip
            g[c] = in ? gk : 0.0f;
        }
    }

    // True when every slot of this chunk is a real row: the stores can then go
    // out back to back.  A branch per store would make the compiler wait for
    // all earlier memory operations (stores included) before each one.
    __device__ __forceinline__ bool all_valid() const
    {
        bool ok = true;
#pragma unroll
        for (int c = 0; c < kN; ++c)
            ok = ok && s[c] != 0xFFFFFFFFu;
        return ok;
    }
};

// buf[slot_of[n]] = x[n div K], one token row and one 16-byte column per
// thread.  slot_of and buf are deliberately not __restrict__: a store to buf
// might then change slot_of, so each destination id is re-read through the
// vector path (an L2 hit) after the previous store, and since stores and
// vector loads retire in order, waiting for that id also waits for the
// previous store.  A thread thus keeps one row store in flight, spaced by one
// L2 round trip.  On the expert-grouped write pattern this measured about 10%
// faster on gfx950 than issuing all K stores back to back, and much faster
// than spacing them by an uncached read.
__device__ __forceinline__ void dispatch_column(const u32x4 *__restrict__ x,
                                                const int32_t *slot_of, u32x4 *buf, int64_t tok,
                                                int32_t V, int32_t v, int32_t K, uint32_t nrows)
{
    const u32x4 val = load_nt(x + tok * V + v);
    const int32_t *so = slot_of + tok * K;
    for (int32_t k = 0; k < K; ++k) {
        const uint32_t sk = (uint32_t)so[k];
        if (sk < nrows)
            store_nt(buf + (int64_t)sk * V + v, val);
    }
}

// Rows of one column block: tokens along grid x (grid-stride), grid y = 1.
// (Written with the column offset blockIdx.y * blockDim.x although it is 0:
// that form measured 2% faster on gfx950 than v = threadIdx.x, repeatably;
// the two differ only in the scalar set-up at kernel entry.)
__global__ __launch_bounds__(kBlock) void dispatch_kernel(const u32x4 *__restrict__ x,
                                                          const int32_t *slot_of, u32x4 *buf,
                                                          int64_t N, int32_t V, int32_t K,
                                                          uint32_t nrows)
{
    const int32_t v = (int32_t)(blockIdx.y * blockDim.x + threadIdx.x);
    if (v >= V)
        return;
    for (int64_t tok = blockIdx.x; tok < N; tok += gridDim.x)
        dispatch_column(x, slot_of, buf, tok, V, v, K, nrows);
}

// Rows of several column blocks: workgroup w = t*ncb + c covers column block
// c of token t, so the blocks of one token's rows are adjacent in launch order
// and each row is written in one pass.
__global__ __launch_bounds__(kBlock) void dispatch_blocks_kernel(const u32x4 *__restrict__ x,
                                                                 const int32_t *slot_of,
                                                                 u32x4 *buf, int64_t N, int32_t V,
                                                                 int32_t ncb, int32_t K,
                                                                 uint32_t nrows)
{
    const uint64_t total = (uint64_t)N * (uint64_t)ncb;
    for (uint64_t w = blockIdx.x; w < total; w += gridDim.x) {
        uint64_t tok;
        uint32_t c;
        if (w < 0xFFFFFFFFull) {
            tok = (uint32_t)w / (uint32_t)ncb;
            c = (uint32_t)w - (uint32_t)tok * (uint32_t)ncb;
        } else {
            tok = w / (uint64_t)ncb;
            c = (uint32_t)(w - tok * (uint64_t)ncb);
        }
        const int32_t v = (int32_t)(c * blockDim.x + threadIdx.x);
        if (v < V)
            dispatch_column(x, slot_of, buf, (int64_t)tok, V, v, K, nrows);
    }
}

// y[t] = bf16(sum_k g * out[slot]).  Each product of an fp32 gate and a bf16
// row element has at most 24 + 8 significant bits, so it is exact in fp64;
// the products are summed in fp64 in ascending k from +0 and the sum is
// rounded once to bf16 (bf16_of_double), whatever the signs of the terms.
// Out-of-range slots contribute nothing.
// Workgroup w = t*nwb + c covers column blocks [c*cpb, (c+1)*cpb) of token t:
// a whole row per workgroup when it is short (under 4 column blocks), one
// column block per workgroup otherwise; both measured best in their range.
template <int KT>
__global__ __launch_bounds__(kBlock) void combine_kernel(const u32x4 *__restrict__ out,
                                                         const float *__restrict__ gates,
                                                         const int32_t *__restrict__ slot_of,
                                                         u32x4 *__restrict__ y, int64_t N,
                                                         int32_t V, int32_t nwb, int32_t cpb,
                                                         int32_t K, uint32_t nrows)
{
    constexpr int kN = Slots<KT>::kN;
    const uint64_t total = (uint64_t)N * (uint64_t)nwb;
    for (uint64_t w = blockIdx.x; w < total; w += gridDim.x) {
        uint64_t tok;
        uint32_t wb;
        if (nwb == 1) {
            tok = w;
            wb = 0;
        } else if (w < 0xFFFFFFFFull) {
            tok = (uint32_t)w / (uint32_t)nwb;
            wb = (uint32_t)w - (uint32_t)tok * (uint32_t)nwb;
        } else {
            tok = w / (uint64_t)nwb;
            wb = (uint32_t)(w - tok * (uint64_t)nwb);
        }
        const int32_t v_end = (int32_t)((wb + 1) * cpb * blockDim.x) < V
                                  ? (int32_t)((wb + 1) * cpb * blockDim.x) : V;
        for (int32_t v = (int32_t)(wb * cpb * blockDim.x + threadIdx.x); v < v_end;
             v += (int32_t)blockDim.x) {
            const int32_t *so = slot_of + (int64_t)tok * K;
            const float *gt = gates + (int64_t)tok * K;
            double acc[8];
#pragma unroll
            for (int j = 0; j < 8; ++j)
                acc[j] = 0.0;
            for (int32_t k0 = 0; k0 < K; k0 += kN) {
                Slots<KT> sl;
                sl.load(so, gt, K, k0, nrows, true);
                u32x4 o[kN];
#pragma unroll
                for (int c = 0; c < kN; ++c)
                    o[c] = load_nt(out + (int64_t)(sl.s[c] != 0xFFFFFFFFu ? sl.s[c] : 0u) * V + v);
                // An out-of-range slot's row (read from row 0) and gate are
                // replaced by zeros: its term is then fma(0, 0, acc) = acc
                // (acc is never -0), which costs five selects per row rather
                // than a select per accumulator update.  The products are
                // exact, so the fused form rounds only the sum.
#pragma unroll
                for (int c = 0; c < kN; ++c) {
                    const bool use = sl.s[c] != 0xFFFFFFFFu;
                    const double g = (double)(use ? sl.g[c] : 0.0f);
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        const uint32_t ow = use ? o[c][j] : 0u;
                        acc[2 * j] = __builtin_fma(g, (double)bf16_lo(ow), acc[2 * j]);
                        acc[2 * j + 1] = __builtin_fma(g, (double)bf16_hi(ow), acc[2 * j + 1]);
                    }
                }
            }
            u32x4 r;
#pragma unroll
            for (int j = 0; j < 4; ++j)
                r[j] = bf16_of_double(acc[2 * j]) | (bf16_of_double(acc[2 * j + 1]) << 16);
            store_nt(y + (int64_t)tok * V + v, r);
        }
    }
}

// dx[t] = bf16(sum_k d_buf[slot_of[t*K+k]]), summed in fp64 in ascending k
// and rounded once; out-of-range slots contribute nothing.  Same grid and
// hoisted loads as combine.
template <int KT>
__global__ __launch_bounds__(kBlock) void dispatch_bwd_kernel(const u32x4 *__restrict__ d_buf,
                                                              const int32_t *__restrict__ slot_of,
                                                              u32x4 *__restrict__ dx, int64_t N,
                                                              int32_t V, int32_t nwb, int32_t cpb,
                                                              int32_t K, uint32_t nrows)
{
    constexpr int kN = Slots<KT>::kN;
    const uint64_t total = (uint64_t)N * (uint64_t)nwb;
    for (uint64_t w = blockIdx.x; w < total; w += gridDim.x) {
        uint64_t tok;
        uint32_t wb;
        if (nwb == 1) {
            tok = w;
            wb = 0;
        } else if (w < 0xFFFFFFFFull) {
            tok = (uint32_t)w / (uint32_t)nwb;
            wb = (uint32_t)w - (uint32_t)tok * (uint32_t)nwb;
        } else {
            tok = w / (uint64_t)nwb;
            wb = (uint32_t)(w - tok * (uint64_t)nwb);
        }
        const int32_t v_end = (int32_t)((wb + 1) * cpb * blockDim.x) < V
                                  ? (int32_t)((wb + 1) * cpb * blockDim.x) : V;
        for (int32_t v = (int32_t)(wb * cpb * blockDim.x + threadIdx.x); v < v_end;
             v += (int32_t)blockDim.x) {
            const int32_t *so = slot_of + (int64_t)tok * K;
            double acc[8];
#pragma unroll
            for (int j = 0; j < 8; ++j)
                acc[j] = 0.0;
            for (int32_t k0 = 0; k0 < K; k0 += kN) {
                Slots<KT> sl;
                sl.load(so, nullptr, K, k0, nrows, false);
                u32x4 o[kN];
#pragma unroll
                for (int c = 0; c < kN; ++c)
                    o[c] = load_nt(d_buf + (int64_t)(sl.s[c] != 0xFFFFFFFFu ? sl.s[c] : 0u) * V + v);
#pragma unroll
                for (int c = 0; c < kN; ++c) {
                    const bool use = sl.s[c] != 0xFFFFFFFFu;
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        const double a0 = acc[2 * j] + (double)bf16_lo(o[c][j]);
                        const double a1 = acc[2 * j + 1] + (double)bf16_hi(o[c][j]);
                        acc[2 * j] = use ? a0 : acc[2 * j];
                        acc[2 * j + 1] = use ? a1 : acc[2 * j + 1];
                    }
                }
            }
            u32x4 r;
#pragma unroll
            for (int j = 0; j < 4; ++j)
                r[j] = bf16_of_double(acc[2 * j]) | (bf16_of_double(acc[2 * j + 1]) << 16);
            store_nt(dx + (int64_t)tok * V + v, r);
        }
    }
}

// d_out[slot_of[n]] = bf16(g_n * dy[tok]) (exact product, one rounding);
// d_gates[n] = <dy[tok], out[slot_of[n]]> in fp32: per-thread partial dots
// over its columns, then a wave butterfly and a cross-wave sum in LDS.
// Workgroup b handles token b, or tok0 + b in the launches of a problem
// larger than one grid (kChunked: the token offset costs each workgroup's
// prologue a dependent load, measured 2-7% on the sweep, so only those
// launches pay it).
template <int KT, bool kChunked>
__global__ __launch_bounds__(kBlock) void combine_bwd_kernel(
    const u32x4 *__restrict__ dy, const u32x4 *__restrict__ out, const float *__restrict__ gates,
    const int32_t *__restrict__ slot_of, u32x4 *__restrict__ d_out, float *__restrict__ d_gates,
    int64_t tok0, int32_t V, int32_t K, uint32_t nrows)
{
    constexpr int kN = Slots<KT>::kN;
    __shared__ float red[kN][kWaves];
    const int64_t tok = kChunked ? tok0 + (int64_t)blockIdx.x : (int64_t)blockIdx.x;
    const int32_t *so = slot_of + tok * K;
    const float *gt = gates + tok * K;
    const int lane = lane_id();
    const int wid = (int)threadIdx.x >> 6;
    const int nw = (int)blockDim.x >> 6;
    for (int32_t k0 = 0; k0 < K; k0 += kN) {
        Slots<KT> sl;
        sl.load(so, gt, K, k0, nrows, true);
        const bool all = sl.all_valid();
        float dot[kN];
#pragma unroll
        for (int c = 0; c < kN; ++c)
            dot[c] = 0.0f;
        for (int32_t v = (int32_t)threadIdx.x; v < V; v += (int32_t)blockDim.x) {
            const u32x4 d = load_nt(dy + tok * V + v);
            u32x4 o[kN];
#pragma unroll
            for (int c = 0; c < kN; ++c)
                o[c] = load_nt(out + (int64_t)(sl.s[c] != 0xFFFFFFFFu ? sl.s[c] : 0u) * V + v);
            float df[8];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                df[2 * j] = bf16_lo(d[j]);
                df[2 * j + 1] = bf16_hi(d[j]);
            }
#pragma unroll
            for (int c = 0; c < kN; ++c) {
                float t = dot[c];
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    t = __builtin_fmaf(df[2 * j], bf16_lo(o[c][j]), t);
                    t = __builtin_fmaf(df[2 * j + 1], bf16_hi(o[c][j]), t);
                }
                dot[c] = sl.s[c] != 0xFFFFFFFFu ? t : 0.0f;
            }
            u32x4 r[kN];
#pragma unroll
            for (int c = 0; c < kN; ++c)
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    r[c][j] = bf16_of_exact_product(sl.g[c], df[2 * j]) |
                              (bf16_of_exact_product(sl.g[c], df[2 * j + 1]) << 16);
            if (all) {
#pragma unroll
                for (int c = 0; c < kN; ++c)
                    store_nt(d_out + (int64_t)sl.s[c] * V + v, r[c]);
            } else {
#pragma unroll
                for (int c = 0; c < kN; ++c)
                    if (sl.s[c] != 0xFFFFFFFFu)
                        store_nt(d_out + (int64_t)sl.s[c] * V + v, r[c]);
            }
        }
#pragma unroll
        for (int c = 0; c < kN; ++c) {
            float t = dot[c];
#pragma unroll
            for (int m = 32; m > 0; m >>= 1)
                t += __shfl_xor(t, m, 64);
            if (lane == 0)
                red[c][wid] = t;
        }
        __syncthreads();
        if ((int)threadIdx.x < kN && k0 + (int)threadIdx.x < K) {
            float t = 0.0f;
            for (int w = 0; w < nw; ++w)
                t += red[threadIdx.x][w];
            d_gates[tok * K + k0 + threadIdx.x] = t;
        }
        __syncthreads();
    }
}

// Instantiations for the usual top-k values; any other K takes the generic
// runtime-K path.
#define MOONEP_BY_K(K, F, ...)                                                   \
    switch (K) {                                                                  \
    case 1: F<1>(__VA_ARGS__); break;                                             \
    case 2: F<2>(__VA_ARGS__); break;                                             \
    case 4: F<4>(__VA_ARGS__); break;                                             \
    case 6: F<6>(__VA_ARGS__); break;                                             \
    case 8: F<8>(__VA_ARGS__); break;                                             \
    default: F<0>(__VA_ARGS__); break;                                            \
    }

template <int KT>
void run_combine(dim3 g, dim3 b, hipStream_t st, const u32x4 *out, const float *gates,
                 const int32_t *so, u32x4 *y, int64_t N, int32_t V, int32_t nwb, int32_t cpb,
                 int32_t K, uint32_t nrows)
{
    const int waves = b.x == kBlock ? kCombineWaves : kCombineBlocksWaves;
    hipLaunchKernelGGL(combine_kernel<KT>, g, b, residency_lds(waves, (int)b.x), st, out,
                       gates, so, y, N, V, nwb, cpb, K, nrows);
}

template <int KT>
void run_dispatch_bwd(dim3 g, dim3 b, hipStream_t st, const u32x4 *d_buf, const int32_t *so,
                      u32x4 *dx, int64_t N, int32_t V, int32_t nwb, int32_t cpb, int32_t K,
                      uint32_t nrows)
{
    hipLaunchKernelGGL(dispatch_bwd_kernel<KT>, g, b, residency_lds(kDispatchBwdWaves, (int)b.x), st,
                       d_buf, so, dx, N, V, nwb, cpb, K, nrows);
}

template <int KT>
void run_combine_bwd(dim3 g, dim3 b, hipStream_t st, const u32x4 *dy, const u32x4 *out,
                     const float *gates, const int32_t *so, u32x4 *d_out, float *d_gates,
                     int64_t total, int64_t tok0, int32_t V, int32_t K, uint32_t nrows)
{
    const size_t lds = residency_lds(V > (int32_t)b.x ? kCombineBwdLongWaves : kCombineBwdWaves, (int)b.x);
    if (tok0 == 0 && g.x == total)
        hipLaunchKernelGGL((combine_bwd_kernel<KT, false>), g, b, lds, st, dy, out, gates, so, d_out,
                           d_gates, tok0, V, K, nrows);
    else
        hipLaunchKernelGGL((combine_bwd_kernel<KT, true>), g, b, lds, st, dy, out, gates, so, d_out,
                           d_gates, tok0, V, K, nrows);
}

int launch_dispatch(const moonep_shape &s, const uint16_t *x, const int32_t *slot_of, uint16_t *buf,
                    hipStream_t st)
{
    const int64_t N = (int64_t)s.R * s.S;
    if (N == 0)
        return MOONEP_OK;
    const int32_t V = s.H / 8;
    const uint32_t nrows = (uint32_t)(N * s.K);
    // one workgroup per row when a row fits one; otherwise 64-thread blocks
    int bs = block_for(V);
    int32_t ncb = (V + bs - 1) / bs;
    if (ncb > 1) {
        bs = 64;
        ncb = (V + 63) / 64;
    }
    const int64_t total = N * ncb;
    const uint32_t grid = (uint32_t)(total < kMaxGrid ? total : kMaxGrid);
    const size_t lds = residency_lds(ncb == 1 ? kDispatchWaves : kDispatchBlocksWaves, bs);
    if (ncb == 1)
        hipLaunchKernelGGL(dispatch_kernel, dim3(grid, 1), dim3(bs), lds, st, (const u32x4 *)x,
                           slot_of, (u32x4 *)buf, N, V, s.K, nrows);
    else
        hipLaunchKernelGGL(dispatch_blocks_kernel, dim3(grid), dim3(bs), lds, st, (const u32x4 *)x,
                           slot_of, (u32x4 *)buf, N, V, ncb, s.K, nrows);
    return hipGetLastError() == hipSuccess ? MOONEP_OK : MOONEP_ERR_HIP;
}

int launch_combine(const moonep_shape &s, const uint16_t *out, const float *gates,
                   const int32_t *slot_of, uint16_t *y, hipStream_t st)
{
    const int64_t N = (int64_t)s.R * s.S;
    if (N == 0)
        return MOONEP_OK;
    const int32_t V = s.H / 8;
    const uint32_t nrows = (uint32_t)(N * s.K);
    // rows of several blocks in 64-thread blocks, as dispatch (adversarial
    // combine 1540 us against 1730 with 256-thread blocks; the DeepSeek-V3-like
    // one unchanged at 2790)
    int bs = block_for(V);
    int32_t ncb = (V + bs - 1) / bs;
    if (ncb > 1) {
        bs = 64;
        ncb = (V + 63) / 64;
    }
    const int32_t cpb = ncb < 4 ? ncb : 1;  // column blocks per workgroup
    const int32_t nwb = (ncb + cpb - 1) / cpb;
    const int64_t total = N * nwb;
    const uint32_t grid = (uint32_t)(total < kMaxGrid ? total : kMaxGrid);
    MOONEP_BY_K(s.K, run_combine, dim3(grid), dim3(bs), st, (const u32x4 *)out, gates, slot_of,
                (u32x4 *)y, N, V, nwb, cpb, s.K, nrows);
    return hipGetLastError() == hipSuccess ? MOONEP_OK : MOONEP_ERR_HIP;
}

int launch_dispatch_bwd(const moonep_shape &s, const uint16_t *d_buf, const int32_t *slot_of,
                        uint16_t *dx, hipStream_t st)
{
    const int64_t N = (int64_t)s.R * s.S;
    if (N == 0)
        return MOONEP_OK;
    const int32_t V = s.H / 8;
    const uint32_t nrows = (uint32_t)(N * s.K);
    // 64-thread column blocks for every row length: on the sweep's 2048-wide
    // rows 196-198 us against 204-205 with one 256-thread workgroup per row
    // (combine is not faster so); on the DeepSeek-V3-like shape 2.74-2.81 ms
    // against 2.83-2.87 with 128-thread blocks
    const int bs = 64;
    const int32_t ncb = (V + 63) / 64;
    const int32_t cpb = ncb < 4 ? ncb : 1;  // column blocks per workgroup, as combine
    const int32_t nwb = (ncb + cpb - 1) / cpb;
    const int64_t total = N * nwb;
    const uint32_t grid = (uint32_t)(total < kMaxGrid ? total : kMaxGrid);
    MOONEP_BY_K(s.K, run_dispatch_bwd, dim3(grid), dim3(bs), st, (const u32x4 *)d_buf, slot_of,
                (u32x4 *)dx, N, V, nwb, cpb, s.K, nrows);
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
    // one token per workgroup, in launches of at most kMaxGrid tokens (a
    // grid-stride loop here would cost the kernel registers it cannot spare
    // at its residency)
    for (int64_t t0 = 0; t0 < N; t0 += kMaxGrid) {
        const uint32_t grid = (uint32_t)(N - t0 < kMaxGrid ? N - t0 : kMaxGrid);
        MOONEP_BY_K(s.K, run_combine_bwd, dim3(grid), dim3(block_for(V)), st, (const u32x4 *)dy,
                    (const u32x4 *)out, gates, slot_of, (u32x4 *)d_out, d_gates, N, t0, V, s.K,
                    nrows);
        if (hipGetLastError() != hipSuccess)
            return MOONEP_ERR_HIP;
    }
    return MOONEP_OK;
}

}  // namespace moonep
