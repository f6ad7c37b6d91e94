// ceilings.hip -- microbenchmarks of the machine ceilings the kernels are
// judged against: HBM streams (copy, read-only, write-only), copies of 4 KiB
// rows at random positions, the matrix pipe's bf16 rate, and LDS-DMA from
// data that sits in the L2.  Built as its
// own library (libmoonep_ceilings.so), outside the C-ABI of libmoonep.
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

__device__ __forceinline__ u32x4 load_nt(const u32x4 *p) { return __builtin_nontemporal_load(p); }
__device__ __forceinline__ void store_nt(u32x4 *p, u32x4 v) { __builtin_nontemporal_store(v, p); }

// mode 0: dst = src; mode 1: read src, one word per thread to sink; mode 2:
// write dst.  16-byte vectors, U vectors per thread in flight (all loads of a
// round issued before its stores), non-temporal loads.  NT_STORE picks
// non-temporal or write-back stores.  WAVE_CHUNKS = false: grid-stride per
// thread (a wave's U vectors are a grid stride apart); true: each wave owns
// runs of U contiguous KiB, the runs a grid of waves apart.
template <int U, bool NT_STORE, bool WAVE_CHUNKS>
__global__ __launch_bounds__(256) void stream_kernel(const u32x4 *__restrict__ src,
                                                     u32x4 *__restrict__ dst, int64_t n,
                                                     int mode, uint32_t *__restrict__ sink)
{
    const int64_t tid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t threads = (int64_t)gridDim.x * blockDim.x;
    // first vector of this thread, distance between its U vectors, and
    // distance between its rounds
    const int64_t i0 = WAVE_CHUNKS ? (tid >> 6) * U * 64 + (tid & 63) : tid;
    const int64_t ustride = WAVE_CHUNKS ? 64 : threads;
    const int64_t step = WAVE_CHUNKS ? (threads >> 6) * U * 64 : U * threads;
    uint32_t acc = 0;
    for (int64_t i = i0; i < n; i += step) {
        u32x4 v[U];
        if (mode != 2) {
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int64_t j = i + u * ustride;
                v[u] = j < n ? load_nt(src + j) : u32x4{0u, 0u, 0u, 0u};
            }
        } else {
#pragma unroll
            for (int u = 0; u < U; ++u)
                v[u] = u32x4{(uint32_t)i, (uint32_t)u, 2u, 3u};
        }
        if (mode == 1) {
#pragma unroll
            for (int u = 0; u < U; ++u)
                acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
        } else {
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int64_t j = i + u * ustride;
                if (j < n) {
                    if (NT_STORE)
                        store_nt(dst + j, v[u]);
                    else
                        dst[j] = v[u];
                }
            }
        }
    }
    if (mode == 1)
        sink[tid] = acc;  // sink holds one word per launched thread
}

typedef void (*stream_fn)(const u32x4 *, u32x4 *, int64_t, int, uint32_t *);

template <int U>
stream_fn pick_stream(int nt_store, int wave_chunks)
{
    if (nt_store)
        return wave_chunks ? stream_kernel<U, true, true> : stream_kernel<U, true, false>;
    return wave_chunks ? stream_kernel<U, false, true> : stream_kernel<U, false, false>;
}

// Rows of `row_vecs` 16-byte vectors: row i of dst (row dst_idx[i], or i when
// dst_idx is null) = row src_idx[i] of src (or i when src_idx is null).  A
// null src writes a constant (write-only); a null dst reads only, one word per
// thread to sink.  One workgroup per row per round, a grid-stride loop over
// rows; each thread moves row_vecs / blockDim.x vectors, all loads issued
// before the stores.  With random indices this is the access pattern of the
// scattered movers (4 KiB rows at random positions) without their arithmetic.
template <int U>
__global__ __launch_bounds__(256) void rows_kernel(const u32x4 *__restrict__ src, u32x4 *__restrict__ dst,
                                                   const int32_t *__restrict__ src_idx,
                                                   const int32_t *__restrict__ dst_idx, int64_t nrows,
                                                   int32_t row_vecs, uint32_t *__restrict__ sink)
{
    uint32_t acc = 0;
    for (int64_t r = blockIdx.x; r < nrows; r += gridDim.x) {
        u32x4 v[U];
        if (src) {
            const int64_t rs = src_idx ? src_idx[r] : r;
            const u32x4 *sp = src + rs * row_vecs;
#pragma unroll
            for (int u = 0; u < U; ++u)
                v[u] = load_nt(sp + u * (int)blockDim.x + (int)threadIdx.x);
        } else {
#pragma unroll
            for (int u = 0; u < U; ++u)
                v[u] = u32x4{(uint32_t)r, (uint32_t)u, 2u, 3u};
        }
        if (dst) {
            const int64_t rd = dst_idx ? dst_idx[r] : r;
            u32x4 *dp = dst + rd * row_vecs;
#pragma unroll
            for (int u = 0; u < U; ++u)
                store_nt(dp + u * (int)blockDim.x + (int)threadIdx.x, v[u]);
        } else {
#pragma unroll
            for (int u = 0; u < U; ++u)
                acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
        }
    }
    if (!dst)
        sink[(int64_t)blockIdx.x * blockDim.x + threadIdx.x] = acc;  // one word per launched thread
}

// kChains independent 32x32x16 bf16 MFMA accumulators per wave, `iters`
// rounds; operands come from the thread id so nothing folds.  One float per
// thread goes to out.
constexpr int kChains = 8;

__global__ __launch_bounds__(256) void mfma_kernel(int iters, float *__restrict__ out)
{
    const int tid = (int)(blockIdx.x * blockDim.x + threadIdx.x);
    bf16x8 a, b;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        a[j] = (__bf16)(float)((tid + j) & 7);
        b[j] = (__bf16)(float)((tid * 3 + j) & 7);
    }
    f32x16 acc[kChains];
#pragma unroll
    for (int c = 0; c < kChains; ++c)
#pragma unroll
        for (int r = 0; r < 16; ++r)
            acc[c][r] = 0.0f;
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int c = 0; c < kChains; ++c)
            acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[c], 0, 0, 0);
    }
    float s = 0.0f;
#pragma unroll
    for (int c = 0; c < kChains; ++c)
        s += acc[c][c];
    out[tid] = s;
}

// LDS-DMA (global_load_lds_dwordx4) from a buffer that stays in the L2: each
// wave loads kDmaLoads KiB per round into its own LDS region (one KiB per
// load: 64 lanes x 16 bytes), walking the buffer from a per-wave start, and
// waits for its loads every round.  One word of LDS per wave goes to out.
constexpr int kDmaLoads = 8;
constexpr int kDmaWaves = 8;

__global__ __launch_bounds__(kDmaWaves * 64) void lds_dma_kernel(const char *__restrict__ buf,
                                                                 int64_t chunks, int iters,
                                                                 uint32_t *__restrict__ out)
{
    __shared__ __align__(16) char lds[kDmaWaves * kDmaLoads * 1024];
    const int wave = (int)threadIdx.x >> 6, lane = (int)threadIdx.x & 63;
    char *mine = lds + wave * kDmaLoads * 1024;
    // chunk = one KiB of the buffer (chunks >= kDmaLoads); this wave starts
    // at a chunk of its own
    int64_t c = ((int64_t)blockIdx.x * kDmaWaves + wave) * kDmaLoads % chunks;
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int l = 0; l < kDmaLoads; ++l) {
            const int64_t cc = c + l < chunks ? c + l : c + l - chunks;
            __builtin_amdgcn_global_load_lds((const void *)(buf + cc * 1024 + lane * 16),
                                             (__attribute__((address_space(3))) void *)(mine + l * 1024),
                                             16, 0, 0);
        }
        __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): this round's loads are in LDS
        c = c + kDmaLoads < chunks ? c + kDmaLoads : c + kDmaLoads - chunks;
    }
    __syncthreads();
    if (lane == 0)
        out[blockIdx.x * kDmaWaves + wave] = *(const uint32_t *)mine;
}

}  // namespace

extern "C" {

// n_vec 16-byte vectors, workgroups of `block` threads (64, 128 or 256),
// `unroll` vectors per thread in flight (4 or 8), non-temporal or write-back
// stores, grid-stride or per-wave runs (see stream_kernel); sink must hold
// grid * block words (mode 1).
int ceil_stream(const void *src, void *dst, int64_t n_vec, int mode, int unroll, int nt_store,
                int wave_chunks, int grid, int block, void *sink, void *stream)
{
    if (n_vec < 0 || grid <= 0 || mode < 0 || mode > 2 || (block != 64 && block != 128 && block != 256) ||
        (unroll != 4 && unroll != 8))
        return -1;
    const stream_fn f = unroll == 4 ? pick_stream<4>(nt_store, wave_chunks) : pick_stream<8>(nt_store, wave_chunks);
    hipLaunchKernelGGL(f, dim3(grid), dim3(block), 0, (hipStream_t)stream, (const u32x4 *)src, (u32x4 *)dst,
                       n_vec, mode, (uint32_t *)sink);
    return hipGetLastError() == hipSuccess ? 0 : -2;
}

// nrows rows of row_vecs 16-byte vectors; src_idx / dst_idx (device, nrows
// entries each, values in [0, nrows)) or null for the identity; src null:
// write-only, dst null: read-only with sink holding grid * block words (one
// of src and dst must be set); block threads per row (64 or 256) with
// row_vecs == U * block for U in {1, 4}.
int ceil_rows(const void *src, void *dst, const int32_t *src_idx, const int32_t *dst_idx, int64_t nrows,
              int row_vecs, int grid, int block, void *sink, void *stream)
{
    if (nrows < 0 || grid <= 0 || (block != 64 && block != 256) || row_vecs <= 0 || row_vecs % block != 0 ||
        (!src && !dst) || (!dst && !sink))
        return -1;
    const int u = row_vecs / block;
    if (u == 1)
        hipLaunchKernelGGL(rows_kernel<1>, dim3(grid), dim3(block), 0, (hipStream_t)stream, (const u32x4 *)src,
                           (u32x4 *)dst, src_idx, dst_idx, nrows, row_vecs, (uint32_t *)sink);
    else if (u == 4)
        hipLaunchKernelGGL(rows_kernel<4>, dim3(grid), dim3(block), 0, (hipStream_t)stream, (const u32x4 *)src,
                           (u32x4 *)dst, src_idx, dst_idx, nrows, row_vecs, (uint32_t *)sink);
    else
        return -1;
    return hipGetLastError() == hipSuccess ? 0 : -2;
}

// out must hold grid * 256 floats.  Flops per launch: grid * 4 waves * iters
// * kChains * 32768.
int ceil_mfma(int grid, int iters, float *out, void *stream)
{
    if (grid <= 0 || iters <= 0)
        return -1;
    hipLaunchKernelGGL(mfma_kernel, dim3(grid), dim3(256), 0, (hipStream_t)stream, iters, out);
    return hipGetLastError() == hipSuccess ? 0 : -2;
}

int ceil_mfma_chains(void) { return kChains; }

// buf holds chunks KiB (chunks >= kDmaLoads); out must hold grid * 8 words.  Bytes
// per launch: grid * 8 waves * iters * kDmaLoads KiB.
int ceil_lds_dma(const void *buf, int64_t chunks, int grid, int iters, uint32_t *out, void *stream)
{
    if (chunks < kDmaLoads || grid <= 0 || iters <= 0)
        return -1;
    hipLaunchKernelGGL(lds_dma_kernel, dim3(grid), dim3(kDmaWaves * 64), 0, (hipStream_t)stream,
                       (const char *)buf, chunks, iters, out);
    return hipGetLastError() == hipSuccess ? 0 : -2;
}

int ceil_lds_dma_loads(void) { return kDmaLoads; }
int ceil_lds_dma_waves(void) { return kDmaWaves; }

}  // extern "C"
